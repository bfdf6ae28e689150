// Top-k selector (topk_select).
//
// Source: 硅星人 article on DeepSeek V4, CSA paragraph (the top-k selector
// keeps the 512 most relevant compressed blocks, 1024 for Pro); DeepSeek-V4
// blog, index visibility (the top-k selector names the entries a CSA query
// sees).  Ties go to the lower index and the output is ascending, which is
// this library's reading of what the pages leave open.
//
// One workgroup per row.  Scores map to order-preserving 32-bit keys; a
// three-pass radix select (11 + 11 + 10 bits, LDS histograms with integer
// atomics, which are order-independent) finds the k-th largest key T and how
// many elements equal to T are still needed.  A final pass walks the row in
// index order and compacts the selected indices with ballot prefix counts, so
// the output is the exact set, ascending, whatever the launch.
#include "kernels.hpp"

namespace csa {

namespace {

constexpr int kThreads = 1024;
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ void __launch_bounds__(kThreads) topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wsum[kThreads / 64];
  __shared__ uint32_t sh_bin, sh_above;
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t n = a.n_valid ? a.n_valid[row] : a.ld;
  n = n < 0 ? 0 : (n > a.ld ? a.ld : n);
  const float* s = a.scores + static_cast<int64_t>(row) * a.ld;
  int32_t* out = a.idx + static_cast<int64_t>(row) * a.k;
  float* out_s = a.top_scores ? a.top_scores + static_cast<int64_t>(row) * a.k : nullptr;
  const int k = a.k;

  uint32_t T = 0u;          // threshold key (k-th largest)
  uint32_t need_eq = 0u;    // elements equal to T to take, lowest index first
  bool take_all = n <= k;
  if (!take_all) {
    uint32_t prefix = 0u, pmask = 0u, remaining = static_cast<uint32_t>(k);
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = shifts[pass];
      const uint32_t bmask = (1u << widths[pass]) - 1u;
      for (int b = tid; b < kBins; b += kThreads) hist[b] = 0u;
      __syncthreads();
      for (int64_t e = tid; e < n; e += kThreads) {
        const uint32_t key = order_key(s[e]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & bmask], 1u);
      }
      __syncthreads();
      // scan bins from the top: find b with above(b) < remaining <= above(b) + hist[b]
      // each thread owns 2 consecutive bins, counted from the top
      const int nb = static_cast<int>(bmask) + 1;
      const int b_hi = nb - 1 - 2 * tid, b_lo = b_hi - 1;
      const uint32_t c0 = b_hi >= 0 ? hist[b_hi] : 0u;
      const uint32_t c1 = b_lo >= 0 ? hist[b_lo] : 0u;
      uint32_t own = c0 + c1;
      // inclusive wave scan of `own`
      uint32_t incl = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (lane == 63) wsum[wv] = incl;
      __syncthreads();
      uint32_t before = 0u;
      for (int w2 = 0; w2 < wv; ++w2) before += wsum[w2];
      const uint32_t excl = before + incl - own;     // count in bins above b_hi
      if (b_hi >= 0) {
        if (excl < remaining && remaining <= excl + c0) { sh_bin = b_hi; sh_above = excl; }
        if (b_lo >= 0 && excl + c0 < remaining && remaining <= excl + c0 + c1) {
          sh_bin = b_lo; sh_above = excl + c0;
        }
      }
      __syncthreads();
      const uint32_t bin = sh_bin, above = sh_above;
      remaining -= above;
      prefix |= bin << sh;
      pmask |= bmask << sh;
      __syncthreads();
    }
    T = prefix;
    need_eq = remaining;
  }

  // compaction in index order
  uint32_t sel_carry = 0u, eq_carry = 0u;
  for (int64_t base = 0; base < n; base += kThreads) {
    const int64_t e = base + tid;
    bool in = false, eq = false;
    float v = 0.0f;
    if (e < n) {
      v = s[e];
      if (take_all) {
        in = true;
      } else {
        const uint32_t key = order_key(v);
        in = key > T;
        eq = key == T;
      }
    }
    const unsigned long long lm = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const unsigned long long eq_mask = __ballot(eq);
    __syncthreads();
    if (lane == 0) wsum[wv] = static_cast<uint32_t>(__popcll(eq_mask));
    __syncthreads();
    uint32_t eq_before = eq_carry;
    for (int w2 = 0; w2 < wv; ++w2) eq_before += wsum[w2];
    uint32_t eq_tot = 0u;
    for (int w2 = 0; w2 < kThreads / 64; ++w2) eq_tot += wsum[w2];
    const uint32_t eq_rank = eq_before + static_cast<uint32_t>(__popcll(eq_mask & lm));
    if (eq && eq_rank < need_eq) in = true;
    eq_carry += eq_tot;
    const unsigned long long in_mask = __ballot(in);
    __syncthreads();
    if (lane == 0) wsum[wv] = static_cast<uint32_t>(__popcll(in_mask));
    __syncthreads();
    uint32_t in_before = sel_carry;
    for (int w2 = 0; w2 < wv; ++w2) in_before += wsum[w2];
    uint32_t in_tot = 0u;
    for (int w2 = 0; w2 < kThreads / 64; ++w2) in_tot += wsum[w2];
    if (in) {
      const uint32_t pos = in_before + static_cast<uint32_t>(__popcll(in_mask & lm));
      if (pos < static_cast<uint32_t>(k)) {
        out[pos] = static_cast<int32_t>(e);
        if (out_s) out_s[pos] = v;
      }
    }
    sel_carry += in_tot;
  }
  const uint32_t total = sel_carry < static_cast<uint32_t>(k) ? sel_carry : static_cast<uint32_t>(k);
  for (int j = static_cast<int>(total) + tid; j < k; j += kThreads) {
    out[j] = -1;
    if (out_s) out_s[j] = -INFINITY;
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.nq), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
