// Top-k selector (topk_select).
//
// Source: 硅星人 article on DeepSeek V4, CSA paragraph (the top-k selector
// keeps the 512 most relevant compressed blocks, 1024 for Pro); DeepSeek-V4
// blog, index visibility (the top-k selector names the entries a CSA query
// sees).  Ties go to the lower index and the output is ascending, which is
// this library's reading of what the pages leave open.
//
// One workgroup of 1024 threads (16 waves) per row.  Wave w owns the contiguous
// range [w*C, (w+1)*C) of the row and reads it 64 consecutive scores at a time
// (coalesced).  Scores map to order-preserving 32-bit keys.
//  1. min / max of the finite scores;
//  2. a 2048-bin histogram linear in the score value over [min, max]
//     (monotone float binning; LDS integer atomics are order-free) gives the
//     bin b* holding the k-th largest score and `need`, the number of its
//     elements that are selected;
//  3. one pass collects the elements of b* (key, index) into LDS and counts,
//     per wave, the elements of higher bins;
//  4. among the candidates the threshold key T and the number of elements
//     equal to T to take (lowest indices first) are found exactly: by direct
//     ranking for few candidates, else by key-space histograms over the LDS
//     list (bins of power-of-two width) -- rows whose b* is too large to keep
//     refine over the row itself;
//  5. per-wave counts give each wave its output offset and every wave writes
//     its indices in order with ballot prefix counts.
// The result is the exact set, ascending, whatever the batch or launch.
// Rows of up to 16384 scores stay in registers; longer rows are re-read from
// memory (L2), in batches of independent loads.
#include "kernels.hpp"

namespace csa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kMaxJ = 16;                  // 64-element steps per wave kept in registers
constexpr int kBinsPerThread = kBins / kThreads;
constexpr int kMaxCand = 4096;             // candidates kept in LDS
constexpr int kRankDirect = 512;           // candidates ranked by direct counting

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

struct TopkSmem {
  uint32_t hist[kBins];
  uint32_t cand_key[kMaxCand];
  uint32_t cand_idx[kMaxCand];
  uint32_t wgt[kWaves];            // per wave: selected elements with key > T
  uint32_t weq[kWaves];            // per wave: elements with key == T
  uint32_t wred[kWaves];
  uint32_t wred2[kWaves];
  uint32_t sh[8];
};

__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, TopkSmem& sm) {
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t a = __shfl_xor(lo, o, 64), b = __shfl_xor(hi, o, 64);
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sm.wred[threadIdx.x >> 6] = lo;
    sm.wred2[threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
  for (int w = 0; w < kWaves; ++w) {
    lo = sm.wred[w] < lo ? sm.wred[w] : lo;
    hi = sm.wred2[w] > hi ? sm.wred2[w] : hi;
  }
}

// Bin b with above(b) < need <= above(b) + hist[b], counting from the top bin.
// Thread t owns the kBinsPerThread bins just below 2047 - kBinsPerThread * t.
__device__ __forceinline__ void find_bin(TopkSmem& sm, uint32_t need, uint32_t* bin,
                                         uint32_t* above) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int top = kBins - 1 - kBinsPerThread * tid;
  uint32_t c[kBinsPerThread], own = 0u;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) { c[i] = sm.hist[top - i]; own += c[i]; }
  uint32_t incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) sm.wred[wv] = incl;
  __syncthreads();
  uint32_t run = incl - own;
  for (int w = 0; w < wv; ++w) run += sm.wred[w];
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    if (run < need && need <= run + c[i]) { sm.sh[0] = top - i; sm.sh[1] = run; }
    run += c[i];
  }
  __syncthreads();
  *bin = sm.sh[0];
  *above = sm.sh[1];
}

// Key-space refinement of [lo, hi] (all keys inside are candidates) over a
// list of candidate keys: returns T and need (elements equal to T to take).
template <typename KeyFn>
__device__ __forceinline__ void refine(TopkSmem& sm, uint32_t lo, uint32_t hi, uint32_t need,
                                       int count, KeyFn key_of, uint32_t* T, uint32_t* need_eq) {
  const int tid = threadIdx.x;
  while (lo != hi) {
    const uint32_t span = hi - lo;
    const int shift = span < kBins ? 0 : (32 - __clz(span)) - 11;
    for (int b = tid; b < kBins; b += kThreads) sm.hist[b] = 0u;
    __syncthreads();
    for (int i = tid; i < count; i += kThreads) {
      const uint32_t key = key_of(i);
      if (key >= lo && key <= hi) atomicAdd(&sm.hist[(key - lo) >> shift], 1u);
    }
    __syncthreads();
    uint32_t b2, ab2;
    find_bin(sm, need, &b2, &ab2);
    need -= ab2;
    const uint32_t nlo = lo + (b2 << shift);
    const uint32_t nhi = (span >> shift) == b2 ? hi : nlo + ((1u << shift) - 1u);
    lo = nlo;
    hi = nhi;
    __syncthreads();
  }
  *T = lo;
  *need_eq = need;
}

template <bool kInRegs>
__device__ void topk_row(const TopkArgs& a, int row, int64_t n, TopkSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* s = a.scores + static_cast<int64_t>(row) * a.ld;
  int32_t* out = a.idx + static_cast<int64_t>(row) * a.k;
  float* out_s = a.top_scores ? a.top_scores + static_cast<int64_t>(row) * a.k : nullptr;
  const uint32_t k = static_cast<uint32_t>(a.k);
  // wave range: C elements, a multiple of 64
  const int64_t C = ((n + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int64_t w0 = wv * C;
  const int nj = kInRegs ? kMaxJ : static_cast<int>(C / 64);
  auto elem = [&](int j) -> int64_t { return w0 + static_cast<int64_t>(j) * 64 + lane; };
  auto valid = [&](int j) -> bool { return static_cast<int64_t>(j) * 64 < C && elem(j) < n; };

  // Visits every element of this lane: f(j, key).  In-register rows loop over a
  // compile-time count; streamed rows load 8 independent scores per step.
  uint32_t reg[kInRegs ? kMaxJ : 1];
  if (kInRegs) {
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) reg[j] = valid(j) ? order_key(s[elem(j)]) : 0u;
  }
  auto for_each = [&](auto&& f) {
    if (kInRegs) {
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j)
        if (valid(j)) f(j, reg[j]);
    } else {
      for (int j0 = 0; j0 < nj; j0 += 8) {
        uint32_t kb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kb[u] = valid(j0 + u) ? order_key(s[elem(j0 + u)]) : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (valid(j0 + u)) f(j0 + u, kb[u]);
      }
    }
  };

  uint32_t T = 0u, need_eq = 0u;
  const bool take_all = n <= static_cast<int64_t>(k);
  if (take_all) {
    uint32_t cnt = 0u;
    for_each([&](int, uint32_t) { ++cnt; });
    for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
    if (lane == 0) { sm.wgt[wv] = cnt; sm.weq[wv] = 0u; }
    __syncthreads();
  } else {
    // ---- 1. value range of the finite scores
    const uint32_t kNegInf = order_key(-INFINITY), kPosInf = order_key(INFINITY);
    uint32_t lo = 0xffffffffu, hi = 0u;
    for_each([&](int, uint32_t key) {
      if (key != kNegInf && key != kPosInf) {
        lo = key < lo ? key : lo;
        hi = key > hi ? key : hi;
      }
    });
    block_minmax(lo, hi, sm);
    float vlo = 0.0f, sc = 0.0f;
    if (lo <= hi) {
      vlo = key_value(lo);
      const float width = key_value(hi) - vlo;
      sc = (width > 0.0f && width < INFINITY) ? static_cast<float>(kBins) / width : 0.0f;
    }
    // monotone in the key: -inf -> 0, +inf -> top bin, finite values linear in value
    auto bin1 = [&](uint32_t key) -> uint32_t {
      if (key <= kNegInf) return 0u;
      if (key >= kPosInf) return kBins - 1;
      const int b = static_cast<int>((key_value(key) - vlo) * sc);
      return static_cast<uint32_t>(b < 0 ? 0 : (b > kBins - 1 ? kBins - 1 : b));
    };
    // ---- 2. value histogram
    for (int b = tid; b < kBins; b += kThreads) sm.hist[b] = 0u;
    if (tid == 0) sm.sh[2] = 0u;
    __syncthreads();
    for_each([&](int, uint32_t key) { atomicAdd(&sm.hist[bin1(key)], 1u); });
    __syncthreads();
    uint32_t bstar, above;
    find_bin(sm, k, &bstar, &above);
    const uint32_t need = k - above;
    const uint32_t cnt = sm.hist[bstar];
    // ---- 3. candidates of b* to LDS, per-wave counts of higher bins
    uint32_t c_above = 0u;
    lo = 0xffffffffu;
    hi = 0u;
    const bool keep = cnt <= kMaxCand;
    for_each([&](int j, uint32_t key) {
      const uint32_t b = bin1(key);
      c_above += b > bstar ? 1u : 0u;
      if (b == bstar) {
        lo = key < lo ? key : lo;
        hi = key > hi ? key : hi;
        if (keep) {
          const uint32_t slot = atomicAdd(&sm.sh[2], 1u);
          sm.cand_key[slot] = key;
          sm.cand_idx[slot] = static_cast<uint32_t>(elem(j));
        }
      }
    });
    for (int o = 32; o >= 1; o >>= 1) c_above += __shfl_xor(c_above, o, 64);
    if (lane == 0) { sm.wgt[wv] = c_above; sm.weq[wv] = 0u; }
    block_minmax(lo, hi, sm);              // key range of b*; its barriers publish the lists
    // ---- 4. exact threshold among the candidates
    if (keep && cnt <= kRankDirect) {
      if (tid < static_cast<int>(cnt)) {
        const uint32_t ck = sm.cand_key[tid], ci = sm.cand_idx[tid];
        uint32_t rank = 0u;
        for (uint32_t j = 0; j < cnt; ++j) {
          const uint32_t ok = sm.cand_key[j], oi = sm.cand_idx[j];
          rank += (ok > ck || (ok == ck && oi < ci)) ? 1u : 0u;
        }
        if (rank == need - 1u) sm.sh[3] = ck;
      }
      __syncthreads();
      T = sm.sh[3];
      // elements equal to T ranked above the threshold candidate are selected
      uint32_t gt = 0u;
      for (uint32_t j = 0; j < cnt; ++j) gt += sm.cand_key[j] > T ? 1u : 0u;
      need_eq = need - gt;
    } else if (keep) {
      refine(sm, lo, hi, need, static_cast<int>(cnt), [&](int i) { return sm.cand_key[i]; }, &T,
             &need_eq);
    } else {
      // a huge b* (e.g. massive ties): refine over the row itself
      uint32_t l2 = lo, h2 = hi, nd = need;
      while (l2 != h2) {
        const uint32_t span = h2 - l2;
        const int shift = span < kBins ? 0 : (32 - __clz(span)) - 11;
        for (int b = tid; b < kBins; b += kThreads) sm.hist[b] = 0u;
        __syncthreads();
        for_each([&](int, uint32_t key) {
          if (key >= l2 && key <= h2) atomicAdd(&sm.hist[(key - l2) >> shift], 1u);
        });
        __syncthreads();
        uint32_t b2, ab2;
        find_bin(sm, nd, &b2, &ab2);
        nd -= ab2;
        const uint32_t nlo = l2 + (b2 << shift);
        const uint32_t nhi = (span >> shift) == b2 ? h2 : nlo + ((1u << shift) - 1u);
        l2 = nlo;
        h2 = nhi;
        __syncthreads();
      }
      T = l2;
      need_eq = nd;
    }
    // per-wave counts of b*'s elements above / equal to T
    if (keep) {
      for (int i = tid; i < static_cast<int>(cnt); i += kThreads) {
        const uint32_t key = sm.cand_key[i];
        const int w = static_cast<int>(static_cast<int64_t>(sm.cand_idx[i]) / C);
        if (key > T) atomicAdd(&sm.wgt[w], 1u);
        else if (key == T) atomicAdd(&sm.weq[w], 1u);
      }
    } else {
      uint32_t g = 0u, e = 0u;
      for_each([&](int, uint32_t key) {
        if (key >= lo && key <= hi) { g += key > T ? 1u : 0u; e += key == T ? 1u : 0u; }
      });
      for (int o = 32; o >= 1; o >>= 1) { g += __shfl_xor(g, o, 64); e += __shfl_xor(e, o, 64); }
      if (lane == 0) { atomicAdd(&sm.wgt[wv], g); atomicAdd(&sm.weq[wv], e); }
    }
    __syncthreads();
  }

  // ---- 5. ordered writes
  uint32_t gt_before = 0u, eq_before = 0u, total_gt = 0u, total_eq = 0u;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wv) { gt_before += sm.wgt[w]; eq_before += sm.weq[w]; }
    total_gt += sm.wgt[w];
    total_eq += sm.weq[w];
  }
  const unsigned long long lm = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto emit = [&](int j, bool gt, bool eq) {
    const unsigned long long mg = __ballot(gt), me = __ballot(eq);
    const uint32_t gp = gt_before + static_cast<uint32_t>(__popcll(mg & lm));
    const uint32_t ep = eq_before + static_cast<uint32_t>(__popcll(me & lm));
    if (gt || (eq && ep < need_eq)) {
      const uint32_t pos = gp + (ep < need_eq ? ep : need_eq);
      if (pos < k) {
        const int64_t e = elem(j);
        out[pos] = static_cast<int32_t>(e);
        if (out_s) out_s[pos] = s[e];
      }
    }
    gt_before += static_cast<uint32_t>(__popcll(mg));
    eq_before += static_cast<uint32_t>(__popcll(me));
  };
  if (kInRegs) {
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      const bool v = valid(j);
      const uint32_t key = reg[j];
      emit(j, v && (take_all || key > T), v && !take_all && key == T);
    }
  } else {
    for (int j0 = 0; j0 < nj; j0 += 8) {
      uint32_t kb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kb[u] = valid(j0 + u) ? order_key(s[elem(j0 + u)]) : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool v = valid(j0 + u);
        emit(j0 + u, v && (take_all || kb[u] > T), v && !take_all && kb[u] == T);
      }
    }
  }
  const uint32_t sel = total_gt + (total_eq < need_eq ? total_eq : need_eq);
  const uint32_t total = sel < k ? sel : k;
  for (uint32_t j = total + tid; j < k; j += kThreads) {
    out[j] = -1;
    if (out_s) out_s[j] = -INFINITY;
  }
}

__global__ void __launch_bounds__(kThreads) topk_kernel(TopkArgs a) {
  __shared__ TopkSmem sm;
  const int row = blockIdx.x;
  int64_t n = a.n_valid ? a.n_valid[row] : a.ld;
  n = n < 0 ? 0 : (n > a.ld ? a.ld : n);
  if (n <= static_cast<int64_t>(kWaves) * 64 * kMaxJ) topk_row<true>(a, row, n, sm);
  else topk_row<false>(a, row, n, sm);
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.nq), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
