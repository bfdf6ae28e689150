// Select-and-pad of context-parallel compression (csa_select_and_pad).
//
// Source: DeepSeek-V4 blog, 百万 token 怎么切分到多张卡 (context parallelism:
// each rank compresses its part of the sequence -- its own tokens after the
// boundary tokens received from the rank before it -- into a fixed-length
// run of compressed blocks with a little padding; after the all-gather of the
// runs, a fused select-and-pad step joins them into one contiguous
// compressed sequence and moves all the padding to its end).
//
// in:  n_shards runs of `cap` rows (row_bytes each), shard s valid in its
//      first min(n_valid[s], cap) rows (n_valid clamped to [0, cap]);
// out: n_shards * cap rows: shard 0's valid rows, then shard 1's, ..., then
//      zero rows.  Pure data movement (integer work): the result does not
//      depend on how the launch is split.  Shard s's valid rows are one
//      contiguous run of `in`, so the join is a flat copy of words.
#include "kernels.hpp"

namespace csa {

namespace {

constexpr int kGThreads = 256;
constexpr int kGWordsPerThread = 4;        // output words per thread per pass (loads in flight)

// The output is a flat array of words (W = 16 bytes where rows allow, else
// 4): shard s's valid rows are one contiguous run of the input, so output
// word w below the valid total comes from the shard whose run holds it, at
// the same offset into that run; words past it are zero.
template <typename W>
__global__ void __launch_bounds__(kGThreads) select_pad_kernel(const W* in, int n_shards, int64_t cap,
                                                               int64_t row_words, const int64_t* n_valid, W* out) {
  // exclusive prefix of the shards' valid counts, in words (n_shards <= 256)
  __shared__ int64_t pre[kGThreads + 1];
  __shared__ int64_t part[kGThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int64_t v = 0;
  if (t < n_shards) {
    v = n_valid[t];
    v = (v < 0 ? 0 : (v > cap ? cap : v)) * row_words;
  }
  int64_t x = v;                                       // inclusive scan: the wave, then the waves
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(x, d);
    x += lane >= d ? y : 0;
  }
  if (lane == 63) part[wv] = x;
  __syncthreads();
  int64_t base = 0;
  for (int w = 0; w < wv; ++w) base += part[w];
  pre[t + 1] = base + x;
  if (t == 0) pre[0] = 0;
  __syncthreads();
  const int64_t total = pre[n_shards];
  const int64_t words = static_cast<int64_t>(n_shards) * cap * row_words;
  const int64_t run = cap * row_words;                 // words per shard run
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kGThreads * kGWordsPerThread;
  for (int64_t w0 = static_cast<int64_t>(blockIdx.x) * kGThreads * kGWordsPerThread + t; w0 < words; w0 += stride) {
    W val[kGWordsPerThread];
#pragma unroll
    for (int u = 0; u < kGWordsPerThread; ++u) {
      const int64_t w = w0 + static_cast<int64_t>(u) * kGThreads;   // coalesced within each u
      val[u] = W{};
      if (w < total) {
        int lo = 0, hi = n_shards - 1;                 // the last s with pre[s] <= w
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pre[mid] <= w) lo = mid; else hi = mid - 1;
        }
        val[u] = in[static_cast<int64_t>(lo) * run + (w - pre[lo])];
      }
    }
#pragma unroll
    for (int u = 0; u < kGWordsPerThread; ++u) {
      const int64_t w = w0 + static_cast<int64_t>(u) * kGThreads;
      if (w < words) out[w] = val[u];
    }
  }
}

}  // namespace

hipError_t launch_select_pad(const void* in, int n_shards, int64_t cap, int64_t row_bytes, const int64_t* n_valid,
                             void* out, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(n_shards) * cap;
  if (rows == 0) return hipSuccess;
  const bool w16 = row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) % 16 == 0;
  const int64_t wb = w16 ? 16 : 4;
  const int64_t words = rows * (row_bytes / wb);
  const int64_t per_wg = static_cast<int64_t>(kGThreads) * kGWordsPerThread;
  const int64_t wgs = (words + per_wg - 1) / per_wg;
  const unsigned grid = static_cast<unsigned>(wgs < 8192 ? wgs : 8192);
  log_launch("select-and-pad: %d shards x %lld rows of %lld bytes, %lld-byte words in %u workgroups", n_shards,
             static_cast<long long>(cap), static_cast<long long>(row_bytes), static_cast<long long>(wb), grid);
  if (w16)
    hipLaunchKernelGGL(select_pad_kernel<uint4>, dim3(grid), dim3(kGThreads), 0, stream, static_cast<const uint4*>(in),
                       n_shards, cap, row_bytes / 16, n_valid, static_cast<uint4*>(out));
  else
    hipLaunchKernelGGL(select_pad_kernel<uint32_t>, dim3(grid), dim3(kGThreads), 0, stream,
                       static_cast<const uint32_t*>(in), n_shards, cap, row_bytes / 4, n_valid,
                       static_cast<uint32_t*>(out));
  return hipGetLastError();
}

}  // namespace csa
