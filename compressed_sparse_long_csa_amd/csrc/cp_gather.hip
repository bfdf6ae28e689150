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
//      depend on how the launch is split.
#include "kernels.hpp"

namespace csa {

namespace {

constexpr int kGThreads = 256;
constexpr int kGRowsPerWg = 16;            // one row per 16 lanes' worth of work, 4 rows per wave

__global__ void __launch_bounds__(kGThreads) select_pad_kernel(const uint32_t* in, int n_shards, int64_t cap,
                                                               int64_t row_words, const int64_t* n_valid,
                                                               uint32_t* out) {
  // exclusive prefix of the shards' valid counts, in LDS (n_shards <= 256)
  __shared__ int64_t pre[kGThreads + 1];
  __shared__ int64_t part[kGThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int64_t v = 0;
  if (t < n_shards) {
    v = n_valid[t];
    v = v < 0 ? 0 : (v > cap ? cap : v);
  }
  // inclusive scan over the block: within the wave by shuffles, then the waves
  int64_t x = v;
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
  const int64_t rows = static_cast<int64_t>(n_shards) * cap;
  // each wave copies one output row at a time: row j < total comes from the
  // shard s with pre[s] <= j < pre[s + 1], row pre[s] + r <- shard s row r
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * kGRowsPerWg + wv; j < rows;
       j += static_cast<int64_t>(gridDim.x) * kGRowsPerWg) {
    for (int64_t jj = j; jj < j + kGRowsPerWg && jj < rows; jj += kGThreads / 64) {
      uint32_t* dst = out + jj * row_words;
      if (jj < total) {
        int lo = 0, hi = n_shards - 1;                 // the last s with pre[s] <= jj
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pre[mid] <= jj) lo = mid; else hi = mid - 1;
        }
        const uint32_t* src = in + (static_cast<int64_t>(lo) * cap + (jj - pre[lo])) * row_words;
        for (int64_t c = lane; c < row_words; c += 64) dst[c] = src[c];
      } else {
        for (int64_t c = lane; c < row_words; c += 64) dst[c] = 0u;
      }
    }
  }
}

}  // namespace

hipError_t launch_select_pad(const void* in, int n_shards, int64_t cap, int64_t row_bytes, const int64_t* n_valid,
                             void* out, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(n_shards) * cap;
  if (rows == 0) return hipSuccess;
  const int64_t wgs = (rows + kGRowsPerWg - 1) / kGRowsPerWg;
  const unsigned grid = static_cast<unsigned>(wgs < 65536 ? wgs : 65536);
  log_launch("select-and-pad: %d shards x %lld rows of %lld bytes in %u workgroups", n_shards,
             static_cast<long long>(cap), static_cast<long long>(row_bytes), grid);
  hipLaunchKernelGGL(select_pad_kernel, dim3(grid), dim3(kGThreads), 0, stream,
                     static_cast<const uint32_t*>(in), n_shards, cap, row_bytes / 4, n_valid,
                     static_cast<uint32_t*>(out));
  return hipGetLastError();
}

}  // namespace csa
