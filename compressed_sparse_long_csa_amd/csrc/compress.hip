// Token-level compressor and cache write path (csa_compress).
//
// Source: 硅星人 article on DeepSeek V4, CSA paragraph (every m = 4 tokens'
// KV fold into one entry) and HCA paragraph (m' = 128); DeepSeek-V4 blog,
// RMSNorm归一化 (norm on the compressed KV head) and Partial RoPE位置编码
// (RoPE on the last dims; BF16 RoPE dims, FP8 others).  The gate convention
// (softmax of per-token or per-channel logits over the block) is this
// library's reading of the unspecified compressor weights.
//
// One workgroup per output entry.  The block sum runs over the m tokens in
// order, the mean square over D in a fixed tree, so an entry's bits depend
// only on its own tokens -- also when several calls share one launch
// (csa_compress_batch: the jobs' blocks are numbered one after another).
//
// Latency: a decode step writes a handful of entries, so the kernel is a
// chain of memory round trips, and it keeps that chain short.  The block's
// tokens and gate logits depend only on the entry number and are loaded
// first (into registers when m * ceil(D / 256) <= 16); the segment of the
// block is found in the same round trip, every thread testing one segment.
#include "compress_dev.hpp"

namespace csa {

namespace {

using namespace cmp;

template <int Kind>
__global__ void __launch_bounds__(kThreads) compress_kernel(CompressArgs a, int64_t n_blocks) {
  extern __shared__ float y[];            // [D] entry values, then [kThreads/64] partials
  __shared__ EntrySlot slot;
  for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x)
    run_block(a, Kind, blk, y, y + a.D, &slot);
}

// Several independent compress calls in one launch: global block b belongs
// to the job j with blk0[j] <= b < blk0[j + 1] (uniform over the workgroup).
template <bool kWithAny>
__global__ void __launch_bounds__(kThreads) compress_jobs_kernel(CompressJobs J) {
  extern __shared__ float y[];
  __shared__ EntrySlot slot;
  const int64_t total = J.blk0[J.n];
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    int j = 0;
    while (j + 1 < J.n && b >= J.blk0[j + 1]) ++j;
    const CompressArgs& a = J.a[j];
    run_block<kWithAny>(a, J.kind[j], b - J.blk0[j], y, y + a.D, &slot);
  }
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  const int64_t n_blocks = a.n_tok / a.m;
  if (n_blocks == 0) return hipSuccess;
  const int64_t grid = n_blocks < 65536 ? n_blocks : 65536;
  const size_t shm = shm_bytes(a.D);
  const dim3 g(static_cast<unsigned>(grid)), b(kThreads);
  switch (block_kind(a)) {
    case kM4C1: hipLaunchKernelGGL(compress_kernel<kM4C1>, g, b, shm, stream, a, n_blocks); break;
    case kM4C2: hipLaunchKernelGGL(compress_kernel<kM4C2>, g, b, shm, stream, a, n_blocks); break;
    case kM1C1: hipLaunchKernelGGL(compress_kernel<kM1C1>, g, b, shm, stream, a, n_blocks); break;
    case kM1C2: hipLaunchKernelGGL(compress_kernel<kM1C2>, g, b, shm, stream, a, n_blocks); break;
    case kM1C4: hipLaunchKernelGGL(compress_kernel<kM1C4>, g, b, shm, stream, a, n_blocks); break;
    default: hipLaunchKernelGGL(compress_kernel<kAny>, g, b, shm, stream, a, n_blocks); break;
  }
  return hipGetLastError();
}

hipError_t launch_compress_jobs(const CompressArgs* jobs, int n, hipStream_t stream) {
  CompressJobs J{};
  J.n = 0;
  J.blk0[0] = 0;
  int maxD = 1;
  bool any = false;
  for (int i = 0; i < n; ++i) {
    const int64_t nb = jobs[i].n_tok / jobs[i].m;
    if (nb == 0) continue;
    J.a[J.n] = jobs[i];
    J.kind[J.n] = block_kind(jobs[i]);
    any = any || J.kind[J.n] == kAny;
    J.blk0[J.n + 1] = J.blk0[J.n] + nb;
    maxD = jobs[i].D > maxD ? jobs[i].D : maxD;
    ++J.n;
  }
  if (J.n == 0) return hipSuccess;
  const int64_t total = J.blk0[J.n];
  const int64_t grid = total < 65536 ? total : 65536;
  log_launch("compress: %d jobs, %lld blocks, grid %lld x %d threads", J.n, static_cast<long long>(total),
             static_cast<long long>(grid), kThreads);
  if (any)
    hipLaunchKernelGGL(compress_jobs_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                       shm_bytes(maxD), stream, J);
  else
    hipLaunchKernelGGL(compress_jobs_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                       shm_bytes(maxD), stream, J);
  return hipGetLastError();
}

}  // namespace csa
