// A decode step's compress jobs, indexer scores and top-k selection in one
// launch (csa_compress_score_topk).
//
// Source: 硅星人 article on DeepSeek V4, CSA paragraph (the lightning indexer
// scores every compressed entry and the top-k selector keeps the k best for
// the attention); DeepSeek-V4 blog, index-visibility rule (query at p sees
// floor((p+1)/m) entries).
//
// The launch is the one-launch compress + score of indexer.hip with the
// selection of indexer_dev.hpp added: workgroups that stream a query's keys
// also count their scores into the query's level-1 bins, and the last
// workgroup to finish a query selects its top-k from the scores just stored
// (still in L2).  So a decode step has no separate top-k launch and no launch
// gap before the attention.  Scores and index sets equal those of
// csa_compress_score followed by topk_select bit for bit.
#include "indexer_dev.hpp"

namespace csa {

namespace {

template <int NHB, bool IL, bool kWithAny, int NB, bool kPaged>
__global__ void __launch_bounds__(256) compress_score_topk_kernel(CompressJobs J, int key_job, NewKeys nk,
                                                                  IndexerArgs a, int64_t n_items, int64_t n_chunk,
                                                                  int R, int n_cwg, TopkFuse tk) {
  __shared__ TkSmem ts;
  tk_clear(ts);
  if (static_cast<int>(blockIdx.x) < n_cwg) {
    extern __shared__ float y[];
    __shared__ cmp::EntrySlot slot;
    const int64_t total = J.blk0[J.n];
    for (int64_t b = blockIdx.x; b < total; b += n_cwg) {
      int j = 0;
      while (j + 1 < J.n && b >= J.blk0[j + 1]) ++j;
      const CompressArgs& c = J.a[j];
      cmp::run_block<kWithAny>(c, J.kind[j], b - J.blk0[j], y, y + c.D, &slot);
      if (j == key_job && slot.ok) {                    // uniform over the workgroup
        if (threadIdx.x == 0) ts.q = -1;
        // the new key's score, and this workgroup's arrival for its query
        score_new_key<NHB, kPaged, true>(a, y, slot.seg, slot.row, tk, &ts, static_cast<uint32_t>(n_chunk) + 1u);
        __syncthreads();
        if (ts.q >= 0)                                  // the query's last arrival: select
          tk_select(tk, ts, ts.q, ts.n, a.scores + static_cast<int64_t>(ts.q) * a.ld);
      }
      __syncthreads();                                  // y, slot and ts are reused by the next block
    }
    return;
  }
  fp8_items<NHB, IL, true, NB, kPaged, true>(a, n_items, n_chunk, R, blockIdx.x - n_cwg, gridDim.x - n_cwg, nk,
                                              tk, &ts);
}

}  // namespace

hipError_t launch_compress_score_topk(const CompressArgs* jobs, int n, int key_job, const IndexerArgs& a,
                                      const TopkFuse& tk, hipStream_t stream) {
  if (a.nq == 0) return n > 0 ? launch_compress_jobs(jobs, n, stream) : hipSuccess;
  if (a.fmt != CSA_FP8 || a.nq >= kShareMinQueries) return hipErrorInvalidValue;   // the ABI checks first
  CompressJobs J{};
  NewKeys nk{};
  int kj = -1, maxD = 1;
  bool any = false;
  J.blk0[0] = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t nb = jobs[i].n_tok / jobs[i].m;
    if (nb == 0) continue;
    if (i == key_job) {
      kj = J.n;
      nk = NewKeys{jobs[i].seg_tok_off, jobs[i].seg_out_row, jobs[i].n_tok, jobs[i].nseg, jobs[i].m};
    }
    J.a[J.n] = jobs[i];
    J.kind[J.n] = cmp::block_kind(jobs[i]);
    any = any || J.kind[J.n] == cmp::kAny;
    J.blk0[J.n + 1] = J.blk0[J.n] + nb;
    maxD = jobs[i].D > maxD ? jobs[i].D : maxD;
    ++J.n;
  }
  StreamPlan p = plan_stream(a);
  const bool il = p.R > 2;
  const int64_t total = J.blk0[J.n];
  const int n_cwg = static_cast<int>(total < 65536 ? total : 65536);
  // the same sizing as the compress + score launch: the compress workgroups
  // take resident slots, so the items are sized to the slots left
  const int64_t slots = static_cast<int64_t>(device_cu_count()) * 2;
  if (p.R <= 2 && p.n_items + n_cwg > slots && slots - n_cwg >= a.nq) {
    const int64_t gp = (a.ld + kGroupKeys - 1) / kGroupKeys;
    p.n_chunk = (slots - n_cwg) / a.nq;
    p.n_items = static_cast<int64_t>(a.nq) * p.n_chunk;
    p.R = (gp + 4 * p.n_chunk - 1) / (4 * p.n_chunk);
    p.grid = static_cast<unsigned>(p.n_items);
  }
  const dim3 grid(static_cast<unsigned>(n_cwg) + p.grid), block(256);
  const size_t shm = J.n > 0 ? cmp::shm_bytes(maxD) : 0;
  const bool paged = a.blk_table != nullptr;
  log_launch("compress+score+top-k: one launch%s, %d jobs in %d workgroups + FP8 indexer of %d queries in %u "
             "workgroups (%lld groups per wave), top-%d selected by each query's last workgroup",
             paged ? " (paged keys)" : "", J.n, n_cwg, a.nq, p.grid, static_cast<long long>(p.R), tk.k);
  const int r = static_cast<int>(p.R);
  const bool three = !il && p.R == 3;
#define CSA_CST_LAUNCH(NB, IL, ANY, BUF)                                                                     \
  do {                                                                                                      \
    if (paged) hipLaunchKernelGGL((compress_score_topk_kernel<NB, IL, ANY, BUF, true>), grid, block, shm,   \
                                  stream, J, kj, nk, a, p.n_items, p.n_chunk, r, n_cwg, tk);                \
    else hipLaunchKernelGGL((compress_score_topk_kernel<NB, IL, ANY, BUF, false>), grid, block, shm, stream, \
                            J, kj, nk, a, p.n_items, p.n_chunk, r, n_cwg, tk);                              \
  } while (0)
#define CSA_CST_CASE(NB)                                                                                    \
  case NB:                                                                                                  \
    if (il) { if (any) CSA_CST_LAUNCH(NB, true, true, 2); else CSA_CST_LAUNCH(NB, true, false, 2); }       \
    else if (three) { if (any) CSA_CST_LAUNCH(NB, false, true, 3); else CSA_CST_LAUNCH(NB, false, false, 3); } \
    else { if (any) CSA_CST_LAUNCH(NB, false, true, 2); else CSA_CST_LAUNCH(NB, false, false, 2); }        \
    break;
  switch (a.H / 16) {
    CSA_CST_CASE(1)
    CSA_CST_CASE(2)
    CSA_CST_CASE(4)
    CSA_CST_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef CSA_CST_CASE
#undef CSA_CST_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
