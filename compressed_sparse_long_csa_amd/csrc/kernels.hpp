// Internal launch interface between the C ABI (csa_abi.hip) and the kernels.
#pragma once

#include "common.hpp"

namespace csa {

__host__ __device__ inline size_t row_bytes(csa_fmt fmt, int D, int R) {
  switch (fmt) {
    case CSA_F32: return 4u * static_cast<size_t>(D);
    case CSA_BF16: return 2u * static_cast<size_t>(D);
    case CSA_FP8: return static_cast<size_t>(D);
    case CSA_MXFP4: return static_cast<size_t>(D / 2 + D / 32);
    case CSA_SPLIT: return static_cast<size_t>(D - R) + 2u * static_cast<size_t>(R);
    default: return 0;
  }
}

struct CompressArgs {
  const void* x; csa_fmt x_fmt; const float* gate; int gate_cols;
  int64_t n_tok; int D; int m; int nseg;
  const int64_t* seg_tok_off; const int64_t* seg_pos0; const int64_t* seg_out_row;
  int normalize; const float* norm_w; float eps; int rope_dim; float rope_base;
  void* out; csa_fmt out_fmt;
  double rope_theta[kMaxRopePairs];
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t stream);

constexpr int kMaxCompressJobs = 4;
struct CompressJobs {
  CompressArgs a[kMaxCompressJobs];
  int64_t blk0[kMaxCompressJobs + 1];   // first global block of each job
  int kind[kMaxCompressJobs];
  int n;
};
static_assert(sizeof(CompressJobs) <= 4096, "kernel arguments are limited to 4 KiB");
// Jobs with no complete block are skipped; n <= kMaxCompressJobs.
hipError_t launch_compress_jobs(const CompressArgs* jobs, int n, hipStream_t stream);

struct IndexerArgs {
  const void* q; const float* w; int nq; int H; int d; const void* keys; csa_fmt fmt;
  const int64_t* key_off; const int64_t* q_pos; int m; float* scores; int64_t ld;
  // paged keys (blk_table != nullptr; key_off unused): row s of query i is pool
  // row blk_table[i * blk_stride + (s >> blk_shift)] * 2^blk_shift + (s mod 2^blk_shift)
  const int32_t* blk_table; int64_t blk_stride; int blk_shift; int64_t pool_rows;
  // query i reads table row blk_row[i] (clamped into [0, blk_rows)) in place of i
  const int32_t* blk_row; int64_t blk_rows;
};
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream);
// jobs (n <= kMaxCompressJobs, none empty) and the indexer in one launch when
// the keys are FP8 and the batch takes the streaming kernel, else the two
// launches one after the other.  key_job: the job that writes a.keys, or -1.
hipError_t launch_compress_score(const CompressArgs* jobs, int n, int key_job, const IndexerArgs& a,
                                 hipStream_t stream);

// The top-k of a decode step selected in its compress + score launch
// (csa_compress_score_topk): FP8 keys, the streaming indexer (nq below
// kShareMinQueries).  ws: per query kTkWsWords words -- the level-1 bins of
// the selection and an arrival counter -- zero on entry and left zero.
constexpr int kShareMinQueries = 1024;   // FP8 batches this large take the shared-key indexer
constexpr int kTkBins = 4096;
constexpr int kTkWsWords = kTkBins + 64;
struct TopkFuse {
  int32_t* idx;      // [nq, k]
  uint32_t* ws;      // [nq, kTkWsWords]
  int k;
};
hipError_t launch_compress_score_topk(const CompressArgs* jobs, int n, int key_job, const IndexerArgs& a,
                                      const TopkFuse& tk, hipStream_t stream);

// Select-and-pad of context-parallel compression: n_shards runs of cap rows
// (row_bytes, a multiple of 4), run s valid in its first n_valid[s] rows
// (device, clamped to [0, cap]); out: the valid rows in shard order, then
// zero rows (n_shards * cap rows).  n_shards <= kSelectPadMaxShards.
constexpr int kSelectPadMaxShards = 256;
hipError_t launch_select_pad(const void* in, int n_shards, int64_t cap, int64_t row_bytes, const int64_t* n_valid,
                             void* out, hipStream_t stream);

struct TopkArgs {
  const float* scores; int64_t ld; int nq; const int64_t* n_valid; int k;
  int32_t* idx; float* top_scores;
};
// Long rows (ld > 33792) take two passes through a device workspace: P slices
// of Cs scores, ws_bytes of candidates (P = 0: one pass, no workspace).
struct TopkPlan { int P; uint32_t Cs; size_t ws_bytes; };
// Rows (or rows x slices) of one launch: one 1024-thread workgroup each, so
// the grid stays below 2^32 threads.
constexpr int kTopkMaxRows = 1 << 22;
TopkPlan plan_topk(int64_t ld, int nq, int k);
// ws: at least plan_topk(...).ws_bytes of device memory (unused when P = 0).
hipError_t launch_topk(const TopkArgs& a, void* ws, hipStream_t stream);
// Size of the library's static top-k candidate array (one per device) and its
// device address on the current device, looked up on the first call per device.
constexpr size_t kTopkScratchBytes = size_t{16} << 20;
hipError_t topk_scratch(void** ptr);

// Attention over [selected or all compressed entries] ++ [window rows].
// The window of query b is `win_count` consecutive rows starting at row
// `win_row0` of `win`, where for decode win_row0 = b*n_win and the count is
// win_len[b]; for prefill they come from the token run (tok_off, tok_pos0).
struct AttnArgs {
  const void* q; csa_fmt q_fmt; int nq; int H; int D;
  const int64_t* q_pos; const float* q_norm_w; float eps; int rope_dim; float rope_base;
  const void* kv; csa_fmt kv_fmt; const int64_t* kv_off; int m;
  const int32_t* idx; int k;
  const void* win; csa_fmt win_fmt; int n_win;
  int win_mode;                                         // 0 none, 1 decode, 2 prefill
  const int32_t* win_len;                               // decode
  const int64_t* tok_off; const int64_t* tok_pos0;      // prefill
  const float* sinks; float scale; void* out; csa_fmt out_fmt; int variant;
  double rope_theta[kMaxRopePairs];
  // paged cache (blk_table != nullptr; kv_off unused): entry e of query b is
  // pool row blk_table[r * blk_stride + (e >> blk_shift)] * 2^blk_shift +
  // (e mod 2^blk_shift), r = blk_row[b] (or b)
  const int32_t* blk_table; int64_t blk_stride; int blk_shift; int64_t pool_rows;
  // decode window kept as a ring (win_start != nullptr, MFMA path): window
  // row t of query b is row b * n_win + (win_start[b] + t) mod n_win of win
  const int32_t* win_start;
  // the block-table row of each query (paged prefill: the queries of one
  // sequence share a row); nullptr: query b uses row b.  Rows are clamped to
  // [0, blk_rows).
  const int32_t* blk_row; int64_t blk_rows;
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);

int device_cu_count();

// Diagnostics from the environment, read once per process.  CSA_LOG >= 1:
// every error message, and each launch's kernel choice and grid, go to
// stderr.  CSA_VARIANT = high | low | full: calls that pass CSA_VARIANT_AUTO take
// that variant instead (explicit variants are kept).
int env_log_level();
int env_variant(int requested);
void log_launch(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

}  // namespace csa
