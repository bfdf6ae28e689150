// C ABI of libcsa: argument validation, format / path dispatch, error state.
// The contract of every entry point is documented in include/csa.h.
#include <stddef.h>
#include <stdio.h>
#include <stdarg.h>
#include <stdlib.h>
#include <string.h>

#include "kernels.hpp"

namespace csa {

namespace {
thread_local char g_err[512] = "";

csa_status fail(csa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  if (env_log_level() >= 1) fprintf(stderr, "[csa] error %d: %s\n", static_cast<int>(s), g_err);
  return s;
}

csa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return CSA_OK;
}

bool fmt_ok(csa_fmt f) { return f >= CSA_F32 && f <= CSA_SPLIT; }

// the layout the Python binding mirrors (LP64)
static_assert(sizeof(csa_compress_job) == 128 && offsetof(csa_compress_job, out_fmt) == 120,
              "csa_compress_job layout");
static_assert(CSA_COMPRESS_MAX_JOBS == kMaxCompressJobs, "job limit");
}  // namespace

int env_log_level() {
  static const int level = [] {
    const char* v = getenv("CSA_LOG");
    return v != nullptr && *v != '\0' ? atoi(v) : 0;
  }();
  return level;
}

int env_variant(int requested) {
  static const int forced = [] {
    const char* v = getenv("CSA_VARIANT");
    if (v == nullptr) return static_cast<int>(CSA_VARIANT_AUTO);
    if (strcmp(v, "high") == 0) return static_cast<int>(CSA_VARIANT_HIGH_OCC);
    if (strcmp(v, "low") == 0) return static_cast<int>(CSA_VARIANT_LOW_OCC);
    if (strcmp(v, "full") == 0) return static_cast<int>(CSA_VARIANT_FULL_DIMS);
    return static_cast<int>(CSA_VARIANT_AUTO);
  }();
  return requested == CSA_VARIANT_AUTO ? forced : requested;
}

void log_launch(const char* fmt, ...) {
  if (env_log_level() < 1) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  fprintf(stderr, "[csa] %s\n", buf);
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {
constexpr uint32_t kLdsBytesPerCu = 160 * 1024;   // gfx950

__global__ void __launch_bounds__(1024) poison_lds_kernel(uint32_t pattern) {
  extern __shared__ uint32_t lds_words[];
  for (uint32_t i = threadIdx.x; i < kLdsBytesPerCu / 4; i += blockDim.x) lds_words[i] = pattern;
  asm volatile("" : : : "memory");                       // the stores are the kernel's only effect
  __syncthreads();
}
}  // namespace

}  // namespace csa

using namespace csa;

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_string(csa_status s) {
  switch (s) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID_ARG: return "CSA_ERR_INVALID_ARG";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
    case CSA_ERR_HIP: return "CSA_ERR_HIP";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE";
    default: return "CSA_ERR_UNKNOWN";
  }
}

const char* csa_last_error(void) { return g_err; }

size_t csa_row_bytes(csa_fmt fmt, int D, int rope_dim) {
  if (!fmt_ok(fmt) || D < 1) return 0;
  if (fmt == CSA_MXFP4 && D % 32 != 0) return 0;
  if (fmt == CSA_SPLIT && (rope_dim < 1 || rope_dim >= D)) return 0;
  return row_bytes(fmt, D, rope_dim);
}

}  // extern "C"

namespace {
// Argument checks and kernel arguments of one compress call ("what" names the
// entry point in the error text); `empty` is set when there is nothing to do.
csa_status compress_args(const char* what, const void* x, csa_fmt x_fmt, const float* gate,
                         int gate_cols, int64_t n_tok, int D, int m, int nseg,
                         const int64_t* seg_tok_off, const int64_t* seg_pos0,
                         const int64_t* seg_out_row, int normalize, const float* norm_w, float eps,
                         int rope_dim, float rope_base, void* out, csa_fmt out_fmt,
                         CompressArgs* a, bool* empty) {
  *empty = false;
  if (n_tok < 0) return fail(CSA_ERR_INVALID_ARG, "%s: n_tok < 0", what);
  if (m < 1) return fail(CSA_ERR_INVALID_ARG, "%s: m must be >= 1", what);
  if (D < 2) return fail(CSA_ERR_INVALID_ARG, "%s: D must be >= 2", what);
  if (D > 4096) return fail(CSA_ERR_UNSUPPORTED, "%s: D > 4096", what);
  if (n_tok % m != 0) return fail(CSA_ERR_INVALID_ARG, "%s: n_tok %% m != 0", what);
  if (x_fmt != CSA_F32 && x_fmt != CSA_BF16)
    return fail(CSA_ERR_INVALID_ARG, "%s: x_fmt must be CSA_F32 or CSA_BF16", what);
  if (!fmt_ok(out_fmt)) return fail(CSA_ERR_INVALID_ARG, "%s: bad out_fmt", what);
  if (gate_cols != 1 && gate_cols != D)
    return fail(CSA_ERR_INVALID_ARG, "%s: gate_cols must be 1 or D", what);
  if (rope_dim < 0 || rope_dim % 2 != 0 || rope_dim > D || rope_dim > 2 * kMaxRopePairs)
    return fail(CSA_ERR_INVALID_ARG, "%s: rope_dim must be even, <= D and <= 128", what);
  if (rope_dim > 0 && !(rope_base > 0.0f))
    return fail(CSA_ERR_INVALID_ARG, "%s: rope_base must be > 0", what);
  if (out_fmt == CSA_MXFP4 && D % 32 != 0)
    return fail(CSA_ERR_INVALID_ARG, "%s: MXFP4 needs D %% 32 == 0", what);
  if (out_fmt == CSA_SPLIT && (rope_dim == 0 || D - rope_dim < 1))
    return fail(CSA_ERR_INVALID_ARG, "%s: SPLIT needs 0 < rope_dim < D", what);
  if (nseg < 1) return fail(CSA_ERR_INVALID_ARG, "%s: nseg must be >= 1", what);
  if (!(eps >= 0.0f)) return fail(CSA_ERR_INVALID_ARG, "%s: eps must be >= 0", what);
  if (n_tok == 0) { *empty = true; return CSA_OK; }
  if (!x || !gate || !seg_tok_off || !seg_pos0 || !seg_out_row || !out)
    return fail(CSA_ERR_INVALID_ARG, "%s: null pointer", what);
  *a = CompressArgs{x, x_fmt, gate, gate_cols, n_tok, D, m, nseg, seg_tok_off, seg_pos0, seg_out_row,
                    normalize, norm_w, eps, rope_dim, rope_base, out, out_fmt, {}};
  fill_rope_theta(a->rope_theta, rope_dim, rope_base);
  return CSA_OK;
}
}  // namespace

extern "C" {

csa_status csa_compress(const void* x, csa_fmt x_fmt, const float* gate, int gate_cols,
                        int64_t n_tok, int D, int m, int nseg, const int64_t* seg_tok_off,
                        const int64_t* seg_pos0, const int64_t* seg_out_row, int normalize,
                        const float* norm_w, float eps, int rope_dim, float rope_base, void* out,
                        csa_fmt out_fmt, hipStream_t stream) {
  CompressArgs a{};
  bool empty = false;
  const csa_status st = compress_args("csa_compress", x, x_fmt, gate, gate_cols, n_tok, D, m, nseg,
                                      seg_tok_off, seg_pos0, seg_out_row, normalize, norm_w, eps,
                                      rope_dim, rope_base, out, out_fmt, &a, &empty);
  if (st != CSA_OK) return st;
  if (empty) { g_err[0] = '\0'; return CSA_OK; }
  return launched(launch_compress(a, stream), "csa_compress");
}

}  // extern "C"

namespace {
csa_status batch_args(const char* what, const csa_compress_job* jobs, int n_jobs, int key,
                      CompressArgs* a, int* n, int* map_key);
}  // namespace

extern "C" {

csa_status csa_compress_batch(const csa_compress_job* jobs, int n_jobs, hipStream_t stream) {
  CompressArgs a[CSA_COMPRESS_MAX_JOBS];
  int n = 0, unused = -1;
  const csa_status st = batch_args("csa_compress_batch", jobs, n_jobs, -1, a, &n, &unused);
  if (st != CSA_OK) return st;
  if (n == 0) { g_err[0] = '\0'; return CSA_OK; }
  return launched(launch_compress_jobs(a, n, stream), "csa_compress_batch");
}

}  // extern "C"

namespace {
// Argument checks of one indexer call; `empty` is set for nq == 0.
csa_status indexer_args(const char* what, const void* q_idx, const float* w, int nq, int n_heads,
                        int d_idx, const void* keys, csa_fmt fmt, const int64_t* key_off,
                        const int64_t* q_pos, int m, float* scores, int64_t ld, IndexerArgs* a,
                        bool* empty) {
  *empty = false;
  if (nq < 0) return fail(CSA_ERR_INVALID_ARG, "%s: nq < 0", what);
  if (n_heads < 1 || d_idx < 1) return fail(CSA_ERR_INVALID_ARG, "%s: n_heads, d_idx must be >= 1", what);
  if (m < 1) return fail(CSA_ERR_INVALID_ARG, "%s: m must be >= 1", what);
  if (ld < 1 || ld > (int64_t{1} << 24))
    return fail(CSA_ERR_INVALID_ARG, "%s: ld must be in [1, 2^24]", what);
  if (fmt != CSA_F32 && fmt != CSA_FP8 && fmt != CSA_MXFP4)
    return fail(CSA_ERR_INVALID_ARG, "%s: fmt must be CSA_F32, CSA_FP8 or CSA_MXFP4", what);
  if (fmt == CSA_F32) {
    if (n_heads > 64 || d_idx > 256)
      return fail(CSA_ERR_UNSUPPORTED, "%s: F32 path supports n_heads <= 64, d_idx <= 256", what);
  } else {
    if (d_idx != 128 || n_heads % 16 != 0 || n_heads > 128)
      return fail(CSA_ERR_UNSUPPORTED, "%s: FP8/MXFP4 paths need d_idx == 128 and n_heads in {16,32,64,128}", what);
    if (n_heads == 48 || n_heads == 80 || n_heads == 96 || n_heads == 112)
      return fail(CSA_ERR_UNSUPPORTED, "%s: n_heads must be 16, 32, 64 or 128", what);
  }
  if (nq == 0) { *empty = true; return CSA_OK; }
  if (!q_idx || !w || !keys || !key_off || !q_pos || !scores)
    return fail(CSA_ERR_INVALID_ARG, "%s: null pointer", what);
  *a = IndexerArgs{q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores, ld};
  return CSA_OK;
}

// Checks of a csa_compress_batch job list; the non-empty jobs go to a[0 .. *n).
// *map_key receives the index in a[] of the input job `key` (-1 if it is empty).
csa_status batch_args(const char* what, const csa_compress_job* jobs, int n_jobs, int key,
                      CompressArgs* a, int* n, int* map_key) {
  if (n_jobs < 0 || n_jobs > CSA_COMPRESS_MAX_JOBS)
    return fail(CSA_ERR_INVALID_ARG, "%s: n_jobs must be in [0, %d]", what, CSA_COMPRESS_MAX_JOBS);
  if (n_jobs > 0 && !jobs) return fail(CSA_ERR_INVALID_ARG, "%s: null jobs", what);
  *n = 0;
  *map_key = -1;
  for (int i = 0; i < n_jobs; ++i) {
    const csa_compress_job& j = jobs[i];
    char w[64];
    snprintf(w, sizeof(w), "%s: job %d", what, i);
    bool empty = false;
    const csa_status st = compress_args(w, j.x, j.x_fmt, j.gate, j.gate_cols, j.n_tok, j.D, j.m,
                                        j.nseg, j.seg_tok_off, j.seg_pos0, j.seg_out_row,
                                        j.normalize, j.norm_w, j.eps, j.rope_dim, j.rope_base,
                                        j.out, j.out_fmt, &a[*n], &empty);
    if (st != CSA_OK) return st;
    if (!empty) {
      if (i == key) *map_key = *n;
      ++*n;
    }
  }
  return CSA_OK;
}
}  // namespace

extern "C" {

csa_status indexer_score(const void* q_idx, const float* w, int nq, int n_heads, int d_idx,
                         const void* keys, csa_fmt fmt, const int64_t* key_off,
                         const int64_t* q_pos, int m, float* scores, int64_t ld,
                         hipStream_t stream) {
  IndexerArgs a{};
  bool empty = false;
  const csa_status st = indexer_args("indexer_score", q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off,
                                     q_pos, m, scores, ld, &a, &empty);
  if (st != CSA_OK) return st;
  if (empty) { g_err[0] = '\0'; return CSA_OK; }
  return launched(launch_indexer(a, stream), "indexer_score");
}

// The paged indexer's arguments: the checks of indexer_score plus the block
// geometry; *empty when there is nothing to score.
static csa_status paged_args(const char* what, const void* q_idx, const float* w, int nq, int n_heads, int d_idx,
                             const void* key_pool, csa_fmt fmt, int64_t pool_rows, const int32_t* block_table,
                             int64_t table_rows, int64_t blocks_per_seq, int block_rows, const int32_t* q_block_row,
                             const int64_t* q_pos, int m, float* scores, int64_t ld, IndexerArgs* a, bool* empty) {
  if (fmt == CSA_F32) return fail(CSA_ERR_UNSUPPORTED, "%s: the paged path takes FP8 or MXFP4 keys", what);
  // (block_table stands in for key_off in the shared null-pointer check)
  const csa_status st = indexer_args(what, q_idx, w, nq, n_heads, d_idx, key_pool, fmt,
                                     reinterpret_cast<const int64_t*>(block_table), q_pos, m, scores, ld, a, empty);
  if (st != CSA_OK) return st;
  if (block_rows < 16 || block_rows > (1 << 20) || (block_rows & (block_rows - 1)) != 0)
    return fail(CSA_ERR_INVALID_ARG, "%s: block_rows must be a power of two in [16, 2^20]", what);
  if (blocks_per_seq < 1 || blocks_per_seq > (int64_t{1} << 26))
    return fail(CSA_ERR_INVALID_ARG, "%s: blocks_per_seq must be in [1, 2^26]", what);
  if (table_rows < 1 || table_rows > (int64_t{1} << 31))
    return fail(CSA_ERR_INVALID_ARG, "%s: table_rows must be in [1, 2^31]", what);
  if (pool_rows < 1) return fail(CSA_ERR_INVALID_ARG, "%s: pool_rows must be >= 1", what);
  if (static_cast<uint64_t>(pool_rows) * row_bytes(fmt, d_idx, 0) > 0xffffffffull)
    return fail(CSA_ERR_UNSUPPORTED, "%s: the key pool must be smaller than 4 GiB", what);
  if (!q_block_row && table_rows < nq)
    return fail(CSA_ERR_INVALID_ARG, "%s: without q_block_row, query i reads table row i (table_rows < nq)", what);
  a->key_off = nullptr;
  a->blk_table = block_table;
  a->blk_stride = blocks_per_seq;
  a->blk_shift = __builtin_ctz(static_cast<unsigned>(block_rows));
  a->pool_rows = pool_rows;
  a->blk_row = q_block_row;
  a->blk_rows = table_rows;
  return CSA_OK;
}

static csa_status indexer_paged(const char* what, const void* q_idx, const float* w, int nq, int n_heads,
                                int d_idx, const void* key_pool, csa_fmt fmt, int64_t pool_rows,
                                const int32_t* block_table, int64_t table_rows, int64_t blocks_per_seq,
                                int block_rows, const int32_t* q_block_row, const int64_t* q_pos, int m,
                                float* scores, int64_t ld, hipStream_t stream) {
  IndexerArgs a{};
  bool empty = false;
  const csa_status st = paged_args(what, q_idx, w, nq, n_heads, d_idx, key_pool, fmt, pool_rows, block_table,
                                   table_rows, blocks_per_seq, block_rows, q_block_row, q_pos, m, scores, ld, &a,
                                   &empty);
  if (st != CSA_OK) return st;
  if (empty) { g_err[0] = '\0'; return CSA_OK; }
  return launched(launch_indexer(a, stream), what);
}

csa_status indexer_score_paged(const void* q_idx, const float* w, int nq, int n_heads, int d_idx,
                               const void* key_pool, csa_fmt fmt, int64_t pool_rows,
                               const int32_t* block_table, int64_t blocks_per_seq, int block_rows,
                               const int64_t* q_pos, int m, float* scores, int64_t ld, hipStream_t stream) {
  return indexer_paged("indexer_score_paged", q_idx, w, nq, n_heads, d_idx, key_pool, fmt, pool_rows, block_table,
                       nq > 0 ? nq : 1, blocks_per_seq, block_rows, nullptr, q_pos, m, scores, ld, stream);
}

csa_status indexer_score_paged_rows(const void* q_idx, const float* w, int nq, int n_heads, int d_idx,
                                    const void* key_pool, csa_fmt fmt, int64_t pool_rows,
                                    const int32_t* block_table, int64_t table_rows, int64_t blocks_per_seq,
                                    int block_rows, const int32_t* q_block_row, const int64_t* q_pos, int m,
                                    float* scores, int64_t ld, hipStream_t stream) {
  return indexer_paged("indexer_score_paged_rows", q_idx, w, nq, n_heads, d_idx, key_pool, fmt, pool_rows,
                       block_table, table_rows, blocks_per_seq, block_rows, q_block_row, q_pos, m, scores, ld,
                       stream);
}

// The jobs of a compress + score call (the key job: the one that writes
// `keys`) and its launch; ia holds the indexer's arguments.
// tk: the fused top-k of csa_compress_score_topk (its checks done), or null.
static csa_status compress_score_common(const char* what, const csa_compress_job* jobs, int n_jobs,
                                        const void* keys, csa_fmt fmt, int d_idx, int nq, const IndexerArgs& ia,
                                        bool no_queries, hipStream_t stream, const TopkFuse* tk = nullptr) {
  int key = -1;
  if (n_jobs > 0 && jobs) {
    for (int i = 0; i < n_jobs && i < CSA_COMPRESS_MAX_JOBS; ++i) {
      if (!keys || jobs[i].out != keys) continue;
      if (key >= 0) return fail(CSA_ERR_INVALID_ARG, "%s: jobs %d and %d both write `keys`", what, key, i);
      key = i;
    }
  }
  if (key >= 0 && !no_queries) {
    const csa_compress_job& kjob = jobs[key];
    if (kjob.out_fmt != fmt || kjob.D != d_idx || kjob.rope_dim != 0 || kjob.nseg != nq)
      return fail(CSA_ERR_INVALID_ARG,
                  "%s: job %d writes `keys`, so it needs out_fmt == fmt, D == d_idx, rope_dim == 0 "
                  "and one segment per query (nseg == nq)", what, key);
  }
  CompressArgs a[CSA_COMPRESS_MAX_JOBS];
  int n = 0, map_key = -1;
  const csa_status st = batch_args(what, jobs, n_jobs, key, a, &n, &map_key);
  if (st != CSA_OK) return st;
  hipError_t e = hipSuccess;
  if (no_queries) e = n > 0 ? launch_compress_jobs(a, n, stream) : hipSuccess;
  else if (tk) e = launch_compress_score_topk(a, n, map_key, ia, *tk, stream);
  else e = launch_compress_score(a, n, map_key, ia, stream);
  return launched(e, what);
}

// Checks of the selection arguments of csa_compress_score_topk(_paged).
static csa_status score_topk_args(const char* what, int nq, csa_fmt fmt, int k, int32_t* idx, void* workspace,
                                  size_t ws_bytes, TopkFuse* tk) {
  if (k < 1 || k > 4096) return fail(CSA_ERR_INVALID_ARG, "%s: k must be in [1, 4096]", what);
  if (nq <= 0) { *tk = TopkFuse{idx, static_cast<uint32_t*>(workspace), k}; return CSA_OK; }
  if (!idx) return fail(CSA_ERR_INVALID_ARG, "%s: null idx", what);
  if (fmt != CSA_FP8) return fail(CSA_ERR_UNSUPPORTED, "%s: the fused selection takes FP8 keys", what);
  if (nq >= kShareMinQueries)
    return fail(CSA_ERR_UNSUPPORTED, "%s: batches of %d queries or more take indexer_score + topk_select", what,
                kShareMinQueries);
  const size_t need = csa_score_topk_workspace_bytes(nq);
  if (!workspace || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "%s: %d queries need a %zu-byte zeroed workspace, got %zu%s", what, nq, need,
                ws_bytes, workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(CSA_ERR_WORKSPACE, "%s: the workspace must be 256-byte aligned", what);
  *tk = TopkFuse{idx, static_cast<uint32_t*>(workspace), k};
  return CSA_OK;
}

csa_status csa_compress_score(const csa_compress_job* jobs, int n_jobs, const void* q_idx,
                              const float* w, int nq, int n_heads, int d_idx, const void* keys,
                              csa_fmt fmt, const int64_t* key_off, const int64_t* q_pos, int m,
                              float* scores, int64_t ld, hipStream_t stream) {
  const char* what = "csa_compress_score";
  IndexerArgs ia{};
  bool no_queries = false;
  const csa_status st = indexer_args(what, q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores,
                                     ld, &ia, &no_queries);
  if (st != CSA_OK) return st;
  return compress_score_common(what, jobs, n_jobs, keys, fmt, d_idx, nq, ia, no_queries, stream);
}

csa_status csa_compress_score_paged(const csa_compress_job* jobs, int n_jobs, const void* q_idx, const float* w,
                                    int nq, int n_heads, int d_idx, const void* key_pool, csa_fmt fmt,
                                    int64_t pool_rows, const int32_t* block_table, int64_t table_rows,
                                    int64_t blocks_per_seq, int block_rows, const int32_t* q_block_row,
                                    const int64_t* q_pos, int m, float* scores, int64_t ld, hipStream_t stream) {
  const char* what = "csa_compress_score_paged";
  IndexerArgs ia{};
  bool no_queries = false;
  const csa_status st = paged_args(what, q_idx, w, nq, n_heads, d_idx, key_pool, fmt, pool_rows, block_table,
                                   table_rows, blocks_per_seq, block_rows, q_block_row, q_pos, m, scores, ld, &ia,
                                   &no_queries);
  if (st != CSA_OK) return st;
  return compress_score_common(what, jobs, n_jobs, key_pool, fmt, d_idx, nq, ia, no_queries, stream);
}

csa_status csa_select_and_pad(const void* in, int n_shards, int64_t cap, int64_t row_bytes,
                              const int64_t* n_valid, void* out, hipStream_t stream) {
  const char* what = "csa_select_and_pad";
  if (n_shards < 1 || n_shards > kSelectPadMaxShards)
    return fail(CSA_ERR_INVALID_ARG, "%s: n_shards must be in [1, %d]", what, kSelectPadMaxShards);
  if (cap < 0 || cap > (int64_t{1} << 31)) return fail(CSA_ERR_INVALID_ARG, "%s: cap must be in [0, 2^31]", what);
  if (row_bytes < 4 || row_bytes % 4 != 0 || row_bytes > (int64_t{1} << 20))
    return fail(CSA_ERR_INVALID_ARG, "%s: row_bytes must be a multiple of 4 in [4, 2^20]", what);
  if (cap == 0) { g_err[0] = '\0'; return CSA_OK; }
  if (!in || !out || !n_valid) return fail(CSA_ERR_INVALID_ARG, "%s: null pointer", what);
  if ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) % 4 != 0)
    return fail(CSA_ERR_INVALID_ARG, "%s: in and out must be 4-byte aligned", what);
  const uint8_t* i0 = static_cast<const uint8_t*>(in);
  const uint8_t* o0 = static_cast<const uint8_t*>(out);
  const int64_t bytes = static_cast<int64_t>(n_shards) * cap * row_bytes;
  if (i0 < o0 + bytes && o0 < i0 + bytes) return fail(CSA_ERR_INVALID_ARG, "%s: in and out overlap", what);
  return launched(launch_select_pad(in, n_shards, cap, row_bytes, n_valid, out, stream), what);
}

size_t csa_score_topk_workspace_bytes(int nq) {
  return nq <= 0 || nq >= kShareMinQueries ? 0 : static_cast<size_t>(nq) * kTkWsWords * sizeof(uint32_t);
}

csa_status csa_compress_score_topk(const csa_compress_job* jobs, int n_jobs, const void* q_idx, const float* w,
                                   int nq, int n_heads, int d_idx, const void* keys, csa_fmt fmt,
                                   const int64_t* key_off, const int64_t* q_pos, int m, float* scores, int64_t ld,
                                   int k, int32_t* idx, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const char* what = "csa_compress_score_topk";
  IndexerArgs ia{};
  bool no_queries = false;
  csa_status st = indexer_args(what, q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores, ld, &ia,
                               &no_queries);
  if (st != CSA_OK) return st;
  TopkFuse tk{};
  st = score_topk_args(what, nq, fmt, k, idx, workspace, ws_bytes, &tk);
  if (st != CSA_OK) return st;
  return compress_score_common(what, jobs, n_jobs, keys, fmt, d_idx, nq, ia, no_queries, stream, &tk);
}

csa_status csa_compress_score_topk_paged(const csa_compress_job* jobs, int n_jobs, const void* q_idx,
                                         const float* w, int nq, int n_heads, int d_idx, const void* key_pool,
                                         csa_fmt fmt, int64_t pool_rows, const int32_t* block_table,
                                         int64_t table_rows, int64_t blocks_per_seq, int block_rows,
                                         const int32_t* q_block_row, const int64_t* q_pos, int m, float* scores,
                                         int64_t ld, int k, int32_t* idx, void* workspace, size_t ws_bytes,
                                         hipStream_t stream) {
  const char* what = "csa_compress_score_topk_paged";
  IndexerArgs ia{};
  bool no_queries = false;
  csa_status st = paged_args(what, q_idx, w, nq, n_heads, d_idx, key_pool, fmt, pool_rows, block_table,
                             table_rows, blocks_per_seq, block_rows, q_block_row, q_pos, m, scores, ld, &ia,
                             &no_queries);
  if (st != CSA_OK) return st;
  TopkFuse tk{};
  st = score_topk_args(what, nq, fmt, k, idx, workspace, ws_bytes, &tk);
  if (st != CSA_OK) return st;
  return compress_score_common(what, jobs, n_jobs, key_pool, fmt, d_idx, nq, ia, no_queries, stream, &tk);
}

size_t csa_topk_workspace_bytes(int nq, int64_t ld, int k) {
  if (nq <= 0 || ld < 1 || k < 1 || k > 4096 || ld > (int64_t{1} << 28)) return 0;
  return plan_topk(ld, nq, k).ws_bytes;
}

namespace {
// Checks shared by both top-k entry points; *pl receives the launch plan.
csa_status topk_check(const char* name, const float* scores, int64_t ld, int nq, int k, const int32_t* idx,
                      TopkPlan* pl) {
  if (nq < 0) return fail(CSA_ERR_INVALID_ARG, "%s: nq < 0", name);
  if (k < 1 || k > 4096) return fail(CSA_ERR_INVALID_ARG, "%s: k must be in [1, 4096]", name);
  if (ld < 1 || ld > (int64_t{1} << 28)) return fail(CSA_ERR_INVALID_ARG, "%s: ld must be in [1, 2^28]", name);
  if (nq > kTopkMaxRows) return fail(CSA_ERR_INVALID_ARG, "%s: nq must be <= %d", name, kTopkMaxRows);
  if (nq == 0) return CSA_OK;
  if (!scores || !idx) return fail(CSA_ERR_INVALID_ARG, "%s: null pointer", name);
  *pl = plan_topk(ld, nq, k);
  if (static_cast<int64_t>(nq) * pl->P > kTopkMaxRows)
    return fail(CSA_ERR_INVALID_ARG, "%s: nq * %d slices exceeds %d workgroups", name, pl->P, kTopkMaxRows);
  return CSA_OK;
}
}  // namespace

csa_status topk_select(const float* scores, int64_t ld, int nq, const int64_t* n_valid, int k,
                       int32_t* idx, float* top_scores, void* workspace, size_t ws_bytes,
                       hipStream_t stream) {
  TopkPlan pl{};
  const csa_status st = topk_check("topk_select", scores, ld, nq, k, idx, &pl);
  if (st != CSA_OK) return st;
  if (nq == 0) { g_err[0] = '\0'; return CSA_OK; }
  if (pl.ws_bytes > 0) {
    if (!workspace || ws_bytes < pl.ws_bytes)
      return fail(CSA_ERR_WORKSPACE, "topk_select: rows of %lld scores need a %zu-byte workspace, got %zu%s",
                  static_cast<long long>(ld), pl.ws_bytes, workspace ? ws_bytes : size_t{0},
                  workspace ? "" : " (NULL)");
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return fail(CSA_ERR_WORKSPACE, "topk_select: the workspace must be 16-byte aligned");
  }
  TopkArgs a{scores, ld, nq, n_valid, k, idx, top_scores};
  return launched(launch_topk(a, workspace, stream), "topk_select");
}

size_t csa_topk_noalloc_max_bytes(void) { return kTopkScratchBytes; }

csa_status topk_select_noalloc(const float* scores, int64_t ld, int nq, const int64_t* n_valid, int k,
                               int32_t* idx, float* top_scores, hipStream_t stream) {
  TopkPlan pl{};
  const csa_status st = topk_check("topk_select_noalloc", scores, ld, nq, k, idx, &pl);
  if (st != CSA_OK) return st;
  if (nq == 0) { g_err[0] = '\0'; return CSA_OK; }
  if (pl.ws_bytes > kTopkScratchBytes)
    return fail(CSA_ERR_WORKSPACE,
                "topk_select_noalloc: %d rows of %lld scores at k=%d need %zu bytes of candidates; the static "
                "scratch holds %zu (use topk_select with a workspace)",
                nq, static_cast<long long>(ld), k, pl.ws_bytes, kTopkScratchBytes);
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    const hipError_t e = topk_scratch(&ws);
    if (e != hipSuccess)
      return fail(CSA_ERR_HIP, "topk_select_noalloc: scratch address lookup failed: %s", hipGetErrorString(e));
  }
  TopkArgs a{scores, ld, nq, n_valid, k, idx, top_scores};
  return launched(launch_topk(a, ws, stream), "topk_select_noalloc");
}

static csa_status attn_common(const char* name, AttnArgs& a, hipStream_t stream) {
  if (a.nq < 0) return fail(CSA_ERR_INVALID_ARG, "%s: query count < 0", name);
  if (a.H < 1 || a.D < 2) return fail(CSA_ERR_INVALID_ARG, "%s: H, D must be positive", name);
  if (a.m < 1) return fail(CSA_ERR_INVALID_ARG, "%s: m must be >= 1", name);
  if (a.n_win < 0) return fail(CSA_ERR_INVALID_ARG, "%s: n_win < 0", name);
  if (a.idx != nullptr && a.k < 1) return fail(CSA_ERR_INVALID_ARG, "%s: k must be >= 1 with idx", name);
  if (a.rope_dim < 0 || a.rope_dim % 2 != 0 || a.rope_dim > a.D || a.rope_dim > 2 * kMaxRopePairs)
    return fail(CSA_ERR_INVALID_ARG, "%s: rope_dim must be even, <= D and <= 128", name);
  if (a.rope_dim > 0 && !(a.rope_base > 0.0f))
    return fail(CSA_ERR_INVALID_ARG, "%s: rope_base must be > 0", name);
  if (!(a.eps >= 0.0f)) return fail(CSA_ERR_INVALID_ARG, "%s: eps must be >= 0", name);
  if (a.variant < CSA_VARIANT_AUTO || a.variant > CSA_VARIANT_FULL_DIMS)
    return fail(CSA_ERR_INVALID_ARG, "%s: bad variant", name);
  if (!fmt_ok(a.q_fmt) || !fmt_ok(a.kv_fmt) || !fmt_ok(a.win_fmt) || !fmt_ok(a.out_fmt))
    return fail(CSA_ERR_INVALID_ARG, "%s: bad format", name);
  const bool all_f32 = a.q_fmt == CSA_F32 && a.kv_fmt == CSA_F32 && a.win_fmt == CSA_F32 &&
                       a.out_fmt == CSA_F32;
  const bool mfma = a.q_fmt == CSA_BF16 && a.kv_fmt == CSA_SPLIT && a.win_fmt == CSA_BF16 &&
                    a.out_fmt == CSA_BF16;
  if (all_f32) {
    if (a.D % 128 != 0 || a.D > 512)
      return fail(CSA_ERR_UNSUPPORTED, "%s: F32 path needs D in {128, 256, 384, 512}", name);
  } else if (mfma) {
    if (a.D != 512 || a.rope_dim != 64)
      return fail(CSA_ERR_UNSUPPORTED, "%s: MFMA path needs D == 512 and rope_dim == 64", name);
    if (a.H % 16 != 0) return fail(CSA_ERR_UNSUPPORTED, "%s: MFMA path needs H %% 16 == 0", name);
  } else {
    return fail(CSA_ERR_UNSUPPORTED,
                "%s: supported formats are all-F32, or q/win/out BF16 with a SPLIT cache", name);
  }
  if (a.nq == 0) { g_err[0] = '\0'; return CSA_OK; }
  if (!a.q || !a.q_pos || !a.kv || (!a.kv_off && !a.blk_table) || !a.sinks || !a.out)
    return fail(CSA_ERR_INVALID_ARG, "%s: null pointer", name);
  if (a.n_win > 0 && !a.win) return fail(CSA_ERR_INVALID_ARG, "%s: null window pointer", name);
  fill_rope_theta(a.rope_theta, a.rope_dim, a.rope_base);
  return launched(launch_attn(a, stream), name);
}

csa_status hybrid_attn_decode(const void* q, csa_fmt q_fmt, int B, int H, int D,
                              const int64_t* q_pos, const float* q_norm_w, float eps,
                              int rope_dim, float rope_base, const void* kv, csa_fmt kv_fmt,
                              const int64_t* kv_off, int m, const int32_t* idx, int k,
                              const void* win, csa_fmt win_fmt, int n_win,
                              const int32_t* win_len, const float* sinks, float scale,
                              void* out, csa_fmt out_fmt, csa_variant variant,
                              hipStream_t stream) {
  if (B > 0 && n_win > 0 && !win_len)
    return fail(CSA_ERR_INVALID_ARG, "hybrid_attn_decode: null win_len");
  AttnArgs a{q, q_fmt, B, H, D, q_pos, q_norm_w, eps, rope_dim, rope_base, kv, kv_fmt, kv_off, m,
             idx, k, win, win_fmt, n_win, n_win > 0 ? 1 : 0, win_len, nullptr, nullptr, sinks,
             scale, out, out_fmt, static_cast<int>(variant), {}};
  return attn_common("hybrid_attn_decode", a, stream);
}

csa_status hybrid_attn_decode_paged(const void* q, csa_fmt q_fmt, int B, int H, int D,
                                    const int64_t* q_pos, const float* q_norm_w, float eps,
                                    int rope_dim, float rope_base, const void* kv_pool, csa_fmt kv_fmt,
                                    int64_t pool_rows, const int32_t* block_table, int64_t blocks_per_seq,
                                    int block_rows, int m, const int32_t* idx, int k,
                                    const void* win, csa_fmt win_fmt, int n_win,
                                    const int32_t* win_start, const int32_t* win_len, const float* sinks,
                                    float scale, void* out, csa_fmt out_fmt, csa_variant variant,
                                    hipStream_t stream) {
  const char* what = "hybrid_attn_decode_paged";
  if (B > 0 && n_win > 0 && !win_len) return fail(CSA_ERR_INVALID_ARG, "%s: null win_len", what);
  if (!(q_fmt == CSA_BF16 && kv_fmt == CSA_SPLIT && win_fmt == CSA_BF16 && out_fmt == CSA_BF16))
    return fail(CSA_ERR_UNSUPPORTED, "%s: the paged path is the MFMA path (BF16 q / window / out, SPLIT cache)",
                what);
  if (block_rows < 1 || block_rows > (1 << 20) || (block_rows & (block_rows - 1)) != 0)
    return fail(CSA_ERR_INVALID_ARG, "%s: block_rows must be a power of two in [1, 2^20]", what);
  if (blocks_per_seq < 1 || blocks_per_seq > (int64_t{1} << 26))
    return fail(CSA_ERR_INVALID_ARG, "%s: blocks_per_seq must be in [1, 2^26]", what);
  if (pool_rows < 1) return fail(CSA_ERR_INVALID_ARG, "%s: pool_rows must be >= 1", what);
  if (static_cast<uint64_t>(pool_rows) * row_bytes(CSA_SPLIT, D, rope_dim) > 0xffffffffull)
    return fail(CSA_ERR_UNSUPPORTED, "%s: the entry pool must be smaller than 4 GiB", what);
  if (B > 0 && !block_table) return fail(CSA_ERR_INVALID_ARG, "%s: null block_table", what);
  AttnArgs a{q, q_fmt, B, H, D, q_pos, q_norm_w, eps, rope_dim, rope_base, kv_pool, kv_fmt, nullptr, m,
             idx, k, win, win_fmt, n_win, n_win > 0 ? 1 : 0, win_len, nullptr, nullptr, sinks,
             scale, out, out_fmt, static_cast<int>(variant), {}, block_table, blocks_per_seq,
             __builtin_ctz(static_cast<unsigned>(block_rows)), pool_rows, win_start, nullptr, B};
  return attn_common(what, a, stream);
}

csa_status hybrid_attn_prefill(const void* q, csa_fmt q_fmt, int nq, int H, int D,
                               const int64_t* q_pos, const float* q_norm_w, float eps,
                               int rope_dim, float rope_base, const void* kv, csa_fmt kv_fmt,
                               const int64_t* kv_off, int m, const int32_t* idx, int k,
                               const void* tok, csa_fmt tok_fmt, const int64_t* tok_off,
                               const int64_t* tok_pos0, int n_win, const float* sinks,
                               float scale, void* out, csa_fmt out_fmt, csa_variant variant,
                               hipStream_t stream) {
  if (nq > 0 && n_win > 0 && (!tok_off || !tok_pos0))
    return fail(CSA_ERR_INVALID_ARG, "hybrid_attn_prefill: null tok_off / tok_pos0");
  AttnArgs a{q, q_fmt, nq, H, D, q_pos, q_norm_w, eps, rope_dim, rope_base, kv, kv_fmt, kv_off, m,
             idx, k, tok, tok_fmt, n_win, n_win > 0 ? 2 : 0, nullptr, tok_off, tok_pos0, sinks,
             scale, out, out_fmt, static_cast<int>(variant), {}};
  return attn_common("hybrid_attn_prefill", a, stream);
}

csa_status hybrid_attn_prefill_paged(const void* q, csa_fmt q_fmt, int nq, int H, int D,
                                     const int64_t* q_pos, const float* q_norm_w, float eps,
                                     int rope_dim, float rope_base, const void* kv_pool, csa_fmt kv_fmt,
                                     int64_t pool_rows, const int32_t* block_table, int64_t table_rows,
                                     int64_t blocks_per_seq, int block_rows, const int32_t* q_block_row,
                                     int m, const int32_t* idx, int k, const void* tok, csa_fmt tok_fmt,
                                     const int64_t* tok_off, const int64_t* tok_pos0, int n_win,
                                     const float* sinks, float scale, void* out, csa_fmt out_fmt,
                                     csa_variant variant, hipStream_t stream) {
  const char* what = "hybrid_attn_prefill_paged";
  if (nq > 0 && n_win > 0 && (!tok_off || !tok_pos0))
    return fail(CSA_ERR_INVALID_ARG, "%s: null tok_off / tok_pos0", what);
  if (!(q_fmt == CSA_BF16 && kv_fmt == CSA_SPLIT && tok_fmt == CSA_BF16 && out_fmt == CSA_BF16))
    return fail(CSA_ERR_UNSUPPORTED, "%s: the paged path is the MFMA path (BF16 q / window / out, SPLIT cache)",
                what);
  if (block_rows < 1 || block_rows > (1 << 20) || (block_rows & (block_rows - 1)) != 0)
    return fail(CSA_ERR_INVALID_ARG, "%s: block_rows must be a power of two in [1, 2^20]", what);
  if (blocks_per_seq < 1 || blocks_per_seq > (int64_t{1} << 26))
    return fail(CSA_ERR_INVALID_ARG, "%s: blocks_per_seq must be in [1, 2^26]", what);
  if (table_rows < 1 || table_rows > (int64_t{1} << 31))
    return fail(CSA_ERR_INVALID_ARG, "%s: table_rows must be in [1, 2^31]", what);
  if (pool_rows < 1) return fail(CSA_ERR_INVALID_ARG, "%s: pool_rows must be >= 1", what);
  if (static_cast<uint64_t>(pool_rows) * row_bytes(CSA_SPLIT, D, rope_dim) > 0xffffffffull)
    return fail(CSA_ERR_UNSUPPORTED, "%s: the entry pool must be smaller than 4 GiB", what);
  if (nq > 0 && !block_table) return fail(CSA_ERR_INVALID_ARG, "%s: null block_table", what);
  if (nq > 0 && !q_block_row && table_rows < nq)
    return fail(CSA_ERR_INVALID_ARG, "%s: without q_block_row, query i reads table row i (table_rows < nq)", what);
  AttnArgs a{q, q_fmt, nq, H, D, q_pos, q_norm_w, eps, rope_dim, rope_base, kv_pool, kv_fmt, nullptr, m,
             idx, k, tok, tok_fmt, n_win, n_win > 0 ? 2 : 0, nullptr, tok_off, tok_pos0, sinks,
             scale, out, out_fmt, static_cast<int>(variant), {}, block_table, blocks_per_seq,
             __builtin_ctz(static_cast<unsigned>(block_rows)), pool_rows, nullptr, q_block_row, table_rows};
  return attn_common(what, a, stream);
}

csa_status csa_debug_poison_lds(uint32_t pattern, hipStream_t stream) {
  static thread_local int attr_dev = -1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CSA_ERR_HIP, "csa_debug_poison_lds: no device");
  if (attr_dev != dev) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&poison_lds_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(kLdsBytesPerCu));
    if (e != hipSuccess) return launched(e, "csa_debug_poison_lds");
    attr_dev = dev;
  }
  // four workgroups per CU, each holding the whole LDS, so every CU runs some
  hipLaunchKernelGGL(poison_lds_kernel, dim3(static_cast<unsigned>(device_cu_count()) * 4), dim3(1024),
                     kLdsBytesPerCu, stream, pattern);
  return launched(hipGetLastError(), "csa_debug_poison_lds");
}

}  // extern "C"
