/*
 * csa.h -- C ABI of libcsa: the CSA / HCA hybrid compressed attention path of
 * DeepSeek-V4 on AMD Instinct MI355X (gfx950).
 *
 * Sources (page title -- section):
 *   "DeepSeek-V4" blog (haiqwa.github.io): CSA / HCA sections, RMSNorm归一化,
 *       Partial RoPE位置编码, 让注意力学会"忽略" (sink), FP4精度加速 (FP4 indexer),
 *       百万 token 怎么切分到多张卡 (index visibility rule);
 *   硅星人 article on DeepSeek V4: the CSA paragraph (compressor, lightning
 *       indexer, top-k 512/1024, 128-token window, core MQA), the HCA paragraph
 *       (m'=128, no indexer / top-k), the partial-RoPE / mixed-precision cache
 *       paragraph, the state-cache / classic-cache paragraph;
 *   QbitAI piece on batch invariance: bit-identical per-token results however
 *       a token is batched; no split-KV.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless marked [host].
 *   - Every call validates its scalar arguments on the host, enqueues its
 *     kernels on `stream` and returns; nothing is synchronised.  On any status
 *     other than CSA_OK nothing was enqueued, except CSA_ERR_HIP, which reports
 *     a failed launch.  csa_last_error() returns a thread-local message.
 *   - The caller owns every buffer, scratch memory included (topk_select's
 *     workspace, sized by csa_topk_workspace_bytes).  The library allocates
 *     no device memory, keeps no pointer after returning and never writes
 *     `const` inputs.  Calls on different streams touching disjoint outputs
 *     and disjoint workspaces may run concurrently.
 *   - Row formats (csa_fmt), for a row of D values:
 *       CSA_F32    4*D bytes, float32
 *       CSA_BF16   2*D bytes, bfloat16
 *       CSA_FP8    D bytes, OCP FP8 E4M3 (bias 7, max 448, no inf)
 *       CSA_MXFP4  D/2 bytes of E2M1 codes (element 2i in the low nibble of
 *                  byte i) then D/32 E8M0 scale bytes, one per 32 elements
 *                  (OCP Microscaling v1.0); 68 bytes for D=128
 *       CSA_SPLIT  (D-R) E4M3 bytes for dims [0, D-R) then R bfloat16 for the
 *                  RoPE dims [D-R, D); 576 bytes for D=512, R=64.  This is the
 *                  cache entry: BF16 RoPE dims, FP8 elsewhere.
 *   - Batch invariance: every output element of every call depends only on
 *     the inputs of its own query / entry / row, through a reduction order
 *     fixed by the shapes (H, D, k, n_win, ...) and never by the batch, its
 *     order or the launch variant.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: caller-owned top-k workspace (CSA_ERR_WORKSPACE), topk_select_noalloc.
 * 3: hybrid_attn_prefill_paged, indexer_score_paged_rows,
 *    csa_compress_score_paged, csa_debug_poison_lds, CSA_VARIANT_FULL_DIMS
 *    (additions only).
 * 4: csa_compress_score_topk, csa_compress_score_topk_paged,
 *    csa_score_topk_workspace_bytes, csa_select_and_pad (additions only). */
#define CSA_ABI_VERSION 4

typedef enum csa_status {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* a null pointer, a size out of range, a mismatch */
  CSA_ERR_UNSUPPORTED = 2, /* a valid combination the library has no kernel for */
  CSA_ERR_HIP = 3,         /* the HIP runtime refused a launch */
  CSA_ERR_WORKSPACE = 4    /* a required workspace is missing, too small or misaligned */
} csa_status;

typedef enum csa_fmt {
  CSA_F32 = 0,
  CSA_BF16 = 1,
  CSA_FP8 = 2,
  CSA_MXFP4 = 3,
  CSA_SPLIT = 4
} csa_fmt;

typedef enum csa_variant {
  CSA_VARIANT_AUTO = 0,     /* the fewest workgroups per (query, 16 heads) --
                               1, 2 or 4 -- that still give every CU one (1
                               only with a selected list, or with at least
                               four (query, 16 heads) per CU) */
  CSA_VARIANT_HIGH_OCC = 1, /* two workgroups per (query, 16 heads), 256 output
                               dims each: for a batch that fills the GPU */
  CSA_VARIANT_LOW_OCC = 2,  /* four, 128 output dims each: for a small batch */
  CSA_VARIANT_FULL_DIMS = 3 /* one workgroup per (query, 16 heads), all 512
                               output dims: for a batch with at least one
                               (query, 16 heads) per CU (prefill chunks, wide
                               ragged batches).
                               All variants give the same bits (the fp32 path
                               has one kernel and ignores the variant). */
} csa_variant;

int csa_abi_version(void);
const char* csa_status_string(csa_status s);
const char* csa_last_error(void);
/* Bytes of one row of D values in `fmt` (rope_dim is used by CSA_SPLIT only);
 * 0 if the combination is invalid. */
size_t csa_row_bytes(csa_fmt fmt, int D, int rope_dim);

/*
 * csa_compress -- the token-level compressor and the cache write path.
 *
 * Source: 硅星人 article, CSA paragraph (every 4 tokens' KV fold into one
 * entry) and HCA paragraph (m' = 128); DeepSeek-V4 blog, RMSNorm归一化 (norm
 * on the compressed KV head) and Partial RoPE位置编码 (RoPE on the last dims;
 * BF16 RoPE dims, FP8 other dims); 硅星人 article, state-cache paragraph
 * (tokens that do not yet fill a block stay in the caller's state cache).
 *
 * For every complete block j of m consecutive tokens of a segment:
 *   w_t   = softmax over the block of the gate logits g_t
 *           (gate_cols = 1: one logit per token; gate_cols = D: per channel)
 *   C     = sum_t w_t * x_t
 *   if normalize: C = gamma * C / sqrt(mean(C^2) + eps)   (gamma = norm_w or 1)
 *   if rope_dim:  rotate pairs (D-R+2i, D-R+2i+1) by pos * rope_base^(-2i/R),
 *                 pos = seg_pos0[s] + j*m
 *   store C in out_fmt at row seg_out_row[s] + j  (round to nearest even;
 *   E4M3 saturates at +-448; MXFP4 per the OCP MX v1.0 scale rule).
 * m = 1, normalize = 1, rope on, out_fmt = BF16 writes sliding-window rows.
 * normalize = 0, rope_dim = 0, out_fmt = FP8 / MXFP4 writes indexer keys or
 * indexer queries.
 *
 *   x            [n_tok, D] tokens, x_fmt CSA_F32 or CSA_BF16
 *   gate         [n_tok, gate_cols] float32 gate logits
 *   seg_tok_off  [nseg+1] int64: segment s holds tokens [seg_tok_off[s],
 *                seg_tok_off[s+1]); seg_tok_off[0] = 0, seg_tok_off[nseg] =
 *                n_tok, every segment length a multiple of m (a block that
 *                would straddle a segment boundary is not written)
 *   seg_pos0     [nseg] int64 absolute position of each segment's first token
 *   seg_out_row  [nseg] int64 output row of each segment's first entry
 *   norm_w       [D] float32 or NULL (gamma = 1)
 *   out          rows of csa_row_bytes(out_fmt, D, rope_dim)
 * Errors: INVALID_ARG for null pointers, n_tok % m != 0, m < 1, D < 2,
 * gate_cols not in {1, D}, odd or too large rope_dim, D % 32 for MXFP4,
 * rope_dim == 0 or D - rope_dim < 1 for SPLIT; UNSUPPORTED for D > 4096.
 */
csa_status csa_compress(const void* x, csa_fmt x_fmt, const float* gate, int gate_cols,
                        int64_t n_tok /*[host]*/, int D, int m, int nseg,
                        const int64_t* seg_tok_off, const int64_t* seg_pos0,
                        const int64_t* seg_out_row, int normalize, const float* norm_w,
                        float eps, int rope_dim, float rope_base, void* out, csa_fmt out_fmt,
                        hipStream_t stream);

/*
 * csa_compress_batch -- several csa_compress calls in one launch.
 *
 * Source: the same passages as csa_compress.  A decode step writes, for the
 * same new tokens, the compressed KV entry, the matching indexer key and the
 * sliding-window row; this call writes all of them with one kernel launch.
 *
 * Job i carries exactly the arguments of one csa_compress call and produces
 * the same bytes as that call would (each output entry is computed by one
 * workgroup in the same order).  The jobs run in no particular order, so
 * their output rows must not overlap and no job may read what another
 * writes.  `jobs` is a host array of n_jobs entries, read during the call
 * only.
 *
 * Errors: INVALID_ARG if n_jobs < 0, n_jobs > CSA_COMPRESS_MAX_JOBS or jobs
 * is NULL with n_jobs > 0; otherwise the first failing job's csa_compress
 * error, with its job number in csa_last_error().  Nothing is launched when
 * any job fails its checks.  Jobs with n_tok = 0 are skipped.
 */
#define CSA_COMPRESS_MAX_JOBS 4
typedef struct csa_compress_job {
  const void* x;
  csa_fmt x_fmt;
  const float* gate;
  int gate_cols;
  int64_t n_tok;
  int D;
  int m;
  int nseg;
  const int64_t* seg_tok_off;
  const int64_t* seg_pos0;
  const int64_t* seg_out_row;
  int normalize;
  const float* norm_w;
  float eps;
  int rope_dim;
  float rope_base;
  void* out;
  csa_fmt out_fmt;
} csa_compress_job;

csa_status csa_compress_batch(const csa_compress_job* jobs /*[host]*/, int n_jobs,
                              hipStream_t stream);

/*
 * indexer_score -- lightning-indexer scores.
 *
 * Source: 硅星人 article, CSA paragraph and the indexer detail (multi-head
 * index queries, ReLU, scores against the compressed index keys); DeepSeek-V4
 * blog, FP4精度加速 (the indexer runs at FP4); DeepSeek-V4 blog, index
 * visibility is a rule for the indexer.
 *
 * Query i sits at absolute position q_pos[i] and sees N_i = floor((q_pos[i]+1)/m)
 * keys, rows key_off[i] .. key_off[i] + N_i - 1 of `keys`.  For s < N_i:
 *   scores[i*ld + s] = sum_{h < n_heads} w[i*n_heads + h] * max(0, q_h . k_s)
 * The dot products are exact (products of the stored values, summed in fp32);
 * the head sum runs in a fixed order.  scores[i*ld + s] for s >= N_i are not
 * written.  N_i is clamped to ld on the device.
 *
 *   q_idx   [nq, n_heads] rows of d_idx values in `fmt`
 *   w       [nq, n_heads] float32 head weights
 *   keys    rows of d_idx values in `fmt`
 *   fmt     CSA_F32, CSA_FP8 or CSA_MXFP4 (queries and keys share it)
 *   key_off [nq] int64, q_pos [nq] int64
 *   scores  [nq, ld] float32
 * Supported: F32 any n_heads <= 64, d_idx <= 256; FP8 / MXFP4 with n_heads a
 * multiple of 16 (<= 128) and d_idx == 128.  Else UNSUPPORTED.  FP8 batches
 * of 1024 queries or more (prefill chunks) run a kernel in which eight
 * queries (four at 128 heads) with the same key_off share each load and
 * widening of their keys; a score has the same bits from either kernel.
 * Errors: INVALID_ARG for ld < 1 or ld > 2^24 (16.7M entries, 64M tokens at
 * m = 4), m < 1, nq < 0, null pointers, a format other than the three above.
 */
csa_status indexer_score(const void* q_idx, const float* w, int nq, int n_heads, int d_idx,
                         const void* keys, csa_fmt fmt, const int64_t* key_off,
                         const int64_t* q_pos, int m, float* scores, int64_t ld,
                         hipStream_t stream);

/*
 * csa_compress_score -- a decode step's compress jobs and its indexer scores
 * in one call.
 *
 * Source: the passages of csa_compress and indexer_score.  In a decode step
 * the new tokens' index key must be compressed before the indexer can score
 * it; this call does both (and any other compress job of the step, such as
 * the KV entry and the window row) with one kernel launch, so the step pays
 * for one launch instead of two.
 *
 * Results: exactly those of csa_compress_batch(jobs, n_jobs) followed by
 * indexer_score(q_idx, ..., ld) -- the same bytes in every output row and
 * the same bits in every score -- provided that:
 *   - at most one job writes the indexer keys (the job whose `out` equals
 *     `keys`; none is allowed), and that job has out_fmt == fmt, D == d_idx,
 *     rope_dim == 0 and one segment per query (nseg == nq): segment i holds
 *     query i's new tokens;
 *   - every key row that job writes in segment i is seen by query i alone,
 *     as its last visible row (row key_off[i] + N_i - 1): a decode step with
 *     one query per sequence, where a sequence completes at most one block;
 *   - no other job writes memory that the indexer reads.
 * Inside the launch, the workgroup that compresses a new key row also scores
 * it for its query, with the indexer's own arithmetic; the indexer's
 * workgroups score every other row.  When the precondition does not hold
 * the scores of the rows being written are undefined (no access leaves the
 * buffers named by the arguments).  FP8 keys with nq < 1024 take the single
 * launch; other formats and larger batches run the two launches in order.
 *
 * Arguments: `jobs` / n_jobs as for csa_compress_batch (host array, read
 * during the call only); the rest as for indexer_score.
 * Errors: those of csa_compress_batch and indexer_score (same checks, names
 * of this entry point in csa_last_error()); INVALID_ARG when two jobs write
 * `keys` or the key job breaks the shape rules above.  Nothing is launched
 * when a check fails.  nq = 0 runs the jobs alone (csa_compress_batch, with
 * no rule on the key job).
 */
csa_status csa_compress_score(const csa_compress_job* jobs /*[host]*/, int n_jobs,
                              const void* q_idx, const float* w, int nq, int n_heads, int d_idx,
                              const void* keys, csa_fmt fmt, const int64_t* key_off,
                              const int64_t* q_pos, int m, float* scores, int64_t ld,
                              hipStream_t stream);

/*
 * csa_compress_score_paged -- csa_compress_score over a paged key cache.
 *
 * Source: the passages of csa_compress_score; 硅星人 article, classic-cache
 * paragraph (keys in fixed blocks of a shared pool, reached through a block
 * table).
 *
 * The indexer side reads keys as indexer_score_paged_rows does (query i
 * through table row q_block_row[i], or row i).  The key job writes the key
 * pool: it is the job whose `out` equals key_pool, and its segment i writes
 * pool rows seg_out_row[i] + j as csa_compress does, so a segment's new rows
 * must lie in one block of the pool (a decode step writes one row per
 * query).  Results: those of csa_compress_batch followed by
 * indexer_score_paged_rows, when every key row written in segment i is the
 * pool row of query i's last visible row (the physical row that query i's
 * table maps logical row N_i - 1 to).
 *
 * Arguments: the jobs as for csa_compress_score; the rest as for
 * indexer_score_paged_rows.
 * Errors: those of csa_compress_score (with key_pool in place of keys) and of
 * indexer_score_paged_rows.
 */
csa_status csa_compress_score_paged(const csa_compress_job* jobs /*[host]*/, int n_jobs, const void* q_idx,
                                    const float* w, int nq, int n_heads, int d_idx, const void* key_pool,
                                    csa_fmt fmt, int64_t pool_rows, const int32_t* block_table,
                                    int64_t table_rows, int64_t blocks_per_seq, int block_rows,
                                    const int32_t* q_block_row, const int64_t* q_pos, int m, float* scores,
                                    int64_t ld, hipStream_t stream);

/*
 * csa_compress_score_topk -- a decode step's compress jobs, indexer scores
 * and top-k selection in one call (one kernel launch).
 *
 * Source: the passages of csa_compress_score and topk_select; 硅星人 article,
 * CSA paragraph (the lightning indexer scores every compressed entry and the
 * top-k selector keeps the k best-scored ones for the attention).
 *
 * Results: exactly those of csa_compress_score(jobs, ..., scores, ld)
 * followed by topk_select(scores, ld, nq, n_valid, k, idx, NULL, ...) with
 * n_valid[i] = N_i = min(floor((q_pos[i] + 1) / m), ld): the same bytes in
 * every compressed row, the same bits in every score (scores are still
 * written) and the same index sets in idx [nq, k] int32 (ascending, -1
 * padded; ties to the lower index), under csa_compress_score's precondition.
 * The workgroups that score a query also count its scores into 4096 integer
 * bins of the scores' order key (order-free atomics), and the last of them
 * to finish selects the query's top-k from the scores just written, so the
 * step needs no separate top-k launch.
 *
 * Supported: fmt == CSA_FP8 with nq < 1024 (the streaming indexer); other
 * formats and larger batches are UNSUPPORTED (use csa_compress_score, or
 * indexer_score, then topk_select).
 * Workspace: caller-owned device memory of at least
 * csa_score_topk_workspace_bytes(nq) bytes (nq * 16,640: per query 4096 bin
 * counts and an arrival counter), 256-byte aligned, holding zeros before the
 * first call.  Every call leaves the part it used at zero again, so the same
 * workspace serves later calls without clearing; calls that may run at the
 * same time need separate workspaces.  When the precondition of
 * csa_compress_score does not hold, idx is undefined and the workspace must
 * be zeroed again.
 * Errors: those of csa_compress_score; INVALID_ARG for k < 1 or k > 4096 or
 * a null idx; UNSUPPORTED as above; WORKSPACE when the workspace is NULL,
 * shorter than required or misaligned.  nq = 0 runs the jobs alone.
 */
csa_status csa_compress_score_topk(const csa_compress_job* jobs /*[host]*/, int n_jobs, const void* q_idx,
                                   const float* w, int nq, int n_heads, int d_idx, const void* keys,
                                   csa_fmt fmt, const int64_t* key_off, const int64_t* q_pos, int m,
                                   float* scores, int64_t ld, int k, int32_t* idx, void* workspace,
                                   size_t ws_bytes, hipStream_t stream);

/*
 * csa_compress_score_topk_paged -- csa_compress_score_topk over a paged key
 * cache: the indexer side and the key job as in csa_compress_score_paged,
 * the selection as in csa_compress_score_topk (same workspace rules).
 *
 * Source: the passages of csa_compress_score_paged and
 * csa_compress_score_topk.
 * Errors: those of csa_compress_score_paged and csa_compress_score_topk.
 */
csa_status csa_compress_score_topk_paged(const csa_compress_job* jobs /*[host]*/, int n_jobs, const void* q_idx,
                                         const float* w, int nq, int n_heads, int d_idx, const void* key_pool,
                                         csa_fmt fmt, int64_t pool_rows, const int32_t* block_table,
                                         int64_t table_rows, int64_t blocks_per_seq, int block_rows,
                                         const int32_t* q_block_row, const int64_t* q_pos, int m, float* scores,
                                         int64_t ld, int k, int32_t* idx, void* workspace, size_t ws_bytes,
                                         hipStream_t stream);

/*
 * csa_select_and_pad -- join the compressed runs of the shards of one
 * sequence into one contiguous run, the padding moved to its end.
 *
 * Source: DeepSeek-V4 blog, 百万 token 怎么切分到多张卡 (context parallelism:
 * each rank receives the last m uncompressed tokens of the rank before it,
 * compresses them with its own tokens into a fixed-length run of compressed
 * blocks with a little padding, the runs are all-gathered, and a fused
 * select-and-pad step reassembles them into one global compressed sequence
 * with every padding row at its end).  On one GPU the shards' runs are
 * regions of one buffer; the compression itself is csa_compress (segment i
 * of a shard starts at the first token of a block, with the carried tokens).
 *
 *   in      [n_shards, cap] rows of row_bytes bytes (device); shard s's run
 *           is valid in its first n_valid[s] rows (n_valid: device int64
 *           [n_shards], clamped to [0, cap] on the device)
 *   out     [n_shards * cap] rows (device): shard 0's valid rows, then shard
 *           1's, ..., then zero rows; must not overlap `in`
 * Pure data movement; the result does not depend on the launch.
 * Errors: INVALID_ARG for n_shards outside [1, 256], cap outside [0, 2^31],
 * row_bytes not a multiple of 4 in [4, 2^20], null pointers, unaligned or
 * overlapping buffers.  cap = 0 does nothing.
 */
csa_status csa_select_and_pad(const void* in, int n_shards, int64_t cap, int64_t row_bytes,
                              const int64_t* n_valid, void* out, hipStream_t stream);

/* Bytes of zeroed workspace csa_compress_score_topk needs for nq queries
 * (nq * 16,640); 0 for nq <= 0 or nq >= 1024. */
size_t csa_score_topk_workspace_bytes(int nq);

/*
 * indexer_score_paged -- indexer_score over a paged key cache.
 *
 * Source: the passages of indexer_score; 硅星人 article, classic-cache
 * paragraph (the compressed caches are kept in fixed blocks of 128 raw tokens,
 * which hold 32 CSA entries and one HCA entry, so that nothing fragments).
 *
 * The keys of query i are not a contiguous run of rows: logical row s (s <
 * N_i, N_i as for indexer_score) is row
 *   block_table[i * blocks_per_seq + (s / block_rows)] * block_rows + s % block_rows
 * of key_pool (pool_rows rows of d_idx values in `fmt`).  block_rows = 32 is
 * one 128-token block of CSA keys.  The scores are those indexer_score gives
 * for the same keys laid out contiguously (the same bits).
 *
 *   block_table  [nq, blocks_per_seq] int32 physical block numbers
 * Preconditions: blocks_per_seq * block_rows >= N_i for every query, and
 * every block a query uses lies inside the pool (otherwise a table entry
 * past the row reads as block 0 and a row past the pool as zeros: wrong
 * scores, no fault).
 * Supported: FP8 / MXFP4 keys with indexer_score's head and dim rules,
 * block_rows a power of two in [16, 2^20], a pool smaller than 4 GiB
 * (UNSUPPORTED otherwise).  Batches take the kernels of indexer_score (the
 * shared-key kernel for FP8 batches of 1024 queries or more).
 * Errors: those of indexer_score (block_table takes key_off's place in the
 * null-pointer check); INVALID_ARG for bad block_rows / blocks_per_seq /
 * pool_rows.
 */
csa_status indexer_score_paged(const void* q_idx, const float* w, int nq, int n_heads, int d_idx,
                               const void* key_pool, csa_fmt fmt, int64_t pool_rows,
                               const int32_t* block_table, int64_t blocks_per_seq, int block_rows,
                               const int64_t* q_pos, int m, float* scores, int64_t ld,
                               hipStream_t stream);

/*
 * indexer_score_paged_rows -- indexer_score_paged with a table row per query.
 *
 * Source: as indexer_score_paged (硅星人 article, classic-cache paragraph).
 *
 * Query i reads block-table row r = q_block_row[i] (q_block_row NULL: r = i)
 * of a table of table_rows rows: its logical row s is row
 *   block_table[r * blocks_per_seq + (s / block_rows)] * block_rows + s % block_rows
 * of key_pool.  The queries of one sequence in a prefill chunk share one
 * table row.  In the shared-key kernel (FP8, 1024 queries or more), queries
 * of one workgroup that name the same row read each key once for all of
 * them.  A q_block_row entry outside [0, table_rows) is clamped into it
 * (memory safety only: the result is then that row's).  The scores are the
 * bits indexer_score gives for the same keys laid out contiguously.
 *
 *   block_table  [table_rows, blocks_per_seq] int32;  q_block_row  [nq] int32 or NULL
 * Preconditions, support and errors: those of indexer_score_paged; also
 * INVALID_ARG for table_rows outside [1, 2^31], or q_block_row NULL with
 * table_rows < nq.
 */
csa_status indexer_score_paged_rows(const void* q_idx, const float* w, int nq, int n_heads, int d_idx,
                                    const void* key_pool, csa_fmt fmt, int64_t pool_rows,
                                    const int32_t* block_table, int64_t table_rows, int64_t blocks_per_seq,
                                    int block_rows, const int32_t* q_block_row, const int64_t* q_pos, int m,
                                    float* scores, int64_t ld, hipStream_t stream);

/*
 * topk_select -- the top-k selector.
 *
 * Source: 硅星人 article, CSA paragraph (keep the 512 most relevant compressed
 * blocks, 1024 for Pro); DeepSeek-V4 blog, index visibility (for CSA the top-k
 * selector names the visible entries).
 *
 * Row i holds n_i = n_valid[i] (or ld when n_valid is NULL) scores.  The
 * selected set is the min(k, n_i) best entries ordered by score descending
 * then index ascending (ties go to the lower index).  idx[i*k ...] receives
 * the selected indices in ascending index order followed by -1 padding;
 * top_scores (optional) the matching scores, padding -inf.  Integer work:
 * the set is exact and does not depend on how rows are batched.  Scores must
 * not be NaN.  n_valid is clamped to [0, ld] on the device.
 *
 *   scores  [nq, ld] float32;  idx [nq, k] int32;  top_scores [nq, k] or NULL
 * Rows longer than 33792 scores (ld > 33792) are selected in two passes: P
 * slices of about 16K scores each give their own exact top-k (P = min(
 * ceil(ld / 16384), max(2, 16384 / k))), written into a candidate row, and
 * the row's top-k is selected from the candidates.  The candidates live in
 * `workspace`, caller-owned device memory of at least
 * csa_topk_workspace_bytes(nq, ld, k) bytes (nq * P * k * 8), 16-byte
 * aligned; its contents on entry do not matter and are left undefined.
 * When that size is 0 (ld <= 33792) workspace may be NULL.  Two calls that
 * may run at the same time need two workspaces.  nq * P must not exceed
 * 2^22 (one 1024-thread workgroup per row or slice).
 * Errors: INVALID_ARG for k < 1, k > 4096, ld < 1, ld > 2^28, nq < 0,
 * nq * P > 2^22, null pointers; WORKSPACE when a workspace is needed and is
 * NULL, smaller than required or misaligned.
 */
csa_status topk_select(const float* scores, int64_t ld, int nq, const int64_t* n_valid, int k,
                       int32_t* idx, float* top_scores, void* workspace, size_t ws_bytes,
                       hipStream_t stream);

/* Bytes of workspace topk_select needs for nq rows of ld scores and this k
 * (0: none); 0 as well for arguments topk_select rejects. */
size_t csa_topk_workspace_bytes(int nq, int64_t ld, int k);

/*
 * topk_select_noalloc -- topk_select for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same selection, same arguments minus the workspace,
 * same results bit for bit.
 *
 * The candidate rows of the two-pass path live in a static device array of
 * the library, csa_topk_noalloc_max_bytes() bytes (16 MiB) per GPU, held from
 * the first call on that GPU until the process ends.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).  Its contents on
 * entry do not matter and nothing needs clearing.  Every call on one GPU
 * shares the array: two calls that may overlap on one GPU (other streams,
 * other threads) race and give undefined results; serialise them or use
 * topk_select with disjoint workspaces.
 * Errors: those of topk_select, and WORKSPACE when
 * csa_topk_workspace_bytes(nq, ld, k) exceeds csa_topk_noalloc_max_bytes()
 * (nothing is enqueued); HIP when the array's address cannot be obtained.
 */
csa_status topk_select_noalloc(const float* scores, int64_t ld, int nq, const int64_t* n_valid, int k,
                               int32_t* idx, float* top_scores, hipStream_t stream);

/* Size of topk_select_noalloc's static candidate array in bytes. */
size_t csa_topk_noalloc_max_bytes(void);

/*
 * hybrid_attn_decode -- sink multi-query attention of one decode token per
 * sequence over its compressed entries (top-k selected for CSA, all for HCA)
 * followed by its sliding window.
 *
 * Source: 硅星人 article, CSA paragraph (selected entries plus the 128 window
 * tokens go to core multi-query attention) and HCA paragraph (all entries
 * plus the window); DeepSeek-V4 blog, Partial RoPE (window of n_win raw
 * entries used with the compressed ones), RMSNorm on the query heads, and
 * 让注意力学会"忽略" (sink logit in the denominator); ai-engineering summary
 * (head dim 512).
 *
 * Query b at absolute position p = q_pos[b] has N_b = floor((p+1)/m) visible
 * entries, rows kv_off[b] .. kv_off[b] + N_b - 1 of `kv`.  The attended list
 * is E = (idx[b*k .. b*k+k) with -1 and out-of-range values dropped, in the
 * given order, which must be ascending) or (0..N_b-1 when idx is NULL),
 * followed by window rows 0 .. win_len[b]-1 of win[b] (oldest first, the last
 * one at position p).  For every head h:
 *   qhat = RoPE_p(RMSNorm(q[b,h]))           (gamma = q_norm_w or 1, eps)
 *   l_j  = scale * qhat . e_j                (the stored entry is key and value)
 *   out[b,h] = sum_j e^{l_j} e_j / (sum_j e^{l_j} + e^{sinks[h]})
 * The reduction order over E is fixed per token, the same in every variant
 * and batch.  F32 path: E in list order.  MFMA path: four interleaved
 * slices -- slice w takes list positions [64 s + 16 w, +16) of the
 * compressed part and window rows [64 t + 16 w, +16) -- each reduced in
 * order, then merged in slice order.  In both the sink joins the denominator after
 * the entries (so sinks[h] = -inf is standard softmax and a large sinks[h]
 * scales the output down without underflowing the weights); a query with
 * nothing to attend gets a zero output.
 *
 *   q, out   [B, H] rows of D values (q_fmt / out_fmt: F32 or BF16)
 *   kv       rows of D values in kv_fmt (SPLIT, or F32 on the fp32 path)
 *   win      [B, n_win] rows in win_fmt (BF16, or F32 on the fp32 path)
 *   win_len  [B] int32 (clamped to [0, n_win] on the device)
 *   sinks    [H] float32
 * Paths: all-F32 (q, kv, win, out F32; any D <= 512, H <= 1024); MFMA path
 * (q BF16, kv SPLIT with D = 512, rope_dim = 64, win BF16, out BF16, H a
 * multiple of 16).  Other combinations: UNSUPPORTED.
 */
csa_status hybrid_attn_decode(const void* q, csa_fmt q_fmt, int B, int H, int D,
                              const int64_t* q_pos, const float* q_norm_w, float eps,
                              int rope_dim, float rope_base, const void* kv, csa_fmt kv_fmt,
                              const int64_t* kv_off, int m, const int32_t* idx, int k,
                              const void* win, csa_fmt win_fmt, int n_win,
                              const int32_t* win_len, const float* sinks, float scale,
                              void* out, csa_fmt out_fmt, csa_variant variant,
                              hipStream_t stream);

/*
 * hybrid_attn_decode_paged -- hybrid_attn_decode over a paged entry cache.
 *
 * Source: the passages of hybrid_attn_decode; 硅星人 article, classic-cache
 * paragraph (fixed 128-token blocks: 32 CSA entries or one HCA entry each).
 *
 * Entry e of query b (e < N_b) is row
 *   block_table[b * blocks_per_seq + (e / block_rows)] * block_rows + e % block_rows
 * of kv_pool (pool_rows SPLIT rows).  The window is the request's state
 * cache, kept as a ring of n_win rows per query (硅星人 article,
 * state-cache paragraph: the 128-token window KV is part of each request's
 * state): window row t (t < win_len[b], oldest first) is row
 *   b * n_win + (win_start[b] + t) mod n_win
 * of win, so the newest token overwrites the oldest slot in place; win_start
 * NULL means 0 (rows in order), and a win_start[b] outside [0, n_win) is
 * taken as 0.  Everything else -- the selected list idx (logical entry
 * numbers, ascending), the sinks, the reduction order -- is that of
 * hybrid_attn_decode, and so are the output bits: a query gives the same
 * bits whether its entries are paged or contiguous and its window a ring or
 * in order.
 *
 *   win_start  [B] int32 or NULL
 *
 * idx NULL attends every visible entry (HCA; block_rows = 1 is one HCA entry
 * per 128-token block).  Lists longer than 1024 positions (k > 1024, or HCA
 * with N_b > 1024) map the positions past the first 1024 one step at a time
 * inside the loop, which costs a dependent load per step.
 * Supported: the MFMA path (BF16 q / window / out, SPLIT cache, D = 512,
 * rope_dim = 64, H a multiple of 16); block_rows a power of two in [1, 2^20];
 * a pool smaller than 4 GiB.  The F32 path: UNSUPPORTED.
 * Preconditions as for indexer_score_paged (blocks_per_seq * block_rows >=
 * N_b; used blocks inside the pool).
 * Errors: those of hybrid_attn_decode; INVALID_ARG for bad block_rows /
 * blocks_per_seq / pool_rows or a NULL block_table.
 */
csa_status hybrid_attn_decode_paged(const void* q, csa_fmt q_fmt, int B, int H, int D,
                                    const int64_t* q_pos, const float* q_norm_w, float eps,
                                    int rope_dim, float rope_base, const void* kv_pool, csa_fmt kv_fmt,
                                    int64_t pool_rows, const int32_t* block_table, int64_t blocks_per_seq,
                                    int block_rows, int m, const int32_t* idx, int k,
                                    const void* win, csa_fmt win_fmt, int n_win,
                                    const int32_t* win_start, const int32_t* win_len, const float* sinks,
                                    float scale, void* out, csa_fmt out_fmt, csa_variant variant,
                                    hipStream_t stream);

/*
 * hybrid_attn_prefill -- the same attention for a chunk of causal queries.
 *
 * Source: as hybrid_attn_decode; causal visibility by rule (DeepSeek-V4 blog,
 * index visibility).
 *
 * Query i at absolute position p = q_pos[i] sees entries
 * kv_off[i] .. kv_off[i] + floor((p+1)/m) - 1 (filtered by its own top-k row
 * idx[i*k ..] for CSA) and the window positions max(0, p-n_win+1) .. p, read
 * from a run of per-token rows: the row of position t is
 * tok_off[i] + (t - tok_pos0[i]) of `tok` (already normalised and rotated,
 * as written by csa_compress with m = 1).  Window positions below tok_pos0[i]
 * are skipped.  A token gets the same bits here as from hybrid_attn_decode
 * given the same entries and window rows.
 *
 *   q, out  [nq, H] rows;  kv_off, tok_off, tok_pos0, q_pos  [nq] int64
 * Formats and paths as hybrid_attn_decode, with tok_fmt in place of win_fmt.
 */
csa_status hybrid_attn_prefill(const void* q, csa_fmt q_fmt, int nq, int H, int D,
                               const int64_t* q_pos, const float* q_norm_w, float eps,
                               int rope_dim, float rope_base, const void* kv, csa_fmt kv_fmt,
                               const int64_t* kv_off, int m, const int32_t* idx, int k,
                               const void* tok, csa_fmt tok_fmt, const int64_t* tok_off,
                               const int64_t* tok_pos0, int n_win, const float* sinks,
                               float scale, void* out, csa_fmt out_fmt, csa_variant variant,
                               hipStream_t stream);

/*
 * hybrid_attn_prefill_paged -- hybrid_attn_prefill over a paged entry cache.
 *
 * Source: the passages of hybrid_attn_prefill; 硅星人 article, classic-cache
 * paragraph (the compressed entries of a request live in fixed blocks of the
 * shared pool, reached through the request's block table).
 *
 * Query i reads block-table row r = q_block_row[i] (q_block_row NULL: r = i);
 * its entry e (e < floor((q_pos[i]+1)/m)) is row
 *   block_table[r * blocks_per_seq + (e / block_rows)] * block_rows + e % block_rows
 * of kv_pool (pool_rows SPLIT rows).  The queries of one sequence in a chunk
 * share one table row, so a chunk needs one row per sequence, not per query.
 * The window is read from per-token rows exactly as in hybrid_attn_prefill
 * (tok, tok_off, tok_pos0).  Everything else -- the top-k rows idx (logical
 * entry numbers), the sinks, the reduction order -- is that of
 * hybrid_attn_prefill, and so are the output bits: a query gives the same
 * bits whether its entries are paged or contiguous.
 *
 *   block_table  [table_rows, blocks_per_seq] int32
 *   q_block_row  [nq] int32 or NULL; a row outside [0, table_rows) is clamped
 *                into it (memory safety only: the result is then that row's)
 *
 * Supported: the MFMA path only (BF16 q / tok / out, SPLIT cache, D = 512,
 * rope_dim = 64, H a multiple of 16); block_rows a power of two in [1, 2^20];
 * blocks_per_seq in [1, 2^26]; table_rows in [1, 2^31]; a pool smaller than
 * 4 GiB.  Preconditions as for hybrid_attn_decode_paged (the table row covers
 * every visible entry; used blocks inside the pool).
 * Errors: those of hybrid_attn_prefill; UNSUPPORTED for other formats;
 * INVALID_ARG for bad block_rows / blocks_per_seq / table_rows / pool_rows, a
 * NULL block_table, or q_block_row NULL with table_rows < nq.
 */
csa_status hybrid_attn_prefill_paged(const void* q, csa_fmt q_fmt, int nq, int H, int D,
                                     const int64_t* q_pos, const float* q_norm_w, float eps,
                                     int rope_dim, float rope_base, const void* kv_pool, csa_fmt kv_fmt,
                                     int64_t pool_rows, const int32_t* block_table, int64_t table_rows,
                                     int64_t blocks_per_seq, int block_rows, const int32_t* q_block_row,
                                     int m, const int32_t* idx, int k, const void* tok, csa_fmt tok_fmt,
                                     const int64_t* tok_off, const int64_t* tok_pos0, int n_win,
                                     const float* sinks, float scale, void* out, csa_fmt out_fmt,
                                     csa_variant variant, hipStream_t stream);

/*
 * csa_debug_poison_lds -- fill the LDS of every compute unit with a pattern.
 *
 * A diagnostic for tests of the kernels' LDS hygiene, not a step of the
 * path: launched on `stream` before a kernel, it leaves every CU's 160 KB of
 * LDS holding the 32-bit `pattern`, so a kernel that read LDS it had not
 * written first would give results that depend on the pattern.  The
 * hardware does not promise that a later kernel finds these bytes; equal
 * results under several patterns are evidence, not proof.
 * Errors: HIP for a failed launch.
 */
csa_status csa_debug_poison_lds(uint32_t pattern, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
