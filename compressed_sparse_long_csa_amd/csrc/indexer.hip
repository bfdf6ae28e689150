// Lightning-indexer scores (indexer_score).
//
// Source: 硅星人 article on DeepSeek V4, CSA paragraph and the indexer detail
// (multi-head index queries with ReLU, scored against compressed index keys
// shared by the heads); DeepSeek-V4 blog, FP4精度加速 (the indexer's products
// run at FP4) and the index-visibility rule (query at p sees floor((p+1)/m)
// entries).
//
//   I[i, s] = sum_h w[i, h] * max(0, q[i, h] . k[s])
//
// Decode streams every visible key once, so the kernels are HBM-bound: each
// wave owns 128 keys, issues the loads of its query and then of all its keys
// (straight from global memory into the MFMA operand registers), and works
// on each 16-key block as soon as that block has arrived, so the arithmetic
// runs under the transfer; two waves per SIMD.
//  * FP8 keys: the products must be exact for the top-k to be reproducible,
//    and FP8 MFMA accumulation is not, so FP8 values are widened to BF16
//    (exact) and multiplied on BF16 MFMA with fp32 accumulation.
//  * MXFP4 keys: scaled FP4 MFMA (E2M1 x E2M1 with per-32 E8M0 scales), whose
//    result is exact for these operands.
//  * F32: plain fp32 FMAs in dim order.
// Prefill batches (1024 queries or more, FP8) run a shared-key kernel: four
// queries of one sequence per workgroup, each key group loaded and widened
// once into LDS and multiplied by every wave against its own query, with the
// streaming kernel's operands, tiles and head sum (the same bits).
// The dims of one 128-dim vector are assigned to k-steps so that each lane
// reads 32 contiguous bytes; the same permutation is applied to queries and
// keys, so each dot product is the same sum.  The MFMA output is heads x
// keys, so the head sum runs inside a lane (a fixed tree over the lane's 16
// heads) and then over the four row groups in a fixed order.
#include "compress_dev.hpp"

namespace csa {

namespace {

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x8 r;
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Sum of a lane value over the four 16-lane rows of the wave, in one fixed
// order ((row0 + row1) + (row2 + row3)); every lane receives the total.
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The MFMA output is heads x keys: lane (key j16, heads 4g .. 4g+3 of each
// 16-head block), so a lane sums its 16 heads and the four row groups are
// added once.  Key rows are read through a buffer descriptor over the
// query's N visible rows: rows past N read as zero, and a row address is a
// 32-bit offset with the block step in the scalar offset.
__device__ __forceinline__ uint4 buf_load_x4(buf_rsrc r, uint32_t voff, uint32_t soff) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0);
  return make_uint4(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
                    static_cast<uint32_t>(v[3]));
}

// max(x, 0) on the bit pattern: a negative float is a negative integer (-0 -> +0)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Score of the 16 keys of one block from its heads x keys MFMA tiles: lane
// sums its 16 heads in a fixed tree (pairs of rows within a head block, then
// head blocks pairwise), then the row groups.  The tree keeps the dependent
// chain short; the order never changes, so the bits do not either.
template <int NHB>
__device__ __forceinline__ float head_sum(const f32x4 (&c)[NHB], const float (&wr)[NHB][4]) {
  float s[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
    s[hb] = fmaf(wr[hb][1], relu(c[hb][1]), wr[hb][0] * relu(c[hb][0])) +
            fmaf(wr[hb][3], relu(c[hb][3]), wr[hb][2] * relu(c[hb][2]));
#pragma unroll
  for (int w = 1; w < NHB; w *= 2)
#pragma unroll
    for (int hb = 0; hb + w < NHB; hb += 2 * w) s[hb] += s[hb + w];
  return rows_sum(s[0]);
}

// --------------------------------------------------------------- FP8, d = 128
// Each wave streams up to R groups of 64 keys (4 blocks of 16) of one query:
// the loads of group t+2 go out as soon as group t has been multiplied, so
// two groups are in flight while one computes, and the query stays in
// registers throughout.  With long shares (R > 2) the W waves of a query
// take its groups in turn (wave w: groups w, w+W, w+2W, ...), so the groups
// being read at any moment lie next to each other in memory; with R <= 2
// every load is issued at once anyway, and wave w takes groups [wR, wR+R).
constexpr int kGroupKeys = 64;

// lane (key j16 of block kb, dims [32g, 32g+32)) = 32 contiguous bytes; a
// group past the run aims past the end of the buffer (zeros, no traffic)
__device__ __forceinline__ void load_group_fp8(buf_rsrc rs, uint32_t voff0, uint32_t stride, int t, int ng,
                                               uint4 (&kr)[4][2]) {
  const uint32_t base = t < ng ? voff0 + static_cast<uint32_t>(t) * stride : 0x80000000u;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    kr[kb][0] = buf_load_x4(rs, base, kb * 2048u);
    kr[kb][1] = buf_load_x4(rs, base + 16u, kb * 2048u);
  }
}

// ---------------------------------------------------------------- paged keys
// A paged key cache: query i's rows come in blocks of BR = 2^sh rows (BR >=
// 16, so that a 16-key MFMA block lies in one block); its logical block j is
// physical block blk_table[i * blk_stride + j] of the pool.  A wave reads the
// table entries of its share once, in the round trip of the query's position
// (two per lane: at most 32 groups of 64 keys, at most four blocks each), and
// takes them with readlane.  Keys are addressed through one descriptor over
// the pool, all of the offset in the per-lane part, so the range check sees
// the whole offset; table entries past the row read as 0 and rows past N are
// multiplied but never stored.
struct PagedTab {
  int32_t e[2];
  int bpg_shift;                                         // log2(blocks per 64-key group)
};

// Block-table row of query i: i, or blk_row[i] clamped into the table (an
// out-of-range row reads row 0 or the last one; the caller checks rows).
__device__ __forceinline__ int64_t table_row(const IndexerArgs& a, int i) {
  if (a.blk_row == nullptr) return i;
  const int64_t r = __builtin_amdgcn_readfirstlane(a.blk_row[i]);
  return r < 0 ? 0 : (r >= a.blk_rows ? a.blk_rows - 1 : r);
}

__device__ __forceinline__ buf_rsrc table_rsrc(const IndexerArgs& a, int64_t row) {
  return make_rsrc(a.blk_table + row * a.blk_stride, static_cast<uint32_t>(a.blk_stride * 4));
}

// Pool row of query i's logical row r (a table entry past the row reads as
// block 0).  Wave-uniform.
__device__ __forceinline__ int64_t pool_row(const IndexerArgs& a, int i, int64_t r) {
  const int64_t lb = r >> a.blk_shift;
  const int32_t blk = lb < a.blk_stride
                          ? __builtin_amdgcn_readfirstlane(a.blk_table[table_row(a, i) * a.blk_stride + lb]) : 0;
  return (static_cast<int64_t>(blk) << a.blk_shift) | (r & ((int64_t{1} << a.blk_shift) - 1));
}

__device__ __forceinline__ void paged_tab_load(const IndexerArgs& a, int i, uint32_t first, uint32_t step,
                                               int R, int lane, PagedTab& pt) {
  const int sh = a.blk_shift;
  pt.bpg_shift = sh >= 6 ? 0 : 6 - sh;
  const buf_rsrc trs = table_rsrc(a, table_row(a, i));
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint32_t e = static_cast<uint32_t>(s * 64 + lane);
    const uint32_t u = e >> pt.bpg_shift, q = e & ((1u << pt.bpg_shift) - 1u);
    const uint32_t lb = (((first + u * step) * static_cast<uint32_t>(kGroupKeys)) >> sh) + q;
    const uint32_t off = u < static_cast<uint32_t>(R) && lb < static_cast<uint32_t>(a.blk_stride) ? lb * 4u
                                                                                                   : 0x80000000u;
    pt.e[s] = __builtin_amdgcn_raw_buffer_load_b32(trs, static_cast<int>(off), 0, 0);
  }
}

// Pool row of the first key of 16-key block kb of the wave's group u (uniform).
__device__ __forceinline__ uint32_t paged_row(const PagedTab& pt, int sh, uint32_t first, uint32_t step, int u,
                                              int kb) {
  const uint32_t key = (first + static_cast<uint32_t>(u) * step) * static_cast<uint32_t>(kGroupKeys) +
                       static_cast<uint32_t>(kb) * 16u;
  const int e = (u << pt.bpg_shift) + ((kb * 16) >> sh);
  const int32_t blk = e < 64 ? __builtin_amdgcn_readlane(pt.e[0], e) : __builtin_amdgcn_readlane(pt.e[1], e - 64);
  return (static_cast<uint32_t>(blk) << sh) | (key & ((1u << sh) - 1u));
}

__device__ __forceinline__ void load_group_fp8_paged(buf_rsrc rs, const PagedTab& pt, int sh, uint32_t first,
                                                     uint32_t step, int t, int ng, int j16, int g,
                                                     uint4 (&kr)[4][2]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint32_t voff = t < ng ? (paged_row(pt, sh, first, step, t, kb) + static_cast<uint32_t>(j16)) * 128u +
                                       static_cast<uint32_t>(g) * 32u
                                 : 0x80000000u;
    kr[kb][0] = buf_load_x4(rs, voff, 0);
    kr[kb][1] = buf_load_x4(rs, voff + 16u, 0);
  }
}

// MFMAs of one group's blocks; the head sum of the block before (held in
// cp) is computed and stored while a block multiplies.  `pend` is the score
// offset (bytes, relative to the lane's first score) of the block in cp, or
// -1 when there is none to keep; `grp` that of this group, or -1 for a group
// past the wave's share.  Every block issues exactly one store (one with
// nothing to keep aims past the buffer), so each pass of the group loop
// issues the same memory operations and the compiler's wait counts stay exact.
template <int NHB>
__device__ __forceinline__ void group_fp8(const uint4 (&kr)[4][2], const bf16x8 (&qb)[NHB][4],
                                          const float (&wr)[NHB][4], f32x4 (&cp)[NHB], int& pend, int grp,
                                          buf_rsrc out_rs, uint32_t out_off) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const bf16x8 kk[4] = {fp8x8_to_bf16(kr[kb][0].x, kr[kb][0].y), fp8x8_to_bf16(kr[kb][0].z, kr[kb][0].w),
                          fp8x8_to_bf16(kr[kb][1].x, kr[kb][1].y), fp8x8_to_bf16(kr[kb][1].z, kr[kb][1].w)};
    f32x4 cc[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) cc[hb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // rows = heads (A), cols = keys (B); the NHB chains interleave
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        cc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[hb][ks], kk[ks], cc[hb], 0, 0, 0);
    const float tot = head_sum<NHB>(cp, wr);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rs,
                                          static_cast<int>(pend >= 0 ? out_off : 0x80000000u),
                                          pend >= 0 ? pend : 0, 0);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) cp[hb] = cc[hb];
    pend = grp >= 0 ? grp + kb * 64 : -1;
  }
}

// Key rows that the same launch writes (compress_score_kernel): segment i
// of the key job holds query i's new tokens, and a row that job writes is,
// for query i, its last visible row.  Its score is computed by the workgroup
// that compresses it; the streaming waves store every other score.  nseg = 0
// when the launch writes no key.
struct NewKeys {
  const int64_t* seg_tok_off;
  const int64_t* seg_out_row;
  int64_t n_tok;
  int nseg;
  int m;
};

// NB: groups in flight per wave (2; 3 where shares of three groups are common)
template <int NHB, bool IL, bool kNew, int NB = 2, bool kPaged = false>   // head blocks of 16; interleaved shares; keys written alongside; paged keys
__device__ __forceinline__ void fp8_items(const IndexerArgs& a, int64_t n_items, int64_t n_chunk, int R,
                                          int64_t item0, int64_t item_step, const NewKeys& nk) {
  constexpr int H = NHB * 16;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 4, j16 = lane & 15;
  const uint8_t* qall = static_cast<const uint8_t*>(a.q);
  for (int64_t item = item0; item < n_items; item += item_step) {
    // query i; item `chunk` holds four of the query's waves
    const int i = static_cast<int>(item / n_chunk);
    const int64_t chunk = item % n_chunk;
    // query operand rows (head hb*16 + j16, dims [32g, 32g+32)) and the
    // weights of the heads this lane sums (hb*16 + 4g + r): their addresses
    // depend on i only, so they go out first, in the same round trip as the
    // query's position and key offset (and before the keys, so that waiting
    // for them never waits for a key group)
    uint4 qraw[NHB][2];
    float4 wraw[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const uint4* qp = reinterpret_cast<const uint4*>(qall + (static_cast<int64_t>(i) * H + hb * 16 + j16) * 128 + g * 32);
      qraw[hb][0] = qp[0];
      qraw[hb][1] = qp[1];
      wraw[hb] = *reinterpret_cast<const float4*>(a.w + static_cast<int64_t>(i) * H + hb * 16 + g * 4);
    }
    const uint32_t W = static_cast<uint32_t>(n_chunk) * 4u;                     // waves of this query
    const uint32_t wq = static_cast<uint32_t>(chunk) * 4u + static_cast<uint32_t>(wv);   // this wave's turn
    // the wave's groups: first, first + step, ...  Contiguous shares split
    // the ld / 64 groups of a row as evenly as the W waves allow (at most R each)
    const uint32_t Gp = static_cast<uint32_t>((a.ld + kGroupKeys - 1) / kGroupKeys);
    const uint32_t first = IL ? wq : static_cast<uint32_t>(static_cast<uint64_t>(wq) * Gp / W);
    const uint32_t step = IL ? W : 1u;
    PagedTab pt{};
    if (kPaged) paged_tab_load(a, i, first, step, R, lane, pt);
    const int64_t qpos = scalar_load(a.q_pos, i), koff = kPaged ? 0 : scalar_load(a.key_off, i);
    int64_t lo = 0, hi = 0, row0 = 0;                  // query i's segment of the key job
    if (kNew && i < nk.nseg) {
      lo = scalar_load(nk.seg_tok_off, i);
      hi = scalar_load(nk.seg_tok_off, i + 1);
      row0 = scalar_load(nk.seg_out_row, i);
    }
    asm volatile("" : : "s"(qpos), "s"(koff), "s"(lo), "s"(hi), "s"(row0) : "memory");   // one round trip; the loads above stay above
    int64_t N = (uniform64(qpos) + 1) / a.m;
    if (N > a.ld) N = a.ld;
    // scores this wave may store: all N, less the last when the launch
    // compresses that row (the rule by which csa_compress places block j of
    // a segment at row seg_out_row + j)
    int64_t Ns = N;
    if (kNew && N >= 1 && i < nk.nseg) {
      // (paged: the pool row of the last visible row)
      const int64_t last = kPaged ? pool_row(a, i, N - 1) : uniform64(koff) + N - 1;
      const int64_t j = last - uniform64(row0);
      const int64_t end = uniform64(lo) + (j + 1) * nk.m;
      if (j >= 0 && uniform64(lo) % nk.m == 0 && end <= uniform64(hi) && end <= nk.n_tok) Ns = N - 1;
    }
    // (N <= 2^24, so group counts fit 32 bits)
    const uint32_t G = static_cast<uint32_t>((N + kGroupKeys - 1) / kGroupKeys);
    const uint64_t pool_bytes = static_cast<uint64_t>(a.pool_rows) * 128u;
    const buf_rsrc rs = kPaged ? make_rsrc(a.keys, pool_bytes < 0xffffffffull ? static_cast<uint32_t>(pool_bytes)
                                                                             : 0xffffffffu)
                               : make_rsrc(static_cast<const uint8_t*>(a.keys) + uniform64(koff) * 128,
                                           static_cast<uint32_t>(N * 128));
    if (first >= G) continue;                            // uniform over the wave (no barriers)
    uint32_t mine;
    if (IL) {
      mine = (G - first + step - 1u) / step;
    } else {
      const uint32_t end = static_cast<uint32_t>(static_cast<uint64_t>(wq + 1u) * Gp / W);
      mine = (end < G ? end : G) - first;
    }
    const int ng = mine < static_cast<uint32_t>(R) ? static_cast<int>(mine) : R;
    const uint32_t s0 = first * kGroupKeys;              // first key of the wave's first group
    const uint32_t stride = step * (kGroupKeys * 128u);
    const uint32_t voff0 = static_cast<uint32_t>(s0 + j16) * 128u + g * 32u;
    uint4 kr[NB][4][2];                                  // NB groups in flight
    auto load = [&](int t, uint4 (&dst)[4][2]) __attribute__((always_inline)) {
      if (kPaged) load_group_fp8_paged(rs, pt, a.blk_shift, first, step, t, ng, j16, g, dst);
      else load_group_fp8(rs, voff0, stride, t, ng, dst);
    };
#pragma unroll
    for (int u = 0; u < NB; ++u) load(u, kr[u]);
    // the query is used only from here on: its conversion must not be
    // scheduled above the key loads (it would wait for the query first)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      asm volatile("" : "+v"(qraw[hb][0].x), "+v"(qraw[hb][0].y), "+v"(qraw[hb][0].z), "+v"(qraw[hb][0].w),
                   "+v"(qraw[hb][1].x), "+v"(qraw[hb][1].y), "+v"(qraw[hb][1].z), "+v"(qraw[hb][1].w),
                   "+v"(wraw[hb].x), "+v"(wraw[hb].y), "+v"(wraw[hb].z), "+v"(wraw[hb].w) : : "memory");
    bf16x8 qb[NHB][4];
    float wr[NHB][4];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      qb[hb][0] = fp8x8_to_bf16(qraw[hb][0].x, qraw[hb][0].y);
      qb[hb][1] = fp8x8_to_bf16(qraw[hb][0].z, qraw[hb][0].w);
      qb[hb][2] = fp8x8_to_bf16(qraw[hb][1].x, qraw[hb][1].y);
      qb[hb][3] = fp8x8_to_bf16(qraw[hb][1].z, qraw[hb][1].w);
      wr[hb][0] = wraw[hb].x; wr[hb][1] = wraw[hb].y; wr[hb][2] = wraw[hb].z; wr[hb][3] = wraw[hb].w;
    }
    // scores: a descriptor over the query's N valid scores drops stores past
    // N; lanes other than row group 0 (which hold the same totals) aim past it
    const buf_rsrc out_rs = make_rsrc(a.scores + static_cast<int64_t>(i) * a.ld, static_cast<uint32_t>(Ns * 4));
    const uint32_t out_off = g == 0 ? static_cast<uint32_t>(s0 + j16) * 4u : 0x80000000u;
    f32x4 cp[NHB];
    for (int hb = 0; hb < NHB; ++hb) cp[hb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int pend = -1;
    const int out_stride = static_cast<int>(step * kGroupKeys * 4u);
    // groups in pairs, both always processed (a group past the wave's share
    // holds zeros and keeps no score)
    for (int t = 0; t < ng; t += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        group_fp8<NHB>(kr[u], qb, wr, cp, pend, t + u < ng ? (t + u) * out_stride : -1, out_rs, out_off);
        load(t + u + NB, kr[u]);
      }
    }
    const float tot = head_sum<NHB>(cp, wr);
    if (pend >= 0)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rs, static_cast<int>(out_off), pend, 0);
  }
}

template <int NHB, bool IL, bool kPaged = false>
__global__ void __launch_bounds__(256) indexer_fp8_kernel(IndexerArgs a, int64_t n_items,
                                                          int64_t n_chunk, int R) {
  fp8_items<NHB, IL, false, 2, kPaged>(a, n_items, n_chunk, R, blockIdx.x, gridDim.x, NewKeys{});
}

// Score of a key row the launch has just compressed (the FP8 rounding of
// y[0 .. 128), as stored) for query s, when that row is the query's last
// visible row.  Wave 0 repeats the streaming kernel's arithmetic for this one
// key: the key sits in the MFMA column the streaming kernel gives it
// ((N - 1) mod 16), with the same dim order, products, chain and head sum,
// so the score has the same bits.
template <int NHB, bool kPaged>
__device__ __forceinline__ void score_new_key(const IndexerArgs& a, const float* y, int s, int64_t row) {
  constexpr int H = NHB * 16;
  if (threadIdx.x >= 64 || s >= a.nq) return;          // wave 0; uniform
  const int lane = threadIdx.x, g = lane >> 4, j16 = lane & 15;
  const uint8_t* qall = static_cast<const uint8_t*>(a.q);
  uint4 qraw[NHB][2];
  float4 wraw[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const uint4* qp = reinterpret_cast<const uint4*>(qall + (static_cast<int64_t>(s) * H + hb * 16 + j16) * 128 + g * 32);
    qraw[hb][0] = qp[0];
    qraw[hb][1] = qp[1];
    wraw[hb] = *reinterpret_cast<const float4*>(a.w + static_cast<int64_t>(s) * H + hb * 16 + g * 4);
  }
  const int64_t qpos = scalar_load(a.q_pos, s), koff = kPaged ? 0 : scalar_load(a.key_off, s);
  int64_t N = (uniform64(qpos) + 1) / a.m;
  if (N > a.ld) N = a.ld;
  if (N < 1) return;
  if ((kPaged ? pool_row(a, s, N - 1) : uniform64(koff) + N - 1) != row) return;
  // lane (column j16, k-slot g) holds dims [32g + 8ks, +8) at k-step ks
  bf16x8 kk[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint32_t w4[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) w4[e >> 2] |= f32_to_e4m3(y[32 * g + 8 * ks + e]) << (8 * (e & 3));
    kk[ks] = fp8x8_to_bf16(w4[0], w4[1]);
  }
  bf16x8 qb[NHB][4];
  float wr[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    qb[hb][0] = fp8x8_to_bf16(qraw[hb][0].x, qraw[hb][0].y);
    qb[hb][1] = fp8x8_to_bf16(qraw[hb][0].z, qraw[hb][0].w);
    qb[hb][2] = fp8x8_to_bf16(qraw[hb][1].x, qraw[hb][1].y);
    qb[hb][3] = fp8x8_to_bf16(qraw[hb][1].z, qraw[hb][1].w);
    wr[hb][0] = wraw[hb].x; wr[hb][1] = wraw[hb].y; wr[hb][2] = wraw[hb].z; wr[hb][3] = wraw[hb].w;
  }
  f32x4 cc[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) cc[hb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      cc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[hb][ks], kk[ks], cc[hb], 0, 0, 0);
  const float tot = head_sum<NHB>(cc, wr);
  if (g == 0 && j16 == static_cast<int>((N - 1) & 15)) a.scores[static_cast<int64_t>(s) * a.ld + N - 1] = tot;
}

// A decode step's compress jobs and its indexer scores in one launch.
// Workgroups [0, n_cwg) compress (the job kernel's loop over the jobs'
// blocks); the workgroup of a new key row also scores it for the query whose
// last visible row it is.  The rest stream every other score.  No workgroup
// waits for another: a query's rows other than its last are not written by
// the launch, and its last row is scored by exactly one side.
template <int NHB, bool IL, bool kWithAny, int NB, bool kPaged>
__global__ void __launch_bounds__(256) compress_score_kernel(CompressJobs J, int key_job, NewKeys nk,
                                                             IndexerArgs a, int64_t n_items, int64_t n_chunk,
                                                             int R, int n_cwg) {
  if (static_cast<int>(blockIdx.x) < n_cwg) {
    extern __shared__ float y[];
    __shared__ cmp::EntrySlot slot;
    const int64_t total = J.blk0[J.n];
    for (int64_t b = blockIdx.x; b < total; b += n_cwg) {
      int j = 0;
      while (j + 1 < J.n && b >= J.blk0[j + 1]) ++j;
      const CompressArgs& c = J.a[j];
      cmp::run_block<kWithAny>(c, J.kind[j], b - J.blk0[j], y, y + c.D, &slot);
      if (j == key_job && slot.ok) score_new_key<NHB, kPaged>(a, y, slot.seg, slot.row);
      __syncthreads();                                  // y and slot are reused by the next block
    }
    return;
  }
  fp8_items<NHB, IL, true, NB, kPaged>(a, n_items, n_chunk, R, blockIdx.x - n_cwg, gridDim.x - n_cwg, nk);
}

// --------------------------------------------------------------- FP8, d = 128, shared keys
// A prefill batch holds many queries of one sequence, which read the same key
// rows.  A workgroup takes QS consecutive queries (one per wave; QS = 8, or 4
// for 128 heads, whose registers leave no room for the longer step) and a
// run of up to kShareGroups 64-key groups.  When they read the same rows
// (equal key offsets), the keys go by in steps of QS blocks of 16: each step
// is loaded once -- wave w loads block w with the lane pattern of the
// streaming kernel -- widened once into LDS, and every wave multiplies it
// against its own query (QS queries share each widening).  The operands, MFMA tiles,
// their order and the head sum are those of the streaming kernel, so a score
// has the same bits whichever kernel computed it.  Keys past a query's own N
// are multiplied but their scores are not stored.  A block whose queries read
// different rows streams each wave's own groups instead.
template <int NHB> constexpr int share_q() { return NHB >= 8 ? 4 : 8; }
constexpr int kShareGroups = 32;
constexpr int kShareMinQueries = 1024;   // batches this large take the shared-key kernel

template <int QS>
struct SharedKeys {
  bf16x8 k[2][QS][4][64];   // [buffer][block][k-step][lane]
};

// One 16-key block from widened operands: the per-block step of group_fp8.
template <int NHB>
__device__ __forceinline__ void block_bf16(const bf16x8 (&kk)[4], const bf16x8 (&qb)[NHB][4],
                                           const float (&wr)[NHB][4], f32x4 (&cp)[NHB], int& pend, int nxt,
                                           buf_rsrc out_rs, uint32_t out_off) {
  f32x4 cc[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) cc[hb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      cc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[hb][ks], kk[ks], cc[hb], 0, 0, 0);
  const float tot = head_sum<NHB>(cp, wr);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rs,
                                        static_cast<int>(pend >= 0 ? out_off : 0x80000000u),
                                        pend >= 0 ? pend : 0, 0);
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) cp[hb] = cc[hb];
  pend = nxt;
}

// kPaged: keys through the block table; the queries of a workgroup share
// their keys when they share a table row.  Wave wv's 16-key block of step s
// lies in one table block (block_rows >= 16, blocks start at multiples of
// 16), so each step needs one table entry per wave: lane s of the wave loads
// the entry of step s when the unit starts, and step s reads it with readlane.
template <int NHB, bool kPaged>
__global__ void __launch_bounds__(share_q<NHB>() * 64) indexer_fp8_shared_kernel(IndexerArgs a, int64_t n_qblk,
                                                                                 int64_t n_kchunk) {
  constexpr int H = NHB * 16;
  constexpr int kShareQ = share_q<NHB>();
  constexpr uint32_t kShareStepKeys = kShareQ * 16;   // keys per step: one 16-key block per wave
  __shared__ SharedKeys<kShareQ> sk;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 4, j16 = lane & 15;
  const uint8_t* qall = static_cast<const uint8_t*>(a.q);
  for (int64_t unit = blockIdx.x; unit < n_qblk * n_kchunk; unit += gridDim.x) {
    const int i0 = static_cast<int>(unit / n_kchunk) * kShareQ;
    const uint32_t t0 = static_cast<uint32_t>(unit % n_kchunk) * kShareGroups;
    const int nqb = a.nq - i0 < kShareQ ? a.nq - i0 : kShareQ;    // queries in the block (uniform)
    const bool mine = wv < nqb;
    const int i = mine ? i0 + wv : i0;                  // a wave past the batch reads query i0, stores nothing
    // this wave's query rows and weights, then the block's positions and key offsets
    uint4 qraw[NHB][2];
    float4 wraw[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const uint4* qp = reinterpret_cast<const uint4*>(qall + (static_cast<int64_t>(i) * H + hb * 16 + j16) * 128 + g * 32);
      qraw[hb][0] = qp[0];
      qraw[hb][1] = qp[1];
      wraw[hb] = *reinterpret_cast<const float4*>(a.w + static_cast<int64_t>(i) * H + hb * 16 + g * 4);
    }
    int64_t koff0 = 0, koff_i = 0, N_i = 0, N_max = 0;
    bool same = true;
#pragma unroll
    for (int q = 0; q < kShareQ; ++q) {
      const int iq = i0 + (q < nqb ? q : 0);
      // paged: the table row stands in for the key offset (same row, same keys)
      const int64_t ko = kPaged ? table_row(a, iq) : uniform64(scalar_load(a.key_off, iq));
      int64_t n = (uniform64(scalar_load(a.q_pos, iq)) + 1) / a.m;
      n = n > a.ld ? a.ld : n;
      if (q == 0) koff0 = ko;
      same = same && ko == koff0;
      N_max = n > N_max ? n : N_max;
      if (q == wv) { koff_i = ko; N_i = n; }
    }
    const uint32_t G = static_cast<uint32_t>((N_max + kGroupKeys - 1) / kGroupKeys);
    if (t0 >= G) continue;                               // uniform over the workgroup
    const uint32_t t1 = G - t0 < static_cast<uint32_t>(kShareGroups) ? G : t0 + kShareGroups;
    bf16x8 qb[NHB][4];
    float wr[NHB][4];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      qb[hb][0] = fp8x8_to_bf16(qraw[hb][0].x, qraw[hb][0].y);
      qb[hb][1] = fp8x8_to_bf16(qraw[hb][0].z, qraw[hb][0].w);
      qb[hb][2] = fp8x8_to_bf16(qraw[hb][1].x, qraw[hb][1].y);
      qb[hb][3] = fp8x8_to_bf16(qraw[hb][1].z, qraw[hb][1].w);
      wr[hb][0] = wraw[hb].x; wr[hb][1] = wraw[hb].y; wr[hb][2] = wraw[hb].z; wr[hb][3] = wraw[hb].w;
    }
    const buf_rsrc out_rs = make_rsrc(a.scores + static_cast<int64_t>(i) * a.ld,
                                      mine ? static_cast<uint32_t>(N_i * 4) : 0u);
    const uint32_t out_off = g == 0 ? static_cast<uint32_t>(j16) * 4u : 0x80000000u;
    f32x4 cp[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) cp[hb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int pend = -1;
    const uint64_t pool_bytes = static_cast<uint64_t>(a.pool_rows) * 128u;
    const uint32_t pool_lim = pool_bytes < 0xffffffffull ? static_cast<uint32_t>(pool_bytes) : 0xffffffffu;
    if (same) {
      // wave wv loads block wv of every step: rows k0 + s*kShareStepKeys + wv*16 + j16, bytes [32g, 32g+32)
      const buf_rsrc rs = kPaged ? make_rsrc(a.keys, pool_lim)
                                 : make_rsrc(static_cast<const uint8_t*>(a.keys) + koff0 * 128,
                                             static_cast<uint32_t>(N_max * 128));
      const uint32_t k0 = t0 * kGroupKeys;                 // first key of the run
      const uint32_t n_st = ((t1 - t0) * kGroupKeys + kShareStepKeys - 1) / kShareStepKeys;
      const uint32_t voff0 = (k0 + static_cast<uint32_t>(wv) * 16u + j16) * 128u + g * 32u;
      // paged: lane s holds the table entry of the wave's block in step s
      // (n_st <= 32); a block past the query's visible rows reads block 0
      // (masked: its scores are never stored)
      int32_t tab_e = 0;
      if (kPaged) {
        const uint32_t key = k0 + static_cast<uint32_t>(lane) * kShareStepKeys + static_cast<uint32_t>(wv) * 16u;
        const uint32_t lb = key >> a.blk_shift;
        const bool ok = static_cast<uint32_t>(lane) < n_st && key < static_cast<uint64_t>(N_max);
        tab_e = __builtin_amdgcn_raw_buffer_load_b32(table_rsrc(a, koff0), ok ? static_cast<int>(lb * 4u)
                                                                               : static_cast<int>(0x80000000u), 0, 0);
      }
      // step s -> buffer s % 2; its loads went out two steps earlier
      auto load = [&](uint4 (&kr)[2], uint32_t st) __attribute__((always_inline)) {
        uint32_t o;
        if (kPaged) {
          const uint32_t key = k0 + st * kShareStepKeys + static_cast<uint32_t>(wv) * 16u;
          const uint32_t blk = static_cast<uint32_t>(__builtin_amdgcn_readlane(tab_e, static_cast<int>(st & 63u)));
          const uint32_t row = (blk << a.blk_shift) | (key & ((1u << a.blk_shift) - 1u));
          o = st < n_st ? (row + static_cast<uint32_t>(j16)) * 128u + static_cast<uint32_t>(g) * 32u : 0x80000000u;
        } else {
          o = st < n_st ? voff0 + st * (kShareStepKeys * 128u) : 0x80000000u;   // past the run: no traffic
        }
        kr[0] = buf_load_x4(rs, o, 0);
        kr[1] = buf_load_x4(rs, o + 16u, 0);
      };
      auto step = [&](uint4 (&kr)[2], uint32_t st, int buf) __attribute__((always_inline)) {
        bf16x8* dst = &sk.k[buf][wv][0][lane];
        dst[0] = fp8x8_to_bf16(kr[0].x, kr[0].y);
        dst[64] = fp8x8_to_bf16(kr[0].z, kr[0].w);
        dst[128] = fp8x8_to_bf16(kr[1].x, kr[1].y);
        dst[192] = fp8x8_to_bf16(kr[1].z, kr[1].w);
        // the buffer holds the whole step once every wave's LDS writes are
        // done (and every wave has read the step two back from it); the
        // barrier waits for LDS only, so the key loads stay in flight
        asm volatile("" : : : "memory");
        __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" : : : "memory");
        load(kr, st + 2);                                // two steps ahead
        asm volatile("" : : : "memory");                 // (issued before the step's LDS reads)
#pragma unroll
        for (int kb = 0; kb < kShareQ; ++kb) {
          const bf16x8 kk[4] = {sk.k[buf][kb][0][lane], sk.k[buf][kb][1][lane], sk.k[buf][kb][2][lane],
                                sk.k[buf][kb][3][lane]};
          block_bf16<NHB>(kk, qb, wr, cp, pend, static_cast<int>((k0 + st * kShareStepKeys + kb * 16u) * 4u),
                          out_rs, out_off);
        }
      };
      uint4 ka[2], kb2[2];
      load(ka, 0);
      asm volatile("" : : : "memory");                   // in this order: the loop's waits count on it
      load(kb2, 1);
      for (uint32_t st = 0; st < n_st; st += 2) {
        step(ka, st, 0);
        if (st + 1 < n_st) step(kb2, st + 1, 1);         // uniform over the workgroup
      }
    } else {
      // the wave's own rows, group by group (no barriers: the branch is
      // uniform over the workgroup and this path has none)
      const buf_rsrc rs = kPaged ? make_rsrc(a.keys, pool_lim)
                                 : make_rsrc(static_cast<const uint8_t*>(a.keys) + koff_i * 128,
                                             static_cast<uint32_t>(N_i * 128));
      const uint32_t voff0 = (t0 * kGroupKeys + j16) * 128u + g * 32u;
      const int ng = static_cast<int>(t1 - t0);
      PagedTab pt{};
      if (kPaged) paged_tab_load(a, i, t0, 1u, ng, lane, pt);
      uint4 ka[4][2];
      for (int t = 0; t < ng; ++t) {
        if (kPaged) load_group_fp8_paged(rs, pt, a.blk_shift, t0, 1u, t, ng, j16, g, ka);
        else load_group_fp8(rs, voff0, kGroupKeys * 128u, t, ng, ka);
        group_fp8<NHB>(ka, qb, wr, cp, pend, static_cast<int>((t0 + static_cast<uint32_t>(t)) * kGroupKeys * 4u),
                       out_rs, out_off);
      }
    }
    const float tot = head_sum<NHB>(cp, wr);
    if (pend >= 0)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rs, static_cast<int>(out_off), pend, 0);
    __syncthreads();                                     // the next unit refills the buffers
  }
}

// --------------------------------------------------------------- MXFP4, d = 128
// Row: 64 bytes of E2M1 codes then 4 E8M0 scales.  Scaled MFMA 16x16x128:
// lane (row j16, k-block g) supplies 16 code bytes and the scale of block g.
// Shares of 64-key groups as in the FP8 kernel.
constexpr uint32_t kRowFp4 = 68;

// voff0: start of the lane's key row; lane takes code bytes [16g, 16g+16) and
// the scale byte 64 + g of each row
__device__ __forceinline__ void load_group_fp4(buf_rsrc rs, uint32_t voff0, uint32_t g, uint32_t stride, int t,
                                               int ng, uint4 (&kc)[4], uint32_t (&ks)[4]) {
  const uint32_t base = t < ng ? voff0 + static_cast<uint32_t>(t) * stride : 0x80000000u;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    kc[kb] = buf_load_x4(rs, base + 16u * g, kb * 16u * kRowFp4);
    ks[kb] = __builtin_amdgcn_raw_buffer_load_b8(rs, static_cast<int>(base + 64u + g),
                                                 static_cast<int>(kb * 16u * kRowFp4), 0);
  }
}

__device__ __forceinline__ void load_group_fp4_paged(buf_rsrc rs, const PagedTab& pt, int sh, uint32_t first,
                                                     uint32_t step, int t, int ng, int j16, uint32_t g,
                                                     uint4 (&kc)[4], uint32_t (&ks)[4]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint32_t base = t < ng ? (paged_row(pt, sh, first, step, t, kb) + static_cast<uint32_t>(j16)) * kRowFp4
                                 : 0x80000000u;
    kc[kb] = buf_load_x4(rs, base + 16u * g, 0);
    ks[kb] = __builtin_amdgcn_raw_buffer_load_b8(rs, static_cast<int>(base + 64u + g), 0, 0);
  }
}

template <int NHB>
__device__ __forceinline__ void group_fp4(const uint4 (&kc)[4], const uint32_t (&ks)[4], const i32x8 (&qop)[NHB],
                                          const int (&qsc)[NHB], const float (&wr)[NHB][4], f32x4 (&cp)[NHB],
                                          int& pend, int grp, buf_rsrc out_rs, uint32_t out_off) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const i32x8 kop = {static_cast<int>(kc[kb].x), static_cast<int>(kc[kb].y), static_cast<int>(kc[kb].z),
                       static_cast<int>(kc[kb].w), 0, 0, 0, 0};
    f32x4 cc[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      cc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          qop[hb], kop, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0, qsc[hb], 0, static_cast<int>(ks[kb]));
    const float tot = head_sum<NHB>(cp, wr);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rs,
                                          static_cast<int>(pend >= 0 ? out_off : 0x80000000u),
                                          pend >= 0 ? pend : 0, 0);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) cp[hb] = cc[hb];
    pend = grp >= 0 ? grp + kb * 64 : -1;
  }
}

template <int NHB, bool IL, bool kPaged = false>
__global__ void __launch_bounds__(256) indexer_mxfp4_kernel(IndexerArgs a, int64_t n_items,
                                                            int64_t n_chunk, int R) {
  constexpr int H = NHB * 16;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 4, j16 = lane & 15;
  const uint8_t* qall = static_cast<const uint8_t*>(a.q);
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int i = static_cast<int>(item / n_chunk);
    const int64_t chunk = item % n_chunk;
    // query codes, scales and weights first, with the position and key offset
    // (see the FP8 kernel)
    i32x8 qop[NHB];
    int qsc[NHB];
    float4 wraw[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const uint8_t* row = qall + (static_cast<int64_t>(i) * H + hb * 16 + j16) * kRowFp4;
      const uint4 c4 = *reinterpret_cast<const uint4*>(row + g * 16);
      qop[hb] = i32x8{static_cast<int>(c4.x), static_cast<int>(c4.y), static_cast<int>(c4.z),
                      static_cast<int>(c4.w), 0, 0, 0, 0};
      qsc[hb] = row[64 + g];
      wraw[hb] = *reinterpret_cast<const float4*>(a.w + static_cast<int64_t>(i) * H + hb * 16 + g * 4);
    }
    const uint32_t W = static_cast<uint32_t>(n_chunk) * 4u;
    const uint32_t wq = static_cast<uint32_t>(chunk) * 4u + static_cast<uint32_t>(wv);
    const uint32_t first = IL ? wq : wq * static_cast<uint32_t>(R);
    const uint32_t step = IL ? W : 1u;
    PagedTab pt{};
    if (kPaged) paged_tab_load(a, i, first, step, R, lane, pt);
    const int64_t qpos = scalar_load(a.q_pos, i), koff = kPaged ? 0 : scalar_load(a.key_off, i);
    asm volatile("" : : "s"(qpos), "s"(koff) : "memory");   // one round trip; the loads above stay above
    int64_t N = (uniform64(qpos) + 1) / a.m;
    if (N > a.ld) N = a.ld;
    const uint32_t G = static_cast<uint32_t>((N + kGroupKeys - 1) / kGroupKeys);
    const uint64_t pool_bytes = static_cast<uint64_t>(a.pool_rows) * kRowFp4;
    const buf_rsrc rs = kPaged ? make_rsrc(a.keys, pool_bytes < 0xffffffffull ? static_cast<uint32_t>(pool_bytes)
                                                                             : 0xffffffffu)
                               : make_rsrc(static_cast<const uint8_t*>(a.keys) + uniform64(koff) * kRowFp4,
                                           static_cast<uint32_t>(N * kRowFp4));
    if (first >= G) continue;                            // uniform over the wave (no barriers)
    const uint32_t mine = (G - first + step - 1u) / step;
    const int ng = mine < static_cast<uint32_t>(R) ? static_cast<int>(mine) : R;
    const uint32_t s0 = first * kGroupKeys;
    const uint32_t stride = step * (kGroupKeys * kRowFp4);
    const uint32_t voff0 = static_cast<uint32_t>(s0 + j16) * kRowFp4;
    uint4 kca[4], kcb[4];
    uint32_t ksa[4], ksb[4];
    auto load = [&](int t, uint4 (&kc)[4], uint32_t (&ks)[4]) __attribute__((always_inline)) {
      if (kPaged) load_group_fp4_paged(rs, pt, a.blk_shift, first, step, t, ng, j16, static_cast<uint32_t>(g), kc, ks);
      else load_group_fp4(rs, voff0, static_cast<uint32_t>(g), stride, t, ng, kc, ks);
    };
    load(0, kca, ksa);
    load(1, kcb, ksb);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      asm volatile("" : "+v"(wraw[hb].x), "+v"(wraw[hb].y), "+v"(wraw[hb].z), "+v"(wraw[hb].w) : : "memory");
    float wr[NHB][4];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      wr[hb][0] = wraw[hb].x; wr[hb][1] = wraw[hb].y; wr[hb][2] = wraw[hb].z; wr[hb][3] = wraw[hb].w;
    }
    const buf_rsrc out_rs = make_rsrc(a.scores + static_cast<int64_t>(i) * a.ld, static_cast<uint32_t>(N * 4));
    const uint32_t out_off = g == 0 ? static_cast<uint32_t>(s0 + j16) * 4u : 0x80000000u;
    f32x4 cp[NHB];
    for (int hb = 0; hb < NHB; ++hb) cp[hb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int pend = -1;
    const int out_stride = static_cast<int>(step * kGroupKeys * 4u);
    for (int t = 0; t < ng; t += 2) {
      group_fp4<NHB>(kca, ksa, qop, qsc, wr, cp, pend, t * out_stride, out_rs, out_off);
      load(t + 2, kca, ksa);
      group_fp4<NHB>(kcb, ksb, qop, qsc, wr, cp, pend, t + 1 < ng ? (t + 1) * out_stride : -1, out_rs, out_off);
      load(t + 3, kcb, ksb);
    }
    const float tot = head_sum<NHB>(cp, wr);
    if (pend >= 0)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rs, static_cast<int>(out_off), pend, 0);
  }
}

// --------------------------------------------------------------- F32 (any small shape)
// One thread per key; query and weights in LDS; dims and heads in order.
__global__ void __launch_bounds__(256) indexer_f32_kernel(IndexerArgs a, int64_t n_chunk) {
  extern __shared__ float qs[];      // [H*d] then [H]
  const int i = static_cast<int>(blockIdx.x / n_chunk);
  const int64_t chunk = blockIdx.x % n_chunk;
  int64_t N = (a.q_pos[i] + 1) / a.m;
  if (N > a.ld) N = a.ld;
  if (chunk * 256 >= N) return;
  const int Hd = a.H * a.d;
  const float* q = static_cast<const float*>(a.q) + static_cast<int64_t>(i) * Hd;
  for (int t = threadIdx.x; t < Hd; t += 256) qs[t] = q[t];
  for (int t = threadIdx.x; t < a.H; t += 256) qs[Hd + t] = a.w[static_cast<int64_t>(i) * a.H + t];
  __syncthreads();
  const int64_t s = chunk * 256 + threadIdx.x;
  if (s >= N) return;
  const float* k = static_cast<const float*>(a.keys) + (a.key_off[i] + s) * a.d;
  float tot = 0.0f;
  for (int h = 0; h < a.H; ++h) {
    float dot = 0.0f;
    for (int c = 0; c < a.d; ++c) dot = fmaf(qs[h * a.d + c], k[c], dot);
    tot = fmaf(qs[Hd + h], fmaxf(dot, 0.0f), tot);
  }
  a.scores[static_cast<int64_t>(i) * a.ld + s] = tot;
}

// Work split of the streaming kernels: enough 64-key groups per wave (the
// share R) that one round of two waves per SIMD covers the batch, at least 2
// (two groups in flight), at most 32; an item is four waves of one query.
struct StreamPlan {
  int64_t R, n_chunk, n_items;
  unsigned grid;
};

StreamPlan plan_stream(const IndexerArgs& a) {
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  const int64_t groups = static_cast<int64_t>(a.nq) * ((a.ld + kGroupKeys - 1) / kGroupKeys);
  const int64_t waves = static_cast<int64_t>(device_cu_count()) * 8;
  int64_t R = (groups + waves - 1) / waves;
  R = R < 2 ? 2 : (R > 32 ? 32 : R);
  const int64_t item_keys = 4 * R * kGroupKeys;
  const int64_t n_chunk = (a.ld + item_keys - 1) / item_keys;
  const int64_t n_items = static_cast<int64_t>(a.nq) * n_chunk;
  return StreamPlan{R, n_chunk, n_items, static_cast<unsigned>(n_items < cap ? n_items : cap)};
}

static_assert(sizeof(CompressJobs) + sizeof(NewKeys) + sizeof(IndexerArgs) + 64 <= 4096,
              "kernel arguments are limited to 4 KiB");

}  // namespace

hipError_t launch_compress_score(const CompressArgs* jobs, int n, int key_job, const IndexerArgs& a,
                                 hipStream_t stream) {
  if (a.fmt != CSA_FP8 || a.nq == 0 || a.nq >= kShareMinQueries) {
    const hipError_t e = launch_compress_jobs(jobs, n, stream);
    return e != hipSuccess ? e : launch_indexer(a, stream);
  }
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
  if (J.n == 0) return launch_indexer(a, stream);
  StreamPlan p = plan_stream(a);
  const bool il = p.R > 2;                             // interleaved shares (long rows)
  const int64_t total = J.blk0[J.n];
  const int n_cwg = static_cast<int>(total < 65536 ? total : 65536);
  // The compress workgroups take resident slots (two workgroups per CU at
  // this kernel's register count).  When the plan's contiguous shares fill
  // every slot, fewer items of slightly longer shares let the whole launch
  // run in one round instead of leaving n_cwg items for a second one.
  const int64_t slots = static_cast<int64_t>(device_cu_count()) * 2;
  if (p.R <= 2 && p.n_items + n_cwg > slots && slots - n_cwg >= a.nq) {
    const int64_t gp = (a.ld + kGroupKeys - 1) / kGroupKeys;
    p.n_chunk = (slots - n_cwg) / a.nq;
    p.n_items = static_cast<int64_t>(a.nq) * p.n_chunk;
    p.R = (gp + 4 * p.n_chunk - 1) / (4 * p.n_chunk);
    p.grid = static_cast<unsigned>(p.n_items);
  }
  const dim3 grid(static_cast<unsigned>(n_cwg) + p.grid), block(256);
  const size_t shm = cmp::shm_bytes(maxD);
  const bool paged = a.blk_table != nullptr;
  log_launch("compress+score: one launch%s, %d jobs in %d workgroups + FP8 indexer of %d queries in %u workgroups "
             "(%lld groups per wave)", paged ? " (paged keys)" : "", J.n, n_cwg, a.nq, p.grid,
             static_cast<long long>(p.R));
  const int r = static_cast<int>(p.R);
  const bool three = !il && p.R == 3;                 // every group of a three-group share in flight
#define CSA_CS_LAUNCH(NB, IL, ANY, BUF)                                                                    \
  do {                                                                                                    \
    if (paged) hipLaunchKernelGGL((compress_score_kernel<NB, IL, ANY, BUF, true>), grid, block, shm, stream, J, \
                                  kj, nk, a, p.n_items, p.n_chunk, r, n_cwg);                             \
    else hipLaunchKernelGGL((compress_score_kernel<NB, IL, ANY, BUF, false>), grid, block, shm, stream, J, kj, \
                            nk, a, p.n_items, p.n_chunk, r, n_cwg);                                       \
  } while (0)
#define CSA_CS_CASE(NB)                                                                                   \
  case NB:                                                                                                \
    if (il) { if (any) CSA_CS_LAUNCH(NB, true, true, 2); else CSA_CS_LAUNCH(NB, true, false, 2); }       \
    else if (three) { if (any) CSA_CS_LAUNCH(NB, false, true, 3); else CSA_CS_LAUNCH(NB, false, false, 3); } \
    else { if (any) CSA_CS_LAUNCH(NB, false, true, 2); else CSA_CS_LAUNCH(NB, false, false, 2); }        \
    break;
  switch (a.H / 16) {
    CSA_CS_CASE(1)
    CSA_CS_CASE(2)
    CSA_CS_CASE(4)
    CSA_CS_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef CSA_CS_CASE
#undef CSA_CS_LAUNCH
  return hipGetLastError();
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  if (a.fmt == CSA_F32) {
    const int64_t n_chunk = (a.ld + 255) / 256;
    const size_t shm = (static_cast<size_t>(a.H) * a.d + a.H) * sizeof(float);
    log_launch("indexer: fp32 kernel, %d queries x %d heads, grid %lld x 256 threads", a.nq, a.H,
               static_cast<long long>(a.nq * n_chunk));
    hipLaunchKernelGGL(indexer_f32_kernel, dim3(static_cast<unsigned>(a.nq * n_chunk)), dim3(256),
                       shm, stream, a, n_chunk);
    return hipGetLastError();
  }
  const int nhb = a.H / 16;
  const StreamPlan p = plan_stream(a);
  const bool paged = a.blk_table != nullptr;
  const int64_t n_items = p.n_items, n_chunk = p.n_chunk;
  const unsigned grid = p.grid;
  const int r = static_cast<int>(p.R);
  const bool il = p.R > 2;
#define CSA_IDX_CASE(K, NB)                                                                              \
  case NB:                                                                                               \
    if (paged) {                                                                                         \
      if (il) hipLaunchKernelGGL((K<NB, true, true>), dim3(grid), dim3(256), 0, stream, a, n_items, n_chunk, r); \
      else hipLaunchKernelGGL((K<NB, false, true>), dim3(grid), dim3(256), 0, stream, a, n_items, n_chunk, r); \
    } else {                                                                                             \
      if (il) hipLaunchKernelGGL((K<NB, true, false>), dim3(grid), dim3(256), 0, stream, a, n_items, n_chunk, r); \
      else hipLaunchKernelGGL((K<NB, false, false>), dim3(grid), dim3(256), 0, stream, a, n_items, n_chunk, r); \
    }                                                                                                    \
    break;
  if (a.fmt == CSA_FP8 && a.nq >= kShareMinQueries) {
    // QS queries (waves) per workgroup; resident workgroups per CU from the
    // kernel's register count (two waves per SIMD at 64 heads and more)
    const int qs = nhb >= 8 ? share_q<8>() : share_q<1>();
    const int64_t n_qblk = (a.nq + qs - 1) / qs;
    const int64_t n_kchunk = ((a.ld + kGroupKeys - 1) / kGroupKeys + kShareGroups - 1) / kShareGroups;
    const int64_t units = n_qblk * n_kchunk;
    const int64_t waves_cu = nhb <= 2 ? 16 : 8;
    const int64_t cap_o = static_cast<int64_t>(device_cu_count()) * (waves_cu / qs);   // resident workgroups
    const unsigned grid_s = static_cast<unsigned>(units < cap_o ? units : cap_o);
    const dim3 blk(static_cast<unsigned>(qs * 64));
    log_launch("indexer: FP8 shared-key kernel%s, %d queries x %d heads, %lld query blocks x %lld key chunks, "
               "grid %u x %u threads", paged ? " (paged)" : "", a.nq, a.H, static_cast<long long>(n_qblk),
               static_cast<long long>(n_kchunk), grid_s, blk.x);
#define CSA_SHARED_CASE(NB)                                                                              \
  case NB:                                                                                               \
    if (paged) hipLaunchKernelGGL((indexer_fp8_shared_kernel<NB, true>), dim3(grid_s), blk, 0, stream, a, n_qblk, n_kchunk); \
    else hipLaunchKernelGGL((indexer_fp8_shared_kernel<NB, false>), dim3(grid_s), blk, 0, stream, a, n_qblk, n_kchunk); \
    break;
    switch (nhb) {
      CSA_SHARED_CASE(1)
      CSA_SHARED_CASE(2)
      CSA_SHARED_CASE(4)
      CSA_SHARED_CASE(8)
      default: return hipErrorInvalidValue;
    }
#undef CSA_SHARED_CASE
    return hipGetLastError();
  }
  log_launch("indexer: %s streaming kernel%s, %d queries x %d heads, ld %lld, %lld items of %d waves x %lld "
             "groups (%s shares), grid %u x 256 threads", a.fmt == CSA_FP8 ? "FP8" : "MXFP4", paged ? " (paged)" : "",
             a.nq, a.H, static_cast<long long>(a.ld), static_cast<long long>(n_items), 4, static_cast<long long>(p.R),
             il ? "interleaved" : "contiguous", grid);
  if (a.fmt == CSA_FP8) {
    switch (nhb) {
      CSA_IDX_CASE(indexer_fp8_kernel, 1)
      CSA_IDX_CASE(indexer_fp8_kernel, 2)
      CSA_IDX_CASE(indexer_fp8_kernel, 4)
      CSA_IDX_CASE(indexer_fp8_kernel, 8)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (nhb) {
      CSA_IDX_CASE(indexer_mxfp4_kernel, 1)
      CSA_IDX_CASE(indexer_mxfp4_kernel, 2)
      CSA_IDX_CASE(indexer_mxfp4_kernel, 4)
      CSA_IDX_CASE(indexer_mxfp4_kernel, 8)
      default: return hipErrorInvalidValue;
    }
  }
#undef CSA_IDX_CASE
  return hipGetLastError();
}

}  // namespace csa
