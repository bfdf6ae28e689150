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
#include "indexer_dev.hpp"

namespace csa {

namespace {

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
