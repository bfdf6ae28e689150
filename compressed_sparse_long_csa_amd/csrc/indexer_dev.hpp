// Device code of the streaming FP8 indexer shared by the translation units
// that launch it: the key loads, the MFMA blocks and the head sum, the item
// loop (fp8_items), the new-key score and the one-launch compress + score
// kernel, and the host-side work split.  See indexer.hip for the method.
#pragma once

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

// ------------------------------------------------------- fused top-k selection
// csa_compress_score_topk: the top-k of each query's scores is selected in
// the launch that computes them (硅星人 article, CSA paragraph: the selector
// keeps the k best-scored entries).  Selection is by an order-preserving
// 32-bit key of each score (NaN -> -inf, -0 -> +0; ties to the lower index),
// taken 12 + 12 + 8 bits at a time:
//  * level 1 while scoring: every stored score adds one to bin key >> 20 of
//    its workgroup's LDS bins; at the end of an item those bins are added to
//    the query's global bins (integer atomics, so the counts do not depend on
//    the order the workgroups run in);
//  * each workgroup then counts itself in the query's arrival counter; the
//    last of the query's arrivals (its items, plus the compressing workgroup
//    when that one scores the new key) selects: it finds the level-1 bin b1
//    holding the k-th largest key, counts keys of b1 by bits 19..8 in LDS
//    (bin b2), then by bits 7..0 (b3), which gives the exact k-th key T and
//    the number of keys equal to T to take; a last pass writes the selected
//    indices in ascending order (a block scan places each thread's run).
// Nothing waits for another workgroup: the last arrival does the work.  The
// global bins and the counter are left at zero for the next call.
// Coherence: each XCD has its own L2, so an agent-scope release fence would
// write back the whole L2 at every arrival.  Instead the data that crosses
// workgroups takes device-coherent accesses: scores are stored and loaded
// with the sc1 cache bit (agent scope), bins and counters are atomics, and an
// arrival waits for its own stores to complete (vmcnt 0) before it counts.
constexpr int kTkSc1 = 16;                     // cache-policy operand: sc1 (agent-coherent access)
// (kTkBins level-1 bins of key >> 20 and the counter per query: kernels.hpp)
constexpr uint32_t kTkTile = 16384;            // scores a pass holds in registers (64 per thread)

struct TkSmem {
  uint32_t h[kTkBins];     // an item's level-1 bins while scoring; level 2 while selecting
  uint32_t h3[256];        // level 3
  uint32_t red[4];         // per-wave scan totals
  uint32_t red2[4];
  uint32_t sh[4];          // b1, keys above b1, b2 .. results passed to every thread
  int last;                // this workgroup made the query's last arrival
  int q;                   // compressing side: query to select (-1: none)
  int64_t n;               // its visible rows
};

__device__ __forceinline__ uint32_t tk_key(float v) {
  v = v == v ? v + 0.0f : -INFINITY;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A score just stored at byte `off` of its row (valid below `lim`) joins its bin.
__device__ __forceinline__ void tk_count(float tot, uint32_t off, uint32_t lim, uint32_t* lh) {
  if (off < lim) atomicAdd(&lh[tk_key(tot) >> 20], 1u);
}

// Zero the LDS bins (every thread of the workgroup; ends with a barrier).
__device__ __forceinline__ void tk_clear(TkSmem& ts) {
  for (int b = threadIdx.x; b < kTkBins; b += 256) ts.h[b] = 0u;
  ts.h3[threadIdx.x] = 0u;
  __syncthreads();
}

// Inclusive prefix of v over the 256 threads in thread order; *tot the sum.
__device__ __forceinline__ uint32_t tk_scan(uint32_t v, TkSmem& ts, uint32_t& tot) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = __shfl_up(v, d);
    v += lane >= d ? u : 0u;
  }
  if (lane == 63) ts.red[wv] = v;
  __syncthreads();
  uint32_t base = 0;
  tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t r = ts.red[w];
    base += w < wv ? r : 0u;
    tot += r;
  }
  __syncthreads();                                       // red is reused by the next scan
  return base + v;
}

// The bin of 16 * threads holding the need-th largest key: thread t holds
// bins [16t, 16t + 16) in c; the thread whose range crosses `need` (counting
// from the top) writes the bin to sh[slot] and the count above it to
// sh[slot + 1].  Ends with a barrier.
__device__ __forceinline__ void tk_find16(const uint32_t (&c)[16], uint32_t need, TkSmem& ts, int slot) {
  uint32_t sum = 0;
#pragma unroll
  for (int b = 0; b < 16; ++b) sum += c[b];
  uint32_t tot;
  const uint32_t incl = tk_scan(sum, ts, tot);
  const uint32_t above = tot - incl;
  if (above < need && above + sum >= need) {
    uint32_t acc = above;
    int b = 15;
    for (; b > 0; --b) {
      if (acc + c[b] >= need) break;
      acc += c[b];
    }
    ts.sh[slot] = 16u * threadIdx.x + static_cast<uint32_t>(b);
    ts.sh[slot + 1] = acc;
  }
  __syncthreads();
}

// Keys of tile `tl` of a row of n scores: wave w holds scores [tl * kTkTile +
// 4096 w, +4096), lane l every 64th from l (kv[c]: score 64 c + l of the
// wave's range), so each load instruction reads 256 contiguous bytes; slots
// past n hold key 0, below every score's key.  rs: a (uniform) descriptor
// over the row; agent-coherent loads.
__device__ __forceinline__ void tk_load(buf_rsrc rs, int64_t n, uint32_t tl, uint32_t (&kv)[64]) {
  const uint32_t e0 = tl * kTkTile + (threadIdx.x >> 6) * 4096u + (threadIdx.x & 63u);
  // every load is issued before any is used (slots past n read zero through
  // the descriptor's range check); without the empty asm the compiler moves
  // each load into the select's branch and waits for it there
  int v[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) v[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>((e0 + 64u * c) * 4u), 0, kTkSc1);
#pragma unroll
  for (int c = 0; c < 64; ++c) asm volatile("" : "+v"(v[c]));
#pragma unroll
  for (int c = 0; c < 64; ++c)
    kv[c] = static_cast<int64_t>(e0 + 64u * c) < n ? tk_key(__int_as_float(v[c])) : 0u;
}

__device__ __forceinline__ uint32_t tk_below(uint64_t mask) {   // set lanes of mask below this lane
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Select query i's top-k from its n scores (row `row`) and the global bins
// `gb`; the whole workgroup calls it.  Not inlined: one copy serves every
// kernel instance (it runs once per query).
__device__ __noinline__ void tk_select(const TopkFuse& tk, TkSmem& ts, int i, int64_t n, const float* row) {
  // (arguments of a call arrive in vector registers: make them wave-uniform)
  i = __builtin_amdgcn_readfirstlane(i);
  n = uniform64(n);
  row = reinterpret_cast<const float*>(uniform64(reinterpret_cast<int64_t>(row)));
  const uint32_t t = threadIdx.x, lane = t & 63u, wv = t >> 6;
  const uint32_t k = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(tk.k));
  uint32_t* gb = reinterpret_cast<uint32_t*>(uniform64(reinterpret_cast<int64_t>(tk.ws))) +
                 static_cast<int64_t>(i) * kTkWsWords;
  int32_t* out = reinterpret_cast<int32_t*>(uniform64(reinterpret_cast<int64_t>(tk.idx))) +
                 static_cast<int64_t>(i) * k;
  // the query's level-1 bins, read coalesced (agent-coherent) into LDS and
  // cleared behind; all loads are in flight before the first is used
  const buf_rsrc gr = make_rsrc(gb, kTkBins * 4u);
  int bv[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) bv[b] = __builtin_amdgcn_raw_buffer_load_b32(gr, static_cast<int>((t + 256u * b) * 4u), 0, kTkSc1);
#pragma unroll
  for (int b = 0; b < 16; ++b) asm volatile("" : "+v"(bv[b]) : : "memory");
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    ts.h[t + 256 * b] = static_cast<uint32_t>(bv[b]);
    __builtin_amdgcn_raw_buffer_store_b32(0u, gr, static_cast<int>((t + 256u * b) * 4u), 0, kTkSc1);
  }
  // every arrival is in: the counter restarts
  if (t == 0) __hip_atomic_store(gb + kTkBins, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  // thread t takes bins [16t, 16t + 16) and leaves them at zero for level 2
  uint32_t c[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    c[b] = ts.h[16 * t + b];
    ts.h[16 * t + b] = 0u;
  }
  if (n <= static_cast<int64_t>(k)) {                    // every visible row is selected
    for (uint32_t j = t; j < k; j += 256) out[j] = static_cast<int64_t>(j) < n ? static_cast<int32_t>(j) : -1;
    return;
  }
  // level 1: bin b1 of key >> 20, and the keys above it
  tk_find16(c, k, ts, 0);
  const uint32_t b1 = ts.sh[0], a1 = ts.sh[1];
  const uint32_t nt = static_cast<uint32_t>((n + kTkTile - 1) / kTkTile);
  const buf_rsrc rs = make_rsrc(row, static_cast<uint32_t>(n * 4));
  uint32_t kv[64];
  tk_load(rs, n, 0, kv);
  // level 2: keys of b1 by bits 19..8
  for (uint32_t tl = 0; tl < nt; ++tl) {
    if (tl > 0) tk_load(rs, n, tl, kv);
#pragma unroll
    for (int e = 0; e < 64; ++e)
      if ((kv[e] >> 20) == b1) atomicAdd(&ts.h[(kv[e] >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    c[b] = ts.h[16 * t + b];
    ts.h[16 * t + b] = 0u;                               // the LDS bins are left at zero
  }
  tk_find16(c, k - a1, ts, 2);
  const uint32_t p2 = (b1 << 12) | ts.sh[2], a2 = a1 + ts.sh[3];
  // level 3: keys of (b1, b2) by bits 7..0
  for (uint32_t tl = 0; tl < nt; ++tl) {
    if (nt > 1) tk_load(rs, n, tl, kv);
#pragma unroll
    for (int e = 0; e < 64; ++e)
      if ((kv[e] >> 8) == p2) atomicAdd(&ts.h3[kv[e] & 0xffu], 1u);
  }
  __syncthreads();
  const uint32_t need3 = k - a2;
  {
    const uint32_t v3 = ts.h3[t];
    uint32_t tot;
    const uint32_t incl = tk_scan(v3, ts, tot);
    const uint32_t above = tot - incl;
    if (above < need3 && above + v3 >= need3) {
      ts.sh[0] = t;
      ts.sh[1] = above;
    }
    ts.h3[t] = 0u;
    __syncthreads();
  }
  const uint32_t T = (p2 << 8) | ts.sh[0];               // the k-th largest key
  const uint32_t r = k - (a2 + ts.sh[1]);                // keys equal to T to take, lowest indices first
  // selected indices in ascending order: per tile, each wave counts its keys
  // above T and equal to T, the four counts place each wave's run, and each
  // wave writes its run in order with ballot prefix counts
  uint32_t sel_all = 0, eq_all = 0;                      // in earlier tiles
  for (uint32_t tl = 0; tl < nt; ++tl) {
    if (nt > 1) tk_load(rs, n, tl, kv);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      gt += static_cast<uint32_t>(__popcll(__ballot(kv[e] > T)));
      eq += static_cast<uint32_t>(__popcll(__ballot(kv[e] == T)));
    }
    if (lane == 0) { ts.red[wv] = gt; ts.red2[wv] = eq; }
    __syncthreads();
    uint32_t run = sel_all, erun = eq_all, eq_tot = 0, sel_tot = 0;
#pragma unroll
    for (uint32_t w = 0; w < 4; ++w) {
      const uint32_t gw = ts.red[w], ew = ts.red2[w];
      const uint32_t before = eq_all + eq_tot;           // equal keys in earlier waves and tiles
      const uint32_t take = r > before ? (r - before < ew ? r - before : ew) : 0u;
      if (w < wv) { run += gw + take; erun += ew; }
      eq_tot += ew;
      sel_tot += gw + take;
    }
    __syncthreads();                                     // red is rewritten by the next tile
    const uint32_t e0 = tl * kTkTile + wv * 4096u + lane;
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      const bool is_gt = kv[e] > T, is_eq = kv[e] == T;
      const uint64_t me = __ballot(is_eq);
      const bool sel = is_gt || (is_eq && erun + tk_below(me) < r);
      const uint64_t ms = __ballot(sel);
      const uint32_t pos = run + tk_below(ms);
      if (sel && pos < k) out[pos] = static_cast<int32_t>(e0 + 64u * e);   // (pos < k always holds)
      run += static_cast<uint32_t>(__popcll(ms));
      erun += static_cast<uint32_t>(__popcll(me));
    }
    eq_all += eq_tot;
    sel_all += sel_tot;
  }
}

// End of a streaming item: its bins join the query's, then the workgroup
// arrives; the query's E-th arrival selects.  Every thread calls it.
__device__ __forceinline__ void tk_arrive(const TopkFuse& tk, TkSmem& ts, int i, int64_t n, uint32_t E,
                                          const float* row) {
  __syncthreads();                                       // every wave's bins are in LDS
  uint32_t* gb = tk.ws + static_cast<int64_t>(i) * kTkWsWords;
  for (int b = threadIdx.x; b < kTkBins; b += 256) {
    const uint32_t cnt = ts.h[b];
    if (cnt) {
      atomicAdd(&gb[b], cnt);
      ts.h[b] = 0u;
    }
  }
  // this wave's (coherent) score stores and bin additions have completed
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    ts.last = __hip_atomic_fetch_add(&gb[kTkBins], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == E;
  __syncthreads();
  if (ts.last) tk_select(tk, ts, i, n, row);            // uniform over the workgroup
  __syncthreads();                                       // ts.last and the LDS bins are reused
}

// MFMAs of one group's blocks; the head sum of the block before (held in
// cp) is computed and stored while a block multiplies.  `pend` is the score
// offset (bytes, relative to the lane's first score) of the block in cp, or
// -1 when there is none to keep; `grp` that of this group, or -1 for a group
// past the wave's share.  Every block issues exactly one store (one with
// nothing to keep aims past the buffer), so each pass of the group loop
// issues the same memory operations and the compiler's wait counts stay exact.
// kTk: each kept score also joins its level-1 bin in lh (valid below byte lim).
template <int NHB, bool kTk = false>
__device__ __forceinline__ void group_fp8(const uint4 (&kr)[4][2], const bf16x8 (&qb)[NHB][4],
                                          const float (&wr)[NHB][4], f32x4 (&cp)[NHB], int& pend, int grp,
                                          buf_rsrc out_rs, uint32_t out_off, uint32_t* lh = nullptr,
                                          uint32_t lim = 0) {
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
                                          pend >= 0 ? pend : 0, kTk ? kTkSc1 : 0);
    if constexpr (kTk) {
      if (pend >= 0) tk_count(tot, out_off + static_cast<uint32_t>(pend), lim, lh);
    }
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
// kTk: the query's top-k is selected in the same launch (tk, ts; see above).
template <int NHB, bool IL, bool kNew, int NB = 2, bool kPaged = false, bool kTk = false>   // head blocks of 16; interleaved shares; keys written alongside; paged keys; fused top-k
__device__ __forceinline__ void fp8_items(const IndexerArgs& a, int64_t n_items, int64_t n_chunk, int R,
                                          int64_t item0, int64_t item_step, const NewKeys& nk,
                                          const TopkFuse& tk = TopkFuse{}, TkSmem* ts = nullptr) {
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
    // waves without a group skip to the end of the item (no barriers inside)
    if (first < G) {
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
          group_fp8<NHB, kTk>(kr[u], qb, wr, cp, pend, t + u < ng ? (t + u) * out_stride : -1, out_rs, out_off,
                              kTk ? ts->h : nullptr, static_cast<uint32_t>(Ns * 4));
          load(t + u + NB, kr[u]);
        }
      }
      const float tot = head_sum<NHB>(cp, wr);
      if (pend >= 0)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rs, static_cast<int>(out_off), pend,
                                              kTk ? kTkSc1 : 0);
      if constexpr (kTk) {
        if (pend >= 0) tk_count(tot, out_off + static_cast<uint32_t>(pend), static_cast<uint32_t>(Ns * 4), ts->h);
      }
    }
    if constexpr (kTk) {
      // arrivals of query i: its n_chunk items, and the compressing workgroup
      // when it scores the new key (Ns = N - 1)
      const uint32_t E = static_cast<uint32_t>(n_chunk) + (Ns != N ? 1u : 0u);
      tk_arrive(tk, *ts, i, N, E, a.scores + static_cast<int64_t>(i) * a.ld);
    }
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
// kTk: the score also joins query s's global level-1 bin and wave 0 makes
// the compressing workgroup's arrival (E: the query's arrival count); when it
// is the last, ts->q / ts->n name the query to select (the caller has set
// ts->q = -1).
template <int NHB, bool kPaged, bool kTk = false>
__device__ __forceinline__ void score_new_key(const IndexerArgs& a, const float* y, int s, int64_t row,
                                              const TopkFuse& tk = TopkFuse{}, TkSmem* ts = nullptr,
                                              uint32_t E = 0) {
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
  if (g == 0 && j16 == static_cast<int>((N - 1) & 15)) {
    float* dst = a.scores + static_cast<int64_t>(s) * a.ld + N - 1;
    if constexpr (kTk) {
      __hip_atomic_store(dst, tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // agent-coherent
      atomicAdd(&tk.ws[static_cast<int64_t>(s) * kTkWsWords + (tk_key(tot) >> 20)], 1u);
    } else {
      *dst = tot;
    }
  }
  if constexpr (kTk) {
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // the score and its bin are in
    if (lane == 0) {
      uint32_t* cnt = tk.ws + static_cast<int64_t>(s) * kTkWsWords + kTkBins;
      if (__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == E) {
        ts->q = s;
        ts->n = N;
      }
    }
  }
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

}  // namespace csa
