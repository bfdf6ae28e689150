// Sink multi-query attention over [compressed entries] ++ [sliding window]
// (hybrid_attn_decode / hybrid_attn_prefill).
//
// Source: 硅星人 article on DeepSeek V4, CSA paragraph (selected entries plus
// the 128-token window go to core multi-query attention) and HCA paragraph
// (all entries plus the window); DeepSeek-V4 blog, RMSNorm归一化 (query heads
// normalised), Partial RoPE位置编码 (RoPE on the last 64 dims; window of raw
// entries used alongside compressed ones) and 让注意力学会"忽略" (a per-head
// sink logit joins the softmax denominator); QbitAI piece on batch
// invariance (no split-KV: one (query, head) is never reduced across
// workgroups).
//
// Two paths:
//  * attn_f32_kernel -- everything float32 (reference-precision path): one
//    wave per (query, head), entries in list order, exact-order wave sums.
//  * attn_mfma_kernel -- q BF16, cache SPLIT (448 FP8 dims + 64 BF16 RoPE
//    dims, D = 512), window BF16, out BF16.  One workgroup (4 waves) per
//    (query, 16-head tile, slice of the output dims).  Entries stream through
//    LDS in tiles of 64: every wave computes the logits of 16 entries of the
//    tile for the 16 heads, the tile max / sum are combined across the 4 waves
//    in a fixed order, and each wave accumulates P.V for its own output dims.
//    Tiles arrive in LDS as the raw stored rows through direct global->LDS
//    loads, double-buffered.  Logits use BF16 MFMA (FP8 -> BF16 is exact; FP8
//    MFMA accumulation is too coarse for logits, whose sum cancels).  For
//    P.V the 448 FP8 dims multiply the raw bytes on FP8 MFMA with the
//    probabilities split into an FP8 high part and an FP8 residual (~8
//    significant bits); the RoPE dims and the window use BF16 MFMA.  V
//    operands are read transposed from the row-major tile with
//    ds_read_tr8 / ds_read_tr16.
//    Every variant runs the same per-tile instruction sequence for a given
//    (query, head); variants only change which workgroup owns which output
//    dims, so the output bits are the same.
#include "kernels.hpp"

namespace csa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ window bounds
__device__ __forceinline__ void window_of(const AttnArgs& a, int b, int64_t p, int64_t* row0,
                                          int* count) {
  if (a.win_mode == 0 || a.n_win == 0) {   // no window
    *row0 = 0;
    *count = 0;
  } else if (a.win_mode == 1) {             // decode: rows [0, win_len) of win[b]
    int c = a.win_len[b];
    c = c < 0 ? 0 : (c > a.n_win ? a.n_win : c);
    *row0 = static_cast<int64_t>(b) * a.n_win;
    *count = c;
  } else {                                  // prefill: positions max(0, p-n_win+1) .. p of the run
    int64_t first = p - a.n_win + 1;
    if (first < 0) first = 0;
    if (first < a.tok_pos0[b]) first = a.tok_pos0[b];
    const int64_t c = p - first + 1;
    *row0 = a.tok_off[b] + (first - a.tok_pos0[b]);
    *count = c > 0 ? static_cast<int>(c) : 0;
  }
}

// ================================================================== fp32 path
// One wave per (query, head); lane holds dims [lane*P, lane*P + P), P = D/64.
template <int P>
__global__ void __launch_bounds__(256) attn_f32_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= a.nq * a.H) return;
  const int b = unit / a.H, h = unit % a.H;
  const int D = a.D, R = a.rope_dim;
  const int64_t p = a.q_pos[b];
  const float* q = static_cast<const float*>(a.q) + (static_cast<int64_t>(b) * a.H + h) * D;
  float qh[P];
  float ss = 0.0f;
#pragma unroll
  for (int t = 0; t < P; ++t) {
    qh[t] = q[lane * P + t];
    ss = fmaf(qh[t], qh[t], ss);
  }
  ss = wave_sum(ss);
  const float r = static_cast<float>(1.0 / sqrt(static_cast<double>(ss) / D + a.eps));
#pragma unroll
  for (int t = 0; t < P; ++t) qh[t] = qh[t] * r * (a.q_norm_w ? a.q_norm_w[lane * P + t] : 1.0f);
  if (R > 0) {
#pragma unroll
    for (int t = 0; t < P; t += 2) {
      const int d = lane * P + t;
      if (d >= D - R) {
        float sn, cs;
        rope_sincos(p, a.rope_theta[(d - (D - R)) / 2], &sn, &cs);
        const float x0 = qh[t], x1 = qh[t + 1];
        qh[t] = x0 * cs - x1 * sn;
        qh[t + 1] = x0 * sn + x1 * cs;
      }
    }
  }
  const int64_t N = (p + 1) / a.m;
  float mx = a.sinks[h], l = 1.0f;
  float acc[P];
#pragma unroll
  for (int t = 0; t < P; ++t) acc[t] = 0.0f;
  auto step = [&](const float* e) {
    float dot = 0.0f;
#pragma unroll
    for (int t = 0; t < P; ++t) dot = fmaf(qh[t], e[lane * P + t], dot);
    dot = wave_sum(dot) * a.scale;
    const float mn = fmaxf(mx, dot);
    const float al = expf(mx - mn), pj = expf(dot - mn);
    l = l * al + pj;
#pragma unroll
    for (int t = 0; t < P; ++t) acc[t] = acc[t] * al + pj * e[lane * P + t];
    mx = mn;
  };
  const float* kv = static_cast<const float*>(a.kv) + a.kv_off[b] * D;
  if (a.idx != nullptr) {
    const int32_t* ix = a.idx + static_cast<int64_t>(b) * a.k;
    for (int j = 0; j < a.k; ++j) {
      const int32_t e = ix[j];
      if (e >= 0 && e < N) step(kv + static_cast<int64_t>(e) * D);
    }
  } else {
    for (int64_t e = 0; e < N; ++e) step(kv + e * D);
  }
  int64_t row0;
  int wc;
  window_of(a, b, p, &row0, &wc);
  const float* win = static_cast<const float*>(a.win) + row0 * D;
  for (int j = 0; j < wc; ++j) step(win + static_cast<int64_t>(j) * D);
  float* o = static_cast<float*>(a.out) + (static_cast<int64_t>(b) * a.H + h) * D;
#pragma unroll
  for (int t = 0; t < P; ++t) o[lane * P + t] = acc[t] / l;
}

// ================================================================== MFMA path
constexpr int kD = 512, kR = 64, kDF8 = 448;            // dims, RoPE dims, FP8 dims
constexpr int kRowSplit = kDF8 + 2 * kR;                // 576 bytes per cache entry
constexpr int kRowBf16 = 2 * kD;                        // 1024 bytes per window row
constexpr int kChunksSplit = kRowSplit / 16;            // 36 chunks of 16 bytes
constexpr int kPitchSplit = kRowSplit + 16;             // LDS row pitch: rows land on distinct banks
constexpr int kPitchWin = kRowBf16 + 16;
constexpr int kTile = 64;                               // entries per tile
constexpr int kThreads = 256;
constexpr int kBufBytes = kTile * kPitchWin;            // raw tile buffer (largest row format)
constexpr int kMaxK = 2048;                             // longest selected list kept in LDS
constexpr int kPPitch8 = 72;                            // padded rows of the fp8 P arrays
constexpr int kPPitch16 = 72;                           // padded rows (elements) of the bf16 P array
constexpr float kPScale = 256.0f;                       // probabilities are stored x 2^8

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Raw rows land in LDS as stored (split: 576-byte rows, window: 1024-byte rows)
// through direct global->LDS loads, one wave instruction per row, at a pitch
// padded by 16 bytes so that neighbouring rows start on different banks.  Every
// operand address is then a per-lane base plus a compile-time offset.
struct __align__(16) AttnSmem {
  uint8_t raw[2][kBufBytes];       // double-buffered tiles
  int32_t sel[kMaxK];              // selected entry list (CSA), -1 where dropped
  uint8_t phi[16][kPPitch8];       // fp8 high part of p * 2^8   [head][entry]
  uint8_t plo[16][kPPitch8];       // fp8 residual
  uint16_t pbf[16][kPPitch16];     // bf16(p * 2^8)
  float red_max[4][16];
  float red_sum[4][16];
  float rope_cs[kR / 2][2];        // cos, sin of the query's RoPE angles
  int valid[2][kTile];
};

__device__ __forceinline__ const lds_u8* lds_ptr(const uint8_t* p) {
  // the tile lives in LDS; a C-style cast changes the address space
  return (const lds_u8*)(p);
}

__device__ __forceinline__ long lds_read_b64(const uint8_t* p) {
  return *reinterpret_cast<const long*>(p);
}

__device__ __forceinline__ long tr8(const uint8_t* p) {
  typedef __attribute__((address_space(3))) i32x2 lds_t;
  i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_t*)(lds_ptr(p)));
  return __builtin_bit_cast(long, v);
}

__device__ __forceinline__ bf16x4 tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_t;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_t*)(lds_ptr(p)));
}

__device__ __forceinline__ uint32_t fp8x2(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t v) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v), false);
}
// two floats -> packed bf16 (hardware conversion, round to nearest even)
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// 8 FP8 values (exact) -> 8 BF16 values.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(long v) {
  const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(static_cast<unsigned long>(v) >> 32);
  const bf16x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
}

// Per-query description of the attended list: n_ct tiles of compressed
// entries (list positions [0, n_list)), then n_wt tiles of window rows.
struct Work {
  int b;
  int64_t p, N, kv0, win_row0;
  int n_list, n_ct, n_wt, win_count;
};

// Issue the direct global->LDS loads of tile `tile` into buffer `buf` and
// write its per-row validity.  One wave instruction moves one row (36 lanes x
// 16 bytes for a split row, 64 lanes for a window row) to the row's padded LDS
// slot.  Rows without an entry load a real row (entry 0 / window row 0) and
// are masked by `valid`, so no stale bits reach P.V.
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const Work& w, int tile, int buf,
                                           AttnSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint8_t* dst = sm.raw[buf];
  if (tile < w.n_ct) {
    const uint8_t* kv = static_cast<const uint8_t*>(a.kv) + w.kv0 * kRowSplit + lane * 16;
    // lane l < 16 looks up the entry of this wave's row 4l + wv; readlane makes it scalar
    int my_e = 0;
    if (lane < kTile / 4) {
      const int pos = tile * kTile + lane * 4 + wv;
      if (pos < w.n_list) {
        const int e = a.idx != nullptr ? sm.sel[pos] : pos;
        my_e = e < 0 ? 0 : e;
      }
    }
    if (lane < kChunksSplit) {
#pragma unroll
      for (int i = 0; i < kTile / 4; ++i) {                             // 16 rows per wave
        const int row = i * 4 + wv;
        const int e = __builtin_amdgcn_readlane(my_e, i);
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(kv + static_cast<int64_t>(e) * kRowSplit),
            (__attribute__((address_space(3))) void*)(lds_ptr(dst + row * kPitchSplit)), 16, 0, 0);
      }
    }
    if (tid < kTile) {
      const int pos = tile * kTile + tid;
      int ok = 0;
      if (pos < w.n_list) ok = a.idx != nullptr ? (sm.sel[pos] >= 0) : 1;
      sm.valid[buf][tid] = ok;
    }
  } else {
    const uint8_t* win = static_cast<const uint8_t*>(a.win) + w.win_row0 * kRowBf16 + lane * 16;
    const int wt = tile - w.n_ct;
#pragma unroll
    for (int i = 0; i < kTile / 4; ++i) {                               // 16 rows per wave
      const int row = i * 4 + wv;
      const int j = wt * kTile + row;
      const int src = j < w.win_count ? j : 0;
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(win + static_cast<int64_t>(src) * kRowBf16),
          (__attribute__((address_space(3))) void*)(lds_ptr(dst + row * kPitchWin)), 16, 0, 0);
    }
    if (tid < kTile) sm.valid[buf][tid] = wt * kTile + tid < w.win_count;
  }
}

// DVS = number of workgroups sharing one (query, 16-head tile): each owns
// 512 / DVS output dims, i.e. DW = 128 / DVS per wave.
template <int DVS>
__global__ void __launch_bounds__(kThreads) attn_mfma_kernel(AttnArgs a, int n_units,
                                                             int n_pad) {
  constexpr int DW = 128 / DVS;        // output dims per wave
  constexpr int NB = DW / 16;          // 16-dim MFMA blocks per wave
  extern __shared__ __align__(16) uint8_t smem_raw[];
  AttnSmem& sm = *reinterpret_cast<AttnSmem*>(smem_raw);

  // XCD-aware unit order: workgroups i, i+8, i+16, ... run on one XCD, so
  // consecutive units (the head tiles and dim slices of one query) share an L2.
  const int gid = blockIdx.x;
  const int per_xcd = n_pad / 8;
  const int unit = (gid % 8) * per_xcd + gid / 8;
  if (unit >= n_units) return;
  const int n_ht = a.H / 16;
  const int dvs = unit % DVS;
  const int ht = (unit / DVS) % n_ht;
  const int b = unit / (DVS * n_ht);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, j16 = lane & 15;

  Work w;
  w.b = b;
  w.p = a.q_pos[b];
  w.N = (w.p + 1) / a.m;
  w.kv0 = a.kv_off[b];
  window_of(a, b, w.p, &w.win_row0, &w.win_count);
  if (a.idx != nullptr) {
    w.n_list = w.N > 0 ? a.k : 0;
    for (int j = tid; j < a.k; j += kThreads) {
      const int32_t e = a.idx[static_cast<int64_t>(b) * a.k + j];
      sm.sel[j] = (e >= 0 && e < w.N) ? e : -1;
    }
  } else {
    w.n_list = static_cast<int>(w.N);
  }
  w.n_ct = (w.n_list + kTile - 1) / kTile;
  w.n_wt = (w.win_count + kTile - 1) / kTile;
  const int n_tiles = w.n_ct + w.n_wt;
  if (tid < kR / 2) {
    float sn, cs;
    rope_sincos(w.p, a.rope_theta[tid], &sn, &cs);
    sm.rope_cs[tid][0] = cs;
    sm.rope_cs[tid][1] = sn;
  }
  __syncthreads();                                      // sel[] and rope_cs ready

  if (n_tiles > 0) issue_tile(a, w, 0, 0, sm);

  // ---------------- prologue: qhat = RoPE(RMSNorm(q)) for 16 heads, staged in raw[1]
  uint16_t(*qbf)[kD] = reinterpret_cast<uint16_t(*)[kD]>(sm.raw[1]);
  {
    const int h = tid >> 4, c = tid & 15;          // head in tile, 32-dim chunk
    const int hg = ht * 16 + h;
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(b) * a.H + hg) * kD + c * 32;
    float x[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(q)[i];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        x[i * 8 + 2 * t] = bf16_to_f32(static_cast<uint16_t>(u[t] & 0xffff));
        x[i * 8 + 2 * t + 1] = bf16_to_f32(static_cast<uint16_t>(u[t] >> 16));
      }
    }
    float ss = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t) ss = fmaf(x[t], x[t], ss);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float r = static_cast<float>(1.0 / sqrt(static_cast<double>(ss) / kD + a.eps));
#pragma unroll
    for (int t = 0; t < 32; ++t) x[t] = x[t] * r * (a.q_norm_w ? a.q_norm_w[c * 32 + t] : 1.0f);
    if (c * 32 >= kD - kR) {
      const int p0 = (c * 32 - (kD - kR)) / 2;
#pragma unroll
      for (int t = 0; t < 32; t += 2) {
        const float cs = sm.rope_cs[p0 + t / 2][0], sn = sm.rope_cs[p0 + t / 2][1];
        const float x0 = x[t], x1 = x[t + 1];
        x[t] = x0 * cs - x1 * sn;
        x[t + 1] = x0 * sn + x1 * cs;
      }
    }
#pragma unroll
    for (int t = 0; t < 32; t += 8) {
      uint4 v;
      v.x = bf16x2_rne(x[t], x[t + 1]);
      v.y = bf16x2_rne(x[t + 2], x[t + 3]);
      v.z = bf16x2_rne(x[t + 4], x[t + 5]);
      v.w = bf16x2_rne(x[t + 6], x[t + 7]);
      *reinterpret_cast<uint4*>(&qbf[h][c * 32 + t]) = v;
    }
  }
  __syncthreads();
  // QK operand of this lane: head j16, dims [32*ks + 8*g, +8)
  bf16x8 qb[kD / 32];
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(&qbf[j16][ks * 32 + g * 8]);
  const float ch = a.scale * kLog2e;
  __syncthreads();                                      // raw[1] free again

  // softmax state for head j16 (identical in all lanes of that head)
  float m_run = a.sinks[ht * 16 + j16] * kLog2e;
  float l_run = 1.0f;
  f32x4 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int dbase = dvs * (kD / DVS) + wv * DW;         // first output dim of this wave

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    const bool is_win = tile >= w.n_ct;
    __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0): this tile's loads landed
    __syncthreads();                                    // ... in every wave; previous P.V done
    if (tile + 1 < n_tiles) issue_tile(a, w, tile + 1, buf ^ 1, sm);
    const uint8_t* T = sm.raw[buf];

    // -------- logits for entries 16*wv .. 16*wv+15 (rows), heads (cols)
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    const int erow = wv * 16 + j16;
    if (!is_win) {
      const uint8_t* rowp = T + erow * kPitchSplit + g * 8;
      long ka[kDF8 / 32];
#pragma unroll
      for (int ks = 0; ks < kDF8 / 32; ++ks) ka[ks] = lds_read_b64(rowp + ks * 32);
      bf16x8 kr[kR / 32];
#pragma unroll
      for (int ks = 0; ks < kR / 32; ++ks)
        kr[ks] = *reinterpret_cast<const bf16x8*>(rowp + kDF8 + g * 8 + ks * 64);
#pragma unroll
      for (int ks = 0; ks < kDF8 / 32; ++ks)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(ka[ks]), qb[ks], s, 0, 0, 0);
#pragma unroll
      for (int ks = 0; ks < kR / 32; ++ks)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks], qb[kDF8 / 32 + ks], s, 0, 0, 0);
    } else {
      const uint8_t* rowp = T + erow * kPitchWin + g * 16;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 kw[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          kw[ks] = *reinterpret_cast<const bf16x8*>(rowp + (half * 8 + ks) * 64);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kw[ks], qb[half * 8 + ks], s, 0, 0, 0);
      }
    }
    // lane holds head j16, entries 16*wv + 4*g + r
    float t[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = sm.valid[buf][wv * 16 + g * 4 + r] != 0;
      t[r] = ok ? s[r] * ch : -INFINITY;
      mx = fmaxf(mx, t[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (lane < 16) sm.red_max[wv][j16] = mx;
    __syncthreads();
    const float tmax = fmaxf(fmaxf(sm.red_max[0][j16], sm.red_max[1][j16]),
                             fmaxf(sm.red_max[2][j16], sm.red_max[3][j16]));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float pv[4];
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = exp2f(t[r] - m_new);
      ps += pv[r];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    if (lane < 16) sm.red_sum[wv][j16] = ps;
    // probabilities to LDS in the P^T operand layout [head][entry]
    {
      const int e0 = wv * 16 + g * 4;
      const float v0 = pv[0] * kPScale, v1 = pv[1] * kPScale, v2 = pv[2] * kPScale, v3 = pv[3] * kPScale;
      const uint32_t h01 = fp8x2(v0, v1), h23 = fp8x2(v2, v3);
      const f32x2 d01 = fp8x2_to_f32(h01), d23 = fp8x2_to_f32(h23);
      const uint32_t l01 = fp8x2(v0 - d01[0], v1 - d01[1]), l23 = fp8x2(v2 - d23[0], v3 - d23[1]);
      *reinterpret_cast<uint32_t*>(&sm.phi[j16][e0]) = h01 | (h23 << 16);
      *reinterpret_cast<uint32_t*>(&sm.plo[j16][e0]) = l01 | (l23 << 16);
      uint2 bb;
      bb.x = bf16x2_rne(v0, v1);
      bb.y = bf16x2_rne(v2, v3);
      *reinterpret_cast<uint2*>(&sm.pbf[j16][e0]) = bb;
    }
    __syncthreads();
    const float tsum = ((sm.red_sum[0][j16] + sm.red_sum[1][j16]) + sm.red_sum[2][j16]) + sm.red_sum[3][j16];
    l_run = l_run * alpha + tsum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[i] *= alpha;

    // -------- P.V for dims [dbase, dbase + DW): rows = dims, cols = heads
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {                     // entries [32*ks, 32*ks + 32)
      const int ebase = ks * 32 + g * 8;
      const long phv = lds_read_b64(&sm.phi[j16][ebase]);
      const long plv = lds_read_b64(&sm.plo[j16][ebase]);
      const bf16x8 pbv = *reinterpret_cast<const bf16x8*>(&sm.pbf[j16][ebase]);
      if (!is_win) {
        // fp8 dims: lane j of group g supplies row (ebase + j/2), bytes d0 + 8*(j%2)
        const uint8_t* b8 = T + (ebase + (j16 >> 1)) * kPitchSplit + dbase + 8 * (j16 & 1);
        // bf16 RoPE dims: lane j supplies row (ebase + j/4), dims d0 + 4*(j%4)
        const uint8_t* b16 = T + (ebase + (j16 >> 2)) * kPitchSplit + kDF8 + (dbase - kDF8) * 2 + 8 * (j16 & 3);
        long v8[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i)
          if (dbase + i * 16 < kDF8) v8[i] = tr8(b8 + i * 16);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (dbase + i * 16 < kDF8) {
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(v8[i], phv, acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(v8[i], plv, acc[i], 0, 0, 0);
          } else {
            const bf16x4 lo4 = tr16(b16 + i * 32);
            const bf16x4 hi4 = tr16(b16 + i * 32 + 4 * kPitchSplit);
            const bf16x8 av = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pbv, acc[i], 0, 0, 0);
          }
        }
      } else {
        const uint8_t* b16 = T + (ebase + (j16 >> 2)) * kPitchWin + dbase * 2 + 8 * (j16 & 3);
        bf16x8 vw[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const bf16x4 lo4 = tr16(b16 + i * 32);
          const bf16x4 hi4 = tr16(b16 + i * 32 + 4 * kPitchWin);
          vw[i] = bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vw[i], pbv, acc[i], 0, 0, 0);
      }
    }
  }

  // -------- epilogue: out = acc / (2^8 * l)
  const float inv = 1.0f / (l_run * kPScale);
  uint16_t* out = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(b) * a.H + ht * 16 + j16) * kD;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int d = dbase + i * 16 + g * 4;
    uint2 v;
    v.x = static_cast<uint32_t>(f32_to_bf16(acc[i][0] * inv)) | (static_cast<uint32_t>(f32_to_bf16(acc[i][1] * inv)) << 16);
    v.y = static_cast<uint32_t>(f32_to_bf16(acc[i][2] * inv)) | (static_cast<uint32_t>(f32_to_bf16(acc[i][3] * inv)) << 16);
    *reinterpret_cast<uint2*>(out + d) = v;
  }
}

}  // namespace

int pick_dvs(int variant, int units, int cus) {
  if (variant == CSA_VARIANT_HIGH_OCC) return 1;
  if (variant == CSA_VARIANT_LOW_OCC) return 4;
  if (units >= 2 * cus) return 1;
  if (units >= cus) return 2;
  return 4;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  const bool f32 = a.q_fmt == CSA_F32;
  if (f32) {
    const int units = a.nq * a.H;
    const dim3 grid((units + 3) / 4);
    switch (a.D / 64) {
      case 2: hipLaunchKernelGGL(attn_f32_kernel<2>, grid, dim3(256), 0, stream, a); break;
      case 4: hipLaunchKernelGGL(attn_f32_kernel<4>, grid, dim3(256), 0, stream, a); break;
      case 6: hipLaunchKernelGGL(attn_f32_kernel<6>, grid, dim3(256), 0, stream, a); break;
      case 8: hipLaunchKernelGGL(attn_f32_kernel<8>, grid, dim3(256), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int base_units = a.nq * (a.H / 16);
  const int dvs = pick_dvs(a.variant, base_units, device_cu_count());
  const int units = base_units * dvs;
  const int n_pad = (units + 7) / 8 * 8;
  const size_t shm = sizeof(AttnSmem);
  // the workgroup needs more than the default 64 KB of dynamic LDS
  static thread_local int attr_set_dev = -1;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (attr_set_dev != dev) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_mfma_kernel<1>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm));
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_mfma_kernel<2>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm));
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_mfma_kernel<4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm));
    if (e != hipSuccess) return e;
    attr_set_dev = dev;
  }
  switch (dvs) {
    case 1: hipLaunchKernelGGL(attn_mfma_kernel<1>, dim3(n_pad), dim3(kThreads), shm, stream, a, units, n_pad); break;
    case 2: hipLaunchKernelGGL(attn_mfma_kernel<2>, dim3(n_pad), dim3(kThreads), shm, stream, a, units, n_pad); break;
    default: hipLaunchKernelGGL(attn_mfma_kernel<4>, dim3(n_pad), dim3(kThreads), shm, stream, a, units, n_pad); break;
  }
  return hipGetLastError();
}

size_t attn_mfma_smem_bytes() { return sizeof(AttnSmem); }

}  // namespace csa
