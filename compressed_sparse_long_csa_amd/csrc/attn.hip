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
//    dims, D = 512), window BF16, out BF16.  One workgroup of 8 waves (two
//    per SIMD) per (query, 16-head tile, slice of the output dims: DVS = 2,
//    4 or 8 workgroups share a tile, 512 / DVS dims each).  The prologue
//    normalises and rotates the tile's 16 query heads once (each wave two
//    heads, shared through LDS).  Each wave then owns a fixed interleaved
//    part of the attended list -- list positions [128 s + 16 w, +16) of the
//    compressed entries in its step s, then window rows [64 t + 8 w, +8) --
//    streams those rows into its own double-buffered LDS with direct
//    global->LDS loads (one instruction per row), and keeps its own online
//    softmax state (log2 domain; the sink enters through wave 0); there is no
//    workgroup barrier in the entry loop.  At the end the eight waves' states
//    are merged in wave order.  Logits use BF16 MFMA on the exactly widened
//    FP8 rows (FP8 MFMA accumulation is too coarse for logits, whose sum
//    cancels).  For P.V the 448 FP8 dims multiply the raw bytes on FP8 MFMA
//    with the probabilities split into an FP8 high part and an FP8 residual
//    (~8 significant bits); the RoPE dims and the window use BF16 MFMA.  V
//    operands are read transposed from the row-major step buffer with
//    ds_read_tr8 / ds_read_tr16.
//    Every variant runs the same per-step instruction sequence for a given
//    (query, head); variants only change which workgroup owns which output
//    dims, so the output bits are the same.
#include "kernels.hpp"

namespace csa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ window bounds
__device__ __forceinline__ void window_of(const AttnArgs& a, int b, int64_t p, int win_len,
                                          int64_t tok_pos0, int64_t tok_off, int64_t* row0,
                                          int* count) {
  if (a.win_mode == 0 || a.n_win == 0) {   // no window
    *row0 = 0;
    *count = 0;
  } else if (a.win_mode == 1) {             // decode: rows [0, win_len) of win[b]
    const int c = win_len < 0 ? 0 : (win_len > a.n_win ? a.n_win : win_len);
    *row0 = static_cast<int64_t>(b) * a.n_win;
    *count = c;
  } else {                                  // prefill: positions max(0, p-n_win+1) .. p of the run
    int64_t first = p - a.n_win + 1;
    if (first < 0) first = 0;
    if (first < tok_pos0) first = tok_pos0;
    const int64_t c = p - first + 1;
    *row0 = tok_off + (first - tok_pos0);
    *count = c > 0 ? static_cast<int>(c) : 0;
  }
}
__device__ __forceinline__ void window_of(const AttnArgs& a, int b, int64_t p, int64_t* row0,
                                          int* count) {
  window_of(a, b, p, a.win_mode == 1 ? a.win_len[b] : 0, a.win_mode == 2 ? a.tok_pos0[b] : 0,
            a.win_mode == 2 ? a.tok_off[b] : 0, row0, count);
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
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;                   // two waves per SIMD
constexpr int kStepE = 16;                              // compressed entries per wave step
constexpr int kStepW = 8;                               // window rows per wave step
constexpr int kBufBytes = kStepE * kPitchSplit;         // one step's rows (>= kStepW * kPitchWin)
constexpr int kPPitch = 20;                             // padded rows of the P arrays
constexpr float kPScale = 256.0f;                       // probabilities are stored x 2^8
constexpr int kQPitch = kD + 8;                         // staging rows of the normalised queries
static_assert(kStepW * kPitchWin <= kBufBytes, "window step must fit a buffer");
static_assert(8 * kQPitch * 2 <= kBufBytes, "eight staged query rows must fit one buffer");

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Each wave owns its LDS: two step buffers that receive raw stored rows by
// direct global->LDS loads (one wave instruction per row, pitch padded by 16
// bytes), and its probability arrays.  No wave reads another wave's buffers,
// so the entry loop has no workgroup barrier.
struct __align__(16) WaveSmem {
  uint8_t buf[2][kBufBytes];
  uint8_t phi[16][kPPitch];        // fp8 high part of p * 2^8   [head][entry]
  uint8_t plo[16][kPPitch];        // fp8 residual
  uint16_t pbf[16][kPPitch];       // bf16(p * 2^8)
};
struct __align__(16) AttnSmem {
  WaveSmem wave[kWaves];
  float rope_cs[kR / 2][2];        // cos, sin of the query's RoPE angles
  float ml[kWaves][2][16];         // per wave: running max and sum of each head
};
static_assert(sizeof(AttnSmem) <= 160 * 1024, "LDS budget of one workgroup per CU");

__device__ __forceinline__ const lds_u8* lds_ptr(const uint8_t* p) {
  // the buffers live in LDS; a C-style cast changes the address space
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

// Combine a value with the same lane of the other 16-lane rows of its half
// (xor 16) and then of the other half (xor 32), in one fixed order.
__device__ __forceinline__ float row_max4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Per-query description of the attended list.  Wave w takes, in step s < ns,
// list positions [128 s + 16 w, +16) of the compressed entries, then in step
// ns + t window rows [64 t + 8 w, +8).  Rows are read through buffer
// descriptors over the query's own cache rows and window rows, so a row
// address is a scalar byte offset.
struct Work {
  int64_t p, N;
  int n_list, win_count, ns, n_steps, k;
  int ring_start, ring_n;          // window ring: first slot, slots (ring_n = 0: rows in order)
  buf_rsrc tbl_rs;                 // the query's block-table row
  int sh;                          // log2(rows per block)
  const int32_t* idx;              // this query's selected list (CSA) or nullptr
  buf_rsrc kv_rs, win_rs;
};

// The selected entries of a wave's first kTabSteps compressed steps, read
// in the prologue: register t, lane l holds step 4 t + l / 16, row l % 16
// (entry 0 where the slot is empty or invalid), and `valid` the matching
// ballot.  Later steps (lists longer than 1024) read theirs in the loop.
constexpr int kTabSteps = 8;
struct EntryTab {
  int e[kTabSteps / 4];
  uint64_t valid[kTabSteps / 4];
};

// Selected entry of list position pos, and whether it is a visible entry
// (paged: its pool row).  Without a selected list (HCA) position pos is
// entry pos.
template <bool PG>   // paged entries (the kernel instance for a block table)
__device__ __forceinline__ int list_entry(const Work& w, int pos, bool* ok) {
  // the load does not wait for the range test: its address is clamped
  const int e = w.idx != nullptr ? w.idx[pos < w.k ? pos : w.k - 1] : pos;
  *ok = pos < w.n_list && e >= 0 && e < w.N;
  const int el = *ok ? e : 0;
  if (!PG) return el;
  const int32_t blk = __builtin_amdgcn_raw_buffer_load_b32(w.tbl_rs, (el >> w.sh) * 4, 0, 0);
  return static_cast<int>((static_cast<uint32_t>(blk) << w.sh) | (static_cast<uint32_t>(el) & ((1u << w.sh) - 1u)));
}

// Direct buffer->LDS loads of one wave step into `dst`; returns the step's
// row-validity mask (bit r = row r holds a real entry).  Rows without an
// entry load entry 0, or read as zeros past the end of the query's rows, and
// stay masked.  A compressed step is 16 load instructions, a window step 8
// (the loop's wait counts rely on it).
template <bool PG>
__device__ __forceinline__ uint32_t issue_step(const Work& w, int step, int wv, const EntryTab& tab,
                                               uint8_t* dst) {
  const int lane = threadIdx.x & 63;
  typedef __attribute__((address_space(3))) void lds_void;
  if (step < w.ns) {
    const int pos0 = step * (kWaves * kStepE) + wv * kStepE;
    uint32_t vmask;
    int ereg = 0, base = 0;
    if (w.idx == nullptr && !PG) {
      const int nv = w.n_list - pos0;
      vmask = nv >= kStepE ? 0xffffu : (nv <= 0 ? 0u : (1u << nv) - 1u);
    } else if (step < kTabSteps) {
      ereg = tab.e[0];
      uint64_t vb = tab.valid[0];
#pragma unroll
      for (int t = 1; t < kTabSteps / 4; ++t)
        if ((step >> 2) == t) { ereg = tab.e[t]; vb = tab.valid[t]; }
      base = (step & 3) * 16;
      vmask = static_cast<uint32_t>(vb >> base) & 0xffffu;
    } else {
      bool ok = false;
      if (lane < kStepE) ereg = list_entry<PG>(w, pos0 + lane, &ok);
      vmask = static_cast<uint32_t>(__ballot(lane < kStepE && ok));
    }
    if (lane < kChunksSplit) {
      if (w.idx == nullptr && !PG) {
        // (an HCA row past the query's N entries reads as zeros: buffer range check)
#pragma unroll
        for (int r = 0; r < kStepE; ++r)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(w.kv_rs, (lds_void*)(lds_ptr(dst + r * kPitchSplit)),
                                                   16, lane * 16, (pos0 + r) * kRowSplit, 0, 0);
      } else {
#pragma unroll
        for (int r = 0; r < kStepE; ++r)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(w.kv_rs, (lds_void*)(lds_ptr(dst + r * kPitchSplit)),
                                                   16, lane * 16,
                                                   __builtin_amdgcn_readlane(ereg, base + r) * kRowSplit, 0, 0);
      }
    }
    return vmask;
  }
  const int j0 = (step - w.ns) * (kWaves * kStepW) + wv * kStepW;
  if (PG && w.ring_n > 0) {
    // ring: window row j sits in slot (ring_start + j) mod n_win; a row past
    // the window loads the first row again (finite data, masked: the ring's
    // other slots may hold anything)
#pragma unroll
    for (int r = 0; r < kStepW; ++r) {
      const int j = j0 + r < w.win_count ? j0 + r : 0;
      const int slot = w.ring_start + j >= w.ring_n ? w.ring_start + j - w.ring_n : w.ring_start + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w.win_rs, (lds_void*)(lds_ptr(dst + r * kPitchWin)), 16,
                                               lane * 16, slot * kRowBf16, 0, 0);
    }
  } else {
#pragma unroll
    for (int r = 0; r < kStepW; ++r)       // rows past the window read as zeros
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w.win_rs, (lds_void*)(lds_ptr(dst + r * kPitchWin)),
                                               16, lane * 16, (j0 + r) * kRowBf16, 0, 0);
  }
  const int nv = w.win_count - j0;
  return nv >= kStepW ? (1u << kStepW) - 1u : (nv <= 0 ? 0u : (1u << nv) - 1u);
}

// s_waitcnt immediate: at most n vector-memory operations outstanding (the
// other counters not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Online-softmax update of head j16 from this lane's 4 logits t (log2
// domain): returns alpha and writes the probabilities p = 2^(t - m_new).
__device__ __forceinline__ float softmax_step(const float (&t)[4], float (&pv)[4], float& m_run,
                                              float& l_run) {
  const float mx = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
  const float m_new = fmaxf(m_run, row_max4(mx));
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  float ps = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pv[r] = __builtin_amdgcn_exp2f(t[r] - m_new);
    ps += pv[r];
  }
  l_run = l_run * alpha + row_sum4(ps);
  m_run = m_new;
  return alpha;
}

// The entry loop of one wave.  NB output blocks of 16 dims starting at dbase,
// the first NF of them FP8 dims (the rest the BF16 RoPE dims).  A step holds
// 16 compressed entries (or 8 window rows); the MFMA tiles are 16 rows and 32
// (16) deep, so the second half of a tile multiplies probabilities set to zero
// by rows of the same step (finite data) -- it adds nothing.
template <int NB, int NF, bool PG>
__device__ __forceinline__ void entry_loop(const Work& w, WaveSmem& ws, int wv, const bf16x8 (&qb)[kD / 32],
                                           float ch, int dbase, float& m_run, float& l_run,
                                           f32x4 (&acc)[NB], const EntryTab& tab, uint32_t vmask_cur) {
  const int lane = threadIdx.x & 63, g = lane >> 4, j16 = lane & 15;
  for (int step = 0; step < w.n_steps; ++step) {
    const int bi = step & 1;
    // the next step's rows go out first (its buffer was read to the end by
    // the previous step), then the wait leaves exactly those loads in flight:
    // two steps of rows are in flight while a step computes
    uint32_t vmask_next = 0u;
    if (step + 1 < w.n_steps) {
      vmask_next = issue_step<PG>(w, step + 1, wv, tab, ws.buf[bi ^ 1]);
      if (step + 1 < w.ns) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kStepE));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(kStepW));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    const uint32_t vmask = vmask_cur;
    vmask_cur = vmask_next;
    const uint8_t* T = ws.buf[bi];
    float alpha;
    const bool split = step < w.ns;
    if (split) {
      // -------- logits of the step's 16 entries (rows) x 16 heads (cols).
      // Every operand read is issued before the math so the LDS latency
      // overlaps; two partial chains (even / odd k-steps) interleave.
      const uint8_t* rowp = T + j16 * kPitchSplit + g * 8;
      long ka[kDF8 / 32];
#pragma unroll
      for (int ks = 0; ks < kDF8 / 32; ++ks) ka[ks] = lds_read_b64(rowp + ks * 32);
      bf16x8 kr[kR / 32];
#pragma unroll
      for (int ks = 0; ks < kR / 32; ++ks)
        kr[ks] = *reinterpret_cast<const bf16x8*>(rowp + kDF8 + g * 8 + ks * 64);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 s2[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int ks = 0; ks < kDF8 / 32; ++ks)
        s2[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(ka[ks]), qb[ks], s2[ks & 1], 0, 0, 0);
#pragma unroll
      for (int ks = 0; ks < kR / 32; ++ks)
        s2[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks], qb[kDF8 / 32 + ks], s2[ks & 1], 0, 0, 0);
      const f32x4 s = s2[0] + s2[1];
      // lane holds head j16, entries 4 g + r
      float t[4], pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (vmask >> (g * 4 + r)) & 1u;
        t[r] = ok ? s[r] * ch : -INFINITY;
      }
      alpha = softmax_step(t, pv, m_run, l_run);
      // probabilities to this wave's LDS in the P^T operand layout [head][entry]
      const float v0 = pv[0] * kPScale, v1 = pv[1] * kPScale, v2 = pv[2] * kPScale, v3 = pv[3] * kPScale;
      if (NF > 0) {
        const uint32_t h01 = fp8x2(v0, v1), h23 = fp8x2(v2, v3);
        const f32x2 d01 = fp8x2_to_f32(h01), d23 = fp8x2_to_f32(h23);
        const uint32_t l01 = fp8x2(v0 - d01[0], v1 - d01[1]), l23 = fp8x2(v2 - d23[0], v3 - d23[1]);
        *reinterpret_cast<uint32_t*>(&ws.phi[j16][g * 4]) = h01 | (h23 << 16);
        *reinterpret_cast<uint32_t*>(&ws.plo[j16][g * 4]) = l01 | (l23 << 16);
      }
      if (NF < NB) {
        uint2 bb;
        bb.x = bf16x2_rne(v0, v1);
        bb.y = bf16x2_rne(v2, v3);
        *reinterpret_cast<uint2*>(&ws.pbf[j16][g * 4]) = bb;
      }
    } else {
      // -------- window step: 8 BF16 rows (tile rows 8..15 repeat them, masked)
      const uint8_t* rowp = T + (j16 & (kStepW - 1)) * kPitchWin + g * 16;
      bf16x8 kw[kD / 32];
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) kw[ks] = *reinterpret_cast<const bf16x8*>(rowp + ks * 64);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 s2[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks)
        s2[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kw[ks], qb[ks], s2[ks & 1], 0, 0, 0);
      const f32x4 s = s2[0] + s2[1];
      float t[4], pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (vmask >> (g * 4 + r)) & 1u;
        t[r] = ok ? s[r] * ch : -INFINITY;
      }
      alpha = softmax_step(t, pv, m_run, l_run);
      if (g < 2) {
        uint2 bb;
        bb.x = bf16x2_rne(pv[0] * kPScale, pv[1] * kPScale);
        bb.y = bf16x2_rne(pv[2] * kPScale, pv[3] * kPScale);
        *reinterpret_cast<uint2*>(&ws.pbf[j16][g * 4]) = bb;
      }
    }
    if (__ballot(alpha != 1.0f) != 0ull) {              // the running max moved for some head
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i] *= alpha;
    }
    __builtin_amdgcn_wave_barrier();
    if (split) {
      // -------- P.V: rows = dims, cols = heads, K = 32 entries of which 16 are
      // this step's (lane groups 0, 1) and 16 carry p = 0 (groups 2, 3)
      const int ebase = (g & 1) * 8;
      long phv = 0, plv = 0;
      bf16x8 pbv = {};
      if (g < 2) {
        if (NF > 0) {
          phv = lds_read_b64(&ws.phi[j16][ebase]);
          plv = lds_read_b64(&ws.plo[j16][ebase]);
        }
        if (NF < NB) pbv = *reinterpret_cast<const bf16x8*>(&ws.pbf[j16][ebase]);
      }
      // fp8 dims: lane j of group g supplies row (ebase + j/2), bytes d0 + 8*(j%2)
      const uint8_t* b8 = T + (ebase + (j16 >> 1)) * kPitchSplit + dbase + 8 * (j16 & 1);
      // bf16 RoPE dims: lane j supplies row (ebase + j/4) and row (ebase + 4 + j/4)
      const uint8_t* b16 = T + (ebase + (j16 >> 2)) * kPitchSplit + kDF8 +
                           (dbase + NF * 16 - kDF8) * 2 + 8 * (j16 & 3);
      long v8[NF > 0 ? NF : 1];
      bf16x8 v16[NB - NF > 0 ? NB - NF : 1];
#pragma unroll
      for (int i = 0; i < NF; ++i) v8[i] = tr8(b8 + i * 16);
#pragma unroll
      for (int i = 0; i < NB - NF; ++i) {
        const bf16x4 lo4 = tr16(b16 + i * 32);
        const bf16x4 hi4 = tr16(b16 + i * 32 + 4 * kPitchSplit);
        v16[i] = bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(v8[i], phv, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(v8[i], plv, acc[i], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NB - NF; ++i)
        acc[NF + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v16[i], pbv, acc[NF + i], 0, 0, 0);
    } else {
      // K = 16 rows: this step's 8 (lane groups 0, 1) and 8 with p = 0
      bf16x4 pbw = {};
      if (g < 2) pbw = *reinterpret_cast<const bf16x4*>(&ws.pbf[j16][g * 4]);
      // lane j of group g supplies row (4 (g % 2) + j/4), dims d0 + 4*(j%4)
      const uint8_t* b16 = T + ((g & 1) * 4 + (j16 >> 2)) * kPitchWin + dbase * 2 + 8 * (j16 & 3);
      bf16x4 vw[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) vw[i] = tr16(b16 + i * 32);
#pragma unroll
      for (int i = 0; i < NB; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vw[i], pbw, acc[i], 0, 0, 0);
    }
  }
}

// DVS = number of workgroups sharing one (query, 16-head tile): each owns
// 512 / DVS output dims; every wave of it accumulates all of them over its
// own entries, and the eight partial states are merged at the end in wave
// order.
// PG: the instance for paged caches (block table, ring window); the other
// instance carries none of that addressing.
template <int DVS, bool PG>
__global__ void __launch_bounds__(kThreads) attn_mfma_kernel(AttnArgs a, int n_units,
                                                             int n_pad) {
  constexpr int DWG = kD / DVS;        // output dims of this workgroup
  constexpr int NB = DWG / 16;         // 16-dim MFMA blocks
  // the last slice holds the BF16 RoPE dims: its first NFR blocks are FP8 dims
  constexpr int NFR = (kDF8 - (kD - DWG)) > 0 ? (kDF8 - (kD - DWG)) / 16 : 0;
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
  const int dbase = dvs * DWG;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j16 = lane & 15;
  WaveSmem& ws = sm.wave[wv];

  // ---------------- everything the prologue reads goes out at once: this
  // lane's part of the query (head 2 wv + lane / 32, dims [16 (lane % 32),
  // +16)), its RoPE frequency, the head's sink, the query's position, cache
  // offset and window, and the wave's selected entries (validated below)
  const int qh = wv * 2 + (lane >> 5), qc = lane & 31;
  uint4 qraw[2];
  {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                    (static_cast<int64_t>(b) * a.H + ht * 16 + qh) * kD + qc * 16);
    qraw[0] = q[0];
    qraw[1] = q[1];
  }
  const double theta = a.rope_theta[tid < kR / 2 ? tid : 0];
  const float sink = a.sinks[ht * 16 + j16];
  constexpr bool paged = PG;
  const int64_t p_ld = a.q_pos[b], kv0_ld = paged ? 0 : a.kv_off[b];
  const int wl_ld = a.win_mode == 1 ? a.win_len[b] : 0;
  const int ws_ld = PG && a.win_mode == 1 && a.win_start != nullptr ? a.win_start[b] : 0;
  const int64_t tp0_ld = a.win_mode == 2 ? a.tok_pos0[b] : 0, toff_ld = a.win_mode == 2 ? a.tok_off[b] : 0;
  const int32_t* idx_q = a.idx != nullptr ? a.idx + static_cast<int64_t>(b) * a.k : nullptr;
  int e_ld[kTabSteps / 4];
#pragma unroll
  for (int t = 0; t < kTabSteps / 4; ++t) {
    const int pos = (4 * t + (lane >> 4)) * (kWaves * kStepE) + wv * kStepE + (lane & 15);
    e_ld[t] = idx_q != nullptr ? idx_q[pos < a.k ? pos : a.k - 1] : pos;   // clamped address; HCA: the position
  }

  Work w;
  w.p = uniform64(p_ld);
  w.N = (w.p + 1) / a.m;
  const int64_t kv0 = uniform64(kv0_ld);
  int64_t win_row0;
  window_of(a, b, w.p, wl_ld, uniform64(tp0_ld), uniform64(toff_ld), &win_row0, &w.win_count);
  w.idx = idx_q;
  w.k = a.k;
  w.n_list = a.idx != nullptr ? (w.N > 0 ? a.k : 0) : static_cast<int>(w.N);
  w.ns = (w.n_list + kWaves * kStepE - 1) / (kWaves * kStepE);
  w.n_steps = w.ns + (w.win_count + kWaves * kStepW - 1) / (kWaves * kStepW);
  // paged: one descriptor over the pool (rows addressed by physical row)
  const uint64_t kv_bytes = static_cast<uint64_t>(paged ? a.pool_rows : w.N) * kRowSplit;
  w.kv_rs = make_rsrc(static_cast<const uint8_t*>(a.kv) + (paged ? 0 : kv0 * kRowSplit),
                      kv_bytes < 0xffffffffull ? static_cast<uint32_t>(kv_bytes) : 0xffffffffu);
  w.ring_n = PG && a.win_mode == 1 && a.win_start != nullptr && w.win_count > 0 ? a.n_win : 0;
  {
    const int ws = __builtin_amdgcn_readfirstlane(ws_ld);
    w.ring_start = ws < 0 ? 0 : (ws >= a.n_win ? 0 : ws);   // out-of-range starts read from slot 0
  }
  w.win_rs = make_rsrc(w.win_count > 0 ? static_cast<const uint8_t*>(a.win) + win_row0 * kRowBf16 : nullptr,
                       static_cast<uint32_t>(w.ring_n > 0 ? w.ring_n : w.win_count) * kRowBf16);
  w.sh = paged ? a.blk_shift : 0;
  w.tbl_rs = make_rsrc(paged ? a.blk_table + static_cast<int64_t>(b) * a.blk_stride : nullptr,
                       paged ? static_cast<uint32_t>(a.blk_stride * 4) : 0u);
  EntryTab tab;
#pragma unroll
  for (int t = 0; t < kTabSteps / 4; ++t) {
    const int step = 4 * t + (lane >> 4);
    const int pos = step * (kWaves * kStepE) + wv * kStepE + (lane & 15);
    const bool ok = (w.idx != nullptr || paged) && step < w.ns && pos < w.n_list && e_ld[t] >= 0 && e_ld[t] < w.N;
    tab.e[t] = ok ? e_ld[t] : 0;
    tab.valid[t] = __ballot(ok);
  }
  if (paged) {
    // logical entry -> pool row through the query's block table (one more
    // dependent round trip before the first rows go out); a slot without an
    // entry maps entry 0 and stays masked
    const int sh = w.sh;
    int32_t blk[kTabSteps / 4];
#pragma unroll
    for (int t = 0; t < kTabSteps / 4; ++t)
      blk[t] = __builtin_amdgcn_raw_buffer_load_b32(w.tbl_rs, (tab.e[t] >> sh) * 4, 0, 0);
#pragma unroll
    for (int t = 0; t < kTabSteps / 4; ++t)
      tab.e[t] = static_cast<int>((static_cast<uint32_t>(blk[t]) << sh) | (static_cast<uint32_t>(tab.e[t]) & ((1u << sh) - 1u)));
  }
  // the first step's rows go out before the query is prepared
  uint32_t vmask0 = 0u;
  if (w.n_steps > 0) vmask0 = issue_step<PG>(w, 0, wv, tab, ws.buf[0]);

  if (tid < kR / 2) {
    float sn, cs;
    rope_sincos(w.p, theta, &sn, &cs);
    sm.rope_cs[tid][0] = cs;
    sm.rope_cs[tid][1] = sn;
  }

  // ---------------- prologue: qhat = RoPE(RMSNorm(q)); wave w prepares heads
  // 2w, 2w+1 (lane: head 2w + lane/32, dims [16 (lane%32), +16)) into a bf16
  // staging copy (heads 0-7 in wave 0's second buffer, 8-15 in wave 1's: the
  // second buffers receive rows only once the loop starts), then every lane
  // takes its QK operand.  Rows are padded to 520 values so that the heads'
  // rows start on different banks.
  auto qrow = [&](int h) __attribute__((always_inline)) {
    return reinterpret_cast<uint16_t*>(&sm.wave[h >> 3].buf[1][0]) + (h & 7) * kQPitch;
  };
  {
    const int h = qh, c = qc;                           // head in tile, 16-dim chunk
    float x[16];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 v = qraw[i];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        x[i * 8 + 2 * t] = bf16_to_f32(static_cast<uint16_t>(u[t] & 0xffff));
        x[i * 8 + 2 * t + 1] = bf16_to_f32(static_cast<uint16_t>(u[t] >> 16));
      }
    }
    float ss = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) ss = fmaf(x[t], x[t], ss);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float r = static_cast<float>(1.0 / sqrt(static_cast<double>(ss) / kD + a.eps));
    if (a.q_norm_w != nullptr) {
      const float4* gw = reinterpret_cast<const float4*>(a.q_norm_w + c * 16);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 gv = gw[t];
        x[4 * t] *= r * gv.x; x[4 * t + 1] *= r * gv.y; x[4 * t + 2] *= r * gv.z; x[4 * t + 3] *= r * gv.w;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) x[t] *= r;
    }
    __syncthreads();                                    // rope_cs ready
    if (c * 16 >= kD - kR) {
      const int p0 = (c * 16 - (kD - kR)) / 2;
#pragma unroll
      for (int t = 0; t < 16; t += 2) {
        const float cs = sm.rope_cs[p0 + t / 2][0], sn = sm.rope_cs[p0 + t / 2][1];
        const float x0 = x[t], x1 = x[t + 1];
        x[t] = x0 * cs - x1 * sn;
        x[t + 1] = x0 * sn + x1 * cs;
      }
    }
#pragma unroll
    for (int t = 0; t < 16; t += 8) {
      uint4 v;
      v.x = bf16x2_rne(x[t], x[t + 1]);
      v.y = bf16x2_rne(x[t + 2], x[t + 3]);
      v.z = bf16x2_rne(x[t + 4], x[t + 5]);
      v.w = bf16x2_rne(x[t + 6], x[t + 7]);
      *reinterpret_cast<uint4*>(qrow(h) + c * 16 + t) = v;
    }
  }
  __syncthreads();
  // QK operand of this lane: head j16, dims [32*ks + 8*g, +8)
  bf16x8 qb[kD / 32];
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qrow(j16) + ks * 32 + g * 8);
  const float ch = a.scale * kLog2e;
  __syncthreads();                                      // the staging copy is free again

  // softmax state of head j16 (the same in the four lanes of that head); the
  // sink enters once, through wave 0
  float m_run = sink * kLog2e;
  float l_run = wv == 0 ? 1.0f : 0.0f;
  f32x4 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (dbase + DWG <= kDF8)
    entry_loop<NB, NB, PG>(w, ws, wv, qb, ch, dbase, m_run, l_run, acc, tab, vmask0);
  else
    entry_loop<NB, NFR, PG>(w, ws, wv, qb, ch, dbase, m_run, l_run, acc, tab, vmask0);

  // -------- merge the waves' states in wave order, then out = acc / (2^8 * l)
  __syncthreads();                                      // every wave is done with its buffers
  if (lane < 16) {
    sm.ml[wv][0][j16] = m_run;
    sm.ml[wv][1][j16] = l_run;
  }
  f32x4* part = reinterpret_cast<f32x4*>(&ws.buf[0][0]);   // [NB][64 lanes]
#pragma unroll
  for (int i = 0; i < NB; ++i) part[i * 64 + lane] = acc[i];
  __syncthreads();
  float f[kWaves];
  float mm = sm.ml[0][0][j16];
#pragma unroll
  for (int v = 1; v < kWaves; ++v) mm = fmaxf(mm, sm.ml[v][0][j16]);
  float L = 0.0f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    f[v] = __builtin_amdgcn_exp2f(sm.ml[v][0][j16] - mm);
    L += sm.ml[v][1][j16] * f[v];
  }
  const float inv = 1.0f / (L * kPScale);
  uint16_t* out = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(b) * a.H + ht * 16 + j16) * kD;
  // block i of the output is finished by wave i % kWaves
  for (int i = wv; i < NB; i += kWaves) {
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < kWaves; ++v)
      o += reinterpret_cast<const f32x4*>(&sm.wave[v].buf[0][0])[i * 64 + lane] * f[v];
    const int d = dbase + i * 16 + g * 4;
    uint2 st;
    st.x = static_cast<uint32_t>(f32_to_bf16(o[0] * inv)) | (static_cast<uint32_t>(f32_to_bf16(o[1] * inv)) << 16);
    st.y = static_cast<uint32_t>(f32_to_bf16(o[2] * inv)) | (static_cast<uint32_t>(f32_to_bf16(o[3] * inv)) << 16);
    *reinterpret_cast<uint2*>(out + d) = st;
  }
}

}  // namespace

// HIGH_OCC: two workgroups per (query, 16 heads), 256 output dims each;
// LOW_OCC: eight, 64 dims each; AUTO fills the chip: the fewest workgroups
// that still give every CU one.
int pick_dvs(int variant, int units, int cus) {
  if (variant == CSA_VARIANT_HIGH_OCC) return 2;
  if (variant == CSA_VARIANT_LOW_OCC) return 8;
  if (units * 2 >= cus) return 2;
  if (units * 4 >= cus) return 4;
  return 8;
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
    const void* fns[] = {reinterpret_cast<const void*>(&attn_mfma_kernel<2, false>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<4, false>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<8, false>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<2, true>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<4, true>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<8, true>)};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm));
      if (e != hipSuccess) return e;
    }
    attr_set_dev = dev;
  }
  const dim3 g(n_pad), blk(kThreads);
  if (a.blk_table != nullptr) {
    switch (dvs) {
      case 2: hipLaunchKernelGGL((attn_mfma_kernel<2, true>), g, blk, shm, stream, a, units, n_pad); break;
      case 4: hipLaunchKernelGGL((attn_mfma_kernel<4, true>), g, blk, shm, stream, a, units, n_pad); break;
      default: hipLaunchKernelGGL((attn_mfma_kernel<8, true>), g, blk, shm, stream, a, units, n_pad); break;
    }
  } else {
    switch (dvs) {
      case 2: hipLaunchKernelGGL((attn_mfma_kernel<2, false>), g, blk, shm, stream, a, units, n_pad); break;
      case 4: hipLaunchKernelGGL((attn_mfma_kernel<4, false>), g, blk, shm, stream, a, units, n_pad); break;
      default: hipLaunchKernelGGL((attn_mfma_kernel<8, false>), g, blk, shm, stream, a, units, n_pad); break;
    }
  }
  return hipGetLastError();
}

size_t attn_mfma_smem_bytes() { return sizeof(AttnSmem); }

}  // namespace csa
