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
//    softmax state (log2 domain, from an empty state); there is no workgroup
//    barrier in the entry loop.  At the end the eight waves' states are
//    merged in wave order and the sink joins the denominator.  Logits use BF16 MFMA on the exactly widened
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
  // online softmax over the entries from an empty state; the sink joins the
  // denominator at the end, so a large or -inf sink neither underflows the
  // probabilities nor makes -inf - -inf
  float mx = -INFINITY, l = 0.0f;
  float acc[P];
#pragma unroll
  for (int t = 0; t < P; ++t) acc[t] = 0.0f;
  auto step = [&](const float* e) {
    float dot = 0.0f;
#pragma unroll
    for (int t = 0; t < P; ++t) dot = fmaf(qh[t], e[lane * P + t], dot);
    dot = wave_sum(dot) * a.scale;
    const float mn = fmaxf(mx, dot);
    const float mu = mn == -INFINITY ? 0.0f : mn;
    const float al = expf(mx - mu), pj = expf(dot - mu);
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
  // out = acc / (l + e^{z - mx}), written so that neither term overflows
  const float z = a.sinks[h];
  const float mu = mx == -INFINITY ? 0.0f : mx;
  float inv;
  if (z <= mu) {
    inv = 1.0f / (l + expf(z - mu));
  } else {
    const float s = expf(mu - z);
    inv = s / (l * s + 1.0f);
  }
  if (!(l > 0.0f)) inv = 0.0f;                 // nothing attended: an empty sum
  float* o = static_cast<float*>(a.out) + (static_cast<int64_t>(b) * a.H + h) * D;
#pragma unroll
  for (int t = 0; t < P; ++t) o[lane * P + t] = acc[t] * inv;
}

// ================================================================== MFMA path
constexpr int kD = 512, kR = 64, kDF8 = 448;            // dims, RoPE dims, FP8 dims
constexpr int kRowSplit = kDF8 + 2 * kR;                // 576 bytes per cache entry
constexpr int kRowBf16 = 2 * kD;                        // 1024 bytes per window row
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;                   // one wave per SIMD
constexpr int kStepE = 16;                              // rows per step (an MFMA tile)
constexpr int kWinLoad = 8;                             // window rows per load (two loads per step)
constexpr int kSlots = 4;                               // per-wave ring of row slots
// A slot holds one load, chunk-major (16-byte chunks): chunk c of cache row r
// (c < 36, r < 16) at cache_chunk(c) + 16 r, chunk c of window row r (c < 64,
// r < 8) at win_chunk(c) + 16 r.  Each 1 KB of a slot is one load
// instruction of 64 lanes x 16 bytes; a window load takes a ninth, spare one.
constexpr int kSlotBytes = 9 * 1024;
constexpr int kLoadInsts = 9;                           // load instructions per slot load
constexpr int kPPitch = 20;                             // padded rows of the P arrays
constexpr float kTau = 2.0f;                            // a head's reference max moves once exceeded by this (log2)
constexpr float kPScale = 64.0f;                        // probabilities (<= 2^kTau) are stored x 2^6
constexpr int kQF8Pitch = kD + 16;                      // staging rows of the scaled query (FP8 parts)
constexpr int kQBfPitch = kD + 8;                       // staging rows of the scaled query (BF16 parts)
constexpr int kTabSteps = 16;                           // compressed steps whose entries the prologue reads
static_assert(16 * kQF8Pitch <= kSlotBytes, "the FP8 query parts of 16 heads must fit a slot");
static_assert(8 * kQBfPitch * 2 <= kSlotBytes, "the BF16 query parts of 8 heads must fit a slot");

// Each wave owns its LDS: a ring of four row slots that receive raw stored
// rows by direct global->LDS loads, and its probability arrays.  No wave
// reads another wave's slots inside the entry loop, so the loop has no
// workgroup barrier.
struct __align__(16) WaveSmem {
  uint8_t slot[kSlots][kSlotBytes];
  uint8_t phi[16][kPPitch];        // FP8 high part of p * 2^6    [head][entry]
  uint8_t plo[16][kPPitch];        // FP8 residual
  uint16_t pbh[16][kPPitch];       // BF16 high part of p * 2^6
  uint16_t pbl[16][kPPitch];       // BF16 residual
  int tab[kTabSteps * kStepE];     // row of (step, row) for the first kTabSteps steps, -1: none
};
struct __align__(16) AttnSmem {
  WaveSmem wave[kWaves];
  float rope_cs[kR / 2][2];        // cos, sin of the query's RoPE angles
  float ml[kWaves][2][16];         // per wave: reference max and sum of each head
  float qsc[16];                   // per head: 2^-e, the inverse of the query's FP8 scale
};
static_assert(sizeof(AttnSmem) <= 160 * 1024, "LDS budget of one workgroup per CU");

__host__ __device__ constexpr int cache_chunk(int c) { return (c >> 2) * 1024 + (c & 3) * 256; }
__host__ __device__ constexpr int win_chunk(int c) { return (c >> 3) * 1024 + (c & 7) * 128; }

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ const lds_u8* lds_ptr(const uint8_t* p) {
  // the buffers live in LDS; a C-style cast changes the address space
  return (const lds_u8*)(p);
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr(p))));
}

// s_waitcnt immediate: at most n vector-memory operations outstanding (the
// other counters not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// A raw buffer descriptor in four scalar registers: base, num_records bytes
// (a load at or past it reads 0 and touches no memory), the flags of
// make_rsrc.
__device__ __forceinline__ i32x4 make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a))),
               static_cast<int>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu)),
               static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000};
}

// Instruction Q of a slot load: a direct buffer->LDS load of 16 bytes per
// lane.  The instruction's immediate offset moves both the source and the LDS
// destination, so with m0 = lds + (1024 - G) Q and offset G Q, lane i's 16
// bytes at voff + G Q land at lds + 1024 Q + 16 i.  Written as assembly so
// that the compiler does not treat the in-flight row loads as pending LDS
// writes and drain them before every LDS access of the loop: the loop waits
// for its own loads with explicit vmcnt waits (wait_loads), each followed by
// a compiler memory barrier.  The instruction has no register result.
template <int Q, int G>
__device__ __forceinline__ void dma_inst(const i32x4& d, uint32_t lds, uint32_t voff) {
  asm volatile("s_add_u32 m0, %0, %3\n\tbuffer_load_dwordx4 %1, %2, 0 offen offset:%4 lds"
               :
               : "s"(lds), "v"(voff), "s"(d), "n"((1024 - G) * Q), "n"(G * Q)
               : "memory");
}
template <int G>
__device__ __forceinline__ void dma_load(const i32x4& d, uint32_t lds, uint32_t voff) {
  dma_inst<0, G>(d, lds, voff); dma_inst<1, G>(d, lds, voff); dma_inst<2, G>(d, lds, voff);
  dma_inst<3, G>(d, lds, voff); dma_inst<4, G>(d, lds, voff); dma_inst<5, G>(d, lds, voff);
  dma_inst<6, G>(d, lds, voff); dma_inst<7, G>(d, lds, voff); dma_inst<8, G>(d, lds, voff);
}

// Wait until at most `loads` slot loads are still in flight.
__device__ __forceinline__ void wait_loads(int loads) {
  if (loads >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadInsts));
  else if (loads == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadInsts));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");                        // no LDS access moves above the wait
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
// 32 bytes of LDS as the 8-register operand of the 16x16x128 FP8 MFMA
__device__ __forceinline__ i32x8 lds_read_b256(const uint8_t* p) {
  const i32x4 a = *reinterpret_cast<const i32x4*>(p);
  const i32x4 b = *reinterpret_cast<const i32x4*>(p + 16);
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// the same from two 16-byte pieces
__device__ __forceinline__ i32x8 lds_read_2x16(const uint8_t* p0, const uint8_t* p1) {
  const i32x4 a = *reinterpret_cast<const i32x4*>(p0);
  const i32x4 b = *reinterpret_cast<const i32x4*>(p1);
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// 16x16x128 MFMA on E4M3 operands with unit block scales (E8M0 127 = 2^0)
__device__ __forceinline__ f32x4 mfma_fp8_k128(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
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
// list positions [64 s + 16 w, +16) of the compressed entries, then in window
// step t the window rows [64 t + 16 w, +16), loaded as two halves of 8 rows.
// A step's rows come through loads: load L < ns is compressed step L, load
// ns + 2 t + h is half h of window step t; load L lands in slot L mod 4.
struct Work {
  int64_t p, N;
  int n_list, win_count, ns, nw, n_loads, k;
  int ring_start, ring_n;          // window ring: first slot, slots (ring_n = 0: rows in order)
  buf_rsrc tbl_rs;                 // the query's block-table row
  int sh;                          // log2(rows per block)
  const int32_t* idx;              // this query's selected list (CSA) or nullptr
  i32x4 kv_d, win_d;               // descriptors over the query's cache rows (or the pool) and window
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

// Load L into the slot at LDS address `lds`; returns its row-validity mask
// (bit r = row r holds a real entry).  Rows without an entry load entry 0, or
// read as zeros past the end of the query's rows, and stay masked.
// The rows of a wave's first kTabSteps compressed steps (the entry, or the
// pool row when paged) sit in the wave's LDS table, written by the prologue;
// a slot without an entry holds ~row of entry 0 (finite data, masked: a free
// pool row may hold anything).  Later steps map theirs here.
template <bool PG>
__device__ __forceinline__ uint32_t issue_load(const Work& w, int L, int wv, const int* tab, uint32_t lds) {
  const int lane = threadIdx.x & 63;
  if (L < w.ns) {
    // lane l: row l % 16, chunks 4 q + l / 16 of instruction q
    const int pos0 = L * (kWaves * kStepE) + wv * kStepE;
    const int r = lane & 15;
    uint32_t vmask;
    int row;
    if (w.idx == nullptr && !PG) {
      const int nv = w.n_list - pos0;
      vmask = nv >= kStepE ? 0xffffu : (nv <= 0 ? 0u : (1u << nv) - 1u);
      row = pos0 + r;                                   // (a row past N reads as zeros)
    } else if (L < kTabSteps) {
      const int e = tab[L * kStepE + r];
      row = e < 0 ? ~e : e;
      vmask = static_cast<uint32_t>(__ballot(lane < kStepE && e >= 0));
    } else {
      bool ok = false;
      row = list_entry<PG>(w, pos0 + r, &ok);
      vmask = static_cast<uint32_t>(__ballot(lane < kStepE && ok));
    }
    dma_load<64>(w.kv_d, lds, static_cast<uint32_t>(row) * kRowSplit + 16u * static_cast<uint32_t>(lane >> 4));
    return vmask;
  }
  // window load: step wl / 2, half wl % 2; lane l: row l % 8, chunks 8 q + l / 8
  const int wl = L - w.ns;
  const int j0 = (wl >> 1) * (kWaves * kStepE) + wv * kStepE + (wl & 1) * kWinLoad;
  int row = j0 + (lane & 7);
  if (PG && w.ring_n > 0) {
    // window row j sits in slot (ring_start + j) mod n_win; a row past the
    // window loads the first row again (finite data, masked: the ring's other
    // slots may hold anything)
    const int j = row < w.win_count ? row : 0;
    row = w.ring_start + j >= w.ring_n ? w.ring_start + j - w.ring_n : w.ring_start + j;
  }
  // (rows past the window in the in-order layout read as zeros; the ninth
  // instruction fills the slot's spare kilobyte)
  dma_load<128>(w.win_d, lds, static_cast<uint32_t>(row) * kRowBf16 + 16u * static_cast<uint32_t>(lane >> 3));
  const int nv = w.win_count - j0;
  return nv >= kWinLoad ? (1u << kWinLoad) - 1u : (nv <= 0 ? 0u : (1u << nv) - 1u);
}

// Online-softmax update of head j16 from this lane's 4 logits t (log2
// domain), against a reference max m_ref that moves only when a logit
// exceeds it by more than kTau (so p = 2^(t - m_ref) <= 2^kTau, and the
// accumulators are rescaled a few times per query instead of at every new
// maximum).  Returns alpha (1 when the reference stays) and writes p.
__device__ __forceinline__ float softmax_step(const float (&t)[4], float (&pv)[4], float& m_ref,
                                              float& l_run) {
  const float mx = row_max4(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
  // (a head with no finite logit yet keeps the reference -inf; p is then
  // taken against 0, and every masked logit gives 0)
  const bool move = mx > m_ref + kTau;
  const float m_new = move ? mx : m_ref;
  const float m_use = m_new == -INFINITY ? 0.0f : m_new;
  const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - m_use) : 1.0f;
  float ps = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pv[r] = __builtin_amdgcn_exp2f(t[r] - m_use);
    ps += pv[r];
  }
  l_run = l_run * alpha + row_sum4(ps);
  m_ref = m_new;
  return alpha;
}

// The query operands of one lane (head j16, lane group g), the query scaled
// by 2^e_h (e_h per head, so that the FP8 parts stay normal and below 448):
//   f8[0..2]  FP8 high part, dims [128 ks + 32 g, +32)      (B of QK, ks < 3)
//   f8[3..5]  FP8 residual, same dims
//   f8[6]     dims [384 + 32 (g % 2), +32): high part for g < 2, residual for g >= 2
//   bh[ks], bl[ks]  BF16 high part and residual, dims [32 ks + 8 g, +8)
struct QOps {
  i32x8 f8[7];
  bf16x8 bh[kD / 32], bl[kD / 32];
};

// Per-lane LDS offsets of a slot's operand reads (precomputed once).
struct LaneOff {
  int qk, qk3, rope;     // cache QK: chunks 8 ks + 2 g (ks < 3), 24 + 2 (g % 2), RoPE chunk 28 + g
  int pv8, pv16;         // cache P.V: FP8 dims (tr8) from the slice's first chunk, RoPE dims (tr16)
  int wqk, wpv;          // window QK (row j16 % 8, chunk g) and P.V (tr16) within a slot
};

// ---------------------------------------------------------------- one step's parts
// Logits of a cache step in slot T (16 rows x 16 heads; lane: head j16, rows
// 4 g + r): FP8 dims on the 16x16x128 FP8 MFMA against the query's FP8 high
// part and residual, RoPE dims on BF16 MFMA against its BF16 high part and
// residual.
__device__ __forceinline__ f32x4 qk_cache(const uint8_t* T, const LaneOff& lo, const QOps& q) {
  i32x8 ka[4];
#pragma unroll
  for (int ks = 0; ks < 3; ++ks) ka[ks] = lds_read_2x16(T + lo.qk + 2048 * ks, T + lo.qk + 2048 * ks + 256);
  ka[3] = lds_read_2x16(T + lo.qk3 + 6144, T + lo.qk3 + 6144 + 256);
  bf16x8 kr[kR / 32];
#pragma unroll
  for (int ks = 0; ks < kR / 32; ++ks) kr[ks] = *reinterpret_cast<const bf16x8*>(T + lo.rope + 7168 + 1024 * ks);
  f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 3; ++ks) {
    s0 = mfma_fp8_k128(ka[ks], q.f8[ks], s0);
    s1 = mfma_fp8_k128(ka[ks], q.f8[3 + ks], s1);
  }
  s0 = mfma_fp8_k128(ka[3], q.f8[6], s0);
#pragma unroll
  for (int ks = 0; ks < kR / 32; ++ks) {
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks], q.bh[kDF8 / 32 + ks], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks], q.bl[kDF8 / 32 + ks], s0, 0, 0, 0);
  }
  return s0 + s1;
}

// Logits of a window step: 16 BF16 rows, rows 0-7 in slot X and 8-15 in slot
// Y (wq: this lane's row offset inside its slot), on BF16 MFMA against the
// query's BF16 high part and residual.  Lane (row j16, g) supplies dims
// [32 ks + 8 g, +8) = chunk 4 ks + g.
__device__ __forceinline__ f32x4 qk_window(const uint8_t* TX, const uint8_t* TY, const LaneOff& lo, const QOps& q) {
  const int j16 = threadIdx.x & 15;
  const uint8_t* rowp = (j16 < kWinLoad ? TX : TY) + lo.wqk;
  bf16x8 kw[kD / 32];
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks)
    kw[ks] = *reinterpret_cast<const bf16x8*>(rowp + (ks >> 1) * 1024 + (ks & 1) * 512);
  f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kw[ks], q.bh[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kw[ks], q.bl[ks], s1, 0, 0, 0);
  }
  return s0 + s1;
}

// Softmax of a step's logits (masked by vmask), then its probabilities to
// this wave's LDS in the P^T operand layout [head][entry]: FP8 high part and
// residual (cache steps with FP8 output dims), BF16 high part and residual
// (cache steps with RoPE output dims, and window steps).  Returns alpha.
template <bool FP8P, bool BFP>
__device__ __forceinline__ float soft_step(const f32x4& s, uint32_t vmask, float ch, WaveSmem& ws, float& m_ref,
                                           float& l_run) {
  const int lane = threadIdx.x & 63, g = lane >> 4, j16 = lane & 15;
  float t[4], pv[4];
  const uint32_t bits = vmask >> (g * 4);
#pragma unroll
  for (int r = 0; r < 4; ++r) t[r] = ((bits >> r) & 1u) ? s[r] * ch : -INFINITY;
  const float alpha = softmax_step(t, pv, m_ref, l_run);
  const float v0 = pv[0] * kPScale, v1 = pv[1] * kPScale, v2 = pv[2] * kPScale, v3 = pv[3] * kPScale;
  if (FP8P) {
    const uint32_t h01 = fp8x2(v0, v1), h23 = fp8x2(v2, v3);
    const f32x2 d01 = fp8x2_to_f32(h01), d23 = fp8x2_to_f32(h23);
    const uint32_t l01 = fp8x2(v0 - d01[0], v1 - d01[1]), l23 = fp8x2(v2 - d23[0], v3 - d23[1]);
    *reinterpret_cast<uint32_t*>(&ws.phi[j16][g * 4]) = h01 | (h23 << 16);
    *reinterpret_cast<uint32_t*>(&ws.plo[j16][g * 4]) = l01 | (l23 << 16);
  }
  if (BFP) {
    const bf16x2 a01 = {static_cast<__bf16>(v0), static_cast<__bf16>(v1)};
    const bf16x2 a23 = {static_cast<__bf16>(v2), static_cast<__bf16>(v3)};
    uint2 hb, lb;
    hb.x = __builtin_bit_cast(uint32_t, a01);
    hb.y = __builtin_bit_cast(uint32_t, a23);
    lb.x = bf16x2_rne(v0 - static_cast<float>(a01[0]), v1 - static_cast<float>(a01[1]));
    lb.y = bf16x2_rne(v2 - static_cast<float>(a23[0]), v3 - static_cast<float>(a23[1]));
    *reinterpret_cast<uint2*>(&ws.pbh[j16][g * 4]) = hb;
    *reinterpret_cast<uint2*>(&ws.pbl[j16][g * 4]) = lb;
  }
  return alpha;
}

// P.V of a cache step in slot T into NB output blocks of 16 dims, the first
// NF of them FP8 dims (the rest the BF16 RoPE dims): rows = dims, cols =
// heads; K = 32: lane group g supplies K [8 g, +8), the step's rows
// 8 (g % 2) .. +8 for every g; groups 0-1 carry the high part of p, groups
// 2-3 its residual.
template <int NB, int NF>
__device__ __forceinline__ void pv_cache(const uint8_t* T, const LaneOff& lo, const WaveSmem& ws,
                                         f32x4 (&acc)[NB]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, j16 = lane & 15;
  const int eb = (g & 1) * 8;
  long pf = 0;
  bf16x8 pb = {};
  if (NF > 0) pf = lds_read_b64(g < 2 ? &ws.phi[j16][eb] : &ws.plo[j16][eb]);
  if (NF < NB) pb = *reinterpret_cast<const bf16x8*>(g < 2 ? &ws.pbh[j16][eb] : &ws.pbl[j16][eb]);
  // FP8 block i: chunk c0 + i (c0 a multiple of 4), lane j of group g reads
  // row eb + j / 2, bytes 8 (j % 2) of it (tr8: column j of the 8 x 16 block)
  constexpr int kChunk = 8;
#pragma unroll
  for (int c0 = 0; c0 < NF; c0 += kChunk) {
    long v8[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      if (c0 + i < NF) v8[i] = tr8(T + lo.pv8 + ((c0 + i) >> 2) * 1024 + ((c0 + i) & 3) * 256);
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      if (c0 + i < NF) acc[c0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(v8[i], pf, acc[c0 + i], 0, 0, 0);
  }
  // RoPE block i (dims 448 + 16 i, chunks 28 + 2 i and 29 + 2 i): rows
  // eb + j / 4 and eb + 4 + j / 4 (tr16: column j of a 4 x 16 block)
  bf16x8 v16[NB - NF > 0 ? NB - NF : 1];
#pragma unroll
  for (int i = 0; i < NB - NF; ++i) {
    const uint8_t* p = T + lo.pv16 + 7168 + (i >> 1) * 1024 + (i & 1) * 512;
    const bf16x4 lo4 = tr16(p);
    const bf16x4 hi4 = tr16(p + 64);
    v16[i] = bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  }
#pragma unroll
  for (int i = 0; i < NB - NF; ++i)
    acc[NF + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v16[i], pb, acc[NF + i], 0, 0, 0);
}

// P.V of a window step (16 BF16 rows: 0-7 in slot X, 8-15 in slot Y), the
// same K layout as a cache step: group g takes rows 0-7 of slot X (even g)
// or Y (odd g), high part of p for g < 2, residual for g >= 2.
template <int NB>
__device__ __forceinline__ void pv_window(const uint8_t* TX, const uint8_t* TY, const LaneOff& lo,
                                          const WaveSmem& ws, f32x4 (&acc)[NB]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, j16 = lane & 15;
  const int eb = (g & 1) * 8;
  const bf16x8 pb = *reinterpret_cast<const bf16x8*>(g < 2 ? &ws.pbh[j16][eb] : &ws.pbl[j16][eb]);
  const uint8_t* base = ((g & 1) ? TY : TX) + lo.wpv;
  constexpr int kChunk = 8;
#pragma unroll
  for (int c0 = 0; c0 < NB; c0 += kChunk) {
    bf16x8 vw[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      if (c0 + i < NB) {
        const uint8_t* p = base + ((c0 + i) >> 2) * 1024 + ((c0 + i) & 3) * 256;
        const bf16x4 lo4 = tr16(p);
        const bf16x4 hi4 = tr16(p + 64);
        vw[i] = bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      if (c0 + i < NB) acc[c0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vw[i], pb, acc[c0 + i], 0, 0, 0);
  }
}

// Multiply the accumulators by alpha when some head's reference max moved
// (rare); the branch stays a branch.
template <int NB>
__device__ __forceinline__ void rescale(f32x4 (&acc)[NB], float alpha) {
  if (__ballot(alpha != 1.0f) != 0ull) {
    float a = alpha;
    asm volatile("" : "+v"(a));                         // the products cannot move above the branch
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[i] *= a;
  }
}

// The row-validity masks of the four slots' current loads.
struct SlotMasks {
  uint32_t m0, m1, m2, m3;
  __device__ __forceinline__ uint32_t get(int s) const {
    return s == 0 ? m0 : (s == 1 ? m1 : (s == 2 ? m2 : m3));
  }
  __device__ __forceinline__ void set(int s, uint32_t v) {
    m0 = s == 0 ? v : m0;
    m1 = s == 1 ? v : m1;
    m2 = s == 2 ? v : m2;
    m3 = s == 3 ? v : m3;
  }
};

// Cache step st in slot S: first the load of step st + 3 goes into slot
// S + 3 (its last reader, step st - 1, is done) and the wait leaves at most
// that load and the one before it in flight; then the P.V of step st
// together with the logits of step st + 1 (slot S + 1), then the softmax of
// step st + 1, whose probabilities overwrite the ones step st's P.V has read
// (the wave's LDS accesses stay in program order).
template <int S, int NB, int NF, bool PG>
__device__ __forceinline__ void cache_iter(const Work& w, WaveSmem& ws, const QOps& q, const int* tab,
                                           const LaneOff& lo, f32x4 (&acc)[NB], float ch, float& m_ref,
                                           float& l_run, int wv, uint32_t sl, SlotMasks& vm, int st) {
  constexpr int S1 = (S + 1) & 3, S3 = (S + 3) & 3;
  if (st + 3 < w.n_loads) vm.set(S3, issue_load<PG>(w, st + 3, wv, tab, sl + S3 * kSlotBytes));
  const bool next = st + 1 < w.ns;
  if (next) {
    const int issued = st + 4 < w.n_loads ? st + 4 : w.n_loads;
    wait_loads(issued - (st + 2));
  }
  pv_cache<NB, NF>(ws.slot[S], lo, ws, acc);
  if (next) {
    const f32x4 s = qk_cache(ws.slot[S1], lo, q);
    rescale<NB>(acc, soft_step<(NF > 0), (NF < NB)>(s, vm.get(S1), ch, ws, m_ref, l_run));
  }
  __builtin_amdgcn_wave_barrier();
}

// The entry loop of one wave: the cache steps software-pipelined through
// the ring (unrolled by its four slots, so slot addresses are constants),
// then the window steps (a few per wave) one after another.
template <int NB, int NF, bool PG>
__device__ __forceinline__ void entry_loop(const Work& w, WaveSmem& ws, const QOps& q, const int* tab,
                                           const LaneOff& lo, f32x4 (&acc)[NB], float ch, float& m_ref,
                                           float& l_run, int wv, uint32_t sl, SlotMasks& vm, int issued) {
  if (w.ns + w.nw == 0) return;
  if (w.ns > 0) {
    wait_loads(issued - 1);
    const f32x4 s = qk_cache(ws.slot[0], lo, q);
    rescale<NB>(acc, soft_step<(NF > 0), (NF < NB)>(s, vm.m0, ch, ws, m_ref, l_run));
    __builtin_amdgcn_wave_barrier();
    for (int st = 0; st < w.ns; st += 4) {
      cache_iter<0, NB, NF, PG>(w, ws, q, tab, lo, acc, ch, m_ref, l_run, wv, sl, vm, st);
      if (st + 1 < w.ns) cache_iter<1, NB, NF, PG>(w, ws, q, tab, lo, acc, ch, m_ref, l_run, wv, sl, vm, st + 1);
      if (st + 2 < w.ns) cache_iter<2, NB, NF, PG>(w, ws, q, tab, lo, acc, ch, m_ref, l_run, wv, sl, vm, st + 2);
      if (st + 3 < w.ns) cache_iter<3, NB, NF, PG>(w, ws, q, tab, lo, acc, ch, m_ref, l_run, wv, sl, vm, st + 3);
    }
    issued = w.ns + 3 < w.n_loads ? w.ns + 3 : w.n_loads;
  }
  for (int t = 0; t < w.nw; ++t) {
    const int L0 = w.ns + 2 * t;
    while (issued < w.n_loads && issued < L0 + kSlots) {
      vm.set(issued & 3, issue_load<PG>(w, issued, wv, tab, sl + (issued & 3) * kSlotBytes));
      ++issued;
    }
    wait_loads(issued - (L0 + 2));
    const uint8_t* TX = ws.slot[0] + (L0 & 3) * kSlotBytes;
    const uint8_t* TY = ws.slot[0] + ((L0 + 1) & 3) * kSlotBytes;
    const f32x4 s = qk_window(TX, TY, lo, q);
    rescale<NB>(acc, soft_step<false, true>(s, vm.get(L0 & 3) | (vm.get((L0 + 1) & 3) << kWinLoad), ch, ws,
                                            m_ref, l_run));
    __builtin_amdgcn_wave_barrier();
    pv_window<NB>(TX, TY, lo, ws, acc);
    __builtin_amdgcn_wave_barrier();
  }
}

// DVS = number of workgroups sharing one (query, 16-head tile) (1, 2 or 4):
// each owns 512 / DVS output dims; every wave of it accumulates all of them over its
// own entries, and the four partial states are merged at the end in wave
// order.
// PG: the instance for paged caches (block table, ring window); the other
// instance carries none of that addressing.
template <int DVS, bool PG>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_mfma_kernel(AttnArgs a, int n_units, int n_pad) {
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
  const uint32_t sl = lds_addr(ws.slot[0]);

  // ---------------- everything the prologue reads goes out at once: this
  // lane's part of the query (head 4 wv + lane / 16, dims [32 (lane % 16),
  // +32)), its RoPE frequency, the head's sink, the query's position, cache
  // offset and window, and the wave's selected entries (validated below)
  const int qh = wv * 4 + (lane >> 4), qc = lane & 15;
  uint4 qraw[4];
  {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                    (static_cast<int64_t>(b) * a.H + ht * 16 + qh) * kD + qc * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) qraw[i] = q[i];
  }
  const double theta = a.rope_theta[tid < kR / 2 ? tid : 0];
  const float sink = a.sinks[ht * 16 + j16];
  constexpr bool paged = PG;
  const int64_t p_ld = a.q_pos[b], kv0_ld = paged ? 0 : a.kv_off[b];
  const int wl_ld = a.win_mode == 1 ? a.win_len[b] : 0;
  const int ws_ld = PG && a.win_mode == 1 && a.win_start != nullptr ? a.win_start[b] : 0;
  const int64_t tp0_ld = a.win_mode == 2 ? a.tok_pos0[b] : 0, toff_ld = a.win_mode == 2 ? a.tok_off[b] : 0;
  const int32_t* idx_q = a.idx != nullptr ? a.idx + static_cast<int64_t>(b) * a.k : nullptr;
  const int32_t trow_ld = PG && a.blk_row != nullptr ? a.blk_row[b] : b;
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
  w.nw = (w.win_count + kWaves * kStepE - 1) / (kWaves * kStepE);
  w.n_loads = w.ns + 2 * w.nw;
  // paged: one descriptor over the pool (rows addressed by physical row)
  const uint64_t kv_bytes = static_cast<uint64_t>(paged ? a.pool_rows : w.N) * kRowSplit;
  w.kv_d = make_desc(static_cast<const uint8_t*>(a.kv) + (paged ? 0 : kv0 * kRowSplit),
                     kv_bytes < 0xffffffffull ? static_cast<uint32_t>(kv_bytes) : 0xffffffffu);
  w.ring_n = PG && a.win_mode == 1 && a.win_start != nullptr && w.win_count > 0 ? a.n_win : 0;
  {
    const int wsr = __builtin_amdgcn_readfirstlane(ws_ld);
    w.ring_start = wsr < 0 ? 0 : (wsr >= a.n_win ? 0 : wsr);   // out-of-range starts read from slot 0
  }
  w.win_d = make_desc(w.win_count > 0 ? static_cast<const uint8_t*>(a.win) + win_row0 * kRowBf16 : nullptr,
                      static_cast<uint32_t>(w.ring_n > 0 ? w.ring_n : w.win_count) * kRowBf16);
  w.sh = paged ? a.blk_shift : 0;
  {
    // the query's block-table row (clamped: an out-of-range row reads row 0 or the last)
    int64_t tr = __builtin_amdgcn_readfirstlane(trow_ld);
    tr = tr < 0 ? 0 : (tr >= a.blk_rows ? a.blk_rows - 1 : tr);
    w.tbl_rs = make_rsrc(paged ? a.blk_table + tr * a.blk_stride : nullptr,
                         paged ? static_cast<uint32_t>(a.blk_stride * 4) : 0u);
  }
  // the wave's rows of its first kTabSteps steps (lane l: step 4 t + l / 16,
  // row l % 16) to its LDS table; paged: logical entry -> pool row through
  // the query's block table (one more dependent round trip before the first
  // rows go out)
  {
    int e[kTabSteps / 4];
    bool valid[kTabSteps / 4];
#pragma unroll
    for (int t = 0; t < kTabSteps / 4; ++t) {
      const int step = 4 * t + (lane >> 4);
      const int pos = step * (kWaves * kStepE) + wv * kStepE + (lane & 15);
      const bool ok = (w.idx != nullptr || paged) && step < w.ns && pos < w.n_list && e_ld[t] >= 0 && e_ld[t] < w.N;
      e[t] = ok ? e_ld[t] : 0;                          // no entry: entry 0's row, masked
      valid[t] = ok;
    }
    if (paged) {
      const int sh = w.sh;
      int32_t blk[kTabSteps / 4];
#pragma unroll
      for (int t = 0; t < kTabSteps / 4; ++t)
        blk[t] = __builtin_amdgcn_raw_buffer_load_b32(w.tbl_rs, (e[t] >> sh) * 4, 0, 0);
#pragma unroll
      for (int t = 0; t < kTabSteps / 4; ++t)
        e[t] = static_cast<int>((static_cast<uint32_t>(blk[t]) << sh) | (static_cast<uint32_t>(e[t]) & ((1u << sh) - 1u)));
    }
#pragma unroll
    for (int t = 0; t < kTabSteps / 4; ++t) ws.tab[64 * t + lane] = valid[t] ? e[t] : ~e[t];
  }
  // the first two loads go out before the query is prepared (slots 2 and 3
  // hold the query staging until the operands are taken)
  uint32_t vm0 = 0u, vm1 = 0u, vm2 = 0u;
  if (w.n_loads > 0) vm0 = issue_load<PG>(w, 0, wv, ws.tab, sl);
  if (w.n_loads > 1) vm1 = issue_load<PG>(w, 1, wv, ws.tab, sl + kSlotBytes);

  if (tid < kR / 2) {
    float sn, cs;
    rope_sincos(w.p, theta, &sn, &cs);
    sm.rope_cs[tid][0] = cs;
    sm.rope_cs[tid][1] = sn;
  }

  // ---------------- prologue: qhat = RoPE(RMSNorm(q)), scaled by 2^e_h;
  // wave w prepares heads 4w .. 4w+3 (lane: head 4w + lane/16, dims [32
  // (lane%16), +32)) and writes the scaled query's FP8 high part and
  // residual (dims < 448) and its BF16 high part and residual (all dims) to
  // staging rows in slots 2 and 3 of waves 0-2; then every lane takes its
  // QK operands.
  uint8_t* const qf8h = sm.wave[0].slot[2];                 // [16][kQF8Pitch]
  uint8_t* const qf8l = sm.wave[0].slot[3];
  auto qbf = [&](int part, int h) __attribute__((always_inline)) {   // part 0: high, 1: residual
    return reinterpret_cast<uint16_t*>(sm.wave[1 + part].slot[2 + (h >> 3)]) + (h & 7) * kQBfPitch;
  };
  {
    const int h = qh, c = qc;                           // head in tile, 32-dim chunk
    float x[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
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
    for (int t = 0; t < 32; ++t) ss = fmaf(x[t], x[t], ss);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float r = static_cast<float>(1.0 / sqrt(static_cast<double>(ss) / kD + a.eps));
    if (a.q_norm_w != nullptr) {
      const float4* gw = reinterpret_cast<const float4*>(a.q_norm_w + c * 32);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float4 gv = gw[t];
        x[4 * t] *= r * gv.x; x[4 * t + 1] *= r * gv.y; x[4 * t + 2] *= r * gv.z; x[4 * t + 3] *= r * gv.w;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 32; ++t) x[t] *= r;
    }
    __syncthreads();                                    // rope_cs ready
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
    // the head's scale 2^e: its largest |value| times 2^e in [128, 256), so
    // the FP8 parts stay normal and unsaturated (0 for an all-zero head)
    float am = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t) am = fmaxf(am, fabsf(x[t]));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    int e = 0;
    if (am > 0.0f) {
      int ea;
      (void)frexpf(am, &ea);                            // am in [2^(ea-1), 2^ea)
      e = 8 - ea;                                       // am * 2^e in [128, 256)
      e = e > 60 ? 60 : (e < -60 ? -60 : e);
    }
    if (c == 0) sm.qsc[h] = ldexpf(1.0f, -e);
#pragma unroll
    for (int t = 0; t < 32; ++t) x[t] = ldexpf(x[t], e);
    if (c * 32 < kDF8) {
#pragma unroll
      for (int t = 0; t < 32; t += 8) {
        uint2 hv, lv;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t hh = fp8x2(x[t + 2 * u], x[t + 2 * u + 1]);
          const f32x2 d = fp8x2_to_f32(hh);
          hw[u] = hh;
          lw[u] = fp8x2(x[t + 2 * u] - d[0], x[t + 2 * u + 1] - d[1]);
        }
        hv.x = hw[0] | (hw[1] << 16); hv.y = hw[2] | (hw[3] << 16);
        lv.x = lw[0] | (lw[1] << 16); lv.y = lw[2] | (lw[3] << 16);
        *reinterpret_cast<uint2*>(qf8h + h * kQF8Pitch + c * 32 + t) = hv;
        *reinterpret_cast<uint2*>(qf8l + h * kQF8Pitch + c * 32 + t) = lv;
      }
    }
#pragma unroll
    for (int t = 0; t < 32; t += 8) {
      uint4 hv, lv;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x2 hh = {static_cast<__bf16>(x[t + 2 * u]), static_cast<__bf16>(x[t + 2 * u + 1])};
        hw[u] = __builtin_bit_cast(uint32_t, hh);
        lw[u] = bf16x2_rne(x[t + 2 * u] - static_cast<float>(hh[0]), x[t + 2 * u + 1] - static_cast<float>(hh[1]));
      }
      hv = uint4{hw[0], hw[1], hw[2], hw[3]};
      lv = uint4{lw[0], lw[1], lw[2], lw[3]};
      *reinterpret_cast<uint4*>(qbf(0, h) + c * 32 + t) = hv;
      *reinterpret_cast<uint4*>(qbf(1, h) + c * 32 + t) = lv;
    }
  }
  __syncthreads();
  // QK operands of this lane: head j16
  QOps qo;
#pragma unroll
  for (int ks = 0; ks < 3; ++ks) {
    qo.f8[ks] = lds_read_b256(qf8h + j16 * kQF8Pitch + 128 * ks + 32 * g);
    qo.f8[3 + ks] = lds_read_b256(qf8l + j16 * kQF8Pitch + 128 * ks + 32 * g);
  }
  qo.f8[6] = lds_read_b256((g < 2 ? qf8h : qf8l) + j16 * kQF8Pitch + 384 + 32 * (g & 1));
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks) {
    qo.bh[ks] = *reinterpret_cast<const bf16x8*>(qbf(0, j16) + 32 * ks + 8 * g);
    qo.bl[ks] = *reinterpret_cast<const bf16x8*>(qbf(1, j16) + 32 * ks + 8 * g);
  }
  const float ch = a.scale * kLog2e * sm.qsc[j16];
  __syncthreads();                                      // the staging slots are free again
  if (w.n_loads > 2) vm2 = issue_load<PG>(w, 2, wv, ws.tab, sl + 2 * kSlotBytes);
  const int issued = w.n_loads < 3 ? w.n_loads : 3;

  // per-lane LDS offsets of the operand reads within a slot
  LaneOff lo;
  {
    const int eb = (g & 1) * 8, h = (j16 >> 1) & 1;
    lo.qk = (g >> 1) * 1024 + (g & 1) * 512 + 16 * j16;
    lo.qk3 = (g & 1) * 512 + 16 * j16;
    lo.rope = g * 256 + 16 * j16;
    lo.pv8 = (dbase >> 6) * 1024 + (eb + (j16 >> 1)) * 16 + 8 * (j16 & 1);
    lo.pv16 = h * 256 + (eb + (j16 >> 2)) * 16 + 8 * (j16 & 1);
    lo.wqk = g * 128 + 16 * (j16 & 7);
    lo.wpv = (dbase >> 6) * 1024 + h * 128 + (j16 >> 2) * 16 + 8 * (j16 & 1);
  }

  // softmax state of head j16 (the same in the four lanes of that head), from
  // an empty state; the sink joins the denominator after the merge
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x4 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  SlotMasks vm{vm0, vm1, vm2, 0u};
  if (dbase + DWG <= kDF8)
    entry_loop<NB, NB, PG>(w, ws, qo, ws.tab, lo, acc, ch, m_run, l_run, wv, sl, vm, issued);
  else
    entry_loop<NB, NFR, PG>(w, ws, qo, ws.tab, lo, acc, ch, m_run, l_run, wv, sl, vm, issued);

  // -------- merge the waves' states in wave order, then out = acc / (2^6 (L + sink))
  __syncthreads();                                      // every wave is done with its slots
  if (lane < 16) {
    sm.ml[wv][0][j16] = m_run;
    sm.ml[wv][1][j16] = l_run;
  }
  // the partial accumulators of block i sit in the slots of the wave that
  // owns block i % kWaves... each wave writes its own blocks into its own slots
  f32x4* part = reinterpret_cast<f32x4*>(&ws.slot[0][0]);   // [NB][64 lanes], NB * 1 KB <= 4 slots
  static_assert(NB * 64 * 16 <= kSlots * kSlotBytes, "partial accumulators must fit a wave's slots");
#pragma unroll
  for (int i = 0; i < NB; ++i) part[i * 64 + lane] = acc[i];
  __syncthreads();
  float f[kWaves];
  float mm = sm.ml[0][0][j16];
#pragma unroll
  for (int v = 1; v < kWaves; ++v) mm = fmaxf(mm, sm.ml[v][0][j16]);
  const float mu = mm == -INFINITY ? 0.0f : mm;
  float L = 0.0f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    f[v] = __builtin_amdgcn_exp2f(sm.ml[v][0][j16] - mu);
    L += sm.ml[v][1][j16] * f[v];
  }
  // out = acc / (2^6 (L + 2^(zs - mu))), zs the sink in the log2 domain,
  // written so that neither term overflows
  const float zs = sink * kLog2e;
  float inv;
  if (zs <= mu) {
    inv = 1.0f / ((L + __builtin_amdgcn_exp2f(zs - mu)) * kPScale);
  } else {
    const float s = __builtin_amdgcn_exp2f(mu - zs);
    inv = s / ((L * s + 1.0f) * kPScale);
  }
  if (!(L > 0.0f)) inv = 0.0f;                          // nothing attended: an empty sum
  uint16_t* out = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(b) * a.H + ht * 16 + j16) * kD;
  // block i of the output is finished by wave i % kWaves
  for (int i = wv; i < NB; i += kWaves) {
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < kWaves; ++v)
      o += reinterpret_cast<const f32x4*>(&sm.wave[v].slot[0][0])[i * 64 + lane] * f[v];
    const int d = dbase + i * 16 + g * 4;
    uint2 st;
    st.x = static_cast<uint32_t>(f32_to_bf16(o[0] * inv)) | (static_cast<uint32_t>(f32_to_bf16(o[1] * inv)) << 16);
    st.y = static_cast<uint32_t>(f32_to_bf16(o[2] * inv)) | (static_cast<uint32_t>(f32_to_bf16(o[3] * inv)) << 16);
    *reinterpret_cast<uint2*>(out + d) = st;
  }
}

}  // namespace

// FULL_DIMS: one workgroup per (query, 16 heads), all 512 output dims;
// HIGH_OCC: two, 256 dims each; LOW_OCC: four, 128 dims each.  AUTO: the
// fewest workgroups that still give every CU one (every workgroup of a head
// tile computes the tile's logits, so fewer workgroups repeat less of that
// work and pay fewer prologues) -- but one per tile only when the queries'
// row counts are bounded (a selected list: at most k + n_win rows) or the
// batch has four tiles per CU: with all-entry lists of very different
// lengths the longest query's workgroups set the time, and splitting its
// output dims over two workgroups halves their P.V work.
int pick_dvs(int variant, int units, int cus, bool bounded_rows) {
  if (variant == CSA_VARIANT_FULL_DIMS) return 1;
  if (variant == CSA_VARIANT_HIGH_OCC) return 2;
  if (variant == CSA_VARIANT_LOW_OCC) return 4;
  if (units >= cus && (bounded_rows || units >= 4 * cus)) return 1;
  if (units * 2 >= cus) return 2;
  return 4;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  const bool f32 = a.q_fmt == CSA_F32;
  if (f32) {
    const int units = a.nq * a.H;
    const dim3 grid((units + 3) / 4);
    log_launch("attention: fp32 path, %d queries x %d heads, D %d, grid %u x 256 threads", a.nq, a.H, a.D, grid.x);
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
  const int variant = env_variant(a.variant);
  const int dvs = pick_dvs(variant, base_units, device_cu_count(), a.idx != nullptr);
  const int units = base_units * dvs;
  const int n_pad = (units + 7) / 8 * 8;
  const size_t shm = sizeof(AttnSmem);
  log_launch("attention: MFMA path%s, %d queries x %d heads, variant %s (%s), %d output-dim slices, "
             "grid %d x 256 threads (%d padding), LDS %zu B",
             a.blk_table != nullptr ? " (paged)" : "", a.nq, a.H,
             dvs == 1 ? "FULL_DIMS" : (dvs == 2 ? "HIGH_OCC" : "LOW_OCC"),
             a.variant != CSA_VARIANT_AUTO ? "requested" : (variant != CSA_VARIANT_AUTO ? "CSA_VARIANT" : "auto"),
             dvs, n_pad,
             n_pad - units, shm);
  // the workgroup needs more than the default 64 KB of dynamic LDS
  static thread_local int attr_set_dev = -1;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (attr_set_dev != dev) {
    const void* fns[] = {reinterpret_cast<const void*>(&attn_mfma_kernel<1, false>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<1, true>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<2, false>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<4, false>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<2, true>),
                         reinterpret_cast<const void*>(&attn_mfma_kernel<4, true>)};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm));
      if (e != hipSuccess) return e;
    }
    attr_set_dev = dev;
  }
  const dim3 g(n_pad), blk(kThreads);
  if (a.blk_table != nullptr) {
    switch (dvs) {
      case 1: hipLaunchKernelGGL((attn_mfma_kernel<1, true>), g, blk, shm, stream, a, units, n_pad); break;
      case 2: hipLaunchKernelGGL((attn_mfma_kernel<2, true>), g, blk, shm, stream, a, units, n_pad); break;
      default: hipLaunchKernelGGL((attn_mfma_kernel<4, true>), g, blk, shm, stream, a, units, n_pad); break;
    }
  } else {
    switch (dvs) {
      case 1: hipLaunchKernelGGL((attn_mfma_kernel<1, false>), g, blk, shm, stream, a, units, n_pad); break;
      case 2: hipLaunchKernelGGL((attn_mfma_kernel<2, false>), g, blk, shm, stream, a, units, n_pad); break;
      default: hipLaunchKernelGGL((attn_mfma_kernel<4, false>), g, blk, shm, stream, a, units, n_pad); break;
    }
  }
  return hipGetLastError();
}

size_t attn_mfma_smem_bytes() { return sizeof(AttnSmem); }

}  // namespace csa
