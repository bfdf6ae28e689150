// Device side of the token-level compressor, shared by the compress kernels
// and by the launch that compresses a decode step's entries next to the
// indexer scores.  The arithmetic is described in compress.hip.
#pragma once

#include "kernels.hpp"

namespace csa {
namespace cmp {

constexpr int kThreads = 256;
constexpr int kMaxSegParallel = kThreads;   // segments tested in parallel

__device__ __forceinline__ float load_x(const void* x, csa_fmt fmt, int64_t i) {
  return fmt == CSA_F32 ? static_cast<const float*>(x)[i]
                        : bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

struct EntrySlot {
  int64_t row;
  int64_t pos;
  int seg;
  int ok;
};

// Segment of the block starting at token t0, its output row and position.
// ok = 0 for a block that straddles a segment boundary.  Ends with a barrier.
__device__ __forceinline__ void locate(const CompressArgs& a, int64_t t0, EntrySlot* slot) {
  const int tid = threadIdx.x;
  const int m = a.m, nseg = a.nseg;
  if (nseg <= kMaxSegParallel) {
    if (tid == 0) slot->ok = 0;
    __syncthreads();
    if (tid < nseg) {
      const int64_t lo = a.seg_tok_off[tid], hi = a.seg_tok_off[tid + 1];
      const int64_t p0 = a.seg_pos0[tid], r0 = a.seg_out_row[tid];
      if (lo <= t0 && t0 < hi && (t0 - lo) % m == 0 && t0 + m <= hi) {
        const int64_t j = (t0 - lo) / m;
        slot->row = r0 + j;
        slot->pos = p0 + j * m;
        slot->seg = tid;
        slot->ok = 1;
      }
    }
  } else if (tid == 0) {
    // the last s with seg_tok_off[s] <= t0
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.seg_tok_off[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    const int64_t off = a.seg_tok_off[lo];
    const int ok = (t0 - off) % m == 0 && t0 + m <= a.seg_tok_off[lo + 1];
    const int64_t j = (t0 - off) / m;
    slot->row = a.seg_out_row[lo] + j;
    slot->pos = a.seg_pos0[lo] + j * m;
    slot->seg = lo;
    slot->ok = ok;
  }
  __syncthreads();
}

// Softmax-gated block sum of channel c (tokens t0 .. t0+m-1 in order).
// xv / gv hold the values already loaded, or nullptr to read them here.
__device__ __forceinline__ float gated_sum(int m, const float* xv, const float* gv) {
  float gmax = -INFINITY;
  for (int t = 0; t < m; ++t) gmax = fmaxf(gmax, gv[t]);
  float den = 0.0f, acc = 0.0f;
  for (int t = 0; t < m; ++t) {
    const float e = expf(gv[t] - gmax);
    den += e;
    acc = fmaf(e, xv[t], acc);
  }
  return acc / den;
}

// Normalise, rotate and store the entry held in y[0 .. D); sq is this
// thread's partial sum of squares.
__device__ __forceinline__ void finish_entry(const CompressArgs& a, float* y, float* red, float sq,
                                             const EntrySlot& slot) {
  const int tid = threadIdx.x;
  const int D = a.D, R = a.rope_dim;
  if (a.normalize) {
    sq = wave_sum(sq);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = sq;
    __syncthreads();
    float tot = 0.0f;
    for (int w = 0; w < kThreads / kWave; ++w) tot += red[w];
    const float r = static_cast<float>(1.0 / sqrt(static_cast<double>(tot) / D + a.eps));
    for (int c = tid; c < D; c += kThreads)
      y[c] = y[c] * r * (a.norm_w ? a.norm_w[c] : 1.0f);
  }
  __syncthreads();
  if (R > 0) {
    for (int i = tid; i < R / 2; i += kThreads) {
      float sn, cs;
      rope_sincos(slot.pos, a.rope_theta[i], &sn, &cs);
      const int d = D - R + 2 * i;
      const float u = y[d], v = y[d + 1];
      y[d] = u * cs - v * sn;
      y[d + 1] = u * sn + v * cs;
    }
    __syncthreads();
  }
  // quantised store
  const size_t rb = row_bytes(a.out_fmt, D, R);
  uint8_t* dst = static_cast<uint8_t*>(a.out) + slot.row * rb;
  switch (a.out_fmt) {
    case CSA_F32:
      for (int c = tid; c < D; c += kThreads) reinterpret_cast<float*>(dst)[c] = y[c];
      break;
    case CSA_BF16:
      for (int c = tid; c < D; c += kThreads) reinterpret_cast<uint16_t*>(dst)[c] = f32_to_bf16(y[c]);
      break;
    case CSA_FP8:
      for (int c = tid; c < D; c += kThreads) dst[c] = static_cast<uint8_t>(f32_to_e4m3(y[c]));
      break;
    case CSA_SPLIT:
      for (int c = tid; c < D; c += kThreads) {
        if (c < D - R) dst[c] = static_cast<uint8_t>(f32_to_e4m3(y[c]));
        else reinterpret_cast<uint16_t*>(dst + (D - R))[c - (D - R)] = f32_to_bf16(y[c]);
      }
      break;
    case CSA_MXFP4:
      for (int b = tid; b < D / 32; b += kThreads) {
        float amax = 0.0f;
        for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(y[b * 32 + e]));
        uint32_t sbyte = 0;
        int shared = 0;
        if (amax > 0.0f) {
          int ex;
          frexpf(amax, &ex);
          shared = ex - 1 - 2;
          shared = shared < -127 ? -127 : (shared > 127 ? 127 : shared);
          sbyte = static_cast<uint32_t>(shared + 127);
        }
        for (int e = 0; e < 32; e += 2) {
          uint32_t c0 = 0, c1 = 0;
          if (amax > 0.0f) {
            c0 = f32_to_e2m1(ldexpf(y[b * 32 + e], -shared));
            c1 = f32_to_e2m1(ldexpf(y[b * 32 + e + 1], -shared));
          }
          dst[(b * 32 + e) / 2] = static_cast<uint8_t>(c0 | (c1 << 4));
        }
        dst[D / 2 + b] = static_cast<uint8_t>(sbyte);
      }
      break;
    default:
      break;
  }
  __syncthreads();
}

// One block of M tokens, D <= 256 * NCH: the block's values are loaded into
// registers before the segment lookup, so both share one round trip.
template <int M, int NCH>
__device__ __forceinline__ void block_small(const CompressArgs& a, int64_t blk, float* y, float* red,
                                            EntrySlot* slot) {
  const int tid = threadIdx.x, D = a.D;
  const bool per_channel = a.gate_cols != 1;
  const int64_t t0 = blk * M;
  float xv[NCH][M], gv[NCH][M];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * kThreads;
    const int cc = c < D ? c : 0;
    const int gc = per_channel ? cc : 0;
#pragma unroll
    for (int t = 0; t < M; ++t) {
      xv[i][t] = load_x(a.x, a.x_fmt, (t0 + t) * D + cc);
      gv[i][t] = a.gate[(t0 + t) * a.gate_cols + gc];
    }
  }
  locate(a, t0, slot);
  if (!slot->ok) return;
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * kThreads;
    if (c < D) {
      const float v = gated_sum(M, xv[i], gv[i]);
      y[c] = v;
      sq = fmaf(v, v, sq);
    }
  }
  finish_entry(a, y, red, sq, *slot);
}

// One block, any m and D: values are read inside the block loop.  With one
// gate logit per token, m <= 256 (HCA's m' = 128) and rows that split into
// 16-byte chunks (8 BF16 or 4 F32 channels, 16-byte aligned) over at most 256 threads, the
// block's weights exp(g_t - max) are computed once per token into LDS, and
// the threads split as (token group, chunk): thread (g, k) sums chunk k over
// the tokens t = g, g + G, g + 2G, ... in order, all its loads in flight at
// once (for D = 512 BF16: 4 groups of 32 tokens, the whole 128 KB block in one
// round trip).  The G partial sums are added into LDS in group order, and the
// weights' sum runs over the tokens in order, so the bits are fixed.
constexpr int kMaxChunkTokens = 32;                    // tokens per thread in that path

__device__ __forceinline__ void block_any(const CompressArgs& a, int64_t blk, float* y, float* red,
                                          EntrySlot* slot) {
  const int tid = threadIdx.x, D = a.D, m = a.m;
  const int64_t t0 = blk * m;
  locate(a, t0, slot);
  if (!slot->ok) return;
  float sq = 0.0f;
  const int per16 = a.x_fmt == CSA_F32 ? 4 : 8;          // channels per 16-byte chunk
  const int chunks = D % per16 == 0 ? D / per16 : 0;
  const int groups = chunks > 0 && chunks <= kThreads && kThreads % chunks == 0 ? kThreads / chunks : 0;
  if (a.gate_cols == 1 && m <= kThreads && groups > 0 && (m + groups - 1) / groups <= kMaxChunkTokens &&
      (reinterpret_cast<uintptr_t>(a.x) & 15u) == 0) {
    __shared__ float e_sh[kThreads];
    float gm = -INFINITY;
    if (tid < m) gm = a.gate[t0 + tid];
    gm = wave_max(gm);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = gm;
    __syncthreads();
    float gmax = red[0];
    for (int w = 1; w < kThreads / kWave; ++w) gmax = fmaxf(gmax, red[w]);
    if (tid < m) e_sh[tid] = expf(a.gate[t0 + tid] - gmax);
    __syncthreads();                                   // e_sh ready; red free again
    float den = 0.0f;
    for (int t = 0; t < m; ++t) den += e_sh[t];
    const int grp = tid / chunks, k = tid % chunks;
    const int nt = grp < m ? (m - grp + groups - 1) / groups : 0;   // tokens of this thread
    const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.x) +
                                                      (t0 * D) * (a.x_fmt == CSA_F32 ? 4 : 2)) + k;
    const int64_t row16 = D / per16;                   // 16-byte chunks per token row
    uint4 raw[kMaxChunkTokens];
#pragma unroll
    for (int u = 0; u < kMaxChunkTokens; ++u)
      if (u < nt) raw[u] = xr[(grp + static_cast<int64_t>(u) * groups) * row16];
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kMaxChunkTokens; ++u) {
      if (u < nt) {
        const float e = e_sh[grp + u * groups];
        const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
        if (per16 == 8) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[2 * j] = fmaf(e, bf16_to_f32(static_cast<uint16_t>(w4[j] & 0xffffu)), acc[2 * j]);
            acc[2 * j + 1] = fmaf(e, bf16_to_f32(static_cast<uint16_t>(w4[j] >> 16)), acc[2 * j + 1]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] = fmaf(e, __uint_as_float(w4[j]), acc[j]);
        }
      }
    }
    // the groups' partial sums, added into y in group order
    for (int gg = 0; gg < groups; ++gg) {
      if (grp == gg) {
        for (int j = 0; j < per16; ++j) y[k * per16 + j] = gg == 0 ? acc[j] : y[k * per16 + j] + acc[j];
      }
      __syncthreads();
    }
    for (int c = tid; c < D; c += kThreads) {
      const float v = y[c] / den;
      y[c] = v;
      sq = fmaf(v, v, sq);
    }
    finish_entry(a, y, red, sq, *slot);
    return;
  }
  for (int c = tid; c < D; c += kThreads) {
    const int gc = a.gate_cols == 1 ? 0 : c;
    float gmax = -INFINITY;
    for (int t = 0; t < m; ++t) gmax = fmaxf(gmax, a.gate[(t0 + t) * a.gate_cols + gc]);
    float den = 0.0f, acc = 0.0f;
    for (int t = 0; t < m; ++t) {
      const float e = expf(a.gate[(t0 + t) * a.gate_cols + gc] - gmax);
      den += e;
      acc = fmaf(e, load_x(a.x, a.x_fmt, (t0 + t) * D + c), acc);
    }
    const float v = acc / den;
    y[c] = v;
    sq = fmaf(v, v, sq);
  }
  finish_entry(a, y, red, sq, *slot);
}

// Block shapes with a register-resident body; kAny covers the rest.
enum BlockKind { kM4C1, kM4C2, kM1C1, kM1C2, kM1C4, kAny };

// kWithAny = false leaves the general-m body out (its token-group path holds
// 32 16-byte loads in registers, which would lower every block shape's
// occupancy); launches whose jobs include a general-m block use true.
template <bool kWithAny = true>
__device__ __forceinline__ void run_block(const CompressArgs& a, int kind, int64_t blk, float* y,
                                          float* red, EntrySlot* slot) {
  switch (kind) {
    case kM4C1: block_small<4, 1>(a, blk, y, red, slot); break;
    case kM4C2: block_small<4, 2>(a, blk, y, red, slot); break;
    case kM1C1: block_small<1, 1>(a, blk, y, red, slot); break;
    case kM1C2: block_small<1, 2>(a, blk, y, red, slot); break;
    case kM1C4: block_small<1, 4>(a, blk, y, red, slot); break;
    default:
      if (kWithAny) block_any(a, blk, y, red, slot);
      break;
  }
}

inline int block_kind(const CompressArgs& a) {
  const int nch = (a.D + kThreads - 1) / kThreads;
  if (a.m == 4 && nch == 1) return kM4C1;
  if (a.m == 4 && nch == 2) return kM4C2;
  if (a.m == 1 && nch == 1) return kM1C1;
  if (a.m == 1 && nch == 2) return kM1C2;
  if (a.m == 1 && nch <= 4) return kM1C4;
  return kAny;
}

inline size_t shm_bytes(int D) { return (static_cast<size_t>(D) + kThreads / kWave) * sizeof(float); }

}  // namespace cmp
}  // namespace csa
