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
// wave owns 16-key blocks, loads them straight from global memory into the
// MFMA operand registers and keeps the query in registers.
//  * FP8 keys: the products must be exact for the top-k to be reproducible,
//    and FP8 MFMA accumulation is not, so FP8 values are widened to BF16
//    (exact) and multiplied on BF16 MFMA with fp32 accumulation.
//  * MXFP4 keys: scaled FP4 MFMA (E2M1 x E2M1 with per-32 E8M0 scales), whose
//    result is exact for these operands.
//  * F32: plain fp32 FMAs in dim order.
// The dims of one 128-dim vector are assigned to k-steps so that each lane
// reads 32 contiguous bytes; the same permutation is applied to queries and
// keys, so each dot product is the same sum.  The head sum runs per lane over
// head blocks in order, then over the 16 lanes of a row group in a fixed
// butterfly.
#include "kernels.hpp"

namespace csa {

namespace {

constexpr int kKeysPerWave = 64;                 // 4 blocks of 16 keys
constexpr int kWaves = 4;
constexpr int kKeysPerWg = kKeysPerWave * kWaves;

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

// --------------------------------------------------------------- FP8, d = 128
template <int NHB>   // head blocks of 16
__global__ void __launch_bounds__(256) indexer_fp8_kernel(IndexerArgs a, int64_t n_items,
                                                          int64_t n_chunk) {
  constexpr int H = NHB * 16;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, j16 = lane & 15;
  const uint8_t* keys = static_cast<const uint8_t*>(a.keys);
  const uint8_t* qall = static_cast<const uint8_t*>(a.q);
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int i = static_cast<int>(item / n_chunk);
    const int64_t chunk = item % n_chunk;
    int64_t N = (a.q_pos[i] + 1) / a.m;
    if (N > a.ld) N = a.ld;
    const int64_t s0 = chunk * kKeysPerWg + wv * kKeysPerWave;
    if (chunk * kKeysPerWg >= N) continue;            // uniform over the workgroup
    if (s0 >= N) continue;                            // uniform over the wave (no barriers below)
    // query operand: head hb*16 + j16, dims [32g, 32g+32) as 4 k-steps of 8
    bf16x8 qb[NHB][4];
    float wh[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int h = hb * 16 + j16;
      const uint4* qp = reinterpret_cast<const uint4*>(qall + (static_cast<int64_t>(i) * H + h) * 128 + g * 32);
      const uint4 v0 = qp[0], v1 = qp[1];
      qb[hb][0] = fp8x8_to_bf16(v0.x, v0.y);
      qb[hb][1] = fp8x8_to_bf16(v0.z, v0.w);
      qb[hb][2] = fp8x8_to_bf16(v1.x, v1.y);
      qb[hb][3] = fp8x8_to_bf16(v1.z, v1.w);
      wh[hb] = a.w[static_cast<int64_t>(i) * H + h];
    }
    const int64_t kbase = a.key_off[i];
    uint4 kr[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int64_t s = s0 + kb * 16 + j16;
      if (s < N) {
        const uint4* kp = reinterpret_cast<const uint4*>(keys + (kbase + s) * 128 + g * 32);
        kr[kb][0] = kp[0];
        kr[kb][1] = kp[1];
      } else {
        kr[kb][0] = make_uint4(0, 0, 0, 0);
        kr[kb][1] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int64_t sb = s0 + kb * 16;
      if (sb >= N) break;
      const bf16x8 k0 = fp8x8_to_bf16(kr[kb][0].x, kr[kb][0].y);
      const bf16x8 k1 = fp8x8_to_bf16(kr[kb][0].z, kr[kb][0].w);
      const bf16x8 k2 = fp8x8_to_bf16(kr[kb][1].x, kr[kb][1].y);
      const bf16x8 k3 = fp8x8_to_bf16(kr[kb][1].z, kr[kb][1].w);
      float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        // rows = keys (A), cols = heads (B): lane holds head j16, keys 4g..4g+3
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb[hb][0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb[hb][1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k2, qb[hb][2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k3, qb[hb][3], c, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) part[r] = fmaf(wh[hb], fmaxf(c[r], 0.0f), part[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) part[r] += __shfl_xor(part[r], o, 64);
      }
      if (j16 < 4) {
        const int64_t s = sb + g * 4 + j16;
        const float v = j16 == 0 ? part[0] : j16 == 1 ? part[1] : j16 == 2 ? part[2] : part[3];
        if (s < N) a.scores[static_cast<int64_t>(i) * a.ld + s] = v;
      }
    }
  }
}

// --------------------------------------------------------------- MXFP4, d = 128
// Row: 64 bytes of E2M1 codes then 4 E8M0 scales.  Scaled MFMA 16x16x128:
// lane (row j16, k-block g) supplies 16 code bytes and the scale of block g.
template <int NHB>
__global__ void __launch_bounds__(256) indexer_mxfp4_kernel(IndexerArgs a, int64_t n_items,
                                                            int64_t n_chunk) {
  constexpr int H = NHB * 16;
  constexpr int RB = 68;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, j16 = lane & 15;
  const uint8_t* keys = static_cast<const uint8_t*>(a.keys);
  const uint8_t* qall = static_cast<const uint8_t*>(a.q);
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int i = static_cast<int>(item / n_chunk);
    const int64_t chunk = item % n_chunk;
    int64_t N = (a.q_pos[i] + 1) / a.m;
    if (N > a.ld) N = a.ld;
    const int64_t s0 = chunk * kKeysPerWg + wv * kKeysPerWave;
    if (chunk * kKeysPerWg >= N) continue;
    if (s0 >= N) continue;
    i32x8 qop[NHB];
    int qsc[NHB];
    float wh[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int h = hb * 16 + j16;
      const uint8_t* row = qall + (static_cast<int64_t>(i) * H + h) * RB;
      const uint32_t* cp = reinterpret_cast<const uint32_t*>(row + g * 16);
      qop[hb] = i32x8{static_cast<int>(cp[0]), static_cast<int>(cp[1]), static_cast<int>(cp[2]),
                      static_cast<int>(cp[3]), 0, 0, 0, 0};
      qsc[hb] = row[64 + g];
      wh[hb] = a.w[static_cast<int64_t>(i) * H + h];
    }
    const int64_t kbase = a.key_off[i];
    i32x8 kop[4];
    int ksc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int64_t s = s0 + kb * 16 + j16;
      if (s < N) {
        const uint8_t* row = keys + (kbase + s) * RB;
        const uint32_t* cp = reinterpret_cast<const uint32_t*>(row + g * 16);
        kop[kb] = i32x8{static_cast<int>(cp[0]), static_cast<int>(cp[1]), static_cast<int>(cp[2]),
                        static_cast<int>(cp[3]), 0, 0, 0, 0};
        ksc[kb] = row[64 + g];
      } else {
        kop[kb] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        ksc[kb] = 127;
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int64_t sb = s0 + kb * 16;
      if (sb >= N) break;
      float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop[kb], qop[hb], c, 4, 4, 0, ksc[kb], 0,
                                                             qsc[hb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) part[r] = fmaf(wh[hb], fmaxf(c[r], 0.0f), part[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) part[r] += __shfl_xor(part[r], o, 64);
      }
      if (j16 < 4) {
        const int64_t s = sb + g * 4 + j16;
        const float v = j16 == 0 ? part[0] : j16 == 1 ? part[1] : j16 == 2 ? part[2] : part[3];
        if (s < N) a.scores[static_cast<int64_t>(i) * a.ld + s] = v;
      }
    }
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

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  if (a.fmt == CSA_F32) {
    const int64_t n_chunk = (a.ld + 255) / 256;
    const size_t shm = (static_cast<size_t>(a.H) * a.d + a.H) * sizeof(float);
    hipLaunchKernelGGL(indexer_f32_kernel, dim3(static_cast<unsigned>(a.nq * n_chunk)), dim3(256),
                       shm, stream, a, n_chunk);
    return hipGetLastError();
  }
  const int64_t n_chunk = (a.ld + kKeysPerWg - 1) / kKeysPerWg;
  const int64_t n_items = static_cast<int64_t>(a.nq) * n_chunk;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  const unsigned grid = static_cast<unsigned>(n_items < cap ? n_items : cap);
  const int nhb = a.H / 16;
#define CSA_IDX_CASE(K, NB) \
  case NB: hipLaunchKernelGGL(K<NB>, dim3(grid), dim3(256), 0, stream, a, n_items, n_chunk); break;
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
