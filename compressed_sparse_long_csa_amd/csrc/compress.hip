// Token-level compressor and cache write path (csa_compress).
//
// Source: 硅星人 article on DeepSeek V4, CSA paragraph (every m = 4 tokens'
// KV fold into one entry) and HCA paragraph (m' = 128); DeepSeek-V4 blog,
// RMSNorm归一化 (norm on the compressed KV head) and Partial RoPE位置编码
// (RoPE on the last dims; BF16 RoPE dims, FP8 others).  The gate convention
// (softmax of per-token or per-channel logits over the block) is this
// library's reading of the unspecified compressor weights.
//
// One workgroup per output entry.  The block sum runs over the m tokens in
// order, the mean square over D in a fixed tree, so an entry's bits depend
// only on its own tokens.
#include "kernels.hpp"

namespace csa {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_x(const void* x, csa_fmt fmt, int64_t i) {
  return fmt == CSA_F32 ? static_cast<const float*>(x)[i]
                        : bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

__global__ void __launch_bounds__(kThreads) compress_kernel(CompressArgs a, int64_t n_blocks) {
  const void* __restrict__ x = a.x;
  const csa_fmt x_fmt = a.x_fmt;
  const float* __restrict__ gate = a.gate;
  const int gate_cols = a.gate_cols, D = a.D, m = a.m, nseg = a.nseg, normalize = a.normalize;
  const int64_t* __restrict__ seg_tok_off = a.seg_tok_off;
  const int64_t* __restrict__ seg_pos0 = a.seg_pos0;
  const int64_t* __restrict__ seg_out_row = a.seg_out_row;
  const float* __restrict__ norm_w = a.norm_w;
  const float eps = a.eps;
  const int R = a.rope_dim;
  uint8_t* __restrict__ out = static_cast<uint8_t*>(a.out);
  const csa_fmt out_fmt = a.out_fmt;
  extern __shared__ float y[];            // [D] entry values, then [kThreads/64] partials
  float* red = y + D;
  const int tid = threadIdx.x;
  for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x) {
    const int64_t t0 = blk * m;
    // segment holding token t0: the last s with seg_tok_off[s] <= t0
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg_tok_off[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    const int64_t off = seg_tok_off[s];
    if ((t0 - off) % m != 0 || t0 + m > seg_tok_off[s + 1]) continue;   // straddling block
    const int64_t j = (t0 - off) / m;
    const int64_t row = seg_out_row[s] + j;
    const int64_t pos = seg_pos0[s] + j * m;

    // softmax-gated block sum
    float sq = 0.0f;
    for (int c = tid; c < D; c += kThreads) {
      const int gc = gate_cols == 1 ? 0 : c;
      float gmax = -INFINITY;
      for (int t = 0; t < m; ++t) gmax = fmaxf(gmax, gate[(t0 + t) * gate_cols + gc]);
      float den = 0.0f, acc = 0.0f;
      for (int t = 0; t < m; ++t) {
        const float e = expf(gate[(t0 + t) * gate_cols + gc] - gmax);
        den += e;
        acc = fmaf(e, load_x(x, x_fmt, (t0 + t) * D + c), acc);
      }
      const float v = acc / den;
      y[c] = v;
      sq = fmaf(v, v, sq);
    }
    if (normalize) {
      sq = wave_sum(sq);
      if ((tid & (kWave - 1)) == 0) red[tid / kWave] = sq;
      __syncthreads();
      float tot = 0.0f;
      for (int w = 0; w < kThreads / kWave; ++w) tot += red[w];
      const float r = static_cast<float>(1.0 / sqrt(static_cast<double>(tot) / D + eps));
      for (int c = tid; c < D; c += kThreads)
        y[c] = y[c] * r * (norm_w ? norm_w[c] : 1.0f);
    }
    __syncthreads();
    if (R > 0) {
      for (int i = tid; i < R / 2; i += kThreads) {
        float sn, cs;
        rope_sincos(pos, a.rope_theta[i], &sn, &cs);
        const int d = D - R + 2 * i;
        const float a = y[d], b = y[d + 1];
        y[d] = a * cs - b * sn;
        y[d + 1] = a * sn + b * cs;
      }
      __syncthreads();
    }
    // quantised store
    const size_t rb = row_bytes(out_fmt, D, R);
    uint8_t* dst = out + row * rb;
    switch (out_fmt) {
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
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  const int64_t n_blocks = a.n_tok / a.m;
  if (n_blocks == 0) return hipSuccess;
  const int64_t grid = n_blocks < 65536 ? n_blocks : 65536;
  const size_t shm = (static_cast<size_t>(a.D) + kThreads / kWave) * sizeof(float);
  hipLaunchKernelGGL(compress_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), shm,
                     stream, a, n_blocks);
  return hipGetLastError();
}

}  // namespace csa
