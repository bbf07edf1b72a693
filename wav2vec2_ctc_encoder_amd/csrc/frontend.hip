// Feature-encoder kernels: conv 0 over raw PCM, the GroupNorm-over-time
// statistics and their application, and the frames-per-row rule.
//
// conv 0 has one input channel (k = 10, s = 5 for wav2vec2), so it is a
// short FIR filter bank: no matrix-core work, bound by writing its
// [B, T0, C] output.  A workgroup takes a chunk of frames of one row,
// stages the PCM samples of the chunk in LDS (coalesced reads, samples at
// or after the valid length replaced by 0), and each wave computes whole
// output frames: every lane owns 8 consecutive channels, so one frame is a
// single 1 KB (fp16) coalesced store per wave.
//
// Group-norm variant: GroupNorm with one group per channel needs mean and
// variance over all T0 frames of a row.  Each workgroup writes, per channel,
// the mean and the centred sum of squares M2 of its own chunk (computed in
// two passes over the chunk, the second recomputing the 10-tap conv from
// LDS instead of re-reading the output); gn_finalize merges the chunk
// partials in a fixed order with Chan's pairwise update, so the statistics
// are deterministic and free of the cancellation of sum / sum-of-squares.
// Layer-norm variant: the per-frame LayerNorm over channels and the GELU are
// done in registers with wave reductions before the single store.
#include "common.h"

namespace w2v2 {
namespace {

constexpr int kChunk = 256;  // frames per workgroup
constexpr int kLanesC = 8;   // channels per lane

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__device__ inline void store8(T* dst, const float* v);

template <>
__device__ inline void store8<half_t>(half_t* dst, const float* v) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  h8 h = {(half_t)v[0], (half_t)v[1], (half_t)v[2], (half_t)v[3],
          (half_t)v[4], (half_t)v[5], (half_t)v[6], (half_t)v[7]};
  *(h8*)dst = h;
}

template <>
__device__ inline void store8<float>(float* dst, const float* v) {
  *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
  *(float4*)(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// KT: compile-time tap count (taps >= k carry zero weights).
template <typename T, int KT>
__global__ __launch_bounds__(256) void conv0_kernel(const float* __restrict__ pcm, const int32_t* __restrict__ valid,
                                                     int L, const float* __restrict__ w0,
                                                     const float* __restrict__ bias, int C, int k, int stride,
                                                     int T0, T* __restrict__ y, float2* __restrict__ stats,
                                                     const float* __restrict__ gamma,
                                                     const float* __restrict__ beta, float eps) {
  extern __shared__ float smem[];
  const int b = blockIdx.y;
  const int chunk = blockIdx.x;
  const int t0 = chunk * kChunk;
  const int nf = min(kChunk, T0 - t0);
  const int nsamp = (nf - 1) * stride + KT;
  float* xs = smem;                                  // [nsamp]
  float* red = smem + ((nsamp + 3) & ~3);            // [4][C] (group variant)

  int vl = valid[b];
  vl = vl < 0 ? 0 : (vl > L ? L : vl);
  const int64_t base = (int64_t)t0 * stride;
  for (int i = threadIdx.x; i < nsamp; i += 256) {
    const int64_t idx = base + i;
    xs[i] = (idx < vl) ? pcm[(int64_t)b * L + idx] : 0.f;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = lane * kLanesC;
  const bool active = c0 < C;
  float w[kLanesC][KT];
  float bv[kLanesC];
#pragma unroll
  for (int c = 0; c < kLanesC; ++c) {
    bv[c] = (active && bias) ? bias[c0 + c] : 0.f;
#pragma unroll
    for (int j = 0; j < KT; ++j) w[c][j] = (active && j < k) ? w0[(c0 + c) * k + j] : 0.f;
  }

  auto conv = [&](int f, float* out) {
    const float* x = xs + f * stride;
#pragma unroll
    for (int c = 0; c < kLanesC; ++c) out[c] = bv[c];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const float xv = x[j];
#pragma unroll
      for (int c = 0; c < kLanesC; ++c) out[c] = fmaf(w[c][j], xv, out[c]);
    }
  };

  if (gamma) {
    // layer variant: per-frame LN over C channels, affine, GELU
    float g[kLanesC], be[kLanesC];
#pragma unroll
    for (int c = 0; c < kLanesC; ++c) {
      g[c] = active ? gamma[c0 + c] : 0.f;
      be[c] = active ? beta[c0 + c] : 0.f;
    }
    const float invC = 1.f / (float)C;
    for (int f = wave; f < nf; f += 4) {
      float v[kLanesC];
      conv(f, v);
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kLanesC; ++c) s += active ? v[c] : 0.f;
      const float mean = wave_sum(s) * invC;
      float q = 0.f;
#pragma unroll
      for (int c = 0; c < kLanesC; ++c) {
        const float d = v[c] - mean;
        q += active ? d * d : 0.f;
      }
      const float rstd = rsqrtf(wave_sum(q) * invC + eps);
#pragma unroll
      for (int c = 0; c < kLanesC; ++c) v[c] = gelu_erf((v[c] - mean) * rstd * g[c] + be[c]);
      if (active) store8<T>(y + ((int64_t)b * T0 + t0 + f) * C + c0, v);
    }
    return;
  }

  // group variant, pass 1: store the conv output, per-channel sums
  float sum[kLanesC];
#pragma unroll
  for (int c = 0; c < kLanesC; ++c) sum[c] = 0.f;
  for (int f = wave; f < nf; f += 4) {
    float v[kLanesC];
    conv(f, v);
#pragma unroll
    for (int c = 0; c < kLanesC; ++c) sum[c] += v[c];
    if (active) store8<T>(y + ((int64_t)b * T0 + t0 + f) * C + c0, v);
  }
  if (active) {
#pragma unroll
    for (int c = 0; c < kLanesC; ++c) red[wave * C + c0 + c] = sum[c];
  }
  __syncthreads();
  float mean[kLanesC];
#pragma unroll
  for (int c = 0; c < kLanesC; ++c) {
    mean[c] = active ? (red[c0 + c] + red[C + c0 + c] + red[2 * C + c0 + c] + red[3 * C + c0 + c]) / (float)nf
                     : 0.f;
  }
  __syncthreads();
  // pass 2: centred sum of squares, recomputing the conv from LDS
  float m2[kLanesC];
#pragma unroll
  for (int c = 0; c < kLanesC; ++c) m2[c] = 0.f;
  for (int f = wave; f < nf; f += 4) {
    float v[kLanesC];
    conv(f, v);
#pragma unroll
    for (int c = 0; c < kLanesC; ++c) {
      const float d = v[c] - mean[c];
      m2[c] = fmaf(d, d, m2[c]);
    }
  }
  if (active) {
#pragma unroll
    for (int c = 0; c < kLanesC; ++c) red[wave * C + c0 + c] = m2[c];
  }
  __syncthreads();
  if (active && wave == 0) {
    const int nchunk = gridDim.x;
#pragma unroll
    for (int c = 0; c < kLanesC; ++c) {
      const float q = red[c0 + c] + red[C + c0 + c] + red[2 * C + c0 + c] + red[3 * C + c0 + c];
      stats[((int64_t)b * nchunk + chunk) * C + c0 + c] = make_float2(mean[c], q);
    }
  }
}

__global__ void gn_finalize_kernel(const float2* __restrict__ stats, int C, int T0, int nchunk,
                                   const float* __restrict__ gamma, const float* __restrict__ beta,
                                   float eps, float2* __restrict__ ss) {
  const int b = blockIdx.y;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  // Chan et al. pairwise merge of (n, mean, M2), chunks in order
  double n = 0.0, mean = 0.0, m2 = 0.0;
  for (int j = 0; j < nchunk; ++j) {
    const float2 p = stats[((int64_t)b * nchunk + j) * C + c];
    const double nb = (double)min(kChunk, T0 - j * kChunk);
    const double nn = n + nb;
    const double delta = (double)p.x - mean;
    mean += delta * nb / nn;
    m2 += (double)p.y + delta * delta * n * nb / nn;
    n = nn;
  }
  const double var = m2 / n;
  const float rstd = (float)(1.0 / sqrt(var + (double)eps));
  const float sc = gamma[c] * rstd;
  ss[(int64_t)b * C + c] = make_float2(sc, beta[c] - (float)mean * sc);
}

template <typename T>
__global__ __launch_bounds__(256) void gn_apply_gelu_kernel(T* __restrict__ y, const float2* __restrict__ ss,
                                                            int T0, int C, int64_t nvec) {
  constexpr int EPV = 16 / sizeof(T);
  const int64_t rowel = (int64_t)T0 * C;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = v * EPV;
    const int b = (int)(e / rowel);
    const int c = (int)(e % C);
    const float2* s = ss + (int64_t)b * C + c;
    uint4 raw = *(const uint4*)(y + e);
    T* el = (T*)&raw;
#pragma unroll
    for (int i = 0; i < EPV; ++i) {
      const float2 p = s[i];
      el[i] = (T)gelu_erf(fmaf((float)el[i], p.x, p.y));
    }
    *(uint4*)(y + e) = raw;
  }
}

struct ConvChain {
  int32_t n;
  int32_t k[8];
  int32_t s[8];
};

__global__ void valid_frames_kernel(const int32_t* __restrict__ valid, int B, int window, ConvChain ch,
                                    int32_t* __restrict__ vf) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int n = valid[b];
  n = n < 0 ? 0 : (n > window ? window : n);
  for (int i = 0; i < ch.n; ++i) n = (n < ch.k[i]) ? 0 : (n - ch.k[i]) / ch.s[i] + 1;
  vf[b] = n;
}

template <typename T, int KT>
hipError_t conv0_t(const float* pcm, const int32_t* valid, int32_t L, int32_t B, const float* w0,
                   const float* bias, int32_t C, int32_t k, int32_t stride, int32_t T0, void* y,
                   float2* stats, const float* gamma, const float* beta, float eps, hipStream_t s) {
  const int nchunk = (T0 + kChunk - 1) / kChunk;
  const int nsamp = (kChunk - 1) * stride + KT;
  const size_t lds = (size_t)(((nsamp + 3) & ~3) + 4 * C) * sizeof(float);
  hipLaunchKernelGGL((conv0_kernel<T, KT>), dim3(nchunk, B), dim3(256), lds, s, pcm, valid, L, w0, bias,
                     C, k, stride, T0, (T*)y, stats, gamma, beta, eps);
  return hipGetLastError();
}

template <typename T>
hipError_t conv0_k(int k, const float* pcm, const int32_t* valid, int32_t L, int32_t B, const float* w0,
                   const float* bias, int32_t C, int32_t stride, int32_t T0, void* y, float2* stats,
                   const float* gamma, const float* beta, float eps, hipStream_t s) {
  if (k == 10) return conv0_t<T, 10>(pcm, valid, L, B, w0, bias, C, k, stride, T0, y, stats, gamma, beta, eps, s);
  return conv0_t<T, 16>(pcm, valid, L, B, w0, bias, C, k, stride, T0, y, stats, gamma, beta, eps, s);
}

}  // namespace

int conv0_chunk_frames() { return kChunk; }

hipError_t launch_conv0(DType t, const float* pcm, const int32_t* valid, int32_t L, int32_t B,
                        const float* w0, const float* bias, int32_t C, int32_t k, int32_t stride,
                        int32_t T0, void* y, float2* stats, const float* gamma, const float* beta,
                        float eps, hipStream_t s) {
  if (t == DType::F16)
    return conv0_k<half_t>(k, pcm, valid, L, B, w0, bias, C, stride, T0, y, stats, gamma, beta, eps, s);
  return conv0_k<float>(k, pcm, valid, L, B, w0, bias, C, stride, T0, y, stats, gamma, beta, eps, s);
}

hipError_t launch_gn_finalize(const float2* stats, int32_t B, int32_t C, int32_t T0, int32_t chunk,
                              const float* gamma, const float* beta, float eps, float2* scale_shift,
                              hipStream_t s) {
  (void)chunk;
  const int nchunk = (T0 + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(gn_finalize_kernel, dim3((C + 255) / 256, B), dim3(256), 0, s, stats, C, T0, nchunk,
                     gamma, beta, eps, scale_shift);
  return hipGetLastError();
}

hipError_t launch_gn_apply_gelu(DType t, void* y, const float2* scale_shift, int32_t B, int32_t T,
                                int32_t C, hipStream_t s) {
  const int64_t n = (int64_t)B * T * C;
  const int epv = t == DType::F16 ? 8 : 4;
  const int64_t nvec = n / epv;
  const int64_t want = (nvec + 255) / 256;
  const int grid = (int)(want < 256 * 64 ? want : 256 * 64);
  if (t == DType::F16)
    hipLaunchKernelGGL(gn_apply_gelu_kernel<half_t>, dim3(grid), dim3(256), 0, s, (half_t*)y, scale_shift, T, C, nvec);
  else
    hipLaunchKernelGGL(gn_apply_gelu_kernel<float>, dim3(grid), dim3(256), 0, s, (float*)y, scale_shift, T, C, nvec);
  return hipGetLastError();
}

hipError_t launch_valid_frames(const int32_t* valid, int32_t B, int32_t window, int32_t n_conv,
                               const int32_t* kernel, const int32_t* stride, int32_t* vframes,
                               hipStream_t s) {
  ConvChain ch{};
  ch.n = n_conv;
  for (int i = 0; i < n_conv && i < 8; ++i) {
    ch.k[i] = kernel[i];
    ch.s[i] = stride[i];
  }
  hipLaunchKernelGGL(valid_frames_kernel, dim3((B + 255) / 256), dim3(256), 0, s, valid, B, window, ch, vframes);
  return hipGetLastError();
}

}  // namespace w2v2
