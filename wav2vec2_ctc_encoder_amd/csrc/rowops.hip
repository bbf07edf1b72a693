// Row-wise and elementwise kernels: LayerNorm (+ optional GELU), the
// zero-padded per-group packing that feeds the positional conv, casts, and
// the true-length helpers (packed-row offset tables, zeroing the logits of
// frames past a row's own frames).
//
// LayerNorm: one wave per row, the row held in registers as float4 groups
// (lane i takes elements 4i, 4i+256, ...), statistics in fp32 with wave
// reductions (biased variance, eps inside the square root), two passes over
// registers for mean then centred variance.  Memory bound: one read of the
// row and one or two writes (fp32 residual stream and/or the fp16 GEMM
// operand).
#include "common.h"

namespace w2v2 {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));

__device__ inline float wave_sum(float v) { return wave_sum64(v); }

template <typename T>
__device__ inline float4 load4(const T* p);
template <>
__device__ inline float4 load4<float>(const float* p) { return *(const float4*)p; }
template <>
__device__ inline float4 load4<half_t>(const half_t* p) {
  const h4 h = *(const h4*)p;
  return make_float4((float)h.x, (float)h.y, (float)h.z, (float)h.w);
}
template <typename T>
__device__ inline void store4(T* p, float4 v);
template <>
__device__ inline void store4<float>(float* p, float4 v) { *(float4*)p = v; }
template <>
__device__ inline void store4<half_t>(half_t* p, float4 v) {
  h4 h = {(half_t)v.x, (half_t)v.y, (half_t)v.z, (half_t)v.w};
  *(h4*)p = h;
}

// NV: float4 groups per lane (C <= 256 * NV).  XT: input type.
// x may alias y32 / yt (in-place use): every lane reads its whole row slice
// before writing it, so no restrict qualifiers here.
// y8 (fp8 mode): e4m3 output y * inv8 instead of yt; amax (calibration):
// raised to the max |y| of the rows.
template <typename T, typename XT, int NV>
__global__ __launch_bounds__(256) void layernorm_kernel(const XT* x, int64_t R, int C,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ beta, float eps,
                                                        float* y32, T* yt, int act, float2* __restrict__ stats,
                                                        uint8_t* __restrict__ y8, float inv8,
                                                        float* __restrict__ amax) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const XT* xr = x + row * C;
  // the affine parameters are requested with the row, not after the
  // reductions, so their latency overlaps the row's
  float4 gv[NV], bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = 4 * (lane + 64 * i);
    if (c < C) {
      gv[i] = *(const float4*)(gamma + c);
      bv[i] = *(const float4*)(beta + c);
    }
  }
  float4 v[NV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = 4 * (lane + 64 * i);
    if (c < C) {
      v[i] = load4<XT>(xr + c);
      s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    } else {
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  const float invC = 1.f / (float)C;
  const float mean = wave_sum(s) * invC;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = 4 * (lane + 64 * i);
    if (c < C) {
      const float a = v[i].x - mean, b = v[i].y - mean, cc = v[i].z - mean, d = v[i].w - mean;
      q += (a * a + b * b) + (cc * cc + d * d);
    }
  }
  const float rstd = rsqrtf(wave_sum(q) * invC + eps);
  if (stats && lane == 0) stats[row] = make_float2(mean, rstd);
  float vmax = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = 4 * (lane + 64 * i);
    if (c < C) {
      const float4 g = gv[i], b = bv[i];
      float4 o;
      o.x = (v[i].x - mean) * rstd * g.x + b.x;
      o.y = (v[i].y - mean) * rstd * g.y + b.y;
      o.z = (v[i].z - mean) * rstd * g.z + b.z;
      o.w = (v[i].w - mean) * rstd * g.w + b.w;
      if (act == 1) {
        o.x = act_fn<1>(o.x); o.y = act_fn<1>(o.y); o.z = act_fn<1>(o.z); o.w = act_fn<1>(o.w);
      } else if (act == 2) {
        o.x = act_fn<2>(o.x); o.y = act_fn<2>(o.y); o.z = act_fn<2>(o.z); o.w = act_fn<2>(o.w);
      }
      if (y32) *(float4*)(y32 + row * C + c) = o;
      if (yt) store4<T>(yt + row * C + c, o);
      if (y8) *(uint32_t*)(y8 + row * C + c) = pack_e4m3x4(o.x, o.y, o.z, o.w, inv8);
      vmax = fmaxf(vmax, fmaxf(fmaxf(fabsf(o.x), fabsf(o.y)), fmaxf(fabsf(o.z), fabsf(o.w))));
    }
  }
  if (amax) wave_raise_amax(vmax, amax);
}

template <typename T, typename XT>
hipError_t ln_dispatch(const XT* x, int64_t R, int C, const float* g, const float* b, float eps, float* y32,
                       T* yt, int act, float2* st, uint8_t* y8, float inv8, float* amax, hipStream_t s) {
  const dim3 grid((unsigned)((R + 3) / 4)), block(256);
  const int nv = (C + 255) / 256;
#define W2V2_LN(NV) \
  hipLaunchKernelGGL((layernorm_kernel<T, XT, NV>), grid, block, 0, s, x, R, C, g, b, eps, y32, yt, act, st, y8, inv8, amax)
  if (nv <= 1) W2V2_LN(1);
  else if (nv == 2) W2V2_LN(2);
  else if (nv == 3) W2V2_LN(3);
  else if (nv == 4) W2V2_LN(4);
  else W2V2_LN(8);
#undef W2V2_LN
  return hipGetLastError();
}

// zg[g][b][p][i] = h[b, p - pad, g*Cg + i] for 0 <= p - pad < T, else 0.
template <typename T>
__global__ __launch_bounds__(256) void pos_pack_kernel(const float* __restrict__ h, int B, int Tn, RowSpan rows,
                                                       int d, int G, int Tp, int pad, T* __restrict__ zg,
                                                       int64_t nvec) {
  const int Cg = d / G;
  const int cv = Cg / 4;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int i4 = (int)(v % cv);
    int64_t r = v / cv;
    const int p = (int)(r % Tp);
    r /= Tp;
    const int b = (int)(r % B);
    const int g = (int)(r / B);
    const int t = p - pad;
    const int Tb = rows.len ? rows.len[b] : Tn;
    const int64_t hrow = rows.start ? (int64_t)rows.start[b] : (int64_t)b * Tn;
    float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t >= 0 && t < Tb) val = *(const float4*)(h + (hrow + t) * d + g * Cg + 4 * i4);
    store4<T>(zg + v * 4, val);
  }
}

// One thread per (table, row, frame): out[start[b] + t] = base[b] + t * mul.
struct RowTables {
  RowTable t[kMaxRowTables];
};
__global__ __launch_bounds__(256) void row_tables_kernel(RowTables rt) {
  const RowTable& tb = rt.t[blockIdx.z];
  const int b = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < tb.len[b]) tb.out[(int64_t)tb.start[b] + t] = tb.base[b] + (int64_t)t * tb.mul;
}

// y [B, T, V]: zero every element of frames t >= len[b].
__global__ __launch_bounds__(256) void zero_tail_kernel(float* __restrict__ y, int B, int T, int V,
                                                        const int32_t* __restrict__ len, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t f = i / V;
    const int t = (int)(f % T), b = (int)(f / T);
    if (t >= len[b]) y[i] = 0.f;
  }
}

template <typename T>
__global__ void cast_to_f32_kernel(const T* __restrict__ x, float* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    y[i] = (float)x[i];
}
template <typename T>
__global__ void cast_from_f32_kernel(const float* __restrict__ x, T* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    y[i] = (T)x[i];
}

inline int grid_for(int64_t work) {
  const int64_t g = (work + 255) / 256;
  return (int)(g < 16384 ? (g < 1 ? 1 : g) : 16384);
}

}  // namespace

hipError_t launch_layernorm(DType t, const float* x_f32, const void* x_t, int64_t R, int32_t C,
                            const float* gamma, const float* beta, float eps, float* y_f32, void* y_t,
                            int32_t act, float2* stats, hipStream_t s, uint8_t* y8, float inv8, float* amax) {
  if (R <= 0) return hipSuccess;
  if (y8 && C % 4) return hipErrorInvalidValue;
  if (t == DType::F16) {
    if (x_f32)
      return ln_dispatch<half_t, float>(x_f32, R, C, gamma, beta, eps, y_f32, (half_t*)y_t, act, stats, y8, inv8,
                                        amax, s);
    return ln_dispatch<half_t, half_t>((const half_t*)x_t, R, C, gamma, beta, eps, y_f32, (half_t*)y_t, act, stats,
                                       y8, inv8, amax, s);
  }
  if (x_f32)
    return ln_dispatch<float, float>(x_f32, R, C, gamma, beta, eps, y_f32, (float*)y_t, act, stats, y8, inv8, amax,
                                     s);
  return ln_dispatch<float, float>((const float*)x_t, R, C, gamma, beta, eps, y_f32, (float*)y_t, act, stats, y8,
                                   inv8, amax, s);
}

hipError_t launch_pos_pack(DType t, const float* h, int32_t B, int32_t T, RowSpan rows, int32_t d, int32_t G,
                           int32_t Kp, int32_t pad, void* zg, hipStream_t s) {
  const int Tp = T + Kp;
  const int64_t nvec = (int64_t)G * B * Tp * (d / G) / 4;
  if (t == DType::F16)
    hipLaunchKernelGGL(pos_pack_kernel<half_t>, dim3(grid_for(nvec)), dim3(256), 0, s, h, B, T, rows, d, G, Tp,
                       pad, (half_t*)zg, nvec);
  else
    hipLaunchKernelGGL(pos_pack_kernel<float>, dim3(grid_for(nvec)), dim3(256), 0, s, h, B, T, rows, d, G, Tp,
                       pad, (float*)zg, nvec);
  return hipGetLastError();
}

hipError_t launch_row_tables(const RowTable* tabs, int32_t n, int32_t B, int32_t tmax, hipStream_t s) {
  if (n < 1 || n > kMaxRowTables || B < 1 || tmax < 1) return hipErrorInvalidValue;
  RowTables rt{};
  for (int i = 0; i < n; ++i) rt.t[i] = tabs[i];
  hipLaunchKernelGGL(row_tables_kernel, dim3((tmax + 255) / 256, B, n), dim3(256), 0, s, rt);
  return hipGetLastError();
}

hipError_t launch_zero_tail_frames(float* y, int32_t B, int32_t T, int32_t V, const int32_t* len, hipStream_t s) {
  const int64_t nvec = (int64_t)B * T * V;
  hipLaunchKernelGGL(zero_tail_kernel, dim3(grid_for(nvec)), dim3(256), 0, s, y, B, T, V, len, nvec);
  return hipGetLastError();
}

hipError_t launch_cast_to_f32(DType t, const void* x, float* y, int64_t n, hipStream_t s) {
  if (t == DType::F16)
    hipLaunchKernelGGL(cast_to_f32_kernel<half_t>, dim3(grid_for(n)), dim3(256), 0, s, (const half_t*)x, y, n);
  else
    hipLaunchKernelGGL(cast_to_f32_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, (const float*)x, y, n);
  return hipGetLastError();
}

hipError_t launch_cast_from_f32(DType t, const float* x, void* y, int64_t n, hipStream_t s) {
  if (t == DType::F16)
    hipLaunchKernelGGL(cast_from_f32_kernel<half_t>, dim3(grid_for(n)), dim3(256), 0, s, x, (half_t*)y, n);
  else
    hipLaunchKernelGGL(cast_from_f32_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, x, (float*)y, n);
  return hipGetLastError();
}

}  // namespace w2v2
