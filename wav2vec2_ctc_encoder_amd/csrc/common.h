// Internal declarations shared by the HIP kernels and the runtime.
// Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w2v2 {

typedef _Float16 half_t;

// Element type of matrix operands: fp16 in the fp16 mode, fp32 in the fp32
// mode; F8 (e4m3) only for the encoder projections of the fp8 mode.
enum class DType : int { F32 = 0, F16 = 1, F8 = 2 };

inline size_t dsize(DType t) { return t == DType::F16 ? 2 : (t == DType::F8 ? 1 : 4); }

// e4m3 (OCP FP8: 1-4-3, bias 7, largest value 448) bytes of four values x * inv,
// rounded to nearest even (v_cvt_pk_fp8_f32) after a clamp to +-448: the
// instruction itself turns values from 480 up into NaN, the quantization of
// the fp8 mode saturates.  Byte i holds value i.
__device__ inline float clamp_e4m3(float x) { return fminf(fmaxf(x, -448.f), 448.f); }
__device__ inline uint32_t pack_e4m3x4(float a, float b, float c, float d, float inv) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a * inv), clamp_e4m3(b * inv), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c * inv), clamp_e4m3(d * inv), w, true);
  return (uint32_t)w;
}

// Calibration statistic: raise *amax to the largest v (>= 0) of the wave.
// Non-negative floats order like their bit patterns, so an unsigned integer
// maximum is the float maximum and the result does not depend on the order.
// Every lane of the wave must call it.
__device__ inline void wave_raise_amax(float v, float* amax) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) atomicMax((unsigned int*)amax, __float_as_uint(v));
}

// Exact (erf) GELU, x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), with erf from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (Hastings' rational approximation, |error| <= 1.5e-7 for z >= 0):
//   erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
//   t = 1 / (1 + p z),  z = |x| / sqrt 2.
// With q = erfc(z) / 2, GELU(x) = x - |x| q for x >= 0 and -|x| q for x < 0,
// i.e. max(x, 0) - |x| q: one fused multiply-add after q, no select.  The
// halving is folded into the coefficients and 1/sqrt 2 into p; the exponent
// -z^2 log2(e) is -(x k)^2 with k^2 = log2(e) / 2.  Absolute error <= ~3e-7
// |x| in fp32, far below the fp16 operand rounding the fp16 mode adds;
// GELU(0) is exactly 0.
__device__ inline float gelu_erf(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164189f, ax, 1.0f));  // p / sqrt 2 = 0.3275911 / sqrt 2
  float p = fmaf(0.5307027145f, t, -0.7265760135f);                    // a5 / 2, a4 / 2
  p = fmaf(p, t, 0.7107068705f);                                        // a3 / 2
  p = fmaf(p, t, -0.142248368f);                                        // a2 / 2
  p = fmaf(p, t, 0.127414796f);                                         // a1 / 2
  p *= t;
  const float u = x * 0.84932180028801904f;                             // k = sqrt(log2(e) / 2)
  const float q = p * __builtin_amdgcn_exp2f(-(u * u));
  return fmaf(-ax, q, fmaxf(x, 0.f));
}

// tanh approximation of GELU, x/2 (1 + tanh(u)) with u = sqrt(2/pi)(x +
// 0.044715 x^3) (Hendrycks & Gimpel), written as x * sigmoid(2u) =
// x / (1 + exp(-2u)): saturates cleanly to x and to -0 for large |x|.  The
// two constant factors of the exponent, sqrt(2/pi) and -2 log2(e), are one.
__device__ inline float gelu_tanh(float x) {
  const float v = fmaf(0.044715f * x, x * x, x);
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.3022081981443f * v));  // -2 log2(e) sqrt(2/pi)
}

// Cross-lane reductions without the LDS crossbar.  v_permlane16_swap /
// v_permlane32_swap (gfx950) with both operands x return, for every lane,
// x of the lane and x of lane ^ 16 (lane ^ 32) as an (even row, odd row) /
// (lower half, upper half) pair; combining the two with a commutative op
// gives both lanes of a pair the same bits.
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x + x of the lane `R` places away by rotation within its row of 16 (DPP
// row_ror); for R = 8, 4, 2, 1 in turn every lane of a row pairs with a lane
// holding the same partial sums, so the row ends with one value.
template <int R>
__device__ inline float add_ror(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + R, 0xF, 0xF, false));
}
// Sum over the 64 lanes of a wave, the same bits in every lane.
__device__ inline float wave_sum64(float v) {
  v = add_ror<8>(v);
  v = add_ror<4>(v);
  v = add_ror<2>(v);
  v = add_ror<1>(v);
  return add_xor32(add_xor16(v));
}

// Activation codes of the kernels: 0 none, 1 erf GELU, 2 tanh GELU.  Hot
// loops take the code as a template argument (selected once per launch) so
// that only one form is compiled into them.
template <int ACT>
__device__ inline float act_fn(float x) {
  if constexpr (ACT == 1) return gelu_erf(x);
  else if constexpr (ACT == 2) return gelu_tanh(x);
  else return x;
}

// Static device scratch (scratch.hip) of the allocation-free entry point:
// its size, and its device address on `device` (resolved once per device
// with that device current; call with the device current).
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_setup(int device, void** addr);

// Kernel-timing hook of the runtime: called around every launch.
struct LaunchHook {
  virtual void before(const char* name, hipStream_t s) = 0;
  virtual void after(const char* name, hipStream_t s) = 0;
  virtual ~LaunchHook() {}
};

// ----------------------------------------------------------------------------
// GEMM:  C[m, n] = epilogue( sum_k A[m, k] * Bw[n, k] )
//   A rows are addressed through a two-level map so the same kernel serves
//   linears, implicit-GEMM strided convs and the grouped positional conv:
//     row m -> seg = m / seg_rows, t = m % seg_rows,
//     A_row(m) = A + group*a_group + seg*a_seg + t*lda      (elements)
//   Bw is [N, K] row-major per group (ldb = K): Bw + group*b_group.
//   Epilogue per element: v = acc + bias[n]; v = act(v); v += residual[m, n];
//   stores fp32 (out_f32) and/or operand type (out_t) at C + group*c_group + m*ldc + n.
//   grid.z = groups.
// ----------------------------------------------------------------------------
// Role of a GEMM launch.  Each role is compiled as its own kernel symbol so
// profilers attribute time per role.
enum GemmRole : int {
  kGemmConv = 0, kGemmProj = 1, kGemmPos = 2, kGemmQKV = 3, kGemmOut = 4, kGemmFFN1 = 5, kGemmFFN2 = 6,
  kGemmHead = 7, kGemmRoles = 8
};

struct GemmArgs {
  int32_t role = kGemmConv;
  const void* A = nullptr;
  int64_t lda = 0, a_seg = 0, a_group = 0;
  int32_t seg_rows = 1;
  // Optional per-row tables (element offsets, M entries each): A row m starts
  // at A + a_group * group + a_rows[m] instead of the segment rule
  // seg * a_seg + t * lda; output row m starts at c_rows[m] instead of
  // m * ldc (plus c_group * group in both cases).
  const int64_t* a_rows = nullptr;
  const int64_t* c_rows = nullptr;
  const void* B = nullptr;
  int64_t b_group = 0;
  int32_t M = 0, N = 0, K = 0, groups = 1;
  const float* bias = nullptr;
  int64_t bias_group = 0;
  const float* residual = nullptr;  // fp32, indexed like C; may alias out_f32
  // Optional LayerNorm applied to the residual as it is read: residual
  // element (m, n) is taken as (r - st.x) * st.y * res_gamma[n] + res_beta[n]
  // with st = res_stats[m] = (mean, rstd) of row m (post-norm blocks keep the
  // raw residual sum in memory and only its row statistics).
  const float2* res_stats = nullptr;
  const float* res_gamma = nullptr;
  const float* res_beta = nullptr;
  float* out_f32 = nullptr;
  void* out_t = nullptr;
  int64_t ldc = 0, c_group = 0;
  int32_t act = 0;  // 0 none, 1 erf GELU, 2 tanh GELU (applied after the bias)
  // Optional per-row argmax (CTC head): for every output row r (r = m, or
  // c_rows[m] / ldc with an output row table) amax[r] is raised with
  // atomicMax to the largest argmax_key of the row's stored fp32 values, so
  // after the launch it holds the row's maximum and its lowest column.  The
  // caller zero-fills amax first.
  uint64_t* amax = nullptr;
  // fp8 mode projections (operand type F8): the accumulator of column n is
  // scaled by col_scale[n] (activation scale times the weight scale of that
  // column's tensor) before the bias.
  const float* col_scale = nullptr;
  // e4m3 operands only: out_t holds fp32 (the fp8 projections of an fp32
  // graph) instead of fp16.
  int32_t out_t_f32 = 0;
  // Optional e4m3 output, laid out like out_t: e4m3(clamp(v * out_f8_inv)).
  uint8_t* out_f8 = nullptr;
  float out_f8_inv = 1.f;
  // Optional calibration: *out_amax is raised to the max |v| of the values
  // stored (see wave_raise_amax).
  float* out_amax = nullptr;
};

// Argmax key of value v in column n: a larger value gives a larger key, and
// equal values give the larger key to the lower column, so the maximum key of
// a row names its first maximum (numpy's argmax convention) whatever order
// the keys are combined in.  -0 counts as +0 (they compare equal); the low
// word is 0xFFFFFFFF - n, so n = 0xFFFFFFFF - (uint32_t)key.
__device__ inline uint64_t argmax_key(float v, int n) {
  const uint32_t u = v == 0.f ? 0u : __float_as_uint(v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
}
__device__ inline uint64_t max_key_xor(uint64_t k, int mask) {
  const uint32_t lo = __shfl_xor((uint32_t)k, mask, 64), hi = __shfl_xor((uint32_t)(k >> 32), mask, 64);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > k ? o : k;
}

// fp16 with K % 64 == 0 and N > 32: 128x128 or 128x64 tiles of the direct-to-LDS
// kernel (chosen from N, K and the tile count); otherwise 128xN tiles (N = 32,
// 48, 64, 128) of the register-staged kernel.
hipError_t launch_gemm(DType t, const GemmArgs& a, hipStream_t s);

// ----------------------------------------------------------------------------
// feature-encoder kernels
// ----------------------------------------------------------------------------
// conv 0 (one input channel) over the zero-padded window, fused with its
// norm and GELU:
//   pcm [B, L] fp32, valid [B]; w0 [C][k] fp32; bias [C] fp32 or null;
//   y [B, T0, C] (operand type).
//   group variant (gamma == null): y = GELU(conv * ss[b, c].x + ss[b, c].y),
//     ss from gn0_finalize.
//   layer variant (gamma != null): y = GELU(LN_c(conv + bias) * gamma + beta).
// Per-row frames: rows.len (frames of row b, null: T0 for every row) and
// rows.start (first packed output row of row b, null: b * T0).
struct RowSpan {
  const int32_t* len = nullptr;
  const int32_t* start = nullptr;
};
hipError_t launch_conv0(DType t, const float* pcm, const int32_t* valid, int32_t L, int32_t B,
                        const float* w0, const float* bias, int32_t C, int32_t k, int32_t stride,
                        int32_t T0, RowSpan rows, void* y, const float2* ss, const float* gamma,
                        const float* beta, float eps, int32_t act, hipStream_t s);
// GroupNorm statistics of conv 0 from the PCM alone: per-chunk means and
// co-moments of the k shifted sample sequences (fp64), then per (b, c)
// scale = gamma * rstd and shift = beta - mean * scale.
// Workspace: B * gn0_partial_doubles(k, T0) doubles (chunk partials, then the
// per-row merged statistics behind them).
int64_t gn0_partial_doubles(int32_t k, int32_t T0);  // per row
// With rows_len set, row b's statistics cover its own rows_len[b] frames.
hipError_t launch_gn0_stats(const float* pcm, const int32_t* valid, int32_t L, int32_t B, int32_t k, int32_t stride,
                            int32_t T0, const int32_t* rows_len, double* part, hipStream_t s);
hipError_t launch_gn0_finalize(double* part, int32_t B, int32_t k, int32_t T0, const int32_t* rows_len,
                               const float* w0, const float* bias, int32_t C, const float* gamma,
                               const float* beta, float eps, float2* ss, hipStream_t s);

// ----------------------------------------------------------------------------
// row kernels
// ----------------------------------------------------------------------------
// LayerNorm over the C entries of each of R rows.  Input fp32 (x_f32) or the
// operand type (x_t); outputs fp32 (y_f32) and/or operand type (y_t); act 1
// (erf GELU) or 2 (tanh GELU) is applied after the affine map; stats, if
// not null, receives (mean, rstd) per row.  Input and output may alias.
// y8 (fp8 mode): write e4m3(y * inv8) there instead of y_t; amax
// (calibration): raised to the max |y| written.
hipError_t launch_layernorm(DType t, const float* x_f32, const void* x_t, int64_t R, int32_t C,
                            const float* gamma, const float* beta, float eps, float* y_f32,
                            void* y_t, int32_t act, float2* stats, hipStream_t s, uint8_t* y8 = nullptr,
                            float inv8 = 1.f, float* amax = nullptr);
// Positional-conv input: h fp32 [B, T, d] -> zg [G][B][T + K][d/G] (operand
// type) with `pad` zero frames before the data and zeros after it.  With
// rows set, h holds packed rows (row b's frame t at rows.start[b] + t) and
// frames t >= rows.len[b] of row b are zero in zg as well.
hipError_t launch_pos_pack(DType t, const float* h, int32_t B, int32_t T, RowSpan rows, int32_t d, int32_t G,
                           int32_t Kp, int32_t pad, void* zg, hipStream_t s);
// dtype conversions [n]
hipError_t launch_cast_to_f32(DType t, const void* x, float* y, int64_t n, hipStream_t s);
hipError_t launch_cast_from_f32(DType t, const float* x, void* y, int64_t n, hipStream_t s);
// Packed-row offset tables: for every table and row b, entries
// out[start[b] + t] = base[b] + t * mul for t < len[b].
struct RowTable {
  const int32_t* start = nullptr;
  const int32_t* len = nullptr;
  const int64_t* base = nullptr;
  int64_t mul = 0;
  int64_t* out = nullptr;
};
constexpr int kMaxRowTables = 10;
hipError_t launch_row_tables(const RowTable* tabs, int32_t n, int32_t B, int32_t tmax, hipStream_t s);
// y [B, T, V] fp32: frames t >= len[b] of row b set to 0.
hipError_t launch_zero_tail_frames(float* y, int32_t B, int32_t T, int32_t V, const int32_t* len,
                                   hipStream_t s);
// frames per row from valid samples (conv length rule)
hipError_t launch_valid_frames(const int32_t* valid, int32_t B, int32_t window, int32_t n_conv,
                               const int32_t* kernel, const int32_t* stride, int32_t* vframes,
                               hipStream_t s);

// ----------------------------------------------------------------------------
// attention: qkv [B*T, 3d] (q | k | v, head h at columns h*dh), out [B*T, d]
// ----------------------------------------------------------------------------
// With rows set, row b has its own rows.len[b] frames starting at packed row
// rows.start[b] of qkv and out, and attends over those frames only.
// shared: another part of the batch runs concurrently on the GPU (the fp16
// kernel then leaves room on each CU for that part's GEMM workgroups).
// out8 (fp8 mode): the output as e4m3(o * inv8) instead of out; amax
// (calibration): raised to the max |o| written.
bool attention_supported(int dh);
hipError_t launch_attention(DType t, const void* qkv, void* out, int32_t B, int32_t T, RowSpan rows,
                            int32_t H, int32_t dh, bool shared, hipStream_t s, uint8_t* out8 = nullptr,
                            float inv8 = 1.f, float* amax = nullptr);

// ----------------------------------------------------------------------------
// CTC
// ----------------------------------------------------------------------------
hipError_t launch_frame_argmax(const float* logits, int64_t rows, int32_t V, int32_t* out,
                               hipStream_t s);
hipError_t launch_ctc_collapse(const int32_t* vframes, int32_t B, int32_t T, int32_t blank,
                               int32_t* ids, int32_t* lens, hipStream_t s);
// The same collapse over paths given as argmax keys (argmax_key) [B, T].
hipError_t launch_ctc_collapse_keys(const uint64_t* keys, const int32_t* vframes, int32_t B, int32_t T,
                                    int32_t blank, int32_t* ids, int32_t* lens, hipStream_t s);
// keys [n] = 0 (before an argmax-raising GEMM)
hipError_t launch_zero_keys(uint64_t* keys, int64_t n, hipStream_t s);

}  // namespace w2v2
