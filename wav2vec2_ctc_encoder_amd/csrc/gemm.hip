// MFMA GEMM for gfx950 with a row-mapped A operand and a fused epilogue.
//
// Serves every dense contraction of the network:
//  * the encoder linears (fused QKV, out, FFN1, FFN2), the feature projection
//    and the CTC head (plain rows: seg_rows = M, lda = K);
//  * the strided feature-encoder convs as implicit GEMM: in the channels-last
//    layout [B, T_in, C] the input window of output frame t is the contiguous
//    run of k*C elements starting at frame s*t, so A row (b, t) begins at
//    b*T_in*C + t*s*C (seg = b, lda = s*C, K = k*C) and the weight is the
//    conv kernel repacked to [C_out, k*C] with K index j*C + c;
//  * the grouped positional conv, one grid.z slice per group, over a
//    zero-padded per-group copy of its input (lda = C_g, K = taps*C_g).
//
// Tiling: 256 threads = 4 waves.  Block tile BM x BN, K step of 128 bytes
// per row (64 fp16 / 32 fp32), double-buffered LDS with the next K step
// prefetched into registers, one barrier per step.  Each wave owns a
// (TN*16) x (TM*16) sub-tile built from 16x16 MFMA blocks.  The MFMA A
// operand is the weight (n side) and the B operand the activation (m side),
// so every lane ends up holding 4 consecutive output columns of one row and
// the epilogue stores 16-byte (fp32) / 8-byte (fp16) vectors.
//
// fp16: v_mfma_f32_16x16x32_f16, one per 16-byte lane fragment.
// fp32: v_mfma_f32_16x16x4_f32, four per 16-byte lane fragment; fragment
//       element j of lane group g carries k = 4g + j for both operands, a
//       permutation of the 16 k values, so the sum is unchanged.
#include "common.h"

namespace w2v2 {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kPitch = 9;  // LDS row pitch in 16-byte units: 128 B of data + 16 B pad

template <typename T>
struct Mma;

template <>
struct Mma<half_t> {
  __device__ static inline void run(const uint4& a, const uint4& b, f4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b),
                                               c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  __device__ static inline void run(const uint4& a, const uint4& b, f4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

__device__ inline float gelu_exact(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

// Spread consecutive workgroups of one XCD over a contiguous range of tiles:
// the dispatcher hands workgroup ids to the 8 XCDs round-robin, and each XCD
// has its own L2, so neighbouring tiles (which share A rows or B columns)
// should land on the same XCD.
__device__ inline int xcd_remap(int pid, int nb) {
  const int x = pid & 7, local = pid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return x * per + (x < rem ? x : rem) + local;
}

template <typename T, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  constexpr int TM = BM / WM / 16;
  constexpr int TN = BN / WN / 16;
  constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int BK = 8 * EPC;           // elements per 128-byte tile row
  constexpr int NLA = (BM * 8 + 255) / 256;
  constexpr int NLB = (BN * 8 + 255) / 256;
  static_assert(WM * WN == 4, "4 waves");

  __shared__ uint4 sA[2][BM * kPitch];
  __shared__ uint4 sB[2][BN * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int group = blockIdx.z;

  // tile coordinates: XCD-aware remap, then grouped raster (8 M-tiles per group)
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  const int pid = xcd_remap(blockIdx.x, gridDim.x);
  constexpr int GM = 8;
  const int width = GM * tiles_n;
  const int first_m = (pid / width) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (pid % width) % gsz;
  const int tn = (pid % width) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const char* Abase = (const char*)a.A + (int64_t)group * a.a_group * sizeof(T);
  const char* Bbase = (const char*)a.B + (int64_t)group * a.b_group * sizeof(T);

  // per-thread source rows of the tile loads
  const char* arow[NLA];
  bool aok[NLA];
#pragma unroll
  for (int i = 0; i < NLA; ++i) {
    const int idx = tid + 256 * i;
    const int r = idx >> 3;
    const int m = m0 + r;
    aok[i] = (idx < BM * 8) && (m < a.M);
    const int mm = aok[i] ? m : 0;
    const int seg = mm / a.seg_rows, t = mm - seg * a.seg_rows;
    arow[i] = Abase + ((int64_t)seg * a.a_seg + (int64_t)t * a.lda) * sizeof(T) + (idx & 7) * 16;
  }
  const char* brow[NLB];
  bool bok[NLB];
#pragma unroll
  for (int i = 0; i < NLB; ++i) {
    const int idx = tid + 256 * i;
    const int r = idx >> 3;
    const int n = n0 + r;
    bok[i] = (idx < BN * 8) && (n < a.N);
    brow[i] = Bbase + ((int64_t)(bok[i] ? n : 0) * a.K) * sizeof(T) + (idx & 7) * 16;
  }

  uint4 ra[NLA], rb[NLB];
  auto load = [&](int kt) {
    const int kbase = kt * BK;
#pragma unroll
    for (int i = 0; i < NLA; ++i) {
      const int idx = tid + 256 * i;
      const bool ok = aok[i] && (kbase + (idx & 7) * EPC < a.K);
      ra[i] = ok ? *(const uint4*)(arow[i] + (int64_t)kbase * sizeof(T)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NLB; ++i) {
      const int idx = tid + 256 * i;
      const bool ok = bok[i] && (kbase + (idx & 7) * EPC < a.K);
      rb[i] = ok ? *(const uint4*)(brow[i] + (int64_t)kbase * sizeof(T)) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLA; ++i) {
      const int idx = tid + 256 * i;
      if (idx < BM * 8) sA[buf][(idx >> 3) * kPitch + (idx & 7)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NLB; ++i) {
      const int idx = tid + 256 * i;
      if (idx < BN * 8) sB[buf][(idx >> 3) * kPitch + (idx & 7)] = rb[i];
    }
  };

  f4 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int nk = (a.K + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();

  const int lr = lane & 15, lg = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      uint4 wv[TN], av[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) wv[i] = sB[cur][(wn * TN * 16 + i * 16 + lr) * kPitch + cc * 4 + lg];
#pragma unroll
      for (int j = 0; j < TM; ++j) av[j] = sA[cur][(wm * TM * 16 + j * 16 + lr) * kPitch + cc * 4 + lg];
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) Mma<T>::run(wv[i], av[j], acc[i][j]);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows m, columns nb .. nb+3
  const bool vec = ((a.ldc & 3) == 0) && ((a.N & 3) == 0) && ((a.c_group & 3) == 0) &&
                   ((a.bias_group & 3) == 0);
  const float* bias = a.bias ? a.bias + (int64_t)group * a.bias_group : nullptr;
  const int64_t cg = (int64_t)group * a.c_group;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = m0 + wm * TM * 16 + j * 16 + lr;
    if (m >= a.M) continue;
    const int64_t rowoff = cg + (int64_t)m * a.ldc;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int nb = n0 + wn * TN * 16 + i * 16 + lg * 4;
      if (nb >= a.N) continue;
      f4 v = acc[i][j];
      if (vec) {
        if (bias) {
          const float4 bb = *(const float4*)(bias + nb);
          v.x += bb.x; v.y += bb.y; v.z += bb.z; v.w += bb.w;
        }
        if (a.act == 1) {
          v.x = gelu_exact(v.x); v.y = gelu_exact(v.y); v.z = gelu_exact(v.z); v.w = gelu_exact(v.w);
        }
        if (a.residual) {
          const float4 rr = *(const float4*)(a.residual + rowoff + nb);
          v.x += rr.x; v.y += rr.y; v.z += rr.z; v.w += rr.w;
        }
        if (a.out_f32) *(float4*)(a.out_f32 + rowoff + nb) = make_float4(v.x, v.y, v.z, v.w);
        if (a.out_t) {
          if constexpr (sizeof(T) == 2) {
            h4 hv = {(half_t)v.x, (half_t)v.y, (half_t)v.z, (half_t)v.w};
            *(h4*)((half_t*)a.out_t + rowoff + nb) = hv;
          } else {
            *(float4*)((float*)a.out_t + rowoff + nb) = make_float4(v.x, v.y, v.z, v.w);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = nb + r;
          if (n >= a.N) break;
          float x = v[r];
          if (bias) x += bias[n];
          if (a.act == 1) x = gelu_exact(x);
          if (a.residual) x += a.residual[rowoff + n];
          if (a.out_f32) a.out_f32[rowoff + n] = x;
          if (a.out_t) ((T*)a.out_t)[rowoff + n] = (T)x;
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int WM, int WN>
hipError_t launch_t(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN>), dim3(tiles, 1, a.groups), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dispatch(const GemmArgs& a, hipStream_t s) {
  if (a.N <= 32) return launch_t<T, 128, 32, 4, 1>(a, s);
  if (a.N <= 48) return launch_t<T, 128, 48, 4, 1>(a, s);
  if (a.N <= 64) return launch_t<T, 128, 64, 4, 1>(a, s);
  return launch_t<T, 128, 128, 2, 2>(a, s);
}

}  // namespace

hipError_t launch_gemm(DType t, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0 || a.groups <= 0) return hipSuccess;
  return t == DType::F16 ? launch_dispatch<half_t>(a, s) : launch_dispatch<float>(a, s);
}

}  // namespace w2v2
