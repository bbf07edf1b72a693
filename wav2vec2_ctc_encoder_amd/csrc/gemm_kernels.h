// MFMA GEMM kernels for gfx950 with a row-mapped A operand and a fused epilogue.
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
// Three kernels, all 256 threads = 4 waves with the weight as the MFMA A
// operand (n side) and the activation as the B operand (m side), so a lane
// holds consecutive output columns of one row:
//
// gemm_dlds_kernel (fp16, K % 64 == 0, N > 32; the hot path): block tile
//   128x128 or 128x64, waves 2 x 2, v_mfma_f32_32x32x16_f16.  K advances in
//   64-wide steps through two LDS buffers filled by wave-wide direct
//   global->LDS loads (global_load_lds_dwordx4, 16 bytes per lane) into
//   XOR-swizzled 128-byte rows; explicit vmcnt waits, one barrier per step.
//   All MFMA fragments of the next step are read from LDS into registers
//   while the current step's MFMAs run, so no MFMA waits on an LDS read.
//   Epilogue: bias and activation in registers, then each wave stages its
//   32-row slabs row-major in LDS and writes whole rows (residual add, fp32
//   and/or fp16 stores), because the 32x32 accumulator layout would
//   otherwise scatter 16-byte pieces over 32 rows per store.
//
// gemm_deep_kernel (fp16 products with K >= 2048 and at most one 128x128
//   tile per CU: the half-batch FFN2): the same tile and fragment pipeline
//   with one workgroup per CU, four LDS stages (three in flight) and the
//   loads of each step spread one per two MFMAs.
//
// gemm_kernel (fp32 mode and the remaining shapes): block tile BM x BN, K
//   step of 128 bytes per row (64 fp16 / 32 fp32), double-buffered LDS with
//   the next K step prefetched into registers, one barrier per step; each
//   wave owns a (TN*16) x (TM*16) sub-tile of 16x16 MFMA blocks and stores
//   16-byte (fp32) / 8-byte (fp16) vectors.
//   fp16: v_mfma_f32_16x16x32_f16, one per 16-byte lane fragment.
//   fp32: v_mfma_f32_16x16x4_f32, four per 16-byte lane fragment; fragment
//         element j of lane group g carries k = 4g + j for both operands, a
//         permutation of the 16 k values, so the sum is unchanged.
//
// A rows come from the segment rule above or, for packed true-length rows,
// from a per-row offset table; output rows likewise (c_rows).
//
// This header holds the kernels and their launch shapes; every GEMM role is
// instantiated in its own translation unit (gemm_role_*.hip), so the roles
// compile in parallel.
#pragma once
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



// Spread consecutive workgroups of one XCD over a contiguous range of tiles:
// the dispatcher hands workgroup ids to the 8 XCDs round-robin, and each XCD
// has its own L2, so neighbouring tiles (which share A rows or B columns)
// should land on the same XCD.
__device__ inline int xcd_remap(int pid, int nb) {
  const int x = pid & 7, local = pid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return x * per + (x < rem ? x : rem) + local;
}

// Residual element(s) of logical row m. With res_stats set, the residual
// buffer holds a raw sum whose LayerNorm (row statistics res_stats[m], affine
// res_gamma/res_beta) is applied here as it is read.
__device__ inline float4 residual4(const GemmArgs& a, int m, int n, const float* r) {
  float4 v = *(const float4*)r;
  if (a.res_stats) {
    const float2 st = a.res_stats[m];
    const float4 g = *(const float4*)(a.res_gamma + n), b = *(const float4*)(a.res_beta + n);
    v.x = (v.x - st.x) * st.y * g.x + b.x;
    v.y = (v.y - st.x) * st.y * g.y + b.y;
    v.z = (v.z - st.x) * st.y * g.z + b.z;
    v.w = (v.w - st.x) * st.y * g.w + b.w;
  }
  return v;
}
__device__ inline float residual1(const GemmArgs& a, int m, int n, float r) {
  if (a.res_stats) {
    const float2 st = a.res_stats[m];
    r = (r - st.x) * st.y * a.res_gamma[n] + a.res_beta[n];
  }
  return r;
}

// Epilogue for 4 consecutive output columns nb..nb+3 of row m:
// v = acc + bias; v = act(v); v += residual; store fp32 and/or operand type.
// Returns the values stored (entries of columns >= N are unspecified).
template <typename T, int ACT>
__device__ inline f4 epilogue4(const GemmArgs& a, const float* bias, int m, int64_t rowoff, int nb, f4 v,
                               bool vec) {
  if (a.col_scale) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] *= a.col_scale[min(nb + r, a.N - 1)];
  }
  if (vec) {
    if (bias) {
      const float4 bb = *(const float4*)(bias + nb);
      v.x += bb.x; v.y += bb.y; v.z += bb.z; v.w += bb.w;
    }
    v.x = act_fn<ACT>(v.x); v.y = act_fn<ACT>(v.y); v.z = act_fn<ACT>(v.z); v.w = act_fn<ACT>(v.w);
    if (a.residual) {
      const float4 rr = residual4(a, m, nb, a.residual + rowoff + nb);
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
      x = act_fn<ACT>(x);
      if (a.residual) x += residual1(a, m, n, a.residual[rowoff + n]);
      if (a.out_f32) a.out_f32[rowoff + n] = x;
      if (a.out_t) ((T*)a.out_t)[rowoff + n] = (T)x;
      v[r] = x;
    }
  }
  return v;
}

// Largest |v| over the valid columns nb..nb+3.
__device__ inline float abs_max4(const f4& v, int nb, int N, float mx) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (nb + r < N) mx = fmaxf(mx, fabsf(v[r]));
  return mx;
}

// Largest argmax key over the valid columns nb..nb+3 of one row's values.
__device__ inline uint64_t best_key4(const f4& v, int nb, int N, uint64_t k) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t c = argmax_key(v[r], nb + r);
    if (nb + r < N && c > k) k = c;
  }
  return k;
}
// Output row of logical row m (the argmax slot of that row).
__device__ inline int64_t amax_row(const GemmArgs& a, int m) { return a.c_rows ? a.c_rows[m] / a.ldc : m; }

template <int N>
struct ActTag {
  static constexpr int value = N;
};

// Element offset of A row m (before the group offset) and of output row m.
__device__ inline int64_t a_row_offset(const GemmArgs& a, int m) {
  if (a.a_rows) return a.a_rows[m];
  const int seg = m / a.seg_rows, t = m - seg * a.seg_rows;
  return (int64_t)seg * a.a_seg + (int64_t)t * a.lda;
}
__device__ inline int64_t c_row_offset(const GemmArgs& a, int m) {
  return a.c_rows ? a.c_rows[m] : (int64_t)m * a.ldc;
}

__device__ inline bool epilogue_vec_ok(const GemmArgs& a) {
  return ((a.ldc & 3) == 0) && ((a.N & 3) == 0) && ((a.c_group & 3) == 0) && ((a.bias_group & 3) == 0);
}

typedef float f16x __attribute__((ext_vector_type(16)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));

// Whole 8-column chunks everywhere: the staged epilogue below stores 16 B of
// fp16 (32 B of fp32) per lane.
__device__ inline bool epilogue_staged_ok(const GemmArgs& a) {
  const uintptr_t ptrs = (uintptr_t)a.out_t | (uintptr_t)a.out_f32 | (uintptr_t)a.residual | (uintptr_t)a.bias |
                         (uintptr_t)a.res_gamma | (uintptr_t)a.res_beta;
  return ((a.ldc & 7) == 0) && ((a.N & 7) == 0) && ((a.c_group & 7) == 0) && ((a.bias_group & 7) == 0) &&
         ((ptrs & 15) == 0);
}

// Epilogue of one wave's (TM*32) x (TN*32) block of 32x32 MFMA accumulators
// (lane l holds, for block (i, j), rows m = j*32 + l%32 and the 4 columns
// n = i*32 + 8q + 4*(l/32) + 0..3 in elements 4q..4q+3).  That layout makes
// direct stores scatter 16-byte pieces over 32 rows per instruction, so each
// 32-row slab goes through the wave's own LDS region instead: bias and the
// activation are applied in registers, the slab is written row-major (row
// pitch padded by 16 bytes to spread the rows over the banks) and read back
// with LPR consecutive lanes covering one row, so the residual loads and the
// output stores move whole contiguous rows.  LDS operations of one wave run in
// order, so no barrier is needed between the write and the read-back.
// NT: non-temporal output stores (conv outputs: hundreds of MB written once
// and read once by the next layer; keeping them out of the caches leaves the
// L2 to the operand tiles).
// F8: the fp8 kernel's epilogue (per-column scales, optional e4m3 output);
// other instantiations carry neither.
template <int TM, int TN, int ACT, bool NT, bool F8 = false>
__device__ inline void epilogue_staged(const GemmArgs& a, f16x (&acc)[TN][TM], float* stage, int m_base,
                                       int n_base, int group, const float* sbias = nullptr, int n0t = 0) {
  constexpr int W = TN * 32;     // columns of the wave block
  constexpr int P = W + 4;       // padded row pitch (floats)
  constexpr int LPR = W / 8;     // lanes per row in the read-back
  constexpr int RPP = 64 / LPR;  // rows per read-back pass
  constexpr int NPS = 32 / RPP;  // read-back passes per 32-row slab
  const int lane = threadIdx.x & 63, l32 = lane & 31, lg = lane >> 5;
  const float* bias = a.bias ? a.bias + (int64_t)group * a.bias_group : nullptr;
  const int64_t cg = (int64_t)group * a.c_group;
  const int rrow = lane / LPR, rcol = (lane % LPR) * 8;
  // Operands that do not depend on the row are loaded once, and every load
  // goes to a clamped in-bounds address without a branch, so the loads issue
  // together instead of each waiting behind the math of the previous chunk
  // (N % 8 == 0 here; values of clamped columns or rows are never stored).
  float4 bv[TN][4], cv[F8 ? TN : 1][4];
  const float* cscale = a.col_scale ? a.col_scale + (int64_t)group * a.bias_group : nullptr;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nc = min(n_base + i * 32 + 8 * q + 4 * lg, a.N - 4);
      bv[i][q] = sbias  ? *(const float4*)(sbias + (nc - n0t))
                 : bias ? *(const float4*)(bias + nc) : make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (F8) cv[i][q] = cscale ? *(const float4*)(cscale + nc) : make_float4(1.f, 1.f, 1.f, 1.f);
    }
  float vmax = 0.f;  // calibration: max |stored value| of this lane
  const int nr = min(n_base + rcol, a.N - 8);  // the lane's 8 read-back columns
  float4 g0 = make_float4(0.f, 0.f, 0.f, 0.f), g1 = g0, e0 = g0, e1 = g0;
  if (a.res_stats) {
    g0 = *(const float4*)(a.res_gamma + nr);
    g1 = *(const float4*)(a.res_gamma + nr + 4);
    e0 = *(const float4*)(a.res_beta + nr);
    e1 = *(const float4*)(a.res_beta + nr + 4);
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    // this slab's residual rows, requested before its activation math
    float4 r0[NPS], r1[NPS];
    float2 rs[NPS];
    if (a.residual) {
#pragma unroll
      for (int ps = 0; ps < NPS; ++ps) {
        const int m = min(m_base + j * 32 + ps * RPP + rrow, a.M - 1);
        const float* r = a.residual + cg + c_row_offset(a, m) + nr;
        r0[ps] = *(const float4*)r;
        r1[ps] = *(const float4*)(r + 4);
        rs[ps] = a.res_stats ? a.res_stats[m] : make_float2(0.f, 1.f);
      }
    }
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = i * 32 + 8 * q + 4 * lg;
        float4 v;
        if constexpr (F8) {
          v = make_float4(fmaf(acc[i][j][4 * q], cv[i][q].x, bv[i][q].x),
                          fmaf(acc[i][j][4 * q + 1], cv[i][q].y, bv[i][q].y),
                          fmaf(acc[i][j][4 * q + 2], cv[i][q].z, bv[i][q].z),
                          fmaf(acc[i][j][4 * q + 3], cv[i][q].w, bv[i][q].w));
        } else {
          v = make_float4(acc[i][j][4 * q] + bv[i][q].x, acc[i][j][4 * q + 1] + bv[i][q].y,
                          acc[i][j][4 * q + 2] + bv[i][q].z, acc[i][j][4 * q + 3] + bv[i][q].w);
        }
        v.x = act_fn<ACT>(v.x); v.y = act_fn<ACT>(v.y); v.z = act_fn<ACT>(v.z); v.w = act_fn<ACT>(v.w);
        *(float4*)(stage + l32 * P + nl) = v;
      }
    }
#pragma unroll
    for (int ps = 0; ps < NPS; ++ps) {
      const int row = ps * RPP + rrow;
      const int m = m_base + j * 32 + row, n = n_base + rcol;
      float4 x0 = *(const float4*)(stage + row * P + rcol);
      float4 x1 = *(const float4*)(stage + row * P + rcol + 4);
      if (a.residual) {
        float4 u0 = r0[ps], u1 = r1[ps];
        if (a.res_stats) {
          // the residual's LayerNorm: (r - mean) * rstd * gamma + beta
          const float mu = rs[ps].x, rstd = rs[ps].y;
          u0.x = (u0.x - mu) * rstd * g0.x + e0.x; u0.y = (u0.y - mu) * rstd * g0.y + e0.y;
          u0.z = (u0.z - mu) * rstd * g0.z + e0.z; u0.w = (u0.w - mu) * rstd * g0.w + e0.w;
          u1.x = (u1.x - mu) * rstd * g1.x + e1.x; u1.y = (u1.y - mu) * rstd * g1.y + e1.y;
          u1.z = (u1.z - mu) * rstd * g1.z + e1.z; u1.w = (u1.w - mu) * rstd * g1.w + e1.w;
        }
        x0.x += u0.x; x0.y += u0.y; x0.z += u0.z; x0.w += u0.w;
        x1.x += u1.x; x1.y += u1.y; x1.z += u1.z; x1.w += u1.w;
      }
      if (a.amax) {
        // the LPR consecutive lanes of this row hold its columns of the wave's block
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint64_t key = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint64_t c = argmax_key(xv[e], n + e);
          if (n + e < a.N && c > key) key = c;
        }
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) key = max_key_xor(key, o);
        if (m < a.M && (lane % LPR) == 0)
          atomicMax((unsigned long long*)(a.amax + amax_row(a, m)), (unsigned long long)key);
      }
      if (a.out_amax && m < a.M && n < a.N)
        vmax = fmaxf(vmax, fmaxf(fmaxf(fmaxf(fabsf(x0.x), fabsf(x0.y)), fmaxf(fabsf(x0.z), fabsf(x0.w))),
                                 fmaxf(fmaxf(fabsf(x1.x), fabsf(x1.y)), fmaxf(fabsf(x1.z), fabsf(x1.w)))));
      if (m < a.M && n < a.N) {
        const int64_t off = cg + c_row_offset(a, m) + n;
        if (F8 && a.out_f8) {
          const uint2 b8 = make_uint2(pack_e4m3x4(x0.x, x0.y, x0.z, x0.w, a.out_f8_inv),
                                      pack_e4m3x4(x1.x, x1.y, x1.z, x1.w, a.out_f8_inv));
          *(uint2*)(a.out_f8 + off) = b8;
        }
        if (a.out_f32) {
          const f4 v0 = {x0.x, x0.y, x0.z, x0.w}, v1 = {x1.x, x1.y, x1.z, x1.w};
          if constexpr (NT) {
            __builtin_nontemporal_store(v0, (f4*)(a.out_f32 + off));
            __builtin_nontemporal_store(v1, (f4*)(a.out_f32 + off + 4));
          } else {
            *(f4*)(a.out_f32 + off) = v0;
            *(f4*)(a.out_f32 + off + 4) = v1;
          }
        }
        if (F8 && a.out_t && a.out_t_f32) {
          const f4 v0 = {x0.x, x0.y, x0.z, x0.w}, v1 = {x1.x, x1.y, x1.z, x1.w};
          *(f4*)((float*)a.out_t + off) = v0;
          *(f4*)((float*)a.out_t + off + 4) = v1;
        } else if (a.out_t) {
          const h8v hv = {(half_t)x0.x, (half_t)x0.y, (half_t)x0.z, (half_t)x0.w,
                          (half_t)x1.x, (half_t)x1.y, (half_t)x1.z, (half_t)x1.w};
          if constexpr (NT) __builtin_nontemporal_store(hv, (h8v*)((half_t*)a.out_t + off));
          else *(h8v*)((half_t*)a.out_t + off) = hv;
        }
      }
    }
  }
  if (a.out_amax) wave_raise_amax(vmax, a.out_amax);
}

template <typename T, int BM, int BN, int WM, int WN, int ROLE>
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
    arow[i] = Abase + a_row_offset(a, mm) * sizeof(T) + (idx & 7) * 16;
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
  const bool vec = epilogue_vec_ok(a);
  const float* bias = a.bias ? a.bias + (int64_t)group * a.bias_group : nullptr;
  const int64_t cg = (int64_t)group * a.c_group;
  float vmax = 0.f;
  auto store_all = [&](auto act_tag) {
    constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + wm * TM * 16 + j * 16 + lr;
      uint64_t key = 0;
      if (m < a.M) {
        const int64_t rowoff = cg + c_row_offset(a, m);
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          const int nb = n0 + wn * TN * 16 + i * 16 + lg * 4;
          if (nb < a.N) {
            const f4 v = epilogue4<T, ACT>(a, bias, m, rowoff, nb, acc[i][j], vec);
            key = best_key4(v, nb, a.N, key);
            vmax = abs_max4(v, nb, a.N, vmax);
          }
        }
      }
      if (a.amax) {
        // the 4 lanes (lg) of row m hold its columns of this wave's block
        key = max_key_xor(max_key_xor(key, 16), 32);
        if (m < a.M && lg == 0) atomicMax((unsigned long long*)(a.amax + amax_row(a, m)), (unsigned long long)key);
      }
    }
  };
  if (a.act == 1) store_all(ActTag<1>{});
  else if (a.act == 2) store_all(ActTag<2>{});
  else store_all(ActTag<0>{});
  if (a.out_amax) wave_raise_amax(vmax, a.out_amax);
}

// One wave-wide direct global->LDS load: lane l's 16 bytes at gptr land at
// LDS byte address lds + 16*l.  Written as inline asm so that the compiler's
// wait-count pass does not treat every later LDS read as dependent on it (it
// would wait for all outstanding loads, serialising the pipeline); the
// kernel waits on vmcnt explicitly.  The instruction has no result register;
// its LDS base is an input bound to m0, so the compiler itself sets m0.
__device__ inline void dma16(const void* gptr, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds) : "memory");
}
// The same with 4 bytes per lane (lane l's dword lands at lds + 4*l).
__device__ inline void dma4(const void* gptr, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(lds) : "memory");
}

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left at their maxima (no wait).
// Encoding (gfx9): vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ inline void wait_vmcnt_imm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0): every LDS read of this wave has returned.
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8)); }

typedef int v8i __attribute__((ext_vector_type(8)));

// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands e4m3 and unit block
// scales (E8M0 127 = 2^0): a 32x32 block, K = 64; lane l supplies row l % 32
// and 32 of the 64 k values (two 16-byte chunks each for the weight and the
// activation fragment).
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ inline f16x mfma_f8(uint4 w0, uint4 w1, uint4 x0, uint4 x1, f16x c) {
  const v8i wv = __builtin_shufflevector(__builtin_bit_cast(v4i, w0), __builtin_bit_cast(v4i, w1), 0, 1, 2, 3, 4, 5,
                                         6, 7);
  const v8i xv = __builtin_shufflevector(__builtin_bit_cast(v4i, x0), __builtin_bit_cast(v4i, x1), 0, 1, 2, 3, 4, 5,
                                         6, 7);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, xv, c, 0, 0, 0, 127, 0, 127);
}

// WPE: waves per SIMD the register budget is fitted to (2 for 128x128 tiles,
// 3 for 128x64, which LDS also allows: 64 / 48 KB per workgroup).
// F8: e4m3 operands (fp8 mode projections): a 128-byte tile row then holds
// 128 k values, the step is two K = 64 MFMA slices, and each 32-row fragment
// of a slice is two 16-byte chunks per lane (the same 4 chunk reads per
// block and step as the fp16 kernel's four K = 16 slices).
template <int BM, int BN, int ROLE, int WPE, bool F8 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void gemm_dlds_kernel(GemmArgs a) {
  constexpr int WM = 2, WN = 2;
  constexpr int TM = BM / WM / 32;  // 32x32 blocks per wave along m
  constexpr int TN = BN / WN / 32;  // ... along n
  constexpr int ES = F8 ? 1 : 2;    // operand bytes
  constexpr int CPR = 8;            // 16-byte chunks per tile row: 128 bytes of K per step
  constexpr int RPI = 64 / CPR;     // tile rows per 1 KB wave load
  constexpr int KEYDIV = 16 / CPR;  // rows sharing a bank-group phase
  constexpr int KS = F8 ? 2 : 4;    // MFMA K slices per step (64-wide fp8, 16-wide fp16)
  constexpr int NF = 4;             // 16-byte fragment chunks per 32-row block per step
  constexpr int JA = BM / RPI / 4;  // 1 KB load instructions per wave per step (A)
  constexpr int JB = BN / RPI / 4;  // (B)
  constexpr int LPS = JA + JB;      // loads per thread per step
  constexpr int ABUF = BM * CPR, BBUF = BN * CPR;  // uint4 per buffer
  static_assert(TM >= 1 && TN >= 1 && JA >= 1 && JB >= 1 && LPS <= 63, "tile");

  // [A buffer 0][A buffer 1][B buffer 0][B buffer 1]; the epilogue reuses all of it
  __shared__ uint4 smem[2 * (ABUF + BBUF)];
  static_assert(4 * 32 * (TN * 32 + 4) * 4 <= 2 * (ABUF + BBUF) * 16, "epilogue staging fits");
  // the tile's bias columns, brought in with the first K step's loads
  __shared__ float sbias[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int group = blockIdx.z;

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

  const char* Abase = (const char*)a.A + (int64_t)group * a.a_group * ES;
  const char* Bbase = (const char*)a.B + (int64_t)group * a.b_group * ES;

  // source rows (clamped) with the swizzled chunk folded in: LDS chunk p of
  // tile row r holds source chunk p ^ key(r)
  const int pos = lane & (CPR - 1);
  const char* asrc[JA];
#pragma unroll
  for (int j = 0; j < JA; ++j) {
    const int r = (wave * JA + j) * RPI + lane / CPR;
    const int m = min(m0 + r, a.M - 1);
    asrc[j] = Abase + a_row_offset(a, m) * ES + ((pos ^ ((r / KEYDIV) & (CPR - 1))) << 4);
  }
  const char* bsrc[JB];
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int r = (wave * JB + j) * RPI + lane / CPR;
    const int n = min(n0 + r, a.N - 1);
    bsrc[j] = Bbase + (int64_t)n * a.K * ES + ((pos ^ ((r / KEYDIV) & (CPR - 1))) << 4);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)&smem[0];
  auto issue = [&](int kt, int buf) {
    const int64_t koff = (int64_t)kt * 128;
#pragma unroll
    for (int j = 0; j < JA; ++j)
      dma16(asrc[j] + koff,
            __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((buf * ABUF + (wave * JA + j) * 64) * 16)));
#pragma unroll
    for (int j = 0; j < JB; ++j)
      dma16(bsrc[j] + koff,
            __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((2 * ABUF + buf * BBUF + (wave * JB + j) * 64) * 16)));
  };

  // per-lane LDS offsets (uint4 units, buffer 0) of every fragment chunk of a
  // step: operand lane l holds row l % 32; fp16 (32x32x16): fragment f is
  // chunk 2f + l/32; fp8 (32x32x64): slice f/2 spans chunks 4(f/2) .. +3, and
  // lane group l/32 takes two of them (f % 2 selects which)
  const int l32 = lane & 31, lg = lane >> 5;
  int aoff[NF][TM], boff[NF][TN];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int ch = F8 ? (4 * (f >> 1) + 2 * lg + (f & 1)) : (2 * f + lg);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int R = wm * TM * 32 + j * 32 + l32;
      aoff[f][j] = R * CPR + (ch ^ ((R / KEYDIV) & (CPR - 1)));
    }
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int R = wn * TN * 32 + i * 32 + l32;
      boff[f][i] = 2 * ABUF + R * CPR + (ch ^ ((R / KEYDIV) & (CPR - 1)));
    }
  }

  f16x acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // two register sets of a whole step's fragments, alternating by step parity
  uint4 fa0[NF][TM], fb0[NF][TN], fa1[NF][TM], fb1[NF][TN];
  auto read_frags = [&](int buf, uint4 (&fa)[NF][TM], uint4 (&fb)[NF][TN]) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
      for (int i = 0; i < TN; ++i) fb[f][i] = smem[boff[f][i] + buf * BBUF];
#pragma unroll
      for (int j = 0; j < TM; ++j) fa[f][j] = smem[aoff[f][j] + buf * ABUF];
    }
  };
  const int nk = a.K / (F8 ? 128 : 64);
  // Step kt: the fragments of kt are in (fac, fbc) and buffer kt & 1 is no
  // longer read by this wave.  Wait for this wave's loads of step kt + 1 (the
  // only ones in flight); after the barrier every wave's have landed and
  // every wave holds its step-kt fragments, so buffer kt & 1 may be refilled
  // with step kt + 2 while the MFMAs of kt run interleaved with the reads of
  // kt + 1.  That read is unconditional (one basic block for the scheduler):
  // past the last step it reads a stale, in-bounds buffer and is never used.
  auto step = [&](int kt, int bcur, uint4 (&fac)[NF][TM], uint4 (&fbc)[NF][TN], uint4 (&fan)[NF][TM],
                  uint4 (&fbn)[NF][TN]) {
    wait_vmcnt_imm<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + 2 < nk) issue(kt + 2, bcur);
    read_frags(bcur ^ 1, fan, fbn);
    if constexpr (F8) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j)
            acc[i][j] = mfma_f8(fbc[2 * ks][i], fbc[2 * ks + 1][i], fac[2 * ks][j], fac[2 * ks + 1][j], acc[i][j]);
      // each MFMA followed by its share of the next step's LDS reads
      constexpr int NM = KS * TM * TN, NR = NF * (TM + TN), RPM = (NR + NM - 1) / NM;
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, fbc[ks][i]),
                                                               __builtin_bit_cast(h8, fac[ks][j]), acc[i][j], 0, 0, 0);
      // one MFMA, one LDS read, alternately; the remaining MFMAs after
#pragma unroll
      for (int q = 0; q < KS * (TM + TN); ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KS * TM * TN - KS * (TM + TN), 0);
    }
    wait_lgkm0();
  };

  const float* biasg = a.bias ? a.bias + (int64_t)group * a.bias_group : nullptr;
  if constexpr (!F8) {
    // wave 0's loads complete in order, so the wait for step 0 below covers these too
    if (biasg && wave == 0) {
#pragma unroll
      for (int h = 0; h < BN / 64; ++h)
        dma4(biasg + min(n0 + h * 64 + lane, a.N - 1),
             __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&sbias[h * 64]));
    }
  }
  issue(0, 0);
  if (nk > 1) {
    issue(1, 1);
    wait_vmcnt_imm<LPS>();
  } else {
    wait_vmcnt_imm<0>();
  }
  __builtin_amdgcn_s_barrier();
  read_frags(0, fa0, fb0);
  wait_lgkm0();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, 0, fa0, fb0, fa1, fb1);
    step(kt + 1, 1, fa1, fb1, fa0, fb0);
  }
  if (kt < nk) step(kt, 0, fa0, fb0, fa1, fb1);

  constexpr bool NT = ROLE == kGemmConv;
  if (epilogue_staged_ok(a)) {
    // every wave is done reading the buffers before any overwrites them
    __builtin_amdgcn_s_barrier();
    float* stage = reinterpret_cast<float*>(smem) + wave * 32 * (TN * 32 + 4);
    const int m_base = m0 + wm * TM * 32, n_base = n0 + wn * TN * 32;
    const float* sb = (!F8 && biasg) ? sbias : nullptr;
    if (a.act == 1) epilogue_staged<TM, TN, 1, NT, F8>(a, acc, stage, m_base, n_base, group, sb, n0);
    else if (a.act == 2) epilogue_staged<TM, TN, 2, NT, F8>(a, acc, stage, m_base, n_base, group, sb, n0);
    else epilogue_staged<TM, TN, 0, NT, F8>(a, acc, stage, m_base, n_base, group, sb, n0);
    return;
  }
  const bool vec = epilogue_vec_ok(a);
  const float* bias = a.bias ? a.bias + (int64_t)group * a.bias_group : nullptr;
  const int64_t cg = (int64_t)group * a.c_group;
  float vmax = 0.f;
  auto store_all = [&](auto act_tag) {
    constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + wm * TM * 32 + j * 32 + l32;
      uint64_t key = 0;
      if (m < a.M) {
        const int64_t rowoff = cg + c_row_offset(a, m);
#pragma unroll
        for (int i = 0; i < TN; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nb = n0 + wn * TN * 32 + i * 32 + 8 * q + 4 * lg;
            if (nb < a.N) {
              const f4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              const f4 o = epilogue4<half_t, ACT>(a, bias, m, rowoff, nb, v, vec);
              key = best_key4(o, nb, a.N, key);
              vmax = abs_max4(o, nb, a.N, vmax);
            }
          }
        }
      }
      if (a.amax) {
        // lanes l32 and l32 + 32 hold row m's columns of this wave's block
        key = max_key_xor(key, 32);
        if (m < a.M && lg == 0) atomicMax((unsigned long long*)(a.amax + amax_row(a, m)), (unsigned long long)key);
      }
    }
  };
  if (a.act == 1) store_all(ActTag<1>{});
  else if (a.act == 2) store_all(ActTag<2>{});
  else store_all(ActTag<0>{});
  if (a.out_amax) wave_raise_amax(vmax, a.out_amax);
}


// Long-K products with at most one 128x128 tile per CU (the half-batch FFN2:
// 150 tiles, K = 3072): one workgroup per CU, four LDS stages with three in
// flight, and each step's eight loads spread one per two MFMAs, so the wave
// never stalls behind a burst of load issues.  Every step issues its loads
// (past the last stage they reload stage nk - 1 into the buffer just
// vacated, which nobody reads again), so the wait before a step is always
// "all but the last two stages".
template <int ROLE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_deep_kernel(GemmArgs a) {
  constexpr int BM = 128, BN = 128, WN = 2, S = 4;
  constexpr int TM = 2, TN = 2;
  constexpr int CPR = 8, RPI = 8, KEYDIV = 2, KS = 4, NF = 4;
  constexpr int JA = BM / RPI / 4, JB = BN / RPI / 4, LPS = JA + JB;
  constexpr int ABUF = BM * CPR, BBUF = BN * CPR;
  static_assert(LPS == 8, "shape");

  __shared__ uint4 smem[S * (ABUF + BBUF)];
  __shared__ float sbias[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

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

  const int pos = lane & (CPR - 1);
  const char* asrc[JA];
#pragma unroll
  for (int j = 0; j < JA; ++j) {
    const int r = (wave * JA + j) * RPI + lane / CPR;
    const int m = min(m0 + r, a.M - 1);
    asrc[j] = (const char*)a.A + a_row_offset(a, m) * 2 + ((pos ^ ((r / KEYDIV) & (CPR - 1))) << 4);
  }
  const char* bsrc[JB];
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int r = (wave * JB + j) * RPI + lane / CPR;
    const int n = min(n0 + r, a.N - 1);
    bsrc[j] = (const char*)a.B + (int64_t)n * a.K * 2 + ((pos ^ ((r / KEYDIV) & (CPR - 1))) << 4);
  }
  const int nk = a.K / 64;
  const uint32_t lds0 = (uint32_t)(uintptr_t)&smem[0];
  // load d (0..7) of stage min(kt, nk - 1) into buffer buf
  auto issue_one = [&](int kt, int buf, int d) {
    const int64_t koff = (int64_t)min(kt, nk - 1) * 128;
    if (d < JA)
      dma16(asrc[d] + koff, __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((buf * ABUF + (wave * JA + d) * 64) * 16)));
    else
      dma16(bsrc[d - JA] + koff, __builtin_amdgcn_readfirstlane(
                                     lds0 + (uint32_t)((S * ABUF + buf * BBUF + (wave * JB + d - JA) * 64) * 16)));
  };

  const int l32 = lane & 31, lg = lane >> 5;
  int aoff[NF][TM], boff[NF][TN];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int ch = 2 * f + lg;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int R = wm * TM * 32 + j * 32 + l32;
      aoff[f][j] = R * CPR + (ch ^ ((R / KEYDIV) & (CPR - 1)));
    }
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int R = wn * TN * 32 + i * 32 + l32;
      boff[f][i] = S * ABUF + R * CPR + (ch ^ ((R / KEYDIV) & (CPR - 1)));
    }
  }

  f16x acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint4 fa0[NF][TM], fb0[NF][TN], fa1[NF][TM], fb1[NF][TN];
  auto read_frags = [&](int buf, uint4 (&fa)[NF][TM], uint4 (&fb)[NF][TN]) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
      for (int i = 0; i < TN; ++i) fb[f][i] = smem[boff[f][i] + buf * BBUF];
#pragma unroll
      for (int j = 0; j < TM; ++j) fa[f][j] = smem[aoff[f][j] + buf * ABUF];
    }
  };
  // step kt (buffer b of stage kt; its fragments are in (fac, fbc)): stage
  // kt + 1 has landed once all but the last two stages' loads are in; after
  // the barrier buffer b is refilled with stage kt + S, one load per two
  // MFMAs, while stage kt + 1's fragments are read between the MFMAs
  auto step = [&](int kt, int b, int bn, uint4 (&fac)[NF][TM], uint4 (&fbc)[NF][TN], uint4 (&fan)[NF][TM],
                  uint4 (&fbn)[NF][TN]) {
    wait_vmcnt_imm<(S - 2) * LPS>();
    __builtin_amdgcn_s_barrier();
    int d = 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = t / TM, j = t % TM;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, fbc[ks][i]),
                                                           __builtin_bit_cast(h8, fac[ks][j]), acc[i][j], 0, 0, 0);
        if ((t & 1) == 0) {
          issue_one(kt + S, b, d);
          ++d;
        }
        if (t < TN) fbn[ks][t] = smem[boff[ks][t] + bn * BBUF];
        else fan[ks][t - TN] = smem[aoff[ks][t - TN] + bn * ABUF];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_lgkm0();
  };

  if (a.bias && wave == 0) {
#pragma unroll
    for (int h = 0; h < BN / 64; ++h)
      dma4(a.bias + min(n0 + h * 64 + lane, a.N - 1), __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&sbias[h * 64]));
  }
#pragma unroll
  for (int st = 0; st < S; ++st)
#pragma unroll
    for (int d = 0; d < LPS; ++d) issue_one(st, st, d);
  wait_vmcnt_imm<(S - 2) * LPS>();  // stages 0 and 1
  __builtin_amdgcn_s_barrier();
  read_frags(0, fa0, fb0);
  wait_lgkm0();
  int kt = 0, b = 0;
  for (; kt + 1 < nk; kt += 2) {
    const int b1 = b + 1 == S ? 0 : b + 1;
    const int b2 = b1 + 1 == S ? 0 : b1 + 1;
    step(kt, b, b1, fa0, fb0, fa1, fb1);
    step(kt + 1, b1, b2, fa1, fb1, fa0, fb0);
    b = b2;
  }
  if (kt < nk) step(kt, b, b + 1 == S ? 0 : b + 1, fa0, fb0, fa1, fb1);
  // the tail's reloads land in buffers the epilogue reuses
  wait_vmcnt_imm<0>();
  __builtin_amdgcn_s_barrier();

  constexpr bool NT = ROLE == kGemmConv;
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * (TN * 32 + 4);
  const int m_base = m0 + wm * TM * 32, n_base = n0 + wn * TN * 32;
  const float* sb = a.bias ? sbias : nullptr;
  if (a.act == 1) epilogue_staged<TM, TN, 1, NT>(a, acc, stage, m_base, n_base, 0, sb, n0);
  else if (a.act == 2) epilogue_staged<TM, TN, 2, NT>(a, acc, stage, m_base, n_base, 0, sb, n0);
  else epilogue_staged<TM, TN, 0, NT>(a, acc, stage, m_base, n_base, 0, sb, n0);
}

inline bool epilogue_staged_ok_host(const GemmArgs& a) {
  const uintptr_t ptrs = (uintptr_t)a.out_t | (uintptr_t)a.out_f32 | (uintptr_t)a.residual | (uintptr_t)a.bias |
                         (uintptr_t)a.res_gamma | (uintptr_t)a.res_beta;
  return ((a.ldc & 7) == 0) && ((a.N & 7) == 0) && ((a.c_group & 7) == 0) && ((a.bias_group & 7) == 0) &&
         ((ptrs & 15) == 0) && !a.amax && !a.out_amax;
}

template <typename T, int BM, int BN, int WM, int WN, int ROLE>
hipError_t launch_t(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, ROLE>), dim3(tiles, 1, a.groups), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int ROLE, int WPE, bool F8 = false>
hipError_t launch_dlds(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_dlds_kernel<BM, BN, ROLE, WPE, F8>), dim3(tiles, 1, a.groups), dim3(256), 0, s, a);
  return hipGetLastError();
}

// fp8 mode projections: e4m3 operands, whole 128-wide K steps, and the
// staged epilogue (the only one that writes e4m3 output).
template <int ROLE>
hipError_t launch_f8(const GemmArgs& a, hipStream_t s) {
  const uintptr_t ptrs = (uintptr_t)a.out_t | (uintptr_t)a.out_f32 | (uintptr_t)a.residual | (uintptr_t)a.bias |
                         (uintptr_t)a.res_gamma | (uintptr_t)a.res_beta | (uintptr_t)a.col_scale |
                         (uintptr_t)a.out_f8;
  if (a.K % 128 || a.N % 8 || a.ldc % 8 || a.c_group % 8 || a.bias_group % 8 || (ptrs & 15) || a.amax)
    return hipErrorInvalidValue;
  const int64_t tiles128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128) * a.groups;
  if (a.N > 64 && (tiles128 >= 400 || (a.K >= 2048 && tiles128 >= 150)))
    return launch_dlds<128, 128, ROLE, 2, true>(a, s);
  // the 128x64 fp8 kernel needs more than the 168 registers of three waves
  // per SIMD (it would spill in its loop); two fit
  return launch_dlds<128, 64, ROLE, 2, true>(a, s);
}

template <typename T, int ROLE>
hipError_t launch_shape(const GemmArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // direct-to-LDS pipeline: whole 64-wide K steps, N wide enough to fill a tile
    if (a.K % 64 == 0 && a.N > 32) {
      const int64_t tiles128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128) * a.groups;
      // 128x128 tiles read less per MFMA and win on the 512-wide conv GEMMs,
      // wherever there are at least ~400 of them, and on long-K products
      // (FFN2, K = 3072) from ~150 of them; with fewer (N = 768 linears with
      // short K: out-proj, projection) 128x64 tiles balance the CUs better.
      // The thresholds were measured with the two batch halves of a forward
      // running concurrently (half-batch FFN1 / QKV / FFN2: M = 3196).
      // long K with at most one tile per CU (half-batch FFN2, 150 tiles):
      // one deep-pipelined workgroup per CU; same-box A/B of the two-stream
      // step 3.721 -> 3.674 ms, bit-identical results
      if (a.N > 64 && a.K >= 2048 && a.groups == 1 && tiles128 <= 256 && epilogue_staged_ok_host(a)) {
        hipLaunchKernelGGL((gemm_deep_kernel<ROLE>), dim3((unsigned)tiles128), dim3(256), 0, s, a);
        return hipGetLastError();
      }
      if (a.N > 64 && (a.N <= 512 || tiles128 >= 400 || (a.K >= 2048 && tiles128 >= 150)))
        return launch_dlds<128, 128, ROLE, 2>(a, s);
      return launch_dlds<128, 64, ROLE, 3>(a, s);
    }
  }
  if (a.N <= 32) return launch_t<T, 64, 32, 4, 1, ROLE>(a, s);
  if (a.N <= 48) return launch_t<T, 128, 48, 4, 1, ROLE>(a, s);
  if (a.N <= 64) return launch_t<T, 128, 64, 4, 1, ROLE>(a, s);
  return launch_t<T, 128, 128, 2, 2, ROLE>(a, s);
}

}  // namespace

// Launch of one GEMM role (fp16 or fp32 operands); explicitly instantiated
// once per role in gemm_role_*.hip.
template <int ROLE>
hipError_t launch_gemm_role(DType t, const GemmArgs& a, hipStream_t s) {
  if (t == DType::F8) {
    if constexpr (ROLE == kGemmQKV || ROLE == kGemmOut || ROLE == kGemmFFN1 || ROLE == kGemmFFN2)
      return launch_f8<ROLE>(a, s);
    return hipErrorInvalidValue;
  }
  return t == DType::F16 ? launch_shape<half_t, ROLE>(a, s) : launch_shape<float, ROLE>(a, s);
}

}  // namespace w2v2
