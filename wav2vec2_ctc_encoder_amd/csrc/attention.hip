// Flash-style multi-head self-attention over all T frames (no mask), gfx950.
//
// Input: the fused projection output qkv [B*T, 3d] (q | k | v; head h at
// columns h*dh of each part).  Output: o [B*T, d], heads concatenated.
// out[q] = sum_key softmax_key(q.k / sqrt(dh)) v[key].
//
// Workgroup = 64 queries of one (batch row, head); 4 waves x 16 queries.
// K and V are streamed through LDS in tiles of 64 keys (V stored
// transposed, [d][key]); softmax is computed online in fp32 with exp2 and a
// running max per query, so the T x T score matrix never leaves registers.
//
// Each wave computes the transposed score block S^T = K Q^T with 16x16 MFMA
// blocks (A operand = 16 keys, B operand = 16 queries), so a lane holds the
// scores of ONE query (lane % 16) for 4 keys per block.  That is exactly the
// B-operand layout P^T needs for O^T = V^T P^T, the second product: the
// scores are turned into probabilities in place and fed back to the matrix
// core without any shuffle.  The MFMA k-slots of the second product carry
// keys {16b + 4g + r}; the V^T operand reads the same keys from LDS, so the
// contraction covers every key once.  Tail keys (>= T) get score -inf and
// zero K/V rows.
//
// True-length rows: with per-row frame counts and packed starts, row b's
// queries and keys are its own frames only (workgroups past them exit).
#include "common.h"

namespace w2v2 {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;   // queries per workgroup
constexpr int kKT = 64;  // keys per tile

template <typename T, int DH>
struct AttnCfg {
  static constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  static constexpr int KC = 64 / sizeof(T);           // d per MFMA chunk (32 fp16, 16 fp32)
  static constexpr int DHP = DH < KC ? KC : DH;       // d padded to whole chunks
  static constexpr int NCH = DHP / KC;                // d chunks of the score product
  static constexpr int KPITCH = DHP * sizeof(T) / 16 + 1;  // K row pitch, 16-byte units
  static constexpr int VPITCH = kKT * sizeof(T) / 16 + 1;  // V^T row pitch, 16-byte units
  static constexpr int ND = DH / 16;                  // 16-row d blocks of the output
};

template <typename T, int DH>
__global__ __launch_bounds__(256) void attention_kernel(const T* __restrict__ qkv, T* __restrict__ out, int Tpad,
                                                        RowSpan rows, int H, float c1) {
  using C = AttnCfg<T, DH>;
  __shared__ uint4 sK[kKT * C::KPITCH];
  __shared__ uint4 sV[DH * C::VPITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int b = blockIdx.z, h = blockIdx.y;
  const int Tn = rows.len ? rows.len[b] : Tpad;                                  // frames of this row
  const int64_t rs = rows.start ? (int64_t)rows.start[b] : (int64_t)b * Tpad;    // its first row
  if (blockIdx.x * kQ >= Tn) return;
  const int dm = H * DH;
  const int64_t ld = 3 * (int64_t)dm;
  const T* base = qkv + rs * ld;
  const int q0 = blockIdx.x * kQ + wave * 16;

  // zero the padded d range of K once (only when DH < one MFMA chunk)
  if (DH < C::DHP) {
    for (int i = tid; i < kKT * C::KPITCH; i += 256) sK[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }

  // Q fragments of this wave's 16 queries: lane (lr, lg), chunk c
  uint4 qf[C::NCH];
  {
    const int q = q0 + lr;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) {
      const int d0 = c * C::KC + lg * C::EPC;
      qf[c] = (q < Tn && d0 < DH) ? *(const uint4*)(base + (int64_t)q * ld + h * DH + d0) : make_uint4(0, 0, 0, 0);
    }
  }

  f4 o[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) o[i] = f4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lsum = 0.f;

  constexpr int CPR = DH / C::EPC;  // 16-byte chunks per K/V row
  for (int k0 = 0; k0 < Tn; k0 += kKT) {
    __syncthreads();
    for (int idx = tid; idx < kKT * CPR; idx += 256) {
      const int r = idx / CPR, ch = idx % CPR;
      const int key = k0 + r;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < Tn) {
        const T* row = base + (int64_t)key * ld + h * DH + ch * C::EPC;
        kv = *(const uint4*)(row + dm);
        vv = *(const uint4*)(row + 2 * dm);
      }
      sK[r * C::KPITCH + ch] = kv;
      const T* ve = (const T*)&vv;
      T* vt = (T*)sV;
#pragma unroll
      for (int e = 0; e < C::EPC; ++e) vt[(ch * C::EPC + e) * (C::VPITCH * C::EPC) + r] = ve[e];
    }
    __syncthreads();

    // scores S^T[key][q] for 4 key blocks of 16
    f4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) {
        const uint4 kf = sK[(kb * 16 + lr) * C::KPITCH + c * 4 + lg];
        if constexpr (sizeof(T) == 2) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, kf), __builtin_bit_cast(h8, qf[c]),
                                                       acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf.x), __uint_as_float(qf[c].x), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf.y), __uint_as_float(qf[c].y), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf.z), __uint_as_float(qf[c].z), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf.w), __uint_as_float(qf[c].w), acc, 0, 0, 0);
        }
      }
      s[kb] = acc;
    }
    // online softmax for query lr (4 lanes share it: lg = 0..3)
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + kb * 16 + lg * 4 + r;
        if (key >= Tn) s[kb][r] = -INFINITY;
        mt = fmaxf(mt, s[kb][r]);
      }
    mt = max_xor16(mt);
    mt = max_xor32(mt);
    const float mnew = fmaxf(mrun, mt);
    const float alpha = exp2f((mrun - mnew) * c1);
    const float mc = mnew * c1;
    mrun = mnew;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(fmaf(s[kb][r], c1, -mc));
        s[kb][r] = p;
        ps += p;
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int i = 0; i < C::ND; ++i) o[i] *= alpha;

    // O^T[d][q] += V^T[d][key] P^T[key][q]
    const T* vt = (const T*)sV;
#pragma unroll
    for (int db = 0; db < C::ND; ++db) {
      const T* vrow = vt + (db * 16 + lr) * (C::VPITCH * C::EPC);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const h4 va = *(const h4*)(vrow + (2 * kp) * 16 + lg * 4);
          const h4 vb = *(const h4*)(vrow + (2 * kp + 1) * 16 + lg * 4);
          const h8 av = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
          const h8 pv = {(half_t)s[2 * kp][0], (half_t)s[2 * kp][1], (half_t)s[2 * kp][2], (half_t)s[2 * kp][3],
                         (half_t)s[2 * kp + 1][0], (half_t)s[2 * kp + 1][1], (half_t)s[2 * kp + 1][2],
                         (half_t)s[2 * kp + 1][3]};
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pv, o[db], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float4 va = *(const float4*)(vrow + kb * 16 + lg * 4);
          o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.x, s[kb][0], o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.y, s[kb][1], o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.z, s[kb][2], o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.w, s[kb][3], o[db], 0, 0, 0);
        }
      }
    }
  }

  lsum = add_xor16(lsum);
  lsum = add_xor32(lsum);
  const float inv = 1.f / lsum;
  const int q = q0 + lr;
  if (q < Tn) {
    T* orow = out + (rs + q) * dm + h * DH;
#pragma unroll
    for (int db = 0; db < C::ND; ++db) {
      const int d0 = db * 16 + lg * 4;
      if constexpr (sizeof(T) == 2) {
        const h4 hv = {(half_t)(o[db][0] * inv), (half_t)(o[db][1] * inv), (half_t)(o[db][2] * inv),
                       (half_t)(o[db][3] * inv)};
        *(h4*)(orow + d0) = hv;
      } else {
        *(float4*)(orow + d0) = make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// fp16 kernel on v_mfma_f32_16x16x32_f16 with 16 queries per wave (small
// register footprint, so several waves per SIMD hide the latency of the
// dependent score -> softmax -> PV chain).  Same S^T / P^T layout as the
// generic kernel above; K and V^T tiles of 64 keys are double-buffered in
// LDS with the next tile prefetched into registers, V is transposed with
// 8-byte LDS writes (4 keys x 4 d per thread), exp2 is the raw hardware
// instruction and only the last tile is masked.
// ----------------------------------------------------------------------------
template <int DH, int NW>
__global__ __launch_bounds__(NW * 64) void attn16_kernel(const half_t* __restrict__ qkv, half_t* __restrict__ out,
                                                        int Tpad, RowSpan rows, int H, float c1) {
  constexpr int KT = 64;
  constexpr int KP = DH / 8 + 1;             // K row pitch (16-byte units)
  constexpr int VP = KT + 4;                 // V^T row pitch (halves)
  constexpr int NCH = DH / 32;               // 32-wide d chunks of the score product
  constexpr int NDB = DH / 16;               // 16-row d blocks of the output
  constexpr int NT = NW * 64;
  constexpr int KCH = KT * DH / 8;
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int VGR = KT * DH / 16;
  constexpr int VPT = (VGR + NT - 1) / NT;

  __shared__ uint4 sK[2][KT * KP];
  __shared__ half_t sV[2][DH * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int b = blockIdx.z, h = blockIdx.y;
  const int Tn = rows.len ? rows.len[b] : Tpad;                                  // frames of this row
  const int64_t rs = rows.start ? (int64_t)rows.start[b] : (int64_t)b * Tpad;    // its first row
  if (blockIdx.x * (NW * 16) >= Tn) return;
  const int dm = H * DH;
  const int64_t ld = 3 * (int64_t)dm;
  const half_t* base = qkv + rs * ld + h * DH;
  const int qw = blockIdx.x * (NW * 16) + wave * 16;
  const bool wave_live = qw < Tn;

  uint4 qf[NCH];
  {
    const int q = min(qw + lr, Tn - 1);
#pragma unroll
    for (int c = 0; c < NCH; ++c) qf[c] = *(const uint4*)(base + (int64_t)q * ld + c * 32 + lg * 8);
  }

  // Keys past the row's last frame are read from that last frame (clamped,
  // no branch): their scores are masked to -inf, so their probabilities are
  // exactly 0 and their (finite) V rows add nothing.
  uint4 rk[KPT];
  uint2 rv[VPT][4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + NT * i;
      if (idx < KCH) {
        const int key = min(k0 + idx / (DH / 8), Tn - 1), ch = idx % (DH / 8);
        rk[i] = *(const uint4*)(base + (int64_t)key * ld + dm + ch * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + NT * i;
      if (idx < VGR) {
        const int dg = idx % (DH / 4), kg = idx / (DH / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = min(k0 + kg * 4 + r, Tn - 1);
          rv[i][r] = *(const uint2*)(base + (int64_t)key * ld + 2 * dm + dg * 4);
        }
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + NT * i;
      if (idx < KCH) sK[buf][(idx / (DH / 8)) * KP + idx % (DH / 8)] = rk[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + NT * i;
      if (idx < VGR) {
        const int dg = idx % (DH / 4), kg = idx / (DH / 4);
        const half_t* e0 = (const half_t*)&rv[i][0];
        const half_t* e1 = (const half_t*)&rv[i][1];
        const half_t* e2 = (const half_t*)&rv[i][2];
        const half_t* e3 = (const half_t*)&rv[i][3];
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          const h4 col = {e0[dd], e1[dd], e2[dd], e3[dd]};
          *(h4*)&sV[buf][(dg * 4 + dd) * VP + kg * 4] = col;
        }
      }
    }
  };

  f4 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lsum = 0.f;

  const int ntile = (Tn + KT - 1) / KT;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int t = 0; t < ntile; ++t) {
    const int cur = t & 1;
    const int k0 = t * KT;
    if (t + 1 < ntile) fetch(k0 + KT);
    if (wave_live) {
      f4 sc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint4 kf = sK[cur][(kb * 16 + lr) * KP + c * 4 + lg];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, kf), __builtin_bit_cast(h8, qf[c]),
                                                       acc, 0, 0, 0);
        }
        sc[kb] = acc;
      }
      if (k0 + KT > Tn) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (k0 + kb * 16 + lg * 4 + r >= Tn) sc[kb][r] = -INFINITY;
      }
      float mt = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, sc[kb][r]);
      mt = max_xor16(mt);
      mt = max_xor32(mt);
      const float mnew = fmaxf(mrun, mt);
      const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * c1);
      const float mc = mnew * c1;
      mrun = mnew;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], c1, -mc));
          sc[kb][r] = pv;
          ps += pv;
        }
      lsum = lsum * alpha + ps;
#pragma unroll
      for (int i = 0; i < NDB; ++i) o[i] *= alpha;
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const h8 pf = {(half_t)sc[2 * kp][0], (half_t)sc[2 * kp][1], (half_t)sc[2 * kp][2], (half_t)sc[2 * kp][3],
                       (half_t)sc[2 * kp + 1][0], (half_t)sc[2 * kp + 1][1], (half_t)sc[2 * kp + 1][2],
                       (half_t)sc[2 * kp + 1][3]};
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const half_t* vrow = &sV[cur][(db * 16 + lr) * VP + kp * 32 + lg * 4];
          const h4 va = *(const h4*)vrow;
          const h4 vb = *(const h4*)(vrow + 16);
          const h8 vf = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf, o[db], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntile) stash(cur ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  lsum = add_xor16(lsum);
  lsum = add_xor32(lsum);
  const float inv = 1.f / lsum;
  const int q = qw + lr;
  if (q < Tn) {
    half_t* orow = out + (rs + q) * dm + h * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const h4 hv = {(half_t)(o[db][0] * inv), (half_t)(o[db][1] * inv), (half_t)(o[db][2] * inv),
                     (half_t)(o[db][3] * inv)};
      *(h4*)(orow + db * 16 + lg * 4) = hv;
    }
  }
}

// shared: another part of the batch runs concurrently.  The kernel then asks
// for enough (unused) dynamic LDS (56 KB per workgroup) that at most two of
// its workgroups share a CU, leaving the rest of the CU (48 KB of LDS, one
// 128x64 GEMM workgroup) to the other part; with the GPU to itself it takes
// up to three per CU.
template <int DH, int NW>
hipError_t launch_a16(const void* qkv, void* out, int B, int Tn, RowSpan rows, int H, bool shared, hipStream_t s) {
  const float c1 = 1.4426950408889634f / sqrtf((float)DH);
  constexpr size_t kStatic = 2 * 64 * (DH / 8 + 1) * 16 + 2 * DH * (64 + 4) * 2;  // sK + sV
  constexpr size_t kTwoPerCu = 56 * 1024;
  const size_t pad = (shared && kStatic < kTwoPerCu) ? kTwoPerCu - kStatic : 0;
  hipLaunchKernelGGL((attn16_kernel<DH, NW>), dim3((Tn + NW * 16 - 1) / (NW * 16), H, B), dim3(NW * 64), pad, s,
                     (const half_t*)qkv, (half_t*)out, Tn, rows, H, c1);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t launch_t(const void* qkv, void* out, int B, int Tn, RowSpan rows, int H, hipStream_t s) {
  const float c1 = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)
  hipLaunchKernelGGL((attention_kernel<T, DH>), dim3((Tn + kQ - 1) / kQ, H, B), dim3(256), 0, s,
                     (const T*)qkv, (T*)out, Tn, rows, H, c1);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dh(const void* qkv, void* out, int B, int Tn, RowSpan rows, int H, int dh, hipStream_t s) {
  switch (dh) {
    case 16: return launch_t<T, 16>(qkv, out, B, Tn, rows, H, s);
    case 32: return launch_t<T, 32>(qkv, out, B, Tn, rows, H, s);
    case 64: return launch_t<T, 64>(qkv, out, B, Tn, rows, H, s);
    case 128: return launch_t<T, 128>(qkv, out, B, Tn, rows, H, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attention_supported(int dh) { return dh == 16 || dh == 32 || dh == 64 || dh == 128; }

hipError_t launch_attention(DType t, const void* qkv, void* out, int32_t B, int32_t T, RowSpan rows, int32_t H,
                            int32_t dh, bool shared, hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  // fp16: 16 queries per wave, 8 waves share each K/V tile
  if (t == DType::F16 && dh == 32) return launch_a16<32, 8>(qkv, out, B, T, rows, H, shared, s);
  if (t == DType::F16 && dh == 64) return launch_a16<64, 8>(qkv, out, B, T, rows, H, shared, s);
  if (t == DType::F16 && dh == 128) return launch_a16<128, 8>(qkv, out, B, T, rows, H, shared, s);
  return t == DType::F16 ? launch_dh<half_t>(qkv, out, B, T, rows, H, dh, s)
                         : launch_dh<float>(qkv, out, B, T, rows, H, dh, s);
}

}  // namespace w2v2
