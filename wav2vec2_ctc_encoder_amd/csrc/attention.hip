// Flash-style multi-head self-attention over all T frames (no mask), gfx950.
//
// Input: the fused projection output qkv [B*T, 3d] (q | k | v; head h at
// columns h*dh of each part).  Output: o [B*T, d], heads concatenated.
// out[q] = sum_key softmax_key(q.k / sqrt(dh)) v[key].
//
// Three kernels share one score / softmax / P.V formulation:
//  * attn64_kernel: fp16, d_h = 64 (the base and large models); 32 queries
//    per wave on 32x32x16 MFMAs, K and V go straight from global memory
//    into LDS and V^T is read with the transposing LDS read;
//  * attn16_kernel: fp16, d_h = 32 and 128; register-staged tiles with V
//    transposed on its way into LDS;
//  * attention_kernel (below): fp32, and head sizes the others do not take.
//
// attention_kernel: workgroup = 64 queries of one (batch row, head); 4 waves x 16 queries.
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

// The dispatcher hands consecutive workgroup ids to the 8 XCDs round-robin;
// this maps them so that each XCD gets one contiguous range of block indices
// (a bijection for any count).
__device__ inline int xcd_block(int pid, int nb) {
  const int x = pid & 7, local = pid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return x * per + (x < rem ? x : rem) + local;
}

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
                                                        RowSpan rows, int H, float c1, uint8_t* __restrict__ out8,
                                                        float inv8, float* __restrict__ amax) {
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
  float vmax = 0.f;
  if (q < Tn) {
    T* orow = out + (rs + q) * dm + h * DH;
#pragma unroll
    for (int db = 0; db < C::ND; ++db) {
      const int d0 = db * 16 + lg * 4;
      const float4 ov = make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
      vmax = fmaxf(vmax, fmaxf(fmaxf(fabsf(ov.x), fabsf(ov.y)), fmaxf(fabsf(ov.z), fabsf(ov.w))));
      if (out8) {
        *(uint32_t*)(out8 + (rs + q) * dm + h * DH + d0) = pack_e4m3x4(ov.x, ov.y, ov.z, ov.w, inv8);
      } else if constexpr (sizeof(T) == 2) {
        const h4 hv = {(half_t)ov.x, (half_t)ov.y, (half_t)ov.z, (half_t)ov.w};
        *(h4*)(orow + d0) = hv;
      } else {
        *(float4*)(orow + d0) = ov;
      }
    }
  }
  if (amax) wave_raise_amax(vmax, amax);
}

// ----------------------------------------------------------------------------
// fp16 kernel on v_mfma_f32_16x16x32_f16 with 16 queries per wave (small
// register footprint, so several waves per SIMD hide the latency of the
// dependent score -> softmax -> PV chain).  Same S^T / P^T layout as the
// generic kernel above; K and V^T tiles of 64 keys are double-buffered in
// LDS with the next tile prefetched into registers, V is transposed with
// 8-byte LDS writes (4 keys x 4 d per thread), exp2 is the raw hardware
// instruction and only the last tile is masked.  The running output is
// rescaled only on tiles where some query's maximum grew.
// ----------------------------------------------------------------------------
// OUT: 0 fp16 output; 1 e4m3 output (fp8 mode); 2 fp16 output and the amax
// of the calibration (compile-time, so the plain kernel carries neither).
template <int DH, int NW, int OUT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DH <= 64 ? 6 : 1))) void attn16_kernel(const half_t* __restrict__ qkv, half_t* __restrict__ out,
                                                        int Tpad, RowSpan rows, int H, float c1,
                                                        uint8_t* __restrict__ out8, float inv8,
                                                        float* __restrict__ amax) {
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
  // 1-D grid of (query block, head, row) in that order, remapped so that the
  // query blocks of one (row, head), which read the same K and V, run one
  // after another on one XCD and share its L2
  const int nqb = (Tpad + NW * 16 - 1) / (NW * 16);
  const int pid = xcd_block(blockIdx.x, gridDim.x);
  const int qb = pid % nqb, h = (pid / nqb) % H, b = pid / (nqb * H);
  const int Tn = rows.len ? rows.len[b] : Tpad;                                  // frames of this row
  const int64_t rs = rows.start ? (int64_t)rows.start[b] : (int64_t)b * Tpad;    // its first row
  if (qb * (NW * 16) >= Tn) return;
  const int dm = H * DH;
  const int64_t ld = 3 * (int64_t)dm;
  const half_t* base = qkv + rs * ld + h * DH;
  const int qw = qb * (NW * 16) + wave * 16;
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
        // column dd of the 4 x 4 block (keys kg*4 + r, d = dg*4 + dd) is
        // half-word dd of rv[i][r]; assembled with shifts and masks, so the
        // registers are never addressed as memory
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          const uint32_t w0 = dd < 2 ? rv[i][0].x : rv[i][0].y, w1 = dd < 2 ? rv[i][1].x : rv[i][1].y;
          const uint32_t w2 = dd < 2 ? rv[i][2].x : rv[i][2].y, w3 = dd < 2 ? rv[i][3].x : rv[i][3].y;
          uint2 col;
          if (dd & 1) {
            col.x = (w0 >> 16) | (w1 & 0xFFFF0000u);
            col.y = (w2 >> 16) | (w3 & 0xFFFF0000u);
          } else {
            col.x = (w0 & 0xFFFFu) | (w1 << 16);
            col.y = (w2 & 0xFFFFu) | (w3 << 16);
          }
          *(uint2*)&sV[buf][(dg * 4 + dd) * VP + kg * 4] = col;
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
      // Rescale only when some query's running max grew: otherwise every
      // alpha is exactly 1, o * 1 is o and fma(l, 1, p) is l + p, so the
      // skip leaves every bit as it was.
      const bool grew = __builtin_amdgcn_ballot_w64(mnew > mrun) != 0;
      const float alpha = grew ? __builtin_amdgcn_exp2f((mrun - mnew) * c1) : 1.f;
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
      if (grew) {
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int i = 0; i < NDB; ++i) o[i] *= alpha;
      } else {
        lsum += ps;
      }
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
  float vmax = 0.f;
  if (q < Tn) {
    half_t* orow = out + (rs + q) * dm + h * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const float4 ov = make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
      if constexpr (OUT == 2)
        vmax = fmaxf(vmax, fmaxf(fmaxf(fabsf(ov.x), fabsf(ov.y)), fmaxf(fabsf(ov.z), fabsf(ov.w))));
      if constexpr (OUT == 1) {
        *(uint32_t*)(out8 + (rs + q) * dm + h * DH + db * 16 + lg * 4) = pack_e4m3x4(ov.x, ov.y, ov.z, ov.w, inv8);
      } else {
        const h4 hv = {(half_t)ov.x, (half_t)ov.y, (half_t)ov.z, (half_t)ov.w};
        *(h4*)(orow + db * 16 + lg * 4) = hv;
      }
    }
  }
  if constexpr (OUT == 2) wave_raise_amax(vmax, amax);
}

// ----------------------------------------------------------------------------
// d_h = 64 fp16 kernel: 32 queries per wave on 32x32x16 MFMAs, with the K
// and V tiles loaded straight into LDS.  The formulation is attn16_kernel's
// (S^T = K Q^T, online softmax in fp32 with exp2, P^T fed back as the B
// operand of O^T = V^T P^T) with bigger blocks:
//  * a lane holds 16 scores of ONE query (l % 32) per 32-key block, keys
//    8i + 4(l / 32) + j (i, j = 0..3); a query's row max and sum take one
//    cross-lane step (lanes l and l ^ 32);
//  * those registers are already P^T's B operand: for the P.V MFMA u (keys
//    16u .. 16u + 15 of the block) a lane's k-slots 8(l/32) + 4a + j carry
//    keys 8(2u + a) + 4(l/32) + j, i.e. its score registers 8u .. 8u + 7;
//  * the V^T operand (d rows, the same keys) comes from gfx950's transposing
//    LDS read (ds_read_b64_tr_b16): within each 16-lane group g, lane
//    4j + q points at V row 8(2u + a) + 4(g / 2) + j, columns
//    32db + 16(g % 2) + 4q .. + 3, and lane i then receives those 4 keys of
//    column 32db + 16(g % 2) + i; two reads (a = 0, 1) give the 8 k-slots;
//  * each K or V fragment read now serves 32 queries (half the LDS reads
//    per query of 16-query waves);
//  * every wave moves 16 rows of K and 16 of V per 64-key tile with
//    wave-wide global_load_lds_dwordx4 (16 bytes per lane), one tile ahead
//    in a ring of two; the address is a wave-uniform tile base in SGPRs plus
//    a loop-invariant 32-bit lane offset.  Rows stay row-major with their
//    16-byte chunks XOR-swizzled by (row & 7);
//  * the loop is unrolled by two, so the LDS buffers are compile-time.
// ----------------------------------------------------------------------------
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

// direct-to-LDS load of 16 bytes per lane from sbase + voff
__device__ inline void dma16s(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
// s_waitcnt vmcnt(N), other counters untouched
template <int N>
__device__ inline void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int NW, int OUT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void attn64_kernel(
    const half_t* __restrict__ qkv, half_t* __restrict__ out, int Tpad, RowSpan rows, int H, float c1,
    uint8_t* __restrict__ out8, float inv8, float* __restrict__ amax) {
  constexpr int DH = 64, KT = 64, TILE = KT * DH;  // halves per K (or V) tile
  constexpr int QW = 32, QB = NW * QW;             // queries per wave, per workgroup
  constexpr int RW = KT / NW;                      // tile rows each wave loads
  static_assert(NW == 4, "16 rows per wave: two load instructions per operand");
  __shared__ half_t sK[2][TILE];
  __shared__ half_t sV[2][TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hg = lane >> 5;
  const int nqb = (Tpad + QB - 1) / QB;
  const int pid = xcd_block(blockIdx.x, gridDim.x);
  const int qb = pid % nqb, h = (pid / nqb) % H, b = pid / (nqb * H);
  const int Tn = rows.len ? rows.len[b] : Tpad;
  const int64_t rs = rows.start ? (int64_t)rows.start[b] : (int64_t)b * Tpad;
  if (qb * QB >= Tn) return;
  const int dm = H * DH;
  const int64_t ld = 3 * (int64_t)dm;
  const half_t* base = qkv + rs * ld + h * DH;
  const int qw = qb * QB + wave * QW;
  const bool wave_live = qw < Tn;

  // Q^T operand of the score MFMAs: query l32, d = 16c + 8hg .. + 7
  uint4 qf[4];
  {
    const int q = min(qw + l32, Tn - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = *(const uint4*)(base + (int64_t)q * ld + c * 16 + hg * 8);
  }

  // Loads: wave w moves rows 16w .. 16w + 15, 8 per instruction; lane l takes
  // row 16w + 8j + l/8 and puts its source chunk (l % 8) ^ (row & 7) at chunk
  // l % 8.  Byte offsets are from the tile's first key row; V sits dm halves
  // after K.  In the last tile, keys past the row's last frame are read from
  // that frame (their scores are masked).
  const int lr8 = lane >> 3;
  uint32_t koffj[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wave * RW + j * 8 + lr8;
    koffj[j] = (uint32_t)(r * ld + dm + (((lane & 7) ^ (r & 7)) * 8)) * 2u;
  }
  const uint32_t vdel = (uint32_t)dm * 2u;
  const uint32_t ldsK = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&sK[0][wave * RW * DH]);
  const uint32_t ldsV = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&sV[0][wave * RW * DH]);
  auto issue = [&](int t, int buf) __attribute__((always_inline)) {
    const half_t* tb = base + (int64_t)t * KT * ld;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t off = koffj[j];
      if (t * KT + KT > Tn) {
        asm volatile("");  // keeps this a branch instead of work in every tile
        const int r = wave * RW + j * 8 + lr8;
        const int key = min(t * KT + r, Tn - 1);
        off = (uint32_t)((key - t * KT) * ld + dm + (((lane & 7) ^ (r & 7)) * 8)) * 2u;
      }
      dma16s(off, tb, ldsK + (buf * TILE + j * 8 * DH) * 2);
      dma16s(off + vdel, tb, ldsV + (buf * TILE + j * 8 * DH) * 2);
    }
  };
  // element offsets of the fragment reads (the swizzle depends on row & 7
  // only, which the block offsets keep)
  // K operand: key 32kb + l32, d chunk 2c + hg
  int koffs[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) koffs[c] = l32 * DH + (((2 * c + hg) ^ (l32 & 7)) << 3);
  // V^T operand: group g, lane i = 4j + q of it: V row 4(g/2) + j (+ 32kb +
  // 8(2u + a)), columns 32db + 16(g % 2) + 4q .. + 3
  int voffs[2];
  {
    const int g = lane >> 4, jj = (lane & 15) >> 2, q = lane & 3;
    const int R = 4 * (g >> 1) + jj;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int col = db * 32 + 16 * (g & 1) + 4 * q;
      voffs[db] = R * DH + (((col >> 3) ^ (R & 7)) << 3) + (col & 7);
    }
  }

  f16v o[2];  // O^T blocks: o[db][r] is d = 32db + 8(r/4) + 4hg + r%4 of query l32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float mrun = -INFINITY, lsum = 0.f;
  const int ntile = (Tn + KT - 1) / KT;

  // one tile from LDS buffer cur; the next tile's loads go to the other one,
  // which every wave finished with before the previous barrier
  auto step = [&](int t, int cur) __attribute__((always_inline)) {
    const int k0 = t * KT;
    if (t + 1 < ntile) issue(t + 1, cur ^ 1);
    if (wave_live) {
      f16v sc[2];  // sc[kb][r]: key 32kb + 8(r/4) + 4hg + r%4 of query l32
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f16v acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 kf = *(const uint4*)&sK[cur][koffs[c] + kb * 32 * DH];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, kf), __builtin_bit_cast(h8, qf[c]), acc,
                                                       0, 0, 0);
        }
        sc[kb] = acc;
      }
      if (k0 + KT > Tn) {
        asm volatile("");  // keeps this a branch instead of work in every tile
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (k0 + kb * 32 + 8 * (r >> 2) + 4 * hg + (r & 3) >= Tn) sc[kb][r] = -INFINITY;
      }
      float mt = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[kb][r]);
      mt = max_xor32(mt);
      const float mnew = fmaxf(mrun, mt);
      // rescale only when some query's running max grew (else alpha is exactly 1)
      const bool grew = __builtin_amdgcn_ballot_w64(mnew > mrun) != 0;
      const float alpha = grew ? __builtin_amdgcn_exp2f((mrun - mnew) * c1) : 1.f;
      const float mc = mnew * c1;
      mrun = mnew;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], c1, -mc));
          sc[kb][r] = pv;
          ps += pv;
        }
      if (grew) {
        asm volatile("");  // keeps this a branch instead of work in every tile
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int i = 0; i < 2; ++i) o[i] *= alpha;
      } else {
        lsum += ps;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const h8 pf = {(half_t)sc[kb][8 * u + 0], (half_t)sc[kb][8 * u + 1], (half_t)sc[kb][8 * u + 2],
                         (half_t)sc[kb][8 * u + 3], (half_t)sc[kb][8 * u + 4], (half_t)sc[kb][8 * u + 5],
                         (half_t)sc[kb][8 * u + 6], (half_t)sc[kb][8 * u + 7]};
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            v4s part[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
              part[a] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) v4s*)&sV[cur][voffs[db] + (kb * 32 + 8 * (2 * u + a)) * DH]);
            const h8 vf = __builtin_bit_cast(h8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, o[db], 0, 0, 0);
          }
        }
    }
    // this wave's part of tile t + 1 has landed
    wait_vm<0>();
    __syncthreads();
  };

  issue(0, 0);
  wait_vm<0>();
  __syncthreads();
  for (int t = 0; t < ntile; t += 2) {
    step(t, 0);
    if (t + 1 < ntile) step(t + 1, 1);
  }

  if (!wave_live) return;
  lsum = add_xor32(lsum);
  const float inv = 1.f / lsum;
  const int q = qw + l32;
  float vmax = 0.f;
  if (q < Tn) {
    half_t* orow = out + (rs + q) * dm + h * DH;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * hg;
        const float4 ov = make_float4(o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv, o[db][4 * r4 + 2] * inv,
                                      o[db][4 * r4 + 3] * inv);
        if constexpr (OUT == 2)
          vmax = fmaxf(vmax, fmaxf(fmaxf(fabsf(ov.x), fabsf(ov.y)), fmaxf(fabsf(ov.z), fabsf(ov.w))));
        if constexpr (OUT == 1) {
          *(uint32_t*)(out8 + (rs + q) * dm + h * DH + d0) = pack_e4m3x4(ov.x, ov.y, ov.z, ov.w, inv8);
        } else {
          const h4 hv = {(half_t)ov.x, (half_t)ov.y, (half_t)ov.z, (half_t)ov.w};
          *(h4*)(orow + d0) = hv;
        }
      }
  }
  if constexpr (OUT == 2) wave_raise_amax(vmax, amax);
}

template <int NW>
hipError_t launch_a64(const void* qkv, void* out, int B, int Tn, RowSpan rows, int H, bool shared, hipStream_t s,
                      uint8_t* out8, float inv8, float* amax) {
  const float c1 = 1.4426950408889634f / sqrtf(64.f);
  // The 32-bit lane offsets of the loads reach 63 rows of the fused q|k|v
  // matrix past a tile's first row.
  if ((int64_t)63 * 3 * H * 64 * 2 + 3 * H * 64 * 2 > (int64_t)0xFFFFFFFF) return hipErrorInvalidValue;
  // Sharing the chip with the other half's GEMMs, each workgroup takes 48 KB
  // of LDS (three per CU, or one beside a GEMM workgroup); same-box medians
  // of the two-stream base 8 x 16 s step with 8-wave workgroups of 16-query
  // waves: 40 KB 3.41 ms, 48 KB 3.41, 56 KB 3.43, 64 KB 3.45.
  constexpr size_t kStatic = 2 * 2 * 64 * 64 * 2;  // sK + sV
  constexpr size_t kShared = 48 * 1024;
  const size_t pad = (shared && kStatic < kShared) ? kShared - kStatic : 0;
  const dim3 grid(((Tn + NW * 32 - 1) / (NW * 32)) * H * B);
  if (out8)
    hipLaunchKernelGGL((attn64_kernel<NW, 1>), grid, dim3(NW * 64), pad, s, (const half_t*)qkv, (half_t*)out, Tn,
                       rows, H, c1, out8, inv8, amax);
  else if (amax)
    hipLaunchKernelGGL((attn64_kernel<NW, 2>), grid, dim3(NW * 64), pad, s, (const half_t*)qkv, (half_t*)out, Tn,
                       rows, H, c1, out8, inv8, amax);
  else
    hipLaunchKernelGGL((attn64_kernel<NW, 0>), grid, dim3(NW * 64), pad, s, (const half_t*)qkv, (half_t*)out, Tn,
                       rows, H, c1, out8, inv8, amax);
  return hipGetLastError();
}

// shared: another part of the batch runs concurrently.  The kernel then asks
// for enough (unused) dynamic LDS (56 KB per workgroup) that at most two of
// its workgroups share a CU, leaving the rest of the CU (48 KB of LDS, one
// 128x64 GEMM workgroup) to the other part; with the GPU to itself it takes
// up to three per CU.
template <int DH, int NW>
hipError_t launch_a16(const void* qkv, void* out, int B, int Tn, RowSpan rows, int H, bool shared, hipStream_t s,
                      uint8_t* out8, float inv8, float* amax) {
  const float c1 = 1.4426950408889634f / sqrtf((float)DH);
  constexpr size_t kStatic = 2 * 64 * (DH / 8 + 1) * 16 + 2 * DH * (64 + 4) * 2;  // sK + sV
  constexpr size_t kTwoPerCu = 56 * 1024;
  const size_t pad = (shared && kStatic < kTwoPerCu) ? kTwoPerCu - kStatic : 0;
  const dim3 grid(((Tn + NW * 16 - 1) / (NW * 16)) * H * B);
  if (out8)
    hipLaunchKernelGGL((attn16_kernel<DH, NW, 1>), grid, dim3(NW * 64), pad, s, (const half_t*)qkv, (half_t*)out, Tn,
                       rows, H, c1, out8, inv8, amax);
  else if (amax)
    hipLaunchKernelGGL((attn16_kernel<DH, NW, 2>), grid, dim3(NW * 64), pad, s, (const half_t*)qkv, (half_t*)out, Tn,
                       rows, H, c1, out8, inv8, amax);
  else
    hipLaunchKernelGGL((attn16_kernel<DH, NW, 0>), grid, dim3(NW * 64), pad, s, (const half_t*)qkv, (half_t*)out, Tn,
                       rows, H, c1, out8, inv8, amax);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t launch_t(const void* qkv, void* out, int B, int Tn, RowSpan rows, int H, hipStream_t s, uint8_t* out8,
                    float inv8, float* amax) {
  const float c1 = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)
  hipLaunchKernelGGL((attention_kernel<T, DH>), dim3((Tn + kQ - 1) / kQ, H, B), dim3(256), 0, s,
                     (const T*)qkv, (T*)out, Tn, rows, H, c1, out8, inv8, amax);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dh(const void* qkv, void* out, int B, int Tn, RowSpan rows, int H, int dh, hipStream_t s,
                     uint8_t* out8, float inv8, float* amax) {
  switch (dh) {
    case 16: return launch_t<T, 16>(qkv, out, B, Tn, rows, H, s, out8, inv8, amax);
    case 32: return launch_t<T, 32>(qkv, out, B, Tn, rows, H, s, out8, inv8, amax);
    case 64: return launch_t<T, 64>(qkv, out, B, Tn, rows, H, s, out8, inv8, amax);
    case 128: return launch_t<T, 128>(qkv, out, B, Tn, rows, H, s, out8, inv8, amax);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attention_supported(int dh) { return dh == 16 || dh == 32 || dh == 64 || dh == 128; }

hipError_t launch_attention(DType t, const void* qkv, void* out, int32_t B, int32_t T, RowSpan rows, int32_t H,
                            int32_t dh, bool shared, hipStream_t s, uint8_t* out8, float inv8, float* amax) {
  if (B <= 0 || T <= 0) return hipSuccess;
  // fp16: 16 queries per wave, 8 waves share each K/V tile
  if (t == DType::F16 && dh == 32) return launch_a16<32, 8>(qkv, out, B, T, rows, H, shared, s, out8, inv8, amax);
  if (t == DType::F16 && dh == 64) return launch_a64<4>(qkv, out, B, T, rows, H, shared, s, out8, inv8, amax);
  if (t == DType::F16 && dh == 128) return launch_a16<128, 8>(qkv, out, B, T, rows, H, shared, s, out8, inv8, amax);
  return t == DType::F16 ? launch_dh<half_t>(qkv, out, B, T, rows, H, dh, s, out8, inv8, amax)
                         : launch_dh<float>(qkv, out, B, T, rows, H, dh, s, out8, inv8, amax);
}

}  // namespace w2v2
