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
// variance over all T0 frames of a row.  Conv 0 is linear in the k shifted
// sample sequences x_j(t) = x[s*t + j], so with mu_j their means and
// S_ij = sum_t (x_i(t) - mu_i)(x_j(t) - mu_j) their co-moments, channel c
// (taps w_c, bias b_c) has mean w_c . mu + b_c and variance w_c^T S w_c / T0.
// gn0_stats reads only the PCM and writes per-chunk (mu, S) partials in
// fp64; gn0_finalize merges them in a fixed order with Chan's pairwise
// update and forms each channel's scale and shift; conv0 then applies
// GroupNorm and GELU before its single store, so the pre-norm conv output
// never goes to memory.  Deterministic, and fp64 keeps the quadratic form
// accurate even when a filter cancels most of the input's energy.
// Layer-norm variant: the per-frame LayerNorm over channels and the GELU are
// done in registers with wave reductions before the single store.
//
// True-length rows: every kernel here can take a per-row frame count; conv 0
// then writes row b's frames to consecutive packed rows from its own start,
// and the statistics cover only that row's frames.
#include "common.h"

namespace w2v2 {
namespace {

constexpr int kChunk = 256;       // frames per conv0 workgroup
constexpr int kStatChunk = 1024;  // frames per GroupNorm-statistics workgroup
constexpr int kLanesC = 8;   // channels per lane

template <int N>
struct ActTag {
  static constexpr int value = N;
};

__device__ inline float wave_sum(float v) { return wave_sum64(v); }

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

// Copy n samples of one PCM row, starting at sample base, into LDS; samples
// at or past vl read as zero.  Each thread issues its loads in groups of 8
// before storing any of them, so their latencies overlap instead of adding
// up (a load-store loop waits for every load before the next one issues).
__device__ inline void stage_pcm(float* xs, const float* __restrict__ row, int64_t base, int n, int vl) {
  for (int i0 = 0; i0 < n; i0 += 256 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + (int)threadIdx.x;
      v[u] = (i < n && base + i < vl) ? row[base + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + (int)threadIdx.x;
      if (i < n) xs[i] = v[u];
    }
  }
}

// KT: compile-time tap count (taps >= k carry zero weights).
template <typename T, int KT>
__global__ __launch_bounds__(256) void conv0_kernel(const float* __restrict__ pcm, const int32_t* __restrict__ valid,
                                                     int L, const float* __restrict__ w0,
                                                     const float* __restrict__ bias, int C, int k, int stride,
                                                     int T0, RowSpan rows, T* __restrict__ y,
                                                     const float2* __restrict__ ss,
                                                     const float* __restrict__ gamma,
                                                     const float* __restrict__ beta, float eps, int act) {
  extern __shared__ float smem[];
  const int b = blockIdx.y;
  const int chunk = blockIdx.x;
  const int t0 = chunk * kChunk;
  const int Tb = rows.len ? rows.len[b] : T0;             // frames of this row
  const int nf = min(kChunk, Tb - t0);
  if (nf <= 0) return;
  const int64_t ybase = rows.start ? (int64_t)rows.start[b] : (int64_t)b * T0;  // its first output row
  const int nsamp = (nf - 1) * stride + KT;
  float* xs = smem;                                  // [nsamp]

  int vl = valid[b];
  vl = vl < 0 ? 0 : (vl > L ? L : vl);
  const int64_t base = (int64_t)t0 * stride;
  // a few samples per thread: a plain loop (batched loads measured slower here)
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
    auto frames = [&](auto act_tag) {
      constexpr int ACT = decltype(act_tag)::value;
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
        for (int c = 0; c < kLanesC; ++c) v[c] = act_fn<ACT>((v[c] - mean) * rstd * g[c] + be[c]);
        if (active) store8<T>(y + (ybase + t0 + f) * C + c0, v);
      }
    };
    if (act == 2) frames(ActTag<2>{});
    else frames(ActTag<1>{});
    return;
  }

  // group variant: per-channel scale / shift from gn0_finalize, then GELU
  float sc[kLanesC], sh[kLanesC];
#pragma unroll
  for (int c = 0; c < kLanesC; ++c) {
    const float2 p = active ? ss[(int64_t)b * C + c0 + c] : make_float2(0.f, 0.f);
    sc[c] = p.x;
    sh[c] = p.y;
  }
  auto frames = [&](auto act_tag) {
    constexpr int ACT = decltype(act_tag)::value;
    for (int f = wave; f < nf; f += 4) {
      float v[kLanesC];
      conv(f, v);
#pragma unroll
      for (int c = 0; c < kLanesC; ++c) v[c] = act_fn<ACT>(fmaf(v[c], sc[c], sh[c]));
      if (active) store8<T>(y + (ybase + t0 + f) * C + c0, v);
    }
  };
  if (act == 2) frames(ActTag<2>{});
  else frames(ActTag<1>{});
}

// conv0 + GroupNorm + GELU of the fp16 mode with the convolution on fp32
// matrix cores.  For a block of 32 frames and 32 channels the conv is a
// 32x32 product with K = taps: D[c][f] = sum_j w[c][j] x[stride f + j],
// v_mfma_f32_32x32x2_f32 taking 2 taps per instruction (fp32 products and
// sums, as on the vector path; taps 2 KS > k carry zero weights).  A lane
// then holds frame f = l % 32 and channels 8q + 4 (l / 32) + 0..3 of the
// block; it applies the folded GroupNorm scale / shift and the GELU, packs
// fp16 and writes the values to its wave's LDS slab, from which whole
// 128-byte row pieces (64 channels of a frame) go to memory.  This takes the
// ten multiply-adds per output off the vector unit, which bounds the
// vector-path kernel.
constexpr int kConv0MaxC = 512;  // channels the matrix-core conv0 handles (its LDS budget)

template <int KS, int ACT>
__global__ __launch_bounds__(256) void conv0_mfma_kernel(const float* __restrict__ pcm,
                                                         const int32_t* __restrict__ valid, int L,
                                                         const float* __restrict__ w0,
                                                         const float* __restrict__ bias, int C, int k, int stride,
                                                         int T0, RowSpan rows, half_t* __restrict__ y,
                                                         const float2* __restrict__ ss) {
  typedef float f16v __attribute__((ext_vector_type(16)));
  typedef _Float16 h4v __attribute__((ext_vector_type(4)));
  constexpr int KT = 2 * KS;   // padded taps
  constexpr int SP = 72;       // slab row pitch in halves: 64 channels + 16 B
  extern __shared__ float smem[];
  float* wl = smem;                                    // [C][KT]
  float2* ssl = reinterpret_cast<float2*>(wl + C * KT);  // [C] (scale, shift with the conv bias folded in)
  float* xs = reinterpret_cast<float*>(ssl + C);         // [(kChunk - 1) * stride + KT]
  const int nx = (kChunk - 1) * stride + KT;
  half_t* slab = reinterpret_cast<half_t*>(xs + ((nx + 3) & ~3));  // [4][32][SP]

  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kChunk;
  const int Tb = rows.len ? rows.len[b] : T0;  // frames of this row
  const int nf = min(kChunk, Tb - t0);
  if (nf <= 0) return;
  const int64_t ybase = rows.start ? (int64_t)rows.start[b] : (int64_t)b * T0;  // its first output row

  int vl = valid[b];
  vl = vl < 0 ? 0 : (vl > L ? L : vl);
  // Weights, scale / shift and samples go to LDS with every thread's loads
  // issued before its stores, so their latencies overlap.  Samples cover
  // every frame slot of the chunk (frames past nf are computed from whatever
  // samples are there and never stored) and read zero at or past vl.
  {
    constexpr int NWL = (kConv0MaxC * KT + 255) / 256, NSS = (kConv0MaxC + 255) / 256;
    float wr[NWL];
    float2 sr[NSS];
    float br[NSS];
#pragma unroll
    for (int u = 0; u < NWL; ++u) {
      const int i = (int)threadIdx.x + 256 * u, c = i / KT, j = i - c * KT;
      wr[u] = (i < C * KT && j < k) ? w0[c * k + j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NSS; ++u) {
      const int c = (int)threadIdx.x + 256 * u;
      sr[u] = c < C ? ss[(int64_t)b * C + c] : make_float2(0.f, 0.f);
      br[u] = (c < C && bias) ? bias[c] : 0.f;
    }
    stage_pcm(xs, pcm + (int64_t)b * L, (int64_t)t0 * stride, nx, vl);
#pragma unroll
    for (int u = 0; u < NWL; ++u) {
      const int i = (int)threadIdx.x + 256 * u;
      if (i < C * KT) wl[i] = wr[u];
    }
#pragma unroll
    for (int u = 0; u < NSS; ++u) {
      const int c = (int)threadIdx.x + 256 * u;
      if (c < C) ssl[c] = make_float2(sr[u].x, fmaf(br[u], sr[u].x, sr[u].y));
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, lg = lane >> 5;
  half_t* st = slab + wave * 32 * SP;
  for (int fb = wave * 32; fb < nf; fb += 128) {
    float xb[KS];
#pragma unroll
    for (int q = 0; q < KS; ++q) xb[q] = xs[stride * (fb + l32) + 2 * q + lg];
    for (int cg = 0; cg < C; cg += 64) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cb = cg + 32 * h;
        f16v acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
        for (int q = 0; q < KS; ++q)
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(wl[(cb + l32) * KT + 2 * q + lg], xb[q], acc, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cl = 32 * h + 8 * q + 4 * lg;  // first of this lane's 4 channels within the 64
          h4v o;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float2 p = ssl[cg + cl + i];
            o[i] = (half_t)act_fn<ACT>(fmaf(acc[4 * q + i], p.x, p.y));
          }
          *(h4v*)(st + l32 * SP + cl) = o;
        }
      }
      // the slab holds 32 frames x 64 channels; LDS operations of one wave
      // complete in order, so the read-back sees every lane's writes
#pragma unroll
      for (int ps = 0; ps < 4; ++ps) {
        const int r = ps * 8 + (lane >> 3), col = (lane & 7) * 8;
        const uint4 v = *(const uint4*)(st + r * SP + col);
        const int f = fb + r;
        if (f < nf) *(uint4*)(y + (ybase + t0 + f) * C + cg + col) = v;
      }
    }
  }
}

// Per (row, chunk of kStatChunk frames): means of the k shifted sequences and
// their co-moments (upper triangle, row-major i <= j), in fp64.
// Output layout per chunk: [mu_0 .. mu_{k-1}, S_00, S_01, .., S_{k-1,k-1}].
// Every thread sums a fixed frame-strided share of one quantity; the shares
// are added in a fixed order, so the result is deterministic.
__global__ __launch_bounds__(256) void gn0_stats_kernel(const float* __restrict__ pcm,
                                                         const int32_t* __restrict__ valid, int L, int k,
                                                         int stride, int T0, const int32_t* __restrict__ rows_len,
                                                         double* __restrict__ part) {
  extern __shared__ float xs[];  // [(kStatChunk - 1) * stride + k]
  __shared__ double red[256];
  __shared__ double mu[16];
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int t0 = chunk * kStatChunk;
  const int Tb = rows_len ? rows_len[b] : T0;  // frames of this row
  const int nf = min(kStatChunk, Tb - t0);
  if (nf <= 0) return;  // past the row's frames: the merge stops before this chunk
  const int nsamp = (nf - 1) * stride + k;
  int vl = valid[b];
  vl = vl < 0 ? 0 : (vl > L ? L : vl);
  const int64_t base = (int64_t)t0 * stride;
  stage_pcm(xs, pcm + (int64_t)b * L, base, nsamp, vl);
  __syncthreads();
  const int ns = k + k * (k + 1) / 2;
  double* out = part + ((int64_t)b * gridDim.x + chunk) * ns;
  const int tid = threadIdx.x;
  // means: k quantities x mp shares
  const int mp = 256 / k;
  if (tid < k * mp) {
    const int j = tid % k, sh = tid / k;
    double acc = 0.0;
    for (int f = sh; f < nf; f += mp) acc += (double)xs[f * stride + j];
    red[tid] = acc;
  }
  __syncthreads();
  if (tid < k) {
    double acc = 0.0;
    for (int sh = 0; sh < mp; ++sh) acc += red[sh * k + tid];
    mu[tid] = acc / nf;
    out[tid] = acc / nf;
  }
  __syncthreads();
  // co-moments: npair quantities x pp shares
  const int npair = k * (k + 1) / 2;
  const int pp = 256 / npair;
  double acc = 0.0;
  int pr = 0;
  if (tid < npair * pp) {
    pr = tid % npair;
    const int sh = tid / npair;
    int i = 0, rem = pr;
    while (rem >= k - i) {
      rem -= k - i;
      ++i;
    }
    const int j = i + rem;
    const double mi = mu[i], mj = mu[j];
    for (int f = sh; f < nf; f += pp) acc += ((double)xs[f * stride + i] - mi) * ((double)xs[f * stride + j] - mj);
  }
  __syncthreads();
  if (tid < npair * pp) red[tid] = acc;
  __syncthreads();
  if (tid < npair) {
    double tot = 0.0;
    for (int sh = 0; sh < pp; ++sh) tot += red[sh * npair + tid];
    out[k + tid] = tot;
  }
}

// One workgroup per row: merge the chunk partials in chunk order with Chan
// et al.'s pairwise update of the mean vector and the co-moment matrix.
// Thread e < k(k+1)/2 owns co-moment entry (i, j) and carries its own running
// copies of mu_i and mu_j (every thread applies the identical update, so the
// copies agree); threads e < k also carry mu_e.  Output per row:
// [mu_0 .. mu_{k-1}, S as a full k x k matrix].
__global__ __launch_bounds__(256) void gn0_merge_kernel(const double* __restrict__ part, int nchunk, int k, int T0,
                                                         const int32_t* __restrict__ rows_len,
                                                         double* __restrict__ merged) {
  constexpr int kBatch = 32;
  __shared__ double stage[kBatch * 152];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int Tb = rows_len ? rows_len[b] : T0;
  const int nuse = min(nchunk, (Tb + kStatChunk - 1) / kStatChunk);  // chunks holding frames of this row
  const int ns = k + k * (k + 1) / 2;
  const int npair = k * (k + 1) / 2;
  int pi = 0, pj = 0;
  if (tid < npair) {
    int rem = tid;
    while (rem >= k - pi) {
      rem -= k - pi;
      ++pi;
    }
    pj = pi + rem;
  }
  double mi = 0.0, mj = 0.0, me = 0.0, S = 0.0, n = 0.0;
  const double* src = part + (int64_t)b * nchunk * ns;
  for (int c0 = 0; c0 < nuse; c0 += kBatch) {
    const int nb = min(kBatch, nuse - c0);
    __syncthreads();
    // all loads of the batch issue before any store (their latencies overlap)
    for (int i0 = 0; i0 < nb * ns; i0 += 256 * 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 256 + tid;
        v[u] = i < nb * ns ? src[(int64_t)c0 * ns + i] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 256 + tid;
        if (i < nb * ns) stage[i] = v[u];
      }
    }
    __syncthreads();
    for (int c = 0; c < nb; ++c) {
      const double* pc = stage + c * ns;
      const double m = (double)min(kStatChunk, Tb - (c0 + c) * kStatChunk);
      const double nn = n + m;
      const double f = m / nn;
      if (tid < npair) {
        const double di = pc[pi] - mi, dj = pc[pj] - mj;
        S += pc[k + tid] + di * dj * n * f;
        mi += di * f;
        mj += dj * f;
      }
      if (tid < k) me += (pc[tid] - me) * f;
      n = nn;
    }
  }
  double* out = merged + (int64_t)b * (k + k * k);
  if (tid < k) out[tid] = me;
  if (tid < npair) {
    out[k + pi * k + pj] = S;
    out[k + pj * k + pi] = S;
  }
}

// Per (row, channel): mean = w.mu + bias, var = w^T S w / T0, then the affine
// GroupNorm map folded into scale = gamma * rstd, shift = beta - mean * scale.
__global__ __launch_bounds__(256) void gn0_finalize_kernel(const double* __restrict__ merged, int k, int T0,
                                                            const int32_t* __restrict__ rows_len,
                                                            const float* __restrict__ w0,
                                                            const float* __restrict__ bias, int C,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta, float eps,
                                                            float2* __restrict__ ss) {
  __shared__ double st[16 + 16 * 16];
  const int b = blockIdx.y;
  const double* src = merged + (int64_t)b * (k + k * k);
  for (int i = threadIdx.x; i < k + k * k; i += 256) st[i] = src[i];
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const float* w = w0 + (int64_t)c * k;
  double mean = bias ? (double)bias[c] : 0.0, q = 0.0;
  for (int i = 0; i < k; ++i) {
    const double wi = (double)w[i];
    mean += wi * st[i];
    double r = 0.0;
    for (int j = 0; j < k; ++j) r += st[k + i * k + j] * (double)w[j];
    q += wi * r;
  }
  const int Tb = rows_len ? rows_len[b] : T0;  // a row without frames never uses its scale and shift
  const double var = fmax(q / (double)max(Tb, 1), 0.0);
  const float rstd = (float)(1.0 / sqrt(var + (double)eps));
  const float scv = gamma[c] * rstd;
  ss[(int64_t)b * C + c] = make_float2(scv, beta[c] - (float)mean * scv);
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
                   const float* bias, int32_t C, int32_t k, int32_t stride, int32_t T0, RowSpan rows, void* y,
                   const float2* ss, const float* gamma, const float* beta, float eps, int32_t act,
                   hipStream_t s) {
  const int nchunk = (T0 + kChunk - 1) / kChunk;
  const int nsamp = (kChunk - 1) * stride + KT;
  const size_t lds = (size_t)((nsamp + 3) & ~3) * sizeof(float);
  hipLaunchKernelGGL((conv0_kernel<T, KT>), dim3(nchunk, B), dim3(256), lds, s, pcm, valid, L, w0, bias,
                     C, k, stride, T0, rows, (T*)y, ss, gamma, beta, eps, act);
  return hipGetLastError();
}

template <typename T>
hipError_t conv0_k(int k, const float* pcm, const int32_t* valid, int32_t L, int32_t B, const float* w0,
                   const float* bias, int32_t C, int32_t stride, int32_t T0, RowSpan rows, void* y,
                   const float2* ss, const float* gamma, const float* beta, float eps, int32_t act,
                   hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // GroupNorm layout, 9 or 10 taps, whole 64-channel slabs: matrix-core conv
    if (!gamma && (k == 9 || k == 10) && C % 64 == 0 && C <= kConv0MaxC) {
      constexpr int KS = 5;
      const int nchunk = (T0 + kChunk - 1) / kChunk;
      const int nx = (kChunk - 1) * stride + 2 * KS;
      const size_t lds = (size_t)C * 2 * KS * 4 + (size_t)C * 8 + (size_t)((nx + 3) & ~3) * 4 + 4 * 32 * 72 * 2;
      if (act == 2)
        hipLaunchKernelGGL((conv0_mfma_kernel<KS, 2>), dim3(nchunk, B), dim3(256), lds, s, pcm, valid, L, w0, bias,
                           C, k, stride, T0, rows, (half_t*)y, ss);
      else
        hipLaunchKernelGGL((conv0_mfma_kernel<KS, 1>), dim3(nchunk, B), dim3(256), lds, s, pcm, valid, L, w0, bias,
                           C, k, stride, T0, rows, (half_t*)y, ss);
      return hipGetLastError();
    }
  }
  if (k == 10)
    return conv0_t<T, 10>(pcm, valid, L, B, w0, bias, C, k, stride, T0, rows, y, ss, gamma, beta, eps, act, s);
  return conv0_t<T, 16>(pcm, valid, L, B, w0, bias, C, k, stride, T0, rows, y, ss, gamma, beta, eps, act, s);
}

}  // namespace

int64_t gn0_partial_doubles(int32_t k, int32_t T0) {
  const int64_t nchunk = (T0 + kStatChunk - 1) / kStatChunk;
  // chunk partials, then the merged statistics (k means + k x k co-moments)
  return nchunk * (k + k * (k + 1) / 2) + k + k * k;
}

hipError_t launch_conv0(DType t, const float* pcm, const int32_t* valid, int32_t L, int32_t B,
                        const float* w0, const float* bias, int32_t C, int32_t k, int32_t stride,
                        int32_t T0, RowSpan rows, void* y, const float2* ss, const float* gamma,
                        const float* beta, float eps, int32_t act, hipStream_t s) {
  if (t == DType::F16)
    return conv0_k<half_t>(k, pcm, valid, L, B, w0, bias, C, stride, T0, rows, y, ss, gamma, beta, eps, act, s);
  return conv0_k<float>(k, pcm, valid, L, B, w0, bias, C, stride, T0, rows, y, ss, gamma, beta, eps, act, s);
}

hipError_t launch_gn0_stats(const float* pcm, const int32_t* valid, int32_t L, int32_t B, int32_t k, int32_t stride,
                            int32_t T0, const int32_t* rows_len, double* part, hipStream_t s) {
  const int nchunk = (T0 + kStatChunk - 1) / kStatChunk;
  const size_t lds = (size_t)((kStatChunk - 1) * stride + k) * sizeof(float);
  hipLaunchKernelGGL(gn0_stats_kernel, dim3(nchunk, B), dim3(256), lds, s, pcm, valid, L, k, stride, T0, rows_len,
                     part);
  return hipGetLastError();
}

hipError_t launch_gn0_finalize(double* part, int32_t B, int32_t k, int32_t T0, const int32_t* rows_len,
                               const float* w0, const float* bias, int32_t C, const float* gamma,
                               const float* beta, float eps, float2* ss, hipStream_t s) {
  const int nchunk = (T0 + kStatChunk - 1) / kStatChunk;
  double* merged = part + (int64_t)B * nchunk * (k + k * (k + 1) / 2);
  hipLaunchKernelGGL(gn0_merge_kernel, dim3(B), dim3(256), 0, s, part, nchunk, k, T0, rows_len, merged);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gn0_finalize_kernel, dim3((C + 255) / 256, B), dim3(256), 0, s, merged, k, T0, rows_len, w0,
                     bias, C, gamma, beta, eps, ss);
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
