// Greedy CTC decoding on the device: per-frame argmax over the vocabulary,
// then per row "merge runs of equal ids, drop the blank" over the valid
// frames, compacted with a block-wide prefix sum.
//
// frame_argmax: one wave per frame, lanes stride over the vocabulary and the
// (value, index) pairs are merged with the lowest index winning ties, so the
// result equals numpy's first-maximum argmax whatever the reduction order.
// ctc_collapse: one workgroup per row; the row's argmax path is first copied
// to LDS, so the compaction can write the ids in place over it.  The path
// comes either from frame_argmax (in ids) or from the per-frame argmax keys
// that the CTC head's GEMM epilogue raises (argmax_key in common.h), which
// saves the second pass over the [B, T, V] logits.
#include <limits.h>

#include "common.h"

namespace w2v2 {
namespace {

__device__ inline bool better(float bv, int bi, float av, int ai) {
  // is (bv, bi) preferred over (av, ai)?
  if (ai == INT_MAX) return bi != INT_MAX;
  if (bi == INT_MAX) return false;
  return (bv > av) || (bv == av && bi < ai);
}

__global__ __launch_bounds__(256) void frame_argmax_kernel(const float* __restrict__ logits, int64_t rows, int V,
                                                           int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* x = logits + row * V;
  float best = 0.f;
  int bi = INT_MAX;
  for (int v = lane; v < V; v += 64) {
    const float val = x[v];
    if (bi == INT_MAX || val > best) {
      best = val;
      bi = v;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, best, bi)) {
      best = ov;
      bi = oi;
    }
  }
  if (lane == 0) out[row] = (bi == INT_MAX) ? 0 : bi;
}

// keys == null: the argmax path is in ids (frame_argmax wrote it there);
// otherwise it is given by the argmax keys (see argmax_key) of each frame.
__global__ __launch_bounds__(1024) void ctc_collapse_kernel(const uint64_t* __restrict__ keys,
                                                            const int32_t* __restrict__ vframes, int T, int blank,
                                                            int32_t* ids, int32_t* __restrict__ lens) {
  extern __shared__ int32_t path[];  // [T]
  __shared__ int32_t wtot[16];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* row = ids + (int64_t)b * T;
  if (keys) {
    for (int t = tid; t < T; t += 1024) path[t] = (int32_t)(0xFFFFFFFFu - (uint32_t)keys[(int64_t)b * T + t]);
  } else {
    for (int t = tid; t < T; t += 1024) path[t] = row[t];
  }
  int vf = vframes[b];
  vf = vf < 0 ? 0 : (vf > T ? T : vf);
  __syncthreads();

  int offset = 0;
  for (int c0 = 0; c0 < vf; c0 += 1024) {
    const int t = c0 + tid;
    bool keep = false;
    int a = 0;
    if (t < vf) {
      a = path[t];
      keep = (a != blank) && (t == 0 || a != path[t - 1]);
    }
    const unsigned long long m = __ballot(keep);
    const int pre = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[wave] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int v = wtot[w];
      before += (w < wave) ? v : 0;
      total += v;
    }
    if (keep) row[offset + before + pre] = a;
    offset += total;
    __syncthreads();
  }
  for (int t = offset + tid; t < T; t += 1024) row[t] = -1;
  if (tid == 0) lens[b] = offset;
}

// Argmax slots start at 0, below every key, before a GEMM raises them (a
// fill kernel, not a memset, so that the forward can be graph-captured).
__global__ __launch_bounds__(256) void zero_keys_kernel(uint64_t* __restrict__ keys, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) keys[i] = 0;
}

}  // namespace

hipError_t launch_frame_argmax(const float* logits, int64_t rows, int32_t V, int32_t* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(frame_argmax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, logits, rows, V, out);
  return hipGetLastError();
}

hipError_t launch_ctc_collapse(const int32_t* vframes, int32_t B, int32_t T, int32_t blank, int32_t* ids,
                               int32_t* lens, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(ctc_collapse_kernel, dim3(B), dim3(1024), (size_t)T * sizeof(int32_t), s, nullptr, vframes, T,
                     blank, ids, lens);
  return hipGetLastError();
}

hipError_t launch_ctc_collapse_keys(const uint64_t* keys, const int32_t* vframes, int32_t B, int32_t T,
                                    int32_t blank, int32_t* ids, int32_t* lens, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(ctc_collapse_kernel, dim3(B), dim3(1024), (size_t)T * sizeof(int32_t), s, keys, vframes, T,
                     blank, ids, lens);
  return hipGetLastError();
}

hipError_t launch_zero_keys(uint64_t* keys, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t g = (n + 255) / 256;
  hipLaunchKernelGGL(zero_keys_kernel, dim3((unsigned)(g < 65535 ? g : 65535)), dim3(256), 0, s, keys, n);
  return hipGetLastError();
}

}  // namespace w2v2
