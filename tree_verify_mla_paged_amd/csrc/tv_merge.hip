// Tree-masked verify attention: LSE merge of the KV splits for gfx950.
//
// Each split of a row holds a normalised partial output o_s and its natural
// log-sum-exp lse_s (page 2 "Flipping the Switch", section "The Broader
// Context": splits run in parallel and are combined by their LSE).  With
// M = max_s lse_s and w_s = exp(lse_s - M):  out = sum_s w_s o_s / sum_s w_s,
// lse = M + ln sum_s w_s.  A row whose splits are all empty (lse_s = -inf)
// gets out = 0, lse = -inf.  Partials are fp32, or fp16 h_s with a scale
// exponent k_s (o_s = h_s 2^k_s, folded into the split's weight exactly).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tv_kernels.h"

namespace tv {

// One row per workgroup, in chunks of up to MERGE_CHUNK splits.  The chunk's
// split LSEs are read once, cooperatively, and turned into weights in LDS;
// then every partial-output load is issued with its weight already known (no
// load waits on another), U per thread in flight.  Thread t owns value dims
// 4*(t & 127) .. +3; the two halves of the workgroup take alternate splits and
// combine through LDS.  Weights are relative to the running maximum M and are
// rescaled when a later chunk raises it.
constexpr int MERGE_CHUNK = 1024;

// Maximum over the workgroup (256 threads); ends with a barrier.
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

template <int OUT, bool F16P>
__global__ __launch_bounds__(256) void tv_merge_kernel(MergeParams p) {
  constexpr int U = 16;
  __shared__ float wgt_s[MERGE_CHUNK];               // w_s
  __shared__ float wnum_s[F16P ? MERGE_CHUNK : 1];   // w_s 2^k_s
  __shared__ f32x4 part_o[128];
  __shared__ float part_w[128];
  __shared__ float red[4];
  const int b = blockIdx.y;
  const int q0 = p.qo_indptr[b];
  const int R = (p.qo_indptr[b + 1] - q0) * p.num_heads;
  const int r = blockIdx.x;
  if (r >= R) return;
  const int L = p.kv_indptr[b + 1] - p.kv_indptr[b];
  const int ns = L > 0 ? (L + p.split_keys - 1) / p.split_keys : 1;
  if (ns <= 1) return;  // written directly by the split kernel
  const int64_t g = (int64_t)q0 * p.num_heads + r;
  const int LS = F16P ? 2 : 1;  // floats per (row, split) in ws_lse
  const float* ls = p.ws_lse + g * p.max_splits * LS;
  const int t = threadIdx.x;
  const int d = (t & 127) * 4;
  const int h = t >> 7;
  const float* po = static_cast<const float*>(p.ws_o) + g * p.max_splits * VD + d;
  const _Float16* ph = static_cast<const _Float16*>(p.ws_o) + g * p.max_splits * VD + d;

  float M = -INFINITY;  // running maximum of the split LSEs
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float W = 0.f;  // this thread's share of sum_s exp(lse_s - M)
  for (int c0 = 0; c0 < ns; c0 += MERGE_CHUNK) {
    const int nc = min(MERGE_CHUNK, ns - c0);
    float m = -INFINITY;
    for (int i = t; i < nc; i += 256) {
      const float v = ls[LS * (c0 + i)];
      wgt_s[i] = v;
      m = fmaxf(m, v);
    }
    const float Mn = fmaxf(M, block_max(m, red));
    if (Mn == -INFINITY) continue;  // every split so far is empty (uniform)
    if (Mn > M) {
      // (w_s and w_s 2^k_s share the factor)
      const float f = M == -INFINITY ? 0.f : __expf(M - Mn);
      acc *= f;
      W *= f;
      M = Mn;
    }
    for (int i = t; i < nc; i += 256) {
      const float w = __expf(wgt_s[i] - M);  // exp(-inf) = 0
      wgt_s[i] = w;
      if (F16P) wnum_s[i] = __builtin_ldexpf(w, (int)ls[LS * (c0 + i) + 1]);
    }
    __syncthreads();
    for (int s0 = h; s0 < nc; s0 += 2 * U) {
      f32x4 v[U];
      f16x4 vh[U];
      float wv[U], wn[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int s = s0 + 2 * j;
        wv[j] = s < nc ? wgt_s[s] : 0.f;
        if (F16P) {
          wn[j] = s < nc ? wnum_s[s] : 0.f;
          vh[j] = wv[j] > 0.f ? *reinterpret_cast<const f16x4*>(ph + (int64_t)(c0 + s) * VD)
                              : f16x4{};
        } else {
          v[j] = wv[j] > 0.f ? *reinterpret_cast<const f32x4*>(po + (int64_t)(c0 + s) * VD)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (F16P) {
          acc += wn[j] * f32x4{(float)vh[j][0], (float)vh[j][1], (float)vh[j][2],
                               (float)vh[j][3]};
        } else {
          acc += wv[j] * v[j];
        }
        W += wv[j];
      }
    }
    __syncthreads();  // wgt_s is rewritten by the next chunk
  }
  if (h == 1) {
    part_o[t & 127] = acc;
    part_w[t & 127] = W;
  }
  __syncthreads();
  if (h == 1) return;
  acc += part_o[t];
  W += part_w[t];
  if (M != -INFINITY) acc *= 1.f / W;
  const float lse = (M == -INFINITY) ? -INFINITY : M + logf(W);
  if (t == 0) p.lse[g] = lse;
  if (OUT == OUT_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + g * VD + d) = acc;
  } else {
    bf16x4 o;
    o[0] = (__bf16)acc[0];
    o[1] = (__bf16)acc[1];
    o[2] = (__bf16)acc[2];
    o[3] = (__bf16)acc[3];
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + g * VD + d) = o;
  }
}

hipError_t launch_merge(const MergeParams& p, int grid_x, int batch, int out, bool f16_parts,
                        hipStream_t st) {
  MergeParams a = p;
  void* args[] = {&a};
  // [out dtype][fp16 partials]
  static const void* const fns[2][2] = {
      {reinterpret_cast<const void*>(&tv_merge_kernel<OUT_BF16, false>),
       reinterpret_cast<const void*>(&tv_merge_kernel<OUT_BF16, true>)},
      {reinterpret_cast<const void*>(&tv_merge_kernel<OUT_F32, false>),
       reinterpret_cast<const void*>(&tv_merge_kernel<OUT_F32, true>)}};
  const void* fn = fns[out == OUT_F32][f16_parts];
  return hipLaunchKernel(fn, dim3(grid_x, batch), dim3(256), args, 0, st);
}
}  // namespace tv
