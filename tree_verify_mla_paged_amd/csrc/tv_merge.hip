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

// One workgroup of 256 threads per (row, slice of VD / DS value dims), in
// chunks of up to MERGE_CHUNK splits.  DS = 4 spreads the rows of a small
// problem over four times as many compute units (each reads a quarter of every
// partial row; the weights are recomputed per slice).  A chunk's split LSEs
// are read first, once, cooperatively; then a thread's first U partial-output
// loads go out, and while they are in flight the LSEs are turned into weights
// in LDS, so that each partial is accumulated as it lands.
// Each load is 16 bytes: a thread owns DPT value dims (8 fp16 or 4 fp32), so a
// split's slice takes TPS threads and the workgroup's NPH = 256 / TPS phases
// take alternate splits, combined through LDS at the end: NPH * U splits are
// in flight at once.  Weights are relative to the running maximum M and are
// rescaled when a later chunk raises it.
constexpr int MERGE_CHUNK = 1024;

constexpr int NT = 256;  // threads per workgroup

// Maximum over the workgroup; ends with a barrier.
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

template <int OUT, bool F16P, int DS>
__global__ __launch_bounds__(NT) void tv_merge_kernel(MergeParams p) {
  constexpr int U = 16;               // loads per thread in flight
  constexpr int DPT = F16P ? 8 : 4;  // value dims per thread: one 16-byte load
  constexpr int TPS = VD / DS / DPT; // threads per split row slice
  constexpr int NPH = NT / TPS;      // splits in flight across the workgroup
  typedef float accv __attribute__((ext_vector_type(DPT)));
  __shared__ float wgt_s[MERGE_CHUNK];               // w_s
  __shared__ float wnum_s[F16P ? MERGE_CHUNK : 1];   // w_s 2^k_s
  __shared__ accv part_o[NPH - 1][TPS];
  __shared__ float part_w[NPH - 1][TPS];
  __shared__ float red[NT / 64];
  const int b = blockIdx.y;
  const int q0 = p.qo_indptr[b];
  const int R = (p.qo_indptr[b + 1] - q0) * p.num_heads;
  const int r = blockIdx.x / DS;
  const int slice = blockIdx.x % DS;
  if (r >= R) return;
  const int L = p.kv_indptr[b + 1] - p.kv_indptr[b];
  // (clamped to the plan: a request longer than max_kv_len breaks the
  // preconditions, and then reads stay inside the row's partials)
  const int ns = min(L > 0 ? (L + p.split_keys - 1) / p.split_keys : 1, p.max_splits);
  if (ns <= 1) return;  // written directly by the split kernel
  const int64_t g = (int64_t)q0 * p.num_heads + r;
  const int LS = F16P ? 2 : 1;  // floats per (row, split) in ws_lse
  const float* ls = p.ws_lse + g * p.max_splits * LS;
  const int t = threadIdx.x;
  const int d = slice * (VD / DS) + (t % TPS) * DPT;
  const int h = t / TPS;  // phase: splits h, h + NPH, ...
  const float* po = static_cast<const float*>(p.ws_o) + g * p.max_splits * VD + d;
  const _Float16* ph = static_cast<const _Float16*>(p.ws_o) + g * p.max_splits * VD + d;

  float M = -INFINITY;  // running maximum of the split LSEs
  accv acc = accv{};
  float W = 0.f;  // this thread's share of sum_s exp(lse_s - M)
  f32x4 v[U];
  f16x8 vh[U];
  // the partial outputs of splits c0 + s0 + NPH*j: every split below ns was
  // written by the split kernel (an empty one as zeros), so these loads need
  // no weight and go out before the weights are known.  A split past ns loads
  // split ns - 1 again, with weight 0 below: the loads are unconditional, so
  // the compiler counts them exactly when it waits for the older LSE loads (a
  // load under a branch makes it wait for every load in flight).
  auto load_batch = [&](int c0, int s0) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int s = min(c0 + s0 + NPH * j, ns - 1);
      if (F16P) vh[j] = *reinterpret_cast<const f16x8*>(ph + (int64_t)s * VD);
      else v[j] = *reinterpret_cast<const f32x4*>(po + (int64_t)s * VD);
    }
  };
  constexpr int PER = MERGE_CHUNK / NT;  // a thread's share of a chunk's splits
  for (int c0 = 0; c0 < ns; c0 += MERGE_CHUNK) {
    const int nc = min(MERGE_CHUNK, ns - c0);
    // the chunk's split LSEs (and scale exponents) go out first: vector loads
    // return in issue order, so behind the partial rows they would wait for
    // all of them, and no accumulation could start before the last row landed
    // (unconditional loads of a clamped split, then a select: a load under a
    // branch would be followed by a wait for every load in flight)
    float lvs[PER], kxs[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = t + NT * u;
      const int ic = c0 + min(i, nc - 1);
      const float lv = ls[LS * ic];
      const float kx = F16P ? ls[LS * ic + 1] : 0.f;
      lvs[u] = i < nc ? lv : -INFINITY;
      kxs[u] = i < nc ? kx : 0.f;
    }
    asm volatile("" ::: "memory");  // (issue order)
    load_batch(c0, h);
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < PER; ++u) m = fmaxf(m, lvs[u]);
    const float Mn = fmaxf(M, block_max(m, red));
    if (Mn == -INFINITY) continue;  // every split so far is empty (uniform)
    if (Mn > M) {
      // (w_s and w_s 2^k_s share the factor)
      const float f = M == -INFINITY ? 0.f : __expf(M - Mn);
      acc *= f;
      W *= f;
      M = Mn;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = t + NT * u;
      if (i < nc) {
        const float w = __expf(lvs[u] - M);  // exp(-inf) = 0
        wgt_s[i] = w;
        if (F16P) wnum_s[i] = __builtin_ldexpf(w, (int)kxs[u]);
      }
    }
    __syncthreads();
    for (int s0 = h; s0 < nc; s0 += NPH * U) {
      if (s0 != h) load_batch(c0, s0);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int s = s0 + NPH * j;
        const float wv = s < nc ? wgt_s[s] : 0.f;
        if constexpr (F16P) {
          const float wn = s < nc ? wnum_s[s] : 0.f;
#pragma unroll
          for (int e = 0; e < DPT; ++e) acc[e] += wn * (float)vh[j][e];
        } else {
#pragma unroll
          for (int e = 0; e < DPT; ++e) acc[e] += wv * v[j][e];
        }
        W += wv;
      }
    }
    __syncthreads();  // wgt_s is rewritten by the next chunk
  }
  if (h > 0) {
    part_o[h - 1][t % TPS] = acc;
    part_w[h - 1][t % TPS] = W;
  }
  __syncthreads();
  if (h > 0) return;
#pragma unroll
  for (int k = 0; k < NPH - 1; ++k) {
    acc += part_o[k][t];
    W += part_w[k][t];
  }
  if (M != -INFINITY) acc *= 1.f / W;
  const float lse = (M == -INFINITY) ? -INFINITY : M + logf(W);
  if (t == 0 && slice == 0) p.lse[g] = lse;
#pragma unroll
  for (int e0 = 0; e0 < DPT; e0 += 4) {
    const f32x4 o4 = f32x4{acc[e0], acc[e0 + 1], acc[e0 + 2], acc[e0 + 3]};
    if (OUT == OUT_F32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + g * VD + d + e0) = o4;
    } else {
      bf16x4 o;
      o[0] = (__bf16)o4[0];
      o[1] = (__bf16)o4[1];
      o[2] = (__bf16)o4[2];
      o[3] = (__bf16)o4[3];
      *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + g * VD + d + e0) = o;
    }
  }
}

// Requests split at most merge_wave_splits(F16P) ways: one wave per row, four rows
// per workgroup.  Lane s holds split s's lse (and scale exponent); every lane
// owns 8 value dims and issues the loads of all the row's splits at once,
// before the weights are known; the weights come from wave reductions, with no
// LDS and no barrier.  Same arithmetic as tv_merge_kernel: M = max_s lse_s,
// w_s = exp(lse_s - M), out = sum_s w_s 2^k_s h_s / sum_s w_s, lse = M + ln sum_s w_s.
//
// The loads are unconditional (a split past ns loads split ns - 1 again and is
// not used), so that the compiler's waits count them exactly: a load under a
// branch is followed by a wait for every load in flight.  CAP, the number
// issued, is the smallest of 4, 8, 16, 32 that holds ns (one instantiation
// each, chosen by a branch that is uniform over the workgroup: its rows share
// a request), so a row of few splits issues few loads.
template <int OUT, bool F16P, int CAP>
__device__ __forceinline__ void merge_row(const MergeParams& p, int64_t g, int ns, int lane) {
  const int LS = F16P ? 2 : 1;
  const float* ls = p.ws_lse + g * p.max_splits * LS;
  const int d = lane * 8;
  // lane s's split lse and scale exponent first (vector loads return in issue
  // order: behind the partial rows they would wait for all of them)
  const int sc = min(lane, ns - 1);
  const float lv0 = ls[LS * sc];
  const float kx0 = F16P ? ls[LS * sc + 1] : 0.f;
  const float lv = lane < ns ? lv0 : -INFINITY;
  const float kx = lane < ns ? kx0 : 0.f;
  asm volatile("" ::: "memory");  // (issue order)
  f16x8 vh[CAP];
  f32x4 v0[CAP], v1[CAP];
#pragma unroll
  for (int s = 0; s < CAP; ++s) {
    const int sl = min(s, ns - 1);
    if (F16P) {
      vh[s] = *reinterpret_cast<const f16x8*>(static_cast<const _Float16*>(p.ws_o) +
                                              (g * p.max_splits + sl) * VD + d);
    } else {
      const float* po = static_cast<const float*>(p.ws_o) + (g * p.max_splits + sl) * VD + d;
      v0[s] = *reinterpret_cast<const f32x4*>(po);
      v1[s] = *reinterpret_cast<const f32x4*>(po + 4);
    }
  }
  // the reductions below wait for the lse: keep them after the row loads
  __builtin_amdgcn_sched_barrier(0);
  float M = lv;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float lse = -INFINITY;
  if (M != -INFINITY) {  // uniform
    const float w = __expf(lv - M);  // exp(-inf) = 0 for lanes past ns and empty splits
    float W = w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) W += __shfl_xor(W, o);
    const float wn = F16P ? __builtin_ldexpf(w, (int)kx) : w;
#pragma unroll
    for (int s = 0; s < CAP; ++s) {
      if (s < ns) {
        const float ws = __shfl(wn, s);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] += ws * (F16P ? (float)vh[s][e] : (e < 4 ? v0[s][e] : v1[s][e - 4]));
      }
    }
    const float inv = 1.f / W;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    lse = M + logf(W);
  }
  if (lane == 0) p.lse[g] = lse;
  if (OUT == OUT_F32) {
    float* o = static_cast<float*>(p.out) + g * VD + d;
    *reinterpret_cast<f32x4*>(o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[e];
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.out) + g * VD + d) = o;
  }
}

template <int OUT, bool F16P>
__global__ __launch_bounds__(NT) void tv_merge_rows_kernel(MergeParams p) {
  constexpr int MS = merge_wave_splits(F16P);
  static_assert(MS == 16 || MS == 32, "");
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);  // wave-uniform
  const int q0 = p.qo_indptr[b];
  const int R = (p.qo_indptr[b + 1] - q0) * p.num_heads;
  if (r >= R) return;
  const int L = p.kv_indptr[b + 1] - p.kv_indptr[b];
  const int ns = min(min(L > 0 ? (L + p.split_keys - 1) / p.split_keys : 1, MS), p.max_splits);
  if (ns <= 1) return;  // written directly by the split kernel
  const int64_t g = (int64_t)q0 * p.num_heads + r;
  if (ns <= 4) merge_row<OUT, F16P, 4>(p, g, ns, lane);
  else if (ns <= 8) merge_row<OUT, F16P, 8>(p, g, ns, lane);
  else if (MS == 16 || ns <= 16) merge_row<OUT, F16P, 16>(p, g, ns, lane);
  else merge_row<OUT, F16P, MS>(p, g, ns, lane);
}

hipError_t launch_merge_rows(const MergeParams& p, int rows, int batch, int out, bool f16_parts,
                             hipStream_t st) {
  MergeParams a = p;
  void* args[] = {&a};
  static const void* const fns[2][2] = {
      {reinterpret_cast<const void*>(&tv_merge_rows_kernel<OUT_BF16, false>),
       reinterpret_cast<const void*>(&tv_merge_rows_kernel<OUT_BF16, true>)},
      {reinterpret_cast<const void*>(&tv_merge_rows_kernel<OUT_F32, false>),
       reinterpret_cast<const void*>(&tv_merge_rows_kernel<OUT_F32, true>)}};
  const int wpg = NT / 64;
  return hipLaunchKernel(fns[out == OUT_F32][f16_parts], dim3((rows + wpg - 1) / wpg, batch),
                         dim3(NT), args, 0, st);
}

hipError_t launch_merge(const MergeParams& p, int rows, int batch, int out, bool f16_parts,
                        bool sliced, hipStream_t st) {
  MergeParams a = p;
  void* args[] = {&a};
  // [out dtype][fp16 partials][4 slices]
  static const void* const fns[2][2][2] = {
      {{reinterpret_cast<const void*>(&tv_merge_kernel<OUT_BF16, false, 1>),
        reinterpret_cast<const void*>(&tv_merge_kernel<OUT_BF16, false, 4>)},
       {reinterpret_cast<const void*>(&tv_merge_kernel<OUT_BF16, true, 1>),
        reinterpret_cast<const void*>(&tv_merge_kernel<OUT_BF16, true, 4>)}},
      {{reinterpret_cast<const void*>(&tv_merge_kernel<OUT_F32, false, 1>),
        reinterpret_cast<const void*>(&tv_merge_kernel<OUT_F32, false, 4>)},
       {reinterpret_cast<const void*>(&tv_merge_kernel<OUT_F32, true, 1>),
        reinterpret_cast<const void*>(&tv_merge_kernel<OUT_F32, true, 4>)}}};
  const void* fn = fns[out == OUT_F32][f16_parts][sliced];
  return hipLaunchKernel(fn, dim3(rows * (sliced ? 4 : 1), batch), dim3(NT), args, 0, st);
}
}  // namespace tv
