// Tree-masked verify attention: mask packing for gfx950.
//
// The visibility mask is one byte per (draft, key) with row stride L_b inside
// each request's block (page 2 "Flipping the Switch", section "The Long Road to
// Parity": mask=(270,) for 9 drafts x 30 keys; page 3 "The Pivot to Live
// Cutover", section "The Technical Investigation": the block of request b is
// located through mask_indptr).  When a wave's rows span more draft tokens
// than the split kernel reads mask bytes for, it reads one 32-bit word per
// (draft token, 32-key tile) instead, built here with wave ballots.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_kernels.h"

namespace tv {

// Word (token qo_indptr[b] + i, tile) bit k = mask byte of key 32*tile + k of draft i;
// keys at or past L_b give 0.  In the prefix-visible form the block holds the
// draft keys only (n_b x n_b bytes) and the bits of the prefix keys are 1.  One
// wave per PACK_SEGS * 64 keys of a draft row: lane l reads key 64j + l of each
// 64-key segment j (one coalesced 64-byte load per segment), and the segment's
// ballot is its two words; lanes 0..2*PACK_SEGS-1 then store one word each.
constexpr int PACK_SEGS = PACK_KEYS / 64;

// Longest-first dispatch order of the split kernel's work items, by one
// workgroup: the splits (b, s) that exist are bucketed by their key count
// (SCHED_BUCKETS classes, longest first; a counting sort), and each takes as many
// consecutive positions as its request has row blocks, one per row block, so
// the row blocks of a split stay together.  Positions left over hold -1.  With
// the hardware dispatching workgroups in position order as compute units free
// up, this is greedy longest-processing-time scheduling.
__device__ void schedule_work(const PackParams& p) {
  constexpr int PER = SCHED_BUCKETS / 256;  // buckets per thread in the scan
  static_assert(SCHED_BUCKETS % 256 == 0, "");
  __shared__ int cnt[SCHED_BUCKETS];
  __shared__ int wsum[4];
  const int t = threadIdx.x;
  for (int i = t; i < SCHED_BUCKETS; i += 256) cnt[i] = 0;
  __syncthreads();
  const int units = p.batch * p.max_splits;
  // bucket of a split and the row blocks it holds (0: the split does not exist)
  auto classify = [&](int u, int& bucket) -> int {
    const int b = u / p.max_splits, s = u - b * p.max_splits;
    const int L = p.kv_indptr[b + 1] - p.kv_indptr[b];
    const int nsplit = L > 0 ? (L + p.split_keys - 1) / p.split_keys : 1;
    if (s >= nsplit) return 0;
    const int keys = L > 0 ? min(L - s * p.split_keys, p.split_keys) : 0;
    bucket = (int)((int64_t)(p.split_keys - keys) * (SCHED_BUCKETS - 1) / p.split_keys);
    const int rows = (p.qo_indptr[b + 1] - p.qo_indptr[b]) * p.num_heads;
    return (rows + ROWS_PER_WG - 1) / ROWS_PER_WG;
  };
  for (int u = t; u < units; u += 256) {
    int bucket;
    const int rbs = classify(u, bucket);
    if (rbs > 0) atomicAdd(&cnt[bucket], rbs);
  }
  __syncthreads();
  // exclusive prefix sum over the buckets, longest class first: each thread
  // scans PER consecutive buckets, the wave scans its threads' totals, the
  // workgroup adds the totals of the waves before
  int v[PER];
  int run = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    v[k] = run;
    run += cnt[PER * t + k];
  }
  const int lane = t & 63, wave = t >> 6;
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = incl - run;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
#pragma unroll
  for (int k = 0; k < PER; ++k) cnt[PER * t + k] = base + v[k];
  // positions past the existing work items hold -1
  for (int i = total + t; i < p.total_work; i += 256) p.order[i] = -1;
  __syncthreads();
  for (int u = t; u < units; u += 256) {
    int bucket;
    const int rbs = classify(u, bucket);
    if (rbs == 0) continue;
    const int start = atomicAdd(&cnt[bucket], rbs);
    for (int rb = 0; rb < rbs; ++rb) p.order[start + rb] = u * p.row_blocks + rb;
  }
}

__global__ __launch_bounds__(256) void tv_pack_mask_kernel(PackParams p) {
  if ((int)blockIdx.x == p.sched_block) {
    if (blockIdx.y == 0) schedule_work(p);
    return;
  }
  const int b = blockIdx.y;
  const int q0 = p.qo_indptr[b];
  const int n = p.qo_indptr[b + 1] - q0;
  const int L = p.kv_indptr[b + 1] - p.kv_indptr[b];
  const int tiles = (L + TILE_KEYS - 1) / TILE_KEYS;
  const int chunks = (L + 64 * PACK_SEGS - 1) / (64 * PACK_SEGS);
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);  // wave-uniform
  if (unit >= n * chunks) return;
  const int i = unit / chunks;
  const int c = unit - i * chunks;
  const int lane = threadIdx.x & 63;
  const int k0 = c * 64 * PACK_SEGS + lane;
  uint8_t v[PACK_SEGS];
  if (p.prefix_visible) {
    // draft keys only: key k >= P of draft i is byte i * n + (k - P) of the
    // block; every prefix key is visible (L >= n is a precondition)
    const int P = L - n;
    const uint8_t* m = p.mask + p.mask_indptr[b] + (int64_t)i * n;
#pragma unroll
    for (int j = 0; j < PACK_SEGS; ++j) {
      const int k = k0 + 64 * j;
      v[j] = k >= L ? 0 : (k < P ? 1 : m[k - P]);
    }
  } else {
    const uint8_t* m = p.mask + p.mask_indptr[b] + (int64_t)i * L;
#pragma unroll
    for (int j = 0; j < PACK_SEGS; ++j) {
      const int k = k0 + 64 * j;
      v[j] = k < L ? m[k] : 0;
    }
  }
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < PACK_SEGS; ++j) {
    const unsigned long long bal = __ballot(v[j] != 0);
    if (lane == 2 * j) mine = (uint32_t)bal;
    if (lane == 2 * j + 1) mine = (uint32_t)(bal >> 32);
  }
  const int tile = c * 2 * PACK_SEGS + lane;
  // (tiles past max_tiles exist only for a request longer than max_kv_len, a
  // broken precondition: their words are not stored, so the row stays inside)
  if (lane < 2 * PACK_SEGS && tile < min(tiles, p.max_tiles))
    p.words[(int64_t)(q0 + i) * p.max_tiles + tile] = mine;
}

hipError_t launch_pack(const PackParams& p, int grid_x, int batch, hipStream_t st) {
  PackParams a = p;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&tv_pack_mask_kernel), dim3(grid_x, batch),
                         dim3(256), args, 0, st);
}
}  // namespace tv
