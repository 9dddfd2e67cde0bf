// Tree-masked verify attention: mask packing for gfx950.
//
// The visibility mask is one byte per (draft, key) with row stride L_b inside
// each request's block (page 2 "Flipping the Switch", section "The Long Road to
// Parity": mask=(270,) for 9 drafts x 30 keys; page 3 "The Pivot to Live
// Cutover", section "The Technical Investigation": the block of request b is
// located through mask_indptr).  The split kernel reads it as one 32-bit word
// per (draft token, 32-key tile), built here with wave ballots.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_kernels.h"

namespace tv {

// Word (token qo_indptr[b] + i, tile) bit k = mask byte of key 32*tile + k of draft i.
// Each half-wave (32 lanes) builds one word; keys at or past L_b give 0.
__global__ __launch_bounds__(256) void tv_pack_mask_kernel(PackParams p) {
  const int b = blockIdx.y;
  const int q0 = p.qo_indptr[b];
  const int n = p.qo_indptr[b + 1] - q0;
  const int L = p.kv_indptr[b + 1] - p.kv_indptr[b];
  const int tiles = (L + TILE_KEYS - 1) / TILE_KEYS;
  const int words = n * tiles;
  const int w = blockIdx.x * 8 + (threadIdx.x >> 5);
  const int k = threadIdx.x & 31;
  bool vis = false;
  int i = 0, tile = 0;
  if (w < words) {
    i = w / tiles;
    tile = w - i * tiles;
    const int key = tile * TILE_KEYS + k;
    if (key < L) vis = p.mask[p.mask_indptr[b] + (int64_t)i * L + key] != 0;
  }
  const uint64_t bits = __ballot(vis);
  if (w < words && k == 0) {
    const uint32_t word = (threadIdx.x & 32) ? (uint32_t)(bits >> 32) : (uint32_t)bits;
    p.words[(int64_t)(q0 + i) * p.max_tiles + tile] = word;
  }
}

hipError_t launch_pack(const PackParams& p, int grid_x, int batch, hipStream_t st) {
  PackParams a = p;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&tv_pack_mask_kernel), dim3(grid_x, batch),
                         dim3(256), args, 0, st);
}
}  // namespace tv
