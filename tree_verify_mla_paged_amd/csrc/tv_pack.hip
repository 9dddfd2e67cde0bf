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

// Word (token qo_indptr[b] + i, tile) bit k = mask byte of key 32*tile + k of draft i;
// keys at or past L_b give 0.  One word per thread: consecutive threads take
// consecutive tiles of a draft row, so a wave reads 64 consecutive 32-byte
// runs, all 32 byte loads of a thread in flight at once.
__global__ __launch_bounds__(256) void tv_pack_mask_kernel(PackParams p) {
  const int b = blockIdx.y;
  const int q0 = p.qo_indptr[b];
  const int n = p.qo_indptr[b + 1] - q0;
  const int L = p.kv_indptr[b + 1] - p.kv_indptr[b];
  const int tiles = (L + TILE_KEYS - 1) / TILE_KEYS;
  const int w = blockIdx.x * 256 + threadIdx.x;
  if (w >= n * tiles) return;
  const int i = w / tiles;
  const int tile = w - i * tiles;
  const int nk = min(TILE_KEYS, L - tile * TILE_KEYS);
  const uint8_t* m = p.mask + p.mask_indptr[b] + (int64_t)i * L + tile * TILE_KEYS;
  uint8_t v[TILE_KEYS];
#pragma unroll
  for (int k = 0; k < TILE_KEYS; ++k) v[k] = k < nk ? m[k] : 0;
  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < TILE_KEYS; ++k) word |= (v[k] != 0 ? 1u : 0u) << k;
  p.words[(int64_t)(q0 + i) * p.max_tiles + tile] = word;
}

hipError_t launch_pack(const PackParams& p, int grid_x, int batch, hipStream_t st) {
  PackParams a = p;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&tv_pack_mask_kernel), dim3(grid_x, batch),
                         dim3(256), args, 0, st);
}
}  // namespace tv
