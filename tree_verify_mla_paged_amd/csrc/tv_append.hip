// Tree-masked verify attention: the marshaling step before the attention call,
// for gfx950.
//
// The pages' parity failure came from this step (page 2 "Flipping the Switch",
// section "The Long Road to Parity"): the draft tokens' latent rows must be in
// the pool at their slots, and those slots must follow the prefix slots in
// kv_indices, with the visibility mask laid out at row stride prefix + drafts.
// Here it is one capture-safe call of two launches:
//   tv_append_scan_kernel  (one workgroup) kv_indptr[b] = prefix_indptr[b] +
//                          qo_indptr[b], and mask_indptr as the running sum of
//                          the requests' mask blocks;
//   tv_append_fill_kernel  the draft rows into the pool, kv_indices, and the
//                          mask bytes of the draft trees.
// Every store is bounded by the capacities the host passes, so indptrs or
// parents that break the preconditions give wrong contents, never a store
// outside a buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_kernels.h"

namespace tv {

// Request b's blocks: kv_indptr[b] = prefix_indptr[b] + qo_indptr[b] (both are
// prefix sums, so this is their sum's prefix sum), and mask_indptr[b] = sum over
// earlier requests of n * (P + n), or n * n in the prefix-visible form.  One
// workgroup scans the requests 256 at a time with a carry.
__global__ __launch_bounds__(256) void tv_append_scan_kernel(AppendParams p) {
  __shared__ int64_t wsum[4];
  __shared__ int64_t carry_s;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base <= p.batch; base += 256) {
    const int b = base + t;
    int64_t blk = 0;
    if (b < p.batch) {
      const int64_t n = (int64_t)p.qo_indptr[b + 1] - p.qo_indptr[b];
      const int64_t P = (int64_t)p.prefix_indptr[b + 1] - p.prefix_indptr[b];
      blk = n * (p.prefix_visible ? n : P + n);
    }
    // inclusive scan of blk over the workgroup
    int64_t incl = blk;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int64_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int64_t excl = before + incl - blk;
    if (b <= p.batch) {
      if (p.kv_indptr) p.kv_indptr[b] = p.prefix_indptr[b] + p.qo_indptr[b];
      if (p.mask_indptr) p.mask_indptr[b] = (int32_t)excl;
    }
    __syncthreads();
    if (t == 255) carry_s = excl + blk;
    __syncthreads();
  }
}

// blockIdx.y = request b.  blockIdx.x runs over three ranges of workgroups:
//   [0, rows_x)            the draft rows: 72 16-byte pieces per 1152-byte row
//                          (3.5 rows per workgroup pass), draft t to pool row
//                          out_cache_loc[t];
//   [rows_x, rows_x+idx_x) kv_indices of request b, 256 keys per workgroup;
//   [rows_x+idx_x, ...)    the mask block of request b, 16 bytes per thread:
//                          prefix keys 1, draft key k of row i 1 iff k is i or
//                          one of its ancestors.
__global__ __launch_bounds__(256) void tv_append_fill_kernel(AppendParams p) {
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int q0 = p.qo_indptr[b];
  const int pf0 = p.prefix_indptr[b];
  // lengths clamped to the host bounds the grid was sized for
  const int n = max(0, min(p.qo_indptr[b + 1] - q0, p.max_q_len));
  const int P = max(0, min(p.prefix_indptr[b + 1] - pf0, p.max_kv_len - n));
  int x = blockIdx.x;
  if (x < p.rows_x) {
    if (!p.draft_kv) return;
    // pieces of this request's rows handled by this workgroup
    constexpr int PIECES = QK * 2 / 16;  // 72
    for (int64_t g = (int64_t)x * 256 + t; g < (int64_t)n * PIECES; g += (int64_t)p.rows_x * 256) {
      const int r = (int)(g / PIECES), c = (int)(g - (int64_t)r * PIECES);
      const int64_t tok = (int64_t)q0 + r;
      if (tok < 0 || tok >= p.total_q) continue;
      const int32_t slot = p.out_cache_loc[tok];
      if (slot < 0 || (int64_t)slot >= p.num_slots) continue;
      const uint4 v = reinterpret_cast<const uint4*>(p.draft_kv + tok * QK)[c];
      reinterpret_cast<uint4*>(p.kv_buf + (int64_t)slot * QK)[c] = v;
    }
    return;
  }
  x -= p.rows_x;
  if (x < p.idx_x) {
    const int L = P + n;
    const int64_t k0 = (int64_t)pf0 + q0;  // kv_indptr[b]
    for (int j = x * 256 + t; j < L; j += p.idx_x * 256) {
      const int64_t dst = k0 + j;
      if (dst < 0 || dst >= p.total_kv) continue;
      int32_t v;
      if (j < P) {
        const int64_t src = (int64_t)pf0 + j;
        v = (src >= 0 && src < p.total_prefix) ? p.prefix_indices[src] : -1;
      } else {
        const int64_t tok = (int64_t)q0 + (j - P);
        v = (tok >= 0 && tok < p.total_q) ? p.out_cache_loc[tok] : -1;
      }
      p.kv_indices[dst] = v;
    }
    return;
  }
  x -= p.idx_x;
  if (!p.parents || !p.mask || !p.mask_indptr) return;
  // the request's mask block as 16-byte words (offsets from the 16-byte
  // aligned mask base); a word wholly inside the block and the capacity is one
  // 16-byte store, a word the block shares with a neighbour is stored bytewise
  const int stride = p.prefix_visible ? n : P + n;
  const int skip = p.prefix_visible ? 0 : P;  // columns before the draft keys
  const int64_t blk0 = p.mask_indptr[b];
  const int64_t lim = min(blk0 + (int64_t)n * stride, p.total_mask);
  if (blk0 < 0 || lim <= blk0 || stride <= 0) return;
  const int64_t w0 = blk0 >> 4;
  const int64_t nw = ((lim + 15) >> 4) - w0;
  for (int64_t wi = (int64_t)x * 256 + t; wi < nw; wi += (int64_t)p.mask_x * 256) {
    const int64_t a0 = (w0 + wi) << 4;
    // row and column of the word's first byte inside the block
    const int64_t off0 = max(a0, blk0) - blk0;
    int i = (int)(off0 / stride);
    int j = (int)(off0 - (int64_t)i * stride);
    uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t a = a0 + e;
      if (a < blk0 || a >= lim) continue;
      uint32_t vis = 1;
      if (j >= skip) {
        // draft key k: walk up from row i; parents precede children, so the
        // walk descends and ends within i + 1 steps (a parent that breaks the
        // order ends it, as a root would)
        const int k = j - skip;
        int anc = i;
        for (int step = 0; step <= i && anc > k; ++step) {
          const int64_t tok = (int64_t)q0 + anc;
          const int pa = (tok >= 0 && tok < p.total_q) ? p.parents[tok] : -1;
          if (pa < -1 || pa >= anc) {
            anc = -1;
            break;
          }
          anc = pa;
        }
        vis = anc == k ? 1u : 0u;
      }
      word[e >> 2] |= vis << (8 * (e & 3));
      if (++j == stride) {
        j = 0;
        ++i;
      }
    }
    if (a0 >= blk0 && a0 + 16 <= lim) {
      reinterpret_cast<uint4*>(p.mask)[w0 + wi] = make_uint4(word[0], word[1], word[2], word[3]);
    } else {
      for (int e = 0; e < 16; ++e) {
        const int64_t a = a0 + e;
        if (a >= blk0 && a < lim) p.mask[a] = (uint8_t)(word[e >> 2] >> (8 * (e & 3)));
      }
    }
  }
}

hipError_t launch_append(const AppendParams& p, int grid_x, hipStream_t st) {
  AppendParams a = p;
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&tv_append_scan_kernel), dim3(1),
                                 dim3(256), args, 0, st);
  if (e != hipSuccess || p.batch == 0 || grid_x == 0) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&tv_append_fill_kernel),
                         dim3(grid_x, p.batch), dim3(256), args, 0, st);
}

}  // namespace tv
