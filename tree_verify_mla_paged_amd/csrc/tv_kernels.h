// Internal interface between the C-ABI host layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int QK = 576;           // key / query dims (512 latent + 64 RoPE)
constexpr int VD = 512;           // value dims
constexpr int ROWS_PER_WG = 128;  // query rows (draft x head) per workgroup: 4 waves x 32
constexpr int TILE_KEYS = 32;     // keys per LDS tile
constexpr int PACK_KEYS = 512;    // keys of a draft row one wave of tv_pack_mask_kernel packs
// When every wave's 32 rows span at most this many draft tokens, the split
// kernel reads their mask bytes itself (two drafts per wave-wide byte load and
// ballot); otherwise tv_pack_mask_kernel packs visibility words first.
constexpr int MASK_BYTES_DRAFTS = 4;
constexpr int OUT_BF16 = 0;
constexpr int OUT_F32 = 1;

// Work item w of the split kernel: request b, KV split s, row block rb with
// w = (b * max_splits + s) * row_blocks + rb.
constexpr int SCHED_BUCKETS = 1024;  // split-length classes of the longest-first order
constexpr int SCHED_MAX_WORK = 65536;  // larger grids keep the natural order

struct PackParams {
  const uint8_t* mask;
  const int32_t* mask_indptr;
  const int32_t* kv_indptr;
  const int32_t* qo_indptr;
  uint32_t* words;            // [total_q, max_tiles] visibility words
  int32_t max_tiles;          // ceil(max_kv_len / 32)
  int32_t sched_block;        // blockIdx.x of the workgroup that writes `order` (-1: none)
  int32_t* order;             // [total_work]: work item at dispatch position p, or -1
  int32_t total_work, max_splits, row_blocks, split_keys, num_heads, batch;
  // 1: the mask block of request b is n_b x n_b (draft keys only) and every
  // draft sees all L_b - n_b prefix keys
  int32_t prefix_visible;
};

struct SplitScalars {
  float scale_log2;           // sm_scale * log2(e)
  int32_t num_heads;
  int32_t split_keys;         // keys per split, multiple of TILE_KEYS
  int32_t max_splits;
  int32_t row_blocks;
  int32_t total_work;         // batch * max_splits * row_blocks
  int32_t max_tiles;
  int32_t xcd_group;          // dispatch positions per XCD group (see tv_split_kernel)
  int32_t mask_bytes;         // 1: visibility read from the mask bytes in the tile loop
                              // (see MASK_BYTES_DRAFTS); 0: from tv_pack_mask_kernel's words
  int32_t total_mask;         // bytes of the mask (its buffer's record count)
  int32_t out_f32;            // output dtype: 1 fp32, 0 bf16
};

struct SplitParams {
  const uint16_t* q;          // bf16 [total_q, H, 576]
  const uint16_t* kv;         // bf16 [num_slots, 576]
  const int32_t* kv_indices;
  const int32_t* kv_indptr;
  const int32_t* qo_indptr;
  const uint8_t* mask;        // the caller's mask bytes (mask_bytes mode)
  const int32_t* mask_indptr;
  const uint32_t* mask_words; // [total_q, max_tiles] from tv_pack_mask_kernel (word mode)
  const int32_t* order;       // longest-first work order from tv_pack_mask_kernel, or null
  void* out;                  // [total_q, H, 512] bf16 or fp32 (requests with one split)
  float* lse;                 // [total_q, H]
  // partial outputs [total_q * H, max_splits, 512]: fp32 in precise mode, else
  // fp16 scaled by a power of two per (row, split)
  void* ws_o;
  // per (row, split): the partial lse (natural log), fp32; without precise mode
  // followed by the scale exponent k (as a float): o = h * 2^k
  float* ws_lse;
  SplitScalars s;
  bool wide;                  // pool larger than 4 GiB: 64-bit gather addresses
  bool precise;               // probabilities as bf16 hi + lo in the P.V product
  // contiguous-prefix form: prefix key j of request b is pool slot
  // kv_indices[kv_indptr[b]] + j; the other prefix entries are not read
  bool contig;
  // key rows loaded non-temporal: set for plans of one row block, where each
  // gathered tile is read by one workgroup only
  bool stream_kv;
};

struct MergeParams {
  const int32_t* kv_indptr;
  const int32_t* qo_indptr;
  const void* ws_o;           // as SplitParams::ws_o
  const float* ws_lse;        // as SplitParams::ws_lse
  void* out;
  float* lse;
  int32_t num_heads;
  int32_t split_keys;
  int32_t max_splits;
};

// The marshaling step (tv_append_draft): see tv_append.hip.
struct AppendParams {
  const uint16_t* draft_kv;       // bf16 [total_q, 576] or null (no pool write)
  const int32_t* out_cache_loc;   // [total_q] pool slot of each draft token
  const int32_t* prefix_indices;  // [total_prefix]
  const int32_t* prefix_indptr;   // [batch + 1]
  const int32_t* qo_indptr;       // [batch + 1]
  const int32_t* parents;         // [total_q] request-local parent, -1 root; null: no mask
  uint16_t* kv_buf;               // bf16 [num_slots, 576]
  int32_t* kv_indices;            // [total_kv]
  int32_t* kv_indptr;             // [batch + 1]
  uint8_t* mask;                  // [total_mask]
  int32_t* mask_indptr;           // [batch + 1]
  int64_t total_q, num_slots, total_prefix, total_kv, total_mask;
  int32_t batch, max_q_len, max_kv_len;
  int32_t prefix_visible;         // mask in the n x n form
  int32_t rows_x, idx_x, mask_x;  // fill-kernel workgroup ranges (see tv_append.hip)
};

hipError_t launch_append(const AppendParams& p, int grid_x, hipStream_t st);
hipError_t launch_pack(const PackParams& p, int grid_x, int batch, hipStream_t st);
// ev0 / ev1 (may be null): stamped with the split kernel's own start and end.
hipError_t launch_split(const SplitParams& p, int grid, hipStream_t st, hipEvent_t ev0,
                        hipEvent_t ev1);
// rows: per request (max_q_len * H); sliced: 4 workgroups per row, each
// merging a quarter of the value dims.
hipError_t launch_merge(const MergeParams& p, int rows, int batch, int out, bool f16_parts,
                        bool sliced, hipStream_t st);
// Plans of at most merge_wave_splits splits: one wave per row, every split's
// partial held in registers (32 fp16 or 16 fp32 partial rows per lane).
constexpr int merge_wave_splits(bool f16_parts) { return f16_parts ? 32 : 16; }
hipError_t launch_merge_rows(const MergeParams& p, int rows, int batch, int out, bool f16_parts,
                             hipStream_t st);
// The current device's copy of the static scratch array (tv_static.hip):
// TV_STATIC_SCRATCH_BYTES bytes, 256-byte aligned.
hipError_t static_scratch(void** ptr);

}  // namespace tv
