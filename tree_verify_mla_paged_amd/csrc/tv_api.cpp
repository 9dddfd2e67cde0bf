// C-ABI host layer of libtreeverify: argument checks, launch plan, launches.
//
// tv_verify_attn enqueues up to three kernels on the caller's stream (mask
// packing, split attention, LSE merge) and nothing else: no allocation, copy,
// memset or synchronisation, so the call can be captured into a HIP graph
// (page 2 "Flipping the Switch", section "The Decision to Flip the Switch":
// the verify kernel consumes the serving stack's static buffers with no host
// syncs, copies or allocations).  The KV split count follows the pages'
// occupancy argument (page 2, section "The Broader Context": more KV splits to
// fill the machine) re-derived for 256 compute units and one 128-row
// workgroup per unit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tv_kernels.h"
#include "treeverify.h"

static_assert(sizeof(tv_problem) == 64 && offsetof(tv_problem, total_q) == 8 &&
                  offsetof(tv_problem, num_slots) == 24 && offsetof(tv_problem, out_dtype) == 52 &&
                  offsetof(tv_problem, flags) == 56,
              "tv_problem layout is part of the ABI");
static_assert(sizeof(tv_plan) == 24 && offsetof(tv_plan, workspace_bytes) == 16,
              "tv_plan layout is part of the ABI");
static_assert(sizeof(tv_append_problem) == 56 && offsetof(tv_append_problem, total_q) == 16 &&
                  offsetof(tv_append_problem, total_mask) == 48,
              "tv_append_problem layout is part of the ABI");

namespace {

constexpr int64_t kMaxInt32 = 2147483647;
constexpr int kCUs = 256;          // MI355X compute units
constexpr int kMinSplitTiles = 4;  // keys per split >= 128 unless the caller asks otherwise
constexpr int kMaxGridY = 65535;   // largest grid y dimension of a launch

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Whether the 32 rows (draft * H + head) of every wave, rows 32k .. 32k + 31 of
// a request, span at most MASK_BYTES_DRAFTS draft tokens.  The span depends on
// 32k mod H only, so k < H covers every case; a request's last wave has fewer
// rows and no wider a span.
bool waves_span_few_drafts(int64_t rows_max, int64_t H) {
  const int64_t waves = std::min<int64_t>(ceil_div(rows_max, 32), H);
  for (int64_t k = 0; k < waves; ++k) {
    const int64_t a = 32 * k, z = std::min<int64_t>(a + 31, rows_max - 1);
    if (z / H - a / H + 1 > tv::MASK_BYTES_DRAFTS) return false;
  }
  return true;
}

struct Layout {
  tv_plan plan;
  int32_t max_tiles;     // 32-key tiles of the longest request
  int64_t words_off, words_bytes;
  int64_t wso_off, wso_bytes;
  int64_t wsl_off, wsl_bytes;
  int64_t order_off, order_bytes;  // longest-first work order (0 bytes: natural order)
  int32_t xcd_group;     // dispatch positions per XCD group
  bool mask_bytes;       // the split kernel reads the mask bytes (no packed words)
  int64_t grid;          // split-kernel workgroups
  bool active;           // anything to compute
};

tv_status make_layout(const tv_problem* p, Layout* lay) {
  if (!p || !lay) return TV_ERR_NULL;
  std::memset(lay, 0, sizeof *lay);
  if (p->batch < 0 || p->num_heads < 1 || p->total_q < 0 || p->max_q_len < 0 ||
      p->max_kv_len < 0 || p->num_slots < 0 || p->total_kv < 0 || p->total_mask < 0 ||
      p->num_splits < 0)
    return TV_ERR_SHAPE;
  if (p->total_kv > kMaxInt32 || p->total_mask > kMaxInt32 || p->num_slots > kMaxInt32 + 1LL)
    return TV_ERR_SHAPE;
  if (p->out_dtype != TV_OUT_BF16 && p->out_dtype != TV_OUT_F32) return TV_ERR_UNSUPPORTED;
  if ((p->flags & ~(TV_FLAG_PRECISE_P | TV_FLAG_PREFIX_VISIBLE | TV_FLAG_CONTIGUOUS_PREFIX)) != 0 ||
      p->reserved != 0)
    return TV_ERR_UNSUPPORTED;
  if (p->max_q_len > p->total_q) return TV_ERR_SHAPE;
  // the pack and merge grids put the request in their y dimension
  if (p->batch > kMaxGridY) return TV_ERR_SHAPE;
  // per-request key offsets are 32-bit byte offsets (4 * key) in the kernels
  if (p->max_kv_len >= (1 << 30)) return TV_ERR_SHAPE;
  if ((int64_t)p->max_q_len * p->num_heads > kMaxInt32 ||
      p->total_q * (int64_t)p->num_heads > kMaxInt32)
    return TV_ERR_SHAPE;
  lay->active = p->batch > 0 && p->total_q > 0 && p->max_q_len > 0;
  if (!lay->active) return TV_OK;

  const int64_t L = p->max_kv_len;
  const int64_t rows_max = (int64_t)p->max_q_len * p->num_heads;
  const int64_t row_blocks = ceil_div(rows_max, tv::ROWS_PER_WG);
  int64_t split_keys;
  if (L == 0) {
    split_keys = tv::TILE_KEYS;
  } else if (p->num_splits > 0) {
    split_keys = ceil_div(ceil_div(L, p->num_splits), tv::TILE_KEYS) * tv::TILE_KEYS;
  } else {
    // splits of >= 4 tiles; one workgroup per compute unit over the whole
    // request, or for a batch (requests of unequal lengths, dispatched longest
    // first) about two, so that the schedule has pieces to balance with.  A
    // key list of exactly batch * max_kv_len entries holds every request at
    // max_kv_len: nothing to balance, and a second workgroup per unit would
    // only pay the per-workgroup start and end twice
    const int64_t kv_tiles = ceil_div(std::max<int64_t>(p->total_kv, L), tv::TILE_KEYS);
    const bool uniform = p->total_kv == (int64_t)p->batch * L;
    const int64_t share = p->batch > 1 && !uniform ? 2 * kCUs : kCUs;
    const int64_t per_wg =
        std::max<int64_t>(kMinSplitTiles, ceil_div(row_blocks * kv_tiles, share));
    split_keys = std::min<int64_t>(per_wg, ceil_div(L, tv::TILE_KEYS)) * tv::TILE_KEYS;
  }
  const int64_t max_splits = std::max<int64_t>(1, ceil_div(L, split_keys));
  const int64_t total_work = (int64_t)p->batch * max_splits * row_blocks;
  lay->xcd_group = (int32_t)std::min<int64_t>(row_blocks, 16);
  if (total_work > kMaxInt32 - 8 * 16) return TV_ERR_SHAPE;
  lay->grid = ceil_div(total_work, 8 * lay->xcd_group) * 8 * lay->xcd_group;

  lay->max_tiles = (int32_t)std::max<int64_t>(1, ceil_div(L, tv::TILE_KEYS));
  // the prefix-visible form always goes through the packed words: the pack
  // kernel expands it, the split kernel sees the same words either way
  lay->mask_bytes = (p->flags & TV_FLAG_PREFIX_VISIBLE) == 0 &&
                    waves_span_few_drafts(rows_max, p->num_heads);
  lay->words_off = 0;
  lay->words_bytes = lay->mask_bytes ? 0 : align256(p->total_q * lay->max_tiles * 4);
  int64_t off = lay->words_bytes;
  if (max_splits > 1) {
    // partial outputs: fp32 in precise mode, else fp16 with a scale exponent
    // stored beside each partial lse
    const bool f16_parts = (p->flags & TV_FLAG_PRECISE_P) == 0;
    const int64_t prow = p->total_q * p->num_heads * max_splits;
    lay->wso_off = off;
    lay->wso_bytes = align256(prow * TV_V_DIM * (f16_parts ? 2 : 4));
    off += lay->wso_bytes;
    lay->wsl_off = off;
    lay->wsl_bytes = align256(prow * (f16_parts ? 8 : 4));
    off += lay->wsl_bytes;
  }
  // requests of unequal lengths: a longest-first dispatch order (written by the
  // pack kernel) balances the compute units.  Not when every work item has a
  // compute unit of its own (one workgroup fits per unit): they all start at
  // once, and the order would only cost a launch
  if (p->batch > 1 && L > 0 && total_work > kCUs && total_work <= tv::SCHED_MAX_WORK) {
    lay->order_off = off;
    lay->order_bytes = align256(total_work * 4);
    off += lay->order_bytes;
  }
  lay->plan.split_keys = (int32_t)split_keys;
  lay->plan.max_splits = (int32_t)max_splits;
  lay->plan.row_blocks = (int32_t)row_blocks;
  lay->plan.merge = max_splits > 1;
  lay->plan.workspace_bytes = off;
  return TV_OK;
}

}  // namespace

namespace {

tv_status verify(const tv_problem* p, const void* q, const void* kv_buf,
                 const int32_t* kv_indices, const int32_t* kv_indptr, const int32_t* qo_indptr,
                 const uint8_t* mask, const int32_t* mask_indptr, float sm_scale, void* out,
                 float* lse, void* workspace, size_t workspace_bytes, hipEvent_t ev0,
                 hipEvent_t ev1, void* stream) {
  Layout lay;
  tv_status st = make_layout(p, &lay);
  if (st != TV_OK) return st;
  // the kernels take the row max before scaling: the scale must be positive
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return TV_ERR_SHAPE;
  if (!lay.active) return TV_OK;
  if (!q || !kv_buf || !kv_indptr || !qo_indptr || !mask_indptr || !out || !lse)
    return TV_ERR_NULL;
  if (p->max_kv_len > 0 && (!kv_indices || !mask)) return TV_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(kv_buf) & 15) || (reinterpret_cast<uintptr_t>(q) & 15) ||
      (reinterpret_cast<uintptr_t>(out) & 15))
    return TV_ERR_SHAPE;
  if (lay.plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < (size_t)lay.plan.workspace_bytes) return TV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return TV_ERR_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* words = reinterpret_cast<uint32_t*>(ws + lay.words_off);

  // the pack kernel: visibility words (waves spanning more draft tokens than
  // the split kernel reads bytes for) and the longest-first order (batches);
  // neither needed, no launch
  const bool want_order = lay.order_bytes > 0;
  if (p->max_kv_len > 0 && (!lay.mask_bytes || want_order)) {
    tv::PackParams pp;
    pp.mask = mask;
    pp.mask_indptr = mask_indptr;
    pp.kv_indptr = kv_indptr;
    pp.qo_indptr = qo_indptr;
    pp.words = words;
    pp.max_tiles = lay.max_tiles;
    pp.order = lay.order_bytes ? reinterpret_cast<int32_t*>(ws + lay.order_off) : nullptr;
    pp.total_work = (int32_t)((int64_t)p->batch * lay.plan.max_splits * lay.plan.row_blocks);
    pp.max_splits = lay.plan.max_splits;
    pp.row_blocks = lay.plan.row_blocks;
    pp.split_keys = lay.plan.split_keys;
    pp.num_heads = p->num_heads;
    pp.batch = p->batch;
    pp.prefix_visible = (p->flags & TV_FLAG_PREFIX_VISIBLE) ? 1 : 0;
    // a wave per draft row and 512 keys (tv_pack_mask_kernel), 4 waves per workgroup
    const int64_t gx =
        lay.mask_bytes
            ? 0
            : ceil_div((int64_t)p->max_q_len * ceil_div(p->max_kv_len, tv::PACK_KEYS), 4);
    if (gx + 1 > kMaxInt32) return TV_ERR_SHAPE;
    pp.sched_block = pp.order ? (int32_t)gx : -1;  // one more workgroup column
    if (tv::launch_pack(pp, (int)gx + (pp.order ? 1 : 0), p->batch, s) != hipSuccess)
      return TV_ERR_LAUNCH;
  }

  tv::SplitParams sp;
  sp.q = static_cast<const uint16_t*>(q);
  sp.kv = static_cast<const uint16_t*>(kv_buf);
  sp.kv_indices = kv_indices;
  sp.kv_indptr = kv_indptr;
  sp.qo_indptr = qo_indptr;
  sp.mask = mask;
  sp.mask_indptr = mask_indptr;
  sp.mask_words = lay.mask_bytes ? nullptr : words;
  sp.order = lay.order_bytes ? reinterpret_cast<const int32_t*>(ws + lay.order_off) : nullptr;
  sp.out = out;
  sp.lse = lse;
  sp.ws_o = lay.plan.merge ? static_cast<void*>(ws + lay.wso_off) : nullptr;
  sp.ws_lse = lay.plan.merge ? reinterpret_cast<float*>(ws + lay.wsl_off) : nullptr;
  sp.s.scale_log2 = (float)((double)sm_scale * 1.4426950408889634074);
  sp.s.num_heads = p->num_heads;
  sp.s.split_keys = lay.plan.split_keys;
  sp.s.max_splits = lay.plan.max_splits;
  sp.s.row_blocks = lay.plan.row_blocks;
  sp.s.total_work = (int32_t)((int64_t)p->batch * lay.plan.max_splits * lay.plan.row_blocks);
  sp.s.max_tiles = lay.max_tiles;
  sp.s.xcd_group = lay.xcd_group;
  sp.s.mask_bytes = lay.mask_bytes ? 1 : 0;
  sp.s.total_mask = (int32_t)p->total_mask;
  sp.s.out_f32 = p->out_dtype == TV_OUT_F32 ? 1 : 0;
  sp.wide = p->num_slots * (int64_t)(TV_QK_DIM * 2) > (int64_t)UINT32_MAX;
  sp.precise = (p->flags & TV_FLAG_PRECISE_P) != 0;
  sp.contig = (p->flags & TV_FLAG_CONTIGUOUS_PREFIX) != 0;
  // one row block: no workgroup shares a gathered tile with another, and the
  // streaming hint keeps the rows from displacing (and writing back) what the
  // caches hold.  Measured cold, one box: S3 call 113 -> 75 us, D 139 -> 98,
  // S1 37.7 -> 30.7; clean-cold unchanged; warm S1 and S3 +8-9 % (the next
  // call no longer finds the rows in the memory-side cache).  With several
  // row blocks (C3) cold gained ~1 % and warm lost 9 %: left off there.
  sp.stream_kv = lay.plan.row_blocks == 1;
  const int grid = (int)lay.grid;
  if (tv::launch_split(sp, grid, s, ev0, ev1) != hipSuccess) return TV_ERR_LAUNCH;

  if (lay.plan.merge) {
    tv::MergeParams mp;
    mp.kv_indptr = kv_indptr;
    mp.qo_indptr = qo_indptr;
    mp.ws_o = sp.ws_o;
    mp.ws_lse = sp.ws_lse;
    mp.out = out;
    mp.lse = lse;
    mp.num_heads = p->num_heads;
    mp.split_keys = lay.plan.split_keys;
    mp.max_splits = lay.plan.max_splits;
    const int64_t gx = (int64_t)p->max_q_len * p->num_heads;  // one row per workgroup
    // few rows split many ways (a long single request with few heads): each
    // row's value dims in 4 slices, one workgroup each, so that more compute
    // units share the reads (measured: at 72 rows x 205 splits it gains, at
    // 512 rows x 61 splits the extra workgroups cost more than they save)
    const bool sliced = gx * p->batch < 4 * kCUs && lay.plan.max_splits > 64;
    // few splits per row (batches of many requests): one wave per row, all of
    // its splits in flight at once, instead of a workgroup per row
    const hipError_t e =
        lay.plan.max_splits <= tv::merge_wave_splits(!sp.precise)
            ? tv::launch_merge_rows(mp, (int)gx, p->batch, p->out_dtype, !sp.precise, s)
            : tv::launch_merge(mp, (int)gx, p->batch, p->out_dtype, !sp.precise, sliced, s);
    if (e != hipSuccess) return TV_ERR_LAUNCH;
  }
  return TV_OK;
}

}  // namespace

extern "C" {

tv_status tv_get_plan(const tv_problem* p, tv_plan* plan) {
  if (!p || !plan) return TV_ERR_NULL;
  Layout lay;
  const tv_status st = make_layout(p, &lay);
  if (st != TV_OK) return st;
  *plan = lay.plan;
  return TV_OK;
}

size_t tv_workspace_bytes(const tv_problem* p) {
  Layout lay;
  if (make_layout(p, &lay) != TV_OK) return 0;
  return (size_t)lay.plan.workspace_bytes;
}

tv_status tv_verify_attn(const tv_problem* p, const void* q, const void* kv_buf,
                         const int32_t* kv_indices, const int32_t* kv_indptr,
                         const int32_t* qo_indptr, const uint8_t* mask,
                         const int32_t* mask_indptr, float sm_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return verify(p, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr, sm_scale, out,
                lse, workspace, workspace_bytes, nullptr, nullptr, stream);
}

tv_status tv_verify_attn_timed(const tv_problem* p, const void* q, const void* kv_buf,
                               const int32_t* kv_indices, const int32_t* kv_indptr,
                               const int32_t* qo_indptr, const uint8_t* mask,
                               const int32_t* mask_indptr, float sm_scale, void* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* split_start_event, void* split_stop_event, void* stream) {
  return verify(p, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr, sm_scale, out,
                lse, workspace, workspace_bytes, static_cast<hipEvent_t>(split_start_event),
                static_cast<hipEvent_t>(split_stop_event), stream);
}

tv_status tv_verify_attn_static(const tv_problem* p, const void* q, const void* kv_buf,
                                const int32_t* kv_indices, const int32_t* kv_indptr,
                                const int32_t* qo_indptr, const uint8_t* mask,
                                const int32_t* mask_indptr, float sm_scale, void* out,
                                float* lse, void* stream) {
  Layout lay;
  const tv_status st = make_layout(p, &lay);
  if (st != TV_OK) return st;
  if (lay.plan.workspace_bytes > (int64_t)TV_STATIC_SCRATCH_BYTES) return TV_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (lay.active && lay.plan.workspace_bytes > 0 && tv::static_scratch(&scratch) != hipSuccess)
    return TV_ERR_HIP;
  return verify(p, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr, sm_scale, out,
                lse, scratch, scratch ? (size_t)TV_STATIC_SCRATCH_BYTES : 0, nullptr, nullptr,
                stream);
}

tv_status tv_check_inputs(const tv_problem* p, const int32_t* kv_indices,
                          const int32_t* kv_indptr, const int32_t* qo_indptr,
                          const int32_t* mask_indptr, void* stream, int32_t* bad_request) {
  if (bad_request) *bad_request = -1;
  Layout lay;
  tv_status st = make_layout(p, &lay);
  if (st != TV_OK) return st;
  if (p->batch == 0) return TV_OK;
  if (!kv_indptr || !qo_indptr || !mask_indptr) return TV_ERR_NULL;
  if (p->total_kv > 0 && !kv_indices) return TV_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool prefix_visible = (p->flags & TV_FLAG_PREFIX_VISIBLE) != 0;
  const bool contig = (p->flags & TV_FLAG_CONTIGUOUS_PREFIX) != 0;
  const size_t nb = (size_t)p->batch + 1;
  std::vector<int32_t> kvp(nb), qop(nb), mp(nb), idx((size_t)p->total_kv);
  if (hipMemcpyAsync(kvp.data(), kv_indptr, nb * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(qop.data(), qo_indptr, nb * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(mp.data(), mask_indptr, nb * 4, hipMemcpyDeviceToHost, s) != hipSuccess)
    return TV_ERR_HIP;
  if (p->total_kv > 0 && hipMemcpyAsync(idx.data(), kv_indices, idx.size() * 4,
                                        hipMemcpyDeviceToHost, s) != hipSuccess)
    return TV_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return TV_ERR_HIP;
  for (int32_t b = 0; b < p->batch; ++b) {
    const int64_t q0 = qop[b], q1 = qop[b + 1], k0 = kvp[b], k1 = kvp[b + 1];
    const int64_t m0 = mp[b], m1 = mp[b + 1];
    const bool bad = q0 < 0 || k0 < 0 || m0 < 0 || q1 < q0 || k1 < k0 || m1 < m0 ||
                     q1 > p->total_q || k1 > p->total_kv || m1 > p->total_mask ||
                     q1 - q0 > p->max_q_len || k1 - k0 > p->max_kv_len ||
                     k1 - k0 < q1 - q0 ||               // draft slots missing from kv_indices
                     // mask stride is not L_b (n_b in the prefix-visible form)
                     m1 - m0 != (q1 - q0) * (prefix_visible ? q1 - q0 : k1 - k0);
    if (bad) {
      if (bad_request) *bad_request = b;
      return TV_ERR_INPUT;
    }
    // keys whose slot comes from kv_indices; a contiguous prefix is the run
    // [kv_indices[k0], + P_b), which must lie in the pool
    int64_t first = k0;
    const int64_t P = (k1 - k0) - (q1 - q0);
    if (contig && P > 0) {
      if (idx[k0] < 0 || idx[k0] + P > p->num_slots) {
        if (bad_request) *bad_request = b;
        return TV_ERR_INPUT;
      }
      first = k0 + P;
    }
    for (int64_t j = first; j < k1; ++j) {
      if (idx[j] < 0 || idx[j] >= p->num_slots) {
        if (bad_request) *bad_request = b;
        return TV_ERR_INPUT;
      }
    }
  }
  return TV_OK;
}

tv_status tv_append_draft(const tv_append_problem* p, const void* draft_kv,
                          const int32_t* out_cache_loc, const int32_t* prefix_indices,
                          const int32_t* prefix_indptr, const int32_t* qo_indptr,
                          const int32_t* parents, void* kv_buf, int32_t* kv_indices,
                          int32_t* kv_indptr, uint8_t* mask, int32_t* mask_indptr,
                          void* stream) {
  if (!p) return TV_ERR_NULL;
  if (p->batch < 0 || p->max_q_len < 0 || p->max_kv_len < 0 || p->total_q < 0 ||
      p->num_slots < 0 || p->total_prefix < 0 || p->total_kv < 0 || p->total_mask < 0)
    return TV_ERR_SHAPE;
  if ((p->flags & ~TV_FLAG_PREFIX_VISIBLE) != 0) return TV_ERR_UNSUPPORTED;
  if (p->total_kv > kMaxInt32 || p->total_mask > kMaxInt32 || p->total_prefix > kMaxInt32 ||
      p->total_q > kMaxInt32 || p->num_slots > kMaxInt32 + 1LL || p->max_q_len > p->max_kv_len ||
      p->max_kv_len >= (1 << 30) || p->batch > kMaxGridY)
    return TV_ERR_SHAPE;
  if (p->batch == 0) return TV_OK;
  if (!prefix_indptr || !qo_indptr || !kv_indptr) return TV_ERR_NULL;
  if (p->total_q > 0 && !out_cache_loc) return TV_ERR_NULL;
  if (p->total_prefix > 0 && !prefix_indices) return TV_ERR_NULL;
  if (p->total_kv > 0 && !kv_indices) return TV_ERR_NULL;
  if (draft_kv && !kv_buf) return TV_ERR_NULL;
  if (parents && (!mask || !mask_indptr)) return TV_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(draft_kv) & 15) || (reinterpret_cast<uintptr_t>(kv_buf) & 15) ||
      (reinterpret_cast<uintptr_t>(mask) & 15))
    return TV_ERR_SHAPE;
  const bool pv = (p->flags & TV_FLAG_PREFIX_VISIBLE) != 0;
  tv::AppendParams ap;
  ap.draft_kv = static_cast<const uint16_t*>(draft_kv);
  ap.out_cache_loc = out_cache_loc;
  ap.prefix_indices = prefix_indices;
  ap.prefix_indptr = prefix_indptr;
  ap.qo_indptr = qo_indptr;
  ap.parents = parents;
  ap.kv_buf = static_cast<uint16_t*>(kv_buf);
  ap.kv_indices = kv_indices;
  ap.kv_indptr = kv_indptr;
  ap.mask = mask;
  ap.mask_indptr = mask_indptr;
  ap.total_q = p->total_q;
  ap.num_slots = p->num_slots;
  ap.total_prefix = p->total_prefix;
  ap.total_kv = p->total_kv;
  ap.total_mask = p->total_mask;
  ap.batch = p->batch;
  ap.max_q_len = p->max_q_len;
  ap.max_kv_len = p->max_kv_len;
  ap.prefix_visible = pv ? 1 : 0;
  // fill-kernel workgroup ranges: draft rows (72 16-byte pieces each),
  // kv_indices (256 keys each), mask rows (256 bytes each)
  ap.rows_x = draft_kv ? (int32_t)ceil_div((int64_t)p->max_q_len * (TV_QK_DIM * 2 / 16), 256) : 0;
  ap.idx_x = (int32_t)ceil_div(p->max_kv_len, 256);
  // 16 mask bytes per thread over the largest block, plus a word for its
  // unaligned start
  const int64_t block_words =
      ceil_div((int64_t)p->max_q_len * (pv ? p->max_q_len : p->max_kv_len), 16) + 1;
  if (block_words > kMaxInt32) return TV_ERR_SHAPE;
  ap.mask_x = (int32_t)ceil_div(block_words, 256);
  const int64_t grid = (int64_t)ap.rows_x + ap.idx_x + (parents ? ap.mask_x : 0);
  if (grid > kMaxInt32) return TV_ERR_SHAPE;
  if (tv::launch_append(ap, (int)grid, static_cast<hipStream_t>(stream)) != hipSuccess)
    return TV_ERR_LAUNCH;
  return TV_OK;
}

const char* tv_status_str(tv_status s) {
  // a C caller may pass any int: read the argument's bytes as one, since
  // loading a value outside the enumerators as tv_status is undefined in C++
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case TV_OK: return "ok";
    case TV_ERR_NULL: return "a required pointer is NULL";
    case TV_ERR_SHAPE: return "a size in tv_problem is out of range or inconsistent";
    case TV_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case TV_ERR_UNSUPPORTED: return "unsupported output dtype or flag, or reserved != 0";
    case TV_ERR_INPUT: return "device-side input violates a precondition";
    case TV_ERR_LAUNCH: return "kernel launch failed (the library holds gfx950 code only)";
    case TV_ERR_HIP: return "HIP runtime call failed";
  }
  return "unknown status";
}

}  // extern "C"
