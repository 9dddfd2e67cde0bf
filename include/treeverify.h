/*
 * treeverify.h -- tree-masked verify attention over a paged MLA latent KV pool,
 * for AMD Instinct MI355X (gfx950).  C ABI of libtreeverify.so.
 *
 * The operation (sources: three pages about one verify-kernel bring-up):
 *
 *   Draft-tree query rows q[t, h, 0:576] (absorbed MLA: 512 latent + 64 RoPE
 *   dims; page 3 "The Pivot to Live Cutover", section "Input Knowledge
 *   Required") attend over keys gathered from a latent pool kv_buf[slot, 0:576]
 *   with page size 1 (same section, and "The Technical Investigation", where the
 *   MLA key buffer is [num_slots, 1, 576]).  The keys of request b are
 *   kv_buf[kv_indices[kv_indptr[b] + j]], j = 0 .. L_b-1: the prefix slots
 *   followed by the slots the draft tokens were written to (page 2 "Flipping
 *   the Switch", section "The Long Road to Parity").  Draft row i of request b
 *   may see key j iff mask[mask_indptr[b] + i*L_b + j] != 0; the mask block of a
 *   request is n_b x L_b bytes with row stride L_b = prefix_len + n_draft (same
 *   section: mask=(270,) = 9 x 30) and is located through mask_indptr (page 3,
 *   section "The Technical Investigation").  All H heads of a draft share its
 *   mask row.  With score s_j = sm_scale * <q[t,h,:], k_j[0:576]> over the
 *   visible keys:
 *
 *       out[t,h,d] = sum_j softmax(s)_j * k_j[d],  d < 512   (V = first 512 dims)
 *       lse[t,h]   = ln sum_j exp(s_j)
 *
 *   A row with no visible key gets out = 0 and lse = -inf.
 *
 * Method: KV-split flash decoding (page 2, section "The Broader Context": the
 * KV length is cut into splits that run in parallel, each yielding a partial
 * output and log-sum-exp) followed by an LSE merge.  The call is capture-safe
 * (page 2, section "The Decision to Flip the Switch": no host syncs, copies or
 * allocations): it only enqueues kernels on `stream`.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_QK_DIM 576 /* key / query dims: 512 latent + 64 RoPE */
#define TV_V_DIM 512  /* value dims: the first 512 latent dims  */

typedef enum {
  TV_OK = 0,
  TV_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  TV_ERR_SHAPE = 2,       /* a size in tv_problem is out of range or inconsistent, or
                             sm_scale is not positive and finite                         */
  TV_ERR_WORKSPACE = 3,   /* workspace is NULL or smaller than tv_workspace_bytes()      */
  TV_ERR_UNSUPPORTED = 4, /* out_dtype or a flags bit unknown, reserved != 0             */
  TV_ERR_INPUT = 5,       /* tv_check_inputs found a device-side precondition violated   */
  TV_ERR_LAUNCH = 6,      /* a kernel launch failed (e.g. the current device is not gfx950) */
  TV_ERR_HIP = 7          /* a HIP runtime call inside tv_check_inputs failed, or the
                             static scratch lookup of tv_verify_attn_static             */
} tv_status;

typedef enum { TV_OUT_BF16 = 0, TV_OUT_F32 = 1 } tv_out_dtype;

/* tv_problem.flags.  The softmax probabilities (fp32) enter the P.V product on
 * the bf16 matrix cores.  By default each is rounded once to bf16, and a split's
 * partial output is kept as fp16 under an exact power-of-two scale; together
 * these bound the output error by (2^-8 + 2^-11) * max |v| over the row's
 * visible keys.  TV_FLAG_PRECISE_P splits each probability into two bf16 terms
 * (hi + lo, about 16 significant bits), runs the P.V product on both and keeps
 * fp32 partial outputs: the bound becomes about 2^-16 * max |v|, for 32 more
 * MFMAs per 32-key tile (68 -> 100) and twice the partial-output traffic.
 * Meant for value distributions with large outliers. */
#define TV_FLAG_PRECISE_P 1

/* tv_problem.flags.  The mask covers the draft keys only: every draft row sees
 * all P_b = L_b - n_b prefix keys of its request, and the mask block of request
 * b is n_b x n_b bytes, row stride n_b, where byte i * n_b + k says whether draft
 * i sees draft k's key (key P_b + k).  This is the prefix-visible form of the
 * custom mask that the pages name as the integration's other option (page 3,
 * "The Pivot to Live Cutover", section "The Technical Investigation"); it spares
 * the caller the n_b x L_b block, which at a 200k prefix is n_b x 200k bytes.
 * The results equal those of the full mask with every prefix byte nonzero. */
#define TV_FLAG_PREFIX_VISIBLE 2

/* tv_problem.flags.  Each request's prefix keys are one contiguous run of the
 * pool, as a defragmented cache lays them out (page 2 "Flipping the Switch",
 * section "The Broader Context", and page 3 "The Pivot to Live Cutover",
 * section "Conclusion": the serving stack's KV defragmentation): with P_b =
 * L_b - n_b, prefix key j < P_b of request b is pool slot
 * kv_indices[kv_indptr[b]] + j.  Of the prefix entries of kv_indices only that
 * first one is read (none when P_b = 0); the entries kv_indptr[b] + 1 ..
 * kv_indptr[b] + P_b - 1 are never read and need not be written.  The n_b
 * draft keys are read from kv_indices as usual.  kv_indptr, the mask and
 * every other argument keep their meaning; the results equal those of the
 * full key list start, start + 1, ..., start + P_b - 1 followed by the draft
 * slots.  The run [start, start + P_b) must lie in the pool (tv_check_inputs
 * checks it). */
#define TV_FLAG_CONTIGUOUS_PREFIX 4

/* Host-side description of one call.  Device-side lengths may vary between
 * calls (or graph replays) as long as they stay within these bounds. */
typedef struct tv_problem {
  int32_t batch;      /* 0 <= B <= 65535 requests                                    */
  int32_t num_heads;  /* H >= 1 query heads sharing one latent KV head               */
  int64_t total_q;    /* rows of q / out / lse (draft tokens), >= qo_indptr[B]       */
  int32_t max_q_len;  /* >= every n_b = qo_indptr[b+1] - qo_indptr[b]                */
  int32_t max_kv_len; /* >= every L_b = kv_indptr[b+1] - kv_indptr[b], draft slots
                         INCLUDED (L_b = prefix_len + n_draft)                        */
  int64_t num_slots;  /* rows of kv_buf                                              */
  int64_t total_kv;   /* entries of kv_indices, >= kv_indptr[B]; < 2^31              */
  int64_t total_mask; /* bytes of mask, >= mask_indptr[B]; < 2^31                     */
  int32_t num_splits; /* 0: chosen by the library.  k > 0: the longest request
                         (max_kv_len keys) is cut into k splits of equal size,
                         rounded up to the 32-key tile; shorter requests use as
                         many splits of that size as they need                      */
  int32_t out_dtype;  /* tv_out_dtype                                                */
  int32_t flags;      /* TV_FLAG_* bits; unknown bits -> TV_ERR_UNSUPPORTED           */
  int32_t reserved;   /* must be 0                                                   */
} tv_problem;

/* Launch plan that tv_verify_attn uses for `p` (host arithmetic only). */
typedef struct tv_plan {
  int32_t split_keys;  /* keys per split (multiple of 32)                           */
  int32_t max_splits;  /* splits of the longest request                             */
  int32_t row_blocks;  /* 128-row blocks of the largest request (n_b * H rows)      */
  int32_t merge;       /* 1 if the merge kernel runs (max_splits > 1)               */
  int64_t workspace_bytes;
} tv_plan;

/* Fills *plan for `p`.  TV_ERR_NULL / TV_ERR_SHAPE on bad arguments. */
tv_status tv_get_plan(const tv_problem* p, tv_plan* plan);

/* Bytes of device workspace tv_verify_attn needs for `p` (0 if `p` is invalid
 * or there is nothing to compute).  It holds, each part rounded up to 256
 * bytes:
 *  - one 32-bit visibility word per (draft token, 32-key tile), only when some
 *    32 consecutive rows (draft * H + head, from a multiple of 32) span more
 *    than 4 draft tokens (H < 8, H = 9), or with TV_FLAG_PREFIX_VISIBLE;
 *    otherwise the kernels read the mask bytes directly;
 *  - when more than one split is used, the per-split partial outputs:
 *    total_q * H * max_splits entries of 512 fp16 values plus two fp32 (lse,
 *    scale exponent), or with TV_FLAG_PRECISE_P of 512 + 1 fp32;
 *  - for a batch of more than one request whose launch has more than 256
 *    work items (request x split x 128-row block), one int32 per work item
 *    (the longest-first dispatch order). */
size_t tv_workspace_bytes(const tv_problem* p);

/*
 * Tree-masked verify attention.  All pointers are device memory owned by the
 * caller; the library keeps no state between calls and allocates nothing.
 *
 *   q           bf16 [total_q, H, 576], contiguous
 *   kv_buf      bf16 [num_slots, 576], contiguous (1152-byte rows), 16-byte aligned
 *   kv_indices  int32 [total_kv]: per request, prefix slots then draft slots
 *   kv_indptr   int32 [B+1], non-decreasing
 *   qo_indptr   int32 [B+1], non-decreasing; request b owns q rows
 *               qo_indptr[b] .. qo_indptr[b+1]-1
 *   mask        uint8 [total_mask], nonzero = visible
 *   mask_indptr int32 [B+1]; mask_indptr[b+1] - mask_indptr[b] = n_b * L_b
 *               (n_b * n_b with TV_FLAG_PREFIX_VISIBLE)
 *   sm_scale    score scale (e.g. 1/sqrt(192)); positive and finite, else
 *               TV_ERR_SHAPE
 *   out         [total_q, H, 512] bf16 (round to nearest even) or fp32
 *   lse         fp32 [total_q, H], natural log
 *   workspace   >= tv_workspace_bytes(p) bytes, 256-byte aligned; contents on
 *               entry are ignored.  May be NULL when that size is 0.
 *   stream      hipStream_t (NULL = default stream)
 *
 * q rows outside every request are left untouched.
 *
 * Errors: host-detectable problems return TV_ERR_* before anything is enqueued
 * (outputs untouched).  Device-content problems (decreasing indptrs, slots
 * outside the pool, L_b < n_b, a mask block that is not n_b * L_b bytes,
 * lengths above the tv_problem bounds) are undefined behaviour here; run
 * tv_check_inputs to detect them.  Concurrent calls need distinct workspaces.
 * Preconditions: the draft tokens' latent rows are already in kv_buf at their
 * slots, every referenced row is finite, and out/lse alias no input.
 */
tv_status tv_verify_attn(const tv_problem* p, const void* q, const void* kv_buf,
                         const int32_t* kv_indices, const int32_t* kv_indptr,
                         const int32_t* qo_indptr, const uint8_t* mask,
                         const int32_t* mask_indptr, float sm_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement variant of tv_verify_attn: the same arguments and the same
 * kernels, plus two caller-created hipEvent_t handles (timing enabled) that
 * take the start and end times of the split-attention kernel's own dispatch
 * (the dominant kernel; hipExtLaunchKernel), so a benchmark can time that
 * kernel alone without adding packets to `stream`.  Either event may be NULL.
 */
tv_status tv_verify_attn_timed(const tv_problem* p, const void* q, const void* kv_buf,
                               const int32_t* kv_indices, const int32_t* kv_indptr,
                               const int32_t* qo_indptr, const uint8_t* mask,
                               const int32_t* mask_indptr, float sm_scale, void* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* split_start_event, void* split_stop_event, void* stream);

/* Bytes of the device-resident scratch array behind tv_verify_attn_static. */
#define TV_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * tv_verify_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same arguments, plan and kernels as
 * tv_verify_attn; the workspace is a static device array of
 * TV_STATIC_SCRATCH_BYTES (64 MiB) that every GPU the library runs on holds
 * from the first use until the process ends.  Nothing is allocated.
 *
 * Limit: a problem whose tv_workspace_bytes() exceeds TV_STATIC_SCRATCH_BYTES
 * returns TV_ERR_WORKSPACE before anything is enqueued (for example 32 requests
 * x 24 drafts x 64 heads split 11 ways needs about 553 MB; one request of 32
 * drafts x 16 heads over 32k keys needs 32 MB).  The first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress; TV_ERR_HIP if
 * that fails), so make it outside stream capture; later calls on the device
 * make no runtime call besides the launches.  All calls on one GPU share its
 * array: calls that overlap on one GPU (two streams, two threads) race.  A
 * call writes every scratch byte it reads, so nothing is cleared between
 * calls.  Errors otherwise as tv_verify_attn.
 */
tv_status tv_verify_attn_static(const tv_problem* p, const void* q, const void* kv_buf,
                                const int32_t* kv_indices, const int32_t* kv_indptr,
                                const int32_t* qo_indptr, const uint8_t* mask,
                                const int32_t* mask_indptr, float sm_scale, void* out,
                                float* lse, void* stream);

/*
 * Debug validator for the device-side preconditions of tv_verify_attn.  Copies
 * the three indptr arrays and kv_indices to the host and synchronises `stream`:
 * NOT capture-safe.  Returns TV_OK, TV_ERR_INPUT (a precondition is violated;
 * *bad_request, if not NULL, receives the first offending request, else -1),
 * TV_ERR_HIP if a copy fails, or the host-side errors of tv_verify_attn.  Checks:
 * indptrs non-decreasing and within total_q / total_kv / total_mask; every
 * n_b <= max_q_len and L_b <= max_kv_len; L_b >= n_b; the mask block of
 * request b is exactly n_b * L_b bytes (n_b * n_b with TV_FLAG_PREFIX_VISIBLE);
 * every slot in [0, num_slots) (with TV_FLAG_CONTIGUOUS_PREFIX: each prefix
 * run inside the pool, and the draft slots).  The last
 * two catch both halves of the marshaling mistake the pages describe (page 2,
 * section "The Long Road to Parity"): draft slots missing from kv_indices, and
 * a mask laid out with the prefix-only row stride.  Mask contents are not read.
 */
tv_status tv_check_inputs(const tv_problem* p, const int32_t* kv_indices,
                          const int32_t* kv_indptr, const int32_t* qo_indptr,
                          const int32_t* mask_indptr, void* stream, int32_t* bad_request);

/*
 * The marshaling step before tv_verify_attn, on the device (page 2 "Flipping
 * the Switch", section "The Long Road to Parity": the draft tokens' latent rows
 * are written into the pool at their slots, and those slots follow the prefix
 * slots in kv_indices; leaving them out was the pages' parity failure).  For
 * request b with P_b = prefix_indptr[b+1] - prefix_indptr[b] prefix keys and
 * n_b = qo_indptr[b+1] - qo_indptr[b] draft tokens:
 *
 *   kv_buf[out_cache_loc[t]] = draft_kv[t]        for every draft token t
 *   kv_indptr[b]   = prefix_indptr[b] + qo_indptr[b]   (so L_b = P_b + n_b)
 *   kv_indices[kv_indptr[b] + j] = prefix_indices[prefix_indptr[b] + j]  (j < P_b)
 *                                = out_cache_loc[qo_indptr[b] + j - P_b] (j >= P_b)
 *   mask_indptr[b] = sum over requests before b of n * L (n * n with
 *                    TV_FLAG_PREFIX_VISIBLE)
 *   mask row i of request b: every prefix key visible; draft key k (column
 *                    P_b + k, or k in the prefix-visible form) visible iff k
 *                    is i or an ancestor of i in the draft tree
 *
 * The tree is given as parents[t] for every draft token t: the request-local
 * index of its parent, -1 for a root, and smaller than the token's own index
 * (parents precede children).  The outputs are exactly the inputs
 * tv_verify_attn takes.  Capture-safe: two kernel launches on `stream`.
 */
typedef struct tv_append_problem {
  int32_t batch;        /* 0 <= B <= 65535                                           */
  int32_t max_q_len;    /* >= every n_b                                             */
  int32_t max_kv_len;   /* >= every P_b + n_b                                       */
  int32_t flags;        /* TV_FLAG_PREFIX_VISIBLE or 0; other bits TV_ERR_UNSUPPORTED */
  int64_t total_q;      /* rows of draft_kv, out_cache_loc, parents; >= qo_indptr[B]  */
  int64_t num_slots;    /* rows of kv_buf                                           */
  int64_t total_prefix; /* entries of prefix_indices                                */
  int64_t total_kv;     /* capacity of kv_indices (>= prefix_indptr[B] + qo_indptr[B]),
                           < 2^31                                                    */
  int64_t total_mask;   /* capacity of mask in bytes, < 2^31                         */
} tv_append_problem;

/*
 *   draft_kv       bf16 [total_q, 576], 16-byte aligned; NULL: the pool is not
 *                  written (the rows are already there) and kv_buf may be NULL
 *   out_cache_loc  int32 [total_q]: pool slot of each draft token
 *   prefix_indices int32 [total_prefix]; prefix_indptr int32 [B+1]
 *   qo_indptr      int32 [B+1]
 *   parents        int32 [total_q], or NULL: no mask bytes are written
 *   kv_buf         bf16 [num_slots, 576], 16-byte aligned, written at the
 *                  draft tokens' slots
 *   kv_indices     int32 [total_kv], kv_indptr int32 [B+1]: written
 *   mask           uint8 [total_mask], 16-byte aligned (needed with parents), mask_indptr
 *                  int32 [B+1] (written if not NULL; needed with parents)
 *
 * All pointers are device memory owned by the caller.  Host-detectable errors
 * (NULL where required, sizes out of range, misalignment) return TV_ERR_*
 * before anything is enqueued.  Device contents that break the preconditions
 * (decreasing indptrs, lengths above the bounds, slots outside the pool,
 * parents out of order, totals above the capacities) give undefined contents
 * but no store outside the buffers: every store is bounded by the capacities
 * above, a draft row whose slot is outside the pool is not written, and a
 * parent out of order ends that row's ancestor walk.  Draft tokens sharing a
 * slot race.
 */
tv_status tv_append_draft(const tv_append_problem* p, const void* draft_kv,
                          const int32_t* out_cache_loc, const int32_t* prefix_indices,
                          const int32_t* prefix_indptr, const int32_t* qo_indptr,
                          const int32_t* parents, void* kv_buf, int32_t* kv_indices,
                          int32_t* kv_indptr, uint8_t* mask, int32_t* mask_indptr,
                          void* stream);

/* Static description of a status code. */
const char* tv_status_str(tv_status s);

#ifdef __cplusplus
}
#endif
#endif /* TREEVERIFY_H */
