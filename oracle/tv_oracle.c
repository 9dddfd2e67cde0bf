/*
 * Oracle for tree-masked verify attention over a paged MLA latent KV pool.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, fp64 CPU definition
 * of what the GPU path computes.  Only the tests, the package smoke check and
 * the benchmark's CPU-baseline leg load it; the library under
 * tree_verify_mla_paged_amd/ never does, and the two share no code.
 *
 * What is computed (sources are the three pages this work follows):
 *
 *  - Keys of request b are the pool rows kv_buf[kv_indices[kv_indptr[b] + j]],
 *    j = 0 .. L_b - 1, page size 1: the prefix slots followed by the slots the
 *    draft tokens were written to.  Page 2 ("Flipping the Switch on a Custom
 *    CUDA Verify Kernel"), section "The Long Road to Parity".
 *  - Row i of request b may see key j iff mask[mask_indptr[b] + i * L_b + j]
 *    is nonzero: one flat block per request located by mask_indptr, row
 *    stride L_b = prefix_len + n_draft (the live mask of 270 = 9 x 30 entries
 *    in the same section; the per-sequence mask_indptr indexing of page 3,
 *    "The Pivot to Live Cutover", section "The Technical Investigation").
 *    The same mask row serves all H heads of draft token i.
 *  - Prefix-visible form (the custom mask without its prefix part, page 3,
 *    section "The Technical Investigation"): every draft row sees all
 *    P_b = L_b - n_b prefix keys, and the block of request b holds only the
 *    draft keys, n_b x n_b bytes with row stride n_b: byte i * n_b + k says
 *    whether row i sees key P_b + k.
 *  - Contiguous-prefix form (the pages' defragmented cache, where a request's
 *    KV sits in one run of the pool: page 2, section "The Broader Context";
 *    page 3, section "Conclusion"): the P_b prefix keys of request b are the
 *    consecutive pool rows kv_indices[kv_indptr[b]] + j, j < P_b, and only
 *    that first prefix entry of kv_indices is read; the draft keys are looked
 *    up as before.
 *  - Absorbed MLA: a query row and a key row have 576 dims (512 latent + 64
 *    RoPE, page 3, section "Input Knowledge Required"); the score uses all
 *    576, the value is the first 512 dims of the same key row.
 *  - Output: softmax-weighted sum of the visible values and the natural-log
 *    sum-exp of the scaled scores.  A row with no visible key gets o = 0 and
 *    lse = -inf.
 *
 * The pages never write the formula out; this is the plain definition of
 * masked softmax attention over the gathered keys, done in two passes in
 * fp64 with the sums taken in ascending order so that results are
 * deterministic.  The KV-split flash-decode that the pages' kernel uses
 * (page 2, section "The Broader Context") reaches the same value up to
 * rounding, so the oracle does not follow it.
 */
#include "tv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 576
#define VD 512

/* bf16 bit pattern -> double.  Exact: bf16 is the top half of an fp32. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int tvo_check(const tvo_args* a) {
  if (!a || a->batch < 0 || a->num_heads < 1 || a->total_q < 0 || a->num_slots < 0)
    return TVO_ERR_SHAPE;
  if (a->batch == 0) return TVO_OK;
  if (!a->kv_indptr || !a->qo_indptr || !a->mask_indptr) return TVO_ERR_NULL;
  for (int32_t b = 0; b < a->batch; ++b) {
    int64_t q0 = a->qo_indptr[b], q1 = a->qo_indptr[b + 1];
    int64_t k0 = a->kv_indptr[b], k1 = a->kv_indptr[b + 1];
    int64_t m0 = a->mask_indptr[b], m1 = a->mask_indptr[b + 1];
    if (q0 < 0 || k0 < 0 || m0 < 0 || q1 < q0 || k1 < k0 || m1 < m0) return TVO_ERR_INDPTR;
    if (q1 > a->total_q || k1 > a->total_kv || m1 > a->total_mask) return TVO_ERR_INDPTR;
    int64_t n = q1 - q0, L = k1 - k0;
    /* draft slots are part of kv_indices, so every draft row has its own key */
    if (L < n) return TVO_ERR_KVLEN;
    if (m1 - m0 != n * (a->prefix_visible ? n : L)) return TVO_ERR_MASKLEN;
    /* keys whose slot is read from kv_indices; with a contiguous prefix the
       run [start, start + P_b) must lie in the pool */
    int64_t first = k0;
    if (a->contiguous_prefix && L > n) {
      const int64_t start = a->kv_indices[k0];
      if (start < 0 || start + (L - n) > a->num_slots) return TVO_ERR_SLOT;
      first = k0 + (L - n);
    }
    for (int64_t j = first; j < k1; ++j)
      if (a->kv_indices[j] < 0 || a->kv_indices[j] >= a->num_slots) return TVO_ERR_SLOT;
  }
  return TVO_OK;
}

/* Pool slot of key j of the request whose keys start at kv_indices[k0]; P keys
 * of prefix (used with a contiguous prefix only). */
static int64_t key_slot(const tvo_args* a, int64_t k0, int64_t P, int64_t j) {
  if (a->contiguous_prefix && j < P) return (int64_t)a->kv_indices[k0] + j;
  return a->kv_indices[k0 + j];
}

/* request that owns query token t, or -1 */
static int32_t owner(const tvo_args* a, int64_t t) {
  int32_t lo = 0, hi = a->batch - 1;
  while (lo <= hi) {
    int32_t mid = (lo + hi) / 2;
    if (t < a->qo_indptr[mid]) hi = mid - 1;
    else if (t >= a->qo_indptr[mid + 1]) lo = mid + 1;
    else return mid;
  }
  return -1;
}

/* One output row: draft token t, head h.  sbuf holds L_b doubles, jbuf L_b ints. */
static void one_row(const tvo_args* a, int64_t t, int32_t h, double* o, double* lse,
                    double* sbuf, int64_t* jbuf) {
  for (int d = 0; d < VD; ++d) o[d] = 0.0;
  *lse = -INFINITY;
  int32_t b = owner(a, t);
  if (b < 0) return;
  const int64_t i = t - a->qo_indptr[b];
  const int64_t k0 = a->kv_indptr[b];
  const int64_t L = a->kv_indptr[b + 1] - k0;
  const int64_t n = a->qo_indptr[b + 1] - a->qo_indptr[b];
  const int64_t P = a->prefix_visible ? L - n : 0; /* keys visible without a mask byte */
  const int64_t Pk = L - n;                         /* prefix keys */
  const uint8_t* mrow = a->mask + a->mask_indptr[b] + i * (a->prefix_visible ? n : L);
  const uint16_t* qrow = a->q + ((size_t)t * a->num_heads + h) * QK;
  const double c = (double)a->sm_scale; /* the fp32 scale, widened exactly */

  double qd[QK];
  for (int d = 0; d < QK; ++d) qd[d] = bf16_to_double(qrow[d]);

  /* visible set, ascending key order */
  int64_t nv = 0;
  for (int64_t j = 0; j < L; ++j)
    if (j < P || mrow[j - P] != 0) jbuf[nv++] = j;
  if (nv == 0) return;

  /* pass 1: scaled scores over all 576 dims, and their maximum */
  double m = -INFINITY;
  for (int64_t v = 0; v < nv; ++v) {
    const uint16_t* k = a->kv + (size_t)key_slot(a, k0, Pk, jbuf[v]) * QK;
    double acc = 0.0;
    for (int d = 0; d < QK; ++d) acc += qd[d] * bf16_to_double(k[d]);
    sbuf[v] = c * acc;
    if (sbuf[v] > m) m = sbuf[v];
  }
  /* pass 2: weights, normaliser, weighted sum of the first 512 dims */
  double z = 0.0;
  for (int64_t v = 0; v < nv; ++v) {
    double w = exp(sbuf[v] - m);
    sbuf[v] = w;
    z += w;
  }
  for (int64_t v = 0; v < nv; ++v) {
    const uint16_t* k = a->kv + (size_t)key_slot(a, k0, Pk, jbuf[v]) * QK;
    const double w = sbuf[v];
    for (int d = 0; d < VD; ++d) o[d] += w * bf16_to_double(k[d]);
  }
  for (int d = 0; d < VD; ++d) o[d] /= z;
  *lse = m + log(z);
}

int tvo_attention(const tvo_args* a, const int64_t* rows, int64_t nrows, int threads,
                  double* out, double* lse) {
  int rc = tvo_check(a);
  if (rc != TVO_OK) return rc;
  if (!out || !lse) return TVO_ERR_NULL;
  const int64_t all = a->total_q * (int64_t)a->num_heads;
  if (!rows) nrows = all;
  for (int64_t r = 0; r < (rows ? nrows : 0); ++r)
    if (rows[r] < 0 || rows[r] >= all) return TVO_ERR_SHAPE;
  int64_t maxL = 0;
  for (int32_t b = 0; b < a->batch; ++b) {
    int64_t L = a->kv_indptr[b + 1] - a->kv_indptr[b];
    if (L > maxL) maxL = L;
  }
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
  int failed = 0;
#pragma omp parallel
  {
    double* sbuf = (double*)malloc(sizeof(double) * (size_t)(maxL + 1));
    int64_t* jbuf = (int64_t*)malloc(sizeof(int64_t) * (size_t)(maxL + 1));
    if (!sbuf || !jbuf) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < nrows; ++r) {
        int64_t g = rows ? rows[r] : r;
        one_row(a, g / a->num_heads, (int32_t)(g % a->num_heads), out + (size_t)r * VD, lse + r,
                sbuf, jbuf);
      }
    }
    free(sbuf);
    free(jbuf);
  }
  return failed ? TVO_ERR_ALLOC : TVO_OK;
}

int tvo_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
