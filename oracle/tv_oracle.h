/*
 * Oracle for tree-masked verify attention (fp64, CPU).  TEST INFRASTRUCTURE:
 * loaded only by the tests, the smoke check and the benchmark's CPU baseline.
 * It shares no code with the HIP library.
 */
#ifndef TV_ORACLE_H
#define TV_ORACLE_H
#include <stdint.h>

enum {
  TVO_OK = 0,
  TVO_ERR_NULL = -1,
  TVO_ERR_SHAPE = -2,
  TVO_ERR_INDPTR = -3,   /* an indptr is negative, decreasing or past its buffer */
  TVO_ERR_KVLEN = -4,    /* L_b < n_b: draft slots missing from kv_indices      */
  TVO_ERR_MASKLEN = -5,  /* mask block of request b is not n_b * L_b bytes
                            (n_b * n_b in the prefix-visible form)               */
  TVO_ERR_SLOT = -6,     /* a key's slot is outside [0, num_slots)               */
  TVO_ERR_ALLOC = -7
};

typedef struct {
  const uint16_t* q;           /* bf16 bits [total_q, num_heads, 576]             */
  const uint16_t* kv;          /* bf16 bits [num_slots, 576]                       */
  const int32_t* kv_indices;   /* [total_kv]                                       */
  const int32_t* kv_indptr;    /* [batch + 1]                                      */
  const int32_t* qo_indptr;    /* [batch + 1]                                      */
  const uint8_t* mask;         /* [total_mask], nonzero = visible                  */
  const int32_t* mask_indptr;  /* [batch + 1]                                      */
  int32_t batch;
  int32_t num_heads;
  int64_t total_q;
  int64_t num_slots;
  int64_t total_kv;
  int64_t total_mask;
  float sm_scale;
  int32_t prefix_visible;      /* 0: block b is n_b x L_b bytes, stride L_b.
                                  1: block b is n_b x n_b bytes (the draft keys,
                                  stride n_b) and every prefix key is visible  */
  int32_t contiguous_prefix;   /* 0: key j of request b is slot
                                  kv_indices[kv_indptr[b] + j].
                                  1: for j < P_b = L_b - n_b it is slot
                                  kv_indices[kv_indptr[b]] + j (the prefix is one
                                  run of the pool); the other prefix entries
                                  are not read                                  */
} tvo_args;

/* Validate every precondition; TVO_OK or the first violation found. */
int tvo_check(const tvo_args* a);

/* Compute output rows.  A row id is g = token * num_heads + head.  rows == NULL
 * computes all total_q * num_heads rows in order.  out: [nrows, 512] fp64,
 * lse: [nrows] fp64 (natural log).  threads <= 0 keeps the OpenMP default. */
int tvo_attention(const tvo_args* a, const int64_t* rows, int64_t nrows, int threads,
                  double* out, double* lse);

int tvo_max_threads(void);
#endif
