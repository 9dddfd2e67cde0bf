"""Oracle for the marshaling step before verify attention (plain Python/numpy).

TEST INFRASTRUCTURE.  Only tests/ and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the HIP library.

What the step produces (page 2, "The Moment of Truth: Flipping the Switch",
section "The Long Road to Parity"): the draft tokens' latent rows are written
into the pool at their cache slots; each request's key list is its prefix
slots followed by its draft slots; its visibility mask has one byte per (draft,
key) at row stride prefix + drafts (the live mask of 9 x 30 bytes), where a
draft sees the whole prefix, itself and its ancestors in the draft tree.  In
the prefix-visible form (page 3, "The Pivot to Live Cutover", section "The
Technical Investigation": the custom mask without its prefix part) a request's
block keeps only the draft-key columns, n x n bytes.
"""
from __future__ import annotations

import numpy as np


def draft_path(parents_b: np.ndarray, i: int) -> set:
    """Draft i and its ancestors: follow parent links up to a root (-1)."""
    out = set()
    a = i
    while a >= 0:
        out.add(a)
        a = int(parents_b[a])
    return out


def append_draft(kv_buf, draft_kv, out_cache_loc, prefix_indices, prefix_indptr, qo_indptr,
                 parents=None, prefix_visible=False):
    """Returns (kv_buf after the writes, kv_indices, kv_indptr, mask, mask_indptr);
    mask and mask_indptr are None without parents.  parents[t] is the
    request-local index of draft token t's parent, -1 for a root."""
    kv = np.array(kv_buf, copy=True)
    B = len(qo_indptr) - 1
    for t in range(int(qo_indptr[B])):
        kv[int(out_cache_loc[t])] = draft_kv[t]
    keys, kv_indptr = [], [0]
    rows, mask_indptr = [], [0]
    for b in range(B):
        p0, p1 = int(prefix_indptr[b]), int(prefix_indptr[b + 1])
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        P, n = p1 - p0, q1 - q0
        keys.append(np.asarray(prefix_indices[p0:p1], dtype=np.int32))
        keys.append(np.asarray(out_cache_loc[q0:q1], dtype=np.int32))
        kv_indptr.append(kv_indptr[-1] + P + n)
        if parents is not None:
            pb = np.asarray(parents[q0:q1])
            for i in range(n):
                path = draft_path(pb, i)
                drafts = np.array([1 if k in path else 0 for k in range(n)], dtype=np.uint8)
                rows.append(drafts if prefix_visible else
                            np.concatenate([np.ones(P, dtype=np.uint8), drafts]))
            mask_indptr.append(mask_indptr[-1] + n * (n if prefix_visible else P + n))
    kv_indices = np.concatenate(keys) if keys else np.zeros(0, np.int32)
    kv_indptr = np.array(kv_indptr, dtype=np.int32)
    if parents is None:
        return kv, kv_indices.astype(np.int32), kv_indptr, None, None
    mask = np.concatenate(rows) if rows else np.zeros(0, np.uint8)
    return (kv, kv_indices.astype(np.int32), kv_indptr, mask.astype(np.uint8),
            np.array(mask_indptr, dtype=np.int32))

