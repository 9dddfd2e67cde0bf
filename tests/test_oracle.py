"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test checks the oracle against something the pages or the mathematics fix:
textbook dense attention done with library routines, brute force on tiny
inputs, closed forms, exact invariances, hand-derived fixtures and the live
shapes that page 2 prints.  Together they are chosen so that a plausible slip
in the oracle (a dropped RoPE term, V taken from the wrong dims, the mask
transposed or with the prefix-only stride, a missing scale, a log2 LSE, a
wrong head/draft mapping, kv_indices ignored, indptr offsets ignored) fails
at least one of them.  No GPU needed.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
import tv_workload as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f64(bits):
    return W.bf16_to_f32(bits).astype(np.float64)


def textbook(w, b, rows_tok, keys_j):
    """Dense softmax(c * Q K^T) V over an explicit key list, via scipy/numpy."""
    k0 = int(w.kv_indptr[b])
    K = f64(w.kv[w.kv_indices[k0 + np.asarray(keys_j)]])
    Q = f64(w.q[rows_tok])  # [n, H, 576]
    c = float(w.sm_scale)
    S = c * np.einsum("nhd,kd->nhk", Q, K)
    P = softmax(S, axis=-1)
    return P @ K[:, :512], logsumexp(S, axis=-1)


def dense_all_visible(w):
    w.mask[:] = 1
    return w


# ---------------------------------------------------------------- I1 dense case

@pytest.mark.parametrize("outlier_p", [0.0, 0.01])
def test_dense_mask_equals_textbook_attention(outlier_p):
    w = dense_all_visible(W.small(11, [37, 5], [4, 3], num_heads=3, outlier_p=outlier_p))
    o, l = oracle.run(w)
    for b in range(w.batch):
        toks = np.arange(w.qo_indptr[b], w.qo_indptr[b + 1])
        L = int(w.kv_lens[b])
        ro, rl = textbook(w, b, toks, np.arange(L))
        np.testing.assert_allclose(o[toks], ro, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l[toks], rl, rtol=1e-13, atol=1e-13)


def test_duplicate_slots_are_separate_keys():
    w = dense_all_visible(W.small(12, [6], [2], num_heads=2))
    w.kv_indices[1] = w.kv_indices[0]   # same slot gathered twice
    w.kv_indices[3] = w.kv_indices[0]
    o, l = oracle.run(w)
    ro, rl = textbook(w, 0, np.arange(2), np.arange(int(w.kv_lens[0])))
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, rl, rtol=1e-13)


# ---------------------------------------------------------- I2 ancestor subset

def test_tree_row_equals_attention_over_its_path():
    w = W.small(13, [23], [9], num_heads=4)
    o, l = oracle.run(w)
    P = w.prefix_lens[0]
    for i in range(9):
        path = W.ancestors_and_self(w.parents[0], i)
        keys = list(range(P)) + [P + k for k in path]
        # same keys in the same ascending order, as a one-row dense request
        sub = W.Workload(q=w.q[i:i + 1], kv=w.kv, kv_indices=w.kv_indices[keys],
                         kv_indptr=np.array([0, len(keys)], np.int32),
                         qo_indptr=np.array([0, 1], np.int32),
                         mask=np.ones(len(keys), np.uint8),
                         mask_indptr=np.array([0, len(keys)], np.int32),
                         sm_scale=w.sm_scale, num_heads=4)
        so, sl = oracle.run(sub)
        assert np.array_equal(so[0], o[i]) and np.array_equal(sl[0], l[i])


# --------------------------------------------------------- I3 slot permutation

def test_slot_permutation_is_bit_identical():
    w = W.small(14, [40, 17], [6, 4], num_heads=2)
    o, l = oracle.run(w)
    rng = np.random.default_rng(0)
    pi = rng.permutation(w.num_slots)
    kv2 = np.empty_like(w.kv)
    kv2[pi] = w.kv                      # row s moves to pi[s]
    w2 = W.Workload(**{**w.__dict__, "kv": kv2, "kv_indices": pi[w.kv_indices].astype(np.int32)})
    o2, l2 = oracle.run(w2)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


# ----------------------------------------------------------------- I4 one key

def test_single_visible_key_returns_its_value():
    w = W.small(15, [8], [3], num_heads=2)
    w.mask[:] = 0
    L = int(w.kv_lens[0])
    picks = [0, 5, L - 1]
    for i, j in enumerate(picks):
        w.mask[i * L + j] = 1
    o, l = oracle.run(w)
    for i, j in enumerate(picks):
        k = f64(w.kv[w.kv_indices[j]])
        for h in range(2):
            assert np.array_equal(o[i, h], k[:512])
            s = float(w.sm_scale) * math.fsum(f64(w.q[i, h]) * k)
            assert abs(l[i, h] - s) <= 1e-13 * max(1.0, abs(s))


# ---------------------------------------------------------- I5 brute force

def brute(w):
    """Scalar loops, math.fsum, exp(s)/sum(exp(s)) with no max shift."""
    N, H = w.q.shape[0], w.num_heads
    out = np.zeros((N, H, 512))
    lse = np.full((N, H), -np.inf)
    c = float(w.sm_scale)
    for b in range(w.batch):
        n = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        L = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
        for i in range(n):
            t = int(w.qo_indptr[b]) + i
            vis = [j for j in range(L) if w.mask[int(w.mask_indptr[b]) + i * L + j]]
            for h in range(H):
                if not vis:
                    continue
                qv = [float(x) for x in f64(w.q[t, h])]
                ks = [[float(x) for x in f64(w.kv[w.kv_indices[int(w.kv_indptr[b]) + j]])]
                      for j in vis]
                e = [math.exp(c * math.fsum(a * bb for a, bb in zip(qv, k))) for k in ks]
                z = math.fsum(e)
                for d in range(512):
                    out[t, h, d] = math.fsum(e[v] * ks[v][d] for v in range(len(vis))) / z
                lse[t, h] = math.log(z)
    return out, lse


@pytest.mark.parametrize("seed,prefix,ndraft,H", [(21, [3], [3], 2), (22, [2, 3], [2, 3], 1),
                                                   (23, [0, 1], [3, 2], 2)])
def test_brute_force_tiny(seed, prefix, ndraft, H):
    w = W.small(seed, prefix, ndraft, num_heads=H)
    # random (not tree) visibility so off-path entries matter too; keep >= 1 visible per row
    rng = np.random.default_rng(seed)
    w.mask[:] = (rng.random(w.mask.size) < 0.6).astype(np.uint8)
    o, l = oracle.run(w)
    bo, bl = brute(w)
    np.testing.assert_allclose(o, bo, rtol=1e-13, atol=1e-13)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(l))
    np.testing.assert_allclose(l[fin], bl[fin], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------ I6 q = 0

def test_zero_query_gives_mean_of_visible_values():
    w = W.small(16, [29, 7], [5, 4], num_heads=3)
    w.q[:] = 0
    o, l = oracle.run(w)
    for b in range(w.batch):
        L = int(w.kv_lens[b])
        for i in range(int(w.q_lens[b])):
            t = int(w.qo_indptr[b]) + i
            row = w.mask[int(w.mask_indptr[b]) + i * L: int(w.mask_indptr[b]) + (i + 1) * L]
            vis = np.flatnonzero(row)
            V = f64(w.kv[w.kv_indices[int(w.kv_indptr[b]) + vis]])[:, :512]
            mean = np.array([math.fsum(V[:, d]) for d in range(512)]) / len(vis)
            for h in range(3):
                np.testing.assert_allclose(o[t, h], mean, rtol=1e-15, atol=1e-15)
                assert abs(l[t, h] - math.log(len(vis))) <= 1e-15 * max(1, math.log(len(vis)))


def test_hand_derived_fixture():
    g = json.load(open(os.path.join(GOLD, "closed_form_tiny.json")))
    kvf = np.zeros((g["num_slots"], 576), np.float32)
    for j, s in enumerate(g["kv_indices"]):
        kvf[s, 0] = g["key_dim0"][j]
        kvf[s, 1] = g["key_dim1"][j]
        kvf[s, 511] = g["key_dim511"][j]
        kvf[s, 512] = g["key_dim512"][j]
    n = len(g["parent"])
    L = g["prefix_len"] + n
    mask = np.array(g["mask"], np.uint8)
    assert mask.size == n * L
    o, l = oracle.attention(np.zeros((n, 1, 576), np.uint16), W.bf16_round(kvf),
                            np.array(g["kv_indices"]), np.array(g["kv_indptr"]),
                            np.array(g["qo_indptr"]), mask, np.array(g["mask_indptr"]),
                            W.SM_SCALE, 1)
    for i in range(n):
        e = g["expected"]["row%d" % i]
        ref = np.zeros(512)
        ref[0], ref[1], ref[511] = e["dim0"], e["dim1"], e["dim511"]
        assert np.array_equal(o[i, 0], ref)
        assert abs(l[i, 0] - e["lse"]) < 1e-15


# ------------------------------------------------------ I7 two visible keys

def test_two_visible_keys_closed_form():
    w = W.small(17, [10], [2], num_heads=2)
    w.mask[:] = 0
    L = int(w.kv_lens[0])
    pairs = [(1, 7), (0, L - 1)]
    for i, (a, b) in enumerate(pairs):
        w.mask[i * L + a] = w.mask[i * L + b] = 1
    o, l = oracle.run(w)
    c = float(w.sm_scale)
    for i, (a, b) in enumerate(pairs):
        ka, kb = f64(w.kv[w.kv_indices[a]]), f64(w.kv[w.kv_indices[b]])
        for h in range(2):
            qv = f64(w.q[i, h])
            sa, sb = c * math.fsum(qv * ka), c * math.fsum(qv * kb)
            wa = 1.0 / (1.0 + math.exp(sb - sa))
            wb = 1.0 / (1.0 + math.exp(sa - sb))
            np.testing.assert_allclose(o[i, h], wa * ka[:512] + wb * kb[:512], rtol=1e-14, atol=1e-14)
            ref_l = max(sa, sb) + math.log1p(math.exp(-abs(sa - sb)))
            assert abs(l[i, h] - ref_l) <= 1e-14 * max(1.0, abs(ref_l))


# -------------------------------------------------------- I8 merge identity

def test_disjoint_key_sets_merge_by_lse():
    """Attention over A u B from the two halves: the identity a KV split relies on."""
    w = W.small(18, [50], [4], num_heads=2)
    o, l = oracle.run(w)
    L = int(w.kv_lens[0])
    cut = 23
    wa = W.Workload(**{**w.__dict__, "mask": w.mask.copy()})
    wb = W.Workload(**{**w.__dict__, "mask": w.mask.copy()})
    for i in range(4):
        wa.mask[i * L + cut:(i + 1) * L] = 0
        wb.mask[i * L:i * L + cut] = 0
    oa, la = oracle.run(wa)
    ob, lb = oracle.run(wb)
    lm = np.logaddexp(la, lb)
    om = np.exp(la - lm)[..., None] * oa + np.exp(lb - lm)[..., None] * ob
    np.testing.assert_allclose(lm, l, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(om, o, rtol=1e-13, atol=1e-13)


# ----------------------------------------------- I9 / I10 relabelings

def test_head_permutation_permutes_outputs():
    w = W.small(19, [31], [5], num_heads=5)
    o, l = oracle.run(w)
    perm = np.array([3, 0, 4, 1, 2])
    w2 = W.Workload(**{**w.__dict__, "q": np.ascontiguousarray(w.q[:, perm])})
    o2, l2 = oracle.run(w2)
    assert np.array_equal(o2, o[:, perm]) and np.array_equal(l2, l[:, perm])


def test_draft_row_permutation_permutes_outputs():
    w = W.small(20, [12], [6], num_heads=2)
    o, l = oracle.run(w)
    L = int(w.kv_lens[0])
    perm = np.array([5, 2, 0, 4, 1, 3])
    m = w.mask.reshape(6, L)[perm].reshape(-1)
    w2 = W.Workload(**{**w.__dict__, "q": np.ascontiguousarray(w.q[perm]), "mask": m})
    o2, l2 = oracle.run(w2)
    assert np.array_equal(o2, o[perm]) and np.array_equal(l2, l[perm])


def test_draft_relabeling_with_key_columns():
    """Relabel the drafts: q rows, mask rows and columns and draft slots move together."""
    w = W.small(24, [9], [5], num_heads=2)
    o, l = oracle.run(w)
    P, n = w.prefix_lens[0], 5
    L = P + n
    perm = np.array([2, 4, 0, 3, 1])  # new draft a is old draft perm[a]
    m = w.mask.reshape(n, L)
    cols = np.concatenate([np.arange(P), P + perm])
    m2 = m[perm][:, cols].reshape(-1)
    ki = w.kv_indices.copy()
    ki[P:] = w.kv_indices[P + perm]
    w2 = W.Workload(**{**w.__dict__, "q": np.ascontiguousarray(w.q[perm]), "mask": m2,
                       "kv_indices": ki})
    o2, l2 = oracle.run(w2)
    np.testing.assert_allclose(o2, o[perm], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l2, l[perm], rtol=1e-14, atol=1e-14)


# ------------------------------------------- batch structure and offsets

def test_batch_equals_requests_run_alone():
    w = W.small(25, [13, 0, 40, 5], [3, 2, 4, 1], num_heads=2)
    o, l = oracle.run(w)
    for b in range(w.batch):
        q0, q1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        k0, k1 = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
        m0, m1 = int(w.mask_indptr[b]), int(w.mask_indptr[b + 1])
        sub = W.Workload(q=w.q[q0:q1], kv=w.kv, kv_indices=w.kv_indices[k0:k1],
                         kv_indptr=np.array([0, k1 - k0], np.int32),
                         qo_indptr=np.array([0, q1 - q0], np.int32), mask=w.mask[m0:m1],
                         mask_indptr=np.array([0, m1 - m0], np.int32), sm_scale=w.sm_scale,
                         num_heads=2)
        so, sl = oracle.run(sub)
        assert np.array_equal(so, o[q0:q1]) and np.array_equal(sl, l[q0:q1])


def test_indptr_offsets_are_honoured():
    w = W.small(26, [7, 19], [3, 2], num_heads=2)
    o, l = oracle.run(w)
    pad_k, pad_m = 11, 29
    ki = np.concatenate([np.zeros(pad_k, np.int32), w.kv_indices])
    mk = np.concatenate([np.full(pad_m, 1, np.uint8), w.mask])
    w2 = W.Workload(**{**w.__dict__, "kv_indices": ki, "mask": mk,
                       "kv_indptr": (w.kv_indptr + pad_k).astype(np.int32),
                       "mask_indptr": (w.mask_indptr + pad_m).astype(np.int32)})
    o2, l2 = oracle.run(w2)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_row_subset_matches_full_run():
    w = W.small(27, [33, 4], [4, 5], num_heads=3)
    o, l = oracle.run(w)
    rows = np.array([0, 5, 13, 26, 9])
    so, sl = oracle.run(w, rows=rows)
    H = 3
    for r, g in enumerate(rows):
        assert np.array_equal(so[r], o[g // H, g % H]) and sl[r] == l[g // H, g % H]


# ---------------------------------------------------------- degenerate cases

def test_row_with_no_visible_key():
    w = W.small(28, [6], [3], num_heads=2)
    L = int(w.kv_lens[0])
    w.mask[L:2 * L] = 0
    o, l = oracle.run(w)
    assert np.all(o[1] == 0) and np.all(l[1] == -np.inf)
    assert np.all(np.isfinite(l[[0, 2]]))


def test_empty_batch_and_empty_request():
    w = W.small(29, [5, 3], [0, 2], num_heads=1)
    o, l = oracle.run(w)
    assert o.shape == (2, 1, 512) and np.all(np.isfinite(l))


def test_poisoned_pool_rows_are_never_read():
    w = W.small(30, [20], [4], num_heads=2, poison=True)
    assert np.isnan(f64(w.kv)).any(axis=1).sum() > 0
    o, l = oracle.run(w)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


# ---------------------------------------------- preconditions / pages' bug

def test_live_shapes_fix_the_mask_stride():
    g = json.load(open(os.path.join(GOLD, "live_shapes.json")))
    n, P = g["n_draft"], g["prefix_len"]
    assert g["mask"][0] == n * (P + n)
    w = W.config(1)
    assert list(w.q.shape) == g["q"] and w.num_heads == g["num_heads_per_rank"]
    assert w.mask.size == g["mask"][0] and int(w.kv_lens[0]) == P + n


def test_marshaling_bug_is_rejected():
    """Both halves of the pages' marshaling bug violate the precondition."""
    w = W.config(1)
    P, n = 21, 9
    assert oracle.check_workload(w) == 0
    # draft slots missing from kv_indices, mask still at the full stride
    w1 = W.Workload(**{**w.__dict__, "kv_indices": w.kv_indices[:P],
                       "kv_indptr": np.array([0, P], np.int32)})
    assert oracle.check_workload(w1) == -5
    # draft slots present, mask laid out with the prefix-only stride
    m = w.mask.reshape(n, P + n)[:, :P].reshape(-1)
    w2 = W.Workload(**{**w.__dict__, "mask": m, "mask_indptr": np.array([0, n * P], np.int32)})
    assert oracle.check_workload(w2) == -5
    with pytest.raises(oracle.OracleError):
        oracle.run(w2)


def test_other_preconditions():
    w = W.small(31, [5], [3], num_heads=1)
    bad = W.Workload(**{**w.__dict__, "kv_indices": w.kv_indices.copy()})
    bad.kv_indices[2] = w.num_slots
    assert oracle.check_workload(bad) == -6
    bad2 = W.Workload(**{**w.__dict__, "kv_indptr": np.array([0, 2], np.int32),
                         "mask_indptr": np.array([0, 6], np.int32)})
    assert oracle.check_workload(bad2) == -4
    bad3 = W.Workload(**{**w.__dict__, "qo_indptr": np.array([2, 1], np.int32)})
    assert oracle.check_workload(bad3) == -3


# ------------------------------------------------- generator structure

def test_generated_configs_structure():
    for k in (1, 2):
        w = W.config(k)
        assert oracle.check_workload(w) == 0
        for b in range(w.batch):
            L, n, P = int(w.kv_lens[b]), int(w.q_lens[b]), w.prefix_lens[b]
            m = w.mask[int(w.mask_indptr[b]):int(w.mask_indptr[b + 1])].reshape(n, L)
            assert np.all(m[:, :P] == 1)
            assert np.all(np.diag(m[:, P:]) == 1)          # each draft sees itself
            assert np.all(np.triu(m[:, P:], 1) == 0)        # never a later draft


# ------------------------------------------- prefix-visible form of the mask

def brute_prefix_visible(w):
    """Scalar loops over the prefix-visible form, read straight from its
    definition: row i of request b sees key j iff j < P_b = L_b - n_b, or
    byte i * n_b + (j - P_b) of the request's n_b x n_b block is nonzero."""
    N, H = w.q.shape[0], w.num_heads
    out = np.zeros((N, H, 512))
    lse = np.full((N, H), -np.inf)
    c = float(w.sm_scale)
    for b in range(w.batch):
        n = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        L = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
        P = L - n
        for i in range(n):
            t = int(w.qo_indptr[b]) + i
            vis = [j for j in range(L)
                   if j < P or w.mask[int(w.mask_indptr[b]) + i * n + (j - P)]]
            for h in range(H):
                if not vis:
                    continue
                qv = [float(x) for x in f64(w.q[t, h])]
                ks = [[float(x) for x in f64(w.kv[w.kv_indices[int(w.kv_indptr[b]) + j]])]
                      for j in vis]
                e = [math.exp(c * math.fsum(a * bb for a, bb in zip(qv, k))) for k in ks]
                z = math.fsum(e)
                for d in range(512):
                    out[t, h, d] = math.fsum(e[v] * ks[v][d] for v in range(len(vis))) / z
                lse[t, h] = math.log(z)
    return out, lse


@pytest.mark.parametrize("seed,prefix,ndraft,H", [(31, [100], [5], 4), (32, [300, 7, 0, 95],
                                                                        [3, 2, 0, 6], 3),
                                                   (33, [0], [4], 2)])
def test_prefix_visible_form_equals_full_mask(seed, prefix, ndraft, H):
    """A tree mask sees its whole prefix, so its prefix-visible form (the draft
    columns only) selects the same keys in the same order: bit-identical."""
    w = W.small(seed, prefix, ndraft, num_heads=H)
    pv = W.prefix_visible_form(w)
    assert pv.mask.size == sum(n * n for n in ndraft)
    a, la = oracle.run(w)
    b, lb = oracle.run(pv)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_prefix_visible_brute_force_with_arbitrary_draft_block():
    """Random (not tree) draft-key bits, some rows seeing no draft key at all."""
    w = W.prefix_visible_form(W.small(34, [3, 0], [3, 2], num_heads=2))
    rng = np.random.default_rng(34)
    w.mask[:] = (rng.random(w.mask.size) < 0.5).astype(np.uint8)
    w.mask[0:3] = 0  # request 0, draft 0 sees only its 3 prefix keys
    o, l = oracle.run(w)
    bo, bl = brute_prefix_visible(w)
    assert np.allclose(o, bo, rtol=1e-13, atol=1e-15)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(l))
    assert np.allclose(l[fin], bl[fin], rtol=1e-13, atol=1e-13)
    # request 1 has no prefix: a row whose draft bits are all 0 sees nothing
    w.mask[w.mask_indptr[1]:w.mask_indptr[1] + 2] = 0
    o, l = oracle.run(w)
    t = int(w.qo_indptr[1])
    assert np.all(o[t] == 0) and np.all(np.isneginf(l[t]))


def test_prefix_visible_stride_is_checked():
    """Mixing the two forms is the marshaling mistake again: a full n x L block
    passed as prefix-visible (or the reverse) is rejected."""
    w = W.small(35, [40], [4], num_heads=1)
    pv = W.prefix_visible_form(w)
    with pytest.raises(oracle.OracleError) as e:
        oracle.attention(w.q, w.kv, w.kv_indices, w.kv_indptr, w.qo_indptr, w.mask,
                         w.mask_indptr, w.sm_scale, w.num_heads, prefix_visible=True)
    assert e.value.code == -5
    with pytest.raises(oracle.OracleError) as e:
        oracle.attention(pv.q, pv.kv, pv.kv_indices, pv.kv_indptr, pv.qo_indptr, pv.mask,
                         pv.mask_indptr, pv.sm_scale, pv.num_heads, prefix_visible=False)
    assert e.value.code == -5


def test_prefix_visible_form_needs_a_visible_prefix():
    w = W.small(36, [10], [3], num_heads=1)
    w.mask[0] = 0
    with pytest.raises(ValueError):
        W.prefix_visible_form(w)


# ------------------------------------------ contiguous-prefix form (N4)

CONTIG = [(41, [100], [5], 4), (42, [300, 7, 0, 95], [3, 2, 0, 6], 3), (43, [0], [4], 2),
          (44, [33, 1], [1, 7], 5)]


@pytest.mark.parametrize("seed,prefix,ndraft,H", CONTIG)
def test_contiguous_prefix_form_equals_the_full_key_list(seed, prefix, ndraft, H):
    """With each prefix one run of the pool, the form that keeps only the run's
    first slot (the other prefix entries -1) selects the same keys in the same
    order as the full key list: bit-identical."""
    w = W.small(seed, prefix, ndraft, num_heads=H, placement="contiguous")
    c = W.contiguous_prefix_form(w)
    assert (c.kv_indices == -1).sum() == sum(max(p - 1, 0) for p in prefix)
    a, la = oracle.run(w)
    b, lb = oracle.run(c)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    # read as a full key list, the -1 entries are slots outside the pool
    assert oracle.check(c.q, c.kv, c.kv_indices, c.kv_indptr, c.qo_indptr, c.mask, c.mask_indptr,
                        c.sm_scale, c.num_heads) == (-6 if max(prefix) > 1 else 0)


@pytest.mark.parametrize("seed,prefix,ndraft,H", CONTIG)
def test_placement_does_not_change_the_result(seed, prefix, ndraft, H):
    """The generator draws the same key values, in key order, under both
    placements: random single slots and contiguous runs (in the contiguous-
    prefix form) give bit-identical outputs."""
    r = W.small(seed, prefix, ndraft, num_heads=H)
    c = W.contiguous_prefix_form(W.small(seed, prefix, ndraft, num_heads=H,
                                         placement="contiguous"))
    assert not np.array_equal(r.kv_indices[:3], c.kv_indices[:3])
    a, la = oracle.run(r)
    b, lb = oracle.run(c)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_contiguous_prefix_closed_form():
    """q = 0: every visible key weighs the same, so the output is the mean of
    the visible value rows, listed here by hand.  Pool of 8 rows with distinct
    values; the prefix run starts at slot 2 (keys at slots 2, 3, 4), the two
    drafts sit at slots 7 and 0; the middle prefix entries hold slots 5 and 6,
    which a reader of the full list would gather instead."""
    H = 2
    kv = np.zeros((8, 576), np.float32)
    for s_ in range(8):
        kv[s_, :512] = np.arange(512) * 0.001 + s_
        kv[s_, 512:] = -s_
    w = W.Workload(q=W.bf16_round(np.zeros((2, H, 576), np.float32)), kv=W.bf16_round(kv),
                   kv_indices=np.array([2, 5, 6, 7, 0], np.int32),
                   kv_indptr=np.array([0, 5], np.int32), qo_indptr=np.array([0, 2], np.int32),
                   mask=np.array([1, 1, 1, 1, 0, 1, 1, 1, 1, 1], np.uint8),
                   mask_indptr=np.array([0, 10], np.int32), sm_scale=W.SM_SCALE, num_heads=H,
                   contiguous_prefix=True)
    o, l = oracle.run(w)
    V = f64(w.kv)[:, :512]
    want0 = (V[2] + V[3] + V[4] + V[7]) / 4          # draft 0 sees its own key (slot 7)
    want1 = (V[2] + V[3] + V[4] + V[7] + V[0]) / 5   # draft 1 sees both drafts
    for h in range(H):
        np.testing.assert_allclose(o[0, h], want0, rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(o[1, h], want1, rtol=1e-15, atol=1e-15)
        assert l[0, h] == pytest.approx(math.log(4), abs=1e-15)
        assert l[1, h] == pytest.approx(math.log(5), abs=1e-15)
    # the full-list reading of the same arrays gathers slots 5 and 6
    o2, _ = oracle.attention(w.q, w.kv, w.kv_indices, w.kv_indptr, w.qo_indptr, w.mask,
                             w.mask_indptr, w.sm_scale, H)
    np.testing.assert_allclose(o2[0, 0], (V[2] + V[5] + V[6] + V[7]) / 4, rtol=1e-15)


def test_contiguous_prefix_run_must_lie_in_the_pool():
    w = W.contiguous_prefix_form(W.small(45, [20], [3], num_heads=1, placement="contiguous"))
    args = lambda ki: (w.q, w.kv, ki, w.kv_indptr, w.qo_indptr, w.mask, w.mask_indptr,  # noqa
                       w.sm_scale, 1)
    assert oracle.check(*args(w.kv_indices), contiguous_prefix=True) == 0
    for start in (-1, w.num_slots - 19, w.num_slots):
        ki = w.kv_indices.copy()
        ki[0] = start
        assert oracle.check(*args(ki), contiguous_prefix=True) == -6, start
    ki = w.kv_indices.copy()
    ki[0] = w.num_slots - 20  # the run ends at the pool's last row
    assert oracle.check(*args(ki), contiguous_prefix=True) == 0
    ki[21] = w.num_slots      # a draft slot outside the pool
    assert oracle.check(*args(ki), contiguous_prefix=True) == -6


# ------------------------------------------------ the marshaling step

import oracle.marshal as M  # noqa: E402


def marshal(w, prefix_visible=False, parents=True):
    x = W.marshal_inputs(w)
    return M.append_draft(x["kv_buf"], x["draft_kv"], x["out_cache_loc"], x["prefix_indices"],
                          x["prefix_indptr"], x["qo_indptr"],
                          x["parents"] if parents else None, prefix_visible=prefix_visible)


@pytest.mark.parametrize("make", [lambda: W.config(1), lambda: W.config(2),
                                  lambda: W.small(41, [300, 7, 0, 95], [3, 2, 0, 6], 2),
                                  lambda: W.chain(42, [5, 0], 4, 1)])
def test_marshal_rebuilds_the_generated_inputs(make):
    """The generator lays out keys and masks by its own route (per-request tree
    masks from ancestor lists); the step's definition must rebuild them exactly
    from the pieces, and put the draft rows back into the pool."""
    w = make()
    kv, ki, kp, m, mp = marshal(w)
    assert np.array_equal(ki, w.kv_indices) and np.array_equal(kp, w.kv_indptr)
    assert np.array_equal(m, w.mask) and np.array_equal(mp, w.mask_indptr)
    assert np.array_equal(kv.view(np.uint16), w.kv.view(np.uint16))
    kv, ki, kp, m, mp = marshal(w, prefix_visible=True)
    pv = W.prefix_visible_form(w)
    assert np.array_equal(m, pv.mask) and np.array_equal(mp, pv.mask_indptr)
    _, _, _, m, mp = marshal(w, parents=False)
    assert m is None and mp is None


def test_marshal_live_shape():
    """The pages' live call: 9 drafts after a 21-token prefix give a 270-byte
    mask at row stride 30 and 30 keys, the draft slots last."""
    live = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "live_shapes.json")))
    w = W.config(1)
    x = W.marshal_inputs(w)
    kv, ki, kp, m, mp = marshal(w)
    n, P = live["n_draft"], live["prefix_len"]
    assert m.size == live["mask"][0] == n * (P + n)
    assert int(kp[-1]) == P + n and np.array_equal(ki[P:], x["out_cache_loc"])


def test_marshal_mask_closed_forms():
    """Row i of the full form has P + depth(i) ones; a chain gives a lower
    triangle over the draft keys, a star (every node a child of node 0) the
    diagonal plus column 0."""
    P, n = 5, 6
    star = np.eye(n, dtype=np.uint8)
    star[:, 0] = 1
    for parents, block in [(np.arange(-1, n - 1), np.tril(np.ones((n, n), np.uint8))),
                           (np.array([-1] + [0] * (n - 1)), star)]:
        w = W.build(43, [P], [parents], 1, 64)
        kv, ki, kp, m, mp = marshal(w)
        rows = m.reshape(n, P + n)
        assert np.all(rows[:, :P] == 1)
        depth = [len(W.ancestors_and_self(parents, i)) for i in range(n)]
        assert list(rows.sum(axis=1)) == [P + d for d in depth]
        assert np.array_equal(rows[:, P:], block)
