"""Parity of the HIP path (called through the C ABI) against the fp64 oracle.

Bar (floating point): max |out - oracle| <= 8e-3 and sum|diff| / sum|oracle| <=
2e-3 on bf16-rounded inputs; a bf16 output may additionally differ by its own
rounding (half a bf16 ulp per element; in the mean relative error, that of the
reference rounded to bf16).  lse: derived from fp32
accumulation of 576-term scores, |diff| <= 2e-4 * max(1, |lse|).

The probabilities enter the P.V product as bf16.  Rounded once (the default),
they move an output by at most 2^-8 * max|v_d| (gpu_util.p_rounding_bound):
with N(0,1) values that stays under the bar, with the x30 outliers of the
large-batch config it does not, and that config is held to the bar with the
precise-probability flag (hi + lo pair, bound 2^-16 * max|v_d|); its
default-mode run is checked only against that derived bound, which is not the
bar.  C3, C4 (every row) and S1 also run with fp32 output at the literal bar,
with no allowance.  Visibility handling is checked exactly (same
visible-key set per row) and results are checked to be independent of the
split count: lse within 1e-5 in either mode, outputs within twice the
rounding bound.
"""
import numpy as np
import pytest

import oracle
import tv_workload as W
from gpu_util import GpuCall, compare, p_rounding_bound, run, sample_rows, upload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU present", allow_module_level=True)

import tree_verify_mla_paged_amd as tv  # noqa: E402  (fails loudly if the library is missing)


PRECISE = tv.FLAG_PRECISE_P


def full_check(w, num_splits=0, out_f32=False, label="", flags=0, **kw):
    ro, rl = oracle.run(w)
    o, l = run(w, num_splits=num_splits, out_f32=out_f32, flags=flags)
    return compare(o, l, ro, rl, bf16_out=not out_f32, label=label, **kw)


# ------------------------------------------------------------- the configs

@pytest.mark.parametrize("out_f32", [False, True])
def test_c1_live_shape(out_f32):
    print("C1 out_f32=%s" % out_f32, flush=True)
    full_check(W.config(1), out_f32=out_f32, label="C1")


@pytest.mark.parametrize("out_f32", [False, True])
def test_c2_segmented_batch(out_f32):
    print("C2 out_f32=%s" % out_f32, flush=True)
    full_check(W.config(2), out_f32=out_f32, label="C2")


_ORACLE = {}


def oracle_full(name, w):
    """The oracle over every row of a named configuration, computed once per
    session (C4's 512 rows x 200k keys take several seconds)."""
    if name not in _ORACLE:
        _ORACLE[name] = oracle.run(w)
    return _ORACLE[name]


@pytest.mark.parametrize("num_splits", [0, 32])
def test_c3_32k_prefix(num_splits):
    """bf16 output, every row."""
    print("C3 num_splits=%d" % num_splits, flush=True)
    w = W.config(3)
    ro, rl = oracle_full("C3", w)
    o, l = run(w, num_splits=num_splits)
    compare(o, l, ro, rl, bf16_out=True, label="C3")


@pytest.mark.parametrize("num_splits", [0, 32])
def test_c3_fp32_output_at_the_literal_bar(num_splits):
    """fp32 output, every row, no allowance: max |diff| <= 8e-3, mean relative
    error <= 2e-3."""
    print("C3 fp32 literal bar num_splits=%d" % num_splits, flush=True)
    w = W.config(3)
    ro, rl = oracle_full("C3", w)
    o, l = run(w, num_splits=num_splits, out_f32=True)
    st = compare(o, l, ro, rl, bf16_out=False, label="C3 f32")
    print("   %s" % st, flush=True)


@pytest.mark.parametrize("out_f32", [True, False])
def test_c4_200k_prefix_every_row(out_f32):
    """All 512 rows; the fp32 output at the literal bar."""
    print("C4 every row out_f32=%s" % out_f32, flush=True)
    w = W.config(4)
    ro, rl = oracle_full("C4", w)
    o, l = run(w, out_f32=out_f32)
    st = compare(o, l, ro, rl, bf16_out=not out_f32, label="C4")
    print("   %s" % st, flush=True)


@pytest.mark.parametrize("out_f32", [False, True])
def test_c5_large_batch_with_outliers(out_f32):
    """The x30 outliers, every row, at the bar, with the precise-probability
    flag: outlier x outlier scores move references by hundreds (log2 units)
    in about a fifth of the tiles, and a row that loses earlier terms at a
    move shows here even where a sample of rows would miss it."""
    print("C5 precise out_f32=%s, every row" % out_f32, flush=True)
    w = W.config(5)
    ro, rl = oracle_full("C5", w)
    o, l = run(w, out_f32=out_f32, flags=PRECISE)
    st = compare(o, l, ro, rl, bf16_out=not out_f32, label="C5 precise")
    print("   %s" % st, flush=True)


@pytest.mark.parametrize("out_f32", [False, True])
def test_c5_default_mode_stays_within_its_derived_error_bound(out_f32):
    """NOT a parity-bar test: without the precise flag the x30 outliers put the
    probability rounding's derived bound, (2^-8 + 2^-11) * max|v_d| (0.4-0.7
    absolute per dim at C5), far above the 8e-3 bar, and this mode is checked
    only against that bound (every row).  C5 meets the bar in precise mode
    (the test above)."""
    print("C5 default out_f32=%s, every row" % out_f32, flush=True)
    w = W.config(5)
    ro, rl = oracle_full("C5", w)
    o, l = run(w, out_f32=out_f32)
    st = compare(o, l, ro, rl, bf16_out=not out_f32, label="C5 default",
                 extra_abs=p_rounding_bound(w, precise=False),
                 mean_rel_max=2.0 ** -8 + 2.0 ** -11)
    print("   %s" % st, flush=True)


@pytest.mark.parametrize("out_f32", [False, True])
def test_long_prefix_live_shape(out_f32):
    """S1 (the live 9-draft, 8-head shape at a 32k prefix), every row; fp32
    output at the literal bar."""
    print("S1 (32k prefix, n=9, H=8) out_f32=%s" % out_f32, flush=True)
    w = W.sweep(1)
    ro, rl = oracle_full("S1", w)
    o, l = run(w, out_f32=out_f32)
    st = compare(o, l, ro, rl, bf16_out=not out_f32, label="S1")
    print("   %s" % st, flush=True)


# ------------------------------------------------ small shapes, every path

SMALL = [
    # seed, prefix lengths, draft counts, heads, num_splits
    (201, [100], [5], 8, 0),          # 4 tiles, ragged tail
    (202, [100], [5], 8, 3),          # 3 splits, ragged last split
    (203, [0], [1], 1, 0),            # one key
    (204, [31], [2], 1, 0),           # 33 keys: tile + 1
    (205, [64], [1], 3, 5),           # H not dividing 128
    (206, [300, 7, 0, 95], [3, 2, 0, 6], 5, 4),  # batch with an empty request
    (207, [250], [20], 16, 2),        # 320 rows: 3 row blocks, last partial
    (208, [40], [2], 64, 0),          # all heads of a model
    (209, [129], [4], 128, 3),        # 512 rows at H=128
    (210, [1000], [9], 8, 7),         # many splits, several tiles each
    (211, [5, 600, 33], [1, 24, 3], 64, 0),
]


@pytest.mark.parametrize("seed,prefix,ndraft,H,ns", SMALL)
@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("flags", [0, 1])
def test_small_shapes(seed, prefix, ndraft, H, ns, out_f32, flags):
    print("small seed=%d H=%d ns=%d f32=%s flags=%d" % (seed, H, ns, out_f32, flags), flush=True)
    w = W.small(seed, prefix, ndraft, num_heads=H)
    full_check(w, num_splits=ns, out_f32=out_f32, label="small%d" % seed, flags=flags)


# Row counts around the epilogue's 32-row blocks: one workgroup holds 1, 31,
# 33, 64, 97, 127 or 128 rows (and 129: a second workgroup of one row), so the
# staging rounds end on a partial block, a whole one and every block count
# from 1 to 4.  H = 1 reads the packed visibility words, H = 8 the mask bytes.
EPILOGUE_ROWS = [(1, 1), (31, 1), (33, 1), (64, 1), (97, 1), (127, 1), (129, 1),
                 (4, 8), (12, 8), (16, 8), (17, 8)]


@pytest.mark.parametrize("ndraft,H", EPILOGUE_ROWS)
@pytest.mark.parametrize("ns", [1, 2])
@pytest.mark.parametrize("flags", [0, 1])
def test_epilogue_row_counts(ndraft, H, ns, flags):
    """Every row against the oracle, fp32 output at the literal bar, with one
    split (the output written by the split kernel) and two (partials and the
    merge)."""
    print("epilogue rows=%d H=%d ns=%d flags=%d" % (ndraft * H, H, ns, flags), flush=True)
    w = W.small(300 + ndraft, [70], [ndraft], num_heads=H)
    full_check(w, num_splits=ns, out_f32=True, label="rows%d" % (ndraft * H), flags=flags)


def test_random_masks_many_splits():
    """Masks that are not trees (arbitrary visibility, rows with no visible key)."""
    w = W.small(220, [90, 13], [7, 4], num_heads=4)
    rng = np.random.default_rng(220)
    w.mask[:] = (rng.random(w.mask.size) < 0.3).astype(np.uint8)
    L0 = int(w.kv_lens[0])
    w.mask[2 * L0:3 * L0] = 0  # draft 2 of request 0 sees nothing
    for ns in (1, 2, 4):
        print("random masks ns=%d" % ns, flush=True)
        full_check(w, num_splits=ns, out_f32=True, label="randmask ns=%d" % ns)


# ------------------------------------------------- split-count invariance

def check_split_drift(o, l, ref_o, ref_l, tol_o, label):
    """Two split counts of one problem: lse within 1e-5; every output within
    twice the bound on the probability rounding (each run is within it of the
    exact result) plus 1e-5 for fp32 accumulation order; and the mean drift
    within 1/100 of that: the bound assumes every rounding error of the
    probabilities aligned, which independent roundings do not (measured at C3
    and S1, both modes: mean drift 0.0008-0.0012 of twice the bound, largest
    single value 0.048), so a drift common to many outputs stands out."""
    dl = float(np.abs(l - ref_l).max())
    do = np.abs(o - ref_o)
    ratio = float(np.mean(do / np.broadcast_to(tol_o, do.shape)))
    print("   %s: max |dlse| %.3g  max |dout| %.3g  mean |dout| / tol %.3g"
          % (label, dl, float(do.max()), ratio), flush=True)
    assert dl <= 1e-5, label
    assert (do <= tol_o).all(), label
    assert ratio <= 0.01, label


@pytest.mark.parametrize("flags", [0, 1])
def test_split_count_invariance(flags):
    """Every split count of C3 against the oracle at the parity bar (sampled
    rows), and against the single split (all rows, check_split_drift).  The
    counts take each merge form at its edges: the per-row merge (up to 32 fp16
    or 16 fp32 splits) issues 4, 8, 16 or 32 loads per row, the per-workgroup
    merge takes the rest."""
    w = W.config(3)
    rows = sample_rows(w, 64, seed=3)
    ro, rl = oracle.run(w, rows=rows)
    tol_o = 2 * p_rounding_bound(w, precise=bool(flags)) + 1e-5
    ref_o = ref_l = None
    for ns in (1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 32, 33, 64, 128):
        print("C3 split invariance ns=%d flags=%d" % (ns, flags), flush=True)
        g = GpuCall(w, num_splits=ns, out_f32=True, flags=flags)
        g.call()
        o, l = g.result()
        o = o.reshape(-1, 512)
        l = l.reshape(-1)
        compare(o[rows], l[rows], ro, rl, bf16_out=False, label="C3 ns=%d" % ns)
        if ref_o is None:
            ref_o, ref_l = o, l
            continue
        check_split_drift(o, l, ref_o, ref_l, tol_o, "ns=%d" % ns)


# ------------------------------------------------------ exact visibility

def test_visible_key_set_is_exact():
    """q = 0 makes every visible score 0, so each visible key gets weight exactly
    1/n_vis.  With V[j] = e_(j mod 512), n_vis * out recovers the visible set."""
    for seed, L_pref, n in ((230, 300, 6), (231, 20, 12)):
        w = W.small(seed, [L_pref], [n], num_heads=3)
        rng = np.random.default_rng(seed)
        w.mask[:] = (rng.random(w.mask.size) < 0.5).astype(np.uint8)
        L = int(w.kv_lens[0])
        assert L <= 512
        w.q[:] = 0
        vals = np.zeros((L, 576), np.float32)
        vals[np.arange(L), np.arange(L) % 512] = 1.0
        w.kv[w.kv_indices] = W.bf16_round(vals)
        o, l = run(w, out_f32=True)
        m = w.mask.reshape(n, L)
        for i in range(n):
            nv = int(m[i].sum())
            for h in range(3):
                if nv == 0:
                    assert l[i, h] == -np.inf and np.all(o[i, h] == 0)
                    continue
                got = np.rint(o[i, h, :L] * nv).astype(int)
                assert np.array_equal(got, m[i].astype(int)), (seed, i, h)
                assert abs(l[i, h] - np.log(nv)) < 1e-6


def test_invisible_sentinel_key_never_leaks():
    """One invisible key per row would dominate the softmax by e^30 if it leaked."""
    w = W.small(232, [77], [5], num_heads=2)
    L = int(w.kv_lens[0])
    qf = W.bf16_to_f32(w.q).astype(np.float64)
    for i in range(5):
        j = (13 * i + 7) % L
        w.mask[i * L + j] = 0
        # make key j score about +30 above the others for both heads of draft i
        k = qf[i].sum(axis=0)
        k = k / np.linalg.norm(k) * (30.0 / float(w.sm_scale)) / np.linalg.norm(qf[i], axis=1).mean()
        w.kv[w.kv_indices[j]] = W.bf16_round(k.astype(np.float32))
    full_check(w, out_f32=True, label="sentinel")


def test_single_visible_key_returns_its_value_bits():
    w = W.small(233, [70], [6], num_heads=4)
    L = int(w.kv_lens[0])
    w.mask[:] = 0
    picks = [0, 31, 32, 50, L - 1, 64]
    for i, j in enumerate(picks):
        w.mask[i * L + j] = 1
    g = GpuCall(w, num_splits=2)
    g.call()
    bits = g.out_bits().view(np.uint16)
    for i, j in enumerate(picks):
        v = w.kv[w.kv_indices[j], :512]
        for h in range(4):
            assert np.array_equal(bits[i, h], v), (i, j, h)


# --------------------------------------------------------- invariances

def test_slot_permutation_is_bit_identical():
    w = W.config(2)
    a = GpuCall(w, out_f32=True)
    a.call()
    rng = np.random.default_rng(5)
    pi = rng.permutation(w.num_slots)
    kv2 = np.empty_like(w.kv)
    kv2[pi] = w.kv
    w2 = W.Workload(**{**w.__dict__, "kv": kv2, "kv_indices": pi[w.kv_indices].astype(np.int32)})
    b = GpuCall(w2, out_f32=True)
    b.call()
    assert np.array_equal(a.out_bits(), b.out_bits())
    assert np.array_equal(a.lse.cpu().numpy(), b.lse.cpu().numpy())


def test_repeat_calls_are_deterministic():
    w = W.config(3)
    g = GpuCall(w)
    g.call()
    first = g.out_bits().copy()
    l1 = g.lse.cpu().numpy().copy()
    for _ in range(2):
        g.call()
        assert np.array_equal(g.out_bits(), first)
        assert np.array_equal(g.lse.cpu().numpy(), l1)


@pytest.mark.parametrize("flags", [0, 1])
def test_score_jumps_beyond_headroom_rescale(flags):
    """Rows whose maximum jumps by far more than 2^64 (log2 units) after their
    first tile, twice in a row (the reference moves and O and l are rescaled
    each time), in a split that also holds rows without a jump: scores of
    ~150 and ~300 (log2 units) after a first tile of unit scores.  The large
    components sit in RoPE dims (keys only, not values), so the outputs stay
    of unit size."""
    w = W.small(240, [400], [4], num_heads=2)
    qv = W.bf16_to_f32(w.q).copy()
    qv[1, 0, :] = 0
    qv[1, 0, 520] = 40.0
    qv[2, 1, 530] = 40.0
    w.q[:] = W.bf16_round(qv)
    for key, dim, val in ((170, 520, 36.0), (300, 520, 72.0), (250, 530, 72.0)):
        k = W.bf16_to_f32(w.kv[w.kv_indices[key]]).copy()
        k[dim] = val  # scores of 0.072 * 1440 = 104 and 0.072 * 2880 = 208 natural units
        w.kv[w.kv_indices[key]] = W.bf16_round(k)
    for ns in (1, 3):
        print("jump ns=%d flags=%d" % (ns, flags), flush=True)
        full_check(w, num_splits=ns, out_f32=True, label="jump ns=%d" % ns, flags=flags)


@pytest.mark.parametrize("flags", [0, 1])
def test_score_jumps_in_value_dims(flags):
    """The same two-jump pattern with the large components in value dims (the
    outputs then hold values up to 40): scores of 58 and 115 natural units
    after a first tile of unit scores."""
    w = W.small(240, [400], [4], num_heads=2)
    qv = W.bf16_to_f32(w.q).copy()
    qv[1, 0, :] = 0
    qv[1, 0, 7] = 40.0
    qv[2, 1, 9] = 40.0
    w.q[:] = W.bf16_round(qv)
    for key, dim, val in ((170, 7, 20.0), (300, 7, 40.0), (250, 9, 40.0)):
        k = W.bf16_to_f32(w.kv[w.kv_indices[key]]).copy()
        k[dim] = val  # scores of 0.072 * 800 = 58 and 0.072 * 1600 = 115 natural units
        w.kv[w.kv_indices[key]] = W.bf16_round(k)
    for ns in (1, 3):
        print("jump (value dims) ns=%d flags=%d" % (ns, flags), flush=True)
        full_check(w, num_splits=ns, out_f32=True, label="jump v ns=%d" % ns, flags=flags)


@pytest.mark.parametrize("flags", [0, 1])
def test_move_just_past_the_threshold_keeps_the_earlier_terms(flags):
    """After a first tile of zero scores a row meets a key scoring ~123.4
    (log2 units) and then one scoring ~126.5: the first holds about an eighth
    of the row's mass.  Whatever references and moves the kernel uses, no
    factor 2^(old - new) may flush it (a reference placed 60 above the first
    maximum would not move at the first key and would need 2^-126.5, below
    the smallest normal fp32, at the second)."""
    w = W.small(241, [300], [4], num_heads=2)
    qv = W.bf16_to_f32(w.q).copy()
    qv[1, 0, :] = 0
    qv[1, 0, 520] = 40.0
    w.q[:] = W.bf16_round(qv)
    kv = W.bf16_to_f32(w.kv).copy()
    kv[w.kv_indices, 520] = 0.0  # every other key of the row scores exactly 0
    kv[w.kv_indices[40], 520] = 29.625  # tile 1
    kv[w.kv_indices[100], 520] = 30.375  # tile 3
    w.kv[:] = W.bf16_round(kv)
    s2 = float(w.sm_scale) * 1.4426950408889634 * 40.0
    s_old, s_new = s2 * 29.625, s2 * 30.375
    # the pattern: the second key ~3.1 above the first, both ~124 above the rest
    assert 123.0 < s_old < 124.0 and 3.0 < s_new - s_old < 3.3
    # precise mode at the bar; the default mode within its derived bounds (per
    # element and relative): two keys carry nearly all the mass, so the bf16
    # rounding of their probabilities does not average out (flushing the
    # first key would miss by ~0.46, ~12 % relative)
    bounds = {} if flags else {"extra_abs": p_rounding_bound(w, precise=False),
                                 "mean_rel_max": 2.0 ** -8 + 2.0 ** -11}
    for ns in (1, 3):
        print("move past the threshold ns=%d flags=%d" % (ns, flags), flush=True)
        full_check(w, num_splits=ns, out_f32=True, label="move ns=%d" % ns, flags=flags,
                   **bounds)


@pytest.mark.parametrize("e", [20, -20])
def test_fp16_partials_keep_value_scale(e):
    """Split partial outputs are fp16 under a power-of-two scale per (row,
    split).  K/V scaled by 2^e and Q by 2^-e leave every score unchanged and
    scale the output by exactly 2^e: at 2^20 unscaled fp16 partials would
    overflow, at 2^-20 they would underflow.  Compared at the normal bar after
    undoing the scale."""
    w = W.small(250, [900], [6], num_heads=8)
    w.q[:] = W.bf16_round(W.bf16_to_f32(w.q) * np.float32(2.0 ** -e))
    ref = w.kv_indices
    w.kv[ref] = W.bf16_round(W.bf16_to_f32(w.kv[ref]) * np.float32(2.0 ** e))
    ro, rl = oracle.run(w)
    for ns in (0, 5):
        print("fp16 partial scale e=%d ns=%d" % (e, ns), flush=True)
        o, l = run(w, num_splits=ns, out_f32=True)
        compare(np.asarray(o, np.float64) * 2.0 ** -e, l, ro * 2.0 ** -e, rl, bf16_out=False,
                label="scale 2^%d ns=%d" % (e, ns),
                extra_abs=p_rounding_bound(w, precise=False) * 2.0 ** -e)


@pytest.mark.parametrize("ns", [0, 5])
def test_batch_longest_first_order(ns):
    """A batch of very unequal requests with several row blocks each (288 rows
    at 48 heads): the longest-first dispatch order must cover every (request,
    split, row block) exactly once."""
    print("longest-first batch ns=%d" % ns, flush=True)
    w = W.small(251, [3000, 10, 700, 0, 1500, 64, 2500], [5, 3, 6, 2, 4, 1, 6], num_heads=48)
    full_check(w, num_splits=ns, label="lpt ns=%d" % ns)


# ------------------------------------------------------------ capture

def test_hip_graph_capture_and_replay():
    w1 = W.config(2)
    w2 = W.config(2)
    # same shapes and bounds, different content: seed a second copy of the inputs
    rng = np.random.default_rng(77)
    w2 = W.Workload(**{**w1.__dict__, "q": W.bf16_round(rng.standard_normal(w1.q.shape,
                                                                             dtype=np.float32))})
    g = GpuCall(w1)
    g.call()
    eager = g.out_bits().copy()
    eager_l = g.lse.cpu().numpy().copy()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        g.call(stream=stream)
    for rep in range(3):
        g.out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(g.out_bits(), eager), rep
        assert np.array_equal(g.lse.cpu().numpy(), eager_l), rep
    # new device-side content, same bounds: the replay follows it
    g.t["q"].copy_(torch.from_numpy(w2.q.view(np.int16)).cuda())
    graph.replay()
    torch.cuda.synchronize()
    o, l = g.result()
    ro, rl = oracle.run(w2)
    compare(o, l, ro, rl, bf16_out=True, label="replay")


# ------------------------------------------------------- input checking

def test_check_inputs_catches_the_marshaling_bug():
    w = W.config(1)
    t = upload(w)
    p = tv.make_problem(1, 8, 9, 9, 30, w.num_slots, 30, 270)
    assert tv.check_inputs(p, t["kv_indices"], t["kv_indptr"], t["qo_indptr"],
                           t["mask_indptr"]) == (0, -1)
    # draft slots missing from kv_indices (L = 21) with the mask at stride 30
    kvp = torch.tensor([0, 21], dtype=torch.int32, device="cuda")
    assert tv.check_inputs(p, t["kv_indices"], kvp, t["qo_indptr"], t["mask_indptr"]) == (5, 0)
    # drafts present, mask laid out with the prefix-only stride (9 x 21 bytes)
    mp = torch.tensor([0, 189], dtype=torch.int32, device="cuda")
    assert tv.check_inputs(p, t["kv_indices"], t["kv_indptr"], t["qo_indptr"], mp) == (5, 0)
    # a slot outside the pool
    bad = t["kv_indices"].clone()
    bad[3] = w.num_slots
    assert tv.check_inputs(p, bad, t["kv_indptr"], t["qo_indptr"], t["mask_indptr"]) == (5, 0)


# ---------------------------------------------- prefix-visible mask form

PV_SHAPES = [
    # seed, prefix lengths, draft counts, heads, num_splits
    (301, [100], [5], 8, 0),
    (302, [250], [20], 16, 2),        # 16 heads: the full form reads bytes, this one words
    (303, [300, 7, 0, 95], [3, 2, 0, 6], 5, 4),
    (304, [1000], [9], 8, 7),
    (305, [0], [4], 3, 0),            # no prefix: the block is the whole mask
]


@pytest.mark.parametrize("seed,prefix,ndraft,H,ns", PV_SHAPES)
@pytest.mark.parametrize("out_f32", [False, True])
def test_prefix_visible_small(seed, prefix, ndraft, H, ns, out_f32):
    print("prefix-visible seed=%d H=%d ns=%d f32=%s" % (seed, H, ns, out_f32), flush=True)
    w = W.prefix_visible_form(W.small(seed, prefix, ndraft, num_heads=H))
    full_check(w, num_splits=ns, out_f32=out_f32, label="pv%d" % seed)


def test_prefix_visible_arbitrary_draft_block():
    """Random draft-key bits; a row of a request without prefix sees nothing."""
    w = W.prefix_visible_form(W.small(306, [70, 0], [6, 3], num_heads=4))
    rng = np.random.default_rng(306)
    w.mask[:] = (rng.random(w.mask.size) < 0.4).astype(np.uint8)
    w.mask[w.mask_indptr[1]:w.mask_indptr[1] + 3] = 0
    for ns in (1, 3):
        print("prefix-visible random block ns=%d" % ns, flush=True)
        full_check(w, num_splits=ns, out_f32=True, label="pv random ns=%d" % ns)


def test_prefix_visible_equals_full_mask_bits():
    """A tree mask and its prefix-visible form give the kernels the same
    visibility, so the outputs agree bit for bit."""
    for w in (W.small(307, [700], [12], num_heads=16), W.config(2)):
        print("prefix-visible vs full: %s" % w.name, flush=True)
        a = GpuCall(w, out_f32=True)
        a.call()
        b = GpuCall(W.prefix_visible_form(w), out_f32=True)
        b.call()
        assert np.array_equal(a.out_bits(), b.out_bits())
        assert np.array_equal(a.lse.cpu().numpy().view(np.int32),
                              b.lse.cpu().numpy().view(np.int32))


def test_prefix_visible_c3():
    """Every row; the oracle is the full mask's (both forms give every row the
    same visible keys, which the oracle's own pins check)."""
    print("C3 prefix-visible", flush=True)
    w = W.config(3)
    ro, rl = oracle_full("C3", w)
    o, l = run(W.prefix_visible_form(w))
    compare(o, l, ro, rl, bf16_out=True, label="C3 prefix-visible")


def test_check_inputs_prefix_visible_stride():
    w = W.prefix_visible_form(W.config(1))
    t = upload(w)
    p = tv.make_problem(1, 8, 9, 9, 30, w.num_slots, 30, 81, flags=tv.FLAG_PREFIX_VISIBLE)
    assert tv.check_inputs(p, t["kv_indices"], t["kv_indptr"], t["qo_indptr"],
                           t["mask_indptr"]) == (0, -1)
    # the full n x L block (270 bytes) announced as prefix-visible
    full = W.config(1)
    p = tv.make_problem(1, 8, 9, 9, 30, w.num_slots, 30, 270, flags=tv.FLAG_PREFIX_VISIBLE)
    mp = torch.from_numpy(full.mask_indptr).to("cuda")
    assert tv.check_inputs(p, t["kv_indices"], t["kv_indptr"], t["qo_indptr"], mp) == (5, 0)


# ------------------------------------ contiguous-prefix form (N4)

CONTIG_SHAPES = [
    # seed, prefix lengths, draft counts, heads, num_splits
    (311, [100], [5], 8, 0),              # 4 tiles, ragged tail
    (312, [250], [20], 16, 2),            # the prefix ends inside a tile
    (313, [300, 7, 0, 95], [3, 2, 0, 6], 5, 4),  # packed words; empty request; no prefix
    (314, [1000], [9], 8, 7),
    (315, [0], [4], 3, 0),                # no prefix at all
    (316, [31, 32, 33], [1, 1, 1], 64, 0),  # prefix ends at, before, after a tile edge
]


@pytest.mark.parametrize("seed,prefix,ndraft,H,ns", CONTIG_SHAPES)
@pytest.mark.parametrize("out_f32", [False, True])
def test_contiguous_prefix_small(seed, prefix, ndraft, H, ns, out_f32):
    """Each prefix one run of the pool, passed by its first slot only (the
    other prefix entries of kv_indices are -1, outside the pool)."""
    print("contiguous prefix seed=%d H=%d ns=%d f32=%s" % (seed, H, ns, out_f32), flush=True)
    w = W.contiguous_prefix_form(W.small(seed, prefix, ndraft, num_heads=H,
                                         placement="contiguous"))
    full_check(w, num_splits=ns, out_f32=out_f32, label="contig%d" % seed)


@pytest.mark.parametrize("flags", [0, 1])
def test_contiguous_prefix_gives_the_random_placement_bits(flags):
    """The generator gives both placements the same key values in key order:
    the run form of the contiguous placement and the key list of the random
    placement give bit-identical outputs (S1, and a batch with packed words)."""
    for make in (lambda pl: W.sweep(1, placement=pl),
                 lambda pl: W.small(317, [3000, 17, 0, 900], [5, 3, 2, 7], num_heads=7,
                                    placement=pl)):
        r = make("random")
        c = W.contiguous_prefix_form(make("contiguous"))
        print("contiguous vs random placement: %s flags=%d" % (r.name, flags), flush=True)
        a = GpuCall(r, out_f32=True, flags=flags)
        a.call()
        b = GpuCall(c, out_f32=True, flags=flags)
        b.call()
        assert np.array_equal(a.out_bits(), b.out_bits())
        assert np.array_equal(a.lse.cpu().numpy().view(np.int32),
                              b.lse.cpu().numpy().view(np.int32))


def test_contiguous_prefix_s1_against_the_oracle():
    print("S1 contiguous prefix", flush=True)
    w = W.contiguous_prefix_form(W.sweep(1, placement="contiguous"))
    ro, rl = oracle.run(w)
    o, l = run(w, out_f32=True)
    compare(o, l, ro, rl, bf16_out=False, label="S1 contiguous")


def test_check_inputs_contiguous_prefix_run():
    w = W.contiguous_prefix_form(W.small(318, [40, 25], [3, 2], num_heads=8,
                                         placement="contiguous"))
    t = upload(w)
    p = tv.make_problem(w.batch, 8, w.total_q, w.max_q_len, w.max_kv_len, w.num_slots,
                        int(w.kv_indices.size), int(w.mask.size), flags=tv.FLAG_CONTIGUOUS_PREFIX)
    assert tv.check_inputs(p, t["kv_indices"], t["kv_indptr"], t["qo_indptr"],
                           t["mask_indptr"]) == (0, -1)
    # read as a full key list, the -1 entries are slots outside the pool
    p.flags = 0
    assert tv.check_inputs(p, t["kv_indices"], t["kv_indptr"], t["qo_indptr"],
                           t["mask_indptr"]) == (5, 0)
    p.flags = tv.FLAG_CONTIGUOUS_PREFIX
    bad = t["kv_indices"].clone()
    bad[int(w.kv_indptr[1])] = w.num_slots - 24  # request 1's run of 25 ends past the pool
    assert tv.check_inputs(p, bad, t["kv_indptr"], t["qo_indptr"], t["mask_indptr"]) == (5, 1)


@pytest.mark.parametrize("flags", [0, 1])
def test_contiguous_prefix_pool_beyond_4gib(flags):
    """The run form in a pool larger than 4 GiB (64-bit gather addresses): the
    same keys moved to the top of the big pool give the same bits."""
    print("contiguous prefix, pool beyond 4 GiB flags=%d" % flags, flush=True)
    w = W.contiguous_prefix_form(W.small(319, [900, 37, 2500], [7, 3, 12], num_heads=8,
                                         placement="contiguous"))
    g = GpuCall(w, num_splits=3, out_f32=True, flags=flags)
    g.call()
    narrow = g.out_bits().copy()
    offset = WIDE_SLOTS - w.num_slots
    big = torch.full((WIDE_SLOTS, 576), 0x7FC0, dtype=torch.int16, device="cuda")
    big[offset:].copy_(g.t["kv"])
    ki = g.t["kv_indices"].long()
    idx = torch.where(ki >= 0, ki + offset, ki).to(torch.int32)  # the -1 entries stay unread
    p = tv.make_problem(w.batch, w.num_heads, w.total_q, w.max_q_len, w.max_kv_len, WIDE_SLOTS,
                        int(w.kv_indices.size), int(w.mask.size), 3, tv.OUT_F32,
                        flags | tv.FLAG_CONTIGUOUS_PREFIX)
    out = torch.full_like(g.out, float("nan"))
    lse = torch.full_like(g.lse, float("nan"))
    ws = torch.empty(max(tv.workspace_bytes(p), 256), dtype=torch.uint8, device="cuda")
    tv.verify_attn(p, g.t["q"], big, idx, g.t["kv_indptr"], g.t["qo_indptr"], g.t["mask"],
                   g.t["mask_indptr"], float(w.sm_scale), out, lse, ws, ws.numel())
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int32).cpu().numpy(), narrow)
    o, l = g.result()
    ro, rl = oracle.run(w)
    compare(o, l, ro, rl, bf16_out=False, label="contig wide flags=%d" % flags)
    del big
    torch.cuda.empty_cache()


# ------------------------------------- long splits over one row block

def _plan_tiles(w, **kw):
    from gpu_util import problem_for
    pl = tv.plan(problem_for(w, **kw))
    return pl, pl["split_keys"] // 32


LONG_SHAPES = [
    # seed, prefix lengths, draft counts, heads, num_splits: one row block (<= 128
    # rows), splits of many tiles with ragged last splits
    (801, [3000], [5], 8, 1),        # 94 tiles in one split
    (802, [3000], [5], 8, 3),        # 32-tile splits, ragged last
    (803, [3000], [5], 8, 12),       # 8-tile splits, last split 6 keys
    (804, [2300], [9], 8, 9),        # 9-tile splits, last split 5 keys
    (805, [8 * 32 * 4 - 5], [5], 3, 4),  # packed words at 3 heads; exactly 8 tiles each
    (806, [3000, 2500, 17, 0], [5, 3, 2, 2], 16, 1),  # short and prefix-less requests
    (807, [4000], [1], 128, 2),      # one draft x 128 heads: a full row block
]


@pytest.mark.parametrize("seed,prefix,ndraft,H,ns", LONG_SHAPES)
@pytest.mark.parametrize("out_f32", [False, True])
def test_long_splits_one_row_block(seed, prefix, ndraft, H, ns, out_f32):
    w = W.small(seed, prefix, ndraft, num_heads=H)
    pl, tiles = _plan_tiles(w, num_splits=ns)
    assert pl["row_blocks"] == 1 and tiles >= 8, pl
    print("long split seed=%d H=%d ns=%d tiles/split=%d f32=%s" % (seed, H, ns, tiles, out_f32),
          flush=True)
    full_check(w, num_splits=ns, out_f32=out_f32, label="long%d" % seed)


@pytest.mark.parametrize("flags", [0, 1])
def test_long_splits_in_every_form(flags):
    """Precise mode, the contiguous-prefix form and the prefix-visible form, and
    arbitrary (non-tree) masks, over long splits of one row block."""
    base = W.small(808, [3100], [6], num_heads=8)
    cont = W.contiguous_prefix_form(W.small(808, [3100], [6], num_heads=8,
                                            placement="contiguous"))
    pv = W.prefix_visible_form(base)
    rnd = W.small(809, [2900], [7], num_heads=8)
    rng = np.random.default_rng(809)
    rnd.mask[:] = (rng.random(rnd.mask.size) < 0.4).astype(np.uint8)
    for w in (base, cont, pv, rnd):
        for ns in (1, 5):
            print("long split form %s ns=%d flags=%d" % (w.name, ns, flags), flush=True)
            full_check(w, num_splits=ns, out_f32=True, flags=flags,
                       label="long %s ns=%d" % (w.name, ns))


def test_s3_200k_every_row():
    """S3 (9 drafts x 8 heads over 200k keys, 25-tile splits): every row, fp32
    output at the literal bar."""
    print("S3 every row", flush=True)
    w = W.sweep(3)
    ro, rl = oracle_full("S3", w)
    o, l = run(w, out_f32=True)
    st = compare(o, l, ro, rl, bf16_out=False, label="S3")
    print("   %s" % st, flush=True)


@pytest.mark.parametrize("flags", [0, 1])
def test_split_invariance_of_a_few_row_request(flags):
    """S1 split 1, 4, 16 and 205 ways (1025, 257, 65 and 5 tiles per split):
    each against the oracle at the parity bar (sampled rows), and against the
    single split (check_split_drift)."""
    w = W.sweep(1)
    rows = sample_rows(w, 24, seed=5)
    ro, rl = oracle.run(w, rows=rows)
    tol_o = 2 * p_rounding_bound(w, precise=bool(flags)) + 1e-5
    ref_o = ref_l = None
    for ns in (1, 4, 16, 205):
        print("S1 split invariance ns=%d flags=%d" % (ns, flags), flush=True)
        g = GpuCall(w, num_splits=ns, out_f32=True, flags=flags)
        g.call()
        o, l = g.result()
        o = o.reshape(-1, 512)
        l = l.reshape(-1)
        compare(o[rows], l[rows], ro, rl, bf16_out=False, label="S1 ns=%d" % ns)
        if ref_o is None:
            ref_o, ref_l = o, l
            continue
        check_split_drift(o, l, ref_o, ref_l, tol_o, "ns=%d" % ns)


# ------------------------------ other workloads of the same kernels

@pytest.mark.parametrize("H", [16, 128])
def test_plain_decode_batch(H):
    """One query token per request (mask: the prefix and itself): plain MLA
    decode over the paged pool."""
    print("plain decode H=%d" % H, flush=True)
    w = W.chain(401, [5000, 32768, 100, 1], 1, num_heads=H)
    full_check(w, out_f32=True, label="decode H=%d" % H)


@pytest.mark.parametrize("ns", [0, 3])
def test_causal_chain_verify(ns):
    """Drafts forming one chain: a causal mask over the draft keys."""
    print("chain verify ns=%d" % ns, flush=True)
    w = W.chain(402, [3000, 17], 12, num_heads=16)
    full_check(w, num_splits=ns, out_f32=True, label="chain ns=%d" % ns)
    full_check(W.prefix_visible_form(w), num_splits=ns, label="chain pv ns=%d" % ns)


# ------------------------------------- guard bands and replays with new lengths

@pytest.mark.parametrize("ns", [1, 3])
def test_rows_outside_requests_are_untouched(ns):
    """q rows before the first request and after the last belong to no request:
    their out and lse entries keep whatever they held (NaN canaries here)."""
    print("guard rows ns=%d" % ns, flush=True)
    import dataclasses
    w = W.small(601, [200, 40], [5, 3], num_heads=8)
    rng = np.random.default_rng(601)
    front = W.bf16_round(rng.standard_normal((3, 8, 576), dtype=np.float32))
    back = W.bf16_round(rng.standard_normal((5, 8, 576), dtype=np.float32))
    w2 = dataclasses.replace(w, q=np.concatenate([front, w.q, back]),
                             qo_indptr=(w.qo_indptr + 3).astype(np.int32))
    for out_f32 in (False, True):
        g = GpuCall(w2, num_splits=ns, out_f32=out_f32)
        g.call()
        o, l = g.result()
        inside = slice(3, 3 + w.total_q)
        assert np.all(np.isnan(o[:3])) and np.all(np.isnan(o[inside.stop:]))
        assert np.all(np.isnan(l[:3])) and np.all(np.isnan(l[inside.stop:]))
        ro, rl = oracle.run(w)
        compare(o[inside], l[inside], ro, rl, bf16_out=not out_f32, label="guard ns=%d" % ns)


@pytest.mark.parametrize("H", [8, 3])  # mask bytes read in the loop / packed words
def test_request_longer_than_the_plan_stays_inside_its_buffers(H):
    """A request of 310 keys under a problem that announces at most 100
    (max_kv_len, a broken precondition) and one split: the kernels take the
    plan's ceil(100 / 32) = 4 tiles, the first 128 keys, so nothing is written
    through the absent partial buffers and no visibility word lands outside
    its row.  The rows of the request equal the oracle on those 128 keys (mask
    rows still at their real stride 310); the rows around it keep their
    canaries."""
    print("over-long request H=%d" % H, flush=True)
    import dataclasses
    w = W.small(604, [300], [10], num_heads=H)
    L, n = int(w.kv_lens[0]), int(w.q_lens[0])
    assert L == 310
    rng = np.random.default_rng(604)
    front = W.bf16_round(rng.standard_normal((2, H, 576), dtype=np.float32))
    back = W.bf16_round(rng.standard_normal((3, H, 576), dtype=np.float32))
    wg = dataclasses.replace(w, q=np.concatenate([front, w.q, back]),
                             qo_indptr=(w.qo_indptr + 2).astype(np.int32))
    g = GpuCall(wg, num_splits=1, out_f32=True, max_kv_len=100)
    assert g.plan["max_splits"] == 1 and g.plan["merge"] == 0
    g.call()
    o, l = g.result()
    inside = slice(2, 2 + n)
    assert np.all(np.isnan(o[:2])) and np.all(np.isnan(o[inside.stop:]))
    assert np.all(np.isnan(l[:2])) and np.all(np.isnan(l[inside.stop:]))
    cut = dataclasses.replace(
        w, kv_indices=w.kv_indices[:128].copy(), kv_indptr=np.array([0, 128], np.int32),
        mask=w.mask.reshape(n, L)[:, :128].copy().reshape(-1),
        mask_indptr=np.array([0, n * 128], np.int32))
    ro, rl = oracle.run(cut)
    compare(o[inside], l[inside], ro, rl, bf16_out=False, label="over-long H=%d" % H)


def test_graph_replay_follows_new_lengths_within_bounds():
    """A captured call replays over device-side lengths that changed after the
    capture (shorter prefixes, one request emptied), within the captured bounds."""
    print("graph replay with new lengths", flush=True)
    big = W.small(602, [3000, 1500, 700], [6, 6, 6], num_heads=8, pool=12000)
    small = W.small(603, [900, 0, 2500], [6, 6, 6], num_heads=8, pool=12000)
    g = GpuCall(big)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        g.call(stream=stream)
    graph.replay()
    torch.cuda.synchronize()
    o, l = g.result()
    ro, rl = oracle.run(big)
    compare(o, l, ro, rl, bf16_out=True, label="replay big")
    # the new inputs go into the front of the same (larger) buffers
    for k, v in (("q", small.q.view(np.int16)), ("kv", small.kv.view(np.int16)),
                 ("kv_indices", small.kv_indices), ("kv_indptr", small.kv_indptr),
                 ("qo_indptr", small.qo_indptr), ("mask", small.mask),
                 ("mask_indptr", small.mask_indptr)):
        src = torch.from_numpy(np.ascontiguousarray(v)).cuda().reshape(-1)
        g.t[k].view(-1)[:src.numel()].copy_(src)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    o, l = g.result()
    ro, rl = oracle.run(small)
    compare(o, l, ro, rl, bf16_out=True, label="replay small")


# ------------------------------------------------- pools beyond 4 GiB

WIDE_SLOTS = 4_200_000  # 4.84 GB of 1152-byte rows: gathers take 64-bit addresses


@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("H", [8, 3])  # mask bytes read in the loop / packed words
def test_pool_beyond_4gib_gives_the_same_bits(flags, H):
    """The same keys moved to the top of a pool larger than 4 GiB (the slot
    offsets no longer fit 32 bits, so the gathers use 64-bit addresses) give
    bit-identical outputs; the rest of the big pool is NaN."""
    print("pool beyond 4 GiB flags=%d H=%d" % (flags, H), flush=True)
    assert WIDE_SLOTS * 1152 > 2 ** 32
    w = W.small(701, [900, 37, 2500], [7, 3, 12], num_heads=H)
    g = GpuCall(w, num_splits=3, out_f32=True, flags=flags)
    g.call()
    narrow = g.out_bits().copy()
    narrow_l = g.lse.cpu().numpy().copy()
    offset = WIDE_SLOTS - w.num_slots
    big = torch.full((WIDE_SLOTS, 576), 0x7FC0, dtype=torch.int16, device="cuda")
    big[offset:].copy_(g.t["kv"])
    idx = (g.t["kv_indices"].long() + offset).to(torch.int32)
    p = tv.make_problem(w.batch, w.num_heads, w.total_q, w.max_q_len, w.max_kv_len, WIDE_SLOTS,
                        int(w.kv_indices.size), int(w.mask.size), 3, tv.OUT_F32, flags)
    out = torch.full_like(g.out, float("nan"))
    lse = torch.full_like(g.lse, float("nan"))
    ws = torch.empty(max(tv.workspace_bytes(p), 256), dtype=torch.uint8, device="cuda")
    tv.verify_attn(p, g.t["q"], big, idx, g.t["kv_indptr"], g.t["qo_indptr"], g.t["mask"],
                   g.t["mask_indptr"], float(w.sm_scale), out, lse, ws, ws.numel())
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int32).cpu().numpy(), narrow)
    assert np.array_equal(lse.cpu().numpy().view(np.int32), narrow_l.view(np.int32))
    o, l = g.result()
    ro, rl = oracle.run(w)
    compare(o, l, ro, rl, bf16_out=False, label="wide flags=%d" % flags)
    del big
    torch.cuda.empty_cache()


def test_timed_entry_point_matches_and_stamps_events():
    """tv_verify_attn_timed runs the same kernels (same bits) and stamps the two
    events with the split kernel's own dispatch: a positive duration."""
    print("timed entry point", flush=True)
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from bench import HipEvents
    w = W.config(2)
    g = GpuCall(w, out_f32=True)
    g.call()
    ref = g.out_bits().copy()
    ref_l = g.lse.cpu().numpy().copy()
    g.out.fill_(0)
    ev = HipEvents()
    a, b = ev.create(), ev.create()
    t = g.t
    tv.verify_attn_timed(g.p, t["q"], t["kv"], t["kv_indices"], t["kv_indptr"], t["qo_indptr"],
                         t["mask"], t["mask_indptr"], float(w.sm_scale), g.out, g.lse, g.ws,
                         g.ws.numel(), a, b)
    ms = ev.elapsed_ms(a, b)
    torch.cuda.synchronize()
    ev.destroy(a)
    ev.destroy(b)
    assert np.array_equal(g.out_bits(), ref)
    assert np.array_equal(g.lse.cpu().numpy(), ref_l)
    assert 0.0 < ms < 100.0, ms


def test_marshaling_bug_runs_but_answers_the_wrong_question():
    """The pages' failure: the draft slots left out of kv_indices (21 keys, not
    30) and the mask at the prefix-only stride (9 x 21).  Such inputs are
    well-formed, so the call runs and matches the oracle on those same inputs,
    but its output is far from the correct inputs' (mean relative error 0.24
    on this seeded workload against the 2e-3 bar)."""
    print("marshaling bug symptom", flush=True)
    import dataclasses
    w = W.config(1)
    bad = dataclasses.replace(w, kv_indices=w.kv_indices[:21].copy(),
                              kv_indptr=np.array([0, 21], np.int32),
                              mask=np.ones(9 * 21, np.uint8),
                              mask_indptr=np.array([0, 189], np.int32))
    o, l = run(bad, out_f32=True)
    rb, lb = oracle.run(bad)
    compare(o, l, rb, lb, bf16_out=False, label="bad inputs, same oracle")
    ro, rl = oracle.run(w)
    rel = float(np.abs(o - ro).sum() / np.abs(ro).sum())
    print("   relative error against the correct inputs: %.3f" % rel, flush=True)
    assert rel > 0.1


def test_many_tiny_requests():
    """3000 requests of 0-3 drafts after 0-40 prefix keys: a 3000-row grid y,
    and a longest-first order over 3000 work items."""
    print("3000 tiny requests", flush=True)
    rng = np.random.default_rng(605)
    prefix = [int(x) for x in rng.integers(0, 40, size=3000)]
    drafts = [int(x) for x in rng.integers(0, 4, size=3000)]
    w = W.small(605, prefix, drafts, 8, max_branch=2)
    full_check(w, out_f32=True, label="3000 requests")
    full_check(w, num_splits=2, label="3000 requests, 2 splits")


@pytest.mark.parametrize("H", [7, 9, 10, 11, 12])
def test_heads_around_the_mask_byte_threshold(H):
    """Waves of 32 rows span at most 4 drafts for H = 8, 10 and 11 and up (the
    split kernel reads the mask bytes, two drafts per load), more for H = 7 and
    9 (packed words): 13 drafts put every residue of a wave's first row in play."""
    print("heads around the mask-byte threshold H=%d" % H, flush=True)
    w = W.small(606 + H, [150, 9], [13, 6], num_heads=H)
    rng = np.random.default_rng(606 + H)
    w.mask[:] = (rng.random(w.mask.size) < 0.6).astype(np.uint8)
    for ns in (1, 3):
        full_check(w, num_splits=ns, out_f32=True, label="H=%d ns=%d" % (H, ns))


def test_batch_beyond_the_ordered_grid_limit():
    """400 requests x 44 one-tile splits x 4 row blocks (4 drafts x 128 heads)
    = 70400 work items, above the longest-first order's 65536: the natural
    dispatch order; with more than 32 splits the merge is the workgroup-per-row
    one."""
    print("70400 work items", flush=True)
    rng = np.random.default_rng(607)
    prefix = [int(x) for x in rng.integers(1270, 1390, size=400)]
    w = W.small(607, prefix, [4] * 400, 128, pool=600_000)
    import tree_verify_mla_paged_amd as tvm
    from gpu_util import problem_for
    pl = tvm.plan(problem_for(w, num_splits=44))
    assert 400 * pl["max_splits"] * pl["row_blocks"] > 65536 and pl["max_splits"] > 32
    rows = sample_rows(w, 200, seed=607)
    ro, rl = oracle.run(w, rows=rows)
    o, l = run(w, num_splits=44, out_f32=True)
    compare(o.reshape(-1, 512)[rows], l.reshape(-1)[rows], ro, rl, bf16_out=False,
            label="70400 work items")


# ---------------------------------------------- a seeded random sweep, every row

def random_case(seed):
    """A small workload drawn from the parameters the kernels branch on: the
    request count, draft counts (tree shapes), prefix lengths around the
    32-key tile, head counts on both sides of the mask-byte threshold, the
    split count, output type, precise mode, x30 outliers and the three mask /
    key-list forms; capped at ~2M (row, key) pairs so the oracle stays fast."""
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 6))
    H = int(rng.choice([1, 2, 3, 5, 8, 9, 16, 24, 64]))
    ndr = [int(rng.integers(1, 33)) for _ in range(B)]
    pre = [int(rng.choice([0, 1, 7, 31, 32, 33, 100, 500, 1500, 4000])) for _ in range(B)]
    while sum(n * H * (p + n) for n, p in zip(ndr, pre)) > 2_000_000:
        pre = [p // 2 for p in pre]
    form = str(rng.choice(["full", "full", "prefix_visible", "contiguous"]))
    outliers = bool(rng.random() < 0.3)
    ns = int(rng.choice([0, 0, 1, 2, 3, 7, 33]))
    out_f32 = bool(rng.random() < 0.5)
    precise = bool(rng.random() < 0.4)
    w = W.small(5000 + seed, pre, ndr, num_heads=H, outlier_p=0.01 if outliers else 0.0,
                placement="contiguous" if form == "contiguous" else "random")
    if form == "prefix_visible":
        w = W.prefix_visible_form(w)
    elif form == "contiguous":
        w = W.contiguous_prefix_form(w)
    return w, ns, out_f32, precise, outliers, "B=%d H=%d drafts=%s prefixes=%s %s ns=%d f32=%s " \
        "precise=%s outliers=%s" % (B, H, ndr, pre, form, ns, out_f32, precise, outliers)


@pytest.mark.parametrize("seed", range(120))
def test_random_workloads_every_row(seed):
    """Every row of each drawn workload against the oracle.  Precise mode at
    the bar.  The default mode per element within its derived bound,
    (2^-8 + 2^-11) * max|v_d|, which is its guarantee: rows of a request
    without a prefix see only their tree ancestors, and with the mass on a
    few keys the bf16 rounding of their probabilities does not average out
    (the configurations, whose rows see many keys, meet the bar itself in the
    tests above); its mean relative error at the bar, or with outliers within
    the derived 2^-8 + 2^-11."""
    w, ns, out_f32, precise, outliers, desc = random_case(seed)
    print("random %d: %s" % (seed, desc), flush=True)
    kw = {}
    if not precise:
        kw["extra_abs"] = p_rounding_bound(w, precise=False)
        if outliers:
            kw["mean_rel_max"] = 2.0 ** -8 + 2.0 ** -11
    full_check(w, num_splits=ns, out_f32=out_f32, label="random %d" % seed,
               flags=PRECISE if precise else 0, **kw)


def random_medium_case(seed):
    """A workload of several row blocks and many or long splits, drawn like
    random_case (capped at ~40M (row, key) pairs)."""
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 5))
    H = int(rng.choice([8, 16, 32, 64, 128]))
    ndr = [int(rng.integers(8, 65)) for _ in range(B)]
    pre = [int(rng.integers(0, 20001)) for _ in range(B)]
    while sum(n * H * (p + n) for n, p in zip(ndr, pre)) > 40_000_000:
        pre = [p // 2 for p in pre]
    form = str(rng.choice(["full", "full", "prefix_visible", "contiguous"]))
    outliers = bool(rng.random() < 0.3)
    ns = int(rng.choice([0, 0, 5, 40]))
    out_f32 = bool(rng.random() < 0.5)
    precise = bool(rng.random() < 0.4)
    w = W.small(7000 + seed, pre, ndr, num_heads=H, outlier_p=0.01 if outliers else 0.0,
                placement="contiguous" if form == "contiguous" else "random")
    if form == "prefix_visible":
        w = W.prefix_visible_form(w)
    elif form == "contiguous":
        w = W.contiguous_prefix_form(w)
    return w, ns, out_f32, precise, outliers, "B=%d H=%d drafts=%s prefixes=%s %s ns=%d f32=%s " \
        "precise=%s outliers=%s" % (B, H, ndr, pre, form, ns, out_f32, precise, outliers)


@pytest.mark.parametrize("seed", range(16))
def test_random_medium_workloads_every_row(seed):
    """Every row of each drawn workload of several row blocks against the
    oracle, with the bounds of test_random_workloads_every_row."""
    w, ns, out_f32, precise, outliers, desc = random_medium_case(seed)
    print("random medium %d: %s" % (seed, desc), flush=True)
    kw = {}
    if not precise:
        kw["extra_abs"] = p_rounding_bound(w, precise=False)
        if outliers:
            kw["mean_rel_max"] = 2.0 ** -8 + 2.0 ** -11
    full_check(w, num_splits=ns, out_f32=out_f32, label="random medium %d" % seed,
               flags=PRECISE if precise else 0, **kw)
