"""The marshaling step on the GPU (tv_append_draft through the C ABI) against
its oracle (oracle/marshal.py): key lists, indptrs, mask bytes and pool rows
must match bit for bit; the verify call on what the step built must then match
the attention oracle."""
import numpy as np
import pytest

import oracle
import oracle.marshal as M
import tv_workload as W
from gpu_util import compare, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU present", allow_module_level=True)

import tree_verify_mla_paged_amd as tv  # noqa: E402  (fails loudly if the library is missing)

SENT_I32 = -7
SENT_U8 = 0xEE


def dev(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    if a.size == 0:
        a = np.zeros(1, dtype=dtype)
    return torch.from_numpy(a.view(np.int16) if dtype == np.uint16 else a).to("cuda")


def gpu_append(w, prefix_visible=False, with_rows=True, with_parents=True, kv_cap=None,
               mask_cap=None, guard=64, parents=None):
    """Runs tv_append_draft on the pieces of workload w; returns host arrays
    (pool, kv_indices incl. guard, kv_indptr, mask incl. guard, mask_indptr)."""
    x = W.marshal_inputs(w)
    if parents is not None:
        x["parents"] = parents
    B = w.batch
    need_kv = int(w.kv_lens.sum())
    n, L = w.q_lens, w.kv_lens
    need_mask = int((n * (n if prefix_visible else L)).sum())
    kv_cap = need_kv if kv_cap is None else kv_cap
    mask_cap = need_mask if mask_cap is None else mask_cap
    pool = dev(x["kv_buf"], np.uint16)
    t = dict(draft_kv=dev(x["draft_kv"], np.uint16), out_cache_loc=dev(x["out_cache_loc"], np.int32),
             prefix_indices=dev(x["prefix_indices"], np.int32),
             prefix_indptr=dev(x["prefix_indptr"], np.int32), qo_indptr=dev(x["qo_indptr"], np.int32),
             parents=dev(x["parents"], np.int32))
    kv_indices = torch.full((kv_cap + guard,), SENT_I32, dtype=torch.int32, device="cuda")
    kv_indptr = torch.full((B + 1,), SENT_I32, dtype=torch.int32, device="cuda")
    mask = torch.full((mask_cap + guard,), SENT_U8, dtype=torch.uint8, device="cuda")
    mask_indptr = torch.full((B + 1,), SENT_I32, dtype=torch.int32, device="cuda")
    p = tv.make_append_problem(B, w.max_q_len, w.max_kv_len, w.total_q, w.num_slots,
                               int(x["prefix_indices"].size), kv_cap, mask_cap,
                               tv.FLAG_PREFIX_VISIBLE if prefix_visible else 0)
    tv.append_draft(p, t["draft_kv"] if with_rows else None, t["out_cache_loc"],
                    t["prefix_indices"], t["prefix_indptr"], t["qo_indptr"],
                    t["parents"] if with_parents else None, pool, kv_indices, kv_indptr,
                    mask, mask_indptr)
    torch.cuda.synchronize()
    return (x, pool.cpu().numpy().view(np.uint16), kv_indices.cpu().numpy(),
            kv_indptr.cpu().numpy(), mask.cpu().numpy(), mask_indptr.cpu().numpy())


def expected(x, prefix_visible=False):
    return M.append_draft(x["kv_buf"], x["draft_kv"], x["out_cache_loc"], x["prefix_indices"],
                          x["prefix_indptr"], x["qo_indptr"], x["parents"],
                          prefix_visible=prefix_visible)


WORKLOADS = {
    "C1": lambda: W.config(1),
    "C2": lambda: W.config(2),
    "batch-with-empty": lambda: W.small(501, [300, 7, 0, 95, 0], [3, 2, 0, 6, 1], 2),
    "chain": lambda: W.chain(502, [1000, 3], 40, 1),
    "C3": lambda: W.config(3),
    "C5": lambda: W.config(5),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("prefix_visible", [False, True])
def test_append_matches_oracle(name, prefix_visible):
    print("append %s prefix_visible=%s" % (name, prefix_visible), flush=True)
    w = WORKLOADS[name]()
    x, pool, ki, kp, m, mp = gpu_append(w, prefix_visible=prefix_visible)
    ekv, eki, ekp, em, emp = expected(x, prefix_visible)
    nk, nm = eki.size, em.size
    assert np.array_equal(kp, ekp)
    assert np.array_equal(ki[:nk], eki) and np.all(ki[nk:] == SENT_I32)
    assert np.array_equal(mp, emp)
    assert np.array_equal(m[:nm], em) and np.all(m[nm:] == SENT_U8)
    assert np.array_equal(pool, ekv)
    # and the generator's own layout
    assert np.array_equal(ki[:nk], w.kv_indices)
    assert np.array_equal(pool, w.kv)


@pytest.mark.parametrize("prefix_visible", [False, True])
def test_verify_on_what_append_built(prefix_visible):
    """The pages' parity failure was in this step; the whole chain must match."""
    print("append + verify prefix_visible=%s" % prefix_visible, flush=True)
    w = W.config(2)
    x, pool, ki, kp, m, mp = gpu_append(w, prefix_visible=prefix_visible, guard=0)
    import dataclasses
    built = dataclasses.replace(w, kv=pool, kv_indices=ki, kv_indptr=kp, mask=m, mask_indptr=mp,
                                prefix_visible=prefix_visible)
    o, l = run(built, out_f32=True)
    ro, rl = oracle.run(w)
    compare(o, l, ro, rl, bf16_out=False, label="append+verify")


def test_append_stores_stay_within_capacities():
    """Capacities below what the indptrs need: the stores stop at them."""
    print("append with short capacities", flush=True)
    w = W.config(2)
    need_kv = int(w.kv_lens.sum())
    need_mask = int(w.mask.size)
    x, pool, ki, kp, m, mp = gpu_append(w, kv_cap=need_kv - 5, mask_cap=need_mask - 7, guard=64)
    ekv, eki, ekp, em, emp = expected(x)
    assert np.array_equal(ki[:need_kv - 5], eki[:need_kv - 5]) and np.all(ki[need_kv - 5:] == SENT_I32)
    assert np.array_equal(m[:need_mask - 7], em[:need_mask - 7]) and np.all(m[need_mask - 7:] == SENT_U8)
    assert np.array_equal(kp, ekp) and np.array_equal(mp, emp)


def test_append_without_rows_or_mask():
    """draft_kv NULL leaves the pool alone; parents NULL writes no mask byte
    (mask_indptr is still the running sum of the blocks)."""
    print("append without rows or parents", flush=True)
    w = W.config(2)
    x, pool, ki, kp, m, mp = gpu_append(w, with_rows=False, with_parents=False)
    ekv, eki, ekp, em, emp = expected(x)
    assert np.array_equal(pool, x["kv_buf"])
    assert np.array_equal(ki[:eki.size], eki) and np.array_equal(kp, ekp)
    assert np.all(m == SENT_U8) and np.array_equal(mp, emp)


def test_append_parent_out_of_order_ends_the_walk():
    """A parent link that does not point to an earlier draft ends that row's
    ancestor walk as a root would: the row sees its path up to the bad link."""
    print("append with a parent out of order", flush=True)
    w = W.chain(503, [10], 6, 1)
    parents = np.array([-1, 0, 1, 3, 3, 4], dtype=np.int32)  # draft 3 names itself
    x, pool, ki, kp, m, mp = gpu_append(w, parents=parents, guard=0)
    rows = m.reshape(6, 16)
    assert np.all(rows[:, :10] == 1)
    expect = np.array([[1, 0, 0, 0, 0, 0], [1, 1, 0, 0, 0, 0], [1, 1, 1, 0, 0, 0],
                       [0, 0, 0, 1, 0, 0], [0, 0, 0, 1, 1, 0], [0, 0, 0, 1, 1, 1]], np.uint8)
    assert np.array_equal(rows[:, 10:], expect)


def test_append_and_verify_captured_in_one_graph():
    """Both entry points only enqueue kernels: the marshaling step and the
    verify call captured together in one HIP graph replay to the eager result,
    with eager work between replays, and follow new draft rows."""
    from gpu_util import GpuCall
    print("append + verify in one graph", flush=True)
    w = W.config(2)
    x = W.marshal_inputs(w)
    B = w.batch
    pieces = dict(draft_kv=dev(x["draft_kv"], np.uint16), out_cache_loc=dev(x["out_cache_loc"], np.int32),
                  prefix_indices=dev(x["prefix_indices"], np.int32),
                  prefix_indptr=dev(x["prefix_indptr"], np.int32),
                  parents=dev(x["parents"], np.int32))
    t = dict(q=dev(w.q, np.uint16), kv=dev(x["kv_buf"], np.uint16),
             kv_indices=torch.full((w.kv_indices.size,), SENT_I32, dtype=torch.int32, device="cuda"),
             kv_indptr=torch.full((B + 1,), SENT_I32, dtype=torch.int32, device="cuda"),
             qo_indptr=dev(w.qo_indptr, np.int32),
             mask=torch.full((w.mask.size,), SENT_U8, dtype=torch.uint8, device="cuda"),
             mask_indptr=torch.full((B + 1,), SENT_I32, dtype=torch.int32, device="cuda"))
    g = GpuCall(w, out_f32=True, tensors=t)
    ap = tv.make_append_problem(B, w.max_q_len, w.max_kv_len, w.total_q, w.num_slots,
                                int(x["prefix_indices"].size), int(w.kv_indices.size),
                                int(w.mask.size))

    def step(stream):
        tv.append_draft(ap, pieces["draft_kv"], pieces["out_cache_loc"], pieces["prefix_indices"],
                        pieces["prefix_indptr"], t["qo_indptr"], pieces["parents"], t["kv"],
                        t["kv_indices"], t["kv_indptr"], t["mask"], t["mask_indptr"],
                        stream=stream)
        g.call(stream=stream)

    step(None)
    o, l = g.result()
    ro, rl = oracle.run(w)
    compare(o, l, ro, rl, bf16_out=False, label="eager append+verify")
    eager = g.out_bits().copy()
    eager_l = g.lse.cpu().numpy().copy()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        step(stream)
    for rep in range(3):
        g.out.fill_(0)
        t["kv_indices"].fill_(SENT_I32)
        t["mask"].fill_(SENT_U8)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(g.out_bits(), eager), rep
        assert np.array_equal(g.lse.cpu().numpy(), eager_l), rep
    # new draft rows: the replay writes them into the pool and attends to them
    rng = np.random.default_rng(78)
    new_rows = W.bf16_round(rng.standard_normal(x["draft_kv"].shape, dtype=np.float32))
    pieces["draft_kv"].copy_(torch.from_numpy(new_rows.view(np.int16)).cuda())
    graph.replay()
    torch.cuda.synchronize()
    kv2 = w.kv.copy()
    kv2[x["out_cache_loc"]] = new_rows
    import dataclasses
    w2 = dataclasses.replace(w, kv=kv2)
    o, l = g.result()
    ro, rl = oracle.run(w2)
    compare(o, l, ro, rl, bf16_out=False, label="replay with new draft rows")


def test_append_many_requests_carries_across_scan_chunks():
    """3000 requests: the indptr scan runs over twelve 256-request chunks, each
    carrying the running totals of the ones before."""
    print("append 3000 requests", flush=True)
    rng = np.random.default_rng(504)
    prefix = [int(x) for x in rng.integers(0, 40, size=3000)]
    drafts = [int(x) for x in rng.integers(0, 4, size=3000)]
    w = W.small(504, prefix, drafts, 1, max_branch=2)
    for pv in (False, True):
        x, pool, ki, kp, m, mp = gpu_append(w, prefix_visible=pv, guard=0)
        ekv, eki, ekp, em, emp = expected(x, pv)
        assert np.array_equal(kp, ekp) and np.array_equal(mp, emp)
        assert np.array_equal(ki, eki) and np.array_equal(m, em)
        assert np.array_equal(pool, ekv)
