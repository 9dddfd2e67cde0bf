"""Host-side checks of the C ABI: no GPU needed, no kernel is launched.

Every call here fails argument validation before the library touches the HIP
runtime, or is pure host arithmetic (plan, workspace size, status strings).
"""
import ctypes
import os
import re

import pytest

import tree_verify_mla_paged_amd as tv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "treeverify.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = header_functions()
    assert set(declared) == set(tv.EXPORTS)
    for name in declared:
        assert hasattr(tv.lib(), name), name


def test_status_strings():
    for code in range(8):
        assert tv.status_str(code) and tv.status_str(code) != "unknown status"
    assert tv.status_str(99) == "unknown status"


def prob(**kw):
    base = dict(batch=1, num_heads=8, total_q=9, max_q_len=9, max_kv_len=30, num_slots=4096,
                total_kv=30, total_mask=270, num_splits=0, out_dtype=tv.OUT_BF16)
    base.update(kw)
    return tv.make_problem(**base)


def test_plan_live_shape_is_one_split():
    pl = tv.plan(prob())
    assert pl["max_splits"] == 1 and pl["merge"] == 0 and pl["row_blocks"] == 1
    assert pl["split_keys"] % 32 == 0 and pl["split_keys"] >= 30
    # one split, and the split kernel reads the mask bytes itself: no workspace
    assert pl["workspace_bytes"] == 0 == tv.workspace_bytes(prob())
    # at 3 heads a wave's rows span up to 12 drafts: packed visibility words,
    # 9 drafts x 1 tile x 4 bytes, 256-byte aligned
    assert tv.workspace_bytes(prob(num_heads=3)) == 256


def drafts_spanned(n, H):
    """Most draft tokens among the 32 rows of any wave of one request (brute force)."""
    rows = n * H
    return max(len({r // H for r in range(a, min(a + 32, rows))}) for a in range(0, rows, 32))


@pytest.mark.parametrize("H", list(range(1, 21)) + [24, 48, 64, 128])
def test_mask_bytes_mode_follows_the_draft_span(H):
    # packed words (and so workspace) exactly when some wave spans more than 4 drafts
    n = 40
    p = prob(num_heads=H, total_q=n, max_q_len=n, total_kv=30 + n, max_kv_len=30 + n,
             total_mask=n * (30 + n))
    assert tv.plan(p)["max_splits"] == 1
    words = -(-(n * 3 * 4) // 256) * 256
    assert tv.workspace_bytes(p) == (words if drafts_spanned(n, H) > 4 else 0)


def test_plan_explicit_splits_cover_the_longest_request():
    p = prob(batch=1, num_heads=16, total_q=32, max_q_len=32, max_kv_len=32800, num_slots=200000,
             total_kv=32800, total_mask=32 * 32800, num_splits=32)
    pl = tv.plan(p)
    assert pl["split_keys"] % 32 == 0
    assert pl["max_splits"] * pl["split_keys"] >= 32800
    assert (pl["max_splits"] - 1) * pl["split_keys"] < 32800
    assert pl["max_splits"] <= 32 and pl["merge"] == 1 and pl["row_blocks"] == 4
    rows = 32 * 16
    words = 0  # 16 heads: each wave's rows are 2 drafts, the mask is read as bytes

    def parts(out_bytes, lse_bytes):
        return -(-(rows * pl["max_splits"] * 512 * out_bytes) // 256) * 256 + \
            -(-(rows * pl["max_splits"] * lse_bytes) // 256) * 256
    # default: fp16 partial outputs, (lse, scale exponent) per (row, split)
    assert pl["workspace_bytes"] == words + parts(2, 8)
    # precise: fp32 partial outputs, the lse alone
    p.flags = tv.FLAG_PRECISE_P
    assert tv.plan(p)["workspace_bytes"] == words + parts(4, 4)


@pytest.mark.parametrize("k", [1, 2, 4, 7, 16, 64, 128, 1000, 5000])
def test_plan_split_count_bounds(k):
    p = prob(max_kv_len=32777, total_kv=32777, total_mask=9 * 32777, num_splits=k)
    pl = tv.plan(p)
    assert pl["max_splits"] <= k
    assert pl["max_splits"] * pl["split_keys"] >= 32777


def test_plan_heuristic_fills_the_chip():
    # 1 request, 512 rows (4 row blocks), 32800 keys: about one workgroup per CU
    p = prob(num_heads=16, total_q=32, max_q_len=32, max_kv_len=32800, total_kv=32800,
             total_mask=32 * 32800, num_slots=200000)
    pl = tv.plan(p)
    assert 200 <= pl["max_splits"] * pl["row_blocks"] <= 256
    # a batch of unequal requests (32 x 1536 rows, the longest 65560 keys, 259k
    # keys in all): splits near half a compute unit's share, so about two
    # workgroups per compute unit once the longest-first order packs them
    p = prob(batch=32, num_heads=64, total_q=768, max_q_len=24, max_kv_len=65560,
             total_kv=259000, total_mask=24 * 259000, num_slots=262144)
    pl = tv.plan(p)
    share = -(-12 * -(-259000 // 32) // 512)
    assert pl["split_keys"] == 32 * share
    # the dispatch order costs one int32 per work item
    assert tv.workspace_bytes(p) >= 32 * pl["max_splits"] * 12 * 4


def test_plan_of_a_batch_of_equal_requests():
    """8 requests of one token x 128 heads, every one at the 32769-key maximum
    (the key list holds exactly 8 x 32769 entries): one workgroup per compute
    unit, as for a single request, and no dispatch order; one entry fewer and
    the batch counts as unequal, about two per unit."""
    base = dict(batch=8, num_heads=128, total_q=8, max_q_len=1, max_kv_len=32769,
                total_mask=8 * 32769, num_slots=262144)
    pl = tv.plan(prob(total_kv=8 * 32769, **base))
    assert pl["row_blocks"] == 1 and 240 <= 8 * pl["max_splits"] <= 256
    prow = 8 * 128 * pl["max_splits"]
    align = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert pl["workspace_bytes"] == align(prow * 1024) + align(prow * 8)  # no order
    pl2 = tv.plan(prob(total_kv=8 * 32769 - 1, **base))
    assert 8 * pl2["max_splits"] > 256


def test_no_dispatch_order_when_every_work_item_has_a_compute_unit():
    """8 requests of 128 rows, keys up to 3968: at most 256 work items, all
    resident at once, so no longest-first order (and no pack launch)."""
    p = prob(batch=8, num_heads=8, total_q=128, max_q_len=16, max_kv_len=3968,
             total_kv=18600, total_mask=16 * 18600, num_slots=65536)
    pl = tv.plan(p)
    assert 8 * pl["max_splits"] * pl["row_blocks"] <= 256 and pl["merge"]
    prow = 128 * 8 * pl["max_splits"]
    align = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert pl["workspace_bytes"] == align(prow * 1024) + align(prow * 8)


def test_bad_shapes_are_rejected():
    for kw in [dict(num_heads=0), dict(batch=-1), dict(batch=65536), dict(max_kv_len=-1),
               dict(num_splits=-2),
               dict(total_kv=2 ** 31), dict(max_q_len=10, total_q=9)]:
        assert tv.workspace_bytes(prob(**kw)) == 0
        with pytest.raises(tv.TreeVerifyError) as e:
            tv.plan(prob(**kw))
        assert e.value.code == 2
    for kw in [dict(out_dtype=7), dict(flags=8), dict(flags=-1)]:
        with pytest.raises(tv.TreeVerifyError) as e:
            tv.plan(prob(**kw))
        assert e.value.code == 4
    bad = prob()
    bad.reserved = 1
    with pytest.raises(tv.TreeVerifyError) as e:
        tv.plan(bad)
    assert e.value.code == 4
    # the precise-probability flag keeps the split plan; its partial outputs are
    # fp32 instead of scaled fp16, so a merging plan needs more workspace
    pp, pd = tv.plan(prob(flags=tv.FLAG_PRECISE_P)), tv.plan(prob())
    assert {k: v for k, v in pp.items() if k != "workspace_bytes"} == \
        {k: v for k, v in pd.items() if k != "workspace_bytes"}
    many = dict(max_kv_len=40000, total_kv=40000, num_splits=8)
    assert tv.plan(prob(**many))["merge"]
    assert tv.workspace_bytes(prob(flags=tv.FLAG_PRECISE_P, **many)) > \
        tv.workspace_bytes(prob(**many))


def test_prefix_visible_flag_packs_words():
    """The prefix-visible mask form goes through the packed visibility words,
    also where the full form reads the mask bytes directly (16 heads), and keeps
    the split plan."""
    base = dict(num_heads=16, max_kv_len=40000, total_kv=40000)
    full, pv = prob(**base), prob(flags=tv.FLAG_PREFIX_VISIBLE, **base)
    pf, pp = tv.plan(full), tv.plan(pv)
    assert {k: v for k, v in pf.items() if k != "workspace_bytes"} == \
        {k: v for k, v in pp.items() if k != "workspace_bytes"}
    words = full.total_q * ((40000 + 31) // 32) * 4
    assert pp["workspace_bytes"] - pf["workspace_bytes"] == (words + 255) // 256 * 256
    both = prob(flags=tv.FLAG_PREFIX_VISIBLE | tv.FLAG_PRECISE_P, **base)
    assert tv.plan(both)["max_splits"] == pf["max_splits"]


def test_null_pointers_and_short_workspace_fail_before_any_launch():
    p = prob(num_heads=3)  # packed visibility words: 256 bytes of workspace
    fake = 1 << 20  # aligned non-null stand-in; never dereferenced on these paths
    args = [fake] * 7
    # q missing
    assert tv.verify_attn_status(p, 0, *args[1:7], 0.07, fake, fake, fake, 1 << 20) == 1
    # out missing
    assert tv.verify_attn_status(p, *args, 0.07, 0, fake, fake, 1 << 20) == 1
    # workspace missing / too small / misaligned
    assert tv.verify_attn_status(p, *args, 0.07, fake, fake, 0, 0) == 3
    assert tv.verify_attn_status(p, *args, 0.07, fake, fake, fake, 255) == 3
    assert tv.verify_attn_status(p, *args, 0.07, fake, fake, fake + 16, 1 << 20) == 3
    # misaligned kv_buf
    assert tv.verify_attn_status(p, fake, fake + 2, *args[2:7], 0.07, fake, fake, fake,
                                 1 << 20) == 2
    # bad problem
    assert tv.verify_attn_status(prob(num_heads=0), *args, 0.07, fake, fake, fake, 1 << 20) == 2
    # the scale must be positive and finite (the kernels take the row max of the raw scores)
    for bad_scale in (0.0, -0.07, float("nan"), float("inf")):
        assert tv.verify_attn_status(p, *args, bad_scale, fake, fake, fake, 1 << 20) == 2


def test_empty_problem_is_a_no_op():
    p = prob(batch=0, total_q=0, max_q_len=0)
    assert tv.workspace_bytes(p) == 0
    assert tv.verify_attn_status(p, 0, 0, 0, 0, 0, 0, 0, 0.07, 0, 0, 0, 0) == 0
    assert tv.check_inputs(p, 0, 0, 0, 0, stream=0) == (0, -1)


def test_check_inputs_validates_host_arguments_first():
    assert tv.check_inputs(prob(), 0, 0, 0, 0, stream=0)[0] == 1
    assert tv.check_inputs(prob(num_heads=0), 0, 0, 0, 0, stream=0)[0] == 2


def test_problem_struct_layout_matches_header():
    # int32, int32, int64, int32, int32, int64, int64, int64, int32, int32, int32, int32
    assert ctypes.sizeof(tv.Problem) == 64
    assert tv.Problem.num_splits.offset == 48 and tv.Problem.out_dtype.offset == 52
    assert tv.Problem.flags.offset == 56 and tv.Problem.reserved.offset == 60
    assert ctypes.sizeof(tv.Plan) == 24


def aprob(**kw):
    base = dict(batch=1, max_q_len=9, max_kv_len=30, total_q=9, num_slots=4096, total_prefix=21,
                total_kv=30, total_mask=270, flags=0)
    base.update(kw)
    return tv.make_append_problem(**base)


def test_append_problem_layout():
    assert ctypes.sizeof(tv.AppendProblem) == 56
    assert tv.AppendProblem.total_q.offset == 16 and tv.AppendProblem.total_mask.offset == 48


def test_append_draft_argument_errors_before_any_launch():
    fake = 1 << 20  # aligned non-null stand-in; never dereferenced on these paths
    args = [fake] * 11  # draft_kv .. mask_indptr
    # sizes
    for kw, code in [(dict(batch=-1), 2), (dict(batch=65536), 2), (dict(total_kv=2 ** 31), 2),
                     (dict(max_q_len=40), 2),
                     (dict(max_kv_len=1 << 30, max_q_len=9), 2), (dict(flags=1), 4),
                     (dict(flags=8), 4)]:
        assert tv.append_draft_status(aprob(**kw), *args) == code, kw
    # nothing to do: no launch, no pointer needed
    assert tv.append_draft_status(aprob(batch=0), *([0] * 11)) == 0
    # required pointers: prefix_indptr, qo_indptr, kv_indptr, out_cache_loc, ...
    for i in (1, 3, 4, 8, 9):
        a = list(args)
        a[i] = 0
        assert tv.append_draft_status(aprob(), *a) == 1, i
    # parents without a mask; draft rows without a pool
    a = list(args)
    a[9] = 0
    assert tv.append_draft_status(aprob(), *a) == 1
    a = list(args)
    a[6] = 0
    assert tv.append_draft_status(aprob(), *a) == 1
    # misaligned rows
    a = list(args)
    a[0] = fake + 8
    assert tv.append_draft_status(aprob(), *a) == 2


class _FakeDeviceTensor:
    """Tensor metadata only (the binding's checks read nothing else)."""

    def __init__(self, dtype, numel, contiguous=True, cuda=True):
        import torch
        self.dtype = dtype
        self._n = numel
        self._c = contiguous
        self.is_cuda = cuda
        self._es = torch.empty(0, dtype=dtype).element_size()

    def numel(self):
        return self._n

    def element_size(self):
        return self._es

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        raise AssertionError("the checks must fail before any pointer is taken")


def _args(p, **over):
    import torch
    rows = p.total_q * p.num_heads
    a = dict(q=_FakeDeviceTensor(torch.bfloat16, rows * 576),
             kv_buf=_FakeDeviceTensor(torch.bfloat16, p.num_slots * 576),
             kv_indices=_FakeDeviceTensor(torch.int32, p.total_kv),
             kv_indptr=_FakeDeviceTensor(torch.int32, p.batch + 1),
             qo_indptr=_FakeDeviceTensor(torch.int32, p.batch + 1),
             mask=_FakeDeviceTensor(torch.uint8, p.total_mask),
             mask_indptr=_FakeDeviceTensor(torch.int32, p.batch + 1),
             out=_FakeDeviceTensor(torch.bfloat16, rows * 512),
             lse=_FakeDeviceTensor(torch.float32, rows))
    a.update(over)
    return a


def test_binding_checks_tensor_arguments_before_the_call():
    """Wrong dtype, non-contiguous, host-resident or undersized tensors are
    refused by the binding before any pointer reaches the C ABI."""
    import torch
    p = prob()
    rows = 9 * 8
    bad = [dict(q=_FakeDeviceTensor(torch.float32, rows * 576)),
           dict(q=_FakeDeviceTensor(torch.bfloat16, rows * 576 - 1)),
           dict(kv_buf=_FakeDeviceTensor(torch.bfloat16, 4096 * 576, contiguous=False)),
           dict(kv_buf=_FakeDeviceTensor(torch.bfloat16, 4096 * 576, cuda=False)),
           dict(kv_indices=_FakeDeviceTensor(torch.int64, 30)),
           dict(kv_indices=_FakeDeviceTensor(torch.int32, 29)),
           dict(mask=_FakeDeviceTensor(torch.uint8, 269)),
           dict(mask_indptr=_FakeDeviceTensor(torch.int32, 1)),
           dict(out=_FakeDeviceTensor(torch.float32, rows * 512)),   # bf16 problem
           dict(out=_FakeDeviceTensor(torch.bfloat16, rows * 512 - 8)),
           dict(lse=_FakeDeviceTensor(torch.bfloat16, rows))]
    for over in bad:
        a = _args(p, **over)
        with pytest.raises(ValueError):
            tv.verify_attn(p, a["q"], a["kv_buf"], a["kv_indices"], a["kv_indptr"],
                           a["qo_indptr"], a["mask"], a["mask_indptr"], 0.07, a["out"], a["lse"],
                           None, 0, stream=0)
    # an fp32-output problem wants 4-byte out elements
    pf = prob(out_dtype=tv.OUT_F32)
    a = _args(pf, out=_FakeDeviceTensor(torch.bfloat16, rows * 512))
    with pytest.raises(ValueError):
        tv.verify_attn(pf, a["q"], a["kv_buf"], a["kv_indices"], a["kv_indptr"], a["qo_indptr"],
                       a["mask"], a["mask_indptr"], 0.07, a["out"], a["lse"], None, 0, stream=0)


def test_static_entry_point_rejects_plans_beyond_its_scratch():
    """tv_verify_attn_static takes its workspace from a fixed device array: a
    plan needing more returns TV_ERR_WORKSPACE before anything is enqueued (the
    fake pointers are never touched); one that needs none, or a bad problem,
    is decided by the same checks as tv_verify_attn."""
    fake = 1 << 20
    args = [fake] * 7
    # 32 requests x 24 drafts x 64 heads over prefixes up to 65k keys: hundreds of MB
    big = prob(batch=32, num_heads=64, total_q=768, max_q_len=24, max_kv_len=65560,
               total_kv=377000, total_mask=24 * 377000, num_slots=524288)
    assert tv.workspace_bytes(big) > tv.STATIC_SCRATCH_BYTES
    assert tv.verify_attn_static_status(big, *args, 0.07, fake, fake) == 3
    # 32 drafts x 16 heads over 32800 keys: 32 MB of partials, within the array
    c3 = prob(num_heads=16, total_q=32, max_q_len=32, max_kv_len=32800, total_kv=32800,
              total_mask=32 * 32800, num_slots=200000)
    assert 0 < tv.workspace_bytes(c3) <= tv.STATIC_SCRATCH_BYTES
    # the problem's own checks come first
    assert tv.verify_attn_static_status(prob(num_heads=0), *args, 0.07, fake, fake) == 2
    assert tv.verify_attn_static_status(prob(), *args, float("nan"), fake, fake) == 2
    p0 = prob(batch=0, total_q=0, max_q_len=0)
    assert tv.verify_attn_static_status(p0, 0, 0, 0, 0, 0, 0, 0, 0.07, 0, 0) == 0


def test_build_refuses_kernels_that_spill():
    """The build reads hipcc's per-kernel resource remarks and refuses a kernel
    with scratch or spilled VGPRs (every build runs that check): the parser on a
    sample with one clean and one spilling kernel."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "tv_build", os.path.join(ROOT, "tree_verify_mla_paged_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    sample = "\n".join([
        "a.hip:1:1: remark: Function Name: _ZN2tv1kE [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 150 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: _ZN2tv1jE [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 832 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert b.resource_usage(sample) == [("_ZN2tv1kE", 0, 0), ("_ZN2tv1jE", 832, 12)]
    assert b.resource_usage("") == []
