"""tv_verify_attn_static (no workspace argument: the library's static device
scratch array) against tv_verify_attn with a caller workspace, on the same
inputs: bit-identical outputs and LSEs.  Several calls in a row share the one
array, each later one with a smaller problem, so each must overwrite what it
reads and ignore what the previous call left behind."""
import numpy as np
import pytest

import tv_workload as W
from gpu_util import GpuCall

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU present", allow_module_level=True)

import tree_verify_mla_paged_amd as tv  # noqa: E402  (fails loudly if the library is missing)


def static_bits(g: GpuCall):
    out = torch.full_like(g.out, float("nan"))
    lse = torch.full_like(g.lse, float("nan"))
    t = g.t
    tv.verify_attn_static(g.p, t["q"], t["kv"], t["kv_indices"], t["kv_indptr"], t["qo_indptr"],
                          t["mask"], t["mask_indptr"], float(g.w.sm_scale), out, lse)
    torch.cuda.synchronize()
    bits = out.view(torch.int32 if g.out_f32 else torch.int16).cpu().numpy()
    return bits, lse.cpu().numpy().view(np.int32)


def test_static_scratch_matches_the_workspace_entry_point():
    cases = [
        # 512 rows x 61 splits of fp32 partials (precise): 61 MiB, near the limit
        ("C3 precise", W.config(3), dict(flags=tv.FLAG_PRECISE_P)),
        # the same request with fp16 partials: 32 MB
        ("C3", W.config(3), dict()),
        # unequal requests at 48 heads: the longest-first dispatch order
        ("order", W.small(251, [3000, 10, 700, 0, 1500, 64, 2500], [5, 3, 6, 2, 4, 1, 6],
                          num_heads=48), dict(num_splits=5)),
        # 3 heads: packed visibility words; 3 splits
        ("words", W.small(801, [900, 37, 2500], [7, 3, 12], num_heads=3),
         dict(num_splits=3, out_f32=True)),
    ]
    prev = None
    for name, w, kw in cases:
        print("static scratch: %s" % name, flush=True)
        g = GpuCall(w, **kw)
        need = tv.workspace_bytes(g.p)
        assert 0 < need <= tv.STATIC_SCRATCH_BYTES, (name, need)
        if prev is not None:
            assert need < prev, "each later call must be smaller"
        prev = need
        g.call()
        ref = g.out_bits().copy()
        ref_l = g.lse.cpu().numpy().view(np.int32).copy()
        o, l = static_bits(g)
        assert np.array_equal(o, ref), name
        assert np.array_equal(l, ref_l), name
        # twice in a row on the same inputs: the array keeps the last call's
        # contents, which the next call must not depend on
        o, l = static_bits(g)
        assert np.array_equal(o, ref), name
