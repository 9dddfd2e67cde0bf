"""Host logic of bench.py (no GPU): workload selection, the algorithmic bytes
and flops that the roofline divides by, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np

import tv_workload as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_counts_by_hand():
    """C1: 9 drafts after a 21-token prefix, 8 heads.  Visible pairs = 9 * 21 +
    sum of tree depths (ancestors + self); flops = 2 * (576 + 512) per visible
    (row, key) pair and head; bytes = keys * 1152 + q + bf16 out + lse +
    4-byte slots + mask bytes."""
    w = W.config(1)
    depth = sum(len(W.ancestors_and_self(w.parents[0], i)) for i in range(9))
    pairs = 9 * 21 + depth
    kv, total, flops = bench.algorithmic(w)
    assert kv == 30 * 1152
    assert flops == 2.0 * 1088 * 8 * pairs
    assert total == 30 * 1152 + 9 * 8 * 1152 + 9 * 8 * 1024 + 9 * 8 * 4 + 30 * 4 + 270


def test_prefix_visible_workload_keeps_the_visible_pairs():
    w, _, _ = bench.workload("3", poison=False)
    pv, desc, _ = bench.workload("3", poison=False, prefix_visible=True)
    assert pv.prefix_visible and "prefix-visible" in desc
    assert pv.visible_pairs() == w.visible_pairs()
    assert pv.mask.size == 32 * 32
    _, tot_w, fl_w = bench.algorithmic(w)
    _, tot_pv, fl_pv = bench.algorithmic(pv)
    assert fl_w == fl_pv and tot_w - tot_pv == w.mask.size - pv.mask.size


def test_extra_workloads():
    d, desc, splits = bench.workload("D", poison=False)
    assert d.batch == 8 and d.num_heads == 128 and list(d.q_lens) == [1] * 8
    assert list(d.kv_lens) == [32769] * 8 and splits is None and desc.startswith("D:")
    k, _, _ = bench.workload("K", poison=False)
    m = k.mask.reshape(16, 32784)
    assert np.all(m[:, :32768] == 1)
    assert np.array_equal(m[:, 32768:], np.tril(np.ones((16, 16), np.uint8)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_contiguous_prefix_workload_and_counts():
    """--contiguous-prefix: contiguous placement, each prefix passed by its first
    slot; the expanded key list is the placement's, and the index bytes the
    call reads are one entry per prefix plus one per draft."""
    w, desc, _ = bench.workload("S1", poison=False, contiguous_prefix=True)
    full, _, _ = bench.workload("S1", poison=False, placement="contiguous")
    assert w.contiguous_prefix and "contiguous" in desc
    assert np.array_equal(bench.key_slots(w), full.kv_indices)
    assert bench.index_entries(w) == 1 + 9 and bench.index_entries(full) == 32768 + 9
    _, tot_c, fl_c = bench.algorithmic(w)
    _, tot_f, fl_f = bench.algorithmic(full)
    assert fl_c == fl_f and tot_f - tot_c == 4 * 32767


def test_traffic_key_ignores_comments_not_code():
    """The counter summary is keyed on the split kernel's code: a comment or
    layout change keeps the key, a changed token does not."""
    a = "int f(int x) {  // one\n  return x + 1;  /* two\n lines */\n}\n"
    b = "int f(int x) {\n  // another comment\n  return x + 1;\n}"
    c = "int f(int x) {\n  return x + 2;\n}"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert len(bench.source_hash()) == 16
