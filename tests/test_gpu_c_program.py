"""The verify call end to end from a C program: tests/c_abi/verify_from_c.c,
built with gcc as C99 against include/treeverify.h and the HIP runtime's C API
only, reads seeded inputs from files, runs tv_check_inputs and tv_verify_attn
on a stream and a workspace of its own, and writes out and lse back; they are
held to the same parity bar against the fp64 oracle as the Python-driven
tests."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import tv_workload as W
from gpu_util import compare

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU present", allow_module_level=True)

import tree_verify_mla_paged_amd as tv  # noqa: E402  (fails loudly if the library is missing)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "verify_from_c.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
LIBDIR = os.path.dirname(tv.LIBRARY_PATH)


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("c_prog") / "verify_from_c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(ROCM, "include"),
                    "-I", os.path.join(ROOT, "include"), SRC,
                    "-L", LIBDIR, "-ltreeverify", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def run_from_c(exe, w, d, num_splits=0, out_f32=False, flags=0):
    flags |= (tv.FLAG_PREFIX_VISIBLE if w.prefix_visible else 0)
    fields = [w.batch, w.num_heads, w.total_q, w.max_q_len, w.max_kv_len, w.num_slots,
              int(w.kv_indices.size), int(w.mask.size), num_splits,
              tv.OUT_F32 if out_f32 else tv.OUT_BF16, flags]
    with open(os.path.join(d, "problem.txt"), "w") as f:
        # 9 significant digits: the same float32 scale the binding passes
        f.write(" ".join(str(int(x)) for x in fields) + " %.9g\n" % np.float32(w.sm_scale))
    for name, arr, dt in (("q", w.q, np.uint16), ("kv", w.kv, np.uint16),
                          ("kv_indices", w.kv_indices, np.int32),
                          ("kv_indptr", w.kv_indptr, np.int32),
                          ("qo_indptr", w.qo_indptr, np.int32), ("mask", w.mask, np.uint8),
                          ("mask_indptr", w.mask_indptr, np.int32)):
        np.ascontiguousarray(arr, dt).tofile(os.path.join(d, name + ".bin"))
    print("C program: %s, splits %d, out_f32 %s, flags %d" % (w.name, num_splits, out_f32, flags),
          flush=True)
    r = subprocess.run([exe, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    n = w.total_q * w.num_heads
    if out_f32:
        o = np.fromfile(os.path.join(d, "out.bin"), np.float32).astype(np.float64)
    else:
        o = W.bf16_to_f32(np.fromfile(os.path.join(d, "out.bin"), np.uint16)).astype(np.float64)
    l = np.fromfile(os.path.join(d, "lse.bin"), np.float32).astype(np.float64)
    assert o.size == n * 512 and l.size == n
    return o.reshape(w.total_q, w.num_heads, 512), l.reshape(w.total_q, w.num_heads)


CASES = [
    ("C1, the live shape: one split, bf16 output", lambda: W.config(1), 0, False, 0),
    ("C2, a batch of 8: partials and the per-row merge", lambda: W.config(2), 0, False, 0),
    ("small, 3 splits, fp32 output, precise", lambda: W.small(41, [700, 90], [7, 12], 16), 3,
     True, tv.FLAG_PRECISE_P),
    ("C1 in the prefix-visible form", lambda: W.prefix_visible_form(W.config(1)), 0, True, 0),
]


@pytest.mark.parametrize("label,make,num_splits,out_f32,flags", CASES, ids=[c[0] for c in CASES])
def test_verify_from_a_c_program(prog, tmp_path, label, make, num_splits, out_f32, flags):
    w = make()
    ro, rl = oracle.run(w)
    o, l = run_from_c(prog, w, str(tmp_path), num_splits, out_f32, flags)
    compare(o, l, ro, rl, bf16_out=not out_f32, label=label)
