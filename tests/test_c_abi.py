"""The boundary as a C program sees it: include/treeverify.h compiled as C99
(and as C++11) with warnings as errors, a program linked against
libtreeverify.so that calls the host-side entry points, and the structs' layout
under the C compiler against the ctypes binding's.  No GPU: nothing here
launches a kernel or touches device memory."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import tree_verify_mla_paged_amd as tv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "plan_from_c.c")
INC = os.path.join(ROOT, "include")
LIBDIR = os.path.dirname(tv.LIBRARY_PATH)

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("c_abi") / "plan_from_c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", INC, SRC,
                    "-L", LIBDIR, "-ltreeverify", "-Wl,-rpath," + LIBDIR, "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def run(exe, *args):
    r = subprocess.run([exe] + [str(a) for a in args], capture_output=True, text=True, timeout=60)
    return r.returncode, r.stdout


def test_header_compiles_as_cxx():
    subprocess.run(["g++", "-std=c++11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-fsyntax-only", "-x", "c++", "-I", INC, SRC],
                   check=True, capture_output=True, text=True)


def test_argument_errors_from_c(prog):
    rc, out = run(prog, "errors")
    assert rc == 0 and out.strip() == "ok", out


def test_struct_layout_matches_the_binding(prog):
    rc, out = run(prog, "layout")
    assert rc == 0
    seen = {}
    for line in out.splitlines():
        parts = line.split()
        if len(parts) == 3:
            seen[parts[0]] = (int(parts[1]), int(parts[2]))
        else:
            seen[parts[0]] = int(parts[1])
    for cname, cls in (("tv_problem", tv.Problem), ("tv_plan", tv.Plan),
                       ("tv_append_problem", tv.AppendProblem)):
        assert seen[cname] == ctypes.sizeof(cls), cname
        for f, t in cls._fields_:
            assert seen["%s.%s" % (cname, f)] == (getattr(cls, f).offset, ctypes.sizeof(t)), f


# about the shapes of the five workloads (C1 the live shape: 9 drafts, 8 heads,
# 21-key prefix; C2 a batch of 8; C3 32 drafts x 16 heads at a 32k prefix; C4
# 64 drafts x 8 heads at 200k; C5 32 requests x 24 drafts x 64 heads), the
# live shape at a 200k prefix, with every flag and both output types
NAMED = [
    (1, 8, 9, 9, 30, 4096, 30, 270, 0, 0, 0),
    (8, 8, 128, 16, 3898, 65536, 18000, 288000, 0, 0, 0),
    (1, 16, 32, 32, 32800, 200000, 32800, 1049600, 0, 0, 0),
    (1, 16, 32, 32, 32800, 200000, 32800, 1049600, 32, 1, 0),
    (1, 8, 64, 64, 200064, 262144, 200064, 12804096, 0, 0, 0),
    (32, 64, 768, 24, 65560, 524288, 380000, 9000000, 0, 0, 1),
    (1, 8, 9, 9, 200009, 262144, 200009, 81, 0, 0, 2),
    (1, 8, 9, 9, 200009, 262144, 200009, 1800081, 0, 1, 5),
]


def random_problems(n, seed=7):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        B = int(rng.integers(0, 64))
        H = int(rng.choice([1, 2, 3, 8, 9, 16, 64, 128]))
        mq = int(rng.integers(0, 40))
        tq = mq * max(B, 1) + int(rng.integers(0, 5))
        mk = int(rng.integers(0, 300000))
        tk = mk * max(B, 1)
        yield (B, H, tq, mq, mk, 1 << 20, min(tk, 2**31 - 1), min(tk * max(mq, 1), 2**31 - 1),
               int(rng.integers(0, 70)), int(rng.integers(0, 2)), int(rng.integers(0, 8)))


@pytest.mark.parametrize("fields", NAMED + list(random_problems(40)))
def test_plan_from_c_matches_the_binding(prog, fields):
    rc, out = run(prog, *fields)
    assert rc == 0
    vals = [int(x) for x in out.split()]
    p = tv.make_problem(*fields)
    status = tv.lib().tv_get_plan(ctypes.byref(p), ctypes.byref(tv.Plan()))
    assert vals[0] == status
    if status == 0:
        pl = tv.plan(p)
        assert vals[1:6] == [pl["split_keys"], pl["max_splits"], pl["row_blocks"], pl["merge"],
                             pl["workspace_bytes"]]
    assert vals[6] == tv.workspace_bytes(p)
