import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _build_if_missing():
    # The package refuses to import without its library; a fresh tree (nothing
    # built yet) gets one build here.  An existing library is used as it is.
    lib = os.path.join(ROOT, "tree_verify_mla_paged_amd", "libtreeverify.so")
    if os.path.exists(lib):
        return
    spec = importlib.util.spec_from_file_location(
        "_tv_hip_build", os.path.join(ROOT, "tree_verify_mla_paged_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build(verbose=True)


_build_if_missing()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
