import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    # Asked for the GPU tests explicitly (-m gpu), they run and fail loudly
    # if there is no GPU; otherwise they are skipped where none is visible.
    if _has_gpu() or config.getoption("markexpr", "").strip() == "gpu":
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# importing the package's build module would import the package (and load the
# library) first, so load build.py by path instead
def _build_if_missing():
    lib = os.path.join(ROOT, "q8_gemv_sparse_amd", "libq8s.so")
    if os.path.exists(lib):
        return
    import importlib.util
    spec = importlib.util.spec_from_file_location("_q8s_build", os.path.join(ROOT, "q8_gemv_sparse_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build()


_build_if_missing()
