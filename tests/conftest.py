import os
import sys

import numpy as np
import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_visible():
        return
    skip = pytest.mark.skip(reason="no GPU visible to torch on this host")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def lib():
    """The HIP library, built in-tree when nothing is built yet."""
    from selective_state_space_84_amd import binding, build_lib
    other = os.environ.get("SSM_TEST_LIBRARY")
    if other:  # a differently built copy of the same sources (the sanitizer build)
        binding._lib = binding.load_library(other)
        return binding._lib
    if not os.path.exists(binding.LIB_PATH):
        build_lib.build()
    return binding.load_library()


def floored_rel_err(got, ref) -> float:
    """max_i |g_i - r_i| / max(|r_i|, 0.1 * rms(r)) in float64."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    floor = max(0.1 * rms, np.finfo(np.float64).tiny)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor)))
