import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle.build(force=False)
    return oracle


@pytest.fixture(autouse=True)
def _debug_build_records_nothing(request):
    """With HSTU_DEBUG=1 the binding runs the debug build (bounds tests on the
    kernels' global indices); then every GPU test must leave no failed test."""
    yield
    if os.environ.get("HSTU_DEBUG") != "1" or request.node.get_closest_marker("gpu") is None:
        return
    import ctypes

    import torch

    from generative_recommender_attention_amd import hstu

    if not torch.cuda.is_available():
        return
    sites = ctypes.c_uint32(0)
    assert hstu.library(debug=True).hstu_debug_take(ctypes.byref(sites)) == hstu.HSTU_OK
    assert sites.value == 0, {b: n for b, n in hstu.DEBUG_SITES.items() if sites.value >> b & 1}
