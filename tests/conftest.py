import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: a CPU test that takes more than a few seconds")


def pytest_collection_modifyitems(config, items):
    # A GPU test collected on a machine without a GPU is skipped, not failed.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def mtl():
    """The binding, with libmtl.so loaded (built first if nothing is built)."""
    import megatron_tensor_transformer_layer_amd as m
    if not os.path.exists(m.LIB_PATH):
        from megatron_tensor_transformer_layer_amd import build
        build.build(verbose=False)
    m.lib()
    return m
