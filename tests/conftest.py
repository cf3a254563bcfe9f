import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


@pytest.fixture(scope="session")
def big():
    """Device weights of the full-size layer (d = 7168, f = 2048, 896 experts,
    2 shared), built once and shared by every GPU test module."""
    import torch
    import gen
    import gen.device
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cfg = gen.get("decode_b1")
    print("building full-size layer weights on device", flush=True)
    wl = gen.device.build(cfg)
    torch.cuda.synchronize()
    return wl
