import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")
    import tests._gpu as g   # progress notes of the GPU tests go through pytest's capture manager
    g.CONFIG = config


@pytest.fixture(scope="session")
def large_oracle():
    """The Large workload's weight (28672x8192 fp32, 0.02 * Student-t(4)) and the oracle's
    quantization of it, computed once for the quantize and GEMM parity tests."""
    import oracle as O
    import synth
    from tests._gpu import note
    note("large weight 28672x8192 fp32: drawing; oracle quantize of 235M elements")
    W = synth.large_weight()
    qo = O.quantize(W.numpy().ravel(), double_quant_on=True)
    return W, qo


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly when they run without a GPU; they are only deselected by -m.
    pass


def pytest_report_header(config):
    return f"repo root: {ROOT}"
