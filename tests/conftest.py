import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity against the oracle")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def large_gemm():
    """The 8192^3 per-channel workload and its exact int32 accumulators from
    the fp64-matmul formulation of the oracle (computed once per session;
    shared by the int8, int32 and f32 full-size checks)."""
    import synth
    from oracle.matmul_f64 import gemm_affine_f64
    d = synth.gemm_large()
    print("computing the 8192^3 reference accumulators", flush=True)
    acc = gemm_affine_f64(d["A"], d["zA"], d["W"], 0)
    return d, acc
