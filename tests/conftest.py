import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (test infrastructure); built with gcc if nothing is built."""
    from oracle import oracle as oracle_mod
    if not os.path.exists(oracle_mod.DEFAULT_LIB):
        from oracle import build as oracle_build
        oracle_build.build()
    return oracle_mod.default()


@pytest.fixture(scope="session")
def gqa_t8192_reference(orc):
    """The 8192-token grouped-query workload (B=1, Hq=16, Hkv=4, d=64, seed 4) with an
    upstream gradient dO drawn after Q, K, V, and the oracle's whole O, LSE, dQ, dK
    and dV for it, computed once per session (the full materialised definition in
    double: tens of seconds on the host cores)."""
    import synthetic_inputs as si
    c = si.CAUSAL_WORKLOADS["gqa_b1_hq16_hkv4_t8192_d64"]
    host = si.causal_inputs(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["seed"], with_do=True)
    scale = 1.0 / 8.0
    ro, rlse = orc.causal_fwd(host["q"], host["k"], host["v"], scale)
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"], scale)
    return {"host": host, "scale": scale, "o": ro, "lse": rlse, "dq": rdq, "dk": rdk, "dv": rdv}
