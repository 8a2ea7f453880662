"""The acceptance checks themselves (CPU): the vectorised routing check used for the largest token counts agrees
with the per-token check, and both reject a planted wrong expert and a planted weight error."""
import numpy as np
import pytest

import oracle
from expert_ffn_canvas_amd import synth
from tests import parity_util as pu


@pytest.fixture(scope="module")
def routed():
    wl = synth.small_workload(T=3000, E=16, K=8, D=128, F=64, bias="zipf", seed=3)
    inp = synth.make_inputs(wl)
    xn, wn = pu.host(inp["x"]), pu.oracle_weights(inp["layers"][0])
    orc = oracle.route(xn, wn["router_w"], wn["router_gamma"], wn.get("router_bias"), 8, synth.RMS_EPS)
    return orc, orc["idx"].copy(), orc["w"].astype(np.float32)


def test_vectorised_routing_check_agrees(routed):
    orc, gi, gw = routed
    assert pu.check_routing(gi, gw, orc, 8, 3000) == pu.check_routing_many(gi, gw, orc, 8, 3000)


@pytest.mark.parametrize("check", [pu.check_routing, pu.check_routing_many])
def test_routing_checks_reject_planted_errors(routed, check):
    orc, gi, gw = routed
    t = int(np.nonzero(orc["gap"] >= pu.TIE)[0][5])
    bad = gi.copy()
    bad[t, 7] = [e for e in range(16) if e not in bad[t]][0]  # a clear token given an expert outside its set
    with pytest.raises(AssertionError):
        check(bad, gw, orc, 8, 3000)
    bw = gw.copy()
    bw[t, 2] += 1e-4  # a routing weight 10x the weight tolerance off
    with pytest.raises(AssertionError):
        check(gi, bw, orc, 8, 3000)
