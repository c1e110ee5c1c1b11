"""CPU checks of what the GPU parity cases are meant to exercise: with the
oracle's routing, the multi-tile GEMM cases put more than two 64-token tiles on
every expert, and the 2048-token workloads spread tokens over many tiles."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import parity_cases  # noqa: E402


def _counts(orc, w, inp):
    ids = np.stack([orc.route_token(w, inp["x"][t], inp["router_w"], inp["router_b"],
                                    inp["groups"])[0] for t in range(inp["x"].shape[0])])
    return np.bincount(ids.ravel(), minlength=w.n_experts)


@pytest.mark.parametrize("kw", parity_cases.MULTI_TILE)
def test_multi_tile_cases_fill_three_tiles_per_expert(orc, synth, kw):
    w = parity_cases.variant(**kw)
    inp = synth.gen_layer(w)
    c = _counts(orc, w, inp)
    assert c.min() > 128, c


@pytest.mark.parametrize("name,lo_tiles", [("prefill", 20), ("latent_q8", 20), ("latent_q4", 20)])
def test_2048_token_workloads_span_many_tiles(orc, synth, name, lo_tiles):
    """At T = 2048 experts hold several 64-token tiles: the prefill router's bias spreads
    the counts (BASELINE: roughly 0-400 per expert)."""
    w = synth.WORKLOADS[name].with_tokens(2048)
    inp = dict(x=synth.gen_x(w), router_w=synth.gen_router(w), router_b=synth.gen_bias(w),
               groups=synth.gen_groups(w))
    c = _counts(orc, w, inp)
    assert c.sum() == 2048 * w.top_k
    multi = int((c > 64).sum())
    assert multi >= lo_tiles, (multi, c.max())
    print(name, "experts with more than one 64-token tile:", multi, "largest bucket:", int(c.max()))
