"""The layer call captured into a HIP graph: every replay must give, bit for bit,
what the same call gives eagerly.  The path launches only kernels (no memset, no
host synchronisation, no allocation), so a serving loop can capture it.  Each
replay runs with other eager layer calls on the same workspace in between, and
alternates two token batches through the captured input buffer."""
import sys

import pytest

from quantized_moe_expert_softmax_amd import synth

pytestmark = pytest.mark.gpu

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_helpers as gh  # noqa: E402


@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 64), ("decode", 1), ("latent_q8", 6),
                                    ("latent_q4", 32), ("latent_q3_k", 1), ("decode_q5_k", 1)])
def test_graph_replay_matches_eager(name, T):
    import torch
    w = synth.Workload(**{**synth.WORKLOADS[name].__dict__, "tokens": T})
    print(f"\n[graph] {name} T={T}", flush=True)
    inp = gh.make_inputs(w)
    layer = gh.gpu_layer(w, inp, max_tokens=T)
    try:
        dev = layer.dev
        xa = torch.from_numpy(synth.gen_x(w, batch=0)).to(dev)
        xb = torch.from_numpy(synth.gen_x(w, batch=1)).to(dev)
        ref_a = layer.forward(xa).clone()
        ref_b = layer.forward(xb).clone()
        torch.cuda.synchronize()
        assert not torch.equal(ref_a, ref_b)

        xin = xa.clone()
        out = torch.full_like(ref_a, float("nan"))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(xin, out=out)
        for rep in range(4):
            src, ref = (xa, ref_a) if rep % 2 == 0 else (xb, ref_b)
            xin.copy_(src)
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"replay {rep} differs from the eager call"
            # eager calls on the same workspace between replays
            other = layer.forward(xb if rep % 2 == 0 else xa)
            torch.cuda.synchronize()
            assert torch.equal(other, ref_b if rep % 2 == 0 else ref_a)
        del g
    finally:
        layer.close()
