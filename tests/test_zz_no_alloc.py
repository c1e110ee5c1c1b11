"""moe_layer_forward_noalloc (the library's static per-GPU workspace, no
allocation) against moe_layer_forward with a caller workspace: two calls in a
row on each layer, the second with fewer tokens, must give bitwise the same
output (the same kernels on the same inputs), and a size whose workspace
exceeds the static array is refused by name."""
import sys

import numpy as np
import pytest

from quantized_moe_expert_softmax_amd import moe, synth

pytestmark = pytest.mark.gpu

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_helpers as gh  # noqa: E402
import parity_cases  # noqa: E402

# (workload or variant, first T, second T): the single-token path, verify
# windows, the 9..32-token path and the grouped GEMM (T > 32), latent layers
CASES = [("decode", 6, 1), ("latent_q8", 6, 1), ("latent_q4", 32, 6), ("tiny", 64, 37),
         ("decode_q4_k", 20, 1), ("multi_tile_q4_0", 300, 40)]


def _workload(name, T):
    if name == "multi_tile_q4_0":
        return parity_cases.variant(**parity_cases.MULTI_TILE[1])
    return synth.WORKLOADS[name].with_tokens(T)


def _noalloc(layer, x, T):
    import torch
    out = torch.full((T, layer.desc.hidden), float("nan"), dtype=torch.float32, device=layer.dev)
    st = torch.cuda.current_stream(layer.dev).cuda_stream
    moe.moe_layer_forward_noalloc(layer.handle, x.data_ptr(), T, layer.router_w.data_ptr(),
                                  layer._ptr(layer.router_b), layer._ptr(layer.groups),
                                  layer.experts.data_ptr(), layer._ptr(layer.D), layer._ptr(layer.U),
                                  layer.k, out.data_ptr(), st)
    return out


@pytest.mark.parametrize("name,T1,T2", CASES)
def test_noalloc_equals_caller_workspace(name, T1, T2):
    import torch
    print(f"\n[noalloc] {name} T={T1} then T={T2}", flush=True)
    w = _workload(name, T1)
    inp = gh.make_inputs(w)
    layer = gh.gpu_layer(w, inp, max_tokens=T1)
    try:
        for T, batch in ((T1, 0), (T2, 1)):
            x = torch.from_numpy(synth.gen_x(w, batch=batch, tokens=T)).to(layer.dev)
            ref = layer.forward(x).clone()
            got = _noalloc(layer, x, T)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), (name, T)
    finally:
        layer.close()


def test_noalloc_refuses_a_workspace_beyond_the_array():
    w = synth.WORKLOADS["prefill"]
    h = moe.moe_layer_create(moe.desc_of(w, max_tokens=2048), 0)
    try:
        need = moe.moe_workspace_bytes(h, 2048)
        assert need > moe.MOE_NOALLOC_WORKSPACE_BYTES
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_layer_forward_noalloc(h, 0, 2048, 0, 0, 0, 0, 0, 0, w.top_k, 0, 0)
        assert ei.value.status == moe.MOE_ENOMEM and "static workspace" in ei.value.message
        # a size that fits is checked as moe_layer_forward checks it (NULL x refused)
        assert moe.moe_workspace_bytes(h, 8) <= moe.MOE_NOALLOC_WORKSPACE_BYTES
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_layer_forward_noalloc(h, 0, 8, 0, 0, 0, 0, 0, 0, w.top_k, 0, 0)
        assert ei.value.status == moe.MOE_EINVAL
    finally:
        moe.moe_layer_destroy(h)
