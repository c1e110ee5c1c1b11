"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs.  Bit-exact: routing ids (near-tie tokens: a valid top-k), Q8_1(x)
bytes, every integer block sum of the tap tokens (gate/up on the GPU's expert
input, down on the GPU's own requantised h, D/U), and each requantisation of a
GPU intermediate.  Q8_1 vectors of z, h and y_lat: equal to the oracle's except
for flips (a code moved by 1 where the oracle's value lies within 2e-3 of a .5
boundary), at most 1e-4 of the codes.  Layer output: within 2e-3 of the oracle's
output RMS on every token without a flip; a token with a flip within 1e-5 of the
oracle evaluated on the GPU's ids and Q8_1 vectors."""
import dataclasses
import sys

import numpy as np
import pytest

from quantized_moe_expert_softmax_amd import moe, synth

pytestmark = pytest.mark.gpu

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_helpers as gh  # noqa: E402
import parity_cases  # noqa: E402

_cache = {}


def _layer(name, max_tokens):
    w = synth.WORKLOADS[name]
    key = (name, max_tokens)
    if key not in _cache:
        for k in list(_cache):
            _cache.pop(k)[0].close()
        inp = gh.make_inputs(w)
        _cache[key] = (gh.gpu_layer(w, inp, max_tokens=max_tokens), inp)
    return _cache[key]


def _report(name, T, rep):
    rep = {k: v for k, v in rep.items() if not k.startswith("_")}
    print(f"\n[parity] {name} T={T}: {rep}", flush=True)


@pytest.mark.parametrize("T", [4, 1, 37, 64])
def test_tiny(T):
    layer, inp = _layer("tiny", 64)
    rep = gh.check_case(synth.WORKLOADS["tiny"], T, tap_tokens=T, layer=layer, inp=inp)
    _report("tiny", T, rep)


@pytest.mark.parametrize("T", [1, 6])
def test_decode(T):
    layer, inp = _layer("decode", 6)
    rep = gh.check_case(synth.WORKLOADS["decode"], T, tap_tokens=min(T, 2), layer=layer, inp=inp)
    _report("decode", T, rep)


@pytest.mark.parametrize("T", [1, 6])
def test_latent_q8(T):
    layer, inp = _layer("latent_q8", 6)
    rep = gh.check_case(synth.WORKLOADS["latent_q8"], T, tap_tokens=min(T, 2), layer=layer, inp=inp)
    _report("latent_q8", T, rep)


@pytest.mark.parametrize("T", [1, 32])
def test_latent_q4(T):
    layer, inp = _layer("latent_q4", 32)
    rep = gh.check_case(synth.WORKLOADS["latent_q4"], T, tap_tokens=2, layer=layer, inp=inp)
    _report("latent_q4", T, rep)


def test_prefill_every_token():
    """The prefill layer at its measured size: ids, weights, Q8_1 vectors and the
    output of all 2048 tokens against the oracle (run on the host's cores)."""
    layer, inp = _layer("prefill", 2048)
    rep = gh.check_case(synth.WORKLOADS["prefill"], 2048, tap_tokens=2, layer=layer, inp=inp)
    _report("prefill", 2048, rep)


@pytest.mark.parametrize("name", ["latent_q8", "latent_q4"])
def test_latent_prefill_every_token(name):
    """Latent prefill at the size it is measured (2048 tokens, about 64 per expert, so
    every expert runs several 64-token tiles): every token against the oracle."""
    layer, inp = _layer(name, 2048)
    rep = gh.check_case(synth.WORKLOADS[name], 2048, tap_tokens=2, layer=layer, inp=inp)
    _report(name, 2048, rep)


# --------------------------------------------------------------- small variants
_variant = parity_cases.variant


@pytest.mark.parametrize("kw", [
    dict(expert_fmt=synth.Q4_0),
    dict(top_k=8),                                   # k = E: full softmax
    dict(n_experts=16, top_k=3, n_groups=4, topk_groups=2),
    dict(latent=256, n_experts=16, top_k=4, n_groups=4, topk_groups=2),
    dict(latent=256, expert_fmt=synth.Q4_0, n_experts=16, top_k=4),
    dict(n_experts=1, top_k=1),
    dict(bias=True, tokens=40),
    dict(hidden=1280, n_ff=768, tokens=9),
    # one token: routed in the gate/up kernel's prologue
    dict(bias=True, tokens=1),
    dict(bias=True, n_experts=16, top_k=3, n_groups=4, topk_groups=2, tokens=1),
    dict(n_experts=1, top_k=1, tokens=1),
    dict(top_k=8, tokens=1),
])
def test_variants(kw):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tap_tokens=w.tokens)
    _report(str(kw), w.tokens, rep)


# many-token path (grouped matrix-core GEMM): several row tiles, ragged token
# tiles, both weight formats, latent D/U, group-limited routing
@pytest.mark.parametrize("kw,sample,taps", [
    (dict(expert_fmt=synth.Q4_0, tokens=100), None, 4),
    (dict(top_k=8, tokens=65), None, 3),
    (dict(n_experts=1, top_k=1, tokens=129), None, 3),
    (dict(latent=256, n_experts=16, top_k=4, n_groups=4, topk_groups=2, tokens=70), None, 3),
    (dict(latent=256, expert_fmt=synth.Q4_0, n_experts=16, top_k=4, tokens=97), None, 3),
    (dict(hidden=1280, n_ff=768, n_experts=32, top_k=4, tokens=300, bias=True),
     None, 2),
    (dict(expert_fmt=synth.Q5_1, tokens=100), None, 4),
    (dict(expert_fmt=synth.Q5_1, hidden=1280, n_ff=768, n_experts=32, top_k=4, tokens=300),
     None, 2),
    (dict(expert_fmt=synth.Q4_K, tokens=100), None, 4),
    (dict(expert_fmt=synth.Q5_K, hidden=1280, n_ff=768, n_experts=32, top_k=4, tokens=300),
     None, 2),
    (dict(expert_fmt=synth.Q3_K, tokens=100), None, 4),
    (dict(expert_fmt=synth.Q3_K, hidden=1280, n_ff=768, n_experts=32, top_k=4, tokens=300,
          bias=True), None, 2),
])
def test_gemm_variants(kw, sample, taps):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tokens=sample, tap_tokens=taps)
    _report("gemm " + str(kw), w.tokens, rep)


# every expert format on the grouped GEMM with buckets of more than 128 tokens
# (4 experts, top-2, 300 tokens: 150 per expert on average), so each expert runs
# two full 64-token tiles and a ragged third; integer sums tapped on every token
@pytest.mark.parametrize("kw", parity_cases.MULTI_TILE)
def test_multi_tile_gemm_every_format(kw):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tap_tokens=w.tokens)
    _report("multi-tile " + str(kw), w.tokens, rep)


@pytest.mark.parametrize("name,T", [("latent_q8", 48), ("latent_q4", 40)])
def test_latent_gemm(name, T):
    layer, inp = _layer(name, T)
    rep = gh.check_case(synth.WORKLOADS[name], T, tap_tokens=2, layer=layer, inp=inp)
    _report(name, T, rep)


# latent D/U in Q4_0 (the Q4 choice of the D/U projections): the single-token
# path, a decode window, the 9..32-token matrix-vector path and the GEMM path
@pytest.mark.parametrize("kw", [
    dict(latent=256, dense_fmt=synth.Q4_0, n_experts=16, top_k=4, n_groups=4, topk_groups=2,
         tokens=1),
    dict(latent=256, dense_fmt=synth.Q4_0, n_experts=16, top_k=4, tokens=6),
    dict(latent=256, dense_fmt=synth.Q4_0, expert_fmt=synth.Q4_0, n_experts=16, top_k=4,
         tokens=20),
    dict(latent=256, dense_fmt=synth.Q4_0, n_experts=16, top_k=4, tokens=70),
    dict(hidden=1280, latent=512, dense_fmt=synth.Q4_0, expert_fmt=synth.Q4_0, n_experts=32,
         top_k=8, n_groups=8, topk_groups=4, tokens=40),
])
def test_q4_0_dense_projections(kw):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tap_tokens=min(w.tokens, 3))
    _report("dense q4_0 " + str(kw), w.tokens, rep)


# Q5_1 experts (the min term takes the Q8_1 block's stored s): decode, a verify
# window, the 9..32-token path, more than 32 tokens (still the matrix-vector
# kernels), latent layers, wider rows
@pytest.mark.parametrize("kw", [
    dict(expert_fmt=synth.Q5_1, tokens=1),
    dict(expert_fmt=synth.Q5_1, tokens=6, n_experts=16, top_k=3, n_groups=4, topk_groups=2),
    dict(expert_fmt=synth.Q5_1, tokens=20),
    dict(expert_fmt=synth.Q5_1, tokens=70, bias=True),
    dict(expert_fmt=synth.Q5_1, latent=256, n_experts=16, top_k=4, tokens=6),
    dict(expert_fmt=synth.Q5_1, latent=256, n_experts=16, top_k=4, tokens=40),
    dict(expert_fmt=synth.Q5_1, hidden=4096, n_ff=1536, n_experts=8, top_k=2, tokens=1),
    dict(expert_fmt=synth.Q5_1, hidden=4096, n_ff=1536, n_experts=8, top_k=2, tokens=6),
])
def test_q5_1_experts(kw):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tap_tokens=min(w.tokens, 3))
    _report("q5_1 " + str(kw), w.tokens, rep)


# Q4_K experts (super-blocks of 256; the min term on each activation block's
# code sum): decode, a verify window, the 9..32-token path, more than 32 tokens,
# latent, decode-sized rows
@pytest.mark.parametrize("kw", [
    dict(expert_fmt=synth.Q4_K, tokens=1),
    dict(expert_fmt=synth.Q4_K, tokens=6, n_experts=16, top_k=3, n_groups=4, topk_groups=2),
    dict(expert_fmt=synth.Q4_K, tokens=20),
    dict(expert_fmt=synth.Q4_K, tokens=70, bias=True),
    dict(expert_fmt=synth.Q4_K, latent=256, n_experts=16, top_k=4, tokens=6),
    dict(expert_fmt=synth.Q4_K, latent=256, n_experts=16, top_k=4, tokens=40),
    dict(expert_fmt=synth.Q4_K, hidden=4096, n_ff=1536, n_experts=8, top_k=2, tokens=1),
    dict(expert_fmt=synth.Q4_K, hidden=4096, n_ff=1536, n_experts=8, top_k=2, tokens=6),
])
def test_q4_k_experts(kw):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tap_tokens=min(w.tokens, 3))
    _report("q4_k " + str(kw), w.tokens, rep)


# Q5_K experts (Q4_K with fifth bits from qh): the same paths
@pytest.mark.parametrize("kw", [
    dict(expert_fmt=synth.Q5_K, tokens=1),
    dict(expert_fmt=synth.Q5_K, tokens=6, n_experts=16, top_k=3, n_groups=4, topk_groups=2),
    dict(expert_fmt=synth.Q5_K, tokens=20),
    dict(expert_fmt=synth.Q5_K, tokens=70, bias=True),
    dict(expert_fmt=synth.Q5_K, latent=256, n_experts=16, top_k=4, tokens=6),
    dict(expert_fmt=synth.Q5_K, hidden=4096, n_ff=1536, n_experts=8, top_k=2, tokens=1),
])
def test_q5_k_experts(kw):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tap_tokens=min(w.tokens, 3))
    _report("q5_k " + str(kw), w.tokens, rep)


# Q3_K experts (super-blocks of 256, 3-bit codes, signed 6-bit scales per 16
# elements): decode, a verify window, the 9..32-token path, more than 32 tokens
# (the matrix cores), latent with group labels, latent prefill, decode-sized rows
@pytest.mark.parametrize("kw", [
    dict(expert_fmt=synth.Q3_K, tokens=1),
    dict(expert_fmt=synth.Q3_K, tokens=6, n_experts=16, top_k=3, n_groups=4, topk_groups=2),
    dict(expert_fmt=synth.Q3_K, tokens=20),
    dict(expert_fmt=synth.Q3_K, tokens=70, bias=True),
    dict(expert_fmt=synth.Q3_K, latent=256, n_experts=16, top_k=4, n_groups=4, topk_groups=2,
         tokens=1),
    dict(expert_fmt=synth.Q3_K, latent=256, n_experts=16, top_k=4, tokens=40),
    dict(expert_fmt=synth.Q3_K, hidden=4096, n_ff=1536, n_experts=8, top_k=2, tokens=1),
    dict(expert_fmt=synth.Q3_K, hidden=4096, n_ff=1536, n_experts=8, top_k=2, tokens=6),
])
def test_q3_k_experts(kw):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tap_tokens=min(w.tokens, 3))
    _report("q3_k " + str(kw), w.tokens, rep)


# NVFP4 experts (E2M1 codes, an E4M3 scale per 16 elements, an fp32 scale per
# tensor; matrix-vector kernels at every T): decode, a verify window with groups
# (slots from the routing ids), the 9..32-token path (per-bucket down), 32
# tokens, more than 32 (bucketed by the many-token router), latent layers,
# decode-sized rows
@pytest.mark.parametrize("kw", [
    dict(expert_fmt=synth.NVFP4, tokens=1),
    dict(expert_fmt=synth.NVFP4, tokens=6, n_experts=16, top_k=3, n_groups=4, topk_groups=2),
    dict(expert_fmt=synth.NVFP4, tokens=20, bias=True),
    dict(expert_fmt=synth.NVFP4, tokens=32),
    dict(expert_fmt=synth.NVFP4, latent=256, n_experts=16, top_k=4, n_groups=4, topk_groups=2,
         tokens=1),
    dict(expert_fmt=synth.NVFP4, latent=256, n_experts=16, top_k=4, tokens=6),
    dict(expert_fmt=synth.NVFP4, latent=256, n_experts=16, top_k=4, tokens=24),
    dict(expert_fmt=synth.NVFP4, tokens=100, bias=True),
    dict(expert_fmt=synth.NVFP4, latent=256, n_experts=16, top_k=4, n_groups=4, topk_groups=2,
         tokens=70),
    dict(expert_fmt=synth.NVFP4, hidden=4096, n_ff=1536, n_experts=8, top_k=2, tokens=1),
    dict(expert_fmt=synth.NVFP4, hidden=4096, n_ff=1536, n_experts=8, top_k=2, tokens=6),
])
def test_nvfp4_experts(kw):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tap_tokens=min(w.tokens, 3))
    _report("nvfp4 " + str(kw), w.tokens, rep)


# the full-size NVFP4 layers: decode shapes and the latent_q4 shapes
@pytest.mark.parametrize("name,T", [("decode_nvfp4", 1), ("decode_nvfp4", 6), ("latent_nvfp4", 1),
                                    ("latent_nvfp4", 32)])
def test_nvfp4_layers(name, T):
    layer, inp = _layer(name, 32)
    rep = gh.check_case(synth.WORKLOADS[name], T, tap_tokens=2, layer=layer, inp=inp)
    _report(name, T, rep)


def test_nvfp4_latent_prefill():
    """latent_nvfp4 at 2048 tokens (matrix-vector experts per bucket, matrix-core D/U)."""
    name, T = "latent_nvfp4", 2048
    layer, inp = _layer(name, T)
    rep = gh.check_case(synth.WORKLOADS[name], T, tap_tokens=2, layer=layer, inp=inp)
    _report(name, T, rep)


# path boundaries (single-token routing at T = 1, the per-token selection kernel with
# bucketing up to 32 tokens, matrix-vector experts up to 32), the few-token router's
# float4-per-thread sizes (H = 256 and 512: one, partly masked; 1280: two, the second
# partly masked; 4096: four; 7168 and 8192: eight), and the largest routing sizes the
# ABI accepts
@pytest.mark.parametrize("kw", [
    dict(hidden=1280, n_ff=768, tokens=1),
    dict(hidden=1280, n_ff=768, n_groups=4, topk_groups=2, tokens=4),
    dict(n_experts=16, top_k=3, n_groups=4, topk_groups=2, tokens=8),
    dict(n_experts=16, top_k=3, n_groups=4, topk_groups=2, tokens=9),
    dict(n_experts=16, top_k=3, n_groups=4, topk_groups=2, tokens=32),
    dict(n_experts=16, top_k=3, n_groups=4, topk_groups=2, tokens=33),
    dict(hidden=256, n_ff=256, n_experts=512, top_k=32, n_groups=64, topk_groups=8, tokens=1),
    dict(hidden=256, n_ff=256, n_experts=512, top_k=32, n_groups=64, topk_groups=8, tokens=6),
    dict(hidden=256, n_ff=256, n_experts=512, top_k=32, tokens=33),
    dict(hidden=8192, n_ff=256, n_experts=2, top_k=1, tokens=1),
    dict(hidden=8192, n_ff=256, n_experts=2, top_k=1, tokens=40),
])
def test_boundaries_and_maximum_sizes(kw):
    w = _variant(**kw)
    rep = gh.check_case(w, w.tokens, tap_tokens=min(w.tokens, 2))
    _report("edge " + str(kw), w.tokens, rep)


def _exact_ids(w, inp, T):
    """GPU ids and the oracle's ids for every token (no near-tie exclusion)."""
    import oracle
    layer = gh.gpu_layer(w, inp, T)
    g = gh.run_taps(layer, w, inp["x"], 0)
    layer.close()
    _, rt = oracle.layer_forward(w, inp["x"], inp["router_w"], inp["router_b"], inp["groups"],
                                 inp["experts"], inp["D"], inp["U"], taps=("ids", "weights"))
    return g, rt


@pytest.mark.parametrize("T", [1, 6, 20, 40])
def test_exact_expert_ties_go_to_lower_id(T):
    """Experts 1 and 3 share a router row (exactly equal logits on both sides),
    scaled so that they often lead: top-1 must pick expert 1, never 3."""
    w = _variant(tokens=T, top_k=1)
    inp = gh.make_inputs(w)
    # a row along the sum of the tokens: a large positive logit for each token
    lead = (inp["x"].sum(0) * (8.0 / w.hidden)).astype(np.float32)
    inp["router_w"][1] = lead
    inp["router_w"][3] = lead
    g, rt = _exact_ids(w, inp, T)
    assert np.array_equal(g["ids"], rt["ids"])
    assert np.all(g["ids"] == 1)


@pytest.mark.parametrize("T", [1, 6, 20, 40])
def test_exact_group_ties_go_to_lower_group(T):
    """Groups 0 and 2 have identical, dominant router rows: with one group kept,
    group 0's experts win the tie, never group 2's."""
    w = _variant(tokens=T, n_experts=16, top_k=2, n_groups=4, topk_groups=1)
    inp = gh.make_inputs(w)
    lead = (inp["x"].sum(0) * (1.0 / w.hidden)).astype(np.float32)
    for j, c in enumerate((8.0, 7.0, 6.0, 5.0)):
        inp["router_w"][j] = lead * np.float32(c)
        inp["router_w"][8 + j] = lead * np.float32(c)
    g, rt = _exact_ids(w, inp, T)
    assert np.array_equal(g["ids"], rt["ids"])
    assert np.all(g["ids"] == np.array([0, 1]))
    assert np.allclose(g["weights"], rt["weights"], rtol=4e-7, atol=0)


def test_zero_input_uniform_weights_zero_output():
    w = _variant(tokens=3)
    inp = gh.make_inputs(w)
    inp["x"] = np.zeros_like(inp["x"])
    layer = gh.gpu_layer(w, inp, 3)
    g = gh.run_taps(layer, w, inp["x"], 3)
    assert np.all(g["out"] == 0)
    assert np.all(g["ids"] == np.arange(2)) and np.all(g["weights"] == np.float32(0.5))
    layer.close()


def test_identical_experts_output_independent_of_routing():
    import oracle
    w = _variant(tokens=6, n_experts=6, top_k=3)
    inp = gh.make_inputs(w)
    one = synth.gen_expert(w, 0)
    inp["experts"] = np.tile(one, w.n_experts)
    layer = gh.gpu_layer(w, inp, 6)
    g = gh.run_taps(layer, w, inp["x"], 0)
    for t in range(6):
        y = oracle.expert_ffn(w, one, g["xq"][t])["y"]
        assert gh.rel_max(g["out"][t], y) < 2e-3
    assert len({tuple(r) for r in g["ids"]}) > 1
    layer.close()


def test_empty_and_refused_calls():
    import torch
    w = _variant(tokens=4)
    inp = gh.make_inputs(w)
    layer = gh.gpu_layer(w, inp, 4)
    out = torch.full((1, w.hidden), 3.0, device=layer.dev)
    ws = layer.workspace(4)
    h = layer.handle
    x = torch.from_numpy(inp["x"]).to(layer.dev)
    # T = 0: no-op
    moe.moe_layer_forward(h, x.data_ptr(), 0, layer.router_w.data_ptr(), 0, 0,
                          layer.experts.data_ptr(), 0, 0, 2, out.data_ptr(), ws.data_ptr(),
                          ws.numel(), 0)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    for T, k, nbytes, status in [(5, 2, ws.numel(), moe.MOE_EINVAL),     # T > max_tokens
                                 (4, 3, ws.numel(), moe.MOE_EINVAL),     # k != top_k
                                 (4, 2, 16, moe.MOE_ENOMEM)]:            # workspace too small
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_layer_forward(h, x.data_ptr(), T, layer.router_w.data_ptr(), 0, 0,
                                  layer.experts.data_ptr(), 0, 0, k, out.data_ptr(),
                                  ws.data_ptr(), nbytes, 0)
        assert ei.value.status == status
    layer.close()


def test_token_permutation_permutes_output():
    w = _variant(tokens=7)
    inp = gh.make_inputs(w)
    layer = gh.gpu_layer(w, inp, 7)
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    o = gh.run_plain(layer, inp["x"])
    op = gh.run_plain(layer, np.ascontiguousarray(inp["x"][perm]))
    assert np.array_equal(op, o[perm])       # each token is computed on its own
    layer.close()


def test_quantizer_double_rounding_blocks():
    """Q8_1 blocks whose s needs the fp32 rounding before the binary16 one."""
    import oracle
    import quant_cases
    blocks = quant_cases.double_rounding_blocks(8)
    w = _variant(tokens=4)
    inp = gh.make_inputs(w)
    x = inp["x"].reshape(-1, 32).copy()
    x[3:3 + 8 * 7:7] = blocks
    x = x.reshape(4, w.hidden)
    layer = gh.gpu_layer(w, inp, 4)
    g = gh.run_taps(layer, w, x, 0)
    assert np.array_equal(g["xq"], oracle.quantize_q8_1(x))
    layer.close()
