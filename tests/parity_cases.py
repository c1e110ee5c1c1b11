"""Workload variants shared by the GPU parity tests and the CPU checks of their
premises (no GPU needed to import this module)."""
from quantized_moe_expert_softmax_amd import synth

# Multi-tile grouped GEMM: 4 experts, top-2, 300 tokens (150 assignments per
# expert on average, more than two 64-token tiles), one case per expert format
# and a latent one whose D/U are Q4_0.
MULTI_TILE = [
    dict(n_experts=4, top_k=2, tokens=300, expert_fmt=fmt) for fmt in
    (synth.Q8_0, synth.Q4_0, synth.Q5_1, synth.Q4_K, synth.Q5_K, synth.Q3_K, synth.NVFP4)
] + [
    dict(n_experts=4, top_k=2, tokens=300, latent=256, expert_fmt=synth.Q4_0,
         dense_fmt=synth.Q4_0),
]


def variant(**kw) -> synth.Workload:
    """The small variant layer the parity tests build on (seed 300)."""
    base = dict(name="v", hidden=512, n_experts=8, top_k=2, n_ff=256, tokens=5, seed=300)
    base.update(kw)
    return synth.Workload(**base)
