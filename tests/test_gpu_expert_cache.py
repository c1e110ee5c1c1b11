"""Experts held apart from one array: the table form of the layer call and the
expert cache (resident packs in device slots in front of a pinned, mapped host
copy that the kernels read over the bus).

The table form runs the kernels of the array form on the same packs, so its
output must equal the array form's bit for bit; it is also compared with the
oracle directly (every token within 2e-3 of the oracle's output RMS).  Each case runs every expert from a
permuted device copy, then from host memory, then through admit/evict cycles
queued on the stream without host synchronisation in between."""
import sys

import numpy as np
import pytest

from quantized_moe_expert_softmax_amd import moe, synth

pytestmark = pytest.mark.gpu

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_helpers as gh  # noqa: E402

# decode (selection in the gate/up prologue), the per-token down kernel, the
# per-slot rows kernels (K-quants), the grouped matrix-core path (T > 32), the
# latent path, and NVFP4 experts (per-token and per-slot down)
CASES = [("tiny", 4), ("tiny", 64), ("decode", 1), ("decode", 6), ("latent_q4", 1),
         ("latent_q8", 40), ("decode_q4_k", 1), ("decode_q3_k", 40), ("latent_nvfp4", 6),
         ("decode_nvfp4", 20)]


def _setup(name, T):
    import torch
    w = synth.Workload(**{**synth.WORKLOADS[name].__dict__, "tokens": T})
    inp = gh.make_inputs(w)
    layer = gh.gpu_layer(w, inp, max_tokens=T)
    x = torch.from_numpy(inp["x"]).to(layer.dev)
    ref = layer.forward(x).clone()
    torch.cuda.synchronize()
    # the per-token oracle expectation (flip-aware) that the table outputs must meet
    rep = gh.check_case(w, T, tap_tokens=0, layer=layer, inp=inp, check_det=False)
    return w, inp, layer, x, ref, rep["_expected"]


def _table_forward(layer, x, table):
    import torch
    T = x.shape[0]
    out = torch.full((T, layer.desc.hidden), float("nan"), dtype=torch.float32, device=layer.dev)
    ws = layer.workspace(T)
    st = torch.cuda.current_stream(layer.dev).cuda_stream
    moe.moe_layer_forward_table(layer.handle, x.data_ptr(), T, layer.router_w.data_ptr(),
                                layer._ptr(layer.router_b), layer._ptr(layer.groups),
                                table.data_ptr(), layer._ptr(layer.D), layer._ptr(layer.U),
                                layer.k, out.data_ptr(), ws.data_ptr(), ws.numel(), st)
    return out


@pytest.mark.parametrize("name,T", CASES)
def test_table_of_permuted_device_packs(name, T):
    import torch
    print(f"\n[table] {name} T={T}", flush=True)
    w, inp, layer, x, ref, exp = _setup(name, T)
    try:
        E, eb = w.n_experts, w.expert_bytes
        assert eb % 256 == 0
        perm = np.random.default_rng(11).permutation(E)          # position i holds expert perm[i]
        idx = torch.from_numpy(perm).to(layer.dev)
        moved = layer.experts.view(E, eb)[idx].contiguous()
        pos = np.empty(E, dtype=np.int64)
        pos[perm] = np.arange(E)
        table = torch.from_numpy(moved.data_ptr() + pos * eb).to(layer.dev)
        out = _table_forward(layer, x, table)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        print("[table] vs oracle:", gh.check_output(w, inp, out.cpu().numpy(), exp),
              flush=True)
    finally:
        layer.close()


def _lru_model(slots, last, tick, named):
    """The documented policy: empty slot first, else the least recently named
    slot not named now (ties: lower slot); experts in ascending id order."""
    for e in sorted(set(named)):
        if e in slots:
            last[slots.index(e)] = tick
    copied = 0
    for e in sorted(set(named)):
        if e in slots:
            continue
        if None in slots:
            v = slots.index(None)
        else:
            cand = [s for s in range(len(slots)) if last[s] < tick]
            v = min(cand, key=lambda s: (last[s], s))
        slots[v] = e
        last[v] = tick
        copied += 1
    return copied


@pytest.mark.parametrize("name,T", CASES)
def test_cache_host_copy_and_evictions(name, T):
    import torch
    print(f"\n[cache] {name} T={T}", flush=True)
    w, inp, layer, x, ref, exp = _setup(name, T)
    cache = None
    try:
        E = w.n_experts
        S = max(2, min(E // 2, 3 * w.top_k))
        cache = moe.ExpertCache(layer, inp["experts"], n_slots=S)
        assert all(cache.slot(e) == -1 for e in range(E))
        # every expert read from the mapped host copy over the bus
        out = cache.forward(x)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "host-resident experts"
        print("[cache] host copy vs oracle:", gh.check_output(w, inp, out.cpu().numpy(), exp),
              flush=True)

        rng = np.random.default_rng(3)
        slots, last = [None] * S, [0] * S
        outs = []
        for tick in range(1, 6):
            n = int(rng.integers(1, S + 1))
            named = [int(e) for e in rng.choice(E, size=n, replace=False)]
            named += named[: n // 3]                      # repeats are allowed
            want = _lru_model(slots, last, tick, named)
            got = cache.admit(named)
            assert got == want, (tick, got, want)
            for s, e in enumerate(slots):
                if e is not None:
                    assert cache.slot(e) == s, (tick, e, s)
            assert sum(cache.slot(e) >= 0 for e in range(E)) == sum(e is not None for e in slots)
            # no host synchronisation between the admit's copies and this call
            outs.append(cache.forward(x))
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o, ref), f"after admit {i + 1}"
        assert cache.admit([]) == 0

        with pytest.raises(moe.MoeError, match="distinct experts"):
            cache.admit(list(range(S + 1)))
        with pytest.raises(moe.MoeError, match="out of range"):
            cache.admit([E])
        # a refused admit leaves the cache as it was
        for s, e in enumerate(slots):
            if e is not None:
                assert cache.slot(e) == s
    finally:
        if cache is not None:
            cache.close()
        layer.close()


def test_cache_refusals():
    import torch
    w = synth.WORKLOADS["tiny"]
    inp = gh.make_inputs(w)
    layer = gh.gpu_layer(w, inp, max_tokens=4)
    try:
        E, eb = w.n_experts, w.expert_bytes
        host = np.zeros(E * eb + 256, dtype=np.uint8)             # pageable: refused
        p = host.ctypes.data + (-host.ctypes.data) % 256
        slots = torch.empty(2 * eb, dtype=torch.uint8, device=layer.dev)
        table = torch.zeros(E, dtype=torch.int64, device=layer.dev)
        with pytest.raises(moe.MoeError, match="pinned"):
            moe.moe_expert_cache_create(layer.handle, p, slots.data_ptr(), 2, table.data_ptr())
        pinned = torch.empty(E * eb, dtype=torch.uint8, pin_memory=True)
        with pytest.raises(moe.MoeError, match="n_slots"):
            moe.moe_expert_cache_create(layer.handle, pinned.data_ptr(), slots.data_ptr(), E + 1,
                                        table.data_ptr())
        with pytest.raises(moe.MoeError, match="slots"):
            moe.moe_expert_cache_create(layer.handle, pinned.data_ptr(), slots.data_ptr(), E,
                                        table.data_ptr())
        with pytest.raises(moe.MoeError, match="table"):
            moe.moe_expert_cache_create(layer.handle, pinned.data_ptr(), slots.data_ptr(), 2,
                                        pinned.data_ptr())
        with pytest.raises(moe.MoeError, match="expert_table"):
            moe.moe_layer_forward_table(layer.handle, 1, 1, 1, 0, 0, 0, 0, 0, w.top_k, 1, 1, 1, 0)
        c = moe.moe_expert_cache_create(layer.handle, pinned.data_ptr(), slots.data_ptr(), 2,
                                        table.data_ptr())
        moe.moe_expert_cache_destroy(c)
        torch.cuda.synchronize()
    finally:
        layer.close()
