"""Helpers of the GPU parity tests: run the layer through the C ABI with taps,
and compare with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
from quantized_moe_expert_softmax_amd import moe, synth


def make_inputs(w: synth.Workload, batch: int = 0):
    return synth.gen_layer(w, batch)


def gpu_layer(w: synth.Workload, inp: dict, max_tokens: int):
    return moe.MoeLayer(moe.desc_of(w, max_tokens=max_tokens), inp, device=0)


def run_taps(layer: moe.MoeLayer, w: synth.Workload, x: np.ndarray, tap_tokens: int):
    """Forward with every tap; returns dict of numpy arrays (and 'out')."""
    import torch
    dev = layer.dev
    T = x.shape[0]
    k, E, H, F, L = w.top_k, w.n_experts, w.hidden, w.n_ff, w.latent
    kin, kout = w.k_in, w.k_out
    A = T * k
    tt = min(tap_tokens, T)
    shapes = dict(logits=((T, E), torch.float64), ids=((T, k), torch.int32),
                  weights=((T, k), torch.float32), xq=((T, H // 32, 36), torch.uint8),
                  h=((A, F), torch.float32), hq=((A, F // 32, 36), torch.uint8),
                  y=((A, kout), torch.float32),
                  isum_gu=((tt * k, 2 * F, kin // 32), torch.int32),
                  isum_dn=((tt * k, kout, F // 32), torch.int32))
    if L:
        shapes.update(z=((T, L), torch.float32), zq=((T, L // 32, 36), torch.uint8),
                      ylat=((T, L), torch.float32), ylq=((T, L // 32, 36), torch.uint8),
                      isum_d=((tt, L, H // 32), torch.int32), isum_u=((tt, H, L // 32), torch.int32))
    bufs = {n: torch.full(s, -7, dtype=dt, device=dev) if dt != torch.uint8 else
            torch.zeros(s, dtype=dt, device=dev) for n, (s, dt) in shapes.items()}
    taps = moe.moe_taps()
    for n, b in bufs.items():
        setattr(taps, n, b.data_ptr())
    taps.tap_tokens = tt
    xd = torch.from_numpy(x).to(dev)
    out = layer.forward(xd, taps=taps)
    torch.cuda.synchronize()
    res = {n: b.cpu().numpy() for n, b in bufs.items()}
    res["out"] = out.cpu().numpy()
    return res


def run_plain(layer: moe.MoeLayer, x: np.ndarray) -> np.ndarray:
    import torch
    out = layer.forward(torch.from_numpy(x).to(layer.dev))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def rel_max(a, ref):
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    return float(np.max(np.abs(a.astype(np.float64) - ref.astype(np.float64)))) / max(rms, 1e-30)


def near_tie_tokens(w, logits: np.ndarray, groups) -> set:
    """Tokens whose k-th and (k+1)-th allowed logits (or group boundary) are within
    1e-9 * max|l|: there the chosen experts may legitimately depend on fp64 summation order."""
    res = set()
    for t in range(logits.shape[0]):
        l = logits[t]
        eps = 1e-9 * max(float(np.max(np.abs(l))), 1e-30)
        if w.n_groups:
            G = w.n_groups
            gmax = np.array([l[groups == g].max() for g in range(G)])
            sg = np.sort(gmax)[::-1]
            if w.topk_groups < G and sg[w.topk_groups - 1] - sg[w.topk_groups] < eps:
                res.add(t)
                continue
            keep = np.argsort(-gmax, kind="stable")[:w.topk_groups]
            l = l[np.isin(groups, keep)]
        s = np.sort(l)[::-1]
        if w.top_k < len(s) and s[w.top_k - 1] - s[w.top_k] < eps:
            res.add(t)
    return res


def dense_isums(fmt, blocks, rows, nblk, acts):
    """Oracle integer block sums and outputs of a block matrix for each Q8_1 vector in acts."""
    ys, iss = [], []
    for a in acts:
        y, i = oracle.matvec(fmt, blocks, rows, nblk, a.reshape(-1), with_isum=True)
        ys.append(y)
        iss.append(i)
    return np.stack(ys), np.stack(iss)


def check_case(w: synth.Workload, T: int, tokens=None, tap_tokens: int = 4, batch: int = 0,
               layer=None, inp=None, check_det: bool = True):
    """Full parity check of one workload at T tokens.  tokens: oracle sample (None = all).

    Unique results are compared exactly: routing ids, Q8_1(x), every integer
    block sum and every requantisation of a GPU intermediate.  Floating-point
    results have more than one correct value: a GPU intermediate computed in a
    different fp32 order can sit on the other side of a Q8_1 rounding boundary
    (a "flip").  Tokens without a flip must match the oracle's output within
    2e-3 of its RMS; tokens with one must match the oracle evaluated on the
    GPU's own quantised intermediates, and flips must be rare."""
    w = dataclasses.replace(w, tokens=T)
    if inp is None:
        inp = make_inputs(w, batch)
    else:
        inp = dict(inp, x=synth.gen_x(w, batch))
    own = layer is None
    if own:
        layer = gpu_layer(w, inp, max_tokens=T)
    x = inp["x"]
    g = run_taps(layer, w, x, tap_tokens)
    sample = list(range(T)) if tokens is None else list(tokens)
    ref, rt = oracle.layer_forward(w, x, inp["router_w"], inp["router_b"], inp["groups"],
                                   inp["experts"], inp["D"], inp["U"], tokens=sample,
                                   taps=("logits", "ids", "weights", "xq", "z", "zq", "h", "hq",
                                         "y", "ylat", "ylq"),
                                   nthreads=8)
    k, F = w.top_k, w.n_ff
    kin, kout = w.k_in, w.k_out
    ngu = w.matrix_bytes(2 * F, kin // 32)     # gate/up bytes of one expert
    eb = w.expert_bytes
    nbi, nbf = kin // 32, F // 32
    report = {}

    # router: logits (fp64, summation order differs), ids (bit-exact), weights
    gl = g["logits"][sample]
    assert np.allclose(gl, rt["logits"], rtol=0, atol=1e-12 * np.abs(rt["logits"]).max())
    ties = near_tie_tokens(w, rt["logits"], inp["groups"])
    for i, t in enumerate(sample):
        if i in ties:
            continue
        assert np.array_equal(g["ids"][t], rt["ids"][i]), (t, g["ids"][t], rt["ids"][i])
        assert np.allclose(g["weights"][t], rt["weights"][i], rtol=4e-7, atol=0), t
    report["near_ties"] = len(ties)

    # Q8_1(x): bit-exact
    assert np.array_equal(g["xq"][sample], oracle.quantize_q8_1(x[sample]))

    # latent D: integer sums bit-exact on the GPU's xq; zq = Q8_1(GPU z) bit-exact
    if w.latent:
        H, L = w.hidden, w.latent
        tt = min(tap_tokens, T)
        z_ref, iss = dense_isums(w.dense_fmt, inp["D"], L, H // 32, g["xq"][:tt])
        assert np.array_equal(g["isum_d"][:tt], iss)
        assert np.allclose(g["z"][:tt], z_ref, rtol=0, atol=1e-5 * np.abs(z_ref).max())
        assert np.array_equal(g["zq"], oracle.quantize_q8_1(g["z"]))
        assert rel_max(g["z"][sample], rt["z"]) < 1e-5
        ain = g["zq"]
    else:
        ain = g["xq"]

    # every requantisation is Q8_1 of the GPU's own intermediate, bit for bit
    assert np.array_equal(g["hq"], oracle.quantize_q8_1(g["h"]))
    if w.latent:
        assert np.array_equal(g["ylq"], oracle.quantize_q8_1(g["ylat"]))

    # integer block sums of gate/up (on the GPU's expert input) and down (on the GPU's hq)
    tt = min(tap_tokens, T)
    for t in range(tt):
        for j in range(k):
            a = t * k + j
            e = int(g["ids"][t, j])
            blob = inp["experts"][e * eb:(e + 1) * eb]
            gu = blob[:ngu]
            y_gu, is_gu = oracle.matvec(w.expert_fmt, gu, 2 * F, nbi, ain[t].reshape(-1), with_isum=True)
            assert np.array_equal(g["isum_gu"][a], is_gu), (t, j)
            # h from the oracle's g and u on the GPU's own input: fp32 order only
            gg, uu = y_gu[:F].astype(np.float64), y_gu[F:].astype(np.float64)
            h_own = (gg / (1.0 + np.exp(-gg)) * uu).astype(np.float32)
            assert rel_max(g["h"][a], h_own) < 1e-4, (t, j, rel_max(g["h"][a], h_own))
            dn = blob[ngu:]
            y_dn, is_dn = oracle.matvec(w.expert_fmt, dn, kout, nbf, g["hq"][a].reshape(-1), with_isum=True)
            assert np.array_equal(g["isum_dn"][a], is_dn), (t, j)
            assert rel_max(g["y"][a], y_dn) < 1e-5
    if w.latent:
        H, L = w.hidden, w.latent
        _, iss = dense_isums(w.dense_fmt, inp["U"], H, L // 32, g["ylq"][:tt])
        assert np.array_equal(g["isum_u"][:tt], iss)

    # the layer output, token by token
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    flips, clean_err = [], 0.0
    for i, t in enumerate(sample):
        if i in ties:
            continue
        a_t = [t * k + j for j in range(k)]
        flipped = not np.array_equal(g["hq"][a_t], rt["hq"][i])
        if w.latent:
            flipped |= not np.array_equal(g["zq"][t], rt["zq"][i])
            flipped |= not np.array_equal(g["ylq"][t], rt["ylq"][i])
        err = float(np.max(np.abs(g["out"][t].astype(np.float64) - ref[i]))) / rms
        if not flipped:
            assert err <= 2e-3, (t, err)
            clean_err = max(clean_err, err)
            continue
        flips.append(t)
        # the oracle on the GPU's own quantised intermediates
        y_own = []
        for j, a in enumerate(a_t):
            e = int(g["ids"][t, j])
            dn = inp["experts"][e * eb:(e + 1) * eb][ngu:]
            y_own.append(oracle.matvec(w.expert_fmt, dn, kout, nbf, g["hq"][a].reshape(-1)))
        y_own = np.stack(y_own).astype(np.float64)
        comb = (g["weights"][t].astype(np.float64)[:, None] * y_own).sum(0)
        if w.latent:
            assert rel_max(g["ylat"][t], comb) < 1e-5, t
            out_own = oracle.matvec(w.dense_fmt, inp["U"], w.hidden, w.latent // 32, g["ylq"][t].reshape(-1))
        else:
            out_own = comb
        assert rel_max(g["out"][t], out_own) < 1e-5, (t, rel_max(g["out"][t], out_own))
    report["out_rel_clean"] = clean_err
    report["flip_tokens"] = flips
    d = g["out"][sample].astype(np.float64) - ref
    report["out_rms_rel"] = float(np.sqrt(np.mean(d ** 2))) / rms
    assert len(flips) <= max(1, len(sample) // 2), report

    if check_det:
        o1 = run_plain(layer, x)
        o2 = run_plain(layer, x)
        assert np.array_equal(o1, o2), "not deterministic"
        assert np.array_equal(o1, g["out"]), "taps changed the output"
    if own:
        layer.close()
    return report
