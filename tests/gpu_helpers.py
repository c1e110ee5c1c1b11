"""Helpers of the GPU parity tests: run the layer through the C ABI with taps,
and compare with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import dataclasses
import os

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
    """Positions whose k-th and (k+1)-th allowed logits (or group boundary) are within
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


def valid_near_tie_ids(w, logits: np.ndarray, gpu_ids: np.ndarray, ref_ids: np.ndarray) -> bool:
    """The GPU's experts for a near-tie token are a valid top-k: distinct, and their
    oracle logits, sorted, equal the oracle's chosen logits within the tie width."""
    eps = 1e-9 * max(float(np.max(np.abs(logits))), 1e-30)
    if len(set(int(e) for e in gpu_ids)) != len(gpu_ids):
        return False
    a = np.sort(logits[gpu_ids])[::-1]
    b = np.sort(logits[ref_ids])[::-1]
    return bool(np.all(np.abs(a - b) <= eps))


# A Q8_1 code may differ from the oracle's only where the value it quantises sits
# within FLIP_TOL (in units of the block's d) of a .5 rounding boundary: the GPU's
# float came out of another fp32 summation order.  Each such flip moves the code by
# exactly 1.  The count is capped at FLIP_RATE_CAP per code compared: on MI355X the
# measured rate is 0.8e-5 to 1.5e-5 per code over the 2048-token layers (largest
# boundary distance seen: 1.1e-4), so the cap allows about seven times that, and at
# least 8 flips for small cases.
FLIP_TOL = 2e-3
FLIP_RATE_CAP = 1e-4


def requant_flips(gq: np.ndarray, v_ref: np.ndarray, what: str):
    """gq: GPU Q8_1 blocks [..., nb, 36]; v_ref: the oracle's float values they quantise
    [..., nb * 32].  Asserts that every difference from the oracle's Q8_1(v_ref) is a flip
    as defined above; returns (codes compared, codes flipped, largest boundary distance)."""
    ref = oracle.quantize_q8_1(v_ref).reshape(-1, 36)
    g = np.ascontiguousarray(gq).reshape(-1, 36)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    ncodes = g.shape[0] * 32
    bad = np.nonzero(np.any(g != ref, axis=1))[0]
    if bad.size == 0:
        return ncodes, 0, 0.0
    gb, rb = g[bad], ref[bad]
    gd = gb[:, 0:2].copy().view("<u2").astype(np.int64).reshape(-1)
    rd = rb[:, 0:2].copy().view("<u2").astype(np.int64).reshape(-1)
    assert np.all(np.abs(gd - rd) <= 1), (what, "binary16 d differs by more than 1 ulp")
    dd = np.nonzero(gd != rd)[0]
    if dd.size:
        # a d that rounds to the other binary16 neighbour: the oracle's fp32
        # amax / 127 lies within 1e-5 (relative) of the midpoint of the two
        va = np.abs(np.asarray(v_ref, dtype=np.float32).reshape(-1, 32)[bad[dd]]).max(axis=1)
        d32 = (va / np.float32(127)).astype(np.float64)
        mid = 0.5 * (gd[dd].astype(np.uint16).view(np.float16).astype(np.float64) +
                     rd[dd].astype(np.uint16).view(np.float16).astype(np.float64))
        assert np.all(np.abs(d32 - mid) <= 1e-5 * d32), (what, "binary16 d differs away from a "
                                                         "rounding boundary")
    dc = gb[:, 4:].view(np.int8).astype(np.int64) - rb[:, 4:].view(np.int8).astype(np.int64)
    assert np.all(np.abs(dc) <= 1), (what, "a code differs by more than 1")
    v = np.asarray(v_ref, dtype=np.float32).reshape(-1, 32)[bad]
    d = (np.abs(v).max(axis=1) / np.float32(127)).astype(np.float64)
    x = np.abs(v.astype(np.float64)) / np.where(d > 0, d, 1.0)[:, None]
    dist = np.abs(x - np.floor(x) - 0.5)
    m = dc != 0
    worst = float(dist[m].max()) if m.any() else 0.0
    assert worst <= FLIP_TOL, (what, "a code differs away from a rounding boundary", worst)
    return ncodes, int(m.sum()), worst


def dense_isums(fmt, blocks, rows, nblk, acts):
    """Oracle integer block sums and outputs of a block matrix for each Q8_1 vector in acts."""
    ys, iss = [], []
    for a in acts:
        y, i = oracle.matvec(fmt, blocks, rows, nblk, a.reshape(-1), with_isum=True)
        ys.append(y)
        iss.append(i)
    return np.stack(ys), np.stack(iss)


def oracle_threads() -> int:
    """Host threads for the oracle in the GPU tests (at most the machine's CPU share)."""
    return max(1, min(16, os.cpu_count() or 1))


def check_case(w: synth.Workload, T: int, tokens=None, tap_tokens: int = 4, batch: int = 0,
               layer=None, inp=None, check_det: bool = True):
    """Full parity check of one workload at T tokens.  tokens: oracle sample (None = all).

    Unique results are compared exactly: routing ids (except near-tie tokens),
    Q8_1(x), every integer block sum of the tap tokens and every requantisation
    of a GPU intermediate.  Every sampled token's output must lie within 2e-3 of
    the oracle's output RMS.  Floating-point intermediates have more than one
    correct value: a GPU float computed in another fp32 order can sit on the
    other side of a Q8_1 rounding boundary.  Each Q8_1 vector (z, h, y_lat) that
    differs from the oracle's is checked to differ only by such flips of the
    oracle's own value computed from the GPU's upstream inputs; a token with any
    such difference (or with near-tie ids) must also match, within 1e-5, the
    oracle evaluated downstream of the GPU's ids and Q8_1 vectors."""
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
    sample = np.arange(T) if tokens is None else np.asarray(sorted(set(tokens)), dtype=np.int64)
    n = len(sample)
    nth = oracle_threads()
    names = ("logits", "ids", "weights", "xq", "h", "hq") + (("z", "zq", "ylat", "ylq") if w.latent else ())
    ref, rt = oracle.layer_forward(w, x, inp["router_w"], inp["router_b"], inp["groups"],
                                   inp["experts"], inp["D"], inp["U"], tokens=sample, taps=names,
                                   nthreads=nth)
    k, F = w.top_k, w.n_ff
    kin, kout = w.k_in, w.k_out
    ngu = w.matrix_bytes(2 * F, kin // 32)     # gate/up bytes of one expert
    eb = w.expert_bytes
    nbi, nbf = kin // 32, F // 32
    report = {}
    flips = {"zq": [0, 0, 0.0], "hq": [0, 0, 0.0], "ylq": [0, 0, 0.0]}

    def tally(name, res):
        c = flips[name]
        c[0] += res[0]
        c[1] += res[1]
        c[2] = max(c[2], res[2])

    # router: logits (fp64, summation order differs), ids (bit-exact), weights
    gl = g["logits"][sample]
    assert np.allclose(gl, rt["logits"], rtol=0, atol=1e-12 * np.abs(rt["logits"]).max())
    ties = near_tie_tokens(w, rt["logits"], inp["groups"])
    gids = g["ids"][sample]
    same_ids = np.all(gids == rt["ids"], axis=1)
    for i in np.nonzero(~same_ids)[0]:
        assert i in ties, ("ids differ on a token without a near tie", int(sample[i]),
                           gids[i], rt["ids"][i])
        assert valid_near_tie_ids(w, rt["logits"][i], gids[i], rt["ids"][i]), int(sample[i])
    assert np.allclose(g["weights"][sample][same_ids], rt["weights"][same_ids], rtol=4e-7, atol=0)
    report["near_ties"] = len(ties)
    report["near_tie_id_changes"] = int((~same_ids).sum())

    # Q8_1(x): bit-exact
    assert np.array_equal(g["xq"][sample], rt["xq"])

    # every requantisation is Q8_1 of the GPU's own intermediate, bit for bit
    assert np.array_equal(g["hq"], oracle.quantize_q8_1(g["h"]))
    if w.latent:
        assert np.array_equal(g["zq"], oracle.quantize_q8_1(g["z"]))
        assert np.array_equal(g["ylq"], oracle.quantize_q8_1(g["ylat"]))

    # per token: the first stage whose GPU Q8_1 vector differs from the oracle's
    A = np.arange(k)[None, :] + k * sample[:, None]           # [n][k] assignment rows
    dev = ~same_ids
    if w.latent:
        H, L = w.hidden, w.latent
        assert rel_max(g["z"][sample], rt["z"]) < 1e-5
        tally("zq", requant_flips(g["zq"][sample], rt["z"], "zq"))
        same_z = np.all(g["zq"][sample].reshape(n, -1) == rt["zq"].reshape(n, -1), axis=1)
        dev |= ~same_z
    # h on the oracle's own expert input, for tokens whose ids and input agree
    clean = np.nonzero(~dev)[0]
    if clean.size:
        gh_ = g["h"][A[clean]]
        assert rel_max(gh_, rt["h"][clean]) < 1e-4, rel_max(gh_, rt["h"][clean])
        tally("hq", requant_flips(g["hq"][A[clean]], rt["h"][clean], "hq"))
    same_h = np.all(g["hq"][A].reshape(n, -1) == rt["hq"].reshape(n, -1), axis=1)
    dev |= ~same_h
    if w.latent:
        clean = np.nonzero(~dev)[0]
        if clean.size:
            tally("ylq", requant_flips(g["ylq"][sample[clean]], rt["ylat"][clean], "ylq"))
        same_yl = np.all(g["ylq"][sample].reshape(n, -1) == rt["ylq"].reshape(n, -1), axis=1)
        dev |= ~same_yl

    # tokens with a flip or near-tie ids: the oracle downstream of the GPU's choices
    expected = ref.copy()
    didx = np.nonzero(dev)[0]
    if didx.size:
        dt = sample[didx]
        given = dict(ids=g["ids"][dt], hq=g["hq"][A[didx]])
        if w.latent:
            given.update(zq=g["zq"][dt], ylq=g["ylq"][dt])
        out_own, ot = oracle.layer_forward(
            w, x, inp["router_w"], inp["router_b"], inp["groups"], inp["experts"], inp["D"],
            inp["U"], tokens=dt, taps=("h", "ylat") if w.latent else ("h",), given=given,
            nthreads=nth)
        expected[didx] = out_own
        # h computed by the oracle on the GPU's ids and expert input
        assert rel_max(g["h"][A[didx]], ot["h"]) < 1e-4
        tally("hq", requant_flips(g["hq"][A[didx]], ot["h"], "hq (GPU upstream)"))
        if w.latent:
            assert rel_max(g["ylat"][dt], ot["ylat"]) < 1e-5
            tally("ylq", requant_flips(g["ylq"][dt], ot["ylat"], "ylq (GPU upstream)"))

    for name, (nc, nf, worst) in flips.items():
        if nc:
            assert nf <= max(8, FLIP_RATE_CAP * nc), (name, nf, nc)
            report[f"{name}_flips"] = f"{nf}/{nc} (max dist {worst:.1e})"
    report["flip_tokens"] = int(dev.sum())

    # integer block sums of gate/up (on the GPU's expert input) and down (on the GPU's hq)
    ain = g["zq"] if w.latent else g["xq"]
    tt = min(tap_tokens, T)
    for t in range(tt):
        for j in range(k):
            a = t * k + j
            e = int(g["ids"][t, j])
            blob = inp["experts"][e * eb:(e + 1) * eb]
            y_gu, is_gu = oracle.matvec(w.expert_fmt, blob[:ngu], 2 * F, nbi, ain[t].reshape(-1),
                                        with_isum=True)
            assert np.array_equal(g["isum_gu"][a], is_gu), (t, j)
            # NVFP4: the tensor scales (gate, up, down) at the start of the expert's tail
            ts = (blob[eb - 256:eb - 244].view("<f4").astype(np.float64)
                  if w.expert_fmt == synth.NVFP4 else np.ones(3))
            y_gu = np.concatenate([y_gu[:F] * ts[0], y_gu[F:] * ts[1]]).astype(np.float32)
            # h from the oracle's g and u on the GPU's own input: fp32 order only
            gg, uu = y_gu[:F].astype(np.float64), y_gu[F:].astype(np.float64)
            h_own = (gg / (1.0 + np.exp(-gg)) * uu).astype(np.float32)
            assert rel_max(g["h"][a], h_own) < 1e-4, (t, j, rel_max(g["h"][a], h_own))
            y_dn, is_dn = oracle.matvec(w.expert_fmt, blob[ngu:], kout, nbf,
                                        g["hq"][a].reshape(-1), with_isum=True)
            assert np.array_equal(g["isum_dn"][a], is_dn), (t, j)
            assert rel_max(g["y"][a], (y_dn * ts[2]).astype(np.float32)) < 1e-5
    if w.latent and tt:
        H, L = w.hidden, w.latent
        z_ref, iss = dense_isums(w.dense_fmt, inp["D"], L, H // 32, g["xq"][:tt])
        assert np.array_equal(g["isum_d"][:tt], iss)
        assert np.allclose(g["z"][:tt], z_ref, rtol=0, atol=1e-5 * np.abs(z_ref).max())
        _, iss = dense_isums(w.dense_fmt, inp["U"], H, L // 32, g["ylq"][:tt])
        assert np.array_equal(g["isum_u"][:tt], iss)

    # the layer output of every sampled token: within 2e-3 of the oracle's RMS where no
    # Q8_1 code flipped; where one did, within 1e-5 of the oracle on the GPU's choices
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    exp = dict(sample=sample, expected=expected, ref=ref, dev=dev, rms=rms)
    report.update(check_against(exp, g["out"]))
    d = g["out"][sample].astype(np.float64) - ref
    report["out_rms_rel"] = float(np.sqrt(np.mean(d ** 2))) / rms
    report["tokens"] = n
    report["_expected"] = exp

    if check_det:
        o1 = run_plain(layer, x)
        o2 = run_plain(layer, x)
        assert np.array_equal(o1, o2), "not deterministic"
        assert np.array_equal(o1, g["out"]), "taps changed the output"
    if own:
        layer.close()
    return report


def check_against(exp: dict, out: np.ndarray) -> dict:
    """A layer output [T][H] against check_case's per-token expectation: tokens without
    a flip within 2e-3 of the oracle's output RMS; tokens with one within 1e-5 (of that
    token's RMS) of the oracle evaluated on the flipped codes, and, as a sanity ceiling,
    within 0.1 of the oracle's RMS (a single flip of Q8_1(z) moves a latent token's
    output by up to about 3e-2 of it: every later requantisation re-rounds)."""
    sample, expected, dev, rms = exp["sample"], exp["expected"], exp["dev"], exp["rms"]
    o = out[sample].astype(np.float64)
    err = np.max(np.abs(o - expected), axis=1) / rms
    res = {"out_rel_clean": 0.0, "out_rel_flipped_vs_oracle": 0.0}
    if (~dev).any():
        ec = np.where(dev, 0.0, err)
        worst = int(np.argmax(ec))
        assert ec[worst] <= 2e-3, ("output beyond 2e-3 of the oracle RMS", int(sample[worst]),
                                   float(ec[worst]))
        res["out_rel_clean"] = float(ec.max())
    for i in np.nonzero(dev)[0]:
        r = rel_max(o[i], expected[i])
        assert r < 1e-5, ("output vs the oracle on the GPU's choices", int(sample[i]), r)
        e0 = float(np.max(np.abs(o[i] - exp["ref"][i]))) / rms
        assert e0 <= 0.1, ("flipped token far from the oracle", int(sample[i]), e0)
        res["out_rel_flipped_vs_oracle"] = max(res["out_rel_flipped_vs_oracle"], e0)
    return res


def check_output(w: synth.Workload, inp: dict, out: np.ndarray, exp: dict) -> dict:
    """An output computed without taps (e.g. through the expert table) against the
    per-token expectation of a check_case run on the same inputs."""
    assert out.shape[0] == len(exp["sample"]) or out.shape[0] > int(exp["sample"].max())
    return check_against(exp, out)
