#!/usr/bin/env python3
"""Throughput of the quantized MoE expert-FFN layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode] [--tokens T]

A step is one whole layer call (router logits, top-k softmax, Q8_1 activation
quantisation, grouped gate/up + SwiGLU + requantisation, grouped down, combine,
and for latent layers the D/U projections) over one batch of synthetic tokens,
with every input already resident in HBM.  Steps rotate over several device
copies of the expert weights and a pool of token batches so that a step cannot
be served from the 256 MB MALL by an earlier one.

Prints one JSON line: tokens/s (value), the dominant kernel's achieved HBM
bandwidth against the 8 TB/s peak (roofline; the kernel's duration comes from
two HIP events recorded by that kernel's own dispatch on the library's stream),
the CPU oracle's throughput on a bounded sample of the same workload
(cpu_baseline), and, unless --no-prefill, the 2048-token prefill layer with the
int8 matrix-core utilisation of its grouped gate/up GEMM.  Also reported: the
10th/50th/90th percentiles of the per-step layer time (events), the same steps
replayed from HIP graphs (graph), and the box's single-launch HBM read rate from
libmoe's 16-byte-load probe at the gate/up launch's size, the down weights' size,
the layer's size and 1 GiB (hbm_probe), as the ceiling for the kernel bandwidths.

Traffic (roofline.traffic) comes from two rocprofv3 counter runs of this script
with --calibration-copy (FETCH_SIZE, then WRITE_SIZE), summarised by
--write-traffic into profiles/traffic_gate_up_<workload>_T<T>.json.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 matrix peak
Q8_1_BLOCK = 36
METRIC = "MoE-layer tokens/s + expert-weight GB/s (% of HBM peak), decode & prefill"
COPY_BYTES = 256 << 20       # the calibration copy kernel moves this many bytes each way


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--workload", default="decode",
                   help="tiny | decode | latent_q8 | latent_q4 | prefill | decode_q5_1 | decode_q4_k | "
                        "decode_q5_k")
    p.add_argument("--tokens", type=int, default=None, help="tokens per step (default: the workload's)")
    p.add_argument("--dense-fmt", choices=("q8_0", "q4_0"), default=None,
                   help="block format of a latent layer's D/U (default: the workload's, Q8_0)")
    p.add_argument("--copies", type=int, default=None, help="device copies of the expert weights")
    p.add_argument("--pool", type=int, default=64, help="distinct token batches")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--profile-steps", action="store_true",
                   help="also print per-stage milliseconds to stderr")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    p.add_argument("--no-hbm-probe", action="store_true", help="skip the HBM read probe")
    p.add_argument("--prefill-steps", type=int, default=20)
    p.add_argument("--expert-cache", action="store_true",
                   help="also time the expert-table path: every expert read from pinned host "
                        "memory over the bus, then with the routed experts admitted to slots")
    p.add_argument("--calibration-copy", action="store_true",
                   help="end with three copy kernels of 256 MiB each way (x * 1.0 in fp32), "
                        "the calibration of the HBM byte counters")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                        "script with --calibration-copy for --workload/--tokens, print the "
                        "record that bench.py reads from profiles/ and exit")
    return p.parse_args()


class HipEvents:
    """hipEvent_t handles from the HIP runtime this process already has mapped
    (the one torch and libmoe share)."""

    def __init__(self):
        import ctypes
        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        self.lib = ctypes.CDLL(path)
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = self.ct.c_void_p()
        if self.lib.hipEventCreate(self.ct.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self.ct.c_float()
        if self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e: int) -> None:
        self.lib.hipEventDestroy(e)


# The sources that the decode gate/up kernel (the roofline kernel of the
# default workload) is compiled and launched from: its translation unit, the
# headers it includes, its launcher and the forward call that picks it.
GATE_UP_SOURCES = ("mv_q8_0.hip", "matvec_kern.h", "matvec.h", "select.h", "kernels.h", "device.h",
                   "moe_internal.h", "matvec.hip", "capi.cpp")


def src_hash() -> str:
    """Hash of GATE_UP_SOURCES: a traffic record counts only while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_expert_softmax_amd", "csrc")
    for f in GATE_UP_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, T, n_active):
    """Bytes the method must move per step, and per launch of the gate/up kernel.

    gate/up: the active experts' gate and up blocks, the quantised expert input
    (T rows of Kin/32 Q8_1 blocks) and the quantised h it writes (T*k rows of F/32
    Q8_1 blocks).  Layer: router weights, x, every active expert's blocks, D and
    U, and out."""
    H, E, k, F, L = w.hidden, w.n_experts, w.top_k, w.n_ff, w.latent
    kin, kout = w.k_in, w.k_out
    gu_w = w.matrix_bytes(2 * F, kin // 32)
    dn_w = w.matrix_bytes(kout, F // 32)
    act_in = T * (kin // 32) * Q8_1_BLOCK
    hq = T * k * (F // 32) * Q8_1_BLOCK
    gate_up = n_active * gu_w + act_in + hq
    dense = 0
    if L:
        from quantized_moe_expert_softmax_amd import synth
        dbb = synth.BLOCK_BYTES[w.dense_fmt]
        dense = L * (H // 32) * dbb + H * (L // 32) * dbb
    layer = E * H * 4 + T * H * 4 + n_active * (gu_w + dn_w) + dense + T * H * 4
    return gate_up, layer, n_active * (gu_w + dn_w)


def measure(w, T, steps, warmup, pool, copies, profile=False, graphs=True):
    """Whole-layer steps of workload w at T tokens: wall-clock throughput over
    `steps` steps, then the same steps with stage events and the gate/up
    kernel's own dispatch events.  Inputs are resident before timing starts."""
    import numpy as np
    import torch

    from quantized_moe_expert_softmax_amd import moe, synth

    dev = torch.device("cuda", 0)
    # keep the token pool within 512 MB of device memory
    pool = max(2, min(pool, (512 << 20) // (T * w.hidden * 4)))
    t_gen = time.time()
    inp = synth.gen_layer(w)
    xs = [synth.gen_x(w, batch=b) for b in range(pool)]
    t_gen = time.time() - t_gen

    desc = moe.desc_of(w, max_tokens=T)
    layer = moe.MoeLayer(desc, inp, device=0)
    if copies is None:
        copies = 1 if w.expert_bytes * w.n_experts * T > (1 << 33) else 4
    ex = [layer.experts] + [layer.experts.clone() for _ in range(copies - 1)]
    Ds = [layer.D] + ([layer.D.clone() for _ in range(copies - 1)] if w.latent else [None] * (copies - 1))
    Us = [layer.U] + ([layer.U.clone() for _ in range(copies - 1)] if w.latent else [None] * (copies - 1))
    xd = torch.from_numpy(np.stack(xs)).to(dev)
    out = torch.empty((T, w.hidden), dtype=torch.float32, device=dev)
    ws = layer.workspace(T)
    st = torch.cuda.current_stream(dev).cuda_stream
    P = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731

    def args(i):
        c = i % copies
        return (layer.handle, xd[i % pool].data_ptr(), T, layer.router_w.data_ptr(),
                P(layer.router_b), P(layer.groups), ex[c].data_ptr(), P(Ds[c]), P(Us[c]),
                w.top_k, out.data_ptr(), ws.data_ptr(), ws.numel(), st)

    # distinct experts per batch (for the byte counts), from the routing tap
    n_active = []
    for b in range(pool):
        ids = torch.empty((T, w.top_k), dtype=torch.int32, device=dev)
        taps = moe.moe_taps()
        taps.ids = ids.data_ptr()
        moe.moe_layer_forward_taps(*args(b), taps)
        torch.cuda.synchronize()
        n_active.append(len(np.unique(ids.cpu().numpy())))
    mean_active = float(np.mean(n_active))

    # timed region: whole-layer steps
    for i in range(warmup):
        moe.moe_layer_forward(*args(i))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.moe_layer_forward(*args(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # the same steps again with HIP events on the library's stream
    he = HipEvents()
    evs = [[he.create() for _ in range(moe.MOE_EV_COUNT)] for _ in range(steps)]
    for i in range(warmup):
        moe.moe_layer_forward(*args(i))
    for i in range(steps):
        moe.moe_layer_forward_events(*args(i), evs[i])
    torch.cuda.synchronize()

    def stage(i0, i1):
        return float(np.mean([he.elapsed_ms(evs[s][i0], evs[s][i1]) for s in range(steps)]))

    layer_ms = np.array([he.elapsed_ms(evs[s][moe.MOE_EV_BEGIN], evs[s][moe.MOE_EV_END])
                         for s in range(steps)])
    pct = {f"p{q}": float(np.percentile(layer_ms, q)) for q in (10, 50, 90)}

    st_ms = {"gate_up_kernel": stage(moe.MOE_EV_GATE_UP_KSTART, moe.MOE_EV_GATE_UP_KEND),
             "route": stage(moe.MOE_EV_BEGIN, moe.MOE_EV_ROUTED),
             "dense_in": stage(moe.MOE_EV_ROUTED, moe.MOE_EV_EXPERT_IN),
             "gate_up": stage(moe.MOE_EV_EXPERT_IN, moe.MOE_EV_GATE_UP),
             "down": stage(moe.MOE_EV_GATE_UP, moe.MOE_EV_DOWN),
             "dense_out": stage(moe.MOE_EV_DOWN, moe.MOE_EV_END),
             "layer_events": stage(moe.MOE_EV_BEGIN, moe.MOE_EV_END)}
    for row in evs:
        for e in row:
            he.destroy(e)
    if profile:
        print(json.dumps({"workload": w.name, "stage_ms": st_ms}), file=sys.stderr)

    # the same steps replayed from HIP graphs, one graph per (weight copy, batch)
    # pair of the rotation, so the host launches one graph per layer call
    graph_ms = None
    if graphs:
        gs = []
        for i in range(min(steps, 2 * copies)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                ga = list(args(i))
                ga[-1] = torch.cuda.current_stream(dev).cuda_stream
                moe.moe_layer_forward(*ga)
            gs.append(g)
        for i in range(warmup):
            gs[i % len(gs)].replay()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for i in range(steps):
            gs[i % len(gs)].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t2) * 1e3 / steps
        del gs
    layer.close()
    return dict(tokens_s=T * steps / (t1 - t0), ms_step=(t1 - t0) * 1e3 / steps, st_ms=st_ms,
                layer_ms_pct=pct, graph_ms_step=graph_ms,
                mean_active=mean_active, copies=copies, pool=pool, t_gen=t_gen, inp=inp, xs=xs)


def measure_cache(w, T, steps, warmup, pool=8):
    """The table form of the layer call through the expert cache: steps with
    every expert read from the pinned host copy (over the bus), then with the
    experts that the token pool routes to admitted into device slots; and the
    host-to-device rate of admitting packs."""
    import numpy as np
    import torch

    from quantized_moe_expert_softmax_amd import moe, synth

    dev = torch.device("cuda", 0)
    inp = synth.gen_layer(w)
    layer = moe.MoeLayer(moe.desc_of(w, max_tokens=T), inp, device=0)
    xd = [torch.from_numpy(synth.gen_x(w, batch=b)).to(dev) for b in range(pool)]
    routed = set()
    for x in xd:
        ids = torch.empty((T, w.top_k), dtype=torch.int32, device=dev)
        taps = moe.moe_taps()
        taps.ids = ids.data_ptr()
        layer.forward(x, taps=taps)
        torch.cuda.synchronize()
        routed |= set(int(e) for e in ids.cpu().numpy().ravel())
    S = len(routed)
    cache = moe.ExpertCache(layer, inp["experts"], n_slots=S)
    out = torch.empty((T, w.hidden), dtype=torch.float32, device=dev)

    def run(n):
        for i in range(n):
            cache.forward(xd[i % pool], out=out)

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3 / steps
    t0 = time.perf_counter()
    copied = cache.admit(sorted(routed))
    torch.cuda.synchronize()
    admit_ms = (time.perf_counter() - t0) * 1e3
    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    slot_ms = (time.perf_counter() - t0) * 1e3 / steps
    # the bytes one step reads from the experts: k packs per token (distinct per
    # batch at T = 1)
    step_bytes = min(T * w.top_k, w.n_experts) * w.expert_bytes
    cache.close()
    layer.close()
    return {"workload": w.name, "tokens_per_step": T, "slots": S,
            "host": {"tokens_per_s": T / (host_ms * 1e-3), "ms_per_step": host_ms,
                     "expert_read_gbs": step_bytes / (host_ms * 1e-3) / 1e9},
            "slots_resident": {"tokens_per_s": T / (slot_ms * 1e-3), "ms_per_step": slot_ms},
            "admit": {"packs": copied, "ms": admit_ms,
                      "h2d_gbs": copied * w.expert_bytes / (admit_ms * 1e-3) / 1e9}}


def probe_regions(sizes, min_total=2 << 30):
    """Buffer size and regions of the HBM read probe: each size rounded down to
    4 KiB, and a buffer of at least min_total bytes that holds at least two
    disjoint regions of the largest size.  Returns (total, [(nbytes, nreg)]):
    launch r of a size reads [(r % nreg) * nbytes, + nbytes), inside the buffer."""
    sizes = [s // 4096 * 4096 for s in sizes]
    if not sizes or min(sizes) <= 0:
        raise ValueError(f"probe sizes must be at least 4 KiB: {sizes}")
    total = max(min_total, 2 * max(sizes))
    return total, [(s, total // s) for s in sizes]


def hbm_probe(sizes, reps=20):
    """The box's single-launch HBM read rate, the ceiling the expert kernels are
    compared with: libmoe's read probe (include/moe_probe.h, 16-byte loads) over
    each size, one launch timed by its own dispatch events, swept over grid sizes,
    loads in flight per thread and the load kind; the best median is reported.
    Launches rotate over disjoint regions of a buffer of random bytes (2 GiB, or
    two of the largest size), so no launch is served from the 256 MB MALL by the
    previous ones."""
    import numpy as np
    import torch

    from quantized_moe_expert_softmax_amd import moe
    dev = torch.device("cuda", 0)
    total, regions = probe_regions(sizes)
    buf = torch.randint(0, 256, (total,), dtype=torch.uint8, device=dev)
    blocks_opts, unroll_opts = (512, 1024, 2048, 4096, 8192), (2, 4, 8)
    sink = torch.empty(max(blocks_opts) * 256, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    he = HipEvents()
    evs = [(he.create(), he.create()) for _ in range(reps)]
    res = []
    for nbytes, nreg in regions:
        best = None
        for blocks in blocks_opts:
            for unroll in unroll_opts:
                for nt in (0, moe.MOE_PROBE_NONTEMPORAL):
                    for r in range(reps + 3):
                        e = evs[r - 3] if r >= 3 else (0, 0)
                        off = (r % nreg) * nbytes
                        assert off + nbytes <= buf.numel(), (off, nbytes, buf.numel())
                        moe.moe_probe_read(buf.data_ptr() + off, nbytes, blocks,
                                           unroll, nt, sink.data_ptr(), st, *e)
                    torch.cuda.synchronize()
                    med = float(np.median([he.elapsed_ms(a, b) for a, b in evs]))
                    if best is None or med < best[0]:
                        best = (med, blocks, unroll, nt)
        med, blocks, unroll, nt = best
        res.append({"bytes": nbytes, "gbs": nbytes / (med * 1e-3) / 1e9, "us": med * 1e3,
                    "blocks": blocks, "loads_in_flight": unroll, "nontemporal": bool(nt)})
    for a, b in evs:
        he.destroy(a)
        he.destroy(b)
    del buf, sink
    torch.cuda.empty_cache()
    return {"kernel": "moe_probe_read: 16-byte loads, one launch per size, dispatch events",
            "reps": reps, "sizes": res}


def host_cpu():
    """The host's CPU model and the threads this process may use (at most 16, the
    GPU machine's CPU share for one GPU)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return model, avail, max(1, min(16, avail))


def cpu_oracle_rate(w, inp, xs, seconds, nthreads):
    """The oracle, untuned, on the host: calls of nthreads tokens each (one per
    thread; every token is routed and computed on its own), taken in turn from
    the token batches stacked into one pool, for about `seconds`.  Returns
    (tokens/s, tokens, calls, elapsed)."""
    import numpy as np

    import oracle
    X = np.ascontiguousarray(np.concatenate(xs, axis=0))
    n = X.shape[0]
    chunk = max(1, min(nthreads, n))
    t0 = time.perf_counter()
    done = calls = 0
    while time.perf_counter() - t0 < seconds:
        first = calls * chunk % n
        oracle.layer_forward(w, X, inp["router_w"], inp["router_b"], inp["groups"],
                             inp["experts"], inp["D"], inp["U"],
                             tokens=[(first + t) % n for t in range(chunk)], nthreads=nthreads)
        done += chunk
        calls += 1
    el = time.perf_counter() - t0
    return done / el, done, calls, el


def graph_rate(T, ms):
    """Layer calls replayed from HIP graphs: tokens/s and ms per step."""
    if ms is None:
        return None
    return {"tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms}


def gemm_int8_ops(w, T):
    """int8 multiply-adds (as 2 ops) of the grouped gate/up GEMM: every
    assignment against 2F rows of Kin."""
    return 2.0 * T * w.top_k * 2 * w.n_ff * w.k_in


def write_traffic(fetch_dir, write_dir):
    """profiles/traffic_gate_up_<workload>_T<T>.json from two rocprofv3 --pmc runs
    of this script with --calibration-copy: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of the gate/up kernel, scaled by what the same counters read for
    the plain copy kernel of COPY_BYTES each way."""
    import csv
    import glob

    def per_kernel(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        acc = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    res = {}
    for name, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        acc = per_kernel(d, counter)
        gu = [v for k, vs in acc.items()
              if "gate_up" in k or "k_mfma_dma<true" in k or "k_mfma_q4<true" in k for v in vs]
        cp = [v for k, vs in acc.items() if "MulFunctor" in k for v in vs]
        if not gu or not cp:
            raise SystemExit(f"{d}: no gate/up or calibration dispatches with {counter}")
        kib_gu = sum(gu) / len(gu)
        kib_cp = sum(cp) / len(cp)
        scale = COPY_BYTES / (kib_cp * 1024.0)
        res[name] = dict(kib_per_dispatch=kib_gu, copy_kib=kib_cp, scale=scale,
                         bytes_per_launch=kib_gu * 1024.0 * scale, dispatches=len(gu))
    res["bytes_per_launch"] = res["fetch"]["bytes_per_launch"] + res["write"]["bytes_per_launch"]
    res["src_hash"] = src_hash()
    return res


def _progress(msg: str):
    """One line per finished phase, on stderr (the result line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    a = parse()
    if a.write_traffic:
        res = write_traffic(*a.write_traffic)
        print(json.dumps(res))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the layer is a "
                          "single-GPU kernel path (several GPUs would split the experts and "
                          "exchange Q8_1 rows and weighted outputs by all-to-all; not built)",
                          "n_gpus": a.gpus}))
        sys.exit(2)

    import torch

    from quantized_moe_expert_softmax_amd import synth

    w0 = synth.WORKLOADS[a.workload]
    T = a.tokens or w0.tokens
    over = {"tokens": T}
    if a.dense_fmt:
        over["dense_fmt"] = synth.Q4_0 if a.dense_fmt == "q4_0" else synth.Q8_0
    w = synth.Workload(**{**w0.__dict__, **over})
    m = measure(w, T, a.steps, a.warmup, a.pool, a.copies, a.profile_steps)
    st_ms = m["st_ms"]
    _progress(f"{w.name} T={T}: {m['ms_step'] * 1e3:.1f} us/step")

    gu_bytes, layer_bytes, expert_bytes = algorithmic_bytes(w, T, m["mean_active"])
    gu_gbs = gu_bytes / (st_ms["gate_up_kernel"] * 1e-3) / 1e9

    traffic = None
    tf = os.path.join(ROOT, "profiles", f"traffic_gate_up_{a.workload}_T{T}.json")
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("src_hash") == src_hash():
            traffic = rec.get("bytes_per_launch")

    cpu = None
    if not a.no_cpu_baseline:
        model, avail, nth = host_cpu()
        rate, done, calls, el = cpu_oracle_rate(w, m["inp"], m["xs"], a.cpu_seconds, nth)
        _progress(f"CPU oracle: {rate:.1f} tokens/s on {nth} threads")
        cpu = {"value": rate, "unit": "tokens/s", "cores": nth, "kind": "oracle",
               "sample": f"{done} tokens of this workload ({calls} oracle calls of {nth} "
                         f"tokens drawn in turn from its {len(m['xs'])} token batches, one token "
                         f"per thread), {el:.1f} s on {nth} host threads",
               "cpu_model": model, "host_cpus_available": avail}
    m.pop("inp"), m.pop("xs")

    prefill = None
    if not a.no_prefill and a.workload != "prefill":
        wp = synth.WORKLOADS["prefill"]
        mp = measure(wp, wp.tokens, a.prefill_steps, 3, 4, 1, a.profile_steps)
        _progress(f"prefill T={wp.tokens}: {mp['ms_step'] * 1e3:.1f} us/step")
        cpu_p = None
        if not a.no_cpu_baseline:
            model, avail, nth = host_cpu()
            rate, done, calls, el = cpu_oracle_rate(wp, mp["inp"], mp["xs"][:1], a.cpu_seconds / 2,
                                                    nth)
            cpu_p = {"value": rate, "unit": "tokens/s", "cores": nth, "kind": "oracle",
                     "sample": f"{done} of the 2048 tokens of one prefill batch ({calls} calls of "
                               f"{nth} tokens, one per thread), {el:.1f} s on {nth} host threads",
                     "cpu_model": model}
        mp.pop("inp"), mp.pop("xs")
        ops = gemm_int8_ops(wp, wp.tokens)
        k_ms = mp["st_ms"]["gate_up_kernel"]
        gb, _, eb = algorithmic_bytes(wp, wp.tokens, mp["mean_active"])
        prefill = {"workload": "prefill", "tokens_per_step": wp.tokens,
                   "tokens_per_s": mp["tokens_s"], "ms_per_step": mp["ms_step"],
                   "mean_active_experts": mp["mean_active"],
                   "int8_mfma": {"kernel": "gate_up (grouped int8 GEMM + SwiGLU + Q8_1)",
                                 "int8_ops_per_launch": ops, "avg_launch_ms": k_ms,
                                 "achieved": ops / (k_ms * 1e-3) / 1e12, "peak": INT8_PEAK_TOPS,
                                 "unit": "TOP/s", "frac": ops / (k_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS},
                   "gate_up_gbs": gb / (k_ms * 1e-3) / 1e9,
                   "stage_ms": mp["st_ms"], "layer_ms_pct": mp["layer_ms_pct"],
                   "graph": graph_rate(wp.tokens, mp["graph_ms_step"]),
                   "cpu_baseline": cpu_p}

    cache = None
    if a.expert_cache:
        cache = measure_cache(w, T, min(a.steps, 40), 3)

    probe = None
    if not a.no_hbm_probe:
        # the gate/up launch's bytes, the down weights', the whole layer's, and 1 GiB
        dn_bytes = m["mean_active"] * w.matrix_bytes(w.k_out, w.n_ff // 32)
        probe = hbm_probe([int(gu_bytes), int(dn_bytes), int(layer_bytes), 1 << 30])
        _progress("HBM read probe done")
        probe["gate_up_vs_probe"] = gu_gbs / probe["sizes"][0]["gbs"]

    if a.calibration_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()

    res = {
        "metric": METRIC,
        "value": m["tokens_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": m["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x int8 -> int32 blocks, fp32 scales/accumulation",
        "data": "synthetic, seeded (counter-based splitmix64)",
        "config": {"workload": a.workload, "hidden": w.hidden, "n_experts": w.n_experts,
                   "top_k": w.top_k, "n_ff": w.n_ff, "latent": w.latent,
                   "expert_fmt": {synth.Q4_0: "Q4_0", synth.Q5_1: "Q5_1", synth.Q4_K: "Q4_K",
                                  synth.Q5_K: "Q5_K", synth.Q3_K: "Q3_K"}.get(w.expert_fmt, "Q8_0"),
                   "dense_fmt": (("Q4_0" if w.dense_fmt == synth.Q4_0 else "Q8_0")
                                 if w.latent else None),
                   "tokens_per_step": T, "weight_copies": m["copies"], "token_batches": m["pool"],
                   "mean_active_experts": m["mean_active"]},
        "roofline": {"bound": "hbm", "kernel": "gate_up (grouped gate/up + SwiGLU + Q8_1)",
                     "achieved": gu_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gu_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": gu_bytes,
                     "avg_launch_ms": st_ms["gate_up_kernel"]},
        "layer_gbs": layer_bytes / (m["ms_step"] * 1e-3) / 1e9,
        "expert_gbs": expert_bytes / ((st_ms["gate_up_kernel"] + st_ms["down"]) * 1e-3) / 1e9,
        "stage_ms": st_ms,
        "layer_ms_pct": m["layer_ms_pct"],
        "graph": graph_rate(T, m["graph_ms_step"]),
        "hbm_probe": probe,
        "prefill": prefill,
        "expert_cache": cache,
        "cpu_baseline": cpu,
        "input_generation_s": m["t_gen"],
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
