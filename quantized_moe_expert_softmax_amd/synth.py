"""Seeded synthetic workloads for the quantized MoE layer.

This module only draws inputs; it holds none of the layer's arithmetic.  The
random numbers come from ``synth.c`` (counter-based splitmix64), so any tensor
or any slice of one can be drawn on its own.  Scales are drawn in double
precision and rounded to IEEE binary16 by numpy's ``astype(np.float16)``.

Distributions (the workloads of the quantized MoE layer, Strata "Q8_0 support"
page, section "GPU expert kernels", and the edge0-strata README, section
"Changes from upstream Strata"):

* activations ``x ~ N(0, 1)`` fp32, router ``W_r ~ N(0, 1/512)`` fp32, optional
  per-expert router bias ``b ~ N(0, 1)``;
* Q8_0 weight blocks: 32 int8 codes uniform in [-127, 127] and a binary16 scale
  ``d = |N(0, 0.02)| / 127``;
* Q4_0 weight blocks: 32 nibbles uniform in [0, 15] and ``d = |N(0, 0.02)| / 8``;
* NVFP4 weight blocks (the edge0-strata README names NVFP4 latent experts;
  the format is read as FP4 E2M1 codes with an FP8 E4M3 scale per 16 elements
  and an fp32 scale per tensor): 32 codes uniform in [0, 15], each 16-element
  half's E4M3 scale with exponent field uniform in 5..9 and mantissa field
  uniform in 0..7 (0.25 to 7.5), and per expert matrix (gate, up, down) a
  tensor scale ``0.002 + |N(0, 0.002)|`` rounded to fp32;
* expert group labels ``group[e] = e // (E // n_groups)``.

Canonical block layouts (little-endian): Q8_0 = binary16 d, 32 x int8 (34 B);
Q4_0 = binary16 d, 16 bytes whose low nibble is element j and high nibble
element j + 16 (18 B); NVFP4 = the E4M3 scales of elements 0..15 and
16..31, then 16 bytes whose byte i holds element 2i in its low nibble and
element 2i + 1 in its high nibble (18 B).  A canonical expert blob holds gate
[F][Kin/32], up [F][Kin/32] and down [Kout][F/32] blocks, in that order, rows
row-major; an NVFP4 blob ends with a 256-byte tail: the three tensor scales
(fp32), then zero bytes.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

Q8_0 = 8
Q4_0 = 2
Q5_1 = 7
Q4_K = 12
Q5_K = 13
Q3_K = 11
NVFP4 = 40
# bytes per 32 elements (Q4_K / Q5_K: 144 / 176-byte super-blocks of 256)
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q5_1: 24, Q4_K: 18, Q5_K: 22, NVFP4: 18}
# bytes after an expert's three matrices (NVFP4: the tensor scales)
EXPERT_TAIL = {NVFP4: 256}
# bytes per super-block of 256 elements
SUPER_BYTES = {Q4_K: 144, Q5_K: 176, Q3_K: 110}


def matrix_bytes(fmt: int, rows: int, nblk: int) -> int:
    """Canonical bytes of a [rows][nblk blocks of 32] matrix of format fmt."""
    if fmt in SUPER_BYTES:
        assert nblk % 8 == 0
        return rows * (nblk // 8) * SUPER_BYTES[fmt]
    return rows * nblk * BLOCK_BYTES[fmt]
S_MIN = 1 << 40      # added to a block set's scale stream for its Q5_1 minimums


def build_synth(force: bool = False) -> str:
    """Compile the generator core with gcc (host code only)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(
            os.path.join(_HERE, "synth.c")):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                               os.path.join(_HERE, "synth.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build_synth()
        lib = ctypes.CDLL(_SO)
        u64, dbl, vp = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, dbl, vp]
        lib.synth_absnormal_f64.argtypes = [u64, u64, u64, u64, dbl, vp]
        lib.synth_int8_sym127.argtypes = [u64, u64, u64, u64, vp]
        lib.synth_nibble_bytes.argtypes = [u64, u64, u64, u64, vp]
        lib.synth_interleave_blocks.argtypes = [u64, vp, vp, u64, vp]
        for f in (lib.synth_normal_f32, lib.synth_absnormal_f64, lib.synth_int8_sym127,
                  lib.synth_nibble_bytes, lib.synth_interleave_blocks):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# stream ids: one per tensor
S_X = 0x100          # + batch index
S_WR = 2
S_BIAS = 3
S_EXP_Q = 0x10000    # + 4 * expert + role
S_EXP_D = 0x20000
S_DENSE = 0x30000    # D quants, D scales, U quants, U scales


def normal_f32(seed: int, stream: int, n: int, scale: float = 1.0, first: int = 0,
               out: Optional[np.ndarray] = None) -> np.ndarray:
    if out is None:
        out = np.empty(n, dtype=np.float32)
    _L().synth_normal_f32(seed, stream, first, n, scale, _ptr(out))
    return out


def absnormal_f64(seed: int, stream: int, n: int, scale: float, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _L().synth_absnormal_f64(seed, stream, first, n, scale, _ptr(out))
    return out


def blocks(fmt: int, seed: int, q_stream: int, d_stream: int, nblk: int,
           out: Optional[np.ndarray] = None) -> np.ndarray:
    """nblk canonical weight blocks of format fmt, as a uint8 array of nblk * 34 (18, 24) bytes."""
    lib = _L()
    if fmt == Q8_0:
        pay = 32
        payload = np.empty(nblk * pay, dtype=np.int8)
        lib.synth_int8_sym127(seed, q_stream, 0, nblk * pay, _ptr(payload))
        scale = absnormal_f64(seed, d_stream, nblk, 0.02 / 127.0)
    elif fmt == Q4_0:
        pay = 16
        payload = np.empty(nblk * pay, dtype=np.uint8)
        lib.synth_nibble_bytes(seed, q_stream, 0, nblk * pay, _ptr(payload))
        scale = absnormal_f64(seed, d_stream, nblk, 0.02 / 8.0)
    elif fmt == Q5_1:
        # binary16 m, then qh (4 bytes) and the 16 nibble bytes, all bits uniform
        pay = 22
        raw = np.empty(nblk * 20, dtype=np.uint8)
        lib.synth_nibble_bytes(seed, q_stream, 0, nblk * 20, _ptr(raw))
        scale = absnormal_f64(seed, d_stream, nblk, 0.02 / 16.0)
        mins = -absnormal_f64(seed, d_stream + S_MIN, nblk, 0.02 / 2.0)
        m16 = mins.astype(np.float16).view(np.uint8).reshape(nblk, 2)
        payload = np.ascontiguousarray(np.concatenate([m16, raw.reshape(nblk, 20)], axis=1)).reshape(-1)
    elif fmt in (Q4_K, Q5_K):
        # super-blocks: binary16 d, binary16 dmin, then 12 scale bytes, (Q5_K:
        # 32 qh bytes,) 128 nibble bytes, all bits uniform
        assert nblk % 8 == 0
        nsb = nblk // 8
        sbb = 144 if fmt == Q4_K else 176
        raw = np.empty(nsb * (sbb - 4), dtype=np.uint8)
        lib.synth_nibble_bytes(seed, q_stream, 0, nsb * (sbb - 4), _ptr(raw))
        scale = absnormal_f64(seed, d_stream, nsb, 0.02 / (512.0 if fmt == Q4_K else 1024.0))
        mins = absnormal_f64(seed, d_stream + S_MIN, nsb, 0.02 / 128.0)
        dm16 = mins.astype(np.float16).view(np.uint8).reshape(nsb, 2)
        payload = np.ascontiguousarray(np.concatenate([dm16, raw.reshape(nsb, sbb - 4)], axis=1)).reshape(-1)
        d16 = scale.astype(np.float16).view(np.uint16)
        if out is None:
            out = np.empty(nsb * sbb, dtype=np.uint8)
        assert out.nbytes == nsb * sbb
        lib.synth_interleave_blocks(nsb, _ptr(d16), _ptr(payload), sbb - 2, _ptr(out))
        return out
    elif fmt == NVFP4:
        # two E4M3 scale bytes (exponent field 5..9, mantissa field 0..7), then
        # 16 code bytes with every bit uniform
        if out is None:
            out = np.empty(nblk * 18, dtype=np.uint8)
        assert out.nbytes == nblk * 18
        o = out.reshape(nblk, 18)
        codes = np.empty(nblk * 16, dtype=np.uint8)
        lib.synth_nibble_bytes(seed, q_stream, 0, nblk * 16, _ptr(codes))
        sraw = np.empty(nblk * 2, dtype=np.uint8)
        lib.synth_nibble_bytes(seed, d_stream, 0, nblk * 2, _ptr(sraw))
        e = 5 + (sraw >> 3) % 5
        o[:, :2] = ((e << 3) | (sraw & 7)).astype(np.uint8).reshape(nblk, 2)
        o[:, 2:] = codes.reshape(nblk, 16)
        return out
    elif fmt == Q3_K:
        # super-blocks: 32 hmask bytes, 64 qs bytes, 12 scale bytes (all bits
        # uniform), then binary16 d
        assert nblk % 8 == 0
        nsb = nblk // 8
        raw = np.empty(nsb * 108, dtype=np.uint8)
        lib.synth_nibble_bytes(seed, q_stream, 0, nsb * 108, _ptr(raw))
        scale = absnormal_f64(seed, d_stream, nsb, 0.02 / 128.0)
        if out is None:
            out = np.empty(nsb * 110, dtype=np.uint8)
        assert out.nbytes == nsb * 110
        o = out.reshape(nsb, 110)
        o[:, :108] = raw.reshape(nsb, 108)
        o[:, 108:] = scale.astype(np.float16).view(np.uint8).reshape(nsb, 2)
        return out
    else:
        raise ValueError(f"unknown block format {fmt}")
    d16 = scale.astype(np.float16).view(np.uint16)
    if out is None:
        out = np.empty(nblk * (2 + pay), dtype=np.uint8)
    assert out.nbytes == nblk * (2 + pay)
    lib.synth_interleave_blocks(nblk, _ptr(d16), _ptr(payload), pay, _ptr(out))
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic MoE layer: shapes, formats and the seed that fills it."""
    name: str
    hidden: int
    n_experts: int
    top_k: int
    n_ff: int
    tokens: int
    latent: int = 0
    expert_fmt: int = Q8_0
    n_groups: int = 0
    topk_groups: int = 0
    bias: bool = False
    seed: int = 0
    dense_fmt: int = Q8_0

    @property
    def k_in(self) -> int:
        return self.latent if self.latent else self.hidden

    @property
    def k_out(self) -> int:
        return self.latent if self.latent else self.hidden

    @property
    def block_bytes(self) -> int:
        return BLOCK_BYTES[self.expert_fmt]

    def role_rows(self):
        """(rows, blocks per row) of gate, up, down."""
        return [(self.n_ff, self.k_in // 32), (self.n_ff, self.k_in // 32),
                (self.k_out, self.n_ff // 32)]

    @property
    def expert_bytes(self) -> int:
        return (sum(matrix_bytes(self.expert_fmt, r, b) for r, b in self.role_rows()) +
                EXPERT_TAIL.get(self.expert_fmt, 0))

    def matrix_bytes(self, rows: int, nblk: int) -> int:
        """Canonical bytes of an expert matrix of `rows` rows of `nblk` blocks."""
        return matrix_bytes(self.expert_fmt, rows, nblk)

    def with_tokens(self, t: int) -> "Workload":
        return dataclasses.replace(self, tokens=t)

    def dense_shapes(self):
        """(rows, blocks per row) of D [L x H] and U [H x L]; empty when not latent."""
        if not self.latent:
            return []
        return [(self.latent, self.hidden // 32), (self.hidden, self.latent // 32)]


# The layers measured and checked here.
WORKLOADS = {
    "tiny": Workload("tiny", hidden=512, n_experts=8, top_k=2, n_ff=256, tokens=4, seed=1000),
    "decode": Workload("decode", hidden=4096, n_experts=128, top_k=8, n_ff=1536, tokens=1,
                       seed=1001),
    "latent_q8": Workload("latent_q8", hidden=4096, n_experts=256, top_k=8, n_ff=1024, tokens=1,
                          latent=1280, n_groups=16, topk_groups=4, seed=1002),
    "latent_q4": Workload("latent_q4", hidden=7168, n_experts=256, top_k=8, n_ff=1024, tokens=1,
                          latent=1792, expert_fmt=Q4_0, n_groups=16, topk_groups=4, seed=1003),
    "prefill": Workload("prefill", hidden=4096, n_experts=128, top_k=8, n_ff=1536, tokens=2048,
                        bias=True, seed=1004),
    "decode_q5_1": Workload("decode_q5_1", hidden=4096, n_experts=128, top_k=8, n_ff=1536,
                            tokens=1, expert_fmt=Q5_1, seed=1005),
    "decode_q4_k": Workload("decode_q4_k", hidden=4096, n_experts=128, top_k=8, n_ff=1536,
                            tokens=1, expert_fmt=Q4_K, seed=1006),
    "decode_q5_k": Workload("decode_q5_k", hidden=4096, n_experts=128, top_k=8, n_ff=1536,
                            tokens=1, expert_fmt=Q5_K, seed=1007),
    "decode_q3_k": Workload("decode_q3_k", hidden=4096, n_experts=128, top_k=8, n_ff=1536,
                            tokens=1, expert_fmt=Q3_K, seed=1008),
    # the latent_q4 shapes with Q3_K latent experts
    "latent_q3_k": Workload("latent_q3_k", hidden=7168, n_experts=256, top_k=8, n_ff=1024,
                            tokens=1, latent=1792, expert_fmt=Q3_K, n_groups=16, topk_groups=4,
                            seed=1009),
    # NVFP4 experts: the decode shapes, and the latent_q4 shapes (decode path
    # only, up to 32 tokens)
    "decode_nvfp4": Workload("decode_nvfp4", hidden=4096, n_experts=128, top_k=8, n_ff=1536,
                             tokens=1, expert_fmt=NVFP4, seed=1010),
    "latent_nvfp4": Workload("latent_nvfp4", hidden=7168, n_experts=256, top_k=8, n_ff=1024,
                             tokens=1, latent=1792, expert_fmt=NVFP4, n_groups=16, topk_groups=4,
                             seed=1011),
}


def gen_x(w: Workload, batch: int = 0, tokens: Optional[int] = None) -> np.ndarray:
    t = w.tokens if tokens is None else tokens
    return normal_f32(w.seed, S_X + batch, t * w.hidden).reshape(t, w.hidden)


def gen_router(w: Workload) -> np.ndarray:
    return normal_f32(w.seed, S_WR, w.n_experts * w.hidden,
                      scale=float(np.sqrt(1.0 / 512.0))).reshape(w.n_experts, w.hidden)


def gen_bias(w: Workload) -> Optional[np.ndarray]:
    if not w.bias:
        return None
    return normal_f32(w.seed, S_BIAS, w.n_experts)


def gen_groups(w: Workload) -> Optional[np.ndarray]:
    if not w.n_groups:
        return None
    per = w.n_experts // w.n_groups
    return (np.arange(w.n_experts, dtype=np.int32) // per).astype(np.int32)


def gen_expert(w: Workload, e: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Canonical blob of expert e (gate, up, down)."""
    if out is None:
        out = np.empty(w.expert_bytes, dtype=np.uint8)
    off = 0
    for role, (rows, nb) in enumerate(w.role_rows()):
        n = w.matrix_bytes(rows, nb)
        blocks(w.expert_fmt, w.seed, S_EXP_Q + 4 * e + role, S_EXP_D + 4 * e + role, rows * nb,
               out=out[off:off + n])
        off += n
    if w.expert_fmt == NVFP4:
        ts = (0.002 + absnormal_f64(w.seed, S_EXP_D + 4 * e + 3, 3, 0.002)).astype(np.float32)
        out[off:off + 12] = ts.view(np.uint8)
        out[off + 12:off + 256] = 0
    return out


def gen_experts(w: Workload, out: Optional[np.ndarray] = None, threads: int = 8) -> np.ndarray:
    """All experts' canonical blobs, drawn on `threads` threads (each expert's
    stream is independent, so the result does not depend on the thread count)."""
    if out is None:
        out = np.empty(w.n_experts * w.expert_bytes, dtype=np.uint8)
    eb = w.expert_bytes
    if threads <= 1:
        for e in range(w.n_experts):
            gen_expert(w, e, out=out[e * eb:(e + 1) * eb])
        return out
    import concurrent.futures as cf
    _L()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda e: gen_expert(w, e, out=out[e * eb:(e + 1) * eb]), range(w.n_experts)))
    return out


def gen_dense(w: Workload):
    """Canonical D [L][H/32] and U [H][L/32] in w.dense_fmt (the same block
    distributions as the experts of that format); (None, None) when not latent."""
    if not w.latent:
        return None, None
    res = []
    for i, (rows, nb) in enumerate(w.dense_shapes()):
        res.append(blocks(w.dense_fmt, w.seed, S_DENSE + 2 * i, S_DENSE + 2 * i + 1, rows * nb))
    return res[0], res[1]


def gen_layer(w: Workload, batch: int = 0):
    """All inputs of one layer call as a dict of numpy arrays (None where absent)."""
    D, U = gen_dense(w)
    return dict(x=gen_x(w, batch), router_w=gen_router(w), router_b=gen_bias(w),
                groups=gen_groups(w), experts=gen_experts(w), D=D, U=U)
