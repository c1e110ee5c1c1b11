"""Python access to the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may import this package; the product path never does.  The oracle is
built with gcc into ``liboracle.so`` next to this file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

Q8_0 = 8
Q4_0 = 2
Q5_1 = 7
Q4_K = 12
Q5_K = 13
Q3_K = 11
NVFP4 = 40
Q8_1_BYTES = 36


def build(force: bool = False) -> str:
    """Compile the oracle: plain C, IEEE semantics, no FMA contraction."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-Wno-unused-function", _SRC, "-o", tmp,
                               "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


class Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("hidden", "n_experts", "top_k", "n_ff", "latent",
                                            "expert_fmt", "n_groups", "topk_groups", "dense_fmt")]


_TAP_FIELDS = [("logits", ctypes.c_void_p), ("ids", ctypes.c_void_p), ("weights", ctypes.c_void_p),
               ("xq", ctypes.c_void_p), ("z", ctypes.c_void_p), ("zq", ctypes.c_void_p),
               ("h", ctypes.c_void_p), ("hq", ctypes.c_void_p), ("y", ctypes.c_void_p),
               ("ylat", ctypes.c_void_p), ("ylq", ctypes.c_void_p), ("isum_gu", ctypes.c_void_p),
               ("isum_dn", ctypes.c_void_p), ("isum_d", ctypes.c_void_p), ("isum_u", ctypes.c_void_p)]


class Taps(ctypes.Structure):
    _fields_ = _TAP_FIELDS


class Given(ctypes.Structure):
    """Intermediates to evaluate the oracle downstream of (NULL = its own)."""
    _fields_ = [("ids", ctypes.c_void_p), ("zq", ctypes.c_void_p), ("hq", ctypes.c_void_p),
                ("ylq", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_SO)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        L.orc_f16_decode.argtypes = [ctypes.c_uint16]
        L.orc_f16_decode.restype = ctypes.c_double
        L.orc_f16_encode.argtypes = [ctypes.c_double]
        L.orc_f16_encode.restype = ctypes.c_uint16
        L.orc_quantize_q8_1.argtypes = [vp, i32, vp]
        L.orc_quantize_q8_1.restype = None
        L.orc_isum_q8_0.argtypes = [vp, vp]
        L.orc_isum_q8_0.restype = ctypes.c_int32
        L.orc_isum_q4_0.argtypes = [vp, vp]
        L.orc_isum_q4_0.restype = ctypes.c_int32
        L.orc_isum_q5_1.argtypes = [vp, vp]
        L.orc_isum_q5_1.restype = ctypes.c_int32
        L.orc_q5_1_code.argtypes = [vp, i32]
        L.orc_q5_1_code.restype = ctypes.c_int
        L.orc_q4_k_code.argtypes = [vp, i32]
        L.orc_q4_k_code.restype = ctypes.c_int
        L.orc_q4_k_scale_min.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        L.orc_q4_k_scale_min.restype = None
        L.orc_isum_q4_k.argtypes = [vp, i32, vp]
        L.orc_isum_q4_k.restype = ctypes.c_int32
        L.orc_q5_k_code.argtypes = [vp, i32]
        L.orc_q5_k_code.restype = ctypes.c_int
        L.orc_isum_q5_k.argtypes = [vp, i32, vp]
        L.orc_isum_q5_k.restype = ctypes.c_int32
        L.orc_q3_k_code.argtypes = [vp, i32]
        L.orc_q3_k_code.restype = ctypes.c_int
        L.orc_q3_k_scale.argtypes = [vp, i32]
        L.orc_q3_k_scale.restype = ctypes.c_int
        L.orc_isum_q3_k.argtypes = [vp, i32, vp]
        L.orc_isum_q3_k.restype = ctypes.c_int32
        L.orc_e2m1_decode.argtypes = [i32]
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [i32]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_nvfp4_code.argtypes = [vp, i32]
        L.orc_nvfp4_code.restype = ctypes.c_int
        L.orc_isum_nvfp4_half.argtypes = [vp, vp, i32]
        L.orc_isum_nvfp4_half.restype = ctypes.c_int32
        L.orc_row_dot_nvfp4.argtypes = [vp, vp, i32, ctypes.c_double, vp]
        L.orc_row_dot_nvfp4.restype = ctypes.c_float
        L.orc_dequant_weight.argtypes = [i32, vp, i32]
        L.orc_dequant_weight.restype = ctypes.c_double
        L.orc_row_dot.argtypes = [i32, vp, vp, i32, vp]
        L.orc_row_dot.restype = ctypes.c_float
        L.orc_matvec.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.orc_matvec.restype = None
        L.orc_route_token.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp, vp]
        L.orc_route_token.restype = None
        L.orc_expert_ffn.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp, vp]
        L.orc_expert_ffn.restype = None
        L.orc_expert_bytes.argtypes = [ctypes.POINTER(Desc)]
        L.orc_expert_bytes.restype = ctypes.c_size_t
        L.orc_layer_forward.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                        vp, ctypes.POINTER(Taps), i32]
        L.orc_layer_forward.restype = ctypes.c_int
        L.orc_layer_forward_given.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp, vp, vp,
                                              i32, vp, ctypes.POINTER(Taps), ctypes.POINTER(Given),
                                              i32]
        L.orc_layer_forward_given.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def desc_of(w) -> Desc:
    """Oracle descriptor from a workload (any object with the workload's fields)."""
    return Desc(w.hidden, w.n_experts, w.top_k, w.n_ff, w.latent, w.expert_fmt, w.n_groups,
                w.topk_groups, getattr(w, "dense_fmt", 8))


def f16_encode(v: float) -> int:
    return int(lib().orc_f16_encode(float(v)))


def f16_decode(h: int) -> float:
    return float(lib().orc_f16_decode(int(h)))


def quantize_q8_1(v: np.ndarray) -> np.ndarray:
    """float32 [..., n] (n % 32 == 0) -> uint8 [..., n/32, 36] canonical Q8_1 blocks."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    n = v.shape[-1]
    assert n % 32 == 0
    out = np.empty(v.shape[:-1] + (n // 32, Q8_1_BYTES), dtype=np.uint8)
    lib().orc_quantize_q8_1(_p(v), int(v.size), _p(out))
    return out


def isum(fmt: int, wblk: np.ndarray, ablk: np.ndarray) -> int:
    wblk = np.ascontiguousarray(wblk, dtype=np.uint8)
    ablk = np.ascontiguousarray(ablk, dtype=np.uint8)
    f = {Q8_0: lib().orc_isum_q8_0, Q4_0: lib().orc_isum_q4_0, Q5_1: lib().orc_isum_q5_1}[fmt]
    return int(f(_p(wblk), _p(ablk)))


def q4_k_code(sblk: np.ndarray, e: int) -> int:
    sblk = np.ascontiguousarray(sblk, dtype=np.uint8)
    return int(lib().orc_q4_k_code(_p(sblk), e))


def q5_k_code(sblk: np.ndarray, e: int) -> int:
    sblk = np.ascontiguousarray(sblk, dtype=np.uint8)
    return int(lib().orc_q5_k_code(_p(sblk), e))


def isum_q5_k(sblk: np.ndarray, b: int, ablk: np.ndarray) -> int:
    sblk = np.ascontiguousarray(sblk, dtype=np.uint8)
    ablk = np.ascontiguousarray(ablk, dtype=np.uint8)
    return int(lib().orc_isum_q5_k(_p(sblk), b, _p(ablk)))


def q4_k_scale_min(sblk: np.ndarray, b: int):
    sblk = np.ascontiguousarray(sblk, dtype=np.uint8)
    sc, mn = ctypes.c_int(), ctypes.c_int()
    lib().orc_q4_k_scale_min(_p(sblk), b, ctypes.byref(sc), ctypes.byref(mn))
    return sc.value, mn.value


def isum_q4_k(sblk: np.ndarray, b: int, ablk: np.ndarray) -> int:
    sblk = np.ascontiguousarray(sblk, dtype=np.uint8)
    ablk = np.ascontiguousarray(ablk, dtype=np.uint8)
    return int(lib().orc_isum_q4_k(_p(sblk), b, _p(ablk)))


def q3_k_code(sblk: np.ndarray, e: int) -> int:
    sblk = np.ascontiguousarray(sblk, dtype=np.uint8)
    return int(lib().orc_q3_k_code(_p(sblk), e))


def q3_k_scale(sblk: np.ndarray, i: int) -> int:
    sblk = np.ascontiguousarray(sblk, dtype=np.uint8)
    return int(lib().orc_q3_k_scale(_p(sblk), i))


def isum_q3_k(sblk: np.ndarray, b: int, ablk: np.ndarray) -> int:
    sblk = np.ascontiguousarray(sblk, dtype=np.uint8)
    ablk = np.ascontiguousarray(ablk, dtype=np.uint8)
    return int(lib().orc_isum_q3_k(_p(sblk), b, _p(ablk)))


def e2m1(code: int) -> float:
    return float(lib().orc_e2m1_decode(code))


def e4m3(byte: int) -> float:
    return float(lib().orc_e4m3_decode(byte))


def nvfp4_code(wblk: np.ndarray, j: int) -> int:
    wblk = np.ascontiguousarray(wblk, dtype=np.uint8)
    return int(lib().orc_nvfp4_code(_p(wblk), j))


def isum_nvfp4_half(wblk: np.ndarray, ablk: np.ndarray, h: int) -> int:
    wblk = np.ascontiguousarray(wblk, dtype=np.uint8)
    ablk = np.ascontiguousarray(ablk, dtype=np.uint8)
    return int(lib().orc_isum_nvfp4_half(_p(wblk), _p(ablk), h))


def row_dot_nvfp4(row: np.ndarray, act: np.ndarray, nblk: int, tensor_scale: float,
                  with_isum: bool = False):
    row = np.ascontiguousarray(row, dtype=np.uint8)
    act = np.ascontiguousarray(act, dtype=np.uint8)
    tap = np.empty(nblk, dtype=np.int32) if with_isum else None
    y = float(lib().orc_row_dot_nvfp4(_p(row), _p(act), nblk, tensor_scale, _p(tap)))
    return (y, tap) if with_isum else y


def q5_1_code(wblk: np.ndarray, j: int) -> int:
    wblk = np.ascontiguousarray(wblk, dtype=np.uint8)
    return int(lib().orc_q5_1_code(_p(wblk), j))


def dequant_weight(fmt: int, wblk: np.ndarray, j: int) -> float:
    wblk = np.ascontiguousarray(wblk, dtype=np.uint8)
    return float(lib().orc_dequant_weight(fmt, _p(wblk), j))


def matvec(fmt: int, W: np.ndarray, rows: int, nblk: int, act: np.ndarray, with_isum: bool = False):
    """rows outputs of block matrix W ([rows][nblk] canonical) times Q8_1 vector act."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    act = np.ascontiguousarray(act, dtype=np.uint8)
    y = np.empty(rows, dtype=np.float32)
    tap = np.empty((rows, nblk), dtype=np.int32) if with_isum else None
    lib().orc_matvec(fmt, rows, nblk, _p(W), _p(act), _p(y), _p(tap))
    return (y, tap) if with_isum else y


def route_token(w, x: np.ndarray, Wr: np.ndarray, br=None, groups=None):
    d = desc_of(w)
    ids = np.empty(w.top_k, dtype=np.int32)
    wt = np.empty(w.top_k, dtype=np.float32)
    logits = np.empty(w.n_experts, dtype=np.float64)
    lib().orc_route_token(ctypes.byref(d), _p(np.ascontiguousarray(x, np.float32)),
                          _p(np.ascontiguousarray(Wr, np.float32)),
                          _p(None if br is None else np.ascontiguousarray(br, np.float32)),
                          _p(None if groups is None else np.ascontiguousarray(groups, np.int32)),
                          _p(ids), _p(wt), _p(logits))
    return ids, wt, logits


def expert_ffn(w, blob: np.ndarray, aq: np.ndarray, with_isum: bool = False):
    """One expert on one quantised input; returns dict(h, hq, y[, isum_gu, isum_dn])."""
    d = desc_of(w)
    kin, kout, F = w.k_in, w.k_out, w.n_ff
    h = np.empty(F, np.float32)
    hq = np.empty((F // 32, Q8_1_BYTES), np.uint8)
    y = np.empty(kout, np.float32)
    igu = np.empty((2 * F, kin // 32), np.int32) if with_isum else None
    idn = np.empty((kout, F // 32), np.int32) if with_isum else None
    lib().orc_expert_ffn(ctypes.byref(d), _p(np.ascontiguousarray(blob, np.uint8)),
                         _p(np.ascontiguousarray(aq, np.uint8)), _p(h), _p(hq), _p(y), _p(igu),
                         _p(idn))
    r = dict(h=h, hq=hq, y=y)
    if with_isum:
        r.update(isum_gu=igu, isum_dn=idn)
    return r


TAP_NAMES = [n for n, _ in _TAP_FIELDS]


def layer_forward(w, x, router_w, router_b=None, groups=None, experts=None, D=None, U=None,
                  tokens: Optional[Sequence[int]] = None, taps: Sequence[str] = (),
                  nthreads: int = 1, given: Optional[dict] = None):
    """The layer for the given tokens (all when None).

    Returns (out [n][H] float32, dict of the requested taps), everything indexed
    by position in the token list.  ``given`` may hold any of ids [n][k],
    zq [n][L/32][36], hq [n][k][F/32][36] and ylq [n][L/32][36]: the oracle
    then takes these experts / Q8_1 vectors in place of its own selection /
    quantisation and computes everything else as usual.
    """
    d = desc_of(w)
    T = x.shape[0]
    lst = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = T if lst is None else len(lst)
    H, E, k, F, L = w.hidden, w.n_experts, w.top_k, w.n_ff, w.latent
    kin, kout = w.k_in, w.k_out
    shapes = dict(logits=((n, E), np.float64), ids=((n, k), np.int32), weights=((n, k), np.float32),
                  xq=((n, H // 32, 36), np.uint8), z=((n, L), np.float32),
                  zq=((n, L // 32, 36), np.uint8), h=((n, k, F), np.float32),
                  hq=((n, k, F // 32, 36), np.uint8), y=((n, k, kout), np.float32),
                  ylat=((n, L), np.float32), ylq=((n, L // 32, 36), np.uint8),
                  isum_gu=((n, k, 2 * F, kin // 32), np.int32),
                  isum_dn=((n, k, kout, F // 32), np.int32),
                  isum_d=((n, L, H // 32), np.int32), isum_u=((n, H, L // 32), np.int32))
    arrs = {}
    t = Taps()
    for name in taps:
        if name in ("z", "zq", "ylat", "ylq", "isum_d", "isum_u") and not L:
            continue
        shp, dt = shapes[name]
        arrs[name] = np.zeros(shp, dtype=dt)
        setattr(t, name, arrs[name].ctypes.data)
    out = np.empty((n, H), dtype=np.float32)
    gv = Given()
    keep = []
    for name, dt, shp in (("ids", np.int32, (n, k)), ("zq", np.uint8, (n, L // 32, 36)),
                          ("hq", np.uint8, (n, k, F // 32, 36)), ("ylq", np.uint8, (n, L // 32, 36))):
        if given is not None and given.get(name) is not None:
            a = np.ascontiguousarray(given[name], dtype=dt)
            assert a.size == int(np.prod(shp)), (name, a.shape, shp)
            keep.append(a)
            setattr(gv, name, a.ctypes.data)
    rc = lib().orc_layer_forward_given(
        ctypes.byref(d), _p(np.ascontiguousarray(x, np.float32)),
        _p(np.ascontiguousarray(router_w, np.float32)),
        _p(None if router_b is None else np.ascontiguousarray(router_b, np.float32)),
        _p(None if groups is None else np.ascontiguousarray(groups, np.int32)),
        _p(experts), _p(D), _p(U), _p(lst), n, _p(out), ctypes.byref(t), ctypes.byref(gv),
        int(nthreads))
    if rc != 0:
        raise ValueError("oracle refused the layer arguments")
    return out, arrs
