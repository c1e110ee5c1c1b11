"""ctypes binding of libmoe (include/moe.h).  Argument marshalling only: every
step of the layer runs in the library's HIP kernels.

The function names mirror the C ABI.  Device buffers are passed as integer
addresses; ``MoeLayer`` is a small convenience wrapper that keeps the packed
weights and the workspace in torch tensors (torch supplies memory and streams).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EDEVICE, MOE_EHIP, MOE_ENOMEM = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_EUNSUPPORTED", -3: "MOE_EDEVICE",
                -4: "MOE_EHIP", -5: "MOE_ENOMEM"}
MOE_FMT_Q8_0, MOE_FMT_Q4_0, MOE_FMT_Q5_1, MOE_FMT_Q4_K, MOE_FMT_Q5_K, MOE_FMT_Q3_K = 8, 2, 7, 12, 13, 11
MOE_FMT_NVFP4 = 40
MOE_PACK_EXPERTS, MOE_PACK_D, MOE_PACK_U = 0, 1, 2

# every function include/moe.h declares
EXPORTS = ["moe_layer_create", "moe_layer_destroy", "moe_desc_check", "moe_pack_bytes",
           "moe_pack_host", "moe_unpack_host", "moe_pack", "moe_workspace_bytes",
           "moe_layer_forward", "moe_layer_forward_taps", "moe_layer_forward_events",
           "moe_layer_forward_table", "moe_expert_cache_create", "moe_expert_cache_admit",
           "moe_expert_cache_slot", "moe_expert_cache_destroy", "moe_last_error", "moe_version",
           "moe_probe_read", "moe_layer_forward_noalloc", "moe_group_labels_check"]
MOE_NOALLOC_WORKSPACE_BYTES = 64 << 20
MOE_PROBE_NONTEMPORAL = 1
(MOE_EV_BEGIN, MOE_EV_ROUTED, MOE_EV_EXPERT_IN, MOE_EV_GATE_UP, MOE_EV_DOWN, MOE_EV_END,
 MOE_EV_GATE_UP_KSTART, MOE_EV_GATE_UP_KEND) = range(8)
MOE_EV_COUNT = 8


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class moe_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "n_experts", "top_k", "n_ff", "latent", "expert_fmt", "dense_fmt",
        "n_groups", "topk_groups", "max_tokens")]


class moe_taps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "ids", "weights", "xq", "z", "zq", "h", "hq", "y", "ylat", "ylq",
        "isum_gu", "isum_dn", "isum_d", "isum_u")] + [("tap_tokens", ctypes.c_int32)]


_lib = None


def lib():
    """Load libmoe.so; raise if it was not built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m quantized_moe_expert_softmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        P = ctypes.POINTER
        L.moe_desc_check.argtypes = [P(moe_desc)]
        L.moe_layer_create.argtypes = [P(moe_desc), i32, P(vp)]
        L.moe_layer_destroy.argtypes = [vp]
        L.moe_layer_destroy.restype = None
        L.moe_pack_bytes.argtypes = [P(moe_desc), i32, P(sz)]
        L.moe_pack_host.argtypes = [P(moe_desc), i32, vp, vp]
        L.moe_unpack_host.argtypes = [P(moe_desc), i32, vp, vp]
        L.moe_pack.argtypes = [vp, i32, vp, vp, vp]
        L.moe_workspace_bytes.argtypes = [vp, i32, P(sz)]
        fwd = [vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
        L.moe_layer_forward.argtypes = fwd
        L.moe_layer_forward_taps.argtypes = fwd + [P(moe_taps)]
        L.moe_layer_forward_events.argtypes = fwd + [P(vp)]
        L.moe_layer_forward_table.argtypes = fwd
        L.moe_layer_forward_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp]
        L.moe_layer_forward_noalloc.restype = ctypes.c_int
        L.moe_group_labels_check.argtypes = [P(moe_desc), vp]
        L.moe_group_labels_check.restype = ctypes.c_int
        L.moe_expert_cache_create.argtypes = [vp, vp, vp, i32, vp, vp, P(vp)]
        L.moe_expert_cache_admit.argtypes = [vp, P(ctypes.c_int32), i32, vp, P(i32)]
        L.moe_expert_cache_slot.argtypes = [vp, i32, P(i32)]
        L.moe_expert_cache_destroy.argtypes = [vp]
        L.moe_expert_cache_destroy.restype = None
        for f in ("moe_desc_check", "moe_layer_create", "moe_pack_bytes", "moe_pack_host",
                  "moe_unpack_host", "moe_pack", "moe_workspace_bytes", "moe_layer_forward",
                  "moe_layer_forward_taps", "moe_layer_forward_events", "moe_layer_forward_table",
                  "moe_expert_cache_create", "moe_expert_cache_admit", "moe_expert_cache_slot"):
            getattr(L, f).restype = ctypes.c_int
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_version.restype = ctypes.c_char_p
        L.moe_version.argtypes = []
        L.moe_probe_read.argtypes = [vp, sz, i32, i32, i32, vp, vp, vp, vp]
        L.moe_probe_read.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_version() -> str:
    return lib().moe_version().decode()


def make_desc(hidden, n_experts, top_k, n_ff, latent=0, expert_fmt=MOE_FMT_Q8_0,
              dense_fmt=MOE_FMT_Q8_0, n_groups=0, topk_groups=0, max_tokens=1) -> moe_desc:
    return moe_desc(hidden, n_experts, top_k, n_ff, latent, expert_fmt, dense_fmt, n_groups,
                    topk_groups, max_tokens)


def desc_of(w, max_tokens: Optional[int] = None) -> moe_desc:
    """Descriptor of a synthetic workload (see synth.Workload)."""
    return make_desc(w.hidden, w.n_experts, w.top_k, w.n_ff, w.latent, w.expert_fmt,
                     getattr(w, "dense_fmt", MOE_FMT_Q8_0), w.n_groups, w.topk_groups,
                     w.tokens if max_tokens is None else max_tokens)


def moe_desc_check(desc: moe_desc) -> None:
    _check(lib().moe_desc_check(ctypes.byref(desc)))


def moe_layer_create(desc: moe_desc, device: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(lib().moe_layer_create(ctypes.byref(desc), device, ctypes.byref(h)))
    return h.value


def moe_layer_destroy(handle: int) -> None:
    lib().moe_layer_destroy(handle)


def moe_pack_bytes(desc: moe_desc, which: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_pack_bytes(ctypes.byref(desc), which, ctypes.byref(n)))
    return n.value


def moe_pack_host(desc: moe_desc, which: int, canonical_ptr: int, packed_ptr: int) -> None:
    _check(lib().moe_pack_host(ctypes.byref(desc), which, canonical_ptr, packed_ptr))


def moe_unpack_host(desc: moe_desc, which: int, packed_ptr: int, canonical_ptr: int) -> None:
    _check(lib().moe_unpack_host(ctypes.byref(desc), which, packed_ptr, canonical_ptr))


def moe_pack(handle: int, which: int, host_canonical_ptr: int, dev_ptr: int, stream: int = 0) -> None:
    _check(lib().moe_pack(handle, which, host_canonical_ptr, dev_ptr, stream))


def moe_workspace_bytes(handle: int, T: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_bytes(handle, T, ctypes.byref(n)))
    return n.value


def moe_layer_forward(handle, x, T, router_w, router_b, groups, experts, D, U, k, out, workspace,
                      workspace_bytes, stream=0) -> None:
    _check(lib().moe_layer_forward(handle, x, T, router_w, router_b, groups, experts, D, U, k, out,
                                   workspace, workspace_bytes, stream))


def moe_group_labels_check(desc: moe_desc, labels) -> None:
    """Raise unless the host int32 labels (numpy array, or None) meet the layer's
    group contract."""
    import numpy as np
    ptr = None
    if labels is not None:
        labels = np.ascontiguousarray(labels, dtype=np.int32)
        ptr = labels.ctypes.data
    _check(lib().moe_group_labels_check(ctypes.byref(desc), ptr))


def moe_layer_forward_noalloc(handle, x, T, router_w, router_b, groups, experts, D, U, k, out,
                              stream=0) -> None:
    """moe_layer_forward on the library's static per-GPU workspace (no allocation)."""
    _check(lib().moe_layer_forward_noalloc(handle, x, T, router_w, router_b, groups, experts, D, U,
                                           k, out, stream))


def moe_layer_forward_taps(handle, x, T, router_w, router_b, groups, experts, D, U, k, out,
                           workspace, workspace_bytes, stream, taps: moe_taps) -> None:
    _check(lib().moe_layer_forward_taps(handle, x, T, router_w, router_b, groups, experts, D, U, k,
                                        out, workspace, workspace_bytes, stream,
                                        ctypes.byref(taps)))


def moe_layer_forward_events(handle, x, T, router_w, router_b, groups, experts, D, U, k, out,
                             workspace, workspace_bytes, stream, events) -> None:
    """events: sequence of MOE_EV_COUNT hipEvent_t handles (ints) or 0."""
    arr = (ctypes.c_void_p * MOE_EV_COUNT)(*[e or None for e in events])
    _check(lib().moe_layer_forward_events(handle, x, T, router_w, router_b, groups, experts, D, U,
                                          k, out, workspace, workspace_bytes, stream, arr))


def moe_layer_forward_table(handle, x, T, router_w, router_b, groups, expert_table, D, U, k, out,
                            workspace, workspace_bytes, stream=0) -> None:
    """expert_table: device address of n_experts pack addresses."""
    _check(lib().moe_layer_forward_table(handle, x, T, router_w, router_b, groups, expert_table, D,
                                         U, k, out, workspace, workspace_bytes, stream))


def moe_expert_cache_create(handle, host_packs, slots, n_slots, table, stream=0) -> int:
    c = ctypes.c_void_p()
    _check(lib().moe_expert_cache_create(handle, host_packs, slots, n_slots, table, stream,
                                         ctypes.byref(c)))
    return c.value


def moe_expert_cache_admit(cache, experts, stream=0) -> int:
    """experts: iterable of expert ids; returns the number of packs copied."""
    ids = list(experts)
    arr = (ctypes.c_int32 * max(len(ids), 1))(*ids)
    n = ctypes.c_int()
    _check(lib().moe_expert_cache_admit(cache, arr, len(ids), stream, ctypes.byref(n)))
    return n.value


def moe_expert_cache_slot(cache, expert: int) -> int:
    s = ctypes.c_int()
    _check(lib().moe_expert_cache_slot(cache, expert, ctypes.byref(s)))
    return s.value


def moe_expert_cache_destroy(cache) -> None:
    lib().moe_expert_cache_destroy(cache)


def moe_probe_read(buf, nbytes, blocks, unroll, flags, sink, stream=0, ev_start=0,
                   ev_stop=0) -> None:
    """One read-probe launch (include/moe_probe.h); raises on a refused argument."""
    rc = lib().moe_probe_read(buf, nbytes, blocks, unroll, flags, sink, stream, ev_start or None,
                              ev_stop or None)
    if rc != 0:
        raise MoeError(rc, "moe_probe_read refused its arguments or failed to launch")


# ---------------------------------------------------------------------------
class MoeLayer:
    """A layer with its packed weights resident in device memory (torch tensors).

    ``inputs`` holds host numpy arrays: router_w, router_b (or None), groups (or
    None), experts (canonical bytes), D and U (canonical bytes or None).
    """

    def __init__(self, desc: moe_desc, inputs: dict, device: int = 0):
        import torch
        self.torch = torch
        self.desc = desc
        self.device = device
        self.dev = torch.device("cuda", device)
        self.handle = moe_layer_create(desc, device)
        self.k = desc.top_k
        self.router_w = torch.from_numpy(inputs["router_w"]).to(self.dev).contiguous()
        rb = inputs.get("router_b")
        self.router_b = None if rb is None else torch.from_numpy(rb).to(self.dev).contiguous()
        gr = inputs.get("groups")
        self.groups = None if gr is None else torch.from_numpy(gr).to(self.dev).contiguous()
        self.experts = self._pack(MOE_PACK_EXPERTS, inputs["experts"])
        self.D = self._pack(MOE_PACK_D, inputs["D"]) if desc.latent else None
        self.U = self._pack(MOE_PACK_U, inputs["U"]) if desc.latent else None
        self.ws = None
        self.ws_T = -1

    def _pack(self, which, canonical):
        n = moe_pack_bytes(self.desc, which)
        assert canonical.nbytes == n, (canonical.nbytes, n)
        dst = self.torch.empty(n, dtype=self.torch.uint8, device=self.dev)
        stream = self.torch.cuda.current_stream(self.dev).cuda_stream
        moe_pack(self.handle, which, canonical.ctypes.data, dst.data_ptr(), stream)
        return dst

    def workspace(self, T: int):
        need = moe_workspace_bytes(self.handle, T)
        if self.ws is None or self.ws.numel() < need:
            self.ws = self.torch.zeros(need, dtype=self.torch.uint8, device=self.dev)
        return self.ws

    @staticmethod
    def _ptr(t):
        return 0 if t is None else t.data_ptr()

    def forward(self, x, out=None, taps: Optional[moe_taps] = None, stream=None):
        """x: device float32 [T][H]; returns out [T][H] float32 (same device)."""
        torch = self.torch
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.desc.hidden), dtype=torch.float32, device=self.dev)
        ws = self.workspace(T)
        st = (torch.cuda.current_stream(self.dev) if stream is None else stream).cuda_stream
        args = (self.handle, x.data_ptr(), T, self.router_w.data_ptr(), self._ptr(self.router_b),
                self._ptr(self.groups), self.experts.data_ptr(), self._ptr(self.D),
                self._ptr(self.U), self.k, out.data_ptr(), ws.data_ptr(), ws.numel(), st)
        if taps is None:
            moe_layer_forward(*args)
        else:
            moe_layer_forward_taps(*args, taps)
        return out

    def close(self):
        if self.handle:
            moe_layer_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ExpertCache:
    """A layer's experts in pinned host memory with ``n_slots`` of them resident
    in device slots (the library's expert cache); ``forward`` runs the layer
    through the cache's address table.  ``layer`` supplies the router, D/U and
    the layer handle."""

    def __init__(self, layer: "MoeLayer", canonical_experts, n_slots: int):
        torch = layer.torch
        self.layer = layer
        self.torch = torch
        n = moe_pack_bytes(layer.desc, MOE_PACK_EXPERTS)
        assert canonical_experts.nbytes == n, (canonical_experts.nbytes, n)
        self.eb = n // layer.desc.n_experts
        self.host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
        moe_pack_host(layer.desc, MOE_PACK_EXPERTS, canonical_experts.ctypes.data,
                      self.host.data_ptr())
        self.slots = torch.empty(max(n_slots, 1) * self.eb, dtype=torch.uint8, device=layer.dev)
        self.table = torch.zeros(layer.desc.n_experts, dtype=torch.int64, device=layer.dev)
        st = torch.cuda.current_stream(layer.dev).cuda_stream
        self.handle = moe_expert_cache_create(layer.handle, self.host.data_ptr(),
                                              self.slots.data_ptr(), n_slots,
                                              self.table.data_ptr(), st)

    def admit(self, experts, stream=None) -> int:
        st = (self.torch.cuda.current_stream(self.layer.dev) if stream is None else stream).cuda_stream
        return moe_expert_cache_admit(self.handle, [int(e) for e in experts], st)

    def slot(self, expert: int) -> int:
        return moe_expert_cache_slot(self.handle, expert)

    def forward(self, x, out=None, stream=None):
        L, torch = self.layer, self.torch
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, L.desc.hidden), dtype=torch.float32, device=L.dev)
        ws = L.workspace(T)
        st = (torch.cuda.current_stream(L.dev) if stream is None else stream).cuda_stream
        moe_layer_forward_table(L.handle, x.data_ptr(), T, L.router_w.data_ptr(), L._ptr(L.router_b),
                                L._ptr(L.groups), self.table.data_ptr(), L._ptr(L.D), L._ptr(L.U),
                                L.k, out.data_ptr(), ws.data_ptr(), ws.numel(), st)
        return out

    def close(self):
        if self.handle:
            moe_expert_cache_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
