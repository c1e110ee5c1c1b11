"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every function include/moe.h declares, descriptors are validated with named
refusals, the packer round-trips and places blocks where the layout says."""
import ctypes
import os
import re

import numpy as np
import pytest

from quantized_moe_expert_softmax_amd import moe, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    try:
        return moe.lib()
    except (ImportError, OSError) as e:
        pytest.fail(f"libmoe.so does not load: {e}")


def test_exports_match_header(L):
    import glob
    hdr = "".join(open(f).read() for f in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    declared = set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", hdr))
    assert declared == set(moe.EXPORTS), declared ^ set(moe.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert moe.moe_version().startswith("moe-gfx950")


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_descs_valid(L, name):
    w = synth.WORKLOADS[name]
    moe.moe_desc_check(moe.desc_of(w, max_tokens=2048))


def _refused(desc, status, word):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_desc_check(desc)
    assert ei.value.status == status, ei.value
    assert word in ei.value.message, ei.value.message


def test_desc_refusals_name_the_cause(L):
    ok = dict(hidden=512, n_experts=8, top_k=2, n_ff=256, max_tokens=4)
    _refused(moe.make_desc(**{**ok, "expert_fmt": 6}), moe.MOE_EUNSUPPORTED, "expert_fmt")
    _refused(moe.make_desc(**{**ok, "latent": 256, "dense_fmt": 7}), moe.MOE_EUNSUPPORTED, "dense_fmt")
    _refused(moe.make_desc(**{**ok, "hidden": 500}), moe.MOE_EUNSUPPORTED, "hidden")
    _refused(moe.make_desc(**{**ok, "hidden": 0}), moe.MOE_EINVAL, "hidden")
    _refused(moe.make_desc(**{**ok, "n_ff": 384}), moe.MOE_EUNSUPPORTED, "n_ff")
    _refused(moe.make_desc(**{**ok, "top_k": 9}), moe.MOE_EINVAL, "top_k")
    _refused(moe.make_desc(**{**ok, "top_k": 0}), moe.MOE_EINVAL, "top_k")
    _refused(moe.make_desc(**{**ok, "n_experts": 0}), moe.MOE_EINVAL, "n_experts")
    _refused(moe.make_desc(**{**ok, "max_tokens": 0}), moe.MOE_EINVAL, "max_tokens")
    _refused(moe.make_desc(**{**ok, "n_groups": 3, "topk_groups": 1}), moe.MOE_EUNSUPPORTED, "n_groups")
    _refused(moe.make_desc(**{**ok, "n_groups": 4, "topk_groups": 0}), moe.MOE_EINVAL, "topk_groups")
    _refused(moe.make_desc(**{**ok, "n_groups": 4, "topk_groups": 5}), moe.MOE_EINVAL, "topk_groups")
    _refused(moe.make_desc(**{**ok, "n_groups": 8, "topk_groups": 1}), moe.MOE_EINVAL, "top_k")
    _refused(moe.make_desc(**{**ok, "latent": 256, "dense_fmt": 7}), moe.MOE_EUNSUPPORTED, "dense_fmt")
    _refused(moe.make_desc(**{**ok, "latent": 300}), moe.MOE_EUNSUPPORTED, "latent")
    _refused(moe.make_desc(**{**ok, "hidden": 8192 + 256}), moe.MOE_EUNSUPPORTED, "hidden")
    assert L.moe_desc_check(None) == moe.MOE_EINVAL


def test_create_without_gpu_is_a_device_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_create(moe.make_desc(512, 8, 2, 256, max_tokens=4), 0)
    assert ei.value.status == moe.MOE_EDEVICE
    # shape errors are reported before the device is looked at
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_create(moe.make_desc(500, 8, 2, 256, max_tokens=4), 0)
    assert ei.value.status == moe.MOE_EUNSUPPORTED


def test_pack_bytes(L):
    w = synth.WORKLOADS["decode"]
    d = moe.desc_of(w)
    assert moe.moe_pack_bytes(d, moe.MOE_PACK_EXPERTS) == 128 * 20_054_016
    with pytest.raises(moe.MoeError):
        moe.moe_pack_bytes(d, moe.MOE_PACK_D)
    w2 = synth.WORKLOADS["latent_q4"]
    d2 = moe.desc_of(w2)
    assert moe.moe_pack_bytes(d2, moe.MOE_PACK_EXPERTS) == 256 * 3_096_576
    assert moe.moe_pack_bytes(d2, moe.MOE_PACK_D) == 1792 * 224 * 34
    assert moe.moe_pack_bytes(d2, moe.MOE_PACK_U) == 7168 * 56 * 34


def _small(fmt=8, latent=0):
    return synth.Workload("pk", hidden=512, n_experts=3, top_k=2, n_ff=256, tokens=2,
                          latent=latent, expert_fmt=fmt, seed=77)


@pytest.mark.parametrize("fmt,latent", [(8, 0), (2, 0), (7, 0), (12, 0), (13, 0), (11, 0), (40, 0),
                                        (8, 256), (2, 256), (7, 256), (12, 256), (13, 256), (11, 256),
                                        (40, 256)])
def test_pack_roundtrip(L, fmt, latent):
    w = _small(fmt, latent)
    d = moe.desc_of(w)
    ex = synth.gen_experts(w)
    packed = np.empty_like(ex)
    moe.moe_pack_host(d, moe.MOE_PACK_EXPERTS, ex.ctypes.data, packed.ctypes.data)
    assert not np.array_equal(packed, ex)
    back = np.zeros_like(ex)
    moe.moe_unpack_host(d, moe.MOE_PACK_EXPERTS, packed.ctypes.data, back.ctypes.data)
    assert np.array_equal(back, ex)
    if latent:
        D, U = synth.gen_dense(w)
        for which, t in ((moe.MOE_PACK_D, D), (moe.MOE_PACK_U, U)):
            p = np.empty_like(t)
            moe.moe_pack_host(d, which, t.ctypes.data, p.ctypes.data)
            b = np.zeros_like(t)
            moe.moe_unpack_host(d, which, p.ctypes.data, b.ctypes.data)
            assert np.array_equal(b, t)


def test_pack_layout_nvfp4(L):
    """The packed NVFP4 layout: each row's 16-byte code chunks hold element j in the low
    nibble and j + 16 in the high nibble (canonical: 2i low, 2i + 1 high), the two E4M3 scale
    bytes of each block follow all the codes, gate/up rows interleave in 32-row tiles, and the
    expert's 256-byte tail (tensor scales, then zeros) is copied unchanged."""
    w = _small(40)
    d = moe.desc_of(w)
    ex = synth.gen_experts(w)
    packed = np.empty_like(ex)
    moe.moe_pack_host(d, moe.MOE_PACK_EXPERTS, ex.ctypes.data, packed.ctypes.data)
    eb, F, nb = w.expert_bytes, w.n_ff, w.k_in // 32
    rows = 2 * F
    for e in (0, 2):
        c = ex[e * eb:(e + 1) * eb]
        p = packed[e * eb:(e + 1) * eb]
        for prow in (0, 31, 32, 63, 64, 130, rows - 1):
            fb, r = divmod(prow, 64)
            crow = fb * 32 + r if r < 32 else F + fb * 32 + (r - 32)
            for b in (0, nb - 1):
                blk = c[(crow * nb + b) * 18:(crow * nb + b + 1) * 18]
                el = [(blk[2 + i // 2] >> (4 * (i % 2))) & 15 for i in range(32)]
                want = np.array([el[j] | el[j + 16] << 4 for j in range(16)], dtype=np.uint8)
                assert np.array_equal(p[(prow * nb + b) * 16:(prow * nb + b + 1) * 16], want)
                so = rows * nb * 16 + (prow * nb + b) * 2
                assert np.array_equal(p[so:so + 2], blk[:2])
        assert np.array_equal(p[eb - 256:], c[eb - 256:])
        assert np.all(c[eb - 244:] == 0) and np.all(c[eb - 256:eb - 244].view("<f4") > 0)
        assert eb % 256 == 0


@pytest.mark.parametrize("fmt", [8, 2, 7])
def test_pack_layout_positions(L, fmt):
    """Spot-check the documented packed layout: codes of all rows, then each block's side
    data (binary16 d; for Q5_1 d, m and qh); gate/up rows interleaved in 32-row tiles."""
    w = _small(fmt)
    d = moe.desc_of(w)
    ex = synth.gen_experts(w)
    packed = np.empty_like(ex)
    moe.moe_pack_host(d, moe.MOE_PACK_EXPERTS, ex.ctypes.data, packed.ctypes.data)
    bb = {8: 34, 2: 18, 7: 24}[fmt]
    sb = 8 if fmt == 7 else 2
    cb = bb - sb
    F, K = w.n_ff, w.hidden
    nb = K // 32
    e = 2
    blob = ex[e * w.expert_bytes:(e + 1) * w.expert_bytes]
    pk = packed[e * w.expert_bytes:(e + 1) * w.expert_bytes]
    codes_gu = pk[:2 * F * nb * cb]
    scales_gu = pk[2 * F * nb * cb:2 * F * nb * bb]
    for (canon_row, packed_row) in [(0, 0), (31, 31), (F + 0, 32), (F + 31, 63), (32, 64),
                                    (F + 33, 97), (F - 1, 64 * (F // 32 - 1) + 31)]:
        for b in (0, nb - 1, 5):
            cblk = blob[(canon_row * nb + b) * bb:(canon_row * nb + b + 1) * bb]
            assert np.array_equal(codes_gu[(packed_row * nb + b) * cb:(packed_row * nb + b + 1) * cb], cblk[sb:])
            assert np.array_equal(scales_gu[(packed_row * nb + b) * sb:(packed_row * nb + b) * sb + sb], cblk[:sb])
    # down matrix: rows in order
    dn_c = blob[2 * F * nb * bb:]
    dn_p = pk[2 * F * nb * bb:]
    nbf = F // 32
    rows = w.k_out
    for r, b in [(0, 0), (rows - 1, nbf - 1), (17, 3)]:
        cblk = dn_c[(r * nbf + b) * bb:(r * nbf + b + 1) * bb]
        assert np.array_equal(dn_p[(r * nbf + b) * cb:(r * nbf + b + 1) * cb], cblk[sb:])
        off = rows * nbf * cb + (r * nbf + b) * sb
        assert np.array_equal(dn_p[off:off + sb], cblk[:sb])


@pytest.mark.parametrize("fmt", [12, 13])
def test_pack_layout_kquant(L, fmt):
    """K-quant super-blocks pack as 128 code bytes per super-block (row-major codes of all
    rows) and the side data per super-block after them: d, dmin and the 12 scale bytes
    (Q4_K, 16 bytes), and the 32 qh bytes too (Q5_K, 48 bytes)."""
    w = _small(fmt)
    sbb, sd = (144, 16) if fmt == 12 else (176, 48)
    d = moe.desc_of(w)
    ex = synth.gen_experts(w)
    packed = np.empty_like(ex)
    moe.moe_pack_host(d, moe.MOE_PACK_EXPERTS, ex.ctypes.data, packed.ctypes.data)
    F, K = w.n_ff, w.hidden
    nsb = K // 256
    e = 1
    blob = ex[e * w.expert_bytes:(e + 1) * w.expert_bytes]
    pk = packed[e * w.expert_bytes:(e + 1) * w.expert_bytes]
    rows = 2 * F
    for canon_row, packed_row in [(0, 0), (F + 0, 32), (33, 65)]:
        for u in (0, nsb - 1):
            c = blob[(canon_row * nsb + u) * sbb:(canon_row * nsb + u + 1) * sbb]
            assert np.array_equal(pk[(packed_row * nsb + u) * 128:(packed_row * nsb + u + 1) * 128], c[sd:])
            off = rows * nsb * 128 + (packed_row * nsb + u) * sd
            assert np.array_equal(pk[off:off + sd], c[:sd])


def test_pack_layout_q3_k(L):
    """Q3_K super-blocks pack as 108 code bytes (eight 12-byte blocks: two words of 2-bit
    codes, element 16h + 4m + p of word h at bits 8p + 2m, and a word of high bits, element
    4m + p at bit 8p + m; then the 12 scale bytes) and the binary16 d as side data, the same
    110 bytes; the packed codes give back every element's code as the oracle reads it from
    the canonical block."""
    import oracle
    w = _small(11)
    d = moe.desc_of(w)
    ex = synth.gen_experts(w)
    packed = np.empty_like(ex)
    moe.moe_pack_host(d, moe.MOE_PACK_EXPERTS, ex.ctypes.data, packed.ctypes.data)
    F, K = w.n_ff, w.hidden
    nsb = K // 256
    e = 1
    blob = ex[e * w.expert_bytes:(e + 1) * w.expert_bytes]
    pk = packed[e * w.expert_bytes:(e + 1) * w.expert_bytes]
    rows = 2 * F
    for canon_row, packed_row in [(0, 0), (F + 0, 32), (33, 65)]:
        for u in (0, nsb - 1):
            c = blob[(canon_row * nsb + u) * 110:(canon_row * nsb + u + 1) * 110]
            pc = pk[(packed_row * nsb + u) * 108:(packed_row * nsb + u + 1) * 108]
            assert np.array_equal(pc[96:108], c[96:108])
            off = rows * nsb * 108 + (packed_row * nsb + u) * 2
            assert np.array_equal(pk[off:off + 2], c[108:110])
            for b in range(8):
                wd = pc[12 * b:12 * b + 12].view("<u4").astype(np.int64)
                for i in range(32):
                    h, m, p = i // 16, (i % 16) // 4, i % 4
                    lo = (wd[h] >> (8 * p + 2 * m)) & 3
                    hi = (wd[2] >> (8 * p + i // 4)) & 1
                    assert lo + 4 * hi - 4 == oracle.q3_k_code(c, 32 * b + i), (b, i)


def test_forward_argument_checks_without_gpu(L):
    # a NULL layer is refused before anything touches a device
    st = L.moe_layer_forward(None, None, 1, None, None, None, None, None, None, 2, None, None, 0, None)
    assert st == moe.MOE_EINVAL
    ws = ctypes.c_size_t()
    assert L.moe_workspace_bytes(None, 1, ctypes.byref(ws)) == moe.MOE_EINVAL


def test_expert_cache_refusals_without_a_device(L):
    """The expert-cache calls refuse NULL handles by name before touching a device."""
    n = ctypes.c_int(-5)
    arr = (ctypes.c_int32 * 1)(0)
    assert L.moe_expert_cache_admit(None, arr, 1, None, ctypes.byref(n)) == moe.MOE_EINVAL
    assert "cache is NULL" in moe.moe_last_error()
    assert n.value == 0
    s = ctypes.c_int()
    assert L.moe_expert_cache_slot(None, 0, ctypes.byref(s)) == moe.MOE_EINVAL
    out = ctypes.c_void_p(1)
    assert L.moe_expert_cache_create(None, None, None, 0, None, None, ctypes.byref(out)) == moe.MOE_EINVAL
    assert out.value is None
    L.moe_expert_cache_destroy(None)
    assert L.moe_layer_forward_table(None, None, 1, None, None, None, None, None, None, 1, None,
                                     None, 0, None) == moe.MOE_EINVAL


def test_group_labels_check(L):
    """The host validator of the group-label contract: every synthetic workload's labels
    pass; out-of-range labels and unequal groups are refused by name."""
    import numpy as np
    for name, w in synth.WORKLOADS.items():
        moe.moe_group_labels_check(moe.desc_of(w), synth.gen_groups(w))
    d = moe.make_desc(512, 16, 3, 256, n_groups=4, topk_groups=2, max_tokens=4)
    good = np.arange(16, dtype=np.int32) // 4
    moe.moe_group_labels_check(d, good)
    moe.moe_group_labels_check(d, good[::-1].copy())          # any order of equal groups
    bad = good.copy()
    bad[5] = 4
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_group_labels_check(d, bad)
    assert ei.value.status == moe.MOE_EINVAL and "expert 5" in ei.value.message
    bad = good.copy()
    bad[0] = 1                                                  # group 0: 3, group 1: 5
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_group_labels_check(d, bad)
    assert "group 0 holds 3" in ei.value.message
    with pytest.raises(moe.MoeError):
        moe.moe_group_labels_check(d, None)
    with pytest.raises(moe.MoeError):
        moe.moe_group_labels_check(moe.make_desc(512, 16, 3, 256, max_tokens=4), good)


def test_oracle_refuses_what_the_label_check_refuses(L):
    """The oracle's own refusal of unequal groups matches the library's validator."""
    import numpy as np
    import oracle
    w = synth.Workload("g", hidden=256, n_experts=8, top_k=2, n_ff=256, tokens=1, n_groups=4,
                       topk_groups=2, seed=1)
    inp = synth.gen_layer(w)
    bad = inp["groups"].copy()
    bad[0] = 1
    with pytest.raises(moe.MoeError):
        moe.moe_group_labels_check(moe.desc_of(w), bad)
    with pytest.raises(ValueError):
        oracle.layer_forward(w, inp["x"], inp["router_w"], groups=bad, experts=inp["experts"])
    oracle.layer_forward(w, inp["x"], inp["router_w"], groups=inp["groups"], experts=inp["experts"])
