// Host side of libmoe: the C ABI declared in include/moe.h.
//
// Validation follows the pages' boundary conventions (Strata "Q8 0 support",
// K-quant follow-up commit: an unsupported (gate/up format, down format, dims)
// combination is refused by name at start-up, and an unknown type is refused
// rather than leaving an output unwritten; Strata PR 24: launchers refuse an
// unsupported device).  Every refusal returns a status and leaves a message
// for moe_last_error().
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "kernels.h"
#include "moe_internal.h"

using namespace moe;

struct moe_layer {
    moe_desc desc;
    Dims dims;
    int device;
};

static thread_local std::string g_err;

static moe_status fail(moe_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

static moe_status hip_fail(hipError_t e, const char* what) {
    return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// The device made current for the lifetime of the object (the caller's again after).
struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        int cur;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

extern "C" const char* moe_last_error(void) { return g_err.c_str(); }
extern "C" const char* moe_version(void) { return "moe-gfx950 0.1"; }

static bool mult(int v, int m) { return v > 0 && v % m == 0; }

extern "C" moe_status moe_desc_check(const moe_desc* d) {
    if (!d) return fail(MOE_EINVAL, "desc is NULL");
    if (d->expert_fmt != MOE_FMT_Q8_0 && d->expert_fmt != MOE_FMT_Q4_0 &&
        d->expert_fmt != MOE_FMT_Q5_1 && !kquant(d->expert_fmt) && d->expert_fmt != MOE_FMT_NVFP4)
        return fail(MOE_EUNSUPPORTED,
                    "expert_fmt %d is none of Q8_0 (8), Q4_0 (2), Q5_1 (7), Q4_K (12), Q5_K (13), "
                    "Q3_K (11), NVFP4 (40)",
                    d->expert_fmt);
    // edge0-strata README, changes from upstream Strata: the latent D/U
    // projections come in Q8 or Q4 (the Q4 rows kernel there is Q4_0 x Q8_1)
    if (d->latent && d->dense_fmt != MOE_FMT_Q8_0 && d->dense_fmt != MOE_FMT_Q4_0)
        return fail(MOE_EUNSUPPORTED, "dense_fmt %d is neither Q8_0 (8) nor Q4_0 (2)", d->dense_fmt);
    if (!mult(d->hidden, 256) || d->hidden > 8192)
        return fail(d->hidden <= 0 ? MOE_EINVAL : MOE_EUNSUPPORTED,
                    "hidden %d must be a positive multiple of 256, at most 8192", d->hidden);
    if (!mult(d->n_ff, 256) || d->n_ff > 8192)
        return fail(d->n_ff <= 0 ? MOE_EINVAL : MOE_EUNSUPPORTED,
                    "n_ff %d must be a positive multiple of 256, at most 8192", d->n_ff);
    if (d->latent != 0 && (!mult(d->latent, 256) || d->latent > 8192))
        return fail(d->latent < 0 ? MOE_EINVAL : MOE_EUNSUPPORTED,
                    "latent %d must be 0 or a positive multiple of 256, at most 8192", d->latent);
    if (d->n_experts < 1 || d->n_experts > 512)
        return fail(MOE_EINVAL, "n_experts %d out of range 1..512", d->n_experts);
    if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > 32)
        return fail(MOE_EINVAL, "top_k %d out of range 1..min(n_experts=%d, 32)", d->top_k,
                    d->n_experts);
    if (d->n_groups < 0) return fail(MOE_EINVAL, "n_groups %d is negative", d->n_groups);
    if (d->n_groups > 0) {
        if (d->n_groups > 64 || d->n_experts % d->n_groups)
            return fail(MOE_EUNSUPPORTED, "n_groups %d must divide n_experts %d and be at most 64",
                        d->n_groups, d->n_experts);
        if (d->topk_groups < 1 || d->topk_groups > d->n_groups)
            return fail(MOE_EINVAL, "topk_groups %d out of range 1..n_groups=%d", d->topk_groups,
                        d->n_groups);
        if (d->topk_groups * (d->n_experts / d->n_groups) < d->top_k)
            return fail(MOE_EINVAL, "topk_groups %d x %d experts per group < top_k %d",
                        d->topk_groups, d->n_experts / d->n_groups, d->top_k);
    }
    if (d->max_tokens < 1 || d->max_tokens > 65536)
        return fail(MOE_EINVAL, "max_tokens %d out of range 1..65536", d->max_tokens);
    const int kin = d->latent ? d->latent : d->hidden;
    if (!mv_config_ok(kin, d->expert_fmt, true))
        return fail(MOE_EUNSUPPORTED, "no gate/up kernel for %d-wide %s rows", kin,
                    d->expert_fmt == MOE_FMT_Q4_0   ? "Q4_0"
                    : d->expert_fmt == MOE_FMT_Q5_1 ? "Q5_1"
                    : d->expert_fmt == MOE_FMT_Q4_K ? "Q4_K"
                    : d->expert_fmt == MOE_FMT_Q5_K ? "Q5_K"
                    : d->expert_fmt == MOE_FMT_Q3_K ? "Q3_K"
                    : d->expert_fmt == MOE_FMT_NVFP4 ? "NVFP4"
                                                    : "Q8_0");
    if (!mv_config_ok(d->n_ff, d->expert_fmt, false))
        return fail(MOE_EUNSUPPORTED, "no down kernel for %d-wide rows", d->n_ff);
    if (d->latent && (!mv_config_ok(d->hidden, d->dense_fmt, false) ||
                      !mv_config_ok(d->latent, d->dense_fmt, false)))
        return fail(MOE_EUNSUPPORTED, "no D/U kernel for hidden %d, latent %d", d->hidden,
                    d->latent);
    g_err.clear();
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// The workspace of moe_layer_forward_noalloc: one file-scope device array, of
// which every GPU the library runs on holds its own copy until the process
// ends.  Host code never passes `scratch` itself to a kernel or a copy (in host
// code it names a host-side stand-in): its device address on each GPU comes
// from hipGetSymbolAddress, once per device, at moe_layer_create.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_WORKSPACE_BYTES];

static const int SCRATCH_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch[SCRATCH_MAX_DEVICES] = {};

// With `device` current: look up that GPU's copy of `scratch` and zero it (the
// workspace contract: zero before first use; every call leaves its counters at
// zero again).
static moe_status scratch_init(int device) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (device < 0 || device >= SCRATCH_MAX_DEVICES)
        return fail(MOE_EDEVICE, "device %d beyond the %d the static workspace supports", device,
                    SCRATCH_MAX_DEVICES);
    if (g_scratch[device]) return MOE_OK;
    DeviceGuard g(device);
    if (!g.ok) return fail(MOE_EDEVICE, "cannot select device %d", device);
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress of the static workspace");
    e = hipMemset(p, 0, MOE_NOALLOC_WORKSPACE_BYTES);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "zeroing the static workspace");
    g_scratch[device] = p;
    return MOE_OK;
}

extern "C" moe_status moe_layer_create(const moe_desc* desc, int device, moe_layer** out) {
    if (!out) return fail(MOE_EINVAL, "out is NULL");
    *out = nullptr;
    moe_status s = moe_desc_check(desc);
    if (s != MOE_OK) return s;
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n == 0) return fail(MOE_EDEVICE, "no HIP device available");
    if (device < 0 || device >= n)
        return fail(MOE_EDEVICE, "device %d out of range (%d devices)", device, n);
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, device);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
        return fail(MOE_EDEVICE, "device %d is %s; the kernels are built for gfx950 only", device,
                    p.gcnArchName);
    s = scratch_init(device);
    if (s != MOE_OK) return s;
    moe_layer* L = new moe_layer;
    L->desc = *desc;
    L->dims = make_dims(*desc);
    L->device = device;
    *out = L;
    return MOE_OK;
}

extern "C" void moe_layer_destroy(moe_layer* layer) { delete layer; }

// ---------------------------------------------------------------------------
// packing

static moe_status tensor_bytes(const moe_desc* d, int which, size_t* bytes, Dims* dims) {
    moe_status s = moe_desc_check(d);
    if (s != MOE_OK) return s;
    Dims m = make_dims(*d);
    if (dims) *dims = m;
    switch (which) {
        case MOE_PACK_EXPERTS: *bytes = (size_t)m.E * m.expert_bytes; return MOE_OK;
        case MOE_PACK_D:
        case MOE_PACK_U:
            if (!m.L) return fail(MOE_EINVAL, "D/U requested for a layer with latent == 0");
            *bytes = which == MOE_PACK_D ? m.D.bytes() : m.U.bytes();
            return MOE_OK;
        default: return fail(MOE_EINVAL, "unknown tensor %d", which);
    }
}

extern "C" moe_status moe_pack_bytes(const moe_desc* d, int which, size_t* bytes) {
    if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
    return tensor_bytes(d, which, bytes, nullptr);
}

// Canonical row index of packed row p of a block matrix.
typedef int (*RowMap)(int p, int F);
static int identity_row(int p, int) { return p; }
static int gate_up_row(int p, int F) {
    int fb = p / 64, r = p % 64;
    return r < 32 ? fb * 32 + r : F + fb * 32 + (r - 32);
}

// Q3_K super-block (canonical: hmask[32], qs[64], scales[12], binary16 d) <->
// packed codes (eight 12-byte blocks + the 12 scale bytes) and side (d).  The
// canonical element e = 128*half + 32*j + l has its two low bits at bits 2j of
// qs[32*half + l] and its high bit at bit 4*half + j of hmask[l]; packed block
// b, element i = 16h + 4m + p (word h) and i = 4m + p (high-bit word).
static void q3_k_to_packed(const uint8_t* c, uint8_t* codes, uint8_t* side) {
    for (int b = 0; b < 8; ++b) {
        uint32_t w[3] = {0u, 0u, 0u};
        for (int i = 0; i < 32; ++i) {
            const int e = 32 * b + i, half = e / 128, j = (e % 128) / 32, l = e % 32;
            const uint32_t lo = (c[32 + 32 * half + l] >> (2 * j)) & 3u;
            const uint32_t hi = (c[l] >> (4 * half + j)) & 1u;
            const int h = i / 16, m = (i % 16) / 4, p = i % 4;
            w[h] |= lo << (8 * p + 2 * m);
            w[2] |= hi << (8 * p + i / 4);
        }
        for (int k = 0; k < 3; ++k)
            for (int t = 0; t < 4; ++t) codes[12 * b + 4 * k + t] = (uint8_t)(w[k] >> (8 * t));
    }
    memcpy(codes + 96, c + 96, 12);
    memcpy(side, c + 108, 2);
}

static void q3_k_to_canonical(const uint8_t* codes, const uint8_t* side, uint8_t* c) {
    memset(c, 0, 96);
    for (int b = 0; b < 8; ++b) {
        uint32_t w[3];
        for (int k = 0; k < 3; ++k)
            w[k] = (uint32_t)codes[12 * b + 4 * k] | (uint32_t)codes[12 * b + 4 * k + 1] << 8 |
                   (uint32_t)codes[12 * b + 4 * k + 2] << 16 | (uint32_t)codes[12 * b + 4 * k + 3] << 24;
        for (int i = 0; i < 32; ++i) {
            const int e = 32 * b + i, half = e / 128, j = (e % 128) / 32, l = e % 32;
            const int h = i / 16, m = (i % 16) / 4, p = i % 4;
            const uint32_t lo = (w[h] >> (8 * p + 2 * m)) & 3u;
            const uint32_t hi = (w[2] >> (8 * p + i / 4)) & 1u;
            c[32 + 32 * half + l] |= (uint8_t)(lo << (2 * j));
            c[l] |= (uint8_t)(hi << (4 * half + j));
        }
    }
    memcpy(c + 96, codes + 96, 12);
    memcpy(c + 108, side, 2);
}

// One matrix: canonical blocks (rows in canonical order) <-> packed codes/scales.
static void convert_matrix(const MatLayout& M, RowMap map, int F, const uint8_t* canon,
                           uint8_t* packed, bool to_packed) {
    // canonical units ([side data][codes], Q3_K: its own block) of ub blocks of 32
    const int nu = (int)M.units();
    const int bb = unit_bytes(M.fmt), cb = unit_code_bytes(M.fmt), sb = unit_side_bytes(M.fmt);
    uint8_t* codes = packed + M.codes_off;
    uint8_t* scales = packed + M.scales_off;
    for (int p = 0; p < M.rows; ++p) {
        const int r = map(p, F);
        for (int b = 0; b < nu; ++b) {
            const size_t cpos = ((size_t)r * nu + b) * bb;
            const size_t ppos = ((size_t)p * nu + b);
            uint8_t* c = const_cast<uint8_t*>(canon) + cpos;
            if (M.fmt == MOE_FMT_Q3_K) {
                if (to_packed)
                    q3_k_to_packed(c, codes + ppos * cb, scales + sb * ppos);
                else
                    q3_k_to_canonical(codes + ppos * cb, scales + sb * ppos, c);
            } else if (M.fmt == MOE_FMT_NVFP4) {
                // canonical byte 2 + i: elements 2i (low nibble), 2i + 1 (high);
                // packed byte j: elements j (low), j + 16 (high), as Q4_0
                uint8_t* pc = codes + ppos * cb;
                if (to_packed) {
                    memcpy(scales + sb * ppos, c, 2);
                    for (int j = 0; j < 16; ++j) {
                        const int lo = (c[2 + j / 2] >> (4 * (j & 1))) & 15;
                        const int hi = (c[2 + (j + 16) / 2] >> (4 * (j & 1))) & 15;
                        pc[j] = (uint8_t)(lo | hi << 4);
                    }
                } else {
                    memcpy(c, scales + sb * ppos, 2);
                    for (int i = 0; i < 16; ++i) {
                        const int e0 = 2 * i, e1 = 2 * i + 1;
                        const int c0 = e0 < 16 ? pc[e0] & 15 : pc[e0 - 16] >> 4;
                        const int c1 = e1 < 16 ? pc[e1] & 15 : pc[e1 - 16] >> 4;
                        c[2 + i] = (uint8_t)(c0 | c1 << 4);
                    }
                }
            } else if (to_packed) {
                memcpy(scales + sb * ppos, c, sb);
                memcpy(codes + ppos * cb, c + sb, cb);
            } else {
                memcpy(c, scales + sb * ppos, sb);
                memcpy(c + sb, codes + ppos * cb, cb);
            }
        }
    }
}

static void convert_expert(const Dims& m, const uint8_t* canon, uint8_t* packed, bool to_packed) {
    convert_matrix(m.gu, gate_up_row, m.F, canon, packed, to_packed);
    convert_matrix(m.dn, identity_row, m.F, canon + m.gu.bytes(), packed + m.dn_off, to_packed);
    if (m.ts_off) {
        // NVFP4 tensor scales: the same 256-byte tail in both forms
        if (to_packed)
            memcpy(packed + m.ts_off, canon + m.ts_off, 256);
        else
            memcpy(const_cast<uint8_t*>(canon) + m.ts_off, packed + m.ts_off, 256);
    }
}

static moe_status convert(const moe_desc* d, int which, const void* src, void* dst, bool to_packed) {
    size_t bytes;
    Dims m;
    moe_status s = tensor_bytes(d, which, &bytes, &m);
    if (s != MOE_OK) return s;
    if (!src || !dst) return fail(MOE_EINVAL, "NULL buffer");
    const uint8_t* canon = (const uint8_t*)(to_packed ? src : dst);
    uint8_t* packed = (uint8_t*)(to_packed ? dst : (void*)src);
    if (which == MOE_PACK_EXPERTS) {
        for (int e = 0; e < m.E; ++e)
            convert_expert(m, canon + (size_t)e * m.expert_bytes, packed + (size_t)e * m.expert_bytes,
                           to_packed);
    } else {
        convert_matrix(which == MOE_PACK_D ? m.D : m.U, identity_row, 0, canon, packed, to_packed);
    }
    return MOE_OK;
}

extern "C" moe_status moe_pack_host(const moe_desc* d, int which, const void* canonical,
                                    void* packed) {
    return convert(d, which, canonical, packed, true);
}

extern "C" moe_status moe_unpack_host(const moe_desc* d, int which, const void* packed,
                                      void* canonical) {
    return convert(d, which, packed, canonical, false);
}

namespace {
}  // namespace

extern "C" moe_status moe_pack(const moe_layer* L, int which, const void* host_canonical,
                               void* dev_dst, void* stream) {
    if (!L) return fail(MOE_EINVAL, "layer is NULL");
    if (!host_canonical || !dev_dst) return fail(MOE_EINVAL, "NULL buffer");
    size_t bytes;
    Dims m;
    moe_status s = tensor_bytes(&L->desc, which, &bytes, &m);
    if (s != MOE_OK) return s;
    DeviceGuard g(L->device);
    if (!g.ok) return fail(MOE_EDEVICE, "cannot select device %d", L->device);
    hipStream_t st = (hipStream_t)stream;
    const uint8_t* src = (const uint8_t*)host_canonical;
    uint8_t* dst = (uint8_t*)dev_dst;
    size_t chunk = which == MOE_PACK_EXPERTS ? m.expert_bytes : bytes;
    std::vector<uint8_t> stage;
    try {
        stage.resize(chunk);
    } catch (...) {
        return fail(MOE_ENOMEM, "host staging of %zu bytes failed", chunk);
    }
    for (size_t off = 0; off < bytes; off += chunk) {
        if (which == MOE_PACK_EXPERTS)
            convert_expert(m, src + off, stage.data(), true);
        else
            convert_matrix(which == MOE_PACK_D ? m.D : m.U, identity_row, 0, src, stage.data(), true);
        hipError_t e = hipMemcpyAsync(dst + off, stage.data(), chunk, hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, "copy of packed weights");
    }
    return MOE_OK;
}

extern "C" moe_status moe_group_labels_check(const moe_desc* d, const int32_t* labels) {
    moe_status s = moe_desc_check(d);
    if (s != MOE_OK) return s;
    if (d->n_groups == 0) {
        if (labels) return fail(MOE_EINVAL, "labels given for a layer with n_groups == 0");
        return MOE_OK;
    }
    if (!labels) return fail(MOE_EINVAL, "n_groups %d needs labels", d->n_groups);
    std::vector<int> count(d->n_groups, 0);
    for (int e = 0; e < d->n_experts; ++e) {
        if (labels[e] < 0 || labels[e] >= d->n_groups)
            return fail(MOE_EINVAL, "label %d of expert %d outside 0..%d", labels[e], e,
                        d->n_groups - 1);
        ++count[labels[e]];
    }
    const int per = d->n_experts / d->n_groups;
    for (int g = 0; g < d->n_groups; ++g)
        if (count[g] != per)
            return fail(MOE_EINVAL, "group %d holds %d experts, not E / n_groups = %d", g,
                        count[g], per);
    g_err.clear();
    return MOE_OK;
}

extern "C" moe_status moe_workspace_bytes(const moe_layer* L, int T, size_t* bytes) {
    if (!L || !bytes) return fail(MOE_EINVAL, "NULL argument");
    if (T < 0 || T > L->desc.max_tokens)
        return fail(MOE_EINVAL, "T %d out of range 0..max_tokens=%d", T, L->desc.max_tokens);
    *bytes = ws_layout(L->dims, std::max(T, 1)).total;
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// forward

// Decode sizes run the down projection per token with the combine fused;
// larger T runs it per expert bucket and combines afterwards.  For K-quant
// experts (whose per-token kernel stages the token's rows in LDS) the fused
// form stops at 6 tokens; measured on one box against the per-bucket kernel,
// us per layer: Q3_K T = 1 42.1 -> 37.9, T = 2 63.7 -> 57.9; Q4_K T = 2
// 67.5 -> 61.4, T = 4 108.0 -> 104.5; T = 6 Q5_K 174.2 -> 171.4, latent Q3_K
// 132.7 -> 127.6, Q3_K 132.5 -> 133.6; Q4_K T = 8 171.9 -> 177.3.
static const int DOWN_TOK_MAX_T = 8;
static const int DOWN_TOK_KQ_MAX_T = 6;
// (the Q8_1(y_lat) arrival counters of the per-token down kernel cover DECODE_T tokens)
static_assert(DOWN_TOK_MAX_T <= DECODE_T && DOWN_TOK_KQ_MAX_T <= DECODE_T, "arrival counters");

static moe_status forward_impl(const moe_layer* L, const float* x, int T, const float* router_w,
                               const float* router_b, const int32_t* groups, ExpertSrc ex,
                               const void* Dp, const void* Up, int k, float* out, void* workspace,
                               size_t ws_bytes, void* stream, const moe_taps* taps,
                               void* const* events) {
    if (!L) return fail(MOE_EINVAL, "layer is NULL");
    const Dims& m = L->dims;
    if (k != m.k) return fail(MOE_EINVAL, "k %d differs from the layer's top_k %d", k, m.k);
    if (T < 0 || T > m.max_tokens)
        return fail(MOE_EINVAL, "T %d out of range 0..max_tokens=%d", T, m.max_tokens);
    if (T == 0) return MOE_OK;
    if (!x || !router_w || !(ex.base || ex.table) || !out || !workspace)
        return fail(MOE_EINVAL, "NULL x, router_w, expert packs (or table), out or workspace");
    if (m.L && (!Dp || !Up)) return fail(MOE_EINVAL, "latent layer needs D and U");
    if (m.G && !groups) return fail(MOE_EINVAL, "n_groups %d needs group_of_expert", m.G);
    const WsLayout w = ws_layout(m, T);
    if (ws_bytes < w.total)
        return fail(MOE_ENOMEM, "workspace of %zu bytes < %zu needed for T=%d", ws_bytes, w.total, T);
    DeviceGuard g(L->device);
    if (!g.ok) return fail(MOE_EDEVICE, "cannot select device %d", L->device);

    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    const int A = T * m.k;
    ActPtr xq{(int8_t*)(ws + w.xq_q), (uint32_t*)(ws + w.xq_ds), (int32_t*)(ws + w.xq_sq)};
    ActPtr zq{(int8_t*)(ws + w.zq_q), (uint32_t*)(ws + w.zq_ds), (int32_t*)(ws + w.zq_sq)};
    ActPtr hq{(int8_t*)(ws + w.hq_q), (uint32_t*)(ws + w.hq_ds), (int32_t*)(ws + w.hq_sq)};
    ActPtr ylq{(int8_t*)(ws + w.ylq_q), (uint32_t*)(ws + w.ylq_ds), (int32_t*)(ws + w.ylq_sq)};
    float* z = (float*)(ws + w.z);
    float* y = (float*)(ws + w.y);
    float* ylat = (float*)(ws + w.ylat);
    Buckets b;
    b.ctrl = (const uint32_t*)(ws + w.ctrl);
    b.active = (const int32_t*)(ws + w.active);
    b.counts = (const int32_t*)(ws + w.counts);
    b.lists = (const int32_t*)(ws + w.lists);
    b.tile_start = (const int32_t*)(ws + w.tile_start);
    b.ids = (const int32_t*)(ws + w.ids);
    b.wts = (const float*)(ws + w.wts);
    Taps tp;
    if (taps) {
        tp.h = taps->h;
        tp.isum_gu = taps->isum_gu;
        tp.isum_dn = taps->isum_dn;
        tp.isum_d = taps->isum_d;
        tp.isum_u = taps->isum_u;
        tp.tap_tokens = std::min(std::max(taps->tap_tokens, 0), T);
        if (!tp.isum_gu && !tp.isum_dn && !tp.isum_d && !tp.isum_u) tp.tap_tokens = 0;
    }
    const bool down_tok = T <= (kquant(m.fmt) ? DOWN_TOK_KQ_MAX_T : DOWN_TOK_MAX_T);
    // many tokens: grouped matrix-core GEMMs over token tiles
    const bool dense_gemm = T > MV_MAX_T;     // the latent D/U
    const bool gemm = dense_gemm;             // the experts
    // latent rows of a single token are quantised by each consumer workgroup as
    // it stages them (no extra launch); with more tokens every workgroup would
    // repeat that work, so z and y_lat are quantised once by their own kernel
    const bool lat_fused_q = T <= LAT_FUSED_Q_MAX_T;
    // a few tokens: the latent D and U on the few-token matrix-core kernel
    // (measured on MI355X against the matrix-vector kernels, us per stage:
    // latent Q4_0 experts at T = 32, D 75 -> 17 and U 42 -> 15; latent Q8_0
    // experts at T = 6, D 15 -> 12 and U 10 -> 8)
    const bool thin = m.L && !dense_gemm && T >= THIN_MIN_T && dense_thin_ok(m.D, T) && dense_thin_ok(m.U, T);
    if (taps && down_tok) tp.y = taps->y;
    const ActPtr none{nullptr, nullptr, nullptr};

    hipError_t e;
#define CK(call, what)                                  \
    do {                                                \
        e = (call);                                     \
        if (e != hipSuccess) return hip_fail(e, what);  \
    } while (0)
#define EV(i)                                                                          \
    do {                                                                               \
        if (events && events[i]) CK(hipEventRecord((hipEvent_t)events[i], st), "event"); \
    } while (0)

    EV(MOE_EV_BEGIN);
    RouteDone routed;
    SelectArgs sel;
    // 2 to DECODE_T tokens whose down projection runs per token: no buckets;
    // the gate/up kernel takes its expert and tokens from the routing ids
    const bool ids_only = T >= 2 && T <= DECODE_T && down_tok;
    // ... and in a latent layer those tokens are selected by T more workgroups
    // of the few-token D launch, which does not depend on the routing
    const bool sel_in_thin = ids_only && thin;
    CK(launch_router(m, w, ws, x, T, router_w, router_b, groups, taps ? taps->logits : nullptr, xq,
                     ids_only, sel_in_thin, &routed, &sel, st), "router");
    if (routed == ROUTE_SELECTED) CK(launch_bucket(m, w, ws, T, st), "bucketing");
    RouteOut rout{(int32_t*)(ws + w.ids), (float*)(ws + w.wts), (int32_t*)(ws + w.counts),
                  (int32_t*)(ws + w.lists), (uint32_t*)(ws + w.ctrl), (int32_t*)(ws + w.active)};
    // a single token is selected and bucketed by one more workgroup of the
    // latent D launch, which does not depend on the routing and runs between
    // the router and the experts; without D, by the gate/up kernel's prologue
    const bool sel_in_d = routed == ROUTE_LOGITS && m.L && !dense_gemm && !thin;
    const SelectArgs* gu_route = routed == ROUTE_LOGITS && !sel_in_d ? &sel : nullptr;
    EV(MOE_EV_ROUTED);
    const int32_t* tile_map = (const int32_t*)(ws + w.tile_map);
    if (m.L) {
        // z = D . Q8_1(x), fp32
        if (dense_gemm) {
            CK(launch_dense_mfma(m.D, (const uint8_t*)Dp, T, xq, z, tp.isum_d, tp.tap_tokens, st), "D");
            CK(launch_quant_rows(z, T, m.L, zq, st), "Q8_1(z)");
        } else if (thin) {
            // K-sliced partial rows, added in slice order by the quantisation
            const int S = thin_splits(m.L, m.H / QK);
            float* zp = S > 1 ? (float*)(ws + w.dpart) : z;
            CK(launch_dense_thin(m.D, (const uint8_t*)Dp, T, xq, zp, S, tp.isum_d, tp.tap_tokens, st,
                                 routed == ROUTE_DEFERRED ? &sel : nullptr, (int32_t*)(ws + w.ids),
                                 (float*)(ws + w.wts)), "D");
            CK(launch_quant_rows_sum(zp, S, S > 1 ? z : nullptr, T, m.L, zq, st), "Q8_1(z)");
        } else {
            CK(launch_dense_mv(m.D, (const uint8_t*)Dp, T, xq, nullptr, none, z, tp.isum_d,
                               tp.tap_tokens, st, sel_in_d ? &sel : nullptr, &rout, m.k), "D");
            // one token: the gate/up kernel quantises z on the way in; more: once, here
            if (!lat_fused_q) CK(launch_quant_rows(z, T, m.L, zq, st), "Q8_1(z)");
        }
    }
    EV(MOE_EV_EXPERT_IN);
    KEvents gev;
    if (events) {
        gev.start = (hipEvent_t)events[MOE_EV_GATE_UP_KSTART];
        gev.stop = (hipEvent_t)events[MOE_EV_GATE_UP_KEND];
    }
    if (gemm)
        CK(launch_gate_up_mfma(m, T, ex, m.L ? zq : xq, b, tile_map, hq, tp, st, gev), "gate/up");
    else if (m.L && lat_fused_q)
        CK(launch_gate_up_mv(m, T, ex, none, z, taps ? zq : none, b, hq, tp, st, gev, gu_route, &rout,
                             false, sel_in_d),
           "gate/up");
    else if (m.L)
        CK(launch_gate_up_mv(m, T, ex, zq, nullptr, none, b, hq, tp, st, gev, gu_route, &rout,
                             routed == ROUTE_IDS || routed == ROUTE_DEFERRED),
           "gate/up");
    else
        CK(launch_gate_up_mv(m, T, ex, xq, nullptr, none, b, hq, tp, st, gev, gu_route, &rout,
                             routed == ROUTE_IDS || routed == ROUTE_DEFERRED),
           "gate/up");
    EV(MOE_EV_GATE_UP);
    float* comb = m.L ? ylat : out;     // the combined expert outputs
    // a latent layer whose down projection runs per token (array form): that
    // kernel also writes Q8_1(y_lat), in 32-row tiles, for the U projection
    const bool ylq_in_down = m.L && down_tok && !ex.table;
    if (down_tok) {
        // (one token: 16-row tiles that hand each Q8_1(y_lat) block to its second
        // finisher, twice the workgroups of 32-row tiles; measured on one box, us
        // per layer: latent_q8 40.6 -> 38.9, latent_q3_k 48.2 -> 46.9, latent_q4
        // 43.3 -> 43.1.  At six tokens 32-row tiles already fill the chip and the
        // hand-off cost 3-3.5 us, so from two tokens on the tiles are 32 rows.)
        CK(launch_down_tok_mv(m, T, ex, hq, b, comb, tp, st, ylq_in_down ? ylq : none,
                              ylq_in_down && T == 1 ? (uint32_t*)(ws + w.yarrive) : nullptr),
           "down+combine");
    } else {
        if (gemm)
            CK(launch_down_mfma(m, T, ex, hq, b, tile_map, y, tp, st), "down");
        else
            CK(launch_down_slot_mv(m, T, ex, hq, b, y, tp, st), "down");
        // a latent layer's combine also quantises y_lat for the U projection
        if (m.L)
            CK(launch_combine_q(y, b.wts, T, m.k, m.kout, comb, ylq, st), "combine+Q8_1");
        else
            CK(launch_combine(y, b.wts, T, m.k, m.kout, comb, st), "combine");
    }
    EV(MOE_EV_DOWN);
    if (m.L) {
        // out = U . Q8_1(y_lat)
        // Q8_1(y_lat) comes from the down kernel (per-token form, array of
        // packs) or from the combine (per-bucket form), else is made here
        const bool ylq_ready = ylq_in_down || !down_tok;
        if (dense_gemm) {
            if (!ylq_ready) CK(launch_quant_rows(ylat, T, m.L, ylq, st), "Q8_1(y_lat)");
            CK(launch_dense_mfma(m.U, (const uint8_t*)Up, T, ylq, out, tp.isum_u, tp.tap_tokens, st), "U");
        } else if (thin) {
            if (!ylq_ready) CK(launch_quant_rows(ylat, T, m.L, ylq, st), "Q8_1(y_lat)");
            CK(launch_dense_thin(m.U, (const uint8_t*)Up, T, ylq, out, 1, tp.isum_u, tp.tap_tokens, st), "U");
        } else if (ylq_in_down) {
            CK(launch_dense_mv(m.U, (const uint8_t*)Up, T, ylq, nullptr, none, out, tp.isum_u,
                               tp.tap_tokens, st), "U");
        } else if (lat_fused_q) {
            // the U kernel quantises y_lat on the way in
            CK(launch_dense_mv(m.U, (const uint8_t*)Up, T, none, ylat, taps ? ylq : none, out,
                               tp.isum_u, tp.tap_tokens, st), "U");
        } else {
            CK(launch_quant_rows(ylat, T, m.L, ylq, st), "Q8_1(y_lat)");
            CK(launch_dense_mv(m.U, (const uint8_t*)Up, T, ylq, nullptr, none, out, tp.isum_u,
                               tp.tap_tokens, st), "U");
        }
    }
    EV(MOE_EV_END);
    if (taps) {
        if (taps->ids) CK(hipMemcpyAsync(taps->ids, b.ids, sizeof(int32_t) * A, hipMemcpyDeviceToDevice, st), "tap ids");
        if (taps->weights) CK(hipMemcpyAsync(taps->weights, b.wts, sizeof(float) * A, hipMemcpyDeviceToDevice, st), "tap weights");
        CK(launch_tap_q8_1(xq, T, m.H, taps->xq, st), "tap xq");
        CK(launch_tap_q8_1(hq, A, m.F, taps->hq, st), "tap hq");
        if (m.L) {
            CK(launch_tap_q8_1(zq, T, m.L, taps->zq, st), "tap zq");
            CK(launch_tap_q8_1(ylq, T, m.L, taps->ylq, st), "tap ylq");
            if (taps->z) CK(hipMemcpyAsync(taps->z, z, sizeof(float) * T * m.L, hipMemcpyDeviceToDevice, st), "tap z");
            if (taps->ylat) CK(hipMemcpyAsync(taps->ylat, ylat, sizeof(float) * T * m.L, hipMemcpyDeviceToDevice, st), "tap ylat");
        }
        if (!down_tok && taps->y)
            CK(hipMemcpyAsync(taps->y, y, sizeof(float) * (size_t)A * m.kout, hipMemcpyDeviceToDevice, st), "tap y");
    }
#undef EV
#undef CK
    return MOE_OK;
}

extern "C" moe_status moe_layer_forward(const moe_layer* L, const float* x, int T,
                                        const float* router_w, const float* router_b,
                                        const int32_t* groups, const void* experts, const void* D,
                                        const void* U, int k, float* out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    return forward_impl(L, x, T, router_w, router_b, groups, ExpertSrc((const uint8_t*)experts), D,
                        U, k, out, workspace, workspace_bytes, stream, nullptr, nullptr);
}

extern "C" moe_status moe_layer_forward_noalloc(const moe_layer* L, const float* x, int T,
                                                const float* router_w, const float* router_b,
                                                const int32_t* groups, const void* experts,
                                                const void* D, const void* U, int k, float* out,
                                                void* stream) {
    if (!L) return fail(MOE_EINVAL, "layer is NULL");
    if (T < 0 || T > L->dims.max_tokens)
        return fail(MOE_EINVAL, "T %d out of range 0..max_tokens=%d", T, L->dims.max_tokens);
    const size_t need = ws_layout(L->dims, std::max(T, 1)).total;
    if (need > (size_t)MOE_NOALLOC_WORKSPACE_BYTES)
        return fail(MOE_ENOMEM,
                    "T=%d needs %zu bytes of workspace; the static workspace holds %zu "
                    "(call moe_layer_forward with a workspace of the caller's)",
                    T, need, (size_t)MOE_NOALLOC_WORKSPACE_BYTES);
    void* ws;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ws = L->device < SCRATCH_MAX_DEVICES ? g_scratch[L->device] : nullptr;
    }
    if (!ws) return fail(MOE_EDEVICE, "no static workspace on device %d", L->device);
    return forward_impl(L, x, T, router_w, router_b, groups, ExpertSrc((const uint8_t*)experts), D,
                        U, k, out, ws, (size_t)MOE_NOALLOC_WORKSPACE_BYTES, stream, nullptr,
                        nullptr);
}

extern "C" moe_status moe_layer_forward_events(const moe_layer* L, const float* x, int T,
                                               const float* router_w, const float* router_b,
                                               const int32_t* groups, const void* experts,
                                               const void* D, const void* U, int k, float* out,
                                               void* workspace, size_t workspace_bytes,
                                               void* stream, void* const* events) {
    return forward_impl(L, x, T, router_w, router_b, groups, ExpertSrc((const uint8_t*)experts), D,
                        U, k, out, workspace, workspace_bytes, stream, nullptr, events);
}

extern "C" moe_status moe_layer_forward_taps(const moe_layer* L, const float* x, int T,
                                             const float* router_w, const float* router_b,
                                             const int32_t* groups, const void* experts,
                                             const void* D, const void* U, int k, float* out,
                                             void* workspace, size_t workspace_bytes, void* stream,
                                             const moe_taps* taps) {
    if (!taps) return fail(MOE_EINVAL, "taps is NULL");
    return forward_impl(L, x, T, router_w, router_b, groups, ExpertSrc((const uint8_t*)experts), D,
                        U, k, out, workspace, workspace_bytes, stream, taps, nullptr);
}

// ---------------------------------------------------------------------------
// Experts held apart from one array: a table of pack addresses, and a cache of
// resident packs in device slots in front of a pinned host copy (edge0-strata
// README, "Changes from upstream Strata": the CPU/PCIe share of expert work for
// experts not resident on the GPU; Strata PR 24 commit log: an expert cache
// whose slot holds one whole expert blob, and a cache once filled from a
// staging ring that had already been overwritten).  Here a non-resident
// expert is read by the same kernels straight from mapped host memory, over
// the bus; a resident one from its slot.

extern "C" moe_status moe_layer_forward_table(const moe_layer* L, const float* x, int T,
                                              const float* router_w, const float* router_b,
                                              const int32_t* groups,
                                              const void* const* expert_table, const void* D,
                                              const void* U, int k, float* out, void* workspace,
                                              size_t workspace_bytes, void* stream) {
    if (!expert_table) return fail(MOE_EINVAL, "expert_table is NULL");
    return forward_impl(L, x, T, router_w, router_b, groups,
                        ExpertSrc(nullptr, (const uint8_t* const*)expert_table), D, U, k, out,
                        workspace, workspace_bytes, stream, nullptr, nullptr);
}

struct moe_expert_cache {
    int device = 0, E = 0, n_slots = 0;
    size_t eb = 0;
    const uint8_t* host = nullptr;      // the caller's pinned copy (copy source)
    const uint8_t* host_dev = nullptr;  // the same memory as the device addresses it
    uint8_t* slots = nullptr;
    const uint8_t** table = nullptr;
    std::vector<int> slot_of;           // expert -> slot, -1 = read from host memory
    std::vector<int> expert_in;         // slot -> expert, -1 = empty
    std::vector<uint64_t> last_use;     // slot -> admit call that last named its expert
    uint64_t tick = 0;
};

// the allocation that holds [p, p + bytes) must be device memory of `device`
static moe_status check_device_range(const void* p, size_t bytes, int device, const char* what) {
    hipPointerAttribute_t a;
    hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess || a.type != hipMemoryTypeDevice || a.device != device) {
        (void)hipGetLastError();
        return fail(MOE_EINVAL, "%s is not device memory of device %d", what, device);
    }
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    e = hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MOE_EINVAL, "%s: no allocation range (%s)", what, hipGetErrorString(e));
    }
    if ((const char*)p + bytes > (const char*)base + size)
        return fail(MOE_EINVAL, "%s: %zu bytes needed past the pointer, the allocation holds %zu", what,
                    bytes, (size_t)((const char*)base + size - (const char*)p));
    return MOE_OK;
}

extern "C" moe_status moe_expert_cache_create(const moe_layer* L, const void* host_packs,
                                              void* slots, int n_slots, void* table, void* stream,
                                              moe_expert_cache** out) {
    if (!out) return fail(MOE_EINVAL, "out is NULL");
    *out = nullptr;
    if (!L) return fail(MOE_EINVAL, "layer is NULL");
    const Dims& m = L->dims;
    if (!host_packs || !table || (n_slots > 0 && !slots))
        return fail(MOE_EINVAL, "NULL host_packs, table or slots");
    if (n_slots < 0 || n_slots > m.E)
        return fail(MOE_EINVAL, "n_slots %d out of range 0..n_experts=%d", n_slots, m.E);
    if ((uintptr_t)host_packs % 256 || (uintptr_t)slots % 256 || (uintptr_t)table % 8)
        return fail(MOE_EINVAL, "host_packs and slots must be 256-byte aligned, table 8-byte");
    DeviceGuard g(L->device);
    if (!g.ok) return fail(MOE_EDEVICE, "cannot select device %d", L->device);
    // the host copy must be pinned and mapped: the kernels read it over the bus
    hipPointerAttribute_t a;
    hipError_t e = hipPointerGetAttributes(&a, host_packs);
    if (e != hipSuccess || a.type != hipMemoryTypeHost || !a.devicePointer) {
        (void)hipGetLastError();
        return fail(MOE_EINVAL, "host_packs is not pinned host memory mapped for the device");
    }
    moe_status s = check_device_range(table, sizeof(void*) * m.E, L->device, "table");
    if (s != MOE_OK) return s;
    if (n_slots > 0) {
        s = check_device_range(slots, m.expert_bytes * n_slots, L->device, "slots");
        if (s != MOE_OK) return s;
    }
    moe_expert_cache* c = new (std::nothrow) moe_expert_cache;
    if (!c) return fail(MOE_ENOMEM, "cache object");
    c->device = L->device;
    c->E = m.E;
    c->n_slots = n_slots;
    c->eb = m.expert_bytes;
    c->host = (const uint8_t*)host_packs;
    c->host_dev = (const uint8_t*)a.devicePointer;
    c->slots = (uint8_t*)slots;
    c->table = (const uint8_t**)table;
    c->slot_of.assign(m.E, -1);
    c->expert_in.assign(n_slots, -1);
    c->last_use.assign(n_slots, 0);
    e = launch_table_fill(c->table, m.E, c->host_dev, c->eb, (hipStream_t)stream);
    if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "table fill");
    }
    *out = c;
    return MOE_OK;
}

extern "C" moe_status moe_expert_cache_admit(moe_expert_cache* c, const int32_t* experts, int n,
                                             void* stream, int* n_copied) {
    if (n_copied) *n_copied = 0;
    if (!c) return fail(MOE_EINVAL, "cache is NULL");
    if (n < 0 || (n > 0 && !experts)) return fail(MOE_EINVAL, "bad expert list (n = %d)", n);
    std::vector<char> named(c->E, 0);
    int distinct = 0;
    for (int i = 0; i < n; ++i) {
        const int e = experts[i];
        if (e < 0 || e >= c->E) return fail(MOE_EINVAL, "expert %d out of range 0..%d", e, c->E - 1);
        if (!named[e]) ++distinct;
        named[e] = 1;
    }
    if (distinct > c->n_slots)
        return fail(MOE_EINVAL, "%d distinct experts named, the cache has %d slots", distinct,
                    c->n_slots);
    DeviceGuard g(c->device);
    if (!g.ok) return fail(MOE_EDEVICE, "cannot select device %d", c->device);
    hipStream_t st = (hipStream_t)stream;
    const uint64_t now = ++c->tick;
    // experts already resident are kept: they are not eviction candidates now
    for (int e = 0; e < c->E; ++e)
        if (named[e] && c->slot_of[e] >= 0) c->last_use[c->slot_of[e]] = now;
    TableUpdate u;
    u.n = 0;
    hipError_t err;
    auto flush = [&]() -> hipError_t {
        hipError_t r = launch_table_set(c->table, u, st);
        u.n = 0;
        return r;
    };
    auto set = [&](int e, const uint8_t* p) -> hipError_t {
        u.expert[u.n] = e;
        u.addr[u.n] = p;
        return ++u.n == TABLE_UPDATE_MAX ? flush() : hipSuccess;
    };
    int copied = 0;
    for (int e = 0; e < c->E; ++e) {
        if (!named[e] || c->slot_of[e] >= 0) continue;
        // an empty slot first, else the least recently named one not named now
        int v = -1;
        for (int s = 0; s < c->n_slots && v < 0; ++s)
            if (c->expert_in[s] < 0) v = s;
        if (v < 0)
            for (int s = 0; s < c->n_slots; ++s)
                if (c->last_use[s] < now && (v < 0 || c->last_use[s] < c->last_use[v])) v = s;
        if (v < 0) return fail(MOE_EINVAL, "no slot to evict");   // unreachable: distinct <= n_slots
        const int old = c->expert_in[v];
        uint8_t* slot = c->slots + (size_t)v * c->eb;
        if (old >= 0) {
            // the evicted expert is read from host memory again; its entry
            // changes before the slot is overwritten (stream order)
            c->slot_of[old] = -1;
            if ((err = set(old, c->host_dev + (size_t)old * c->eb)) != hipSuccess ||
                (err = flush()) != hipSuccess)
                return hip_fail(err, "table update");
        }
        err = hipMemcpyAsync(slot, c->host + (size_t)e * c->eb, c->eb, hipMemcpyHostToDevice, st);
        if (err != hipSuccess) return hip_fail(err, "expert copy into a slot");
        c->expert_in[v] = e;
        c->slot_of[e] = v;
        c->last_use[v] = now;
        if ((err = set(e, slot)) != hipSuccess) return hip_fail(err, "table update");
        ++copied;
    }
    if ((err = flush()) != hipSuccess) return hip_fail(err, "table update");
    if (n_copied) *n_copied = copied;
    return MOE_OK;
}

extern "C" moe_status moe_expert_cache_slot(const moe_expert_cache* c, int expert, int* slot) {
    if (!c || !slot) return fail(MOE_EINVAL, "NULL argument");
    if (expert < 0 || expert >= c->E)
        return fail(MOE_EINVAL, "expert %d out of range 0..%d", expert, c->E - 1);
    *slot = c->slot_of[expert];
    return MOE_OK;
}

extern "C" void moe_expert_cache_destroy(moe_expert_cache* c) { delete c; }
