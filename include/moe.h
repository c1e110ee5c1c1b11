/*
 * moe.h - C ABI of the quantized mixture-of-experts expert FFN for AMD MI355X
 * (gfx950).  Implemented by libmoe.so (hand-written HIP kernels).
 *
 * The layer (sources are the pages' titles and sections):
 *   - "Q8 0 support" (Strata pull request 255), section "GPU expert kernels":
 *     Q8_0 expert weights in blocks of 32, multiplied against activations
 *     quantised to Q8_1 blocks; the grouped gate/up/down expert kernels;
 *     the follow-up commit: the Q8_1 block sum is the sum of the quantised
 *     activations; unsupported format pairs are refused by name at start-up.
 *   - "Sync upstream Strata v0.1.39 into Lanes" (pull request 24), the SYCL port
 *     commits: per-token top-k routing over 256/512 experts, tokens grouped by
 *     expert, activation quantisation that matches byte for byte only with a
 *     correctly rounded fp32 divide, a split-K down kernel bit-identical to the
 *     single-token one.
 *   - edge0-strata README, section "Changes from upstream Strata": latent MoE,
 *     dense Q8 D/U projections into a 1280- or 1792-wide latent space, expert
 *     group labels, Q4_0 expert rows against Q8_1 activations.
 *
 * For each token t (x_t fp32, H wide):
 *   1. router logits l_e = x_t . W_r[e] (+ b_e), accumulated in fp64;
 *   2. with group labels: keep the experts of the topk_groups groups with the
 *      largest member logit; top_k experts by logit (ties: lower id);
 *      w_j = softmax over the chosen logits;
 *   3. a = Q8_1(x_t) (latent: a = Q8_1(z_t), z_t = D . Q8_1(x_t));
 *   4. per chosen expert e_j: g = W_gate a, u = W_up a, h = silu(g) * u,
 *      y_j = W_down . Q8_1(h);
 *   5. out_t = sum_j w_j y_j in rank order (latent: out_t = U . Q8_1(that sum)).
 * Q8_1 of 32 floats: d = max|v| / 127 (fp32 divide), q = round-half-away(v / d),
 * stored as binary16 d, binary16 s = d * sum(q), 32 int8 q.
 *
 * Conventions for every function below:
 *   - Returns MOE_OK or a negative moe_status; no exception crosses the ABI.
 *     moe_last_error() then names the refused argument (thread-local text).
 *   - All shape, format and device checks happen in moe_layer_create / the
 *     pack calls; moe_layer_forward re-checks only T, k and pointers.
 *   - The caller owns every buffer.  The library allocates no device memory;
 *     moe_layer holds host metadata only.  (The one exception is static: the
 *     workspace array of moe_layer_forward_noalloc, 64 MiB per GPU, which the
 *     first moe_layer_create on a GPU looks up and zeroes.)
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *     Forward calls are asynchronous on it and never synchronise the host.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,          /* bad argument: null pointer, size, T or k out of range   */
    MOE_EUNSUPPORTED = -2,    /* valid but unsupported: format pair, dims not multiples  */
    MOE_EDEVICE = -3,         /* no device, or the device is not gfx950                  */
    MOE_EHIP = -4,            /* a HIP runtime call failed                                */
    MOE_ENOMEM = -5           /* workspace or host staging too small / allocation failed  */
} moe_status;

/* Block formats.  The values mirror the pages' "case 8" of the format switch
 * (ggml's type numbers).  Q5_1 ("Q8 0 support" page, the K-quant follow-up
 * commit: Q5_1 experts): 24-byte blocks of binary16 d, binary16 m, a 32-bit
 * little-endian qh of fifth bits and 16 nibble bytes, value d*q + m; its dot
 * with a Q8_1 block adds m times the block's stored s (d times the sum of the
 * quantised activations).  Q4_K (same commit: Q4_K experts): 144-byte
 * super-blocks of 256 (binary16 d and dmin, 12 bytes of 6-bit sub-block scales
 * and mins, 128 nibble bytes), value d*scale*q - dmin*min, the min term on
 * each Q8_1 block's code sum times its d; it needs Kin and n_ff to be
 * multiples of 256.  Q5_K (same commit): 176-byte super-blocks, the Q4_K
 * header and scales, 32 bytes of fifth bits (bit b of byte i for element i of
 * sub-block b), then the nibbles; same value and dot as Q4_K with q in 0..31.
 * Q3_K (edge0-strata README, changes from upstream Strata: Q3_K latent
 * experts; the block is ggml's): 110-byte super-blocks of 256, 32 bytes hmask,
 * 64 bytes qs, 12 bytes of 6-bit sub-block scales, binary16 d; element e
 * (half = e/128, j = e%128/32, l = e%32) has low bits (qs[32*half+l] >> 2j) & 3
 * and high bit (hmask[l] >> (4*half+j)) & 1, code low + 4*high - 4; sub-block i
 * of 16 has scale (lo | hi << 4) - 32 with lo the low (i < 8) or high (i >= 8)
 * nibble of byte i % 8 and hi bits 2*(i/4) of byte 8 + i%4; value
 * d*scale*code; a Q8_1 block's dot is d*d_a times the sum over its two halves
 * of scale * sum(code * q_a).
 * Q5_1, Q4_K, Q5_K and Q3_K are expert formats only. */
enum { MOE_FMT_Q8_0 = 8, MOE_FMT_Q4_0 = 2, MOE_FMT_Q5_1 = 7, MOE_FMT_Q4_K = 12, MOE_FMT_Q5_K = 13,
       MOE_FMT_Q3_K = 11, MOE_FMT_NVFP4 = 40 };

/* Which packed tensor a pack call is about. */
enum { MOE_PACK_EXPERTS = 0, MOE_PACK_D = 1, MOE_PACK_U = 2 };

typedef struct {
    int32_t hidden;       /* H: multiple of 256                                          */
    int32_t n_experts;    /* E: 1..512                                                    */
    int32_t top_k;        /* k: 1..min(E, 32)                                             */
    int32_t n_ff;         /* F: expert intermediate width, multiple of 256                */
    int32_t latent;       /* L: 0 = plain MoE; else the latent width, multiple of 256     */
    int32_t expert_fmt;   /* MOE_FMT_Q8_0, _Q4_0, _Q5_1, _Q4_K, _Q5_K, _Q3_K or _NVFP4   */
    int32_t dense_fmt;    /* D/U format: MOE_FMT_Q8_0 or MOE_FMT_Q4_0 (latent == 0: unused)*/
    int32_t n_groups;     /* 0 = no group limit; else divides E                           */
    int32_t topk_groups;  /* groups kept per token: 1..n_groups, topk_groups*E/n_groups>=k*/
    int32_t max_tokens;   /* largest T a forward call may pass: 1..65536                  */
} moe_desc;

typedef struct moe_layer moe_layer;

/*
 * Canonical (host, array-of-structs) layouts that the pack calls accept:
 *   Q8_0 block = binary16 d (little-endian) + 32 int8 q              (34 bytes)
 *   Q4_0 block = binary16 d + 16 bytes; byte j: element j in the low nibble,
 *                element j+16 in the high nibble; value d*(c-8)       (18 bytes)
 *   NVFP4 block of 32 (edge0-strata README, section "Changes from upstream
 *          Strata", names NVFP4 latent experts; read as FP4 E2M1 codes, an
 *          FP8 E4M3 scale per 16 elements and an fp32 scale per tensor) =
 *          E4M3 scale of elements 0..15, E4M3 scale of 16..31, 16 bytes; byte
 *          i: element 2i in the low nibble, 2i+1 in the high nibble     (18 bytes)
 *   EXPERTS: for e in 0..E-1: gate [F][Kin/32], up [F][Kin/32], down [Kout][F/32]
 *            blocks, rows row-major; Kin = Kout = latent ? L : H.  An NVFP4
 *            expert then holds a 256-byte tail: its tensor scales gate, up,
 *            down (fp32), then zero bytes.
 *   D: [L][H/32] Q8_0 blocks.  U: [H][L/32] Q8_0 blocks.
 * The packed (device) layout has the same byte count; it splits codes from
 * scales and orders gate/up rows in 32-row pairs.  It is private to the library.
 */

/* Validates desc and checks that `device` is a gfx950 GPU.  Shape and format
 * errors are reported before the device is looked at.  *out receives a new
 * host object; free it with moe_layer_destroy. */
moe_status moe_layer_create(const moe_desc* desc, int device, moe_layer** out);
void moe_layer_destroy(moe_layer* layer);

/* Validates desc only (no device needed); the same checks as moe_layer_create. */
moe_status moe_desc_check(const moe_desc* desc);

/* Bytes of the canonical = packed form of one tensor (which = MOE_PACK_*).
 * Needs no device.  MOE_PACK_D/U on a plain layer give MOE_EINVAL. */
moe_status moe_pack_bytes(const moe_desc* desc, int which, size_t* bytes);

/* Host-to-host layout conversion, canonical -> packed and back.  Needs no
 * device.  Buffers hold moe_pack_bytes bytes and must not overlap. */
moe_status moe_pack_host(const moe_desc* desc, int which, const void* canonical, void* packed);
moe_status moe_unpack_host(const moe_desc* desc, int which, const void* packed, void* canonical);

/* Converts a host canonical tensor and copies it to device memory dev_dst
 * (moe_pack_bytes bytes), in chunks through host staging memory that the call
 * allocates and frees.  Returns when the copy is complete. */
moe_status moe_pack(const moe_layer* layer, int which, const void* host_canonical,
                    void* dev_dst, void* stream);

/* Checks host group labels (group_of_expert's content, E int32) against the
 * contract of a layer with n_groups > 0 (the expert group labels of the
 * edge0-strata README, section "Changes from upstream Strata", read as equal
 * groups, step 2 above): every label in [0, n_groups) and exactly
 * E / n_groups experts per label.  MOE_EINVAL names the first label or
 * group that breaks it.  With n_groups == 0, labels must be NULL.  Needs no
 * device. */
moe_status moe_group_labels_check(const moe_desc* desc, const int32_t* labels);

/* Device workspace a forward call with T tokens needs (T <= max_tokens).
 * The workspace must be zero-filled before its first use; every call leaves
 * its internal counters at zero again, so one zeroing suffices. */
moe_status moe_workspace_bytes(const moe_layer* layer, int T, size_t* bytes);

/*
 * The layer on device memory.  x [T][H] fp32; router_w [E][H] fp32; router_b
 * [E] fp32 or NULL; group_of_expert [E] int32 labels in [0, n_groups) with
 * E/n_groups experts per label, or NULL when n_groups == 0; expert_packs, D, U
 * the packed tensors (D, U NULL when latent == 0); k must equal desc.top_k;
 * out [T][H] fp32.  T == 0 is a no-op.  Inputs must be finite (NaN/Inf:
 * unspecified output).  Deterministic: the same inputs give bitwise the same
 * out.  Calls sharing one workspace must not overlap in time.  The kernels do
 * not re-check the group labels: labels outside that contract (out of range,
 * or groups of unequal size) give an unspecified output; moe_group_labels_check
 * validates them on the host once per layer.
 */
moe_status moe_layer_forward(const moe_layer* layer, const float* x, int T,
                             const float* router_w, const float* router_b,
                             const int32_t* group_of_expert, const void* expert_packs,
                             const void* D, const void* U, int k, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-step outputs for checking, all device pointers, each NULL to skip.
 * Token-major; a = t*k + j indexes assignments.  Q8_1 taps use the canonical
 * 36-byte block (binary16 d, binary16 s, 32 int8).  Integer block sums are
 * recorded only for tokens t < tap_tokens.
 */
typedef struct {
    double*  logits;   /* [T][E]                                                   */
    int32_t* ids;      /* [T][k]                                                   */
    float*   weights;  /* [T][k]                                                   */
    uint8_t* xq;       /* [T][H/32][36]  Q8_1(x)                                   */
    float*   z;        /* [T][L]         latent only                               */
    uint8_t* zq;       /* [T][L/32][36]  latent only                               */
    float*   h;        /* [T*k][F]       silu(g)*u                                 */
    uint8_t* hq;       /* [T*k][F/32][36]                                          */
    float*   y;        /* [T*k][Kout]    each expert's down output                 */
    float*   ylat;     /* [T][L]         latent only, the combined latent vector   */
    uint8_t* ylq;      /* [T][L/32][36]  latent only                               */
    int32_t* isum_gu;  /* [tap_tokens*k][2F][Kin/32]  gate rows, then up rows      */
    int32_t* isum_dn;  /* [tap_tokens*k][Kout][F/32]                               */
    int32_t* isum_d;   /* [tap_tokens][L][H/32]   latent only                      */
    int32_t* isum_u;   /* [tap_tokens][H][L/32]   latent only                      */
    int32_t  tap_tokens;
} moe_taps;

/* moe_layer_forward that also fills the non-NULL taps (slower kernels of the
 * same code).  out is identical to moe_layer_forward's. */
moe_status moe_layer_forward_taps(const moe_layer* layer, const float* x, int T,
                                  const float* router_w, const float* router_b,
                                  const int32_t* group_of_expert, const void* expert_packs,
                                  const void* D, const void* U, int k, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  const moe_taps* taps);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_layer_forward with the library's own workspace instead of one passed in.
 * That workspace is a static device array of MOE_NOALLOC_WORKSPACE_BYTES
 * (64 MiB), one copy per GPU, looked up and zeroed by the first
 * moe_layer_create on that GPU and held until the process ends.  The call
 * allocates nothing.  A T whose workspace (moe_workspace_bytes) exceeds the
 * array is refused with MOE_ENOMEM; every decode and verify size fits, the
 * 2048-token prefill layers do not.  Every call on one GPU, from any layer,
 * shares that GPU's array: calls that overlap in time on one GPU race and give
 * undefined results, so the caller orders them (one stream, or events).  Each
 * call leaves the array's counters at zero for the next one.  Arguments,
 * results and errors are otherwise those of moe_layer_forward.
 */
#define MOE_NOALLOC_WORKSPACE_BYTES (64u << 20)

moe_status moe_layer_forward_noalloc(const moe_layer* layer, const float* x, int T,
                                     const float* router_w, const float* router_b,
                                     const int32_t* group_of_expert, const void* expert_packs,
                                     const void* D, const void* U, int k, float* out,
                                     void* stream);

/*
 * Stage boundaries for timing (the pages' per-stage profiler idea: milliseconds
 * per stage of a layer).  moe_layer_forward_events records events[i] (each a
 * hipEvent_t created by the caller, passed as void*; NULL entries are skipped)
 * on `stream` at these points of the kernel sequence:
 *   MOE_EV_BEGIN    before the first kernel
 *   MOE_EV_ROUTED   after quantising x, routing and bucketing (T == 1: after the
 *                   router logits; the selection runs in the gate/up kernel)
 *   MOE_EV_EXPERT_IN after the latent D projection (== ROUTED when latent == 0)
 *   MOE_EV_GATE_UP  after the grouped gate/up + SwiGLU + requantisation
 *   MOE_EV_DOWN     after the grouped down projection and the combine
 *   MOE_EV_END      after the last kernel (latent: after U)
 *   MOE_EV_GATE_UP_KSTART, MOE_EV_GATE_UP_KEND
 *                   the start and end of the grouped gate/up kernel itself,
 *                   recorded by its own dispatch (no event packets around it),
 *                   so their elapsed time is that kernel's duration
 * The kernels and out are those of moe_layer_forward.
 */
enum { MOE_EV_BEGIN = 0, MOE_EV_ROUTED, MOE_EV_EXPERT_IN, MOE_EV_GATE_UP, MOE_EV_DOWN,
       MOE_EV_END, MOE_EV_GATE_UP_KSTART, MOE_EV_GATE_UP_KEND, MOE_EV_COUNT };

moe_status moe_layer_forward_events(const moe_layer* layer, const float* x, int T,
                                    const float* router_w, const float* router_b,
                                    const int32_t* group_of_expert, const void* expert_packs,
                                    const void* D, const void* U, int k, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    void* const* events);

/*
 * Experts held apart (edge0-strata README, "Changes from upstream Strata": the
 * CPU/PCIe share of expert work for experts that are not resident on the GPU;
 * Strata PR 24 commit log: an expert cache whose slot holds one whole expert
 * blob).
 *
 * moe_layer_forward_table is moe_layer_forward with expert e's pack (the
 * moe_pack_bytes(EXPERTS) / n_experts bytes of one expert, in the packed
 * layout) at expert_table[e] instead of at expert_packs + e * that size.
 * expert_table is a device array of n_experts addresses; each address is
 * 256-byte aligned and lies either in device memory of the layer's device or
 * in pinned host memory mapped for it (hipHostMalloc), which the kernels then
 * read over the bus.  The library cannot check the entries: a wrong address
 * faults the device.  The kernels and out are those of moe_layer_forward, so
 * the same packs give bitwise the same out.
 */
moe_status moe_layer_forward_table(const moe_layer* layer, const float* x, int T,
                                   const float* router_w, const float* router_b,
                                   const int32_t* group_of_expert,
                                   const void* const* expert_table, const void* D,
                                   const void* U, int k, float* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * A cache of resident experts that keeps such a table.  host_packs: all
 * n_experts packs (moe_pack_host's output) in pinned host memory mapped for
 * the device, 256-byte aligned; slots: device memory for n_slots packs
 * (0 <= n_slots <= n_experts), 256-byte aligned; table: device memory for
 * n_experts addresses, passed to moe_layer_forward_table.  The caller owns all
 * three and keeps them alive while the cache lives.  create points every entry
 * at the host copy (on `stream`); it refuses host memory that is not pinned and
 * mapped, and slots or a table that is not device memory of the layer's device
 * or is smaller than stated.
 *
 * admit makes the n experts listed (host int32 ids; at most n_slots distinct)
 * resident: each one not yet in a slot takes an empty slot, else the slot whose
 * expert was named least recently by an earlier admit (ties: lower slot); the
 * evicted expert's entry points at the host copy again before its slot is
 * overwritten.  The copies and entry updates are queued on `stream` in that
 * order, so calls that read the table on the same stream afterwards see whole
 * packs; calls on other streams must be ordered by the caller.  *n_copied
 * (may be NULL) receives the number of packs copied.  slot gives an expert's
 * slot, or -1 when it is read from host memory.
 */
typedef struct moe_expert_cache moe_expert_cache;
moe_status moe_expert_cache_create(const moe_layer* layer, const void* host_packs, void* slots,
                                   int n_slots, void* table, void* stream,
                                   moe_expert_cache** out);
moe_status moe_expert_cache_admit(moe_expert_cache* cache, const int32_t* experts, int n,
                                  void* stream, int* n_copied);
moe_status moe_expert_cache_slot(const moe_expert_cache* cache, int expert, int* slot);
void moe_expert_cache_destroy(moe_expert_cache* cache);

/* Text of the last error on this thread ("" when none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
