// Host side of the C ABI declared in include/dynconv.h: argument checks,
// path selection, workspace carving and kernel dispatch. Every check runs
// before the first HIP call, so an invalid call touches neither the device
// nor any output (and needs no GPU at all).
#include "dynconv.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <mutex>

#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

dynconv_status_t fail(dynconv_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

dynconv_status_t ok() {
    g_err[0] = '\0';
    return DYNCONV_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr long kMaxElems = (1L << 31) - 1;  // per tensor
constexpr size_t kWsAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int d_cout(const dynconv_desc_t *d) { return d->Cout; }

// Shape checks shared by every entry point. On success fills `g`.
dynconv_status_t check_desc(const dynconv_desc_t *d, dynconv::Geom &g, bool need_conv) {
    if (!d) return fail(DYNCONV_ERR_INVALID_ARG, "desc is NULL");
    if (d->B < 1 || d->Cin < 1 || d->H < 1 || d->W < 1 || d->n < 1)
        return fail(DYNCONV_ERR_INVALID_ARG, "B, Cin, H, W and n must be >= 1 (got B=%d Cin=%d H=%d W=%d n=%d)",
                    d->B, d->Cin, d->H, d->W, d->n);
    if (d->dtype != DYNCONV_F32 && d->dtype != DYNCONV_BF16)
        return fail(DYNCONV_ERR_INVALID_ARG, "dtype %d is not a dynconv_dtype_t", d->dtype);
    g = dynconv::Geom{};
    g.B = d->B; g.Cin = d->Cin; g.H = d->H; g.W = d->W; g.n = d->n;
    g.bf16 = d->dtype == DYNCONV_BF16;
    if ((long)d->B * d->Cin * d->H * d->W > kMaxElems)
        return fail(DYNCONV_ERR_UNSUPPORTED, "x has more than 2^31-1 elements");
    g.n_pad = (d->n + 1) & ~1;
    g.Cin_pad = (d->Cin + 31) / 32 * 32;
    if (!need_conv) return DYNCONV_OK;
    if (d->Cout < 1 || d->kh < 1 || d->kw < 1 || d->stride < 1 || d->pad < 0 || d->groups < 1)
        return fail(DYNCONV_ERR_INVALID_ARG,
                    "Cout, kh, kw, stride, groups must be >= 1 and pad >= 0 (got Cout=%d kh=%d kw=%d stride=%d pad=%d groups=%d)",
                    d->Cout, d->kh, d->kw, d->stride, d->pad, d->groups);
    if (d->Cin % d->groups || d->Cout % d->groups)
        return fail(DYNCONV_ERR_INVALID_ARG, "groups=%d must divide Cin=%d and Cout=%d", d->groups,
                    d->Cin, d->Cout);
    const long Ho = ((long)d->H + 2L * d->pad - d->kh) / d->stride + 1;
    const long Wo = ((long)d->W + 2L * d->pad - d->kw) / d->stride + 1;
    if ((long)d->H + 2L * d->pad < d->kh || (long)d->W + 2L * d->pad < d->kw || Ho < 1 || Wo < 1)
        return fail(DYNCONV_ERR_INVALID_ARG, "kernel %dx%d larger than padded input %dx%d", d->kh,
                    d->kw, d->H + 2 * d->pad, d->W + 2 * d->pad);
    if (d->groups != 1 && !(d->groups == d->Cin && d->Cin == d->Cout))
        return fail(DYNCONV_ERR_UNSUPPORTED,
                    "groups=%d: only groups == 1 or depthwise (groups == Cin == Cout) are implemented",
                    d->groups);
    if ((long)d->B * d->Cout * Ho * Wo > kMaxElems)
        return fail(DYNCONV_ERR_UNSUPPORTED, "y has more than 2^31-1 elements");
    const long wsize = (long)d->Cout * (d->Cin / d->groups) * d->kh * d->kw;
    if (wsize * d->n > kMaxElems || wsize * d->B > kMaxElems)
        return fail(DYNCONV_ERR_UNSUPPORTED, "expert bank or mixed kernels exceed 2^31-1 elements");
    g.Cout = d->Cout; g.KH = d->kh; g.KW = d->kw; g.stride = d->stride; g.pad = d->pad;
    g.groups = d->groups;
    g.Ho = (int)Ho; g.Wo = (int)Wo; g.P = (int)(Ho * Wo); g.KT = d->kh * d->kw;
    g.cpg = d->Cin / d->groups;
    return DYNCONV_OK;
}

long kernel_elems(const dynconv::Geom &g) { return (long)g.Cout * g.cpg * g.KT; }
size_t esize(const dynconv::Geom &g) { return g.bf16 ? 2 : 4; }
bool depthwise(const dynconv::Geom &g) { return g.groups != 1; }
// bf16 groups == 1 layers with more than 16 experts mix on the matrix cores
// from a bank in the convolution's weight order (KernelWarehouse's n > 100)
bool wide(const dynconv::Geom &g) { return g.bf16 && g.groups == 1 && g.n_pad > 16; }

// Resolve AUTO and check that the chosen path exists for this layer.
dynconv_status_t resolve_policy(const dynconv::Geom &g, int32_t policy, int32_t &out) {
    if (policy != DYNCONV_POLICY_AUTO && policy != DYNCONV_POLICY_PREMIX &&
        policy != DYNCONV_POLICY_FUSED)
        return fail(DYNCONV_ERR_INVALID_ARG, "policy %d is not a dynconv_policy_t", policy);
    if (depthwise(g)) {
        if (!dynconv::depthwise_supported(g))
            return fail(DYNCONV_ERR_UNSUPPORTED,
                        "depthwise layer: kernel taps must be <= 64 and the padded plane must fit in 64 KB of LDS");
        out = policy == DYNCONV_POLICY_AUTO ? DYNCONV_POLICY_FUSED : policy;
        return DYNCONV_OK;
    }
    if (!g.bf16) {
        if (policy == DYNCONV_POLICY_FUSED)
            return fail(DYNCONV_ERR_UNSUPPORTED, "float32 layers have no fused path");
        out = DYNCONV_POLICY_PREMIX;
        return DYNCONV_OK;
    }
    if (wide(g) && !dynconv::pack_wide_supported(g))
        return fail(DYNCONV_ERR_UNSUPPORTED, "more than 16 experts: one expert's Cin x kh x kw block must fit 64 KB");
    const bool fused_ok = g.n_pad <= 16 && dynconv::fused_conv_supported(g);
    const bool premix_ok = dynconv::premix_conv_supported(g);
    if (policy == DYNCONV_POLICY_FUSED) {
        if (!fused_ok)
            return fail(DYNCONV_ERR_UNSUPPORTED,
                        "fused path needs n <= 4, even W, Ho*Wo <= 256 and the 4 example tiles in LDS (n=%d, Ho*Wo=%d)",
                        g.n, g.P);
        out = policy;
        return DYNCONV_OK;
    }
    if (policy == DYNCONV_POLICY_PREMIX) {
        if (!premix_ok)
            return fail(DYNCONV_ERR_UNSUPPORTED, "premix path: input row band does not fit in LDS");
        out = policy;
        return DYNCONV_OK;
    }
    // AUTO: fuse when one example's mixed kernel is at least its input plus output.
    const long wb_bytes = kernel_elems(g) * (long)esize(g);
    const long xy_bytes = ((long)g.Cin * g.H * g.W + (long)g.Cout * g.P) * (long)esize(g);
    if (fused_ok && wb_bytes >= xy_bytes) out = DYNCONV_POLICY_FUSED;
    else if (premix_ok) out = DYNCONV_POLICY_PREMIX;
    else if (fused_ok) out = DYNCONV_POLICY_FUSED;
    else return fail(DYNCONV_ERR_UNSUPPORTED, "no convolution path fits this layer in LDS");
    return DYNCONV_OK;
}

// Workspace of the resolved policy; pieces are 256-byte aligned.
size_t forward_ws(const dynconv::Geom &g, int32_t policy) {
    if (depthwise(g))
        return policy == DYNCONV_POLICY_PREMIX ? round_up((size_t)g.B * kernel_elems(g) * esize(g), kWsAlign) : 0;
    if (!g.bf16) return round_up((size_t)g.B * kernel_elems(g) * sizeof(float), kWsAlign);
    if (wide(g))  // many experts: the bank in the conv's weight order, then W_b
        return round_up(dynconv::wide_bank_bytes(g), kWsAlign) + round_up(dynconv::premixed_bytes(g), kWsAlign);
    size_t ws = round_up(dynconv::packed_experts_bytes(g), kWsAlign);
    if (policy == DYNCONV_POLICY_PREMIX) ws += round_up(dynconv::premixed_bytes(g), kWsAlign);
    return ws;
}

dynconv_status_t hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess)
        return fail(DYNCONV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// bf16 layers with groups == 1 keep a packed bank: [t][o][c'][i'] for at most
// 16 experts, the wide layout [i][t][o][c'] for more.
bool packable(const dynconv::Geom &g) {
    return g.bf16 && g.groups == 1 && (g.n_pad <= 16 || dynconv::pack_wide_supported(g));
}
size_t packed_bank_bytes(const dynconv::Geom &g) {
    return wide(g) ? dynconv::wide_bank_bytes(g) : dynconv::packed_experts_bytes(g);
}

// bf16, groups == 1: the convolution from a packed bank. `ws` holds the
// premixed kernels for the PREMIX policy.
dynconv_status_t forward_from_packed(const dynconv::Geom &g, int32_t p, const void *x,
                                     const uint16_t *packed, const float *alpha, void *y,
                                     char *ws, hipStream_t st, dynconv::ChanAttn att = {}) {
    if (p == DYNCONV_POLICY_FUSED)
        return hip_status(dynconv::launch_conv_fused(g, static_cast<const uint16_t *>(x), packed,
                                                     alpha, static_cast<uint16_t *>(y), st, att),
                          "fused convolution launch");
    uint16_t *wt = reinterpret_cast<uint16_t *>(ws);
    hipError_t e = dynconv::launch_premix(g, alpha, packed, wt, st, att);
    if (e != hipSuccess) return hip_status(e, "premix launch");
    return hip_status(dynconv::launch_conv_premix(g, static_cast<const uint16_t *>(x), wt,
                                                  static_cast<uint16_t *>(y), st, att),
                      "convolution launch");
}

// Policy of a bf16 groups == 1 layer with channel attentions: the fused path
// where the small-image 3x3 kernel takes them, else PREMIX (AUTO resolves as
// for the plain layer, then falls back to PREMIX).
dynconv_status_t resolve_attn_policy(const dynconv::Geom &g, int32_t policy, int32_t &out) {
    if (policy == DYNCONV_POLICY_FUSED && !dynconv::fused_wave_attn_ok(g))
        return fail(DYNCONV_ERR_UNSUPPORTED,
                    "channel attentions on the fused path need the 3x3 pad-1 small-image kernel (n <= 4, up to "
                    "14x14, Cin <= 768)");
    dynconv_status_t s = resolve_policy(g, policy, out);
    if (s != DYNCONV_OK) return s;
    if (out == DYNCONV_POLICY_FUSED && !dynconv::fused_wave_attn_ok(g))
        return resolve_policy(g, DYNCONV_POLICY_PREMIX, out);
    return DYNCONV_OK;
}

// The forward of dynconv_forward and dynconv_forward_attn.
dynconv_status_t forward_impl(const dynconv_desc_t *desc, int32_t policy, const void *x,
                              const void *experts, const float *alpha, void *y, void *workspace,
                              size_t workspace_bytes, void *stream, dynconv::ChanAttn att) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    if (!x || !experts || !alpha || !y)
        return fail(DYNCONV_ERR_INVALID_ARG, "x, experts, alpha and y must not be NULL");
    if (!aligned16(x) || !aligned16(experts) || !aligned16(alpha) || !aligned16(y) ||
        (att.in && !aligned16(att.in)) || (att.out && !aligned16(att.out)))
        return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const bool attn = att.in || att.out;
    if (attn && wide(g))
        return fail(DYNCONV_ERR_UNSUPPORTED, "channel attentions support n <= 16 experts on bf16 groups == 1 layers");
    int32_t p;
    if (attn && !depthwise(g) && g.bf16) {
        s = resolve_attn_policy(g, policy, p);
    } else {
        s = resolve_policy(g, policy, p);
    }
    if (s != DYNCONV_OK) return s;
    const size_t need = forward_ws(g, p);
    if (need > 0 && (workspace_bytes < need || !workspace || !aligned16(workspace)))
        return fail(DYNCONV_ERR_WORKSPACE, "forward needs %zu bytes of 16-byte aligned workspace (got %zu)",
                    need, workspace_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    hipError_t e;
    if (depthwise(g)) {
        const void *wm = nullptr;
        if (p == DYNCONV_POLICY_PREMIX) {
            e = dynconv::launch_mix_natural(g, kernel_elems(g), alpha, experts, ws, st);
            if (e != hipSuccess) return hip_status(e, "dynconv_forward mix launch");
            wm = ws;
        }
        return hip_status(dynconv::launch_conv_depthwise(g, x, experts, alpha, wm, y, st, att),
                          "dynconv_forward depthwise launch");
    }
    if (!g.bf16) {
        e = dynconv::launch_mix_natural(g, kernel_elems(g), alpha, experts, ws, st);
        if (e != hipSuccess) return hip_status(e, "dynconv_forward mix launch");
        return hip_status(dynconv::launch_conv_direct_f32(g, static_cast<const float *>(x),
                                                          reinterpret_cast<const float *>(ws),
                                                          static_cast<float *>(y), st, att),
                          "dynconv_forward conv launch");
    }
    if (wide(g)) {
        uint16_t *bank = reinterpret_cast<uint16_t *>(ws);
        uint16_t *wt = reinterpret_cast<uint16_t *>(ws + round_up(dynconv::wide_bank_bytes(g), kWsAlign));
        e = dynconv::launch_pack_wide(g, static_cast<const uint16_t *>(experts), bank, st);
        if (e != hipSuccess) return hip_status(e, "dynconv_forward wide pack launch");
        e = dynconv::launch_mix_wide(g, (long)g.KT * g.Cout * g.Cin_pad, alpha, bank, wt, st, true);
        if (e != hipSuccess) return hip_status(e, "dynconv_forward wide mix launch");
        return hip_status(dynconv::launch_conv_premix(g, static_cast<const uint16_t *>(x), wt,
                                                      static_cast<uint16_t *>(y), st),
                          "convolution launch");
    }
    uint16_t *packed = reinterpret_cast<uint16_t *>(ws);
    e = dynconv::launch_pack_experts(g, static_cast<const uint16_t *>(experts), packed, st);
    if (e != hipSuccess) return hip_status(e, "dynconv_forward pack launch");
    return forward_from_packed(g, p, x, packed, alpha, y,
                               ws + round_up(dynconv::packed_experts_bytes(g), kWsAlign), st, att);
}

// The input gradient of a stride-1 layer is the forward layer applied to
// dy with the transposed, flipped bank and padding k - 1 - p: `t` is that
// layer's descriptor (input dy [B,Cout,Ho,Wo], output dx [B,Cin,H,W]).
// The data gradient runs as the forward layer on the transposed, flipped bank
// when that layer exists (stride 1, square kernel, padding below the kernel
// size); otherwise W_b is mixed into the workspace and a direct transposed
// convolution gathers each dx element.
bool backward_data_via_forward(const dynconv::Geom &g) {
    return g.stride == 1 && g.KH == g.KW && g.pad <= g.KH - 1;
}

size_t backward_data_direct_ws(const dynconv::Geom &g) {
    return round_up((size_t)g.B * kernel_elems(g) * esize(g), kWsAlign);
}

dynconv_status_t backward_data_desc(const dynconv_desc_t *desc, dynconv::Geom &g, dynconv_desc_t &t) {
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    t = *desc;
    if (!backward_data_via_forward(g)) return DYNCONV_OK;
    t.Cin = desc->Cout;
    t.Cout = desc->Cin;
    t.H = g.Ho;
    t.W = g.Wo;
    t.pad = g.KH - 1 - g.pad;
    dynconv::Geom gt;
    return check_desc(&t, gt, true);
}

size_t flipped_bytes(const dynconv::Geom &g) {
    return round_up((size_t)g.n * kernel_elems(g) * esize(g), kWsAlign);
}

size_t backward_weights_ws(const dynconv::Geom &g) { return round_up(dynconv::wgrad_bytes(g), kWsAlign); }

size_t route_backward_ws(const dynconv::Geom &g) {
    return 2 * round_up((size_t)g.B * g.Cin * sizeof(float), kWsAlign) +
           round_up((size_t)g.B * g.n * sizeof(float), kWsAlign);
}

// Workspace of dynconv_forward_sparse: W_b in the premix layout (through
// the packed bank for n <= 16, the wide bank otherwise), then, unless the
// one-pass band kernel takes the layer, the compacted active positions and
// the channel-innermost copy of x.
size_t sparse_tail_ws(const dynconv::Geom &g) {
    return round_up(dynconv::premixed_bytes(g), kWsAlign) +
           (dynconv::gated_one_pass(g) ? 0 : round_up(dynconv::sparse_index_bytes(g), kWsAlign));
}
size_t sparse_bank_bytes(const dynconv::Geom &g) {
    return round_up(wide(g) ? dynconv::wide_bank_bytes(g) : dynconv::packed_experts_bytes(g), kWsAlign);
}
size_t sparse_ws(const dynconv::Geom &g) { return sparse_bank_bytes(g) + sparse_tail_ws(g); }

// Pointer and overlap checks shared by the gated entry points (`bank` is the
// experts or the packed bank).
dynconv_status_t check_sparse_ptrs(const dynconv::Geom &g, const void *x, const void *bank, const float *alpha,
                                   const uint8_t *mask, const void *y) {
    if (!x || !bank || !alpha || !mask || !y)
        return fail(DYNCONV_ERR_INVALID_ARG, "x, the experts, alpha, mask and y must not be NULL");
    const void *ptrs[] = {x, bank, alpha, mask, y};
    for (const void *q : ptrs)
        if (!aligned16(q)) return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), y0 = reinterpret_cast<uintptr_t>(y);
    const uintptr_t xn = (uintptr_t)g.B * g.Cin * g.H * g.W * 2, yn = (uintptr_t)g.B * g.Cout * g.P * 2;
    if (x0 < y0 + yn && y0 < x0 + xn) return fail(DYNCONV_ERR_INVALID_ARG, "y must not overlap x");
    if (!dynconv::premix_conv_supported(g))
        return fail(DYNCONV_ERR_UNSUPPORTED, "the mixed kernels' layout does not fit this layer");
    return DYNCONV_OK;
}

// W_b from a bank in the premix kernels' layout (packed for n <= 16, wide
// otherwise) into `tail`, then the gated kernels (their index scratch after
// W_b).
dynconv_status_t sparse_from_bank(const dynconv::Geom &g, const void *x, const uint16_t *bank, const float *alpha,
                                  const uint8_t *mask, int32_t residual, void *y, char *tail, hipStream_t st) {
    uint16_t *wt = reinterpret_cast<uint16_t *>(tail);
    int *idx = reinterpret_cast<int *>(tail + round_up(dynconv::premixed_bytes(g), kWsAlign));
    const hipError_t e = wide(g) ? dynconv::launch_mix_wide(g, (long)g.KT * g.Cout * g.Cin_pad, alpha, bank, wt, st, true)
                                 : dynconv::launch_premix(g, alpha, bank, wt, st);
    if (e != hipSuccess) return hip_status(e, "gated evaluation mix launch");
    return hip_status(dynconv::launch_conv_sparse(g, static_cast<const uint16_t *>(x), wt, mask, residual, idx,
                                                  static_cast<uint16_t *>(y), st),
                      "gated evaluation launch");
}

dynconv_status_t check_sparse(const dynconv_desc_t *desc, dynconv::Geom &g, int32_t residual) {
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    if (!g.bf16 || g.groups != 1)
        return fail(DYNCONV_ERR_UNSUPPORTED, "gated evaluation supports bf16 layers with groups == 1");
    if (wide(g) && !dynconv::pack_wide_supported(g))
        return fail(DYNCONV_ERR_UNSUPPORTED, "more than 16 experts: one expert's Cin x kh x kw block must fit 64 KB");
    if (residual != 0 && residual != 1) return fail(DYNCONV_ERR_INVALID_ARG, "residual must be 0 or 1");
    if (g.B > 65535) return fail(DYNCONV_ERR_UNSUPPORTED, "gated evaluation supports B <= 65535 (got %d)", g.B);
    if (residual && (g.Cin != g.Cout || g.Ho != g.H || g.Wo != g.W))
        return fail(DYNCONV_ERR_INVALID_ARG, "a residual block needs Cin == Cout and an output the size of the input");
    return DYNCONV_OK;
}

// ---- workspace of the no-allocation forward --------------------------------
// A fixed device array per GPU (each GPU holds its own copy from the first
// use until the process ends). In host code `scratch` only names the symbol:
// its device address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = DYNCONV_NOALLOC_MAX_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
dynconv_status_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DYNCONV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DYNCONV_ERR_UNSUPPORTED, "device %d: the no-allocation forward supports devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(DYNCONV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DYNCONV_OK;
}
}  // namespace

extern "C" {

int32_t dynconv_abi_version(void) { return 1; }

const char *dynconv_status_string(dynconv_status_t s) {
    switch (s) {
    case DYNCONV_OK: return "ok";
    case DYNCONV_ERR_INVALID_ARG: return "invalid argument";
    case DYNCONV_ERR_UNSUPPORTED: return "unsupported layer";
    case DYNCONV_ERR_WORKSPACE: return "workspace missing or too small";
    case DYNCONV_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *dynconv_last_error(void) { return g_err; }

size_t dynconv_route_workspace_bytes(const dynconv_desc_t *desc) {
    dynconv::Geom g;
    if (check_desc(desc, g, false) != DYNCONV_OK) return 0;
    return round_up(dynconv::route_workspace_bytes(g), kWsAlign);
}

dynconv_status_t dynconv_route(const dynconv_desc_t *desc, const void *x, const float *fc_w,
                               const float *fc_b, int32_t mode, float temperature, float *alpha,
                               void *workspace, size_t workspace_bytes, void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, false);
    if (s != DYNCONV_OK) return s;
    if (!x || !fc_w || !alpha)
        return fail(DYNCONV_ERR_INVALID_ARG, "x, fc_w and alpha must not be NULL");
    if (!aligned16(x) || !aligned16(fc_w) || !aligned16(alpha) || (fc_b && !aligned16(fc_b)))
        return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (mode != DYNCONV_SIGMOID && mode != DYNCONV_SOFTMAX)
        return fail(DYNCONV_ERR_INVALID_ARG, "mode %d is not a dynconv_route_mode_t", mode);
    if (mode == DYNCONV_SOFTMAX && !(temperature > 0.f && std::isfinite(temperature)))
        return fail(DYNCONV_ERR_INVALID_ARG, "softmax temperature must be finite and > 0");
    if (g.n > 256) return fail(DYNCONV_ERR_UNSUPPORTED, "routing supports n <= 256 experts (got %d)", g.n);
    const size_t need = dynconv_route_workspace_bytes(desc);
    if (need > 0 && (workspace_bytes < need || !workspace || !aligned16(workspace)))
        return fail(DYNCONV_ERR_WORKSPACE, "route needs %zu bytes of 16-byte aligned workspace (got %zu)",
                    need, workspace_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(dynconv::launch_route(g, x, fc_w, fc_b, mode, temperature, workspace, alpha, st),
                      "dynconv_route launch");
}

dynconv_status_t dynconv_mix(const dynconv_desc_t *desc, const float *alpha, const void *experts,
                             void *mixed, void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    if (!alpha || !experts || !mixed)
        return fail(DYNCONV_ERR_INVALID_ARG, "alpha, experts and mixed must not be NULL");
    if (!aligned16(alpha) || !aligned16(experts) || !aligned16(mixed))
        return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(dynconv::launch_mix_natural(g, kernel_elems(g), alpha, experts, mixed, st),
                      "dynconv_mix launch");
}

int32_t dynconv_forward_policy(const dynconv_desc_t *desc) {
    dynconv::Geom g;
    if (check_desc(desc, g, true) != DYNCONV_OK) return -1;
    int32_t p;
    if (resolve_policy(g, DYNCONV_POLICY_AUTO, p) != DYNCONV_OK) return -1;
    return p;
}

size_t dynconv_forward_workspace_bytes(const dynconv_desc_t *desc, int32_t policy) {
    dynconv::Geom g;
    if (check_desc(desc, g, true) != DYNCONV_OK) return 0;
    int32_t p;
    if (resolve_policy(g, policy, p) != DYNCONV_OK) return 0;
    return forward_ws(g, p);
}

dynconv_status_t dynconv_forward(const dynconv_desc_t *desc, int32_t policy, const void *x,
                                 const void *experts, const float *alpha, void *y,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    return forward_impl(desc, policy, x, experts, alpha, y, workspace, workspace_bytes, stream, {});
}

dynconv_status_t dynconv_forward_noalloc(const dynconv_desc_t *desc, int32_t policy, const void *x,
                                         const void *experts, const float *alpha, void *y, void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    if (!x || !experts || !alpha || !y)
        return fail(DYNCONV_ERR_INVALID_ARG, "x, experts, alpha and y must not be NULL");
    if (!aligned16(x) || !aligned16(experts) || !aligned16(alpha) || !aligned16(y))
        return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    int32_t p;
    s = resolve_policy(g, policy, p);
    if (s != DYNCONV_OK) return s;
    const size_t need = forward_ws(g, p);
    if (need > kScratchBytes)
        return fail(DYNCONV_ERR_UNSUPPORTED,
                    "this layer needs %zu bytes of workspace; the no-allocation forward holds %zu (use dynconv_forward "
                    "with a caller-provided workspace)",
                    need, kScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        s = scratch_address(&ws);
        if (s != DYNCONV_OK) return s;
    }
    return forward_impl(desc, policy, x, experts, alpha, y, ws, need, stream, {});
}

size_t dynconv_forward_attn_workspace_bytes(const dynconv_desc_t *desc, int32_t policy) {
    dynconv::Geom g;
    if (check_desc(desc, g, true) != DYNCONV_OK) return 0;
    int32_t p;
    if (wide(g)) return 0;  // channel attentions: n <= 16 on bf16 groups == 1 layers
    if (!depthwise(g) && g.bf16) {
        if (resolve_attn_policy(g, policy, p) != DYNCONV_OK) return 0;
    } else if (resolve_policy(g, policy, p) != DYNCONV_OK) {
        return 0;
    }
    return forward_ws(g, p);
}

dynconv_status_t dynconv_forward_attn(const dynconv_desc_t *desc, int32_t policy, const void *x,
                                      const void *experts, const float *alpha, const float *a_in,
                                      const float *a_out, void *y, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    dynconv::ChanAttn att;
    att.in = a_in;
    att.out = a_out;
    return forward_impl(desc, policy, x, experts, alpha, y, workspace, workspace_bytes, stream, att);
}

size_t dynconv_route_attn_workspace_bytes(const dynconv_desc_t *desc) {
    dynconv::Geom g;
    if (check_desc(desc, g, true) != DYNCONV_OK) return 0;
    return round_up((size_t)g.B * g.Cin * sizeof(float), kWsAlign);
}

dynconv_status_t dynconv_route_attn(const dynconv_desc_t *desc, const void *x, const float *fc_w,
                                    const float *fc_b, int32_t mode, float temperature,
                                    const float *fc_w_in, const float *fc_b_in, const float *fc_w_out,
                                    const float *fc_b_out, float *alpha, float *a_in, float *a_out,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    if (!x || !fc_w || !fc_w_in || !fc_w_out || !alpha || !a_in || !a_out)
        return fail(DYNCONV_ERR_INVALID_ARG, "x, the three FC weights and the three outputs must not be NULL");
    const void *ptrs[] = {x, fc_w, fc_b, fc_w_in, fc_b_in, fc_w_out, fc_b_out, alpha, a_in, a_out};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (mode != DYNCONV_SIGMOID && mode != DYNCONV_SOFTMAX)
        return fail(DYNCONV_ERR_INVALID_ARG, "mode %d is not a dynconv_route_mode_t", mode);
    if (mode == DYNCONV_SOFTMAX && !(temperature > 0.f && std::isfinite(temperature)))
        return fail(DYNCONV_ERR_INVALID_ARG, "softmax temperature must be finite and > 0");
    if (g.n > 256 || g.Cin > 256 || d_cout(desc) > 256)
        return fail(DYNCONV_ERR_UNSUPPORTED, "attention routing supports n, Cin and Cout <= 256 (got %d, %d, %d)",
                    g.n, g.Cin, d_cout(desc));
    const size_t need = dynconv_route_attn_workspace_bytes(desc);
    if (workspace_bytes < need || !workspace || !aligned16(workspace))
        return fail(DYNCONV_ERR_WORKSPACE, "attention routing needs %zu bytes of 16-byte aligned workspace (got %zu)",
                    need, workspace_bytes);
    const float *ws_[3] = {fc_w, fc_w_in, fc_w_out};
    const float *bs_[3] = {fc_b, fc_b_in, fc_b_out};
    const int nout[3] = {g.n, g.Cin, d_cout(desc)};
    const int modes[3] = {mode, DYNCONV_SIGMOID, DYNCONV_SIGMOID};
    float *outs[3] = {alpha, a_in, a_out};
    return hip_status(dynconv::launch_route_heads(g, x, 3, ws_, bs_, nout, modes, temperature,
                                                  static_cast<float *>(workspace), outs,
                                                  static_cast<hipStream_t>(stream)),
                      "dynconv_route_attn launch");
}

size_t dynconv_packed_experts_bytes(const dynconv_desc_t *desc) {
    dynconv::Geom g;
    if (check_desc(desc, g, true) != DYNCONV_OK || !packable(g)) return 0;
    return packed_bank_bytes(g);
}

dynconv_status_t dynconv_pack_experts(const dynconv_desc_t *desc, const void *experts,
                                      void *packed, size_t packed_bytes, void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    if (!packable(g))
        return fail(DYNCONV_ERR_UNSUPPORTED,
                    "packing applies to bf16 layers with groups == 1 (more than 16 experts: one expert's Cin x kh x "
                    "kw block must fit 64 KB)");
    if (!experts || !packed) return fail(DYNCONV_ERR_INVALID_ARG, "experts and packed must not be NULL");
    if (!aligned16(experts) || !aligned16(packed))
        return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (packed_bytes < packed_bank_bytes(g))
        return fail(DYNCONV_ERR_INVALID_ARG, "packed holds %zu bytes, %zu needed", packed_bytes,
                    packed_bank_bytes(g));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (wide(g))
        return hip_status(dynconv::launch_pack_wide(g, static_cast<const uint16_t *>(experts),
                                                    static_cast<uint16_t *>(packed), st),
                          "dynconv_pack_experts launch");
    return hip_status(dynconv::launch_pack_experts(g, static_cast<const uint16_t *>(experts),
                                                   static_cast<uint16_t *>(packed), st),
                      "dynconv_pack_experts launch");
}

size_t dynconv_forward_packed_workspace_bytes(const dynconv_desc_t *desc, int32_t policy) {
    dynconv::Geom g;
    if (check_desc(desc, g, true) != DYNCONV_OK || !packable(g)) return 0;
    int32_t p;
    if (resolve_policy(g, policy, p) != DYNCONV_OK) return 0;
    return p == DYNCONV_POLICY_PREMIX || wide(g) ? round_up(dynconv::premixed_bytes(g), kWsAlign) : 0;
}

dynconv_status_t dynconv_forward_packed(const dynconv_desc_t *desc, int32_t policy,
                                        const void *x, const void *packed, const float *alpha,
                                        void *y, void *workspace, size_t workspace_bytes,
                                        void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    if (!x || !packed || !alpha || !y)
        return fail(DYNCONV_ERR_INVALID_ARG, "x, packed, alpha and y must not be NULL");
    if (!aligned16(x) || !aligned16(packed) || !aligned16(alpha) || !aligned16(y))
        return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (!packable(g))
        return fail(DYNCONV_ERR_UNSUPPORTED, "packed experts apply to bf16 layers with groups == 1");
    int32_t p;
    s = resolve_policy(g, policy, p);
    if (s != DYNCONV_OK) return s;
    const size_t need =
        p == DYNCONV_POLICY_PREMIX || wide(g) ? round_up(dynconv::premixed_bytes(g), kWsAlign) : 0;
    if (need > 0 && (workspace_bytes < need || !workspace || !aligned16(workspace)))
        return fail(DYNCONV_ERR_WORKSPACE, "forward_packed needs %zu bytes of 16-byte aligned workspace (got %zu)",
                    need, workspace_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (wide(g)) {
        // many experts: W_b from the wide bank on the matrix cores, then the premix convolution
        uint16_t *wt = static_cast<uint16_t *>(workspace);
        hipError_t e = dynconv::launch_mix_wide(g, (long)g.KT * g.Cout * g.Cin_pad, alpha,
                                                static_cast<const uint16_t *>(packed), wt, st, true);
        if (e != hipSuccess) return hip_status(e, "dynconv_forward_packed wide mix launch");
        return hip_status(dynconv::launch_conv_premix(g, static_cast<const uint16_t *>(x), wt,
                                                      static_cast<uint16_t *>(y), st),
                          "dynconv_forward_packed convolution launch");
    }
    return forward_from_packed(g, p, x, static_cast<const uint16_t *>(packed), alpha, y,
                               static_cast<char *>(workspace), st);
}

size_t dynconv_backward_data_workspace_bytes(const dynconv_desc_t *desc, int32_t policy) {
    dynconv::Geom g;
    dynconv_desc_t t;
    if (backward_data_desc(desc, g, t) != DYNCONV_OK) return 0;
    if (!backward_data_via_forward(g)) {
        const bool known = policy == DYNCONV_POLICY_AUTO || policy == DYNCONV_POLICY_PREMIX ||
                           policy == DYNCONV_POLICY_FUSED;
        return known ? backward_data_direct_ws(g) : 0;
    }
    const size_t fw = dynconv_forward_workspace_bytes(&t, policy);
    dynconv::Geom gt;
    int32_t p;
    if (check_desc(&t, gt, true) != DYNCONV_OK || resolve_policy(gt, policy, p) != DYNCONV_OK) return 0;
    return flipped_bytes(g) + fw;
}

dynconv_status_t dynconv_backward_data(const dynconv_desc_t *desc, int32_t policy, const void *dy,
                                       const void *experts, const float *alpha, void *dx, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    dynconv::Geom g;
    dynconv_desc_t t;
    dynconv_status_t s = backward_data_desc(desc, g, t);
    if (s != DYNCONV_OK) return s;
    if (!dy || !experts || !alpha || !dx)
        return fail(DYNCONV_ERR_INVALID_ARG, "dy, experts, alpha and dx must not be NULL");
    if (!aligned16(dy) || !aligned16(experts) || !aligned16(alpha) || !aligned16(dx))
        return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (!backward_data_via_forward(g)) {
        if (policy != DYNCONV_POLICY_AUTO && policy != DYNCONV_POLICY_PREMIX && policy != DYNCONV_POLICY_FUSED)
            return fail(DYNCONV_ERR_INVALID_ARG, "policy %d is not a dynconv_policy_t", policy);
        const size_t need = backward_data_direct_ws(g);
        if (workspace_bytes < need || !workspace || !aligned16(workspace))
            return fail(DYNCONV_ERR_WORKSPACE, "backward_data needs %zu bytes of 16-byte aligned workspace (got %zu)",
                        need, workspace_bytes);
        hipStream_t st = static_cast<hipStream_t>(stream);
        s = hip_status(dynconv::launch_mix_natural(g, kernel_elems(g), alpha, experts, workspace, st),
                       "backward_data mix launch");
        if (s != DYNCONV_OK) return s;
        return hip_status(dynconv::launch_dgrad_direct(g, dy, workspace, dx, st), "backward_data launch");
    }
    dynconv::Geom gt;
    int32_t p;
    s = check_desc(&t, gt, true);
    if (s != DYNCONV_OK) return s;
    s = resolve_policy(gt, policy, p);
    if (s != DYNCONV_OK) return s;
    const size_t flip = flipped_bytes(g);
    const size_t need = flip + forward_ws(gt, p);
    if (workspace_bytes < need || !workspace || !aligned16(workspace))
        return fail(DYNCONV_ERR_WORKSPACE, "backward_data needs %zu bytes of 16-byte aligned workspace (got %zu)",
                    need, workspace_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    s = hip_status(dynconv::launch_flip_experts(g, experts, ws, st), "backward_data flip launch");
    if (s != DYNCONV_OK) return s;
    return forward_impl(&t, policy, dy, ws, alpha, dx, ws + flip, workspace_bytes - flip, stream, {});
}

size_t dynconv_backward_weights_workspace_bytes(const dynconv_desc_t *desc) {
    dynconv::Geom g;
    if (check_desc(desc, g, true) != DYNCONV_OK) return 0;
    return backward_weights_ws(g);
}

dynconv_status_t dynconv_backward_weights(const dynconv_desc_t *desc, const void *x, const void *dy,
                                          const void *experts, const float *alpha, float *dalpha,
                                          float *dexperts, void *workspace, size_t workspace_bytes,
                                          void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    if (!x || !dy || !experts || !alpha)
        return fail(DYNCONV_ERR_INVALID_ARG, "x, dy, experts and alpha must not be NULL");
    if (!dalpha && !dexperts)
        return fail(DYNCONV_ERR_INVALID_ARG, "dalpha and dexperts are both NULL: nothing to compute");
    const void *ptrs[] = {x, dy, experts, alpha, dalpha, dexperts};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (g.B > 65535) return fail(DYNCONV_ERR_UNSUPPORTED, "backward_weights supports B <= 65535 (got %d)", g.B);
    if (depthwise(g) && !dynconv::wgrad_dw_supported(g))
        return fail(DYNCONV_ERR_UNSUPPORTED, "depthwise backward_weights supports up to 64 kernel taps");
    const size_t need = backward_weights_ws(g);
    if (workspace_bytes < need || !workspace || !aligned16(workspace))
        return fail(DYNCONV_ERR_WORKSPACE, "backward_weights needs %zu bytes of 16-byte aligned workspace (got %zu)",
                    need, workspace_bytes);
    return hip_status(dynconv::launch_backward_weights(g, x, dy, experts, alpha, static_cast<float *>(workspace),
                                                       dalpha, dexperts, static_cast<hipStream_t>(stream)),
                      "dynconv_backward_weights launch");
}

size_t dynconv_backward_data_attn_workspace_bytes(const dynconv_desc_t *desc, int32_t policy) {
    dynconv::Geom g;
    dynconv_desc_t t;
    if (backward_data_desc(desc, g, t) != DYNCONV_OK || !backward_data_via_forward(g)) return 0;
    const size_t fw = dynconv_forward_attn_workspace_bytes(&t, policy);
    dynconv::Geom gt;
    if (check_desc(&t, gt, true) != DYNCONV_OK || wide(gt)) return 0;
    int32_t p;
    const bool ok = (!depthwise(gt) && gt.bf16) ? resolve_attn_policy(gt, policy, p) == DYNCONV_OK
                                                 : resolve_policy(gt, policy, p) == DYNCONV_OK;
    return ok ? flipped_bytes(g) + fw : 0;
}

dynconv_status_t dynconv_backward_data_attn(const dynconv_desc_t *desc, int32_t policy, const void *dy,
                                            const void *experts, const float *alpha, const float *a_in,
                                            const float *a_out, void *dx, void *workspace, size_t workspace_bytes,
                                            void *stream) {
    dynconv::Geom g;
    dynconv_desc_t t;
    dynconv_status_t s = backward_data_desc(desc, g, t);
    if (s != DYNCONV_OK) return s;
    if (!dy || !experts || !alpha || !dx)
        return fail(DYNCONV_ERR_INVALID_ARG, "dy, experts, alpha and dx must not be NULL");
    const void *ptrs[] = {dy, experts, alpha, dx, a_in, a_out};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (!backward_data_via_forward(g))
        return fail(DYNCONV_ERR_UNSUPPORTED,
                    "backward_data_attn needs stride 1, a square kernel and pad <= k - 1 (the transposed layer)");
    const size_t flip = flipped_bytes(g);
    const size_t need = dynconv_backward_data_attn_workspace_bytes(desc, policy);
    if (need == 0) {
        // report the reason the transposed layer has no attention path
        dynconv::Geom gt;
        s = check_desc(&t, gt, true);
        if (s != DYNCONV_OK) return s;
        if (wide(gt))
            return fail(DYNCONV_ERR_UNSUPPORTED, "channel attentions support n <= 16 experts on bf16 groups == 1 layers");
        int32_t p;
        return (!depthwise(gt) && gt.bf16) ? resolve_attn_policy(gt, policy, p) : resolve_policy(gt, policy, p);
    }
    if (workspace_bytes < need || !workspace || !aligned16(workspace))
        return fail(DYNCONV_ERR_WORKSPACE,
                    "backward_data_attn needs %zu bytes of 16-byte aligned workspace (got %zu)", need, workspace_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    s = hip_status(dynconv::launch_flip_experts(g, experts, ws, st), "backward_data_attn flip launch");
    if (s != DYNCONV_OK) return s;
    // the transposed layer reads dy's channels (the layer's outputs, scaled by
    // a_out) and writes dx's channels (the layer's inputs, scaled by a_in)
    dynconv::ChanAttn att;
    att.in = a_out;
    att.out = a_in;
    return forward_impl(&t, policy, dy, ws, alpha, dx, ws + flip, workspace_bytes - flip, stream, att);
}

size_t dynconv_backward_weights_attn_workspace_bytes(const dynconv_desc_t *desc) {
    dynconv::Geom g;
    if (check_desc(desc, g, true) != DYNCONV_OK) return 0;
    return round_up(dynconv::wgrad_attn_bytes(g), kWsAlign);
}

dynconv_status_t dynconv_backward_weights_attn(const dynconv_desc_t *desc, const void *x, const void *dy,
                                               const void *experts, const float *alpha, const float *a_in,
                                               const float *a_out, float *dalpha, float *dexperts, float *da_in,
                                               float *da_out, void *workspace, size_t workspace_bytes,
                                               void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, true);
    if (s != DYNCONV_OK) return s;
    if (!x || !dy || !experts || !alpha)
        return fail(DYNCONV_ERR_INVALID_ARG, "x, dy, experts and alpha must not be NULL");
    if (!dalpha && !dexperts && !da_in && !da_out)
        return fail(DYNCONV_ERR_INVALID_ARG, "dalpha, dexperts, da_in and da_out are all NULL: nothing to compute");
    const void *ptrs[] = {x, dy, experts, alpha, a_in, a_out, dalpha, dexperts, da_in, da_out};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (g.B > 65535) return fail(DYNCONV_ERR_UNSUPPORTED, "backward_weights_attn supports B <= 65535 (got %d)", g.B);
    if (depthwise(g) && !dynconv::wgrad_dw_supported(g))
        return fail(DYNCONV_ERR_UNSUPPORTED, "depthwise backward_weights_attn supports up to 64 kernel taps");
    const size_t need = round_up(dynconv::wgrad_attn_bytes(g), kWsAlign);
    if (workspace_bytes < need || !workspace || !aligned16(workspace))
        return fail(DYNCONV_ERR_WORKSPACE,
                    "backward_weights_attn needs %zu bytes of 16-byte aligned workspace (got %zu)", need,
                    workspace_bytes);
    dynconv::ChanAttn att;
    att.in = a_in;
    att.out = a_out;
    return hip_status(dynconv::launch_backward_weights_attn(g, x, dy, experts, alpha, att,
                                                            static_cast<float *>(workspace), dalpha, dexperts,
                                                            da_in, da_out, static_cast<hipStream_t>(stream)),
                      "dynconv_backward_weights_attn launch");
}

size_t dynconv_route_backward_workspace_bytes(const dynconv_desc_t *desc) {
    dynconv::Geom g;
    if (check_desc(desc, g, false) != DYNCONV_OK) return 0;
    return route_backward_ws(g);
}

dynconv_status_t dynconv_route_backward(const dynconv_desc_t *desc, const void *x, const float *fc_w,
                                        int32_t mode, float temperature, const float *alpha,
                                        const float *dalpha, float *dfc_w, float *dfc_b, void *dx,
                                        void *workspace, size_t workspace_bytes, void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_desc(desc, g, false);
    if (s != DYNCONV_OK) return s;
    if (!x || !fc_w || !alpha || !dalpha || !dfc_w)
        return fail(DYNCONV_ERR_INVALID_ARG, "x, fc_w, alpha, dalpha and dfc_w must not be NULL");
    const void *ptrs[] = {x, fc_w, alpha, dalpha, dfc_w, dfc_b, dx};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(DYNCONV_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (mode != DYNCONV_SIGMOID && mode != DYNCONV_SOFTMAX)
        return fail(DYNCONV_ERR_INVALID_ARG, "mode %d is not a dynconv_route_mode_t", mode);
    if (mode == DYNCONV_SOFTMAX && !(temperature > 0.f && std::isfinite(temperature)))
        return fail(DYNCONV_ERR_INVALID_ARG, "softmax temperature must be finite and > 0");
    if (g.n > 256) return fail(DYNCONV_ERR_UNSUPPORTED, "routing supports n <= 256 experts (got %d)", g.n);
    const size_t need = route_backward_ws(g);
    if (workspace_bytes < need || !workspace || !aligned16(workspace))
        return fail(DYNCONV_ERR_WORKSPACE, "route_backward needs %zu bytes of 16-byte aligned workspace (got %zu)",
                    need, workspace_bytes);
    char *ws = static_cast<char *>(workspace);
    const size_t bc = round_up((size_t)g.B * g.Cin * sizeof(float), kWsAlign);
    float *gap = reinterpret_cast<float *>(ws);
    float *dgap = reinterpret_cast<float *>(ws + bc);
    float *dz = reinterpret_cast<float *>(ws + 2 * bc);
    return hip_status(dynconv::launch_route_backward(g, x, fc_w, mode, temperature, alpha, dalpha, gap, dz, dgap,
                                                     dfc_w, dfc_b, dx, static_cast<hipStream_t>(stream)),
                      "dynconv_route_backward launch");
}

size_t dynconv_forward_sparse_workspace_bytes(const dynconv_desc_t *desc) {
    dynconv::Geom g;
    if (check_sparse(desc, g, 0) != DYNCONV_OK) return 0;
    return sparse_ws(g);
}

dynconv_status_t dynconv_forward_sparse(const dynconv_desc_t *desc, const void *x, const void *experts,
                                        const float *alpha, const uint8_t *mask, int32_t residual, void *y,
                                        void *workspace, size_t workspace_bytes, void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_sparse(desc, g, residual);
    if (s != DYNCONV_OK) return s;
    s = check_sparse_ptrs(g, x, experts, alpha, mask, y);
    if (s != DYNCONV_OK) return s;
    const size_t need = sparse_ws(g);
    if (workspace_bytes < need || !workspace || !aligned16(workspace))
        return fail(DYNCONV_ERR_WORKSPACE, "forward_sparse needs %zu bytes of 16-byte aligned workspace (got %zu)",
                    need, workspace_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    uint16_t *bank = reinterpret_cast<uint16_t *>(ws);
    const hipError_t e = wide(g) ? dynconv::launch_pack_wide(g, static_cast<const uint16_t *>(experts), bank, st)
                                 : dynconv::launch_pack_experts(g, static_cast<const uint16_t *>(experts), bank, st);
    if (e != hipSuccess) return hip_status(e, "dynconv_forward_sparse pack launch");
    return sparse_from_bank(g, x, bank, alpha, mask, residual, y, ws + sparse_bank_bytes(g), st);
}

size_t dynconv_forward_sparse_packed_workspace_bytes(const dynconv_desc_t *desc) {
    dynconv::Geom g;
    if (check_sparse(desc, g, 0) != DYNCONV_OK) return 0;
    return sparse_tail_ws(g);
}

dynconv_status_t dynconv_forward_sparse_packed(const dynconv_desc_t *desc, const void *x, const void *packed,
                                               const float *alpha, const uint8_t *mask, int32_t residual, void *y,
                                               void *workspace, size_t workspace_bytes, void *stream) {
    dynconv::Geom g;
    dynconv_status_t s = check_sparse(desc, g, residual);
    if (s != DYNCONV_OK) return s;
    s = check_sparse_ptrs(g, x, packed, alpha, mask, y);
    if (s != DYNCONV_OK) return s;
    const size_t need = sparse_tail_ws(g);
    if (workspace_bytes < need || !workspace || !aligned16(workspace))
        return fail(DYNCONV_ERR_WORKSPACE,
                    "forward_sparse_packed needs %zu bytes of 16-byte aligned workspace (got %zu)", need,
                    workspace_bytes);
    return sparse_from_bank(g, x, static_cast<const uint16_t *>(packed), alpha, mask, residual, y,
                            static_cast<char *>(workspace), static_cast<hipStream_t>(stream));
}

}  // extern "C"
