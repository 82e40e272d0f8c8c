/*
 * dynconv.h - C ABI of the MI355X (gfx950) CondConv-style dynamic convolution.
 *
 * The method (CondConv: Conditionally Parameterized Convolutions, abstract;
 * KernelWarehouse: Rethinking the Design of Dynamic Convolution, abstract):
 * each example b gets its own convolution kernel, a linear mixture
 *     W_b = sum_i alpha[b,i] * E_i
 * of n static expert kernels E_0..E_{n-1}, weighted by input-dependent
 * attentions alpha[b,:]; the layer output is one ordinary convolution of the
 * example with W_b. The attentions come from a router: global average pool
 * of the layer input, a fully connected layer with bias, then a sigmoid or a
 * softmax of the logits divided by a temperature (FMDConv: Fast
 * multi-attention dynamic convolution, abstract, which puts a temperature on
 * the kernel attention; the pages give no further detail of the router).
 *
 * Conventions shared by every entry point
 *   - Memory: every tensor pointer is a DEVICE pointer into memory the
 *     caller owns (for example a torch tensor's data_ptr()), densely packed
 *     in the row-major layout stated per argument. The library never
 *     allocates, frees or keeps a pointer after the call returns.
 *   - Alignment: tensor pointers must be 16-byte aligned.
 *   - Element types: x, experts, mixed kernels and y share desc->dtype
 *     (DYNCONV_F32: IEEE float32; DYNCONV_BF16: bfloat16). Attentions and
 *     router weights are always float32. bf16 arithmetic accumulates in
 *     float32; mixed kernels are rounded to bf16 (nearest-even) before the
 *     convolution's products; outputs are rounded to the output type.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the
 *     default stream) and the call returns without waiting. The library
 *     never synchronizes. Calls on one stream run in order.
 *   - Errors: every argument is checked on the host before anything is
 *     enqueued. On any error nothing is launched and no output is written;
 *     dynconv_last_error() then describes the failure (thread-local text).
 *     DYNCONV_ERR_HIP reports a failed launch (hipGetLastError after the
 *     launch). No C++ exception crosses this interface.
 *   - State: the library holds no state between calls besides the
 *     thread-local error text; calls from several threads are safe.
 *   - Supported shapes: groups == 1, or depthwise (groups == Cin == Cout).
 *     Other groupings return DYNCONV_ERR_UNSUPPORTED.
 */
#ifndef DYNCONV_H
#define DYNCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DYNCONV_OK = 0,
    DYNCONV_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad enum, misalignment */
    DYNCONV_ERR_UNSUPPORTED = 2, /* valid layer this library does not implement */
    DYNCONV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    DYNCONV_ERR_HIP = 4          /* the HIP runtime refused a launch */
} dynconv_status_t;

typedef enum { DYNCONV_F32 = 0, DYNCONV_BF16 = 1 } dynconv_dtype_t;

/* Router nonlinearity: sigmoid of the logits (attentions not normalised),
 * or softmax of logits / temperature (attentions sum to 1). */
typedef enum { DYNCONV_SIGMOID = 0, DYNCONV_SOFTMAX = 1 } dynconv_route_mode_t;

/* How dynconv_forward builds each example's kernel.
 *   PREMIX: one kernel writes every W_b to the workspace, the convolution
 *           reads it back (cheap when W_b is small next to the activations).
 *   FUSED:  the convolution mixes W_b tile by tile from the expert bank as
 *           it goes; W_b never reaches memory (when W_b per example is at
 *           least the example's activations, the ResNet-50-shaped case).
 *   AUTO:   FUSED when the fused kernel supports the shape and one
 *           example's mixed kernel is at least as large as its input plus
 *           output; otherwise PREMIX. */
typedef enum {
    DYNCONV_POLICY_AUTO = 0,
    DYNCONV_POLICY_PREMIX = 1,
    DYNCONV_POLICY_FUSED = 2
} dynconv_policy_t;

/* Layer descriptor. Output size: Ho = (H + 2*pad - kh)/stride + 1, likewise
 * Wo; both must be >= 1. Convolution is cross-correlation with zero padding,
 * dilation 1 and no bias. */
typedef struct {
    int32_t B;       /* examples in the batch, >= 1 */
    int32_t Cin;     /* input channels */
    int32_t H, W;    /* input height, width */
    int32_t Cout;    /* output channels */
    int32_t kh, kw;  /* kernel height, width */
    int32_t stride;  /* >= 1, both directions */
    int32_t pad;     /* >= 0, zero padding on every side */
    int32_t groups;  /* 1, or Cin (== Cout) for depthwise */
    int32_t n;       /* experts, >= 1 */
    int32_t dtype;   /* dynconv_dtype_t */
} dynconv_desc_t;

/* Routing: alpha[b,i] for every example.
 *   gap[b,c] = mean over h,w of x[b,c,h,w]
 *   z[b,i]   = sum_c fc_w[i,c] * gap[b,c] + fc_b[i]
 *   alpha    = sigmoid(z)                       (mode DYNCONV_SIGMOID)
 *            = softmax over i of z[b,i] / temperature (mode DYNCONV_SOFTMAX)
 * (KernelWarehouse abstract: the attentions depend on the input; FMDConv
 * abstract: temperature-scaled kernel attention.)
 * Arguments: x [B,Cin,H,W] (dtype), fc_w [n,Cin] float32, fc_b [n] float32 or
 * NULL for no bias, temperature > 0 (ignored for sigmoid), alpha [B,n]
 * float32 (written). workspace: device memory of at least
 * dynconv_route_workspace_bytes(desc) bytes (may be NULL when that is 0,
 * which is the case from 64 examples up, routed with one workgroup per
 * example). Below 64 examples the workspace starts with one 32-bit ticket
 * counter per example (the size rounded up to 256 bytes), followed by the
 * B*Cin channel means: the counters MUST be zero when a workspace is first
 * used (allocate it zero-filled, e.g. hipMemset once); every call leaves
 * them zero again, so a workspace can be reused by later calls (also from a
 * captured graph) without clearing. Two calls that run at the same time
 * must not share a workspace. Planes too large for the one-launch routers
 * (more than 8192 bf16 or 4096 float32 elements) use the workspace as
 * B*Cin channel means only, whose contents on entry do not matter. Only
 * desc->B, Cin, H, W, n and dtype are read. The result is deterministic:
 * the counters only pick which workgroup finishes an example, and every sum
 * runs in a fixed order. */
dynconv_status_t dynconv_route(const dynconv_desc_t *desc, const void *x,
                               const float *fc_w, const float *fc_b,
                               int32_t mode, float temperature, float *alpha,
                               void *workspace, size_t workspace_bytes,
                               void *stream);
size_t dynconv_route_workspace_bytes(const dynconv_desc_t *desc);

/* Mixing: mixed[b] = sum_i alpha[b,i] * experts[i] for every example
 * (KernelWarehouse abstract: a linear mixture of n static kernels).
 * experts [n,Cout,Cin/groups,kh,kw] (dtype), alpha [B,n] float32,
 * mixed [B,Cout,Cin/groups,kh,kw] (dtype, written). Sums run in float32 in
 * expert order; bf16 results are rounded to nearest-even once. */
dynconv_status_t dynconv_mix(const dynconv_desc_t *desc, const float *alpha,
                             const void *experts, void *mixed, void *stream);

/* The layer: y[b] = conv(x[b], sum_i alpha[b,i] * experts[i]) for every
 * example (CondConv abstract: a specialised kernel per example, mixed once,
 * then one ordinary convolution). x [B,Cin,H,W], experts
 * [n,Cout,Cin/groups,kh,kw], y [B,Cout,Ho,Wo] (all dtype); alpha [B,n]
 * float32, typically written by dynconv_route (one routing may feed several
 * layers). policy: dynconv_policy_t; DYNCONV_POLICY_AUTO unless a test needs
 * a particular path (FUSED returns DYNCONV_ERR_UNSUPPORTED for shapes the
 * fused kernel does not cover). workspace: at least
 * dynconv_forward_workspace_bytes(desc, policy) bytes of device memory
 * (contents on entry do not matter; clobbered). Deterministic: two calls on
 * the same inputs give bitwise-equal y. bf16 layers with groups == 1 and
 * more than 16 experts (KernelWarehouse abstract: n > 100) run on
 * DYNCONV_POLICY_PREMIX only (FUSED returns DYNCONV_ERR_UNSUPPORTED): the
 * bank is put in the convolution's weight order and mixed on the matrix
 * cores with the experts as the reduction dimension; one expert's
 * Cin * kh * kw bf16 values must fit 64 KB. */
dynconv_status_t dynconv_forward(const dynconv_desc_t *desc, int32_t policy,
                                 const void *x, const void *experts,
                                 const float *alpha, void *y, void *workspace,
                                 size_t workspace_bytes, void *stream);
size_t dynconv_forward_workspace_bytes(const dynconv_desc_t *desc, int32_t policy);

/* Expert bank in the layout the bf16 MFMA path reads (bf16 layers with
 * groups == 1): for at most 16 experts packed[t][o][c'][i'] with t = kh*kw
 * tap (row-major), o = output channel, c' < Cin rounded up to 32 (zero beyond
 * Cin), and i' < n rounded up to even (zero beyond n), so that two experts'
 * values of one kernel element share a 32-bit word; for more experts (the
 * many-expert layers of KernelWarehouse: Rethinking the Design of Dynamic
 * Convolution, abstract) packed[i][t][o][c'], the weight order the matrix-core
 * mix over the expert dimension reads (one expert's Cin x kh x kw block must
 * fit 64 KB, else DYNCONV_ERR_UNSUPPORTED). A pure layout transform of the
 * static experts: a bank can be packed once and then reused by
 * dynconv_forward_packed for every batch. dynconv_forward packs internally on
 * every call. experts [n,Cout,Cin,kh,kw] bf16; packed: device memory of at
 * least dynconv_packed_experts_bytes(desc) bytes (written). Unsupported
 * layers return DYNCONV_ERR_UNSUPPORTED (and 0 bytes). */
size_t dynconv_packed_experts_bytes(const dynconv_desc_t *desc);
dynconv_status_t dynconv_pack_experts(const dynconv_desc_t *desc, const void *experts,
                                      void *packed, size_t packed_bytes, void *stream);

/* dynconv_forward with an expert bank already packed by dynconv_pack_experts
 * (bf16, groups == 1). Same arguments, policies and results as
 * dynconv_forward; the workspace holds only what the policy needs besides
 * the packed bank (the premixed kernels for DYNCONV_POLICY_PREMIX and for
 * banks of more than 16 experts, nothing for DYNCONV_POLICY_FUSED). */
dynconv_status_t dynconv_forward_packed(const dynconv_desc_t *desc, int32_t policy,
                                        const void *x, const void *packed,
                                        const float *alpha, void *y, void *workspace,
                                        size_t workspace_bytes, void *stream);
size_t dynconv_forward_packed_workspace_bytes(const dynconv_desc_t *desc, int32_t policy);

/* dynconv_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The library keeps one fixed scratch array
 * of DYNCONV_NOALLOC_MAX_BYTES per GPU (held from the first call on that GPU
 * until the process ends) and uses it as the workspace; the call itself
 * allocates and frees nothing. The caller still owns x, experts, alpha and y
 * (as dynconv_forward); the call runs on the current device, which must be
 * the one `stream` belongs to. Layers whose workspace
 * (dynconv_forward_workspace_bytes(desc, policy)) exceeds the array return
 * DYNCONV_ERR_UNSUPPORTED before anything is enqueued. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads) race and must be serialised by the caller; calls on
 * one stream are ordered and safe. Nothing in the array needs to start at
 * zero. Results are bitwise those of dynconv_forward with the same policy. */
#define DYNCONV_NOALLOC_MAX_BYTES (64ull << 20)
dynconv_status_t dynconv_forward_noalloc(const dynconv_desc_t *desc, int32_t policy, const void *x,
                                         const void *experts, const float *alpha, void *y, void *stream);

/* FMDConv's multi-attention layer (FMDConv: Fast multi-attention dynamic
 * convolution via speed-accuracy trade-off, abstract: input attention,
 * temperature-degraded kernel attention and output attention). The page
 * gives no formulas; the reading implemented: each attention is a head of
 * its own on the layer input's global average pool (an FC with bias), the
 * kernel attention with `mode` (softmax(z/T) for the temperature form), the
 * input and output attentions with a sigmoid; the input attention scales the
 * example's input channels before the convolution and the output attention
 * its output channels after it:
 *   y[b,o] = a_out[b,o] * conv(a_in[b,:] * x[b], sum_i alpha[b,i] E_i)[o].
 *
 * dynconv_route_attn: the three heads from one pooling of x [B,Cin,H,W]
 * (dtype). fc_w [n,Cin], fc_w_in [Cin,Cin], fc_w_out [Cout,Cin] float32,
 * row-major; the biases fc_b [n], fc_b_in [Cin], fc_b_out [Cout] may be NULL.
 * Writes alpha [B,n], a_in [B,Cin], a_out [B,Cout] (float32). n, Cin and Cout
 * <= 256 (DYNCONV_ERR_UNSUPPORTED otherwise). workspace: at least
 * dynconv_route_attn_workspace_bytes(desc) bytes (the B*Cin channel means;
 * clobbered). Reads desc->B, Cin, H, W, Cout, n, dtype (and checks the rest
 * of the layer description as dynconv_forward does). */
dynconv_status_t dynconv_route_attn(const dynconv_desc_t *desc, const void *x,
                                    const float *fc_w, const float *fc_b, int32_t mode,
                                    float temperature, const float *fc_w_in, const float *fc_b_in,
                                    const float *fc_w_out, const float *fc_b_out, float *alpha,
                                    float *a_in, float *a_out, void *workspace,
                                    size_t workspace_bytes, void *stream);
size_t dynconv_route_attn_workspace_bytes(const dynconv_desc_t *desc);

/* dynconv_forward with the channel attentions a_in [B,Cin] and a_out
 * [B,Cout] (float32; either may be NULL, meaning all ones). bf16 layers with
 * groups == 1 (at most 16 experts; more return DYNCONV_ERR_UNSUPPORTED) run
 * on DYNCONV_POLICY_PREMIX (AUTO resolves to it; FUSED returns
 * DYNCONV_ERR_UNSUPPORTED): the input attention scales the premixed
 * kernels' input channels before their bf16 rounding and the output
 * attention scales the accumulators before the bf16 output. Depthwise layers
 * scale each plane's taps by a_in[b,c] * a_out[b,c] before their rounding to
 * the storage type; float32 layers scale the input values and the sums.
 * workspace: at least dynconv_forward_attn_workspace_bytes(desc, policy)
 * bytes. Other arguments, errors and determinism as dynconv_forward. */
dynconv_status_t dynconv_forward_attn(const dynconv_desc_t *desc, int32_t policy, const void *x,
                                      const void *experts, const float *alpha, const float *a_in,
                                      const float *a_out, void *y, void *workspace,
                                      size_t workspace_bytes, void *stream);
size_t dynconv_forward_attn_workspace_bytes(const dynconv_desc_t *desc, int32_t policy);

/* The layer evaluated only where a gate says so (Dynamic Convolutions:
 * Exploiting Spatial Sparsity for Faster Inference, abstract: a small gating
 * branch picks the spatial positions a residual block evaluates; the work is
 * done with a gather-scatter approach). The gate is an input here:
 *   y[b,o,r,s] = (residual ? x[b,o,r,s] : 0) + [mask[b,r,s] != 0] * layer(x)[b,o,r,s]
 * where layer is dynconv_forward's convolution with W_b = sum_i alpha[b,i] E_i.
 * mask: [B,Ho,Wo] uint8 (nonzero = evaluate). residual: 0 or 1; 1 needs
 * Cin == Cout and Ho == H, Wo == W. bf16 layers with groups == 1 (any n;
 * more than 16 experts as dynconv_forward). The convolution runs only at the
 * active positions: their im2col rows are gathered, multiplied on the matrix
 * cores and scattered back; the other positions receive 0 or x. y
 * [B,Cout,Ho,Wo] must not overlap x (DYNCONV_ERR_INVALID_ARG). workspace: at
 * least dynconv_forward_sparse_workspace_bytes(desc) bytes (the mixed
 * kernels and the compacted positions; 0 for an unsupported layer). y is
 * rounded once to bf16 (the residual is added in float32 first);
 * deterministic. */
dynconv_status_t dynconv_forward_sparse(const dynconv_desc_t *desc, const void *x, const void *experts,
                                        const float *alpha, const uint8_t *mask, int32_t residual, void *y,
                                        void *workspace, size_t workspace_bytes, void *stream);
size_t dynconv_forward_sparse_workspace_bytes(const dynconv_desc_t *desc);

/* dynconv_forward_sparse with an expert bank already packed by
 * dynconv_pack_experts (so the static experts are laid out once, not on
 * every call). Same arguments, checks, results and determinism as
 * dynconv_forward_sparse, with packed in place of experts. workspace: at
 * least dynconv_forward_sparse_packed_workspace_bytes(desc) bytes (the mixed
 * kernels and, outside the one-pass band kernel's shapes, the compacted
 * positions; 0 for an unsupported layer). Results are bitwise those of
 * dynconv_forward_sparse. */
dynconv_status_t dynconv_forward_sparse_packed(const dynconv_desc_t *desc, const void *x, const void *packed,
                                               const float *alpha, const uint8_t *mask, int32_t residual,
                                               void *y, void *workspace, size_t workspace_bytes, void *stream);
size_t dynconv_forward_sparse_packed_workspace_bytes(const dynconv_desc_t *desc);

/* ---- gradients ------------------------------------------------------------
 * The pages train dynamic convolutions end to end (CondConv: Conditionally
 * Parameterized Convolutions, abstract, where the per-example kernels are
 * learned; KernelWarehouse: Rethinking the Design of Dynamic Convolution,
 * abstract, where the mixture of static kernels and its attentions are
 * learned) but print no backward pass. These entry points compute the derivative of the forward
 * definition above for a given output gradient dy [B,Cout,Ho,Wo] (same
 * element type as x). Calls are asynchronous on `stream`, validate every
 * argument before any launch (nothing is launched or written on failure)
 * and run in a fixed order (deterministic). */

/* Input gradient of the layer:
 *   dx[b] = the transposed convolution of dy[b] with W_b = sum_i alpha[b,i] E_i,
 * i.e. dx[b,c,h,w] = sum of W_b[o,c',u,v] * dy[b,o,r,s] over the (o, r, s,
 * u, v) whose forward output read x[b,c,h,w]. For stride 1, kh == kw and
 * pad <= kh - 1 it is computed as the forward layer (any policy of
 * dynconv_forward; AUTO picks as for that layer) applied to dy with the bank
 * transposed in its channels, flipped in its taps, and padding k - 1 - pad;
 * workspace: the flipped bank, then the forward's workspace. Any other
 * stride, padding or kernel shape mixes W_b into the workspace (as
 * dynconv_mix: B * Cout * (Cin/g) * kh * kw elements of the layer's type) and
 * gathers each dx element directly; the policy is then only checked. dy:
 * [B,Cout,Ho,Wo]; experts, alpha as dynconv_forward; dx: [B,Cin,H,W],
 * written (not accumulated), in the layer's element type with one rounding.
 * Groups 1 or depthwise (else DYNCONV_ERR_UNSUPPORTED). workspace: at least
 * dynconv_backward_data_workspace_bytes(desc, policy) bytes; 0 if the
 * descriptor is invalid. */
dynconv_status_t dynconv_backward_data(const dynconv_desc_t *desc, int32_t policy, const void *dy,
                                       const void *experts, const float *alpha, void *dx,
                                       void *workspace, size_t workspace_bytes, void *stream);
size_t dynconv_backward_data_workspace_bytes(const dynconv_desc_t *desc, int32_t policy);

/* Gradients of the attentions and of the expert bank:
 *   dW_b[o,c',u,v] = sum_{r,s} dy[b,o,r,s] * x[b, gc, r*stride-pad+u, s*stride-pad+v]
 *   dalpha[b,i]    = sum_e dW_b[e] * E_i[e]          (float32 [B,n])
 *   dexperts[i,e]  = sum_b alpha[b,i] * dW_b[e]      (float32 [n,Cout,Cin/g,kh,kw])
 * x outside the image counts as 0. dW_b is formed in float32 from the stored
 * x and dy (bf16 products are exact in float32) and kept in the workspace,
 * followed by partial sums of dalpha and, for larger batches, of dexperts
 * per group of examples: at least dynconv_backward_weights_workspace_bytes(desc)
 * bytes (B * Cout * (Cin/g) * kh * kw floats and the partial sums, each
 * piece rounded up to 256 bytes). dalpha or dexperts may be NULL (not
 * computed), not both. Any stride and padding; groups 1 or depthwise (at
 * most 64 taps); B <= 65535. Both outputs are written, not accumulated. */
dynconv_status_t dynconv_backward_weights(const dynconv_desc_t *desc, const void *x, const void *dy,
                                          const void *experts, const float *alpha, float *dalpha,
                                          float *dexperts, void *workspace, size_t workspace_bytes,
                                          void *stream);
size_t dynconv_backward_weights_workspace_bytes(const dynconv_desc_t *desc);

/* Gradients of the layer with FMDConv's channel attentions (FMDConv: Fast
 * multi-attention dynamic convolution, abstract; the forward is
 * dynconv_forward_attn: y = a_out * conv(a_in * x, W_b), a_in [B,Cin] scaling
 * input channels, a_out [B,Cout] output channels, float32, either NULL
 * meaning all ones). With G_b = the dW_b of dynconv_backward_weights formed
 * from x and dy alone:
 *   dW'_b[o,c',u,v] = a_out[b,o] * a_in[b,gc] * G_b[o,c',u,v]
 *   dalpha[b,i]     = sum_e dW'_b[e] * E_i[e]        (float32 [B,n])
 *   dexperts[i,e]   = sum_b alpha[b,i] * dW'_b[e]    (float32 [n,Cout,Cin/g,kh,kw])
 *   da_in[b,gc]     = sum over the o of gc's group and (u,v) of a_out[b,o] * G_b[o,c',u,v] * W_b[o,c',u,v]
 *   da_out[b,o]     = sum over (c',u,v) of a_in[b,gc] * G_b[o,c',u,v] * W_b[o,c',u,v]
 * (float32 [B,Cin] and [B,Cout]; gc = (o / (Cout/g)) * (Cin/g) + c'). W_b is
 * mixed in float32 for these sums, the attention factors multiply G_b in
 * float32: no rounding to the element type enters. Any output may be NULL
 * (not computed), not all four. Any stride and padding; groups 1 or depthwise
 * (at most 64 taps); B <= 65535. workspace: at least
 * dynconv_backward_weights_attn_workspace_bytes(desc) bytes (G_b in float32,
 * the partial sums, and B * Cout * (Cin/g) floats); outputs written, not
 * accumulated; deterministic. Other arguments and errors as
 * dynconv_backward_weights. */
dynconv_status_t dynconv_backward_weights_attn(const dynconv_desc_t *desc, const void *x, const void *dy,
                                               const void *experts, const float *alpha, const float *a_in,
                                               const float *a_out, float *dalpha, float *dexperts, float *da_in,
                                               float *da_out, void *workspace, size_t workspace_bytes,
                                               void *stream);
size_t dynconv_backward_weights_attn_workspace_bytes(const dynconv_desc_t *desc);

/* Input gradient of the layer with FMDConv's channel attentions:
 *   dx[b,gc,h,w] = a_in[b,gc] * (the transposed convolution of a_out[b,:] * dy[b] with W_b)
 * computed as dynconv_forward_attn of the transposed layer (stride 1, kh ==
 * kw and pad <= kh - 1 only; else DYNCONV_ERR_UNSUPPORTED): the bank
 * transposed and flipped as in dynconv_backward_data, a_out as that layer's
 * input attention and a_in as its output attention, with the policies and
 * roundings of dynconv_forward_attn (bf16 groups == 1 layers: at most 16
 * experts). workspace: at least dynconv_backward_data_attn_workspace_bytes(
 * desc, policy) bytes (the flipped bank, then the forward's workspace; 0 for
 * an unsupported layer or policy). Other arguments as
 * dynconv_backward_data. */
dynconv_status_t dynconv_backward_data_attn(const dynconv_desc_t *desc, int32_t policy, const void *dy,
                                            const void *experts, const float *alpha, const float *a_in,
                                            const float *a_out, void *dx, void *workspace, size_t workspace_bytes,
                                            void *stream);
size_t dynconv_backward_data_attn_workspace_bytes(const dynconv_desc_t *desc, int32_t policy);

/* Gradient of the routing (dynconv_route) for the attention gradient dalpha:
 *   sigmoid:      dz = dalpha * alpha * (1 - alpha)
 *   softmax(z/T): dz_i = alpha_i * (dalpha_i - sum_k alpha_k dalpha_k) / T
 *   dfc_w[i,c] = sum_b dz[b,i] * gap[b,c],  dfc_b[i] = sum_b dz[b,i]
 *   dgap[b,c]  = sum_i dz[b,i] * fc_w[i,c]
 * alpha [B,n] must be dynconv_route's output for the same x, fc_w, fc_b,
 * mode and temperature; gap is recomputed from x. dfc_w [n,Cin] and dfc_b
 * [n] (may be NULL) are written (float32). When dx [B,Cin,H,W] (layer
 * element type) is not NULL, dgap[b,c] / (H*W) is ADDED to every position of
 * dx[b,c] in float32 and rounded once to the element type: pass the input
 * gradient from dynconv_backward_data to get the whole input gradient.
 * Only B, Cin, H, W, n and dtype of desc are read; n <= 256. workspace: at
 * least dynconv_route_backward_workspace_bytes(desc) bytes. */
dynconv_status_t dynconv_route_backward(const dynconv_desc_t *desc, const void *x, const float *fc_w,
                                        int32_t mode, float temperature, const float *alpha,
                                        const float *dalpha, float *dfc_w, float *dfc_b, void *dx,
                                        void *workspace, size_t workspace_bytes, void *stream);
size_t dynconv_route_backward_workspace_bytes(const dynconv_desc_t *desc);

/* The policy DYNCONV_POLICY_AUTO resolves to for this layer
 * (DYNCONV_POLICY_PREMIX or DYNCONV_POLICY_FUSED), or -1 for an invalid or
 * unsupported descriptor. */
int32_t dynconv_forward_policy(const dynconv_desc_t *desc);

/* Static text for a status code (never NULL). */
const char *dynconv_status_string(dynconv_status_t status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char *dynconv_last_error(void);

/* ABI version: bumped whenever a signature or layout above changes. */
int32_t dynconv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DYNCONV_H */
