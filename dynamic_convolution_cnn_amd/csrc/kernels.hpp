// Launchers of the gfx950 kernels, called by the host-side C ABI (api.cpp).
// Every launcher only enqueues work on `stream`; argument checking is done
// by the caller before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dynconv {

// Layer geometry after validation (sizes in elements).
struct Geom {
    int B, Cin, H, W, Cout, KH, KW, stride, pad, groups, n;
    int Ho, Wo;
    int P;        // Ho * Wo, output positions per channel plane
    int KT;       // KH * KW taps
    int cpg;      // Cin / groups, input channels per group
    int Cin_pad;  // Cin rounded up to a multiple of 32 (MFMA K chunk)
    int n_pad;    // n rounded up to an even count (expert pairs)
    bool bf16;    // element type of x, experts, mixed kernels and y
};

// FMDConv's channel attentions (FMDConv: Fast multi-attention dynamic
// convolution, abstract): in[b * Cin + c] scales input channel c of example
// b before the convolution, out[b * Cout + o] scales output channel o after
// it (float32). Either may be null: all ones.
struct ChanAttn {
    const float *in = nullptr;
    const float *out = nullptr;
};

// ---- routing -------------------------------------------------------------
// alpha[B,n] from the channel means of x, the FC and the nonlinearity.
// `workspace` holds route_workspace_bytes(g) bytes: none for one workgroup
// per example; tickets (zero on entry, left zero) and B*Cin channel means for
// the split router; B*Cin means for the two-kernel path.
bool route_single_kernel(const Geom &g);
size_t route_workspace_bytes(const Geom &g);
hipError_t launch_route(const Geom &g, const void *x, const float *fc_w,
                        const float *fc_b, int mode, float temperature,
                        void *workspace, float *alpha, hipStream_t stream);
// Channel means of x into gap[B*Cin] (float).
hipError_t launch_gap(const Geom &g, const void *x, float *gap, hipStream_t stream);
// GAP into `gap` (B*Cin floats), then nout[h] logits per example for each of
// `heads` FC heads (fc_w[h]: [nout[h]][Cin], fc_b[h] or null), each through
// its own nonlinearity mode[h] into out[h] [B][nout[h]]. nout[h] <= 256.
hipError_t launch_route_heads(const Geom &g, const void *x, int heads, const float *const *fc_w,
                              const float *const *fc_b, const int *nout, const int *mode,
                              float temperature, float *gap, float *const *out, hipStream_t stream);

// ---- mixing --------------------------------------------------------------
// mixed[b, e] = sum_i alpha[b, i] * experts[i, e], natural layout, wsize
// elements per expert; element type per g.bf16.
hipError_t launch_mix_natural(const Geom &g, long wsize, const float *alpha,
                              const void *experts, void *mixed, hipStream_t stream);

// Expert bank to the kernel-ready layout packed[t][o][cp][ip] (bf16):
// t = tap, o = output channel, cp < Cin_pad (zero for cp >= Cin),
// ip < n_pad (zero for ip >= n). Expert pairs sit in one 32-bit word.
size_t packed_experts_bytes(const Geom &g);
hipError_t launch_pack_experts(const Geom &g, const uint16_t *experts,
                               uint16_t *packed, hipStream_t stream);

// Many experts (bf16): mixed[b][w] = sum_i alpha[b,i] bank[i][w] for a bank
// of n rows of wsize weights (wsize a multiple of 8), on the matrix cores
// with the experts as the reduction dimension; any n.
bool mix_wide_supported(long wsize);
// conv_feed: the mix writes W_b for the premix convolution that runs next.
hipError_t launch_mix_wide(const Geom &g, long wsize, const float *alpha, const uint16_t *experts, uint16_t *mixed,
                           hipStream_t stream, bool conv_feed = false);
// The natural bank in the convolution's weight order, wide[i][t][o][cp]
// (bf16, zeros for cp >= Cin): the forward's bank for n > 16.
size_t wide_bank_bytes(const Geom &g);
bool pack_wide_supported(const Geom &g);  // one expert's Cin x KT block fits 64 KB of LDS
hipError_t launch_pack_wide(const Geom &g, const uint16_t *experts, uint16_t *wide, hipStream_t stream);

// Mixed kernels in the convolution's layout wt[b][t][o][cp] (bf16) from
// the packed bank.
size_t premixed_bytes(const Geom &g);
// att.in scales the mixed kernels' input channels (att.out is not used).
hipError_t launch_premix(const Geom &g, const float *alpha, const uint16_t *packed,
                         uint16_t *wt, hipStream_t stream, ChanAttn att = {});

// ---- convolution -----------------------------------------------------------
// Implicit-GEMM bf16 MFMA convolution with mixed kernels read from `wt`.
bool premix_conv_supported(const Geom &g);
// att.out scales the output channels (att.in is not used: it is folded into wt).
hipError_t launch_conv_premix(const Geom &g, const uint16_t *x, const uint16_t *wt,
                              uint16_t *y, hipStream_t stream, ChanAttn att = {});

// 3x3 stride-1 pad-1 premix convolution with 4x2 / 2x4 wave tiles
// (conv_pm3w.hip); launch_conv_premix dispatches to it.
bool pm3w_ok(const Geom &g);
hipError_t launch_conv_pm3w(const Geom &g, const uint16_t *x, const uint16_t *wt, uint16_t *y,
                            hipStream_t stream, const float *a_out);

// Implicit-GEMM bf16 MFMA convolution that mixes each kernel tile from the
// packed bank in registers (no mixed kernel in memory).
bool fused_conv_supported(const Geom &g);
hipError_t launch_conv_fused(const Geom &g, const uint16_t *x, const uint16_t *packed,
                             const float *alpha, uint16_t *y, hipStream_t stream, ChanAttn att = {});
// The 3x3 pad-1 case up to 14 x 14 outputs with one wave per example
// (conv_fused_wave.hip); launch_conv_fused dispatches to it.
bool fused_wave_ok(const Geom &g);
// ... and with channel attentions (the input attentions of 4 examples in LDS)
bool fused_wave_attn_ok(const Geom &g);
hipError_t launch_conv_fused_wave(const Geom &g, const uint16_t *x, const uint16_t *packed,
                                  const float *alpha, uint16_t *y, hipStream_t stream, ChanAttn att = {});

// Direct float32 convolution (groups == 1) with mixed kernels in natural
// layout [B][Cout][Cin][KH][KW].
hipError_t launch_conv_direct_f32(const Geom &g, const float *x, const float *wmixed,
                                  float *y, hipStream_t stream, ChanAttn att = {});

// Depthwise convolution (groups == Cin == Cout). With `wmixed` == nullptr
// each plane's taps are mixed in the kernel from experts and alpha;
// otherwise they are read from wmixed [B][C][KH][KW].
bool depthwise_supported(const Geom &g);
// With attentions, each plane's taps are scaled by in[b,c] * out[b,c].
hipError_t launch_conv_depthwise(const Geom &g, const void *x, const void *experts,
                                 const float *alpha, const void *wmixed, void *y,
                                 hipStream_t stream, ChanAttn att = {});
// The matrix-core form of it (bf16, stride 1, square 3/5/7 taps, output
// planes of at most 32 x 32); launch_conv_depthwise picks it where it applies.
bool depthwise_mfma_ok(const Geom &g, bool premixed);
hipError_t launch_depthwise_mfma(const Geom &g, const uint16_t *x, const uint16_t *experts, const float *alpha,
                                 const uint16_t *wmixed, uint16_t *y, hipStream_t stream, ChanAttn att);

// ---- gated (spatially sparse) evaluation ----------------------------------
// y = (residual ? x : 0) + [mask != 0] * conv(x, W_b) with W_b premixed in
// wt[b][t][o][cp] (bf16, groups == 1); mask [B][Ho*Wo] uint8 over the output
// positions; idx: sparse_index_bytes(g) of scratch (the compacted positions
// and their counts, then a channel-innermost copy of x). y must not overlap x.
size_t sparse_index_bytes(const Geom &g);
// True where the one-pass band kernel takes the layer (3x3, stride 1, pad 1,
// Cin and Cout up to 64, W a multiple of 8); it needs no index scratch.
bool gated_one_pass(const Geom &g);
hipError_t launch_conv_sparse(const Geom &g, const uint16_t *x, const uint16_t *wt, const uint8_t *mask, int residual,
                              int *idx, uint16_t *y, hipStream_t stream);

// ---- gradients ---------------------------------------------------------------
// Bank transposed in its channels and flipped in its taps: for groups == 1
// flipped[i][c][o][u][v] = experts[i][o][c][KH-1-u][KW-1-v]; depthwise
// flipped[i][c][0][u][v] = experts[i][c][0][KH-1-u][KW-1-v]. Element type
// per g.bf16. The forward layer with this bank and padding k - 1 - p,
// applied to dy, is the input gradient of a stride-1 layer.
hipError_t launch_flip_experts(const Geom &g, const void *experts, void *flipped, hipStream_t stream);
// Input gradient dx [B][Cin][H][W] from dy [B][Cout][Ho][Wo] and the mixed
// kernels W_b [B][Cout][Cin/g][KH][KW] (element type per g.bf16), any stride,
// padding and kernel shape; groups 1 or depthwise.
hipError_t launch_dgrad_direct(const Geom &g, const void *dy, const void *wb, void *dx, hipStream_t stream);

// Per-example kernel gradients dW_b (float32, [B][Cout][Cin/g][KH][KW]) of
// x and dy (element type per g.bf16), then dalpha[B][n] = <dW_b, E_i> and
// dexperts[n][...] = sum_b alpha[b][i] dW_b (either output may be null).
size_t wgrad_bytes(const Geom &g);
bool wgrad_dw_supported(const Geom &g);
hipError_t launch_backward_weights(const Geom &g, const void *x, const void *dy, const void *experts,
                                   const float *alpha, float *dwb, float *dalpha, float *dexperts,
                                   hipStream_t stream);

// The kernel gradient of the layer with FMDConv's channel attentions (att.in
// [B*Cin], att.out [B*Cout], either null = ones): dalpha and dexperts of
// y = a_out * conv(a_in * x, W_b) through dW_b in the workspace, and
// da_in [B*Cin], da_out [B*Cout] (float32). Any output may be null.
size_t wgrad_attn_bytes(const Geom &g);
hipError_t launch_backward_weights_attn(const Geom &g, const void *x, const void *dy, const void *experts,
                                        const float *alpha, ChanAttn att, float *ws, float *dalpha,
                                        float *dexperts, float *da_in, float *da_out, hipStream_t stream);

// The fused kernel gradient (wgrad_fused.hip: bf16, groups == 1, stride 1,
// n <= 4, 1 x 1 or k x 3 kernels; dW_b never stored): its scratch bytes,
// 0 where it does not apply, and its launch with that scratch.
size_t wgrad_fused_bytes(const Geom &g);
hipError_t launch_wgrad_fused(const Geom &g, const void *x, const void *dy, const void *experts, const float *alpha,
                              float *scratch, float *dalpha, float *dexperts, hipStream_t stream);
// de[j] = sum over groups of dep[g * total + j]; dalpha[b * n + i] = sum over
// chunks ch < nch of dpart[(b * rows + i) * nch + ch] (in chunk order).
hipError_t launch_dE_reduce(const float *dep, float *de, long total, int groups, hipStream_t stream);
hipError_t launch_dalpha_reduce(const float *dpart, float *dalpha, int B, int n, int rows, int nch,
                                hipStream_t stream);

// Routing gradient: gap (B*Cin), dz (B*n) and dgap (B*Cin) are scratch;
// dfc_w[n][Cin], dfc_b[n] (may be null) are written; when dx is not null,
// dgap[b][c] / (H W) is added to every position of dx[b][c] (one rounding
// to the element type). mode 0 = sigmoid, 1 = softmax(z / temperature).
hipError_t launch_route_backward(const Geom &g, const void *x, const float *fc_w, int mode, float temperature,
                                 const float *alpha, const float *dalpha, float *gap, float *dz, float *dgap,
                                 float *dfc_w, float *dfc_b, void *dx, hipStream_t stream);

}  // namespace dynconv
