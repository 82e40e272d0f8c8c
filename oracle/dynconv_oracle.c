/*
 * CPU oracle for CondConv-style dynamic convolution.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it. It shares no code, header, table or helper
 * with the HIP library and includes nothing from it.
 *
 * What it computes, and where the pages define it:
 *   - per-example kernels: every example gets a kernel of its own (CondConv:
 *     Conditionally Parameterized Convolutions, abstract);
 *   - each example's kernel is a linear mixture of n static kernels weighted
 *     by input-dependent attentions (KernelWarehouse: Rethinking the Design
 *     of Dynamic Convolution, abstract);
 *   - the attentions are computed by global average pooling of the layer
 *     input, a fully connected layer with bias, then a sigmoid, or a softmax
 *     of the logits divided by a temperature (temperature-scaled kernel
 *     attention: FMDConv: Fast multi-attention dynamic convolution, abstract).
 *     The pages name no further detail of the routing function; the
 *     plainest reading is taken.
 *
 * Arithmetic: every input is read as the exact value stored (bf16 inputs
 * arrive already widened to float, which is exact); every sum and product is
 * carried in double precision; no intermediate is rounded.
 *
 * Convolution reading: cross-correlation (no kernel flip), zero padding,
 * dilation 1, no bias, output size floor((H + 2p - k) / s) + 1.
 *
 * Parity is pinned by the not-gpu tests (torch conv2d in float64 for the
 * single-expert case, one-hot selection, brute-force linearity, routing
 * closed forms and a hand-worked example); the gradients by torch autograd
 * in float64, unit-impulse brute force and Euler's identity for the
 * bilinear layer; see the test suite.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

static int out_size(int in, int k, int stride, int pad)
{
    return (in + 2 * pad - k) / stride + 1;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Global average pool of one example's channel plane: the mean over all
 * H*W positions (the routing input: the attentions depend on the example,
 * KernelWarehouse abstract).
 * gap[b*C + c] = (1/(H*W)) * sum_{h,w} x[b,c,h,w]
 */
int oracle_gap(int B, int C, int H, int W, const float *x, double *gap)
{
    if (B < 0 || C < 1 || H < 1 || W < 1 || !x || !gap) return ORACLE_BAD_ARG;
    long hw = (long)H * W;
#pragma omp parallel for schedule(static)
    for (long bc = 0; bc < (long)B * C; ++bc) {
        const float *p = x + bc * hw;
        double s = 0.0;
        for (long i = 0; i < hw; ++i) s += (double)p[i];
        gap[bc] = s / (double)hw;
    }
    return ORACLE_OK;
}

/*
 * Routing (attention) for every example:
 *   z[b,i]  = sum_c fc_w[i,c] * gap[b,c] + fc_b[i]
 *   mode 0: alpha[b,i] = 1 / (1 + exp(-z[b,i]))            (sigmoid)
 *   mode 1: alpha[b,i] = exp(z_i/T - m) / sum_j exp(z_j/T - m),
 *           m = max_j z_j/T                                  (softmax, temperature T)
 * fc_b may be NULL (no bias). The sigmoid uses the split form so that
 * exp never overflows.
 */
int oracle_route(int B, int C, int H, int W, int n, const float *x,
                 const float *fc_w, const float *fc_b, int mode, double T,
                 double *gap_out, double *z_out, double *alpha)
{
    if (B < 0 || C < 1 || H < 1 || W < 1 || n < 1 || !x || !fc_w || !alpha)
        return ORACLE_BAD_ARG;
    if (mode != 0 && mode != 1) return ORACLE_BAD_ARG;
    if (mode == 1 && !(T > 0.0)) return ORACLE_BAD_ARG;
    double *gap = (double *)malloc(sizeof(double) * ((size_t)B * C + 1));
    double *z = (double *)malloc(sizeof(double) * ((size_t)B * n + 1));
    if (!gap || !z) { free(gap); free(z); return ORACLE_BAD_ARG; }
    oracle_gap(B, C, H, W, x, gap);
#pragma omp parallel for schedule(static)
    for (int b = 0; b < B; ++b) {
        double *zb = z + (long)b * n;
        for (int i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int c = 0; c < C; ++c)
                acc += (double)fc_w[(long)i * C + c] * gap[(long)b * C + c];
            if (fc_b) acc += (double)fc_b[i];
            zb[i] = acc;
        }
        double *ab = alpha + (long)b * n;
        if (mode == 0) {
            for (int i = 0; i < n; ++i) {
                if (zb[i] >= 0.0) {
                    ab[i] = 1.0 / (1.0 + exp(-zb[i]));
                } else {
                    double e = exp(zb[i]);
                    ab[i] = e / (1.0 + e);
                }
            }
        } else {
            double m = -INFINITY;
            for (int i = 0; i < n; ++i)
                if (zb[i] / T > m) m = zb[i] / T;
            double s = 0.0;
            for (int i = 0; i < n; ++i) s += exp(zb[i] / T - m);
            for (int i = 0; i < n; ++i) ab[i] = exp(zb[i] / T - m) / s;
        }
    }
    if (gap_out)
        for (long i = 0; i < (long)B * C; ++i) gap_out[i] = gap[i];
    if (z_out)
        for (long i = 0; i < (long)B * n; ++i) z_out[i] = z[i];
    free(gap);
    free(z);
    return ORACLE_OK;
}

/*
 * Mixing: W_b = sum_i alpha[b,i] * E_i  (KernelWarehouse abstract: a linear
 * mixture of n static kernels weighted by the attentions).
 * experts: [n, wsize], alpha: [B, n], mixed: [B, wsize].
 */
int oracle_mix(int B, int n, long wsize, const double *alpha,
               const float *experts, double *mixed)
{
    if (B < 0 || n < 1 || wsize < 1 || !alpha || !experts || !mixed)
        return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < B; ++b) {
        for (long e = 0; e < wsize; ++e) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i)
                acc += alpha[(long)b * n + i] * (double)experts[(long)i * wsize + e];
            mixed[(long)b * wsize + e] = acc;
        }
    }
    return ORACLE_OK;
}

/*
 * Per-example convolution with the example's own kernel (CondConv abstract).
 *   y[b,o,r,s] = sum_{c'<Cin/g} sum_{u<kh} sum_{v<kw}
 *                wb[b,o,c',u,v] * x[b, grp(o)*(Cin/g) + c', r*st - p + u, s*st - p + v]
 * with grp(o) = o / (Cout/g) and x read as 0 outside the image.
 * x: [B,Cin,H,W] float; wb: [B,Cout,Cin/g,kh,kw] double; y: [B,Cout,Ho,Wo] double.
 */
int oracle_conv(int B, int Cin, int H, int W, int Cout, int kh, int kw,
                int stride, int pad, int groups, const float *x,
                const double *wb, double *y)
{
    if (B < 0 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || kh < 1 || kw < 1 ||
        stride < 1 || pad < 0 || groups < 1 || !x || !wb || !y)
        return ORACLE_BAD_ARG;
    if (Cin % groups || Cout % groups) return ORACLE_BAD_ARG;
    int Ho = out_size(H, kh, stride, pad), Wo = out_size(W, kw, stride, pad);
    if (Ho < 1 || Wo < 1) return ORACLE_BAD_ARG;
    int cpg = Cin / groups, opg = Cout / groups;
    long wsz = (long)Cout * cpg * kh * kw;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int o = 0; o < Cout; ++o) {
            int g = o / opg;
            const double *wo = wb + (long)b * wsz + (long)o * cpg * kh * kw;
            for (int r = 0; r < Ho; ++r) {
                for (int s = 0; s < Wo; ++s) {
                    double acc = 0.0;
                    for (int c = 0; c < cpg; ++c) {
                        const float *xp = x + (((long)b * Cin + (long)g * cpg + c) * H) * W;
                        for (int u = 0; u < kh; ++u) {
                            int h = r * stride - pad + u;
                            if (h < 0 || h >= H) continue;
                            for (int v = 0; v < kw; ++v) {
                                int w = s * stride - pad + v;
                                if (w < 0 || w >= W) continue;
                                acc += wo[((long)c * kh + u) * kw + v] * (double)xp[(long)h * W + w];
                            }
                        }
                    }
                    y[(((long)b * Cout + o) * Ho + r) * Wo + s] = acc;
                }
            }
        }
    }
    return ORACLE_OK;
}

/*
 * The whole layer for given attentions: mix the example's kernel, then
 * convolve (CondConv abstract: mix first, one convolution per example).
 * The mixed kernel of one example is built into a per-thread buffer so that
 * the layer never holds all B mixed kernels at once.
 */
int oracle_forward(int B, int Cin, int H, int W, int Cout, int kh, int kw,
                   int stride, int pad, int groups, int n, const float *x,
                   const float *experts, const double *alpha, double *y)
{
    if (B < 0 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || kh < 1 || kw < 1 ||
        stride < 1 || pad < 0 || groups < 1 || n < 1 || !x || !experts ||
        !alpha || !y)
        return ORACLE_BAD_ARG;
    if (Cin % groups || Cout % groups) return ORACLE_BAD_ARG;
    int Ho = out_size(H, kh, stride, pad), Wo = out_size(W, kw, stride, pad);
    if (Ho < 1 || Wo < 1) return ORACLE_BAD_ARG;
    int cpg = Cin / groups, opg = Cout / groups;
    long per_o = (long)cpg * kh * kw;
    long wsz = (long)Cout * per_o;
    int failed = 0;
#pragma omp parallel
    {
    double *wo = (double *)malloc(sizeof(double) * (size_t)per_o);
    if (!wo) {
#pragma omp atomic write
        failed = 1;
    }
#pragma omp for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int o = 0; o < Cout; ++o) {
            if (!wo) continue;
            int g = o / opg;
            for (long e = 0; e < per_o; ++e) {
                double acc = 0.0;
                for (int i = 0; i < n; ++i)
                    acc += alpha[(long)b * n + i] *
                           (double)experts[(long)i * wsz + (long)o * per_o + e];
                wo[e] = acc;
            }
            for (int r = 0; r < Ho; ++r) {
                for (int s = 0; s < Wo; ++s) {
                    double acc = 0.0;
                    for (int c = 0; c < cpg; ++c) {
                        const float *xp = x + (((long)b * Cin + (long)g * cpg + c) * H) * W;
                        for (int u = 0; u < kh; ++u) {
                            int h = r * stride - pad + u;
                            if (h < 0 || h >= H) continue;
                            for (int v = 0; v < kw; ++v) {
                                int w = s * stride - pad + v;
                                if (w < 0 || w >= W) continue;
                                acc += wo[((long)c * kh + u) * kw + v] * (double)xp[(long)h * W + w];
                            }
                        }
                    }
                    y[(((long)b * Cout + o) * Ho + r) * Wo + s] = acc;
                }
            }
        }
    }
    free(wo);
    }
    return failed ? ORACLE_BAD_ARG : ORACLE_OK;
}

/*
 * Selected outputs of the layer, one by one, for checks at full size:
 * idx holds m quadruples (b, o, r, s); out[j] = y[b,o,r,s] as oracle_forward
 * defines it. Each output mixes only the kernel row it needs.
 */
int oracle_forward_points(int B, int Cin, int H, int W, int Cout, int kh,
                          int kw, int stride, int pad, int groups, int n,
                          const float *x, const float *experts,
                          const double *alpha, long m, const int32_t *idx,
                          double *out)
{
    if (B < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || kh < 1 || kw < 1 ||
        stride < 1 || pad < 0 || groups < 1 || n < 1 || m < 0 || !x ||
        !experts || !alpha || !idx || !out)
        return ORACLE_BAD_ARG;
    if (Cin % groups || Cout % groups) return ORACLE_BAD_ARG;
    int Ho = out_size(H, kh, stride, pad), Wo = out_size(W, kw, stride, pad);
    if (Ho < 1 || Wo < 1) return ORACLE_BAD_ARG;
    for (long j = 0; j < m; ++j) {
        int b = idx[4 * j], o = idx[4 * j + 1], r = idx[4 * j + 2], s = idx[4 * j + 3];
        if (b < 0 || b >= B || o < 0 || o >= Cout || r < 0 || r >= Ho || s < 0 || s >= Wo)
            return ORACLE_BAD_ARG;
    }
    int cpg = Cin / groups, opg = Cout / groups;
    long per_o = (long)cpg * kh * kw;
    long wsz = (long)Cout * per_o;
#pragma omp parallel for schedule(dynamic, 16)
    for (long j = 0; j < m; ++j) {
        int b = idx[4 * j], o = idx[4 * j + 1], r = idx[4 * j + 2], s = idx[4 * j + 3];
        int g = o / opg;
        double acc = 0.0;
        for (int c = 0; c < cpg; ++c) {
            const float *xp = x + (((long)b * Cin + (long)g * cpg + c) * H) * W;
            for (int u = 0; u < kh; ++u) {
                int h = r * stride - pad + u;
                if (h < 0 || h >= H) continue;
                for (int v = 0; v < kw; ++v) {
                    int w = s * stride - pad + v;
                    if (w < 0 || w >= W) continue;
                    long e = (long)o * per_o + ((long)c * kh + u) * kw + v;
                    double wv = 0.0;
                    for (int i = 0; i < n; ++i)
                        wv += alpha[(long)b * n + i] * (double)experts[(long)i * wsz + e];
                    acc += wv * (double)xp[(long)h * W + w];
                }
            }
        }
        out[j] = acc;
    }
    return ORACLE_OK;
}

/*
 * The layer with FMDConv's input and output attentions (FMDConv: Fast
 * multi-attention dynamic convolution, abstract: input attention, kernel
 * attention and output attention). The page gives no formula; the reading
 * taken: the input attention scales each input channel of the example before
 * the convolution, the output attention scales each output channel after it,
 * and the kernel attention is alpha as above:
 *   y[b,o,r,s] = a_out[b,o] * sum_{c,u,v} W_b[o,c,u,v] * a_in[b,gc] * x[b,gc,h,w],
 *   gc = (o / (Cout/groups)) * (Cin/groups) + c, h = r*stride - pad + u,
 *   w = s*stride - pad + v (zero outside the image).
 * a_in [B, Cin] and a_out [B, Cout] may be NULL (all ones).
 */
int oracle_forward_attn(int B, int Cin, int H, int W, int Cout, int kh, int kw,
                        int stride, int pad, int groups, int n, const float *x,
                        const float *experts, const double *alpha,
                        const double *a_in, const double *a_out, double *y)
{
    if (B < 0 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || kh < 1 || kw < 1 ||
        stride < 1 || pad < 0 || groups < 1 || n < 1 || !x || !experts ||
        !alpha || !y)
        return ORACLE_BAD_ARG;
    if (Cin % groups || Cout % groups) return ORACLE_BAD_ARG;
    int Ho = out_size(H, kh, stride, pad), Wo = out_size(W, kw, stride, pad);
    if (Ho < 1 || Wo < 1) return ORACLE_BAD_ARG;
    int cpg = Cin / groups, opg = Cout / groups;
    long per_o = (long)cpg * kh * kw;
    long wsz = (long)Cout * per_o;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int o = 0; o < Cout; ++o) {
            int g = o / opg;
            double so = a_out ? a_out[(long)b * Cout + o] : 1.0;
            for (int r = 0; r < Ho; ++r) {
                for (int s = 0; s < Wo; ++s) {
                    double acc = 0.0;
                    for (int c = 0; c < cpg; ++c) {
                        int gc = g * cpg + c;
                        double si = a_in ? a_in[(long)b * Cin + gc] : 1.0;
                        const float *xp = x + (((long)b * Cin + gc) * H) * W;
                        for (int u = 0; u < kh; ++u) {
                            int h = r * stride - pad + u;
                            if (h < 0 || h >= H) continue;
                            for (int v = 0; v < kw; ++v) {
                                int w = s * stride - pad + v;
                                if (w < 0 || w >= W) continue;
                                long e = (long)o * per_o + ((long)c * kh + u) * kw + v;
                                double wv = 0.0;
                                for (int i = 0; i < n; ++i)
                                    wv += alpha[(long)b * n + i] * (double)experts[(long)i * wsz + e];
                                acc += wv * (si * (double)xp[(long)h * W + w]);
                            }
                        }
                    }
                    y[(((long)b * Cout + o) * Ho + r) * Wo + s] = so * acc;
                }
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Gradients of the layer (mix, then per-example convolution) for a given
 * output gradient dy. The pages train these layers (CondConv abstract: the
 * per-example kernels are learned; KernelWarehouse abstract: the mixture and
 * its attentions are learned) but print no backward pass; what
 * follows is the derivative of the forward definition above, term by term.
 * With W_b = sum_i alpha[b,i] E_i and y = conv(x_b, W_b):
 *   dW_b[o,c,u,v] = sum_{r,s} dy[b,o,r,s] * x[b, gc, r*st - p + u, s*st - p + v]
 *   dalpha[b,i]   = sum_e dW_b[e] * E_i[e]
 *   dE_i[e]       = sum_b alpha[b,i] * dW_b[e]
 *   dx[b,gc,h,w]  = sum over (o, r, s, u, v) with h = r*st - p + u and
 *                   w = s*st - p + v of W_b[o,c,u,v] * dy[b,o,r,s]
 * (gc = (o / (Cout/groups)) * (Cin/groups) + c; positions outside the image
 * take no part). dx, dalpha and dexperts may each be NULL (not computed).
 * dy: [B,Cout,Ho,Wo]; dx: [B,Cin,H,W]; dalpha: [B,n]; dexperts: [n, wsize].
 */
int oracle_backward(int B, int Cin, int H, int W, int Cout, int kh, int kw,
                    int stride, int pad, int groups, int n, const float *x,
                    const float *experts, const double *alpha, const float *dy,
                    double *dx, double *dalpha, double *dexperts)
{
    if (B < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || kh < 1 || kw < 1 ||
        stride < 1 || pad < 0 || groups < 1 || n < 1 || !x || !experts ||
        !alpha || !dy)
        return ORACLE_BAD_ARG;
    if (Cin % groups || Cout % groups) return ORACLE_BAD_ARG;
    int Ho = out_size(H, kh, stride, pad), Wo = out_size(W, kw, stride, pad);
    if (Ho < 1 || Wo < 1) return ORACLE_BAD_ARG;
    int cpg = Cin / groups, opg = Cout / groups;
    long per_o = (long)cpg * kh * kw;
    long wsz = (long)Cout * per_o;
    /* dW_b for every example, then the two contractions over it */
    double *dwb = (double *)calloc((size_t)B * wsz, sizeof(double));
    double *wb = (double *)malloc(sizeof(double) * (size_t)B * wsz);
    if (!dwb || !wb) { free(dwb); free(wb); return ORACLE_BAD_ARG; }
#pragma omp parallel for schedule(static)
    for (int b = 0; b < B; ++b) {
        double *w = wb + (long)b * wsz;
        for (long e = 0; e < wsz; ++e) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i)
                acc += alpha[(long)b * n + i] * (double)experts[(long)i * wsz + e];
            w[e] = acc;
        }
        double *dw = dwb + (long)b * wsz;
        double *dxb = dx ? dx + (long)b * Cin * H * W : NULL;
        if (dxb)
            for (long j = 0; j < (long)Cin * H * W; ++j) dxb[j] = 0.0;
        for (int o = 0; o < Cout; ++o) {
            int g = o / opg;
            for (int r = 0; r < Ho; ++r) {
                for (int s = 0; s < Wo; ++s) {
                    double d = (double)dy[(((long)b * Cout + o) * Ho + r) * Wo + s];
                    for (int c = 0; c < cpg; ++c) {
                        long xoff = (((long)b * Cin + (long)g * cpg + c) * H) * W;
                        for (int u = 0; u < kh; ++u) {
                            int h = r * stride - pad + u;
                            if (h < 0 || h >= H) continue;
                            for (int v = 0; v < kw; ++v) {
                                int ww = s * stride - pad + v;
                                if (ww < 0 || ww >= W) continue;
                                long e = (long)o * per_o + ((long)c * kh + u) * kw + v;
                                dw[e] += d * (double)x[xoff + (long)h * W + ww];
                                if (dxb)
                                    dxb[xoff - (long)b * Cin * H * W + (long)h * W + ww] += w[e] * d;
                            }
                        }
                    }
                }
            }
        }
        if (dalpha) {
            for (int i = 0; i < n; ++i) {
                double acc = 0.0;
                for (long e = 0; e < wsz; ++e)
                    acc += dw[e] * (double)experts[(long)i * wsz + e];
                dalpha[(long)b * n + i] = acc;
            }
        }
    }
    if (dexperts) {
#pragma omp parallel for schedule(static)
        for (long e = 0; e < wsz; ++e) {
            for (int i = 0; i < n; ++i) {
                double acc = 0.0;
                for (int b = 0; b < B; ++b)
                    acc += alpha[(long)b * n + i] * dwb[(long)b * wsz + e];
                dexperts[(long)i * wsz + e] = acc;
            }
        }
    }
    free(dwb);
    free(wb);
    return ORACLE_OK;
}

/*
 * Gradients of the layer with FMDConv's channel attentions
 * (oracle_forward_attn; FMDConv: Fast multi-attention dynamic convolution,
 * abstract) for a given output gradient dy. With
 *   z[b,o,r,s] = sum_{c,u,v} W_b[o,c,u,v] * a_in[b,gc] * x[b,gc,h,w],
 *   y[b,o,r,s] = a_out[b,o] * z[b,o,r,s],   W_b = sum_i alpha[b,i] E_i,
 * the derivative of the loss sum(dy * y), term by term:
 *   dW_b[o,c,u,v] = a_out[b,o] * a_in[b,gc] * sum_{r,s} dy[b,o,r,s] * x[b,gc,h,w]
 *   dalpha[b,i]   = sum_e dW_b[e] * E_i[e],   dE_i[e] = sum_b alpha[b,i] * dW_b[e]
 *   da_out[b,o]   = sum_{r,s} dy[b,o,r,s] * z[b,o,r,s]
 *   da_in[b,gc]   = sum over (o, r, s, u, v) of dy[b,o,r,s] * a_out[b,o] * W_b[o,c,u,v] * x[b,gc,h,w]
 *   dx[b,gc,h,w]  = a_in[b,gc] * sum over the (o, r, s, u, v) whose output read x[b,gc,h,w]
 *                   of a_out[b,o] * W_b[o,c,u,v] * dy[b,o,r,s]
 * (h = r*stride - pad + u, w = s*stride - pad + v; positions outside the image
 * take no part). a_in or a_out may be NULL (all ones); each output may be
 * NULL (not computed). da_in: [B,Cin]; da_out: [B,Cout]; the rest as
 * oracle_backward.
 */
int oracle_backward_attn(int B, int Cin, int H, int W, int Cout, int kh, int kw,
                         int stride, int pad, int groups, int n, const float *x,
                         const float *experts, const double *alpha, const double *a_in,
                         const double *a_out, const float *dy, double *dx,
                         double *dalpha, double *dexperts, double *da_in, double *da_out)
{
    if (B < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || kh < 1 || kw < 1 ||
        stride < 1 || pad < 0 || groups < 1 || n < 1 || !x || !experts ||
        !alpha || !dy)
        return ORACLE_BAD_ARG;
    if (Cin % groups || Cout % groups) return ORACLE_BAD_ARG;
    int Ho = out_size(H, kh, stride, pad), Wo = out_size(W, kw, stride, pad);
    if (Ho < 1 || Wo < 1) return ORACLE_BAD_ARG;
    int cpg = Cin / groups, opg = Cout / groups;
    long per_o = (long)cpg * kh * kw;
    long wsz = (long)Cout * per_o;
    double *dwb = (double *)calloc((size_t)B * wsz, sizeof(double));
    double *wb = (double *)malloc(sizeof(double) * (size_t)B * wsz);
    if (!dwb || !wb) { free(dwb); free(wb); return ORACLE_BAD_ARG; }
#pragma omp parallel for schedule(static)
    for (int b = 0; b < B; ++b) {
        double *w = wb + (long)b * wsz;
        for (long e = 0; e < wsz; ++e) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i)
                acc += alpha[(long)b * n + i] * (double)experts[(long)i * wsz + e];
            w[e] = acc;
        }
        double *dw = dwb + (long)b * wsz;
        double *dxb = dx ? dx + (long)b * Cin * H * W : NULL;
        if (dxb)
            for (long j = 0; j < (long)Cin * H * W; ++j) dxb[j] = 0.0;
        if (da_in)
            for (int c = 0; c < Cin; ++c) da_in[(long)b * Cin + c] = 0.0;
        for (int o = 0; o < Cout; ++o) {
            int g = o / opg;
            double so = a_out ? a_out[(long)b * Cout + o] : 1.0;
            double dso = 0.0; /* sum over (r, s) of dy * z */
            for (int r = 0; r < Ho; ++r) {
                for (int s = 0; s < Wo; ++s) {
                    double d = (double)dy[(((long)b * Cout + o) * Ho + r) * Wo + s];
                    double z = 0.0;
                    for (int c = 0; c < cpg; ++c) {
                        int gc = g * cpg + c;
                        double si = a_in ? a_in[(long)b * Cin + gc] : 1.0;
                        long xoff = (((long)b * Cin + gc) * H) * W;
                        double dsi = 0.0;
                        for (int u = 0; u < kh; ++u) {
                            int h = r * stride - pad + u;
                            if (h < 0 || h >= H) continue;
                            for (int v = 0; v < kw; ++v) {
                                int ww = s * stride - pad + v;
                                if (ww < 0 || ww >= W) continue;
                                long e = (long)o * per_o + ((long)c * kh + u) * kw + v;
                                double xv = (double)x[xoff + (long)h * W + ww];
                                z += w[e] * si * xv;
                                dw[e] += so * si * d * xv;
                                dsi += d * so * w[e] * xv;
                                if (dxb)
                                    dxb[xoff - (long)b * Cin * H * W + (long)h * W + ww] += si * so * w[e] * d;
                            }
                        }
                        if (da_in) da_in[(long)b * Cin + gc] += dsi;
                    }
                    dso += d * z;
                }
            }
            if (da_out) da_out[(long)b * Cout + o] = dso;
        }
        if (dalpha) {
            for (int i = 0; i < n; ++i) {
                double acc = 0.0;
                for (long e = 0; e < wsz; ++e)
                    acc += dw[e] * (double)experts[(long)i * wsz + e];
                dalpha[(long)b * n + i] = acc;
            }
        }
    }
    if (dexperts) {
#pragma omp parallel for schedule(static)
        for (long e = 0; e < wsz; ++e) {
            for (int i = 0; i < n; ++i) {
                double acc = 0.0;
                for (int b = 0; b < B; ++b)
                    acc += alpha[(long)b * n + i] * dwb[(long)b * wsz + e];
                dexperts[(long)i * wsz + e] = acc;
            }
        }
    }
    free(dwb);
    free(wb);
    return ORACLE_OK;
}
