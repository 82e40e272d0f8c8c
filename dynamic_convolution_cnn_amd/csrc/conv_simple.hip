// Convolutions that are not MFMA contractions.
//
// conv_direct_f32_kernel: float32 per-example convolution (groups == 1) with
//   the mixed kernels W_b already in memory, one output element per thread,
//   accumulating in float32 in (channel, row tap, column tap) order. It
//   serves the float32 layers, where the contract is 1e-5 relative and no
//   bf16 rounding may occur.
// depthwise_kernel: depthwise convolution (groups == Cin == Cout), one
//   (example, channel) plane per workgroup. The plane's kh*kw taps are mixed
//   in the workgroup from the n experts (W_b[c] = sum_i alpha_bi E_i[c];
//   KernelWarehouse abstract) and, for bf16, rounded to bf16 like every
//   other mixed kernel; the zero-padded input plane is staged in LDS as
//   float; each thread computes a strip of outputs along a row, so input
//   values are reused from registers across the strip.
#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

__global__ __launch_bounds__(256) void conv_direct_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ w, float *__restrict__ y, int B,
    int Cin, int H, int W, int Cout, int KH, int KW, int stride, int pad, int Ho, int Wo) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const long total = (long)B * Cout * Ho * Wo;
    if (idx >= total) return;
    const int s = (int)(idx % Wo);
    long r1 = idx / Wo;
    const int r = (int)(r1 % Ho);
    r1 /= Ho;
    const int o = (int)(r1 % Cout);
    const int b = (int)(r1 / Cout);
    const float *wo = w + ((long)b * Cout + o) * Cin * KH * KW;
    const float *xb = x + (long)b * Cin * H * W;
    float acc = 0.f;
    for (int c = 0; c < Cin; ++c) {
        const float *xc = xb + (long)c * H * W;
        const float *wc = wo + (long)c * KH * KW;
        for (int u = 0; u < KH; ++u) {
            const int h = r * stride - pad + u;
            if (h < 0 || h >= H) continue;
            for (int v = 0; v < KW; ++v) {
                const int ww = s * stride - pad + v;
                if (ww < 0 || ww >= W) continue;
                acc = fmaf(wc[u * KW + v], xc[h * W + ww], acc);
            }
        }
    }
    y[idx] = acc;
}

constexpr int kDwMaxTaps = 64;
constexpr int kDwStrip = 4;  // outputs per thread along a row

template <typename T>
__global__ __launch_bounds__(256) void depthwise_kernel(
    const T *__restrict__ x, const T *__restrict__ experts, const float *__restrict__ alpha,
    const T *__restrict__ wmixed, T *__restrict__ y, int B, int C, int H, int W, int KH, int KW,
    int stride, int pad, int Ho, int Wo, int n) {
    extern __shared__ __attribute__((aligned(16))) float plane[];
    __shared__ float taps[kDwMaxTaps];
    const int bc = blockIdx.x;
    const int b = bc / C, c = bc - b * C;
    const int KT = KH * KW;
    const int Hp = H + 2 * pad, Wp = W + 2 * pad;
    if (threadIdx.x < KT) {
        float wv;
        if (wmixed) {
            wv = Elem<T>::to_f32(wmixed[(long)bc * KT + threadIdx.x]);
        } else {
            float s = 0.f;
            for (int i = 0; i < n; ++i)
                s = fmaf(alpha[(long)b * n + i],
                         Elem<T>::to_f32(experts[((long)i * C + c) * KT + threadIdx.x]), s);
            // mixed kernel in the storage type, as the materialised path would hold it
            wv = Elem<T>::to_f32(Elem<T>::from_f32(s));
        }
        taps[threadIdx.x] = wv;
    }
    const T *xp = x + (long)bc * H * W;
    for (int i = threadIdx.x; i < Hp * Wp; i += 256) {
        const int hh = i / Wp - pad, ww = i % Wp - pad;
        plane[i] = (hh >= 0 && hh < H && ww >= 0 && ww < W) ? Elem<T>::to_f32(xp[hh * W + ww]) : 0.f;
    }
    __syncthreads();
    const int strips_per_row = (Wo + kDwStrip - 1) / kDwStrip;
    T *yp = y + (long)bc * Ho * Wo;
    for (int task = threadIdx.x; task < Ho * strips_per_row; task += 256) {
        const int r = task / strips_per_row;
        const int s0 = (task - r * strips_per_row) * kDwStrip;
        float acc[kDwStrip];
#pragma unroll
        for (int j = 0; j < kDwStrip; ++j) acc[j] = 0.f;
        for (int u = 0; u < KH; ++u) {
            const float *row = plane + (r * stride + u) * Wp;
            for (int v = 0; v < KW; ++v) {
                const float wv = taps[u * KW + v];
#pragma unroll
                for (int j = 0; j < kDwStrip; ++j) {
                    const int col = min(s0 + j, Wo - 1) * stride + v;
                    acc[j] = fmaf(wv, row[col], acc[j]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kDwStrip; ++j)
            if (s0 + j < Wo) yp[r * Wo + s0 + j] = Elem<T>::from_f32(acc[j]);
    }
}

}  // namespace

hipError_t launch_conv_direct_f32(const Geom &g, const float *x, const float *wmixed, float *y,
                                  hipStream_t stream) {
    const long total = (long)g.B * g.Cout * g.Ho * g.Wo;
    hipLaunchKernelGGL(conv_direct_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, stream, x, wmixed, y, g.B, g.Cin, g.H, g.W, g.Cout, g.KH, g.KW,
                       g.stride, g.pad, g.Ho, g.Wo);
    return hipGetLastError();
}

static size_t dw_lds_bytes(const Geom &g) {
    return (size_t)(g.H + 2 * g.pad) * (g.W + 2 * g.pad) * sizeof(float);
}

bool depthwise_supported(const Geom &g) {
    return g.groups == g.Cin && g.Cin == g.Cout && g.KT <= kDwMaxTaps &&
           dw_lds_bytes(g) <= 64 * 1024;
}

hipError_t launch_conv_depthwise(const Geom &g, const void *x, const void *experts,
                                 const float *alpha, const void *wmixed, void *y,
                                 hipStream_t stream) {
    const size_t lds = dw_lds_bytes(g);
    const dim3 grid((unsigned)((long)g.B * g.Cin));
    if (g.bf16) {
        hipLaunchKernelGGL(depthwise_kernel<uint16_t>, grid, dim3(256), lds, stream,
                           static_cast<const uint16_t *>(x),
                           static_cast<const uint16_t *>(experts), alpha,
                           static_cast<const uint16_t *>(wmixed), static_cast<uint16_t *>(y),
                           g.B, g.Cin, g.H, g.W, g.KH, g.KW, g.stride, g.pad, g.Ho, g.Wo, g.n);
    } else {
        hipLaunchKernelGGL(depthwise_kernel<float>, grid, dim3(256), lds, stream,
                           static_cast<const float *>(x), static_cast<const float *>(experts),
                           alpha, static_cast<const float *>(wmixed), static_cast<float *>(y),
                           g.B, g.Cin, g.H, g.W, g.KH, g.KW, g.stride, g.pad, g.Ho, g.Wo, g.n);
    }
    return hipGetLastError();
}

}  // namespace dynconv
