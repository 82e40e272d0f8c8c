// Gradients of the dynamic convolution layer and of its routing on gfx950.
//
// The pages train these layers end to end ("learn specialized convolutional
// kernels for each example", CondConv: Conditionally Parameterized
// Convolutions, abstract; "learns a linear mixture of n static kernels
// weighted with their input-dependent attentions", KernelWarehouse:
// Rethinking the Design of Dynamic Convolution, abstract) without printing a
// backward pass. The kernels below compute the derivative of the forward
// W_b = sum_i alpha[b,i] E_i, y_b = conv(x_b, W_b):
//
//   dW_b[o][c,u,v] = sum_{r,s} dy[b,o,r,s] * x[b,c, r*st-p+u, s*st-p+v]
//   dalpha[b,i]    = <dW_b, E_i>,    dE_i = sum_b alpha[b,i] dW_b
//   dx_b           = the transposed convolution of dy_b with W_b
//
// The data gradient runs through the forward convolutions (api.cpp): for
// stride 1 it is the forward layer applied to dy with the bank transposed in
// its channels and flipped in its taps (flip_experts_kernel) and padding
// k - 1 - p. The kernel gradient is a GEMM per example (M = output
// channels, N = kernel columns (c, u, v), reduction over output positions)
// on the matrix cores; dW_b goes to an fp32 workspace and two contraction
// kernels reduce it to dalpha and dE.
#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

// ---- bank transposed in its channels and flipped in its taps --------------
// src [n][R][S][KH][KW] -> dst [n][S][R][KH][KW], dst[i][s][r][u][v] =
// src[i][r][s][KH-1-u][KW-1-v]. groups == 1: R = Cout, S = Cin; depthwise:
// R = 1, S = C (a flip only).
template <typename T>
__global__ __launch_bounds__(256) void flip_experts_kernel(const T *__restrict__ src, T *__restrict__ dst,
                                                           long total, int R, int S, int KH, int KW) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int KT = KH * KW;
    const int t = (int)(idx % KT);
    const long q = idx / KT;
    const int r = (int)(q % R);
    const long q2 = q / R;
    const int s = (int)(q2 % S);
    const long i = q2 / S;
    const int u = t / KW, v = t - u * KW;
    dst[idx] = src[((i * R + r) * S + s) * KT + (KH - 1 - u) * KW + (KW - 1 - v)];
}

// ---- kernel gradient per example (groups == 1) ------------------------------
// Workgroup (tile, b): a 64 x 64 block of dW_b (output channels o0.., kernel
// columns K0.., K = c * KT + t) reduced over the example's output positions
// in chunks of 32. Both operands are staged position-contiguous in LDS:
//   A[o][p] = dy[b, o, p],   B[K][p] = x[b, c, r*st - pad + u, s*st - pad + v]
// (zero outside the image, past P, Cout or Kdim), so a lane's MFMA fragment
// (8 consecutive positions of one row) is one 16-byte LDS read. Four waves
// each own a 32 x 32 quarter of the block.
struct WgArgs {
    int B, Cin, H, W, Cout, KW, stride, pad, Wo, P, KT, Kdim, n_ktiles;
};

template <typename T> struct WgPitch;
template <> struct WgPitch<uint16_t> { static constexpr int v = 40; };  // 80-byte LDS rows
template <> struct WgPitch<float> { static constexpr int v = 36; };     // 144-byte LDS rows

template <typename T>
__device__ __forceinline__ void lds_store8(T *dst, const T (&v)[8]);
template <>
__device__ __forceinline__ void lds_store8<uint16_t>(uint16_t *dst, const uint16_t (&v)[8]) {
    u32x4_t w;
    w.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
    w.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
    w.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
    w.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
    *reinterpret_cast<u32x4_t *>(dst) = w;
}
template <>
__device__ __forceinline__ void lds_store8<float>(float *dst, const float (&v)[8]) {
    f32x4_t a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    reinterpret_cast<f32x4_t *>(dst)[0] = a;
    reinterpret_cast<f32x4_t *>(dst)[1] = b;
}

template <typename T>
__global__ __launch_bounds__(256) void wgrad_kernel(const T *__restrict__ x, const T *__restrict__ dy,
                                                    float *__restrict__ dw, WgArgs a) {
    constexpr int PITCH = WgPitch<T>::v;
    __shared__ __attribute__((aligned(16))) T s_a[64 * PITCH];
    __shared__ __attribute__((aligned(16))) T s_b[64 * PITCH];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int mh = wave & 1, nh = wave >> 1;
    const int b = blockIdx.y;
    const int ot = blockIdx.x / a.n_ktiles, kt = blockIdx.x - ot * a.n_ktiles;
    const int o0 = ot * 64, K0 = kt * 64;
    // staging role: row `row` of both tiles, positions 8 * seg .. + 7 of the chunk
    const int row = tid >> 2, seg = tid & 3;
    const int o = o0 + row;
    const bool o_ok = o < a.Cout;
    const T *dyrow = dy + ((long)b * a.Cout + (o_ok ? o : 0)) * a.P;
    const int K = K0 + row;
    const bool k_ok = K < a.Kdim;
    const int kc = k_ok ? K / a.KT : 0;
    const int kt_ = k_ok ? K - kc * a.KT : 0;
    const int ku = kt_ / a.KW, kv = kt_ - ku * a.KW;
    const T *xplane = x + ((long)b * a.Cin + kc) * a.H * a.W;
    f32x16_t acc = {};
    for (int p0 = 0; p0 < a.P; p0 += 32) {
        T av[8], bv[8];
        const int p = p0 + 8 * seg;
        int r = p / a.Wo, s = p - r * a.Wo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool pin = p + j < a.P;
            av[j] = (o_ok && pin) ? dyrow[p + j] : T(0);
            const int h = r * a.stride - a.pad + ku, w = s * a.stride - a.pad + kv;
            const bool xin = k_ok && pin && h >= 0 && h < a.H && w >= 0 && w < a.W;
            bv[j] = xin ? xplane[(long)h * a.W + w] : T(0);
            if (++s == a.Wo) { s = 0; ++r; }
        }
        __syncthreads();  // the previous chunk's fragment reads are done
        lds_store8<T>(s_a + row * PITCH + 8 * seg, av);
        lds_store8<T>(s_b + row * PITCH + 8 * seg, bv);
        __syncthreads();
        const T *pa = s_a + (32 * mh + l32) * PITCH;
        const T *pb = s_b + (32 * nh + l32) * PITCH;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8_t af = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(pa + 16 * ks + 8 * lh));
                const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(pb + 16 * ks + 8 * lh));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 16; ++ks)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(pa[2 * ks + lh], pb[2 * ks + lh], acc, 0, 0, 0);
        }
    }
    // D(lane, 4j + q) = row 8j + 4 lh + q, column l32 of the wave's quarter
    const int KK = K0 + 32 * nh + l32;
    if (KK >= a.Kdim) return;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int oo = o0 + 32 * mh + 8 * j + 4 * lh + q;
            if (oo < a.Cout) dw[((long)b * a.Cout + oo) * a.Kdim + KK] = acc[4 * j + q];
        }
}

// ---- kernel gradient per example, depthwise --------------------------------
// Workgroup (c, b): dW_b[c][t] = sum_p dy[b,c,p] * x[b,c, shifted by tap t].
// Each thread sums its positions for every tap, then the block reduces.
constexpr int kDwTaps = 64;
template <typename T>
__global__ __launch_bounds__(256) void wgrad_dw_kernel(const T *__restrict__ x, const T *__restrict__ dy,
                                                       float *__restrict__ dw, WgArgs a) {
    __shared__ float s_red[4][kDwTaps];
    const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const T *xp = x + ((long)b * a.Cin + c) * a.H * a.W;
    const T *dp = dy + ((long)b * a.Cin + c) * a.P;
    float part[kDwTaps];
#pragma unroll
    for (int t = 0; t < kDwTaps; ++t) part[t] = 0.f;
    for (int p = tid; p < a.P; p += 256) {
        const int r = p / a.Wo, s = p - r * a.Wo;
        const float d = Elem<T>::to_f32(dp[p]);
#pragma unroll
        for (int t = 0; t < kDwTaps; ++t) {
            if (t < a.KT) {
                const int u = t / a.KW, v = t - u * a.KW;
                const int h = r * a.stride - a.pad + u, w = s * a.stride - a.pad + v;
                if (h >= 0 && h < a.H && w >= 0 && w < a.W) part[t] += d * Elem<T>::to_f32(xp[(long)h * a.W + w]);
            }
        }
    }
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int t = 0; t < kDwTaps; ++t) {
        if (t < a.KT) {
            const float v = wave_sum(part[t]);
            if (lane == 0) s_red[wave][t] = v;
        }
    }
    __syncthreads();
    if (tid < a.KT)
        dw[((long)b * a.Cin + c) * a.KT + tid] = (s_red[0][tid] + s_red[1][tid]) + (s_red[2][tid] + s_red[3][tid]);
}

// ---- contractions of dW_b -----------------------------------------------------
// dalpha[b][i] = sum_e dW_b[e] * E_i[e]: workgroup per example, up to 8
// experts per pass over dW_b.
template <typename T>
__global__ __launch_bounds__(256) void dalpha_kernel(const float *__restrict__ dw, const T *__restrict__ e,
                                                     float *__restrict__ dalpha, long wsize, int n) {
    __shared__ float s_red[4][8];
    const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const float *d = dw + (long)b * wsize;
    for (int i0 = 0; i0 < n; i0 += 8) {
        float acc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = 0.f;
        for (long j = tid; j < wsize; j += 256) {
            const float v = d[j];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (i0 + k < n) acc[k] += v * Elem<T>::to_f32(e[(long)(i0 + k) * wsize + j]);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float v = wave_sum(acc[k]);
            if (lane == 0) s_red[wave][k] = v;
        }
        __syncthreads();
        if (tid < 8 && i0 + tid < n)
            dalpha[(long)b * n + i0 + tid] = (s_red[0][tid] + s_red[1][tid]) + (s_red[2][tid] + s_red[3][tid]);
        __syncthreads();
    }
}

// dE[i][e] = sum_b alpha[b][i] * dW_b[e]: thread per element e, up to 8
// experts per pass; every example's dW_b is read once per pass.
__global__ __launch_bounds__(256) void dexperts_kernel(const float *__restrict__ dw, const float *__restrict__ alpha,
                                                       float *__restrict__ de, long wsize, int B, int n) {
    const long j = (long)blockIdx.x * 256 + threadIdx.x;
    if (j >= wsize) return;
    for (int i0 = 0; i0 < n; i0 += 8) {
        float acc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = 0.f;
        for (int b = 0; b < B; ++b) {
            const float v = dw[(long)b * wsize + j];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (i0 + k < n) acc[k] += alpha[(long)b * n + i0 + k] * v;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (i0 + k < n) de[(long)(i0 + k) * wsize + j] = acc[k];
    }
}

// ---- routing gradient -----------------------------------------------------------
// Workgroup per example: dz from alpha and dalpha (sigmoid:
// dalpha * alpha * (1 - alpha); softmax(z/T): alpha * (dalpha - <alpha,
// dalpha>) / T), then dgap[b][c] = sum_i dz[b][i] fc_w[i][c].
__global__ __launch_bounds__(256) void route_dz_kernel(const float *__restrict__ alpha,
                                                       const float *__restrict__ dalpha,
                                                       const float *__restrict__ fc_w, float *__restrict__ dz,
                                                       float *__restrict__ dgap, int n, int C, int mode,
                                                       float inv_t) {
    __shared__ float s_dz[256];
    __shared__ float s_red[4];
    const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const float a = tid < n ? alpha[(long)b * n + tid] : 0.f;
    const float d = tid < n ? dalpha[(long)b * n + tid] : 0.f;
    float z;
    if (mode == 0) {
        z = d * a * (1.f - a);
    } else {
        const float part = wave_sum(a * d);
        if (lane == 0) s_red[wave] = part;
        __syncthreads();
        const float inner = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
        z = a * (d - inner) * inv_t;
    }
    if (tid < n) {
        s_dz[tid] = z;
        dz[(long)b * n + tid] = z;
    }
    __syncthreads();
    for (int c = tid; c < C; c += 256) {
        float acc = 0.f;
        for (int i = 0; i < n; ++i) acc += s_dz[i] * fc_w[(long)i * C + c];
        dgap[(long)b * C + c] = acc;
    }
}

// dfc_w[i][c] = sum_b dz[b][i] gap[b][c] (thread per (i, c)); the threads
// of column c == 0 also write dfc_b[i] = sum_b dz[b][i].
__global__ __launch_bounds__(256) void route_dfc_kernel(const float *__restrict__ dz, const float *__restrict__ gap,
                                                        float *__restrict__ dfc_w, float *__restrict__ dfc_b,
                                                        int B, int n, int C) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)n * C) return;
    const int i = (int)(idx / C), c = (int)(idx - (long)i * C);
    float acc = 0.f, accb = 0.f;
    for (int b = 0; b < B; ++b) {
        const float z = dz[(long)b * n + i];
        acc += z * gap[(long)b * C + c];
        accb += z;
    }
    dfc_w[idx] = acc;
    if (c == 0 && dfc_b) dfc_b[i] = accb;
}

// dx[b][c][h][w] += dgap[b][c] / (H W): the pooling's share of the input
// gradient, added in float32 and rounded once to the element type.
template <typename T>
__global__ __launch_bounds__(256) void add_pool_grad_kernel(T *__restrict__ dx, const float *__restrict__ dgap,
                                                            long total, int hw, float inv_hw) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const float v = Elem<T>::to_f32(dx[idx]) + dgap[idx / hw] * inv_hw;
    dx[idx] = Elem<T>::from_f32(v);
}

unsigned blocks_for(long total) { return (unsigned)((total + 255) / 256); }

}  // namespace

hipError_t launch_flip_experts(const Geom &g, const void *experts, void *flipped, hipStream_t stream) {
    const int R = g.groups == 1 ? g.Cout : 1;
    const int S = g.Cin;
    const long total = (long)g.n * R * S * g.KT;
    if (g.bf16)
        hipLaunchKernelGGL(flip_experts_kernel<uint16_t>, dim3(blocks_for(total)), dim3(256), 0, stream,
                           static_cast<const uint16_t *>(experts), static_cast<uint16_t *>(flipped), total, R, S,
                           g.KH, g.KW);
    else
        hipLaunchKernelGGL(flip_experts_kernel<float>, dim3(blocks_for(total)), dim3(256), 0, stream,
                           static_cast<const float *>(experts), static_cast<float *>(flipped), total, R, S, g.KH,
                           g.KW);
    return hipGetLastError();
}

size_t wgrad_bytes(const Geom &g) { return (size_t)g.B * g.Cout * g.cpg * g.KT * sizeof(float); }

bool wgrad_dw_supported(const Geom &g) { return g.KT <= kDwTaps; }

hipError_t launch_backward_weights(const Geom &g, const void *x, const void *dy, const void *experts,
                                   const float *alpha, float *dwb, float *dalpha, float *dexperts,
                                   hipStream_t stream) {
    WgArgs a;
    a.B = g.B; a.Cin = g.Cin; a.H = g.H; a.W = g.W; a.Cout = g.Cout; a.KW = g.KW;
    a.stride = g.stride; a.pad = g.pad; a.Wo = g.Wo; a.P = g.P; a.KT = g.KT;
    a.Kdim = g.cpg * g.KT;
    a.n_ktiles = ceil_div(a.Kdim, 64);
    if (g.groups == 1) {
        const dim3 grid((unsigned)(ceil_div(g.Cout, 64) * a.n_ktiles), (unsigned)g.B);
        if (g.bf16)
            hipLaunchKernelGGL(wgrad_kernel<uint16_t>, grid, dim3(256), 0, stream,
                               static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(dy), dwb, a);
        else
            hipLaunchKernelGGL(wgrad_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float *>(x),
                               static_cast<const float *>(dy), dwb, a);
    } else {
        const dim3 grid((unsigned)g.Cin, (unsigned)g.B);
        if (g.bf16)
            hipLaunchKernelGGL(wgrad_dw_kernel<uint16_t>, grid, dim3(256), 0, stream,
                               static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(dy), dwb, a);
        else
            hipLaunchKernelGGL(wgrad_dw_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float *>(x),
                               static_cast<const float *>(dy), dwb, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long wsize = (long)g.Cout * g.cpg * g.KT;
    if (dalpha) {
        if (g.bf16)
            hipLaunchKernelGGL(dalpha_kernel<uint16_t>, dim3((unsigned)g.B), dim3(256), 0, stream, dwb,
                               static_cast<const uint16_t *>(experts), dalpha, wsize, g.n);
        else
            hipLaunchKernelGGL(dalpha_kernel<float>, dim3((unsigned)g.B), dim3(256), 0, stream, dwb,
                               static_cast<const float *>(experts), dalpha, wsize, g.n);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (dexperts) {
        hipLaunchKernelGGL(dexperts_kernel, dim3(blocks_for(wsize)), dim3(256), 0, stream, dwb, alpha, dexperts,
                           wsize, g.B, g.n);
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_route_backward(const Geom &g, const void *x, const float *fc_w, int mode, float temperature,
                                 const float *alpha, const float *dalpha, float *gap, float *dz, float *dgap,
                                 float *dfc_w, float *dfc_b, void *dx, hipStream_t stream) {
    hipError_t e = launch_gap(g, x, gap, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_dz_kernel, dim3((unsigned)g.B), dim3(256), 0, stream, alpha, dalpha, fc_w, dz, dgap,
                       g.n, g.Cin, mode, mode == 1 ? 1.f / temperature : 1.f);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long nc = (long)g.n * g.Cin;
    hipLaunchKernelGGL(route_dfc_kernel, dim3(blocks_for(nc)), dim3(256), 0, stream, dz, gap, dfc_w, dfc_b, g.B,
                       g.n, g.Cin);
    e = hipGetLastError();
    if (e != hipSuccess || !dx) return e;
    const long total = (long)g.B * g.Cin * g.H * g.W;
    const int hw = g.H * g.W;
    if (g.bf16)
        hipLaunchKernelGGL(add_pool_grad_kernel<uint16_t>, dim3(blocks_for(total)), dim3(256), 0, stream,
                           static_cast<uint16_t *>(dx), dgap, total, hw, 1.f / (float)hw);
    else
        hipLaunchKernelGGL(add_pool_grad_kernel<float>, dim3(blocks_for(total)), dim3(256), 0, stream,
                           static_cast<float *>(dx), dgap, total, hw, 1.f / (float)hw);
    return hipGetLastError();
}

}  // namespace dynconv
