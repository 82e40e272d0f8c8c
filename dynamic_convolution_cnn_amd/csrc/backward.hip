// Gradients of the dynamic convolution layer and of its routing on gfx950.
//
// The pages train these layers end to end (CondConv: Conditionally
// Parameterized Convolutions, abstract, where each example's kernel is
// learned; KernelWarehouse: Rethinking the Design of Dynamic Convolution,
// abstract, where the mixture of static kernels and its attentions are
// learned) without printing a backward pass. The kernels below compute the derivative of the forward
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
// on the matrix cores (depthwise: per-plane tap sums on the VALU). For bf16
// stride-1 layers with n <= 4 and 1 x 1 or k x 3 kernels the contraction is
// fused into that GEMM (wgrad_fused.hip); elsewhere dW_b goes to an fp32
// workspace, and one pass over it (contract_kernel) yields dE and per-chunk
// partial sums of dalpha, which a small kernel reduces.
#include <algorithm>

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
// Workgroup (tile, b): a 128 x 64 block of dW_b (output channels o0..,
// kernel columns K0.., K = c * KT + t) reduced over the example's output
// positions in chunks of 32. Both operands are staged position-contiguous in
// LDS:
//   A[o][p] = dy[b, o, p],   B[K][p] = x[b, c, r*st - pad + u, s*st - pad + v]
// (zero outside the image, past P, Cout or Kdim), so a lane's MFMA fragment
// (8 consecutive positions of one row) is one 16-byte LDS read. Wave w owns
// output rows 64 (w & 1) .. + 63 (two 32-row blocks) and kernel columns
// 32 (w >> 1) .. + 31. The next chunk's global loads are issued before the
// current chunk's MFMAs, so their latency hides behind the matrix work.
struct WgArgs {
    int B, Cin, H, W, Cout, KW, stride, pad, Ho, Wo, P, KT, Kdim, n_ktiles;
    int dy_vec;  // P % 4 == 0: rows of dy are read with 8- or 16-byte loads
};

template <typename T> struct WgPitch;
template <> struct WgPitch<uint16_t> { static constexpr int v = 40; };  // 80-byte LDS rows (32 positions + pad)
template <> struct WgPitch<float> { static constexpr int v = 36; };     // 144-byte LDS rows

// 8 consecutive elements of one staged row, in registers.
template <typename T> struct Row8;
template <> struct Row8<uint16_t> {
    u32x4_t v;
    __device__ __forceinline__ void zero() { v = u32x4_t{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ void set(int j, uint16_t h) {
        const uint32_t m = (j & 1) ? 0xffff0000u : 0x0000ffffu;
        const uint32_t w = (j & 1) ? ((uint32_t)h << 16) : (uint32_t)h;
        v[j >> 1] = (v[j >> 1] & ~m) | w;
    }
    __device__ __forceinline__ void load_vec(const uint16_t *p) {  // 8-byte aligned
        const u32x2_t a = *reinterpret_cast<const u32x2_t *>(p);
        const u32x2_t b = *reinterpret_cast<const u32x2_t *>(p + 4);
        v = u32x4_t{a.x, a.y, b.x, b.y};
    }
    __device__ __forceinline__ void store(uint16_t *dst) const { *reinterpret_cast<u32x4_t *>(dst) = v; }
    __device__ __forceinline__ void pack(const uint16_t (&h)[8]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (uint32_t)h[2 * j] | ((uint32_t)h[2 * j + 1] << 16);
    }
};
template <> struct Row8<float> {
    f32x4_t v0, v1;
    __device__ __forceinline__ void zero() { v0 = f32x4_t{0.f, 0.f, 0.f, 0.f}; v1 = v0; }
    __device__ __forceinline__ void set(int j, float f) {
        if (j < 4) v0[j] = f;
        else v1[j - 4] = f;
    }
    __device__ __forceinline__ void load_vec(const float *p) {  // 16-byte aligned
        v0 = reinterpret_cast<const f32x4_t *>(p)[0];
        v1 = reinterpret_cast<const f32x4_t *>(p)[1];
    }
    __device__ __forceinline__ void store(float *dst) const {
        reinterpret_cast<f32x4_t *>(dst)[0] = v0;
        reinterpret_cast<f32x4_t *>(dst)[1] = v1;
    }
    __device__ __forceinline__ void pack(const float (&h)[8]) {
        v0 = f32x4_t{h[0], h[1], h[2], h[3]};
        v1 = f32x4_t{h[4], h[5], h[6], h[7]};
    }
};

template <typename T>
__global__ __launch_bounds__(256) void wgrad_kernel(const T *__restrict__ x, const T *__restrict__ dy,
                                                    float *__restrict__ dw, WgArgs a) {
    constexpr int PITCH = WgPitch<T>::v;
    __shared__ __attribute__((aligned(16))) T s_a[128 * PITCH];
    __shared__ __attribute__((aligned(16))) T s_b[64 * PITCH];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int mq = wave & 1, nh = wave >> 1;
    const int b = blockIdx.y;
    const int ot = blockIdx.x / a.n_ktiles, kt = blockIdx.x - ot * a.n_ktiles;
    const int o0 = ot * 128, K0 = kt * 64;
    // staging roles: dy rows `row` and `row + 64`, im2col row `row`;
    // positions 8 * seg .. + 7 of the chunk
    const int row = tid >> 2, seg = tid & 3;
    const T *dyrow[2];
    bool o_ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int o = o0 + row + 64 * h;
        o_ok[h] = o < a.Cout;
        dyrow[h] = dy + ((long)b * a.Cout + (o_ok[h] ? o : 0)) * a.P;
    }
    const int K = K0 + row;
    const bool k_ok = K < a.Kdim;
    const int kc = k_ok ? K / a.KT : 0;
    const int kt_ = k_ok ? K - kc * a.KT : 0;
    const int ku = kt_ / a.KW, kv = kt_ - ku * a.KW;
    const T *xplane = x + ((long)b * a.Cin + kc) * a.H * a.W;
    const int r_lo = max(0, ceil_div(a.pad - ku, a.stride)), r_hi = ceil_div(a.H + a.pad - ku, a.stride);
    const int s_lo = max(0, ceil_div(a.pad - kv, a.stride)), s_hi = ceil_div(a.W + a.pad - kv, a.stride);
    const long row_step = (long)a.stride * a.W - (long)a.Wo * a.stride;
    Row8<T> ra[2], rb;
    auto load = [&](int p0) {
        const int p = p0 + 8 * seg;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (a.dy_vec && o_ok[h] && p + 8 <= a.P) {
                ra[h].load_vec(dyrow[h] + p);
            } else {
                ra[h].zero();
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (o_ok[h] && p + j < a.P) ra[h].set(j, dyrow[h][p + j]);
            }
        }
        // the thread's tap is fixed: output row r reads inside the image for
        // r in [r_lo, r_hi), column s for s in [s_lo, s_hi); the x address
        // moves by the stride along a row and by row_step to the next row
        T xv[8];
        int r = p / a.Wo, s = p - r * a.Wo;
        long addr = (long)(r * a.stride - a.pad + ku) * a.W + (s * a.stride - a.pad + kv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            xv[j] = T(0);
            if (k_ok && p + j < a.P && r >= r_lo && r < r_hi && s >= s_lo && s < s_hi) xv[j] = xplane[addr];
            addr += a.stride;
            if (++s == a.Wo) { s = 0; ++r; addr += row_step; }
        }
        rb.pack(xv);
    };
    f32x16_t acc[2] = {};
    load(0);
    for (int p0 = 0; p0 < a.P; p0 += 32) {
        __syncthreads();  // the previous chunk's fragment reads are done
        ra[0].store(s_a + row * PITCH + 8 * seg);
        ra[1].store(s_a + (row + 64) * PITCH + 8 * seg);
        rb.store(s_b + row * PITCH + 8 * seg);
        __syncthreads();
        if (p0 + 32 < a.P) load(p0 + 32);
        const T *pb = s_b + (32 * nh + l32) * PITCH;
        const T *pa0 = s_a + (64 * mq + l32) * PITCH;
        const T *pa1 = pa0 + 32 * PITCH;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int off = 16 * ks + 8 * lh;
                const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(pb + off));
                const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(pa0 + off));
                const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(pa1 + off));
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bf, acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bf, acc[1], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                const float bf = pb[2 * ks + lh];
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(pa0[2 * ks + lh], bf, acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(pa1[2 * ks + lh], bf, acc[1], 0, 0, 0);
            }
        }
    }
    // D(lane, 4j + q) = row 8j + 4 lh + q, column l32 of a 32 x 32 block
    const int KK = K0 + 32 * nh + l32;
    if (KK >= a.Kdim) return;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int oo = o0 + 64 * mq + 32 * mb + 8 * j + 4 * lh + q;
                if (oo < a.Cout) dw[((long)b * a.Cout + oo) * a.Kdim + KK] = acc[mb][4 * j + q];
            }
}

// ---- kernel gradient per example, depthwise --------------------------------
// Workgroup (c, b): dW_b[c][u][v] = sum_{r,s} dy[b,c,r,s] * x[b,c, r*st-pad+u, s*st-pad+v].
// The example's input plane, with its zero border, and its dy plane are
// staged in LDS as float32 (tile row i, column j <-> x row i - pad, column
// j - pad). Thread (u, g) owns kernel row u and output rows g, g + G, ...
// (G = 256 / K row groups): along each output row it slides a K-wide window
// of the tile row r*st + u, so every multiply-add reads at most one new x
// value, and keeps the K sums of kernel row u in registers. The G partial
// sums of each tap are then added in LDS in a fixed order.
template <typename T, int K>
__global__ __launch_bounds__(256) void wgrad_dw_kernel(const T *__restrict__ x, const T *__restrict__ dy,
                                                       float *__restrict__ dw, WgArgs a, int Hp, int Wp) {
    constexpr int KK = K * K;
    constexpr int G = 256 / K;
    extern __shared__ float s_dyn[];
    float *s_x = s_dyn;                 // Hp * Wp
    float *s_d = s_dyn + Hp * Wp;       // P
    __shared__ float s_part[G * KK];
    const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const T *xp = x + ((long)b * a.Cin + c) * a.H * a.W;
    const T *dp = dy + ((long)b * a.Cin + c) * a.P;
    for (int i = tid; i < Hp * Wp; i += 256) {
        const int ii = i / Wp;
        const int hh = ii - a.pad, ww = i - ii * Wp - a.pad;
        s_x[i] = (hh >= 0 && hh < a.H && ww >= 0 && ww < a.W) ? Elem<T>::to_f32(xp[(long)hh * a.W + ww]) : 0.f;
    }
    for (int i = tid; i < a.P; i += 256) s_d[i] = Elem<T>::to_f32(dp[i]);
    __syncthreads();
    const int u = tid % K, g = tid / K;
    float part[K];
#pragma unroll
    for (int v = 0; v < K; ++v) part[v] = 0.f;
    if (g < G) {
        for (int r = g; r < a.Ho; r += G) {
            const float *xr = s_x + (r * a.stride + u) * Wp;
            const float *dr = s_d + r * a.Wo;
            if (a.stride == 1) {
                float w[K];
#pragma unroll
                for (int v = 0; v < K - 1; ++v) w[v] = xr[v];
                for (int s = 0; s < a.Wo; ++s) {
                    w[K - 1] = xr[s + K - 1];
                    const float d = dr[s];
#pragma unroll
                    for (int v = 0; v < K; ++v) part[v] += d * w[v];
#pragma unroll
                    for (int v = 0; v < K - 1; ++v) w[v] = w[v + 1];
                }
            } else {
                for (int s = 0; s < a.Wo; ++s) {
                    const float d = dr[s];
                    const float *xs = xr + s * a.stride;
#pragma unroll
                    for (int v = 0; v < K; ++v) part[v] += d * xs[v];
                }
            }
        }
#pragma unroll
        for (int v = 0; v < K; ++v) s_part[g * KK + u * K + v] = part[v];
    }
    __syncthreads();
    if (tid < KK) {
        float sum = 0.f;
        for (int j = 0; j < G; ++j) sum += s_part[j * KK + tid];
        dw[((long)b * a.Cin + c) * KK + tid] = sum;
    }
}

// Any other depthwise kernel size (up to 64 taps), bounds-checked global reads.
constexpr int kDwTaps = 64;
template <typename T>
__global__ __launch_bounds__(256) void wgrad_dw_any_kernel(const T *__restrict__ x, const T *__restrict__ dy,
                                                           float *__restrict__ dw, WgArgs a) {
    __shared__ float s_red[4][kDwTaps];
    const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const T *xp = x + ((long)b * a.Cin + c) * a.H * a.W;
    const T *dp = dy + ((long)b * a.Cin + c) * a.P;
    const int wave = tid >> 6, lane = tid & 63;
    for (int t = 0; t < a.KT; ++t) {
        const int u = t / a.KW, v = t - u * a.KW;
        float part = 0.f;
        for (int p = tid; p < a.P; p += 256) {
            const int r = p / a.Wo, s = p - r * a.Wo;
            const int hh = r * a.stride - a.pad + u, ww = s * a.stride - a.pad + v;
            if (hh >= 0 && hh < a.H && ww >= 0 && ww < a.W)
                part += Elem<T>::to_f32(dp[p]) * Elem<T>::to_f32(xp[(long)hh * a.W + ww]);
        }
        part = wave_sum(part);
        if (lane == 0) s_red[wave][t] = part;
    }
    __syncthreads();
    if (tid < a.KT)
        dw[((long)b * a.Cin + c) * a.KT + tid] = (s_red[0][tid] + s_red[1][tid]) + (s_red[2][tid] + s_red[3][tid]);
}

// ---- contraction of dW_b into dalpha and dE ---------------------------------------
// One pass over dW_b [B][wsize] for NE experts i0 .. i0 + NE - 1. Workgroup
// (ch, bg) owns elements ch * 256 * VEC .. (VEC per thread) and the examples
// bg * bpg .. + bpg - 1:
//   dEp[bg][i][e]   = sum_{b in group} alpha[b][i] * dW_b[e]
//   dpart[b][i][ch] = sum_{e in chunk} dW_b[e] * E_i[e]
// With one example group dEp is dE itself; otherwise dE_reduce_kernel adds
// the groups, and dalpha_reduce_kernel adds the chunks of dpart. The
// workgroup's slice of the bank stays in registers; dW_b rows are loaded
// kCtU examples ahead.
constexpr int kCtB = 16;  // examples per LDS round of partial sums
constexpr int kCtU = 4;   // examples whose dW_b rows are in flight together
template <typename T, int NE, int VEC>
__global__ __launch_bounds__(256) void contract_kernel(const float *__restrict__ dw, const T *__restrict__ ex,
                                                       const float *__restrict__ alpha, float *__restrict__ dep,
                                                       float *__restrict__ dpart, long wsize, int B, int bpg, int n,
                                                       int i0, int nch) {
    __shared__ float s_red[4][kCtB][NE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const long e0 = ((long)blockIdx.x * 256 + tid) * VEC;
    const bool in = e0 < wsize;  // VEC == 4 only when wsize % 4 == 0
    const int bbeg = blockIdx.y * bpg, bend = min(B, bbeg + bpg);
    float ev[NE][VEC], acc[NE][VEC];
#pragma unroll
    for (int k = 0; k < NE; ++k)
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            ev[k][j] = (in && i0 + k < n) ? Elem<T>::to_f32(ex[(long)(i0 + k) * wsize + e0 + j]) : 0.f;
            acc[k][j] = 0.f;
        }
    for (int b0 = bbeg; b0 < bend; b0 += kCtB) {
        const int nb = min(kCtB, bend - b0);
        for (int u0 = 0; u0 < nb; u0 += kCtU) {
            float d[kCtU][VEC];
#pragma unroll
            for (int uu = 0; uu < kCtU; ++uu) {
                const int b = b0 + u0 + uu;
                const bool ok = in && u0 + uu < nb;
                if constexpr (VEC == 4) {
                    const f32x4_t v = ok ? *reinterpret_cast<const f32x4_t *>(dw + (long)b * wsize + e0)
                                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
                    d[uu][0] = v[0]; d[uu][1] = v[1]; d[uu][2] = v[2]; d[uu][3] = v[3];
                } else {
                    d[uu][0] = ok ? dw[(long)b * wsize + e0] : 0.f;
                }
            }
#pragma unroll
            for (int uu = 0; uu < kCtU; ++uu) {
                if (u0 + uu >= nb) break;
                const int b = b0 + u0 + uu;
                float part[NE];
#pragma unroll
                for (int k = 0; k < NE; ++k) {
                    const float al = i0 + k < n ? alpha[(long)b * n + i0 + k] : 0.f;
                    part[k] = 0.f;
#pragma unroll
                    for (int j = 0; j < VEC; ++j) {
                        acc[k][j] += al * d[uu][j];
                        part[k] += d[uu][j] * ev[k][j];
                    }
                }
                // transpose-reduce: each halving step swaps half of the
                // partials with the partner lane (xor m) and adds, so after
                // log2(NE) steps lane L holds the partial of expert
                // bitrev(L mod NE); xor steps over the other lane bits finish
                // the sums in lanes 0 .. NE - 1 (fixed order: deterministic)
#pragma unroll
                for (int h = NE / 2, m = 1; h >= 1; h >>= 1, m <<= 1) {
                    const bool up = (lane & m) != 0;
#pragma unroll
                    for (int j = 0; j < h; ++j) {
                        const float send = up ? part[j] : part[j + h];
                        const float keep = up ? part[j + h] : part[j];
                        part[j] = keep + __shfl_xor(send, m, 64);
                    }
                }
#pragma unroll
                for (int m = NE; m < 64; m <<= 1) part[0] += __shfl_xor(part[0], m, 64);
                if (lane < NE) {
                    int k = 0;
#pragma unroll
                    for (int bit = 1, val = NE / 2; bit < NE; bit <<= 1, val >>= 1)
                        if (lane & bit) k += val;
                    s_red[wave][u0 + uu][k] = part[0];
                }
            }
        }
        __syncthreads();
        if (tid < nb * NE) {
            const int bb = tid / NE, k = tid - bb * NE;
            if (i0 + k < n)
                dpart[((long)(b0 + bb) * n + i0 + k) * nch + blockIdx.x] =
                    (s_red[0][bb][k] + s_red[1][bb][k]) + (s_red[2][bb][k] + s_red[3][bb][k]);
        }
        __syncthreads();
    }
    if (!in || dep == nullptr) return;
    float *out = dep + (long)blockIdx.y * n * wsize;
#pragma unroll
    for (int k = 0; k < NE; ++k)
        if (i0 + k < n)
#pragma unroll
            for (int j = 0; j < VEC; ++j) out[(long)(i0 + k) * wsize + e0 + j] = acc[k][j];
}

// dE[j] = sum over example groups of dEp[g][j] (j over n * wsize), in group order.
__global__ __launch_bounds__(256) void dE_reduce_kernel(const float *__restrict__ dep, float *__restrict__ de,
                                                        long total, int groups) {
    const long j = (long)blockIdx.x * 256 + threadIdx.x;
    if (j >= total) return;
    float s = 0.f;
    for (int g = 0; g < groups; ++g) s += dep[(long)g * total + j];
    de[j] = s;
}

// dalpha[b][i] = sum over chunks of dpart[b * rows + i][ch] (rows >= n
// expert rows per example): one wave per (b, i); lane l adds chunks l,
// l + 64, ... into four partial sums (chunk l + 64 m goes to sum m % 4) in
// order, then adds them and a fixed-tree wave sum.
__global__ __launch_bounds__(256) void dalpha_reduce_kernel(const float *__restrict__ dpart,
                                                            float *__restrict__ dalpha, int total, int nch, int n,
                                                            int rows) {
    const int idx = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (idx >= total) return;
    const int b = idx / n, i = idx - b * n;
    const float *p = dpart + ((long)b * rows + i) * nch;
    // four independent partial sums (their loads in flight together), fixed order
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    int c = lane;
    for (; c + 192 < nch; c += 256) {
        s0 += p[c];
        s1 += p[c + 64];
        s2 += p[c + 128];
        s3 += p[c + 192];
    }
    for (; c < nch; c += 64) s0 += p[c];
    float s = wave_sum((s0 + s1) + (s2 + s3));
    if (lane == 0) dalpha[idx] = s;
}

// ---- gradients of FMDConv's channel attentions -------------------------------
// With G = dW_b formed from x and dy alone (launch_wgrad_gemm) and
// y = a_out * conv(a_in * x, W_b) (FMDConv: Fast multi-attention dynamic
// convolution, abstract):
//   H[b][o][c]   = sum_t G[b][o][c][t] * W_b[o][c][t]
//   da_out[b,o]  = sum_c a_in[b, g(o) cpg + c] * H[b][o][c]
//   da_in[b,gc]  = sum over o of gc's group of a_out[b,o] * H[b][o][c]
//   dW'_b        = a_out[b,o] * a_in[b,gc] * G   (then the usual contraction)
// W_b is mixed on the fly in float32 (experts in order), so no rounding of the
// mixed kernels enters these gradients. Every sum runs in a fixed order.

// one thread per (b, o, c)
template <typename T>
__global__ __launch_bounds__(256) void attn_h_kernel(const float *__restrict__ G, const T *__restrict__ ex,
                                                     const float *__restrict__ alpha, float *__restrict__ H,
                                                     long total, int Cout, int cpg, int KT, int n, long wsize) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const long per_b = (long)Cout * cpg;
    const int b = (int)(idx / per_b);
    const long oc = idx - (long)b * per_b;  // o * cpg + c
    const long e0 = oc * KT;
    const float *al = alpha + (long)b * n;
    const float *g = G + (long)b * wsize + e0;
    float h = 0.f;
    for (int t = 0; t < KT; ++t) {
        float w = 0.f;
        for (int i = 0; i < n; ++i) w = fmaf(al[i], Elem<T>::to_f32(ex[(long)i * wsize + e0 + t]), w);
        h = fmaf(g[t], w, h);
    }
    H[idx] = h;
}

// one thread per (b, o); a_in may be null (ones)
__global__ __launch_bounds__(256) void attn_dout_kernel(const float *__restrict__ H, const float *__restrict__ a_in,
                                                        float *__restrict__ da_out, int B, int Cin, int Cout, int cpg,
                                                        int opg) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)B * Cout) return;
    const int b = (int)(idx / Cout), o = (int)(idx - (long)b * Cout);
    const int c0 = (o / opg) * cpg;
    const float *h = H + idx * cpg;
    float s = 0.f;
    for (int c = 0; c < cpg; ++c) s = fmaf(a_in ? a_in[(long)b * Cin + c0 + c] : 1.f, h[c], s);
    da_out[idx] = s;
}

// one thread per (b, gc); a_out may be null (ones)
__global__ __launch_bounds__(256) void attn_din_kernel(const float *__restrict__ H, const float *__restrict__ a_out,
                                                       float *__restrict__ da_in, int B, int Cin, int Cout, int cpg,
                                                       int opg) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)B * Cin) return;
    const int b = (int)(idx / Cin), gc = (int)(idx - (long)b * Cin);
    const int grp = gc / cpg, c = gc - grp * cpg;
    float s = 0.f;
    for (int o = grp * opg; o < (grp + 1) * opg; ++o)
        s = fmaf(a_out ? a_out[(long)b * Cout + o] : 1.f, H[((long)b * Cout + o) * cpg + c], s);
    da_in[idx] = s;
}

// G[b][e] *= a_out[b,o] * a_in[b,gc] (either may be null: ones)
__global__ __launch_bounds__(256) void attn_scale_kernel(float *__restrict__ G, const float *__restrict__ a_in,
                                                         const float *__restrict__ a_out, long total, long wsize,
                                                         int Cin, int Cout, int cpg, int opg, int KT) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int b = (int)(idx / wsize);
    const long e = idx - (long)b * wsize;
    const int o = (int)(e / ((long)cpg * KT)), c = (int)((e / KT) % cpg);
    const float fo = a_out ? a_out[(long)b * Cout + o] : 1.f;
    const float fi = a_in ? a_in[(long)b * Cin + (o / opg) * cpg + c] : 1.f;
    G[idx] *= fo * fi;
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

// dfc_w[i][c] = sum_b dz[b][i] gap[b][c] and dfc_b[i] = sum_b dz[b][i].
// Workgroup (i, 32-channel chunk): thread (c, g) sums the examples
// g, g + 8, ... of channel c; the 8 partial sums are added in LDS in group order.
__global__ __launch_bounds__(256) void route_dfc_kernel(const float *__restrict__ dz, const float *__restrict__ gap,
                                                        float *__restrict__ dfc_w, float *__restrict__ dfc_b,
                                                        int B, int n, int C) {
    __shared__ float s_w[8][32];
    __shared__ float s_b[8][32];
    const int i = blockIdx.x, cl = threadIdx.x & 31, gr = threadIdx.x >> 5;
    const int c = blockIdx.y * 32 + cl;
    float acc = 0.f, accb = 0.f;
    if (c < C) {
#pragma unroll 4
        for (int b = gr; b < B; b += 8) {
            const float z = dz[(long)b * n + i];
            acc += z * gap[(long)b * C + c];
            accb += z;
        }
    }
    s_w[gr][cl] = acc;
    s_b[gr][cl] = accb;
    __syncthreads();
    if (gr == 0 && c < C) {
        float w = 0.f, wb = 0.f;
        for (int k = 0; k < 8; ++k) {
            w += s_w[k][cl];
            wb += s_b[k][cl];
        }
        dfc_w[(long)i * C + c] = w;
        if (c == 0 && dfc_b) dfc_b[i] = wb;
    }
}

// dx[b][c][h][w] += dgap[b][c] / (H W): the pooling's share of the input
// gradient, added in float32 and rounded once to the element type. VEC
// consecutive elements per thread (VEC divides H W, so they share a plane).
template <typename T, int VEC>
__global__ __launch_bounds__(256) void add_pool_grad_kernel(T *__restrict__ dx, const float *__restrict__ dgap,
                                                            long total, int hw, float inv_hw) {
    const long idx = ((long)blockIdx.x * 256 + threadIdx.x) * VEC;
    if (idx >= total) return;
    const float add = dgap[idx / hw] * inv_hw;
#pragma unroll
    for (int j = 0; j < VEC; ++j) dx[idx + j] = Elem<T>::from_f32(Elem<T>::to_f32(dx[idx + j]) + add);
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

namespace {
long bank_elems(const Geom &g) { return (long)g.Cout * g.cpg * g.KT; }
int contract_vec(const Geom &g) { return bank_elems(g) % 4 == 0 ? 4 : 1; }
int contract_chunks(const Geom &g) { return (int)((bank_elems(g) + 256L * contract_vec(g) - 1) / (256L * contract_vec(g))); }
// Examples per contraction workgroup: enough example groups that the grid
// has about 1024 workgroups, with at least 8 examples per group.
int contract_bpg(const Geom &g) {
    const int want = std::max(1, std::min(ceil_div(1024, contract_chunks(g)), ceil_div(g.B, 8)));
    return ceil_div(g.B, want);
}
int contract_groups(const Geom &g) { return ceil_div(g.B, contract_bpg(g)); }
size_t align256(size_t v) { return (v + 255) / 256 * 256; }
size_t dwb_bytes(const Geom &g) { return align256((size_t)g.B * bank_elems(g) * sizeof(float)); }
size_t dpart_bytes(const Geom &g) { return align256((size_t)g.B * g.n * contract_chunks(g) * sizeof(float)); }
size_t dep_bytes(const Geom &g) {
    return contract_groups(g) > 1 ? align256((size_t)contract_groups(g) * g.n * bank_elems(g) * sizeof(float)) : 0;
}
bool dw_lds_plane(const Geom &g, int &Hp, int &Wp) {
    if (g.KH != g.KW || (g.KH != 3 && g.KH != 5)) return false;
    Hp = (g.Ho - 1) * g.stride + g.KH;
    Wp = (g.Wo - 1) * g.stride + g.KW;
    return ((long)Hp * Wp + g.P) * 4 <= 64 * 1024;
}

template <typename T, int NE>
hipError_t launch_contract_t(const Geom &g, const float *dwb, const void *experts, const float *alpha, float *dep,
                             float *dpart, int i0, hipStream_t stream) {
    const long wsize = bank_elems(g);
    const int nch = contract_chunks(g);
    const dim3 grid((unsigned)nch, (unsigned)contract_groups(g));
    if (contract_vec(g) == 4)
        hipLaunchKernelGGL((contract_kernel<T, NE, 4>), grid, dim3(256), 0, stream, dwb,
                           static_cast<const T *>(experts), alpha, dep, dpart, wsize, g.B, contract_bpg(g), g.n, i0,
                           nch);
    else
        hipLaunchKernelGGL((contract_kernel<T, NE, 1>), grid, dim3(256), 0, stream, dwb,
                           static_cast<const T *>(experts), alpha, dep, dpart, wsize, g.B, contract_bpg(g), g.n, i0,
                           nch);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_contract(const Geom &g, const float *dwb, const void *experts, const float *alpha, float *dep,
                           float *dpart, hipStream_t stream) {
    for (int i0 = 0; i0 < g.n; i0 += 8) {
        const int left = g.n - i0;
        hipError_t e;
        if (left >= 5) e = launch_contract_t<T, 8>(g, dwb, experts, alpha, dep, dpart, i0, stream);
        else if (left >= 3) e = launch_contract_t<T, 4>(g, dwb, experts, alpha, dep, dpart, i0, stream);
        else if (left == 2) e = launch_contract_t<T, 2>(g, dwb, experts, alpha, dep, dpart, i0, stream);
        else e = launch_contract_t<T, 1>(g, dwb, experts, alpha, dep, dpart, i0, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}
}  // namespace

size_t wgrad_bytes(const Geom &g) {
    if (const size_t f = wgrad_fused_bytes(g)) return f;
    return dwb_bytes(g) + dpart_bytes(g) + dep_bytes(g);
}

bool wgrad_dw_supported(const Geom &g) { return g.KT <= kDwTaps; }

namespace {
// dW_b of every example into dwb (float32, [B][Cout][Cin/g][KH][KW]).
hipError_t launch_wgrad_gemm(const Geom &g, const void *x, const void *dy, float *dwb, hipStream_t stream) {
    WgArgs a;
    a.B = g.B; a.Cin = g.Cin; a.H = g.H; a.W = g.W; a.Cout = g.Cout; a.KW = g.KW;
    a.stride = g.stride; a.pad = g.pad; a.Ho = g.Ho; a.Wo = g.Wo; a.P = g.P; a.KT = g.KT;
    a.Kdim = g.cpg * g.KT;
    a.n_ktiles = ceil_div(a.Kdim, 64);
    a.dy_vec = g.P % 4 == 0;
    if (g.groups == 1) {
        const dim3 grid((unsigned)(ceil_div(g.Cout, 128) * a.n_ktiles), (unsigned)g.B);
        if (g.bf16)
            hipLaunchKernelGGL(wgrad_kernel<uint16_t>, grid, dim3(256), 0, stream,
                               static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(dy), dwb, a);
        else
            hipLaunchKernelGGL(wgrad_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float *>(x),
                               static_cast<const float *>(dy), dwb, a);
    } else {
        const dim3 grid((unsigned)g.Cin, (unsigned)g.B);
        int Hp = 0, Wp = 0;
        if (dw_lds_plane(g, Hp, Wp)) {
            const size_t lds = ((size_t)Hp * Wp + g.P) * sizeof(float);
            if (g.bf16 && g.KH == 3)
                hipLaunchKernelGGL((wgrad_dw_kernel<uint16_t, 3>), grid, dim3(256), lds, stream,
                                   static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(dy), dwb, a, Hp, Wp);
            else if (g.bf16)
                hipLaunchKernelGGL((wgrad_dw_kernel<uint16_t, 5>), grid, dim3(256), lds, stream,
                                   static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(dy), dwb, a, Hp, Wp);
            else if (g.KH == 3)
                hipLaunchKernelGGL((wgrad_dw_kernel<float, 3>), grid, dim3(256), lds, stream,
                                   static_cast<const float *>(x), static_cast<const float *>(dy), dwb, a, Hp, Wp);
            else
                hipLaunchKernelGGL((wgrad_dw_kernel<float, 5>), grid, dim3(256), lds, stream,
                                   static_cast<const float *>(x), static_cast<const float *>(dy), dwb, a, Hp, Wp);
        } else if (g.bf16) {
            hipLaunchKernelGGL(wgrad_dw_any_kernel<uint16_t>, grid, dim3(256), 0, stream,
                               static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(dy), dwb, a);
        } else {
            hipLaunchKernelGGL(wgrad_dw_any_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float *>(x),
                               static_cast<const float *>(dy), dwb, a);
        }
    }
    return hipGetLastError();
}

// dalpha and dexperts from dW_b in dwb; the partial sums follow dW_b in the
// scratch: dW_b | dalpha partial sums | dE per example group.
hipError_t launch_contract_all(const Geom &g, float *dwb, const void *experts, const float *alpha, float *dalpha,
                               float *dexperts, hipStream_t stream) {
    hipError_t e;
    char *base = reinterpret_cast<char *>(dwb);
    float *dpart = reinterpret_cast<float *>(base + dwb_bytes(g));
    const int groups = contract_groups(g);
    float *dep = groups > 1 ? reinterpret_cast<float *>(base + dwb_bytes(g) + dpart_bytes(g)) : dexperts;
    if (!dexperts) dep = nullptr;
    e = g.bf16 ? launch_contract<uint16_t>(g, dwb, experts, alpha, dep, dpart, stream)
               : launch_contract<float>(g, dwb, experts, alpha, dep, dpart, stream);
    if (e != hipSuccess) return e;
    if (dexperts && groups > 1) {
        e = launch_dE_reduce(dep, dexperts, (long)g.n * bank_elems(g), groups, stream);
        if (e != hipSuccess) return e;
    }
    if (!dalpha) return hipSuccess;
    return launch_dalpha_reduce(dpart, dalpha, g.B, g.n, g.n, contract_chunks(g), stream);
}
}  // namespace

hipError_t launch_backward_weights(const Geom &g, const void *x, const void *dy, const void *experts,
                                   const float *alpha, float *dwb, float *dalpha, float *dexperts,
                                   hipStream_t stream) {
    if (wgrad_fused_bytes(g)) return launch_wgrad_fused(g, x, dy, experts, alpha, dwb, dalpha, dexperts, stream);
    hipError_t e = launch_wgrad_gemm(g, x, dy, dwb, stream);
    if (e != hipSuccess) return e;
    return launch_contract_all(g, dwb, experts, alpha, dalpha, dexperts, stream);
}

size_t wgrad_attn_bytes(const Geom &g) {
    return dwb_bytes(g) + dpart_bytes(g) + dep_bytes(g) + align256((size_t)g.B * g.Cout * g.cpg * sizeof(float));
}

hipError_t launch_backward_weights_attn(const Geom &g, const void *x, const void *dy, const void *experts,
                                        const float *alpha, ChanAttn att, float *ws, float *dalpha,
                                        float *dexperts, float *da_in, float *da_out, hipStream_t stream) {
    // scratch: dW_b | dalpha partial sums | dE per example group | H
    hipError_t e = launch_wgrad_gemm(g, x, dy, ws, stream);
    if (e != hipSuccess) return e;
    const long wsize = bank_elems(g);
    const int opg = g.Cout / g.groups;
    if (da_in || da_out) {
        float *h = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + dwb_bytes(g) + dpart_bytes(g) +
                                             dep_bytes(g));
        const long nh = (long)g.B * g.Cout * g.cpg;
        if (g.bf16)
            hipLaunchKernelGGL(attn_h_kernel<uint16_t>, dim3(blocks_for(nh)), dim3(256), 0, stream, ws,
                               static_cast<const uint16_t *>(experts), alpha, h, nh, g.Cout, g.cpg, g.KT, g.n, wsize);
        else
            hipLaunchKernelGGL(attn_h_kernel<float>, dim3(blocks_for(nh)), dim3(256), 0, stream, ws,
                               static_cast<const float *>(experts), alpha, h, nh, g.Cout, g.cpg, g.KT, g.n, wsize);
        if (da_out)
            hipLaunchKernelGGL(attn_dout_kernel, dim3(blocks_for((long)g.B * g.Cout)), dim3(256), 0, stream, h,
                               att.in, da_out, g.B, g.Cin, g.Cout, g.cpg, opg);
        if (da_in)
            hipLaunchKernelGGL(attn_din_kernel, dim3(blocks_for((long)g.B * g.Cin)), dim3(256), 0, stream, h,
                               att.out, da_in, g.B, g.Cin, g.Cout, g.cpg, opg);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!dalpha && !dexperts) return hipSuccess;
    if (att.in || att.out) {
        const long total = (long)g.B * wsize;
        hipLaunchKernelGGL(attn_scale_kernel, dim3(blocks_for(total)), dim3(256), 0, stream, ws, att.in, att.out,
                           total, wsize, g.Cin, g.Cout, g.cpg, opg, g.KT);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_contract_all(g, ws, experts, alpha, dalpha, dexperts, stream);
}

hipError_t launch_dE_reduce(const float *dep, float *de, long total, int groups, hipStream_t stream) {
    hipLaunchKernelGGL(dE_reduce_kernel, dim3(blocks_for(total)), dim3(256), 0, stream, dep, de, total, groups);
    return hipGetLastError();
}

hipError_t launch_dalpha_reduce(const float *dpart, float *dalpha, int B, int n, int rows, int nch,
                                hipStream_t stream) {
    const int total = B * n;
    hipLaunchKernelGGL(dalpha_reduce_kernel, dim3((unsigned)ceil_div(total, 4)), dim3(256), 0, stream, dpart, dalpha,
                       total, nch, n, rows);
    return hipGetLastError();
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
    hipLaunchKernelGGL(route_dfc_kernel, dim3((unsigned)g.n, (unsigned)ceil_div(g.Cin, 32)), dim3(256), 0, stream,
                       dz, gap, dfc_w, dfc_b, g.B, g.n, g.Cin);
    e = hipGetLastError();
    if (e != hipSuccess || !dx) return e;
    const long total = (long)g.B * g.Cin * g.H * g.W;
    const int hw = g.H * g.W;
    const float inv = 1.f / (float)hw;
    if (hw % 8 == 0) {
        const unsigned nb = blocks_for(total / 8);
        if (g.bf16)
            hipLaunchKernelGGL((add_pool_grad_kernel<uint16_t, 8>), dim3(nb), dim3(256), 0, stream,
                               static_cast<uint16_t *>(dx), dgap, total, hw, inv);
        else
            hipLaunchKernelGGL((add_pool_grad_kernel<float, 8>), dim3(nb), dim3(256), 0, stream,
                               static_cast<float *>(dx), dgap, total, hw, inv);
    } else if (hw % 4 == 0) {
        const unsigned nb = blocks_for(total / 4);
        if (g.bf16)
            hipLaunchKernelGGL((add_pool_grad_kernel<uint16_t, 4>), dim3(nb), dim3(256), 0, stream,
                               static_cast<uint16_t *>(dx), dgap, total, hw, inv);
        else
            hipLaunchKernelGGL((add_pool_grad_kernel<float, 4>), dim3(nb), dim3(256), 0, stream,
                               static_cast<float *>(dx), dgap, total, hw, inv);
    } else if (g.bf16) {
        hipLaunchKernelGGL((add_pool_grad_kernel<uint16_t, 1>), dim3(blocks_for(total)), dim3(256), 0, stream,
                           static_cast<uint16_t *>(dx), dgap, total, hw, inv);
    } else {
        hipLaunchKernelGGL((add_pool_grad_kernel<float, 1>), dim3(blocks_for(total)), dim3(256), 0, stream,
                           static_cast<float *>(dx), dgap, total, hw, inv);
    }
    return hipGetLastError();
}

namespace {

// Input gradient for the layers the forward machinery does not transpose
// (stride above 1, kh != kw, or padding of k or more): dx[b,c,h,w] is the sum
// of W_b[o,c',u,v] * dy[b,o,r,s] over the output positions (r, s) and taps
// (u, v) with r * stride + u - pad = h and s * stride + v - pad = w, o over
// the output channels of c's group (c' = c within its group). W_b is mixed
// into the workspace first (the layer's element type, one rounding, as the
// forward uses it); products accumulate in fp32 and dx is rounded once. One
// thread per dx element, positions fastest, so a wave reads one W_b row per
// (o, u, v) (a broadcast) and neighbouring dy elements.
struct DgradArgs {
    int B, Cin, H, W, Cout, KH, KW, stride, pad, groups, Ho, Wo;
};
template <typename T>
__global__ __launch_bounds__(256) void dgrad_direct_kernel(const T *__restrict__ dy, const T *__restrict__ wb,
                                                           T *__restrict__ dx, DgradArgs a) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const long total = (long)a.B * a.Cin * a.H * a.W;
    if (idx >= total) return;
    const int w = (int)(idx % a.W);
    long t = idx / a.W;
    const int h = (int)(t % a.H);
    t /= a.H;
    const int c = (int)(t % a.Cin);
    const int b = (int)(t / a.Cin);
    const int cpg_in = a.Cin / a.groups, cpg_out = a.Cout / a.groups;
    const int grp = c / cpg_in, ci = c - grp * cpg_in;
    float acc = 0.f;
    for (int oo = 0; oo < cpg_out; ++oo) {
        const int o = grp * cpg_out + oo;
        const T *wp = wb + (((long)b * a.Cout + o) * cpg_in + ci) * a.KH * a.KW;
        const T *dp = dy + ((long)b * a.Cout + o) * a.Ho * a.Wo;
        for (int u = 0; u < a.KH; ++u) {
            const int th = h + a.pad - u;
            if (th < 0 || th % a.stride != 0) continue;
            const int r = th / a.stride;
            if (r >= a.Ho) continue;
            for (int v = 0; v < a.KW; ++v) {
                const int tw = w + a.pad - v;
                if (tw < 0 || tw % a.stride != 0) continue;
                const int s = tw / a.stride;
                if (s >= a.Wo) continue;
                acc = fmaf(Elem<T>::to_f32(wp[u * a.KW + v]), Elem<T>::to_f32(dp[(long)r * a.Wo + s]), acc);
            }
        }
    }
    dx[idx] = Elem<T>::from_f32(acc);
}

}  // namespace

hipError_t launch_dgrad_direct(const Geom &g, const void *dy, const void *wb, void *dx, hipStream_t stream) {
    DgradArgs a{g.B, g.Cin, g.H, g.W, g.Cout, g.KH, g.KW, g.stride, g.pad, g.groups, g.Ho, g.Wo};
    const long total = (long)g.B * g.Cin * g.H * g.W;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (g.bf16)
        hipLaunchKernelGGL(dgrad_direct_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t *>(dy), static_cast<const uint16_t *>(wb),
                           static_cast<uint16_t *>(dx), a);
    else
        hipLaunchKernelGGL(dgrad_direct_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float *>(dy),
                           static_cast<const float *>(wb), static_cast<float *>(dx), a);
    return hipGetLastError();
}

}  // namespace dynconv
