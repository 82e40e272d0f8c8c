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
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

__global__ __launch_bounds__(256) void conv_direct_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ w, float *__restrict__ y, int B,
    int Cin, int H, int W, int Cout, int KH, int KW, int stride, int pad, int Ho, int Wo,
    const float *__restrict__ a_in, const float *__restrict__ a_out) {
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
        const float si = a_in ? a_in[(long)b * Cin + c] : 1.f;  // input attention
        for (int u = 0; u < KH; ++u) {
            const int h = r * stride - pad + u;
            if (h < 0 || h >= H) continue;
            for (int v = 0; v < KW; ++v) {
                const int ww = s * stride - pad + v;
                if (ww < 0 || ww >= W) continue;
                acc = fmaf(wc[u * KW + v], si * xc[h * W + ww], acc);
            }
        }
    }
    y[idx] = a_out ? a_out[(long)b * Cout + o] * acc : acc;  // output attention
}

constexpr int kDwMaxTaps = 64;
constexpr int kDwStrip = 4;  // outputs per thread along a row

template <typename T>
__global__ __launch_bounds__(256) void depthwise_kernel(
    const T *__restrict__ x, const T *__restrict__ experts, const float *__restrict__ alpha,
    const T *__restrict__ wmixed, T *__restrict__ y, int B, int C, int H, int W, int KH, int KW,
    int stride, int pad, int Ho, int Wo, int n, const float *__restrict__ a_in,
    const float *__restrict__ a_out) {
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
            wv = s;
        }
        // channel attentions of a depthwise plane scale its taps; the tap is
        // held in the storage type, as a materialised kernel would be
        const float sc = (a_in ? a_in[(long)b * C + c] : 1.f) * (a_out ? a_out[(long)b * C + c] : 1.f);
        taps[threadIdx.x] = Elem<T>::to_f32(Elem<T>::from_f32(wv * sc));
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

// Depthwise for square K x K taps (K = 3, 5, 7) and stride ST (1, 2): one
// wave per (example, channel) plane, 4 planes per workgroup.
//   - The zero-padded plane goes to the wave's LDS region as float, row pitch
//     a multiple of 4 floats and wide enough for the last strip's window;
//     16-byte loads when the plane is 16-byte aligned.
//   - Lanes 0..K*K-1 mix the plane's taps (sum_i alpha_bi E_i[c], rounded to
//     the storage type), which every lane then keeps in registers.
//   - A lane computes DW_S consecutive outputs of a row: per kernel row it
//     reads the (DW_S - 1) * ST + K input values once into registers and
//     does DW_S * K multiply-adds from them.
constexpr int kDwS = 8;          // outputs per lane task along a row
constexpr int kDwPlanes = 4;     // planes (waves) per workgroup
constexpr int kDwPlaneFloats = 3840;  // LDS floats per plane at most (4 planes + taps < 64 KB)

__host__ __device__ constexpr int dw_win(int K, int ST) { return (kDwS - 1) * ST + K; }

template <typename T, int K, int ST>
__global__ __launch_bounds__(64 * kDwPlanes) void depthwise_strip_kernel(
    const T *__restrict__ x, const T *__restrict__ experts, const float *__restrict__ alpha,
    const T *__restrict__ wmixed, T *__restrict__ y, int B, int C, int H, int W, int pad, int Ho,
    int Wo, int n, int pitch, const float *__restrict__ a_in, const float *__restrict__ a_out) {
    constexpr int KT = K * K;
    constexpr int WIN = dw_win(K, ST);
    extern __shared__ __attribute__((aligned(16))) float planes[];  // kDwPlanes x plane_floats
    __shared__ float taps_sh[kDwPlanes][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long nplanes = (long)B * C;
    const long bc_raw = (long)blockIdx.x * kDwPlanes + wave;
    const bool valid = bc_raw < nplanes;
    const long bc = valid ? bc_raw : nplanes - 1;
    const int b = (int)(bc / C), c = (int)(bc - (long)b * C);
    const int Hp = (Ho - 1) * ST + K;  // padded rows read
    float *pl = planes + wave * Hp * pitch;  // Hp * pitch is a multiple of 4

    const T *xp = x + bc * H * W;
    const int hw = H * W;
    constexpr int VE = 16 / sizeof(T);  // elements per 16-byte load
    constexpr int kPre = 4;             // 16-byte loads per lane issued before the taps
    const bool vec = (reinterpret_cast<uintptr_t>(xp) & 15) == 0 && hw % VE == 0;
    const int nv = hw / VE;
    u32x4_t pre[kPre];
    if (vec) {
#pragma unroll
        for (int k = 0; k < kPre; ++k) pre[k] = reinterpret_cast<const u32x4_t *>(xp)[min(lane + 64 * k, nv - 1)];
    }
    // taps: expert values and attentions load 8 at a time (clamped indices,
    // no branches), so their latencies overlap with each other and the plane's
    if (lane < KT) {
        float wv;
        if (wmixed) {
            wv = Elem<T>::to_f32(wmixed[bc * KT + lane]);
        } else {
            float sm = 0.f;
            for (int i0 = 0; i0 < n; i0 += 8) {
                float ev[8], av[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = min(i0 + k, n - 1);
                    ev[k] = Elem<T>::to_f32(experts[((long)i * C + c) * KT + lane]);
                    av[k] = alpha[(long)b * n + i];
                }
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (i0 + k < n) sm = fmaf(av[k], ev[k], sm);
            }
            wv = sm;
        }
        // channel attentions of a depthwise plane scale its taps; the tap is
        // held in the storage type, as a materialised kernel would be
        const float sc = (a_in ? a_in[(long)b * C + c] : 1.f) * (a_out ? a_out[(long)b * C + c] : 1.f);
        taps_sh[wave][lane] = Elem<T>::to_f32(Elem<T>::from_f32(wv * sc));
    }
    // zero the padded plane, then the interior
    for (int i = lane; i < Hp * pitch; i += 64) pl[i] = 0.f;
    auto put = [&](int v, const u32x4_t &q) {
        float f[VE];
        if constexpr (sizeof(T) == 2) {
            f[0] = bf16_lo(q.x); f[1] = bf16_hi(q.x); f[2] = bf16_lo(q.y); f[3] = bf16_hi(q.y);
            f[4] = bf16_lo(q.z); f[5] = bf16_hi(q.z); f[6] = bf16_lo(q.w); f[7] = bf16_hi(q.w);
        } else {
            f[0] = __uint_as_float(q.x); f[1] = __uint_as_float(q.y);
            f[2] = __uint_as_float(q.z); f[3] = __uint_as_float(q.w);
        }
        int h = (v * VE) / W, w = v * VE - h * W;
#pragma unroll
        for (int j = 0; j < VE; ++j) {
            if (h + pad < Hp) pl[(h + pad) * pitch + w + pad] = f[j];
            if (++w == W) { w = 0; ++h; }
        }
    };
    if (vec) {
#pragma unroll
        for (int k = 0; k < kPre; ++k)
            if (lane + 64 * k < nv) put(lane + 64 * k, pre[k]);
        for (int v = lane + 64 * kPre; v < nv; v += 64) put(v, reinterpret_cast<const u32x4_t *>(xp)[v]);
    } else {
        for (int i = lane; i < hw; i += 64) {
            const int h = i / W, w = i - h * W;
            if (h + pad < Hp) pl[(h + pad) * pitch + w + pad] = Elem<T>::to_f32(xp[i]);
        }
    }
    __syncthreads();
    float tap[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) tap[t] = taps_sh[wave][t];

    const int strips = (Wo + kDwS - 1) / kDwS;
    T *yp = y + bc * Ho * Wo;
    for (int task = lane; task < Ho * strips; task += 64) {
        const int r = task / strips;
        const int s0 = (task - r * strips) * kDwS;
        float acc[kDwS];
#pragma unroll
        for (int j = 0; j < kDwS; ++j) acc[j] = 0.f;
#pragma unroll
        for (int u = 0; u < K; ++u) {
            const float *row = pl + (r * ST + u) * pitch + s0 * ST;
            float win[WIN];
            if constexpr (ST == 1) {
                // 16-byte aligned: s0 is a multiple of 8 and the pitch of 4
#pragma unroll
                for (int q = 0; q < WIN / 4; ++q) {
                    const f32x4_t v4 = reinterpret_cast<const f32x4_t *>(row)[q];
                    win[4 * q] = v4[0]; win[4 * q + 1] = v4[1]; win[4 * q + 2] = v4[2]; win[4 * q + 3] = v4[3];
                }
#pragma unroll
                for (int q = (WIN / 4) * 4; q < WIN; ++q) win[q] = row[q];
            } else {
#pragma unroll
                for (int q = 0; q < WIN; ++q) win[q] = row[q];
            }
#pragma unroll
            for (int j = 0; j < kDwS; ++j)
#pragma unroll
                for (int v = 0; v < K; ++v) acc[j] = fmaf(tap[u * K + v], win[j * ST + v], acc[j]);
        }
        if (valid) {
#pragma unroll
            for (int j = 0; j < kDwS; ++j)
                if (s0 + j < Wo) yp[r * Wo + s0 + j] = Elem<T>::from_f32(acc[j]);
        }
    }
}

// Depthwise for bf16 planes with square K x K taps (K = 3, 5, 7), stride ST
// (1, 2) and W even, products on v_dot2_f32_bf16 (two bf16 products summed
// in fp32 per instruction). Shared by the two kernels below:
//   - The zero-padded plane sits in the wave's LDS region as bf16: row pitch
//     a multiple of 8 elements, wide enough for the last strip's window,
//     interior at column pad. Rows arrive as 4-element pieces (8 bytes) when
//     W % 4 == 0, else as 2-element words.
//   - The mixed taps (sum_i alpha_bi E_i[c], rounded to bf16 like every other
//     mixed kernel) are kept as bf16 pairs: row u, columns 2q and 2q + 1;
//     past an odd K the pair ends in 0.
//   - A lane task is 8 consecutive outputs of a row. Per kernel row it reads
//     the window with 16-byte LDS reads; output j and tap pair q take input
//     elements j*ST + 2q and j*ST + 2q + 1: a window word when j*ST is even,
//     else a word assembled from two neighbours (alignbit).
constexpr int kDw2S = 8;              // outputs per lane task along a row
constexpr int kDw2PlaneBytes = 8192;  // LDS bytes per plane at most
constexpr int kDw2Pre = 4;            // plane pieces per lane held in registers

__host__ __device__ constexpr int dw2_pairs(int K) { return (K + 1) / 2; }
__host__ __device__ constexpr int dw2_words(int K, int ST) { return ((kDw2S - 1) * ST + 2 * dw2_pairs(K) + 1) / 2; }

// One plane's pieces: first kDw2Pre per lane (clamped indices, no branches
// between the loads).
__device__ __forceinline__ void dw2_fetch(const uint16_t *__restrict__ xp, int lane, int npc, bool q4,
                                          u32x2_t (&pc)[kDw2Pre]) {
#pragma unroll
    for (int k = 0; k < kDw2Pre; ++k) {
        const int p = min(lane + 64 * k, npc - 1);
        if (q4) {
            pc[k] = reinterpret_cast<const u32x2_t *>(xp)[p];
        } else {
            pc[k].x = reinterpret_cast<const uint32_t *>(xp)[p];
            pc[k].y = 0u;
        }
    }
}

// Writes piece p (pe elements at element p * pe of the plane) into the padded
// LDS plane; rows below the last one read (stride 2) are skipped.
__device__ __forceinline__ void dw2_put(uint32_t *pl, int p, u32x2_t v, int pe, bool q4, float invW, int W,
                                        int pad, int pitch, int Hp) {
    const int e = p * pe;
    // (e + 0.5) / W rounded down is exact in float for e < 2^12, W <= 2^8
    const int h = (int)(((float)e + 0.5f) * invW);
    if (h + pad >= Hp) return;
    const int off = (h + pad) * pitch + (e - h * W) + pad;  // element offset
    if ((pad & 1) == 0) {
        pl[off >> 1] = v.x;
        if (q4) pl[(off >> 1) + 1] = v.y;
    } else {
        uint16_t *pl16 = reinterpret_cast<uint16_t *>(pl);
        pl16[off] = (uint16_t)v.x;
        pl16[off + 1] = (uint16_t)(v.x >> 16);
        if (q4) {
            pl16[off + 2] = (uint16_t)v.y;
            pl16[off + 3] = (uint16_t)(v.y >> 16);
        }
    }
}

// 8 outputs of row r from column s0 of the staged plane.
template <int K, int ST>
__device__ __forceinline__ void dw2_task(const uint32_t *pl, int pw, const uint32_t (&tp)[K][dw2_pairs(K)], int r,
                                         int s0, float (&acc)[kDw2S]) {
    constexpr int KP = dw2_pairs(K);
    constexpr int NQ = (dw2_words(K, ST) + 3) / 4;  // 16-byte window reads per kernel row
#pragma unroll
    for (int j = 0; j < kDw2S; ++j) acc[j] = 0.f;
#pragma unroll
    for (int u = 0; u < K; ++u) {
        // window start: element s0 * ST of padded row r * ST + u (16-byte aligned)
        const u32x4_t *row = reinterpret_cast<const u32x4_t *>(pl + (r * ST + u) * pw + ((s0 * ST) >> 1));
        uint32_t wd[4 * NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const u32x4_t v4 = row[q];
            wd[4 * q] = v4.x; wd[4 * q + 1] = v4.y; wd[4 * q + 2] = v4.z; wd[4 * q + 3] = v4.w;
        }
#pragma unroll
        for (int j = 0; j < kDw2S; ++j)
#pragma unroll
            for (int q = 0; q < KP; ++q) {
                const int e0 = j * ST + 2 * q;
                const uint32_t pr = (e0 & 1) == 0 ? wd[e0 >> 1]
                                                  : __builtin_amdgcn_alignbit(wd[(e0 >> 1) + 1], wd[e0 >> 1], 16);
                acc[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, tp[u][q]),
                                                         __builtin_bit_cast(bf16x2_t, pr), acc[j], false);
            }
    }
}

// Stores a task's outputs (8-byte stores when Wo % 4 == 0).
__device__ __forceinline__ void dw2_store(uint16_t *dst, int s0, int Wo, bool st8, const float (&acc)[kDw2S]) {
    if (st8) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if (s0 + 4 * h + 4 <= Wo) {
                u32x2_t o;
                o.x = pack_bf16x2(acc[4 * h], acc[4 * h + 1]);
                o.y = pack_bf16x2(acc[4 * h + 2], acc[4 * h + 3]);
                reinterpret_cast<u32x2_t *>(dst)[h] = o;
            }
    } else {
#pragma unroll
        for (int j = 0; j < kDw2S; ++j)
            if (s0 + j < Wo) dst[j] = f32_to_bf16(acc[j]);
    }
}

// Plane-per-wave form (any n, or taps already mixed in wmixed): wave w of
// workgroup g takes plane 4 g + w. Lanes 0..2*K*KP-1 mix the plane's taps.
template <int K, int ST>
__global__ __launch_bounds__(64 * kDwPlanes) void depthwise_dot2_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ experts, const float *__restrict__ alpha,
    const uint16_t *__restrict__ wmixed, uint16_t *__restrict__ y, int B, int C, int H, int W, int pad,
    int Ho, int Wo, int n, int pitch, const float *__restrict__ a_in, const float *__restrict__ a_out) {
    constexpr int KT = K * K;
    constexpr int KP = dw2_pairs(K);
    extern __shared__ __attribute__((aligned(16))) uint32_t dwl[];  // kDwPlanes planes
    __shared__ uint32_t taps_sh[kDwPlanes][K * KP];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long nplanes = (long)B * C;
    const long bc_raw = (long)blockIdx.x * kDwPlanes + wave;
    const bool valid = bc_raw < nplanes;
    const long bc = valid ? bc_raw : nplanes - 1;
    const int b = (int)(bc / C), c = (int)(bc - (long)b * C);
    const int Hp = (Ho - 1) * ST + K;  // padded rows read
    const int pw = pitch >> 1;         // words per padded row (a multiple of 4)
    uint32_t *pl = dwl + wave * Hp * pw;
    const uint16_t *xp = x + bc * H * W;
    const int hw = H * W;
    const bool q4 = (W & 3) == 0;
    const int pe = q4 ? 4 : 2;  // elements per piece
    const int npc = hw / pe;
    const float invW = 1.f / (float)W;

    u32x2_t pre[kDw2Pre];
    dw2_fetch(xp, lane, npc, q4, pre);
    // taps: element (u, v) of the pair table, v < 2 KP; expert values and
    // attentions load 8 at a time
    if (lane < K * 2 * KP) {
        const int u = lane / (2 * KP), v = lane - u * (2 * KP);
        uint16_t tv = 0;
        if (v < K) {
            const int t = u * K + v;
            float tf;
            if (wmixed) {
                tf = bf16_to_f32(wmixed[bc * KT + t]);
            } else {
                float sm = 0.f;
                for (int i0 = 0; i0 < n; i0 += 8) {
                    float ev[8], av[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int i = min(i0 + k, n - 1);
                        ev[k] = bf16_to_f32(experts[((long)i * C + c) * KT + t]);
                        av[k] = alpha[(long)b * n + i];
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        if (i0 + k < n) sm = fmaf(av[k], ev[k], sm);
                }
                tf = sm;
            }
            // channel attentions of a depthwise plane scale its taps (one bf16 rounding)
            tv = f32_to_bf16(tf * (a_in ? a_in[(long)b * C + c] : 1.f) * (a_out ? a_out[(long)b * C + c] : 1.f));
        }
        reinterpret_cast<uint16_t *>(taps_sh[wave])[lane] = tv;
    }
    // zero the padded plane, then write the interior (LDS operations of a
    // wave complete in order; the empty asm statements keep the compiler
    // from reordering them)
    for (int i = lane; i < Hp * pw / 4; i += 64) reinterpret_cast<u32x4_t *>(pl)[i] = u32x4_t{0u, 0u, 0u, 0u};
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < kDw2Pre; ++k)
        if (lane + 64 * k < npc) dw2_put(pl, lane + 64 * k, pre[k], pe, q4, invW, W, pad, pitch, Hp);
    for (int p = lane + 64 * kDw2Pre; p < npc; p += 64) {
        u32x2_t v;
        if (q4) {
            v = reinterpret_cast<const u32x2_t *>(xp)[p];
        } else {
            v.x = reinterpret_cast<const uint32_t *>(xp)[p];
            v.y = 0u;
        }
        dw2_put(pl, p, v, pe, q4, invW, W, pad, pitch, Hp);
    }
    asm volatile("" ::: "memory");
    uint32_t tp[K][KP];
#pragma unroll
    for (int u = 0; u < K; ++u)
#pragma unroll
        for (int q = 0; q < KP; ++q) tp[u][q] = taps_sh[wave][u * KP + q];

    const int strips = (Wo + kDw2S - 1) / kDw2S;
    const float inv_Ho = 1.f / (float)Ho;
    uint16_t *yp = y + bc * Ho * Wo;
    const bool st8 = (Wo & 3) == 0;
    for (int task = lane; task < Ho * strips; task += 64) {
        // strip-major: neighbouring lanes take neighbouring rows of one strip
        const int sidx = (int)(((float)task + 0.5f) * inv_Ho);
        const int r = task - sidx * Ho, s0 = sidx * kDw2S;
        float acc[kDw2S];
        dw2_task<K, ST>(pl, pw, tp, r, s0, acc);
        if (valid) dw2_store(yp + r * Wo + s0, s0, Wo, st8, acc);
    }
}

// Channel-major form for n <= 8: workgroup (c, g) takes channel c of
// examples [16 g, 16 g + 16); wave w takes the examples 16 g + 4 w + k
// (k < 4) one after the other. The channel's expert values of the lane's tap
// load once per wave; each example's attentions are 8 unconditional loads of
// one address per wave; the next example's plane loads before the current
// one mixes, stages and computes.
constexpr int kDwChanPB = 4;  // examples (planes) per wave
template <int K, int ST>
__global__ __launch_bounds__(64 * kDwPlanes) void depthwise_chan_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ experts, const float *__restrict__ alpha,
    uint16_t *__restrict__ y, int B, int C, int H, int W, int pad, int Ho, int Wo, int n, int pitch,
    const float *__restrict__ a_in, const float *__restrict__ a_out) {
    constexpr int KT = K * K;
    constexpr int KP = dw2_pairs(K);
    extern __shared__ __attribute__((aligned(16))) uint32_t dwl[];
    __shared__ uint32_t taps_sh[kDwPlanes][K * KP];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int c = blockIdx.x % C;
    const int b0 = (blockIdx.x / C) * (kDwPlanes * kDwChanPB) + wave * kDwChanPB;
    const int Hp = (Ho - 1) * ST + K;
    const int pw = pitch >> 1;
    uint32_t *pl = dwl + wave * Hp * pw;
    const int hw = H * W;
    const bool q4 = (W & 3) == 0;
    const int pe = q4 ? 4 : 2;
    const int npc = hw / pe;
    const float invW = 1.f / (float)W;
    const int tl = lane < K * 2 * KP ? lane : 0;  // tap-table element of this lane
    const int tu = tl / (2 * KP), tv = tl - tu * (2 * KP);
    const bool tap_lane = lane < K * 2 * KP && tv < K;
    const int tt = tu * K + min(tv, K - 1);
    float ev[8];  // this channel's expert values of the lane's tap, 0 past n
#pragma unroll
    for (int i = 0; i < 8; ++i) ev[i] = i < n ? bf16_to_f32(experts[((long)min(i, n - 1) * C + c) * KT + tt]) : 0.f;
    for (int i = lane; i < Hp * pw / 4; i += 64) reinterpret_cast<u32x4_t *>(pl)[i] = u32x4_t{0u, 0u, 0u, 0u};
    const int strips = (Wo + kDw2S - 1) / kDw2S;
    const float inv_Ho = 1.f / (float)Ho;
    const bool st8 = (Wo & 3) == 0;
    u32x2_t cur[kDw2Pre];
    dw2_fetch(x + ((long)min(b0, B - 1) * C + c) * hw, lane, npc, q4, cur);
    for (int k = 0; k < kDwChanPB; ++k) {
        const int b = b0 + k;
        if (b >= B) break;
        u32x2_t nxt[kDw2Pre];
        dw2_fetch(x + ((long)min(b + 1, B - 1) * C + c) * hw, lane, npc, q4, nxt);
        {
            float av[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) av[i] = alpha[(long)b * n + min(i, n - 1)];
            float sm = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) sm = fmaf(av[i], ev[i], sm);
            // channel attentions of a depthwise plane scale its taps (one bf16 rounding)
            const uint16_t tv =
                f32_to_bf16(sm * (a_in ? a_in[(long)b * C + c] : 1.f) * (a_out ? a_out[(long)b * C + c] : 1.f));
            if (lane < K * 2 * KP)
                reinterpret_cast<uint16_t *>(taps_sh[wave])[lane] = tap_lane ? tv : (uint16_t)0;
        }
        asm volatile("" ::: "memory");
        const uint16_t *xp = x + ((long)b * C + c) * hw;
#pragma unroll
        for (int q = 0; q < kDw2Pre; ++q)
            if (lane + 64 * q < npc) dw2_put(pl, lane + 64 * q, cur[q], pe, q4, invW, W, pad, pitch, Hp);
        for (int p = lane + 64 * kDw2Pre; p < npc; p += 64) {
            u32x2_t v;
            if (q4) {
                v = reinterpret_cast<const u32x2_t *>(xp)[p];
            } else {
                v.x = reinterpret_cast<const uint32_t *>(xp)[p];
                v.y = 0u;
            }
            dw2_put(pl, p, v, pe, q4, invW, W, pad, pitch, Hp);
        }
        asm volatile("" ::: "memory");
        uint32_t tp[K][KP];
#pragma unroll
        for (int u = 0; u < K; ++u)
#pragma unroll
            for (int q = 0; q < KP; ++q) tp[u][q] = taps_sh[wave][u * KP + q];
        uint16_t *yp = y + ((long)b * C + c) * Ho * Wo;
        for (int task = lane; task < Ho * strips; task += 64) {
            const int sidx = (int)(((float)task + 0.5f) * inv_Ho);
            const int r = task - sidx * Ho, s0 = sidx * kDw2S;
            float acc[kDw2S];
            dw2_task<K, ST>(pl, pw, tp, r, s0, acc);
            dw2_store(yp + r * Wo + s0, s0, Wo, st8, acc);
        }
        asm volatile("" ::: "memory");  // this plane's last LDS reads before the next plane's writes
#pragma unroll
        for (int q = 0; q < kDw2Pre; ++q) cur[q] = nxt[q];
    }
}

}  // namespace

hipError_t launch_conv_direct_f32(const Geom &g, const float *x, const float *wmixed, float *y,
                                  hipStream_t stream, ChanAttn att) {
    const long total = (long)g.B * g.Cout * g.Ho * g.Wo;
    hipLaunchKernelGGL(conv_direct_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, stream, x, wmixed, y, g.B, g.Cin, g.H, g.W, g.Cout, g.KH, g.KW,
                       g.stride, g.pad, g.Ho, g.Wo, att.in, att.out);
    return hipGetLastError();
}

static size_t dw_lds_bytes(const Geom &g) {
    return (size_t)(g.H + 2 * g.pad) * (g.W + 2 * g.pad) * sizeof(float);
}

bool depthwise_supported(const Geom &g) {
    return g.groups == g.Cin && g.Cin == g.Cout && g.KT <= kDwMaxTaps &&
           dw_lds_bytes(g) <= 64 * 1024;
}

// row pitch (floats) of the strip kernel's plane: the last strip's window
// stays inside, rounded up to a multiple of 4
static int dw_pitch(const Geom &g) {
    const int strips = (g.Wo + kDwS - 1) / kDwS;
    const int need = (strips * kDwS - 1) * g.stride + g.KW;
    return (std::max(need, g.W + 2 * g.pad) + 3) / 4 * 4;
}

static bool dw_strip_ok(const Geom &g) {
    const int Hp = (g.Ho - 1) * g.stride + g.KH;
    return g.KH == g.KW && (g.KH == 3 || g.KH == 5 || g.KH == 7) && (g.stride == 1 || g.stride == 2) &&
           (long)Hp * dw_pitch(g) <= kDwPlaneFloats;
}

template <typename T>
static hipError_t launch_dw_strip(const Geom &g, const T *x, const T *experts, const float *alpha,
                                  const T *wmixed, T *y, hipStream_t stream, ChanAttn att) {
    const long planes = (long)g.B * g.Cin;
    const dim3 grid((unsigned)((planes + kDwPlanes - 1) / kDwPlanes));
    const int pitch = dw_pitch(g);
    const size_t lds = (size_t)kDwPlanes * ((g.Ho - 1) * g.stride + g.KH) * pitch * sizeof(float);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(64 * kDwPlanes), lds, stream, x, experts, alpha, wmixed, y,
                           g.B, g.Cin, g.H, g.W, g.pad, g.Ho, g.Wo, g.n, pitch, att.in, att.out);
        return hipGetLastError();
    };
    const int key = g.KH * 10 + g.stride;
    switch (key) {
    case 31: return go(depthwise_strip_kernel<T, 3, 1>);
    case 32: return go(depthwise_strip_kernel<T, 3, 2>);
    case 51: return go(depthwise_strip_kernel<T, 5, 1>);
    case 52: return go(depthwise_strip_kernel<T, 5, 2>);
    case 71: return go(depthwise_strip_kernel<T, 7, 1>);
    default: return go(depthwise_strip_kernel<T, 7, 2>);
    }
}

static int dw2_pitch(const Geom &g) {
    const int strips = (g.Wo + kDw2S - 1) / kDw2S;
    const int words = dw2_words(g.KW, g.stride);
    const int need = (strips - 1) * kDw2S * g.stride + 8 * ((words + 3) / 4);
    return (std::max(need, g.W + 2 * g.pad) + 7) / 8 * 8;
}

// bf16 planes for the dot2 kernels: square 3/5/7 taps, stride 1 or 2, W even
// (2-element words), planes of at most 4096 elements and rows of at most 256
// (exact float index splits), padded plane within kDw2PlaneBytes.
static bool dw2_ok(const Geom &g) {
    const int Hp = (g.Ho - 1) * g.stride + g.KH;
    return g.bf16 && g.KH == g.KW && (g.KH == 3 || g.KH == 5 || g.KH == 7) && (g.stride == 1 || g.stride == 2) &&
           g.W % 2 == 0 && g.H * g.W <= 4096 && g.W <= 256 && g.Ho <= 256 &&
           g.Ho * ((g.Wo + kDw2S - 1) / kDw2S) < 4096 &&
           (long)Hp * dw2_pitch(g) * 2 <= kDw2PlaneBytes;
}

template <typename F>
static hipError_t dw2_dispatch(const Geom &g, F &&go) {
    switch (g.KH * 10 + g.stride) {
    case 31: return go(std::integral_constant<int, 3>{}, std::integral_constant<int, 1>{});
    case 32: return go(std::integral_constant<int, 3>{}, std::integral_constant<int, 2>{});
    case 51: return go(std::integral_constant<int, 5>{}, std::integral_constant<int, 1>{});
    case 52: return go(std::integral_constant<int, 5>{}, std::integral_constant<int, 2>{});
    case 71: return go(std::integral_constant<int, 7>{}, std::integral_constant<int, 1>{});
    default: return go(std::integral_constant<int, 7>{}, std::integral_constant<int, 2>{});
    }
}

static hipError_t launch_dw2(const Geom &g, const uint16_t *x, const uint16_t *experts, const float *alpha,
                             const uint16_t *wmixed, uint16_t *y, hipStream_t stream, ChanAttn att) {
    const int pitch = dw2_pitch(g);
    const size_t lds = (size_t)kDwPlanes * ((g.Ho - 1) * g.stride + g.KH) * pitch * sizeof(uint16_t);
    if (!wmixed && g.n <= 8) {
        const int per_wg = kDwPlanes * kDwChanPB;
        const dim3 grid((unsigned)((long)g.Cin * ((g.B + per_wg - 1) / per_wg)));
        return dw2_dispatch(g, [&](auto k, auto st) {
            hipLaunchKernelGGL((depthwise_chan_kernel<decltype(k)::value, decltype(st)::value>), grid,
                               dim3(64 * kDwPlanes), lds, stream, x, experts, alpha, y, g.B, g.Cin, g.H, g.W,
                               g.pad, g.Ho, g.Wo, g.n, pitch, att.in, att.out);
            return hipGetLastError();
        });
    }
    const long planes = (long)g.B * g.Cin;
    const dim3 grid((unsigned)((planes + kDwPlanes - 1) / kDwPlanes));
    return dw2_dispatch(g, [&](auto k, auto st) {
        hipLaunchKernelGGL((depthwise_dot2_kernel<decltype(k)::value, decltype(st)::value>), grid,
                           dim3(64 * kDwPlanes), lds, stream, x, experts, alpha, wmixed, y, g.B, g.Cin, g.H,
                           g.W, g.pad, g.Ho, g.Wo, g.n, pitch, att.in, att.out);
        return hipGetLastError();
    });
}

hipError_t launch_conv_depthwise(const Geom &g, const void *x, const void *experts,
                                 const float *alpha, const void *wmixed, void *y,
                                 hipStream_t stream, ChanAttn att) {
    if (depthwise_mfma_ok(g, wmixed != nullptr))
        return launch_depthwise_mfma(g, static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(experts),
                                     alpha, static_cast<const uint16_t *>(wmixed), static_cast<uint16_t *>(y),
                                     stream, att);
    if (dw2_ok(g))
        return launch_dw2(g, static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(experts), alpha,
                          static_cast<const uint16_t *>(wmixed), static_cast<uint16_t *>(y), stream, att);
    if (dw_strip_ok(g)) {
        if (g.bf16)
            return launch_dw_strip<uint16_t>(g, static_cast<const uint16_t *>(x),
                                             static_cast<const uint16_t *>(experts), alpha,
                                             static_cast<const uint16_t *>(wmixed),
                                             static_cast<uint16_t *>(y), stream, att);
        return launch_dw_strip<float>(g, static_cast<const float *>(x), static_cast<const float *>(experts),
                                      alpha, static_cast<const float *>(wmixed), static_cast<float *>(y),
                                      stream, att);
    }
    const size_t lds = dw_lds_bytes(g);
    const dim3 grid((unsigned)((long)g.B * g.Cin));
    if (g.bf16) {
        hipLaunchKernelGGL(depthwise_kernel<uint16_t>, grid, dim3(256), lds, stream,
                           static_cast<const uint16_t *>(x),
                           static_cast<const uint16_t *>(experts), alpha,
                           static_cast<const uint16_t *>(wmixed), static_cast<uint16_t *>(y),
                           g.B, g.Cin, g.H, g.W, g.KH, g.KW, g.stride, g.pad, g.Ho, g.Wo, g.n, att.in, att.out);
    } else {
        hipLaunchKernelGGL(depthwise_kernel<float>, grid, dim3(256), lds, stream,
                           static_cast<const float *>(x), static_cast<const float *>(experts),
                           alpha, static_cast<const float *>(wmixed), static_cast<float *>(y),
                           g.B, g.Cin, g.H, g.W, g.KH, g.KW, g.stride, g.pad, g.Ho, g.Wo, g.n, att.in, att.out);
    }
    return hipGetLastError();
}

}  // namespace dynconv
