// Routing: input-dependent attentions of each example (KernelWarehouse:
// Rethinking the Design of Dynamic Convolution, abstract: "input-dependent
// attentions"; FMDConv, abstract: temperature-scaled kernel attention).
//
//   gap[b,c] = mean_{h,w} x[b,c,h,w]
//   z[b,i]   = sum_c fc_w[i,c] gap[b,c] + fc_b[i]
//   alpha    = sigmoid(z)  or  softmax_i(z / T)
//
// Two kernels. The pooling kernel streams x once from HBM with 8-16 byte
// vector loads: every channel plane is reduced by a group of lanes (16-64
// lanes, sized to the plane) so that many planes are in flight per CU and
// the chip is filled even at small batch. The FC kernel is tiny (one wave
// per example). No atomics: sums run in a fixed order, so the result is
// deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

constexpr int kGapThreads = 256;
// batches at least this large route with one workgroup per example
constexpr int kRouteMinB = 64;

// VEC elements per load (VEC * sizeof(T) bytes); LPR lanes per plane.
template <typename T, int VEC, int LPR>
__global__ __launch_bounds__(kGapThreads) void gap_kernel(const T *__restrict__ x,
                                                          float *__restrict__ gap,
                                                          long rows, int hw) {
    constexpr int kRowsPerBlock = kGapThreads / LPR;
    const int lane_in_row = threadIdx.x % LPR;
    const long row = (long)blockIdx.x * kRowsPerBlock + threadIdx.x / LPR;
    const bool active = row < rows;
    const long r = active ? row : rows - 1;
    const int nvec = hw / VEC;
    const T *p = x + r * (long)hw;
    float s = 0.f;
    if constexpr (sizeof(T) == 2 && VEC == 8) {
        const u32x4_t *v = reinterpret_cast<const u32x4_t *>(p);
#pragma unroll 4
        for (int i = lane_in_row; i < nvec; i += LPR) {
            u32x4_t q = __builtin_nontemporal_load(v + i);
            s += (bf16_lo(q.x) + bf16_hi(q.x)) + (bf16_lo(q.y) + bf16_hi(q.y)) +
                 ((bf16_lo(q.z) + bf16_hi(q.z)) + (bf16_lo(q.w) + bf16_hi(q.w)));
        }
    } else if constexpr (sizeof(T) == 2 && VEC == 4) {
        const u32x2_t *v = reinterpret_cast<const u32x2_t *>(p);
#pragma unroll 4
        for (int i = lane_in_row; i < nvec; i += LPR) {
            u32x2_t q = __builtin_nontemporal_load(v + i);
            s += (bf16_lo(q.x) + bf16_hi(q.x)) + (bf16_lo(q.y) + bf16_hi(q.y));
        }
    } else if constexpr (sizeof(T) == 4 && VEC == 4) {
        const f32x4_t *v = reinterpret_cast<const f32x4_t *>(p);
#pragma unroll 4
        for (int i = lane_in_row; i < nvec; i += LPR) {
            f32x4_t q = __builtin_nontemporal_load(v + i);
            s += (q[0] + q[1]) + (q[2] + q[3]);
        }
    } else {
        static_assert(VEC == 1, "unsupported vector width");
#pragma unroll 4
        for (int i = lane_in_row; i < nvec; i += LPR) s += Elem<T>::to_f32(p[i]);
    }
    s = group_sum<LPR>(s);
    if (active && lane_in_row == 0) gap[row] = s / (float)hw;
}

// One wave per example. Lanes run over channels (coalesced reads of gap and
// fc_w) and keep partial logits for up to 16 experts at a time; a fixed
// butterfly reduction finishes each logit. Logits go through LDS so that
// lane j then owns experts j, j+64, ... for the nonlinearity.
constexpr int kMaxJ = 4;     // n <= 256
constexpr int kIChunk = 16;  // experts per pass over the channels
__global__ __launch_bounds__(256) void route_fc_kernel(const float *__restrict__ gap,
                                                       const float *__restrict__ fc_w,
                                                       const float *__restrict__ fc_b,
                                                       float *__restrict__ alpha, int B,
                                                       int C, int n, int mode, float temp) {
    __shared__ float zs[4][64 * kMaxJ];
    const int wv = threadIdx.x / 64;
    const int b = blockIdx.x * 4 + wv;
    const int lane = threadIdx.x % 64;
    if (b >= B) return;  // whole wave leaves together; no barriers below
    const float *gb = gap + (long)b * C;
    for (int i0 = 0; i0 < n; i0 += kIChunk) {
        float part[kIChunk];
#pragma unroll
        for (int ii = 0; ii < kIChunk; ++ii) part[ii] = 0.f;
        for (int c = lane; c < C; c += 64) {
            const float gc = gb[c];
#pragma unroll
            for (int ii = 0; ii < kIChunk; ++ii)
                if (i0 + ii < n) part[ii] = fmaf(fc_w[(long)(i0 + ii) * C + c], gc, part[ii]);
        }
#pragma unroll
        for (int ii = 0; ii < kIChunk; ++ii) {
            if (i0 + ii < n) {
                const float zt = wave_sum(part[ii]);
                if (lane == 0) zs[wv][i0 + ii] = zt + (fc_b ? fc_b[i0 + ii] : 0.f);
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float z[kMaxJ];
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) z[j] = (lane + 64 * j < n) ? zs[wv][lane + 64 * j] : 0.f;
    if (mode == 0) {
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) {
            const int i = lane + 64 * j;
            if (i < n) {
                float a;
                if (z[j] >= 0.f) {
                    a = 1.f / (1.f + expf(-z[j]));
                } else {
                    const float e = expf(z[j]);
                    a = e / (1.f + e);
                }
                alpha[(long)b * n + i] = a;
            }
        }
    } else {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j)
            if (lane + 64 * j < n) m = fmaxf(m, z[j] / temp);
        m = wave_max(m);
        float e[kMaxJ];
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) {
            e[j] = (lane + 64 * j < n) ? expf(z[j] / temp - m) : 0.f;
            s += e[j];
        }
        s = wave_sum(s);
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) {
            const int i = lane + 64 * j;
            if (i < n) alpha[(long)b * n + i] = e[j] / s;
        }
    }
}

// Single-kernel routing for batches of at least kRouteMinB examples: one
// workgroup of 1024 threads per example. Phase 1 reduces the example's
// channel planes into channel means in LDS: LPR lanes per plane, and every
// lane issues all of its (at most kRouteMaxK) vector loads of a plane before
// it adds any, so a CU keeps about 128 KB of loads in flight and a few dozen
// workgroups already saturate HBM. Phase 2 computes the logits (one wave per
// expert, lanes over channels, fixed-order reduction); phase 3 applies the
// nonlinearity. No workspace, no atomics, one launch.
constexpr int kRouteThreads = 1024;
constexpr int kRouteMaxC = 4096;
constexpr int kRouteMaxK = 16;  // vector loads per lane and plane
// One load of VEC elements and its float sum (split so that a lane can issue
// all of its loads before the first sum).
template <typename T, int VEC> struct VecLoad;
template <> struct VecLoad<uint16_t, 8> {
    using V = u32x4_t;
    static __device__ __forceinline__ float sum(V q) {
        return (bf16_lo(q.x) + bf16_hi(q.x)) + (bf16_lo(q.y) + bf16_hi(q.y)) +
               ((bf16_lo(q.z) + bf16_hi(q.z)) + (bf16_lo(q.w) + bf16_hi(q.w)));
    }
};
template <> struct VecLoad<uint16_t, 4> {
    using V = u32x2_t;
    static __device__ __forceinline__ float sum(V q) {
        return (bf16_lo(q.x) + bf16_hi(q.x)) + (bf16_lo(q.y) + bf16_hi(q.y));
    }
};
template <> struct VecLoad<uint16_t, 1> {
    using V = uint16_t;
    static __device__ __forceinline__ float sum(V q) { return bf16_to_f32(q); }
};
template <> struct VecLoad<float, 4> {
    using V = f32x4_t;
    static __device__ __forceinline__ float sum(V q) { return (q[0] + q[1]) + (q[2] + q[3]); }
};
template <> struct VecLoad<float, 1> {
    using V = float;
    static __device__ __forceinline__ float sum(V q) { return q; }
};
// Phases 2 and 3 of the single-kernel router, after the channel means of
// example b are in gsh (and a barrier): logits by one wave per expert (lanes
// over channels, fixed-order reduction), then the nonlinearity in wave 0.
// The weights of a wave's first expert for channels lane + 64 k (k < kFcPre)
// are loaded before the pooling starts, so their latency hides under it.
constexpr int kFcPre = 8;
struct FcPre {
    float w[kFcPre];
    float bias;
};
__device__ __forceinline__ FcPre route_prefetch_fc(const float *__restrict__ fc_w,
                                                   const float *__restrict__ fc_b, int C, int n) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    FcPre f;
    const int i = min(wave, n - 1);
#pragma unroll
    for (int k = 0; k < kFcPre; ++k) f.w[k] = fc_w[(long)i * C + min(lane + 64 * k, C - 1)];
    f.bias = fc_b ? fc_b[i] : 0.f;
    return f;
}
__device__ __forceinline__ void route_finish(const float *gsh, float *zsh, const float *__restrict__ fc_w,
                                             const float *__restrict__ fc_b, float *__restrict__ alpha,
                                             int b, int C, int n, int mode, float temp, const FcPre &pre) {
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    for (int i = wave; i < n; i += kRouteThreads / 64) {
        float part = 0.f;
        int c0 = 0;
        if (i == wave) {  // first expert of this wave: prefetched weights
#pragma unroll
            for (int k = 0; k < kFcPre; ++k) {
                const int c = lane + 64 * k;
                if (c < C) part = fmaf(pre.w[k], gsh[c], part);
            }
            c0 = 64 * kFcPre;
        }
        for (int c = c0 + lane; c < C; c += 64) part = fmaf(fc_w[(long)i * C + c], gsh[c], part);
        part = wave_sum(part);
        if (lane == 0) zsh[i] = part + (i == wave ? pre.bias : (fc_b ? fc_b[i] : 0.f));
    }
    __syncthreads();
    if (wave != 0) return;
    float z[kMaxJ];
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) z[j] = (lane + 64 * j < n) ? zsh[lane + 64 * j] : 0.f;
    if (mode == 0) {
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) {
            const int i = lane + 64 * j;
            if (i < n) {
                float av;
                if (z[j] >= 0.f) {
                    av = 1.f / (1.f + expf(-z[j]));
                } else {
                    const float e = expf(z[j]);
                    av = e / (1.f + e);
                }
                alpha[(long)b * n + i] = av;
            }
        }
    } else {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j)
            if (lane + 64 * j < n) m = fmaxf(m, z[j] / temp);
        m = wave_max(m);
        float e[kMaxJ];
        float ssum = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) {
            e[j] = (lane + 64 * j < n) ? expf(z[j] / temp - m) : 0.f;
            ssum += e[j];
        }
        ssum = wave_sum(ssum);
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) {
            const int i = lane + 64 * j;
            if (i < n) alpha[(long)b * n + i] = e[j] / ssum;
        }
    }
}

template <typename T, int VEC, int LPR>
__global__ __launch_bounds__(kRouteThreads) void route_fused_kernel(
    const T *__restrict__ x, const float *__restrict__ fc_w, const float *__restrict__ fc_b,
    float *__restrict__ alpha, int C, int hw, int n, int mode, float temp) {
    __shared__ float gsh[kRouteMaxC];
    __shared__ float zsh[64 * kMaxJ];
    constexpr int kPlanes = kRouteThreads / LPR;  // planes per pass
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int grp = tid / LPR, lane_in = tid % LPR;
    const int nvec = hw / VEC;  // at most LPR * kRouteMaxK
    const T *xb = x + (long)b * C * hw;
    const FcPre pre = route_prefetch_fc(fc_w, fc_b, C, n);
    for (int c0 = 0; c0 < C; c0 += kPlanes) {
        const int c = c0 + grp;
        const T *p = xb + (long)min(c, C - 1) * hw;
        // unconditional loads at clamped indices (no branch between them, so
        // all are in flight at once); lanes past the plane's end add 0
        using L = VecLoad<T, VEC>;
        const typename L::V *pv = reinterpret_cast<const typename L::V *>(p);
        typename L::V q[kRouteMaxK];
#pragma unroll
        for (int k = 0; k < kRouteMaxK; ++k) q[k] = pv[min(lane_in + LPR * k, nvec - 1)];
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < kRouteMaxK; ++k) s += lane_in + LPR * k < nvec ? L::sum(q[k]) : 0.f;
        s = group_sum<LPR>(s);
        if (lane_in == 0 && c < C) gsh[c] = s / (float)hw;
    }
    __syncthreads();
    route_finish(gsh, zsh, fc_w, fc_b, alpha, b, C, n, mode, temp, pre);
}

template <typename T, int VEC>
hipError_t launch_route_fused_vec(const T *x, const float *fc_w, const float *fc_b, float *alpha,
                                  int B, int C, int hw, int n, int mode, float temp,
                                  hipStream_t s) {
    const int nvec = hw / VEC;
    // fewest lanes per plane that keep a lane's loads within kRouteMaxK
    int lpr = 1;
    while (lpr * kRouteMaxK < nvec) lpr *= 2;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(B), dim3(kRouteThreads), 0, s, x, fc_w, fc_b, alpha, C, hw,
                           n, mode, temp);
        return hipGetLastError();
    };
    switch (lpr) {
    case 1: return go(route_fused_kernel<T, VEC, 1>);
    case 2: return go(route_fused_kernel<T, VEC, 2>);
    case 4: return go(route_fused_kernel<T, VEC, 4>);
    case 8: return go(route_fused_kernel<T, VEC, 8>);
    case 16: return go(route_fused_kernel<T, VEC, 16>);
    case 32: return go(route_fused_kernel<T, VEC, 32>);
    default: return go(route_fused_kernel<T, VEC, 64>);
    }
}

template <typename T, int VEC>
hipError_t launch_gap_vec(const T *x, float *gap, long rows, int hw, hipStream_t s) {
    const int nvec = hw / VEC;
    // lanes per plane: about 4 vectors per lane, between 8 and 64 lanes
    int lpr = 8;
    while (lpr < 64 && lpr * 4 < nvec) lpr *= 2;
    auto go = [&](auto kern, int l) {
        const long blocks = (rows + (kGapThreads / l) - 1) / (kGapThreads / l);
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kGapThreads), 0, s, x, gap,
                           rows, hw);
        return hipGetLastError();
    };
    switch (lpr) {
    case 8: return go(gap_kernel<T, VEC, 8>, 8);
    case 16: return go(gap_kernel<T, VEC, 16>, 16);
    case 32: return go(gap_kernel<T, VEC, 32>, 32);
    default: return go(gap_kernel<T, VEC, 64>, 64);
    }
}


// Several FC heads on the channel means, for FMDConv's kernel, input and
// output attentions. Workgroup (b, j): chunk j of the heads' logits of
// example b. A head with the softmax (its normalisation spans all its
// logits) is one chunk of up to 256 logits; a sigmoid head is cut into
// chunks of 64. Wave w computes the chunk's logits w, w + 4, ..., four at a
// time with the lanes over channels (coalesced rows of fc_w) and a fixed
// butterfly per logit; the nonlinearity runs after a barrier.
constexpr int kHeadsMax = 3;
struct RouteHeads {
    const float *w[kHeadsMax];
    const float *b[kHeadsMax];
    float *out[kHeadsMax];
    int n[kHeadsMax], mode[kHeadsMax], first[kHeadsMax + 1];  // first chunk of each head
    int heads;
};
__global__ __launch_bounds__(256) void route_heads_kernel(const float *__restrict__ gap, RouteHeads hp,
                                                          int C, float temp) {
    __shared__ float z[256];
    const int b = blockIdx.x, j = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int h = 0;
    while (h + 1 < hp.heads && j >= hp.first[h + 1]) ++h;
    const int n = hp.n[h], mode = hp.mode[h];
    const int per = mode == 1 ? n : 64;
    const int i0 = (j - hp.first[h]) * per, cnt = min(per, n - i0);
    const float *gb = gap + (long)b * C;
    const float *W = hp.w[h];
    for (int q = wave * 4; q < cnt; q += 16) {
        float part[4] = {0.f, 0.f, 0.f, 0.f};
        for (int c = lane; c < C; c += 64) {
            const float gc = gb[c];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                part[k] = fmaf(W[(long)(i0 + min(q + k, cnt - 1)) * C + c], gc, part[k]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float t = wave_sum(part[k]);
            if (lane == 0 && q + k < cnt) z[q + k] = t + (hp.b[h] ? hp.b[h][i0 + q + k] : 0.f);
        }
    }
    __syncthreads();
    float *out = hp.out[h] + (long)b * n + i0;
    if (mode == 0) {
        for (int i = tid; i < cnt; i += 256) {
            const float v = z[i];
            float a;
            if (v >= 0.f) {
                a = 1.f / (1.f + expf(-v));
            } else {
                const float e = expf(v);
                a = e / (1.f + e);
            }
            out[i] = a;
        }
    } else if (wave == 0) {
        float m = -INFINITY;
        for (int i = lane; i < cnt; i += 64) m = fmaxf(m, z[i] / temp);
        m = wave_max(m);
        float s = 0.f;
        for (int i = lane; i < cnt; i += 64) s += expf(z[i] / temp - m);
        s = wave_sum(s);
        for (int i = lane; i < cnt; i += 64) out[i] = expf(z[i] / temp - m) / s;
    }
}

}  // namespace

static_assert(kMaxJ * 64 >= 256, "route kernel covers n <= 256");

bool route_single_kernel(const Geom &g) {
    // planes up to 64 lanes x kRouteMaxK vectors (bf16: 8192 elements with 16-byte loads)
    return g.B >= kRouteMinB && g.Cin <= kRouteMaxC && g.H * g.W <= 64 * kRouteMaxK;
}

hipError_t launch_route(const Geom &g, const void *x, const float *fc_w, const float *fc_b,
                        int mode, float temperature, float *gap, float *alpha,
                        hipStream_t stream) {
    const long rows = (long)g.B * g.Cin;
    const int hw = g.H * g.W;
    const float tp = mode == 1 ? temperature : 1.0f;
    if (route_single_kernel(g)) {
        if (g.bf16) {
            const uint16_t *xb = static_cast<const uint16_t *>(x);
            if (hw % 8 == 0) return launch_route_fused_vec<uint16_t, 8>(xb, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
            if (hw % 4 == 0) return launch_route_fused_vec<uint16_t, 4>(xb, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
            return launch_route_fused_vec<uint16_t, 1>(xb, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
        }
        const float *xf = static_cast<const float *>(x);
        if (hw % 4 == 0) return launch_route_fused_vec<float, 4>(xf, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
        return launch_route_fused_vec<float, 1>(xf, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
    }
    hipError_t e;
    if (g.bf16) {
        const uint16_t *xb = static_cast<const uint16_t *>(x);
        if (hw % 8 == 0) e = launch_gap_vec<uint16_t, 8>(xb, gap, rows, hw, stream);
        else if (hw % 4 == 0) e = launch_gap_vec<uint16_t, 4>(xb, gap, rows, hw, stream);
        else e = launch_gap_vec<uint16_t, 1>(xb, gap, rows, hw, stream);
    } else {
        const float *xf = static_cast<const float *>(x);
        if (hw % 4 == 0) e = launch_gap_vec<float, 4>(xf, gap, rows, hw, stream);
        else e = launch_gap_vec<float, 1>(xf, gap, rows, hw, stream);
    }
    if (e != hipSuccess) return e;
    const float temp = mode == 1 ? temperature : 1.0f;
    hipLaunchKernelGGL(route_fc_kernel, dim3((g.B + 3) / 4), dim3(256), 0, stream, gap, fc_w,
                       fc_b, alpha, g.B, g.Cin, g.n, mode, temp);
    return hipGetLastError();
}

hipError_t launch_gap(const Geom &g, const void *x, float *gap, hipStream_t stream) {
    const long rows = (long)g.B * g.Cin;
    const int hw = g.H * g.W;
    if (g.bf16) {
        const uint16_t *xb = static_cast<const uint16_t *>(x);
        if (hw % 8 == 0) return launch_gap_vec<uint16_t, 8>(xb, gap, rows, hw, stream);
        if (hw % 4 == 0) return launch_gap_vec<uint16_t, 4>(xb, gap, rows, hw, stream);
        return launch_gap_vec<uint16_t, 1>(xb, gap, rows, hw, stream);
    }
    const float *xf = static_cast<const float *>(x);
    if (hw % 4 == 0) return launch_gap_vec<float, 4>(xf, gap, rows, hw, stream);
    return launch_gap_vec<float, 1>(xf, gap, rows, hw, stream);
}

hipError_t launch_route_heads(const Geom &g, const void *x, int heads, const float *const *fc_w,
                              const float *const *fc_b, const int *nout, const int *mode,
                              float temperature, float *gap, float *const *out, hipStream_t stream) {
    if (heads < 1 || heads > kHeadsMax) return hipErrorInvalidValue;
    hipError_t e = launch_gap(g, x, gap, stream);
    if (e != hipSuccess) return e;
    // all heads from the same channel means, in one launch
    RouteHeads hp{};
    hp.heads = heads;
    int chunks = 0;
    for (int h = 0; h < heads; ++h) {
        if (nout[h] < 1 || nout[h] > 256) return hipErrorInvalidValue;
        hp.w[h] = fc_w[h];
        hp.b[h] = fc_b[h];
        hp.out[h] = out[h];
        hp.n[h] = nout[h];
        hp.mode[h] = mode[h];
        hp.first[h] = chunks;
        chunks += mode[h] == 1 ? 1 : ceil_div(nout[h], 64);
    }
    hp.first[heads] = chunks;
    hipLaunchKernelGGL(route_heads_kernel, dim3((unsigned)g.B, (unsigned)chunks), dim3(256), 0, stream, gap,
                       hp, g.Cin, temperature);
    return hipGetLastError();
}

}  // namespace dynconv
