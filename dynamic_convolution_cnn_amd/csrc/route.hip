// Routing: the attentions of each example, computed from its input
// (KernelWarehouse: Rethinking the Design of Dynamic Convolution, abstract;
// FMDConv, abstract: temperature-scaled kernel attention).
//
//   gap[b,c] = mean_{h,w} x[b,c,h,w]
//   z[b,i]   = sum_c fc_w[i,c] gap[b,c] + fc_b[i]
//   alpha    = sigmoid(z)  or  softmax_i(z / T)
//
// One launch in the common cases: one workgroup per example from 64
// examples up, several per example below that (the split router, whose last
// workgroup per example finishes the FC). Planes too large for those take
// two kernels: a pooling kernel that streams x once with 8-16 byte vector
// loads (16-64 lanes per plane), then a small FC kernel (one wave per
// example). Every sum runs in a fixed order, so the result is deterministic.

#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

constexpr int kGapThreads = 256;
// batches below this route with several workgroups per example (split
// router), larger ones with one workgroup per example
constexpr int kRouteSplitMaxB = 64;
constexpr int kSplitThreads = 512;
// s_waitcnt operand: vector memory count 0, the other counters unconstrained
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;
// bytes of tickets at the start of the split router's workspace
constexpr size_t kRouteTicketBytes(int B) { return ((size_t)B * sizeof(unsigned) + 255) / 256 * 256; }

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

// Single-kernel routing for batches of at least kRouteSplitMaxB examples: one
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
// Logits of one example (NT threads, the channel means in gsh). Wave w takes
// experts w, w + NT / 64, ...: its first expert from the weights prefetched
// before the pooling, the rest in batches of kLogitEB whose weights (up to
// kLogitCB blocks of 64 channels each) are all loaded before the first
// multiply, so one memory round trip serves a batch instead of one per
// expert. Every logit sums c = lane + 64 j in ascending j, then the wave's
// fixed butterfly, whatever the batching.
constexpr int kLogitEB = 8;
constexpr int kLogitCB = 2;
template <int NT = kRouteThreads>
__device__ __forceinline__ void route_logits(const float *gsh, float *zsh, const float *__restrict__ fc_w,
                                             const float *__restrict__ fc_b, int C, int n, const FcPre &pre) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    if (wave < n) {  // first expert of this wave: prefetched weights
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < kFcPre; ++k) {
            const int c = lane + 64 * k;
            if (c < C) part = fmaf(pre.w[k], gsh[c], part);
        }
        for (int c = 64 * kFcPre + lane; c < C; c += 64) part = fmaf(fc_w[(long)wave * C + c], gsh[c], part);
        part = wave_sum(part);
        if (lane == 0) zsh[wave] = part + pre.bias;
    }
    for (int i0 = wave + NW; i0 < n; i0 += kLogitEB * NW) {
        float part[kLogitEB];
#pragma unroll
        for (int e = 0; e < kLogitEB; ++e) part[e] = 0.f;
        for (int c0 = 0; c0 < C; c0 += 64 * kLogitCB) {
            float wv[kLogitEB][kLogitCB];
#pragma unroll
            for (int e = 0; e < kLogitEB; ++e)
#pragma unroll
                for (int j = 0; j < kLogitCB; ++j)
                    wv[e][j] = i0 + NW * e < n ? fc_w[(long)(i0 + NW * e) * C + min(c0 + lane + 64 * j, C - 1)] : 0.f;
#pragma unroll
            for (int e = 0; e < kLogitEB; ++e)
#pragma unroll
                for (int j = 0; j < kLogitCB; ++j) {
                    const int c = c0 + lane + 64 * j;
                    if (c < C) part[e] = fmaf(wv[e][j], gsh[c], part[e]);
                }
        }
#pragma unroll
        for (int e = 0; e < kLogitEB; ++e) {
            const int i = i0 + NW * e;
            if (i < n) {
                const float t = wave_sum(part[e]);
                if (lane == 0) zsh[i] = t + (fc_b ? fc_b[i] : 0.f);
            }
        }
    }
}

// The nonlinearity of router phase 3, in wave 0, from the logits in zsh
// (after a barrier).
__device__ __forceinline__ void route_activate(const float *zsh, float *__restrict__ alpha, int b, int n, int mode,
                                               float temp) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
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


template <int NT = kRouteThreads>
__device__ __forceinline__ void route_finish(const float *gsh, float *zsh, const float *__restrict__ fc_w,
                                             const float *__restrict__ fc_b, float *__restrict__ alpha,
                                             int b, int C, int n, int mode, float temp, const FcPre &pre) {
    route_logits<NT>(gsh, zsh, fc_w, fc_b, C, n, pre);
    __syncthreads();
    route_activate(zsh, alpha, b, n, mode, temp);
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

// The same single-kernel router for bf16 planes of an even number of
// elements that is not a multiple of 8 (14 x 14): 16-byte loads through a
// buffer descriptor over x (dword-aligned planes; the last vector of a plane
// runs into the next plane, or past the tensor, where the read returns 0),
// its elements past the plane left out of the sum. Half the load
// instructions of 8-byte vectors, twice the bytes per request.
constexpr int kRouteMaxK16 = 8;  // 16-byte loads per lane and plane
template <int LPR>
__global__ __launch_bounds__(kRouteThreads) void route_fused16_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ fc_w, const float *__restrict__ fc_b,
    float *__restrict__ alpha, int C, int hw, int n, int mode, float temp, int x_bytes) {
    __shared__ float gsh[kRouteMaxC];
    __shared__ float zsh[64 * kMaxJ];
    constexpr int kPlanes = kRouteThreads / LPR;  // planes per pass
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int grp = tid / LPR, lane_in = tid % LPR;
    const int nvec = (hw + 7) / 8;              // at most LPR * kRouteMaxK16
    const int tail_words = (hw - 8 * (nvec - 1)) / 2;  // valid words of the last vector (1..4)
    const uint64_t q = reinterpret_cast<uint64_t>(x);
    const uint64_t qs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)q) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(q >> 32)) << 32);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(qs), 0,
                                                      __builtin_amdgcn_readfirstlane(x_bytes), 0x00020000);
    const FcPre pre = route_prefetch_fc(fc_w, fc_b, C, n);
    for (int c0 = 0; c0 < C; c0 += kPlanes) {
        const int c = c0 + grp;
        const int base = (((b * C) + min(c, C - 1)) * hw) * 2;  // bytes (x_bytes < 2^31)
        // every load before the first sum (clamped vector index, no branch)
        u32x4_t v[kRouteMaxK16];
#pragma unroll
        for (int k = 0; k < kRouteMaxK16; ++k)
            v[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rs, base + 16 * min(lane_in + LPR * k, nvec - 1), 0, 0));
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < kRouteMaxK16; ++k) {
            const int vi = lane_in + LPR * k;
            const int words = vi < nvec - 1 ? 4 : (vi == nvec - 1 ? tail_words : 0);
            const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) t += j < words ? bf16_lo(w[j]) + bf16_hi(w[j]) : 0.f;
            s += t;
        }
        s = group_sum<LPR>(s);
        if (lane_in == 0 && c < C) gsh[c] = s / (float)hw;
    }
    __syncthreads();
    route_finish(gsh, zsh, fc_w, fc_b, alpha, b, C, n, mode, temp, pre);
}

// Split router for batches below kRouteSplitMaxB. The channel planes of
// example b are pooled by S workgroups of 512 threads, one pass of 512 / LPR
// planes each with every lane's loads in flight before its first add, so
// that B * S workgroups spread the loads over the chip at B = 32 (one
// workgroup per example would leave most CUs idle). Each workgroup stores its channel
// means to the workspace and draws a ticket from the example's counter; the
// one that draws ticket S - 1 holds the last piece, reads all of the
// example's means back and finishes the FC and the nonlinearity exactly as
// the one-workgroup router does (same fixed order of every sum), then puts
// the counter back to zero for the next call. The ticket only decides which
// workgroup finishes, so the result is deterministic. The means are written
// and read back with device-scope atomic accesses (coherent across the XCDs'
// separate L2 caches) and each workgroup takes its ticket only after its
// means stores have completed, so the finishing workgroup, which reads them
// after drawing the last ticket, sees every workgroup's means.
template <typename T, int VEC, int LPR, bool EVEN16>
__global__ __launch_bounds__(kSplitThreads) void route_split_kernel(
    const T *__restrict__ x, const float *__restrict__ fc_w, const float *__restrict__ fc_b,
    float *__restrict__ alpha, float *__restrict__ means, unsigned *__restrict__ tickets, int C, int hw, int n,
    int mode, float temp, int S, int x_bytes) {
    __shared__ float gsh[kRouteMaxC];
    __shared__ float zsh[64 * kMaxJ];
    __shared__ int is_last;
    constexpr int kPlanes = kSplitThreads / LPR;  // planes per workgroup
    const int b = blockIdx.x / S, part = blockIdx.x - b * S;
    const int tid = threadIdx.x;
    const int grp = tid / LPR, lane_in = tid % LPR;
    const int c = part * kPlanes + grp;
    const FcPre pre = route_prefetch_fc(fc_w, fc_b, C, n);
    float s = 0.f;
    if constexpr (EVEN16) {
        // bf16 planes of an even size that is not a multiple of 8: 16-byte
        // loads through a buffer descriptor (reads past the tensor return 0),
        // elements past the plane left out of the sum
        const int nvec = (hw + 7) / 8;
        const int tail_words = (hw - 8 * (nvec - 1)) / 2;
        const uint64_t q = reinterpret_cast<uint64_t>(x);
        const uint64_t qs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)q) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(q >> 32)) << 32);
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(qs), 0,
                                                          __builtin_amdgcn_readfirstlane(x_bytes), 0x00020000);
        const int base = (((b * C) + min(c, C - 1)) * hw) * 2;  // bytes (x_bytes < 2^31)
        u32x4_t v[kRouteMaxK16];
#pragma unroll
        for (int k = 0; k < kRouteMaxK16; ++k)
            v[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rs, base + 16 * min(lane_in + LPR * k, nvec - 1), 0, 0));
#pragma unroll
        for (int k = 0; k < kRouteMaxK16; ++k) {
            const int vi = lane_in + LPR * k;
            const int words = vi < nvec - 1 ? 4 : (vi == nvec - 1 ? tail_words : 0);
            const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) t += j < words ? bf16_lo(w[j]) + bf16_hi(w[j]) : 0.f;
            s += t;
        }
    } else {
        const int nvec = hw / VEC;
        using L = VecLoad<T, VEC>;
        const typename L::V *pv =
            reinterpret_cast<const typename L::V *>(x + ((long)b * C + min(c, C - 1)) * hw);
        typename L::V q[kRouteMaxK];
#pragma unroll
        for (int k = 0; k < kRouteMaxK; ++k) q[k] = pv[min(lane_in + LPR * k, nvec - 1)];
#pragma unroll
        for (int k = 0; k < kRouteMaxK; ++k) s += lane_in + LPR * k < nvec ? L::sum(q[k]) : 0.f;
    }
    s = group_sum<LPR>(s);
    if (lane_in == 0 && c < C)
        __hip_atomic_store(&means[(long)b * C + c], s / (float)hw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every wave waits until its means stores are complete at device scope
    // before the barrier, so the ticket below is taken after all of them
    // (a device-scope fence would instead write back and invalidate the
    // whole L2 of the XCD, in every workgroup)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
        const unsigned t = __hip_atomic_fetch_add(&tickets[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = t == (unsigned)(S - 1);
    }
    __syncthreads();
    if (!is_last) return;  // uniform over the workgroup
    for (int i = tid; i < C; i += kSplitThreads)
        gsh[i] = __hip_atomic_load(&means[(long)b * C + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) __hip_atomic_store(&tickets[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    route_finish<kSplitThreads>(gsh, zsh, fc_w, fc_b, alpha, b, C, n, mode, temp, pre);
}

// lanes per plane for the split router: the fewest that keep a lane's loads
// within its per-plane limit, or 0 when a plane needs more than 64 lanes
int split_lpr(int nvec, int maxk) {
    int lpr = 1;
    while (lpr * maxk < nvec) lpr *= 2;
    return lpr <= 64 ? lpr : 0;
}

template <typename T, int VEC, bool EVEN16>
hipError_t launch_route_split_t(const T *x, const float *fc_w, const float *fc_b, float *alpha, float *means,
                                unsigned *tickets, int B, int C, int hw, int n, int mode, float temp,
                                hipStream_t s) {
    const int nvec = EVEN16 ? (hw + 7) / 8 : hw / VEC;
    const int lpr = split_lpr(nvec, EVEN16 ? kRouteMaxK16 : kRouteMaxK);
    const int S = ceil_div(C, kSplitThreads / lpr);
    const int x_bytes = EVEN16 ? (int)((long)B * C * hw * 2) : 0;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)(B * S)), dim3(kSplitThreads), 0, s, x, fc_w, fc_b, alpha, means,
                           tickets, C, hw, n, mode, temp, S, x_bytes);
        return hipGetLastError();
    };
    switch (lpr) {
    case 1: return go(route_split_kernel<T, VEC, 1, EVEN16>);
    case 2: return go(route_split_kernel<T, VEC, 2, EVEN16>);
    case 4: return go(route_split_kernel<T, VEC, 4, EVEN16>);
    case 8: return go(route_split_kernel<T, VEC, 8, EVEN16>);
    case 16: return go(route_split_kernel<T, VEC, 16, EVEN16>);
    case 32: return go(route_split_kernel<T, VEC, 32, EVEN16>);
    default: return go(route_split_kernel<T, VEC, 64, EVEN16>);
    }
}

hipError_t launch_route_fused16(const uint16_t *x, const float *fc_w, const float *fc_b, float *alpha, int B, int C,
                                int hw, int n, int mode, float temp, hipStream_t s) {
    const int nvec = (hw + 7) / 8;
    int lpr = 1;
    while (lpr * kRouteMaxK16 < nvec) lpr *= 2;
    const int x_bytes = (int)((long)B * C * hw * 2);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(B), dim3(kRouteThreads), 0, s, x, fc_w, fc_b, alpha, C, hw, n, mode, temp,
                           x_bytes);
        return hipGetLastError();
    };
    switch (lpr) {
    case 1: return go(route_fused16_kernel<1>);
    case 2: return go(route_fused16_kernel<2>);
    case 4: return go(route_fused16_kernel<4>);
    case 8: return go(route_fused16_kernel<8>);
    case 16: return go(route_fused16_kernel<16>);
    case 32: return go(route_fused16_kernel<32>);
    default: return go(route_fused16_kernel<64>);
    }
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

// The pooling kernel for bf16 planes of an even size that is not a multiple
// of 8 (14 x 14): 16-byte loads through a buffer descriptor over x (the last
// vector of a plane reads into the next plane, or past the tensor, where the
// read returns 0; its elements past the plane are left out of the sum), LPR
// lanes per plane with at most kGap16Loads loads each, all in flight before
// the first add.
constexpr int kGap16Loads = 4;
template <int LPR>
__global__ __launch_bounds__(kGapThreads) void gap16_kernel(const uint16_t *__restrict__ x, float *__restrict__ gap,
                                                            long rows, int hw, int x_bytes) {
    constexpr int kRowsPerBlock = kGapThreads / LPR;
    const int lane_in = threadIdx.x % LPR;
    const long row = (long)blockIdx.x * kRowsPerBlock + threadIdx.x / LPR;
    const bool active = row < rows;
    const long r = active ? row : rows - 1;
    const int nvec = (hw + 7) / 8;
    const int tail_words = (hw - 8 * (nvec - 1)) / 2;
    const uint64_t q = reinterpret_cast<uint64_t>(x);
    const uint64_t qs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)q) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(q >> 32)) << 32);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(qs), 0,
                                                      __builtin_amdgcn_readfirstlane(x_bytes), 0x00020000);
    const int base = (int)(r * hw * 2);  // bytes (x_bytes < 2^31)
    u32x4_t v[kGap16Loads];
#pragma unroll
    for (int k = 0; k < kGap16Loads; ++k)
        v[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                               rs, base + 16 * min(lane_in + LPR * k, nvec - 1), 0, 0));
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kGap16Loads; ++k) {
        const int vi = lane_in + LPR * k;
        const int words = vi < nvec - 1 ? 4 : (vi == nvec - 1 ? tail_words : 0);
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) t += j < words ? bf16_lo(w[j]) + bf16_hi(w[j]) : 0.f;
        s += t;
    }
    s = group_sum<LPR>(s);
    if (active && lane_in == 0) gap[row] = s / (float)hw;
}

// lanes per plane for gap16_kernel, or 0 when a plane needs more than 64
int gap16_lpr(int hw) {
    const int nvec = (hw + 7) / 8;
    int lpr = 1;
    while (lpr * kGap16Loads < nvec) lpr *= 2;
    return lpr <= 64 ? lpr : 0;
}

hipError_t launch_gap16(const uint16_t *x, float *gap, long rows, int hw, hipStream_t s) {
    const int lpr = gap16_lpr(hw);
    const int x_bytes = (int)(rows * hw * 2);
    auto go = [&](auto kern, int l) {
        const long blocks = (rows + (kGapThreads / l) - 1) / (kGapThreads / l);
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kGapThreads), 0, s, x, gap, rows, hw, x_bytes);
        return hipGetLastError();
    };
    switch (lpr) {
    case 1: return go(gap16_kernel<1>, 1);
    case 2: return go(gap16_kernel<2>, 2);
    case 4: return go(gap16_kernel<4>, 4);
    case 8: return go(gap16_kernel<8>, 8);
    case 16: return go(gap16_kernel<16>, 16);
    case 32: return go(gap16_kernel<32>, 32);
    default: return go(gap16_kernel<64>, 64);
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
// output attentions. Workgroup (e, j): chunk j of the heads' logits of
// examples 8 e .. 8 e + 7. A head with the softmax (its normalisation spans
// all its logits) is one chunk of up to 256 logits (four passes of 64 rows);
// a sigmoid head is cut into chunks of 64. Per pass of 64 logit rows and per
// tile of 128 channels, the rows of fc_w and the 8 examples' channel means
// are staged in LDS with coalesced loads; thread t then owns row t & 63 for
// examples 2 (t >> 6) and 2 (t >> 6) + 1 and walks the tile's channels in
// order (16-byte LDS reads), so each fc_w value serves 8 examples and every
// logit is one fixed-order sum. The nonlinearity runs after a barrier.
constexpr int kHeadsMax = 3;
constexpr int kHeadsEB = 8;    // examples per workgroup
constexpr int kHeadsCT = 128;  // channels per staged tile
constexpr int kHeadsWP = kHeadsCT + 4;  // padded row (16-byte reads of 64 rows on distinct banks)
struct RouteHeads {
    const float *w[kHeadsMax];
    const float *b[kHeadsMax];
    float *out[kHeadsMax];
    int n[kHeadsMax], mode[kHeadsMax], first[kHeadsMax + 1];  // first chunk of each head
    int heads;
};
__global__ __launch_bounds__(256) void route_heads_kernel(const float *__restrict__ gap, RouteHeads hp, int B,
                                                          int C, float temp) {
    __shared__ __attribute__((aligned(16))) float sW[64][kHeadsWP];
    __shared__ __attribute__((aligned(16))) float sG[kHeadsEB][kHeadsCT];
    __shared__ float z[kHeadsEB][256];
    const int b0 = blockIdx.x * kHeadsEB, j = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int h = 0;
    while (h + 1 < hp.heads && j >= hp.first[h + 1]) ++h;
    const int n = hp.n[h], mode = hp.mode[h];
    const int per = mode == 1 ? n : 64;
    const int i0 = (j - hp.first[h]) * per, cnt = min(per, n - i0);
    const float *W = hp.w[h];
    const int r = lane, e0 = 2 * wave;
    for (int rp = 0; rp < cnt; rp += 64) {  // passes of 64 logit rows
        float acc0 = 0.f, acc1 = 0.f;
        for (int c0 = 0; c0 < C; c0 += kHeadsCT) {
            // every load of the tile in flight before the first LDS store
            constexpr int kW4 = 64 * kHeadsCT / 4 / 256;  // 16-byte pieces of fc_w per thread
            f32x4_t wq[kW4];
            f32x4_t gq;
            if ((C & 3) == 0) {
#pragma unroll
                for (int i = 0; i < kW4; ++i) {
                    const int idx = tid + 256 * i, row = idx / (kHeadsCT / 4), c = 4 * (idx % (kHeadsCT / 4));
                    const bool in = rp + row < cnt && c0 + c < C;
                    wq[i] = in ? *reinterpret_cast<const f32x4_t *>(&W[(long)(i0 + rp + row) * C + c0 + c])
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
                {
                    const int e = tid / (kHeadsCT / 4), c = 4 * (tid % (kHeadsCT / 4));
                    gq = (b0 + e < B && c0 + c < C) ? *reinterpret_cast<const f32x4_t *>(&gap[(long)(b0 + e) * C + c0 + c])
                                                    : f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            } else {
#pragma unroll
                for (int i = 0; i < kW4; ++i) {
                    const int idx = tid + 256 * i, row = idx / (kHeadsCT / 4), c = 4 * (idx % (kHeadsCT / 4));
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        wq[i][k] = (rp + row < cnt && c0 + c + k < C) ? W[(long)(i0 + rp + row) * C + c0 + c + k] : 0.f;
                }
                const int e = tid / (kHeadsCT / 4), c = 4 * (tid % (kHeadsCT / 4));
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    gq[k] = (b0 + e < B && c0 + c + k < C) ? gap[(long)(b0 + e) * C + c0 + c + k] : 0.f;
            }
            __syncthreads();  // the previous tile's reads are done
#pragma unroll
            for (int i = 0; i < kW4; ++i) {
                const int idx = tid + 256 * i, row = idx / (kHeadsCT / 4), c = 4 * (idx % (kHeadsCT / 4));
                *reinterpret_cast<f32x4_t *>(&sW[row][c]) = wq[i];
            }
            *reinterpret_cast<f32x4_t *>(&sG[tid / (kHeadsCT / 4)][4 * (tid % (kHeadsCT / 4))]) = gq;
            __syncthreads();
#pragma unroll 4
            for (int c = 0; c < kHeadsCT; c += 4) {
                const f32x4_t wv = *reinterpret_cast<const f32x4_t *>(&sW[r][c]);
                const f32x4_t g0 = *reinterpret_cast<const f32x4_t *>(&sG[e0][c]);
                const f32x4_t g1 = *reinterpret_cast<const f32x4_t *>(&sG[e0 + 1][c]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    acc0 = fmaf(wv[k], g0[k], acc0);
                    acc1 = fmaf(wv[k], g1[k], acc1);
                }
            }
        }
        if (rp + r < cnt) {
            const float bias = hp.b[h] ? hp.b[h][i0 + rp + r] : 0.f;
            z[e0][rp + r] = acc0 + bias;
            z[e0 + 1][rp + r] = acc1 + bias;
        }
    }
    __syncthreads();
    if (mode == 0) {
        for (int e = 0; e < kHeadsEB && b0 + e < B; ++e) {
            float *out = hp.out[h] + (long)(b0 + e) * n + i0;
            for (int i = tid; i < cnt; i += 256) {
                const float v = z[e][i];
                float a;
                if (v >= 0.f) {
                    a = 1.f / (1.f + expf(-v));
                } else {
                    const float ev = expf(v);
                    a = ev / (1.f + ev);
                }
                out[i] = a;
            }
        }
    } else {
        // softmax(z / T) over the head's logits, one wave per example
        for (int e = wave; e < kHeadsEB && b0 + e < B; e += 4) {
            float *out = hp.out[h] + (long)(b0 + e) * n + i0;
            float m = -INFINITY;
            for (int i = lane; i < cnt; i += 64) m = fmaxf(m, z[e][i] / temp);
            m = wave_max(m);
            float sum = 0.f;
            for (int i = lane; i < cnt; i += 64) sum += expf(z[e][i] / temp - m);
            sum = wave_sum(sum);
            for (int i = lane; i < cnt; i += 64) out[i] = expf(z[e][i] / temp - m) / sum;
        }
    }
}

}  // namespace

static_assert(kMaxJ * 64 >= 256, "route kernel covers n <= 256");
static_assert(kHeadsEB * kHeadsCT == 4 * 256, "one 16-byte piece of channel means per thread and tile");

namespace {

// Load variant of the split router for this layer: 8 = 16-byte vectors of 8
// bf16, 16 = 16-byte loads over even-sized bf16 planes, 4 / 1 = vectors of 4
// or single elements (either dtype); 0 when a plane is too large for one
// pass of at most 64 lanes.
int split_variant(const Geom &g) {
    const int hw = g.H * g.W;
    if (g.bf16) {
        if (hw % 8 == 0) return split_lpr(hw / 8, kRouteMaxK) ? 8 : 0;
        if (hw % 2 == 0 && (long)g.B * g.Cin * hw * 2 < (1L << 31) - 64 && split_lpr((hw + 7) / 8, kRouteMaxK16))
            return 16;
    }
    if (hw % 4 == 0) return split_lpr(hw / 4, kRouteMaxK) ? 4 : 0;
    return split_lpr(hw, kRouteMaxK) ? 1 : 0;
}

bool route_split(const Geom &g) {
    return g.B < kRouteSplitMaxB && g.Cin <= kRouteMaxC && split_variant(g) != 0;
}

}  // namespace

bool route_single_kernel(const Geom &g) {
    // planes up to 64 lanes x kRouteMaxK vectors (bf16: 8192 elements with 16-byte loads)
    return g.B >= kRouteSplitMaxB && g.Cin <= kRouteMaxC && g.H * g.W <= 64 * kRouteMaxK;
}

size_t route_workspace_bytes(const Geom &g) {
    if (route_single_kernel(g)) return 0;
    const size_t means = (size_t)g.B * g.Cin * sizeof(float);
    if (route_split(g)) return kRouteTicketBytes(g.B) + means;
    return means;
}

hipError_t launch_route(const Geom &g, const void *x, const float *fc_w, const float *fc_b,
                        int mode, float temperature, void *workspace, float *alpha,
                        hipStream_t stream) {
    const long rows = (long)g.B * g.Cin;
    const int hw = g.H * g.W;
    const float tp = mode == 1 ? temperature : 1.0f;
    float *gap = static_cast<float *>(workspace);
    if (route_single_kernel(g)) {
        if (g.bf16) {
            const uint16_t *xb = static_cast<const uint16_t *>(x);
            if (hw % 8 == 0) return launch_route_fused_vec<uint16_t, 8>(xb, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
            if (hw % 2 == 0 && hw <= 8 * 64 * kRouteMaxK16 && (long)g.B * g.Cin * hw * 2 < (1L << 31) - 64)
                return launch_route_fused16(xb, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
            if (hw % 4 == 0) return launch_route_fused_vec<uint16_t, 4>(xb, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
            return launch_route_fused_vec<uint16_t, 1>(xb, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
        }
        const float *xf = static_cast<const float *>(x);
        if (hw % 4 == 0) return launch_route_fused_vec<float, 4>(xf, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
        return launch_route_fused_vec<float, 1>(xf, fc_w, fc_b, alpha, g.B, g.Cin, hw, g.n, mode, tp, stream);
    }
    if (route_split(g)) {
        // workspace: the tickets, then the channel means
        unsigned *tickets = static_cast<unsigned *>(workspace);
        float *means = reinterpret_cast<float *>(static_cast<char *>(workspace) + kRouteTicketBytes(g.B));
        const int var = split_variant(g);
        if (g.bf16) {
            const uint16_t *xb = static_cast<const uint16_t *>(x);
            if (var == 8) return launch_route_split_t<uint16_t, 8, false>(xb, fc_w, fc_b, alpha, means, tickets, g.B, g.Cin, hw, g.n, mode, tp, stream);
            if (var == 16) return launch_route_split_t<uint16_t, 8, true>(xb, fc_w, fc_b, alpha, means, tickets, g.B, g.Cin, hw, g.n, mode, tp, stream);
            if (var == 4) return launch_route_split_t<uint16_t, 4, false>(xb, fc_w, fc_b, alpha, means, tickets, g.B, g.Cin, hw, g.n, mode, tp, stream);
            return launch_route_split_t<uint16_t, 1, false>(xb, fc_w, fc_b, alpha, means, tickets, g.B, g.Cin, hw, g.n, mode, tp, stream);
        }
        const float *xf = static_cast<const float *>(x);
        if (var == 4) return launch_route_split_t<float, 4, false>(xf, fc_w, fc_b, alpha, means, tickets, g.B, g.Cin, hw, g.n, mode, tp, stream);
        return launch_route_split_t<float, 1, false>(xf, fc_w, fc_b, alpha, means, tickets, g.B, g.Cin, hw, g.n, mode, tp, stream);
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
        if (hw % 2 == 0 && gap16_lpr(hw) && rows * hw * 2 < (1L << 31) - 64)
            return launch_gap16(xb, gap, rows, hw, stream);
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
    hipLaunchKernelGGL(route_heads_kernel, dim3((unsigned)ceil_div(g.B, kHeadsEB), (unsigned)chunks), dim3(256), 0,
                       stream, gap, hp, g.B, g.Cin, temperature);
    return hipGetLastError();
}

}  // namespace dynconv
