// Pieces shared by the two MFMA convolution sources (conv_fused.hip and
// conv_premix.hip): the kernel argument block, the XCD-aware tile mapping,
// LDS and epilogue helpers, and the launch-side argument set-up.
//
// For one example b the convolution is a GEMM (CondConv: Conditionally
// Parameterized Convolutions, abstract: one ordinary convolution per example
// with that example's own kernel):
//   Y_b[p][o] = sum_k X_b[p][k] * W_b[k][o],  p = output position (r, s),
//   o = output channel, k = (tap t = (u, v), input channel c),
// contracted in chunks of kChunk input channels.
#pragma once

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

constexpr int kPosStride = 40;  // bf16 per LDS position (32 channels + pad)
constexpr int kChunk = 32;      // input channels per K chunk
constexpr int kLdsBudget = 160 * 1024;

struct ConvArgs {
    int B, Cin, H, W, Cout, KH, KW, stride, pad, Ho, Wo, P, KT, Cin_pad, n;
    int ncols;      // LDS tile columns = W + 2 * pad (column j <-> input column j - pad)
    int tile_rows;  // LDS tile rows
    int n_ptiles, n_otiles, n_btiles;
    long x_bstride;  // Cin * H * W
};

// Blocks are dispatched round-robin over the 8 XCDs: block i runs on XCD
// i % 8. Give each XCD a contiguous range of logical tile ids so that tiles
// sharing data (same example, or same expert slice) share one L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
    if (total % 8 != 0) return id;
    return (id % 8) * (total / 8) + id / 8;
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xffff0000u);
}

__device__ __forceinline__ void zero_lds(uint16_t *p, int elems, int tid, int nthreads) {
    u32x4_t z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < elems / 8; i += nthreads) reinterpret_cast<u32x4_t *>(p)[i] = z;
}

// D fragment -> y: lane holds positions pbase..pbase+3 of channel o.
__device__ __forceinline__ void store_frag(uint16_t *__restrict__ y, const ConvArgs &a, int b,
                                           int o, int pbase, const f32x4_t &d) {
    if (o >= a.Cout || pbase >= a.P) return;
    uint16_t *yo = y + ((long)b * a.Cout + o) * a.P;
    if ((a.P & 3) == 0 && pbase + 3 < a.P) {
        u32x2_t v;
        v.x = pack_bf16x2(d[0], d[1]);
        v.y = pack_bf16x2(d[2], d[3]);
        *reinterpret_cast<u32x2_t *>(yo + pbase) = v;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (pbase + j < a.P) yo[pbase + j] = f32_to_bf16(d[j]);
    }
}

// Element offset of 16-byte channel granule g (0..3) of tile position q:
// 64-byte positions, granules permuted by bits 1..2 of q.
__device__ __forceinline__ int swz(int q, int g) {
    return q * 32 + ((g ^ ((q >> 1) & 3)) << 3);
}

inline ConvArgs base_args(const Geom &g) {
    ConvArgs a{};
    a.B = g.B; a.Cin = g.Cin; a.H = g.H; a.W = g.W; a.Cout = g.Cout;
    a.KH = g.KH; a.KW = g.KW; a.stride = g.stride; a.pad = g.pad;
    a.Ho = g.Ho; a.Wo = g.Wo; a.P = g.P; a.KT = g.KT; a.Cin_pad = g.Cin_pad; a.n = g.n;
    a.ncols = g.W + 2 * g.pad;
    a.x_bstride = (long)g.Cin * g.H * g.W;
    return a;
}

template <typename K>
hipError_t set_lds(K kern, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace
}  // namespace dynconv
