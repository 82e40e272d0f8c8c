// The dynamic convolution evaluated only at gated positions (Dynamic
// Convolutions: Exploiting Spatial Sparsity for Faster Inference, abstract:
// a small gating branch picks the spatial positions a residual block
// evaluates, run with a gather-scatter approach). The gate arrives as a mask
// over the output positions; for example b:
//   y[b,o,p] = (residual ? x[b,o,p] : 0) + [mask[b,p] != 0] * conv(x_b, W_b)[o,p]
// with W_b premixed in the convolution's layout wt[b][t][o][cp] (bf16).
//   1. compact_mask_kernel lists each example's active positions in
//      increasing order (a block prefix sum: deterministic);
//   2. fill_sparse_kernel writes the inactive value (0, or x for a residual
//      block) everywhere (y never overlaps x: the gathers read x around
//      positions that other workgroups write);
//   3. nhwc_kernel copies x channel-innermost, xt[b][h*W + w][cp] (Cin
//      padded to a multiple of 32 with zeros), so that 8 channels of one
//      position are one 16-byte load;
//   4. conv_sparse_kernel gathers the im2col rows of 64 active positions,
//      multiplies them with 64 output channels of W_b on
//      v_mfma_f32_32x32x16_bf16 and scatters the results back (adding them
//      to the residual in float32, one rounding).
#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

// Workgroup per example: idx[b][k] = k-th active position, count[b] = their number.
__global__ __launch_bounds__(256) void compact_mask_kernel(const uint8_t *__restrict__ mask, int *__restrict__ idx,
                                                           int *__restrict__ count, int P) {
    __shared__ int s_w[4];
    const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint8_t *m = mask + (long)b * P;
    int *out = idx + (long)b * P;
    int base = 0;
    for (int p0 = 0; p0 < P; p0 += 256) {
        const int p = p0 + tid;
        const int on = (p < P && m[p] != 0) ? 1 : 0;
        // inclusive scan within the wave, then across the 4 waves
        const uint64_t bal = __ballot(on);
        const int below = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        if (lane == 63) s_w[wave] = below + on;
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += s_w[w];
        if (on) out[off + below] = p;
        base += (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
        __syncthreads();
    }
    if (tid == 0) count[b] = base;
}

// y = residual ? x : 0 over all of y (8 bf16 per thread, element by element
// in a partial last group).
__global__ __launch_bounds__(256) void fill_sparse_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ y,
                                                          long total, int residual) {
    const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= total) return;
    if (i + 8 <= total) {
        const u32x4_t v = residual ? *reinterpret_cast<const u32x4_t *>(x + i) : u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t *>(y + i) = v;
    } else {
        for (long j = i; j < total; ++j) y[j] = residual ? x[j] : (uint16_t)0;
    }
}

// x [B][Cin][HW] -> xt [B][HW][Cin_pad] through a 64 x 64 LDS tile: reads
// along positions and writes 8-channel vectors, both coalesced.
__global__ __launch_bounds__(256) void nhwc_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ xt, int Cin,
                                                   int Cin_pad, int HW) {
    __shared__ uint16_t s_t[64][66];
    const int b = blockIdx.z, p0 = blockIdx.x * 64, c0 = blockIdx.y * 64, tid = threadIdx.x;
    for (int e = tid; e < 64 * 64; e += 256) {
        const int c = e >> 6, pp = e & 63;
        s_t[c][pp] = (c0 + c < Cin && p0 + pp < HW) ? x[((long)b * Cin + c0 + c) * HW + p0 + pp] : (uint16_t)0;
    }
    __syncthreads();
    for (int v = tid; v < 512; v += 256) {
        const int pp = v >> 3, cv = (v & 7) * 8;
        if (p0 + pp < HW && c0 + cv < Cin_pad) {
            u32x4_t w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = (uint32_t)s_t[cv + 2 * j][pp] | ((uint32_t)s_t[cv + 2 * j + 1][pp] << 16);
            *reinterpret_cast<u32x4_t *>(xt + ((long)b * HW + p0 + pp) * Cin_pad + c0 + cv) = w;
        }
    }
}

struct SparseArgs {
    int B, Cin, H, W, Cout, KW, KT, stride, pad, Wo, P, Cin_pad, residual;
};

// Workgroup (position tile, 64 output channels, example): wave w owns active
// positions 64 tile + 32 (w & 1) .. + 31 (MFMA columns) and output channels
// 64 ot + 32 (w >> 1) .. + 31 (MFMA rows). A lane's position fragment is 8 input
// channels of its position at one tap (one 16-byte load from the
// channel-innermost copy, zero outside the image); its B fragment is 8
// consecutive input channels of one output channel's W_b row (one 16-byte
// load).
__global__ __launch_bounds__(256) void conv_sparse_kernel(const uint16_t *__restrict__ xt, const uint16_t *__restrict__ wt,
                                                          const int *__restrict__ idx, const int *__restrict__ count,
                                                          uint16_t *__restrict__ y, SparseArgs a) {
    const int b = blockIdx.z, ot = blockIdx.y, pt = blockIdx.x;
    const int cnt = count[b];
    if (pt * 64 >= cnt) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;
    const int mh = wave & 1, nh = wave >> 1;
    const int ka = pt * 64 + 32 * mh + l32;
    const bool a_ok = ka < cnt;
    const int pa = a_ok ? idx[(long)b * a.P + ka] : 0;
    const int r = pa / a.Wo, s = pa - r * a.Wo;
    const int o = ot * 64 + 32 * nh + l32;
    const bool o_ok = o < a.Cout;
    const long hw = (long)a.H * a.W;
    const uint16_t *xb = xt + (long)b * hw * a.Cin_pad;
    const uint16_t *wb = wt + (long)b * a.KT * a.Cout * a.Cin_pad + (long)(o_ok ? o : 0) * a.Cin_pad;
    f32x16_t acc = {};
    for (int t = 0; t < a.KT; ++t) {
        const int u = t / a.KW, v = t - u * a.KW;
        const int hh = r * a.stride - a.pad + u, ww = s * a.stride - a.pad + v;
        const bool in = a_ok && hh >= 0 && hh < a.H && ww >= 0 && ww < a.W;
        const uint16_t *xp = xb + (in ? ((long)hh * a.W + ww) * a.Cin_pad : 0);
        const uint16_t *wp = wb + (long)t * a.Cout * a.Cin_pad;
        // 64 channels per step: all fragment loads of the step are issued
        // before its MFMAs (Cin_pad is a multiple of 32)
        for (int c0 = 0; c0 < a.Cin_pad; c0 += 64) {
            u32x4_t av[4], bv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cb = c0 + 16 * j + 8 * kg;
                const bool cj = c0 + 16 * j < a.Cin_pad;
                av[j] = (in && cj) ? *reinterpret_cast<const u32x4_t *>(xp + cb) : u32x4_t{0u, 0u, 0u, 0u};
                bv[j] = (o_ok && cj) ? *reinterpret_cast<const u32x4_t *>(wp + cb) : u32x4_t{0u, 0u, 0u, 0u};
            }
            // W_b rows as the A operand, positions as the B operand: the
            // result's columns are positions, so a lane stores one position
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bv[j]),
                                                               __builtin_bit_cast(bf16x8_t, av[j]), acc, 0, 0, 0);
        }
    }
    // D(lane, 4j + q) = output channel 64 ot + 32 nh + 8j + 4 kg + q, the lane's
    // position pa: lanes 0-31 of a store cover 32 consecutive active
    // positions of one channel plane
    if (!a_ok) return;
    uint16_t *yp = y + (long)b * a.Cout * a.P + pa;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int oo = ot * 64 + 32 * nh + 8 * j + 4 * kg + q;
            if (oo < a.Cout) {
                const long off = (long)oo * a.P;
                const float base = a.residual ? bf16_to_f32(yp[off]) : 0.f;
                yp[off] = f32_to_bf16(base + acc[4 * j + q]);
            }
        }
}

}  // namespace

// scratch: compacted positions and counts, then the channel-innermost x
size_t sparse_index_bytes(const Geom &g) {
    const size_t idx = ((size_t)g.B * g.P + g.B) * sizeof(int);
    return (idx + 255) / 256 * 256 + (size_t)g.B * g.H * g.W * g.Cin_pad * sizeof(uint16_t);
}

hipError_t launch_conv_sparse(const Geom &g, const uint16_t *x, const uint16_t *wt, const uint8_t *mask, int residual,
                              int *idx, uint16_t *y, hipStream_t stream) {
    int *count = idx + (long)g.B * g.P;
    uint16_t *xt = reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(idx) +
                                                (((size_t)g.B * g.P + g.B) * sizeof(int) + 255) / 256 * 256);
    hipLaunchKernelGGL(compact_mask_kernel, dim3((unsigned)g.B), dim3(256), 0, stream, mask, idx, count, g.P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int hw = g.H * g.W;
    hipLaunchKernelGGL(nhwc_kernel, dim3((unsigned)ceil_div(hw, 64), (unsigned)ceil_div(g.Cin_pad, 64), (unsigned)g.B),
                       dim3(256), 0, stream, x, xt, g.Cin, g.Cin_pad, hw);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        const long total = (long)g.B * g.Cout * g.P;
        hipLaunchKernelGGL(fill_sparse_kernel, dim3((unsigned)(((total + 7) / 8 + 255) / 256)), dim3(256), 0, stream,
                           x, y, total, residual);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    SparseArgs a;
    a.B = g.B; a.Cin = g.Cin; a.H = g.H; a.W = g.W; a.Cout = g.Cout; a.KW = g.KW; a.KT = g.KT;
    a.stride = g.stride; a.pad = g.pad; a.Wo = g.Wo; a.P = g.P; a.Cin_pad = g.Cin_pad; a.residual = residual;
    const dim3 grid((unsigned)ceil_div(g.P, 64), (unsigned)ceil_div(g.Cout, 64), (unsigned)g.B);
    hipLaunchKernelGGL(conv_sparse_kernel, grid, dim3(256), 0, stream, xt, wt, idx, count, y, a);
    return hipGetLastError();
}

}  // namespace dynconv
