// Mixing for banks of many experts (bf16, n > 16 in the forward, n > 64 in
// dynconv_mix). KernelWarehouse (KernelWarehouse: Rethinking the Design of
// Dynamic Convolution, abstract) pushes the expert count past 100, where
// W_b = sum_i alpha[b,i] E_i is a real GEMM, [examples x n] . [n x weights],
// with n as the reduction dimension. mix_mfma_wide_kernel walks that
// dimension in chunks of 32 experts on v_mfma_f32_32x32x16_bf16:
//   * a workgroup owns kMixWW consecutive weights and 32*MT examples;
//   * each chunk's [32 experts x kMixWW weights] slice is staged in LDS
//     (double-buffered, the next chunk's loads in flight during the current
//     chunk's MFMAs) and read as A fragments with LDS transpose reads, two
//     groups of 16 experts per chunk;
//   * the chunk's attentions are split into three bf16 parts (24 bits, a
//     float32 significand), so the exact products summed in fp32 equal a
//     float32 mix before its one bf16 rounding;
//   * results leave through LDS as 16-byte row stores.
// The weights are whatever order the bank is stored in: the natural layout
// for dynconv_mix, or the convolution's [t][o][cp] order (pack_wide_kernel)
// for the forward, which then writes W_b straight into the premix layout.
#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

constexpr int kMixWW = 256;                // weights per workgroup (4 waves x 64)
constexpr int kMixWPitch = kMixWW + 8;     // bf16 per staged output row
typedef short s16x4_w_t __attribute__((ext_vector_type(4)));

constexpr int kWideChunk = 32;  // experts per staged chunk (two MFMA groups of 16)
template <int MT>
__global__ __launch_bounds__(256) void mix_mfma_wide_kernel(const float *__restrict__ alpha,
                                                            const uint16_t *__restrict__ experts,
                                                            uint16_t *__restrict__ mixed, int B, int n, long wsize) {
    constexpr int KC = kWideChunk;
    constexpr int NV = KC * (kMixWW / 8) / 256;  // 16-byte staging vectors per thread per chunk
    __shared__ __attribute__((aligned(16))) uint16_t s_e[2][KC][kMixWW];
    __shared__ __attribute__((aligned(16))) uint16_t s_o[32 * MT][kMixWPitch];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const long w0 = (long)blockIdx.x * kMixWW;
    const int bc0 = blockIdx.y * 32 * MT;
    const int nchunks = ceil_div(n, KC);
    // staging: KC rows x 32 vectors of 16 bytes; loads are clamped (always in
    // bounds), the LDS stores masked
    auto load = [&](int ch, u32x4_t (&q)[NV]) {
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int v = tid + 256 * it, k = v >> 5, c = v & 31;
            const long w = min(w0 + 8 * c, wsize - 8);
            q[it] = *reinterpret_cast<const u32x4_t *>(experts + (long)min(KC * ch + k, n - 1) * wsize + w);
        }
    };
    auto store = [&](int buf, int ch, const u32x4_t (&q)[NV]) {
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int v = tid + 256 * it, k = v >> 5, c = v & 31;
            const bool in = KC * ch + k < n && w0 + 8 * c < wsize;
            *reinterpret_cast<u32x4_t *>(&s_e[buf][k][8 * c]) = in ? q[it] : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    // this lane's attentions for a chunk: example bc0 + 32 mt + l32, experts
    // KC ch + 16 g + 8 lh + (0..7)
    auto load_alpha = [&](int ch, float (&av)[MT][2][8]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int b = bc0 + 32 * mt + l32;
            const float *ab = alpha + (long)min(b, B - 1) * n;
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int k = KC * ch + 16 * g + 8 * lh + q;
                    av[mt][g][q] = (b < B && k < n) ? ab[k] : 0.f;
                }
        }
    };
    f32x16_t acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;
    u32x4_t q[NV];
    float av[MT][2][8];
    load(0, q);
    load_alpha(0, av);
    store(0, 0, q);
    const int si = lane & 15;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        float avn[MT][2][8];
        if (ch + 1 < nchunks) {
            load(ch + 1, q);
            load_alpha(ch + 1, avn);
        }
        __syncthreads();  // chunk ch is in s_e[buf]; the reads of s_e[buf ^ 1] are done
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            // expert operands (A: rows = weights): experts 16 g + 8 lh + (0..7)
            // of the chunk, weight 64 wave + 32 nt + l32. Within a group of 16
            // lanes, the LDS transpose read gives lane i element i & 3 of the 8
            // bytes that lanes 4 j + (i >> 2) address, as its element j; lane
            // s = 4 j + r addresses expert row 16 g + 8 lh + 4 h + j at weights
            // wg + 4 r .. + 3, so lane i gets experts 16 g + 8 lh + 4 h + (0..3)
            // of weight wg + i.
            bf16x8_t ef[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int wg = 64 * wave + 32 * nt + 16 * ((lane >> 4) & 1);
                s16x4_w_t h[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_w_t *)(
                        &s_e[buf][16 * g + 8 * lh + 4 * hh + (si >> 2)][wg + 4 * (si & 3)]));
                const u32x2_t lo = __builtin_bit_cast(u32x2_t, h[0]), hi = __builtin_bit_cast(u32x2_t, h[1]);
                ef[nt] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
            }
            // attention operands (B: columns = examples), three exact bf16 parts
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint32_t pw[3][4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    uint16_t p2[3][2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        float r = av[mt][g][2 * jj + e];
#pragma unroll
                        for (int part = 0; part < 3; ++part) {
                            p2[part][e] = f32_to_bf16(r);
                            r -= bf16_to_f32(p2[part][e]);  // exact
                        }
                    }
#pragma unroll
                    for (int part = 0; part < 3; ++part)
                        pw[part][jj] = (uint32_t)p2[part][0] | ((uint32_t)p2[part][1] << 16);
                }
#pragma unroll
                for (int part = 2; part >= 0; --part) {  // small parts first
                    const bf16x8_t ap =
                        __builtin_bit_cast(bf16x8_t, u32x4_t{pw[part][0], pw[part][1], pw[part][2], pw[part][3]});
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[nt], ap, acc[mt][nt], 0, 0, 0);
                }
            }
        }
        if (ch + 1 < nchunks) {
            store(buf ^ 1, ch + 1, q);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int g = 0; g < 2; ++g)
#pragma unroll
                    for (int k = 0; k < 8; ++k) av[mt][g][k] = avn[mt][g][k];
        }
    }
    // weights as the rows: D(lane, 4 j + r) = weight 64 wave + 32 nt + 8 j + 4 lh + r,
    // example 32 mt + l32: 4 consecutive weights of one W_b row (one 8-byte LDS write)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x2_t *>(&s_o[32 * mt + l32][64 * wave + 32 * nt + 8 * j + 4 * lh]) =
                    u32x2_t{pack_bf16x2(acc[mt][nt][4 * j], acc[mt][nt][4 * j + 1]),
                            pack_bf16x2(acc[mt][nt][4 * j + 2], acc[mt][nt][4 * j + 3])};
    __syncthreads();
    constexpr int kRowVec = kMixWW / 8;
#pragma unroll
    for (int it = 0; it < 32 * MT * kRowVec / 256; ++it) {
        const int v = tid + 256 * it;
        const int r = v / kRowVec, c = v - r * kRowVec;
        const int b = bc0 + r;
        const long w = w0 + 8 * c;
        if (b < B && w < wsize)
            *reinterpret_cast<u32x4_t *>(mixed + (long)b * wsize + w) = *reinterpret_cast<const u32x4_t *>(&s_o[r][8 * c]);
    }
}

// Natural bank [n][Cout][Cin][KT] -> the convolution's weight order
// [n][KT][Cout][Cin_pad] (zeros for input channels past Cin). Workgroup
// (i, o) reads the contiguous Cin x KT block of expert i, output channel o,
// into LDS and writes it back as KT rows of Cin_pad channels, both sides
// coalesced.
__global__ __launch_bounds__(256) void pack_wide_kernel(const uint16_t *__restrict__ src, uint16_t *__restrict__ dst,
                                                        int Cout, int Cin, int Cin_pad, int KT) {
    extern __shared__ uint16_t s_blk[];
    const long io = blockIdx.x;  // i * Cout + o
    const long i = io / Cout;
    const int o = (int)(io - i * Cout);
    const int m = Cin * KT;
    const uint16_t *sp = src + io * m;
    for (int e = threadIdx.x; e < m; e += 256) s_blk[e] = sp[e];
    __syncthreads();
    for (int e = threadIdx.x; e < KT * Cin_pad; e += 256) {
        const int t = e / Cin_pad, cp = e - t * Cin_pad;
        dst[((i * KT + t) * Cout + o) * Cin_pad + cp] = cp < Cin ? s_blk[cp * KT + t] : (uint16_t)0;
    }
}

}  // namespace

bool mix_wide_supported(long wsize) { return wsize >= 8 && wsize % 8 == 0; }

hipError_t launch_mix_wide(const Geom &g, long wsize, const float *alpha, const uint16_t *experts, uint16_t *mixed,
                           hipStream_t stream) {
    if (!mix_wide_supported(wsize)) return hipErrorInvalidValue;
    const unsigned tiles = (unsigned)((wsize + kMixWW - 1) / kMixWW);
    // 64 examples per workgroup only when the grid still has four workgroups per CU
    if (g.B > 32 && (long)tiles * ceil_div(g.B, 64) >= 1024)
        hipLaunchKernelGGL(mix_mfma_wide_kernel<2>, dim3(tiles, (unsigned)ceil_div(g.B, 64)), dim3(256), 0, stream,
                           alpha, experts, mixed, g.B, g.n, wsize);
    else
        hipLaunchKernelGGL(mix_mfma_wide_kernel<1>, dim3(tiles, (unsigned)ceil_div(g.B, 32)), dim3(256), 0, stream,
                           alpha, experts, mixed, g.B, g.n, wsize);
    return hipGetLastError();
}

size_t wide_bank_bytes(const Geom &g) { return (size_t)g.n * g.KT * g.Cout * g.Cin_pad * sizeof(uint16_t); }

bool pack_wide_supported(const Geom &g) { return (long)g.Cin * g.KT * 2 <= 64 * 1024; }

hipError_t launch_pack_wide(const Geom &g, const uint16_t *experts, uint16_t *wide, hipStream_t stream) {
    if (!pack_wide_supported(g)) return hipErrorInvalidValue;
    const size_t lds = (size_t)g.Cin * g.KT * sizeof(uint16_t);
    hipLaunchKernelGGL(pack_wide_kernel, dim3((unsigned)((long)g.n * g.Cout)), dim3(256), lds, stream, experts, wide,
                       g.Cout, g.Cin, g.Cin_pad, g.KT);
    return hipGetLastError();
}

}  // namespace dynconv
