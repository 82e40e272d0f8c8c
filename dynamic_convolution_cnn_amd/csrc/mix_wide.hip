// Mixing for banks of many experts (bf16, n > 16 in the forward, n > 64 in
// dynconv_mix). KernelWarehouse (KernelWarehouse: Rethinking the Design of
// Dynamic Convolution, abstract) pushes the expert count past 100, where
// W_b = sum_i alpha[b,i] E_i is a real GEMM, [examples x n] . [n x weights],
// with n as the reduction dimension. mix_mfma_wide_kernel walks that
// dimension in chunks of 32 experts on v_mfma_f32_32x32x16_bf16:
//   * a workgroup owns kMixWW consecutive weights and 32*MT examples;
//   * each chunk's [32 experts x kMixWW weights] slice is staged in LDS
//     (double-buffered, the next two chunks' loads in flight during the
//     current chunk's MFMAs) and read as A fragments with LDS transpose
//     reads, two groups of 16 experts per chunk;
//   * the chunk's attentions of the workgroup's 32*MT examples arrive with
//     coalesced 16-byte loads and are split once, by the thread that loaded
//     them, into three bf16 parts (24 bits, a float32 significand) staged in
//     LDS beside the expert slice, so the exact products summed in fp32
//     equal a float32 mix before its one bf16 rounding;
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
constexpr int kWideDepth = 2;   // chunks in flight per workgroup of 32 examples (3 costs a wave per SIMD)
constexpr long kWideMaxW = 1L << 27;  // weights per expert: 8 rows of them stay under 2^31 bytes

// A16: n is a multiple of 4 and alpha 16-byte aligned (attention rows load as
// 16-byte vectors). DEPTH: chunks in flight.
template <int MT, bool A16, int DEPTH>
__global__ __launch_bounds__(256) void mix_mfma_wide_kernel(const float *__restrict__ alpha,
                                                            const uint16_t *__restrict__ experts,
                                                            uint16_t *__restrict__ mixed, int B, int n, long wsize) {
    constexpr int KC = kWideChunk;
    constexpr int NV = KC * (kMixWW / 8) / 256;  // 16-byte staging vectors per thread per chunk
    __shared__ __attribute__((aligned(16))) uint16_t s_e[2][KC][kMixWW];
    // the output rows share their storage with the attentions of the
    // workgroup's examples as three bf16 parts, [buffer][part][example][expert]
    // (rows padded by 8 against bank conflicts of the 16-byte reads), which
    // are dead once the last chunk is done
    __shared__ __attribute__((aligned(16))) union {
        uint16_t o[32 * MT][kMixWPitch];
        uint16_t a[2][3][32 * MT][KC + 8];
    } s_u;
    auto &s_o = s_u.o;
    auto &s_a = s_u.a;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const long w0 = (long)blockIdx.x * kMixWW;
    const int bc0 = blockIdx.y * 32 * MT;
    const int nchunks = ceil_div(n, KC);
    // staging: KC rows x 32 vectors of 16 bytes. Round it covers expert rows
    // KC ch + 8 it + (0..7) through a buffer descriptor over just those rows
    // that exist, so rows past n (including whole chunks past the end, which
    // the two-deep prefetch asks for) read as zeros without touching memory.
    // Columns are clamped: a tile's weights past wsize hold copies of real
    // weights and only feed output rows that are never written.
    const uint32_t lane_off =
        (uint32_t)(((tid >> 5) * wsize + min(w0 + 8 * (tid & 31), wsize - 8)) * (long)sizeof(uint16_t));
    auto load = [&](int ch, u32x4_t (&q)[NV]) {
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int row0 = min(KC * ch + 8 * it, n), rows = min(8, n - row0);
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t *>(experts + (long)row0 * wsize), 0, (int)(rows * wsize * (long)sizeof(uint16_t)),
                0x00020000);
            q[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, 0, 0));
        }
    };
    auto store = [&](int buf, const u32x4_t (&q)[NV]) {
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int v = tid + 256 * it, k = v >> 5, c = v & 31;
            *reinterpret_cast<u32x4_t *>(&s_e[buf][k][8 * c]) = q[it];
        }
    };
    // the chunk's attentions, 32 MT examples x KC experts: coalesced 16-byte
    // loads (thread t: example t / 8 (+ 32 per round), experts 4 (t % 8) ..
    // + 3; clamped). Each thread splits its four into three exact bf16 parts
    // (24 bits, a float32 significand) and stages them in s_a next to the
    // expert slice; experts past n become zeros. Examples past B keep the
    // clamped copies: they only feed output columns that are never written.
    constexpr int NA = 32 * MT * KC / 4 / 256;  // 16-byte attention pieces per thread per chunk
    auto load_alpha = [&](int ch, f32x4_t (&ga)[NA]) {
#pragma unroll
        for (int it = 0; it < NA; ++it) {
            const int v = tid + 256 * it, r = v >> 3, kq = 4 * (v & 7);
            const int b = min(bc0 + r, B - 1), k = KC * ch + kq;
            if constexpr (A16) {
                ga[it] = *reinterpret_cast<const f32x4_t *>(alpha + (long)b * n + min(k, n - 4));
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) ga[it][j] = alpha[(long)b * n + min(k + j, n - 1)];
            }
        }
    };
    auto store_alpha = [&](int buf, int ch, const f32x4_t (&ga)[NA]) {
#pragma unroll
        for (int it = 0; it < NA; ++it) {
            const int v = tid + 256 * it, r = v >> 3, kq = 4 * (v & 7);
            float val[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) val[j] = KC * ch + kq + j < n ? ga[it][j] : 0.f;
            uint32_t pw[3][2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float x = val[2 * jj], y = val[2 * jj + 1];
#pragma unroll
                for (int part = 0; part < 3; ++part) {
                    const uint32_t p = pack_bf16x2(x, y);
                    pw[part][jj] = p;
                    x -= __uint_as_float(p << 16);  // exact
                    y -= __uint_as_float(p & 0xffff0000u);
                }
            }
#pragma unroll
            for (int part = 0; part < 3; ++part)
                *reinterpret_cast<u32x2_t *>(&s_a[buf][part][r][kq]) = u32x2_t{pw[part][0], pw[part][1]};
        }
    };
    f32x16_t acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;
    // DEPTH chunks in flight in DEPTH register sets: while chunk ch is
    // multiplied from LDS, chunks ch + 1 .. ch + DEPTH - 1 wait in their sets
    // and chunk ch + DEPTH loads into the set that chunk ch left (the loop is
    // unrolled DEPTH times so the sets rotate without copies).
    u32x4_t qs[DEPTH][NV];
    f32x4_t gs[DEPTH][NA];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        load(d, qs[d]);
        load_alpha(d, gs[d]);
    }
    store(0, qs[0]);
    store_alpha(0, 0, gs[0]);
    const int si = lane & 15;
    // qn, gn: chunk ch + 1, in flight (DEPTH > 1) or to load (DEPTH 1, the
    // same set as qf, gf); qf, gf: take chunk ch + DEPTH
    auto step = [&](int ch, u32x4_t (&qn)[NV], f32x4_t (&gn)[NA], u32x4_t (&qf)[NV], f32x4_t (&gf)[NA]) {
        const int buf = ch & 1;
        load(ch + DEPTH, qf);
        load_alpha(ch + DEPTH, gf);
        // keep the loads first and the staging of chunk ch + 1 last: the
        // scheduler would otherwise start the attention split (pure VALU)
        // early and wait there for every load in flight
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // chunk ch is in s_e[buf] and s_a[buf]; the reads of the other buffers are done
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
            // attention operands (B: columns = examples): one bf16 part of
            // example 32 mt + l32, experts 16 g + 8 lh + (0..7) of the chunk
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int part = 2; part >= 0; --part) {  // small parts first
                    const bf16x8_t ap =
                        *reinterpret_cast<const bf16x8_t *>(&s_a[buf][part][32 * mt + l32][16 * g + 8 * lh]);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[nt], ap, acc[mt][nt], 0, 0, 0);
                }
            }
        }
        // unconditional, so that no path leaves a register set with loads
        // pending into the next step (after the last chunk it stores zeros
        // nobody reads)
        __builtin_amdgcn_sched_barrier(0);
        store(buf ^ 1, qn);
        store_alpha(buf ^ 1, ch + 1, gn);
    };
    int ch = 0;
    for (; ch + DEPTH <= nchunks; ch += DEPTH) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) step(ch + j, qs[(j + 1) % DEPTH], gs[(j + 1) % DEPTH], qs[j], gs[j]);
    }
#pragma unroll
    for (int j = 0; j + 1 < DEPTH; ++j)
        if (ch + j < nchunks) step(ch + j, qs[(j + 1) % DEPTH], gs[(j + 1) % DEPTH], qs[j], gs[j]);
    __syncthreads();  // every wave's reads of the attentions, which s_o overwrites, are done
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

bool mix_wide_supported(long wsize) { return wsize >= 8 && wsize % 8 == 0 && wsize < kWideMaxW; }

hipError_t launch_mix_wide(const Geom &g, long wsize, const float *alpha, const uint16_t *experts, uint16_t *mixed,
                           hipStream_t stream, bool conv_feed) {
    if (!mix_wide_supported(wsize)) return hipErrorInvalidValue;
    const unsigned tiles = (unsigned)((wsize + kMixWW - 1) / kMixWW);
    // 64 examples per workgroup only when the grid still has four workgroups
    // per CU; for the forward's mix (W_b in the premix layout, read by the
    // convolution next) from two per CU: at n = 128, B = 64 that forward took
    // 44.6-45.1 us back to back against 46.0-46.1 us with 32 examples, while
    // the stand-alone mix lost (21.7-21.9 against 19.8 us)
    const bool a16 = g.n % 4 == 0 && reinterpret_cast<uintptr_t>(alpha) % 16 == 0;
    const bool mt2 = g.B > 32 && (long)tiles * ceil_div(g.B, 64) >= (conv_feed ? 512 : 1024);
    const dim3 grid(tiles, (unsigned)ceil_div(g.B, mt2 ? 64 : 32));
    // more register sets than one would cost MT = 2 its second wave per SIMD
    auto k = mt2 ? (a16 ? mix_mfma_wide_kernel<2, true, 1> : mix_mfma_wide_kernel<2, false, 1>)
                 : (a16 ? mix_mfma_wide_kernel<1, true, kWideDepth> : mix_mfma_wide_kernel<1, false, kWideDepth>);
    hipLaunchKernelGGL(k, grid, dim3(256), 0, stream, alpha, experts, mixed, g.B, g.n, wsize);
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
