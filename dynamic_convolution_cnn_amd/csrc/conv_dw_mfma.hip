// Depthwise dynamic convolution on the matrix cores (bf16, stride 1, square
// 3/5/7 kernels, output planes up to 32 x 32).
//
// Each (example, channel) plane has its own K x K taps, mixed from the
// channel's n experts (W_b[c] = sum_i alpha_bi E_i[c]; KernelWarehouse
// abstract: a linear mixture of n static kernels with input-dependent
// attentions; CondConv abstract: per-example kernels, EfficientNet-B0's
// depthwise layers among them). The taps are rounded to bf16 once, like
// every other mixed kernel, and the sums are float32.
//
// The plane's sums are written as K matrix products, one per kernel row u:
//
//   Y[r][s] = sum_u sum_k T_u[s][k] * P[r + u][k],   T_u[s][k] = w[u][k + d - s]
//
// with P the zero-padded input plane as staged in LDS (its first d = pad % 4
// padded columns dropped, so that every staged row starts 8-byte aligned;
// those columns are zero, so the taps that would meet them add nothing) and
// T_u a band (Toeplitz) matrix holding row u of the taps: row s of T_u is
// zero except for the K columns s - d .. s - d + K - 1. One
// v_mfma_f32_32x32x16_bf16 takes a 32 x 16 slice of T_u (rows s = output
// columns) and a 16 x 32 slice of P (columns r = output rows), so a plane
// of up to 32 x 32 outputs is 2 K products per 16 staged columns: 10
// MFMAs for the EfficientNet-B0 5x5 layer on 28 x 28 planes. The band
// wastes most of each product, but at 32 cycles per MFMA a plane costs a
// few hundred matrix-core cycles where the same sums as bf16 dot2 vector
// instructions cost about four hundred issue slots of four cycles each.
//
// A lane's slice of T_u (8 consecutive columns of one row s) is read from
// LDS with one 16-byte read. Row u of the taps is kept as 8 copies of the
// zero-extended row shifted by 0..7 elements, so that every lane's 8
// elements start on a 16-byte boundary; only the two 16-byte windows of a
// copy that can hold taps are stored, and lanes whose slice misses the band
// read a zero window. A plane's taps touch the same 8 K bf16 slots of the
// table every time; the rest of the table stays zero from the kernel's
// start, as do the padding rows and columns of the staged plane.
//
// Organisation: workgroup (c, g) of 4 independent waves takes channel c of
// the examples [16 g, 16 g + 16), wave w the examples 16 g + 4 w + k (k < 4)
// one after the other; each wave has its own LDS region and never waits for
// the others. Lane l loads the channel's n <= 8 expert values of tap l % KT
// once and mixes that tap for each example; with the taps already mixed in
// memory (more than 8 experts, or the PREMIX policy) it reads them instead.
// Each example's plane is loaded into registers while the previous one
// computes, and its results leave through a dense copy of the output plane
// in LDS, so that loads and stores are whole 16-byte pieces of consecutive
// elements where the plane sizes allow. Stores scattered over the rows as
// the accumulators hold them (16 bytes per row per instruction) made the
// layer about a third slower.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

constexpr int kDmWaves = 4;       // waves (independent) per workgroup
constexpr int kDmPB = 4;          // examples per wave
constexpr int kDmDepth = 1;       // planes loading ahead of the one computing
constexpr int kDmAhead = 2;       // MFMA operand reads issued ahead of the product using them
constexpr int kDmPitch = 40;      // bf16 per staged row: 80 bytes, so 8 lanes' 16-byte reads of 8 rows miss each other's banks
constexpr int kDmCopyBytes = 32;  // two 16-byte windows of one shifted copy of a tap row
constexpr int kDmTapRow = 8 * kDmCopyBytes + 16;  // 8 copies and a zero window
constexpr int kDmOutBytes = 2048 + 16;            // dense output plane (1024 elements at most) and a spare slot

template <int K>
struct DmLayout {
    static constexpr int rows = 32 + K - 1;  // staged rows: output rows 0..31 read rows r .. r + K - 1
    static constexpr int plane_bytes = rows * kDmPitch * 2;
    static constexpr int tap_bytes = K * kDmTapRow;
    static constexpr int wave_bytes = plane_bytes + tap_bytes + kDmOutBytes;
    static_assert(plane_bytes % 16 == 0 && wave_bytes % 16 == 0, "16-byte LDS windows");
};

// Planes move between HBM and registers in pieces of PBY bytes (16, 8 or 4):
// a lane holds NQ pieces of a plane of at most 2 KiB in 8 words.
template <int PBY>
struct DmPiece {
    static constexpr int words = PBY / 4;     // 32-bit words per piece
    static constexpr int nq = 8 / words;      // pieces per lane
    static constexpr int elems = PBY / 2;     // bf16 per piece
    static constexpr int parts = PBY == 16 ? 2 : 1;  // LDS writes per piece (rows hold whole 8-byte parts)
};

// One plane into registers; piece indices are clamped, so every load is in
// bounds and unconditional (lanes past the end load the last piece again).
template <int PBY>
__device__ __forceinline__ void dm_fetch(const uint16_t *__restrict__ xp, int lane, int npc, uint32_t (&w)[8]) {
    using P = DmPiece<PBY>;
#pragma unroll
    for (int q = 0; q < P::nq; ++q) {
        const int p = min(lane + 64 * q, npc - 1);
        if constexpr (PBY == 16) {
            const u32x4_t v = reinterpret_cast<const u32x4_t *>(xp)[p];
            w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
        } else if constexpr (PBY == 8) {
            const u32x2_t v = reinterpret_cast<const u32x2_t *>(xp)[p];
            w[2 * q] = v.x; w[2 * q + 1] = v.y;
        } else {
            w[q] = reinterpret_cast<const uint32_t *>(xp)[p];
        }
    }
}

// A wave's body is straight-line code: example, piece and chunk indices are
// clamped rather than branched on (a ragged wave repeats its last example;
// repeated pieces and chunks write the same values to the same places),
// every lane writes a tap (lanes past the taps repeat one), and lanes whose
// results fall outside the plane write them to a spare LDS slot. With no
// branches the compiler's memory-counter waits are exact, so each plane's
// loads stay in flight until the step that stages it. The results go
// through a dense copy of the output plane in LDS, so that the stores are
// whole PBY-byte chunks of consecutive outputs.
template <int K, int NCH, int PBY>
__global__ __launch_bounds__(64 * kDmWaves) void depthwise_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ experts, const float *__restrict__ alpha,
    const uint16_t *__restrict__ wmixed, uint16_t *__restrict__ y, int B, int C, int H, int W, int pad,
    int Ho, int Wo, int n, const float *__restrict__ a_in, const float *__restrict__ a_out) {
    using L = DmLayout<K>;
    using P = DmPiece<PBY>;
    constexpr int KT = K * K;
    __shared__ __attribute__((aligned(16))) u32x4_t lds[kDmWaves * L::wave_bytes / 16];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int c = blockIdx.x % C;
    const int b0 = (blockIdx.x / C) * (kDmWaves * kDmPB) + wave * kDmPB;
    if (b0 >= B) return;  // the waves never meet at a barrier
    const int blast = min(b0 + kDmPB, B) - 1;
    char *const plane = reinterpret_cast<char *>(lds) + wave * L::wave_bytes;
    char *const taps = plane + L::plane_bytes;
    char *const outp = taps + L::tap_bytes;
    for (int i = lane; i < (L::plane_bytes + L::tap_bytes) / 16; i += 64)
        reinterpret_cast<u32x4_t *>(plane)[i] = u32x4_t{0u, 0u, 0u, 0u};

    // tap inputs first (their loads are the oldest, so waiting for them
    // leaves the plane loads in flight). Lane l takes tap l % KT: tap (u, v)
    // goes to copy s8 of row u at element 32 + v - s8, in the copy's windows
    // 3 and 4 (elements 24..39); lanes sharing a tap compute the same value
    // and write it to the same slots. ev[i]: expert i's value of the lane's
    // tap (mixing), or the mixed tap of example b0 + i (premixed).
    const int tl = lane % KT;
    const int tu = tl / K, tv = tl - tu * K;
    const int toff = tu * kDmTapRow + (32 + tv - 24) * 2;  // copy 0; copy s8 is 30 s8 bytes on
    const long tstride = (long)C * KT;
    const uint16_t *tsrc = (wmixed ? wmixed + (long)b0 * tstride : experts) + (long)c * KT + tu * K + tv;
    const int tcnt = wmixed ? blast - b0 + 1 : n;
    float ev[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ev[i] = bf16_to_f32(tsrc[min(i, tcnt - 1) * tstride]);
    float asc[kDmPB];  // a_in * a_out of each example's plane
#pragma unroll
    for (int k = 0; k < kDmPB; ++k) {
        const long bc = (long)min(b0 + k, blast) * C + c;
        asc[k] = (a_in ? a_in[bc] : 1.f) * (a_out ? a_out[bc] : 1.f);
    }

    const int d = pad & 3;  // padded columns not staged
    const int hw = H * W, howo = Ho * Wo;
    const int npc = hw / P::elems;        // pieces per input plane
    const int nch = howo * 2 / PBY;       // chunks per output plane
    uint32_t pc[kDmDepth + 1][8];
#pragma unroll
    for (int k = 0; k < kDmDepth; ++k) dm_fetch<PBY>(x + ((long)min(b0 + k, blast) * C + c) * hw, lane, npc, pc[k]);
    asm volatile("" ::: "memory");  // the plane loads issue before the wait for the tap inputs
    __builtin_amdgcn_sched_barrier(0);

    // each example's taps: sum_i alpha_bi E_i (fixed order) or the premixed
    // value, times the plane's attentions, rounded to bf16 once
    uint16_t tb[kDmPB];
#pragma unroll
    for (int k = 0; k < kDmPB; ++k) {
        const int b = min(b0 + k, blast);
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) t = fmaf(alpha[(long)b * n + min(i, n - 1)], i < n ? ev[i] : 0.f, t);
        tb[k] = f32_to_bf16((wmixed ? ev[k] : t) * asc[k]);
    }

    // LDS byte offsets of the lane's piece parts in the staged plane
    constexpr int NPART = P::nq * P::parts;
    int poff[NPART];
#pragma unroll
    for (int q = 0; q < P::nq; ++q)
#pragma unroll
        for (int h = 0; h < P::parts; ++h) {
            const int e = min(lane + 64 * q, npc - 1) * P::elems + 4 * h;
            const int r = e / W, w = e - r * W;
            poff[q * P::parts + h] = ((r + pad) * kDmPitch + w + pad - d) * 2;
        }

    // MFMA operands: A = rows s = lane % 32 of T_u, columns 16 m + 8 (lane / 32) .. + 7;
    // B = columns r = lane % 32 of P[r + u], rows (staged columns) the same
    const int s = lane & 31, hh = lane >> 5;
    int aoff[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
        const int sig = 32 + 16 * m + 8 * hh + d - s;  // zero-extended tap row index of the first element
        const int cp = sig & 7, win = sig >> 3;
        aoff[m] = (win == 3 || win == 4) ? cp * kDmCopyBytes + (win - 3) * 16 : 8 * kDmCopyBytes;
    }
    const int boff = s * kDmPitch * 2 + hh * 16;
    // LDS offsets in the dense output plane of the lane's 4 x 4 results
    // (row s, columns 8 j + 4 hh ..), or the spare slot
    constexpr int kSpare = 2048;
    int ooff[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int s0 = 8 * j + 4 * hh;
        const int o = (s * Wo + s0) * 2;
        ooff[j][0] = s < Ho && s0 + (PBY >= 8 ? 4 : 2) <= Wo ? o : kSpare;
        ooff[j][1] = s < Ho && s0 + 4 <= Wo ? o + 4 : kSpare;
    }

#pragma unroll
    for (int k = 0; k < kDmPB; ++k) {
        const int b = min(b0 + k, blast);
        const uint32_t(&cur)[8] = pc[k % (kDmDepth + 1)];
        // the plane kDmDepth examples on loads into the set used last step
        if (k + kDmDepth < kDmPB)
            dm_fetch<PBY>(x + ((long)min(b0 + k + kDmDepth, blast) * C + c) * hw, lane, npc,
                          pc[(k + kDmDepth) % (kDmDepth + 1)]);
        asm volatile("" ::: "memory");  // the previous example's LDS reads come first
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) *reinterpret_cast<uint16_t *>(taps + toff + 30 * s8) = tb[k];
#pragma unroll
        for (int q = 0; q < NPART; ++q) {
            if constexpr (PBY == 4)
                *reinterpret_cast<uint32_t *>(plane + poff[q]) = cur[q];
            else
                *reinterpret_cast<u32x2_t *>(plane + poff[q]) = u32x2_t{cur[2 * q], cur[2 * q + 1]};
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // operands of product j = NCH u + m; the reads run kDmAhead products
        // ahead (scheduling barriers keep each read group behind the product
        // kDmAhead before it, so kDmAhead + 1 operand sets are live)
        constexpr int NP = K * NCH;
        bf16x8_t fa[NP], fb[NP];
        auto rd = [&](int j) {
            const int u = j / NCH, m = j - u * NCH;
            fa[j] = *reinterpret_cast<const bf16x8_t *>(taps + u * kDmTapRow + aoff[m]);
            fb[j] = *reinterpret_cast<const bf16x8_t *>(plane + boff + u * kDmPitch * 2 + 32 * m);
        };
#pragma unroll
        for (int j = 0; j < kDmAhead && j < NP; ++j) rd(j);
        f32x16_t acc = {};
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            if (j + kDmAhead < NP) rd(j + kDmAhead);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j], fb[j], acc, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // lane holds Y[r][8 j + 4 hh + i] in acc[4 j + i]: into the dense
        // plane, then out in whole chunks
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = pack_bf16x2(acc[4 * j], acc[4 * j + 1]);
            const uint32_t hi = pack_bf16x2(acc[4 * j + 2], acc[4 * j + 3]);
            if constexpr (PBY >= 8) {
                *reinterpret_cast<u32x2_t *>(outp + ooff[j][0]) = u32x2_t{lo, hi};
            } else {
                *reinterpret_cast<uint32_t *>(outp + ooff[j][0]) = lo;
                *reinterpret_cast<uint32_t *>(outp + ooff[j][1]) = hi;
            }
        }
        asm volatile("" ::: "memory");
        uint16_t *yp = y + ((long)b * C + c) * howo;
#pragma unroll
        for (int q = 0; q < P::nq; ++q) {
            const int ch = min(lane + 64 * q, nch - 1);
            if constexpr (PBY == 16)
                reinterpret_cast<u32x4_t *>(yp)[ch] = reinterpret_cast<const u32x4_t *>(outp)[ch];
            else if constexpr (PBY == 8)
                reinterpret_cast<u32x2_t *>(yp)[ch] = reinterpret_cast<const u32x2_t *>(outp)[ch];
            else
                reinterpret_cast<uint32_t *>(yp)[ch] = reinterpret_cast<const uint32_t *>(outp)[ch];
        }
    }
}

int dm_chunks(const Geom &g) { return (g.W + 2 * g.pad - (g.pad & 3) + 15) / 16; }

}  // namespace

// bf16, depthwise, square 3/5/7 taps, stride 1, output planes of at most
// 32 x 32 whose staged columns fit two 16-column slices, even W and Wo,
// planes of at most 1024 elements, and n <= 8 experts unless the taps are
// already mixed.
bool depthwise_mfma_ok(const Geom &g, bool premixed) {
    return g.bf16 && g.KH == g.KW && (g.KH == 3 || g.KH == 5 || g.KH == 7) && g.stride == 1 && g.pad >= 0 &&
           g.Ho >= 1 && g.Wo >= 1 && g.Ho <= 32 && g.Wo <= 32 && g.W % 2 == 0 && g.Wo % 2 == 0 &&
           g.H * g.W <= 1024 && dm_chunks(g) <= 2 && (premixed || g.n <= 8);
}

// Piece size: 16 bytes where both planes are whole 16-byte chunks and rows
// hold whole 8-byte parts, 8 bytes where rows are multiples of 4 elements,
// else 4.
static int dm_piece_bytes(const Geom &g) {
    if (g.W % 4 == 0 && g.Wo % 4 == 0)
        return (g.H * g.W) % 8 == 0 && (g.Ho * g.Wo) % 8 == 0 ? 16 : 8;
    return 4;
}

hipError_t launch_depthwise_mfma(const Geom &g, const uint16_t *x, const uint16_t *experts, const float *alpha,
                                 const uint16_t *wmixed, uint16_t *y, hipStream_t stream, ChanAttn att) {
    const int per_wg = kDmWaves * kDmPB;
    const dim3 grid((unsigned)((long)g.Cin * ((g.B + per_wg - 1) / per_wg)));
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(64 * kDmWaves), 0, stream, x, experts, alpha, wmixed, y, g.B, g.Cin,
                           g.H, g.W, g.pad, g.Ho, g.Wo, g.n, att.in, att.out);
        return hipGetLastError();
    };
    const bool two = dm_chunks(g) == 2;
    const int pby = dm_piece_bytes(g);
    auto pick = [&](auto k) {
        constexpr int K = decltype(k)::value;
        if (pby == 16)
            return two ? go(depthwise_mfma_kernel<K, 2, 16>) : go(depthwise_mfma_kernel<K, 1, 16>);
        if (pby == 8) return two ? go(depthwise_mfma_kernel<K, 2, 8>) : go(depthwise_mfma_kernel<K, 1, 8>);
        return two ? go(depthwise_mfma_kernel<K, 2, 4>) : go(depthwise_mfma_kernel<K, 1, 4>);
    };
    switch (g.KH) {
    case 3: return pick(std::integral_constant<int, 3>{});
    case 5: return pick(std::integral_constant<int, 5>{});
    default: return pick(std::integral_constant<int, 7>{});
    }
}

}  // namespace dynconv
