// Fused mixing + convolution on bf16 MFMA (gfx950): the per-example kernel
// W_b = sum_i alpha_bi E_i (KernelWarehouse: Rethinking the Design of Dynamic
// Convolution, abstract) is formed inside the GEMM from the packed expert
// bank packed[t][o][cp][ip] and never reaches memory.
//
// conv_fused_kernel: any shape with n <= 4 and at most 256 output positions.
//   A workgroup owns 4 examples (one per wave pair) and 64 output channels;
//   B fragments are mixed with bf16 dot2 instructions into a shared LDS
//   stage; A fragments come from an [input row][input col][channel] LDS tile
//   (80-byte position stride), one 128-bit read per lane and fragment.
// conv_fused_row16_kernel: 3x3 stride-1 layers up to 14x14 (see below).
#include "conv_common.hpp"

namespace dynconv {
namespace {

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Each dword shifted by v lanes within its 16-lane row (lane i takes lane
// i + v; lanes past the row end read 0): v_mov_b32_dpp row_shl:v.
__device__ __forceinline__ uint32_t dpp_shl_1(uint32_t x, int v) {
    switch (v) {
    case 1: return __builtin_amdgcn_mov_dpp(x, 0x101, 0xf, 0xf, true);
    case 2: return __builtin_amdgcn_mov_dpp(x, 0x102, 0xf, 0xf, true);
    case 3: return __builtin_amdgcn_mov_dpp(x, 0x103, 0xf, 0xf, true);
    case 4: return __builtin_amdgcn_mov_dpp(x, 0x104, 0xf, 0xf, true);
    case 5: return __builtin_amdgcn_mov_dpp(x, 0x105, 0xf, 0xf, true);
    case 6: return __builtin_amdgcn_mov_dpp(x, 0x106, 0xf, 0xf, true);
    default: return __builtin_amdgcn_mov_dpp(x, 0x107, 0xf, 0xf, true);
    }
}
__device__ __forceinline__ u32x4_t dpp_shl(u32x4_t x, int v) {
    return u32x4_t{dpp_shl_1(x.x, v), dpp_shl_1(x.y, v), dpp_shl_1(x.z, v), dpp_shl_1(x.w, v)};
}

// Input staging of the fused kernel, split in two phases so that the loads
// of the next chunk are in flight while the current chunk computes:
// stage_load issues a lane's global loads into registers, stage_store writes
// them to the tile. The per-task source and destination offsets do not
// depend on the chunk and are computed once (StageMap). Paired layout only
// (W even): a task is 2 neighbouring positions x 8 channels; of the NL lanes
// staging one example, lane owns tasks lane, lane + NL, ...
template <int XT>
struct StageMap {
    int src[XT];  // element offset from the chunk's first channel plane
    int dst[XT];  // element offset in the tile; -1: no task
};

template <int XT, int NL>
__device__ __forceinline__ void stage_map(const ConvArgs &a, int nrows, int h_tile0, int lane,
                                          StageMap<XT> &m) {
    const int HW = a.H * a.W;
    const int pairs = a.W >> 1;
    const int per_g = nrows * pairs;
    const int ntasks = 4 * per_g;
#pragma unroll
    for (int k = 0; k < XT; ++k) {
        const int task = lane + NL * k;
        const int g = task / per_g;
        const int rem = task - g * per_g;
        const int row = rem / pairs;
        const int pr = rem - row * pairs;
        const bool ok = task < ntasks;
        m.src[k] = ok ? 8 * g * HW + row * a.W + 2 * pr : 0;
        m.dst[k] = ok ? ((row - h_tile0) * a.ncols + 2 * pr + a.pad) * kPosStride + 8 * g : -1;
    }
}

template <int XT>
__device__ __forceinline__ void stage_load(const uint16_t *__restrict__ xc, const ConvArgs &a,
                                           int c0, const StageMap<XT> &m, uint32_t (&r)[XT][8]) {
    const int HW2 = (a.H * a.W) >> 1;  // words per channel plane
    const bool tail = c0 + kChunk > a.Cin;
#pragma unroll
    for (int k = 0; k < XT; ++k) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(xc + m.src[k]);
        if (!tail) {
#pragma unroll
            for (int j = 0; j < 8; ++j) r[k][j] = src[(long)j * HW2];
        } else {
            // channel of word j is c0 + 8g + j; 8g is the tile offset modulo kPosStride
            const int cb = c0 + (m.dst[k] >= 0 ? m.dst[k] % kPosStride : 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int jj = min(j, max(a.Cin - 1 - cb, 0));
                const uint32_t v = src[(long)jj * HW2];
                r[k][j] = cb + j < a.Cin ? v : 0u;
            }
        }
    }
}

template <int XT>
__device__ __forceinline__ void stage_store(uint16_t *__restrict__ tile, const StageMap<XT> &m,
                                            const uint32_t (&r)[XT][8]) {
#pragma unroll
    for (int k = 0; k < XT; ++k) {
        if (m.dst[k] >= 0) {
            u32x4_t o0, o1;
            o0.x = lo_pair(r[k][0], r[k][1]); o0.y = lo_pair(r[k][2], r[k][3]);
            o0.z = lo_pair(r[k][4], r[k][5]); o0.w = lo_pair(r[k][6], r[k][7]);
            o1.x = hi_pair(r[k][0], r[k][1]); o1.y = hi_pair(r[k][2], r[k][3]);
            o1.z = hi_pair(r[k][4], r[k][5]); o1.w = hi_pair(r[k][6], r[k][7]);
            *reinterpret_cast<u32x4_t *>(tile + m.dst[k]) = o0;
            *reinterpret_cast<u32x4_t *>(tile + m.dst[k] + kPosStride) = o1;
        }
    }
}

// Packed expert words of one (tap, chunk) step for this lane's fragment:
// 8 channels x NP2 expert pairs.
template <int NP2>
__device__ __forceinline__ void load_packed(const uint32_t *__restrict__ packed, const ConvArgs &a,
                                            int t, int c0, long prow, uint32_t (&w)[8 * NP2]) {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
        packed + ((long)t * a.Cout * a.Cin_pad + c0) * NP2 + prow);
#pragma unroll
    for (int q = 0; q < 2 * NP2; ++q) {
        const u32x4_t v4 = src[q];
        w[4 * q + 0] = v4.x; w[4 * q + 1] = v4.y;
        w[4 * q + 2] = v4.z; w[4 * q + 3] = v4.w;
    }
}

// One B fragment: W_b[c][o] = sum_i alpha_bi E_i[c][o] over this lane's 8
// channels, as two bf16 dot2 chains (attention high and low parts), rounded
// once to bf16.
template <int NP2>
__device__ __forceinline__ u32x4_t mix_frag(const uint32_t (&w)[8 * NP2], const uint32_t *ahi,
                                            const uint32_t *alo) {
    float f[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < NP2; ++p) s = dot2(w[c * NP2 + p], ahi[p], s);
#pragma unroll
        for (int p = 0; p < NP2; ++p) s = dot2(w[c * NP2 + p], alo[p], s);
        f[c] = s;
    }
    u32x4_t pk;
    pk.x = pack_bf16x2(f[0], f[1]); pk.y = pack_bf16x2(f[2], f[3]);
    pk.z = pack_bf16x2(f[4], f[5]); pk.w = pack_bf16x2(f[6], f[7]);
    return pk;
}

// Fused: a workgroup owns 4 examples and 64 output channels; 8 waves, two
// per SIMD, so that one wave's mixing and memory work overlaps the other
// wave's MFMAs. The convolution runs on v_mfma_f32_32x32x16_bf16 (32
// positions x 32 channels x 16 K per instruction).
//   - MFMAs: waves w and w+4 share example e = w & 3; wave w < 4 takes the
//     first PBW blocks of 32 positions, wave w + 4 the rest, all 64 channels;
//     A fragments come from the example's input tile, B fragments from the
//     stage below.
//   - Mixing: per step (32 input channels of one tap) each example needs 4 B
//     fragments (2 blocks of 32 output channels x 2 halves of 16 input
//     channels). Wave w mixes fragment w & 3 for examples 2(w >> 2) and
//     2(w >> 2) + 1, and writes the bf16 fragments to a double-buffered LDS
//     stage, so the expert tile is read once per pair of waves.
//   - Staging: the two waves of an example stage its input chunk together.
// Software pipeline over steps s = (chunk c, tap t), one barrier per step:
// the MFMAs of step s run while the B fragments of step s+1 are mixed and
// the expert words of step s+2 load; the next input chunk loads into
// registers during a chunk and is written to the tile after its last tap.
template <int PBW, int NP2, int XT>
__global__ __launch_bounds__(512) void conv_fused_kernel(const uint16_t *__restrict__ x,
                                                         const uint32_t *__restrict__ packed,
                                                         const float *__restrict__ alpha,
                                                         uint16_t *__restrict__ y, ConvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    constexpr int CB = 2;  // 2 x 32 output channels
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int ex = wave & 3, half = wave >> 2;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int ot = logical / a.n_btiles;
    const int bt = logical - ot * a.n_btiles;
    const int o0 = ot * CB * 32;
    const int tile_elems = a.tile_rows * a.ncols * kPosStride;
    uint16_t *tile = lds + ex * tile_elems;
    // B stage: [2 buffers][4 examples][4 fragments][64 lanes] x 16 bytes
    u32x4_t *bstage = reinterpret_cast<u32x4_t *>(lds + 4 * tile_elems);
    auto bslot = [&](int buf, int e, int f) { return bstage + ((buf * 4 + e) * 4 + f) * 64 + lane; };

    // mixing role: fragment mf for examples 2*half and 2*half + 1
    const int mf = wave & 3;
    uint32_t ahi[2][NP2], alo[2][NP2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int be = min(bt * 4 + 2 * half + k, a.B - 1);
#pragma unroll
        for (int p = 0; p < NP2; ++p) {
            const float a0 = 2 * p < a.n ? alpha[(long)be * a.n + 2 * p] : 0.f;
            const float a1 = 2 * p + 1 < a.n ? alpha[(long)be * a.n + 2 * p + 1] : 0.f;
            ahi[k][p] = pack_bf16x2(a0, a1);
            alo[k][p] = pack_bf16x2(a0 - bf16_lo(ahi[k][p]), a1 - bf16_hi(ahi[k][p]));
        }
    }
    const long prow =
        ((long)min(o0 + 32 * (mf >> 1) + l32, a.Cout - 1) * a.Cin_pad + 16 * (mf & 1) + 8 * lh) * NP2;

    // convolution role: example ex, position blocks [pb0, pb0 + npb)
    const int b_raw = bt * 4 + ex;
    const bool valid = b_raw < a.B;
    const int b = valid ? b_raw : a.B - 1;
    const int pbt = ceil_div(a.P, 32);
    const int pb0 = half * PBW;
    const int npb = min(PBW, pbt - pb0);

    zero_lds(tile, tile_elems, half * 64 + lane, 128);

    int aoff[PBW];
#pragma unroll
    for (int pb = 0; pb < PBW; ++pb) {
        const int p = min((pb0 + pb) * 32 + l32, a.P - 1);
        const int r = p / a.Wo;
        const int s = p - r * a.Wo;
        aoff[pb] = ((r * a.stride) * a.ncols + s * a.stride) * kPosStride + 8 * lh;
    }
    const uint16_t *xb = x + (long)b * a.x_bstride;

    f32x16_t acc[PBW][CB];
#pragma unroll
    for (int i = 0; i < PBW; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // input rows the tile holds (rows below the last output's reach are not needed)
    const int h_tile0 = -a.pad;
    const int nrows = min(a.H, h_tile0 + a.tile_rows);
    const int nchunks = a.Cin_pad / kChunk;
    const int nsteps = nchunks * a.KT;
    const int HW = a.H * a.W;

    StageMap<XT> smap;
    stage_map<XT, 128>(a, nrows, h_tile0, half * 64 + lane, smap);
    uint32_t xr[XT][8];
    lds_barrier();  // tile zeroed by both waves of the example
    stage_load<XT>(xb, a, 0, smap, xr);
    stage_store<XT>(tile, smap, xr);

    uint32_t w[8 * NP2];
    load_packed<NP2>(packed, a, 0, 0, prow, w);
#pragma unroll
    for (int k = 0; k < 2; ++k) *bslot(0, 2 * half + k, mf) = mix_frag<NP2>(w, ahi[k], alo[k]);
    if (nsteps > 1) load_packed<NP2>(packed, a, 1 % a.KT, (1 / a.KT) * kChunk, prow, w);
    lds_barrier();

    int t = 0, c0 = 0;
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        if (t == 0 && c0 + kChunk < a.Cin_pad)
            stage_load<XT>(xb + (long)(c0 + kChunk) * HW, a, c0 + kChunk, smap, xr);
        const int u = t / a.KW, v = t - u * a.KW;
        const int toff = (u * a.ncols + v) * kPosStride;
        bf16x8_t bfr[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) bfr[f] = __builtin_bit_cast(bf16x8_t, *bslot(buf, ex, f));
        // K half outermost: the MFMAs between two updates of one accumulator
        // keep the matrix pipeline full
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            bf16x8_t afr[PBW];
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb)
                afr[pb] = *reinterpret_cast<const bf16x8_t *>(tile + aoff[pb] + toff + 16 * kh);
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb) {
                if (pb < npb) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[pb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[pb], bfr[cb * 2 + kh],
                                                                              acc[pb][cb], 0, 0, 0);
                }
            }
        }
        // mix step s+1 and fetch step s+2 (the last steps redo a valid step
        // whose result is never read)
#pragma unroll
        for (int k = 0; k < 2; ++k) *bslot(buf ^ 1, 2 * half + k, mf) = mix_frag<NP2>(w, ahi[k], alo[k]);
        {
            const int s2 = min(s + 2, nsteps - 1);
            const int c2 = s2 / a.KT;
            load_packed<NP2>(packed, a, s2 - c2 * a.KT, c2 * kChunk, prow, w);
        }
        if (++t == a.KT) {
            t = 0;
            if (c0 + kChunk < a.Cin_pad) {
                // the example's other wave may still read this chunk's tile
                // for the current step: meet it before overwriting the tile
                lds_barrier();
                stage_store<XT>(tile, smap, xr);
            }
            c0 += kChunk;
        }
        lds_barrier();
    }
    if (!valid) return;
    // D of a 32x32 block: lane holds column l32 and rows 8j + 4*lh + (0..3), j = 0..3
#pragma unroll
    for (int pb = 0; pb < PBW; ++pb) {
        if (pb >= npb) break;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4_t d = {acc[pb][cb][4 * j], acc[pb][cb][4 * j + 1], acc[pb][cb][4 * j + 2],
                                   acc[pb][cb][4 * j + 3]};
                store_frag(y, a, b, o0 + 32 * cb + l32, (pb0 + pb) * 32 + 8 * j + 4 * lh, d);
            }
    }
}

// Fused, stride-1 3x3 layers on small images (W + 2*pad <= 16, Ho <= 14):
// the ResNet-50-shaped 14x14 case. A workgroup owns 4 examples and 64 output
// channels with 8 waves, two per SIMD (up to 256 registers each).
//   - Mixing on the matrix cores: v_mfma_f32_4x4x4_16b_bf16 computes 16
//     independent 4x4x4 products; with the 4 examples' attention rows as A
//     (the same in every block) and one weight's 4 expert values per lane as
//     B, lane l receives the 4 examples' mixed values of its own weight. Each
//     wave mixes half of one B fragment (32 output channels x 16 input
//     channels) of each step for all 4 examples with 4 such products per
//     attention part (high and low bf16 halves, summed in fp32) and writes it
//     to a double-buffered LDS stage; the expert tile is read once per
//     workgroup.
//   - Convolution: the two waves of example e split its 7 blocks of 32
//     positions (4 + 3) over all 64 channels on v_mfma_f32_32x32x16_bf16.
//     Output rows are padded to 16 positions, so a 32-position A fragment is
//     two output rows, one per 16-lane DPP row; for column tap v the fragment
//     is the tap-0 fragment shifted by v lanes (v_mov_b32_dpp row_shl:v): one
//     LDS read per fragment and kernel row instead of kw. Junk columns are
//     dropped.
//   - Input tiles: 64-byte position stride with the 16-byte channel groups
//     XOR-swizzled by position; two per example, for the current chunk of
//     32 input channels and the next.
//   - 3x3 taps only: the 9 steps of a chunk (tap x 32 input channels) are
//     fully unrolled, so every prefetch slot and every staging decision is a
//     compile-time constant and the step has no branches.
//   - Exchange without exposed latency: step s mixes B_{s+1} into the stage
//     buffer that B_{s-1} occupied and multiplies fragments read before its
//     barrier or during the previous step; one barrier per step publishes
//     the new buffer.
//   - Prefetch in registers: the expert words a mixing uses load one step
//     earlier. The next chunk's input loads straight from x in steps 0..6
//     (dword buffer loads, one per channel and position pair) and reaches the
//     other tile two steps later, transposed in registers. All loads are
//     ordinary vector loads issued in a fixed order (expert words, then
//     input), so the compiler's wait counts stay exact and no wait covers a
//     younger load.
//   - The epilogue gathers each output block as dense channel planes in the
//     idle tiles and copies them to y with 16-byte stores.
constexpr int kRow16MaxPos = 256;  // tile positions (16 x 16)
constexpr int kRow16Slots = 7;     // staging slots per chunk (loads in steps 0..6)
// Two tiles per example (chunk parity), then the double-buffered B stage.
__shared__ __attribute__((aligned(16))) u32x4_t s_tiles[2 * 4 * kRow16MaxPos * 4];
__shared__ __attribute__((aligned(16))) u32x4_t s_bstage[2 * 4 * 4 * 64];

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Attention row of example (lane & 3) as a 4x4x4 A operand: experts 0..3 as
// bf16, high part (rounded) and low part (the rounding remainder).
__device__ __forceinline__ void alpha_rows(const float *__restrict__ alpha, int be, int n,
                                           s16x4_t &hi, s16x4_t &lo) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float v = k < n ? alpha[(long)be * n + k] : 0.f;
        const uint16_t h = f32_to_bf16(v);
        hi[k] = (short)h;
        lo[k] = (short)f32_to_bf16(v - bf16_to_f32(h));
    }
}

// Mixed B fragment words for the 4 examples: out[e] = 8 bf16 (channels
// j = 0..7 of this lane's fragment column) of sum_k alpha[e][k] E_k.
template <int NP2>
__device__ __forceinline__ void mix4_frag(const uint32_t (&w)[8 * NP2], s16x4_t ahi, s16x4_t alo,
                                          u32x4_t (&out)[4]) {
    f32x4_t d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        u32x2_t e2;
        e2.x = w[j * NP2];
        e2.y = NP2 == 2 ? w[j * NP2 + 1] : 0u;
        const s16x4_t ev = __builtin_bit_cast(s16x4_t, e2);
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        d[j] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi, ev, z, 0, 0, 0);
        d[j] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo, ev, d[j], 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        out[e].x = pack_bf16x2(d[0][e], d[1][e]);
        out[e].y = pack_bf16x2(d[2][e], d[3][e]);
        out[e].z = pack_bf16x2(d[4][e], d[5][e]);
        out[e].w = pack_bf16x2(d[6][e], d[7][e]);
    }
}

// Expert words of one (tap, chunk) step for half of this lane's fragment
// column: channels r = 4 h .. 4 h + 3 of the lane's 8 (prow includes 4 h) x
// NP2 expert pairs, NP2 16-byte loads.
template <int NP2>
__device__ __forceinline__ void load_packed_half(const uint32_t *__restrict__ packed, const ConvArgs &a,
                                                 int t, int c0, long prow, uint32_t (&w)[4 * NP2]) {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
        packed + ((long)t * a.Cout * a.Cin_pad + c0) * NP2 + prow);
#pragma unroll
    for (int q = 0; q < NP2; ++q) {
        const u32x4_t v4 = src[q];
        w[4 * q + 0] = v4.x; w[4 * q + 1] = v4.y;
        w[4 * q + 2] = v4.z; w[4 * q + 3] = v4.w;
    }
}

// Half a B fragment for the 4 examples: out[e] = 4 bf16 (channels 4 h ..
// 4 h + 3 of the lane's column) of sum_k alpha[e][k] E_k, on
// v_mfma_f32_4x4x4_16b_bf16 (high and low attention parts summed in fp32).
template <int NP2>
__device__ __forceinline__ void mix4_half(const uint32_t (&w)[4 * NP2], s16x4_t ahi, s16x4_t alo,
                                          u32x2_t (&out)[4]) {
    f32x4_t d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x2_t e2;
        e2.x = w[j * NP2];
        e2.y = NP2 == 2 ? w[j * NP2 + 1] : 0u;
        const s16x4_t ev = __builtin_bit_cast(s16x4_t, e2);
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        d[j] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi, ev, z, 0, 0, 0);
        d[j] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo, ev, d[j], 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        out[e].x = pack_bf16x2(d[0][e], d[1][e]);
        out[e].y = pack_bf16x2(d[2][e], d[3][e]);
    }
}

// 8 waves, two per SIMD: waves w and w + 4 (same SIMD) convolve example
// e = w & 3, wave w over position blocks 0..3 and wave w + 4 over blocks
// 4..6 (7 blocks of 32 positions = two padded rows each), both over all 64
// channels, so one A fragment feeds two MFMAs. The two waves of a SIMD share
// its matrix core: one wave's LDS round trips, waits and barrier skew overlap
// the other's MFMAs. Wave w also mixes half h = w & 1 of B fragment w >> 1
// for all 4 examples, and stages the 16 input channels [16 hs, 16 hs + 16),
// hs = w >> 2, of its example's next chunk into the example's other tile.
template <int NP2, int PBW>
__device__ __forceinline__ void row16_wave(const uint16_t *__restrict__ x, const uint32_t *__restrict__ packed,
                                           const float *__restrict__ alpha, uint16_t *__restrict__ y,
                                           const ConvArgs &a, int pb0) {
    constexpr int CB = 2;  // 2 x 32 output channels
    constexpr int K = 3;   // 3 x 3 taps: a chunk is 9 steps, fully unrolled
    constexpr int KT = K * K;
    constexpr int RL = 2;  // a staging slot loads in step i and reaches the tile in step i + RL
    static_assert(kRow16Slots + RL <= KT, "staging must end by the chunk's last step");
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int ot = logical / a.n_btiles;
    const int bt = logical - ot * a.n_btiles;
    const int o0 = ot * CB * 32;
    // convolution role
    const int e = wave & 3, hs = wave >> 2;
    auto tile_of = [&](int par) { return reinterpret_cast<uint16_t *>(s_tiles + (par * 4 + e) * kRow16MaxPos * 4); };
    auto bslot = [&](int buf, int ex, int f) { return s_bstage + ((buf * 4 + ex) * 4 + f) * 64 + lane; };
    auto bread = [&](int buf, int ex, int f) { return __builtin_bit_cast(bf16x8_t, *bslot(buf, ex, f)); };
    // mixing role: fragment mf = (channel block mf >> 1, K half mf & 1), half mh
    const int mf = wave >> 1, mh = wave & 1;
    s16x4_t ahi, alo;
    alpha_rows(alpha, min(bt * 4 + (lane & 3), a.B - 1), a.n, ahi, alo);
    const long prow = ((long)min(o0 + 32 * (mf >> 1) + l32, a.Cout - 1) * a.Cin_pad + 16 * (mf & 1) +
                       8 * lh + 4 * mh) * NP2;

    const int b_raw = bt * 4 + e;
    const bool valid = b_raw < a.B;
    const int b = valid ? b_raw : a.B - 1;
    // both tiles (their padding stays zero: staging writes interior positions only)
    zero_lds(tile_of(0), kRow16MaxPos * 32, lane + 64 * hs, 128);
    zero_lds(tile_of(1), kRow16MaxPos * 32, lane + 64 * hs, 128);

    int aq[PBW];
#pragma unroll
    for (int pb = 0; pb < PBW; ++pb) {
        const int r = min(2 * (pb0 + pb) + (l32 >> 4), a.Ho - 1);
        const int c = min(l32 & 15, a.ncols - 1);
        aq[pb] = r * a.ncols + c;
    }
    const uint16_t *xb = x + (long)b * a.x_bstride;
    const int HW = a.H * a.W;
    const int plane = HW * 2;  // bytes per input channel plane
    const int pairs = a.W >> 1;
    const int per_g = min(a.H, a.tile_rows - a.pad) * pairs;  // position pairs the tile holds per channel

    // Staging of this wave's 16 input channels [cc + 16 hs, cc + 16 hs + 16)
    // of a chunk, as half-tasks of 2 neighbouring positions x 4 channels:
    // 4 dword loads (one per channel, both positions) and, transposed in
    // registers, two 8-byte tile writes (half a 16-byte channel granule per
    // position). Lane l of slot s takes channel quad l & 3 of position pair
    // 16 s + (l >> 2) (pairs past the last repeat it: same bytes to the same
    // place). Its first write goes to the pair's first or second position
    // as (quad ^ pair) & 1 says, the second write to the other one, so that
    // the 16 lanes of a write phase spread over both halves of the bank row
    // and over the swizzled granules. Channels past Cin are beyond the
    // buffer's extent and read as zeros.
    // (The descriptor must live in scalar registers: its fields are passed
    // through readfirstlane, which they equal on every lane anyway.)
    auto rsrc_of = [&](int cc) {
        const int c0 = min(cc + 16 * hs, a.Cin - 1);
        const int nbytes = __builtin_amdgcn_readfirstlane(max(0, min(16, a.Cin - cc - 16 * hs)) * plane);
        const uint64_t p = reinterpret_cast<uint64_t>(xb + (long)c0 * HW);
        const uint64_t ps = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)) << 32);
        return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ps), 0, nbytes, 0x00020000);
    };
    // (p + 0.5) / pairs rounded down is exact in float for p < 2^12, pairs <= 2^8
    const float inv_pairs = 1.f / (float)pairs;
    auto pair_of = [&](int s, int ln) { return min(16 * s + (ln >> 2), per_g - 1); };
    auto stage_load = [&](__amdgpu_buffer_rsrc_t rs, int s, int ln, uint32_t (&r)[4]) {
        const int vo = 4 * (ln & 3) * plane + 4 * pair_of(s, ln);
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo + j * plane, 0, 0);
    };
    auto stage_store = [&](uint16_t *t, int s, int ln, const uint32_t (&r)[4]) {
        const int pg = pair_of(s, ln), quad = ln & 3;
        const int row = (int)(((float)pg + 0.5f) * inv_pairs);
        const int q = (row + a.pad) * a.ncols + 2 * (pg - row * pairs) + a.pad;
        const int g = 2 * hs + (quad >> 1), ho = 4 * (quad & 1);
        const int sel = (quad ^ pg) & 1;  // 1: first write goes to position q + 1
        // byte selectors: low halves (position q) or high halves (q + 1) of
        // two channel words
        const uint32_t bs0 = 0x05040100u + (uint32_t)sel * 0x02020202u;
        const uint32_t bs1 = 0x07060302u - (uint32_t)sel * 0x02020202u;
        u32x2_t p0, p1;
        p0.x = __builtin_amdgcn_perm(r[1], r[0], bs0); p0.y = __builtin_amdgcn_perm(r[3], r[2], bs0);
        p1.x = __builtin_amdgcn_perm(r[1], r[0], bs1); p1.y = __builtin_amdgcn_perm(r[3], r[2], bs1);
        *reinterpret_cast<u32x2_t *>(t + swz(q + sel, g) + ho) = p0;
        *reinterpret_cast<u32x2_t *>(t + swz(q + 1 - sel, g) + ho) = p1;
    };

    f32x16_t acc[PBW][CB];
#pragma unroll
    for (int i = 0; i < PBW; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    const int nchunks = a.Cin_pad / kChunk;
    const int nsteps = nchunks * KT;

    // chunk 0: loads first, so that their latencies overlap with each other
    // and with the first mixings
    uint32_t r0[kRow16Slots][4];
    {
        const auto rs = rsrc_of(0);
#pragma unroll
        for (int s = 0; s < kRow16Slots; ++s) stage_load(rs, s, lane, r0[s]);
    }

    auto words = [&](int st, uint32_t (&w)[4 * NP2]) {
        st = min(st, nsteps - 1);
        const int c = st / KT;
        load_packed_half<NP2>(packed, a, st - c * KT, c * kChunk, prow, w);
    };
    auto mix_to = [&](const uint32_t (&w)[4 * NP2], int buf) {
        u32x2_t m[4];
        mix4_half<NP2>(w, ahi, alo, m);
#pragma unroll
        for (int ex = 0; ex < 4; ++ex) reinterpret_cast<u32x2_t *>(bslot(buf, ex, mf))[mh] = m[ex];
    };
    // One barrier per step, between its two K halves, so that no MFMA waits
    // for it: step s
    //   reads B_s's K-half-1 fragments from stage buffer s & 1,
    //   runs the K-half-0 MFMAs (fragments read during step s - 1) and, before
    //   or after them, mixes its half of B_{s+1} into buffer (s+1) & 1
    //   (B_{s-1}'s, whose last reads came before the previous barrier) and
    //   does its staging slot,
    //   meets the barrier, which publishes B_{s+1},
    //   reads B_{s+1}'s K-half-0 fragments while the K-half-1 MFMAs run.
    // The words a mixing uses were loaded right after the previous mixing.
    uint32_t w[4 * NP2];
    uint32_t rb[RL][4];  // staging slot in flight, ring index = (step within chunk) % RL
    bf16x8_t bk0[2];     // K-half-0 fragments (channel blocks 0, 1) of the coming step
    words(0, w);
    mix_to(w, 0);
    words(1, w);
    lds_barrier();  // tiles zeroed, B_0 staged
#pragma unroll
    for (int s = 0; s < kRow16Slots; ++s) stage_store(tile_of(0), s, lane, r0[s]);
    lds_barrier();  // chunk 0 in tile 0
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) bk0[cb] = bread(0, e, 2 * cb);

    for (int c = 0; c < nchunks; ++c) {
        const uint16_t *tile = tile_of(c & 1);
        uint16_t *tnext = tile_of((c + 1) & 1);  // chunk c - 1's, whose last reads preceded this chunk
        // the last chunk stages a harmless copy of itself into the idle tile
        const auto rs = rsrc_of(min(c + 1, nchunks - 1) * kChunk);
        // Lane index kept opaque per chunk: the staging addresses are
        // recomputed where used rather than held across the whole loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int u = 0; u < K; ++u) {
            // Positions kept opaque per kernel row, like the lane above: the
            // swizzled fragment addresses are computed next to their reads.
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb) asm volatile("" : "+v"(aq[pb]));
            u32x4_t a0f[PBW][2];
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
                    a0f[pb][kh] = *reinterpret_cast<const u32x4_t *>(tile + swz(aq[pb] + u * a.ncols, 2 * kh + lh));
#pragma unroll
            for (int v = 0; v < K; ++v) {
                const int i = u * K + v;       // step within the chunk (compile-time)
                const int par = (c + i) & 1;   // parity of the global step 9 c + i
                bf16x8_t bk1[2];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    bk1[cb] = bread(par, e, 2 * cb + 1);
                // All blocks are computed (rows past Ho are clamped duplicates,
                // dropped in the epilogue), so the MFMA stream has no branches.
                auto mfma_half = [&](int kh, const bf16x8_t (&bf)[2]) {
#pragma unroll
                    for (int pb = 0; pb < PBW; ++pb) {
                        const bf16x8_t afr =
                            __builtin_bit_cast(bf16x8_t, v == 0 ? a0f[pb][kh] : dpp_shl(a0f[pb][kh], v));
#pragma unroll
                        for (int cb = 0; cb < 2; ++cb)
                            acc[pb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bf[cb], acc[pb][cb], 0, 0, 0);
                    }
                };
                // The two waves of a SIMD take the K-half-0 part in opposite
                // orders (pinned with scheduling barriers): the 4-block wave
                // issues its MFMAs first and then mixes and stages, the
                // 3-block wave mixes and stages first, so that each one's
                // dependent mixing chain runs under the other's MFMAs.
                constexpr bool mix_first = PBW == 3;
                if constexpr (!mix_first) {
                    mfma_half(0, bk0);
                    __builtin_amdgcn_sched_barrier(0);
                }
                mix_to(w, par ^ 1);            // B of step 9 c + i + 1
                words(c * KT + i + 2, w);      // for the next step's mixing
                // The slot loaded RL steps ago goes to the next chunk's tile,
                // then this step's slot loads (after the expert words, so
                // waiting for a slot never waits for younger expert words).
                // Every tile write precedes the barrier of step 8, after
                // which the next chunk's first fragments are read.
                if (i >= RL) stage_store(tnext, i - RL, ln, rb[i % RL]);
                if (i < kRow16Slots) stage_load(rs, i, ln, rb[i % RL]);
                if constexpr (mix_first) {
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_half(0, bk0);
                }
                lds_barrier();
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    bk0[cb] = bread(par ^ 1, e, 2 * cb);
                mfma_half(1, bk1);
            }
        }
    }

    // Epilogue through LDS: channel block cb goes to the example's tile
    // cb (no wave reads either any more). D holds, per lane, channel o0 +
    // 32 cb + l32 and positions 8 j + 4 lh + (0..3): 4 consecutive columns
    // of padded row 2 pb + (j >> 1). The valid ones go to
    // ebuf[channel][row * Wo + col] as 2-element words (Wo is even, so a
    // group holds 0, 2 or 4 valid columns). After a barrier (the example's
    // two waves fill the same planes) each block's 32 channel planes are one
    // dense run, as in y; wave hs copies block hs out with 16-byte (or
    // 4-byte) stores.
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        uint16_t *ebuf = tile_of(cb);
        uint32_t *ech = reinterpret_cast<uint32_t *>(ebuf + l32 * a.P);
#pragma unroll
        for (int pb = 0; pb < PBW; ++pb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 2 * (pb0 + pb) + (j >> 1);
                const int col = 8 * (j & 1) + 4 * lh;
                const int e2 = (r * a.Wo + col) >> 1;  // word index (row * Wo + col is even)
                if (r < a.Ho && col < a.Wo) ech[e2] = pack_bf16x2(acc[pb][cb][4 * j], acc[pb][cb][4 * j + 1]);
                if (r < a.Ho && col + 2 < a.Wo)
                    ech[e2 + 1] = pack_bf16x2(acc[pb][cb][4 * j + 2], acc[pb][cb][4 * j + 3]);
            }
        }
    }
    lds_barrier();
    const int cbo = hs;  // block this wave copies out
    const int och = min(32, a.Cout - (o0 + 32 * cbo));  // channels of this block that exist
    if (valid && och > 0) {
        const int bytes = och * a.P * 2;
        char *dst = reinterpret_cast<char *>(y + ((long)b * a.Cout + o0 + 32 * cbo) * a.P);
        const char *src = reinterpret_cast<const char *>(tile_of(cbo));
        if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0 && (bytes & 15) == 0) {
#pragma unroll 4
            for (int off = lane * 16; off < bytes; off += 1024)
                *reinterpret_cast<u32x4_t *>(dst + off) = *reinterpret_cast<const u32x4_t *>(src + off);
        } else {
            for (int off = lane * 4; off < bytes; off += 256)
                *reinterpret_cast<uint32_t *>(dst + off) = *reinterpret_cast<const uint32_t *>(src + off);
        }
    }
}

template <int NP2>
__global__ __launch_bounds__(512) void conv_fused_row16_kernel(const uint16_t *__restrict__ x,
                                                               const uint32_t *__restrict__ packed,
                                                               const float *__restrict__ alpha,
                                                               uint16_t *__restrict__ y, ConvArgs a) {
    // waves 0..3: position blocks 0..3; waves 4..7: blocks 4..6
    if ((threadIdx.x >> 6) < 4) row16_wave<NP2, 4>(x, packed, alpha, y, a, 0);
    else row16_wave<NP2, 3>(x, packed, alpha, y, a, 4);
}

constexpr int kFusedPBW = 4;  // position blocks of 32 per wave: 2 waves cover <= 256 positions
constexpr int kFusedXT = 4;   // staging tasks per lane: 4 * rows * W/2 <= 512 over 128 lanes

int fused_tile_rows(const Geom &g) { return (g.Ho - 1) * g.stride + g.KH; }

size_t fused_lds_bytes(const Geom &g) {
    const size_t tiles = 4 * (size_t)fused_tile_rows(g) * (g.W + 2 * g.pad) * kPosStride * sizeof(uint16_t);
    return tiles + 2 * 4 * 4 * 64 * 16;  // + double-buffered B stage
}

// Static LDS of the row-16 kernel: 2 x 4 tiles of 16 x 16 positions (chunk
// parity x example) and the double-buffered B stage. Conditions: 3x3 taps
// at stride 1, padded rows of at most 16 positions, at most 14 output rows,
// W even (position pairs are 4-byte words of a channel plane, and output
// pieces of 2 elements are 4-byte aligned) and at most 7 x 64 half-tasks
// (2 positions x 4 channels) per wave and chunk.
bool row16_ok(const Geom &g) {
    const int tile_pos = fused_tile_rows(g) * (g.W + 2 * g.pad);
    const int per_g = std::min(g.H, fused_tile_rows(g) - g.pad) * (g.W / 2);
    return g.stride == 1 && g.KH == 3 && g.KW == 3 && g.W + 2 * g.pad <= 16 && g.Ho <= 14 &&
           g.W % 2 == 0 && tile_pos <= kRow16MaxPos && 4 * per_g <= kRow16Slots * 64;
}

template <int NP2>
hipError_t launch_fused_np(const Geom &g, const uint16_t *x, const uint32_t *packed,
                           const float *alpha, uint16_t *y, hipStream_t stream) {
    ConvArgs a = base_args(g);
    a.tile_rows = fused_tile_rows(g);
    a.n_btiles = ceil_div(g.B, 4);
    a.n_otiles = ceil_div(g.Cout, 64);
    const long blocks = (long)a.n_btiles * a.n_otiles;
    if (row16_ok(g)) {
        hipLaunchKernelGGL(conv_fused_row16_kernel<NP2>, dim3((unsigned)blocks), dim3(512), 0, stream, x,
                           packed, alpha, y, a);
        return hipGetLastError();
    }
    const size_t lds = fused_lds_bytes(g);
    auto k = conv_fused_kernel<kFusedPBW, NP2, kFusedXT>;
    if (hipError_t e = set_lds(k, lds); e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(512), lds, stream, x, packed, alpha, y, a);
    return hipGetLastError();
}

}  // namespace

bool fused_conv_supported(const Geom &g) {
    const int rows = std::min(g.H, fused_tile_rows(g) - g.pad);
    return g.bf16 && g.groups == 1 && g.n_pad <= 4 && g.P <= 2 * kFusedPBW * 32 &&
           g.W % 2 == 0 && 4 * rows * (g.W / 2) <= 128 * kFusedXT &&
           fused_lds_bytes(g) <= (size_t)kLdsBudget;
}

hipError_t launch_conv_fused(const Geom &g, const uint16_t *x, const uint16_t *packed,
                             const float *alpha, uint16_t *y, hipStream_t stream, ChanAttn att) {
    // channel attentions: the 3x3 small-image kernel only
    if (att.in || att.out)
        return fused_wave_attn_ok(g) ? launch_conv_fused_wave(g, x, packed, alpha, y, stream, att)
                                     : hipErrorInvalidValue;
    if (fused_wave_ok(g)) return launch_conv_fused_wave(g, x, packed, alpha, y, stream);
    const uint32_t *pk = reinterpret_cast<const uint32_t *>(packed);
    switch (g.n_pad / 2) {
    case 1: return launch_fused_np<1>(g, x, pk, alpha, y, stream);
    case 2: return launch_fused_np<2>(g, x, pk, alpha, y, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dynconv
