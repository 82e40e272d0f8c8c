// Fused mixing + 3x3 convolution for small images (rows of at most 14
// outputs, at most 14 output rows): the ResNet-50-shaped layer, 256 -> 256
// channels at 14x14. W_b = sum_i alpha_bi E_i (KernelWarehouse: Rethinking
// the Design of Dynamic Convolution, abstract) is formed inside the GEMM and
// never reaches memory; the convolution with it is one ordinary convolution
// per example (CondConv: Conditionally Parameterized Convolutions, abstract).
//
// Work split. A workgroup owns 4 examples and 64 output channels with 8
// waves, two per SIMD (waves w and w + 4 share a SIMD). An example's
// outputs are 7 blocks of 32 positions (two output rows padded to 16) x 2
// tiles of 32 channels: 14 accumulator tiles of 32x32 fp32. Wave w owns
// example w & 3 and half w >> 2 of its tiles: blocks 0..3 without channel
// tile 1 of block 3, or blocks 3..6 without channel tile 0 of block 3. The
// two waves of a SIMD thus do equal work on one example and each hides the
// other's waits. Each MFMA (v_mfma_f32_32x32x16_bf16) takes 32 positions x
// 16 input channels of one tap as A and 16 input channels x 32 output
// channels of W_b as B.
//
// Input tile. The two waves of an example stage its input, 16 channels at a
// time, into the example's LDS tile of 16 x 16 positions (tile row = input
// row + 1, tile column = input column; padding rows and the columns past the
// image stay zero) after one zero guard position. Positions are 48 bytes
// apart (32 bytes of channels and 16 of padding), so the 16-byte reads of
// any 16 consecutive positions fall on distinct banks. Tap (u, v) of output
// position (r, c) is tile column c + v - 1 of tile row r + u. Only the
// centre tap (v = 1) of each kernel row is read from LDS (one 16-byte read
// per lane and position block); a lane holds one column of a 16-lane row,
// so the left and right taps are the same registers moved one lane within
// the row (DPP), with a zero entering at the row ends.
//
// Mixing on the matrix cores. v_mfma_f32_4x4x4_16b_bf16 computes 16
// independent 4x4x4 products: with the 4 examples' attention rows as A and
// one weight's 4 expert values per lane as B (from the packed bank,
// packed[t][o][c][i]), lane l receives the 4 examples' mixed values of its
// weight. Attentions are split in a bf16 high part and the rounding
// remainder (two products accumulated in fp32); the sum is rounded once to
// bf16. Every lane of the workgroup mixes 2 input channels of one output
// channel for the three taps of a kernel row, so the workgroup forms all of
// a group's B fragments for all 4 examples and each expert word is read once
// per workgroup. The fragments pass to their waves through a double-buffered
// LDS stage.
//
// Schedule. The K loop runs over groups g = (16-channel chunk, kernel row
// u): 3 taps per group. During group g a wave mixes group g + 1 from expert
// words loaded during group g - 1 and loads the words of group g + 2. One
// workgroup barrier per group, placed after the second tap: it publishes
// group g + 1's fragments; those of its first two taps are read before the
// third tap's MFMAs, the rest (with the next row's centre fragments) after.
// The next chunk's input loads a chunk ahead and reaches the other tile
// during the chunk's first two groups.
//
// Epilogue. Each wave writes its valid outputs into LDS as 64 dense channel
// planes of its example (the example's part of y is one contiguous run), and
// the example's two waves copy them to y with 16-byte stores.
#include <type_traits>

#include "conv_common.hpp"

namespace dynconv {
namespace {

constexpr int kWvChunk = 16;                       // input channels per chunk
constexpr int kWvPosBytes = 48;                    // 16 channels x 2 bytes + 16 bytes of padding
constexpr int kWvTileBytes = 12800;                // guard + 16 x 16 positions (+ overreach of junk lanes)
constexpr int kWvStageBytes = 2 * 3 * 2 * 4 * 1024;  // [buf][tap][tile][example] x 1 KB
constexpr int kWvLdsBytes = 4 * 2 * kWvTileBytes + kWvStageBytes;  // 148 KB
constexpr int kWvRounds = 4;                       // staging rounds of 128 tasks (two waves) per chunk
constexpr int kWvThreads = 512;
static_assert((1 + 16 * 16 + 1) * kWvPosBytes <= kWvTileBytes, "tile holds the guard and every read");
constexpr int kWvAinMax = 768;  // input channels (padded) whose attentions fit beside the tiles and the stage

__shared__ __attribute__((aligned(16))) u32x4_t s_wv[kWvLdsBytes / 16];

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Byte offset in a tile of tile position q (the guard is position -1).
__device__ __forceinline__ int wv_pos(int q) { return (q + 1) * kWvPosBytes; }

// Lanes 16 k .. 16 k + 15 of an A fragment hold the 16 columns of one tile
// row. The left and right taps of a position are the centre taps of its
// left and right neighbours: the centre fragment read from lane l - 1
// (v_mov_b32_dpp row_shr:1) or lane l + 1 (row_shl:1) of the same row of 16
// lanes. A lane whose source is outside its row receives 0: on the left that
// is the zero padding column; on the right the lane is column 15, past every
// output column.
__device__ __forceinline__ u32x4_t left_neighbour(u32x4_t x) {
    return u32x4_t{(uint32_t)__builtin_amdgcn_mov_dpp((int)x.x, 0x111, 0xf, 0xf, true),
                   (uint32_t)__builtin_amdgcn_mov_dpp((int)x.y, 0x111, 0xf, 0xf, true),
                   (uint32_t)__builtin_amdgcn_mov_dpp((int)x.z, 0x111, 0xf, 0xf, true),
                   (uint32_t)__builtin_amdgcn_mov_dpp((int)x.w, 0x111, 0xf, 0xf, true)};
}
__device__ __forceinline__ u32x4_t right_neighbour(u32x4_t x) {
    return u32x4_t{(uint32_t)__builtin_amdgcn_mov_dpp((int)x.x, 0x101, 0xf, 0xf, true),
                   (uint32_t)__builtin_amdgcn_mov_dpp((int)x.y, 0x101, 0xf, 0xf, true),
                   (uint32_t)__builtin_amdgcn_mov_dpp((int)x.z, 0x101, 0xf, 0xf, true),
                   (uint32_t)__builtin_amdgcn_mov_dpp((int)x.w, 0x101, 0xf, 0xf, true)};
}

// 64-bit pointer as a buffer descriptor of nbytes (reads past it return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wv_rsrc(const void *p, int nbytes) {
    const uint64_t q = reinterpret_cast<uint64_t>(p);
    const uint64_t qs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)q) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(q >> 32)) << 32);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(qs), 0,
                                             __builtin_amdgcn_readfirstlane(nbytes), 0x00020000);
}

// 4 experts: each weight is two words (expert pairs) of the packed bank.
// ATT: FMDConv's channel attentions (either pointer may be null): a_in[b,c]
// scales every mixed weight of input channel c before its rounding, a_out[b,o]
// scales the fp32 accumulators of output channel o before theirs.
template <bool ATT>
__global__ __launch_bounds__(kWvThreads) void conv_fused_wave_kernel(const uint16_t *__restrict__ x,
                                                                     const uint32_t *__restrict__ packed,
                                                                     const float *__restrict__ alpha,
                                                                     uint16_t *__restrict__ y, ConvArgs a,
                                                                     const float *__restrict__ a_in,
                                                                     const float *__restrict__ a_out) {
    char *lds = reinterpret_cast<char *>(s_wv);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int e = w & 3;   // example of this wave
    const int h = w >> 2;  // output rows 0..7 or 8..13
    const int lane = tid & 63;
    // XCD k holds logical tiles [32k, 32k + 32): 8 example quads x all 4
    // channel tiles, so an example's input and a channel tile's expert slice
    // are both fetched once per XCD.
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int ot = logical % a.n_otiles;
    const int bt = logical / a.n_otiles;
    const int o0 = ot * 64;
    const int b_raw = bt * 4 + e;
    const bool valid = b_raw < a.B;
    const int b = valid ? b_raw : a.B - 1;

    auto tile = [&](int ex, int buf) { return lds + (ex * 2 + buf) * kWvTileBytes; };
    auto stage = [&](int buf, int v, int n, int ex) {
        return lds + 4 * 2 * kWvTileBytes + (((buf * 3 + v) * 2 + n) * 4 + ex) * 1024;
    };
    // input attentions of the 4 examples, zero past Cin (visible to the mixing
    // after the prologue's first barrier)
    __shared__ __attribute__((aligned(16))) float s_ain[ATT ? 4 * kWvAinMax : 1];
    if constexpr (ATT) {
        if (a_in)
            for (int i = tid; i < 4 * a.Cin_pad; i += kWvThreads) {
                const int ex = i / a.Cin_pad, c = i - ex * a.Cin_pad;
                const int bb = bt * 4 + ex;
                s_ain[i] = (c < a.Cin && bb < a.B) ? a_in[(long)bb * a.Cin + c] : 0.f;
            }
    }

    // ---- mixing role: output channel o0 + om, channels 8 kh + 2 mp and
    // 8 kh + 2 mp + 1 of each chunk
    const int om = 16 * e + (lane >> 2);
    const int kh = h;
    const int mp = lane & 3;
    s16x4_t ahi, alo;
    {
        const int be = min(bt * 4 + (lane & 3), a.B - 1);
        const bool live = bt * 4 + (lane & 3) < a.B;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float v = (k < a.n && live) ? alpha[(long)be * a.n + k] : 0.f;
            const uint16_t hb = f32_to_bf16(v);
            ahi[k] = (short)hb;
            alo[k] = (short)f32_to_bf16(v - bf16_to_f32(hb));
        }
    }
    // Expert words: the bank as a buffer (groups past the last read zeros);
    // lane offset for output channel o0 + om and its channel pair of chunk 0,
    // one scalar offset per tap. A channel's 4 experts are 8 bytes, so the
    // pair is one 16-byte load.
    const int tap_bytes = a.Cout * a.Cin_pad * 8;
    const auto bank = wv_rsrc(packed, 9 * tap_bytes);
    const int wlane = (min(o0 + om, a.Cout - 1) * a.Cin_pad + 8 * kh + 2 * mp) * 8;
    const int nchunks = a.Cin_pad / kWvChunk;
    auto load_words = [&](int c, int u, u32x4_t (&wd)[3]) {
        const int vo = wlane + c * (kWvChunk * 8);
#pragma unroll
        for (int v = 0; v < 3; ++v) {
            const int so = __builtin_amdgcn_readfirstlane((3 * u + v) * tap_bytes);
            wd[v] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(bank, vo, so, 0));
        }
    };
    // Consumer lanes of the mixed words: output channel om & 31 of tile
    // om >> 5 holds channels 0..7 of the chunk in lane om & 31 and channels
    // 8..15 in lane 32 + (om & 31); channel pair mp is its 4 bytes at 4 mp.
    // One stage write of a wave covers 16 whole consumer lanes: 256
    // contiguous bytes.
    const int moff = ((om & 31) + 32 * kh) * 16 + mp * 4;
    const int mtile = om >> 5;
    // The input attentions of the lane's two channels of chunk cm for the 4
    // examples (ones without input attentions).
    auto read_ain = [&](int cm, f32x2_t (&ai)[4]) {
#pragma unroll
        for (int ex = 0; ex < 4; ++ex) ai[ex] = f32x2_t{1.f, 1.f};
        if constexpr (ATT) {
            if (a_in) {
                const int ch = cm * kWvChunk + 8 * kh + 2 * mp;
#pragma unroll
                for (int ex = 0; ex < 4; ++ex) ai[ex] = *reinterpret_cast<const f32x2_t *>(&s_ain[ex * a.Cin_pad + ch]);
            }
        }
    };
    // One tap: the high-part products of both channels, the low-part products
    // accumulated onto them (times the input attentions ai), one 4-byte stage
    // write per example.
    auto mix_tap = [&](const u32x4_t wv, int buf, int v, const f32x2_t (&ai)[4]) {
        u32x2_t e0, e1;
        e0.x = wv.x; e0.y = wv.y;
        e1.x = wv.z; e1.y = wv.w;
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        f32x4_t d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi, __builtin_bit_cast(s16x4_t, e0), z, 0, 0, 0);
        f32x4_t d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi, __builtin_bit_cast(s16x4_t, e1), z, 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo, __builtin_bit_cast(s16x4_t, e0), d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo, __builtin_bit_cast(s16x4_t, e1), d1, 0, 0, 0);
        if constexpr (ATT) {
#pragma unroll
            for (int ex = 0; ex < 4; ++ex) {
                d0[ex] *= ai[ex][0];
                d1[ex] *= ai[ex][1];
            }
        }
#pragma unroll
        for (int ex = 0; ex < 4; ++ex)
            *reinterpret_cast<uint32_t *>(stage(buf, v, mtile, ex) + moff) = pack_bf16x2(d0[ex], d1[ex]);
    };

    // ---- convolution role
    // zero both tiles of this example (guard, padding rows and columns)
    {
        u32x4_t z = {0u, 0u, 0u, 0u};
        u32x4_t *t0 = reinterpret_cast<u32x4_t *>(tile(e, 0));
        for (int i = h * 64 + lane; i < 2 * kWvTileBytes / 16; i += 128) t0[i] = z;
    }
    const uint16_t *xb = x + (long)b * a.x_bstride;
    const int HW = a.H * a.W;
    const int plane = HW * 2;  // bytes per input channel plane
    const int pairs = a.W >> 1;
    const int per_g = a.H * pairs;  // position pairs per channel
    const int ntasks = 4 * per_g;   // (position pair, channel quad) tasks per chunk
    // Buffer descriptor of chunk c's 16 channel planes; channels past Cin
    // are beyond its extent and read as zeros.
    auto rsrc_of = [&](int c) {
        const int c0 = min(c * kWvChunk, a.Cin - 1);
        return wv_rsrc(xb + (long)c0 * HW, max(0, min(kWvChunk, a.Cin - c * kWvChunk)) * plane);
    };
    // Staging task k: channel quad k / per_g, row r, column pair kp: 4 dword
    // loads (one per channel, both positions) and two 8-byte tile writes.
    // The example's two waves take tasks 128 i + 64 h + lane (the last
    // repeats: same bytes, same place). Source and destination offsets do
    // not depend on the chunk: computed once, packed as source | destination
    // << 16 (both below 2^16).
    uint32_t stask[kWvRounds];
#pragma unroll
    for (int i = 0; i < kWvRounds; ++i) {
        const int k = min(i * 128 + h * 64 + lane, ntasks - 1);
        const int g4 = k / per_g, rem = k - g4 * per_g;
        const int row = rem / pairs, kp = rem - row * pairs;
        const int vo = 4 * g4 * plane + 4 * rem;  // channel 4 g4, row r, columns 2 kp, 2 kp + 1
        const int dst = wv_pos((row + 1) * 16 + 2 * kp) + 8 * g4;  // position + 1 is 48 bytes further
        stask[i] = (uint32_t)vo | ((uint32_t)dst << 16);
    }
    auto st_load = [&](__amdgpu_buffer_rsrc_t rs, int round, uint32_t (&r)[4]) {
        const int vo = (int)(stask[round] & 0xffffu);
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo + j * plane, 0, 0);
    };
    auto st_store = [&](char *t, int round, const uint32_t (&r)[4]) {
        const int dst = (int)(stask[round] >> 16);
        u32x2_t p0, p1;
        p0.x = __builtin_amdgcn_perm(r[1], r[0], 0x05040100u); p0.y = __builtin_amdgcn_perm(r[3], r[2], 0x05040100u);
        p1.x = __builtin_amdgcn_perm(r[1], r[0], 0x07060302u); p1.y = __builtin_amdgcn_perm(r[3], r[2], 0x07060302u);
        *reinterpret_cast<u32x2_t *>(t + dst) = p0;
        *reinterpret_cast<u32x2_t *>(t + dst + kWvPosBytes) = p1;
    };

    // A fragments: block pb, lane: output row 2 pb + (lane & 31) / 16, column
    // lane & 15, channel half lane / 32; the centre tap of kernel row u adds
    // 16 (u - 1) positions to the output position's own tile position
    // (row + 1, col).
    const int aoff = wv_pos((((lane & 31) >> 4) + 1) * 16 + (lane & 15)) + 16 * (lane >> 5);
    auto read_b = [&](int buf, int v, bf16x8_t (&bf)[2]) {
#pragma unroll
        for (int n = 0; n < 2; ++n) bf[n] = *reinterpret_cast<const bf16x8_t *>(stage(buf, v, n, e) + lane * 16);
    };

    // The wave's tiles: blocks 3 HF .. 3 HF + 3 (local block 0..3), both
    // channel tiles except on block 3, which the two halves split (channel
    // tile 0 to the first, 1 to the second): 7 tiles per wave. Both halves
    // run the same sequence of barriers.
    auto body = [&](auto hf_c) {
        constexpr int HF = decltype(hf_c)::value;
        constexpr int PB0 = 3 * HF;
        constexpr int NPB = 4;
        auto owns = [](int pb, int n) { return PB0 + pb != 3 || n == HF; };
        auto read_centre = [&](const char *t, int u, u32x4_t (&f)[NPB]) {
            const char *tb = t + aoff + (16 * (u - 1) + PB0 * 32) * kWvPosBytes;
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb) f[pb] = *reinterpret_cast<const u32x4_t *>(tb + pb * 32 * kWvPosBytes);
        };
        f32x16_t acc[NPB][2];
#pragma unroll
        for (int i = 0; i < NPB; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
        auto mfma_pb = [&](const u32x4_t af, const bf16x8_t (&bf)[2], int pb) {
            const bf16x8_t av = __builtin_bit_cast(bf16x8_t, af);
#pragma unroll
            for (int n = 0; n < 2; ++n)
                if (owns(pb, n)) acc[pb][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bf[n], acc[pb][n], 0, 0, 0);
        };

        // ---- prologue: chunk 0 staged, chunk 1's input in flight, group 0
        // mixed into stage buffer 0, words of groups 1 and 2 in flight
        uint32_t sr[kWvRounds][4];  // the next chunk's input, loaded a chunk ahead of its tile writes
        u32x4_t wq[2][3];           // words of groups of each parity, loaded two groups ahead
        {
            const auto rs0 = rsrc_of(0);
#pragma unroll
            for (int i = 0; i < kWvRounds; ++i) st_load(rs0, i, sr[i]);
            load_words(0, 0, wq[0]);
            lds_barrier();  // both waves' tile zeroing precedes the staging writes
#pragma unroll
            for (int i = 0; i < kWvRounds; ++i) st_store(tile(e, 0), i, sr[i]);
            const auto rs1 = rsrc_of(min(1, nchunks - 1));
#pragma unroll
            for (int i = 0; i < kWvRounds; ++i) st_load(rs1, i, sr[i]);
            load_words(0, 1, wq[1]);
            {
                f32x2_t ai0[4];
                read_ain(0, ai0);
#pragma unroll
                for (int v = 0; v < 3; ++v) mix_tap(wq[0][v], 0, v, ai0);
            }
        }
        load_words(0, 2, wq[0]);
        lds_barrier();  // stage buffer 0 and tile 0 complete
        bf16x8_t bcur[3][2];
#pragma unroll
        for (int v = 0; v < 3; ++v) read_b(0, v, bcur[v]);
        u32x4_t acur[NPB];  // centre-column fragments of the current group
        read_centre(tile(e, 0), 0, acur);

        // Chunk c (its parity CP fixes which word buffer each group uses).
        auto chunk = [&](int c, auto cp_c) {
            constexpr int CP = decltype(cp_c)::value;
            const char *tcur = tile(e, CP);
            char *tnext = tile(e, CP ^ 1);
            const auto rs2 = rsrc_of(min(c + 2, nchunks - 1));
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int nb = (u + CP + 1) & 1;  // stage buffer of group g + 1
                u32x4_t (&wn)[3] = wq[nb];        // words of group g + 1
                // the next chunk's input goes to its tile (written during
                // groups 0 and 1; the last chunk rewrites a copy of itself
                // into the idle tile), and the chunk after it starts loading
                // into the same registers
                if (u < 2) {
#pragma unroll
                    for (int i = 2 * u; i < 2 * u + 2; ++i) st_store(tnext, i, sr[i]);
#pragma unroll
                    for (int i = 2 * u; i < 2 * u + 2; ++i) st_load(rs2, i, sr[i]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // tap 0 (left column: the centre fragments one lane down)
                // with the mixing of group g + 1's tap 0
#pragma unroll
                for (int pb = 0; pb < NPB; ++pb) mfma_pb(left_neighbour(acur[pb]), bcur[0], pb);
                f32x2_t ai[4];
                read_ain(u < 2 ? c : c + 1, ai);  // chunk of group g + 1
                mix_tap(wn[0], nb, 0, ai);
                __builtin_amdgcn_sched_barrier(0);
                // tap 1 (centre) with the rest; then the words of group g + 3
                // load into the buffer just used
#pragma unroll
                for (int pb = 0; pb < NPB; ++pb) mfma_pb(acur[pb], bcur[1], pb);
                mix_tap(wn[1], nb, 1, ai);
                mix_tap(wn[2], nb, 2, ai);
                __builtin_amdgcn_sched_barrier(0);
                // group g + 3 is (chunk c + 1, row u)
                load_words(c + 1, u, wn);
                // the group's B fragments are in registers (read after the
                // previous barrier), so the stage buffer g + 1 writes into is
                // free
                lds_barrier();
                // taps 0 and 1 of the next group replace those of this one
                read_b(nb, 0, bcur[0]);
                read_b(nb, 1, bcur[1]);
                __builtin_amdgcn_sched_barrier(0);
                // tap 2 (right column: the centre fragments one lane up)
#pragma unroll
                for (int pb = 0; pb < NPB; ++pb) mfma_pb(right_neighbour(acur[pb]), bcur[2], pb);
                // each block's 4 lane moves just ahead of its MFMAs
                // (mask 0x002: VALU, 0x008: MFMA)
                if constexpr (HF == 0) {
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                } else {
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                // the next group's centre fragments and tap-2 B fragments
                read_centre(u < 2 ? tcur : tnext, u < 2 ? u + 1 : 0, acur);
                read_b(nb, 2, bcur[2]);
            }
        };
        for (int c = 0; c < nchunks; c += 2) {
            chunk(c, std::integral_constant<int, 0>{});
            if (c + 1 < nchunks) chunk(c + 1, std::integral_constant<int, 1>{});
        }

        // ---- epilogue: dense channel planes of the example in LDS
        lds_barrier();  // every wave is done with the tiles and the stage
        const int P = a.P;
        const int ah = lane >> 5;
        uint32_t *ew = reinterpret_cast<uint32_t *>(lds + e * (64 * P * 2));
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int ch = 32 * n + (lane & 31);
            if constexpr (ATT) {
                if (a_out) {
                    const float ao = a_out[(long)b * a.Cout + min(o0 + ch, a.Cout - 1)];
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
                        for (int q = 0; q < 16; ++q) acc[pb][n][q] *= ao;
                }
            }
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb) {
                if (!owns(pb, n)) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 2 * (PB0 + pb) + (j >> 1);
                    const int col = 8 * (j & 1) + 4 * ah;
                    const int w2 = (ch * P + r * a.Wo + col) >> 1;  // P and Wo even: word aligned
                    if (r < a.Ho && col < a.Wo) ew[w2] = pack_bf16x2(acc[pb][n][4 * j], acc[pb][n][4 * j + 1]);
                    if (r < a.Ho && col + 2 < a.Wo)
                        ew[w2 + 1] = pack_bf16x2(acc[pb][n][4 * j + 2], acc[pb][n][4 * j + 3]);
                }
            }
        }
    };
    if (h == 0) body(std::integral_constant<int, 0>{});
    else body(std::integral_constant<int, 1>{});

    // ---- copy-out: the example's two waves copy its planes with 16-byte
    // stores
    lds_barrier();  // both halves of every example are in LDS
    const int P = a.P;
    const char *ebuf = lds + e * (64 * P * 2);
    const int och = min(64, a.Cout - o0);
    if (valid && och > 0) {
        const int bytes = och * P * 2;
        char *dst = reinterpret_cast<char *>(y + ((long)b * a.Cout + o0) * P);
        if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0 && (bytes & 15) == 0) {
            for (int off = (h * 64 + lane) * 16; off < bytes; off += 2048)
                *reinterpret_cast<u32x4_t *>(dst + off) = *reinterpret_cast<const u32x4_t *>(ebuf + off);
        } else {
            for (int off = (h * 64 + lane) * 4; off < bytes; off += 512)
                *reinterpret_cast<uint32_t *>(dst + off) = *reinterpret_cast<const uint32_t *>(ebuf + off);
        }
    }
}

}  // namespace

// 3x3, stride 1, padding 1, at most 14 x 14 outputs (7 blocks of two rows
// padded to 16), 3 or 4 experts (two expert-pair words per weight), even W
// (position pairs are 4-byte words of a channel plane), the staging tasks of
// a chunk within 4 rounds of 128 lanes, and the four examples' output planes
// within the LDS.
bool fused_wave_ok(const Geom &g) {
    return g.stride == 1 && g.KH == 3 && g.KW == 3 && g.pad == 1 && g.H <= 14 && g.W <= 14 &&
           g.W % 2 == 0 && g.H * (g.W / 2) * 4 <= kWvRounds * 128 && 4 * 64 * g.P * 2 <= kWvLdsBytes &&
           16 * g.H * g.W * 2 < (1 << 16) && 9L * g.Cout * g.Cin_pad * 8 < (1L << 31) && g.n_pad == 4 &&
           g.Cin_pad % kWvChunk == 0;
}

bool fused_wave_attn_ok(const Geom &g) { return fused_wave_ok(g) && g.Cin_pad <= kWvAinMax; }

hipError_t launch_conv_fused_wave(const Geom &g, const uint16_t *x, const uint16_t *packed, const float *alpha,
                                  uint16_t *y, hipStream_t stream, ChanAttn att) {
    ConvArgs a = base_args(g);
    a.tile_rows = 16;
    a.n_btiles = ceil_div(g.B, 4);
    a.n_otiles = ceil_div(g.Cout, 64);
    const long blocks = (long)a.n_btiles * a.n_otiles;
    const uint32_t *pk = reinterpret_cast<const uint32_t *>(packed);
    if (att.in || att.out) {
        if (!fused_wave_attn_ok(g)) return hipErrorInvalidValue;
        hipLaunchKernelGGL(conv_fused_wave_kernel<true>, dim3((unsigned)blocks), dim3(kWvThreads), 0, stream, x, pk,
                           alpha, y, a, att.in, att.out);
    } else {
        hipLaunchKernelGGL(conv_fused_wave_kernel<false>, dim3((unsigned)blocks), dim3(kWvThreads), 0, stream, x, pk,
                           alpha, y, a, nullptr, nullptr);
    }
    return hipGetLastError();
}

}  // namespace dynconv
