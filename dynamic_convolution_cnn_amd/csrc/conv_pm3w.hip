// Per-example 3x3 stride-1 convolution on bf16 MFMA from mixed kernels
// already in memory, wt[b][t][o][cp] (the premix layout): one ordinary
// convolution per example with that example's own kernel (CondConv:
// Conditionally Parameterized Convolutions, abstract), for images too large
// for the fused small-image kernels (the ResNet-18-shaped 56x56 layer and the
// many-expert 28x28 layer).
//
// Work split. A workgroup of 4 waves owns example b, NT = 32 NCB output
// channels and MT = 4 * 32 NPB consecutive output positions (row-major);
// wave w owns position blocks w NPB .. w NPB + NPB - 1 (32 positions each)
// over all NT channels: NPB x NCB accumulator tiles of
// v_mfma_f32_32x32x16_bf16 (positions x channels). An A fragment feeds NCB
// MFMAs and a B fragment NPB, so a step reads (NPB + NCB) KB of LDS per
// NPB NCB MFMAs. Launched with 2 x 2 tiles: 256 positions x 64 channels,
// whose LDS (at most 80 KB at the 56x56 and 28x28 layers) lets two
// workgroups share a CU, so each SIMD runs two waves and the grid covers
// the 56x56 planes with 6 % padding instead of 14 %. Larger per-wave tiles
// read less LDS per MFMA but leave one workgroup per CU; measured slower.
//
// K loop. Chunks of 16 input channels; within a chunk, 9 steps (taps), one
// MFMA K of 16 each. Per chunk two LDS buffers are filled for the next chunk
// while the current one is read:
//   - the input tile: the padded input rows the tile's outputs read, 48-byte
//     positions (16 channels + 16 bytes of padding, so any 8 consecutive
//     positions fall on distinct banks), zero padding written once; tap
//     (u, v) of an output is its tile position plus u rows and v columns, a
//     fixed offset per (lane, u) plus an immediate;
//   - the B tile: the chunk's slice of W_b for the NT channels and 9 taps,
//     laid out as the MFMA's B fragments (1 KB per (tap, channel block)).
// Both load into registers two chunks ahead of their use (two register sets,
// loads in the chunk's steps 3..8) and reach LDS in steps 0..2 of the chunk
// before their use. One workgroup
// barrier per chunk, before the last step's MFMAs, publishes them; the next
// chunk's first fragments are read while those MFMAs run.
//
// Epilogue. The accumulators (times the optional output attention) go to LDS
// as NT channel rows of MT positions, then out along y's rows with 16-byte
// stores.
#include <type_traits>

#include "conv_common.hpp"

namespace dynconv {
namespace {

constexpr int kQChunk = 16;   // input channels per chunk (one MFMA K)
constexpr int kQPos = 48;     // bytes per input tile position
constexpr int kQLdsMax = 160 * 1024;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t q_rsrc(const void *p, int nbytes) {
    const uint64_t q = reinterpret_cast<uint64_t>(p);
    const uint64_t qs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)q) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(q >> 32)) << 32);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(qs), 0,
                                             __builtin_amdgcn_readfirstlane(nbytes), 0x00020000);
}

// XR: input staging rounds of 256 tasks per chunk; BR: B pieces (16 bytes)
// per lane per chunk.
template <int NPB, int NCB, int XR, int BR>
__global__ __launch_bounds__(256) void conv_pm3w_kernel(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ wt,
                                                        uint16_t *__restrict__ y, ConvArgs a, int tile_bytes,
                                                        const float *__restrict__ a_out) {
    extern __shared__ __attribute__((aligned(16))) char q_lds[];
    constexpr int MT = 4 * NPB * 32;
    constexpr int NT = NCB * 32;
    constexpr int BT = 9 * NCB * 1024;  // B tile bytes
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int per_b = a.n_ptiles * a.n_otiles;
    const int b = logical / per_b;
    const int rem = logical - b * per_b;
    const int pt = rem / a.n_otiles, ot = rem - pt * a.n_otiles;
    const int p0 = pt * MT, o0 = ot * NT;
    const int r_first = p0 / a.Wo;
    const int h_tile0 = r_first - a.pad;  // input row of tile row 0
    const int h_lo = max(0, h_tile0), h_hi = min(a.H, h_tile0 + a.tile_rows);
    auto xtile = [&](int buf) { return q_lds + buf * tile_bytes; };
    auto btile = [&](int buf) { return q_lds + 2 * tile_bytes + buf * BT; };


    // A fragment base offsets: block pb, kernel row u (column tap v is +48 v)
    int aoff[3][NPB];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
        const int p = min(p0 + 32 * (wave * NPB + pb) + l32, a.P - 1);
        const int r = p / a.Wo, s = p - r * a.Wo;
        const int q = (r - r_first) * a.ncols + s;
#pragma unroll
        for (int u = 0; u < 3; ++u) aoff[u][pb] = (q + u * a.ncols) * kQPos + 16 * lh;
    }

    // ---- input staging: task p = (channel octet p / per_g, staged row, column
    // pair), taken by a pair of adjacent lanes: lane half h loads channels
    // 4 h .. 4 h + 3 of the octet (4 dword loads, one per channel, both
    // positions), the pair swaps one 8-byte half (DPP), and lane h writes the
    // octet of position 2 kp + h as one 16-byte piece. The pieces of 8
    // consecutive lanes (4 column pairs, 96 bytes apart) fall on distinct
    // banks; as 8-byte writes of channel quads they met 4 to a bank.
    const uint16_t *xb = x + (long)b * a.x_bstride;
    const int HW = a.H * a.W, plane = HW * 2, pairs = a.W >> 1;
    const int nrows = max(1, h_hi - h_lo);
    const int per_g = nrows * pairs;
    const int npt = 2 * per_g;  // pair tasks per chunk
    const int half = tid & 1;
    // (k + 0.5) * fl(1 / d) rounded down is k / d exactly in float32 for
    // k < 8192 and d <= 4096 (checked exhaustively), which the launch
    // conditions guarantee; it avoids integer division in the prologue.
    const float inv_g = 1.f / (float)per_g, inv_pairs = 1.f / (float)pairs;
    int xsrc[XR], xdst[XR];
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        // lanes past the last task repeat it (same data to the same place)
        const int k = min(128 * i + (tid >> 1), npt - 1);
        const int g8 = (int)(((float)k + 0.5f) * inv_g), rr = k - g8 * per_g;
        const int row = (int)(((float)rr + 0.5f) * inv_pairs), kp = rr - row * pairs;
        xsrc[i] = (8 * g8 + 4 * half) * plane + (row * a.W + 2 * kp) * 2;
        xdst[i] = ((h_lo - h_tile0 + row) * a.ncols + 2 * kp + a.pad + half) * kQPos + 16 * g8;
    }
    auto x_rsrc = [&](int c) {
        const int c0 = min(c * kQChunk, a.Cin - 1);
        const int nb = max(0, min(kQChunk, a.Cin - c * kQChunk)) * plane - h_lo * a.W * 2;
        return q_rsrc(xb + (long)c0 * HW + (long)h_lo * a.W, max(0, nb));
    };
    auto x_load1 = [&](__amdgpu_buffer_rsrc_t rs, int i, uint32_t (&r)[XR][4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[i][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, xsrc[i] + j * plane, 0, 0);
    };
    auto x_store1 = [&](char *t, int i, const uint32_t (&r)[XR][4]) {
        // q0: this lane's 4 channels at position 2 kp, q1: at 2 kp + 1
        uint32_t q0x = __builtin_amdgcn_perm(r[i][1], r[i][0], 0x05040100u);
        uint32_t q0y = __builtin_amdgcn_perm(r[i][3], r[i][2], 0x05040100u);
        uint32_t q1x = __builtin_amdgcn_perm(r[i][1], r[i][0], 0x07060302u);
        uint32_t q1y = __builtin_amdgcn_perm(r[i][3], r[i][2], 0x07060302u);
        // the even lane sends its position-1 quad, the odd lane its
        // position-0 quad (quad_perm [1, 0, 3, 2] swaps adjacent lanes)
        const uint32_t sx = half ? q0x : q1x, sy = half ? q0y : q1y;
        const uint32_t rx = (uint32_t)__builtin_amdgcn_mov_dpp((int)sx, 0xB1, 0xF, 0xF, false);
        const uint32_t ry = (uint32_t)__builtin_amdgcn_mov_dpp((int)sy, 0xB1, 0xF, 0xF, false);
        const u32x4_t o = half ? u32x4_t{rx, ry, q1x, q1y} : u32x4_t{q0x, q0y, rx, ry};
        *reinterpret_cast<u32x4_t *>(t + xdst[i]) = o;
    };
    auto x_load = [&](__amdgpu_buffer_rsrc_t rs, uint32_t (&r)[XR][4]) {
#pragma unroll
        for (int i = 0; i < XR; ++i) x_load1(rs, i, r);
    };
    auto x_store = [&](char *t, const uint32_t (&r)[XR][4]) {
#pragma unroll
        for (int i = 0; i < XR; ++i) x_store1(t, i, r);
    };

    // ---- B staging: piece k = (tap, output channel, channel half) of the
    // chunk's 16 channels, 16 bytes from wt, 16 bytes to the B tile
    int bsrc[BR], bdst[BR];
#pragma unroll
    for (int i = 0; i < BR; ++i) {
        const int k = min(256 * i + tid, 9 * NT * 2 - 1);
        const int t = k / (2 * NT), rr = k - t * 2 * NT;
        const int ol = rr >> 1, h = rr & 1;
        const int o = min(o0 + ol, a.Cout - 1);
        bsrc[i] = ((t * a.Cout + o) * a.Cin_pad + 8 * h) * 2;
        bdst[i] = (t * NCB + (ol >> 5)) * 1024 + ((ol & 31) + 32 * h) * 16;
    }
    const int wbytes = 9 * a.Cout * a.Cin_pad * 2;
    const auto wrs = q_rsrc(wt + (long)b * 9 * a.Cout * a.Cin_pad, wbytes);
    auto b_load1 = [&](int c, int i, u32x4_t (&r)[BR]) {
        r[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrs, bsrc[i] + c * kQChunk * 2, 0, 0));
    };
    auto b_load = [&](int c, u32x4_t (&r)[BR]) {
#pragma unroll
        for (int i = 0; i < BR; ++i) b_load1(c, i, r);
    };
    auto b_store = [&](char *t, const u32x4_t (&r)[BR]) {
#pragma unroll
        for (int i = 0; i < BR; ++i) *reinterpret_cast<u32x4_t *>(t + bdst[i]) = r[i];
    };

    // ---- fragments and MFMAs of one step (tap t of a chunk)
    auto read_a = [&](const char *t, int tap, u32x4_t (&f)[NPB]) {
        const int u = tap / 3, v = tap - 3 * (tap / 3);
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) f[pb] = *reinterpret_cast<const u32x4_t *>(t + aoff[u][pb] + v * kQPos);
    };
    auto read_b = [&](const char *t, int tap, bf16x8_t (&f)[NCB]) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            f[cb] = *reinterpret_cast<const bf16x8_t *>(t + (tap * NCB + cb) * 1024 + lane * 16);
    };
    f32x16_t acc[NPB][NCB];
#pragma unroll
    for (int i = 0; i < NPB; ++i)
#pragma unroll
        for (int j = 0; j < NCB; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    auto mfma_step = [&](const u32x4_t (&af)[NPB], const bf16x8_t (&bf)[NCB]) {
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
            const bf16x8_t av = __builtin_bit_cast(bf16x8_t, af[pb]);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                acc[pb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bf[cb], acc[pb][cb], 0, 0, 0);
        }
    };

    // The chunk count is even (Cin_pad is a multiple of 32): chunks run in
    // pairs, so chunk c reads buffers c & 1 with that parity known at compile
    // time, and two register sets alternate. Chunk c + 2's loads go out at
    // chunk c's first step; chunk c + 1's data (loaded during chunk c - 1)
    // reach LDS at chunk c's seventh step.
    const int nchunks = a.Cin_pad / kQChunk;
    uint32_t xr0[XR][4], xr1[XR][4];
    u32x4_t br0[BR], br1[BR];
    {
        x_load(x_rsrc(0), xr0);
        b_load(0, br0);
        x_load(x_rsrc(1), xr1);  // chunk 1 (nchunks >= 2)
        b_load(1, br1);
        // zero both input tiles while the loads are in flight (padding
        // positions stay zero from here on)
        const u32x4_t z = {0u, 0u, 0u, 0u};
        for (int i = tid; i < 2 * tile_bytes / 16; i += 256) reinterpret_cast<u32x4_t *>(q_lds)[i] = z;
        lds_barrier();  // tiles zeroed
        x_store(xtile(0), xr0);
        b_store(btile(0), br0);
        lds_barrier();
    }
    u32x4_t acur[NPB];
    bf16x8_t bcur[NCB];
    read_a(xtile(0), 0, acur);
    read_b(btile(0), 0, bcur);

    auto chunk = [&](int c, auto par, uint32_t (&xs)[XR][4], u32x4_t (&bs)[BR], uint32_t (&xl)[XR][4],
                     u32x4_t (&bl)[BR]) {
        constexpr int P = decltype(par)::value;
        const char *xt = xtile(P), *bt = btile(P);
        char *xn = xtile(P ^ 1);
        char *bn = btile(P ^ 1);
        const bool more = c + 1 < nchunks, more2 = c + 2 < nchunks;
        const auto rs2 = x_rsrc(c + 2);
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            // Chunk c + 1's data (loaded during chunk c - 1) go to buffers
            // P ^ 1 in steps 0..2, before any of chunk c + 2's loads is
            // issued (steps 3..8): a store then never waits for a load issued
            // in this chunk, whatever the wait counts across the loop say.
            // Buffers P ^ 1 were last read before the previous chunk's
            // barrier.
            if (more && t < 3) {
#pragma unroll
                for (int i = t; i < XR; i += 3) x_store1(xn, i, xs);
#pragma unroll
                for (int i = t; i < BR; i += 3) *reinterpret_cast<u32x4_t *>(bn + bdst[i]) = bs[i];
            }
            if (more2 && t >= 3) {
#pragma unroll
                for (int i = t - 3; i < XR; i += 6) x_load1(rs2, i, xl);
#pragma unroll
                for (int i = t - 3; i < BR; i += 6) b_load1(c + 2, i, bl);
            }
            u32x4_t anx[NPB];
            bf16x8_t bnx[NCB];
            if (t < 8) {
                read_a(xt, t + 1, anx);
                read_b(bt, t + 1, bnx);
            }
            if (t == 8) {
                lds_barrier();  // the next chunk's tiles are complete
                if (more) {
                    read_a(xn, 0, anx);
                    read_b(bn, 0, bnx);
                }
            }
            // the next step's fragment reads go out before this step's MFMAs
            __builtin_amdgcn_sched_barrier(0);
            mfma_step(acur, bcur);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb) acur[pb] = anx[pb];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) bcur[cb] = bnx[cb];
        }
    };
    for (int c = 0; c < nchunks; c += 2) {
        chunk(c, std::integral_constant<int, 0>{}, xr1, br1, xr0, br0);      // stores chunk c + 1, loads c + 2
        chunk(c + 1, std::integral_constant<int, 1>{}, xr0, br0, xr1, br1);  // stores chunk c + 2, loads c + 3
    }

    // ---- epilogue
    lds_barrier();  // every wave is done with the tiles
    if (a_out)  // output attention: a scale per output channel
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const float so = a_out[(long)b * a.Cout + min(o0 + 32 * cb + l32, a.Cout - 1)];
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[pb][cb][q] *= so;
        }
    constexpr int pitch = MT + 8;  // bf16 per staged output row
    uint16_t *s_out = reinterpret_cast<uint16_t *>(q_lds);
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x2_t o;
                o.x = pack_bf16x2(acc[pb][cb][4 * j], acc[pb][cb][4 * j + 1]);
                o.y = pack_bf16x2(acc[pb][cb][4 * j + 2], acc[pb][cb][4 * j + 3]);
                const int pos = 32 * (wave * NPB + pb) + 8 * j + 4 * lh;
                *reinterpret_cast<u32x2_t *>(s_out + (32 * cb + l32) * pitch + pos) = o;
            }
    lds_barrier();
    const int npos = min(MT, a.P - p0);
    constexpr int kRowVec = MT / 8;
    for (int v = tid; v < NT * kRowVec; v += 256) {
        const int ch = v / kRowVec, cv = v - ch * kRowVec;
        const int o = o0 + ch;
        if (o < a.Cout && 8 * cv < npos)
            *reinterpret_cast<u32x4_t *>(y + ((long)b * a.Cout + o) * a.P + p0 + 8 * cv) =
                *reinterpret_cast<const u32x4_t *>(s_out + ch * pitch + 8 * cv);
    }
}

struct Pm3wShape {
    int npb, ncb;
};

Pm3wShape pm3w_shape(const Geom &) { return Pm3wShape{2, 2}; }

int pm3w_tile_rows(const Geom &g, int MT) {
    int rows_out = (MT - 1) / g.Wo + 2;
    if (rows_out > g.Ho) rows_out = g.Ho;
    return rows_out - 1 + 3;
}

size_t pm3w_lds(const Geom &g, int &tile_bytes) {
    const Pm3wShape sh = pm3w_shape(g);
    const int MT = 4 * sh.npb * 32, NT = sh.ncb * 32;
    tile_bytes = (pm3w_tile_rows(g, MT) * (g.W + 2 * g.pad) * kQPos + 15) / 16 * 16;
    const size_t tiles = 2 * (size_t)tile_bytes + 2 * (size_t)9 * sh.ncb * 1024;
    const size_t epi = (size_t)NT * (MT + 8) * 2;
    return tiles > epi ? tiles : epi;
}

template <int NPB, int NCB, int XR>
hipError_t launch_pm3w_t(const Geom &g, const uint16_t *x, const uint16_t *wt, uint16_t *y, hipStream_t stream,
                         const float *a_out) {
    constexpr int MT = 4 * NPB * 32, NT = NCB * 32;
    constexpr int BR = (9 * NT * 2 + 255) / 256;
    ConvArgs a = base_args(g);
    a.tile_rows = pm3w_tile_rows(g, MT);
    a.n_ptiles = ceil_div(g.P, MT);
    a.n_otiles = ceil_div(g.Cout, NT);
    int tile_bytes = 0;
    const size_t lds = pm3w_lds(g, tile_bytes);
    auto k = conv_pm3w_kernel<NPB, NCB, XR, BR>;
    if (hipError_t e = set_lds(k, lds); e != hipSuccess) return e;
    const long blocks = (long)g.B * a.n_ptiles * a.n_otiles;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), lds, stream, x, wt, y, a, tile_bytes, a_out);
    return hipGetLastError();
}

// staging rounds of 256 (position pair, channel quad) tasks per chunk
int pm3w_rounds(const Geom &g) {
    const Pm3wShape sh = pm3w_shape(g);
    const int MT = 4 * sh.npb * 32;
    const int h_rows = std::min(g.H, pm3w_tile_rows(g, MT));
    return ceil_div(4 * h_rows * (g.W / 2), 256);
}

}  // namespace

// 3x3 stride-1 pad-1 bf16 layers with even W (position pairs), P % 8 == 0
// (16-byte output rows), at most 6 staging rounds per chunk and the LDS
// within budget; byte offsets of the input planes and of one example's W_b
// below 2^31.
bool pm3w_ok(const Geom &g) {
    if (!(g.bf16 && g.groups == 1 && g.KH == 3 && g.KW == 3 && g.stride == 1 && g.pad == 1 && g.W % 2 == 0 &&
          g.P % 8 == 0))
        return false;
    if (pm3w_rounds(g) > 6) return false;
    if (16L * g.H * g.W * 2 >= (1L << 31) || 9L * g.Cout * g.Cin_pad * 2 >= (1L << 31)) return false;
    int tb = 0;
    return pm3w_lds(g, tb) <= (size_t)kQLdsMax;
}

hipError_t launch_conv_pm3w(const Geom &g, const uint16_t *x, const uint16_t *wt, uint16_t *y, hipStream_t stream,
                            const float *a_out) {
    const Pm3wShape sh = pm3w_shape(g);
    const int xr = pm3w_rounds(g);
    auto go = [&](auto npb_c, auto ncb_c) {
        constexpr int NPB = decltype(npb_c)::value, NCB = decltype(ncb_c)::value;
        switch (xr) {
        case 1: return launch_pm3w_t<NPB, NCB, 1>(g, x, wt, y, stream, a_out);
        case 2: return launch_pm3w_t<NPB, NCB, 2>(g, x, wt, y, stream, a_out);
        case 3: return launch_pm3w_t<NPB, NCB, 3>(g, x, wt, y, stream, a_out);
        case 4: return launch_pm3w_t<NPB, NCB, 4>(g, x, wt, y, stream, a_out);
        case 5: return launch_pm3w_t<NPB, NCB, 5>(g, x, wt, y, stream, a_out);
        default: return launch_pm3w_t<NPB, NCB, 6>(g, x, wt, y, stream, a_out);
        }
    };
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    if (sh.npb == 4) return go(I4{}, I2{});
    if (sh.ncb == 4) return go(I2{}, I4{});
    return go(I2{}, I2{});
}

}  // namespace dynconv
