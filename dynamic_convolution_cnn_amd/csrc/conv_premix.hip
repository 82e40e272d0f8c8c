// Per-example convolution on bf16 MFMA (gfx950) from mixed kernels already
// in memory: wt[b][t][o][cp] (the premix layout, channels padded to kChunk).
//
// conv_premix_kernel: any bf16 groups == 1 shape, v_mfma_f32_16x16x32_bf16.
//   A workgroup owns one example, a tile of MT = NW*FM*16 output positions
//   and NT = FN*16 output channels. Each chunk of 32 input channels of the
//   example's input rows is staged once into an LDS tile laid out
//   [input row][input col][channel] (80-byte position stride: 32 channels +
//   16 bytes of padding, so eight consecutive positions fall in eight
//   distinct 16-byte bank groups), zero halo written once; every tap reads its
//   A fragments from that tile with one 128-bit LDS read per lane, so the
//   im2col expansion never exists in memory. B fragments (8 channels of one
//   output channel, 16 bytes per lane) load straight from wt.
// conv_pm3_kernel / conv_pm1_kernel: the 3x3 and 1x1 stride-1 layers on
//   v_mfma_f32_32x32x16_bf16 (see below).
#include "conv_common.hpp"

namespace dynconv {
namespace {

// Stage input channels [c0, c0 + 32) of one example (rows [h_lo, h_hi) of
// the image) into the LDS tile whose row 0 is input row h_tile0. Channels
// >= Cin are written as zeros. Task order (position pair fastest, then row,
// then 8-channel group) makes consecutive lanes read consecutive words of
// one channel plane.
template <bool PAIRED>
__device__ __forceinline__ void stage_chunk(const uint16_t *__restrict__ xb,
                                            uint16_t *__restrict__ tile, const ConvArgs &a,
                                            int c0, int h_lo, int h_hi, int h_tile0, int tid,
                                            int nthreads) {
    const int HW = a.H * a.W;
    const int nrows = h_hi - h_lo;
    if (nrows <= 0) return;
    if constexpr (PAIRED) {
        const int pairs = a.W >> 1;
        const int per_g = nrows * pairs;
        const int ntasks = 4 * per_g;
        for (int task = tid; task < ntasks; task += nthreads) {
            const int g = task / per_g;
            const int rem = task - g * per_g;
            const int row = rem / pairs;
            const int pr = rem - row * pairs;
            const int h = h_lo + row;
            const int cb = c0 + 8 * g;
            const uint32_t *src =
                reinterpret_cast<const uint32_t *>(xb + (long)cb * HW + h * a.W + 2 * pr);
            uint32_t w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                w[k] = (cb + k < a.Cin) ? src[(long)k * (HW >> 1)] : 0u;
            u32x4_t o0, o1;
            o0.x = lo_pair(w[0], w[1]); o0.y = lo_pair(w[2], w[3]);
            o0.z = lo_pair(w[4], w[5]); o0.w = lo_pair(w[6], w[7]);
            o1.x = hi_pair(w[0], w[1]); o1.y = hi_pair(w[2], w[3]);
            o1.z = hi_pair(w[4], w[5]); o1.w = hi_pair(w[6], w[7]);
            uint16_t *dst = tile + ((h - h_tile0) * a.ncols + 2 * pr + a.pad) * kPosStride + 8 * g;
            *reinterpret_cast<u32x4_t *>(dst) = o0;
            *reinterpret_cast<u32x4_t *>(dst + kPosStride) = o1;
        }
    } else {
        const int per_g = nrows * a.W;
        const int ntasks = 4 * per_g;
        for (int task = tid; task < ntasks; task += nthreads) {
            const int g = task / per_g;
            const int rem = task - g * per_g;
            const int row = rem / a.W;
            const int col = rem - row * a.W;
            const int h = h_lo + row;
            const int cb = c0 + 8 * g;
            const uint16_t *src = xb + (long)cb * HW + h * a.W + col;
            uint32_t e[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) e[k] = (cb + k < a.Cin) ? (uint32_t)src[(long)k * HW] : 0u;
            u32x4_t o;
            o.x = e[0] | (e[1] << 16); o.y = e[2] | (e[3] << 16);
            o.z = e[4] | (e[5] << 16); o.w = e[6] | (e[7] << 16);
            uint16_t *dst = tile + ((h - h_tile0) * a.ncols + col + a.pad) * kPosStride + 8 * g;
            *reinterpret_cast<u32x4_t *>(dst) = o;
        }
    }
}

template <int FM, int FN, int NW, bool PAIRED>
__global__ __launch_bounds__(NW * 64) void conv_premix_kernel(const uint16_t *__restrict__ x,
                                                              const uint16_t *__restrict__ wt,
                                                              uint16_t *__restrict__ y,
                                                              ConvArgs a, const float *__restrict__ a_out) {
    extern __shared__ __attribute__((aligned(16))) uint16_t tile[];
    constexpr int MT = NW * FM * 16;
    constexpr int NT = FN * 16;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int per_b = a.n_ptiles * a.n_otiles;
    const int b = logical / per_b;
    const int rem = logical - b * per_b;
    const int pt = rem / a.n_otiles;
    const int ot = rem - pt * a.n_otiles;
    const int p0 = pt * MT, o0 = ot * NT;
    const int r_first = p0 / a.Wo;
    const int h_tile0 = r_first * a.stride - a.pad;
    const int h_lo = max(0, h_tile0), h_hi = min(a.H, h_tile0 + a.tile_rows);

    zero_lds(tile, a.tile_rows * a.ncols * kPosStride, tid, NW * 64);

    int aoff[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int p = min(p0 + (wave * FM + fm) * 16 + lr, a.P - 1);
        const int r = p / a.Wo;
        const int s = p - r * a.Wo;
        aoff[fm] = (((r - r_first) * a.stride) * a.ncols + s * a.stride) * kPosStride + 8 * lg;
    }
    const uint16_t *xb = x + (long)b * a.x_bstride;
    const uint16_t *wb = wt + (long)b * a.KT * a.Cout * a.Cin_pad;
    long wrow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) wrow[fn] = (long)min(o0 + fn * 16 + lr, a.Cout - 1) * a.Cin_pad + 8 * lg;

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < a.Cin_pad; c0 += kChunk) {
        __syncthreads();
        stage_chunk<PAIRED>(xb, tile, a, c0, h_lo, h_hi, h_tile0, tid, NW * 64);
        __syncthreads();
        for (int t = 0; t < a.KT; ++t) {
            const int u = t / a.KW, v = t - u * a.KW;
            const int toff = (u * a.ncols + v) * kPosStride;
            const uint16_t *wtap = wb + (long)t * a.Cout * a.Cin_pad + c0;
            bf16x8_t bfr[FN];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bfr[fn] = *reinterpret_cast<const bf16x8_t *>(wtap + wrow[fn]);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const bf16x8_t afr = *reinterpret_cast<const bf16x8_t *>(tile + aoff[fm] + toff);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[fn], acc[fm][fn], 0, 0, 0);
            }
        }
    }
    if (a_out)  // output attention: a scale of output channel o0 + 16 fn + lr
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const float so = a_out[(long)b * a.Cout + min(o0 + fn * 16 + lr, a.Cout - 1)];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[fm][fn][q] *= so;
        }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            store_frag(y, a, b, o0 + fn * 16 + lr, p0 + (wave * FM + fm) * 16 + 4 * lg, acc[fm][fn]);
}

// ---- premix 3x3 convolution on 32x32x16 MFMA -------------------------------
// Stride-1 3x3 layers with W_b in memory (wt[b][t][o][cp]) and images too
// wide for the row-16 kernel. A workgroup of 4 waves owns example b, 64
// output channels and kPmMT consecutive output positions (row-major).
//   - Input tile: the padded input rows the tile's outputs read, 64-byte
//     positions whose 16-byte channel granules are XOR-swizzled by position
//     (swz), two buffers: the current chunk of 32 input channels and the next.
//   - A fragment (32 positions x 16 channels): each lane reads the granule of
//     its own output position shifted by the tap, tile position q + u * ncols
//     + v; the next step's fragments are read during the current step.
//   - B fragments (16 channels x 32 output channels): wave w loads fragment
//     w of each step (output-channel block w >> 1, K half w & 1) three steps
//     ahead into a register ring, writes it to a double-buffered LDS stage one
//     step ahead, and one barrier per step publishes it; every wave then
//     reads the step's four fragments from the stage.
//   - Staging of the next chunk as in the row-16 kernel: dword buffer loads
//     of position pairs (channels past Cin read as zeros), a register
//     transpose, 8-byte tile writes two steps later; slots in steps 0..6.
//   - Epilogue through LDS: the accumulators go into the idle tiles as 64
//     channel rows of kPmMT positions, then out along y's rows with 16-byte
//     stores.
constexpr int kPmPB = 2;                 // position blocks of 32 per wave
constexpr int kPmMT = 4 * kPmPB * 32;    // positions per workgroup
constexpr int kPmMaxPos = 512;           // tile positions per buffer
constexpr int kPmSlots = 7;              // staging slots per chunk (steps 0..6)
constexpr int kPmOutPitch = kPmMT + 8;   // bf16 per staged output row
__shared__ __attribute__((aligned(16))) u32x4_t s_pm[2 * kPmMaxPos * 4];  // 2 x 32 KB
__shared__ __attribute__((aligned(16))) u32x4_t s_pmb[2 * 4 * 64];        // 2 x 4 B fragments
static_assert(64 * kPmOutPitch * 2 <= 2 * kPmMaxPos * 64, "epilogue rows fit in the tiles");

__global__ __launch_bounds__(256) void conv_pm3_kernel(const uint16_t *__restrict__ x,
                                                       const uint16_t *__restrict__ wt,
                                                       uint16_t *__restrict__ y, ConvArgs a,
                                                       const float *__restrict__ a_out) {
    constexpr int KT = 9, CB = 2, RL = 2;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int per_b = a.n_ptiles * a.n_otiles;
    const int b = logical / per_b;
    const int rem = logical - b * per_b;
    const int pt = rem / a.n_otiles, ot = rem - pt * a.n_otiles;
    const int p0 = pt * kPmMT, o0 = ot * 64;
    const int r_first = p0 / a.Wo;
    const int h_tile0 = r_first - a.pad;  // input row of tile row 0
    const int h_lo = max(0, h_tile0), h_hi = min(a.H, h_tile0 + a.tile_rows);
    auto tile_of = [&](int par) { return reinterpret_cast<uint16_t *>(s_pm + par * kPmMaxPos * 4); };
    zero_lds(tile_of(0), 2 * kPmMaxPos * 32, tid, 256);

    int aq[kPmPB];  // tile position of the lane's output in each block (tap 0)
#pragma unroll
    for (int pb = 0; pb < kPmPB; ++pb) {
        const int p = min(p0 + 32 * (wave * kPmPB + pb) + l32, a.P - 1);
        const int r = p / a.Wo, s = p - r * a.Wo;
        aq[pb] = (r - r_first) * a.ncols + s;
    }
    const uint16_t *wb = wt + (long)b * KT * a.Cout * a.Cin_pad;
    long wrow[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) wrow[cb] = (long)min(o0 + 32 * cb + l32, a.Cout - 1) * a.Cin_pad + 8 * lh;
    // this wave's fragment of step 9 c + t (clamped to the last step)
    const int nsteps = (a.Cin_pad / kChunk) * KT;
    const long wfrag = wrow[wave >> 1] + 16 * (wave & 1);
    auto load_b = [&](int st) {
        st = min(st, nsteps - 1);
        const int c = st / KT, t = st - c * KT;
        return *reinterpret_cast<const u32x4_t *>(wb + (long)t * a.Cout * a.Cin_pad + c * kChunk + wfrag);
    };
    auto bslot = [&](int buf, int f) { return s_pmb + (buf * 4 + f) * 64 + lane; };
    auto read_b = [&](int buf, bf16x8_t (&bw)[CB][2]) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) bw[cb][kh] = __builtin_bit_cast(bf16x8_t, *bslot(buf, 2 * cb + kh));
    };
    auto read_a = [&](const uint16_t *tile, int t, u32x4_t (&af)[kPmPB][2]) {
        const int u = t / 3, v = t - 3 * (t / 3);
#pragma unroll
        for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
                af[pb][kh] = *reinterpret_cast<const u32x4_t *>(tile + swz(aq[pb] + u * a.ncols + v, 2 * kh + lh));
    };

    // staging: half-task t = 256 slot + tid is channel quad t & 7 of position
    // pair t >> 3 of the staged rows [h_lo, h_hi); pairs past the last
    // repeat it (same bytes to the same place)
    const uint16_t *xb = x + (long)b * a.x_bstride;
    const int HW = a.H * a.W, plane = HW * 2, pairs = a.W >> 1;
    const int npairs = max(1, (h_hi - h_lo) * pairs);
    const float inv_pairs = 1.f / (float)pairs;
    auto rsrc_of = [&](int cc) {
        const int c0 = min(cc, a.Cin - 1);
        const int nb = max(0, min(kChunk, a.Cin - cc)) * plane - h_lo * a.W * 2;
        const int nbytes = __builtin_amdgcn_readfirstlane(max(0, nb));
        const uint64_t p = reinterpret_cast<uint64_t>(xb + (long)c0 * HW + (long)h_lo * a.W);
        const uint64_t ps = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)) << 32);
        return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ps), 0, nbytes, 0x00020000);
    };
    auto pair_of = [&](int s, int ln) { return min((256 * s + ln) >> 3, npairs - 1); };
    auto stage_load = [&](__amdgpu_buffer_rsrc_t rs, int s, int ln, uint32_t (&r)[4]) {
        const int vo = 4 * (ln & 7) * plane + 4 * pair_of(s, ln);
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo + j * plane, 0, 0);
    };
    auto stage_store = [&](uint16_t *t, int s, int ln, const uint32_t (&r)[4]) {
        const int pg = pair_of(s, ln), quad = ln & 7;
        const int row = (int)(((float)pg + 0.5f) * inv_pairs);
        const int q = (h_lo - h_tile0 + row) * a.ncols + 2 * (pg - row * pairs) + a.pad;
        const int g = quad >> 1, ho = 4 * (quad & 1);
        const int sel = (quad ^ pg) & 1;
        const uint32_t bs0 = 0x05040100u + (uint32_t)sel * 0x02020202u;
        const uint32_t bs1 = 0x07060302u - (uint32_t)sel * 0x02020202u;
        u32x2_t q0, q1;
        q0.x = __builtin_amdgcn_perm(r[1], r[0], bs0); q0.y = __builtin_amdgcn_perm(r[3], r[2], bs0);
        q1.x = __builtin_amdgcn_perm(r[1], r[0], bs1); q1.y = __builtin_amdgcn_perm(r[3], r[2], bs1);
        *reinterpret_cast<u32x2_t *>(t + swz(q + sel, g) + ho) = q0;
        *reinterpret_cast<u32x2_t *>(t + swz(q + 1 - sel, g) + ho) = q1;
    };

    f32x16_t acc[kPmPB][CB];
#pragma unroll
    for (int i = 0; i < kPmPB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    const int nchunks = a.Cin_pad / kChunk;

    // chunk 0
    {
        const auto rs = rsrc_of(0);
        uint32_t r0[kPmSlots][4];
#pragma unroll
        for (int s = 0; s < kPmSlots; ++s) stage_load(rs, s, tid, r0[s]);
        lds_barrier();  // tiles zeroed
#pragma unroll
        for (int s = 0; s < kPmSlots; ++s) stage_store(tile_of(0), s, tid, r0[s]);
    }
    // B ring: slot k holds this wave's fragment of a step s with s % 3 == k
    u32x4_t wring[3];
    wring[0] = load_b(0);
    wring[1] = load_b(1);
    wring[2] = load_b(2);
    *bslot(0, wave) = wring[0];
    wring[0] = load_b(3);
    lds_barrier();  // chunk 0 in tile 0, B_0 staged
    bf16x8_t bw[CB][2];
    read_b(0, bw);
    u32x4_t af[kPmPB][2];
    read_a(tile_of(0), 0, af);

    for (int c = 0; c < nchunks; ++c) {
        const uint16_t *tile = tile_of(c & 1);
        uint16_t *tnext = tile_of((c + 1) & 1);  // chunk c - 1's, whose last reads preceded the last barrier
        const auto rs = rsrc_of(min(c + 1, nchunks - 1) * kChunk);
        int ln = tid;
        asm volatile("" : "+v"(ln));
        uint32_t rb[RL][4];
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            // step s = 9 c + t; the ring slot of step s + 1 is (t + 1) % 3
            const int nbuf = (c + t + 1) & 1;  // stage buffer of B_{s+1}
            u32x4_t an[kPmPB][2];
            if (t + 1 < KT) read_a(tile, t + 1, an);
#pragma unroll
            for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const bf16x8_t afr = __builtin_bit_cast(bf16x8_t, af[pb][kh]);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[pb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bw[cb][kh], acc[pb][cb], 0, 0, 0);
                }
            // B_{s+1} to the stage (buffer nbuf held B_{s-1}, read before the
            // previous barrier), then B_{s+4} into the freed ring slot
            *bslot(nbuf, wave) = wring[(t + 1) % 3];
            wring[(t + 1) % 3] = load_b(9 * c + t + 4);
            if (t >= RL && t - RL < kPmSlots) stage_store(tnext, t - RL, ln, rb[t % RL]);
            if (t < kPmSlots) stage_load(rs, t, ln, rb[t % RL]);
            lds_barrier();  // B_{s+1} published; at the chunk's end also the next tile
            if (t + 1 == KT) read_a(tnext, 0, an);
            read_b(nbuf, bw);
#pragma unroll
            for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) af[pb][kh] = an[pb][kh];
        }
    }
    // epilogue: D(lane, 4 j + q) = channel o0 + 32 cb + l32, position
    // 32 (wave kPmPB + pb) + 8 j + 4 lh + q of the tile
    lds_barrier();  // last A reads of every wave done
    if (a_out)  // output attention: a scale of output channel o0 + 32 cb + l32
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const float so = a_out[(long)b * a.Cout + min(o0 + 32 * cb + l32, a.Cout - 1)];
#pragma unroll
            for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[pb][cb][q] *= so;
        }
    uint16_t *s_out = tile_of(0);
#pragma unroll
    for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x2_t o;
                o.x = pack_bf16x2(acc[pb][cb][4 * j], acc[pb][cb][4 * j + 1]);
                o.y = pack_bf16x2(acc[pb][cb][4 * j + 2], acc[pb][cb][4 * j + 3]);
                const int pos = 32 * (wave * kPmPB + pb) + 8 * j + 4 * lh;
                *reinterpret_cast<u32x2_t *>(s_out + (32 * cb + l32) * kPmOutPitch + pos) = o;
            }
    lds_barrier();
    const int npos = min(kPmMT, a.P - p0);
    constexpr int kRowVec = kPmMT / 8;
    for (int v = tid; v < 64 * kRowVec; v += 256) {
        const int ch = v / kRowVec, cv = v - ch * kRowVec;
        const int o = o0 + ch;
        if (o < a.Cout && 8 * cv < npos)
            *reinterpret_cast<u32x4_t *>(y + ((long)b * a.Cout + o) * a.P + p0 + 8 * cv) =
                *reinterpret_cast<const u32x4_t *>(s_out + ch * kPmOutPitch + 8 * cv);
    }
}

// ---- premix 1x1 convolution on 32x32x16 MFMA -------------------------------
// Stride-1 1x1 layers without padding (the MBConv expand and project
// layers, HBM-bound): a workgroup of 4 waves owns example b, 64 output
// channels and kPmMT consecutive positions. Per chunk of 32 input channels,
// the x slice is read with 16-byte loads along the positions (32 lanes
// cover 512 contiguous bytes of one channel plane) into a [channel][position]
// LDS tile, and the transpose to MFMA A fragments (8 channels of one
// position per lane) happens in the 2-byte LDS reads. The W_b slice is one
// 16-byte fragment piece per thread. Both load at the start of the previous
// chunk and go to the other LDS buffer at its end; one barrier per chunk.
// Outputs leave through LDS as 16-byte row stores.
// CB blocks of 32 output channels per tile: 2 (64 channels) or 3 (96, for
// layers such as the MBConv project layer's 80 channels, which then fit one
// tile instead of two).
constexpr int kCUs = 256;             // compute units of the MI355X
constexpr int kPm1Tile = kPmMT * 32;  // bf16 per x tile buffer (32 channels x 256 positions)
constexpr int pm1_lds_bytes(int CB) {  // 2 x 16 KB tiles, or the epilogue rows
    return 32 * CB * kPmOutPitch * 2 > 2 * kPm1Tile * 2 ? 32 * CB * kPmOutPitch * 2 : 2 * kPm1Tile * 2;
}
// workgroups per CU (LDS: 3 x 41 KB with 2 blocks, 2 x 63 KB with 3)
constexpr int pm1_resident(int CB) { return CB == 2 ? 3 : 2; }

// byte offset of position q of channel row c in a [32][256] tile: the
// 16-byte pieces of rows 8..15 and 24..31 are XOR-swapped by 4 pieces, so
// that the two half-waves of a fragment read (rows 8 apart) use different
// banks
__device__ __forceinline__ int pm1_off(int c, int q) {
    return c * (kPmMT * 2) + ((((q >> 3) ^ (((c >> 3) & 1) << 2))) << 4) + ((q & 7) << 1);
}

template <int CB>
__global__ __launch_bounds__(256) void conv_pm1_kernel(const uint16_t *__restrict__ x,
                                                       const uint16_t *__restrict__ wt,
                                                       uint16_t *__restrict__ y, ConvArgs a,
                                                       const float *__restrict__ a_out) {
    constexpr int NF = 2 * CB;             // W_b fragments per chunk (block, K half)
    constexpr int NFW = (NF + 3) / 4;      // fragments staged per thread
    __shared__ __attribute__((aligned(16))) u32x4_t s_pm1x[pm1_lds_bytes(CB) / 16];
    __shared__ __attribute__((aligned(16))) u32x4_t s_pm1w[2 * NF * 64];
    constexpr int kLoads = 32 * kPmMT * 2 / 16 / 256;  // 16-byte x loads per thread per chunk (4)
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    auto xtile = [&](int par) { return reinterpret_cast<char *>(s_pm1x + par * (kPm1Tile / 8)); };
    auto wslot = [&](int par, int f) { return s_pm1w + (par * NF + f) * 64; };
    const int nchunks = a.Cin_pad / kChunk;
    const int plane = a.P * 2;  // bytes per channel plane (H W = P)
    // Persistent workgroups: tiles (example b, position tile pt, channel tile
    // ot) in that order are cut into 8 contiguous ranges, one per XCD
    // (workgroup i runs on XCD i % 8; the grid is a multiple of 8), so the
    // channel tiles of one position tile share an L2. Workgroup i walks its
    // XCD's range with stride gridDim.x / 8.
    const int per_b = a.n_ptiles * a.n_otiles;
    const int ntiles = a.B * per_b;
    const int xcd = blockIdx.x & 7, g8 = gridDim.x >> 3;
    const int hi = (int)((long)ntiles * (xcd + 1) / 8);
    const int first = (int)((long)ntiles * xcd / 8) + (blockIdx.x >> 3);
    if (first >= hi) return;
    struct Tile {
        int b, p0, o0, npos;
    };
    auto tile_at = [&](int t) {
        Tile ti;
        ti.b = t / per_b;
        const int rem = t - ti.b * per_b;
        const int pt = rem / a.n_otiles;
        ti.p0 = pt * kPmMT;
        ti.o0 = (rem - pt * a.n_otiles) * 32 * CB;
        ti.npos = min(kPmMT, a.P - ti.p0);
        return ti;
    };
    struct Stage {
        u32x4_t r[kLoads];
        u32x4_t w[NFW];
    };
    // Chunk c of tile ti. x: load u = 256 k + tid is piece u & 31 (8
    // positions) of channel row u >> 5; rows past Cin read as zeros, and
    // pieces at positions past the plane's end take an offset beyond the
    // buffer's extent (zeros, with no memory traffic). W: thread tid holds
    // lane tid & 63 of fragments f = (tid >> 6) + 4 k (block f >> 1, K half
    // f & 1) for f < NF.
    // (The descriptor's fields go through readfirstlane: scalar registers.)
    auto load = [&](const Tile &ti, int c, Stage &st) {
        const int cc = c * kChunk;
        const int c0 = min(cc, a.Cin - 1);
        const int nbytes = __builtin_amdgcn_readfirstlane(max(0, min(kChunk, a.Cin - cc)) * plane - ti.p0 * 2);
        const uint64_t p = reinterpret_cast<uint64_t>(x + (long)ti.b * a.x_bstride + (long)c0 * a.P + ti.p0);
        const uint64_t ps = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)) << 32);
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ps), 0, max(0, nbytes), 0x00020000);
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const int u = 256 * k + tid;
            const int off = 8 * (u & 31) < ti.npos ? (u >> 5) * plane + ((u & 31) << 4) : 0x7ffffff0;
            st.r[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < NFW; ++k) {
            const int f = min(wave + 4 * k, NF - 1);
            const long wrow = (long)min(ti.o0 + 32 * (f >> 1) + l32, a.Cout - 1) * a.Cin_pad + 16 * (f & 1) + 8 * lh;
            st.w[k] = *reinterpret_cast<const u32x4_t *>(wt + (long)ti.b * a.Cout * a.Cin_pad + wrow + cc);
        }
    };
    auto store = [&](int par, const Stage &st) {
        char *t = xtile(par);
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const int u = 256 * k + tid;
            *reinterpret_cast<u32x4_t *>(t + pm1_off(u >> 5, (u & 31) << 3)) = st.r[k];
        }
#pragma unroll
        for (int k = 0; k < NFW; ++k)
            if (wave + 4 * k < NF) wslot(par, wave + 4 * k)[lane] = st.w[k];
    };
    // A fragment: position q, channels 8 g .. 8 g + 7 of the chunk
    auto afrag = [&](const char *t, int q, int g) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = *reinterpret_cast<const uint16_t *>(t + pm1_off(8 * g + i, q));
        u32x4_t v;
        v.x = h[0] | (h[1] << 16); v.y = h[2] | (h[3] << 16);
        v.z = h[4] | (h[5] << 16); v.w = h[6] | (h[7] << 16);
        return __builtin_bit_cast(bf16x8_t, v);
    };
    f32x16_t acc[kPmPB][CB];
    auto compute = [&](int par) {
        const char *t = xtile(par);
        bf16x8_t bw[CB][2];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) bw[cb][kh] = __builtin_bit_cast(bf16x8_t, wslot(par, 2 * cb + kh)[lane]);
#pragma unroll
        for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const bf16x8_t afr = afrag(t, 32 * (wave * kPmPB + pb) + l32, 2 * kh + lh);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    acc[pb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bw[cb][kh], acc[pb][cb], 0, 0, 0);
            }
    };
    uint16_t *s_out = reinterpret_cast<uint16_t *>(s_pm1x);  // epilogue rows (over the x tiles)
    int t = first;
    Tile ti = tile_at(t);
    Stage st;
    load(ti, 0, st);
    while (true) {
        // chunk 0 of this tile: loaded during the previous tile's last chunk
        // and epilogue (whose LDS reads ended before the last barrier)
        store(0, st);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < kPmPB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
        const int tn = t + g8;
        const bool more = tn < hi;
        const Tile tin = tile_at(more ? tn : t);
        for (int c = 0; c < nchunks; ++c) {
            const int par = c & 1;
            if (c + 1 < nchunks) load(ti, c + 1, st);
            else if (more) load(tin, 0, st);
            compute(par);
            // the other buffer was last read in chunk c - 1, before the previous barrier
            if (c + 1 < nchunks) store(par ^ 1, st);
            lds_barrier();
        }
        // epilogue (as the 3x3 kernel): D(lane, 4 j + q) = channel o0 + 32 cb + l32,
        // position 32 (wave kPmPB + pb) + 8 j + 4 lh + q
        if (a_out)  // output attention
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const float so = a_out[(long)ti.b * a.Cout + min(ti.o0 + 32 * cb + l32, a.Cout - 1)];
#pragma unroll
                for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
                    for (int q = 0; q < 16; ++q) acc[pb][cb][q] *= so;
            }
#pragma unroll
        for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    u32x2_t o;
                    o.x = pack_bf16x2(acc[pb][cb][4 * j], acc[pb][cb][4 * j + 1]);
                    o.y = pack_bf16x2(acc[pb][cb][4 * j + 2], acc[pb][cb][4 * j + 3]);
                    const int pos = 32 * (wave * kPmPB + pb) + 8 * j + 4 * lh;
                    *reinterpret_cast<u32x2_t *>(s_out + (32 * cb + l32) * kPmOutPitch + pos) = o;
                }
        lds_barrier();
        constexpr int kRowVec = kPmMT / 8;
        for (int v = tid; v < 32 * CB * kRowVec; v += 256) {
            const int ch = v / kRowVec, cv = v - ch * kRowVec;
            const int o = ti.o0 + ch;
            if (o < a.Cout && 8 * cv < ti.npos)
                *reinterpret_cast<u32x4_t *>(y + ((long)ti.b * a.Cout + o) * a.P + ti.p0 + 8 * cv) =
                    *reinterpret_cast<const u32x4_t *>(s_out + ch * kPmOutPitch + 8 * cv);
        }
        if (!more) break;
        lds_barrier();  // the epilogue's LDS reads end before the next chunk 0 lands there
        t = tn;
        ti = tin;
    }
}

// ---- 1x1 convolution with few input channels (Cin <= 64) ----------------
// The MBConv expand layers write many more bytes than they read. A
// workgroup owns one example's kPmMT positions and all output channels: its
// x slice (NCH <= 2 chunks) loads once into a [channel][position] LDS tile
// (the layout and reads of conv_pm1_kernel), then it walks the 64-channel
// output tiles, loading the next tile's W_b slice while it multiplies, and
// sends each tile out through a 32-channel LDS stage in two passes, so that
// one tile's output stores overlap the next tile's work.
constexpr int kPm1xOutPitch = kPmMT + 8;  // bf16 per staged output row
template <int NCH>
__global__ __launch_bounds__(256) void conv_pm1x_kernel(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ wt,
                                                        uint16_t *__restrict__ y, ConvArgs a,
                                                        const float *__restrict__ a_out) {
    constexpr int CB = 2;
    constexpr int kLoads = 32 * kPmMT * 2 / 16 / 256;  // 16-byte x loads per thread per chunk (4)
    __shared__ __attribute__((aligned(16))) u32x4_t s_x[NCH * kPm1Tile / 8];     // NCH x 16 KB
    __shared__ __attribute__((aligned(16))) u32x4_t s_w[2 * NCH * 4 * 64];       // 2 x NCH x 4 fragments
    __shared__ __attribute__((aligned(16))) uint16_t s_o[32 * kPm1xOutPitch];    // one 32-channel block
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int b = logical / a.n_ptiles, pt = logical - b * a.n_ptiles;
    const int p0 = pt * kPmMT, npos = min(kPmMT, a.P - p0);
    const int plane = a.P * 2;  // bytes per channel plane
    auto xtile = [&](int c) { return reinterpret_cast<char *>(s_x + c * (kPm1Tile / 8)); };
    auto wslot = [&](int buf, int c, int f) { return s_w + ((buf * NCH + c) * 4 + f) * 64; };
    const uint16_t *wb = wt + (long)b * a.Cout * a.Cin_pad;
    // W_b piece of output tile ot, chunk c: lane tid & 63 of fragment f = tid >> 6
    auto wload = [&](int ot, int c) {
        const long row = (long)min(64 * ot + 32 * (wave >> 1) + l32, a.Cout - 1) * a.Cin_pad;
        return *reinterpret_cast<const u32x4_t *>(wb + row + c * kChunk + 16 * (wave & 1) + 8 * lh);
    };
    // x: as conv_pm1_kernel (rows past Cin and positions past the plane read as zeros)
    {
        u32x4_t r[NCH][kLoads];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int cc = c * kChunk;
            const int c0 = min(cc, a.Cin - 1);
            const int nbytes = __builtin_amdgcn_readfirstlane(max(0, min(kChunk, a.Cin - cc)) * plane - p0 * 2);
            const uint64_t p = reinterpret_cast<uint64_t>(x + (long)b * a.x_bstride + (long)c0 * a.P + p0);
            const uint64_t ps = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p) |
                                ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)) << 32);
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ps), 0, max(0, nbytes), 0x00020000);
#pragma unroll
            for (int k = 0; k < kLoads; ++k) {
                const int u = 256 * k + tid;
                const int off = 8 * (u & 31) < npos ? (u >> 5) * plane + ((u & 31) << 4) : 0x7ffffff0;
                r[c][k] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
            }
        }
        u32x4_t w0[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) w0[c] = wload(0, c);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
#pragma unroll
            for (int k = 0; k < kLoads; ++k) {
                const int u = 256 * k + tid;
                *reinterpret_cast<u32x4_t *>(xtile(c) + pm1_off(u >> 5, (u & 31) << 3)) = r[c][k];
            }
            wslot(0, c, wave)[lane] = w0[c];
        }
    }
    lds_barrier();
    auto afrag = [&](const char *t, int q, int g) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = *reinterpret_cast<const uint16_t *>(t + pm1_off(8 * g + i, q));
        u32x4_t v;
        v.x = h[0] | (h[1] << 16); v.y = h[2] | (h[3] << 16);
        v.z = h[4] | (h[5] << 16); v.w = h[6] | (h[7] << 16);
        return __builtin_bit_cast(bf16x8_t, v);
    };
    for (int ot = 0; ot < a.n_otiles; ++ot) {
        const int buf = ot & 1;
        const bool more = ot + 1 < a.n_otiles;
        u32x4_t wn[NCH];
        if (more)
#pragma unroll
            for (int c = 0; c < NCH; ++c) wn[c] = wload(ot + 1, c);
        f32x16_t acc[kPmPB][CB];
#pragma unroll
        for (int i = 0; i < kPmPB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const char *t = xtile(c);
            bf16x8_t bw[CB][2];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
                    bw[cb][kh] = __builtin_bit_cast(bf16x8_t, wslot(buf, c, 2 * cb + kh)[lane]);
#pragma unroll
            for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const bf16x8_t afr = afrag(t, 32 * (wave * kPmPB + pb) + l32, 2 * kh + lh);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[pb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bw[cb][kh], acc[pb][cb], 0, 0, 0);
                }
        }
        // the next tile's W_b goes to the other buffer, last read during tile ot - 1
        if (more)
#pragma unroll
            for (int c = 0; c < NCH; ++c) wslot(buf ^ 1, c, wave)[lane] = wn[c];
        // epilogue, one 32-channel block per pass: D(lane, 4 j + q) = channel
        // 64 ot + 32 cb + l32, position 32 (wave kPmPB + pb) + 8 j + 4 lh + q
        if (a_out)  // output attention
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const float so = a_out[(long)b * a.Cout + min(64 * ot + 32 * cb + l32, a.Cout - 1)];
#pragma unroll
                for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
                    for (int q = 0; q < 16; ++q) acc[pb][cb][q] *= so;
            }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int pb = 0; pb < kPmPB; ++pb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    u32x2_t o;
                    o.x = pack_bf16x2(acc[pb][cb][4 * j], acc[pb][cb][4 * j + 1]);
                    o.y = pack_bf16x2(acc[pb][cb][4 * j + 2], acc[pb][cb][4 * j + 3]);
                    const int pos = 32 * (wave * kPmPB + pb) + 8 * j + 4 * lh;
                    *reinterpret_cast<u32x2_t *>(s_o + l32 * kPm1xOutPitch + pos) = o;
                }
            lds_barrier();
            constexpr int kRowVec = kPmMT / 8;
            for (int v = tid; v < 32 * kRowVec; v += 256) {
                const int ch = v / kRowVec, cv = v - ch * kRowVec;
                const int o = 64 * ot + 32 * cb + ch;
                if (o < a.Cout && 8 * cv < npos)
                    *reinterpret_cast<u32x4_t *>(y + ((long)b * a.Cout + o) * a.P + p0 + 8 * cv) =
                        *reinterpret_cast<const u32x4_t *>(s_o + ch * kPm1xOutPitch + 8 * cv);
            }
            lds_barrier();  // the stage is read before the next pass writes it
        }
    }
}

// Premix tile shapes: (FM, FN, NW) -> MT = NW*FM*16 positions, NT = FN*16 channels.
struct PremixCfg { int FM, FN, NW; };
constexpr PremixCfg kPremixLarge{7, 4, 7};  // MT 784, NT 64
constexpr PremixCfg kPremixSmall{2, 4, 7};  // MT 224, NT 64

int tile_rows_for(const Geom &g, int MT) {
    int rows_out = (MT - 1) / g.Wo + 2;
    if (rows_out > g.Ho) rows_out = g.Ho;
    return (rows_out - 1) * g.stride + g.KH;
}

size_t premix_lds_bytes(const Geom &g, const PremixCfg &c) {
    const int MT = c.NW * c.FM * 16;
    return (size_t)tile_rows_for(g, MT) * (g.W + 2 * g.pad) * kPosStride * sizeof(uint16_t);
}

PremixCfg pick_premix(const Geom &g) {
    return g.P >= 512 ? kPremixLarge : kPremixSmall;
}

bool paired_ok(const Geom &g) { return (g.W % 2) == 0; }

template <int FM, int FN, int NW>
hipError_t launch_premix_cfg(const Geom &g, const uint16_t *x, const uint16_t *wt, uint16_t *y,
                             hipStream_t stream, const float *a_out) {
    ConvArgs a = base_args(g);
    constexpr int MT = NW * FM * 16, NT = FN * 16;
    a.tile_rows = tile_rows_for(g, MT);
    a.n_ptiles = ceil_div(g.P, MT);
    a.n_otiles = ceil_div(g.Cout, NT);
    const size_t lds = (size_t)a.tile_rows * a.ncols * kPosStride * sizeof(uint16_t);
    const long blocks = (long)g.B * a.n_ptiles * a.n_otiles;
    if (paired_ok(g)) {
        auto k = conv_premix_kernel<FM, FN, NW, true>;
        if (hipError_t e = set_lds(k, lds); e != hipSuccess) return e;
        hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(NW * 64), lds, stream, x, wt, y, a, a_out);
    } else {
        auto k = conv_premix_kernel<FM, FN, NW, false>;
        if (hipError_t e = set_lds(k, lds); e != hipSuccess) return e;
        hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(NW * 64), lds, stream, x, wt, y, a, a_out);
    }
    return hipGetLastError();
}

}  // namespace

// The convolution reads W_b only (any expert count: the mix that fills it
// depends on n, this kernel does not).
bool premix_conv_supported(const Geom &g) {
    return g.bf16 && g.groups == 1 && premix_lds_bytes(g, pick_premix(g)) <= (size_t)kLdsBudget;
}

// The 32x32x16 premix kernel: bf16 3x3 stride-1 layers with W even (position
// pairs), P % 8 == 0 (16-byte output rows), a tile of at most kPmMaxPos
// padded positions and at most kPmSlots x 256 staging half-tasks per chunk.
static bool pm3_ok(const Geom &g) {
    if (!(g.bf16 && g.groups == 1 && g.KH == 3 && g.KW == 3 && g.stride == 1 && g.W % 2 == 0 && g.P % 8 == 0))
        return false;
    const int tr = tile_rows_for(g, kPmMT);
    return tr * (g.W + 2 * g.pad) <= kPmMaxPos && tr * (g.W / 2) * 8 <= kPmSlots * 256;
}

// The 1x1 premix kernel: bf16 1x1 stride-1 layers without padding, P even
// and P % 8 == 0 (position pairs, 16-byte output rows).
static bool pm1_ok(const Geom &g) {
    return g.bf16 && g.groups == 1 && g.KH == 1 && g.KW == 1 && g.stride == 1 && g.pad == 0 && g.P % 8 == 0;
}

hipError_t launch_conv_premix(const Geom &g, const uint16_t *x, const uint16_t *wt, uint16_t *y,
                              hipStream_t stream, ChanAttn att) {
    if (pm1_ok(g) && g.Cin <= 2 * kChunk) {
        ConvArgs a = base_args(g);
        a.n_ptiles = ceil_div(g.P, kPmMT);
        a.n_otiles = ceil_div(g.Cout, 64);
        const long blocks = (long)g.B * a.n_ptiles;
        if (g.Cin <= kChunk)
            hipLaunchKernelGGL(conv_pm1x_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, x, wt, y, a, att.out);
        else
            hipLaunchKernelGGL(conv_pm1x_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, x, wt, y, a, att.out);
        return hipGetLastError();
    }
    if (pm1_ok(g)) {
        // tiles of 96 output channels where they pad less than tiles of 64
        const bool cb3 = ceil_div(g.Cout, 96) * 96 < ceil_div(g.Cout, 64) * 64;
        ConvArgs a = base_args(g);
        a.n_ptiles = ceil_div(g.P, kPmMT);
        a.n_otiles = ceil_div(g.Cout, cb3 ? 96 : 64);
        // persistent: at most pm1_resident workgroups per CU, a multiple of 8
        const long tiles = (long)g.B * a.n_ptiles * a.n_otiles;
        const long blocks = std::min(ceil_div((int)std::min(tiles, (long)INT32_MAX - 8), 8) * 8L,
                                     (long)kCUs * pm1_resident(cb3 ? 3 : 2));
        if (cb3)
            hipLaunchKernelGGL(conv_pm1_kernel<3>, dim3((unsigned)blocks), dim3(256), 0, stream, x, wt, y, a, att.out);
        else
            hipLaunchKernelGGL(conv_pm1_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, x, wt, y, a, att.out);
        return hipGetLastError();
    }
    if (pm3w_ok(g)) return launch_conv_pm3w(g, x, wt, y, stream, att.out);
    if (pm3_ok(g)) {
        ConvArgs a = base_args(g);
        a.tile_rows = tile_rows_for(g, kPmMT);
        a.n_ptiles = ceil_div(g.P, kPmMT);
        a.n_otiles = ceil_div(g.Cout, 64);
        const long blocks = (long)g.B * a.n_ptiles * a.n_otiles;
        hipLaunchKernelGGL(conv_pm3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, wt, y, a, att.out);
        return hipGetLastError();
    }
    const PremixCfg c = pick_premix(g);
    if (c.FM == kPremixLarge.FM)
        return launch_premix_cfg<kPremixLarge.FM, kPremixLarge.FN, kPremixLarge.NW>(g, x, wt, y, stream, att.out);
    return launch_premix_cfg<kPremixSmall.FM, kPremixSmall.FN, kPremixSmall.NW>(g, x, wt, y, stream, att.out);
}

}  // namespace dynconv
