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
#include <algorithm>

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

// ---- one-pass form: 3x3, stride 1, pad 1, Cin and Cout up to 64 -----------
// Workgroup (example b, band of R output rows) of 512 threads, everything in
// LDS: the example's W_b (rows o of 9 x CI bf16 in tap-major, channel-minor
// order, 16 bytes of padding per row so that 8 lanes reading 8 rows hit
// different banks) and the band's input rows with one halo row above and
// below, channel-innermost (16-byte chunks of 8 channels per position,
// swizzled by position so gathers of neighbouring positions spread over the
// banks), with zero columns left and right.
//   1. W_b and the input rows load; the band's own rows of y are written as
//      x (residual) or 0 from the same registers; the band's mask is
//      compacted into a list of active positions (ordered prefix sum);
//   2. each wave takes (32 active positions, 32 output channels) items: 9
//      taps x CI / 16 products of v_mfma_f32_32x32x16_bf16 with W_b rows as A
//      and the active positions' gathered 8-channel slices as B;
//   3. the residual joins the sums in float32 and each active output is
//      rounded once and stored (after the workgroup barrier that completes
//      the plain copy, so the later store wins).
// The input is read once (plus two halo rows per band), y written once, and
// nothing is staged in HBM.
constexpr int kGbThreads = 512;
constexpr int kGbLds = 163840;                     // the whole LDS of a CU
constexpr int kGbCoutMax = 64;
constexpr int kGbListMax = 1024;                   // active-position list (ushort)
__host__ __device__ constexpr int gb_wpitch(int CI) { return 9 * CI * 2 + 16; }
__host__ __device__ constexpr int gb_xbytes(int CI) { return kGbLds - kGbCoutMax * gb_wpitch(CI) - kGbListMax * 2 - 64; }

struct GbArgs {
    int B, Cin, Cout, H, W, R, nbands, residual, per_xcd;
};

template <int CI>
__global__ __launch_bounds__(kGbThreads) void conv_gated_band_kernel(const uint16_t *__restrict__ x,
                                                                     const uint16_t *__restrict__ wt,
                                                                     const uint8_t *__restrict__ mask,
                                                                     uint16_t *__restrict__ y, GbArgs a) {
    constexpr int NC = CI / 8;        // 16-byte channel chunks per position
    constexpr int WP = gb_wpitch(CI);
    __shared__ __attribute__((aligned(16))) unsigned char sm[kGbLds];
    unsigned char *sW = sm;
    unsigned char *sX = sm + kGbCoutMax * WP;
    uint16_t *sList = reinterpret_cast<uint16_t *>(sm + kGbCoutMax * WP + gb_xbytes(CI));
    int *sCnt = reinterpret_cast<int *>(sm + kGbCoutMax * WP + gb_xbytes(CI) + kGbListMax * 2);  // 9 ints
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // workgroups go to the 8 XCDs in turn: item i = (example, band) in
    // example-major order runs on XCD i / per_xcd, so an example's bands
    // share one L2 (its W_b and their halo rows are fetched once)
    const int item = (int)(blockIdx.x & 7) * a.per_xcd + (int)(blockIdx.x >> 3);
    const int b = item / a.nbands, band = item - b * a.nbands;
    if (b >= a.B) return;
    const int H = a.H, W = a.W, W2 = W + 2, HW = H * W;
    const int r0 = band * a.R, rows = min(a.R, H - r0);
    const float inv_w = 1.f / (float)W;
    // the band's gate bytes load with everything else (clamped, unconditional)
    const int np = rows * W;
    const uint8_t *mb = mask + (long)b * HW + (long)r0 * W;
    constexpr int NMK = kGbListMax / kGbThreads;
    uint8_t mk[NMK];
#pragma unroll
    for (int j = 0; j < NMK; ++j) mk[j] = mb[min(j * kGbThreads + tid, np - 1)];
    // LDS byte offset of 8 channels at a tile position; the chunk index is
    // swizzled by the column and its 8-column group, so that both the
    // staging writes (neighbouring lanes 8 columns apart) and the gathers
    // (neighbouring active positions) spread over the banks
    auto xchunk = [&](int rho, int kap, int cc) {
        return ((rho * W2 + kap) * NC + (cc ^ ((kap ^ (kap >> 3)) & (NC - 1)))) * 16;
    };
    // exact quotients of non-negative integers below 2^20 through a float
    // reciprocal (the product's error stays far below the 0.5 / d margin)
    auto qdiv = [](int n, float inv) { return (int)(((float)n + 0.5f) * inv); };

    // ---- 1a, 1b. loads first: W_b of example b (chunk q = (t, o, cc) of
    // wt[b][t][o][cp]) and the input rows r0 - 1 .. r0 + rows as 8 x 8
    // (channel x position) blocks, every index clamped so that all loads are
    // in flight together; then the LDS writes. A block is transposed in
    // registers into 8-channel chunks, and the band's rows of y get x
    // (residual) from the same registers. Repeated (clamped) chunks and
    // blocks write the same values to the same places.
    {
        constexpr int NWQ = (9 * kGbCoutMax * NC + kGbThreads - 1) / kGbThreads;
        constexpr int NXB = 2;  // blocks per thread: (R + 2) * NC * W / 8 <= 2 * 512 by the LDS bound
        const int nq = 9 * a.Cout * NC;
        const int nw8 = W / 8, nblk = (rows + 2) * NC * nw8;
        const float inv_wq = 1.f / (float)(a.Cout * NC), inv_blk = 1.f / (float)(NC * nw8), inv_nw8 = 1.f / (float)nw8;
        const uint16_t *wb = wt + (long)b * 9 * a.Cout * CI;
        const uint16_t *xb = x + (long)b * a.Cin * HW;
        uint16_t *yb = y + (long)b * a.Cout * HW;
        u32x4_t wv[NWQ], xv[NXB][8];
#pragma unroll
        for (int k = 0; k < NWQ; ++k) wv[k] = reinterpret_cast<const u32x4_t *>(wb)[min(tid + kGbThreads * k, nq - 1)];
#pragma unroll
        for (int m = 0; m < NXB; ++m) {
            const int blk = min(tid + kGbThreads * m, nblk - 1);
            const int rho = qdiv(blk, inv_blk), rem = blk - rho * (NC * nw8), c8 = qdiv(rem, inv_nw8),
                      w8 = rem - c8 * nw8;
            const int h = min(max(r0 - 1 + rho, 0), H - 1);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                xv[m][i] = *reinterpret_cast<const u32x4_t *>(xb + ((long)min(c8 * 8 + i, a.Cin - 1) * H + h) * W + w8 * 8);
        }
#pragma unroll
        for (int k = 0; k < NWQ; ++k) {
            const int q = min(tid + kGbThreads * k, nq - 1);
            const int t = qdiv(q, inv_wq), rem = q - t * (a.Cout * NC), o = rem / NC, cc = rem - o * NC;
            *reinterpret_cast<u32x4_t *>(sW + o * WP + (t * CI + cc * 8) * 2) = wv[k];
        }
#pragma unroll
        for (int m = 0; m < NXB; ++m) {
            const int blk = min(tid + kGbThreads * m, nblk - 1);
            const int rho = qdiv(blk, inv_blk), rem = blk - rho * (NC * nw8), c8 = qdiv(rem, inv_nw8),
                      w8 = rem - c8 * nw8;
            const int h = r0 - 1 + rho;
            const bool hin = h >= 0 && h < H;
            u32x4_t v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool ok = hin && c8 * 8 + i < a.Cin;
                v[i] = ok ? xv[m][i] : u32x4_t{0u, 0u, 0u, 0u};
            }
            if (a.residual && rho >= 1 && rho <= rows) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int c = c8 * 8 + i;
                    if (c < a.Cout) *reinterpret_cast<u32x4_t *>(yb + ((long)c * H + h) * W + w8 * 8) = v[i];
                }
            }
            // position j of the block: channels 2k, 2k + 1 from word j / 2 of v[2k], v[2k + 1]
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t o;
                o.x = __builtin_amdgcn_perm(v[1][j >> 1], v[0][j >> 1], sel);
                o.y = __builtin_amdgcn_perm(v[3][j >> 1], v[2][j >> 1], sel);
                o.z = __builtin_amdgcn_perm(v[5][j >> 1], v[4][j >> 1], sel);
                o.w = __builtin_amdgcn_perm(v[7][j >> 1], v[6][j >> 1], sel);
                *reinterpret_cast<u32x4_t *>(sX + xchunk(rho, w8 * 8 + j + 1, c8)) = o;
            }
        }
        // rows past Cout up to the next multiple of 32 read as zeros
        const int opad = (a.Cout + 31) / 32 * 32;
        for (int i = tid; i < (opad - a.Cout) * (WP / 16); i += kGbThreads)
            reinterpret_cast<u32x4_t *>(sW + a.Cout * WP)[i] = u32x4_t{0u, 0u, 0u, 0u};
        // zero columns left and right of every tile row
        for (int i = tid; i < (rows + 2) * 2 * NC; i += kGbThreads) {
            const int rho = i / (2 * NC), rem = i - rho * 2 * NC, side = rem / NC, cc = rem - side * NC;
            *reinterpret_cast<u32x4_t *>(sX + xchunk(rho, side ? W + 1 : 0, cc)) = u32x4_t{0u, 0u, 0u, 0u};
        }
        // without the residual, the band's rows of y start at 0
        if (!a.residual) {
            const int nz = a.Cout * rows * nw8;
            for (int i = tid; i < nz; i += kGbThreads) {
                const int o = i / (rows * nw8), rem = i - o * rows * nw8, rr = rem / nw8, w8 = rem - rr * nw8;
                *reinterpret_cast<u32x4_t *>(yb + ((long)o * H + r0 + rr) * W + w8 * 8) = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    }
    // ---- 1c. the band's active positions in increasing order
    {
        int base = 0;
#pragma unroll
        for (int j = 0; j < NMK; ++j) {
            const int p = j * kGbThreads + tid;
            if (j * kGbThreads >= np) break;
            const int on = (p < np && mk[j] != 0) ? 1 : 0;
            const uint64_t bal = __ballot(on);
            const int below = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
            if (lane == 0) sCnt[wave] = __popcll(bal);
            __syncthreads();
            int off = base;
            for (int w = 0; w < wave; ++w) off += sCnt[w];
            if (on) sList[off + below] = (uint16_t)p;
            for (int w = 0; w < kGbThreads / 64; ++w) base += sCnt[w];
            __syncthreads();
        }
        if (tid == 0) sCnt[8] = base;
    }
    __syncthreads();

    // ---- 2, 3. (32 positions, 32 channels) items over the waves: wave w
    // takes items w, w + 8, ... The first round's products overlap the
    // draining of the plain copy's stores; then every wave waits for its own
    // stores and meets the others (the barrier alone waits only for LDS), so
    // no active output is stored before the copy that it overwrites.
    const int cnt = sCnt[8];
    const int nog = (a.Cout + 31) / 32, nitems = (cnt + 31) / 32 * nog;
    const int l32 = lane & 31, hh = lane >> 5;
    constexpr int NW = kGbThreads / 64;
    for (int it = wave; it < ((nitems + NW - 1) / NW) * NW || it == wave; it += NW) {
        const bool have = it < nitems;
        const int itc = have ? it : 0;
        const int g = itc / nog, og = itc - g * nog;
        const int k = g * 32 + l32;
        const bool ok = have && k < cnt;
        const int p = sList[k < cnt ? k : 0];
        const int rl = qdiv(p, inv_w), s = p - rl * W;  // band row and column of the lane's position
        const unsigned char *arow = sW + (og * 32 + l32) * WP + hh * 16;
        f32x16_t acc = {};
        if (have) {
            // product j = (tap t, 16-channel slice q); operand reads run two
            // products ahead (the scheduling barriers keep that order)
            constexpr int NP = 9 * (CI / 16);
            bf16x8_t fa[NP], fb[NP];
            auto rd = [&](int j) {
                const int t = j / (CI / 16), q = j - t * (CI / 16), u = t / 3, v = t - u * 3;
                fa[j] = *reinterpret_cast<const bf16x8_t *>(arow + (t * CI + 16 * q) * 2);
                fb[j] = *reinterpret_cast<const bf16x8_t *>(sX + xchunk(rl + u, s + v, 2 * q + hh));
            };
            __builtin_amdgcn_sched_barrier(0);
            rd(0);
            rd(1);
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                if (j + 2 < NP) rd(j + 2);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j], fb[j], acc, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (it == wave) {  // first round: the plain copy completes everywhere first
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        // D(lane, 4j + i): output channel 32 og + 8j + 4hh + i at the lane's position
        if (ok) {
            uint16_t *yp = y + (long)b * a.Cout * HW + (long)(r0 + rl) * W + s;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int oc = og * 32 + 8 * j + 4 * hh;  // 4 consecutive channels, one 8-channel chunk
                uint32_t xr0 = 0u, xr1 = 0u;
                if (a.residual) {
                    const u32x2_t xv =
                        *reinterpret_cast<const u32x2_t *>(sX + xchunk(rl + 1, s + 1, oc >> 3) + (oc & 7) * 2);
                    xr0 = xv.x;
                    xr1 = xv.y;
                }
                const float res[4] = {bf16_lo(xr0), bf16_hi(xr0), bf16_lo(xr1), bf16_hi(xr1)};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (oc + i < a.Cout) yp[(long)(oc + i) * HW] = f32_to_bf16(res[i] + acc[4 * j + i]);
            }
        }
    }
}

}  // namespace

// scratch: compacted positions and counts, then the channel-innermost x
size_t sparse_index_bytes(const Geom &g) {
    const size_t idx = ((size_t)g.B * g.P + g.B) * sizeof(int);
    return (idx + 255) / 256 * 256 + (size_t)g.B * g.H * g.W * g.Cin_pad * sizeof(uint16_t);
}

// Band rows for the one-pass form: the most that fit LDS, then fewer so
// that there are at least 256 workgroups (one per CU) where the batch
// allows; 0 if the layer does not fit.
static int gb_rows(const Geom &g) {
    if (!(g.KH == 3 && g.KW == 3 && g.stride == 1 && g.pad == 1 && g.Cin_pad <= 64 && g.Cout <= kGbCoutMax &&
          g.W % 8 == 0 && g.Ho == g.H && g.Wo == g.W))
        return 0;
    const int CI = g.Cin_pad <= 32 ? 32 : 64;
    // LDS for the input rows, the position list, and at most 2 input blocks per thread
    const int rmax = std::min({gb_xbytes(CI) / ((g.W + 2) * CI * 2) - 2, kGbListMax / g.W,
                               2 * kGbThreads / ((CI / 8) * (g.W / 8)) - 2});
    if (rmax < 1) return 0;
    const int want_bands = std::max(1, (256 + g.B - 1) / g.B);
    return std::max(1, std::min(rmax, (g.H + want_bands - 1) / want_bands));
}

bool gated_one_pass(const Geom &g) { return gb_rows(g) > 0; }

hipError_t launch_conv_sparse(const Geom &g, const uint16_t *x, const uint16_t *wt, const uint8_t *mask, int residual,
                              int *idx, uint16_t *y, hipStream_t stream) {
    if (const int R = gb_rows(g)) {
        GbArgs a;
        a.Cin = g.Cin; a.Cout = g.Cout; a.H = g.H; a.W = g.W; a.R = R; a.nbands = ceil_div(g.H, R);
        a.residual = residual;
        a.per_xcd = ceil_div(g.B * a.nbands, 8);
        a.B = g.B;
        const dim3 grid((unsigned)(8 * a.per_xcd));
        if (g.Cin_pad <= 32)
            hipLaunchKernelGGL(conv_gated_band_kernel<32>, grid, dim3(kGbThreads), 0, stream, x, wt, mask, y, a);
        else
            hipLaunchKernelGGL(conv_gated_band_kernel<64>, grid, dim3(kGbThreads), 0, stream, x, wt, mask, y, a);
        return hipGetLastError();
    }
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
