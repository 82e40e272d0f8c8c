// Kernel gradient of the dynamic convolution fused with its contraction
// (bf16, groups == 1, stride 1, n <= 4, 1 x 1 or k x 3 kernels).
//
// The layer's derivative (CondConv: Conditionally Parameterized Convolutions,
// abstract: each example's kernel is learned; KernelWarehouse: Rethinking the
// Design of Dynamic Convolution, abstract: the mixture of static kernels and
// its attentions are learned) with W_b = sum_i alpha[b,i] E_i:
//   dW_b[o][c,u,v] = sum_{r,s} dy[b,o,r,s] * x[b,c, r-p+u, s-p+v]
//   dalpha[b,i]    = <dW_b, E_i>,    dE_i = sum_b alpha[b,i] dW_b
// computed without storing dW_b. Built with the matrix-core results in
// VGPRs (the contraction reads them directly).
#include <algorithm>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

unsigned wf_blocks(long total) { return (unsigned)((total + 255) / 256); }
size_t wf_align(size_t v) { return (v + 255) / 256 * 256; }

// ---- kernel gradient fused with its contraction (bf16, groups == 1,
// stride 1, n <= 4) -----------------------------------------------------------
// dW_b is never stored. Workgroup (64 output channels o0.., 64 kernel columns
// K0.., examples of one group) keeps its dE_i tile (float32) and its E_i tile
// (bf16 pairs) in registers and for each example b:
//   1. computes its 64 x 64 block of dW_b on the matrix cores,
//   2. adds alpha[b,i] dW_b to dE_i and sums <dW_b, E_i> over the block (per
//      row of 16 lanes in LDS, then per wave in a fixed order into
//      dpart[b][i][slot], which dalpha_reduce_kernel adds in slot order).
// Positions run over a zero-padded grid q = r Wp + s (Wp a multiple of 8, at
// least W + 2 pad), in chunks of R output rows of NS products of 16
// positions (NS * 16 >= R Wp). Two passes first write dy as one zero-padded
// run of NS * 16 positions per chunk (zeros for s >= Wo and past the chunk's
// rows) and x as zero-bordered planes of pitch Wp (zero rows down to the
// last chunk's window). The im2col value of column (c, u, v) at position q
// is then the padded x plane at q + u Wp + v, so with KW copies of each
// staged channel window (copy v shifted by v elements) every 8-position
// slice of a column is one aligned 16-byte LDS read, and every 8-position
// slice of a dy row one aligned 16-byte global read straight into the MFMA
// operand, with no bounds test.
//
// The (example, chunk) stages form one software pipeline: while a stage's
// products run, the next stage's x chunks are already in flight and each dy
// operand register is reloaded for the next stage right after its product
// has read it, so memory latency hides behind the matrix work.
constexpr int kWfOT = 64;     // output channels per workgroup
constexpr int kWfKT = 64;     // kernel columns per workgroup
constexpr int kWfNE = 4;      // experts per workgroup pass (layers with fewer run as zero experts)

struct WfArgs {
    int B, Cin, H, W, Cout, KH, KW, pad, Ho, Wo, KT, Kdim, n;
    int Wp;       // padded row pitch
    int Hx;       // rows of a padded x plane (nchunk R + KH - 1 >= H + 2 pad)
    int R;        // output rows per chunk
    int nchunk;   // chunks per example
    int PL;       // LDS elements per staged channel window (multiple of 8)
    int CS;       // LDS elements per copy (>= nch PL, multiple of 8)
    int nch;      // channel slots (the most channels a 64-column tile spans)
    int n_ktiles, ntiles, bper, groups, nslots;
    int want_de;  // 0: the dE tiles are not written
};

// dyq[b][o][ch][j] (j < len = NS * 16): dy[b][o][ch R + j / Wp][j % Wp]
// where j < R Wp, the row is below Ho and j % Wp < Wo, else 0; one thread per
// 8 output elements (one row segment: Wp is a multiple of 8), read as 4
// element pairs (Wo is even, so a pair is all in the row or all out).
__global__ __launch_bounds__(256) void pad_dy_kernel(const uint16_t *__restrict__ dy, uint16_t *__restrict__ dyq,
                                                     long nvec, int Ho, int Wo, int Wp, int R, int nchunk, int len) {
    const long v = (long)blockIdx.x * 256 + threadIdx.x;
    if (v >= nvec) return;
    const int per_chunk = len / 8;
    const long run = v / per_chunk;  // (b, o, ch)
    const int j0 = (int)(v - run * per_chunk) * 8;
    const long bo = run / nchunk;
    const int ch = (int)(run - bo * nchunk);
    const int r = j0 / Wp, s0 = j0 - r * Wp, row = ch * R + r;
    const bool rin = j0 < R * Wp && row < Ho;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(dy + bo * Ho * Wo + (long)(rin ? row : 0) * Wo);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = rin && s0 + 2 * k < Wo ? src[(s0 >> 1) + k] : 0u;
    reinterpret_cast<u32x4_t *>(dyq)[v] = u32x4_t{w[0], w[1], w[2], w[3]};
}

// xq[b][c][h'][w'] = x[b][c][h' - pad][w' - pad] inside the image, else 0
// (Hx rows of Wp); one thread per 8 output elements. For even W the source
// is read as element pairs (and, for odd pad, each output pair joins the
// halves of two source pairs).
__global__ __launch_bounds__(256) void pad_x_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ xq,
                                                    long nvec, int H, int W, int Hx, int Wp, int pad) {
    const long v = (long)blockIdx.x * 256 + threadIdx.x;
    if (v >= nvec) return;
    const int per_row = Wp / 8;
    const long row = v / per_row;  // (b, c, h')
    const int w0 = (int)(v - row * per_row) * 8 - pad;  // source column of output element 0
    const long bc = row / Hx;
    const int h = (int)(row - bc * Hx) - pad;
    const bool hin = h >= 0 && h < H;
    const uint16_t *src = x + (bc * H + (hin ? h : 0)) * W;
    uint32_t w[4];
    if ((W & 1) == 0) {
        const uint32_t *s32 = reinterpret_cast<const uint32_t *>(src);
        // source pairs starting at an even column e: all in or all out of the row
        auto pr = [&](int e) { return hin && e >= 0 && e < W ? s32[e >> 1] : 0u; };
        if ((pad & 1) == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = pr(w0 + 2 * j);
        } else {
            uint32_t d[5];
#pragma unroll
            for (int m = 0; m < 5; ++m) d[m] = pr(w0 - 1 + 2 * m);
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = __builtin_amdgcn_alignbit(d[j + 1], d[j], 16);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int a0 = w0 + 2 * j, a1 = a0 + 1;
            const uint32_t lo = hin && a0 >= 0 && a0 < W ? src[a0] : 0u;
            const uint32_t hi = hin && a1 >= 0 && a1 < W ? src[a1] : 0u;
            w[j] = lo | (hi << 16);
        }
    }
    reinterpret_cast<u32x4_t *>(xq)[v] = u32x4_t{w[0], w[1], w[2], w[3]};
}

// buffer descriptor over nbytes from p (reads past the end return zeros)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wf_rsrc(const void *p, long nbytes) {
    const uint64_t q = reinterpret_cast<uint64_t>(p);
    const uint64_t ps = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)q) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(q >> 32)) << 32);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ps), 0,
                                             __builtin_amdgcn_readfirstlane((int)nbytes), 0x00020000);
}

constexpr int kWfMasked = 0x7ffffff0;  // a buffer offset past every tensor: the read returns zeros

// x + (the value of lane l ^ 1 / l ^ 2 / l + 4 / l + 8 within its row of 16)
__device__ __forceinline__ float add_xor1(float k, float s) {
    return k + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xf, 0xf, true));
}
__device__ __forceinline__ float add_xor2(float k, float s) {
    return k + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xf, 0xf, true));
}
__device__ __forceinline__ float add_ror(float k, int ctrl4or8) {
    const int r = ctrl4or8 == 4 ? __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, k), 0x124, 0xf, 0xf, true)
                                : __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, k), 0x128, 0xf, 0xf, true);
    return k + __builtin_bit_cast(float, r);
}

// LDS pitch (elements) of a staged dy row of a chunk: an odd number of
// 16-byte units, so that the A reads of 16 consecutive rows hit distinct banks
constexpr int wf_apitch(int ns) { return ns * 16 + 8; }

// NS products of 16 positions per stage, KW kernel columns, XL staged x
// chunks per thread per stage. Dynamic LDS: the x copies [KW][CS], the dy
// rows of the workgroup's 64 output channels [64][wf_apitch(NS)], then the
// row sums of <dW_b, E_i> of the group's examples [example][wave][row][i].
template <int NS, int KW, int XL>
__global__ __launch_bounds__(256) void wgrad_fused_kernel(const uint16_t *__restrict__ xq,
                                                          const uint16_t *__restrict__ dyq,
                                                          const uint16_t *__restrict__ ex,
                                                          const float *__restrict__ alpha, float *__restrict__ de,
                                                          float *__restrict__ dpart, WfArgs a) {
    constexpr int NE = kWfNE;
    constexpr bool EF32 = NS == 14 && KW == 3;  // E unpacked once (fits two waves per SIMD here)
    constexpr int LEN = NS * 16;             // padded positions of a chunk
    constexpr int AP = wf_apitch(NS);        // LDS pitch of a dy row
    constexpr int JW = NS == 14 ? 32 : 16;   // threads per dy row in the staging (LEN / 8 of them load)
    constexpr int RSTEP = 256 / JW;          // rows per staging step
    constexpr int NDY = kWfOT / RSTEP;       // staging steps (16-byte dy chunks per thread)
    static_assert(LEN / 8 <= JW && NDY * RSTEP == kWfOT, "dy staging layout");
    extern __shared__ __attribute__((aligned(16))) uint16_t s_x[];
    uint16_t *s_a = s_x + KW * a.CS;
    float *s_p = reinterpret_cast<float *>(s_a + kWfOT * AP);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    // XCD-aware: consecutive logical ids (one example group's tiles) share an XCD
    const int total = a.ntiles * a.groups;
    const int lid = (total & 7) == 0 ? (int)(blockIdx.x & 7) * (total >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
    const int grp = lid / a.ntiles, tile = lid - grp * a.ntiles;
    const int ot = tile / a.n_ktiles, kt = tile - ot * a.n_ktiles;
    const int o0 = ot * kWfOT, K0 = kt * kWfKT;
    const int b_lo = grp * a.bper, b_hi = min(a.B, b_lo + a.bper);
    const int ob = wave & 1, kb = wave >> 1;
    const int c_lo = K0 / a.KT;
    const int nc = min(a.nch, a.Cin - c_lo);
    const int xrows = a.R + a.KH - 1;      // staged x rows per chunk
    const int xchunks = xrows * a.Wp / 8;  // staged 16-byte chunks per channel window
    const int nitems = nc * xchunks;
    const int Px = a.Hx * a.Wp;            // elements of a padded x plane

    // the lane's B column (c, u, v): columns past Kdim read channel slot 0 (finite, and E is 0 there)
    const int col = K0 + 32 * kb + l32;
    const bool col_ok = col < a.Kdim;
    const int c = col_ok ? col / a.KT : c_lo, t = col_ok ? col - c * a.KT : 0;
    const int u = t / KW, v = t - u * KW;
    const int boff = (v * a.CS + (c - c_lo) * a.PL + u * a.Wp + 8 * hh) * 2;  // bytes
    // the lane's A row: staged dy row 32 ob + l32 (output channel o0 + 32 ob + l32)
    const int aoff = ((32 * ob + l32) * AP + 8 * hh) * 2;  // bytes
    // D(lane, 4j + q): output channel o0 + 32 ob + 8j + 4hh + q, column col.
    // The lane's E values as bf16 pairs (element 2k in the low half); masked
    // buffer reads (zeros outside the bank) so that all the loads issue together.
    uint32_t er[NE][8];
    float dea[NE][16];
    {
        const auto rs_e = wf_rsrc(ex, (long)a.n * a.Cout * a.Kdim * 2);
#pragma unroll
        for (int i = 0; i < NE; ++i) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                uint32_t w = 0u;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kk = 2 * k + h;
                    const int o = o0 + 32 * ob + 8 * (kk >> 2) + 4 * hh + (kk & 3);
                    const int off =
                        o < a.Cout && col_ok && i < a.n ? ((i * a.Cout + o) * a.Kdim + col) * 2 : kWfMasked;
                    w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs_e, off, 0, 0) << (16 * h);
                }
                er[i][k] = w;
            }
#pragma unroll
            for (int k = 0; k < 16; ++k) dea[i][k] = 0.f;
        }
    }
    // descriptors over all of dyq and xq (byte offsets below 2^31, checked on the host)
    const auto rs_dy = wf_rsrc(dyq, (long)a.B * a.Cout * a.nchunk * LEN * 2);
    const auto rs_x = wf_rsrc(xq, (long)a.B * a.Cin * Px * 2);
    // the copies' tails past the staged window (read only at positions
    // whose dy is zero) and the slots of channels past Cin hold zeros
    for (int i = tid; i < KW * a.CS / 8; i += 256) reinterpret_cast<u32x4_t *>(s_x)[i] = u32x4_t{0u, 0u, 0u, 0u};

    // the thread's x staging items (channel slot, 16-byte chunk); threads past
    // the items load a repeated one (in bounds) and store nothing
    int xl_off[XL], xs_off[XL];  // global (bytes, within the stage's window) and LDS (elements) offsets
#pragma unroll
    for (int m = 0; m < XL; ++m) {
        const int it = (tid + 256 * m) % nitems;
        const int cl = it / xchunks, k = it - cl * xchunks;
        xl_off[m] = (cl * Px + 8 * k) * 2;
        xs_off[m] = cl * a.PL + 8 * k;
    }
    // the thread's dy staging: chunk j of rows r0 + RSTEP m (rows past Cout
    // repeat row Cout - 1; lanes with j >= LEN / 8 read zeros and store nothing)
    const int dj = tid % JW, dr = tid / JW;
    const bool dj_ok = dj < LEN / 8;
    const int rowb = a.nchunk * LEN * 2;  // bytes between dy rows of one example
    int dl_off[NDY];
#pragma unroll
    for (int m = 0; m < NDY; ++m)
        dl_off[m] = dj_ok ? min(o0 + dr + RSTEP * m, a.Cout - 1) * rowb + dj * 16 : kWfMasked;
    const int ds_off = dr * AP + 8 * dj;  // LDS elements
    // stage (b, ch): uniform byte offsets of its x window and dy runs
    auto x_soff = [&](int b, int ch) { return (int)((((long)b * a.Cin + c_lo) * Px + (long)ch * a.R * a.Wp) * 2); };
    auto dy_soff = [&](int b, int ch) { return (int)((((long)b * a.Cout * a.nchunk) + ch) * LEN * 2); };
    // chunk k of the window, and for KW == 3 the first word of chunk k + 1
    // (all that the shifts by 1 and 2 take from it); the dy chunks
    u32x4_t xv[XL];
    uint32_t xw[XL];
    u32x4_t dv[NDY];
    auto load_stage = [&](int b, int ch) {
        const int so = x_soff(b, ch);
#pragma unroll
        for (int m = 0; m < XL; ++m) {
            xv[m] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_x, xl_off[m], so, 0));
            if (KW == 3) xw[m] = __builtin_amdgcn_raw_buffer_load_b32(rs_x, xl_off[m] + 16, so, 0);
        }
        const int sd = dy_soff(b, ch);
#pragma unroll
        for (int m = 0; m < NDY; ++m)
            dv[m] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_dy, dl_off[m], sd, 0));
    };
    const int nstages = (b_hi - b_lo) * a.nchunk;
    load_stage(b_lo, 0);
    f32x16_t acc = {};
    int b = b_lo, ch = 0;
    for (int st = 0; st < nstages; ++st) {
        __syncthreads();  // zero fill / the previous stage's LDS reads are done
#pragma unroll
        for (int m = 0; m < XL; ++m) {
            if (tid + 256 * m < nitems) {
                u32x4_t *dst = reinterpret_cast<u32x4_t *>(s_x + xs_off[m]);
                const u32x4_t c0 = xv[m];
                dst[0] = c0;
                if (KW == 3) {
                    const uint32_t w4 = xw[m];
                    const int cp = a.CS / 8;  // one copy, in 16-byte units
                    dst[cp] = u32x4_t{__builtin_amdgcn_alignbit(c0.y, c0.x, 16),
                                      __builtin_amdgcn_alignbit(c0.z, c0.y, 16),
                                      __builtin_amdgcn_alignbit(c0.w, c0.z, 16), __builtin_amdgcn_alignbit(w4, c0.w, 16)};
                    dst[2 * cp] = u32x4_t{c0.y, c0.z, c0.w, w4};
                }
            }
        }
        if (dj_ok) {
#pragma unroll
            for (int m = 0; m < NDY; ++m) *reinterpret_cast<u32x4_t *>(s_a + ds_off + RSTEP * m * AP) = dv[m];
        }
        __syncthreads();
        // the next stage's operands (past the last stage: the group's first
        // again, never used) load during this stage's products
        const bool last = ch + 1 == a.nchunk;
        int b1 = last ? b + 1 : b, ch1 = last ? 0 : ch + 1;
        if (st + 1 == nstages) b1 = b_lo;
        load_stage(b1, ch1);
        __builtin_amdgcn_sched_barrier(0);
        const char *pa = reinterpret_cast<const char *>(s_a) + aoff;
        const char *pb = reinterpret_cast<const char *>(s_x) + boff;
        bf16x8_t fa0 = *reinterpret_cast<const bf16x8_t *>(pa), fb0 = *reinterpret_cast<const bf16x8_t *>(pb);
        bf16x8_t fa1 = *reinterpret_cast<const bf16x8_t *>(pa + 32), fb1 = *reinterpret_cast<const bf16x8_t *>(pb + 32);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const bf16x8_t ca = fa0, cb = fb0;
            fa0 = fa1;
            fb0 = fb1;
            if (k + 2 < NS) {
                fa1 = *reinterpret_cast<const bf16x8_t *>(pa + 32 * (k + 2));
                fb1 = *reinterpret_cast<const bf16x8_t *>(pb + 32 * (k + 2));
            }
            if (k == 0 && a.nchunk == 1)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca, cb, f32x16_t{}, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca, cb, acc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (last) {
            // contraction with example b's attentions (zero for i >= n). With
            // EF32 the unpacked E values stay live across the loop (fewer
            // instructions per example); otherwise the packed words count as
            // changed here, so that their unpacking stays in the contraction
            // instead of living as 16 NE floats
            if (!EF32) {
#pragma unroll
                for (int i = 0; i < NE; ++i)
#pragma unroll
                    for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(er[i][k]));
            }
            float p[NE];
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const float al0 = alpha[(long)b * a.n + min(i, a.n - 1)];
                const float al = i < a.n ? al0 : 0.f;
                float s = 0.f;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    dea[i][k] = fmaf(al, acc[k], dea[i][k]);
                    s = fmaf(acc[k], (k & 1) ? bf16_hi(er[i][k >> 1]) : bf16_lo(er[i][k >> 1]), s);
                }
                p[i] = s;
            }
            // the four sums over each row of 16 lanes: lane 4m + i of the row
            // ends with expert i's (pairs of experts swap halves across lane
            // bit 0, then bit 1, then the row adds its four quads)
            const bool b0 = lane & 1, b1l = lane & 2;
            const float q0 = add_xor1(b0 ? p[1] : p[0], b0 ? p[0] : p[1]);
            const float q1 = add_xor1(b0 ? p[3] : p[2], b0 ? p[2] : p[3]);
            float r = add_xor2(b1l ? q1 : q0, b1l ? q0 : q1);
            r = add_ror(r, 4);
            r = add_ror(r, 8);
            if ((lane & 12) == 0) s_p[(((b - b_lo) * 4 + wave) * 4 + (lane >> 4)) * 4 + (lane & 3)] = r;
            if (a.nchunk > 1) acc = f32x16_t{};
        }
        b = b1;
        ch = ch1;
    }
    // the wave sums out, rows added in order: dpart[b * NE + i][tile * 4 + wave]
    __syncthreads();
    for (int j = tid; j < (b_hi - b_lo) * 4; j += 256) {
        const float *q = s_p + j * 16;
        const int bl = j >> 2, w = j & 3;
#pragma unroll
        for (int i = 0; i < NE; ++i)
            dpart[((long)(b_lo + bl) * NE + i) * a.nslots + tile * 4 + w] = ((q[i] + q[4 + i]) + q[8 + i]) + q[12 + i];
    }
    if (!a.want_de) return;
    float *out = de + (long)grp * a.n * a.Cout * a.Kdim;
#pragma unroll
    for (int i = 0; i < NE; ++i)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int o = o0 + 32 * ob + 8 * (k >> 2) + 4 * hh + (k & 3);
            if (i < a.n && o < a.Cout && col_ok) out[((long)i * a.Cout + o) * a.Kdim + col] = dea[i][k];
        }
}

// Plan of the fused kernel gradient (bf16, groups == 1, stride 1, n <= 4,
// KW 1 or 3, Wo even): false where it does not apply or would waste more
// than a third of its products on padding. Chunks of R output rows take NS =
// 14 or 8 products of 16 padded positions (whichever wastes less). The LDS
// strides of the staged windows and copies are padded (in 16-byte steps) so
// that the B reads of each group of 16 lanes spread over the banks. The
// example groups minimise (workgroups per compute unit) x (examples per
// workgroup) plus the cost of each group's dE partial sums in memory.
struct WfPlan {
    WfArgs a;
    size_t lds;
    int ns, xl;
};
constexpr size_t kWfLds = 80 * 1024;  // two workgroups per compute unit

// Worst bank-conflict degree of the B reads (64 banks of 4 bytes, 16 lanes
// per pass) over the first k-tiles, for window stride PL and copy stride CS.
int wf_conflicts(const WfArgs &a, int PL, int CS) {
    int worst = 0;
    for (int kt = 0; kt < std::min(a.n_ktiles, 3); ++kt) {
        const int K0 = kt * kWfKT, c_lo = K0 / a.KT;
        for (int grp = 0; grp < 8; ++grp) {  // kb (2) x hh (2) x 16-lane half (2)
            const int kb = grp >> 2, hh = (grp >> 1) & 1, half = grp & 1;
            int cnt[16] = {0};
            for (int l = 0; l < 16; ++l) {
                const int col = std::min(K0 + 32 * kb + 16 * half + l, a.Kdim - 1);
                const int c = col / a.KT, t = col - c * a.KT, u = t / a.KW, v = t - u * a.KW;
                const int e = v * CS + (c - c_lo) * PL + u * a.Wp + 8 * hh;
                ++cnt[(e / 8) & 15];
            }
            for (int q = 0; q < 16; ++q) worst = std::max(worst, cnt[q]);
        }
    }
    return worst;
}

bool wf_plan_uncached(const Geom &g, WfPlan &pl) {
    if (!(g.bf16 && g.groups == 1 && g.stride == 1 && g.n <= kWfNE && (g.KW == 1 || g.KW == 3) && g.Wo % 2 == 0 &&
          g.Ho >= 1))
        return false;
    WfArgs &a = pl.a;
    a = WfArgs{};
    a.B = g.B; a.Cin = g.Cin; a.H = g.H; a.W = g.W; a.Cout = g.Cout; a.KH = g.KH; a.KW = g.KW; a.pad = g.pad;
    a.Ho = g.Ho; a.Wo = g.Wo; a.KT = g.KT; a.Kdim = g.Cin * g.KT; a.n = g.n;
    a.Wp = (g.W + 2 * g.pad + 7) / 8 * 8;
    // the most channels 64 consecutive columns can span: the first starts at
    // tap KT - 1 of its channel at worst, so 62 / KT + 2
    a.nch = std::min(g.Cin, (kWfKT - 2) / g.KT + 2);
    long best = -1;
    int plane = 0;
    for (int NS : {14, 8}) {
        for (int R = std::min(g.Ho, NS * 16 / a.Wp); R >= 1; --R) {
            const int pln = (g.KH - 1) * a.Wp + 16 * NS;
            const int xchunks = (R + g.KH - 1) * a.Wp / 8;
            if ((size_t)g.KW * (a.nch * (pln + 64) + 64) * 2 + (size_t)kWfOT * wf_apitch(NS) * 2 + 64 * 256 > kWfLds ||
                a.nch * xchunks > 256 * 2)
                continue;
            const long cost = (long)ceil_div(g.Ho, R) * NS;
            if (best < 0 || cost < best) {
                best = cost;
                a.R = R; plane = pln; pl.ns = NS;
                pl.xl = a.nch * xchunks > 256 ? 2 : 1;
            }
            break;
        }
    }
    if (best < 0 || best * 16 * 2 > (long)g.Ho * a.Wp * 3) return false;
    a.nchunk = ceil_div(g.Ho, a.R);
    a.Hx = a.nchunk * a.R + g.KH - 1;
    // byte offsets of the buffer reads (padded copies, bank) stay below 2^31
    if ((long)g.B * g.Cin * a.Hx * a.Wp * 2 + 64 >= (1L << 31) ||
        (long)g.B * g.Cout * a.nchunk * pl.ns * 16 * 2 + 64 >= (1L << 31) || (long)g.n * g.Cout * a.Kdim * 2 + 64 >= (1L << 31))
        return false;
    a.n_ktiles = ceil_div(a.Kdim, kWfKT);
    a.ntiles = ceil_div(g.Cout, kWfOT) * a.n_ktiles;
    a.nslots = a.ntiles * 4;
    int bestc = 1 << 30;
    for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 8; ++j) {
            const int PL = plane + 8 * i, CS = a.nch * PL + 8 * j;
            const int cf = wf_conflicts(a, PL, CS);
            if (cf < bestc) { bestc = cf; a.PL = PL; a.CS = CS; }
        }
    const size_t fixed = (size_t)g.KW * a.CS * 2 + (size_t)kWfOT * wf_apitch(pl.ns) * 2;
    // row sums of at most this many examples fit beside the windows
    const int bmax = (int)((kWfLds - fixed) / 256);
    // Cost of c example groups in units of one workgroup's example (about
    // 2.1 us per 14 products with two workgroups per compute unit): rounds of
    // 512 resident workgroups times the examples per workgroup, plus each
    // group's dE partial sums (written, then read again, at 5 TB/s). The
    // fewest groups within 10 % of the cheapest win (fewer partial sums).
    const double t_ex = 2.1e-6 * (double)(a.nchunk * pl.ns) / 14.0;
    const double pen = (double)g.n * g.Cout * a.Kdim * 8 / 5e12 / t_ex;
    const int cmax = std::min(g.B, 64);
    std::vector<double> cost(cmax + 1, -1.0);
    double cheapest = -1.0;
    for (int c = 1; c <= cmax; ++c) {
        if (ceil_div(g.B, c) > bmax) continue;
        cost[c] = (double)ceil_div(a.ntiles * c, 512) * ceil_div(g.B, c) + (c > 1 ? c * pen : 0.0);
        if (cheapest < 0 || cost[c] < cheapest) cheapest = cost[c];
    }
    int G = 0;
    for (int c = 1; c <= cmax && G == 0; ++c)
        if (cost[c] >= 0 && cost[c] <= 1.1 * cheapest) G = c;
    if (G == 0) return false;
    a.bper = ceil_div(g.B, G);
    a.groups = ceil_div(g.B, a.bper);
    pl.lds = fixed + (size_t)a.bper * 256;
    return true;
}
// The plan (its bank search takes about 0.1 ms) for the last few layer
// shapes: the workspace query and the launch of one call, and the calls of a
// training loop, share one search.
bool wf_plan(const Geom &g, WfPlan &pl) {
    struct Entry {
        Geom g;
        bool ok;
        WfPlan pl;
    };
    constexpr int kSlots = 16;
    static Entry cache[kSlots];
    static int used = 0, next = 0;
    static std::mutex mu;
    auto same = [](const Geom &x, const Geom &y) {
        return x.B == y.B && x.Cin == y.Cin && x.H == y.H && x.W == y.W && x.Cout == y.Cout && x.KH == y.KH &&
               x.KW == y.KW && x.stride == y.stride && x.pad == y.pad && x.groups == y.groups && x.n == y.n &&
               x.bf16 == y.bf16;
    };
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (same(cache[i].g, g)) {
                pl = cache[i].pl;
                return cache[i].ok;
            }
    }
    const bool ok = wf_plan_uncached(g, pl);
    std::lock_guard<std::mutex> lock(mu);
    cache[next] = Entry{g, ok, pl};
    next = (next + 1) % kSlots;
    used = std::max(used, next == 0 ? kSlots : next);
    return ok;
}
size_t wf_dpart_bytes(const WfArgs &a) { return wf_align((size_t)a.B * kWfNE * a.nslots * sizeof(float)); }
size_t wf_dep_bytes(const WfArgs &a) {
    return a.groups > 1 ? wf_align((size_t)a.groups * a.n * a.Cout * a.Kdim * sizeof(float)) : 0;
}
size_t wf_dyq_bytes(const WfArgs &a, int ns) { return wf_align((size_t)a.B * a.Cout * a.nchunk * ns * 16 * 2); }
size_t wf_xq_bytes(const WfArgs &a) { return wf_align((size_t)a.B * a.Cin * a.Hx * a.Wp * 2); }

}  // namespace

size_t wgrad_fused_bytes(const Geom &g) {
    WfPlan pl;
    if (!wf_plan(g, pl)) return 0;
    return wf_dpart_bytes(pl.a) + wf_dep_bytes(pl.a) + wf_dyq_bytes(pl.a, pl.ns) + wf_xq_bytes(pl.a);
}

hipError_t launch_wgrad_fused(const Geom &g, const void *x, const void *dy, const void *experts,
                              const float *alpha, float *scratch, float *dalpha, float *dexperts, hipStream_t stream) {
    {
        WfPlan pl;
        if (wf_plan(g, pl)) {
            WfArgs &f = pl.a;
            const size_t lds = pl.lds;
            // scratch: dalpha partial sums | dE per example group | dy with
            // padded rows | x as padded planes
            char *base = reinterpret_cast<char *>(scratch);
            float *dpart = scratch;
            float *dep = f.groups > 1 ? reinterpret_cast<float *>(base + wf_dpart_bytes(f)) : dexperts;
            uint16_t *dyq = reinterpret_cast<uint16_t *>(base + wf_dpart_bytes(f) + wf_dep_bytes(f));
            uint16_t *xq =
                reinterpret_cast<uint16_t *>(base + wf_dpart_bytes(f) + wf_dep_bytes(f) + wf_dyq_bytes(f, pl.ns));
            f.want_de = dexperts != nullptr;
            hipError_t e;
            {
                const int len = pl.ns * 16;
                const long nv = (long)g.B * g.Cout * f.nchunk * (len / 8);
                hipLaunchKernelGGL(pad_dy_kernel, dim3(wf_blocks(nv)), dim3(256), 0, stream,
                                   static_cast<const uint16_t *>(dy), dyq, nv, g.Ho, g.Wo, f.Wp, f.R, f.nchunk, len);
                const long nx = (long)g.B * g.Cin * f.Hx * (f.Wp / 8);
                hipLaunchKernelGGL(pad_x_kernel, dim3(wf_blocks(nx)), dim3(256), 0, stream,
                                   static_cast<const uint16_t *>(x), xq, nx, g.H, g.W, f.Hx, f.Wp, g.pad);
                e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
            const dim3 grid((unsigned)(f.ntiles * f.groups));
            auto go = [&](auto kern) {
                hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (e2 != hipSuccess) return e2;
                hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, xq, dyq,
                                   static_cast<const uint16_t *>(experts), alpha, dep, dpart, f);
                return hipGetLastError();
            };
            const int sel = (pl.ns == 14 ? 4 : 0) + (g.KW == 3 ? 2 : 0) + (pl.xl == 2 ? 1 : 0);
            switch (sel) {
            case 0: e = go(wgrad_fused_kernel<8, 1, 1>); break;
            case 1: e = go(wgrad_fused_kernel<8, 1, 2>); break;
            case 2: e = go(wgrad_fused_kernel<8, 3, 1>); break;
            case 3: e = go(wgrad_fused_kernel<8, 3, 2>); break;
            case 4: e = go(wgrad_fused_kernel<14, 1, 1>); break;
            case 5: e = go(wgrad_fused_kernel<14, 1, 2>); break;
            case 6: e = go(wgrad_fused_kernel<14, 3, 1>); break;
            default: e = go(wgrad_fused_kernel<14, 3, 2>); break;
            }
            if (e != hipSuccess) return e;
            if (dexperts && f.groups > 1) {
                e = launch_dE_reduce(dep, dexperts, (long)g.n * g.Cout * f.Kdim, f.groups, stream);
                if (e != hipSuccess) return e;
            }
            if (!dalpha) return hipSuccess;
            return launch_dalpha_reduce(dpart, dalpha, g.B, g.n, kWfNE, f.nslots, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace dynconv
