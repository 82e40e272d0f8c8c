// Mixing: each example's kernel is a linear mixture of the n static expert
// kernels weighted by its attentions, W_b = sum_i alpha[b,i] E_i
// (KernelWarehouse: Rethinking the Design of Dynamic Convolution, abstract).
//
// mix_natural_kernel: the stand-alone mix in the experts' own layout. Each
//   thread owns 8 consecutive kernel elements and a tile of BT examples: it
//   reads its 8 elements of every expert once (16-32 byte loads), widens
//   them to float once, and writes BT mixed vectors, so the expert bank is
//   read once per batch tile while the B mixed kernels stream out.
// mix_mfma_kernel: the stand-alone mix of bf16 banks with more than 8
//   experts, as a small-K product on the matrix cores (see the kernel).
// pack_experts_kernel: the expert bank in the layout the MFMA convolution
//   reads, packed[t][o][cp][ip]: tap-major, channels contiguous and padded
//   to the 32-wide K chunk, expert pairs sharing one 32-bit word so that a
//   bf16 dot2 instruction mixes two experts at once.
// premix_kernel: mixed kernels in the convolution's layout wt[b][t][o][cp],
//   computed from the packed bank with bf16 dot2 instructions;
//   premix_mfma_kernel the same on the matrix cores when the padded expert
//   count is a multiple of 8.
//
// Precision: natural mixing sums in float32 in expert order and rounds
// once. The dot2 mixes split each float32 attention into a bf16 high part
// and a bf16 low part (alpha = hi + lo up to 2^-17 relative), so two dot2
// terms per expert pair keep the attentions' precision well below the
// final bf16 rounding of the mixed kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace dynconv {
namespace {

constexpr int kMixThreads = 256;
constexpr int kMixBT = 8;     // examples per thread in the natural mix
constexpr int kMixChunk = 4;  // experts widened per pass

template <typename T>
struct Vec8;  // 8 consecutive elements
template <> struct Vec8<uint16_t> {
    u32x4_t v;
    __device__ __forceinline__ void load(const uint16_t *p) {
        v = *reinterpret_cast<const u32x4_t *>(p);
    }
    __device__ __forceinline__ void widen(float f[8]) const {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
    static __device__ __forceinline__ void store(uint16_t *p, const float f[8]) {
        u32x4_t o;
        o.x = pack_bf16x2(f[0], f[1]); o.y = pack_bf16x2(f[2], f[3]);
        o.z = pack_bf16x2(f[4], f[5]); o.w = pack_bf16x2(f[6], f[7]);
        *reinterpret_cast<u32x4_t *>(p) = o;
    }
};
template <> struct Vec8<float> {
    f32x4_t a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = reinterpret_cast<const f32x4_t *>(p)[0];
        b = reinterpret_cast<const f32x4_t *>(p)[1];
    }
    __device__ __forceinline__ void widen(float f[8]) const {
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    }
    static __device__ __forceinline__ void store(float *p, const float f[8]) {
        f32x4_t o0 = {f[0], f[1], f[2], f[3]}, o1 = {f[4], f[5], f[6], f[7]};
        reinterpret_cast<f32x4_t *>(p)[0] = o0;
        reinterpret_cast<f32x4_t *>(p)[1] = o1;
    }
};

// Vector path: wsize % 8 == 0. grid.x over 8-element vectors, grid.y over
// batch tiles of kMixBT examples.
template <typename T>
__global__ __launch_bounds__(kMixThreads) void mix_natural_kernel(
    const float *__restrict__ alpha, const T *__restrict__ experts, T *__restrict__ mixed,
    int B, int n, long wsize) {
    const long nvec = wsize / 8;
    const long v = (long)blockIdx.x * kMixThreads + threadIdx.x;
    if (v >= nvec) return;
    const int b0 = blockIdx.y * kMixBT;
    const int nb = min(kMixBT, B - b0);
    float acc[kMixBT][8];
#pragma unroll
    for (int j = 0; j < kMixBT; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[j][k] = 0.f;
    for (int i0 = 0; i0 < n; i0 += kMixChunk) {
        float e[kMixChunk][8];
#pragma unroll
        for (int ii = 0; ii < kMixChunk; ++ii) {
            if (i0 + ii < n) {
                Vec8<T> q;
                q.load(experts + (long)(i0 + ii) * wsize + v * 8);
                q.widen(e[ii]);
            }
        }
#pragma unroll
        for (int j = 0; j < kMixBT; ++j) {
            if (j < nb) {
                const float *a = alpha + (long)(b0 + j) * n + i0;
#pragma unroll
                for (int ii = 0; ii < kMixChunk; ++ii) {
                    if (i0 + ii < n) {
                        const float aj = a[ii];
#pragma unroll
                        for (int k = 0; k < 8; ++k) acc[j][k] = fmaf(aj, e[ii][k], acc[j][k]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kMixBT; ++j)
        if (j < nb) Vec8<T>::store(mixed + (long)(b0 + j) * wsize + v * 8, acc[j]);
}

// Vector path for n <= kMixMaxN: all of a thread's expert vectors load at
// once (clamped indices, no branches, so their latencies overlap); experts
// past n get attention 0. Then expert by expert: widen, and accumulate into
// the kMixBT examples (attentions are uniform across the workgroup).
constexpr int kMixMaxN = 8;  // above this the accumulate is VALU-bound; chunked kernel
template <typename T, int NMAX>
__global__ __launch_bounds__(kMixThreads) void mix_natural_all_kernel(
    const float *__restrict__ alpha, const T *__restrict__ experts, T *__restrict__ mixed,
    int B, int n, long wsize) {
    const long nvec = wsize / 8;
    const long v = min((long)blockIdx.x * kMixThreads + threadIdx.x, nvec - 1);
    const bool active = (long)blockIdx.x * kMixThreads + threadIdx.x < nvec;
    const int b0 = blockIdx.y * kMixBT;
    const int nb = min(kMixBT, B - b0);
    Vec8<T> q[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) q[i].load(experts + (long)min(i, n - 1) * wsize + v * 8);
    float acc[kMixBT][8];
#pragma unroll
    for (int j = 0; j < kMixBT; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[j][k] = 0.f;
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        float e[8];
        q[i].widen(e);
#pragma unroll
        for (int j = 0; j < kMixBT; ++j) {
            const float aj = (i < n && j < nb) ? alpha[(long)(b0 + j) * n + min(i, n - 1)] : 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[j][k] = fmaf(aj, e[k], acc[j][k]);
        }
    }
    if (!active) return;
#pragma unroll
    for (int j = 0; j < kMixBT; ++j)
        if (j < nb) Vec8<T>::store(mixed + (long)(b0 + j) * wsize + v * 8, acc[j]);
}

// Scalar path for any wsize: one element per thread, all examples.
template <typename T>
__global__ __launch_bounds__(kMixThreads) void mix_scalar_kernel(
    const float *__restrict__ alpha, const T *__restrict__ experts, T *__restrict__ mixed,
    int B, int n, long wsize) {
    const long e = (long)blockIdx.x * kMixThreads + threadIdx.x;
    if (e >= wsize) return;
    for (int b = blockIdx.y; b < B; b += gridDim.y) {
        float acc = 0.f;
        for (int i = 0; i < n; ++i)
            acc = fmaf(alpha[(long)b * n + i], Elem<T>::to_f32(experts[(long)i * wsize + e]), acc);
        mixed[(long)b * wsize + e] = Elem<T>::from_f32(acc);
    }
}

// One (tap, output channel, input channel) triple per thread: it loads the
// n experts' values of that weight together and writes its NP2 expert-pair
// words as one vector store, next to those of the neighbouring threads
// (neighbouring input channels). NP2 = 0: any pair count, one word at a time.
// experts[i][o][c][t] (c < Cin, groups == 1) -> packed[t][o][cp][ip]
template <int NP2>
__global__ __launch_bounds__(256) void pack_experts_kernel(const uint16_t *__restrict__ e,
                                                           uint32_t *__restrict__ packed,
                                                           int n, int Cout, int Cin, int KT,
                                                           int Cin_pad, int np2) {
    const long d = (long)blockIdx.x * 256 + threadIdx.x;  // (t Cout + o) Cin_pad + cp
    if (d >= (long)KT * Cout * Cin_pad) return;
    const int c = (int)(d % Cin_pad);
    const long r = d / Cin_pad;
    const int o = (int)(r % Cout), t = (int)(r / Cout);
    const bool cv = c < Cin;
    const long wsize = (long)Cout * Cin * KT;
    const uint16_t *src = e + ((long)o * Cin + min(c, Cin - 1)) * KT + t;
    if constexpr (NP2 > 0) {
        uint32_t v[2 * NP2];
#pragma unroll
        for (int i = 0; i < 2 * NP2; ++i) v[i] = cv && i < n ? src[(long)i * wsize] : 0u;
        uint32_t w[NP2];
#pragma unroll
        for (int p = 0; p < NP2; ++p) w[p] = v[2 * p] | (v[2 * p + 1] << 16);
        uint32_t *dst = packed + d * NP2;
        if constexpr (NP2 % 4 == 0) {
#pragma unroll
            for (int p = 0; p < NP2; p += 4)
                *reinterpret_cast<u32x4_t *>(dst + p) = u32x4_t{w[p], w[p + 1], w[p + 2], w[p + 3]};
        } else if constexpr (NP2 % 2 == 0) {
#pragma unroll
            for (int p = 0; p < NP2; p += 2) *reinterpret_cast<u32x2_t *>(dst + p) = u32x2_t{w[p], w[p + 1]};
        } else {
#pragma unroll
            for (int p = 0; p < NP2; ++p) dst[p] = w[p];
        }
    } else {
        uint32_t *dst = packed + d * np2;
        for (int p = 0; p < np2; ++p) {
            const int i0 = 2 * p, i1 = 2 * p + 1;
            const uint32_t lo = cv && i0 < n ? src[(long)i0 * wsize] : 0u;
            const uint32_t hi = cv && i1 < n ? src[(long)i1 * wsize] : 0u;
            dst[p] = lo | (hi << 16);
        }
    }
}

__device__ __forceinline__ void split_alpha(float a0, float a1, uint32_t &hi, uint32_t &lo) {
    hi = pack_bf16x2(a0, a1);
    lo = pack_bf16x2(a0 - bf16_lo(hi), a1 - bf16_hi(hi));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// premix: thread -> one 8-channel vector of wt[b][t][o][cp], for kPremixBT
// examples. NP2 = n_pad / 2 expert pairs (compile-time).
// 2 examples per thread: 3.93 -> 3.50 us at the ResNet-18 layer against 4 (1: 3.85)
constexpr int kPremixBT = 2;
template <int NP2>
__global__ __launch_bounds__(256) void premix_kernel(const float *__restrict__ alpha,
                                                     const uint32_t *__restrict__ packed,
                                                     uint16_t *__restrict__ wt, int B, int n,
                                                     long nvec /* KT*Cout*Cin_pad/8 */,
                                                     const float *__restrict__ a_in, int Cin, int Cin_pad) {
    const long v = (long)blockIdx.x * 256 + threadIdx.x;
    if (v >= nvec) return;
    const int cp = (int)((v * 8) % Cin_pad);  // first input channel of this vector
    const int b0 = blockIdx.y * kPremixBT;
    // 8 channels x NP2 words, contiguous
    uint32_t w[8][NP2];
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(packed + v * 8 * NP2);
#pragma unroll
    for (int q = 0; q < 2 * NP2; ++q) {
        const u32x4_t t = src[q];
        const int base = q * 4;
        w[(base + 0) / NP2][(base + 0) % NP2] = t.x;
        w[(base + 1) / NP2][(base + 1) % NP2] = t.y;
        w[(base + 2) / NP2][(base + 2) % NP2] = t.z;
        w[(base + 3) / NP2][(base + 3) % NP2] = t.w;
    }
    for (int j = 0; j < kPremixBT; ++j) {
        const int b = b0 + j;
        if (b >= B) break;
        uint32_t ahi[NP2], alo[NP2];
#pragma unroll
        for (int p = 0; p < NP2; ++p) {
            const float a0 = 2 * p < n ? alpha[(long)b * n + 2 * p] : 0.f;
            const float a1 = 2 * p + 1 < n ? alpha[(long)b * n + 2 * p + 1] : 0.f;
            split_alpha(a0, a1, ahi[p], alo[p]);
        }
        float f[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float s = 0.f;
#pragma unroll
            for (int p = 0; p < NP2; ++p) s = dot2(w[c][p], ahi[p], s);
#pragma unroll
            for (int p = 0; p < NP2; ++p) s = dot2(w[c][p], alo[p], s);
            f[c] = s;
        }
        if (a_in)  // input attention: a scale of the mixed kernel's input channel
#pragma unroll
            for (int c = 0; c < 8; ++c) f[c] *= a_in[(long)b * Cin + min(cp + c, Cin - 1)];
        Vec8<uint16_t>::store(wt + ((long)b * nvec + v) * 8, f);
    }
}

// Stand-alone mix on the matrix cores for bf16 banks with more experts
// (kMixMaxN < n <= 16 kMixMfmaMaxG): W_b[w] = sum_i alpha[b,i] E_i[w] is the
// product [examples x experts] . [experts x weights], computed with
// v_mfma_f32_32x32x16_bf16. A workgroup stages the bank's slice of kMixMW
// weights (all experts, zeros past n and past wsize) in LDS with 16-byte
// copies in the natural layout; wave w takes weights [64 w, 64 w + 64) of it
// as two [32 weights x 16 experts] operands per 16 experts, gathered per
// weight from the LDS rows. The attentions of 32 examples, [16 experts x 32
// examples], are split into three bf16 parts (high, middle, low: 24 bits, as
// a float32 significand), so the three exact products summed in fp32 match a
// float32 mix before its one bf16 rounding. With the weights as the result's
// rows, a lane holds 4 consecutive weights of one example's W_b row.
// Workgroup (i, c) takes the 32 examples of chunk c and weight tiles
// i, i + gridDim.x, ... in turn (about two each): the 32 x kMixMW results of
// a tile go through LDS as bf16 rows and leave as 16-byte stores along each
// W_b row while the next tile's expert slice is in flight, so the bank's
// reads overlap the (four times larger) W_b writes.
constexpr int kMixMW = 256;       // weights per workgroup (4 waves x 64)
typedef short s16x4_lds_t __attribute__((ext_vector_type(4)));
constexpr int kMixMfmaMaxG = 4;   // expert groups of 16: n <= 64
constexpr int kMixOutPitch = kMixMW + 8;  // bf16 per staged output row (rows 4 apart on other banks)
constexpr int kMixEx = 32;                // examples per workgroup

template <int NKG>
__global__ __launch_bounds__(256) void mix_mfma_kernel(const float *__restrict__ alpha,
                                                       const uint16_t *__restrict__ experts,
                                                       uint16_t *__restrict__ mixed, int B, int n, long wsize,
                                                       int ntiles) {
    __shared__ __attribute__((aligned(16))) uint16_t s_e[NKG * 16][kMixMW];
    __shared__ __attribute__((aligned(16))) uint16_t s_o[kMixEx][kMixOutPitch];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int bc0 = blockIdx.y * kMixEx;
    // Expert slice of weight tile t: clamped unconditional loads (the
    // masking happens at the LDS store).
    constexpr int kRowVec = kMixMW / 8;            // 16-byte vectors per row
    constexpr int kIt = NKG * 16 * kRowVec / 256;  // expert vectors per thread
    auto load_tile = [&](int t, u32x4_t (&q)[kIt]) {
        const long w0 = (long)t * kMixMW;
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int v = tid + 256 * it;
            const int k = v / kRowVec, c = v - k * kRowVec;
            const long w = min(w0 + 8 * c, wsize - 8);
            q[it] = *reinterpret_cast<const u32x4_t *>(experts + (long)min(k, n - 1) * wsize + w);
        }
    };
    // the first tile's slice loads first, so that its latency overlaps the
    // attention split below
    u32x4_t q[kIt];
    load_tile(blockIdx.x, q);
    // attention operands (B: columns = examples): example bc0 + l32, experts
    // 16 g + 8 lh + (0..7), three parts; the same for every tile
    bf16x8_t ap[3][NKG];
    {
        const int b = bc0 + l32;
        const float *ab = alpha + (long)min(b, B - 1) * n;
#pragma unroll
        for (int g = 0; g < NKG; ++g) {
            uint32_t pw[3][4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint16_t p2[3][2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = 16 * g + 8 * lh + 2 * jj + e;
                    const float a = ab[min(k, n - 1)];
                    float r = (k < n && b < B) ? a : 0.f;
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
            for (int part = 0; part < 3; ++part)
                ap[part][g] = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[part][0], pw[part][1], pw[part][2], pw[part][3]});
        }
    }
    // one tile from the register set qc, the next tile loading into qn
    auto tile_body = [&](int t, const u32x4_t (&qc)[kIt], u32x4_t (&qn)[kIt]) {
        const long w0 = (long)t * kMixMW;
        // stage (masked); the previous tile's operand reads and output
        // copies finished before its second barrier
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int v = tid + 256 * it;
            const int k = v / kRowVec, c = v - k * kRowVec;
            const bool in = k < n && w0 + 8 * c < wsize;
            *reinterpret_cast<u32x4_t *>(&s_e[k][8 * c]) = in ? qc[it] : u32x4_t{0u, 0u, 0u, 0u};
        }
        lds_barrier();
        // the next tile's slice loads during this tile's products and stores
        load_tile(min(t + (int)gridDim.x, ntiles - 1), qn);
        // expert operands (A: rows = weights): experts 16 g + 8 lh + (0..7), weight 64 wave + 32 nt + l32
        // Each half of an operand is one LDS transpose read (ds_read_b64_tr_b16):
        // within a group of 16 lanes, lane i receives element i & 3 of the 8 bytes
        // that lanes 4 j + (i >> 2) (j = 0..3) address, as its element j. Lane
        // s = 4 j + r of the group addresses expert row k0 + 4 h + j at weights
        // wg + 4 r .. wg + 4 r + 3, so lane i gets experts k0 + 4 h + (0..3) of
        // weight wg + i.
        bf16x8_t ef[2][NKG];
        {
            const int si = lane & 15;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int g = 0; g < NKG; ++g) {
                    const int wg = 64 * wave + 32 * nt + 16 * ((lane >> 4) & 1);
                    const int k0 = 16 * g + 8 * lh;
                    s16x4_lds_t h[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4_lds_t *)(&s_e[k0 + 4 * hh + (si >> 2)][wg + 4 * (si & 3)]));
                    const u32x2_t lo = __builtin_bit_cast(u32x2_t, h[0]), hi = __builtin_bit_cast(u32x2_t, h[1]);
                    ef[nt][g] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
                }
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x16_t acc;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
            for (int g = 0; g < NKG; ++g)
#pragma unroll
                for (int part = 2; part >= 0; --part)  // small parts first
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[nt][g], ap[part][g], acc, 0, 0, 0);
            // weights as the rows: D(lane, 4 j + r) = weight 64 wave + 32 nt + 8 j + 4 lh + r,
            // example l32, so a lane's 4 registers of group j are 4
            // consecutive weights of one W_b row (one 8-byte LDS write)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x2_t *>(&s_o[l32][64 * wave + 32 * nt + 8 * j + 4 * lh]) =
                    u32x2_t{pack_bf16x2(acc[4 * j], acc[4 * j + 1]), pack_bf16x2(acc[4 * j + 2], acc[4 * j + 3])};
        }
        lds_barrier();
        // rows out: kMixEx examples x kRowVec vectors
#pragma unroll
        for (int it = 0; it < kMixEx * kRowVec / 256; ++it) {
            const int v = tid + 256 * it;
            const int r = v / kRowVec, c = v - r * kRowVec;
            const int b = bc0 + r;
            const long w = w0 + 8 * c;
            if (b < B && w < wsize)
                *reinterpret_cast<u32x4_t *>(mixed + (long)b * wsize + w) =
                    *reinterpret_cast<const u32x4_t *>(&s_o[r][8 * c]);
        }
    };
    // two register sets in turn, so that each waits for its loads only where
    // it is stored
    u32x4_t q1[kIt];
    for (int t = blockIdx.x; t < ntiles; t += 2 * gridDim.x) {
        tile_body(t, q, q1);
        if (t + (int)gridDim.x < ntiles) tile_body(t + gridDim.x, q1, q);
    }
}

// Premix on the matrix cores for banks whose padded expert count is a
// multiple of 8: as mix_mfma_kernel (persistent over weight tiles, the next
// tile's expert records in flight during the current tile's stores), but the
// experts of each weight come straight from the packed bank (8 consecutive
// experts = 16 bytes of a weight's record, no LDS transpose) and the mixed
// kernels are written in the convolution's layout wt[b][t][o][cp], which has
// the packed bank's weight order.
template <int NKG>
__global__ __launch_bounds__(256) void premix_mfma_kernel(const float *__restrict__ alpha,
                                                          const uint16_t *__restrict__ packed,
                                                          uint16_t *__restrict__ wt, int B, int n, int n_pad,
                                                          long wsize, const float *__restrict__ a_in, int Cin,
                                                          int Cin_pad, int ntiles) {
    __shared__ __attribute__((aligned(16))) uint16_t s_o[kMixEx][kMixOutPitch];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int bc0 = blockIdx.y * kMixEx;
    // expert operands of weight tile t (A: rows = weights): experts
    // 16 g + 8 lh + (0..7) of weight 256 t + 64 wave + 32 nt + l32
    // (raw records; experts past n_pad are masked where the operands are used,
    // so that a wave waits for these loads only there)
    auto load_tile = [&](int t, u32x4_t (&ef)[2][NKG]) {
        const long w0 = (long)t * kMixMW;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const long w = min(w0 + 64 * wave + 32 * nt + l32, wsize - 1);
#pragma unroll
            for (int g = 0; g < NKG; ++g)
                ef[nt][g] = *reinterpret_cast<const u32x4_t *>(packed + w * n_pad + min(16 * g + 8 * lh, n_pad - 8));
        }
    };
    u32x4_t ef[2][NKG];
    load_tile(blockIdx.x, ef);
    // attention operands (B: columns = examples): example bc0 + l32, experts 16 g + 8 lh + (0..7), three parts
    bf16x8_t ap[3][NKG];
    {
        const int b = bc0 + l32;
        const float *ab = alpha + (long)min(b, B - 1) * n;
#pragma unroll
        for (int g = 0; g < NKG; ++g) {
            uint32_t pw[3][4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint16_t p2[3][2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = 16 * g + 8 * lh + 2 * jj + e;
                    const float a = ab[min(k, n - 1)];
                    float r = (k < n && b < B) ? a : 0.f;
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
            for (int part = 0; part < 3; ++part)
                ap[part][g] = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[part][0], pw[part][1], pw[part][2], pw[part][3]});
        }
    }
    constexpr int kRowVec = kMixMW / 8;
    // one tile from the operands efc, the next tile loading into efn
    auto tile_body = [&](int t, const u32x4_t (&efc)[2][NKG], u32x4_t (&efn)[2][NKG]) {
        const long w0 = (long)t * kMixMW;
        f32x16_t acc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nt][i] = 0.f;
#pragma unroll
            for (int g = 0; g < NKG; ++g)
#pragma unroll
                for (int part = 2; part >= 0; --part)
                    acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, 16 * g + 8 * lh < n_pad ? efc[nt][g] : u32x4_t{0u, 0u, 0u, 0u}),
                        ap[part][g], acc[nt], 0, 0, 0);
        }
        // the next tile's expert records load during this tile's stores
        load_tile(min(t + (int)gridDim.x, ntiles - 1), efn);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            // weights as the rows: D(lane, 4 j + r) = weight 64 wave + 32 nt + 8 j + 4 lh + r,
            // example l32 (one 8-byte LDS write per group j)
            if (a_in) {
                // input attention: weight w's input channel is w % Cin_pad (a
                // 32-aligned weight block holds 32 consecutive channels)
                const int cb = (int)((w0 + 64 * wave + 32 * nt) % Cin_pad);
                const float *ai = a_in + (long)min(bc0 + l32, B - 1) * Cin;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[nt][i] *= ai[min(cb + 8 * (i >> 2) + 4 * lh + (i & 3), Cin - 1)];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x2_t *>(&s_o[l32][64 * wave + 32 * nt + 8 * j + 4 * lh]) =
                    u32x2_t{pack_bf16x2(acc[nt][4 * j], acc[nt][4 * j + 1]),
                            pack_bf16x2(acc[nt][4 * j + 2], acc[nt][4 * j + 3])};
        }
        lds_barrier();
#pragma unroll
        for (int it = 0; it < kMixEx * kRowVec / 256; ++it) {
            const int v = tid + 256 * it;
            const int r = v / kRowVec, c = v - r * kRowVec;
            const int b = bc0 + r;
            const long w = w0 + 8 * c;
            if (b < B && w < wsize)
                *reinterpret_cast<u32x4_t *>(wt + (long)b * wsize + w) = *reinterpret_cast<const u32x4_t *>(&s_o[r][8 * c]);
        }
        // the copies read s_o before the next tile writes it
        lds_barrier();
    };
    u32x4_t ef1[2][NKG];
    for (int t = blockIdx.x; t < ntiles; t += 2 * gridDim.x) {
        tile_body(t, ef, ef1);
        if (t + (int)gridDim.x < ntiles) tile_body(t + gridDim.x, ef1, ef);
    }
}

// Workgroups per example chunk for the persistent matrix-core mixes, each
// taking the same number of weight tiles. With at least 4 tile items per CU,
// one workgroup per CU streaming its tiles (the next tile's loads in flight
// during the current tile's stores) ran fastest: at the many-expert layer
// (1152 items) premix 12.7 -> 10.4 us and mix 9.5 -> 9.0 us against 2-3
// workgroups per CU with 2 tiles each, while grids just above one workgroup
// per CU left a second round on a few CUs. Smaller banks keep about
// kMixWorkers workgroups (one or two tiles each).
constexpr int kMixWorkers = 640;
constexpr int kMixCUs = 256;
int mix_workers(int ntiles, int B) {
    const long chunks = (B + kMixEx - 1) / kMixEx;
    const long items = (long)ntiles * chunks;
    const long workers = items >= 4L * kMixCUs ? kMixCUs : kMixWorkers;
    const long per = std::max(1L, (items + workers - 1) / workers);
    return (int)((ntiles + per - 1) / per);
}

}  // namespace

hipError_t launch_mix_natural(const Geom &g, long wsize, const float *alpha, const void *experts,
                              void *mixed, hipStream_t stream) {
    if (wsize % 8 == 0) {
        const long nvec = wsize / 8;
        dim3 grid((unsigned)((nvec + kMixThreads - 1) / kMixThreads),
                  (unsigned)((g.B + kMixBT - 1) / kMixBT));
        if (g.n <= kMixMaxN) {
            auto go = [&](auto kb, auto kf) {
                if (g.bf16)
                    hipLaunchKernelGGL(kb, grid, dim3(kMixThreads), 0, stream, alpha,
                                       static_cast<const uint16_t *>(experts),
                                       static_cast<uint16_t *>(mixed), g.B, g.n, wsize);
                else
                    hipLaunchKernelGGL(kf, grid, dim3(kMixThreads), 0, stream, alpha,
                                       static_cast<const float *>(experts), static_cast<float *>(mixed),
                                       g.B, g.n, wsize);
                return hipGetLastError();
            };
            if (g.n <= 4) return go(mix_natural_all_kernel<uint16_t, 4>, mix_natural_all_kernel<float, 4>);
            return go(mix_natural_all_kernel<uint16_t, 8>, mix_natural_all_kernel<float, 8>);
        }
        if (g.bf16 && g.n > 16 * kMixMfmaMaxG) return launch_mix_wide(g, wsize, alpha,
                                                                      static_cast<const uint16_t *>(experts),
                                                                      static_cast<uint16_t *>(mixed), stream);
        if (g.bf16 && g.n <= 16 * kMixMfmaMaxG) {
            const int ntiles = (int)((wsize + kMixMW - 1) / kMixMW);
            const dim3 mgrid((unsigned)mix_workers(ntiles, g.B), (unsigned)((g.B + kMixEx - 1) / kMixEx));
            auto go = [&](auto kern) {
                hipLaunchKernelGGL(kern, mgrid, dim3(256), 0, stream, alpha,
                                   static_cast<const uint16_t *>(experts), static_cast<uint16_t *>(mixed), g.B,
                                   g.n, wsize, ntiles);
                return hipGetLastError();
            };
            if (g.n <= 16) return go(mix_mfma_kernel<1>);
            if (g.n <= 32) return go(mix_mfma_kernel<2>);
            if (g.n <= 48) return go(mix_mfma_kernel<3>);
            return go(mix_mfma_kernel<4>);
        }
        if (g.bf16)
            hipLaunchKernelGGL(mix_natural_kernel<uint16_t>, grid, dim3(kMixThreads), 0, stream,
                               alpha, static_cast<const uint16_t *>(experts),
                               static_cast<uint16_t *>(mixed), g.B, g.n, wsize);
        else
            hipLaunchKernelGGL(mix_natural_kernel<float>, grid, dim3(kMixThreads), 0, stream,
                               alpha, static_cast<const float *>(experts),
                               static_cast<float *>(mixed), g.B, g.n, wsize);
    } else {
        dim3 grid((unsigned)((wsize + kMixThreads - 1) / kMixThreads),
                  (unsigned)min(g.B, 64));
        if (g.bf16)
            hipLaunchKernelGGL(mix_scalar_kernel<uint16_t>, grid, dim3(kMixThreads), 0, stream,
                               alpha, static_cast<const uint16_t *>(experts),
                               static_cast<uint16_t *>(mixed), g.B, g.n, wsize);
        else
            hipLaunchKernelGGL(mix_scalar_kernel<float>, grid, dim3(kMixThreads), 0, stream,
                               alpha, static_cast<const float *>(experts),
                               static_cast<float *>(mixed), g.B, g.n, wsize);
    }
    return hipGetLastError();
}

size_t packed_experts_bytes(const Geom &g) {
    return (size_t)g.KT * g.Cout * g.Cin_pad * g.n_pad * sizeof(uint16_t);
}

hipError_t launch_pack_experts(const Geom &g, const uint16_t *experts, uint16_t *packed,
                               hipStream_t stream) {
    const int np2 = g.n_pad / 2;
    const long total = (long)g.KT * g.Cout * g.Cin_pad;
    const dim3 grid((unsigned)((total + 255) / 256));
    uint32_t *dst = reinterpret_cast<uint32_t *>(packed);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, experts, dst, g.n, g.Cout, g.Cin, g.KT,
                           g.Cin_pad, np2);
    };
    switch (np2) {
    case 1: go(pack_experts_kernel<1>); break;
    case 2: go(pack_experts_kernel<2>); break;
    case 3: go(pack_experts_kernel<3>); break;
    case 4: go(pack_experts_kernel<4>); break;
    case 5: go(pack_experts_kernel<5>); break;
    case 6: go(pack_experts_kernel<6>); break;
    case 7: go(pack_experts_kernel<7>); break;
    case 8: go(pack_experts_kernel<8>); break;
    default: go(pack_experts_kernel<0>); break;
    }
    return hipGetLastError();
}

size_t premixed_bytes(const Geom &g) {
    return (size_t)g.B * g.KT * g.Cout * g.Cin_pad * sizeof(uint16_t);
}

hipError_t launch_premix(const Geom &g, const float *alpha, const uint16_t *packed,
                         uint16_t *wt, hipStream_t stream, ChanAttn att) {
    const long nvec = (long)g.KT * g.Cout * g.Cin_pad / 8;
    // matrix-core premix when the padded expert records are 16-byte multiples
    if (g.n_pad % 8 == 0 && g.n_pad <= 16 * kMixMfmaMaxG) {
        const long wsize = nvec * 8;
        const int ntiles = (int)((wsize + kMixMW - 1) / kMixMW);
        const dim3 mgrid((unsigned)mix_workers(ntiles, g.B), (unsigned)((g.B + kMixEx - 1) / kMixEx));
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, mgrid, dim3(256), 0, stream, alpha, packed, wt, g.B, g.n, g.n_pad, wsize,
                               att.in, g.Cin, g.Cin_pad, ntiles);
            return hipGetLastError();
        };
        const int nkg = (g.n_pad + 15) / 16;
        if (nkg == 1) return go(premix_mfma_kernel<1>);
        if (nkg == 2) return go(premix_mfma_kernel<2>);
        if (nkg == 3) return go(premix_mfma_kernel<3>);
        return go(premix_mfma_kernel<4>);
    }
    dim3 grid((unsigned)((nvec + 255) / 256), (unsigned)((g.B + kPremixBT - 1) / kPremixBT));
    const uint32_t *pk = reinterpret_cast<const uint32_t *>(packed);
    switch (g.n_pad / 2) {
    case 1: hipLaunchKernelGGL(premix_kernel<1>, grid, dim3(256), 0, stream, alpha, pk, wt, g.B, g.n, nvec, att.in, g.Cin, g.Cin_pad); break;
    case 2: hipLaunchKernelGGL(premix_kernel<2>, grid, dim3(256), 0, stream, alpha, pk, wt, g.B, g.n, nvec, att.in, g.Cin, g.Cin_pad); break;
    case 3: hipLaunchKernelGGL(premix_kernel<3>, grid, dim3(256), 0, stream, alpha, pk, wt, g.B, g.n, nvec, att.in, g.Cin, g.Cin_pad); break;
    case 4: hipLaunchKernelGGL(premix_kernel<4>, grid, dim3(256), 0, stream, alpha, pk, wt, g.B, g.n, nvec, att.in, g.Cin, g.Cin_pad); break;
    case 5: hipLaunchKernelGGL(premix_kernel<5>, grid, dim3(256), 0, stream, alpha, pk, wt, g.B, g.n, nvec, att.in, g.Cin, g.Cin_pad); break;
    case 6: hipLaunchKernelGGL(premix_kernel<6>, grid, dim3(256), 0, stream, alpha, pk, wt, g.B, g.n, nvec, att.in, g.Cin, g.Cin_pad); break;
    case 7: hipLaunchKernelGGL(premix_kernel<7>, grid, dim3(256), 0, stream, alpha, pk, wt, g.B, g.n, nvec, att.in, g.Cin, g.Cin_pad); break;
    case 8: hipLaunchKernelGGL(premix_kernel<8>, grid, dim3(256), 0, stream, alpha, pk, wt, g.B, g.n, nvec, att.in, g.Cin, g.Cin_pad); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dynconv
