// mfma_kernel.h -- fused deformable sampling + MFMA GEMM for groups == 1:
// the kernel templates, included by the translation units that instantiate
// them (k_mfma_*.hip) and by the planner (k_mfma.hip).
//
// The contraction out[b, co, l] = bias[co] + sum_r W[co, r] S[r, (b, l)] is a
// GEMM with M = C_out, N = B*L_out and reduction r = ci*K + k over the
// weight viewed as [C_out, C_in*K] (conv1d operator page, Description; the
// article's Step 3 weighted summation).  S is the deformable sample matrix
// (the article's Step 2); it lives only as a small double-buffered tile in
// LDS, never in HBM.
//
// Workgroup: 8 waves in two roles (warp specialisation), one per SIMD each:
//   * 4 MFMA waves in a 2 x 2 grid over the BM x BN = 256 x 128 output
//     tile, each owning 128 rows x 64 columns; they read operand fragments
//     from LDS and issue MFMAs, and stage the next chunk's weight tile,
//     whose load latency hides under their MFMAs.
//   * 4 sampler waves.  They stage the zero-padded x windows from HBM into
//     LDS and compute the sample tile of the next reduction chunk.
// The hardware interleaves the two roles on every SIMD: MFMAs of one wave
// run while the other wave's VALU, LDS and memory instructions issue.  The
// reduction runs in chunks of BK = 32 rows; in iteration c the MFMA waves
// consume chunk c and stage chunk c+1's weight tile while the sampler waves
// produce chunk c+1's sample tile and stage windows two chunks ahead; one
// barrier per chunk.  Sample tiles, weight tiles and windows are all
// double-buffered.
//
// Position table (built once per workgroup): for each (offset group, tap,
// column) the left neighbour i0 and the fraction f of the sample position
// (dc1d page, Demo notebook: linear interpolation between neighbours), and
// the mask value when there is one (dc1d page, Modulation; applied as a
// plain multiply, so an all-ones mask gives the no-mask bits).
//
// Windows: the columns of a tile fall into at most NSEG batch segments; for
// each segment the smallest and largest left neighbour over the tile give a
// window [lo, hi + 1] of the input row, staged per channel with zeros
// outside [0, L_in) (torchvision issue demo: samples off the ends read
// zero).  Interpolation is then one paired LDS read and two FMAs, with no
// bounds checks.  When the offsets spread wider than the window capacity, or
// the tile crosses too many batches, the workgroup gathers x from global
// memory instead (same arithmetic, bounds-checked loads).
//
// Columns past the end of N and reduction rows past Kred are computed on
// clamped, finite inputs and never stored (an MFMA output column depends
// only on its own B column, and the weight rows past Kred are zero).
//
// Split reduction: when there are too few output tiles to fill the GPU, the
// reduction range is split over several workgroups.  Each writes its fp32
// partial tile into the workspace; a second, small kernel on the same stream
// adds the partials in split order (so the result is deterministic), adds
// the bias and stores the output.  Kernel order on the stream is the only
// synchronisation, so the workspace needs no initialisation.
#pragma once

#include "dc1d_internal.h"

#include <limits.h>

#include <algorithm>
#include <type_traits>

namespace dc1d {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef int i4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int NWM = 4;          // MFMA waves
constexpr int NTM = 64 * NWM;   // MFMA threads
constexpr int NTS = 256;        // sampler threads (4 waves)
constexpr int NTT = NTM + NTS;  // threads per workgroup
constexpr int BK = 32;          // reduction rows per chunk
constexpr int NSEG = 4;         // batch segments a windowed tile may span

struct Pos {
    int j;    // windowed: index into the tile's window row; global: left neighbour clamped to [-2, L_in]
    float f;  // interpolation fraction
};

struct MfmaArgs {
    Params p;
    FastDiv fd_K, fd_cpo, fd_Lout;
    int tiles_m, tiles_n, splits, chunks;
    int64_t N;
    float *partials;  // split partial tiles [splits][tiles][BM*BN], or null
    int wt_max;       // window capacity per channel row (elements); 0: always gather
    int vec_w;        // weight rows can be read in aligned 16-byte words
    int vec_x;        // channel-block order: x rows can be staged in aligned 16-byte words
                      // (L_in a multiple of the word, x aligned); windows then start on a word
    int off_mask, off_w, off_s, off_x;  // byte offsets of the LDS regions
    // channel-block order only: the reduction runs over ncb blocks of CB
    // input channels (outer) and nkb groups of 32/CB taps (inner); wb holds
    // the weights rearranged into [nkb][C_out][ncb][32] chunk rows
    const void *wb;
    int ncb, nkb;
    FastDiv fd_nkb;
    // plain GEMM only (k_gemm): B element (k, n = b*L_out + j) sits at
    // x[b*bbatch + j + k*brow]
    int64_t brow, bbatch;
};

__device__ __forceinline__ int remap_xcd(int u, int U) {
    // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
    // that consecutive unit ids (which share a weight slice) run on one XCD
    // and hit its L2.
    const int q = U >> 3, r = U & 7, xcd = u & 7, loc = u >> 3;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + loc;
}

// ---- per-dtype traits ---------------------------------------------------------
//
// MFMA lane (i = lane % 32, h = lane / 32) holds, per chunk, the 16 weights
// W[m0 + 32*mb + i][r0 + 16h .. r0 + 16h + 15] of each 32-row block and the 16
// samples S[r0 + 16h .. + 15][column] of each 32-column block.  fp32 pairs
// them in 16 v_mfma_f32_32x32x2_f32 (element j of both halves per
// instruction); bf16 in 2 v_mfma_f32_32x32x16_bf16 (elements 8s .. 8s+7).
//
// The weight tile in LDS is [BM][BK] without padding; its 16-byte words are
// XOR-swizzled by row so that lanes reading one word each of consecutive
// rows hit distinct banks.  The sample tile is [BN][BK + pad]: a lane's 16
// samples are contiguous, and the pad spreads consecutive columns over the
// banks.

struct TrF32 {
    using D = F32;
    using T = float;
    static constexpr int MB = 4, NB = 2;  // per MFMA wave: 128 rows x 64 columns
    static constexpr int WPR = BK / 4;    // 16-byte words per weight-tile row (8)
    static constexpr int SLD = BK + 4;    // sample-tile row (elements)
    struct Frag { float v[16]; };
    static __device__ __forceinline__ int swz(int row, int word) { return word ^ (row & 7); }
    static __device__ __forceinline__ void lds_a(const float *tile, int row, int h, Frag &a) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f4 t = *(const f4 *)(tile + row * BK + 4 * swz(row, 4 * h + q));
            a.v[4 * q] = t[0]; a.v[4 * q + 1] = t[1]; a.v[4 * q + 2] = t[2]; a.v[4 * q + 3] = t[3];
        }
    }
    static __device__ __forceinline__ void lds_b(const float *src, Frag &b) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f4 t = ((const f4 *)src)[q];
            b.v[4 * q] = t[0]; b.v[4 * q + 1] = t[1]; b.v[4 * q + 2] = t[2]; b.v[4 * q + 3] = t[3];
        }
    }
    static __device__ __forceinline__ void store_b(float *dst, const float (&v)[16]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) ((f4 *)dst)[q] = f4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    }
    static __device__ __forceinline__ void mma(const Frag &a, const Frag &b, f16v &acc) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void st1(float *dst, float v) { *dst = v; }
};

// fp32 with half the rows per MFMA wave (a 128 x 128 tile): the packed
// layer's head GEMM, whose short reduction makes the tile's write-out, not
// its MFMAs, the long phase; the smaller tile lets two workgroups share a CU.
struct TrF32H : TrF32 {
    static constexpr int MB = 2;
};

// Two floats -> two bfloat16 (round to nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf2 r = __builtin_convertvector(f2{lo, hi}, bf2);
    return __builtin_bit_cast(uint32_t, r);
}

struct TrBF16 {
    using D = BF16;
    using T = uint16_t;
    static constexpr int MB = 4, NB = 2;  // per MFMA wave: 128 rows x 64 columns
    static constexpr int WPR = BK / 8;    // 4
    static constexpr int SLD = BK + 8;
    struct Frag { u4 v[2]; };
    static __device__ __forceinline__ int swz(int row, int word) { return word ^ ((row >> 1) & 3); }
    static __device__ __forceinline__ void lds_a(const uint16_t *tile, int row, int h, Frag &a) {
        a.v[0] = *(const u4 *)(tile + row * BK + 8 * swz(row, 2 * h));
        a.v[1] = *(const u4 *)(tile + row * BK + 8 * swz(row, 2 * h + 1));
    }
    static __device__ __forceinline__ void lds_b(const uint16_t *src, Frag &b) {
        b.v[0] = ((const u4 *)src)[0];
        b.v[1] = ((const u4 *)src)[1];
    }
    static __device__ __forceinline__ void store_b(uint16_t *dst, const float (&v)[16]) {
        ((u4 *)dst)[0] = u4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7])};
        ((u4 *)dst)[1] = u4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                            pack_bf16x2(v[14], v[15])};
    }
    static __device__ __forceinline__ void mma(const Frag &a, const Frag &b, f16v &acc) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8, a.v[s]),
                                                          __builtin_bit_cast(bf8, b.v[s]), acc, 0, 0, 0);
    }
    // one output element, rounded to nearest even by the conversion instruction
    static __device__ __forceinline__ void st1(uint16_t *dst, float v) {
        *dst = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
    }
};

template <class Tr>
struct Geo {
    // the MFMA waves form a WM x WN grid over the BM x BN tile (BM = 256,
    // BN = 128); each owns 32*MB rows and 32*NB columns, which balances the
    // weight and sample fragments it reads from LDS per chunk
    static constexpr int WM = 2, WN = NWM / WM;
    static constexpr int BM = 32 * Tr::MB * WM;
    static constexpr int BN = 32 * Tr::NB * WN;
    static __device__ __forceinline__ int row0(int wv) { return 32 * Tr::MB * (wv / WN); }
    static __device__ __forceinline__ int col0(int wv) { return 32 * Tr::NB * (wv % WN); }
    static constexpr int WV = BM * Tr::WPR / NTM;  // 16-byte weight words per MFMA thread per chunk
};

// Shared per-workgroup state the two roles read.
struct Tile {
    int m0, tm, tn, sp, c_begin, c_end;
    int64_t n0;
    bool win;
    int WT, nseg, b_first;
};

// GEMMs whose rows are the packed layer's generator head channels store
// their output offsets-shaped.  OUT 1: rows g*K + k (g < G) go to p.out
// [B][G][L_out][K].  OUT 2: the offset and mask heads stacked, rows
// [0, G*K) as OUT 1 and rows G*K + g*K + k to the mask tensor (p.mask, same
// shape) through the logistic sigmoid.  OUT 0 is the convolution's
// [B][M][L_out].
// (the reciprocal instruction, within an ulp, instead of a full division:
// the write-out of the mask head is arithmetic-bound otherwise)
__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Destination row (b, g) of the run of L_out*K elements that holds head
// group gg (offset group gg, or mask group gg - G), and whether it is a
// mask group.
template <class Tr, int OUT>
__device__ __forceinline__ typename Tr::T *head_run(const Params &p, int b, int gg, bool &is_mask) {
    using T = typename Tr::T;
    is_mask = OUT == 2 && gg >= p.G;
    T *base = is_mask ? (T *)p.mask : (T *)p.out;
    const int g = is_mask ? gg - p.G : gg;
    return base + ((int64_t)b * p.G + g) * p.L_out * p.K;
}

// One element, stored where it belongs (the split-K reduction's path).
template <class Tr, int OUT>
__device__ __forceinline__ void store_head(const Params &p, int b, int l, int row, float v) {
    static_assert(OUT == 1 || OUT == 2, "head layouts only");
    const int gg = row / p.K, k = row - gg * p.K;
    bool is_mask;
    typename Tr::T *run = head_run<Tr, OUT>(p, b, gg, is_mask);
    Tr::D::st(run, (int64_t)l * p.K + k, is_mask ? sigmoid(v) : v);
}

// The direct path stages the finished tile (without bias) in LDS as
// [BM][BN + 1] floats, followed by the tile rows' biases, and then all the
// workgroup's threads write it out in destination order: for each offset
// group g the tile covers, its columns l0 .. l0+BN-1 times its K taps are one
// contiguous run of the output (per batch), so consecutive threads store
// consecutive addresses.
constexpr int kHeadLd = 128 + 1;  // staging row pitch (floats) for BN = 128

// ---- the MFMA role -------------------------------------------------------------
//
// Weight layout WL: 0: the weight viewed as [C_out][Kred], chunk c at
// reduction rows 32c .. 32c+31; 1: the rearranged copy a.wb (channel-block
// order, rows of 32 contiguous elements, always in bounds); 2: channel-block
// order read straight from the weight when a chunk row's four taps of one
// channel are one aligned 16-byte word (fp32, 32/CB == 4, K % 4 == 0).
template <class Tr, int WL, int OUT = 0>
__device__ __forceinline__ void mfma_role(const MfmaArgs &a, const Tile &tl, typename Tr::T *s_w,
                                          const typename Tr::T *s_S) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    using Frag = typename Tr::Frag;
    constexpr int MB = Tr::MB, NB = Tr::NB, BM = Geo<Tr>::BM, BN = Geo<Tr>::BN, SLD = Tr::SLD;
    constexpr int WPR = Tr::WPR, WV = Geo<Tr>::WV;
    constexpr int EPW = 16 / sizeof(T);  // elements per 16-byte word
    static_assert(WV * NTM == BM * WPR, "weight tile split");
    static_assert(WL != 2 || EPW == 4, "direct channel-block weights are fp32 words of four taps");
    const Params &p = a.p;
    const int t = threadIdx.x;
    const int wv = t / 64, lane = t % 64, li = lane % 32, lh = lane / 32;
    const int row0 = Geo<Tr>::row0(wv), col0 = Geo<Tr>::col0(wv);
    const int M = p.C_out, Kred = p.Kred, C_in = p.C_in;
    const T *__restrict__ w = (const T *)p.w;
    const bool m_full = tl.m0 + BM <= M;  // no rows past C_out in this tile

    // The weight tile of chunk c+1 is written to LDS after chunk c's MFMAs.
    // With two register sets (W2: the bf16 tile's 4 words per thread) its
    // loads were issued an iteration earlier, so their latency hides under
    // two chunks of MFMAs; fp32 tiles (8 words) load at the start of
    // iteration c.  Loads never wait on a bounds test: words outside the
    // matrix load a clamped address and are zeroed in commit_w.
    constexpr bool W2 = WV <= 4;
    // Word v of this thread is row prow + RV*v, 16-byte word ppart of the
    // row, for every chunk; in tiles wholly inside C_out the loads are a
    // per-thread base plus a wave-uniform stride (no clamps in the loop).
    constexpr int RV = NTM / WPR;  // rows between one thread's words
    static_assert(RV % 8 == 0, "the word swizzle is the same for all of a thread's rows");
    const int prow = t / WPR, ppart = t % WPR;
    const T *wfast = w;
    int64_t vstride = 0;
    if (WL == 1) {
        wfast = (const T *)a.wb + (int64_t)(tl.m0 + prow) * a.ncb * BK + ppart * EPW;
        vstride = (int64_t)RV * a.ncb * BK;
    } else if (WL == 2) {
        wfast = w + (int64_t)(tl.m0 + prow) * C_in * p.K;
        vstride = (int64_t)RV * C_in * p.K;
    }
    auto fetch_w = [&](int cw, u4 (&wreg)[WV]) {
        const int r0 = cw * BK;
        if ((WL == 1 || WL == 2) && m_full) {
            const int cb = (int)fdiv((uint32_t)cw, a.fd_nkb), kb = cw - cb * a.nkb;
            const T *base = WL == 1 ? wfast + ((int64_t)kb * M * a.ncb + cb) * BK
                                    : wfast + (int64_t)min(cb * (BK / 4) + ppart, C_in - 1) * p.K + 4 * kb;
#pragma unroll
            for (int v = 0; v < WV; ++v) wreg[v] = *(const u4 *)(base + v * vstride);
        } else if (WL == 1) {
            const int cb = (int)fdiv((uint32_t)cw, a.fd_nkb), kb = cw - cb * a.nkb;
            const T *wb = (const T *)a.wb + ((int64_t)kb * M * a.ncb + cb) * BK;
#pragma unroll
            for (int v = 0; v < WV; ++v) {
                const int e = t + NTM * v;
                const int row = e / WPR, part = e % WPR;
                const int m = min(tl.m0 + row, M - 1);
                wreg[v] = *(const u4 *)(wb + (int64_t)m * a.ncb * BK + part * EPW);
            }
        } else if (WL == 2) {
            const int cb = (int)fdiv((uint32_t)cw, a.fd_nkb), kb = cw - cb * a.nkb;
            // word `part` of a row: channel CB*cb + part, taps 4kb .. 4kb+3
            const T *wk = w + 4 * kb;
#pragma unroll
            for (int v = 0; v < WV; ++v) {
                const int e = t + NTM * v;
                const int row = e / WPR, part = e % WPR;
                const int m = min(tl.m0 + row, M - 1);
                const int ci = min(cb * (BK / 4) + part, C_in - 1);
                wreg[v] = *(const u4 *)(wk + ((int64_t)m * C_in + ci) * p.K);
            }
        } else if (a.vec_w) {
            // Kred is a multiple of the word size: a word is wholly inside or outside
#pragma unroll
            for (int v = 0; v < WV; ++v) {
                const int e = t + NTM * v;
                const int row = e / WPR, part = e % WPR;
                const int m = tl.m0 + row, rb = r0 + part * EPW;
                const bool ok = m < M && rb < Kred;
                wreg[v] = *(const u4 *)(w + (ok ? (int64_t)m * Kred + rb : 0));
            }
        } else {
#pragma unroll
            for (int v = 0; v < WV; ++v) {
                const int e = t + NTM * v;
                const int row = e / WPR, part = e % WPR;
                const int m = tl.m0 + row, rb = r0 + part * EPW;
                const T *src = w + (int64_t)(m < M ? m : M - 1) * Kred;
                T tmp[EPW];
#pragma unroll
                for (int z = 0; z < EPW; ++z) tmp[z] = (m < M && rb + z < Kred) ? src[min(rb + z, Kred - 1)] : (T)0;
                wreg[v] = __builtin_bit_cast(u4, tmp);
            }
        }
    };
    // registers -> LDS (swizzled words).  Tiles wholly inside the matrix
    // store without tests.
    T *const wdst = s_w + prow * BK + EPW * Tr::swz(prow, ppart);  // word 0 of this thread, buffer 0
    auto commit_w = [&](int cw, const u4 (&wreg)[WV]) {
        T *dw = s_w + (cw & 1) * BM * BK;
        const int r0 = cw * BK;
        const int cb = WL == 2 ? (int)fdiv((uint32_t)cw, a.fd_nkb) : 0;
        const bool full = m_full && (WL == 1 || (WL == 2 ? (cb + 1) * (BK / 4) <= C_in : r0 + BK <= Kred));
        if (full) {
            T *d0 = wdst + (cw & 1) * BM * BK;
#pragma unroll
            for (int v = 0; v < WV; ++v) *(u4 *)(d0 + v * RV * BK) = wreg[v];
        } else {
#pragma unroll
            for (int v = 0; v < WV; ++v) {
                const int e = t + NTM * v;
                const int row = e / WPR, part = e % WPR;
                const bool ok = tl.m0 + row < M && (WL == 1 || (WL == 2 ? cb * (BK / 4) + part < C_in
                                                                         : r0 + part * EPW < Kred));
                *(u4 *)(dw + row * BK + EPW * Tr::swz(row, part)) = ok ? wreg[v] : u4{0, 0, 0, 0};
            }
        }
    };

    f16v acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;
    // issue priority over the other role's wave on the same SIMD, so that
    // the matrix unit is fed first and the other role fills the gaps
    __builtin_amdgcn_s_setprio(2);

    u4 wA[WV], wB[WV];
    const int c_last = max(tl.c_end - 1, 0);
    if (tl.c_begin < tl.c_end) {
        fetch_w(tl.c_begin, wA);
        commit_w(tl.c_begin, wA);
    }
    if (W2) fetch_w(min(tl.c_begin + 1, c_last), wA);
    // prologue barriers shared with the sampler role: staging done, first sample tile done
    __syncthreads();
    __syncthreads();
    // Chunk c: `cur` holds (W2) or receives chunk c+1's weights, `nxt`
    // receives chunk c+2's (W2).  The loads are issued after the first row
    // block's MFMAs and the LDS commit before the last block's, so that both
    // run while the matrix unit is busy (scheduling barriers keep them
    // there).  Both happen on every step, past the range on the last chunk's
    // words (unused; the buffer written is not read again): with branches
    // around them the compiler's wait for `cur` also waited for the loads
    // just issued.
    // (the plain fp32 GEMM's single register set keeps the loads at the top
    // of the step and the commit at its end: held across the MFMAs it spills)
    constexpr bool MID = WL != 0 || W2;
    auto step = [&](int c, u4 (&cur)[WV], u4 (&nxt)[WV]) {
        if constexpr (!MID) {
            if (c + 1 < tl.c_end) fetch_w(c + 1, cur);
        }
        const T *tile = s_w + (c & 1) * BM * BK;
        const T *st = s_S + (c & 1) * BN * SLD;
        Frag bf[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) Tr::lds_b(st + (col0 + 32 * nb + li) * SLD + 16 * lh, bf[nb]);
        // weight fragments double-buffered: block mb+1's reads are in flight
        // while block mb's MFMAs run
        Frag af[2];
        Tr::lds_a(tile, row0 + li, lh, af[0]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb + 1 < MB) Tr::lds_a(tile, row0 + 32 * (mb + 1) + li, lh, af[(mb + 1) & 1]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Tr::mma(af[mb & 1], bf[nb], acc[mb][nb]);
            if (MID && mb == 0) {
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (W2)
                    fetch_w(min(c + 2, c_last), nxt);
                else
                    fetch_w(min(c + 1, c_last), cur);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (MID && (mb == MB - 2 || (MB == 1 && mb == 0))) {
                __builtin_amdgcn_sched_barrier(0);
                commit_w(c + 1, cur);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (!MID) {
            if (c + 1 < tl.c_end) commit_w(c + 1, cur);
        }
        __syncthreads();
    };
    if constexpr (W2) {
        for (int c = tl.c_begin; c < tl.c_end; c += 2) {
            step(c, wA, wB);
            if (c + 1 < tl.c_end) step(c + 1, wB, wA);
        }
    } else {
        for (int c = tl.c_begin; c < tl.c_end; ++c) step(c, wA, wA);
    }

    // ---- epilogue
    const T *__restrict__ bias = (const T *)p.bias;
    T *__restrict__ out = (T *)p.out;
    const int L_out = p.L_out;
    constexpr int NQ = MB * NB * 4;  // f4 groups per thread
    if (a.splits > 1) {
        // fp32 partial tile, in this thread's register order; summed over the
        // splits in split order by k_split_reduce
        const int tile = tl.tm * a.tiles_n + tl.tn;
        f4 *part = (f4 *)(a.partials + ((int64_t)tl.sp * a.tiles_m * a.tiles_n + tile) * (BM * BN));
#pragma unroll
        for (int q4 = 0; q4 < NQ; ++q4) {
            const int mb = q4 / (NB * 4), nb = (q4 / 4) % NB, qq = (q4 & 3) * 4;
            part[q4 * NTM + t] = f4{acc[mb][nb][qq], acc[mb][nb][qq + 1], acc[mb][nb][qq + 2], acc[mb][nb][qq + 3]};
        }
        return;
    }
    if constexpr (OUT != 0) {
        // stage for the workgroup-wide write-out (every LDS read of the
        // main loop is behind its last barrier)
        static_assert(BN + 1 == kHeadLd, "staging pitch");
        float *s_out = (float *)s_w;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int rl = row0 + 32 * mb + 8 * (q >> 2) + 4 * lh + (q & 3);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) s_out[rl * kHeadLd + col0 + 32 * nb + li] = acc[mb][nb][q];
            }
        return;
    }
    // The bias of this thread's rows is loaded before the first store: a
    // wait for a load also waits for every store issued before it, so bias
    // loads between the stores would serialise them on the write latency.
    float bq[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = tl.m0 + row0 + 32 * mb + 8 * (q >> 2) + 4 * lh + (q & 3);
            bq[mb][q] = bias ? D::ld(bias, min(row, M - 1)) : 0.0f;
        }
    if (L_out % EPW == 0 && ((uintptr_t)out & 15) == 0) {
        // Whole 16-byte words of output rows.  A word never straddles a
        // batch (L_out is a multiple of the word) nor the end of N (nor is
        // N).  The wave stages each 32-row block of its tile (bias added) in
        // the LDS that the main loop used, then every lane writes EPW
        // consecutive columns of one row: 32 / RPI stores per block instead
        // of one per element.
        constexpr int WC = 32 * NB, PITCH = WC + 8;  // staging row (floats): rows 4 apart land 32 banks apart
        constexpr int LPR = WC / EPW, RPI = 64 / LPR;  // lanes per row, rows per store
        static_assert(NWM * 32 * PITCH * 4 <= 2 * BM * BK * sizeof(T) + 2 * BN * SLD * sizeof(T),
                      "staging fits in the weight and sample tiles");
        float *stg = (float *)s_w + wv * 32 * PITCH;
        const int rl = lane / LPR, cl = (lane % LPR) * EPW;
        const int col = (int)tl.n0 + col0 + cl;
        const bool col_ok = col < a.N;
        const int b = (int)fdiv((uint32_t)(col_ok ? col : 0), a.fd_Lout);
        T *ob = out + (int64_t)b * M * L_out + (col - b * L_out);
        // LDS is shared by the wave's lanes only here; fences order each
        // lane's accesses around the exchange
        auto wave_sync = [] {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            wave_sync();  // the previous block's reads are done
#pragma unroll
            for (int q = 0; q < 16; ++q)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    stg[(8 * (q >> 2) + 4 * lh + (q & 3)) * PITCH + 32 * nb + li] = acc[mb][nb][q] + bq[mb][q];
            wave_sync();
#pragma unroll
            for (int it = 0; it < 32 / RPI; ++it) {
                const int r = it * RPI + rl;
                const int row = tl.m0 + row0 + 32 * mb + r;
                const float *src = stg + r * PITCH + cl;
                u4 word;
                if constexpr (EPW == 4) {
                    word = __builtin_bit_cast(u4, *(const f4 *)src);
                } else {
                    const f4 v0 = *(const f4 *)src, v1 = *(const f4 *)(src + 4);
                    word = u4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v1[0], v1[1]),
                              pack_bf16x2(v1[2], v1[3])};
                }
                if (col_ok && (m_full || row < M)) *(u4 *)(ob + (int64_t)row * L_out) = word;
            }
        }
        return;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int col = (int)tl.n0 + col0 + 32 * nb + li;
        if (col >= a.N) continue;
        const int b = (int)fdiv((uint32_t)col, a.fd_Lout);
        const int l = col - b * L_out;
        T *ob = out + (int64_t)b * M * L_out + l;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = tl.m0 + row0 + 32 * mb + 8 * (q >> 2) + 4 * lh + (q & 3);
                if (m_full || row < M) Tr::st1(ob + (int64_t)row * L_out, acc[mb][nb][q] + bq[mb][q]);
            }
    }
}

// The write-out of a staged head tile (all threads of the workgroup; see
// kHeadLd).  Thread t takes the pairs j = t, t + NTT, ... of (column c, tap
// k) = (j / K, j % K) and, for each offset group g the tile covers, the
// element at row g*K + k: consecutive threads hold consecutive addresses of
// one group's run.  Bias and the head's sigmoid are applied here.
template <class Tr, int OUT>
__device__ __forceinline__ void head_writeout(const MfmaArgs &a, const Tile &tl, const float *s_out,
                                              const float *s_bias) {
    constexpr int BM = Geo<Tr>::BM, BN = Geo<Tr>::BN;
    const Params &p = a.p;
    const int K = p.K, M = p.C_out, L_out = p.L_out;
    const int rows = min(BM, M - tl.m0);
    const int ncol = (int)min((int64_t)BN, a.N - tl.n0);
    const int g_first = (int)fdiv((uint32_t)tl.m0, a.fd_K);
    const int ng = (int)fdiv((uint32_t)(tl.m0 + rows - 1), a.fd_K) - g_first + 1;
    if constexpr (sizeof(typename Tr::T) == 4) {
        // In 16-byte words when the tile's columns lie in one batch and every
        // run (l0 .. l0+ncol-1 times K taps of one group) starts on a word:
        // the (group, word) pairs spread over all the workgroup's threads.  A
        // word holding taps of rows outside this tile (the first or last
        // group, when BM is not a multiple of K) stores only its own elements.
        const int b0 = (int)fdiv((uint32_t)tl.n0, a.fd_Lout);
        const int l0 = (int)(tl.n0 - (int64_t)b0 * L_out);
        const bool aligned = ((uintptr_t)p.out & 15) == 0 && (OUT != 2 || ((uintptr_t)p.mask & 15) == 0);
        if (aligned && l0 + ncol <= L_out && ((int64_t)L_out * K) % 4 == 0 && ((int64_t)l0 * K) % 4 == 0 &&
            (ncol * K) % 4 == 0) {
            const int wpr = ncol * K / 4;  // words per run
            for (int idx = threadIdx.x; idx < ng * wpr; idx += NTT) {
                const int gi = idx / wpr, e0 = 4 * (idx - gi * wpr);
                const int g = g_first + gi;
                int c = (int)fdiv((uint32_t)e0, a.fd_K), k = e0 - c * K;
                bool is_mask;
                float *dst = (float *)head_run<Tr, OUT>(p, b0, g, is_mask) + ((int64_t)l0 * K + e0);
                float v[4];
                bool own[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rl = g * K + k - tl.m0;
                    own[q] = rl >= 0 && rl < rows;
                    v[q] = own[q] ? s_out[rl * kHeadLd + c] + s_bias[rl] : 0.0f;
                    if (is_mask) v[q] = sigmoid(v[q]);
                    if (++k == K) {
                        k = 0;
                        ++c;
                    }
                }
                if (own[0] && own[1] && own[2] && own[3]) {
                    *(f4 *)dst = f4{v[0], v[1], v[2], v[3]};
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (own[q]) dst[q] = v[q];
                }
            }
            return;
        }
    }
    for (int j = threadIdx.x; j < BN * K; j += NTT) {
        const int c = (int)fdiv((uint32_t)j, a.fd_K);
        const int k = j - c * K;
        if (c >= ncol) continue;
        const int n = (int)tl.n0 + c;
        const int b = (int)fdiv((uint32_t)n, a.fd_Lout);
        const int64_t at = (int64_t)(n - b * L_out) * K + k;  // (l, k) inside a run
        int rl = g_first * K + k - tl.m0;
#pragma unroll 4
        for (int gi = 0; gi < ng; ++gi, rl += K) {
            if (rl < 0 || rl >= rows) continue;
            bool is_mask;
            typename Tr::T *run = head_run<Tr, OUT>(p, b, g_first + gi, is_mask);
            const float v = s_out[rl * kHeadLd + c] + s_bias[rl];
            Tr::D::st(run, at, is_mask ? sigmoid(v) : v);
        }
    }
}

// ---- the sampler role ------------------------------------------------------------
//
// Sampler wave sw computes the samples of reduction rows r0 + 16*h .. + 15
// (h = sw & 1) for 64 columns (64*(sw >> 1) + lane), so that a row's
// position-table row and window row are the same for the whole wave and are
// computed in scalar registers.  Windows are double-buffered and staged
// through registers: the loads of chunk c+3 are issued in iteration c and
// written to LDS at the start of iteration c+1, a full iteration later.
//
// NCH channel rows of WTM = SLOT * NTS elements each are staged per chunk
// (compile-time counts, so the staging code is straight-line): thread ts
// owns positions ts + NTS*q (q < SLOT) of every row.
template <class Tr, bool MASK, bool WIN, int NCH, int SLOT>
__device__ __forceinline__ void sampler_role(const MfmaArgs &a, const Tile &tl, const Pos *s_tab,
                                             const float *s_m, typename Tr::T *s_S, float *s_x,
                                             const int *s_lo, const int *s_base) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    constexpr int BN = Geo<Tr>::BN, SLD = Tr::SLD;
    constexpr int WTM = SLOT * NTS;   // window row length (elements)
    constexpr int XBUF = NCH * WTM;  // floats per window buffer
    static_assert(BN == 128, "two sampler waves per 64 columns");
    const Params &p = a.p;
    const int ts = threadIdx.x - NTM;  // 0 .. NTS-1
    const int lane = ts % 64;
    const int sw = __builtin_amdgcn_readfirstlane(ts / 64);
    const int h = sw & 1;
    const int col = 64 * (sw >> 1) + lane;
    const int Kred = p.Kred, K = p.K, L_in = p.L_in, L_out = p.L_out, C_in = p.C_in, cpo = p.cpo;
    const T *__restrict__ x = (const T *)p.x;
    const int WT = tl.WT;

    // Per slot: the x offset of its window position in channel 0 (clamped to
    // a real element) and whether the position lies inside [0, L_in).  Loads
    // are unconditional; positions outside are zeroed when committed.
    int64_t xoff[SLOT];
    bool xval[SLOT];
#pragma unroll
    for (int q = 0; q < SLOT; ++q) {
        const int jj = ts + NTS * q;
        int64_t o = 0;
        bool ok = false;
        if (WIN && jj < WT) {
            int sg = 0;
            while (sg + 1 < tl.nseg && s_base[sg + 1] <= jj) ++sg;
            const int pos = s_lo[sg] + (jj - s_base[sg]);
            ok = pos >= 0 && pos < L_in;
            o = (int64_t)(tl.b_first + sg) * C_in * L_in + (ok ? pos : 0);
        }
        xoff[q] = o;
        xval[q] = ok;
    }
    const int64_t colg = tl.n0 + col;
    const T *xcol = x + (colg < a.N ? (colg / L_out) * (int64_t)C_in * L_in : 0);

    float xreg[NCH][SLOT];
    int xci = 0;  // first channel of the rows held in xreg
    auto fetch_x = [&](int cx) {
        xci = (int)fdiv((uint32_t)(cx * BK), a.fd_K);
#pragma unroll
        for (int cr = 0; cr < NCH; ++cr) {
            const int64_t rowo = (int64_t)min(xci + cr, C_in - 1) * L_in;
#pragma unroll
            for (int q = 0; q < SLOT; ++q) xreg[cr][q] = D::ld(x, xoff[q] + rowo);
        }
    };
    auto commit_x = [&](int cx) {
        float *dx = s_x + (cx & 1) * XBUF + ts;
#pragma unroll
        for (int cr = 0; cr < NCH; ++cr) {
            const bool cok = xci + cr < C_in;
#pragma unroll
            for (int q = 0; q < SLOT; ++q) dx[cr * WTM + NTS * q] = (cok && xval[q]) ? xreg[cr][q] : 0.0f;
        }
    };

    // The 16 samples (rows r0 + 16h + s) of this lane's column for chunk c,
    // into the sample tile.  Row descriptors are wave-uniform (scalar).
    auto sample = [&](int c) {
        const int r0 = c * BK;
        const int ci_lo = (int)fdiv((uint32_t)r0, a.fd_K);
        // Row descriptors, wave-uniform: walk rows rs, rs+1, ... as (ci, k)
        // and ci's offset group g, in scalar registers.  Rows past Kred
        // repeat the last row (their weights are zero).
        int toff[16], xo[16];
        {
            const int rs = __builtin_amdgcn_readfirstlane(min(r0 + 16 * h, Kred - 1));
            const int adv = Kred - 1 - rs;  // steps that stay inside the reduction
            int ci = __builtin_amdgcn_readfirstlane((int)fdiv((uint32_t)rs, a.fd_K));
            int k = rs - ci * K;
            int g = __builtin_amdgcn_readfirstlane((int)fdiv((uint32_t)ci, a.fd_cpo));
            int cg = ci - g * cpo;  // channel within its offset group
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                toff[s] = (g * K + k) * BN;
                xo[s] = WIN ? (c & 1) * XBUF + (ci - ci_lo) * WTM : ci;
                // branch-free advance (selects, not jumps)
                k += (s < adv) ? 1 : 0;
                const int wk = (k == K) ? 1 : 0;
                k = wk ? 0 : k;
                ci += wk;
                cg += wk;
                const int wg = (cg == cpo) ? 1 : 0;
                cg = wg ? 0 : cg;
                g += wg;
            }
        }
        Pos ps[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) ps[s] = s_tab[toff[s] + col];
        float x0[16], x1[16];
        if (WIN) {
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const float *rw = s_x + xo[s] + ps[s].j;
                x0[s] = rw[0];
                x1[s] = rw[1];
            }
        } else {
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const T *rw = xcol + (int64_t)xo[s] * L_in;
                const int i0 = ps[s].j;
                const float a0 = D::ld(rw, min(max(i0, 0), L_in - 1));
                const float a1 = D::ld(rw, min(max(i0 + 1, 0), L_in - 1));
                x0[s] = (i0 >= 0 && i0 < L_in) ? a0 : 0.0f;
                x1[s] = (i0 + 1 >= 0 && i0 + 1 < L_in) ? a1 : 0.0f;
            }
        }
        float v[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) v[s] = fmaf(ps[s].f, x1[s] - x0[s], x0[s]);
        if (MASK) {
#pragma unroll
            for (int s = 0; s < 16; ++s) v[s] *= s_m[toff[s] + col];
        }
        Tr::store_b(s_S + (c & 1) * BN * SLD + col * SLD + 16 * h, v);
    };

    const int c0 = tl.c_begin, c1 = tl.c_end;
    // prologue: windows of c0 and c0+1 in LDS, the loads of c0+2 in registers
    if (WIN) {
        if (c0 < c1) {
            fetch_x(c0);
            commit_x(c0);
        }
        if (c0 + 1 < c1) {
            fetch_x(c0 + 1);
            commit_x(c0 + 1);
        }
        if (c0 + 2 < c1) fetch_x(c0 + 2);
    }
    __syncthreads();
    if (c0 < c1) sample(c0);
    __syncthreads();
    for (int c = c0; c < c1; ++c) {
        if (WIN && c + 2 < c1) commit_x(c + 2);  // loaded during the previous iteration
        if (c + 1 < c1) sample(c + 1);
        // issued after the samples so that nothing in them waits for these loads
        if (WIN && c + 3 < c1) fetch_x(c + 3);
        __syncthreads();
    }
}

// ---- per-workgroup set-up ----------------------------------------------------------
//
// The tile a workgroup owns (output rows, columns, reduction range) and its
// position table: for each (offset group, tap, column) the left neighbour
// and fraction of the sample position (dc1d page, Demo notebook: linear
// interpolation between neighbours) and the mask value (dc1d page,
// Modulation; applied as a plain multiply).  When the tile's positions fit
// the window capacity a.wt_max, the left neighbours become indices into the
// tile's window row: batch segment s occupies [s_base[s], s_base[s+1]) and
// holds input positions s_lo[s] .. s_hi[s] + 1.
template <class Tr, bool MASK>
__device__ __forceinline__ void setup_tile(const MfmaArgs &a, Tile &tl, Pos *s_tab, float *s_m, int *s_lo,
                                           int *s_hi, int *s_base, int *s_win) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    constexpr int BM = Geo<Tr>::BM, BN = Geo<Tr>::BN;
    const Params &p = a.p;
    const int t = threadIdx.x;
    const int U = a.tiles_m * a.tiles_n * a.splits;
    const int u = remap_xcd(blockIdx.x, U);
    tl.tn = u % a.tiles_n;
    const int rest = u / a.tiles_n;
    tl.sp = rest % a.splits;
    tl.tm = rest / a.splits;
    tl.m0 = tl.tm * BM;
    tl.n0 = (int64_t)tl.tn * BN;
    tl.c_begin = (int)((int64_t)tl.sp * a.chunks / a.splits);
    tl.c_end = (int)((int64_t)(tl.sp + 1) * a.chunks / a.splits);
    const int K = p.K, L_in = p.L_in, L_out = p.L_out;
    const int GK = p.G * K;
    const T *__restrict__ off = (const T *)p.off;
    const T *__restrict__ mask = (const T *)p.mask;

    // ---- column tile geometry (N < 2^31: 32-bit column arithmetic)
    const int n_end = (int)((tl.n0 + BN < a.N) ? tl.n0 + BN : a.N);
    tl.b_first = (int)fdiv((uint32_t)tl.n0, a.fd_Lout);
    tl.nseg = (int)fdiv((uint32_t)(n_end - 1), a.fd_Lout) - tl.b_first + 1;
    const bool win = (a.wt_max > 0) && (tl.nseg <= NSEG);
    if (t < NSEG) {
        s_lo[t] = INT_MAX;
        s_hi[t] = INT_MIN;
    }

    // ---- position table, pass 1: left neighbours, fractions, mask; per-segment extent.
    // Thread t serves column n = t % BN (its batch b and position l computed
    // once) and every (NTT/BN)-th entry (g, k) of it.
    constexpr int TPCOL = NTT / BN;  // threads per column
    static_assert(NTT % BN == 0, "whole columns per thread");
    const int n = t % BN;
    const int col = (int)tl.n0 + n;
    const bool cok = col < n_end;
    const int cb_ = cok ? (int)fdiv((uint32_t)col, a.fd_Lout) : tl.b_first;
    const int cl = cok ? col - cb_ * L_out : 0;
    const int sg = cb_ - tl.b_first;  // batch segment of the column
    const int64_t obase = ((int64_t)cb_ * p.G * L_out + cl) * K;
    const int64_t gstride = (int64_t)L_out * K;
    const int grid0 = cl * p.stride - p.padding;
    int lo = INT_MAX, hi = INT_MIN;
    {
        constexpr int TB = 4;  // entries per thread per batch of loads
        for (int gk0 = t / BN; gk0 < GK; gk0 += TPCOL * TB) {
            float ov[TB], mv[TB];
#pragma unroll
            for (int q = 0; q < TB; ++q) {
                const int gk = gk0 + TPCOL * q;
                const int g = (int)fdiv((uint32_t)gk, a.fd_K), k = gk - g * K;
                const bool ok = cok && gk < GK;
                const int64_t oi = ok ? obase + g * gstride + k : 0;
                ov[q] = D::ld(off, oi);
                mv[q] = MASK ? D::ld(mask, oi) : 1.0f;
            }
#pragma unroll
            for (int q = 0; q < TB; ++q) {
                const int gk = gk0 + TPCOL * q;
                if (gk >= GK) break;
                const int k = gk - (int)fdiv((uint32_t)gk, a.fd_K) * K;
                Pos ps = {0, 0.0f};
                if (cok) {
                    int i0;
                    split_position(ov[q], grid0 + k * p.dilation, tap_range(p, k), i0, ps.f);
                    ps.j = min(max(i0, -2), L_in);  // x~ reads zero at both neighbours beyond these bounds
                    lo = min(lo, ps.j);
                    hi = max(hi, ps.j);
                }
                s_tab[gk * BN + n] = ps;
                if (MASK) s_m[gk * BN + n] = cok ? mv[q] : 0.0f;
            }
        }
    }
    __syncthreads();  // s_lo / s_hi initialised
    if (win) {
#pragma unroll
        for (int z = 0; z < NSEG; ++z) {
            int zl = (z == sg) ? lo : INT_MAX, zh = (z == sg) ? hi : INT_MIN;
            for (int o = 32; o > 0; o >>= 1) {
                zl = min(zl, __shfl_xor(zl, o));
                zh = max(zh, __shfl_xor(zh, o));
            }
            if ((t & 63) == 0 && z < tl.nseg && zl <= zh) {
                atomicMin(&s_lo[z], zl);
                atomicMax(&s_hi[z], zh);
            }
        }
    }
    __syncthreads();
    if (t == 0) {
        constexpr int V = 16 / sizeof(T);  // elements per 16-byte word
        int base = 0;
        for (int z = 0; z < (win ? tl.nseg : 0); ++z) {
            int len;
            if (a.vec_x) {  // segments start and end on whole words of x and of the window row
                s_lo[z] &= -V;
                len = (s_hi[z] + 2 - s_lo[z] + V - 1) & -V;
            } else {
                len = s_hi[z] + 2 - s_lo[z];
            }
            s_base[z] = base;
            base += len;
        }
        s_base[win ? tl.nseg : 0] = base;
        // two elements of slack past the last window position (paired reads)
        *s_win = win && base + 2 <= a.wt_max;
    }
    __syncthreads();
    tl.win = *s_win;
    tl.WT = tl.win ? s_base[tl.nseg] : 0;
    // ---- pass 2 (windowed): left neighbour -> index into the tile's window row
    if (tl.win && cok) {
        const int shift = s_base[sg] - s_lo[sg];
        for (int gk = t / BN; gk < GK; gk += TPCOL) s_tab[gk * BN + n].j += shift;
    }
    __syncthreads();  // position table complete

}

template <class Tr, bool MASK, int NCH, int SLOT>
__global__ void __launch_bounds__(NTT) k_mfma(MfmaArgs a) {
    using T = typename Tr::T;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    Pos *s_tab = (Pos *)smem;                   // [G*K][BN]
    float *s_m = (float *)(smem + a.off_mask);  // [G*K][BN] if MASK
    T *s_w = (T *)(smem + a.off_w);             // [2][BM][BK], swizzled
    T *s_S = (T *)(smem + a.off_s);             // [2][BN][SLD]
    float *s_x = (float *)(smem + a.off_x);     // [2][NCH][SLOT * NTS]
    __shared__ int s_lo[NSEG], s_hi[NSEG], s_base[NSEG + 1];
    __shared__ int s_win;
    Tile tl;
    setup_tile<Tr, MASK>(a, tl, s_tab, s_m, s_lo, s_hi, s_base, &s_win);
    if (threadIdx.x < NTM) {
        mfma_role<Tr, 0>(a, tl, s_w, s_S);
    } else if (tl.win) {
        sampler_role<Tr, MASK, true, NCH, SLOT>(a, tl, s_tab, s_m, s_S, s_x, s_lo, s_base);
    } else {
        sampler_role<Tr, MASK, false, 1, 1>(a, tl, s_tab, s_m, s_S, s_x, s_lo, s_base);
    }
}

// ---- channel-block order ------------------------------------------------------------
//
// The reduction over r = (ci, k) may run in any order as long as the weight
// tile and the sample tile agree.  In channel-block order a chunk of 32
// reduction rows is CB consecutive input channels (ci = CB*cb + i) at
// TPC = 32/CB consecutive taps (k = TPC*kb + t), row i*TPC + t; the chunks
// run over taps (kb, inner) within channel blocks (cb, outer).  Then:
//   * a sampler thread's 16 rows are 16/TPC channels at all TPC taps of the
//     chunk and lie in one offset group, so it reads TPC (j, f) pairs (and
//     mask values) per chunk from the position table and reuses each over
//     its channels;
//   * the x window of a channel block (CB rows covering every tap's reach)
//     is staged once and serves all nkb chunks of the block.
// The weights are read in the same order: straight from [C_out][C_in][K]
// when a chunk row's taps are one aligned 16-byte word (DW), else from a copy
// rearranged into [nkb][C_out][ncb][32] by k_weight_blocks.  Taps past K and
// channels past C_in get zero weights.
//
// Window staging: a block's window is NL = CB*SLOT lines of NTS positions
// (thread ts owns position ts of each line; a row holds WTM = SLOT*NTS
// positions).  While the sampler works on block B it stages block B+1 in nkb
// parts of LPP lines, one part per chunk: the loads of a part are issued at
// the end of one iteration and written to LDS at the end of the next, after
// its samples, so their latency hides behind a barrier and a sampling pass.
// Windows are double-buffered by block parity.
template <class Tr, bool MASK, bool WIN, int CB, int SLOT, int LPP, bool VX = false>
__device__ __forceinline__ void sampler_cb(const MfmaArgs &a, const Tile &tl, const Pos *s_tab,
                                           const float *s_m, typename Tr::T *s_S, typename Tr::T *s_x,
                                           const int *s_lo, const int *s_base) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    constexpr int BN = Geo<Tr>::BN, SLD = Tr::SLD;
    constexpr int TPC = BK / CB;    // taps per chunk
    constexpr int CPT = 16 / TPC;   // channels per sampler thread
    constexpr int NL = CB * SLOT;   // staging lines per block
    constexpr int WTM = SLOT * NTS;  // window row (elements)
    constexpr int XBUF = CB * WTM;   // window buffer (elements)
    constexpr bool BF = sizeof(T) == 2;
    static_assert(BN == 128, "two sampler waves per 64 columns");
    static_assert(LPP % SLOT == 0, "a part holds whole window rows");
    static_assert(NL % LPP == 0, "a non-empty part is a full part");
    const Params &p = a.p;
    const int ts = threadIdx.x - NTM;  // 0 .. NTS-1
    const int lane = ts % 64;
    const int sw = __builtin_amdgcn_readfirstlane(ts / 64);
    const int h = sw & 1;
    const int col = 64 * (sw >> 1) + lane;
    const int K = p.K, L_in = p.L_in, L_out = p.L_out, C_in = p.C_in;
    const int nkb = a.nkb;
    const T *__restrict__ x = (const T *)p.x;
    const int i0 = 16 * h / TPC;  // this thread's first channel in a block

    // Per slot: the x offset of its window position in channel 0 (clamped to
    // a real element) and whether the position lies inside [0, L_in).
    int64_t xoff[SLOT];
    bool xval[SLOT];
#pragma unroll
    for (int q = 0; q < SLOT; ++q) {
        const int jj = ts + NTS * q;
        int64_t o = 0;
        bool ok = false;
        if (WIN && jj < tl.WT) {
            int sg = 0;
            while (sg + 1 < tl.nseg && s_base[sg + 1] <= jj) ++sg;
            const int pos = s_lo[sg] + (jj - s_base[sg]);
            ok = pos >= 0 && pos < L_in;
            o = (int64_t)(tl.b_first + sg) * C_in * L_in + (ok ? pos : 0);
        }
        xoff[q] = o;
        xval[q] = ok;
    }
    const int colg = (int)tl.n0 + col;
    const T *xcol = x + (colg < a.N ? (int64_t)fdiv((uint32_t)colg, a.fd_Lout) * C_in * L_in : 0);

    // Word staging (VX): a window row is VPR 16-byte words of V elements;
    // thread ts stages word vv of rows vr, vr + RSTEP, ... of each part.  A
    // word starts on a multiple of V in x, and L_in is a multiple of V, so it
    // lies wholly inside [0, L_in) or wholly outside (then zeros).
    constexpr int V = 16 / sizeof(T);
    constexpr int VPR = WTM / V;          // words per window row
    constexpr int RSTEP = NTS / VPR;      // rows between one thread's words
    constexpr int VPT = VX ? LPP / V : 1;  // words per thread per part
    static_assert(!VX || (LPP % V == 0 && NTS % VPR == 0), "a part is whole words for every thread");
    const int vv = ts % VPR, vr = ts / VPR;
    int64_t vxoff = 0;
    bool vval = false;
    if (VX && WIN && vv * V < tl.WT) {
        const int jj = vv * V;
        int sg = 0;
        while (sg + 1 < tl.nseg && s_base[sg + 1] <= jj) ++sg;
        const int pos = s_lo[sg] + (jj - s_base[sg]);
        vval = pos >= 0 && pos < L_in;
        vxoff = (int64_t)(tl.b_first + sg) * C_in * L_in + (vval ? pos : 0);
    }

    // ---- window staging
    // A part in flight: lines l0 .. l0+LPP-1 of block blk (l0 >= NL: none),
    // loaded into registers and written to LDS later by commit_part.
    struct Part {
        int blk, l0;
        T xr[VX ? 1 : LPP];
        u4 v[VPT];
    };
    auto load_part = [&](Part &q, int blk, int part) {
        q.blk = blk;
        q.l0 = part * LPP;
        if (q.l0 < NL) {  // uniform
            const int ib = q.l0 / SLOT;
            if constexpr (VX) {
#pragma unroll
                for (int n = 0; n < VPT; ++n) {
                    const int ci = min(blk * CB + ib + vr + RSTEP * n, C_in - 1);
                    q.v[n] = *(const u4 *)(x + vxoff + (int64_t)ci * L_in);
                }
            } else {
#pragma unroll
                for (int n = 0; n < LPP; ++n) {
                    const int ci = min(blk * CB + ib + n / SLOT, C_in - 1);
                    q.xr[n] = x[xoff[n % SLOT] + (int64_t)ci * L_in];
                }
            }
        }
    };
    auto commit_part = [&](Part &q) {
        if (q.l0 < NL) {  // uniform
            const int ib = q.l0 / SLOT;
            if constexpr (VX) {
                T *dx = s_x + (q.blk & 1) * XBUF + vv * V;
#pragma unroll
                for (int n = 0; n < VPT; ++n) {
                    const int row = ib + vr + RSTEP * n;
                    const bool ok = vval && q.blk * CB + row < C_in;
                    *(u4 *)(dx + row * WTM) = ok ? q.v[n] : u4{0, 0, 0, 0};
                }
            } else {
                T *dx = s_x + (q.blk & 1) * XBUF + ib * WTM + ts;
                const int cib = q.blk * CB + ib;
#pragma unroll
                for (int n = 0; n < LPP; ++n) {
                    const int qq = n % SLOT;
                    dx[(n / SLOT) * WTM + NTS * qq] = (xval[qq] && cib + n / SLOT < C_in) ? q.xr[n] : (T)0;
                }
            }
        }
        q.l0 = NL;
    };
    Part q0, q1;  // the parts of the next two chunks (see the main loop)
    q0.blk = q1.blk = 0;
    q0.l0 = q1.l0 = NL;
    auto stage_block = [&](int blk) {
        for (int part = 0; part * LPP < NL; ++part) {
            load_part(q0, blk, part);
            commit_part(q0);
        }
    };
    // part kb(u) of the block after chunk u's, if this workgroup uses that block
    auto load_for = [&](Part &q, int u) {
        if (u < tl.c_end) {
            const int bu = (int)fdiv((uint32_t)u, a.fd_nkb);
            if ((bu + 1) * nkb < tl.c_end) load_part(q, bu + 1, u - bu * nkb);
        }
    };

    // ---- the 16 samples (rows 16h .. 16h+15) of this lane's column for chunk u
    auto sample = [&](int u) {
        const int cb = (int)fdiv((uint32_t)u, a.fd_nkb), kb = u - cb * nkb;
        const int g = (int)fdiv((uint32_t)min(cb * CB + i0, C_in - 1), a.fd_cpo);
        const T *xw = s_x + (cb & 1) * XBUF + i0 * WTM;
        // all reads first (the position pairs, then every neighbour pair),
        // then the arithmetic, so that the LDS latency is paid once
        Pos ps[TPC];
        float mk[TPC];
#pragma unroll
        for (int tt = 0; tt < TPC; ++tt) {
            const int k = min(kb * TPC + tt, K - 1);  // taps past K have zero weights
            const int te = (g * K + k) * BN + col;
            ps[tt] = s_tab[te];
            mk[tt] = MASK ? s_m[te] : 1.0f;
        }
        float x0[16], x1[16];
        if (WIN) {
            if constexpr (BF) {
                // the two neighbours from the aligned dword pair holding them
                uint32_t d0[16], d1[16];
#pragma unroll
                for (int tt = 0; tt < TPC; ++tt)
#pragma unroll
                    for (int ii = 0; ii < CPT; ++ii) {
                        const uint32_t *w32 = (const uint32_t *)(xw + ii * WTM) + (ps[tt].j >> 1);
                        d0[ii * TPC + tt] = w32[0];
                        d1[ii * TPC + tt] = w32[1];
                    }
#pragma unroll
                for (int tt = 0; tt < TPC; ++tt)
#pragma unroll
                    for (int ii = 0; ii < CPT; ++ii) {
                        const int s = ii * TPC + tt;
                        const uint32_t pr = __builtin_amdgcn_alignbit(d1[s], d0[s], (ps[tt].j & 1) * 16);
                        x0[s] = __uint_as_float(pr << 16);
                        x1[s] = __uint_as_float(pr & 0xffff0000u);
                    }
            } else {
#pragma unroll
                for (int tt = 0; tt < TPC; ++tt)
#pragma unroll
                    for (int ii = 0; ii < CPT; ++ii) {
                        const float *rw = xw + ii * WTM + ps[tt].j;
                        x0[ii * TPC + tt] = rw[0];
                        x1[ii * TPC + tt] = rw[1];
                    }
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < TPC; ++tt)
#pragma unroll
                for (int ii = 0; ii < CPT; ++ii) {
                    const T *rw = xcol + (int64_t)min(cb * CB + i0 + ii, C_in - 1) * L_in;
                    const int j = ps[tt].j;
                    const float a0 = D::ld(rw, min(max(j, 0), L_in - 1));
                    const float a1 = D::ld(rw, min(max(j + 1, 0), L_in - 1));
                    x0[ii * TPC + tt] = (j >= 0 && j < L_in) ? a0 : 0.0f;
                    x1[ii * TPC + tt] = (j + 1 >= 0 && j + 1 < L_in) ? a1 : 0.0f;
                }
        }
        float v[16];
#pragma unroll
        for (int tt = 0; tt < TPC; ++tt)
#pragma unroll
            for (int ii = 0; ii < CPT; ++ii) {
                const int s = ii * TPC + tt;
                float val = fmaf(ps[tt].f, x1[s] - x0[s], x0[s]);
                if (MASK) val *= mk[tt];
                v[s] = val;
            }
        Tr::store_b(s_S + (u & 1) * BN * SLD + col * SLD + 16 * h, v);
    };

    const int c0 = tl.c_begin, c1 = tl.c_end;
    // Staging schedule: the part P(u) (part kb(u) of the block after chunk
    // u's) is loaded into registers in iteration u-3 and written to LDS in
    // iteration u-1, after that iteration's samples: its loads have two
    // iterations to arrive.  The two parts in flight alternate between q0
    // and q1 (P(u) in q[(u - c0) & 1]).
    // Prologue: the windows of the blocks of chunks c0 and c0+1 in LDS; the
    // parts of the following block that the steady state would already have
    // written, in LDS; P(c0+1) and P(c0+2) in flight.
    if (WIN && c0 < c1) {
        const int b0 = (int)fdiv((uint32_t)c0, a.fd_nkb);
        stage_block(b0);
        if (c0 + 1 < c1) {
            const int b1 = (int)fdiv((uint32_t)(c0 + 1), a.fd_nkb), k1 = c0 + 1 - b1 * nkb;
            if (b1 != b0) stage_block(b1);
            if ((b1 + 1) * nkb < c1) {
                for (int part = 0; part < k1; ++part) {
                    load_part(q0, b1 + 1, part);
                    commit_part(q0);
                }
            }
            load_for(q1, c0 + 1);
            load_for(q0, c0 + 2);
        }
    }
    __syncthreads();
    if (c0 < c1) sample(c0);
    __syncthreads();
    // iteration c: the samples of chunk c+1, then P(c+1) to LDS and P(c+3) loaded, both in q
    auto iter = [&](int c, Part &q) {
        if (c + 1 < c1) sample(c + 1);
        if (WIN) {
            commit_part(q);
            load_for(q, c + 3);
        }
        __syncthreads();
    };
    for (int c = c0; c < c1; c += 2) {
        iter(c, q1);
        if (c + 1 < c1) iter(c + 1, q0);
    }
}

// ---- channel-block order, bf16: windows stored position-major --------------------
//
// With bfloat16 storage and blocks of 32 channels at one tap per chunk, the
// window of a channel block can be kept position-major: row j holds the
// block's 32 channels at window position j (kTPitch elements; the 16-byte
// pad puts consecutive rows on different banks).  A sampler thread's 16
// channels at one position are then two 16-byte words, so the two
// neighbours of its 16 samples are four 16-byte LDS reads, where the
// channel-major window takes two 4-byte reads per sample.  The
// interpolation is the same instruction sequence as sampler_cb's, so both
// give the same bits.
//
// Staging transposes in registers: item (position word pw, channel octet
// co) is one thread's; it loads positions 8pw .. 8pw+7 of its 8 channels
// (eight 16-byte words of x; window segments start on words, so a word lies
// wholly inside [0, L_in) or wholly outside) and writes 8 words, one per
// position, of its 8 channels.  Block B's window is loaded into registers in
// iteration B*nkb - 4 and written to LDS in iteration B*nkb - 2, after that
// iteration's samples (its buffer's previous block is finished by then and
// the block's first chunk is sampled in the next iteration); the first two
// blocks of the workgroup's range are staged before the main loop.  Needs
// nkb >= 2 (a block's window serves at least two chunks).
constexpr int kTPitch = 40;  // bf16 elements per window row: 32 channels + 8 pad (80 bytes)

template <bool MASK, int NPOS>
__device__ __forceinline__ void sampler_cbt(const MfmaArgs &a, const Tile &tl, const Pos *s_tab,
                                            const float *s_m, uint16_t *s_S, uint16_t *s_x, const int *s_lo,
                                            const int *s_base) {
    using Tr = TrBF16;
    using T = uint16_t;
    constexpr int BN = Geo<Tr>::BN, SLD = Tr::SLD, CB = 32;
    constexpr int XBUF = NPOS * kTPitch;           // window buffer (elements)
    constexpr int NITEM = (NPOS / 8) * (CB / 8);   // staging items per block
    static_assert(NPOS % 8 == 0 && NITEM <= NTS, "at most one staging item per thread");
    const Params &p = a.p;
    const int ts = threadIdx.x - NTM;  // 0 .. NTS-1
    const int lane = ts % 64;
    const int sw = __builtin_amdgcn_readfirstlane(ts / 64);
    const int h = sw & 1;
    const int col = 64 * (sw >> 1) + lane;
    const int K = p.K, L_in = p.L_in, C_in = p.C_in;
    const int nkb = a.nkb;
    const T *__restrict__ x = (const T *)p.x;
    const int ic = 16 * h;  // this thread's first channel in a block

    // ---- staging item of this thread
    const bool has_item = ts < NITEM;
    const int pw = ts >> 2, co = ts & 3;
    int64_t ixoff = 0;
    bool ival = false;
    if (has_item && pw * 8 < tl.WT) {
        const int jj = pw * 8;
        int sg = 0;
        while (sg + 1 < tl.nseg && s_base[sg + 1] <= jj) ++sg;
        const int pos = s_lo[sg] + (jj - s_base[sg]);
        ival = pos >= 0 && pos < L_in;
        ixoff = (int64_t)(tl.b_first + sg) * C_in * L_in + (ival ? pos : 0);
    }
    u4 xr[8];
    auto load_blk = [&](int blk) {
        if (!has_item) return;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ci = min(blk * CB + co * 8 + c, C_in - 1);
            xr[c] = *(const u4 *)(x + ixoff + (int64_t)ci * L_in);
        }
    };
    auto commit_blk = [&](int blk) {
        if (!has_item) return;
        uint32_t keep[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) keep[c] = (ival && blk * CB + co * 8 + c < C_in) ? 0xffffffffu : 0u;
        T *dst = s_x + (blk & 1) * XBUF + pw * 8 * kTPitch + co * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // positions 2q, 2q+1: dword q of every channel's word
            u4 ev, od;
#pragma unroll
            for (int i = 0; i < 4; ++i) {  // channels 2i, 2i+1
                const uint32_t lo = xr[2 * i][q] & keep[2 * i], hi = xr[2 * i + 1][q] & keep[2 * i + 1];
                ev[i] = (lo & 0xffffu) | (hi << 16);
                od[i] = (lo >> 16) | (hi & 0xffff0000u);
            }
            *(u4 *)(dst + (2 * q) * kTPitch) = ev;
            *(u4 *)(dst + (2 * q + 1) * kTPitch) = od;
        }
    };

    // ---- the 16 samples (channels ic .. ic+15 of the block, one tap) of this lane's column for chunk u.
    // The chunk's position pair (and mask value) is read at the end of the
    // previous chunk's samples, so that its LDS latency passes in the barrier.
    Pos ps;
    float mk;
    auto fetch_pos = [&](int u) {
        const int cb = (int)fdiv((uint32_t)u, a.fd_nkb), k = u - cb * nkb;  // one tap per chunk: kb is the tap
        const int g = (int)fdiv((uint32_t)min(cb * CB + ic, C_in - 1), a.fd_cpo);
        const int te = (g * K + k) * BN + col;
        ps = s_tab[te];
        mk = MASK ? s_m[te] : 1.0f;
    };
    auto sample = [&](int u) {
        const int cb = (int)fdiv((uint32_t)u, a.fd_nkb);
        const T *xw = s_x + (cb & 1) * XBUF + __umul24((uint32_t)ps.j, kTPitch) + ic;
        const u4 a0 = *(const u4 *)xw, a1 = *(const u4 *)(xw + 8);
        const u4 b0 = *(const u4 *)(xw + kTPitch), b1 = *(const u4 *)(xw + kTPitch + 8);
        float x0[16], x1[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x0[2 * i] = __uint_as_float(a0[i] << 16);
            x0[2 * i + 1] = __uint_as_float(a0[i] & 0xffff0000u);
            x0[8 + 2 * i] = __uint_as_float(a1[i] << 16);
            x0[8 + 2 * i + 1] = __uint_as_float(a1[i] & 0xffff0000u);
            x1[2 * i] = __uint_as_float(b0[i] << 16);
            x1[2 * i + 1] = __uint_as_float(b0[i] & 0xffff0000u);
            x1[8 + 2 * i] = __uint_as_float(b1[i] << 16);
            x1[8 + 2 * i + 1] = __uint_as_float(b1[i] & 0xffff0000u);
        }
        float v[16];
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
            float val = fmaf(ps.f, x1[s2] - x0[s2], x0[s2]);
            if (MASK) val *= mk;
            v[s2] = val;
        }
        Tr::store_b(s_S + (u & 1) * BN * SLD + col * SLD + 16 * h, v);
        fetch_pos(min(u + 1, tl.c_end - 1));
    };

    const int c0 = tl.c_begin, c1 = tl.c_end;
    const int b0 = c0 < c1 ? (int)fdiv((uint32_t)c0, a.fd_nkb) : 0;
    fetch_pos(max(min(c0, c1 - 1), 0));
    // prologue: blocks b0 and b0+1 in LDS; block b0+2 in registers when its
    // regular load iteration lies before c0
    if (c0 < c1) {
        load_blk(b0);
        commit_blk(b0);
        if ((b0 + 1) * nkb < c1) {
            load_blk(b0 + 1);
            commit_blk(b0 + 1);
        }
        if ((b0 + 2) * nkb < c1 && (b0 + 2) * nkb - 4 < c0) load_blk(b0 + 2);
    }
    __syncthreads();
    if (c0 < c1) sample(c0);
    __syncthreads();
    for (int c = c0; c < c1; ++c) {
        if (c + 1 < c1) sample(c + 1);
        // block (c+2)/nkb to LDS, then block (c+4)/nkb into registers (blocks
        // from b0+2 on whose first chunk is inside the range)
        const int bc = (int)fdiv((uint32_t)(c + 2), a.fd_nkb);
        if (bc * nkb == c + 2 && bc >= b0 + 2 && c + 2 < c1) commit_blk(bc);
        const int bl = (int)fdiv((uint32_t)(c + 4), a.fd_nkb);
        if (bl * nkb == c + 4 && bl >= b0 + 2 && c + 4 < c1) load_blk(bl);
        __syncthreads();
    }
}

// The bf16 channel-block kernel with position-major windows (sampler_cbt);
// tiles whose offsets spread wider than the window gather with sampler_cb.
template <bool MASK, int NPOS>
__global__ void __launch_bounds__(NTT) k_mfma_cbt(MfmaArgs a) {
    using Tr = TrBF16;
    using T = uint16_t;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    Pos *s_tab = (Pos *)smem;                   // [G*K][BN]
    float *s_m = (float *)(smem + a.off_mask);  // [G*K][BN] if MASK
    T *s_w = (T *)(smem + a.off_w);             // [2][BM][BK], swizzled
    T *s_S = (T *)(smem + a.off_s);             // [2][BN][SLD]
    T *s_x = (T *)(smem + a.off_x);             // [2][NPOS][kTPitch]
    __shared__ int s_lo[NSEG], s_hi[NSEG], s_base[NSEG + 1];
    __shared__ int s_win;
    Tile tl;
    setup_tile<Tr, MASK>(a, tl, s_tab, s_m, s_lo, s_hi, s_base, &s_win);
    if (threadIdx.x < NTM)
        mfma_role<Tr, 1>(a, tl, s_w, s_S);
    else if (tl.win)
        sampler_cbt<MASK, NPOS>(a, tl, s_tab, s_m, s_S, s_x, s_lo, s_base);
    else
        sampler_cb<Tr, MASK, false, 32, 1, 4>(a, tl, s_tab, s_m, s_S, s_x, s_lo, s_base);
}

template <class Tr, bool MASK, int CB, int SLOT, int LPP, bool DW>
__global__ void __launch_bounds__(NTT) k_mfma_cb(MfmaArgs a) {
    using T = typename Tr::T;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    Pos *s_tab = (Pos *)smem;                   // [G*K][BN]
    float *s_m = (float *)(smem + a.off_mask);  // [G*K][BN] if MASK
    T *s_w = (T *)(smem + a.off_w);             // [2][BM][BK], swizzled
    T *s_S = (T *)(smem + a.off_s);             // [2][BN][SLD]
    T *s_x = (T *)(smem + a.off_x);             // [2][CB][SLOT * NTS]
    __shared__ int s_lo[NSEG], s_hi[NSEG], s_base[NSEG + 1];
    __shared__ int s_win;
    Tile tl;
    setup_tile<Tr, MASK>(a, tl, s_tab, s_m, s_lo, s_hi, s_base, &s_win);
    if (threadIdx.x < NTM) {
        mfma_role<Tr, DW ? 2 : 1>(a, tl, s_w, s_S);
    } else if (tl.win) {
        if constexpr (LPP % (16 / sizeof(T)) == 0) {
            if (a.vec_x) {
                sampler_cb<Tr, MASK, true, CB, SLOT, LPP, true>(a, tl, s_tab, s_m, s_S, s_x, s_lo, s_base);
                return;
            }
        }
        sampler_cb<Tr, MASK, true, CB, SLOT, LPP>(a, tl, s_tab, s_m, s_S, s_x, s_lo, s_base);
    } else {
        sampler_cb<Tr, MASK, false, CB, 1, 4>(a, tl, s_tab, s_m, s_S, s_x, s_lo, s_base);
    }
}

// Weights [C_out][C_in][K] -> chunk rows [nkb][C_out][ncb][32]: element
// (kb, m, cb, i*TPC + t) = W[m][CB*cb + i][TPC*kb + t], zero past C_in or K.
// A plain copy of the stored bits; one workgroup per destination row.
template <class T>
__global__ void __launch_bounds__(256) k_weight_blocks(const T *__restrict__ w, T *__restrict__ wb, int C_out,
                                                       int C_in, int K, int tpc_log2, int ncb) {
    const int row = blockIdx.x;  // kb * C_out + m
    const int kb = row / C_out, m = row - kb * C_out;
    const int len = ncb * BK, cbs = BK >> tpc_log2, tmask = (1 << tpc_log2) - 1;
    const T *__restrict__ wm = w + (int64_t)m * C_in * K;
    T *__restrict__ dst = wb + (int64_t)row * len;
    for (int j = threadIdx.x; j < len; j += 256) {
        const int r = j & (BK - 1);
        const int ci = (j >> 5) * cbs + (r >> tpc_log2), k = (kb << tpc_log2) + (r & tmask);
        dst[j] = (ci < C_in && k < K) ? wm[ci * K + k] : (T)0;
    }
}

// ---- plain GEMM (used by the backward) -------------------------------------------
//
// C[b][m][j] = sum_k A[m][k] * B(k, n),  n = b*L_out + j, for A = p.w row-major
// [M = p.C_out][p.Kred] and B(k, n) = p.x[b*bbatch + j + k*brow]; C = p.out
// [B][M][L_out].  The MFMA role is the forward's (weights = A); the second
// role loads the B tile instead of sampling it: thread (h, col) loads rows
// 16h .. 16h+15 of its column one chunk ahead into registers and writes them
// to the sample tile an iteration later, so the load latency hides behind
// the MFMAs.
template <class Tr>
__device__ __forceinline__ void loader_role(const MfmaArgs &a, const Tile &tl, typename Tr::T *s_S) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    constexpr int BN = Geo<Tr>::BN, SLD = Tr::SLD;
    const Params &p = a.p;
    const int ts = threadIdx.x - NTM;
    const int lane = ts % 64;
    const int sw = __builtin_amdgcn_readfirstlane(ts / 64);
    const int h = sw & 1;
    const int col = 64 * (sw >> 1) + lane;
    const int n = (int)tl.n0 + col;
    const bool cok = n < a.N;
    const int b = cok ? (int)fdiv((uint32_t)n, a.fd_Lout) : 0;
    const T *__restrict__ bcol = (const T *)p.x + (cok ? (int64_t)b * a.bbatch + (n - b * p.L_out) : 0);
    const int Kred = p.Kred;
    float breg[16];
    auto fetch = [&](int c) {  // clamped addresses; rows past Kred are zeroed in put
        const int r0 = c * BK + 16 * h;
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) breg[s2] = D::ld(bcol, (int64_t)min(r0 + s2, Kred - 1) * a.brow);
    };
    auto put = [&](int c) {
        const int r0 = c * BK + 16 * h;
        float v[16];
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) v[s2] = (cok && r0 + s2 < Kred) ? breg[s2] : 0.0f;
        Tr::store_b(s_S + (c & 1) * BN * SLD + col * SLD + 16 * h, v);
    };
    const int c0 = tl.c_begin, c1 = tl.c_end;
    if (c0 < c1) {
        fetch(c0);
        put(c0);
    }
    if (c0 + 1 < c1) fetch(c0 + 1);
    // the MFMA role's two prologue barriers
    __syncthreads();
    __syncthreads();
    for (int c = c0; c < c1; ++c) {
        if (c + 1 < c1) put(c + 1);    // loaded during the previous iteration
        if (c + 2 < c1) fetch(c + 2);
        __syncthreads();
    }
}

template <class Tr, int OUT>
__global__ void __launch_bounds__(NTT) k_gemm(MfmaArgs a) {
    using T = typename Tr::T;
    constexpr int BM = Geo<Tr>::BM, BN = Geo<Tr>::BN;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *s_w = (T *)(smem + a.off_w);  // [2][BM][BK], swizzled
    T *s_S = (T *)(smem + a.off_s);  // [2][BN][SLD]
    const int U = a.tiles_m * a.tiles_n * a.splits;
    const int u = remap_xcd(blockIdx.x, U);
    Tile tl;
    tl.tn = u % a.tiles_n;
    const int rest = u / a.tiles_n;
    tl.sp = rest % a.splits;
    tl.tm = rest / a.splits;
    tl.m0 = tl.tm * BM;
    tl.n0 = (int64_t)tl.tn * BN;
    tl.c_begin = (int)((int64_t)tl.sp * a.chunks / a.splits);
    tl.c_end = (int)((int64_t)(tl.sp + 1) * a.chunks / a.splits);
    tl.win = false;
    tl.WT = tl.nseg = tl.b_first = 0;
    if (threadIdx.x < NTM)
        mfma_role<Tr, 0, OUT>(a, tl, s_w, s_S);
    else
        loader_role<Tr>(a, tl, s_S);
    if constexpr (OUT != 0) {
        if (a.splits == 1) {  // uniform: the direct path staged the tile in LDS
            float *s_bias = (float *)s_w + BM * kHeadLd;
            const T *__restrict__ bias = (const T *)a.p.bias;
            for (int r = threadIdx.x - NTM; r >= 0 && r < BM; r += NTT - NTM) {
                const int row = tl.m0 + r;
                s_bias[r] = (bias && row < a.p.C_out) ? Tr::D::ld(bias, row) : 0.0f;
            }
            __syncthreads();
            head_writeout<Tr, OUT>(a, tl, (const float *)s_w, s_bias);
        }
    }
}

// Sum of the split partial tiles (in split order), plus bias, into out.
// One thread per 4-float vector of a partial tile: vector (q4, t) holds what
// MFMA thread t of every split's workgroup kept in its register group q4, so
// the register-order layout maps back to (row, column) exactly as in the
// direct epilogue.
template <class Tr, int OUT = 0>
__global__ void __launch_bounds__(256) k_split_reduce(MfmaArgs a) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    constexpr int MB = Tr::MB, NB = Tr::NB, BM = Geo<Tr>::BM, BN = Geo<Tr>::BN;
    constexpr int VPT = BM * BN / 4;  // vectors per tile
    const Params &p = a.p;
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= tiles * VPT) return;
    const int tile = (int)(v / VPT);
    const int rem = (int)(v - (int64_t)tile * VPT);
    const int q4 = rem / NTM, t = rem % NTM;
    const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
    const int wv = t / 64, lane = t % 64, li = lane % 32, lh = lane / 32;
    const f4 *part = (const f4 *)a.partials + v;
    f4 tot = part[0];
    for (int s2 = 1; s2 < a.splits; ++s2) tot += part[(int64_t)s2 * tiles * VPT];
    const int mb = q4 / (NB * 4), nb = (q4 / 4) % NB, qq = (q4 & 3) * 4;
    const int col = tn * BN + Geo<Tr>::col0(wv) + 32 * nb + li;
    if (col >= a.N) return;
    const int L_out = p.L_out, M = p.C_out;
    const int b = (int)fdiv((uint32_t)col, a.fd_Lout);
    const int l = col - b * L_out;
    const T *__restrict__ bias = (const T *)p.bias;
    T *ob = (T *)p.out + (int64_t)b * M * L_out + l;
    const int row_q = tm * BM + Geo<Tr>::row0(wv) + 32 * mb + 8 * (qq >> 2) + 4 * lh;  // rows row_q + z
    float bz[4];
#pragma unroll
    for (int z = 0; z < 4; ++z) bz[z] = bias ? D::ld(bias, min(row_q + z, M - 1)) : 0.0f;  // before any store
#pragma unroll
    for (int z = 0; z < 4; ++z) {
        const int row = row_q + z;
        if (row >= M) continue;
        const float val = tot[z] + bz[z];
        if constexpr (OUT == 0)
            Tr::st1(ob + (int64_t)row * L_out, val);
        else
            store_head<Tr, OUT>(p, b, l, row, val);
    }
}


// ---- launch ----------------------------------------------------------------------

// Window staging shapes the sampler role is compiled for: (channel rows per
// chunk, 256-element slots per row).  The plan picks the smallest that holds a
// chunk's channel rows and the tiles' expected window extent.
struct Combo {
    int nch, slot;
};
constexpr Combo kCombos[] = {{2, 1}, {2, 2}, {3, 2}, {5, 2}, {8, 2}, {12, 1}, {12, 2}, {16, 1}};
constexpr int kNumCombos = sizeof(kCombos) / sizeof(kCombos[0]);

template <class Tr, bool MASK, int I>
void launch_combo(int idx, const MfmaArgs &a, dim3 grid, size_t lds, hipStream_t stream) {
    if constexpr (I < kNumCombos) {
        if (idx == I)
            hipLaunchKernelGGL((k_mfma<Tr, MASK, kCombos[I].nch, kCombos[I].slot>), grid, dim3(NTT), lds, stream, a);
        else
            launch_combo<Tr, MASK, I + 1>(idx, a, grid, lds, stream);
    }
}

// Staging shapes of the channel-block kernel: (channels per block, window
// slots of NTS positions, lines staged per chunk, weights read directly).
struct CbCombo {
    int cb, slot, lpp;
    bool dw;
};
constexpr CbCombo kCbCombos[] = {
    {8, 1, 4, false},   {8, 1, 8, false},   {8, 2, 4, false},   {8, 2, 8, false},   {8, 2, 16, false},
    {16, 1, 4, false},  {16, 1, 8, false},  {16, 1, 16, false}, {16, 2, 4, false},  {16, 2, 8, false},
    {16, 2, 16, false}, {16, 2, 32, false}, {32, 1, 4, false},  {32, 1, 8, false},  {32, 1, 16, false},
    {32, 1, 32, false}, {32, 2, 4, false},  {32, 2, 8, false},  {32, 2, 16, false}, {32, 2, 32, false},
    {8, 1, 4, true},    {8, 1, 8, true},    {8, 2, 4, true},    {8, 2, 8, true},    {8, 2, 16, true}};
constexpr int kNumCbCombos = sizeof(kCbCombos) / sizeof(kCbCombos[0]);

template <class Tr, bool MASK, int I>
void launch_cb_combo(int idx, const MfmaArgs &a, dim3 grid, size_t lds, hipStream_t stream) {
    if constexpr (I < kNumCbCombos) {
        constexpr CbCombo c = kCbCombos[I];
        if constexpr (!c.dw || sizeof(typename Tr::T) == 4) {  // direct weights: fp32 only
            if (idx == I) {
                hipLaunchKernelGGL((k_mfma_cb<Tr, MASK, c.cb, c.slot, c.lpp, c.dw>), grid, dim3(NTT), lds, stream, a);
                return;
            }
        }
        launch_cb_combo<Tr, MASK, I + 1>(idx, a, grid, lds, stream);
    }
}

// Window sizes (positions) the position-major bf16 kernel is compiled for.
constexpr int kTposOpts[] = {256, 320, 384, 512};
constexpr int kNumTpos = sizeof(kTposOpts) / sizeof(kTposOpts[0]);

template <bool MASK, int I>
void launch_cbt(int npos, const MfmaArgs &a, dim3 grid, size_t lds, hipStream_t stream) {
    if constexpr (I < kNumTpos) {
        if (npos == kTposOpts[I])
            hipLaunchKernelGGL((k_mfma_cbt<MASK, kTposOpts[I]>), grid, dim3(NTT), lds, stream, a);
        else
            launch_cbt<MASK, I + 1>(npos, a, grid, lds, stream);
    }
}

template <class Tr, bool MASK>
hipError_t launch_for(const Params &p, const MfmaPlan &pl, hipStream_t stream) {
    using T = typename Tr::T;
    MfmaArgs a;
    a.p = p;
    a.fd_K = make_fastdiv((uint32_t)p.K);
    a.fd_cpo = make_fastdiv((uint32_t)p.cpo);
    a.fd_Lout = make_fastdiv((uint32_t)p.L_out);
    a.tiles_m = pl.tiles_m;
    a.tiles_n = pl.tiles_n;
    a.splits = pl.splits;
    a.chunks = pl.chunks;
    a.N = (int64_t)p.B * p.L_out;
    a.wt_max = pl.wt_max;
    a.off_mask = pl.off_mask;
    a.off_w = pl.off_w;
    a.off_s = pl.off_s;
    a.off_x = pl.off_x;
    const int vec_elems = 16 / (int)sizeof(T);
    a.vec_w = (p.Kred % vec_elems == 0) && (((uintptr_t)p.w & 15) == 0);
    a.vec_x = pl.blocked && (p.L_in % vec_elems == 0) && (((uintptr_t)p.x & 15) == 0);
    a.wb = nullptr;
    a.ncb = pl.ncb;
    a.nkb = pl.nkb;
    a.fd_nkb = make_fastdiv((uint32_t)(pl.nkb > 0 ? pl.nkb : 1));
    a.partials = pl.splits > 1 ? (float *)((char *)p.ws + pl.wb_bytes) : nullptr;
    const dim3 grid((unsigned)pl.blocks);
    if (pl.blocked) {
        int variant = pl.variant;
        if (pl.variant_dw >= 0 && ((uintptr_t)p.w & 15) == 0) variant = pl.variant_dw;
        if (variant < 0 || variant >= kNumCbCombos) return hipErrorInvalidValue;
        const bool cbt = std::is_same<Tr, TrBF16>::value && pl.tpos > 0 && a.vec_x;
        if (cbt || !kCbCombos[variant].dw) {
            T *wb = (T *)p.ws;
            a.wb = wb;
            int tpc_log2 = 0;
            while ((BK >> tpc_log2) > pl.cb) ++tpc_log2;
            hipLaunchKernelGGL((k_weight_blocks<T>), dim3((unsigned)(pl.nkb * p.C_out)), dim3(256), 0, stream,
                               (const T *)p.w, wb, p.C_out, p.C_in, p.K, tpc_log2, pl.ncb);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        mark_event(p.ev_start, stream);
        if constexpr (std::is_same<Tr, TrBF16>::value) {
            if (cbt) {
                a.wt_max = pl.tpos;
                launch_cbt<MASK, 0>(pl.tpos, a, grid, pl.lds_bytes, stream);
            } else {
                launch_cb_combo<Tr, MASK, 0>(variant, a, grid, pl.lds_bytes, stream);
            }
        } else {
            launch_cb_combo<Tr, MASK, 0>(variant, a, grid, pl.lds_bytes, stream);
        }
        mark_event(p.ev_stop, stream);
    } else {
        if (pl.variant < 0 || pl.variant >= kNumCombos) return hipErrorInvalidValue;
        mark_event(p.ev_start, stream);
        launch_combo<Tr, MASK, 0>(pl.variant, a, grid, pl.lds_bytes, stream);
        mark_event(p.ev_stop, stream);
    }
    if (pl.splits > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
        const int64_t vecs = tiles * (Geo<Tr>::BM * Geo<Tr>::BN / 4);
        hipLaunchKernelGGL((k_split_reduce<Tr>), dim3((unsigned)((vecs + 255) / 256)), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace dc1d
