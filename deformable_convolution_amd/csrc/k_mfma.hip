// k_mfma.hip -- fused deformable sampling + MFMA GEMM for groups == 1.
//
// The contraction out[b, co, l] = bias[co] + sum_r W[co, r] S[r, (b, l)] is a
// GEMM with M = C_out, N = B*L_out and reduction r = ci*K + k over the
// weight viewed as [C_out, C_in*K] (conv1d operator page, Description; the
// article's Step 3 weighted summation).  S is the deformable sample matrix
// (the article's Step 2); it lives only as a small double-buffered tile in
// LDS, never in HBM.
//
// Workgroup: 8 waves in two roles (warp specialisation), one per SIMD each:
//   * 4 MFMA waves.  MFMA wave w owns the 32*NB columns [32*NB*w, ...) of
//     the BM x BN output tile and all its BM rows; it reads operand
//     fragments from LDS and issues MFMAs, and stages the next chunk's
//     weight tile, whose load latency hides under its MFMAs.
//   * 4 sampler waves.  They stage the zero-padded x windows from HBM into
//     LDS and compute the sample tile of the next reduction chunk.
// The hardware interleaves the two roles on every SIMD: MFMAs of one wave
// run while the other wave's VALU, LDS and memory instructions issue.  The
// reduction runs in chunks of BK = 32 rows; in iteration c the MFMA waves
// consume chunk c and stage chunk c+1's weight tile while the sampler waves
// produce chunk c+1's sample tile and stage windows two chunks ahead; one
// barrier per chunk.  Sample tiles and weight tiles are double-buffered,
// windows triple-buffered.
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
    FastDiv fd_K, fd_cpo;
    int tiles_m, tiles_n, splits, chunks;
    int64_t N;
    float *partials;  // split partial tiles [splits][tiles][BM*BN], or null
    int nch;          // input channels a chunk can touch
    int wt_max;       // window capacity per channel row (elements); 0: always gather
    int off_mask, off_row, off_w, off_s, off_x;  // byte offsets of the LDS regions
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
    static constexpr int MB = 8, NB = 1;  // BM = 256, BN = 128
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
};

// Two floats -> two bfloat16 (round to nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf2 r = __builtin_convertvector(f2{lo, hi}, bf2);
    return __builtin_bit_cast(uint32_t, r);
}

struct TrBF16 {
    using D = BF16;
    using T = uint16_t;
    static constexpr int MB = 8, NB = 1;  // BM = 256, BN = 128
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
};

template <class Tr>
struct Geo {
    static constexpr int BM = 32 * Tr::MB;
    static constexpr int BN = NWM * 32 * Tr::NB;
    static constexpr int WV = BM * Tr::WPR / NTM;  // 16-byte weight words per MFMA thread per chunk
};

// Shared per-workgroup state the two roles read.
struct Tile {
    int m0, tm, tn, sp, c_begin, c_end;
    int64_t n0;
    bool win;
    int WT, nseg, b_first;
};

// ---- the MFMA role -------------------------------------------------------------
template <class Tr, bool VEC_W>
__device__ __forceinline__ void mfma_role(const MfmaArgs &a, const Tile &tl, typename Tr::T *s_w,
                                          const typename Tr::T *s_S) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    using Frag = typename Tr::Frag;
    constexpr int MB = Tr::MB, NB = Tr::NB, BM = Geo<Tr>::BM, BN = Geo<Tr>::BN, SLD = Tr::SLD;
    constexpr int WPR = Tr::WPR, WV = Geo<Tr>::WV;
    constexpr int EPW = 16 / sizeof(T);  // elements per 16-byte word
    static_assert(WV * NTM == BM * WPR, "weight tile split");
    const Params &p = a.p;
    const int t = threadIdx.x;
    const int wv = t / 64, lane = t % 64, li = lane % 32, lh = lane / 32;
    const int M = p.C_out, Kred = p.Kred;
    const T *__restrict__ w = (const T *)p.w;

    // The weight tile of chunk c+1 is loaded into registers at the start of
    // iteration c and written to LDS after chunk c's MFMAs, so its load
    // latency hides under them.
    u4 wreg[WV];
    // global -> registers: weight tile of chunk cw
    auto fetch_w = [&](int cw) {
        const int r0 = cw * BK;
#pragma unroll
        for (int v = 0; v < WV; ++v) {
            const int e = t + NTM * v;
            const int row = e / WPR, part = e % WPR;
            const int m = tl.m0 + row, rb = r0 + part * EPW;
            const T *src = w + (int64_t)(m < M ? m : M - 1) * Kred + rb;
            u4 q = {0, 0, 0, 0};
            if (VEC_W) {
                // Kred is a multiple of the word size: a word is wholly inside or outside
                if (m < M && rb < Kred) q = *(const u4 *)src;
            } else {
                T tmp[EPW];
#pragma unroll
                for (int z = 0; z < EPW; ++z) tmp[z] = (m < M && rb + z < Kred) ? src[z] : (T)0;
                q = __builtin_bit_cast(u4, tmp);
            }
            wreg[v] = q;
        }
    };
    auto commit_w = [&](int cw) {
        T *dw = s_w + (cw & 1) * BM * BK;
#pragma unroll
        for (int v = 0; v < WV; ++v) {
            const int e = t + NTM * v;
            const int row = e / WPR, part = e % WPR;
            *(u4 *)(dw + row * BK + EPW * Tr::swz(row, part)) = wreg[v];
        }
    };

    f16v acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;

    if (tl.c_begin < tl.c_end) {
        fetch_w(tl.c_begin);
        commit_w(tl.c_begin);
    }
    // prologue barriers shared with the sampler role: staging done, first sample tile done
    __syncthreads();
    __syncthreads();
    for (int c = tl.c_begin; c < tl.c_end; ++c) {
        const bool more = c + 1 < tl.c_end;
        if (more) fetch_w(c + 1);
        const T *tile = s_w + (c & 1) * BM * BK;
        const T *st = s_S + (c & 1) * BN * SLD;
        Frag bf[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) Tr::lds_b(st + (32 * (NB * wv + nb) + li) * SLD + 16 * lh, bf[nb]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            Frag af;
            Tr::lds_a(tile, 32 * mb + li, lh, af);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Tr::mma(af, bf[nb], acc[mb][nb]);
        }
        if (more) commit_w(c + 1);
        __syncthreads();
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
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t col = tl.n0 + 32 * (NB * wv + nb) + li;
        if (col >= a.N) continue;
        const int b = (int)(col / L_out);
        const int l = (int)(col - (int64_t)b * L_out);
        T *ob = out + (int64_t)b * M * L_out + l;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = tl.m0 + 32 * mb + 8 * (q >> 2) + 4 * lh + (q & 3);
                if (row < M) D::st(ob, (int64_t)row * L_out, acc[mb][nb][q] + (bias ? D::ld(bias, row) : 0.0f));
            }
    }
}

// ---- the sampler role ------------------------------------------------------------
//
// Sampler wave sw computes the samples of reduction rows r0 + 16*h .. + 15
// (h = sw & 1) for 64 columns (64*(sw >> 1) + lane), so that a row's
// position-table row and window row are the same for the whole wave and are
// computed in scalar registers.  Windows are triple-buffered: the loads of
// chunk c+3 are issued in iteration c and written to LDS at the start of
// iteration c+1, a full iteration after they were issued.
template <class Tr, bool MASK, bool WIN, int NCHM, int SLOTM>
__device__ __forceinline__ void sampler_role(const MfmaArgs &a, const Tile &tl, const Pos *s_tab,
                                             const float *s_m, typename Tr::T *s_S, float *s_x,
                                             const int *s_lo, const int *s_base) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    constexpr int BN = Geo<Tr>::BN, SLD = Tr::SLD;
    static_assert(BN == 128, "two sampler waves per 64 columns");
    const Params &p = a.p;
    const int ts = threadIdx.x - NTM;  // 0 .. NTS-1
    const int lane = ts % 64;
    const int sw = __builtin_amdgcn_readfirstlane(ts / 64);
    const int h = sw & 1;
    const int col = 64 * (sw >> 1) + lane;
    const int Kred = p.Kred, K = p.K, L_in = p.L_in, L_out = p.L_out;
    const T *__restrict__ x = (const T *)p.x;
    const int nch = a.nch;  // <= NCHM by the plan
    const int wt_max = a.wt_max;
    const int WT = tl.WT;
    const int xbuf = nch * wt_max;  // floats per window buffer

    // window slots of this thread: positions jj = ts + NTS*q of the window row
    const int nslot = WIN ? (WT + NTS - 1) / NTS : 0;  // <= SLOTM by the plan
    int64_t xoff[SLOTM];  // per slot: element offset of x~ at channel 0, or -1 for a zero
#pragma unroll
    for (int q = 0; q < SLOTM; ++q) {
        const int jj = ts + NTS * q;
        int64_t o = -1;
        if (WIN && q < nslot && jj < WT) {
            int s = 0;
            while (s + 1 < tl.nseg && s_base[s + 1] <= jj) ++s;
            const int pos = s_lo[s] + (jj - s_base[s]);
            if (pos >= 0 && pos < L_in) o = (int64_t)(tl.b_first + s) * p.C_in * L_in + pos;
        }
        xoff[q] = o;
    }
    const int64_t colg = tl.n0 + col;
    const T *xcol = x + (colg < a.N ? (colg / L_out) * (int64_t)p.C_in * L_in : 0);

    float xreg[NCHM][SLOTM];
    auto fetch_x = [&](int cx) {
        const int ci_lo = (int)fdiv((uint32_t)(cx * BK), a.fd_K);
#pragma unroll
        for (int cr = 0; cr < NCHM; ++cr) {
            const int ci = ci_lo + cr;
#pragma unroll
            for (int q = 0; q < SLOTM; ++q) {
                const int64_t o = xoff[q];
                xreg[cr][q] = (cr < nch && ci < p.C_in && o >= 0) ? D::ld(x, o + (int64_t)ci * L_in) : 0.0f;
            }
        }
    };
    auto commit_x = [&](int cx) {
        float *dx = s_x + (cx % 3) * xbuf;
#pragma unroll
        for (int cr = 0; cr < NCHM; ++cr)
#pragma unroll
            for (int q = 0; q < SLOTM; ++q)
                if (cr < nch && q < nslot && ts + NTS * q < WT) dx[cr * wt_max + ts + NTS * q] = xreg[cr][q];
    };

    // The 16 samples (rows r0 + 16h + s) of this lane's column for chunk c,
    // into the sample tile.  Row descriptors are wave-uniform (scalar).
    auto sample = [&](int c) {
        const int r0 = c * BK;
        const int ci_lo = (int)fdiv((uint32_t)r0, a.fd_K);
        int toff[16], xo[16];
        {
            int r = min(r0 + 16 * h, Kred - 1);
            int ci = (int)fdiv((uint32_t)r, a.fd_K);
            int k = r - ci * K;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int g = (int)fdiv((uint32_t)ci, a.fd_cpo);
                toff[s] = (g * K + k) * BN;
                xo[s] = WIN ? (c % 3) * xbuf + (ci - ci_lo) * wt_max : ci;
                if (r0 + 16 * h + s + 1 < Kred) {  // rows past Kred repeat the last row (zero weights)
                    if (++k == K) {
                        k = 0;
                        ++ci;
                    }
                }
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
    // prologue: windows of c0, c0+1, c0+2 (loads of c0+2 stay in registers)
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
        if (WIN && c + 2 < c1) {
            commit_x(c + 2);  // loaded during the previous iteration
            if (c + 3 < c1) fetch_x(c + 3);
        }
        if (c + 1 < c1) sample(c + 1);
        __syncthreads();
    }
}

template <class Tr, bool VEC_W, bool MASK, int NCHM, int SLOTM>
__global__ void __launch_bounds__(NTT) k_mfma(MfmaArgs a) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    constexpr int BM = Geo<Tr>::BM, BN = Geo<Tr>::BN;

    extern __shared__ __attribute__((aligned(16))) char smem[];
    Pos *s_tab = (Pos *)smem;                   // [G*K][BN]
    float *s_m = (float *)(smem + a.off_mask);  // [G*K][BN] if MASK
    T *s_w = (T *)(smem + a.off_w);             // [2][BM][BK], swizzled
    T *s_S = (T *)(smem + a.off_s);             // [2][BN][SLD]
    float *s_x = (float *)(smem + a.off_x);     // [3][nch][wt_max]
    __shared__ int s_lo[NSEG], s_hi[NSEG], s_base[NSEG + 1];
    __shared__ int s_win;

    const Params &p = a.p;
    const int t = threadIdx.x;
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
    const int K = p.K, L_in = p.L_in, L_out = p.L_out;
    const int GK = p.G * K;
    const T *__restrict__ off = (const T *)p.off;
    const T *__restrict__ mask = (const T *)p.mask;

    // ---- column tile geometry
    const int64_t n_end = (tl.n0 + BN < a.N) ? tl.n0 + BN : a.N;
    tl.b_first = (int)(tl.n0 / L_out);
    tl.nseg = (int)((n_end - 1) / L_out) - tl.b_first + 1;
    bool win = (a.wt_max > 0) && (tl.nseg <= NSEG);
    if (t < NSEG) {
        s_lo[t] = INT_MAX;
        s_hi[t] = INT_MIN;
    }
    __syncthreads();

    // ---- position table, pass 1: left neighbours, fractions, mask; per-segment extent
    {
        int lo[NSEG], hi[NSEG];
#pragma unroll
        for (int q = 0; q < NSEG; ++q) {
            lo[q] = INT_MAX;
            hi[q] = INT_MIN;
        }
        constexpr int TB = 4;  // entries per thread per batch of loads
        for (int e0 = 0; e0 < GK * BN; e0 += NTT * TB) {
            float ov[TB], mv[TB];
            int64_t oi[TB];
            bool ok[TB];
#pragma unroll
            for (int q = 0; q < TB; ++q) {
                const int e = e0 + t + NTT * q;
                const int n = e % BN, gk = e / BN;
                const int g = gk / K, k = gk - g * K;
                const int64_t col = tl.n0 + n;
                ok[q] = e < GK * BN && col < a.N;
                const int b = (int)(col / L_out), l = (int)(col - (int64_t)b * L_out);
                oi[q] = ok[q] ? (((int64_t)b * p.G + g) * L_out + l) * K + k : 0;
            }
#pragma unroll
            for (int q = 0; q < TB; ++q) {
                ov[q] = D::ld(off, oi[q]);
                mv[q] = MASK ? D::ld(mask, oi[q]) : 1.0f;
            }
#pragma unroll
            for (int q = 0; q < TB; ++q) {
                const int e = e0 + t + NTT * q;
                if (e >= GK * BN) continue;
                const int n = e % BN, gk = e / BN;
                const int k = gk % K;
                const int64_t col = tl.n0 + n;
                Pos ps = {0, 0.0f};
                if (ok[q]) {
                    const int b = (int)(col / L_out), l = (int)(col - (int64_t)b * L_out);
                    int i0;
                    split_position(ov[q], l * p.stride - p.padding + k * p.dilation, i0, ps.f);
                    ps.j = min(max(i0, -2), L_in);  // x~ reads zero at both neighbours beyond these bounds
                    const int sg = b - tl.b_first;
#pragma unroll
                    for (int z = 0; z < NSEG; ++z) {
                        lo[z] = (z == sg) ? min(lo[z], ps.j) : lo[z];
                        hi[z] = (z == sg) ? max(hi[z], ps.j) : hi[z];
                    }
                }
                s_tab[e] = ps;
                if (MASK) s_m[e] = ok[q] ? mv[q] : 0.0f;
            }
        }
        if (win) {
#pragma unroll
            for (int z = 0; z < NSEG; ++z) {
                for (int o = 32; o > 0; o >>= 1) {
                    lo[z] = min(lo[z], __shfl_xor(lo[z], o));
                    hi[z] = max(hi[z], __shfl_xor(hi[z], o));
                }
                if ((t & 63) == 0 && z < tl.nseg) {
                    atomicMin(&s_lo[z], lo[z]);
                    atomicMax(&s_hi[z], hi[z]);
                }
            }
        }
    }
    __syncthreads();
    if (t == 0) {
        int base = 0;
        for (int s = 0; s < (win ? tl.nseg : 0); ++s) {
            s_base[s] = base;
            base += s_hi[s] + 2 - s_lo[s];
        }
        s_base[win ? tl.nseg : 0] = base;
        s_win = win && base <= a.wt_max;
    }
    __syncthreads();
    tl.win = s_win;
    tl.WT = tl.win ? s_base[tl.nseg] : 0;
    // ---- pass 2 (windowed): left neighbour -> index into the tile's window row
    if (tl.win) {
        for (int e = t; e < GK * BN; e += NTT) {
            const int64_t col = tl.n0 + e % BN;
            if (col < a.N) {
                const int s = (int)(col / L_out) - tl.b_first;
                s_tab[e].j += s_base[s] - s_lo[s];
            }
        }
    }
    __syncthreads();  // position table complete

    if (t < NTM) {
        mfma_role<Tr, VEC_W>(a, tl, s_w, s_S);
    } else if (tl.win) {
        sampler_role<Tr, MASK, true, NCHM, SLOTM>(a, tl, s_tab, s_m, s_S, s_x, s_lo, s_base);
    } else {
        sampler_role<Tr, MASK, false, 1, 1>(a, tl, s_tab, s_m, s_S, s_x, s_lo, s_base);
    }
}

// Sum of the split partial tiles (in split order), plus bias, into out.
// One thread per 4-float vector of a partial tile: vector (q4, t) holds what
// MFMA thread t of every split's workgroup kept in its register group q4, so
// the register-order layout maps back to (row, column) exactly as in the
// direct epilogue.
template <class Tr>
__global__ void __launch_bounds__(256) k_split_reduce(MfmaArgs a) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    constexpr int MB = Tr::MB, NB = Tr::NB, BM = Geo<Tr>::BM, BN = Geo<Tr>::BN;
    constexpr int NQ = MB * NB * 4;
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
    const int64_t col = (int64_t)tn * BN + 32 * (NB * wv + nb) + li;
    if (col >= a.N) return;
    const int L_out = p.L_out, M = p.C_out;
    const int b = (int)(col / L_out);
    const int l = (int)(col - (int64_t)b * L_out);
    const T *__restrict__ bias = (const T *)p.bias;
    T *ob = (T *)p.out + (int64_t)b * M * L_out + l;
#pragma unroll
    for (int z = 0; z < 4; ++z) {
        const int q = qq + z;
        const int row = tm * BM + 32 * mb + 8 * (q >> 2) + 4 * lh + (q & 3);
        if (row < M) D::st(ob, (int64_t)row * L_out, tot[z] + (bias ? D::ld(bias, row) : 0.0f));
    }
}

template <class Tr>
void plan_for(const Params &p, int num_cus, MfmaPlan &pl) {
    using T = typename Tr::T;
    constexpr int BM = Geo<Tr>::BM, BN = Geo<Tr>::BN;
    pl.bm = BM;
    pl.bn = BN;
    pl.bk = BK;
    pl.threads = NTT;
    const int64_t N = (int64_t)p.B * p.L_out;
    pl.tiles_m = (p.C_out + BM - 1) / BM;
    pl.tiles_n = (int)((N + BN - 1) / BN);
    pl.chunks = (p.Kred + BK - 1) / BK;

    // LDS: position table (+ mask), row descriptors, weight tiles, sample
    // tiles, x windows
    const size_t tab = (size_t)p.G * p.K * BN * sizeof(Pos);
    const size_t msk = p.mask ? (size_t)p.G * p.K * BN * 4 : 0;
    const size_t rows = 0;
    const size_t wtile = 2 * (size_t)BM * BK * sizeof(T);
    const size_t stile = 2 * (size_t)BN * Tr::SLD * sizeof(T);
    const int nch = (BK - 1) / p.K + 2;
    // window staging variant (compile-time register budget): K >= 8 -> at
    // most 5 channel rows x 4 slots; 3 <= K < 8 -> 12 rows x 2 slots; K < 3 ->
    // no window (gather from global memory).
    int slotm = 0;
    if (p.K >= 8) {
        pl.variant = 0;
        slotm = 4;
    } else if (p.K >= 3) {
        pl.variant = 1;
        slotm = 2;
    } else {
        pl.variant = 2;
        slotm = 0;
    }
    // window capacity: the tile's grid span per batch segment plus a margin
    // for the offsets' spread, within the staging slots
    const int seg_possible = (p.L_out % BN == 0) ? 1 : (int)std::min<int64_t>(NSEG, (BN - 1) / p.L_out + 2);
    const int64_t span = (int64_t)(std::min<int64_t>(BN, p.L_out) - 1) * p.stride +
                         (int64_t)(p.K - 1) * p.dilation + 2 + 64;
    int64_t wt = span * seg_possible;
    if (wt > (int64_t)slotm * NTS) wt = (int64_t)slotm * NTS;
    if (wt < 64) wt = 0;  // too little room for a window: gather from global memory
    const size_t lds_cap = 160 * 1024 - 1024;
    size_t xwin = 3 * (size_t)nch * wt * 4;
    if (tab + msk + rows + wtile + stile + xwin > lds_cap) {
        wt = 0;
        xwin = 0;
    }
    pl.nch = nch;
    pl.wt_max = (int)wt;
    pl.off_mask = (int)tab;
    pl.off_row = (int)((tab + msk + 15) & ~(size_t)15);
    pl.off_w = (int)(pl.off_row + rows);
    pl.off_s = (int)(pl.off_w + wtile);
    pl.off_x = (int)(pl.off_s + stile);
    pl.lds_bytes = pl.off_x + xwin;
    if (pl.lds_bytes > lds_cap) {
        pl.ok = false;
        return;
    }

    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
    const int64_t slots = num_cus;  // one 8-wave workgroup per CU
    // Split the reduction when the tiles alone leave the CUs badly filled:
    // pick the split count minimising (waves of workgroups) x (chunks per
    // workgroup + pipeline fill).
    int best_s = 1;
    double best = 1e300;
    const int s_max = pl.chunks < 16 ? pl.chunks : 16;
    for (int s = 1; s <= s_max; ++s) {
        const int64_t units = tiles * s;
        if (units > ((int64_t)1 << 30)) break;
        const int64_t waves = (units + slots - 1) / slots;
        const double cost = (double)waves * ((pl.chunks + s - 1) / s + 2) * (s > 1 ? 1.03 : 1.0);
        if (cost < best - 1e-9) {
            best = cost;
            best_s = s;
        }
    }
    pl.splits = best_s;
    pl.blocks = tiles * best_s;
    pl.ws_bytes = best_s > 1 ? (size_t)tiles * best_s * BM * BN * 4 : 0;
}

template <class Tr>
hipError_t launch_for(const Params &p, const MfmaPlan &pl, hipStream_t stream) {
    MfmaArgs a;
    a.p = p;
    a.fd_K = make_fastdiv((uint32_t)p.K);
    a.fd_cpo = make_fastdiv((uint32_t)p.cpo);
    a.tiles_m = pl.tiles_m;
    a.tiles_n = pl.tiles_n;
    a.splits = pl.splits;
    a.chunks = pl.chunks;
    a.N = (int64_t)p.B * p.L_out;
    a.nch = pl.nch;
    a.wt_max = pl.wt_max;
    a.off_mask = pl.off_mask;
    a.off_row = pl.off_row;
    a.off_w = pl.off_w;
    a.off_s = pl.off_s;
    a.off_x = pl.off_x;
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
    a.partials = pl.splits > 1 ? (float *)p.ws : nullptr;
    const int vec_elems = 16 / (int)sizeof(typename Tr::T);
    const bool vec = (p.Kred % vec_elems == 0) && (((uintptr_t)p.w & 15) == 0);
    const dim3 grid((unsigned)pl.blocks), block(NTT);
#define DC1D_LAUNCH(V, MK, A, B) hipLaunchKernelGGL((k_mfma<Tr, V, MK, A, B>), grid, block, pl.lds_bytes, stream, a)
#define DC1D_LAUNCH_V(MK, A, B)           \
    do {                                  \
        if (vec)                          \
            DC1D_LAUNCH(true, MK, A, B);  \
        else                              \
            DC1D_LAUNCH(false, MK, A, B); \
    } while (0)
#define DC1D_LAUNCH_M(A, B)             \
    do {                                \
        if (p.mask)                     \
            DC1D_LAUNCH_V(true, A, B);  \
        else                            \
            DC1D_LAUNCH_V(false, A, B); \
    } while (0)
    if (pl.variant == 0)
        DC1D_LAUNCH_M(5, 4);
    else if (pl.variant == 1)
        DC1D_LAUNCH_M(12, 2);
    else
        DC1D_LAUNCH_M(1, 1);
#undef DC1D_LAUNCH_M
#undef DC1D_LAUNCH_V
#undef DC1D_LAUNCH
    if (pl.splits > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t vecs = tiles * (Geo<Tr>::BM * Geo<Tr>::BN / 4);
        hipLaunchKernelGGL((k_split_reduce<Tr>), dim3((unsigned)((vecs + 255) / 256)), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

MfmaPlan plan_mfma(const Params &p, int num_cus) {
    MfmaPlan pl = {};
    pl.ok = false;
    pl.name = "none";
    if (p.groups != 1) return pl;
    if (p.C_out < 32 || p.Kred < 16) return pl;  // too small to fill a tile: the direct kernel serves
    pl.ok = true;
    if (p.dtype == kF32) {
        pl.name = "mfma_f32";
        plan_for<TrF32>(p, num_cus, pl);
    } else {
        pl.name = "mfma_bf16";
        plan_for<TrBF16>(p, num_cus, pl);
    }
    return pl;
}

hipError_t launch_mfma(const Params &p, const MfmaPlan &pl, hipStream_t stream) {
    if (pl.blocks == 0) return hipSuccess;
    return p.dtype == kF32 ? launch_for<TrF32>(p, pl, stream) : launch_for<TrBF16>(p, pl, stream);
}

}  // namespace dc1d
