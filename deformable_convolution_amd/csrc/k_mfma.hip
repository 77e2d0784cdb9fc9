// k_mfma.hip -- fused deformable im2col + MFMA GEMM for groups == 1.
//
// The contraction out[b, co, l] = bias[co] + sum_r W[co, r] S[r, (b, l)] is a
// GEMM with M = C_out, N = B*L_out and reduction r = ci*K + k over the
// weight viewed as [C_out, C_in*K] (conv1d operator page, Description; the
// article's Step 3 weighted summation).  S is the deformable sample matrix
// (the article's Step 2): it never touches HBM.  Each workgroup owns a
// BM x BN output tile and a contiguous range of reduction chunks; per chunk
// of BK reduction rows it
//   1. gathers x at the two neighbours of every (row, column) sample
//      position -- the positions themselves (left index, right index and
//      the two interpolation weights with the mask folded in) were computed
//      once per workgroup into an LDS table indexed by (offset group, tap,
//      column);
//   2. runs the MFMAs of the previous chunk while those loads are in flight;
//   3. interpolates and writes the chunk's samples into an LDS tile.
// The weight operand goes straight from global memory (L2) into the MFMA A
// registers: every wave owns distinct output rows, so no weight value is
// loaded twice by one workgroup.
//
// Split reduction: when there are too few output tiles to fill the GPU, the
// reduction range is split over several workgroups.  Each writes its fp32
// partial tile into the workspace and bumps the tile's arrival counter; the
// last to arrive adds the partials in split order (so the result does not
// depend on arrival order), adds the bias, stores the output, and resets the
// counter to zero for the next call.
#include "dc1d_internal.h"

namespace dc1d {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

namespace {

constexpr int NT = 256;     // threads per workgroup (4 waves)
constexpr int GK_MAX = 32;  // offset groups x taps covered by the position table

struct TabEntry {
    int idx0, idx1;  // clamped in-row indices of the two neighbours
    float w0, w1;    // (1 - f) * m and f * m, or 0 for a neighbour outside [0, L_in)
};

struct MfmaArgs {
    Params p;
    FastDiv fd_K, fd_cpo;
    int tiles_m, tiles_n, splits, chunks;
    int64_t N;
    int *counters;
    float *partials;
};

__device__ __forceinline__ int remap_xcd(int u, int U) {
    // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
    // that consecutive unit ids (which share a weight slice) run on one XCD
    // and hit its L2.
    const int q = U >> 3, r = U & 7, xcd = u & 7, loc = u >> 3;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + loc;
}

// Build the per-workgroup position table: entry [g*K + k][n] for the tile's
// columns n0 .. n0 + BN - 1.
template <class D, int BN>
__device__ __forceinline__ void build_table(const MfmaArgs &a, int64_t n0, TabEntry *s_tab) {
    using T = typename D::T;
    const Params &p = a.p;
    const T *__restrict__ off = (const T *)p.off;
    const T *__restrict__ mask = (const T *)p.mask;
    const int GK = p.G * p.K;
    for (int e = threadIdx.x; e < GK * BN; e += NT) {
        const int n = e % BN;
        const int gk = e / BN;
        const int g = gk / p.K, k = gk - g * p.K;
        const int64_t col = n0 + n;
        TabEntry te = {0, 0, 0.0f, 0.0f};
        if (col < a.N) {
            const int b = (int)(col / p.L_out), l = (int)(col - (int64_t)b * p.L_out);
            const int64_t oi = (((int64_t)b * p.G + g) * p.L_out + l) * p.K + k;
            const float m = mask ? D::ld(mask, oi) : 1.0f;
            int i0;
            float f;
            split_position(D::ld(off, oi), l * p.stride - p.padding + k * p.dilation, i0, f);
            const bool v0 = i0 >= 0 && i0 < p.L_in;
            const bool v1 = i0 + 1 >= 0 && i0 + 1 < p.L_in;
            te.idx0 = v0 ? i0 : 0;
            te.idx1 = v1 ? i0 + 1 : 0;
            te.w0 = v0 ? (1.0f - f) * m : 0.0f;
            te.w1 = v1 ? f * m : 0.0f;
        }
        s_tab[e] = te;
    }
}

// ---------------------------------------------------------------------------
// fp32: v_mfma_f32_32x32x2_f32.  Lane (i = lane % 32, h = lane / 32) feeds
// A[i][h] and B[h][i]; the 32x32 result sits in 16 registers per lane, row
// 8*(q/4) + 4*h + q%4, column i.

constexpr int F_BM = 128, F_BN = 64, F_BK = 32;
constexpr int F_SLD = F_BK + 4;  // padded LDS row of the sample tile [BN][SLD]

template <bool VEC_W>
__global__ void __launch_bounds__(NT, 2) k_mfma_f32(MfmaArgs a) {
    __shared__ TabEntry s_tab[GK_MAX * F_BN];
    __shared__ __attribute__((aligned(16))) float s_S[2][F_BN * F_SLD];
    __shared__ int s_last;

    const Params &p = a.p;
    const int t = threadIdx.x;
    const int U = a.tiles_m * a.tiles_n * a.splits;
    const int u = remap_xcd(blockIdx.x, U);
    const int tn = u % a.tiles_n;
    const int rest = u / a.tiles_n;
    const int sp = rest % a.splits;
    const int tm = rest / a.splits;
    const int m0 = tm * F_BM;
    const int64_t n0 = (int64_t)tn * F_BN;
    const int c_begin = (int)((int64_t)sp * a.chunks / a.splits);
    const int c_end = (int)((int64_t)(sp + 1) * a.chunks / a.splits);
    const int M = p.C_out, Kred = p.Kred, K = p.K, L_in = p.L_in;

    build_table<F32, F_BN>(a, n0, s_tab);

    // sampler role: column sn, rows 8*srg .. 8*srg + 7 of each chunk
    const int sn = t % F_BN, srg = t / F_BN;
    const int64_t scol = n0 + sn;
    const bool scol_ok = scol < a.N;
    const float *__restrict__ xb =
        (const float *)p.x + (scol_ok ? (scol / p.L_out) * (int64_t)p.C_in * L_in : 0);

    // MFMA role: wave wv owns rows m0 + 32*wv .. +31
    const int wv = t / 64, lane = t % 64, li = lane % 32, lh = lane / 32;
    const int am = m0 + 32 * wv + li;
    const float *__restrict__ wrow = (const float *)p.w + (int64_t)(am < M ? am : M - 1) * Kred;

    float areg[16], anext[16];
    float xv0[8], xv1[8], ww0[8], ww1[8];
    f16v acc[2];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        acc[0][q] = 0.0f;
        acc[1][q] = 0.0f;
    }

    auto load_a = [&](int c, float(&ar)[16]) {
        const int rb = c * F_BK + 16 * lh;
        if (VEC_W && rb + 16 <= Kred) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const f4 q = *(const f4 *)(wrow + rb + 4 * v);
                ar[4 * v] = q[0];
                ar[4 * v + 1] = q[1];
                ar[4 * v + 2] = q[2];
                ar[4 * v + 3] = q[3];
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) ar[j] = (rb + j < Kred) ? wrow[rb + j] : 0.0f;
        }
        if (am >= M) {
#pragma unroll
            for (int j = 0; j < 16; ++j) ar[j] = 0.0f;
        }
    };

    // issue the x gathers of chunk c into registers
    auto gather = [&](int c) {
        const int r_first = c * F_BK + 8 * srg;
        int ci = (int)fdiv((uint32_t)r_first, a.fd_K);
        int k = r_first - ci * K;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int r = r_first + e;
            xv0[e] = 0.0f;
            xv1[e] = 0.0f;
            ww0[e] = 0.0f;
            ww1[e] = 0.0f;
            if (scol_ok && r < Kred) {
                const int g = (p.G == 1) ? 0 : (int)fdiv((uint32_t)ci, a.fd_cpo);
                const TabEntry te = s_tab[(g * K + k) * F_BN + sn];
                const float *xr = xb + (int64_t)ci * L_in;
                xv0[e] = xr[te.idx0];
                xv1[e] = xr[te.idx1];
                ww0[e] = te.w0;
                ww1[e] = te.w1;
            }
            if (++k == K) {
                k = 0;
                ++ci;
            }
        }
    };

    // interpolate the gathered values and store them in the sample tile
    auto finish = [&](float *dst) {
        f4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) lo[e] = fmaf(ww1[e], xv1[e], ww0[e] * xv0[e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) hi[e] = fmaf(ww1[e + 4], xv1[e + 4], ww0[e + 4] * xv0[e + 4]);
        f4 *d = (f4 *)(dst + sn * F_SLD + 8 * srg);
        d[0] = lo;
        d[1] = hi;
    };

    auto mfma_chunk = [&](const float *src, const float(&ar)[16]) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const f4 *bp = (const f4 *)(src + (32 * nb + li) * F_SLD + 16 * lh);
            const f4 b0 = bp[0], b1 = bp[1], b2 = bp[2], b3 = bp[3];
            const float bv[16] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3],
                                  b2[0], b2[1], b2[2], b2[3], b3[0], b3[1], b3[2], b3[3]};
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[j], bv[j], acc[nb], 0, 0, 0);
        }
    };

    __syncthreads();  // position table ready
    int buf = 0;
    if (c_begin < c_end) {
        load_a(c_begin, areg);
        gather(c_begin);
        finish(s_S[0]);
    }
    __syncthreads();
    for (int c = c_begin; c < c_end; ++c) {
        const bool more = c + 1 < c_end;
        if (more) {
            load_a(c + 1, anext);
            gather(c + 1);
        }
        mfma_chunk(s_S[buf], areg);
        if (more) finish(s_S[buf ^ 1]);
        __syncthreads();
        buf ^= 1;
#pragma unroll
        for (int j = 0; j < 16; ++j) areg[j] = anext[j];
    }

    // ---- epilogue
    const float *__restrict__ bias = (const float *)p.bias;
    float *__restrict__ out = (float *)p.out;
    if (a.splits > 1) {
        const int tile = tm * a.tiles_n + tn;
        f4 *part = (f4 *)(a.partials + ((int64_t)tile * a.splits + sp) * (F_BM * F_BN));
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) {
            const int nb = q4 >> 2, qq = (q4 & 3) * 4;
            f4 v = {acc[nb][qq], acc[nb][qq + 1], acc[nb][qq + 2], acc[nb][qq + 3]};
            part[q4 * NT + t] = v;
        }
        __threadfence();
        __syncthreads();
        if (t == 0) s_last = (atomicAdd(&a.counters[tile], 1) == a.splits - 1);
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        const f4 *part0 = (const f4 *)(a.partials + (int64_t)tile * a.splits * (F_BM * F_BN));
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) {
            f4 tot = part0[q4 * NT + t];
            for (int s2 = 1; s2 < a.splits; ++s2) tot += part0[(int64_t)s2 * (F_BM * F_BN / 4) + q4 * NT + t];
            const int nb = q4 >> 2, qq = (q4 & 3) * 4;
            acc[nb][qq] = tot[0];
            acc[nb][qq + 1] = tot[1];
            acc[nb][qq + 2] = tot[2];
            acc[nb][qq + 3] = tot[3];
        }
        if (t == 0) a.counters[tile] = 0;
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t col = n0 + 32 * nb + li;
        if (col >= a.N) continue;
        const int b = (int)(col / p.L_out);
        const int l = (int)(col - (int64_t)b * p.L_out);
        float *ob = out + (int64_t)b * M * p.L_out + l;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = m0 + 32 * wv + 8 * (q >> 2) + 4 * lh + (q & 3);
            if (row < M) ob[(int64_t)row * p.L_out] = acc[nb][q] + (bias ? bias[row] : 0.0f);
        }
    }
}

}  // namespace

MfmaPlan plan_mfma(const Params &p, int num_cus) {
    MfmaPlan pl = {};
    pl.ok = false;
    pl.name = "none";
    if (p.groups != 1 || p.G * p.K > GK_MAX || p.dtype != kF32) return pl;
    if (p.C_out < 32 || p.Kred < 16) return pl;  // too small for a 128-row tile: the direct kernel serves
    pl.ok = true;
    pl.name = "mfma_f32";
    pl.bm = F_BM;
    pl.bn = F_BN;
    pl.bk = F_BK;
    pl.threads = NT;
    const int64_t N = (int64_t)p.B * p.L_out;
    pl.tiles_m = (p.C_out + F_BM - 1) / F_BM;
    pl.tiles_n = (int)((N + F_BN - 1) / F_BN);
    pl.chunks = (p.Kred + F_BK - 1) / F_BK;
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
    // Split the reduction when the tiles alone leave the GPU's workgroup
    // slots (2 per CU) badly filled: pick the split count minimising
    // (waves of workgroups) x (chunks per workgroup).
    const int64_t slots = 2 * (int64_t)num_cus;
    int best_s = 1;
    double best = 1e300;
    const int s_max = pl.chunks < 16 ? pl.chunks : 16;
    for (int s = 1; s <= s_max; ++s) {
        const int64_t units = tiles * s;
        if (units > (int64_t)1 << 30) break;
        const int64_t waves = (units + slots - 1) / slots;
        const double cost = (double)waves * ((pl.chunks + s - 1) / s) * (s > 1 ? 1.03 : 1.0);
        if (cost < best - 1e-9) {
            best = cost;
            best_s = s;
        }
    }
    pl.splits = best_s;
    pl.blocks = tiles * best_s;
    pl.lds_bytes = 0;
    if (best_s > 1) {
        const size_t cnt = ((size_t)tiles * 4 + 255) & ~(size_t)255;
        pl.ws_bytes = cnt + (size_t)tiles * best_s * F_BM * F_BN * 4;
    } else {
        pl.ws_bytes = 0;
    }
    return pl;
}

hipError_t launch_mfma(const Params &p, const MfmaPlan &pl, hipStream_t stream) {
    if (pl.blocks == 0) return hipSuccess;
    MfmaArgs a;
    a.p = p;
    a.fd_K = make_fastdiv((uint32_t)p.K);
    a.fd_cpo = make_fastdiv((uint32_t)p.cpo);
    a.tiles_m = pl.tiles_m;
    a.tiles_n = pl.tiles_n;
    a.splits = pl.splits;
    a.chunks = pl.chunks;
    a.N = (int64_t)p.B * p.L_out;
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
    if (pl.splits > 1) {
        const size_t cnt = ((size_t)tiles * 4 + 255) & ~(size_t)255;
        a.counters = (int *)p.ws;
        a.partials = (float *)((char *)p.ws + cnt);
    } else {
        a.counters = nullptr;
        a.partials = nullptr;
    }
    const bool vec = (p.Kred % 4 == 0) && (((uintptr_t)p.w & 15) == 0);
    if (vec)
        hipLaunchKernelGGL(k_mfma_f32<true>, dim3((unsigned)pl.blocks), dim3(NT), 0, stream, a);
    else
        hipLaunchKernelGGL(k_mfma_f32<false>, dim3((unsigned)pl.blocks), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dc1d
