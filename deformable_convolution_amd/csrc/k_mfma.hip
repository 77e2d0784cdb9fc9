// k_mfma.hip -- fused deformable im2col + MFMA GEMM for groups == 1.
//
// The contraction out[b, co, l] = bias[co] + sum_r W[co, r] S[r, (b, l)] is a
// GEMM with M = C_out, N = B*L_out and reduction r = ci*K + k over the
// weight viewed as [C_out, C_in*K] (conv1d operator page, Description; the
// article's Step 3 weighted summation).  S is the deformable sample matrix
// (the article's Step 2); it never touches HBM.  Each workgroup owns a
// BM x BN output tile and a contiguous range of reduction chunks of 32 rows.
// Per chunk it
//   1. gathers x at the two neighbours of each (row, column) sample -- the
//      positions (left index, right index, and the two interpolation weights
//      with the mask folded in) were computed once per workgroup into an LDS
//      table indexed by (offset group, tap, column);
//   2. runs the MFMAs of the previous chunk while those loads are in flight;
//   3. interpolates and writes the chunk's samples into an LDS tile in the
//      MFMA's B-operand order.
// The weight operand goes straight from global memory (L2) into the MFMA A
// registers: each wave owns distinct output rows, so no weight value is
// loaded twice by one workgroup.
//
// Two instantiations share the structure: fp32 storage on
// v_mfma_f32_32x32x2_f32, and bf16 storage on v_mfma_f32_32x32x16_bf16 (fp32
// accumulation, one round-to-nearest-even of the output).  In both, lane
// (i = lane % 32, h = lane / 32) of a wave holds, per chunk and 32-row
// block, the 16 weights W[m0 + i][r0 + 16h .. r0 + 16h + 15] and, per 32-column
// block, the 16 samples S[r0 + 16h .. + 15][n0 + i]; the MFMA sequence pairs
// them element by element, so every reduction row meets its own sample.
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
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int BK = 32;      // reduction rows per chunk
constexpr int GK_MAX = 24;  // offset groups x taps covered by the position table (LDS)

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

// ---- per-dtype MFMA traits --------------------------------------------------

struct TrF32 {
    using D = F32;
    using T = float;
    static constexpr int BM = 128, BN = 64, NT = 256;
    static constexpr int WM = 4, WN = 1;   // wave grid
    static constexpr int SLD = BK + 4;     // padded LDS row (elements) of the sample tile [BN][SLD]
    struct AFrag { float v[16]; };
    struct BFrag { float v[16]; };
    static __device__ __forceinline__ void load_a(const float *row, int rb, int Kred, bool vec, bool live,
                                                  AFrag &a) {
        if (vec && rb + 16 <= Kred) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 t = *(const f4 *)(row + rb + 4 * q);
                a.v[4 * q] = t[0]; a.v[4 * q + 1] = t[1]; a.v[4 * q + 2] = t[2]; a.v[4 * q + 3] = t[3];
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) a.v[j] = (rb + j < Kred) ? row[rb + j] : 0.0f;
        }
        if (!live) {
#pragma unroll
            for (int j = 0; j < 16; ++j) a.v[j] = 0.0f;
        }
    }
    static __device__ __forceinline__ void load_b(const float *src, BFrag &b) {
        const f4 *p = (const f4 *)src;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f4 t = p[q];
            b.v[4 * q] = t[0]; b.v[4 * q + 1] = t[1]; b.v[4 * q + 2] = t[2]; b.v[4 * q + 3] = t[3];
        }
    }
    static __device__ __forceinline__ void mma(const AFrag &a, const BFrag &b, f16v &acc) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], acc, 0, 0, 0);
    }
    // 8 samples -> LDS (two 16-byte stores)
    static __device__ __forceinline__ void store_samples(float *dst, const float (&v)[8]) {
        f4 lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
        ((f4 *)dst)[0] = lo;
        ((f4 *)dst)[1] = hi;
    }
    static __device__ __forceinline__ float to_out(float v) { return v; }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

struct TrBF16 {
    using D = BF16;
    using T = uint16_t;
    static constexpr int BM = 128, BN = 128, NT = 256;
    static constexpr int WM = 2, WN = 2;
    static constexpr int SLD = BK + 8;
    struct AFrag { u4 v[2]; };  // 16 bf16
    struct BFrag { u4 v[2]; };
    static __device__ __forceinline__ void load_a(const uint16_t *row, int rb, int Kred, bool vec, bool live,
                                                  AFrag &a) {
        if (vec && rb + 16 <= Kred) {
            a.v[0] = *(const u4 *)(row + rb);
            a.v[1] = *(const u4 *)(row + rb + 8);
        } else {
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t lo = (rb + 2 * j < Kred) ? row[rb + 2 * j] : 0u;
                const uint32_t hi = (rb + 2 * j + 1 < Kred) ? row[rb + 2 * j + 1] : 0u;
                w[j] = lo | (hi << 16);
            }
            a.v[0] = u4{w[0], w[1], w[2], w[3]};
            a.v[1] = u4{w[4], w[5], w[6], w[7]};
        }
        if (!live) {
            a.v[0] = u4{0, 0, 0, 0};
            a.v[1] = u4{0, 0, 0, 0};
        }
    }
    static __device__ __forceinline__ void load_b(const uint16_t *src, BFrag &b) {
        b.v[0] = ((const u4 *)src)[0];
        b.v[1] = ((const u4 *)src)[1];
    }
    static __device__ __forceinline__ void mma(const AFrag &a, const BFrag &b, f16v &acc) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8, a.v[s]),
                                                          __builtin_bit_cast(bf8, b.v[s]), acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void store_samples(uint16_t *dst, const float (&v)[8]) {
        u4 q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                pack_bf16x2(v[6], v[7])};
        *(u4 *)dst = q;
    }
};

// Build the per-workgroup position table: entry [g*K + k][n] for the tile's
// columns n0 .. n0 + BN - 1.
template <class Tr>
__device__ __forceinline__ void build_table(const MfmaArgs &a, int64_t n0, TabEntry *s_tab) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    const Params &p = a.p;
    const T *__restrict__ off = (const T *)p.off;
    const T *__restrict__ mask = (const T *)p.mask;
    const int GK = p.G * p.K;
    for (int e = threadIdx.x; e < GK * Tr::BN; e += Tr::NT) {
        const int n = e % Tr::BN;
        const int gk = e / Tr::BN;
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

template <class Tr, bool VEC_W>
__global__ void __launch_bounds__(Tr::NT, 2) k_mfma(MfmaArgs a) {
    using D = typename Tr::D;
    using T = typename Tr::T;
    constexpr int BM = Tr::BM, BN = Tr::BN, NT = Tr::NT, SLD = Tr::SLD;
    constexpr int TM = BM / Tr::WM, TN = BN / Tr::WN;  // per-wave tile
    constexpr int MB = TM / 32, NB = TN / 32;          // 32x32 blocks per wave
    constexpr int SPT = BN * 4 / NT;                   // sampled columns per thread (8 rows each)
    static_assert(Tr::WM * Tr::WN * 64 == NT, "wave grid");

    extern __shared__ TabEntry s_tab[];  // [G*K][BN], sized at launch
    __shared__ __attribute__((aligned(16))) T s_S[2][BN * SLD];
    __shared__ int s_last;

    const Params &p = a.p;
    const int t = threadIdx.x;
    const int U = a.tiles_m * a.tiles_n * a.splits;
    const int u = remap_xcd(blockIdx.x, U);
    const int tn = u % a.tiles_n;
    const int rest = u / a.tiles_n;
    const int sp = rest % a.splits;
    const int tm = rest / a.splits;
    const int m0 = tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    const int c_begin = (int)((int64_t)sp * a.chunks / a.splits);
    const int c_end = (int)((int64_t)(sp + 1) * a.chunks / a.splits);
    const int M = p.C_out, Kred = p.Kred, K = p.K, L_in = p.L_in;

    build_table<Tr>(a, n0, s_tab);

    // sampler role: columns sn + BN/SPT*q (q < SPT), rows 8*srg .. 8*srg + 7 of each chunk
    const int sn = t % (BN / SPT), srg = t / (BN / SPT);
    const T *__restrict__ xs[SPT];
    bool sok[SPT];
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
        const int64_t col = n0 + sn + (BN / SPT) * q;
        sok[q] = col < a.N;
        xs[q] = (const T *)p.x + (sok[q] ? (col / p.L_out) * (int64_t)p.C_in * L_in : 0);
    }

    // MFMA role
    const int wv = t / 64, lane = t % 64, li = lane % 32, lh = lane / 32;
    const int wm = wv % Tr::WM, wn = wv / Tr::WM;
    const T *__restrict__ wrow[MB];
    bool alive[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int am = m0 + wm * TM + 32 * mb + li;
        alive[mb] = am < M;
        wrow[mb] = (const T *)p.w + (int64_t)(alive[mb] ? am : M - 1) * Kred;
    }

    typename Tr::AFrag acur[MB], anext[MB];
    f16v acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;

    float xv0[SPT][8], xv1[SPT][8], ww0[SPT][8], ww1[SPT][8];

    auto load_a = [&](int c, typename Tr::AFrag (&af)[MB]) {
        const int rb = c * BK + 16 * lh;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) Tr::load_a(wrow[mb], rb, Kred, VEC_W, alive[mb], af[mb]);
    };

    // issue the x gathers of chunk c into registers
    auto gather = [&](int c) {
        const int r_first = c * BK + 8 * srg;
        const int ci0 = (int)fdiv((uint32_t)r_first, a.fd_K);
        const int k0 = r_first - ci0 * K;
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
            int ci = ci0, k = k0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = r_first + e;
                xv0[q][e] = 0.0f;
                xv1[q][e] = 0.0f;
                ww0[q][e] = 0.0f;
                ww1[q][e] = 0.0f;
                if (sok[q] && r < Kred) {
                    const int g = (p.G == 1) ? 0 : (int)fdiv((uint32_t)ci, a.fd_cpo);
                    const TabEntry te = s_tab[(g * K + k) * BN + sn + (BN / SPT) * q];
                    const T *xr = xs[q] + (int64_t)ci * L_in;
                    xv0[q][e] = D::ld(xr, te.idx0);
                    xv1[q][e] = D::ld(xr, te.idx1);
                    ww0[q][e] = te.w0;
                    ww1[q][e] = te.w1;
                }
                if (++k == K) {
                    k = 0;
                    ++ci;
                }
            }
        }
    };

    // interpolate the gathered values and store them in the sample tile
    auto finish = [&](T *dst) {
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = fmaf(ww1[q][e], xv1[q][e], ww0[q][e] * xv0[q][e]);
            Tr::store_samples(dst + (sn + (BN / SPT) * q) * SLD + 8 * srg, v);
        }
    };

    auto mfma_chunk = [&](const T *src, const typename Tr::AFrag (&af)[MB]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            typename Tr::BFrag bf;
            Tr::load_b(src + (wn * TN + 32 * nb + li) * SLD + 16 * lh, bf);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) Tr::mma(af[mb], bf, acc[mb][nb]);
        }
    };

    __syncthreads();  // position table ready
    int buf = 0;
    if (c_begin < c_end) {
        load_a(c_begin, acur);
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
        mfma_chunk(s_S[buf], acur);
        if (more) finish(s_S[buf ^ 1]);
        __syncthreads();
        buf ^= 1;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acur[mb] = anext[mb];
    }

    // ---- epilogue
    const T *__restrict__ bias = (const T *)p.bias;
    T *__restrict__ out = (T *)p.out;
    constexpr int NQ = MB * NB * 4;  // f4 groups per thread
    if (a.splits > 1) {
        const int tile = tm * a.tiles_n + tn;
        f4 *part = (f4 *)(a.partials + ((int64_t)tile * a.splits + sp) * (BM * BN));
#pragma unroll
        for (int q4 = 0; q4 < NQ; ++q4) {
            const int mb = q4 / (NB * 4), nb = (q4 / 4) % NB, qq = (q4 & 3) * 4;
            f4 v = {acc[mb][nb][qq], acc[mb][nb][qq + 1], acc[mb][nb][qq + 2], acc[mb][nb][qq + 3]};
            part[q4 * NT + t] = v;
        }
        __threadfence();
        __syncthreads();
        if (t == 0) s_last = (atomicAdd(&a.counters[tile], 1) == a.splits - 1);
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        const f4 *part0 = (const f4 *)(a.partials + (int64_t)tile * a.splits * (BM * BN));
#pragma unroll
        for (int q4 = 0; q4 < NQ; ++q4) {
            f4 tot = part0[q4 * NT + t];
            for (int s2 = 1; s2 < a.splits; ++s2) tot += part0[(int64_t)s2 * (BM * BN / 4) + q4 * NT + t];
            const int mb = q4 / (NB * 4), nb = (q4 / 4) % NB, qq = (q4 & 3) * 4;
            acc[mb][nb][qq] = tot[0];
            acc[mb][nb][qq + 1] = tot[1];
            acc[mb][nb][qq + 2] = tot[2];
            acc[mb][nb][qq + 3] = tot[3];
        }
        if (t == 0) a.counters[tile] = 0;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t col = n0 + wn * TN + 32 * nb + li;
        if (col >= a.N) continue;
        const int b = (int)(col / p.L_out);
        const int l = (int)(col - (int64_t)b * p.L_out);
        T *ob = out + (int64_t)b * M * p.L_out + l;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = m0 + wm * TM + 32 * mb + 8 * (q >> 2) + 4 * lh + (q & 3);
                if (row < M) D::st(ob, (int64_t)row * p.L_out, acc[mb][nb][q] + (bias ? D::ld(bias, row) : 0.0f));
            }
    }
}

template <class Tr>
void plan_for(const Params &p, int num_cus, MfmaPlan &pl) {
    pl.bm = Tr::BM;
    pl.bn = Tr::BN;
    pl.bk = BK;
    pl.threads = Tr::NT;
    const int64_t N = (int64_t)p.B * p.L_out;
    pl.tiles_m = (p.C_out + Tr::BM - 1) / Tr::BM;
    pl.tiles_n = (int)((N + Tr::BN - 1) / Tr::BN);
    pl.chunks = (p.Kred + BK - 1) / BK;
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
        if (units > ((int64_t)1 << 30)) break;
        const int64_t waves = (units + slots - 1) / slots;
        const double cost = (double)waves * ((pl.chunks + s - 1) / s) * (s > 1 ? 1.03 : 1.0);
        if (cost < best - 1e-9) {
            best = cost;
            best_s = s;
        }
    }
    pl.splits = best_s;
    pl.blocks = tiles * best_s;
    pl.lds_bytes = (size_t)p.G * p.K * Tr::BN * sizeof(TabEntry);
    if (best_s > 1) {
        const size_t cnt = ((size_t)tiles * 4 + 255) & ~(size_t)255;
        pl.ws_bytes = cnt + (size_t)tiles * best_s * Tr::BM * Tr::BN * 4;
    } else {
        pl.ws_bytes = 0;
    }
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
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
    if (pl.splits > 1) {
        const size_t cnt = ((size_t)tiles * 4 + 255) & ~(size_t)255;
        a.counters = (int *)p.ws;
        a.partials = (float *)((char *)p.ws + cnt);
    } else {
        a.counters = nullptr;
        a.partials = nullptr;
    }
    const int vec_elems = 16 / (int)sizeof(typename Tr::T);
    const bool vec = (p.Kred % vec_elems == 0) && (((uintptr_t)p.w & 15) == 0);
    if (vec)
        hipLaunchKernelGGL((k_mfma<Tr, true>), dim3((unsigned)pl.blocks), dim3(Tr::NT), pl.lds_bytes, stream, a);
    else
        hipLaunchKernelGGL((k_mfma<Tr, false>), dim3((unsigned)pl.blocks), dim3(Tr::NT), pl.lds_bytes, stream, a);
    return hipGetLastError();
}

}  // namespace

MfmaPlan plan_mfma(const Params &p, int num_cus) {
    MfmaPlan pl = {};
    pl.ok = false;
    pl.name = "none";
    if (p.groups != 1 || p.G * p.K > GK_MAX) return pl;
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
