// k_mfma.hip -- planning for the fused deformable sampling + MFMA GEMM
// kernel (mfma_kernel.h): tile shape, window staging shape, LDS layout and
// split of the reduction; and the dispatch to the instantiating translation
// units (one per storage dtype and mask presence).
#include "mfma_kernel.h"

namespace dc1d {
namespace {

// Channel rows that one chunk of BK reduction rows r = ci*K + k can touch:
// the largest floor(last/K) - floor(first/K) + 1 over the chunks (the
// pattern repeats after K chunks).
int chunk_channels(const Params &p, int chunks) {
    int best = 0;
    const int period = chunks < p.K ? chunks : p.K;
    for (int c = 0; c < period; ++c) {
        const int64_t r0 = (int64_t)c * BK;
        const int64_t r1 = std::min<int64_t>(r0 + BK, p.Kred) - 1;
        best = std::max(best, (int)(r1 / p.K - r0 / p.K + 1));
    }
    return best;
}

// Split the reduction when the tiles alone leave the CUs badly filled: pick
// the split count minimising (waves of workgroups) x (chunks per workgroup +
// pipeline fill).
void plan_splits(int64_t tiles, int chunks, int num_cus, MfmaPlan &pl) {
    const int64_t slots = num_cus;  // one 8-wave workgroup per CU
    int best_s = 1;
    double best = 1e300;
    const int s_max = chunks < 16 ? chunks : 16;
    for (int s = 1; s <= s_max; ++s) {
        const int64_t units = tiles * s;
        if (units > ((int64_t)1 << 30)) break;
        const int64_t waves = (units + slots - 1) / slots;
        const double cost = (double)waves * ((chunks + s - 1) / s + 2) * (s > 1 ? 1.03 : 1.0);
        if (cost < best - 1e-9) {
            best = cost;
            best_s = s;
        }
    }
    pl.splits = best_s;
    pl.blocks = tiles * best_s;
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
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;

    // LDS: position table (+ mask), weight tiles, sample tiles, x windows
    const size_t tab = (size_t)p.G * p.K * BN * sizeof(Pos);
    const size_t msk = p.mask ? (size_t)p.G * p.K * BN * 4 : 0;
    const size_t wtile = 2 * (size_t)BM * BK * sizeof(T);
    const size_t stile = 2 * (size_t)BN * Tr::SLD * sizeof(T);
    const size_t lds_cap = 160 * 1024 - 1024;
    pl.off_mask = (int)tab;
    pl.off_w = (int)((tab + msk + 15) & ~(size_t)15);
    pl.off_s = (int)(pl.off_w + wtile);
    pl.off_x = (int)(pl.off_s + stile);
    const size_t fixed = (size_t)pl.off_x;
    if (fixed > lds_cap) {
        pl.ok = false;
        return;
    }

    // Window extent a tile is expected to need: the grid span of its BN
    // columns plus, per batch segment, the taps' reach, both neighbours and
    // a margin for the offsets' spread.
    const int64_t seg_possible =
        (p.L_out % BN == 0) ? 1 : std::min<int64_t>(NSEG, (BN - 1) / p.L_out + 2);
    // (+ 2 words per segment: windows staged in 16-byte words start and end
    // on whole words)
    constexpr int V = 16 / (int)sizeof(T);
    const bool vx = p.L_in % V == 0;
    const int64_t want = (int64_t)(std::min<int64_t>(BN, N) - 1) * p.stride +
                         seg_possible * ((int64_t)(p.K - 1) * p.dilation + 2 + 32 + (vx ? 2 * V : 0));

    // ---- channel-block order (preferred): the block size with the fewest
    // padded taps, then the largest whose window fits in LDS
    int best = -1, best_waste = INT_MAX, best_nkb = 0;
    const int slot = (int)std::min<int64_t>((want + 2 + NTS - 1) / NTS, 2);  // window row: slot*NTS
    if ((int64_t)p.K * p.C_out < ((int64_t)1 << 30)) {
        for (int cb : {32, 16, 8}) {
            const int tpc = BK / cb;
            if (p.cpo % (16 / tpc) != 0) continue;  // a thread's channels must share an offset group
            const int nkb = (p.K + tpc - 1) / tpc;
            const int waste = nkb * tpc - p.K;
            if (fixed + 2 * (size_t)cb * slot * NTS * sizeof(T) > lds_cap) continue;
            // staging lines per part: the block's window over its chunks, and
            // whole words per thread when staging in words
            const int need = std::max((cb * slot + nkb - 1) / nkb, vx ? V : 1);
            int pick = -1;
            for (int i = 0; i < kNumCbCombos; ++i)
                if (!kCbCombos[i].dw && kCbCombos[i].cb == cb && kCbCombos[i].slot == slot &&
                    kCbCombos[i].lpp >= need) {
                    pick = i;
                    break;
                }
            if (pick < 0) continue;
            if (waste < best_waste) {
                best = pick;
                best_waste = waste;
                best_nkb = nkb;
            }
        }
    }
    if (best >= 0) {
        pl.blocked = 1;
        pl.variant = best;
        pl.cb = kCbCombos[best].cb;
        pl.slot = kCbCombos[best].slot;
        pl.lpp = kCbCombos[best].lpp;
        pl.nkb = best_nkb;
        pl.ncb = (p.C_in + pl.cb - 1) / pl.cb;
        pl.nch = pl.cb;
        pl.wt_max = pl.slot * NTS;
        pl.chunks = pl.ncb * pl.nkb;
        pl.lds_bytes = fixed + 2 * (size_t)pl.cb * pl.wt_max * sizeof(T);
        // fp32 blocks of 8 channels x 4 taps with K % 4 == 0: the weights can
        // be read in place (when the pointer is 16-byte aligned)
        pl.variant_dw = -1;
        if (sizeof(T) == 4 && pl.cb == 8 && p.K % 4 == 0)
            for (int i = 0; i < kNumCbCombos; ++i)
                if (kCbCombos[i].dw && kCbCombos[i].cb == pl.cb && kCbCombos[i].slot == pl.slot &&
                    kCbCombos[i].lpp == pl.lpp)
                    pl.variant_dw = i;
        pl.wb_bytes = ((size_t)pl.nkb * p.C_out * pl.ncb * BK * sizeof(T) + 255) & ~(size_t)255;
        // bf16, blocks of 32 channels at one tap per chunk, rows staged in
        // words: the position-major window (k_mfma_cbt) when one of its
        // compiled sizes holds the expected extent and fits
        pl.tpos = 0;
        if (sizeof(T) == 2 && pl.cb == 32 && pl.nkb >= 2 && vx) {
            for (int i = 0; i < kNumTpos; ++i) {
                const size_t xw = 2 * (size_t)kTposOpts[i] * kTPitch * sizeof(T);
                if (kTposOpts[i] >= want + 2 && fixed + xw <= lds_cap) {
                    pl.tpos = kTposOpts[i];  // (wt_max stays the channel-major fallback's capacity)
                    pl.lds_bytes = std::max(pl.lds_bytes, fixed + xw);
                    break;
                }
            }
        }
        plan_splits(tiles, pl.chunks, num_cus, pl);
        pl.ws_bytes = pl.wb_bytes + (pl.splits > 1 ? (size_t)tiles * pl.splits * BM * BN * 4 : 0);
        // the one-wave-per-SIMD kernel (256 x 256 tiles) when its tiles alone
        // fill the GPU, a compiled tap count and window fit, and a tile spans
        // at most three batch segments (L_out >= 128).  With K odd it runs an
        // even number of blocks: an odd count gets a block of zero weights,
        // taken only when that adds at most a fifth (five blocks or more).
        pl.wide = 0;
        pl.fallback_blocks = pl.blocks;
        pl.fallback_splits = pl.splits;
        const int wncb = (p.C_in + 31) / 32;
        const bool pad = (p.K % 2 == 1) && (wncb % 2 == 1);
        if (sizeof(T) == 2 && p.cpo % 16 == 0 && vx && p.K >= 2 && p.K <= 4 && p.L_out >= 128 &&
            (!pad || wncb >= 5)) {
            const int64_t wtm = (p.C_out + 255) / 256, wtn = (N + 255) / 256;
            const int64_t segw = (p.L_out % 256 == 0) ? 1 : std::min<int64_t>(4, 255 / p.L_out + 2);
            const int64_t want_w = (std::min<int64_t>(256, N) - 1) * p.stride +
                                   segw * ((int64_t)(p.K - 1) * p.dilation + 2 + 32 + 16);
            if (wtm * wtn >= num_cus && wtm * wtn < ((int64_t)1 << 31)) {
                for (int i = 0, npos; (npos = wide_npos_option(i)) > 0; ++i) {
                    const size_t lds = wide_lds_bytes(npos);
                    if (npos >= want_w + 2 && lds <= lds_cap && wide_npos_compiled(npos, p.K)) {
                        pl.wide = npos;
                        pl.wide_tiles_m = (int)wtm;
                        pl.wide_tiles_n = (int)wtn;
                        pl.wide_lds = lds;
                        pl.wide_ncb = wncb + (pad ? 1 : 0);
                        pl.wide_wb_bytes =
                            ((size_t)p.K * p.C_out * pl.wide_ncb * BK * sizeof(T) + 255) & ~(size_t)255;
                        pl.blocks = wtm * wtn;
                        pl.threads = 256;
                        pl.splits = 1;
                        // the rearranged weights, then a byte per tile (gathered tiles)
                        pl.ws_bytes = std::max(pl.ws_bytes, pl.wide_wb_bytes + (size_t)(wtm * wtn));
                        break;
                    }
                }
            }
        }
        return;
    }

    // ---- reduction order ci-major (r = ci*K + k): any offset grouping
    pl.blocked = 0;
    pl.variant_dw = -1;
    pl.chunks = (p.Kred + BK - 1) / BK;
    const int nch = chunk_channels(p, pl.chunks);
    const int64_t slots_wanted = (want + NTS - 1) / NTS;
    // Smallest compiled staging shape with enough channel rows, then the
    // smallest slot count covering the extent (or the largest there is) that
    // fits in LDS; none: gather from global memory.
    int pick = -1;
    for (int i = 0; i < kNumCombos; ++i) {
        if (kCombos[i].nch < nch) continue;
        if (pick >= 0 && kCombos[i].nch != kCombos[pick].nch) break;
        const size_t xwin = 2 * (size_t)kCombos[i].nch * kCombos[i].slot * NTS * 4;
        if (fixed + xwin > lds_cap) break;
        pick = i;
        if (kCombos[i].slot >= slots_wanted) break;
    }
    // K < 3: a chunk spans too many channels for staging to pay; gather
    if (p.K < 3) pick = -1;
    if (pick < 0) {
        pl.variant = 0;  // any instantiation: its windowed role is not used
        pl.nch = 0;
        pl.wt_max = 0;
    } else {
        pl.variant = pick;
        pl.nch = kCombos[pick].nch;
        pl.wt_max = kCombos[pick].slot * NTS;
    }
    pl.lds_bytes = fixed + 2 * (size_t)pl.nch * pl.wt_max * 4;
    pl.wb_bytes = 0;
    plan_splits(tiles, pl.chunks, num_cus, pl);
    pl.ws_bytes = pl.splits > 1 ? (size_t)tiles * pl.splits * BM * BN * 4 : 0;
}

}  // namespace

MfmaPlan plan_mfma(const Params &p, int num_cus) {
    MfmaPlan pl = {};
    pl.ok = false;
    pl.name = "none";
    if (p.groups != 1) return pl;
    if (p.C_out < 32 || p.Kred < 16) return pl;  // too small to fill a tile: the direct kernel serves
    if ((int64_t)p.B * p.L_out >= ((int64_t)1 << 31)) return pl;  // columns are 32-bit in these kernels
    pl.ok = true;
    if (p.dtype == kF32) {
        pl.name = "mfma_f32";
        plan_for<TrF32>(p, num_cus, pl);
    } else {
        pl.name = "mfma_bf16";
        plan_for<TrBF16>(p, num_cus, pl);
    }
    if (pl.blocked) {
        static const char *const names[2][3] = {{"mfma_f32_cb8", "mfma_f32_cb16", "mfma_f32_cb32"},
                                                {"mfma_bf16_cb8", "mfma_bf16_cb16", "mfma_bf16_cb32"}};
        pl.name = pl.wide ? "mfma_bf16_wide"
                          : (pl.tpos ? "mfma_bf16_cb32t"
                                     : names[p.dtype == kF32 ? 0 : 1][pl.cb == 8 ? 0 : (pl.cb == 16 ? 1 : 2)]);
    }
    return pl;
}

// The plain GEMM's tiling: 256 x 128 tiles for the backward's contractions
// (out_mode 0), 128 x 128 for the packed layer's heads (out_mode 1, 2).
template <class Tr>
MfmaPlan gemm_plan(const Params &q, int num_cus) {
    constexpr int BM = Geo<Tr>::BM, BN = Geo<Tr>::BN;
    MfmaPlan pl = {};
    const int64_t N = (int64_t)q.B * q.L_out;
    pl.tiles_m = (q.C_out + BM - 1) / BM;
    pl.tiles_n = (int)((N + BN - 1) / BN);
    pl.chunks = (q.Kred + BK - 1) / BK;
    plan_splits((int64_t)pl.tiles_m * pl.tiles_n, pl.chunks, num_cus, pl);
    return pl;
}

template <class Tr>
size_t gemm_ws(const Params &q, int num_cus) {
    const MfmaPlan pl = gemm_plan<Tr>(q, num_cus);
    return pl.splits > 1 ? (size_t)pl.tiles_m * pl.tiles_n * pl.splits * Geo<Tr>::BM * Geo<Tr>::BN * 4 : 0;
}

template <class Tr, int OUT>
hipError_t launch_gemm_t(const Params &q, int64_t brow, int64_t bbatch, int num_cus, hipStream_t stream) {
    constexpr int BM = Geo<Tr>::BM, BN = Geo<Tr>::BN;
    const int64_t N = (int64_t)q.B * q.L_out;
    if (N == 0 || q.C_out == 0) return hipSuccess;
    const MfmaPlan pl = gemm_plan<Tr>(q, num_cus);
    MfmaArgs a = {};
    a.p = q;
    a.fd_Lout = make_fastdiv((uint32_t)q.L_out);
    a.fd_K = a.fd_cpo = a.fd_nkb = make_fastdiv(1);
    if (OUT != 0) a.fd_K = make_fastdiv((uint32_t)q.K);  // the head write-out's tap divisor
    a.tiles_m = pl.tiles_m;
    a.tiles_n = pl.tiles_n;
    a.splits = pl.splits;
    a.chunks = pl.chunks;
    a.N = N;
    constexpr int EPW = 16 / (int)sizeof(typename Tr::T);  // elements per 16-byte weight word
    a.vec_w = (q.Kred % EPW == 0) && (((uintptr_t)q.w & 15) == 0);
    a.off_w = 0;
    a.off_s = 2 * BM * BK * (int)sizeof(typename Tr::T);
    a.partials = pl.splits > 1 ? (float *)q.ws : nullptr;
    a.brow = brow;
    a.bbatch = bbatch;
    size_t lds = (size_t)a.off_s + 2 * (size_t)BN * Tr::SLD * sizeof(typename Tr::T);
    if (OUT != 0) {
        if (BN + 1 != kHeadLd || q.K < 1 || (int64_t)BN * q.K >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
        lds = std::max(lds, (size_t)BM * (kHeadLd + 1) * 4);  // the staged head tile and its biases
    }
    hipLaunchKernelGGL((k_gemm<Tr, OUT>), dim3((unsigned)pl.blocks), dim3(NTT), lds, stream, a);
    if (pl.splits > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
        const int64_t vecs = tiles * (BM * BN / 4);
        hipLaunchKernelGGL((k_split_reduce<Tr, OUT>), dim3((unsigned)((vecs + 255) / 256)), dim3(256), 0, stream,
                           a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const Params &q, int64_t brow, int64_t bbatch, int num_cus, hipStream_t stream) {
    return launch_gemm_t<TrBF16, 0>(q, brow, bbatch, num_cus, stream);
}

size_t gemm_bf16_workspace_bytes(const Params &q, int num_cus) { return gemm_ws<TrBF16>(q, num_cus); }

// out_mode 0 (the plain product): 256 x 128 tiles, or 128 x 128 ones when
// those fill the GPU without splitting the reduction and the larger ones
// would need a split -- the same MFMA work per CU, without the partial
// tiles' round trip and the reduction kernel.
bool gemm_f32_half(const Params &q, int num_cus) {
    return gemm_plan<TrF32>(q, num_cus).splits > 1 && gemm_plan<TrF32H>(q, num_cus).splits == 1;
}

size_t gemm_workspace_bytes(const Params &q, int out_mode, int num_cus) {
    if (out_mode == 0) return gemm_f32_half(q, num_cus) ? gemm_ws<TrF32H>(q, num_cus) : gemm_ws<TrF32>(q, num_cus);
    return gemm_ws<TrF32H>(q, num_cus);
}

hipError_t launch_gemm_f32(const Params &q, int64_t brow, int64_t bbatch, int out_mode, int num_cus,
                           hipStream_t stream) {
    switch (out_mode) {
    case 0:
        return gemm_f32_half(q, num_cus) ? launch_gemm_t<TrF32H, 0>(q, brow, bbatch, num_cus, stream)
                                         : launch_gemm_t<TrF32, 0>(q, brow, bbatch, num_cus, stream);
    case 1: return launch_gemm_t<TrF32H, 1>(q, brow, bbatch, num_cus, stream);
    case 2: return launch_gemm_t<TrF32H, 2>(q, brow, bbatch, num_cus, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mfma(const Params &p, const MfmaPlan &pl, hipStream_t stream) {
    if (pl.blocks == 0) return hipSuccess;
    if (pl.wide && ((uintptr_t)p.x & 15) == 0) return launch_mfma_wide(p, pl, stream);
    if (pl.wide) {  // x not 16-byte aligned: the channel-block kernel, on its own grid
        MfmaPlan q = pl;
        q.wide = 0;
        q.blocks = pl.fallback_blocks;
        q.splits = pl.fallback_splits;
        q.threads = NTT;
        return p.mask ? launch_mfma_bf16_mask(p, q, stream) : launch_mfma_bf16(p, q, stream);
    }
    if (p.dtype == kF32) return p.mask ? launch_mfma_f32_mask(p, pl, stream) : launch_mfma_f32(p, pl, stream);
    return p.mask ? launch_mfma_bf16_mask(p, pl, stream) : launch_mfma_bf16(p, pl, stream);
}

}  // namespace dc1d
