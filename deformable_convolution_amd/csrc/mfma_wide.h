// mfma_wide.h -- the bf16 fused deformable sampling + MFMA GEMM with one
// wave per SIMD doing both roles; included by k_mfma_wide.hip.
//
// The contraction and the reduction order are those of the channel-block
// kernel (mfma_kernel.h, blocks of CB = 32 input channels at one tap per
// chunk, the weights rearranged by k_weight_blocks); the tile and the split
// of the work between waves differ.  In the two-role kernels an MFMA wave
// holds 128 accumulator registers (two waves share each SIMD), a 128 x 64
// piece of the output, and reads 12 KB of operand fragments from LDS per
// 16 MFMAs; with the sampler wave's reads queued behind them, a chunk takes
// several times its MFMA time.  Here a workgroup is four waves, one per
// SIMD, each with the SIMD's whole register file:
//
//   * the tile is 256 output rows x 256 columns; wave w owns every row and
//     columns 64w .. 64w+63, i.e. 8 x 2 blocks of 32 x 32 fp32 accumulators
//     (256 registers, in the accumulation registers);
//   * per chunk of 32 reduction rows (32 channels of a block, one tap) a
//     lane computes the 16 samples of its two columns' MFMA B fragments
//     itself (channels 16h .. 16h+15, h the lane's half) from the
//     position-major x window in LDS -- the sample tile never exists; no
//     column is sampled twice, since each belongs to one wave;
//   * the weight tile [256][32] is staged in LDS by all threads (two
//     buffers, loaded into registers one chunk ahead) and each wave reads
//     its 8 row blocks' weight fragments from it, one row block ahead;
//   * the samples of chunk c+1 are computed between the MFMAs of chunk c:
//     the vector work is dealt out over the 32 MFMA slots in source order
//     and a scheduling fence after each slot keeps it there (left alone,
//     the compiler groups it ahead of the MFMAs, where it overlaps
//     nothing); one barrier per chunk;
//   * the MFMA takes the samples as its A operand and the weights as B, so
//     that a lane's accumulators are one output row and four consecutive
//     columns per register group: the epilogue adds the row's bias, and
//     stages each 32-row block through LDS so that eight lanes write one
//     row's 128 contiguous bytes.
//
// Interpolation: a sample is (1 - f) m x[j] + f m x[j+1] (m the mask, 1
// without one).  The weights w0 = (1 - f) m and w1 = f m are computed in
// fp32 once per column and tap; a sample is fma(w1, x[j+1], w0 x[j]) in
// fp32 (the bf16 inputs widened by a shift or a mask), rounded to bf16 for
// the MFMA.  Per channel pair: four widenings, two multiplies, two fmas and
// one conversion; the mask costs nothing more.  (The bf16 dot-product
// instruction would take fewer instructions, but it does not overlap the
// MFMAs the way plain vector arithmetic does.)
//
// The sample position and weights of each of a lane's two columns are held
// in registers for the K taps of its channels' offset group; the next
// block's are computed from its offsets (loaded a block ahead) in the
// second-to-last chunk of a block, after that chunk's samples.
// Windows: per batch segment of the tile, the input positions its taps can
// reach (extent computed once per tile from the offsets, as in
// setup_tile), position-major [NPOS][kTPitch] bf16, two buffers by block
// parity; staged in KT parts per block, each part loaded into registers two
// chunks before it is written, a thread's item being 8 positions of 4
// channels (four 16-byte loads of x, eight 8-byte LDS writes).  A tile
// whose offsets spread wider than the window samples global memory instead
// (bounds-checked, same arithmetic): the windowed instantiation (WIN) marks
// such a tile in a byte per tile and leaves it, and a second launch of the
// gathering instantiation computes the marked tiles only.  Keeping the two
// apart keeps the gather's addresses and loads out of the windowed loop's
// registers.
//
// The main loop has one back edge and no exit in mid-trip (the accumulators
// fill the accumulation registers exactly; a second path to the epilogue
// would need copies of them): a trip is one block when K is even and two
// blocks when K is odd, the prefetch register sets alternating with the
// chunk's parity at compile time.  With K odd the block count is even (an
// odd count is padded with a block of zero weights and zero samples).
// Every iteration stages, loads and samples unconditionally; past the last
// block the indices are clamped to real data and the writes land in window
// buffers no longer read.
//
// The chunk order (blocks outer, taps inner) and the MFMA grouping of a
// chunk's rows are the channel-block kernel's.
#pragma once

#include "mfma_kernel.h"

namespace dc1d {
namespace {

typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int kWT = 256;                      // threads per workgroup: four waves
constexpr int kWBM = 256, kWBN = 256;         // tile
constexpr int kWMB = kWBM / 32;               // 32-row blocks per wave (all 8)
constexpr int kWNB = 2;                       // 32-column blocks per wave
constexpr int kWSEG = 4;                      // batch segments a windowed tile may span
constexpr int kWV = kWBM * (BK / 8) / kWT;    // 16-byte weight words per thread per chunk (4)
constexpr int kWRV = kWT / (BK / 8);          // rows between one thread's weight words (64)
constexpr size_t kWideWLds = (size_t)2 * kWBM * BK * 2;  // the two weight tiles (bytes)
// the gathering instantiation's LDS: the weight tiles (the epilogue's
// staging rows fit in them)
constexpr size_t kWideGatherLds = kWideWLds;

struct WideArgs {
    Params p;
    FastDiv fd_Lout, fd_cpo;
    int tiles_m, tiles_n, ncb;  // ncb: blocks the loop runs (chunks = ncb * KT), even when KT is odd
    int64_t N;
    const uint16_t *wb;  // weights [KT][C_out][ncb][32] (k_weight_blocks, 32-channel blocks, one tap)
    uint8_t *gather;     // [tiles_m * tiles_n]: 1 where the tile's window does not fit (set by WIN)
};

// The (x[j], x[j+1]) pair of the channels in the low (SEL_LO) or high
// (SEL_HI) halves of two words of bf16 channel pairs at positions j, j+1.
constexpr uint32_t kSelLo = 0x05040100u, kSelHi = 0x07060302u;

// The weight tile's 16-byte words: word w of row r is stored at word
// w ^ ((r >> 2) & 3) of the row, so that the 16 rows an A-fragment read
// serves at once (4 rows per 256-byte bank cycle, 4 words each) fall on
// distinct banks.
__device__ __forceinline__ int wswz(int row, int word) { return word ^ ((row >> 2) & 3); }
__device__ __forceinline__ void wide_lds_a(const uint16_t *tile, int row, int h, TrBF16::Frag &a) {
    a.v[0] = *(const u4 *)(tile + row * BK + 8 * wswz(row, 2 * h));
    a.v[1] = *(const u4 *)(tile + row * BK + 8 * wswz(row, 2 * h + 1));
}


// f(integral_constant<int, I>) for I = 0, 1, ...: a loop whose index is a
// compile-time constant in every trip whatever the unroller's size limits
// (an index it left variable would put the register arrays in memory)
template <class F, int... I>
__device__ __forceinline__ void static_for(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}

// An empty statement that takes v in a vector register and gives it back:
// the value is computed before this point, which code motion (that would
// otherwise sink a result to its first use, an iteration later) leaves in
// place.
__device__ __forceinline__ void pin(uint32_t &v) { asm volatile("" : "+v"(v)); }


template <bool MASK, int NPOS, int KT, bool WIN>
__global__ void __launch_bounds__(kWT, 1) k_mfma_wide(WideArgs a) {
    using T = uint16_t;
    using Frag = TrBF16::Frag;
    constexpr int XBUF = NPOS * kTPitch;          // window buffer (elements)
    constexpr int NITEM = (NPOS / 8) * 8;         // staging items: (8-position word, 4-channel quad)
    constexpr int IPP = (NITEM + KT - 1) / KT;    // items per part (a block is staged in KT parts)
    static_assert(NPOS % 8 == 0 && IPP <= kWT, "at most one staging item per thread and part");
    static_assert(KT >= 2, "a block's window serves at least two chunks");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *s_w = (T *)smem;                            // [2][kWBM][BK], 16-byte words swizzled (wswz)
    T *s_x = (T *)(smem + 2 * kWBM * BK * 2);      // [2][NPOS][kTPitch]
    __shared__ int s_lo[kWSEG], s_hi[kWSEG], s_base[kWSEG + 1];
    __shared__ int s_win;

    const Params &p = a.p;
    const int t = threadIdx.x;
    const int wv = t / 64, lane = t % 64, li = lane % 32, lh = lane / 32;
    const int M = p.C_out, C_in = p.C_in, L_in = p.L_in, L_out = p.L_out, G = p.G;
    const int ncb = a.ncb, nchunk = ncb * KT;
    const T *__restrict__ x = (const T *)p.x;
    const T *__restrict__ off = (const T *)p.off;
    const T *__restrict__ mask = (const T *)p.mask;

    // ---- the tile
    const int U = a.tiles_m * a.tiles_n;
    const int unit = remap_xcd(blockIdx.x, U);
    // row tiles fastest: the row tiles of one column block run side by side
    // on one XCD and share its x windows (and offsets) in that XCD's L2; the
    // weight slices are far smaller than x
    const int tm = unit % a.tiles_m, tn = unit / a.tiles_m;
    const int m0 = tm * kWBM;
    const int n0 = tn * kWBN;  // N < 2^31: 32-bit column arithmetic
    const int n_end = (int)min((int64_t)n0 + kWBN, a.N);
    const int b_first = (int)fdiv((uint32_t)n0, a.fd_Lout);
    const int nseg = (int)fdiv((uint32_t)(n_end - 1), a.fd_Lout) - b_first + 1;
    if (!WIN && a.gather[unit] == 0) return;  // computed by the windowed launch

    // ---- weight staging (all threads): word v of thread t is row prow + kWRV*v, 16-byte word ppart.
    // Rows past C_out repeat row C_out - 1: they feed only accumulator rows
    // that are not stored.
    const int prow = t / (BK / 8), ppart = t % (BK / 8);
    const T *__restrict__ wrow = a.wb + (int64_t)ppart * 8;
    int64_t wro[kWV];  // element offset of each word's row
#pragma unroll
    for (int v = 0; v < kWV; ++v) wro[v] = (int64_t)min(m0 + prow + kWRV * v, M - 1) * ncb * BK;
    auto wbase = [&](int cw) {
        const int cb = (int)((uint32_t)cw / (uint32_t)KT), kb = cw - cb * KT;
        return wrow + ((int64_t)kb * M * ncb + cb) * BK;
    };
    auto fetch_w = [&](int cw, u4 (&wreg)[kWV]) {
        const T *base = wbase(cw);
#pragma unroll
        for (int v = 0; v < kWV; ++v) wreg[v] = *(const u4 *)(base + wro[v]);
    };
    T *const wdst = s_w + prow * BK + 8 * wswz(prow, ppart);
    auto commit_w = [&](int cw, const u4 (&wreg)[kWV]) {
        T *d0 = wdst + (cw & 1) * kWBM * BK;
#pragma unroll
        for (int v = 0; v < kWV; ++v) *(u4 *)(d0 + v * kWRV * BK) = wreg[v];
    };
    // the weight tile of chunk 0 (independent of everything below)
    u4 wr[kWV];
    fetch_w(0, wr);

    // ---- window extent: thread t reads every offset of column n0 + t
    if (WIN && t < kWSEG) {
        s_lo[t] = INT_MAX;
        s_hi[t] = INT_MIN;
    }
    if (WIN) {
        const int colx = n0 + t;
        const bool cok = colx < n_end;
        const int bx = cok ? (int)fdiv((uint32_t)colx, a.fd_Lout) : b_first;
        const int lx = cok ? colx - bx * L_out : 0;
        const int sgx = bx - b_first;
        int lo = INT_MAX, hi = INT_MIN;
        if (cok) {
            const int64_t ob = ((int64_t)bx * G * L_out + lx) * KT;
            const int64_t gs = (int64_t)L_out * KT;
            const int grid0 = lx * p.stride - p.padding;
            const int GK = G * KT;
            constexpr int EB = 16;  // offsets loaded per batch
            for (int e0 = 0; e0 < GK; e0 += EB) {
                float ov[EB];
#pragma unroll
                for (int q = 0; q < EB; ++q) {
                    const int e = min(e0 + q, GK - 1);
                    const int g = e / KT, k = e - g * KT;
                    ov[q] = BF16::ld(off, ob + g * gs + k);
                }
#pragma unroll
                for (int q = 0; q < EB; ++q) {
                    const int e = e0 + q;
                    const int k = e % KT;
                    int i0;
                    float f;
                    split_position(ov[q], grid0 + k * p.dilation, tap_range(p, k), i0, f);
                    const int j = min(max(i0, -2), L_in);
                    if (e < GK) {
                        lo = min(lo, j);
                        hi = max(hi, j);
                    }
                }
            }
        }
        __syncthreads();  // s_lo / s_hi initialised
        if (nseg <= kWSEG) {
#pragma unroll
            for (int z = 0; z < kWSEG; ++z) {
                int zl = (z == sgx) ? lo : INT_MAX, zh = (z == sgx) ? hi : INT_MIN;
                for (int o = 32; o > 0; o >>= 1) {
                    zl = min(zl, __shfl_xor(zl, o));
                    zh = max(zh, __shfl_xor(zh, o));
                }
                if (lane == 0 && z < nseg && zl <= zh) {
                    atomicMin(&s_lo[z], zl);
                    atomicMax(&s_hi[z], zh);
                }
            }
        }
        __syncthreads();
        if (t == 0) {
            int base = 0;
            const bool fits = nseg <= kWSEG;
            for (int z = 0; z < (fits ? nseg : 0); ++z) {
                // segments start and end on whole 16-byte words of x (L_in is a multiple of 8)
                s_lo[z] &= -8;
                const int len = (s_hi[z] + 2 - s_lo[z] + 7) & -8;
                s_base[z] = base;
                base += len;
            }
            s_base[fits ? nseg : 0] = base;
            // two positions of slack past the last one (the right neighbour's row)
            s_win = fits && base + 2 <= NPOS;
        }
        __syncthreads();
    }
    if (WIN && t == 0) a.gather[unit] = !s_win;
    if (WIN && !s_win) return;  // left to the gathering launch
    constexpr bool win = WIN;
    const int WT = win ? s_base[nseg] : 0;

    // ---- this lane's two columns
    int cb_b[kWNB], cb_l[kWNB], shift[kWNB];
    bool cok[kWNB];
#pragma unroll
    for (int nb = 0; nb < kWNB; ++nb) {
        const int col = n0 + 64 * wv + 32 * nb + li;
        cok[nb] = col < n_end;
        cb_b[nb] = cok[nb] ? (int)fdiv((uint32_t)col, a.fd_Lout) : b_first;
        cb_l[nb] = cok[nb] ? col - cb_b[nb] * L_out : 0;
        const int sg = cb_b[nb] - b_first;
        shift[nb] = (win && cok[nb]) ? s_base[sg] - s_lo[sg] : 0;
    }
    // positions (window rows, or x positions when gathering) and the
    // interpolation weights of the lane's columns for the K taps of one
    // offset group; the raw offsets (and mask) of the next block wait in
    // registers
    float raw_o[kWNB][KT], raw_m[kWNB][KT];
    int pj[kWNB][KT];
    float w0[kWNB][KT], w1[kWNB][KT];
    auto load_raw = [&](int cb) {
        const int g = (int)fdiv((uint32_t)min(cb * 32 + 16 * lh, C_in - 1), a.fd_cpo);
#pragma unroll
        for (int nb = 0; nb < kWNB; ++nb) {
            const int64_t ob = (((int64_t)cb_b[nb] * G + g) * L_out + cb_l[nb]) * KT;
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                raw_o[nb][k] = BF16::ld(off, ob + k);
                raw_m[nb][k] = MASK ? BF16::ld(mask, ob + k) : 1.0f;
            }
        }
    };
    auto split_one = [&](int nb, int k) {
                int i0;
                float f;
                split_position(raw_o[nb][k], cb_l[nb] * p.stride - p.padding + k * p.dilation, tap_range(p, k), i0,
                               f);
                // windowed: index into the window row; gathered: the left neighbour clamped to [-2, L_in]
                const int j = min(max(i0, -2), L_in);
                const int pjn = cok[nb] ? (win ? j + shift[nb] : j) : 0;
                uint32_t a1 = __float_as_uint(cok[nb] ? f * raw_m[nb][k] : 0.0f);
                uint32_t a0 = __float_as_uint(cok[nb] ? (1.0f - f) * raw_m[nb][k] : 0.0f);
                uint32_t jj = (uint32_t)pjn;
                pin(a0);
                pin(a1);
                pin(jj);
                w0[nb][k] = __uint_as_float(a0);
                w1[nb][k] = __uint_as_float(a1);
                pj[nb][k] = (int)jj;
    };
    auto split_raw = [&]() {
#pragma unroll
        for (int nb = 0; nb < kWNB; ++nb)
#pragma unroll
            for (int k = 0; k < KT; ++k) split_one(nb, k);
    };

    // ---- window staging.  Item it of a block: positions 8*(it>>3) .. +7 of
    // the window, channels 4*(it&7) .. +3 of the block; part q holds items
    // q*IPP .. q*IPP + IPP - 1; this thread's item of part q is q*IPP + js,
    // js = t (eight consecutive lanes on one position word's 64 contiguous
    // bytes of a window row)
    const int js = t;
    // xq: x at the item's position word, channel 4*(it&7) of block 0 (an
    // item outside the window, or past [0, L_in), reads position 0: in
    // bounds, and zeroed on the way to LDS where it is inside the window);
    // zw: some lane of the wave has an item inside the window that must be
    // zeros (wave-uniform)
    const T *xq[KT];
    int doff[KT];
    bool ival[KT], ihave[KT], zw[KT];
#pragma unroll
    for (int q = 0; q < KT; ++q) {
        const int it = q * IPP + js, cq = it & 7;
        ihave[q] = win && js < IPP && it < NITEM;
        const int jj = (it >> 3) * 8;
        const bool inwin = ihave[q] && jj < WT;
        int64_t io = 0;
        ival[q] = false;
        if (inwin) {
            int sg = 0;
            while (sg + 1 < nseg && s_base[sg + 1] <= jj) ++sg;
            const int pos = s_lo[sg] + (jj - s_base[sg]);
            ival[q] = pos >= 0 && pos < L_in;  // a word lies wholly inside [0, L_in) or outside
            io = (int64_t)(b_first + sg) * C_in * L_in + (ival[q] ? pos : 0);
        }
        xq[q] = x + io + (int64_t)(4 * cq) * L_in;
        doff[q] = (it >> 3) * 8 * kTPitch + 4 * cq;
        zw[q] = __builtin_amdgcn_ballot_w64(inwin && !ival[q]) != 0;
    }
    // (a block that is not whole -- the last one, a padding block, blocks
    // past the end -- reads clamped channels: in bounds, zeroed, never
    // sampled past the end)
    // channel c of the item's quad
    auto load_part_c = [&](int blk, int q, int c, u4 &xr) {
        if (!ihave[q]) return;
        if (blk * 32 + 32 <= C_in) {
            xr = *(const u4 *)(xq[q] + (int64_t)(blk * 32 + c) * L_in);
        } else {
            const int cq = (q * IPP + js) & 7;
            const int ci = min(blk * 32 + 4 * cq + c, C_in - 1);
            xr = *(const u4 *)(xq[q] - (int64_t)(4 * cq) * L_in + (int64_t)ci * L_in);
        }
    };
    auto load_part = [&](int blk, int q, u4 (&xr)[4]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) load_part_c(blk, q, c, xr[c]);
    };
    auto commit_part = [&](int blk, int q, const u4 (&xr)[4]) {
        if (!ihave[q]) return;
        T *dst = s_x + (blk & 1) * XBUF + doff[q];
        auto put = [&](const uint32_t (&c)[4][4]) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {  // positions 2d, 2d+1: dword d of each channel's word
                *(u2 *)(dst + (2 * d) * kTPitch) = u2{__builtin_amdgcn_perm(c[1][d], c[0][d], kSelLo),
                                                      __builtin_amdgcn_perm(c[3][d], c[2][d], kSelLo)};
                *(u2 *)(dst + (2 * d + 1) * kTPitch) = u2{__builtin_amdgcn_perm(c[1][d], c[0][d], kSelHi),
                                                          __builtin_amdgcn_perm(c[3][d], c[2][d], kSelHi)};
            }
        };
        uint32_t c[4][4];
        if (!zw[q] && blk * 32 + 32 <= C_in) {  // whole block, no zeros in this wave
#pragma unroll
            for (int ch = 0; ch < 4; ++ch)
#pragma unroll
                for (int d = 0; d < 4; ++d) c[ch][d] = xr[ch][d];
        } else {
            const int cq = (q * IPP + js) & 7;
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                const uint32_t keep = (ival[q] && blk * 32 + 4 * cq + ch < C_in) ? 0xffffffffu : 0u;
#pragma unroll
                for (int d = 0; d < 4; ++d) c[ch][d] = xr[ch][d] & keep;
            }
        }
        put(c);
    };
    // The part committed in iteration u (and loaded in u - 2): block B, part
    // q with u = (B - 1) * KT + q - 1.
    auto part_of = [&](int u, int &blk, int &q) {
        const int v = u + 1 + KT;  // = B * KT + q
        blk = (int)((uint32_t)v / (uint32_t)KT);
        q = v - blk * KT;
    };

    // ---- the samples of chunk (cb, k) for this lane's two columns: the two
    // rows' words (x[j] and x[j+1], channels 16h .. 16h+15), then the math
    u4 xv[kWNB][4];
    auto sample_reads_nb = [&](int cb, int k, int nb) {
        {
            if constexpr (WIN) {
                const T *xw = s_x + (cb & 1) * XBUF + __umul24((uint32_t)pj[nb][k], kTPitch) + 16 * lh;
                xv[nb][0] = *(const u4 *)xw;
                xv[nb][1] = *(const u4 *)(xw + 8);
                xv[nb][2] = *(const u4 *)(xw + kTPitch);
                xv[nb][3] = *(const u4 *)(xw + kTPitch + 8);
            } else {
                const int j = pj[nb][k];
                const T *xr = x + ((int64_t)cb_b[nb] * C_in) * L_in;
                const bool v0 = j >= 0 && j < L_in, v1 = j + 1 >= 0 && j + 1 < L_in;
                const int j0 = min(max(j, 0), L_in - 1), j1 = min(max(j + 1, 0), L_in - 1);
#pragma unroll
                for (int i = 0; i < 8; ++i) {  // channels 2i, 2i+1
                    const T *r0 = xr + (int64_t)min(cb * 32 + 16 * lh + 2 * i, C_in - 1) * L_in;
                    const T *r1 = xr + (int64_t)min(cb * 32 + 16 * lh + 2 * i + 1, C_in - 1) * L_in;
                    const uint32_t a0 = v0 ? r0[j0] : 0u, b0 = v0 ? r1[j0] : 0u;
                    const uint32_t a1 = v1 ? r0[j1] : 0u, b1 = v1 ? r1[j1] : 0u;
                    xv[nb][i >> 2][i & 3] = a0 | (b0 << 16);
                    xv[nb][2 + (i >> 2)][i & 3] = a1 | (b1 << 16);
                }
            }
        }
    };
    auto sample_reads = [&](int cb, int k) {
#pragma unroll
        for (int nb = 0; nb < kWNB; ++nb) sample_reads_nb(cb, k, nb);
    };
    // channel pair i (channels 2i, 2i+1 of the lane's 16) of column block nb
    // (x[j], x[j+1]) of the even (low halves) or odd (high halves) channel
    auto interp_even = [&](int k, int nb, uint32_t r0, uint32_t r1) {
        return fmaf(w1[nb][k], __uint_as_float(r1 << 16), w0[nb][k] * __uint_as_float(r0 << 16));
    };
    auto interp_odd = [&](int k, int nb, uint32_t r0, uint32_t r1) {
        return fmaf(w1[nb][k], __uint_as_float(r1 & 0xffff0000u), w0[nb][k] * __uint_as_float(r0 & 0xffff0000u));
    };
    auto sample_pair = [&](int k, int nb, int i, Frag &bo) {
        const uint32_t r0 = xv[nb][i >> 2][i & 3], r1 = xv[nb][2 + (i >> 2)][i & 3];
        const float s0 = interp_even(k, nb, r0, r1);
        const float s1 = interp_odd(k, nb, r0, r1);
        uint32_t r = pack_bf16x2(s0, s1);
        pin(r);
        bo.v[i >> 2][i & 3] = r;
    };
    // half hf of channel pair hf / 2: the even channel's sample (kept), or
    // the odd one's and the pair written to the fragment
    float sv[8 * kWNB];
    auto sample_half = [&](int k, int hf, Frag (&bo)[kWNB]) {
        const int pr = hf >> 1, nb = pr >> 3, i = pr & 7;
        const uint32_t r0 = xv[nb][i >> 2][i & 3], r1 = xv[nb][2 + (i >> 2)][i & 3];
        if ((hf & 1) == 0) {
            sv[pr] = interp_even(k, nb, r0, r1);
        } else {
            const float s1 = interp_odd(k, nb, r0, r1);
            uint32_t r = pack_bf16x2(sv[pr], s1);
            pin(r);
            bo[nb].v[i >> 2][i & 3] = r;
        }
    };
    auto sample_math = [&](int k, Frag (&bo)[kWNB]) {
#pragma unroll
        for (int nb = 0; nb < kWNB; ++nb)
#pragma unroll
            for (int i = 0; i < 8; ++i) sample_pair(k, nb, i, bo[nb]);
    };

    // ---- prologue: windows of block 0 and of block 1's first part, the
    // parts iterations 0 and 1 write, the positions of block 0's group and
    // the next block's offsets, the first weight tile, chunk 0's samples
    u4 xs[2][4];  // two parts in flight
    if constexpr (WIN) {
        u4 xp[KT + 1][4];
#pragma unroll
        for (int q = 0; q < KT; ++q) load_part(0, q, xp[q]);
        load_part(1, 0, xp[KT]);
#pragma unroll
        for (int q = 0; q < KT; ++q) commit_part(0, q, xp[q]);
        commit_part(1, 0, xp[KT]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int blk, q;
            part_of(u, blk, q);
            load_part(blk, q, xs[u]);
        }
    }
    load_raw(0);
    split_raw();
    load_raw(1);
    commit_w(0, wr);
    f16v acc[kWMB][kWNB];
#pragma unroll
    for (int mb = 0; mb < kWMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < kWNB; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;
    __syncthreads();  // windows, the first weight tile and the bias in LDS
    Frag bq[2][kWNB];  // B fragments: chunk u's in bq[u & 1]
    sample_reads(0, 0);
    sample_math(0, bq[0]);

    // ---- main loop: iteration (cb, k) = chunk u = cb*KT + k (par = u & 1
    // at compile time) multiplies chunk u and samples chunk u+1
    auto iteration = [&](int cb, int k, auto par_c) {
        constexpr int par = decltype(par_c)::value;
        const int u = cb * KT + k;
        // the window part loaded two iterations ago to LDS; then into
        // registers the weight tile of chunk u+1 (clamped past the end:
        // unused) and, after it, the window part for two iterations ahead
        // (so that the wait for the weights at this iteration's end leaves
        // the window loads in flight)
        if constexpr (WIN) {
            int blk, q;
            part_of(u, blk, q);
            commit_part(blk, q, xs[par]);
        }
        fetch_w(min(u + 1, nchunk - 1), wr);
        if constexpr (WIN) {
            int blk, q;
            part_of(u + 2, blk, q);
            load_part(blk, q, xs[par]);
        }
        // chunk u+1's rows (column block 0 now, 1 in slot 12): next tap of
        // this block, or the first tap of the next block
        const int cn = k == KT - 1 ? cb + 1 : cb, kn = k == KT - 1 ? 0 : k + 1;
        const T *tile = s_w + par * kWBM * BK;
        // 32 MFMA slots (row block mb = s / 4; within it (h, nb) = (0, 0),
        // (0, 1), (1, 0), (1, 1), so that consecutive MFMAs use different
        // accumulators); the weight fragments are read one row block ahead.
        // The vector work is dealt out over slots 4 .. 31 in source order and
        // a scheduling fence after each slot keeps it there: the 32 halves of
        // chunk u+1's channel pairs and, in the second-to-last chunk of a
        // block, the next block's positions and weights, written in place:
        // taps 0 .. K-2 over slots 4 .. 19 (this chunk's samples read tap
        // K-1 only), tap K-1 of column block 0 at slot 20 (after its last
        // sample at slot 17) and of column block 1 after the slots.
        constexpr int NS = 2 * kWMB * kWNB;
        constexpr int NEARLY = kWNB * (KT - 1);
        static_assert(4 + 15 * (NS - 4) / (16 * kWNB) < 20, "column block 0's samples end before slot 20");
        Frag af[2];
        wide_lds_a(tile, li, lh, af[0]);  // (before the sample rows: LDS reads return in order)
        sample_reads_nb(cn, kn, 0);
        static_for([&](auto slc) {
            constexpr int sl = decltype(slc)::value;
            constexpr int mb = sl >> 2, h = (sl >> 1) & 1, nb = sl & 1;
            if constexpr ((sl & 3) == 0 && mb + 1 < kWMB) wide_lds_a(tile, 32 * (mb + 1) + li, lh, af[(mb + 1) & 1]);
            if constexpr (sl == 12) sample_reads_nb(cn, kn, 1);
            // samples as the A operand, weights as B: the accumulator holds
            // the output transposed (lane = output row, registers = columns)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8, bq[par][nb].v[h]),
                                                                  __builtin_bit_cast(bf8, af[mb & 1].v[h]),
                                                                  acc[mb][nb], 0, 0, 0);
            static_for([&](auto hc) {
                constexpr int hf = decltype(hc)::value;
                if constexpr (4 + hf * (NS - 4) / (16 * kWNB) == sl) sample_half(kn, hf, bq[par ^ 1]);
            }, std::make_integer_sequence<int, 16 * kWNB>{});
            if (k == KT - 2) {
                static_for([&](auto ec) {
                    constexpr int e = decltype(ec)::value;
                    if constexpr (4 + e * 16 / NEARLY == sl) split_one(e / (KT - 1), e % (KT - 1));
                }, std::make_integer_sequence<int, NEARLY>{});
                if constexpr (sl == 20) split_one(0, KT - 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }, std::make_integer_sequence<int, NS>{});
        if (k == KT - 2) {
            split_one(1, KT - 1);  // (every sample of this chunk is taken)
            load_raw(cb + 2);
        }
        // weights of chunk u+1 to LDS (loaded at this iteration's start)
        commit_w(u + 1, wr);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    if constexpr (KT % 2 == 0) {
        for (int cb = 0; cb < ncb; ++cb) {
#pragma unroll
            for (int k = 0; k < KT; k += 2) {
                iteration(cb, k, P0{});
                iteration(cb, k + 1, P1{});
            }
        }
    } else {
        for (int cb = 0; cb < ncb; cb += 2) {  // ncb is even
#pragma unroll
            for (int k = 0; k + 1 < KT; k += 2) {
                iteration(cb, k, P0{});
                iteration(cb, k + 1, P1{});
            }
            iteration(cb, KT - 1, P0{});
#pragma unroll
            for (int k = 0; k + 1 < KT; k += 2) {
                iteration(cb + 1, k, P1{});
                iteration(cb + 1, k + 1, P0{});
            }
            iteration(cb + 1, KT - 1, P1{});
        }
    }

    // ---- epilogue: register q of accumulator (mb, nb) is output row
    // m0 + 32 mb + li, column n0 + 64 wv + 32 nb + 8 (q >> 2) + 4 lh + (q & 3):
    // four consecutive columns per q >> 2, stored with the row's bias as one
    // 8-byte word of bf16 (or element by element when rows are not whole
    // words)
    T *__restrict__ out = (T *)p.out;
    const bool m_full = m0 + kWBM <= M;
    float bv[kWMB];
    {
        const T *__restrict__ bias = (const T *)p.bias;
#pragma unroll
        for (int mb = 0; mb < kWMB; ++mb) bv[mb] = bias ? BF16::ld(bias, min(m0 + 32 * mb + li, M - 1)) : 0.0f;
    }
    if (L_out % 8 == 0 && ((uintptr_t)out & 15) == 0) {
        // Whole 16-byte words of output rows (a word never straddles a batch
        // nor the end of N: L_out, and so N, is a multiple of 8).  Each
        // 32-row block of the wave's 256 x 64 piece goes through LDS (the
        // weight tiles, free after the main loop's last barrier), bf16 with
        // the bias added: lane li writes its row's 64 columns, then eight
        // lanes write one row's 128 contiguous bytes, 4 stores per block.
        // Written straight from the accumulators, a store would cover 16
        // bytes of each of 32 rows.
        constexpr int PITCH = 64 + 8;  // staging row (elements): 144 bytes
        static_assert(4 * 32 * PITCH * 2 <= kWideWLds, "staging fits in the weight tiles");
        T *stg = (T *)smem + wv * 32 * PITCH;
        const int rl = lane / 8, cl = (lane % 8) * 8;
        const int col = n0 + 64 * wv + cl;
        const bool col_ok = col < n_end;
        const int b = (int)fdiv((uint32_t)(col_ok ? col : n0), a.fd_Lout);
        T *ob = out + (int64_t)b * M * L_out + (col - b * L_out);
        // LDS is shared by the wave's lanes only here; fences order each
        // lane's accesses around the exchange
        auto wave_sync = [] {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };
#pragma unroll
        for (int mb = 0; mb < kWMB; ++mb) {
            wave_sync();  // the previous block's reads are done
#pragma unroll
            for (int nb = 0; nb < kWNB; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *(u2 *)(stg + li * PITCH + 32 * nb + 8 * g + 4 * lh) =
                        u2{pack_bf16x2(acc[mb][nb][4 * g] + bv[mb], acc[mb][nb][4 * g + 1] + bv[mb]),
                           pack_bf16x2(acc[mb][nb][4 * g + 2] + bv[mb], acc[mb][nb][4 * g + 3] + bv[mb])};
            wave_sync();
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int r = 8 * it + rl;
                const int row = m0 + 32 * mb + r;
                const u4 word = *(const u4 *)(stg + r * PITCH + cl);
                if (col_ok && (m_full || row < M)) *(u4 *)(ob + (int64_t)row * L_out) = word;
            }
        }
        return;
    }
    if (L_out % 4 == 0 && ((uintptr_t)out & 7) == 0) {
        int64_t cbase[kWNB][4];
        bool cval[kWNB][4];
#pragma unroll
        for (int nb = 0; nb < kWNB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + 64 * wv + 32 * nb + 8 * g + 4 * lh;
                cval[nb][g] = col < n_end;
                const int b = (int)fdiv((uint32_t)(cval[nb][g] ? col : 0), a.fd_Lout);
                cbase[nb][g] = (int64_t)b * M * L_out + (col - b * L_out);
            }
#pragma unroll
        for (int mb = 0; mb < kWMB; ++mb) {
            const int row = m0 + 32 * mb + li;
            if (!m_full && row >= M) continue;
#pragma unroll
            for (int nb = 0; nb < kWNB; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    if (cval[nb][g])
                        *(u2 *)(out + cbase[nb][g] + (int64_t)row * L_out) =
                            u2{pack_bf16x2(acc[mb][nb][4 * g] + bv[mb], acc[mb][nb][4 * g + 1] + bv[mb]),
                               pack_bf16x2(acc[mb][nb][4 * g + 2] + bv[mb], acc[mb][nb][4 * g + 3] + bv[mb])};
        }
        return;
    }
#pragma unroll
    for (int nb = 0; nb < kWNB; ++nb)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int col = n0 + 64 * wv + 32 * nb + 8 * (q >> 2) + 4 * lh + (q & 3);
            if (col >= n_end) continue;
            const int b = (int)fdiv((uint32_t)col, a.fd_Lout);
            T *ob = out + (int64_t)b * M * L_out + (col - b * L_out);
#pragma unroll
            for (int mb = 0; mb < kWMB; ++mb) {
                const int row = m0 + 32 * mb + li;
                if (m_full || row < M) TrBF16::st1(ob + (int64_t)row * L_out, acc[mb][nb][q] + bv[mb]);
            }
        }
}

// Window capacities (positions) the wide kernel is compiled for (each with
// K = 2 .. 4 where NPOS <= 256 K: one staging item per thread and part; with
// K = 5 the unrolled two-block trip is too long for the accumulators to stay
// in registers).
constexpr int kWideNpos[] = {320, 448, 576, 768};
constexpr int kWideMaxK = 4;
constexpr int kNumWideNpos = sizeof(kWideNpos) / sizeof(kWideNpos[0]);

}  // namespace
}  // namespace dc1d
