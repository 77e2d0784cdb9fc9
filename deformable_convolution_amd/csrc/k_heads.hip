// k_heads.hip -- the packed layer's generator heads as a persistent MFMA
// kernel.
//
// The dc1d page's packed layer (section PackedDeformConv1d; the modulated
// form, section Modulation (DCNv2)) follows its depthwise trunk with
// pointwise heads: per column (b, l) of the trunk t [B][C][L], the offsets
// are off[b,g,l,k] = ob[g*K + k] + sum_c ow[g*K + k][c] t[b,c,l], and the
// mask the logistic sigmoid of the same form with the mask head's weights.
// Both are stored [B][G][L][K].  Here the heads are one matrix H [M][C]
// (the offset head's G*K rows, then the mask head's), M = G*K or 2*G*K.
//
// The contraction is short (C = 64 on the packed workload) and the output
// large (M values per column): the work is M*C multiply-adds and M stores
// per column.  Two workgroups per CU walk column tiles of 128 (one batch
// each: L is a multiple of 32 and tiles start at multiples of 128):
//
//   * wave w owns a slab of 32*K rows, i.e. 32 whole head groups -- the
//     rows of those groups' [l][k] runs -- and S = ceil(M / (32*K)) slabs
//     cover H; with S < 4 the waves also split the tile's four 32-column
//     blocks (wave w: slab w % S, column blocks from (w / S) * S);
//   * a lane keeps its slab's weights in registers for the whole kernel:
//     the MFMA's A operand, H[row][2*kk + h] for k-pair kk (h the lane's
//     half), zero past M and past C;
//   * the trunk tile [2*NKP][128] is staged in LDS (rows past C zero); two
//     workgroups share a CU, so that one's loads, write-out and barriers
//     overlap the other's MFMAs.  With fp32 storage the tile is computed
//     here from x (each thread four consecutive outputs of a channel, its
//     taps in k_trunk's order), so the trunk never reaches memory;
//   * per k-pair and column block one LDS read gives the B operand, shared
//     by the slab's K row blocks (v_mfma_f32_32x32x2_f32, fp32 throughout);
//   * the write-out stages each 32-column block of the slab through LDS in
//     [group][l][k] order -- the order of the destination runs -- adding
//     the bias, 16 groups at a time, and every lane stores 16-byte words of
//     the runs (the mask head's through the sigmoid).
#include "dc1d_internal.h"

#include <algorithm>

namespace dc1d {
namespace {

typedef float hf4 __attribute__((ext_vector_type(4)));
typedef float hf16 __attribute__((ext_vector_type(16)));

constexpr int kHT = 256;          // threads: four waves
constexpr int kHBN = 128;         // columns per tile
constexpr int kHSBP = kHBN + 32;  // trunk tile pitch (floats): rows 2kk and 2kk+1 on different banks

// the mask head's activation (the reciprocal instruction, within an ulp)
__device__ __forceinline__ float head_sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

template <int KT, int NKP, bool TRUNK>
__global__ void __launch_bounds__(kHT, 2) k_heads(HeadArgs a) {
    constexpr int CP = 2 * NKP;                // trunk rows staged (C padded)
    constexpr int NBV = CP * kHBN / 4 / kHT;   // 16-byte trunk words per thread per tile
    constexpr int SROWS = 32 * KT;             // rows per slab
    constexpr int STG = 16 * 32 * KT;          // staging floats per wave (16 groups x 32 columns x K)
    static_assert(NBV >= 1 && CP * kHBN % (4 * kHT) == 0, "whole trunk words per thread");
    extern __shared__ __attribute__((aligned(16))) float smem[];
    float *s_b = smem;                          // [CP][kHSBP]
    float *s_stg = smem + CP * kHSBP;           // [4][STG]
    float *s_bias = s_stg + 4 * STG;            // [4 * SROWS]

    const int t = threadIdx.x, wv = t / 64, lane = t % 64, li = lane % 32, lh = lane / 32;
    const int S = a.slabs, NBW = S;            // slabs (1, 2 or 4); column blocks per wave
    const int slab = wv % S, cb0 = (wv / S) * NBW;
    const int r0 = slab * SROWS;
    const int C = a.C, L = a.L, M = a.M, G = a.G;

    // the slab's weights (A operand) and the biases of every slab; with the
    // fused trunk the mask head's rows (from G*K on) come from w2 and bias2
    const int GK = G * KT;
    float aw[KT][NKP];
#pragma unroll
    for (int mb = 0; mb < KT; ++mb) {
        const int row = r0 + 32 * mb + li;
        const float *wr = (TRUNK && row >= GK) ? a.w2 + (int64_t)(row - GK) * C : a.w + (int64_t)row * C;
#pragma unroll
        for (int kk = 0; kk < NKP; ++kk) {
            const int c = 2 * kk + lh;
            aw[mb][kk] = (row < M && c < C) ? wr[c] : 0.0f;
        }
    }
    for (int r = t; r < 4 * SROWS; r += kHT) {
        const float *bs = (TRUNK && r >= GK) ? a.bias2 : a.bias;
        const int rb = (TRUNK && r >= GK) ? r - GK : r;
        s_bias[r] = (bs && r < M) ? bs[rb] : 0.0f;
    }

    // trunk words of tile T: word v = t + kHT*z is row v / 32, columns 4*(v % 32) .. +3
    hf4 br[NBV];
    auto fetch_b = [&](int T) {
        const int b = T / a.tiles_per_b, l0 = (T - b * a.tiles_per_b) * kHBN;
#pragma unroll
        for (int z = 0; z < NBV; ++z) {
            const int v = t + kHT * z, c = v / 32, col = 4 * (v % 32);
            br[z] = (c < C && l0 + col < L) ? *(const hf4 *)(a.t + ((int64_t)b * C + c) * L + l0 + col)
                                            : hf4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    // the fused trunk: the tile's words computed from x and written to LDS
    // one at a time (word z: the four outputs l0 + col .. +3 of channel c,
    // the taps added in k_trunk's order); the caller's barrier after the
    // previous tile has freed the tile
    auto trunk_b = [&](int T) {
        const int b = T / a.tiles_per_b, l0 = (T - b * a.tiles_per_b) * kHBN;
#pragma unroll 2
        for (int z = 0; z < NBV; ++z) {
            const int v = t + kHT * z, c = v / 32, col = 4 * (v % 32);
            const int cc = min(c, C - 1);
            const float *xr = a.x + ((int64_t)b * C + cc) * a.L_in;
            const float *twc = a.tw + cc * KT;
            const float tb = a.tb ? a.tb[cc] : 0.0f;
            float tv[4];
            if (a.xvec) {
                // stride 1, padding, dilation and L_in multiples of 4, x
                // aligned: tap k's four inputs are one 16-byte word, wholly
                // inside the row or wholly outside
                float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < KT; ++k) {
                    const int pos = l0 + col - a.padding + k * a.dilation;
                    const hf4 xv = (pos >= 0 && pos < a.L_in) ? *(const hf4 *)(xr + pos) : hf4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] += twc[k] * xv[j];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) tv[j] = (c < C && l0 + col < L) ? acc[j] + tb : 0.0f;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int base = (l0 + col + j) * a.stride - a.padding;
                    float acc = 0.0f;
#pragma unroll
                    for (int k = 0; k < KT; ++k) {
                        const int pos = base + k * a.dilation;
                        acc += twc[k] * ((pos >= 0 && pos < a.L_in) ? xr[pos] : 0.0f);
                    }
                    tv[j] = (c < C && l0 + col < L) ? acc + tb : 0.0f;
                }
            }
            *(hf4 *)(s_b + c * kHSBP + col) = hf4{tv[0], tv[1], tv[2], tv[3]};
        }
    };
    auto commit_b = [&]() {
#pragma unroll
        for (int z = 0; z < NBV; ++z) {
            const int v = t + kHT * z;
            *(hf4 *)(s_b + (v / 32) * kHSBP + 4 * (v % 32)) = br[z];
        }
    };
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    float *stg = s_stg + wv * STG;
    for (int i = blockIdx.x; i < a.tiles; i += gridDim.x) {
        // tiles from the last batch down: the first batches' offsets, which
        // the forward reads first, are the last written (still in the
        // memory-side cache when it starts)
        const int T = a.tiles - 1 - i;
        // this tile's trunk rows (the other workgroup on the CU computes
        // while they load)
        if constexpr (TRUNK) {
            trunk_b(T);
        } else {
            fetch_b(T);
            commit_b();
        }
        __syncthreads();
        const int b = T / a.tiles_per_b, l0 = (T - b * a.tiles_per_b) * kHBN;
        // one 32-column block at a time: its K accumulators over every
        // k-pair, then its write-out (whose stores drain while the next
        // block's MFMAs run)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            if (nb >= NBW) continue;
            hf16 acc[KT];
#pragma unroll
            for (int mb = 0; mb < KT; ++mb)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[mb][q] = 0.0f;
            const float *bcol = s_b + lh * kHSBP + 32 * (cb0 + nb) + li;
#pragma unroll
            for (int kk = 0; kk < NKP; ++kk) {
                const float bv = bcol[2 * kk * kHSBP];
#pragma unroll
                for (int mb = 0; mb < KT; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(aw[mb][kk], bv, acc[mb], 0, 0, 0);
            }
            // accumulator register q of row block mb is slab row
            // 32*mb + 8*(q >> 2) + 4*lh + (q & 3), column 32*(cb0 + nb) + li
            const int lc = l0 + 32 * (cb0 + nb);  // the block's first column (L is a multiple of 32)
            // in two halves of 16 groups (slab rows 16*K*hv .. 16*K*hv + 16*K - 1)
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
                wave_sync();  // the previous half's reads are done
#pragma unroll
                for (int mb = 0; mb < KT; ++mb)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int rl = 32 * mb + 8 * (q >> 2) + 4 * lh + (q & 3);
                        const int gl = rl / KT - 16 * hv, k = rl % KT;
                        if (gl >= 0 && gl < 16) stg[(gl * 32 + li) * KT + k] = acc[mb][q] + s_bias[r0 + rl];
                    }
                wave_sync();
                if (lc < L) {
                    // words: group gl's 32*K floats are 8*K words
#pragma unroll
                    for (int z = 0; z < 2 * KT; ++z) {
                        const int wd = lane + 64 * z, gl = wd / (8 * KT), e = 4 * (wd - gl * 8 * KT);
                        const int gg = slab * 32 + 16 * hv + gl;  // head group: offset group gg, or mask group gg - G
                        const bool is_mask = gg >= G;
                        if (gg >= (a.mask ? 2 * G : G)) continue;
                        hf4 v = *(const hf4 *)(stg + gl * 32 * KT + e);
                        if (is_mask) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) v[j] = head_sigmoid(v[j]);
                        }
                        float *run = (is_mask ? a.mask : a.off) + ((int64_t)b * G + (is_mask ? gg - G : gg)) * L * KT;
                        *(hf4 *)(run + (int64_t)lc * KT + e) = v;
                    }
                }
            }
        }
        __syncthreads();  // every wave is done with this tile's trunk rows
    }
}

template <int KT>
hipError_t launch_kt(const HeadArgs &a, int nkp, dim3 grid, size_t lds, hipStream_t stream) {
    if (a.x) {
        if (nkp == 16)
            hipLaunchKernelGGL((k_heads<KT, 16, true>), grid, dim3(kHT), lds, stream, a);
        else
            hipLaunchKernelGGL((k_heads<KT, 32, true>), grid, dim3(kHT), lds, stream, a);
    } else {
        if (nkp == 16)
            hipLaunchKernelGGL((k_heads<KT, 16, false>), grid, dim3(kHT), lds, stream, a);
        else
            hipLaunchKernelGGL((k_heads<KT, 32, false>), grid, dim3(kHT), lds, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

bool heads_fit(int C, int K, int M, int L, const void *t, const void *off, const void *mask) {
    const int slabs = (M + 32 * K - 1) / (32 * K);
    auto al = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    return K >= 1 && K <= 4 && C >= 1 && C <= 64 && slabs >= 1 && slabs <= 4 && L % 32 == 0 && al(t) && al(off) &&
           (!mask || al(mask));
}

hipError_t launch_heads(HeadArgs a, int num_cus, hipStream_t stream) {
    if (!heads_fit(a.C, a.K, a.M, a.L, a.x ? nullptr : a.t, a.off, a.mask)) return hipErrorInvalidValue;
    if (a.x && (!a.tw || (a.mask && !a.w2) || a.L_in < 1 || a.stride < 1 || a.dilation < 1))
        return hipErrorInvalidValue;
    a.xvec = a.x && a.stride == 1 && a.padding % 4 == 0 && a.dilation % 4 == 0 && a.L_in % 4 == 0 &&
             ((uintptr_t)a.x & 15) == 0;
    a.slabs = (a.M + 32 * a.K - 1) / (32 * a.K);
    if (a.slabs == 3) a.slabs = 4;  // (three slabs: one wave idle)
    a.tiles_per_b = (a.L + kHBN - 1) / kHBN;
    const int64_t tiles = (int64_t)a.B * a.tiles_per_b;
    if (tiles == 0) return hipSuccess;
    if (tiles >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    a.tiles = (int)tiles;
    const int nkp = a.C <= 32 ? 16 : 32;
    const size_t lds = ((size_t)2 * nkp * kHSBP + 4 * (16 * 32 * a.K) + 4 * 32 * a.K) * 4;
    const dim3 grid((unsigned)std::min<int64_t>(tiles, 2 * (int64_t)num_cus));  // two workgroups per CU
    switch (a.K) {
    case 1: return launch_kt<1>(a, nkp, grid, lds, stream);
    case 2: return launch_kt<2>(a, nkp, grid, lds, stream);
    case 3: return launch_kt<3>(a, nkp, grid, lds, stream);
    case 4: return launch_kt<4>(a, nkp, grid, lds, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dc1d
