// k_mfma_wide.hip -- instantiates and launches the one-wave-per-SIMD bf16
// kernel of mfma_wide.h (the weights rearranged first by k_weight_blocks,
// as for the 32-channel-block kernels).
#include "mfma_wide.h"

namespace dc1d {
namespace {

// The windowed launch, then the gathering one for the tiles it marked
// (every other workgroup of the second launch returns at once).
template <bool MASK, int KT, int I>
void launch_npos(int npos, const WideArgs &a, dim3 grid, size_t lds, hipStream_t stream) {
    if constexpr (I < kNumWideNpos) {
        if (npos == kWideNpos[I]) {
            if constexpr (kWideNpos[I] <= kWT * KT) {
                hipLaunchKernelGGL((k_mfma_wide<MASK, kWideNpos[I], KT, true>), grid, dim3(kWT), lds, stream, a);
                hipLaunchKernelGGL((k_mfma_wide<MASK, kWideNpos[I], KT, false>), grid, dim3(kWT), kWideGatherLds,
                                   stream, a);
            }
        } else {
            launch_npos<MASK, KT, I + 1>(npos, a, grid, lds, stream);
        }
    }
}

template <bool MASK>
hipError_t launch_wide_t(const Params &p, const MfmaPlan &pl, hipStream_t stream) {
    WideArgs a;
    a.p = p;
    a.fd_Lout = make_fastdiv((uint32_t)p.L_out);
    a.fd_cpo = make_fastdiv((uint32_t)p.cpo);
    a.tiles_m = pl.wide_tiles_m;
    a.tiles_n = pl.wide_tiles_n;
    a.ncb = pl.wide_ncb;
    a.N = (int64_t)p.B * p.L_out;
    uint16_t *wb = (uint16_t *)p.ws;
    a.wb = wb;
    a.gather = (uint8_t *)p.ws + pl.wide_wb_bytes;
    // weights -> [K][C_out][ncb][32]: blocks of 32 channels at one tap (a
    // padding block, when there is one, gets zeros)
    hipLaunchKernelGGL((k_weight_blocks<uint16_t>), dim3((unsigned)(p.K * p.C_out)), dim3(256), 0, stream,
                       (const uint16_t *)p.w, wb, p.C_out, p.C_in, p.K, 0, pl.wide_ncb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(pl.wide_tiles_m * pl.wide_tiles_n));
    mark_event(p.ev_start, stream);
    switch (p.K) {
    case 2: launch_npos<MASK, 2, 0>(pl.wide, a, grid, pl.wide_lds, stream); break;
    case 3: launch_npos<MASK, 3, 0>(pl.wide, a, grid, pl.wide_lds, stream); break;
    case 4: launch_npos<MASK, 4, 0>(pl.wide, a, grid, pl.wide_lds, stream); break;
    default: return hipErrorInvalidValue;
    }
    mark_event(p.ev_stop, stream);
    return hipGetLastError();
}

}  // namespace

bool wide_npos_compiled(int npos, int K) {
    for (int i = 0; i < kNumWideNpos; ++i)
        if (kWideNpos[i] == npos) return K >= 2 && K <= kWideMaxK && npos <= kWT * K;
    return false;
}

int wide_npos_option(int i) { return i < kNumWideNpos ? kWideNpos[i] : 0; }

size_t wide_lds_bytes(int npos) { return kWideWLds + (size_t)2 * npos * kTPitch * 2; }

hipError_t launch_mfma_wide(const Params &p, const MfmaPlan &pl, hipStream_t stream) {
    if (p.dtype != kBF16 || !wide_npos_compiled(pl.wide, p.K)) return hipErrorInvalidValue;
    return p.mask ? launch_wide_t<true>(p, pl, stream) : launch_wide_t<false>(p, pl, stream);
}

}  // namespace dc1d
