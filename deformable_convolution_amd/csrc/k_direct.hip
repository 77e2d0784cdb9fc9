// k_direct.hip -- the VALU kernels of libdc1d:
//   * positions: the sampling-position split alone (test aid);
//   * direct: one thread per output, any groups / offset groups / mask;
//   * depthwise: one input channel per output (C_in/groups == 1), the
//     bandwidth-bound shape whose offsets dominate the bytes moved.
//
// Every kernel samples by linear interpolation between the two integer
// neighbours of the moved tap position, with zeros outside [0, L_in)
// (dc1d page, Demo notebook; torchvision issue demo), multiplies by the mask
// as given (dc1d page, Modulation), and sums weight * sample over the
// group's channels and taps before adding the bias (conv1d operator page,
// Description).
#include "dc1d_internal.h"

namespace dc1d {

// ---------------------------------------------------------------------------
// positions

template <class D>
__global__ void __launch_bounds__(256) k_positions(const typename D::T *__restrict__ off, int64_t n,
                                                   int L_out, int K, int stride, int padding,
                                                   int dilation, int L_in, int32_t *__restrict__ i0o,
                                                   float *__restrict__ fro, uint8_t *__restrict__ vao) {
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int k = (int)(idx % K);
        const int l = (int)((idx / K) % L_out);
        int i0;
        float f;
        split_position(D::ld(off, idx), l * stride - padding + k * dilation, i0, f);
        i0o[idx] = i0;
        fro[idx] = f;
        vao[idx] = (uint8_t)((i0 >= 0 && i0 < L_in ? 1 : 0) | (i0 + 1 >= 0 && i0 + 1 < L_in ? 2 : 0));
    }
}

// Elementwise storage conversion: bf16 -> fp32 is exact; fp32 -> bf16 rounds
// to nearest even (the conversion instruction).  Grid-stride.
template <class S, class D>
__global__ void __launch_bounds__(256) k_convert(const typename S::T *__restrict__ src,
                                                 typename D::T *__restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        D::st(dst, i, S::ld(src, i));
}

hipError_t launch_convert(const void *src, int src_dtype, void *dst, int dst_dtype, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    const dim3 grid((unsigned)blocks);
    if (src_dtype == kBF16 && dst_dtype == kF32)
        hipLaunchKernelGGL((k_convert<BF16, F32>), grid, dim3(256), 0, stream, (const uint16_t *)src, (float *)dst, n);
    else if (src_dtype == kF32 && dst_dtype == kBF16)
        hipLaunchKernelGGL((k_convert<F32, BF16>), grid, dim3(256), 0, stream, (const float *)src, (uint16_t *)dst, n);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_positions(const void *off, int dtype, int64_t n, int L_out, int K, int stride,
                            int padding, int dilation, int L_in, int32_t *i0, float *frac,
                            uint8_t *valid, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (dtype == kF32)
        hipLaunchKernelGGL(k_positions<F32>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const float *)off, n, L_out, K, stride, padding, dilation, L_in, i0, frac, valid);
    else
        hipLaunchKernelGGL(k_positions<BF16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t *)off, n, L_out, K, stride, padding, dilation, L_in, i0, frac, valid);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// direct: out[b, co, l] for one (b, co, l) per thread

template <class D>
__global__ void __launch_bounds__(256) k_direct(Params p) {
    using T = typename D::T;
    const T *__restrict__ x = (const T *)p.x;
    const T *__restrict__ off = (const T *)p.off;
    const T *__restrict__ mask = (const T *)p.mask;
    const T *__restrict__ w = (const T *)p.w;
    const T *__restrict__ bias = (const T *)p.bias;
    T *__restrict__ out = (T *)p.out;
    const int64_t total = (int64_t)p.B * p.C_out * p.L_out;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(idx % p.L_out);
        const int64_t bco = idx / p.L_out;
        const int co = (int)(bco % p.C_out);
        const int b = (int)(bco / p.C_out);
        const int grp = co / p.opg;
        float acc = 0.0f;
        for (int cl = 0; cl < p.cpg; ++cl) {
            const int ci = grp * p.cpg + cl;
            const int g = ci / p.cpo;
            const T *xrow = x + ((int64_t)b * p.C_in + ci) * p.L_in;
            const int64_t ob = (((int64_t)b * p.G + g) * p.L_out + l) * p.K;
            const T *wrow = w + ((int64_t)co * p.cpg + cl) * p.K;
            for (int k = 0; k < p.K; ++k) {
                int i0;
                float f;
                split_position(D::ld(off, ob + k), l * p.stride - p.padding + k * p.dilation, tap_range(p, k), i0,
                               f);
                const float x0 = (i0 >= 0 && i0 < p.L_in) ? D::ld(xrow, i0) : 0.0f;
                const float x1 = (i0 + 1 >= 0 && i0 + 1 < p.L_in) ? D::ld(xrow, i0 + 1) : 0.0f;
                float v = fmaf(f, x1 - x0, x0);
                if (mask) v *= D::ld(mask, ob + k);
                acc = fmaf(D::ld(wrow, k), v, acc);
            }
        }
        if (bias) acc += D::ld(bias, co);
        D::st(out, idx, acc);
    }
}

hipError_t launch_direct(const Params &p, hipStream_t stream) {
    const int64_t total = (int64_t)p.B * p.C_out * p.L_out;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    if (p.dtype == kF32)
        hipLaunchKernelGGL(k_direct<F32>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(k_direct<BF16>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// depthwise: C_in / groups == 1.
//
// A streaming kernel: the bytes are the offsets (K per output), the output
// and one read of x; every output costs K interpolations.  A block computes
// LT = 256*OPT consecutive outputs l of one (b, co); thread t owns outputs
// l0 + OPT*t .. +OPT-1, whose OPT*K offsets (and mask values) are one
// contiguous run that it loads straight into registers with 2- or 4-element vector
// loads.  The input row is staged in LDS over a fixed window: the tile's
// grid span plus kDwMargin positions on each side, zero outside [0, L_in).
// Samples whose offset moves them outside the window read x from global
// memory (bounds-checked), so any offset is served and the window needs no
// pass over the offsets first.

constexpr int kDwThreads = 256;
constexpr int kDwOpt = 2;      // outputs per thread (few registers: high occupancy)
constexpr int kDwMargin = 16;  // window margin per side (input positions)
constexpr int kDwWinU = 3;     // window positions per thread loaded up front (covers K * dilation <= 40 at stride 1)

// VW consecutive elements (VW = 2 or 4) as floats, in one load.
template <class D, int VW>
__device__ __forceinline__ void ldv(const typename D::T *p, float *v) {
    if constexpr (sizeof(typename D::T) == 4) {
        if constexpr (VW == 4) {
            const float4 q = *(const float4 *)p;
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else {
            const float2 q = *(const float2 *)p;
            v[0] = q.x; v[1] = q.y;
        }
    } else {
        if constexpr (VW == 4) {
            const uint2 q = *(const uint2 *)p;
            v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
            v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
        } else {
            const uint32_t q = *(const uint32_t *)p;
            v[0] = __uint_as_float(q << 16); v[1] = __uint_as_float(q & 0xffff0000u);
        }
    }
}
template <class D, int VW>
__device__ __forceinline__ void stv(typename D::T *p, const float *v) {
    if constexpr (sizeof(typename D::T) == 4) {
        if constexpr (VW == 4)
            *(float4 *)p = float4{v[0], v[1], v[2], v[3]};
        else
            *(float2 *)p = float2{v[0], v[1]};
    } else {
        const uint32_t a = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        if constexpr (VW == 4)
            *(uint2 *)p = uint2{a, (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16)};
        else
            *(uint32_t *)p = a;
    }
}

// KT: compile-time K (0: any K, read per tap); MASK: a mask is given.
template <class D, int KT, bool MASK>
__global__ void __launch_bounds__(kDwThreads) k_depthwise(Params p, int WIN, int tiles_l) {
    using T = typename D::T;
    constexpr int OPT = kDwOpt;
    constexpr int NV = KT > 0 ? OPT * KT : 1;  // offsets held per thread
    constexpr int VW = OPT % 4 == 0 ? 4 : 2;    // vector width of loads and stores
    static_assert(OPT % VW == 0, "whole vectors per thread");
    extern __shared__ float s_x[];               // WIN input positions from lo
    const int K = KT > 0 ? KT : p.K;
    const int t = threadIdx.x;
    const int tile = blockIdx.x % tiles_l;
    const int row = blockIdx.x / tiles_l;  // b * C_out + co
    const int co = row % p.C_out, b = row / p.C_out;
    const int ci = co / p.opg;  // cpg == 1: the conv group index is the input channel
    const int g = ci / p.cpo;
    const int l0 = tile * (kDwThreads * OPT);
    const T *__restrict__ xrow = (const T *)p.x + ((int64_t)b * p.C_in + ci) * p.L_in;
    const T *__restrict__ off = (const T *)p.off;
    const T *__restrict__ mask = MASK ? (const T *)p.mask : nullptr;
    const int L_in = p.L_in;
    const int lo = l0 * p.stride - p.padding - kDwMargin;

    // x window (WIN == 0: every sample reads global memory).  Without a
    // mask the first WU * kDwThreads positions are loaded at clamped
    // (in-bounds) addresses before the offsets, so all these loads are in
    // flight together, and written to LDS (zero outside [0, L_in)) after
    // them, wider windows loading the rest in a loop (depthwise 5-tap layer:
    // 177 -> 171 us); with a mask that measured slower (packed layer's 3-tap
    // pass: 102 -> 105 us), so there the window is loaded first, in a loop.
    constexpr int WU = MASK ? 0 : kDwWinU;
    float xw[WU > 0 ? WU : 1];
    if constexpr (WU == 0) {
        for (int j = t; j < WIN; j += kDwThreads) {
            const int i = lo + j;
            s_x[j] = (i >= 0 && i < L_in) ? D::ld(xrow, i) : 0.0f;
        }
    }
#pragma unroll
    for (int u = 0; u < WU; ++u)  // (lanes past the window reread its last position: no extra lines)
        xw[u] = D::ld(xrow, min(max(lo + min(t + u * kDwThreads, WIN - 1), 0), L_in - 1));
    // this thread's offsets and mask values
    const int lt = l0 + OPT * t;
    const int nvalid = min(OPT, p.L_out - lt);  // may be <= 0
    const int64_t e0 = (((int64_t)b * p.G + g) * p.L_out + lt) * K;
    float ov[NV], mv[MASK ? NV : 1];
    if (KT > 0) {
        const bool vec = nvalid == OPT && (((uintptr_t)(off + e0) & (VW * sizeof(T) - 1)) == 0) &&
                         (!MASK || (((uintptr_t)(mask + e0) & (VW * sizeof(T) - 1)) == 0));
        if (vec) {
#pragma unroll
            for (int c = 0; c < NV / VW; ++c) {
                ldv<D, VW>(off + e0 + VW * c, ov + VW * c);
                if (MASK) ldv<D, VW>(mask + e0 + VW * c, mv + VW * c);
            }
        } else {
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const bool ok = q < nvalid * K;
                ov[q] = ok ? D::ld(off, e0 + q) : 0.0f;
                if (MASK) mv[q] = ok ? D::ld(mask, e0 + q) : 0.0f;
            }
        }
    }
    if constexpr (WU > 0) {
#pragma unroll
        for (int u = 0; u < WU; ++u) {
            const int j = t + u * kDwThreads, i = lo + j;
            if (j < WIN) s_x[j] = (i >= 0 && i < L_in) ? xw[u] : 0.0f;
        }
        for (int j = t + WU * kDwThreads; j < WIN; j += kDwThreads) {
            const int i = lo + j;
            s_x[j] = (i >= 0 && i < L_in) ? D::ld(xrow, i) : 0.0f;
        }
    }
    __syncthreads();
    if (nvalid <= 0) return;

    const T *__restrict__ wrow = (const T *)p.w + (int64_t)co * K;
    const float bias = p.bias ? D::ld((const T *)p.bias, co) : 0.0f;
    float res[OPT];
#pragma unroll
    for (int o = 0; o < OPT; ++o) {
        const int l = lt + o;
        const int base0 = l * p.stride - p.padding;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {  // unrolled when K is a constant
            float ofs, m = 1.0f;
            if (KT > 0) {
                ofs = ov[o * KT + k];
                if (MASK) m = mv[o * KT + k];
            } else {
                const bool ok = o < nvalid;
                ofs = ok ? D::ld(off, e0 + o * K + k) : 0.0f;
                if (MASK) m = ok ? D::ld(mask, e0 + o * K + k) : 0.0f;
            }
            int i0;
            float f;
            split_position(ofs, base0 + k * p.dilation, tap_range(p, k), i0, f);
            const int j = i0 - lo;
            float x0, x1;
            if (WIN > 1 && (unsigned)j < (unsigned)(WIN - 1)) {
                x0 = s_x[j];
                x1 = s_x[j + 1];
            } else {
                x0 = (i0 >= 0 && i0 < L_in) ? D::ld(xrow, i0) : 0.0f;
                x1 = (i0 + 1 >= 0 && i0 + 1 < L_in) ? D::ld(xrow, i0 + 1) : 0.0f;
            }
            float v = fmaf(f, x1 - x0, x0);
            if (MASK) v *= m;
            acc = fmaf(D::ld(wrow, k), v, acc);
        }
        res[o] = acc + bias;
    }
    T *__restrict__ out = (T *)p.out + (int64_t)row * p.L_out + lt;
    if (nvalid == OPT && ((uintptr_t)out & (VW * sizeof(T) - 1)) == 0) {
#pragma unroll
        for (int c = 0; c < OPT / VW; ++c) stv<D, VW>(out + VW * c, res + VW * c);
    } else {
#pragma unroll
        for (int o = 0; o < OPT; ++o)
            if (o < nvalid) D::st(out, o, res[o]);
    }
}

DepthwisePlan plan_depthwise(const Params &p) {
    DepthwisePlan pl;
    const int LT = kDwThreads * kDwOpt;
    // window: the tile's grid span, both neighbours and the margins, in
    // whole 64-element lines, at most 12 K positions (48 KB); wider spans
    // gather from global memory
    int64_t win = (int64_t)(LT - 1) * p.stride + (int64_t)(p.K - 1) * p.dilation + 2 + 2 * kDwMargin;
    win = (win + 63) / 64 * 64;
    if (win > 12288) win = 0;
    pl.outputs_per_block = LT;
    pl.window = (int)win;
    pl.lds_bytes = (size_t)win * 4;
    const int64_t tiles_l = (p.L_out + LT - 1) / LT;
    pl.blocks = tiles_l * p.C_out * p.B;
    return pl;
}

template <class D, bool MASK>
static hipError_t launch_dw(const Params &p, const DepthwisePlan &pl, hipStream_t stream) {
    const int tiles_l = (p.L_out + pl.outputs_per_block - 1) / pl.outputs_per_block;
    const dim3 grid((unsigned)pl.blocks), block(kDwThreads);
    switch (p.K) {
#define DC1D_DW(KK) \
    case KK: hipLaunchKernelGGL((k_depthwise<D, KK, MASK>), grid, block, pl.lds_bytes, stream, p, pl.window, tiles_l); break;
        DC1D_DW(1)
        DC1D_DW(2)
        DC1D_DW(3)
        DC1D_DW(4)
        DC1D_DW(5)
        DC1D_DW(7)
        DC1D_DW(9)
#undef DC1D_DW
        default:
            hipLaunchKernelGGL((k_depthwise<D, 0, MASK>), grid, block, pl.lds_bytes, stream, p, pl.window, tiles_l);
    }
    return hipGetLastError();
}

hipError_t launch_depthwise(const Params &p, const DepthwisePlan &pl, hipStream_t stream) {
    if (pl.blocks == 0) return hipSuccess;
    if (p.dtype == kF32) return p.mask ? launch_dw<F32, true>(p, pl, stream) : launch_dw<F32, false>(p, pl, stream);
    return p.mask ? launch_dw<BF16, true>(p, pl, stream) : launch_dw<BF16, false>(p, pl, stream);
}

}  // namespace dc1d
