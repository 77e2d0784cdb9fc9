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
                split_position(D::ld(off, ob + k), l * p.stride - p.padding + k * p.dilation, i0, f);
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
// One block computes LT consecutive outputs l of one (b, co).  Its offsets
// (and mask) for those outputs are one contiguous run of LT*K values in HBM
// ([B, G, L_out, K] with K fastest); the block streams that run into LDS
// with coalesced loads, bounds the x window the positions can touch from the
// run's smallest and largest offset, stages that window of the input row in
// LDS with zero fill outside [0, L_in), and then interpolates from LDS.  When
// the offsets spread wider than the window capacity, the block gathers x from
// global memory instead (same arithmetic, bounds-checked loads).

constexpr int kDwThreads = 256;

template <class D>
__global__ void __launch_bounds__(kDwThreads) k_depthwise(Params p, int LT, int WCAP, int tiles_l,
                                                          int64_t n_blocks) {
    using T = typename D::T;
    extern __shared__ float smem[];
    const int K = p.K;
    float *s_w = smem;                           // K
    float *s_off = s_w + ((K + 3) & ~3);         // LT*K
    float *s_mask = s_off + LT * K;              // LT*K (if mask)
    float *s_x = s_mask + (p.mask ? LT * K : 0); // WCAP
    __shared__ float s_red[2][kDwThreads / 64];

    const T *__restrict__ off = (const T *)p.off;
    const T *__restrict__ mask = (const T *)p.mask;
    const int t = threadIdx.x;

    for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x) {
        int64_t rest = blk;
        const int tile = (int)(rest % tiles_l);
        rest /= tiles_l;
        const int co = (int)(rest % p.C_out);
        const int b = (int)(rest / p.C_out);
        const int ci = co / p.opg;  // cpg == 1: the conv group index is the input channel
        const int g = ci / p.cpo;
        const int l0 = tile * LT;
        const int nl = min(LT, p.L_out - l0);
        const T *__restrict__ xrow = (const T *)p.x + ((int64_t)b * p.C_in + ci) * p.L_in;
        const int64_t e0 = (((int64_t)b * p.G + g) * p.L_out + l0) * K;

        __syncthreads();  // LDS reuse across loop iterations
        float vmin = kOffsetClamp, vmax = -kOffsetClamp;
        for (int j = t; j < nl * K; j += kDwThreads) {
            float v = D::ld(off, e0 + j);
            v = fminf(fmaxf(v, -kOffsetClamp), kOffsetClamp);
            s_off[j] = v;
            vmin = fminf(vmin, v);
            vmax = fmaxf(vmax, v);
        }
        if (mask)
            for (int j = t; j < nl * K; j += kDwThreads) s_mask[j] = D::ld(mask, e0 + j);
        for (int j = t; j < K; j += kDwThreads) s_w[j] = D::ld((const T *)p.w, (int64_t)co * K + j);

        // block min / max of the offsets
        for (int o = 32; o > 0; o >>= 1) {
            vmin = fminf(vmin, __shfl_xor(vmin, o));
            vmax = fmaxf(vmax, __shfl_xor(vmax, o));
        }
        if ((t & 63) == 0) {
            s_red[0][t >> 6] = vmin;
            s_red[1][t >> 6] = vmax;
        }
        __syncthreads();
        vmin = s_red[0][0];
        vmax = s_red[1][0];
#pragma unroll
        for (int q = 1; q < kDwThreads / 64; ++q) {
            vmin = fminf(vmin, s_red[0][q]);
            vmax = fmaxf(vmax, s_red[1][q]);
        }
        // Every left neighbour i0 of this block lies in [lo_b, hi_b]; clamped
        // to [-2, L_in] (where both neighbours read zero outside the
        // sequence) it lies in [lo, hi].
        const int lo_b = l0 * p.stride - p.padding + (int)floorf(vmin);
        const int hi_b = (l0 + nl - 1) * p.stride - p.padding + (K - 1) * p.dilation + (int)floorf(vmax);
        const int lo = min(max(lo_b, -2), p.L_in);
        const int hi = min(max(hi_b, -2), p.L_in);
        const int W = hi - lo + 2;  // window elements x~(lo .. hi + 1)
        const bool windowed = (W <= WCAP);
        if (windowed) {
            for (int j = t; j < W; j += kDwThreads) {
                const int i = lo + j;
                s_x[j] = (i >= 0 && i < p.L_in) ? D::ld(xrow, i) : 0.0f;
            }
        }
        __syncthreads();

        T *__restrict__ out = (T *)p.out + ((int64_t)b * p.C_out + co) * p.L_out;
        const float bias = p.bias ? D::ld((const T *)p.bias, co) : 0.0f;
        for (int ll = t; ll < nl; ll += kDwThreads) {
            const int l = l0 + ll;
            const int base0 = l * p.stride - p.padding;
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int i0;
                float f;
                split_position(s_off[ll * K + k], base0 + k * p.dilation, i0, f);
                float x0, x1;
                if (windowed) {
                    int j = min(max(i0, -2), p.L_in) - lo;
                    j = min(max(j, 0), W - 2);
                    x0 = s_x[j];
                    x1 = s_x[j + 1];
                } else {
                    x0 = (i0 >= 0 && i0 < p.L_in) ? D::ld(xrow, i0) : 0.0f;
                    x1 = (i0 + 1 >= 0 && i0 + 1 < p.L_in) ? D::ld(xrow, i0 + 1) : 0.0f;
                }
                float v = fmaf(f, x1 - x0, x0);
                if (mask) v *= s_mask[ll * K + k];
                acc = fmaf(s_w[k], v, acc);
            }
            D::st(out, l, acc + bias);
        }
    }
}

DepthwisePlan plan_depthwise(const Params &p) {
    DepthwisePlan pl;
    // outputs per block: as many as keep the offsets (+ mask) run and the x
    // window within ~48 KB of LDS, a multiple of the block size, at most 1024.
    const int per_out = p.K * (p.mask ? 2 : 1) * 4;
    int LT = 1024;
    while (LT > kDwThreads && (size_t)LT * per_out > 32768) LT -= kDwThreads;
    if (LT > p.L_out) LT = ((p.L_out + kDwThreads - 1) / kDwThreads) * kDwThreads;
    // window: the taps' grid span plus a margin of 512 for the offsets' spread
    int64_t span = (int64_t)(LT - 1) * p.stride + (int64_t)(p.K - 1) * p.dilation + 2;
    int64_t wcap = span + 512;
    if (wcap > 8192) wcap = 8192;
    pl.outputs_per_block = LT;
    pl.window = (int)wcap;
    pl.lds_bytes = (size_t)(((p.K + 3) & ~3) * 4) + (size_t)LT * per_out + (size_t)wcap * 4;
    const int tiles_l = (p.L_out + LT - 1) / LT;
    pl.blocks = (int64_t)tiles_l * p.C_out * p.B;
    return pl;
}

hipError_t launch_depthwise(const Params &p, const DepthwisePlan &pl, hipStream_t stream) {
    if (pl.blocks == 0) return hipSuccess;
    const int tiles_l = (p.L_out + pl.outputs_per_block - 1) / pl.outputs_per_block;
    const unsigned grid = (unsigned)(pl.blocks < (1 << 30) ? pl.blocks : (1 << 30));
    if (p.dtype == kF32)
        hipLaunchKernelGGL(k_depthwise<F32>, dim3(grid), dim3(kDwThreads), pl.lds_bytes, stream, p,
                           pl.outputs_per_block, pl.window, tiles_l, pl.blocks);
    else
        hipLaunchKernelGGL(k_depthwise<BF16>, dim3(grid), dim3(kDwThreads), pl.lds_bytes, stream, p,
                           pl.outputs_per_block, pl.window, tiles_l, pl.blocks);
    return hipGetLastError();
}

}  // namespace dc1d
