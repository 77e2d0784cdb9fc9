// k_dc2d.hip -- 2D modulated deformable convolution (DCNv2).
//
// The deformable convolution article (section Deformable Convolution) moves
// every tap p0 + pn of a 2D kernel by a learned offset and samples the input
// there by bilinear interpolation between the four surrounding pixels (Step
// 2), then weighs the samples with the kernel (Step 3); the modulation mask
// multiplies each sample.  Offsets come in the layout of torchvision's
// deform_conv2d, which its documentation issue settles as: per offset group
// g, kernel row i, kernel column j, the pair (row offset, column offset) --
// channel 2*((g*kh + i)*kw + j) and the next.
//
// Tap (i, j) of output (oh, ow) samples row oh*sh - ph + i*dh + dy and column
// ow*sw - pw + j*dw + dx.  Each axis is split like the 1D position
// (split_position: exact integer grid term plus the floor of the offset);
// neighbours outside the image read zero.
//
// Dense layers (groups == 1, C_out >= 32) run in two kernels:
//   k_im2col2d  the sampled matrix S [B][C_in*T][Ho*Wo] (row ci*T + tap) in
//               the storage dtype -- a thread takes one (b, g, tap, output
//               position) and a run of the group's channels, splits the
//               position and forms the four bilinear weights once, then
//               gathers and blends each channel, storing coalesced along the
//               output positions;
//   k_gemm      out = W S on the MFMA kernel's plain-GEMM form (M = C_out,
//               N = B*Ho*Wo, Kred = C_in*T), the bias in its epilogue.
// Other layers use k_direct2d, one thread per output.
#include "dc1d_internal.h"

namespace dc1d {
namespace {

constexpr int kChanRun = 32;  // channels per im2col thread
constexpr int kUnroll = 8;    // channels whose gathers are in flight together

// The four bilinear neighbours of one (tap, output position): element
// offsets inside a channel plane and their weights (0 outside the image).
struct Corners {
    int idx[4];
    float wt[4];
};

__device__ __forceinline__ Corners corners(const Params2 &p, float dy, float dx, int oh, int ow, int i, int j) {
    int r0, c0;
    float fy, fx;
    split_position(dy, oh * p.sh - p.ph + i * p.dh, r0, fy);
    split_position(dx, ow * p.sw - p.pw + j * p.dw, c0, fx);
    const bool vr0 = (unsigned)r0 < (unsigned)p.H, vr1 = (unsigned)(r0 + 1) < (unsigned)p.H;
    const bool vc0 = (unsigned)c0 < (unsigned)p.W, vc1 = (unsigned)(c0 + 1) < (unsigned)p.W;
    Corners c;
    c.wt[0] = (vr0 && vc0) ? (1.0f - fy) * (1.0f - fx) : 0.0f;
    c.wt[1] = (vr0 && vc1) ? (1.0f - fy) * fx : 0.0f;
    c.wt[2] = (vr1 && vc0) ? fy * (1.0f - fx) : 0.0f;
    c.wt[3] = (vr1 && vc1) ? fy * fx : 0.0f;
    // clamped indices: a zero-weight neighbour still reads inside the plane
    const int ra = min(max(r0, 0), p.H - 1), rb = min(max(r0 + 1, 0), p.H - 1);
    const int ca = min(max(c0, 0), p.W - 1), cb = min(max(c0 + 1, 0), p.W - 1);
    c.idx[0] = ra * p.W + ca;
    c.idx[1] = ra * p.W + cb;
    c.idx[2] = rb * p.W + ca;
    c.idx[3] = rb * p.W + cb;
    return c;
}

template <class D>
__device__ __forceinline__ float blend(const typename D::T *plane, const Corners &c) {
    float v = c.wt[0] * D::ld(plane, c.idx[0]);
    v = fmaf(c.wt[1], D::ld(plane, c.idx[1]), v);
    v = fmaf(c.wt[2], D::ld(plane, c.idx[2]), v);
    return fmaf(c.wt[3], D::ld(plane, c.idx[3]), v);
}

// grid: (ceil(Ho*Wo / 256), G*T*ceil(cpo / kChanRun), B)
template <class D, bool MASK>
__global__ void __launch_bounds__(256) k_im2col2d(Params2 p, int runs) {
    using T = typename D::T;
    const int HWo = p.Ho * p.Wo;
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q >= HWo) return;
    const int run = blockIdx.y % runs;
    const int gt = blockIdx.y / runs;  // g*T + tap
    const int g = gt / p.T, tap = gt - g * p.T;
    const int i = tap / p.kw, j = tap - i * p.kw;
    const int b = blockIdx.z;
    const int oh = q / p.Wo, ow = q - oh * p.Wo;
    const T *__restrict__ off = (const T *)p.off + ((int64_t)b * 2 * p.G * p.T + 2 * gt) * HWo + q;
    const Corners c = corners(p, D::ld(off, 0), D::ld(off, HWo), oh, ow, i, j);
    const float m = MASK ? D::ld((const T *)p.mask, ((int64_t)b * p.G * p.T + gt) * HWo + q) : 1.0f;
    const int c_lo = g * p.cpo + run * kChanRun, c_hi = min(c_lo + kChanRun, (g + 1) * p.cpo);
    const T *__restrict__ x = (const T *)p.x;
    T *__restrict__ S = (T *)p.ws;
    const int64_t plane = (int64_t)p.H * p.W;
    // kUnroll channels at a time: all their gathers issued before the blends
    for (int c0 = c_lo; c0 < c_hi; c0 += kUnroll) {
        float xv[kUnroll][4];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const T *xp = x + ((int64_t)b * p.C_in + min(c0 + u, c_hi - 1)) * plane;
#pragma unroll
            for (int z = 0; z < 4; ++z) xv[u][z] = D::ld(xp, c.idx[z]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (c0 + u >= c_hi) break;
            float v = c.wt[0] * xv[u][0];
            v = fmaf(c.wt[1], xv[u][1], v);
            v = fmaf(c.wt[2], xv[u][2], v);
            v = fmaf(c.wt[3], xv[u][3], v);
            if (MASK) v *= m;
            D::st(S, (((int64_t)b * p.C_in + c0 + u) * p.T + tap) * HWo + q, v);
        }
    }
}

// The same matrix with the input staged in LDS: a block takes 256
// consecutive output positions of one batch and a run of one offset group's
// channels; each thread splits its position's TT taps once (registers), and
// for every channel the block stages the band of input rows those positions
// can reach -- their rows' span plus kBandR rows of offset on each side,
// zero outside the image -- in LDS (double-buffered, one barrier per
// channel, the next channel's band loaded while this one is sampled), so
// that every tap's four neighbours are LDS reads.  Taps moved beyond the
// band read global memory.
constexpr int kBandR = 4;
constexpr int kBandRun = 16;  // channels per block (measured: 8 and 32 were slower on the 64 x 64 workloads)
constexpr int kBandPer = 8;  // band elements per thread (the band holds at most 256 * kBandPer)
constexpr size_t kBandLds = 48 * 1024;

template <class D, bool MASK, int TT>
__global__ void __launch_bounds__(256) k_im2col2d_band(Params2 p, int runs, int band_cap) {
    using T = typename D::T;
    extern __shared__ float s_band[];  // [2][band_cap]
    const int HWo = p.Ho * p.Wo;
    const int q0 = blockIdx.x * 256;
    const int q = q0 + threadIdx.x;
    const bool valid = q < HWo;
    const int run = blockIdx.y % runs;
    const int g = blockIdx.y / runs;
    const int b = blockIdx.z;
    const int qq = valid ? q : HWo - 1;
    const int oh = qq / p.Wo, ow = qq - oh * p.Wo;
    const int oh_a = q0 / p.Wo, oh_b = min(q0 + 255, HWo - 1) / p.Wo;
    const int r_lo = oh_a * p.sh - p.ph - kBandR;
    const int nrows = (oh_b - oh_a) * p.sh + (p.kh - 1) * p.dh + 2 * kBandR + 2;
    const int W = p.W;
    // this position's taps, once: band-relative indices of the left
    // neighbours in the two rows, column weights, and row weights with the
    // mask folded in; ia = -1 marks a tap moved beyond the band
    int ia[TT], ib[TT];
    float wx0[TT], wx1[TT], wt[TT], wb[TT];
    const T *__restrict__ off = (const T *)p.off + ((int64_t)b * 2 * p.G + 2 * g) * TT * HWo + qq;
    const T *__restrict__ msk = MASK ? (const T *)p.mask + ((int64_t)b * p.G + g) * TT * HWo + qq : nullptr;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int i = t / p.kw, j = t - i * p.kw;
        int r0, c0;
        float fy, fx;
        split_position(D::ld(off, (int64_t)2 * t * HWo), oh * p.sh - p.ph + i * p.dh, r0, fy);
        split_position(D::ld(off, (int64_t)(2 * t + 1) * HWo), ow * p.sw - p.pw + j * p.dw, c0, fx);
        const float m = MASK ? D::ld(msk, (int64_t)t * HWo) : 1.0f;
        const bool vc0 = (unsigned)c0 < (unsigned)W, vc1 = (unsigned)(c0 + 1) < (unsigned)W;
        const int ca = min(max(c0, 0), W - 1), cb = min(max(c0 + 1, 0), W - 1);
        const int rb = r0 - r_lo;
        const bool inband = (unsigned)rb <= (unsigned)(nrows - 2);
        ia[t] = inband ? rb * W + ca : -1;
        ib[t] = inband ? rb * W + cb : 0;
        wx0[t] = vc0 ? 1.0f - fx : 0.0f;
        wx1[t] = vc1 ? fx : 0.0f;
        wt[t] = (1.0f - fy) * m;
        wb[t] = fy * m;
    }
    const int c_lo = g * p.cpo + run * kBandRun, c_hi = min(c_lo + kBandRun, (g + 1) * p.cpo);
    const T *__restrict__ x = (const T *)p.x;
    const int64_t plane = (int64_t)p.H * W;
    const int nband = nrows * W;
    // the band of channel ci + 1 is loaded into registers before channel
    // ci's samples are stored, so waiting for those loads never waits for
    // the stores (one memory counter tracks both)
    // this thread's band elements e = t + 256u: their offset in a channel's
    // plane (-1: outside the image or past the band), the same for every channel
    int boff[kBandPer];
#pragma unroll
    for (int u = 0; u < kBandPer; ++u) {
        const int e = threadIdx.x + 256 * u;
        const int rr = e / W, col = e - rr * W, r = r_lo + rr;
        boff[u] = (e < nband && r >= 0 && r < p.H) ? r * W + col : -1;
    }
    // bf16: the loads are unconditional (entries outside the image or past
    // the band read the plane's first element, zeroed when put) and the
    // sample stores below too, so the compiler can count the memory
    // operations in flight: waiting for the band's loads then waits for them
    // alone, not for the stores issued after them (the values stay in
    // storage format until put, so that widening them does not wait either).
    // Measured on the 64 x 64 workloads: bf16 119 -> 73 us; fp32 116 -> 123
    // us, so fp32 keeps the conditional loads and stores.
    constexpr bool kFlat = sizeof(T) == 2;
    T xv[kBandPer];
    auto fetch = [&](int ci) {
        const T *__restrict__ xp = x + ((int64_t)b * p.C_in + ci) * plane;
#pragma unroll
        for (int u = 0; u < kBandPer; ++u) {
            if constexpr (kFlat)
                xv[u] = xp[max(boff[u], 0)];
            else
                xv[u] = boff[u] >= 0 ? xp[boff[u]] : T(0);
        }
    };
    auto put = [&](float *band) {
        float v[kBandPer];
#pragma unroll
        for (int u = 0; u < kBandPer; ++u) v[u] = boff[u] >= 0 ? D::ld(xv, u) : 0.0f;
#pragma unroll
        for (int u = 0; u < kBandPer; ++u) {
            const int e = threadIdx.x + 256 * u;
            if (e < nband) band[e] = v[u];
        }
    };
    if (c_lo < c_hi) {
        fetch(c_lo);
        put(s_band);
    }
    __syncthreads();
    for (int ci = c_lo; ci < c_hi; ++ci) {
        float *band = s_band + ((ci - c_lo) & 1) * band_cap;
        const T *__restrict__ xp = x + ((int64_t)b * p.C_in + ci) * plane;
        const bool more = ci + 1 < c_hi;
        if (more) fetch(ci + 1);
        // (bf16: lanes past the end store the last position's sample -- the
        // same value at the same address)
        if (kFlat || valid) {
            T *__restrict__ st = (T *)p.ws + ((int64_t)b * p.C_in + ci) * TT * HWo + qq;
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                float v;
                if (ia[t] >= 0) {
                    const float top = fmaf(wx1[t], band[ib[t]], wx0[t] * band[ia[t]]);
                    const float bot = fmaf(wx1[t], band[ib[t] + W], wx0[t] * band[ia[t] + W]);
                    v = fmaf(wb[t], bot, wt[t] * top);
                } else {  // moved beyond the band: the neighbours from global memory
                    const int i = t / p.kw, j = t - i * p.kw;
                    int r0, c0;
                    float fy, fx;
                    split_position(D::ld(off, (int64_t)2 * t * HWo), oh * p.sh - p.ph + i * p.dh, r0, fy);
                    split_position(D::ld(off, (int64_t)(2 * t + 1) * HWo), ow * p.sw - p.pw + j * p.dw, c0, fx);
                    const int ca = min(max(c0, 0), W - 1), cb = min(max(c0 + 1, 0), W - 1);
                    const int ra = min(max(r0, 0), p.H - 1), rc = min(max(r0 + 1, 0), p.H - 1);
                    const bool vr0 = (unsigned)r0 < (unsigned)p.H, vr1 = (unsigned)(r0 + 1) < (unsigned)p.H;
                    const float top = vr0 ? fmaf(wx1[t], D::ld(xp, (int64_t)ra * W + cb), wx0[t] * D::ld(xp, (int64_t)ra * W + ca))
                                          : 0.0f;
                    const float bot = vr1 ? fmaf(wx1[t], D::ld(xp, (int64_t)rc * W + cb), wx0[t] * D::ld(xp, (int64_t)rc * W + ca))
                                          : 0.0f;
                    v = fmaf(wb[t], bot, wt[t] * top);
                }
                D::st(st, (int64_t)t * HWo, v);
            }
        }
        if (more) put(s_band + ((ci + 1 - c_lo) & 1) * band_cap);
        __syncthreads();
    }
}

// One thread per output (b, co, oh, ow): the group's channels and taps in
// ascending order.
template <class D, bool MASK>
__global__ void __launch_bounds__(256) k_direct2d(Params2 p) {
    using T = typename D::T;
    const int HWo = p.Ho * p.Wo;
    const int64_t total = (int64_t)p.B * p.C_out * HWo;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const int q = (int)(e % HWo);
    const int64_t bc = e / HWo;
    const int co = (int)(bc % p.C_out), b = (int)(bc / p.C_out);
    const int oh = q / p.Wo, ow = q - oh * p.Wo;
    const int grp = co / p.opg;
    const T *__restrict__ x = (const T *)p.x;
    const T *__restrict__ w = (const T *)p.w + (int64_t)co * p.Kred;
    const int64_t plane = (int64_t)p.H * p.W;
    float acc = 0.0f;
    for (int cl = 0; cl < p.cpg; ++cl) {
        const int ci = grp * p.cpg + cl;
        const int g = ci / p.cpo;
        const T *xp = x + ((int64_t)b * p.C_in + ci) * plane;
        for (int tap = 0; tap < p.T; ++tap) {
            const int gt = g * p.T + tap;
            const int i = tap / p.kw, j = tap - i * p.kw;
            const T *off = (const T *)p.off + ((int64_t)b * 2 * p.G * p.T + 2 * gt) * HWo + q;
            const Corners c = corners(p, D::ld(off, 0), D::ld(off, HWo), oh, ow, i, j);
            float v = blend<D>(xp, c);
            if (MASK) v *= D::ld((const T *)p.mask, ((int64_t)b * p.G * p.T + gt) * HWo + q);
            acc = fmaf(D::ld(w, cl * p.T + tap), v, acc);
        }
    }
    if (p.bias) acc += D::ld((const T *)p.bias, co);
    D::st((T *)p.out, e, acc);
}

bool dense(const Params2 &p) { return p.groups == 1 && p.C_out >= 32 && p.Kred >= 16; }

// The banded sampler's LDS band (floats per buffer), or 0 when it does not
// serve this shape (taps other than 1x1, 2x2, 3x3 square counts 1, 4, 9 with
// kw matching, or a band beyond kBandLds).
int band_cap(const Params2 &p) {
    if (p.T != 1 && p.T != 4 && p.T != 9) return 0;
    const int64_t dr = 255 / p.Wo + 1;  // output rows a block of 256 positions spans, minus one (at most)
    const int64_t nrows = dr * p.sh + (int64_t)(p.kh - 1) * p.dh + 2 * kBandR + 2;
    const int64_t cap = nrows * p.W;
    return cap <= 256 * kBandPer && 2 * cap * 4 <= (int64_t)kBandLds ? (int)cap : 0;
}

// The contraction's GEMM arguments: A = weight [C_out][Kred], B(k, n) =
// S[b][k][q], C = out [B][C_out][Ho*Wo].
Params gemm_args(const Params2 &p, void *part) {
    Params q = {};
    q.dtype = p.dtype;
    q.w = p.w;
    q.x = p.ws;
    q.out = p.out;
    q.bias = p.bias;
    q.B = p.B;
    q.C_out = p.C_out;
    q.Kred = p.Kred;
    q.L_out = p.Ho * p.Wo;
    q.ws = part;
    return q;
}

size_t s_bytes(const Params2 &p) {
    const size_t es = p.dtype == kF32 ? 4 : 2;
    return ((size_t)p.B * p.Kred * p.Ho * p.Wo * es + 255) & ~(size_t)255;
}

template <class D, bool MASK>
hipError_t launch_typed(const Params2 &p, int num_cus, hipStream_t stream) {
    const int64_t HWo = (int64_t)p.Ho * p.Wo;
    if (dense(p)) {
        const int runs = (p.cpo + kChanRun - 1) / kChanRun;
        const int cap = band_cap(p);
        if (cap > 0) {
            const int runs_b = (p.cpo + kBandRun - 1) / kBandRun;
            const int64_t gy = (int64_t)p.G * runs_b;
            if (gy > 65535 || p.B > 65535) return hipErrorInvalidValue;
            const dim3 grid((unsigned)((HWo + 255) / 256), (unsigned)gy, (unsigned)p.B);
            const size_t lds = 2 * (size_t)cap * 4;
            switch (p.T) {
            case 1: hipLaunchKernelGGL((k_im2col2d_band<D, MASK, 1>), grid, dim3(256), lds, stream, p, runs_b, cap); break;
            case 4: hipLaunchKernelGGL((k_im2col2d_band<D, MASK, 4>), grid, dim3(256), lds, stream, p, runs_b, cap); break;
            case 9: hipLaunchKernelGGL((k_im2col2d_band<D, MASK, 9>), grid, dim3(256), lds, stream, p, runs_b, cap); break;
            default: return hipErrorInvalidValue;
            }
        } else {
            const int64_t gy = (int64_t)p.G * p.T * runs;
            if (gy > 65535 || p.B > 65535) return hipErrorInvalidValue;
            const dim3 grid((unsigned)((HWo + 255) / 256), (unsigned)gy, (unsigned)p.B);
            hipLaunchKernelGGL((k_im2col2d<D, MASK>), grid, dim3(256), 0, stream, p, runs);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const Params q = gemm_args(p, (char *)p.ws + s_bytes(p));
        const int64_t brow = HWo, bbatch = (int64_t)p.Kred * HWo;
        return p.dtype == kF32 ? launch_gemm_f32(q, brow, bbatch, 0, num_cus, stream)
                               : launch_gemm_bf16(q, brow, bbatch, num_cus, stream);
    }
    const int64_t total = (int64_t)p.B * p.C_out * HWo;
    const int64_t blocks = (total + 255) / 256;
    if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_direct2d<D, MASK>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

size_t dc2d_workspace(const Params2 &p, int num_cus) {
    if (!dense(p)) return 0;
    const Params q = gemm_args(p, nullptr);
    const size_t part = p.dtype == kF32 ? gemm_workspace_bytes(q, 0, num_cus) : gemm_bf16_workspace_bytes(q, num_cus);
    return s_bytes(p) + part;
}

const char *dc2d_kernel_name(const Params2 &p) {
    if (!dense(p)) return "direct2d";
    return p.dtype == kF32 ? "im2col2d_gemm_f32" : "im2col2d_gemm_bf16";
}

hipError_t launch_dc2d(const Params2 &p, int num_cus, hipStream_t stream) {
    if (p.B == 0) return hipSuccess;
    if (p.dtype == kF32) return p.mask ? launch_typed<F32, true>(p, num_cus, stream)
                                       : launch_typed<F32, false>(p, num_cus, stream);
    return p.mask ? launch_typed<BF16, true>(p, num_cus, stream) : launch_typed<BF16, false>(p, num_cus, stream);
}

}  // namespace dc1d
