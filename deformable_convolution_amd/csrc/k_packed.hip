// k_packed.hip -- the trunk of the packed layer's offset generator.
//
// The packed layer (dc1d page, section PackedDeformConv1d) computes its
// offsets from its input with a depthwise-separable block; its trunk is a
// depthwise conv1d with the layer's kernel size, stride, padding and
// dilation, so that it yields one column per output position:
//     t[b,c,l] = tb[c] + sum_k tw[c,k] * x~[b,c, l*s - p + k*d]
// (x~ zero outside [0, L_in)).  The pointwise heads that follow are the
// MFMA GEMM (k_gemm with a head epilogue) and the deformable forward is the
// library's own; this file holds only the trunk (whose launch also stacks
// the two heads' weights for that GEMM when the layer is modulated).
//
// One block takes kTrLT consecutive outputs of one (b, c) row.  The row's
// input span for those outputs is staged in LDS, sized to the span, when it
// fits (each x element then leaves HBM once), else every tap reads global
// memory (bounds-checked).  Thread t computes outputs l0 + t + 256*j (j < kTrOpt),
// so every load and store of a j is coalesced.
#include "dc1d_internal.h"

namespace dc1d {
namespace {

constexpr int kTrThreads = 256;
constexpr int kTrOpt = 8;
constexpr int kTrLT = kTrThreads * kTrOpt;  // outputs per block
constexpr int kTrWinMax = 16384;            // largest LDS window (floats)
constexpr int kTrFill = 9;                  // window loads per thread in flight together

// win: the LDS window's capacity in floats (the span of a full tile), or 0
// when that would exceed kTrWinMax (every tap then reads global memory).
template <class D>
__global__ void __launch_bounds__(kTrThreads) k_trunk(TrunkArgs a, int tiles_l, int win_cap) {
    using T = typename D::T;
    extern __shared__ float s_x[];
    const int64_t blk = blockIdx.x;
    const int64_t row = blk / tiles_l;  // b*C + c
    const int tile = (int)(blk - row * tiles_l);
    const int c = (int)(row % a.C);
    const int l0 = tile * kTrLT;
    if (a.wcat) {  // the heads' stacking, spread over the grid
        const int64_t nw = (int64_t)a.GK * a.C, n = nw > a.GK ? nw : a.GK;
        for (int64_t i = blk * kTrThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kTrThreads) {
            if (i < nw) {
                a.wcat[i] = a.ow[i];
                a.wcat[nw + i] = a.mw[i];
            }
            if (i < a.GK) {
                a.bcat[i] = a.ob ? a.ob[i] : 0.0f;
                a.bcat[a.GK + i] = a.mb ? a.mb[i] : 0.0f;
            }
        }
    }
    const T *__restrict__ xr = (const T *)a.x + row * a.L_in;
    const int K = a.K, s = a.stride, d = a.dilation;
    const int lo = l0 * s - a.padding;
    const int nout = min(kTrLT, a.L_out - l0);
    const int span = (nout - 1) * s + (K - 1) * d + 1;
    const bool win = span <= win_cap;
    if (win) {
        // kTrFill loads per thread issued together, then the rest (spans
        // beyond kTrFill * kTrThreads: strides or dilations above one)
        float v[kTrFill];
#pragma unroll
        for (int q = 0; q < kTrFill; ++q) {
            const int i = threadIdx.x + kTrThreads * q, pos = lo + i;
            v[q] = (i < span && pos >= 0 && pos < a.L_in) ? D::ld(xr, pos) : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < kTrFill; ++q) {
            const int i = threadIdx.x + kTrThreads * q;
            if (i < span) s_x[i] = v[q];
        }
        for (int i = threadIdx.x + kTrThreads * kTrFill; i < span; i += kTrThreads) {
            const int pos = lo + i;
            s_x[i] = (pos >= 0 && pos < a.L_in) ? D::ld(xr, pos) : 0.0f;
        }
        __syncthreads();
    }
    const float *__restrict__ tw = a.tw + (int64_t)c * K;
    const float bias = a.tb ? a.tb[c] : 0.0f;
    float *__restrict__ tr = a.t + row * a.L_out;
#pragma unroll
    for (int j = 0; j < kTrOpt; ++j) {
        const int lo_j = threadIdx.x + kTrThreads * j;  // output index inside the tile
        if (lo_j >= nout) break;
        float acc = 0.0f;
        if (win) {
            for (int k = 0; k < K; ++k) acc += tw[k] * s_x[lo_j * s + k * d];
        } else {
            for (int k = 0; k < K; ++k) {
                const int pos = lo + lo_j * s + k * d;
                acc += tw[k] * ((pos >= 0 && pos < a.L_in) ? D::ld(xr, pos) : 0.0f);
            }
        }
        tr[l0 + lo_j] = acc + bias;
    }
}

}  // namespace

hipError_t launch_trunk(const TrunkArgs &a, hipStream_t stream) {
    if (a.B == 0 || a.L_out == 0) return hipSuccess;
    const int tiles_l = (a.L_out + kTrLT - 1) / kTrLT;
    const int64_t blocks = (int64_t)a.B * a.C * tiles_l;
    if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int64_t span = (int64_t)(kTrLT - 1) * a.stride + (int64_t)(a.K - 1) * a.dilation + 1;
    const int win_cap = span <= kTrWinMax ? (int)span : 0;
    if (a.dtype == kF32)
        hipLaunchKernelGGL((k_trunk<F32>), dim3((unsigned)blocks), dim3(kTrThreads), (size_t)win_cap * 4, stream, a,
                           tiles_l, win_cap);
    else if (a.dtype == kBF16)
        hipLaunchKernelGGL((k_trunk<BF16>), dim3((unsigned)blocks), dim3(kTrThreads), (size_t)win_cap * 4, stream,
                           a, tiles_l, win_cap);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace dc1d
