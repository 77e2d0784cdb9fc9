// k_backward.hip -- gradients of the forward: for an incoming gradient dout
// of the output, the gradients of sum(dout * out) with respect to x, the
// offsets, the mask, the weight and the bias (fp32 storage).
//
// They are the derivatives of the forward taken term by term (the dc1d page
// trains the offsets and checks their gradient against a finite difference,
// section Demo notebook):
//   dS[b,ci,k,l] = sum over the group's output channels of w[co,ci_local,k] * dout[b,co,l]
//   grad_x[b,ci,i0] += dS * m * (1 - f),  grad_x[b,ci,i0+1] += dS * m * f   (inside [0, L_in))
//   grad_offsets[b,g,l,k] = sum over ci in g of dS * m * (x~(i0+1) - x~(i0))
//   grad_mask[b,g,l,k]    = sum over ci in g of dS * ((1-f) x~(i0) + f x~(i0+1))
//   grad_weight[co,cl,k]  = sum over (b, l) of dout[b,co,l] * S[b,ci,k,l]
//   grad_bias[co]         = sum over (b, l) of dout[b,co,l]
// with i0, f the position split of the forward (split_position) and S the
// forward's interpolated, modulated sample.  The offset derivative is the
// interpolation formula's with i0 held fixed (the right derivative at
// integer offsets).
//
// Kernels (one pass each, in this order on the caller's stream):
//   k_bwd_zero     clears grad_x (it is accumulated with atomics);
//   k_bwd_samples  one thread per (b, ci, k, l): dS, the sample S (for the
//                  weight gradient) and the two grad_x contributions;
//   k_bwd_offmask  one thread per (b, g, l, k): the offset and mask
//                  gradients, summed over the group's channels from dS;
//   k_bwd_weight   one workgroup per weight element row: dout against S;
//   k_bwd_bias     one workgroup per output channel.
// dS and S live in the workspace as [B][C_in][K][L_out] fp32.
#include "dc1d_internal.h"

namespace dc1d {

namespace {

__global__ void __launch_bounds__(256) k_bwd_zero(float *__restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

__global__ void __launch_bounds__(256) k_bwd_samples(BwdParams a) {
    const Params &p = a.p;
    const float *__restrict__ x = (const float *)p.x;
    const float *__restrict__ off = (const float *)p.off;
    const float *__restrict__ mask = (const float *)p.mask;
    const float *__restrict__ w = (const float *)p.w;
    const int64_t n = (int64_t)p.B * p.C_in * p.K * p.L_out;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        const int l = (int)(e % p.L_out);
        const int64_t r1 = e / p.L_out;
        const int k = (int)(r1 % p.K);
        const int64_t r2 = r1 / p.K;
        const int ci = (int)(r2 % p.C_in);
        const int b = (int)(r2 / p.C_in);
        const int grp = ci / p.cpg, cl = ci - grp * p.cpg, g = ci / p.cpo;
        // dS: the group's output channels against this tap's weights
        const float *dcol = a.dout + ((int64_t)b * p.C_out + (int64_t)grp * p.opg) * p.L_out + l;
        const float *wcol = w + ((int64_t)grp * p.opg * p.cpg + cl) * p.K + k;
        float ds = 0.0f;
        for (int oc = 0; oc < p.opg; ++oc) ds = fmaf(wcol[(int64_t)oc * p.cpg * p.K], dcol[(int64_t)oc * p.L_out], ds);
        a.dS[e] = ds;
        const int64_t oi = (((int64_t)b * p.G + g) * p.L_out + l) * p.K + k;
        int i0;
        float f;
        split_position(off[oi], l * p.stride - p.padding + k * p.dilation, i0, f);
        const float m = mask ? mask[oi] : 1.0f;
        const float *xrow = x + ((int64_t)b * p.C_in + ci) * p.L_in;
        const bool v0 = i0 >= 0 && i0 < p.L_in, v1 = i0 + 1 >= 0 && i0 + 1 < p.L_in;
        if (a.S) {
            const float x0 = v0 ? xrow[i0] : 0.0f, x1 = v1 ? xrow[i0 + 1] : 0.0f;
            a.S[e] = fmaf(f, x1 - x0, x0) * m;
        }
        if (a.gx) {
            float *grow = a.gx + ((int64_t)b * p.C_in + ci) * p.L_in;
            const float dm = ds * m;
            if (v0) unsafeAtomicAdd(grow + i0, dm * (1.0f - f));
            if (v1) unsafeAtomicAdd(grow + i0 + 1, dm * f);
        }
    }
}

__global__ void __launch_bounds__(256) k_bwd_offmask(BwdParams a) {
    const Params &p = a.p;
    const float *__restrict__ x = (const float *)p.x;
    const float *__restrict__ off = (const float *)p.off;
    const float *__restrict__ mask = (const float *)p.mask;
    const int64_t n = (int64_t)p.B * p.G * p.L_out * p.K;
    for (int64_t oi = (int64_t)blockIdx.x * 256 + threadIdx.x; oi < n; oi += (int64_t)gridDim.x * 256) {
        const int k = (int)(oi % p.K);
        const int64_t r1 = oi / p.K;
        const int l = (int)(r1 % p.L_out);
        const int64_t r2 = r1 / p.L_out;
        const int g = (int)(r2 % p.G);
        const int b = (int)(r2 / p.G);
        int i0;
        float f;
        split_position(off[oi], l * p.stride - p.padding + k * p.dilation, i0, f);
        const float m = mask ? mask[oi] : 1.0f;
        const bool v0 = i0 >= 0 && i0 < p.L_in, v1 = i0 + 1 >= 0 && i0 + 1 < p.L_in;
        float ao = 0.0f, am = 0.0f;
        for (int ci = g * p.cpo; ci < (g + 1) * p.cpo; ++ci) {
            const float *xrow = x + ((int64_t)b * p.C_in + ci) * p.L_in;
            const float x0 = v0 ? xrow[i0] : 0.0f, x1 = v1 ? xrow[i0 + 1] : 0.0f;
            const float ds = a.dS[(((int64_t)b * p.C_in + ci) * p.K + k) * p.L_out + l];
            ao = fmaf(ds * m, x1 - x0, ao);
            am = fmaf(ds, fmaf(f, x1 - x0, x0), am);
        }
        if (a.goff) a.goff[oi] = ao;
        if (a.gmask) a.gmask[oi] = am;
    }
}

// One workgroup per (co, cl): its K weight gradients, each a sum over
// (b, l) of dout[b, co, l] * S[b, ci, k, l]; threads stride over l, then a
// tree reduction in LDS (fixed order: deterministic).
__global__ void __launch_bounds__(256) k_bwd_weight(BwdParams a) {
    const Params &p = a.p;
    __shared__ float s_red[256];
    const int row = blockIdx.x;  // co * cpg + cl
    const int co = row / p.cpg, cl = row - co * p.cpg;
    const int ci = (co / p.opg) * p.cpg + cl;
    for (int k = 0; k < p.K; ++k) {
        float acc = 0.0f;
        for (int b = 0; b < p.B; ++b) {
            const float *d = a.dout + ((int64_t)b * p.C_out + co) * p.L_out;
            const float *srow = a.S + (((int64_t)b * p.C_in + ci) * p.K + k) * p.L_out;
            for (int l = threadIdx.x; l < p.L_out; l += 256) acc = fmaf(d[l], srow[l], acc);
        }
        s_red[threadIdx.x] = acc;
        __syncthreads();
        for (int h = 128; h > 0; h >>= 1) {
            if ((int)threadIdx.x < h) s_red[threadIdx.x] += s_red[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) a.gw[(int64_t)row * p.K + k] = s_red[0];
        __syncthreads();
    }
}

__global__ void __launch_bounds__(256) k_bwd_bias(BwdParams a) {
    const Params &p = a.p;
    __shared__ float s_red[256];
    const int co = blockIdx.x;
    float acc = 0.0f;
    for (int b = 0; b < p.B; ++b) {
        const float *d = a.dout + ((int64_t)b * p.C_out + co) * p.L_out;
        for (int l = threadIdx.x; l < p.L_out; l += 256) acc += d[l];
    }
    s_red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) s_red[threadIdx.x] += s_red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.gb[co] = s_red[0];
}

unsigned grid_for(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < (1 << 20) ? (b > 0 ? b : 1) : (1 << 20));
}

}  // namespace

size_t backward_workspace_bytes(const Params &p, bool want_weight) {
    const size_t n = (size_t)p.B * p.C_in * p.K * p.L_out;
    const size_t one = (n * 4 + 255) & ~(size_t)255;
    return one * (want_weight ? 2 : 1);
}

hipError_t launch_backward(BwdParams a, hipStream_t stream) {
    const Params &p = a.p;
    const int64_t n = (int64_t)p.B * p.C_in * p.K * p.L_out;
    if (a.gx) {
        const int64_t nx = (int64_t)p.B * p.C_in * p.L_in;
        hipLaunchKernelGGL(k_bwd_zero, dim3(grid_for(nx)), dim3(256), 0, stream, a.gx, nx);
    }
    if (n > 0 && (a.gx || a.goff || a.gmask || a.gw)) {
        hipLaunchKernelGGL(k_bwd_samples, dim3(grid_for(n)), dim3(256), 0, stream, a);
        if (a.goff || a.gmask) {
            const int64_t no = (int64_t)p.B * p.G * p.L_out * p.K;
            hipLaunchKernelGGL(k_bwd_offmask, dim3(grid_for(no)), dim3(256), 0, stream, a);
        }
    }
    if (a.gw) {
        if (n > 0) {
            hipLaunchKernelGGL(k_bwd_weight, dim3((unsigned)(p.C_out * p.cpg)), dim3(256), 0, stream, a);
        } else {
            const int64_t nw = (int64_t)p.C_out * p.cpg * p.K;
            hipLaunchKernelGGL(k_bwd_zero, dim3(grid_for(nw)), dim3(256), 0, stream, a.gw, nw);
        }
    }
    if (a.gb) hipLaunchKernelGGL(k_bwd_bias, dim3((unsigned)p.C_out), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dc1d
