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
// Dense shapes (groups == 1), in order on the caller's stream:
//   k_bwd_zero       clears grad_x (it is accumulated with atomics);
//   k_transpose      W -> W^T [C_in*K][C_out] (workspace);
//   k_gemm           dS = W^T dout on the MFMA kernel, [B][C_in*K][L_out];
//   k_bwd_samples_t  per (b, l, ci, k): the sample S in [(b,l)][C_in*K]
//                    (for the weight gradient) and dS scattered into grad_x;
//   k_bwd_offmask    per (b, g, l, k): offset and mask gradients from dS;
//   k_restride_dout  dout -> [C_out][B*L_out];
//   k_gemm           grad_weight = dout S^T on the MFMA kernel;
//   k_bwd_bias       one workgroup per output channel.
// Other shapes: k_bwd_samples (dS by a loop over the group's output
// channels, S and the grad_x scatter per (b, ci, k, l)), k_bwd_offmask,
// k_bwd_weight (one workgroup per (co, ci_local)), k_bwd_bias.
#include "dc1d_internal.h"

#include <algorithm>

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

// Dense path (groups == 1): dS = W^T dout and grad_weight = dout S^T are
// two plain GEMMs on the MFMA kernel.  This kernel writes the samples for
// the weight gradient in the GEMM's layout [(b, l)][ci*K + k] (one thread
// per element, (ci, k) fastest) and scatters dS into grad_x.
__global__ void __launch_bounds__(256) k_bwd_samples_t(BwdParams a) {
    const Params &p = a.p;
    const float *__restrict__ x = (const float *)p.x;
    const float *__restrict__ off = (const float *)p.off;
    const float *__restrict__ mask = (const float *)p.mask;
    const int CK = p.C_in * p.K;
    const int64_t n = (int64_t)p.B * p.L_out * CK;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        const int r = (int)(e % CK);
        const int64_t bl = e / CK;
        const int l = (int)(bl % p.L_out);
        const int b = (int)(bl / p.L_out);
        const int ci = r / p.K, k = r - ci * p.K, g = ci / p.cpo;
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
            const float ds = a.dS[((int64_t)b * CK + r) * p.L_out + l];
            float *grow = a.gx + ((int64_t)b * p.C_in + ci) * p.L_in;
            const float dm = ds * m;
            if (v0) unsafeAtomicAdd(grow + i0, dm * (1.0f - f));
            if (v1) unsafeAtomicAdd(grow + i0 + 1, dm * f);
        }
    }
}

// out[c][r] = in[r][c] for a rows x cols matrix (32 x 32 tiles through LDS).
__global__ void __launch_bounds__(256) k_transpose(const float *__restrict__ in, float *__restrict__ out, int rows,
                                                   int cols) {
    __shared__ float tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 32 x 8
    for (int j = ty; j < 32; j += 8)
        if (r0 + j < rows && c0 + tx < cols) tile[j][tx] = in[(int64_t)(r0 + j) * cols + c0 + tx];
    __syncthreads();
    for (int j = ty; j < 32; j += 8)
        if (c0 + j < cols && r0 + tx < rows) out[(int64_t)(c0 + j) * rows + r0 + tx] = tile[tx][j];
}

// A[co][b*L_out + l] = dout[b][co][l]
__global__ void __launch_bounds__(256) k_restride_dout(BwdParams a, float *__restrict__ A) {
    const Params &p = a.p;
    const int64_t n = (int64_t)p.B * p.C_out * p.L_out;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        const int l = (int)(e % p.L_out);
        const int64_t r = e / p.L_out;
        const int co = (int)(r % p.C_out);
        const int b = (int)(r / p.C_out);
        A[((int64_t)co * p.B + b) * p.L_out + l] = a.dout[e];
    }
}

unsigned grid_for(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < (1 << 20) ? (b > 0 ? b : 1) : (1 << 20));
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

bool dense_path(const Params &p) {
    return p.groups == 1 && (int64_t)p.B * p.L_out < ((int64_t)1 << 31) && (int64_t)p.C_in * p.K < ((int64_t)1 << 31) &&
           p.C_out <= 65535 * 32;  // transpose grid
}

// The GEMM arguments of the two dense contractions.
Params gemm_ds(const Params &p, const float *wt, const float *dout, float *dS, void *ws) {
    Params q = {};
    q.dtype = kF32;
    q.w = wt;           // W^T [C_in*K][C_out]
    q.x = dout;         // B(k = co, n = (b, l)) = dout[b][co][l]
    q.out = dS;         // [B][C_in*K][L_out]
    q.B = p.B;
    q.C_out = p.C_in * p.K;
    q.Kred = p.C_out;
    q.L_out = p.L_out;
    q.ws = ws;
    return q;
}
Params gemm_dw(const Params &p, const float *A, const float *S, float *gw, void *ws) {
    Params q = {};
    q.dtype = kF32;
    q.w = A;            // dout as [C_out][B*L_out]
    q.x = S;            // B(k = (b, l), n = ci*K + k) = S[(b, l)][ci*K + k]
    q.out = gw;         // [1][C_out][C_in*K]
    q.B = 1;
    q.C_out = p.C_out;
    q.Kred = p.B * p.L_out;
    q.L_out = p.C_in * p.K;
    q.ws = ws;
    return q;
}

struct BwdLayout {
    size_t dS, wt, S, A, part, total;
};

BwdLayout layout(const Params &p, bool want_weight, int num_cus) {
    BwdLayout L = {};
    const size_t nds = (size_t)p.B * p.C_in * p.K * p.L_out * 4;
    size_t o = 0;
    L.dS = o;
    o += align256(nds);
    if (dense_path(p)) {
        L.wt = o;
        o += align256((size_t)p.C_out * p.C_in * p.K * 4);
        size_t part = gemm_workspace_bytes(gemm_ds(p, nullptr, nullptr, nullptr, nullptr), num_cus);
        if (want_weight) {
            L.S = o;
            o += align256(nds);
            L.A = o;
            o += align256((size_t)p.B * p.C_out * p.L_out * 4);
            part = std::max(part, gemm_workspace_bytes(gemm_dw(p, nullptr, nullptr, nullptr, nullptr), num_cus));
        }
        L.part = o;
        o += align256(part);
    } else if (want_weight) {
        L.S = o;
        o += align256(nds);
    }
    L.total = o;
    return L;
}

}  // namespace

size_t backward_workspace_bytes(const Params &p, bool want_weight, int num_cus) {
    return layout(p, want_weight, num_cus).total;
}

hipError_t launch_backward(BwdParams a, int num_cus, hipStream_t stream) {
    const Params &p = a.p;
    const int64_t n = (int64_t)p.B * p.C_in * p.K * p.L_out;
    char *ws = (char *)a.dS;  // the workspace base
    const BwdLayout L = layout(p, a.gw != nullptr, num_cus);
    if (a.gx) {
        const int64_t nx = (int64_t)p.B * p.C_in * p.L_in;
        hipLaunchKernelGGL(k_bwd_zero, dim3(grid_for(nx)), dim3(256), 0, stream, a.gx, nx);
    }
    const bool want_ds = a.gx || a.goff || a.gmask || a.gw;
    if (n > 0 && want_ds && dense_path(p)) {
        float *wt = (float *)(ws + L.wt);
        const int CK = p.C_in * p.K;
        hipLaunchKernelGGL(k_transpose, dim3((unsigned)((CK + 31) / 32), (unsigned)((p.C_out + 31) / 32)), dim3(256),
                           0, stream, (const float *)p.w, wt, p.C_out, CK);
        hipError_t e = launch_gemm_f32(gemm_ds(p, wt, a.dout, a.dS, ws + L.part), p.L_out, (int64_t)p.C_out * p.L_out,
                                       num_cus, stream);
        if (e != hipSuccess) return e;
        a.S = a.gw ? (float *)(ws + L.S) : nullptr;
        if (a.gx || a.S) hipLaunchKernelGGL(k_bwd_samples_t, dim3(grid_for(n)), dim3(256), 0, stream, a);
        if (a.goff || a.gmask) {
            const int64_t no = (int64_t)p.B * p.G * p.L_out * p.K;
            hipLaunchKernelGGL(k_bwd_offmask, dim3(grid_for(no)), dim3(256), 0, stream, a);
        }
        if (a.gw) {
            float *A = (float *)(ws + L.A);
            const int64_t nd = (int64_t)p.B * p.C_out * p.L_out;
            hipLaunchKernelGGL(k_restride_dout, dim3(grid_for(nd)), dim3(256), 0, stream, a, A);
            e = launch_gemm_f32(gemm_dw(p, A, a.S, a.gw, ws + L.part), CK, 0, num_cus, stream);
            if (e != hipSuccess) return e;
        }
    } else if (n > 0 && want_ds) {
        a.S = a.gw ? (float *)(ws + L.S) : nullptr;
        hipLaunchKernelGGL(k_bwd_samples, dim3(grid_for(n)), dim3(256), 0, stream, a);
        if (a.goff || a.gmask) {
            const int64_t no = (int64_t)p.B * p.G * p.L_out * p.K;
            hipLaunchKernelGGL(k_bwd_offmask, dim3(grid_for(no)), dim3(256), 0, stream, a);
        }
        if (a.gw) hipLaunchKernelGGL(k_bwd_weight, dim3((unsigned)(p.C_out * p.cpg)), dim3(256), 0, stream, a);
    }
    if (a.gw && n == 0) {
        const int64_t nw = (int64_t)p.C_out * p.cpg * p.K;
        hipLaunchKernelGGL(k_bwd_zero, dim3(grid_for(nw)), dim3(256), 0, stream, a.gw, nw);
    }
    if (a.gb) hipLaunchKernelGGL(k_bwd_bias, dim3((unsigned)p.C_out), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dc1d
