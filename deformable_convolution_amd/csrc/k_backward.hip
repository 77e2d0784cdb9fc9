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
// Kernels, in order on the caller's stream:
//   k_bwd_zero_set   clears, in one launch, grad_x when it is scattered and
//                    (other than on dense shapes) the gather's flag;
//   dS               dense shapes (groups == 1): k_transpose W -> W^T (it
//                    also clears the gather's flag), then
//                    k_gemm dS = W^T dout on the MFMA kernel; other shapes:
//                    k_bwd_samples (a loop over the group's output channels);
//                    dS is [B][C_in][K][L_out] in the workspace;
//   samples          for the weight gradient: k_bwd_samples_t writes them in
//                    the weight GEMM's layout [(b, l)][C_in*K] (dense, one
//                    workgroup per row), or
//                    k_bwd_samples beside dS as [B][C_in][K][L_out];
//   k_bwd_dx         grad_offsets, grad_mask from dS (tiled, LDS windows),
//                    and grad_x (LDS atomics) when the gather does not fit;
//   k_bwd_dxg        grad_x gathered from dS (no clear, no atomics), then
//                    k_bwd_dxg_fix for samples moved beyond its reach;
//   weight gradient  dense: k_restride_bias (dout restrided, and grad_bias
//                    from the same reads) then k_gemm grad_weight =
//                    dout S^T; other shapes: k_bwd_weight;
//   k_bwd_bias       (where k_restride_bias did not run) one workgroup per
//                    output channel, fixed order, no atomics.
#include "dc1d_internal.h"

#include <algorithm>

namespace dc1d {

namespace {

__global__ void __launch_bounds__(256) k_bwd_zero(float *__restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

// Up to six buffers cleared in one launch (the clears a backward call
// needs before its accumulating kernels; one launch instead of several).
struct ZeroSet {
    float *p[6];
    int64_t n[6];
    int count;
    int64_t most;
    void add(float *q, int64_t m) {
        if (q && m > 0) {
            p[count] = q;
            n[count] = m;
            ++count;
            if (m > most) most = m;
        }
    }
};

__global__ void __launch_bounds__(256) k_bwd_zero_set(ZeroSet z) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int b = 0; b < z.count; ++b)
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < z.n[b]; i += stride) z.p[b][i] = 0.0f;
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
        split_position(off[oi], l * p.stride - p.padding + k * p.dilation, tap_range(p, k), i0, f);
        const float m = mask ? mask[oi] : 1.0f;
        const float *xrow = x + ((int64_t)b * p.C_in + ci) * p.L_in;
        const bool v0 = i0 >= 0 && i0 < p.L_in, v1 = i0 + 1 >= 0 && i0 + 1 < p.L_in;
        if (a.S) {
            const float x0 = v0 ? xrow[i0] : 0.0f, x1 = v1 ? xrow[i0 + 1] : 0.0f;
            a.S[e] = fmaf(f, x1 - x0, x0) * m;
        }
    }
}

// One workgroup per weight element (co, cl, k): a sum over (b, l) of
// dout[b, co, l] * S[b, ci, k, l]; threads stride over l, then a tree
// reduction in LDS (fixed order: deterministic).
__global__ void __launch_bounds__(256) k_bwd_weight(BwdParams a) {
    const Params &p = a.p;
    __shared__ float s_red[256];
    const int e = blockIdx.x;  // (co * cpg + cl) * K + k
    const int k = e % p.K, row = e / p.K;
    const int co = row / p.cpg, cl = row - co * p.cpg;
    const int ci = (co / p.opg) * p.cpg + cl;
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
    if (threadIdx.x == 0) a.gw[e] = s_red[0];
}

// One workgroup per output channel co: grad_bias[co] = the sum of its dout
// rows over the batch, in a fixed order (thread t adds elements t, t + 256,
// ... of the channel's B * L_out values, b-major; then a tree over the
// threads) and stored once: no clear, no atomics, the same bits on every
// run.  (The flat index keeps several independent loads in flight per
// thread when the rows are short.)
__global__ void __launch_bounds__(256) k_bwd_bias(BwdParams a) {
    const Params &p = a.p;
    __shared__ float s_red[256];
    const int co = blockIdx.x;
    const int64_t n = (int64_t)p.B * p.L_out;
    const float *d = a.dout + (int64_t)co * p.L_out;
    float acc = 0.0f;
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < n; i += 256) {
        const int64_t b = i / p.L_out, l = i - b * p.L_out;
        acc += d[b * p.C_out * p.L_out + l];
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
// the weight gradient in the GEMM's layout [(b, l)][ci*K + k]: a workgroup
// per row (b, l) (grid-stride), (ci, k) fastest, 32-bit index arithmetic
// inside a row.
//
// Workgroups are dealt to the 8 XCDs in turn (id mod 8), each XCD with its
// own L2; with one workgroup per row the ids are remapped so that each XCD
// takes a contiguous run of rows -- whole batches, whose x rows it then
// fetches alone -- instead of every XCD fetching all of x.
constexpr int kSampU = 4;
__global__ void __launch_bounds__(256) k_bwd_samples_t(BwdParams a, FastDiv fd_K, FastDiv fd_cpo) {
    const Params &p = a.p;
    const float *__restrict__ off = (const float *)p.off;
    const float *__restrict__ mask = (const float *)p.mask;
    const int K = p.K, CK = p.C_in * K, L_in = p.L_in;
    const int64_t rows = (int64_t)p.B * p.L_out;
    int64_t first = blockIdx.x;
    if ((int64_t)gridDim.x == rows) {  // XCD j takes rows [j*q + min(j, r), ...), q = rows / 8, r = rows % 8
        const int U = (int)gridDim.x, q = U >> 3, r = U & 7, xcd = (int)blockIdx.x & 7, loc = (int)blockIdx.x >> 3;
        first = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + loc;
    }
    for (int64_t bl = first; bl < rows; bl += gridDim.x) {
        const int b = (int)(bl / p.L_out), l = (int)(bl - (int64_t)b * p.L_out);
        const float *__restrict__ xb = (const float *)p.x + (int64_t)b * p.C_in * L_in;
        const int64_t orow = (int64_t)b * p.G * p.L_out + l;  // offsets row (b, g = 0) at l
        const int base0 = l * p.stride - p.padding;
        float *__restrict__ dst = a.S + bl * CK;
        // four elements per thread at a time, every load and store
        // unconditional (x at clamped positions, zeroed outside [0, L_in);
        // lanes past the row's end redo its last element, the same value at
        // the same address), so the loads of the four are in flight together
        // and waiting for them never waits for the previous stores
        for (int r0 = threadIdx.x; r0 < CK; r0 += 256 * kSampU) {
            int rr[kSampU], ci[kSampU], k[kSampU];
            float o[kSampU], m[kSampU];
#pragma unroll
            for (int u = 0; u < kSampU; ++u) {
                rr[u] = min(r0 + 256 * u, CK - 1);
                ci[u] = (int)fdiv((uint32_t)rr[u], fd_K);
                k[u] = rr[u] - ci[u] * K;
                const int g = (int)fdiv((uint32_t)ci[u], fd_cpo);
                const int64_t oi = (orow + (int64_t)g * p.L_out) * K + k[u];
                o[u] = off[oi];
                m[u] = mask ? mask[oi] : 1.0f;
            }
            float x0[kSampU], x1[kSampU], f[kSampU];
            bool v0[kSampU], v1[kSampU];
#pragma unroll
            for (int u = 0; u < kSampU; ++u) {
                int i0;
                split_position(o[u], base0 + k[u] * p.dilation, tap_range(p, k[u]), i0, f[u]);
                v0[u] = i0 >= 0 && i0 < L_in;
                v1[u] = i0 + 1 >= 0 && i0 + 1 < L_in;
                const float *__restrict__ xrow = xb + (int64_t)ci[u] * L_in;
                x0[u] = xrow[min(max(i0, 0), L_in - 1)];
                x1[u] = xrow[min(max(i0 + 1, 0), L_in - 1)];
            }
#pragma unroll
            for (int u = 0; u < kSampU; ++u) {
                const float a0 = v0[u] ? x0[u] : 0.0f, a1 = v1[u] ? x1[u] : 0.0f;
                dst[rr[u]] = fmaf(f[u], a1 - a0, a0) * m[u];
            }
        }
    }
}

// grad_x, grad_offsets and grad_mask from dS, tiled.  A workgroup takes
// one batch b, a block of CBX channels inside one offset group and LT
// consecutive outputs; each thread owns fixed (k, l) pairs, splits their
// positions once, and loops over the block's channels reading dS (coalesced
// along l) and x from an LDS window of the rows (the tile's span plus
// kBwdMargin on each side, zero outside [0, L_in)).  The grad_x
// contributions accumulate in an LDS window (LDS atomics) that is added to
// grad_x once at the end; samples moved outside the window use global
// atomics directly.  The offset and mask gradients of a pair accumulate in
// registers over the block's channels and are stored: straight into the
// gradients when a block holds the whole offset group, else into the
// block's slot of the workspace (the group's channel blocks each own one,
// [nsub][2][B*G*L_out*K]), which k_bwd_om_sum adds in slot order -- no
// atomics, the same bits on every run.
constexpr int kBwdMargin = 32;
constexpr int kFillU = 8;  // window entries per thread loaded together

struct DxPlan {
    int cbx, lt, win, tiles_l, ngrp_blocks;
    bool atomic_om;  // several channel blocks per offset group: their sums go to slots
    int nsub;        // channel blocks per offset group (slots)
    size_t lds;
};

__global__ void __launch_bounds__(256) k_bwd_dx(BwdParams a, DxPlan pl, float *__restrict__ om_slots) {
    const Params &p = a.p;
    extern __shared__ float smem[];
    const int CBX = pl.cbx, LT = pl.lt, W = pl.win;
    float *xs = smem;                  // [CBX][W]
    float *gacc = smem + CBX * W;      // [CBX][W]
    const int K = p.K, L_in = p.L_in, L_out = p.L_out;
    int blk = blockIdx.x;
    const int tile = blk % pl.tiles_l;
    blk /= pl.tiles_l;
    const int cblk = blk % pl.ngrp_blocks;  // channel block over all of C_in
    const int b = blk / pl.ngrp_blocks;
    const int ci0 = cblk * CBX, g = ci0 / p.cpo;
    const int l0 = tile * LT;
    const int lo = l0 * p.stride - p.padding - kBwdMargin;
    const float *__restrict__ x = (const float *)p.x + ((int64_t)b * p.C_in + ci0) * L_in;
    // the windows, kFillU entries per thread at a time: loads at clamped
    // (in-bounds) entries and positions, all in flight before the LDS
    // writes (zero outside [0, L_in); lanes past the end write nothing)
    const int nwin = CBX * W;
    for (int e0 = threadIdx.x; e0 < nwin; e0 += 256 * kFillU) {
        float v[kFillU];
#pragma unroll
        for (int u = 0; u < kFillU; ++u) {
            const int e = min(e0 + 256 * u, nwin - 1);
            const int c = e / W, j = e - c * W;
            v[u] = x[(int64_t)c * L_in + min(max(lo + j, 0), L_in - 1)];
        }
#pragma unroll
        for (int u = 0; u < kFillU; ++u) {
            const int e = e0 + 256 * u;
            if (e < nwin) {
                const int c = e / W, pos = lo + (e - c * W);
                xs[e] = (pos >= 0 && pos < L_in) ? v[u] : 0.0f;
                gacc[e] = 0.0f;
            }
        }
    }
    __syncthreads();
    const float *__restrict__ off = (const float *)p.off;
    const float *__restrict__ mask = (const float *)p.mask;
    float *__restrict__ gx = a.gx ? a.gx + ((int64_t)b * p.C_in + ci0) * L_in : nullptr;
    // pairs (k, l) of the tile, l fastest; thread t owns pairs t, t+256, ...
    const int npair = K * LT;
    for (int pq = threadIdx.x; pq < npair; pq += 256) {
        const int k = pq / LT, ll = pq - k * LT, l = l0 + ll;
        if (l >= L_out) continue;
        const int64_t oi = (((int64_t)b * p.G + g) * L_out + l) * K + k;
        int i0;
        float f;
        split_position(off[oi], l * p.stride - p.padding + k * p.dilation, tap_range(p, k), i0, f);
        const float m = mask ? mask[oi] : 1.0f;
        const int j = i0 - lo;
        const bool inwin = W > 1 && (unsigned)j < (unsigned)(W - 1);
        const bool v0 = i0 >= 0 && i0 < L_in, v1 = i0 + 1 >= 0 && i0 + 1 < L_in;
        const float *__restrict__ dsp = a.dS + (((int64_t)b * p.C_in + ci0) * K + k) * L_out + l;
        const int64_t dstride = (int64_t)K * L_out;
        float ao = 0.0f, am = 0.0f;
        for (int c0 = 0; c0 < CBX; c0 += 8) {
            // eight channels' dS in flight at once (clamped reads; channels
            // past the block are skipped below)
            float dsv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) dsv[u] = dsp[(int64_t)min(c0 + u, CBX - 1) * dstride];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
            const int c = c0 + u;
            if (c >= CBX) break;
            const float ds = dsv[u];
            float x0, x1;
            if (inwin) {
                x0 = xs[c * W + j];
                x1 = xs[c * W + j + 1];
            } else {
                const float *xr = x + (int64_t)c * L_in;
                x0 = v0 ? xr[i0] : 0.0f;
                x1 = v1 ? xr[i0 + 1] : 0.0f;
            }
            ao = fmaf(ds * m, x1 - x0, ao);
            am = fmaf(ds, fmaf(f, x1 - x0, x0), am);
            if (gx) {
                const float dm = ds * m;
                if (inwin) {
                    atomicAdd(gacc + c * W + j, dm * (1.0f - f));
                    atomicAdd(gacc + c * W + j + 1, dm * f);
                } else {
                    if (v0) unsafeAtomicAdd(gx + (int64_t)c * L_in + i0, dm * (1.0f - f));
                    if (v1) unsafeAtomicAdd(gx + (int64_t)c * L_in + i0 + 1, dm * f);
                }
            }
            }
        }
        if (!tap_moves(p, off[oi], tap_range(p, k))) ao = 0.0f;  // a clamped tap: its offset has no effect
        if (pl.atomic_om) {
            const int64_t no = (int64_t)p.B * p.G * L_out * K;
            float *slot = om_slots + (int64_t)(cblk % pl.nsub) * 2 * no;
            if (a.goff) slot[oi] = ao;
            if (a.gmask) slot[no + oi] = am;
        } else {
            if (a.goff) a.goff[oi] = ao;
            if (a.gmask) a.gmask[oi] = am;
        }
    }
    if (!gx) return;
    __syncthreads();
    for (int e = threadIdx.x; e < CBX * W; e += 256) {
        const int c = e / W, j = e - c * W, pos = lo + j;
        const float v = gacc[e];
        if (pos >= 0 && pos < L_in && v != 0.0f) unsafeAtomicAdd(gx + (int64_t)c * L_in + pos, v);
    }
}

// The offset and mask gradients from k_bwd_dx's slots, added in slot
// order (the group's channel blocks in channel order).
__global__ void __launch_bounds__(256) k_bwd_om_sum(BwdParams a, const float *__restrict__ om_slots, int nsub) {
    const Params &p = a.p;
    const int64_t no = (int64_t)p.B * p.G * p.L_out * p.K;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < no; i += (int64_t)gridDim.x * 256) {
        float so = 0.0f, sm = 0.0f;
        for (int s2 = 0; s2 < nsub; ++s2) {
            so += om_slots[(int64_t)s2 * 2 * no + i];
            sm += om_slots[(int64_t)s2 * 2 * no + no + i];
        }
        if (a.goff) a.goff[i] = so;
        if (a.gmask) a.gmask[i] = sm;
    }
}

DxPlan plan_dx(const Params &p) {
    DxPlan pl;
    int cbx = 1;  // the largest divisor of the offset group's channel count up to 32
    for (int c = 32; c >= 1; --c)
        if (p.cpo % c == 0) {
            cbx = c;
            break;
        }
    int lt = 2048 / p.K;  // about eight (k, l) pairs per thread
    lt = lt < 32 ? 32 : (lt > 1024 ? 1024 : lt / 32 * 32);
    if (lt > p.L_out) lt = (p.L_out + 31) / 32 * 32;
    int64_t win = (int64_t)(lt - 1) * p.stride + (int64_t)(p.K - 1) * p.dilation + 2 + 2 * kBwdMargin;
    while (2 * (size_t)cbx * win * 4 > 48 * 1024 && lt > 32) {  // keep the two windows within 48 KB
        lt /= 2;
        win = (int64_t)(lt - 1) * p.stride + (int64_t)(p.K - 1) * p.dilation + 2 + 2 * kBwdMargin;
    }
    if (2 * (size_t)cbx * win * 4 > 48 * 1024) win = 0;  // no window: everything through global memory
    pl.cbx = cbx;
    pl.lt = lt;
    pl.win = (int)win;
    pl.tiles_l = (p.L_out + lt - 1) / lt;
    pl.ngrp_blocks = p.C_in / cbx;
    pl.atomic_om = cbx < p.cpo;
    pl.nsub = p.cpo / cbx;
    pl.lds = 2 * (size_t)cbx * win * 4;
    return pl;
}

// Depthwise shapes (one input channel per group and per output channel)
// whose gather arrays do not fit in LDS (k_bwd_dwg below serves the others):
// every gradient in one pass, nothing materialised.  A block takes 512
// consecutive outputs l of one (b, c); thread t owns outputs l0 + 2t, +1 and
// all their taps.  dS = w[c,k] * dout[b,c,l] is formed on the fly; x comes
// from an LDS window of the row (the tile's span plus kDwbMargin each side)
// and grad_x accumulates in a second LDS window, added to grad_x with one
// atomic per touched position at the end (global atomics for samples moved
// outside the window).  The offset and mask gradients are stored directly
// (one channel per offset group) or added atomically (several); the weight
// gradient's partial sums are reduced over the block (registers, wave
// shuffles, LDS) and added to grad_weight with one atomic per tap.
constexpr int kDwbMargin = 64;
constexpr int kDwbOpt = 2;

template <int KT>
__global__ void __launch_bounds__(256) k_bwd_dw(BwdParams a, int WIN, int tiles_l) {
    const Params &p = a.p;
    extern __shared__ float smem[];
    float *xs = smem;           // [WIN]
    float *gacc = smem + WIN;   // [WIN]
    __shared__ float wred[KT];
    const int L_in = p.L_in, L_out = p.L_out;
    const int tile = blockIdx.x % tiles_l;
    const int row = blockIdx.x / tiles_l;  // b * C_in + c
    const int c = row % p.C_in, b = row / p.C_in;
    const int g = c / p.cpo;
    const int l0 = tile * (256 * kDwbOpt);
    const int lo = l0 * p.stride - p.padding - kDwbMargin;
    const float *__restrict__ xrow = (const float *)p.x + (int64_t)row * L_in;
    for (int j = threadIdx.x; j < WIN; j += 256) {
        const int pos = lo + j;
        xs[j] = (pos >= 0 && pos < L_in) ? xrow[pos] : 0.0f;
        gacc[j] = 0.0f;
    }
    if (threadIdx.x < KT) wred[threadIdx.x] = 0.0f;
    __syncthreads();
    const float *__restrict__ off = (const float *)p.off;
    const float *__restrict__ mask = (const float *)p.mask;
    const float *__restrict__ w = (const float *)p.w + (int64_t)c * KT;  // co = c (one output per input)
    const float *__restrict__ dout = a.dout + (int64_t)row * L_out;     // [b][co = c][l]
    float *__restrict__ gxr = a.gx ? a.gx + (int64_t)row * L_in : nullptr;
    const bool om_atomic = p.cpo > 1;
    float wk[KT], wacc[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        wk[k] = w[k];
        wacc[k] = 0.0f;
    }
    // this thread's two outputs: their 2*KT offsets (and mask values) are
    // one contiguous run, loaded up front (8-byte vectors when aligned)
    constexpr int NV = kDwbOpt * KT;
    const int lt = l0 + kDwbOpt * threadIdx.x;
    const int nvalid = min(kDwbOpt, L_out - lt);
    const int64_t e0 = (((int64_t)b * p.G + g) * L_out + lt) * KT;
    const bool vec = nvalid == kDwbOpt && ((((uintptr_t)(off + e0)) & 7) == 0) &&
                     (!mask || (((uintptr_t)(mask + e0)) & 7) == 0);
    float ov[NV], mv[NV], dv[kDwbOpt];
    if (nvalid > 0) {
        if (vec) {
#pragma unroll
            for (int q = 0; q < NV; q += 2) {
                const float2 t = *(const float2 *)(off + e0 + q);
                ov[q] = t.x;
                ov[q + 1] = t.y;
                if (mask) {
                    const float2 u = *(const float2 *)(mask + e0 + q);
                    mv[q] = u.x;
                    mv[q + 1] = u.y;
                } else {
                    mv[q] = mv[q + 1] = 1.0f;
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const bool ok = q < nvalid * KT;
                ov[q] = ok ? off[e0 + q] : 0.0f;
                mv[q] = (ok && mask) ? mask[e0 + q] : 1.0f;
            }
        }
#pragma unroll
        for (int o = 0; o < kDwbOpt; ++o) dv[o] = o < nvalid ? dout[lt + o] : 0.0f;
    }
    float go[NV], gm[NV];
#pragma unroll
    for (int o = 0; o < kDwbOpt; ++o) {
        const int l = lt + o;
        const int base0 = l * p.stride - p.padding;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int q = o * KT + k;
            go[q] = gm[q] = 0.0f;
            if (o >= nvalid) continue;
            int i0;
            float f;
            const TapRange r = tap_range(p, k);
            split_position(ov[q], base0 + k * p.dilation, r, i0, f);
            const float m = mv[q];
            const int j = i0 - lo;
            const bool inwin = WIN > 1 && (unsigned)j < (unsigned)(WIN - 1);
            float x0, x1;
            if (inwin) {
                x0 = xs[j];
                x1 = xs[j + 1];
            } else {
                x0 = (i0 >= 0 && i0 < L_in) ? xrow[i0] : 0.0f;
                x1 = (i0 + 1 >= 0 && i0 + 1 < L_in) ? xrow[i0 + 1] : 0.0f;
            }
            const float d = dv[o];
            const float ds = wk[k] * d;
            const float lerp = fmaf(f, x1 - x0, x0);
            wacc[k] = fmaf(d, lerp * m, wacc[k]);
            go[q] = tap_moves(p, ov[q], r) ? ds * m * (x1 - x0) : 0.0f;
            gm[q] = ds * lerp;
            if (gxr) {
                const float dm = ds * m;
                if (inwin) {
                    atomicAdd(gacc + j, dm * (1.0f - f));
                    atomicAdd(gacc + j + 1, dm * f);
                } else {
                    if (i0 >= 0 && i0 < L_in) unsafeAtomicAdd(gxr + i0, dm * (1.0f - f));
                    if (i0 + 1 >= 0 && i0 + 1 < L_in) unsafeAtomicAdd(gxr + i0 + 1, dm * f);
                }
            }
        }
    }
    // offset and mask gradients of the two outputs
    if (nvalid > 0 && (a.goff || a.gmask)) {
        if (om_atomic) {
#pragma unroll
            for (int q = 0; q < NV; ++q)
                if (q < nvalid * KT) {
                    if (a.goff) unsafeAtomicAdd(a.goff + e0 + q, go[q]);
                    if (a.gmask) unsafeAtomicAdd(a.gmask + e0 + q, gm[q]);
                }
        } else if (vec) {
#pragma unroll
            for (int q = 0; q < NV; q += 2) {
                if (a.goff) *(float2 *)(a.goff + e0 + q) = float2{go[q], go[q + 1]};
                if (a.gmask) *(float2 *)(a.gmask + e0 + q) = float2{gm[q], gm[q + 1]};
            }
        } else {
#pragma unroll
            for (int q = 0; q < NV; ++q)
                if (q < nvalid * KT) {
                    if (a.goff) a.goff[e0 + q] = go[q];
                    if (a.gmask) a.gmask[e0 + q] = gm[q];
                }
        }
    }
    // weight gradient partials: wave sums, then LDS, then one atomic per tap
    if (a.gw) {
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            float v = wacc[k];
            for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
            if ((threadIdx.x & 63) == 0) atomicAdd(wred + k, v);
        }
    }
    __syncthreads();
    if (a.gw && threadIdx.x < KT) unsafeAtomicAdd(a.gw + (int64_t)c * KT + threadIdx.x, wred[threadIdx.x]);
    if (gxr) {
        for (int j = threadIdx.x; j < WIN; j += 256) {
            const int pos = lo + j;
            const float v = gacc[j];
            if (pos >= 0 && pos < L_in && v != 0.0f) unsafeAtomicAdd(gxr + pos, v);
        }
    }
}

// The same depthwise pass with grad_x gathered instead of scattered: LDS
// float atomics (two per sample) are the slow part of k_bwd_dw, so here each
// block OWNS a run of input positions -- tile t of a row owns
// [t*LT*s - p, (t+1)*LT*s - p), the first tile from 0, the last to L_in --
// and computes their gradient itself, with plain stores (deterministic):
//   phase 1: every sample that could land in the owned run (the tile's
//            outputs and a halo of outputs on both sides, for floor(offset)
//            within kDwgR) puts its left neighbour i0 and its two weighted
//            contributions dS*m*(1-f), dS*m*f into LDS ([tap][output]);
//            the tile's own samples also produce their offset / mask /
//            weight gradients as in k_bwd_dw;
//   phase 2: owned position i sums, per tap, the samples whose i0 is i or
//            i - 1 -- only outputs within R (the block's largest
//            |floor(offset)|) of the tap's grid position can be among them.
// Samples with |floor(offset)| > kDwgR are left to k_bwd_dwg_fix (global
// atomics after this kernel), which runs only if one was seen (*flag).
constexpr int kDwgT = 512;      // threads per block (one output each: twice the waves of k_bwd_dw per block)
constexpr int kDwgOpt = 1;      // outputs per thread
constexpr int kDwgLT = kDwgT * kDwgOpt;
constexpr int kDwgR = 16;       // largest |floor(offset)| gathered
constexpr int kDwgMargin = 24;  // x window margin (>= kDwgR + 2)
constexpr int kDwgWinU = 2;     // x window positions per thread loaded with the offsets
constexpr int kDwgTail = 2 * kDwgR + 6;  // sentinel entries after each tap's filled outputs (phase 2
                                         // reads up to (2 kDwgR + 3) + 3 candidates from the first one,
                                         // which may be the last filled output)
constexpr int kIrregular = INT_MIN / 2;

__device__ __forceinline__ int floor_div(int a, int b) {
    if (b == 1) return a;
    return a >= 0 ? a / b : -((-a + b - 1) / b);
}

struct DwgGeo {
    int l0, lh0, lh1, i_lo, i_hi;
};

__device__ __forceinline__ DwgGeo dwg_geo(const Params &p, int tile, int tiles_l, int LT = kDwgLT) {
    DwgGeo g;
    g.l0 = tile * LT;
    g.i_lo = tile == 0 ? 0 : max(0, g.l0 * p.stride - p.padding);
    g.i_hi = tile == tiles_l - 1 ? p.L_in : min(p.L_in, (g.l0 + LT) * p.stride - p.padding);
    // outputs whose taps can reach [i_lo - 1, i_hi) with |floor(offset)| <= kDwgR
    g.lh0 = max(0, -floor_div(-(g.i_lo - 1 + p.padding - (p.K - 1) * p.dilation - kDwgR), p.stride));
    g.lh1 = min(p.L_out, floor_div(g.i_hi - 1 + p.padding + kDwgR, p.stride) + 1);
    g.lh0 = min(g.lh0, g.l0);
    g.lh1 = max(g.lh1, min(g.l0 + LT, p.L_out));
    return g;
}

template <int KT>
__global__ void __launch_bounds__(kDwgT, 4) k_bwd_dwg(BwdParams a, int WIN, int NHP, int tiles_l, int *flag,
                                                      bool bias_here, float *__restrict__ wslots) {
    const Params &p = a.p;
    extern __shared__ float smem[];
    float *xs = smem;                          // [WIN]
    int *I0 = (int *)(smem + WIN);             // [KT][NHP]
    float *WL = smem + WIN + KT * NHP;         // [KT][NHP]
    float *WR = smem + WIN + 2 * KT * NHP;     // [KT][NHP]
    // each wave's weight-gradient sums (taps) and grad_bias sum, added in
    // wave order into the block's workspace slot
    __shared__ float wpart[kDwgT / 64][KT + 1];
    __shared__ int s_R, s_irr;
    const int L_in = p.L_in, L_out = p.L_out;
    const int tile = blockIdx.x % tiles_l;
    const int row = blockIdx.x / tiles_l;  // b * C_in + c
    const int c = row % p.C_in, b = row / p.C_in;
    const int g = c / p.cpo;
    const DwgGeo geo = dwg_geo(p, tile, tiles_l);
    const int l0 = geo.l0, lh0 = geo.lh0;
    const int lo = l0 * p.stride - p.padding - kDwgMargin;
    const float *__restrict__ xrow = (const float *)p.x + (int64_t)row * L_in;
    // the x window's first kDwgWinU * kDwgT positions: loaded here at
    // clamped addresses, written to LDS after the offset, mask and dout
    // loads below are issued, so all of them are in flight together
    float xw[kDwgWinU];
#pragma unroll
    for (int u = 0; u < kDwgWinU; ++u)
        xw[u] = xrow[min(max(lo + min((int)threadIdx.x + u * kDwgT, WIN - 1), 0), L_in - 1)];
    {  // entries past the filled outputs match no position
        const int nhl = geo.lh1 - lh0;
        for (int e = threadIdx.x; e < KT * NHP; e += kDwgT) {
            const int k = e / NHP, h = e - k * NHP;
            if (h >= nhl) I0[e] = kIrregular;
        }
    }
    if (threadIdx.x == 0) {
        s_R = 0;
        s_irr = 0;
    }
    const float *__restrict__ off = (const float *)p.off;
    const float *__restrict__ mask = (const float *)p.mask;
    const float *__restrict__ w = (const float *)p.w + (int64_t)c * KT;
    const float *__restrict__ dout = a.dout + (int64_t)row * L_out;
    const int64_t orow = ((int64_t)b * p.G + g) * L_out;  // offsets row of (b, g)
    const bool om_atomic = p.cpo > 1;
    float wk[KT], wacc[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        wk[k] = w[k];
        wacc[k] = 0.0f;
    }
    int rmax = 0;
    bool irregular = false;
    // ---- phase 1a: the tile's own samples (two outputs x KT taps per thread)
    constexpr int NV = kDwgOpt * KT;
    const int lt = l0 + kDwgOpt * threadIdx.x;
    const int nvalid = min(kDwgOpt, L_out - lt);
    const int64_t e0 = (orow + lt) * KT;
    const bool vec = NV % 2 == 0 && nvalid == kDwgOpt && ((((uintptr_t)(off + e0)) & 7) == 0) &&
                     (!mask || (((uintptr_t)(mask + e0)) & 7) == 0);
    float ov[NV], mv[NV], dv[kDwgOpt];
    if (nvalid > 0) {
        if (vec) {
#pragma unroll
            for (int q = 0; q < NV; q += 2) {
                const float2 t = *(const float2 *)(off + e0 + q);
                ov[q] = t.x;
                ov[q + 1] = t.y;
                if (mask) {
                    const float2 u = *(const float2 *)(mask + e0 + q);
                    mv[q] = u.x;
                    mv[q + 1] = u.y;
                } else {
                    mv[q] = mv[q + 1] = 1.0f;
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const bool ok = q < nvalid * KT;
                ov[q] = ok ? off[e0 + q] : 0.0f;
                mv[q] = (ok && mask) ? mask[e0 + q] : 1.0f;
            }
        }
#pragma unroll
        for (int o = 0; o < kDwgOpt; ++o) dv[o] = o < nvalid ? dout[lt + o] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kDwgWinU; ++u) {
        const int jj = threadIdx.x + u * kDwgT, pos = lo + jj;
        if (jj < WIN) xs[jj] = (pos >= 0 && pos < L_in) ? xw[u] : 0.0f;
    }
    for (int jj = threadIdx.x + kDwgWinU * kDwgT; jj < WIN; jj += kDwgT) {
        const int pos = lo + jj;
        xs[jj] = (pos >= 0 && pos < L_in) ? xrow[pos] : 0.0f;
    }
    __syncthreads();
    float go[NV], gm[NV];
#pragma unroll
    for (int o = 0; o < kDwgOpt; ++o) {
        const int l = lt + o;
        const int base0 = l * p.stride - p.padding;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int q = o * KT + k;
            go[q] = gm[q] = 0.0f;
            if (o >= nvalid) continue;
            int i0;
            float f;
            const TapRange r = tap_range(p, k);
            const int base = base0 + k * p.dilation;
            split_position(ov[q], base, r, i0, f);
            const float m = mv[q];
            const int j = i0 - lo;
            float x0, x1;
            if ((unsigned)j < (unsigned)(WIN - 1)) {
                x0 = xs[j];
                x1 = xs[j + 1];
            } else {
                x0 = (i0 >= 0 && i0 < L_in) ? xrow[i0] : 0.0f;
                x1 = (i0 + 1 >= 0 && i0 + 1 < L_in) ? xrow[i0 + 1] : 0.0f;
            }
            const float d = dv[o];
            const float ds = wk[k] * d;
            const float lerp = fmaf(f, x1 - x0, x0);
            wacc[k] = fmaf(d, lerp * m, wacc[k]);
            go[q] = tap_moves(p, ov[q], r) ? ds * m * (x1 - x0) : 0.0f;
            gm[q] = ds * lerp;
            const int fl = i0 - base;
            const bool reg = fl >= -kDwgR && fl <= kDwgR;
            irregular |= !reg;
            if (reg) rmax = max(rmax, abs(fl));
            const int h = l - lh0;
            const float dm = ds * m;
            I0[k * NHP + h] = reg ? i0 : kIrregular;
            WL[k * NHP + h] = dm * (1.0f - f);
            WR[k * NHP + h] = dm * f;
        }
    }
    // ---- phase 1b: halo samples (outputs outside the tile that can reach the owned run)
    {
        const int nleft = l0 - lh0, nright = geo.lh1 - min(l0 + kDwgLT, L_out);
        const int nh = (nleft + nright) * KT;
        for (int e = threadIdx.x; e < nh; e += kDwgT) {
            const int hk = e / KT, k = e - hk * KT;
            const int l = hk < nleft ? lh0 + hk : min(l0 + kDwgLT, L_out) + (hk - nleft);
            const int64_t oi = (orow + l) * KT + k;
            int i0;
            float f;
            const TapRange r = tap_range(p, k);
            const int base = l * p.stride - p.padding + k * p.dilation;
            split_position(off[oi], base, r, i0, f);
            const float dm = w[k] * dout[l] * (mask ? mask[oi] : 1.0f);
            const int fl = i0 - base;
            const bool reg = fl >= -kDwgR && fl <= kDwgR;
            if (reg) rmax = max(rmax, abs(fl));
            const int h = l - lh0;
            I0[k * NHP + h] = reg ? i0 : kIrregular;
            WL[k * NHP + h] = dm * (1.0f - f);
            WR[k * NHP + h] = dm * f;
        }
    }
    // offset and mask gradients of the tile's outputs (stored after the halo's
    // loads: waiting for a load also waits for the stores issued before it)
    if (nvalid > 0 && (a.goff || a.gmask)) {
        if (om_atomic) {
#pragma unroll
            for (int q = 0; q < NV; ++q)
                if (q < nvalid * KT) {
                    if (a.goff) unsafeAtomicAdd(a.goff + e0 + q, go[q]);
                    if (a.gmask) unsafeAtomicAdd(a.gmask + e0 + q, gm[q]);
                }
        } else if (vec) {
#pragma unroll
            for (int q = 0; q < NV; q += 2) {
                if (a.goff) *(float2 *)(a.goff + e0 + q) = float2{go[q], go[q + 1]};
                if (a.gmask) *(float2 *)(a.gmask + e0 + q) = float2{gm[q], gm[q + 1]};
            }
        } else {
#pragma unroll
            for (int q = 0; q < NV; ++q)
                if (q < nvalid * KT) {
                    if (a.goff) a.goff[e0 + q] = go[q];
                    if (a.gmask) a.gmask[e0 + q] = gm[q];
                }
        }
    }
    // weight gradient partials: wave sums (a fixed butterfly), then LDS
    if (a.gw) {
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            float v = wacc[k];
            for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
            if ((threadIdx.x & 63) == 0) wpart[threadIdx.x / 64][k] = v;
        }
    }
    if (bias_here) {  // grad_bias[c]: this block's outputs' dout, summed
        float v = 0.0f;
#pragma unroll
        for (int o = 0; o < kDwgOpt; ++o) v += (o < nvalid) ? dv[o] : 0.0f;
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        if ((threadIdx.x & 63) == 0) wpart[threadIdx.x / 64][KT] = v;
    }
    for (int o = 32; o > 0; o >>= 1) rmax = max(rmax, __shfl_xor(rmax, o));
    const bool irr_w = __any(irregular);
    if ((threadIdx.x & 63) == 0) {
        atomicMax(&s_R, rmax);
        if (irr_w) s_irr = 1;
    }
    __syncthreads();
    // the block's sums into its slot [c][b*tiles_l + tile][KT + 1], added
    // over the row's blocks in order by k_bwd_dw_wsum
    if ((threadIdx.x < KT && a.gw) || (threadIdx.x == KT && bias_here)) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kDwgT / 64; ++w) sum += wpart[w][threadIdx.x];
        wslots[((int64_t)c * p.B * tiles_l + (int64_t)b * tiles_l + tile) * (KT + 1) + threadIdx.x] = sum;
    }
    if (threadIdx.x == 0 && s_irr) atomicOr(flag, 1);
    if (!a.gx) return;
    // ---- phase 2: the owned positions, gathered
    const int R = s_R;
    const int nhl = geo.lh1 - lh0;
    float *__restrict__ gxr = a.gx + (int64_t)row * L_in;
    // A thread owns two consecutive positions i, i+1.  Candidates per tap:
    // outputs l with l*s in [t - 1 - R, t + 1 + R] (a sample whose left
    // neighbour is i - 1, i or i + 1 with |floor(offset)| <= R has its grid
    // position in that range), at most (2R + 2)/s + 1 of them; a uniform
    // trip count (the largest any lane has) in pairs, so that the LDS reads
    // of a pair are in flight together.  The run read starts at the range's
    // first output clamped to [0, filled outputs]: outputs outside the range
    // cannot match, and past the filled ones sit sentinels (kDwgTail of
    // them), so no read needs a bounds test.  Each position's terms are
    // added in the same order as one position per thread would (taps, then
    // outputs).
    const int ncand = (2 * R + 2) / p.stride + 1;
    for (int i = geo.i_lo + 2 * threadIdx.x; i < geo.i_hi; i += 2 * kDwgT) {
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll 1
        for (int k = 0; k < KT; ++k) {
            const int t = i + p.padding - k * p.dilation;  // l*s for i0 == i with floor(offset) 0
            const int h0 = min(max(-floor_div(-(t - 1 - R), p.stride) - lh0, 0), nhl);
            const int *__restrict__ i0k = I0 + k * NHP + h0;
            const float *__restrict__ wlk = WL + k * NHP + h0, *__restrict__ wrk = WR + k * NHP + h0;
            for (int m0 = 0; m0 < ncand; m0 += 2) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int v = i0k[m0 + u];
                    const float wl = wlk[m0 + u], wr = wrk[m0 + u];
                    // at most one of a position's two terms is nonzero
                    const bool e0 = v == i;
                    acc0 += e0 ? wl : (v == i - 1 ? wr : 0.0f);
                    acc1 += e0 ? wr : (v == i + 1 ? wl : 0.0f);
                }
            }
        }
        gxr[i] = acc0;
        if (i + 1 < geo.i_hi) gxr[i + 1] = acc1;
    }
}

// grad_x gathered from a materialised dS ([B][C_in][K][L_out]: dense and
// grouped shapes) -- the same ownership as k_bwd_dwg, without LDS atomics:
// a block takes one batch, a block of cbx channels of one offset group and
// the input positions owned by a tile of lt outputs.  Phase 1 stores, per
// (tap, output) of the tile and its halo, the left neighbour and the two
// interpolation weights times the mask (shared by the block's channels).
// Phase 2: a thread owns two consecutive positions of CPT channels and
// sums, per tap, over the candidate outputs (as in k_bwd_dwg) the products
// dS * weight, reading dS from global memory (the CPT channels' values of
// one candidate are one load each, their weights computed once).  Samples
// moved further than kDwgR are added afterwards by k_bwd_dxg_fix.
struct DxgPlan {
    int lt, nhp, tiles_l, cbx, cblocks, cpt;
    size_t lds;  // 0: not served (the scattering k_bwd_dx computes grad_x)
};

template <int CPT>
__global__ void __launch_bounds__(256) k_bwd_dxg(BwdParams a, DxgPlan pl, int *flag) {
    const Params &p = a.p;
    extern __shared__ float smem[];
    const int K = p.K, NHP = pl.nhp, L_in = p.L_in, L_out = p.L_out;
    int *I0 = (int *)smem;       // [K][NHP]
    float *ML = smem + K * NHP;  // [K][NHP]: m * (1 - f)
    float *MR = smem + 2 * K * NHP;  // [K][NHP]: m * f
    __shared__ int s_R, s_irr;
    int blk = blockIdx.x;
    const int tile = blk % pl.tiles_l;
    blk /= pl.tiles_l;
    const int cblk = blk % pl.cblocks;
    const int b = blk / pl.cblocks;
    const int ci0 = cblk * pl.cbx, g = ci0 / p.cpo;
    const DwgGeo geo = dwg_geo(p, tile, pl.tiles_l, pl.lt);
    const int lh0 = geo.lh0, nhl = geo.lh1 - lh0;
    if (threadIdx.x == 0) {
        s_R = 0;
        s_irr = 0;
    }
    __syncthreads();
    // ---- phase 1: positions of the tile's and the halo's samples (sentinels past them)
    const float *__restrict__ off = (const float *)p.off;
    const float *__restrict__ mask = (const float *)p.mask;
    const int64_t orow = ((int64_t)b * p.G + g) * L_out;
    int rmax = 0;
    bool irregular = false;
    for (int e = threadIdx.x; e < K * NHP; e += 256) {
        const int k = e / NHP, h = e - k * NHP;
        int v = kIrregular;
        float ml = 0.0f, mr = 0.0f;
        if (h < nhl) {
            const int l = lh0 + h;
            const int64_t oi = (orow + l) * K + k;
            const int base = l * p.stride - p.padding + k * p.dilation;
            int i0;
            float f;
            split_position(off[oi], base, tap_range(p, k), i0, f);
            const float m = mask ? mask[oi] : 1.0f;
            const int fl = i0 - base;
            if (fl >= -kDwgR && fl <= kDwgR) {
                v = i0;
                rmax = max(rmax, abs(fl));
            } else {
                irregular = true;
            }
            ml = m * (1.0f - f);
            mr = m * f;
        }
        I0[e] = v;
        ML[e] = ml;
        MR[e] = mr;
    }
    for (int o = 32; o > 0; o >>= 1) rmax = max(rmax, __shfl_xor(rmax, o));
    const bool irr_w = __any(irregular);
    if ((threadIdx.x & 63) == 0) {
        atomicMax(&s_R, rmax);
        if (irr_w) s_irr = 1;
    }
    __syncthreads();
    if (threadIdx.x == 0 && s_irr) atomicOr(flag, 1);
    // ---- phase 2: (position pair, channel group) tasks, consecutive threads on consecutive pairs
    const int R = s_R;
    const int ncand = (2 * R + 2) / p.stride + 1;
    const int npairs = (geo.i_hi - geo.i_lo + 1) / 2;
    const int ntask = npairs * (pl.cbx / CPT);
    const int64_t cs = (int64_t)K * L_out;  // dS channel stride
    const float *__restrict__ dsb = a.dS + ((int64_t)b * p.C_in + ci0) * cs;
    float *__restrict__ gxb = a.gx + ((int64_t)b * p.C_in + ci0) * L_in;
    for (int task = threadIdx.x; task < ntask; task += 256) {
        const int q = task % npairs, cq = task / npairs;
        const int i = geo.i_lo + 2 * q;
        float acc0[CPT], acc1[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc0[c] = acc1[c] = 0.0f;
        const float *__restrict__ dsc = dsb + (int64_t)cq * CPT * cs;
#pragma unroll 1
        for (int k = 0; k < K; ++k) {
            const int t = i + p.padding - k * p.dilation;  // l*s for i0 == i with floor(offset) 0
            const int h0 = min(max(-floor_div(-(t - 1 - R), p.stride) - lh0, 0), nhl);
            const int *__restrict__ i0k = I0 + k * NHP + h0;
            const float *__restrict__ mlk = ML + k * NHP + h0, *__restrict__ mrk = MR + k * NHP + h0;
            const float *__restrict__ dsk = dsc + (int64_t)k * L_out + lh0 + h0;
            const int last = nhl - 1 - h0;  // candidates past the filled outputs read the last one's dS
            // four candidates at a time (their 4 * CPT dS loads in flight
            // together); the up to three past ncand are sentinels or outputs
            // that cannot reach i or i + 1, so they add exact zeros
            for (int m0 = 0; m0 < ncand; m0 += 4) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int v = i0k[m0 + u];
                    const float ml = mlk[m0 + u], mr = mrk[m0 + u];
                    // at most one of a position's two terms is nonzero
                    const bool e0 = v == i;
                    const float w0 = e0 ? ml : (v == i - 1 ? mr : 0.0f);
                    const float w1 = e0 ? mr : (v == i + 1 ? ml : 0.0f);
                    const int hd = min(m0 + u, last);
#pragma unroll
                    for (int c = 0; c < CPT; ++c) {
                        const float ds = dsk[c * cs + hd];
                        acc0[c] = fmaf(ds, w0, acc0[c]);
                        acc1[c] = fmaf(ds, w1, acc1[c]);
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            float *gr = gxb + (int64_t)(cq * CPT + c) * L_in;
            gr[i] = acc0[c];
            if (i + 1 < geo.i_hi) gr[i + 1] = acc1[c];
        }
    }
}

// The samples k_bwd_dxg left out (|floor(offset)| > kDwgR), added to grad_x
// for every channel of their offset group with global atomics once every
// owned run is stored.  Runs only if one was seen.
__global__ void __launch_bounds__(256) k_bwd_dxg_fix(BwdParams a, const int *flag) {
    if (*flag == 0) return;
    const Params &p = a.p;
    const float *__restrict__ off = (const float *)p.off;
    const float *__restrict__ mask = (const float *)p.mask;
    const int K = p.K, L_out = p.L_out, L_in = p.L_in;
    const int64_t n = (int64_t)p.B * p.G * L_out * K;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        const int k = (int)(e % K);
        const int64_t r = e / K;
        const int l = (int)(r % L_out);
        const int64_t bg = r / L_out;
        const int g = (int)(bg % p.G), b = (int)(bg / p.G);
        const int base = l * p.stride - p.padding + k * p.dilation;
        int i0;
        float f;
        split_position(off[e], base, tap_range(p, k), i0, f);
        const int fl = i0 - base;
        if (fl >= -kDwgR && fl <= kDwgR) continue;
        const float m = mask ? mask[e] : 1.0f;
        const bool v0 = i0 >= 0 && i0 < L_in, v1 = i0 + 1 >= 0 && i0 + 1 < L_in;
        if (!v0 && !v1) continue;
        for (int ci = g * p.cpo; ci < (g + 1) * p.cpo; ++ci) {
            const float dm = a.dS[(((int64_t)b * p.C_in + ci) * K + k) * L_out + l] * m;
            float *gr = a.gx + ((int64_t)b * p.C_in + ci) * L_in;
            if (v0) unsafeAtomicAdd(gr + i0, dm * (1.0f - f));
            if (v1) unsafeAtomicAdd(gr + i0 + 1, dm * f);
        }
    }
}

DxgPlan plan_dxg(const Params &p) {
    DxgPlan pl = {};
    const int64_t s = p.stride, span = (int64_t)(p.K - 1) * p.dilation;
    const int64_t halo = (span + kDwgR + 1 + s - 1) / s + kDwgR / s + 2;
    // the largest tile (a multiple of 32 outputs, at most 512) whose arrays fit in 64 KB
    for (int64_t lt = std::min<int64_t>(512, ((int64_t)p.L_out + 31) / 32 * 32); lt >= 32; lt /= 2) {
        const int64_t nh = std::min<int64_t>(lt, p.L_out) + halo;
        const int64_t nhp = (nh + kDwgTail + 31) / 32 * 32 + 1;
        const size_t lds = 3 * (size_t)p.K * (size_t)nhp * 4;
        if (lds <= 64 * 1024) {
            pl.lt = (int)lt;
            pl.nhp = (int)nhp;
            pl.lds = lds;
            break;
        }
    }
    if (pl.lds == 0) return pl;
    pl.tiles_l = (p.L_out + pl.lt - 1) / pl.lt;
    pl.cbx = 1;  // the largest divisor of the offset group's channel count up to 32
    for (int c = 32; c >= 1; --c)
        if (p.cpo % c == 0) {
            pl.cbx = c;
            break;
        }
    pl.cpt = pl.cbx % 4 == 0 ? 4 : 1;
    pl.cblocks = p.C_in / pl.cbx;
    if ((int64_t)p.B * pl.cblocks * pl.tiles_l >= ((int64_t)1 << 31)) pl.lds = 0;
    return pl;
}

// The samples k_bwd_dwg left out (|floor(offset)| > kDwgR), added to grad_x
// with global atomics once every owned run is stored.  Runs only if one was
// seen.
template <int KT>
// A small grid strides over the (row, tile) units: when no sample moved that
// far (the usual case) the pass costs one flag read per block.
__global__ void __launch_bounds__(256) k_bwd_dwg_fix(BwdParams a, int tiles_l, const int *flag) {
    if (*flag == 0) return;
    const Params &p = a.p;
    const int64_t units = (int64_t)p.B * p.C_in * tiles_l;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int tile = (int)(u % tiles_l);
        const int64_t row = u / tiles_l;
        const int c = (int)(row % p.C_in);
        const int64_t b = row / p.C_in;
        const int g = c / p.cpo;
        const int64_t orow = (b * p.G + g) * p.L_out;
        const float *__restrict__ w = (const float *)p.w + (int64_t)c * KT;
        float *__restrict__ gxr = a.gx + row * p.L_in;
        const int l1 = min((tile + 1) * kDwgLT, p.L_out);
        for (int l = tile * kDwgLT + threadIdx.x; l < l1; l += 256) {
            const float d = a.dout[row * p.L_out + l];
            for (int k = 0; k < KT; ++k) {
                const int64_t oi = (orow + l) * KT + k;
                int i0;
                float f;
                const int base = l * p.stride - p.padding + k * p.dilation;
                split_position(((const float *)p.off)[oi], base, tap_range(p, k), i0, f);
                const int fl = i0 - base;
                if (fl >= -kDwgR && fl <= kDwgR) continue;
                const float dm = w[k] * d * (p.mask ? ((const float *)p.mask)[oi] : 1.0f);
                if (i0 >= 0 && i0 < p.L_in) unsafeAtomicAdd(gxr + i0, dm * (1.0f - f));
                if (i0 + 1 >= 0 && i0 + 1 < p.L_in) unsafeAtomicAdd(gxr + i0 + 1, dm * f);
            }
        }
    }
}

// out[c][r] = in[r][c] for a rows x cols matrix (32 x 32 tiles through LDS);
// also clears *clear (a flag of a later pass) when given.
__global__ void __launch_bounds__(256) k_transpose(const float *__restrict__ in, float *__restrict__ out, int rows,
                                                   int cols, int *clear) {
    __shared__ float tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    if (clear && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *clear = 0;
    const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 32 x 8
    for (int j = ty; j < 32; j += 8)
        if (r0 + j < rows && c0 + tx < cols) tile[j][tx] = in[(int64_t)(r0 + j) * cols + c0 + tx];
    __syncthreads();
    for (int j = ty; j < 32; j += 8)
        if (c0 + j < cols && r0 + tx < rows) out[(int64_t)(c0 + j) * rows + r0 + tx] = tile[tx][j];
}

// A[co][b*L_out + l] = dout[b][co][l], one workgroup per output channel
// (its B * L_out values in k_bwd_bias's order), and with a bias gradient
// wanted grad_bias[co] summed as k_bwd_bias sums it, in the same order.
__global__ void __launch_bounds__(256) k_restride_bias(BwdParams a, float *__restrict__ A) {
    const Params &p = a.p;
    __shared__ float s_red[256];
    const int co = blockIdx.x;
    const int64_t n = (int64_t)p.B * p.L_out;
    const float *d = a.dout + (int64_t)co * p.L_out;
    float *arow = A + (int64_t)co * n;
    float acc = 0.0f;
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < n; i += 256) {
        const int64_t b = i / p.L_out, l = i - b * p.L_out;
        const float v = d[b * p.C_out * p.L_out + l];
        arow[i] = v;
        acc += v;
    }
    if (!a.gb) return;
    s_red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) s_red[threadIdx.x] += s_red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.gb[co] = s_red[0];
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

// Grid of the flagged fix passes (grid-stride kernels that usually return at
// once): small, so that the no-op case costs a few microseconds.
constexpr int64_t kFixBlocks = 512;
unsigned fix_grid(int64_t units) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>(units, kFixBlocks)); }

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
    size_t dS, wt, S, A, part, om, flag, total;
};

hipError_t launch_bias(const BwdParams &a, hipStream_t stream) {
    const Params &p = a.p;
    if (a.gb && p.C_out > 0)  // (C_out < 2^31 by validation; an empty batch gives zeros)
        hipLaunchKernelGGL(k_bwd_bias, dim3((unsigned)p.C_out), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// The fused depthwise pass serves C_in == C_out == groups with K in 1..9.
bool depthwise_path(const Params &p) {
    return p.cpg == 1 && p.opg == 1 && p.K >= 1 && p.K <= 9 && p.K != 6 && p.K != 8 &&
           (int64_t)p.B * p.C_in * ((p.L_out + 256 * kDwbOpt - 1) / (256 * kDwbOpt)) < ((int64_t)1 << 31);
}

// LDS of the gather pass (k_bwd_dwg) for this shape: the x window and the
// [K][NHP] sample arrays, or 0 when they exceed kDwgLds (then the
// scattering k_bwd_dw runs).
constexpr size_t kDwgLds = 64 * 1024;
struct DwgPlan {
    int win, nhp;
    size_t lds;
};
DwgPlan plan_dwg(const Params &p) {
    const int64_t LT = kDwgLT, s = p.stride;
    const int64_t span = (int64_t)(p.K - 1) * p.dilation;
    int64_t win = (LT - 1) * s + span + kDwgR + kDwgMargin + 4;
    win = (win + 63) / 64 * 64;
    const int64_t nh = LT + (span + kDwgR + 1 + s - 1) / s + kDwgR / s + 2;
    // pitch = 1 (mod 32): taps on distinct banks; room for the sentinels
    const int64_t nhp = (nh + kDwgTail + 31) / 32 * 32 + 1;
    DwgPlan pl = {0, 0, 0};
    const size_t lds = ((size_t)win + 3 * (size_t)p.K * nhp) * 4;
    if (lds <= kDwgLds && win >= 2) pl = {(int)win, (int)nhp, lds};
    return pl;
}

// The depthwise gather pass's per-block grad_weight / grad_bias slots
// ([C_in][B * tiles][K + 1] floats), 256 bytes past its flag.
size_t dwg_slot_bytes(const Params &p) {
    const int64_t tiles_g = (p.L_out + kDwgLT - 1) / kDwgLT;
    return align256((size_t)p.C_in * p.B * tiles_g * (p.K + 1) * 4);
}

BwdLayout layout(const Params &p, bool want_weight, int num_cus) {
    BwdLayout L = {};
    if (depthwise_path(p)) {  // the gather pass's flag and slots
        L.total = plan_dwg(p).lds > 0 ? 256 + dwg_slot_bytes(p) : 0;
        return L;
    }
    const size_t nds = (size_t)p.B * p.C_in * p.K * p.L_out * 4;
    size_t o = 0;
    L.dS = o;
    o += align256(nds);
    if (dense_path(p)) {
        L.wt = o;
        o += align256((size_t)p.C_out * p.C_in * p.K * 4);
        size_t part = gemm_workspace_bytes(gemm_ds(p, nullptr, nullptr, nullptr, nullptr), 0, num_cus);
        if (want_weight) {
            L.S = o;
            o += align256(nds);
            L.A = o;
            o += align256((size_t)p.B * p.C_out * p.L_out * 4);
            part = std::max(part, gemm_workspace_bytes(gemm_dw(p, nullptr, nullptr, nullptr, nullptr), 0, num_cus));
        }
        L.part = o;
        o += align256(part);
    } else if (want_weight) {
        L.S = o;
        o += align256(nds);
    }
    const DxPlan dx = plan_dx(p);
    if (dx.atomic_om) {  // k_bwd_dx's slots for the offset and mask gradients
        L.om = o;
        o += align256((size_t)dx.nsub * 2 * p.B * p.G * p.L_out * p.K * 4);
    }
    L.flag = o;  // the grad_x gather's flag
    o += 256;
    L.total = o;
    return L;
}

}  // namespace

size_t backward_workspace_bytes(const Params &p, bool want_weight, int num_cus) {
    return layout(p, want_weight, num_cus).total;
}

// grad_weight (and grad_bias) of the depthwise gather pass: one wave per
// channel adds that channel's per-block slot sums, lane j taking blocks j,
// j + 64, ... in order and a fixed butterfly combining the lanes, so every
// call sums in the same order.
__global__ void __launch_bounds__(256) k_bwd_dw_wsum(BwdParams a, const float *__restrict__ wslots, int nblk,
                                                     bool bias_here) {
    const Params &p = a.p;
    const int c = blockIdx.x * 4 + (int)(threadIdx.x / 64), lane = threadIdx.x & 63;
    if (c >= p.C_in) return;
    const int K1 = p.K + 1;
    const float *sl = wslots + (int64_t)c * nblk * K1;
    float acc[10];
#pragma unroll
    for (int k = 0; k < 10; ++k) acc[k] = 0.0f;
    for (int j = lane; j < nblk; j += 64) {
#pragma unroll
        for (int k = 0; k < 10; ++k)
            if (k < K1) acc[k] += sl[(int64_t)j * K1 + k];
    }
#pragma unroll
    for (int k = 0; k < 10; ++k) {
        if (k < K1) {  // uniform over the wave
            float v = acc[k];
            for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
            if (lane == 0) {
                if (k < p.K) {
                    if (a.gw) a.gw[(int64_t)c * p.K + k] = v;
                } else if (bias_here) {
                    a.gb[c] = v;
                }
            }
        }
    }
}

hipError_t launch_backward_dw(BwdParams a, int *flag, hipStream_t stream, bool *bias_done) {
    if (bias_done) *bias_done = false;
    const Params &p = a.p;
    const int LT = 256 * kDwbOpt;
    const int tiles_l = (p.L_out + LT - 1) / LT;
    const DwgPlan g = plan_dwg(p);
    const bool gather = g.lds > 0 && flag != nullptr;
    // grad_bias from the dout the gather pass reads anyway (C_out == C_in here)
    const bool bias_here = gather && a.gb != nullptr;
    ZeroSet z = {};
    if (!gather) z.add(a.gx, (int64_t)p.B * p.C_in * p.L_in);  // the scattering pass accumulates into grad_x
    int64_t win = (int64_t)(LT - 1) * p.stride + (int64_t)(p.K - 1) * p.dilation + 2 + 2 * kDwbMargin;
    win = (win + 63) / 64 * 64;
    if (win > 6144) win = 0;  // wider spans: global memory only
    const size_t lds = 2 * (size_t)win * 4;
    const int64_t no = (int64_t)p.B * p.G * p.L_out * p.K;
    if (p.cpo > 1) {
        z.add(a.goff, no);
        z.add(a.gmask, no);
    }
    if (!gather) z.add(a.gw, (int64_t)p.C_out * p.K);  // the scattering pass accumulates grad_weight
    if (gather) z.add((float *)flag, 1);
    if (z.count > 0) hipLaunchKernelGGL(k_bwd_zero_set, dim3(grid_for(z.most)), dim3(256), 0, stream, z);
    const dim3 grid((unsigned)((int64_t)p.B * p.C_in * tiles_l));
    if (gather) {
        const int tiles_g = (p.L_out + kDwgLT - 1) / kDwgLT;
        const dim3 grid((unsigned)((int64_t)p.B * p.C_in * tiles_g));
        float *wslots = (float *)((char *)flag + 256);
        if (bias_done) *bias_done = bias_here;
        switch (p.K) {
#define DC1D_BDWG(KK)                                                                                              \
    case KK:                                                                                                       \
        hipLaunchKernelGGL((k_bwd_dwg<KK>), grid, dim3(kDwgT), g.lds, stream, a, g.win, g.nhp, tiles_g, flag,     \
                           bias_here, wslots);                                                                     \
        if (a.gx)                                                                                                  \
            hipLaunchKernelGGL((k_bwd_dwg_fix<KK>), dim3(fix_grid((int64_t)p.B * p.C_in * tiles_g)), dim3(256), 0,  \
                               stream, a, tiles_g, (const int *)flag);                                             \
        break;
            DC1D_BDWG(1)
            DC1D_BDWG(2)
            DC1D_BDWG(3)
            DC1D_BDWG(4)
            DC1D_BDWG(5)
            DC1D_BDWG(7)
            DC1D_BDWG(9)
#undef DC1D_BDWG
            default: return hipErrorInvalidValue;
        }
        if (a.gw || bias_here)
            hipLaunchKernelGGL(k_bwd_dw_wsum, dim3((unsigned)((p.C_in + 3) / 4)), dim3(256), 0, stream, a,
                               (const float *)wslots, p.B * tiles_g, bias_here);
        return hipGetLastError();
    }
    switch (p.K) {
#define DC1D_BDW(KK) \
    case KK: hipLaunchKernelGGL((k_bwd_dw<KK>), grid, dim3(256), lds, stream, a, (int)win, tiles_l); break;
        DC1D_BDW(1)
        DC1D_BDW(2)
        DC1D_BDW(3)
        DC1D_BDW(4)
        DC1D_BDW(5)
        DC1D_BDW(7)
        DC1D_BDW(9)
#undef DC1D_BDW
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_backward(BwdParams a, int num_cus, hipStream_t stream) {
    const Params &p = a.p;
    const int64_t n = (int64_t)p.B * p.C_in * p.K * p.L_out;
    char *ws = (char *)a.dS;  // the workspace base
    const BwdLayout L = layout(p, a.gw != nullptr, num_cus);
    const DxPlan dx = plan_dx(p);
    const bool want_dx = a.gx || a.goff || a.gmask;
    if (n > 0 && (want_dx || a.gw) && depthwise_path(p)) {
        bool bias_done = false;
        const hipError_t e = launch_backward_dw(a, L.total > 0 ? (int *)ws : nullptr, stream, &bias_done);
        if (e != hipSuccess) return e;
        return bias_done ? hipGetLastError() : launch_bias(a, stream);
    }
    const DxgPlan xg = plan_dxg(p);
    const bool gather_x = a.gx && xg.lds > 0;  // grad_x gathered (no clear, no atomics) or scattered
    bool bias_done = false;
    ZeroSet z = {};
    if (!gather_x) z.add(a.gx, (int64_t)p.B * p.C_in * p.L_in);
    const int64_t no = (int64_t)p.B * p.G * p.L_out * p.K;
    float *om_slots = dx.atomic_om ? (float *)(ws + L.om) : nullptr;
    int *flag = (int *)(ws + L.flag);
    // the dense path's k_transpose clears the flag; the others clear it here
    const bool dense_run = n > 0 && (want_dx || a.gw) && dense_path(p);
    if (gather_x && n > 0 && !dense_run) z.add((float *)flag, 1);
    if (z.count > 0) hipLaunchKernelGGL(k_bwd_zero_set, dim3(grid_for(z.most)), dim3(256), 0, stream, z);
    const int64_t dx_blocks = (int64_t)p.B * dx.ngrp_blocks * dx.tiles_l;
    if (dx_blocks >= ((int64_t)1 << 31) || (int64_t)p.C_out * p.cpg * p.K >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;  // grids beyond the launch limits
    if (n > 0 && (want_dx || a.gw)) {
        const bool dense = dense_path(p);
        BwdParams s = a;  // the samples pass: no grad_x scatter here
        s.gx = nullptr;
        s.S = a.gw ? (float *)(ws + L.S) : nullptr;
        if (dense) {
            float *wt = (float *)(ws + L.wt);
            const int CK = p.C_in * p.K;
            hipLaunchKernelGGL(k_transpose, dim3((unsigned)((CK + 31) / 32), (unsigned)((p.C_out + 31) / 32)),
                               dim3(256), 0, stream, (const float *)p.w, wt, p.C_out, CK, gather_x ? flag : nullptr);
            const hipError_t e = launch_gemm_f32(gemm_ds(p, wt, a.dout, a.dS, ws + L.part), p.L_out,
                                                 (int64_t)p.C_out * p.L_out, 0, num_cus, stream);
            if (e != hipSuccess) return e;
            if (s.S && (int64_t)p.B * p.L_out > 0)
                hipLaunchKernelGGL(k_bwd_samples_t, dim3((unsigned)std::min<int64_t>((int64_t)p.B * p.L_out, 1 << 20)),
                                   dim3(256), 0, stream, s, make_fastdiv((uint32_t)p.K), make_fastdiv((uint32_t)p.cpo));
        } else {
            hipLaunchKernelGGL(k_bwd_samples, dim3(grid_for(n)), dim3(256), 0, stream, s);
        }
        BwdParams ad = a;  // the offset and mask gradients (and grad_x when not gathered)
        if (gather_x) ad.gx = nullptr;
        if ((ad.gx || ad.goff || ad.gmask) && dx_blocks > 0)
            hipLaunchKernelGGL(k_bwd_dx, dim3((unsigned)dx_blocks), dim3(256), dx.lds, stream, ad, dx, om_slots);
        if (dx.atomic_om && (ad.goff || ad.gmask) && dx_blocks > 0)
            hipLaunchKernelGGL(k_bwd_om_sum, dim3(grid_for(no)), dim3(256), 0, stream, ad, (const float *)om_slots,
                               dx.nsub);
        if (gather_x) {
            const dim3 grid((unsigned)((int64_t)p.B * xg.cblocks * xg.tiles_l));
            if (xg.cpt == 4)
                hipLaunchKernelGGL((k_bwd_dxg<4>), grid, dim3(256), xg.lds, stream, a, xg, flag);
            else
                hipLaunchKernelGGL((k_bwd_dxg<1>), grid, dim3(256), xg.lds, stream, a, xg, flag);
            hipLaunchKernelGGL(k_bwd_dxg_fix, dim3(fix_grid((no + 255) / 256)), dim3(256), 0, stream, a,
                               (const int *)flag);
        }
        if (a.gw) {
            if (dense) {
                float *A = (float *)(ws + L.A);
                const int64_t nd = (int64_t)p.B * p.C_out * p.L_out;
                if (a.gb && p.C_out < (1 << 20)) {  // grad_bias from the same reads
                    hipLaunchKernelGGL(k_restride_bias, dim3((unsigned)p.C_out), dim3(256), 0, stream, a, A);
                    bias_done = true;
                } else {
                    hipLaunchKernelGGL(k_restride_dout, dim3(grid_for(nd)), dim3(256), 0, stream, a, A);
                }
                const hipError_t e = launch_gemm_f32(gemm_dw(p, A, s.S, a.gw, ws + L.part), p.C_in * p.K, 0,
                                                     0, num_cus, stream);
                if (e != hipSuccess) return e;
            } else {
                hipLaunchKernelGGL(k_bwd_weight, dim3((unsigned)(p.C_out * p.cpg * p.K)), dim3(256), 0, stream, s);
            }
        }
    }
    if (a.gw && n == 0) {
        const int64_t nw = (int64_t)p.C_out * p.cpg * p.K;
        hipLaunchKernelGGL(k_bwd_zero, dim3(grid_for(nw)), dim3(256), 0, stream, a.gw, nw);
    }
    return bias_done ? hipGetLastError() : launch_bias(a, stream);
}

}  // namespace dc1d
