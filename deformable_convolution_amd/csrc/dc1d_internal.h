// dc1d_internal.h -- private declarations shared by the libdc1d sources:
// the launch parameter block, device helpers (dtype access, position split),
// and the kernel launchers each translation unit provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace dc1d {

// Offsets are clamped to +-2^29 before they are floored.  Under the size
// limits the library enforces (L_in + padding <= 2^29) every position whose
// offset reaches the clamp already reads zero, and the integer arithmetic
// on positions stays far inside int32.
constexpr float kOffsetClamp = 536870912.0f;  // 2^29

enum Dtype : int { kF32 = 0, kBF16 = 1 };

// Everything a launcher needs; filled and validated by the C ABI layer.
struct Params {
    const void *x, *off, *mask, *w, *bias;
    void *out;
    int dtype;
    int B, C_in, C_out, L_in, L_out, K, stride, padding, dilation, groups, G;
    int cpg;   // input channels per conv group  (C_in / groups)
    int opg;   // output channels per conv group (C_out / groups)
    int cpo;   // input channels per offset group (C_in / G)
    int Kred;  // reduction length of one output: cpg * K
    int constrained;  // taps kept inside the undeformed kernel window (tap_range)
    void *ws;
    size_t ws_bytes;
    // profiling: HIP events recorded on the launch stream right before and
    // right after the call's dominant kernel (null: none)
    void *ev_start, *ev_stop;
};

// Records a profiling event (see Params::ev_start) when one is set.
inline void mark_event(void *ev, hipStream_t stream) {
    if (ev) (void)hipEventRecord((hipEvent_t)ev, stream);
}

// Division by a run-time invariant d >= 1 for numerators n < 2^31:
// q = (umulhi(n, mul) + n) >> shift, with 2^shift >= d and
// mul = floor(2^32 (2^shift - d) / d) + 1.
struct FastDiv {
    uint32_t d, mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.shift = s;
    f.mul = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
    return (__umulhi(n, f.mul) + n) >> f.shift;
}

// ---- storage dtypes ------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bfloat16, round to nearest even (NaN stays a quiet NaN): the
// conversion instruction, on a pair whose second half is dropped.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
    const bf2_t r = __builtin_convertvector(f2_t{f, 0.0f}, bf2_t);
    return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xffffu);
}

struct F32 {
    using T = float;
    static __device__ __forceinline__ float ld(const T *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void st(T *p, int64_t i, float v) { p[i] = v; }
};

struct BF16 {
    using T = uint16_t;
    static __device__ __forceinline__ float ld(const T *p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void st(T *p, int64_t i, float v) { p[i] = f32_to_bf16_rne(v); }
};

// ---- the sampling position ------------------------------------------------
//
// A tap at grid position base = l*stride - padding + k*dilation moved by the
// offset o samples between the integer neighbours i0 = base + floor(o) and
// i0 + 1 with weights 1 - f and f, f = o - floor(o).  Only the offset is
// floored; the grid term is an exact integer, so i0 is exact for any
// sequence length (no rounding of base + o in floating point).
__device__ __forceinline__ void split_position(float o, int base, int &i0, float &f) {
    o = fminf(fmaxf(o, -kOffsetClamp), kOffsetClamp);  // a NaN becomes -2^29
    const float fl = floorf(o);
    i0 = base + (int)fl;
    f = o - fl;
}

// The offsets tap k may use.  Constrained mode (the dc1d page's default,
// section Usage / DeformConv1d: each tap stays inside its receptive field;
// read as the undeformed kernel's window [l*s - p, l*s - p + (K-1)*d] of its
// output) clamps the offset to [-k*d, (K-1-k)*d]; otherwise only the global
// clamp applies.  The bounds are exact floats ((K-1)*d < 2^24 is checked).
struct TapRange {
    float lo, hi;
};
__device__ __forceinline__ TapRange tap_range(const Params &p, int k) {
    if (p.constrained) return {-(float)(k * p.dilation), (float)((p.K - 1 - k) * p.dilation)};
    return {-kOffsetClamp, kOffsetClamp};
}
__device__ __forceinline__ void split_position(float o, int base, TapRange r, int &i0, float &f) {
    o = fminf(fmaxf(o, r.lo), r.hi);  // a NaN becomes r.lo
    const float fl = floorf(o);
    i0 = base + (int)fl;
    f = o - fl;
}
// Whether moving the offset up moves the sample (the right derivative of the
// clamp: 1 on [lo, hi), 0 at and beyond hi and below lo); always in
// unconstrained mode.
__device__ __forceinline__ bool tap_moves(const Params &p, float o, TapRange r) {
    return !p.constrained || (o >= r.lo && o < r.hi);
}

// ---- launchers ------------------------------------------------------------

hipError_t launch_positions(const void *off, int dtype, int64_t n, int L_out, int K, int stride,
                            int padding, int dilation, int L_in, int32_t *i0, float *frac,
                            uint8_t *valid, hipStream_t stream);

// dst[i] = src[i] converted between storage dtypes (kBF16 -> kF32 exactly,
// kF32 -> kBF16 rounded to nearest even), i < n.
hipError_t launch_convert(const void *src, int src_dtype, void *dst, int dst_dtype, int64_t n, hipStream_t stream);

// Generic one-thread-per-output kernel: any groups / offset groups / mask.
hipError_t launch_direct(const Params &p, hipStream_t stream);

// One input channel per output (C_in / groups == 1): depthwise and
// depthwise-multiplier shapes.  Streams each row's offsets once through LDS.
struct DepthwisePlan {
    int outputs_per_block;  // LT
    int window;             // x window capacity in elements
    size_t lds_bytes;
    int64_t blocks;
};
DepthwisePlan plan_depthwise(const Params &p);
hipError_t launch_depthwise(const Params &p, const DepthwisePlan &pl, hipStream_t stream);

// Fused deformable im2col + MFMA GEMM (groups == 1).
struct MfmaPlan {
    bool ok;          // shape supported by this kernel
    int bm, bn, bk;   // block tile
    int tiles_m, tiles_n, splits, chunks;
    int64_t blocks;
    int threads;
    size_t lds_bytes;
    size_t ws_bytes;  // counters + partials (0 when splits == 1)
    const char *name;
    int variant;      // compiled window staging shape (index into its table)
    int nch, wt_max;  // channel rows per chunk, window capacity per row (0: gather)
    int off_mask, off_w, off_s, off_x;  // LDS layout (bytes)
    // channel-block reduction order (blocked != 0): CB channels per block,
    // ncb blocks, nkb tap groups, staging shape; the rearranged weights take
    // the first wb_bytes of the workspace, split partials follow
    int blocked, cb, slot, lpp, ncb, nkb;
    int variant_dw;  // the same shape reading the weights directly when they are 16-byte aligned (-1: none)
    size_t wb_bytes;
    // bf16 blocks of 32 channels at one tap per chunk: window positions of the
    // position-major kernel (k_mfma_cbt), taken when x is 16-byte aligned
    // (0: not planned; `variant` is then, or otherwise, the kernel)
    int tpos;
    // the one-wave-per-SIMD bf16 kernel (k_mfma_wide, 256 x 256 tiles): its
    // window capacity (0: not planned), tiles and LDS bytes; taken when x is
    // 16-byte aligned, the kernel above otherwise (grid `blocks` of the plan
    // below is then the one reported)
    int wide, wide_tiles_m, wide_tiles_n, wide_ncb;
    size_t wide_lds, wide_wb_bytes;
    int64_t fallback_blocks;
    int fallback_splits;
};
MfmaPlan plan_mfma(const Params &p, int num_cus);
hipError_t launch_mfma(const Params &p, const MfmaPlan &pl, hipStream_t stream);
// one per storage dtype and mask presence (k_mfma_*.hip)
hipError_t launch_mfma_f32(const Params &p, const MfmaPlan &pl, hipStream_t stream);
hipError_t launch_mfma_f32_mask(const Params &p, const MfmaPlan &pl, hipStream_t stream);
hipError_t launch_mfma_bf16(const Params &p, const MfmaPlan &pl, hipStream_t stream);
hipError_t launch_mfma_bf16_mask(const Params &p, const MfmaPlan &pl, hipStream_t stream);
// the one-wave-per-SIMD bf16 kernel (k_mfma_wide.hip); pl.wide must be planned
hipError_t launch_mfma_wide(const Params &p, const MfmaPlan &pl, hipStream_t stream);
bool wide_npos_compiled(int npos, int K);
int wide_npos_option(int i);  // compiled window capacities, ascending; 0 past the last
size_t wide_lds_bytes(int npos);

// Backward (fp32): gradients of sum(dout * out).  Any gradient pointer may
// be null (not computed); dS and S point into the workspace (S only when the
// weight gradient is wanted).
struct BwdParams {
    Params p;  // forward arguments; p.out unused
    const float *dout;
    float *gx, *goff, *gmask, *gw, *gb;
    float *dS, *S;
};
// Plain fp32 GEMM on the MFMA kernel (k_mfma.hip): C[b][m][j] =
// sum_k A[m][k] * x[b*bbatch + j + k*brow] with A = q.w [q.C_out][q.Kred],
// C = q.out [q.B][q.C_out][q.L_out]; split partials in q.ws.  out_mode 1 and
// 2 store instead the packed layer's generator heads: row g*q.K + k (g <
// q.G) of column (b, l) at q.out[((b*q.G + g)*q.L_out + l)*q.K + k]; with
// out_mode 2 the rows q.G*q.K + g*q.K + k are the mask head, stored the same
// way into q.mask through the logistic sigmoid.
size_t gemm_workspace_bytes(const Params &q, int out_mode, int num_cus);
hipError_t launch_gemm_f32(const Params &q, int64_t brow, int64_t bbatch, int out_mode, int num_cus,
                           hipStream_t stream);
// The same GEMM on bf16 operands (A = q.w, B from q.x, both bf16; fp32
// accumulation; C stored in bf16, RNE), out_mode 0 only.
hipError_t launch_gemm_bf16(const Params &q, int64_t brow, int64_t bbatch, int num_cus, hipStream_t stream);
size_t gemm_bf16_workspace_bytes(const Params &q, int num_cus);
// The packed layer's generator heads (k_heads.hip): off[b,g,l,k] =
// bias[g*K + k] + sum_c w[g*K + k][c] t[b,c,l] and, with mask, mask[b,g,l,k]
// = sigmoid(bias[G*K + g*K + k] + sum_c w[G*K + g*K + k][c] t[b,c,l]); t
// [B][C][L], w [M][C] (M = G*K, or 2*G*K with the mask head), off and mask
// [B][G][L][K], all fp32.  heads_fit: the shapes and alignments the kernel
// serves (K <= 4, C <= 64, M <= 128*K, L a multiple of 32, 16-byte aligned
// t, off, mask); the general head GEMM (launch_gemm_f32, out_mode 1 or 2)
// serves the rest.  With x non-null (fp32 x [B][C][L_in]) the kernel
// computes the trunk itself, t[b,c,l] = tb[c] + sum_k tw[c,k] *
// x~[b,c, l*stride - padding + k*dilation] (x~ zero outside [0, L_in)),
// the same sum in the same order as k_trunk, and t is not read; the head
// rows are then w (the offset head, G*K rows) and w2 (the mask head), with
// biases bias and bias2.
struct HeadArgs {
    const float *t, *w, *bias;  // bias may be null
    float *off, *mask;          // mask null without the mask head
    int B, C, L, G, K, M;
    // the fused trunk (x null: t is read)
    const float *x, *tw, *tb, *w2, *bias2;  // tb, bias2 may be null; w2 null without the mask head
    int L_in, stride, padding, dilation;
    int slabs, tiles_per_b, tiles, xvec;  // set by launch_heads
};
bool heads_fit(int C, int K, int M, int L, const void *t, const void *off, const void *mask);
hipError_t launch_heads(HeadArgs a, int num_cus, hipStream_t stream);
// The packed layer's trunk (fp32 storage): t[b,c,l] = tb[c] +
// sum_k tw[c,k] * x~[b,c, l*stride - padding + k*dilation], t [B][C][L_out].
struct TrunkArgs {
    const void *x;
    const float *tw, *tb;  // [C][K], [C] or null
    float *t;
    int dtype, B, C, L_in, L_out, K, stride, padding, dilation;
    // With wcat non-null the same launch also stacks the packed layer's two
    // heads for one GEMM: wcat = [ow; mw] ([2*GK][C] row-major), bcat =
    // [ob; mb] (null biases as zeros).
    const float *ow, *ob, *mw, *mb;
    float *wcat, *bcat;
    int GK;
};
hipError_t launch_trunk(const TrunkArgs &a, hipStream_t stream);
// ---- 2D modulated deformable convolution ---------------------------------
//
// x [B][C_in][H][W]; offsets [B][2*G*T][Ho][Wo] (T = kh*kw taps; channel
// 2*((g*kh + i)*kw + j) the row offset of tap (i, j) of group g, the next its
// column offset); mask [B][G*T][Ho][Wo] or null; weight
// [C_out][C_in/groups][kh][kw]; out [B][C_out][Ho][Wo].
struct Params2 {
    const void *x, *off, *mask, *w, *bias;
    void *out;
    int dtype;
    int B, C_in, C_out, H, W, Ho, Wo, kh, kw, sh, sw, ph, pw, dh, dw, groups, G;
    int cpg, opg, cpo, T, Kred;  // C_in/groups, C_out/groups, C_in/G, kh*kw, cpg*T
    void *ws;
    size_t ws_bytes;
};
// Workspace of the dense (groups == 1) path: the sampled matrix
// S [B][C_in*T][Ho*Wo] in the storage dtype, then the GEMM's split partials;
// 0 for the direct path.
size_t dc2d_workspace(const Params2 &p, int num_cus);
// Dense path (sampling kernel, then the MFMA GEMM) when groups == 1 and
// C_out >= 32, else one thread per output.
hipError_t launch_dc2d(const Params2 &p, int num_cus, hipStream_t stream);
const char *dc2d_kernel_name(const Params2 &p);

size_t backward_workspace_bytes(const Params &p, bool want_weight, int num_cus);
hipError_t launch_backward(BwdParams a, int num_cus, hipStream_t stream);

}  // namespace dc1d
