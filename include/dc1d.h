/*
 * dc1d.h -- C ABI of libdc1d, the MI355X (gfx950) forward pass of 1D
 * deformable convolution with an optional modulation mask.
 *
 * The operation (restated from the pages; each part cited by page and
 * section):
 *
 *   out[b, co, l] = bias[co]
 *       + sum_{ci in co's group} sum_{k < K} weight[co, ci_local, k] * S[b, ci, k, l]
 *
 *   S[b, ci, k, l] = m * ( (1 - f) * x~(i0) + f * x~(i0 + 1) )
 *       i0 = l*stride - padding + k*dilation + floor(o),   f = o - floor(o)
 *       o  = offsets[b, g, l, k],   g = ci / (C_in / offset_groups)
 *       m  = mask[b, g, l, k], or 1 when no mask is given
 *       x~(i) = x[b, ci, i] for 0 <= i < L_in, else 0
 *
 *   - The sum and its grid position l*stride - padding + k*dilation are the
 *     conv1d cross-correlation (conv1d operator page, section Description);
 *     the offset moves each tap's sampling point (dilated/deformable
 *     convolution article, section Deformable Convolution, the y(p0)
 *     formula, and its Step 2 / Step 3 workflow: sample, then weigh).
 *   - Sampling between integer positions is linear (dc1d page, section Demo
 *     notebook: integer offsets shift exactly, fractional ones interpolate
 *     linearly); samples off either end read zero (torchvision issue on the
 *     deform_conv2d offset layout, its printed demo output).
 *   - Offsets are [B, offset_groups, L_out, K] with offset_groups dividing
 *     C_in (dc1d page, section Usage / DeformConv1d); the mask has the same
 *     shape and is applied as given, no sigmoid inside (dc1d page, section
 *     Modulation (DCNv2)).
 *   - groups split channels into contiguous independent blocks, weight is
 *     [C_out, C_in/groups, K], bias [C_out] (conv1d operator page, sections
 *     Arguments and Axis convention).
 *   - L_out = floor((L_in + 2*padding - dilation*(K-1) - 1)/stride + 1)
 *     (conv1d operator page, section Shape).
 *
 * Layout: every tensor is dense, contiguous, row-major, channels-first
 * ([B, C, L], conv1d operator page, section Axis convention).  All tensors of
 * one call share one dtype; the output has the input's dtype (conv1d page:
 * the computation stays in the input dtype).  Arithmetic is fp32 inside the
 * kernels (bf16 values are widened exactly; a bf16 output is rounded once,
 * to nearest even).
 *
 * Ownership: the caller owns every buffer (device memory for tensors and the
 * workspace).  The library allocates nothing, keeps no pointer after a call
 * returns, and has no mutable global state other than a per-device
 * capability cache filled once.  Work is enqueued on the given HIP stream and
 * the call returns without synchronising; buffers must stay alive until that
 * stream's work is done.  Calls are re-entrant; calls that share a workspace
 * must be ordered on one stream.
 *
 * Logging: with the environment variable DC1D_LOG set to a non-zero value
 * (read once, at the first call that launches work), each such call writes
 * one line to stderr naming the entry, the shapes, the dtype, the kernel
 * chosen, its grid and split count and the workspace bytes.
 *
 * Errors: every entry returns a dc1d_status.  Errors detected on the host
 * return before any device work and write nothing.  Faults inside a kernel
 * surface at the caller's next synchronisation.  No C++ exception crosses
 * this boundary.
 */
#ifndef DC1D_H
#define DC1D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtypes. */
typedef enum dc1d_dtype {
    DC1D_F32 = 0,  /* IEEE binary32 */
    DC1D_BF16 = 1  /* bfloat16 (upper half of a binary32) */
} dc1d_dtype;

typedef enum dc1d_status {
    DC1D_OK = 0,
    DC1D_ERR_NULL_PTR = 1,  /* a required descriptor or data pointer is NULL */
    DC1D_ERR_BAD_ARG = 2,   /* stride/padding/dilation/groups/offset_groups/K out of range,
                               groups or offset_groups not dividing the channels,
                               offset_groups disagreeing with offsets->shape[1] */
    DC1D_ERR_BAD_SHAPE = 3, /* a tensor's rank or shape disagrees, L_out <= 0, or a size
                               beyond the supported limits (see dc1d_forward) */
    DC1D_ERR_BAD_DTYPE = 4, /* unsupported dtype, or dtypes mixed within a call */
    DC1D_ERR_ALIAS = 5,     /* out overlaps an input */
    DC1D_ERR_WORKSPACE = 6, /* workspace NULL, smaller than dc1d_workspace_bytes(), or not
                               256-byte aligned */
    DC1D_ERR_DEVICE = 7,    /* no current HIP device, or it is not a gfx950 */
    DC1D_ERR_LAUNCH = 8     /* the kernel launch reported an error */
} dc1d_status;

/* A dense, contiguous tensor in device memory.  shape[i] for i >= ndim is
 * ignored.  data may be NULL only when the tensor has no elements. */
typedef struct dc1d_tensor {
    void *data;
    int32_t dtype; /* a dc1d_dtype */
    int32_t ndim;
    int64_t shape[4];
} dc1d_tensor;

/*
 * conv1d output length (conv1d operator page, section Shape):
 *   floor((L_in + 2*padding - dilation*(K-1) - 1)/stride + 1).
 * Returns -1 when an argument is out of range (L_in < 0, K < 1, stride < 1,
 * padding < 0, dilation < 1) or the result is not positive.  Host only.
 */
int64_t dc1d_output_length(int64_t L_in, int64_t K, int64_t stride, int64_t padding,
                           int64_t dilation);

/*
 * Bytes of device workspace that dc1d_forward needs for these arguments on
 * the current device (0 when the chosen kernels need none).  Only the
 * descriptors' dtype, ndim and shape are read; data pointers may be NULL.
 * The same validation as dc1d_forward applies (except pointers and
 * aliasing).  What the workspace holds is described at dc1d_forward.
 */
int dc1d_workspace_bytes(const dc1d_tensor *x, const dc1d_tensor *offsets,
                         const dc1d_tensor *mask_or_null, const dc1d_tensor *weight,
                         const dc1d_tensor *bias_or_null, int64_t stride, int64_t padding,
                         int64_t dilation, int64_t groups, int64_t offset_groups,
                         size_t *bytes_out);

/*
 * Forward pass.  Overwrites all of out; never accumulates into it.
 *
 *   x       [B, C_in, L_in]
 *   offsets [B, offset_groups, L_out, K]     (K fastest)
 *   mask    [B, offset_groups, L_out, K] or NULL (NULL means a mask of ones;
 *           an all-ones mask gives bit-identical results)
 *   weight  [C_out, C_in/groups, K]
 *   bias    [C_out] or NULL (NULL means zero)
 *   out     [B, C_out, L_out]
 *
 * offset_groups must equal offsets->shape[1] (a double entry, checked).
 * stream is a hipStream_t (NULL: the null stream).
 *
 * workspace: device memory of at least dc1d_workspace_bytes() bytes, aligned
 * to 256 bytes, or NULL with workspace_bytes 0 when that is 0.  It holds the
 * weights rearranged into the kernel's reduction order (written by a first
 * kernel of the call) and the fp32 partial sums of a split reduction, passed
 * from the main kernel to a last one on the same stream; it needs no
 * initialisation and holds nothing between calls.  Calls in flight at the
 * same time must not share a workspace.
 *
 * An empty input sequence (L_in == 0) is rejected with DC1D_ERR_BAD_SHAPE
 * even when the padding would give L_out >= 1 (as conv1d rejects it).
 *
 * Limits (DC1D_ERR_BAD_SHAPE beyond them): L_in + padding <= 2^29,
 * dilation*(K-1) <= 2^29, L_out*stride <= 2^30, C_in*K <= 2^30,
 * C_out <= 2^30.  Offsets whose magnitude exceeds 2^29 are clamped to
 * +-2^29, which under these limits only moves a sample that already reads
 * zero.  Non-finite offsets or masks are outside the contract: the kernels
 * stay memory-safe but the values are unspecified.
 *
 * B == 0 is a valid no-op.  The call is asynchronous.
 */
int dc1d_forward(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                 const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                 int64_t stride, int64_t padding, int64_t dilation, int64_t groups,
                 int64_t offset_groups, void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as dc1d_forward (same kernels, same results bit for bit), with
 * its workspace taken from a scratch array that the library keeps in device
 * memory, one per device, of dc1d_noalloc_scratch_bytes() bytes (64 MiB),
 * held from the library's first use on that device until the process ends.
 * The call allocates nothing (no hipMalloc, no allocating library routine);
 * the caller still passes inputs and out.  Returns DC1D_ERR_WORKSPACE,
 * before any device work, when dc1d_workspace_bytes() for these arguments
 * exceeds the scratch size; DC1D_ERR_DEVICE if the scratch address cannot
 * be looked up.  Every call on one device shares that device's scratch
 * (it needs no initialisation and holds nothing useful between calls):
 * calls that may run at the same time on one device (different streams
 * without an ordering between them) race on it and must be serialised by
 * the caller.  Other arguments and errors as dc1d_forward.
 */
int dc1d_forward_noalloc(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                         const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                         int64_t stride, int64_t padding, int64_t dilation, int64_t groups,
                         int64_t offset_groups, void *stream);

/* Size in bytes of the per-device scratch array dc1d_forward_noalloc uses. */
size_t dc1d_noalloc_scratch_bytes(void);

/*
 * Profiling aid.  While set, every forward call made on the calling thread
 * (dc1d_forward, dc1d_forward_constrained, dc1d_forward_noalloc) records
 * start_event on its stream immediately before it launches its dominant
 * kernel (the fused sampling + MFMA kernel, or the depthwise or direct
 * kernel) and stop_event immediately after, so that the elapsed time
 * between them is that kernel's alone, without the small kernels the call
 * may also enqueue (the weight rearrangement before it, the split
 * reduction after it).  Both are hipEvent_t handles owned by the caller,
 * passed as void*; (NULL, NULL) turns the hook off.  The setting is
 * per thread and changes no result.  Returns DC1D_ERR_NULL_PTR when exactly
 * one of the two is NULL.
 */
int dc1d_set_kernel_events(void *start_event, void *stop_event);

/*
 * Constrained mode: dc1d_forward with every tap kept inside its receptive
 * field (the dc1d page's default, section Usage / DeformConv1d: each kernel
 * tap is constrained to its own receptive field unless the layer is made
 * unconstrained).  The page does not give the rule; this library reads the
 * receptive field as the undeformed kernel's window of the output,
 * [l*stride - padding, l*stride - padding + (K-1)*dilation], so tap k's
 * offset is clamped to [-k*dilation, (K-1-k)*dilation] before the position
 * is split; positions in the window outside [0, L_in) still read zero.
 * Same arguments, workspace and errors as dc1d_forward, plus
 * DC1D_ERR_BAD_ARG when (K-1)*dilation >= 2^24.
 */
int dc1d_forward_constrained(const dc1d_tensor *x, const dc1d_tensor *offsets,
                             const dc1d_tensor *mask_or_null, const dc1d_tensor *weight,
                             const dc1d_tensor *bias_or_null, const dc1d_tensor *out, int64_t stride,
                             int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward (fp32 or bf16 storage; every gradient has its input's dtype, and
 * grad_out the inputs' dtype).  For
 * grad_out = dL/d(out) [B, C_out, L_out], writes the gradients of
 * L = sum(grad_out * out) with respect to the inputs of dc1d_forward, each
 * into a caller buffer shaped like that input (NULL: not computed):
 *
 *   dS[b,ci,k,l]    = sum over co's group of weight[co,ci_local,k] * grad_out[b,co,l]
 *   grad_x[b,ci,i0] += dS*m*(1-f);  grad_x[b,ci,i0+1] += dS*m*f  (indices inside [0, L_in))
 *   grad_offsets[b,g,l,k] = sum over ci in g of dS*m*(x~(i0+1) - x~(i0))
 *   grad_mask[b,g,l,k]    = sum over ci in g of dS*((1-f)*x~(i0) + f*x~(i0+1))
 *   grad_weight[co,cl,k]  = sum over (b,l) of grad_out[b,co,l] * S[b,ci,k,l]
 *   grad_bias[co]         = sum over (b,l) of grad_out[b,co,l]
 *
 * with i0, f, m, x~ and S as in dc1d_forward: the derivatives of the
 * forward's definition term by term (the dc1d page trains the offsets and
 * checks their gradient against a finite difference, section Demo
 * notebook).  The offset gradient is that of the interpolation formula with
 * i0 held fixed, i.e. the right derivative at integer offsets.  Every
 * requested gradient is overwritten.  grad_x is gathered (each position's
 * sum formed by one thread in a fixed order) when the shape's gather arrays
 * fit in LDS, samples moved more than 16 positions then added with atomics;
 * otherwise it is cleared and accumulated with atomics.  grad_bias and, for
 * some shapes, the other gradients are accumulated with atomics.  Where
 * atomics are used the last bits may differ between runs.  grad_mask needs
 * a mask.  Gradients must not overlap the inputs, each other or the
 * workspace.
 *
 * bf16 storage: the inputs are widened exactly into fp32 copies in the
 * workspace, the fp32 kernels compute every gradient there (fp32
 * arithmetic, as above), and each requested gradient is rounded once, to
 * nearest even, into its bf16 buffer (the dc1d page trains the layer with
 * torch.autograd, whose gradients keep the input dtype; intro and section
 * Demo notebook).
 *
 * workspace: at least dc1d_backward_workspace_bytes() bytes, 256-byte
 * aligned, when that is not 0 (for bf16 it first holds the fp32 copies of
 * the inputs and the fp32 gradients; then dS = the gradient of the samples,
 * the transposed weight and the samples for the weight gradient, split
 * partial sums, and the grad_x gather's flag, depending on the shape;
 * depthwise shapes need only the flag, or nothing); no initialisation;
 * nothing kept.
 */
int dc1d_backward_workspace_bytes(const dc1d_tensor *x, const dc1d_tensor *offsets,
                                  const dc1d_tensor *mask_or_null, const dc1d_tensor *weight,
                                  const dc1d_tensor *grad_out, int want_grad_weight, int64_t stride,
                                  int64_t padding, int64_t dilation, int64_t groups,
                                  int64_t offset_groups, size_t *bytes_out);

int dc1d_backward(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                  const dc1d_tensor *weight, const dc1d_tensor *grad_out,
                  const dc1d_tensor *grad_x_or_null, const dc1d_tensor *grad_offsets_or_null,
                  const dc1d_tensor *grad_mask_or_null, const dc1d_tensor *grad_weight_or_null,
                  const dc1d_tensor *grad_bias_or_null, int64_t stride, int64_t padding,
                  int64_t dilation, int64_t groups, int64_t offset_groups, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * The packed layer (fp32 or bf16 storage, one dtype for every tensor of the
 * call): the layer computes its own offsets, and optionally its mask, from its input,
 * then runs the forward above with them (dc1d page, section
 * PackedDeformConv1d: offsets from a depthwise-separable convolutional
 * block; section Modulation (DCNv2): a second pointwise branch off the same
 * depthwise trunk, ending in a sigmoid, predicts the mask).  The block's
 * layers are only sketched there; this library reads them as:
 *
 *   t[b,c,l]          = trunk_bias[c] + sum_k trunk_weight[c,0,k] * x~[b,c, l*stride - padding + k*dilation]
 *   offsets[b,g,l,k]  = off_bias[g*K+k] + sum_c off_weight[g*K+k, c, 0] * t[b,c,l]
 *   mask[b,g,l,k]     = sigmoid(mask_bias[g*K+k] + sum_c mask_weight[g*K+k, c, 0] * t[b,c,l])
 *   out               = dc1d_forward(x, offsets, mask or none, weight, bias)
 *
 * i.e. a depthwise conv1d with the layer's K, stride, padding and dilation
 * (so it yields L_out columns), no activation, then pointwise convs whose
 * output channel g*K + k is tap k of offset group g; sigmoid(z) =
 * 1 / (1 + exp(-z)).  Shapes: x [B, C_in, L_in]; trunk_weight [C_in, 1, K];
 * trunk_bias [C_in]; off_weight and mask_weight [G*K, C_in, 1] (G = offset
 * groups, dividing C_in, implied by the shape); off_bias and mask_bias
 * [G*K]; weight, bias, out as in dc1d_forward; offsets_out and mask_out
 * [B, G, L_out, K].  Biases may be NULL (zero); mask_weight NULL means no
 * mask (then mask_bias and mask_out must be NULL too).  offsets_out /
 * mask_out, when given, receive the generated offsets / mask (the layer's
 * with_offsets output); otherwise they live in the workspace.  Outputs
 * must not overlap the inputs, each other or the workspace.
 * B * L_out must be below 2^31.
 *
 * bf16 storage: the generator (trunk and heads) runs in fp32 on the input
 * and on its parameters widened exactly; the offsets and mask it produces
 * are rounded once (to nearest even) to bf16, and the bf16 forward reads
 * those, as a layer computing in its input dtype does (conv1d operator
 * page: the computation stays in the input dtype).
 *
 * workspace: at least dc1d_packed_workspace_bytes() bytes, 256-byte
 * aligned, when that is not 0 (the trunk [B, C_in, L_out], the offsets and
 * mask in fp32, for bf16 also the widened parameters and the bf16 offsets
 * and mask, and the forward's own workspace); no initialisation; nothing
 * kept.
 */
int dc1d_packed_workspace_bytes(const dc1d_tensor *x, const dc1d_tensor *trunk_weight,
                                const dc1d_tensor *off_weight, const dc1d_tensor *mask_weight_or_null,
                                const dc1d_tensor *weight, int64_t stride, int64_t padding,
                                int64_t dilation, int64_t groups, size_t *bytes_out);

int dc1d_packed_forward(const dc1d_tensor *x, const dc1d_tensor *trunk_weight,
                        const dc1d_tensor *trunk_bias_or_null, const dc1d_tensor *off_weight,
                        const dc1d_tensor *off_bias_or_null, const dc1d_tensor *mask_weight_or_null,
                        const dc1d_tensor *mask_bias_or_null, const dc1d_tensor *weight,
                        const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                        const dc1d_tensor *offsets_out_or_null, const dc1d_tensor *mask_out_or_null,
                        int64_t stride, int64_t padding, int64_t dilation, int64_t groups,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * dc1d_packed_forward_constrained: the packed layer with the forward in the
 * constrained mode of dc1d_forward_constrained (each tap's offset clamped
 * to its window before the split).  The generated offsets, and the offsets
 * output, are the heads' own (unclamped).  Same arguments, workspace and
 * errors as dc1d_packed_forward, plus DC1D_ERR_BAD_ARG when
 * (K-1)*dilation >= 2^24.
 */
int dc1d_packed_forward_constrained(const dc1d_tensor *x, const dc1d_tensor *trunk_weight,
                        const dc1d_tensor *trunk_bias_or_null, const dc1d_tensor *off_weight,
                        const dc1d_tensor *off_bias_or_null, const dc1d_tensor *mask_weight_or_null,
                        const dc1d_tensor *mask_bias_or_null, const dc1d_tensor *weight,
                        const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                        const dc1d_tensor *offsets_out_or_null, const dc1d_tensor *mask_out_or_null,
                        int64_t stride, int64_t padding, int64_t dilation, int64_t groups,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of dc1d_forward_constrained: the gradients above at the clamped
 * offsets, with grad_offsets multiplied by the clamp's right derivative
 * (1 for an offset in [-k*dilation, (K-1-k)*dilation), 0 otherwise: a tap
 * held at its window's edge does not move).  Same arguments, workspace and
 * errors as dc1d_backward.
 */
int dc1d_backward_constrained(const dc1d_tensor *x, const dc1d_tensor *offsets,
                              const dc1d_tensor *mask_or_null, const dc1d_tensor *weight,
                              const dc1d_tensor *grad_out, const dc1d_tensor *grad_x_or_null,
                              const dc1d_tensor *grad_offsets_or_null, const dc1d_tensor *grad_mask_or_null,
                              const dc1d_tensor *grad_weight_or_null, const dc1d_tensor *grad_bias_or_null,
                              int64_t stride, int64_t padding, int64_t dilation, int64_t groups,
                              int64_t offset_groups, void *workspace, size_t workspace_bytes, void *stream);

/*
 * 2D modulated deformable convolution (DCNv2), the variant the deformable
 * convolution article describes (section Deformable Convolution: every tap
 * of a 2D kernel moved by its own offset, Step 2 bilinear sampling between
 * the four surrounding pixels, Step 3 the weighted sum), with the offset
 * layout of torchvision's deform_conv2d as its documentation issue settles
 * it:
 *
 *   x        [B, C_in, H, W]
 *   offsets  [B, 2*G*kh*kw, H_out, W_out]: channel 2*((g*kh + i)*kw + j) is
 *            the row (height) offset of kernel tap (i, j) for offset group g,
 *            the next channel its column (width) offset
 *   mask     [B, G*kh*kw, H_out, W_out] or NULL (channel (g*kh + i)*kw + j),
 *            multiplied as given
 *   weight   [C_out, C_in/groups, kh, kw];  bias [C_out] or NULL
 *   out      [B, C_out, H_out, W_out], overwritten
 *
 *   out[b,co,oh,ow] = bias[co] + sum over the group's ci and taps (i, j) of
 *       weight[co,ci_local,i,j] * m * bilinear(x[b,ci], oh*stride_h - pad_h +
 *       i*dil_h + dy, ow*stride_w - pad_w + j*dil_w + dx)
 *
 * with channel ci in offset group ci / (C_in/G); each coordinate split as
 * in the 1D forward (integer grid term plus the floor of the offset);
 * bilinear weights (1-fy)(1-fx), (1-fy)fx, fy(1-fx), fy fx on the four
 * neighbours, a neighbour outside the image reading 0.  H_out and W_out
 * follow dc1d_output_length per axis.  Storage fp32 or bf16 (one dtype per
 * call; fp32 arithmetic, bf16 samples rounded once for the bf16 MFMA).
 * Limits (DC1D_ERR_BAD_SHAPE beyond them): H >= 1 and W >= 1 (an empty
 * image is rejected even when the padding would give outputs), H*W < 2^31, B <= 65535,
 * B*H_out*W_out < 2^31, G*kh*kw <= 2^24, and the 1D position limits per
 * axis.  workspace: at least dc2d_workspace_bytes() bytes, 256-byte aligned,
 * when that is not 0 (the sampled matrix [B, C_in*kh*kw, H_out*W_out] in the
 * storage dtype and split partial sums; dense layers only); no
 * initialisation; nothing kept.  Errors as dc1d_forward.
 */
int dc2d_workspace_bytes(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                         const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, int64_t stride_h,
                         int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w,
                         int64_t groups, int64_t offset_groups, size_t *bytes_out);

int dc2d_forward(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                 const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                 int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w,
                 int64_t groups, int64_t offset_groups, void *workspace, size_t workspace_bytes, void *stream);

/* Which path dc2d_forward takes ("im2col2d_gemm_f32", "im2col2d_gemm_bf16",
 * "direct2d"); same validation as dc2d_workspace_bytes, no device query. */
int dc2d_plan(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
              const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, int64_t stride_h, int64_t stride_w,
              int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w, int64_t groups, int64_t offset_groups,
              const char **kernel_name);

/*
 * Test aid: the sampling positions the forward kernels use, from the same
 * device function.  For every (b, g, l, k) of offsets [B, G, L_out, K]
 * (K = offsets->shape[3]; L_out must equal dc1d_output_length(L_in, K, ...)):
 *   i0[idx]    = l*stride - padding + k*dilation + floor(o)   (int32, exact)
 *   frac[idx]  = o - floor(o)                                 (fp32)
 *   valid[idx] = (0 <= i0 < L_in) | (0 <= i0+1 < L_in) << 1
 * i0, frac and valid are device buffers of B*G*L_out*K elements each.
 */
int dc1d_debug_positions(const dc1d_tensor *offsets, int64_t L_in, int64_t stride,
                         int64_t padding, int64_t dilation, int32_t *i0, float *frac,
                         uint8_t *valid, void *stream);

/*
 * Which kernel dc1d_forward would launch for these arguments on the
 * current device, as a short static string ("mfma_f32", "mfma_bf16",
 * "depthwise", "direct", ...), and its launch shape.  Same validation as
 * dc1d_workspace_bytes.  For logging, tests and profiling.
 */
int dc1d_plan(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
              const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, int64_t stride,
              int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups,
              const char **kernel_name, int64_t *grid_blocks, int32_t *block_threads,
              int32_t *splits);

/* A static, NUL-terminated description of a status code. */
const char *dc1d_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DC1D_H */
