// api.hip -- the C ABI of libdc1d (include/dc1d.h): argument validation,
// kernel choice, and launch.  No allocation, no synchronisation, no
// exceptions across the boundary.
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dc1d.h"
#include "dc1d_internal.h"

using namespace dc1d;

namespace {

constexpr int64_t kMaxPos = (int64_t)1 << 29;  // position-range limit (see dc1d.h)
constexpr int kMaxDevices = 64;

struct DeviceInfo {
    bool gfx950;
    int num_cus;
};

std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];

// Profiling hook (dc1d_set_kernel_events): per calling thread.
thread_local void *t_ev_start = nullptr, *t_ev_stop = nullptr;

// Dispatch log: with the environment variable DC1D_LOG set to a non-zero
// value when the library first looks, every call that launches work writes
// one line to stderr (entry, shapes, dtype, the kernel chosen, its grid and
// split count, workspace bytes).  Read once.
bool log_on() {
    static const bool on = [] {
        const char *v = getenv("DC1D_LOG");
        return v && v[0] && strcmp(v, "0") != 0;
    }();
    return on;
}

// The current device's capability, probed once per device.
int current_device(DeviceInfo *info) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return DC1D_ERR_DEVICE;
    }
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        DeviceInfo di = {false, 0};
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
            di.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            di.num_cus = prop.multiProcessorCount;
        } else {
            (void)hipGetLastError();
        }
        g_dev[dev] = di;
    });
    *info = g_dev[dev];
    return info->gfx950 ? DC1D_OK : DC1D_ERR_DEVICE;
}

// The element count of a tensor, or -1 when its rank is outside 0..4, a
// dimension is negative, or the count exceeds kMaxElems; each product is
// checked before it is formed, so no arithmetic overflows.
constexpr int64_t kMaxElems = (int64_t)1 << 48;
int64_t numel_checked(const dc1d_tensor *t) {
    if (t->ndim < 0 || t->ndim > 4) return -1;
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) {
        const int64_t s = t->shape[i];
        if (s < 0) return -1;
        if (s > 0 && n > kMaxElems / s) return -1;
        n *= s;
    }
    return n;
}

// The element count of a tensor that validation has accepted.
int64_t numel(const dc1d_tensor *t) { return numel_checked(t); }

size_t elem_size(int dtype) { return dtype == DC1D_F32 ? 4 : 2; }

bool shape_is(const dc1d_tensor *t, int ndim, const int64_t *s) {
    if (t->ndim != ndim) return false;
    for (int i = 0; i < ndim; ++i)
        if (t->shape[i] != s[i]) return false;
    return true;
}

// Validate shapes and arguments and fill p (pointers included).
int validate(const dc1d_tensor *x, const dc1d_tensor *off, const dc1d_tensor *mask,
             const dc1d_tensor *w, const dc1d_tensor *bias, const dc1d_tensor *out, int64_t stride,
             int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups, Params *p) {
    if (!x || !off || !w) return DC1D_ERR_NULL_PTR;
    if (stride < 1 || padding < 0 || dilation < 1 || groups < 1 || offset_groups < 1)
        return DC1D_ERR_BAD_ARG;
    if (x->ndim != 3 || w->ndim != 3 || off->ndim != 4) return DC1D_ERR_BAD_SHAPE;
    const int dt = x->dtype;
    if (dt != DC1D_F32 && dt != DC1D_BF16) return DC1D_ERR_BAD_DTYPE;
    if (off->dtype != dt || w->dtype != dt || (mask && mask->dtype != dt) ||
        (bias && bias->dtype != dt) || (out && out->dtype != dt))
        return DC1D_ERR_BAD_DTYPE;
    const int64_t B = x->shape[0], C_in = x->shape[1], L_in = x->shape[2];
    const int64_t C_out = w->shape[0], K = w->shape[2];
    // an empty input sequence has nothing to sample (conv1d rejects it too),
    // and the kernels' samplers assume at least one element per row
    if (B < 0 || C_in < 1 || L_in < 1 || C_out < 1 || K < 1) return DC1D_ERR_BAD_SHAPE;
    // every size bounded on its own before any product of two is formed
    const int64_t lim30 = (int64_t)1 << 30;
    if (L_in > kMaxPos || padding > kMaxPos || K > kMaxPos || dilation > kMaxPos || stride > lim30 ||
        C_in > lim30 || C_out > lim30 || B > lim30 || offset_groups > lim30)
        return DC1D_ERR_BAD_SHAPE;
    if (C_in % groups || C_out % groups || C_in % offset_groups) return DC1D_ERR_BAD_ARG;
    if (off->shape[1] != offset_groups) return DC1D_ERR_BAD_ARG;
    if (w->shape[1] != C_in / groups) return DC1D_ERR_BAD_SHAPE;
    // size limits that keep all position arithmetic inside int32
    if (L_in + padding > kMaxPos || dilation * (K - 1) > kMaxPos || C_in * K > lim30 ||
        offset_groups * K > lim30)
        return DC1D_ERR_BAD_SHAPE;
    const int64_t L_out = dc1d_output_length(L_in, K, stride, padding, dilation);
    if (L_out < 1 || L_out * stride > lim30) return DC1D_ERR_BAD_SHAPE;
    // the sampled tensor [B, C_in, K, L_out] (the backward's workspace holds
    // it) and every operand stay countable
    if (B > 0 && C_in * K * B > kMaxElems / L_out) return DC1D_ERR_BAD_SHAPE;
    const dc1d_tensor *ts[6] = {x, off, mask, w, bias, out};
    for (const dc1d_tensor *t : ts)
        if (t && numel_checked(t) < 0) return DC1D_ERR_BAD_SHAPE;
    const int64_t so[4] = {B, offset_groups, L_out, K};
    if (!shape_is(off, 4, so)) return DC1D_ERR_BAD_SHAPE;
    if (mask && !shape_is(mask, 4, so)) return DC1D_ERR_BAD_SHAPE;
    const int64_t sb[1] = {C_out};
    if (bias && !shape_is(bias, 1, sb)) return DC1D_ERR_BAD_SHAPE;
    const int64_t sout[3] = {B, C_out, L_out};
    if (out && !shape_is(out, 3, sout)) return DC1D_ERR_BAD_SHAPE;

    memset(p, 0, sizeof(*p));
    p->x = x->data;
    p->off = off->data;
    p->mask = mask ? mask->data : nullptr;
    p->w = w->data;
    p->bias = bias ? bias->data : nullptr;
    p->out = out ? out->data : nullptr;
    p->dtype = dt;
    p->B = (int)B;
    p->C_in = (int)C_in;
    p->C_out = (int)C_out;
    p->L_in = (int)L_in;
    p->L_out = (int)L_out;
    p->K = (int)K;
    p->stride = (int)stride;
    p->padding = (int)padding;
    p->dilation = (int)dilation;
    p->groups = (int)groups;
    p->G = (int)offset_groups;
    p->cpg = (int)(C_in / groups);
    p->opg = (int)(C_out / groups);
    p->cpo = (int)(C_in / offset_groups);
    p->Kred = (int)(C_in / groups * K);
    return DC1D_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

enum Kernel { kDirect, kDepthwise, kMfma };

struct Plan {
    Kernel kernel;
    MfmaPlan mfma;
    DepthwisePlan dw;
    size_t ws_bytes;
    const char *name;
    int64_t grid;
    int block;
    int splits;
};

Plan make_plan(const Params &p, const DeviceInfo &dev) {
    Plan pl = {};
    pl.mfma = plan_mfma(p, dev.num_cus);
    if (pl.mfma.ok) {
        pl.kernel = kMfma;
        pl.ws_bytes = pl.mfma.ws_bytes;
        pl.name = pl.mfma.name;
        pl.grid = pl.mfma.blocks;
        pl.block = pl.mfma.threads;
        pl.splits = pl.mfma.splits;
        return pl;
    }
    if (p.cpg == 1 && plan_depthwise(p).blocks < ((int64_t)1 << 31)) {
        pl.kernel = kDepthwise;
        pl.dw = plan_depthwise(p);
        pl.name = "depthwise";
        pl.grid = pl.dw.blocks;
        pl.block = 256;
        pl.splits = 1;
        return pl;
    }
    pl.kernel = kDirect;
    pl.name = "direct";
    const int64_t total = (int64_t)p.B * p.C_out * p.L_out;
    pl.grid = (total + 255) / 256;
    pl.block = 256;
    pl.splits = 1;
    return pl;
}

}  // namespace

extern "C" {

int64_t dc1d_output_length(int64_t L_in, int64_t K, int64_t stride, int64_t padding, int64_t dilation) {
    if (L_in < 0 || K < 1 || stride < 1 || padding < 0 || dilation < 1) return -1;
    if (L_in > ((int64_t)1 << 40) || padding > ((int64_t)1 << 40) || K > ((int64_t)1 << 40) ||
        dilation > ((int64_t)1 << 20))
        return -1;  // keeps the arithmetic below exact in int64
    const int64_t num = L_in + 2 * padding - dilation * (K - 1) - 1;
    if (num < 0) return -1;
    return num / stride + 1;
}

int dc1d_workspace_bytes(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                         const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, int64_t stride,
                         int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups,
                         size_t *bytes_out) {
    if (!bytes_out) return DC1D_ERR_NULL_PTR;
    Params p;
    int st = validate(x, offsets, mask_or_null, weight, bias_or_null, nullptr, stride, padding, dilation,
                      groups, offset_groups, &p);
    if (st) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev))) return st;
    *bytes_out = make_plan(p, dev).ws_bytes;
    return DC1D_OK;
}

int dc1d_plan(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
              const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, int64_t stride, int64_t padding,
              int64_t dilation, int64_t groups, int64_t offset_groups, const char **kernel_name,
              int64_t *grid_blocks, int32_t *block_threads, int32_t *splits) {
    Params p;
    int st = validate(x, offsets, mask_or_null, weight, bias_or_null, nullptr, stride, padding, dilation,
                      groups, offset_groups, &p);
    if (st) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev))) return st;
    const Plan pl = make_plan(p, dev);
    if (kernel_name) *kernel_name = pl.name;
    if (grid_blocks) *grid_blocks = pl.grid;
    if (block_threads) *block_threads = pl.block;
    if (splits) *splits = pl.splits;
    return DC1D_OK;
}

}  // extern "C"

namespace {

// The constrained mode's tap bounds -k*d and (K-1-k)*d must be exact floats.
bool constrained_ok(const Params &p) { return (int64_t)(p.K - 1) * p.dilation < ((int64_t)1 << 24); }

// The allocation-free entry's workspace: one fixed array per device, in
// device memory for the life of the process.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the device address is looked up once per device and kept.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];

// The current device's scratch address (nullptr if the lookup failed).
void *scratch_address(int dev) {
    std::call_once(g_scratch_once[dev], [dev]() {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            ptr = nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    });
    return g_scratch_ptr[dev];
}

int forward_impl(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                 const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                 int64_t stride, int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups,
                 void *workspace, size_t workspace_bytes, void *stream, int constrained,
                 bool use_scratch = false) {
    if (!out) return DC1D_ERR_NULL_PTR;
    Params p;
    int st = validate(x, offsets, mask_or_null, weight, bias_or_null, out, stride, padding, dilation, groups,
                      offset_groups, &p);
    if (st) return st;
    if (constrained && !constrained_ok(p)) return DC1D_ERR_BAD_ARG;
    p.constrained = constrained;
    // data pointers: required for every tensor with elements
    const dc1d_tensor *all[6] = {x, offsets, mask_or_null, weight, bias_or_null, out};
    for (const dc1d_tensor *t : all)
        if (t && numel(t) > 0 && !t->data) return DC1D_ERR_NULL_PTR;
    // out must not overlap any input
    const size_t es = elem_size(p.dtype);
    const size_t out_bytes = (size_t)numel(out) * es;
    for (int i = 0; i < 5; ++i)
        if (all[i] && overlaps(out->data, out_bytes, all[i]->data, (size_t)numel(all[i]) * es))
            return DC1D_ERR_ALIAS;
    DeviceInfo dev;
    if ((st = current_device(&dev))) return st;
    const Plan pl = make_plan(p, dev);
    if (use_scratch) {
        if (pl.ws_bytes > kScratchBytes) return DC1D_ERR_WORKSPACE;
        int d = -1;
        if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices) return DC1D_ERR_DEVICE;
        workspace = pl.ws_bytes > 0 ? scratch_address(d) : nullptr;
        if (pl.ws_bytes > 0 && !workspace) return DC1D_ERR_DEVICE;
        workspace_bytes = pl.ws_bytes > 0 ? kScratchBytes : 0;
    }
    if (pl.ws_bytes > 0) {
        if (!workspace || workspace_bytes < pl.ws_bytes || ((uintptr_t)workspace & 255))
            return DC1D_ERR_WORKSPACE;
        if (overlaps(workspace, pl.ws_bytes, out->data, out_bytes)) return DC1D_ERR_ALIAS;
        for (int i = 0; i < 5; ++i)
            if (all[i] && overlaps(workspace, pl.ws_bytes, all[i]->data, (size_t)numel(all[i]) * es))
                return DC1D_ERR_ALIAS;
    }
    if (p.B == 0) return DC1D_OK;
    if (log_on())
        fprintf(stderr,
                "dc1d: %s B=%d C_in=%d C_out=%d L_in=%d L_out=%d K=%d s=%d p=%d d=%d groups=%d G=%d mask=%d %s "
                "-> %s grid=%lld block=%d splits=%d ws=%zu\n",
                use_scratch ? "forward_noalloc" : (constrained ? "forward_constrained" : "forward"), p.B, p.C_in,
                p.C_out, p.L_in, p.L_out, p.K, p.stride, p.padding, p.dilation, p.groups, p.G, p.mask != nullptr,
                p.dtype == DC1D_F32 ? "f32" : "bf16", pl.name, (long long)pl.grid, pl.block, pl.splits, pl.ws_bytes);
    p.ws = workspace;
    p.ws_bytes = workspace_bytes;
    p.ev_start = t_ev_start;
    p.ev_stop = t_ev_stop;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (pl.kernel) {
    case kMfma: e = launch_mfma(p, pl.mfma, s); break;
    case kDepthwise:
        mark_event(p.ev_start, s);
        e = launch_depthwise(p, pl.dw, s);
        mark_event(p.ev_stop, s);
        break;
    default:
        mark_event(p.ev_start, s);
        e = launch_direct(p, s);
        mark_event(p.ev_stop, s);
        break;
    }
    return e == hipSuccess ? DC1D_OK : DC1D_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int dc1d_forward(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                 const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                 int64_t stride, int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups,
                 void *workspace, size_t workspace_bytes, void *stream) {
    return forward_impl(x, offsets, mask_or_null, weight, bias_or_null, out, stride, padding, dilation, groups,
                        offset_groups, workspace, workspace_bytes, stream, 0);
}

int dc1d_forward_noalloc(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                         const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                         int64_t stride, int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups,
                         void *stream) {
    return forward_impl(x, offsets, mask_or_null, weight, bias_or_null, out, stride, padding, dilation, groups,
                        offset_groups, nullptr, 0, stream, 0, true);
}

size_t dc1d_noalloc_scratch_bytes(void) { return kScratchBytes; }

int dc1d_set_kernel_events(void *start_event, void *stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) return DC1D_ERR_NULL_PTR;
    t_ev_start = start_event;
    t_ev_stop = stop_event;
    return DC1D_OK;
}

int dc1d_forward_constrained(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                             const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                             int64_t stride, int64_t padding, int64_t dilation, int64_t groups,
                             int64_t offset_groups, void *workspace, size_t workspace_bytes, void *stream) {
    return forward_impl(x, offsets, mask_or_null, weight, bias_or_null, out, stride, padding, dilation, groups,
                        offset_groups, workspace, workspace_bytes, stream, 1);
}

}  // extern "C"

namespace {

// Backward arguments: the forward's (without bias and out) plus grad_out and
// the optional gradients, each shaped like its input.
int validate_backward(const dc1d_tensor *x, const dc1d_tensor *off, const dc1d_tensor *mask,
                      const dc1d_tensor *w, const dc1d_tensor *gout, const dc1d_tensor *gx,
                      const dc1d_tensor *goff, const dc1d_tensor *gmask, const dc1d_tensor *gw,
                      const dc1d_tensor *gb, int64_t stride, int64_t padding, int64_t dilation,
                      int64_t groups, int64_t offset_groups, Params *p) {
    if (!gout) return DC1D_ERR_NULL_PTR;
    int st = validate(x, off, mask, w, nullptr, gout, stride, padding, dilation, groups, offset_groups, p);
    if (st) return st;
    if (gmask && !mask) return DC1D_ERR_BAD_ARG;
    // every gradient has its input's dtype
    const dc1d_tensor *pairs[4][2] = {{gx, x}, {goff, off}, {gmask, mask}, {gw, w}};
    for (auto &pr : pairs) {
        if (!pr[0]) continue;
        if (pr[0]->dtype != p->dtype) return DC1D_ERR_BAD_DTYPE;
        if (!shape_is(pr[0], pr[1]->ndim, pr[1]->shape)) return DC1D_ERR_BAD_SHAPE;
    }
    if (gb) {
        const int64_t sb[1] = {p->C_out};
        if (gb->dtype != p->dtype) return DC1D_ERR_BAD_DTYPE;
        if (!shape_is(gb, 1, sb)) return DC1D_ERR_BAD_SHAPE;
    }
    return DC1D_OK;
}

// A bf16 backward runs the fp32 kernels on fp32 copies of its inputs and
// rounds each gradient once into the caller's bf16 buffer.  The copies and
// the fp32 gradients sit at the start of the workspace (byte offsets below),
// the fp32 backward's own workspace after them.
struct Bf16Bwd {
    size_t x, off, mask, w, dout, gx, goff, gmask, gw, gb, total;
};

Bf16Bwd bf16_backward_layout(const Params &p) {
    Bf16Bwd L = {};
    size_t o = 0;
    auto take = [&](int64_t n) {
        const size_t at = o;
        o += ((size_t)n * 4 + 255) & ~(size_t)255;
        return at;
    };
    const int64_t nx = (int64_t)p.B * p.C_in * p.L_in, no = (int64_t)p.B * p.G * p.L_out * p.K;
    const int64_t nw = (int64_t)p.C_out * p.cpg * p.K, nd = (int64_t)p.B * p.C_out * p.L_out;
    L.x = take(nx);
    L.off = take(no);
    L.mask = p.mask ? take(no) : 0;
    L.w = take(nw);
    L.dout = take(nd);
    L.gx = take(nx);
    L.goff = take(no);
    L.gmask = p.mask ? take(no) : 0;
    L.gw = take(nw);
    L.gb = take(p.C_out);
    L.total = o;
    return L;
}

// Workspace of a backward call: the fp32 backward's, plus the copies of a bf16 call.
size_t backward_ws(const Params &p, bool want_weight, int num_cus) {
    if (p.dtype != DC1D_BF16) return backward_workspace_bytes(p, want_weight, num_cus);
    Params q = p;
    q.dtype = DC1D_F32;
    return bf16_backward_layout(p).total + backward_workspace_bytes(q, want_weight, num_cus);
}

}  // namespace

extern "C" {

int dc1d_backward_workspace_bytes(const dc1d_tensor *x, const dc1d_tensor *offsets,
                                  const dc1d_tensor *mask_or_null, const dc1d_tensor *weight,
                                  const dc1d_tensor *grad_out, int want_grad_weight, int64_t stride,
                                  int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups,
                                  size_t *bytes_out) {
    if (!bytes_out) return DC1D_ERR_NULL_PTR;
    Params p;
    int st = validate_backward(x, offsets, mask_or_null, weight, grad_out, nullptr, nullptr, nullptr, nullptr,
                               nullptr, stride, padding, dilation, groups, offset_groups, &p);
    if (st) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev))) return st;
    *bytes_out = backward_ws(p, want_grad_weight != 0, dev.num_cus);
    return DC1D_OK;
}

}  // extern "C"

namespace {

int backward_impl(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                  const dc1d_tensor *weight, const dc1d_tensor *grad_out, const dc1d_tensor *grad_x_or_null,
                  const dc1d_tensor *grad_offsets_or_null, const dc1d_tensor *grad_mask_or_null,
                  const dc1d_tensor *grad_weight_or_null, const dc1d_tensor *grad_bias_or_null, int64_t stride,
                  int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups, void *workspace,
                  size_t workspace_bytes, void *stream, int constrained) {
    Params p;
    int st = validate_backward(x, offsets, mask_or_null, weight, grad_out, grad_x_or_null, grad_offsets_or_null,
                               grad_mask_or_null, grad_weight_or_null, grad_bias_or_null, stride, padding,
                               dilation, groups, offset_groups, &p);
    if (st) return st;
    if (constrained && !constrained_ok(p)) return DC1D_ERR_BAD_ARG;
    p.constrained = constrained;
    const dc1d_tensor *ins[5] = {x, offsets, mask_or_null, weight, grad_out};
    const dc1d_tensor *outs[5] = {grad_x_or_null, grad_offsets_or_null, grad_mask_or_null, grad_weight_or_null,
                                  grad_bias_or_null};
    for (const dc1d_tensor *t : ins)
        if (t && numel(t) > 0 && !t->data) return DC1D_ERR_NULL_PTR;
    for (const dc1d_tensor *t : outs)
        if (t && numel(t) > 0 && !t->data) return DC1D_ERR_NULL_PTR;
    // no gradient may overlap an input or another gradient
    const size_t es = elem_size(p.dtype);
    for (int i = 0; i < 5; ++i) {
        const dc1d_tensor *o = outs[i];
        if (!o) continue;
        const size_t ob = (size_t)numel(o) * es;
        for (const dc1d_tensor *t : ins)
            if (t && overlaps(o->data, ob, t->data, (size_t)numel(t) * es)) return DC1D_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (outs[j] && overlaps(o->data, ob, outs[j]->data, (size_t)numel(outs[j]) * es)) return DC1D_ERR_ALIAS;
    }
    DeviceInfo dev;
    if ((st = current_device(&dev))) return st;
    // ... nor the workspace
    const size_t need = backward_ws(p, grad_weight_or_null != nullptr, dev.num_cus);
    for (const dc1d_tensor *o : outs)
        if (o && workspace && overlaps(o->data, (size_t)numel(o) * es, workspace, need)) return DC1D_ERR_ALIAS;
    const bool want_ds = grad_x_or_null || grad_offsets_or_null || grad_mask_or_null || grad_weight_or_null;
    const bool bf16 = p.dtype == DC1D_BF16;  // the copies need the workspace whatever the shape
    if ((want_ds && need > 0 && (int64_t)p.B * p.C_in * p.K * p.L_out > 0) || (bf16 && need > 0)) {
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255)) return DC1D_ERR_WORKSPACE;
        for (const dc1d_tensor *t : ins)
            if (t && overlaps(workspace, need, t->data, (size_t)numel(t) * es)) return DC1D_ERR_ALIAS;
    }
    if (log_on())
        fprintf(stderr,
                "dc1d: %s B=%d C_in=%d C_out=%d L_in=%d L_out=%d K=%d s=%d p=%d d=%d groups=%d G=%d mask=%d f32 "
                "grads=%s%s%s%s%s ws=%zu\n",
                constrained ? "backward_constrained" : "backward", p.B, p.C_in, p.C_out, p.L_in, p.L_out, p.K,
                p.stride, p.padding, p.dilation, p.groups, p.G, p.mask != nullptr, grad_x_or_null ? "x," : "",
                grad_offsets_or_null ? "offsets," : "", grad_mask_or_null ? "mask," : "",
                grad_weight_or_null ? "weight," : "", grad_bias_or_null ? "bias" : "", need);
    BwdParams a;
    a.p = p;
    a.dout = (const float *)grad_out->data;
    a.gx = grad_x_or_null ? (float *)grad_x_or_null->data : nullptr;
    a.goff = grad_offsets_or_null ? (float *)grad_offsets_or_null->data : nullptr;
    a.gmask = grad_mask_or_null ? (float *)grad_mask_or_null->data : nullptr;
    a.gw = grad_weight_or_null ? (float *)grad_weight_or_null->data : nullptr;
    a.gb = grad_bias_or_null ? (float *)grad_bias_or_null->data : nullptr;
    a.dS = (float *)workspace;  // the workspace base; launch_backward lays it out
    a.S = nullptr;
    hipStream_t s = (hipStream_t)stream;
    if (!bf16) {
        const hipError_t e = launch_backward(a, dev.num_cus, s);
        return e == hipSuccess ? DC1D_OK : DC1D_ERR_LAUNCH;
    }
    // bf16: widen the inputs into the workspace, run the fp32 backward on
    // them into fp32 gradients there, round each gradient into its buffer
    const Bf16Bwd L = bf16_backward_layout(p);
    char *ws = (char *)workspace;
    const int64_t nx = (int64_t)p.B * p.C_in * p.L_in, no = (int64_t)p.B * p.G * p.L_out * p.K;
    const int64_t nw = (int64_t)p.C_out * p.cpg * p.K, nd = (int64_t)p.B * p.C_out * p.L_out;
    hipError_t e = hipSuccess;
    auto widen = [&](const void *src, size_t at, int64_t n) {
        if (e == hipSuccess) e = launch_convert(src, kBF16, ws + at, kF32, n, s);
    };
    widen(p.x, L.x, nx);
    widen(p.off, L.off, no);
    if (p.mask) widen(p.mask, L.mask, no);
    widen(p.w, L.w, nw);
    widen(grad_out->data, L.dout, nd);
    BwdParams b = a;
    b.p.dtype = kF32;
    b.p.x = ws + L.x;
    b.p.off = ws + L.off;
    b.p.mask = p.mask ? ws + L.mask : nullptr;
    b.p.w = ws + L.w;
    b.dout = (const float *)(ws + L.dout);
    b.gx = a.gx ? (float *)(ws + L.gx) : nullptr;
    b.goff = a.goff ? (float *)(ws + L.goff) : nullptr;
    b.gmask = a.gmask ? (float *)(ws + L.gmask) : nullptr;
    b.gw = a.gw ? (float *)(ws + L.gw) : nullptr;
    b.gb = a.gb ? (float *)(ws + L.gb) : nullptr;
    b.dS = (float *)(ws + L.total);
    if (e == hipSuccess) e = launch_backward(b, dev.num_cus, s);
    auto narrow = [&](const float *src, void *dst, int64_t n) {
        if (e == hipSuccess && dst) e = launch_convert(src, kF32, dst, kBF16, n, s);
    };
    narrow(b.gx, a.gx, nx);
    narrow(b.goff, a.goff, no);
    narrow(b.gmask, a.gmask, no);
    narrow(b.gw, a.gw, nw);
    narrow(b.gb, a.gb, p.C_out);
    return e == hipSuccess ? DC1D_OK : DC1D_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int dc1d_backward(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                  const dc1d_tensor *weight, const dc1d_tensor *grad_out, const dc1d_tensor *grad_x_or_null,
                  const dc1d_tensor *grad_offsets_or_null, const dc1d_tensor *grad_mask_or_null,
                  const dc1d_tensor *grad_weight_or_null, const dc1d_tensor *grad_bias_or_null, int64_t stride,
                  int64_t padding, int64_t dilation, int64_t groups, int64_t offset_groups, void *workspace,
                  size_t workspace_bytes, void *stream) {
    return backward_impl(x, offsets, mask_or_null, weight, grad_out, grad_x_or_null, grad_offsets_or_null,
                         grad_mask_or_null, grad_weight_or_null, grad_bias_or_null, stride, padding, dilation, groups,
                         offset_groups, workspace, workspace_bytes, stream, 0);
}

int dc1d_backward_constrained(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                              const dc1d_tensor *weight, const dc1d_tensor *grad_out,
                              const dc1d_tensor *grad_x_or_null, const dc1d_tensor *grad_offsets_or_null,
                              const dc1d_tensor *grad_mask_or_null, const dc1d_tensor *grad_weight_or_null,
                              const dc1d_tensor *grad_bias_or_null, int64_t stride, int64_t padding,
                              int64_t dilation, int64_t groups, int64_t offset_groups, void *workspace,
                              size_t workspace_bytes, void *stream) {
    return backward_impl(x, offsets, mask_or_null, weight, grad_out, grad_x_or_null, grad_offsets_or_null,
                         grad_mask_or_null, grad_weight_or_null, grad_bias_or_null, stride, padding, dilation, groups,
                         offset_groups, workspace, workspace_bytes, stream, 1);
}

}  // extern "C"

namespace {

// The packed layer's call: the forward's parameters (offsets and mask point
// at the generated tensors once the workspace is known), the trunk, the two
// heads and the workspace layout.
struct Packed {
    Params fwd;
    TrunkArgs trunk;
    const float *ow, *ob, *mw, *mb;
    int G, K;
    bool given_off, given_mask;
    size_t t_bytes, off_bytes, mask_bytes, cat_bytes, shared_bytes, total;
    // bf16 storage: fp32 copies of the generator's parameters and the bf16
    // offsets / mask the forward reads (conv_bytes of the workspace)
    int dtype;
    size_t conv_bytes;
};

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// The heads' GEMM: rows g*K + k (the offset head; with a mask, the mask
// head's rows follow, M = 2*G*K), reduction over the C_in trunk channels,
// columns (b, l); stored offsets-shaped by the head epilogue.
Params head_gemm(const Packed &pk, const float *hw, const float *hb, void *off, void *mask, void *ws) {
    Params q = {};
    q.dtype = kF32;
    q.w = hw;
    q.x = pk.trunk.t;  // B(k = c, n = (b, l)) = t[b][c][l]
    q.out = off;
    q.mask = mask;
    q.bias = hb;
    q.B = pk.fwd.B;
    q.C_out = pk.G * pk.K * (pk.mw ? 2 : 1);
    q.Kred = pk.fwd.C_in;
    q.L_out = pk.fwd.L_out;
    q.K = pk.K;
    q.G = pk.G;
    q.ws = ws;
    return q;
}

int validate_packed(const dc1d_tensor *x, const dc1d_tensor *tw, const dc1d_tensor *tb, const dc1d_tensor *ow,
                    const dc1d_tensor *ob, const dc1d_tensor *mw, const dc1d_tensor *mb, const dc1d_tensor *w,
                    const dc1d_tensor *bias, const dc1d_tensor *out, const dc1d_tensor *off_out,
                    const dc1d_tensor *mask_out, int64_t stride, int64_t padding, int64_t dilation,
                    int64_t groups, Packed *pk) {
    if (!x || !tw || !ow || !w) return DC1D_ERR_NULL_PTR;
    if (stride < 1 || padding < 0 || dilation < 1 || groups < 1) return DC1D_ERR_BAD_ARG;
    if (!mw && (mb || mask_out)) return DC1D_ERR_BAD_ARG;
    const dc1d_tensor *all[12] = {x, tw, tb, ow, ob, mw, mb, w, bias, out, off_out, mask_out};
    if (x->dtype != DC1D_F32 && x->dtype != DC1D_BF16) return DC1D_ERR_BAD_DTYPE;
    for (const dc1d_tensor *t : all)
        if (t && t->dtype != x->dtype) return DC1D_ERR_BAD_DTYPE;
    if (x->ndim != 3 || tw->ndim != 3 || ow->ndim != 3) return DC1D_ERR_BAD_SHAPE;
    const int64_t B = x->shape[0], C_in = x->shape[1], L_in = x->shape[2], K = tw->shape[2];
    if (C_in < 1 || K < 1 || tw->shape[0] != C_in || tw->shape[1] != 1) return DC1D_ERR_BAD_SHAPE;
    if (ow->shape[0] < 1 || ow->shape[0] % K || ow->shape[1] != C_in || ow->shape[2] != 1) return DC1D_ERR_BAD_SHAPE;
    const int64_t G = ow->shape[0] / K;
    if (C_in % G) return DC1D_ERR_BAD_ARG;
    if (mw && !shape_is(mw, 3, ow->shape)) return DC1D_ERR_BAD_SHAPE;
    const int64_t sc[1] = {C_in}, sh[1] = {G * K};
    if (tb && !shape_is(tb, 1, sc)) return DC1D_ERR_BAD_SHAPE;
    if ((ob && !shape_is(ob, 1, sh)) || (mb && !shape_is(mb, 1, sh))) return DC1D_ERR_BAD_SHAPE;
    const int64_t L_out = dc1d_output_length(L_in, K, stride, padding, dilation);
    if (L_out < 1) return DC1D_ERR_BAD_SHAPE;
    dc1d_tensor offT = {nullptr, x->dtype, 4, {B, G, L_out, K}};
    int st = validate(x, &offT, mw ? &offT : nullptr, w, bias, out, stride, padding, dilation, groups, G,
                      &pk->fwd);
    if (st) return st;
    if (off_out && !shape_is(off_out, 4, offT.shape)) return DC1D_ERR_BAD_SHAPE;
    if (mask_out && !shape_is(mask_out, 4, offT.shape)) return DC1D_ERR_BAD_SHAPE;
    if (B * L_out >= ((int64_t)1 << 31)) return DC1D_ERR_BAD_SHAPE;
    // the trunk [B, C_in, L_out] stays countable (B*L_out < 2^31, C_in <= 2^30)
    if (C_in * (B * L_out) > kMaxElems) return DC1D_ERR_BAD_SHAPE;
    const dc1d_tensor *ps[6] = {tw, tb, ow, ob, mw, mb};
    for (const dc1d_tensor *t : ps)
        if (t && numel_checked(t) < 0) return DC1D_ERR_BAD_SHAPE;
    pk->G = (int)G;
    pk->K = (int)K;
    pk->ow = (const float *)ow->data;
    pk->ob = ob ? (const float *)ob->data : nullptr;
    pk->mw = mw ? (const float *)mw->data : nullptr;
    pk->mb = mb ? (const float *)mb->data : nullptr;
    pk->given_off = off_out != nullptr;
    pk->given_mask = mask_out != nullptr;
    TrunkArgs &t = pk->trunk;
    t = TrunkArgs{};
    t.x = x->data;
    t.tw = (const float *)tw->data;
    t.tb = tb ? (const float *)tb->data : nullptr;
    t.dtype = kF32;
    t.B = (int)B;
    t.C = (int)C_in;
    t.L_in = (int)L_in;
    t.L_out = (int)L_out;
    t.K = (int)K;
    t.stride = (int)stride;
    t.padding = (int)padding;
    t.dilation = (int)dilation;
    // workspace: trunk | offsets | mask | stacked head weights and biases
    // (with a mask) | max(head GEMM partials, the forward's workspace)
    const size_t n_off = (size_t)B * G * L_out * K * 4;
    pk->t_bytes = round256((size_t)B * C_in * L_out * 4);
    pk->off_bytes = round256(n_off);
    pk->mask_bytes = mw ? round256(n_off) : 0;
    pk->cat_bytes = mw ? round256((size_t)2 * G * K * C_in * 4) + round256((size_t)2 * G * K * 4) : 0;
    pk->dtype = x->dtype;
    pk->conv_bytes = 0;
    if (x->dtype == DC1D_BF16) {
        // fp32 copies of trunk_weight, trunk_bias, off_weight, off_bias (and
        // the mask head's), then the offsets (and mask) in bf16
        const size_t gk = (size_t)G * K, heads = mw ? 2 : 1;
        pk->conv_bytes = round256((size_t)C_in * K * 4) + round256((size_t)C_in * 4) +
                         heads * (round256(gk * C_in * 4) + round256(gk * 4)) +
                         (mw ? 2 : 1) * round256((size_t)B * G * L_out * K * 2);
    }
    pk->shared_bytes = pk->total = 0;
    return DC1D_OK;
}

// The part of the workspace that depends on the device (the head GEMM's and
// the forward's plans); after validate_packed.
void size_packed(const DeviceInfo &dev, Packed *pk) {
    const size_t gemm =
        gemm_workspace_bytes(head_gemm(*pk, nullptr, nullptr, nullptr, nullptr, nullptr), 1, dev.num_cus);
    const size_t fwd = make_plan(pk->fwd, dev).ws_bytes;
    pk->shared_bytes = round256(gemm > fwd ? gemm : fwd);
    pk->total = pk->t_bytes + pk->off_bytes + pk->mask_bytes + pk->cat_bytes + pk->conv_bytes + pk->shared_bytes;
}

}  // namespace

extern "C" {

int dc1d_packed_workspace_bytes(const dc1d_tensor *x, const dc1d_tensor *trunk_weight,
                                const dc1d_tensor *off_weight, const dc1d_tensor *mask_weight_or_null,
                                const dc1d_tensor *weight, int64_t stride, int64_t padding, int64_t dilation,
                                int64_t groups, size_t *bytes_out) {
    if (!bytes_out) return DC1D_ERR_NULL_PTR;
    Packed pk;
    int st = validate_packed(x, trunk_weight, nullptr, off_weight, nullptr, mask_weight_or_null, nullptr, weight,
                             nullptr, nullptr, nullptr, nullptr, stride, padding, dilation, groups, &pk);
    if (st) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev))) return st;
    size_packed(dev, &pk);
    *bytes_out = pk.total;
    return DC1D_OK;
}

}  // extern "C"

namespace {

int packed_forward_impl(const dc1d_tensor *x, const dc1d_tensor *trunk_weight,
                        const dc1d_tensor *trunk_bias_or_null, const dc1d_tensor *off_weight,
                        const dc1d_tensor *off_bias_or_null, const dc1d_tensor *mask_weight_or_null,
                        const dc1d_tensor *mask_bias_or_null, const dc1d_tensor *weight,
                        const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                        const dc1d_tensor *offsets_out_or_null, const dc1d_tensor *mask_out_or_null,
                        int64_t stride, int64_t padding, int64_t dilation, int64_t groups, void *workspace,
                        size_t workspace_bytes, void *stream, int constrained) {
    if (!out) return DC1D_ERR_NULL_PTR;
    Packed pk;
    int st = validate_packed(x, trunk_weight, trunk_bias_or_null, off_weight, off_bias_or_null,
                             mask_weight_or_null, mask_bias_or_null, weight, bias_or_null, out, offsets_out_or_null,
                             mask_out_or_null, stride, padding, dilation, groups, &pk);
    if (st) return st;
    // the forward's taps clamped to their windows; the generated offsets
    // (and the offsets output) are the heads' own
    if (constrained && !constrained_ok(pk.fwd)) return DC1D_ERR_BAD_ARG;
    pk.fwd.constrained = constrained;
    const dc1d_tensor *ins[9] = {x, trunk_weight, trunk_bias_or_null, off_weight, off_bias_or_null,
                                 mask_weight_or_null, mask_bias_or_null, weight, bias_or_null};
    const dc1d_tensor *outs[3] = {out, offsets_out_or_null, mask_out_or_null};
    for (const dc1d_tensor *t : ins)
        if (t && numel(t) > 0 && !t->data) return DC1D_ERR_NULL_PTR;
    for (const dc1d_tensor *t : outs)
        if (t && numel(t) > 0 && !t->data) return DC1D_ERR_NULL_PTR;
    const size_t es = elem_size(pk.dtype);
    for (int i = 0; i < 3; ++i) {
        const dc1d_tensor *o = outs[i];
        if (!o) continue;
        const size_t ob = (size_t)numel(o) * es;
        for (const dc1d_tensor *t : ins)
            if (t && overlaps(o->data, ob, t->data, (size_t)numel(t) * es)) return DC1D_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (outs[j] && overlaps(o->data, ob, outs[j]->data, (size_t)numel(outs[j]) * es)) return DC1D_ERR_ALIAS;
    }
    DeviceInfo dev;
    if ((st = current_device(&dev))) return st;
    size_packed(dev, &pk);
    if (pk.total > 0) {
        if (!workspace || workspace_bytes < pk.total || ((uintptr_t)workspace & 255)) return DC1D_ERR_WORKSPACE;
        for (const dc1d_tensor *t : ins)
            if (t && overlaps(workspace, pk.total, t->data, (size_t)numel(t) * es)) return DC1D_ERR_ALIAS;
        for (const dc1d_tensor *t : outs)
            if (t && overlaps(workspace, pk.total, t->data, (size_t)numel(t) * es)) return DC1D_ERR_ALIAS;
    }
    if (log_on())
        fprintf(stderr, "dc1d: %s B=%d C_in=%d C_out=%d L_in=%d L_out=%d K=%d s=%d p=%d d=%d groups=%d G=%d mask=%d "
                        "%s -> trunk, heads GEMM, %s ws=%zu\n",
                constrained ? "packed_forward_constrained" : "packed_forward", pk.fwd.B, pk.fwd.C_in, pk.fwd.C_out,
                pk.fwd.L_in, pk.fwd.L_out, pk.K, pk.fwd.stride, pk.fwd.padding, pk.fwd.dilation, pk.fwd.groups,
                pk.G, pk.mw != nullptr, pk.dtype == DC1D_F32 ? "f32" : "bf16", make_plan(pk.fwd, dev).name,
                pk.total);
    if (pk.fwd.B == 0) return DC1D_OK;

    char *ws = (char *)workspace;
    float *t = (float *)ws;
    const bool bf16 = pk.dtype == DC1D_BF16;
    // the heads write fp32: straight into the caller's buffers for fp32
    // storage, into the workspace for bf16 (rounded into the bf16 tensors
    // the forward reads afterwards)
    void *off = (pk.given_off && !bf16) ? offsets_out_or_null->data : (void *)(ws + pk.t_bytes);
    void *mask = pk.mw ? ((pk.given_mask && !bf16) ? mask_out_or_null->data
                                                   : (void *)(ws + pk.t_bytes + pk.off_bytes))
                       : nullptr;
    char *cat = ws + pk.t_bytes + pk.off_bytes + pk.mask_bytes;
    char *conv = cat + pk.cat_bytes;
    void *shared = conv + pk.conv_bytes;
    hipStream_t s = (hipStream_t)stream;
    pk.trunk.t = t;
    pk.trunk.dtype = pk.dtype;
    const int GK = pk.G * pk.K;
    void *off16 = nullptr, *mask16 = nullptr;
    if (bf16) {
        // the generator's parameters widened to fp32 (exact)
        const int64_t C = pk.fwd.C_in;
        char *c = conv;
        hipError_t e = hipSuccess;
        auto widen = [&](const float *&dst_ptr, const void *src, int64_t n) {
            float *dst = (float *)c;
            c += round256((size_t)n * 4);
            if (!src) return;
            if (e == hipSuccess) e = launch_convert(src, kBF16, dst, kF32, n, s);
            dst_ptr = dst;
        };
        widen(pk.trunk.tw, trunk_weight->data, C * pk.K);
        widen(pk.trunk.tb, trunk_bias_or_null ? trunk_bias_or_null->data : nullptr, C);
        widen(pk.ow, off_weight->data, (int64_t)GK * C);
        widen(pk.ob, off_bias_or_null ? off_bias_or_null->data : nullptr, GK);
        if (pk.mw) {
            widen(pk.mw, mask_weight_or_null->data, (int64_t)GK * C);
            widen(pk.mb, mask_bias_or_null ? mask_bias_or_null->data : nullptr, GK);
        }
        const size_t n16 = round256((size_t)pk.fwd.B * GK * pk.fwd.L_out * 2);
        off16 = pk.given_off ? offsets_out_or_null->data : (void *)c;
        c += n16;
        if (pk.mw) mask16 = pk.given_mask ? mask_out_or_null->data : (void *)c;
        if (e != hipSuccess) return DC1D_ERR_LAUNCH;
    }
    // with a mask: one GEMM for both heads, their weights and biases stacked
    // by the trunk's launch
    float *wcat = pk.mw ? (float *)cat : nullptr;
    float *bcat = pk.mw ? (float *)(cat + round256((size_t)2 * GK * pk.fwd.C_in * 4)) : nullptr;
    pk.trunk.ow = pk.ow;
    pk.trunk.ob = pk.ob;
    pk.trunk.mw = pk.mw;
    pk.trunk.mb = pk.mb;
    pk.trunk.wcat = wcat;
    pk.trunk.bcat = bcat;
    pk.trunk.GK = GK;
    const int64_t brow = pk.fwd.L_out, bbatch = (int64_t)pk.fwd.C_in * pk.fwd.L_out;
    const int M = GK * (pk.mw ? 2 : 1);
    // fp32 storage: the persistent head kernel computes the trunk itself
    // (no trunk launch, no stacked head weights); bf16: the trunk kernel
    // first, then the head kernel reads it
    const bool fused = !bf16 && heads_fit(pk.fwd.C_in, pk.K, M, pk.fwd.L_out, nullptr, off, mask);
    hipError_t e = hipSuccess;
    if (!fused) {
        e = launch_trunk(pk.trunk, s);
        if (e != hipSuccess) return DC1D_ERR_LAUNCH;
    }
    if (fused || heads_fit(pk.fwd.C_in, pk.K, M, pk.fwd.L_out, t, off, mask)) {  // the persistent head kernel
        HeadArgs h = {};
        h.t = t;
        h.w = pk.mw && !fused ? wcat : pk.ow;
        h.bias = pk.mw && !fused ? bcat : pk.ob;
        h.off = (float *)off;
        h.mask = (float *)mask;
        h.B = pk.fwd.B;
        h.C = pk.fwd.C_in;
        h.L = pk.fwd.L_out;
        h.G = pk.G;
        h.K = pk.K;
        h.M = M;
        if (fused) {
            h.x = (const float *)x->data;
            h.tw = pk.trunk.tw;
            h.tb = pk.trunk.tb;
            h.w2 = pk.mw;
            h.bias2 = pk.mb;
            h.L_in = pk.fwd.L_in;
            h.stride = pk.fwd.stride;
            h.padding = pk.fwd.padding;
            h.dilation = pk.fwd.dilation;
        }
        e = launch_heads(h, dev.num_cus, s);
    } else if (pk.mw) {
        e = launch_gemm_f32(head_gemm(pk, wcat, bcat, off, mask, shared), brow, bbatch, 2, dev.num_cus, s);
    } else {
        e = launch_gemm_f32(head_gemm(pk, pk.ow, pk.ob, off, nullptr, shared), brow, bbatch, 1, dev.num_cus, s);
    }
    if (e != hipSuccess) return DC1D_ERR_LAUNCH;
    if (bf16) {  // the generated offsets (and mask) rounded once into bf16 for the bf16 forward
        const int64_t n = (int64_t)pk.fwd.B * GK * pk.fwd.L_out;
        e = launch_convert(off, kF32, off16, kBF16, n, s);
        if (e == hipSuccess && pk.mw) e = launch_convert(mask, kF32, mask16, kBF16, n, s);
        if (e != hipSuccess) return DC1D_ERR_LAUNCH;
        off = off16;
        mask = mask16;
    }
    Params p = pk.fwd;
    p.off = off;
    p.mask = mask;
    p.ws = shared;
    p.ws_bytes = pk.shared_bytes;
    const Plan pl = make_plan(p, dev);
    switch (pl.kernel) {
    case kMfma: e = launch_mfma(p, pl.mfma, s); break;
    case kDepthwise: e = launch_depthwise(p, pl.dw, s); break;
    default: e = launch_direct(p, s); break;
    }
    return e == hipSuccess ? DC1D_OK : DC1D_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int dc1d_packed_forward(const dc1d_tensor *x, const dc1d_tensor *trunk_weight,
                        const dc1d_tensor *trunk_bias_or_null, const dc1d_tensor *off_weight,
                        const dc1d_tensor *off_bias_or_null, const dc1d_tensor *mask_weight_or_null,
                        const dc1d_tensor *mask_bias_or_null, const dc1d_tensor *weight,
                        const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                        const dc1d_tensor *offsets_out_or_null, const dc1d_tensor *mask_out_or_null,
                        int64_t stride, int64_t padding, int64_t dilation, int64_t groups, void *workspace,
                        size_t workspace_bytes, void *stream) {
    return packed_forward_impl(x, trunk_weight, trunk_bias_or_null, off_weight, off_bias_or_null,
                               mask_weight_or_null, mask_bias_or_null, weight, bias_or_null, out,
                               offsets_out_or_null, mask_out_or_null, stride, padding, dilation, groups, workspace,
                               workspace_bytes, stream, 0);
}

int dc1d_packed_forward_constrained(const dc1d_tensor *x, const dc1d_tensor *trunk_weight,
                                    const dc1d_tensor *trunk_bias_or_null, const dc1d_tensor *off_weight,
                                    const dc1d_tensor *off_bias_or_null, const dc1d_tensor *mask_weight_or_null,
                                    const dc1d_tensor *mask_bias_or_null, const dc1d_tensor *weight,
                                    const dc1d_tensor *bias_or_null, const dc1d_tensor *out,
                                    const dc1d_tensor *offsets_out_or_null, const dc1d_tensor *mask_out_or_null,
                                    int64_t stride, int64_t padding, int64_t dilation, int64_t groups,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    return packed_forward_impl(x, trunk_weight, trunk_bias_or_null, off_weight, off_bias_or_null,
                               mask_weight_or_null, mask_bias_or_null, weight, bias_or_null, out,
                               offsets_out_or_null, mask_out_or_null, stride, padding, dilation, groups, workspace,
                               workspace_bytes, stream, 1);
}

}  // extern "C"

namespace {

int validate2d(const dc1d_tensor *x, const dc1d_tensor *off, const dc1d_tensor *mask, const dc1d_tensor *w,
               const dc1d_tensor *bias, const dc1d_tensor *out, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
               int64_t dh, int64_t dw, int64_t groups, int64_t offset_groups, Params2 *p) {
    if (!x || !off || !w) return DC1D_ERR_NULL_PTR;
    if (sh < 1 || sw < 1 || ph < 0 || pw < 0 || dh < 1 || dw < 1 || groups < 1 || offset_groups < 1)
        return DC1D_ERR_BAD_ARG;
    if (x->ndim != 4 || w->ndim != 4 || off->ndim != 4) return DC1D_ERR_BAD_SHAPE;
    const int dt = x->dtype;
    if (dt != DC1D_F32 && dt != DC1D_BF16) return DC1D_ERR_BAD_DTYPE;
    if (off->dtype != dt || w->dtype != dt || (mask && mask->dtype != dt) || (bias && bias->dtype != dt) ||
        (out && out->dtype != dt))
        return DC1D_ERR_BAD_DTYPE;
    const int64_t B = x->shape[0], C_in = x->shape[1], H = x->shape[2], W = x->shape[3];
    const int64_t C_out = w->shape[0], kh = w->shape[2], kw = w->shape[3];
    // an empty image has nothing to sample; the samplers assume H, W >= 1
    if (B < 0 || C_in < 1 || H < 1 || W < 1 || C_out < 1 || kh < 1 || kw < 1) return DC1D_ERR_BAD_SHAPE;
    // every size bounded on its own before any product of two is formed
    const int64_t lim30 = (int64_t)1 << 30;
    if (H > kMaxPos || W > kMaxPos || ph > kMaxPos || pw > kMaxPos || kh > kMaxPos || kw > kMaxPos ||
        dh > kMaxPos || dw > kMaxPos || sh > lim30 || sw > lim30 || C_in > lim30 || C_out > lim30 || B > 65535 ||
        offset_groups > ((int64_t)1 << 24))
        return DC1D_ERR_BAD_SHAPE;
    if (C_in % groups || C_out % groups || C_in % offset_groups) return DC1D_ERR_BAD_ARG;
    if (w->shape[1] != C_in / groups) return DC1D_ERR_BAD_SHAPE;
    if (kh * kw > lim30) return DC1D_ERR_BAD_SHAPE;
    const int64_t T = kh * kw;
    if (H + ph > kMaxPos || W + pw > kMaxPos || dh * (kh - 1) > kMaxPos || dw * (kw - 1) > kMaxPos ||
        H * W >= ((int64_t)1 << 31) || C_in / groups * T > lim30 || offset_groups * T > ((int64_t)1 << 24))
        return DC1D_ERR_BAD_SHAPE;
    const int64_t Ho = dc1d_output_length(H, kh, sh, ph, dh), Wo = dc1d_output_length(W, kw, sw, pw, dw);
    if (Ho < 1 || Wo < 1 || Ho * sh > lim30 || Wo * sw > lim30 || Ho * Wo >= ((int64_t)1 << 31) ||
        B * Ho * Wo >= ((int64_t)1 << 31))
        return DC1D_ERR_BAD_SHAPE;
    const dc1d_tensor *ts[6] = {x, off, mask, w, bias, out};
    for (const dc1d_tensor *t : ts)
        if (t && numel_checked(t) < 0) return DC1D_ERR_BAD_SHAPE;
    const int64_t so[4] = {B, 2 * offset_groups * T, Ho, Wo};
    if (!shape_is(off, 4, so)) return DC1D_ERR_BAD_SHAPE;
    const int64_t sm[4] = {B, offset_groups * T, Ho, Wo};
    if (mask && !shape_is(mask, 4, sm)) return DC1D_ERR_BAD_SHAPE;
    const int64_t sb[1] = {C_out};
    if (bias && !shape_is(bias, 1, sb)) return DC1D_ERR_BAD_SHAPE;
    const int64_t sout[4] = {B, C_out, Ho, Wo};
    if (out && !shape_is(out, 4, sout)) return DC1D_ERR_BAD_SHAPE;
    memset(p, 0, sizeof(*p));
    p->x = x->data;
    p->off = off->data;
    p->mask = mask ? mask->data : nullptr;
    p->w = w->data;
    p->bias = bias ? bias->data : nullptr;
    p->out = out ? out->data : nullptr;
    p->dtype = dt;
    p->B = (int)B;
    p->C_in = (int)C_in;
    p->C_out = (int)C_out;
    p->H = (int)H;
    p->W = (int)W;
    p->Ho = (int)Ho;
    p->Wo = (int)Wo;
    p->kh = (int)kh;
    p->kw = (int)kw;
    p->sh = (int)sh;
    p->sw = (int)sw;
    p->ph = (int)ph;
    p->pw = (int)pw;
    p->dh = (int)dh;
    p->dw = (int)dw;
    p->groups = (int)groups;
    p->G = (int)offset_groups;
    p->cpg = (int)(C_in / groups);
    p->opg = (int)(C_out / groups);
    p->cpo = (int)(C_in / offset_groups);
    p->T = (int)T;
    p->Kred = (int)(C_in / groups * T);
    return DC1D_OK;
}

}  // namespace

extern "C" {

int dc2d_workspace_bytes(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                         const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, int64_t stride_h,
                         int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w,
                         int64_t groups, int64_t offset_groups, size_t *bytes_out) {
    if (!bytes_out) return DC1D_ERR_NULL_PTR;
    Params2 p;
    int st = validate2d(x, offsets, mask_or_null, weight, bias_or_null, nullptr, stride_h, stride_w, pad_h, pad_w,
                        dil_h, dil_w, groups, offset_groups, &p);
    if (st) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev))) return st;
    *bytes_out = dc2d_workspace(p, dev.num_cus);
    return DC1D_OK;
}

int dc2d_plan(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
              const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, int64_t stride_h, int64_t stride_w,
              int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w, int64_t groups, int64_t offset_groups,
              const char **kernel_name) {
    Params2 p;
    int st = validate2d(x, offsets, mask_or_null, weight, bias_or_null, nullptr, stride_h, stride_w, pad_h, pad_w,
                        dil_h, dil_w, groups, offset_groups, &p);
    if (st) return st;
    if (kernel_name) *kernel_name = dc2d_kernel_name(p);
    return DC1D_OK;
}

int dc2d_forward(const dc1d_tensor *x, const dc1d_tensor *offsets, const dc1d_tensor *mask_or_null,
                 const dc1d_tensor *weight, const dc1d_tensor *bias_or_null, const dc1d_tensor *out, int64_t stride_h,
                 int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w, int64_t groups,
                 int64_t offset_groups, void *workspace, size_t workspace_bytes, void *stream) {
    if (!out) return DC1D_ERR_NULL_PTR;
    Params2 p;
    int st = validate2d(x, offsets, mask_or_null, weight, bias_or_null, out, stride_h, stride_w, pad_h, pad_w, dil_h,
                        dil_w, groups, offset_groups, &p);
    if (st) return st;
    const dc1d_tensor *all[6] = {x, offsets, mask_or_null, weight, bias_or_null, out};
    for (const dc1d_tensor *t : all)
        if (t && numel(t) > 0 && !t->data) return DC1D_ERR_NULL_PTR;
    const size_t es = elem_size(p.dtype);
    const size_t out_bytes = (size_t)numel(out) * es;
    for (int i = 0; i < 5; ++i)
        if (all[i] && overlaps(out->data, out_bytes, all[i]->data, (size_t)numel(all[i]) * es)) return DC1D_ERR_ALIAS;
    DeviceInfo dev;
    if ((st = current_device(&dev))) return st;
    const size_t need = dc2d_workspace(p, dev.num_cus);
    if (need > 0 && p.B > 0) {
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255)) return DC1D_ERR_WORKSPACE;
        for (int i = 0; i < 6; ++i)
            if (all[i] && overlaps(workspace, need, all[i]->data, (size_t)numel(all[i]) * es)) return DC1D_ERR_ALIAS;
    }
    if (log_on())
        fprintf(stderr, "dc1d: dc2d_forward B=%d C_in=%d C_out=%d %dx%d -> %dx%d k=%dx%d groups=%d G=%d mask=%d %s "
                        "-> %s ws=%zu\n",
                p.B, p.C_in, p.C_out, p.H, p.W, p.Ho, p.Wo, p.kh, p.kw, p.groups, p.G, p.mask != nullptr,
                p.dtype == DC1D_F32 ? "f32" : "bf16", dc2d_kernel_name(p), need);
    p.ws = workspace;
    p.ws_bytes = workspace_bytes;
    const hipError_t e = launch_dc2d(p, dev.num_cus, (hipStream_t)stream);
    return e == hipSuccess ? DC1D_OK : DC1D_ERR_LAUNCH;
}

int dc1d_debug_positions(const dc1d_tensor *offsets, int64_t L_in, int64_t stride, int64_t padding,
                         int64_t dilation, int32_t *i0, float *frac, uint8_t *valid, void *stream) {
    if (!offsets) return DC1D_ERR_NULL_PTR;
    if (stride < 1 || padding < 0 || dilation < 1 || L_in < 0) return DC1D_ERR_BAD_ARG;
    if (offsets->ndim != 4) return DC1D_ERR_BAD_SHAPE;
    if (offsets->dtype != DC1D_F32 && offsets->dtype != DC1D_BF16) return DC1D_ERR_BAD_DTYPE;
    const int64_t K = offsets->shape[3];
    if (K < 1 || K > kMaxPos || L_in > kMaxPos || padding > kMaxPos || dilation > kMaxPos ||
        L_in + padding > kMaxPos || dilation * (K - 1) > kMaxPos)
        return DC1D_ERR_BAD_SHAPE;
    const int64_t L_out = dc1d_output_length(L_in, K, stride, padding, dilation);
    if (L_out < 1 || L_out * (stride > kMaxPos ? kMaxPos : stride) > ((int64_t)1 << 30) ||
        offsets->shape[2] != L_out || offsets->shape[0] < 0 || offsets->shape[1] < 1)
        return DC1D_ERR_BAD_SHAPE;
    const int64_t n = numel_checked(offsets);
    if (n < 0 || n >= ((int64_t)1 << 40)) return DC1D_ERR_BAD_SHAPE;
    if (n > 0 && (!offsets->data || !i0 || !frac || !valid)) return DC1D_ERR_NULL_PTR;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st) return st;
    hipError_t e = launch_positions(offsets->data, offsets->dtype, n, (int)L_out, (int)K, (int)stride,
                                    (int)padding, (int)dilation, (int)L_in, i0, frac, valid,
                                    (hipStream_t)stream);
    return e == hipSuccess ? DC1D_OK : DC1D_ERR_LAUNCH;
}

const char *dc1d_status_string(int status) {
    switch (status) {
    case DC1D_OK: return "ok";
    case DC1D_ERR_NULL_PTR: return "a required pointer is NULL";
    case DC1D_ERR_BAD_ARG: return "argument out of range or inconsistent (stride, padding, dilation, groups, offset_groups, K)";
    case DC1D_ERR_BAD_SHAPE: return "tensor rank or shape disagrees, L_out <= 0, or size beyond the supported limits";
    case DC1D_ERR_BAD_DTYPE: return "unsupported or mixed dtypes";
    case DC1D_ERR_ALIAS: return "output or workspace overlaps another buffer";
    case DC1D_ERR_WORKSPACE: return "workspace missing or too small";
    case DC1D_ERR_DEVICE: return "no current HIP device, or it is not a gfx950";
    case DC1D_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

}  // extern "C"
