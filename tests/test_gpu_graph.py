"""HIP graph capture of the library's calls (the bench times graph replays).

Each call is captured once into a torch.cuda.CUDAGraph with its workspace
and outputs allocated beforehand, replayed several times with eager work
and synchronisations in between, and every replay is compared with the
eager result: bit for bit for the forward (deterministic, split sums in a
fixed order) and the packed layer, within the backward parity tolerance for
the backward (its atomics may reorder sums).
"""
import pytest
import torch

from deformable_convolution_amd import dc1d, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def capture(step):
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(DEV).wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def replays(g, eager, result, cmp, n=4):
    for i in range(n):
        junk = torch.randn(1 << 20, device=DEV) * 3.0  # eager work between replays
        junk.sum().item()
        g.replay()
        torch.cuda.synchronize()
        cmp(result(), eager, i)


@pytest.mark.parametrize("name", ["dc1d_layer", "depthwise", "long_seq_bf16", "dcnv2_bf16"])
def test_forward_graph_replays_match_eager(name):
    w = inputs.WORKLOADS[name].with_batch(1)
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_inputs(w, seed=11).items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    nws = dc1d.workspace_bytes(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], **kw)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV) if nws else None
    out = torch.empty((w.B, w.C_out, w.L_out), dtype=t["x"].dtype, device=DEV)

    def step():
        dc1d.forward(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], out=out, workspace=ws, **kw)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    out.fill_(float("nan"))
    g = capture(step)

    def cmp(a, b, i):
        assert torch.equal(a, b), "replay %d differs" % i

    replays(g, eager, lambda: out, cmp)


def test_packed_graph_replays_match_eager():
    w = inputs.PACKED_WORKLOADS["packed_page_modulated"]
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_packed_inputs(w, seed=12).items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    args = (t["x"], t["trunk_weight"], t["trunk_bias"], t["off_weight"], t["off_bias"], t["weight"], t["bias"],
            t["mask_weight"], t["mask_bias"])
    nws = dc1d.packed_workspace_bytes(t["x"], t["trunk_weight"], t["off_weight"], t["weight"], t["mask_weight"],
                                      **kw)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    out = torch.empty((w.B, w.C_out, w.L_out), device=DEV)

    def step():
        dc1d.packed_forward(*args, out=out, workspace=ws, **kw)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    out.zero_()
    g = capture(step)
    replays(g, eager, lambda: out, lambda a, b, i: torch.equal(a, b) or pytest.fail("replay %d differs" % i))


@pytest.mark.parametrize("name", ["dc1d_layer", "depthwise"])
def test_backward_graph_replays_match_eager(name):
    w = inputs.WORKLOADS[name].with_batch(1)
    if name == "depthwise":
        w = inputs.custom("depthwise[C=64]", B=1, C_in=64, C_out=64, L_in=4096, K=5, padding=2, dilation=2,
                          groups=64, G=64, L_out=4092, off_dist=("uniform", -4.0, 4.0), w_var=1 / 5)
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_inputs(w, seed=13).items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    dout = torch.randn((w.B, w.C_out, w.L_out), device=DEV)
    nws = dc1d.backward_workspace_bytes(t["x"], t["offsets"], t["weight"], dout, t["mask"], **kw)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV) if nws else None
    res = {}

    def step():
        res["g"] = dc1d.backward(t["x"], t["offsets"], t["weight"], dout, t["mask"], workspace=ws, **kw)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in res["g"].items()}
    g = capture(step)
    captured = res["g"]  # the graph's output tensors

    def cmp(a, b, i):
        for k in b:
            scale = float(b[k].abs().max()) + 1e-6
            assert torch.allclose(a[k], b[k], rtol=1e-5, atol=1e-5 * scale), "replay %d grad_%s" % (i, k)

    replays(g, eager, lambda: captured, cmp)
