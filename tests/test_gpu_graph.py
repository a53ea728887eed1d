"""The layer captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library never allocates, synchronises or clears memory with a memset, so
a whole layer step can be captured once and replayed.  Each test replays
several times with new input values copied into the captured buffers, runs
the same step eagerly on a second set of buffers between replays, and checks
every replay bit-exactly against that eager run (all kernels are
deterministic).  The backward's tile queues must be left zero-filled by every
replay, since nothing else clears them.
"""
import pytest
import torch

import grouped_gemm_moe_amd as moe
import workloads
from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayer
from tests.gpu_util import bf16_dev, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _same_bits(a, b, what, i):
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"replay {i}: {what} differs"


def test_decode_forward_graph_replays(dev):
    wl = workloads.decode()
    d = wl.dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    print(f"graph: decode forward {shape}", flush=True)
    w1, w2 = bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    probs = torch.from_numpy(wl["probs"]).to(dev)
    x = bf16_dev(wl["x"], dev)
    layer, ref = MoeLayer(shape, dev), MoeLayer(shape, dev)
    g = _capture(lambda: layer.forward(x, ids, probs, w1, w2, fused="auto", keep_h=False))
    gen = torch.Generator(device=dev).manual_seed(11)
    for i in range(4):
        x_i = torch.randn(x.shape, generator=gen, device=dev).to(torch.bfloat16)
        x.copy_(x_i)
        g.replay()
        ref.forward(x_i, ids, probs, w1, w2, fused="auto", keep_h=False)
        torch.cuda.synchronize()
        _same_bits(layer.out, ref.out, "out", i)
        _same_bits(layer.tokens_per_expert, ref.tokens_per_expert, "tokens_per_expert", i)
    assert int(layer.dev_err.item()) == 0


def test_routed_decode_forward_graph_replays(dev):
    """moe_decode_fwd (routing inside the gate_up GMM) captured and replayed
    with new token rows and a new routing each time: every output, the maps
    included, bit-identical to the same call run eagerly."""
    wl = workloads.decode()
    d = wl.dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    print(f"graph: routed decode forward {shape}", flush=True)
    w1, w2 = bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    probs = torch.from_numpy(wl["probs"]).to(dev)
    x = bf16_dev(wl["x"], dev)
    layer = MoeLayer(shape, dev, gather_rows=True)
    ref = MoeLayer(shape, dev, gather_rows=True)
    g = _capture(lambda: layer.forward_decode(x, ids, probs, w1, w2))
    gen = torch.Generator(device=dev).manual_seed(12)
    for i in range(4):
        x_i = torch.randn(x.shape, generator=gen, device=dev).to(torch.bfloat16)
        ids_i = torch.stack([torch.randperm(d["E"], generator=gen, device=dev)[: d["K"]] for _ in range(d["T"])])
        ids_i = ids_i.to(torch.int32)
        x.copy_(x_i)
        ids.copy_(ids_i)
        g.replay()
        ref.forward_decode(x_i, ids_i, probs, w1, w2)
        torch.cuda.synchronize()
        R = int(ref.tokens_per_expert.sum().item())
        for name in ("out", "row_id_map", "tokens_per_expert"):
            _same_bits(getattr(layer, name), getattr(ref, name), name, i)
        for name in ("sorted_slot", "h", "a", "yp"):
            _same_bits(getattr(layer, name)[:R], getattr(ref, name)[:R], name, i)
    assert int(layer.dev_err.item()) == 0


@pytest.mark.parametrize("fuse_swiglu_bwd", [True, False])
def test_layer_forward_backward_graph_replays(dev, fuse_swiglu_bwd):
    # several row tiles per expert, ragged tails and both backward pairs on the
    # persistent kernels (tile queues in the layer's workspace)
    wl = workloads.moe_layer("graph", 21, T=512, K=4, E=16, H=512, I=256)
    d = wl.dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    print(f"graph: forward + backward {shape} fuse_swiglu_bwd={fuse_swiglu_bwd}", flush=True)
    w1, w2 = bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    probs = torch.from_numpy(wl["probs"]).to(dev)
    x = bf16_dev(wl["x"], dev)
    dout = torch.zeros((d["T"], d["H"]), dtype=torch.bfloat16, device=dev)
    mk = lambda: MoeLayer(shape, dev, with_backward=True, fuse_swiglu_bwd=fuse_swiglu_bwd)  # noqa: E731
    layer, ref = mk(), mk()

    def step(L, xx, dd):
        L.forward(xx, ids, probs, w1, w2, fused=True, keep_h=True)
        L.backward_full(dd, probs, w1, w2)

    g = _capture(lambda: step(layer, x, dout))
    gen = torch.Generator(device=dev).manual_seed(12)
    for i in range(4):
        x_i = torch.randn(x.shape, generator=gen, device=dev).to(torch.bfloat16)
        d_i = torch.randn(dout.shape, generator=gen, device=dev).to(torch.bfloat16)
        x.copy_(x_i)
        dout.copy_(d_i)
        g.replay()
        step(ref, x_i, d_i)
        torch.cuda.synchronize()
        for name in ("out", "dx_tokens", "dprobs", "dw1", "dw2", "dh"):
            _same_bits(getattr(layer, name), getattr(ref, name), name, i)
        assert int(torch.count_nonzero(layer.ws_gmm[:moe.GMM_QUEUE_BYTES]).item()) == 0, f"replay {i}: tile queues not left zeroed"
    assert int(layer.dev_err.item()) == 0
