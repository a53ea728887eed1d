"""Two layer steps enqueued on two streams at once, each with its own buffers
and workspaces (calls that may overlap need distinct workspaces).

The persistent backward kernels size their grids to the CU count and take
tiles from a queue in the workspace, so two of them running together each get
only part of the GPU and late workgroups find an empty queue.  Results must
still be bit-identical to the same steps run one after another.
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


def test_two_streams_match_sequential(dev):
    wls = [workloads.moe_layer(f"streams{i}", 30 + i, T=1024, K=4, E=16, H=512, I=256) for i in range(2)]
    d = wls[0].dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    print(f"two streams: {shape}", flush=True)
    ins = []
    for i, wl in enumerate(wls):
        g = torch.Generator(device=dev).manual_seed(40 + i)
        ins.append(dict(x=bf16_dev(wl["x"], dev), ids=torch.from_numpy(wl["topk_ids"]).to(dev),
                        probs=torch.from_numpy(wl["probs"]).to(dev), w1=bf16_dev(wl["w1"], dev),
                        w2=bf16_dev(wl["w2"], dev),
                        dout=torch.randn((d["T"], d["H"]), generator=g, device=dev).to(torch.bfloat16)))

    def step(L, a):
        L.forward(a["x"], a["ids"], a["probs"], a["w1"], a["w2"], fused=True, keep_h=True)
        L.backward_full(a["dout"], a["probs"], a["w1"], a["w2"])

    seq = [MoeLayer(shape, dev, with_backward=True) for _ in range(2)]
    for L, a in zip(seq, ins):
        step(L, a)
    torch.cuda.synchronize()

    par = [MoeLayer(shape, dev, with_backward=True) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    main = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(main)
    for rep in range(3):
        for L, a, s in zip(par, ins, streams):
            with torch.cuda.stream(s):
                step(L, a)
        torch.cuda.synchronize()
        for k, (Lp, Ls) in enumerate(zip(par, seq)):
            for name in ("out", "dx_tokens", "dprobs", "dw1", "dw2"):
                a, b = getattr(Lp, name), getattr(Ls, name)
                if a.dtype == torch.bfloat16:
                    a, b = a.view(torch.int16), b.view(torch.int16)
                assert torch.equal(a, b), f"rep {rep}, layer {k}: {name} differs from the sequential run"
            assert int(torch.count_nonzero(Lp.ws_gmm[:moe.GMM_QUEUE_BYTES]).item()) == 0
            assert int(Lp.dev_err.item()) == 0


def test_routed_decode_on_two_streams_matches_sequential(dev):
    """moe_decode_fwd takes no workspace, so two calls may overlap on two
    streams with their own buffers; each must equal the same call run alone."""
    wls = [workloads.decode(), workloads.decode_skewed()]
    d = wls[0].dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    print(f"two streams: routed decode {shape}", flush=True)
    ins = [dict(x=bf16_dev(wl["x"], dev), ids=torch.from_numpy(wl["topk_ids"]).to(dev),
                probs=torch.from_numpy(wl["probs"]).to(dev), w1=bf16_dev(wl["w1"], dev),
                w2=bf16_dev(wl["w2"], dev)) for wl in wls]
    seq = [MoeLayer(shape, dev, gather_rows=True) for _ in range(2)]
    for L, a in zip(seq, ins):
        L.forward_decode(a["x"], a["ids"], a["probs"], a["w1"], a["w2"])
    torch.cuda.synchronize()
    par = [MoeLayer(shape, dev, gather_rows=True) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    main = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(main)
    for rep in range(3):
        for L, a, s in zip(par, ins, streams):
            with torch.cuda.stream(s):
                L.forward_decode(a["x"], a["ids"], a["probs"], a["w1"], a["w2"])
        torch.cuda.synchronize()
        for k, (Lp, Ls) in enumerate(zip(par, seq)):
            R = int(Ls.tokens_per_expert.sum().item())
            for name in ("out", "row_id_map", "tokens_per_expert", "sorted_slot", "yp"):
                a, b = getattr(Lp, name), getattr(Ls, name)
                if name in ("sorted_slot", "yp"):
                    a, b = a[:R], b[:R]
                if a.dtype == torch.bfloat16:
                    a, b = a.view(torch.int16), b.view(torch.int16)
                assert torch.equal(a, b), f"rep {rep}, layer {k}: {name} differs from the sequential run"
            assert int(Lp.dev_err.item()) == 0
