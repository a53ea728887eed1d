"""The whole routed-expert layer on the GPU vs the oracle chain.

Forward: permute -> gate_up GMM -> SwiGLU -> down GMM -> weighted unpermute.
Backward of the expert block from dYp (the gradient at the down-GMM output,
in permuted order).  The GPU chain uses its own intermediates; the oracle
chain rounds to bf16 at the same boundary points.  Row-local results use the
plain tolerance; weight gradients, which sum a chained intermediate over many
rows, add the one-ulp propagation term of chained_reduction_slack().
Indices and counts must match bit-exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayer
from tests.gpu_util import (assert_close, bf16_dev, chained_reduction_slack, dev_bits, dev_f64, f64,
                            require_gpu)

pytestmark = pytest.mark.gpu

SENT = np.uint16(0x7FC1)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _run_forward(dev, wl, with_backward=False, dyp_bits=None, low_memory=False, fuse_swiglu_bwd=True):
    d = wl.dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    print(f"layer {wl.name}: {shape} low_memory={low_memory} fuse_swiglu_bwd={fuse_swiglu_bwd}", flush=True)
    layer = MoeLayer(shape, dev, with_backward=with_backward, low_memory=low_memory,
                     fuse_swiglu_bwd=fuse_swiglu_bwd)
    w1, w2 = bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev)
    layer.forward(bf16_dev(wl["x"], dev), torch.from_numpy(wl["topk_ids"]).to(dev),
                  torch.from_numpy(wl["probs"]).to(dev), w1, w2)
    if with_backward:
        layer.backward(bf16_dev(dyp_bits, dev), w1, w2)
    torch.cuda.synchronize()
    assert int(layer.dev_err.item()) == 0
    return layer


def _check_forward(layer, ref, R):
    np.testing.assert_array_equal(layer.tokens_per_expert.cpu().numpy(), ref["tokens_per_expert"])
    np.testing.assert_array_equal(layer.row_id_map.cpu().numpy(), ref["row_id_map"])
    np.testing.assert_array_equal(layer.sorted_slot.cpu().numpy()[:R], ref["sorted_slot"])
    np.testing.assert_array_equal(dev_f64(layer.x_perm)[:R], ref["x_perm"])
    assert_close(dev_f64(layer.h)[:R], ref["h"][:R], "h = gate_up GMM")
    assert_close(dev_f64(layer.a)[:R], ref["a"][:R], "a = SwiGLU")
    assert_close(dev_f64(layer.yp)[:R], ref["yp"][:R], "yp = down GMM")
    assert_close(dev_f64(layer.out), ref["out"], "out = weighted unpermute")


def _slack_per_expert(u, v, gl):
    off = oracle.expert_offsets(gl)
    return np.stack([chained_reduction_slack(u[off[e]:off[e + 1]], v[off[e]:off[e + 1]])
                     for e in range(len(gl))])


def _oracle_forward(wl):
    return oracle.moe_layer_forward(f64(wl["x"]), wl["topk_ids"], wl["probs"].astype(np.float64),
                                    f64(wl["w1"]), f64(wl["w2"]), wl.dims["E"])


@pytest.mark.parametrize("fuse_swiglu_bwd", [True, False])
def test_tiny_forward_backward(dev, fuse_swiglu_bwd):
    wl = workloads.tiny()
    R = 5
    S = wl.dims["T"] * wl.dims["K"]
    dyp = np.full((S, wl.dims["H"]), SENT, dtype=np.uint16)   # rows >= R undefined (NaN)
    dyp[:R] = wl["dyp"]
    layer = _run_forward(dev, wl, with_backward=True, dyp_bits=dyp, fuse_swiglu_bwd=fuse_swiglu_bwd)
    ref = _oracle_forward(wl)
    assert ref["tokens_per_expert"].tolist() == [1, 2, 0, 2]
    _check_forward(layer, ref, R)
    g = oracle.expert_block_backward(ref["x_perm"], ref["h"], ref["a"], f64(wl["dyp"]),
                                     f64(wl["w1"]), f64(wl["w2"]), ref["tokens_per_expert"],
                                     fused_swiglu_bwd=fuse_swiglu_bwd)
    if not fuse_swiglu_bwd:  # the fused backward never stores dA
        assert_close(dev_f64(layer.da)[:R], g["da"][:R], "dA")
    assert_close(dev_f64(layer.dh)[:R], g["dh"][:R], "dH")
    assert_close(dev_f64(layer.dx)[:R], g["dx"][:R], "dX")
    assert_close(dev_f64(layer.dw2), g["dw2"], "dW2", extra=_slack_per_expert(ref["a"], f64(wl["dyp"]), [1, 2, 0, 2]))
    assert_close(dev_f64(layer.dw1), g["dw1"], "dW1", extra=_slack_per_expert(ref["x_perm"], g["dh"], [1, 2, 0, 2]))
    assert (dev_bits(layer.dw1)[2] == 0).all() and (dev_bits(layer.dw2)[2] == 0).all()


@pytest.mark.parametrize("name", ["prefill", "decode", "decode_skewed"])
def test_layer_forward(dev, name):
    wl = getattr(workloads, name)()
    layer = _run_forward(dev, wl)
    ref = _oracle_forward(wl)
    _check_forward(layer, ref, int(ref["tokens_per_expert"].sum()))


@pytest.mark.parametrize("low_memory", [False, True])
def test_ep_rank_forward_backward_sampled(dev, low_memory):
    """Full-size expert-parallel share (E=32, H=4096, I=1536, 16384 rows, top_k=1
    after the local re-routing).  Row-local results are recomputed by the
    oracle for sampled rows; weight gradients for sampled weight rows of a few
    experts (the oracle then runs those experts' whole chains).  With
    low_memory the backward recomputes A from H and writes its gradients
    over the forward's dead buffers, so only the gradients are compared."""
    wl = workloads.ep_slice()
    gl = wl["group_list"]
    layer = _run_forward(dev, wl, with_backward=True, dyp_bits=wl["dyp"], low_memory=low_memory)
    ss, rmap, cnt = oracle.permute_maps(wl["topk_ids"], 32)
    np.testing.assert_array_equal(layer.tokens_per_expert.cpu().numpy(), gl)
    np.testing.assert_array_equal(cnt, gl)
    np.testing.assert_array_equal(layer.row_id_map.cpu().numpy(), rmap)
    np.testing.assert_array_equal(layer.sorted_slot.cpu().numpy(), ss)
    off = oracle.expert_offsets(gl)
    eo = np.repeat(np.arange(32), gl)
    rng = np.random.default_rng(77)
    w1, w2 = wl["w1"], wl["w2"]
    x_perm_bits = wl["x"][ss]                       # top_k = 1: slot == token
    rows = np.unique(np.concatenate([off[:-1][gl > 0], off[1:][gl > 0] - 1,
                                     rng.integers(0, 16384, 48)]))
    idx = torch.from_numpy(rows).to(dev)
    # dA is not stored (the SwiGLU backward runs in the down GMM's backward)
    kept = ("dh", "dx") if low_memory else ("h", "a", "yp", "dh", "dx")
    got = {k: dev_f64(getattr(layer, k)[idx]) for k in kept}
    out_tok = dev_f64(layer.out[torch.from_numpy(ss[rows]).to(dev)])
    probs = wl["probs"].astype(np.float64)
    for i, r in enumerate(rows):
        e = eo[r]
        one = np.array([1])
        xr = f64(x_perm_bits[r:r + 1])
        h = oracle.round_bf16(oracle.gmm(xr, f64(w1[e:e + 1]), one))
        a = oracle.round_bf16(oracle.swiglu(h))
        yp = oracle.round_bf16(oracle.gmm(a, f64(w2[e:e + 1]), one))
        da = oracle.gmm_bwd_input(f64(wl["dyp"][r:r + 1]), f64(w2[e:e + 1]), one)  # not rounded: fused
        dh = oracle.round_bf16(oracle.swiglu_bwd(da, h))
        dx = oracle.gmm_bwd_input(dh, f64(w1[e:e + 1]), one)
        for k, ref in (("h", h), ("a", a), ("yp", yp), ("da", da), ("dh", dh), ("dx", dx)):
            if k in got:
                assert_close(got[k][i], ref[0], f"ep {k} row {r} (expert {e})")
        assert_close(out_tok[i], probs[ss[r], 0] * yp[0], f"ep out token {ss[r]}")
    # weight gradients: the two smallest non-empty experts and one random one
    live = np.nonzero(gl > 0)[0]
    picks = list(live[np.argsort(gl[live])[:2]]) + [int(rng.choice(live))]
    for e in picks:
        n = int(gl[e])
        xe = f64(x_perm_bits[off[e]:off[e + 1]])
        h = oracle.round_bf16(oracle.gmm(xe, f64(w1[e:e + 1]), [n]))
        a = oracle.round_bf16(oracle.swiglu(h))
        dye = f64(wl["dyp"][off[e]:off[e + 1]])
        da = oracle.gmm_bwd_input(dye, f64(w2[e:e + 1]), [n])  # not rounded: fused
        dh = oracle.round_bf16(oracle.swiglu_bwd(da, h))
        ks1 = rng.integers(0, 4096, 4)
        ks2 = rng.integers(0, 1536, 4)
        ref1 = oracle.gmm_bwd_weight(xe[:, ks1], dh, [n])[0]
        ref2 = oracle.gmm_bwd_weight(a[:, ks2], dye, [n])[0]
        # dh and a are chained intermediates: allow their boundary roundings
        assert_close(dev_f64(layer.dw1[e, torch.from_numpy(ks1).to(dev)]), ref1, f"ep dW1 expert {e}",
                     extra=chained_reduction_slack(xe[:, ks1], dh))
        assert_close(dev_f64(layer.dw2[e, torch.from_numpy(ks2).to(dev)]), ref2, f"ep dW2 expert {e}",
                     extra=chained_reduction_slack(a[:, ks2], dye))
    for e in np.nonzero(gl == 0)[0]:
        assert (dev_bits(layer.dw1[e]) == 0).all() and (dev_bits(layer.dw2[e]) == 0).all()


def test_ep_bench_step_sampled(dev):
    """The expert-parallel share's training step exactly as bench.py times it
    (MoeLayer.training_step_calls: fused gate_up + SwiGLU keeping H, down
    GMM, unpermute, the down pair with the SwiGLU backward, the gate_up pair
    as one gmm_bwd launch), at full size.  Sampled rows of h, a, yp, out, dh
    and dx against the oracle; dW1 and dW2 of the largest and the smallest
    non-empty expert on one weight row in every 256-row k-tile, all columns,
    so every tile rectangle of the weight-gradient schedule is hit."""
    wl = workloads.ep_slice()
    gl = wl["group_list"]
    d = wl.dims
    E, H, I, R = d["E"], d["H"], d["I"], d["R"]
    print(f"ep bench step: E={E} H={H} I={I} R={R}", flush=True)
    layer = MoeLayer(LayerShape(R, 1, E, H, I), dev, with_backward=True)
    w1, w2 = bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev)
    calls = layer.training_step_calls(bf16_dev(wl["x"], dev), torch.from_numpy(wl["topk_ids"]).to(dev),
                                      torch.from_numpy(wl["probs"]).to(dev), bf16_dev(wl["dyp"], dev),
                                      w1, w2)
    assert [n for n, _ in calls] == ["moe_permute", "gmm_fwd_swiglu", "gmm_fwd_down", "moe_unpermute",
                                     "gmm_bwd_swiglu_down", "gmm_bwd_gate_up"]
    for _, fn in calls:
        fn()
    torch.cuda.synchronize()
    assert int(layer.dev_err.item()) == 0
    ss, rmap, cnt = oracle.permute_maps(wl["topk_ids"], E)
    np.testing.assert_array_equal(layer.tokens_per_expert.cpu().numpy(), gl)
    np.testing.assert_array_equal(layer.row_id_map.cpu().numpy(), rmap)
    np.testing.assert_array_equal(layer.sorted_slot.cpu().numpy(), ss)
    off = oracle.expert_offsets(gl)
    eo = np.repeat(np.arange(E), gl)
    rng = np.random.default_rng(78)
    x_perm_bits = wl["x"][ss]                       # top_k = 1: slot == token
    rows = np.unique(np.concatenate([off[:-1][gl > 0], off[1:][gl > 0] - 1, rng.integers(0, R, 64)]))
    idx = torch.from_numpy(rows).to(dev)
    got = {k: dev_f64(getattr(layer, k)[idx]) for k in ("h", "a", "yp", "dh", "dx")}
    out_tok = dev_f64(layer.out[torch.from_numpy(ss[rows]).to(dev)])
    probs = wl["probs"].astype(np.float64)
    one = np.array([1])
    for i, r in enumerate(rows):
        e = eo[r]
        xr = f64(x_perm_bits[r:r + 1])
        h_exact = oracle.gmm(xr, f64(wl["w1"][e:e + 1]), one)
        h = oracle.round_bf16(h_exact)
        a = oracle.round_bf16(oracle.gmm_swiglu(xr, f64(wl["w1"][e:e + 1]), one))  # from the accumulators
        yp = oracle.round_bf16(oracle.gmm(a, f64(wl["w2"][e:e + 1]), one))
        da = oracle.gmm_bwd_input(f64(wl["dyp"][r:r + 1]), f64(wl["w2"][e:e + 1]), one)  # fused: unrounded
        dh = oracle.round_bf16(oracle.swiglu_bwd(da, h))
        dx = oracle.gmm_bwd_input(dh, f64(wl["w1"][e:e + 1]), one)
        for k, ref in (("h", h), ("a", a), ("yp", yp), ("dh", dh), ("dx", dx)):
            assert_close(got[k][i], ref[0], f"ep step {k} row {r} (expert {e})")
        assert_close(out_tok[i], probs[ss[r], 0] * yp[0], f"ep step out token {ss[r]}")
    live = np.nonzero(gl > 0)[0]
    for e in (int(live[np.argmax(gl[live])]), int(live[np.argmin(gl[live])])):
        n = int(gl[e])
        print(f"ep bench step: weight gradients of expert {e} ({n} rows)", flush=True)
        xe = f64(x_perm_bits[off[e]:off[e + 1]])
        w1e = f64(wl["w1"][e:e + 1])
        h = oracle.round_bf16(oracle.gmm(xe, w1e, [n]))
        a = oracle.round_bf16(oracle.gmm_swiglu(xe, w1e, [n]))
        dye = f64(wl["dyp"][off[e]:off[e + 1]])
        da = oracle.gmm_bwd_input(dye, f64(wl["w2"][e:e + 1]), [n])
        dh = oracle.round_bf16(oracle.swiglu_bwd(da, h))
        # one weight row in every 256-row k-tile, every column
        ks1 = np.arange(0, H, 256) + rng.integers(0, 256, H // 256)
        ks2 = np.arange(0, I, 256) + rng.integers(0, 256, I // 256)
        ref1 = oracle.gmm_bwd_weight(xe[:, ks1], dh, [n])[0]
        ref2 = oracle.gmm_bwd_weight(a[:, ks2], dye, [n])[0]
        assert_close(dev_f64(layer.dw1[e, torch.from_numpy(ks1).to(dev)]), ref1, f"ep step dW1 expert {e}",
                     extra=chained_reduction_slack(xe[:, ks1], dh))
        assert_close(dev_f64(layer.dw2[e, torch.from_numpy(ks2).to(dev)]), ref2, f"ep step dW2 expert {e}",
                     extra=chained_reduction_slack(a[:, ks2], dye))
    for e in np.nonzero(gl == 0)[0]:
        assert (dev_bits(layer.dw1[e]) == 0).all() and (dev_bits(layer.dw2[e]) == 0).all()
