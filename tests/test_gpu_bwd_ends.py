"""Backward of the two ends of the path on the GPU vs the oracle:
moe_unpermute_bwd (dYp = probs * dout, dprobs = <dout, Yp row>) and
moe_permute_bwd (dx[t] = sum of the token's slot rows), plus the whole
layer's backward from dout on the worked example."""
import numpy as np
import pytest
import torch

import grouped_gemm_moe_amd as moe
import oracle
import workloads
from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayer
from tests.gpu_util import (RTOL, ATOL, assert_close, bf16_dev, chained_reduction_slack, dev_bits,
                            dev_f64, f64, require_gpu)

pytestmark = pytest.mark.gpu

SENT = np.uint16(0x7FC1)

CASES = [
    (4096, 8, 2048, 0.0),   # prefill
    (64, 8, 2048, 0.1),     # decode
    (16384, 1, 4096, 0.0),  # ep rank (top_k = 1)
    (50, 32, 64, 0.5),      # max top_k, many masked slots
    (33, 3, 8, 0.3),        # top_k not a power of two, minimum hidden
    (7, 5, 7168, 0.2),      # hidden not a multiple of the 2048 columns a pass covers
    (21, 4, 16, 1.0),       # every slot masked
]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _random_row_map(rng, T, K, mask_frac):
    """A permutation of the valid slots onto rows 0..R-1, -1 for masked slots."""
    S = T * K
    valid = rng.random(S) >= mask_frac
    rmap = np.full(S, -1, dtype=np.int32)
    rmap[valid] = rng.permutation(int(valid.sum())).astype(np.int32)
    return rmap


@pytest.mark.parametrize("T,K,H,mask", CASES)
def test_unpermute_bwd(dev, T, K, H, mask):
    rng = np.random.default_rng(T * 7 + K + H)
    S = T * K
    rmap = _random_row_map(rng, T, K, mask)
    R = int((rmap >= 0).sum())
    y = workloads.normal_bf16(rng, (S, H))
    dout = workloads.normal_bf16(rng, (T, H))
    probs = rng.random((T, K)).astype(np.float32)
    print(f"moe_unpermute_bwd T={T} K={K} H={H} R={R}", flush=True)
    dyp_d = bf16_dev(np.full((S, H), SENT, np.uint16), dev)
    dp_d = torch.full((T, K), float("nan"), dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.moe_unpermute_bwd(bf16_dev(dout, dev), bf16_dev(y, dev), torch.from_numpy(rmap).to(dev),
                          torch.from_numpy(probs).to(dev), out=(dyp_d, dp_d), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref_dyp, ref_dp = oracle.unpermute_bwd(f64(dout), f64(y)[:R], rmap, probs.astype(np.float64))
    got_dyp = dev_f64(dyp_d)
    assert_close(got_dyp[:R], ref_dyp, "dy_perm")
    assert (dev_bits(dyp_d)[R:] == SENT).all(), "rows no slot points at must stay untouched"
    got_dp = dp_d.cpu().numpy().astype(np.float64)
    assert_close(got_dp, ref_dp, "dprobs")
    assert np.all(got_dp.reshape(-1)[rmap < 0] == 0.0)


@pytest.mark.parametrize("T,K,H,mask", CASES)
def test_permute_bwd(dev, T, K, H, mask):
    rng = np.random.default_rng(T * 11 + K + H)
    S = T * K
    rmap = _random_row_map(rng, T, K, mask)
    R = int((rmap >= 0).sum())
    dxp = workloads.normal_bf16(rng, (S, H))
    print(f"moe_permute_bwd T={T} K={K} H={H} R={R}", flush=True)
    dx = moe.moe_permute_bwd(bf16_dev(dxp, dev), torch.from_numpy(rmap).to(dev), T)
    torch.cuda.synchronize()
    ref = oracle.permute_bwd(f64(dxp)[:R], rmap, T)
    assert_close(dev_f64(dx), ref, "dx")
    if K == 1 and mask == 0.0:
        # one slot per token: the gradient is an exact copy (a -0.0 input may
        # come back as +0.0: the sum starts from +0.0)
        np.testing.assert_array_equal(dev_f64(dx), f64(dxp)[rmap])


def test_end_backward_bad_row_map_reported(dev):
    rng = np.random.default_rng(12)
    T, K, H = 16, 2, 64
    rmap = _random_row_map(rng, T, K, 0.0)
    rmap[3] = T * K + 5
    rmap[7] = -9
    ok = rmap.copy()
    ok[[3, 7]] = -1
    y = workloads.normal_bf16(rng, (T * K, H))
    dout = workloads.normal_bf16(rng, (T, H))
    probs = rng.random((T, K)).astype(np.float32)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dyp, dp = moe.moe_unpermute_bwd(bf16_dev(dout, dev), bf16_dev(y, dev), torch.from_numpy(rmap).to(dev),
                                    torch.from_numpy(probs).to(dev), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & moe.DEVERR_ROW_MAP
    _, ref_dp = oracle.unpermute_bwd(f64(dout), f64(y), ok, probs.astype(np.float64))
    assert_close(dp.cpu().numpy().astype(np.float64), ref_dp, "dprobs with bad rows masked")
    err.zero_()
    dx = moe.moe_permute_bwd(bf16_dev(y, dev), torch.from_numpy(rmap).to(dev), T, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & moe.DEVERR_ROW_MAP
    assert_close(dev_f64(dx), oracle.permute_bwd(f64(y), ok, T), "dx with bad rows masked")


@pytest.mark.parametrize("low_memory,fuse_swiglu_bwd", [(False, True), (True, True), (False, False),
                                                       (True, False)])
def test_tiny_full_layer_backward(dev, low_memory, fuse_swiglu_bwd):
    """Worked example: forward, then the whole backward from dout; every
    gradient (dYp, dprobs, dA, dH, dX_perm, dW1, dW2, dx) against the oracle
    chain, which rounds at the same boundary points.  low_memory: the same
    gradients from the memory-optimised backward (A recomputed from H,
    gradients over dead forward buffers)."""
    wl = workloads.tiny()
    d = wl.dims
    T, K, H = d["T"], d["K"], d["H"]
    R = 5
    print(f"tiny full-layer backward, low_memory={low_memory} fuse_swiglu_bwd={fuse_swiglu_bwd}", flush=True)
    layer = MoeLayer(LayerShape(T, K, d["E"], H, d["I"]), dev, with_backward=True,
                     low_memory=low_memory, fuse_swiglu_bwd=fuse_swiglu_bwd)
    w1, w2 = bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev)
    probs_d = torch.from_numpy(wl["probs"]).to(dev)
    layer.forward(bf16_dev(wl["x"], dev), torch.from_numpy(wl["topk_ids"]).to(dev), probs_d, w1, w2)
    layer.backward_full(bf16_dev(wl["dout"], dev), probs_d, w1, w2)
    torch.cuda.synchronize()
    assert int(layer.dev_err.item()) == 0
    probs = wl["probs"].astype(np.float64)
    fwd = oracle.moe_layer_forward(f64(wl["x"]), wl["topk_ids"], probs, f64(wl["w1"]), f64(wl["w2"]), d["E"])
    g = oracle.moe_layer_backward(fwd, f64(wl["dout"]), probs, f64(wl["w1"]), f64(wl["w2"]),
                                  fused_swiglu_bwd=fuse_swiglu_bwd)
    gl = [1, 2, 0, 2]
    off = oracle.expert_offsets(gl)
    rmap = fwd["row_id_map"].reshape(T, K)
    assert_close(dev_f64(layer.dyp)[:R], g["dyp"], "dYp")
    # dprobs sums dout * Yp, and Yp is an intermediate each chain rounded itself
    dout = f64(wl["dout"])
    slack = np.zeros((T, K))
    for t in range(T):
        for k in range(K):
            if rmap[t, k] >= 0:
                slack[t, k] = chained_reduction_slack(dout[t][:, None], fwd["yp"][rmap[t, k]][:, None])[0, 0]
    assert_close(layer.dprobs.cpu().numpy().astype(np.float64), g["dprobs"], "dprobs", extra=slack)
    if not fuse_swiglu_bwd:  # the fused backward never stores dA
        assert_close(dev_f64(layer.da)[:R], g["da"], "dA")
    assert_close(dev_f64(layer.dh)[:R], g["dh"], "dH")
    assert_close(dev_f64(layer.dx)[:R], g["dx_perm"], "dX_perm")
    for name, u, v in (("dw1", fwd["x_perm"], g["dh"]), ("dw2", fwd["a"], g["dyp"])):
        extra = np.stack([chained_reduction_slack(u[off[e]:off[e + 1]], v[off[e]:off[e + 1]])
                          for e in range(4)])
        assert_close(dev_f64(getattr(layer, name)), g[name], name, extra=extra)
    # dx adds up to top_k rows of dX_perm, each within the row tolerance
    bound = (K - 1) * ATOL + RTOL * oracle.permute_bwd(np.abs(g["dx_perm"]), fwd["row_id_map"], T)
    assert_close(dev_f64(layer.dx_tokens), g["dx"], "dx", extra=bound)
    assert (dev_bits(layer.dw1)[2] == 0).all() and (dev_bits(layer.dw2)[2] == 0).all()
