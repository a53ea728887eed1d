"""moe_decode_fwd: the decode-shaped layer forward with the routing fused
into the gate_up GMM.

Every workgroup of the routed gate_up launch counts the expert histogram and
ranks its own expert's slots (no permute launch); every output
(out, row_id_map, sorted_slot, tokens_per_expert, h, a, y_perm) must be
bit-identical to the chain moe_permute_index -> gmm_fwd_gather ->
swiglu_gmm_fwd -> moe_unpermute on the same inputs, and out must match the
oracle layer (rtol = atol = 1e-2).  Cases: the decode workload, its skewed
variant (one expert with ~50 rows), masked slots, tokens with every slot
masked (zero output rows), a token routing two slots to one expert, ids out
of range (masked, MOE_DEVERR_EXPERT_ID), buffers reused by a second call on
other inputs, tiny shapes with fewer than 256 output columns, and an empty
call.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_moe_amd as moe
import oracle
import workloads
from tests.gpu_util import assert_close, bf16_dev, dev_bits, dev_f64, f64, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _inputs(wl, dev):
    return (bf16_dev(wl["x"], dev), torch.from_numpy(wl["topk_ids"]).to(dev),
            torch.from_numpy(wl["probs"]).to(dev), bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev))


def _chain(x, ids, probs, w1, w2, E):
    err = torch.zeros(1, dtype=torch.int32, device=x.device)
    rmap, ss, tpe = moe.moe_permute_index(ids, E, dev_err=err)
    h = moe.gmm_fwd_gather(x, ss, ids.shape[1], w1, tpe, dev_err=err)
    a, yp = moe.swiglu_gmm_fwd(h, w2, tpe, dev_err=err)
    out = moe.moe_unpermute(yp, rmap, probs, dev_err=err)
    return (out, rmap, ss, tpe, h, a, yp), err


def _compare(fused, chain, R):
    names = ["out", "row_id_map", "sorted_slot", "tokens_per_expert", "h", "a", "y_perm"]
    for i, n in enumerate(names):
        f, c = fused[i], chain[i]
        if n in ("sorted_slot", "h", "a", "y_perm"):
            f, c = f[:R], c[:R]  # rows >= R are left untouched by both
        if f.dtype == torch.bfloat16:
            np.testing.assert_array_equal(dev_bits(f), dev_bits(c), err_msg=n)
        else:
            np.testing.assert_array_equal(f.cpu().numpy(), c.cpu().numpy(), err_msg=n)


def _run(dev, wl, out=None):
    x, ids, probs, w1, w2 = _inputs(wl, dev)
    E = wl.dims["E"]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    fused = moe.moe_decode_fwd(x, ids, probs, w1, w2, out=out, dev_err=err)
    chain, cerr = _chain(x, ids, probs, w1, w2, E)
    torch.cuda.synchronize()
    R = int(chain[3].sum().item())
    _compare(fused, chain, R)
    assert int(err.item()) == int(cerr.item())
    return fused, int(err.item())


@pytest.mark.parametrize("name", ["decode", "decode_skewed"])
def test_decode_fwd_bit_identical_to_chain_and_close_to_oracle(dev, name):
    print(f"moe_decode_fwd {name}", flush=True)
    wl = getattr(workloads, name)()
    fused, err = _run(dev, wl)
    assert err == 0
    ref = oracle.moe_layer_forward(f64(wl["x"]), wl["topk_ids"], wl["probs"].astype(np.float64),
                                   f64(wl["w1"]), f64(wl["w2"]), wl.dims["E"])
    np.testing.assert_array_equal(fused[3].cpu().numpy(), ref["tokens_per_expert"])
    np.testing.assert_array_equal(fused[1].cpu().numpy(), ref["row_id_map"])
    assert_close(dev_f64(fused[0]), ref["out"], f"{name}: out vs oracle")


def _masked_workload(seed, T, K, E, H, I, bad_ids=False):
    """Routing with masked slots, tokens with every slot masked, a token with
    two slots on one expert, and (bad_ids) ids outside [-1, E)."""
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=K, replace=K > E) for _ in range(T)]).astype(np.int32)
    ids[rng.random((T, K)) < 0.3] = -1
    ids[1, :] = -1
    ids[T - 1, :] = -1
    if K >= 2:
        ids[2, 0] = ids[2, 1] = E - 1
    if bad_ids:
        ids[3, 0] = E
        ids[4, K - 1] = -7
    arrays = dict(topk_ids=ids, probs=rng.uniform(0.0, 1.0, (T, K)).astype(np.float32),
                  x=workloads.normal_bf16(rng, (T, H)), w1=workloads.normal_bf16(rng, (E, H, 2 * I), 0.05),
                  w2=workloads.normal_bf16(rng, (E, I, H), 0.05))
    return workloads.Workload("masked", dict(T=T, K=K, E=E, H=H, I=I), arrays)


@pytest.mark.parametrize("T,K,E,H,I", [(40, 4, 32, 512, 256), (12, 2, 8, 64, 32), (6, 8, 16, 136, 40)])
def test_decode_fwd_masked_slots_and_empty_tokens(dev, T, K, E, H, I):
    print(f"moe_decode_fwd masked T={T} K={K} E={E} H={H} I={I}", flush=True)
    wl = _masked_workload(T + E, T, K, E, H, I)
    fused, err = _run(dev, wl)
    assert err == 0
    out = dev_bits(fused[0])
    assert (out[1] == 0).all() and (out[T - 1] == 0).all()
    d = wl.dims
    ref = oracle.moe_layer_forward(f64(wl["x"]), wl["topk_ids"], wl["probs"].astype(np.float64),
                                   f64(wl["w1"]), f64(wl["w2"]), d["E"])
    assert_close(dev_f64(fused[0]), ref["out"], "masked: out vs oracle")


def test_decode_fwd_bad_ids_are_masked_and_flagged(dev):
    print("moe_decode_fwd bad ids", flush=True)
    wl = _masked_workload(3, 24, 4, 16, 256, 128, bad_ids=True)
    fused, err = _run(dev, wl)
    assert err & moe.DEVERR_EXPERT_ID
    rmap = fused[1].cpu().numpy()
    assert rmap[3 * 4 + 0] == -1 and rmap[4 * 4 + 3] == -1


def test_decode_fwd_reused_buffers(dev):
    """Two calls on different inputs into the same buffers: the second
    call's outputs must equal the chain on its own inputs."""
    print("moe_decode_fwd reuse", flush=True)
    a = workloads.decode()
    b = workloads.decode_skewed()
    rng = np.random.default_rng(11)
    b.arrays["x"] = workloads.normal_bf16(rng, b["x"].shape)
    b.arrays["probs"] = rng.uniform(0.0, 1.0, b["probs"].shape).astype(np.float32)
    first, _ = _run(dev, a)
    bufs = tuple(t for t in first)
    second, err = _run(dev, b, out=bufs)
    assert err == 0
    assert all(s.data_ptr() == f.data_ptr() for s, f in zip(second, bufs))


def test_decode_fwd_single_token_and_single_expert(dev):
    print("moe_decode_fwd T=1 / E=1", flush=True)
    for (T, K, E) in ((1, 1, 4), (3, 2, 1)):
        rng = np.random.default_rng(T * 10 + E)
        ids = rng.integers(0, E, (T, K)).astype(np.int32)
        arrays = dict(topk_ids=ids, probs=rng.uniform(0.0, 1.0, (T, K)).astype(np.float32),
                      x=workloads.normal_bf16(rng, (T, 64)), w1=workloads.normal_bf16(rng, (E, 64, 64), 0.05),
                      w2=workloads.normal_bf16(rng, (E, 32, 64), 0.05))
        wl = workloads.Workload("small", dict(T=T, K=K, E=E, H=64, I=32), arrays)
        fused, err = _run(dev, wl)
        assert err == 0
        ref = oracle.moe_layer_forward(f64(wl["x"]), ids, wl["probs"].astype(np.float64), f64(wl["w1"]),
                                       f64(wl["w2"]), E)
        assert_close(dev_f64(fused[0]), ref["out"], f"T={T} E={E}: out vs oracle")


def test_decode_fwd_empty_call_and_shape_limits(dev):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    ids = torch.zeros((0, 2), dtype=torch.int32, device=dev)
    probs = torch.zeros((0, 2), dtype=torch.float32, device=dev)
    w1 = torch.zeros((4, 64, 64), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((4, 32, 64), dtype=torch.bfloat16, device=dev)
    tpe = torch.full((4,), 7, dtype=torch.int64, device=dev)
    res = moe.moe_decode_fwd(x, ids, probs, w1, w2, out=(None, None, None, tpe, None, None, None))
    torch.cuda.synchronize()
    assert res[3].tolist() == [0, 0, 0, 0]
    # more than 8 slots per expert: not a decode shape
    x = torch.zeros((40, 64), dtype=torch.bfloat16, device=dev)
    ids = torch.zeros((40, 2), dtype=torch.int32, device=dev)
    probs = torch.zeros((40, 2), dtype=torch.float32, device=dev)
    with pytest.raises(moe.MoeError):
        moe.moe_decode_fwd(x, ids, probs, w1, w2)


@pytest.mark.parametrize("name", ["decode", "decode_skewed"])
def test_decode_fwd_mx_bit_identical_to_gathered_chain(dev, name):
    """moe_decode_fwd_mx against MoeLayerMX(gather_rows=True).forward (mx_quantize,
    moe_permute_index, gmm_mx_fwd_swiglu_gather, gmm_mx_fwd, moe_unpermute):
    every output bit for bit, twice in a row on the same buffers."""
    from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayerMX

    print(f"moe_decode_fwd_mx {name}", flush=True)
    wl = getattr(workloads, name)()
    d = wl.dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    x, ids, probs, w1, w2 = _inputs(wl, dev)
    w1mx, w2mx = MoeLayerMX.prepare_weights(w1, w2)
    chain = MoeLayerMX(shape, dev, gather_rows=True)
    routed = MoeLayerMX(shape, dev, gather_rows=True)
    for rep in range(2):
        chain.forward(x, ids, probs, w1mx, w2mx)
        routed.forward_decode(x, ids, probs, w1mx, w2mx)
        torch.cuda.synchronize()
        R = int(chain.tokens_per_expert.sum().item())
        for nm in ("out", "row_id_map", "tokens_per_expert"):
            a, b = getattr(routed, nm), getattr(chain, nm)
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (rep, nm)
        for nm in ("sorted_slot", "aq", "as_", "yp"):
            a, b = getattr(routed, nm)[:R], getattr(chain, nm)[:R]
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (rep, nm)
        assert int(routed.dev_err.item()) == 0
    # the masked / bad-id routing: maps and flags as the chain's
    wl = _masked_workload(5, 24, 4, 16, 256, 128, bad_ids=True)
    d = wl.dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    x, ids, probs, w1, w2 = _inputs(wl, dev)
    w1mx, w2mx = MoeLayerMX.prepare_weights(w1, w2)
    chain = MoeLayerMX(shape, dev, gather_rows=True)
    routed = MoeLayerMX(shape, dev, gather_rows=True)
    chain.forward(x, ids, probs, w1mx, w2mx)
    routed.forward_decode(x, ids, probs, w1mx, w2mx)
    torch.cuda.synchronize()
    assert torch.equal(routed.out.view(torch.int16), chain.out.view(torch.int16))
    assert torch.equal(routed.row_id_map, chain.row_id_map)
    assert int(routed.dev_err.item()) == int(chain.dev_err.item()) == moe.DEVERR_EXPERT_ID
