"""The index-only permute and the gathered forward GMMs on the GPU.

moe_permute_index must give the oracle's maps and counts bit for bit (the
same as moe_permute's).  gmm_fwd_gather / gmm_fwd_swiglu_gather read the
grouped rows as x[sorted_slot[r] / top_k] instead of from x_perm; their
outputs are checked against the oracle's per-expert products of those rows
(rtol = atol = 1e-2) and bit for bit against gmm_fwd / gmm_fwd_swiglu on
moe_permute's x_perm, which run the same MFMAs in the same order -- on the
row-tile kernels and on the weight-streaming kernels.  Rows at or past
sum(group_list) stay untouched.  A sorted_slot entry out of range gives a
zero row and MOE_DEVERR_SLOT.  Finally the forward-only layer with the
gather is bit-identical to the one that materialises x_perm, on the
prefill and decode workloads.
"""
import os

import numpy as np
import pytest
import torch

import grouped_gemm_moe_amd as moe
import oracle
import workloads
from tests.gpu_util import assert_close, bf16_dev, dev_bits, f64, require_gpu

pytestmark = pytest.mark.gpu

SENT = np.uint16(0x7FC1)  # a NaN pattern no kernel writes


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _ids(rng, T, K, E, mask_frac=0.0):
    ids = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    if mask_frac:
        ids[rng.random((T, K)) < mask_frac] = -1
    return ids


class force_variant:
    """MOEGMM_FORCE_VARIANT for the calls inside the block (None: the
    library's own choice)."""

    def __init__(self, v):
        self.v = v

    def __enter__(self):
        self.old = os.environ.get("MOEGMM_FORCE_VARIANT")
        if self.v is None:
            os.environ.pop("MOEGMM_FORCE_VARIANT", None)
        else:
            os.environ["MOEGMM_FORCE_VARIANT"] = self.v

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop("MOEGMM_FORCE_VARIANT", None)
        else:
            os.environ["MOEGMM_FORCE_VARIANT"] = self.old


@pytest.mark.parametrize("T,K,E,mask", [
    (4, 2, 4, 0.0),          # one block (the single-workgroup permute)
    (0, 8, 16, 0.0),         # no tokens: counts zeroed
    (3000, 8, 128, 0.05),    # scan and scatter in one launch
    (20000, 8, 1024, 0.05),  # the segmented scan
])
def test_permute_index_matches_oracle_and_permute(dev, T, K, E, mask):
    print(f"moe_permute_index T={T} K={K} E={E} mask={mask}", flush=True)
    rng = np.random.default_rng(T + 7 * E)
    ids = _ids(rng, T, K, E, mask) if T else np.zeros((0, K), dtype=np.int32)
    tid = torch.from_numpy(ids).to(dev)
    S = T * K
    rm = torch.full((S,), -7, dtype=torch.int32, device=dev)
    ss = torch.full((S,), -7, dtype=torch.int32, device=dev)
    tpe = torch.full((E,), -7, dtype=torch.int64, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.moe_permute_index(tid, E, out=(rm, ss, tpe), dev_err=err)
    x = bf16_dev(workloads.normal_bf16(rng, (T, 64)), dev)
    _, rm2, ss2, tpe2 = moe.moe_permute(x, tid, E)
    torch.cuda.synchronize()
    ref_ss, ref_rm, ref_cnt = oracle.permute_maps(ids, E)
    R = len(ref_ss)
    assert int(err.item()) == 0
    np.testing.assert_array_equal(tpe.cpu().numpy(), ref_cnt)
    np.testing.assert_array_equal(rm.cpu().numpy(), ref_rm)
    np.testing.assert_array_equal(ss.cpu().numpy()[:R], ref_ss)
    assert (ss.cpu().numpy()[R:] == -7).all()
    assert torch.equal(rm, rm2) and torch.equal(ss[:R], ss2[:R]) and torch.equal(tpe, tpe2)


def _case(dev, T, K, E, H, N, mask, seed):
    rng = np.random.default_rng(seed)
    x_bits = workloads.normal_bf16(rng, (T, H))
    w_bits = workloads.normal_bf16(rng, (E, H, N), std=0.02)
    ids = _ids(rng, T, K, E, mask)
    x = bf16_dev(x_bits, dev)
    w = bf16_dev(w_bits, dev)
    x_perm, rm, ss, tpe = moe.moe_permute(x, torch.from_numpy(ids).to(dev), E)
    torch.cuda.synchronize()
    R = int(tpe.sum().item())
    return x_bits, w_bits, ids, x, w, x_perm, ss, tpe, R


# (T, top_k, E, H, N, mask, variant): row tiles (auto at these shapes, then
# forced) and weight streaming (auto for a few rows per expert, then forced
# onto a row-tile shape)
SHAPES = [
    (600, 8, 16, 512, 768, 0.0, None),
    (600, 8, 16, 512, 768, 0.1, "stream"),
    (24, 4, 32, 1024, 512, 0.2, None),
    (24, 4, 32, 1024, 512, 0.0, "tile"),
    (1000, 1, 8, 520, 264, 0.0, None),
    # many experts, most of them empty; reduction and column tails
    (300, 3, 1024, 520, 264, 0.1, None),
    (300, 3, 1024, 520, 264, 0.1, "tile"),
    # the largest top_k
    (40, 32, 64, 256, 512, 0.05, None),
]


@pytest.mark.parametrize("T,K,E,H,N,mask,variant", SHAPES)
def test_gmm_fwd_gather(dev, T, K, E, H, N, mask, variant):
    print(f"gmm_fwd_gather T={T} K={K} E={E} H={H} N={N} mask={mask} variant={variant}", flush=True)
    x_bits, w_bits, ids, x, w, x_perm, ss, tpe, R = _case(dev, T, K, E, H, N, mask, seed=T + N)
    S = T * K
    y = bf16_dev(np.full((S, N), SENT, dtype=np.uint16), dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    with force_variant(variant):
        moe.gmm_fwd_gather(x, ss, K, w, tpe, out=y, dev_err=err)
        y_ref = moe.gmm_fwd(x_perm, w, tpe)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = dev_bits(y)
    np.testing.assert_array_equal(got[:R], dev_bits(y_ref)[:R])
    assert (got[R:] == SENT).all(), "rows >= R must stay untouched"
    ref_ss, _, cnt = oracle.permute_maps(ids, E)
    ref = oracle.gmm(f64(x_bits[ref_ss // K]), f64(w_bits), cnt)
    assert_close(f64(got[:R]), ref, "gmm_fwd_gather vs oracle")


@pytest.mark.parametrize("T,K,E,H,N,mask,variant", SHAPES[:4])
@pytest.mark.parametrize("with_h", [False, True])
def test_gmm_fwd_swiglu_gather(dev, T, K, E, H, N, mask, variant, with_h):
    print(f"gmm_fwd_swiglu_gather T={T} K={K} E={E} H={H} N={N} variant={variant} h={with_h}", flush=True)
    x_bits, w_bits, ids, x, w, x_perm, ss, tpe, R = _case(dev, T, K, E, H, N, mask, seed=3 * T + N)
    S, I = T * K, N // 2
    a = bf16_dev(np.full((S, I), SENT, dtype=np.uint16), dev)
    h = bf16_dev(np.full((S, N), SENT, dtype=np.uint16), dev) if with_h else None
    h_ref = torch.empty((S, N), dtype=torch.bfloat16, device=dev) if with_h else None
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    with force_variant(variant):
        moe.gmm_fwd_swiglu_gather(x, ss, K, w, tpe, out=a, h_out=h, dev_err=err)
        a_ref = moe.gmm_fwd_swiglu(x_perm, w, tpe, h_out=h_ref)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = dev_bits(a)
    np.testing.assert_array_equal(got[:R], dev_bits(a_ref)[:R])
    assert (got[R:] == SENT).all()
    if with_h:
        np.testing.assert_array_equal(dev_bits(h)[:R], dev_bits(h_ref)[:R])
        assert (dev_bits(h)[R:] == SENT).all()
    ref_ss, _, cnt = oracle.permute_maps(ids, E)
    ref = oracle.gmm_swiglu(f64(x_bits[ref_ss // K]), f64(w_bits), cnt)
    assert_close(f64(got[:R]), ref, "gmm_fwd_swiglu_gather vs oracle")


def test_gather_empty_call(dev):
    """No tokens: the gathered calls enqueue nothing and return."""
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    ss = torch.empty((0,), dtype=torch.int32, device=dev)
    w = torch.zeros((4, 64, 128), dtype=torch.bfloat16, device=dev)
    g = torch.zeros(4, dtype=torch.int64, device=dev)
    y = moe.gmm_fwd_gather(x, ss, 2, w, g)
    a = moe.gmm_fwd_swiglu_gather(x, ss, 2, w, g)
    torch.cuda.synchronize()
    assert y.shape == (0, 128) and a.shape == (0, 64)


@pytest.mark.parametrize("variant", ["tile", "stream"])
def test_gather_slot_out_of_range(dev, variant):
    """Two grouped rows get a slot outside [0, T*top_k): they read zeros
    (outputs exactly 0), MOE_DEVERR_SLOT is set, every other row is as
    before."""
    T, K, E, H, N = 64, 4, 16, 512, 512
    print(f"gather bad slot variant={variant}", flush=True)
    _, _, _, x, w, x_perm, ss, tpe, R = _case(dev, T, K, E, H, N, 0.0, seed=99)
    bad = ss.clone()
    bad[3] = T * K + 5
    bad[R - 1] = -2
    y = torch.empty((T * K, N), dtype=torch.bfloat16, device=dev)
    a = torch.empty((T * K, N // 2), dtype=torch.bfloat16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    err2 = torch.zeros(1, dtype=torch.int32, device=dev)
    with force_variant(variant):
        moe.gmm_fwd_gather(x, bad, K, w, tpe, out=y, dev_err=err)
        moe.gmm_fwd_swiglu_gather(x, bad, K, w, tpe, out=a, dev_err=err2)
        y_ref = moe.gmm_fwd(x_perm, w, tpe)
        a_ref = moe.gmm_fwd_swiglu(x_perm, w, tpe)
    torch.cuda.synchronize()
    assert int(err.item()) == moe.DEVERR_SLOT and int(err2.item()) == moe.DEVERR_SLOT
    for got, ref in ((dev_bits(y), dev_bits(y_ref)), (dev_bits(a), dev_bits(a_ref))):
        keep = np.ones(R, dtype=bool)
        keep[[3, R - 1]] = False
        np.testing.assert_array_equal(got[:R][keep], ref[:R][keep])
        assert (got[[3, R - 1]] == 0).all()


@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_layer_forward_gathered_is_bit_identical(dev, name):
    from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayer

    print(f"layer forward gathered {name}", flush=True)
    wl = getattr(workloads, name)()
    d = wl.dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    x = bf16_dev(wl["x"], dev)
    w1 = bf16_dev(wl["w1"], dev)
    w2 = bf16_dev(wl["w2"], dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    probs = torch.from_numpy(wl["probs"]).to(dev)
    plain = MoeLayer(shape, dev)
    gath = MoeLayer(shape, dev, gather_rows=True)
    assert gath.x_perm is None
    out_p = plain.forward(x, ids, probs, w1, w2, fused="auto", keep_h=False).clone()
    out_g = gath.forward(x, ids, probs, w1, w2, fused="auto", keep_h=False).clone()
    torch.cuda.synchronize()
    assert int(gath.dev_err.item()) == 0
    assert torch.equal(gath.tokens_per_expert, plain.tokens_per_expert)
    np.testing.assert_array_equal(dev_bits(out_g), dev_bits(out_p))


def test_gather_rows_is_forward_only(dev):
    from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayer

    with pytest.raises(ValueError):
        MoeLayer(LayerShape(8, 2, 4, 64, 32), dev, with_backward=True, gather_rows=True)


# --- the A8W8-FP (MXFP8) GMM1 reading quantised token rows -------------------

MX_SHAPES = [
    (600, 8, 16, 512, 384, 0.1, None),   # row tiles
    (600, 8, 16, 512, 384, 0.0, "stream"),
    (24, 4, 32, 1024, 256, 0.2, None),   # weight streaming
    (24, 4, 32, 1024, 256, 0.0, "tile"),
]


@pytest.mark.parametrize("T,K,E,H,I,mask,variant", MX_SHAPES)
def test_gmm_mx_fwd_swiglu_gather(dev, T, K, E, H, I, mask, variant):
    """Q_MX is row-wise, so the token rows quantised once hold the bytes
    moe_permute_mx writes for each slot row; GMM1 through sorted_slot on them
    is bit-identical to GMM1 on the permuted rows."""
    print(f"gmm_mx_fwd_swiglu_gather T={T} K={K} E={E} H={H} I={I} variant={variant}", flush=True)
    rng = np.random.default_rng(T + I)
    x = bf16_dev(workloads.normal_bf16(rng, (T, H)), dev)
    w1 = bf16_dev(workloads.normal_bf16(rng, (E, H, 2 * I), std=0.02), dev)
    ids = torch.from_numpy(_ids(rng, T, K, E, mask)).to(dev)
    w1q, w1s = moe.mx_quantize(w1.transpose(1, 2).contiguous())
    xq_p, xs_p, _, ss, tpe = moe.moe_permute_mx(x, ids, E)
    xq_t, xs_t = moe.mx_quantize(x)
    torch.cuda.synchronize()
    R = int(tpe.sum().item())
    tok = ss[:R].long() // K
    assert torch.equal(xq_t[tok], xq_p[:R])
    nb = H // 32
    assert torch.equal(xs_t[tok][:, :nb], xs_p[:R, :nb])
    S, ld_a = T * K, moe.mx_scale_ld(I)
    aq = torch.full((S, I), 0xA5, dtype=torch.uint8, device=dev)
    asc = torch.full((S, ld_a), 0xA5, dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    with force_variant(variant):
        moe.gmm_mx_fwd_swiglu_gather(xq_t, xs_t, ss, K, w1q, w1s, tpe, out=(aq, asc), dev_err=err)
        aq_ref, as_ref = moe.gmm_mx_fwd_swiglu(xq_p, xs_p, w1q, w1s, tpe)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(aq[:R], aq_ref[:R])
    assert torch.equal(asc[:R, :I // 32], as_ref[:R, :I // 32])
    assert (aq[R:] == 0xA5).all() and (asc[R:] == 0xA5).all()


@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_layer_mx_gathered_is_bit_identical(dev, name):
    from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayerMX

    print(f"MX layer forward gathered {name}", flush=True)
    wl = getattr(workloads, name)()
    d = wl.dims
    shape = LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"])
    x = bf16_dev(wl["x"], dev)
    wmx = MoeLayerMX.prepare_weights(bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev))
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    probs = torch.from_numpy(wl["probs"]).to(dev)
    plain = MoeLayerMX(shape, dev)
    gath = MoeLayerMX(shape, dev, gather_rows=True)
    assert gath.xq.shape[0] == d["T"]
    out_p = plain.forward(x, ids, probs, *wmx).clone()
    out_g = gath.forward(x, ids, probs, *wmx).clone()
    torch.cuda.synchronize()
    assert int(gath.dev_err.item()) == 0
    np.testing.assert_array_equal(dev_bits(out_g), dev_bits(out_p))


# --- SwiGLU and the down GMM in one call --------------------------------------

@pytest.mark.parametrize("T,K,E,I,N,mask,variant", [
    (64, 8, 256, 512, 2048, 0.0, None),      # decode shape: one streaming launch
    (64, 8, 256, 512, 2048, 0.1, "tile"),    # forced: swiglu, then the row tiles
    (600, 8, 16, 256, 520, 0.0, None),       # row tiles
    (24, 4, 32, 264, 264, 0.2, "stream"),    # a reduction tail
])
def test_swiglu_gmm_fwd(dev, T, K, E, I, N, mask, variant):
    """a and y bit-identical to swiglu then gmm_fwd; rows >= R untouched."""
    print(f"swiglu_gmm_fwd T={T} K={K} E={E} I={I} N={N} variant={variant}", flush=True)
    rng = np.random.default_rng(T + I + N)
    ids = _ids(rng, T, K, E, mask)
    g = torch.from_numpy(oracle.tokens_per_expert(ids, E)).to(dev)
    S = T * K
    R = int(g.sum().item())
    h_b = workloads.normal_bf16(rng, (S, 2 * I))
    w_b = workloads.normal_bf16(rng, (E, I, N), std=0.02)
    h, w2 = bf16_dev(h_b, dev), bf16_dev(w_b, dev)
    a = bf16_dev(np.full((S, I), SENT, dtype=np.uint16), dev)
    y = bf16_dev(np.full((S, N), SENT, dtype=np.uint16), dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    with force_variant(variant):
        moe.swiglu_gmm_fwd(h, w2, g, out=(a, y), dev_err=err)
        a_ref = moe.swiglu(h, g)
        y_ref = moe.gmm_fwd(a_ref, w2, g)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    np.testing.assert_array_equal(dev_bits(a)[:R], dev_bits(a_ref)[:R])
    np.testing.assert_array_equal(dev_bits(y)[:R], dev_bits(y_ref)[:R])
    assert (dev_bits(a)[R:] == SENT).all() and (dev_bits(y)[R:] == SENT).all()
    ref = oracle.gmm(f64(dev_bits(a_ref)[:R]), f64(w_b), oracle.tokens_per_expert(ids, E))
    assert_close(f64(dev_bits(y)[:R]), ref, "swiglu_gmm_fwd vs oracle")
