"""swiglu, swiglu_bwd and moe_unpermute on the GPU vs the oracle."""
import numpy as np
import pytest
import torch

import grouped_gemm_moe_amd as moe
import oracle
import workloads
from tests.gpu_util import assert_close, bf16_dev, dev_bits, dev_f64, f64, require_gpu

pytestmark = pytest.mark.gpu

SENT = np.uint16(0x7FC1)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("M,I,gl", [
    (32768, 512, None),            # prefill shape, R = M
    (700, 1536, [100, 0, 500]),    # R < M_cap
    (64, 32, [1, 2, 0, 2]),        # tiny
    (16, 8, [0, 0]),               # R = 0
])
def test_swiglu_and_bwd(dev, M, I, gl):
    rng = np.random.default_rng(M + I)
    gl = np.array([M] if gl is None else gl, dtype=np.int64)
    R = int(gl.sum())
    h = workloads.normal_bf16(rng, (M, 2 * I), 2.0)
    da = workloads.normal_bf16(rng, (M, I))
    print(f"swiglu M={M} I={I} R={R}", flush=True)
    g = torch.from_numpy(gl).to(dev)
    a = moe.swiglu(bf16_dev(h, dev), g, out=bf16_dev(np.full((M, I), SENT, np.uint16), dev))
    dh = moe.swiglu_bwd(bf16_dev(da, dev), bf16_dev(h, dev), g,
                        out=bf16_dev(np.full((M, 2 * I), SENT, np.uint16), dev))
    torch.cuda.synchronize()
    hf = f64(h)
    assert_close(dev_f64(a)[:R], oracle.swiglu(hf[:R]), "swiglu")
    assert_close(dev_f64(dh)[:R], oracle.swiglu_bwd(f64(da)[:R], hf[:R]), "swiglu_bwd")
    assert (dev_bits(a)[R:] == SENT).all() and (dev_bits(dh)[R:] == SENT).all()


def test_swiglu_extremes(dev):
    """Large |G| (exp overflow) and zeros stay finite and exact where closed forms say so."""
    I = 8
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 80.0, -80.0, 3.0])
    u = np.array([5.0, 1.0, 2.0, 1.0, 1.0, 1.0, 1.0, -2.0])
    h = oracle.to_bf16_bits(np.concatenate([g, u])[None, :])
    a = moe.swiglu(bf16_dev(h, dev), torch.tensor([1], dtype=torch.int64, device=dev))
    torch.cuda.synchronize()
    got = dev_f64(a)[0]
    assert got[0] == 0.0 and np.isfinite(got).all()
    assert_close(got, oracle.swiglu(f64(h))[0], "swiglu extremes")


def _random_row_map(rng, T, K, mask_frac):
    S = T * K
    rmap = rng.permutation(S).astype(np.int32)
    rmap[rng.random(S) < mask_frac] = -1
    return rmap


@pytest.mark.parametrize("T,K,H,mask", [
    (4096, 8, 2048, 0.0),   # prefill
    (64, 8, 2048, 0.1),     # decode
    (16384, 1, 4096, 0.0),  # ep rank (top_k = 1)
    (50, 32, 64, 0.5),      # max top_k, many masked slots
    (33, 4, 8, 1.0),        # every slot masked -> zeros
])
def test_unpermute(dev, T, K, H, mask):
    rng = np.random.default_rng(T + K + H)
    S = T * K
    y = workloads.normal_bf16(rng, (S, H))
    rmap = _random_row_map(rng, T, K, mask)
    probs = rng.random((T, K)).astype(np.float32)
    print(f"moe_unpermute T={T} K={K} H={H}", flush=True)
    out = moe.moe_unpermute(bf16_dev(y, dev), torch.from_numpy(rmap).to(dev),
                            torch.from_numpy(probs).to(dev))
    torch.cuda.synchronize()
    ref = oracle.unpermute(f64(y), rmap, probs.astype(np.float64))
    assert_close(dev_f64(out), ref, "unpermute")


def test_unpermute_roundtrip_exact(dev):
    """probs one-hot at k=0 returns the token rows bit-exactly."""
    rng = np.random.default_rng(8)
    T, K, E, H = 512, 4, 16, 256
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    x = workloads.normal_bf16(rng, (T, H))
    xd = bf16_dev(x, dev)
    xp, rmap, _, _ = moe.moe_permute(xd, torch.from_numpy(ids).to(dev), E)
    probs = np.zeros((T, K), np.float32)
    probs[:, 0] = 1.0
    out = moe.moe_unpermute(xp, rmap, torch.from_numpy(probs).to(dev))
    ones = moe.moe_unpermute(xp, rmap, torch.ones((T, K), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev_bits(out), x)
    np.testing.assert_array_equal(dev_f64(ones), oracle.round_bf16(K * f64(x)))


def test_unpermute_bad_row_map_reported(dev):
    rng = np.random.default_rng(9)
    T, K, H = 16, 2, 64
    y = workloads.normal_bf16(rng, (T * K, H))
    rmap = _random_row_map(rng, T, K, 0.0)
    rmap[3] = T * K + 5
    rmap[7] = -9
    probs = rng.random((T, K)).astype(np.float32)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    out = moe.moe_unpermute(bf16_dev(y, dev), torch.from_numpy(rmap).to(dev),
                            torch.from_numpy(probs).to(dev), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & moe.DEVERR_ROW_MAP
    ok = rmap.copy()
    ok[[3, 7]] = -1
    assert_close(dev_f64(out), oracle.unpermute(f64(y), ok, probs.astype(np.float64)), "masked bad rows")
