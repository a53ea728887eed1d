"""moe_permute on the GPU vs the oracle: bit-exact indices, counts and rows."""
import numpy as np
import pytest
import torch

import grouped_gemm_moe_amd as moe
import oracle
import workloads
from tests.gpu_util import bf16_dev, dev_bits, require_gpu

pytestmark = pytest.mark.gpu

SENT = np.uint16(0x7FC1)  # a NaN pattern no kernel writes


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _random_ids(rng, T, K, E, mask_frac=0.0):
    ids = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=K, replace=False) if K <= E else rng.integers(0, E, K)
    if mask_frac:
        ids[rng.random((T, K)) < mask_frac] = -1
    return ids


def run_permute(dev, x_bits, ids, E):
    T, K = ids.shape
    H = x_bits.shape[1]
    print(f"moe_permute T={T} K={K} E={E} H={H}", flush=True)
    x = bf16_dev(x_bits, dev)
    tid = torch.from_numpy(ids).to(dev)
    S = T * K
    xp = bf16_dev(np.full((S, H), SENT, dtype=np.uint16), dev)
    rmap = torch.full((S,), -7, dtype=torch.int32, device=dev)
    ss = torch.full((S,), -7, dtype=torch.int32, device=dev)
    tpe = torch.full((E,), -7, dtype=torch.int64, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.moe_permute(x, tid, E, out=(xp, rmap, ss, tpe), dev_err=err)
    torch.cuda.synchronize()
    return dev_bits(xp), rmap.cpu().numpy(), ss.cpu().numpy(), tpe.cpu().numpy(), int(err.item())


def check_permute(dev, x_bits, ids, E, expect_err=0, ref_ids=None):
    xp, rmap, ss, tpe, err = run_permute(dev, x_bits, ids, E)
    ref_ids = ids if ref_ids is None else ref_ids
    K = ids.shape[1]
    ref_ss, ref_rmap, ref_cnt = oracle.permute_maps(ref_ids, E)
    R = len(ref_ss)
    assert err == expect_err
    np.testing.assert_array_equal(tpe, ref_cnt)
    np.testing.assert_array_equal(rmap, ref_rmap)
    np.testing.assert_array_equal(ss[:R], ref_ss)
    assert (ss[R:] == -7).all(), "sorted_slot entries >= R must stay untouched"
    np.testing.assert_array_equal(xp[:R], x_bits[ref_ss // K])
    assert (xp[R:] == SENT).all(), "x_perm rows >= R must stay untouched"


def test_worked_example(dev):
    w = workloads.tiny()
    check_permute(dev, w["x"], w["topk_ids"], 4)


@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_layer_routings(dev, name):
    w = getattr(workloads, name)(with_weights=False)
    check_permute(dev, w["x"], w["topk_ids"], w.dims["E"])


def test_ep_slice_routing(dev):
    w = workloads.ep_slice(with_weights=False, with_acts=False)
    rng = np.random.default_rng(21)
    x = workloads.normal_bf16(rng, (w.dims["R"], 64))
    check_permute(dev, x, w["topk_ids"], 32)


@pytest.mark.parametrize("T,K,E,H,mask", [
    (1000, 4, 64, 64, 0.25),
    (37, 2, 1, 16, 0.5),          # one expert
    (300, 32, 1024, 8, 0.1),      # max top_k, max experts
    (20000, 8, 64, 8, 0.05),      # many chunks (160k slots)
    (5, 3, 700, 24, 0.0),         # most experts empty
    (64, 8, 256, 2048, 1.0),      # every slot masked
    (1536, 8, 1024, 8, 0.0),      # 12 chunks x 1024 experts: the largest table scanned per block
    (4000, 8, 1024, 8, 0.1),      # 32 chunks x 1024 experts: the two-launch segmented scan
    (20000, 8, 1024, 8, 0.05),    # 157 chunks x 1024 experts: three scan segments
])
def test_random_routings(dev, T, K, E, H, mask):
    rng = np.random.default_rng(T * 31 + K)
    ids = _random_ids(rng, T, K, E, mask)
    x = workloads.normal_bf16(rng, (T, H))
    check_permute(dev, x, ids, E)


def test_zero_tokens(dev):
    E = 16
    tpe = torch.full((E,), -7, dtype=torch.int64, device=dev)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((0, 2), dtype=torch.int32, device=dev)
    moe.moe_permute(x, ids, E, out=(torch.empty((0, 64), dtype=torch.bfloat16, device=dev),
                                    torch.empty(0, dtype=torch.int32, device=dev),
                                    torch.empty(0, dtype=torch.int32, device=dev), tpe))
    torch.cuda.synchronize()
    assert (tpe.cpu().numpy() == 0).all()


def test_invalid_ids_are_masked_and_reported(dev):
    rng = np.random.default_rng(5)
    T, K, E = 200, 4, 32
    ids = _random_ids(rng, T, K, E, 0.1)
    bad = ids.copy()
    bad[3, 1] = E
    bad[50, 0] = -5
    bad[199, 3] = 1 << 20
    ref = bad.copy()
    ref[(ref >= E) | (ref < -1)] = -1
    x = workloads.normal_bf16(rng, (T, 32))
    check_permute(dev, x, bad, E, expect_err=moe.DEVERR_EXPERT_ID, ref_ids=ref)


def test_deterministic_repeat(dev):
    w = workloads.prefill(with_weights=False)
    a = run_permute(dev, w["x"], w["topk_ids"], 128)
    b = run_permute(dev, w["x"], w["topk_ids"], 128)
    for u, v in zip(a[:4], b[:4]):
        np.testing.assert_array_equal(u, v)
