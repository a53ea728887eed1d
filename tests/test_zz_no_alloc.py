"""moe_permute_noalloc (the entry point that allocates nothing: its scratch is
the library's static device array) against moe_permute with a workspace.

Both run through the C ABI (ctypes, device pointers of preallocated
tensors) on the same seeded routing: row_id_map, sorted_slot,
tokens_per_expert and x_perm must be bit-identical.  Two calls in a row, the
second with a smaller input, so the second sees the first's contents left in
the shared scratch; plus a single-workgroup (decode-sized) call and a call
past the scratch limit, which must return MOE_ERR_WORKSPACE.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from grouped_gemm_moe_amd import _lib
from tests.gpu_util import bf16_dev, require_gpu

pytestmark = pytest.mark.gpu

MOE_OK, MOE_ERR_WORKSPACE = 0, 3


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _bufs(dev, T, K, H, E):
    S = T * K
    return dict(x_perm=torch.full((S, H), float("nan"), dtype=torch.bfloat16, device=dev),
                rmap=torch.full((S,), -7, dtype=torch.int32, device=dev),
                ss=torch.full((S,), -7, dtype=torch.int32, device=dev),
                tpe=torch.full((E,), -7, dtype=torch.int64, device=dev),
                err=torch.zeros(1, dtype=torch.int32, device=dev))


def _run(lib, dev, x, ids, E, noalloc):
    T, H = x.shape
    K = ids.shape[1]
    b = _bufs(dev, T, K, H, E)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if noalloc:
        st = lib.moe_permute_noalloc(_p(x), _p(ids), T, K, H, E, _p(b["x_perm"]), _p(b["rmap"]), _p(b["ss"]),
                                     _p(b["tpe"]), _p(b["err"]), stream)
    else:
        nbytes = lib.moe_permute_workspace_size(T, K, E)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        st = lib.moe_permute(_p(x), _p(ids), T, K, H, E, _p(b["x_perm"]), _p(b["rmap"]), _p(b["ss"]),
                             _p(b["tpe"]), _p(ws), nbytes, _p(b["err"]), stream)
    assert st == MOE_OK, lib.moe_status_string(st)
    return b


def _case(seed, T, K, E, H):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    ids[rng.random((T, K)) < 0.05] = -1  # some masked slots
    x = workloads.normal_bf16(rng, (T, H))
    return x, ids


@pytest.mark.parametrize("shapes", [
    # (T, top_k, E, H): a multi-block call, then a smaller one on the same
    # scratch (both above the 4096 slots of the single-workgroup path, which
    # needs no scratch), then a decode-sized call
    [(4096, 8, 128, 2048), (2000, 4, 96, 512), (64, 8, 256, 2048)],
    [(16384, 1, 32, 4096), (600, 8, 256, 2048)],
])
def test_noalloc_matches_workspace_call(dev, shapes):
    lib = _lib.load()
    for i, (T, K, E, H) in enumerate(shapes):
        print(f"moe_permute_noalloc call {i}: T={T} top_k={K} E={E} H={H}", flush=True)
        xb, ib = _case(100 + i + T, T, K, E, H)
        x, ids = bf16_dev(xb, dev), torch.from_numpy(ib).to(dev)
        ref = _run(lib, dev, x, ids, E, noalloc=False)
        got = _run(lib, dev, x, ids, E, noalloc=True)
        torch.cuda.synchronize()
        R = int(ref["tpe"].sum().item())
        assert int(got["err"].item()) == 0 and int(ref["err"].item()) == 0
        assert torch.equal(got["tpe"], ref["tpe"])
        assert torch.equal(got["rmap"], ref["rmap"])
        assert torch.equal(got["ss"][:R], ref["ss"][:R])
        assert torch.equal(got["x_perm"][:R].view(torch.int16), ref["x_perm"][:R].view(torch.int16))
        assert torch.isnan(got["x_perm"][R:].float()).all(), "rows >= R written"


def test_noalloc_rejects_calls_past_its_scratch(dev):
    lib = _lib.load()
    T, K, E, H = 1 << 20, 1, 1024, 8   # 1024 histogram blocks x 1024 experts x 4 B = 4 MiB
    assert lib.moe_permute_workspace_size(T, K, E) > (1 << 20)
    fake = ctypes.c_void_p(1 << 20)     # never dereferenced: the call returns before enqueueing
    st = lib.moe_permute_noalloc(fake, fake, T, K, H, E, fake, fake, fake, fake, None, None)
    assert st == MOE_ERR_WORKSPACE
