"""Helpers for the GPU parity tests: upload seeded inputs, download results,
compare against the oracle with the bf16 tolerance of the GMM page
(rtol = atol = 1e-2, elementwise: |gpu - ref| <= atol + rtol*|ref|)."""
import numpy as np
import torch

import oracle

RTOL = 1e-2
ATOL = 1e-2


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import grouped_gemm_moe_amd as g

    g.library()  # raises if the HIP library is missing
    return torch.device("cuda:0")


def bf16_dev(bits: np.ndarray, dev) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(dev)


def dev_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(dev_bits(t))


def f64(bits) -> np.ndarray:
    return oracle.bf16_to_f64(bits)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, rtol=RTOL, atol=ATOL, extra=0.0):
    """|got - ref| <= atol + rtol*|ref| + extra, elementwise.

    ``extra`` (default 0) is only used for reductions whose inputs are
    chained intermediates: see chained_reduction_slack()."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref) + extra
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"max err {err.max():.4g}; first {idx.tolist()} "
                             f"got {got[tuple(idx[0])]:.6g} ref {ref[tuple(idx[0])]:.6g}")


def chained_reduction_slack(u: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Extra tolerance for C = u^T v when u or v is an intermediate that each
    side rounded to bf16 itself (a layer chain).

    The two chains may round an intermediate element to neighbouring bf16
    values (one ulp, at most 2^-7 relative), because its own inputs came from
    different fp32 accumulation orders.  Those flips enter C[k, n] as
    sum_r u[r,k] v[r,n] d[r] with |d[r]| <= 2^-7 and independent signs, whose
    size is 2^-7 * ||u[:,k] * v[:,n]||_2.  Returns that matrix."""
    u = np.asarray(u, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    return 2.0 ** -7 * np.sqrt((u * u).T @ (v * v))
