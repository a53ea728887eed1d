"""Seeded synthetic inputs for the routed-expert MoE path.

This module only draws random numbers and packs them; it holds none of the
path's arithmetic.  Both the oracle and the HIP path consume what it returns,
and neither imports the other.

Every tensor is returned as a NumPy array on the host:

* bf16 tensors as ``uint16`` bit patterns (the rounding from the fp32 draw is
  done by PyTorch's CPU cast, a library routine, so both sides see identical
  bits);
* expert ids as ``int32`` (``-1`` marks a masked slot);
* gate weights ("probs") as ``float32``;
* group lists as ``int64`` counts.

Distributions follow the workload descriptions: activations and incoming
gradients N(0, 1), weights N(0, sigma) with sigma read as the standard
deviation, gate weights U(0, 1) or a softmax over N(0, 1) router logits.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def _to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns via PyTorch's CPU cast (RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return _to_bf16_bits(a)


def softmax_topk_routing(rng: np.random.Generator, T: int, E: int, K: int):
    """Router stand-in: softmax of N(0,1) logits, then the K largest.

    Ids come out in descending-probability order per token (ties by lower
    expert id); the probabilities are not renormalised.
    """
    logits = rng.standard_normal(size=(T, E), dtype=np.float32).astype(np.float64)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :K]
    ids = order.astype(np.int32)
    probs = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return ids, probs


@dataclass
class Workload:
    name: str
    dims: dict
    arrays: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.arrays[k]


# ---------------------------------------------------------------------------
# tiny worked example: 4 tokens, top-2, E=4 (group list [1, 2, 0, 2])
# ---------------------------------------------------------------------------
TINY_TOPK_IDS = np.array([[1, 3], [1, -1], [0, -1], [3, -1]], dtype=np.int32)


def tiny(seed: int = 0) -> Workload:
    T, K, E, H, I = 4, 2, 4, 64, 32
    rng = np.random.default_rng(seed)
    arrays = dict(
        topk_ids=TINY_TOPK_IDS.copy(),
        x=normal_bf16(rng, (T, H)),
        w1=normal_bf16(rng, (E, H, 2 * I), 0.05),
        w2=normal_bf16(rng, (E, I, H), 0.05),
        probs=rng.uniform(0.0, 1.0, size=(T, K)).astype(np.float32),
        dyp=normal_bf16(rng, (5, H)),
        dout=normal_bf16(rng, (T, H)),  # drawn last: the arrays above keep their values
    )
    return Workload("tiny", dict(T=T, K=K, E=E, H=H, I=I), arrays)


# ---------------------------------------------------------------------------
# plain GMM sweep: E=8, [1024, 512] x [8, 512, 1024], three group lists
# ---------------------------------------------------------------------------
def sweep_group_list(variant: int, rng: np.random.Generator, M: int = 1024, E: int = 8):
    if variant == 0:
        return np.full(E, M // E, dtype=np.int64)
    if variant == 1:
        p = rng.dirichlet(np.ones(E))
        return rng.multinomial(M, p).astype(np.int64)
    if variant == 2:
        live = [e for e in range(E) if e not in (0, 3, 7)]
        p = rng.dirichlet(np.ones(len(live)))
        c = rng.multinomial(M, p)
        gl = np.zeros(E, dtype=np.int64)
        gl[live] = c
        return gl
    raise ValueError(variant)


def sweep(variant: int, M: int = 1024, K: int = 512, N: int = 1024, E: int = 8) -> Workload:
    seed = 1 + variant
    rng = np.random.default_rng(seed)
    gl = sweep_group_list(variant, rng, M, E)
    arrays = dict(
        group_list=gl,
        x=normal_bf16(rng, (M, K)),
        w=normal_bf16(rng, (E, K, N), 0.02),
        dy=normal_bf16(rng, (M, N)),
    )
    return Workload(f"sweep{variant}", dict(M=M, K=K, N=N, E=E), arrays)


# ---------------------------------------------------------------------------
# full MoE layer shapes: prefill (T=4096, top-8, E=128) and decode (T=64, E=256)
# ---------------------------------------------------------------------------
def moe_layer(name: str, seed: int, T: int, K: int, E: int, H: int, I: int,
              w_std: float = 0.02, with_weights: bool = True) -> Workload:
    rng = np.random.default_rng(seed)
    ids, probs = softmax_topk_routing(rng, T, E, K)
    arrays = dict(topk_ids=ids, probs=probs, x=normal_bf16(rng, (T, H)))
    if with_weights:
        arrays["w1"] = normal_bf16(rng, (E, H, 2 * I), w_std)
        arrays["w2"] = normal_bf16(rng, (E, I, H), w_std)
    return Workload(name, dict(T=T, K=K, E=E, H=H, I=I), arrays)


def prefill(**kw) -> Workload:
    return moe_layer("prefill", 4, T=4096, K=8, E=128, H=2048, I=512, **kw)


def decode(**kw) -> Workload:
    return moe_layer("decode", 6, T=64, K=8, E=256, H=2048, I=512, **kw)


def decode_skewed(hot: int = 7, extra_tokens: int = 48) -> Workload:
    """The decode workload with one hot expert: tokens 0 .. extra_tokens-1
    route their last slot to expert `hot` (unless it is already among their
    experts), so it holds about 50 rows while the others hold 0-6."""
    wl = decode()
    ids = wl["topk_ids"].copy()
    for t in range(extra_tokens):
        if hot not in ids[t]:
            ids[t, -1] = hot
    arrays = dict(wl.arrays)
    arrays["topk_ids"] = ids
    return Workload("decode_skewed", dict(wl.dims), arrays)


# ---------------------------------------------------------------------------
# one expert-parallel rank's share: E=32 local experts, 16384 received rows
# ---------------------------------------------------------------------------
def zipf_group_list(rng: np.random.Generator, R: int, E: int, s: float = 1.2,
                    n_empty: int = 3) -> np.ndarray:
    empty = rng.choice(E, size=n_empty, replace=False)
    live = np.array([e for e in range(E) if e not in set(empty.tolist())])
    rank = rng.permutation(len(live)) + 1
    shares = rank.astype(np.float64) ** (-s)
    shares /= shares.sum()
    gl = np.zeros(E, dtype=np.int64)
    gl[live] = rng.multinomial(R, shares)
    return gl


def ep_slice(seed: int = 5, R: int = 16384, E: int = 32, H: int = 4096, I: int = 1536,
             with_weights: bool = True, with_acts: bool = True) -> Workload:
    """Rows received by one expert-parallel rank, each with one local expert id.

    The received rows arrive in a shuffled order; the local permute (top_k=1)
    groups them by expert, which reproduces the Zipf group list.
    """
    rng = np.random.default_rng(seed)
    gl = zipf_group_list(rng, R, E)
    ids = np.repeat(np.arange(E, dtype=np.int32), gl)
    ids = ids[rng.permutation(R)].reshape(R, 1)
    arrays = dict(group_list=gl, topk_ids=ids,
                  probs=rng.uniform(0.0, 1.0, size=(R, 1)).astype(np.float32))
    if with_acts:
        arrays["x"] = normal_bf16(rng, (R, H))
        arrays["dyp"] = normal_bf16(rng, (R, H))
    if with_weights:
        arrays["w1"] = normal_bf16(rng, (E, H, 2 * I), 0.02)
        arrays["w2"] = normal_bf16(rng, (E, I, H), 0.02)
    return Workload("ep", dict(T=R, K=1, E=E, H=H, I=I, R=R), arrays)


def random_group_list(rng: np.random.Generator, M: int, E: int, empty_frac: float = 0.3,
                      fill: float = 1.0) -> np.ndarray:
    """Group sizes summing to about fill*M, with some experts forced empty."""
    total = int(M * fill)
    live = rng.random(E) >= empty_frac
    if not live.any():
        live[rng.integers(E)] = True
    p = rng.dirichlet(np.ones(int(live.sum())))
    gl = np.zeros(E, dtype=np.int64)
    gl[live] = rng.multinomial(total, p)
    return gl


# ---------------------------------------------------------------------------
# MXFP8 (A8W8-FP) layouts: the same bf16 weights, stored reduction-contiguous
# ---------------------------------------------------------------------------
def reduction_major_weights(wl: Workload):
    """(w1t [E, 2I, H], w2t [E, H, I]) bf16 bit patterns: w1 and w2 of a layer
    workload transposed so each output column's weights are contiguous (the
    layout the MX weights are quantised in).  Only a copy of bits."""
    w1t = np.ascontiguousarray(np.transpose(wl["w1"], (0, 2, 1)))
    w2t = np.ascontiguousarray(np.transpose(wl["w2"], (0, 2, 1)))
    return w1t, w2t


def wide_range_bf16(rng: np.random.Generator, shape, lo: int = -40, hi: int = 40,
                    zero_frac: float = 0.02) -> np.ndarray:
    """N(0,1) rows times 2^u with u uniform in [lo, hi) per 32-element group,
    with some groups zeroed: exercises every E8M0 scale path of Q_MX."""
    a = rng.standard_normal(size=shape, dtype=np.float32)
    K = shape[-1]
    G = (K + 31) // 32
    e = rng.integers(lo, hi, size=shape[:-1] + (G,)).astype(np.float32)
    z = rng.random(shape[:-1] + (G,)) < zero_frac
    f = np.where(z, np.float32(0), np.exp2(e)).astype(np.float32)
    a = a * np.repeat(f, 32, axis=-1)[..., :K]
    return _to_bf16_bits(a)


def mx_random(rng: np.random.Generator, shape, std: float = 0.02):
    """A synthetic MX tensor (E4M3 code bytes [..., K], E8M0 scale bytes
    [..., K/32]) whose values spread like N(0, std^2) weights: elements
    N(0, 64^2) packed into float8_e4m3fn by PyTorch's CPU cast (a library
    routine, as for the bf16 draws), one scale per group of 32 near std/64
    with a random +-1 in its exponent.  Drawn directly: neither side computes
    these operands, and the stand-in for MX-quantised weights costs no
    quantisation pass."""
    import torch

    K = shape[-1]
    assert K % 32 == 0
    # the normal draws come from a torch CPU generator seeded from rng (fast
    # for weight-sized tensors, and just as reproducible)
    g = torch.Generator().manual_seed(int(rng.integers(0, 2 ** 62)))
    a = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    a.mul_(64.0).clamp_(-448.0, 448.0)
    codes = a.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    base = 127 + int(np.rint(np.log2(std))) - 6
    scales = (base + rng.integers(-1, 2, size=tuple(shape[:-1]) + (K // 32,))).astype(np.uint8)
    return codes, scales


def mx_small_integers(rng: np.random.Generator, shape, scale_exps=(-5, -4)):
    """MX operands (E4M3 code bytes [..., K], E8M0 scale bytes [..., K/32])
    whose elements are integers in [-8, 8], packed by PyTorch's CPU
    float8_e4m3fn cast (exact for these), with one scale 2^u per row, u drawn
    from scale_exps.  Any product of two such operands is an integer times a
    power of two, so every sum of them is exact in an accumulator a few bits
    wide: a product-sum then has one right answer on every implementation."""
    import torch

    K = shape[-1]
    assert K % 32 == 0
    v = rng.integers(-8, 9, size=tuple(shape)).astype(np.float32)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    u = rng.choice(np.asarray(scale_exps), size=tuple(shape[:-1]) + (1,))
    scales = np.repeat(127 + u, K // 32, axis=-1).astype(np.uint8)
    return codes, scales
