"""CPU oracle for the MXFP8 (A8W8-FP) variant of the expert block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP library and imports nothing from it.

Source: "MegaMoE" (ops-transformer, mc2/mega_moe), the A8W8-FP scenario --
tokens gathered per expert are MX-quantised in groups of 32 (a shared exponent
per group, FP8 elements, FLOAT8_E8M0 scales); GMM1 multiplies the dequantised
input by the dequantised gate and up halves of W1; the activation output is
MX-quantised again; GMM2 multiplies it by the dequantised W2; dequantisation
happens inside the matmul.  The parameter table gives the activation scales
the shape (rows, CeilDiv(H, 32)) and says the hidden size is the LAST
dimension of weight1, i.e. quantised weights are stored reduction-contiguous,
[E, N, K] with scales [E, N, CeilDiv(K, 32)].

The group quantiser Q_MX follows the published OCP Microscaling (MX) v1.0
definition, restated here:
  * E8M0 scale byte b stands for 2^(b - 127); 255 is NaN.
  * For a group V of 32 values: shared_exp = floor(log2(max|V|)) - emax, with
    emax = 8 for FP8 E4M3 (its largest normal is 1.75 * 2^8 = 448); an all-
    zero group takes the smallest scale 2^-127; shared_exp is clamped to
    [-127, 127].
  * Each element is V / 2^shared_exp rounded to the nearest E4M3 value, ties
    to even, saturating at +-448 (E4M3 "FN" has no infinity; 0x7F / 0xFF are
    NaN and are produced only for NaN input).
Where the pages leave the rounding and saturation of the element conversion
open, this is the reading taken.

Everything here works in float64 on exactly representable values.
"""
from __future__ import annotations

import numpy as np

from .moe_ref import sigmoid

GROUP = 32          # MX block size along the reduction dimension
E4M3_EMAX = 8       # exponent of the largest E4M3 normal
E4M3_MAX = 448.0    # largest finite E4M3 magnitude
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUB_STEP = 2.0 ** -9


# ---------------------------------------------------------------------------
# FP8 E4M3 (FN) and E8M0 codes
# ---------------------------------------------------------------------------


def e4m3_decode(codes) -> np.ndarray:
    """uint8 E4M3FN codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    sub = sign * man * E4M3_SUB_STEP
    v = np.where(exp == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def _round_half_even(x: np.ndarray) -> np.ndarray:
    return np.rint(x)  # NumPy rounds halves to even


def e4m3_encode(v) -> np.ndarray:
    """float64 -> E4M3FN codes: round to nearest, ties to even, saturate at
    +-448; NaN -> 0x7F (sign kept)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.int64)
    # subnormal range (and zero): multiples of 2^-9
    sub = a < E4M3_MIN_NORMAL
    m = _round_half_even(np.where(sub, a / E4M3_SUB_STEP, 0.0)).astype(np.int64)
    # m == 8 is the smallest normal, code 0b0001_000 == 8: the same integer
    out = np.where(sub, m, out)
    # normal range: 3 mantissa bits at the value's binade
    nrm = ~sub & np.isfinite(a)
    e = np.floor(np.log2(np.where(nrm, a, 1.0))).astype(np.int64)
    step = np.exp2(e - 3.0)
    q = _round_half_even(np.where(nrm, a / step, 0.0)) * step      # rounded magnitude
    q = np.minimum(q, E4M3_MAX)                                      # saturate
    e2 = np.floor(np.log2(np.where(nrm, q, 1.0))).astype(np.int64)  # binade after rounding
    man = np.round((q / np.exp2(e2) - 1.0) * 8.0).astype(np.int64)
    code_n = ((e2 + 7) << 3) | man
    out = np.where(nrm, code_n, out)
    out = np.where(np.isinf(a), 0x7E, out)                           # saturate infinities
    out = np.where(np.isnan(v), 0x7F, out)
    out = out | np.where(sign, 0x80, 0)
    return out.astype(np.uint8)


def e8m0_decode(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


# ---------------------------------------------------------------------------
# Q_MX / DQ_MX along the last axis, groups of 32
# ---------------------------------------------------------------------------


def mx_quantize(a):
    """a [..., K] float64 -> (codes [..., K] uint8, scales [..., ceil(K/32)]
    uint8 E8M0).  A ragged last group is quantised on its own elements."""
    a = np.asarray(a, dtype=np.float64)
    K = a.shape[-1]
    G = (K + GROUP - 1) // GROUP
    pad = G * GROUP - K
    ap = np.concatenate([a, np.zeros(a.shape[:-1] + (pad,))], axis=-1) if pad else a
    blocks = ap.reshape(a.shape[:-1] + (G, GROUP))
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), -np.inf)
    shared = np.where(np.isfinite(e), e - E4M3_EMAX, -127.0)
    shared = np.clip(shared, -127.0, 127.0)
    scales = (shared + 127.0).astype(np.uint8)
    codes = e4m3_encode(blocks / np.exp2(shared)[..., None])
    codes = codes.reshape(ap.shape)[..., :K]
    return codes, scales


_E4M3_VALUES = None


def _e4m3_table() -> np.ndarray:
    """e4m3_decode of every code, for decoding large tensors by lookup."""
    global _E4M3_VALUES
    if _E4M3_VALUES is None:
        _E4M3_VALUES = e4m3_decode(np.arange(256, dtype=np.uint8))
    return _E4M3_VALUES


def mx_dequantize(codes, scales) -> np.ndarray:
    """(codes [..., K], scales [..., ceil(K/32)]) -> float64 [..., K]."""
    v = _e4m3_table()[np.asarray(codes, dtype=np.uint8)]
    K = v.shape[-1]
    s = np.repeat(e8m0_decode(scales), GROUP, axis=-1)[..., :K]
    return v * s


# ---------------------------------------------------------------------------
# MX grouped matmul, its SwiGLU-fused form, and the A8W8-FP expert block
# ---------------------------------------------------------------------------


def gmm_mx(xq, xs, wq, ws, group_list) -> np.ndarray:
    """y[rows_e] = DQ(x[rows_e]) @ DQ(w[e])^T with w stored [E, N, K]."""
    x = mx_dequantize(xq, xs)
    gl = np.asarray(group_list, dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(gl)])
    y = np.zeros((x.shape[0], wq.shape[1]), dtype=np.float64)
    for e, n in enumerate(gl):
        if n:  # an empty expert's weights are never read
            y[off[e]:off[e] + n] = x[off[e]:off[e] + n] @ mx_dequantize(wq[e], ws[e]).T
    return y


def gmm_swiglu_mx(xq, xs, w1q, w1s, group_list) -> np.ndarray:
    """A = SiLU(G) * U with [G | U] = DQ(x) @ DQ(w1)^T, w1 stored [E, 2I, K]
    (gate rows first): the activation before its own MX quantisation."""
    h = gmm_mx(xq, xs, w1q, w1s, group_list)
    I = h.shape[1] // 2
    g, u = h[:, :I], h[:, I:]
    return g * sigmoid(g) * u


def expert_block_mx(x_perm, w1q, w1s, w2q, w2s, group_list) -> dict:
    """The A8W8-FP expert block on gathered rows: Q_MX(x) -> GMM1 + SwiGLU ->
    Q_MX(A) -> GMM2.  Returns every quantised intermediate and the output
    (exact; the device rounds it to bf16 once)."""
    xq, xs = mx_quantize(x_perm)
    a = gmm_swiglu_mx(xq, xs, w1q, w1s, group_list)
    aq, as_ = mx_quantize(a)
    y = gmm_mx(aq, as_, w2q, w2s, group_list)
    return dict(xq=xq, xs=xs, a=a, aq=aq, as_=as_, y=y)


def moe_layer_forward_mx(x, topk_ids, probs, w1q, w1s, w2q, w2s, num_experts: int,
                         rounding=None) -> dict:
    """permute -> the A8W8-FP expert block -> weighted unpermute.

    ["MegaMoE", A8W8-FP scenario, composed with the A16W16 dispatch and
    combine.]  x holds bf16 values (float64); each row is MX-quantised as it
    is gathered (row-wise quantisation commutes with the gather).  Yp, the
    down GMM output, crosses the boundary in bf16 (``rounding``, e.g. the
    oracle's round_bf16; None keeps it exact); ``out`` is returned exact.
    """
    from .moe_ref import permute, unpermute
    rnd = rounding if rounding is not None else (lambda v: v)
    x_perm, row_id_map, sorted_slot, counts = permute(x, topk_ids, num_experts)
    blk = expert_block_mx(x_perm, w1q, w1s, w2q, w2s, counts)
    yp = rnd(blk["y"])
    out = unpermute(yp, row_id_map, probs)
    return dict(x_perm=x_perm, row_id_map=row_id_map, sorted_slot=sorted_slot,
                tokens_per_expert=counts, yp=yp, out=out, **blk)
