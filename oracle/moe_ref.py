"""CPU oracle for the routed-expert grouped-GEMM MoE path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP library (``grouped_gemm_moe_amd``) and imports nothing
from it; the two meet only through the seeded inputs of ``workloads``.

Everything here is the plain definition of what the path computes, written
out with NumPy in float64 on values that are exactly representable in bf16.
Sources (web pages, cited by title and section):

* [GMM]      "NPU Training Operators - GMM" (shaojiemike.top):
             section 算子语义 (operator semantics) -- the per-expert for-loop,
             the input table and the worked example with group list [1,2,0,2];
             the backward formulas right after it; section "Qwen3.5 MoE 路径"
             (the routed-expert chain permute -> histc -> gate_up GMM ->
             SwiGLU -> down GMM -> weighted unpermute, and the GMM shape table).
* [MegaMoE]  "MegaMoE" (ops-transformer, mc2/mega_moe): section 功能说明,
             activation formulas (sigma, SiLU, SwiGLU with clamp c), and the
             A16W16 (non-quantised) scenario: Dispatch (X_e, row(i,k)),
             Expert Compute (H_e = X_e W1[e], split into G|U, Y_e = A_e W2[e]),
             Token Combine (y_i = sum_k w_k Y_{e_ik}[row(i,k)]).
* [PermGrad] "CANN ops-transformer 算子详解：MoeTokenPermuteWithRoutingMapGrad"
             (mhpq.cn): section 2.2 (the probs gradient), section 2.3 (the
             token gradient: an index-add of the permuted rows' gradients
             back onto their tokens), section 4.1 (-1 marks an invalid slot
             that takes no part), section 6.2 (each output token walks its
             top-k slots and accumulates in FP32, cast back once).
* [MegaBlocks] "03 · grouped GEMM 路径" (MegaBlocks chapter 3): section 2
             (rows of all groups concatenated, weight [groups, k, n], a list of
             per-group row counts).

Readings where the pages are silent or ambiguous:

* group_list holds per-expert COUNTS (int64), not a cumulative sum.
* A slot (token t, choice k) has flat index s = t*top_k + k; id -1 = masked.
* Order of rows inside an expert: ascending slot index (stable).
* gate = first I columns of the gate_up output, up = last I columns.
* SwiGLU clamp off (c = +inf).
* Rounding points: every bf16 tensor crossing the library boundary is rounded
  once, round-to-nearest-even, from the exact value; the layer chain rounds at
  those same points so a layer comparison measures kernel error only.
* SwiGLU backward is not on the pages; it is derived by calculus.
* The backward of the weighted unpermute (dYp, dprobs) is the derivative of
  the Token Combine formula; the permute backward sums each token's slot
  rows in ascending k (the per-token walk of [PermGrad] 6.2).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# bf16 helpers (bit patterns <-> float64)
# ---------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """Round to bf16 (RNE), returning float64 values.

    Two steps: float64 -> float32 (NumPy, RNE), then float32 -> bf16 by
    round-to-nearest-even on the bit pattern (add 0x7FFF plus the lowest kept
    bit, truncate the low 16 bits).  NaN stays NaN.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    r = u.astype(np.uint32).view(np.float32)
    r = np.where(np.isnan(f), np.float32(np.nan), r)
    return r.astype(np.float64)


def to_bf16_bits(a) -> np.ndarray:
    """Round to bf16 (RNE) and return the uint16 bit patterns."""
    r = np.ascontiguousarray(round_bf16(a).astype(np.float32))
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# A1 histogram and A2 permute  [GMM: routed-expert chain, histc; worked example]
# ---------------------------------------------------------------------------


def tokens_per_expert(topk_ids, num_experts: int) -> np.ndarray:
    """n_e = number of slots whose expert id is e; masked (-1) slots skipped."""
    ids = np.asarray(topk_ids).reshape(-1)
    counts = np.zeros(num_experts, dtype=np.int64)
    valid = ids >= 0
    np.add.at(counts, ids[valid], 1)
    return counts


def expert_offsets(group_list) -> np.ndarray:
    """Exclusive cumulative sum, length E+1: expert e owns rows off[e]:off[e+1]."""
    gl = np.asarray(group_list, dtype=np.int64)
    off = np.zeros(gl.shape[0] + 1, dtype=np.int64)
    np.cumsum(gl, out=off[1:])
    return off


def permute_maps(topk_ids, num_experts: int):
    """Group slots by expert, stable in slot order.

    Returns (sorted_slot[R], row_id_map[T*top_k], tokens_per_expert[E]):
    row r of the permuted buffer holds slot sorted_slot[r]; slot s lands in
    row row_id_map[s] (-1 when masked).  [MegaMoE, Dispatch: X_e stacks the
    tokens routed to e in a fixed order, row(i,k) locates token i in it.]
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    counts = tokens_per_expert(ids, num_experts)
    valid = np.nonzero(ids >= 0)[0]
    sorted_slot = valid[np.argsort(ids[valid], kind="stable")]
    row_id_map = np.full(ids.shape[0], -1, dtype=np.int64)
    row_id_map[sorted_slot] = np.arange(sorted_slot.shape[0])
    return sorted_slot, row_id_map, counts


def permute(x, topk_ids, num_experts: int):
    """x_perm[r] = x[token of sorted_slot[r]] (exact copies)."""
    top_k = np.asarray(topk_ids).shape[1]
    sorted_slot, row_id_map, counts = permute_maps(topk_ids, num_experts)
    x_perm = np.asarray(x)[sorted_slot // top_k]
    return x_perm, row_id_map, sorted_slot, counts


# ---------------------------------------------------------------------------
# A3/A5 grouped matmul and B1/B2 its gradients  [GMM: operator semantics]
# ---------------------------------------------------------------------------


def gmm(x, w, group_list) -> np.ndarray:
    """y[off_e:off_e+n_e] = x[off_e:off_e+n_e] @ w[e], one expert at a time.

    An empty expert owns the empty range off_e:off_e and leaves later offsets
    unchanged.  Rows at or beyond sum(group_list) are returned as zero (they
    are undefined in the library and never compared).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = np.zeros((x.shape[0], w.shape[2]), dtype=np.float64)
    start = 0
    for e, n in enumerate(np.asarray(group_list, dtype=np.int64)):
        end = start + int(n)
        if n > 0:
            y[start:end] = x[start:end] @ w[e]
        start = end
    return y


def gmm_bwd_input(dy, w, group_list) -> np.ndarray:
    """grad_input_e = grad_output_e @ W_e^T over the same row ranges."""
    dy = np.asarray(dy, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dx = np.zeros((dy.shape[0], w.shape[1]), dtype=np.float64)
    start = 0
    for e, n in enumerate(np.asarray(group_list, dtype=np.int64)):
        end = start + int(n)
        if n > 0:
            dx[start:end] = dy[start:end] @ w[e].T
        start = end
    return dx


def gmm_bwd_weight(x, dy, group_list) -> np.ndarray:
    """grad_weight_e = X_e^T @ grad_output_e; exact zeros for an empty expert."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    gl = np.asarray(group_list, dtype=np.int64)
    dw = np.zeros((gl.shape[0], x.shape[1], dy.shape[1]), dtype=np.float64)
    start = 0
    for e, n in enumerate(gl):
        end = start + int(n)
        if n > 0:
            dw[e] = x[start:end].T @ dy[start:end]
        start = end
    return dw


# ---------------------------------------------------------------------------
# A4 SwiGLU and B3 its derivative  [MegaMoE: activation formulas, swiglu]
# ---------------------------------------------------------------------------


def sigmoid(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def swiglu(h) -> np.ndarray:
    """A = SiLU(G) * U with G = h[:, :I], U = h[:, I:], SiLU(z) = z*sigma(z)."""
    h = np.asarray(h, dtype=np.float64)
    I = h.shape[1] // 2
    g, u = h[:, :I], h[:, I:]
    return g * sigmoid(g) * u


def swiglu_bwd(da, h) -> np.ndarray:
    """dH = [dG | dU] for A = SiLU(G)*U (derived; not on the pages).

    d SiLU(g)/dg = s + g*s*(1-s) with s = sigma(g), so
    dG = dA * U * s * (1 + G*(1-s)) and dU = dA * G * s.
    """
    da = np.asarray(da, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    I = h.shape[1] // 2
    g, u = h[:, :I], h[:, I:]
    s = sigmoid(g)
    dg = da * u * s * (1.0 + g * (1.0 - s))
    du = da * g * s
    return np.concatenate([dg, du], axis=1)


# ---------------------------------------------------------------------------
# A6 probs-weighted unpermute  [MegaMoE: Token Combine; PermGrad 6.2]
# ---------------------------------------------------------------------------


def unpermute(y_perm, row_id_map, probs) -> np.ndarray:
    """out[t] = sum over valid k of probs[t,k] * y_perm[row_id_map[t*K+k]].

    Masked slots (-1) add nothing; a token with no valid slot gives zeros.
    """
    y_perm = np.asarray(y_perm, dtype=np.float64)
    probs = np.asarray(probs, dtype=np.float64)
    T, K = probs.shape
    rmap = np.asarray(row_id_map, dtype=np.int64).reshape(T, K)
    out = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for k in range(K):
        valid = rmap[:, k] >= 0
        out[valid] += probs[valid, k:k + 1] * y_perm[rmap[valid, k]]
    return out


def gmm_swiglu(x, w1, group_list) -> np.ndarray:
    """A = SiLU(G) * U with [G | U] = the gate_up GMM x @ w1[e] over each
    expert's rows, with no rounding in between.

    [MegaMoE: Expert Compute -- H_e = X_e W1[e] split along its columns into
    G and U, then the activation.]  The fused call rounds only A.
    """
    return swiglu(gmm(x, w1, group_list))


# ---------------------------------------------------------------------------
# backward of the two ends of the path: the weighted unpermute (Token Combine)
# and the permute  [MegaMoE: Token Combine; PermGrad: 2.2, 2.3, 6.2]
# ---------------------------------------------------------------------------


def unpermute_bwd(dout, y_perm, row_id_map, probs):
    """Gradients of out[t] = sum_k probs[t,k] * y_perm[row(t,k)].

    dy_perm[row(t,k)] = probs[t,k] * dout[t]   (rows no slot points at: 0)
    dprobs[t,k]       = <dout[t], y_perm[row(t,k)]>   (0 for a masked slot)
    """
    dout = np.asarray(dout, dtype=np.float64)
    y_perm = np.asarray(y_perm, dtype=np.float64)
    probs = np.asarray(probs, dtype=np.float64)
    T, K = probs.shape
    rmap = np.asarray(row_id_map, dtype=np.int64).reshape(T, K)
    dy_perm = np.zeros_like(y_perm)
    dprobs = np.zeros((T, K), dtype=np.float64)
    for k in range(K):
        valid = rmap[:, k] >= 0
        rows = rmap[valid, k]
        dy_perm[rows] = probs[valid, k:k + 1] * dout[valid]
        dprobs[valid, k] = np.sum(dout[valid] * y_perm[rows], axis=1)
    return dy_perm, dprobs


def permute_bwd(dx_perm, row_id_map, num_tokens: int):
    """dx[t] = sum over valid k, ascending, of dx_perm[row(t,k)].

    The gradient of the gather x_perm[r] = x[token(r)]: every permuted row
    hands its gradient back to the token it was copied from, and a token
    copied into several rows (top_k > 1) receives their sum.  Masked slots add
    nothing; a token with no valid slot gets zeros.
    """
    dx_perm = np.asarray(dx_perm, dtype=np.float64)
    rmap = np.asarray(row_id_map, dtype=np.int64).reshape(num_tokens, -1)
    dx = np.zeros((num_tokens, dx_perm.shape[1]), dtype=np.float64)
    for k in range(rmap.shape[1]):
        valid = rmap[:, k] >= 0
        dx[valid] += dx_perm[rmap[valid, k]]
    return dx


# ---------------------------------------------------------------------------
# chains (rounding at the library boundary)
# ---------------------------------------------------------------------------


def moe_layer_forward(x, topk_ids, probs, w1, w2, num_experts: int,
                      rounding=round_bf16) -> dict:
    """permute -> gate_up GMM -> SwiGLU -> down GMM -> weighted unpermute.

    [GMM: Qwen3.5 MoE routed-expert chain; MegaMoE: A16W16 scenario.]
    Inputs are float64 arrays of bf16 values.  Hbuf, A and Yp are rounded to
    bf16 as they would cross the boundary (``rounding``; pass ``None`` for
    the exact chain); ``out`` is returned exact.
    """
    rnd = rounding if rounding is not None else (lambda v: v)
    x_perm, row_id_map, sorted_slot, counts = permute(x, topk_ids, num_experts)
    h = rnd(gmm(x_perm, w1, counts))
    a = rnd(swiglu(h))
    yp = rnd(gmm(a, w2, counts))
    out = unpermute(yp, row_id_map, probs)
    return dict(x_perm=x_perm, row_id_map=row_id_map, sorted_slot=sorted_slot,
                tokens_per_expert=counts, h=h, a=a, yp=yp, out=out)


def expert_block_backward(x_perm, h, a, dyp, w1, w2, group_list,
                          rounding=round_bf16, fused_swiglu_bwd=False) -> dict:
    """Backward of gate_up GMM -> SwiGLU -> down GMM from dYp (permuted rows).

    dA = dYp W2^T, dW2 = A^T dYp, dH = swiglu_bwd(dA, H), dX = dH W1^T,
    dW1 = X^T dH; dA and dH rounded to bf16 at the boundary (``rounding``;
    ``None`` for the exact chain).  ``fused_swiglu_bwd``: the SwiGLU backward
    runs on the unrounded dA (dA never crosses a boundary); the returned dA
    is still its rounded value, for reference.
    """
    rnd = rounding if rounding is not None else (lambda v: v)
    da_exact = gmm_bwd_input(dyp, w2, group_list)
    da = rnd(da_exact)
    dw2 = gmm_bwd_weight(a, dyp, group_list)
    dh = rnd(swiglu_bwd(da_exact if fused_swiglu_bwd else da, h))
    dx = gmm_bwd_input(dh, w1, group_list)
    dw1 = gmm_bwd_weight(x_perm, dh, group_list)
    return dict(da=da, dw2=dw2, dh=dh, dx=dx, dw1=dw1)


def moe_layer_backward(fwd, dout, probs, w1, w2, rounding=round_bf16, fused_swiglu_bwd=False) -> dict:
    """Full layer backward from dout, given the forward dict ``fwd``.

    unpermute_bwd -> expert block backward -> permute_bwd.  dYp and dX_perm
    are rounded to bf16 as they cross the boundary (``rounding``; ``None``
    for the exact chain); dprobs (fp32 on the device) and dx are returned
    exact.
    """
    rnd = rounding if rounding is not None else (lambda v: v)
    T = np.asarray(dout).shape[0]
    dyp, dprobs = unpermute_bwd(dout, fwd["yp"], fwd["row_id_map"], probs)
    dyp = rnd(dyp)
    blk = expert_block_backward(fwd["x_perm"], fwd["h"], fwd["a"], dyp, w1, w2,
                                fwd["tokens_per_expert"], rounding=rounding,
                                fused_swiglu_bwd=fused_swiglu_bwd)
    dx_perm = rnd(blk["dx"])
    dx = permute_bwd(dx_perm, fwd["row_id_map"], T)
    return dict(dyp=dyp, dprobs=dprobs, da=blk["da"], dw2=blk["dw2"], dh=blk["dh"],
                dx_perm=dx_perm, dw1=blk["dw1"], dx=dx)
