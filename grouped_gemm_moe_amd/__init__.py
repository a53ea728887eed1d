"""Routed-expert MoE hot path on AMD MI355X (gfx950): Python binding.

Every function here only marshals torch tensors into the C ABI of
``libmoegmm.so`` (declared in ``include/moegmm.h``) and enqueues the HIP
kernels on the current torch stream; no arithmetic of the path runs in
Python or in PyTorch.  PyTorch provides device memory and streams only.

Names and argument order follow the C ABI:
    moe_permute, gmm_fwd, gmm_bwd_input, gmm_bwd_weight, swiglu, swiglu_bwd,
    moe_unpermute, and the MXFP8 calls mx_quantize, moe_permute_mx,
    gmm_mx_fwd, gmm_mx_fwd_swiglu (an MX tensor is a pair of uint8 tensors:
    codes [rows, K] and scales [rows, mx_scale_ld(K)])
Outputs are allocated with ``torch.empty`` unless passed via ``out=``; rows
at or beyond R = sum(group_list) of a permuted-row output are left as they
were (undefined for a fresh allocation).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as _L

__all__ = [
    "MoeError", "moe_permute", "moe_permute_noalloc", "moe_permute_index", "gmm_fwd", "gmm_fwd_swiglu",
    "gmm_fwd_gather", "gmm_fwd_swiglu_gather", "swiglu_gmm_fwd", "gmm_bwd_input", "gmm_bwd_weight", "gmm_bwd",
    "gmm_bwd_swiglu",
    "swiglu",
    "swiglu_bwd", "moe_unpermute", "moe_unpermute_bwd", "moe_permute_bwd", "moe_decode_fwd", "moe_decode_fwd_mx",
    "moe_permute_workspace_size", "gmm_workspace_size", "mx_scale_ld", "mx_quantize",
    "moe_permute_mx", "gmm_mx_fwd", "gmm_mx_fwd_swiglu", "gmm_mx_fwd_swiglu_gather",
    "library", "DEVERR_EXPERT_ID", "DEVERR_GROUP_LIST", "DEVERR_ROW_MAP", "DEVERR_SLOT",
]

DEVERR_EXPERT_ID = 1
DEVERR_GROUP_LIST = 2
DEVERR_ROW_MAP = 4
DEVERR_SLOT = 8
OP_FWD, OP_BWD_INPUT, OP_BWD_WEIGHT, OP_BWD = 0, 1, 2, 3
GMM_QUEUE_BYTES = 1152  # the zero-filled prefix of a GMM workspace


class MoeError(RuntimeError):
    pass


def library() -> ctypes.CDLL:
    return _L.load()


def _check(status: int, what: str):
    if status != 0:
        msg = library().moe_status_string(status).decode()
        raise MoeError(f"{what}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype) -> torch.Tensor:
    if not t.is_cuda:
        raise MoeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    return t


def _out(out, shape, dtype, device, name):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev(out, name, dtype)
    if tuple(out.shape) != tuple(shape):
        raise MoeError(f"{name} must have shape {tuple(shape)}, got {tuple(out.shape)}")
    return out


_ZEROED_WS = {}


def _workspace(nbytes: int, device, ws, zeroed: bool = False):
    """The caller's workspace, else a new one.  A `zeroed` workspace (GMM tile
    queue at its start, then scratch) must start zero-filled and is left so
    where the queue lies by every call, so one per (device, stream) is kept
    and reused."""
    if nbytes == 0:
        return None, 0
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    if zeroed:
        key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
        buf = _ZEROED_WS.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            _ZEROED_WS[key] = buf
        return buf, buf.numel()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def moe_permute_workspace_size(T: int, top_k: int, E: int) -> int:
    return int(library().moe_permute_workspace_size(T, top_k, E))


def gmm_workspace_size(E: int, M_cap: int, K: int, N: int, op: int) -> int:
    return int(library().gmm_workspace_size(E, M_cap, K, N, op))


def moe_permute(x, topk_ids, num_experts: int, *, out=None, ws=None, dev_err=None):
    """Histogram + stable permute.  Returns (x_perm, row_id_map, sorted_slot,
    tokens_per_expert); see moe_permute in include/moegmm.h."""
    _dev(x, "x", torch.bfloat16)
    _dev(topk_ids, "topk_ids", torch.int32)
    T, H = x.shape
    top_k = topk_ids.shape[1]
    if topk_ids.shape[0] != T:
        raise MoeError("topk_ids must be [T, top_k]")
    S = T * top_k
    dev = x.device
    if out is None:
        out = (None, None, None, None)
    x_perm = _out(out[0], (S, H), torch.bfloat16, dev, "x_perm")
    row_id_map = _out(out[1], (S,), torch.int32, dev, "row_id_map")
    sorted_slot = _out(out[2], (S,), torch.int32, dev, "sorted_slot")
    tpe = _out(out[3], (num_experts,), torch.int64, dev, "tokens_per_expert")
    nbytes = moe_permute_workspace_size(T, top_k, num_experts)
    ws, ws_bytes = _workspace(nbytes, dev, ws)
    _check(library().moe_permute(_ptr(x), _ptr(topk_ids), T, top_k, H, num_experts, _ptr(x_perm),
                                 _ptr(row_id_map), _ptr(sorted_slot), _ptr(tpe), _ptr(ws), ws_bytes,
                                 _ptr(dev_err), _stream(dev)), "moe_permute")
    return x_perm, row_id_map, sorted_slot, tpe


def moe_permute_noalloc(x, topk_ids, num_experts: int, *, out, dev_err=None):
    """moe_permute whose scratch is the library's static device array: no
    workspace, and nothing allocated here either -- every output comes in
    through out = (x_perm, row_id_map, sorted_slot, tokens_per_expert).  See
    moe_permute_noalloc in include/moegmm.h for the size limit and the rule
    that calls on one device must not overlap."""
    _dev(x, "x", torch.bfloat16)
    _dev(topk_ids, "topk_ids", torch.int32)
    T, H = x.shape
    top_k = topk_ids.shape[1]
    if topk_ids.shape[0] != T:
        raise MoeError("topk_ids must be [T, top_k]")
    if out is None or len(out) != 4 or any(o is None for o in out):
        raise MoeError("moe_permute_noalloc takes every output through out=")
    S = T * top_k
    dev = x.device
    x_perm = _out(out[0], (S, H), torch.bfloat16, dev, "x_perm")
    row_id_map = _out(out[1], (S,), torch.int32, dev, "row_id_map")
    sorted_slot = _out(out[2], (S,), torch.int32, dev, "sorted_slot")
    tpe = _out(out[3], (num_experts,), torch.int64, dev, "tokens_per_expert")
    _check(library().moe_permute_noalloc(_ptr(x), _ptr(topk_ids), T, top_k, H, num_experts, _ptr(x_perm),
                                         _ptr(row_id_map), _ptr(sorted_slot), _ptr(tpe), _ptr(dev_err),
                                         _stream(dev)), "moe_permute_noalloc")
    return x_perm, row_id_map, sorted_slot, tpe


def moe_permute_index(topk_ids, num_experts: int, *, out=None, ws=None, dev_err=None):
    """moe_permute without the row gather.  Returns (row_id_map, sorted_slot,
    tokens_per_expert); see moe_permute_index in include/moegmm.h."""
    _dev(topk_ids, "topk_ids", torch.int32)
    if topk_ids.dim() != 2:
        raise MoeError("topk_ids must be [T, top_k]")
    T, top_k = topk_ids.shape
    S = T * top_k
    dev = topk_ids.device
    if out is None:
        out = (None, None, None)
    row_id_map = _out(out[0], (S,), torch.int32, dev, "row_id_map")
    sorted_slot = _out(out[1], (S,), torch.int32, dev, "sorted_slot")
    tpe = _out(out[2], (num_experts,), torch.int64, dev, "tokens_per_expert")
    nbytes = moe_permute_workspace_size(T, top_k, num_experts)
    ws, ws_bytes = _workspace(nbytes, dev, ws)
    _check(library().moe_permute_index(_ptr(topk_ids), T, top_k, num_experts, _ptr(row_id_map),
                                       _ptr(sorted_slot), _ptr(tpe), _ptr(ws), ws_bytes, _ptr(dev_err),
                                       _stream(dev)), "moe_permute_index")
    return row_id_map, sorted_slot, tpe


def _gather_args(x, sorted_slot, top_k):
    _dev(x, "x", torch.bfloat16)
    _dev(sorted_slot, "sorted_slot", torch.int32)
    if x.dim() != 2 or sorted_slot.dim() != 1:
        raise MoeError("x must be [T, K] and sorted_slot [M_cap]")
    return x.shape[0], x.shape[1], sorted_slot.shape[0], int(top_k)


def gmm_fwd_gather(x, sorted_slot, top_k: int, w, group_list, *, out=None, ws=None, dev_err=None):
    """gmm_fwd on the rows x[sorted_slot[r] // top_k] without a permuted copy
    (x holds the token rows); y is [len(sorted_slot), N] in grouped row order."""
    T, K, M, top_k = _gather_args(x, sorted_slot, top_k)
    _dev(w, "w", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    E, K2, N = w.shape
    if K2 != K or group_list.shape[0] != E:
        raise MoeError("shape mismatch: x [T, K], w [E, K, N], group_list [E]")
    y = _out(out, (M, N), torch.bfloat16, x.device, "y")
    ws, ws_bytes = _workspace(gmm_workspace_size(E, M, K, N, OP_FWD), x.device, ws, zeroed=True)
    _check(library().gmm_fwd_gather(_ptr(x), _ptr(sorted_slot), T, top_k, _ptr(w), _ptr(group_list), E,
                                    M, K, N, _ptr(y), _ptr(ws), ws_bytes, _ptr(dev_err),
                                    _stream(x.device)), "gmm_fwd_gather")
    return y


def gmm_fwd_swiglu_gather(x, sorted_slot, top_k: int, w1, group_list, *, out=None, h_out=None, ws=None,
                          dev_err=None):
    """gmm_fwd_swiglu on the rows x[sorted_slot[r] // top_k] without a
    permuted copy; a is [len(sorted_slot), I] in grouped row order."""
    T, K, M, top_k = _gather_args(x, sorted_slot, top_k)
    _dev(w1, "w1", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    E, K2, N2 = w1.shape
    if K2 != K or N2 % 2 or group_list.shape[0] != E:
        raise MoeError("shape mismatch: x [T, K], w1 [E, K, 2I], group_list [E]")
    I = N2 // 2
    a = _out(out, (M, I), torch.bfloat16, x.device, "a")
    if h_out is not None:
        _out(h_out, (M, N2), torch.bfloat16, x.device, "h_out")
    ws, ws_bytes = _workspace(gmm_workspace_size(E, M, K, N2, OP_FWD), x.device, ws, zeroed=True)
    _check(library().gmm_fwd_swiglu_gather(_ptr(x), _ptr(sorted_slot), T, top_k, _ptr(w1),
                                           _ptr(group_list), E, M, K, I, _ptr(a), _ptr(h_out), _ptr(ws),
                                           ws_bytes, _ptr(dev_err), _stream(x.device)),
           "gmm_fwd_swiglu_gather")
    return a


def swiglu_gmm_fwd(h, w2, group_list, *, out=None, dev_err=None):
    """a = SiLU(G) * U of h = [G | U], then y[rows_e] = a[rows_e] @ w2[e]:
    the activation and the down GMM in one call.  Returns (a, y)."""
    _dev(h, "h", torch.bfloat16)
    _dev(w2, "w2", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    M, I2 = h.shape
    E, I, N = w2.shape
    if I2 != 2 * I or group_list.shape[0] != E:
        raise MoeError("shape mismatch: h [M, 2I], w2 [E, I, N], group_list [E]")
    if out is None:
        out = (None, None)
    a = _out(out[0], (M, I), torch.bfloat16, h.device, "a")
    y = _out(out[1], (M, N), torch.bfloat16, h.device, "y")
    _check(library().swiglu_gmm_fwd(_ptr(h), _ptr(w2), _ptr(group_list), E, M, I, N, _ptr(a), _ptr(y),
                                    _ptr(dev_err), _stream(h.device)), "swiglu_gmm_fwd")
    return a, y


def gmm_fwd(x, w, group_list, *, out=None, ws=None, dev_err=None):
    """y[rows_e] = x[rows_e] @ w[e] for every expert e."""
    _dev(x, "x", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    M, K = x.shape
    E, K2, N = w.shape
    if K2 != K or group_list.shape[0] != E:
        raise MoeError("shape mismatch: x [M, K], w [E, K, N], group_list [E]")
    y = _out(out, (M, N), torch.bfloat16, x.device, "y")
    ws, ws_bytes = _workspace(gmm_workspace_size(E, M, K, N, OP_FWD), x.device, ws, zeroed=True)
    _check(library().gmm_fwd(_ptr(x), _ptr(w), _ptr(group_list), E, M, K, N, _ptr(y), _ptr(ws),
                             ws_bytes, _ptr(dev_err), _stream(x.device)), "gmm_fwd")
    return y


def gmm_fwd_swiglu(x, w1, group_list, *, out=None, h_out=None, ws=None, dev_err=None):
    """a = SiLU(G) * U with [G | U] = x[rows_e] @ w1[e], from the fp32
    accumulators; ``h_out`` ([M, 2I], optional) also receives [G | U]."""
    _dev(x, "x", torch.bfloat16)
    _dev(w1, "w1", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    M, K = x.shape
    E, K2, N2 = w1.shape
    if K2 != K or N2 % 2 or group_list.shape[0] != E:
        raise MoeError("shape mismatch: x [M, K], w1 [E, K, 2I], group_list [E]")
    I = N2 // 2
    a = _out(out, (M, I), torch.bfloat16, x.device, "a")
    if h_out is not None:
        _out(h_out, (M, N2), torch.bfloat16, x.device, "h_out")
    ws, ws_bytes = _workspace(gmm_workspace_size(E, M, K, N2, OP_FWD), x.device, ws, zeroed=True)
    _check(library().gmm_fwd_swiglu(_ptr(x), _ptr(w1), _ptr(group_list), E, M, K, I, _ptr(a),
                                    _ptr(h_out), _ptr(ws), ws_bytes, _ptr(dev_err),
                                    _stream(x.device)), "gmm_fwd_swiglu")
    return a


def gmm_bwd_input(dy, w, group_list, *, out=None, ws=None, dev_err=None):
    """dx[rows_e] = dy[rows_e] @ w[e]^T."""
    _dev(dy, "dy", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    M, N = dy.shape
    E, K, N2 = w.shape
    if N2 != N or group_list.shape[0] != E:
        raise MoeError("shape mismatch: dy [M, N], w [E, K, N], group_list [E]")
    dx = _out(out, (M, K), torch.bfloat16, dy.device, "dx")
    ws, ws_bytes = _workspace(gmm_workspace_size(E, M, K, N, OP_BWD_INPUT), dy.device, ws, zeroed=True)
    _check(library().gmm_bwd_input(_ptr(dy), _ptr(w), _ptr(group_list), E, M, K, N, _ptr(dx),
                                   _ptr(ws), ws_bytes, _ptr(dev_err), _stream(dy.device)),
           "gmm_bwd_input")
    return dx


def gmm_bwd_weight(x, dy, group_list, *, out=None, ws=None, dev_err=None):
    """dw[e] = x[rows_e]^T @ dy[rows_e]; zeros for empty experts."""
    _dev(x, "x", torch.bfloat16)
    _dev(dy, "dy", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    M, K = x.shape
    M2, N = dy.shape
    E = group_list.shape[0]
    if M2 != M:
        raise MoeError("shape mismatch: x [M, K], dy [M, N]")
    dw = _out(out, (E, K, N), torch.bfloat16, x.device, "dw")
    ws, ws_bytes = _workspace(gmm_workspace_size(E, M, K, N, OP_BWD_WEIGHT), x.device, ws, zeroed=True)
    _check(library().gmm_bwd_weight(_ptr(x), _ptr(dy), _ptr(group_list), E, M, K, N, _ptr(dw),
                                    _ptr(ws), ws_bytes, _ptr(dev_err), _stream(x.device)),
           "gmm_bwd_weight")
    return dw


def gmm_bwd(x, dy, w, group_list, *, dx_out=None, dw_out=None, ws=None, dev_err=None):
    """(dx, dw): dx[rows_e] = dy[rows_e] @ w[e]^T and dw[e] = x[rows_e]^T @ dy[rows_e]
    in one launch; bit-identical to gmm_bwd_input and gmm_bwd_weight."""
    _dev(x, "x", torch.bfloat16)
    _dev(dy, "dy", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    M, K = x.shape
    M2, N = dy.shape
    E = group_list.shape[0]
    if M2 != M or tuple(w.shape) != (E, K, N):
        raise MoeError("shape mismatch: x [M, K], dy [M, N], w [E, K, N]")
    dx = _out(dx_out, (M, K), torch.bfloat16, x.device, "dx")
    dw = _out(dw_out, (E, K, N), torch.bfloat16, x.device, "dw")
    ws, ws_bytes = _workspace(gmm_workspace_size(E, M, K, N, OP_BWD), x.device, ws, zeroed=True)
    _check(library().gmm_bwd(_ptr(x), _ptr(dy), _ptr(w), _ptr(group_list), E, M, K, N, _ptr(dx),
                             _ptr(dw), _ptr(ws), ws_bytes, _ptr(dev_err), _stream(x.device)),
           "gmm_bwd")
    return dx, dw


def gmm_bwd_swiglu(x, dy, w, h, group_list, *, dh_out=None, dw_out=None, ws=None, dev_err=None):
    """(dh, dw) of the down GMM with the SwiGLU backward fused: dh =
    swiglu_bwd(dy[rows_e] @ w[e]^T, h) (the product not rounded in between),
    dw[e] = x[rows_e]^T @ dy[rows_e].  dh_out may be h (in place)."""
    _dev(x, "x", torch.bfloat16)
    _dev(dy, "dy", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    _dev(h, "h", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    M, K = x.shape
    M2, N = dy.shape
    E = group_list.shape[0]
    if M2 != M or tuple(w.shape) != (E, K, N) or tuple(h.shape) != (M, 2 * K):
        raise MoeError("shape mismatch: x [M, K], dy [M, N], w [E, K, N], h [M, 2K]")
    dh = _out(dh_out, (M, 2 * K), torch.bfloat16, x.device, "dh")
    dw = _out(dw_out, (E, K, N), torch.bfloat16, x.device, "dw")
    ws, ws_bytes = _workspace(gmm_workspace_size(E, M, K, N, OP_BWD), x.device, ws, zeroed=True)
    _check(library().gmm_bwd_swiglu(_ptr(x), _ptr(dy), _ptr(w), _ptr(h), _ptr(group_list), E, M, K, N,
                                    _ptr(dh), _ptr(dw), _ptr(ws), ws_bytes, _ptr(dev_err),
                                    _stream(x.device)), "gmm_bwd_swiglu")
    return dh, dw


def swiglu(h, group_list, *, out=None):
    """a = SiLU(h[:, :I]) * h[:, I:] for rows < sum(group_list)."""
    _dev(h, "h", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    M, I2 = h.shape
    I = I2 // 2
    a = _out(out, (M, I), torch.bfloat16, h.device, "a")
    _check(library().swiglu(_ptr(h), _ptr(group_list), group_list.shape[0], M, I, _ptr(a),
                            _stream(h.device)), "swiglu")
    return a


def swiglu_bwd(da, h, group_list, *, out=None):
    """dh = [dG | dU] for a = SiLU(G) * U."""
    _dev(da, "da", torch.bfloat16)
    _dev(h, "h", torch.bfloat16)
    _dev(group_list, "group_list", torch.int64)
    M, I2 = h.shape
    I = I2 // 2
    if tuple(da.shape) != (M, I):
        raise MoeError("da must be [M, I] for h [M, 2I]")
    dh = _out(out, (M, I2), torch.bfloat16, h.device, "dh")
    _check(library().swiglu_bwd(_ptr(da), _ptr(h), _ptr(group_list), group_list.shape[0], M, I,
                                _ptr(dh), _stream(h.device)), "swiglu_bwd")
    return dh


def moe_unpermute(y_perm, row_id_map, probs, *, out=None, dev_err=None):
    """out[t] = sum_k probs[t,k] * y_perm[row_id_map[t*K+k]] (fp32, one rounding)."""
    _dev(y_perm, "y_perm", torch.bfloat16)
    _dev(row_id_map, "row_id_map", torch.int32)
    _dev(probs, "probs", torch.float32)
    T, top_k = probs.shape
    S, H = y_perm.shape
    if S != T * top_k or row_id_map.numel() != S:
        raise MoeError("y_perm must be [T*top_k, H] and row_id_map [T*top_k]")
    o = _out(out, (T, H), torch.bfloat16, y_perm.device, "out")
    _check(library().moe_unpermute(_ptr(y_perm), _ptr(row_id_map), _ptr(probs), T, top_k, H,
                                   _ptr(o), _ptr(dev_err), _stream(y_perm.device)), "moe_unpermute")
    return o


def moe_decode_fwd(x, topk_ids, probs, w1, w2, *, out=None, dev_err=None):
    """The decode-shaped layer forward with the routing fused into the
    gate_up GMM (three launches, no permute launch).  Returns (out,
    row_id_map, sorted_slot, tokens_per_expert, h, a, y_perm), all
    bit-identical to moe_permute_index -> gmm_fwd_gather -> swiglu_gmm_fwd ->
    moe_unpermute; out= takes a tuple of the same seven (None entries are
    allocated)."""
    _dev(x, "x", torch.bfloat16)
    _dev(topk_ids, "topk_ids", torch.int32)
    _dev(probs, "probs", torch.float32)
    _dev(w1, "w1", torch.bfloat16)
    _dev(w2, "w2", torch.bfloat16)
    T, H = x.shape
    E, H1, I2 = w1.shape
    I = I2 // 2
    if topk_ids.dim() != 2 or topk_ids.shape[0] != T or tuple(probs.shape) != tuple(topk_ids.shape):
        raise MoeError("topk_ids and probs must be [T, top_k] for x [T, H]")
    if H1 != H or tuple(w2.shape) != (E, I, H) or I2 != 2 * I:
        raise MoeError("shape mismatch: x [T, H], w1 [E, H, 2I], w2 [E, I, H]")
    top_k = topk_ids.shape[1]
    S = T * top_k
    dev = x.device
    o = tuple(out) if out is not None else (None,) * 7
    if len(o) != 7:
        raise MoeError("out= takes (out, row_id_map, sorted_slot, tokens_per_expert, h, a, y_perm)")
    res = (_out(o[0], (T, H), torch.bfloat16, dev, "out"),
           _out(o[1], (S,), torch.int32, dev, "row_id_map"),
           _out(o[2], (S,), torch.int32, dev, "sorted_slot"),
           _out(o[3], (E,), torch.int64, dev, "tokens_per_expert"),
           _out(o[4], (S, 2 * I), torch.bfloat16, dev, "h"),
           _out(o[5], (S, I), torch.bfloat16, dev, "a"),
           _out(o[6], (S, H), torch.bfloat16, dev, "y_perm"))
    _check(library().moe_decode_fwd(_ptr(x), _ptr(topk_ids), _ptr(probs), _ptr(w1), _ptr(w2), T, top_k, H, I,
                                    E, *[_ptr(t) for t in res], _ptr(dev_err), _stream(dev)), "moe_decode_fwd")
    return res


def moe_decode_fwd_mx(xq, xs, topk_ids, probs, w1q, w1s, w2q, w2s, *, out=None, dev_err=None):
    """The A8W8-FP decode layer forward with the routing fused into GMM1:
    (xq, xs) = mx_quantize(x) token rows, MX weights w1 [E, 2I, H], w2
    [E, H, I].  Returns (out, row_id_map, sorted_slot, tokens_per_expert, aq,
    as, y_perm), bit-identical to moe_permute_index -> gmm_mx_fwd_swiglu_gather
    -> gmm_mx_fwd -> moe_unpermute; out= takes a tuple of the same seven."""
    H, ld_x = _mx_pair(xq, xs, "x")
    H1, ld_w1 = _mx_pair(w1q, w1s, "w1")
    I, ld_w2 = _mx_pair(w2q, w2s, "w2")
    _dev(topk_ids, "topk_ids", torch.int32)
    _dev(probs, "probs", torch.float32)
    T = xq.shape[0]
    E, N2, _ = w1q.shape
    if H1 != H or N2 != 2 * I or tuple(w2q.shape) != (E, H, I):
        raise MoeError("shape mismatch: x [T, H], w1 [E, 2I, H], w2 [E, H, I]")
    if topk_ids.dim() != 2 or topk_ids.shape[0] != T or tuple(probs.shape) != tuple(topk_ids.shape):
        raise MoeError("topk_ids and probs must be [T, top_k] for x [T, H]")
    top_k = topk_ids.shape[1]
    S = T * top_k
    ld_a = mx_scale_ld(I)
    dev = xq.device
    o = tuple(out) if out is not None else (None,) * 7
    if len(o) != 7:
        raise MoeError("out= takes (out, row_id_map, sorted_slot, tokens_per_expert, aq, as, y_perm)")
    res = (_out(o[0], (T, H), torch.bfloat16, dev, "out"),
           _out(o[1], (S,), torch.int32, dev, "row_id_map"),
           _out(o[2], (S,), torch.int32, dev, "sorted_slot"),
           _out(o[3], (E,), torch.int64, dev, "tokens_per_expert"),
           _out(o[4], (S, I), torch.uint8, dev, "aq"),
           _out(o[5], (S, ld_a), torch.uint8, dev, "as"),
           _out(o[6], (S, H), torch.bfloat16, dev, "y_perm"))
    r = [_ptr(t) for t in res]
    _check(library().moe_decode_fwd_mx(_ptr(xq), _ptr(xs), ld_x, _ptr(topk_ids), _ptr(probs), _ptr(w1q),
                                       _ptr(w1s), ld_w1, _ptr(w2q), _ptr(w2s), ld_w2, T, top_k, H, I, E,
                                       r[0], r[1], r[2], r[3], r[4], r[5], ld_a, r[6], _ptr(dev_err),
                                       _stream(dev)), "moe_decode_fwd_mx")
    return res


def moe_unpermute_bwd(dout, y_perm, row_id_map, probs, *, out=None, dev_err=None):
    """Gradients of moe_unpermute: dy_perm[row(t,k)] = probs[t,k] * dout[t] and
    dprobs[t,k] = <dout[t], y_perm[row(t,k)]> (fp32).  Returns (dy_perm, dprobs);
    ``out`` may pass both buffers as a pair."""
    _dev(dout, "dout", torch.bfloat16)
    _dev(y_perm, "y_perm", torch.bfloat16)
    _dev(row_id_map, "row_id_map", torch.int32)
    _dev(probs, "probs", torch.float32)
    T, top_k = probs.shape
    S, H = y_perm.shape
    if S != T * top_k or row_id_map.numel() != S or tuple(dout.shape) != (T, H):
        raise MoeError("dout must be [T, H], y_perm [T*top_k, H] and row_id_map [T*top_k]")
    dyp_out, dp_out = out if out is not None else (None, None)
    dyp = _out(dyp_out, (S, H), torch.bfloat16, y_perm.device, "dy_perm")
    dp = _out(dp_out, (T, top_k), torch.float32, y_perm.device, "dprobs")
    _check(library().moe_unpermute_bwd(_ptr(dout), _ptr(y_perm), _ptr(row_id_map), _ptr(probs), T,
                                       top_k, H, _ptr(dyp), _ptr(dp), _ptr(dev_err),
                                       _stream(y_perm.device)), "moe_unpermute_bwd")
    return dyp, dp


def moe_permute_bwd(dx_perm, row_id_map, num_tokens: int, *, out=None, dev_err=None):
    """dx[t] = sum over valid k, ascending, of dx_perm[row_id_map[t*K+k]] (fp32, one rounding)."""
    _dev(dx_perm, "dx_perm", torch.bfloat16)
    _dev(row_id_map, "row_id_map", torch.int32)
    S, H = dx_perm.shape
    T = int(num_tokens)
    if T <= 0 or S % T != 0 or row_id_map.numel() != S:
        raise MoeError("dx_perm must be [T*top_k, H] and row_id_map [T*top_k]")
    top_k = S // T
    dx = _out(out, (T, H), torch.bfloat16, dx_perm.device, "dx")
    _check(library().moe_permute_bwd(_ptr(dx_perm), _ptr(row_id_map), T, top_k, H, _ptr(dx),
                                     _ptr(dev_err), _stream(dx_perm.device)), "moe_permute_bwd")
    return dx


# ---------------------------------------------------------------------------
# MXFP8 (A8W8-FP)
# ---------------------------------------------------------------------------


def mx_scale_ld(K: int) -> int:
    """Scale row stride for K codes: ceil(K/32) rounded up to 16 bytes."""
    g = (K + 31) // 32
    return (g + 15) // 16 * 16


def mx_quantize(x, *, out=None):
    """Q_MX of every row (last dimension) of a bf16 tensor; returns
    (codes uint8 like x, scales uint8 [..., mx_scale_ld(K)])."""
    _dev(x, "x", torch.bfloat16)
    K = x.shape[-1]
    rows = x.numel() // K if K else 0
    ld = mx_scale_ld(K)
    if out is None:
        out = (None, None)
    q = _out(out[0], tuple(x.shape), torch.uint8, x.device, "q")
    sc = _out(out[1], tuple(x.shape[:-1]) + (ld,), torch.uint8, x.device, "scales")
    _check(library().mx_quantize(_ptr(x), rows, K, ld, _ptr(q), _ptr(sc), _stream(x.device)),
           "mx_quantize")
    return q, sc


def moe_permute_mx(x, topk_ids, num_experts: int, *, out=None, ws=None, dev_err=None):
    """moe_permute whose gather writes Q_MX of each row.  Returns (xq, xs,
    row_id_map, sorted_slot, tokens_per_expert)."""
    _dev(x, "x", torch.bfloat16)
    _dev(topk_ids, "topk_ids", torch.int32)
    T, H = x.shape
    top_k = topk_ids.shape[1]
    if topk_ids.shape[0] != T:
        raise MoeError("topk_ids must be [T, top_k]")
    S = T * top_k
    dev = x.device
    ld = mx_scale_ld(H)
    if out is None:
        out = (None,) * 5
    xq = _out(out[0], (S, H), torch.uint8, dev, "xq")
    xs = _out(out[1], (S, ld), torch.uint8, dev, "xs")
    row_id_map = _out(out[2], (S,), torch.int32, dev, "row_id_map")
    sorted_slot = _out(out[3], (S,), torch.int32, dev, "sorted_slot")
    tpe = _out(out[4], (num_experts,), torch.int64, dev, "tokens_per_expert")
    nbytes = moe_permute_workspace_size(T, top_k, num_experts)
    ws, ws_bytes = _workspace(nbytes, dev, ws)
    _check(library().moe_permute_mx(_ptr(x), _ptr(topk_ids), T, top_k, H, num_experts, _ptr(xq),
                                    _ptr(xs), ld, _ptr(row_id_map), _ptr(sorted_slot), _ptr(tpe),
                                    _ptr(ws), ws_bytes, _ptr(dev_err), _stream(dev)),
           "moe_permute_mx")
    return xq, xs, row_id_map, sorted_slot, tpe


def _mx_pair(q, s, name):
    _dev(q, name + " codes", torch.uint8)
    _dev(s, name + " scales", torch.uint8)
    if tuple(q.shape[:-1]) != tuple(s.shape[:-1]):
        raise MoeError(f"{name}: codes and scales disagree on the row shape")
    return q.shape[-1], s.shape[-1]


def gmm_mx_fwd(xq, xs, wq, wsc, group_list, *, out=None, dev_err=None):
    """y[rows_e] = DQ(x)[rows_e] @ DQ(w[e])^T with w stored [E, N, K]; bf16 y."""
    K, ld_x = _mx_pair(xq, xs, "x")
    K2, ld_w = _mx_pair(wq, wsc, "w")
    _dev(group_list, "group_list", torch.int64)
    M = xq.shape[0]
    E, N, _ = wq.shape
    if K2 != K or group_list.shape[0] != E:
        raise MoeError("shape mismatch: x [M, K], w [E, N, K], group_list [E]")
    y = _out(out, (M, N), torch.bfloat16, xq.device, "y")
    _check(library().gmm_mx_fwd(_ptr(xq), _ptr(xs), ld_x, _ptr(wq), _ptr(wsc), ld_w,
                                _ptr(group_list), E, M, K, N, _ptr(y), _ptr(dev_err),
                                _stream(xq.device)), "gmm_mx_fwd")
    return y


def gmm_mx_fwd_swiglu(xq, xs, w1q, w1s, group_list, *, out=None, dev_err=None):
    """GMM1 + SwiGLU + Q_MX: returns (aq [M, I], as [M, mx_scale_ld(I)]) with
    w1 stored [E, 2I, K] (gate rows, then up rows)."""
    K, ld_x = _mx_pair(xq, xs, "x")
    K2, ld_w = _mx_pair(w1q, w1s, "w1")
    _dev(group_list, "group_list", torch.int64)
    M = xq.shape[0]
    E, N2, _ = w1q.shape
    if K2 != K or group_list.shape[0] != E or N2 % 2:
        raise MoeError("shape mismatch: x [M, K], w1 [E, 2I, K], group_list [E]")
    I = N2 // 2
    ld_a = mx_scale_ld(I)
    if out is None:
        out = (None, None)
    aq = _out(out[0], (M, I), torch.uint8, xq.device, "aq")
    asc = _out(out[1], (M, ld_a), torch.uint8, xq.device, "as")
    _check(library().gmm_mx_fwd_swiglu(_ptr(xq), _ptr(xs), ld_x, _ptr(w1q), _ptr(w1s), ld_w,
                                       _ptr(group_list), E, M, K, I, _ptr(aq), _ptr(asc), ld_a,
                                       _ptr(dev_err), _stream(xq.device)), "gmm_mx_fwd_swiglu")
    return aq, asc


def gmm_mx_fwd_swiglu_gather(xq, xs, sorted_slot, top_k: int, w1q, w1s, group_list, *, out=None,
                             dev_err=None):
    """gmm_mx_fwd_swiglu on the token rows (xq, xs) [T, ...] read through
    sorted_slot (grouped row r = token sorted_slot[r] // top_k); returns
    (aq [M, I], as [M, mx_scale_ld(I)]) with M = len(sorted_slot)."""
    K, ld_x = _mx_pair(xq, xs, "x")
    K2, ld_w = _mx_pair(w1q, w1s, "w1")
    _dev(sorted_slot, "sorted_slot", torch.int32)
    _dev(group_list, "group_list", torch.int64)
    if sorted_slot.dim() != 1:
        raise MoeError("sorted_slot must be [M_cap]")
    T, M = xq.shape[0], sorted_slot.shape[0]
    E, N2, _ = w1q.shape
    if K2 != K or group_list.shape[0] != E or N2 % 2:
        raise MoeError("shape mismatch: x [T, K], w1 [E, 2I, K], group_list [E]")
    I = N2 // 2
    ld_a = mx_scale_ld(I)
    if out is None:
        out = (None, None)
    aq = _out(out[0], (M, I), torch.uint8, xq.device, "aq")
    asc = _out(out[1], (M, ld_a), torch.uint8, xq.device, "as")
    _check(library().gmm_mx_fwd_swiglu_gather(_ptr(xq), _ptr(xs), ld_x, _ptr(sorted_slot), T, int(top_k),
                                              _ptr(w1q), _ptr(w1s), ld_w, _ptr(group_list), E, M, K, I,
                                              _ptr(aq), _ptr(asc), ld_a, _ptr(dev_err), _stream(xq.device)),
           "gmm_mx_fwd_swiglu_gather")
    return aq, asc
