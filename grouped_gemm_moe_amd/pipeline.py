"""The routed-expert MoE layer as a chain of C-ABI calls on preallocated buffers.

Forward ("NPU Training Operators - GMM", section "Qwen3.5 MoE 路径"):
    moe_permute -> gmm_fwd(W1) -> swiglu -> gmm_fwd(W2) -> moe_unpermute
or, fused, moe_permute -> gmm_fwd_swiglu(W1) -> gmm_fwd(W2) -> moe_unpermute
(H written only when a backward will need it).  A forward-only layer can
also skip the permuted copy of x (gather_rows=True; "MegaMoE", 功能说明:
dispatch fused with the first linear layer): moe_permute_index computes the
maps only and the gate_up GMM reads token rows through sorted_slot
(gmm_fwd_gather / gmm_fwd_swiglu_gather), with bit-identical results.
Backward of the expert block, from the gradient dYp at the down-GMM output
(permuted row order):
    dA = gmm_bwd_input(dYp, W2); dW2 = gmm_bwd_weight(A, dYp);
    dH = swiglu_bwd(dA, H);      dX  = gmm_bwd_input(dH, W1);
    dW1 = gmm_bwd_weight(X_perm, dH)
each input/weight gradient pair as one gmm_bwd launch (same bits), and by
default the first pair with the SwiGLU backward in the same launch
(gmm_bwd_swiglu: dH from dA before rounding; dA is not stored).

Backward of the whole layer from dout (the gradient at the layer output):
    dYp, dprobs = moe_unpermute_bwd(dout, Yp, probs); the expert block as
    above; dx = moe_permute_bwd(dX_perm)

Memory-optimised backward (low_memory=True; "03 · grouped GEMM 路径",
section 4: recompute the activation in the backward instead of keeping it,
write gradients into dead buffers): the forward's A is not kept; the
backward recomputes A = swiglu(H) into the dead Yp buffer, writes dA into
A's buffer, dH over H (swiglu_bwd in place) and dX over X_perm (after dW1
has read it, so that pair runs as two launches).  No dA, dH or dX buffer is allocated: S*(I + 2I + H) bf16
elements fewer, for one extra swiglu pass.

The A8W8-FP (MXFP8) forward ("MegaMoE", A8W8-FP scenario), MoeLayerMX:
    moe_permute_mx (gather + Q_MX) -> gmm_mx_fwd_swiglu(W1; GMM1, SwiGLU and
    Q_MX of A in one call) -> gmm_mx_fwd(W2) -> moe_unpermute
or, with gather_rows=True, mx_quantize of the T token rows -> moe_permute_index
-> gmm_mx_fwd_swiglu_gather (GMM1 reads the quantised token rows through
sorted_slot) -> gmm_mx_fwd(W2) -> moe_unpermute, bit-identical.

Every step runs in the HIP kernels of libmoegmm; this module only owns the
buffers and the call order.  group_list (tokens_per_expert) stays on the
device between the calls.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (gmm_bwd, gmm_bwd_input, gmm_bwd_swiglu, gmm_bwd_weight, gmm_fwd, gmm_fwd_gather, gmm_fwd_swiglu,
               gmm_fwd_swiglu_gather, gmm_mx_fwd, gmm_mx_fwd_swiglu, gmm_mx_fwd_swiglu_gather,
               gmm_workspace_size, moe_decode_fwd, moe_decode_fwd_mx, moe_permute,
               moe_permute_bwd, moe_permute_index, moe_permute_mx, moe_permute_workspace_size, moe_unpermute,
               moe_unpermute_bwd, mx_quantize, mx_scale_ld, swiglu, swiglu_bwd, swiglu_gmm_fwd)


@dataclass
class LayerShape:
    T: int
    top_k: int
    E: int
    H: int
    I: int

    @property
    def S(self) -> int:
        return self.T * self.top_k


class MoeLayer:
    """Buffers for one layer shape; forward() and backward() enqueue on the
    current torch stream and never synchronise."""

    def __init__(self, shape: LayerShape, device, with_backward: bool = False,
                 low_memory: bool = False, fuse_swiglu_bwd: bool = True, gather_rows: bool = False):
        s = shape
        self.shape = s
        # forward only: the gate_up GMM reads token rows through sorted_slot
        # and no permuted copy of x is made (the W1 gradient would need one)
        self.gather_rows = bool(gather_rows)
        if self.gather_rows and with_backward:
            raise ValueError("gather_rows is forward-only: the W1 weight gradient reads X_perm")
        self.x_tokens = None
        self.low_memory = bool(low_memory and with_backward)
        # dH straight from the down GMM's backward (gmm_bwd_swiglu): dA is
        # neither rounded nor stored, and no separate swiglu_bwd runs
        self.fuse_swiglu_bwd = bool(fuse_swiglu_bwd)
        d = device
        bf = torch.bfloat16
        S = s.S
        self.x_perm = None if self.gather_rows else torch.empty((S, s.H), dtype=bf, device=d)
        self.row_id_map = torch.empty(S, dtype=torch.int32, device=d)
        self.sorted_slot = torch.empty(S, dtype=torch.int32, device=d)
        self.tokens_per_expert = torch.empty(s.E, dtype=torch.int64, device=d)
        self.h = torch.empty((S, 2 * s.I), dtype=bf, device=d)
        self.a = torch.empty((S, s.I), dtype=bf, device=d)
        self.yp = torch.empty((S, s.H), dtype=bf, device=d)
        self.out = torch.empty((s.T, s.H), dtype=bf, device=d)
        self.dev_err = torch.zeros(1, dtype=torch.int32, device=d)
        self.ws_perm = torch.empty(max(1, moe_permute_workspace_size(s.T, s.top_k, s.E)),
                                   dtype=torch.uint8, device=d)
        ws = max(gmm_workspace_size(s.E, S, k, n, op)
                 for (k, n) in ((s.H, 2 * s.I), (s.I, s.H)) for op in (0, 1, 2, 3))
        # tile queues: zero-filled once, left zero-filled by every call
        self.ws_gmm = torch.zeros(ws, dtype=torch.uint8, device=d) if ws > 0 else None
        if with_backward and self.low_memory:
            # gradients live in dead forward buffers (see the module docstring)
            self.da = self.a
            self.dh = self.h
            self.dx = self.x_perm
            self.a_recomputed = self.yp.view(-1)[: S * s.I].view(S, s.I)
        elif with_backward:
            self.da = None if self.fuse_swiglu_bwd else torch.empty((S, s.I), dtype=bf, device=d)
            self.dh = torch.empty((S, 2 * s.I), dtype=bf, device=d)
            self.dx = torch.empty((S, s.H), dtype=bf, device=d)
        if with_backward:
            self.dw1 = torch.empty((s.E, s.H, 2 * s.I), dtype=bf, device=d)
            self.dw2 = torch.empty((s.E, s.I, s.H), dtype=bf, device=d)
            self.dyp = torch.empty((S, s.H), dtype=bf, device=d)
            self.dprobs = torch.empty((s.T, s.top_k), dtype=torch.float32, device=d)
            self.dx_tokens = torch.empty((s.T, s.H), dtype=bf, device=d)

    # -- forward ---------------------------------------------------------
    def permute(self, x, topk_ids):
        if self.gather_rows:
            self.x_tokens = x
            moe_permute_index(topk_ids, self.shape.E, ws=self.ws_perm, dev_err=self.dev_err,
                              out=(self.row_id_map, self.sorted_slot, self.tokens_per_expert))
            return
        moe_permute(x, topk_ids, self.shape.E, ws=self.ws_perm, dev_err=self.dev_err,
                    out=(self.x_perm, self.row_id_map, self.sorted_slot, self.tokens_per_expert))

    def gate_up(self, w1, fused, keep_h=True):
        """The gate_up GMM of the rows permute() grouped: A (and H when
        keep_h) if fused, else H only."""
        g, ws, err = self.tokens_per_expert, self.ws_gmm, self.dev_err
        h = self.h if keep_h else None
        if self.gather_rows:
            x, slot, k = self.x_tokens, self.sorted_slot, self.shape.top_k
            if fused:
                gmm_fwd_swiglu_gather(x, slot, k, w1, g, out=self.a, h_out=h, ws=ws, dev_err=err)
            else:
                gmm_fwd_gather(x, slot, k, w1, g, out=self.h, ws=ws, dev_err=err)
        elif fused:
            gmm_fwd_swiglu(self.x_perm, w1, g, out=self.a, h_out=h, ws=ws, dev_err=err)
        else:
            gmm_fwd(self.x_perm, w1, g, out=self.h, ws=ws, dev_err=err)

    def use_fused(self, fused) -> bool:
        """fused="auto": the fused gate_up + SwiGLU call unless the shape is
        decode-like (at most 8 rows per expert), where the weight-streaming
        gate_up followed by swiglu measures faster."""
        if fused == "auto":
            return self.shape.S > 8 * self.shape.E
        return bool(fused)

    def experts_forward(self, w1, w2, fused=False, keep_h=True):
        """fused: one gate_up GMM + SwiGLU call writes A (and H only when
        keep_h, as the backward needs it); otherwise gate_up GMM -> H, then
        SwiGLU and the down GMM in one swiglu_gmm_fwd call (A written too).
        fused may be "auto" (see use_fused)."""
        g = self.tokens_per_expert
        if self.use_fused(fused):
            self.gate_up(w1, True, keep_h)
            gmm_fwd(self.a, w2, g, out=self.yp, ws=self.ws_gmm, dev_err=self.dev_err)
        else:
            self.gate_up(w1, False)
            # SwiGLU and the down GMM: one launch on weight-streaming shapes
            swiglu_gmm_fwd(self.h, w2, g, out=(self.a, self.yp), dev_err=self.dev_err)

    def unpermute(self, probs):
        moe_unpermute(self.yp, self.row_id_map, probs, out=self.out, dev_err=self.dev_err)

    def decode_applies(self) -> bool:
        """Whether forward_decode takes this shape: a few rows per expert
        (at most 8 slots per expert, at most 16384 slots) and H, I <= 4096."""
        s = self.shape
        return s.S <= 8 * s.E and s.S <= 16384 and s.H <= 4096 and s.I <= 4096

    def forward_decode(self, x, topk_ids, probs, w1, w2):
        """The same forward with the routing fused into the gate_up GMM
        (moe_decode_fwd: no permute launch).  Fills the same buffers as
        forward(..., fused=False) with a gather_rows layer, bit for bit."""
        self.x_tokens = x
        moe_decode_fwd(x, topk_ids, probs, w1, w2,
                       out=(self.out, self.row_id_map, self.sorted_slot, self.tokens_per_expert, self.h,
                            self.a, self.yp),
                       dev_err=self.dev_err)
        return self.out

    def forward(self, x, topk_ids, probs, w1, w2, fused=False, keep_h=True):
        self.permute(x, topk_ids)
        self.experts_forward(w1, w2, fused=fused, keep_h=keep_h)
        self.unpermute(probs)
        return self.out

    # -- backward of the expert block --------------------------------------
    def backward(self, dyp, w1, w2):
        """dYp -> dA, dW2, dH, dX_perm, dW1.  With low_memory, A is
        recomputed from H first, Yp, A, H and X_perm are overwritten, and
        dyp must not be the Yp buffer."""
        g = self.tokens_per_expert
        ws, err = self.ws_gmm, self.dev_err
        if self.low_memory:
            a = self.a_recomputed
            swiglu(self.h, g, out=a)
            if self.fuse_swiglu_bwd:
                # dH written over H in the same launch (each tile reads G, U first)
                gmm_bwd_swiglu(a, dyp, w2, self.h, g, dh_out=self.dh, dw_out=self.dw2, ws=ws, dev_err=err)
            else:
                # dA goes to A's buffer, which this pair does not read (A is in Yp's)
                gmm_bwd(a, dyp, w2, g, dx_out=self.da, dw_out=self.dw2, ws=ws, dev_err=err)
                swiglu_bwd(self.da, self.h, g, out=self.dh)  # in place over H
            gmm_bwd_weight(self.x_perm, self.dh, g, out=self.dw1, ws=ws, dev_err=err)
            gmm_bwd_input(self.dh, w1, g, out=self.dx, ws=ws, dev_err=err)
            return
        if self.fuse_swiglu_bwd:
            gmm_bwd_swiglu(self.a, dyp, w2, self.h, g, dh_out=self.dh, dw_out=self.dw2, ws=ws, dev_err=err)
        else:
            gmm_bwd(self.a, dyp, w2, g, dx_out=self.da, dw_out=self.dw2, ws=ws, dev_err=err)
            swiglu_bwd(self.da, self.h, g, out=self.dh)
        gmm_bwd(self.x_perm, self.dh, w1, g, dx_out=self.dx, dw_out=self.dw1, ws=ws, dev_err=err)

    # -- one training step of the expert block, call by call ----------------
    def training_step_calls(self, x, topk_ids, probs, dyp, w1, w2):
        """The forward and the expert-block backward from dYp as (name, call)
        pairs in launch order, so that a caller can time each call:
        permute -> gate_up GMM + SwiGLU (H kept) -> down GMM -> unpermute ->
        down pair with the SwiGLU backward (dH, dW2) -> gate_up pair (dX,
        dW1).  The same launches as forward(fused=True, keep_h=True)
        followed by backward(dyp) with the fused SwiGLU backward."""
        if self.low_memory or not self.fuse_swiglu_bwd or not hasattr(self, "dw1"):
            raise ValueError("training_step_calls needs with_backward=True, low_memory=False and "
                             "fuse_swiglu_bwd=True")
        g, ws, err = self.tokens_per_expert, self.ws_gmm, self.dev_err
        return [
            ("moe_permute", lambda: self.permute(x, topk_ids)),
            ("gmm_fwd_swiglu", lambda: gmm_fwd_swiglu(self.x_perm, w1, g, out=self.a, h_out=self.h,
                                                      ws=ws, dev_err=err)),
            ("gmm_fwd_down", lambda: gmm_fwd(self.a, w2, g, out=self.yp, ws=ws, dev_err=err)),
            ("moe_unpermute", lambda: self.unpermute(probs)),
            ("gmm_bwd_swiglu_down", lambda: gmm_bwd_swiglu(self.a, dyp, w2, self.h, g, dh_out=self.dh,
                                                           dw_out=self.dw2, ws=ws, dev_err=err)),
            ("gmm_bwd_gate_up", lambda: gmm_bwd(self.x_perm, self.dh, w1, g, dx_out=self.dx,
                                                dw_out=self.dw1, ws=ws, dev_err=err)),
        ]

    # -- backward of the two ends and of the whole layer --------------------
    def unpermute_backward(self, dout, probs):
        moe_unpermute_bwd(dout, self.yp, self.row_id_map, probs, out=(self.dyp, self.dprobs),
                          dev_err=self.dev_err)

    def permute_backward(self):
        moe_permute_bwd(self.dx, self.row_id_map, self.shape.T, out=self.dx_tokens,
                        dev_err=self.dev_err)

    def backward_full(self, dout, probs, w1, w2):
        """dout -> (dx_tokens, dprobs, dw1, dw2), every intermediate kept."""
        self.unpermute_backward(dout, probs)
        self.backward(self.dyp, w1, w2)
        self.permute_backward()


class MoeLayerMX:
    """Buffers for the A8W8-FP forward of one layer shape.  Weights are MX
    pairs (codes, scales) stored reduction-contiguous: W1 as [E, 2I, H] (gate
    rows, then up rows), W2 as [E, H, I]; prepare_weights builds them from
    the bf16 [E, H, 2I] / [E, I, H] weights."""

    def __init__(self, shape: LayerShape, device, gather_rows: bool = False):
        s = shape
        self.shape = s
        d = device
        u8 = dict(dtype=torch.uint8, device=d)
        S = s.S
        # gather_rows: the token rows are quantised once ([T, H]) and GMM1
        # reads them through sorted_slot; else the permute writes the
        # quantised rows of every slot ([S, H])
        self.gather_rows = bool(gather_rows)
        rows = s.T if self.gather_rows else S
        self.xq = torch.empty((rows, s.H), **u8)
        self.xs = torch.empty((rows, mx_scale_ld(s.H)), **u8)
        self.aq = torch.empty((S, s.I), **u8)
        self.as_ = torch.empty((S, mx_scale_ld(s.I)), **u8)
        self.row_id_map = torch.empty(S, dtype=torch.int32, device=d)
        self.sorted_slot = torch.empty(S, dtype=torch.int32, device=d)
        self.tokens_per_expert = torch.empty(s.E, dtype=torch.int64, device=d)
        self.yp = torch.empty((S, s.H), dtype=torch.bfloat16, device=d)
        self.out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=d)
        self.dev_err = torch.zeros(1, dtype=torch.int32, device=d)
        self.ws_perm = torch.empty(max(1, moe_permute_workspace_size(s.T, s.top_k, s.E)),
                                   dtype=torch.uint8, device=d)

    @staticmethod
    def prepare_weights(w1, w2):
        """bf16 W1 [E, H, 2I] and W2 [E, I, H] -> MX pairs of W1^T [E, 2I, H]
        and W2^T [E, H, I] (the transposes are copies made once, off the
        path; Q_MX runs in the library)."""
        return (mx_quantize(w1.transpose(1, 2).contiguous()),
                mx_quantize(w2.transpose(1, 2).contiguous()))

    def forward(self, x, topk_ids, probs, w1mx, w2mx):
        (w1q, w1s), (w2q, w2s) = w1mx, w2mx
        g = self.tokens_per_expert
        if self.gather_rows:
            mx_quantize(x, out=(self.xq, self.xs))
            moe_permute_index(topk_ids, self.shape.E, ws=self.ws_perm, dev_err=self.dev_err,
                              out=(self.row_id_map, self.sorted_slot, g))
            gmm_mx_fwd_swiglu_gather(self.xq, self.xs, self.sorted_slot, self.shape.top_k, w1q, w1s, g,
                                     out=(self.aq, self.as_), dev_err=self.dev_err)
        else:
            moe_permute_mx(x, topk_ids, self.shape.E, ws=self.ws_perm, dev_err=self.dev_err,
                           out=(self.xq, self.xs, self.row_id_map, self.sorted_slot, g))
            gmm_mx_fwd_swiglu(self.xq, self.xs, w1q, w1s, g, out=(self.aq, self.as_),
                              dev_err=self.dev_err)
        gmm_mx_fwd(self.aq, self.as_, w2q, w2s, g, out=self.yp, dev_err=self.dev_err)
        moe_unpermute(self.yp, self.row_id_map, probs, out=self.out, dev_err=self.dev_err)
        return self.out

    def forward_decode(self, x, topk_ids, probs, w1mx, w2mx):
        """The same forward (gather_rows=True buffers) with the routing fused
        into GMM1 (moe_decode_fwd_mx: no permute launch), bit for bit."""
        if not self.gather_rows:
            raise ValueError("forward_decode reads the quantised token rows: build with gather_rows=True")
        (w1q, w1s), (w2q, w2s) = w1mx, w2mx
        mx_quantize(x, out=(self.xq, self.xs))
        moe_decode_fwd_mx(self.xq, self.xs, topk_ids, probs, w1q, w1s, w2q, w2s,
                          out=(self.out, self.row_id_map, self.sorted_slot, self.tokens_per_expert, self.aq,
                               self.as_, self.yp),
                          dev_err=self.dev_err)
        return self.out
