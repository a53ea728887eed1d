"""gmm_fwd / gmm_bwd_input / gmm_bwd_weight on the GPU vs the oracle.

Tolerance: rtol = atol = 1e-2 elementwise (the bf16 fused-vs-eager tolerance
of "NPU Training Operators - GMM", conclusions and verification table).
Only rows < R = sum(group_list) are compared; rows >= R must stay untouched.
"""
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


def _gl(dev, gl):
    return torch.from_numpy(np.asarray(gl, dtype=np.int64)).to(dev)


def _sentinel(dev, shape):
    return bf16_dev(np.full(shape, SENT, dtype=np.uint16), dev)


def run_all(dev, x_bits, w_bits, dy_bits, gl, tag):
    """Run fwd, dX and dW; return host arrays (float64) and the error word."""
    M, K = x_bits.shape
    E, _, N = w_bits.shape
    print(f"gmm {tag}: E={E} M={M} K={K} N={N} R={int(np.sum(gl))}", flush=True)
    x, w, dy, g = bf16_dev(x_bits, dev), bf16_dev(w_bits, dev), bf16_dev(dy_bits, dev), _gl(dev, gl)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    y = moe.gmm_fwd(x, w, g, out=_sentinel(dev, (M, N)), dev_err=err)
    dx = moe.gmm_bwd_input(dy, w, g, out=_sentinel(dev, (M, K)), dev_err=err)
    dw = moe.gmm_bwd_weight(x, dy, g, out=_sentinel(dev, (E, K, N)), dev_err=err)
    # both gradients in one launch: the same bits, rows >= R untouched
    dx2, dw2 = moe.gmm_bwd(x, dy, w, g, dx_out=_sentinel(dev, (M, K)), dw_out=_sentinel(dev, (E, K, N)),
                           dev_err=err)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits(dx2), dev_bits(dx)), f"{tag}: gmm_bwd dx differs from gmm_bwd_input"
    if moe.gmm_workspace_size(E, M, K, N, moe.OP_BWD_WEIGHT) > moe.GMM_QUEUE_BYTES:
        # few tiles: gmm_bwd_weight splits the row reduction (another fp32
        # summation order than gmm_bwd's whole-range tiles); both vs the oracle
        ref = oracle.gmm_bwd_weight(f64(x_bits), f64(dy_bits), gl)
        assert_close(f64(dev_bits(dw2)), ref, f"{tag} gmm_bwd dW")
    else:
        assert np.array_equal(dev_bits(dw2), dev_bits(dw)), f"{tag}: gmm_bwd dw differs from gmm_bwd_weight"
    return dev_bits(y), dev_bits(dx), dev_bits(dw), int(err.item())


def check_all(dev, x_bits, w_bits, dy_bits, gl, tag):
    y, dx, dw, err = run_all(dev, x_bits, w_bits, dy_bits, gl, tag)
    assert err == 0
    R = int(np.sum(gl))
    x, w, dy = f64(x_bits), f64(w_bits), f64(dy_bits)
    assert_close(f64(y)[:R], oracle.gmm(x, w, gl)[:R], f"{tag} fwd")
    assert_close(f64(dx)[:R], oracle.gmm_bwd_input(dy, w, gl)[:R], f"{tag} dX")
    assert_close(f64(dw), oracle.gmm_bwd_weight(x, dy, gl), f"{tag} dW")
    assert (y[R:] == SENT).all() and (dx[R:] == SENT).all(), f"{tag}: rows >= R were written"
    for e in np.nonzero(np.asarray(gl) == 0)[0]:
        assert (dw[e] == 0).all(), f"{tag}: dW of empty expert {e} not exactly zero"


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_sweep(dev, variant):
    wl = workloads.sweep(variant)
    check_all(dev, wl["x"], wl["w"], wl["dy"], wl["group_list"], f"sweep{variant}")


def test_worked_example_shapes(dev):
    wl = workloads.tiny()
    rng = np.random.default_rng(0)
    x = workloads.normal_bf16(rng, (5, 64))
    dy = workloads.normal_bf16(rng, (5, 64))
    check_all(dev, x, wl["w1"], dy, [1, 2, 0, 2], "tiny")


@pytest.mark.parametrize("M,K,N,gl", [
    (300, 200, 136, [300]),                   # E=1: dense, ragged tiles in every dim
    (777, 72, 264, [0, 777, 0]),              # all rows in one expert
    (513, 520, 128, [1, 0, 255, 0, 0, 257]),  # group sizes around the tile size
    (129, 8, 8, [64, 1, 64]),                 # tiny K and N
    (64, 4096, 64, [31, 33]),                 # long reduction, short everything else
])
def test_ragged_shapes(dev, M, K, N, gl):
    rng = np.random.default_rng(M + K + N)
    E = len(gl)
    x = workloads.normal_bf16(rng, (M, K))
    w = workloads.normal_bf16(rng, (E, K, N), 0.05)
    dy = workloads.normal_bf16(rng, (M, N))
    check_all(dev, x, w, dy, np.array(gl, dtype=np.int64), f"ragged{M}x{K}x{N}")


def test_max_experts(dev):
    """E = 1024 (the API limit): the schedules scan 1024 counts and the
    weight gradient ranks all 1024 experts."""
    rng = np.random.default_rng(1024)
    E, M, K, N = 1024, 3000, 64, 136
    gl = workloads.random_group_list(rng, M, E, empty_frac=0.7, fill=0.95)
    x = workloads.normal_bf16(rng, (M, K))
    w = workloads.normal_bf16(rng, (E, K, N), 0.05)
    dy = workloads.normal_bf16(rng, (M, N))
    check_all(dev, x, w, dy, gl, "E1024")


def test_max_reduction_length(dev):
    """K = 2^21 (the API limit: 256 rows of 2^21 bf16 still fit the 32-bit
    buffer offsets): one forward tile runs 65536 reduction steps, the weight
    gradient has 8192 k-tiles, the input gradient 8192 column tiles."""
    rng = np.random.default_rng(21)
    E, M, K, N = 2, 64, 1 << 21, 8
    gl = np.array([40, 24], dtype=np.int64)
    x = workloads.normal_bf16(rng, (M, K))
    w = workloads.normal_bf16(rng, (E, K, N), 0.01)
    dy = workloads.normal_bf16(rng, (M, N))
    check_all(dev, x, w, dy, gl, "K=2^21")


def test_rows_beyond_R_hold_nan(dev):
    """Capacity rows past R are undefined memory: NaN there must not leak."""
    rng = np.random.default_rng(3)
    M, K, N = 640, 256, 192
    gl = np.array([100, 0, 200, 57], dtype=np.int64)
    R = int(gl.sum())
    x = workloads.normal_bf16(rng, (M, K))
    dy = workloads.normal_bf16(rng, (M, N))
    x[R:] = SENT
    dy[R:] = SENT
    w = workloads.normal_bf16(rng, (4, K, N), 0.05)
    check_all(dev, x, w, dy, gl, "nan-tail")


def test_empty_expert_weights_never_read(dev):
    rng = np.random.default_rng(4)
    M, K, N = 512, 128, 256
    gl = np.array([0, 200, 0, 0, 312, 0], dtype=np.int64)
    x = workloads.normal_bf16(rng, (M, K))
    dy = workloads.normal_bf16(rng, (M, N))
    w = workloads.normal_bf16(rng, (6, K, N), 0.05)
    w[gl == 0] = SENT
    y, dx, dw, err = run_all(dev, x, w, dy, gl, "nan-empty-weights")
    assert err == 0
    wf = f64(w)
    wf[gl == 0] = 0.0
    assert_close(f64(y), oracle.gmm(f64(x), wf, gl), "fwd with NaN empty weights")
    assert_close(f64(dx), oracle.gmm_bwd_input(f64(dy), wf, gl), "dX with NaN empty weights")
    assert (dw[gl == 0] == 0).all()


def test_all_experts_empty(dev):
    rng = np.random.default_rng(5)
    M, K, N = 128, 64, 64
    gl = np.zeros(4, dtype=np.int64)
    x = workloads.normal_bf16(rng, (M, K))
    dy = workloads.normal_bf16(rng, (M, N))
    w = workloads.normal_bf16(rng, (4, K, N))
    y, dx, dw, err = run_all(dev, x, w, dy, gl, "all-empty")
    assert err == 0 and (y == SENT).all() and (dx == SENT).all() and (dw == 0).all()


@pytest.mark.parametrize("skew", [False, True])
def test_decode_shaped_forward(dev, skew):
    """E=256, 512 rows: the weight-streaming forward."""
    wl = workloads.decode(with_weights=True)
    gl = oracle.tokens_per_expert(wl["topk_ids"], 256)
    if skew:  # one expert with many rows (several streaming passes)
        gl = gl.copy()
        gl[17] += 40
        gl[200] = 0
    M = int(gl.sum()) + 7
    rng = np.random.default_rng(6)
    x = workloads.normal_bf16(rng, (M, 2048))
    print(f"decode fwd skew={skew} R={int(gl.sum())}", flush=True)
    y = moe.gmm_fwd(bf16_dev(x, dev), bf16_dev(wl["w1"], dev), _gl(dev, gl),
                    out=_sentinel(dev, (M, 1024)))
    y2 = moe.gmm_fwd(bf16_dev(x[:, :512].copy(), dev), bf16_dev(wl["w2"], dev), _gl(dev, gl),
                     out=_sentinel(dev, (M, 2048)))
    torch.cuda.synchronize()
    R = int(gl.sum())
    assert_close(dev_f64(y)[:R], oracle.gmm(f64(x), f64(wl["w1"]), gl)[:R], "decode gate_up")
    assert_close(dev_f64(y2)[:R], oracle.gmm(f64(x[:, :512]), f64(wl["w2"]), gl)[:R], "decode down")
    assert (dev_bits(y)[R:] == SENT).all()


@pytest.mark.parametrize("M", [256, 1024])
def test_group_list_errors_reported(dev, M):
    """sum(group_list) > M_cap and negative counts set the error bit; the
    kernels clamp to the buffer, so the call itself is safe.  At M = 1024 the
    weight gradient's 3 tiles take the split-row path (4 chunks)."""
    rng = np.random.default_rng(7)
    K, N = 64, 64
    x = bf16_dev(workloads.normal_bf16(rng, (M, K)), dev)
    dy = bf16_dev(workloads.normal_bf16(rng, (M, N)), dev)
    w = bf16_dev(workloads.normal_bf16(rng, (3, K, N)), dev)
    split = moe.gmm_workspace_size(3, M, K, N, moe.OP_BWD_WEIGHT) > moe.GMM_QUEUE_BYTES
    assert split == (M == 1024)
    over = [M - 56, 100, 10]  # sum past M_cap
    for gl in (over, [-5, 100, 10], [0, 0, 4 * M]):
        print(f"group_list error case {gl}", flush=True)
        for fn in ("fwd", "dx", "dw"):
            err = torch.zeros(1, dtype=torch.int32, device=dev)
            g = _gl(dev, gl)
            if fn == "fwd":
                moe.gmm_fwd(x, w, g, dev_err=err)
            elif fn == "dx":
                moe.gmm_bwd_input(dy, w, g, dev_err=err)
            else:
                moe.gmm_bwd_weight(x, dy, g, dev_err=err)
            torch.cuda.synchronize()
            assert int(err.item()) & moe.DEVERR_GROUP_LIST, (gl, fn)


def test_deterministic_repeat(dev):
    wl = workloads.sweep(1)
    a = run_all(dev, wl["x"], wl["w"], wl["dy"], wl["group_list"], "repeat-a")
    b = run_all(dev, wl["x"], wl["w"], wl["dy"], wl["group_list"], "repeat-b")
    for u, v in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(u, v)


# ---------------------------------------------------------------------------
# full size: one expert-parallel rank's share (E=32, H=4096, I=1536, 16384
# rows, Zipf group sizes with empty experts), sampled outputs computed by the
# oracle one row / one weight row at a time
# ---------------------------------------------------------------------------


def _sample_rows(gl, rng, per_expert=3):
    off = oracle.expert_offsets(gl)
    rows = []
    for e in range(len(gl)):
        if gl[e] == 0:
            continue
        rows += [off[e], off[e + 1] - 1]
        rows += list(rng.integers(off[e], off[e + 1], per_expert))
    return np.unique(np.array(rows, dtype=np.int64))


def _expert_of(gl):
    return np.repeat(np.arange(len(gl)), gl)


def test_half_height_tiles_prefill_groups(dev):
    """The prefill routing (128 experts of ~256 rows): the forward and
    input-gradient launches take an expert's last rows into its last full
    tile (tall tiles, at most 64 rows past it) where that removes a tile
    round -- here the [32768, 512] x [512, 2048] forward and the input
    gradient with 2048 output columns -- while gmm_bwd's queue runs them as
    half-height tiles.  Sampled rows (every expert's first and last rows among
    them) against the oracle, and bit-equality of the two shapes' dX."""
    wl = workloads.prefill(with_weights=False)
    gl = oracle.tokens_per_expert(wl["topk_ids"], 128)
    R, E, K, N = int(gl.sum()), 128, 512, 2048
    rng = np.random.default_rng(77)
    a_b = workloads.normal_bf16(rng, (R, K))
    w_b = workloads.normal_bf16(rng, (E, K, N), std=0.02)
    g = _gl(dev, gl)
    a, w = bf16_dev(a_b, dev), bf16_dev(w_b, dev)
    # [E, N, K]: the input gradient a @ wt[e]^T has N = 2048 output columns
    # over a reduction of K = 512, and equals a @ w[e]
    wt = w.transpose(1, 2).contiguous()
    print("half-height tiles: fwd [32768,512]x[512,2048], dX with 2048 output columns", flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    y = moe.gmm_fwd(a, w, g, dev_err=err)                 # [R, 2048]
    dx = moe.gmm_bwd_input(a, wt, g, dev_err=err)         # [R, 2048]
    ws = torch.zeros(moe.gmm_workspace_size(E, R, N, K, moe.OP_BWD), dtype=torch.uint8, device=dev)
    dx2, _ = moe.gmm_bwd(y, a, wt, g, ws=ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(dx2.view(torch.int16), dx.view(torch.int16)), "gmm_bwd dx != gmm_bwd_input"
    rows = _sample_rows(gl, rng, per_expert=1)
    eo = _expert_of(gl)
    ridx = torch.from_numpy(rows).to(dev)
    y_s, dx_s = dev_f64(y[ridx]), dev_f64(dx[ridx])
    wf = f64(w_b)
    for i, r in enumerate(rows):
        ref = f64(a_b[r]) @ wf[eo[r]]
        assert_close(y_s[i], ref, f"fwd row {r}")
        assert_close(dx_s[i], ref, f"dX row {r}")


def _check_rows(dev, a_b, w_b, gl, outs, rng, tag):
    """Sampled rows of each output in outs (name -> (tensor, weight bits
    [E, K, N] it multiplies by)) against the oracle's row products."""
    rows = _sample_rows(gl, rng, per_expert=1)
    eo = _expert_of(gl)
    ridx = torch.from_numpy(rows).to(dev)
    for name, (t, wb) in outs.items():
        got = dev_f64(t[ridx])
        wf = f64(wb)
        for i, r in enumerate(rows):
            assert_close(got[i], f64(a_b[r]) @ wf[eo[r]], f"{tag} {name} row {r}")


@pytest.mark.parametrize("shape", ["tall", "half"])
def test_tall_and_half_tile_schedules(dev, shape):
    """The static forward / input-gradient schedules at their boundaries.
    tall: 256 experts of 257 .. 320 rows (1 .. 64 past a full tile) with
    256 output columns: tall last tiles halve the tile count (2 rounds -> 1),
    half-height tiles do not.  half: 356 rows each (100 past a full tile:
    no tall tile) with 1024 output columns: half-height tiles take 8 rounds to
    6.  The SwiGLU forward (always tall) on the same rows, its H bit-equal to
    gmm_fwd with the same weights; dX bit-equal to gmm_bwd's (always
    half-height tiles)."""
    E = 256
    if shape == "tall":
        gl = np.array([(257, 280, 300, 320)[e % 4] for e in range(E)], dtype=np.int64)
        K, N = 256, 256
    else:
        gl = np.full(E, 356, dtype=np.int64)
        K, N = 256, 1024
    R = int(gl.sum())
    rng = np.random.default_rng(91)
    a_b = workloads.normal_bf16(rng, (R, K))
    w_b = workloads.normal_bf16(rng, (E, K, N), std=0.02)
    g = _gl(dev, gl)
    a, w = bf16_dev(a_b, dev), bf16_dev(w_b, dev)
    wt = w.transpose(1, 2).contiguous()  # [E, N, K]: a @ wt[e]^T = a @ w[e]
    print(f"tile schedules {shape}: E={E} R={R} K={K} N={N}", flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    y = moe.gmm_fwd(a, w, g, dev_err=err)
    dx = moe.gmm_bwd_input(a, wt, g, dev_err=err)
    ws = torch.zeros(moe.gmm_workspace_size(E, R, N, K, moe.OP_BWD), dtype=torch.uint8, device=dev)
    dx2, _ = moe.gmm_bwd(y, a, wt, g, ws=ws, dev_err=err)
    h = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
    a_sw = moe.gmm_fwd_swiglu(a, w, g, h_out=h, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(dx2.view(torch.int16), dx.view(torch.int16)), "gmm_bwd dx != gmm_bwd_input"
    assert torch.equal(h.view(torch.int16), y.view(torch.int16)), "gmm_fwd_swiglu H != gmm_fwd"
    _check_rows(dev, a_b, w_b, gl, {"fwd": (y, w_b), "dX": (dx, w_b)}, rng, shape)
    # A = SiLU(G) * U from the same rows
    rows = _sample_rows(gl, rng, per_expert=1)
    eo = _expert_of(gl)
    got = dev_f64(a_sw[torch.from_numpy(rows).to(dev)])
    I = N // 2
    wf = f64(w_b)
    for i, r in enumerate(rows):
        gu = f64(a_b[r]) @ wf[eo[r]]
        ref = gu[:I] / (1.0 + np.exp(-gu[:I])) * gu[I:]
        assert_close(got[i], ref, f"{shape} swiglu row {r}")


def test_ep_full_size_sampled(dev):
    wl = workloads.ep_slice()
    gl = wl["group_list"]
    R, E, H, I = 16384, 32, 4096, 1536
    rng = np.random.default_rng(55)
    x_b, dy_b = wl["x"], wl["dyp"]
    dh_b = workloads.normal_bf16(rng, (R, 2 * I))
    g = _gl(dev, gl)
    x, dyp, dh = bf16_dev(x_b, dev), bf16_dev(dy_b, dev), bf16_dev(dh_b, dev)
    w1, w2 = bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev)
    print("ep full size: fwd(W1), dX(W2), dX(W1), dW1", flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    y = moe.gmm_fwd(x, w1, g, dev_err=err)            # [R, 3072]
    da = moe.gmm_bwd_input(dyp, w2, g, dev_err=err)   # [R, 1536]
    dx = moe.gmm_bwd_input(dh, w1, g, dev_err=err)    # [R, 4096]
    dw1 = moe.gmm_bwd_weight(x, dh, g, dev_err=err)   # [32, 4096, 3072]
    # the fused launches at full size: gmm_bwd (input- and weight-gradient
    # tiles from one queue) and the gate_up GMM fused with SwiGLU keeping H
    # give the bits of the separate calls over every element
    ws = torch.zeros(moe.gmm_workspace_size(E, R, H, 2 * I, moe.OP_BWD), dtype=torch.uint8, device=dev)
    dx2, dw1b = moe.gmm_bwd(x, dh, w1, g, ws=ws, dev_err=err)
    a_f, h_f = torch.empty((R, I), dtype=torch.bfloat16, device=dev), torch.empty_like(y)
    moe.gmm_fwd_swiglu(x, w1, g, out=a_f, h_out=h_f, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(dx2.view(torch.int16), dx.view(torch.int16)), "gmm_bwd dx != gmm_bwd_input"
    assert torch.equal(dw1b.view(torch.int16), dw1.view(torch.int16)), "gmm_bwd dw != gmm_bwd_weight"
    assert torch.equal(h_f.view(torch.int16), y.view(torch.int16)), "gmm_fwd_swiglu h != gmm_fwd"
    assert int(ws[:moe.GMM_QUEUE_BYTES].count_nonzero().item()) == 0, "gmm_bwd left its queue non-zero"
    rows = _sample_rows(gl, rng)
    eo = _expert_of(gl)
    xs, w1f, w2f = f64(x_b[rows]), wl["w1"], wl["w2"]
    y_s = dev_f64(y[torch.from_numpy(rows).to(dev)])
    a_s = dev_f64(a_f[torch.from_numpy(rows).to(dev)])  # fused: from the unrounded accumulators
    da_s = dev_f64(da[torch.from_numpy(rows).to(dev)])
    dx_s = dev_f64(dx[torch.from_numpy(rows).to(dev)])
    dys, dhs = f64(dy_b[rows]), f64(dh_b[rows])
    for i, r in enumerate(rows):
        e = eo[r]
        assert_close(y_s[i], xs[i] @ f64(w1f[e]), f"ep fwd row {r}")
        assert_close(a_s[i], oracle.gmm_swiglu(xs[i:i + 1], f64(w1f[e:e + 1]), [1])[0],
                     f"ep fwd+swiglu row {r}")
        assert_close(da_s[i], dys[i] @ f64(w2f[e]).T, f"ep dX(W2) row {r}")
        assert_close(dx_s[i], dhs[i] @ f64(w1f[e]).T, f"ep dX(W1) row {r}")
    # weight gradient: sampled weight rows k of sampled experts, all columns
    off = oracle.expert_offsets(gl)
    dw_host = {}
    for e in range(E):
        ks = rng.integers(0, H, 4)
        got = dev_f64(dw1[e, torch.from_numpy(ks).to(dev)])
        if gl[e] == 0:
            assert (got == 0).all(), f"dW1 of empty expert {e}"
            continue
        xe = f64(x_b[off[e]:off[e + 1]][:, ks])        # [n_e, 4]
        dhe = f64(dh_b[off[e]:off[e + 1]])             # [n_e, 3072]
        assert_close(got, xe.T @ dhe, f"ep dW1 expert {e} rows {ks.tolist()}")
        dw_host[e] = True
    assert len(dw_host) == int((gl > 0).sum())


def test_dw_tile_queue_workspace(dev):
    """gmm_bwd_weight's tile queue (and, on split grids, its partial tiles)
    lives in the caller's workspace: the call leaves the queue zero-filled,
    so back-to-back calls of different shapes through one workspace give the
    same bits as calls with fresh workspaces."""
    rng = np.random.default_rng(11)
    ws = torch.zeros(moe.gmm_workspace_size(8, 1000, 520, 264, moe.OP_BWD_WEIGHT), dtype=torch.uint8,
                     device=dev)
    cases = [(1000, 520, 264, [300, 0, 200, 100, 0, 150, 250, 0]), (300, 64, 64, [100, 100, 100]),
             (1000, 520, 264, [0, 0, 1000, 0, 0, 0, 0, 0])]
    for M, K, N, gl in cases:
        print(f"dw queue: M={M} K={K} N={N} E={len(gl)}", flush=True)
        x = bf16_dev(workloads.normal_bf16(rng, (M, K)), dev)
        dy = bf16_dev(workloads.normal_bf16(rng, (M, N)), dev)
        g = _gl(dev, gl)
        shared = moe.gmm_bwd_weight(x, dy, g, ws=ws)
        torch.cuda.synchronize()
        assert int(ws[:moe.GMM_QUEUE_BYTES].count_nonzero().item()) == 0, "queue not left zero-filled"
        fresh = moe.gmm_bwd_weight(x, dy, g, ws=torch.zeros_like(ws))
        torch.cuda.synchronize()
        assert np.array_equal(dev_bits(shared), dev_bits(fresh))
        assert_close(f64(dev_bits(shared)), oracle.gmm_bwd_weight(f64(dev_bits(x)), f64(dev_bits(dy)), gl),
                     "dw queue")


def _bwd_swiglu_case(dev, x_b, dy_b, w_b, h_b, gl, in_place, tag):
    M, K = x_b.shape
    R = int(np.sum(gl))
    print(f"gmm_bwd_swiglu {tag}: E={len(gl)} M={M} K={K} N={dy_b.shape[1]} in_place={in_place}", flush=True)
    x, dy, w, h = (bf16_dev(b, dev) for b in (x_b, dy_b, w_b, h_b))
    g = _gl(dev, gl)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    if in_place:
        dh, dw = moe.gmm_bwd_swiglu(x, dy, w, h, g, dh_out=h, dev_err=err)
    else:
        dh, dw = moe.gmm_bwd_swiglu(x, dy, w, h, g, dh_out=_sentinel(dev, (M, 2 * K)), dev_err=err)
    dw_ref_bits = dev_bits(moe.gmm_bwd_weight(x, dy, g, dev_err=err))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = oracle.swiglu_bwd(oracle.gmm_bwd_input(f64(dy_b), f64(w_b), gl), f64(h_b))
    assert_close(f64(dev_bits(dh))[:R], ref[:R], f"gmm_bwd_swiglu {tag} dH")
    tail = dev_bits(dh)[R:]
    assert (tail == (h_b[R:] if in_place else SENT)).all(), "rows >= R were written"
    E, N = len(gl), dy_b.shape[1]
    if moe.gmm_workspace_size(E, M, K, N, moe.OP_BWD_WEIGHT) > moe.GMM_QUEUE_BYTES:
        # few tiles: gmm_bwd_weight splits the row reduction; both vs the oracle
        ref_w = oracle.gmm_bwd_weight(f64(x_b), f64(dy_b), gl)
        assert_close(f64(dev_bits(dw)), ref_w, f"gmm_bwd_swiglu {tag} dW")
        assert_close(f64(dw_ref_bits), ref_w, f"gmm_bwd_weight {tag} dW")
    else:
        assert np.array_equal(dev_bits(dw), dw_ref_bits), "dW differs from gmm_bwd_weight"


def test_bwd_swiglu_limits(dev):
    """gmm_bwd_swiglu at the API limits: E = 1024 experts (mostly empty), and a
    2^21-long reduction for the input gradient (N = 2^21)."""
    rng = np.random.default_rng(2024)
    E, M, K, N = 1024, 3000, 64, 136
    gl = workloads.random_group_list(rng, M, E, empty_frac=0.7, fill=0.95)
    _bwd_swiglu_case(dev, workloads.normal_bf16(rng, (M, K)), workloads.normal_bf16(rng, (M, N)),
                     workloads.normal_bf16(rng, (E, K, N), 0.05), workloads.normal_bf16(rng, (M, 2 * K), 1.5),
                     gl, False, "E1024")
    E, M, K, N = 2, 64, 8, 1 << 21
    gl = np.array([40, 24], dtype=np.int64)
    _bwd_swiglu_case(dev, workloads.normal_bf16(rng, (M, K)), workloads.normal_bf16(rng, (M, N)),
                     workloads.normal_bf16(rng, (E, K, N), 0.001), workloads.normal_bf16(rng, (M, 2 * K), 1.5),
                     gl, True, "N=2^21")


@pytest.mark.parametrize("M,K,N,gl,in_place", [
    (1000, 264, 520, [300, 0, 200, 100, 0, 150, 250, 0], False),  # ragged tiles, empty experts
    (777, 72, 264, [0, 777, 0], True),                            # dH written over H
    (129, 8, 8, [64, 1, 64], False),                              # tiny K and N
    (600, 512, 2048, [256, 128, 216], True),                      # several full tiles
])
def test_bwd_swiglu(dev, M, K, N, gl, in_place):
    """gmm_bwd_swiglu: dH = swiglu_bwd(dy @ w[e]^T, h) with the product kept
    in fp32, and dW bit-identical to gmm_bwd_weight (or, where that call
    splits the row reduction of a few-tile grid, both against the oracle);
    rows >= R untouched."""
    rng = np.random.default_rng(M + K + N)
    E = len(gl)
    _bwd_swiglu_case(dev, workloads.normal_bf16(rng, (M, K)), workloads.normal_bf16(rng, (M, N)),
                     workloads.normal_bf16(rng, (E, K, N), std=0.05),
                     workloads.normal_bf16(rng, (M, 2 * K), std=1.5), gl, in_place, "sweep")


@pytest.mark.parametrize("swiglu", [False, True])
def test_forced_variants_agree_on_decode(dev, swiglu):
    """MOEGMM_FORCE_VARIANT (test-only) runs the row-tile and the
    weight-streaming forward on one decode-shaped input (512 rows over 256
    experts, hidden 2048, gate_up 1024 columns): both against the oracle,
    rows >= R untouched."""
    import os

    wl = workloads.decode(with_weights=False)
    gl = np.bincount(wl["topk_ids"].ravel(), minlength=256).astype(np.int64)
    rng = np.random.default_rng(91)
    M, K, I = 512 + 8, 2048, 512
    x_b = workloads.normal_bf16(rng, (M, K))
    w_b = workloads.normal_bf16(rng, (256, K, 2 * I), std=0.02)
    R = int(gl.sum())
    x, w, g = bf16_dev(x_b, dev), bf16_dev(w_b, dev), _gl(dev, gl)
    ref_h = oracle.gmm(f64(x_b), f64(w_b), gl)[:R]
    outs = {}
    try:
        for variant in ("tile", "stream"):
            os.environ["MOEGMM_FORCE_VARIANT"] = variant
            print(f"forced {variant}: swiglu={swiglu} R={R}", flush=True)
            err = torch.zeros(1, dtype=torch.int32, device=dev)
            if swiglu:
                a, h = _sentinel(dev, (M, I)), _sentinel(dev, (M, 2 * I))
                moe.gmm_fwd_swiglu(x, w, g, out=a, h_out=h, dev_err=err)
                outs[variant] = (dev_bits(a), dev_bits(h))
            else:
                y = moe.gmm_fwd(x, w, g, out=_sentinel(dev, (M, 2 * I)), dev_err=err)
                outs[variant] = (dev_bits(y),)
            torch.cuda.synchronize()
            assert int(err.item()) == 0
    finally:
        os.environ.pop("MOEGMM_FORCE_VARIANT", None)
    for variant, res in outs.items():
        assert all((r[R:] == SENT).all() for r in res), f"{variant}: rows >= R written"
        if swiglu:
            a, h = res
            assert_close(f64(h)[:R], ref_h, f"forced {variant} h")
            assert_close(f64(a)[:R], oracle.gmm_swiglu(f64(x_b), f64(w_b), gl)[:R], f"forced {variant} a")
        else:
            assert_close(f64(res[0])[:R], ref_h, f"forced {variant} y")



def test_dw_split_few_tiles_dense(dev):
    """A weight gradient whose tile grid cannot fill the CUs (one expert,
    K = 2048, N = 1024: 32 tiles) splits each tile's row reduction into
    chunks whose fp32 partials meet in the workspace.  Against the oracle on
    one weight row per 256-row k-tile (all columns); bit-identical on a
    repeat; the workspace's queue left zero-filled."""
    rng = np.random.default_rng(21)
    M, K, N = 32768, 2048, 1024
    x_b = workloads.normal_bf16(rng, (M, K))
    dy_b = workloads.normal_bf16(rng, (M, N))
    gl = np.array([M], dtype=np.int64)
    x, dy, g = bf16_dev(x_b, dev), bf16_dev(dy_b, dev), _gl(dev, gl)
    nbytes = moe.gmm_workspace_size(1, M, K, N, moe.OP_BWD_WEIGHT)
    assert nbytes > moe.GMM_QUEUE_BYTES, "this grid takes the split path"
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    print(f"dW split: M={M} K={K} N={N} workspace={nbytes}", flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dw1 = moe.gmm_bwd_weight(x, dy, g, ws=ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(ws[:moe.GMM_QUEUE_BYTES].count_nonzero().item()) == 0, "queue not left zero-filled"
    dw2 = moe.gmm_bwd_weight(x, dy, g, ws=ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(dev_bits(dw1), dev_bits(dw2)), "split dW not bit-reproducible"
    ks = np.arange(0, K, 256) + rng.integers(0, 256, K // 256)
    got = dev_f64(dw1[0, torch.from_numpy(ks).to(dev)])
    assert_close(got, f64(x_b[:, ks]).T @ f64(dy_b), "split dW rows")


@pytest.mark.parametrize("K,N", [(512, 520), (520, 264)])
def test_dw_split_few_tiles_ragged(dev, K, N):
    """Few tiles over several experts: a long expert split into many chunks,
    an empty one (exact zeros), a short one kept whole; whole-tensor parity
    with the oracle, and the fused gmm_bwd (no split) within tolerance.  The
    last tile column (N = 520) or the last tile row and column (K = 520,
    N = 264) hold 8 of their 256 outputs."""
    rng = np.random.default_rng(22)
    M = 5100
    gl = np.array([5000, 0, 37], dtype=np.int64)
    x_b = workloads.normal_bf16(rng, (M, K))
    dy_b = workloads.normal_bf16(rng, (M, N))
    w_b = workloads.normal_bf16(rng, (3, K, N), std=0.02)
    x, dy, w, g = bf16_dev(x_b, dev), bf16_dev(dy_b, dev), bf16_dev(w_b, dev), _gl(dev, gl)
    assert moe.gmm_workspace_size(3, M, K, N, moe.OP_BWD_WEIGHT) > moe.GMM_QUEUE_BYTES
    print(f"dW split ragged: gl={gl.tolist()} K={K} N={N}", flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dw = moe.gmm_bwd_weight(x, dy, g, out=_sentinel(dev, (3, K, N)), dev_err=err)
    _, dw_fused = moe.gmm_bwd(x, dy, w, g, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = oracle.gmm_bwd_weight(f64(x_b), f64(dy_b), gl)
    assert_close(dev_f64(dw), ref, "split dW ragged")
    assert_close(dev_f64(dw_fused), ref, "gmm_bwd dW ragged")
    assert (dev_bits(dw)[1] == 0).all(), "empty expert's dW not exact zeros"
