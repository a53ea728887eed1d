"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin is a function ``check_*(impl...)`` that raises AssertionError on a
mismatch.  The tests run them on the oracle; the mutation tests at the end
plant plausible mistakes in copies of oracle functions (on the CPU) and check
that at least one pin catches each.

Sources: the worked example and loop definition of the grouped matmul, and the
backward formulas, from "NPU Training Operators - GMM" (section 算子语义);
SwiGLU and the weighted combine from "MegaMoE" (activation formulas, A16W16
scenario); masked slots and FP32 accumulation from the
MoeTokenPermuteWithRoutingMapGrad article (sections 4.1 and 6.2).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_values(rng, shape, std=1.0):
    """Random values already representable in bf16 (float64)."""
    return oracle.round_bf16(rng.standard_normal(shape) * std)


# ---------------------------------------------------------------------------
# pin 1: the pages' worked example (tests/golden/worked_example.json)
# ---------------------------------------------------------------------------


def _load_worked(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        return json.load(f)


def check_worked_example(g, permute_maps, tokens_per_expert, gmm):
    page, rd = g["from_page"], g["from_readings"]
    ids = np.array(rd["topk_ids"], dtype=np.int32)
    # the valid slots of the id matrix are exactly the page's pairs
    pairs = sorted((t, int(e)) for t in range(4) for e in ids[t] if e >= 0)
    assert pairs == sorted(tuple(p) for p in page["pairs_token_expert"])
    counts = tokens_per_expert(ids, 4)
    assert counts.tolist() == page["group_list"]
    sorted_slot, row_id_map, counts2 = permute_maps(ids, 4)
    assert counts2.tolist() == page["group_list"]
    src_tokens = (np.asarray(sorted_slot) // 2).tolist()
    # per-expert token lists of the page
    off = np.concatenate([[0], np.cumsum(page["group_list"])])
    for e in range(4):
        assert src_tokens[off[e]:off[e + 1]] == page["rows_by_expert_tokens"][e]
    assert off.tolist() == rd["offsets"]
    assert np.asarray(sorted_slot).tolist() == rd["sorted_slot"]
    assert np.asarray(row_id_map).tolist() == rd["row_id_map"]
    assert src_tokens == rd["permuted_source_tokens"]
    # row-to-weight table: weight[e] = (e+1) * identity, so each output row is
    # its input row scaled by (index of the weight used + 1)
    H = 8
    x = np.arange(5 * H, dtype=np.float64).reshape(5, H) + 1.0
    w = np.stack([(e + 1.0) * np.eye(H) for e in range(4)])
    y = gmm(x, w, np.array(page["group_list"]))
    for lo, hi, widx in page["row_ranges_to_weight"]:
        for r in range(lo, hi):
            np.testing.assert_array_equal(y[r], (widx + 1.0) * x[r])


def test_worked_example(golden_dir):
    check_worked_example(_load_worked(golden_dir), oracle.permute_maps,
                         oracle.tokens_per_expert, oracle.gmm)


# ---------------------------------------------------------------------------
# pin 2: bf16 rounding against PyTorch's CPU cast (a library routine)
# ---------------------------------------------------------------------------


def check_bf16_rounding(round_fn):
    import torch

    rng = _rng(11)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormals
        (rng.standard_normal(2000) * 1e38).astype(np.float32),  # near overflow
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895314e38,
                  1.00390625, 1.01171875, 1.0078125 + 2 ** -24], dtype=np.float32),
    ])
    # exact ties: halfway between two bf16 values, both parities
    base = (rng.integers(0, 2 ** 15, 4000, dtype=np.uint32) << 16) | 0x8000
    vals = np.concatenate([vals, base.view(np.float32)])
    vals = vals[np.isfinite(vals) | np.isinf(vals)]
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_fn(vals.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert np.isnan(round_fn(np.array([np.nan]))).all()


def test_bf16_rounding_matches_torch():
    check_bf16_rounding(oracle.round_bf16)


def test_bf16_bits_roundtrip():
    rng = _rng(3)
    v = rng.standard_normal(1000)
    bits = oracle.to_bf16_bits(v)
    np.testing.assert_array_equal(oracle.bf16_to_f64(bits), oracle.round_bf16(v))


# ---------------------------------------------------------------------------
# pin 3: grouped matmul against a pure-Python triple loop (brute force, fp64)
# ---------------------------------------------------------------------------


def _brute_gmm(x, w, gl):
    K = x.shape[1]
    E, _, N = w.shape
    y = [[0.0] * N for _ in range(int(sum(gl)))]
    row = 0
    for e in range(E):
        for _ in range(int(gl[e])):
            for j in range(N):
                acc = 0.0
                for k in range(K):
                    acc += float(x[row, k]) * float(w[e, k, j])
                y[row][j] = acc
            row += 1
    return np.array(y)


GROUP_CASES = [
    [3, 2, 4],
    [0, 5, 0, 2, 0],   # empties at start, middle, end
    [7],
    [0, 0, 6],
    [2, 0, 0, 0, 1, 3],
]


def check_gmm_brute(gmm):
    rng = _rng(5)
    for gl in GROUP_CASES:
        gl = np.array(gl)
        M, K, N = int(gl.sum()), 5, 3
        x = _bf16_values(rng, (M + 2, K))  # two spare rows beyond R
        w = _bf16_values(rng, (len(gl), K, N))
        got = gmm(x, w, gl)[:M]
        np.testing.assert_allclose(got, _brute_gmm(x, w, gl), rtol=1e-12, atol=1e-12)


def test_gmm_bruteforce():
    check_gmm_brute(oracle.gmm)


# ---------------------------------------------------------------------------
# pin 4: block-diagonal closed form -- one dense product of a different layout
# ---------------------------------------------------------------------------


def check_gmm_block_diagonal(gmm):
    rng = _rng(6)
    gl = np.array([4, 0, 9, 1, 0, 6])
    E, K, N = len(gl), 7, 5
    R = int(gl.sum())
    x = _bf16_values(rng, (R, K))
    w = _bf16_values(rng, (E, K, N))
    # X~ [R, E*K]: row r of expert e placed in column block e; W~ = vstack(W_e)
    xt = np.zeros((R, E * K))
    expert_of_row = np.repeat(np.arange(E), gl)
    for r in range(R):
        e = expert_of_row[r]
        xt[r, e * K:(e + 1) * K] = x[r]
    wt = w.reshape(E * K, N)
    np.testing.assert_allclose(gmm(x, w, gl), xt @ wt, rtol=1e-12, atol=1e-12)


def test_gmm_block_diagonal():
    check_gmm_block_diagonal(oracle.gmm)


# ---------------------------------------------------------------------------
# pin 5: orientation -- a one-hot input row selects a ROW of W[e]
# ---------------------------------------------------------------------------


def check_gmm_one_hot(gmm):
    rng = _rng(7)
    gl = np.array([2, 0, 3])
    K, N = 4, 6
    w = _bf16_values(rng, (3, K, N))
    x = np.zeros((5, K))
    picks = [1, 3, 0, 2, 3]
    for r, k in enumerate(picks):
        x[r, k] = 1.0
    y = gmm(x, w, gl)
    experts = [0, 0, 2, 2, 2]
    for r in range(5):
        np.testing.assert_array_equal(y[r], w[experts[r], picks[r], :])


def test_gmm_one_hot_rows():
    check_gmm_one_hot(oracle.gmm)


def test_gmm_single_expert_is_dense_matmul():
    """E=1 reduces to a plain dense product (textbook special case)."""
    rng = _rng(8)
    x = _bf16_values(rng, (33, 17))
    w = _bf16_values(rng, (1, 17, 9))
    np.testing.assert_allclose(oracle.gmm(x, w, [33]), x @ w[0], rtol=1e-13, atol=1e-13)
    dy = _bf16_values(rng, (33, 9))
    np.testing.assert_allclose(oracle.gmm_bwd_input(dy, w, [33]), dy @ w[0].T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.gmm_bwd_weight(x, dy, [33])[0], x.T @ dy, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# pin 6: backward by finite differences of f = <gmm(x, w), dy> (fp64)
# ---------------------------------------------------------------------------


def check_gmm_grads_fd(gmm, bwd_input, bwd_weight):
    rng = _rng(9)
    gl = np.array([3, 0, 4, 2])
    E, K, N = len(gl), 6, 5
    M = int(gl.sum())
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((E, K, N))
    dy = rng.standard_normal((M, N))

    def f(xx, ww):
        return float(np.sum(gmm(xx, ww, gl)[:M] * dy))

    dx = bwd_input(dy, w, gl)
    dw = bwd_weight(x, dy, gl)
    h = 1e-5
    for i in range(M):
        for k in range(K):
            xp, xm = x.copy(), x.copy()
            xp[i, k] += h
            xm[i, k] -= h
            fd = (f(xp, w) - f(xm, w)) / (2 * h)
            assert abs(fd - dx[i, k]) <= 1e-6 * max(1.0, abs(fd)), (i, k, fd, dx[i, k])
    for e in range(E):
        for k in range(K):
            for j in range(N):
                wp, wm = w.copy(), w.copy()
                wp[e, k, j] += h
                wm[e, k, j] -= h
                fd = (f(x, wp) - f(x, wm)) / (2 * h)
                assert abs(fd - dw[e, k, j]) <= 1e-6 * max(1.0, abs(fd)), (e, k, j)
    # the empty expert's gradient is exactly zero
    assert np.all(dw[1] == 0.0)


def test_gmm_grads_finite_differences():
    check_gmm_grads_fd(oracle.gmm, oracle.gmm_bwd_input, oracle.gmm_bwd_weight)


def test_gmm_adjoint_identities():
    """<gmm(x,w), dy> = <x, dX> = sum_e <W_e, dW_e> (both are linear in x, w)."""
    rng = _rng(10)
    gl = np.array([5, 0, 8, 3, 0])
    M, K, N = int(gl.sum()), 12, 10
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((len(gl), K, N))
    dy = rng.standard_normal((M, N))
    lhs = np.sum(oracle.gmm(x, w, gl) * dy)
    assert abs(lhs - np.sum(x * oracle.gmm_bwd_input(dy, w, gl))) < 1e-10
    assert abs(lhs - np.sum(w * oracle.gmm_bwd_weight(x, dy, gl))) < 1e-10


# ---------------------------------------------------------------------------
# pin 7: SwiGLU closed forms and its derivative by finite differences
# ---------------------------------------------------------------------------


def check_swiglu_values(swiglu):
    # G in the first half, U in the second
    h = np.array([[0.0, 1.0, 30.0, -30.0, 2.0, 3.0, 0.5, 7.0]])
    a = swiglu(h)[0]
    assert a.shape == (4,)
    assert a[0] == 0.0                                   # SiLU(0) = 0
    assert abs(a[1] - 3.0 / (1.0 + math.exp(-1.0))) < 1e-15  # SiLU(1)*3
    assert abs(a[2] - 30.0 * 0.5) < 1e-10                # SiLU(30) ~ 30
    assert abs(a[3]) < 1e-10                             # SiLU(-30) ~ 0
    # textbook value: SiLU(1) = 0.7310585786300049
    assert abs(swiglu(np.array([[1.0, 1.0]]))[0, 0] - 0.7310585786300049) < 1e-15


def test_swiglu_closed_forms():
    check_swiglu_values(oracle.swiglu)


def check_swiglu_bwd_fd(swiglu, swiglu_bwd):
    rng = _rng(12)
    R, I = 4, 6
    h = rng.standard_normal((R, 2 * I)) * 2.0
    da = rng.standard_normal((R, I))
    dh = swiglu_bwd(da, h)
    eps = 1e-5
    for r in range(R):
        for c in range(2 * I):
            hp, hm = h.copy(), h.copy()
            hp[r, c] += eps
            hm[r, c] -= eps
            fd = (np.sum(swiglu(hp) * da) - np.sum(swiglu(hm) * da)) / (2 * eps)
            assert abs(fd - dh[r, c]) <= 1e-6 * max(1.0, abs(fd)), (r, c, fd, dh[r, c])


def test_swiglu_bwd_finite_differences():
    check_swiglu_bwd_fd(oracle.swiglu, oracle.swiglu_bwd)


# ---------------------------------------------------------------------------
# pin 8: permute / unpermute round trips and invariants
# ---------------------------------------------------------------------------


def _random_ids(rng, T, K, E, mask_frac=0.2):
    ids = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=K, replace=False) if K <= E else rng.integers(0, E, K)
    ids[rng.random((T, K)) < mask_frac] = -1
    return ids


def check_permute_invariants(permute_maps):
    rng = _rng(13)
    for (T, K, E) in [(1, 1, 1), (7, 2, 4), (50, 4, 16), (33, 8, 9), (5, 1, 40)]:
        ids = _random_ids(rng, T, K, E)
        flat = ids.reshape(-1)
        sorted_slot, row_id_map, counts = permute_maps(ids, E)
        valid = flat >= 0
        np.testing.assert_array_equal(counts, np.bincount(flat[valid], minlength=E))
        assert counts.sum() == valid.sum()
        # brute-force construction: walk experts in order, slots in order
        brute = [s for e in range(E) for s in range(T * K) if flat[s] == e]
        assert np.asarray(sorted_slot).tolist() == brute
        for r, s in enumerate(brute):
            assert row_id_map[s] == r
        assert all(row_id_map[s] == -1 for s in range(T * K) if flat[s] < 0)


def test_permute_invariants():
    check_permute_invariants(oracle.permute_maps)


def check_roundtrip(permute, unpermute):
    rng = _rng(14)
    for K in (2, 4, 8):
        T, E, H = 24, 16, 8
        ids = _random_ids(rng, T, K, E, mask_frac=0.0)
        x = _bf16_values(rng, (T, H))
        x_perm, row_id_map, _, _ = permute(x, ids, E)
        for s in range(T * K):
            np.testing.assert_array_equal(x_perm[row_id_map[s]], x[s // K])
        onehot = np.zeros((T, K))
        onehot[:, 0] = 1.0
        np.testing.assert_array_equal(unpermute(x_perm, row_id_map, onehot), x)
        ones = np.ones((T, K))
        np.testing.assert_array_equal(unpermute(x_perm, row_id_map, ones), K * x)
    # masked slots add nothing; a fully masked token gives zeros
    ids = np.array([[2, -1], [-1, -1], [0, 1]], dtype=np.int32)
    x = _bf16_values(rng, (3, 4))
    x_perm, row_id_map, _, _ = permute(x, ids, 3)
    out = unpermute(x_perm, row_id_map, np.array([[0.5, 9.0], [3.0, 4.0], [1.0, 2.0]]))
    np.testing.assert_array_equal(out[0], 0.5 * x[0])
    np.testing.assert_array_equal(out[1], np.zeros(4))
    np.testing.assert_array_equal(out[2], 3.0 * x[2])


def test_permute_unpermute_roundtrip():
    check_roundtrip(oracle.permute, oracle.unpermute)


# ---------------------------------------------------------------------------
# pin 9: the whole layer against the per-token MegaMoE formula
#        y_i = sum_k w_k * FFN_{e_ik}(x_i), no permutation involved
# ---------------------------------------------------------------------------


def check_layer_per_token(layer_forward):
    rng = _rng(15)
    T, K, E, H, I = 9, 3, 5, 8, 6
    ids = _random_ids(rng, T, K, E, mask_frac=0.15)
    x = _bf16_values(rng, (T, H))
    w1 = _bf16_values(rng, (E, H, 2 * I), 0.3)
    w2 = _bf16_values(rng, (E, I, H), 0.3)
    probs = rng.random((T, K))
    got = layer_forward(x, ids, probs, w1, w2, E, rounding=None)["out"]
    ref = np.zeros((T, H))
    for i in range(T):
        for k in range(K):
            e = ids[i, k]
            if e < 0:
                continue
            h = x[i] @ w1[e]
            g, u = h[:I], h[I:]
            a = g / (1.0 + np.exp(-g)) * u
            ref[i] += probs[i, k] * (a @ w2[e])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_layer_matches_per_token_formula():
    check_layer_per_token(oracle.moe_layer_forward)


def check_block_backward_fd(layer_forward, block_backward, gmm, swiglu):
    """Expert-block gradients of f = <down(SwiGLU(gate_up(X))), dYp> by FD."""
    rng = _rng(16)
    gl = np.array([2, 0, 3])
    E, H, I = 3, 4, 3
    M = int(gl.sum())
    x = rng.standard_normal((M, H))
    w1 = rng.standard_normal((E, H, 2 * I)) * 0.5
    w2 = rng.standard_normal((E, I, H)) * 0.5
    dyp = rng.standard_normal((M, H))

    def f(xx, a1, a2):
        return float(np.sum(gmm(swiglu(gmm(xx, a1, gl)), a2, gl) * dyp))

    h = gmm(x, w1, gl)
    a = swiglu(h)
    g = block_backward(x, h, a, dyp, w1, w2, gl, rounding=None)
    eps = 1e-6
    for arr, grad, name in ((x, g["dx"], "x"), (w1, g["dw1"], "w1"), (w2, g["dw2"], "w2")):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            args_p = dict(x=x, w1=w1, w2=w2)
            args_m = dict(x=x, w1=w1, w2=w2)
            args_p[name], args_m[name] = p, m
            fd = (f(args_p["x"], args_p["w1"], args_p["w2"]) - f(args_m["x"], args_m["w1"], args_m["w2"])) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_block_backward_finite_differences():
    check_block_backward_fd(oracle.moe_layer_forward, oracle.expert_block_backward,
                            oracle.gmm, oracle.swiglu)


# ---------------------------------------------------------------------------
# pin 10: empty experts never contribute (NaN weights for empty experts)
# ---------------------------------------------------------------------------


def test_empty_expert_weights_never_read():
    rng = _rng(17)
    gl = np.array([0, 4, 0, 3, 0])
    M, K, N = 7, 6, 5
    x = _bf16_values(rng, (M, K))
    w = _bf16_values(rng, (5, K, N))
    dy = _bf16_values(rng, (M, N))
    w_nan = w.copy()
    w_nan[gl == 0] = np.nan
    np.testing.assert_array_equal(oracle.gmm(x, w_nan, gl), oracle.gmm(x, w, gl))
    np.testing.assert_array_equal(oracle.gmm_bwd_input(dy, w_nan, gl), oracle.gmm_bwd_input(dy, w, gl))
    dw = oracle.gmm_bwd_weight(x, dy, gl)
    assert np.all(dw[gl == 0] == 0.0)


# ---------------------------------------------------------------------------
# pin 11: permute backward -- the worked example, the adjoint of the gather,
#         a brute-force walk
# ---------------------------------------------------------------------------


def check_permute_bwd_worked(g, permute_bwd):
    """With dX_perm = the identity rows, dx[t] marks exactly the permuted rows
    copied from token t (the page's rows, laid out by readings 2-3)."""
    rmap = np.asarray(g["from_readings"]["row_id_map"])
    src = g["from_readings"]["permuted_source_tokens"]
    R = len(src)
    dx = permute_bwd(np.eye(R), rmap, 4)
    for t in range(4):
        np.testing.assert_array_equal(dx[t], [1.0 if src[r] == t else 0.0 for r in range(R)])


def check_permute_adjoint(permute, permute_bwd):
    """<permute(x), g> == <x, permute_bwd(g)> for every x and g: the permute
    backward is the adjoint of the gather, masked slots included."""
    rng = _rng(21)
    for (T, K, E, H) in [(6, 2, 3, 5), (20, 4, 7, 3), (9, 8, 12, 4), (4, 1, 2, 6)]:
        ids = _random_ids(rng, T, K, E, mask_frac=0.25)
        x = rng.standard_normal((T, H))
        x_perm, rmap, _, _ = permute(x, ids, E)
        gr = rng.standard_normal(x_perm.shape)
        lhs = float(np.sum(x_perm * gr))
        rhs = float(np.sum(x * permute_bwd(gr, rmap, T)))
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (T, K, lhs, rhs)


def check_permute_bwd_brute(permute_bwd):
    rng = _rng(22)
    T, K, H, R = 7, 3, 4, 12
    rmap = np.full(T * K, -1, dtype=np.int64)
    slots = rng.choice(T * K, size=R, replace=False)
    rmap[slots] = rng.permutation(R)
    gr = rng.standard_normal((R, H))
    got = permute_bwd(gr, rmap, T)
    for t in range(T):
        ref = np.zeros(H)
        for k in range(K):
            r = rmap[t * K + k]
            if r >= 0:
                ref = ref + gr[r]
        np.testing.assert_allclose(got[t], ref, rtol=0, atol=1e-14)


def test_permute_bwd_worked_example(golden_dir):
    check_permute_bwd_worked(_load_worked(golden_dir), oracle.permute_bwd)


def test_permute_bwd_adjoint():
    check_permute_adjoint(oracle.permute, oracle.permute_bwd)


def test_permute_bwd_bruteforce():
    check_permute_bwd_brute(oracle.permute_bwd)


# ---------------------------------------------------------------------------
# pin 12: unpermute backward -- L = <dout, unpermute(Yp, probs)> is linear in
#         Yp and in probs, so <dYp, Yp> = L = <dprobs, probs>, and a one-
#         coordinate difference quotient is the derivative exactly
# ---------------------------------------------------------------------------


def check_unpermute_bwd(permute, unpermute, unpermute_bwd):
    rng = _rng(23)
    for (T, K, E, H) in [(8, 2, 4, 6), (15, 4, 9, 3), (5, 8, 10, 4)]:
        ids = _random_ids(rng, T, K, E, mask_frac=0.25)
        x = rng.standard_normal((T, H))
        _, rmap, _, _ = permute(x, ids, E)
        R = int(np.sum(ids >= 0))
        yp = rng.standard_normal((R, H))
        probs = rng.random((T, K))
        dout = rng.standard_normal((T, H))

        def loss(y, p):
            return float(np.sum(dout * unpermute(y, rmap, p)))

        L = loss(yp, probs)
        dyp, dprobs = unpermute_bwd(dout, yp, rmap, probs)
        assert dyp.shape == yp.shape and dprobs.shape == probs.shape
        assert abs(float(np.sum(dyp * yp)) - L) <= 1e-12 * max(1.0, abs(L))
        assert abs(float(np.sum(dprobs * probs)) - L) <= 1e-12 * max(1.0, abs(L))
        flat = ids.reshape(-1)
        assert np.all(dprobs.reshape(-1)[flat < 0] == 0.0)
        for _ in range(6):
            i, j = rng.integers(R), rng.integers(H)
            y2 = yp.copy()
            y2[i, j] += 1.0
            assert abs((loss(y2, probs) - L) - dyp[i, j]) <= 1e-12 * max(1.0, abs(L))
            t, k = rng.integers(T), rng.integers(K)
            p2 = probs.copy()
            p2[t, k] += 1.0
            assert abs((loss(yp, p2) - L) - dprobs[t, k]) <= 1e-12 * max(1.0, abs(L))


def test_unpermute_bwd_identities():
    check_unpermute_bwd(oracle.permute, oracle.unpermute, oracle.unpermute_bwd)


# ---------------------------------------------------------------------------
# pin 13: the whole layer backward (dx, dprobs, dW1, dW2) by central finite
#         differences of f = <dout, layer(x, probs, W1, W2)>, exact chain
# ---------------------------------------------------------------------------


def check_layer_backward_fd(layer_forward, layer_backward):
    rng = _rng(24)
    T, K, E, H, I = 6, 2, 3, 4, 3
    ids = _random_ids(rng, T, K, E, mask_frac=0.2)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, H, 2 * I)) * 0.5
    w2 = rng.standard_normal((E, I, H)) * 0.5
    probs = rng.random((T, K))
    dout = rng.standard_normal((T, H))

    def f(xx, pp, a1, a2):
        return float(np.sum(dout * layer_forward(xx, ids, pp, a1, a2, E, rounding=None)["out"]))

    fwd = layer_forward(x, ids, probs, w1, w2, E, rounding=None)
    g = layer_backward(fwd, dout, probs, w1, w2, rounding=None)
    eps = 1e-6
    args = dict(x=x, probs=probs, w1=w1, w2=w2)
    grads = dict(x=g["dx"], probs=g["dprobs"], w1=g["dw1"], w2=g["dw2"])
    for name in ("x", "probs", "w1", "w2"):
        arr = args[name]
        for _ in range(8):
            idx = tuple(int(rng.integers(n)) for n in arr.shape)
            vals = []
            for sgn in (1, -1):
                a = dict(args)
                a[name] = arr.copy()
                a[name][idx] += sgn * eps
                vals.append(f(a["x"], a["probs"], a["w1"], a["w2"]))
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - grads[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grads[name][idx])


def test_layer_backward_finite_differences():
    check_layer_backward_fd(oracle.moe_layer_forward, oracle.moe_layer_backward)


# ---------------------------------------------------------------------------
# pin 14: the fused gate_up GMM + SwiGLU, row by row with explicit loops
# ---------------------------------------------------------------------------


def check_gmm_swiglu_brute(gmm_swiglu):
    rng = _rng(25)
    gl = np.array([3, 0, 2, 1])
    K, I = 5, 3
    M = int(gl.sum())
    x = rng.standard_normal((M, K))
    w1 = rng.standard_normal((4, K, 2 * I))
    got = gmm_swiglu(x, w1, gl)
    assert got.shape == (M, I)
    r = 0
    for e, n in enumerate(gl):
        for _ in range(n):
            for j in range(I):
                g = sum(x[r, q] * w1[e, q, j] for q in range(K))
                u = sum(x[r, q] * w1[e, q, I + j] for q in range(K))
                ref = g / (1.0 + np.exp(-g)) * u
                assert abs(got[r, j] - ref) <= 1e-12 * max(1.0, abs(ref)), (r, j)
            r += 1


def test_gmm_swiglu_bruteforce():
    check_gmm_swiglu_brute(oracle.gmm_swiglu)


def test_fused_swiglu_bwd_moves_only_a_rounding_point():
    """The fused chain differs from the plain one only in where dA is rounded:
    with no rounding both are the same chain; with bf16 rounding dA itself is
    unchanged, and dH = round(swiglu_bwd(dA, H)) follows the unrounded dA."""
    rng = np.random.default_rng(5)
    gl = [3, 0, 2]
    R, H, I = 5, 16, 8
    x = oracle.round_bf16(rng.standard_normal((R, H)))
    w1 = oracle.round_bf16(rng.standard_normal((3, H, 2 * I)) * 0.3)
    w2 = oracle.round_bf16(rng.standard_normal((3, I, H)) * 0.3)
    dyp = oracle.round_bf16(rng.standard_normal((R, H)))
    h = oracle.round_bf16(oracle.gmm(x, w1, gl))
    a = oracle.round_bf16(oracle.swiglu(h))
    exact = [oracle.expert_block_backward(x, h, a, dyp, w1, w2, gl, rounding=None, fused_swiglu_bwd=f)
             for f in (False, True)]
    for k in exact[0]:
        np.testing.assert_array_equal(exact[0][k], exact[1][k])
    plain = oracle.expert_block_backward(x, h, a, dyp, w1, w2, gl)
    fused = oracle.expert_block_backward(x, h, a, dyp, w1, w2, gl, fused_swiglu_bwd=True)
    np.testing.assert_array_equal(plain["da"], fused["da"])
    da_exact = oracle.gmm_bwd_input(dyp, w2, gl)
    np.testing.assert_array_equal(fused["dh"], oracle.round_bf16(oracle.swiglu_bwd(da_exact, h)))
    assert not np.array_equal(plain["dh"], fused["dh"])  # the rounding point does move


# ---------------------------------------------------------------------------
# mutation tests: a planted mistake in a copy of an oracle function must trip
# at least one pin (run on the CPU only)
# ---------------------------------------------------------------------------


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _mut_gmm_transposed(x, w, gl):
    # W[e] read through its transpose (same element count, wrong layout)
    w = np.asarray(w, float)
    wt = np.stack([w[e].T.reshape(w.shape[1], w.shape[2]) for e in range(w.shape[0])])
    return oracle.gmm(x, wt, gl)


def _mut_gmm_empty_shift(x, w, gl):
    # an empty expert wrongly consumes the next expert's weight slot
    x = np.asarray(x, float)
    y = np.zeros((x.shape[0], w.shape[2]))
    start, widx = 0, 0
    for n in gl:
        if n == 0:
            continue
        y[start:start + n] = x[start:start + n] @ w[widx]
        start += n
        widx += 1
    return y


def _mut_gmm_drop_last_row(x, w, gl):
    y = oracle.gmm(x, w, gl)
    off = np.cumsum(gl)
    for e, end in enumerate(off):
        if gl[e] > 0:
            y[end - 1] = 0.0
    return y


def _mut_bwd_input_no_transpose(dy, w, gl):
    w = np.asarray(w, float)
    dx = np.zeros((dy.shape[0], w.shape[1]))
    start = 0
    for e, n in enumerate(gl):
        if n > 0:
            dx[start:start + n] = (dy[start:start + n] @ w[e].T) * (1.0 + 1e-3)
        start += n
    return dx


def _mut_bwd_weight_wrong_expert(x, dy, gl):
    dw = oracle.gmm_bwd_weight(x, dy, gl)
    return np.roll(dw, 1, axis=0)


def _mut_swiglu_swapped(h):
    I = h.shape[1] // 2
    return oracle.swiglu(np.concatenate([h[:, I:], h[:, :I]], axis=1))


def _mut_swiglu_bwd_sign(da, h):
    I = h.shape[1] // 2
    g, u = h[:, :I], h[:, I:]
    s = oracle.sigmoid(g)
    dg = da * u * s * (1.0 - g * (1.0 - s))   # wrong sign
    return np.concatenate([dg, da * g * s], axis=1)


def _mut_permute_unstable(ids, E):
    sorted_slot, row_id_map, counts = oracle.permute_maps(ids, E)
    flat = np.asarray(ids).reshape(-1)
    ss = np.array(sorted_slot)
    for e in range(E):
        sel = np.nonzero(flat[ss] == e)[0]
        ss[sel] = ss[sel][::-1]
    rmap = np.full(flat.shape[0], -1)
    rmap[ss] = np.arange(ss.shape[0])
    return ss, rmap, counts


def _mut_hist_counts_masked(ids, E):
    ids = np.asarray(ids).reshape(-1)
    return np.bincount(np.where(ids < 0, 0, ids), minlength=E).astype(np.int64)


def _mut_unpermute_bwd_no_probs(dout, y_perm, row_id_map, probs):
    _, dprobs = oracle.unpermute_bwd(dout, y_perm, row_id_map, probs)
    dyp, _ = oracle.unpermute_bwd(dout, y_perm, row_id_map, np.ones_like(probs))
    return dyp, dprobs  # dYp forgets the probs factor


def _mut_unpermute_bwd_next_slot(dout, y_perm, row_id_map, probs):
    dyp, dprobs = oracle.unpermute_bwd(dout, y_perm, row_id_map, probs)
    return dyp, np.roll(dprobs, 1, axis=1)  # dprobs paired with the wrong slot


def _mut_permute_bwd_masked(dx_perm, row_id_map, num_tokens):
    rmap = np.asarray(row_id_map, dtype=np.int64).reshape(num_tokens, -1)
    dx = np.zeros((num_tokens, np.asarray(dx_perm).shape[1]))
    for k in range(rmap.shape[1]):
        dx += np.asarray(dx_perm)[rmap[:, k]]  # -1 indexes the last row
    return dx


def _mut_permute_bwd_first_slot(dx_perm, row_id_map, num_tokens):
    rmap = np.asarray(row_id_map, dtype=np.int64).reshape(num_tokens, -1)
    return oracle.permute_bwd(dx_perm, rmap[:, :1].reshape(-1), num_tokens)


def _mut_layer_bwd_dprobs_doubled(fwd, dout, probs, w1, w2, rounding=None):
    g = oracle.moe_layer_backward(fwd, dout, probs, w1, w2, rounding=rounding)
    g = dict(g)
    g["dprobs"] = g["dprobs"] * 2.0  # double-counted combine weight
    return g


def _mut_gmm_swiglu_up_gate(x, w1, gl):
    I = np.asarray(w1).shape[2] // 2
    w = np.concatenate([np.asarray(w1)[:, :, I:], np.asarray(w1)[:, :, :I]], axis=2)
    return oracle.gmm_swiglu(x, w, gl)  # gate and up halves swapped


def _mut_round_truncate(a):
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def test_mutants_are_caught(golden_dir):
    g = _load_worked(golden_dir)
    caught = {
        "gmm_empty_shift": _fails(check_worked_example, g, oracle.permute_maps,
                                  oracle.tokens_per_expert, _mut_gmm_empty_shift)
        or _fails(check_gmm_brute, _mut_gmm_empty_shift),
        "gmm_transposed": _fails(check_gmm_one_hot, _mut_gmm_transposed)
        or _fails(check_gmm_brute, _mut_gmm_transposed),
        "gmm_drop_last_row": _fails(check_gmm_block_diagonal, _mut_gmm_drop_last_row),
        "bwd_input_scaled": _fails(check_gmm_grads_fd, oracle.gmm, _mut_bwd_input_no_transpose,
                                   oracle.gmm_bwd_weight),
        "bwd_weight_wrong_expert": _fails(check_gmm_grads_fd, oracle.gmm, oracle.gmm_bwd_input,
                                          _mut_bwd_weight_wrong_expert),
        "swiglu_swapped": _fails(check_swiglu_values, _mut_swiglu_swapped),
        "swiglu_bwd_sign": _fails(check_swiglu_bwd_fd, oracle.swiglu, _mut_swiglu_bwd_sign),
        "permute_unstable": _fails(check_worked_example, g, _mut_permute_unstable,
                                   oracle.tokens_per_expert, oracle.gmm)
        or _fails(check_permute_invariants, _mut_permute_unstable),
        "hist_counts_masked": _fails(check_worked_example, g, oracle.permute_maps,
                                     _mut_hist_counts_masked, oracle.gmm),
        "round_truncate": _fails(check_bf16_rounding, _mut_round_truncate),
        "unpermute_bwd_no_probs": _fails(check_unpermute_bwd, oracle.permute, oracle.unpermute,
                                         _mut_unpermute_bwd_no_probs),
        "unpermute_bwd_next_slot": _fails(check_unpermute_bwd, oracle.permute, oracle.unpermute,
                                          _mut_unpermute_bwd_next_slot),
        "permute_bwd_masked": _fails(check_permute_adjoint, oracle.permute, _mut_permute_bwd_masked),
        "permute_bwd_first_slot": _fails(check_permute_bwd_worked, g, _mut_permute_bwd_first_slot)
        or _fails(check_permute_adjoint, oracle.permute, _mut_permute_bwd_first_slot),
        "layer_bwd_dprobs_doubled": _fails(check_layer_backward_fd, oracle.moe_layer_forward,
                                           _mut_layer_bwd_dprobs_doubled),
        "gmm_swiglu_up_gate": _fails(check_gmm_swiglu_brute, _mut_gmm_swiglu_up_gate),
    }
    missed = [k for k, v in caught.items() if not v]
    assert not missed, f"mutants not caught by any pin: {missed}"
