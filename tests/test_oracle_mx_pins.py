"""Pins for the MXFP8 part of the CPU oracle (oracle/mx_ref.py).

Each pin checks the oracle against something other than itself: PyTorch's own
float8_e4m3fn conversion (a library implementation of the OCP E4M3 format),
values fixed by the OCP Microscaling (MX) v1.0 definition and worked out by
hand, exact round trips, the format's error bound, and brute force with
torch-decoded operands.  The mutation test at the end plants plausible
mistakes in copies of oracle functions (on the CPU) and checks that at least
one pin catches each.

The method: "MegaMoE", A8W8-FP scenario (MX quantisation in groups of 32 with
E8M0 scales; GMM1 -> activation -> requantisation -> GMM2).
"""
import math

import numpy as np
import pytest
import torch

import oracle.mx_ref as mx

GROUP = 32


def _torch_decode(codes):
    c = torch.as_tensor(np.asarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e8m0(b):
    b = np.asarray(b, dtype=np.int64)
    return np.where(b == 255, np.nan, np.power(2.0, (b - 127).astype(np.float64)))


# ---------------------------------------------------------------------------
# pin MX1: decoding every code agrees with PyTorch's float8_e4m3fn
# ---------------------------------------------------------------------------


def check_decode_all_codes(decode):
    d = decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode(np.arange(256))
    assert np.array_equal(np.isnan(d), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(d[ok], ref[ok])
    assert np.array_equal(np.signbit(d[ok]), np.signbit(ref[ok]))


def test_decode_matches_torch():
    check_decode_all_codes(mx.e4m3_decode)


# ---------------------------------------------------------------------------
# pin MX2: encoding agrees with PyTorch's round-to-nearest-even conversion
# over the finite range (torch turns overflow into NaN; MX saturates)
# ---------------------------------------------------------------------------


def check_encode_vs_torch(encode):
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(4000) * 60.0,
        rng.standard_normal(2000) * 2.0 ** -7,          # subnormal range
        rng.uniform(-464.0, 464.0, 2000),
    ]).astype(np.float32)
    # every midpoint between adjacent positive codes (ties to even)
    pos = _torch_decode(np.arange(0, 0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, pos.astype(np.float32)])
    v = v[np.abs(v) <= 464.0]
    got = encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:8]


def test_encode_matches_torch_in_range():
    check_encode_vs_torch(mx.e4m3_encode)


# ---------------------------------------------------------------------------
# pin MX3: special values fixed by the E4M3 (FN) definition and MX's
# saturating conversion, worked by hand
# ---------------------------------------------------------------------------


def check_encode_special(encode):
    cases = [
        (448.0, 0x7E), (480.0, 0x7E), (1e6, 0x7E), (math.inf, 0x7E), (-1e6, 0xFE),
        (1.0, 0x38), (2.0, 0x40), (0.5, 0x30), (1.125, 0x39), (-1.0, 0xB8),
        (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07),
        (2.0 ** -10, 0x00),        # tie between 0 and the smallest subnormal: even
        (3 * 2.0 ** -10, 0x02),    # tie between codes 1 and 2: even
        (1.0625, 0x38),            # tie between 1.0 (even) and 1.125
        (1.1875, 0x3A),            # tie between 1.125 and 1.25 (even)
        (0.0, 0x00), (-0.0, 0x80),
    ]
    got = encode(np.array([v for v, _ in cases]))
    assert got.tolist() == [c for _, c in cases], got
    assert int(encode(np.array([math.nan]))[0]) & 0x7F == 0x7F


def test_encode_special_values():
    check_encode_special(mx.e4m3_encode)


def test_e8m0_values():
    d = mx.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255], dtype=np.uint8))
    assert d[:6].tolist() == [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127]
    assert np.isnan(d[6])


# ---------------------------------------------------------------------------
# pin MX4: the shared-exponent choice on hand-worked blocks
# ---------------------------------------------------------------------------


def check_quantize_worked(quantize):
    # block 0: max |v| = 1.0 -> shared exponent 0 - 8, scale byte 119;
    #   1.0 * 2^8 = 256 -> 0x78, 0.5 -> 128 -> 0x70, -0.25 -> 64 -> 0xE8
    # block 1: all zero -> scale byte 0, zero codes
    # block 2: max |v| = 3.0 (log2 in [1, 2)) -> shared -7, byte 120;
    #   3 * 2^7 = 384 -> 0x7C, 1/128 * 2^7 = 1 -> 0x38
    # block 3: max |v| = 2^-130 (bf16 subnormal) -> shared clamps to -127,
    #   byte 0; 2^-130 * 2^127 = 1/8 -> 0x20
    a = np.zeros((1, 4 * GROUP))
    a[0, 0:3] = [1.0, 0.5, -0.25]
    a[0, 64] = 3.0
    a[0, 65] = 1.0 / 128
    a[0, 96] = 2.0 ** -130
    q, s = quantize(a)
    assert s.tolist() == [[119, 0, 120, 0]]
    assert q[0, 0:3].tolist() == [0x78, 0x70, 0xE8]
    assert not q[0, 3:64].any()
    assert q[0, 64:66].tolist() == [0x7C, 0x38]
    assert q[0, 96] == 0x20
    # a ragged last group is scaled by its own elements only
    r = np.zeros((1, 40))
    r[0, 0] = 100.0
    r[0, 35] = 0.75
    q, s = quantize(r)
    assert s.shape == (1, 2) and s[0, 1] == 127 - 1 - 8
    assert q[0, 35] == mx.e4m3_encode(np.array([0.75 * 2.0 ** 9]))[0] == 0x78 + 4


def test_quantize_worked_blocks():
    check_quantize_worked(mx.mx_quantize)


# ---------------------------------------------------------------------------
# pin MX5: exact round trip of already-quantised data whose block maximum
# lies in the top binade, and the format's error bound on random data
# ---------------------------------------------------------------------------


def check_roundtrip(quantize, dequantize):
    rng = np.random.default_rng(5)
    rows, G = 7, 5
    codes = rng.integers(0, 0x7F, size=(rows, G * GROUP)).astype(np.uint8)
    codes |= (rng.random((rows, G * GROUP)) < 0.5).astype(np.uint8) << 7
    top = rng.integers(0x78, 0x7F, size=(rows, G)).astype(np.uint8)
    where = rng.integers(0, GROUP, size=(rows, G))
    for r in range(rows):
        for g in range(G):
            codes[r, g * GROUP + where[r, g]] = top[r, g] | (codes[r, g * GROUP] & 0x80)
    scales = rng.integers(60, 200, size=(rows, G)).astype(np.uint8)
    v = _torch_decode(codes) * np.repeat(_e8m0(scales), GROUP, axis=1)
    assert np.array_equal(dequantize(codes, scales), v)
    q2, s2 = quantize(v)
    assert np.array_equal(s2, scales)
    assert np.array_equal(q2, codes)


def check_error_bound(quantize, dequantize):
    rng = np.random.default_rng(6)
    a = rng.standard_normal((64, 3 * GROUP)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))
    q, s = quantize(a)
    d = dequantize(q, s)
    shared = np.repeat(s.astype(np.float64) - 127, GROUP, axis=1)
    mag = np.floor(np.log2(np.abs(a)))
    bound = np.maximum(np.exp2(mag - 4), np.exp2(shared - 10))  # half a step
    # above 448 * 2^shared the element saturates: exactly that value
    sat = np.abs(a) > 448.0 * np.exp2(shared)
    assert np.all(np.abs(d - a)[~sat] <= bound[~sat])
    assert np.array_equal(d[sat], np.sign(a[sat]) * 448.0 * np.exp2(shared[sat]))
    assert sat.any()  # the block maximum can land in (448, 512) * 2^shared
    assert np.all(np.abs(a) < 512.0 * np.exp2(shared))


def test_quantize_roundtrip_and_error_bound():
    check_roundtrip(mx.mx_quantize, mx.mx_dequantize)
    check_error_bound(mx.mx_quantize, mx.mx_dequantize)


# ---------------------------------------------------------------------------
# pin MX6: the MX grouped matmul -- a closed form that depends only on the
# scales (unit codes), and brute force with torch-decoded operands over a
# ragged group_list with empty experts
# ---------------------------------------------------------------------------


def check_gmm_mx_closed_form(gmm_mx):
    rng = np.random.default_rng(7)
    M, N, G = 5, 3, 4
    xq = np.full((M, G * GROUP), 0x38, dtype=np.uint8)  # 1.0
    wq = np.full((1, N, G * GROUP), 0x38, dtype=np.uint8)
    xs = rng.integers(120, 135, size=(M, G)).astype(np.uint8)
    ws = rng.integers(120, 135, size=(1, N, G)).astype(np.uint8)
    y = gmm_mx(xq, xs, wq, ws, np.array([M]))
    for m in range(M):
        for n in range(N):
            want = sum(GROUP * 2.0 ** (int(xs[m, j]) - 127) * 2.0 ** (int(ws[0, n, j]) - 127)
                       for j in range(G))
            assert y[m, n] == want


def _brute_gmm_mx(xq, xs, wq, ws, gl):
    x = _torch_decode(xq)
    w = _torch_decode(wq)
    M, K = x.shape
    E, N, _ = w.shape
    y = np.zeros((M, N))
    row = 0
    for e in range(E):
        for _ in range(int(gl[e])):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += (x[row, k] * 2.0 ** (int(xs[row, k // GROUP]) - 127)
                            * w[e, n, k] * 2.0 ** (int(ws[e, n, k // GROUP]) - 127))
                y[row, n] = acc
            row += 1
    return y


def _rand_mx(rng, shape, lo=110, hi=140):
    q = rng.integers(0, 0x7F, size=shape).astype(np.uint8)
    q |= (rng.random(shape) < 0.5).astype(np.uint8) << 7
    s = rng.integers(lo, hi, size=shape[:-1] + (shape[-1] // GROUP,)).astype(np.uint8)
    return q, s


def check_gmm_mx_brute(gmm_mx):
    rng = np.random.default_rng(8)
    gl = np.array([2, 0, 3, 1, 0])
    E, N, K = len(gl), 3, 2 * GROUP
    xq, xs = _rand_mx(rng, (int(gl.sum()), K))
    wq, ws = _rand_mx(rng, (E, N, K))
    y = gmm_mx(xq, xs, wq, ws, gl)
    np.testing.assert_allclose(y, _brute_gmm_mx(xq, xs, wq, ws, gl), rtol=1e-12, atol=0)


def test_gmm_mx_closed_form_and_brute_force():
    check_gmm_mx_closed_form(mx.gmm_mx)
    check_gmm_mx_brute(mx.gmm_mx)


# ---------------------------------------------------------------------------
# pin MX7: the fused gate_up GMM + SwiGLU reads gate rows first, then up rows
# (brute force, the activation from its textbook form)
# ---------------------------------------------------------------------------


def check_gmm_swiglu_mx_brute(gmm_swiglu_mx):
    rng = np.random.default_rng(9)
    gl = np.array([1, 0, 2])
    E, I, K = len(gl), 2, GROUP
    xq, xs = _rand_mx(rng, (int(gl.sum()), K), 112, 120)
    wq, ws = _rand_mx(rng, (E, 2 * I, K), 112, 120)
    h = _brute_gmm_mx(xq, xs, wq, ws, gl)
    want = np.zeros((int(gl.sum()), I))
    for r in range(want.shape[0]):
        for c in range(I):
            g, u = h[r, c], h[r, I + c]
            want[r, c] = g / (1.0 + math.exp(-g)) * u
    got = gmm_swiglu_mx(xq, xs, wq, ws, gl)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)


def test_gmm_swiglu_mx_brute_force():
    check_gmm_swiglu_mx_brute(mx.gmm_swiglu_mx)


def check_block_mx(block):
    rng = np.random.default_rng(10)
    gl = np.array([2, 0, 1])
    E, H, I = len(gl), 2 * GROUP, GROUP
    x = rng.standard_normal((int(gl.sum()), H))
    w1q, w1s = _rand_mx(rng, (E, 2 * I, H), 112, 118)
    w2q, w2s = _rand_mx(rng, (E, H, I), 112, 118)
    out = block(x, w1q, w1s, w2q, w2s, gl)
    # the steps in the pages' order, each by brute force
    xq, xs = mx.mx_quantize(x)
    assert np.array_equal(out["xq"], xq) and np.array_equal(out["xs"], xs)
    h = _brute_gmm_mx(xq, xs, w1q, w1s, gl)
    a = h[:, :I] / (1.0 + np.exp(-h[:, :I])) * h[:, I:]
    np.testing.assert_allclose(out["a"], a, rtol=1e-12, atol=1e-300)
    aq, as_ = mx.mx_quantize(out["a"])
    assert np.array_equal(out["aq"], aq) and np.array_equal(out["as_"], as_)
    np.testing.assert_allclose(out["y"], _brute_gmm_mx(aq, as_, w2q, w2s, gl), rtol=1e-12,
                               atol=1e-300)


def test_expert_block_mx_steps():
    check_block_mx(mx.expert_block_mx)


def check_layer_mx_per_token(layer):
    """out[t] = sum_k probs[t, k] * block_e(x[t]) with e = topk_ids[t, k],
    one token at a time through a one-row group_list (masked slots skipped)."""
    rng = np.random.default_rng(12)
    T, K, E, H, I = 5, 2, 3, 2 * GROUP, GROUP
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    ids[1, 1] = -1
    probs = rng.random((T, K))
    x = rng.standard_normal((T, H))
    w1q, w1s = _rand_mx(rng, (E, 2 * I, H), 112, 118)
    w2q, w2s = _rand_mx(rng, (E, H, I), 112, 118)
    out = layer(x, ids, probs, w1q, w1s, w2q, w2s, E)["out"]
    for t in range(T):
        want = np.zeros(H)
        for k in range(K):
            e = int(ids[t, k])
            if e < 0:
                continue
            gl = np.zeros(E, dtype=np.int64)
            gl[e] = 1
            xq, xs = mx.mx_quantize(x[t:t + 1])
            h = _brute_gmm_mx(xq, xs, w1q, w1s, gl)
            a = h[:, :I] / (1.0 + np.exp(-h[:, :I])) * h[:, I:]
            aq, as_ = mx.mx_quantize(a)
            want += probs[t, k] * _brute_gmm_mx(aq, as_, w2q, w2s, gl)[0]
        np.testing.assert_allclose(out[t], want, rtol=1e-12, atol=1e-300)


def test_layer_mx_per_token():
    check_layer_mx_per_token(mx.moe_layer_forward_mx)


# ---------------------------------------------------------------------------
# mutation test: each planted mistake must fail at least one pin
# ---------------------------------------------------------------------------


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _mut_decode_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp, man = (c >> 3) & 0xF, c & 0x7
    v = np.where(exp == 0, sign * man * 2.0 ** -10, sign * (1 + man / 8) * np.exp2(exp - 8.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def _mut_encode_half_away(v):
    # ties away from zero instead of to even
    v = np.asarray(v, dtype=np.float64)
    nudged = np.where(np.isfinite(v), np.nextafter(np.abs(v), np.inf) * np.sign(v), v)
    nudged = np.where(v == 0, v, nudged)
    return mx.e4m3_encode(nudged)


def _mut_encode_no_saturate(v):
    v = np.asarray(v, dtype=np.float64)
    out = mx.e4m3_encode(v)
    return np.where(np.abs(v) >= 464.0, out | 0x7F, out).astype(np.uint8)


def _mut_quantize_emax7(a):
    saved = mx.E4M3_EMAX
    mx.E4M3_EMAX = 7
    try:
        return mx.mx_quantize(a)
    finally:
        mx.E4M3_EMAX = saved


def _mut_quantize_ceil_log2(a):
    # shared exponent from ceil(log2(amax)) instead of floor
    a = np.asarray(a, dtype=np.float64)
    G = a.shape[-1] // GROUP
    blocks = a.reshape(a.shape[:-1] + (G, GROUP))
    amax = np.max(np.abs(blocks), axis=-1)
    e = np.ceil(np.log2(np.where(amax > 0, amax, 2.0 ** -200)))
    shared = np.clip(np.where(amax > 0, e - 8, -127), -127, 127)
    codes = mx.e4m3_encode(blocks / np.exp2(shared)[..., None]).reshape(a.shape)
    return codes, (shared + 127).astype(np.uint8)


def _mut_dequant_tile(codes, scales):
    v = mx.e4m3_decode(codes)
    K = v.shape[-1]
    reps = -(-K // scales.shape[-1])
    s = np.tile(mx.e8m0_decode(scales), reps)[..., :K]  # blocks interleaved
    return v * s


def _mut_gmm_mx_one_block_scale(xq, xs, wq, ws, gl):
    # every block of a row takes the scale of the row's first block
    return mx.gmm_mx(xq, np.repeat(xs[..., :1], xs.shape[-1], axis=-1), wq, ws, gl)


def _mut_gmm_swiglu_mx_up_gate(xq, xs, w1q, w1s, gl):
    h = mx.gmm_mx(xq, xs, w1q, w1s, gl)
    I = h.shape[1] // 2
    g, u = h[:, I:], h[:, :I]
    return g / (1.0 + np.exp(-g)) * u


def _mut_block_no_requant(x, w1q, w1s, w2q, w2s, gl):
    # GMM2 fed the activation itself, not its MX quantisation
    out = mx.expert_block_mx(x, w1q, w1s, w2q, w2s, gl)
    w2 = mx.mx_dequantize(w2q, w2s)
    off = np.concatenate([[0], np.cumsum(gl)])
    y = np.zeros_like(out["y"])
    for e in range(len(gl)):
        y[off[e]:off[e + 1]] = out["a"][off[e]:off[e + 1]] @ w2[e].T
    out["y"] = y
    return out


def test_mutants_are_caught():
    cases = {
        "decode_bias8": lambda: _fails(check_decode_all_codes, _mut_decode_bias8),
        "encode_half_away": lambda: _fails(check_encode_special, _mut_encode_half_away)
        or _fails(check_encode_vs_torch, _mut_encode_half_away),
        "encode_no_saturate": lambda: _fails(check_encode_special, _mut_encode_no_saturate),
        "quantize_emax7": lambda: _fails(check_quantize_worked, _mut_quantize_emax7),
        "quantize_ceil_log2": lambda: _fails(check_quantize_worked, _mut_quantize_ceil_log2),
        "dequant_tile": lambda: _fails(check_roundtrip, mx.mx_quantize, _mut_dequant_tile),
        "gmm_mx_one_block_scale": lambda: _fails(check_gmm_mx_closed_form,
                                                 _mut_gmm_mx_one_block_scale),
        "gmm_swiglu_mx_up_gate": lambda: _fails(check_gmm_swiglu_mx_brute,
                                                _mut_gmm_swiglu_mx_up_gate),
        "block_no_requant": lambda: _fails(check_block_mx, _mut_block_no_requant),
    }
    missed = [name for name, caught in cases.items() if not caught()]
    assert not missed, f"mutants not caught by any pin: {missed}"
