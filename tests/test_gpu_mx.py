"""MXFP8 (A8W8-FP) path on the GPU against the oracle (oracle/mx_ref.py).

* mx_quantize and moe_permute_mx: bit-exact codes and scales (both sides
  decide on the same bf16 inputs, exactly).
* gmm_mx_fwd: identical quantised operands on both sides; bf16 output within
  rtol = atol = 1e-2 of the exact result.
* gmm_mx_fwd_swiglu: the requantisation of A is decided on the kernel's A
  (fp32 accumulators fed by the scaled fp8 MFMA), the oracle's on the exact
  A.  Neither the pages nor the OCP MX definition fix how precisely the MFMA
  sums a block of fp8 products, so two checks split the question:
  - integer-valued operands (test_gmm_mx_swiglu_requant_exact): every block
    sum is exact in any accumulator as wide as a bf16 significand, so both
    sides decide on the same G and U; codes and scales must be bit-exact
    except within a few fp32 ulps of the activation of a rounding boundary;
  - random operands: the block sums are taken as accurate to the fp16
    significand of each block's largest product, block errors independent
    (BLOCK_SUM_ERR, a stated reading, not a measurement).  A code or scale
    may differ only where the exact value lies within that bound of a
    rounding boundary; there either neighbour is valid, and at most
    AMBIGUOUS_CAP of the decisions may be such cases.  Everything else is
    bit-exact.
* the whole MX layer: outputs within rtol = atol = 1e-2, plus, per element,
  the largest change those boundary cases can cause downstream.

Scale padding bytes are filled with 0xFF (an E8M0 NaN) before each call: a
kernel that read padding as a scale would produce NaNs.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_moe_amd as moe
import oracle
import workloads
from oracle import mx_ref
from tests.gpu_util import assert_close, bf16_dev, dev_f64, f64, require_gpu

pytestmark = pytest.mark.gpu

GROUP = 32


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _u8(t):
    return t.detach().cpu().numpy()


def _scales_buf(rows_shape, K, dev):
    ld = moe.mx_scale_ld(K)
    return torch.full(tuple(rows_shape) + (ld,), 0xFF, dtype=torch.uint8, device=dev)


def _mx_dev(codes, scales, dev):
    """Upload an MX pair, scales padded to the device stride with 0xFF."""
    K = codes.shape[-1]
    ld = moe.mx_scale_ld(K)
    pad = np.full(scales.shape[:-1] + (ld,), 0xFF, dtype=np.uint8)
    pad[..., :scales.shape[-1]] = scales
    return torch.from_numpy(np.ascontiguousarray(codes)).to(dev), torch.from_numpy(pad).to(dev)


def _quantize_dev(bits, dev):
    """Device Q_MX of bf16 bits with poisoned scale padding."""
    x = bf16_dev(bits, dev)
    K = x.shape[-1]
    q = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    s = _scales_buf(x.shape[:-1], K, dev)
    moe.mx_quantize(x, out=(q, s))
    return q, s


# ---------------------------------------------------------------------------
# quantiser and permute: bit-exact
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("rows,K", [(1, 32), (5, 64), (37, 224), (300, 2048), (64, 4096)])
def test_mx_quantize_bit_exact(dev, rows, K):
    rng = np.random.default_rng(rows * 7 + K)
    bits = workloads.wide_range_bf16(rng, (rows, K))
    if rows >= 5:
        bits[1, :32] = 0x0001        # smallest bf16 subnormal: scale clamps at 2^-127
        bits[2, :] = 0x8000          # -0.0 everywhere
        bits[3, :32] = 0x7F7F        # largest finite bf16
    print(f"mx_quantize rows={rows} K={K}", flush=True)
    q, s = _quantize_dev(bits, dev)
    torch.cuda.synchronize()
    rq, rs = mx_ref.mx_quantize(f64(bits))
    KB = rs.shape[1]
    assert np.array_equal(_u8(s)[:, :KB], rs)
    assert np.array_equal(_u8(q), rq)
    assert (_u8(s)[:, KB:] == 0xFF).all()  # padding untouched


def _routing(name):
    if name == "tiny":
        wl = workloads.tiny()
        return wl["x"], wl["topk_ids"], wl.dims["E"]
    if name == "decode":
        wl = workloads.decode(with_weights=False)
        return wl["x"], wl["topk_ids"], wl.dims["E"]
    rng = np.random.default_rng(91)
    T, K, E, H = 1000, 8, 128, 2048   # ragged token count, masked slots
    ids, _ = workloads.softmax_topk_routing(rng, T, E, K)
    ids[rng.random((T, K)) < 0.1] = -1
    return workloads.wide_range_bf16(rng, (T, H), -8, 8), ids, E


@pytest.mark.parametrize("name", ["tiny", "decode", "masked"])
def test_permute_mx_bit_exact(dev, name):
    x, ids, E = _routing(name)
    T, H = x.shape
    S = T * ids.shape[1]
    print(f"moe_permute_mx {name}: T={T} top_k={ids.shape[1]} H={H} E={E}", flush=True)
    xs = _scales_buf((S,), H, dev)
    xq, xs, rmap, sslot, tpe = moe.moe_permute_mx(
        bf16_dev(x, dev), torch.from_numpy(ids).to(dev), E,
        out=(None, xs, None, None, None))
    torch.cuda.synchronize()
    x_perm, row_id_map, sorted_slot, counts = oracle.permute(f64(x), ids, E)
    R = int(counts.sum())
    assert _u8(tpe).tolist() == counts.tolist()
    assert _u8(rmap).tolist() == row_id_map.tolist()
    rq, rs = mx_ref.mx_quantize(x_perm)
    KB = rs.shape[1]
    assert np.array_equal(_u8(xq)[:R], rq)
    assert np.array_equal(_u8(xs)[:R, :KB], rs)


# ---------------------------------------------------------------------------
# MX grouped matmul
# ---------------------------------------------------------------------------


def _gmm_case(name):
    """x (bf16 bits, quantised by each side) and w as an MX pair: drawn as
    bf16 and quantised by each side for the small cases, drawn directly as
    MX bytes for the large ones."""
    rng = np.random.default_rng({"tiny": 51, "ragged": 52, "sweep": 53, "decode": 54,
                                 "ep": 55, "stream_ragged": 56, "e1024_stream": 57,
                                 "e1024_tile": 58}[name])
    if name.startswith("e1024"):
        # E = 1024 (the API limit), most experts empty; M_cap <= 8E streams
        M = 3000 if name == "e1024_stream" else 9000
        gl = workloads.random_group_list(rng, M, 1024, empty_frac=0.7, fill=0.95)
        M_cap = int(gl.sum()) + 16
        x = workloads.normal_bf16(rng, (M_cap, 128))
        return x, ("bf16", workloads.normal_bf16(rng, (1024, 136, 128), 0.02)), gl
    if name == "ep":
        wl = workloads.ep_slice(with_weights=False, with_acts=False)
        gl = wl["group_list"]
        M, K, N = int(gl.sum()), 4096, 3072
    else:
        M, K, N, gl = {
            "tiny": (5, 64, 64, [1, 2, 0, 2]),
            "ragged": (700, 224, 520, [0, 300, 0, 250, 100, 50]),  # K % 64 == 32
            # weight streaming (M_cap <= 8E): an expert past 32 rows, ragged K and N
            "stream_ragged": (100, 224, 520, [3, 0, 40, 1, 0, 0, 2, 9, 0, 5, 0, 33, 0, 1, 6, 0]),
            "sweep": (1024, 512, 1024, None),
            "decode": (512, 2048, 1024, None),
        }[name]
        if gl is None:
            E = 8 if name == "sweep" else 256
            gl = rng.multinomial(M, np.ones(E) / E)
    gl = np.asarray(gl, dtype=np.int64)
    M_cap = int(gl.sum()) + 16
    x = workloads.normal_bf16(rng, (M_cap, K))
    if name in ("tiny", "ragged", "sweep", "stream_ragged"):
        w_bits = workloads.normal_bf16(rng, (len(gl), N, K), 0.02)
        return x, ("bf16", w_bits), gl
    return x, ("mx",) + workloads.mx_random(rng, (len(gl), N, K), 0.02), gl


def _weights(kind, dev):
    """(device codes, device scales, oracle codes, oracle scales)."""
    if kind[0] == "bf16":
        wq, wsc = _quantize_dev(kind[1], dev)
        rq, rs = mx_ref.mx_quantize(f64(kind[1]))
        return wq, wsc, rq, rs
    wq, wsc = _mx_dev(kind[1], kind[2], dev)
    return wq, wsc, kind[1], kind[2]


def _sample_rows(gl, n, rng, max_experts=8):
    """First and last row of up to max_experts experts (the largest, the
    smallest non-empty, the rest at random) plus n random rows of those."""
    off = np.concatenate([[0], np.cumsum(gl)])
    live = np.nonzero(gl)[0]
    order = live[np.argsort(-gl[live], kind="stable")]
    pick = set([int(order[0]), int(order[-1])])
    rest = [int(e) for e in order[1:-1]]
    rng.shuffle(rest)
    pick.update(rest[:max(0, max_experts - len(pick))])
    rows = []
    for e in sorted(pick):
        rows += [off[e], off[e + 1] - 1]
        rows += list(rng.integers(off[e], off[e + 1], size=max(1, n // len(pick))))
    return np.unique(np.asarray(rows, dtype=np.int64))


def _expert_of_rows(gl, rows):
    off = np.concatenate([[0], np.cumsum(gl)])
    return np.searchsorted(off, rows, side="right") - 1


@pytest.mark.parametrize("name", ["tiny", "ragged", "stream_ragged", "sweep", "decode", "ep",
                                  "e1024_stream", "e1024_tile"])
def test_gmm_mx_fwd(dev, name):
    x, wkind, gl = _gmm_case(name)
    E, N, K = wkind[1].shape
    M_cap, R = x.shape[0], int(gl.sum())
    print(f"gmm_mx_fwd {name}: M_cap={M_cap} K={K} N={N} E={E} R={R}", flush=True)
    xq, xs = _quantize_dev(x, dev)
    wq, wsc, rwq, rws = _weights(wkind, dev)
    g = torch.from_numpy(gl).to(dev)
    y = torch.full((M_cap, N), float("nan"), dtype=torch.bfloat16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.gmm_mx_fwd(xq, xs, wq, wsc, g, out=y, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    yd = dev_f64(y)
    assert np.isnan(yd[R:]).all()  # rows past R untouched
    rows = np.arange(R) if R <= 2048 else _sample_rows(gl, 192, np.random.default_rng(7))
    rxq, rxs = mx_ref.mx_quantize(f64(x[rows]))
    if R <= 2048:
        ref = mx_ref.gmm_mx(rxq, rxs, rwq, rws, gl)
    else:  # the per-row definition, expert by expert
        ex = _expert_of_rows(gl, rows)
        ref = np.zeros((len(rows), N))
        for e in np.unique(ex):
            sel = ex == e
            ref[sel] = mx_ref.gmm_mx(rxq[sel], rxs[sel], rwq[e:e + 1], rws[e:e + 1],
                                     np.array([int(sel.sum())]))
    assert_close(yd[rows], ref, f"gmm_mx_fwd {name}")


# ---------------------------------------------------------------------------
# fused GMM1 + SwiGLU + Q_MX
# ---------------------------------------------------------------------------


# Precision of the scaled fp8 MFMA's block sum (v_mfma_scale_f32_32x32x64_f8f6f4
# adds 64 exact fp8 products per instruction).  The pages name the formats but
# not this precision, and the OCP MX v1.0 definition leaves it to the
# implementation.  Reading: each block sum is accurate to the fp16
# significand of its largest product, |error| <= 2^-10 * m_j, and the errors
# of different blocks are independent, so along a row they add as
# 2^-10 * sqrt(sum_j m_j^2); the fp32 accumulation across blocks adds 2^-22
# of the absolute sum of the products.
BLOCK_SUM_ERR = 2.0 ** -10
# At that bound, about 4-11 % of the requantisation decisions on the random
# cases below have a rounding boundary within reach (the fraction depends on
# the exact A and the bound only, not on the device); more than this means
# the bound no longer discriminates.
AMBIGUOUS_CAP = 0.12


def _a_error_bound(h, habs, hpmx):
    """Bound on |A_kernel - A_exact| for A = SiLU(G) U (G and U from the
    MFMA chain; see above), plus the fp32 activation itself (ACT_ERR |A|)."""
    I = h.shape[1] // 2
    G, U = h[:, :I], h[:, I:]
    d = BLOCK_SUM_ERR * hpmx + 2.0 ** -22 * habs
    dG, dU = d[:, :I], d[:, I:]
    s = mx_ref.sigmoid(G)
    dA_dG = np.abs(U * (s + G * s * (1 - s)))
    dA_dU = np.abs(G * s)
    return dA_dG * dG + dA_dU * dU + ACT_ERR * np.abs(G * s * U) + 1e-30


# fp32 evaluation of SiLU(G) * U = G * U / (1 + e^-G): a few roundings and
# exp's argument reduction (|G| < 2^6 here) stay below 2^-18 relative.
ACT_ERR = 2.0 ** -18


def check_requantized(aq, as_, a_ref, delta, what, cap=AMBIGUOUS_CAP):
    """Device (aq, as_) against Q_MX of the exact A: equal wherever the
    decision is unique for every value within +-delta of A; elsewhere one of
    the decisions some value in that interval takes.  Returns, per element,
    the largest change of the dequantised value those cases allow."""
    rows, I = a_ref.shape
    G = I // GROUP
    rq, rs = mx_ref.mx_quantize(a_ref)
    amax = np.abs(a_ref).reshape(rows, G, GROUP).max(axis=2)
    dmax = delta.reshape(rows, G, GROUP).max(axis=2)
    # scale: floor(log2 amax) over [amax - dmax, amax + dmax]
    lo = np.floor(np.log2(np.maximum(amax - dmax, 1e-300)))
    hi = np.floor(np.log2(np.maximum(amax + dmax, 1e-300)))
    scale_amb = (lo != hi) & (amax > 0)
    as_dev = as_[:, :G].astype(np.int64)
    ok_scale = (as_dev == rs) | (scale_amb & (np.abs(as_dev - rs.astype(np.int64)) <= 1))
    assert ok_scale.all(), f"{what}: {int((~ok_scale).sum())} scale bytes differ"
    # codes, in groups whose scale is unique: the codes of A -+ delta
    X = np.repeat(rs.astype(np.float64) - 127, GROUP, axis=1)
    f = a_ref / np.exp2(X)
    d = delta / np.exp2(X)
    c_lo, c_hi = mx_ref.e4m3_encode(f - d), mx_ref.e4m3_encode(f + d)
    grp_amb = np.repeat(scale_amb, GROUP, axis=1)
    code_amb = (c_lo != c_hi) & ~grp_amb
    exact = ~code_amb & ~grp_amb
    bad = exact & (aq != rq)
    if bad.any():
        idx = np.argwhere(bad)[:8]
        lines = [f"  [{r},{c}] A={a_ref[r, c]:.9g} scaled={f[r, c]:.9g} bound={d[r, c]:.3g} "
                 f"dev={mx_ref.e4m3_decode(aq[r:r + 1, c])[0]:.6g} "
                 f"ref={mx_ref.e4m3_decode(rq[r:r + 1, c])[0]:.6g}" for r, c in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} codes with a unique decision differ; "
                             f"rows {np.unique(np.argwhere(bad)[:, 0]).size}, cols "
                             f"{np.unique(np.argwhere(bad)[:, 1])[:16].tolist()}\n"
                             + "\n".join(lines))
    va, vb = mx_ref.e4m3_decode(c_lo[code_amb]), mx_ref.e4m3_decode(c_hi[code_amb])
    vd = mx_ref.e4m3_decode(aq[code_amb])
    assert np.all((vd >= np.minimum(va, vb)) & (vd <= np.maximum(va, vb))), \
        f"{what}: a boundary code outside its two candidates"
    frac = (code_amb | grp_amb).mean()
    print(f"{what}: {frac:.2%} of the code decisions lie within the error bound of a "
          f"boundary; {scale_amb.mean():.2%} of the scale decisions", flush=True)
    assert frac <= cap, f"{what}: {frac:.2e} of the decisions are ambiguous (cap {cap})"
    # change bound: one E4M3 step at the element's binade for a boundary
    # code; for a group whose scale is ambiguous, a step at twice the scale
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(f), 2.0 ** -6))) - 3 + X)
    slack = np.where(code_amb, step, 0.0)
    return np.where(grp_amb, 2.0 * np.maximum(step, np.exp2(X - 8)), slack)


def _reference_h(xdq, ex, w_dq):
    """Per row, through its expert: [G | U] (exact), the absolute sum of the
    products, and sqrt(sum_j m_j^2) with m_j the largest |product| of the
    64-element MFMA block j."""
    R, K = xdq.shape
    N = next(iter(w_dq.values())).shape[0]
    nb = (K + 63) // 64
    h = np.zeros((R, N))
    habs = np.zeros((R, N))
    hpmx = np.zeros((R, N))
    for e in np.unique(ex):
        w = w_dq[e]
        wa = np.zeros((N, nb * 64))
        wa[:, :K] = np.abs(w)
        wa = wa.reshape(N, nb, 64)
        for i in np.nonzero(ex == e)[0]:
            h[i] = w @ xdq[i]
            xa = np.zeros(nb * 64)
            xa[:K] = np.abs(xdq[i])
            p = wa * xa.reshape(1, nb, 64)
            habs[i] = p.sum(axis=(1, 2))
            m = p.max(axis=2)
            hpmx[i] = np.sqrt((m * m).sum(axis=1))
    return h, habs, hpmx


def _swiglu_case(name):
    rng = np.random.default_rng({"tiny": 61, "ragged": 62, "decode": 63, "prefill": 64,
                                 "stream_ragged": 65}[name])
    M, K, I, gl = {
        "tiny": (5, 64, 32, [1, 2, 0, 2]),
        "ragged": (700, 224, 160, [0, 300, 0, 250, 100, 50]),  # I not a multiple of 128
        "stream_ragged": (100, 224, 160, [3, 0, 40, 1, 0, 0, 2, 9, 0, 5, 0, 33, 0, 1, 6, 0]),
        "decode": (512, 2048, 512, None),
        "prefill": (32768, 2048, 512, None),
    }[name]
    if gl is None:
        E = 256 if name == "decode" else 128
        gl = rng.multinomial(M, np.ones(E) / E)
    gl = np.asarray(gl, dtype=np.int64)
    M_cap = int(gl.sum()) + 16
    x = workloads.normal_bf16(rng, (M_cap, K))
    w1q, w1s = workloads.mx_random(rng, (len(gl), 2 * I, K), 0.05)
    return x, w1q, w1s, gl


@pytest.mark.parametrize("name", ["tiny", "ragged", "stream_ragged", "decode", "prefill"])
def test_gmm_mx_swiglu_requant(dev, name):
    x, w1q, w1s, gl = _swiglu_case(name)
    E, N2, K = w1q.shape
    I = N2 // 2
    M_cap, R = x.shape[0], int(gl.sum())
    print(f"gmm_mx_fwd_swiglu {name}: M_cap={M_cap} K={K} I={I} E={E} R={R}", flush=True)
    xq, xs = _quantize_dev(x, dev)
    wq, wsc = _mx_dev(w1q, w1s, dev)
    g = torch.from_numpy(gl).to(dev)
    aq = torch.full((M_cap, I), 0x5A, dtype=torch.uint8, device=dev)
    asc = _scales_buf((M_cap,), I, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.gmm_mx_fwd_swiglu(xq, xs, wq, wsc, g, out=(aq, asc), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    aq_d, as_d = _u8(aq), _u8(asc)
    assert (aq_d[R:] == 0x5A).all() and (as_d[R:] == 0xFF).all()
    assert (as_d[:, I // GROUP:] == 0xFF).all()
    rows = np.arange(R) if R <= 4096 else _sample_rows(gl, 256, np.random.default_rng(8))
    ex = _expert_of_rows(gl, rows)
    rxq, rxs = mx_ref.mx_quantize(f64(x[rows]))
    xdq = mx_ref.mx_dequantize(rxq, rxs)
    w_dq = {e: mx_ref.mx_dequantize(w1q[e], w1s[e]) for e in np.unique(ex)}
    h, habs, hpmx = _reference_h(xdq, ex, w_dq)
    a_ref = h[:, :I] * mx_ref.sigmoid(h[:, :I]) * h[:, I:]
    if R <= 4096:  # the oracle's own fused composition over the whole call
        np.testing.assert_allclose(a_ref, mx_ref.gmm_swiglu_mx(rxq, rxs, w1q, w1s, gl),
                                   rtol=1e-12, atol=1e-300)
    check_requantized(aq_d[rows], as_d[rows], a_ref, _a_error_bound(h, habs, hpmx),
                      f"gmm_mx_fwd_swiglu {name}")


@pytest.mark.parametrize("name", ["tiny", "ragged", "stream_ragged", "decode", "prefill"])
def test_gmm_mx_swiglu_requant_exact(dev, name):
    """Integer-valued operands (workloads.mx_small_integers): G and U are
    exact on both sides, so the requantisation is decided on the same values
    up to the fp32 evaluation of the activation; codes and scales must be
    bit-exact outside that band, which holds a fraction of a percent of the
    decisions (on the 160 of the tiny case, the two A = 0 whose sign of zero
    may go either way)."""
    x, w1q, _, gl = _swiglu_case(name)
    rng = np.random.default_rng(len(name) * 101 + x.shape[0])
    E, N2, K = w1q.shape
    I = N2 // 2
    M_cap, R = x.shape[0], int(gl.sum())
    xq, xs = workloads.mx_small_integers(rng, (M_cap, K))
    w1q, w1s = workloads.mx_small_integers(rng, (E, N2, K))
    print(f"gmm_mx_fwd_swiglu exact {name}: M_cap={M_cap} K={K} I={I} E={E} R={R}", flush=True)
    xqd, xsd = _mx_dev(xq, xs, dev)
    wq, wsc = _mx_dev(w1q, w1s, dev)
    g = torch.from_numpy(gl).to(dev)
    aq = torch.full((M_cap, I), 0x5A, dtype=torch.uint8, device=dev)
    asc = _scales_buf((M_cap,), I, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.gmm_mx_fwd_swiglu(xqd, xsd, wq, wsc, g, out=(aq, asc), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    aq_d, as_d = _u8(aq), _u8(asc)
    assert (aq_d[R:] == 0x5A).all() and (as_d[R:] == 0xFF).all()
    rows = np.arange(R) if R <= 4096 else _sample_rows(gl, 256, np.random.default_rng(8))
    ex = _expert_of_rows(gl, rows)
    xdq = mx_ref.mx_dequantize(xq[rows], xs[rows])
    h = np.zeros((len(rows), N2))
    for e in np.unique(ex):
        sel = ex == e
        h[sel] = xdq[sel] @ mx_ref.mx_dequantize(w1q[e], w1s[e]).T  # exact in float64
    G, U = h[:, :I], h[:, I:]
    assert np.abs(h).max() < 2.0 ** 6, "keep exp's argument small (ACT_ERR)"
    a_ref = G * mx_ref.sigmoid(G) * U
    if R <= 4096:
        np.testing.assert_allclose(a_ref, mx_ref.gmm_swiglu_mx(xq[:R], xs[:R], w1q, w1s, gl),
                                   rtol=1e-12, atol=1e-300)
    check_requantized(aq_d[rows], as_d[rows], a_ref, ACT_ERR * np.abs(a_ref) + 1e-30,
                      f"gmm_mx_fwd_swiglu exact {name}", cap=0.02)


# ---------------------------------------------------------------------------
# the whole A8W8-FP layer: permute_mx -> GMM1+SwiGLU+Q -> GMM2 -> unpermute
# ---------------------------------------------------------------------------


def _layer_case(name):
    wl = {"tiny": workloads.tiny, "decode": lambda: workloads.decode(with_weights=False),
          "prefill": lambda: workloads.prefill(with_weights=False)}[name]()
    d = wl.dims
    rng = np.random.default_rng({"tiny": 71, "decode": 72, "prefill": 73}[name])
    std = 0.05 if name == "tiny" else 0.02
    w1 = workloads.mx_random(rng, (d["E"], 2 * d["I"], d["H"]), std)
    w2 = workloads.mx_random(rng, (d["E"], d["H"], d["I"]), std)
    return wl, w1, w2


def _dev_rows_for(ids, toks, E):
    """Rows of the full call's permutation that hold the sampled tokens'
    slots, in the order the oracle's call on those tokens uses (by expert,
    then slot)."""
    T, K = ids.shape
    _, row_id_map, _ = oracle.permute_maps(ids, E)
    full = np.asarray(row_id_map).reshape(T, K)
    sub_sorted, _, _ = oracle.permute_maps(ids[toks], E)
    sub_sorted = np.asarray(sub_sorted)
    return full[toks[sub_sorted // K], sub_sorted % K]


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_layer_mx(dev, name):
    wl, (w1q, w1s), (w2q, w2s) = _layer_case(name)
    d = wl.dims
    x, ids, probs = wl["x"], wl["topk_ids"], wl["probs"]
    E = d["E"]
    print(f"A8W8-FP layer {name}: T={d['T']} top_k={d['K']} E={E} H={d['H']} I={d['I']}",
          flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    w1qd, w1sd = _mx_dev(w1q, w1s, dev)
    w2qd, w2sd = _mx_dev(w2q, w2s, dev)
    xq, xs, rmap, _, tpe = moe.moe_permute_mx(bf16_dev(x, dev), torch.from_numpy(ids).to(dev), E,
                                              dev_err=err)
    aq, asc = moe.gmm_mx_fwd_swiglu(xq, xs, w1qd, w1sd, tpe, dev_err=err)
    yp = moe.gmm_mx_fwd(aq, asc, w2qd, w2sd, tpe, dev_err=err)
    out = moe.moe_unpermute(yp, rmap, torch.from_numpy(probs).to(dev), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # the oracle on all tokens, or on a sample of them: a token's output
    # depends on its own row only
    T = d["T"]
    toks = np.arange(T) if T <= 512 else np.unique(np.random.default_rng(9).integers(0, T, 96))
    ref = mx_ref.moe_layer_forward_mx(f64(x[toks]), ids[toks], probs[toks].astype(np.float64),
                                      w1q, w1s, w2q, w2s, E)
    # how far requantisation at fp32 may move things: A -> Yp -> out
    gl = ref["tokens_per_expert"]
    ex = _expert_of_rows(gl, np.arange(int(gl.sum())))
    xdq = mx_ref.mx_dequantize(ref["xq"], ref["xs"])
    w1d = {e: mx_ref.mx_dequantize(w1q[e], w1s[e]) for e in np.unique(ex)}
    h, habs, hpmx = _reference_h(xdq, ex, w1d)
    rows = _dev_rows_for(ids, toks, E)
    slack_a = check_requantized(_u8(aq)[rows], _u8(asc)[rows], ref["a"],
                                _a_error_bound(h, habs, hpmx), f"layer {name} A")
    w2abs = {e: np.abs(mx_ref.mx_dequantize(w2q[e], w2s[e])) for e in np.unique(ex)}
    slack_y = np.stack([w2abs[e] @ slack_a[i] for i, e in enumerate(ex)])
    assert_close(dev_f64(yp)[rows], ref["y"], f"layer {name} Yp", extra=slack_y)
    rmap_ref = ref["row_id_map"].reshape(len(toks), -1)
    pr = probs[toks].astype(np.float64)
    slack_o = np.zeros((len(toks), d["H"]))
    for k in range(rmap_ref.shape[1]):
        v = rmap_ref[:, k] >= 0
        slack_o[v] += pr[v, k:k + 1] * slack_y[rmap_ref[v, k]]
    assert_close(dev_f64(out)[toks], ref["out"], f"layer {name} out", extra=slack_o)


def test_layer_mx_pipeline_and_weight_preparation(dev):
    """MoeLayerMX runs the same four calls (bit-identical outputs to the
    explicit chain), and prepare_weights is Q_MX of the transposed bf16
    weights, bit-exact against the oracle."""
    from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayerMX

    wl = workloads.tiny()
    d = wl.dims
    w1, w2 = bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev)
    print("MoeLayerMX tiny: prepare_weights + forward", flush=True)
    (w1q, w1s), (w2q, w2s) = MoeLayerMX.prepare_weights(w1, w2)
    torch.cuda.synchronize()
    w1t, w2t = workloads.reduction_major_weights(wl)
    for (q, s), bits in (((w1q, w1s), w1t), ((w2q, w2s), w2t)):
        rq, rs = mx_ref.mx_quantize(f64(bits))
        assert np.array_equal(_u8(q), rq)
        assert np.array_equal(_u8(s)[..., :rs.shape[-1]], rs)
    L = MoeLayerMX(LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"]), dev)
    x = bf16_dev(wl["x"], dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    probs = torch.from_numpy(wl["probs"]).to(dev)
    out = L.forward(x, ids, probs, (w1q, w1s), (w2q, w2s)).clone()
    xq, xs, rmap, _, tpe = moe.moe_permute_mx(x, ids, d["E"])
    aq, asc = moe.gmm_mx_fwd_swiglu(xq, xs, w1q, w1s, tpe)
    yp = moe.gmm_mx_fwd(aq, asc, w2q, w2s, tpe)
    out2 = moe.moe_unpermute(yp, rmap, probs)
    torch.cuda.synchronize()
    assert int(L.dev_err.item()) == 0
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert L.tokens_per_expert.cpu().tolist() == [1, 2, 0, 2]
