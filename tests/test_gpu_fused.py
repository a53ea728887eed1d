"""gmm_fwd_swiglu on the GPU: A = SiLU(G) * U straight from the gate_up
accumulators, against the oracle's unrounded composition; the optional H
output must equal what gmm_fwd writes, bit for bit (same kernels, same
reduction order)."""
import numpy as np
import pytest
import torch

import grouped_gemm_moe_amd as moe
import oracle
import workloads
from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayer
from tests.gpu_util import assert_close, bf16_dev, dev_bits, dev_f64, f64, require_gpu

pytestmark = pytest.mark.gpu

SENT = np.uint16(0x7FC1)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _case(name):
    rng = np.random.default_rng({"tiny": 41, "ragged_I": 42, "decode": 43, "prefill": 44,
                                 "stream_fine": 46}.get(name, 45))
    if name.startswith("sweep"):
        wl = workloads.sweep(int(name[-1]))
        return wl["x"], wl["w"], wl["group_list"], wl.dims["M"]
    shapes = {
        "tiny": (5, 64, 32, [1, 2, 0, 2]),
        "ragged_I": (700, 200, 520, [0, 300, 0, 250, 100]),   # I not a multiple of the 128-column tile
        "decode": (512, 2048, 512, None),                        # weight-streaming path
        # weight streaming with a long reduction (K = 1024), I not a multiple of the
        # 128-column slice, 0-12 rows per expert (up to three row groups)
        "stream_fine": (100, 1024, 504, [12, 0, 9, 1, 2, 3, 5, 0, 12, 4, 7, 11, 6, 8, 10, 10]),
        "prefill": (32768, 2048, 512, None),
    }
    M, K, I, gl = shapes[name]
    if gl is None:
        E = 256 if name == "decode" else 128
        gl = rng.multinomial(M, np.ones(E) / E)
    gl = np.asarray(gl, dtype=np.int64)
    M_cap = M + 16  # rows past R stay untouched
    x = workloads.normal_bf16(rng, (M_cap, K))
    w1 = workloads.normal_bf16(rng, (len(gl), K, 2 * I), 0.05)
    return x, w1, gl, M_cap


@pytest.mark.parametrize("name", ["tiny", "sweep0", "sweep2", "ragged_I", "decode", "stream_fine", "prefill"])
def test_fused_gate_up_swiglu(dev, name):
    x, w1, gl, M_cap = _case(name)
    R = int(gl.sum())
    I = w1.shape[2] // 2
    print(f"gmm_fwd_swiglu {name}: M_cap={M_cap} K={x.shape[1]} I={I} E={len(gl)} R={R}", flush=True)
    xd, wd, g = bf16_dev(x, dev), bf16_dev(w1, dev), torch.from_numpy(gl).to(dev)
    a = bf16_dev(np.full((M_cap, I), SENT, np.uint16), dev)
    a2 = bf16_dev(np.full((M_cap, I), SENT, np.uint16), dev)
    h = bf16_dev(np.full((M_cap, 2 * I), SENT, np.uint16), dev)
    h_ref = bf16_dev(np.full((M_cap, 2 * I), SENT, np.uint16), dev)
    moe.gmm_fwd_swiglu(xd, wd, g, out=a)
    moe.gmm_fwd_swiglu(xd, wd, g, out=a2, h_out=h)
    moe.gmm_fwd(xd, wd, g, out=h_ref)
    torch.cuda.synchronize()
    ref = oracle.gmm_swiglu(f64(x)[:R], f64(w1), gl)
    assert_close(dev_f64(a)[:R], ref, f"{name} a")
    assert (dev_bits(a)[R:] == SENT).all(), "rows past R must stay untouched"
    np.testing.assert_array_equal(dev_bits(a2), dev_bits(a))
    np.testing.assert_array_equal(dev_bits(h), dev_bits(h_ref))


def test_fused_ep_rank_sampled(dev):
    """EP-rank gate_up shape (16384 rows, K=4096, I=1536, Zipf groups), rows
    sampled at every expert's first and last row and at random."""
    wl = workloads.ep_slice(with_acts=False)
    gl = wl["group_list"]
    rng = np.random.default_rng(31)
    x = workloads.normal_bf16(rng, (16384, 4096))
    g = torch.from_numpy(gl).to(dev)
    a = moe.gmm_fwd_swiglu(bf16_dev(x, dev), bf16_dev(wl["w1"], dev), g)
    torch.cuda.synchronize()
    off = oracle.expert_offsets(gl)
    rows = np.unique(np.concatenate([off[:-1][gl > 0], off[1:][gl > 0] - 1, rng.integers(0, 16384, 32)]))
    eo = np.repeat(np.arange(32), gl)
    got = dev_f64(a[torch.from_numpy(rows).to(dev)])
    for i, r in enumerate(rows):
        e = eo[r]
        ref = oracle.gmm_swiglu(f64(x[r:r + 1]), f64(wl["w1"][e:e + 1]), np.array([1]))
        assert_close(got[i], ref[0], f"ep a row {r} (expert {e})")


def test_fused_layer_forward_prefill(dev):
    """The prefill layer with the fused call and no H: out against the oracle
    chain that rounds A once from the unrounded gate_up result."""
    wl = workloads.prefill()
    d = wl.dims
    layer = MoeLayer(LayerShape(d["T"], d["K"], d["E"], d["H"], d["I"]), dev)
    w1, w2 = bf16_dev(wl["w1"], dev), bf16_dev(wl["w2"], dev)
    layer.forward(bf16_dev(wl["x"], dev), torch.from_numpy(wl["topk_ids"]).to(dev),
                  torch.from_numpy(wl["probs"]).to(dev), w1, w2, fused=True, keep_h=False)
    torch.cuda.synchronize()
    assert int(layer.dev_err.item()) == 0
    x_perm, rmap, _, counts = oracle.permute(f64(wl["x"]), wl["topk_ids"], d["E"])
    R = int(counts.sum())
    a = oracle.round_bf16(oracle.gmm_swiglu(x_perm, f64(wl["w1"]), counts))
    yp = oracle.round_bf16(oracle.gmm(a, f64(wl["w2"]), counts))
    out = oracle.unpermute(yp, rmap, wl["probs"].astype(np.float64))
    assert_close(dev_f64(layer.a)[:R], a, "a (fused)")
    assert_close(dev_f64(layer.yp)[:R], yp, "yp")
    assert_close(dev_f64(layer.out), out, "out")
