"""Seeded input generators: shapes, seeds and structure of the workloads."""
import numpy as np

import oracle
import workloads


def test_tiny_matches_worked_example():
    w = workloads.tiny()
    assert oracle.tokens_per_expert(w["topk_ids"], 4).tolist() == [1, 2, 0, 2]
    assert w["x"].dtype == np.uint16 and w["x"].shape == (4, 64)
    assert w["w1"].shape == (4, 64, 64) and w["w2"].shape == (4, 32, 64)
    assert w["dyp"].shape == (5, 64)
    assert (w["probs"] >= 0).all() and (w["probs"] < 1).all()


def test_tiny_is_deterministic():
    a, b = workloads.tiny(), workloads.tiny()
    for k in a.arrays:
        np.testing.assert_array_equal(a[k], b[k])


def test_sweep_group_lists():
    for v in range(3):
        w = workloads.sweep(v)
        gl = w["group_list"]
        assert gl.sum() == 1024 and gl.shape == (8,)
    assert (workloads.sweep(0)["group_list"] == 128).all()
    gl2 = workloads.sweep(2)["group_list"]
    assert gl2[[0, 3, 7]].tolist() == [0, 0, 0]


def test_ep_slice_structure():
    w = workloads.ep_slice(with_weights=False, with_acts=False)
    gl = w["group_list"]
    assert gl.sum() == 16384 and (gl == 0).sum() >= 3
    # the shuffled ids reproduce the group list
    np.testing.assert_array_equal(oracle.tokens_per_expert(w["topk_ids"], 32), gl)


def test_decode_routing_distinct_experts():
    w = workloads.decode(with_weights=False)
    ids, probs = w["topk_ids"], w["probs"]
    assert ids.shape == (64, 8) and probs.shape == (64, 8)
    for t in range(64):
        assert len(set(ids[t].tolist())) == 8
        assert (np.diff(probs[t]) <= 0).all()
