"""Pins of the oracle's routing: logits against a numpy fp64 matmul, scores
against scipy's expit, selection against full stable sorts and an
exhaustive enumeration of the kept group subsets, weights against their
invariants, and the special cases (E = K, ungrouped, exact ties).
"""
import itertools

import numpy as np
import pytest
import scipy.special
import torch

import fixtures


def _bf16_to_f64(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).double().numpy()


def _case(spec, T, seed, rows="iid", requests=1):
    c = fixtures.make_case(spec, T, seed, rows=rows, requests=requests)
    return fixtures.host_case(c, experts=[])


def _bias64(spec, bias):
    return _bf16_to_f64(bias) if spec["bias_bf16"] else bias.astype(np.float64)


def test_scores_match_library(orc):
    spec = fixtures.spec_with("tiny", n_experts=32)
    h = _case(spec, 3, 21)
    x64 = _bf16_to_f64(h["x"]); w64 = _bf16_to_f64(h["router_w"])
    for r in range(3):
        l, s, b = orc.scores(spec, h["x"][r], h["router_w"], h["bias"])
        ref = w64 @ x64[r]
        assert np.allclose(l, ref, rtol=0, atol=1e-13)
        assert np.allclose(s, scipy.special.expit(l), rtol=1e-15, atol=0)
        assert np.array_equal(b, s + _bias64(spec, h["bias"]))


def _brute_route(spec, b, s):
    """Selection by full sorts / subset enumeration (independent of the oracle's loops)."""
    E, K, ng, kg = spec["n_experts"], spec["top_k"], spec["n_group"], spec["topk_group"]
    if ng > 1:
        gsz = E // ng
        gs = [sum(sorted(b[j * gsz:(j + 1) * gsz])[-2:]) for j in range(ng)]
        key = lambda j: (-gs[j], j)
        valid = [S for S in itertools.combinations(range(ng), kg)
                 if all(key(a) < key(o) for a in S for o in range(ng) if o not in S)]
        assert len(valid) == 1
        cand = [e for e in range(E) if e // gsz in valid[0]]
    else:
        cand = list(range(E))
    ids = sorted(cand, key=lambda e: (-b[e], e))[:K]
    w = np.array([s[e] for e in ids])
    return ids, w / w.sum() * spec["routed_scale"]


@pytest.mark.parametrize("name,over,T", [
    ("tiny", {}, 40),
    ("tiny", dict(n_group=4, topk_group=2), 60),          # E=16, 4 groups of 4, keep 2
    ("tiny", dict(n_group=8, topk_group=3, top_k=5), 40),
    ("v3", dict(hidden=256, inter=128, shared_inter=128), 24),   # 256 experts, 8 groups keep 4, top-8
    ("v4", dict(hidden=256, inter=128, shared_inter=128), 24),   # top-6, bf16 bias
])
def test_route_brute_force(orc, name, over, T):
    spec = fixtures.spec_with(name, **over)
    h = _case(spec, T, 100 + T)
    ids, w, ge, gg = orc.route(spec, h["x"], h["router_w"], h["bias"])
    for r in range(T):
        _, s, b = orc.scores(spec, h["x"][r], h["router_w"], h["bias"])
        bi, bw = _brute_route(spec, b, s)
        assert ids[r].tolist() == bi
        assert np.allclose(w[r], bw, rtol=1e-15, atol=0)
        assert len(set(ids[r].tolist())) == spec["top_k"]
        assert np.all(w[r] > 0)
        assert abs(w[r].sum() - spec["routed_scale"]) < 1e-13
        assert ge[r] >= 0 and gg[r] >= 0


def test_all_experts_when_k_equals_e(orc):
    spec = fixtures.spec_with("tiny", n_experts=8, top_k=8)
    h = _case(spec, 5, 3)
    ids, w, _, _ = orc.route(spec, h["x"], h["router_w"], h["bias"])
    for r in range(5):
        _, s, b = orc.scores(spec, h["x"][r], h["router_w"], h["bias"])
        assert sorted(ids[r].tolist()) == list(range(8))
        assert ids[r].tolist() == sorted(range(8), key=lambda e: (-b[e], e))
        assert np.allclose(w[r], s[ids[r]] / s.sum() * 2.5, rtol=1e-15)


def test_one_group_equals_ungrouped(orc):
    """n_group = k_g (every group kept) selects exactly like n_group = 1."""
    spec1 = fixtures.spec_with("tiny", n_experts=32, top_k=6)
    spec4 = dict(spec1, n_group=4, topk_group=4)
    h = _case(spec1, 20, 9)
    a = orc.route(spec1, h["x"], h["router_w"], h["bias"])
    b = orc.route(spec4, h["x"], h["router_w"], h["bias"])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_exact_ties_break_by_lower_index(orc):
    spec = fixtures.spec_with("tiny", n_experts=16, top_k=4)
    h = _case(spec, 6, 4)
    rw = h["router_w"].copy(); bias = h["bias"].copy()
    # duplicate expert 3 into 9 and 12: identical logits, scores and keys
    rw[9] = rw[3]; rw[12] = rw[3]; bias[9] = bias[3]; bias[12] = bias[3]
    # make expert 3 win for every row: large positive bias
    bias[3] = bias[9] = bias[12] = 5.0
    ids, w, _, _ = orc.route(spec, h["x"], rw, bias)
    for r in range(6):
        assert ids[r, :3].tolist() == [3, 9, 12]
        assert w[r, 0] == w[r, 1] == w[r, 2]


def test_group_ties_break_by_lower_group(orc):
    spec = fixtures.spec_with("tiny", n_experts=16, top_k=2, n_group=4, topk_group=1)
    h = _case(spec, 3, 8)
    rw = h["router_w"].copy(); bias = h["bias"].copy()
    # groups 1 and 2 become identical copies and dominate every row
    rw[8:12] = rw[4:8]; bias[8:12] = bias[4:8] = 3.0
    ids, _, _, gg = orc.route(spec, h["x"], rw, bias)
    for r in range(3):
        assert all(4 <= e < 8 for e in ids[r])
        assert gg[r] >= 0


def test_bias_only_steers_selection(orc):
    """Weights use the unbiased score: with a constant bias added to every
    expert the picks and the weights stay the same."""
    spec = fixtures.spec_with("tiny")
    h = _case(spec, 8, 12)
    a = orc.route(spec, h["x"], h["router_w"], h["bias"])
    b = orc.route(spec, h["x"], h["router_w"], h["bias"] + np.float32(0.5))
    assert np.array_equal(a[0], b[0])
    assert np.allclose(a[1], b[1], rtol=1e-15, atol=0)
