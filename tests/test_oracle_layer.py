"""Pins of the oracle's grouping, expert FFN and layer combine.

* grouping: invariants that determine the table uniquely (every use in
  exactly one column of its expert's group, groups in order of first use,
  columns in ascending use order, shared group first with every row);
* expert FFN: one-hot activations give the dequantised weight column
  (closed form, weights decoded by torch's casts), a random activation
  matches a dense numpy/scipy fp64 formulation, and the down projection is
  linear in its block scales;
* layer: zero routed scale gives exactly the shared expert, zero shared
  weights give exactly the routed sum, rows are permutation-equivariant,
  and the whole tiny layer matches a dense formulation that computes every
  expert for every row with library matmuls.
"""
import numpy as np
import pytest
import scipy.special
import torch

import _bf16
import fixtures


def _f8(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double().numpy()


def _deq_fp8(q, s):
    N, K = q.shape
    return _f8(q) * np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:N, :K]


def _bf(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).double().numpy()


# ---------------------------------------------------------------- grouping
@pytest.mark.parametrize("T,seed,rows", [(1, 1, "iid"), (8, 2, "corr"), (16, 3, "corr"), (33, 4, "iid")])
def test_groups_invariants(orc, T, seed, rows):
    spec = fixtures.spec_with("v3", hidden=256, inter=128, shared_inter=128)
    h = fixtures.host_case(fixtures.make_case(spec, T, seed, rows=rows, requests=max(1, T // 4)), experts=[])
    ids, _, _, _ = orc.route(spec, h["x"], h["router_w"], h["bias"])
    K = spec["top_k"]
    ge, gn, gs, cols, ug = orc.groups(spec, ids)
    G = len(ge)
    assert G == 1 + len(set(ids.ravel().tolist()))
    assert ge[0] == -1 and gn[0] == T
    assert [c for c in cols[gs[0]:gs[0] + T]] == [r * 16 + K for r in range(T)]
    assert len(set(ge[1:].tolist())) == G - 1
    seen = set()
    first_u = []
    for g in range(1, G):
        cl = cols[gs[g]:gs[g] + gn[g]]
        us = [(c // 16) * K + (c % 16) for c in cl]
        assert us == sorted(us)
        for u in us:
            assert ids.ravel()[u] == ge[g] and ug[u] == g
            assert u not in seen
            seen.add(u)
        first_u.append(us[0])
    assert seen == set(range(T * K))
    assert first_u == sorted(first_u)
    assert np.array_equal(gs, np.concatenate([[0], np.cumsum(gn)[:-1]]))


# ---------------------------------------------------------------- expert FFN
def _expert(seed, H=256, I=128, fmt=fixtures.FMT_FP8_B128):
    g = torch.Generator().manual_seed(seed)
    wgu = torch.randn(2 * I, H, generator=g) * 0.02
    wd = torch.randn(H, I, generator=g) * 0.02
    if fmt == fixtures.FMT_FP8_B128:
        a, b = fixtures.quant_fp8_b128(wgu)
        c, d = fixtures.quant_fp8_b128(wd)
    else:
        a, b = fixtures.quant_mxfp4(wgu)
        c, d = fixtures.quant_mxfp4(wd)
    return a.numpy(), b.numpy(), c.numpy(), d.numpy()


def test_ffn_one_hot_closed_form(orc):
    H, I = 256, 128
    q1, s1, q2, s2 = _expert(1)
    Wgu = _deq_fp8(q1, s1); Wd = _deq_fp8(q2, s2)
    for j in (0, 77, 200):
        x = np.zeros(H); x[j] = 1.0
        y, mid = orc.expert_ffn(0, H, I, q1, s1, q2, s2, x)
        g, u = Wgu[:I, j], Wgu[I:, j]
        want_mid = g * scipy.special.expit(g) * u
        assert np.allclose(mid, want_mid, rtol=1e-14, atol=0)
        assert np.allclose(y, Wd @ want_mid, rtol=1e-12, atol=1e-18)


def test_ffn_dense_formulation_fp8(orc):
    H, I = 256, 128
    q1, s1, q2, s2 = _expert(2)
    Wgu = _deq_fp8(q1, s1); Wd = _deq_fp8(q2, s2)
    x = np.random.default_rng(3).standard_normal(H)
    y, mid = orc.expert_ffn(0, H, I, q1, s1, q2, s2, x)
    g, u = Wgu[:I] @ x, Wgu[I:] @ x
    m = g * scipy.special.expit(g) * u
    assert np.allclose(mid, m, rtol=1e-12, atol=1e-16)
    assert np.allclose(y, Wd @ m, rtol=1e-11, atol=1e-16)


def _deq_mxfp4(q, s):
    # E2M1 codes embedded into E4M3 bytes and decoded by torch (see test_oracle_formats)
    lo = q & 0xF; hi = q >> 4
    codes = np.stack([lo, hi], -1).reshape(q.shape[0], -1)
    sgn = (codes >> 3) & 1; e = (codes >> 1) & 3; m = codes & 1
    mag = np.where(e == 0, np.where(m == 0, 0, 6 << 3), ((e + 6) << 3) | (m << 2))
    v = _f8(((sgn << 7) | mag).astype(np.uint8))
    return v * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, 1)


def test_ffn_dense_formulation_mxfp4(orc):
    H, I = 256, 128
    q1, s1, q2, s2 = _expert(4, fmt=fixtures.FMT_MXFP4)
    Wgu = _deq_mxfp4(q1, s1); Wd = _deq_mxfp4(q2, s2)
    x = np.random.default_rng(5).standard_normal(H)
    y, mid = orc.expert_ffn(1, H, I, q1, s1, q2, s2, x)
    g, u = Wgu[:I] @ x, Wgu[I:] @ x
    m = g * scipy.special.expit(g) * u
    assert np.allclose(mid, m, rtol=1e-12, atol=1e-16)
    assert np.allclose(y, Wd @ m, rtol=1e-11, atol=1e-16)


def test_ffn_down_linear_in_scale(orc):
    H, I = 256, 128
    q1, s1, q2, s2 = _expert(6)
    x = np.random.default_rng(7).standard_normal(H)
    y, _ = orc.expert_ffn(0, H, I, q1, s1, q2, s2, x)
    s2b = s2.copy(); s2b[1, 0] *= 4  # rows 128..255 of W_down
    y2, _ = orc.expert_ffn(0, H, I, q1, s1, q2, s2b, x)
    assert np.array_equal(y2[128:], 4 * y[128:]) and np.array_equal(y2[:128], y[:128])


# ---------------------------------------------------------------- layer
def _tiny(T=4, seed=31, **over):
    spec = fixtures.spec_with("tiny", **over)
    case = fixtures.make_case(spec, T, seed, rows="corr" if T % 2 == 0 else "iid", requests=max(1, T // 2))
    return spec, fixtures.host_case(case)


def test_zero_routed_scale_gives_shared(orc):
    spec, h = _tiny(routed_scale=0.0)
    out64, outb = orc.forward(spec, h)
    for r in range(h["x"].shape[0]):
        y, _ = orc.expert_ffn(0, 256, 128, h["sh_w_gate_up"], h["sh_s_gate_up"], h["sh_w_down"],
                              h["sh_s_down"], _bf(h["x"][r]))
        assert np.array_equal(out64[r], y)


def test_zero_shared_gives_routed(orc):
    spec, h = _tiny()
    h0 = dict(h); h0["sh_w_gate_up"] = np.zeros_like(h["sh_w_gate_up"])
    out64, _ = orc.forward(spec, h0)
    ids, w, _, _ = orc.route(spec, h["x"], h["router_w"], h["bias"])
    for r in range(h["x"].shape[0]):
        acc = np.zeros(256)
        for p in range(spec["top_k"]):
            e = ids[r, p]
            y, _ = orc.expert_ffn(0, 256, 128, h["w_gate_up"][e], h["s_gate_up"][e],
                                  h["w_down"][e], h["s_down"][e], _bf(h["x"][r]))
            acc = acc + w[r, p] * y
        assert np.array_equal(out64[r], 0.0 + acc)


def test_row_permutation_equivariance(orc):
    spec, h = _tiny(T=6)
    out64, outb = orc.forward(spec, h)
    perm = np.array([4, 2, 5, 0, 3, 1])
    hp = dict(h); hp["x"] = h["x"][perm].copy()
    o2, b2 = orc.forward(spec, hp)
    assert np.array_equal(o2, out64[perm]) and np.array_equal(b2, outb[perm])


def test_layer_dense_formulation(orc):
    """Every expert for every row with numpy matmuls on torch-decoded weights,
    then masked by the (separately pinned) routing."""
    spec, h = _tiny(T=6, seed=44)
    out64, outb = orc.forward(spec, h)
    ids, w, _, _ = orc.route(spec, h["x"], h["router_w"], h["bias"])
    X = _bf(h["x"])                                  # [T,H]
    E, I = spec["n_experts"], spec["inter"]

    def ffn(wgu, sgu, wd, sd):
        Wgu = _deq_fp8(wgu, sgu); Wd = _deq_fp8(wd, sd)
        G = X @ Wgu[:I].T; U = X @ Wgu[I:].T
        return (G * scipy.special.expit(G) * U) @ Wd.T   # [T,H]

    Y = np.stack([ffn(h["w_gate_up"][e], h["s_gate_up"][e], h["w_down"][e], h["s_down"][e]) for e in range(E)])
    dense_w = np.zeros((X.shape[0], E))
    for r in range(X.shape[0]):
        dense_w[r, ids[r]] = w[r]
    want = ffn(h["sh_w_gate_up"], h["sh_s_gate_up"], h["sh_w_down"], h["sh_s_down"]) \
        + np.einsum("te,eth->th", dense_w, Y)
    assert np.allclose(out64, want, rtol=1e-11, atol=1e-14)
    # the bf16 output is the fp64 output rounded once
    assert all(outb.ravel()[i] == orc.bf16_rne(out64.ravel()[i]) for i in range(0, out64.size, 17))


def test_missing_used_expert_is_an_error(orc):
    spec, h = _tiny(T=2)
    ids, _, _, _ = orc.route(spec, h["x"], h["router_w"], h["bias"])
    h2 = dict(h); h2["w_gate_up"] = list(h["w_gate_up"]); h2["w_gate_up"][int(ids[0, 0])] = None
    with pytest.raises(ValueError):
        orc.forward(spec, h2)


# ---------------------------------------------------------------- residual
def test_residual_zero_is_the_layer(orc):
    """A zero residual (either sign) leaves the layer's output as it is."""
    spec, h = _tiny(T=3)
    out64, outb = orc.forward(spec, h)
    zero = np.zeros_like(h["x"])
    o64, ob = orc.forward_residual(spec, h, zero)
    assert np.array_equal(o64, out64) and np.array_equal(ob, outb)
    o64n, obn = orc.forward_residual(spec, h, zero | np.uint16(0x8000))
    assert np.array_equal(o64n, out64 + 0.0) and np.array_equal(obn, outb)


def test_residual_alone_with_zero_weights(orc):
    """With every expert weight zero the layer is exactly 0, so the output is
    the residual itself, bit for bit (it is already bf16)."""
    spec, h = _tiny(T=2)
    hz = dict(h)
    for k in ("w_gate_up", "w_down"):
        hz[k] = [np.zeros_like(a) for a in h[k]]
    hz["sh_w_gate_up"] = np.zeros_like(h["sh_w_gate_up"])
    hz["sh_w_down"] = np.zeros_like(h["sh_w_down"])
    res = fixtures.bits16(torch.randn(2, 256, generator=torch.Generator().manual_seed(5)).bfloat16())
    o64, ob = orc.forward_residual(spec, hz, res)
    assert np.array_equal(ob, res)
    assert np.array_equal(o64, _bf(res))


def test_residual_is_rounded_once(orc):
    """With the residual set to minus the layer's own bf16 output, one
    rounding of (layer + residual) leaves the layer's rounding error as a
    bf16 value, RNE(layer64 - RNE(layer64)), nonzero wherever the layer is
    not already a bf16 value; rounding the layer to bf16 first and then
    adding would give exactly zero everywhere.  The expected codes come from
    an exact fp64 difference and a brute-force bf16 rounding over the table
    of every bf16 value, not from the oracle's own rounding."""
    spec, h = _tiny(T=3)
    out64, outb = orc.forward(spec, h)
    res = outb ^ np.uint16(0x8000)
    o64, ob = orc.forward_residual(spec, h, res)
    codes, vals = _bf16.table()
    err = out64 - _bf(outb)                 # exact (the operands are within a bf16 ulp)
    assert np.array_equal(o64, err)
    want = np.array([_bf16.brute_rne(float(v), codes, vals) for v in err.ravel()], np.uint16).reshape(ob.shape)
    assert np.array_equal(ob, want)
    assert np.count_nonzero(ob & np.uint16(0x7FFF)) > 0.95 * ob.size


# ---------------------------------------------------------------- expert parallelism
def test_expert_range_all_is_the_layer(orc):
    """Holding every expert (count E, or 0 meaning all) is the whole layer."""
    spec, h = _tiny(T=3)
    full64, fullb = orc.forward(spec, h)
    for first, count in ((0, 16), (0, 0)):
        o64, ob = orc.forward(dict(spec, expert_first=first, expert_count=count), h)
        assert np.array_equal(o64, full64) and np.array_equal(ob, fullb)


def test_expert_shards_sum_to_the_layer(orc):
    """Four shards of four experts each, the shared expert in the first: the
    fp64 shares add up to the whole layer (up to the order of the fp64
    additions); a share is zero for a row none of whose picks it holds."""
    spec, h = _tiny(T=6)
    full64, _ = orc.forward(spec, h)
    ids, _, _, _ = orc.route(spec, h["x"], h["router_w"], h["bias"])
    total = np.zeros_like(full64)
    for s in range(4):
        sp = dict(spec, expert_first=4 * s, expert_count=4, n_shared=1 if s == 0 else 0)
        o64, _ = orc.forward(sp, h)
        total += o64
        if s:
            for r in range(6):
                if not any(4 * s <= e < 4 * s + 4 for e in ids[r]):
                    assert np.all(o64[r] == 0.0)
    assert np.max(np.abs(total - full64)) <= 1e-12 * np.max(np.abs(full64))


def test_expert_shard_without_local_picks_is_the_shared_expert(orc):
    """A row none of whose picks lies in the held range gets exactly the
    shared expert's output (the layer with routed_scale 0)."""
    spec, h = _tiny(T=6)
    ids, _, _, _ = orc.route(spec, h["x"], h["router_w"], h["bias"])
    shared64, _ = orc.forward(dict(spec, routed_scale=0.0), h)
    checked = 0
    for s in range(4):
        sp = dict(spec, expert_first=4 * s, expert_count=4)
        o64, _ = orc.forward(sp, h)
        for r in range(6):
            if not any(4 * s <= e < 4 * s + 4 for e in ids[r]):
                assert np.array_equal(o64[r], shared64[r])
                checked += 1
    assert checked > 0


def test_expert_range_checked(orc):
    spec, h = _tiny(T=1)
    for first, count in ((-1, 4), (14, 4), (3, 0)):
        with pytest.raises(ValueError):
            orc.forward(dict(spec, expert_first=first, expert_count=count), h)
