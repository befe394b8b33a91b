"""GPU path against the fp64 oracle, through the C ABI.

Small cases run the whole batch through the oracle; they are sized to span
several weight chunks (1024-element K chunks, 16-row tiles) with ragged
tails.  Full-size cases (DeepSeek-V3 shape at 1, 8 and 64 rows; the
V4-style MXFP4 layer at 16 rows) are checked on sampled rows the oracle
computes one by one.  Routing must match bit-exactly (ids and order),
outputs within 2e-2 relative L2 and 1e-1 max-abs of the fp64 oracle."""
import numpy as np
import pytest
import torch

import fixtures
import mixture_experts_decode_sigmoid_amd as moe
from _gpu import (MAX_ABS, REL_L2, gpu_case, oracle_route, oracle_rows, parity, run_forward, say)

pytestmark = pytest.mark.gpu

# (name, spec overrides, T, seed, row recipe)
SMALL = [
    ("tiny_t1", dict(), 1, 1, "iid"),
    ("tiny_t8", dict(), 8, 11, "corr"),
    ("tiny_t64", dict(), 64, 12, "iid"),
    ("grouped_k6_bf16bias", dict(n_experts=32, top_k=6, n_group=4, topk_group=2, bias_bf16=1), 13, 13, "iid"),
    ("multichunk_ragged", dict(hidden=1152, inter=640, shared_inter=384, n_experts=24, top_k=5), 9, 14, "corr"),
    ("wide_h3072", dict(hidden=3072, inter=256, shared_inter=256, n_experts=16, top_k=4,
                        n_group=4, topk_group=2), 20, 15, "iid"),
    ("mxfp4_small", dict(hidden=1536, inter=1536, shared_inter=512, n_experts=16, top_k=6,
                         routed_fmt=1, bias_bf16=1), 16, 16, "corr"),
    ("no_shared", dict(n_shared=0, hidden=512, inter=256, n_experts=12, top_k=3), 7, 17, "iid"),
    ("k_equals_e", dict(n_experts=8, top_k=8, hidden=256, inter=128), 3, 18, "iid"),
    # hidden > 16 * 256: a CU's down slice spans two 16-row tiles (the second ragged)
    ("two_down_tiles", dict(hidden=4352, inter=256, shared_inter=256, n_experts=16, top_k=4), 5, 19, "corr"),
    ("two_down_tiles_wide", dict(hidden=4352, inter=256, shared_inter=256, n_experts=16, top_k=4), 24, 20, "iid"),
    ("mxfp4_two_tiles", dict(hidden=4608, inter=512, shared_inter=256, n_experts=16, top_k=6,
                             routed_fmt=1, bias_bf16=1), 12, 21, "corr"),
    # up to 4 rows (one activation load per item, 4 lanes per column) and up
    # to 8 (two loads, 2 lanes per column), with MXFP4 experts, with every
    # row of one request sharing experts (jobs at full column capacity), and
    # with two down tiles
    ("mxfp4_t3", dict(hidden=1536, inter=1536, shared_inter=512, n_experts=16, top_k=6,
                      routed_fmt=1, bias_bf16=1), 3, 22, "corr"),
    ("mxfp4_t6", dict(hidden=1536, inter=1536, shared_inter=512, n_experts=16, top_k=6,
                      routed_fmt=1, bias_bf16=1), 6, 23, "corr"),
    ("four_rows_one_request", dict(hidden=1024, inter=512, shared_inter=256, n_experts=12, top_k=4), 4, 24, "corr"),
    ("two_down_tiles_t2", dict(hidden=4352, inter=256, shared_inter=256, n_experts=16, top_k=4), 2, 25, "corr"),
]


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    moe.lib()
    assert torch.cuda.is_available()


def _spec(over):
    return fixtures.spec_with("tiny", **over)


@pytest.mark.parametrize("name,over,T,seed,rows", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(name, over, T, seed, rows):
    say(f"case {name} T={T} seed={seed}")
    spec = _spec(over)
    case = gpu_case(spec, T, seed, rows=rows, requests=max(1, T // 4))
    layer = moe.Layer(spec, case, max_rows=max(T, 1))
    ids_o, w_o, ge, gg = oracle_route(spec, case)
    assert np.min(ge) > 1e-9 and np.min(gg) > 1e-9
    ids, wts = layer.route(case["x"])
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.allclose(wts.cpu().numpy(), w_o, rtol=1e-6, atol=0)
    out = run_forward(layer, case["x"])
    assert layer.read_error() == 0
    o64, _ = oracle_rows(spec, case, range(T), ids=ids_o)
    rel, mx = parity(out, o64, list(range(T)))
    say(f"  rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


# (E, n_group, topk_group, K, T): group sizes 2..128, powers of two and not
ROUTING = [(48, 4, 2, 6, 9), (256, 2, 1, 8, 5), (256, 4, 2, 8, 7), (256, 8, 4, 8, 16),
           (128, 64, 8, 8, 3), (64, 16, 5, 7, 4), (200, 8, 3, 5, 11)]


@pytest.mark.parametrize("E,ng,kg,K,T", ROUTING, ids=[f"e{r[0]}_g{r[1]}_k{r[3]}" for r in ROUTING])
def test_routing_groupings(E, ng, kg, K, T):
    say(f"routing E={E} ng={ng} kg={kg} K={K} T={T}")
    spec = _spec(dict(n_experts=E, n_group=ng, topk_group=kg, top_k=K))
    case = gpu_case(spec, T, 100 + E + ng, rows="iid")
    layer = moe.Layer(spec, case, max_rows=T)
    ids_o, w_o, ge, gg = oracle_route(spec, case)
    assert np.min(ge) > 1e-9 and np.min(gg) > 1e-9
    ids, wts = layer.route(case["x"])
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.allclose(wts.cpu().numpy(), w_o, rtol=1e-6, atol=0)


@pytest.mark.parametrize("name,over,T,seed,rows", SMALL[:6], ids=[s[0] for s in SMALL[:6]])
def test_small_groups_exact(name, over, T, seed, rows):
    import oracle
    say(f"groups {name} T={T}")
    spec = _spec(over)
    case = gpu_case(spec, T, seed, rows=rows, requests=max(1, T // 4))
    layer = moe.Layer(spec, case, max_rows=T)
    ids_o, _, _, _ = oracle_route(spec, case)
    ge_o, gn_o, gs_o, cols_o, _ = oracle.groups(spec, ids_o)
    ge, gn, gs, cols = layer.groups(case["x"])
    assert ge == ge_o.tolist() and gn == gn_o.tolist() and gs == gs_o.tolist()
    assert cols == cols_o.tolist()


FULL = [
    ("v3_t1", [0]),
    ("v3_t8", [0, 3, 5, 7]),
    ("v3_t64", [0, 17, 42, 63]),
    ("v4_t16", [0, 6, 15]),
    # the 8-way tensor-parallel share of the V3 layer (intermediate 256)
    ("v3tp8_t1", [0]),
    ("v3tp8_t8", [0, 4, 7]),
]


@pytest.fixture(scope="module")
def full_cases():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            spec, case = fixtures.make_workload(name, device="cuda")
            cache[name] = (spec, case)
        return cache[name]
    return get


@pytest.mark.parametrize("name,rows", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled(full_cases, name, rows):
    say(f"full {name} rows={rows}")
    spec, case = full_cases(name)
    T = case["x"].shape[0]
    layer = moe.Layer(spec, case, max_rows=T)
    ids_o, w_o, ge, gg = oracle_route(spec, case)
    assert np.min(ge) > 1e-9 and np.min(gg) > 1e-9
    ids, wts = layer.route(case["x"])
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    D = len(set(ids_o.ravel().tolist()))
    say(f"  distinct routed experts D={D}")
    out = run_forward(layer, case["x"])
    assert layer.read_error() == 0
    o64, _ = oracle_rows(spec, case, rows, ids=ids_o)
    rel, mx = parity(out, o64, rows)
    say(f"  rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS
    assert np.all(np.isfinite(out.view(np.int16).astype(np.float64)))


# The residual add folded into the combine (moe_forward_residual): parity with
# the oracle's one-rounding reading, in place (residual is out) equal to out
# of place bit for bit, in the 1-row, 8-row narrow and the wide stream.
RESID = [
    ("tiny_t1", dict(), 1, 41, "iid"),
    ("tiny_t8", dict(), 8, 42, "corr"),
    ("multichunk_ragged_t9", dict(hidden=1152, inter=640, shared_inter=384, n_experts=24, top_k=5), 9, 43, "corr"),
    ("wide_t37", dict(hidden=512, inter=256, shared_inter=256, n_experts=16, top_k=4), 37, 44, "iid"),
]


@pytest.mark.parametrize("name,over,T,seed,rows", RESID, ids=[s[0] for s in RESID])
def test_residual_parity(name, over, T, seed, rows):
    import oracle
    say(f"residual {name} T={T}")
    spec = _spec(over)
    case = gpu_case(spec, T, seed, rows=rows, requests=max(1, T // 4))
    layer = moe.Layer(spec, case, max_rows=T)
    H = spec["hidden"]
    res = torch.randn(T, H, generator=torch.Generator().manual_seed(seed)).bfloat16().cuda()
    out = layer.forward(case["x"], residual=res)
    torch.cuda.synchronize()
    assert layer.read_error() == 0
    got = fixtures.bits16(out)
    ids, _, _, _ = oracle_route(spec, case)
    used = sorted(set(int(e) for r in range(T) for e in ids[r]))
    h = fixtures.host_case(case, experts=used)
    o64, _ = oracle.forward_residual(spec, h, fixtures.bits16(res))
    rel, mx = parity(got, o64, list(range(T)))
    assert rel <= REL_L2 and mx <= MAX_ABS, (rel, mx)
    # in place: the residual buffer receives the output
    inplace = res.clone()
    layer.forward(case["x"], out=inplace, residual=inplace)
    torch.cuda.synchronize()
    assert np.array_equal(fixtures.bits16(inplace), got)
    # a zero residual gives moe_forward's output bit for bit (no negative zeros
    # in a random layer's output)
    plain = run_forward(layer, case["x"])
    zero = layer.forward(case["x"], residual=torch.zeros_like(res))
    torch.cuda.synchronize()
    assert np.array_equal(fixtures.bits16(zero), plain)
