"""GPU path against the fp64 oracle, through the C ABI.

Small cases run the whole batch through the oracle; they are sized to span
several weight chunks (1024-element K chunks, 16-row tiles) with ragged
tails.  Full-size cases (DeepSeek-V3 shape at 1, 8 and 64 rows; the
V4-style MXFP4 layer at 16 rows; the tensor- and expert-parallel shares) are
checked on every row, with the oracle given only the experts the rows use.  Routing must match bit-exactly (ids and order),
outputs within 2e-2 relative L2 and 1e-1 max-abs of the fp64 oracle."""
import numpy as np
import pytest
import torch

import fixtures
import mixture_experts_decode_sigmoid_amd as moe
from _gpu import (MAX_ABS, REL_L2, bf16_to_f64, gpu_case, oracle_route, oracle_rows, parity, run_forward, say)

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
    ("mxfp4_small", dict(hidden=2048, inter=1536, shared_inter=512, n_experts=16, top_k=6,
                         routed_fmt=1, bias_bf16=1), 16, 16, "corr"),
    ("no_shared", dict(n_shared=0, hidden=512, inter=256, n_experts=12, top_k=3), 7, 17, "iid"),
    # no shared expert above 8 rows: every routing wave publishes its rows'
    # picks and every CU reads them before any streaming (nothing to stream
    # meanwhile); 40 rows: the whole-workgroup grouping and claimed down jobs
    ("no_shared_t12", dict(n_shared=0, hidden=512, inter=256, n_experts=12, top_k=3), 12, 26, "iid"),
    ("no_shared_t40", dict(n_shared=0, hidden=512, inter=256, n_experts=24, top_k=4), 40, 27, "corr"),
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
    ("mxfp4_t3", dict(hidden=2048, inter=1536, shared_inter=512, n_experts=16, top_k=6,
                      routed_fmt=1, bias_bf16=1), 3, 22, "corr"),
    ("mxfp4_t6", dict(hidden=2048, inter=1536, shared_inter=512, n_experts=16, top_k=6,
                      routed_fmt=1, bias_bf16=1), 6, 23, "corr"),
    # MXFP4 above 16 rows: two-tile up/gate items with down units claimed whole
    ("mxfp4_t37", dict(hidden=2048, inter=1536, shared_inter=512, n_experts=16, top_k=6,
                       routed_fmt=1, bias_bf16=1), 37, 28, "iid"),
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
    ("v3_t8", list(range(8))),
    ("v3_t64", list(range(64))),
    ("v4_t16", list(range(16))),
    # the 8-way tensor-parallel share of the V3 layer (intermediate 256)
    ("v3tp8_t1", [0]),
    ("v3tp8_t8", list(range(8))),
    ("v3tp4_t1", [0]),
    ("v3tp4_t8", list(range(8))),
    # the 8-way expert-parallel share (experts 0..31 and the shared expert)
    ("v3ep8_t8", list(range(8))),
    ("v3ep8_t64", list(range(64))),
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
def test_full_size_every_row(full_cases, name, rows):
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
    # every row on its own, too
    for r in rows:
        rel_r, mx_r = parity(out, o64, [r])
        assert rel_r <= REL_L2 and mx_r <= MAX_ABS, (r, rel_r, mx_r)
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


# The DeepSeek-V3 routing geometry (256 experts in 8 groups of 32, keep 4,
# top-8) on a small layer, at batch sizes the wide stream serves (its
# routing is its own code: many rows per wave, read after a flag barrier):
# routing and every row's output against the oracle for the whole batch.
V3R = dict(hidden=1024, inter=256, shared_inter=256, n_experts=256, top_k=8, n_group=8, topk_group=4)


@pytest.mark.parametrize("T,seed,rows", [(17, 61, "iid"), (37, 62, "corr"), (64, 63, "iid")])
def test_v3_routing_wide_whole_batch(T, seed, rows):
    say(f"v3 routing wide T={T}")
    spec = _spec(V3R)
    case = gpu_case(spec, T, seed, rows=rows, requests=max(1, T // 4))
    layer = moe.Layer(spec, case, max_rows=T)
    ids_o, w_o, ge, gg = oracle_route(spec, case)
    assert np.min(ge) > 1e-9 and np.min(gg) > 1e-9
    ids, wts = layer.route(case["x"])
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.allclose(wts.cpu().numpy(), w_o, rtol=1e-6, atol=0)
    out = run_forward(layer, case["x"])
    o64, _ = oracle_rows(spec, case, range(T), ids=ids_o)
    rel, mx = parity(out, o64, list(range(T)))
    say(f"  rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


# The residual is added before the single rounding: with the residual set to
# minus moe_forward's own bf16 output, the kernel's fp32 chain plus the
# residual is the chain's rounding error, whose bf16 value is nonzero almost
# everywhere and at most half a bf16 ulp of the output; a kernel that rounded
# the layer to bf16 before adding would return exactly zero.
@pytest.mark.parametrize("name,over,T,seed,rows", RESID, ids=[s[0] for s in RESID])
def test_residual_single_rounding_bits(name, over, T, seed, rows):
    say(f"residual rounding {name} T={T}")
    spec = _spec(over)
    case = gpu_case(spec, T, seed, rows=rows, requests=max(1, T // 4))
    layer = moe.Layer(spec, case, max_rows=T)
    plain = run_forward(layer, case["x"])
    neg = torch.from_numpy((plain ^ np.uint16(0x8000)).view(np.int16)).view(torch.bfloat16).cuda()
    got = fixtures.bits16(layer.forward(case["x"], residual=neg))
    torch.cuda.synchronize()
    assert layer.read_error() == 0
    nz = (got & np.uint16(0x7FFF)) != 0
    say(f"  nonzero {nz.mean():.4f}")
    assert nz.mean() > 0.9
    p = np.abs(bf16_to_f64(plain))
    r = np.abs(bf16_to_f64(got))
    ulp = np.where(p > 0, np.exp2(np.floor(np.log2(np.where(p > 0, p, 1.0))) - 7), 2.0 ** -133)
    assert np.all(r <= ulp / 2)


# The unfused four-launch layout (routed MoE, shared gate/up, shared down,
# add) of the same layer: within the tolerance of the oracle, and within one
# bf16 rounding of the fused output (its routed and shared sums are rounded
# to bf16 before the add).
UNFUSED = [
    ("tiny_t1", dict(), 1, 81, "iid"),
    ("v3r_t8", V3R, 8, 82, "corr"),
    ("multichunk_ragged_t9", dict(hidden=1152, inter=640, shared_inter=384, n_experts=24, top_k=5), 9, 83, "corr"),
    ("v3r_t37", V3R, 37, 84, "iid"),
    ("mxfp4_t16", dict(hidden=2048, inter=1536, shared_inter=512, n_experts=16, top_k=6, routed_fmt=1, bias_bf16=1),
     16, 85, "corr"),
    # above 16 rows: the shared-expert launches are FP8 instances with FP8
    # tiles while the routed pass has two-tile MXFP4 items
    ("mxfp4_t24", dict(hidden=2048, inter=1536, shared_inter=512, n_experts=16, top_k=6, routed_fmt=1, bias_bf16=1),
     24, 86, "iid"),
]


@pytest.mark.parametrize("name,over,T,seed,rows", UNFUSED, ids=[u[0] for u in UNFUSED])
def test_unfused_layout(name, over, T, seed, rows):
    say(f"unfused {name} T={T}")
    spec = _spec(over)
    case = gpu_case(spec, T, seed, rows=rows, requests=max(1, T // 4))
    layer = moe.Layer(spec, case, max_rows=T)
    fused = run_forward(layer, case["x"])
    out = torch.empty_like(case["x"])
    t_r, t_s = torch.empty_like(out), torch.empty_like(out)
    moe.moe_forward_unfused(layer.cfg, layer.w, case["x"], out, t_r, t_s, layer.ws)
    torch.cuda.synchronize()
    assert layer.read_error() == 0
    got = fixtures.bits16(out)
    o64, _ = oracle_rows(spec, case, range(T))
    rel, mx = parity(got, o64, list(range(T)))
    say(f"  rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS
    # the two paths differ only by the roundings of the two partial sums
    f, u = bf16_to_f64(fused), bf16_to_f64(got)
    assert np.max(np.abs(f - u)) <= 4 * 2.0 ** -8 * max(1.0, np.max(np.abs(f)))
    # the routed part alone is the fused pass of the layer without a shared expert
    spec_r = dict(spec, n_shared=0)
    layer_r = moe.Layer(spec_r, case, max_rows=T)
    assert np.array_equal(fixtures.bits16(t_r), run_forward(layer_r, case["x"]))


# One device's share under expert parallelism (the config's expert range):
# every row routed over all experts, the output summing only the held
# experts' terms, plus the shared expert's on the one device that holds it.
# Each shard against the oracle's reading, rows with neither a held pick nor
# the shared expert exactly zero, the grouping equal to the oracle's with
# the other experts' groups taken out, and the shards' outputs adding up to
# the whole layer's.
EP = [
    ("tiny_4x4", dict(), 4, 6, 91, "corr"),
    ("v3r_8x32_t8", V3R, 8, 8, 92, "iid"),
    ("v3r_8x32_t40", V3R, 8, 40, 93, "corr"),
    ("mxfp4_2x8_t12", dict(hidden=2048, inter=512, shared_inter=256, n_experts=16, top_k=6,
                           routed_fmt=1, bias_bf16=1), 2, 12, 94, "corr"),
]


def _shard(spec, case, s, n):
    per = spec["n_experts"] // n
    sp = dict(spec, expert_first=s * per, expert_count=per, n_shared=spec["n_shared"] if s == 0 else 0)
    sub = dict(case)
    for k in ("w_gate_up", "s_gate_up", "w_down", "s_down"):
        sub[k] = case[k][s * per:(s + 1) * per].clone()
    if s:
        for k in ("sh_w_gate_up", "sh_s_gate_up", "sh_w_down", "sh_s_down"):
            sub.pop(k, None)
    return sp, sub


@pytest.mark.parametrize("name,over,n,T,seed,rows", EP, ids=[e[0] for e in EP])
def test_expert_shards(name, over, n, T, seed, rows):
    import oracle
    say(f"expert shards {name} n={n} T={T}")
    spec = _spec(over)
    case = gpu_case(spec, T, seed, rows=rows, requests=max(1, T // 4))
    H = spec["hidden"]
    full = bf16_to_f64(run_forward(moe.Layer(spec, case, max_rows=T), case["x"]))
    ids_o, _, _, _ = oracle_route(spec, case)
    ge_o, gn_o, gs_o, cols_o, _ = oracle.groups(spec, ids_o)
    total = np.zeros((T, H))
    for s in range(n):
        sp, sub = _shard(spec, case, s, n)
        f, c = fixtures.held(sp)
        layer = moe.Layer(sp, sub, max_rows=T)
        ids, _ = layer.route(case["x"])
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ids_o)
        out = run_forward(layer, case["x"])
        live = [r for r in range(T) if sp["n_shared"] or any(f <= e < f + c for e in ids_o[r])]
        dead = [r for r in range(T) if r not in live]
        assert not np.any(out[dead]), (s, dead)
        if live:
            o64, _ = oracle_rows(sp, sub, live, ids=ids_o)
            rel, mx = parity(out, o64, live)
            say(f"  shard {s}: {len(live)} live rows rel_l2={rel:.3e} max_abs={mx:.3e}")
            assert rel <= REL_L2 and mx <= MAX_ABS, (s, rel, mx)
        # grouping: the oracle's groups of held experts (and the shared one),
        # columns renumbered in the same order
        keep = [g for g in range(len(ge_o)) if ge_o[g] < 0 and sp["n_shared"] or f <= ge_o[g] < f + c]
        ge, gn, gs, cols = layer.groups(case["x"])
        assert ge == [int(ge_o[g]) for g in keep]
        assert gn == [int(gn_o[g]) for g in keep]
        assert gs == [sum(gn[:g]) for g in range(len(gn))]
        assert cols == [int(v) for g in keep for v in cols_o[gs_o[g]:gs_o[g] + gn_o[g]]]
        total += bf16_to_f64(out)
    rel = float(np.linalg.norm(total - full) / np.linalg.norm(full))
    say(f"  shards sum vs layer rel_l2={rel:.3e}")
    assert rel <= REL_L2 and float(np.max(np.abs(total - full))) <= MAX_ABS
