"""Bitwise properties of the GPU path that need no oracle: a row's output is
identical alone or inside any batch (batch invariance), repeated calls are
identical (determinism), unused experts are never read (poisoned with NaN
codes, the output does not change), exact routing ties resolve by index,
and a non-finite activation raises the device error word."""
import numpy as np
import pytest
import torch

import fixtures
import mixture_experts_decode_sigmoid_amd as moe
from _gpu import gpu_case, oracle_route, run_forward, say

pytestmark = pytest.mark.gpu

MID = dict(hidden=2048, inter=512, shared_inter=512, n_experts=64, top_k=6, n_group=8, topk_group=3)
# hidden > 16 * 256: two 16-row down tiles per CU, split over the waves
MID2 = dict(hidden=4352, inter=256, shared_inter=256, n_experts=32, top_k=4, n_group=4, topk_group=2)
# MXFP4 routed experts: from 5 rows up the up/gate items are two 16-row tiles
# on one activation operand, up to 4 rows one tile; the bits must not change
MID3 = dict(hidden=2048, inter=512, shared_inter=512, n_experts=48, top_k=6, routed_fmt=1, bias_bf16=1)


# DeepSeek-V3 routing geometry (256 experts in 8 groups of 32, keep 4,
# top-8) on a small layer.
V3R = dict(hidden=1024, inter=256, shared_inter=256, n_experts=256, top_k=8, n_group=8, topk_group=4)


def _layer(spec, case, T):
    return moe.Layer(spec, case, max_rows=T)


@pytest.mark.parametrize("mid,T", [(1, 1), (1, 2), (1, 5), (1, 8), (1, 16), (1, 37), (1, 64),
                                   (2, 1), (2, 9), (2, 16), (2, 17),
                                   (3, 4), (3, 5), (3, 16), (3, 17), (3, 64)])
def test_batch_invariance_mid(mid, T):
    say(f"batch invariance mid{mid} T={T}")
    spec = fixtures.spec_with("tiny", **{1: MID, 2: MID2, 3: MID3}[mid])
    case = gpu_case(spec, 64, 21, rows="corr", requests=16)
    layer = _layer(spec, case, 64)
    full = run_forward(layer, case["x"])
    g = torch.Generator().manual_seed(T)
    perm = torch.randperm(64, generator=g)[:T]
    sub = run_forward(layer, case["x"][perm.cuda()].contiguous())
    assert np.array_equal(sub, full[perm.numpy()])
    for r in perm[:3].tolist():
        one = run_forward(layer, case["x"][r:r + 1].contiguous())
        assert np.array_equal(one[0], full[r])


def test_batch_invariance_v3_t8():
    say("batch invariance v3 t8")
    spec, case = fixtures.make_workload("v3_t8", device="cuda")
    layer = _layer(spec, case, 8)
    full = run_forward(layer, case["x"])
    for r in range(8):
        one = run_forward(layer, case["x"][r:r + 1].contiguous())
        assert np.array_equal(one[0], full[r]), r
    rev = run_forward(layer, case["x"].flip(0).contiguous())
    assert np.array_equal(rev, full[::-1])


@pytest.mark.parametrize("name", ["v3_t64", "v4_t16"])
def test_batch_invariance_full_size(name):
    """Every row of the 64-row DeepSeek-V3 batch (wide stream) and of the
    16-row MXFP4 top-6 batch (narrow stream) alone, through the one-row
    kernel, equals its row in the batch bit for bit; so does the batch in
    reverse order."""
    say(f"batch invariance {name}")
    spec, case = fixtures.make_workload(name, device="cuda")
    T = case["x"].shape[0]
    layer = _layer(spec, case, T)
    full = run_forward(layer, case["x"])
    for r in range(T):
        one = run_forward(layer, case["x"][r:r + 1].contiguous())
        assert np.array_equal(one[0], full[r]), r
    rev = run_forward(layer, case["x"].flip(0).contiguous())
    assert np.array_equal(rev, full[::-1])
    del layer, case
    torch.cuda.empty_cache()


def _score_slots(layer, T, E):
    """The fp64 scores of the last call, as left in its workspace's tagged
    slots (two 64-bit words each: tag and high half, tag and low half; a
    row's slots in the kernel's own order), one row of slots per row."""
    torch.cuda.synchronize()
    off = 4096 + 256  # after the per-CU flags and the error word
    n = 4 * ((E + 3) // 4)
    w = layer.ws[off:off + 16 * T * n].cpu().numpy().view(np.uint64).reshape(T, n, 2)
    return ((w[..., 0] & np.uint64(0xFFFFFFFF)) << np.uint64(32)) | (w[..., 1] & np.uint64(0xFFFFFFFF))


def test_router_logits_same_bits_at_every_batch_size():
    """Activations spread over five decades make the fp64 logit sums inexact,
    so their bits depend on the summation order: a row's scores must still
    be the same bits whether it is routed alone or in a batch of 8 or 37
    rows (the logit kernels differ by batch size), in moe_route and in
    moe_forward."""
    say("router logits order")
    spec = fixtures.spec_with("tiny", **V3R)
    T, E = 37, spec["n_experts"]
    g = torch.Generator().manual_seed(77)
    mag = torch.pow(10.0, torch.rand(T, spec["hidden"], generator=g) * 5 - 4)
    sign = torch.where(torch.rand(T, spec["hidden"], generator=g) < 0.5, -1.0, 1.0)
    case = gpu_case(spec, T, 78)
    case["x"] = (mag * sign).bfloat16().cuda()
    layer = _layer(spec, case, T)
    ref = {}
    for call in ("route", "forward"):
        for n in (37, 8, 1):
            x = case["x"][:n].contiguous()
            if call == "route":
                layer.route(x)
            else:
                run_forward(layer, x)
            s = _score_slots(layer, n, E)
            for r in range(n):
                if r in ref:
                    assert np.array_equal(s[r], ref[r]), (call, n, r)
                else:
                    ref[r] = s[r]
    # the slots hold probabilities: the reading of the layout is right
    sv = ref[0].view(np.float64)
    assert np.all((sv > 0) & (sv < 1))


def test_determinism_and_negative_control():
    say("determinism")
    spec = fixtures.spec_with("tiny", **MID)
    case = gpu_case(spec, 16, 22, rows="corr", requests=4)
    layer = _layer(spec, case, 16)
    ref = run_forward(layer, case["x"])
    for _ in range(20):
        assert np.array_equal(run_forward(layer, case["x"]), ref)
    x2 = case["x"].clone()
    x2[3, 100] = -x2[3, 100]
    alt = run_forward(layer, x2)
    assert not np.array_equal(alt[3], ref[3])
    assert np.array_equal(np.delete(alt, 3, 0), np.delete(ref, 3, 0))


@pytest.mark.parametrize("fmt", [0, 1])
def test_poisoned_unused_experts(fmt):
    say(f"poison unused fmt={fmt}")
    over = dict(MID)
    if fmt:
        over.update(routed_fmt=1, bias_bf16=1, n_group=1, topk_group=1)
    spec = fixtures.spec_with("tiny", **over)
    case = gpu_case(spec, 8, 23, rows="corr", requests=2)
    layer = _layer(spec, case, 8)
    ref = run_forward(layer, case["x"])
    ids, _, _, _ = oracle_route(spec, case)
    unused = sorted(set(range(spec["n_experts"])) - set(ids.ravel().tolist()))
    assert unused
    for e in unused:
        if fmt == 0:
            case["w_gate_up"][e].fill_(0x7F)   # E4M3 NaN
            case["w_down"][e].fill_(0x7F)
        else:
            case["s_gate_up"][e].fill_(0xFF)   # E8M0 NaN
            case["s_down"][e].fill_(0xFF)
    # a layer built on the poisoned weights (MXFP4 scales are packed when a
    # layer is built)
    layer2 = _layer(spec, case, 8)
    out = run_forward(layer2, case["x"])
    assert np.array_equal(out, ref)
    assert layer2.read_error() == 0


def test_routing_exact_ties():
    say("routing ties")
    spec = fixtures.spec_with("tiny", **MID)
    case = gpu_case(spec, 6, 24)
    rw, bias = case["router_w"], case["bias"]
    rw[40] = rw[9]
    rw[50] = rw[9]
    bias[9] = bias[40] = bias[50] = 3.0
    layer = _layer(spec, case, 6)
    ids, wts = layer.route(case["x"])
    ids_o, w_o, _, _ = oracle_route(spec, case)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    # ties resolve to the lower index, in order
    for r in range(6):
        row = ids_o[r].tolist()
        assert row.index(9) < row.index(40) < row.index(50)


def test_error_word_on_nan_activation():
    say("error word")
    spec = fixtures.spec_with("tiny")
    case = gpu_case(spec, 2, 25)
    layer = _layer(spec, case, 2)
    x = case["x"].clone()
    x[1, 7] = float("nan")
    run_forward(layer, x, check=False)
    bits = layer.read_error()
    assert bits & (moe.MOE_DEVERR_NONFINITE_SCORE | moe.MOE_DEVERR_NONFINITE_MID)
    assert layer.read_error() == 0          # read clears
    run_forward(layer, case["x"])
    assert layer.read_error() == 0


@pytest.mark.parametrize("fmt,T", [(0, 2), (0, 20), (1, 3), (1, 20)])
def test_error_word_on_nan_weight_code_in_a_used_expert(fmt, T):
    """A NaN weight code (E4M3 0x7F) or a NaN block scale (E8M0 0xFF) in an
    expert a row uses sets MOE_DEVERR_NONFINITE_MID (narrow and wide stream);
    the same bytes in an unused expert set nothing (see the poison test)."""
    say(f"error word used expert fmt={fmt} T={T}")
    over = dict(MID)
    if fmt:
        over.update(routed_fmt=1, bias_bf16=1, n_group=1, topk_group=1)
    spec = fixtures.spec_with("tiny", **over)
    case = gpu_case(spec, T, 27 + T)
    ids, _, _, _ = oracle_route(spec, case)
    e = int(ids[0, 0])
    if fmt == 0:
        case["w_gate_up"][e, 3, 17] = 0x7F      # one weight of one gate row
    else:
        case["s_down"][e, 5, 2] = 0xFF          # one block scale of one down row
    layer = _layer(spec, case, T)               # (MXFP4 scales are packed here)
    run_forward(layer, case["x"], check=False)
    bits = layer.read_error()
    assert bits & moe.MOE_DEVERR_NONFINITE_MID, bits
    assert not bits & moe.MOE_DEVERR_WAIT_TIMEOUT


def test_rows_zero_and_limits():
    spec = fixtures.spec_with("tiny")
    case = gpu_case(spec, 4, 26)
    layer = _layer(spec, case, 4)
    empty = torch.empty(0, spec["hidden"], dtype=torch.bfloat16, device="cuda")
    layer.forward(empty, out=torch.empty_like(empty))
    with pytest.raises(moe.MoeError) as e:
        big = torch.zeros(5, spec["hidden"], dtype=torch.bfloat16, device="cuda")
        layer.forward(big)
    assert e.value.code == moe.MOE_ERR_ROWS
    with pytest.raises(moe.MoeError) as e:
        layer.forward(case["x"], out=case["x"])
    assert e.value.code == moe.MOE_ERR_ALIAS


# The V3 routing geometry: the paths that hold for 32-lane groups and for
# ties at the top-k threshold.


def _route_both(spec, case, T):
    layer = _layer(spec, case, T)
    ids, wts = layer.route(case["x"])
    ids_o, w_o, _, _ = oracle_route(spec, case)
    ids = ids.cpu().numpy()
    assert np.array_equal(ids, ids_o)
    assert np.allclose(wts.cpu().numpy(), w_o, rtol=1e-6, atol=0)
    return ids


@pytest.mark.parametrize("T", [1, 3, 8])
def test_routing_group_tie_at_the_kept_boundary(T):
    """Groups 2 and 5 are copies of each other and tie for the last kept
    group: the lower group (2) is kept, so its experts are picked and group
    5's identical ones are not."""
    say(f"group tie T={T}")
    spec = fixtures.spec_with("tiny", **V3R)
    case = gpu_case(spec, T, 31)
    rw, bias = case["router_w"], case["bias"]
    bias.zero_()
    for g in (0, 1, 3):
        bias[32 * g + 1] = 5.0
        bias[32 * g + 7] = 5.0
    bias[64 + 2] = 3.0
    bias[64 + 9] = 3.0
    rw[160:192] = rw[64:96]
    bias[160:192] = bias[64:96]
    ids = _route_both(spec, case, T)
    for r in range(T):
        row = set(ids[r].tolist())
        assert {66, 73} <= row and not row & set(range(160, 192))


@pytest.mark.parametrize("T", [1, 8])
def test_routing_ties_past_k(T):
    """Ten experts (five in each of groups 0 and 1) share one router row and
    one bias, so the top-k threshold is a ten-way exact tie: the eight lowest
    indices win, in index order."""
    say(f"ties past k T={T}")
    spec = fixtures.spec_with("tiny", **V3R)
    case = gpu_case(spec, T, 32)
    rw, bias = case["router_w"], case["bias"]
    bias.zero_()
    tied = [0, 1, 2, 3, 4, 32, 33, 34, 35, 36]
    for e in tied:
        rw[e] = rw[0]
        bias[e] = 3.0
    ids = _route_both(spec, case, T)
    for r in range(T):
        assert ids[r].tolist() == tied[:8]


@pytest.mark.parametrize("T", [1, 8, 37])
def test_graph_replay_matches_eager(T):
    """moe_forward captured in a HIP graph (the launch-cost removal of the
    upstream-overlap item): every replay, with eager work and eager calls of
    the layer between replays, gives the eager output bit for bit.  The call
    records one kernel launch and no memory set."""
    say(f"graph replay T={T}")
    spec = fixtures.spec_with("tiny", **MID)
    case = gpu_case(spec, T, 50 + T, rows="corr", requests=max(1, T // 4))
    layer = _layer(spec, case, T)
    x = case["x"]
    eager = run_forward(layer, x)
    out = torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, out=out)
    torch.cuda.synchronize()
    for _ in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(fixtures.bits16(out), eager)
        assert np.array_equal(run_forward(layer, x), eager)
    assert layer.read_error() == 0


@pytest.mark.parametrize("T", [1, 8, 37])
def test_forward_after_ready_word(T):
    """moe_forward_after with the ready word raised by a producer earlier on
    the same stream (a copy of x, then a fill of the word) gives moe_forward's
    output bit for bit; so does a counter that wrapped past the value, and a
    residual is added as in moe_forward_residual."""
    say(f"forward after ready word T={T}")
    spec = fixtures.spec_with("tiny", **MID)
    case = gpu_case(spec, T, 70 + T, rows="corr", requests=max(1, T // 4))
    layer = _layer(spec, case, T)
    ref = run_forward(layer, case["x"])
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    x2 = torch.empty_like(case["x"])
    x2.copy_(case["x"])
    word.fill_(5)
    out = torch.empty_like(x2)
    moe.moe_forward_after(layer.cfg, layer.w, x2, out, layer.ws, word, 5)
    torch.cuda.synchronize()
    assert layer.read_error() == 0
    assert np.array_equal(fixtures.bits16(out), ref)
    word.fill_(3)  # 0xFFFFFFF8 + 11 wraps to 3: reached
    out2 = torch.empty_like(x2)
    moe.moe_forward_after(layer.cfg, layer.w, x2, out2, layer.ws, word, 0xFFFFFFF8)
    torch.cuda.synchronize()
    assert layer.read_error() == 0
    assert np.array_equal(fixtures.bits16(out2), ref)
    res = torch.randn(T, spec["hidden"], generator=torch.Generator().manual_seed(T)).bfloat16().cuda()
    want = fixtures.bits16(layer.forward(case["x"], residual=res))
    out3 = torch.empty_like(x2)
    moe.moe_forward_after(layer.cfg, layer.w, x2, out3, layer.ws, word, 3, residual=res)
    torch.cuda.synchronize()
    assert layer.read_error() == 0
    assert np.array_equal(fixtures.bits16(out3), want)


def test_forward_after_word_never_raised():
    """A ready word the host never raises: every CU's bounded wait (64 polls
    here) gives up, the timeout bit is set and the call ends; the next
    ordinary call on a re-initialised workspace is unaffected."""
    say("forward after: word never raised")
    spec = fixtures.spec_with("tiny", **MID)
    case = gpu_case(spec, 4, 79)
    layer = _layer(spec, case, 4)
    ref = run_forward(layer, case["x"])
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(case["x"])
    moe.moe_forward_after(layer.cfg, layer.w, case["x"], out, layer.ws, word, 7, max_polls=64)
    torch.cuda.synchronize()
    assert layer.read_error() & moe.MOE_DEVERR_WAIT_TIMEOUT
    moe.moe_workspace_init(layer.ws)
    assert np.array_equal(run_forward(layer, case["x"]), ref)


def test_prefill_chunks_are_batch_invariant():
    """moe_forward_prefill over 150 rows in chunks of 64 (64, 64, 22): every
    row's output equals a one-row moe_forward call of it, bit for bit, and
    equals the chunks run as separate calls."""
    say("prefill chunks")
    spec = fixtures.spec_with("tiny", **V3R)
    case = gpu_case(spec, 150, 88, rows="corr", requests=30)
    layer = _layer(spec, case, 64)
    x = case["x"]
    out = torch.empty_like(x)
    moe.moe_forward_prefill(layer.cfg, layer.w, x, out, layer.ws)
    torch.cuda.synchronize()
    assert layer.read_error() == 0
    got = fixtures.bits16(out)
    for r0, n in ((0, 64), (64, 64), (128, 22)):
        assert np.array_equal(got[r0:r0 + n], run_forward(layer, x[r0:r0 + n].contiguous()))
    for r in (0, 63, 64, 127, 128, 149):
        assert np.array_equal(got[r], run_forward(layer, x[r:r + 1].contiguous())[0]), r
