"""Seeded synthetic inputs for the decode MoE layer.

This module only draws random numbers and stores them in the layer's input
formats; it holds none of the layer's arithmetic (no routing, no expert
math, no decoding).  It is the one module that both the HIP path's tests and
the oracle's tests use.

Recipe (the pages publish no tensors, so every input is synthetic):
  * router weights Wr ~ N(0, 1/H) rounded to bf16, so that a logit of an
    N(0,1) activation row is ~N(0,1);
  * correction bias ~ U(-0.1, 0.1), fp32 (or rounded to bf16 for the
    DeepSeek-V4-style layer, whose bias is bf16);
  * activations bf16: "iid" rows ~ N(0,1); "corr" rows are grouped in
    requests, row = base_request + 0.3 * noise with base and noise ~ N(0,1),
    which makes rows of one request share most of their picks (MTP-style
    verify rows; row r belongs to request r // ceil(T / requests));
  * expert weights ~ N(0, 0.02) in fp32, then quantised:
      FP8 E4M3FN with one fp32 scale per 128x128 block, s = amax/448,
      q = RNE(w/s) (torch's cast) after clamping to +-448;
      MXFP4: per 32 consecutive k, X = floor(log2(amax)) - 2, scale byte
      X + 127, element = E2M1 round-to-nearest-even of w / 2^X, saturating
      at +-6, two elements a byte with the even k in the low nibble.
    The shared expert is always FP8.
Draw order is fixed: router weights, bias, activations, shared expert, then
routed experts 0..E-1 (gate/up then down).
"""
from __future__ import annotations

import math

import numpy as np
import torch

FMT_FP8_B128 = 0
FMT_MXFP4 = 1

# Layer shapes.  DeepSeek-V3: hidden 7168, expert intermediate 2048, 256
# routed experts, top-8 in 8 groups keeping 4, one shared expert, scale 2.5.
# The V4-style layer routes top-6 without groups, MXFP4 routed experts and a
# bf16 bias.  "tiny" is the small case used for fast checks.
SPECS = {
    "tiny": dict(hidden=256, inter=128, shared_inter=128, n_experts=16, top_k=4,
                 n_group=1, topk_group=1, n_shared=1, routed_scale=2.5,
                 routed_fmt=FMT_FP8_B128, bias_bf16=0),
    "v3": dict(hidden=7168, inter=2048, shared_inter=2048, n_experts=256, top_k=8,
               n_group=8, topk_group=4, n_shared=1, routed_scale=2.5,
               routed_fmt=FMT_FP8_B128, bias_bf16=0),
    "v4": dict(hidden=7168, inter=2048, shared_inter=2048, n_experts=256, top_k=6,
               n_group=1, topk_group=1, n_shared=1, routed_scale=2.5,
               routed_fmt=FMT_MXFP4, bias_bf16=1),
    # one GPU's share of the V3 layer under 8-way tensor parallelism: the
    # intermediate dimension split 8 ways (2048 / 8), the router whole
    "v3tp8": dict(hidden=7168, inter=256, shared_inter=256, n_experts=256, top_k=8,
                  n_group=8, topk_group=4, n_shared=1, routed_scale=2.5,
                  routed_fmt=FMT_FP8_B128, bias_bf16=0),
    # ... and under 4-way tensor parallelism (2048 / 4)
    "v3tp4": dict(hidden=7168, inter=512, shared_inter=512, n_experts=256, top_k=8,
                  n_group=8, topk_group=4, n_shared=1, routed_scale=2.5,
                  routed_fmt=FMT_FP8_B128, bias_bf16=0),
    # one GPU's share of the V3 layer under 8-way expert parallelism: routed
    # experts 0..31 (the first routing group) and the shared expert; every
    # row is routed over all 256 experts
    "v3ep8": dict(hidden=7168, inter=2048, shared_inter=2048, n_experts=256, top_k=8,
                  n_group=8, topk_group=4, n_shared=1, routed_scale=2.5,
                  routed_fmt=FMT_FP8_B128, bias_bf16=0, expert_first=0, expert_count=32),
}

# The workloads: (spec, rows, row recipe, seed, requests).
WORKLOADS = {
    "tiny_t1": ("tiny", 1, "iid", 1, 1),
    "v3_t1": ("v3", 1, "iid", 2, 1),
    "v3_t8": ("v3", 8, "corr", 3, 2),
    "v3_t64": ("v3", 64, "iid", 4, 64),
    "v4_t16": ("v4", 16, "corr", 5, 4),
    "v3tp8_t1": ("v3tp8", 1, "iid", 6, 1),
    "v3tp8_t8": ("v3tp8", 8, "corr", 7, 2),
    "v3tp4_t1": ("v3tp4", 1, "iid", 10, 1),
    "v3tp4_t8": ("v3tp4", 8, "corr", 11, 2),
    # 8 and 64 rows (8 data-parallel ranks of 8 rows each) at one
    # expert-parallel device
    "v3ep8_t8": ("v3ep8", 8, "corr", 8, 2),
    "v3ep8_t64": ("v3ep8", 64, "iid", 9, 64),
}


def spec_with(name: str, **over) -> dict:
    s = dict(SPECS[name])
    s.update(over)
    return s


def held(spec: dict) -> tuple[int, int]:
    """(first, count) of the routed experts a device holds: the spec's
    expert range, or all E experts."""
    c = int(spec.get("expert_count", 0))
    return (int(spec.get("expert_first", 0)), c) if c else (0, int(spec["n_experts"]))


def held_distinct(spec: dict, ids) -> int:
    """Distinct held experts among the picks `ids` (any iterable of ints)."""
    f, c = held(spec)
    return len(set(int(e) for e in ids if f <= int(e) < f + c))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def quant_fp8_b128(w: torch.Tensor):
    """w [..., N, K] fp32 -> (q [..., N, K] uint8 E4M3FN codes, s [..., N/128, K/128] fp32)."""
    *lead, N, K = w.shape
    blk = w.reshape(*lead, N // 128, 128, K // 128, 128)
    amax = blk.abs().amax(dim=(-3, -1))
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / s[..., :, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.reshape(*lead, N, K).view(torch.uint8), s.to(torch.float32)


def _e2m1_code(mag: torch.Tensor) -> torch.Tensor:
    # grid 0, .5, 1, 1.5, 2, 3, 4, 6 has codes 0..7; midpoints resolved to the
    # even code (round to nearest, ties to even), values above 6 saturate.
    idx = ((mag > 0.25).to(torch.uint8) + (mag >= 0.75).to(torch.uint8)
           + (mag > 1.25).to(torch.uint8) + (mag >= 1.75).to(torch.uint8)
           + (mag > 2.5).to(torch.uint8) + (mag >= 3.5).to(torch.uint8)
           + (mag > 5.0).to(torch.uint8))
    return idx


def quant_mxfp4(w: torch.Tensor):
    """w [..., N, K] fp32 -> (q [..., N, K/2] uint8, s [..., N, K/32] uint8 E8M0)."""
    *lead, N, K = w.shape
    blk = w.reshape(*lead, N, K // 32, 32)
    amax = blk.abs().amax(dim=-1)
    X = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2
    X = X.clamp(-127, 127)
    scaled = blk / torch.pow(2.0, X)[..., None]
    code = _e2m1_code(scaled.abs()) | ((scaled < 0).to(torch.uint8) << 3)
    code = code.reshape(*lead, N, K // 2, 2)
    q = code[..., 0] | (code[..., 1] << 4)
    s = (X + 127).to(torch.uint8)
    return q.contiguous(), s.contiguous()


def _quant(w, fmt):
    return quant_fp8_b128(w) if fmt == FMT_FP8_B128 else quant_mxfp4(w)


def make_case(spec: dict, T: int, seed: int, device="cpu", rows: str = "iid",
              requests: int = 1, experts: bool = True) -> dict:
    """Draws one seeded case.  Returns torch tensors on `device`:
    x [T,H] bf16, router_w [E,H] bf16, bias [E] fp32|bf16,
    w_gate_up [E,2I,H] u8 (or [E,2I,H/2] for MXFP4), s_gate_up,
    w_down [E,H,I] u8 (or [E,H,I/2]), s_down, and the shared expert's
    sh_w_gate_up [2I_s,H] u8, sh_s_gate_up, sh_w_down [H,I_s] u8, sh_s_down.
    experts=False stops after the router weights, bias and activations.
    With an expert range in the spec (expert_first, expert_count) the routed
    tensors hold those experts only (same draws as the whole layer's)."""
    H, I, Is, E = spec["hidden"], spec["inter"], spec["shared_inter"], spec["n_experts"]
    fmt = spec["routed_fmt"]
    ef, ec = held(spec)
    g = _gen(device, seed)
    dev = torch.device(device)
    rw = (torch.randn(E, H, generator=g, device=dev) / math.sqrt(H)).to(torch.bfloat16)
    bias = (torch.rand(E, generator=g, device=dev) * 0.2 - 0.1)
    bias = bias.to(torch.bfloat16) if spec["bias_bf16"] else bias.to(torch.float32)
    if rows == "iid":
        x = torch.randn(T, H, generator=g, device=dev)
    elif rows == "corr":
        # row r belongs to request r // ceil(T / requests)
        per = -(-T // requests)
        base = torch.randn(requests, H, generator=g, device=dev)
        z = torch.randn(T, H, generator=g, device=dev)
        x = base.repeat_interleave(per, dim=0)[:T] + 0.3 * z
    else:
        raise ValueError(rows)
    x = x.to(torch.bfloat16)
    case = dict(x=x, router_w=rw, bias=bias)
    if not experts:
        return case
    if spec["n_shared"]:
        wsh = torch.randn(2 * Is, H, generator=g, device=dev) * 0.02
        case["sh_w_gate_up"], case["sh_s_gate_up"] = quant_fp8_b128(wsh)
        wsh = torch.randn(H, Is, generator=g, device=dev) * 0.02
        case["sh_w_down"], case["sh_s_down"] = quant_fp8_b128(wsh)
        del wsh
    if fmt == FMT_FP8_B128:
        wgu = torch.empty(ec, 2 * I, H, dtype=torch.uint8, device=dev)
        sgu = torch.empty(ec, 2 * I // 128, H // 128, dtype=torch.float32, device=dev)
        wd = torch.empty(ec, H, I, dtype=torch.uint8, device=dev)
        sd = torch.empty(ec, H // 128, I // 128, dtype=torch.float32, device=dev)
    else:
        wgu = torch.empty(ec, 2 * I, H // 2, dtype=torch.uint8, device=dev)
        sgu = torch.empty(ec, 2 * I, H // 32, dtype=torch.uint8, device=dev)
        wd = torch.empty(ec, H, I // 2, dtype=torch.uint8, device=dev)
        sd = torch.empty(ec, H, I // 32, dtype=torch.uint8, device=dev)
    # experts past the held range need no draws
    for e in range(ef + ec):
        w = torch.randn(2 * I, H, generator=g, device=dev) * 0.02
        if e >= ef:
            wgu[e - ef], sgu[e - ef] = _quant(w, fmt)
        w = torch.randn(H, I, generator=g, device=dev) * 0.02
        if e >= ef:
            wd[e - ef], sd[e - ef] = _quant(w, fmt)
        del w
    case.update(w_gate_up=wgu, s_gate_up=sgu, w_down=wd, s_down=sd)
    return case


def make_workload(name: str, device="cpu", **over) -> tuple[dict, dict]:
    """(spec, case) of one of the named workloads."""
    sname, T, rows, seed, req = WORKLOADS[name]
    spec = spec_with(sname)
    return spec, make_case(spec, T, seed, device=device, rows=rows, requests=req, **over)


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 array of its bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_case(case: dict, experts=None, spec=None) -> dict:
    """Host (numpy) copy for the oracle.  Only experts listed in `experts`
    are copied (others None), so a full-size case needs host memory only for
    the experts a step uses.  With a spec that holds an expert range, the
    lists are indexed by global expert (length E) and only held experts can
    be copied."""
    if spec is not None:
        E = int(spec["n_experts"])
        ef, ec = held(spec)
    else:
        E = case["w_gate_up"].shape[0]
        ef, ec = 0, E
    if experts is None:
        experts = range(ef, ef + ec)
    experts = set(int(e) for e in experts if ef <= int(e) < ef + ec)
    out = dict(x=bits16(case["x"]), router_w=bits16(case["router_w"]))
    b = case["bias"]
    out["bias"] = bits16(b) if b.dtype == torch.bfloat16 else b.cpu().numpy()
    for k in ("sh_w_gate_up", "sh_s_gate_up", "sh_w_down", "sh_s_down"):
        if k in case:
            out[k] = case[k].cpu().numpy()
    for k in ("w_gate_up", "s_gate_up", "w_down", "s_down"):
        out[k] = [case[k][e - ef].cpu().numpy() if e in experts else None for e in range(E)]
    return out


def weight_bytes(spec: dict) -> dict:
    """Bytes of each weight tensor the layer reads (values + scales)."""
    H, I, Is, E = spec["hidden"], spec["inter"], spec["shared_inter"], spec["n_experts"]
    if spec["routed_fmt"] == FMT_FP8_B128:
        routed = 3 * I * H + 4 * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128))
    else:
        routed = 3 * I * H // 2 + (2 * I * (H // 32) + H * (I // 32))
    shared = (3 * Is * H + 4 * ((2 * Is // 128) * (H // 128) + (H // 128) * (Is // 128))) if spec["n_shared"] else 0
    router = 2 * E * H + (2 if spec["bias_bf16"] else 4) * E
    return dict(routed_expert=routed, shared_expert=shared, router=router)


def algorithmic_bytes(spec: dict, distinct: int) -> int:
    """Bytes the layer must move for one call: every used expert's weights and
    scales once (the shared expert and `distinct` routed experts) plus the
    router weights and bias.  Activations, mid values and outputs (<0.1%)
    are not counted."""
    b = weight_bytes(spec)
    return b["shared_expert"] + distinct * b["routed_expert"] + b["router"]
