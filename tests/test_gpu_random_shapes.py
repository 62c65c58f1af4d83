"""GPU parity on seeded random shapes, through the C ABI.

The shapes are drawn once from a fixed seed within the library's limits
(hidden and intermediate multiples of 64, E + S <= 512, top_k <= E), with
both operand types and with and without a padding mask, so the launch
configurations (tile counts, ragged tails, schedules below and above one
round of tiles) vary from case to case.  Each case is compared element by
element with the fp64 oracle under the same bars as the other parity tests.
One more case gives experts thousands of rows (16 row tiles each), so that
the row tiles sharing a weight tile outnumber a start group, and one has
start groups larger than the workgroups of an XCD.  The backward, and the
training forward with the backward from its saved projections, are checked
on the same shapes.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_feed_amd import binding as B
from mixture_experts_feed_amd import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _draw_cases(n=10, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = {}
    for c in range(n):
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        S = int(rng.integers(0, 4))
        kw = dict(T=int(rng.integers(1, 3001)), hidden=64 * int(rng.integers(1, 6)), n_routed=E, top_k=k,
                  n_shared=S, intermediate=64 * int(rng.integers(1, 4)),
                  dtype="f32" if rng.random() < 0.3 else "bf16",
                  route_scale=float(rng.choice([1.0, 2.5, 8.0])),
                  gate_dist=("uniform", 0.05), bias_dist=("uniform", 0.05))
        mask_frac = float(rng.choice([0.0, 0.0, 0.2]))
        name = (f"r{c}_T{kw['T']}_H{kw['hidden']}_E{E}_k{k}_S{S}_I{kw['intermediate']}_{kw['dtype']}"
                f"{'_pad' if mask_frac else ''}")
        cases[name] = (wl.custom(name=name, **kw), mask_frac)
    # experts of 4096 rows: 16 row tiles per weight tile
    w = wl.custom(name="big_experts", T=4096, hidden=128, n_routed=4, top_k=4, n_shared=1, intermediate=64)
    cases["big_experts_T4096_E4_k4"] = (w, 0.0)
    # nine tiles in all, two workgroups per XCD, start groups of eight row tiles
    w = wl.custom(name="few_workgroups", T=2048, hidden=64, n_routed=1, top_k=1, n_shared=1, intermediate=64)
    cases["few_workgroups_T2048_E1"] = (w, 0.0)
    return cases


CASES = _draw_cases()


def _draw_wide_cases(n=14, seed=202):
    """Wider ranges than _draw_cases: E up to 256 (past one wave of experts per
    lane), k up to 12, S up to 4, hidden up to 1024, intermediate up to 512,
    token counts at and around the tile and word boundaries (1, 7, 63-65, 255,
    257, 2047, 2049, 4100), masks that pad some or every token."""
    rng = np.random.default_rng(seed)
    cases = {}
    for c in range(n):
        E = int(rng.choice([1, 3, 8, 17, 64, 130, 256]))
        k = int(rng.integers(1, min(E, 12) + 1))
        S = int(rng.integers(0, 5))
        kw = dict(T=int(rng.choice([1, 7, 63, 64, 65, 255, 257, 1000, 2047, 2049, 4100])),
                  hidden=64 * int(rng.integers(1, 17)), n_routed=E, top_k=k, n_shared=S,
                  intermediate=64 * int(rng.integers(1, 9)),
                  dtype="f32" if rng.random() < 0.25 else "bf16",
                  route_scale=float(rng.choice([1.0, 2.5, 8.0])),
                  gate_dist=("uniform", 0.05), bias_dist=("uniform", 0.05))
        mask_frac = float(rng.choice([0.0, 0.0, 0.3, 1.0]))
        name = (f"w{c}_T{kw['T']}_H{kw['hidden']}_E{E}_k{k}_S{S}_I{kw['intermediate']}_{kw['dtype']}"
                f"{'_pad' if mask_frac else ''}")
        cases[name] = (wl.custom(name=name, **kw), mask_frac)
    return cases


WIDE = _draw_wide_cases()


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_random_shape(name):
    w, mask_frac = CASES[name]
    _say(f"[random] {name}")
    inp = wl.make_inputs(w, device=DEV)
    mask = None
    if mask_frac > 0:
        g = torch.Generator().manual_seed(w.T)
        mask = (torch.rand((w.T,), generator=g) < mask_frac).to(torch.uint8).to(DEV)
    S = w.n_shared
    out, routing = B.forward(inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"],
                             inp["wsh_gu"] if S else None, inp["wsh_d"] if S else None, w.top_k,
                             inp["route_scale"], inp["global_scale"], padding_mask=mask,
                             return_routing=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = P.oracle_route(inp, w.top_k, mask)
    band = P.check_routing(routing, ref, w.top_k)
    pm = None if mask is None else mask.cpu().numpy().astype(bool)
    o_ref, _ = oracle.moe_forward(P.host(inp["x"]), P.host(inp["gate_bank"]), P.host(inp["bias"]),
                                  P.HostExperts(inp["w_gu"]), P.HostExperts(inp["w_d"]),
                                  P.HostExperts(inp["wsh_gu"] if S else None),
                                  P.HostExperts(inp["wsh_d"] if S else None),
                                  w.top_k, w.route_scale, w.global_scale, padding_mask=pm, routing=ref)
    rel = P.check_output(out, o_ref, w.dtype)
    _say(f"[random] ok: band={band} max_err/rms={rel:.2e}")


@pytest.mark.parametrize("name", list(CASES))
def test_random_shape_backward(name):
    """The backward on the same shapes: dx, the gate-bank gradient and every
    weight gradient against the oracle's, under the backward's bars."""
    from tests.test_gpu_backward import _full_backward
    w, mask_frac = CASES[name]
    _say(f"[random backward] {name}")
    mask = None
    if mask_frac > 0:
        g = torch.Generator().manual_seed(w.T)
        mask = (torch.rand((w.T,), generator=g) < mask_frac).to(torch.uint8).to(DEV)
    _full_backward(w, padding_mask=mask)


@pytest.mark.parametrize("name", list(CASES))
def test_random_shape_saved_backward(name):
    """The training forward and the backward from its saved projections on the
    same shapes: output and every gradient bit-identical to the forward's and
    the recomputing backward's."""
    from tests.test_gpu_backward import saved_vs_recompute
    w, mask_frac = CASES[name]
    mask = None
    if mask_frac > 0:
        g = torch.Generator().manual_seed(w.T)
        mask = (torch.rand((w.T,), generator=g) < mask_frac).to(torch.uint8).to(DEV)
    saved_vs_recompute(name, w, mask)


@pytest.mark.parametrize("name", list(WIDE))
def test_wide_random_shape(name):
    """Forward parity on the wider draw; the backward too where the oracle's
    backward stays quick (T <= 2100, hidden <= 512)."""
    w, mask_frac = WIDE[name]
    _say(f"[wide] {name}")
    inp = wl.make_inputs(w, device=DEV)
    mask = None
    if mask_frac > 0:
        g = torch.Generator().manual_seed(w.T + 1)
        mask = (torch.rand((w.T,), generator=g) < mask_frac).to(torch.uint8).to(DEV)
    S = w.n_shared
    out, routing = B.forward(inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"],
                             inp["wsh_gu"] if S else None, inp["wsh_d"] if S else None, w.top_k,
                             inp["route_scale"], inp["global_scale"], padding_mask=mask,
                             return_routing=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = P.oracle_route(inp, w.top_k, mask)
    band = P.check_routing(routing, ref, w.top_k)
    pm = None if mask is None else mask.cpu().numpy().astype(bool)
    o_ref, _ = oracle.moe_forward(P.host(inp["x"]), P.host(inp["gate_bank"]), P.host(inp["bias"]),
                                  P.HostExperts(inp["w_gu"]), P.HostExperts(inp["w_d"]),
                                  P.HostExperts(inp["wsh_gu"] if S else None),
                                  P.HostExperts(inp["wsh_d"] if S else None),
                                  w.top_k, w.route_scale, w.global_scale, padding_mask=pm, routing=ref)
    rel = P.check_output(out, o_ref, w.dtype)
    _say(f"[wide] forward ok: band={band} max_err/rms={rel:.2e}")
    if w.T <= 2100 and w.hidden <= 512:
        from tests.test_gpu_backward import _full_backward
        _full_backward(w, padding_mask=mask)
