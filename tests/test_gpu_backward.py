"""GPU parity of inkling_moe_backward against the fp64 oracle's backward.

Every gradient (dx, gate bank, routed and shared gate_up / down weights) is
compared element by element on small workloads; at hidden=6144 the gradients
of sampled tokens and of sampled experts are compared.

Bars.  fp32 operands: max |gpu - oracle| <= 1e-4 * RMS(oracle) for every
gradient.  bf16 operands: dx and the gate-bank gradient, max |gpu - oracle| <=
2e-2 * RMS (the forward's bar); the weight gradients are sums over rows of
products u_r v_r of which one factor (dh for gate_up, a = gamma * silu(g) * u for
down) is rounded to bf16 to feed the bf16 matrix cores (unit roundoff 2^-8:
8 significand bits), the other an exact bf16 input, with fp32 accumulation; so
each element obeys the componentwise bound |err| <= (2^-8 + K 2^-24) sum_r |u_r v_r|,
at most (2^-8 + 2^-10) sum_r |u_r v_r| for K <= 16384 rows; the oracle returns
those sums.
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
TOL = {"bf16": 2e-2, "f32": 1e-4}
ABS_BOUND = P.WGRAD_ABS_BOUND


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _dout(w, seed=7):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((w.T, w.hidden), generator=g).to(w.torch_dtype).to(DEV)


def _close(name, gpu, ref, dtype, report=None):
    g = gpu.float().cpu().numpy().astype(np.float64) if isinstance(gpu, torch.Tensor) else gpu
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    rel = err / rms if rms > 0 else 0.0
    _say(f"[backward]   {name}: max_err/rms={rel:.2e}")
    assert err <= TOL[dtype] * rms + 1e-30, f"{name}: max abs err {err:.3e} > {TOL[dtype]} * RMS {rms:.3e}"
    return rel


def _close_wgrad(name, gpu, ref, absref, dtype):
    """Weight gradients: the componentwise bound for bf16, the RMS bar for fp32."""
    if dtype == "f32":
        return _close(name, gpu, ref, dtype)
    g = gpu.float().cpu().numpy().astype(np.float64)
    n_above, worst = P.wgrad_excess(g, ref, absref)
    rms = float(np.sqrt(np.mean(np.asarray(ref, dtype=np.float64) ** 2)))
    _say(f"[backward]   {name}: max |err| / sum|u v| = {worst:.2e} (bound {ABS_BOUND:.2e}), "
         f"max_err/rms={float(np.max(np.abs(g - ref))) / rms if rms > 0 else 0.0:.2e}")
    assert n_above == 0, f"{name}: {n_above} elements above the bound"
    return worst


def _run(w, inp, dout, padding_mask=None):
    S = w.n_shared
    out = B.backward(inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"],
                     inp["wsh_gu"] if S else None, inp["wsh_d"] if S else None, w.top_k, inp["route_scale"],
                     inp["global_scale"], dout, padding_mask=padding_mask, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    return out


def _full_backward(w, padding_mask=None, dout=None, dout_rows=None):
    """dout_rows: the only tokens where dout is non-zero; dx is then compared
    on those rows (its RMS over all rows would be diluted by exact zeros), and
    must be exactly zero on the others."""
    _say(f"[backward] {w}")
    inp = wl.make_inputs(w, device=DEV)
    dout = _dout(w) if dout is None else dout
    g = _run(w, inp, dout, padding_mask)
    S = w.n_shared
    pm = None if padding_mask is None else padding_mask.cpu().numpy().astype(bool)
    ref = oracle.moe_backward(P.host(inp["x"]), P.host(inp["gate_bank"]), P.host(inp["bias"]),
                              P.HostExperts(inp["w_gu"]), P.HostExperts(inp["w_d"]),
                              P.HostExperts(inp["wsh_gu"] if S else None), P.HostExperts(inp["wsh_d"] if S else None),
                              w.top_k, w.route_scale, w.global_scale, P.host(dout), padding_mask=pm, with_abs=True)
    E = w.n_routed
    st = lambda d: np.stack([d[e] for e in range(E)])
    if dout_rows is not None:
        others = np.setdiff1d(np.arange(w.T), dout_rows)
        assert not bool(g["dx"][torch.as_tensor(others, device=g["dx"].device)].any()), "dx non-zero where dout is 0"
        rel = {"dx": _close("dx", g["dx"][list(dout_rows)], ref["dx"][dout_rows], w.dtype)}
    else:
        rel = {"dx": _close("dx", g["dx"], ref["dx"], w.dtype)}
    rel.update({
           "d_gate_bank": _close("d_gate_bank", g["d_gate_bank"], ref["d_gate_bank"], w.dtype),
           "d_w_gu": _close_wgrad("d_w_gu", g["d_w_gu"], st(ref["d_w_gu"]), st(ref["abs_w_gu"]), w.dtype),
           "d_w_d": _close_wgrad("d_w_d", g["d_w_d"], st(ref["d_w_d"]), st(ref["abs_w_d"]), w.dtype)})
    if S:
        rel["d_wsh_gu"] = _close_wgrad("d_wsh_gu", g["d_wsh_gu"], ref["d_wsh_gu"], ref["abs_wsh_gu"], w.dtype)
        rel["d_wsh_d"] = _close_wgrad("d_wsh_d", g["d_wsh_d"], ref["d_wsh_d"], ref["abs_wsh_d"], w.dtype)
    _say("[backward] ok: " + " ".join(f"{k}={v:.2e}" for k, v in rel.items()))
    return g


CASES = {
    "tiny_fp32": wl.WORKLOADS["tiny_fp32"],
    "ragged_bf16": wl.custom(T=200, hidden=256, n_routed=16, top_k=4, n_shared=2, intermediate=128,
                             route_scale=2.5, gate_dist=("uniform", 0.05), bias_dist=("uniform", 0.05)),
    "few_rows_empty_experts": wl.custom(T=37, hidden=256, n_routed=32, top_k=3, n_shared=1, intermediate=192),
    "no_shared": wl.custom(T=100, hidden=128, n_routed=8, top_k=2, n_shared=0, intermediate=64),
    "f32_many_rows": wl.custom(T=300, hidden=128, n_routed=4, top_k=2, n_shared=1, intermediate=64, dtype="f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward(name):
    _full_backward(CASES[name])


def test_backward_padding_mask():
    w = CASES["ragged_bf16"]
    g = torch.Generator().manual_seed(11)
    mask = (torch.rand((w.T,), generator=g) < 0.3).to(torch.uint8).to(DEV)
    _full_backward(w, padding_mask=mask)


@pytest.mark.parametrize("S", [2, 0])
def test_backward_every_token_padded(S):
    """No routed rows: the routed weight gradients are exact zeros, and without
    shared experts so are dx and the gate-bank gradient."""
    w = CASES["ragged_bf16"]
    if S != w.n_shared:
        w = wl.custom(T=w.T, hidden=w.hidden, n_routed=w.n_routed, top_k=w.top_k, n_shared=S,
                      intermediate=w.intermediate)
    mask = torch.ones((w.T,), dtype=torch.uint8, device=DEV)
    g = _full_backward(w, padding_mask=mask)
    assert not bool(g["d_w_gu"].any()) and not bool(g["d_w_d"].any())
    if S == 0:
        assert not bool(g["dx"].any()) and not bool(g["d_gate_bank"].any())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_sparse_dout_at_stage_edges(dtype):
    """Experts of 4083 rows (every token picks all four experts, so row r of
    each expert is token r; K pads to 4096) with dout non-zero only on about
    30 tokens: the first and last rows of K stages, the rows around a middle
    stage start, and rows of the padded last stage.  Each weight-gradient
    element then sums over those rows only, so the componentwise bf16 bound
    (and the fp32 RMS bar) sees any dropped, doubled or misplaced row of the
    K loop; tests/test_parity_bars.py shows the bound rejecting such errors."""
    w = wl.custom(name=f"sparse_dout_{dtype}", T=4083, hidden=256, n_routed=4, top_k=4, n_shared=1,
                  intermediate=128, dtype=dtype, route_scale=2.5, gate_dist=("uniform", 0.05),
                  bias_dist=("uniform", 0.05))
    rows = P.stage_edge_rows(w.T)
    g = torch.Generator().manual_seed(13)
    dout = torch.zeros((w.T, w.hidden), dtype=torch.float32)
    dout[rows] = torch.randn((len(rows), w.hidden), generator=g)
    _say(f"[backward] sparse dout on {len(rows)} rows: {rows}")
    _full_backward(w, dout=dout.to(w.torch_dtype).to(DEV), dout_rows=rows)


def test_backward_small_bf16():
    _full_backward(wl.WORKLOADS["small_bf16"])


def test_backward_deterministic():
    w = CASES["ragged_bf16"]
    inp = wl.make_inputs(w, device=DEV)
    dout = _dout(w)
    a = _run(w, inp, dout)
    b = _run(w, inp, dout)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def test_backward_prefill_h6144_sampled():
    """hidden=6144, T=8192: dx of sampled tokens, the weight gradients of two
    routed experts and of the shared experts, against the oracle."""
    w = wl.WORKLOADS["prefill_h6144"]
    inp = wl.make_inputs(w, device=DEV)
    dout = _dout(w)
    g = _run(w, inp, dout)
    rng = np.random.default_rng(5)
    rows = sorted(set([0, w.T - 1] + rng.choice(w.T, size=10, replace=False).tolist()))
    experts = [3, 77]
    ref = oracle.moe_backward(P.host(inp["x"]), P.host(inp["gate_bank"]), P.host(inp["bias"]),
                              P.HostExperts(inp["w_gu"]), P.HostExperts(inp["w_d"]), P.HostExperts(inp["wsh_gu"]),
                              P.HostExperts(inp["wsh_d"]), w.top_k, w.route_scale, w.global_scale, P.host(dout),
                              tokens=rows, experts=experts, with_abs=True)
    rel = {"dx": _close("dx", g["dx"][rows], ref["dx"], "bf16")}
    for e in experts:
        rel[f"d_w_gu[{e}]"] = _close_wgrad("d_w_gu", g["d_w_gu"][e], ref["d_w_gu"][e], ref["abs_w_gu"][e], "bf16")
        rel[f"d_w_d[{e}]"] = _close_wgrad("d_w_d", g["d_w_d"][e], ref["d_w_d"][e], ref["abs_w_d"][e], "bf16")
    rel["d_wsh_gu"] = _close_wgrad("d_wsh_gu", g["d_wsh_gu"], ref["d_wsh_gu"], ref["abs_wsh_gu"], "bf16")
    rel["d_wsh_d"] = _close_wgrad("d_wsh_d", g["d_wsh_d"], ref["d_wsh_d"], ref["abs_wsh_d"], "bf16")
    _say("[backward] prefill_h6144 ok: " + " ".join(f"{k}={v:.2e}" for k, v in rel.items()))


SAVED_CASES = {
    "ragged_bf16": CASES["ragged_bf16"],
    "f32_many_rows": CASES["f32_many_rows"],
    "few_rows_empty_experts": CASES["few_rows_empty_experts"],
    "no_shared": CASES["no_shared"],
    # <= 48 rows per expert: the forward runs the few-token tiles, the backward
    # the 256-row tiles; the projections agree bit for bit all the same
    "few_token_tiles": wl.custom(T=24, hidden=256, n_routed=32, top_k=3, n_shared=2, intermediate=128),
    "prefill_h6144": wl.WORKLOADS["prefill_h6144"],
}


@pytest.mark.parametrize("name", list(SAVED_CASES))
def test_training_forward_and_saved_backward(name):
    """inkling_moe_forward_train gives the forward's output bit for bit, and the
    backward from its saved projections gives the recomputing backward's
    gradients bit for bit (same routing, same GEMM K order)."""
    w = SAVED_CASES[name]
    g = torch.Generator().manual_seed(11)
    mask = None
    if name == "ragged_bf16":
        mask = (torch.rand((w.T,), generator=g) < 0.3).to(torch.uint8).to(DEV)
    saved_vs_recompute(name, w, mask)


def saved_vs_recompute(name, w, mask):
    _say(f"[saved] {w}")
    inp = wl.make_inputs(w, device=DEV)
    S = w.n_shared
    args = (inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"], inp["wsh_gu"] if S else None,
            inp["wsh_d"] if S else None, w.top_k, inp["route_scale"], inp["global_scale"])
    dims = B.make_dims(w.T, w.hidden, w.n_routed, w.top_k, S, w.intermediate, w.torch_dtype)
    saved = torch.empty(B.saved_size(dims), dtype=torch.uint8, device=DEV)
    out_f = B.forward(*args, padding_mask=mask)
    out_t = B.forward(*args, padding_mask=mask, saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_t), "training forward output differs from the forward"
    dout = _dout(w)
    g_re = B.backward(*args, dout, padding_mask=mask, dx_dtype=torch.float32)
    g_sv = B.backward(*args, dout, padding_mask=mask, dx_dtype=torch.float32, saved=saved)
    torch.cuda.synchronize()
    for k in g_re:
        if g_re[k] is not None:
            assert torch.equal(g_re[k], g_sv[k]), f"{k} differs between saved and recomputed projections"
    _say(f"[saved] {name} ok: forward and every gradient bit-identical")


BF16_GRAD_CASES = {
    "ragged_bf16": CASES["ragged_bf16"],
    "f32_many_rows": CASES["f32_many_rows"],
    "few_rows_empty_experts": CASES["few_rows_empty_experts"],
    "no_shared": CASES["no_shared"],
    "prefill_h6144": wl.WORKLOADS["prefill_h6144"],
}


@pytest.mark.parametrize("name", list(BF16_GRAD_CASES))
def test_bf16_weight_gradients_are_the_rounded_fp32_ones(name):
    """weight_grad_dtype = bf16 stores each weight gradient as its fp32 value
    rounded to nearest-even, bit for bit; dx and the gate-bank gradient do not
    change.  (The fp32 gradients are the ones compared with the oracle.)"""
    w = BF16_GRAD_CASES[name]
    _say(f"[bf16 grads] {w}")
    inp = wl.make_inputs(w, device=DEV)
    S = w.n_shared
    args = (inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"], inp["wsh_gu"] if S else None,
            inp["wsh_d"] if S else None, w.top_k, inp["route_scale"], inp["global_scale"])
    dout = _dout(w)
    g32 = B.backward(*args, dout)
    g16 = B.backward(*args, dout, weight_grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for k in ("d_w_gu", "d_w_d", "d_wsh_gu", "d_wsh_d"):
        if g32[k] is None:
            assert g16[k] is None
            continue
        assert g16[k].dtype == torch.bfloat16
        assert torch.equal(g16[k], g32[k].to(torch.bfloat16)), f"{k}: bf16 gradient is not the rounded fp32 one"
    for k in ("dx", "d_gate_bank"):
        assert torch.equal(g16[k], g32[k]), k
    _say(f"[bf16 grads] {name} ok")
