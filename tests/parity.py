"""Helpers of the GPU-vs-oracle parity tests (not collected by pytest).

Bars (from the layer's contract):
  * expert indices and per-expert counts: bit-exact (tokens whose oracle
    top-k margin is below 1e-12 -- none in practice -- are reported and only
    required to be a valid top-k there);
  * offsets and sorted slots: bit-exact against a stable order;
  * gammas (topk_weights, shared_gammas): |gpu - oracle| <= 1e-5 * |oracle|;
  * output: max |gpu - oracle| <= 2e-2 * RMS(oracle) for bf16 inputs, 1e-4 * RMS
    for fp32, on the fp32 output of the layer (out_dtype fp32).  The bf16
    output is then required to be exactly that fp32 output rounded to
    nearest-even, so its only extra error is the rounding of the result itself
    (up to 2^-8 of each element, which at the largest elements of a heavy-tailed
    output exceeds 2e-2 * RMS for any bf16 result, exact or not).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TIE_BAND = 1e-12
GAMMA_RTOL = 1e-5
OUT_TOL = {"bf16": 2e-2, "f32": 1e-4}
# bf16 weight gradients: each element is a sum over rows of products u_r v_r
# of which one factor is rounded to bf16 (unit roundoff 2^-8) and the other is
# an exact input, accumulated in fp32 (K 2^-24 <= 2^-10 for K <= 16384 rows):
# |err| <= (2^-8 + 2^-10) sum_r |u_r v_r|
WGRAD_ABS_BOUND = 2.0 ** -8 + 2.0 ** -10
# weight-gradient K stages hold 32 rows of K (64-byte bf16 rows); K is an
# expert's row count padded to a multiple of 64
WGRAD_STAGE_ROWS = 32


class HostExperts:
    """Per-expert fp64 view of device weights (read one expert at a time)."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __len__(self):
        return 0 if self.t is None else self.t.shape[0]

    def __getitem__(self, e):
        return self.t[int(e)].float().cpu().numpy()


def host(t):
    return t.float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float32) else t.cpu().numpy()


def oracle_route(inp, top_k, padding_mask=None):
    x = host(inp["x"])
    bank = host(inp["gate_bank"])
    bias = host(inp["bias"])
    E = bias.shape[0]
    z = oracle.gate_logits(x, bank)
    tw, ti, sg, s = oracle.route(z, bias, E, top_k, inp["route_scale"], inp["global_scale"])
    pm = None if padding_mask is None else padding_mask.cpu().numpy().astype(bool)
    counts, offsets, sorted_slots = oracle.permutation(ti, E, pm)
    return dict(logits=z, topk_weights=tw, topk_indices=ti, shared_gammas=sg, scores=s,
                counts=counts, offsets=offsets, sorted_slots=sorted_slots,
                margin=oracle.topk_margin(s, top_k))


def check_routing(gpu, ref, top_k, check_perm=True):
    """Compare a GPU routing dict with the oracle's.  Returns the band size."""
    idx = gpu["topk_indices"].cpu().numpy().astype(np.int64)
    # near-ties only: exact ties (margin 0, e.g. duplicated gate rows) are
    # computed identically on both sides and must follow the lower-index rule
    band = (ref["margin"] > 0) & (ref["margin"] < TIE_BAND)
    ok = ~band
    assert np.array_equal(idx[ok], ref["topk_indices"][ok]), "expert indices differ from the oracle"
    if band.any():  # only a valid top-k is required there
        s = ref["scores"]
        for t in np.nonzero(band)[0]:
            kth = np.sort(s[t])[::-1][top_k - 1]
            assert np.all(s[t][idx[t]] >= kth - TIE_BAND)
    tw = gpu["topk_weights"].cpu().numpy().astype(np.float64)
    rw = ref["topk_weights"]
    assert np.all(np.abs(tw[ok] - rw[ok]) <= GAMMA_RTOL * np.abs(rw[ok])), \
        f"topk_weights rel err {np.max(np.abs(tw[ok] - rw[ok]) / np.abs(rw[ok]))}"
    sg = gpu["shared_gammas"].cpu().numpy().astype(np.float64)
    rs = ref["shared_gammas"]
    if rs.size:
        assert np.all(np.abs(sg - rs) <= GAMMA_RTOL * np.abs(rs)), \
            f"shared_gammas rel err {np.max(np.abs(sg - rs) / np.abs(rs))}"
    if check_perm and "expert_counts" in gpu and not band.any():
        assert np.array_equal(gpu["expert_counts"].cpu().numpy(), ref["counts"])
        assert np.array_equal(gpu["expert_offsets"].cpu().numpy(), ref["offsets"])
        n = int(ref["offsets"][-1])
        assert np.array_equal(gpu["sorted_slots"].cpu().numpy()[:n], ref["sorted_slots"])
    return int(band.sum())


def check_output(out_gpu, out_ref, dtype, rows=None):
    """max |gpu - oracle| over the compared rows <= tol * RMS(oracle)."""
    g = out_gpu.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g = g[rows]
    rms = float(np.sqrt(np.mean(out_ref ** 2)))
    err = float(np.max(np.abs(g - out_ref))) if out_ref.size else 0.0
    assert err <= OUT_TOL[dtype] * rms, f"max abs err {err:.3e} > {OUT_TOL[dtype]} * RMS {rms:.3e}"
    return err / rms if rms > 0 else 0.0


def wgrad_excess(g, ref, absref):
    """Elements of a bf16 weight gradient g above the componentwise bound
    WGRAD_ABS_BOUND * sum|u v| (plus 1e-6 RMS for the fp32 error already in
    the rounded factor).  Returns (number above, worst |err| / sum|u v|)."""
    g = np.asarray(g, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    absref = np.asarray(absref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    diff = np.abs(g - ref)
    excess = diff - WGRAD_ABS_BOUND * absref - 1e-6 * rms
    worst = float(np.max(diff / (absref + 1e-30 * rms + 1e-300))) if ref.size else 0.0
    return int(np.sum(excess > 0)), worst


def stage_edge_rows(n_rows, stage=WGRAD_STAGE_ROWS, extra=()):
    """Row positions of a weight-gradient K loop where a dropped, doubled or
    misplaced row is most likely: the first and last row of every eighth
    stage, the rows around the start of the middle stage, and rows spread over
    the last stage, which holds the padding when n_rows is not a multiple of
    64 (rows n_rows .. the next multiple read zeros).  About 30 rows for a few
    thousand."""
    rows = set()
    n_st = (n_rows + stage - 1) // stage
    for st in range(0, n_st, max(1, n_st // 8)):
        rows.update((st * stage, st * stage + stage - 1))
    mid = (n_st // 2) * stage
    rows.update((mid - 1, mid, mid + 1))
    last0 = ((n_rows - 1) // stage) * stage
    rows.update(range(last0, n_rows, max(1, (n_rows - last0) // 6)))
    rows.update((n_rows - 2, n_rows - 1))
    rows.update(extra)
    return sorted(r for r in rows if 0 <= r < n_rows)
