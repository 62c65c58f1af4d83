"""The parity bars reject the mistakes they are meant to catch (CPU only).

The bf16 weight-gradient bar is componentwise: |err| <= (2^-8 + 2^-10) sum_r
|u_r v_r| per element.  Over thousands of rows a single wrong row would hide
under that sum, so the GPU test that guards the weight-gradient K loop
(tests/test_gpu_backward.py, test_backward_sparse_dout_at_stage_edges) gives
dout non-zero rows only at K-stage edges and in the padded last stage.  Here,
on the same construction at a smaller size, the oracle's own gradient passes
the bar, and the same gradient with any one of those rows dropped, doubled or
paired with its neighbour's operand fails it.  The weight gradients are linear
in dout (the routing does not depend on it), so a row's contribution is the
gradient minus the gradient with that row of dout set to zero.
"""
import numpy as np
import pytest

import oracle
from tests import parity as P


def _case(seed=3, T=83, H=64, I=64, E=4, k=4, S=1):
    r = np.random.default_rng(seed)
    c = dict(x=r.standard_normal((T, H)), bank=r.uniform(-0.05, 0.05, (E + S, H)), bias=r.uniform(-0.05, 0.05, E),
             w_gu=r.normal(0, 0.02, (E, 2 * I, H)), w_d=r.normal(0, 0.02, (E, H, I)),
             wsh_gu=r.normal(0, 0.02, (S, 2 * I, H)), wsh_d=r.normal(0, 0.02, (S, H, I)), k=k)
    rows = P.stage_edge_rows(T)
    dout = np.zeros((T, H))
    dout[rows] = r.standard_normal((len(rows), H))
    return c, rows, dout


def _grads(c, dout):
    g = oracle.moe_backward(c["x"], c["bank"], c["bias"], c["w_gu"], c["w_d"], c["wsh_gu"], c["wsh_d"], c["k"],
                            2.5, 1.0, dout, with_abs=True)
    E = c["bias"].shape[0]
    st = lambda d: np.stack([d[e] for e in range(E)])
    return {"d_w_gu": (st(g["d_w_gu"]), st(g["abs_w_gu"])), "d_w_d": (st(g["d_w_d"]), st(g["abs_w_d"])),
            "d_wsh_gu": (g["d_wsh_gu"], g["abs_wsh_gu"]), "d_wsh_d": (g["d_wsh_d"], g["abs_wsh_d"])}


def test_stage_edge_rows_cover_stage_edges_and_the_padded_stage():
    rows = P.stage_edge_rows(4083)
    assert 0 in rows and 31 in rows and 4082 in rows
    assert any(r % 32 == 0 and r > 0 for r in rows) and any(r % 32 == 31 and r > 31 for r in rows)
    assert sum(r >= 4064 for r in rows) >= 4          # the last stage (rows 4083..4095 are padding)
    assert 20 <= len(rows) <= 40


def test_wgrad_bound_accepts_the_oracle_and_rounded_operands():
    c, rows, dout = _case()
    for name, (ref, absref) in _grads(c, dout).items():
        assert P.wgrad_excess(ref, ref, absref)[0] == 0, name
        # an error of 2^-9 |u v| in every product (one bf16 rounding) stays inside
        r = np.random.default_rng(1)
        noisy = ref + (2.0 ** -9) * absref * r.uniform(-1, 1, ref.shape)
        assert P.wgrad_excess(noisy, ref, absref)[0] == 0, name


@pytest.mark.parametrize("mistake", ["dropped", "doubled", "neighbour"])
def test_wgrad_bound_rejects_one_wrong_row(mistake):
    """For every chosen row, and every weight gradient it feeds, the bar fails."""
    c, rows, dout = _case()
    full = _grads(c, dout)
    for i, r in enumerate(rows):
        d0 = dout.copy()
        d0[r] = 0.0
        without = _grads(c, d0)
        if mistake == "neighbour":
            # row r's dout paired with the next chosen row's operands: its
            # contribution computed from a shifted row
            d1 = dout.copy()
            d1[r] = 0.0
            d1[rows[(i + 1) % len(rows)]] += dout[r]
            wrong = _grads(c, d1)
        for name, (ref, absref) in full.items():
            bad = {"dropped": without[name][0], "doubled": 2 * ref - without[name][0],
                   "neighbour": wrong[name][0] if mistake == "neighbour" else None}[mistake]
            n_above, _ = P.wgrad_excess(bad, ref, absref)
            assert n_above > 0, f"{mistake} row {r} passes the {name} bar"
