"""Pins of the CPU oracle against what the Inkling layers page and plain
mathematics fix, independently of the oracle's own formulas.

Every check here would fail under a plausible mistake in the oracle: a biased
logit leaking into the gammas, the shared logits dropped from the softmax,
route_scale not applied to the shared gammas, gate/up swapped in the
interleave, a transposed weight, a wrong tie rule, an unstable permutation.
"""
import itertools
import math

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("seed", range(40))
def test_topk_bruteforce_all_subsets(seed):
    """The chosen set maximises the summed score over all C(E,k) subsets, and the
    order is descending score (InklingGate top-k on sigmoid + bias)."""
    r = _rng(seed)
    E = int(r.integers(2, 10))
    k = int(r.integers(1, E + 1))
    T, H = 3, 5
    x = r.normal(size=(T, H))
    bank = r.normal(size=(E + 1, H))
    bias = r.uniform(-0.3, 0.3, size=E)
    z = oracle.gate_logits(x, bank)
    _, idx, _, s = oracle.route(z, bias, E, k, 1.0, 1.0)
    for t in range(T):
        st = [1.0 / (1.0 + math.exp(-float(z[t, e]))) + float(bias[e]) for e in range(E)]
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(st[e] for e in c))
        assert sorted(idx[t].tolist()) == sorted(best)
        picked = [st[e] for e in idx[t]]
        assert all(picked[i] >= picked[i + 1] for i in range(k - 1))
        # rank-count characterisation: e selected <=> fewer than k experts beat it
        for e in range(E):
            beaten_by = sum(1 for f in range(E) if st[f] > st[e] or (st[f] == st[e] and f < e))
            assert (e in idx[t]) == (beaten_by < k)


def test_topk_forced_ties_lower_index_wins():
    """Duplicated gate rows with equal bias give exactly equal scores; the lower
    expert index must be taken first and ordered first."""
    H, E, k = 4, 6, 3
    r = _rng(7)
    bank = r.normal(size=(E + 1, H))
    bank[4] = bank[1]            # experts 1 and 4 tie exactly
    bank[5] = bank[1]            # and 5
    x = r.normal(size=(1, H))
    bias = np.zeros(E)
    z = oracle.gate_logits(x, bank)
    # make the tied experts the best three by raising their logits
    bank[[1, 4, 5]] *= 0  # z = 0 for all three; push the others down
    bank[[0, 2, 3]] = -np.sign(x) * 5
    z = oracle.gate_logits(x, bank)
    assert z[0, 1] == z[0, 4] == z[0, 5]
    _, idx, _, _ = oracle.route(z, bias, E, k, 1.0, 1.0)
    assert idx[0].tolist() == [1, 4, 5]
    _, idx2, _, _ = oracle.route(z, bias, E, 2, 1.0, 1.0)
    assert idx2[0].tolist() == [1, 4]
    # a tie straddling the cut: only the lower index gets in
    bias2 = np.zeros(E)
    bias2[1] = 0.1
    _, idx3, _, _ = oracle.route(z, bias2, E, 2, 1.0, 1.0)
    assert idx3[0].tolist() == [1, 4]


def test_topk_zero_bias_is_topk_of_logits():
    """With zero bias the selection is the top-k of the raw logits (sigma is monotone)."""
    r = _rng(3)
    x = r.normal(size=(50, 16))
    bank = r.normal(size=(13, 16))
    z = oracle.gate_logits(x, bank)
    _, idx, _, _ = oracle.route(z, np.zeros(12), 12, 4, 1.0, 1.0)
    ref = np.argsort(-z[:, :12], axis=1, kind="stable")[:, :4]
    assert np.array_equal(idx, ref)


def test_topk_margin_hand_set():
    """s_(k) - s_(k+1): the k-th largest score minus the (k+1)-th, per row.
    Scores with distinct gaps (1/8, 1/4, 3/8, 1/2 in descending order) give
    a different margin for every k, so an off-by-one in either index fails;
    k = E has nothing left out (inf); an exact tie at the cut gives 0."""
    s = np.array([[0.125, 0.875, -0.375, 0.5, 0.75]])   # descending: .875 .75 .5 .125 -.375
    want = {1: 0.125, 2: 0.25, 3: 0.375, 4: 0.5}
    for k, m in want.items():
        assert oracle.topk_margin(s, k)[0] == m, k
    assert np.isinf(oracle.topk_margin(s, 5)[0])
    ties = np.array([[0.5, 0.25, 0.5, -1.0], [0.25, 0.5, 0.75, 1.0]])
    assert oracle.topk_margin(ties, 1).tolist() == [0.0, 0.25]
    assert oracle.topk_margin(ties, 2).tolist() == [0.25, 0.25]
    assert oracle.topk_margin(ties, 3).tolist() == [1.25, 0.25]


def test_bias_changes_selection_not_weights():
    """The correction bias steers selection only; the weights come from the
    unbiased logits (InklingGate: selection uses sigmoid + bias, weights use the
    log-sigmoid softmax of the logits)."""
    r = _rng(11)
    x = r.normal(size=(20, 8))
    bank = r.normal(size=(10, 8))
    z = oracle.gate_logits(x, bank)
    b = r.uniform(-0.5, 0.5, size=8)
    w, idx, sg, _ = oracle.route(z, b, 8, 3, 2.0, 1.0)
    sig = 1.0 / (1.0 + np.exp(-z))
    for t in range(20):
        den = sig[t, idx[t]].sum() + sig[t, 8:].sum()
        assert np.allclose(w[t], 2.0 * sig[t, idx[t]] / den, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- gammas

@pytest.mark.parametrize("rs,gs", [(1.0, 1.0), (2.5, 1.0), (8.0, 0.75)])
def test_gammas_closed_form_and_sum(rs, gs):
    """softmax(log sigma(l)) = sigma(l) / sum sigma(l); all k+S gammas sum to rs*gs."""
    r = _rng(5)
    E, S, k, H = 16, 2, 4, 32
    x = r.normal(size=(64, H)) * 3
    bank = r.normal(size=(E + S, H))
    bias = r.uniform(-0.05, 0.05, size=E)
    z = oracle.gate_logits(x, bank)
    w, idx, sg, _ = oracle.route(z, bias, E, k, rs, gs)
    allg = np.concatenate([w, sg], axis=1)
    assert np.allclose(allg.sum(axis=1), rs * gs, rtol=1e-12, atol=0)
    sig = 1.0 / (1.0 + np.exp(-z))
    sel = np.concatenate([np.take_along_axis(sig[:, :E], idx, 1), sig[:, E:]], axis=1)
    closed = rs * gs * sel / sel.sum(axis=1, keepdims=True)
    assert np.allclose(allg, closed, rtol=1e-13, atol=0)
    # linearity in rs * gs
    w1, _, sg1, _ = oracle.route(z, bias, E, k, 1.0, 1.0)
    assert np.allclose(w, w1 * rs * gs, rtol=1e-14, atol=0)
    assert np.allclose(sg, sg1 * rs * gs, rtol=1e-14, atol=0)


def test_gammas_no_shared_experts():
    """S = 0: the softmax runs over the selected routed logits only."""
    r = _rng(9)
    x = r.normal(size=(10, 8))
    bank = r.normal(size=(6, 8))
    z = oracle.gate_logits(x, bank)
    w, idx, sg, _ = oracle.route(z, np.zeros(6), 6, 2, 1.0, 1.0)
    assert sg.shape == (10, 0)
    assert np.allclose(w.sum(1), 1.0, rtol=1e-14)


def test_log_sigmoid_extremes():
    z = np.array([-800.0, -40.0, -1.0, 0.0, 1.0, 40.0, 800.0])
    ls = oracle.log_sigmoid(z)
    assert np.all(np.isfinite(ls))
    assert ls[0] == -800.0 and ls[-1] == 0.0
    assert abs(ls[3] + math.log(2.0)) < 1e-16
    assert abs(ls[2] - math.log(1.0 / (1.0 + math.e))) < 1e-15


# ---------------------------------------------------------------- SwiGLU / experts

def test_interleaved_swiglu_equals_deinterleaved():
    """inkling_swiglu on [g0,u0,g1,u1,...] == silu(W_g x) * (W_u x) with
    W_g = W_gu[0::2], W_u = W_gu[1::2] (textbook SwiGLU written out here)."""
    r = _rng(2)
    H, I = 24, 10
    x = r.normal(size=(7, H))
    w_gu = r.normal(size=(2 * I, H))
    g = x @ w_gu[0::2].T
    u = x @ w_gu[1::2].T
    ref = (g / (1.0 + np.exp(-g))) * u
    got = oracle.swiglu_interleaved(x @ w_gu.T)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-15)
    # swapping gate and up would not agree
    swapped = (u / (1.0 + np.exp(-u))) * g
    assert not np.allclose(got, swapped)
    wts = r.uniform(0.1, 2.0, size=(7, 1))
    assert np.allclose(oracle.swiglu_interleaved(x @ w_gu.T, wts), ref * wts, rtol=1e-15, atol=0)


def _dense_mlp(x, w_gu, w_d):
    """Textbook SwiGLU MLP: W_d (silu(W_g x) * W_u x), de-interleaved weights."""
    wg, wu = w_gu[0::2], w_gu[1::2]
    g = x @ wg.T
    return ((g / (1.0 + np.exp(-g))) * (x @ wu.T)) @ w_d.T


def test_one_expert_top1_equals_dense_mlp():
    """E = 1, k = 1, S = 0, rs = gs = 1: the gamma is 1 and the MoE is the dense
    SwiGLU MLP (the InklingDenseMLP form without its scale)."""
    r = _rng(4)
    T, H, I = 9, 16, 12
    x = r.normal(size=(T, H))
    bank = r.normal(size=(1, H))
    w_gu = r.normal(size=(1, 2 * I, H)) * 0.3
    w_d = r.normal(size=(1, H, I)) * 0.3
    out, rt = oracle.moe_forward(x, bank, np.zeros(1), w_gu, w_d, [], [], 1, 1.0, 1.0)
    assert np.allclose(rt["topk_weights"], 1.0, rtol=0, atol=1e-15)
    assert np.allclose(out, _dense_mlp(x, w_gu[0], w_d[0]), rtol=1e-12, atol=1e-13)


def test_one_expert_plus_identical_shared_equals_dense_mlp():
    """E = 1, k = 1, S = 1 with the shared weights equal to the routed weights:
    the two gammas sum to 1, so the output again equals the dense MLP."""
    r = _rng(6)
    T, H, I = 11, 16, 8
    x = r.normal(size=(T, H))
    bank = r.normal(size=(2, H))
    w_gu = r.normal(size=(1, 2 * I, H)) * 0.3
    w_d = r.normal(size=(1, H, I)) * 0.3
    out, rt = oracle.moe_forward(x, bank, np.zeros(1), w_gu, w_d, w_gu, w_d, 1, 1.0, 1.0)
    assert not np.allclose(rt["topk_weights"], 1.0)
    assert np.allclose(out, _dense_mlp(x, w_gu[0], w_d[0]), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- whole layer

def _random_layer(seed, T=12, H=16, E=6, k=2, S=2, I=8):
    r = _rng(seed)
    return dict(
        x=r.normal(size=(T, H)),
        gate_bank=r.normal(size=(E + S, H)) * 0.5,
        bias=r.uniform(-0.1, 0.1, size=E),
        w_gu=r.normal(size=(E, 2 * I, H)) * 0.2,
        w_d=r.normal(size=(E, H, I)) * 0.2,
        wsh_gu=r.normal(size=(S, 2 * I, H)) * 0.2,
        wsh_d=r.normal(size=(S, H, I)) * 0.2,
        top_k=k, route_scale=2.5, global_scale=1.0)


def test_token_independence_and_sampled_rows():
    L = _random_layer(1)
    out, _ = oracle.moe_forward(**L)
    for t in [0, 5, 11]:
        one = dict(L, x=L["x"][t:t + 1])
        o1, _ = oracle.moe_forward(**one)
        assert np.allclose(o1[0], out[t], rtol=1e-13, atol=1e-14)
    sub, _ = oracle.moe_forward(**L, tokens=[3, 7])
    assert np.allclose(sub, out[[3, 7]], rtol=1e-13, atol=1e-14)


def test_brute_force_per_token_loop():
    """Every output row equals the per-token definition written out with loops."""
    L = _random_layer(8, T=5, H=6, E=4, k=2, S=1, I=3)
    out, rt = oracle.moe_forward(**L)
    x, E, k = L["x"], 4, 2
    for t in range(5):
        z = [sum(x[t, h] * L["gate_bank"][j, h] for h in range(6)) for j in range(E + 1)]
        sig = [1.0 / (1.0 + math.exp(-v)) for v in z]
        sc = [sig[e] + L["bias"][e] for e in range(E)]
        sel = sorted(range(E), key=lambda e: (-sc[e], e))[:k]
        den = sum(sig[e] for e in sel) + sig[E]
        gam = [L["route_scale"] * sig[e] / den for e in sel] + [L["route_scale"] * sig[E] / den]
        ws = [(L["w_gu"][e], L["w_d"][e]) for e in sel] + [(L["wsh_gu"][0], L["wsh_d"][0])]
        acc = [0.0] * 6
        for (wg, wd), g in zip(ws, gam):
            hvec = [sum(wg[n, h] * x[t, h] for h in range(6)) for n in range(6)]
            a = [hvec[2 * j] / (1.0 + math.exp(-hvec[2 * j])) * hvec[2 * j + 1] for j in range(3)]
            for h in range(6):
                acc[h] += g * sum(wd[h, j] * a[j] for j in range(3))
        assert rt["topk_indices"][t].tolist() == sel
        assert np.allclose(out[t], acc, rtol=1e-12, atol=1e-14)


def test_expert_relabelling_equivariance():
    """Permuting the routed experts consistently (gate rows, bias, weights)
    permutes the indices and leaves the output unchanged."""
    L = _random_layer(3)
    out, rt = oracle.moe_forward(**L)
    E = 6
    perm = np.array([3, 0, 5, 1, 4, 2])          # new expert j is old expert perm[j]
    inv = np.argsort(perm)
    L2 = dict(L)
    L2["gate_bank"] = np.concatenate([L["gate_bank"][perm], L["gate_bank"][E:]])
    L2["bias"] = L["bias"][perm]
    L2["w_gu"] = L["w_gu"][perm]
    L2["w_d"] = L["w_d"][perm]
    out2, rt2 = oracle.moe_forward(**L2)
    assert np.allclose(out2, out, rtol=1e-12, atol=1e-14)
    assert np.array_equal(rt2["topk_indices"], inv[rt["topk_indices"]])


def test_permutation_properties():
    r = _rng(12)
    T, E, k = 200, 9, 3
    idx = np.stack([r.permutation(E)[:k] for _ in range(T)])
    counts, offsets, ss = oracle.permutation(idx, E)
    assert counts.tolist() == np.bincount(idx.reshape(-1), minlength=E).tolist()
    assert counts.sum() == T * k and offsets[-1] == T * k
    for e in range(E):
        seg = ss[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                      # stable: ascending slots
        assert np.all(idx.reshape(-1)[seg] == e)
    assert sorted(ss.tolist()) == list(range(T * k))
    mask = r.uniform(size=T) < 0.3
    c2, o2, s2 = oracle.permutation(idx, E, mask)
    assert c2.sum() == (~mask).sum() * k
    assert not np.any(mask[s2 // k])


def test_padding_mask_removes_routed_part_only():
    L = _random_layer(5)
    mask = np.zeros(12, dtype=bool)
    mask[[2, 9]] = True
    out, _ = oracle.moe_forward(**L, padding_mask=mask)
    full, rt = oracle.moe_forward(**L)
    shared_only = oracle.shared_experts(L["x"], L["wsh_gu"], L["wsh_d"], rt["shared_gammas"])
    assert np.allclose(out[mask], shared_only[mask], rtol=1e-13, atol=1e-14)
    assert np.allclose(out[~mask], full[~mask], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- worked example

def test_hand_derived_example():
    """A case small enough to derive by hand.

    x = [1, 2]; routed gate rows give logits z = [0, ln 3, -ln 3], the shared
    row gives 0; bias [0.3, 0, 0].  Scores: 0.5+0.3, 0.75, 0.25.
    k=1 picks expert 0 (the bias beats expert 1); gammas over
    [sigma(0), sigma(0)] = [1/2, 1/2] * rs*gs (rs=2, gs=1.5) = [1.5, 1.5].
    Expert 0: gate row [0,1] -> g=2, up row [1,1] -> u=3, down [1,-2]:
      y0 = 1.5 * silu(2) * 3 * [1, -2].
    Shared: gate [1,0] -> g=1, up [-1,1] -> u=1, down [2,1]:
      ysh = 1.5 * silu(1) * 1 * [2, 1].
    k=2 picks [0, 1]; gammas 3*[1/2, 3/4, 1/2]/(7/4) = [6/7, 9/7, 6/7];
    expert 1: gate [1,0] -> g=1, up [0,1] -> u=2, down [1,1].
    """
    ln3 = math.log(3.0)
    x = np.array([[1.0, 2.0]])
    bank = np.array([[0.0, 0.0], [ln3, 0.0], [-ln3, 0.0], [0.0, 0.0]])
    bias = np.array([0.3, 0.0, 0.0])
    w_gu = np.zeros((3, 2, 2))
    w_d = np.zeros((3, 2, 1))
    w_gu[0] = [[0, 1], [1, 1]]
    w_d[0] = [[1], [-2]]
    w_gu[1] = [[1, 0], [0, 1]]
    w_d[1] = [[1], [1]]
    wsh_gu = np.array([[[1.0, 0.0], [-1.0, 1.0]]])
    wsh_d = np.array([[[2.0], [1.0]]])

    def silu(v):
        return v / (1.0 + math.exp(-v))

    out, rt = oracle.moe_forward(x, bank, bias, w_gu, w_d, wsh_gu, wsh_d, 1, 2.0, 1.5)
    assert rt["topk_indices"].tolist() == [[0]]
    assert np.allclose(rt["topk_weights"], [[1.5]], rtol=1e-15)
    assert np.allclose(rt["shared_gammas"], [[1.5]], rtol=1e-15)
    exp = [4.5 * silu(2) + 3 * silu(1), -9 * silu(2) + 1.5 * silu(1)]
    assert np.allclose(out[0], exp, rtol=1e-14, atol=0)

    out2, rt2 = oracle.moe_forward(x, bank, bias, w_gu, w_d, wsh_gu, wsh_d, 2, 2.0, 1.5)
    assert rt2["topk_indices"].tolist() == [[0, 1]]
    assert np.allclose(rt2["topk_weights"], [[6 / 7, 9 / 7]], rtol=1e-14)
    assert np.allclose(rt2["shared_gammas"], [[6 / 7]], rtol=1e-14)
    y0 = (6 / 7) * 3 * silu(2) * np.array([1.0, -2.0])
    y1 = (9 / 7) * 2 * silu(1) * np.array([1.0, 1.0])
    ysh = (6 / 7) * silu(1) * np.array([2.0, 1.0])
    assert np.allclose(out2[0], y0 + y1 + ysh, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- dense MLP

def test_dense_mlp_is_textbook_swiglu_times_scale():
    rng = np.random.default_rng(21)
    T, H, I = 9, 12, 5
    x = rng.standard_normal((T, H))
    w_gu = rng.standard_normal((2 * I, H)) * 0.3
    w_d = rng.standard_normal((H, I)) * 0.3
    g, u = x @ w_gu[0::2].T, x @ w_gu[1::2].T
    textbook = ((g / (1.0 + np.exp(-g))) * u) @ w_d.T
    out = oracle.dense_mlp(x, w_gu, w_d, 0.75)
    assert np.allclose(out, 0.75 * textbook, rtol=1e-13, atol=1e-14)
    # linear in global_scale; zero scale gives zero
    assert np.allclose(oracle.dense_mlp(x, w_gu, w_d, 1.5), 2.0 * out, rtol=1e-14, atol=0)
    assert np.all(oracle.dense_mlp(x, w_gu, w_d, 0.0) == 0.0)


def test_dense_mlp_equals_one_expert_moe_with_route_scale_as_global_scale():
    """A top-1 MoE over a single expert with no shared experts gives that expert
    gamma = route_scale * global_scale (softmax over one logit is 1), so it is
    the dense MLP with that scale, whatever the gate bank and bias."""
    rng = np.random.default_rng(22)
    T, H, I = 7, 10, 6
    x = rng.standard_normal((T, H))
    w_gu = rng.standard_normal((1, 2 * I, H)) * 0.3
    w_d = rng.standard_normal((1, H, I)) * 0.3
    bank = rng.standard_normal((1, H))
    bias = rng.standard_normal(1)
    moe, _ = oracle.moe_forward(x, bank, bias, w_gu, w_d, [], [], 1, 2.0, 0.625)
    assert np.allclose(moe, oracle.dense_mlp(x, w_gu[0], w_d[0], 1.25), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- backward

def _bw_case(seed, T=3, H=6, E=4, k=2, S=1, I=3, rs=1.7, gs=0.9):
    rng = np.random.default_rng(seed)
    c = dict(x=rng.standard_normal((T, H)), bank=rng.standard_normal((E + S, H)) * 0.5,
             bias=rng.standard_normal(E) * 0.1, w_gu=rng.standard_normal((E, 2 * I, H)) * 0.4,
             w_d=rng.standard_normal((E, H, I)) * 0.4, wsh_gu=rng.standard_normal((S, 2 * I, H)) * 0.4,
             wsh_d=rng.standard_normal((S, H, I)) * 0.4, dout=rng.standard_normal((T, H)), k=k, rs=rs, gs=gs)
    return c


def _loss(c, pad=None, **over):
    p = dict(c)
    p.update(over)
    out, _ = oracle.moe_forward(p["x"], p["bank"], p["bias"], p["w_gu"], p["w_d"], p["wsh_gu"], p["wsh_d"],
                                p["k"], p["rs"], p["gs"], padding_mask=pad)
    return float(np.sum(out * p["dout"]))


def _fd_grad(c, name, pad=None, eps=1e-6):
    base = c[name]
    g = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        hi, lo = base.copy(), base.copy()
        hi[idx] += eps
        lo[idx] -= eps
        g[idx] = (_loss(c, pad, **{name: hi}) - _loss(c, pad, **{name: lo})) / (2 * eps)
    return g


def _margins_clear(c, tol=1e-3):
    z = oracle.gate_logits(c["x"], c["bank"])
    s = oracle.selection_scores(z[:, :c["bias"].shape[0]], c["bias"])
    return np.all(oracle.topk_margin(s, c["k"]) > tol)


@pytest.mark.parametrize("seed,kw,padded", [
    (31, {}, False),
    (32, dict(S=2, k=1), False),
    (33, dict(S=0, k=2), False),
    (38, {}, True),
])
def test_backward_matches_finite_differences(seed, kw, padded):
    """Every gradient of L = <dout, out> against central differences of the
    forward oracle (the selection does not change under the perturbation: all
    top-k margins exceed 1e-3)."""
    c = _bw_case(seed, **kw)
    assert _margins_clear(c)
    pad = np.array([False, True, False]) if padded else None
    g = oracle.moe_backward(c["x"], c["bank"], c["bias"], c["w_gu"], c["w_d"], c["wsh_gu"], c["wsh_d"], c["k"],
                            c["rs"], c["gs"], c["dout"], padding_mask=pad)
    E = c["bias"].shape[0]
    checks = [("x", g["dx"]), ("bank", g["d_gate_bank"]),
              ("w_gu", np.stack([g["d_w_gu"][e] for e in range(E)])),
              ("w_d", np.stack([g["d_w_d"][e] for e in range(E)]))]
    if c["wsh_gu"].shape[0]:
        checks += [("wsh_gu", g["d_wsh_gu"]), ("wsh_d", g["d_wsh_d"])]
    for name, analytic in checks:
        fd = _fd_grad(c, name, pad)
        assert np.allclose(analytic, fd, rtol=1e-6, atol=1e-8), name
    # the correction bias only moves the selection: its finite difference is 0
    assert np.allclose(_fd_grad(c, "bias", pad), 0.0, atol=1e-8)


def test_backward_token_and_expert_subsets_agree_with_full():
    c = _bw_case(35, T=6, E=5, k=2, S=1)
    args = (c["x"], c["bank"], c["bias"], c["w_gu"], c["w_d"], c["wsh_gu"], c["wsh_d"], c["k"], c["rs"], c["gs"],
            c["dout"])
    full = oracle.moe_backward(*args)
    part = oracle.moe_backward(*args, tokens=[4, 1], experts=[3, 0])
    assert np.allclose(part["dx"], full["dx"][[4, 1]], rtol=1e-13, atol=1e-14)
    assert np.allclose(part["dz"], full["dz"][[4, 1]], rtol=1e-13, atol=1e-14)
    for e in (3, 0):
        assert np.allclose(part["d_w_gu"][e], full["d_w_gu"][e], rtol=1e-13, atol=1e-14)
        assert np.allclose(part["d_w_d"][e], full["d_w_d"][e], rtol=1e-13, atol=1e-14)
    assert np.allclose(part["d_wsh_gu"], full["d_wsh_gu"], rtol=1e-13, atol=1e-14)
    assert part["d_gate_bank"] is None


def test_router_backward_weights_sum_rule():
    """The gammas sum to rs*gs, so dout-independent: a dgamma that is the same
    for every expert of a token gives dz = 0."""
    c = _bw_case(36, T=4, E=5, k=2, S=2)
    z = oracle.gate_logits(c["x"], c["bank"])
    tw, ti, sg, _ = oracle.route(z, c["bias"], 5, 2, c["rs"], c["gs"])
    const = np.full((4, 2), 0.37)
    dz = oracle.router_backward(z, c["bias"], 5, ti, tw, sg, const, np.full((4, 2), 0.37), c["rs"], c["gs"])
    assert np.allclose(dz, 0.0, atol=1e-14)


def test_backward_abs_sums_bound_the_gradients():
    """The absolute-product sums returned for the tolerance bound are >= |grad|
    elementwise, and equal to it for an expert that received a single row."""
    c = _bw_case(37, T=5, E=4, k=2, S=1)
    g = oracle.moe_backward(c["x"], c["bank"], c["bias"], c["w_gu"], c["w_d"], c["wsh_gu"], c["wsh_d"], c["k"],
                            c["rs"], c["gs"], c["dout"], with_abs=True)
    for e in g["d_w_gu"]:
        assert np.all(g["abs_w_gu"][e] >= np.abs(g["d_w_gu"][e]) - 1e-14)
        assert np.all(g["abs_w_d"][e] >= np.abs(g["d_w_d"][e]) - 1e-14)
    assert np.all(g["abs_wsh_gu"] >= np.abs(g["d_wsh_gu"]) - 1e-14)
    ti = oracle.route(oracle.gate_logits(c["x"], c["bank"]), c["bias"], 4, 2, c["rs"], c["gs"])[1]
    single = [e for e in range(4) if np.sum(ti == e) == 1]
    for e in single:
        assert np.allclose(g["abs_w_gu"][e], np.abs(g["d_w_gu"][e]), rtol=1e-13, atol=1e-15)
