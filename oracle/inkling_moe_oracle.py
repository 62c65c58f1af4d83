"""Plain fp64 CPU oracle of the Inkling MoE feed-forward.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call this module.  It shares no code
with the HIP library and imports nothing from it; inputs reach both sides from
mixture_experts_feed_amd/workloads.py, which draws random numbers only.

What it computes follows the Inkling layers page
(nemo_automodel.components.models.inkling.layers):

  * InklingGate: logits of the hidden states against a gate bank of n_routed
    routed rows plus n_shared shared rows (fp32 gate precision); selection by
    sigmoid(logit) + InklingCorrectionBias; returned weights = softmax of
    log-sigmoid over [selected routed logits || shared logits], times
    route_scale * global_scale.
  * inkling_swiglu: SwiGLU on the interleaved [g0, u0, g1, u1, ...] layout,
    the activated output scaled by the routing weight.
  * InklingSharedExperts: always-on experts whose outputs are weighted by the
    shared gammas before summation.
  * InklingMoE.forward: routed + shared outputs summed, output shaped like the
    input; masked tokens get no routed rows.
  * InklingDenseMLP: the dense SwiGLU MLP on the same interleaved layout,
    scaled by its global_scale parameter.
  * The backward of InklingMoE.forward: gradients of <dout, out> with respect
    to the hidden states, the gate bank and every expert weight, by the chain
    rule through the down projection, SwiGLU, the gate_up projection and the
    log-sigmoid softmax of the gate (the correction bias only moves the
    selection and gets no gradient).

Everything runs in float64 on the exact input values (bf16 and fp32 inputs widen
to fp64 without error, and their pairwise products are exact in fp64), with
numpy's matmul, argsort and cumsum as the only library steps.  Readings taken
where the pages are silent:
  * gate-bank row order: routed rows 0..E-1, shared rows E..E+S-1;
  * top-k order: descending biased score, equal scores -> lower expert index;
  * route_scale * global_scale scales the shared gammas too;
  * SwiGLU is silu(gate) * up with no clamp (hidden_act 'silu' on the
    configuration page, InklingTextConfig);
  * no normalisation of the hidden states inside the gate;
  * padded tokens still pass through the shared experts;
  * InklingDenseMLP's global_scale scales the MLP output.

Pins (tests/test_oracle_pins.py, all CPU): brute-force top-k over every subset
on tiny inputs, forced exact ties, the closed form sigma/sum(sigma) of the
log-sigmoid softmax, gammas summing to route_scale*global_scale, the
interleaved SwiGLU against the de-interleaved textbook form, a one-expert top-1
MoE against a dense SwiGLU MLP, token independence, expert relabelling, a
hand-derived worked example (test_hand_derived_example), and the dense MLP
against the textbook SwiGLU and against a one-expert top-1 MoE; the backward
against central finite differences of the forward oracle for every input.  Agreement with
the HuggingFace InklingTopkRouter or a real checkpoint: parity unpinned (neither
exists here).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# --------------------------------------------------------------------------
# InklingGate (layers page, InklingGate; InklingCorrectionBias)
# --------------------------------------------------------------------------

def gate_logits(x, gate_bank) -> np.ndarray:
    """z[t, j] = sum_h x[t, h] * bank[j, h]; rows j < E routed, E <= j shared.

    InklingGate: the weight bank holds the routed rows plus n_shared_experts
    rows; gate_precision defaults to float32, i.e. fp32 operands.  Here the sum
    is taken in fp64 over exactly widened operands.
    """
    return _f64(x) @ _f64(gate_bank).T


def sigmoid(z) -> np.ndarray:
    """sigma(z) = 1 / (1 + exp(-z))."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def log_sigmoid(z) -> np.ndarray:
    """log sigma(z) = -log(1 + exp(-z)), written for both signs of z without overflow."""
    z = _f64(z)
    return np.where(z >= 0, -np.log1p(np.exp(-np.abs(z))), z - np.log1p(np.exp(-np.abs(z))))


def selection_scores(z_routed, bias) -> np.ndarray:
    """s[t, e] = sigma(z[t, e]) + b[e]  (Inkling layers page, InklingGate: the
    sigmoid of each routed logit shifted by expert e's own bias term;
    InklingCorrectionBias.forward adds it in the routing score dtype, fp64
    here)."""
    return sigmoid(z_routed) + _f64(bias)[None, :]


def topk_select(scores, k: int) -> np.ndarray:
    """Indices [T, k] of the k largest scores per row, in descending score order,
    equal scores ordered by lower expert index (InklingGate.top_k =
    num_experts_per_tok; the tie rule is the reading taken here).

    A stable argsort of -s keeps equal keys in ascending index order.
    """
    s = _f64(scores)
    order = np.argsort(-s, axis=1, kind="stable")
    return order[:, :k]


def softmax(v, axis=-1) -> np.ndarray:
    v = _f64(v)
    m = np.max(v, axis=axis, keepdims=True)
    e = np.exp(v - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def route(z, bias, n_routed: int, top_k: int, route_scale: float, global_scale: float):
    """InklingGate.forward from the logits.

    Returns (topk_weights [T,k] fp64, topk_indices [T,k] int64,
    shared_gammas [T,S] fp64, scores [T,E] fp64).  The weights come from the
    unbiased logits: softmax(log sigma([z_sel || z_shared])) * rs * gs.
    """
    z = _f64(z)
    zr, zs = z[:, :n_routed], z[:, n_routed:]
    s = selection_scores(zr, bias)
    idx = topk_select(s, top_k)
    z_sel = np.take_along_axis(zr, idx, axis=1)
    ell = log_sigmoid(np.concatenate([z_sel, zs], axis=1))
    gam = softmax(ell, axis=1) * (float(route_scale) * float(global_scale))
    return gam[:, :top_k], idx.astype(np.int64), gam[:, top_k:], s


def topk_margin(scores, k: int) -> np.ndarray:
    """s_(k) - s_(k+1) per token (inf when k == E): how far the k-th pick is from
    the first one left out; used to report near-ties."""
    s = -np.sort(-_f64(scores), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


# --------------------------------------------------------------------------
# Token permutation (dispatch to GroupedExperts)
# --------------------------------------------------------------------------

def permutation(topk_indices, n_routed: int, token_mask=None):
    """Expert-sorted order of the routed slots.

    slot = t * k + i.  counts[e] = number of slots routed to e; offsets =
    exclusive prefix sum (length E+1); sorted_slots lists the slots of expert 0,
    then expert 1, ..., each in ascending slot order.  Tokens whose mask entry
    is True (padding) are left out (Inkling layers page, InklingMoE.forward:
    masked tokens get no routed rows).
    Returns (counts int64 [E], offsets int64 [E+1], sorted_slots int64 [n]).
    """
    idx = np.asarray(topk_indices, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    slots = np.arange(T * k, dtype=np.int64)
    if token_mask is not None:
        keep = ~np.repeat(np.asarray(token_mask, dtype=bool), k)
        flat, slots = flat[keep], slots[keep]
    counts = np.bincount(flat, minlength=n_routed).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    return counts, offsets, slots[order]


# --------------------------------------------------------------------------
# Experts (inkling_swiglu, InklingSharedExperts)
# --------------------------------------------------------------------------

def silu(v) -> np.ndarray:
    v = _f64(v)
    return v * sigmoid(v)


def swiglu_interleaved(h, routing_weights=None) -> np.ndarray:
    """inkling_swiglu: last axis interleaves [g0, u0, g1, u1, ...] (::2 gate,
    1::2 up); result silu(g) * u, scaled by routing_weights broadcast to
    [..., I]."""
    h = _f64(h)
    a = silu(h[..., 0::2]) * h[..., 1::2]
    if routing_weights is not None:
        a = a * _f64(routing_weights)
    return a


def expert_ffn(rows, w_gu, w_d, routing_weights=None) -> np.ndarray:
    """down_proj(inkling_swiglu(gate_up_proj(rows), w)) with nn.Linear layouts
    gate_up [2I, H] and down [H, I]."""
    h = _f64(rows) @ _f64(w_gu).T
    return swiglu_interleaved(h, routing_weights) @ _f64(w_d).T


def shared_experts(x, wsh_gu, wsh_d, gammas) -> np.ndarray:
    """InklingSharedExperts.forward: sum over s of gamma[:, s] * expert_s(x);
    each shared expert's output is multiplied by its gamma, then added."""
    x = _f64(x)
    g = _f64(gammas)
    out = np.zeros((x.shape[0], _f64(wsh_d[0]).shape[0] if len(wsh_d) else x.shape[1]), dtype=F64)
    for s in range(len(wsh_gu)):
        out += g[:, s:s + 1] * expert_ffn(x, wsh_gu[s], wsh_d[s])
    return out


# --------------------------------------------------------------------------
# InklingMoE.forward
# --------------------------------------------------------------------------

def moe_forward(x, gate_bank, bias, w_gu, w_d, wsh_gu, wsh_d, top_k: int,
                route_scale: float, global_scale: float, padding_mask=None,
                tokens=None, routing=None):
    """Output of the layer in fp64.

    x [T, H]; w_gu[e] [2I, H]; w_d[e] [H, I] for e < E (any sequence indexable
    per expert that yields arrays: weights are widened one expert at a time);
    wsh_* likewise for the S shared experts.  `tokens` (optional) restricts the
    output to those token rows (routing still covers every token, so counts and
    the permutation stay those of the full batch).  `routing` may pass a route()
    result computed earlier for the same inputs.

    Returns (out [len(tokens) or T, H] fp64, routing dict).
    """
    x = _f64(x)
    T = x.shape[0]
    E = _f64(bias).shape[0]
    if routing is None:
        z = gate_logits(x, gate_bank)
        tw, ti, sg, s = route(z, bias, E, top_k, route_scale, global_scale)
        counts, offsets, sorted_slots = permutation(ti, E, padding_mask)
        routing = dict(logits=z, topk_weights=tw, topk_indices=ti, shared_gammas=sg,
                       scores=s, counts=counts, offsets=offsets, sorted_slots=sorted_slots)
    tw, ti, sg = routing["topk_weights"], routing["topk_indices"], routing["shared_gammas"]
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    pad = np.zeros(T, dtype=bool) if padding_mask is None else np.asarray(padding_mask, dtype=bool)
    xr = x[rows]
    H = x.shape[1]
    out = np.zeros((len(rows), H), dtype=F64)
    # routed experts, one expert at a time over the (token, choice) pairs it received
    local_t, local_i = np.nonzero(ti[rows] >= 0)
    sel_e = ti[rows][local_t, local_i]
    live = ~pad[rows][local_t]
    local_t, local_i, sel_e = local_t[live], local_i[live], sel_e[live]
    for e in np.unique(sel_e):
        m = sel_e == e
        lt, li = local_t[m], local_i[m]
        y = expert_ffn(xr[lt], w_gu[e], w_d[e], tw[rows][lt, li][:, None])
        np.add.at(out, lt, y)
    if len(wsh_gu):
        out += shared_experts(xr, wsh_gu, wsh_d, sg[rows])
    return out, routing


# --------------------------------------------------------------------------
# InklingDenseMLP (layers page, InklingDenseMLP)
# --------------------------------------------------------------------------

def dense_mlp(x, w_gu, w_d, global_scale: float) -> np.ndarray:
    """InklingDenseMLP.forward (Inkling layers page): one SwiGLU MLP whose
    gate and up weights sit interleaved in a single projection [2I, H] (row
    2j gate_j, 2j+1 up_j), a down projection [H, I], and the module's
    global_scale parameter.  The page does not say
    where global_scale enters; it is read as scaling the MLP output (equal in
    exact arithmetic to scaling the activation, since down_proj is linear)."""
    return float(global_scale) * expert_ffn(x, w_gu, w_d)


# --------------------------------------------------------------------------
# Backward of InklingMoE.forward (gradients of L = <dout, out>)
# --------------------------------------------------------------------------

def silu_grad(v) -> np.ndarray:
    """d silu(v) / dv = sigma(v) * (1 + v * (1 - sigma(v)))."""
    v = _f64(v)
    s = sigmoid(v)
    return s * (1.0 + v * (1.0 - s))


def expert_backward(rows, w_gu, w_d, gammas, dout_rows, with_abs=False):
    """Backward of gamma * down(swiglu(gate_up(rows))) for the rows one expert
    received.  Returns (d rows [n, H], d gate_up [2I, H], d down [H, I],
    d gammas [n]); with_abs adds the sums of absolute products of the two
    weight-gradient contractions, |dh|^T |rows| and |dout|^T |a| (the scale of
    the componentwise rounding-error bound of those sums)."""
    X, Wgu, Wd, G = _f64(rows), _f64(w_gu), _f64(w_d), _f64(dout_rows)
    gam = _f64(gammas)
    h = X @ Wgu.T
    g, u = h[:, 0::2], h[:, 1::2]
    p = silu(g) * u                       # activation before the routing weight
    a = p * gam[:, None]                  # activation the down projection sees
    da = G @ Wd                           # [n, I]
    d_wd = G.T @ a                        # [H, I]
    d_gam = np.sum(da * p, axis=1)
    dp = da * gam[:, None]
    dh = np.empty_like(h)
    dh[:, 0::2] = dp * u * silu_grad(g)
    dh[:, 1::2] = dp * silu(g)
    if with_abs:
        return dh @ Wgu, dh.T @ X, d_wd, d_gam, np.abs(dh).T @ np.abs(X), np.abs(G).T @ np.abs(a)
    return dh @ Wgu, dh.T @ X, d_wd, d_gam


def router_backward(z, bias, n_routed: int, topk_indices, topk_weights, shared_gammas, d_topk_weights,
                    d_shared_gammas, route_scale: float, global_scale: float):
    """Gradient of the gate logits z [T, E+S] from the gradients of the
    returned weights.  gamma = c * softmax(l), c = route_scale * global_scale,
    l_j = log sigmoid(z_j) over the selected routed and the shared logits, so
    dl_j = q_j (c dgamma_j - sum_m q_m c dgamma_m) with q = gamma / c, and
    dz_j = dl_j (1 - sigma(z_j)).  Unselected routed logits and the correction
    bias, which only moves the selection, get no gradient."""
    z = _f64(z)
    T = z.shape[0]
    E = n_routed
    c = float(route_scale) * float(global_scale)
    zj = np.concatenate([np.take_along_axis(z[:, :E], topk_indices, axis=1), z[:, E:]], axis=1)
    q = np.concatenate([_f64(topk_weights), _f64(shared_gammas)], axis=1) / c
    dq = c * np.concatenate([_f64(d_topk_weights), _f64(d_shared_gammas)], axis=1)
    dl = q * (dq - np.sum(q * dq, axis=1, keepdims=True))
    dzj = dl * (1.0 - sigmoid(zj))
    dz = np.zeros_like(z)
    k = topk_indices.shape[1]
    np.add.at(dz, (np.repeat(np.arange(T), k), topk_indices.reshape(-1)), dzj[:, :k].reshape(-1))
    dz[:, E:] = dzj[:, k:]
    return dz


def moe_backward(x, gate_bank, bias, w_gu, w_d, wsh_gu, wsh_d, top_k: int, route_scale: float,
                 global_scale: float, dout, padding_mask=None, routing=None, tokens=None, experts=None,
                 with_abs=False):
    """Gradients of L = sum(dout * InklingMoE.forward(x)) in fp64.

    Returns a dict:
      dx [T or len(tokens), H]; d_gate_bank [E+S, H] (only when tokens is None);
      d_w_gu {e: [2I, H]}, d_w_d {e: [H, I]} for the routed experts in
      `experts` (default all; an expert that received no token has zero
      gradients); d_wsh_gu [S, 2I, H], d_wsh_d [S, H, I]; dz [T', E+S];
      d_topk_weights [T', k], d_shared_gammas [T', S];
      with_abs: abs_w_gu / abs_w_d (dicts like d_w_gu / d_w_d) and abs_wsh_gu /
      abs_wsh_d, the sums of absolute products of each weight gradient.
    Padded tokens skip the routed experts (their routed weights get no
    gradient) and keep the shared experts."""
    x, G = _f64(x), _f64(dout)
    T, H = x.shape
    E = _f64(bias).shape[0]
    S = len(wsh_gu)
    if routing is None:
        z = gate_logits(x, gate_bank)
        tw, ti, sg, s = route(z, bias, E, top_k, route_scale, global_scale)
        routing = dict(logits=z, topk_weights=tw, topk_indices=ti, shared_gammas=sg)
    z, tw, ti, sg = routing["logits"], routing["topk_weights"], routing["topk_indices"], routing["shared_gammas"]
    pad = np.zeros(T, dtype=bool) if padding_mask is None else np.asarray(padding_mask, dtype=bool)
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    want = range(E) if experts is None else [int(e) for e in experts]
    R = len(rows)
    dx = np.zeros((R, H), dtype=F64)
    d_tw = np.zeros((R, top_k), dtype=F64)
    d_sg = np.zeros((R, S), dtype=F64)
    res = {"d_w_gu": {}, "d_w_d": {}, "abs_w_gu": {}, "abs_w_d": {}}
    # routed experts: pairs (local row, choice) of the rows asked for
    lt_all, li_all = np.nonzero(~pad[rows][:, None] & (ti[rows] >= 0))
    e_all = ti[rows][lt_all, li_all]
    for e in np.unique(e_all):
        m = e_all == e
        lt, li = lt_all[m], li_all[m]
        out = expert_backward(x[rows][lt], w_gu[e], w_d[e], tw[rows][lt, li], G[rows][lt],
                              with_abs=with_abs and tokens is None)
        dX, dgu, dd, dgam = out[:4]
        np.add.at(dx, lt, dX)
        d_tw[lt, li] = dgam
        if tokens is None:
            res["d_w_gu"][int(e)], res["d_w_d"][int(e)] = dgu, dd
            if with_abs:
                res["abs_w_gu"][int(e)], res["abs_w_d"][int(e)] = out[4], out[5]
    # weight gradients of the asked experts over every token (when rows was a subset)
    for e in want:
        if e in res["d_w_gu"]:
            continue
        t_e, i_e = np.nonzero(~pad[:, None] & (ti == e))
        if len(t_e) == 0:
            res["d_w_gu"][e] = res["abs_w_gu"][e] = np.zeros_like(_f64(w_gu[e]))
            res["d_w_d"][e] = res["abs_w_d"][e] = np.zeros_like(_f64(w_d[e]))
            continue
        out = expert_backward(x[t_e], w_gu[e], w_d[e], tw[t_e, i_e], G[t_e], with_abs=with_abs)
        res["d_w_gu"][e], res["d_w_d"][e] = out[1], out[2]
        if with_abs:
            res["abs_w_gu"][e], res["abs_w_d"][e] = out[4], out[5]
    if experts is not None:
        for name in ("d_w_gu", "d_w_d", "abs_w_gu", "abs_w_d"):
            res[name] = {e: res[name][e] for e in want if e in res[name]}
    # shared experts: every token
    d_wsh_gu, d_wsh_d, abs_wsh_gu, abs_wsh_d = [], [], [], []
    for s in range(S):
        full = expert_backward(x, wsh_gu[s], wsh_d[s], sg[:, s], G, with_abs=with_abs)
        if tokens is None:
            dX, dgam = full[0], full[3]
        else:
            dX, _, _, dgam = expert_backward(x[rows], wsh_gu[s], wsh_d[s], sg[rows, s], G[rows])
        dx += dX
        d_sg[:, s] = dgam
        d_wsh_gu.append(full[1])
        d_wsh_d.append(full[2])
        if with_abs:
            abs_wsh_gu.append(full[4])
            abs_wsh_d.append(full[5])
    # router
    dz = router_backward(z[rows], bias, E, ti[rows], tw[rows], sg[rows], d_tw, d_sg, route_scale, global_scale)
    dx += dz @ _f64(gate_bank)
    res.update(dx=dx, dz=dz, d_topk_weights=d_tw, d_shared_gammas=d_sg,
               d_wsh_gu=np.array(d_wsh_gu).reshape((S,) + np.shape(_f64(wsh_gu[0])) if S else (0,)),
               d_wsh_d=np.array(d_wsh_d).reshape((S,) + np.shape(_f64(wsh_d[0])) if S else (0,)))
    res["d_gate_bank"] = dz.T @ x if tokens is None else None
    if with_abs:
        res["abs_wsh_gu"] = np.array(abs_wsh_gu).reshape(res["d_wsh_gu"].shape)
        res["abs_wsh_d"] = np.array(abs_wsh_d).reshape(res["d_wsh_d"].shape)
    return res
