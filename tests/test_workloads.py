"""The seeded input generator: determinism, shapes, distributions, and the
skewed workload's calibrated bias (checked with the oracle's routing)."""
import json
import os

import numpy as np
import torch

import oracle
from mixture_experts_feed_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))


def test_shapes_and_dtypes_tiny():
    w = wl.WORKLOADS["tiny_fp32"]
    d = wl.make_inputs(w)
    assert d["x"].shape == (64, 128) and d["x"].dtype == torch.float32
    assert d["gate_bank"].shape == (9, 128) and d["gate_bank"].dtype == torch.float32
    assert d["bias"].shape == (8,)
    assert d["w_gu"].shape == (8, 128, 128) and d["w_d"].shape == (8, 128, 64)
    assert d["wsh_gu"].shape == (1, 128, 128) and d["wsh_d"].shape == (1, 128, 64)


def test_deterministic_and_per_expert_streams():
    w = wl.custom(T=16, hidden=64, n_routed=4, intermediate=64)
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    for k in ("x", "gate_bank", "bias", "w_gu", "w_d", "wsh_gu", "wsh_d"):
        assert torch.equal(a[k], b[k]), k
    # experts are independent streams
    assert not torch.equal(a["w_gu"][0], a["w_gu"][1])


def test_distributions_small_bf16():
    w = wl.WORKLOADS["small_bf16"]
    x = wl.hidden_states(w).float()
    assert x.dtype == torch.float32 and abs(float(x.std()) - 1.0) < 0.01
    g = wl.gate_bank(w)
    assert g.shape == (65, 2048) and float(g.abs().max()) <= 0.05
    b = wl.correction_bias(w)
    assert float(b.abs().max()) <= 0.05


def test_skewed_bias_leaves_a_fifth_of_experts_empty():
    with open(os.path.join(HERE, "golden", "skew_lambda.json")) as f:
        ref = json.load(f)
    assert wl.SKEW_LAMBDA == ref["lam"]
    w = wl.WORKLOADS["skewed_h6144"]
    x = wl.hidden_states(w).float().numpy()
    z = oracle.gate_logits(x, wl.gate_bank(w).numpy())
    _, idx, _, _ = oracle.route(z, wl.correction_bias(w).double().numpy(), w.n_routed,
                                w.top_k, w.route_scale, w.global_scale)
    counts, _, _ = oracle.permutation(idx, w.n_routed)
    assert int((counts == 0).sum()) == ref["target_empty"] == 26
    # outlier rows: about 10% of rows have std 4
    rs = np.std(x, axis=1)
    assert 0.08 < float(np.mean(rs > 2.0)) < 0.12


def test_inkling_default_shape_matches_configuration_page():
    """InklingTextConfig defaults (configuration page): hidden_size 6144,
    n_routed_experts 256, num_experts_per_tok 6, n_shared_experts 2,
    moe_intermediate_size 3072, route_scale 8.0; init std 0.02 (layers page)."""
    w = wl.WORKLOADS["inkling_default_h6144"]
    assert (w.hidden, w.n_routed, w.top_k, w.n_shared, w.intermediate) == (6144, 256, 6, 2, 3072)
    assert w.route_scale == 8.0 and w.global_scale == 1.0 and w.w_std == 0.02
    assert w.dtype == "bf16"
