"""Seeded synthetic workloads for the Inkling MoE feed-forward.

This module only draws random inputs; it holds none of the layer's arithmetic.
It is the one piece shared by the HIP path's tests/bench and the CPU oracle:
both receive exactly the tensors made here.

Shapes follow the layer as the Inkling layers page
(nemo_automodel.components.models.inkling.layers) states it: hidden states
[T, hidden]; an fp32 gate bank of n_routed + n_shared rows (InklingGate); an
fp32 correction bias of n_routed entries (InklingCorrectionBias); per expert
an interleaved gate_up projection [2*I, hidden] and a down projection
[hidden, I] in nn.Linear [out, in] layout (InklingSharedExperts, inkling_swiglu).
The default scale of 0.02 for weights matches init_std of InklingMoE.init_weights.

Random streams: every tensor (and every expert's weights) has its own seed
derived from (workload family seed, tensor id, expert id), so one expert can be
regenerated on its own.  Hidden states, the gate bank and the bias are drawn on
the CPU with torch's CPU generator (bit-reproducible on any host).  Expert
weights are drawn on the device where they will live (torch's generator for that
device): gigabytes of weights are impractical to draw on a CPU generator, and
the oracle always reads the very same bytes back from that device.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

# tensor ids of the random streams
_TID_X = 1
_TID_X_MIX = 2
_TID_GATE = 3
_TID_BIAS = 4
_TID_W_GU = 5
_TID_W_D = 6
_TID_WSH_GU = 7
_TID_WSH_D = 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    hidden: int
    n_routed: int
    top_k: int
    n_shared: int
    intermediate: int
    dtype: str                      # "f32" or "bf16": hidden states, expert weights, output
    route_scale: float
    global_scale: float
    gate_dist: tuple                # ("normal", std) or ("uniform", half_width)
    bias_dist: tuple                # ("uniform", half_width) or ("zipf", s, lam)
    x_outlier: Optional[tuple] = None   # (fraction, std) of rows drawn with a larger std
    w_std: float = 0.02
    family_seed: int = 0            # seed of gate bank / bias / weight streams
    x_seed: int = 0                 # seed of the hidden-state stream

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def n_total(self) -> int:
        return self.n_routed + self.n_shared

    def flops_alg(self) -> float:
        """Algorithmic FLOPs of one forward: gate logits + (k+S) expert FFNs per token."""
        T, H, I = self.T, self.hidden, self.intermediate
        return 2.0 * T * H * self.n_total + 6.0 * T * (self.top_k + self.n_shared) * H * I

    def expert_bytes(self) -> int:
        """Bytes of one expert's gate_up + down weights."""
        es = 4 if self.dtype == "f32" else 2
        return 3 * self.hidden * self.intermediate * es


# Skewed-routing bias scale.  The bias is lam * log p_e with p_e ~ (e+1)^-1.2
# (Zipf popularity).  lam = 1 leaves far more than a fifth of the experts
# empty, so lam is calibrated on the seeded inputs until 26 of 128 experts
# (20%) receive no token; tests/golden/make_skew_lambda.py recomputes it with
# the oracle's routing and tests/test_workloads.py checks the count.
SKEW_LAMBDA = 0.103

WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload(
        "tiny_fp32", T=64, hidden=128, n_routed=8, top_k=2, n_shared=1, intermediate=64,
        dtype="f32", route_scale=1.0, global_scale=1.0,
        gate_dist=("normal", 0.02), bias_dist=("uniform", 0.01), family_seed=0, x_seed=0),
    "small_bf16": Workload(
        "small_bf16", T=4096, hidden=2048, n_routed=64, top_k=6, n_shared=1, intermediate=768,
        dtype="bf16", route_scale=2.5, global_scale=1.0,
        gate_dist=("uniform", 0.05), bias_dist=("uniform", 0.05), family_seed=0, x_seed=0),
    "prefill_h6144": Workload(
        "prefill_h6144", T=8192, hidden=6144, n_routed=128, top_k=8, n_shared=2, intermediate=2048,
        dtype="bf16", route_scale=2.5, global_scale=1.0,
        gate_dist=("uniform", 0.05), bias_dist=("uniform", 0.05), family_seed=0, x_seed=0),
    "decode_h6144": Workload(
        "decode_h6144", T=32, hidden=6144, n_routed=128, top_k=8, n_shared=2, intermediate=2048,
        dtype="bf16", route_scale=2.5, global_scale=1.0,
        gate_dist=("uniform", 0.05), bias_dist=("uniform", 0.05), family_seed=0, x_seed=0),
    # Inkling's own MoE defaults (InklingTextConfig on the configuration page:
    # hidden 6144, 256 routed experts, 6 per token, 2 shared, moe intermediate
    # 3072, route_scale 8), at the prefill token count and value distributions
    "inkling_default_h6144": Workload(
        "inkling_default_h6144", T=8192, hidden=6144, n_routed=256, top_k=6, n_shared=2, intermediate=3072,
        dtype="bf16", route_scale=8.0, global_scale=1.0,
        gate_dist=("uniform", 0.05), bias_dist=("uniform", 0.05), family_seed=0, x_seed=0),
    # the GEMM shapes of one GPU's share of the prefill layer under 8-way
    # expert parallelism: 1024 local tokens through the replicated shared
    # experts, and 16 local experts receiving T*k/8 = 8192 routed rows (about
    # 512 each); the routing here is local, where a real dispatch would bring
    # the rows from every GPU
    "ep8_shard_h6144": Workload(
        "ep8_shard_h6144", T=1024, hidden=6144, n_routed=16, top_k=8, n_shared=2, intermediate=2048,
        dtype="bf16", route_scale=2.5, global_scale=1.0,
        gate_dist=("uniform", 0.05), bias_dist=("uniform", 0.05), family_seed=0, x_seed=0),
    "skewed_h6144": Workload(
        "skewed_h6144", T=16384, hidden=6144, n_routed=128, top_k=8, n_shared=2, intermediate=2048,
        dtype="bf16", route_scale=2.5, global_scale=1.0,
        gate_dist=("uniform", 0.05), bias_dist=("zipf", 1.2, SKEW_LAMBDA),
        x_outlier=(0.1, 4.0), family_seed=0, x_seed=0),
}


def custom(name: str = "custom", **kw) -> Workload:
    """A workload with explicit sizes (parity cases, edge cases)."""
    base = dict(T=64, hidden=128, n_routed=8, top_k=2, n_shared=1, intermediate=64,
                dtype="bf16", route_scale=1.0, global_scale=1.0,
                gate_dist=("normal", 0.02), bias_dist=("uniform", 0.01))
    base.update(kw)
    return Workload(name, **base)


def _seed(w: Workload, tensor_id: int, expert_id: int = 0, base: Optional[int] = None) -> int:
    b = w.family_seed if base is None else base
    # distinct, fixed 63-bit seeds per (base, tensor, expert)
    return ((b * 1_000_003 + tensor_id) * 65_537 + expert_id + 1) & 0x7FFF_FFFF_FFFF_FFFF


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _draw(shape, dist, gen, device="cpu") -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.float32, device=device)
    if dist[0] == "normal":
        t.normal_(0.0, dist[1], generator=gen)
    elif dist[0] == "uniform":
        t.uniform_(-dist[1], dist[1], generator=gen)
    else:
        raise ValueError(dist)
    return t


def hidden_states(w: Workload, T: Optional[int] = None) -> torch.Tensor:
    """x [T, hidden] in the workload dtype, on the CPU.  N(0,1) rows; with
    x_outlier=(f, s) a seeded fraction f of rows is drawn with std s instead."""
    T = w.T if T is None else T
    x = torch.empty((T, w.hidden), dtype=torch.float32)
    x.normal_(0.0, 1.0, generator=_gen(_seed(w, _TID_X, T, base=w.x_seed)))
    if w.x_outlier is not None:
        frac, std = w.x_outlier
        pick = torch.rand((T,), generator=_gen(_seed(w, _TID_X_MIX, T, base=w.x_seed))) < frac
        x[pick] *= std
    return x.to(w.torch_dtype)


def gate_bank(w: Workload) -> torch.Tensor:
    """fp32 [n_routed + n_shared, hidden]: routed rows first, then shared rows."""
    return _draw((w.n_total, w.hidden), w.gate_dist, _gen(_seed(w, _TID_GATE)))


def correction_bias(w: Workload) -> torch.Tensor:
    """fp32 [n_routed]."""
    if w.bias_dist[0] == "zipf":
        _, s, lam = w.bias_dist
        logp = [-s * math.log(e + 1.0) for e in range(w.n_routed)]
        lse = math.log(sum(math.exp(v) for v in logp))
        return torch.tensor([lam * (v - lse) for v in logp], dtype=torch.float64).to(torch.float32)
    return _draw((w.n_routed,), w.bias_dist, _gen(_seed(w, _TID_BIAS)))


def expert_weights(w: Workload, device="cpu"):
    """(w_gu [E,2I,H], w_d [E,H,I], wsh_gu [S,2I,H], wsh_d [S,H,I]) in the workload
    dtype on `device`.  Drawn N(0, w_std) in fp32 per expert, then rounded."""
    E, S, H, I = w.n_routed, w.n_shared, w.hidden, w.intermediate
    dt = w.torch_dtype
    out = []
    for tid_gu, tid_d, n in ((_TID_W_GU, _TID_W_D, E), (_TID_WSH_GU, _TID_WSH_D, S)):
        gu = torch.empty((n, 2 * I, H), dtype=dt, device=device)
        dn = torch.empty((n, H, I), dtype=dt, device=device)
        for e in range(n):
            gu[e].copy_(_draw((2 * I, H), ("normal", w.w_std), _gen(_seed(w, tid_gu, e), device), device))
            dn[e].copy_(_draw((H, I), ("normal", w.w_std), _gen(_seed(w, tid_d, e), device), device))
        out += [gu, dn]
    return tuple(out)


def make_inputs(w: Workload, device="cpu", T: Optional[int] = None, with_experts: bool = True):
    """All layer inputs.  x / gate bank / bias are drawn on the CPU then moved."""
    d = {
        "x": hidden_states(w, T).to(device),
        "gate_bank": gate_bank(w).to(device),
        "bias": correction_bias(w).to(device),
        "route_scale": w.route_scale,
        "global_scale": w.global_scale,
    }
    if with_experts:
        d["w_gu"], d["w_d"], d["wsh_gu"], d["wsh_d"] = expert_weights(w, device)
    return d


# ---- InklingDenseMLP -------------------------------------------------------
_TID_DENSE_X = 11
_TID_DENSE_GU = 12
_TID_DENSE_D = 13


@dataclasses.dataclass(frozen=True)
class DenseWorkload:
    """InklingDenseMLP inputs: x [T, hidden] ~ N(0,1); gate_up [2I, hidden] and
    down [hidden, I] ~ N(0, w_std); the module's global_scale."""
    name: str
    T: int
    hidden: int
    intermediate: int
    dtype: str = "bf16"
    global_scale: float = 1.0
    w_std: float = 0.02
    seed: int = 0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def flops_alg(self) -> float:
        return 6.0 * self.T * self.hidden * self.intermediate


DENSE_WORKLOADS: Dict[str, DenseWorkload] = {
    # the first Inkling layer's dense MLP (dense_mlp_idx 0): intermediate_size
    # 24576 on the configuration page, at the prefill token count
    "dense_h6144": DenseWorkload("dense_h6144", T=8192, hidden=6144, intermediate=24576),
}


def dense_custom(name: str = "dense_custom", **kw) -> DenseWorkload:
    return DenseWorkload(name, **kw)


def dense_inputs(w: DenseWorkload, device="cpu") -> Dict[str, torch.Tensor]:
    """x drawn on the CPU generator; the weights on `device` (as for experts)."""
    x = torch.empty((w.T, w.hidden), dtype=torch.float32)
    x.normal_(0.0, 1.0, generator=_gen(_seed_plain(w.seed, _TID_DENSE_X, w.T)))
    gu = _draw((2 * w.intermediate, w.hidden), ("normal", w.w_std),
               _gen(_seed_plain(w.seed, _TID_DENSE_GU, 0), device), device)
    dn = _draw((w.hidden, w.intermediate), ("normal", w.w_std),
               _gen(_seed_plain(w.seed, _TID_DENSE_D, 0), device), device)
    return {"x": x.to(w.torch_dtype).to(device), "gate_up": gu.to(w.torch_dtype), "down": dn.to(w.torch_dtype),
            "global_scale": w.global_scale}


def _seed_plain(base: int, tensor_id: int, sub: int) -> int:
    return ((base * 1_000_003 + tensor_id) * 65_537 + sub + 1) & 0x7FFF_FFFF_FFFF_FFFF
