"""inkling_moe_forward_noalloc through the C ABI, against inkling_moe_forward.

The variant without a workspace argument keeps its scratch in a static device
array of the library (INKLING_NOALLOC_SCRATCH_BYTES per GPU).  Two calls in a
row, the second with fewer tokens (so it runs on what the first left in the
array), must each give the bits of inkling_moe_forward with a freshly
allocated workspace: the output, the routing and the permutation.  The
decode-shaped case runs at hidden 6144 with the decode tile configuration.
"""
import ctypes
import sys

import pytest
import torch

from mixture_experts_feed_amd import binding as B
from mixture_experts_feed_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _args(w, inp):
    S = w.n_shared
    return (inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"], inp["wsh_gu"] if S else None,
            inp["wsh_d"] if S else None, w.top_k, inp["route_scale"], inp["global_scale"])


def _same(w, inp, out_dtype=None, padding_mask=None):
    args = _args(w, inp)
    ref, r_ref = B.forward(*args, return_routing=True, out_dtype=out_dtype, padding_mask=padding_mask)
    got, r_got = B.forward_noalloc(*args, return_routing=True, out_dtype=out_dtype, padding_mask=padding_mask)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), f"{w.name}: output differs from inkling_moe_forward"
    for k in r_ref:
        assert torch.equal(r_got[k], r_ref[k]), f"{w.name}: {k} differs from inkling_moe_forward"


PAIRS = {
    # prefill tiles (256 x 256), then a smaller call on the same scratch
    "bf16_T300_then_T37": (wl.custom("na_big", T=300, hidden=256, n_routed=16, top_k=4, n_shared=2,
                                     intermediate=128, route_scale=2.5, gate_dist=("uniform", 0.05),
                                     bias_dist=("uniform", 0.05)),
                           wl.custom("na_small", T=37, hidden=256, n_routed=16, top_k=4, n_shared=2,
                                     intermediate=128, route_scale=2.5, gate_dist=("uniform", 0.05),
                                     bias_dist=("uniform", 0.05))),
    "f32_T200_then_T64": (wl.custom("na_f32_big", T=200, hidden=128, n_routed=8, top_k=2, n_shared=1,
                                    intermediate=64, dtype="f32"),
                          wl.custom("na_f32_small", T=64, hidden=128, n_routed=8, top_k=2, n_shared=1,
                                    intermediate=64, dtype="f32")),
    # decode shapes at full width (few-token tiles, one-workgroup permutation for T <= 64)
    "h6144_T96_then_T32": (wl.custom("na_dec_big", T=96, hidden=6144, n_routed=16, top_k=8, n_shared=2,
                                     intermediate=2048, route_scale=2.5, gate_dist=("uniform", 0.05),
                                     bias_dist=("uniform", 0.05)),
                           wl.custom("na_dec_small", T=32, hidden=6144, n_routed=16, top_k=8, n_shared=2,
                                     intermediate=2048, route_scale=2.5, gate_dist=("uniform", 0.05),
                                     bias_dist=("uniform", 0.05))),
}


@pytest.mark.parametrize("name", list(PAIRS))
def test_noalloc_matches_forward_on_two_calls(name):
    first, second = PAIRS[name]
    _say(f"[noalloc] {name}")
    inp1 = wl.make_inputs(first, device=DEV)
    inp2 = wl.make_inputs(second, device=DEV)
    _same(first, inp1)
    _same(second, inp2)
    if first.dtype == "bf16":
        _same(second, inp2, out_dtype=torch.float32)
    g = torch.Generator().manual_seed(9)
    mask = (torch.rand((second.T,), generator=g) < 0.25).to(torch.uint8).to(DEV)
    _same(second, inp2, padding_mask=mask)
    _say(f"[noalloc] {name} ok")


def test_noalloc_too_large_enqueues_nothing():
    """Beyond the static scratch the call returns INKLING_ERR_TOO_LARGE and
    writes nothing (the sizes are checked before any launch)."""
    w = wl.custom("na_too_big", T=1024, hidden=6144, n_routed=16, top_k=8, n_shared=2, intermediate=2048)
    inp = wl.make_inputs(w, device=DEV, with_experts=False)
    out = torch.zeros((w.T, w.hidden), dtype=torch.bfloat16, device=DEV)
    dims = B.make_dims(w.T, w.hidden, w.n_routed, w.top_k, w.n_shared, w.intermediate, torch.bfloat16)
    assert B.workspace_size(dims) > B.INKLING_NOALLOC_SCRATCH_BYTES
    gate = B.Gate(inp["gate_bank"].data_ptr(), inp["bias"].data_ptr(), w.route_scale, w.global_scale)
    weights = torch.zeros((4,), dtype=torch.bfloat16, device=DEV)   # never read: the call stops first
    ex = B.Experts(weights.data_ptr(), weights.data_ptr(), weights.data_ptr(), weights.data_ptr())
    rc = B.load().inkling_moe_forward_noalloc(ctypes.byref(dims), inp["x"].data_ptr(), ctypes.byref(gate),
                                              ctypes.byref(ex), None, out.data_ptr(), None,
                                              torch.cuda.current_stream().cuda_stream)
    assert rc == B.INKLING_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert not bool(out.any())


def test_noalloc_graph_replay():
    """The callers it is for capture it in graphs: a captured call replays bit
    for bit, also after eager calls of another size have overwritten the
    static scratch in between."""
    w = PAIRS["bf16_T300_then_T37"][0]
    other_w = PAIRS["bf16_T300_then_T37"][1]
    _say(f"[noalloc] graph replay {w.name}")
    inp = wl.make_inputs(w, device=DEV)
    other = wl.make_inputs(other_w, device=DEV)
    args = _args(w, inp)
    ref = B.forward(*args)
    other_ref = B.forward(*_args(other_w, other))
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.forward_noalloc(*args, out=out)   # warm-up (and the scratch's set-up) before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.forward_noalloc(*args, out=out)
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from inkling_moe_forward"
        got = B.forward_noalloc(*_args(other_w, other))   # eager call of another size on the same scratch
        torch.cuda.synchronize()
        assert torch.equal(got, other_ref)
    _say("[noalloc] graph replay ok: 4 replays bit-identical")
