"""The entry points allocate nothing and synchronise nothing, so a caller can
capture them in a HIP graph: each test captures calls on a side stream,
replays the graph several times with eager library work in between, and
checks every replay bit for bit against the eager result."""
import sys

import pytest
import torch

from mixture_experts_feed_amd import binding as B
from mixture_experts_feed_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


CASES = {
    "ragged_bf16": wl.custom(T=200, hidden=256, n_routed=16, top_k=4, n_shared=2, intermediate=128),
    "few_token_tiles": wl.custom(T=24, hidden=256, n_routed=32, top_k=3, n_shared=2, intermediate=128),
}


def _args(w, inp):
    S = w.n_shared
    return (inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"], inp["wsh_gu"] if S else None,
            inp["wsh_d"] if S else None, w.top_k, inp["route_scale"], inp["global_scale"])


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replay(name):
    w = CASES[name]
    _say(f"[graph] forward {w}")
    inp = wl.make_inputs(w, device=DEV)
    args = _args(w, inp)
    dims = B.make_dims(w.T, w.hidden, w.n_routed, w.top_k, w.n_shared, w.intermediate, w.torch_dtype)
    ref = B.forward(*args)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    ws = B.alloc_workspace(dims, DEV)
    g = _capture(lambda: B.forward(*args, out=out, workspace=ws))
    for i in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager forward"
        other = B.forward(*args)   # eager library work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, ref)
    _say(f"[graph] forward {name} ok: 4 replays bit-identical")


def test_training_step_graph_replay():
    """The training forward and the backward from its kept projections in one graph."""
    w = CASES["ragged_bf16"]
    _say(f"[graph] training step {w}")
    inp = wl.make_inputs(w, device=DEV)
    args = _args(w, inp)
    dims = B.make_dims(w.T, w.hidden, w.n_routed, w.top_k, w.n_shared, w.intermediate, w.torch_dtype)
    dout = torch.randn((w.T, w.hidden), generator=torch.Generator().manual_seed(5)).to(w.torch_dtype).to(DEV)
    saved = torch.empty(B.saved_size(dims), dtype=torch.uint8, device=DEV)
    ref_out = B.forward(*args, saved=saved)
    ref = B.backward(*args, dout, saved=saved)
    torch.cuda.synchronize()
    out = torch.empty_like(ref_out)
    ws = B.alloc_workspace(dims, DEV)
    bws = torch.empty(B.backward_workspace_size(dims), dtype=torch.uint8, device=DEV)
    grads = {k: torch.empty_like(v) for k, v in ref.items() if v is not None}
    grads.update({k: None for k, v in ref.items() if v is None})

    def step():
        B.forward(*args, out=out, workspace=ws, saved=saved)
        B.backward(*args, dout, workspace=bws, grads=grads, saved=saved)

    g = _capture(step)
    for i in range(3):
        for v in grads.values():
            if v is not None:
                v.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}: forward output differs"
        for k, v in ref.items():
            if v is not None:
                assert torch.equal(grads[k], v), f"replay {i}: {k} differs"
        B.forward(*args)   # eager work between replays
        torch.cuda.synchronize()
    _say("[graph] training step ok: 3 replays bit-identical")
