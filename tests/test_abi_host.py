"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, sizes its workspace, and rejects bad arguments on the host
before anything is launched."""
import ctypes
import os
import re

import pytest

from mixture_experts_feed_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "inkling_moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from mixture_experts_feed_amd import build
        build.build(verbose=False)
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(inkling_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_stage_event_count_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+INKLING_STAGE_EVENTS\s+(\d+)", text)
    assert m and int(m.group(1)) == B.INKLING_STAGE_EVENTS == len(B.STAGES) + 1


def _dims(**kw):
    d = dict(T=64, hidden=128, n_routed=8, top_k=2, n_shared=1, intermediate=64, dtype=B.INKLING_BF16,
             out_dtype=B.INKLING_BF16)
    d.update(kw)
    return B.Dims(d["T"], d["hidden"], d["n_routed"], d["top_k"], d["n_shared"], d["intermediate"], d["dtype"],
                  d["out_dtype"])


def _ws(lib, **kw):
    n = ctypes.c_size_t(0)
    rc = lib.inkling_moe_workspace_size(ctypes.byref(_dims(**kw)), ctypes.byref(n))
    return rc, n.value


def test_workspace_size_grows_with_tokens(lib):
    rc0, n0 = _ws(lib, T=0)
    rc1, n1 = _ws(lib, T=64)
    rc2, n2 = _ws(lib, T=4096)
    assert rc0 == rc1 == rc2 == B.INKLING_OK
    assert 0 <= n0 < n1 < n2
    # the per-slot down-projection rows dominate: T*k*H*elem bytes
    assert n2 >= 4096 * 2 * 128 * 2


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=9), B.INKLING_ERR_INVALID_ARGUMENT),      # top_k > n_routed
    (dict(top_k=0), B.INKLING_ERR_INVALID_ARGUMENT),
    (dict(T=-1), B.INKLING_ERR_INVALID_ARGUMENT),
    (dict(n_shared=-1), B.INKLING_ERR_INVALID_ARGUMENT),
    (dict(hidden=0), B.INKLING_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), B.INKLING_ERR_UNSUPPORTED),
    (dict(out_dtype=3), B.INKLING_ERR_UNSUPPORTED),
    (dict(hidden=96), B.INKLING_ERR_UNSUPPORTED),          # hidden % 64
    (dict(intermediate=96), B.INKLING_ERR_UNSUPPORTED),    # intermediate % 64
    (dict(n_routed=600, top_k=2), B.INKLING_ERR_UNSUPPORTED),
    (dict(n_routed=64, top_k=33), B.INKLING_ERR_UNSUPPORTED),
    (dict(n_shared=17), B.INKLING_ERR_UNSUPPORTED),
    (dict(T=2 ** 30, top_k=2), B.INKLING_ERR_UNSUPPORTED),   # T * top_k past the int32 slot indices
])
def test_invalid_dims_rejected(lib, kw, code):
    rc, _ = _ws(lib, **kw)
    assert rc == code
    d = _dims(**kw)
    fake = ctypes.c_void_p(0x1000)
    gate = B.Gate(0x1000, 0x1000, 1.0, 1.0)
    ex = B.Experts(0x1000, 0x1000, 0x1000, 0x1000)
    rc = lib.inkling_moe_forward(ctypes.byref(d), fake, ctypes.byref(gate), ctypes.byref(ex), None,
                                 ctypes.c_void_p(0x2000), None, fake, 1 << 40, None)
    assert rc == code


def test_null_pointers_and_small_workspace_rejected(lib):
    d = _dims()
    gate = B.Gate(0x1000, 0x1000, 1.0, 1.0)
    ex = B.Experts(0x1000, 0x1000, 0x1000, 0x1000)
    ws = ctypes.c_void_p(0x3000)
    x = ctypes.c_void_p(0x4000)
    out = ctypes.c_void_p(0x5000)
    fwd = lib.inkling_moe_forward
    assert fwd(ctypes.byref(d), None, ctypes.byref(gate), ctypes.byref(ex), None, out, None, ws, 1 << 40,
               None) == B.INKLING_ERR_INVALID_ARGUMENT
    assert fwd(ctypes.byref(d), x, None, ctypes.byref(ex), None, out, None, ws, 1 << 40,
               None) == B.INKLING_ERR_INVALID_ARGUMENT
    bad_gate = B.Gate(None, 0x1000, 1.0, 1.0)
    assert fwd(ctypes.byref(d), x, ctypes.byref(bad_gate), ctypes.byref(ex), None, out, None, ws, 1 << 40,
               None) == B.INKLING_ERR_INVALID_ARGUMENT
    no_shared = B.Experts(0x1000, 0x1000, None, None)
    assert fwd(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(no_shared), None, out, None, ws, 1 << 40,
               None) == B.INKLING_ERR_INVALID_ARGUMENT
    # out aliasing x
    assert fwd(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, x, None, ws, 1 << 40,
               None) == B.INKLING_ERR_INVALID_ARGUMENT
    # workspace too small / missing
    assert fwd(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, out, None, ws, 16,
               None) == B.INKLING_ERR_WORKSPACE
    assert fwd(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, out, None, None, 1 << 40,
               None) == B.INKLING_ERR_WORKSPACE
    # route: required outputs
    ro = B.RouteOut(None, 0x1000, 0x1000, None, None, None)
    assert lib.inkling_moe_route(ctypes.byref(d), x, ctypes.byref(gate), None, ctypes.byref(ro), ws, 1 << 40,
                                 None) == B.INKLING_ERR_INVALID_ARGUMENT
    ro = B.RouteOut(0x1000, 0x1000, 0x1000, None, None, None)
    assert lib.inkling_moe_route(ctypes.byref(d), x, ctypes.byref(gate), None, ctypes.byref(ro), ws, 8,
                                 None) == B.INKLING_ERR_WORKSPACE


def test_zero_tokens_is_a_noop(lib):
    d = _dims(T=0)
    gate = B.Gate(None, None, 1.0, 1.0)
    assert lib.inkling_moe_forward(ctypes.byref(d), None, ctypes.byref(gate), None, None, None, None, None, 0,
                                   None) == B.INKLING_OK
    assert lib.inkling_moe_route(ctypes.byref(d), None, None, None, None, None, 0, None) == B.INKLING_OK


def test_strerror(lib):
    for c in (0, -1, -2, -3, -4, -5, -99):
        assert isinstance(lib.inkling_moe_strerror(c), bytes)
    assert lib.inkling_moe_last_hip_error() == 0


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), B.INKLING_ERR_INVALID_ARGUMENT),
    (dict(hidden=0), B.INKLING_ERR_INVALID_ARGUMENT),
    (dict(intermediate=0), B.INKLING_ERR_INVALID_ARGUMENT),
    (dict(dtype=5), B.INKLING_ERR_UNSUPPORTED),
    (dict(out_dtype=5), B.INKLING_ERR_UNSUPPORTED),
    (dict(hidden=96), B.INKLING_ERR_UNSUPPORTED),
    (dict(intermediate=160), B.INKLING_ERR_UNSUPPORTED),
])
def test_dense_invalid_dims_rejected(lib, kw, code):
    d = dict(T=64, hidden=128, intermediate=256, dtype=B.INKLING_BF16, out_dtype=B.INKLING_BF16)
    d.update(kw)
    dims = B.DenseDims(d["T"], d["hidden"], d["intermediate"], d["dtype"], d["out_dtype"])
    n = ctypes.c_size_t(0)
    assert lib.inkling_dense_mlp_workspace_size(ctypes.byref(dims), ctypes.byref(n)) == code
    fake = ctypes.c_void_p(0x1000)
    assert lib.inkling_dense_mlp_forward(ctypes.byref(dims), fake, fake, fake, 1.0, ctypes.c_void_p(0x2000), fake,
                                         1 << 40, None) == code


def test_dense_pointer_and_workspace_checks(lib):
    dims = B.DenseDims(64, 128, 256, B.INKLING_BF16, B.INKLING_BF16)
    n = ctypes.c_size_t(0)
    assert lib.inkling_dense_mlp_workspace_size(ctypes.byref(dims), ctypes.byref(n)) == B.INKLING_OK
    # gamma + counters + act [T][I] (2 bytes); the down projection writes the output directly
    assert n.value >= 64 * 256 * 2 + 64 * 4
    x, w, out, ws = (ctypes.c_void_p(v) for v in (0x1000, 0x2000, 0x3000, 0x4000))
    f = lib.inkling_dense_mlp_forward
    assert f(ctypes.byref(dims), None, w, w, 1.0, out, ws, n.value, None) == B.INKLING_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(dims), x, None, w, 1.0, out, ws, n.value, None) == B.INKLING_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(dims), x, w, w, 1.0, x, ws, n.value, None) == B.INKLING_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(dims), x, w, w, 1.0, out, ws, n.value - 1, None) == B.INKLING_ERR_WORKSPACE
    zero = B.DenseDims(0, 128, 256, B.INKLING_BF16, B.INKLING_BF16)
    assert f(ctypes.byref(zero), None, None, None, 1.0, None, None, 0, None) == B.INKLING_OK


def test_backward_argument_checks(lib):
    d = _dims()
    n = ctypes.c_size_t(0)
    assert lib.inkling_moe_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.INKLING_OK
    nf = ctypes.c_size_t(0)
    lib.inkling_moe_workspace_size(ctypes.byref(d), ctypes.byref(nf))
    assert n.value > nf.value
    gate = B.Gate(0x1000, 0x1000, 1.0, 1.0)
    ex = B.Experts(0x1000, 0x1000, 0x1000, 0x1000)
    gr = B.Grads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    x, dout, dx, ws = (ctypes.c_void_p(v) for v in (0x4000, 0x5000, 0x6000, 0x7000))
    bw = lib.inkling_moe_backward
    assert bw(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, None, None, dx, ctypes.byref(gr), ws,
              n.value, None) == B.INKLING_ERR_INVALID_ARGUMENT
    assert bw(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, dout, None, dout, ctypes.byref(gr), ws,
              n.value, None) == B.INKLING_ERR_INVALID_ARGUMENT
    no_sh = B.Grads(0x1000, 0x1000, 0x1000, None, None)
    assert bw(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, dout, None, dx, ctypes.byref(no_sh), ws,
              n.value, None) == B.INKLING_ERR_INVALID_ARGUMENT
    assert bw(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, dout, None, dx, ctypes.byref(gr), ws,
              n.value - 1, None) == B.INKLING_ERR_WORKSPACE
    # weight gradients are fp32 (the zero default) or bf16; nothing else
    for code in (2, -1):
        odd = B.Grads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, code)
        assert bw(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, dout, None, dx, ctypes.byref(odd),
                  ws, n.value, None) == B.INKLING_ERR_UNSUPPORTED
    bad = _dims(hidden=96)
    assert lib.inkling_moe_backward_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == B.INKLING_ERR_UNSUPPORTED


def test_training_forward_argument_checks(lib):
    """saved_size = (T*top_k + T*n_shared) * 2I fp32 + T*(E+S) fp64; the training forward needs
    its saved buffer and checks its other arguments as the forward does."""
    d = _dims()
    n = ctypes.c_size_t(0)
    assert lib.inkling_moe_saved_size(ctypes.byref(d), ctypes.byref(n)) == B.INKLING_OK
    assert n.value == d.T * (d.top_k + d.n_shared) * 2 * d.intermediate * 4 + d.T * (d.n_routed + d.n_shared) * 8
    assert lib.inkling_moe_saved_size(ctypes.byref(d), None) == B.INKLING_ERR_INVALID_ARGUMENT
    bad = _dims(hidden=96)
    assert lib.inkling_moe_saved_size(ctypes.byref(bad), ctypes.byref(n)) == B.INKLING_ERR_UNSUPPORTED
    nw = ctypes.c_size_t(0)
    lib.inkling_moe_workspace_size(ctypes.byref(d), ctypes.byref(nw))
    gate = B.Gate(0x1000, 0x1000, 1.0, 1.0)
    ex = B.Experts(0x1000, 0x1000, 0x1000, 0x1000)
    x, out, saved, ws = (ctypes.c_void_p(v) for v in (0x4000, 0x5000, 0x6000, 0x7000))
    ft = lib.inkling_moe_forward_train
    assert ft(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, out, None, ws, nw.value,
              None) == B.INKLING_ERR_INVALID_ARGUMENT
    assert ft(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, x, saved, ws, nw.value,
              None) == B.INKLING_ERR_INVALID_ARGUMENT
    assert ft(ctypes.byref(d), x, ctypes.byref(gate), ctypes.byref(ex), None, out, saved, ws, nw.value - 1,
              None) == B.INKLING_ERR_WORKSPACE
    zero = _dims(T=0)
    assert ft(ctypes.byref(zero), None, None, None, None, None, None, None, 0, None) == B.INKLING_OK


def test_largest_token_count_accepted(lib):
    """T * top_k = 2^31 - 257 is the largest accepted slot count (only the size
    query runs; nothing is allocated)."""
    rc, n = _ws(lib, T=2 ** 31 - 257, top_k=1)
    assert rc == B.INKLING_OK and n > 0
    rc, _ = _ws(lib, T=2 ** 31 - 256, top_k=1)
    assert rc == B.INKLING_ERR_UNSUPPORTED


def _noalloc(lib, d):
    gate = B.Gate(None, None, 1.0, 1.0)
    return lib.inkling_moe_forward_noalloc(ctypes.byref(d), None, ctypes.byref(gate), None, None, None, None, None)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+INKLING_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.INKLING_NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """inkling_moe_forward_noalloc returns INKLING_ERR_TOO_LARGE, before any
    HIP call, exactly when the workspace of the same dims exceeds its static
    scratch (the first token count past the limit at the prefill shapes);
    bad dims give the usual codes and T = 0 is a no-op."""
    shape = dict(hidden=6144, n_routed=128, top_k=8, n_shared=2, intermediate=2048)
    cap = B.INKLING_NOALLOC_SCRATCH_BYTES
    lo, hi = 1, 1 << 16
    while lo < hi:   # largest T whose workspace fits
        mid = (lo + hi + 1) // 2
        rc, n = _ws(lib, T=mid, **shape)
        assert rc == B.INKLING_OK
        lo, hi = (mid, hi) if n <= cap else (lo, mid - 1)
    assert 32 < lo < 8192   # decode batches fit, prefill batches do not
    assert _noalloc(lib, _dims(T=lo + 1, **shape)) == B.INKLING_ERR_TOO_LARGE
    assert _noalloc(lib, _dims(T=8192, **shape)) == B.INKLING_ERR_TOO_LARGE
    assert _noalloc(lib, _dims(T=-1)) == B.INKLING_ERR_INVALID_ARGUMENT
    assert _noalloc(lib, _dims(hidden=96)) == B.INKLING_ERR_UNSUPPORTED
    assert _noalloc(lib, _dims(T=0)) == B.INKLING_OK
