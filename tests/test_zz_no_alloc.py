"""sparse_ffn_decode_static (the decode step over the library's static per-device scratch
array, for callers that cannot allocate) against sparse_ffn_decode (the same step over the
handle's workspace), through the C ABI: two calls in a row, the second with a smaller
input; a handle created without any workspace; graph capture and replay; and the size
limit. Deterministic handles, so lists, counts, token bits and y must be equal bit for bit
(the tolerance of the oracle comparison, 1e-3, is then met trivially)."""
import ctypes as C

import numpy as np
import pytest
import torch

from gpu_util import build, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import activation_sparse_decode_rank_amd  # noqa: F401  (fails loudly without the HIP library)
    torch.cuda.init()
    yield


def cfg(name):
    from synth import get_config
    return get_config(name)


def tokens(c, B, d, tag=200):
    from synth import make_tokens
    return make_tokens(c, B, tag, "cuda", d=d)


def _static(s_handle, n, d, X, with_tok=True, scores=None, stream=None):
    from activation_sparse_decode_rank_amd import _native as N
    B = X.shape[0]
    y = torch.full((B, d), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    tok = torch.zeros(n, dtype=torch.int64, device="cuda") if with_tok else None
    st = (stream or torch.cuda.current_stream()).cuda_stream
    N.sparse_ffn_decode_static(s_handle, X.data_ptr(), B, y.data_ptr(), idx.data_ptr(),
                               cnt.data_ptr(), None if tok is None else tok.data_ptr(),
                               None if scores is None else scores.data_ptr(), st)
    return y, idx, cnt, tok


def _same(ref, got, with_tok=True):
    y_r, i_r, c_r, t_r = ref
    y_g, i_g, c_g, t_g = got
    torch.cuda.synchronize()
    k = int(c_r.item())
    assert int(c_g.item()) == k
    assert np.array_equal(to_np(i_g)[:k], to_np(i_r)[:k])
    if with_tok:
        assert np.array_equal(to_np(t_g)[:k], to_np(t_r)[:k])
    assert np.array_equal(to_np(y_g), to_np(y_r))
    return k


@pytest.mark.parametrize("name,d,n,r,B1,B2", [
    ("C2", 1024, 3000, 128, 1, 1),    # single token, then a smaller layer (below)
    ("C3", 512, 1100, 64, 8, 2),      # matrix-core tiles, 8 then 2 tokens
    ("C3", 1024, 2500, 128, 24, 3),   # stream-K up kernel and its counters, then 3 tokens
    ("C1", 768, 3072, 64, 5, 4),      # vector small-batch path (fp32 weights)
])
def test_static_equals_workspace_decode(name, d, n, r, B1, B2):
    c = cfg(name)
    say(f"static decode {name} d={d} n={n} r={r} B={B1} then {B2}")
    s, _, _ = build(c, 0, d=d, n=n, rank=r, max_batch=max(B1, B2), deterministic=True)
    # a second, smaller layer whose call follows on the same device array
    s2, _, _ = build(c, 1, d=d, n=n // 2 + 8, rank=r, max_batch=B2, deterministic=True)
    X1 = tokens(c, B1, d, tag=410)
    X2 = tokens(c, B2, d, tag=411)
    ref1 = [t.clone() for t in s.decode(X1)]
    ref2 = [t.clone() for t in s2.decode(X2)]
    torch.cuda.synchronize()
    k1 = _same(ref1, _static(s.handle, s.n, d, X1))
    k2 = _same(ref2, _static(s2.handle, s2.n, d, X2))
    # and back to the first layer, whose range table the second call overwrote
    k3 = _same(ref1, _static(s.handle, s.n, d, X1))
    say(f"  counts {k1} {k2} {k3}")
    assert k1 == k3


def test_static_handle_without_workspace():
    """A handle created with workspace NULL: the static decode runs on it and equals the
    workspace decode of an ordinary handle over the same weights; every workspace entry
    point rejects it."""
    from activation_sparse_decode_rank_amd import _native as N
    c = cfg("C3")
    B, d = 4, 512
    say("static decode, handle without workspace")
    s, _, _ = build(c, 0, d=d, n=1100, rank=64, max_batch=B, deterministic=True)
    D = N.SffnDesc()
    C.memmove(C.byref(D), C.byref(s.desc), C.sizeof(N.SffnDesc))
    D.workspace, D.workspace_bytes, D.neuron_freq = None, 0, s._freq.ctypes.data
    h = N.sparse_ffn_create(D)
    try:
        X = tokens(c, B, d, tag=412)
        ref = [t.clone() for t in s.decode(X)]
        _same(ref, _static(h, s.n, d, X))
        _same(ref, _static(h, s.n, d, X, with_tok=False), with_tok=False)
        L = N.lib()
        y = torch.empty((B, d), device="cuda")
        idx = torch.empty(s.n, dtype=torch.int32, device="cuda")
        cnt = torch.empty(1, dtype=torch.int32, device="cuda")
        rc = L.sparse_ffn_decode(h, X.data_ptr(), B, y.data_ptr(), idx.data_ptr(), cnt.data_ptr(),
                                 None, None, None)
        assert rc == N.SFFN_ERR_INVALID
        rc = L.sparse_ffn_predict(h, X.data_ptr(), B, y.data_ptr(), None)
        assert rc == N.SFFN_ERR_INVALID
    finally:
        N.sparse_ffn_destroy(h)


def test_static_graph_replay():
    """The static decode captured in a HIP graph and replayed three times, with eager static
    decodes of other tokens (which overwrite the shared array) in between: every replay
    equals the eager workspace decode bitwise."""
    c = cfg("C3")
    B, d = 24, 1024
    say("static decode under graph capture")
    s, _, _ = build(c, 0, d=d, n=2500, rank=128, max_batch=B, deterministic=True)
    X = tokens(c, B, d, tag=413)
    other = tokens(c, B, d, tag=414)
    ref = [t.clone() for t in s.decode(X)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        out = _static(s.handle, s.n, d, X, stream=side)
    for rep in range(3):
        out[0].fill_(float("nan"))
        out[1].fill_(-7)
        g.replay()
        _same(ref, out)
        _static(s.handle, s.n, d, other)
        torch.cuda.synchronize()


def test_static_rejects_too_large():
    """A call needing more scratch than the array holds is refused with its own status
    before anything is enqueued (an OPT-175B-shaped layer at 64 tokens needs 19.7 MiB). The
    buffers are real allocations of the full size, uninitialised."""
    from activation_sparse_decode_rank_amd import _native as N
    say("static decode size limit")
    d, n, r, B = 12288, 49152, 1024, 64
    f16 = dict(dtype=torch.float16, device="cuda")
    w_a = torch.empty((n, d), **f16)
    w_o = torch.empty((n, d), **f16)
    p1 = torch.empty((r, d), **f16)
    p2 = torch.empty((n, r), **f16)
    D = N.SffnDesc()
    D.d, D.d_ffn, D.rank, D.max_batch = d, n, r, B
    D.w_dtype = D.p_dtype = N.SFFN_F16
    D.deterministic = 1
    D.w_act, D.w_down_t, D.p1, D.p2 = w_a.data_ptr(), w_o.data_ptr(), p1.data_ptr(), p2.data_ptr()
    D.workspace, D.workspace_bytes = None, 0
    assert N.sparse_ffn_workspace_bytes(D) > N.SFFN_STATIC_SCRATCH_BYTES
    h = N.sparse_ffn_create(D)
    try:
        X = torch.zeros((B, d), dtype=torch.float32, device="cuda")
        y = torch.empty((B, d), dtype=torch.float32, device="cuda")
        idx = torch.empty(n, dtype=torch.int32, device="cuda")
        cnt = torch.empty(1, dtype=torch.int32, device="cuda")
        rc = N.lib().sparse_ffn_decode_static(h, X.data_ptr(), B, y.data_ptr(), idx.data_ptr(),
                                              cnt.data_ptr(), None, None, None)
        assert rc == N.SFFN_ERR_TOO_LARGE
        assert "static scratch" in N.sparse_ffn_status_string(rc)
    finally:
        N.sparse_ffn_destroy(h)
