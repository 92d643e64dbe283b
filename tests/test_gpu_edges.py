"""GPU parity on the branches the workload shapes do not reach: every neuron active in
layers long enough that one down-projection split holds more rows than its LDS list window
(single-token and vector small-batch paths), the matrix-core fallbacks that compact in two
passes (predictor rank too large for the score kernel's LDS; more than 65536 neurons), a
decode that asks for no token bits, and large-magnitude inputs on the matrix-core path.

With every neuron active the sparse output must equal the dense FFN (novita.ai
activation-sparsity article, section 激活稀疏性的可行性: only rows whose ReLU output is zero
are skipped, so listing every row computes the dense layer). Index lists, counts and token
bits are compared bit for bit; outputs to max |y - y_ref| / max |y_ref| <= 1e-3 per token."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import REL_TOL, build, check_mask, gpu_mask_orig, rel_err_rows, say, to_np

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


def _all_active_decode(name, d, n, r, B, deterministic, activity=None):
    c = cfg(name)
    s, L, _ = build(c, 0, d=d, n=n, rank=r, max_batch=B, threshold=float("-inf"),
                    deterministic=deterministic, activity=activity)
    X = tokens(c, B, d)
    y, idx, count, tok = s.decode(X)
    torch.cuda.synchronize()
    k = int(count.item())
    assert k == n
    assert np.array_equal(to_np(idx)[:n], np.arange(n, dtype=np.int32))
    full = np.uint64((1 << B) - 1) if B < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
    assert np.all(to_np(tok)[:n].astype(np.uint64) == full)
    Xh = to_np(X)
    D = oracle.dense(Xh, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(to_np(y), D)
    say(f"  count={k} err={max(errs):.2e}")
    assert max(errs) <= REL_TOL, errs
    return s


def test_single_token_long_split_deterministic():
    """One token, every neuron active, deterministic mode: the down projection keeps two
    row splits of 10000 rows each, past its 8192-entry list window, so every split takes
    the windowed branch that publishes the list window by window."""
    say("long split, one token, deterministic: d=512 n=20000")
    s = _all_active_decode("C2", 512, 20000, 64, 1, True)
    assert s.deterministic


def test_single_token_long_split_fast_mode():
    """One token, every neuron active, fast mode, d = 4096: four row splits of 9000 rows
    (the profile expects 2% activity, so no extra splits are cut), each past the window."""
    say("long split, one token, fast mode: d=4096 n=36000")
    _all_active_decode("C2", 4096, 36000, 256, 1, False, activity=0.02)


@pytest.mark.parametrize("name,d", [("C1", 512), ("C2", 520)])
def test_vector_batch_window_all_active(name, d):
    """Four tokens on the vector path (fp32 weights, or fp16 with d not a multiple of 256),
    every neuron active, deterministic mode: two row splits of 10000 rows, so the vector
    down projection expands and publishes its list in windows."""
    say(f"vector window, 4 tokens: {name} d={d} n=20000")
    _all_active_decode(name, d, 20000, 64, 4, True)


def _decode_raw(s, X, tokmask=True, scores=None):
    """sparse_ffn_decode through the C ABI, tokmask optionally NULL."""
    from activation_sparse_decode_rank_amd import _native as N
    B = X.shape[0]
    y = torch.empty((B, s.d), dtype=torch.float32, device="cuda")
    idx = torch.empty(s.n, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    tok = torch.empty(s.n, dtype=torch.int64, device="cuda") if tokmask else None
    N.sparse_ffn_decode(s.handle, X.data_ptr(), B, y.data_ptr(), idx.data_ptr(), cnt.data_ptr(),
                        None if tok is None else tok.data_ptr(),
                        None if scores is None else scores.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    k = int(cnt.item())
    return to_np(y), to_np(idx)[:k], (to_np(tok)[:k] if tok is not None else None), k


@pytest.mark.parametrize("name,d,n,r,B", [
    ("C5", 1024, 2100, 1024, 4),   # rank 1024: q does not fit the score kernel's LDS
    ("C2", 256, 70000, 64, 4),     # 1094 union words: more than the up kernel lists itself
    ("C3", 512, 67000, 64, 3),     # the same fallback, gated
])
def test_tile_fallbacks(name, d, n, r, B):
    """The matrix-core path's two-pass compaction: scores into the caller's buffer or, with
    none given, into the workspace's activation buffer (which the up projection overwrites
    only after compaction has read it), then the list, then the up tile kernel reading it.
    Run with and without scores and with and without a token mask: lists bit-exact with the
    oracle's compaction of the predict entry point's scores (the same arithmetic), y equal
    bitwise across the four calls (deterministic mode) and within tolerance of the oracle."""
    c = cfg(name)
    say(f"tile fallback {name} d={d} n={n} r={r} B={B}")
    s, L, _ = build(c, 0, d=d, n=n, rank=r, max_batch=B, deterministic=True)
    X = tokens(c, B, d)
    Sg = to_np(s.predict(X))
    ri, rk, rt = oracle.compact(oracle.threshold(Sg.astype(np.float32), 0.0))
    sc = torch.empty((B, n), dtype=torch.float32, device="cuda")
    runs = []
    for want_tok, scores in [(True, None), (False, None), (True, sc), (False, sc)]:
        y, idx, tok, k = _decode_raw(s, X, tokmask=want_tok, scores=scores)
        assert k == rk
        assert np.array_equal(idx, ri)
        assert np.all(np.diff(idx) > 0)
        if tok is not None:
            assert np.array_equal(tok.astype(np.uint64), rt)
        if scores is not None:
            assert np.array_equal(to_np(scores), Sg)
        runs.append(y)
    for y in runs[1:]:
        assert np.array_equal(y, runs[0])
    Xh = to_np(X)
    S = oracle.predict(Xh, L["p1"], L["p2"], L["c"])
    Mg = gpu_mask_orig(s.perm, ri, rk, rt, B, n)
    M, nband = check_mask(Mg, S)
    oi, _, ot = oracle.compact(M)
    Y = oracle.forward(Xh, L["w_a"], L["w_o"], oi, ot, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(runs[0], Y)
    say(f"  count={rk} band={nband} err={max(errs):.2e}")
    assert max(errs) <= REL_TOL, errs


@pytest.mark.parametrize("B", [1, 4, 16])
def test_decode_without_token_mask(B):
    """tokmask = NULL is allowed at every batch size: the list and y equal those of the same
    decode with a mask (single-token, matrix-core listing-in-up-kernel paths)."""
    c = cfg("C3")
    say(f"decode without token mask B={B}")
    s, _, _ = build(c, 0, d=512, n=1100, rank=64, max_batch=B, deterministic=True)
    X = tokens(c, B, 512)
    y1, i1, t1, k1 = _decode_raw(s, X, tokmask=True)
    y2, i2, t2, k2 = _decode_raw(s, X, tokmask=False)
    assert k1 == k2 and np.array_equal(i1, i2) and np.array_equal(y1, y2)


@pytest.mark.parametrize("scale", [30.0, 100.0])
def test_tile_path_large_magnitude(scale):
    """Tokens scaled up (|x| to a few hundred, |h| to thousands) on the matrix-core path,
    where fp32 values travel as fp16 hi + lo pairs: still within tolerance while every |x|
    and |h| stays below the fp16 range (the header states the limit)."""
    c = cfg("C3")
    B, d, n = 4, 512, 1100
    say(f"large magnitude x{scale}")
    s, L, _ = build(c, 0, d=d, n=n, rank=64, max_batch=B)
    X = (tokens(c, B, d) * scale).contiguous()
    y, idx, count, tok = s.decode(X)
    torch.cuda.synchronize()
    k = int(count.item())
    Xh = to_np(X)
    S = oracle.predict(Xh, L["p1"], L["p2"], L["c"])
    Mg = gpu_mask_orig(s.perm, to_np(idx), k, to_np(tok), B, n)
    M, _ = check_mask(Mg, S)
    ri, _, rt = oracle.compact(M)
    Y = oracle.forward(Xh, L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    A = oracle.preact(Xh, L["w_a"], L["b_a"])
    U = oracle.preact(Xh, L["w_u"], None)
    hmax = float(np.max(np.abs(np.maximum(A, 0) * U)))
    assert hmax < 65504 and np.max(np.abs(Xh)) < 65504
    errs = rel_err_rows(to_np(y), Y)
    say(f"  count={k} max|h|={hmax:.1f} err={max(errs):.2e}")
    assert np.all(np.isfinite(to_np(y)))
    assert max(errs) <= REL_TOL, errs
