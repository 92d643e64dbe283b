"""GPU parity of the matrix-core prefill (sparse_ffn_prefill) against the fp64 oracle's dense
FFN (oracle.dense): every neuron for many tokens, the pages' dense prefill (PowerInfer-2
article, section 4.1.1 NPU-Centric Prefill). Ragged token counts and neuron counts, plain
and gated, split and bundle layouts, several chunks, the full gated Llama-7B layer at 512
tokens (sampled tokens against the oracle). y within 1e-3 of max|y| per token (reading of
the fp32 accumulation bound), bitwise equal from run to run.

The fp16-activation form (SFFN_PREFILL_FP16_ACT) rounds x and h to fp16 once: it is checked
against the oracle's fp16-activation FFN (oracle.dense_f16act, the same two roundings; the
same 1e-3 reading), and against the exact FFN within the first-order bound those roundings
allow."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import REL_TOL, build, rel_err_rows, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import activation_sparse_decode_rank_amd  # noqa: F401  (fails loudly without the HIP library)
    torch.cuda.init()
    yield


def cfg(name):
    from synth import get_config
    return get_config(name)


def _prefill(s, X, chunk, fp16_act=False):
    work = s.prefill_work(chunk)
    assert work is not None
    y1 = s.prefill(X, work=work, fp16_activations=fp16_act)
    y2 = s.prefill(X, work=work, fp16_activations=fp16_act)
    torch.cuda.synchronize()
    a, b = to_np(y1), to_np(y2)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    return a


@pytest.mark.parametrize("name,d,n,B,chunk,bundle", [
    ("C3", 512, 1100, 1, 128, False),     # one token, ragged neuron count
    ("C3", 512, 1100, 130, 128, False),   # two chunks, the last of 2 tokens
    ("C2", 1024, 2000, 300, 256, False),  # plain, two chunks of 256
    ("C3", 1024, 1408, 257, 512, True),   # gated bundle layout, one chunk
    ("C2", 256, 700, 64, 128, True),      # plain bundle
    ("C3", 2048, 3000, 384, 384, False),  # split down projection (few output tiles)
    ("C2", 512, 8192, 512, 512, False),   # plain, 128-neuron tiles (64 elsewhere at these sizes)
])
def test_prefill_matches_oracle(name, d, n, B, chunk, bundle):
    c = cfg(name)
    say(f"prefill {name} d={d} n={n} B={B} chunk={chunk} bundle={bundle}")
    s, L, _ = build(c, 0, d=d, n=n, rank=64, max_batch=4, bundle=bundle)
    from synth import make_tokens
    X = make_tokens(c, B, 520, "cuda", d=d)
    y = _prefill(s, X, chunk)
    Xh = to_np(X)
    Y = oracle.dense(Xh, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(y, Y)
    say(f"  err={max(errs):.2e}")
    assert max(errs) <= REL_TOL, max(errs)
    # the decode kernels' dense route gives the same FFN to rounding
    yd = to_np(s.dense(X))
    assert max(rel_err_rows(y, yd)) <= 1e-5


@pytest.mark.parametrize("name,d,n,gated", [("C2", 512, 9000, False), ("C3", 512, 9000, True)])
def test_prefill_192_neuron_tiles(name, d, n, gated):
    """512 tokens over 9000 neurons: 192-neuron tiles finish in one round where 128-neuron
    tiles take two, so the up kernel takes its 192-row form (plain and gated); eight sampled
    tokens against the oracle."""
    c = cfg(name)
    say(f"prefill 192-neuron tiles {name} d={d} n={n}")
    s, L, _ = build(c, 0, d=d, n=n, rank=64, max_batch=4)
    from synth import make_tokens
    X = make_tokens(c, 512, 522, "cuda", d=d)
    y = _prefill(s, X, 512)
    sel = [0, 5, 127, 128, 300, 383, 384, 511]
    Xh = to_np(X)[sel]
    Y = oracle.dense(Xh, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(y[sel], Y)
    say(f"  err={max(errs):.2e}")
    assert max(errs) <= REL_TOL, max(errs)


def test_prefill_full_size_gated():
    """The full Llama-7B-shaped gated layer (d 4096, d_ffn 11008) at 512 tokens in one chunk:
    four sampled tokens against the oracle."""
    c = cfg("C3")
    say("prefill full C3 layer, 512 tokens")
    s, L, _ = build(c, 0, max_batch=4, profile_tokens=256)
    from synth import make_tokens
    X = make_tokens(c, 512, 521, "cuda")
    y = _prefill(s, X, 512)
    sel = [0, 1, 255, 511]
    Xh = to_np(X)[sel]
    Y = oracle.dense(Xh, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(y[sel], Y)
    say(f"  err={max(errs):.2e}")
    assert max(errs) <= REL_TOL, max(errs)


def test_prefill_full_size_opt175b_slice():
    """The full OPT-175B-shaped slice (d 12288, d_ffn 49152, plain) at 256 tokens in one
    chunk: 96 output column tiles, two token tiles, the down projection split; three sampled
    tokens against the oracle."""
    c = cfg("C5")
    say("prefill full C5 slice, 256 tokens")
    s, L, _ = build(c, 0, max_batch=4, profile_tokens=256)
    from synth import make_tokens
    X = make_tokens(c, 256, 522, "cuda")
    y = _prefill(s, X, 256)
    sel = [0, 130, 255]
    Xh = to_np(X)[sel]
    Y = oracle.dense(Xh, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(y[sel], Y)
    say(f"  err={max(errs):.2e}")
    assert max(errs) <= REL_TOL, max(errs)


def test_prefill_rejects():
    """fp32 weights have no matrix-core prefill (SFFN_ERR_UNSUPPORTED; the Python layer then
    takes the dense route); scratch below one 128-token chunk is refused."""
    from activation_sparse_decode_rank_amd import _native as N
    say("prefill argument checks")
    s32, _, _ = build(cfg("C1"), 0, d=256, n=600, rank=64)
    assert N.sparse_ffn_prefill_work_bytes(s32.handle, 128) == 0
    X = torch.zeros((4, 256), dtype=torch.float32, device="cuda")
    y = torch.empty_like(X)
    work = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    L = N.lib()
    assert L.sparse_ffn_prefill(s32.handle, X.data_ptr(), 4, y.data_ptr(), work.data_ptr(),
                                work.numel(), None) == N.SFFN_ERR_UNSUPPORTED
    s16, _, _ = build(cfg("C2"), 0, d=512, n=1000, rank=64)
    need = N.sparse_ffn_prefill_work_bytes(s16.handle, 128)
    assert need > 0
    X = torch.zeros((4, 512), dtype=torch.float32, device="cuda")
    y = torch.empty_like(X)
    assert L.sparse_ffn_prefill(s16.handle, X.data_ptr(), 4, y.data_ptr(), work.data_ptr(),
                                need - 256, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_prefill(s16.handle, X.data_ptr(), 0, y.data_ptr(), work.data_ptr(),
                                need, None) == N.SFFN_ERR_INVALID
    yf = s32.prefill(torch.zeros((3, 256), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert yf.shape == (3, 256)


U16 = 2.0 ** -11  # unit roundoff of round-to-nearest fp16 (normal range)


def _f16act_bound(X, L):
    """First-order bound on |y - FFN(x)| that the two roundings of the fp16-activation
    prefill allow (x before the up products, h before the down product; worst-case signs):
    u (sum_k |W_o[k]| (dh_k + |h_k|)) with dh_k <= u A_k, A_k = |W_a[k]| . |x| (plain), or
    |W_g[k]| . |x| |v_k| + relu(g_k) |W_u[k]| . |x| (gated, v = W_u x); all from the exact
    quantities, in fp64."""
    X = np.asarray(X, np.float64)
    Wa = np.asarray(L["w_a"], np.float64)
    Wo = np.asarray(L["w_o"], np.float64)
    Wu = None if L["w_u"] is None else np.asarray(L["w_u"], np.float64)
    ba = 0.0 if L["b_a"] is None else np.asarray(L["b_a"], np.float64)
    ax = np.abs(X)
    ge = X @ Wa.T + ba
    he = np.maximum(ge, 0.0)
    A = ax @ np.abs(Wa).T
    if Wu is not None:
        ve = X @ Wu.T
        A = A * np.abs(ve) + he * (ax @ np.abs(Wu).T)
        he = he * ve
    return U16 * (A + np.abs(he)) @ np.abs(Wo)


def _oracle_f16act(X, L):
    return oracle.dense_f16act(X, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])


@pytest.mark.parametrize("name,d,n,B,chunk,bundle", [
    ("C3", 512, 1100, 130, 128, False),   # gated, two chunks, the last of 2 tokens
    ("C2", 1024, 2000, 300, 256, False),  # plain, two chunks of 256
    ("C3", 1024, 1408, 257, 512, True),   # gated bundle layout, one chunk
    ("C2", 512, 9000, 512, 512, False),   # 192-neuron tiles
    ("C3", 2048, 3000, 384, 384, False),  # split down projection
])
def test_prefill_fp16_act(name, d, n, B, chunk, bundle):
    c = cfg(name)
    say(f"prefill fp16 activations {name} d={d} n={n} B={B} chunk={chunk} bundle={bundle}")
    s, L, _ = build(c, 0, d=d, n=n, rank=64, max_batch=4, bundle=bundle)
    from synth import make_tokens
    X = make_tokens(c, B, 523, "cuda", d=d)
    y = _prefill(s, X, chunk, fp16_act=True)
    sel = sorted(set([0, 1, B // 2, B - 1] + list(range(0, B, max(1, B // 8)))))
    Xh = to_np(X)[sel]
    R, bound = _oracle_f16act(Xh, L), _f16act_bound(Xh, L)
    errs = rel_err_rows(y[sel], R)
    say(f"  err vs the oracle's fp16-activation FFN={max(errs):.2e}")
    assert max(errs) <= REL_TOL, max(errs)
    Y = oracle.dense(Xh, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    scale = np.max(np.abs(Y), axis=1, keepdims=True)
    excess = np.abs(y[sel] - Y) - (2.0 * bound + REL_TOL * scale)
    say(f"  err vs exact={max(rel_err_rows(y[sel], Y)):.2e}, worst margin={excess.max():.2e}")
    assert np.all(excess <= 0.0)
    # the fp32-activation form is closer to the exact FFN than this one's bound
    y32 = _prefill(s, X, chunk)
    assert max(rel_err_rows(y32[sel], Y)) <= REL_TOL


def test_prefill_fp16_act_full_size_gated():
    """The full Llama-7B-shaped gated layer at 512 tokens with fp16 activations: sampled
    tokens against the oracle's fp16-activation FFN."""
    c = cfg("C3")
    say("prefill fp16 activations, full C3 layer, 512 tokens")
    s, L, _ = build(c, 0, max_batch=4, profile_tokens=256)
    from synth import make_tokens
    X = make_tokens(c, 512, 524, "cuda")
    y = _prefill(s, X, 512, fp16_act=True)
    sel = [0, 100, 255, 511]
    R = _oracle_f16act(to_np(X)[sel], L)
    errs = rel_err_rows(y[sel], R)
    say(f"  err={max(errs):.2e}")
    assert max(errs) <= REL_TOL, max(errs)


def test_prefill_ex_flags():
    """Unknown flag bits are refused; flags 0 is sparse_ffn_prefill itself, bit for bit."""
    from activation_sparse_decode_rank_amd import _native as N
    say("prefill_ex flags")
    s, _, _ = build(cfg("C2"), 0, d=512, n=1000, rank=64)
    need = N.sparse_ffn_prefill_work_bytes(s.handle, 128)
    work = torch.empty(need, dtype=torch.uint8, device="cuda")
    from synth import make_tokens
    X = make_tokens(cfg("C2"), 5, 525, "cuda", d=512)
    y0 = torch.empty_like(X)
    y1 = torch.empty_like(X)
    L = N.lib()
    for bad in (2, 4, -1, 1 << 30):
        assert L.sparse_ffn_prefill_ex(s.handle, X.data_ptr(), 5, y0.data_ptr(), work.data_ptr(),
                                       need, bad, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_prefill_ex(s.handle, X.data_ptr(), 5, y0.data_ptr(), work.data_ptr(),
                                   need, 0, None) == N.SFFN_OK
    assert L.sparse_ffn_prefill(s.handle, X.data_ptr(), 5, y1.data_ptr(), work.data_ptr(),
                                need, None) == N.SFFN_OK
    torch.cuda.synchronize()
    assert np.array_equal(to_np(y0).view(np.uint32), to_np(y1).view(np.uint32))
