"""GPU parity of the dense route (every neuron, no predictor): sparse_ffn_dense for any number
of tokens (prefill, in chunks of the workspace's batch), and the decode step's switch to it
above the union crossover, against the fp64 oracle's dense FFN.

PowerInfer-2 runs prefill dense (PowerInfer-2 article, section 4.1.1 NPU-Centric Prefill), and
the benefit of sparsity shrinks as a batch's union of active sets grows (novita.ai
activation-sparsity article, section 批次大小影響). Outputs to max |y - y_ref| / max |y_ref|
<= 1e-3 per token; lists bit for bit."""
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


def tokens(c, B, d, tag=200):
    from synth import make_tokens
    return make_tokens(c, B, tag, "cuda", d=d)


@pytest.mark.parametrize("name,d,n,r,mb,B", [
    ("C3", 512, 1100, 64, 16, 1),     # one token
    ("C3", 512, 1100, 64, 16, 16),    # matrix-core tiles, one chunk
    ("C3", 512, 1100, 64, 16, 40),    # three chunks, the last ragged
    ("C2", 256, 700, 64, 64, 200),    # prefill of 200 tokens in chunks of 64
    ("C2", 1024, 2000, 128, 64, 64),  # four token tiles
    ("C1", 768, 3072, 64, 8, 21),     # fp32 weights: the vector path, chunks of 8
    ("C2", 520, 900, 64, 4, 9),       # d not a multiple of 256: the vector path
    ("C2", 512, 1000, 64, 1, 3),      # a single-token workspace: one token at a time
])
@pytest.mark.parametrize("bundle", [False, True])
def test_dense_route_matches_oracle(name, d, n, r, mb, B, bundle):
    c = cfg(name)
    say(f"dense route {name} d={d} n={n} max_batch={mb} B={B} bundle={bundle}")
    s, L, _ = build(c, 0, d=d, n=n, rank=r, max_batch=mb, bundle=bundle)
    X = tokens(c, B, d)
    y = to_np(s.dense(X))
    torch.cuda.synchronize()
    D = oracle.dense(to_np(X), L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(y, D)
    say(f"  err={max(errs):.2e}")
    assert max(errs) <= REL_TOL, errs


def test_decode_switches_to_dense_above_crossover():
    """With dense_union = 0.5, decode stays sparse up to the batch size whose expected union
    (from the profile frequencies) first exceeds one half, and from there computes every
    neuron: list = all neurons with every token's bit, y = the dense FFN."""
    c = cfg("C3")
    d, n, r, mb = 512, 1100, 64, 32
    say("decode crossover to the dense route")
    s, L, _ = build(c, 0, d=d, n=n, rank=r, max_batch=mb)
    f = np.clip(s._freq.astype(np.float64), 0.0, 1.0)
    union = [1.0 - np.mean((1.0 - f) ** b) for b in range(1, mb + 1)]
    b_cross = next((b for b in range(1, mb + 1) if union[b - 1] > 0.5), None)
    assert b_cross is not None and b_cross > 1, union
    sw = s.clone(dense_union=0.5)
    for B in (b_cross - 1, b_cross, mb):
        X = tokens(c, B, d, tag=600 + B)
        y, idx, count, tok = sw.decode(X)
        torch.cuda.synchronize()
        k = int(count.item())
        Xh = to_np(X)
        if B < b_cross:
            y0, i0, c0, t0 = s.decode(X)
            torch.cuda.synchronize()
            assert k == int(c0.item()) and np.array_equal(to_np(idx)[:k], to_np(i0)[:k])
            assert max(rel_err_rows(to_np(y), to_np(y0))) <= 1e-5
            assert k < n
        else:
            full = np.uint64((1 << B) - 1) if B < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
            assert k == n and np.array_equal(to_np(idx)[:n], np.arange(n, dtype=np.int32))
            assert np.all(to_np(tok)[:n].astype(np.uint64) == full)
            D = oracle.dense(Xh, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
            assert max(rel_err_rows(to_np(y), D)) <= REL_TOL
        say(f"  B={B} count={k} (crossover at {b_cross})")


def test_dense_rejects():
    from activation_sparse_decode_rank_amd import _native as N
    c = cfg("C2")
    s, _, _ = build(c, 0, d=256, n=300, rank=64, max_batch=2)
    L = N.lib()
    x = torch.zeros((4, 256), device="cuda")
    y = torch.zeros((4, 256), device="cuda")
    assert L.sparse_ffn_dense(s.handle, x.data_ptr(), 0, y.data_ptr(), None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_dense(None, x.data_ptr(), 1, y.data_ptr(), None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_dense(s.handle, x.data_ptr() + 4, 1, y.data_ptr(), None) == N.SFFN_ERR_INVALID
