"""GPU parity of the matrix-core prefill (sparse_ffn_prefill) against the fp64 oracle's dense
FFN (oracle.dense): every neuron for many tokens, the pages' dense prefill (PowerInfer-2
article, section 4.1.1 NPU-Centric Prefill). Ragged token counts and neuron counts, plain
and gated, split and bundle layouts, several chunks, the full gated Llama-7B layer at 512
tokens (sampled tokens against the oracle). y within 1e-3 of max|y| per token (reading of
the fp32 accumulation bound), bitwise equal from run to run."""

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


def _prefill(s, X, chunk):
    work = s.prefill_work(chunk)
    assert work is not None
    y1 = s.prefill(X, work=work)
    y2 = s.prefill(X, work=work)
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
