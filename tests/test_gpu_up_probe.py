"""GPU parity of the input-sparse up projection probe (sparse_ffn_up_probe) against the
fp64 oracle's pre-activations W_u x (oracle.preact): the row-gather layout for the listed
neurons, and the column-major layout that skips zero inputs and unlisted 16-byte pieces,
on tokens of the ReLU-fied gated shape (x = relu(rmsnorm(z)), about half zeros: novita.ai
activation-sparsity article, section 第二階段). Values to 1e-5 of the row's largest |W_u x|
(fp32 accumulation of at most 4096 products); pieces without a listed neuron exactly 0."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import build, say, to_np

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import activation_sparse_decode_rank_amd  # noqa: F401  (fails loudly without the HIP library)
    torch.cuda.init()
    yield


def _words(idx, n):
    w = np.zeros((n + 63) // 64, np.uint64)
    for i in np.asarray(idx, np.int64):
        w[i // 64] |= np.uint64(1) << np.uint64(i % 64)
    return torch.from_numpy(w.view(np.int64)).cuda()


def _probe(w_rows, x, idx):
    """Both layouts through the C ABI; returns (u_rows[:count], u_cols[n])."""
    from activation_sparse_decode_rank_amd import _native as N
    n, d = w_rows.shape
    w_cols = w_rows.t().contiguous()
    idx_d = torch.as_tensor(np.asarray(idx, np.int32), device="cuda")
    if idx_d.numel() == 0:
        idx_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    cnt = torch.tensor([len(idx)], dtype=torch.int32, device="cuda")
    words = _words(idx, n)
    u_r = torch.full((n,), float("nan"), device="cuda")
    u_c = torch.full((n,), float("nan"), device="cuda")
    wb = N.sparse_ffn_up_probe_work_bytes(n)
    work = torch.empty(wb // 4, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    N.sparse_ffn_up_probe(w_rows.data_ptr(), N.SFFN_UP_ROWS, d, n, x.data_ptr(), idx_d.data_ptr(),
                          cnt.data_ptr(), None, u_r.data_ptr(), None, 0, st)
    N.sparse_ffn_up_probe(w_cols.data_ptr(), N.SFFN_UP_COLUMNS, d, n, x.data_ptr(), None, None,
                          words.data_ptr(), u_c.data_ptr(), work.data_ptr(), wb, st)
    torch.cuda.synchronize()
    return to_np(u_r)[:len(idx)], to_np(u_c)


def _check(w_rows, x, idx):
    n = w_rows.shape[0]
    U = oracle.preact(to_np(x)[None, :], to_np(w_rows), None)[0]
    scale = max(float(np.max(np.abs(U))), 1e-30)
    u_r, u_c = _probe(w_rows, x, idx)
    idx = np.asarray(idx, np.int64)
    if len(idx):
        assert float(np.max(np.abs(u_r - U[idx]))) <= TOL * scale
    live = np.zeros(n // 8, bool)
    live[idx // 8] = True
    live_n = np.repeat(live, 8)
    assert np.all(u_c[~live_n] == 0.0)
    if live.any():
        assert float(np.max(np.abs(u_c[live_n] - U[live_n]))) <= TOL * scale
    return float((to_np(x) == 0).mean())


@pytest.mark.parametrize("d,n,frac", [(512, 1104, 0.1), (1024, 2048, 0.0), (512, 1104, 1.0),
                                      (8192, 1104, 0.1), (16384, 520, 0.3),
                                      (4096, 11008, 0.1)])
def test_up_probe_matches_oracle(d, n, frac):
    from synth import get_config, make_layer, make_tokens
    c = get_config("C3")
    say(f"up probe d={d} n={n} listed={frac}")
    Lt = make_layer(c, 0, "cuda", d=d, n=n)
    w = Lt.w_u.contiguous()
    x = make_tokens(c, 1, 600, "cuda", d=d)[0].contiguous()
    rng = np.random.Generator(np.random.PCG64(61))
    idx = np.sort(rng.choice(n, int(round(frac * n)), replace=False))
    zeros = _check(w, x, idx)
    say(f"  listed={len(idx)} zero inputs={zeros:.3f}")
    assert 0.3 < zeros < 0.7


def test_up_probe_on_decode_list():
    """The full gated Llama-7B-shaped layer, packed hot-first, with the list the decode step
    publishes for a token: the two layouts agree with the oracle on the packed rows."""
    from synth import get_config, make_tokens
    c = get_config("C3")
    say("up probe on a decode list, full C3 layer")
    s, L, Lt = build(c, 0, max_batch=1, profile_tokens=512)
    x = make_tokens(c, 1, 601, "cuda")
    _, idx, count, _ = s.decode(x)
    torch.cuda.synchronize()
    k = int(count.item())
    perm = torch.as_tensor(s.perm, device="cuda").long()
    w_packed = Lt.w_u.index_select(0, perm).contiguous()
    _check(w_packed, x[0].contiguous(), to_np(idx)[:k])
