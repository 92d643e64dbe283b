"""y bitwise reproducible in the library's default mode at the full workload shapes.

The down projections split the active rows between workgroups; in the default
(deterministic) mode two splits add into a zeroed y (exact in either order) and more meet
in a last-arrival join that adds the splits' sums in split order. Each test decodes the
same tokens twice with a decode of other tokens in between (which leaves other sums in the
join's slots), and requires y, the list, the count and the token bits to be identical bit
for bit; it also checks that y stays within fp32 rounding of the fast mode's (float
atomics) and, once, within tolerance of the oracle (sampled tokens, own masks)."""

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


def _twice(s, X, other):
    outs = []
    for t in (X, other, X):
        y, idx, count, tok = s.decode(t)
        torch.cuda.synchronize()
        k = int(count.item())
        outs.append((to_np(y).copy(), to_np(idx)[:k].copy(), k, to_np(tok)[:k].copy()))
    a, b = outs[0], outs[2]
    assert a[2] == b[2]
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[3], b[3])
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    return outs[0]


@pytest.mark.parametrize("name,layer,B", [
    ("C2_10", 0, 1),   # the 10%-activity headline shape: four single-token splits, joined
    ("C2", 31, 1),
    ("C3", 0, 1),
    ("C4", 0, 16),     # matrix-core tiles, 16 tokens: four splits, joined
    ("C4", 0, 32),
])
def test_default_mode_bitwise_full_size(name, layer, B):
    from synth import get_config, make_tokens
    c = get_config(name)
    say(f"default-mode repeatability {name} layer {layer} B={B}")
    s, L, Lt = build(c, layer, max_batch=B, profile_tokens=1024)
    del Lt
    assert s.deterministic
    X = make_tokens(c, B, 500, "cuda")
    other = make_tokens(c, B, 501, "cuda")
    y, idx, k, tok = _twice(s, X, other)
    # fast mode over the same weights: the same list, y within fp32 rounding
    f = s.clone(deterministic=False)
    yf, idxf, countf, _ = f.decode(X)
    torch.cuda.synchronize()
    assert int(countf.item()) == k and np.array_equal(to_np(idxf)[:k], idx)
    assert max(rel_err_rows(to_np(yf), y)) <= 1e-5
    # oracle on two sampled tokens under the GPU's own (band-checked) masks
    Xh = to_np(X)
    sel = [0, B - 1] if B > 1 else [0]
    Mg = gpu_mask_orig(s.perm, idx, k, tok, B, c.n)[sel]
    S = oracle.predict(Xh[sel], L["p1"], L["p2"], L["c"])
    M, nband = check_mask(Mg, S)
    ri, _, rt = oracle.compact(M)
    Y = oracle.forward(Xh[sel], L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"],
                       b_o=L["b_o"])
    errs = rel_err_rows(y[sel], Y)
    say(f"  count={k} band={nband} err={max(errs):.2e}")
    assert max(errs) <= REL_TOL
