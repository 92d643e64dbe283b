"""GPU parity of the neuron-bundle layout and the single-pass single-token decode (gather and
down projection in one pass over each active neuron's bundle, then a fixed-order reduction of
the workgroups' partial outputs) against the fp64 oracle, and against the three-launch path.

The bundle follows PowerInfer-2's neuron clusters (PowerInfer-2 article, section 4.4
Neuron-Cluster-Level Pipeline: a neuron's gate, up and down rows are used together and stored
together). Lists, counts and token bits are compared bit for bit, scores bitwise against the
predict entry point, outputs to max |y - y_ref| / max |y_ref| <= 1e-3 per token."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (REL_TOL, build, check_mask, gpu_mask_orig, rel_err_rows, say, to_np)

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


def _check_decode(s, L, X, B):
    """Decode with scores: scores bitwise equal to predict's, the list bit-exact with the
    oracle's compaction of those scores, the mask equal to the oracle's outside the band, y
    within tolerance of the oracle under the GPU's list. Returns (y, idx, count, tok)."""
    n = s.n
    scores = torch.empty((B, n), dtype=torch.float32, device="cuda")
    y, idx, count, tok = s.decode(X, scores=scores)
    torch.cuda.synchronize()
    k = int(count.item())
    idx_h, tok_h = to_np(idx), to_np(tok)
    Sg = to_np(s.predict(X))
    assert np.array_equal(Sg, to_np(scores))
    ri, rk, rt = oracle.compact(oracle.threshold(Sg.astype(np.float32), s.threshold))
    assert rk == k and np.array_equal(idx_h[:k], ri)
    assert np.array_equal(tok_h[:k].astype(np.uint64), rt)
    Xh = to_np(X)
    S = oracle.predict(Xh, L["p1"], L["p2"], L["c"])
    Mg = gpu_mask_orig(s.perm, idx_h, k, tok_h, B, n)
    M, nband = check_mask(Mg, S, s.threshold)
    oi, _, ot = oracle.compact(M)
    Y = oracle.forward(Xh, L["w_a"], L["w_o"], oi, ot, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(to_np(y), Y)
    say(f"  count={k} band={nband} err={max(errs):.2e}")
    assert max(errs) <= REL_TOL, errs
    return to_np(y), idx_h[:k], k, tok_h[:k]


@pytest.mark.parametrize("name,d,n,r", [
    ("C1", 768, 3072, 64),     # fp32 weights and predictor
    ("C2", 512, 1000, 64),
    ("C2", 4096, 1500, 256),   # the OPT-6.7B width: two input and two down chunks a thread
    ("C3", 512, 1100, 64),     # gated bundle [gate, up, down]
    ("C3", 4096, 1100, 256),   # gated at the Llama-7B width
    ("C2", 2048, 5000, 128),   # several ranges per workgroup left over at the end
])
@pytest.mark.parametrize("bundle", [True, False])
def test_single_pass_decode(name, d, n, r, bundle):
    c = cfg(name)
    say(f"single pass {name} d={d} n={n} r={r} bundle={bundle}")
    s, L, _ = build(c, 0, d=d, n=n, rank=r, bundle=bundle, single_pass=True)
    X = tokens(c, 1, d)
    y1, i1, k1, _ = _check_decode(s, L, X, 1)
    # run twice: bitwise the same (no float atomics anywhere on this path)
    y2, i2, k2, _ = [v for v in _check_decode(s, L, X, 1)]
    assert k1 == k2 and np.array_equal(i1, i2) and np.array_equal(y1, y2)
    # the three-launch path on the same weights: the same list, y to rounding
    t = s.clone(single_pass=False)
    yt, it, ct, _ = t.decode(X)
    torch.cuda.synchronize()
    assert int(ct.item()) == k1 and np.array_equal(to_np(it)[:k1], i1)
    assert max(rel_err_rows(y1, to_np(yt))) <= 1e-5


@pytest.mark.parametrize("name,layer", [("C2_10", 31), ("C3", 0), ("C1", 0)])
def test_single_pass_full_size(name, layer):
    """The launch configuration a benchmark would time, at full size: OPT-6.7B layer 31 at
    10% activity, the Llama-7B gated layer, the OPT-125m layer; run twice, bitwise equal."""
    c = cfg(name)
    say(f"single pass full size {name} layer {layer}")
    s, L, Lt = build(c, layer, max_batch=1, profile_tokens=1024, bundle=True, single_pass=True)
    del Lt
    X = tokens(c, 1, c.d)
    y1, i1, k1, _ = _check_decode(s, L, X, 1)
    y2, i2, k2, _ = s.decode(X)
    torch.cuda.synchronize()
    assert int(k2.item()) == k1 and np.array_equal(to_np(y2), y1)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("d", [256, 1024])
def test_single_pass_integer_fixture_bit_exact(gated, d):
    """Integer weights and tokens: every sum exact, so the single pass reproduces the oracle
    bit for bit (scores, list and y), from both layouts."""
    from activation_sparse_decode_rank_amd import SparseFFN
    from synth import integer_layer
    n, r = 1000, 32
    say(f"single pass integer fixture gated={gated} d={d}")
    lo, hi = (-1, 1) if gated else (-2, 2)
    L = integer_layer(d, n, r, gated=gated, seed=91 + d, B=1, lo=lo, hi=hi)
    T = {k: (torch.from_numpy(v).cuda() if v is not None else None) for k, v in L.items()}
    Xp = torch.from_numpy(integer_layer(d, n, r, gated=gated, seed=5, B=64, lo=lo, hi=hi)["x"]).cuda()
    for bundle in (True, False):
        s = SparseFFN(w_act=T["w_a"], w_up=T["w_u"], w_down_t=T["w_o"], p1=T["p1"], p2=T["p2"],
                      b_act=T["b_a"], b_out=T["b_o"], p_bias=T["c"], max_batch=1, profile_x=Xp,
                      hot_frac=0.2, bundle=bundle, single_pass=True)
        scores = torch.empty((1, n), dtype=torch.float32, device="cuda")
        y, idx, count, tok = s.decode(T["x"], scores=scores)
        torch.cuda.synchronize()
        S = oracle.predict(L["x"], L["p1"], L["p2"], L["c"])
        Sg = np.empty_like(to_np(scores))
        Sg[:, s.perm] = to_np(scores)
        assert np.array_equal(Sg.astype(np.float64), S)
        k = int(count.item())
        M = oracle.threshold(S)
        assert np.array_equal(gpu_mask_orig(s.perm, to_np(idx), k, to_np(tok), 1, n), M)
        ri, _, rt = oracle.compact(M)
        Y = oracle.forward(L["x"], L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
        assert np.array_equal(to_np(y).astype(np.float64), Y)


@pytest.mark.parametrize("tau,expect", [(float("-inf"), "all"), (float("inf"), "none")])
def test_single_pass_all_and_none(tau, expect):
    """Every neuron listed: y equals the dense FFN (oracle); none listed: y = b_out."""
    c = cfg("C3")
    d, n = 512, 3000
    say(f"single pass {expect} active")
    s, L, _ = build(c, 0, d=d, n=n, rank=64, threshold=tau, bundle=True, single_pass=True)
    X = tokens(c, 1, d)
    y, idx, count, tok = s.decode(X)
    torch.cuda.synchronize()
    k = int(count.item())
    if expect == "all":
        assert k == n and np.array_equal(to_np(idx)[:n], np.arange(n, dtype=np.int32))
        D = oracle.dense(to_np(X), L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
        assert max(rel_err_rows(to_np(y), D)) <= REL_TOL
    else:
        assert k == 0
        assert np.array_equal(to_np(y)[0], L["b_o"].astype(np.float32))


@pytest.mark.parametrize("name,d,n,r,B", [
    ("C2", 1024, 3000, 128, 1),   # three-launch single-token path
    ("C1", 768, 3072, 64, 5),     # vector small-batch path (fp32)
    ("C3", 512, 1100, 64, 4),     # matrix-core tiles
    ("C3", 1024, 2500, 128, 24),  # stream-K up kernel
    ("C2", 520, 1000, 64, 16),    # vector path at 16 tokens (d not a multiple of 256)
])
def test_bundle_layout_matches_split_layout(name, d, n, r, B):
    """The bundle layout through every other kernel (strided rows): bitwise the same lists
    and y as the split layout (deterministic mode), through decode and forward."""
    c = cfg(name)
    say(f"bundle vs split layout {name} d={d} n={n} r={r} B={B}")
    a, _, _ = build(c, 0, d=d, n=n, rank=r, max_batch=B, deterministic=True, bundle=True)
    b, _, _ = build(c, 0, d=d, n=n, rank=r, max_batch=B, deterministic=True, bundle=False)
    X = tokens(c, B, d)
    ya, ia, ca, ta = a.decode(X)
    yb, ib, cb, tb = b.decode(X)
    torch.cuda.synchronize()
    k = int(ca.item())
    assert int(cb.item()) == k
    assert np.array_equal(to_np(ia)[:k], to_np(ib)[:k]) and np.array_equal(to_np(ta)[:k], to_np(tb)[:k])
    assert np.array_equal(to_np(ya), to_np(yb))
    fa = a.forward(X, ia, ca, ta if B > 1 else None)
    fb = b.forward(X, ib, cb, tb if B > 1 else None)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(fa), to_np(fb))


def test_bundle_layout_lookahead():
    """The fused look-ahead decode over bundle-layout layers equals the split layout's."""
    from activation_sparse_decode_rank_amd import LookaheadBuffers, decode_lookahead_fused
    c = cfg("C2")
    d, n, r = 1024, 3000, 128
    say("bundle layout look-ahead")
    outs = []
    for bundle in (True, False):
        layers = [build(c, l, d=d, n=n, rank=r, deterministic=True, bundle=bundle)[0] for l in range(3)]
        xs = [tokens(c, 1, d, tag=500 + l) for l in range(3)]
        bufs = LookaheadBuffers(layers, 1)
        decode_lookahead_fused(layers, xs, bufs)
        torch.cuda.synchronize()
        outs.append(([to_np(v).copy() for v in bufs.y], to_np(bufs.count).copy()))
    assert np.array_equal(outs[0][1], outs[1][1])
    for ya, yb in zip(outs[0][0], outs[1][0]):
        assert np.array_equal(ya, yb)


def test_single_pass_graph_replay():
    """The single-pass decode captured in a HIP graph and replayed three times, with eager
    decodes of other tokens in between: every replay bitwise equal to the eager result."""
    c = cfg("C3")
    d, n = 1024, 2500
    say("single pass graph replay")
    s, _, _ = build(c, 0, d=d, n=n, rank=128, bundle=True, single_pass=True)
    X = tokens(c, 1, d, tag=330)
    other = tokens(c, 1, d, tag=331)
    y_e, i_e, c_e, t_e = [t.clone() for t in s.decode(X)]
    torch.cuda.synchronize()
    y, idx, cnt, tok = [torch.empty_like(t) for t in (y_e, i_e, c_e, t_e)]
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        s.decode(X, y=y, idx=idx, count=cnt, tokmask=tok, stream=side)
    k = int(c_e.item())
    for rep in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert int(cnt.item()) == k
        assert np.array_equal(to_np(idx)[:k], to_np(i_e)[:k])
        assert np.array_equal(to_np(y), to_np(y_e))
        s.decode(other)
        torch.cuda.synchronize()
