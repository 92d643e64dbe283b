"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded
inputs. Integer work (compaction, index lists, counts, packing) is compared bit for bit;
floating-point outputs to max |y - y_ref| / max |y_ref| <= 1e-3 per token; predictor masks
exactly, except neurons whose oracle score lies within 1e-4 of the threshold."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (BAND, REL_TOL, build, check_mask, gpu_mask_orig, oracle_pipeline,
                      rel_err_rows, say, to_np)

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


# --------------------------------------------------------------------------- compaction
def _compact_handle(n, max_batch=64):
    from synth import get_config
    s, _, _ = build(get_config("C2"), 0, d=16, n=n, rank=16, max_batch=max_batch, pack=False)
    return s


def _check_compact(s, S_np, tau=0.0):
    B = S_np.shape[0]
    S = torch.from_numpy(np.ascontiguousarray(S_np, np.float32)).cuda()
    idx, count, tok = s.compact(S)
    torch.cuda.synchronize()
    k = int(count.item())
    ri, rk, rt = oracle.compact(oracle.threshold(S_np.astype(np.float32), tau))
    assert k == rk
    assert np.array_equal(to_np(idx)[:k], ri)
    assert np.array_equal(to_np(tok)[:k].astype(np.uint64), rt)


def test_compact_exhaustive_16():
    """Every sign pattern of 16 scores (65,536 patterns, 64 per call as a batch of tokens):
    union, count and per-token bits exact."""
    n = 16
    say("compact exhaustive n=16")
    s = _compact_handle(n)
    pats = np.arange(1 << n, dtype=np.int64)
    bits = ((pats[:, None] >> np.arange(n)[None, :]) & 1).astype(np.float32)
    allS = np.where(bits > 0, 1.0, -1.0).astype(np.float32)
    for c0 in range(0, 1 << n, 64):
        _check_compact(s, allS[c0:c0 + 64])


def test_compact_exhaustive_single_token_10():
    n = 10
    say("compact exhaustive single token n=10")
    s = _compact_handle(n, max_batch=1)
    for p in range(1 << n):
        S = np.where((p >> np.arange(n)) & 1, 1.0, -1.0).astype(np.float32)[None, :]
        _check_compact(s, S)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, 3072, 16391])
@pytest.mark.parametrize("B", [1, 3, 64])
def test_compact_boundaries(n, B):
    say(f"compact boundaries n={n} B={B}")
    s = _compact_handle(n, max_batch=64)
    rng = np.random.Generator(np.random.PCG64(n * 131 + B))
    cases = [np.full((B, n), -1.0), np.full((B, n), 1.0),
             np.tile(np.where(np.arange(n) % 2 == 0, 1.0, -1.0), (B, 1)),
             np.where(rng.random((B, n)) < 0.1, 1.0, -1.0),
             np.zeros((B, n)),                                    # exact ties: inactive
             rng.choice([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-38, -1e-38], size=(B, n))]
    for S in cases:
        _check_compact(s, S.astype(np.float32))


# --------------------------------------------------------------------------- predictor
@pytest.mark.parametrize("name,d,n,r,B", [("C1", 768, 3072, 64, 1), ("C2", 512, 1000, 64, 1),
                                          ("C2", 256, 777, 128, 4), ("C3", 256, 555, 64, 2),
                                          ("C5", 1024, 2100, 256, 1),
                                          # the matrix-core score kernel (9+ tokens)
                                          ("C2", 512, 1000, 64, 16), ("C3", 1024, 2000, 256, 33),
                                          ("C2", 1024, 3000, 256, 64), ("C5", 1024, 2100, 1024, 12)])
def test_predict_scores_and_mask(name, d, n, r, B):
    c = cfg(name)
    say(f"predict {name} d={d} n={n} r={r} B={B}")
    s, L, _ = build(c, 0, d=d, n=n, rank=r, max_batch=max(B, 1))
    X = tokens(c, B, d)
    Sg = to_np(s.predict(X))
    Xh = to_np(X)
    S = oracle.predict(Xh, L["p1"], L["p2"], L["c"])
    Sg_orig = np.empty_like(Sg)
    Sg_orig[:, s.perm] = Sg          # packed position p holds neuron perm[p]
    err = np.max(np.abs(Sg_orig - S))
    assert err <= 2e-5 * max(1.0, np.max(np.abs(S))), err
    band = np.abs(S) < BAND
    assert np.array_equal((Sg_orig > 0)[~band], (S > 0)[~band])


# --------------------------------------------------------------------------- forward / decode
SHAPES = [
    # name, d, n, r, B          (several 256-neuron tiles and a ragged tail each)
    ("C1", 768, 3072, 64, 1),
    ("C2", 512, 1000, 64, 1),
    ("C2", 256, 777, 64, 3),
    ("C3", 256, 555, 64, 1),
    ("C3", 512, 1100, 64, 4),
    ("C5", 1024, 2100, 256, 1),
    ("C2", 4096, 1500, 256, 2),
    # the vector small-batch path (weights the tile path does not take): its 4- and
    # 8-token middle kernel forms and down projections
    ("C1", 768, 3072, 64, 5),       # fp32 weights
    ("C2", 640, 1000, 64, 4),       # d not a multiple of 256
    ("C3", 384, 900, 64, 2),
    ("C3", 384, 900, 64, 7),
    # 2 tokens and more take the matrix-core tile path (fp16, d a multiple of 256)
    ("C3", 512, 1100, 64, 6),
    ("C2", 1024, 2000, 128, 8),
    ("C2", 1280, 2000, 128, 8),     # the up kernel's pipelined pairs plus a leftover pair
    ("C2", 2048, 1500, 128, 12),
    ("C2", 1536, 1200, 128, 16),    # two row tiles per workgroup, eight waves, a leftover pair
    ("C3", 1536, 1500, 128, 16),
    ("C3", 1536, 1500, 128, 24),
    ("C2", 512, 1000, 64, 9),
    ("C3", 512, 1100, 64, 16),
    ("C2", 1024, 3000, 128, 32),
    ("C3", 256, 777, 64, 20),       # ragged token tile
    ("C2", 512, 2000, 64, 64),
    ("C3", 520, 900, 64, 16),       # d not a multiple of 256: the vector path at batch 16
    ("C2", 264, 700, 64, 12),       # the vector path at 12 tokens (two 8-token groups)
    ("C2", 1024, 3000, 256, 64),    # 64 tokens x rank 256: the largest q the score kernel stages
    # wide inputs on the tile path
    ("C3", 4096, 1100, 128, 4),     # gated, full model width
    ("C2", 4096, 1300, 128, 16),    # two row tiles per workgroup
    ("C2", 2048, 1200, 128, 24),    # two token tiles
    ("C3", 2048, 1500, 128, 64),    # four token tiles
    ("C5", 12288, 900, 128, 3),     # the OPT-175B width
    ("C2", 256, 20000, 64, 4),      # more union words than the up kernel has threads
    ("C5", 8192, 1500, 512, 1),     # one token at rank 512: the four-row stage 1
]


@pytest.mark.parametrize("name,d,n,r,B", SHAPES)
def test_forward_given_mask(name, d, n, r, B):
    """Forward entry point on the oracle's own list (the same list goes to both sides)."""
    c = cfg(name)
    say(f"forward {name} d={d} n={n} r={r} B={B}")
    s, L, _ = build(c, 0, d=d, n=n, rank=r, max_batch=B)
    X = tokens(c, B, d)
    Xh = to_np(X)
    S, M, idx_o, tok_o, Y = oracle_pipeline(L, Xh)
    inv = np.empty(n, np.int64)
    inv[s.perm] = np.arange(n)
    order = np.argsort(inv[idx_o])                 # ascending packed positions
    idx_p = inv[idx_o][order].astype(np.int32)
    tok_p = tok_o[order]
    dev = X.device
    idx_t = torch.from_numpy(idx_p).to(dev) if len(idx_p) else torch.zeros(1, dtype=torch.int32, device=dev)
    cnt_t = torch.tensor([len(idx_p)], dtype=torch.int32, device=dev)
    tok_t = torch.from_numpy(tok_p.view(np.int64)).to(dev) if len(idx_p) else torch.zeros(1, dtype=torch.int64, device=dev)
    y = to_np(s.forward(X, idx_t, cnt_t, tok_t if B > 1 else None))
    errs = rel_err_rows(y, Y)
    assert max(errs) <= REL_TOL, errs


@pytest.mark.parametrize("name,d,n,r,B", SHAPES)
def test_decode_pipeline(name, d, n, r, B):
    """Fused decode: mask checked against the oracle outside the band, output against the
    oracle under that mask, and the separate predict/compact/forward calls agree."""
    c = cfg(name)
    say(f"decode {name} d={d} n={n} r={r} B={B}")
    s, L, _ = build(c, 0, d=d, n=n, rank=r, max_batch=B)
    X = tokens(c, B, d)
    Xh = to_np(X)
    scores = torch.empty((B, n), dtype=torch.float32, device="cuda")
    y, idx, count, tok = s.decode(X, scores=scores)
    torch.cuda.synchronize()
    k = int(count.item())
    idx_h, tok_h = to_np(idx), to_np(tok)
    assert np.all(np.diff(idx_h[:k]) > 0)          # ascending, no repeats
    S = oracle.predict(Xh, L["p1"], L["p2"], L["c"])
    Mg = gpu_mask_orig(s.perm, idx_h, k, tok_h, B, n)
    M, nband = check_mask(Mg, S)
    ri, rk, rt = oracle.compact(M)
    Y = oracle.forward(Xh, L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(to_np(y), Y)
    assert max(errs) <= REL_TOL, errs
    # the scores the fused kernel wrote equal the predict entry point's (same arithmetic)
    Sg = to_np(s.predict(X))
    assert np.array_equal(Sg, to_np(scores))
    # separate entry points give the same list and (to rounding) the same output
    i2, c2, t2 = s.compact(torch.from_numpy(Sg).cuda())
    torch.cuda.synchronize()
    assert int(c2.item()) == k
    assert np.array_equal(to_np(i2)[:k], idx_h[:k])
    if B > 1:
        assert np.array_equal(to_np(t2)[:k], tok_h[:k])
    y2 = to_np(s.forward(X, i2, c2, t2 if B > 1 else None))
    assert max(rel_err_rows(y2, Y)) <= REL_TOL
    say(f"  count={k} band={nband} err={max(errs):.2e}")


@pytest.mark.parametrize("name,d,n,r,B", [("C2", 512, 1000, 64, 1), ("C2", 512, 1000, 64, 4),
                                          ("C3", 512, 1100, 64, 2)])
def test_lookahead_stack(name, d, n, r, B):
    """Look-ahead schedule over a 3-layer stack: layer l >= 1 takes its active set from layer
    l - 1's input through its own predictor (layer 0 from its own input), predicted on a side
    stream beside the previous forward. Each mask is checked against the oracle outside the
    band, each output against the oracle under the GPU's own list, and the two-stream run
    equals the same calls issued on one stream, bit for bit (deterministic handles)."""
    from activation_sparse_decode_rank_amd import LookaheadBuffers, decode_lookahead
    c = cfg(name)
    say(f"look-ahead {name} d={d} n={n} r={r} B={B}")
    stack = [build(c, l, d=d, n=n, rank=r, max_batch=B, deterministic=True) for l in range(3)]
    layers = [s for s, _, _ in stack]
    xs = [tokens(c, B, d, tag=300 + l) for l in range(3)]
    side = torch.cuda.Stream()
    main = torch.cuda.Stream()
    bufs = LookaheadBuffers(layers, B)
    with torch.cuda.stream(main):
        for _ in range(2):  # the second call reuses the buffers
            decode_lookahead(layers, xs, bufs, stream=main, side_stream=side)
    torch.cuda.synchronize()
    for l, (s, L, _) in enumerate(stack):
        k = int(bufs.count[l].item())
        idx_h, tok_h = to_np(bufs.idx[l]), to_np(bufs.tokmask[l])
        Xsrc = to_np(xs[0] if l == 0 else xs[l - 1])
        S = oracle.predict(Xsrc, L["p1"], L["p2"], L["c"])
        Mg = gpu_mask_orig(s.perm, idx_h, k, tok_h, B, n)
        M, nband = check_mask(Mg, S)
        ri, rk, rt = oracle.compact(M)
        Y = oracle.forward(to_np(xs[l]), L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"],
                           b_o=L["b_o"])
        errs = rel_err_rows(to_np(bufs.y[l]), Y)
        assert max(errs) <= REL_TOL, (l, errs)
        say(f"  layer {l}: count={k} band={nband} err={max(errs):.2e}")
    # the same calls on one stream
    for l, s in enumerate(layers):
        src = xs[0] if l == 0 else xs[l - 1]
        sc = s.predict(src)
        i2, c2, t2 = s.compact(sc)
        y2 = s.forward(xs[l], i2, c2, t2)
        torch.cuda.synchronize()
        k = int(c2.item())
        assert k == int(bufs.count[l].item())
        assert np.array_equal(to_np(i2)[:k], to_np(bufs.idx[l])[:k])
        assert np.array_equal(to_np(y2), to_np(bufs.y[l]))



@pytest.mark.parametrize("name,d,n,r,nl,det", [
    ("C2", 512, 1000, 64, 3, True), ("C3", 512, 1100, 64, 3, True),
    ("C2", 1024, 3000, 128, 3, False), ("C3", 2048, 2500, 128, 3, True),
    ("C2", 4096, 16384, 256, 2, False), ("C3", 4096, 11008, 256, 2, False),
    ("C5", 12288, 6144, 1024, 2, False), ("C5", 2048, 3000, 512, 3, True),
    ("C1", 768, 3072, 64, 3, True), ("C1", 1024, 2000, 128, 3, False),
    ("C3", 6144, 1500, 128, 2, True), ("C3", 8192, 1200, 128, 2, False),
    ("C2", 8192, 2000, 128, 2, False)])
def test_lookahead_fused(name, d, n, r, nl, det):
    """Fused look-ahead decode (two launches a layer): layer l >= 1 takes its active set from
    layer l - 1's input through its own predictor, layer 0 from its own input. Each mask
    against the oracle outside the band, each output against the oracle under the GPU's own
    list; each list bit-exact with the single-token decode step's on the input it was
    predicted from (below rank 512, where both sum stage 1 in the same order; from 512 on,
    equal outside the score band); with the same token fed to every layer, y equals the
    decode step's over the same list (bitwise in the deterministic mode). Run twice: the
    held sets and buffers are reused."""
    from activation_sparse_decode_rank_amd import LookaheadBuffers, decode_lookahead_fused
    c = cfg(name)
    say(f"fused look-ahead {name} d={d} n={n} r={r} layers={nl} det={det}")
    stack = [build(c, l, d=d, n=n, rank=r, deterministic=det) for l in range(nl)]
    layers = [s for s, _, _ in stack]
    xs = [tokens(c, 1, d, tag=310 + l) for l in range(nl)]
    bufs = LookaheadBuffers(layers, 1)
    for _ in range(2):
        decode_lookahead_fused(layers, xs, bufs)
    torch.cuda.synchronize()
    for l, (s, L, _) in enumerate(stack):
        k = int(bufs.count[l].item())
        idx_h, tok_h = to_np(bufs.idx[l]), to_np(bufs.tokmask[l])
        assert np.all(np.diff(idx_h[:k]) > 0)
        assert np.all(tok_h[:k] == 1)
        src = xs[0] if l == 0 else xs[l - 1]
        S = oracle.predict(to_np(src), L["p1"], L["p2"], L["c"])
        M, nband = check_mask(gpu_mask_orig(s.perm, idx_h, k, tok_h, 1, n), S)
        ri, rk, rt = oracle.compact(M)
        Y = oracle.forward(to_np(xs[l]), L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"],
                           b_o=L["b_o"])
        errs = rel_err_rows(to_np(bufs.y[l]), Y)
        assert max(errs) <= REL_TOL, (l, errs)
        # the decode step on the input the set was predicted from makes the same list
        _, i2, c2, t2 = s.decode(src)
        torch.cuda.synchronize()
        if r < 512:
            assert int(c2.item()) == k
            assert np.array_equal(to_np(i2)[:k], idx_h[:k])
        else:
            M2 = gpu_mask_orig(s.perm, to_np(i2), int(c2.item()), to_np(t2), 1, n)
            band = np.abs(S - 0.0) < BAND
            assert not np.any((M2 != gpu_mask_orig(s.perm, idx_h, k, tok_h, 1, n)) & ~band)
        say(f"  layer {l}: count={k} band={nband} err={max(errs):.2e}")
    # one token for every layer: the held set is the layer's own, so y is the decode step's
    same = [xs[0]] * nl
    decode_lookahead_fused(layers, same, bufs)
    torch.cuda.synchronize()
    for l, s in enumerate(layers):
        y2, i2, c2, _ = s.decode(xs[0])
        torch.cuda.synchronize()
        k = int(c2.item())
        if r >= 512 and (k != int(bufs.count[l].item()) or
                         not np.array_equal(to_np(i2)[:k], to_np(bufs.idx[l])[:k])):
            continue  # a score within rounding of the threshold went the other way
        assert k == int(bufs.count[l].item())
        assert np.array_equal(to_np(i2)[:k], to_np(bufs.idx[l])[:k])
        if det:
            assert np.array_equal(to_np(y2), to_np(bufs.y[l]))
        else:
            scale = float(np.abs(to_np(y2)).max())
            assert float(np.abs(to_np(y2) - to_np(bufs.y[l])).max()) <= 1e-5 * scale


def test_lookahead_fused_rejects():
    """The fused look-ahead entry points reject a layer paired with itself or with a layer
    of another width, a pair of different weight types, and shapes their kernels do not
    cover (an input row of 2048 fp16 chunks), before anything is enqueued."""
    from activation_sparse_decode_rank_amd import _native as N
    say("fused look-ahead argument checks")
    a, _, _ = build(cfg("C2"), 0, d=512, n=1000, rank=64)
    f32, _, _ = build(cfg("C1"), 0, d=256, n=600, rank=64)
    f32w, _, _ = build(cfg("C1"), 0, d=512, n=600, rank=64)
    wide, _, _ = build(cfg("C2"), 0, d=16384, n=300, rank=64)
    x = tokens(cfg("C2"), 1, 512)
    y = torch.empty((1, 512), dtype=torch.float32, device="cuda")
    idx = torch.empty(1000, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    L = N.lib()
    assert L.sparse_ffn_decode_lookahead(a.handle, a.handle, x.data_ptr(), y.data_ptr(),
                                         idx.data_ptr(), cnt.data_ptr(), None, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_decode_lookahead(a.handle, f32.handle, x.data_ptr(), y.data_ptr(),
                                         idx.data_ptr(), cnt.data_ptr(), None, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_decode_lookahead(a.handle, f32w.handle, x.data_ptr(), y.data_ptr(),
                                         idx.data_ptr(), cnt.data_ptr(), None, None) == N.SFFN_ERR_UNSUPPORTED
    xw = tokens(cfg("C2"), 1, 16384)
    assert L.sparse_ffn_lookahead_begin(wide.handle, xw.data_ptr(), None) == N.SFFN_ERR_UNSUPPORTED



@pytest.mark.parametrize("name,d,n,r,B", [("C2", 1024, 3000, 128, 1), ("C3", 1024, 2500, 128, 4),
                                          ("C3", 1024, 2500, 128, 24)])
def test_graph_replay_matches_eager(name, d, n, r, B):
    """The decode step captured in a HIP graph and replayed several times, with eager decodes
    of other tokens in between, gives each time exactly the eager result for its token
    (lists bitwise; y bitwise in the deterministic mode). At 24 tokens this runs the
    stream-K up kernel, whose tile counters must come back to zero after every replay."""
    c = cfg(name)
    say(f"graph replay {name} d={d} n={n} r={r} B={B}")
    s, _, _ = build(c, 0, d=d, n=n, rank=r, max_batch=B, deterministic=True)
    X = tokens(c, B, d, tag=320)
    other = tokens(c, B, d, tag=321)
    y_e, i_e, c_e, t_e = [t.clone() for t in s.decode(X)]
    torch.cuda.synchronize()
    y = torch.empty_like(y_e)
    idx = torch.empty_like(i_e)
    cnt = torch.empty_like(c_e)
    tok = torch.empty_like(t_e)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        s.decode(X, y=y, idx=idx, count=cnt, tokmask=tok, stream=side)
    k = int(c_e.item())
    for rep in range(3):
        y.zero_()
        idx.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert int(cnt.item()) == k, rep
        assert np.array_equal(to_np(idx)[:k], to_np(i_e)[:k]), rep
        if B > 1:
            assert np.array_equal(to_np(tok)[:k], to_np(t_e)[:k]), rep
        assert np.array_equal(to_np(y), to_np(y_e)), rep
        s.decode(other)  # eager work on the same handle between replays
        torch.cuda.synchronize()


def test_graph_replay_lookahead():
    """The fused look-ahead decode of a 3-layer stack captured in a HIP graph and replayed
    three times, with eager decodes in between, equals the eager look-ahead run bitwise
    (deterministic handles)."""
    from activation_sparse_decode_rank_amd import LookaheadBuffers, decode_lookahead_fused
    c = cfg("C2")
    say("graph replay of the fused look-ahead")
    layers = [build(c, l, d=1024, n=3000, rank=128, deterministic=True)[0] for l in range(3)]
    xs = [tokens(c, 1, 1024, tag=330 + l) for l in range(3)]
    ref = LookaheadBuffers(layers, 1)
    decode_lookahead_fused(layers, xs, ref)
    torch.cuda.synchronize()
    bufs = LookaheadBuffers(layers, 1)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        decode_lookahead_fused(layers, xs, bufs, stream=side)
    for rep in range(3):
        for yb in bufs.y:
            yb.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(bufs.count), to_np(ref.count)), rep
        for l in range(3):
            k = int(ref.count[l].item())
            assert np.array_equal(to_np(bufs.idx[l])[:k], to_np(ref.idx[l])[:k]), (rep, l)
            assert np.array_equal(to_np(bufs.y[l]), to_np(ref.y[l])), (rep, l)
        for l, s in enumerate(layers):
            s.decode(xs[(l + 1) % 3])  # eager work that also overwrites the held sets
        torch.cuda.synchronize()



def test_lookahead_never_predicted_is_empty():
    """A layer that no look-ahead call has predicted holds the empty set (its range words are
    cleared at create): decode_ahead then lists nothing and writes y = b_out, twice in a row,
    while predicting the next layer, whose set then matches the decode step's."""
    c = cfg("C2")
    say("look-ahead on a never-predicted layer")
    (a, La, _), (b, Lb, _) = [build(c, l, d=512, n=1000, rank=64, deterministic=True)
                              for l in range(2)]
    x = tokens(c, 1, 512, tag=340)
    for _ in range(2):
        y, idx, cnt, _ = a.decode_ahead(x, b)
        torch.cuda.synchronize()
        assert int(cnt.item()) == 0
        assert np.array_equal(to_np(y)[0], La["b_o"].astype(np.float32))
    y2, i2, c2, _ = b.decode_ahead(x, None)
    _, i3, c3, _ = b.decode(x)
    torch.cuda.synchronize()
    k = int(c3.item())
    assert int(c2.item()) == k and np.array_equal(to_np(i2)[:k], to_np(i3)[:k])


def test_decode_deterministic():
    """deterministic=1: repeated decodes give bitwise-identical y and lists, and match the
    oracle (the vector down projection splits rows at most two ways)."""
    c = cfg("C2")
    say("decode determinism")
    s, L, _ = build(c, 0, d=1024, n=4096, rank=128, max_batch=4, deterministic=True)
    X = tokens(c, 4, 1024)
    outs = []
    for _ in range(3):
        y, idx, count, tok = s.decode(X)
        torch.cuda.synchronize()
        outs.append((to_np(y).copy(), to_np(idx)[: int(count.item())].copy()))
    for y, idx in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(idx, outs[0][1])
    y, idx, count, tok = s.decode(X)
    torch.cuda.synchronize()
    Xh = to_np(X)
    k = int(count.item())
    S = oracle.predict(Xh, L["p1"], L["p2"], L["c"])
    M, _ = check_mask(gpu_mask_orig(s.perm, to_np(idx), k, to_np(tok), 4, s.n), S)
    ri, _, rt = oracle.compact(M)
    Y = oracle.forward(Xh, L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    assert max(rel_err_rows(to_np(y), Y)) <= REL_TOL


def test_decode_fast_mode_repeatable():
    """deterministic=0: lists stay bit-exact across runs; y may differ only in rounding of
    the float atomics that join the down projection's row splits."""
    c = cfg("C2")
    say("decode fast-mode repeatability")
    s, _, _ = build(c, 0, d=1024, n=4096, rank=128, max_batch=4, deterministic=False)
    X = tokens(c, 4, 1024)
    outs = []
    for _ in range(3):
        y, idx, count, tok = s.decode(X)
        torch.cuda.synchronize()
        outs.append((to_np(y).copy(), to_np(idx)[: int(count.item())].copy(),
                     to_np(tok)[: int(count.item())].copy()))
    for y, idx, tok in outs[1:]:
        assert np.array_equal(idx, outs[0][1]) and np.array_equal(tok, outs[0][2])
        assert max(rel_err_rows(y, outs[0][0])) <= 1e-6


def test_batch_rows_equal_single_token_calls():
    """Row b of a batched decode equals decoding token b alone (to fp32 rounding of a
    different summation grouping)."""
    c = cfg("C3")
    say("batch vs single")
    s, _, _ = build(c, 0, d=512, n=1100, rank=64, max_batch=8)
    X = tokens(c, 8, 512)
    yb = to_np(s.decode(X)[0])
    for b in range(8):
        y1 = to_np(s.decode(X[b:b + 1].contiguous())[0])
        assert max(rel_err_rows(yb[b:b + 1], y1)) <= 1e-5


# --------------------------------------------------------------------------- invariants on the GPU
@pytest.mark.parametrize("gated", [False, True])
def test_all_active_and_true_sign_equal_dense(gated):
    """I1/I2 on the GPU: with every neuron listed, and with the list of truly active
    neurons, the sparse output equals the dense FFN (oracle)."""
    c = cfg("C3" if gated else "C2")
    d, n, r, B = 512, 1200, 64, 2
    say(f"all-active / true-sign gated={gated}")
    s, L, _ = build(c, 0, d=d, n=n, rank=r, max_batch=B)
    X = tokens(c, B, d)
    Xh = to_np(X)
    D = oracle.dense(Xh, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    dev = X.device
    allp = torch.arange(n, dtype=torch.int32, device=dev)
    y = to_np(s.forward(X, allp, torch.tensor([n], dtype=torch.int32, device=dev),
                        torch.full((n,), -1, dtype=torch.int64, device=dev)))
    assert max(rel_err_rows(y, D)) <= REL_TOL
    A = oracle.preact(Xh, L["w_a"], L["b_a"])
    T = (A > 0).astype(np.uint8)
    inv = np.empty(n, np.int64)
    inv[s.perm] = np.arange(n)
    idx_o, k, tok_o = oracle.compact(T)
    order = np.argsort(inv[idx_o])
    y2 = to_np(s.forward(X, torch.from_numpy(inv[idx_o][order].astype(np.int32)).to(dev),
                         torch.tensor([k], dtype=torch.int32, device=dev),
                         torch.from_numpy(tok_o[order].view(np.int64)).to(dev)))
    assert max(rel_err_rows(y2, D)) <= REL_TOL


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("B,d", [(1, 64), (5, 64), (16, 128), (6, 256), (16, 256), (24, 256),
                                 (24, 1024), (16, 2048)])
def test_integer_fixture_bit_exact(gated, B, d):
    """Integer weights and tokens: every partial sum is exact in fp32 (and each activation
    is exactly hi + lo in fp16), so the HIP path must reproduce the oracle bit for bit,
    scores, list and output, on the vector path (d = 64, 128) and on the matrix-core tile
    path with its matrix-core score kernel (d = 256, rank 32), the two-row-tile up kernel
    (16 tokens, d = 2048) and the stream-K up projection with its split tiles (24 tokens,
    d = 1024)."""
    from activation_sparse_decode_rank_amd import SparseFFN
    from synth import integer_layer
    n, r = 1000, (32 if d % 256 == 0 else 16)
    say(f"integer fixture gated={gated} B={B}")
    lo, hi = (-1, 1) if gated else (-2, 2)
    L = integer_layer(d, n, r, gated=gated, seed=77 + B, B=B, lo=lo, hi=hi)
    T = {k: (torch.from_numpy(v).cuda() if v is not None else None) for k, v in L.items()}
    Xp = torch.from_numpy(integer_layer(d, n, r, gated=gated, seed=5, B=64, lo=lo, hi=hi)["x"]).cuda()
    s = SparseFFN(w_act=T["w_a"], w_up=T["w_u"], w_down_t=T["w_o"], p1=T["p1"], p2=T["p2"],
                  b_act=T["b_a"], b_out=T["b_o"], p_bias=T["c"], max_batch=B, profile_x=Xp,
                  hot_frac=0.2)
    # profile counts: exact integers on both sides
    cnt_o = oracle.profile_counts(to_np(Xp), L["w_a"], L["b_a"])
    assert np.array_equal(s.profile_counts, cnt_o)
    assert np.array_equal(s.perm, oracle.permutation(cnt_o, int(np.ceil(0.2 * n))))
    X = T["x"]
    scores = torch.empty((B, n), dtype=torch.float32, device="cuda")
    y, idx, count, tok = s.decode(X, scores=scores)
    torch.cuda.synchronize()
    S = oracle.predict(L["x"], L["p1"], L["p2"], L["c"])
    Sg = np.empty_like(to_np(scores))
    Sg[:, s.perm] = to_np(scores)
    assert np.array_equal(Sg.astype(np.float64), S)
    k = int(count.item())
    M = oracle.threshold(S)
    Mg = gpu_mask_orig(s.perm, to_np(idx), k, to_np(tok), B, n)
    assert np.array_equal(Mg, M)
    ri, rk, rt = oracle.compact(M)
    Y = oracle.forward(L["x"], L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    assert np.array_equal(to_np(y).astype(np.float64), Y)


@pytest.mark.parametrize("B,d", [(1, 256), (2, 256), (24, 1024)])
def test_empty_mask_gives_output_bias(B, d):
    """No active neuron: y = b_out, on the single-token path, the tile path and the
    stream-K up kernel (24 tokens)."""
    c = cfg("C2")
    say(f"empty mask B={B} d={d}")
    s, L, _ = build(c, 0, d=d, n=700, rank=64, max_batch=B, threshold=float("inf"))
    X = tokens(c, B, d)
    for _ in range(2):  # the second call sees the counters the first left
        y, idx, count, tok = s.decode(X)
        torch.cuda.synchronize()
        assert int(count.item()) == 0
        assert np.array_equal(to_np(y), np.tile(L["b_o"], (B, 1)))


@pytest.mark.parametrize("tau", [0.2, 0.5, 1.0])
def test_stream_k_small_unions(tau):
    """Stream-K up kernel (24 tokens, d = 1024) on unions of a few tiles down to a handful of
    rows (raised thresholds): list bit-exact with the oracle on the GPU's own scores, output
    within tolerance under that list, and the same result on a second call (the tiles'
    arrival counters are back at zero)."""
    c = cfg("C2")
    B, d, n = 24, 1024, 1500
    say(f"stream-K small union tau={tau}")
    s, L, _ = build(c, 0, d=d, n=n, rank=128, max_batch=B, threshold=tau, deterministic=True)
    X = tokens(c, B, d)
    scores = torch.empty((B, n), dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(2):
        y, idx, count, tok = s.decode(X, scores=scores)
        torch.cuda.synchronize()
        outs.append((to_np(y).copy(), int(count.item()), to_np(idx).copy(), to_np(tok).copy()))
    (y1, k, idx_h, tok_h), (y2, k2, idx2, tok2) = outs
    assert k == k2 and np.array_equal(y1, y2) and np.array_equal(idx_h[:k], idx2[:k])
    ri, rk, rt = oracle.compact(oracle.threshold(to_np(scores).astype(np.float32), tau))
    assert rk == k
    assert np.array_equal(idx_h[:k], ri)
    assert np.array_equal(tok_h[:k].astype(np.uint64), rt)
    Mg = gpu_mask_orig(s.perm, idx_h, k, tok_h, B, n)
    ro, rko, rto = oracle.compact(Mg)
    Y = oracle.forward(to_np(X), L["w_a"], L["w_o"], ro, rto, Wu=L["w_u"], b_a=L["b_a"],
                       b_o=L["b_o"])
    assert max(rel_err_rows(y1, Y)) <= REL_TOL
    say(f"  count={k}")


# --------------------------------------------------------------------------- offline steps
def test_pack_rows_bit_exact():
    from activation_sparse_decode_rank_amd import pack_rows
    say("pack rows")
    rng = np.random.Generator(np.random.PCG64(3))
    for rows, shape, dt in [(1000, (1000, 72), np.float16), (777, (777,), np.float32),
                            (300, (300, 2, 40), np.float16)]:
        src = rng.standard_normal(shape).astype(dt)
        perm = rng.permutation(rows).astype(np.int32)
        dst = to_np(pack_rows(torch.from_numpy(src).cuda(), torch.from_numpy(perm).cuda()))
        torch.cuda.synchronize()
        assert np.array_equal(dst.view(np.uint8), oracle.pack_rows(src, perm).view(np.uint8))
    # strided: the gated bundle
    g = rng.standard_normal((50, 24)).astype(np.float16)
    u = rng.standard_normal((50, 24)).astype(np.float16)
    perm = rng.permutation(50).astype(np.int32)
    pd = torch.from_numpy(perm).cuda()
    bundle = torch.empty((50, 2, 24), dtype=torch.float16, device="cuda")
    pack_rows(torch.from_numpy(g).cuda(), pd, bundle, 0, 96)
    pack_rows(torch.from_numpy(u).cuda(), pd, bundle, 48, 96)
    b = to_np(bundle)
    assert np.array_equal(b[:, 0], oracle.pack_rows(g, perm)) and np.array_equal(b[:, 1], oracle.pack_rows(u, perm))


def test_profile_counts_float_within_band():
    from activation_sparse_decode_rank_amd import profile_counts
    from synth import make_layer, make_tokens
    c = cfg("C2")
    say("profile counts float")
    Lt = make_layer(c, 0, "cuda", d=512, n=1000, rank=64)
    X = make_tokens(c, 300, 100, "cuda", d=512)
    cg = to_np(profile_counts(Lt.w_a, Lt.b_a, X))
    A = oracle.preact(to_np(X), to_np(Lt.w_a), to_np(Lt.b_a))
    co = (A > 0).sum(axis=0)
    slack = (np.abs(A) < BAND).sum(axis=0)
    assert np.all(np.abs(cg - co) <= slack)


# --------------------------------------------------------------------------- full sizes
@pytest.mark.parametrize("name,layer", [("C1", 0), ("C2", 31), ("C3", 0), ("C5", 0)])
def test_full_size_layer_decode(name, layer):
    """Full configuration shapes, the launch configuration the benchmark times: one layer,
    one token (C2's last layer is its 10%-active one)."""
    c = cfg(name)
    say(f"full size {name} layer {layer}")
    s, L, Lt = build(c, layer, max_batch=1, profile_tokens=1024)
    del Lt
    X = tokens(c, 1, c.d)
    Xh = to_np(X)
    y, idx, count, tok = s.decode(X)
    torch.cuda.synchronize()
    k = int(count.item())
    _check_published_list(s, X, 1, to_np(idx), k, to_np(tok))
    S = oracle.predict(Xh, L["p1"], L["p2"], L["c"])
    Mg = gpu_mask_orig(s.perm, to_np(idx), k, to_np(tok), 1, c.n)
    M, nband = check_mask(Mg, S)
    ri, rk, rt = oracle.compact(M)
    Y = oracle.forward(Xh, L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(to_np(y), Y)
    say(f"  count={k} ({k / c.n:.3f}) band={nband} err={max(errs):.2e}")
    assert max(errs) <= REL_TOL


def _check_published_list(s, X, B, idx_h, k, tok_h):
    """The list a full-size decode publishes (idx, count, token bits; read by nothing in the
    step itself, whose down kernels take the ranges' activity words) must be the compaction
    of the decode's own scores, bit for bit: a second decode that also returns its scores
    publishes the same list, strictly ascending, equal to the oracle's compaction of those
    scores (the same fp32 values on both sides, no band)."""
    scores = torch.empty((B, s.n), dtype=torch.float32, device="cuda")
    _, idx2, count2, tok2 = s.decode(X, scores=scores)
    torch.cuda.synchronize()
    assert int(count2.item()) == k
    assert np.array_equal(to_np(idx2)[:k], idx_h[:k])
    assert np.array_equal(to_np(tok2)[:k], tok_h[:k])
    assert np.all(np.diff(idx_h[:k]) > 0)
    ri, rk, rt = oracle.compact(oracle.threshold(to_np(scores).astype(np.float32), s.threshold))
    assert rk == k
    assert np.array_equal(idx_h[:k], ri)
    assert np.array_equal(tok_h[:k].astype(np.uint64), rt)


@pytest.mark.parametrize("B", [2, 4, 8, 16, 32])
def test_full_size_batch_decode(B):
    """The batch sweep's shape (Llama-7B-shaped gated layer, d=4096, d_ffn=11008) at 2 to 32
    tokens with independent per-token masks: the matrix-core tile path in the launch
    configuration the benchmark times, checked per token against the oracle under the
    GPU's own (band-checked) masks."""
    c = cfg("C4")
    say(f"full size batch {B}")
    s, L, Lt = build(c, 0, max_batch=B, profile_tokens=1024)
    del Lt
    X = tokens(c, B, c.d)
    Xh = to_np(X)
    y, idx, count, tok = s.decode(X)
    torch.cuda.synchronize()
    k = int(count.item())
    _check_published_list(s, X, B, to_np(idx), k, to_np(tok))
    S = oracle.predict(Xh, L["p1"], L["p2"], L["c"])
    Mg = gpu_mask_orig(s.perm, to_np(idx), k, to_np(tok), B, c.n)
    M, nband = check_mask(Mg, S)
    ri, rk, rt = oracle.compact(M)
    Y = oracle.forward(Xh, L["w_a"], L["w_o"], ri, rt, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    errs = rel_err_rows(to_np(y), Y)
    say(f"  union={k} ({k / c.n:.3f}) band={nband} err={max(errs):.2e}")
    assert max(errs) <= REL_TOL


def test_batch_tiles_deterministic():
    """deterministic=1 on the tile path: bitwise-identical outputs across runs."""
    c = cfg("C3")
    say("tile path determinism")
    s, _, _ = build(c, 0, d=512, n=1100, rank=64, max_batch=32, deterministic=True)
    X = tokens(c, 32, 512)
    outs = [to_np(s.decode(X)[0]).copy() for _ in range(3)]
    for y in outs[1:]:
        assert np.array_equal(y, outs[0])
