"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix, not
against the oracle itself. Each pin is a plain function that raises AssertionError on a
mismatch, so the same pins run against the real oracle (test_oracle.py) and against
deliberately broken copies of it (test_oracle_mutants.py)."""
import numpy as np

import oracle
from golden_io import ints, mat, read, vec


# ----------------------------------------------------------------------------- helpers
def numpy_dense(X, Wa, Wo, Wu=None, b_a=None, b_o=None):
    """Textbook dense FFN in numpy fp64 (library matmul, independent summation order)."""
    X = np.asarray(X, np.float64)
    A = X @ np.asarray(Wa, np.float64).T
    if b_a is not None:
        A = A + np.asarray(b_a, np.float64)
    H = np.maximum(A, 0.0)
    if Wu is not None:
        H = H * (X @ np.asarray(Wu, np.float64).T)
    Y = H @ np.asarray(Wo, np.float64)
    if b_o is not None:
        Y = Y + np.asarray(b_o, np.float64)
    return Y


def rel_err(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / den)


def float_layer(rng, d, n, r, gated, wdt=np.float16, B=1):
    w = lambda *s: (rng.standard_normal(s) * 0.02).astype(wdt)  # noqa: E731
    L = dict(w_a=w(n, d), w_u=w(n, d) if gated else None, w_o=w(n, d),
             b_a=(rng.standard_normal(n) * 0.1).astype(np.float32),
             b_o=(rng.standard_normal(d) * 0.01).astype(np.float32),
             p1=(rng.standard_normal((r, d)) / np.sqrt(d)).astype(wdt),
             p2=w(n, r), c=(rng.standard_normal(n) * 0.05).astype(np.float32))
    X = rng.standard_normal((B, d)).astype(np.float32)
    return L, X


# ----------------------------------------------------------------------------- pins
def pin_half_decoder_exhaustive():
    """Every binary16 bit pattern decodes to numpy's float16 -> float64 value."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def pin_tiny_hand_fixture():
    """The paper-computed layer in tests/golden/tiny_ffn_hand.txt, every quantity exactly."""
    g = read("tiny_ffn_hand.txt")
    x = vec(g["x"]).astype(np.float32)[None, :]
    for wdt in (np.float16, np.float32, np.float64):
        Wa, Wu, Wo = (mat(g[k]).astype(wdt) for k in ("w_a", "w_u", "w_o"))
        b_a, b_o = vec(g["b_a"]).astype(np.float32), vec(g["b_o"]).astype(np.float32)
        assert np.array_equal(oracle.preact(x, Wa, b_a)[0], vec(g["preact"]))
        assert np.array_equal(oracle.dense(x, Wa, Wo, b_a=b_a, b_o=b_o)[0], vec(g["plain_dense"]))
        assert np.array_equal(oracle.dense(x, Wa, Wo, Wu=Wu, b_a=b_a, b_o=b_o)[0], vec(g["gated_dense"]))
        cases = [("plain_mask_2", [2], None), ("plain_mask_0", [0], None), ("plain_mask_1", [1], None),
                 ("plain_mask_empty", [], None), ("plain_dense", [0, 1, 2], None),
                 ("plain_dense", ints(g["true_set"]), None),
                 ("gated_mask_2", [2], Wu), ("gated_mask_0", [0], Wu), ("gated_dense", [0, 1, 2], Wu)]
        for key, M, wu in cases:
            y = oracle.forward(x, Wa, Wo, np.array(M, np.int32), Wu=wu, b_a=b_a, b_o=b_o)[0]
            assert np.array_equal(y, vec(g[key])), (key, y)
        p1, p2 = mat(g["p1"]).astype(wdt), mat(g["p2"]).astype(wdt)
        s = oracle.predict(x, p1, p2, vec(g["c"]).astype(np.float32))
        assert np.array_equal(s[0], vec(g["scores"]))
        assert list(np.flatnonzero(oracle.threshold(s, 0.0)[0])) == ints(g["active_tau_0"])
        assert list(np.flatnonzero(oracle.threshold(s, 0.5)[0])) == ints(g["active_tau_0.5"])


def pin_compaction_hand_batch():
    g = read("compaction_batch_hand.txt")
    S = np.stack([vec(g[f"scores{b}"]) for b in range(3)]).astype(np.float32)
    idx, k, tok = oracle.compact(oracle.threshold(S, 0.0))
    assert k == int(g["count"])
    assert list(idx) == ints(g["idx"])
    assert [int(t) for t in tok] == ints(g["tokmask"])


def pin_permutation_hand():
    g = read("permutation_hand.txt")
    counts = np.array(ints(g["counts"]), np.int64)
    for h in (4, 0, 8, 1):
        assert list(oracle.permutation(counts, h)) == ints(g[f"perm_hot{h}"]), h


def pin_worked_example():
    """Hot/cold placement never changes which neurons are computed: only the predicted set
    counts (novita.ai article, section 單層計算優化)."""
    g = read("powerinfer_worked_example.txt")
    n = int(g["n"])
    hot, pred, comp = ints(g["hot"]), ints(g["predicted"]), ints(g["computed"])
    counts = np.zeros(n, np.int64)
    counts[hot] = 100
    perm = oracle.permutation(counts, len(hot))
    assert sorted(perm[: len(hot)]) == sorted(hot)
    scores = -np.ones((1, n))
    scores[0, pred] = 1.0
    packed_scores = scores[:, perm]                 # packed position p holds neuron perm[p]
    idx, k, _ = oracle.compact(oracle.threshold(packed_scores, 0.0))
    assert sorted(perm[idx].tolist()) == comp
    assert 7 in hot and 7 not in perm[idx].tolist()  # hot but not predicted: skipped


def pin_dense_matches_numpy():
    """I1: D(x) equals the textbook dense FFN; F(x, all) equals D(x) exactly."""
    rng = np.random.Generator(np.random.PCG64(11))
    for (d, n, gated, wdt, B) in [(24, 37, False, np.float16, 3), (16, 29, True, np.float32, 2),
                                  (40, 64, False, np.float64, 1), (8, 70, True, np.float16, 4)]:
        L, X = float_layer(rng, d, n, 4, gated, wdt, B)
        Yd = oracle.dense(X, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
        Yn = numpy_dense(X, L["w_a"], L["w_o"], L["w_u"], L["b_a"], L["b_o"])
        assert rel_err(Yd, Yn) < 1e-12, rel_err(Yd, Yn)
        Yf = oracle.forward(X, L["w_a"], L["w_o"], np.arange(n, dtype=np.int32), Wu=L["w_u"],
                            b_a=L["b_a"], b_o=L["b_o"])
        assert np.array_equal(Yf, Yd)


def pin_true_sign_superset():
    """I2: with any mask covering every neuron whose ReLU input is > 0, the sparse output is
    bit-identical to the dense one (skipped rows contribute exact zeros)."""
    rng = np.random.Generator(np.random.PCG64(12))
    for gated in (False, True):
        L, X = float_layer(rng, 32, 90, 4, gated, np.float16, 1)
        A = oracle.preact(X, L["w_a"], L["b_a"])[0]
        T = np.flatnonzero(A > 0)
        # compare against numpy (independent of the oracle) and against the oracle's dense
        Yn = numpy_dense(X, L["w_a"], L["w_o"], L["w_u"], L["b_a"], L["b_o"])
        Yd = oracle.dense(X, L["w_a"], L["w_o"], Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
        for extra in (0.0, 0.3, 1.0):
            M = np.union1d(T, np.flatnonzero(rng.random(90) < extra)).astype(np.int32)
            Y = oracle.forward(X, L["w_a"], L["w_o"], M, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
            assert np.array_equal(Y, Yd)
            assert rel_err(Y, Yn) < 1e-12
        # a mask missing a truly active neuron must differ
        if len(T) > 0:
            M = np.setdiff1d(T, T[:1]).astype(np.int32)
            Y = oracle.forward(X, L["w_a"], L["w_o"], M, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
            assert not np.allclose(Y, Yd, rtol=0, atol=1e-9)


def pin_brute_force_masks():
    """I5: for tiny layers, every one of the 2^n masks gives the dense FFN of the layer whose
    down rows outside the mask are zeroed (computed by numpy)."""
    rng = np.random.Generator(np.random.PCG64(13))
    for (d, n, gated) in [(6, 7, False), (5, 6, True)]:
        L, X = float_layer(rng, d, n, 2, gated, np.float64, 2)
        for bits in range(1 << n):
            M = np.array([i for i in range(n) if (bits >> i) & 1], np.int32)
            keep = np.zeros((n, 1))
            keep[M] = 1.0
            Yn = numpy_dense(X, L["w_a"], L["w_o"] * keep, L["w_u"], L["b_a"], L["b_o"])
            Y = oracle.forward(X, L["w_a"], L["w_o"], M, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
            assert np.allclose(Y, Yn, rtol=1e-12, atol=1e-15), bits


def pin_compaction_exhaustive(nmax=16):
    """I5: compaction of every sign pattern of n <= nmax scores is the ascending list of set
    positions, and count is the popcount."""
    for n in (1, 5, nmax):
        for bits in range(1 << n):
            s = np.array([1.0 if (bits >> i) & 1 else -1.0 for i in range(n)])
            idx, k, tok = oracle.compact(oracle.threshold(s[None, :], 0.0))
            ref = [i for i in range(n) if (bits >> i) & 1]
            assert k == bin(bits).count("1") and list(idx) == ref
            assert all(int(t) == 1 for t in tok)


def pin_compaction_batch_random():
    """Batch compaction: union ascending; bit b of tokmask[k] is token b's membership."""
    rng = np.random.Generator(np.random.PCG64(14))
    for B in (1, 2, 7, 33, 64):
        M = (rng.random((B, 150)) < 0.08).astype(np.uint8)
        idx, k, tok = oracle.compact(M)
        union = np.flatnonzero(M.any(axis=0))
        assert np.array_equal(idx, union) and k == len(union)
        for j, i in enumerate(idx):
            assert int(tok[j]) == sum(int(M[b, i]) << b for b in range(B))


def pin_threshold_strict_nan():
    s = np.array([[0.0, -0.0, 1e-300, -1e-300, np.nan, np.inf, -np.inf, 0.5]])
    assert list(oracle.threshold(s, 0.0)[0]) == [0, 0, 1, 0, 0, 1, 0, 1]
    assert list(oracle.threshold(s, 0.5)[0]) == [0, 0, 0, 0, 0, 1, 0, 0]


def pin_integer_additivity():
    """I7: on integer fixtures F(M1 u M2) = F(M1) + F(M2) - b_o exactly, F(empty) = b_o."""
    from synth import integer_layer
    for gated in (False, True):
        L = integer_layer(20, 40, 4, gated=gated, seed=15, B=3, lo=-1 if gated else -2,
                          hi=1 if gated else 2)
        X = L["x"]
        rng = np.random.Generator(np.random.PCG64(16))
        perm = rng.permutation(40)
        M1, M2 = np.sort(perm[:17]).astype(np.int32), np.sort(perm[17:30]).astype(np.int32)
        kw = dict(Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
        F = lambda M: oracle.forward(X, L["w_a"], L["w_o"], M, **kw)  # noqa: E731
        assert np.array_equal(F(np.union1d(M1, M2).astype(np.int32)), F(M1) + F(M2) - L["b_o"])
        assert np.array_equal(F(np.zeros(0, np.int32)), np.tile(L["b_o"].astype(np.float64), (3, 1)))
        Yn = numpy_dense(X, L["w_a"], L["w_o"], L["w_u"], L["b_a"], L["b_o"])
        assert np.array_equal(F(np.arange(40, dtype=np.int32)), Yn)  # integers: exact in any order


def pin_batch_equals_single():
    """I8: row b of a batched forward equals the single-token forward under token b's mask."""
    rng = np.random.Generator(np.random.PCG64(17))
    for gated in (False, True):
        L, X = float_layer(rng, 24, 80, 4, gated, np.float16, 6)
        Mb = (rng.random((6, 80)) < 0.2).astype(np.uint8)
        idx, k, tok = oracle.compact(Mb)
        kw = dict(Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
        Y = oracle.forward(X, L["w_a"], L["w_o"], idx, tok, **kw)
        for b in range(6):
            yb = oracle.forward(X[b:b + 1], L["w_a"], L["w_o"], np.flatnonzero(Mb[b]).astype(np.int32), **kw)
            assert np.array_equal(Y[b], yb[0]), b


def pin_permutation_invariance():
    """I3: packing rows by a permutation and mapping the mask through it leaves the output
    unchanged (exact on integer fixtures; summation order differs only)."""
    from synth import integer_layer
    rng = np.random.Generator(np.random.PCG64(18))
    for gated in (False, True):
        L = integer_layer(16, 50, 4, gated=gated, seed=19, B=2, lo=-1 if gated else -2, hi=1 if gated else 2)
        counts = rng.integers(0, 30, size=50).astype(np.int64)
        perm = oracle.permutation(counts, 10)
        inv = np.empty(50, np.int64)
        inv[perm] = np.arange(50)
        P = {k: (oracle.pack_rows(L[k], perm) if L[k] is not None else None) for k in ("w_a", "w_u", "w_o", "b_a", "p2", "c")}
        for k in ("w_a", "w_o", "b_a", "c"):
            assert np.array_equal(P[k], L[k][perm])
        M = np.sort(rng.choice(50, 13, replace=False)).astype(np.int32)
        Mp = np.sort(inv[M]).astype(np.int32)
        Y0 = oracle.forward(L["x"], L["w_a"], L["w_o"], M, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
        Y1 = oracle.forward(L["x"], P["w_a"], P["w_o"], Mp, Wu=P["w_u"], b_a=P["b_a"], b_o=L["b_o"])
        assert np.array_equal(Y0, Y1)
        S0 = oracle.predict(L["x"], L["p1"], L["p2"], L["c"])
        S1 = oracle.predict(L["x"], L["p1"], P["p2"], P["c"])
        assert np.array_equal(S1, S0[:, perm])


def pin_full_rank_predictor():
    """I4: r = d, P1 = I, P2 = W_a, c = b_a, tau = 0 makes the predicted mask the true ReLU
    sign mask exactly, and the scores the pre-activations."""
    rng = np.random.Generator(np.random.PCG64(20))
    d, n = 24, 60
    L, X = float_layer(rng, d, n, 4, False, np.float32, 3)
    S = oracle.predict(X, np.eye(d, dtype=np.float32), L["w_a"], L["b_a"])
    A = oracle.preact(X, L["w_a"], L["b_a"])
    assert np.array_equal(S, A)
    assert np.array_equal(oracle.threshold(S, 0.0), (A > 0).astype(np.uint8))
    An = X.astype(np.float64) @ L["w_a"].astype(np.float64).T + L["b_a"]
    assert rel_err(A, An) < 1e-12


def pin_predictor_associativity():
    """Scores equal numpy's (P2 @ P1) @ x + c, a different association and summation order."""
    rng = np.random.Generator(np.random.PCG64(21))
    for (d, n, r, wdt) in [(32, 70, 8, np.float16), (20, 33, 5, np.float32)]:
        L, X = float_layer(rng, d, n, r, False, wdt, 4)
        S, Q = oracle.predict(X, L["p1"], L["p2"], L["c"], return_q=True)
        P1, P2 = L["p1"].astype(np.float64), L["p2"].astype(np.float64)
        ref = X.astype(np.float64) @ (P2 @ P1).T + L["c"]
        assert rel_err(S, ref) < 1e-12
        assert rel_err(Q, X.astype(np.float64) @ P1.T) < 1e-13
        # without c the scores drop exactly the bias term
        assert rel_err(oracle.predict(X, L["p1"], L["p2"]), S - L["c"].astype(np.float64)) < 1e-13


def pin_profile_counts():
    """Profile counts equal numpy's count of positive pre-activations (integer fixture: exact
    pre-activations, so no sign is in doubt)."""
    from synth import integer_layer
    L = integer_layer(16, 45, 4, gated=False, seed=22, B=64)
    c = oracle.profile_counts(L["x"], L["w_a"], L["b_a"])
    A = L["x"].astype(np.float64) @ L["w_a"].astype(np.float64).T + L["b_a"]
    assert np.array_equal(c, (A > 0).sum(axis=0))


def pin_pack_rows():
    rng = np.random.Generator(np.random.PCG64(23))
    for shape, dt in [((30, 7), np.float16), ((30,), np.float32), ((30, 2, 5), np.float16)]:
        src = rng.standard_normal(shape).astype(dt)
        perm = rng.permutation(30).astype(np.int32)
        dst = oracle.pack_rows(src, perm)
        assert np.array_equal(dst, src[perm])
        inv = np.empty(30, np.int32)
        inv[perm] = np.arange(30)
        assert np.array_equal(oracle.pack_rows(dst, inv), src)


def pin_round_half_ieee():
    """binary16 rounding equals numpy's IEEE 754 conversion (a library routine: nearest,
    ties to even) on random magnitudes over the normal and subnormal ranges, on exact ties
    in every binade and among the subnormals, and at the overflow boundary (65504 stays,
    65520 and above go to infinity), for both signs."""
    rng = np.random.Generator(np.random.PCG64(31))
    v = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.uniform(-30.0, 17.0, 20000)),
        # ties: (m + 1/2) spacings in binade [2^e, 2^(e+1)), spacing 2^(e-10)
        np.array([(2 * m + 1) * 2.0 ** (e - 11) for e in range(-14, 16) for m in (1024, 1500, 2045)]),
        # ties among the subnormals (spacing 2^-24)
        np.array([(2 * k + 1) * 2.0 ** -25 for k in range(0, 1024, 37)]),
        np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e300, 2.0 ** -25, 2.0 ** -26, 0.0]),
    ])
    v = np.concatenate([v, -v])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).astype(np.float64)
    got = oracle.round_half(v)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:5]


def pin_dense_f16act_exact_inputs():
    """With every x and every h exactly representable in binary16 (small integers, |h| <
    2048), both roundings are identities and the fp16-activation dense FFN equals the dense
    FFN bit for bit."""
    rng = np.random.Generator(np.random.PCG64(32))
    for gated, d, n, B in ((False, 24, 40, 3), (True, 8, 33, 2)):
        Wa = rng.integers(-1, 2, (n, d)).astype(np.float16)
        Wu = rng.integers(-1, 2, (n, d)).astype(np.float16) if gated else None
        Wo = rng.integers(-2, 3, (n, d)).astype(np.float16)
        X = rng.integers(-2, 3, (B, d)).astype(np.float32)
        b_a = rng.integers(-3, 4, n).astype(np.float32)
        b_o = rng.integers(-3, 4, d).astype(np.float32)
        g = X.astype(np.float64) @ Wa.astype(np.float64).T + b_a
        h = np.maximum(g, 0.0) * (X.astype(np.float64) @ Wu.astype(np.float64).T if gated else 1.0)
        assert np.abs(h).max() < 2048 and np.any(h != 0)
        Y = oracle.dense(X, Wa, Wo, Wu=Wu, b_a=b_a, b_o=b_o)
        Yf = oracle.dense_f16act(X, Wa, Wo, Wu=Wu, b_a=b_a, b_o=b_o)
        assert np.array_equal(Y, Yf)


def pin_dense_f16act_rounds_x_and_h():
    """Each rounding alone, on a one-neuron layer with unit weights. x = 1 + 2^-11 lies
    halfway between 1 and 1 + 2^-10 and enters the product as 1 (ties to even); x = 1 +
    3 2^-11 enters as 1 + 2^-9. With x = 0 and b_act = 2049 (halfway between 2048 and 2050)
    h enters the down product as 2048; with 2051, as 2052. The dense FFN keeps them all."""
    W = np.ones((1, 1), np.float16)
    X = np.array([[1 + 2.0 ** -11], [1 + 3 * 2.0 ** -11]], np.float32)
    assert np.array_equal(oracle.dense_f16act(X, W, W), [[1.0], [1 + 2.0 ** -9]])
    assert np.array_equal(oracle.dense(X, W, W), X.astype(np.float64))
    # the x rounding where h's cannot hide it: W_act = (1, -1), x = (1 + 2^-11, 1) gives
    # h = 0 from the rounded x but 2^-11 (exact in binary16) from x as given
    Wa2 = np.array([[1.0, -1.0]], np.float16)
    Wo2 = np.ones((1, 2), np.float16)
    X2 = np.array([[1 + 2.0 ** -11, 1.0]], np.float32)
    assert np.array_equal(oracle.dense_f16act(X2, Wa2, Wo2), [[0.0, 0.0]])
    assert np.array_equal(oracle.dense(X2, Wa2, Wo2), [[2.0 ** -11, 2.0 ** -11]])
    X0 = np.zeros((1, 1), np.float32)
    for b, r in ((2049.0, 2048.0), (2051.0, 2052.0)):
        ba = np.array([b], np.float32)
        assert oracle.dense_f16act(X0, W, W, b_a=ba)[0, 0] == r
        assert oracle.dense(X0, W, W, b_a=ba)[0, 0] == b


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def all_pin_names():
    return [f.__name__ for f in ALL_PINS]


def run_all():
    for f in ALL_PINS:
        f()

