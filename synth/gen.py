"""Seeded generation of layers, predictors and tokens.

Recipe (every input is synthetic; no dataset or trained model is used):
  - weights ~ N(0, 0.02^2), drawn in fp32 from a torch generator seeded by
    (config id, layer, matrix id) and rounded once to the storage dtype;
  - per-neuron activation frequencies follow Zipf(s) over a seeded permutation of the
    neurons, scaled so their mean is the layer's target activity (power-law hot/cold
    neurons, unite.ai PowerInfer overview, introduction);
  - the bias inside the ReLU is set so each neuron's pre-activation is positive with its
    target frequency under the token distribution (a central-limit approximation; realized
    frequencies are measured by the tests, not assumed);
  - the predictor is a calibrated random-subspace predictor: P1 has r orthonormal rows, P2
    is W_a projected onto them, and c is set like the bias so predicted frequencies follow
    the same Zipf law (the pages train predictors on real activations, which needs data
    and weights that are not available).
All arithmetic here is workload calibration, not the decode method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import Config

_TORCH_DTYPE = {"f16": torch.float16, "f32": torch.float32}

# matrix ids inside a layer seed
_M_WA, _M_WU, _M_WO, _M_PERM, _M_P1, _M_BO = 1, 2, 3, 7, 11, 13


def seed_for(cid: int, layer: int, matrix: int) -> int:
    return ((cid * 1_000_003 + layer) * 1009 + matrix) & 0x7FFFFFFFFFFF


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def zipf_targets(n: int, s: float, activity: float) -> np.ndarray:
    """f_k = clip(C (k+1)^-s, 1e-4, 0.99) for ranks k = 0..n-1, C found by bisection so
    that mean(f) equals `activity`."""
    ranks = np.arange(1, n + 1, dtype=np.float64)
    base = ranks ** (-float(s))

    def mean_for(Cc):
        return np.clip(Cc * base, 1e-4, 0.99).mean()

    lo, hi = 0.0, 1.0
    while mean_for(hi) < activity:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mean_for(mid) < activity:
            lo = mid
        else:
            hi = mid
    return np.clip(hi * base, 1e-4, 0.99)


def layer_activity_target(cfg: Config, layer: int) -> float:
    return cfg.layer_activity(layer % cfg.layers)


def _x_moments(x_kind: str):
    """Mean and variance of one token coordinate under the token distribution."""
    if x_kind == "normal":
        return 0.0, 1.0
    if x_kind == "relu_rmsnorm":  # relu of a standard normal
        return 1.0 / math.sqrt(2.0 * math.pi), 0.5 - 1.0 / (2.0 * math.pi)
    raise ValueError(x_kind)


@dataclass
class Layer:
    """One FFN layer in original (unpacked) neuron order. Rows are neurons.

    w_a: [n, d] the ReLU-input matrix (W_up for the plain form, W_gate for the gated form)
    w_u: [n, d] W_up of the gated form, else None
    w_o: [n, d] W_down transposed (row i = neuron i's output weights)
    b_a: [n] fp32 bias inside the ReLU; b_o: [d] fp32 output bias
    p1: [r, d], p2: [n, r], c: [n] fp32 predictor
    freq: [n] fp64 target activation frequency per neuron
    """
    w_a: torch.Tensor
    w_u: Optional[torch.Tensor]
    w_o: torch.Tensor
    b_a: torch.Tensor
    b_o: torch.Tensor
    p1: torch.Tensor
    p2: torch.Tensor
    c: torch.Tensor
    freq: np.ndarray
    tau: float = 0.0

    @property
    def gated(self) -> bool:
        return self.w_u is not None

    def to(self, device) -> "Layer":
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return Layer(mv(self.w_a), mv(self.w_u), mv(self.w_o), mv(self.b_a), mv(self.b_o),
                     mv(self.p1), mv(self.p2), mv(self.c), self.freq, self.tau)

    def numpy(self) -> dict:
        cv = lambda t: None if t is None else t.detach().cpu().numpy()  # noqa: E731
        return dict(w_a=cv(self.w_a), w_u=cv(self.w_u), w_o=cv(self.w_o), b_a=cv(self.b_a),
                    b_o=cv(self.b_o), p1=cv(self.p1), p2=cv(self.p2), c=cv(self.c))


def make_layer(cfg: Config, layer: int, device="cpu", *, nonzero_b_o: bool = False,
               d: Optional[int] = None, n: Optional[int] = None, rank: Optional[int] = None,
               activity: Optional[float] = None) -> Layer:
    """Generate one layer of `cfg` (shape overridable for small test cases) on `device`."""
    d = cfg.d if d is None else d
    n = cfg.n if n is None else n
    r = cfg.rank if rank is None else rank
    act = layer_activity_target(cfg, layer) if activity is None else activity
    wdt, pdt = _TORCH_DTYPE[cfg.w_dtype], _TORCH_DTYPE[cfg.p_dtype]
    dev = torch.device(device)
    cid = cfg.cid

    def normal(shape, matrix):
        g = _gen(dev, seed_for(cid, layer, matrix))
        return torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * 0.02

    w_a = normal((n, d), _M_WA).to(wdt)
    w_u = normal((n, d), _M_WU).to(wdt) if cfg.gated else None
    w_o = normal((n, d), _M_WO).to(wdt)
    b_o = (normal((d,), _M_BO) if nonzero_b_o else torch.zeros(d, device=dev)).to(torch.float32)

    # Zipf frequencies over a seeded permutation of the neurons
    f_rank = zipf_targets(n, cfg.zipf_s, act)
    perm = torch.randperm(n, generator=_gen("cpu", seed_for(cid, layer, _M_PERM))).numpy()
    freq = np.empty(n, np.float64)
    freq[perm] = f_rank
    z = torch.special.ndtri(torch.from_numpy(freq)).to(dev)  # Phi^-1(f_i)

    m_x, v_x = _x_moments(cfg.x_kind)
    wa64 = w_a.to(torch.float64)
    b_a = (math.sqrt(v_x) * wa64.norm(dim=1) * z - m_x * wa64.sum(dim=1)).to(torch.float32)
    del wa64

    # predictor: r orthonormal directions (QR of a seeded Gaussian, fp64 on the host)
    gq = _gen("cpu", seed_for(cid, layer, _M_P1))
    G = torch.randn(d, r, generator=gq, dtype=torch.float64)
    Q, _ = torch.linalg.qr(G)
    p1 = Q.T.contiguous().to(pdt).to(dev)
    p2 = (w_a.to(torch.float32) @ p1.to(torch.float32).T).to(pdt)
    p2_64 = p2.to(torch.float64)
    p1_colsum = p1.to(torch.float64).sum(dim=1)  # P1 @ 1
    c = (math.sqrt(v_x) * p2_64.norm(dim=1) * z - m_x * (p2_64 @ p1_colsum)).to(torch.float32)
    return Layer(w_a, w_u, w_o, b_a, b_o, p1, p2.contiguous(), c, freq)


def make_tokens(cfg: Config, T: int, tag: int, device="cpu", d: Optional[int] = None) -> torch.Tensor:
    """T tokens [T, d] fp32 for `cfg` from seed tag `tag` (profile set 100, timed set 200)."""
    d = cfg.d if d is None else d
    g = _gen(torch.device(device), seed_for(cfg.cid, 10_000 + tag, 0))
    z = torch.randn(T, d, generator=g, device=device, dtype=torch.float32)
    if cfg.x_kind == "normal":
        return z
    # relu(rmsnorm(z)) with unit gain: the second ReLU-fication stage's sparse input
    rms = torch.sqrt((z.double() ** 2).mean(dim=1, keepdim=True) + 1e-6).float()
    return torch.relu(z / rms)


def integer_layer(d: int, n: int, r: int, *, gated: bool, seed: int, lo: int = -2, hi: int = 2,
                  w_dtype=np.float16, p_dtype=np.float16, B: int = 1, x_zero_frac: float = 0.0):
    """A layer and tokens whose entries are small integers, so that every partial sum in
    any order and any of fp16/fp32/fp64 is exact. Returns a dict of numpy arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ri = lambda *s: rng.integers(lo, hi + 1, size=s).astype(np.float64)  # noqa: E731
    out = dict(
        w_a=ri(n, d).astype(w_dtype),
        w_u=ri(n, d).astype(w_dtype) if gated else None,
        w_o=ri(n, d).astype(w_dtype),
        b_a=ri(n).astype(np.float32),
        b_o=ri(d).astype(np.float32),
        p1=ri(r, d).astype(p_dtype),
        p2=ri(n, r).astype(p_dtype),
        c=ri(n).astype(np.float32),
    )
    X = ri(B, d)
    if x_zero_frac > 0:
        X[rng.random((B, d)) < x_zero_frac] = 0.0
    out["x"] = X.astype(np.float32)
    return out
