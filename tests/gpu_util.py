"""Shared helpers of the GPU parity tests: build a layer from the seeded generator, hand the
same bytes to the HIP path (through the C ABI) and to the fp64 oracle, and compare."""
import sys

import numpy as np
import torch

import oracle

BAND = 1e-4    # predictor scores this close to the threshold may fall either way
REL_TOL = 1e-3  # max |y - y_ref| / max |y_ref| per token vector (fp16 weights, fp32 accumulation)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_np(t):
    return None if t is None else t.detach().cpu().numpy()


def rel_err_rows(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    out = []
    for b in range(ref.shape[0]):
        den = max(np.max(np.abs(ref[b])), 1e-30)
        out.append(float(np.max(np.abs(y[b] - ref[b])) / den))
    return out


def build(cfg, layer=0, *, d=None, n=None, rank=None, activity=None, max_batch=1,
          nonzero_b_o=True, profile_tokens=256, hot_frac=None, threshold=0.0, pack=True,
          gen_device="cuda", deterministic=True, bundle=False, single_pass=False):
    """Generate a layer (original order) and a SparseFFN over it; returns (sffn, L_np, Lt).
    deterministic defaults to the library's own default (True)."""
    from activation_sparse_decode_rank_amd import SparseFFN
    from synth import make_layer, make_tokens
    Lt = make_layer(cfg, layer, gen_device, nonzero_b_o=nonzero_b_o, d=d, n=n, rank=rank,
                    activity=activity).to("cuda")
    dd = Lt.w_a.shape[1]
    Xp = make_tokens(cfg, profile_tokens, 100, "cuda", d=dd) if pack else None
    s = SparseFFN(w_act=Lt.w_a, w_up=Lt.w_u, w_down_t=Lt.w_o, p1=Lt.p1, p2=Lt.p2, b_act=Lt.b_a,
                  b_out=Lt.b_o, p_bias=Lt.c, threshold=threshold, max_batch=max_batch,
                  profile_x=Xp, hot_frac=cfg.hot_frac if hot_frac is None else hot_frac,
                  deterministic=deterministic, bundle=bundle, single_pass=single_pass)
    torch.cuda.synchronize()
    return s, Lt.numpy(), Lt


def oracle_pipeline(L, X, tau=0.0):
    """Oracle scores, mask, (original-order) list, tokmask, output under its own mask."""
    S = oracle.predict(X, L["p1"], L["p2"], L["c"])
    M = oracle.threshold(S, tau)
    idx, k, tok = oracle.compact(M)
    Y = oracle.forward(X, L["w_a"], L["w_o"], idx, tok, Wu=L["w_u"], b_a=L["b_a"], b_o=L["b_o"])
    return S, M, idx, tok, Y


def gpu_mask_orig(perm, idx, count, tokmask, B, n):
    """Per-token masks [B, n] in original neuron order from the HIP path's packed list."""
    k = int(count)
    idx = np.asarray(idx[:k], np.int64)
    tok = np.asarray(tokmask[:k]).astype(np.uint64)
    M = np.zeros((B, n), np.uint8)
    for b in range(B):
        sel = ((tok >> np.uint64(b)) & np.uint64(1)).astype(bool)
        M[b, perm[idx[sel]]] = 1
    return M


def check_mask(Mg, S, tau=0.0):
    """The HIP mask must equal the oracle's everywhere outside the score band; returns the
    mask to use for output parity (oracle decisions outside the band, HIP decisions inside,
    where either decision is correct) and the number of band neurons."""
    Mo = (S > tau).astype(np.uint8)
    band = np.abs(S - tau) < BAND
    bad = (Mg != Mo) & ~band
    assert not bad.any(), f"{int(bad.sum())} mask mismatches outside the band"
    M = np.where(band, Mg, Mo).astype(np.uint8)
    return M, int(band.sum())
