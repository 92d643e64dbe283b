"""Importing the package before torch. The library has to bind the HIP runtime that torch
uses: torch's wheel carries its own copy, and with two runtimes in one process the
library's launches on torch's memory fail. A fresh process imports the package first, then
builds and decodes a small gated layer."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, %r)
import activation_sparse_decode_rank_amd as P  # before torch
import torch
from synth import get_config, make_layer, make_tokens
torch.cuda.set_device(0)
cfg = get_config("C3")
Lt = make_layer(cfg, 0, "cuda", d=512, n=1100, rank=64)
Xp = make_tokens(cfg, 256, 100, "cuda", d=512)
s = P.SparseFFN(w_act=Lt.w_a, w_up=Lt.w_u, w_down_t=Lt.w_o, p1=Lt.p1, p2=Lt.p2, b_act=Lt.b_a,
                b_out=Lt.b_o, p_bias=Lt.c, max_batch=2, profile_x=Xp, hot_frac=cfg.hot_frac)
y, idx, count, tok = s.decode(make_tokens(cfg, 2, 200, "cuda", d=512))
torch.cuda.synchronize()
k = int(count.item())
assert 0 < k <= 1100 and bool(torch.isfinite(y).all()), (k,)
print("decode ok", k, flush=True)
""" % ROOT


@pytest.mark.gpu
def test_package_imported_before_torch():
    r = subprocess.run([sys.executable, "-c", SCRIPT], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout[-1000:] + r.stderr[-3000:]
    assert "decode ok" in r.stdout
