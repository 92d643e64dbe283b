"""CPU tests of the C-ABI library: it loads without a GPU, exports every function the
public header declares, validates arguments on the host before any HIP call, and its pure
host helper (the hot-first permutation) matches the hand-worked fixture and the oracle."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from golden_io import ints, read

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_ffn.h")


@pytest.fixture(scope="module")
def N():
    from activation_sparse_decode_rank_amd import _native
    return _native


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_ffn_\w+)\s*\(", text)))


def test_header_compiles_as_c():
    src = '#include "sparse_ffn.h"\nint main(void){ sffn_desc d; (void)d; return 0; }\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I",
                        os.path.dirname(HEADER), "-x", "c", "-"], input=src, text=True,
                       capture_output=True)
    assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol(N):
    names = declared_functions()
    assert len(names) == 22, names
    lib = C.CDLL(N.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(N.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True,
                         text=True).stdout
    for name in names:
        assert re.search(rf"\bT {name}\b", out), name


def test_desc_layout_matches_header(N):
    # field order and size of the ctypes mirror against the C compiler's view
    src = r'''
#include <stddef.h>
#include <stdio.h>
#include "sparse_ffn.h"
int main(void){
 printf("%zu %zu %zu %zu %zu %zu %zu\n", sizeof(sffn_desc), offsetof(sffn_desc, threshold),
  offsetof(sffn_desc, w_act), offsetof(sffn_desc, workspace), offsetof(sffn_desc, workspace_bytes),
  offsetof(sffn_desc, neuron_freq), offsetof(sffn_desc, deterministic));
 return 0; }
'''
    exe = os.path.join(ROOT, "_build", "desc_layout")
    os.makedirs(os.path.dirname(exe), exist_ok=True)
    r = subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), "-x", "c", "-", "-o", exe],
                       input=src, text=True, capture_output=True)
    assert r.returncode == 0, r.stderr
    got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    D = N.SffnDesc
    assert got == [C.sizeof(D), D.threshold.offset, D.w_act.offset, D.workspace.offset,
                   D.workspace_bytes.offset, D.neuron_freq.offset, D.deterministic.offset]


def _valid_desc(N, **over):
    D = N.SffnDesc()
    D.d, D.d_ffn, D.rank, D.max_batch, D.gated = 64, 100, 16, 4, 0
    D.w_dtype = D.p_dtype = N.SFFN_F16
    D.threshold = 0.0
    fake = 0x10000  # 16-byte aligned, never dereferenced: validation fails first
    D.w_act = D.w_down_t = D.p1 = D.p2 = D.workspace = fake
    for k, v in over.items():
        setattr(D, k, v)
    return D


def test_python_layer_defaults_to_deterministic():
    """The Python layer's default mode keeps y bitwise reproducible (fixed-order joins of
    the down projection's splits, no float atomics into y)."""
    import inspect
    from activation_sparse_decode_rank_amd import SparseFFN
    assert inspect.signature(SparseFFN.__init__).parameters["deterministic"].default is True


def test_workspace_bytes(N):
    D = _valid_desc(N)
    ws = N.sparse_ffn_workspace_bytes(D)
    assert ws > 0
    D2 = _valid_desc(N, max_batch=8)
    assert N.sparse_ffn_workspace_bytes(D2) > ws
    assert N.sparse_ffn_workspace_bytes(_valid_desc(N, d=60)) == 0       # d % 8 != 0
    assert N.sparse_ffn_workspace_bytes(_valid_desc(N, max_batch=65)) == 0


@pytest.mark.parametrize("over", [
    dict(d=0), dict(d_ffn=-1), dict(rank=12), dict(d=36), dict(max_batch=0), dict(max_batch=65),
    dict(gated=2), dict(w_dtype=7), dict(p_dtype=-1), dict(w_act=None), dict(p2=None),
    dict(workspace=None), dict(w_act=0x10004), dict(b_out=0x10008),
    dict(workspace_bytes=16),  # too small
    dict(dense_union=1.5), dict(dense_union=-0.1), dict(dense_union=float("nan")),
    dict(layout=2), dict(single_pass=2), dict(layout=1),  # bundle layout with a w_down_t
])
def test_create_rejects_invalid(N, over):
    D = _valid_desc(N)
    D.workspace_bytes = N.sparse_ffn_workspace_bytes(D)
    for k, v in over.items():
        setattr(D, k, v)
    h = C.c_void_p()
    rc = N.lib().sparse_ffn_create(C.byref(D), C.byref(h))
    assert rc == N.SFFN_ERR_INVALID
    assert h.value is None


def test_calls_reject_null_handle_and_bad_batch(N):
    L = N.lib()
    assert L.sparse_ffn_predict(None, 0x10000, 1, 0x10000, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_compact(None, 0x10000, 1, 0x10000, 0x10000, None, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_forward(None, 0x10000, 1, 0x10000, 0x10000, None, 0x10000, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_decode(None, 0x10000, 1, 0x10000, 0x10000, 0x10000, None, None, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_decode_static(None, 0x10000, 1, 0x10000, 0x10000, 0x10000, None, None,
                                      None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_destroy(None) == N.SFFN_OK
    assert L.sparse_ffn_set_timing_events(None, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_lookahead_begin(None, 0x10000, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_decode_lookahead(None, None, 0x10000, 0x10000, 0x10000, 0x10000, None,
                                         None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_pack_rows(0x10000, 0x10000, 0x10000, 4, 6, 0, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_pack_rows(0x10000, 0x10000, 0x10000, 4, 8, 4, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_profile_counts(None, 1, 0, None, 8, 8, 0x10000, 4, 0x10000, None) == N.SFFN_ERR_INVALID
    # read probe: null buffer or sink, a size that is not a positive multiple of 16, an
    # unaligned buffer, a negative grid
    assert L.sparse_ffn_read_probe(None, 1024, 1, 0x10000, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_read_probe(0x10000, 1024, 1, None, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_read_probe(0x10000, 1000, 1, 0x10000, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_read_probe(0x10000, 0, 1, 0x10000, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_read_probe(0x10008, 1024, 1, 0x10000, None) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_read_probe(0x10000, 1024, -1, 0x10000, None) == N.SFFN_ERR_INVALID
    # prefill: a NULL handle is refused before anything else
    assert L.sparse_ffn_prefill_work_bytes(None, 128) == 0
    assert L.sparse_ffn_prefill(None, 0x10000, 4, 0x10000, 0x10000, 1 << 20, None) == N.SFFN_ERR_INVALID
    for flags in (0, N.SFFN_PREFILL_FP16_ACT, 2, -1):
        assert L.sparse_ffn_prefill_ex(None, 0x10000, 4, 0x10000, 0x10000, 1 << 20, flags,
                                       None) == N.SFFN_ERR_INVALID
    # the input-sparse up probe: every argument check fires before anything is enqueued
    A = 0x10000
    W = L.sparse_ffn_up_probe_work_bytes(1104)
    assert W == 16 * 1104 * 4 and L.sparse_ffn_up_probe_work_bytes(0) == 0
    up = L.sparse_ffn_up_probe
    assert up(None, 0, 512, 1104, A, A, A, None, A, None, 0, None) == N.SFFN_ERR_INVALID
    assert up(A, 2, 512, 1104, A, A, A, A, A, A, W, None) == N.SFFN_ERR_INVALID       # layout
    assert up(A, 0, 500, 1104, A, A, A, None, A, None, 0, None) == N.SFFN_ERR_INVALID  # d % 8
    assert up(A, 0, 512, 1104, A, None, A, None, A, None, 0, None) == N.SFFN_ERR_INVALID
    assert up(A, 0, 512, 1104, A + 8, A, A, None, A, None, 0, None) == N.SFFN_ERR_INVALID
    assert up(A, 1, 512, 1100, A, None, None, A, A, A, W, None) == N.SFFN_ERR_INVALID  # n % 8
    assert up(A, 1, 512, 1104, A, None, None, None, A, A, W, None) == N.SFFN_ERR_INVALID
    assert up(A, 1, 512, 1104, A, None, None, A, A, A, W - 4, None) == N.SFFN_ERR_INVALID
    assert up(A, 1, 512, 1104, A, None, None, A, A, None, W, None) == N.SFFN_ERR_INVALID


def test_status_strings(N):
    assert N.sparse_ffn_status_string(0) == "ok"
    assert "invalid" in N.sparse_ffn_status_string(-1)
    assert "unsupported" in N.sparse_ffn_status_string(-2)
    assert "HIP" in N.sparse_ffn_status_string(-3)
    assert "static scratch" in N.sparse_ffn_status_string(-4)


def test_permutation_hand_fixture(N):
    from activation_sparse_decode_rank_amd import permutation
    g = read("permutation_hand.txt")
    counts = np.array(ints(g["counts"]), np.int64)
    for h in (4, 0, 8, 1):
        assert list(permutation(counts, h)) == ints(g[f"perm_hot{h}"])


def test_permutation_matches_oracle(N):
    from activation_sparse_decode_rank_amd import permutation
    rng = np.random.Generator(np.random.PCG64(5))
    for n, hi in [(1, 3), (97, 5), (3072, 50), (16384, 4096)]:
        counts = rng.integers(0, hi, size=n).astype(np.int64)   # many ties
        for h in (0, 1, n // 5, n):
            assert np.array_equal(permutation(counts, h), oracle.permutation(counts, h))


def test_permutation_rejects(N):
    L = N.lib()
    c = np.zeros(4, np.int64)
    p = np.zeros(4, np.int32)
    assert L.sparse_ffn_permutation(c.ctypes.data, 4, 5, p.ctypes.data) == N.SFFN_ERR_INVALID
    assert L.sparse_ffn_permutation(None, 4, 1, p.ctypes.data) == N.SFFN_ERR_INVALID
