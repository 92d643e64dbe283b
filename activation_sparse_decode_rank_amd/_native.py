"""ctypes binding of libsparse_ffn.so: the C-ABI entry points of include/sparse_ffn.h under
the same names. Arguments are plain integers (device addresses, sizes, a stream handle);
this module only marshals them and turns a non-zero status into SparseFFNError. There is no
fallback: if the HIP library is not built, importing this module raises."""
from __future__ import annotations

import ctypes as C
import os

# torch first: its wheel carries its own HIP runtime, which its libraries load by file
# name. Loaded after this library (which binds the system runtime of the same soname), it
# would be a second runtime in the process, and device memory torch allocates would not be
# valid for this library's launches. Loaded before, this library binds torch's runtime.
import torch  # noqa: F401,E402

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_ffn.so")

SFFN_OK, SFFN_ERR_INVALID, SFFN_ERR_UNSUPPORTED, SFFN_ERR_HIP, SFFN_ERR_TOO_LARGE = 0, -1, -2, -3, -4
SFFN_STATIC_SCRATCH_BYTES = 16 << 20
SFFN_F32, SFFN_F16 = 0, 1
SFFN_LAYOUT_SPLIT, SFFN_LAYOUT_BUNDLE = 0, 1
SFFN_UP_ROWS, SFFN_UP_COLUMNS = 0, 1
SFFN_PREFILL_FP16_ACT = 1
SFFN_MAX_BATCH = 64


class SffnDesc(C.Structure):
    _fields_ = [
        ("d", C.c_int32), ("d_ffn", C.c_int32), ("rank", C.c_int32), ("max_batch", C.c_int32),
        ("gated", C.c_int32), ("w_dtype", C.c_int32), ("p_dtype", C.c_int32),
        ("threshold", C.c_float),
        ("w_act", C.c_void_p), ("w_down_t", C.c_void_p), ("b_act", C.c_void_p),
        ("b_out", C.c_void_p), ("p1", C.c_void_p), ("p2", C.c_void_p), ("p_bias", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
        ("neuron_freq", C.c_void_p),
        ("deterministic", C.c_int32),
        ("layout", C.c_int32), ("single_pass", C.c_int32), ("dense_union", C.c_float),
    ]


class SparseFFNError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {sparse_ffn_status_string(status)} (status {status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: the HIP library is required (run "
            "`python -m activation_sparse_decode_rank_amd.build`); there is no fallback path")
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    sig = {
        "sparse_ffn_workspace_bytes": (SZ, [C.POINTER(SffnDesc)]),
        "sparse_ffn_create": (C.c_int, [C.POINTER(SffnDesc), C.POINTER(P)]),
        "sparse_ffn_destroy": (C.c_int, [P]),
        "sparse_ffn_predict": (C.c_int, [P, P, I32, P, P]),
        "sparse_ffn_compact": (C.c_int, [P, P, I32, P, P, P, P]),
        "sparse_ffn_forward": (C.c_int, [P, P, I32, P, P, P, P, P]),
        "sparse_ffn_decode": (C.c_int, [P, P, I32, P, P, P, P, P, P]),
        "sparse_ffn_decode_static": (C.c_int, [P, P, I32, P, P, P, P, P, P]),
        "sparse_ffn_dense": (C.c_int, [P, P, I32, P, P]),
        "sparse_ffn_lookahead_begin": (C.c_int, [P, P, P]),
        "sparse_ffn_decode_lookahead": (C.c_int, [P, P, P, P, P, P, P, P]),
        "sparse_ffn_status_string": (C.c_char_p, [C.c_int]),
        "sparse_ffn_set_timing_events": (C.c_int, [P, C.POINTER(P)]),
        "sparse_ffn_profile_counts": (C.c_int, [P, I32, I32, P, I32, I32, P, I32, P, P]),
        "sparse_ffn_permutation": (C.c_int, [P, I32, I32, P]),
        "sparse_ffn_pack_rows": (C.c_int, [P, P, P, I32, I64, I64, P]),
        "sparse_ffn_read_probe": (C.c_int, [P, SZ, I32, P, P]),
        "sparse_ffn_up_probe_work_bytes": (SZ, [I32]),
        "sparse_ffn_prefill_work_bytes": (SZ, [P, I32]),
        "sparse_ffn_prefill": (C.c_int, [P, P, I32, P, P, SZ, P]),
        "sparse_ffn_prefill_ex": (C.c_int, [P, P, I32, P, P, SZ, I32, P]),
        "sparse_ffn_up_probe": (C.c_int, [P, I32, I32, I32, P, P, P, P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("sparse_ffn_workspace_bytes", "sparse_ffn_create", "sparse_ffn_destroy",
            "sparse_ffn_predict", "sparse_ffn_compact", "sparse_ffn_forward", "sparse_ffn_decode",
            "sparse_ffn_decode_static", "sparse_ffn_dense",
            "sparse_ffn_lookahead_begin", "sparse_ffn_decode_lookahead",
            "sparse_ffn_status_string", "sparse_ffn_set_timing_events",
            "sparse_ffn_profile_counts", "sparse_ffn_permutation", "sparse_ffn_pack_rows",
            "sparse_ffn_read_probe", "sparse_ffn_up_probe_work_bytes", "sparse_ffn_up_probe",
            "sparse_ffn_prefill_work_bytes", "sparse_ffn_prefill", "sparse_ffn_prefill_ex")


def lib():
    return _lib


def _ck(status: int, what: str):
    if status != SFFN_OK:
        raise SparseFFNError(status, what)


def sparse_ffn_status_string(status: int) -> str:
    return _lib.sparse_ffn_status_string(int(status)).decode()


def sparse_ffn_workspace_bytes(desc: SffnDesc) -> int:
    return int(_lib.sparse_ffn_workspace_bytes(C.byref(desc)))


def sparse_ffn_create(desc: SffnDesc) -> int:
    h = C.c_void_p()
    _ck(_lib.sparse_ffn_create(C.byref(desc), C.byref(h)), "sparse_ffn_create")
    return int(h.value)


def sparse_ffn_destroy(h: int) -> None:
    _ck(_lib.sparse_ffn_destroy(h), "sparse_ffn_destroy")


def sparse_ffn_predict(h, x, B, scores, stream) -> None:
    _ck(_lib.sparse_ffn_predict(h, x, B, scores, stream), "sparse_ffn_predict")


def sparse_ffn_compact(h, scores, B, idx, count, tokmask, stream) -> None:
    _ck(_lib.sparse_ffn_compact(h, scores, B, idx, count, tokmask, stream), "sparse_ffn_compact")


def sparse_ffn_forward(h, x, B, idx, count, tokmask, y, stream) -> None:
    _ck(_lib.sparse_ffn_forward(h, x, B, idx, count, tokmask, y, stream), "sparse_ffn_forward")


def sparse_ffn_decode(h, x, B, y, idx, count, tokmask, scores, stream) -> None:
    _ck(_lib.sparse_ffn_decode(h, x, B, y, idx, count, tokmask, scores, stream), "sparse_ffn_decode")


def sparse_ffn_dense(h, x, B, y, stream) -> None:
    _ck(_lib.sparse_ffn_dense(h, x, B, y, stream), "sparse_ffn_dense")


def sparse_ffn_decode_static(h, x, B, y, idx, count, tokmask, scores, stream) -> None:
    _ck(_lib.sparse_ffn_decode_static(h, x, B, y, idx, count, tokmask, scores, stream),
        "sparse_ffn_decode_static")


def sparse_ffn_lookahead_begin(h, x, stream) -> None:
    _ck(_lib.sparse_ffn_lookahead_begin(h, x, stream), "sparse_ffn_lookahead_begin")


def sparse_ffn_decode_lookahead(cur, nxt, x, y, idx, count, tokmask, stream) -> None:
    _ck(_lib.sparse_ffn_decode_lookahead(cur, nxt, x, y, idx, count, tokmask, stream),
        "sparse_ffn_decode_lookahead")


def sparse_ffn_set_timing_events(h, events) -> None:
    """events: None or six hipEvent_t handles (ints): a start/end pair per decode kernel."""
    arr = None if events is None else (C.c_void_p * 6)(*events)
    _ck(_lib.sparse_ffn_set_timing_events(h, arr), "sparse_ffn_set_timing_events")


def sparse_ffn_profile_counts(w_act, w_dtype, gated, b_act, d, d_ffn, x, N, counts, stream) -> None:
    _ck(_lib.sparse_ffn_profile_counts(w_act, w_dtype, gated, b_act, d, d_ffn, x, N, counts, stream),
        "sparse_ffn_profile_counts")


def sparse_ffn_permutation(counts_host, d_ffn, n_hot, perm_host) -> None:
    _ck(_lib.sparse_ffn_permutation(counts_host, d_ffn, n_hot, perm_host), "sparse_ffn_permutation")


def sparse_ffn_pack_rows(src, perm, dst, rows, row_bytes, dst_stride_bytes, stream) -> None:
    _ck(_lib.sparse_ffn_pack_rows(src, perm, dst, rows, row_bytes, dst_stride_bytes, stream),
        "sparse_ffn_pack_rows")


def sparse_ffn_read_probe(buf, nbytes, workgroups, sink, stream) -> None:
    _ck(_lib.sparse_ffn_read_probe(buf, nbytes, workgroups, sink, stream), "sparse_ffn_read_probe")


def sparse_ffn_prefill_work_bytes(handle, chunk_tokens) -> int:
    return int(_lib.sparse_ffn_prefill_work_bytes(handle, chunk_tokens))


def sparse_ffn_prefill(handle, x, B, y, work, work_bytes, stream) -> None:
    _ck(_lib.sparse_ffn_prefill(handle, x, B, y, work, work_bytes, stream), "sparse_ffn_prefill")


def sparse_ffn_prefill_ex(handle, x, B, y, work, work_bytes, flags, stream) -> None:
    _ck(_lib.sparse_ffn_prefill_ex(handle, x, B, y, work, work_bytes, flags, stream),
        "sparse_ffn_prefill_ex")


def sparse_ffn_up_probe_work_bytes(d_ffn) -> int:
    return int(_lib.sparse_ffn_up_probe_work_bytes(d_ffn))


def sparse_ffn_up_probe(w_up, layout, d, d_ffn, x, idx, count, words, u, work, work_bytes,
                        stream) -> None:
    _ck(_lib.sparse_ffn_up_probe(w_up, layout, d, d_ffn, x, idx, count, words, u, work,
                                 work_bytes, stream), "sparse_ffn_up_probe")
