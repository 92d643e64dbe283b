"""SparseFFN: one activation-sparse FFN layer held in device memory, prepared offline and
called through the C ABI. torch supplies device memory and the current stream; every step
of the method (profile counts, permutation, row packing, predict, compact, forward) runs in
the library.

Offline preparation (unite.ai PowerInfer overview, "Fase fuera de línea" and "Colocación y
gestión de neuronas"): activation counts over profiling tokens -> hot-first permutation ->
rows packed in that order; `perm[p]` maps packed position p back to the original neuron.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from . import _native as N

_DT = {torch.float16: N.SFFN_F16, torch.float32: N.SFFN_F32}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def n_hot_for(n: int, hot_frac: float) -> int:
    return int(math.ceil(float(hot_frac) * n))


def profile_counts(w_act: torch.Tensor, b_act: Optional[torch.Tensor], x: torch.Tensor,
                   gated: bool = False, stream=None) -> torch.Tensor:
    """counts[i] (int64, device) = #profiling tokens with w_act[i] . x + b_act[i] > 0.
    For gated layers pass the gate matrix [n, d] (gated=False) or a bundle (gated=True)."""
    n = w_act.shape[0]
    d = x.shape[1]
    counts = torch.empty(n, dtype=torch.int64, device=w_act.device)
    N.sparse_ffn_profile_counts(_ptr(w_act), _DT[w_act.dtype], int(gated), _ptr(b_act), d, n,
                                _ptr(x), x.shape[0], _ptr(counts), _stream(stream))
    return counts


def permutation(counts: np.ndarray, n_hot: int) -> np.ndarray:
    """perm[new] = old, hot-first (host)."""
    counts = np.ascontiguousarray(counts, dtype=np.int64)
    perm = np.empty(counts.shape[0], np.int32)
    N.sparse_ffn_permutation(counts.ctypes.data, counts.shape[0], int(n_hot), perm.ctypes.data)
    return perm


def pack_rows(src: torch.Tensor, perm_dev: torch.Tensor, dst: Optional[torch.Tensor] = None,
              dst_offset_bytes: int = 0, dst_stride_bytes: int = 0, stream=None) -> torch.Tensor:
    """Row gather copy on the device: dst row i = src row perm[i]."""
    rows = src.shape[0]
    row_bytes = src.numel() * src.element_size() // rows
    if dst is None:
        dst = torch.empty_like(src)
    N.sparse_ffn_pack_rows(_ptr(src), _ptr(perm_dev), dst.data_ptr() + dst_offset_bytes, rows,
                           row_bytes, dst_stride_bytes, _stream(stream))
    return dst


class SparseFFN:
    """An FFN layer in packed order with a library handle.

    w_act: [n, d] W_up (plain) or W_gate (gated); w_up: [n, d] for the gated form, else None;
    w_down_t: [n, d] W_down transposed; p1: [r, d]; p2: [n, r]; biases fp32.
    profile_x: [N, d] fp32 profiling tokens; when given, neurons are profiled and the
    hottest ceil(hot_frac * n) packed first, and their frequencies balance the work split.
    deterministic: keep y bitwise reproducible from run to run (the default: the down
    projection's splits are summed in a fixed order); False lets them add into y with float
    atomics, a few percent faster, and y may then vary in the last bits.
    bundle: store each neuron's rows together ([gate,] up, down: one [n, m, d] tensor, the
    PowerInfer-2 neuron bundle) instead of separate matrices.
    single_pass: the single-token decode gathers each active neuron's input and down rows in
    one pass and adds the workgroups' partial outputs in a fixed order (y bitwise
    reproducible); shapes it does not cover fall back to the three-launch path.
    dense_union: decode computes every neuron (the dense FFN, no predictor) from the batch
    size whose expected union of predicted sets exceeds this fraction (0: never; needs the
    profile).
    """

    def __init__(self, *, w_act, w_down_t, p1, p2, b_act=None, b_out=None, p_bias=None,
                 w_up=None, threshold: float = 0.0, max_batch: int = 1,
                 profile_x: Optional[torch.Tensor] = None, hot_frac: float = 0.2,
                 perm: Optional[np.ndarray] = None, deterministic: bool = True,
                 bundle: bool = False, single_pass: bool = False, dense_union: float = 0.0,
                 stream=None):
        dev = w_act.device
        if dev.type != "cuda":
            raise ValueError("SparseFFN needs device tensors")
        for t in (w_act, w_down_t, p1, p2, w_up, b_act, b_out, p_bias, profile_x):
            if t is not None and not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
        n, d = w_act.shape
        r = p1.shape[0]
        self.n, self.d, self.r = n, d, r
        self.gated = w_up is not None
        self.max_batch = int(max_batch)
        self.threshold = float(threshold)
        s = _stream(stream)

        freq = None
        if perm is None and profile_x is not None:
            counts = profile_counts(w_act, b_act, profile_x, gated=False, stream=stream)
            counts_h = counts.cpu().numpy()
            perm = permutation(counts_h, n_hot_for(n, hot_frac))
            freq = (counts_h[perm] / float(profile_x.shape[0])).astype(np.float32)
            self.profile_counts = counts_h
        elif perm is None:
            perm = np.arange(n, dtype=np.int32)
        self.perm = np.ascontiguousarray(perm, dtype=np.int32)
        perm_dev = torch.from_numpy(self.perm).to(dev)

        # packed copies, made by the library's row-gather kernel
        eb = w_act.element_size()
        self.bundle = bool(bundle)
        if self.bundle:
            # neuron i's rows side by side: [gate,] up, down
            rows = [w_act, w_up, w_down_t] if self.gated else [w_act, w_down_t]
            m = len(rows)
            self.w_act = torch.empty((n, m, d), dtype=w_act.dtype, device=dev)
            for k, src in enumerate(rows):
                pack_rows(src, perm_dev, self.w_act, k * d * eb, m * d * eb, stream)
            self.w_down_t = None
        else:
            if self.gated:
                self.w_act = torch.empty((n, 2, d), dtype=w_act.dtype, device=dev)
                pack_rows(w_act, perm_dev, self.w_act, 0, 2 * d * eb, stream)
                pack_rows(w_up, perm_dev, self.w_act, d * eb, 2 * d * eb, stream)
            else:
                self.w_act = pack_rows(w_act, perm_dev, stream=stream)
            self.w_down_t = pack_rows(w_down_t, perm_dev, stream=stream)
        self.single_pass = bool(single_pass)
        self.dense_union = float(dense_union)
        self.p2 = pack_rows(p2, perm_dev, stream=stream)
        self.b_act = None if b_act is None else pack_rows(b_act.contiguous(), perm_dev, stream=stream)
        self.p_bias = None if p_bias is None else pack_rows(p_bias.contiguous(), perm_dev, stream=stream)
        self.p1 = p1
        self.b_out = b_out
        torch.cuda.current_stream(dev).synchronize() if stream is None else stream.synchronize()

        self._w_dtype, self._p_dtype = _DT[w_act.dtype], _DT[p1.dtype]
        self._freq = freq  # host frequencies: read by every create over these weights
        self.perm_dev = perm_dev
        self._create(self.threshold, bool(deterministic), self.max_batch)

    def _create(self, threshold: float, deterministic: bool, max_batch: int) -> None:
        """A library handle over this object's packed weights, with its own workspace."""
        self.threshold = float(threshold)
        self.deterministic = bool(deterministic)
        self.max_batch = int(max_batch)
        self.desc = N.SffnDesc()
        D = self.desc
        D.d, D.d_ffn, D.rank, D.max_batch = self.d, self.n, self.r, self.max_batch
        D.gated = int(self.gated)
        D.w_dtype, D.p_dtype = self._w_dtype, self._p_dtype
        D.threshold = self.threshold
        D.deterministic = int(self.deterministic)
        D.layout = N.SFFN_LAYOUT_BUNDLE if self.bundle else N.SFFN_LAYOUT_SPLIT
        D.single_pass = int(self.single_pass)
        D.dense_union = self.dense_union
        D.w_act, D.w_down_t = _ptr(self.w_act), _ptr(self.w_down_t)
        D.b_act, D.b_out = _ptr(self.b_act), _ptr(self.b_out)
        D.p1, D.p2, D.p_bias = _ptr(self.p1), _ptr(self.p2), _ptr(self.p_bias)
        ws = N.sparse_ffn_workspace_bytes(D)
        if ws == 0:
            raise N.SparseFFNError(N.SFFN_ERR_INVALID, "sparse_ffn_workspace_bytes")
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.w_act.device)
        D.workspace, D.workspace_bytes = self.workspace.data_ptr(), ws
        D.neuron_freq = None if self._freq is None else self._freq.ctypes.data
        self.handle = N.sparse_ffn_create(D)
        D.neuron_freq = None

    def clone(self, *, threshold: Optional[float] = None, deterministic: Optional[bool] = None,
              max_batch: Optional[int] = None, single_pass: Optional[bool] = None,
              dense_union: Optional[float] = None) -> "SparseFFN":
        """Another handle over the same packed weights (no copy), with its own workspace and
        the given threshold, mode or batch limit (default: this layer's). For example
        threshold=-inf lists every neuron: the library's own dense FFN."""
        c = object.__new__(SparseFFN)
        c.__dict__.update({k: v for k, v in self.__dict__.items()
                           if k not in ("handle", "desc", "workspace")})
        if single_pass is not None:
            c.single_pass = bool(single_pass)
        if dense_union is not None:
            c.dense_union = float(dense_union)
        c._create(self.threshold if threshold is None else threshold,
                  self.deterministic if deterministic is None else deterministic,
                  self.max_batch if max_batch is None else max_batch)
        return c

    # ---------------------------------------------------------------- calls
    def _check_x(self, x):
        if x.dtype != torch.float32 or not x.is_contiguous() or x.dim() != 2 or x.shape[1] != self.d:
            raise ValueError("x must be a contiguous fp32 [B, d] device tensor")
        B = x.shape[0]
        if not 1 <= B <= self.max_batch:
            raise ValueError(f"batch {B} outside 1..{self.max_batch}")
        return B

    def predict(self, x, scores=None, stream=None):
        B = self._check_x(x)
        if scores is None:
            scores = torch.empty((B, self.n), dtype=torch.float32, device=x.device)
        N.sparse_ffn_predict(self.handle, x.data_ptr(), B, scores.data_ptr(), _stream(stream))
        return scores

    def compact(self, scores, idx=None, count=None, tokmask=None, stream=None):
        B = scores.shape[0]
        dev = scores.device
        idx = torch.empty(self.n, dtype=torch.int32, device=dev) if idx is None else idx
        count = torch.empty(1, dtype=torch.int32, device=dev) if count is None else count
        if tokmask is None:
            tokmask = torch.empty(self.n, dtype=torch.int64, device=dev)
        N.sparse_ffn_compact(self.handle, scores.data_ptr(), B, idx.data_ptr(), count.data_ptr(),
                             tokmask.data_ptr(), _stream(stream))
        return idx, count, tokmask

    def forward(self, x, idx, count, tokmask=None, y=None, stream=None):
        B = self._check_x(x)
        if y is None:
            y = torch.empty((B, self.d), dtype=torch.float32, device=x.device)
        N.sparse_ffn_forward(self.handle, x.data_ptr(), B, idx.data_ptr(), count.data_ptr(),
                             _ptr(tokmask), y.data_ptr(), _stream(stream))
        return y

    def decode(self, x, y=None, idx=None, count=None, tokmask=None, scores=None, stream=None):
        B = self._check_x(x)
        dev = x.device
        y = torch.empty((B, self.d), dtype=torch.float32, device=dev) if y is None else y
        idx = torch.empty(self.n, dtype=torch.int32, device=dev) if idx is None else idx
        count = torch.empty(1, dtype=torch.int32, device=dev) if count is None else count
        if tokmask is None:
            tokmask = torch.empty(self.n, dtype=torch.int64, device=dev)
        N.sparse_ffn_decode(self.handle, x.data_ptr(), B, y.data_ptr(), idx.data_ptr(),
                            count.data_ptr(), tokmask.data_ptr(), _ptr(scores), _stream(stream))
        return y, idx, count, tokmask

    def dense(self, x, y=None, stream=None):
        """The dense FFN over every neuron for x ([B, d] fp32, any B: prefill), no predictor
        (sparse_ffn_dense)."""
        if x.dtype != torch.float32 or not x.is_contiguous() or x.dim() != 2 or x.shape[1] != self.d:
            raise ValueError("x must be a contiguous fp32 [B, d] device tensor")
        B = x.shape[0]
        if y is None:
            y = torch.empty((B, self.d), dtype=torch.float32, device=x.device)
        N.sparse_ffn_dense(self.handle, x.data_ptr(), B, y.data_ptr(), _stream(stream))
        return y

    def prefill_work(self, chunk=512):
        """Scratch for prefill in chunks of `chunk` tokens (a uint8 device tensor), or None
        when the layer has no matrix-core prefill (fp32 weights, or d not a multiple of 128)."""
        nb = N.sparse_ffn_prefill_work_bytes(self.handle, int(chunk))
        if nb == 0:
            return None
        return torch.empty(nb, dtype=torch.uint8, device=self.w_act.device)

    def prefill(self, x, y=None, work=None, stream=None, fp16_activations=False):
        """The dense FFN over every neuron for x ([B, d] fp32, any B) on the matrix cores with
        the weights reused across 128-token tiles (sparse_ffn_prefill_ex); layers it does not
        cover take sparse_ffn_dense. work: scratch from prefill_work (allocated here when
        None). fp16_activations: round x and h to fp16 once and run each product once
        (SFFN_PREFILL_FP16_ACT) instead of as an fp16 hi + lo pair."""
        if x.dtype != torch.float32 or not x.is_contiguous() or x.dim() != 2 or x.shape[1] != self.d:
            raise ValueError("x must be a contiguous fp32 [B, d] device tensor")
        B = x.shape[0]
        if y is None:
            y = torch.empty((B, self.d), dtype=torch.float32, device=x.device)
        if work is None:
            work = self.prefill_work(min(max(B, 1), 512))
        if work is None:
            N.sparse_ffn_dense(self.handle, x.data_ptr(), B, y.data_ptr(), _stream(stream))
            return y
        N.sparse_ffn_prefill_ex(self.handle, x.data_ptr(), B, y.data_ptr(), work.data_ptr(),
                                work.numel(), N.SFFN_PREFILL_FP16_ACT if fp16_activations else 0,
                                _stream(stream))
        return y

    def lookahead_begin(self, x, stream=None):
        """Predict this layer's active set from x ([1, d] fp32) and hold it for
        decode_ahead (sparse_ffn_lookahead_begin)."""
        if self._check_x(x) != 1:
            raise ValueError("the look-ahead decode takes one token")
        N.sparse_ffn_lookahead_begin(self.handle, x.data_ptr(), _stream(stream))

    def decode_ahead(self, x, nxt=None, y=None, idx=None, count=None, tokmask=None, stream=None):
        """This layer on x ([1, d] fp32) over the set held from lookahead_begin or from the
        previous layer's decode_ahead, predicting nxt's set from x when nxt (the next
        SparseFFN) is given (sparse_ffn_decode_lookahead). Returns y, idx, count, tokmask."""
        if self._check_x(x) != 1:
            raise ValueError("the look-ahead decode takes one token")
        dev = x.device
        y = torch.empty((1, self.d), dtype=torch.float32, device=dev) if y is None else y
        idx = torch.empty(self.n, dtype=torch.int32, device=dev) if idx is None else idx
        count = torch.empty(1, dtype=torch.int32, device=dev) if count is None else count
        N.sparse_ffn_decode_lookahead(self.handle, nxt.handle if nxt is not None else None,
                                      x.data_ptr(), y.data_ptr(), idx.data_ptr(),
                                      count.data_ptr(), _ptr(tokmask), _stream(stream))
        return y, idx, count, tokmask

    def close(self):
        if getattr(self, "handle", None):
            N.sparse_ffn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LookaheadBuffers:
    """Per-layer device buffers of a look-ahead decode: scores [B, n], the active list
    (idx, count, tokmask) and the output y [B, d] of every layer."""

    def __init__(self, layers, B: int, device="cuda"):
        self.B = int(B)
        self.scores = [torch.empty((B, s.n), dtype=torch.float32, device=device) for s in layers]
        self.idx = [torch.empty(s.n, dtype=torch.int32, device=device) for s in layers]
        self.count = torch.zeros(len(layers), dtype=torch.int32, device=device)
        self.tokmask = [torch.empty(s.n, dtype=torch.int64, device=device) for s in layers]
        self.y = [torch.empty((B, s.d), dtype=torch.float32, device=device) for s in layers]


def decode_lookahead(layers, xs, bufs: LookaheadBuffers, stream=None, side_stream=None):
    """Look-ahead ("asynchronous") decode through a stack of layers (novita.ai
    activation-sparsity article, section 上下文稀疏性: the next layer's sparsity is
    predicted ahead of time, off the critical path).

    Layer 0's active set comes from its own input xs[0]; layer l >= 1's from the previous
    layer's input xs[l - 1], through layer l's own predictor. Its predict and compact run
    on side_stream while layer l - 1's forward runs on stream, so the critical path of a
    layer is its forward alone (once the side stream keeps up). Output: bufs.y[l] =
    forward of layer l on xs[l] over that active set. Only host scheduling happens here:
    every step is a C-ABI call (predict, compact, forward) on the given streams, ordered
    with events:
      - the side stream starts layer l + 1's prediction once the stream has reached layer
        l's forward (xs[l] is ready there; in a model it is the previous layer's output);
      - the stream waits for layer l + 1's list before layer l + 1's forward, so the side
        work of a call ends inside it (graph capture sees a fork and a join).
    A layer's handle is used by one stream at a time, and a call reuses its buffers only
    after the previous call's stream work on them."""
    main = stream if stream is not None else torch.cuda.current_stream()
    side = side_stream
    if side is None:
        raise ValueError("decode_lookahead needs a side stream")
    L = len(layers)
    if len(xs) != L:
        raise ValueError("one input per layer")

    def predict_list(l, x, s):
        layers[l].predict(x, scores=bufs.scores[l], stream=s)
        layers[l].compact(bufs.scores[l], idx=bufs.idx[l], count=bufs.count[l:l + 1],
                          tokmask=bufs.tokmask[l], stream=s)

    predict_list(0, xs[0], main)
    for l in range(L):
        if l + 1 < L:
            ready = torch.cuda.Event()
            ready.record(main)
            side.wait_event(ready)
            predict_list(l + 1, xs[l], side)
            listed = torch.cuda.Event()
            listed.record(side)
        layers[l].forward(xs[l], bufs.idx[l], bufs.count[l:l + 1], tokmask=bufs.tokmask[l],
                          y=bufs.y[l], stream=main)
        if l + 1 < L:
            main.wait_event(listed)
    return bufs.y


def decode_lookahead_fused(layers, xs, bufs: LookaheadBuffers, stream=None):
    """The look-ahead decode of decode_lookahead for one token, in two launches a layer on
    one stream (sparse_ffn_lookahead_begin, then sparse_ffn_decode_lookahead per layer):
    the next layer's prediction shares the launches of the current layer's gather and
    down projection instead of running on a second stream. Same sets and outputs:
    bufs.y[l] = layer l on xs[l] over the set its predictor gives for xs[l - 1] (layer 0:
    xs[0]); bufs.idx / count / tokmask hold each layer's list."""
    main = stream if stream is not None else torch.cuda.current_stream()
    L = len(layers)
    if len(xs) != L:
        raise ValueError("one input per layer")
    if bufs.B != 1:
        raise ValueError("the fused look-ahead decode takes one token")
    layers[0].lookahead_begin(xs[0], stream=main)
    for l in range(L):
        layers[l].decode_ahead(xs[l], layers[l + 1] if l + 1 < L else None, y=bufs.y[l],
                               idx=bufs.idx[l], count=bufs.count[l:l + 1],
                               tokmask=bufs.tokmask[l], stream=main)
    return bufs.y
