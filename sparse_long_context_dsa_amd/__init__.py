"""Python binding of libdsa.so, the DSA hot path for MI355X (gfx950).

Argument marshalling only: every function below checks dtypes and shapes of the
torch tensors it is given, passes their device pointers and the current HIP
stream to the C function of the same name (include/dsa.h), and raises if it
returns an error.  All arithmetic runs in the library's HIP kernels; PyTorch
only provides device memory and the stream.
"""

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (  # noqa: F401
    DSA_D, DSA_DI, DSA_DV, DSA_H, DSA_HI, DSA_KMAX, DSA_OP_FORWARD, DSA_OP_MLA_DECODE,
    DSA_NOALLOC_SCRATCH_BYTES, DSA_OP_MLA_DENSE, DSA_OP_MLA_PREFILL, DSA_OP_TOPK, DsaError, KvLayoutC, QueriesC,
)

__all__ = [
    "HipEvents", "Queries", "KvLayout", "dsa_quantize_fp8", "dsa_quantize_fp8_e8m0", "dsa_indexer_scores",
    "dsa_indexer_scores_e8m0", "dsa_topk",
    "dsa_sparse_mla_decode", "dsa_sparse_mla_decode_noalloc", "dsa_sparse_mla_prefill", "dsa_dense_mla", "dsa_indexer_kl_sparse",
    "dsa_indexer_kl_dense", "dsa_indexer_backward", "dsa_forward", "dsa_workspace_bytes",
    "workspace", "lib_path",
]


def lib_path():
    return _lib.LIB_PATH


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_device(t):
    return t.is_cuda


def _need(t, dtype, shape=None, name="tensor"):
    """dtype, then shape, then device and layout: a host tensor of the wrong
    shape is reported as a shape error."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not _on_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _need_rows(t, dtype, rows, name, min_cols=0):
    """A 2-D [rows, ld] tensor with ld >= min_cols (row-major, ld = its width):
    the kernels index row i at i * ld, so fewer rows would be read or written
    past the allocation."""
    _need(t, dtype, None, name)
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] < min_cols:
        raise ValueError(f"{name}: expected shape ({rows}, ld) with ld >= {min_cols}, got {tuple(t.shape)}")
    return t


@dataclass
class Queries:
    """Queries of a call: sequence id and visible-history length per query
    (int32 device tensors) and a host-side upper bound of the lengths."""
    q_seq: torch.Tensor
    q_nvis: torch.Tensor
    max_nvis: int

    def c(self):
        n = int(self.q_seq.numel())
        if n:
            _need(self.q_seq, torch.int32, (n,), "q_seq")
            _need(self.q_nvis, torch.int32, (n,), "q_nvis")
        return QueriesC(n, int(self.max_nvis), _ptr(self.q_seq).value if n else None,
                        _ptr(self.q_nvis).value if n else None)

    @property
    def num_q(self):
        return int(self.q_seq.numel())


@dataclass
class KvLayout:
    """Cache layout: contiguous (seq_row0, int64 [num_seqs]) or paged
    (block_table, int32 [num_seqs, max_blocks], block_size > 0)."""
    num_seqs: int
    num_rows: int
    seq_row0: Optional[torch.Tensor] = None
    block_table: Optional[torch.Tensor] = None
    block_size: int = 0

    def c(self):
        if self.block_size == 0:
            _need(self.seq_row0, torch.int64, (self.num_seqs,), "seq_row0")
            return KvLayoutC(self.num_seqs, 0, 0, 0, self.num_rows, None, self.seq_row0.data_ptr())
        bt = _need(self.block_table, torch.int32, None, "block_table")
        if bt.dim() != 2 or bt.shape[0] != self.num_seqs or bt.shape[1] < 1:
            raise ValueError(f"block_table: expected shape ({self.num_seqs}, max_blocks), got {tuple(bt.shape)}")
        return KvLayoutC(self.num_seqs, self.block_size, int(bt.shape[1]), 0, self.num_rows, bt.data_ptr(), None)


def dsa_workspace_bytes(op: int, queries: Queries, k: int) -> int:
    qc = queries.c()
    return int(_lib.lib().dsa_workspace_bytes(op, ctypes.byref(qc), k))


def workspace(op: int, queries: Queries, k: int, device="cuda") -> Optional[torch.Tensor]:
    """A zero-filled byte tensor of dsa_workspace_bytes(op, ...) (torch's
    allocator returns blocks aligned to at least 256 bytes).  Zero is the
    state dsa_forward leaves it in, so reusing it across calls is the fast
    path."""
    n = dsa_workspace_bytes(op, queries, k)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def dsa_quantize_fp8(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None):
    rows, cols = x.shape
    _need(x, torch.float32, None, "x")
    _need(codes, torch.uint8, (rows, cols), "codes")
    _need(scales, torch.float32, (rows,), "scales")
    _lib.check("dsa_quantize_fp8", _lib.lib().dsa_quantize_fp8(
        _ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))


def dsa_quantize_fp8_e8m0(x: torch.Tensor, codes: torch.Tensor, e8m0: torch.Tensor, scales=None, stream=None):
    rows, cols = x.shape
    _need(x, torch.float32, None, "x")
    _need(codes, torch.uint8, (rows, cols), "codes")
    _need(e8m0, torch.uint8, (rows,), "e8m0")
    if scales is not None:
        _need(scales, torch.float32, (rows,), "scales")
    _lib.check("dsa_quantize_fp8_e8m0", _lib.lib().dsa_quantize_fp8_e8m0(
        _ptr(x), rows, cols, _ptr(codes), _ptr(e8m0), _ptr(scales), _stream(stream)))


def dsa_indexer_scores_e8m0(queries: Queries, layout: KvLayout, q_fp8, q_scale, w, k_fp8, k_scale_e8m0,
                            scores, stream=None):
    nq = queries.num_q
    _need(q_fp8, torch.uint8, (nq, DSA_HI, DSA_DI), "q_fp8")
    if q_scale is not None:
        _need(q_scale, torch.float32, (nq, DSA_HI), "q_scale")
    _need(w, torch.float32, (nq, DSA_HI), "w")
    _need(k_fp8, torch.uint8, (layout.num_rows, DSA_DI), "k_fp8")
    _need(k_scale_e8m0, torch.uint8, (layout.num_rows,), "k_scale_e8m0")
    _need_rows(scores, torch.float32, nq, "scores", queries.max_nvis)
    qc, lc = queries.c(), layout.c()
    _lib.check("dsa_indexer_scores_e8m0", _lib.lib().dsa_indexer_scores_e8m0(
        ctypes.byref(qc), ctypes.byref(lc), _ptr(q_fp8), _ptr(q_scale), _ptr(w), _ptr(k_fp8),
        _ptr(k_scale_e8m0), _ptr(scores), scores.shape[1], _stream(stream)))


def dsa_indexer_scores(queries: Queries, layout: KvLayout, q_fp8, q_scale, w, k_fp8, k_scale,
                       scores, stream=None):
    nq = queries.num_q
    _need(q_fp8, torch.uint8, (nq, DSA_HI, DSA_DI), "q_fp8")
    if q_scale is not None:
        _need(q_scale, torch.float32, (nq, DSA_HI), "q_scale")
    _need(w, torch.float32, (nq, DSA_HI), "w")
    _need(k_fp8, torch.uint8, (layout.num_rows, DSA_DI), "k_fp8")
    _need(k_scale, torch.float32, (layout.num_rows,), "k_scale")
    _need_rows(scores, torch.float32, nq, "scores", queries.max_nvis)
    qc, lc = queries.c(), layout.c()
    _lib.check("dsa_indexer_scores", _lib.lib().dsa_indexer_scores(
        ctypes.byref(qc), ctypes.byref(lc), _ptr(q_fp8), _ptr(q_scale), _ptr(w), _ptr(k_fp8),
        _ptr(k_scale), _ptr(scores), scores.shape[1], _stream(stream)))


def dsa_topk(queries: Queries, scores, k: int, idx, count=None, ws=None, stream=None):
    nq = queries.num_q
    _need(idx, torch.int32, (nq, k), "idx")
    if count is not None:
        _need(count, torch.int32, (nq,), "count")
    if scores is not None:
        _need_rows(scores, torch.float32, nq, "scores", queries.max_nvis)
    if ws is None:
        ws = workspace(DSA_OP_TOPK, queries, k, idx.device)
    qc = queries.c()
    _lib.check("dsa_topk", _lib.lib().dsa_topk(
        ctypes.byref(qc), _ptr(scores), scores.shape[1] if scores is not None else 0, k, _ptr(idx),
        _ptr(count), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def _mla(name, op, queries, layout, q, kv, idx, count, k, softmax_scale, out, lse, ws, stream):
    nq = queries.num_q
    _need(q, torch.bfloat16, (nq, DSA_H, DSA_D), "q")
    _need(kv, torch.bfloat16, (layout.num_rows, DSA_D), "kv")
    _need(idx, torch.int32, (nq, k), "idx")
    if count is not None:
        _need(count, torch.int32, (nq,), "count")
    _need(out, torch.float32, (nq, DSA_H, DSA_DV), "out")
    if lse is not None:
        _need(lse, torch.float32, (nq, DSA_H), "lse")
    if ws is None:
        ws = workspace(op, queries, k, q.device)
    qc, lc = queries.c(), layout.c()
    _lib.check(name, getattr(_lib.lib(), name)(
        ctypes.byref(qc), ctypes.byref(lc), _ptr(q), _ptr(kv), _ptr(idx), _ptr(count), k,
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def dsa_sparse_mla_decode(queries, layout, q, kv, idx, count, k, softmax_scale, out, lse=None, ws=None,
                          stream=None):
    return _mla("dsa_sparse_mla_decode", DSA_OP_MLA_DECODE, queries, layout, q, kv, idx, count, k,
                softmax_scale, out, lse, ws, stream)


def dsa_sparse_mla_decode_noalloc(queries, layout, q, kv, idx, count, k, softmax_scale, out, lse=None,
                                  stream=None):
    """dsa_sparse_mla_decode with its split partials in the library's own
    scratch (no workspace, nothing allocated; calls on one GPU must not
    overlap)."""
    nq = queries.num_q
    _need(q, torch.bfloat16, (nq, DSA_H, DSA_D), "q")
    _need(kv, torch.bfloat16, (layout.num_rows, DSA_D), "kv")
    _need(idx, torch.int32, (nq, k), "idx")
    if count is not None:
        _need(count, torch.int32, (nq,), "count")
    _need(out, torch.float32, (nq, DSA_H, DSA_DV), "out")
    if lse is not None:
        _need(lse, torch.float32, (nq, DSA_H), "lse")
    qc, lc = queries.c(), layout.c()
    _lib.check("dsa_sparse_mla_decode_noalloc", _lib.lib().dsa_sparse_mla_decode_noalloc(
        ctypes.byref(qc), ctypes.byref(lc), _ptr(q), _ptr(kv), _ptr(idx), _ptr(count), k, float(softmax_scale),
        _ptr(out), _ptr(lse), _stream(stream)))


def dsa_sparse_mla_prefill(queries, layout, q, kv, idx, count, k, softmax_scale, out, lse=None, ws=None,
                           stream=None):
    return _mla("dsa_sparse_mla_prefill", DSA_OP_MLA_PREFILL, queries, layout, q, kv, idx, count, k,
                softmax_scale, out, lse, ws, stream)


def dsa_dense_mla(queries, layout, q, kv, softmax_scale, out, lse=None, ws=None, stream=None):
    """Attention over every visible position of each query (no selection)."""
    nq = queries.num_q
    _need(q, torch.bfloat16, (nq, DSA_H, DSA_D), "q")
    _need(kv, torch.bfloat16, (layout.num_rows, DSA_D), "kv")
    _need(out, torch.float32, (nq, DSA_H, DSA_DV), "out")
    if lse is not None:
        _need(lse, torch.float32, (nq, DSA_H), "lse")
    if ws is None:
        ws = workspace(DSA_OP_MLA_DENSE, queries, 1, q.device)
    qc, lc = queries.c(), layout.c()
    _lib.check("dsa_dense_mla", _lib.lib().dsa_dense_mla(
        ctypes.byref(qc), ctypes.byref(lc), _ptr(q), _ptr(kv), float(softmax_scale), _ptr(out), _ptr(lse),
        _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def dsa_indexer_kl_sparse(queries, layout, q, kv, idx, count, k, lse, softmax_scale, scores, grad, kl,
                          target=None, loss=None, stream=None):
    """Indexer KL loss over each query's selected set: grad [num_q, k] = dL/dI in
    set order, kl [num_q], optional target [num_q, k] and loss [1]."""
    nq = queries.num_q
    _need(q, torch.bfloat16, (nq, DSA_H, DSA_D), "q")
    _need(kv, torch.bfloat16, (layout.num_rows, DSA_D), "kv")
    _need(idx, torch.int32, (nq, k), "idx")
    if count is not None:
        _need(count, torch.int32, (nq,), "count")
    _need(lse, torch.float32, (nq, DSA_H), "lse")
    _need_rows(scores, torch.float32, nq, "scores", queries.max_nvis)
    _need(grad, torch.float32, (nq, k), "grad")
    _need(kl, torch.float32, (nq,), "kl")
    if target is not None:
        _need(target, torch.float32, (nq, k), "target")
    if loss is not None:
        _need(loss, torch.float32, (1,), "loss")
    qc, lc = queries.c(), layout.c()
    _lib.check("dsa_indexer_kl_sparse", _lib.lib().dsa_indexer_kl_sparse(
        ctypes.byref(qc), ctypes.byref(lc), _ptr(q), _ptr(kv), _ptr(idx), _ptr(count), k, _ptr(lse),
        float(softmax_scale), _ptr(scores), scores.shape[-1], _ptr(grad), _ptr(target), _ptr(kl), _ptr(loss),
        _stream(stream)))


def dsa_indexer_kl_dense(queries, layout, q, kv, lse, softmax_scale, scores, grad, kl, target=None, loss=None,
                         stream=None):
    """Indexer KL loss over every visible position: grad [num_q, ld] = dL/dI by
    position (s < q_nvis), kl [num_q], optional target (like grad) and loss [1]."""
    nq = queries.num_q
    _need(q, torch.bfloat16, (nq, DSA_H, DSA_D), "q")
    _need(kv, torch.bfloat16, (layout.num_rows, DSA_D), "kv")
    _need(lse, torch.float32, (nq, DSA_H), "lse")
    _need_rows(scores, torch.float32, nq, "scores", queries.max_nvis)
    _need_rows(grad, torch.float32, nq, "grad", queries.max_nvis)
    _need(kl, torch.float32, (nq,), "kl")
    if target is not None:
        _need(target, torch.float32, tuple(grad.shape), "target")
    if loss is not None:
        _need(loss, torch.float32, (1,), "loss")
    qc, lc = queries.c(), layout.c()
    _lib.check("dsa_indexer_kl_dense", _lib.lib().dsa_indexer_kl_dense(
        ctypes.byref(qc), ctypes.byref(lc), _ptr(q), _ptr(kv), _ptr(lse), float(softmax_scale), _ptr(scores),
        scores.shape[-1], _ptr(grad), _ptr(target), grad.shape[-1], _ptr(kl), _ptr(loss), _stream(stream)))


def dsa_indexer_backward(queries, layout, q_fp8, q_scale, w, k_fp8, k_scale, idx, count, k, grad, dq, dw, dk,
                         stream=None):
    """Gradients of the indexer score with respect to w, the dequantised q and
    the dequantised k, given grad = dL/dI over each query's set (idx [num_q, k]
    with grad in set order, or idx None: every visible position, grad by
    position).  dq [num_q, 64, 128] and dw [num_q, 64] are overwritten; dk
    [rows, 128] is added to."""
    nq = queries.num_q
    _need(q_fp8, torch.uint8, (nq, DSA_HI, DSA_DI), "q_fp8")
    if q_scale is not None:
        _need(q_scale, torch.float32, (nq, DSA_HI), "q_scale")
    _need(w, torch.float32, (nq, DSA_HI), "w")
    _need(k_fp8, torch.uint8, (layout.num_rows, DSA_DI), "k_fp8")
    _need(k_scale, torch.float32, (layout.num_rows,), "k_scale")
    if idx is not None:
        _need(idx, torch.int32, (nq, k), "idx")
        _need(grad, torch.float32, (nq, k), "grad")
    else:
        _need_rows(grad, torch.float32, nq, "grad", queries.max_nvis)
        k = 0
    if count is not None:
        _need(count, torch.int32, (nq,), "count")
    _need(dq, torch.float32, (nq, DSA_HI, DSA_DI), "dq")
    _need(dw, torch.float32, (nq, DSA_HI), "dw")
    _need(dk, torch.float32, (layout.num_rows, DSA_DI), "dk")
    qc, lc = queries.c(), layout.c()
    _lib.check("dsa_indexer_backward", _lib.lib().dsa_indexer_backward(
        ctypes.byref(qc), ctypes.byref(lc), _ptr(q_fp8), _ptr(q_scale), _ptr(w), _ptr(k_fp8), _ptr(k_scale),
        _ptr(idx), _ptr(count), k, _ptr(grad), grad.shape[-1], _ptr(dq), _ptr(dw), _ptr(dk), _stream(stream)))


def dsa_forward(queries: Queries, layout: KvLayout, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, k,
                softmax_scale, out, lse=None, idx_out=None, ws=None, stream=None, events=None):
    """events: optional ctypes array of 5 hipEvent_t handles; when given the
    call goes through dsa_forward_profiled, which records them between the
    stages on the same stream (before the first kernel, before the indexer,
    after it, after the top-k, after the attention)."""
    nq = queries.num_q
    _need(q_fp8, torch.uint8, (nq, DSA_HI, DSA_DI), "q_fp8")
    if q_scale is not None:
        _need(q_scale, torch.float32, (nq, DSA_HI), "q_scale")
    _need(w, torch.float32, (nq, DSA_HI), "w")
    _need(k_fp8, torch.uint8, (layout.num_rows, DSA_DI), "k_fp8")
    _need(k_scale, torch.float32, (layout.num_rows,), "k_scale")
    _need(q, torch.bfloat16, (nq, DSA_H, DSA_D), "q")
    _need(kv, torch.bfloat16, (layout.num_rows, DSA_D), "kv")
    _need(out, torch.float32, (nq, DSA_H, DSA_DV), "out")
    if lse is not None:
        _need(lse, torch.float32, (nq, DSA_H), "lse")
    if idx_out is not None:
        _need(idx_out, torch.int32, (nq, k), "idx_out")
    if ws is None:
        ws = workspace(DSA_OP_FORWARD, queries, k, q.device)
    qc, lc = queries.c(), layout.c()
    args = (ctypes.byref(qc), ctypes.byref(lc), _ptr(q_fp8), _ptr(q_scale), _ptr(w), _ptr(k_fp8),
            _ptr(k_scale), _ptr(q), _ptr(kv), k, float(softmax_scale), _ptr(out), _ptr(lse),
            _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream))
    if events is None:
        _lib.check("dsa_forward", _lib.lib().dsa_forward(*args))
    else:
        _lib.check("dsa_forward_profiled", _lib.lib().dsa_forward_profiled(*args, events))
    return ws


class HipEvents:
    """A few hipEvent_t handles from the HIP runtime, for in-stream stage timing
    (torch.cuda.Event does not expose its handle)."""

    def __init__(self, n):
        self._rt = ctypes.CDLL("libamdhip64.so")
        self._rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self._rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles[i] = h
        self.n = n

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self._rt.hipEventElapsedTime(ctypes.byref(ms), self.handles[a], self.handles[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for i in range(self.n):
            if self.handles[i]:
                self._rt.hipEventDestroy(self.handles[i])
                self.handles[i] = None
