"""ctypes view of libdsa.so (the C ABI declared in include/dsa.h).

Loading fails loudly when the library has not been built: there is no other
implementation of the path to fall back to.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_HI, DSA_DI, DSA_H, DSA_D, DSA_DV, DSA_KMAX = 64, 128, 128, 576, 512, 2048
DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = 0, 1, 2, 3, 4
DSA_OP_TOPK, DSA_OP_MLA_DECODE, DSA_OP_MLA_PREFILL, DSA_OP_FORWARD, DSA_OP_MLA_DENSE = 1, 2, 3, 4, 5
DSA_NOALLOC_SCRATCH_BYTES = 72 << 20

EXPORTED = (
    "dsa_quantize_fp8",
    "dsa_quantize_fp8_e8m0",
    "dsa_indexer_scores",
    "dsa_indexer_scores_e8m0",
    "dsa_topk",
    "dsa_sparse_mla_decode",
    "dsa_sparse_mla_decode_noalloc",
    "dsa_sparse_mla_prefill",
    "dsa_dense_mla",
    "dsa_indexer_kl_sparse",
    "dsa_indexer_kl_dense",
    "dsa_indexer_backward",
    "dsa_forward",
    "dsa_forward_profiled",
    "dsa_workspace_bytes",
    "dsa_status_string",
    "dsa_last_error",
)


class KvLayoutC(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("num_rows", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("seq_row0", ctypes.c_void_p),
    ]


class QueriesC(ctypes.Structure):
    _fields_ = [
        ("num_q", ctypes.c_int32),
        ("max_nvis", ctypes.c_int32),
        ("q_seq", ctypes.c_void_p),
        ("q_nvis", ctypes.c_void_p),
    ]


class DsaError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if libdsa.so is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m sparse_long_context_dsa_amd.build` "
            "(hipcc, gfx950).  The DSA path has no other implementation.")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    qp, lp = ctypes.POINTER(QueriesC), ctypes.POINTER(KvLayoutC)
    sig = {
        "dsa_quantize_fp8": [vp, i64, i32, vp, vp, vp],
        "dsa_quantize_fp8_e8m0": [vp, i64, i32, vp, vp, vp, vp],
        "dsa_indexer_scores": [qp, lp, vp, vp, vp, vp, vp, vp, i64, vp],
        "dsa_indexer_scores_e8m0": [qp, lp, vp, vp, vp, vp, vp, vp, i64, vp],
        "dsa_topk": [qp, vp, i64, i32, vp, vp, vp, sz, vp],
        "dsa_sparse_mla_decode": [qp, lp, vp, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp],
        "dsa_sparse_mla_decode_noalloc": [qp, lp, vp, vp, vp, vp, i32, f32, vp, vp, vp],
        "dsa_sparse_mla_prefill": [qp, lp, vp, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp],
        "dsa_dense_mla": [qp, lp, vp, vp, f32, vp, vp, vp, sz, vp],
        "dsa_indexer_kl_sparse": [qp, lp, vp, vp, vp, vp, i32, vp, f32, vp, i64, vp, vp, vp, vp, vp],
        "dsa_indexer_kl_dense": [qp, lp, vp, vp, vp, f32, vp, i64, vp, vp, i64, vp, vp, vp],
        "dsa_indexer_backward": [qp, lp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i64, vp, vp, vp, vp],
        "dsa_forward": [qp, lp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, vp, sz, vp],
        "dsa_forward_profiled": [qp, lp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, vp, sz, vp, vp],
        "dsa_workspace_bytes": [ctypes.c_int, qp, i32],
        "dsa_status_string": [ctypes.c_int],
        "dsa_last_error": [],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.dsa_workspace_bytes.restype = ctypes.c_size_t
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def check(fn_name, status):
    if status != DSA_OK:
        detail = lib().dsa_last_error().decode()
        raise DsaError(fn_name, status, detail or lib().dsa_status_string(status).decode())
