"""ctypes front end of the C oracle in ``oracle.c`` (test infrastructure only).

Argument marshalling only: every number the oracle returns is computed by the
C code in fp64.  See ``oracle.c`` for the definition it follows and the page
sections it cites.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORACLE_ERR_ARG = -1
ORACLE_ERR_PAGE = -2
ORACLE_ERR_TABLE = -3

# Row status bits of the page-4 table builder (see oracle.c).
PAGE4_EMPTY = 1
PAGE4_PARTIAL = 2
PAGE4_TAIL = 4
PAGE4_PAGE = 8
PAGE4_OVERFLOW = 16
PAGE4_SEQ = 32
PAGE4_LONG = 64
PAGE4_MAX_LIVE = 1 << 26

# Row status bits of the top-k/top-p masking (see oracle.c).
MASK_BAD_K = 1
MASK_BAD_P = 2


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle returned error code {code}")
        self.code = code


def build(out_path: str = _LIB, extra_flags: tuple[str, ...] = ()) -> str:
    """Compile oracle.c with gcc into a shared library (IEEE fp64, no contraction)."""
    tmp = f"{out_path}.{os.getpid()}.tmp"   # concurrent builders never share a temp file
    cmd = [
        "gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", *extra_flags,
        _SRC, "-o", tmp, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


_lib_cache: dict[str, ctypes.CDLL] = {}


def load(path: str = _LIB) -> ctypes.CDLL:
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        if path != _LIB:
            raise FileNotFoundError(path)
        build(path)
    lib = ctypes.CDLL(path)
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_f16_value.restype = ctypes.c_double
    lib.oracle_f16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3_table.restype = None
    lib.oracle_e4m3_table.argtypes = [ctypes.c_void_p]
    lib.oracle_f16_decode.restype = None
    lib.oracle_f16_decode.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_paged_gqa.restype = ctypes.c_int
    lib.oracle_paged_gqa.argtypes = [
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_double, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
    ]
    lib.oracle_topk_select.restype = ctypes.c_int
    lib.oracle_topk_select.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_qsa_page4_table.restype = ctypes.c_int
    lib.oracle_qsa_page4_table.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_void_p]
    lib.oracle_topk_topp_mask.restype = ctypes.c_int
    lib.oracle_topk_topp_mask.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_void_p]
    _lib_cache[path] = lib
    return lib


def num_threads(lib_path: str = _LIB) -> int:
    return int(load(lib_path).oracle_num_threads())


def e4m3_value(code: int, lib_path: str = _LIB) -> float:
    return float(load(lib_path).oracle_e4m3_value(code))


def e4m3_table(lib_path: str = _LIB) -> np.ndarray:
    out = np.empty(256, dtype=np.float64)
    load(lib_path).oracle_e4m3_table(out.ctypes.data)
    return out


def f16_decode(bits: np.ndarray, lib_path: str = _LIB) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    load(lib_path).oracle_f16_decode(bits.ctypes.data, bits.size, out.ctypes.data)
    return out


def _ptr(arr: np.ndarray, elem_offset: int) -> int:
    if not arr.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle inputs must be C-contiguous")
    return arr.ctypes.data + int(elem_offset) * arr.itemsize


def paged_gqa(*, q: np.ndarray, k_store: np.ndarray, v_store: np.ndarray,
              k_offset: int, v_offset: int, page_stride: int, token_stride: int,
              head_stride: int, num_pages: int, page_size: int, kv_dtype: int,
              k_scale: float, v_scale: float, table: np.ndarray, lens: np.ndarray,
              sm_scale: float, num_kv_heads: int, seq_ids=None,
              lib_path: str = _LIB) -> np.ndarray:
    """fp64 paged GQA attention.

    q: float16 [n_seq][Hq][D].  k_store / v_store: the pool storage arrays
    (uint8 FP8-E4M3 codes or float16), with K/V element (0,0,0,0) at element
    offset k_offset / v_offset.  table: int32 [n_seq][max_pages].
    Returns float64 [len(seq_ids) or n_seq][Hq][D].
    """
    q = np.ascontiguousarray(q, dtype=np.float16)
    n_seq, hq, d = q.shape
    table = np.ascontiguousarray(table, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    if table.ndim != 2 or table.shape[0] != n_seq or lens.shape != (n_seq,):
        raise ValueError("table must be [n_seq][max_pages] and lens [n_seq]")
    want_itemsize = 2 if kv_dtype == 0 else 1
    for s in (k_store, v_store):
        if s.itemsize != want_itemsize:
            raise ValueError("pool storage element size does not match kv_dtype")
    if seq_ids is None:
        ids_ptr, n_ids = None, n_seq
    else:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        ids_ptr, n_ids = ids.ctypes.data, ids.size
    out = np.empty((n_ids, hq, d), dtype=np.float64)
    rc = load(lib_path).oracle_paged_gqa(
        q.view(np.uint16).ctypes.data, n_seq, hq, num_kv_heads, d,
        _ptr(k_store, k_offset), _ptr(v_store, v_offset),
        page_stride, token_stride, head_stride,
        num_pages, page_size, kv_dtype, float(k_scale), float(v_scale),
        table.ctypes.data, table.shape[1], lens.ctypes.data, float(sm_scale),
        ids_ptr, n_ids, out.ctypes.data)
    if rc != 0:
        raise OracleError(rc)
    return out


def topk_select(scores: np.ndarray, k: int, n_valid=None, n_blocks: int | None = None,
                lib_path: str = _LIB):
    """Top-k block selection per row (see oracle.c).  scores: float32
    [rows][row_stride], of which the first n_blocks columns (default: all) may
    be selected.  Returns (idx int32 [rows][k] ascending then -1,
    count int32 [rows])."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    rows, stride = scores.shape
    nb = stride if n_blocks is None else int(n_blocks)
    nv = None if n_valid is None else np.ascontiguousarray(n_valid, dtype=np.int32)
    idx = np.empty((rows, k), dtype=np.int32)
    cnt = np.empty(rows, dtype=np.int32)
    rc = load(lib_path).oracle_topk_select(scores.ctypes.data, stride,
                                           None if nv is None else nv.ctypes.data,
                                           rows, nb, k, idx.ctypes.data, cnt.ctypes.data)
    if rc != 0:
        raise OracleError(rc)
    return idx, cnt


def qsa_page4_table(tokens: np.ndarray, live_len, block_table: np.ndarray, *, num_pages: int,
                    page_size: int, vpages_per_page: int, out_stride: int, row_seq=None,
                    lib_path: str = _LIB):
    """Virtual page-4 table of each row's expanded QSA selection (see
    oracle.c).  tokens: int32 [rows][n_tokens] logical positions (-1 =
    padding); live_len: int32 [rows]; block_table: int32 [n_seqs][max_pages]
    physical page of each logical page of `page_size` tokens; row_seq: int32
    [rows] or None (all rows in sequence 0).  Returns (table int32
    [rows][out_stride], lens int32 [rows], status int32 [rows])."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    if tokens.ndim != 2:
        raise ValueError("tokens must be [rows][n_tokens]")
    rows, n_tok = tokens.shape
    live = np.ascontiguousarray(live_len, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    if bt.ndim == 1:
        bt = bt[None, :]
    seq = None if row_seq is None else np.ascontiguousarray(row_seq, dtype=np.int32)
    if live.shape != (rows,) or (seq is not None and seq.shape != (rows,)):
        raise ValueError("live_len and row_seq must be [rows]")
    table = np.empty((rows, out_stride), dtype=np.int32)
    lens = np.empty(rows, dtype=np.int32)
    status = np.empty(rows, dtype=np.int32)
    rc = load(lib_path).oracle_qsa_page4_table(
        tokens.ctypes.data, n_tok, n_tok, live.ctypes.data, bt.ctypes.data, bt.shape[1],
        None if seq is None else seq.ctypes.data, bt.shape[0], num_pages, page_size,
        vpages_per_page, rows,
        table.ctypes.data, out_stride, lens.ctypes.data, status.ctypes.data)
    if rc != 0:
        raise OracleError(rc)
    return table, lens, status


def topk_topp_mask(logits: np.ndarray, k, p, *, k_max: int = 1024, lib_path: str = _LIB):
    """Combined top-k/top-p masking of each row of fp32 logits [rows][V] (see
    oracle.c).  k: int32 [rows]; p: float32 [rows].  Returns (out float32
    [rows][V], status int32 [rows], n_kept int32 [rows])."""
    z = np.ascontiguousarray(logits, dtype=np.float32)
    rows, V = z.shape
    kk = np.ascontiguousarray(np.broadcast_to(np.asarray(k, dtype=np.int32), (rows,)))
    pp = np.ascontiguousarray(np.broadcast_to(np.asarray(p, dtype=np.float32), (rows,)))
    out = np.empty_like(z)
    status = np.empty(rows, dtype=np.int32)
    kept = np.empty(rows, dtype=np.int32)
    rc = load(lib_path).oracle_topk_topp_mask(z.ctypes.data, V, rows, V, kk.ctypes.data,
                                              pp.ctypes.data, k_max, out.ctypes.data, V,
                                              status.ctypes.data, kept.ctypes.data)
    if rc != 0:
        raise OracleError(rc)
    return out, status, kept
