"""ctypes binding of libpgqa (include/pgqa.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors are
torch tensors on the GPU (PyTorch provides device memory and streams); the
computation is done entirely by the library's HIP kernels.  The library sees
only pointers, so before each call the binding checks what the tensors say
about them (dtype, shape, layout, device, and that a KV pool's tensors hold
every element its strides address) and raises ValueError otherwise.  There
is no fallback: if ``libpgqa.so`` is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpgqa.so")

PGQA_OK = 0
PGQA_ERR_NULL = -1
PGQA_ERR_SHAPE = -2
PGQA_ERR_LAYOUT = -3
PGQA_ERR_DTYPE = -4
PGQA_ERR_WORKSPACE = -5
PGQA_ERR_HIP = -6
PGQA_ERR_ARG = -7
PGQA_KV_FP16 = 0
PGQA_KV_E4M3 = 1
HEAD_DIM = 256
SIZE_MAX = ctypes.c_size_t(-1).value
NOALLOC_SCRATCH_BYTES = 8 << 20  # PGQA_NOALLOC_SCRATCH_BYTES

# Every symbol include/pgqa.h declares.
EXPORTS = ("paged_gqa_workspace_bytes", "paged_gqa_num_splits", "paged_gqa_decode",
           "paged_gqa_prefill_sparse", "paged_gqa_decode_partial", "paged_gqa_merge_partials",
           "paged_gqa_decode_noalloc",
           "e4m3_decode_table", "qsa_topk_select", "qsa_build_page4_table",
           "sampler_topk_topp_workspace_bytes", "sampler_topk_topp_mask", "pgqa_error_string")
QSA_MAX_BLOCKS = 65536
QSA_MAX_SEL_TOKENS = 8192
# Row status bits of qsa_build_page4_table.
PAGE4_EMPTY, PAGE4_PARTIAL, PAGE4_TAIL, PAGE4_PAGE = 1, 2, 4, 8
PAGE4_OVERFLOW, PAGE4_SEQ, PAGE4_LONG = 16, 32, 64
PAGE4_MAX_LIVE = 1 << 26
SAMPLER_MAX_K = 256
SAMPLER_MAX_VOCAB = 524288
# Row status bits of sampler_topk_topp_mask.
SAMPLER_MASK_BAD_K, SAMPLER_MASK_BAD_P = 1, 2


class PgqaError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _lib().pgqa_error_string(code).decode() if _LIB else str(code)
        super().__init__(f"{where}: {msg} (code {code})")
        self.code = code


class KVPoolC(ctypes.Structure):
    """Mirror of pgqa_kv_pool."""
    _fields_ = [
        ("k_base", ctypes.c_void_p), ("v_base", ctypes.c_void_p),
        ("page_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64), ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
    ]


_LIB = None


def _lib(path: str = LIB_PATH) -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is not built; run `python -m fp8_kv_amd.build` (there is no fallback)")
    # torch ships its own HIP runtime: load it first so that this library
    # binds to that same runtime (and sees the tensors torch allocates)
    # instead of starting a second one from the system ROCm.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.paged_gqa_workspace_bytes.restype = sz
    lib.paged_gqa_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_gqa_num_splits.restype = i32
    lib.paged_gqa_num_splits.argtypes = [i32, i32, i32, i32]
    attn_args = [vp, ctypes.POINTER(KVPoolC), vp, i32, vp, i32, i32, i32, i32, i32, f32, i32,
                 vp, vp, sz, vp]
    for name in ("paged_gqa_decode", "paged_gqa_prefill_sparse"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = attn_args
    lib.paged_gqa_decode_partial.restype = ctypes.c_int
    lib.paged_gqa_decode_partial.argtypes = [vp, ctypes.POINTER(KVPoolC), vp, i32, vp, i32, i32,
                                             i32, i32, i32, f32, i32, vp, vp, vp]
    lib.paged_gqa_decode_noalloc.restype = ctypes.c_int
    lib.paged_gqa_decode_noalloc.argtypes = [vp, ctypes.POINTER(KVPoolC), vp, i32, vp, i32, i32,
                                             i32, i32, i32, f32, i32, vp, vp]
    lib.paged_gqa_merge_partials.restype = ctypes.c_int
    lib.paged_gqa_merge_partials.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.e4m3_decode_table.restype = ctypes.c_int
    lib.e4m3_decode_table.argtypes = [vp, vp]
    lib.qsa_topk_select.restype = ctypes.c_int
    lib.qsa_topk_select.argtypes = [vp, ctypes.c_int64, vp, i32, i32, i32, vp, vp, vp]
    lib.qsa_build_page4_table.restype = ctypes.c_int
    lib.qsa_build_page4_table.argtypes = [vp, ctypes.c_int64, i32, vp, vp, i32, vp, i32, i32, i32,
                                          i32, i32, vp, i32, vp, vp, vp]
    lib.sampler_topk_topp_workspace_bytes.restype = sz
    lib.sampler_topk_topp_workspace_bytes.argtypes = [i32, i32, i32]
    lib.sampler_topk_topp_mask.restype = ctypes.c_int
    lib.sampler_topk_topp_mask.argtypes = [vp, ctypes.c_int64, i32, i32, vp, vp, i32, vp,
                                           ctypes.c_int64, vp, vp, sz, vp]
    lib.pgqa_error_string.restype = ctypes.c_char_p
    lib.pgqa_error_string.argtypes = [ctypes.c_int]
    _LIB = lib
    return lib


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    return _lib(path)


@dataclass
class KVPool:
    """A paged KV pool in device memory.  `k` and `v` are tensors whose
    data_ptr() is the address of K/V element (page 0, slot 0, head 0, dim 0);
    strides are in elements (see pgqa_kv_pool in include/pgqa.h)."""

    k: object
    v: object
    page_stride: int
    token_stride: int
    head_stride: int
    num_pages: int
    page_size: int
    kv_dtype: int
    k_scale: float = 1.0
    v_scale: float = 1.0
    storage: tuple = ()  # tensors kept alive with the pool

    def as_c(self) -> KVPoolC:
        return KVPoolC(self.k.data_ptr(), self.v.data_ptr(), self.page_stride,
                       self.token_stride, self.head_stride, self.num_pages, self.page_size,
                       self.kv_dtype, self.k_scale, self.v_scale)


def _stream_handle(stream) -> int | None:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _check(rc: int, where: str) -> None:
    if rc != PGQA_OK:
        raise PgqaError(rc, where)


def _expect(t, name: str, dtype, shape=None, *, dense: bool = True) -> None:
    """Checks a tensor before its address goes to the library, which sees only
    pointers: dtype, shape (None matches any size) and dense row-major layout
    when the C side assumes one.  _device checks where it lives, after every
    tensor of a call has passed these."""
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and (t.dim() != len(shape) or
                              any(w is not None and w != d for w, d in zip(shape, t.shape))):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _device(**tensors) -> None:
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name}: must be a device tensor")


def _bytes_after(t) -> int:
    """Bytes of t's storage from t.data_ptr() to the storage's end."""
    st = t.untyped_storage()
    return st.nbytes() - (t.data_ptr() - st.data_ptr())


def _pool_extent(kv: "KVPool", num_kv_heads: int) -> int | None:
    """Bytes from K's (and V's) start to the end of the farthest element the
    strides address, (num_pages-1, page_size-1, num_kv_heads-1, 255); None
    for sizes the library rejects by itself."""
    dims = (kv.num_pages, kv.page_size, num_kv_heads)
    strides = (kv.page_stride, kv.token_stride, kv.head_stride)
    if min(dims) < 1 or min(strides) < 0:
        return None
    es = 1 if kv.kv_dtype == PGQA_KV_E4M3 else 2
    return (sum((d - 1) * st for d, st in zip(dims, strides)) + HEAD_DIM) * es


def _check_pool(kv: "KVPool", num_kv_heads: int) -> None:
    extent = _pool_extent(kv, num_kv_heads)
    if extent is None:
        return
    for name, t in (("kv.k", kv.k), ("kv.v", kv.v)):
        if _bytes_after(t) < extent:
            raise ValueError(f"{name}: {_bytes_after(t)} bytes from its start, the strides "
                             f"address {extent}")


def paged_gqa_workspace_bytes(n: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
                              num_splits: int = 0, head_dim: int = HEAD_DIM) -> int:
    r = _lib().paged_gqa_workspace_bytes(n, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                         num_splits)
    if r == SIZE_MAX:
        raise PgqaError(PGQA_ERR_ARG, "paged_gqa_workspace_bytes")
    return int(r)


def paged_gqa_num_splits(n: int, num_kv_heads: int, max_seq_len: int, num_splits: int = 0) -> int:
    r = _lib().paged_gqa_num_splits(n, num_kv_heads, max_seq_len, num_splits)
    if r < 0:
        raise PgqaError(r, "paged_gqa_num_splits")
    return int(r)


def paged_gqa_decode(q, kv: KVPool, page_table, seq_lens, max_seq_len: int, sm_scale: float,
                     out, num_kv_heads: int = 1, workspace=None, num_splits: int = 0,
                     stream=None) -> None:
    """q, out: fp16 [B][Hq][256]; page_table: int32 [B][max_pages];
    seq_lens: int32 [B]; workspace: any device tensor of at least
    paged_gqa_workspace_bytes(...) bytes (None when that is 0)."""
    _call("paged_gqa_decode", q, kv, page_table, seq_lens, max_seq_len, num_kv_heads, sm_scale,
          num_splits, out, workspace, stream)


def paged_gqa_prefill_sparse(q, kv: KVPool, row_tables, row_lens, max_row_len: int,
                             sm_scale: float, out, num_kv_heads: int = 1, workspace=None,
                             num_splits: int = 0, stream=None) -> None:
    """Sparse prefill: rows in place of sequences (see include/pgqa.h)."""
    _call("paged_gqa_prefill_sparse", q, kv, row_tables, row_lens, max_row_len, num_kv_heads,
          sm_scale, num_splits, out, workspace, stream)


def _check_inputs(q, kv, table, lens, hkv) -> None:
    import torch

    _expect(q, "q", torch.float16, (None, None, None))
    n = q.shape[0]
    _expect(table, "page table", torch.int32, (n, None))
    _expect(lens, "lengths", torch.int32, (n,))
    _check_pool(kv, hkv)


def _call(fn_name, q, kv, table, lens, max_len, hkv, sm_scale, num_splits, out, workspace,
          stream):
    import torch

    _check_inputs(q, kv, table, lens, hkv)
    _expect(out, "out", torch.float16, tuple(q.shape))
    if workspace is not None:
        _expect(workspace, "workspace", workspace.dtype)
    _device(q=q, page_table=table, lengths=lens, kv_k=kv.k, kv_v=kv.v, out=out,
            workspace=workspace)
    n, hq, d = q.shape
    c_pool = kv.as_c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = getattr(_lib(), fn_name)(
        _ptr(q), ctypes.byref(c_pool), _ptr(table), int(table.shape[1]), _ptr(lens),
        int(max_len), int(n), int(hq), int(hkv), int(d), float(sm_scale), int(num_splits),
        _ptr(out), _ptr(workspace), int(ws_bytes), _stream_handle(stream))
    _check(rc, fn_name)


def paged_gqa_decode_noalloc(q, kv: KVPool, page_table, seq_lens, max_seq_len: int,
                             sm_scale: float, out, num_kv_heads: int = 1, num_splits: int = 0,
                             stream=None) -> None:
    """paged_gqa_decode without a workspace: the split partials live in the
    library's per-device scratch (at most PGQA_NOALLOC_SCRATCH_BYTES), so the
    call allocates nothing.  Calls that overlap on one GPU race."""
    import torch

    _check_inputs(q, kv, page_table, seq_lens, num_kv_heads)
    _expect(out, "out", torch.float16, tuple(q.shape))
    _device(q=q, page_table=page_table, lengths=seq_lens, kv_k=kv.k, kv_v=kv.v, out=out)
    n, hq, d = q.shape
    c_pool = kv.as_c()
    rc = _lib().paged_gqa_decode_noalloc(
        _ptr(q), ctypes.byref(c_pool), _ptr(page_table), int(page_table.shape[1]),
        _ptr(seq_lens), int(max_seq_len), int(n), int(hq), int(num_kv_heads), int(d),
        float(sm_scale), int(num_splits), _ptr(out), _stream_handle(stream))
    _check(rc, "paged_gqa_decode_noalloc")


def paged_gqa_decode_partial(q, kv: KVPool, page_table, seq_lens, max_seq_len: int,
                             sm_scale: float, part_o, part_lse, num_kv_heads: int = 1,
                             num_splits: int = 0, stream=None) -> None:
    """part_o: fp32 [B][Hq][S][256]; part_lse: fp32 [B][Hq][S] with
    S = paged_gqa_num_splits(B, num_kv_heads, max_seq_len, num_splits)."""
    import torch

    _check_inputs(q, kv, page_table, seq_lens, num_kv_heads)
    n, hq, d = q.shape
    S = paged_gqa_num_splits(n, num_kv_heads, max_seq_len, num_splits)
    _expect(part_o, "part_o", torch.float32, (n, hq, S, d))
    _expect(part_lse, "part_lse", torch.float32, (n, hq, S))
    _device(q=q, page_table=page_table, lengths=seq_lens, kv_k=kv.k, kv_v=kv.v, part_o=part_o,
            part_lse=part_lse)
    c_pool = kv.as_c()
    rc = _lib().paged_gqa_decode_partial(
        _ptr(q), ctypes.byref(c_pool), _ptr(page_table), int(page_table.shape[1]),
        _ptr(seq_lens), int(max_seq_len), int(n), int(hq), int(num_kv_heads), int(d),
        float(sm_scale), int(num_splits), _ptr(part_o), _ptr(part_lse), _stream_handle(stream))
    _check(rc, "paged_gqa_decode_partial")


def paged_gqa_merge_partials(part_o, part_lse, out, stream=None) -> None:
    """part_o: fp32 [rows][S][256]; part_lse: fp32 [rows][S]; out: fp16 [rows][256]
    (any leading shape that flattens to these)."""
    import torch

    _expect(part_lse, "part_lse", torch.float32)
    splits = part_lse.shape[-1] if part_lse.dim() else 0
    rows = part_lse.numel() // splits if splits else 0
    _expect(part_o, "part_o", torch.float32)
    _expect(out, "out", torch.float16)
    d = part_o.shape[-1] if part_o.dim() else 0
    if part_o.numel() != rows * splits * d or out.numel() != rows * d:
        raise ValueError(f"part_o {tuple(part_o.shape)} / out {tuple(out.shape)} do not hold "
                         f"{rows} rows of {splits} splits")
    _device(part_o=part_o, part_lse=part_lse, out=out)
    rc = _lib().paged_gqa_merge_partials(_ptr(part_o), _ptr(part_lse), int(rows), int(splits),
                                         int(part_o.shape[-1]), _ptr(out),
                                         _stream_handle(stream))
    _check(rc, "paged_gqa_merge_partials")


def e4m3_decode_table(out, stream=None) -> None:
    """out: float32 [256] device tensor."""
    import torch

    _expect(out, "out", torch.float32, (256,))
    _device(out=out)
    _check(_lib().e4m3_decode_table(_ptr(out), _stream_handle(stream)), "e4m3_decode_table")


def qsa_topk_select(scores, k: int, n_valid=None, n_blocks: int | None = None, out_idx=None,
                    out_count=None, stream=None):
    """QSA top-k block selection per row.

    scores: fp32 device tensor [rows][n] (row stride taken from the tensor);
    the first n_blocks columns (default n) may be selected, row r only its
    first n_valid[r].  Returns (out_idx int32 [rows][k], out_count int32
    [rows]), allocating them when not given."""
    import torch

    if scores.dim() != 2 or scores.dtype != torch.float32 or scores.stride(1) != 1:
        raise ValueError("scores must be a float32 [rows][n] tensor with unit column stride")
    rows = scores.shape[0]
    nb = scores.shape[1] if n_blocks is None else int(n_blocks)
    if nb > scores.shape[1] and rows > 0:
        raise ValueError(f"n_blocks {nb} exceeds the {scores.shape[1]} score columns")
    if n_valid is not None:
        _expect(n_valid, "n_valid", torch.int32, (rows,))
    if out_idx is None:
        out_idx = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    elif k > 0:
        _expect(out_idx, "out_idx", torch.int32, (rows, k))
    if out_count is None:
        out_count = torch.empty(rows, dtype=torch.int32, device=scores.device)
    else:
        _expect(out_count, "out_count", torch.int32, (rows,))
    _device(scores=scores, n_valid=n_valid, out_idx=out_idx, out_count=out_count)
    stride = scores.stride(0) if rows > 1 else max(scores.shape[1], nb)
    rc = _lib().qsa_topk_select(_ptr(scores), int(stride), _ptr(n_valid), int(rows), int(nb),
                                int(k), _ptr(out_idx) if k > 0 else None, _ptr(out_count),
                                _stream_handle(stream))
    _check(rc, "qsa_topk_select")
    return out_idx, out_count


def qsa_build_page4_table(tokens, live_len, block_table, *, num_pages: int, page_size: int,
                          vpages_per_page: int, out_stride: int, row_seq=None, out_table=None,
                          out_len=None, out_status=None, stream=None):
    """Virtual page-4 table of each row's expanded QSA selection (see
    include/pgqa.h).  tokens: int32 device tensor [rows][n] (row stride taken
    from the tensor); live_len int32 [rows]; block_table int32
    [n_seqs][max_pages]; row_seq int32 [rows] or None.  Returns (out_table
    int32 [rows][out_stride], out_len int32 [rows], out_status int32 [rows]),
    allocating them when not given."""
    import torch

    if tokens.dim() != 2 or tokens.dtype != torch.int32 or (tokens.shape[1] > 1 and
                                                            tokens.stride(1) != 1):
        raise ValueError("tokens must be an int32 [rows][n] tensor with unit column stride")
    if block_table.dim() != 2 or block_table.dtype != torch.int32 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [n_seqs][max_pages] tensor")
    rows, n = tokens.shape
    dev = tokens.device
    _expect(live_len, "live_len", torch.int32, (rows,))
    if row_seq is not None:
        _expect(row_seq, "row_seq", torch.int32, (rows,))
    if out_table is None:
        out_table = torch.empty((rows, out_stride), dtype=torch.int32, device=dev)
    else:
        _expect(out_table, "out_table", torch.int32, (rows, out_stride))
    if out_len is None:
        out_len = torch.empty(rows, dtype=torch.int32, device=dev)
    else:
        _expect(out_len, "out_len", torch.int32, (rows,))
    if out_status is None:
        out_status = torch.empty(rows, dtype=torch.int32, device=dev)
    else:
        _expect(out_status, "out_status", torch.int32, (rows,))
    _device(tokens=tokens, live_len=live_len, block_table=block_table, row_seq=row_seq,
            out_table=out_table, out_len=out_len, out_status=out_status)
    stride = tokens.stride(0) if rows > 1 and n > 0 else n
    rc = _lib().qsa_build_page4_table(
        _ptr(tokens), int(stride), int(n), _ptr(live_len), _ptr(block_table),
        int(block_table.shape[1]), _ptr(row_seq), int(block_table.shape[0]), int(num_pages),
        int(page_size), int(vpages_per_page), int(rows), _ptr(out_table), int(out_stride),
        _ptr(out_len), _ptr(out_status), _stream_handle(stream))
    _check(rc, "qsa_build_page4_table")
    return out_table, out_len, out_status


def sampler_topk_topp_workspace_bytes(rows: int, vocab: int, k_max: int = SAMPLER_MAX_K) -> int:
    r = _lib().sampler_topk_topp_workspace_bytes(int(rows), int(vocab), int(k_max))
    if r == ctypes.c_size_t(-1).value:
        raise PgqaError(PGQA_ERR_SHAPE, "sampler_topk_topp_workspace_bytes")
    return int(r)


def sampler_topk_topp_mask(logits, k, p, *, k_max: int = SAMPLER_MAX_K, out=None, status=None,
                           workspace=None, stream=None):
    """Combined top-k/top-p masking of fp32 logits [rows][vocab] (see
    include/pgqa.h).  k: int32 [rows]; p: float32 [rows] (device tensors).
    out may be `logits` (in place).  Returns (out, status), allocating them
    and the workspace when not given."""
    import torch

    if logits.dim() != 2 or logits.dtype != torch.float32 or logits.stride(1) != 1:
        raise ValueError("logits must be a float32 [rows][vocab] tensor with unit column stride")
    rows, vocab = logits.shape
    dev = logits.device
    _expect(k, "k", torch.int32, (rows,))
    _expect(p, "p", torch.float32, (rows,))
    if out is None:
        out = torch.empty_like(logits)
    else:
        _expect(out, "out", torch.float32, (rows, vocab), dense=False)
        if vocab > 1 and out.stride(1) != 1:
            raise ValueError("out must have unit column stride")
    if status is None:
        status = torch.empty(rows, dtype=torch.int32, device=dev)
    else:
        _expect(status, "status", torch.int32, (rows,))
    if workspace is None:
        wsb = sampler_topk_topp_workspace_bytes(rows, vocab, k_max)
        workspace = torch.empty(max(wsb, 8), dtype=torch.uint8, device=dev)
    else:
        _expect(workspace, "workspace", workspace.dtype)
    _device(logits=logits, k=k, p=p, out=out, status=status, workspace=workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    stride = logits.stride(0) if rows > 1 else vocab
    ostride = out.stride(0) if rows > 1 else vocab
    rc = _lib().sampler_topk_topp_mask(_ptr(logits), int(stride), int(rows), int(vocab), _ptr(k),
                                       _ptr(p), int(k_max), _ptr(out), int(ostride),
                                       _ptr(status), _ptr(workspace), ws_bytes,
                                       _stream_handle(stream))
    _check(rc, "sampler_topk_topp_mask")
    return out, status


# ------------------------------------------------------------ device inputs
def device_case(case, device="cuda"):
    """Copy a host PagedCase (fp8_kv_amd.inputs) to device memory.

    Returns (q, pool, table, lens) as device tensors / KVPool."""
    import torch

    q = torch.from_numpy(case.q).to(device)
    ks = torch.from_numpy(case.k_store).to(device)
    if case.v_store is case.k_store:
        vs = ks
    else:
        vs = torch.from_numpy(case.v_store).to(device)
    kflat, vflat = ks.reshape(-1), vs.reshape(-1)
    pool = KVPool(k=kflat[case.k_offset:], v=vflat[case.v_offset:],
                  page_stride=case.page_stride, token_stride=case.token_stride,
                  head_stride=case.head_stride, num_pages=case.num_pages,
                  page_size=case.page_size, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                  v_scale=case.v_scale, storage=(ks, vs))
    table = torch.from_numpy(case.table).to(device)
    lens = torch.from_numpy(case.lens).to(device)
    return q, pool, table, lens


def run_case(case, *, prefill: bool = False, num_splits: int = 0, device="cuda", stream=None):
    """Run one PagedCase through the library; returns the fp16 output tensor."""
    import torch

    q, pool, table, lens = device_case(case, device)
    n, hq, _ = q.shape
    out = torch.empty_like(q)
    wsb = paged_gqa_workspace_bytes(n, hq, case.num_kv_heads, case.max_seq_len, num_splits)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=device) if wsb else None
    fn = paged_gqa_prefill_sparse if prefill else paged_gqa_decode
    fn(q, pool, table, lens, case.max_seq_len, case.sm_scale, out,
       num_kv_heads=case.num_kv_heads, workspace=ws, num_splits=num_splits, stream=stream)
    return out
