"""ctypes binding of libmsa_index_score.so (argument marshalling only).

Every step of the operator runs in the HIP library; this module only turns
torch tensors into the C ABI's plain descriptors and pointers, passes torch's
current HIP stream, and turns a non-zero status into an exception.  If the
library is missing the call raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsa_index_score.so")

# msa_dtype_t / msa_layout_t / msa_status_t of include/msa_index_score.h
DTYPE_CODE = {
    torch.float16: 0,
    torch.bfloat16: 1,
    torch.int8: 2,
    torch.float8_e4m3fn: 3,
    torch.float8_e5m2: 4,
    torch.uint8: 5,          # MXFP4: E2M1 pairs, with E8M0 group scales alongside
}
LAYOUT_CODE = {"TND": 0, "BBND": 1, "BNBD": 2}
STATUS_NAMES = ["MSA_OK", "MSA_ERR_NULL", "MSA_ERR_LAYOUT", "MSA_ERR_DTYPE", "MSA_ERR_SHAPE",
                "MSA_ERR_STRIDE", "MSA_ERR_SCALE", "MSA_ERR_ATTR", "MSA_ERR_HIP"]
EXPORTED = ("msa_index_score", "msa_index_score_family", "msa_index_score_ex",
            "msa_index_score_mxfp4", "msa_index_score_mxfp4_family",
            "msa_index_score_out_width", "msa_status_str",
            "msa_index_score_kernel_family", "msa_block_topk")
LOCAL_MODE_CODE = {"request": 0, "query": 1}


class MsaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else status}: "
                         f"{message}")
        self.status = status


class MsaLayoutError(MsaError, ValueError):
    pass


_lock = threading.Lock()
_lib = None


def load_library(path: Optional[str] = None):
    """Load the HIP library (built in-tree by ``block_max_qk_amd.build``)."""
    global _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"HIP library {p} is not built; run "
                               "`python -m block_max_qk_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(p)
        ptr = ctypes.c_void_p
        i32 = ctypes.c_int32
        # query, key, start_loc, block_table, max_blocks, scale, cu_seqlens_q,
        # kv_len, batch, block_size, layout, sparse_mode, init_blocks,
        # local_blocks, out, out_width, stream
        args = [ctypes.POINTER(MsaTensor), ctypes.POINTER(MsaTensor), ptr, ptr, ctypes.c_int64,
                ptr, ptr, ptr, i32, i32, i32, i32, i32, i32, ptr, ctypes.c_int64, ptr]
        lib.msa_index_score.argtypes = args
        lib.msa_index_score.restype = ctypes.c_int
        lib.msa_index_score_family.argtypes = args + [i32]
        lib.msa_index_score_family.restype = ctypes.c_int
        # local_mode after local_blocks, family last
        lib.msa_index_score_ex.argtypes = args[:14] + [i32] + args[14:] + [i32]
        lib.msa_index_score_ex.restype = ctypes.c_int
        lib.msa_index_score_mxfp4.argtypes = [
            ctypes.POINTER(MsaTensor), ptr, ctypes.POINTER(MsaTensor), ptr, ptr, ptr,
            ctypes.c_int64, ptr, ptr, i32, i32, i32, i32, i32, i32, i32, ptr, ctypes.c_int64,
            ptr]
        lib.msa_index_score_mxfp4.restype = ctypes.c_int
        lib.msa_index_score_mxfp4_family.argtypes = (lib.msa_index_score_mxfp4.argtypes +
                                                     [ctypes.c_int32])
        lib.msa_index_score_mxfp4_family.restype = ctypes.c_int
        lib.msa_index_score_out_width.argtypes = [ctypes.c_int64]
        lib.msa_index_score_out_width.restype = ctypes.c_int64
        lib.msa_status_str.argtypes = [ctypes.c_int32]
        lib.msa_status_str.restype = ctypes.c_char_p
        lib.msa_index_score_kernel_family.argtypes = [ctypes.c_int64, ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.c_int32]
        lib.msa_index_score_kernel_family.restype = ctypes.c_int32
        lib.msa_block_topk.argtypes = [ptr, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int32, ptr, ptr]
        lib.msa_block_topk.restype = ctypes.c_int
        if path is None:
            _lib = lib
        return lib


def describe(t: torch.Tensor, dtype_code: Optional[int] = None) -> MsaTensor:
    """Descriptor of a tensor: data pointer, element type, shape, strides."""
    d = MsaTensor()
    d.data = t.data_ptr() if t.numel() else (t.data_ptr() or None)
    d.dtype = DTYPE_CODE.get(t.dtype, -1) if dtype_code is None else dtype_code
    d.ndim = t.dim()
    for i in range(min(t.dim(), 4)):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _layout_code(layout) -> int:
    if isinstance(layout, str):
        return LAYOUT_CODE.get(layout.upper(), -1)
    return int(layout)


def msa_index_score_out_width(max_blocks: int) -> int:
    return int(load_library().msa_index_score_out_width(int(max_blocks)))


def msa_status_str(status: int) -> str:
    return load_library().msa_status_str(int(status)).decode()


def msa_index_score_kernel_family(T: int, batch: int, Hq: int, Hkv: int) -> int:
    return int(load_library().msa_index_score_kernel_family(int(T), int(batch), int(Hq),
                                                            int(Hkv)))


BLOCK_SIZE = 128   # tokens per logical block (guide to msa_index_score, section 四)
MASK_SHAPE = (2048, 2048)   # the compressed causal template of sparse_mode 3


def _stream_handle(stream, dev):
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def _local_mode_code(local_mode) -> int:
    return LOCAL_MODE_CODE.get(local_mode, -1) if isinstance(local_mode, str) else int(local_mode)


def _check_batch(query, out, start_loc, block_table, cu_seqlens_q, kv_len, max_blocks,
                 local_mode) -> int:
    """Sizes the C ABI takes on trust (it sees plain pointers): the request
    count B from kv_len, and the tensors whose extents follow from it and from
    the query.  Returns B."""
    if kv_len.dim() != 1:
        raise ValueError("kv_len must be 1-D [B] (per-request lengths)")
    B = int(kv_len.numel())
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.numel() != B + 1:
        raise ValueError(f"cu_seqlens_q must be [B+1] = [{B + 1}], got "
                         f"{tuple(cu_seqlens_q.shape)}")
    if start_loc is None:
        if _local_mode_code(local_mode) != 1 and B > 0:
            raise ValueError("start_loc is required unless local_mode is 'query'")
    elif start_loc.dim() != 1 or start_loc.numel() != B:
        raise ValueError(f"start_loc must be [B] = [{B}], got {tuple(start_loc.shape)}")
    if block_table is not None:
        if (block_table.dim() != 2 or block_table.shape[0] < B or
                block_table.shape[1] != int(max_blocks)):
            raise ValueError(f"block_table must be [>= {B}, max_blocks = {int(max_blocks)}], "
                             f"got {tuple(block_table.shape)}")
    if query.dim() == 3 and (out.shape[0] != query.shape[1] or out.shape[1] != query.shape[0]):
        raise ValueError(f"out must be [Hq, T, W] = [{query.shape[1]}, {query.shape[0]}, W], "
                         f"got {tuple(out.shape)}")
    return B


def _key_rows(key: torch.Tensor, layout: int):
    """(rows, Hkv) of a key tensor: token rows of one KV head across the cache
    (NP * 128 paged, T2 packed) and the KV head count, or None if the shape
    does not fit the layout (the C ABI then reports it)."""
    if layout == 0 and key.dim() == 3:
        return key.shape[0], key.shape[1]
    if layout == 1 and key.dim() == 3:
        return key.shape[0] * key.shape[1], 1
    if layout == 1 and key.dim() == 4:
        return key.shape[0] * key.shape[1], key.shape[2]
    if layout == 2 and key.dim() == 4:
        return key.shape[0] * key.shape[2], key.shape[1]
    return None


def _raise_status(st: int):
    if st != 0:
        cls = MsaLayoutError if st == 2 else MsaError
        raise cls(st, msa_status_str(st))


def msa_index_score(query: torch.Tensor, key: torch.Tensor, start_loc: torch.Tensor,
                    block_table: Optional[torch.Tensor], scale: Optional[torch.Tensor],
                    cu_seqlens_q: torch.Tensor, kv_len: torch.Tensor, layout,
                    sparse_mode: int, init_blocks: int, local_blocks: int, out: torch.Tensor,
                    max_blocks: int, stream=None, family: int = -1,
                    local_mode=0, block_size: int = BLOCK_SIZE) -> torch.Tensor:
    """Call the C ABI on device tensors; ``out`` ([Hq, T, W] float32) is filled
    asynchronously on ``stream`` (default: torch's current stream).
    ``kv_len`` holds per-request lengths [B] for every layout.
    ``local_mode`` 0/"request" ends the local window at start_loc, 1/"query"
    at each token's own block (start_loc may then be None)."""
    lib = load_library()
    dev = out.device
    for name, t in (("query", query), ("key", key), ("start_loc", start_loc),
                    ("cu_seqlens_q", cu_seqlens_q), ("kv_len", kv_len),
                    ("block_table", block_table), ("scale", scale)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, out on {dev}")
    for name, t in (("start_loc", start_loc), ("cu_seqlens_q", cu_seqlens_q),
                    ("kv_len", kv_len), ("block_table", block_table)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    if scale is not None and (scale.dtype != torch.float32 or not scale.is_contiguous()):
        raise ValueError("scale must be a contiguous float32 tensor")
    if out.dtype != torch.float32 or not out.is_contiguous() or out.dim() != 3:
        raise ValueError("out must be a contiguous float32 [Hq, T, W] tensor")
    B = _check_batch(query, out, start_loc, block_table, cu_seqlens_q, kv_len, max_blocks,
                     local_mode)
    lay = _layout_code(layout)
    kr = _key_rows(key, lay)
    if scale is not None and kr is not None and scale.numel() != kr[0] * kr[1]:
        # paged [NP, Hkv, 128], packed [T2, Hkv]: one float per key row and head
        raise ValueError(f"scale must hold {kr[0] * kr[1]} floats (one per key token and KV "
                         f"head), got {scale.numel()}")
    stream = _stream_handle(stream, dev)
    qd, kd = describe(query), describe(key)
    args = (ctypes.byref(qd), ctypes.byref(kd), _ptr(start_loc), _ptr(block_table),
            int(max_blocks), _ptr(scale), _ptr(cu_seqlens_q), _ptr(kv_len), B,
            int(block_size), lay, int(sparse_mode), int(init_blocks), int(local_blocks),
            _ptr(out), int(out.shape[2]), ctypes.c_void_p(stream))
    lm = _local_mode_code(local_mode)
    if lm != 0:
        st = lib.msa_index_score_ex(*args[:14], lm, *args[14:], int(family))
    elif family == -1:
        st = lib.msa_index_score(*args)
    else:
        st = lib.msa_index_score_family(*args, int(family))
    _raise_status(st)
    return out


def msa_index_score_mxfp4(query: torch.Tensor, query_scale: torch.Tensor, key: torch.Tensor,
                          key_scale: torch.Tensor, start_loc: Optional[torch.Tensor],
                          block_table: Optional[torch.Tensor], cu_seqlens_q: torch.Tensor,
                          kv_len: torch.Tensor, layout, sparse_mode: int, init_blocks: int,
                          local_blocks: int, out: torch.Tensor, max_blocks: int, stream=None,
                          local_mode=0, family: int = -1,
                          block_size: int = BLOCK_SIZE) -> torch.Tensor:
    """The MXFP4 entry: ``query`` [T, Hq, 64] and ``key`` (layout-shaped, last
    axis 64) uint8 hold E2M1 pairs; ``query_scale`` [T, Hq, 4] and
    ``key_scale`` (the key's layout with a last axis of 4) uint8 hold E8M0.
    ``family`` -1 picks the kernel family from the sizes, 0/1 force the
    decode/prefill tiles."""
    lib = load_library()
    dev = out.device
    for name, t in (("query", query), ("query_scale", query_scale), ("key", key),
                    ("key_scale", key_scale), ("start_loc", start_loc),
                    ("cu_seqlens_q", cu_seqlens_q), ("kv_len", kv_len),
                    ("block_table", block_table)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, out on {dev}")
    for name, t in (("query", query), ("key", key), ("query_scale", query_scale),
                    ("key_scale", key_scale)):
        if t.dtype != torch.uint8:
            raise ValueError(f"{name} must be uint8 (MXFP4 values / E8M0 scales)")
    for name, t in (("start_loc", start_loc), ("cu_seqlens_q", cu_seqlens_q),
                    ("kv_len", kv_len), ("block_table", block_table)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    for name, t in (("query_scale", query_scale), ("key_scale", key_scale)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out.dtype != torch.float32 or not out.is_contiguous() or out.dim() != 3:
        raise ValueError("out must be a contiguous float32 [Hq, T, W] tensor")
    B = _check_batch(query, out, start_loc, block_table, cu_seqlens_q, kv_len, max_blocks,
                     local_mode)
    lay = _layout_code(layout)
    # one E8M0 byte per 32 elements: 4 per 64-byte row
    if query.dim() == 3 and query_scale.numel() != query.shape[0] * query.shape[1] * 4:
        raise ValueError("query_scale must be [T, Hq, 4]")
    kr = _key_rows(key, lay)
    if kr is not None and key_scale.numel() != kr[0] * kr[1] * 4:
        raise ValueError("key_scale must hold 4 bytes per key token and KV head (the key's "
                         "layout with a last axis of 4)")
    stream = _stream_handle(stream, dev)
    qd, kd = describe(query), describe(key)
    st = lib.msa_index_score_mxfp4_family(
        ctypes.byref(qd), _ptr(query_scale), ctypes.byref(kd), _ptr(key_scale),
        _ptr(start_loc), _ptr(block_table), int(max_blocks), _ptr(cu_seqlens_q),
        _ptr(kv_len), B, int(block_size), lay, int(sparse_mode), int(init_blocks),
        int(local_blocks), _local_mode_code(local_mode), _ptr(out), int(out.shape[2]),
        ctypes.c_void_p(stream), int(family))
    _raise_status(st)
    return out


def index_score(query: torch.Tensor, key: torch.Tensor, start_loc: torch.Tensor, *,
                block_table: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                atten_mask: Optional[torch.Tensor] = None,
                actual_seq_qlen: Optional[torch.Tensor] = None,
                actual_seq_klen: Optional[torch.Tensor] = None, layout_key: str = "BBND",
                sparse_mode: int = 3, init_blocks: int = 0, local_blocks: int = 1,
                max_blocks: Optional[int] = None, stream=None, family: int = -1,
                local_mode=0) -> torch.Tensor:
    """The guide's keyword interface (sections 三 and 四): allocate
    ``[Hq, T, RoundUp(MB, 16)]`` float32 and fill it.

    * ``layout_key`` is upper-cased; anything but TND/BBND/BNBD is a ValueError.
    * ``atten_mask``: with ``sparse_mode`` 3 an int8 ``[2048, 2048]`` tensor
      is required, with 0 none may be passed.  It is only checked: the
      right-down causal window is computed from the lengths, the mask
      template is never read.
    * ``actual_seq_qlen``: the ``[B+1]`` query prefix sum.
    * ``actual_seq_klen``: paged layouts take the ``[B]`` per-request lengths,
      TND the ``[B+1]`` prefix sum of the packed key, which is differenced
      into lengths here.
    * MB is ``block_table.shape[1]`` for paged keys; for packed keys pass
      ``max_blocks`` or it is the largest ``ceil(length / 128)``, read from a
      host copy of the lengths (a device synchronisation), ``ceil(T2/128)``
      when the batch is empty.
    """
    lay = layout_key.upper() if isinstance(layout_key, str) else layout_key
    if isinstance(lay, str) and lay not in LAYOUT_CODE:
        raise ValueError(f"layout_key must be one of TND/BBND/BNBD, got {layout_key!r}")
    if int(sparse_mode) == 3:
        if atten_mask is None:
            raise ValueError("sparse_mode 3 needs the [2048, 2048] int8 atten_mask")
        if tuple(atten_mask.shape) != MASK_SHAPE or atten_mask.dtype != torch.int8:
            raise ValueError(f"atten_mask must be int8 {list(MASK_SHAPE)}, got "
                             f"{atten_mask.dtype} {list(atten_mask.shape)}")
    elif atten_mask is not None:
        raise ValueError(f"atten_mask must not be passed with sparse_mode {sparse_mode}")
    if actual_seq_qlen is None or actual_seq_klen is None:
        raise ValueError("actual_seq_qlen and actual_seq_klen are required")
    packed = (lay == "TND") if isinstance(lay, str) else int(lay) == 0
    kv_len = actual_seq_klen
    if packed:
        if actual_seq_klen.dim() != 1 or actual_seq_klen.numel() < 1:
            raise ValueError("TND actual_seq_klen must be the [B+1] key prefix sum")
        kv_len = (actual_seq_klen[1:] - actual_seq_klen[:-1]).to(torch.int32).contiguous()
    if max_blocks is None:
        if block_table is not None:
            max_blocks = int(block_table.shape[1])
        else:
            kv = kv_len.to("cpu", torch.int64)
            max_blocks = (int(((kv + 127) // 128).max()) if kv.numel()
                          else (int(key.shape[0]) + 127) // 128)
    W = msa_index_score_out_width(max_blocks)
    out = torch.empty((query.shape[1], query.shape[0], W), dtype=torch.float32,
                      device=query.device)
    return msa_index_score(query, key, start_loc, block_table, scale, actual_seq_qlen, kv_len,
                           lay, sparse_mode, init_blocks, local_blocks, out, max_blocks,
                           stream=stream, family=family, local_mode=local_mode)


def msa_block_topk(scores: torch.Tensor, num_valid: int, k: int, out: torch.Tensor,
                   stream=None) -> torch.Tensor:
    """Call the C ABI: ``out`` ([T, Hq, k] int32) receives, for every row of
    ``scores`` ([Hq, T, W] float32 on the same device), the k best blocks
    below ``num_valid`` in ascending block order with a -1 tail;
    asynchronous on ``stream`` (default: torch's current stream)."""
    lib = load_library()
    if scores.dtype != torch.float32 or not scores.is_contiguous() or scores.dim() != 3:
        raise ValueError("scores must be a contiguous float32 [Hq, T, W] tensor")
    Hq, T, W = scores.shape
    if out.dtype != torch.int32 or not out.is_contiguous() or tuple(out.shape) != (T, Hq, k):
        raise ValueError(f"out must be a contiguous int32 [{T}, {Hq}, {k}] tensor")
    if out.device != scores.device:
        raise ValueError(f"scores are on {scores.device}, out on {out.device}")
    if stream is None:
        stream = torch.cuda.current_stream(scores.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    st = lib.msa_block_topk(_ptr(scores), Hq, T, W, int(num_valid), int(k), _ptr(out),
                            ctypes.c_void_p(stream))
    if st != 0:
        raise MsaError(st, msa_status_str(st))
    return out


def block_topk(scores: torch.Tensor, num_valid: Optional[int] = None, k: int = 16,
               stream=None) -> torch.Tensor:
    """Allocate ``[T, Hq, k]`` int32 and fill it with the top-k selection of
    the score rows (``num_valid`` defaults to the row width)."""
    Hq, T, W = scores.shape
    out = torch.empty((T, Hq, k), dtype=torch.int32, device=scores.device)
    return msa_block_topk(scores, W if num_valid is None else num_valid, k, out, stream=stream)
