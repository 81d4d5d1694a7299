"""CPU oracle for the MSA index-branch block score.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path (the HIP
library and its Python binding) never imports this package.

The arithmetic lives in ``msa_oracle.c`` (plain loops, binary64); this module
compiles it with gcc and marshals CPU tensors into it with ctypes.

Parity pins (see tests/test_oracle_pins.py): every decoder against torch's own
conversion over all codes; a vectorised brute force (full Q.K^T -> mask ->
reshape -> amax, the form of the DSA block-selection sketch); closed forms for
the causal window; GQA, layout, paging, poison and homogeneity invariants; the
int8 dequant identity; the local_mask constants; and the worked tiny example's
structure.  The top-k selection is pinned by a rank-counting brute force, by
its invariance under a strictly increasing map of the scores (the exp-free
property) and by constructed cases (ties, -inf rows, forced blocks).  Finite values of the worked example are not printed by the pages,
so beyond the brute force they are parity-unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "msa_oracle.c")
LIB = os.path.join(HERE, "libmsa_oracle.so")

_DT = {
    torch.float16: 0,
    torch.bfloat16: 1,
    torch.int8: 2,
    torch.float8_e4m3fn: 3,
    torch.float8_e5m2: 4,
    torch.uint8: 5,          # MXFP4: E2M1 values packed two per byte, low nibble first
}
_LAYOUT = {"TND": 0, "BBND": 1, "BNBD": 2}

_lock = threading.Lock()
_lib = None


def default_threads() -> int:
    """Worker threads when the caller passes 0: OMP_NUM_THREADS if set, else
    up to 16 of the host's cores."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, os.cpu_count() or 1))


def build(force: bool = False, out: str = LIB, src: str = SRC) -> str:
    """Compile the oracle (gcc, -O2, no FP contraction)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                               "-pthread", "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def load(path: Optional[str] = None):
    """Load the compiled oracle (building it first if needed)."""
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None:
            _lib = _bind(ctypes.CDLL(build()))
        return _lib


def _bind(lib):
    c = ctypes
    p = c.c_void_p
    common = [p, c.c_int, c.c_int64, c.c_int, c.c_int,          # q
              p, c.c_int, c.c_int, c.c_int64, c.c_int, c.c_int,  # k
              p, p, p, c.c_int64, p, p, p, p, p, c.c_int,        # strides..B
              c.c_int, c.c_int, c.c_int, c.c_int]                # modes, counts
    lib.orc_index_score.argtypes = common + [p, c.c_int]
    lib.orc_index_score.restype = c.c_int
    lib.orc_index_score_points.argtypes = common + [p, c.c_int64, p, c.c_int]
    lib.orc_index_score_points.restype = c.c_int
    lib.orc_out_width.argtypes = [c.c_int64]
    lib.orc_out_width.restype = c.c_int64
    lib.orc_decode_e2m1.argtypes = [c.c_uint8]
    lib.orc_decode_e2m1.restype = c.c_double
    lib.orc_decode_e8m0.argtypes = [c.c_uint8]
    lib.orc_decode_e8m0.restype = c.c_double
    lib.orc_decode_buffer.argtypes = [p, c.c_int, c.c_int64, p]
    lib.orc_decode_buffer.restype = None
    lib.orc_block_topk.argtypes = [p, c.c_int64, c.c_int64, c.c_int64, c.c_int64, c.c_int, p]
    lib.orc_block_topk.restype = c.c_int
    return lib


def out_width(max_blocks: int, lib=None) -> int:
    return int((lib or load()).orc_out_width(int(max_blocks)))


def decode(buf: torch.Tensor, lib=None) -> np.ndarray:
    """Decode every element of a CPU tensor to float64 with the oracle's own
    decoders (uint8 holds packed MXFP4 pairs: two elements per byte, without
    their group scales)."""
    buf = buf.contiguous()
    n = buf.numel() * (2 if buf.dtype == torch.uint8 else 1)
    out = np.empty(n, dtype=np.float64)
    (lib or load()).orc_decode_buffer(ctypes.c_void_p(buf.data_ptr()), _DT[buf.dtype],
                                      n, out.ctypes.data)
    return out


def _i32(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    assert t.device.type == "cpu"
    return t.to(torch.int32).contiguous()


def _common(query, key, layout, start_loc, block_table, scale, cu_seqlens_q, kv_len,
            max_blocks, sparse_mode, init_blocks, local_blocks, local_mode=0,
            q_mx_scale=None, k_mx_scale=None, block_size=128):
    layout = layout.upper()
    assert query.device.type == "cpu" and key.device.type == "cpu"
    q = query.contiguous()
    T, Hq, D = q.shape
    mx = q.dtype == torch.uint8           # MXFP4: the last axis holds 2 elements per byte
    if mx:
        D *= 2
    if layout == "TND":
        Hkv, P = key.shape[1], int(block_size)
        strides = list(key.stride()) + [0]
    elif layout == "BBND":
        Hkv, P = key.shape[2], key.shape[1]
        strides = list(key.stride())
    elif layout == "BNBD":
        Hkv, P = key.shape[1], key.shape[2]
        strides = list(key.stride())
    else:
        raise ValueError(layout)
    if mx:
        # element strides of the packed key: outer axes in bytes * 2, D axis 1
        strides = [2 * x for x in strides[:-1]] + [1] if layout != "TND" else \
            [2 * strides[0], 2 * strides[1], 1, 0]
    ks = np.asarray(strides, dtype=np.int64)
    sl = _i32(start_loc)
    bt = _i32(block_table)
    cu = _i32(cu_seqlens_q)
    kv = _i32(kv_len)
    sc = scale.to(torch.float32).contiguous() if scale is not None else None
    qmx = q_mx_scale.contiguous() if q_mx_scale is not None else None
    kmx = k_mx_scale.contiguous() if k_mx_scale is not None else None
    keep = (q, key, ks, sl, bt, cu, kv, sc, qmx, kmx)

    def ptr(t):
        if t is None:
            return None
        if isinstance(t, np.ndarray):
            return t.ctypes.data
        return t.data_ptr()

    args = [ptr(q), _DT[q.dtype], T, Hq, D,
            ptr(key), _DT[key.dtype], _LAYOUT[layout], key.shape[0], Hkv, P,
            ptr(ks), ptr(sl), ptr(bt), int(max_blocks), ptr(sc), ptr(qmx), ptr(kmx),
            ptr(cu), ptr(kv),
            int(kv.numel()), int(sparse_mode), int(init_blocks), int(local_blocks),
            int(local_mode)]
    return args, keep, (Hq, T)


def index_score(query, key, layout, start_loc, block_table, scale, cu_seqlens_q, kv_len,
                max_blocks, sparse_mode=3, init_blocks=0, local_blocks=1, local_mode=0,
                q_mx_scale=None, k_mx_scale=None,
                nthreads: int = 0, lib=None) -> Tuple[torch.Tensor, int]:
    """Full output ``[Hq, T, RoundUp(MB,16)]`` float32 and the thread count used.
    ``local_mode`` 1 ends the local_mask window at each token's own block
    (start_loc is then not read)."""
    lib = lib or load()
    args, keep, (Hq, T) = _common(query, key, layout, start_loc, block_table, scale,
                                  cu_seqlens_q, kv_len, max_blocks, sparse_mode,
                                  init_blocks, local_blocks, local_mode, q_mx_scale,
                                  k_mx_scale)
    W = out_width(max_blocks, lib)
    out = torch.empty((Hq, T, W), dtype=torch.float32)
    rc = lib.orc_index_score(*args, out.data_ptr(), int(nthreads or default_threads()))
    if rc < 0:
        raise ValueError(f"oracle: inputs break the caller contract (code {rc})")
    del keep
    return out, rc


def index_score_points(query, key, layout, start_loc, block_table, scale, cu_seqlens_q,
                       kv_len, max_blocks, sparse_mode, init_blocks, local_blocks,
                       points: torch.Tensor, local_mode=0, q_mx_scale=None,
                       k_mx_scale=None, nthreads: int = 0, lib=None) -> torch.Tensor:
    """Entries ``out[h, t, beta]`` for the rows of ``points`` (int64 [n, 3])."""
    lib = lib or load()
    args, keep, _ = _common(query, key, layout, start_loc, block_table, scale,
                            cu_seqlens_q, kv_len, max_blocks, sparse_mode, init_blocks,
                            local_blocks, local_mode, q_mx_scale, k_mx_scale)
    pts = points.to(torch.int64).contiguous()
    vals = torch.empty(pts.shape[0], dtype=torch.float32)
    rc = lib.orc_index_score_points(*args, pts.data_ptr(), pts.shape[0], vals.data_ptr(),
                                    int(nthreads or default_threads()))
    if rc < 0:
        raise ValueError(f"oracle: inputs break the caller contract (code {rc})")
    del keep
    return vals


def case_args(case) -> dict:
    """Keyword arguments for ``index_score`` from any object carrying the
    operator's inputs as attributes (e.g. a generated test case)."""
    return dict(query=case.query, key=case.key, layout=case.layout,
                start_loc=case.start_loc, block_table=case.block_table, scale=case.scale,
                cu_seqlens_q=case.cu_seqlens_q, kv_len=case.kv_len,
                max_blocks=case.max_blocks, sparse_mode=case.sparse_mode,
                init_blocks=case.init_blocks, local_blocks=case.local_blocks,
                local_mode=getattr(case, "local_mode", 0),
                q_mx_scale=getattr(case, "q_mx_scale", None),
                k_mx_scale=getattr(case, "k_mx_scale", None))


def index_score_case(case, nthreads: int = 0, lib=None) -> torch.Tensor:
    return index_score(**case_args(case), nthreads=nthreads, lib=lib)[0]


def index_score_case_points(case, points, nthreads: int = 0, lib=None) -> torch.Tensor:
    return index_score_points(**case_args(case), points=points, nthreads=nthreads, lib=lib)


def block_topk(scores: torch.Tensor, num_valid: Optional[int] = None, k: int = 16,
               lib=None) -> torch.Tensor:
    """Top-k block selection on a CPU float32 score tensor [Hq, T, W]: for each
    (t, h) the k best blocks among beta < num_valid (default W) with a score
    above -inf, highest score first and ties to the lower index, returned as
    int32 [T, Hq, k] in ascending block order with -1 for missing entries."""
    assert scores.device.type == "cpu" and scores.dtype == torch.float32 and scores.dim() == 3
    s = scores.contiguous()
    Hq, T, W = s.shape
    nv = W if num_valid is None else int(num_valid)
    out = torch.empty((T, Hq, k), dtype=torch.int32)
    rc = (lib or load()).orc_block_topk(ctypes.c_void_p(s.data_ptr()), Hq, T, W, nv, int(k),
                                        ctypes.c_void_p(out.data_ptr()))
    if rc != 0:
        raise ValueError("block_topk: contract violation (%d)" % rc)
    return out
