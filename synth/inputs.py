"""Seeded synthetic inputs for ``msa_index_score``.

Everything here is input *generation*: drawing index queries/keys, int8 keys
and their fp32 scales, paged block tables and per-request lengths, and laying
them out in the three key layouts the operator accepts (packed TND, paged BBND
``[pages, block, kv_heads, dim]`` and paged BNBD ``[pages, kv_heads, block,
dim]``).  No score, mask or maximum is computed here.

Random numbers come from numpy's PCG64 ``Generator`` seeded per case, drawn in
a fixed order: ``kv_len`` -> ``block_table`` -> query -> key -> scale.  Large
tensors are filled chunk by chunk into a preallocated buffer so that a 512 MB
key cache never needs a second full-size float32 copy.

Distributions (from the workload descriptions):
  * query/key of a float type: N(0, 1) in float32, rounded to nearest even in
    the storage type; for fp8 e4m3 the float32 value is clamped to +-448 first.
  * int8 key: uniform integers in [-127, 127].
  * int8 scale: lognormal(mu=-6, sigma=0.5), float32.
  * MXFP4 query/key: N(0, 1) in float32 encoded as OCP microscaling FP4 --
    per group of 32 elements along D a shared E8M0 exponent
    floor(log2(max|v|)) - 2 (E2M1's largest exponent) and the elements
    divided by it and rounded to the nearest E2M1 value (ties to the even
    code, saturating at 6); two elements per byte, the even one in the low
    nibble.  This is the encoding of the inputs, not part of the operator.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

DTYPES = {
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "i8": torch.int8,
    "f8e4m3": torch.float8_e4m3fn,
    "f8e5m2": torch.float8_e5m2,
    "mxfp4": torch.uint8,               # packed E2M1 pairs, with E8M0 group scales
}

# The five workloads the operator is measured on, in order.
CONFIG_NAMES = (
    "tiny_bbnd_f16",        # B=1, T=32, Hq=8, Hkv=1, kv_len=256, 8 pages, MB=2
    "decode_bbnd_bf16",     # B=64 q_len=1, Hq=16, Hkv=1, kv_len~U[1,32768], 16384 pages
    "prefill_tnd_bf16",     # B=4 q_len {1K,2K,4K,8K} after {0,4K,16K,56K} prefix, Hq=32, Hkv=4
    "decode_bnbd_i8",       # B=32 q_len=1, Hq=16, Hkv=1, kv_len~U[65536,131072], int8 K + scale
    "prefill_bbnd_f8e4m3",  # B=1, 4096 tokens after 126976 prefix, Hq=64, Hkv=8, fp8 e4m3
)

_CHUNK = 1 << 22


@dataclasses.dataclass
class MsaCase:
    """One set of operator inputs (CPU tensors)."""

    name: str
    query: torch.Tensor                 # [T, Hq, D]
    key: torch.Tensor                   # layout-shaped view, dim0 may be strided
    key_storage: torch.Tensor           # the buffer ``key`` views
    layout: str                         # "TND" | "BBND" | "BNBD"
    block_table: Optional[torch.Tensor]  # int32 [B, MB] (paged layouts)
    scale: Optional[torch.Tensor]       # float32, int8 keys only
    cu_seqlens_q: torch.Tensor          # int32 [B+1]
    kv_len: torch.Tensor                # int32 [B]
    start_loc: torch.Tensor             # int32 [B], logical block index
    max_blocks: int                     # MB
    sparse_mode: int
    init_blocks: int
    local_blocks: int
    block_size: int = 128
    gap: int = 0                        # unused pages between used ones (paged)
    poison: Optional[str] = None
    local_mode: int = 0                 # 0: window at start_loc; 1: at each token's block
    q_mx_scale: Optional[torch.Tensor] = None   # MXFP4: uint8 E8M0 [T, Hq, D/32]
    k_mx_scale: Optional[torch.Tensor] = None   # MXFP4: uint8 E8M0, key layout with D/32

    @property
    def batch(self) -> int:
        return int(self.kv_len.numel())

    @property
    def T(self) -> int:
        return int(self.query.shape[0])

    @property
    def Hq(self) -> int:
        return int(self.query.shape[1])

    @property
    def Hkv(self) -> int:
        if self.layout == "BNBD":
            return int(self.key.shape[1])
        return int(self.key.shape[-2])

    @property
    def D(self) -> int:
        return int(self.query.shape[2]) * (2 if self.query.dtype == torch.uint8 else 1)

    def key_dtype_name(self) -> str:
        return _dtype_name(self.key.dtype)

    def query_dtype_name(self) -> str:
        return _dtype_name(self.query.dtype)


def _dtype_name(dt: torch.dtype) -> str:
    for k, v in DTYPES.items():
        if v == dt:
            return k
    raise KeyError(dt)


def _fill_normal(out: torch.Tensor, rng: np.random.Generator, clamp: Optional[float] = None):
    flat = out.view(-1)
    n = flat.numel()
    if n == 0:
        return
    buf = np.empty(min(n, _CHUNK), dtype=np.float32)
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        b = buf[:m]
        rng.standard_normal(out=b, dtype=np.float32)
        tb = torch.from_numpy(b)
        if clamp is not None:
            tb.clamp_(-clamp, clamp)
        flat[i:i + m].copy_(tb)


def _fill_int8(out: torch.Tensor, rng: np.random.Generator):
    flat = out.view(-1)
    n = flat.numel()
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        flat[i:i + m].copy_(torch.from_numpy(rng.integers(-127, 128, size=m, dtype=np.int8)))


def _fill_values(out: torch.Tensor, rng: np.random.Generator):
    if out.dtype == torch.int8:
        _fill_int8(out, rng)
    elif out.dtype in (torch.float8_e4m3fn,):
        _fill_normal(out, rng, clamp=448.0)
    elif out.dtype in (torch.float8_e5m2,):
        _fill_normal(out, rng, clamp=57344.0)
    else:
        _fill_normal(out, rng)


_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _encode_mxfp4(x: np.ndarray):
    """float32 [n, D] -> (packed E2M1 uint8 [n, D/2], E8M0 uint8 [n, D/32])."""
    n, D = x.shape
    g = x.reshape(n, D // 32, 32)
    amax = np.abs(g).max(axis=2)
    _, ex = np.frexp(amax)                     # amax = m * 2^ex, m in [0.5, 1)
    e = np.where(amax > 0, ex - 1, -127) - 2   # floor(log2 amax) - 2
    code = np.clip(e + 127, 0, 254).astype(np.uint8)
    v = g / np.exp2(code.astype(np.float32) - 127.0)[:, :, None]
    a = np.minimum(np.abs(v), 6.0)
    dist = np.abs(a[..., None] - _E2M1_MAG) + (np.arange(8) & 1) * 1e-6
    idx = np.argmin(dist, axis=-1).astype(np.uint8)
    nib = idx | (((v < 0) & (idx > 0)).astype(np.uint8) << 3)
    nib = nib.reshape(n, D)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, code


def _fill_mxfp4(vals: torch.Tensor, scales: torch.Tensor, rng: np.random.Generator):
    """vals uint8 [..., D/2], scales uint8 [..., D/32]: rows of N(0,1) encoded."""
    half = vals.shape[-1]
    fv = vals.reshape(-1, half)
    fs = scales.reshape(-1, scales.shape[-1])
    rows = fv.shape[0]
    step = max(1, _CHUNK // (2 * half))
    for i in range(0, rows, step):
        m = min(step, rows - i)
        x = rng.standard_normal(size=(m, 2 * half), dtype=np.float32)
        pk, sc = _encode_mxfp4(x)
        fv[i:i + m].copy_(torch.from_numpy(pk))
        fs[i:i + m].copy_(torch.from_numpy(sc))


def _fill_scale(out: torch.Tensor, rng: np.random.Generator):
    flat = out.view(-1)
    n = flat.numel()
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        flat[i:i + m].copy_(torch.from_numpy(
            rng.lognormal(mean=-6.0, sigma=0.5, size=m).astype(np.float32)))


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def make_case(name: str, seed: int, *, q_lens: Sequence[int], kv_lens: Sequence[int],
              Hq: int, Hkv: int, qdtype: str, kdtype: Optional[str] = None,
              layout: str = "BBND", D: int = 128, P: int = 128,
              MB: Optional[int] = None, NP: Optional[int] = None, gap: int = 0,
              table: str = "perm", sparse_mode: int = 3, init_blocks: int = 0,
              local_blocks: int = 1, start_loc: Optional[Sequence[int]] = None,
              kv_len_draw: Optional[tuple] = None, B: Optional[int] = None,
              extra_pages: int = 0, local_mode: int = 0) -> MsaCase:
    """Build one case.

    ``kv_len_draw=(lo, hi)`` draws ``kv_len`` uniformly in [lo, hi] from the
    case's generator instead of using ``kv_lens`` (then ``B`` gives the count).
    ``table`` is "perm" (a random permutation of the pages) or "arange".
    Paged layouts get ``NP`` pages, by default ``B*MB + extra_pages`` (the
    extra pages are never referenced by a request's visible blocks).
    ``start_loc`` defaults to the block holding each request's first query
    token, ``max(0, kv_len - q_len) // P``.  ``local_mode`` 1 anchors the
    local_mask window at each query token's own block instead.
    """
    layout = layout.upper()
    kdtype = kdtype or qdtype
    rng = np.random.default_rng(seed)

    # 1. kv_len
    if kv_len_draw is not None:
        lo, hi = kv_len_draw
        kv = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    else:
        kv = np.asarray(kv_lens, dtype=np.int64)
    B = int(kv.size)
    ql = np.asarray(q_lens, dtype=np.int64)
    if ql.size == 1 and B > 1:
        ql = np.full(B, int(ql[0]), dtype=np.int64)
    assert ql.size == B
    T = int(ql.sum())
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(ql)
    nb = np.array([_ceil_div(int(x), P) for x in kv], dtype=np.int64)
    if MB is None:
        MB = max(1, int(nb.max()) if B else 1)

    # 2. block_table (paged layouts)
    block_table = None
    if layout in ("BBND", "BNBD"):
        if NP is None:
            NP = B * MB + extra_pages
        assert NP >= 1
        if table == "perm":
            assert NP >= B * MB, "a permutation table needs NP >= B*MB"
            bt = rng.permutation(NP)[: B * MB].reshape(B, MB)
        elif table == "arange":
            assert NP >= B * MB
            bt = np.arange(B * MB).reshape(B, MB)
        else:
            raise ValueError(table)
        block_table = torch.from_numpy(bt.astype(np.int32)).contiguous()

    # 3. query
    mx = qdtype == "mxfp4"
    assert mx == (kdtype == "mxfp4"), "MXFP4 query and key go together"
    Dq = D // 2 if mx else D                   # stored last axis (bytes for MXFP4)
    query = torch.empty((T, Hq, Dq), dtype=DTYPES[qdtype])
    q_mx = k_mx = None
    if mx:
        q_mx = torch.empty((T, Hq, D // 32), dtype=torch.uint8)
        _fill_mxfp4(query, q_mx, rng)
    else:
        _fill_values(query, rng)

    # 4. key (MXFP4: the scales are indexed by logical page, dim0 gaps or not)
    if layout == "TND":
        T2 = int(kv.sum())
        key_storage = torch.empty((T2, Hkv, Dq), dtype=DTYPES[kdtype])
        if mx:
            k_mx = torch.empty((T2, Hkv, D // 32), dtype=torch.uint8)
            _fill_mxfp4(key_storage, k_mx, rng)
        else:
            _fill_values(key_storage, rng)
        key = key_storage
    else:
        NPs = NP * (gap + 1)
        shape = (NPs, P, Hkv, Dq) if layout == "BBND" else (NPs, Hkv, P, Dq)
        key_storage = torch.empty(shape, dtype=DTYPES[kdtype])
        if mx:
            sshape = (NPs, P, Hkv, D // 32) if layout == "BBND" else (NPs, Hkv, P, D // 32)
            full = torch.empty(sshape, dtype=torch.uint8)
            _fill_mxfp4(key_storage, full, rng)
            k_mx = (full[:: gap + 1] if gap else full).contiguous()
        else:
            _fill_values(key_storage, rng)
        key = key_storage[:: gap + 1] if gap else key_storage

    # 5. scale (int8 keys)
    scale = None
    if kdtype == "i8":
        if layout == "TND":
            scale = torch.empty((int(kv.sum()), Hkv), dtype=torch.float32)
        else:
            scale = torch.empty((NP, Hkv, P), dtype=torch.float32)
        _fill_scale(scale, rng)

    if start_loc is None:
        sl = np.maximum(kv - ql, 0) // P
    else:
        sl = np.asarray(start_loc, dtype=np.int64)
    return MsaCase(
        name=name, query=query, key=key, key_storage=key_storage, layout=layout,
        block_table=block_table, scale=scale,
        cu_seqlens_q=torch.from_numpy(cu.astype(np.int32)),
        kv_len=torch.from_numpy(kv.astype(np.int32)),
        start_loc=torch.from_numpy(sl.astype(np.int32)),
        max_blocks=int(MB), sparse_mode=sparse_mode, init_blocks=init_blocks,
        local_blocks=local_blocks, block_size=P, gap=gap, local_mode=local_mode,
        q_mx_scale=q_mx, k_mx_scale=k_mx)


def config_case(c: int) -> MsaCase:
    """The c-th measured workload (0-based, same order as ``CONFIG_NAMES``)."""
    name = CONFIG_NAMES[c]
    seed = 20261200 + c + 1
    if c == 0:
        return make_case(name, seed, q_lens=[32], kv_lens=[256], Hq=8, Hkv=1, qdtype="f16",
                         layout="BBND", MB=2, NP=8, table="arange", sparse_mode=3,
                         init_blocks=0, local_blocks=1, start_loc=[1])
    if c == 1:
        return make_case(name, seed, q_lens=[1], kv_lens=None, kv_len_draw=(1, 32768), B=64,
                         Hq=16, Hkv=1, qdtype="bf16", layout="BBND", MB=256, NP=16384,
                         table="perm", sparse_mode=3, init_blocks=0, local_blocks=1)
    if c == 2:
        q_lens = [1024, 2048, 4096, 8192]
        prefix = [0, 4096, 16384, 57344]
        kv = [p + q for p, q in zip(prefix, q_lens)]
        return make_case(name, seed, q_lens=q_lens, kv_lens=kv, Hq=32, Hkv=4, qdtype="bf16",
                         layout="TND", sparse_mode=3, init_blocks=1, local_blocks=2)
    if c == 3:
        return make_case(name, seed, q_lens=[1], kv_lens=None, kv_len_draw=(65536, 131072), B=32,
                         Hq=16, Hkv=1, qdtype="f16", kdtype="i8", layout="BNBD", MB=1024,
                         NP=32768, table="perm", sparse_mode=3, init_blocks=0, local_blocks=1)
    if c == 4:
        return make_case(name, seed, q_lens=[4096], kv_lens=[131072], Hq=64, Hkv=8,
                         qdtype="f8e4m3", layout="BBND", MB=1024, NP=1024, table="perm",
                         sparse_mode=3, init_blocks=1, local_blocks=4)
    raise IndexError(c)


def e5m2_config_case() -> MsaCase:
    """The chunked fp8 prefill workload with e5m2 query and key instead of
    e4m3: 4096 tokens after a 126976-token prefix, Hq = 64 over Hkv = 8,
    1024 paged blocks (drawn from its own seed)."""
    return make_case("prefill_bbnd_f8e5m2", 20261206, q_lens=[4096], kv_lens=[131072], Hq=64,
                     Hkv=8, qdtype="f8e5m2", layout="BBND", MB=1024, NP=1024, table="perm",
                     sparse_mode=3, init_blocks=1, local_blocks=4)


def i8_prefill_config_case() -> MsaCase:
    """The varlen prefill workload with an fp16 query and int8 packed keys
    with their per-token scales: requests of 1K, 2K, 4K and 8K tokens after
    prefixes of 0, 4K, 16K and 56K keys, Hq = 32 over Hkv = 4."""
    q_lens = [1024, 2048, 4096, 8192]
    prefix = [0, 4096, 16384, 57344]
    kv = [p + q for p, q in zip(prefix, q_lens)]
    return make_case("prefill_tnd_i8", 20261207, q_lens=q_lens, kv_lens=kv, Hq=32, Hkv=4,
                     qdtype="f16", kdtype="i8", layout="TND", sparse_mode=3, init_blocks=1,
                     local_blocks=2)


# The MXFP4 variants of three workloads: the same shapes, lengths and tables,
# with MXFP4 query and key (N(0,1) encoded per 32-element group).
MX_CONFIG_NAMES = ("decode_bbnd_mxfp4", "prefill_tnd_mxfp4", "prefill_bbnd_mxfp4")
_MX_OF = {"decode_bbnd_mxfp4": 1, "prefill_tnd_mxfp4": 2, "prefill_bbnd_mxfp4": 4}


def mx_config_case(name: str) -> MsaCase:
    c = _MX_OF[name]
    seed = 20261300 + c + 1
    if c == 1:
        return make_case(name, seed, q_lens=[1], kv_lens=None, kv_len_draw=(1, 32768), B=64,
                         Hq=16, Hkv=1, qdtype="mxfp4", layout="BBND", MB=256, NP=16384,
                         table="perm", sparse_mode=3, init_blocks=0, local_blocks=1)
    if c == 2:
        q_lens = [1024, 2048, 4096, 8192]
        prefix = [0, 4096, 16384, 57344]
        kv = [p + q for p, q in zip(prefix, q_lens)]
        return make_case(name, seed, q_lens=q_lens, kv_lens=kv, Hq=32, Hkv=4, qdtype="mxfp4",
                         layout="TND", sparse_mode=3, init_blocks=1, local_blocks=2)
    return make_case(name, seed, q_lens=[4096], kv_lens=[131072], Hq=64, Hkv=8,
                     qdtype="mxfp4", layout="BBND", MB=1024, NP=1024, table="perm",
                     sparse_mode=3, init_blocks=1, local_blocks=4)


# ---------------------------------------------------------------------------
# poisoning of bytes the operator must never let into a result
# ---------------------------------------------------------------------------

_POISON = {
    # pattern -> value per storage dtype
    # (MXFP4 values have no NaN: 0x77 is 6.0 twice, 0xFF is -6.0 twice; its
    # E8M0 scales poison as 2^-127, 2^127 and the NaN code 255)
    "zero": {"f16": 0.0, "bf16": 0.0, "f8e4m3": 0.0, "f8e5m2": 0.0, "i8": 0, "scale": 0.0,
             "mxfp4": 0, "mx_scale": 0},
    "big": {"f16": 65504.0, "bf16": 3.0e38, "f8e4m3": 448.0, "f8e5m2": 57344.0, "i8": 127,
            "scale": 3.0e38, "mxfp4": 0x77, "mx_scale": 254},
    "nan": {"f16": float("nan"), "bf16": float("nan"), "f8e4m3": float("nan"),
            "f8e5m2": float("nan"), "i8": -128, "scale": float("nan"), "mxfp4": 0xFF,
            "mx_scale": 255},
}


def poison_case(case: MsaCase, pattern: str) -> MsaCase:
    """Copy of a paged case with every byte the operator may not read as data
    set to ``pattern`` ("zero", "big" or "nan"):

    * pages no request references below its block count (incl. dim0 gaps),
    * rows at or past ``kv_len`` inside each request's last page,
    * the matching int8 scale entries,
    * block-table entries at or past a request's block count are redirected to
      such unused pages (kept inside the page range).
    """
    if case.layout == "TND":
        return dataclasses.replace(case, poison=pattern)
    P = case.block_size
    ks = case.key_storage.clone()
    gap = case.gap
    key = ks[:: gap + 1] if gap else ks
    bt = case.block_table.clone()
    scale = case.scale.clone() if case.scale is not None else None
    mxs = case.k_mx_scale.clone() if case.k_mx_scale is not None else None
    mxv = _POISON[pattern]["mx_scale"]
    kname = case.key_dtype_name()
    kval = _POISON[pattern][kname]
    NP = int(key.shape[0])
    used = np.zeros(NP, dtype=bool)
    kv = case.kv_len.numpy()
    for b in range(case.batch):
        nb = _ceil_div(int(kv[b]), P)
        used[bt[b, :nb].numpy()] = True
    unused = np.nonzero(~used)[0]
    # every storage page not used as data
    if gap:
        ks_used = np.zeros(ks.shape[0], dtype=bool)
        ks_used[np.nonzero(used)[0] * (gap + 1)] = True
        ks[torch.from_numpy(~ks_used)] = kval
    elif unused.size:
        ks[torch.from_numpy(unused)] = kval
    if scale is not None and unused.size:
        scale[torch.from_numpy(unused)] = _POISON[pattern]["scale"]
    if mxs is not None and unused.size:
        mxs[torch.from_numpy(unused)] = mxv
    k = 0
    for b in range(case.batch):
        L = int(kv[b])
        nb = _ceil_div(L, P)
        if nb > 0 and L % P:
            page = int(bt[b, nb - 1])
            tail = L - (nb - 1) * P
            if case.layout == "BBND":
                key[page, tail:] = kval
            else:
                key[page, :, tail:] = kval
            if scale is not None:
                scale[page, :, tail:] = _POISON[pattern]["scale"]
            if mxs is not None:
                if case.layout == "BBND":
                    mxs[page, tail:] = mxv
                else:
                    mxs[page, :, tail:] = mxv
        if unused.size:
            for beta in range(nb, bt.shape[1]):
                bt[b, beta] = int(unused[k % unused.size])
                k += 1
    return dataclasses.replace(case, key=key, key_storage=ks, block_table=bt, scale=scale,
                               k_mx_scale=mxs,
                               poison=pattern)


# ---------------------------------------------------------------------------
# the small edge-case suite (categories of the operator's published test matrix)
# ---------------------------------------------------------------------------

def edge_cases() -> List[MsaCase]:
    """Small cases spanning several tiles and ragged tails; each builds in well
    under a second on one CPU core."""
    cs: List[MsaCase] = []
    s = 7000

    def add(name, **kw):
        nonlocal s
        s += 1
        cs.append(make_case(name, s, **kw))

    cs.append(config_case(0))
    # dtype x layout matrix, mixed lengths with ragged tails
    for qd, kd in (("f16", "f16"), ("bf16", "bf16"), ("f16", "i8"), ("f8e4m3", "f8e4m3")):
        for lay in ("BBND", "BNBD", "TND"):
            add(f"mix_{lay.lower()}_{kd}", q_lens=[3, 1, 37], kv_lens=[300, 129, 600], Hq=8,
                Hkv=2, qdtype=qd, kdtype=kd, layout=lay, extra_pages=4,
                init_blocks=1, local_blocks=2)
    # mixed batch padding: q_len=0 and kv_len=0 requests
    add("pad_qlen0_kvlen0", q_lens=[2, 0, 5, 3], kv_lens=[200, 50, 0, 130], Hq=4, Hkv=1,
        qdtype="bf16", layout="BBND", extra_pages=12)
    add("pad_tnd_kvlen0", q_lens=[4, 2], kv_lens=[0, 260], Hq=4, Hkv=2, qdtype="f16",
        layout="TND", init_blocks=1, local_blocks=1)
    # a whole batch with no query tokens
    add("empty_batch", q_lens=[0, 0], kv_lens=[128, 0], Hq=4, Hkv=1, qdtype="bf16",
        layout="BBND", extra_pages=4)
    # every request with kv_len = 0 (MB clamps to 1)
    add("all_kv_empty_tnd", q_lens=[3, 2], kv_lens=[0, 0], Hq=4, Hkv=1, qdtype="bf16",
        layout="TND")
    # paged key with gaps between pages in dim0
    add("dim0_gap2_bbnd", q_lens=[2, 3], kv_lens=[333, 140], Hq=8, Hkv=1, qdtype="bf16",
        layout="BBND", extra_pages=10, gap=2)
    add("dim0_gap2_bnbd_i8", q_lens=[1, 4], kv_lens=[257, 513], Hq=8, Hkv=2, qdtype="f16",
        kdtype="i8", layout="BNBD", extra_pages=12, gap=2)
    # wide block tables (257 / 275 columns -> out width 272 / 288)
    add("wide_table_257", q_lens=[1, 2], kv_lens=[1000, 77], Hq=4, Hkv=1, qdtype="bf16",
        layout="BBND", MB=257, extra_pages=600)
    add("decode_q4_kv4_table275", q_lens=[4], kv_lens=[4], Hq=8, Hkv=1, qdtype="f16",
        layout="BBND", MB=275, extra_pages=300)
    add("decode_q4_kv275", q_lens=[4], kv_lens=[275], Hq=8, Hkv=1, qdtype="f16",
        layout="BBND", extra_pages=8)
    # speculative decode (q_len > 1)
    add("spec_decode_q3", q_lens=[3, 3, 3], kv_lens=[500, 1024, 3], Hq=16, Hkv=1,
        qdtype="bf16", layout="BBND", extra_pages=20)
    # long kv spanning many blocks
    add("kv4096_bnbd", q_lens=[2], kv_lens=[4096], Hq=8, Hkv=1, qdtype="bf16",
        layout="BNBD", extra_pages=40)
    # tiny kv tails
    add("tiny_kv_tail", q_lens=[1, 1, 2], kv_lens=[1, 129, 2], Hq=8, Hkv=1, qdtype="f16",
        layout="BBND", extra_pages=6)
    # more query tokens than kv tokens (rows that see nothing)
    add("q_longer_than_kv", q_lens=[10, 4], kv_lens=[6, 130], Hq=4, Hkv=1, qdtype="bf16",
        layout="BBND", extra_pages=4, init_blocks=1, local_blocks=1)
    # no causal mask
    add("mode0_bbnd", q_lens=[5, 1], kv_lens=[300, 200], Hq=8, Hkv=1, qdtype="bf16",
        layout="BBND", extra_pages=8, sparse_mode=0)
    add("mode0_tnd", q_lens=[40], kv_lens=[700], Hq=4, Hkv=4, qdtype="f16", layout="TND",
        sparse_mode=0, init_blocks=2, local_blocks=3)
    # local_mask variants
    add("no_local_mask", q_lens=[3], kv_lens=[400], Hq=4, Hkv=1, qdtype="bf16",
        layout="BBND", extra_pages=4, init_blocks=0, local_blocks=0)
    add("init_only", q_lens=[3], kv_lens=[400], Hq=4, Hkv=1, qdtype="bf16", layout="BBND",
        extra_pages=4, init_blocks=3, local_blocks=0)
    add("local_window_clipped", q_lens=[2], kv_lens=[300], Hq=4, Hkv=1, qdtype="bf16",
        layout="BBND", extra_pages=4, init_blocks=1, local_blocks=3, start_loc=[1])
    add("init_local_overlap", q_lens=[2], kv_lens=[300], Hq=4, Hkv=1, qdtype="bf16",
        layout="BBND", extra_pages=4, init_blocks=2, local_blocks=2, start_loc=[1])
    # GQA group sizes: 1, odd, and larger than one MFMA tile of rows
    add("gqa_g1_tnd", q_lens=[20], kv_lens=[150], Hq=3, Hkv=3, qdtype="bf16", layout="TND")
    add("gqa_g3_bbnd", q_lens=[7, 2], kv_lens=[260, 90], Hq=6, Hkv=2, qdtype="f16",
        layout="BBND", extra_pages=6)
    add("gqa_g40_bbnd", q_lens=[2], kv_lens=[200], Hq=40, Hkv=1, qdtype="bf16",
        layout="BBND", extra_pages=2)
    # prefill-shaped: many tokens per request (several row tiles, causal diagonal)
    add("prefill_tnd_small", q_lens=[300, 77], kv_lens=[556, 77], Hq=16, Hkv=2,
        qdtype="bf16", layout="TND", init_blocks=1, local_blocks=2)
    add("prefill_bbnd_f8", q_lens=[200], kv_lens=[450], Hq=16, Hkv=2, qdtype="f8e4m3",
        layout="BBND", extra_pages=6, init_blocks=1, local_blocks=2)
    add("prefill_bnbd_i8", q_lens=[150], kv_lens=[400], Hq=8, Hkv=1, qdtype="f16",
        kdtype="i8", layout="BNBD", extra_pages=5, init_blocks=0, local_blocks=1)
    add("prefill_bbnd_f16_g16", q_lens=[64, 40], kv_lens=[64, 300], Hq=16, Hkv=1,
        qdtype="f16", layout="BBND", extra_pages=6)
    # fp8 e5m2 (same kernels, the other OCP operand format)
    add("mix_bbnd_f8e5m2", q_lens=[3, 1, 37], kv_lens=[300, 129, 600], Hq=8, Hkv=2,
        qdtype="f8e5m2", layout="BBND", extra_pages=4, init_blocks=1, local_blocks=2)
    add("prefill_tnd_f8e5m2", q_lens=[130], kv_lens=[400], Hq=16, Hkv=2, qdtype="f8e5m2",
        layout="TND", init_blocks=1, local_blocks=1)
    # per-query local window (each token's own block and the ones before it)
    add("perq_prefill_tnd", q_lens=[300, 77], kv_lens=[556, 77], Hq=16, Hkv=2,
        qdtype="bf16", layout="TND", init_blocks=1, local_blocks=2, local_mode=1)
    add("perq_mode0_bbnd", q_lens=[200, 3], kv_lens=[700, 260], Hq=8, Hkv=1, qdtype="f16",
        layout="BBND", extra_pages=6, sparse_mode=0, local_blocks=3, local_mode=1)
    add("perq_q_longer_than_kv", q_lens=[10, 4], kv_lens=[6, 130], Hq=4, Hkv=1,
        qdtype="bf16", layout="BBND", extra_pages=4, init_blocks=1, local_blocks=1,
        local_mode=1)
    add("perq_spec_decode_i8", q_lens=[3, 1, 2], kv_lens=[500, 129, 0], Hq=8, Hkv=2,
        qdtype="f16", kdtype="i8", layout="BNBD", extra_pages=5, local_blocks=2,
        local_mode=1)
    add("perq_prefill_bbnd_f8", q_lens=[200], kv_lens=[450], Hq=16, Hkv=2, qdtype="f8e4m3",
        layout="BBND", extra_pages=6, init_blocks=1, local_blocks=2, local_mode=1)
    add("perq_prefill_bnbd_wide", q_lens=[260], kv_lens=[1000], Hq=8, Hkv=1, qdtype="bf16",
        layout="BNBD", MB=40, extra_pages=4, init_blocks=2, local_blocks=4, local_mode=1)
    # MXFP4 query and key (E2M1 values, E8M0 scale per 32 elements)
    add("mx_mix_bbnd", q_lens=[3, 1, 37], kv_lens=[300, 129, 600], Hq=8, Hkv=2,
        qdtype="mxfp4", layout="BBND", extra_pages=4, init_blocks=1, local_blocks=2)
    add("mx_mix_bnbd_gap", q_lens=[3, 1, 37], kv_lens=[300, 129, 600], Hq=8, Hkv=2,
        qdtype="mxfp4", layout="BNBD", extra_pages=4, gap=1, init_blocks=1, local_blocks=2)
    add("mx_prefill_tnd", q_lens=[300, 77], kv_lens=[556, 77], Hq=16, Hkv=2, qdtype="mxfp4",
        layout="TND", init_blocks=1, local_blocks=2)
    add("mx_q_longer_than_kv", q_lens=[10, 4], kv_lens=[6, 130], Hq=4, Hkv=1, qdtype="mxfp4",
        layout="BBND", extra_pages=4, init_blocks=1, local_blocks=1)
    add("mx_perq_prefill_bbnd", q_lens=[200], kv_lens=[450], Hq=16, Hkv=2, qdtype="mxfp4",
        layout="BBND", extra_pages=6, init_blocks=1, local_blocks=2, local_mode=1)
    add("mx_decode_g16", q_lens=[1] * 5, kv_lens=[1, 127, 128, 129, 700], Hq=16, Hkv=1,
        qdtype="mxfp4", layout="BBND", extra_pages=3)
    return cs


def large_batch_cases() -> List[MsaCase]:
    """Batches of more than 64 requests (several 64-request chunks, the last
    one past a 256-chunk table), with short lengths so the oracle stays quick:
    one-token decode, speculative and empty requests, paged and packed keys;
    and a 64-request batch whose workgroup slices run past one page window."""
    rng = np.random.default_rng(777)
    out = []

    def lens(B, lo, hi):
        return [int(x) for x in rng.integers(lo, hi + 1, size=B)]

    out.append(make_case("batch65_bbnd_bf16", 7001, q_lens=[1] * 65, kv_lens=lens(65, 0, 700),
                         Hq=8, Hkv=1, qdtype="bf16", layout="BBND", sparse_mode=3,
                         init_blocks=1, local_blocks=1))
    out.append(make_case("batch300_bnbd_i8_spec", 7002,
                         q_lens=[int(x) for x in rng.choice([0, 1, 2, 3], size=300)],
                         kv_lens=lens(300, 0, 1000), Hq=16, Hkv=2, qdtype="f16", kdtype="i8",
                         layout="BNBD", sparse_mode=3, init_blocks=0, local_blocks=2))
    out.append(make_case("batch1000_tnd_f16", 7003, q_lens=[1] * 1000, kv_lens=lens(1000, 0, 400),
                         Hq=4, Hkv=1, qdtype="f16", layout="TND", sparse_mode=3,
                         init_blocks=1, local_blocks=1))
    out.append(make_case("batch200_bbnd_f16_perq", 7005,
                         q_lens=[int(x) for x in rng.choice([1, 2, 5], size=200)],
                         kv_lens=lens(200, 0, 900), Hq=8, Hkv=2, qdtype="f16", layout="BBND",
                         sparse_mode=3, init_blocks=1, local_blocks=2, local_mode=1))
    out.append(make_case("batch16500_tnd_bf16", 7004,
                         q_lens=[int(x) for x in rng.choice([0, 1, 1, 1], size=16500)],
                         kv_lens=lens(16500, 0, 200), Hq=2, Hkv=1, qdtype="bf16", layout="TND",
                         sparse_mode=3, init_blocks=0, local_blocks=1))
    # 64 requests (the at-most-64 kernel instance) with 128 heads per KV head:
    # 16 units of eight head chunks share the chip, so each workgroup's slice
    # holds ~90 (tile, block) entries over about three requests per 64 entries
    # (its waves load the page window again past entry 64), and two-token
    # requests have two tiles.
    out.append(make_case("batch64_bbnd_bf16_g128", 7006,
                         q_lens=[int(x) for x in rng.choice([1, 1, 2], size=64)],
                         kv_lens=lens(64, 0, 6000), Hq=256, Hkv=2, qdtype="bf16", layout="BBND",
                         sparse_mode=3, init_blocks=1, local_blocks=2))
    return out


def random_cases(n: int, seed: int = 4242) -> List[MsaCase]:
    """n small cases with every knob drawn at random (lengths, heads, key type,
    layout, mode, local_mask counts, table width, dim0 gap), for sweeps."""
    rng = np.random.default_rng(seed)
    pairs = [("f16", "f16"), ("bf16", "bf16"), ("f16", "i8"), ("f8e4m3", "f8e4m3"),
             ("f8e5m2", "f8e5m2")]
    out = []
    for i in range(n):
        B = int(rng.integers(1, 6))
        q_lens = [int(x) for x in rng.choice([0, 1, 2, 3, 5, 17, 40, 90], size=B)]
        kv_lens = [int(x) for x in rng.choice([0, 1, 100, 127, 128, 129, 300, 511, 700],
                                               size=B)]
        Hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 8, 16, 20]))
        qd, kd = pairs[int(rng.integers(len(pairs)))]
        layout = str(rng.choice(["BBND", "BNBD", "TND"]))
        mode = int(rng.choice([0, 3]))
        nb = max(1, max(-(-k // 128) for k in kv_lens))
        MB = None if layout == "TND" else nb + int(rng.integers(0, 20))
        limit = (MB if MB is not None else ((nb + 15) // 16) * 16)
        init = int(rng.integers(0, min(3, limit) + 1))
        local = int(rng.integers(0, min(3, limit) + 1))
        starts = [int(rng.integers(0, MB if MB is not None else nb)) for _ in range(B)]
        gap = int(rng.choice([0, 0, 1])) if layout != "TND" else 0
        # drawn from a generator of its own, so the other draws stay as they were
        local_mode = int(np.random.default_rng(seed + 100000 + i).integers(0, 2))
        out.append(make_case(f"rand{i}_{layout.lower()}_{kd}_g{g}", seed + 1 + i,
                             q_lens=q_lens, kv_lens=kv_lens, Hq=Hkv * g, Hkv=Hkv, qdtype=qd,
                             kdtype=kd, layout=layout, MB=MB, extra_pages=int(rng.integers(0, 4)),
                             gap=gap, sparse_mode=mode, init_blocks=init, local_blocks=local,
                             start_loc=starts, local_mode=local_mode))
    return out


def mx_random_cases(n: int, seed: int = 9090) -> List[MsaCase]:
    """n small MXFP4 cases with the knobs drawn at random as in random_cases
    (lengths, heads, layout, mode, local_mask counts and window, table width,
    dim0 gap); query and key are both MXFP4."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 6))
        q_lens = [int(x) for x in rng.choice([0, 1, 2, 3, 5, 17, 40, 90], size=B)]
        kv_lens = [int(x) for x in rng.choice([0, 1, 100, 127, 128, 129, 300, 511, 700],
                                               size=B)]
        Hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 8, 16, 20]))
        layout = str(rng.choice(["BBND", "BNBD", "TND"]))
        mode = int(rng.choice([0, 3]))
        nb = max(1, max(-(-k // 128) for k in kv_lens))
        MB = None if layout == "TND" else nb + int(rng.integers(0, 20))
        limit = (MB if MB is not None else ((nb + 15) // 16) * 16)
        init = int(rng.integers(0, min(3, limit) + 1))
        local = int(rng.integers(0, min(3, limit) + 1))
        starts = [int(rng.integers(0, MB if MB is not None else nb)) for _ in range(B)]
        gap = int(rng.choice([0, 0, 1])) if layout != "TND" else 0
        local_mode = int(rng.integers(0, 2))
        out.append(make_case(f"mxrand{i}_{layout.lower()}_g{g}", seed + 1 + i,
                             q_lens=q_lens, kv_lens=kv_lens, Hq=Hkv * g, Hkv=Hkv,
                             qdtype="mxfp4", layout=layout, MB=MB,
                             extra_pages=int(rng.integers(0, 4)), gap=gap, sparse_mode=mode,
                             init_blocks=init, local_blocks=local, start_loc=starts,
                             local_mode=local_mode))
    return out


def case_summary(case: MsaCase) -> dict:
    return {
        "name": case.name, "layout": case.layout, "q": case.query_dtype_name(),
        "k": case.key_dtype_name(), "B": case.batch, "T": case.T, "Hq": case.Hq,
        "Hkv": case.Hkv, "MB": case.max_blocks, "mode": case.sparse_mode,
        "init": case.init_blocks, "local": case.local_blocks, "poison": case.poison,
        "local_mode": case.local_mode,
    }


def score_rows(seed: int, Hq: int, T: int, W: int, ties: bool = True) -> torch.Tensor:
    """Seeded float32 score rows [Hq, T, W] for the top-k selection: values
    from a small pool (many exact ties, including the local_mask constants
    1e30 and 1e29) with some normal noise, or all normal with ties=False;
    about 20% -inf and 1% NaN entries."""
    rng = np.random.default_rng(seed)
    if ties:
        pool = np.array([-3.5, -1.0, 0.0, 0.25, 2.0, 2.0, 7.75, 1e29, 1e30], dtype=np.float32)
        s = rng.choice(pool, size=(Hq, T, W)).astype(np.float32)
        s += (rng.choice([0, 0, 0, 1], size=s.shape).astype(np.float32) *
              rng.standard_normal(s.shape).astype(np.float32))
    else:
        s = rng.standard_normal((Hq, T, W)).astype(np.float32)
    s[rng.random(s.shape) < 0.2] = -np.inf
    s[rng.random(s.shape) < 0.01] = np.nan
    return torch.from_numpy(s)
