"""The C ABI on the CPU: the library loads, exports every declared function, and
rejects each malformed call with its status before touching the GPU.

No call here reaches a kernel launch: every one fails validation or has T = 0
(which returns without launching).
"""
import ctypes
import json
import os
import re

import pytest
import torch

import block_max_qk_amd as m
from block_max_qk_amd._binding import MsaTensor, describe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa_index_score.h")

OK, NULL, LAYOUT, DTYPE, SHAPE, STRIDE, SCALE, ATTR = range(8)
DT = {"f16": 0, "bf16": 1, "i8": 2, "e4m3": 3, "e5m2": 4}


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(m.LIB_PATH)
    names = declared_functions()
    assert set(names) == set(m.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_out_width_matches_golden():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "out_width.json")))
    for mb, w in g["max_blocks_to_width"]:
        assert m.msa_index_score_out_width(mb) == w


def test_status_strings():
    for s in range(9):
        assert m.msa_status_str(s)
    assert m.msa_status_str(99) == "unknown status"


def test_kernel_family_choice():
    assert m.msa_index_score_kernel_family(64, 64, 16, 1) == 0        # decode batch
    assert m.msa_index_score_kernel_family(32, 32, 16, 1) == 0        # int8 decode batch
    assert m.msa_index_score_kernel_family(15360, 4, 32, 4) == 1      # varlen prefill
    assert m.msa_index_score_kernel_family(4096, 1, 64, 8) == 1       # chunked prefill
    # one short request: 32 or 64 tokens x 8 heads spread further as 16-row
    # decode tiles than as one prefill tile; from 1024 query rows on, prefill
    assert m.msa_index_score_kernel_family(32, 1, 8, 1) == 0          # the guide's tiny example
    assert m.msa_index_score_kernel_family(64, 1, 8, 1) == 0
    assert m.msa_index_score_kernel_family(128, 1, 8, 1) == 1
    assert m.msa_index_score_kernel_family(64, 1, 16, 1) == 1
    assert m.msa_index_score_kernel_family(1024, 8, 8, 1) == 1
    assert m.msa_index_score_kernel_family(1024, 128, 8, 1) == 0      # 8 tokens per request


# ---------------------------------------------------------------------------
# validation: fake device addresses, never dereferenced
# ---------------------------------------------------------------------------

FAKE = 0x7F0000000000


def tdesc(shape, stride=None, dtype=0, addr=FAKE):
    d = MsaTensor()
    d.data = addr
    d.dtype = dtype
    d.ndim = len(shape)
    if stride is None:
        stride, acc = [], 1
        for s in reversed(shape):
            stride.insert(0, acc)
            acc *= s
    for i, (a, b) in enumerate(zip(shape, stride)):
        d.shape[i] = a
        d.stride[i] = b
    return d


def call(q=None, k=None, *, start=FAKE, table=FAKE, mb=2, scale=None, cu=FAKE, kv=FAKE, B=1,
         bs=128, layout=1, mode=3, init=0, local=1, out=FAKE, width=16, family=None,
         local_mode=None):
    lib = m.load_library()
    q = q if q is not None else tdesc([32, 8, 128], dtype=DT["f16"])
    k = k if k is not None else tdesc([8, 128, 1, 128], dtype=DT["f16"])
    args = [ctypes.byref(q) if q is not False else None,
            ctypes.byref(k) if k is not False else None,
            start, table, mb, scale, cu, kv, B, bs, layout, mode, init, local, out, width, None]
    if local_mode is not None:
        return lib.msa_index_score_ex(*args[:14], local_mode, *args[14:],
                                      -1 if family is None else family)
    if family is None:
        return lib.msa_index_score(*args)
    return lib.msa_index_score_family(*args, family)


def test_valid_empty_call_returns_ok_without_launch():
    q = tdesc([0, 8, 128], dtype=DT["f16"])
    assert call(q=q, B=1) == OK
    assert call(q=q, B=1, out=None) == OK                      # T = 0: out never written
    assert call(q=q, B=0, kv=None, start=None, table=None) == OK   # no requests
    assert call(q=q, B=1, kv=None) == NULL


def test_null_pointers():
    assert call(q=False) == NULL
    assert call(k=False) == NULL
    assert call(out=None) == NULL
    assert call(cu=None) == NULL
    assert call(kv=None) == NULL
    assert call(start=None) == NULL
    assert call(table=None) == NULL              # paged layouts need a block table


@pytest.mark.parametrize("layout", [-1, 3, 7])
def test_bad_layout(layout):
    assert call(layout=layout) == LAYOUT


def test_python_layout_key_is_case_insensitive_and_checked():
    with pytest.raises(ValueError):
        m.index_score(torch.zeros(1, 8, 128, dtype=torch.float16),
                      torch.zeros(2, 128, 1, 128, dtype=torch.float16),
                      torch.zeros(1, dtype=torch.int32), layout_key="bhsd",
                      block_table=torch.zeros(1, 2, dtype=torch.int32),
                      actual_seq_qlen=torch.tensor([0, 1], dtype=torch.int32),
                      actual_seq_klen=torch.tensor([1], dtype=torch.int32))


@pytest.mark.parametrize("qd,kd,with_scale,want", [
    ("bf16", "f16", False, DTYPE),      # mixed 16-bit types
    ("f16", "bf16", False, DTYPE),
    ("bf16", "i8", True, DTYPE),        # int8 keys need an fp16 query
    ("e4m3", "e5m2", False, DTYPE),     # FP8 query and key of one format
    ("e4m3", "f16", False, DTYPE),
    ("f16", "i8", False, SCALE),        # int8 without scale
    ("f16", "f16", True, SCALE),        # scale with a non-int8 key
    ("e4m3", "e4m3", True, SCALE),
])
def test_dtype_and_scale_rules(qd, kd, with_scale, want):
    q = tdesc([4, 8, 128], dtype=DT[qd])
    k = tdesc([8, 128, 1, 128], dtype=DT[kd])
    assert call(q=q, k=k, scale=FAKE if with_scale else None) == want


def test_unknown_dtype_code():
    assert call(q=tdesc([4, 8, 128], dtype=9)) == DTYPE


def test_shape_rules():
    assert call(q=tdesc([4, 8, 64], dtype=0)) == SHAPE                           # D != 128
    assert call(k=tdesc([8, 64, 1, 128], dtype=0)) == SHAPE                      # P != 128
    assert call(k=tdesc([8, 128, 3, 128], dtype=0)) == SHAPE                     # Hq % Hkv
    assert call(k=tdesc([8, 1, 128, 128], dtype=0), layout=1) == SHAPE           # BNBD shape as BBND
    assert call(k=tdesc([128, 1, 128], dtype=0), layout=1) == SHAPE              # 3-D TND shape as BBND
    assert call(width=32) == SHAPE                                               # out width
    assert call(mb=0) == SHAPE                                                   # paged MB >= 1
    assert call(B=0) == SHAPE                                                    # T > 0, no requests
    assert call(layout=0, k=tdesc([300, 1, 128], dtype=0), table=FAKE) == SHAPE  # TND takes no table


def test_three_dim_bbnd_and_tnd_accepted_shapes_with_t0():
    q0 = tdesc([0, 8, 128], dtype=0)
    assert call(q=q0, k=tdesc([8, 128, 128], dtype=0), layout=1) == OK
    assert call(q=q0, k=tdesc([300, 1, 128], dtype=0), layout=0, table=None, mb=3) == OK
    assert call(q=q0, k=tdesc([0, 1, 128], dtype=0), layout=0, table=None, mb=0) == OK


def test_stride_rules():
    # dim0 gap is allowed for paged keys
    gap = tdesc([8, 128, 1, 128], [3 * 128 * 128, 128, 128, 1], dtype=0)
    assert call(q=tdesc([0, 8, 128], dtype=0), k=gap) == OK
    # inner axes must be compact
    bad = tdesc([8, 128, 2, 128], [128 * 2 * 128, 2 * 128, 256, 1], dtype=0)
    assert call(k=bad, q=tdesc([4, 8, 128], dtype=0)) == STRIDE
    bad_d = tdesc([8, 128, 1, 128], [128 * 128 * 2, 256, 128, 2], dtype=0)
    assert call(k=bad_d) == STRIDE
    # an extent-1 head axis is not addressed: any stride is fine
    odd = tdesc([8, 128, 1, 128], [128 * 128, 128, 7, 1], dtype=0)
    assert call(q=tdesc([0, 8, 128], dtype=0), k=odd) == OK
    # TND keys must be fully compact
    tnd = tdesc([300, 2, 128], [512, 128, 1], dtype=0)
    assert call(q=tdesc([4, 8, 128], dtype=0), k=tnd, layout=0, table=None, mb=3) == STRIDE
    # query must be compact
    assert call(q=tdesc([4, 8, 128], [2048, 128, 1], dtype=0)) == STRIDE
    # misaligned pointers / page strides
    assert call(q=tdesc([4, 8, 128], dtype=0, addr=FAKE + 2)) == STRIDE
    mis = tdesc([8, 128, 1, 128], [128 * 128 + 1, 128, 128, 1], dtype=0)
    assert call(k=mis) == STRIDE
    assert call(out=FAKE + 4) == STRIDE


def test_attribute_rules():
    assert call(mode=1) == ATTR
    assert call(mode=2) == ATTR
    assert call(init=-1) == ATTR
    assert call(local=-1) == ATTR
    assert call(init=3, mb=2) == ATTR                 # paged limit: MB
    assert call(local=3, mb=2) == ATTR
    q0 = tdesc([0, 8, 128], dtype=0)
    assert call(q=q0, init=2, local=2, mb=2) == OK
    # packed keys: limit is the aligned output width
    tnd = tdesc([300, 1, 128], dtype=0)
    assert call(q=q0, k=tnd, layout=0, table=None, mb=3, init=16, local=16) == OK
    assert call(q=q0, k=tnd, layout=0, table=None, mb=3, init=17) == ATTR
    assert call(family=2) == ATTR
    assert call(family=-2) == ATTR


def test_local_mode_rules():
    q0 = tdesc([0, 8, 128], dtype=0)
    assert call(local_mode=2) == ATTR
    assert call(local_mode=-1) == ATTR
    assert call(q=q0, local_mode=0) == OK
    assert call(q=q0, local_mode=1) == OK
    # start_loc is needed for the per-request window only
    assert call(start=None, local_mode=0) == NULL
    assert call(q=q0, start=None, local_mode=1) == OK
    assert call(start=None, local_mode=1, family=5) == ATTR   # validation goes on past it
    # the other checks are the same as msa_index_score's
    assert call(mode=1, local_mode=1) == ATTR
    assert call(width=32, local_mode=1) == SHAPE
    assert call(cu=None, local_mode=1) == NULL


def mx_call(q=None, k=None, *, qs=FAKE, ks=FAKE, start=FAKE, table=FAKE, mb=2, cu=FAKE,
            kv=FAKE, B=1, bs=128, layout=1, mode=3, init=0, local=1, local_mode=0, out=FAKE,
            width=16, family=None):
    lib = m.load_library()
    q = q if q is not None else tdesc([32, 8, 64], dtype=5)
    k = k if k is not None else tdesc([8, 128, 1, 64], dtype=5)
    args = (ctypes.byref(q), qs, ctypes.byref(k), ks, start, table, mb, cu, kv, B, bs, layout,
            mode, init, local, local_mode, out, width, None)
    if family is None:
        return lib.msa_index_score_mxfp4(*args)
    return lib.msa_index_score_mxfp4_family(*args, family)


def test_mxfp4_rules():
    q0 = tdesc([0, 8, 64], dtype=5)
    assert mx_call(q=q0) == OK
    assert mx_call(q=q0, k=tdesc([300, 1, 64], dtype=5), layout=0, table=None, mb=3) == OK
    assert mx_call(qs=None) == NULL                                   # scales are required
    assert mx_call(ks=None) == NULL
    assert mx_call(q=q0, qs=None, ks=None) == OK                      # ... unless T = 0
    assert mx_call(q=tdesc([4, 8, 128], dtype=0)) == DTYPE            # not MXFP4
    assert mx_call(k=tdesc([8, 128, 1, 128], dtype=1)) == DTYPE
    assert mx_call(q=tdesc([4, 8, 128], dtype=5)) == SHAPE            # 64 bytes per row
    assert mx_call(k=tdesc([8, 128, 1, 128], dtype=5)) == SHAPE
    assert mx_call(qs=FAKE + 2) == STRIDE                             # 4-byte aligned scales
    assert mx_call(ks=FAKE + 1) == STRIDE
    assert mx_call(local_mode=3) == ATTR
    assert mx_call(mode=1) == ATTR
    # the family entry: -1, 0, 1 accepted, anything else rejected; the same
    # checks otherwise
    for fam in (-1, 0, 1):
        assert mx_call(q=q0, family=fam) == OK
        assert mx_call(qs=None, family=fam) == NULL
    assert mx_call(q=q0, family=2) == ATTR
    assert mx_call(q=q0, family=-2) == ATTR
    assert mx_call(q=tdesc([4, 8, 128], dtype=0), family=0) == DTYPE
    # the other entries cannot carry the group scales
    assert call(q=tdesc([4, 8, 64], dtype=5), k=tdesc([8, 128, 1, 64], dtype=5)) == SCALE
    assert call(q=tdesc([4, 8, 64], dtype=5), k=tdesc([8, 128, 1, 64], dtype=5),
                local_mode=1) == SCALE


def test_block_topk_validation_without_launch():
    # Every call below fails validation or has no rows, so nothing launches.
    f = m.load_library().msa_block_topk
    P = ctypes.c_void_p(FAKE)
    assert f(P, 0, 5, 16, 16, 16, P, None) == OK          # Hq * T = 0
    assert f(P, 3, 0, 16, 16, 16, P, None) == OK
    assert f(None, 0, 0, 0, 0, 16, None, None) == OK
    assert f(P, 2, 3, 16, 16, 0, P, None) == ATTR         # k out of [1, 64]
    assert f(P, 2, 3, 16, 16, 65, P, None) == ATTR
    assert f(P, 2, 3, 16, 17, 16, P, None) == SHAPE       # num_valid > width
    assert f(P, 2, 3, 16, -1, 16, P, None) == SHAPE
    assert f(P, -1, 3, 16, 4, 16, P, None) == SHAPE
    assert f(P, 2, 3, (1 << 24) + 16, 4, 16, P, None) == SHAPE
    assert f(P, 65536, 3, 16, 4, 16, P, None) == SHAPE    # Hq is the grid's y extent
    assert f(P, 2, 1 << 34, 16, 4, 16, P, None) == SHAPE  # ceil(T / 4) blocks in x
    assert f(P, 1 << 14, 1 << 30, 1 << 24, 4, 16, P, None) == SHAPE   # element count
    assert f(None, 2, 3, 16, 4, 16, P, None) == NULL      # scores needed
    assert f(P, 2, 3, 16, 4, 16, None, None) == NULL      # out needed
    assert f(ctypes.c_void_p(FAKE + 2), 2, 3, 16, 4, 16, P, None) == STRIDE
    assert f(P, 2, 3, 16, 4, 16, ctypes.c_void_p(FAKE + 1), None) == STRIDE


def test_block_topk_binding_checks_shapes():
    s = torch.zeros(2, 3, 16)
    with pytest.raises(ValueError):
        m.msa_block_topk(s, 16, 16, torch.zeros(3, 2, 8, dtype=torch.int32))
    with pytest.raises(ValueError):
        m.msa_block_topk(s.double(), 16, 16, torch.zeros(3, 2, 16, dtype=torch.int32))


def test_block_size_must_be_128():
    # The logical block is the 128-token page (guide, section 四); every score
    # entry takes block_size and rejects any other value before launching.
    q0 = tdesc([0, 8, 128], dtype=0)
    assert call(q=q0) == OK
    for bs in (0, 64, 127, 129, 256):
        assert call(q=q0, bs=bs) == SHAPE
        assert call(q=q0, bs=bs, local_mode=1) == SHAPE
        assert call(q=q0, bs=bs, family=0) == SHAPE
        assert mx_call(q=tdesc([0, 8, 64], dtype=5), bs=bs) == SHAPE
        assert mx_call(q=tdesc([0, 8, 64], dtype=5), bs=bs, family=1) == SHAPE


# ---------------------------------------------------------------------------
# the Python wrappers: sizes the C ABI cannot see, and the guide's keyword API
# ---------------------------------------------------------------------------

def _cpu_args(B=2, T=0, Hq=8, mb=4):
    """Host tensors for a paged fp16 call with T query tokens (T = 0 never
    launches)."""
    return dict(query=torch.zeros(T, Hq, 128, dtype=torch.float16),
                key=torch.zeros(8, 128, 1, 128, dtype=torch.float16),
                start_loc=torch.zeros(B, dtype=torch.int32),
                block_table=torch.zeros(B, mb, dtype=torch.int32), scale=None,
                cu_seqlens_q=torch.zeros(B + 1, dtype=torch.int32),
                kv_len=torch.ones(B, dtype=torch.int32), layout="BBND", sparse_mode=3,
                init_blocks=0, local_blocks=1,
                out=torch.empty(Hq, T, m.msa_index_score_out_width(mb)), max_blocks=mb,
                stream=0)


def test_wrapper_accepts_consistent_sizes():
    m.msa_index_score(**_cpu_args())       # T = 0: validated, nothing launched


@pytest.mark.parametrize("change,what", [
    (dict(cu_seqlens_q=torch.zeros(2, dtype=torch.int32)), "cu_seqlens_q"),    # not [B+1]
    (dict(cu_seqlens_q=torch.zeros(4, dtype=torch.int32)), "cu_seqlens_q"),
    (dict(start_loc=torch.zeros(3, dtype=torch.int32)), "start_loc"),          # not [B]
    (dict(start_loc=None), "start_loc"),                                       # per-request window
    (dict(block_table=torch.zeros(1, 4, dtype=torch.int32)), "block_table"),  # fewer rows than B
    (dict(block_table=torch.zeros(2, 5, dtype=torch.int32)), "block_table"),  # width != MB
    (dict(kv_len=torch.ones(2, 1, dtype=torch.int32)), "kv_len"),             # not 1-D
    (dict(out=torch.empty(4, 0, 16)), "out"),                                  # Hq mismatch
    (dict(out=torch.empty(8, 3, 16)), "out"),                                  # T mismatch
])
def test_wrapper_rejects_inconsistent_sizes(change, what):
    a = _cpu_args()
    a.update(change)
    with pytest.raises(ValueError, match=what):
        m.msa_index_score(**a)


def test_wrapper_start_loc_optional_per_query():
    a = _cpu_args()
    a.update(start_loc=None, local_mode="query")
    m.msa_index_score(**a)


def test_wrapper_scale_size():
    a = _cpu_args()
    a.update(query=torch.zeros(0, 8, 128, dtype=torch.float16),
             key=torch.zeros(8, 1, 128, 128, dtype=torch.int8), layout="BNBD")
    a["scale"] = torch.ones(8, 1, 128)                 # [NP, Hkv, P]: one per token and head
    m.msa_index_score(**a)
    a["scale"] = torch.ones(8, 1, 64)
    with pytest.raises(ValueError, match="scale"):
        m.msa_index_score(**a)


def test_mxfp4_wrapper_sizes():
    B, mb = 2, 4
    base = dict(query=torch.zeros(0, 8, 64, dtype=torch.uint8),
                query_scale=torch.zeros(0, 8, 4, dtype=torch.uint8),
                key=torch.zeros(8, 128, 1, 64, dtype=torch.uint8),
                key_scale=torch.zeros(8, 128, 1, 4, dtype=torch.uint8),
                start_loc=torch.zeros(B, dtype=torch.int32),
                block_table=torch.zeros(B, mb, dtype=torch.int32),
                cu_seqlens_q=torch.zeros(B + 1, dtype=torch.int32),
                kv_len=torch.ones(B, dtype=torch.int32), layout="BBND", sparse_mode=3,
                init_blocks=0, local_blocks=1, out=torch.empty(8, 0, 16), max_blocks=mb,
                stream=0)
    m.msa_index_score_mxfp4(**base)
    for change, what in ((dict(key_scale=torch.zeros(8, 128, 1, 2, dtype=torch.uint8)),
                          "key_scale"),
                         (dict(query=torch.zeros(1, 8, 64, dtype=torch.uint8),
                               query_scale=torch.zeros(1, 8, 2, dtype=torch.uint8),
                               out=torch.empty(8, 1, 16)), "query_scale"),
                         (dict(cu_seqlens_q=torch.zeros(B, dtype=torch.int32)), "cu_seqlens_q"),
                         (dict(block_table=torch.zeros(B, mb + 1, dtype=torch.int32)),
                          "block_table")):
        a = dict(base, **change)
        with pytest.raises(ValueError, match=what):
            m.msa_index_score_mxfp4(**a)


def _guide_args(**kw):
    a = dict(block_table=torch.zeros(1, 2, dtype=torch.int32),
             atten_mask=torch.zeros(2048, 2048, dtype=torch.int8),
             actual_seq_qlen=torch.tensor([0, 0], dtype=torch.int32),
             actual_seq_klen=torch.tensor([256], dtype=torch.int32), stream=0)
    a.update(kw)
    return (torch.zeros(0, 8, 128, dtype=torch.float16),
            torch.zeros(8, 128, 1, 128, dtype=torch.float16),
            torch.tensor([1], dtype=torch.int32)), a


def test_guide_api_atten_mask_rules():
    # guide, sections 四 and 十: sparse_mode 3 takes the [2048, 2048] int8
    # template, sparse_mode 0 none; the host checks it, the device never reads it
    pos, kw = _guide_args()
    out = m.index_score(*pos, **kw)
    assert tuple(out.shape) == (8, 0, 16)
    for bad in (None, torch.zeros(2048, 2048, dtype=torch.bool),
                torch.zeros(1024, 2048, dtype=torch.int8)):
        pos, kw = _guide_args(atten_mask=bad)
        with pytest.raises(ValueError, match="atten_mask"):
            m.index_score(*pos, **kw)
    pos, kw = _guide_args(sparse_mode=0)
    with pytest.raises(ValueError, match="atten_mask"):
        m.index_score(*pos, **kw)
    pos, kw = _guide_args(sparse_mode=0, atten_mask=None)
    m.index_score(*pos, **kw)


def test_guide_api_tnd_prefix_sum(monkeypatch):
    # guide, section 四 and 6.3: a TND actual_seq_klen is the [B+1] prefix sum
    # of the packed key; the wrapper passes per-request lengths to the C ABI
    # and takes MB as the largest ceil(length / 128).
    seen = {}

    def spy(*a, **k):
        seen["kv_len"] = a[6].clone()
        seen["max_blocks"] = a[12]
        return a[11]

    monkeypatch.setattr(m._binding, "msa_index_score", spy)
    q = torch.zeros(0, 8, 128, dtype=torch.float16)
    key = torch.zeros(2200, 1, 128, dtype=torch.float16)
    out = m.index_score(q, key, torch.zeros(2, dtype=torch.int32),
                        atten_mask=torch.zeros(2048, 2048, dtype=torch.int8),
                        actual_seq_qlen=torch.zeros(3, dtype=torch.int32),
                        actual_seq_klen=torch.tensor([0, 2100, 2200], dtype=torch.int32),
                        layout_key="tnd", stream=0)
    assert seen["kv_len"].tolist() == [2100, 100]
    assert seen["kv_len"].dtype == torch.int32
    assert seen["max_blocks"] == 17 and tuple(out.shape) == (8, 0, 32)
    # an empty batch falls back to ceil(T2 / 128)
    m.index_score(q, key, torch.zeros(0, dtype=torch.int32),
                  atten_mask=torch.zeros(2048, 2048, dtype=torch.int8),
                  actual_seq_qlen=torch.zeros(1, dtype=torch.int32),
                  actual_seq_klen=torch.tensor([0], dtype=torch.int32), layout_key="TND",
                  stream=0)
    assert seen["max_blocks"] == (2200 + 127) // 128
