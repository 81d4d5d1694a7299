"""Pins of the CPU oracle to things other than itself (CPU only).

Each test fixes part of the definition by an independent route: torch's own
format conversions, a vectorised brute force (masked_fill -> reshape -> amax),
hand-derived closed forms of the causal window, structural invariants (GQA map,
layouts, paging, poison, homogeneity), the int8 dequant identity, the printed
local_mask constants and the worked tiny example's structure.
"""
import dataclasses
import json
import os
import struct

import numpy as np
import pytest
import torch

import oracle
import synth
from brute import brute_force
from compare import INIT_BITS, LOCAL_BITS, NEG_INF_BITS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EDGE = synth.edge_cases()


def bits(x: torch.Tensor) -> torch.Tensor:
    return x.contiguous().view(torch.int32)


def assert_close_ulp(a: torch.Tensor, b: torch.Tensor, ulps: int = 1):
    """Equal specials bit for bit; finite entries within ``ulps`` float32 ulps."""
    assert a.shape == b.shape
    ab, bb = bits(a), bits(b)
    fin_a, fin_b = torch.isfinite(a), torch.isfinite(b)
    assert torch.equal(fin_a, fin_b)
    assert torch.equal(ab[~fin_a], bb[~fin_b])
    big = (a.abs() >= 1e28)
    assert torch.equal(ab[big], bb[big])
    fa, fb = a[fin_a & ~big].double(), b[fin_b & ~big].double()
    if fa.numel():
        ulp = torch.from_numpy(np.spacing(np.abs(fb.numpy()).astype(np.float32))).double()
        assert bool(((fa - fb).abs() <= ulps * ulp).all()), float(((fa - fb).abs() / ulp).max())


# ---------------------------------------------------------------------------
# decoders: every code against torch's conversion
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,nbits", [(torch.float16, 16), (torch.bfloat16, 16),
                                          (torch.float8_e4m3fn, 8), (torch.float8_e5m2, 8)])
def test_decoder_all_codes(dtype, nbits):
    if nbits == 16:
        codes = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(dtype)
    else:
        codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(dtype)
    want = codes.to(torch.float64).numpy()
    got = oracle.decode(codes)
    nan_w, nan_g = np.isnan(want), np.isnan(got)
    assert np.array_equal(nan_w, nan_g)
    assert np.array_equal(want[~nan_w], got[~nan_g])


def test_decoder_int8():
    codes = torch.arange(-128, 128, dtype=torch.int8)
    assert np.array_equal(oracle.decode(codes), np.arange(-128, 128, dtype=np.float64))


# ---------------------------------------------------------------------------
# printed constants and shapes
# ---------------------------------------------------------------------------

def test_out_width_golden():
    g = json.load(open(os.path.join(GOLDEN, "out_width.json")))
    for mb, w in g["max_blocks_to_width"]:
        assert oracle.out_width(mb) == w, (mb, w)


def test_local_mask_constant_bits():
    g = json.load(open(os.path.join(GOLDEN, "local_mask_constants.json")))
    assert struct.unpack("<i", struct.pack("<f", g["init_value"]))[0] == int(g["init_float32_bits"], 16)
    assert struct.unpack("<i", struct.pack("<f", g["local_value"]))[0] == int(g["local_float32_bits"], 16)
    assert INIT_BITS == int(g["init_float32_bits"], 16)
    assert LOCAL_BITS == int(g["local_float32_bits"], 16)
    assert NEG_INF_BITS == struct.unpack("<i", struct.pack("<I", int(g["fill_float32_bits"], 16)))[0]
    c = synth.make_case("consts", 11, q_lens=[2], kv_lens=[300], Hq=2, Hkv=1, qdtype="bf16",
                        layout="BBND", init_blocks=2, local_blocks=1, start_loc=[2])
    o = bits(oracle.index_score_case(c))
    assert bool((o[:, :, 0:2] == INIT_BITS).all())
    assert bool((o[:, :, 2] == LOCAL_BITS).all())
    assert bool((o[:, :, 3:] == NEG_INF_BITS).all())


def test_worked_tiny_example_structure():
    g = json.load(open(os.path.join(GOLDEN, "tiny_example.json")))
    c = synth.config_case(0)
    inp = g["inputs"]
    assert (c.T, c.Hq, c.Hkv, c.D, c.block_size, c.batch, c.key.shape[0], c.max_blocks) == (
        inp["T"], inp["Hq"], inp["Hkv"], inp["D"], inp["P"], inp["B"], inp["NP"], inp["MB"])
    assert c.cu_seqlens_q.tolist() == inp["cu_seqlens_q"] and c.kv_len.tolist() == inp["kv_len"]
    assert c.start_loc.tolist() == inp["start_loc"] and c.block_table.tolist() == [[0, 1]]
    o = oracle.index_score_case(c)
    assert list(o.shape) == g["expected"]["shape"]
    ob = bits(o)
    assert bool((ob[:, :, 1] == int(g["expected"]["column_1_bits_all_rows"], 16)).all())
    assert bool((ob[:, :, 2:] == NEG_INF_BITS).all())
    # column 0: every query position sees all of block 0 -> a plain matmul + amax
    q = c.query.to(torch.float64)                      # [32, 8, 128]
    k0 = c.key[0, :, 0, :].to(torch.float64)           # [128, 128]
    want = torch.matmul(q, k0.T).amax(-1).T.to(torch.float32)   # [8, 32]
    assert_close_ulp(o[:, :, 0].contiguous(), want.contiguous())


# ---------------------------------------------------------------------------
# brute force agreement over the whole edge suite
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("idx", range(len(EDGE)), ids=[c.name for c in EDGE])
def test_brute_force_agreement(idx):
    c = EDGE[idx]
    assert_close_ulp(oracle.index_score_case(c), brute_force(c))


RANDOM = synth.random_cases(40)


@pytest.mark.parametrize("idx", range(len(RANDOM)), ids=[c.name for c in RANDOM])
def test_brute_force_agreement_random(idx):
    c = RANDOM[idx]
    assert_close_ulp(oracle.index_score_case(c), brute_force(c))


MX_RANDOM = synth.mx_random_cases(12)


@pytest.mark.parametrize("idx", range(len(MX_RANDOM)), ids=[c.name for c in MX_RANDOM])
def test_brute_force_agreement_mx_random(idx):
    c = MX_RANDOM[idx]
    assert_close_ulp(oracle.index_score_case(c), brute_force(c))


# ---------------------------------------------------------------------------
# closed forms of the causal window
# ---------------------------------------------------------------------------

def _ramp_case(name, q_lens, kv_lens, layout, mode, qdtype="bf16"):
    """q = e_0, k_j[0] = j mod P (exact in fp16/bf16), all else 0: the score of a
    block is the offset of its last visible key inside the block."""
    c = synth.make_case(name, 5, q_lens=q_lens, kv_lens=kv_lens, Hq=2, Hkv=1, qdtype=qdtype,
                        layout=layout, sparse_mode=mode, init_blocks=0, local_blocks=0)
    q = torch.zeros_like(c.query)
    q[:, :, 0] = 1
    ks = torch.zeros_like(c.key_storage)
    ramp = torch.arange(128, dtype=torch.float32).to(ks.dtype)
    if layout == "BBND":
        ks[:, :, :, 0] = ramp[None, :, None]
    elif layout == "BNBD":
        ks[:, :, :, 0] = ramp[None, None, :]
    else:
        off = 0
        for L in kv_lens:
            ks[off:off + L, :, 0] = (torch.arange(L) % 128).to(ks.dtype)[:, None]
            off += L
    return dataclasses.replace(c, query=q, key=ks, key_storage=ks)


@pytest.mark.parametrize("layout", ["BBND", "BNBD", "TND"])
def test_window_closed_form_decode(layout):
    # one query token per request, right-down causal: it sees the whole KV.
    kv = [1, 127, 128, 129, 300, 512]
    c = _ramp_case("ramp_dec", [1] * len(kv), kv, layout, 3)
    o = oracle.index_score_case(c)
    for b, L in enumerate(kv):
        nb = -(-L // 128)
        for beta in range(o.shape[2]):
            if beta < nb - 1:
                want = 127.0
            elif beta == nb - 1:
                want = float((L - 1) - beta * 128)
            else:
                want = float("-inf")
            assert float(o[0, b, beta]) == want and float(o[1, b, beta]) == want


@pytest.mark.parametrize("mode", [3, 0])
def test_window_closed_form_prefill(mode):
    # request 0: no prefix (q_pos(i) = i); request 1: prefix of 200 (q_pos = 200 + i)
    q_lens, kv = [300, 90], [300, 290]
    c = _ramp_case("ramp_pre", q_lens, kv, "TND", mode)
    o = oracle.index_score_case(c)
    t = 0
    for b, (Lq, L) in enumerate(zip(q_lens, kv)):
        for i in range(Lq):
            qpos = (L - Lq + i) if mode == 3 else L - 1
            for beta in range(o.shape[2]):
                lo = beta * 128
                if lo <= qpos and lo < L:
                    want = float(min(qpos - lo, 127, L - 1 - lo))
                else:
                    want = float("-inf")
                assert float(o[0, t, beta]) == want, (b, i, beta)
            t += 1


# ---------------------------------------------------------------------------
# structural invariants
# ---------------------------------------------------------------------------

def test_gqa_replicated_heads_equal_single_kv_head():
    base = synth.make_case("g1", 21, q_lens=[3, 2], kv_lens=[200, 300], Hq=4, Hkv=1,
                           qdtype="bf16", layout="BBND", extra_pages=2)
    rep = base.key.expand(-1, -1, 4, -1).contiguous()           # Hkv = Hq = 4
    c4 = dataclasses.replace(base, key=rep, key_storage=rep)
    assert torch.equal(bits(oracle.index_score_case(base)), bits(oracle.index_score_case(c4)))


def test_gqa_head_map_one_hot():
    Hq, Hkv = 8, 4           # g = 2: heads (0,1)->0, (2,3)->1, ...
    c = synth.make_case("onehot", 22, q_lens=[2], kv_lens=[150], Hq=Hq, Hkv=Hkv, qdtype="f16",
                        layout="BBND", init_blocks=0, local_blocks=0)
    q = torch.zeros_like(c.query)
    q[:, :, :Hkv] = 1
    ks = torch.zeros_like(c.key_storage)
    for hk in range(Hkv):
        ks[:, :, hk, hk] = hk + 1
    o = oracle.index_score_case(dataclasses.replace(c, query=q, key=ks, key_storage=ks))
    for h in range(Hq):
        assert bool((o[h, :, :2] == float(h // (Hq // Hkv) + 1)).all())


def _as_bnbd(c):
    kb = c.key.permute(0, 2, 1, 3).contiguous()
    sc = c.scale
    return dataclasses.replace(c, key=kb, key_storage=kb, layout="BNBD", scale=sc, gap=0)


def _as_tnd(c):
    P = c.block_size
    keys, scales = [], []
    for b in range(c.batch):
        L = int(c.kv_len[b])
        nb = -(-L // P)
        pages = c.block_table[b, :nb].long()
        kp = c.key[pages]
        keys.append(kp.reshape(nb * P, kp.shape[2], kp.shape[3])[:L])
        if c.scale is not None:
            scales.append(c.scale[pages].permute(0, 2, 1).reshape(nb * P, -1)[:L])
    kt = torch.cat(keys).contiguous()
    st = torch.cat(scales).contiguous() if scales else None
    return dataclasses.replace(c, key=kt, key_storage=kt, layout="TND", block_table=None,
                               scale=st, gap=0)


def _repaged(c, seed):
    """Same logical keys behind a different physical page permutation."""
    g = torch.Generator().manual_seed(seed)
    NP = c.key.shape[0]
    perm = torch.randperm(NP, generator=g)          # new page of old page p is perm[p]
    kn = torch.empty_like(c.key)
    kn[perm] = c.key
    sn = None
    if c.scale is not None:
        sn = torch.empty_like(c.scale)
        sn[perm] = c.scale
    bt = perm[c.block_table.long()].to(torch.int32)
    return dataclasses.replace(c, key=kn, key_storage=kn, block_table=bt, scale=sn, gap=0)


@pytest.mark.parametrize("kd", ["bf16", "i8", "f8e4m3"])
def test_layouts_and_paging_equivalent(kd):
    qd = "f16" if kd == "i8" else kd
    c = synth.make_case("lay", 31, q_lens=[3, 1, 20], kv_lens=[260, 1, 400], Hq=4, Hkv=2,
                        qdtype=qd, kdtype=kd, layout="BBND", extra_pages=3, init_blocks=1,
                        local_blocks=2)
    ref = bits(oracle.index_score_case(c))
    assert torch.equal(ref, bits(oracle.index_score_case(_as_bnbd(c))))
    assert torch.equal(ref, bits(oracle.index_score_case(_as_tnd(c))))
    assert torch.equal(ref, bits(oracle.index_score_case(_repaged(c, 5))))


def test_dim0_gap_equivalent():
    c = synth.make_case("gap", 32, q_lens=[2, 2], kv_lens=[300, 129], Hq=4, Hkv=1,
                        qdtype="bf16", layout="BBND", extra_pages=2, gap=2)
    assert c.key.stride(0) == 3 * c.key[0].numel()
    dense = c.key.contiguous()
    ref = bits(oracle.index_score_case(c))
    assert torch.equal(ref, bits(oracle.index_score_case(
        dataclasses.replace(c, key=dense, key_storage=dense, gap=0))))


@pytest.mark.parametrize("name", ["mix_bbnd_bf16", "mix_bnbd_i8", "mix_bbnd_f8e4m3",
                                  "dim0_gap2_bnbd_i8", "wide_table_257", "tiny_kv_tail"])
def test_poison_invariance(name):
    c = next(x for x in EDGE if x.name == name)
    ref = bits(oracle.index_score_case(c))
    for pat in ("zero", "big", "nan"):
        assert torch.equal(ref, bits(oracle.index_score_case(synth.poison_case(c, pat)))), pat


def test_homogeneity_power_of_two():
    c = next(x for x in EDGE if x.name == "mix_bbnd_bf16")
    o1 = oracle.index_score_case(c)
    o2 = oracle.index_score_case(dataclasses.replace(c, query=c.query * 2))
    fin = torch.isfinite(o1) & (o1.abs() < 1e28)
    assert torch.equal(bits(o1[~fin]), bits(o2[~fin]))
    assert torch.equal(o2[fin], 2 * o1[fin])


# ---------------------------------------------------------------------------
# int8: Q.(K s) == (Q.cast K) s
# ---------------------------------------------------------------------------

def test_dequant_identity_power_of_two_scales():
    c = synth.make_case("dq", 41, q_lens=[2, 5], kv_lens=[300, 77], Hq=4, Hkv=2, qdtype="f16",
                        kdtype="i8", layout="BNBD", extra_pages=2, init_blocks=0, local_blocks=0)
    g = torch.Generator().manual_seed(3)
    e = torch.randint(-9, -3, c.scale.shape, generator=g)
    s = torch.ldexp(torch.ones_like(c.scale), e)                   # 2^e, exact
    ci = dataclasses.replace(c, scale=s)
    kf = (c.key.to(torch.float32) * s[:, :, :, None]).to(torch.float16)   # exact in fp16
    assert torch.equal(kf.to(torch.float32), c.key.to(torch.float32) * s[:, :, :, None])
    cf = dataclasses.replace(c, key=kf, key_storage=kf, scale=None)
    assert torch.equal(bits(oracle.index_score_case(ci)), bits(oracle.index_score_case(cf)))


def test_dequant_unit_scale_is_cast():
    c = synth.make_case("dq1", 42, q_lens=[3], kv_lens=[250], Hq=4, Hkv=1, qdtype="f16",
                        kdtype="i8", layout="BBND")
    ci = dataclasses.replace(c, scale=torch.ones_like(c.scale))
    kf = c.key.to(torch.float16)
    cf = dataclasses.replace(c, key=kf, key_storage=kf, scale=None)
    assert torch.equal(bits(oracle.index_score_case(ci)), bits(oracle.index_score_case(cf)))


# ---------------------------------------------------------------------------
# empty requests and batches
# ---------------------------------------------------------------------------

def test_empty_kv_request_all_neg_inf():
    c = next(x for x in EDGE if x.name == "pad_tnd_kvlen0")    # request 0: kv_len = 0
    o = bits(oracle.index_score_case(c))
    assert c.kv_len[0] == 0 and c.init_blocks == 1
    assert bool((o[:, 0:4, :] == NEG_INF_BITS).all())        # no local_mask either
    assert bool((o[:, 4:, 0] == INIT_BITS).all())


def test_empty_batch_shapes():
    c = next(x for x in EDGE if x.name == "empty_batch")
    assert c.T == 0
    assert tuple(oracle.index_score_case(c).shape) == (4, 0, 16)
    c = next(x for x in EDGE if x.name == "all_kv_empty_tnd")
    o = oracle.index_score_case(c)
    assert tuple(o.shape) == (4, 5, 16) and bool((bits(o) == NEG_INF_BITS).all())


def test_rows_that_see_nothing_get_neg_inf_then_local_mask():
    c = next(x for x in EDGE if x.name == "q_longer_than_kv")   # L_q = 10 > kv_len = 6
    o = bits(oracle.index_score_case(c))
    # rows 0..3 have q_pos < 0 and see nothing; start_loc = 0, so block 0 is
    # forced by the local window (which overrides the init block), the rest -inf
    assert int(c.start_loc[0]) == 0 and c.init_blocks == 1 and c.local_blocks == 1
    assert bool((o[:, 0:4, 0] == LOCAL_BITS).all())
    assert bool((o[:, 0:4, 1:] == NEG_INF_BITS).all())


def test_contract_violation_raises():
    c = synth.make_case("bad", 51, q_lens=[1], kv_lens=[300], Hq=2, Hkv=1, qdtype="bf16",
                        layout="BBND")
    bad = dataclasses.replace(c, kv_len=torch.tensor([1000], dtype=torch.int32))
    with pytest.raises(ValueError):
        oracle.index_score_case(bad)


def test_packed_key_block_count_above_max_blocks_raises():
    # Packed (TND) keys: MB is the largest ceil(kv_len / 128) of the batch
    # (guide, section 五), so a request with more blocks than MB breaks the
    # contract even when its blocks would still fit the aligned width.
    c = synth.make_case("tnd_mb", 52, q_lens=[2, 3], kv_lens=[300, 700], Hq=2, Hkv=1,
                        qdtype="bf16", layout="TND")
    assert c.max_blocks == 6
    oracle.index_score_case(c)                     # NB = 3 and 6: within MB
    for mb in (5, 3):                              # W stays 16 > NB = 6
        with pytest.raises(ValueError):
            oracle.index_score_case(dataclasses.replace(c, max_blocks=mb))


# ---------------------------------------------------------------------------
# MXFP4 element and scale decoders
# ---------------------------------------------------------------------------

def test_e2m1_decoder_matches_the_e4m3fn_route():
    # An E2M1 code (bias 1) is the e4m3fn code with exponent + 6 and the
    # fraction bit moved up (tests/brute.py), which torch decodes.
    from brute import _e2m1_as_e4m3fn
    lib = oracle.load()
    codes = torch.arange(16, dtype=torch.uint8)
    want = _e2m1_as_e4m3fn(codes).tolist()
    got = [lib.orc_decode_e2m1(int(c)) for c in codes]
    assert got == want
    # the format's shape: largest 6, smallest positive 0.5, symmetric
    assert max(got) == 6.0 and min(x for x in got if x > 0) == 0.5
    assert [abs(x) for x in got[8:]] == got[:8] and all(x <= 0 for x in got[8:])


def test_e8m0_decoder_matches_torch():
    lib = oracle.load()
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e8m0fnu).to(torch.float64).tolist()
    got = [lib.orc_decode_e8m0(int(c)) for c in codes]
    assert all((g == w) or (g != g and w != w) for g, w in zip(got, want))
