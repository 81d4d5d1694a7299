"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases: every entry of the output, for both kernel families and the
automatic choice, against the oracle's full output.  Paged cases are also run
with every non-visible byte poisoned three ways; the GPU output must not move
by a single bit.  Full-size workloads: every entry of the decode batches'
outputs, and for the prefill workloads over a thousand stratified full rows
(every request and KV group, prefill-tile edges, local-window tokens) plus
random single entries, each with its top-k block sets.
"""
import os
import sys
import time

import pytest
import torch

import oracle
import synth
from compare import TOL, check, compare_values

pytestmark = pytest.mark.gpu

EDGE = synth.edge_cases()
PAGED = [c for c in EDGE if c.layout != "TND"]
RANDOM = synth.random_cases(40)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_max_qk_amd
    block_max_qk_amd.load_library()
    return torch.device("cuda:0")


def to_device(case, dev):
    ks = case.key_storage.to(dev)
    key = ks[:: case.gap + 1] if (case.gap and case.layout != "TND") else ks
    assert key.stride() == case.key.stride()
    mx = lambda t: None if t is None else t.to(dev)   # noqa: E731
    return dict(
        query=case.query.to(dev), key=key, start_loc=case.start_loc.to(dev),
        block_table=None if case.block_table is None else case.block_table.to(dev),
        scale=None if case.scale is None else case.scale.to(dev),
        cu_seqlens_q=case.cu_seqlens_q.to(dev), kv_len=case.kv_len.to(dev),
        q_mx=mx(case.q_mx_scale), k_mx=mx(case.k_mx_scale))


def run_gpu(case, dev, family=-1):
    """The GPU output of a case through the C ABI (MXFP4 cases take their own
    entry)."""
    import block_max_qk_amd as m
    d = to_device(case, dev)
    W = m.msa_index_score_out_width(case.max_blocks)
    out = torch.full((case.Hq, case.T, W), 12345.0, dtype=torch.float32, device=dev)
    if case.q_mx_scale is not None:
        m.msa_index_score_mxfp4(d["query"], d["q_mx"], d["key"], d["k_mx"], d["start_loc"],
                                d["block_table"], d["cu_seqlens_q"], d["kv_len"], case.layout,
                                case.sparse_mode, case.init_blocks, case.local_blocks, out,
                                case.max_blocks, local_mode=case.local_mode, family=family)
        torch.cuda.synchronize()
        return out.cpu()
    m.msa_index_score(d["query"], d["key"], d["start_loc"], d["block_table"], d["scale"],
                      d["cu_seqlens_q"], d["kv_len"], case.layout, case.sparse_mode,
                      case.init_blocks, case.local_blocks, out, case.max_blocks, family=family,
                      local_mode=case.local_mode)
    torch.cuda.synchronize()
    return out.cpu()


_ORACLE = {}


def oracle_out(case):
    key = (case.name, case.poison)
    if key not in _ORACLE:
        _ORACLE[key] = oracle.index_score_case(case)
    return _ORACLE[key]


def tol_of(case):
    return TOL[case.key_dtype_name()]


@pytest.mark.parametrize("family", [-1, 0, 1])
@pytest.mark.parametrize("idx", range(len(EDGE)), ids=[c.name for c in EDGE])
def test_edge_case_parity(idx, family, dev):
    c = EDGE[idx]
    log(f"[gpu] edge {c.name} family={family} {synth.case_summary(c)}")
    ref = oracle_out(c)
    got = run_gpu(c, dev, family)
    r = check(ref, got, tol_of(c))
    assert r["ok"], r


@pytest.mark.parametrize("family", [0, 1])
@pytest.mark.parametrize("idx", range(len(RANDOM)), ids=[c.name for c in RANDOM])
def test_random_sweep_parity(idx, family, dev):
    c = RANDOM[idx]
    log(f"[gpu] random {c.name} family={family} {synth.case_summary(c)}")
    r = check(oracle_out(c), run_gpu(c, dev, family), tol_of(c))
    assert r["ok"], r


LARGE_BATCH_NAMES = ["batch65_bbnd_bf16", "batch300_bnbd_i8_spec", "batch1000_tnd_f16",
                     "batch200_bbnd_f16_perq", "batch16500_tnd_bf16", "batch64_bbnd_bf16_g128"]
_LARGE = []


def large_batch(idx):
    # built on first use (about 2 GB of host tensors), not at collection
    if not _LARGE:
        _LARGE.extend(synth.large_batch_cases())
        assert [c.name for c in _LARGE] == LARGE_BATCH_NAMES
    return _LARGE[idx]


@pytest.mark.parametrize("family", [0, 1])
@pytest.mark.parametrize("idx", range(len(LARGE_BATCH_NAMES)), ids=LARGE_BATCH_NAMES)
def test_large_batch_parity(idx, family, dev):
    # more than one 64-request chunk: the decode kernel's chunk table and
    # contiguous fill items, and the prefill request lookup, past 16384
    # requests included; and 64 requests whose decode workgroup slices run
    # past one 64-entry page window, several requests to a window
    c = large_batch(idx)
    log(f"[gpu] large batch {c.name} family={family} {synth.case_summary(c)}")
    r = check(oracle_out(c), run_gpu(c, dev, family), tol_of(c))
    assert r["ok"], r


MX_RANDOM = synth.mx_random_cases(12)


@pytest.mark.parametrize("family", [0, 1])
@pytest.mark.parametrize("idx", range(len(MX_RANDOM)), ids=[c.name for c in MX_RANDOM])
def test_mx_random_sweep_parity(idx, family, dev):
    c = MX_RANDOM[idx]
    log(f"[gpu] mx random {c.name} family={family} {synth.case_summary(c)}")
    r = check(oracle_out(c), run_gpu(c, dev, family), tol_of(c))
    assert r["ok"], r


@pytest.mark.parametrize("family", [0, 1])
@pytest.mark.parametrize("idx", range(len(PAGED)), ids=[c.name for c in PAGED])
def test_poison_invariance(idx, family, dev):
    c = PAGED[idx]
    base = run_gpu(c, dev, family)
    for pat in ("zero", "big", "nan"):
        log(f"[gpu] poison {c.name} family={family} pattern={pat}")
        got = run_gpu(synth.poison_case(c, pat), dev, family)
        assert torch.equal(base.view(torch.int32), got.view(torch.int32)), pat


def test_tiny_config_full(dev):
    c = synth.config_case(0)
    log(f"[gpu] config {c.name}")
    r = check(oracle_out(c), run_gpu(c, dev), tol_of(c))
    assert r["ok"], r


# Query tokens per prefill tile by key type (the tile is 4 waves of 32-row
# MFMA N tiles holding the g heads of a KV group for consecutive tokens); only
# used to aim samples at tile edges, where the causal window cuts the tile's
# diagonal block differently for its first and last token.
PREFILL_TILE_ROWS = {"f16": 384, "bf16": 384, "i8": 256, "f8e4m3": 256, "f8e5m2": 256,
                     "mxfp4": 512}


def stratified_rows(case, n_rows, seed):
    """About n_rows distinct (h, t) rows spread over every request: the
    first and last token of the request, the first and last token of prefill
    tiles spaced evenly along it (their diagonal blocks are masked
    differently), the first and last token whose own block is the request's
    local_mask anchor (start_loc), and random tokens; heads cycle over all
    Hq, so every KV group is covered."""
    g = torch.Generator().manual_seed(seed)
    cu, kv = case.cu_seqlens_q.long(), case.kv_len.long()
    live = [b for b in range(case.batch) if int(cu[b + 1]) > int(cu[b])]
    if not live:
        return []
    g_heads = case.Hq // case.Hkv
    tpt = max(1, PREFILL_TILE_ROWS[case.key_dtype_name()] // min(g_heads, 256))
    quota = max(8, -(-n_rows // len(live)))
    rows = []
    for b in live:
        t0, t1 = int(cu[b]), int(cu[b + 1])
        Lq, L = t1 - t0, int(kv[b])
        toks = [t0, t1 - 1]
        ntile = -(-Lq // tpt)
        for k in torch.linspace(0, ntile - 1, max(1, min(ntile, quota // 4))).round().long():
            s0 = t0 + int(k) * tpt
            toks += [s0, min(s0 + tpt, t1) - 1]
        anchor = int(case.start_loc[b])
        pos0 = L - Lq
        own = [t0 + i for i in (anchor * 128 - pos0, anchor * 128 + 127 - pos0) if 0 <= i < Lq]
        toks += own
        toks = list(dict.fromkeys(toks))[: quota]
        off = int(torch.randint(0, case.Hq, (1,), generator=g))
        mine = dict.fromkeys(((off + i) % case.Hq, t) for i, t in enumerate(toks))
        want = min(quota, Lq * case.Hq)
        while len(mine) < want:       # random rows of the request up to its quota
            mine[(int(torch.randint(0, case.Hq, (1,), generator=g)),
                  int(torch.randint(t0, t1, (1,), generator=g)))] = None
        rows += list(mine)
    return rows


def row_points(rows, W):
    """All (h, t, beta) entries of the given rows, row-major."""
    hs = torch.tensor([h for h, _ in rows], dtype=torch.int64)
    ts = torch.tensor([t for _, t in rows], dtype=torch.int64)
    n = len(rows)
    return torch.stack([hs.repeat_interleave(W), ts.repeat_interleave(W),
                        torch.arange(W).repeat(n)], 1)


_ROWS = {}


def oracle_rows(case, n_rows, seed):
    """The oracle's full rows at stratified (h, t): (rows, [n, W] values);
    cached per workload for the top-k tests, which reuse them."""
    key = (case.name, case.local_mode, n_rows, seed)
    if key not in _ROWS:
        W = ((max(case.max_blocks, 1) + 15) // 16) * 16
        rows = stratified_rows(case, n_rows, seed)
        t1 = time.time()
        vals = oracle.index_score_case_points(case, row_points(rows, W)).reshape(len(rows), W)
        log(f"[gpu] {case.name}: oracle on {len(rows)} full rows in {time.time() - t1:.1f}s")
        _ROWS[key] = (rows, vals)
    return _ROWS[key]


def gpu_rows(got, rows):
    hs = torch.tensor([h for h, _ in rows], dtype=torch.int64)
    ts = torch.tensor([t for _, t in rows], dtype=torch.int64)
    return got[hs, ts]


# Near-tie bound: top-k sets may differ only on blocks whose oracle scores lie
# within the score tolerance of the oracle's k-th score, and on at most 1% of
# the rows compared (the GPU's float32 sums can reorder two blocks only when
# their exact scores are that close).
NEAR_TIE_ROW_FRACTION = 0.01


def assert_rows_match(ref, got, tol, what):
    r = check(ref, got, tol)
    log(f"[gpu] {what}: {r}")
    assert r["ok"], r
    t = r["topk"]
    assert t["near_tie_rows"] <= NEAR_TIE_ROW_FRACTION * max(t["rows"], 1), t
    return r


FULL_SIZE_ROWS = 1024


@pytest.mark.parametrize("c_idx", [1, 2, 3, 4])
def test_full_size_config_parity(c_idx, dev):
    t0 = time.time()
    c = synth.config_case(c_idx)
    log(f"[gpu] config {c.name} generated in {time.time() - t0:.1f}s")
    got = run_gpu(c, dev)
    if c.T <= 256:
        # decode batches: every entry of the output against the oracle's
        t1 = time.time()
        ref = oracle_out(c)
        log(f"[gpu] {c.name}: whole oracle output in {time.time() - t1:.1f}s")
        assert_rows_match(ref, got, tol_of(c), f"{c.name} whole output")
        return
    # prefill workloads: stratified full rows (every request and KV group,
    # tile edges, local-window tokens), then random single entries
    rows, ref = oracle_rows(c, FULL_SIZE_ROWS, 99 + c_idx)
    assert len(rows) >= FULL_SIZE_ROWS
    assert len({(h // (c.Hq // c.Hkv)) for h, _ in rows}) == c.Hkv
    assert_rows_match(ref, gpu_rows(got, rows), tol_of(c), f"{c.name} {len(rows)} full rows")
    g = torch.Generator().manual_seed(7 + c_idx)
    Hq, T, W = got.shape
    rnd = torch.stack([torch.randint(0, Hq, (20000,), generator=g),
                       torch.randint(0, T, (20000,), generator=g),
                       torch.randint(0, W, (20000,), generator=g)], 1)
    r2 = compare_values(oracle.index_score_case_points(c, rnd),
                        got[rnd[:, 0], rnd[:, 1], rnd[:, 2]], tol_of(c))
    assert r2["ok"], r2


def _sample_points(case, out_shape, n_rows, n_points, seed):
    """Full rows at stratified (h, t) plus random single entries."""
    g = torch.Generator().manual_seed(seed)
    Hq, T, W = out_shape
    rows = stratified_rows(case, n_rows, seed)
    rnd = torch.stack([torch.randint(0, Hq, (n_points,), generator=g),
                       torch.randint(0, T, (n_points,), generator=g),
                       torch.randint(0, W, (n_points,), generator=g)], 1)
    return torch.cat([row_points(rows, W), rnd]), len(rows)


@pytest.mark.parametrize("c_idx", [2, 4])
def test_full_size_per_query_local_window(c_idx, dev):
    # The prefill workloads with the local window at each token's own block:
    # sampled rows and entries against the oracle, and on every row of the
    # output the token's own block carries the forced 1e29.
    import dataclasses
    c = dataclasses.replace(synth.config_case(c_idx), local_mode=1)
    log(f"[gpu] config {c.name}, per-query local window")
    got = run_gpu(c, dev)
    pts, nrows = _sample_points(c, got.shape, 256, 10000, 199 + c_idx)
    ref = oracle.index_score_case_points(c, pts)
    gv = got[pts[:, 0], pts[:, 1], pts[:, 2]]
    W = got.shape[2]
    nfull = nrows * W
    assert_rows_match(ref[:nfull].reshape(nrows, W), gv[:nfull].reshape(nrows, W), tol_of(c),
                      f"{c.name} per-query {nrows} full rows")
    r2 = compare_values(ref[nfull:], gv[nfull:], tol_of(c))
    assert r2["ok"], r2
    cu, kv = c.cu_seqlens_q.long(), c.kv_len.long()
    for b in range(c.batch):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        pos = int(kv[b]) - (t1 - t0) + torch.arange(t1 - t0)
        own = got[:, t0:t1].gather(2, (pos // 128).clamp(min=0)[None, :, None].expand(c.Hq, -1, 1))
        assert bool((own[:, pos >= 0] == 1e29).all()), c.name


@pytest.mark.parametrize("which", ["e5m2", "i8"])
def test_full_size_variant(which, dev):
    # The chunked fp8 prefill with e5m2 operands (the other OCP fp8 format,
    # same kernels), and the varlen prefill with int8 packed keys and their
    # scales: stratified full rows and random entries.
    c = synth.e5m2_config_case() if which == "e5m2" else synth.i8_prefill_config_case()
    log(f"[gpu] config {c.name}")
    got = run_gpu(c, dev)
    pts, nrows = _sample_points(c, got.shape, 256, 10000, 555)
    ref = oracle.index_score_case_points(c, pts)
    gv = got[pts[:, 0], pts[:, 1], pts[:, 2]]
    W = got.shape[2]
    nfull = nrows * W
    assert len({(h // (c.Hq // c.Hkv)) for h, _ in stratified_rows(c, 256, 555)}) == c.Hkv
    assert_rows_match(ref[:nfull].reshape(nrows, W), gv[:nfull].reshape(nrows, W), tol_of(c),
                      f"{c.name} {nrows} full rows")
    r2 = compare_values(ref[nfull:], gv[nfull:], tol_of(c))
    assert r2["ok"], r2


@pytest.mark.parametrize("name", ["decode_bbnd_mxfp4", "prefill_tnd_mxfp4",
                                  "prefill_bbnd_mxfp4"])
def test_full_size_mxfp4(name, dev):
    # The MXFP4 variants at their measured sizes: the whole decode batch, and
    # stratified full rows and random entries of the two prefills.
    c = synth.mx_config_case(name)
    log(f"[gpu] config {c.name}")
    got = run_gpu(c, dev)
    if name.startswith("decode"):
        assert_rows_match(oracle_out(c), got, tol_of(c), f"{c.name} whole output")
        return
    pts, nrows = _sample_points(c, got.shape, 512, 10000, 333)
    ref = oracle.index_score_case_points(c, pts)
    gv = got[pts[:, 0], pts[:, 1], pts[:, 2]]
    W = got.shape[2]
    nfull = nrows * W
    assert_rows_match(ref[:nfull].reshape(nrows, W), gv[:nfull].reshape(nrows, W), tol_of(c),
                      f"{c.name} {nrows} full rows")
    r2 = compare_values(ref[nfull:], gv[nfull:], tol_of(c))
    assert r2["ok"], r2
