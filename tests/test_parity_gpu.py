"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases: every entry of the output, for both kernel families and the
automatic choice, against the oracle's full output.  Paged cases are also run
with every non-visible byte poisoned three ways; the GPU output must not move
by a single bit.  Full-size workloads: the GPU output of the configuration
that is benchmarked is compared entry by entry where the oracle can afford it
(decode batches) and on sampled full rows plus random entries otherwise.
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


def _sample_points(case, out_shape, n_rows, n_points, seed):
    """Full rows of a few (h, t) per request plus random single entries."""
    g = torch.Generator().manual_seed(seed)
    Hq, T, W = out_shape
    cu = case.cu_seqlens_q.long()
    rows = []
    for b in range(case.batch):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        if t1 <= t0:
            continue
        k = max(1, n_rows // max(case.batch, 1))
        ts = torch.randint(t0, t1, (k,), generator=g)
        ts[0] = t1 - 1                               # the last token sees the most blocks
        hs = torch.randint(0, Hq, (k,), generator=g)
        rows += list(zip(hs.tolist(), ts.tolist()))
    pts = [(h, t, beta) for h, t in rows for beta in range(W)]
    rnd = torch.stack([torch.randint(0, Hq, (n_points,), generator=g),
                       torch.randint(0, T, (n_points,), generator=g),
                       torch.randint(0, W, (n_points,), generator=g)], 1)
    full = torch.tensor(pts, dtype=torch.int64).reshape(-1, 3)
    return torch.cat([full, rnd]), len(rows)


@pytest.mark.parametrize("c_idx", [1, 2, 3, 4])
def test_full_size_config_parity(c_idx, dev):
    t0 = time.time()
    c = synth.config_case(c_idx)
    log(f"[gpu] config {c.name} generated in {time.time() - t0:.1f}s")
    got = run_gpu(c, dev)
    if c_idx == 1:
        ref = oracle_out(c)                  # decode batch: the whole output
        r = check(ref, got, tol_of(c))
        log(f"[gpu] {c.name} full: {r}")
        assert r["ok"], r
        return
    pts, nrows = _sample_points(c, got.shape, 64, 20000, 99 + c_idx)
    t1 = time.time()
    ref = oracle.index_score_case_points(c, pts)
    log(f"[gpu] {c.name}: oracle on {pts.shape[0]} sampled entries in {time.time() - t1:.1f}s")
    gv = got[pts[:, 0], pts[:, 1], pts[:, 2]]
    W = got.shape[2]
    nfull = nrows * W
    r = check(ref[:nfull].reshape(nrows, W), gv[:nfull].reshape(nrows, W), tol_of(c))
    log(f"[gpu] {c.name} sampled rows: {r}")
    assert r["ok"], r
    r2 = compare_values(ref[nfull:], gv[nfull:], tol_of(c))
    assert r2["ok"], r2


@pytest.mark.parametrize("c_idx", [2, 4])
def test_full_size_per_query_local_window(c_idx, dev):
    # The prefill workloads with the local window at each token's own block:
    # sampled rows and entries against the oracle, and on every row of the
    # output the token's own block carries the forced 1e29.
    import dataclasses
    c = dataclasses.replace(synth.config_case(c_idx), local_mode=1)
    log(f"[gpu] config {c.name}, per-query local window")
    got = run_gpu(c, dev)
    pts, nrows = _sample_points(c, got.shape, 32, 10000, 199 + c_idx)
    ref = oracle.index_score_case_points(c, pts)
    gv = got[pts[:, 0], pts[:, 1], pts[:, 2]]
    W = got.shape[2]
    nfull = nrows * W
    r = check(ref[:nfull].reshape(nrows, W), gv[:nfull].reshape(nrows, W), tol_of(c))
    log(f"[gpu] {c.name} per-query sampled rows: {r}")
    assert r["ok"], r
    r2 = compare_values(ref[nfull:], gv[nfull:], tol_of(c))
    assert r2["ok"], r2
    cu, kv = c.cu_seqlens_q.long(), c.kv_len.long()
    for b in range(c.batch):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        pos = int(kv[b]) - (t1 - t0) + torch.arange(t1 - t0)
        own = got[:, t0:t1].gather(2, (pos // 128).clamp(min=0)[None, :, None].expand(c.Hq, -1, 1))
        assert bool((own[:, pos >= 0] == 1e29).all()), c.name



@pytest.mark.parametrize("name", ["decode_bbnd_mxfp4", "prefill_bbnd_mxfp4"])
def test_full_size_mxfp4(name, dev):
    # The MXFP4 variants at their measured sizes: the whole decode batch, and
    # sampled rows and entries of the chunked prefill.
    c = synth.mx_config_case(name)
    log(f"[gpu] config {c.name}")
    got = run_gpu(c, dev)
    if name.startswith("decode"):
        r = check(oracle_out(c), got, tol_of(c))
        log(f"[gpu] {c.name} full: {r}")
        assert r["ok"], r
        return
    pts, nrows = _sample_points(c, got.shape, 32, 10000, 333)
    ref = oracle.index_score_case_points(c, pts)
    gv = got[pts[:, 0], pts[:, 1], pts[:, 2]]
    W = got.shape[2]
    nfull = nrows * W
    r = check(ref[:nfull].reshape(nrows, W), gv[:nfull].reshape(nrows, W), tol_of(c))
    log(f"[gpu] {c.name} sampled rows: {r}")
    assert r["ok"], r
    r2 = compare_values(ref[nfull:], gv[nfull:], tol_of(c))
    assert r2["ok"], r2
