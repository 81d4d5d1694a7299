"""Parity of the HIP top-k block selection (msa_block_topk, through the C ABI)
with the CPU oracle.

Integer work, so the bar is bit-exactness: on seeded score rows full of exact
ties, -inf holes, NaN and the local_mask constants, and on the score rows the
HIP path itself produces for every benchmark workload (so the selection runs
on exactly the same floats on both sides).  Row lengths cover the register
paths (up to 2048 blocks) and the re-reading path above it, with num_valid
cutting rows short and k at its limits.  The full pipeline (GPU scores -> GPU
top-k) is also compared with the oracle's own scores -> oracle top-k, where
sets may differ only on blocks tied within the score tolerance.
"""
import sys

import pytest
import torch

import oracle
import synth
from compare import TOL
from test_parity_gpu import run_gpu

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_max_qk_amd
    block_max_qk_amd.load_library()
    return torch.device("cuda:0")


def gpu_topk(scores_cpu, dev, num_valid, k):
    import block_max_qk_amd as m
    s = scores_cpu.to(dev)
    Hq, T, W = s.shape
    out = torch.full((T, Hq, k), 777, dtype=torch.int32, device=dev)
    m.msa_block_topk(s, num_valid, k, out)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("W", [1, 16, 100, 256, 512, 1000, 1024, 2048, 2100, 4112])
@pytest.mark.parametrize("k", [1, 16, 64])
def test_random_rows_exact(W, k, dev):
    s = synth.score_rows(9000 + 3 * W + k, 3, 5, W)
    for nv in sorted({0, W // 3, W}):
        log(f"topk rows W={W} k={k} num_valid={nv}")
        assert torch.equal(gpu_topk(s, dev, nv, k), oracle.block_topk(s, nv, k)), (W, k, nv)


@pytest.mark.parametrize("ties", [True, False])
def test_many_rows_exact(ties, dev):
    s = synth.score_rows(31 if ties else 32, 8, 700, 512, ties=ties)
    log(f"topk many rows ties={ties}")
    assert torch.equal(gpu_topk(s, dev, 512, 16), oracle.block_topk(s, 512, 16))


@pytest.mark.parametrize("W,nv,ties", [(100, 100, True), (512, 300, False), (1024, 1024, True)])
def test_many_rows_ragged_tail(W, nv, ties, dev):
    # Enough rows that each wave takes several in turn, with T leaving a
    # partial group of rows at the end of every head.
    s = synth.score_rows(40 + W, 2, 40003, W, ties=ties)
    log(f"topk many rows, ragged T: W={W} num_valid={nv} ties={ties}")
    assert torch.equal(gpu_topk(s, dev, nv, 16), oracle.block_topk(s, nv, 16))


def test_degenerate_rows(dev):
    W = 300
    s = torch.full((2, 3, W), float("-inf"))
    s[0, 0, 7] = 1.0                     # one candidate
    s[0, 1, :] = 2.5                     # all tied: the lowest 16 indices
    s[0, 2, :] = float("nan")            # nothing selectable
    s[1, 0, ::2] = 1e30                  # more forced blocks than k
    s[1, 1, 5:9] = 1e29                  # fewer forced blocks than k, rest -inf
    s[1, 2, :] = torch.arange(W, dtype=torch.float32)   # strictly increasing
    for k in (1, 16, 64):
        log(f"topk degenerate k={k}")
        assert torch.equal(gpu_topk(s, dev, W, k), oracle.block_topk(s, W, k))
    assert gpu_topk(s, dev, 0, 16).eq(-1).all()


def limit_rows(W):
    """Rows at the limits of the register path's compaction (64 entries) and
    of its upper bound (forced local_mask blocks around k)."""
    g = torch.Generator().manual_seed(77 + W)
    rows = []
    for n in (16, 17, 63, 64, 65, 128):        # n equal candidates, -inf elsewhere
        r = torch.full((W,), float("-inf"))
        r[:n] = 1.0
        rows.append(r)
    for n in (64, 65):                          # n distinct candidates spread over the row
        r = torch.full((W,), float("-inf"))
        r[torch.randperm(W, generator=g)[:n]] = torch.randn(n, generator=g) * 11 + 30
        rows.append(r)
    for f in (15, 16, 17, 40):                  # f forced blocks on computed scores
        r = torch.randn(W, generator=g) * 11 + 30
        pos = torch.randperm(W, generator=g)[:f]
        r[pos] = 1e29
        r[pos[: f // 3]] = 1e30
        rows.append(r)
    r = torch.zeros(W)                          # -0.0 and +0.0 are one score: lower blocks first
    r[torch.randperm(W, generator=g)[: W // 2]] = -0.0
    rows.append(r)
    r = torch.randn(W, generator=g) * 11 + 30   # NaN and -inf holes among the scores
    r[torch.randperm(W, generator=g)[: W // 4]] = float("nan")
    r[torch.randperm(W, generator=g)[: W // 4]] = float("-inf")
    rows.append(r)
    return torch.stack(rows)[None].contiguous()


@pytest.mark.parametrize("W", [512, 1024])
def test_compaction_and_bound_limits(W, dev):
    s = limit_rows(W)
    for nv in (W, W - 37):
        for k in (1, 8, 16, 17):
            log(f"topk limit rows W={W} num_valid={nv} k={k}")
            assert torch.equal(gpu_topk(s, dev, nv, k), oracle.block_topk(s, nv, k)), (W, nv, k)


def test_empty_sizes_launch_nothing(dev):
    import block_max_qk_amd as m
    for shape in ((0, 4, 16), (3, 0, 16)):
        s = torch.zeros(shape, device=dev)
        out = torch.empty((shape[1], shape[0], 16), dtype=torch.int32, device=dev)
        m.msa_block_topk(s, 16, 16, out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("c", range(len(synth.CONFIG_NAMES)), ids=synth.CONFIG_NAMES)
def test_workload_scores_exact(c, dev):
    case = synth.config_case(c)
    log(f"topk on the GPU scores of {case.name}")
    scores = run_gpu(case, dev)
    Hq, T, W = scores.shape
    got = gpu_topk(scores, dev, case.max_blocks, 16)
    if Hq * T <= 4096:
        want = oracle.block_topk(scores, case.max_blocks, 16)
        assert torch.equal(got, want)
        return
    g = torch.Generator().manual_seed(77 + c)
    rows = torch.randperm(Hq * T, generator=g)[:3000]
    h, t = rows // T, rows % T
    want = oracle.block_topk(scores[h, t][None], case.max_blocks, 16)[:, 0]
    assert torch.equal(got[t, h], want)


def _sets_differ_beyond_near_ties(got, want, ref_rows, tau):
    """Rows (of [n, k] selections and [n, W] oracle scores) whose selected
    sets differ, and those of them where some block of the symmetric
    difference is not within tau of the oracle's k-th selected score."""
    differ = bad = 0
    for i in range(got.shape[0]):
        a = set(int(x) for x in got[i] if x >= 0)
        b = set(int(x) for x in want[i] if x >= 0)
        if a == b:
            continue
        differ += 1
        kth = min(float(ref_rows[i, x]) for x in b)
        if any(abs(float(ref_rows[i, x]) - kth) > tau for x in a ^ b):
            bad += 1
    return differ, bad


@pytest.mark.parametrize("c", range(len(synth.CONFIG_NAMES)), ids=synth.CONFIG_NAMES)
def test_pipeline_against_oracle_scores(c, dev):
    # GPU scores -> GPU top-k against oracle scores -> oracle top-k, on every
    # row of the decode batches and on the stratified full rows of the
    # prefill workloads (the rows the score parity test compares): the sets
    # may differ only where the oracle scores tie within the score tolerance
    # of the k-th one, and on at most 1% of the rows.
    from test_parity_gpu import FULL_SIZE_ROWS, NEAR_TIE_ROW_FRACTION, oracle_out, oracle_rows
    case = synth.config_case(c)
    log(f"topk pipeline {case.name}")
    scores = run_gpu(case, dev)
    Hq, T, W = scores.shape
    got_all = gpu_topk(scores, dev, case.max_blocks, 16)
    if T <= 256:
        ref = oracle_out(case)
        rows = [(h, t) for t in range(T) for h in range(Hq)]
        ref_rows = ref.permute(1, 0, 2).reshape(T * Hq, W)
    else:
        rows, ref_rows = oracle_rows(case, FULL_SIZE_ROWS, 99 + c)
    hs = torch.tensor([h for h, _ in rows])
    ts = torch.tensor([t for _, t in rows])
    got = got_all[ts, hs]
    want = oracle.block_topk(ref_rows[None].contiguous(), case.max_blocks, 16)[:, 0]
    fin = torch.isfinite(ref_rows) & (ref_rows.abs() < 1e28)
    M = float(ref_rows[fin].abs().max()) if fin.any() else 0.0
    tau = TOL[case.key_dtype_name()] * M
    differ, bad = _sets_differ_beyond_near_ties(got, want, ref_rows, tau)
    log(f"topk pipeline {case.name}: {len(rows)} rows, {differ} near-tie rows, {bad} beyond")
    assert bad == 0, f"{case.name}: {bad} rows differ beyond near ties"
    assert differ <= NEAR_TIE_ROW_FRACTION * len(rows), (differ, len(rows))
