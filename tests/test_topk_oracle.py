"""Pins of the oracle's top-k block selection (CPU only).

The selection follows the follow-on stage the pages describe after the block
score (the notes "MiniMax Sparse Attention: paper algorithm and code",
section 4.7 "Top-k Block Selection",
section 5.3 "Top-k" with the sparse_topk_select contract, section 6.1
"Exp-free Top-k"): per (t, h) row, the k best blocks among beta < num_valid
whose score is above -inf, ties to the lower block index (a reading: the pages
leave the tie order open), emitted in ascending block order with a -1 tail.

The oracle sorts; the pins below do not.  The brute force ranks every
candidate by counting the candidates that beat it, which shares no step with
a sort, and the constructed cases fix the rules one at a time.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
import synth

NINF = float("-inf")


def rank_brute(scores: np.ndarray, num_valid: int, k: int) -> np.ndarray:
    """out[t, h, :] by counting: a candidate is selected iff fewer than k
    candidates have a higher score, or an equal score and a lower index."""
    Hq, T, W = scores.shape
    out = np.full((T, Hq, k), -1, dtype=np.int32)
    idx = np.arange(num_valid)
    for h in range(Hq):
        for t in range(T):
            row = scores[h, t, :num_valid].astype(np.float64)
            cand = row > NINF                    # False for -inf and NaN
            beats = cand[None, :] & ((row[None, :] > row[:, None]) |
                                     ((row[None, :] == row[:, None]) &
                                      (idx[None, :] < idx[:, None])))
            rank = beats.sum(axis=1)
            chosen = idx[cand & (rank < k)]      # ascending by construction
            out[t, h, :len(chosen)] = chosen
    return out


def random_scores(rng, Hq, T, W, tie_pool=True):
    return synth.score_rows(int(rng.integers(1 << 30)), Hq, T, W, ties=tie_pool).numpy()


@pytest.mark.parametrize("W", [1, 16, 48, 257])
@pytest.mark.parametrize("k", [1, 16, 64])
def test_matches_rank_counting_brute_force(W, k):
    rng = np.random.default_rng(1000 + 7 * W + k)
    for Hq, T in ((1, 1), (3, 5)):
        s = random_scores(rng, Hq, T, W)
        for nv in sorted({0, W // 2, W}):
            got = oracle.block_topk(torch.from_numpy(s), num_valid=nv, k=k).numpy()
            assert np.array_equal(got, rank_brute(s, nv, k)), (W, k, Hq, T, nv)


def test_structure_invariants():
    rng = np.random.default_rng(7)
    s = random_scores(rng, 4, 6, 200, tie_pool=False)
    k = 16
    got = oracle.block_topk(torch.from_numpy(s), k=k).numpy()
    for t in range(6):
        for h in range(4):
            row, sel = s[h, t], got[t, h]
            m = int((sel >= 0).sum())
            ncand = int((row > NINF).sum())
            assert m == min(k, ncand)
            assert np.all(sel[m:] == -1) and np.all(np.diff(sel[:m]) > 0)
            chosen = row[sel[:m]]
            rest = np.delete(row, sel[:m])
            rest = rest[rest > NINF]
            if m and rest.size:
                assert chosen.min() >= rest.max()


def test_constructed_cases():
    def one(row, k=4, nv=None):
        s = torch.tensor([[row]], dtype=torch.float32)
        return oracle.block_topk(s, num_valid=nv, k=k)[0, 0].tolist()

    # ties at the threshold go to the lower indices; output is index order
    assert one([5.0, 1.0, 5.0, 5.0, 5.0, 9.0], k=3) == [0, 2, 5]
    # fewer candidates than k: all of them, then -1
    assert one([NINF, 2.0, NINF, -7.0], k=4) == [1, 3, -1, -1]
    # an all -inf row selects nothing
    assert one([NINF] * 5, k=2) == [-1, -1]
    # NaN is never a candidate
    assert one([float("nan"), 1.0, float("nan")], k=3) == [1, -1, -1]
    # num_valid cuts the row before selection
    assert one([1.0, 2.0, 3.0, 4.0], k=2, nv=2) == [0, 1]
    assert one([1.0, 2.0, 3.0, 4.0], k=2, nv=0) == [-1, -1]
    # forced blocks (local_mask constants) win over any finite score; the
    # 1e30 init blocks before the 1e29 local window
    assert one([3e28, 1e30, -1.0, 1e29, 1e29, 5.0], k=3) == [1, 3, 4]
    assert one([1e29, 1e30, 1e29, 1e29, 7.0], k=2) == [0, 1]
    # k = 1 picks the maximum, the first one on a tie
    assert one([0.5, 2.5, 2.5], k=1) == [1]


def test_exp_free_selection_is_invariant_under_increasing_maps():
    # Selecting on raw scores equals selecting on exp(s - max) / sum (section
    # 6.1): any strictly increasing map keeps the order, hence the set.
    rng = np.random.default_rng(11)
    s = (rng.permutation(4 * 3 * 90).reshape(4, 3, 90) * 0.01).astype(np.float32)
    s[rng.random(s.shape) < 0.1] = NINF
    e = np.exp(s.astype(np.float64) - np.nanmax(np.where(s > NINF, s, np.nan), axis=2,
                                                   keepdims=True))
    e = (e / e.sum(axis=2, keepdims=True)).astype(np.float32)
    e[s == NINF] = NINF
    assert np.unique(s[s > NINF]).size == (s > NINF).sum()   # no ties to begin with
    for k in (1, 16, 64):
        a = oracle.block_topk(torch.from_numpy(s), k=k)
        b = oracle.block_topk(torch.from_numpy(e), k=k)
        assert torch.equal(a, b)


def test_contract_violations():
    s = torch.zeros(2, 3, 8)
    for kw in ({"k": 0}, {"k": 65}, {"num_valid": 9}, {"num_valid": -1}):
        with pytest.raises(ValueError):
            oracle.block_topk(s, **kw)
    # empty shapes are fine
    assert oracle.block_topk(torch.zeros(0, 3, 8)).shape == (3, 0, 16)
    assert oracle.block_topk(torch.zeros(2, 0, 8)).shape == (0, 2, 16)
    assert (oracle.block_topk(torch.zeros(2, 3, 0)) == -1).all()


MUTANTS = {
    "ties_to_higher_index": ("return (u->b > v->b) - (u->b < v->b);",
                             "return (u->b < v->b) - (u->b > v->b);"),
    "lowest_scores": ("  if (u->s > v->s) return -1;\n  if (u->s < v->s) return 1;",
                      "  if (u->s > v->s) return 1;\n  if (u->s < v->s) return -1;"),
    "neg_inf_kept": ("if (row[b] > -INFINITY) {", "if (row[b] >= -INFINITY) {"),
    "score_order_output": ("      qsort(sel, (size_t)m, sizeof(int32_t), orc_index_order);\n", ""),
    "num_valid_ignored": ("for (int64_t b = 0; b < num_valid; ++b) {",
                          "for (int64_t b = 0; b < W; ++b) {"),
    "row_index_transposed": ("const float* row = scores + (h * T + t) * W;",
                             "const float* row = scores + (t * Hq + h) * W;"),
}


def _agrees(lib) -> bool:
    rng = np.random.default_rng(5)
    for W, k in ((16, 4), (48, 16), (257, 16)):
        s = random_scores(rng, 3, 5, W)
        for nv in (W // 2, W):
            got = oracle.block_topk(torch.from_numpy(s), num_valid=nv, k=k, lib=lib).numpy()
            if not np.array_equal(got, rank_brute(s, nv, k)):
                return False
    return True


def test_unmutated_topk_agrees():
    assert _agrees(oracle.load())


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_topk_mutant_is_caught(mutant):
    old, new = MUTANTS[mutant]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    d = tempfile.mkdtemp()
    try:
        path = os.path.join(d, "mutant.c")
        open(path, "w").write(src.replace(old, new))
        so = os.path.join(d, "libmutant.so")
        subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-pthread", "-o", so, path,
                               "-lm"])
        assert not _agrees(oracle.load(so)), f"mutant {mutant} slipped through the pins"
    finally:
        shutil.rmtree(d, ignore_errors=True)
