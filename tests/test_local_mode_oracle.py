"""Pins of the oracle's per-query local window (CPU only).

The operator's local_mask forces 1e29 on a window of blocks that ends at the
request's start_loc (guide to msa_index_score, section 二).  The paper forces
instead each query's own block, b_local(i) = floor(i / B_k) (notes "MiniMax
Sparse Attention: paper algorithm and code", section 4.7, on the forced local
block, which notes that a request-wide window is not the same thing in a long
prefill).  With local_mode 1 the oracle ends the window at floor(pos / P),
pos = kv_len - L_q + i the token's position (a reading: the pages give the
formula in the query's own index).  Beyond the brute-force agreement over the
edge and random suites (tests/test_oracle_pins.py), these pins fix the mode
from the definition alone.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

P = 128


def positions(case):
    """(row t, request b, position) for every packed query token."""
    cu = case.cu_seqlens_q.tolist()
    kv = case.kv_len.tolist()
    out = []
    for b in range(case.batch):
        Lq = cu[b + 1] - cu[b]
        for i in range(Lq):
            out.append((cu[b] + i, b, kv[b] - Lq + i))
    return out


def with_mode(case, local_mode, init_blocks=None, local_blocks=None, start_loc=None):
    import dataclasses
    kw = {"local_mode": local_mode}
    if init_blocks is not None:
        kw["init_blocks"] = init_blocks
    if local_blocks is not None:
        kw["local_blocks"] = local_blocks
    if start_loc is not None:
        kw["start_loc"] = start_loc
    return dataclasses.replace(case, **kw)


@pytest.mark.parametrize("layout", ["BBND", "TND"])
def test_decode_rows_equal_a_last_block_start_loc(layout):
    # One query token per request sits at position kv_len - 1, so its own
    # block is the request's last block: the per-request window anchored
    # there must give the same output, entry for entry.
    c = synth.make_case("dec", 91, q_lens=[1] * 5, kv_lens=[1, 127, 128, 129, 700], Hq=8,
                        Hkv=2, qdtype="bf16", layout=layout, extra_pages=3, init_blocks=1,
                        local_blocks=2)
    last = torch.tensor([(int(k) - 1) // P for k in c.kv_len], dtype=torch.int32)
    a = oracle.index_score_case(with_mode(c, 1))
    b = oracle.index_score_case(with_mode(c, 0, start_loc=last))
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("mode", [3, 0])
def test_forced_entries_sit_on_each_tokens_block(mode):
    # init 0, local 1: the 1e29 entries of a row are exactly its own block
    # (none before position 0, none for an empty request).
    c = synth.make_case("perq", 92, q_lens=[300, 5, 10, 2], kv_lens=[556, 260, 6, 0],
                        Hq=4, Hkv=1, qdtype="f16", layout="BBND", extra_pages=2,
                        sparse_mode=mode, init_blocks=0, local_blocks=1, local_mode=1)
    out = oracle.index_score_case(c)
    forced = (out == 1e29)
    assert not (out == 1e30).any()
    for t, b, pos in positions(c):
        want = set()
        if int(c.kv_len[b]) > 0 and pos >= 0:
            want = {pos // P}
        for h in range(c.Hq):
            got = set(torch.nonzero(forced[h, t]).flatten().tolist())
            assert got == want, (t, b, pos, h, got, want)


def test_window_length_and_init_override():
    # local 3 covers the token's block and the two before it (clipped at 0);
    # it overrides the init block where they meet; start_loc is not read.
    c = synth.make_case("perq3", 93, q_lens=[260], kv_lens=[1000], Hq=2, Hkv=1,
                        qdtype="bf16", layout="TND", init_blocks=2, local_blocks=3,
                        local_mode=1, start_loc=[999])
    out = oracle.index_score_case(c)
    for t, b, pos in positions(c):
        a = pos // P
        for beta in range(out.shape[2]):
            v = float(out[0, t, beta])
            if max(0, a - 2) <= beta <= a:
                assert v == np.float32(1e29), (t, beta)
            elif beta < 2:
                assert v == np.float32(1e30), (t, beta)
            else:
                assert v < 1e28, (t, beta)


def test_top_k_keeps_every_tokens_own_block():
    # The point of the mode (paper, Equation (7)): with the local window no
    # wider than k, the top-k of every row holds the token's own block.
    c = synth.make_case("perqk", 94, q_lens=[200, 64], kv_lens=[3000, 1200], Hq=4, Hkv=2,
                        qdtype="bf16", layout="BBND", extra_pages=2, init_blocks=1,
                        local_blocks=4, local_mode=1)
    scores = oracle.index_score_case(c)
    sel = oracle.block_topk(scores, c.max_blocks, 16)
    for t, b, pos in positions(c):
        for h in range(c.Hq):
            assert pos // P in set(sel[t, h].tolist())
    # the per-request window (start_loc = first query token's block) does not
    # give that for the later tokens of a long prefill
    req = oracle.block_topk(oracle.index_score_case(with_mode(c, 0)), c.max_blocks, 16)
    missing = sum(pos // P not in set(req[t, 0].tolist()) for t, b, pos in positions(c))
    assert missing > 0
