"""The far placements of tests/far.py, checked on the CPU with the oracle.

Moving a paged case's pages to page numbers past the 4 GiB mark of a larger
cache (and renumbering the block table), or giving a packed-key case a
leading request with no query tokens and a 4 GiB key segment, must leave the
operator's result unchanged: the result depends on a page only through the
block table, and on a request only through its own keys.  The oracle run on
the far placement must therefore give the small case's output bit for bit.
This pins the GPU far-address tests' inputs (they compare the GPU on the far
placement with the oracle on the small case) and the oracle's own 64-bit
indexing.  Each case allocates 4.3 GB of host memory.
"""
import pytest
import torch

import far
import oracle


def _oracle_on(case, d):
    return oracle.index_score(
        query=d["query"], key=d["key"], layout=case.layout, start_loc=d["start_loc"],
        block_table=d["block_table"], scale=d["scale"], cu_seqlens_q=d["cu_seqlens_q"],
        kv_len=d["kv_len"], max_blocks=case.max_blocks, sparse_mode=case.sparse_mode,
        init_blocks=case.init_blocks, local_blocks=case.local_blocks,
        local_mode=case.local_mode, q_mx_scale=case.q_mx_scale, k_mx_scale=d["k_mx"])[0]


@pytest.mark.parametrize("name", ["far_bbnd_bf16", "far_bnbd_i8"])
def test_oracle_far_pages_unchanged(name):
    case = far.paged_case(name)
    ref = oracle.index_score_case(case)
    d = far.far_paged(case, "cpu")
    assert d["key_bytes"] > far.FAR
    # the case's pages straddle the 4 GiB mark
    lo = d["offset"] * far.page_bytes(case)
    assert lo < far.FAR < lo + case.key_storage.shape[0] * far.page_bytes(case)
    got = _oracle_on(case, d)
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))


@pytest.mark.parametrize("name", ["far_tnd_bf16", "far_tnd_i8"])
def test_oracle_far_packed_keys_unchanged(name):
    case = far.packed_case(name)
    ref = oracle.index_score_case(case)
    d = far.far_tnd(case, "cpu")
    assert d["offset"] * far.token_bytes(case) > far.FAR
    got = _oracle_on(case, d)
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))


def test_far_case_shapes():
    # the packed cases' table width is the one their leading segment needs,
    # and the far output passes 2^31 elements at the largest output width
    for name, _, kd in far.PACKED:
        c = far.packed_case(name)
        k0 = far.tnd_far_tokens(far.token_bytes(c))
        assert c.max_blocks == -(-k0 // 128)
        assert k0 % 128 != 0
    c = far.far_output_case()
    W = oracle.out_width(c.max_blocks)
    assert W == 1 << 24
    assert c.Hq * c.T * W > 2 ** 31
    assert (c.Hq - 1) * c.T * W > 2 ** 31     # the last head's rows all lie past it
