"""GPU parity at addresses past 32-bit offsets.

The header's size limits let a caller pass key caches of more than 4 GiB and
outputs of more than 2^31 elements; the kernels index the block bases, the
packed-key offsets and the output rows with 64-bit integers.  These cases put
every such offset past 2^32 bytes (2^31 elements and more), through both
kernel families:

* paged keys (bf16 BBND, int8 BNBD with its scales, fp8 BBND, MXFP4 BBND with
  its scales) whose pages sit around the 4 GiB mark of a larger cache;
* packed keys (bf16, int8, MXFP4) whose requests follow a 4 GiB key segment;
* an output of 8 x 20 x 2^24 float32 (10.7 GB, the largest output width), the
  local_mask windows of two requests at its last columns, and the top-k
  selection over its full rows;
* two requests past a million keys (a decode token and a speculative step),
  compared whole, with the top-k selection on their ~12k-block rows;
* a 6144-token prefill at the end of a million-key context (8192-block rows),
  bf16 and MXFP4, compared on stratified whole rows.

The far inputs are the small cases of tests/far.py placed so that the result
is unchanged (checked with the oracle on the CPU in test_far_cpu.py), so the
expected output is the oracle's on the small case.
"""
import sys

import pytest
import torch

import far
import oracle
from compare import TOL, check, compare_values
from test_parity_gpu import tol_of

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


def launch(case, d, family, dev):
    import block_max_qk_amd as m
    W = m.msa_index_score_out_width(case.max_blocks)
    out = torch.full((case.Hq, case.T, W), 12345.0, dtype=torch.float32, device=dev)
    if case.q_mx_scale is not None:
        m.msa_index_score_mxfp4(d["query"], d["q_mx"], d["key"], d["k_mx"], d["start_loc"],
                                d["block_table"], d["cu_seqlens_q"], d["kv_len"], case.layout,
                                case.sparse_mode, case.init_blocks, case.local_blocks, out,
                                case.max_blocks, local_mode=case.local_mode, family=family)
    else:
        m.msa_index_score(d["query"], d["key"], d["start_loc"], d["block_table"], d["scale"],
                          d["cu_seqlens_q"], d["kv_len"], case.layout, case.sparse_mode,
                          case.init_blocks, case.local_blocks, out, case.max_blocks,
                          family=family, local_mode=case.local_mode)
    torch.cuda.synchronize()
    return out


_REF = {}


def _ref(case):
    if case.name not in _REF:
        _REF[case.name] = oracle.index_score_case(case)
    return _REF[case.name]


@pytest.mark.parametrize("family", [0, 1])
@pytest.mark.parametrize("name", [p[0] for p in far.PAGED])
def test_far_pages(name, family, dev):
    case = far.paged_case(name)
    ref = _ref(case)
    d = far.far_paged(case, dev)
    log(f"[gpu] far pages {name} family={family}: pages {d['offset']}.. of a "
        f"{d['key_bytes'] / 2**30:.2f} GiB cache")
    got = launch(case, d, family, dev).cpu()
    del d
    torch.cuda.empty_cache()
    r = check(ref, got, tol_of(case))
    assert r["ok"], r


@pytest.mark.parametrize("family", [0, 1])
@pytest.mark.parametrize("name", [p[0] for p in far.PACKED])
def test_far_packed_keys(name, family, dev):
    case = far.packed_case(name)
    ref = _ref(case)
    d = far.far_tnd(case, dev)
    log(f"[gpu] far packed keys {name} family={family}: requests after a "
        f"{d['offset']}-token segment, {d['key_bytes'] / 2**30:.2f} GiB of keys")
    got = launch(case, d, family, dev).cpu()
    del d
    torch.cuda.empty_cache()
    r = check(ref, got, tol_of(case))
    assert r["ok"], r


@pytest.fixture(scope="module")
def far_out():
    # the oracle's [8, 20, 2^24] output (10.7 GB of host memory), for both
    # families, released after them
    case = far.far_output_case()
    box = [case, oracle.index_score_case(case)]
    yield box
    box.clear()


@pytest.mark.parametrize("family", [0, 1])
def test_far_output_and_topk(family, dev, far_out):
    import block_max_qk_amd as m
    from test_topk_gpu import _sets_differ_beyond_near_ties
    case, ref = far_out
    Hq, T, W = ref.shape
    log(f"[gpu] far output family={family}: [{Hq}, {T}, {W}] float32, "
        f"{Hq * T * W * 4 / 2**30:.1f} GiB")
    d = {k: (None if v is None else v.to(dev)) for k, v in dict(
        query=case.query, key=case.key, start_loc=case.start_loc, block_table=None,
        scale=None, cu_seqlens_q=case.cu_seqlens_q, kv_len=case.kv_len).items()}
    out = launch(case, d, family, dev)
    tol = TOL["bf16"]
    for h in range(Hq):                                  # one head (1.3 GB) at a time
        r = compare_values(ref[h], out[h].cpu(), tol)
        assert r["ok"], (h, r)
    # every local_mask entry at the far columns, and the top-k sets over the
    # full rows (num_valid = W), against the oracle's selection on its scores
    assert torch.equal(out[:, :, W - 8:].cpu().view(torch.int32),
                       ref[:, :, W - 8:].view(torch.int32))
    k = 16
    sel = torch.full((T, Hq, k), -7, dtype=torch.int32, device=dev)
    m.msa_block_topk(out, W, k, sel)
    torch.cuda.synchronize()
    del out
    torch.cuda.empty_cache()
    want = oracle.block_topk(ref, W, k)                  # [T, Hq, k]
    got = sel.cpu()
    rows_ref = ref.reshape(Hq * T, W)
    g = got.permute(1, 0, 2).reshape(Hq * T, k)
    w = want.permute(1, 0, 2).reshape(Hq * T, k)
    fin = torch.isfinite(ref[:, :, :64]) & (ref[:, :, :64].abs() < 1e28)
    tau = tol * float(ref[:, :, :64][fin].abs().max())
    differ, bad = _sets_differ_beyond_near_ties(g, w, rows_ref, tau)
    log(f"[gpu] far output top-k: {Hq * T} rows, {differ} near-tie rows, {bad} beyond")
    assert bad == 0 and differ <= 2


@pytest.fixture(scope="module")
def long_ctx():
    case = far.long_context_case()
    return case, oracle.index_score_case(case)


@pytest.mark.parametrize("family", [0, 1])
def test_long_context_and_topk(family, dev, long_ctx):
    import block_max_qk_amd as m
    from test_parity_gpu import run_gpu, to_device
    from test_topk_gpu import _sets_differ_beyond_near_ties
    case, ref = long_ctx
    Hq, T, W = ref.shape
    log(f"[gpu] long context family={family}: kv_len {case.kv_len.tolist()}, [{Hq}, {T}, {W}]")
    got = run_gpu(case, dev, family)
    r = check(ref, got, tol_of(case))
    assert r["ok"], r
    # top-k on the GPU scores against the oracle's selection on its own
    k = 16
    sel = torch.full((T, Hq, k), -7, dtype=torch.int32, device=dev)
    m.msa_block_topk(got.to(dev), case.max_blocks, k, sel)
    torch.cuda.synchronize()
    want = oracle.block_topk(ref, case.max_blocks, k)
    g = sel.cpu().permute(1, 0, 2).reshape(Hq * T, k)
    w = want.permute(1, 0, 2).reshape(Hq * T, k)
    fin = torch.isfinite(ref) & (ref.abs() < 1e28)
    tau = tol_of(case) * float(ref[fin].abs().max())
    differ, bad = _sets_differ_beyond_near_ties(g, w, ref.reshape(Hq * T, W), tau)
    log(f"[gpu] long context top-k: {Hq * T} rows, {differ} near-tie rows, {bad} beyond")
    assert bad == 0 and differ <= 2


_LONG = {}


@pytest.mark.parametrize("family", [0, 1])
@pytest.mark.parametrize("qdtype", ["bf16", "mxfp4"])
def test_long_prefill(qdtype, family, dev):
    from test_parity_gpu import assert_rows_match, gpu_rows, oracle_rows, run_gpu
    if qdtype not in _LONG:
        _LONG.clear()                              # one case's inputs held at a time
        _LONG[qdtype] = far.long_prefill_case(qdtype)
    case = _LONG[qdtype]
    log(f"[gpu] long prefill {qdtype} family={family}: q {case.T} tokens, "
        f"kv_len {case.kv_len.tolist()}")
    rows, ref = oracle_rows(case, 64, 8501)      # cached for the second family
    got = gpu_rows(run_gpu(case, dev, family), rows)
    assert_rows_match(ref, got, tol_of(case), f"long prefill family={family}")
