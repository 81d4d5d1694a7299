"""The C-ABI entry points captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must give the eager launch's output bit for bit.

The library's calls are plain kernel launches on the caller's stream (no
memsets, copies or synchronisation), so a caller may capture them.  Each case
captures one call, then replays the graph three times with eager work of the
program between the replays (the output refilled with a poison value, an eager
call of the same entry on other inputs, a synchronisation) and compares every
replay with the eager result; the eager result itself is checked against the
oracle by the parity tests, and here once more for the small cases.
"""
import sys

import pytest
import torch

import oracle
import synth
from compare import check
from test_parity_gpu import run_gpu, to_device, tol_of

pytestmark = pytest.mark.gpu

# paged decode (bf16, int8 with scales), packed prefill, the MXFP4 entry on
# both kernel families, and a per-query window
CASES = ["mix_bbnd_bf16", "mix_bnbd_i8", "prefill_tnd_small", "prefill_bbnd_f8",
         "mx_mix_bbnd", "mx_prefill_tnd", "perq_prefill_tnd"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_max_qk_amd
    block_max_qk_amd.load_library()
    return torch.device("cuda:0")


def _call(case, d, out, family):
    import block_max_qk_amd as m
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


@pytest.mark.parametrize("family", [0, 1])
@pytest.mark.parametrize("name", CASES)
def test_graph_replay_matches_eager(name, family, dev):
    import block_max_qk_amd as m
    cases = {c.name: c for c in synth.edge_cases()}
    case = cases[name]
    log(f"graph replay {name} family={family}")
    eager = run_gpu(case, dev, family)
    assert check(oracle.index_score_case(case), eager, tol_of(case))["ok"], name

    d = to_device(case, dev)
    W = m.msa_index_score_out_width(case.max_blocks)
    out = torch.full((case.Hq, case.T, W), 12345.0, dtype=torch.float32, device=dev)
    # the other inputs of the eager call between replays: the query halved
    other = dict(d)
    other["query"] = d["query"].clone()
    if case.q_mx_scale is None:
        other["query"] = (other["query"].float() * 0.5).to(d["query"].dtype)
    other_out = torch.empty_like(out)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        _call(case, d, out, family)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for rep in range(3):
        out.fill_(float("nan"))
        _call(case, other, other_out, family)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu()
        assert torch.equal(got.view(torch.int32), eager.view(torch.int32)), (name, family, rep)


@pytest.mark.parametrize("k", [8, 16])
def test_graph_replay_topk(k, dev):
    import block_max_qk_amd as m
    scores = synth.score_rows(4711 + k, 4, 300, 512).to(dev)
    eager = torch.empty((300, 4, k), dtype=torch.int32, device=dev)
    m.msa_block_topk(scores, 500, k, eager)
    torch.cuda.synchronize()
    assert torch.equal(eager.cpu(), oracle.block_topk(scores.cpu(), 500, k))
    out = torch.empty_like(eager)
    other = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        m.msa_block_topk(scores, 500, k, out)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        out.fill_(-7)
        m.msa_block_topk(scores, 100, k, other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), eager.cpu()), (k, rep)
