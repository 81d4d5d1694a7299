"""Concurrent callers: host threads, each on its own stream, calling the C-ABI
entry points at the same time (ctypes releases the interpreter lock during a
call, so the calls overlap on the host and their kernels on the GPU).

The library keeps no device memory and no state between calls except the
per-device workgroup slot count, filled on first use; every call's output
must equal the same call made alone afterwards, bit for bit.  The concurrent
calls come first, so in a fresh process the threads also fill the slot
count at the same time.
"""
import sys
import threading

import pytest
import torch

import oracle
import synth
from compare import check
from test_parity_gpu import run_gpu, to_device, tol_of

pytestmark = pytest.mark.gpu

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


def _call(case, d, out, family, stream):
    import block_max_qk_amd as m
    if case.q_mx_scale is not None:
        m.msa_index_score_mxfp4(d["query"], d["q_mx"], d["key"], d["k_mx"], d["start_loc"],
                                d["block_table"], d["cu_seqlens_q"], d["kv_len"], case.layout,
                                case.sparse_mode, case.init_blocks, case.local_blocks, out,
                                case.max_blocks, local_mode=case.local_mode, family=family,
                                stream=stream)
    else:
        m.msa_index_score(d["query"], d["key"], d["start_loc"], d["block_table"], d["scale"],
                          d["cu_seqlens_q"], d["kv_len"], case.layout, case.sparse_mode,
                          case.init_blocks, case.local_blocks, out, case.max_blocks,
                          family=family, local_mode=case.local_mode, stream=stream)


@pytest.mark.parametrize("family", [-1, 0, 1])
def test_threads_on_streams_match_alone(family, dev):
    import block_max_qk_amd as m
    cases = {c.name: c for c in synth.edge_cases()}
    work = []
    for name in CASES:
        case = cases[name]
        d = to_device(case, dev)
        W = m.msa_index_score_out_width(case.max_blocks)
        outs = [torch.full((case.Hq, case.T, W), float("nan"), device=dev) for _ in range(4)]
        work.append((name, case, d, outs, torch.cuda.Stream(device=dev)))
    torch.cuda.synchronize()
    log(f"concurrency family={family}: {len(work)} threads x 4 calls")

    errors = []
    start = threading.Barrier(len(work))

    def run(item):
        name, case, d, outs, s = item
        try:
            start.wait()
            with torch.cuda.stream(s):
                for o in outs:
                    _call(case, d, o, family, s)
        except Exception as e:          # reported below, with the case
            errors.append((name, repr(e)))

    threads = [threading.Thread(target=run, args=(w,)) for w in work]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for name, case, d, outs, _ in work:
        alone = run_gpu(case, dev, family)
        assert check(oracle.index_score_case(case), alone, tol_of(case))["ok"], name
        for i, o in enumerate(outs):
            assert torch.equal(o.cpu().view(torch.int32), alone.view(torch.int32)), (name, i)
