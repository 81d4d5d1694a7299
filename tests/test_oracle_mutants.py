"""The pins must catch plausible oracle mistakes (CPU only).

Each mutant is a one-line change to a copy of the oracle's C source (a dropped
term, an off-by-one, a wrong index or operand), compiled to a temporary
library.  The brute force, the decoders and the closed-form window must
disagree with every mutant somewhere.
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
from brute import brute_force

MUTANTS = {
    "window_off_by_one": ("if (jhi > qpos) jhi = qpos;", "if (jhi > qpos + 1) jhi = qpos + 1;"),
    "qpos_shift": ("? L - Lq + i : L - 1;", "? L - Lq + i - 1 : L - 1;"),
    "block_end_off_by_one": ("int64_t jhi = beta * a->P + a->P - 1;",
                             "int64_t jhi = beta * a->P + a->P;"),
    "gqa_modulo": ("int hk = h / g;", "int hk = h % a->Hkv;"),
    "dequant_dropped": ("if (a->k_dtype == ORC_I8) dot *= (double)a->scale[sidx];", ""),
    "bbnd_axes_swapped": ("*off = page * a->ks[0] + jj * a->ks[1] + (int64_t)hk * a->ks[2];",
                          "*off = page * a->ks[0] + jj * a->ks[2] + (int64_t)hk * a->ks[1];"),
    "tnd_offset_dropped": ("int64_t row = a->koff[b] + j;", "int64_t row = j;"),
    "local_value_swapped": ("v = 1e29f;", "v = 1e30f;"),
    "local_window_exclusive": ("if (beta >= lo && beta <= s) v = 1e29f;",
                               "if (beta >= lo && beta < s) v = 1e29f;"),
    "empty_kv_not_skipped": ("if (L == 0) return -INFINITY;", ""),
    "bf16_exponent": ("v = ldexp((double)(128 + f), e - 134);",
                      "v = ldexp((double)(128 + f), e - 133);"),
    "e4m3_nan_rule": ("if (e == 15 && f == 7)", "if (e == 15)"),
    "scale_index_token_major": ("*sidx = (page * a->Hkv + hk) * a->P + jj;",
                                "*sidx = (page * a->P + jj) * a->Hkv + hk;"),
    "init_after_local": ("    if (beta < a->init_blocks) v = 1e30f;\n", ""),
    # per-query local window
    "per_query_ignored": ("if (a->local_mode == 0) {", "if (1) {"),
    "per_query_block_end": ("s = pos >= 0 ? pos / a->P : -1;",
                            "s = pos >= 0 ? (pos + 1) / a->P : -1;"),
    "per_query_from_window_end": ("int64_t pos = L - Lq + i;",
                                  "int64_t pos = (a->sparse_mode == 3) ? L - Lq + i : L - 1;"),
    "per_query_negative_to_block0": ("s = pos >= 0 ? pos / a->P : -1;",
                                     "s = pos >= 0 ? pos / a->P : 0;"),
    # MXFP4
    "mx_nibble_order": ("[i >> 1] >> (4 * (i & 1))) & 15);", "[i >> 1] >> (4 * (~i & 1))) & 15);"),
    "mx_e2m1_subnormal": ("double v = e == 0 ? 0.5 * f :", "double v = e == 0 ? 1.0 * f :"),
    "mx_e8m0_bias": ("ldexp(1.0, (int)e - 127); }", "ldexp(1.0, (int)e - 128); }"),
    "mx_query_group": ("(int64_t)(a->D / 32) + d / 32]);", "(int64_t)(a->D / 32) + d / 64]);"),
    "mx_key_scale_bbnd_axes": ("return ((page * a->P + jj) * a->Hkv + hk) * groups;",
                               "return ((page * a->Hkv + hk) * a->P + jj) * groups;"),
    "mx_key_scale_dropped": ("if (a->k_dtype == ORC_MXFP4) kv *= orc_decode_e8m0(a->k_mx[mxr + d / 32]);",
                             ""),
}

CASE_NAMES = ["tiny_bbnd_f16", "mix_bbnd_bf16", "mix_bnbd_bf16", "mix_tnd_bf16",
              "mix_bbnd_i8", "mix_bnbd_i8", "mix_tnd_i8", "mix_bbnd_f8e4m3",
              "pad_tnd_kvlen0", "q_longer_than_kv", "init_local_overlap", "mode0_tnd",
              "gqa_g3_bbnd", "gqa_g40_bbnd", "dim0_gap2_bnbd_i8",
              "perq_prefill_tnd", "perq_mode0_bbnd", "perq_q_longer_than_kv",
              "mx_mix_bbnd", "mx_mix_bnbd_gap", "mx_prefill_tnd"]


@pytest.fixture(scope="module")
def cases():
    allc = {c.name: c for c in synth.edge_cases()}
    cs = [allc[n] for n in CASE_NAMES]
    return [(c, brute_force(c)) for c in cs]


def _agrees(lib, cases) -> bool:
    for c, want in cases:
        try:
            got = oracle.index_score_case(c, lib=lib)
        except ValueError:
            return False
        gb, wb = got.view(torch.int32), want.view(torch.int32)
        fin = torch.isfinite(want) & (want.abs() < 1e28)
        if not torch.equal(gb[~fin], wb[~fin]):
            return False
        d = (got[fin].double() - want[fin].double()).abs()
        ulp = torch.from_numpy(np.spacing(np.abs(want[fin].numpy()))).double()
        if bool((d > ulp).any()):
            return False
    for dt, n in ((torch.bfloat16, 65536), (torch.float8_e4m3fn, 256)):
        codes = torch.arange(n, dtype=torch.int32).to(torch.int16 if n > 256 else torch.uint8)
        codes = codes.view(dt)
        w = codes.to(torch.float64).numpy()
        g = oracle.decode(codes, lib=lib)
        if not np.array_equal(np.isnan(w), np.isnan(g)) or not np.array_equal(
                w[~np.isnan(w)], g[~np.isnan(g)]):
            return False
    # MXFP4 packing (a reading: the even element in the low nibble).  A swap
    # applied to query and key alike leaves every score unchanged, so the
    # order is pinned on the element decoder: byte 0x21 holds E2M1 codes 1
    # (0.5) then 2 (1.0).
    g = oracle.decode(torch.tensor([0x21, 0xF0], dtype=torch.uint8), lib=lib)
    if list(g[:4]) != [0.5, 1.0, 0.0, -6.0]:
        return False
    return True


def test_unmutated_oracle_agrees(cases):
    assert _agrees(oracle.load(), cases)


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, cases):
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
        lib = oracle.load(so)
        assert not _agrees(lib, cases), f"mutant {mutant} slipped through the pins"
    finally:
        shutil.rmtree(d, ignore_errors=True)
