"""Inputs past 32-bit offsets, built from small seeded cases.

Each builder places a small case's inputs so that the operator's result is
unchanged while the addresses it reads lie more than 4 GiB (2^31 elements and
more) into the key buffers:

* ``far_paged``: the case's pages move to page numbers around the 4 GiB mark
  of a larger key cache (the block table renumbered by the same offset); the
  pages in front of them are never referenced and hold the byte 0xFF (NaN in
  the float formats and in E8M0, -6 in E2M1, -1 in int8).
* ``far_tnd``: a packed-key case whose first request has no query tokens gets
  a key segment of more than 4 GiB for that request (0xFF bytes); the other
  requests' keys follow it unchanged.  The case must already carry the table
  width the longer segment needs (``tnd_far_blocks``).

No arithmetic of the operator lives here: the builders copy and renumber.
"""
import torch

FAR = 1 << 32          # byte offset the far placements reach past


def _ceil_div(a, b):
    return -(-a // b)


def _blank(shape, dtype, device):
    t = torch.empty(shape, dtype=dtype, device=device)
    t.view(torch.uint8).fill_(0xFF)
    return t


def page_bytes(case) -> int:
    ks = case.key_storage
    return ks[0].numel() * ks.element_size()


def far_paged(case, device) -> dict:
    """Operator inputs of a paged case (no dim0 gap) with its pages moved to
    page numbers OFF .. OFF + NP - 1, OFF chosen so that the pages straddle
    the 4 GiB mark of the key cache.  Returns the inputs as ``to_device``
    does, plus ``offset`` and ``key_bytes`` (size of the whole key cache)."""
    assert case.layout in ("BBND", "BNBD") and not case.gap
    NP = case.key_storage.shape[0]
    off = _ceil_div(FAR, page_bytes(case)) - NP // 2
    key = _blank((off + NP,) + tuple(case.key_storage.shape[1:]), case.key_storage.dtype, device)
    key[off:] = case.key_storage.to(device)
    d = dict(query=case.query.to(device), key=key, start_loc=case.start_loc.to(device),
             block_table=(case.block_table + off).to(device),
             cu_seqlens_q=case.cu_seqlens_q.to(device), kv_len=case.kv_len.to(device),
             scale=None, q_mx=None, k_mx=None, offset=off,
             key_bytes=key.numel() * key.element_size())
    if case.scale is not None:            # int8: [NP, Hkv, P] by page number
        d["scale"] = _blank((off + NP,) + tuple(case.scale.shape[1:]), torch.float32, device)
        d["scale"][off:] = case.scale.to(device)
    if case.k_mx_scale is not None:       # MXFP4 key scales, by page number
        km = case.k_mx_scale
        d["k_mx"] = _blank((off + NP,) + tuple(km.shape[1:]), km.dtype, device)
        d["k_mx"][off:] = km.to(device)
        d["q_mx"] = case.q_mx_scale.to(device)
    return d


def tnd_far_tokens(token_bytes: int) -> int:
    """Length of a leading key segment that puts the next request's keys past
    4 GiB (and off a block boundary)."""
    return _ceil_div(FAR, token_bytes) + 77


def tnd_far_blocks(token_bytes: int) -> int:
    """The table width (MB) a packed-key batch with that segment needs."""
    return _ceil_div(tnd_far_tokens(token_bytes), 128)


def token_bytes(case) -> int:
    ks = case.key_storage
    return ks[0].numel() * ks.element_size()


def far_tnd(case, device) -> dict:
    """Operator inputs of a packed-key case whose request 0 has no query
    tokens and no keys, with request 0 given the leading key segment of
    ``tnd_far_tokens`` tokens instead."""
    assert case.layout == "TND"
    assert int(case.cu_seqlens_q[1]) == 0 and int(case.kv_len[0]) == 0
    k0 = tnd_far_tokens(token_bytes(case))
    assert case.max_blocks >= _ceil_div(k0, 128)
    T2 = case.key_storage.shape[0]
    key = _blank((k0 + T2,) + tuple(case.key_storage.shape[1:]), case.key_storage.dtype, device)
    key[k0:] = case.key_storage.to(device)
    kv = case.kv_len.clone()
    kv[0] = k0
    d = dict(query=case.query.to(device), key=key, start_loc=case.start_loc.to(device),
             block_table=None, cu_seqlens_q=case.cu_seqlens_q.to(device), kv_len=kv.to(device),
             scale=None, q_mx=None, k_mx=None, offset=k0,
             key_bytes=key.numel() * key.element_size())
    if case.scale is not None:            # int8: [T2, Hkv]
        d["scale"] = _blank((k0 + T2,) + tuple(case.scale.shape[1:]), torch.float32, device)
        d["scale"][k0:] = case.scale.to(device)
    if case.k_mx_scale is not None:       # MXFP4: [T2, Hkv, D/32]
        km = case.k_mx_scale
        d["k_mx"] = _blank((k0 + T2,) + tuple(km.shape[1:]), km.dtype, device)
        d["k_mx"][k0:] = km.to(device)
        d["q_mx"] = case.q_mx_scale.to(device)
    return d


def _token_bytes_of(kdtype: str, Hkv: int, D: int = 128) -> int:
    """Bytes of one packed key token: Hkv rows of D elements (MXFP4: D / 2)."""
    return Hkv * {"bf16": 2 * D, "f16": 2 * D, "i8": D, "f8e4m3": D, "mxfp4": D // 2}[kdtype]


# (query type, key type, layout) of the far-page and far-packed-key cases
PAGED = [("far_bbnd_bf16", "bf16", "bf16", "BBND"), ("far_bnbd_i8", "f16", "i8", "BNBD"),
         ("far_bbnd_f8", "f8e4m3", "f8e4m3", "BBND"), ("far_bbnd_mx", "mxfp4", "mxfp4", "BBND")]
PACKED = [("far_tnd_bf16", "bf16", "bf16"), ("far_tnd_i8", "f16", "i8"),
          ("far_tnd_mx", "mxfp4", "mxfp4")]
FAR_OUT_MB = (1 << 24) - 5       # output width 2^24, the largest the operator takes


def paged_case(name: str):
    import synth
    i = [p[0] for p in PAGED].index(name)
    _, qd, kd, layout = PAGED[i]
    # one-token decode, a long and a short prefill, an empty request and a
    # request one past a block boundary; GQA 4
    return synth.make_case(name, 8100 + i, q_lens=[1, 5, 40, 0, 3],
                           kv_lens=[700, 1000, 2000, 300, 129], Hq=8, Hkv=2, qdtype=qd,
                           kdtype=kd, layout=layout, init_blocks=1, local_blocks=2,
                           extra_pages=3)


def packed_case(name: str):
    """Request 0 has no tokens and no keys; far_tnd gives it the 4 GiB
    segment.  MB is the width that segment needs."""
    import synth
    i = [p[0] for p in PACKED].index(name)
    _, qd, kd = PACKED[i]
    kd_bytes = _token_bytes_of(kd, 2)
    return synth.make_case(name, 8200 + i, q_lens=[0, 5, 40, 3], kv_lens=[0, 1000, 2000, 129],
                           Hq=8, Hkv=2, qdtype=qd, kdtype=kd, layout="TND",
                           MB=tnd_far_blocks(kd_bytes), init_blocks=1, local_blocks=2)


def far_output_case():
    """An output of 8 x 20 x 2^24 float32 (2.7e9 elements, 10.7 GB): rows
    h * 20 + t >= 128 start past element 2^31.  Two requests anchor their
    local_mask window at the last columns."""
    import synth
    W = 1 << 24
    return synth.make_case("far_out_tnd_bf16", 8300, q_lens=[5, 12, 3],
                           kv_lens=[700, 5000, 130], Hq=8, Hkv=2, qdtype="bf16", layout="TND",
                           MB=FAR_OUT_MB, init_blocks=1, local_blocks=3,
                           start_loc=[W - 6, 2, W - 1])


def long_context_case():
    """Two requests past a million keys (8193 and 11719 blocks): a one-token
    decode and a three-token speculative step, 8 heads over one KV head, bf16
    keys in 19912 pages (1.2 GB) behind a random table.  Each request's work
    list and output row run to ~12k blocks, and the top-k selection on its
    rows takes the search over rows longer than 2048 blocks."""
    import synth
    return synth.make_case("long_ctx_bbnd_bf16", 8400, q_lens=[1, 3],
                           kv_lens=[(1 << 20) + 77, 1_500_000], Hq=8, Hkv=1, qdtype="bf16",
                           layout="BBND", init_blocks=1, local_blocks=2)


def long_prefill_case(qdtype: str = "bf16"):
    """A prefill of 6144 tokens at the end of a 1,048,576-key context (its
    rows span 8192 blocks, the causal diagonal at the last 48) and one of 100
    tokens over 200,000 keys; 8 heads over one KV head, bf16 (320 MB) or
    MXFP4 (80 MB and scales) packed keys, output 8 x 6244 x 8192 float32
    (1.6 GB)."""
    import synth
    return synth.make_case(f"long_prefill_tnd_{qdtype}", 8500 if qdtype == "bf16" else 8501,
                           q_lens=[6144, 100], kv_lens=[1 << 20, 200_000], Hq=8, Hkv=1,
                           qdtype=qdtype, layout="TND", init_blocks=1, local_blocks=2)
