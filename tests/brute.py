"""Vectorised brute force for the block score, used only to pin the oracle.

It follows the block-selection sketch of the DSA forward-path notes (section
3, from token scores to block selection): full token scores, ``masked_fill``
of every invisible position with -inf, ``reshape`` into blocks of P tokens and
``amax`` over each block; then the local_mask constants of the msa_index_score
guide (section 二), with the window at start_loc or, per query, at each token's
own block (the paper's local block, MSA notes section 4.7).  Inputs are decoded with torch's own ``.to(float64)`` and
products are taken with torch matmul, so it shares nothing with the C oracle.
"""
import torch


def _round16(n):
    n = max(int(n), 1)
    return (n + 15) // 16 * 16


def _e2m1_as_e4m3fn(nib: torch.Tensor) -> torch.Tensor:
    """float64 values of E2M1 codes through torch's e4m3fn decoder: an E2M1
    code (sign s, exponent e, fraction f; bias 1) is the e4m3fn code (s,
    e + 6, 4 f) (bias 7); its subnormal 0.5 (e = 0, f = 1) is e4m3fn (0, 6,
    0) and its zero is zero."""
    nib = nib.to(torch.int32)
    s, e, f = (nib >> 3) & 1, (nib >> 1) & 3, nib & 1
    code = torch.where(e > 0, (e + 6) << 3 | (f << 2), torch.where(f > 0, 6 << 3, 0))
    code = code | (s << 7)
    return code.to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)


def decode_mxfp4(vals: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """Packed E2M1 [..., D/2] (even element in the low nibble) with E8M0
    group scales [..., D/32] -> float64 [..., D]; scales via torch's e8m0."""
    lo, hi = vals & 15, vals >> 4
    nib = torch.stack([lo, hi], dim=-1).reshape(*vals.shape[:-1], vals.shape[-1] * 2)
    x = _e2m1_as_e4m3fn(nib)
    sc = scales.view(torch.float8_e8m0fnu).to(torch.float64)
    return x * sc.repeat_interleave(32, dim=-1)


def _query(case, t0, t1):
    if case.query.dtype == torch.uint8:
        return decode_mxfp4(case.query[t0:t1], case.q_mx_scale[t0:t1])
    return case.query[t0:t1].to(torch.float64)


def request_keys(case, b):
    """Dequantised keys k~ of request b as float64 [L, Hkv, D]."""
    P = case.block_size
    L = int(case.kv_len[b])
    nb = -(-L // P)
    mx = case.key.dtype == torch.uint8
    if case.layout == "TND":
        off = int(case.kv_len[:b].sum())
        k = (decode_mxfp4(case.key[off:off + L], case.k_mx_scale[off:off + L]) if mx
             else case.key[off:off + L].to(torch.float64))
        s = case.scale[off:off + L].to(torch.float64) if case.scale is not None else None
    else:
        pages = case.block_table[b, :nb].long()
        if mx:
            kp = decode_mxfp4(case.key[pages], case.k_mx_scale[pages])
        else:
            kp = case.key[pages].to(torch.float64)          # [nb, P, Hkv, D] or [nb, Hkv, P, D]
        if case.layout == "BNBD":
            kp = kp.permute(0, 2, 1, 3)
        k = kp.reshape(nb * P, kp.shape[2], kp.shape[3])[:L]
        s = None
        if case.scale is not None:
            s = case.scale[pages].to(torch.float64).permute(0, 2, 1).reshape(nb * P, -1)[:L]
    if s is not None:
        k = k * s[:, :, None]          # k~ = cast(k) * scale, exact in binary64
    return k


def brute_force(case) -> torch.Tensor:
    P = case.block_size
    Hq, T = case.Hq, case.T
    W = _round16(case.max_blocks)
    g = Hq // case.Hkv
    out = torch.full((Hq, T, W), float("-inf"), dtype=torch.float64)
    cu = case.cu_seqlens_q.long()
    for b in range(case.batch):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        Lq, L = t1 - t0, int(case.kv_len[b])
        if Lq == 0 or L == 0:
            continue
        nb = -(-L // P)
        q = _query(case, t0, t1)                              # [Lq, Hq, D]
        k = request_keys(case, b)                             # [L, Hkv, D]
        kh = k.repeat_interleave(g, dim=1)                    # [L, Hq, D]
        s = torch.matmul(q.permute(1, 0, 2), kh.permute(1, 2, 0))   # [Hq, Lq, L]
        i = torch.arange(Lq)[:, None]
        j = torch.arange(L)[None, :]
        qpos = (L - Lq + i) if case.sparse_mode == 3 else torch.full_like(i, L - 1)
        visible = (j <= qpos) & (j < L)
        s = s.masked_fill(~visible[None], float("-inf"))
        pad = torch.full((Hq, Lq, nb * P - L), float("-inf"), dtype=torch.float64)
        blocks = torch.cat([s, pad], dim=2).reshape(Hq, Lq, nb, P).amax(-1)
        out[:, t0:t1, :nb] = blocks
        if case.init_blocks > 0 or case.local_blocks > 0:
            out[:, t0:t1, :case.init_blocks] = 1e30
            if getattr(case, "local_mode", 0) == 0:
                st = int(case.start_loc[b])
                lo = max(0, st + 1 - case.local_blocks)
                if st >= lo:
                    out[:, t0:t1, lo:st + 1] = 1e29
            else:
                # each token's own block: the floor of its position over P
                # (negative before position 0, which leaves no window)
                anchor = torch.div(L - Lq + torch.arange(Lq), P, rounding_mode="floor")
                col = torch.arange(W)[None, :]
                win = (col <= anchor[:, None]) & (col >= anchor[:, None] + 1 - case.local_blocks)
                out[:, t0:t1, :] = torch.where(win[None], torch.tensor(1e29, dtype=torch.float64),
                                               out[:, t0:t1, :])
    return out.to(torch.float32)
