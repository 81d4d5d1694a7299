"""Comparison rules between an expected score tensor and a computed one.

* -inf entries (no visible key, or padding) and the forced local_mask entries
  (1e30, 1e29) must match bit for bit;
* every other entry is finite and must satisfy |got - ref| <= tol * M with
  M = max |ref| over those finite entries (tol 1e-3 for fp16/bf16/int8 keys,
  2e-2 for fp8);
* the per-(h, t) top-k block sets (k = 16, ties to the lower block index) must
  agree, except for blocks whose expected score lies within tol * M of the
  expected k-th value (near ties), which are counted and reported.
"""
import torch

NEG_INF_BITS = -8388608          # 0xFF800000 as int32
INIT_BITS = 0x7149F2CA           # float32(1e30)
LOCAL_BITS = 0x6FA18F08          # float32(1e29)

TOL = {"f16": 1e-3, "bf16": 1e-3, "i8": 1e-3, "f8e4m3": 2e-2, "f8e5m2": 2e-2,
       # MXFP4: products of E2M1 values and power-of-two scales are exact, so
       # the only error is float32 summation over D = 128 terms, at most about
       # 128 * 2^-24 * sum|q_d k_d| (~6e-4 for N(0,1)-encoded rows, whose block
       # maxima are ~40)
       "mxfp4": 1e-4}


def _special(bits):
    return (bits == NEG_INF_BITS) | (bits == INIT_BITS) | (bits == LOCAL_BITS)


def compare_values(ref: torch.Tensor, got: torch.Tensor, tol: float) -> dict:
    assert ref.shape == got.shape, (ref.shape, got.shape)
    ref = ref.float().reshape(-1)
    got = got.float().reshape(-1).to(ref.device)
    rb, gb = ref.view(torch.int32), got.view(torch.int32)
    rs, gs = _special(rb), _special(gb)
    special_mismatch = int(((rs | gs) & (rb != gb)).sum())
    nan = int(torch.isnan(got).sum())
    fin = ~rs
    if bool(fin.any()):
        M = float(ref[fin].abs().max())
        err = (ref[fin].double() - got[fin].double()).abs()
        max_err = float(err.max())
    else:
        M, max_err = 0.0, 0.0
    ok = special_mismatch == 0 and nan == 0 and max_err <= tol * M
    return {"ok": ok, "special_mismatch": special_mismatch, "nan": nan, "max_abs_err": max_err,
            "M": M, "rel_err": (max_err / M if M > 0 else 0.0), "tol": tol,
            "n": int(ref.numel()), "n_finite": int(fin.sum())}


def _topk_mask(x: torch.Tensor, kk: torch.Tensor, k: int) -> torch.Tensor:
    """Bool mask of the top-kk[row] entries of each row (ties to lower index)."""
    order = torch.sort(x, dim=1, descending=True, stable=True).indices[:, :k]
    rank_ok = torch.arange(order.shape[1], device=x.device)[None, :] < kk[:, None]
    mask = torch.zeros_like(x, dtype=torch.bool)
    mask.scatter_(1, order, rank_ok)
    return mask


def compare_topk(ref: torch.Tensor, got: torch.Tensor, tau: float, k: int = 16) -> dict:
    """ref/got: [..., W] score rows."""
    W = ref.shape[-1]
    r = ref.float().reshape(-1, W)
    g = got.float().reshape(-1, W).to(r.device)
    if r.shape[0] == 0 or W == 0:
        return {"ok": True, "rows": 0, "near_tie_rows": 0, "bad_rows": 0, "k": k}
    kk = torch.clamp((r > float("-inf")).sum(1), max=min(k, W))
    mr = _topk_mask(r, kk, min(k, W))
    mg = _topk_mask(g, kk, min(k, W))
    diff = mr ^ mg
    rows = diff.any(1)
    kth = torch.gather(torch.sort(r, dim=1, descending=True, stable=True).values, 1,
                       torch.clamp(kk - 1, min=0)[:, None])
    near = ((r - kth).abs() <= tau) | ~diff
    bad = rows & ~near.all(1)
    return {"ok": not bool(bad.any()), "rows": int(r.shape[0]), "near_tie_rows": int(rows.sum()),
            "bad_rows": int(bad.sum()), "k": k}


def check(ref: torch.Tensor, got: torch.Tensor, tol: float, k: int = 16) -> dict:
    v = compare_values(ref, got, tol)
    t = compare_topk(ref, got, tol * v["M"], k)
    v["topk"] = t
    v["ok"] = v["ok"] and t["ok"]
    return v
