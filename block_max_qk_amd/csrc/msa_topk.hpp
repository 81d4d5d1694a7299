// Top-k block selection on the score rows, for gfx950.
//
// The stage after the block score (the notes "MiniMax Sparse Attention:
// paper algorithm and code", section 4.7
// "Top-k Block Selection" and section 5.3 "Top-k" with the sparse_topk_select
// contract; section 6.1 "Exp-free Top-k"): for every (query token t, index
// head h), the k best blocks of the row score[h, t, 0:num_valid] among those
// scoring above -inf, highest score first and equal scores by lower block
// index, written to out[t, h, 0:k] in ascending block order with a -1 tail.
// It works on the raw scores (no exp or normalisation).
//
// One wave per row at a time (with many rows a wave takes two in turn,
// loading the second while it selects on the first).  Scores map to order-preserving 32-bit keys (0 for
// blocks that cannot be selected); the k-th largest key tau is found bit by bit from
// the top, each step counting the keys at or above a candidate threshold with
// wave ballots.  As soon as at most 64 keys remain at or
// above the threshold being built, they move (in index order) into one
// register per lane and the rest of the search runs on that register alone.
// The selection is compacted in index order: every key above tau, and keys
// equal to tau while slots remain, lowest index first -- which also yields the
// ascending output without a sort.  Rows of up to 64 * J blocks keep their
// keys in registers (read once, 256 contiguous bytes per load instruction);
// longer rows (J = 0) re-read the row, from L2, at every step.
#pragma once

#include "msa_device.hpp"

namespace msa {

constexpr int kTopkMax = 64;   // k is at most one wave of lanes

// Order-preserving key of a score that can be selected; 0 for -inf and NaN.
__device__ __forceinline__ uint32_t topk_key(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return f > -__builtin_inff() ? key : 0u;
}

// All ones when b < n, else 0 (arithmetic, so no branch forms around it).
__device__ __forceinline__ uint32_t below_mask(int b, int n) { return (uint32_t)((b - n) >> 31); }

constexpr int kTopkWaves = 4;  // waves per workgroup
// Cache-policy operand of a buffer access: the nontemporal bit.
constexpr int kCachePolicyNT = 2;
// From this many rows on, each wave takes two rows in turn.
constexpr int64_t kTopkManyRows = 65536;

// The selection on one row whose scores (J > 0) are already in v: v[j] in
// lane l holds block 64 j + l (any value past nv).  J = 0 re-reads the row.
// slot: this wave's 128-entry LDS area; sel: its 64-entry output area.  The
// k results go to dst with one store per lane (lanes past k repeat slot k - 1),
// so every row issues the same memory operations.
template <int J>
__device__ __forceinline__ void topk_row(const float* __restrict__ row, const float (&v)[J > 0 ? J : 1],
                                         int nv, int k, int32_t* __restrict__ dst, uint2* slot,
                                         int32_t* sel) {
  const int l = lane_id();
  const int nch = (nv + 63) / 64;          // 64-block chunks holding candidates
  const int nj = J > 0 ? J : nch;
  uint32_t keys[J > 0 ? J : 1];
  if constexpr (J > 0) {
#pragma unroll
    for (int j = 0; j < J; ++j) keys[j] = topk_key(v[j]) & below_mask(j * 64 + l, nv);
  }
  auto key = [&](int j) -> uint32_t {
    if constexpr (J > 0) {
      return keys[j];
    } else {
      const int b = j * 64 + l;
      return topk_key(row[min(b, nv - 1)]) & below_mask(b, nv);
    }
  };
  // number of keys >= c over the row
  auto count_ge = [&](uint32_t c) -> int {
    int n = 0;
    for (int j = 0; j < nj; ++j) n += __popcll(__ballot(key(j) >= c));
    return n;
  };

  // tau = the k-th largest key (0 when the row has at most k candidates), or
  // any lower threshold that exactly k keys reach: the search stops there.
  // Invariant: at least k keys reach tau, and the bits of tau above the bit mb
  // under test are final.  Once at most 64 keys reach tau, they are compacted in index
  // order into one register per lane (through a per-wave LDS slot), and the
  // remaining steps and the selection work on that register alone.
  uint32_t tau = 0;
  bool comp = false;
  uint32_t ck = 0;            // compacted key (0 in lanes past the count)
  int ci = -1;                // its block index
  int cnt = count_ge(1u);     // keys >= tau, tau = 0: the candidates
  uint32_t mb = 0x80000000u;   // the bit of tau under test; 0 once all are final
  // With lb <= (the final tau) <= ub and tau <= lb: every value in [lb, ub]
  // has the leading bits lb and ub share, so tau takes them and the search
  // goes on below them.
  auto narrow = [&](uint32_t lb, uint32_t ub) {
    if (lb >= ub) {
      tau = ub;
      mb = 0u;
    } else {
      mb = 0x80000000u >> __builtin_clz(lb ^ ub);
      tau = ub & ~(2u * mb - 1u);
    }
  };
  if (cnt > k) {
    if (cnt > 64) {
      // phase 1: counts over all chunks while more than 64 keys reach tau.
      // With a candidate in every lane, the smallest lane maximum lo is a
      // lower bound (64 keys reach it) and the largest key an upper one.  At
      // the first threshold c that fewer than k keys reach, the largest key
      // below c is the tighter upper bound (it skips the few forced blocks
      // far above the rest).
      uint32_t lo = 0u;
      if constexpr (J > 0) {
        uint32_t mx = keys[0];
#pragma unroll
        for (int j = 1; j < J; ++j) mx = max(mx, keys[j]);
        uint32_t hi;
        wave_min_max(mx, mx, lo, hi);
        if (lo != 0u) narrow(lo, hi);
      }
      // steps up to the first threshold fewer than k keys reach
      uint32_t c = 0u;
      bool failed = false;
      while (mb != 0u) {
        c = tau | mb;
        const int n = count_ge(c);
        if (n < k) {
          failed = true;
          break;
        }
        tau = c;
        cnt = n;
        mb >>= 1;
        if (n <= 64) break;
      }
      if (failed) {
        if constexpr (J > 0) {
          uint32_t m2 = 0u;
#pragma unroll
          for (int j = 0; j < J; ++j) m2 = max(m2, keys[j] < c ? keys[j] : 0u);
          uint32_t unused, hi2;
          wave_min_max(m2, m2, unused, hi2);
          narrow(max(lo, tau), hi2);
        } else {
          mb >>= 1;
        }
        while (mb != 0u) {
          c = tau | mb;
          const int n = count_ge(c);
          const bool ok = n >= k;
          tau = ok ? c : tau;
          cnt = ok ? n : cnt;
          mb >>= 1;
          if (cnt <= 64) break;
        }
      }
    }
    // the keys reaching tau (all candidates when tau is still 0), in index
    // order, one per lane; lanes whose key does not qualify write to the
    // spare half of the slot, so the stores need no branch
    if (cnt <= 64) {
      const uint32_t floor_key = tau == 0u ? 1u : tau;
      int base = 0;
      for (int j = 0; j < nj; ++j) {
        const uint32_t kv = key(j);
        const bool q = kv >= floor_key;
        const uint64_t m = __ballot(q);
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        slot[q ? base + rank : 64 + l] = make_uint2(kv, j * 64 + l);
        base += __popcll(m);
      }
      wave_lds_sync();
      const uint2 e = slot[l];
      ck = l < base ? e.x : 0u;
      ci = l < base ? (int)e.y : -1;
      comp = true;
      // phase 2: the remaining bits on that register alone, stopping as soon
      // as exactly k keys reach tau, with the same refinement (the smallest
      // compacted key is a lower bound)
      if (cnt > k) {
        uint32_t c = 0u;
        bool failed = false;
        while (mb != 0u) {
          c = tau | mb;
          const int n = __popcll(__ballot(ck >= c));
          if (n < k) {
            failed = true;
            break;
          }
          tau = c;
          mb = n == k ? 0u : mb >> 1;
        }
        if (failed) {
          uint32_t lo2, hi2;
          wave_min_max(ck != 0u ? ck : ~0u, ck < c ? ck : 0u, lo2, hi2);
          narrow(max(lo2, tau), hi2);
          while (mb != 0u) {
            c = tau | mb;
            const int n = __popcll(__ballot(ck >= c));
            tau = n >= k ? c : tau;
            mb = n == k ? 0u : mb >> 1;
          }
        }
      }
    }
  }
  // keys above tau all fit; ties at tau fill the remaining slots
  const uint64_t below = (1ull << l) - 1ull;
  int taken = 0;
  if (comp) {
    const int need_eq = k - __popcll(__ballot(ck > tau));
    const bool eq = ck == tau;
    const uint64_t em = __ballot(eq);
    const bool take = ck > tau || (eq && __popcll(em & below) < need_eq);
    const uint64_t tm = __ballot(take);
    if (take) sel[__popcll(tm & below)] = ci;
    taken = __popcll(tm);
  } else {
    const int need_eq = tau == 0 ? 0 : k - count_ge(tau + 1u);
    int eq_seen = 0;
    for (int j = 0; j < nj; ++j) {
      const uint32_t kv = key(j);
      const bool eq = tau != 0u && kv == tau;
      const uint64_t em = __ballot(eq);
      const bool take = kv > tau || (eq && eq_seen + __popcll(em & below) < need_eq);
      const uint64_t tm = __ballot(take);
      if (take) sel[taken + __popcll(tm & below)] = j * 64 + l;
      taken += __popcll(tm);
      eq_seen += __popcll(em);
    }
  }
  if (l < k && l >= taken) sel[l] = -1;
  wave_lds_sync();
  const int o = min(l, k - 1);
  dst[o] = sel[o];
}

// grid (ceil(T / (4 R)), Hq): wave w of block (x, h) takes the rows
// (h, t) for t = (4 x + w) R + i, i < R; rows past T repeat row T - 1 (same
// result, same place).  Every lane loads and masks afterwards, so no load
// carries a branch and a row's loads are all in flight together.
template <int J, int R>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores, int64_t T,
                                                   int64_t Hq, int64_t W, int nv, int k,
                                                   int32_t* __restrict__ out) {
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = ((int64_t)blockIdx.x * kTopkWaves + w) * R;
  if (t0 >= T) return;
  const int64_t h = blockIdx.y;
  auto dst_of = [&](int i) { return out + (min(t0 + i, T - 1) * Hq + h) * k; };
  if (nv == 0) {                           // nothing to select; scores may be NULL
    for (int i = 0; i < R; ++i)
      if (l < k) dst_of(i)[l] = -1;
    return;
  }
  __shared__ uint2 packed[kTopkWaves][128];
  __shared__ int32_t chosen[kTopkWaves][64];
  auto row_of = [&](int i) { return scores + (h * T + min(t0 + i, T - 1)) * W; };
  // A row is read through a buffer descriptor (scalar base = the row, size =
  // nv floats): lane l's load j takes byte offset 4 l + 256 j, the same for
  // every row, and offsets past the size read as 0 (masked to key 0 later).
  // The loads skip the caches' usual allocation (nontemporal), being read
  // once.
  float v[J > 0 ? J : 1], vn[J > 0 ? J : 1];
  auto load = [&](float (&d)[J > 0 ? J : 1], const float* row) {
    if constexpr (J > 0) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(row), 0, 4 * nv, kBufferWord3);
#pragma unroll
      for (int j = 0; j < J; ++j)
        d[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * l + 256 * j, 0, kCachePolicyNT));
    }
  };
  load(vn, row_of(0));
#pragma unroll
  for (int i = 0; i < R; ++i) {
    // the next row's loads stay below the previous row's selection, so at
    // most two rows' scores are held at a time
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < (J > 0 ? J : 1); ++j) v[j] = vn[j];
    if (i + 1 < R) load(vn, row_of(i + 1));
    topk_row<J>(row_of(i), v, nv, k, dst_of(i), packed[w], chosen[w]);
  }
}

}  // namespace msa
