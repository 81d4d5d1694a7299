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
// A wave's LDS area holds 64 compacted entries, then a spare entry per lane
// for the stores of lanes with nothing to compact: 128 entries.  Rows held in
// up to 8 registers per lane get room for every key of the row (64 J
// entries, then the spare ones), so their compaction needs no bound on its
// store positions (4.6 KB per wave at J = 8, which still leaves eight waves
// per SIMD).
constexpr int kTopkSpare = 64;
template <int J>
constexpr bool topk_roomy() { return J > 0 && J <= 8; }
template <int J>
constexpr int topk_area_entries() { return topk_roomy<J>() ? 64 * J + 64 : 128; }

// Order-preserving key of a score that can be selected; 0 for -inf and NaN.
__device__ __forceinline__ uint32_t topk_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);   // -0 and +0 are one score
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

// The threshold search on one row.  J > 0: keys[j] in lane l is the key
// (topk_key, 0 past nv) of block 64 j + l.  J = 0 re-reads the row.
// slot: this wave's LDS area (at least 128 entries); sel: its 64-entry output area.  The
// k results go to dst with one store per lane (lanes past k repeat slot k - 1),
// so every row issues the same memory operations.
template <int J>
__device__ __forceinline__ void topk_row_search(const float* __restrict__ row,
                                                const uint32_t (&keys)[J > 0 ? J : 1], int nv, int k,
                                                int32_t* __restrict__ dst, uint2* slot, int32_t* sel) {
  const int l = lane_id();
  const int nch = (nv + 63) / 64;          // 64-block chunks holding candidates
  const int nj = J > 0 ? J : nch;
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

// Rotated key: topk_key's order on every selectable score, moved up by
// 2^23 - 1 with wrap-around, so that NaN and -inf fall below kKeyFloor (the
// key of -FLT_MAX) and no compare or select is needed to exclude them.
constexpr uint32_t kKeyShift = 0x007FFFFFu;
constexpr uint32_t kKeyFloor = 0x00FFFFFFu;
__device__ __forceinline__ uint32_t topk_key_rot(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);   // -0 and +0 are one score
  return (u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u)) + kKeyShift;
}
// The score whose rotated key is r (r >= kKeyFloor).
__device__ __forceinline__ float topk_key_rot_score(uint32_t r) {
  const uint32_t u = r - kKeyShift;
  return __uint_as_float((u & 0x80000000u) ? (u ^ 0x80000000u) : ~u);
}
// max(a, b, c) as the hardware computes it, without the quieting maxima the
// compiler puts around fmaxf on values of unknown origin: a NaN input can
// only lower a lane's maximum to a NaN, which the caller counts as nothing.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// The fast path covers k up to this many.
constexpr int kTopkFastK = 16;

// x holds, in every lane of each row of 16 lanes, that row's value; the
// smallest (or largest) over the four rows: row_bcast:15 passes lane 15 of
// each row to the next row (rows 1 and 3 take it), row_bcast:31 lane 31 to
// rows 2 and 3, so lane 63 ends with all four.
// (Written out: one DPP min or max per step, the rows outside the row mask
// keeping their value; the nops are the wait states a DPP read needs after a
// vector write of its source.)
template <bool MAX>
__device__ __forceinline__ uint32_t rows_combine(uint32_t x) {
  if constexpr (MAX)
    asm volatile(
        "s_nop 1\n\tv_max_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\tv_max_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\ts_nop 1"
        : "+v"(x));
  else
    asm volatile(
        "s_nop 1\n\tv_min_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\tv_min_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\ts_nop 1"
        : "+v"(x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Selection on one row held in registers, for k <= 16: x[j] in lane l is the
// score of block 64 j + l (-inf past nv).  Returns false, having written
// nothing to dst, when more than 64 scores reach the lower bound below; the
// caller then runs the general search.  Scores are compared as floats (NaN
// and -inf never qualify) until the compaction; the compacted candidates then
// turn into rotated keys.
//
// Lower bound: in each eight-lane half row, the two largest lane maxima are
// keys of two different blocks, so the smallest such second maximum over the
// eight half rows, t0, is reached by at least 16 >= k keys: the k-th largest
// key is >= t0.  On rows of independent scores about 30 keys reach t0, so
// one pass compacts them (in index order) into one register per lane, and
// the threshold search runs on that register alone: no step of it reads the
// whole row again.
template <int J>
__device__ __forceinline__ bool topk_row_fast(const float (&x)[J], int k,
                                              int32_t* __restrict__ dst, uint2* slot,
                                              int32_t* sel) {
  const int l = lane_id();
  // the lane's largest score, as a rotated key (below kKeyFloor when the lane
  // has nothing selectable)
  float mf = x[0];
  {
    int j = 1;
#pragma unroll
    for (; j + 1 < J; j += 2) mf = max3_raw(mf, x[j], x[j + 1]);
    if (j < J) mf = max3_raw(mf, x[j], x[j]);
  }
  const uint32_t m = topk_key_rot(mf == mf ? mf : -__builtin_inff());
  // the two largest lane maxima (a1 >= a2) of every pair, quad, then half row
  uint32_t a1, a2;
  {
    const uint32_t b = dpp_u32<0xB1>(m);  // quad_perm 1,0,3,2
    a1 = max(m, b);
    a2 = min(m, b);
  }
  {
    const uint32_t b1 = dpp_u32<0x4E>(a1), b2 = dpp_u32<0x4E>(a2);  // quad_perm 2,3,0,1
    a2 = max(min(a1, b1), max(a2, b2));
    a1 = max(a1, b1);
  }
  {
    const uint32_t b1 = dpp_u32<0x141>(a1), b2 = dpp_u32<0x141>(a2);  // row_half_mirror
    a2 = max(min(a1, b1), max(a2, b2));
  }
  a2 = min(a2, dpp_u32<0x140>(a2));  // row_mirror: both half rows of a row
  const uint32_t t0 = max(rows_combine<false>(a2), kKeyFloor);
  const float t0f = topk_key_rot_score(t0);

  // compaction of the keys >= t0, in index order, as (key, block) entries.
  // Each store goes to the area's byte address 8 base (scalar; 8 min(base,
  // 64) in a 128-entry area) plus 8 times the lane's rank in the chunk;
  // lanes whose key does not qualify write to their spare entry, so the
  // stores need no branch.  A row with more than 64 such keys goes to the
  // general search; until this pass ends its stores stay inside the area
  // (index at most 64 J - 1, or 64 + 63 in a 128-entry area).
  // (For J > 8 the lane number passes through an empty asm, so that the
  // block numbers are formed at each store rather than held in registers
  // across rows.)
  uint32_t lv = (uint32_t)l;
  if constexpr (J > 8) asm volatile("" : "+v"(lv));
  constexpr bool ROOMY = topk_roomy<J>();
  char* const area = reinterpret_cast<char*>(slot);
  char* const area_end = area + 8 * 64;
  uint2* const spare = slot + (ROOMY ? 64 * J : kTopkSpare) + l;
  char* next = area;                         // area + 8 (entries so far)
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const bool q = x[j] >= t0f;
    const uint64_t mk = __ballot(q);
    const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
    uint2* const at =
        reinterpret_cast<uint2*>(ROOMY ? next : (next < area_end ? next : area_end)) + r;
    *(q ? at : spare) = make_uint2(__float_as_uint(x[j]), lv + (uint32_t)(j * 64));
    next += 8 * __popcll(mk);
  }
  const int base = (int)((next - area) >> 3);
  if (base > 64) return false;
  wave_lds_sync();
  const uint2 e = slot[l];
  const uint32_t ck = l < base ? topk_key_rot(__uint_as_float(e.x)) : 0u;   // 0: no candidate

  // tau: the k-th largest compacted key, or a lower threshold that exactly k
  // keys reach; below every candidate when there are at most k.
  uint32_t tau = kKeyFloor - 1u;
  if (base > k) {
    // Bounds: t0 from below.  From above, the largest compacted key under
    // the key of 1e28 when fewer than k keys reach that key (the forced
    // local_mask values 1e30 and 1e29 are the only scores that do, far above
    // every computed one), else the largest key.
    const uint32_t hi_cut = topk_key_rot(1e28f);
    const int n_hi = __popcll(__ballot(ck >= hi_cut));
    uint32_t x = (n_hi < k && ck >= hi_cut) ? 0u : ck;
    x = max(x, dpp_u32<0xB1>(x));
    x = max(x, dpp_u32<0x4E>(x));
    x = max(x, dpp_u32<0x141>(x));
    x = max(x, dpp_u32<0x140>(x));
    const uint32_t ub = rows_combine<true>(x);
    // tau takes the leading bits t0 and ub share; the search goes on below
    // them, one bit a step: the bit stays when at least k keys reach
    // tau | bit, and the search ends once exactly k do (scalar registers
    // throughout, one vector compare a step)
    if (t0 >= ub) {
      tau = ub;
    } else {
      uint32_t mb = 0x80000000u >> __builtin_clz(t0 ^ ub);
      tau = ub & ~(2u * mb - 1u);
      uint32_t c, n;
      asm volatile(
          "1:\n\t"
          "s_or_b32 %[c], %[tau], %[mb]\n\t"
          "v_cmp_le_u32 vcc, %[c], %[ck]\n\t"
          "s_bcnt1_i32_b64 %[n], vcc\n\t"
          "s_cmp_ge_u32 %[n], %[k]\n\t"
          "s_cselect_b32 %[tau], %[c], %[tau]\n\t"
          "s_cmp_eq_u32 %[n], %[k]\n\t"
          "s_cbranch_scc1 2f\n\t"
          "s_lshr_b32 %[mb], %[mb], 1\n\t"   // SCC: the result is not 0
          "s_cbranch_scc1 1b\n"
          "2:"
          : [tau] "+s"(tau), [mb] "+s"(mb), [c] "=&s"(c), [n] "=&s"(n)
          : [ck] "v"(ck), [k] "s"((uint32_t)k)
          : "vcc", "scc");
    }
  }
  // keys above tau all fit; ties at tau fill the remaining slots, lowest
  // index first; the taken blocks, in index order, then -1
  auto rank_in = [](uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
  };
  bool take = ck >= tau;
  uint64_t tm = __ballot(take);
  if (__popcll(tm) > k) {                  // ties at tau (rare)
    const int need_eq = k - __popcll(__ballot(ck > tau));
    const bool eq = ck == tau;
    take = ck > tau || (eq && rank_in(__ballot(eq)) < need_eq);
    tm = __ballot(take);
  }
  if (take) sel[rank_in(tm)] = (int32_t)e.y;
  const int taken = __popcll(tm);
  wave_lds_sync();
  const int o = min(l, k - 1);
  const int32_t got = sel[o];
  dst[o] = o < taken ? got : -1;
  return true;
}

// The selection on one row whose scores (J > 0) are already in v: v[j] in
// lane l holds block 64 j + l (any value past nv).  J = 0 re-reads the row.
// FULL: nv == 64 J (no block past nv in the registers).
template <int J, bool FULL>
__device__ __forceinline__ void topk_row(const float* __restrict__ row, float (&v)[J > 0 ? J : 1],
                                         int nv, int k, int32_t* __restrict__ dst, uint2* slot,
                                         int32_t* sel) {
  uint32_t keys[J > 0 ? J : 1];
  if constexpr (J > 0) {
    const int l = lane_id();
    if (k <= kTopkFastK) {
      if constexpr (!FULL) {
#pragma unroll
        for (int j = 0; j < J; ++j) v[j] = j * 64 + l < nv ? v[j] : -__builtin_inff();
      }
      if (topk_row_fast<J>(v, k, dst, slot, sel)) return;
    }
    // the general search, on the row read again (from L2, rarely): the fast
    // path's registers are then free for it
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(row), 0, 4 * nv, kBufferWord3);
    uint32_t lv = (uint32_t)l;             // formed here, not held from the kernel's start
    asm volatile("" : "+v"(lv));
#pragma unroll
    for (int j = 0; j < J; ++j)
      keys[j] = topk_key(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lv + 256 * j, 0, 0))) &
                below_mask(j * 64 + (int)lv, nv);
  }
  topk_row_search<J>(row, keys, nv, k, dst, slot, sel);
}

// grid (ceil(T / (4 R)), Hq): wave w of block (x, h) takes the rows
// (h, t) for t = (4 x + w) R + i, i < R; rows past T repeat row T - 1 (same
// result, same place).  Every lane loads and masks afterwards, so no load
// carries a branch and a row's loads are all in flight together.
template <int J, int R, bool FULL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores, int64_t T,
                                                   int64_t Hq, int64_t W, int nv, int k,
                                                   int32_t* __restrict__ out) {
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = ((int64_t)blockIdx.x * kTopkWaves + w) * R;
  if (t0 >= T) return;
  const int64_t h = blockIdx.y;
  // row i of this wave is row min(i, last) (rows past T repeat row T - 1);
  // from the wave's first row the row pointer steps by W floats and the
  // output by Hq k entries
  const int last = (int)min(T - 1 - t0, (int64_t)(R - 1));
  int32_t* const out0 = out + (t0 * Hq + h) * k;
  const int out_step = (int)Hq * k;
  auto dst_of = [&](int i) { return out0 + min(i, last) * out_step; };
  if (nv == 0) {                           // nothing to select; scores may be NULL
    for (int i = 0; i < R; ++i)
      if (l < k) dst_of(i)[l] = -1;
    return;
  }
  __shared__ uint2 packed[kTopkWaves][topk_area_entries<J>()];
  __shared__ int32_t chosen[kTopkWaves][64];
  const float* const row0 = scores + (h * T + t0) * W;
  auto row_of = [&](int i) { return row0 + min(i, last) * (int)W; };
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
    topk_row<J, FULL>(row_of(i), v, nv, k, dst_of(i), packed[w], chosen[w]);
  }
}

}  // namespace msa
