// MSA index-score kernels for gfx950.
//
// Both kernels compute, for one work item (KV head, head chunk, range of
// blocks, tile of query tokens of one request), the block maximum
//   score[h, t, beta] = max_{visible j in beta} < q[t, h], k~[j, h / g] >
// (gitcode cann/ops-transformer issue #4117, section 计算过程; the order
// DOT -> DEQUANT -> MASK -> MAX) and write the tile's rows of columns
// [c0, c1) of the [Hq, T, W] float32 output, including the -inf fill and the
// local_mask constants.
//
// decode_kernel  -- 16 rows per tile (the g heads of a KV group for one or a
//   few tokens).  Key traffic dominates and nothing is reused across rows, so
//   each wave streams whole blocks straight from HBM into MFMA operand
//   registers (16x16 tiles, key tokens on M, rows on N) and many waves per CU
//   keep enough bytes in flight.
// prefill_kernel -- 384 rows per tile for 16-bit keys (48 tokens x 8 heads for
//   g = 8), 256 for fp8 and int8.  A key block is staged once per workgroup
//   into LDS in a bank-conflict-free XOR-swizzled layout (straight from
//   HBM/L2 for 16-bit and fp8, widened to fp16 through registers for int8)
//   and read by all four waves, each holding 96 (or 64) query rows in
//   registers (32x32 MFMA tiles, key tokens on M).
//
// In both, a lane's accumulators hold several key tokens of one row, so the
// 128-wide block maximum is an in-register max over the lane's values (after
// the int8 column scale and, on blocks cut by the causal window or kv_len, a
// select to -inf) followed by one or two cross-lane steps.
#pragma once

#include <type_traits>

#include "msa_device.hpp"

namespace msa {

constexpr int kDecodeRows = 16;
constexpr int kPrefillRows = 256;   // family choice threshold: half of this per request
// Blocks per prefill work item: the work item's query tile and ring set-up
// (and for MXFP4 its scale staging) are amortised over them; one A/B each:
//  16-bit keys: varlen prefill 4.00 ms with 16, 3.90 with 32, 3.99 with 64;
//               then 4.00 with 32, 3.92 with 40, 3.93 with 48 on another box
//  fp8:         chunked prefill 3.15 ms with 32, 3.13 with 48 or 64
//  MXFP4:       varlen prefill 1.345 ms with 32, 1.313 with 48, 1.338 with 64
//  int8:        32 (no prefill workload of its own)
constexpr int kPrefillChunk = 32;
constexpr int prefill_chunk(int kk) {
  return kk == KMXFP4 ? 48 : (kk == KF8E4M3 || kk == KF8E5M2) ? 48
       : (kk == KF16 || kk == KBF16) ? 40 : kPrefillChunk;
}
constexpr int kPrefillWaves = 4;   // waves per prefill workgroup

// 32-row MFMA N tiles each prefill wave holds; a workgroup's tile is four
// waves of them.  More N tiles let one key fragment read from LDS feed more
// MFMAs, at the cost of query registers (and so waves per SIMD): 16-bit keys
// take three (two waves per SIMD), fp8 and int8 two.
constexpr int prefill_ntw(int kk) {
  return (kk == KF16 || kk == KBF16) ? 3 : kk == KMXFP4 ? 4 : 2;
}
constexpr int prefill_rows(int kk) { return 4 * 32 * prefill_ntw(kk); }

// ---------------------------------------------------------------------------
// decode
//
// The batch's work is the list of (tile, visible block) pairs, tiles in
// request order and blocks ascending; its length N is known only on the
// device.  Each workgroup takes an equal contiguous slice of the list, so
// every CU streams about the same number of key blocks whatever the spread
// of kv_len.  With at most 64 requests a workgroup holds all of a CU's waves
// and they take the slice's pairs from an LDS counter as they finish blocks;
// with more, four-wave workgroups (two to four per CU) and each wave takes
// every fourth pair of its workgroup's slice.  The grid is one round of
// workgroups (as many as the chip holds at once), so no workgroup waits for
// a slot.  Columns a tile cannot see (past its last
// visible block, up to the output width) are written by a fill pass.
// Key blocks are loaded to registers: 16-bit, fp8 and int8 blocks pass
// through a per-wave LDS area into the MFMA operand order; MXFP4 blocks
// (8 KB) load straight into it and take four workgroups per CU instead of
// two (measured: 8 KB blocks gain nothing from loading two to four of a
// wave's blocks together at two workgroups per CU).
// ---------------------------------------------------------------------------

// Visible blocks of tile j of a request (kv_len L, L_q query tokens): up to
// the block of the tile's last visible key, never past MB.
__device__ __forceinline__ int tile_blocks(const Params& p, int L, int Lq, int j) {
  if (L <= 0) return 0;
  const int ilast = min((j + 1) * p.tpt, Lq) - 1;
  const int qpos = p.causal ? (L - Lq + ilast) : (L - 1);
  const int lim = min(qpos, L - 1);
  return lim < 0 ? 0 : min(lim / kP + 1, p.MB);
}

__device__ __forceinline__ int tiles_of(const Params& p, int Lq) {
  return (Lq + p.tpt - 1) / p.tpt;
}

// Position in the work list.
struct Cursor {
  int b, j, beta, nvis;    // request, tile of the request, block, blocks of the tile
  int cu, Lq, L;           // cu_seqlens_q[b], L_q, kv_len
  int64_t koff;            // packed-key offset of the request
};

// Per-lane view of 64 consecutive requests: lengths, their work-list and
// tile counts, and wave-wide inclusive prefix sums of those.
// With SL, also each request's start_loc (0 under the per-query window, where
// it is not read).
struct Scan64 {
  int cu, lq, kv, sl, tasks, tiles;
  int inc_tasks, inc_tiles;
  int64_t inc_kv;
};

template <bool SL = false>
__device__ __forceinline__ Scan64 scan64(const Params& p, int base) {
  Scan64 s;
  const int b = base + lane_id();
  s.cu = s.lq = s.kv = s.sl = s.tasks = s.tiles = 0;
  if (b < p.B) {
    s.cu = p.cu_q[b];
    s.lq = p.cu_q[b + 1] - s.cu;
    s.kv = p.kv_len[b];
    if (SL && !p.local_per_query) s.sl = p.start_loc[b];
    s.tiles = tiles_of(p, s.lq);
    for (int j = 0; j < s.tiles; ++j) s.tasks += tile_blocks(p, s.kv, s.lq, j);
  }
  s.inc_tasks = wave_incl_scan(s.tasks);
  s.inc_tiles = wave_incl_scan(s.tiles);
  s.inc_kv = wave_incl_scan((int64_t)s.kv);
  return s;
}

// Totals over the batch: work-list length and number of tiles.  A batch of
// at most 64 requests is scanned once and `first` is kept for seek().
__device__ __forceinline__ void count_work(const Params& p, Scan64& first, int& ntask,
                                           int& ntile) {
  ntask = ntile = 0;
  for (int base = 0; base < p.B; base += 64) {
    const Scan64 s = scan64<true>(p, base);
    if (base == 0) first = s;
    ntask += lane_at(s.inc_tasks, 63);
    ntile += lane_at(s.inc_tiles, 63);
  }
}

// Batches of more than 64 requests: the work-list, tile and packed-key
// offsets at the start of each 64-request chunk (the first kChunkTab chunks),
// kept in LDS, so that a cursor is placed by one search over the table and
// one scan of its chunk instead of a scan of the batch from its start.
constexpr int kChunkTab = 256;
struct ChunkTable {
  int tasks[kChunkTab + 1];
  int tiles[kChunkTab + 1];
  int64_t kv[kChunkTab + 1];
  int wave_tasks[4], wave_tiles[4];
};

// Totals over the batch (as count_work) and the chunk table: the four waves
// scan every fourth chunk, then wave 0 turns the chunk totals into offsets.
// Every wave of the workgroup calls it (it holds two workgroup barriers).
__device__ __forceinline__ void count_work_table(const Params& p, ChunkTable& tab, int& ntask,
                                                 int& ntile) {
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int nch = (p.B + 63) >> 6;
  const int ntab = min(nch, kChunkTab);
  int wt = 0, wl = 0;
  for (int ch = wave; ch < nch; ch += 4) {
    const Scan64 s = scan64(p, ch << 6);
    const int t = lane_at(s.inc_tasks, 63);
    const int u = lane_at(s.inc_tiles, 63);
    const int64_t kvt = lane_at(s.inc_kv, 63);
    if (ch < kChunkTab && l == 0) {
      tab.tasks[ch + 1] = t;
      tab.tiles[ch + 1] = u;
      tab.kv[ch + 1] = kvt;
    }
    wt += t;
    wl += u;
  }
  if (l == 0) {
    tab.wave_tasks[wave] = wt;
    tab.wave_tiles[wave] = wl;
  }
  __syncthreads();
  ntask = tab.wave_tasks[0] + tab.wave_tasks[1] + tab.wave_tasks[2] + tab.wave_tasks[3];
  ntile = tab.wave_tiles[0] + tab.wave_tiles[1] + tab.wave_tiles[2] + tab.wave_tiles[3];
  if (wave == 0) {
    int at = 0, al = 0;
    int64_t ak = 0;
    for (int base = 0; base < ntab; base += 64) {
      const int e = base + l + 1;      // chunk e - 1's total, then chunk e's offset
      const bool in = e <= ntab;
      const int it = wave_incl_scan(in ? tab.tasks[e] : 0);
      const int il = wave_incl_scan(in ? tab.tiles[e] : 0);
      const int64_t ik = wave_incl_scan(in ? tab.kv[e] : (int64_t)0);
      if (in) {
        tab.tasks[e] = at + it;
        tab.tiles[e] = al + il;
        tab.kv[e] = ak + ik;
      }
      at += lane_at(it, 63);
      al += lane_at(il, 63);
      ak += lane_at(ik, 63);
    }
    if (l == 0) {
      tab.tasks[0] = 0;
      tab.tiles[0] = 0;
      tab.kv[0] = 0;
    }
  }
  __syncthreads();
}

// seek() for batches with a chunk table: the scan starts at request base0
// with the offsets acc0 (entries or tiles) and kacc0 (packed keys) before it.
__device__ __forceinline__ void seek_from(const Params& p, int base0, int acc0, int64_t kacc0,
                                          int tau, bool by_tile, Cursor& c) {
  int acc = acc0;
  int64_t kacc = kacc0;
  for (int base = base0; base < p.B; base += 64) {
    const Scan64 s = scan64(p, base);
    const int cnt = by_tile ? s.tiles : s.tasks;
    const int incl = by_tile ? s.inc_tiles : s.inc_tasks;
    const int total = lane_at(incl, 63);
    if (tau < acc + total) {
      const int src = __ffsll((long long)__ballot(acc + incl > tau)) - 1;
      c.b = base + src;
      c.Lq = lane_at(s.lq, src);
      c.L = lane_at(s.kv, src);
      c.koff = kacc + lane_at(s.inc_kv, src) - c.L;
      c.cu = lane_at(s.cu, src);
      int local = tau - (acc + lane_at(incl, src) - lane_at(cnt, src));
      if (by_tile) {
        c.j = local;
        c.beta = 0;
        c.nvis = tile_blocks(p, c.L, c.Lq, c.j);
        return;
      }
      for (int j = 0;; ++j) {
        const int nv = tile_blocks(p, c.L, c.Lq, j);
        if (local < nv) {
          c.j = j;
          c.beta = local;
          c.nvis = nv;
          return;
        }
        local -= nv;
      }
    }
    acc += total;
    kacc += lane_at(s.inc_kv, 63);
  }
}

// Cursor at work-list entry tau (< N) of a batch of at most 64 requests,
// whose scan is `first`: no memory reads.  With by_tile, tau counts tiles
// instead and the cursor lands on block 0 of tile tau.
__device__ __forceinline__ void seek(const Params& p, const Scan64& first, int tau,
                                     bool by_tile, Cursor& c) {
  const int cnt = by_tile ? first.tiles : first.tasks;
  const int incl = by_tile ? first.inc_tiles : first.inc_tasks;
  const int src = __ffsll((long long)__ballot(incl > tau)) - 1;
  c.b = src;
  c.Lq = lane_at(first.lq, src);
  c.L = lane_at(first.kv, src);
  c.koff = lane_at(first.inc_kv, src) - c.L;
  c.cu = lane_at(first.cu, src);
  int local = tau - (lane_at(incl, src) - lane_at(cnt, src));
  if (by_tile) {
    c.j = local;
    c.beta = 0;
    c.nvis = tile_blocks(p, c.L, c.Lq, c.j);
    return;
  }
  for (int j = 0;; ++j) {
    const int nv = tile_blocks(p, c.L, c.Lq, j);
    if (local < nv) {
      c.j = j;
      c.beta = local;
      c.nvis = nv;
      return;
    }
    local -= nv;
  }
}

// The same through the chunk table: the last table chunk whose offset is at
// most tau (the offsets do not decrease), then the scan from there.
__device__ __forceinline__ void seek_table(const Params& p, const ChunkTable& tab, int tau,
                                           bool by_tile, Cursor& c) {
  const int ntab = min((p.B + 63) >> 6, kChunkTab);
  const int* pre = by_tile ? tab.tiles : tab.tasks;
  int ch = 0;
  for (int base = 0; base < ntab; base += 64) {
    const int e = base + lane_id();
    const int cnt = __popcll(__ballot(e < ntab && pre[e] <= tau));
    if (cnt > 0) ch = base + cnt - 1;
    if (cnt < 64) break;
  }
  seek_from(p, ch << 6, pre[ch], tab.kv[ch], tau, by_tile, c);
}

// Move a cursor that sits on block 0 of a tile to block 0 of the next tile.
__device__ __forceinline__ void next_tile(const Params& p, Cursor& c) {
  ++c.j;
  while (c.j >= tiles_of(p, c.Lq)) {
    c.koff += c.L;
    ++c.b;
    c.cu = p.cu_q[c.b];
    c.Lq = p.cu_q[c.b + 1] - c.cu;
    c.L = consumed(p.kv_len[c.b]);
    c.j = 0;
  }
  c.beta = 0;
  c.nvis = tile_blocks(p, c.L, c.Lq, c.j);
}

// Move the cursor `step` entries forward; the caller guarantees the target
// entry exists.
__device__ __forceinline__ void advance(const Params& p, Cursor& c, int step) {
  c.beta += step;
  while (c.beta >= c.nvis) {
    c.beta -= c.nvis;
    ++c.j;
    while (c.j >= tiles_of(p, c.Lq)) {
      c.koff += c.L;
      ++c.b;
      c.cu = p.cu_q[c.b];
      c.Lq = p.cu_q[c.b + 1] - c.cu;
      c.L = consumed(p.kv_len[c.b]);
      c.j = 0;
    }
    c.nvis = tile_blocks(p, c.L, c.Lq, c.j);
  }
}

// advance() for a batch of at most 64 requests, whose lengths the scan
// `first` holds: no memory reads.
__device__ __forceinline__ void advance_scan(const Params& p, const Scan64& f, Cursor& c,
                                             int step) {
  c.beta += step;
  while (c.beta >= c.nvis) {
    c.beta -= c.nvis;
    ++c.j;
    while (c.j >= tiles_of(p, c.Lq)) {
      c.koff += c.L;
      ++c.b;
      c.cu = lane_at(f.cu, c.b);
      c.Lq = lane_at(f.lq, c.b);
      c.L = lane_at(f.kv, c.b);
      c.j = 0;
    }
    c.nvis = tile_blocks(p, c.L, c.Lq, c.j);
  }
}

// Waves per decode workgroup.  A batch of at most 64 requests runs one
// workgroup per CU holding all of the CU's waves (two per SIMD for 16-bit
// keys, three for int8 and fp8, four for MXFP4), which share the workgroup's
// slice of the work list through an LDS counter; the chunk-table instance
// (larger batches) runs four-wave workgroups with fixed shares.
template <int KK, bool BIG>
constexpr int decode_waves() {
  return BIG ? 4
             : 4 * (Kind<KK>::is_fp4 ? 4 : (Kind<KK>::is_i8 || Kind<KK>::is_f8) ? 3 : 2);
}

// Workgroups per CU the decode kernel is built for (its register budget).
template <int KK, bool BIG>
constexpr int decode_min_groups() {
  return BIG ? (Kind<KK>::is_fp4 ? 4 : (Kind<KK>::is_i8 ? 3 : 2)) : 1;
}

// Work of the cursor's tile as seen by the block helpers.
__device__ __forceinline__ Work tile_work(const Params& p, const Cursor& c, int hk, int hc) {
  Work w;
  w.valid = 1;
  w.hk = hk;
  w.hc = hc;
  w.c0 = 0;
  w.c1 = p.W;
  w.b = c.b;
  w.t0 = c.cu + c.j * p.tpt;
  w.ntok = min(p.tpt, c.Lq - c.j * p.tpt);
  w.Lq = c.Lq;
  w.L = c.L;
  w.koff = c.koff;
  w.sl = -1;                   // (decode reads start_loc through local_anchor)
  return w;
}

// BIG: the batch has more than 64 requests (the chunk-table paths).
template <int KK, bool BIG>
__global__ __launch_bounds__((64 * decode_waves<KK, BIG>()), (decode_min_groups<KK, BIG>()))
void decode_kernel(Params p) {
  using Kd = Kind<KK>;
  constexpr int NW = decode_waves<KK, BIG>();
  // int8: each wave's current block of column scales, staged so that every
  // lane can read the four consecutive scales of its accumulator tokens
  __shared__ __attribute__((aligned(16))) float dscl[Kd::is_i8 ? NW : 1][kP];
  // four transpose areas per wave, each one 16-token sub-tile of key rows
  // (MXFP4 reads its operands straight from memory and uses none)
  constexpr int RBY = kD * Kd::k_bytes;        // key row bytes
  __shared__ __attribute__((aligned(16))) uint8_t dkt[Kd::is_fp4 ? 1 : NW][Kd::is_fp4 ? 1 : 4]
                                                     [Kd::is_fp4 ? 16 : 16 * RBY];
  // Batches of at most 64 requests: the two counters the waves take entries
  // from (blocks of the workgroup's slice, then its fill items).
  __shared__ int ctr[BIG ? 1 : 2];
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int n = l & 15;          // this lane's row (MFMA N index) and key token (M index)
  const int G = l >> 4;          // this lane's k group, 0..3
  if constexpr (!BIG) {
    // (before any wave takes an entry; every wave passes this barrier)
    if (threadIdx.x == 0) {
      ctr[0] = NW;
      ctr[1] = NW;
    }
    __syncthreads();
  }

  const int unit = blockIdx.x % p.units;
  const int wi = blockIdx.x / p.units;
  const int gu = gridDim.x / p.units;
  const int hk = unit / p.hchunks;
  const int hc = unit - hk * p.hchunks;

  // Batches of up to 64 requests keep their one chunk in registers; larger
  // ones build the chunk table.
  __shared__ std::conditional_t<BIG, ChunkTable, int> ctab;
  int ntask, ntile;
  Scan64 first;
  if constexpr (BIG)
    count_work_table(p, ctab, ntask, ntile);
  else
    count_work(p, first, ntask, ntile);
  auto place = [&](int tau, bool by_tile, Cursor& c) {
    if constexpr (BIG)
      seek_table(p, ctab, tau, by_tile, c);
    else
      seek(p, first, tau, by_tile, c);
  };
  // last block of a row's local_mask window (the scan holds start_loc when
  // the batch has at most 64 requests)
  auto anchor = [&](const Work& w, int i) -> int {
    if constexpr (BIG)
      return local_anchor(p, w, i);
    else
      return p.local_per_query ? query_anchor(w, i) : lane_at(first.sl, w.b);
  };

  // Fill, after the compute pass: the columns past each tile's last visible
  // block get -inf (and local_mask).  Items are (tile, row) pairs; each
  // workgroup takes a contiguous range of them.  A row's columns are written
  // as 16-byte stores (a scalar head up to the first 16-byte boundary, which
  // the compute pass does not touch).  Run first, its stores and index reads
  // delayed every wave's first key loads by several microseconds.  With the
  // chunk table the whole workgroup writes each item in turn, its cursor
  // stepped from tile to tile (placing it anew for every item cost a scan per
  // item); with at most 64 requests each wave takes items from an LDS counter
  // once it runs out of blocks, so the waves that finish last take none.
  auto fill_item = [&](const Cursor& c, int r, int tix, int nthr) {
    const Work w = tile_work(p, c, hk, hc);
    const int ri = r / p.hpt;
    const int rh = hc * p.hpt + (r - ri * p.hpt);
    if (r >= p.hpt * p.tpt || ri >= w.ntok || rh >= p.g) return;
    float* const row = p.out + (((int64_t)hk * p.g + rh) * p.T + (w.t0 + ri)) * p.W;
    const int start = anchor(w, c.j * p.tpt + ri);
    const int v0 = c.nvis;
    const int a0 = min((v0 + 3) & ~3, p.W);
    if (tix < a0 - v0)
      row[v0 + tix] = finish(p, w.L, start, v0 + tix, false, 0.f);
    for (int cc = a0 + 4 * tix; cc < p.W; cc += 4 * nthr) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = finish(p, w.L, start, cc + e, false, 0.f);
      *reinterpret_cast<f32x4*>(row + cc) = v;
    }
  };
  auto fill_pass = [&]() {
    if constexpr (BIG) {
      const int nitems = ntile * kDecodeRows;
      const int per = (nitems + gu - 1) / gu;
      const int i0 = wi * per;
      const int i1 = min(nitems, i0 + per);
      if (i0 >= i1) return;
      int ck = i0 / kDecodeRows;
      Cursor c;
      seek_table(p, ctab, ck, true, c);
      for (int it = i0; it < i1; ++it) {
        const int k = it / kDecodeRows;
        for (; ck < k; ++ck) next_tile(p, c);
        fill_item(c, it - k * kDecodeRows, (int)threadIdx.x, 256);
      }
    }
  };

  // compute pass over this workgroup's slice of the work list
  const int per = (ntask + gu - 1) / gu;
  const int s0 = wi * per;
  const int s1 = min(ntask, s0 + per);
  int task = s0 + wave;
  Cursor c;
  // Batches of at most 64 requests: the waves take the slice's entries from
  // an LDS counter, each its first one by its index, so that waves whose
  // loads the memory system serves sooner take more blocks (with fixed
  // shares, the workgroups of one CU finished 8-20 us apart: the CU's older
  // waves are served first).  The next entry is taken as soon as a block's
  // key loads are issued, so that the LDS round trip overlaps the wait for
  // the keys.  Page indices come from a window of 64 consecutive entries of
  // the slice held one per lane and read with readlane; a wave loads the
  // window again only when it takes an entry past it.
  auto take = [&](int which) -> int {
    int r = 0;
    if (l == 0) r = atomicAdd(&ctr[which], 1);
    return __builtin_amdgcn_readfirstlane(r);
  };
  // Page index of entry wb + l (entries past the slice repeat its last):
  // the entry belongs to the last request whose work starts at or before it,
  // searched from the request of `from` (an entry at or before wb); its tile
  // and block follow from the tiles' visible-block counts.
  auto load_window = [&](int wb, const Cursor& from) -> int {
    const int tau = min(wb + l, s1 - 1);
    // lane r: first entry of request r; the requests after from.b that start
    // inside the window are the only other candidates, and the last one
    // starting at or before tau is found by halving steps over them
    const int start = first.inc_tasks - first.tasks;
    const int nreq = min(p.B, 64);
    const int ncand = __popcll(__ballot(l > from.b && l < nreq && start <= wb + 63));
    int b = from.b;
    for (int step = ncand ? 1 << (31 - __builtin_clz(ncand)) : 0; step > 0; step >>= 1) {
      const int r = b + step;
      const int st = __shfl(start, min(r, 63));
      if (r <= from.b + ncand && st <= tau) b = r;
    }
    const int ex = __shfl(start, b);
    const int L = __shfl(first.kv, b), Lq = __shfl(first.lq, b);
    int local = tau - ex;
    int j = 0;
    for (int nv = tile_blocks(p, L, Lq, 0); local >= nv; nv = tile_blocks(p, L, Lq, ++j))
      local -= nv;
    return p.block_table[(int64_t)b * p.MB + local];
  };
  int v = __builtin_amdgcn_readfirstlane(wave);  // entry of the slice (from s0)
  int vnext = 0;
  int wb = 0, pwin = 0;                          // page window: entries [s0 + wb, +64)
  auto take_next = [&]() {
    if constexpr (!BIG) {
      vnext = take(0);
      if (p.paged && vnext < s1 - s0 && vnext - wb >= 64) {
        wb = vnext;
        // (waited for here: it follows this block's key loads, which the
        // block waits for anyway; left pending, the compiler would wait
        // for every memory operation at the top of each block)
        pwin = consumed(load_window(s0 + wb, c));
      }
    }
  };
  if constexpr (BIG) {
    if (task >= s1) {
      fill_pass();
      return;
    }
    place(task, false, c);
  } else if (v < s1 - s0) {
    task = s0 + v;       // (wave-uniform to the compiler, as the cursor must be)
    if (p.paged) {
      Cursor c0;
      place(s0, false, c0);
      pwin = load_window(s0, c0);
    }
    place(task, false, c);
    pwin = consumed(pwin);
  }
  int cur_b = -1, cur_j = -1;
  Work w;
  i32x4 qv[4];
  int qs = 127;                  // MXFP4: the query scale of this lane's 32-element group
  int lim = -1, lim_lo = -1, start = 0;
  // Paged keys with the chunk table: page indices of this wave's next blocks
  // of the tile, lane k holding the k-th (blocks beta, beta + 4, ...), read
  // with readlane; pk is the next lane to read (64: load again).  One load
  // per tile instead of one per block keeps conditional memory reads out of
  // the steady-state loop.
  int pidx = 0, pk = 64;
  // A block's result is stored once the next block's key loads are issued:
  // storing it at the end of its own iteration made the compiler wait for
  // that store (the memory counter is in order) before the next key loads.
  bool pend_ok = false;
  float* pend_ptr = p.out;
  float pend_val = 0.f;
  bool row_ok = false;
  int ti = 0, hg = 0;
  for (;;) {
    int dpage = 0;
    if constexpr (!BIG) {
      if (v >= s1 - s0) break;
      if (task != s0 + v) {
        advance_scan(p, first, c, s0 + v - task);
        task = s0 + v;
      }
      if (p.paged) dpage = __builtin_amdgcn_readlane(pwin, v - wb);
    }
    if (c.b != cur_b || c.j != cur_j) {
      // new tile: its query rows, windows and local_mask anchor
      cur_b = c.b;
      cur_j = c.j;
      pk = 64;
      w = tile_work(p, c, hk, hc);
      const int i0 = c.j * p.tpt;
      ti = n / p.hpt;
      hg = hc * p.hpt + (n - ti * p.hpt);
      row_ok = (n < p.hpt * p.tpt) && (ti < w.ntok) && (hg < p.g);
      lim = row_ok ? last_visible(p, w, i0 + ti) : -1;
      lim_lo = last_visible(p, w, i0);
      start = anchor(w, i0 + ti);
#pragma unroll
      for (int s = 0; s < 4; ++s) qv[s] = i32x4{0, 0, 0, 0};
      if (row_ok) {
        const uint8_t* qr =
            p.q + ((int64_t)(w.t0 + ti) * p.Hq + (hk * p.g + hg)) * kD * Kd::q_bytes;
        if constexpr (Kd::is_fp4) {
          // 32-element group G of the row (B operand) and its scale byte
          const int64_t qrow = (int64_t)(w.t0 + ti) * p.Hq + (hk * p.g + hg);
          qv[0] = ld16(p.q + qrow * (kD / 2) + 16 * G);
          qs = p.q_mx[qrow * (kD / 32) + G];
        } else if constexpr (Kd::is_f8) {
          qv[0] = ld16(qr + 32 * G);
          qv[1] = ld16(qr + 32 * G + 16);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            // 16-bit keys: k step s holds 8-element chunk 4s+G of the row;
            // int8 keys:   chunk 4G+s (a lane's 32 key bytes are contiguous).
            const int ch = Kd::is_i8 ? (4 * G + s) : (4 * s + G);
            qv[s] = ld16(qr + 16 * ch);
          }
        }
      }
    }

    const int beta = c.beta;
    int64_t boff, soff;         // key byte offset, int8 scale element (MXFP4: byte) offset
    if (p.paged) {
      int page = dpage;
      if constexpr (BIG) {
        if (pk == 64) {
          const int bb = beta + 4 * l;
          pidx = consumed(bb < c.nvis ? p.block_table[(int64_t)w.b * p.MB + bb] : 0);
          pk = 0;
        }
        page = __builtin_amdgcn_readlane(pidx, pk);
        ++pk;
      }
      boff = (int64_t)page * p.k_page_stride;
      soff = Kd::is_fp4 ? (int64_t)page * p.mx_page_stride + (int64_t)hk * p.mx_head_stride
                        : (int64_t)page * p.s_page_stride + (int64_t)hk * p.s_head_stride;
    } else {
      boff = (w.koff + (int64_t)beta * kP) * p.k_row_stride;
      soff = Kd::is_fp4
                 ? (w.koff + (int64_t)beta * kP) * p.mx_row_stride + (int64_t)hk * p.mx_head_stride
                 : (w.koff + (int64_t)beta * kP) * p.s_row_stride + (int64_t)hk * p.s_head_stride;
    }
    // wave-uniform block base (scalar registers); per-lane offsets within a
    // block fit 32 bits (checked on the host), which gives the loads the
    // scalar-base + 32-bit-offset form
    const uint8_t* kb = p.k + uniform64(boff + (int64_t)hk * p.k_head_stride);
    const int nvalid = min(kP, w.L - beta * kP);
    const bool full = beta * kP + kP - 1 <= lim_lo;
    // int8: the block's scales, two per lane, issued with the key loads;
    // tokens past kv_len repeat the last valid one's (always in bounds)
    float s_lo = 0.f, s_hi = 0.f;
    if constexpr (Kd::is_i8) {
      const float* sb = p.scale + soff;
      s_lo = sb[(int64_t)min(2 * l, nvalid - 1) * p.s_row_stride];
      s_hi = sb[(int64_t)min(2 * l + 1, nvalid - 1) * p.s_row_stride];
    }

    float m;
    if constexpr (Kd::is_fp4) {
      // MXFP4: instruction s reads tokens 16s..16s+15 whole (64 bytes each,
      // one contiguous KB), lane (n, G) taking 32-element group G of token
      // 16s + n: the A operand of a 16x16x128 scaled MFMA as loaded.  The
      // scale word of the same token holds the four group scales.  Token rows
      // past kv_len re-read the last valid row (in bounds; masked).
      const uint8_t* sb = p.k_mx + uniform64(soff);
      i32x4 a[8];
      uint32_t sw[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int row = min(16 * s + n, nvalid - 1);
        a[s] = ld16_stream(kb + (uint32_t)(row * p.k_row_stride + 16 * G));
        sw[s] = *reinterpret_cast<const uint32_t*>(sb + (uint32_t)(row * p.mx_row_stride));
      }
      auto score = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        float mm = -__builtin_inff();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const f32x4 acc = mfma16x16x128_fp4(a[s], qv[0], f32x4{0.f, 0.f, 0.f, 0.f},
                                              (sw[s] >> (8 * G)) & 255, qs);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jr = 16 * s + 4 * G + r;          // key token of acc[r]
            float v = acc[r];
            if constexpr (MASKED) v = (beta * kP + jr <= lim) ? v : -__builtin_inff();
            mm = fmaxf(mm, v);
          }
        }
        return mm;
      };
      if (pend_ok) *pend_ptr = pend_val;
      take_next();
      m = full ? score(std::false_type{}) : score(std::true_type{});
    } else if constexpr (Kd::is_f8 || Kd::is_i8) {
      // Key loads: instruction i reads rows 8i..8i+7 of the block whole (lane
      // l: row 8i + l/8, 16-byte chunk l%8), eight full 128-byte lines per
      // instruction.  (Loading straight into the MFMA operand layout would
      // touch sixteen half lines per instruction, which measured 16% slower
      // on random pages.)  Token rows past kv_len re-read the last valid row
      // (in bounds; the mask discards them), so every load is unconditional
      // and all of a block's loads are in flight together.
      i32x4 raw[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = min(8 * i + (l >> 3), nvalid - 1);
        raw[i] = ld16_stream(kb + (uint32_t)(row * p.k_row_stride + 16 * (l & 7)));
      }
      if constexpr (Kd::is_i8) {
        *reinterpret_cast<float2*>(&dscl[wave][2 * l]) = float2{s_lo, s_hi};
        wave_lds_sync();
      }
      // MASKED selects -inf for key tokens past the row's last visible one;
      // only blocks cut by the window or by kv_len take it (uniform branch)
      auto score = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        float mm = -__builtin_inff();
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
          // sub-tiles pass through the LDS four at a time (tokens 16jt..16jt+15
          // in area jt % 4): written as loaded, read back as lane (n, G) <-
          // bytes [32G, 32G+32) of token n; 16-byte chunk c of row r sits at
          // chunk c ^ (r & 7)
          uint8_t* area = dkt[wave][jt & 3];
          if ((jt & 3) == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                const int r = 8 * q + (l >> 3);
                *reinterpret_cast<i32x4*>(dkt[wave][u] + r * 128 + (((l & 7) ^ (r & 7)) << 4)) =
                    raw[2 * (jt + u) + q];
              }
            }
            wave_lds_sync();
          }
          i32x4 k0 = *reinterpret_cast<const i32x4*>(area + n * 128 + (((2 * G) ^ (n & 7)) << 4));
          i32x4 k1 = *reinterpret_cast<const i32x4*>(area + n * 128 + (((2 * G + 1) ^ (n & 7)) << 4));
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if constexpr (Kd::is_f8) {
            acc = mfma16x16x128_f8<KK>(cat(k0, k1), cat(qv[0], qv[1]), acc);
          } else {
            i32x4 a0, a1, a2, a3;
            i8x16_to_f16x16(k0, a0, a1);
            i8x16_to_f16x16(k1, a2, a3);
            acc = mfma16x16x32<KF16>(a0, qv[0], acc);
            acc = mfma16x16x32<KF16>(a1, qv[1], acc);
            acc = mfma16x16x32<KF16>(a2, qv[2], acc);
            acc = mfma16x16x32<KF16>(a3, qv[3], acc);
          }
          f32x4 sc4 = {0.f, 0.f, 0.f, 0.f};
          if constexpr (Kd::is_i8)
            sc4 = *reinterpret_cast<const f32x4*>(&dscl[wave][jt * 16 + 4 * G]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jr = jt * 16 + 4 * G + r;         // key token of acc[r]
            float v = acc[r];
            if constexpr (Kd::is_i8) v *= sc4[r];
            if constexpr (MASKED) v = (beta * kP + jr <= lim) ? v : -__builtin_inff();
            mm = fmaxf(mm, v);
          }
        }
        return mm;
      };
      if (pend_ok) *pend_ptr = pend_val;
      take_next();
      m = full ? score(std::false_type{}) : score(std::true_type{});
    } else {
      // instruction i reads rows 4i..4i+3 whole (lane l: row 4i + l/16,
      // 16-byte chunk l%16): eight full lines, as above
      i32x4 raw[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = min(4 * i + (l >> 4), nvalid - 1);
        raw[i] = ld16_stream(kb + (uint32_t)(row * p.k_row_stride + 16 * (l & 15)));
      }
      auto score = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        float mm = -__builtin_inff();
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
          // sub-tiles pass through the LDS four at a time, read back as lane
          // (n, G) <- chunk 4s + G of token n for k step s; chunk c of row r
          // sits at c ^ r
          uint8_t* area = dkt[wave][jt & 3];
          if ((jt & 3) == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int r = 4 * q + (l >> 4);
                *reinterpret_cast<i32x4*>(dkt[wave][u] + r * 256 + (((l & 15) ^ r) << 4)) =
                    raw[4 * (jt + u) + q];
              }
            }
            wave_lds_sync();
          }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const i32x4 kf =
                *reinterpret_cast<const i32x4*>(area + n * 256 + (((4 * s + G) ^ n) << 4));
            acc = mfma16x16x32<KK>(kf, qv[s], acc);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jr = jt * 16 + 4 * G + r;
            float v = acc[r];
            if constexpr (MASKED) v = (beta * kP + jr <= lim) ? v : -__builtin_inff();
            mm = fmaxf(mm, v);
          }
        }
        return mm;
      };
      if (pend_ok) *pend_ptr = pend_val;
      take_next();
      m = full ? score(std::false_type{}) : score(std::true_type{});
    }
    // the four k groups (lanes n + 16 G) hold disjoint key tokens of the
    // same row
    m = max_xor32(max_xor16(m));
    pend_ok = G == 0 && row_ok;
    pend_ptr = p.out + (((int64_t)hk * p.g + hg) * p.T + (w.t0 + ti)) * p.W + beta;
    pend_val = finish(p, w.L, start, beta, true, m);

    if constexpr (BIG) {
      task += 4;
      if (task >= s1) break;
      advance(p, c, 4);
    } else {
      v = vnext;
    }
  }
  if (pend_ok) *pend_ptr = pend_val;
  if constexpr (BIG) {
    fill_pass();
  } else {
    // fill items of the workgroup's range, taken from the second counter by
    // the waves as they run out of blocks; no memory reads
    const int nitems = ntile * kDecodeRows;
    const int fper = (nitems + gu - 1) / gu;
    const int f0 = wi * fper;
    const int f1 = min(nitems, f0 + fper);
    for (int u = __builtin_amdgcn_readfirstlane(wave); f0 + u < f1; u = take(1)) {
      const int it = f0 + u;
      const int k = it / kDecodeRows;
      Cursor cf;
      seek(p, first, k, true, cf);
      fill_item(cf, it - k * kDecodeRows, l, 64);
    }
  }
}

// ---------------------------------------------------------------------------
// prefill
// ---------------------------------------------------------------------------

// floor(r / d) for 0 <= r < 2^16 and 1 <= d < 2^16, without a division per
// call: the high half of r * m with m = recip_small(d) = ceil(2^32 / d) (the
// rounding error of m times r stays below 2^32, so the quotient never reaches
// the next integer); m is 2^32 itself for d = 1.
__device__ __forceinline__ uint64_t recip_small(int d) {
  return (uint64_t)(0xFFFFFFFFu / (uint32_t)d) + 1;
}
__device__ __forceinline__ int div_small(int r, uint64_t m) {
  return (int)(((uint64_t)(uint32_t)r * m) >> 32);
}

// Columns [c_lo, c_hi) (multiples of 4, at most 64 of them) of every output
// row of a prefill work item's tile (at most 512 rows) where no block is
// scored: -inf, with the local_mask constants where the init blocks or a
// row's local window fall (guide to msa_index_score, sections 二 and 四).
// The workgroup walks the (row, 16-byte piece) pairs in order, one store per
// lane, so that an instruction writes consecutive pieces of consecutive rows
// and every lane stores.  With the window at start_loc whether any piece can
// hold a constant is known for the whole item; otherwise per row.  (A loop
// over four rows per wave step, sixteen lanes to a row, with the row's
// division and window recomputed per step, made the items that only write
// fill take ~6% of the varlen MXFP4 prefill.)
__device__ __forceinline__ void fill_tile_columns(const Params& p, const Work& w, int i0,
                                                  int c_lo, int c_hi) {
  const int np4 = (c_hi - c_lo) >> 2;
  if (np4 <= 0) return;
  const int nrows = p.hpt * w.ntok;
  const bool marks = w.L > 0 && (p.init_blocks > 0 || p.local_blocks > 0);
  // the request's window end (per query: from each row's position)
  const int req_anchor = (marks && !p.local_per_query) ? w.sl : -1;
  const bool any_mark =
      marks && (p.local_per_query || c_lo < p.init_blocks ||
                (c_hi > max(0, req_anchor + 1 - p.local_blocks) && c_lo <= req_anchor));
  const uint64_t pinv = recip_small(np4);
  const uint64_t hinv = recip_small(p.hpt);
  float* const base = p.out + (((int64_t)w.hk * p.g + w.hc * p.hpt) * p.T + w.t0) * p.W;
  const int n = nrows * np4;           // below 2^16: 512 rows x 16 pieces at most
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int r = div_small(e, pinv);
    const int q = e - r * np4;
    const int ti = div_small(r, hinv);
    const int hl = r - ti * p.hpt;     // head within the tile's head chunk
    if (w.hc * p.hpt + hl >= p.g) continue;
    const int beta = c_lo + 4 * q;
    f32x4 v = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
    if (any_mark) {
      const int anchor = p.local_per_query ? query_anchor(w, i0 + ti) : req_anchor;
      const int lo = max(0, anchor + 1 - p.local_blocks);
      if (beta < p.init_blocks || (beta + 3 >= lo && beta <= anchor)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = finish(p, w.L, anchor, beta + k, false, 0.f);
      }
    }
    *reinterpret_cast<f32x4*>(base + ((int64_t)hl * p.T + ti) * p.W + beta) = v;
  }
}

template <int KK>
__global__ __launch_bounds__(256, (Kind<KK>::is_i8 || prefill_ntw(KK) >= 3) ? 2 : 3)
void prefill_kernel(Params p) {
  using Kd = Kind<KK>;
  constexpr int NTW = prefill_ntw(KK);
  // Key blocks pass through a two-deep LDS ring of stages, one block per
  // stage (MXFP4: two), so a stage's copy has the previous stage's compute
  // to land: 16-bit keys 32 KB, fp8 16 KB, MXFP4 16 KB (their scales are
  // staged for the whole work item up front), int8 widened to fp16 through
  // registers, 32 KB.  All of it fits two workgroups per CU, three for fp8.
  // (16-bit keys ran stages of 64 tokens in a three-deep ring before:
  // whole-block stages halve the barriers and the per-stage work, and left
  // the LDS room to bank a row's results eight blocks at a time; varlen
  // bf16 prefill 3730 -> 3435 us in one A/B.)
  constexpr int RB = Kd::is_fp4 ? 64 : (Kd::is_f8 ? 128 : 256);   // LDS bytes per key token
  constexpr bool ASYNC = !Kd::is_i8;           // copy HBM/L2 -> LDS directly
  constexpr int BPS = Kd::is_fp4 ? 2 : 1;      // blocks per stage
  constexpr int ST = BPS * kP;                 // tokens per stage
  constexpr int RING = 2;
  constexpr int SBYTES = ST * RB;
  constexpr int NI = SBYTES / 1024 / 4;        // copy instructions per wave per stage
  __shared__ __attribute__((aligned(16))) uint8_t kl[RING * SBYTES];
  __shared__ float scl[Kd::is_i8 ? 2 : 1][Kd::is_i8 ? kP : 1];
  // MXFP4: the scale words of every block of the work item, lane-major:
  // [block][n][mt] holds token 32 mt + n's word, so that lane (n, G) reads its
  // block's four M tiles with one 16-byte LDS read.  Copied once, before the
  // block loop, so that the loop issues no register loads: with register
  // loads in flight beside the LDS copies (and stores) the compiler waits for
  // every memory operation before using them.
  constexpr int CHUNK = prefill_chunk(KK);     // blocks per work item at most
  static_assert(CHUNK <= 64, "page indices are held one per lane");
  __shared__ __attribute__((aligned(16)))
  uint32_t kmx[Kd::is_fp4 ? CHUNK : 1][Kd::is_fp4 ? 32 : 1][Kd::is_fp4 ? 4 : 1];

  const Work w = uniform_work(locate(p));
  if (!w.valid) return;

  const int tid = threadIdx.x;
  // a scalar, so that the LDS destinations of the key copies (which go
  // through M0) are computed in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = lane_id();
  const int n = l & 31;          // row within an N tile / key token within an M tile
  const int G = l >> 5;          // k group, 0..1
  const int i0 = w.t0 - p.cu_q[w.b];

  const int nb = min((w.L + kP - 1) / kP, p.MB);
  const int lim_lo = (w.L > 0 && w.ntok > 0) ? last_visible(p, w, i0) : -1;
  const int lim_hi = (w.L > 0 && w.ntok > 0) ? last_visible(p, w, i0 + w.ntok - 1) : -1;
  const int vend = min(min(w.c1, nb), lim_hi >= 0 ? lim_hi / kP + 1 : 0);
  const bool busy = w.c0 < vend;      // some block of this work item is visible
  if (!busy) {
    // nothing to score: the item's columns are fill only
    fill_tile_columns(p, w, i0, w.c0, w.c1);
    return;
  }

  int lim[NTW];
  i32x4 qv[NTW][8];
  // MXFP4: this lane's query scales, byte s for k step s (the MFMA selects
  // the byte)
  int qsw[NTW];
  const uint64_t hinv = recip_small(p.hpt);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int r = wave * 32 * NTW + nt * 32 + n;
    const int ti = div_small(r, hinv);
    const int hg = w.hc * p.hpt + (r - ti * p.hpt);
    const bool ok = (r < p.hpt * p.tpt) && (ti < w.ntok) && (hg < p.g);
    lim[nt] = ok ? last_visible(p, w, i0 + ti) : -1;
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[nt][s] = i32x4{0, 0, 0, 0};
    qsw[nt] = 0x7F7F;
    if (ok && busy) {
      const int64_t qrow = (int64_t)(w.t0 + ti) * p.Hq + (w.hk * p.g + hg);
      const uint8_t* qr = p.q + qrow * Kd::q_row;
      if constexpr (Kd::is_fp4) {
        // k step s (64 deep) of group G: bytes [32s + 16G, +16), scale 2s + G
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(p.q_mx + qrow * (kD / 32));
#pragma unroll
        for (int s = 0; s < 2; ++s) qv[nt][s] = ld16(qr + 32 * s + 16 * G);
        qsw[nt] = (int)(((sw >> (8 * G)) & 0xFF) | (((sw >> (8 * (2 + G))) & 0xFF) << 8));
      } else if constexpr (Kd::is_f8) {
        // k step s (64 deep) of group G: bytes [64s + 32G, +32)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          qv[nt][2 * s] = ld16(qr + 64 * s + 32 * G);
          qv[nt][2 * s + 1] = ld16(qr + 64 * s + 32 * G + 16);
        }
      } else {
        // k step s (16 deep) of group G: 8-element chunk 2s+G
#pragma unroll
        for (int s = 0; s < 8; ++s) qv[nt][s] = ld16(qr + 16 * (2 * s + G));
      }
    }
  }

  // ---- key block staging into LDS buffer `buf` -------------------------
  // LDS layout: token jj's 16-byte chunk c sits at jj*RB + ((c ^ swz(jj)) << 4)
  // with swz(jj) = jj & 15 (256-byte rows) or (jj >> 1) & 7 (128-byte rows),
  // so the 32 tokens an MFMA operand read touches hit distinct banks.
  // fp16/bf16/fp8: each wave instruction copies 1 KB straight from HBM/L2 into
  // LDS (global_load_lds, no registers); LDS receives lane l's 16 bytes at
  // base + 16*l, so the swizzle is applied to the global address instead.
  // int8: loaded to registers, widened to fp16, written with the swizzle.
  // page indices of the work item's blocks, one per lane, read with readlane
  int pidx = 0;
  if (p.paged && busy && l < vend - w.c0) pidx = p.block_table[(int64_t)w.b * p.MB + w.c0 + l];
  auto block_bytes = [&](int beta) -> int64_t {
    if (p.paged) return (int64_t)__builtin_amdgcn_readlane(pidx, beta - w.c0) * p.k_page_stride;
    return (w.koff + (int64_t)beta * kP) * p.k_row_stride;
  };
  auto block_scale = [&](int beta) -> int64_t {
    if (p.paged)
      return (int64_t)__builtin_amdgcn_readlane(pidx, beta - w.c0) * p.s_page_stride +
             (int64_t)w.hk * p.s_head_stride;
    return (w.koff + (int64_t)beta * kP) * p.s_row_stride + (int64_t)w.hk * p.s_head_stride;
  };

  i32x4 st[4];
  float sv = 0.f;
  // stage sg (block c0 + sg; MXFP4 blocks c0 + 2 sg, + 1) into ring slot `slot`;
  // always exactly NI copy instructions per wave (the ring's waits count
  // them): token rows at or past kv_len copy row 0 of the block instead, which
  // the masked path discards
  // copy instruction q of stage sg
  constexpr int RPI = 1024 / RB;                    // tokens per copy instruction
  // This lane's byte offset within a stage for each of its wave's copy
  // instructions (token jl of the stage, swizzled 16-byte chunk c), computed
  // once per work item.
  // The swizzle repeats every 16 rows and a wave's copies are RPI rows apart,
  // so copies 16 / RPI apart share a pattern: that many offsets (4 for
  // 16-bit keys, 2 for fp8, 1 for MXFP4) and a row offset for the rest.
  constexpr int NCOF = ASYNC ? (NI < 16 / RPI ? NI : 16 / RPI) : 1;
  uint32_t cof[NCOF];
#pragma unroll
  for (int q = 0; q < NCOF; ++q) {
    // (MXFP4: token jl of the stage's two blocks, row jl mod 128 of its block)
    const int jl = (wave * NI + q) * RPI + l / (RB / 16);
    const int jb = Kd::is_fp4 ? (jl & (kP - 1)) : jl;
    const int c = (l % (RB / 16)) ^
                  (RB == 256 ? (jb & 15) : RB == 128 ? ((jb >> 1) & 7) : ((jb >> 2) & 3));
    cof[q] = (uint32_t)(jb * p.k_row_stride + 16 * c);
  }
  // Copy instruction q of stage sg, through a raw buffer over the block's
  // rows below kv_len (its size nvalid rows): lanes of rows at or past
  // kv_len read zeros, which only blocks that take the masked path contain.
  // No per-copy branch or clamp; the block base and LDS destination are
  // scalar values.
  // (MXFP4: a stage is blocks c0 + 2 sg and c0 + 2 sg + 1; waves 0-1 copy
  // the first, 2-3 the second, from the block base `kbytes` of their own
  // block, which may lie past the request's last block: then nothing is read)
  auto stage_copy = [&](int q, int sg, int slot, int64_t kbytes) {
    const int beta = Kd::is_fp4 ? w.c0 + BPS * sg + (wave >> 1) : w.c0 + sg;
    // offsets within a block fit 32 bits (checked on the host)
    const uint8_t* kb = p.k + uniform64(kbytes + (int64_t)w.hk * p.k_head_stride);
    // (a scalar: computed in vector registers, the buffer descriptor made the
    // compiler wrap each copy in a loop over lanes)
    const int nvalid = __builtin_amdgcn_readfirstlane(max(0, min(kP, w.L - beta * kP)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kb), 0, nvalid * p.k_row_stride, kBufferWord3);
    const int X = wave * NI + q;
    const uint32_t co = cof[q % NCOF] + (uint32_t)((q / NCOF) * 16 * p.k_row_stride);
    buffer_copy16_lds(rs, kl + slot * SBYTES + X * 1024, co);
  };
  // MXFP4: the scale words of the work item's nblk blocks, copied straight
  // into kmx: two copies per block, wave w taking blocks w, w + 4, ...; lane
  // l of copy k loads token 32 (l & 3) + 16 k + (l >> 2), whose word lands at
  // slot 64 k + l = 4 n + mt of the block's [n][mt] area.  The buffer ends at
  // the block's last row below kv_len, so rows past it read zeros (their
  // scores are masked).  (Register loads and LDS stores took 24 loads per
  // lane before the first block: 2-4% of the MXFP4 prefill.)
  auto stage_scales = [&](int nblk) {
    const uint32_t tof = (uint32_t)((32 * (l & 3) + (l >> 2)) * p.mx_row_stride);
    const uint32_t tof16 = tof + 16u * (uint32_t)p.mx_row_stride;
    for (int bi = wave; bi < nblk; bi += kPrefillWaves) {
      const int beta = w.c0 + bi;
      const int64_t base =
          (p.paged ? (int64_t)__builtin_amdgcn_readlane(pidx, bi) * p.mx_page_stride
                   : (w.koff + (int64_t)beta * kP) * p.mx_row_stride) +
          (int64_t)w.hk * p.mx_head_stride;
      const int nvalid = min(kP, w.L - beta * kP);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(p.k_mx + uniform64(base)), 0,
          (nvalid - 1) * p.mx_row_stride + 4, kBufferWord3);
      uint8_t* const dst = reinterpret_cast<uint8_t*>(kmx) + bi * 512;
      buffer_copy4_lds(rs, dst, tof);
      buffer_copy4_lds(rs, dst + 256, tof16);
    }
  };
  auto stage_async = [&](int sg, int slot, int64_t kbytes) {
#pragma unroll
    for (int q = 0; q < NI; ++q) stage_copy(q, sg, slot, kbytes);
  };
  auto gload_i8 = [&](int beta) {
    const uint8_t* kb = p.k + block_bytes(beta) + (int64_t)w.hk * p.k_head_stride;
    const int nvalid = min(kP, w.L - beta * kP);
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const int jj = ps * 32 + (tid >> 3);
      st[ps] = (jj < nvalid) ? ld16(kb + (int64_t)jj * p.k_row_stride + 16 * (tid & 7))
                             : i32x4{0, 0, 0, 0};
    }
    if (tid < kP)
      sv = (tid < nvalid) ? p.scale[block_scale(beta) + (int64_t)tid * p.s_row_stride] : 0.f;
  };
  auto lstore_i8 = [&](int slot) {
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const int jj = ps * 32 + (tid >> 3);
      const int sc = tid & 7;
      i32x4 a, b;
      i8x16_to_f16x16(st[ps], a, b);
      uint8_t* row = kl + slot * SBYTES + jj * 256;
      *reinterpret_cast<i32x4*>(row + (((2 * sc) ^ (jj & 15)) << 4)) = a;
      *reinterpret_cast<i32x4*>(row + (((2 * sc + 1) ^ (jj & 15)) << 4)) = b;
    }
    if (tid < kP) scl[slot][tid] = sv;
  };

  // The output rows this lane writes: after the cross-half reduction both k
  // groups hold every N tile's results; lanes of group G write N tiles G,
  // G + 2, ...  Each block's result is stored soon after it is known (the L2
  // merges a row's columns).
  constexpr int NOUT = (NTW + 1) / 2;
  bool orow_ok[NOUT];
  float* orow_ptr[NOUT];
  int oanc[NOUT];               // last block of each output row's local window
#pragma unroll
  for (int u = 0; u < NOUT; ++u) {
    const int orow = wave * 32 * NTW + (G + 2 * u) * 32 + n;
    const int oti = div_small(orow, hinv);
    const int ohg = w.hc * p.hpt + (orow - oti * p.hpt);
    orow_ok[u] = G + 2 * u < NTW && orow < p.hpt * p.tpt && oti < w.ntok && ohg < p.g;
    orow_ptr[u] = p.out + (((int64_t)w.hk * p.g + ohg) * p.T + (w.t0 + oti)) * p.W;
    oanc[u] = p.local_per_query ? query_anchor(w, i0 + oti) : w.sl;
  }

  const int nst = busy ? vend - w.c0 : 0;   // blocks of this work item (stages but MXFP4)
  if constexpr (ASYNC) {
    // the first block's page index is read before any copy is in flight
    // (MXFP4: the wave's own block of the first stage)
    const int64_t kb0 = nst > 0 ? block_bytes(w.c0 + (Kd::is_fp4 ? (wave >> 1) : 0)) : 0;
    if constexpr (Kd::is_fp4) {
      if (nst > 0) stage_scales(vend - w.c0);
    }
    if (nst > 0) stage_async(0, 0, kb0);
    // (the loop's first barrier makes every wave's writes visible)
  } else {
    if (nst > 0) {
      gload_i8(w.c0);
      lstore_i8(0);
    }
  }
  // running block maxima, one per N tile; a vector value rather than an
  // array, so that picking a lane's output tile cannot become a private
  // memory access (which the ring's memory-counter waits would wait on)
  static_assert(NTW <= 4, "running maxima are held in a four-wide vector");
  f32x4 run;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) run[nt] = -__builtin_inff();
  // Block results of this lane's row collect RG blocks at a time and are
  // written as RG consecutive floats (16-byte stores).  16-bit keys and
  // MXFP4: a block's result for each output row goes to a per-wave LDS area,
  // one store per row, and the flush reads a row's RG values back (in
  // registers, choosing the register of a block by its uniform but not
  // constant position in the group takes a select per register and row, and
  // the registers of 16-bit keys are full); groups of 8 blocks keep two
  // workgroups within a CU's LDS.  fp8 and int8 hold 16 in registers (for fp8
  // an LDS area made the compiler wait for the next stage's copies before
  // fragment reads in the block loop).
  constexpr bool LDS_RES = Kd::is_fp4 || (ASYNC && RB == 256);
  constexpr int RG = LDS_RES ? 8 : 16;
  __shared__ float resl[LDS_RES ? kPrefillWaves : 1][LDS_RES ? NOUT : 1][LDS_RES ? RG : 1][64];
  float resv[NOUT][LDS_RES ? 1 : RG];
  int pend = -1;                 // first block of a group waiting to be written
  // Whether a column of the group can hold a local_mask constant is, with
  // the window at start_loc, the same for every row of the item: groups that
  // miss both windows skip the per-column rule.
  const bool marks = w.L > 0 && (p.init_blocks > 0 || p.local_blocks > 0);
  auto flush = [&](int g0) {
    auto write = [&](auto rule) {
#pragma unroll
      for (int u = 0; u < NOUT; ++u) {
        if (orow_ok[u]) {
#pragma unroll
          for (int c = 0; c < RG; c += 4) {
            if (g0 + c < w.c1) {
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int beta = g0 + c + e;
                float r;
                if constexpr (LDS_RES)
                  r = resl[wave][u][c + e][l];
                else
                  r = resv[u][c + e];
                if constexpr (decltype(rule)::value)
                  v[e] = finish(p, w.L, oanc[u], beta, beta < vend, r);
                else
                  v[e] = beta < vend ? r : -__builtin_inff();
              }
              *reinterpret_cast<f32x4*>(orow_ptr[u] + g0 + c) = v;
            }
          }
        }
      }
    };
    if (marks && (p.local_per_query || g0 < p.init_blocks ||
                  (g0 + RG > max(0, w.sl + 1 - p.local_blocks) && g0 <= w.sl)))
      write(std::true_type{});
    else
      write(std::false_type{});
  };
  if constexpr (Kd::is_fp4) {
    // Stages of two blocks, A = c0 + 2 sg and B = A + 1 (B may lie past the
    // item's last block; its results are then dropped).  The 32-token M
    // tiles of the two blocks alternate (A0 B0 A1 B1 ...), A's on accumulator
    // set 0 and B's on set 1, and a tile's maxima are taken while the next
    // tile's MFMAs run, so that only B's last tile ends the stage with vector
    // work waiting on its own MFMAs; one barrier per two blocks.
    const int nst2 = (vend - w.c0 + 1) >> 1;
    f32x4 run2[2];
    f32x16 acc2[2][NTW];
    auto finalize2 = [&](int bis, int bb) {
      const int kk = (bb - w.c0) % RG;
      // lanes of group G write N tile 2u + G: one swap and maximum per pair
#pragma unroll
      for (int u = 0; u < NOUT; ++u)
        resl[wave][u][kk][l] = max_pair32(run2[bis][2 * u],
                                          run2[bis][2 * u + 1 < NTW ? 2 * u + 1 : 2 * u]);
      if (kk == RG - 1 || bb == vend - 1) pend = bb - kk;
    };
    for (int sg = 0; sg < nst2; ++sg) {
      const int slot = sg & 1;
      const int beta0 = w.c0 + 2 * sg;
      const bool hasB = beta0 + 1 < vend;
      // this stage has landed (every wave's copies) and every wave is done
      // with the slot the copy below refills
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (pend >= 0) {
        flush(pend);
        pend = -1;
      }
      const int csg = sg + 1;
      const bool copy_next = csg < nst2;
      const int64_t ckb = copy_next ? block_bytes(w.c0 + 2 * csg + (wave >> 1)) : 0;
      const uint8_t* kc = kl + slot * SBYTES;
#pragma unroll
      for (int bis = 0; bis < 2; ++bis) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) run2[bis][nt] = -__builtin_inff();
      }
      const bool unmasked = (hasB ? beta0 + 1 : beta0) * kP + kP - 1 <= lim_lo;
      auto stage = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        constexpr int NFR = 16;      // (M tile, block, k step), k step fastest
        // fragments read ahead: four (one more spills the masked variant,
        // whose mask tests hold more registers; it reads two ahead)
        constexpr int LEAD = MASKED ? 2 : 4;
        auto frag = [&](int i) -> i32x4 {
          const int mt = i >> 2, bis = (i >> 1) & 1, q = i & 1;
          const int jj = mt * 32 + n;
          const int c = 2 * q + G;   // bytes [32q + 16G, +16) of the token
          return *reinterpret_cast<const i32x4*>(kc + bis * (kP * RB) + jj * RB +
                                                  ((c ^ ((jj >> 2) & 3)) << 4));
        };
        i32x4 f[NFR];
#pragma unroll
        for (int i = 0; i < LEAD; ++i) f[i] = frag(i);
        // the two blocks' scale words, token 32 mt + n in word mt, shifted
        // so that byte 2q is this lane's group 2q + G (the MFMA selects it)
        uint32_t ksw[2][4];
#pragma unroll
        for (int bis = 0; bis < 2; ++bis) {
          const uint4 kw =
              *reinterpret_cast<const uint4*>(&kmx[min(beta0 + bis - w.c0, CHUNK - 1)][n][0]);
          const int sh = 8 * G;
          ksw[bis][0] = kw.x >> sh;
          ksw[bis][1] = kw.y >> sh;
          ksw[bis][2] = kw.z >> sh;
          ksw[bis][3] = kw.w >> sh;
        }
        // a[nt][r] is key token 32 mt + 8 (r / 4) + 4 G + r % 4 of the block
        // for row n of N tile nt; masked: kept iff at most the row's last
        // visible token, i.e. 8 (r / 4) + r % 4 <= lim - (block start + 32 mt
        // + 4 G)
        auto tile_max = [&](const f32x16 (&a)[NTW], int bis, int mt, int nt0, int nt1) {
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
            if (nt < nt0 || nt >= nt1) continue;
            const int vis = MASKED ? lim[nt] - ((beta0 + bis) * kP + mt * 32 + 4 * G) : 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float v = a[nt][r];
              if constexpr (MASKED) v = (8 * (r >> 2) + (r & 3) <= vis) ? v : -__builtin_inff();
              run2[bis][nt] = fmaxf(run2[bis][nt], v);
            }
          }
        };
#pragma unroll
        for (int i = 0; i < NFR; ++i) {
          if (copy_next && i == 0) {
#pragma unroll
            for (int q = 0; q < NI; ++q) stage_copy(q, csg, csg & 1, ckb);
          }
          if (i + LEAD < NFR) f[i + LEAD] = frag(i + LEAD);
          const int mt = i >> 2, bis = (i >> 1) & 1, q = i & 1, k = i >> 1;
          f32x16 (&ac)[NTW] = acc2[bis];
          if (q == 0) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) ac[nt] = f32x16{};
          }
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
            ac[nt] = q == 0
                ? mfma32x32x64_fp4_sel<0, 0>(f[i], qv[nt][0], ac[nt], ksw[bis][mt], qsw[nt])
                : mfma32x32x64_fp4_sel<2, 1>(f[i], qv[nt][1], ac[nt], ksw[bis][mt], qsw[nt]);
          if (k > 0) {
            // tile k - 1 (the other block's), half of its N tiles per fragment
            const int pb = (k - 1) & 1, pm = (k - 1) >> 1;
            if (q == 0)
              tile_max(acc2[pb], pb, pm, 0, NTW / 2);
            else
              tile_max(acc2[pb], pb, pm, NTW / 2, NTW);
          }
          if (i == NFR - 1) tile_max(ac, 1, 3, 0, NTW);
          if constexpr (!MASKED) {
            // one MFMA, then four of the previous tile's maxima (v_max3),
            // so that a wave's vector work issues while its own MFMAs run
            if (k > 0) {
#pragma unroll
              for (int kk = 0; kk < NTW; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
              }
            }
          }
          // keep this shape: one fragment read, its MFMAs, (an epilogue)
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (unmasked)
        stage(std::false_type{});
      else
        stage(std::true_type{});
      finalize2(0, beta0);
      if (hasB) finalize2(1, beta0 + 1);
    }
    if (pend >= 0) flush(pend);
  } else {
    for (int sg = 0; sg < nst; ++sg) {
      const int slot = sg % RING;
      const int beta = w.c0 + sg;
      // Stage sg has landed (every wave's copies) and every wave is done with
      // the slot the copy below reuses.  Written out because __syncthreads()
      // leaves the wait to the compiler.
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // a finished group of results is written here, ahead of the next
      // copies, so that the copies stay the newest memory operations the
      // waits count
      if (pend >= 0) {
        flush(pend);
        pend = -1;
      }
      // The copy of stage sg + 1 (into the slot every wave has just left) is
      // issued from inside this stage's compute, spread over it where
      // registers allow: issued all at once after the barrier, the copies of a
      // workgroup's four waves stalled instruction issue for hundreds of
      // cycles.
      const int csg = sg + 1;
      const bool copy_next = csg < nst;
      const int64_t ckb = (ASYNC && copy_next) ? block_bytes(w.c0 + csg) : 0;
      if constexpr (!ASYNC) {
        if (copy_next) gload_i8(beta + 1);
      }
      const uint8_t* kc = kl + slot * SBYTES;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) run[nt] = -__builtin_inff();
      // One pass over the block's four 32-token M tiles; MASKED selects -inf for
      // key tokens past each row's last visible one (only blocks cut by the
      // window or by kv_len need it).  The branch below is uniform per block.
      auto block = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        // Key fragments (MFMA A operand), 16 bytes each, in the order they are
        // consumed: M tile mt (32 tokens), k step s, and for fp8 the two halves
        // of a 32-byte operand.  Fragment i + LEAD is read from LDS while
        // fragment i feeds the MFMAs, which hides the LDS latency with only
        // LEAD + 1 fragments live.
        constexpr int PER_MT = Kd::is_f8 ? 4 : 8;   // fragments per M tile
        constexpr int NFR = (ST / 32) * PER_MT;
        constexpr int LEAD = Kd::is_f8 ? 4 : (NTW >= 3 ? 1 : 2);
        auto frag = [&](int i) -> i32x4 {
          const int mt = i / PER_MT, q = i % PER_MT;
          const int jj = mt * 32 + n;
          if constexpr (Kd::is_f8) {
            // q = 2*s + half: bytes [64s + 32G + 16*half, +16) of the token
            const int c = 4 * (q >> 1) + 2 * G + (q & 1);
            return *reinterpret_cast<const i32x4*>(kc + jj * 128 + ((c ^ ((jj >> 1) & 7)) << 4));
          } else {
            const int c = 2 * q + G;
            return *reinterpret_cast<const i32x4*>(kc + jj * 256 + ((c ^ (jj & 15)) << 4));
          }
        };
        i32x4 f[NFR];
#pragma unroll
        for (int i = 0; i < LEAD; ++i) f[i] = frag(i);
        f32x16 acc[NTW];
#pragma unroll
        for (int i = 0; i < NFR; ++i) {
          if constexpr (ASYNC) {
            // copy points per stage: two for 16-bit keys; one for fp8, whose
            // three waves per SIMD leave no registers for more
            constexpr int CPTS = RB == 256 ? 2 : 1;
            static_assert(NFR % CPTS == 0 && NI % CPTS == 0, "copies spread evenly");
            if (copy_next && i % (NFR / CPTS) == 0) {
#pragma unroll
              for (int q = 0; q < NI / CPTS; ++q)
                stage_copy((i / (NFR / CPTS)) * (NI / CPTS) + q, csg, csg % RING, ckb);
            }
          }
          if (i + LEAD < NFR) f[i + LEAD] = frag(i + LEAD);
          const int mt = i / PER_MT, q = i % PER_MT;
          if (q == 0) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) acc[nt] = f32x16{};
          }
          if constexpr (Kd::is_f8) {
            if (q & 1) {
              const int s = q >> 1;
              const i32x8 a = cat(f[i - 1], f[i]);
#pragma unroll
              for (int nt = 0; nt < NTW; ++nt)
                acc[nt] = mfma32x32x64_f8<KK>(a, cat(qv[nt][2 * s], qv[nt][2 * s + 1]), acc[nt]);
            }
          } else {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
              acc[nt] = mfma32x32x16<Kd::mfma_kind>(f[i], qv[nt][q], acc[nt]);
          }
          if (q == PER_MT - 1) {
            // acc[nt][r] holds key token mt*32 + 8*(r/4) + 4*G + r%4 of row n
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int jr = mt * 32 + 8 * (r >> 2) + 4 * G + (r & 3);
              float sc = 1.f;
              if constexpr (Kd::is_i8) sc = scl[slot][jr];
#pragma unroll
              for (int nt = 0; nt < NTW; ++nt) {
                float v = acc[nt][r];
                if constexpr (Kd::is_i8) v *= sc;
                if constexpr (MASKED) {
                  const int j = beta * kP + jr;
                  v = (j <= lim[nt]) ? v : -__builtin_inff();
                }
                run[nt] = fmaxf(run[nt], v);
              }
            }
          }
          // keep this shape: one fragment read, its MFMAs, (an epilogue); the
          // compiler would otherwise hoist every read and run out of registers
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (beta * kP + kP - 1 <= lim_lo)
        block(std::false_type{});
      else
        block(std::true_type{});

      {
        // the two k groups hold the two halves of each 32-token M tile; lanes
        // of group G write N tile 2u + G: one swap and maximum per pair
        const int kk = (beta - w.c0) % RG;
#pragma unroll
        for (int u = 0; u < NOUT; ++u) {
          const float v = max_pair32(run[2 * u], run[2 * u + 1 < NTW ? 2 * u + 1 : 2 * u]);
          if constexpr (LDS_RES) {
            resl[wave][u][kk][l] = v;
          } else {
#pragma unroll
            for (int k = 0; k < RG; ++k) resv[u][k] = (k == kk) ? v : resv[u][k];
          }
        }
        if (kk == RG - 1 || beta == vend - 1) pend = beta - kk;
      }
      if constexpr (!ASYNC) {
        if (sg + 1 < nst) lstore_i8(slot ^ 1);
      }
    }

    if (pend >= 0) flush(pend);
  }
  // columns of the work item past the last group: -inf and local_mask
  fill_tile_columns(p, w, i0, w.c0 + ((vend - w.c0 + RG - 1) / RG) * RG, w.c1);
}

}  // namespace msa
