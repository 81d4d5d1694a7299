// Device-side building blocks of the MSA index-score kernels (gfx950 only).
//
// Terms used below.  A "block" is one logical KV block of P = 128 tokens
// (one physical page for paged keys).  A "row" is one (query token, index
// head) pair; the heads of one KV group are the rows that share a key
// (gitcode cann/ops-transformer issue #4117, section 计算过程: h_kv = h / g).
// Scores S = K . Q^T are taken on MFMA with the key tokens j as the M side and
// the rows as the N side, so each lane ends up holding several j of one row in
// registers and the block maximum is mostly an in-register reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kP = 128;   // tokens per logical block
constexpr int kD = 128;   // index head dimension

// Element kinds of the key (the query kind follows from it).
enum KeyKind : int { KF16 = 0, KBF16 = 1, KI8 = 2, KF8E4M3 = 3, KF8E5M2 = 4, KMXFP4 = 5 };

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// Everything a launch needs; built and validated on the host.
struct Params {
  const uint8_t* q;            // query [T, Hq, D]
  const uint8_t* k;            // key (layout per the strides below)
  const float* scale;          // int8 dequant scale or nullptr
  const int32_t* block_table;  // [B, MB] (paged) or nullptr
  const int32_t* cu_q;         // [B+1]
  const int32_t* kv_len;       // [B]
  const int32_t* start_loc;    // [B]
  float* out;                  // [Hq, T, W]
  int64_t k_page_stride;       // bytes between physical pages (paged)
  int32_t k_row_stride;        // bytes between consecutive key tokens
  int32_t k_head_stride;       // bytes between KV heads
  int64_t s_page_stride;       // scale elements between pages (paged)
  int32_t s_row_stride;        // scale elements between tokens
  int32_t s_head_stride;       // scale elements between KV heads
  // MXFP4: E8M0 scales, one byte per 32 elements, a token row's D/32 bytes
  // contiguous; query [T, Hq, D/32]; key strides in bytes (page by logical
  // page index)
  const uint8_t* q_mx;
  const uint8_t* k_mx;
  int64_t mx_page_stride;
  int32_t mx_row_stride, mx_head_stride;
  int64_t T;
  int32_t B, Hq, Hkv, g;
  int32_t MB, W;
  int32_t paged, causal;
  int32_t init_blocks, local_blocks;
  int32_t local_per_query;     // 1: the local window ends at each token's own block
  int32_t hpt;                 // heads of a KV group per tile
  int32_t tpt;                 // query tokens per tile
  int32_t hchunks;             // ceil(g / hpt)
  int32_t chunk;               // blocks per work item
  int32_t nchunks;             // ceil(W / chunk)
  int32_t units;               // Hkv * hchunks * nchunks
  int32_t ntiles;              // upper bound of token tiles over the batch
};

// ---------------------------------------------------------------------------
// wave-level helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum over the wave's 64 lanes, by DPP steps with no LDS
// round trip: row_shr 1, 2, 4, 8 within each row of 16 lanes (a lane whose
// source lies before its row adds 0), then row_bcast:15 adds lane 15's sum to
// rows 1 and 3 and row_bcast:31 lane 31's to rows 2 and 3.  (Every lane of the
// wave must be active.)
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_or_zero(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int64_t dpp_or_zero(int64_t v) {
  const uint32_t lo = (uint32_t)dpp_or_zero<CTRL, ROWS>((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)dpp_or_zero<CTRL, ROWS>((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T x) {
  x += dpp_or_zero<0x111, 0xF>(x);
  x += dpp_or_zero<0x112, 0xF>(x);
  x += dpp_or_zero<0x114, 0xF>(x);
  x += dpp_or_zero<0x118, 0xF>(x);
  x += dpp_or_zero<0x142, 0xA>(x);
  x += dpp_or_zero<0x143, 0xC>(x);
  return x;
}

// Lane src's value (src the same in every lane), through v_readlane.
__device__ __forceinline__ int lane_at(int x, int src) {
  return __builtin_amdgcn_readlane(x, src);
}
__device__ __forceinline__ int64_t lane_at(int64_t x, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), src);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Value of another lane in the same row of 16, by a DPP lane pattern.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Smallest value of x and largest value of y over the whole wave (every
// lane active): within each row of 16 lanes by swapping neighbours, then
// quads, then mirroring half rows and rows; then over the four rows.
__device__ __forceinline__ void wave_min_max(uint32_t x, uint32_t y, uint32_t& lo, uint32_t& hi) {
  uint32_t a = x, b = y;
  a = min(a, dpp_u32<0xB1>(a));    // quad_perm 1,0,3,2
  b = max(b, dpp_u32<0xB1>(b));
  a = min(a, dpp_u32<0x4E>(a));    // quad_perm 2,3,0,1
  b = max(b, dpp_u32<0x4E>(b));
  a = min(a, dpp_u32<0x141>(a));   // row_half_mirror
  b = max(b, dpp_u32<0x141>(b));
  a = min(a, dpp_u32<0x140>(a));   // row_mirror
  b = max(b, dpp_u32<0x140>(b));
  auto lane = [](uint32_t v, int i) { return (uint32_t)__builtin_amdgcn_readlane((int)v, i); };
  lo = min(min(lane(a, 0), lane(a, 16)), min(lane(a, 32), lane(a, 48)));
  hi = max(max(lane(b, 0), lane(b, 16)), max(lane(b, 32), lane(b, 48)));
}

// max(x[l], x[l ^ 32]) in every lane l: v_permlane32_swap exchanges the
// upper half of its first register with the lower half of its second, so two
// copies of x become the two halves side by side, and one v_max_f32 combines
// them.  (Written out: clang's builtin for the swap loses its second result
// in this toolchain, and a separate fmaxf on asm results adds canonicalising
// maxima.)  The nops are the wait states around the cross-lane operation.
__device__ __forceinline__ float max_xor32(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a);
}

// Lanes 0-31: max(a[l], a[l + 32]); lanes 32-63: max(b[l - 32], b[l]).  The
// swap puts the upper half of a beside the lower half of b, so the lower
// lanes hold both halves of a and the upper lanes both halves of b, and one
// v_max_f32 finishes both (half the work of max_xor32 on each).
__device__ __forceinline__ float max_pair32(float a, float b) {
  uint32_t x = __builtin_bit_cast(uint32_t, a), y = __builtin_bit_cast(uint32_t, b);
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(x), "+v"(y));
  return __builtin_bit_cast(float, x);
}

// max(x[l], x[l ^ 16]) in every lane l: v_permlane16_swap exchanges the odd
// rows (16 lanes each) of its first register with the even rows of its
// second, so two copies of x become each row pair's two rows side by side,
// and one v_max_f32 combines them (written out as max_xor32 is).
__device__ __forceinline__ float max_xor16(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a);
}

// Fourth word of a raw buffer descriptor on this architecture (32-bit data
// format; stride 0 makes the size a byte count checked per access, and
// accesses past it read zeros).
constexpr int kBufferWord3 = 0x00020000;

// One 16-byte piece per lane from a raw buffer (byte offset voff) straight
// into LDS: lane l's piece lands at lds + 16 l (the base goes through M0).
// (A helper of its own: called from a lambda inside a kernel template, the
// builtin made the host pass drop that kernel's launch stub.)
__device__ __forceinline__ void buffer_copy16_lds(__amdgpu_buffer_rsrc_t rs, uint8_t* lds,
                                                  uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// One 4-byte word per lane from a raw buffer straight into LDS: lane l's
// word lands at lds + 4 l.
__device__ __forceinline__ void buffer_copy4_lds(__amdgpu_buffer_rsrc_t rs, uint8_t* lds,
                                                 uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 4,
                                           voff, 0, 0, 0);
}

__device__ __forceinline__ i32x4 ld16(const uint8_t* p) {
  return *reinterpret_cast<const i32x4*>(p);
}

// Streaming load for data read once per launch (decode key blocks): the
// nontemporal hint keeps single-use lines from displacing reused ones in the
// caches, which on MI355X more than doubles the rate of random 32 KB block
// reads compared with plain loads.
__device__ __forceinline__ i32x4 ld16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}

// A loaded value, waited for here.  Used on rare paths inside the decode
// loop (new tile, new request): without it the compiler may place the wait
// for such a load after the branch, on every iteration, where (the memory
// counter being in order) it would also wait for the previous block's result
// store.
__device__ __forceinline__ int consumed(int v) {
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"(v));
  return v;
}

// A value every lane of the wave holds, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Keeps this wave's LDS stores ahead of its following LDS loads in the
// instruction stream; the LDS executes one wave's operations in order, so the
// loads then see the stores of every lane of the wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Work decomposition.
//
// A work item is (unit, tile): a unit is (KV head, head chunk, block chunk),
// a tile is `tpt` consecutive query tokens of one request.  The hardware
// hands workgroups to the eight XCDs round-robin by workgroup id, so the id is
// remapped such that each XCD walks runs of eight consecutive tiles of one
// unit: the workgroups of a run start together and read the same key blocks
// through that XCD's L2.  Successive runs of a unit go to successive XCDs,
// which deals every unit's work over all eight.  (Keeping each unit on one
// XCD would give the most L2 reuse, but under the causal window low block
// chunks carry far more work than high ones, and the XCDs holding them would
// finish last.)
// ---------------------------------------------------------------------------

struct Work {
  int valid;
  int hk, hc, c0, c1;          // KV head, head chunk, block range [c0, c1)
  int b, t0, ntok;             // request, first token, tokens in the tile
  int Lq, L;                   // query length and kv_len of the request
  int64_t koff;                // packed-key offset of the request (TND)
  int sl;                      // start_loc of the request (prefill items; read
                               // with the lookup, not with the per-query window)
};

__device__ __forceinline__ Work locate(const Params& p) {
  Work w;
  w.valid = 0;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int ui = slot / p.ntiles;
  const int tile = slot - ui * p.ntiles;
  const int unit = ui * 8 + ((xcd + tile / 8) & 7);
  if (unit >= p.units) return w;
  w.hk = unit / (p.hchunks * p.nchunks);
  const int rem = unit - w.hk * (p.hchunks * p.nchunks);
  w.hc = rem / p.nchunks;
  const int ch = rem - w.hc * p.nchunks;
  w.c0 = ch * p.chunk;
  w.c1 = min(w.c0 + p.chunk, p.W);

  // Find the request holding `tile`: a wave-wide prefix sum of the per-request
  // tile counts ceil(L_q / tpt), 64 requests at a time.
  const int l = lane_id();
  int acc = 0;
  int64_t kacc = 0;
  for (int base = 0; base < p.B; base += 64) {
    const int b = base + l;
    int lq = 0, kv = 0, sl = -1;
    if (b < p.B) {
      lq = p.cu_q[b + 1] - p.cu_q[b];
      kv = p.kv_len[b];
      if (!p.local_per_query) sl = p.start_loc[b];
    }
    const int n = (lq + p.tpt - 1) / p.tpt;
    const int incl = wave_incl_scan(n);
    const int64_t kincl = wave_incl_scan((int64_t)kv);
    const int total = lane_at(incl, 63);
    if (tile < acc + total) {
      const unsigned long long m = __ballot(acc + incl > tile);
      const int src = __ffsll((long long)m) - 1;
      const int n_s = lane_at(n, src);
      const int incl_s = lane_at(incl, src);
      const int kv_s = lane_at(kv, src);
      const int64_t kincl_s = lane_at(kincl, src);
      w.b = base + src;
      const int tin = tile - (acc + incl_s - n_s);
      w.Lq = lane_at(lq, src);
      w.L = kv_s;
      w.t0 = p.cu_q[w.b] + tin * p.tpt;
      w.ntok = min(p.tpt, w.Lq - tin * p.tpt);
      w.koff = kacc + kincl_s - kv_s;
      w.sl = lane_at(sl, src);
      w.valid = 1;
      return w;
    }
    acc += total;
    kacc += lane_at(kincl, 63);
  }
  return w;
}

// The work item with every field in scalar registers.  locate() broadcasts
// them from one lane with shuffles, which leaves them in vector registers;
// values derived from them (block bases, kv_len tests) are then vector values
// too, and branches on them run both ways under lane masks.
__device__ __forceinline__ Work uniform_work(Work w) {
  auto u = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  w.valid = u(w.valid);
  w.hk = u(w.hk);
  w.hc = u(w.hc);
  w.c0 = u(w.c0);
  w.c1 = u(w.c1);
  w.b = u(w.b);
  w.t0 = u(w.t0);
  w.ntok = u(w.ntok);
  w.Lq = u(w.Lq);
  w.L = u(w.L);
  w.koff = uniform64(w.koff);
  w.sl = u(w.sl);
  return w;
}

// Last visible key index of query token t of the work item's request:
// min(q_pos, kv_len - 1), with q_pos = kv_len - L_q + i under the right-down
// causal mode and kv_len - 1 without it (issue #4117, section 计算过程;
// guide to msa_index_score, section 四: sparse_mode 3 / 0).
__device__ __forceinline__ int last_visible(const Params& p, const Work& w, int i) {
  const int qpos = p.causal ? (w.L - w.Lq + i) : (w.L - 1);
  return min(qpos, w.L - 1);
}

// Final value of output column beta of a row (after the block maximum `v`
// when the block was scored): -inf fill, then local_mask (guide to
// msa_index_score, section 二: 1e30 on [0, init_blocks), then 1e29 on
// [max(0, start_loc+1-local_blocks), start_loc], skipped when both are 0;
// requests with kv_len = 0 are skipped whole, section 四).
// Last block of the local_mask window for token i of the work item's request:
// start_loc[b], or (per query) the block of the token's own position
// L - Lq + i, -1 (no window) before position 0 -- the paper's per-query local
// block (notes "MiniMax Sparse Attention: paper algorithm and code", section
// 4.7, forced local block).
__device__ __forceinline__ int query_anchor(const Work& w, int i) {
  const int pos = w.L - w.Lq + i;
  return pos >= 0 ? pos / kP : -1;
}

__device__ __forceinline__ int local_anchor(const Params& p, const Work& w, int i) {
  return p.local_per_query ? query_anchor(w, i) : p.start_loc[w.b];
}

__device__ __forceinline__ float finish(const Params& p, int L, int start, int beta,
                                        bool scored, float v) {
  float r = scored ? v : -__builtin_inff();
  if (L > 0 && (p.init_blocks > 0 || p.local_blocks > 0)) {
    if (beta < p.init_blocks) r = 1e30f;
    const int lo = max(0, start + 1 - p.local_blocks);
    if (beta >= lo && beta <= start) r = 1e29f;
  }
  return r;
}

// ---------------------------------------------------------------------------
// element conversion and MFMA wrappers
// ---------------------------------------------------------------------------

// 4 int8 -> 4 fp16 exactly: bias each byte to u = x + 128, place it in the
// low mantissa byte of 1024.0h (0x6400 | u = 1024 + u) and subtract 1152.
__device__ __forceinline__ void i8x4_to_f16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) - bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, b) - bias);
}

// 16 int8 (one i32x4) -> 16 fp16 (two i32x4), byte order kept.
__device__ __forceinline__ void i8x16_to_f16x16(i32x4 v, i32x4& first, i32x4& second) {
  uint32_t a0, a1, b0, b1, c0, c1, d0, d1;
  i8x4_to_f16x4((uint32_t)v.x, a0, a1);
  i8x4_to_f16x4((uint32_t)v.y, b0, b1);
  i8x4_to_f16x4((uint32_t)v.z, c0, c1);
  i8x4_to_f16x4((uint32_t)v.w, d0, d1);
  first = i32x4{(int)a0, (int)a1, (int)b0, (int)b1};
  second = i32x4{(int)c0, (int)c1, (int)d0, (int)d1};
}

// 16x16 output tile, 32-deep k of 16-bit elements.
template <int KK>
__device__ __forceinline__ f32x4 mfma16x16x32(i32x4 a, i32x4 b, f32x4 c) {
  if constexpr (KK == KBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 32x32 output tile, 16-deep k of 16-bit elements.
template <int KK>
__device__ __forceinline__ f32x16 mfma32x32x16(i32x4 a, i32x4 b, f32x16 c) {
  if constexpr (KK == KBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ i32x8 cat(i32x4 a, i32x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// OCP fp8 operands: format code 0 = e4m3, 1 = e5m2 (no block scaling).
template <int KK>
__device__ __forceinline__ f32x4 mfma16x16x128_f8(i32x8 a, i32x8 b, f32x4 c) {
  constexpr int fmt = (KK == KF8E5M2) ? 1 : 0;
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, fmt, fmt, 0, 0, 0, 0);
}

template <int KK>
__device__ __forceinline__ f32x16 mfma32x32x64_f8(i32x8 a, i32x8 b, f32x16 c) {
  constexpr int fmt = (KK == KF8E5M2) ? 1 : 0;
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, fmt, fmt, 0, 0, 0, 0);
}

// MXFP4 (E2M1) operands with per-lane E8M0 scales (byte 0 of sa / sb):
// lane l covers row l % 32 and the 32 elements 32 (l / 32) + [0, 32) of the
// 64-deep k step, 16 bytes, two elements per byte (the even one in the low
// nibble); the scale is that group's.
__device__ __forceinline__ f32x16 mfma32x32x64_fp4(i32x4 a, i32x4 b, f32x16 c, int sa, int sb) {
  const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const i32x8 b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}

// The same with the scale bytes chosen by the instruction: byte SA of sa
// and byte SB of sb.
template <int SA, int SB>
__device__ __forceinline__ f32x16 mfma32x32x64_fp4_sel(i32x4 a, i32x4 b, f32x16 c, int sa,
                                                       int sb) {
  const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const i32x8 b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, SA, sa, SB, sb);
}

// The 16x16x128 form: lane l covers row l % 16 and the 32 elements
// 32 (l / 16) + [0, 32) of the 128-deep product (16 bytes), scale byte 0 of
// sa / sb; lane l's result is column l % 16, rows 4 (l / 16) + [0, 4).
__device__ __forceinline__ f32x4 mfma16x16x128_fp4(i32x4 a, i32x4 b, f32x4 c, int sa, int sb) {
  const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const i32x8 b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}

template <int KK>
struct Kind {
  static constexpr bool is_f8 = (KK == KF8E4M3 || KK == KF8E5M2);
  static constexpr bool is_i8 = (KK == KI8);
  static constexpr bool is_fp4 = (KK == KMXFP4);
  static constexpr int q_bytes = is_f8 ? 1 : 2;   // query element size (not MXFP4)
  static constexpr int k_bytes = (is_f8 || is_i8) ? 1 : 2;
  static constexpr int q_row = is_fp4 ? kD / 2 : kD * q_bytes;   // bytes per query row
  static constexpr int mfma_kind = is_i8 ? KF16 : KK;  // operand type fed to MFMA
};

}  // namespace msa
