// Host side of the msa_index_score C ABI (and of msa_block_topk, the top-k
// selection over its output): argument validation (all of it before any HIP
// call), work planning, and the launch of one gfx950 kernel on the caller's
// stream.  The library allocates nothing; the only state it keeps is one
// figure per device and key type, the decode kernel's workgroup slot count,
// looked up on the first decode launch there.
#include "msa_index_score.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <tuple>

#include "msa_kernels.hpp"
#include "msa_topk.hpp"

namespace {

using msa::Params;

int64_t round_up16(int64_t mb) {
  if (mb < 1) mb = 1;
  return (mb + 15) / 16 * 16;
}

int elem_bytes(int32_t dt) {
  switch (dt) {
    case MSA_DTYPE_F16:
    case MSA_DTYPE_BF16: return 2;
    case MSA_DTYPE_I8:
    case MSA_DTYPE_F8E4M3:
    case MSA_DTYPE_F8E5M2:
    case MSA_DTYPE_MXFP4: return 1;   // MXFP4: a byte holds two elements
    default: return 0;
  }
}

// Supported (query, key) element pairs (guide to msa_index_score, section 七:
// int8 keys take an fp16 query and a float32 scale; FP8 query and key share
// one format and take no scale).
bool pair_ok(int32_t qd, int32_t kd) {
  if (qd == MSA_DTYPE_F16 && (kd == MSA_DTYPE_F16 || kd == MSA_DTYPE_I8)) return true;
  if (qd == MSA_DTYPE_BF16 && kd == MSA_DTYPE_BF16) return true;
  if (qd == MSA_DTYPE_F8E4M3 && kd == MSA_DTYPE_F8E4M3) return true;
  if (qd == MSA_DTYPE_F8E5M2 && kd == MSA_DTYPE_F8E5M2) return true;
  if (qd == MSA_DTYPE_MXFP4 && kd == MSA_DTYPE_MXFP4) return true;
  return false;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Extent-1 axes are never addressed, so their strides are not compared.
bool compact_axis(int64_t extent, int64_t stride, int64_t want) {
  return extent <= 1 || stride == want;
}

// Kernel family.  Prefill tiles (hundreds of rows sharing each key block
// staged in LDS) pay off once requests carry about half a 256-row tile of
// query rows on average and the batch holds a few tiles' worth of rows in all
// (T * Hq >= 1024); otherwise the 16-row decode tiles, whose (tile, block)
// work list spreads even one short request over the whole chip.  Measured on
// one paged bf16 request (B = 1, Hkv = 1): 32 tokens x 8 heads, 2 blocks,
// 7.9 us on decode tiles against 13.0 us on one prefill tile; with 16384
// keys, 64 tokens x 8 heads, 16.6 against 112 us; from 1024 tokens x 8
// heads on, prefill tiles win at every kv length tried (256 to 16384).
int32_t choose_family(int64_t T, int32_t B, int32_t Hq, int32_t Hkv) {
  const int64_t g = std::max<int32_t>(Hq / std::max<int32_t>(Hkv, 1), 1);
  const int64_t rows = T * std::min<int64_t>(g, msa::kPrefillRows);
  const bool long_runs = rows >= (int64_t)(msa::kPrefillRows / 2) * std::max<int32_t>(B, 1);
  return long_runs && T * (int64_t)Hq >= 1024 ? 1 : 0;
}

// Blocks per prefill work item.  The key type's default (msa_kernels.hpp,
// prefill_chunk) amortises a work item's set-up over many blocks; when that
// leaves fewer than kPrefillMinItems work items for the whole launch, the
// chunk shrinks (to a multiple of 4 blocks, at least 4: the kernels write a
// row's columns in aligned groups of 4) until the items cover the chip: one
// workgroup per work item runs its blocks in sequence, so a short prefill of
// a long context would otherwise take tens of blocks per workgroup on a few
// dozen CUs.  Measured on one bf16 request of 16384 keys, 256 tokens x 8
// heads: 113 us with 40-block items, 30 us with 8-block ones.
constexpr int64_t kPrefillMinItems = 1024;

int32_t prefill_chunk_for(int32_t dflt, int64_t W, int64_t units_per_chunk, int64_t ntiles) {
  const int64_t per_chunk = std::max<int64_t>(units_per_chunk * ntiles, 1);
  if (per_chunk * ((W + dflt - 1) / dflt) >= kPrefillMinItems) return dflt;
  const int64_t want = (kPrefillMinItems + per_chunk - 1) / per_chunk;   // chunks per row
  int64_t c = (W + want - 1) / want;
  c = (c + 3) / 4 * 4;
  return (int32_t)std::min<int64_t>(std::max<int64_t>(c, 4), dflt);
}

// Launch `kern` with these arguments (converted to its parameter types) and
// return the status of this launch alone.  (hipGetLastError after a
// triple-chevron launch would also return, and clear, an error left pending
// by earlier unrelated HIP calls of the caller.)
template <typename... KA, typename... A>
hipError_t launch_kernel(void (*kern)(KA...), dim3 grid, dim3 block, hipStream_t s, A... a) {
  static_assert(sizeof...(KA) == sizeof...(A), "one value per kernel parameter");
  std::tuple<KA...> vals{static_cast<KA>(a)...};
  void* ptrs[sizeof...(KA)];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, 0, s);
}

// Decode: one round of workgroups, as many as fit on the device at once,
// split evenly over the units (KV head x head chunk).  The device's slot
// count for each decode kernel is looked up once per device (the runtime
// queries cost microseconds, as much as a short decode launch).
template <int KK, bool BIG>
hipError_t launch_decode(Params& p, hipStream_t s) {
  constexpr int kThreads = 64 * msa::decode_waves<KK, BIG>();
  constexpr int kMaxDevices = 64;
  static std::atomic<int64_t> slots_of[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  int64_t slots = cached ? slots_of[dev].load(std::memory_order_relaxed) : 0;
  if (slots == 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, msa::decode_kernel<KK, BIG>,
                                                       kThreads, 0);
    if (e != hipSuccess) return e;
    slots = (int64_t)std::max(cus, 1) * std::max(per_cu, 1);
    if (cached) slots_of[dev].store(slots, std::memory_order_relaxed);
  }
  const int64_t gu = std::max<int64_t>(1, slots / p.units);
  return launch_kernel(msa::decode_kernel<KK, BIG>, dim3((unsigned)(gu * p.units)),
                       dim3(kThreads), s, p);
}

template <int KK>
hipError_t launch(int family, Params& p, int64_t prefill_grid, hipStream_t s) {
  if (family == 1)
    return launch_kernel(msa::prefill_kernel<KK>, dim3((unsigned)prefill_grid), dim3(256), s, p);
  // batches of more than 64 requests: the kernel with the chunk table
  return p.B > 64 ? launch_decode<KK, true>(p, s) : launch_decode<KK, false>(p, s);
}

msa_status_t run(const msa_tensor_t* query, const msa_tensor_t* key, const int32_t* start_loc,
                 const int32_t* block_table, int64_t max_blocks, const float* scale,
                 const uint8_t* q_mx, const uint8_t* k_mx,
                 const int32_t* cu_seqlens_q, const int32_t* kv_len, int32_t batch,
                 int32_t block_size, int32_t layout, int32_t sparse_mode, int32_t init_blocks,
                 int32_t local_blocks, int32_t local_mode, float* out, int64_t out_width,
                 void* stream, int32_t family, bool mx_entry) {
  // Pointers that a call with no requests (B = 0) or no query tokens (T = 0)
  // never reads may be NULL there; torch hands empty tensors a NULL address.
  // start_loc is not read with the per-query local window.
  if (!query || !key || !cu_seqlens_q) return MSA_ERR_NULL;
  if (batch > 0 && (!kv_len || (!start_loc && local_mode != MSA_LOCAL_PER_QUERY)))
    return MSA_ERR_NULL;
  if (query->ndim == 3 && query->shape[0] > 0 && !out) return MSA_ERR_NULL;
  if (layout != MSA_LAYOUT_TND && layout != MSA_LAYOUT_BBND && layout != MSA_LAYOUT_BNBD)
    return MSA_ERR_LAYOUT;
  const bool paged = layout != MSA_LAYOUT_TND;

  // element types and scale
  if (elem_bytes(query->dtype) == 0 || elem_bytes(key->dtype) == 0) return MSA_ERR_DTYPE;
  if (!pair_ok(query->dtype, key->dtype)) return MSA_ERR_DTYPE;
  const bool is_i8 = key->dtype == MSA_DTYPE_I8;
  if (is_i8 != (scale != nullptr)) return MSA_ERR_SCALE;
  // MXFP4 comes through its own entry only, the one that carries the E8M0
  // group scales (and only it takes scales of that kind); its last axis
  // holds D/2 bytes
  const bool is_mx = key->dtype == MSA_DTYPE_MXFP4;
  if (is_mx != mx_entry || (!is_mx && (q_mx || k_mx))) return MSA_ERR_SCALE;
  const int64_t DB = is_mx ? msa::kD / 2 : msa::kD;     // stored last-axis extent

  // query [T, Hq, D], compact
  if (query->ndim != 3) return MSA_ERR_SHAPE;
  const int64_t T = query->shape[0], Hq = query->shape[1], D = query->shape[2];
  if (T < 0 || Hq < 1 || D != DB) return MSA_ERR_SHAPE;
  // the logical block is the page: 128 tokens (guide, section 四: block_size
  // 128; a paged key's P axis must match it)
  if (block_size != msa::kP) return MSA_ERR_SHAPE;
  if (is_mx && T > 0 && (!q_mx || !k_mx)) return MSA_ERR_NULL;
  if (!compact_axis(D, query->stride[2], 1) || !compact_axis(Hq, query->stride[1], D) ||
      !compact_axis(T, query->stride[0], Hq * D))
    return MSA_ERR_STRIDE;

  // key layout, shape and strides
  int64_t NP = 0, P = msa::kP, Hkv = 0, KD = 0;
  int64_t s_page = 0, s_row = 0, s_head = 0;        // element strides
  const int64_t* ks = key->stride;
  if (layout == MSA_LAYOUT_TND) {
    if (key->ndim != 3) return MSA_ERR_SHAPE;
    NP = key->shape[0];
    Hkv = key->shape[1];
    KD = key->shape[2];
    if (Hkv < 1 || KD != DB || NP < 0) return MSA_ERR_SHAPE;
    if (!compact_axis(KD, ks[2], 1) || !compact_axis(Hkv, ks[1], KD) ||
        !compact_axis(NP, ks[0], Hkv * KD))
      return MSA_ERR_STRIDE;
    s_row = Hkv * KD;
    s_head = KD;
  } else if (layout == MSA_LAYOUT_BBND && key->ndim == 3) {
    // [NP, P, D]: a single KV head with the head axis left out
    NP = key->shape[0];
    P = key->shape[1];
    Hkv = 1;
    KD = key->shape[2];
    if (P != msa::kP || KD != DB || NP < 1) return MSA_ERR_SHAPE;
    if (!compact_axis(KD, ks[2], 1) || !compact_axis(P, ks[1], KD)) return MSA_ERR_STRIDE;
    s_page = ks[0];
    s_row = KD;
    s_head = 0;
  } else {
    if (key->ndim != 4) return MSA_ERR_SHAPE;
    NP = key->shape[0];
    KD = key->shape[3];
    if (layout == MSA_LAYOUT_BBND) {
      P = key->shape[1];
      Hkv = key->shape[2];
    } else {
      Hkv = key->shape[1];
      P = key->shape[2];
    }
    if (P != msa::kP || KD != DB || Hkv < 1 || NP < 1) return MSA_ERR_SHAPE;
    if (!compact_axis(KD, ks[3], 1)) return MSA_ERR_STRIDE;
    if (layout == MSA_LAYOUT_BBND) {
      if (!compact_axis(Hkv, ks[2], KD) || !compact_axis(P, ks[1], Hkv * KD))
        return MSA_ERR_STRIDE;
      s_row = Hkv * KD;
      s_head = KD;
    } else {
      if (!compact_axis(P, ks[2], KD) || !compact_axis(Hkv, ks[1], P * KD))
        return MSA_ERR_STRIDE;
      s_row = KD;
      s_head = P * KD;
    }
    s_page = ks[0];
  }
  if (Hq % Hkv != 0) return MSA_ERR_SHAPE;
  if (paged && NP > 1 && s_page < 1) return MSA_ERR_STRIDE;
  const int kb = elem_bytes(key->dtype);
  if (paged && ((s_page * kb) % 16) != 0) return MSA_ERR_STRIDE;

  // table, widths and attributes
  if (max_blocks < 0 || batch < 0) return MSA_ERR_SHAPE;
  if (paged) {
    if (!block_table && batch > 0) return MSA_ERR_NULL;
    if (max_blocks < 1) return MSA_ERR_SHAPE;
  } else if (block_table) {
    return MSA_ERR_SHAPE;   // packed keys take no block table
  }
  const int64_t W = round_up16(max_blocks);
  if (out_width != W) return MSA_ERR_SHAPE;
  if (batch == 0 && T > 0) return MSA_ERR_SHAPE;
  if (sparse_mode != 0 && sparse_mode != 3) return MSA_ERR_ATTR;
  const int64_t limit = paged ? max_blocks : W;
  if (init_blocks < 0 || local_blocks < 0 || init_blocks > limit || local_blocks > limit)
    return MSA_ERR_ATTR;
  if (family < -1 || family > 1) return MSA_ERR_ATTR;
  if (local_mode != MSA_LOCAL_PER_REQUEST && local_mode != MSA_LOCAL_PER_QUERY)
    return MSA_ERR_ATTR;

  // sizes the kernels index with 32-bit integers
  if (W > (1 << 24) || Hq > (1 << 16) || batch > (1 << 30) || T > (int64_t(1) << 31) - 1 ||
      (msa::kP - 1) * s_row * kb + DB * kb > INT32_MAX || s_head * kb > INT32_MAX)
    return MSA_ERR_SHAPE;

  if (!aligned16(query->data) || !aligned16(key->data) || !aligned16(out))
    return MSA_ERR_STRIDE;
  if ((reinterpret_cast<uintptr_t>(q_mx) & 3u) || (reinterpret_cast<uintptr_t>(k_mx) & 3u))
    return MSA_ERR_STRIDE;

  if (T == 0) return MSA_OK;

  // plan
  const int32_t g = (int32_t)(Hq / Hkv);
  const int fam = family >= 0 ? family : choose_family(T, batch, (int32_t)Hq, (int32_t)Hkv);
  const int rows = fam == 1 ? msa::prefill_rows(is_mx ? msa::KMXFP4 : key->dtype)
                            : msa::kDecodeRows;
  Params p{};
  p.q = static_cast<const uint8_t*>(query->data);
  p.k = static_cast<const uint8_t*>(key->data);
  p.scale = scale;
  p.q_mx = q_mx;
  p.k_mx = k_mx;
  if (layout == MSA_LAYOUT_BNBD) {   // key scales [NP, Hkv, P, D/32]
    p.mx_row_stride = msa::kD / 32;
    p.mx_head_stride = msa::kP * (msa::kD / 32);
    p.mx_page_stride = Hkv * msa::kP * (msa::kD / 32);
  } else {                           // [NP, P, Hkv, D/32] or [T2, Hkv, D/32]
    p.mx_row_stride = (int32_t)(Hkv * (msa::kD / 32));
    p.mx_head_stride = msa::kD / 32;
    p.mx_page_stride = paged ? msa::kP * Hkv * (msa::kD / 32) : 0;
  }
  p.block_table = paged ? block_table : nullptr;
  p.cu_q = cu_seqlens_q;
  p.kv_len = kv_len;
  p.start_loc = start_loc;
  p.out = out;
  p.k_page_stride = paged ? s_page * kb : 0;
  p.k_row_stride = (int32_t)(s_row * kb);
  p.k_head_stride = Hkv > 1 ? (int32_t)(s_head * kb) : 0;
  if (paged) {
    p.s_page_stride = Hkv * msa::kP;   // scale [NP, Hkv, P]
    p.s_head_stride = msa::kP;
    p.s_row_stride = 1;
  } else {
    p.s_page_stride = 0;               // scale [T2, Hkv]
    p.s_head_stride = 1;
    p.s_row_stride = (int32_t)Hkv;
  }
  p.T = T;
  p.B = batch;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.g = g;
  p.MB = (int32_t)std::max<int64_t>(max_blocks, 1);
  p.W = (int32_t)W;
  p.paged = paged ? 1 : 0;
  p.causal = sparse_mode == 3 ? 1 : 0;
  p.init_blocks = init_blocks;
  p.local_blocks = local_blocks;
  p.local_per_query = local_mode == MSA_LOCAL_PER_QUERY ? 1 : 0;
  p.hpt = std::min<int32_t>(g, rows);
  p.tpt = rows / p.hpt;
  p.hchunks = (g + p.hpt - 1) / p.hpt;
  // prefill units: (KV head, head chunk, block chunk); decode units: (KV
  // head, head chunk), each walking its own copy of the batch's work list
  const int64_t bound = (T + (int64_t)batch * (p.tpt - 1)) / p.tpt;
  p.ntiles = (int32_t)std::min<int64_t>(T, bound);
  p.chunk = msa::prefill_chunk(is_mx ? msa::KMXFP4 : key->dtype);
  if (fam == 1) p.chunk = prefill_chunk_for(p.chunk, W, (int64_t)p.Hkv * p.hchunks, p.ntiles);
  p.nchunks = fam == 1 ? (int32_t)((W + p.chunk - 1) / p.chunk) : 1;
  p.units = p.Hkv * p.hchunks * p.nchunks;
  const int64_t units8 = ((int64_t)p.units + 7) / 8 * 8;
  const int64_t grid = units8 * p.ntiles;
  if (grid > INT32_MAX || (int64_t)p.units * p.ntiles > INT32_MAX) return MSA_ERR_SHAPE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (key->dtype) {
    case MSA_DTYPE_F16: e = launch<msa::KF16>(fam, p, grid, s); break;
    case MSA_DTYPE_BF16: e = launch<msa::KBF16>(fam, p, grid, s); break;
    case MSA_DTYPE_I8: e = launch<msa::KI8>(fam, p, grid, s); break;
    case MSA_DTYPE_F8E4M3: e = launch<msa::KF8E4M3>(fam, p, grid, s); break;
    case MSA_DTYPE_MXFP4: e = launch<msa::KMXFP4>(fam, p, grid, s); break;
    default: e = launch<msa::KF8E5M2>(fam, p, grid, s); break;
  }
  return e == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

}  // namespace

extern "C" {

msa_status_t msa_index_score(const msa_tensor_t* query, const msa_tensor_t* key,
                             const int32_t* start_loc, const int32_t* block_table,
                             int64_t max_blocks, const float* scale,
                             const int32_t* cu_seqlens_q, const int32_t* kv_len,
                             int32_t batch, int32_t block_size, int32_t layout,
                             int32_t sparse_mode, int32_t init_blocks, int32_t local_blocks,
                             float* out, int64_t out_width, void* stream) {
  return run(query, key, start_loc, block_table, max_blocks, scale, nullptr, nullptr,
             cu_seqlens_q, kv_len, batch, block_size, layout, sparse_mode, init_blocks,
             local_blocks, MSA_LOCAL_PER_REQUEST, out, out_width, stream, -1, false);
}

msa_status_t msa_index_score_family(const msa_tensor_t* query, const msa_tensor_t* key,
                                    const int32_t* start_loc, const int32_t* block_table,
                                    int64_t max_blocks, const float* scale,
                                    const int32_t* cu_seqlens_q, const int32_t* kv_len,
                                    int32_t batch, int32_t block_size, int32_t layout,
                                    int32_t sparse_mode, int32_t init_blocks,
                                    int32_t local_blocks, float* out, int64_t out_width,
                                    void* stream, int32_t family) {
  return run(query, key, start_loc, block_table, max_blocks, scale, nullptr, nullptr,
             cu_seqlens_q, kv_len, batch, block_size, layout, sparse_mode, init_blocks,
             local_blocks, MSA_LOCAL_PER_REQUEST, out, out_width, stream, family, false);
}

msa_status_t msa_index_score_ex(const msa_tensor_t* query, const msa_tensor_t* key,
                                const int32_t* start_loc, const int32_t* block_table,
                                int64_t max_blocks, const float* scale,
                                const int32_t* cu_seqlens_q, const int32_t* kv_len,
                                int32_t batch, int32_t block_size, int32_t layout,
                                int32_t sparse_mode, int32_t init_blocks, int32_t local_blocks,
                                int32_t local_mode, float* out, int64_t out_width, void* stream,
                                int32_t family) {
  return run(query, key, start_loc, block_table, max_blocks, scale, nullptr, nullptr,
             cu_seqlens_q, kv_len, batch, block_size, layout, sparse_mode, init_blocks,
             local_blocks, local_mode, out, out_width, stream, family, false);
}

msa_status_t msa_block_topk(const float* scores, int64_t Hq, int64_t T, int64_t width,
                            int64_t num_valid, int32_t k, int32_t* out, void* stream) {
  if (Hq < 0 || T < 0 || width < 0 || width > (1 << 24) || num_valid < 0 || num_valid > width)
    return MSA_ERR_SHAPE;
  if (k < 1 || k > msa::kTopkMax) return MSA_ERR_ATTR;
  if (Hq == 0 || T == 0) return MSA_OK;
  // grid (ceil(T / 4), Hq), one row per wave
  if (Hq > 65535 || (T + 3) / 4 > INT32_MAX || T > INT64_MAX / Hq / std::max<int64_t>(width, 1))
    return MSA_ERR_SHAPE;
  if (!out || (num_valid > 0 && !scores)) return MSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(scores) & 3u) || (reinterpret_cast<uintptr_t>(out) & 3u))
    return MSA_ERR_STRIDE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nv = (int)num_valid;
  // Keys of up to 64 * J blocks stay in registers, longer rows are re-read.
  // With many rows of up to 512 blocks a wave takes R = 4 of them in turn
  // (each row's loads overlap the selection on the row before); few rows
  // keep one per wave, for parallelism, and so do longer rows, where a
  // second row's registers would cost occupancy.
  const int R = Hq * T >= (int64_t)msa::kTopkManyRows && nv <= 512 ? 4 : 1;
  const dim3 grid((unsigned)((T + msa::kTopkWaves * R - 1) / (msa::kTopkWaves * R)), (unsigned)Hq);
  const dim3 block(64 * msa::kTopkWaves);
  hipError_t e;
  // (a kernel per register count J, rows per wave R, and whether nv fills
  // the J registers exactly)
#define MSA_TOPK_GO(J, R, F) \
  e = launch_kernel(msa::topk_kernel<J, R, F>, grid, block, s, scores, T, Hq, width, nv, k, out)
#define MSA_TOPK_LAUNCH(J)        \
  if (R == 4 && nv == 64 * J)     \
    MSA_TOPK_GO(J, 4, true);      \
  else if (R == 4)                \
    MSA_TOPK_GO(J, 4, false);     \
  else if (nv == 64 * J)          \
    MSA_TOPK_GO(J, 1, true);      \
  else                            \
    MSA_TOPK_GO(J, 1, false)
  if (nv <= 128) {
    MSA_TOPK_LAUNCH(2);
  } else if (nv <= 256) {
    MSA_TOPK_LAUNCH(4);
  } else if (nv <= 512) {
    MSA_TOPK_LAUNCH(8);
  } else if (nv <= 1024) {
    if (nv == 1024)
      MSA_TOPK_GO(16, 1, true);
    else
      MSA_TOPK_GO(16, 1, false);
  } else if (nv <= 2048) {
    if (nv == 2048)
      MSA_TOPK_GO(32, 1, true);
    else
      MSA_TOPK_GO(32, 1, false);
  } else {
    MSA_TOPK_GO(0, 1, false);
  }
#undef MSA_TOPK_LAUNCH
#undef MSA_TOPK_GO
  return e == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

msa_status_t msa_index_score_mxfp4(const msa_tensor_t* query, const uint8_t* query_scale,
                                   const msa_tensor_t* key, const uint8_t* key_scale,
                                   const int32_t* start_loc, const int32_t* block_table,
                                   int64_t max_blocks, const int32_t* cu_seqlens_q,
                                   const int32_t* kv_len, int32_t batch, int32_t block_size,
                                   int32_t layout, int32_t sparse_mode, int32_t init_blocks,
                                   int32_t local_blocks, int32_t local_mode, float* out,
                                   int64_t out_width, void* stream) {
  if (!query || !key) return MSA_ERR_NULL;
  if (query->dtype != MSA_DTYPE_MXFP4 || key->dtype != MSA_DTYPE_MXFP4) return MSA_ERR_DTYPE;
  return run(query, key, start_loc, block_table, max_blocks, nullptr, query_scale, key_scale,
             cu_seqlens_q, kv_len, batch, block_size, layout, sparse_mode, init_blocks,
             local_blocks, local_mode, out, out_width, stream, -1, true);
}

msa_status_t msa_index_score_mxfp4_family(const msa_tensor_t* query, const uint8_t* query_scale,
                                          const msa_tensor_t* key, const uint8_t* key_scale,
                                          const int32_t* start_loc, const int32_t* block_table,
                                          int64_t max_blocks, const int32_t* cu_seqlens_q,
                                          const int32_t* kv_len, int32_t batch,
                                          int32_t block_size, int32_t layout,
                                          int32_t sparse_mode, int32_t init_blocks,
                                          int32_t local_blocks, int32_t local_mode, float* out,
                                          int64_t out_width, void* stream, int32_t family) {
  if (!query || !key) return MSA_ERR_NULL;
  if (query->dtype != MSA_DTYPE_MXFP4 || key->dtype != MSA_DTYPE_MXFP4) return MSA_ERR_DTYPE;
  return run(query, key, start_loc, block_table, max_blocks, nullptr, query_scale, key_scale,
             cu_seqlens_q, kv_len, batch, block_size, layout, sparse_mode, init_blocks,
             local_blocks, local_mode, out, out_width, stream, family, true);
}

int64_t msa_index_score_out_width(int64_t max_blocks) { return round_up16(max_blocks); }

int32_t msa_index_score_kernel_family(int64_t T, int32_t batch, int32_t Hq, int32_t Hkv) {
  return choose_family(T, batch, Hq, Hkv);
}

const char* msa_status_str(int32_t s) {
  switch (s) {
    case MSA_OK: return "ok";
    case MSA_ERR_NULL: return "a required pointer is NULL";
    case MSA_ERR_LAYOUT: return "layout must be TND, BBND or BNBD";
    case MSA_ERR_DTYPE: return "unsupported query/key element types";
    case MSA_ERR_SHAPE: return "inconsistent shapes";
    case MSA_ERR_STRIDE: return "non-compact or misaligned axis";
    case MSA_ERR_SCALE: return "scale must be given exactly for int8 keys";
    case MSA_ERR_ATTR: return "sparse_mode, init_blocks, local_blocks or family out of range";
    case MSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
