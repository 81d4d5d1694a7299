/*
 * msa_index_score.h -- C ABI of the MSA index-branch block-score operator for
 * AMD Instinct MI355X (gfx950).
 *
 * The operator (gitcode cann/ops-transformer issue #4117 "MsaIndexScore",
 * section 计算过程; xxmr.cn guide to cann_ops_transformer.msa_index_score,
 * sections 二, 四, 五) computes, for every packed query token t of request b,
 * every index head h and every logical KV block beta of P = 128 tokens:
 *
 *   score[h, t, beta] = max_{j in block beta, j <= q_pos(t), j < kv_len[b]}
 *                       < query[t, h, :], k~[j, h / g, :] >
 *
 * with g = Hq / Hkv, q_pos(t) = kv_len[b] - L_q(b) + (t - cu_seqlens_q[b])
 * under the right-down causal mode (sparse_mode 3) and kv_len[b] - 1 without a
 * causal mask (sparse_mode 0).  k~ is the key row of logical block beta: for a
 * paged key it lives in physical page block_table[b, beta]; for a packed (TND)
 * key it is token sum_{b' < b} kv_len[b'] + j.  For an int8 key the dot product
 * is multiplied by scale[page, h_kv, j mod P] (TND: scale[token, h_kv]) before
 * the mask and the maximum (issue #4117: DOT -> DEQUANT -> MASK -> MAX).
 * Blocks with no visible key score -inf, requests with kv_len = 0 score -inf
 * everywhere, and output columns past a request's block count up to the
 * output width are -inf.  Then local_mask (guide, section 二) writes 1e30f on
 * blocks [0, init_blocks) and 1e29f on [max(0, start_loc[b]+1-local_blocks),
 * start_loc[b]] (the latter overriding), unless both counts are 0.  The output
 * is float32 [Hq, T, RoundUp(MB, 16)] (guide, section 五).
 *
 * No torch or HIP types appear here: pointers are plain device pointers and
 * the stream is a hipStream_t passed as void* (NULL = the null stream).
 */
#ifndef MSA_INDEX_SCORE_H
#define MSA_INDEX_SCORE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every check runs on the host before any device work; on a
 * non-zero status nothing is launched and `out` is untouched. */
typedef enum {
  MSA_OK = 0,
  MSA_ERR_NULL = 1,    /* a required pointer is NULL */
  MSA_ERR_LAYOUT = 2,  /* layout is not TND, BBND or BNBD (guide, section 三) */
  MSA_ERR_DTYPE = 3,   /* unsupported query/key element types (guide, section 七) */
  MSA_ERR_SHAPE = 4,   /* shapes disagree with each other or with the layout */
  MSA_ERR_STRIDE = 5,  /* a key axis other than dim0 is not compact (guide, 8.1) */
  MSA_ERR_SCALE = 6,   /* int8 key without scale, or scale with a non-int8 key */
  MSA_ERR_ATTR = 7,    /* sparse_mode not 0/3, init/local_blocks out of range, or
                          another attribute (family, local_mode, top-k k) invalid */
  MSA_ERR_HIP = 8      /* a HIP runtime call or kernel launch failed */
} msa_status_t;

/* Key layouts (guide, section 四): packed [T2, Hkv, D]; paged
 * [NP, P, Hkv, D] (BBND) and [NP, Hkv, P, D] (BNBD). */
typedef enum { MSA_LAYOUT_TND = 0, MSA_LAYOUT_BBND = 1, MSA_LAYOUT_BNBD = 2 } msa_layout_t;

/* Where local_mask's window of local_blocks blocks ends.  PER_REQUEST: at
 * start_loc[b] for every token of request b (guide, section 二).  PER_QUERY:
 * at each query token's own block, floor(pos / 128) with pos = kv_len[b] -
 * L_q(b) + i the token's position in the sequence -- the paper's forced local
 * block b_local(i) (notes "MiniMax Sparse Attention: paper algorithm and
 * code", section 4.7, which observes that a request-wide window is not the
 * same in a long prefill).  A token before position 0 gets no window. */
typedef enum { MSA_LOCAL_PER_REQUEST = 0, MSA_LOCAL_PER_QUERY = 1 } msa_local_mode_t;

/* Element types.  Supported (query, key) pairs: (F16, F16), (BF16, BF16),
 * (F16, I8) with a float32 scale, (F8E4M3, F8E4M3) and (F8E5M2, F8E5M2)
 * (guide, section 七: int8 needs an fp16 query; FP8 query and key of one type,
 * no scale).  F8E4M3 is OCP e4m3 "fn" (finite, max 448); F8E5M2 is OCP e5m2. */
typedef enum {
  MSA_DTYPE_F16 = 0,
  MSA_DTYPE_BF16 = 1,
  MSA_DTYPE_I8 = 2,
  MSA_DTYPE_F8E4M3 = 3,
  MSA_DTYPE_F8E5M2 = 4,
  MSA_DTYPE_MXFP4 = 5  /* E2M1 pairs, one byte each; see msa_index_score_mxfp4 */
} msa_dtype_t;

/* A strided view of device memory.  `data` points at element [0, 0, ...];
 * `stride` is in elements.  Only the first `ndim` entries are read. */
typedef struct {
  const void* data;
  int32_t dtype;       /* msa_dtype_t */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} msa_tensor_t;

/*
 * Compute the block scores.
 *
 * query        [T, Hq, D] compact; D must be 128.
 * key          TND [T2, Hkv, D] fully compact; BBND [NP, P, Hkv, D] or
 *              BNBD [NP, Hkv, P, D] with P = 128, any dim0 stride (pages may
 *              sit apart in memory, guide 8.1), other axes of extent > 1
 *              compact (extent-1 axes are not addressed, so their stride is
 *              ignored).  A 3-D BBND key [NP, P, D] means Hkv = 1.
 * start_loc    device int32 [B]: logical block index of the request's current
 *              query (guide, section 四); used only by local_mask.
 * block_table  device int32 [B, max_blocks] row-major, paged layouts only
 *              (NULL for TND).  Entries at or past a request's block count
 *              ceil(kv_len/128) are never read.
 * max_blocks   MB: the block_table width for paged layouts; for TND the
 *              largest ceil(kv_len[b]/128) over the batch (an all-empty batch
 *              may pass 0 or 1).
 * scale        device float32, int8 keys only (NULL otherwise): paged
 *              [NP, Hkv, P] indexed by logical page number, TND [T2, Hkv].
 * cu_seqlens_q device int32 [B+1], cu_seqlens_q[0] = 0, non-decreasing,
 *              cu_seqlens_q[B] = T.
 * kv_len       device int32 [B], visible KV length of each request (for TND
 *              the requests' keys are packed back to back in this order;
 *              the guide's TND actual_seq_klen is the [B+1] prefix sum of
 *              these lengths, which the caller differences first).
 * batch        B, the number of requests (>= 0; 0 only when T = 0).
 * block_size   tokens per logical block, which is also a paged key's P axis
 *              (guide, section 四: the kernel splits every request's keys into
 *              blocks of block_size = 128); must be 128 (MSA_ERR_SHAPE
 *              otherwise).
 * layout       msa_layout_t.
 * sparse_mode  3 (right-down causal) or 0 (no causal mask).
 * init_blocks, local_blocks
 *              local_mask counts, each in [0, limit] with limit = MB for
 *              paged layouts and RoundUp(MB,16) for TND (guide, section 十).
 * out          device float32 [Hq, T, out_width], compact, written in full.
 * out_width    must equal msa_index_score_out_width(max_blocks).
 * stream       hipStream_t (as void*); the call is asynchronous on it.
 *
 * Device-data preconditions (the caller's contract, not checked on device):
 * the cu_seqlens_q rules above; paged: kv_len[b] <= MB*128 and
 * block_table[b, beta] in [0, NP) for beta < ceil(kv_len[b]/128); TND:
 * sum(kv_len) = T2 and ceil(kv_len[b]/128) <= MB.  Blocks at or past MB are
 * never scored or read, whatever kv_len says.
 *
 * NULL is accepted for pointers the call cannot read: kv_len, start_loc and
 * block_table when batch = 0, and out when T = 0.
 *
 * Ownership: every pointer is caller-owned; the library allocates no device
 * memory.  The only state it keeps between calls is one figure per device,
 * key type and batch kind (at most 64 requests, or more): the decode
 * kernel's workgroup slot count (CU count times occupancy), asked of the HIP
 * runtime on the first such decode launch on that device (read and written
 * atomically).  Calls may overlap, from several host threads and on the same
 * or different streams: they share no device memory.  Returns MSA_OK
 * or an error status; T = 0 returns MSA_OK without launching anything.
 * MSA_ERR_HIP reports a failure of this call's own runtime queries or
 * launch, never an error pending from earlier HIP work.  query, key and out
 * must be 16-byte aligned and a paged key's dim0 stride a multiple of 16
 * bytes (MSA_ERR_STRIDE otherwise).  Sizes past the kernels' 32-bit indexing
 * return MSA_ERR_SHAPE: out_width > 2^24, Hq > 2^16, batch > 2^30, T >= 2^31,
 * or one 128-token block of one head spanning 2 GiB or more of key memory.
 */
msa_status_t msa_index_score(const msa_tensor_t* query, const msa_tensor_t* key,
                             const int32_t* start_loc, const int32_t* block_table,
                             int64_t max_blocks, const float* scale,
                             const int32_t* cu_seqlens_q, const int32_t* kv_len,
                             int32_t batch, int32_t block_size, int32_t layout,
                             int32_t sparse_mode, int32_t init_blocks, int32_t local_blocks,
                             float* out, int64_t out_width, void* stream);

/* Same as msa_index_score, with the kernel family chosen by the caller:
 * family = -1 picks it from the sizes (as msa_index_score does), 0 forces the
 * decode tiles, 1 the prefill tiles.  Both families compute the same
 * definition for every valid input; the choice only changes speed.  Any other
 * family value returns MSA_ERR_ATTR.  For tests and benchmarks. */
msa_status_t msa_index_score_family(const msa_tensor_t* query, const msa_tensor_t* key,
                                    const int32_t* start_loc, const int32_t* block_table,
                                    int64_t max_blocks, const float* scale,
                                    const int32_t* cu_seqlens_q, const int32_t* kv_len,
                                    int32_t batch, int32_t block_size, int32_t layout,
                                    int32_t sparse_mode, int32_t init_blocks,
                                    int32_t local_blocks, float* out, int64_t out_width,
                                    void* stream, int32_t family);

/* Same as msa_index_score_family, with the local_mask window's placement
 * chosen by local_mode (msa_local_mode_t; any other value returns
 * MSA_ERR_ATTR).  With MSA_LOCAL_PER_QUERY start_loc is not read and may be
 * NULL; everything else (arguments, ownership, errors) is as for
 * msa_index_score.  msa_index_score is this call with MSA_LOCAL_PER_REQUEST
 * and family -1. */
msa_status_t msa_index_score_ex(const msa_tensor_t* query, const msa_tensor_t* key,
                                const int32_t* start_loc, const int32_t* block_table,
                                int64_t max_blocks, const float* scale,
                                const int32_t* cu_seqlens_q, const int32_t* kv_len,
                                int32_t batch, int32_t block_size, int32_t layout,
                                int32_t sparse_mode, int32_t init_blocks, int32_t local_blocks,
                                int32_t local_mode, float* out, int64_t out_width, void* stream,
                                int32_t family);

/* The block score on MXFP4 index vectors: the FP4 indexer variant of the
 * notes "MiniMax Sparse Attention: paper algorithm and code" (section 4.6,
 * path B, and section 8.2: MXFP4 is E2M1 values with an E8M0 scale per group
 * of elements, the block scores stay float32).  Same definition as
 * msa_index_score, with q and k~ the decoded MXFP4 vectors: element d of a
 * row is its E2M1 value times 2^(s - 127), s the E8M0 scale byte of group
 * d / 32 (E2M1: sign, 2 exponent bits with bias 1, 1 fraction bit; exponent
 * 0 gives 0 or 0.5; largest 6.  E8M0 255 is NaN).  The product is exact in
 * the MFMA's float32 accumulation up to summation rounding; the result
 * approximates the higher-precision score only as far as the encoding does.
 *
 * query        dtype MSA_DTYPE_MXFP4, [T, Hq, 64] bytes (128 elements, two per
 *              byte, the even element in the low nibble), compact, 16-byte
 *              aligned.
 * query_scale  device uint8 [T, Hq, 4] compact: E8M0 of elements 32c..32c+31.
 * key          dtype MSA_DTYPE_MXFP4, layouts as msa_index_score with a last
 *              axis of 64 bytes: TND [T2, Hkv, 64], BBND [NP, 128, Hkv, 64],
 *              BNBD [NP, Hkv, 128, 64]; paged dim0 stride any multiple of 16
 *              bytes.
 * key_scale    device uint8, compact, the key's layout with a last axis of 4:
 *              TND [T2, Hkv, 4], BBND [NP, 128, Hkv, 4], BNBD [NP, Hkv, 128, 4],
 *              indexed by page number (whatever the key's dim0 stride);
 *              4-byte aligned, like query_scale.
 * local_mode   msa_local_mode_t.  Everything else as msa_index_score.
 *
 * The kernel family is picked from the sizes, as msa_index_score does.
 * Returns as msa_index_score, plus MSA_ERR_DTYPE unless query and key are
 * MSA_DTYPE_MXFP4 and MSA_ERR_NULL for a NULL scale when T > 0 (with no
 * query tokens nothing is read and both scales may be NULL).  (msa_index_score and
 * its variants return MSA_ERR_SCALE for MXFP4 tensors: they cannot carry the
 * group scales.) */
msa_status_t msa_index_score_mxfp4(const msa_tensor_t* query, const uint8_t* query_scale,
                                   const msa_tensor_t* key, const uint8_t* key_scale,
                                   const int32_t* start_loc, const int32_t* block_table,
                                   int64_t max_blocks, const int32_t* cu_seqlens_q,
                                   const int32_t* kv_len, int32_t batch, int32_t block_size,
                                   int32_t layout, int32_t sparse_mode, int32_t init_blocks,
                                   int32_t local_blocks, int32_t local_mode, float* out,
                                   int64_t out_width, void* stream);

/* Same as msa_index_score_mxfp4, with the kernel family chosen by the caller
 * as for msa_index_score_family (-1 from the sizes, 0 the decode tiles, 1 the
 * prefill tiles; any other value returns MSA_ERR_ATTR).  For tests and
 * benchmarks. */
msa_status_t msa_index_score_mxfp4_family(const msa_tensor_t* query, const uint8_t* query_scale,
                                          const msa_tensor_t* key, const uint8_t* key_scale,
                                          const int32_t* start_loc, const int32_t* block_table,
                                          int64_t max_blocks, const int32_t* cu_seqlens_q,
                                          const int32_t* kv_len, int32_t batch,
                                          int32_t block_size, int32_t layout,
                                          int32_t sparse_mode, int32_t init_blocks,
                                          int32_t local_blocks, int32_t local_mode, float* out,
                                          int64_t out_width, void* stream, int32_t family);

/* Top-k block selection on the score rows: the stage the pages place after
 * the block score (the notes "MiniMax Sparse Attention: paper algorithm and
 * code", section 4.7 "Top-k Block
 * Selection", section 5.3 "Top-k" with the sparse_topk_select contract,
 * section 6.1 "Exp-free Top-k").
 *
 * For every query token t and index head h, among the blocks beta < num_valid
 * of the row scores[h, t, :] whose score is above -inf (NaN never qualifies),
 * the k with the highest scores, equal scores taken by lower block index,
 * are written to out[t, h, 0:k] in ascending block order; the slots past the
 * number selected hold -1.  Selection works on the raw scores, compared as
 * floats (so -0.0 and +0.0 are equal scores).
 *
 * scores     device float32 [Hq, T, width], compact (msa_index_score's out),
 *            4-byte aligned; not read when num_valid = 0.
 * Hq, T, width  sizes, >= 0, Hq <= 65535, T <= 2^33, width <= 2^24, and
 *            Hq * T * width below 2^63.
 * num_valid  blocks to consider, in [0, width] (the table width MB for an
 *            msa_index_score output; columns past it are padding).
 * k          1..64 (the sparse_topk_select contract uses 16).
 * out        device int32 [T, Hq, k], compact, 4-byte aligned, written in full.
 * stream     hipStream_t (as void*); the call is asynchronous on it.
 *
 * Ownership: caller-owned pointers; nothing is allocated or kept.  Returns
 * MSA_OK (also, without launching or checking pointers, when Hq * T = 0),
 * MSA_ERR_SHAPE for sizes out of range, MSA_ERR_ATTR for k out of range,
 * MSA_ERR_NULL for a NULL pointer the call must use, MSA_ERR_STRIDE for a
 * misaligned one, MSA_ERR_HIP if the launch fails. */
msa_status_t msa_block_topk(const float* scores, int64_t Hq, int64_t T, int64_t width,
                            int64_t num_valid, int32_t k, int32_t* out, void* stream);

/* Output width RoundUp(max(max_blocks, 1), 16) (guide, section 五: the last
 * axis is aligned to 16, and an all-empty packed batch clamps MB to 1). */
int64_t msa_index_score_out_width(int64_t max_blocks);

/* A static, human-readable name for a status code. */
const char* msa_status_str(int32_t status);

/* Which kernel family a call with these sizes would use: 0 = decode tiles
 * (16 query rows per tile, for short query runs per request), 1 = prefill
 * tiles (hundreds of query rows per tile), chosen when requests average at
 * least 128 query rows (tokens times heads per KV group) and the batch has
 * at least 1024 (T * Hq).  Host-only; for benchmarks and tests. */
int32_t msa_index_score_kernel_family(int64_t T, int32_t batch, int32_t Hq, int32_t Hkv);

#ifdef __cplusplus
}
#endif

#endif /* MSA_INDEX_SCORE_H */
