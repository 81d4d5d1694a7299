/*
 * msa_oracle.c -- plain, slow CPU oracle for the MSA index-branch block score.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the test suite, the package's smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library: its decoders, addressing and loops are written here from the
 * operator's definition.
 *
 * Definition followed (gitcode cann/ops-transformer issue #4117, "MsaIndexScore",
 * section "计算过程"; and the xxmr.cn guide to cann_ops_transformer.msa_index_score,
 * sections 二, 四, 五 and 八):
 *
 *   For a packed query token t of request b (cu_q[b] <= t < cu_q[b+1]),
 *   index head h and logical KV block beta of size P:
 *
 *     score[h,t,beta] = max over j in [beta*P, beta*P+P), j <= q_pos(t),
 *                       j < kv_len[b]  of  < q[t,h,:] , k~[j, h/g, :] >
 *
 *   g = Hq/Hkv; q_pos(t) = kv_len[b] - L_q(b) + (t - cu_q[b]) for the
 *   right-down causal mode (sparse_mode 3), kv_len[b]-1 for sparse_mode 0.
 *   k~ is the key row of logical block beta: for paged keys it is read from the
 *   physical page block_table[b,beta]; for packed (TND) keys from token
 *   koff_b + j with koff_b the sum of the earlier requests' kv_len.
 *   int8 keys: k~ = cast(k_int8) * scale[page, h_kv, j mod P] (TND:
 *   scale[koff_b + j, h_kv]); applied as a column scale of the dot product
 *   (Q.(K s) = (Q.cast K) s), in the order DOT -> DEQUANT -> MASK -> MAX.
 *   A block with no visible j scores -inf.  A request with kv_len = 0 skips the
 *   product entirely and all its entries are -inf (guide, section 四 and 8.2).
 *   After the block max, local_mask (guide, section 二) writes 1e30 on blocks
 *   [0, init_blocks) and then 1e29 on [max(0, start_loc+1-local_blocks),
 *   start_loc], the second overriding the first; it is skipped when both
 *   counts are 0.  With local_mode 1 the window ends instead at the block of
 *   the token's own position pos = kv_len[b] - L_q(b) + i, floor(pos / P):
 *   the paper's per-query local block b_local(i) = floor(i / B_k) (notes
 *   "MiniMax Sparse Attention: paper algorithm and code", section 4.7, on the
 *   forced local block); start_loc is then not read, and a token before
 *   position 0 gets no window.  Columns past the request's block count, up to
 *   the output width RoundUp(MB, 16), are -inf.
 *
 * Arithmetic: every input element is decoded exactly to a double (all input
 * formats embed exactly in binary64); the dot product is summed in binary64 in
 * ascending d; the int8 scale multiplies the binary64 sum; the maximum is
 * taken in binary64 and rounded once to binary32 (round-to-nearest-even by the
 * C conversion).  Rounding is monotone, so this is the correctly rounded block
 * maximum up to binary64 summation error.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* element type codes accepted by this oracle */
enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_I8 = 2, ORC_F8E4M3 = 3, ORC_F8E5M2 = 4, ORC_MXFP4 = 5 };
/* key layouts */
enum { ORC_TND = 0, ORC_BBND = 1, ORC_BNBD = 2 };

/* IEEE 754 binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
double orc_decode_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);              /* subnormal: f * 2^(1-15-10) */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/2^10) * 2^(e-15) */
  return s ? -v : v;
}

/* bfloat16: the high 16 bits of binary32: sign, 8-bit exponent (bias 127),
 * 7-bit fraction. */
double orc_decode_bf16(uint16_t x) {
  int s = x >> 15, e = (x >> 7) & 255, f = x & 127;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);             /* f * 2^(1-127-7) */
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + f), e - 134);  /* (1 + f/2^7) * 2^(e-127) */
  return s ? -v : v;
}

/* OCP 8-bit floating point, E4M3 ("fn": finite-only): sign, 4-bit exponent
 * (bias 7), 3-bit fraction; no infinities, S.1111.111 is NaN, largest 448. */
double orc_decode_e4m3fn(uint8_t x) {
  int s = x >> 7, e = (x >> 3) & 15, f = x & 7;
  double v;
  if (e == 15 && f == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)f, -9);               /* f * 2^(1-7-3) */
  else
    v = ldexp((double)(8 + f), e - 10);     /* (1 + f/8) * 2^(e-7) */
  return s ? -v : v;
}

/* OCP 8-bit floating point, E5M2: sign, 5-bit exponent (bias 15), 2-bit
 * fraction; exponent 31 holds infinities and NaNs as in IEEE 754. */
double orc_decode_e5m2(uint8_t x) {
  int s = x >> 7, e = (x >> 2) & 31, f = x & 3;
  double v;
  if (e == 31)
    v = f ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)f, -16);              /* f * 2^(1-15-2) */
  else
    v = ldexp((double)(4 + f), e - 17);     /* (1 + f/4) * 2^(e-15) */
  return s ? -v : v;
}

/* OCP microscaling FP4 element, E2M1: sign, 2-bit exponent (bias 1), 1-bit
 * fraction; exponent 0 is subnormal (0 or 0.5); no infinities or NaNs;
 * largest 6. */
double orc_decode_e2m1(uint8_t x) {
  int s = (x >> 3) & 1, e = (x >> 1) & 3, f = x & 1;
  double v = e == 0 ? 0.5 * f : ldexp((double)(2 + f), e - 2);   /* (1 + f/2) * 2^(e-1) */
  return s ? -v : v;
}

/* OCP microscaling shared scale, E8M0: an unsigned power-of-two exponent,
 * 2^(e - 127); e = 255 is NaN. */
double orc_decode_e8m0(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

static double elem(const void* base, int dtype, int64_t i) {
  switch (dtype) {
    case ORC_F16: return orc_decode_f16(((const uint16_t*)base)[i]);
    case ORC_BF16: return orc_decode_bf16(((const uint16_t*)base)[i]);
    case ORC_I8: return (double)((const int8_t*)base)[i];
    case ORC_F8E4M3: return orc_decode_e4m3fn(((const uint8_t*)base)[i]);
    case ORC_F8E5M2: return orc_decode_e5m2(((const uint8_t*)base)[i]);
    /* MXFP4 values: two per byte, element 2k in the low nibble (the group
     * scale is applied by the caller) */
    case ORC_MXFP4: return orc_decode_e2m1((((const uint8_t*)base)[i >> 1] >> (4 * (i & 1))) & 15);
    default: return NAN;
  }
}

/* Decode a whole buffer (used by the decoder tests). */
void orc_decode_buffer(const void* src, int dtype, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = elem(src, dtype, i);
}

typedef struct {
  const void* q; int q_dtype; int64_t T; int Hq; int D;
  const void* k; int k_dtype; int layout; int64_t k_dim0; int Hkv; int P;
  int64_t ks[4];                 /* key strides in elements */
  const int32_t* start_loc;
  const int32_t* block_table; int64_t MB;
  const float* scale;            /* int8 keys only */
  const uint8_t* q_mx;           /* MXFP4: E8M0 scale per 32 query elements [T, Hq, D/32] */
  const uint8_t* k_mx;           /* MXFP4: the same for keys, the key's layout with D/32 */
  const int32_t* cu_q; const int32_t* kv_len; int B;
  int sparse_mode; int init_blocks; int local_blocks;
  int local_mode;                /* 0: window ends at start_loc[b]; 1: at the token's block */
  int64_t W;                     /* output width */
  int64_t* koff;                 /* [B] packed-key offsets (TND) */
} orc_args;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* request that owns packed token t, or -1 */
static int owner(const orc_args* a, int64_t t) {
  for (int b = 0; b < a->B; ++b)
    if (a->cu_q[b] <= t && t < a->cu_q[b + 1]) return b;
  return -1;
}

/* Element offset of key[row j of request b][kv head hk][d = 0] and the index
 * of its int8 scale. */
static void key_row(const orc_args* a, int b, int64_t j, int hk, int64_t* off,
                    int64_t* sidx) {
  if (a->layout == ORC_TND) {
    int64_t row = a->koff[b] + j;
    *off = row * a->ks[0] + (int64_t)hk * a->ks[1];
    *sidx = row * a->Hkv + hk;
  } else {
    int64_t page = a->block_table[(int64_t)b * a->MB + j / a->P];
    int64_t jj = j % a->P;
    if (a->layout == ORC_BBND)
      *off = page * a->ks[0] + jj * a->ks[1] + (int64_t)hk * a->ks[2];
    else
      *off = page * a->ks[0] + (int64_t)hk * a->ks[1] + jj * a->ks[2];
    *sidx = (page * a->Hkv + hk) * a->P + jj;
  }
}

/* Index of the first MXFP4 scale of key row j of request b, head hk: the
 * scales form a compact tensor in the key's layout with D/32 per row. */
static int64_t mx_key_row(const orc_args* a, int b, int64_t j, int hk) {
  int64_t groups = a->D / 32;
  if (a->layout == ORC_TND) return ((a->koff[b] + j) * a->Hkv + hk) * groups;
  int64_t page = a->block_table[(int64_t)b * a->MB + j / a->P];
  int64_t jj = j % a->P;
  if (a->layout == ORC_BBND) return ((page * a->P + jj) * a->Hkv + hk) * groups;
  return ((page * a->Hkv + hk) * a->P + jj) * groups;
}

static int64_t d_stride(const orc_args* a) {
  return a->layout == ORC_TND ? a->ks[2] : a->ks[3];
}

/* One output entry out[h, t, beta], straight from the definition. */
static float entry(const orc_args* a, int h, int64_t t, int64_t beta, double* qrow) {
  int b = owner(a, t);
  if (b < 0) return -INFINITY;
  int64_t L = a->kv_len[b];
  if (L == 0) return -INFINITY;                 /* empty KV: request skipped */
  int64_t Lq = a->cu_q[b + 1] - a->cu_q[b];
  int64_t i = t - a->cu_q[b];
  int64_t qpos = (a->sparse_mode == 3) ? L - Lq + i : L - 1;

  double best = -INFINITY;
  int64_t NB = ceil_div(L, a->P);
  if (beta < NB) {
    int g = a->Hq / a->Hkv;
    int hk = h / g;
    int64_t jlo = beta * a->P;
    int64_t jhi = beta * a->P + a->P - 1;
    if (jhi > qpos) jhi = qpos;
    if (jhi > L - 1) jhi = L - 1;
    if (jhi >= jlo) {
      for (int d = 0; d < a->D; ++d) {
        qrow[d] = elem(a->q, a->q_dtype, (t * a->Hq + h) * (int64_t)a->D + d);
        if (a->q_dtype == ORC_MXFP4)             /* the group's shared scale */
          qrow[d] *= orc_decode_e8m0(a->q_mx[(t * a->Hq + h) * (int64_t)(a->D / 32) + d / 32]);
      }
      int64_t dst = d_stride(a);
      for (int64_t j = jlo; j <= jhi; ++j) {
        int64_t off, sidx;
        key_row(a, b, j, hk, &off, &sidx);
        int64_t mxr = a->k_dtype == ORC_MXFP4 ? mx_key_row(a, b, j, hk) : 0;
        double dot = 0.0;                        /* DOT */
        for (int d = 0; d < a->D; ++d) {
          double kv = elem(a->k, a->k_dtype, off + d * dst);
          if (a->k_dtype == ORC_MXFP4) kv *= orc_decode_e8m0(a->k_mx[mxr + d / 32]);
          dot += qrow[d] * kv;
        }
        if (a->k_dtype == ORC_I8) dot *= (double)a->scale[sidx];   /* DEQUANT */
        if (dot > best) best = dot;              /* MAX over the visible j */
      }
    }
  }
  float v = (float)best;                         /* one rounding to binary32 */

  /* local_mask, after the max; the local window overrides the init blocks.
   * Its last block is start_loc[b] (per request), or with local_mode 1 the
   * block holding the token itself, floor(pos / P) at its position
   * pos = L - Lq + i in the sequence; a token before position 0 has no block
   * and no window. */
  if (a->init_blocks > 0 || a->local_blocks > 0) {
    if (beta < a->init_blocks) v = 1e30f;
    int64_t s;
    if (a->local_mode == 0) {
      s = a->start_loc[b];
    } else {
      int64_t pos = L - Lq + i;
      s = pos >= 0 ? pos / a->P : -1;
    }
    int64_t lo = s + 1 - a->local_blocks;
    if (lo < 0) lo = 0;
    if (beta >= lo && beta <= s) v = 1e29f;
  }
  return v;
}

/* Caller-contract checks; returns 0 when the inputs are well formed. */
static int check(orc_args* a) {
  if (a->Hkv <= 0 || a->Hq % a->Hkv) return -1;
  if (a->B < 0 || a->cu_q[0] != 0 || a->cu_q[a->B] != a->T) return -2;
  for (int b = 0; b < a->B; ++b)
    if (a->cu_q[b + 1] < a->cu_q[b] || a->kv_len[b] < 0) return -3;
  int64_t acc = 0;
  for (int b = 0; b < a->B; ++b) {
    a->koff[b] = acc;
    acc += a->kv_len[b];
    int64_t NB = ceil_div(a->kv_len[b], a->P);
    if (NB > a->W) return -4;
    /* every layout: MB is the largest block count (paged: the table width;
       packed: max ceil(kv_len/P), guide section 五) */
    if (NB > a->MB) return -5;
    if (a->layout != ORC_TND) {
      for (int64_t beta = 0; beta < NB; ++beta) {
        int32_t p = a->block_table[(int64_t)b * a->MB + beta];
        if (p < 0 || p >= a->k_dim0) return -6;
      }
    }
  }
  if (a->layout == ORC_TND && acc != a->k_dim0) return -7;
  return 0;
}

typedef struct {
  orc_args* a;
  float* out;                /* full output, or NULL */
  const int64_t* pts;        /* (h, t, beta) triples, or NULL */
  int64_t n;                 /* number of tokens (full) or points */
  int tid, nth;
} job_t;

static void* worker(void* p) {
  job_t* J = (job_t*)p;
  orc_args* a = J->a;
  double* qrow = (double*)malloc(sizeof(double) * (a->D > 0 ? a->D : 1));
  if (J->pts == NULL) {
    for (int64_t t = J->tid; t < J->n; t += J->nth)
      for (int h = 0; h < a->Hq; ++h)
        for (int64_t beta = 0; beta < a->W; ++beta)
          J->out[((int64_t)h * a->T + t) * a->W + beta] = entry(a, h, t, beta, qrow);
  } else {
    for (int64_t i = J->tid; i < J->n; i += J->nth)
      J->out[i] = entry(a, (int)J->pts[3 * i], J->pts[3 * i + 1], J->pts[3 * i + 2], qrow);
  }
  free(qrow);
  return NULL;
}

static int run(orc_args* a, float* out, const int64_t* pts, int64_t n, int nthreads) {
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  if (n < nthreads) nthreads = n > 0 ? (int)n : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  job_t* jobs = (job_t*)malloc(sizeof(job_t) * nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].a = a; jobs[i].out = out; jobs[i].pts = pts; jobs[i].n = n;
    jobs[i].tid = i; jobs[i].nth = nthreads;
    pthread_create(&th[i], NULL, worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  return nthreads;
}

/* Output width: the block count rounded up to a multiple of 16 (guide,
 * section 五), with an all-empty packed batch clamped to one block. */
int64_t orc_out_width(int64_t max_blocks) {
  if (max_blocks < 1) max_blocks = 1;
  return (max_blocks + 15) / 16 * 16;
}

#define ORC_FILL_ARGS                                                          \
  orc_args a;                                                                  \
  memset(&a, 0, sizeof(a));                                                    \
  a.q = q; a.q_dtype = q_dtype; a.T = T; a.Hq = Hq; a.D = D;                   \
  a.k = k; a.k_dtype = k_dtype; a.layout = layout; a.k_dim0 = k_dim0;          \
  a.Hkv = Hkv; a.P = P;                                                        \
  for (int i = 0; i < 4; ++i) a.ks[i] = k_strides[i];                          \
  a.start_loc = start_loc; a.block_table = block_table; a.MB = MB;             \
  a.scale = scale; a.q_mx = q_mx; a.k_mx = k_mx;                              \
  a.cu_q = cu_q; a.kv_len = kv_len; a.B = B;                                   \
  a.sparse_mode = sparse_mode; a.init_blocks = init_blocks;                    \
  a.local_blocks = local_blocks; a.local_mode = local_mode;                    \
  a.W = orc_out_width(MB);                                                     \
  a.koff = (int64_t*)calloc(B > 0 ? B : 1, sizeof(int64_t));                   \
  int rc = check(&a);                                                          \
  if (rc) { free(a.koff); return rc; }

/* Full output [Hq, T, W] (W = orc_out_width(MB)).  Returns the number of
 * threads used (> 0), or a negative contract-violation code. */
int orc_index_score(const void* q, int q_dtype, int64_t T, int Hq, int D,
                    const void* k, int k_dtype, int layout, int64_t k_dim0, int Hkv,
                    int P, const int64_t* k_strides, const int32_t* start_loc,
                    const int32_t* block_table, int64_t MB, const float* scale,
                    const uint8_t* q_mx, const uint8_t* k_mx,
                    const int32_t* cu_q, const int32_t* kv_len, int B, int sparse_mode,
                    int init_blocks, int local_blocks, int local_mode, float* out,
                    int nthreads) {
  ORC_FILL_ARGS
  int used = run(&a, out, NULL, T, nthreads);
  free(a.koff);
  return used;
}

/* Selected entries: pts holds n triples (h, t, beta); vals receives them. */
int orc_index_score_points(const void* q, int q_dtype, int64_t T, int Hq, int D,
                           const void* k, int k_dtype, int layout, int64_t k_dim0, int Hkv,
                           int P, const int64_t* k_strides, const int32_t* start_loc,
                           const int32_t* block_table, int64_t MB, const float* scale,
                           const uint8_t* q_mx, const uint8_t* k_mx,
                           const int32_t* cu_q, const int32_t* kv_len, int B,
                           int sparse_mode, int init_blocks, int local_blocks,
                           int local_mode, const int64_t* pts, int64_t n, float* vals,
                           int nthreads) {
  ORC_FILL_ARGS
  int used = run(&a, vals, pts, n, nthreads);
  free(a.koff);
  return used;
}

/* ------------------------------------------------------------------------
 * Top-k block selection on the score rows (the follow-on stage the pages
 * describe after the block score: the notes "MiniMax Sparse Attention: paper
 * algorithm and code", section 4.7
 * "Equation (7): Top-k Block Selection" and section 5.3 "Top-k", with the
 * sparse_topk_select contract listed there; section 6.1 "Exp-free Top-k").
 *
 * For each query token t and index head h, over the row score[h, t, :]:
 *   candidates  = blocks beta < num_valid whose score is above -inf (a block
 *                 with no visible key is invalid; NaN is never a candidate);
 *   order       = by score, highest first, equal scores by lower beta first
 *                 (the pages leave the tie order open; this is the reading);
 *   selection   = the first min(k, #candidates) of that order;
 *   output      = out[t, h, 0:k]: the selected block indices in ascending
 *                 index order (not score order), then -1 for the rest.
 * Selection works on the raw scores (no exp or normalisation).
 * ------------------------------------------------------------------------ */
typedef struct {
  float s;
  int64_t b;
} orc_cand;

static int orc_cand_order(const void* x, const void* y) {
  const orc_cand* u = (const orc_cand*)x;
  const orc_cand* v = (const orc_cand*)y;
  if (u->s > v->s) return -1;
  if (u->s < v->s) return 1;
  return (u->b > v->b) - (u->b < v->b);
}

static int orc_index_order(const void* x, const void* y) {
  const int32_t u = *(const int32_t*)x, v = *(const int32_t*)y;
  return (u > v) - (u < v);
}

/* scores: [Hq, T, W] float32; out: [T, Hq, k] int32.  Returns 0, or -1 for a
 * contract violation (negative sizes, num_valid outside [0, W], k outside
 * [1, 64], W above 2^31 - 1). */
int orc_block_topk(const float* scores, int64_t Hq, int64_t T, int64_t W,
                   int64_t num_valid, int k, int32_t* out) {
  if (Hq < 0 || T < 0 || W < 0 || W > INT32_MAX || num_valid < 0 || num_valid > W ||
      k < 1 || k > 64)
    return -1;
  orc_cand* cand = (orc_cand*)malloc((size_t)(W > 0 ? W : 1) * sizeof(orc_cand));
  int32_t sel[64];
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < Hq; ++h) {
      const float* row = scores + (h * T + t) * W;
      int64_t n = 0;
      for (int64_t b = 0; b < num_valid; ++b) {
        if (row[b] > -INFINITY) {
          cand[n].s = row[b];
          cand[n].b = b;
          ++n;
        }
      }
      qsort(cand, (size_t)n, sizeof(orc_cand), orc_cand_order);
      const int m = n < k ? (int)n : k;
      for (int i = 0; i < m; ++i) sel[i] = (int32_t)cand[i].b;
      qsort(sel, (size_t)m, sizeof(int32_t), orc_index_order);
      int32_t* dst = out + (t * Hq + h) * k;
      for (int i = 0; i < k; ++i) dst[i] = i < m ? sel[i] : -1;
    }
  }
  free(cand);
  return 0;
}
