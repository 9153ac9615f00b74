/*
 * Plain fp64 CPU oracle for split-KV MLA decode attention over a paged FP8 cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this
 * file; only the test suite, the smoke check and the benchmark's CPU-baseline leg use
 * it. It shares no code, header, table or constant generator with the HIP library.
 *
 * What it computes is the plain, unsplit definition of attention decode that the
 * split-KV method reaches faster:
 *
 *   Geometry [TensorRT-LLM issue #20510 "CuTe DSL FP8 MLA decode slower after #19338",
 *   Setup]: each cached token is one row of 576 FP8 E4M3 bytes, a 512-wide latent
 *   followed by a 64-wide rope part; the cache is paged with 32 tokens per page; q and
 *   KV are both E4M3. V is the 512-wide latent of the same row (MLA absorption: the
 *   latent serves as both the K prefix and V).
 *
 *   Scales [same issue, Repro 1: the run() arguments softmax_scale and output_scale]:
 *   scores are softmax_scale * (q . k); output_scale multiplies O only.
 *
 *   Causal MTP verify [the q = 8 "MTP verify" shape of the same issue's Setup]: with
 *   q_len query tokens per request, query token j sees KV tokens 0 .. L - q_len + j
 *   inclusive, i.e. n_j = L - q_len + j + 1 of them; q_len = 1 gives n = L.
 *
 *   For each request b, query j, head h:
 *     s_i  = softmax_scale * sum_{d<576} q_d * K_{i,d}            (fp64, exact sum)
 *     m    = max_i s_i,  w_i = exp(s_i - m),  l = sum_i w_i
 *     O_d  = output_scale * sum_i w_i * V_{i,d} / l                (d < 512)
 *     LSE  = m + ln(l)        (natural log of sum_i exp(s_i); output_scale excluded)
 *
 * The (max, sum, O) triple is the per-row state the reduction merges [TensorRT-LLM PR
 * #20380 "trtllm-gen FMHA: split the KV partials of a row across thread groups in
 * fmhaReductionKernel", Description]; here it is formed once over all keys, unsplit.
 *
 * E4M3 decoding follows the OCP FP8 E4M3 ("fn") encoding: 1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits, subnormals m * 2^-9, the codes 0x7F / 0xFF are NaN and
 * there is no infinity. Every E4M3 value is exact in fp64 (and in BF16, as PR #17441
 * "m3 decode perf clean" notes for the widening of E4M3 to BF16).
 *
 * BF16 cache variant [issue #20510, Repro 2: the BF16 kernel measured beside the FP8
 * one]: q and the cache hold BF16 values instead (1 sign bit, 8 exponent bits with bias
 * 127, 7 mantissa bits, subnormals m * 2^-133, exponent 255 for infinities and NaN);
 * rows are 576 BF16 values (1152 bytes) and everything else is unchanged. BF16 values
 * are exact in fp64; a BF16 dot product is not always exact in fp64 (the product
 * exponents can span more than 53 bits), so there the sum is the fp64 sum in dimension
 * order.
 *
 * Exactness of the dot product: every E4M3 product is a multiple of 2^-18 with
 * magnitude below 2^18, so every partial sum of at most 576 of them is a multiple of
 * 2^-18 below 2^28 and fits fp64's 53-bit significand; the sum is exact in any order.
 *
 * Row order: flat row id r = (b * q_len + j) * H + h, the layout of q [B][q_len][H][576]
 * and of O [B][q_len][H][512].
 *
 * Attention sinks [the same PR, Description: the reduction applies sinks after the
 * combine]: the pages name sinks without a formula; this oracle takes the usual form,
 * one extra logit sigma_h per head that joins the softmax denominator only:
 *     m = max(max_i s_i, sigma_h),  l = sum_i exp(s_i - m) + exp(sigma_h - m)
 *     O_d = output_scale * sum_i exp(s_i - m) V_{i,d} / l,   LSE = m + ln(l)
 * so LSE is the log of the whole denominator and O_d = sum_i exp(s_i - LSE) V_{i,d}.
 * sigma_h = -inf gives back the definition without a sink.
 *
 * MXFP8 output [TensorRT-LLM PR #17441 "m3 decode perf clean", the commit messages on
 * the MXFP8 quantize-tile epilogue, on its scale byte 0, and on the sparse decode merge:
 * the merge emits E4M3 values with UE8M0 block scales next to the BF16 O it stores,
 * bit-identical to quantizing that BF16 tensor afterwards]: blocks of 32 consecutive
 * elements of a row. The block scale is amax / 448 rounded up to a power of two, with
 * the outcome those messages state for the two edge cases:
 *   - a block whose amax is exactly 1.75 * 2^k (= 448 * 2^(k-8)) gets the next
 *     exponent, k - 7: the scale is 2^e with e the smallest integer such that
 *     amax < 448 * 2^e (strictly), clamped to the E8M0 range [-127, 127] and stored
 *     as e + 127;
 *   - a block whose scale byte is 0 (e = -127: amax < 448 * 2^-127, including an
 *     all-zero block) saturates: the reciprocal of its scale is taken as infinite, so
 *     every non-zero element becomes the largest E4M3 magnitude, 448, with its sign.
 *     A zero element has no magnitude to saturate and stays a zero code with its sign
 *     (a reading: the messages say only that the block saturates).
 * Otherwise each element is the E4M3 value nearest to x / 2^e, ties to the even code,
 * with the sign of x (|x / 2^e| < 448, so nothing else saturates).
 *
 * Key bounds [issue #20510, Repro 1: kv_bounds is one of the run() arguments added
 * after #19338, named without a description]: read here as one half-open window
 * [start_b, end_b) of key positions per request, int32 [B][2], that every query of
 * request b is confined to in addition to the causal rule: query j sees the keys i
 * with start_b <= i < end_b and i <= L - q_len + j. A negative start counts as 0; keys
 * outside the window are never read, so block-table entries of pages wholly outside it
 * may hold anything. A row whose window holds no visible key has O = 0 and
 * LSE = -inf (LSE = sigma_h with a sink: the sink is then the whole denominator).
 *
 * Threads: rows are handed out to POSIX threads through an atomic counter; each row's
 * arithmetic is sequential and independent of the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_D_QK 576
#define ORACLE_D_V 512
#define ORACLE_PAGE 32

/* Decode one OCP E4M3FN code to fp64. */
double oracle_e4m3_to_double(uint8_t code) {
  int sign = code >> 7;
  int expo = (code >> 3) & 15;
  int mant = code & 7;
  double v;
  if (expo == 15 && mant == 7) return NAN;
  if (expo == 0)
    v = ldexp((double)mant, -9); /* 0.mmm * 2^(1-7) */
  else
    v = ldexp(8.0 + mant, expo - 7 - 3); /* 1.mmm * 2^(e-7) */
  return sign ? -v : v;
}

/* Decode one BF16 bit pattern to fp64. */
double oracle_bf16_to_double(uint16_t code) {
  int sign = code >> 15;
  int expo = (code >> 7) & 0xFF;
  int mant = code & 0x7F;
  double v;
  if (expo == 0xFF) return mant ? NAN : (sign ? -INFINITY : INFINITY);
  if (expo == 0)
    v = ldexp((double)mant, -126 - 7);          /* 0.mmmmmmm * 2^-126 */
  else
    v = ldexp(128.0 + mant, expo - 127 - 7);    /* 1.mmmmmmm * 2^(e-127) */
  return sign ? -v : v;
}

int oracle_hw_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

typedef struct {
  const uint8_t* q;
  const uint8_t* kv;
  const int32_t* bt;
  const int32_t* kv_lens;
  int32_t batch, q_len, heads;
  int64_t bt_stride, num_pages;
  double softmax_scale, output_scale;
  const double* sinks; /* [heads] extra logits, or NULL */
  const int32_t* bounds; /* [batch][2] key windows [start, end), or NULL */
  int bf16;            /* 0: E4M3 elements (1 byte), 1: BF16 elements (2 bytes) */
  double* table16;     /* BF16 decode table (65536 entries) when bf16 */
  const int64_t* rows;
  int64_t nrows;
  double* out_o;
  double* out_lse;
  double table[256];
  int64_t next; /* atomic row counter */
  int error;    /* first error seen (atomic) */
} oracle_job;

/* Error codes (negative). */
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_PAGE (-2)
#define ORACLE_ERR_ROW (-3)
#define ORACLE_ERR_NOMEM (-4)

/* Decode the 576 elements of one row (of q or of the cache) to fp64. */
static void decode_row(const oracle_job* J, const uint8_t* src, double* dst) {
  if (J->bf16) {
    for (int d = 0; d < ORACLE_D_QK; ++d) {
      uint16_t code = (uint16_t)(src[2 * d] | (src[2 * d + 1] << 8)); /* little endian */
      dst[d] = J->table16[code];
    }
  } else {
    for (int d = 0; d < ORACLE_D_QK; ++d) dst[d] = J->table[src[d]];
  }
}

static int one_row(oracle_job* J, int64_t idx, double* s, double* acc) {
  int64_t r = J->rows ? J->rows[idx] : idx;
  int64_t rows_total = (int64_t)J->batch * J->q_len * J->heads;
  if (r < 0 || r >= rows_total) return ORACLE_ERR_ROW;
  int64_t bj = r / J->heads;
  int32_t b = (int32_t)(bj / J->q_len);
  int32_t j = (int32_t)(bj % J->q_len);
  int64_t L = J->kv_lens[b];
  int64_t n = L - J->q_len + j + 1; /* causal rule: query token j sees keys 0 .. n-1 */
  if (n < 1) return ORACLE_ERR_ARG;
  if ((n + ORACLE_PAGE - 1) / ORACLE_PAGE > J->bt_stride) return ORACLE_ERR_ARG;
  /* keys of the row: [k0, k1), the causal range cut to the request's window */
  int64_t k0 = 0, k1 = n;
  if (J->bounds) {
    int64_t start = J->bounds[2 * (int64_t)b], end = J->bounds[2 * (int64_t)b + 1];
    if (start > k0) k0 = start;
    if (end < k1) k1 = end;
  }

  const int64_t row_bytes = (int64_t)ORACLE_D_QK * (J->bf16 ? 2 : 1);
  double qd[ORACLE_D_QK], kd[ORACLE_D_QK];
  decode_row(J, J->q + r * row_bytes, qd);

  /* scores s_i = softmax_scale * (q . K_i) */
  double m = -INFINITY;
  for (int64_t i = k0; i < k1; ++i) {
    int64_t page = J->bt[(int64_t)b * J->bt_stride + i / ORACLE_PAGE];
    if (page < 0 || page >= J->num_pages) return ORACLE_ERR_PAGE;
    decode_row(J, J->kv + (page * ORACLE_PAGE + i % ORACLE_PAGE) * row_bytes, kd);
    double dot = 0.0;
    for (int d = 0; d < ORACLE_D_QK; ++d) dot += qd[d] * kd[d];
    s[i] = J->softmax_scale * dot;
    if (s[i] > m) m = s[i];
  }
  /* a sink logit joins the max and, below, the normaliser */
  double sigma = J->sinks ? J->sinks[r % J->heads] : -INFINITY;
  if (sigma > m) m = sigma;
  /* weights, normaliser, and the weighted sum of V (the first 512 bytes of each row) */
  for (int d = 0; d < ORACLE_D_V; ++d) acc[d] = 0.0;
  double l = J->sinks ? exp(sigma - m) : 0.0;
  for (int64_t i = k0; i < k1; ++i) {
    int64_t page = J->bt[(int64_t)b * J->bt_stride + i / ORACLE_PAGE];
    decode_row(J, J->kv + (page * ORACLE_PAGE + i % ORACLE_PAGE) * row_bytes, kd);
    double w = exp(s[i] - m);
    l += w;
    for (int d = 0; d < ORACLE_D_V; ++d) acc[d] += w * kd[d]; /* V: the first 512 */
  }
  double* o = J->out_o + idx * ORACLE_D_V;
  if (l == 0.0) { /* no visible key and no sink */
    for (int d = 0; d < ORACLE_D_V; ++d) o[d] = 0.0;
    J->out_lse[idx] = -INFINITY;
    return 0;
  }
  for (int d = 0; d < ORACLE_D_V; ++d) o[d] = J->output_scale * acc[d] / l;
  J->out_lse[idx] = m + log(l);
  return 0;
}

static void* worker(void* arg) {
  oracle_job* J = (oracle_job*)arg;
  int64_t cap = 0;
  double* s = NULL;
  double acc[ORACLE_D_V];
  for (;;) {
    int64_t idx = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
    if (idx >= J->nrows) break;
    if (__atomic_load_n(&J->error, __ATOMIC_RELAXED) != 0) break;
    int64_t r = J->rows ? J->rows[idx] : idx;
    int64_t need = 1;
    if (r >= 0 && r < (int64_t)J->batch * J->q_len * J->heads) {
      int32_t b = (int32_t)(r / J->heads / J->q_len);
      need = J->kv_lens[b] > 0 ? J->kv_lens[b] : 1;
    }
    if (need > cap) {
      free(s);
      s = (double*)malloc(sizeof(double) * (size_t)need);
      cap = need;
      if (!s) {
        int zero = 0;
        __atomic_compare_exchange_n(&J->error, &zero, ORACLE_ERR_NOMEM, 0, __ATOMIC_RELAXED,
                                    __ATOMIC_RELAXED);
        break;
      }
    }
    int rc = one_row(J, idx, s, acc);
    if (rc != 0) {
      int zero = 0;
      __atomic_compare_exchange_n(&J->error, &zero, rc, 0, __ATOMIC_RELAXED, __ATOMIC_RELAXED);
      break;
    }
  }
  free(s);
  return NULL;
}

/*
 * Compute O (fp64 [nrows][512]) and LSE (fp64 [nrows]) for the listed flat rows
 * (rows == NULL: all B*q_len*H rows in order). Inputs are host arrays:
 *   q       uint8 E4M3 [B][q_len][H][576]
 *   kv      uint8 E4M3 [num_pages][32][576]
 *   bt      int32 [B][bt_stride], page indices into kv
 *   kv_lens int32 [B], each >= q_len
 * sinks   fp64 [H] sink logits (see the header), or NULL for none
 * bf16    0: q and kv hold E4M3 codes; 1: BF16 bit patterns (2 bytes per element)
 * nthreads <= 0 uses every online core. Returns 0 or a negative error code; on error
 * the outputs are unspecified.
 */
int oracle_mla_decode_rows_bounded(const uint8_t* q, const uint8_t* kv, const int32_t* bt,
                                   const int32_t* kv_lens, int32_t batch, int32_t q_len,
                                   int32_t num_heads, int64_t bt_stride, int64_t num_pages,
                                   double softmax_scale, double output_scale,
                                   const double* sinks, int bf16, const int32_t* kv_bounds,
                                   const int64_t* rows, int64_t nrows, double* out_o,
                                   double* out_lse, int nthreads) {
  if (!q || !kv || !bt || !kv_lens || !out_o || !out_lse) return ORACLE_ERR_ARG;
  if (batch < 1 || q_len < 1 || num_heads < 1 || bt_stride < 1 || num_pages < 1 || nrows < 0)
    return ORACLE_ERR_ARG;
  oracle_job* J = (oracle_job*)calloc(1, sizeof(oracle_job));
  if (!J) return ORACLE_ERR_NOMEM;
  J->q = q;
  J->kv = kv;
  J->bt = bt;
  J->kv_lens = kv_lens;
  J->batch = batch;
  J->q_len = q_len;
  J->heads = num_heads;
  J->bt_stride = bt_stride;
  J->num_pages = num_pages;
  J->softmax_scale = softmax_scale;
  J->output_scale = output_scale;
  J->sinks = sinks;
  J->bounds = kv_bounds;
  J->bf16 = bf16 ? 1 : 0;
  J->rows = rows;
  J->nrows = nrows;
  J->out_o = out_o;
  J->out_lse = out_lse;
  for (int c = 0; c < 256; ++c) J->table[c] = oracle_e4m3_to_double((uint8_t)c);
  if (J->bf16) {
    J->table16 = (double*)malloc(sizeof(double) * 65536);
    if (!J->table16) {
      free(J);
      return ORACLE_ERR_NOMEM;
    }
    for (int c = 0; c < 65536; ++c) J->table16[c] = oracle_bf16_to_double((uint16_t)c);
  }

  int nt = nthreads > 0 ? nthreads : oracle_hw_threads();
  if (nt > nrows) nt = nrows > 0 ? (int)nrows : 1;
  if (nt > 256) nt = 256;
  pthread_t tid[256];
  int started = 0;
  for (int t = 1; t < nt; ++t) {
    if (pthread_create(&tid[started], NULL, worker, J) == 0) ++started;
  }
  worker(J);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
  int rc = J->error;
  free(J->table16);
  free(J);
  return rc;
}

/* The same without key bounds. */
int oracle_mla_decode_rows_ex(const uint8_t* q, const uint8_t* kv, const int32_t* bt,
                              const int32_t* kv_lens, int32_t batch, int32_t q_len,
                              int32_t num_heads, int64_t bt_stride, int64_t num_pages,
                              double softmax_scale, double output_scale, const double* sinks,
                              int bf16, const int64_t* rows, int64_t nrows, double* out_o,
                              double* out_lse, int nthreads) {
  return oracle_mla_decode_rows_bounded(q, kv, bt, kv_lens, batch, q_len, num_heads, bt_stride,
                                        num_pages, softmax_scale, output_scale, sinks, bf16,
                                        NULL, rows, nrows, out_o, out_lse, nthreads);
}

/* The same without sinks. */
int oracle_mla_decode_rows(const uint8_t* q, const uint8_t* kv, const int32_t* bt,
                           const int32_t* kv_lens, int32_t batch, int32_t q_len,
                           int32_t num_heads, int64_t bt_stride, int64_t num_pages,
                           double softmax_scale, double output_scale, const int64_t* rows,
                           int64_t nrows, double* out_o, double* out_lse, int nthreads) {
  return oracle_mla_decode_rows_ex(q, kv, bt, kv_lens, batch, q_len, num_heads, bt_stride,
                                   num_pages, softmax_scale, output_scale, NULL, 0, rows,
                                   nrows, out_o, out_lse, nthreads);
}

/*
 * Round each x[i] to the nearest BF16 value (8 significant bits, fp32's exponent range,
 * subnormals down to 2^-133), ties to even; magnitudes that round past the largest
 * finite BF16 value become infinities. NaN stays NaN.
 */
void oracle_round_bf16(const double* x, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    double v = x[i];
    if (v == 0.0 || isnan(v) || isinf(v)) {
      out[i] = v;
      continue;
    }
    int k;
    frexp(v, &k);               /* |v| in [2^(k-1), 2^k) */
    int e = k - 1;              /* floor(log2 |v|) */
    if (e < -126) e = -126;     /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, e - 7);
    double r = nearbyint(v / quantum) * quantum; /* default rounding: to nearest even */
    if (fabs(r) >= ldexp(1.0, 128)) r = v > 0 ? INFINITY : -INFINITY;
    out[i] = r;
  }
}

/* The E4M3 code nearest to y (|y| <= 448), ties to the even code, sign of y kept. */
static uint8_t e4m3_nearest(double y) {
  double a = fabs(y);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double err = fabs(oracle_e4m3_to_double((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/*
 * MXFP8 quantization of nrows rows of 512 values (each already a BF16 value): codes
 * uint8 E4M3 [nrows][512], scales uint8 E8M0 [nrows][16] (one per 32 consecutive
 * elements, biased by 127). Returns 0, or ORACLE_ERR_ARG for a non-finite input.
 */
int oracle_mxfp8_quantize(const double* x, int64_t nrows, uint8_t* codes, uint8_t* scales) {
  const int block = 32;
  for (int64_t r = 0; r < nrows; ++r) {
    for (int blk = 0; blk < ORACLE_D_V / block; ++blk) {
      const double* xb = x + r * ORACLE_D_V + blk * block;
      double amax = 0.0;
      for (int i = 0; i < block; ++i) {
        if (!isfinite(xb[i])) return ORACLE_ERR_ARG;
        if (fabs(xb[i]) > amax) amax = fabs(xb[i]);
      }
      /* smallest e with amax < 448 * 2^e, within the E8M0 range */
      int e = -127;
      while (e < 127 && amax >= ldexp(448.0, e)) ++e;
      scales[r * (ORACLE_D_V / block) + blk] = (uint8_t)(e + 127);
      for (int i = 0; i < block; ++i) {
        uint8_t* c = &codes[r * ORACLE_D_V + blk * block + i];
        if (e == -127) {
          /* scale byte 0: the block saturates; zeros stay zeros */
          uint8_t neg = signbit(xb[i]) ? 0x80 : 0x00;
          *c = (uint8_t)(neg | (xb[i] != 0.0 ? 0x7E : 0x00));
        } else {
          *c = e4m3_nearest(ldexp(xb[i], -e));
        }
      }
    }
  }
  return 0;
}
