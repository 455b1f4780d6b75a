/*
 * Reference oracle for single-token MLA decode: TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 C.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this file's shared library; the product
 * path never does.  It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * What it computes (kernelindex.com "kernelbot-amd-mixed-mla-695854", the
 * chunked torch attention fallback and its mxfp4 slice dequantiser): for each
 * request b and query head h,
 *     s_t = (q_hat . k_hat_t) / sqrt(576)      over the request's tokens t
 *     p   = softmax(s)
 *     o   = sum_t p_t * k_hat_t[0:512]         (V is the first 512 latent dims)
 * on dequantised inputs, then o is rounded to bfloat16 (round to nearest even).
 * The softmax scale 1/sqrt(576) is the one both "kernelbot-amd-mixed-mla-668813"
 * and "...-600081" define from the 576-wide query/key head.
 *
 * Dequantisers, written from the number formats themselves:
 *   bf16       : exact widening of the upper half of an IEEE fp32.
 *   fp8 e4m3fn : OCP 8-bit float, bias 7, no infinities, S.1111.111 = NaN,
 *                subnormals m/8 * 2^-6; times the per-tensor fp32 scale
 *                (the "fp8" kv entry is a (buffer, scale) pair on page 695854).
 *   mxfp4      : OCP MX e2m1 element times an e8m0 block scale 2^(e-127), one
 *                scale per 32 consecutive elements; byte i of a packed row holds
 *                element 2i in its low nibble and 2i+1 in its high nibble
 *                (page 668813, the e2m1 lookup table and the stage-1 nibble
 *                unpacking; page 695854, the mxfp4 slice dequantiser).
 *
 * Paging (a reading; the pages address the cache either contiguously by token
 * or through aiter page tables): token t of request b sits at logical position
 * g = base_b + t where base_b = kv_indptr[b] when page_indptr is NULL (one
 * page table over the concatenated token stream), else base_b = 0 and the
 * request's own table starts at page_table[page_indptr[b]].  Its physical row
 * is page_table[first + g / P] * P + g % P.
 *
 * Split cache (page 695854, its mxfp4 q=1 routes): the keys may come from
 * one cache and the values from another holding the same tokens in the same
 * physical rows - there the mxfp4 cache supplies all 576 key dims and the
 * fp8 cache (with its per-tensor scale) the first 512 value dims.  With a
 * separate value cache, v_t is that cache's dequantised row t, dims 0..511;
 * otherwise it is k_hat_t[0:512] as above.
 *
 * Split-wise variant (page 668813, the split-K stage 1 and its log2 combine;
 * page 600081, the split-K kernels): the token range of a request is cut into
 * S chunks of ceil(L/S) tokens; each non-empty chunk yields a normalised
 * partial output and its log-sum-exp; the partials are merged with weights
 * exp(lse_s - max lse).  Empty chunks are skipped.  This is an exact
 * re-association of the same softmax; the oracle keeps it only to pin the
 * unsplit path (they must agree to rounding).
 *
 * Quantisers used to build caches (fp8 per-tensor and OCP MX mxfp4):
 *   fp8 : amax = max |x| (>= 1e-12); scale = amax / 448 in fp32; code =
 *         nearest e4m3fn value to clamp(x / scale, -448, 448) with x / scale
 *         an fp32 division, ties to the even code (page 668813, the naive
 *         per-tensor fp8 quantiser).  A static scale may be passed instead.
 *   mxfp4: per block of 32: X = floor(log2(amax)) - 2, e8m0 = X + 127 clamped
 *         to [0, 254]; element code = nearest e2m1 value to x / 2^X, ties to
 *         even, saturating at +-6; an all-zero block gets e8m0 = 0.  (OCP MX
 *         v1.0 scale rule; the pages call a library quantiser whose rule they
 *         do not print.)
 * Both quantisers search the code table exhaustively for the nearest value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_HEADS 16
#define ORC_DQK 576
#define ORC_DV 512
#define ORC_PACKED 288
#define ORC_NBLK 18

enum { ORC_BF16 = 0, ORC_FP8 = 1, ORC_MXFP4 = 2 };
enum { ORC_OK = 0, ORC_EARG = -1, ORC_EINDEX = -2, ORC_ENOMEM = -3 };

/* ---------------------------------------------------------------- codecs */

double orc_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

double orc_e4m3fn_to_f64(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

double orc_e2m1_to_f64(uint8_t nib) {
  /* S EE M: exponent bias 1, subnormal 0.5 * M */
  int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

double orc_e8m0_to_f64(uint8_t c) {
  if (c == 255) return NAN;
  return ldexp(1.0, (int)c - 127);
}

/* Round a double to the nearest bfloat16, ties to even; returns the bits. */
uint16_t orc_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  double a = fabs(x);
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) -> leading bit weight 2^(e-1) */
  int lead = e - 1;
  if (lead < -126) lead = -126; /* subnormal spacing 2^-133 */
  double quantum = ldexp(1.0, lead - 7);
  double r = nearbyint(a / quantum) * quantum; /* current mode is nearest-even */
  if (r > 3.3895313892515355e38) return sign | 0x7F80; /* overflow to inf */
  float f = (float)r;                                  /* exact */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* --------------------------------------------------------- quantisers */

/* Nearest e4m3fn code to v (|v| <= 448 assumed after clamping), ties to the
 * code with an even mantissa LSB; exhaustive search over the 127 finite
 * non-negative codes. */
static uint8_t nearest_e4m3fn(float v) {
  double a = fabs((double)v);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 127; c++) {
    double d = fabs(orc_e4m3fn_to_f64((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)((signbit(v) ? 0x80 : 0) | best);
}

static uint8_t nearest_e2m1(double v) {
  double a = fabs(v);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 8; c++) {
    double d = fabs(orc_e2m1_to_f64((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  if (a > 6.0) best = 7;
  return (uint8_t)((signbit(v) ? 8 : 0) | best);
}

/* amax over bf16 values, as fp32 (exact: it is one of the inputs). */
float orc_amax_bf16(const uint16_t* x, int64_t n) {
  double m = 0.0;
  for (int64_t i = 0; i < n; i++) {
    double a = fabs(orc_bf16_to_f64(x[i]));
    if (a > m) m = a;
  }
  return (float)m;
}

/* fp8 per-tensor scale from an amax: max(amax, 1e-12) / 448 in fp32. */
float orc_fp8_scale_from_amax(float amax) {
  float a = amax < 1e-12f ? 1e-12f : amax;
  volatile float r = a / 448.0f;
  return r;
}

/* Quantise n bf16 values with a given fp32 scale. */
int orc_quant_fp8(const uint16_t* x, int64_t n, float scale, uint8_t* codes) {
  if (!x || !codes || n < 0 || !(scale > 0.0f)) return ORC_EARG;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    float xf = (float)orc_bf16_to_f64(x[i]);
    volatile float q = xf / scale; /* fp32 IEEE division */
    float c = q;
    if (c > 448.0f) c = 448.0f;
    if (c < -448.0f) c = -448.0f;
    codes[i] = nearest_e4m3fn(c);
  }
  return ORC_OK;
}

/* OCP MX mxfp4 over rows of `cols` bf16 values (cols a multiple of 32). */
int orc_quant_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* packed, uint8_t* scales) {
  if (!x || !packed || !scales || rows < 0 || cols <= 0 || cols % 32) return ORC_EARG;
  int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    const uint16_t* xr = x + r * cols;
    for (int64_t b = 0; b < nb; b++) {
      double amax = 0.0;
      for (int i = 0; i < 32; i++) {
        double a = fabs(orc_bf16_to_f64(xr[b * 32 + i]));
        if (a > amax) amax = a;
      }
      int X;
      uint8_t sc;
      if (amax == 0.0) {
        sc = 0;
        X = -127;
      } else {
        int e;
        frexp(amax, &e); /* floor(log2 amax) = e - 1 */
        X = (e - 1) - 2;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
        sc = (uint8_t)(X + 127);
      }
      scales[r * nb + b] = sc;
      for (int i = 0; i < 32; i += 2) {
        double v0 = ldexp(orc_bf16_to_f64(xr[b * 32 + i]), -X);
        double v1 = ldexp(orc_bf16_to_f64(xr[b * 32 + i + 1]), -X);
        uint8_t c0 = nearest_e2m1(v0), c1 = nearest_e2m1(v1);
        packed[r * (cols / 2) + (b * 32 + i) / 2] = (uint8_t)(c0 | (c1 << 4));
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------- decode */

typedef struct {
  int32_t batch;
  int32_t q_dtype;
  const void* q;         /* bf16 [B,rows,576] | e4m3fn [B,rows,576] | packed [B,rows,288] */
  double q_scale;        /* fp8 Q per-tensor scale */
  const uint8_t* q_e8m0; /* mxfp4 Q scales [B*rows, 18] */
  int32_t kv_dtype;
  const void* kv;        /* physical rows: bf16 [R,576] | e4m3fn [R,576] | packed [R,288] */
  int64_t kv_rows;
  double kv_scale;
  const uint8_t* kv_e8m0; /* [R, 18] */
  const int32_t* kv_indptr;
  const int32_t* page_indptr; /* may be NULL */
  const int32_t* page_table;
  int64_t page_table_len;
  int32_t page_size;
  int32_t rows; /* query rows per request (q_seq_len x heads); 0 means 16 */
  const void* v; /* optional value cache, same physical rows: bf16 | e4m3fn [R,576]; NULL = V from kv */
  int32_t v_dtype;
  double v_scale; /* fp8 value cache per-tensor scale */
} orc_problem;

static void deq_row(int dtype, const void* base, int64_t row, double scale, const uint8_t* e8m0, double* out) {
  if (dtype == ORC_BF16) {
    const uint16_t* p = (const uint16_t*)base + row * ORC_DQK;
    for (int i = 0; i < ORC_DQK; i++) out[i] = orc_bf16_to_f64(p[i]);
  } else if (dtype == ORC_FP8) {
    const uint8_t* p = (const uint8_t*)base + row * ORC_DQK;
    for (int i = 0; i < ORC_DQK; i++) out[i] = orc_e4m3fn_to_f64(p[i]) * scale;
  } else {
    const uint8_t* p = (const uint8_t*)base + row * ORC_PACKED;
    const uint8_t* s = e8m0 + row * ORC_NBLK;
    for (int i = 0; i < ORC_DQK; i++) {
      uint8_t byte = p[i / 2];
      uint8_t nib = (i & 1) ? (byte >> 4) : (byte & 15);
      out[i] = orc_e2m1_to_f64(nib) * orc_e8m0_to_f64(s[i / 32]);
    }
  }
}

/* Physical row of token t of request b, or -1 if the page table is out of range. */
static int64_t phys_row(const orc_problem* P, int b, int64_t t) {
  int64_t base = P->page_indptr ? 0 : P->kv_indptr[b];
  int64_t first = P->page_indptr ? P->page_indptr[b] : 0;
  int64_t g = base + t;
  int64_t idx = first + g / P->page_size;
  if (idx < 0 || idx >= P->page_table_len) return -1;
  int64_t pg = P->page_table[idx];
  int64_t row = pg * P->page_size + g % P->page_size;
  if (pg < 0 || row < 0 || row >= P->kv_rows) return -1;
  return row;
}

static int check_problem(const orc_problem* P) {
  if (!P || P->batch < 0 || !P->q || !P->kv || !P->kv_indptr || !P->page_table) return ORC_EARG;
  if (P->page_size <= 0) return ORC_EARG;
  if (P->q_dtype < 0 || P->q_dtype > 2 || P->kv_dtype < 0 || P->kv_dtype > 2) return ORC_EARG;
  if (P->q_dtype == ORC_MXFP4 && !P->q_e8m0) return ORC_EARG;
  if (P->kv_dtype == ORC_MXFP4 && !P->kv_e8m0) return ORC_EARG;
  if (P->v && P->v_dtype != ORC_BF16 && P->v_dtype != ORC_FP8) return ORC_EARG;
  for (int b = 0; b < P->batch; b++)
    if (P->kv_indptr[b + 1] < P->kv_indptr[b]) return ORC_EARG;
  return ORC_OK;
}

/*
 * Unsplit decode of the (b, h) pairs listed in sel (2*nsel ints), or of every
 * pair when sel is NULL; h is a query row of request b (rows per request:
 * P->rows, 16 by default).  Every query row of a request attends to the
 * request's whole cache with no mask: page 695854's chunked torch fallback
 * (_run_chunked_torch_attention) treats q_seq_len x num_heads rows this way.
 * Writes o in fp64 and its bf16 rounding, both laid out [B, rows, 512]; pairs
 * not selected are left untouched.  num_splits == 0 means
 * one softmax over the whole request; num_splits >= 1 runs the split-wise
 * partial/merge form.  nthreads > 0 sets the OpenMP thread count.
 */
int orc_decode(const orc_problem* P, int32_t num_splits, double* out_f64, uint16_t* out_bf16,
               const int32_t* sel, int64_t nsel, int32_t nthreads) {
  int rc = check_problem(P);
  if (rc) return rc;
  if (num_splits < 0) return ORC_EARG;
  const int rows = P->rows > 0 ? P->rows : ORC_HEADS;
  int64_t npairs = sel ? nsel : (int64_t)P->batch * rows;
  int bad = 0;
  if (nthreads <= 0) nthreads = 1;
  /* source of V: the separate value cache when one is given */
  const int sep_v = P->v != NULL;
  const int v_dtype = sep_v ? P->v_dtype : P->kv_dtype;
  const void* v_src = sep_v ? P->v : P->kv;
  const double v_scale = sep_v ? P->v_scale : P->kv_scale;
  const uint8_t* v_e8m0 = sep_v ? NULL : P->kv_e8m0;
  const double inv_sqrt = 1.0 / sqrt((double)ORC_DQK);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
  for (int64_t pi = 0; pi < npairs; pi++) {
    int b = sel ? sel[2 * pi] : (int)(pi / rows);
    int h = sel ? sel[2 * pi + 1] : (int)(pi % rows);
    if (b < 0 || b >= P->batch || h < 0 || h >= rows) {
      bad |= 1;
      continue;
    }
    int64_t L = (int64_t)P->kv_indptr[b + 1] - P->kv_indptr[b];
    double q[ORC_DQK], k[ORC_DQK];
    int64_t qrow = (int64_t)b * rows + h;
    deq_row(P->q_dtype, P->q, qrow, P->q_scale, P->q_e8m0, q);
    double* o = (double*)calloc(ORC_DV, sizeof(double));
    double* s = (double*)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    if (!o || !s) {
      free(o);
      free(s);
      bad |= 4;
      continue;
    }
    /* logits; a token outside the page table or the cache fails this pair */
    int pair_err = 0;
    for (int64_t t = 0; t < L; t++) {
      int64_t row = phys_row(P, b, t);
      if (row < 0) {
        pair_err = 1;
        break;
      }
      deq_row(P->kv_dtype, P->kv, row, P->kv_scale, P->kv_e8m0, k);
      double dot = 0.0;
      for (int i = 0; i < ORC_DQK; i++) dot += q[i] * k[i];
      s[t] = dot * inv_sqrt;
    }
    if (pair_err) {
      bad |= 2;
      free(o);
      free(s);
      continue;
    }
    if (L > 0) {
      int S = num_splits == 0 ? 1 : num_splits;
      int64_t chunk = (L + S - 1) / S;
      double Mx = -INFINITY;
      double* lse = (double*)malloc(sizeof(double) * S);
      double* os = (double*)calloc((size_t)S * ORC_DV, sizeof(double));
      if (!lse || !os) {
        free(lse);
        free(os);
        free(o);
        free(s);
        bad |= 4;
        continue;
      }
      for (int sp = 0; sp < S; sp++) {
        int64_t t0 = (int64_t)sp * chunk, t1 = t0 + chunk < L ? t0 + chunk : L;
        lse[sp] = -INFINITY;
        if (t0 >= t1) continue; /* empty split */
        double m = -INFINITY;
        for (int64_t t = t0; t < t1; t++)
          if (s[t] > m) m = s[t];
        double l = 0.0;
        for (int64_t t = t0; t < t1; t++) {
          double p = exp(s[t] - m);
          l += p;
          deq_row(v_dtype, v_src, phys_row(P, b, t), v_scale, v_e8m0, k);
          for (int i = 0; i < ORC_DV; i++) os[(size_t)sp * ORC_DV + i] += p * k[i];
        }
        for (int i = 0; i < ORC_DV; i++) os[(size_t)sp * ORC_DV + i] /= l;
        lse[sp] = m + log(l);
        if (lse[sp] > Mx) Mx = lse[sp];
      }
      double wsum = 0.0;
      for (int sp = 0; sp < S; sp++) {
        if (lse[sp] == -INFINITY) continue;
        double w = exp(lse[sp] - Mx);
        wsum += w;
        for (int i = 0; i < ORC_DV; i++) o[i] += w * os[(size_t)sp * ORC_DV + i];
      }
      for (int i = 0; i < ORC_DV; i++) o[i] /= wsum;
      free(lse);
      free(os);
    }
    for (int i = 0; i < ORC_DV; i++) {
      size_t idx = ((size_t)b * rows + h) * ORC_DV + i;
      if (out_f64) out_f64[idx] = o[i];
      if (out_bf16) out_bf16[idx] = orc_f64_to_bf16(o[i]);
    }
    free(o);
    free(s);
  }
  if (bad & 1) return ORC_EARG;
  if (bad & 2) return ORC_EINDEX;
  if (bad & 4) return ORC_ENOMEM;
  return ORC_OK;
}
