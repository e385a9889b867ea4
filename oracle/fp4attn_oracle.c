/*
 * fp4attn_oracle.c -- plain, slow CPU oracle for FP4 attention with Direct-P.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or constant
 * with the GPU library and must never be reached from the product path.
 *
 * What it computes follows "Hardware-Aware FP4 FlashAttention-4" (arXiv:2609.04105) as
 * described by the gist.science technical summary of that paper ("Technical Summary:
 * Hardware-Aware FP4 FlashAttention-4": Problem Statement; Methodology 1 "Direct-P for
 * Forward Inference"; Methodology 2 "Quantized Causal Backward") and the paper's arXiv
 * abstract. The pages give no formulas; the element formats are those of the OCP
 * Microscaling (MX) v1.0 specification (E2M1, E4M3, E8M0), which the pages name but do not
 * define. Every point the pages leave open is resolved by one written reading, listed in
 * the design notes of this repository and repeated at the function that applies it.
 *
 * Arithmetic policy: every quantity that decides an integer (a block exponent, a
 * probability code) is computed in IEEE binary32, with the exact sequence of fp32
 * operations stated at each step (this file is built with -ffp-contract=off; the only
 * fused operation is the explicit fmaf). Everything else (dot products, the running O and
 * l, the rescale factors, LSE, gradients) is accumulated in binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_INEXACT 2
#define ORC_ERR_NOMEM 3

#define ORC_FMT_E2M1 1
#define ORC_FMT_E4M3 2

#define ORC_P_DIRECT 0 /* Direct-P: E2M1 probability codes by threshold classification */
#define ORC_P_E4M3 1   /* FP8 probabilities: round-to-nearest-even E4M3 of 2^u */
#define ORC_P_EXACT 2  /* no probability quantizer (identity); exact exponentials */
#define ORC_P_DIRECT_ANCHOR 3 /* Direct-P on the integer-log2 anchor: per-block codes of 2^(S c) */

/* ------------------------------------------------------------------------------------
 * Element formats (OCP MX v1.0; the summary's Problem Statement names the 4-bit E2M1
 * payload, Methodology 1 "Format Selection" the power-of-two block scales, Methodology 2
 * the FP8 operands).
 * ---------------------------------------------------------------------------------- */

/* E2M1: sign bit 3, two exponent bits (bias 1), one mantissa bit; exponent field 0 is
 * subnormal (0 or 0.5). */
double orc_e2m1_decode(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* E4M3 (the "FN" variant of OCP FP8): sign bit 7, four exponent bits (bias 7), three
 * mantissa bits; no infinities; S.1111.111 is NaN; exponent field 0 is subnormal. */
double orc_e4m3_decode(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* E8M0 block scale: 2^(s - 127); 255 is NaN. */
double orc_e8m0_decode(int s) { return (s & 255) == 255 ? NAN : ldexp(1.0, (s & 255) - 127); }

/* Non-negative magnitudes of each format in increasing order, indexed by magnitude code. */
static double E2M1_MAG[8];
static double E4M3_MAG[127];
static int mags_ready = 0;

static void init_mags(void) {
  if (mags_ready) return;
  for (int c = 0; c < 8; c++) E2M1_MAG[c] = orc_e2m1_decode(c);
  for (int c = 0; c < 127; c++) E4M3_MAG[c] = orc_e4m3_decode(c);
  mags_ready = 1;
}

/* Nearest magnitude code of a >= 0 on an increasing grid g[0..n-1] (g[0] = 0): round to
 * nearest, ties to the even code (the even mantissa), saturating at the largest
 * magnitude. Midpoints of adjacent grid values are exact in binary64, so the comparison
 * below decides ties exactly. */
static int nearest_mag_code(double a, const double* g, int n) {
  if (!(a < g[n - 1])) return n - 1;
  int lo = 0, hi = n - 1; /* g[lo] <= a < g[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (g[mid] <= a) lo = mid; else hi = mid;
  }
  double midpoint = 0.5 * (g[lo] + g[hi]);
  if (a < midpoint) return lo;
  if (a > midpoint) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

/* Encoders keep the sign: a negative value that rounds to zero gives negative zero. */
int orc_e2m1_encode(double x) {
  init_mags();
  int s = signbit(x) ? 8 : 0;
  return s | nearest_mag_code(fabs(x), E2M1_MAG, 8);
}

int orc_e4m3_encode(double x) {
  init_mags();
  int s = signbit(x) ? 128 : 0;
  return s | nearest_mag_code(fabs(x), E4M3_MAG, 127);
}

static double fmt_decode(int fmt, int code) { return fmt == ORC_FMT_E2M1 ? orc_e2m1_decode(code) : orc_e4m3_decode(code); }
static int fmt_encode(int fmt, double x) { return fmt == ORC_FMT_E2M1 ? orc_e2m1_encode(x) : orc_e4m3_encode(x); }
/* Largest element exponent of the format: 2 for E2M1 (max 6 = 1.5 * 2^2), 8 for E4M3
 * (max 448 = 1.75 * 2^8). */
static int fmt_emax(int fmt) { return fmt == ORC_FMT_E2M1 ? 2 : 8; }

/* ------------------------------------------------------------------------------------
 * MX block quantization (OCP MX v1.0 scale rule). Reading of the pages: every MX tensor
 * uses blocks of 32 consecutive elements along the stated axis, with the shared E8M0
 * exponent floor(log2(amax)) - emax_elem, clamped to [-127, 127]; elements are rounded to
 * nearest-even on the format's grid with saturation, keeping the sign.
 * ---------------------------------------------------------------------------------- */

/* floor(log2(amax)) - emax, clamped; amax == 0 gives -127. */
int orc_mx_block_exponent(double amax, int fmt) {
  if (!(amax > 0.0)) return -127;
  int k;
  frexp(amax, &k); /* amax = f * 2^k, f in [0.5, 1) */
  int e = (k - 1) - fmt_emax(fmt);
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* x: nvec vectors of length len (len % 32 == 0), blocks along the length.
 * codes: one logical element code per element; scales: one E8M0 byte per block. */
int orc_mx_quantize_f64(const double* x, int64_t nvec, int64_t len, int fmt, uint8_t* codes, uint8_t* scales) {
  if (!x || !codes || !scales || len % 32 != 0 || nvec < 0) return ORC_ERR_ARG;
  if (fmt != ORC_FMT_E2M1 && fmt != ORC_FMT_E4M3) return ORC_ERR_ARG;
  init_mags();
  int64_t nblk = nvec * (len / 32);
#pragma omp parallel for schedule(static)
  for (int64_t bi = 0; bi < nblk; bi++) {
    const double* xb = x + bi * 32;
    double amax = 0.0;
    for (int t = 0; t < 32; t++) amax = fmax(amax, fabs(xb[t]));
    int e = orc_mx_block_exponent(amax, fmt);
    scales[bi] = (uint8_t)(e + 127);
    for (int t = 0; t < 32; t++) codes[bi * 32 + t] = (uint8_t)fmt_encode(fmt, ldexp(xb[t], -e));
  }
  return ORC_OK;
}

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

int orc_bf16_to_f64(const uint16_t* x, int64_t n, double* out) {
  if (!x || !out || n < 0) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = bf16_value(x[i]);
  return ORC_OK;
}

/* Round binary64 to bfloat16, nearest-even, directly (one rounding). */
int orc_f64_to_bf16(const double* x, int64_t n, uint16_t* out) {
  if (!x || !out || n < 0) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    double v = x[i], a = fabs(v);
    double y;
    if (a == 0.0 || isnan(v) || isinf(v)) {
      y = a;
    } else {
      int k;
      frexp(a, &k);                         /* a in [2^(k-1), 2^k) */
      int e = k - 1 < -126 ? -126 : k - 1;  /* bf16 subnormals share the 2^-126 binade spacing */
      double ulp = ldexp(1.0, e - 7);
      y = nearbyint(a / ulp) * ulp;         /* default rounding mode: nearest, ties to even */
      if (y >= ldexp(1.0, 128)) y = INFINITY;
    }
    float f = (float)(signbit(v) ? -y : y);
    if (isnan(v)) f = NAN;
    uint32_t u;
    memcpy(&u, &f, 4);
    out[i] = (uint16_t)(u >> 16);
  }
  return ORC_OK;
}

int orc_mx_quantize_bf16(const uint16_t* x, int64_t nvec, int64_t len, int fmt, uint8_t* codes, uint8_t* scales) {
  if (!x) return ORC_ERR_ARG;
  int64_t n = nvec * len;
  double* tmp = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  if (!tmp) return ORC_ERR_NOMEM;
  orc_bf16_to_f64(x, n, tmp);
  int rc = orc_mx_quantize_f64(tmp, nvec, len, fmt, codes, scales);
  free(tmp);
  return rc;
}

int orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t nvec, int64_t len, int fmt, double* out) {
  if (!codes || !scales || !out || len % 32 != 0 || nvec < 0) return ORC_ERR_ARG;
  if (fmt != ORC_FMT_E2M1 && fmt != ORC_FMT_E4M3) return ORC_ERR_ARG;
  int64_t n = nvec * len;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = fmt_decode(fmt, codes[i]) * orc_e8m0_decode(scales[i / 32]);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------
 * NVFP4-style block quantization (summary, Methodology 1 "Format Selection": NVFP4 for Q and
 * K, i.e. finer block scales than MXFP4). Reading: blocks of 16 consecutive elements along the
 * stated axis, E2M1 elements, one E4M3 scale per block, and a per-tensor scale chosen by the
 * caller as a power of two 2^g:
 *   s = RNE_E4M3(amax / 6 / 2^g), saturating at 448 (zero when amax / 6 / 2^g rounds to zero);
 *   element code = RNE_E2M1(x / (s 2^g)), saturating, sign kept; magnitude code 0 (sign kept)
 *   for every element when s = 0;
 *   represented value x_hat = E2M1(code) s 2^g.
 * Both quotients are formed in binary64. They are correctly rounded divisions of a bf16 value by
 * a value with at most 4 significant bits, so a quotient lands on a rounding midpoint only when
 * the exact quotient is that midpoint: the nearest-even decisions are those of the exact values.
 * ---------------------------------------------------------------------------------- */
int orc_nvfp4_quantize(const double* x, int64_t nvec, int64_t len, int g, uint8_t* codes, uint8_t* scales,
                       double* xhat) {
  if (!x || !codes || !scales || !xhat || len % 16 != 0 || nvec < 0 || g < -126 || g > 126) return ORC_ERR_ARG;
  init_mags();
  const int64_t nblk = nvec * (len / 16);
  const double tg = ldexp(1.0, g);
#pragma omp parallel for schedule(static)
  for (int64_t bi = 0; bi < nblk; bi++) {
    const double* xb = x + bi * 16;
    double amax = 0.0;
    for (int t = 0; t < 16; t++) amax = fmax(amax, fabs(xb[t]));
    const int sc = orc_e4m3_encode(amax / 6.0 / tg); /* non-negative: a code 0..126 */
    const double s = orc_e4m3_decode(sc);
    scales[bi] = (uint8_t)sc;
    for (int t = 0; t < 16; t++) {
      int c = 0;
      if (s > 0.0) c = orc_e2m1_encode(xb[t] / (s * tg));
      else if (signbit(xb[t])) c = 8; /* a zero block keeps each element's sign, like the MX rule */
      codes[bi * 16 + t] = (uint8_t)c;
      xhat[bi * 16 + t] = orc_e2m1_decode(c) * s * tg;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------
 * Direct-P probability codes (summary, Methodology 1, "Direct Mapping"; arXiv abstract:
 * scores are mapped directly to FP4 probabilities). Reading: probability construction is
 * a classification of the normalized log-score u (affine in the raw score) into the eight
 * non-negative E2M1 magnitudes. The class boundaries are the exact step points of
 * round-to-nearest-even E2M1 applied to the exact value 2^u, as binary32 values:
 * code(u) = number of thresholds T_k with u >= T_k.
 * ---------------------------------------------------------------------------------- */
static const uint32_t DIRECTP_T_BITS[7] = {
    0xBFFFFFFFu, /* 2^u > 0.25: the tie at exactly 0.25 (u = -2) rounds to code 0 */
    0xBED47FCBu, /* 2^u >= 0.75 */
    0x3EA4D3C3u, /* 2^u > 1.25 */
    0x3F4EAED0u, /* 2^u >= 1.75 */
    0x3FA934F1u, /* 2^u > 2.5 */
    0x3FE75768u, /* 2^u >= 3.5 */
    0x40149A79u, /* 2^u > 5 */
};

static float f32_from_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}

int orc_directp_code(float u) {
  int code = 0;
  for (int k = 0; k < 7; k++)
    if (u >= f32_from_bits(DIRECTP_T_BITS[k])) code++;
  return code;
}

void orc_directp_thresholds(float* out7) {
  for (int k = 0; k < 7; k++) out7[k] = f32_from_bits(DIRECTP_T_BITS[k]);
}

/* FP8 probabilities on the causal path: E4M3 code of the exact value 2^u, round to
 * nearest even, saturating at 448. 2^u is evaluated in long double; the nearest E4M3
 * midpoint is never within its rounding error for binary32 u. */
int orc_e4m3_code_of_exp2(float u) {
  init_mags();
  long double p = exp2l((long double)u);
  if (!(p < (long double)E4M3_MAG[126])) return 126;
  int lo = 0, hi = 126;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if ((long double)E4M3_MAG[mid] <= p) lo = mid; else hi = mid;
  }
  long double midpoint = 0.5L * ((long double)E4M3_MAG[lo] + (long double)E4M3_MAG[hi]);
  if (p < midpoint) return lo;
  if (p > midpoint) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

/* c = scale * log2(e) in binary32, scale = 1/sqrt(D), rounded once from binary64. */
float orc_log2e_scale(int64_t D) { return (float)(1.4426950408889634 / sqrt((double)D)); }

/* Probabilities of one 32-key block (or the visible part of one) relative to the running
 * max m, in a quantized mode (Direct-P E2M1 or FP8 E4M3):
 *   e_b = max(floor(fp32(fp32(S_bmax - m) * c)) - emax, -127)
 *   off = fp32(-fp32(m * c) - e_b);  u_j = fmaf(S_j, c, off)
 *   P_j = magnitude(code(u_j)) * 2^e_b
 * s: n <= 32 binary32 scores (all visible). Writes P_j to p and returns e_b. */
int orc_block_probs(const float* s, int n, float m, float cf, int pmode, double* p) {
  init_mags();
  const int emax = (pmode == ORC_P_E4M3) ? 8 : 2;
  float sbmax = -INFINITY;
  for (int j = 0; j < n; j++) sbmax = fmaxf(sbmax, s[j]);
  const float d1 = sbmax - m;
  const float d2 = d1 * cf;
  int eb = (int)floorf(d2) - emax;
  if (eb < -127) eb = -127;
  const float mc = m * cf;
  const float off = -mc - (float)eb;
  const double sc = ldexp(1.0, eb);
  for (int j = 0; j < n; j++) {
    const float u = fmaf(s[j], cf, off);
    if (pmode == ORC_P_DIRECT) p[j] = E2M1_MAG[orc_directp_code(u)] * sc;
    else p[j] = E4M3_MAG[orc_e4m3_code_of_exp2(u)] * sc;
  }
  return eb;
}
/* Direct-P on the integer-log2 anchor (summary, Methodology 1, "Direct Mapping" and "Range
 * Guarding"). Reading: each 32-key block's scores are normalized by the block's own leading
 * binade, t_b = floor(fp32(S_bmax * c)), instead of by the row's running max:
 *   u_j = fmaf(S_j, c, 2 - t_b)               (one fused multiply-add; 2 - t_b is an integer)
 *   P_j = E2M1[code(u_j)] * 2^(t_b - 2)
 * which is the MX quantization (block exponent floor(log2 amax) - 2) of the unnormalized
 * exponentials 2^(S_j c) = e^(S_j / sqrt(D)). The codes depend on no row quantity, so a kernel may
 * keep its accumulators relative to any integer anchor (an exact power-of-two scale) and move it
 * only to stay in range; the block exponent is absolute and unclamped here (binary64 holds it).
 * s: n <= 32 binary32 scores (all visible). Writes P_j to p and returns t_b - 2. */
int orc_block_probs_anchored(const float* s, int n, float cf, double* p) {
  init_mags();
  float sbmax = -INFINITY;
  for (int j = 0; j < n; j++) sbmax = fmaxf(sbmax, s[j]);
  const float x = sbmax * cf;
  const int t = (int)floorf(x);
  const float off = (float)(2 - t);
  const double sc = ldexp(1.0, t - 2);
  for (int j = 0; j < n; j++) p[j] = E2M1_MAG[orc_directp_code(fmaf(s[j], cf, off))] * sc;
  return t - 2;
}

/* ------------------------------------------------------------------------------------
 * Forward attention with the online (running-max) softmax of FlashAttention (the base
 * algorithm the paper modifies; summary, Problem Statement: score reduction,
 * exponentials, probability construction, scaling between the two matrix products).
 *
 * Inputs are already-dequantized operands Q [B,H,N,D], K [B,Hkv,N,D], V [B,Hkv,N,D]
 * (binary64 holding the represented values). Query head h reads KV head h / (H/Hkv).
 * Keys are processed in blocks of KB (a multiple of 32) in increasing order; the running
 * max m is updated once per key block and the probabilities of that block are formed
 * relative to the updated max. Inside a key block, P is formed per 32-key block b:
 *
 *   e_b  = max(floor(fp32(fp32(S_bmax - m) * c)) - emax, -127)   (emax 2 for E2M1, 8 for E4M3)
 *   off  = fp32(-fp32(m * c) - e_b)
 *   u_ij = fmaf(S_ij, c, off)
 *   Direct-P: P_ij = E2M1[code(u_ij)] * 2^e_b
 *   FP8:      P_ij = E4M3[RNE_sat(2^u_ij)] * 2^e_b
 *
 * which is the MX quantization (same scale rule as the operand quantizer) of the
 * probabilities exp2((S - m) c). Consistent normalization (summary, Methodology 1): the
 * normalizer l accumulates exactly these represented values, the same ones the P.V
 * product consumes. When the max grows from m_old to m_new, O and l are multiplied by
 * exp2((m_old - m_new) * c). Output: O = O_acc / l, LSE = m / sqrt(D) + ln(l).
 *
 * Causal (summary, Methodology 2): key j is visible to query i iff j <= i; key blocks and
 * 32-key blocks with no visible key are skipped (they would contribute nothing).
 *
 * pmode ORC_P_DIRECT_ANCHOR forms every 32-key block's probabilities with
 * orc_block_probs_anchored (no running max, no rescale; KB plays no part), accumulates
 * l = sum_j P_j and O = sum_j P_j V_j / l in binary64, and reports LSE = ln(l): P_j there
 * approximates e^(S_j / sqrt(D)) itself. The reported "m" is the row's largest score.
 *
 * In the quantized modes every score must be exactly representable in binary32 (the
 * block-scaled products of MX operands are exact); check_exact makes that an error
 * instead of an assumption.
 *
 * rows: optional list of flattened [B,H,N] row indices; NULL means all rows in order.
 * Outputs per listed row: O [nrows, D], lse [nrows], and optionally l [nrows] and the
 * final running max [nrows].
 * ---------------------------------------------------------------------------------- */
int orc_attn_fwd(const double* Q, const double* K, const double* V, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                 int64_t D, int64_t KB, int causal, int pmode, int check_exact, const int64_t* rows, int64_t nrows,
                 double* O, double* lse, double* l_out, double* m_out) {
  if (!Q || !K || !V || !O || !lse) return ORC_ERR_ARG;
  if (B < 1 || H < 1 || Hkv < 1 || N < 1 || D < 1 || H % Hkv != 0) return ORC_ERR_ARG;
  if (KB < 32 || KB % 32 != 0) return ORC_ERR_ARG;
  if (pmode != ORC_P_DIRECT && pmode != ORC_P_E4M3 && pmode != ORC_P_EXACT && pmode != ORC_P_DIRECT_ANCHOR)
    return ORC_ERR_ARG;
  if (!rows && nrows != B * H * N) return ORC_ERR_ARG;
  init_mags();
  const int64_t group = H / Hkv;
  const float cf = orc_log2e_scale(D);
  const double scale = 1.0 / sqrt((double)D);
  const double c_exact = 1.4426950408889634 * scale;
  int err = ORC_OK;

#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t t = 0; t < nrows; t++) {
    if (err != ORC_OK) continue;
    const int64_t r = rows ? rows[t] : t;
    if (r < 0 || r >= B * H * N) {
#pragma omp atomic write
      err = ORC_ERR_ARG;
      continue;
    }
    const int64_t b = r / (H * N), h = (r / N) % H, i = r % N;
    const int64_t g = h / group;
    const double* q = Q + r * D;
    const double* Kh = K + (b * Hkv + g) * N * D;
    const double* Vh = V + (b * Hkv + g) * N * D;
    const int64_t jend = causal ? i + 1 : N;
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    double* acc = (double*)calloc((size_t)D, sizeof(double));
    if (!s || !acc) {
      free(s);
      free(acc);
#pragma omp atomic write
      err = ORC_ERR_NOMEM;
      continue;
    }
    /* Scores S_ij = Q_i . K_j (exact in binary64 for MX operands). */
    int inexact = 0;
    for (int64_t j = 0; j < jend; j++) {
      double d = 0.0;
      for (int64_t k = 0; k < D; k++) d += q[k] * Kh[j * D + k];
      s[j] = d;
      if (check_exact && pmode != ORC_P_EXACT && (double)(float)d != d) inexact = 1;
    }
    if (inexact) {
      free(s);
      free(acc);
#pragma omp atomic write
      err = ORC_ERR_INEXACT;
      continue;
    }
    double m = -INFINITY, l = 0.0;
    if (pmode == ORC_P_DIRECT_ANCHOR) {
      for (int64_t sb0 = 0; sb0 < jend; sb0 += 32) {
        const int n = (int)(((sb0 + 32 < jend) ? sb0 + 32 : jend) - sb0);
        float sf[32];
        double p[32];
        for (int j = 0; j < n; j++) {
          sf[j] = (float)s[sb0 + j];
          m = fmax(m, s[sb0 + j]);
        }
        orc_block_probs_anchored(sf, n, cf, p);
        for (int j = 0; j < n; j++) {
          if (p[j] == 0.0) continue;
          l += p[j];
          for (int64_t k = 0; k < D; k++) acc[k] += p[j] * Vh[(sb0 + j) * D + k];
        }
      }
      for (int64_t k = 0; k < D; k++) O[t * D + k] = acc[k] / l;
      lse[t] = log(l);
      if (l_out) l_out[t] = l;
      if (m_out) m_out[t] = m;
      free(s);
      free(acc);
      continue;
    }
    for (int64_t kb0 = 0; kb0 < jend; kb0 += KB) {
      const int64_t kb1 = (kb0 + KB < jend) ? kb0 + KB : jend;
      double mblk = -INFINITY;
      for (int64_t j = kb0; j < kb1; j++) mblk = fmax(mblk, s[j]);
      const double mnew = fmax(m, mblk);
      if (m != -INFINITY && mnew != m) {
        double alpha = (pmode == ORC_P_EXACT) ? exp2((m - mnew) * c_exact) : exp2((m - mnew) * (double)cf);
        for (int64_t k = 0; k < D; k++) acc[k] *= alpha;
        l *= alpha;
      }
      m = mnew;
      if (pmode == ORC_P_EXACT) {
        for (int64_t j = kb0; j < kb1; j++) {
          double p = exp2((s[j] - m) * c_exact);
          l += p;
          for (int64_t k = 0; k < D; k++) acc[k] += p * Vh[j * D + k];
        }
        continue;
      }
      const float mf = (float)m;
      for (int64_t sb0 = kb0; sb0 < kb1; sb0 += 32) {
        const int n = (int)(((sb0 + 32 < kb1) ? sb0 + 32 : kb1) - sb0);
        float sf[32];
        double p[32];
        for (int j = 0; j < n; j++) sf[j] = (float)s[sb0 + j];
        orc_block_probs(sf, n, mf, cf, pmode, p);
        for (int j = 0; j < n; j++) {
          if (p[j] == 0.0) continue;
          l += p[j];
          for (int64_t k = 0; k < D; k++) acc[k] += p[j] * Vh[(sb0 + j) * D + k];
        }
      }
    }
    for (int64_t k = 0; k < D; k++) O[t * D + k] = acc[k] / l;
    lse[t] = m * scale + log(l);
    if (l_out) l_out[t] = l;
    if (m_out) m_out[t] = m;
    free(s);
    free(acc);
  }
  return err;
}

/* ------------------------------------------------------------------------------------
 * Backward of the causal path (summary, Methodology 2 "Quantized Causal Backward";
 * arXiv abstract). Probabilities are rebuilt from the saved quantized Q/K and the saved
 * LSE, with no separate score path:
 *
 *   S_ij  = Qs_i . Ks_j                        (saved MXFP4 operands, exact)
 *   P_ij  = fp32(2^(fmaf(S_ij, c, -fp32(LSE_i * log2e))))     for visible j, else 0
 *   dP_ij = dOd_i . Vd_j                       (FP8 views along D)
 *   Delta_i = sum_d dO_id * O_id               (forward's output O)
 *   dS_ij = P_ij (dP_ij - Delta_i)
 *   dV_j  = sum_i MX8_Q(P)_ij dOq_i            (P and dO blocked along queries)
 *   dQ_i  = scale * sum_j MX8_K(dS)_ij Kk_j    (dS and K blocked along keys)
 *   dK_j  = scale * sum_i MX8_Q(dS)_ij Qq_i    (dS and Q blocked along queries)
 *
 * Reading: "FP8 gradient operands" means MXFP8 (E4M3 elements, E8M0 scale per 32 along
 * each product's contraction axis) for every operand of the four gradient products; the
 * operand views (dOd, Vd, dOq, Kk, Qq) are passed in already dequantized. MX8_Q / MX8_K
 * quantize P and dS inside the backward. With quant == 0 every quantizer is the identity
 * and P = exp(S * scale - LSE) in binary64 (the textbook gradient).
 *
 * Grouped-query attention: dK and dV of KV head g sum over the query heads h with
 * h / (H/Hkv) == g. qrows lists flattened [B,H,N] rows of dQ; kcols lists flattened
 * [B,Hkv,N] key rows of dK/dV (NULL = all, in order).
 * ---------------------------------------------------------------------------------- */
static void mx8_roundtrip_vec(double* x, int64_t n) {
  /* n % 32 == 0; in place: quantize blocks of 32 to MXFP8 and dequantize */
  for (int64_t b0 = 0; b0 < n; b0 += 32) {
    double amax = 0.0;
    for (int t = 0; t < 32; t++) amax = fmax(amax, fabs(x[b0 + t]));
    int e = orc_mx_block_exponent(amax, ORC_FMT_E4M3);
    for (int t = 0; t < 32; t++) {
      int code = orc_e4m3_encode(ldexp(x[b0 + t], -e));
      x[b0 + t] = ldexp(orc_e4m3_decode(code), e);
    }
  }
}

static double bwd_prob(double s, double lse_i, int quant, float cf, double scale) {
  if (!quant) return exp(s * scale - lse_i);
  const float nl = -((float)lse_i * 1.44269504f);
  const float u = fmaf((float)s, cf, nl);
  return (double)(float)exp2((double)u);
}

/* The quantized backward's probability for one score (test hook): s and lse as binary32,
 * D selects c. */
double orc_bwd_prob(float s, float lse, int64_t D) {
  return bwd_prob((double)s, (double)lse, 1, orc_log2e_scale(D), 1.0 / sqrt((double)D));
}

int orc_attn_bwd(const double* Qs, const double* Ks, const double* dOd, const double* Vd, const double* dOq,
                 const double* Kk, const double* Qq, const double* O, const double* dO, const double* lse, int64_t B,
                 int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal, int quant, const int64_t* qrows,
                 int64_t nq, double* dQ, const int64_t* kcols, int64_t nk, double* dK, double* dV) {
  if (!Qs || !Ks || !dOd || !Vd || !dOq || !Kk || !Qq || !O || !dO || !lse) return ORC_ERR_ARG;
  if (B < 1 || H < 1 || Hkv < 1 || N < 1 || D < 1 || H % Hkv != 0 || N % 32 != 0) return ORC_ERR_ARG;
  if ((nq > 0 && !dQ) || (nk > 0 && (!dK || !dV))) return ORC_ERR_ARG;
  if (!qrows && nq != 0 && nq != B * H * N) return ORC_ERR_ARG;
  if (!kcols && nk != 0 && nk != B * Hkv * N) return ORC_ERR_ARG;
  init_mags();
  const int64_t group = H / Hkv;
  const float cf = orc_log2e_scale(D);
  const double scale = 1.0 / sqrt((double)D);
  int err = ORC_OK;

  /* dQ rows */
#pragma omp parallel for schedule(dynamic, 2)
  for (int64_t t = 0; t < nq; t++) {
    if (err != ORC_OK) continue;
    const int64_t r = qrows ? qrows[t] : t;
    if (r < 0 || r >= B * H * N) {
#pragma omp atomic write
      err = ORC_ERR_ARG;
      continue;
    }
    const int64_t b = r / (H * N), h = (r / N) % H, i = r % N, g = h / group;
    const int64_t kvbase = (b * Hkv + g) * N;
    double* ds = (double*)calloc((size_t)N, sizeof(double));
    if (!ds) {
#pragma omp atomic write
      err = ORC_ERR_NOMEM;
      continue;
    }
    double delta = 0.0;
    for (int64_t k = 0; k < D; k++) delta += dO[r * D + k] * O[r * D + k];
    const int64_t jend = causal ? i + 1 : N;
    for (int64_t j = 0; j < jend; j++) {
      double sij = 0.0, dp = 0.0;
      for (int64_t k = 0; k < D; k++) {
        sij += Qs[r * D + k] * Ks[(kvbase + j) * D + k];
        dp += dOd[r * D + k] * Vd[(kvbase + j) * D + k];
      }
      const double p = bwd_prob(sij, lse[r], quant, cf, scale);
      ds[j] = p * (dp - delta);
    }
    if (quant) mx8_roundtrip_vec(ds, N);
    for (int64_t k = 0; k < D; k++) {
      double a = 0.0;
      for (int64_t j = 0; j < jend; j++) a += ds[j] * Kk[(kvbase + j) * D + k];
      dQ[t * D + k] = scale * a;
    }
    free(ds);
  }
  if (err != ORC_OK) return err;

  /* dK, dV key rows */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < nk; t++) {
    if (err != ORC_OK) continue;
    const int64_t c = kcols ? kcols[t] : t;
    if (c < 0 || c >= B * Hkv * N) {
#pragma omp atomic write
      err = ORC_ERR_ARG;
      continue;
    }
    const int64_t b = c / (Hkv * N), g = (c / N) % Hkv, j = c % N;
    double* pcol = (double*)calloc((size_t)N, sizeof(double));
    double* dscol = (double*)calloc((size_t)N, sizeof(double));
    double* dk = (double*)calloc((size_t)D, sizeof(double));
    double* dv = (double*)calloc((size_t)D, sizeof(double));
    if (!pcol || !dscol || !dk || !dv) {
      free(pcol); free(dscol); free(dk); free(dv);
#pragma omp atomic write
      err = ORC_ERR_NOMEM;
      continue;
    }
    const int64_t istart = causal ? j : 0;
    for (int64_t h = g * group; h < (g + 1) * group; h++) {
      const int64_t qbase = (b * H + h) * N;
      memset(pcol, 0, sizeof(double) * (size_t)N);
      memset(dscol, 0, sizeof(double) * (size_t)N);
      for (int64_t i = istart; i < N; i++) {
        const int64_t r = qbase + i;
        double sij = 0.0, dp = 0.0, delta = 0.0;
        for (int64_t k = 0; k < D; k++) {
          sij += Qs[r * D + k] * Ks[c * D + k];
          dp += dOd[r * D + k] * Vd[c * D + k];
          delta += dO[r * D + k] * O[r * D + k];
        }
        const double p = bwd_prob(sij, lse[r], quant, cf, scale);
        pcol[i] = p;
        dscol[i] = p * (dp - delta);
      }
      if (quant) {
        mx8_roundtrip_vec(pcol, N);
        mx8_roundtrip_vec(dscol, N);
      }
      for (int64_t i = istart; i < N; i++) {
        const int64_t r = qbase + i;
        for (int64_t k = 0; k < D; k++) {
          dv[k] += pcol[i] * dOq[r * D + k];
          dk[k] += dscol[i] * Qq[r * D + k];
        }
      }
    }
    for (int64_t k = 0; k < D; k++) {
      dV[t * D + k] = dv[k];
      dK[t * D + k] = scale * dk[k];
    }
    free(pcol); free(dscol); free(dk); free(dv);
  }
  return err;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
