/*
 * detint oracle: a plain, slow CPU implementation of the integer-only
 * transformer forward pass. TEST INFRASTRUCTURE ONLY: the HIP library never
 * links, loads or calls this file, and this file includes nothing of it.
 *
 * Sources (page title, section):
 *   [README]   "DetLLM - Fully Deterministic LLM Inference": intro, "Why LLM
 *              inference is nondeterministic - and how integers fix it",
 *              "Layout", "Demo".
 *   [BLOG]     DetLLM blog post on removing LLM-inference nondeterminism with
 *              pure integer arithmetic (Chinese-language page): sections
 *              "DetLLM", "perplexity and speed", footnotes 8 and 9.
 *   [BITEXACT] "BitExact LLM" blog: "Fix the arithmetic, not just the random
 *              seed", "Three execution paths", "What the checks actually
 *              compare".
 *
 * Every step is integer arithmetic on int64 (__int128 only where a 16-bit
 * weight product times two 15-bit mantissas can pass 2^63). The pages leave
 * the integer formulas open; the readings taken here are the ones written in
 * each function's comment. Bounds are asserted after every op: a violated
 * bound sets an error (orc_error) and the op returns nonzero.
 *
 * Right shifts of negative values are arithmetic (floor), as GCC defines.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef __int128 i128;

/* ------------------------------------------------------------------ */
/* error reporting                                                     */

static volatile int g_err = 0;
static char g_msg[512];

static void orc_fail(const char *what, int line) {
#pragma omp critical(orc_err)
  {
    if (!g_err) {
      g_err = 1;
      snprintf(g_msg, sizeof g_msg, "bound violated: %s (oracle line %d)", what, line);
    }
  }
}
#define CHECK(c, what) do { if (!(c)) orc_fail(what, __LINE__); } while (0)

int orc_error(void) { return g_err; }
const char *orc_error_msg(void) { return g_err ? g_msg : ""; }
void orc_clear_error(void) { g_err = 0; g_msg[0] = 0; }

/* ------------------------------------------------------------------ */
/* primitives                                                          */

/* Round-half-up right shift R(x, s) = floor(x / 2^s + 1/2) for s >= 1,
 * x for s = 0, x * 2^-s for s < 0. This is the single frozen rounding rule
 * every dyadic rescale uses ([BLOG] "DetLLM": a rescale is one integer
 * multiply plus one shift under one fixed rounding rule; [BITEXACT] "Fix the
 * arithmetic": explicit integer rounding rules). */
int64_t orc_rshift_round(int64_t x, int s) {
  if (s > 0) {
    CHECK(s <= 62, "shift > 62");
    if (s > 62) return 0;
    int64_t half = (int64_t)1 << (s - 1);
    CHECK(x <= INT64_MAX - half, "R add overflow");
    return (x + half) >> s;
  }
  if (s == 0) return x;
  CHECK(-s <= 62, "left shift > 62");
  if (-s > 62) return 0;
  int64_t lim = (int64_t)1 << (62 + s);
  CHECK(x < lim && x > -lim, "R left-shift overflow");
  return x * ((int64_t)1 << (-s));
}

static int64_t R(int64_t x, int s) { return orc_rshift_round(x, s); }

/* same rule on a 128-bit product, result must fit int64 */
static int64_t R128(i128 x, int s) {
  if (s > 0) {
    CHECK(s <= 120, "shift > 120");
    i128 r = (x + ((i128)1 << (s - 1))) >> s;
    CHECK(r <= INT64_MAX && r >= INT64_MIN, "R128 result exceeds int64");
    return (int64_t)r;
  }
  CHECK(s > -62, "R128 left shift");
  i128 r = x * ((i128)1 << (-s));
  CHECK(r <= INT64_MAX && r >= INT64_MIN, "R128 result exceeds int64");
  return (int64_t)r;
}

/* RD(a, b) = floor((2a + b) / (2b)): a / b rounded half up, a >= 0, b > 0. */
int64_t orc_div_round(int64_t a, int64_t b) {
  CHECK(a >= 0 && b > 0, "RD domain");
  CHECK(a < ((int64_t)1 << 61) && b < ((int64_t)1 << 61), "RD range");
  if (b <= 0) return 0;
  return (2 * a + b) / (2 * b);
}

/* floor(sqrt(n)) by bisection on [0, 2^32). */
uint64_t orc_isqrt(uint64_t n) {
  uint64_t lo = 0, hi = (uint64_t)1 << 32; /* invariant: lo^2 <= n < hi^2 */
  while (hi - lo > 1) {
    uint64_t mid = lo + (hi - lo) / 2;
    if ((unsigned __int128)mid * mid <= n) lo = mid; else hi = mid;
  }
  return lo;
}

/* number of bits needed to write x >= 0 (0 for x = 0) */
int orc_bitlen(uint64_t x) {
  int b = 0;
  while (x) { b++; x >>= 1; }
  return b;
}

static int8_t clamp8(int64_t x) { return (int8_t)(x > 127 ? 127 : (x < -127 ? -127 : x)); }

/* Per-token dynamic quantisation DQ ([BLOG] "DetLLM": each token's
 * activations are quantised from that token's own values). Reading: a
 * power-of-two scale chosen from the row's absolute maximum A,
 * e = max(0, bl(A) - 7), q_i = clamp8(R(y_i, e)), so y_i ~ q_i * 2^e. */
void orc_dq(const int64_t *y, int64_t n, int8_t *q, int32_t *e) {
  uint64_t A = 0;
  for (int64_t i = 0; i < n; i++) {
    uint64_t a = y[i] < 0 ? (uint64_t)(-(y[i] + 1)) + 1 : (uint64_t)y[i];
    if (a > A) A = a;
  }
  int b = orc_bitlen(A);
  int ee = b > 7 ? b - 7 : 0;
  for (int64_t i = 0; i < n; i++) q[i] = clamp8(R(y[i], ee));
  *e = ee;
}

/* Integer inverse RMS for DI-RMSNorm ([README] "Layout": ops/ holds an integer
 * RMSNorm; [BLOG] "DetLLM": RMSNorm is shift-based integer arithmetic on
 * dyadic values). For S = sum of squares > 0 over n entries, returns (m, sh)
 * with 1/sqrt(S/n) ~ m * 2^-sh, m in [2^14, 2^15):
 *   c = max(0, floor((62 - bl(S)) / 2)), u = floor(S * 4^c / n),
 *   r = isqrt(u), T = bl(r) + 14, m = RD(2^T, r) (if m = 2^15 then
 *   m = 2^14, T = T - 1), sh = T - c.  No epsilon term. */
void orc_irms(int64_t S, int64_t n, int32_t *m, int32_t *sh) {
  CHECK(S > 0 && n > 0, "irms domain");
  if (S <= 0 || n <= 0) { *m = 1 << 14; *sh = 14; return; }
  int b = orc_bitlen((uint64_t)S);
  CHECK(b <= 62, "irms S >= 2^62");
  int c = b < 62 ? (62 - b) / 2 : 0;
  uint64_t u = ((uint64_t)S << (2 * c)) / (uint64_t)n;
  uint64_t r = orc_isqrt(u);
  int T = orc_bitlen(r) + 14;
  int64_t mm = orc_div_round((int64_t)1 << T, (int64_t)r);
  if (mm == (1 << 15)) { mm = 1 << 14; T -= 1; }
  *m = (int32_t)mm;
  *sh = T - c;
}

/* DI-Exp: shift-based integer exponential ([README] "Layout": ops/ DI-Exp;
 * [BLOG] "DetLLM": exp is shift-based integer arithmetic). Input u <= 0 is a
 * base-2 exponent in Q15 (value 2^(u/2^15)). With v = -u, n = v >> 15 and
 * r = v mod 2^15, the fractional power is the linear shift form
 * 2^(-r/2^15) ~ 1 - r/2^16 (the I-ViT Shiftmax construction): f = 2^15 - R(r, 1),
 * E = R(f, n), E in [0, 2^15], E ~ 2^15 * 2^(u/2^15). */
int32_t orc_diexp(int64_t u) {
  CHECK(u <= 0, "diexp input > 0");
  int64_t v = -u;
  int64_t n = v >> 15;
  int64_t r = v & 32767;
  int64_t f = 32768 - R(r, 1);
  if (n > 30) return 0;
  return (int32_t)R(f, (int)n);
}

static void dyadic_of(double x, int32_t *M, int32_t *K) {
  int ex;
  double f = frexp(x, &ex);
  int64_t m = (int64_t)floor(f * 32768.0 + 0.5);
  int k = 15 - ex;
  if (m == 32768) { m = 16384; k -= 1; }
  *M = (int32_t)m;
  *K = k;
}

#define ORC_LOG2E 1.4426950408889634

/* Softmax exponent multiplier: maps an integer score difference (q8 . k8 with
 * q at exponent 0) to base-2 Q15 units: log2(e) / sqrt(d) times the K-cache
 * dequant scale 2^kq_k / kq_m times 2^-2f_n, as a dyadic (M, K). */
void orc_softmax_mult(int32_t kq_m, int32_t kq_k, int64_t d, int32_t f_n,
                      int32_t *M, int32_t *K) {
  double mult = ldexp(ORC_LOG2E, 15 + kq_k - 2 * f_n) / ((double)kq_m * sqrt((double)d));
  dyadic_of(mult, M, K);
}

/* SiLU exponent multiplier: gate in f_a fixed point -> base-2 Q15 units. */
void orc_swiglu_mult(int32_t f_a, int32_t *M, int32_t *K) {
  dyadic_of(ldexp(ORC_LOG2E, 15 - f_a), M, K);
}

/* V-cache dequant scale, the dyadic inverse of the quant scale vq_m/2^vq_k. */
void orc_v_dequant(int32_t vq_m, int32_t vq_k, int32_t *m, int32_t *k) {
  int64_t mm = orc_div_round((int64_t)1 << 29, vq_m);
  int kk = 29 - vq_k;
  if (mm == 32768) { mm = 16384; kk -= 1; }
  *m = (int32_t)mm;
  *k = kk;
}

/* RoPE tables ([BLOG] "DetLLM": rotary embedding uses precomputed int16 sin
 * and cos tables). Q1.14: C[p][i] = floor(2^14 cos(p * theta_i) + 1/2),
 * S likewise with sin, theta_i = base^(-2i/d), computed once in float64
 * (table construction is offline; the forward pass only reads the table). */
int orc_rope_tables(int16_t *cos_t, int16_t *sin_t, int64_t P, int64_t d, int64_t base) {
  int64_t half = d / 2;
  for (int64_t p = 0; p < P; p++)
    for (int64_t i = 0; i < half; i++) {
      double theta = pow((double)base, -(double)(2 * i) / (double)d);
      double ang = (double)p * theta;
      cos_t[p * half + i] = (int16_t)floor(16384.0 * cos(ang) + 0.5);
      sin_t[p * half + i] = (int16_t)floor(16384.0 * sin(ang) + 0.5);
    }
  return 0;
}

/* ------------------------------------------------------------------ */
/* GEMM                                                                */

/* acc[i][j] = sum_k A[i][k] * W[j][k], exactly ([README] intro / [BLOG]
 * "DetLLM": the one hardware-dispatched primitive is int8 x int8 -> int32
 * matmul). When W16 is given the weights are 16-bit fixed point and acc is
 * the exact int64 sum ([BITEXACT] "Fix the arithmetic": limb products are
 * combined into wide accumulators; the exact result is the direct product). */
int orc_gemm(const int8_t *A, const int8_t *W, const int16_t *W16,
             int64_t M, int64_t N, int64_t K, int64_t *acc) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < N; j++) {
    for (int64_t i = 0; i < M; i++) {
      int64_t s = 0;
      const int8_t *a = A + i * K;
      if (W16) {
        const int16_t *w = W16 + j * K;
        for (int64_t k = 0; k < K; k++) s += (int64_t)a[k] * (int64_t)w[k];
      } else {
        const int8_t *w = W + j * K;
        for (int64_t k = 0; k < K; k++) s += (int64_t)a[k] * (int64_t)w[k];
      }
      acc[i * N + j] = s;
    }
  }
  return g_err;
}

enum { ORC_RAW = 0, ORC_REQ_I8 = 1, ORC_FIX = 2, ORC_RES_ADD = 3 };

/* Dyadic epilogue of a GEMM ([README] "Layout": dyadic.py (data, m, k)
 * requant; [BLOG] "DetLLM": a dyadic rescale is one multiply and one shift):
 *   RAW     out_i32 = acc (must fit int32)
 *   REQ_I8  out_i8  = clamp8(R(acc * m_r * m_c, k_r + k_c))
 *   FIX     out_i32 = R(acc * m_r * m_c, k_r + k_c - frac)
 *   RES_ADD out_i32 += R(acc * m_r * m_c, k_r + k_c - frac)              */
int orc_epilogue(const int64_t *acc, int64_t M, int64_t N,
                 const int32_t *row_m, const int32_t *row_k,
                 const int32_t *col_m, int32_t col_k, int32_t frac,
                 int32_t mode, void *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; i++)
    for (int64_t j = 0; j < N; j++) {
      int64_t a = acc[i * N + j];
      if (mode == ORC_RAW) {
        CHECK(a <= INT32_MAX && a >= INT32_MIN, "raw acc exceeds int32");
        ((int32_t *)out)[i * N + j] = (int32_t)a;
        continue;
      }
      i128 p = (i128)a * row_m[i] * col_m[j];
      int s = row_k[i] + col_k - (mode == ORC_REQ_I8 ? 0 : frac);
      int64_t y = R128(p, s);
      if (mode == ORC_REQ_I8) {
        ((int8_t *)out)[i * N + j] = clamp8(y);
      } else if (mode == ORC_FIX) {
        CHECK(y <= INT32_MAX && y >= INT32_MIN, "fix output exceeds int32");
        ((int32_t *)out)[i * N + j] = (int32_t)y;
      } else {
        int64_t h = (int64_t)((int32_t *)out)[i * N + j] + y;
        CHECK(h <= INT32_MAX && h >= INT32_MIN, "residual exceeds int32");
        ((int32_t *)out)[i * N + j] = (int32_t)h;
      }
    }
  return g_err;
}

/* ------------------------------------------------------------------ */
/* exact mode: bf16 weights as fixed point                             */

/* Exact-mode weights ([BITEXACT] "Three execution paths": exact mode keeps
 * the original bf16 weights of the linear layers and multiplies them with
 * fixed-point activations; "Fix the arithmetic": products split into integer
 * limbs and combined in wide accumulators). A bf16 pattern (sign s, 8-bit
 * exponent field E, 7-bit fraction f) is the real number (-1)^s * M *
 * 2^(E' - 134), with M = 128 + f and E' = E for E >= 1 (normal numbers), M = f
 * and E' = 1 for E = 0 (zero and subnormals); E = 255 (infinity, NaN) has no
 * integer form and is an error. Reading taken (the pages state no format):
 * each output channel (row j of W [N, K]) gets a power-of-two scale, the
 * smallest E' among its nonzero entries (emin_j; 1 for an all-zero row), and
 * its integers W_int[j][k] = (-1)^s * M * 2^(E'_k - emin_j), so that
 * w[j][k] = W_int[j][k] * 2^row_exp[j] exactly with row_exp[j] = emin_j - 134.
 * Bound: |W_int| < 2^31, i.e. exponents within a row span at most 23. */
int orc_exact_weights(const uint16_t *W, int64_t N, int64_t K, int32_t *W_int, int32_t *row_exp) {
  for (int64_t j = 0; j < N; j++) {
    const uint16_t *w = W + j * K;
    int emin = 255;
    for (int64_t k = 0; k < K; k++) {
      const int E = (w[k] >> 7) & 255, f = w[k] & 127;
      CHECK(E != 255, "exact weights: infinity or NaN");
      const int Ep = E ? E : 1, M = E ? 128 + f : f;
      if (M != 0 && Ep < emin) emin = Ep;
    }
    if (emin == 255) emin = 1;   /* all zeros */
    for (int64_t k = 0; k < K; k++) {
      const int E = (w[k] >> 7) & 255, f = w[k] & 127;
      const int Ep = E ? E : 1, M = E ? 128 + f : f;
      int64_t v = 0;
      if (M != 0 && E != 255) {
        CHECK(Ep - emin <= 23, "exact weights: exponents of a row span more than 23");
        v = (Ep - emin <= 23) ? (int64_t)M << (Ep - emin) : 0;
      }
      W_int[j * K + k] = (int32_t)((w[k] & 0x8000) ? -v : v);
    }
    row_exp[j] = emin - 134;
  }
  return g_err;
}

/* acc[i][j] = sum_k A[i][k] * W_int[j][k], exactly (int8 activations times
 * the exact-mode integers; |acc| < 2^7 * 2^31 * K must fit int64). */
int orc_gemm_exact(const int8_t *A, const int32_t *W_int, int64_t M, int64_t N, int64_t K,
                   int64_t *acc) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < N; j++)
    for (int64_t i = 0; i < M; i++) {
      i128 s = 0;
      for (int64_t k = 0; k < K; k++) s += (i128)A[i * K + k] * W_int[j * K + k];
      CHECK(s <= INT64_MAX && s >= INT64_MIN, "exact acc exceeds int64");
      acc[i * N + j] = (int64_t)s;
    }
  return g_err;
}

/* Dyadic epilogue of an exact-mode product. Row i of the activations stands
 * for x8 * m_r * 2^-k_r and column j's weights for W_int * 2^row_exp[j], so
 * the real output is acc * m_r * 2^(row_exp[j] - k_r):
 *   RAW     out_i64 = acc
 *   REQ_I8  out_i8  = clamp8(R(acc * m_r, k_r - row_exp[j]))
 *   FIX     out_i32 = R(acc * m_r, k_r - row_exp[j] - frac) (must fit int32) */
int orc_exact_epilogue(const int64_t *acc, int64_t M, int64_t N, const int32_t *row_m,
                       const int32_t *row_k, const int32_t *row_exp, int32_t frac, int32_t mode,
                       void *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; i++)
    for (int64_t j = 0; j < N; j++) {
      const int64_t a = acc[i * N + j];
      if (mode == ORC_RAW) {
        ((int64_t *)out)[i * N + j] = a;
        continue;
      }
      const int sh = row_k[i] - row_exp[j] - (mode == ORC_REQ_I8 ? 0 : frac);
      const i128 p = (i128)a * row_m[i];
      int64_t y;
      if (sh > 120) {
        y = 0;
      } else {
        CHECK(sh > -62, "exact epilogue left shift");
        y = R128(p, sh);
      }
      if (mode == ORC_REQ_I8) {
        ((int8_t *)out)[i * N + j] = clamp8(y);
      } else {
        CHECK(y <= INT32_MAX && y >= INT32_MIN, "exact fix output exceeds int32");
        ((int32_t *)out)[i * N + j] = (int32_t)y;
      }
    }
  return g_err;
}

/* ------------------------------------------------------------------ */
/* row ops                                                             */

/* DI-RMSNorm of one row ([README] "Layout": ops/ DI-RMSNorm). The output
 * x8 * m_r * 2^-k_r approximates h_i * (g_i / 2^12) / rms(h):
 *   S = sum h_i^2, (m, sh) = irms(S, n), (x8, e) = DQ(h_i * g_i),
 *   m_r = m, k_r = sh + 12 - e.
 * An all-zero row gives x8 = 0 with scale (2^14, 26), i.e. irms = 1. */
static void rmsnorm_row(const int32_t *h, const int16_t *g, int64_t n,
                        int8_t *x8, int32_t *m_r, int32_t *k_r, int64_t *tmp) {
  int64_t S = 0;
  for (int64_t i = 0; i < n; i++) {
    CHECK(h[i] < (1 << 25) && h[i] > -(1 << 25), "rmsnorm input |h| >= 2^25");
    S += (int64_t)h[i] * h[i];
  }
  if (S == 0) {
    for (int64_t i = 0; i < n; i++) x8[i] = 0;
    *m_r = 1 << 14; *k_r = 26;
    return;
  }
  int32_t m, sh, e;
  orc_irms(S, n, &m, &sh);
  for (int64_t i = 0; i < n; i++) tmp[i] = (int64_t)h[i] * g[i];
  orc_dq(tmp, n, x8, &e);
  *m_r = m;
  *k_r = sh + 12 - e;
}

int orc_rmsnorm(const int32_t *h, const int16_t *g, int64_t rows, int64_t n,
                int8_t *x8, int32_t *m_r, int32_t *k_r) {
#pragma omp parallel
  {
    int64_t *tmp = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; r++)
      rmsnorm_row(h + r * n, g, n, x8 + r * n, m_r + r, k_r + r, tmp);
    free(tmp);
  }
  return g_err;
}

/* DQ applied to each row of an int32 matrix: q = clamp8(R(y, e_row)). */
int orc_requant_rows(const int32_t *y, int64_t rows, int64_t n, int8_t *q, int32_t *e) {
#pragma omp parallel
  {
    int64_t *tmp = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
      for (int64_t i = 0; i < n; i++) tmp[i] = y[r * n + i];
      orc_dq(tmp, n, q + r * n, e + r);
    }
    free(tmp);
  }
  return g_err;
}

/* Requantisation at a fixed dyadic scale ([BLOG] "DetLLM": K and V are
 * quantised once at fixed offline scales): q = clamp8(R(y * m, k)). */
int orc_requant_fixed(const int32_t *y, int64_t n, int32_t m, int32_t k, int8_t *q) {
  for (int64_t i = 0; i < n; i++) q[i] = clamp8(R((int64_t)y[i] * m, k));
  return g_err;
}

/* Per-head RMSNorm of q or k (Qwen3 q/k-norm, which [BLOG] footnote 8 places
 * before RoPE). Input a_j = acc_j * m_c_j (the per-tensor column shift and the
 * row scale cancel in a normalisation). Pre-shift p = max(0, bl(max|a|) - 24),
 * a' = R(a, p); (m, sh) = irms(sum a'^2, d);
 * out_j = R(a'_j * g_j * m, sh + 12 - f_n): normalised value times gain in
 * f_n fractional bits. A zero head gives zeros. */
static void head_norm(const int64_t *a, const int16_t *g, int64_t d, int32_t f_n, int64_t *out) {
  uint64_t A = 0;
  for (int64_t j = 0; j < d; j++) {
    uint64_t v = a[j] < 0 ? (uint64_t)(-a[j]) : (uint64_t)a[j];
    if (v > A) A = v;
  }
  int b = orc_bitlen(A);
  int p = b > 24 ? b - 24 : 0;
  int64_t ap[512];
  int64_t S = 0;
  for (int64_t j = 0; j < d; j++) { ap[j] = R(a[j], p); S += ap[j] * ap[j]; }
  if (S == 0) { for (int64_t j = 0; j < d; j++) out[j] = 0; return; }
  int32_t m, sh;
  orc_irms(S, d, &m, &sh);
  for (int64_t j = 0; j < d; j++) out[j] = R(ap[j] * g[j] * m, sh + 12 - f_n);
}

/* Integer RoPE on one head vector at position pos: pairs (i, i + d/2),
 * x'_i = R(x_i C - x_{i+d/2} S, 14), x'_{i+d/2} = R(x_{i+d/2} C + x_i S, 14). */
static void rope_vec(int64_t *x, int64_t d, const int16_t *cos_row, const int16_t *sin_row) {
  int64_t half = d / 2;
  for (int64_t i = 0; i < half; i++) {
    int64_t a = x[i], b = x[i + half];
    int64_t c = cos_row[i], s = sin_row[i];
    x[i] = R(a * c - b * s, 14);
    x[i + half] = R(b * c + a * s, 14);
  }
}

int orc_rope(int32_t *x, const int32_t *pos, const int16_t *cos_t, const int16_t *sin_t,
             int64_t rows, int64_t heads, int64_t d, int64_t max_pos) {
  CHECK(d > 0 && d <= 512 && d % 2 == 0, "rope head_dim");
  if (g_err) return g_err;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    CHECK(pos[r] >= 0 && pos[r] < max_pos, "rope position out of table");
    if (pos[r] < 0 || pos[r] >= max_pos) continue;
    for (int64_t h = 0; h < heads; h++) {
      int64_t v[512];
      int32_t *p = x + (r * heads + h) * d;
      for (int64_t j = 0; j < d; j++) v[j] = p[j];
      rope_vec(v, d, cos_t + pos[r] * (d / 2), sin_t + pos[r] * (d / 2));
      for (int64_t j = 0; j < d; j++) {
        CHECK(v[j] <= INT32_MAX && v[j] >= INT32_MIN, "rope output exceeds int32");
        p[j] = (int32_t)v[j];
      }
    }
  }
  return g_err;
}

/* DI-Softmax over one row of integer scores, 15-bit probabilities ([BLOG]
 * footnote 8: probabilities carry 15 bits). With mx the row max over the
 * valid entries, u_j = R((s_j - mx) * M, K - shift) is the base-2 Q15
 * exponent, E_j = DI-Exp(u_j), D = sum E_j, Rn = floor(2^46 / D),
 * P_j = min(R(E_j * Rn, 31), 2^15 - 1); entries past the valid length get 0. */
static void softmax_row(const int32_t *s, int64_t valid, int32_t M, int32_t K,
                        int32_t shift, int32_t *E, int16_t *P, int64_t C) {
  int64_t mx = INT64_MIN;
  for (int64_t j = 0; j < valid; j++) if (s[j] > mx) mx = s[j];
  int64_t D = 0;
  for (int64_t j = 0; j < valid; j++) {
    int64_t u = R(((int64_t)s[j] - mx) * M, K - shift);
    E[j] = orc_diexp(u);
    D += E[j];
  }
  int64_t Rn = D > 0 ? ((int64_t)1 << 46) / D : 0;
  for (int64_t j = 0; j < C; j++) {
    if (j < valid) {
      int64_t p = R((int64_t)E[j] * Rn, 31);
      P[j] = (int16_t)(p > 32767 ? 32767 : p);
    } else {
      P[j] = 0;
    }
  }
}

int orc_softmax(const int32_t *s, const int32_t *valid, const int32_t *shift,
                int64_t rows, int64_t C, int32_t M, int32_t K, int16_t *P) {
#pragma omp parallel
  {
    int32_t *E = (int32_t *)malloc(sizeof(int32_t) * (C > 0 ? C : 1));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
      CHECK(valid[r] >= 1 && valid[r] <= C, "softmax valid length");
      if (valid[r] < 1 || valid[r] > C) continue;
      softmax_row(s + r * C, valid[r], M, K, shift[r], E, P + r * C, C);
    }
    free(E);
  }
  return g_err;
}

/* DI-SwiGLU of one row ([README] "Layout": ops/ DI-SwiGLU). g, u are the gate
 * and up projections in f_a fractional bits. Integer sigmoid in Q15 from
 * sigmoid(|g|) = 1/(1 + e^-|g|): E = DI-Exp(-R(|g| * Mg, Kg)),
 * s+ = RD(2^30, 2^15 + E); s = s+ for g >= 0 else 2^15 - s+ (so s(-g) = 2^15 - s(g)
 * exactly). silu = R(g * s, 15); p = silu * u; (a8, e) = DQ(p) with row scale
 * (2^14, 2 f_a - e + 14). */
int32_t orc_sigmoid_q15(int64_t g, int32_t Mg, int32_t Kg) {
  int64_t ag = g < 0 ? -g : g;
  int64_t E = orc_diexp(-R(ag * Mg, Kg));
  int64_t sp = orc_div_round((int64_t)1 << 30, 32768 + E);
  return (int32_t)(g >= 0 ? sp : 32768 - sp);
}

static void swiglu_row(const int32_t *g, const int32_t *u, int64_t n, int32_t f_a,
                       int8_t *a8, int32_t *m_r, int32_t *k_r, int64_t *tmp) {
  int32_t Mg, Kg;
  orc_swiglu_mult(f_a, &Mg, &Kg);
  for (int64_t j = 0; j < n; j++) {
    int64_t gj = g[j], uj = u[j];
    CHECK(gj < (1 << 24) && gj > -(1 << 24), "swiglu |g| >= 2^24");
    CHECK(uj < (1 << 24) && uj > -(1 << 24), "swiglu |u| >= 2^24");
    int64_t silu = R(gj * orc_sigmoid_q15(gj, Mg, Kg), 15);
    tmp[j] = silu * uj;
  }
  int32_t e;
  orc_dq(tmp, n, a8, &e);
  *m_r = 1 << 14;
  *k_r = 2 * f_a - e + 14;
}

int orc_swiglu(const int32_t *gu, int64_t rows, int64_t n, int32_t f_a,
               int8_t *a8, int32_t *m_r, int32_t *k_r) {
#pragma omp parallel
  {
    int64_t *tmp = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; r++)
      swiglu_row(gu + r * 2 * n, gu + r * 2 * n + n, n, f_a, a8 + r * n, m_r + r, k_r + r, tmp);
    free(tmp);
  }
  return g_err;
}

/* ------------------------------------------------------------------ */
/* model                                                               */

typedef struct {
  const int8_t *wqkv; const int16_t *wqkv16; const int32_t *wqkv_m;
  const int8_t *wo;   const int16_t *wo16;   const int32_t *wo_m;
  const int8_t *wgu;  const int16_t *wgu16;  const int32_t *wgu_m;
  const int8_t *wd;   const int16_t *wd16;   const int32_t *wd_m;
  const int16_t *attn_norm, *ffn_norm, *q_norm, *k_norm;
  int32_t kq_m, kq_k, vq_m, vq_k;
  const int8_t *k_gain; /* [n_kv][d] per-channel key gains in [0, 7], or NULL */
} orc_layer;

typedef struct {
  int64_t n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab, max_pos;
  int32_t qk_norm, wide, w_k, f_res, f_n, f_a, f_l, pad_;
  const int8_t *emb; const int16_t *emb16; const int32_t *emb_m;
  const int16_t *final_norm;
  const int16_t *rope_cos, *rope_sin;   /* [max_pos][d/2] */
  const orc_layer *layers;
} orc_model;

/* optional per-layer intermediates (any pointer may be NULL) */
typedef struct {
  int8_t *x1; int32_t *x1_m, *x1_k;
  int64_t *qkv_acc;
  int8_t *q8; int32_t *eq;
  int32_t *attn;
  int8_t *o8; int32_t *o_m, *o_k;
  int32_t *h_mid;
  int8_t *x2; int32_t *x2_m, *x2_k;
  int32_t *gu;
  int8_t *a8; int32_t *a_m, *a_k;
} orc_dump;

/* KV cache layout (oracle's own): [layer][slot][kv head][position][d] int8 */
static int8_t *kv_at(int8_t *cache, const orc_model *md, int64_t slots,
                     int64_t l, int64_t slot, int64_t h, int64_t p) {
  return cache + ((((l * slots + slot) * md->n_kv + h) * md->max_pos + p) * md->head_dim);
}

/* Linear layer + epilogue; W8 or W16 chosen by the model's weight width. */
static void linear(const orc_model *md, const int8_t *x8, int64_t R_, int64_t K,
                   const int8_t *w8, const int16_t *w16, int64_t N, int64_t *acc) {
  orc_gemm(x8, md->wide ? NULL : w8, md->wide ? w16 : NULL, R_, N, K, acc);
}

/* Attention of R query rows over one layer's int8 cache [slot][kv head]
 * [position][d] (oracle layout). Row r sits at position pos[r] of slot slot[r]
 * and attends positions 0..pos[r] (causal, keys already cached). Query head hh
 * reads KV head hh * nkv / nq (grouped-query). Scores s_j = q8 . k8_j go
 * through DI-Softmax with shift e_q[r][hh] (15-bit P, [BLOG] footnote 8) and
 * out[r][hh][t] = sum_j P_j * v8_j[t], exactly. */
int orc_attention(const int8_t *q8, const int32_t *eq, const int8_t *kc, const int8_t *vc,
                  const int32_t *pos, const int32_t *slot, int64_t R_, int64_t nq, int64_t nkv,
                  int64_t d, int64_t slots, int64_t max_pos, int32_t sm_M, int32_t sm_K,
                  int32_t *att) {
  for (int64_t r = 0; r < R_; r++)
    CHECK(pos[r] >= 0 && pos[r] < max_pos && slot[r] >= 0 && slot[r] < slots, "attention row position/slot");
  if (g_err) return g_err;
#pragma omp parallel
  {
    int32_t *sc = malloc(4 * max_pos), *E = malloc(4 * max_pos);
    int16_t *P = malloc(2 * max_pos);
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < R_; r++)
      for (int64_t hh = 0; hh < nq; hh++) {
        const int64_t p = pos[r], kvh = hh * nkv / nq;
        const int8_t *kb = kc + ((slot[r] * nkv + kvh) * max_pos) * d;
        const int8_t *vb = vc + ((slot[r] * nkv + kvh) * max_pos) * d;
        const int8_t *q = q8 + (r * nq + hh) * d;
        for (int64_t j = 0; j <= p; j++) {
          int64_t s = 0;
          for (int64_t t = 0; t < d; t++) s += (int64_t)q[t] * kb[j * d + t];
          sc[j] = (int32_t)s;
        }
        softmax_row(sc, p + 1, sm_M, sm_K, eq[r * nq + hh], E, P, p + 1);
        for (int64_t t = 0; t < d; t++) {
          int64_t o = 0;
          for (int64_t j = 0; j <= p; j++) o += (int64_t)P[j] * vb[j * d + t];
          CHECK(o < ((int64_t)1 << 31) && o > -((int64_t)1 << 31), "attention output exceeds int32");
          att[(r * nq + hh) * d + t] = (int32_t)o;
        }
      }
    free(sc); free(E); free(P);
  }
  return g_err;
}

/* Row index -> (sequence, absolute position). */
static void row_positions(const int32_t *cu, const int32_t *start, int64_t S,
                          int64_t *seq_of, int64_t *pos_of) {
  for (int64_t s = 0; s < S; s++)
    for (int64_t r = cu[s]; r < cu[s + 1]; r++) {
      seq_of[r] = s;
      pos_of[r] = start[s] + (r - cu[s]);
    }
}

/* One decoder layer over R packed rows (sequence s owns rows cu[s]..cu[s+1]-1
 * at positions start[s]..; its KV lives in cache slot slot[s]).
 * Step order ([README] "Layout": IntQwen3 runtime; [BLOG] "DetLLM"):
 * RMSNorm -> QKV -> (q/k-norm) -> RoPE -> q DQ, K/V to the int8 cache at
 * fixed scales -> attention with DI-Softmax -> DQ -> O-proj + residual ->
 * RMSNorm -> gate/up -> DI-SwiGLU -> down + residual. */
int orc_layer_forward(const orc_model *md, int64_t l, int32_t *h, int64_t R_,
                      const int32_t *cu, const int32_t *start, const int32_t *slot,
                      int64_t S, int8_t *kc, int8_t *vc, int64_t slots, orc_dump *dump) {
  const orc_layer *L = &md->layers[l];
  const int64_t H = md->hidden, nq = md->n_q, nkv = md->n_kv, d = md->head_dim, F = md->ffn;
  const int64_t Nqkv = (nq + 2 * nkv) * d;
  const int32_t wk = md->w_k;
  int64_t *seq_of = malloc(sizeof(int64_t) * R_), *pos_of = malloc(sizeof(int64_t) * R_);
  row_positions(cu, start, S, seq_of, pos_of);
  for (int64_t r = 0; r < R_; r++)
    CHECK(pos_of[r] >= 0 && pos_of[r] < md->max_pos, "position beyond cache/table");
  if (g_err) { free(seq_of); free(pos_of); return g_err; }

  int64_t maxK = H;
  if (F > maxK) maxK = F;
  if (nq * d > maxK) maxK = nq * d;
  int8_t *x8 = malloc(R_ * maxK);
  int32_t *xm = malloc(4 * R_), *xk = malloc(4 * R_);
  int64_t maxN = Nqkv > 2 * F ? Nqkv : 2 * F;
  if (H > maxN) maxN = H;
  int64_t *acc = malloc(8 * R_ * maxN);
  int8_t *q8 = malloc(R_ * nq * d);
  int32_t *eq = malloc(4 * R_ * nq);
  int32_t *att = malloc(4 * R_ * nq * d);
  int32_t *gu = malloc(4 * R_ * 2 * F);
  int32_t sm_M, sm_K, vd_m, vd_k;
  orc_softmax_mult(L->kq_m, L->kq_k, d, md->f_n, &sm_M, &sm_K);
  orc_v_dequant(L->vq_m, L->vq_k, &vd_m, &vd_k);

  /* 1. attention RMSNorm -> x8 */
  orc_rmsnorm(h, L->attn_norm, R_, H, x8, xm, xk);
  if (dump && dump->x1) { memcpy(dump->x1, x8, R_ * H); memcpy(dump->x1_m, xm, 4 * R_); memcpy(dump->x1_k, xk, 4 * R_); }

  /* 2. QKV projection (exact accumulators) */
  linear(md, x8, R_, H, L->wqkv, L->wqkv16, Nqkv, acc);
  if (dump && dump->qkv_acc) memcpy(dump->qkv_acc, acc, 8 * R_ * Nqkv);

  /* 3. per-head post-processing: q/k-norm or fixed-point rescale, RoPE,
   *    q dynamic quant, K/V quantised once at fixed scales into the cache
   *    ([BLOG] "DetLLM": K/V use fixed offline scales so prefill and decode
   *    see the same cached bits). */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R_; r++) {
    const int64_t *ar = acc + r * Nqkv;
    const int64_t p = pos_of[r];
    const int16_t *cr = md->rope_cos + p * (d / 2), *sr = md->rope_sin + p * (d / 2);
    for (int64_t hh = 0; hh < nq + 2 * nkv; hh++) {
      int64_t v[512], a[512];
      const int64_t c0 = hh * d;
      const int is_q = hh < nq, is_k = hh >= nq && hh < nq + nkv;
      if (!is_q && !is_k) {
        /* V: fixed point f_n, then the static cache scale */
        int64_t kvh = hh - nq - nkv;
        int8_t *dst = kv_at(vc, md, slots, l, slot[seq_of[r]], kvh, p);
        for (int64_t j = 0; j < d; j++) {
          int64_t vf = R128((i128)ar[c0 + j] * xm[r] * L->wqkv_m[c0 + j], xk[r] + wk - md->f_n);
          CHECK(vf < ((int64_t)1 << 31) && vf > -((int64_t)1 << 31), "v exceeds int32");
          dst[j] = clamp8(R(vf * L->vq_m, L->vq_k));
        }
        continue;
      }
      if (md->qk_norm) {
        for (int64_t j = 0; j < d; j++) a[j] = ar[c0 + j] * L->wqkv_m[c0 + j];
        head_norm(a, is_q ? L->q_norm : L->k_norm, d, md->f_n, v);
      } else {
        for (int64_t j = 0; j < d; j++)
          v[j] = R128((i128)ar[c0 + j] * xm[r] * L->wqkv_m[c0 + j], xk[r] + wk - md->f_n);
      }
      for (int64_t j = 0; j < d; j++)
        CHECK(v[j] < ((int64_t)1 << 31) && v[j] > -((int64_t)1 << 31), "q/k exceeds int32");
      rope_vec(v, d, cr, sr);
      for (int64_t j = 0; j < d; j++)
        CHECK(v[j] < ((int64_t)1 << 31) && v[j] > -((int64_t)1 << 31), "rotated q/k exceeds int32");
      /* per-channel key rescale (DetLLM blog footnote 8): key channel j
       * of KV head h scaled by 2^g, query channel j of the heads sharing h
       * by 2^-g before their quantisation, g = k_gain[h][j] */
      const int64_t kvh = is_q ? hh / (nq / nkv) : hh - nq;
      const int8_t *g = L->k_gain ? L->k_gain + kvh * d : NULL;
      if (g) {
        CHECK(L->kq_k >= 8, "key gains need kq_k >= 8");
        for (int64_t j = 0; j < d; j++) CHECK(g[j] >= 0 && g[j] <= 7, "key gain outside [0, 7]");
      }
      if (is_q) {
        if (g)
          for (int64_t j = 0; j < d; j++) v[j] = R(v[j], g[j]);
        orc_dq(v, d, q8 + (r * nq + hh) * d, eq + r * nq + hh);
      } else {
        int8_t *dst = kv_at(kc, md, slots, l, slot[seq_of[r]], kvh, p);
        for (int64_t j = 0; j < d; j++)
          dst[j] = clamp8(R(v[j] * L->kq_m, L->kq_k - (g ? g[j] : 0)));
      }
    }
  }
  if (dump && dump->q8) { memcpy(dump->q8, q8, R_ * nq * d); memcpy(dump->eq, eq, 4 * R_ * nq); }

  /* 4. attention over the cache */
  {
    int32_t *po = malloc(4 * R_), *so = malloc(4 * R_);
    for (int64_t r = 0; r < R_; r++) { po[r] = (int32_t)pos_of[r]; so[r] = slot[seq_of[r]]; }
    orc_attention(q8, eq, kc + l * slots * nkv * md->max_pos * d, vc + l * slots * nkv * md->max_pos * d,
                  po, so, R_, nq, nkv, d, slots, md->max_pos, sm_M, sm_K, att);
    free(po); free(so);
  }
  if (dump && dump->attn) memcpy(dump->attn, att, 4 * R_ * nq * d);

  /* 5. DQ over the concatenated heads; row scale folds the V dequant scale,
   *    the Q15 probability scale and f_n: (vd_m, vd_k + 15 + f_n - e) */
  int32_t *oe = malloc(4 * R_);
  orc_requant_rows(att, R_, nq * d, x8, oe);
  for (int64_t r = 0; r < R_; r++) { xm[r] = vd_m; xk[r] = vd_k + 15 + md->f_n - oe[r]; }
  free(oe);
  if (dump && dump->o8) { memcpy(dump->o8, x8, R_ * nq * d); memcpy(dump->o_m, xm, 4 * R_); memcpy(dump->o_k, xk, 4 * R_); }

  /* 6. O projection + residual */
  linear(md, x8, R_, nq * d, L->wo, L->wo16, H, acc);
  orc_epilogue(acc, R_, H, xm, xk, L->wo_m, wk, md->f_res, ORC_RES_ADD, h);
  for (int64_t i = 0; i < R_ * H; i++) CHECK(h[i] < (1 << 25) && h[i] > -(1 << 25), "residual |h| >= 2^25");
  if (dump && dump->h_mid) memcpy(dump->h_mid, h, 4 * R_ * H);

  /* 7. FFN RMSNorm, gate/up, DI-SwiGLU */
  orc_rmsnorm(h, L->ffn_norm, R_, H, x8, xm, xk);
  if (dump && dump->x2) { memcpy(dump->x2, x8, R_ * H); memcpy(dump->x2_m, xm, 4 * R_); memcpy(dump->x2_k, xk, 4 * R_); }
  linear(md, x8, R_, H, L->wgu, L->wgu16, 2 * F, acc);
  orc_epilogue(acc, R_, 2 * F, xm, xk, L->wgu_m, wk, md->f_a, ORC_FIX, gu);
  if (dump && dump->gu) memcpy(dump->gu, gu, 4 * R_ * 2 * F);
  orc_swiglu(gu, R_, F, md->f_a, x8, xm, xk);
  if (dump && dump->a8) { memcpy(dump->a8, x8, R_ * F); memcpy(dump->a_m, xm, 4 * R_); memcpy(dump->a_k, xk, 4 * R_); }

  /* 8. down projection + residual */
  linear(md, x8, R_, F, L->wd, L->wd16, H, acc);
  orc_epilogue(acc, R_, H, xm, xk, L->wd_m, wk, md->f_res, ORC_RES_ADD, h);
  for (int64_t i = 0; i < R_ * H; i++) CHECK(h[i] < (1 << 25) && h[i] > -(1 << 25), "residual |h| >= 2^25");

  free(seq_of); free(pos_of); free(x8); free(xm); free(xk); free(acc);
  free(q8); free(eq); free(att); free(gu);
  return g_err;
}

/* Embedding lookup onto the residual stream ([BITEXACT] "Three execution
 * paths": the embedding enters the integer residual once, by one rounding to
 * its fixed-point grid). The table entry's real value is E[id] * m_v[id] *
 * 2^-w_k; in units of 2^-f_res that is E * m_v * 2^(f_res - w_k), rounded
 * by the one rule: h0 = R(E[id] * m_v[id], w_k - f_res). */
int orc_embed(const orc_model *md, const int32_t *ids, int64_t R_, int32_t *h) {
  const int64_t H = md->hidden;
  for (int64_t r = 0; r < R_; r++) {
    CHECK(ids[r] >= 0 && ids[r] < md->vocab, "token id out of range");
    if (ids[r] < 0 || ids[r] >= md->vocab) return g_err;
    for (int64_t i = 0; i < H; i++) {
      int64_t e = md->wide ? md->emb16[ids[r] * H + i] : md->emb[ids[r] * H + i];
      int64_t v = R(e * md->emb_m[ids[r]], md->w_k - md->f_res);
      CHECK(v < (1 << 25) && v > -(1 << 25), "embedding |h| >= 2^25");
      h[r * H + i] = (int32_t)v;
    }
  }
  return g_err;
}

/* Greedy token: the lowest index among the row's maxima ([BLOG] "DetLLM":
 * argmax prefers the smallest token id on ties). */
int orc_argmax(const int32_t *logits, int64_t rows, int64_t V, int32_t *out) {
  for (int64_t o = 0; o < rows; o++) {
    int64_t best = 0;
    for (int64_t j = 1; j < V; j++)
      if (logits[o * V + j] > logits[o * V + best]) best = j;
    out[o] = (int32_t)best;
  }
  return 0;
}

/* Integer sampling with temperature and top-k ([BITEXACT] intro: sampling
 * rules are part of the integer arithmetic, and deterministic sampling is
 * named among its unavoidable costs; [BLOG] limits section: integer sampling
 * left open). The pages give no formula; the reading taken here:
 *  - order: key(j) ranks a larger logit first and, among equal logits, the
 *    lower id first (the greedy tie rule, [BLOG] "DetLLM");
 *  - top-k: the k highest-ranked ids are kept (k <= 0 or k >= V keeps all);
 *  - weights: E_j = DI-Exp(R((l_j - l_max) * t_m, t_k)) for kept ids, else 0:
 *    the temperature is the dyadic t_m / 2^t_k applied to the logit gap in
 *    DI-Exp's base-2 Q15 units (the softmax's own exponential), so the
 *    maximum gets E = 2^15 and D = sum E >= 2^15;
 *  - top-p (nucleus), p = top_p / 2^16 with 1 <= top_p <= 2^16 (2^16: off):
 *    with D_k = sum of E over the top-k ids and P = ceil(top_p D_k / 2^16),
 *    keep the shortest prefix of the ranking whose weight sum reaches P
 *    (equal logits have equal weights, so ties again go to the lower id);
 *  - draw: the caller's uniform 32-bit integer r selects t = floor(r D / 2^32),
 *    in [0, D), D the weight sum of the kept ids;
 *  - token: the smallest id j with E_0 + ... + E_j > t (kept ids only).
 * Bounds: 1 <= t_m < 2^24, 0 <= t_k <= 62 (the gap times t_m stays < 2^56). */
static const int32_t *g_sort_row;
static int key_desc(const void *a, const void *b) {
  const int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
  const int32_t li = g_sort_row[i], lj = g_sort_row[j];
  if (li != lj) return li > lj ? -1 : 1;
  return i < j ? -1 : (i > j ? 1 : 0);
}

int orc_sample(const int32_t *logits, int64_t rows, int64_t V, int64_t k, int32_t top_p,
               int32_t t_m, int32_t t_k, const uint32_t *draws, int32_t *out) {
  CHECK(V >= 1, "sample: V < 1");
  CHECK(t_m >= 1 && t_m < (1 << 24) && t_k >= 0 && t_k <= 62, "sample: temperature dyadic");
  CHECK(top_p >= 1 && top_p <= 65536, "sample: top_p outside [1, 2^16]");
  if (g_err) return g_err;
  const int64_t keep = (k <= 0 || k >= V) ? V : k;
  int32_t *idx = (int32_t *)malloc((size_t)V * sizeof(int32_t));
  uint8_t *kept = (uint8_t *)malloc((size_t)V);
  for (int64_t o = 0; o < rows && !g_err; o++) {
    const int32_t *l = logits + o * V;
    int64_t lmax = l[0];
    for (int64_t j = 1; j < V; j++) if (l[j] > lmax) lmax = l[j];
    if (keep == V && top_p == 65536) {
      memset(kept, 1, (size_t)V);
    } else {
      for (int64_t j = 0; j < V; j++) idx[j] = (int32_t)j;
      g_sort_row = l;
      qsort(idx, (size_t)V, sizeof(int32_t), key_desc);
      int64_t m = keep;
      if (top_p < 65536) {
        int64_t Dk = 0;
        for (int64_t i = 0; i < keep; i++) Dk += orc_diexp(R(((int64_t)l[idx[i]] - lmax) * t_m, t_k));
        const int64_t P = ((int64_t)top_p * Dk + 65535) >> 16;
        int64_t cum = 0;
        for (m = 0; m < keep && cum < P; m++) cum += orc_diexp(R(((int64_t)l[idx[m]] - lmax) * t_m, t_k));
      }
      memset(kept, 0, (size_t)V);
      for (int64_t i = 0; i < m; i++) kept[idx[i]] = 1;
    }
    int64_t D = 0;
    for (int64_t j = 0; j < V; j++)
      if (kept[j]) D += orc_diexp(R(((int64_t)l[j] - lmax) * t_m, t_k));
    CHECK(D >= 32768, "sample: D < 2^15");
    const int64_t t = (int64_t)(((unsigned __int128)draws[o] * (uint64_t)D) >> 32);
    int64_t cum = 0, tok = -1;
    for (int64_t j = 0; j < V && tok < 0; j++) {
      if (kept[j]) cum += orc_diexp(R(((int64_t)l[j] - lmax) * t_m, t_k));
      if (cum > t) tok = j;
    }
    CHECK(tok >= 0, "sample: no token");
    out[o] = (int32_t)tok;
  }
  free(idx);
  free(kept);
  return g_err;
}

/* Whole forward: ids -> embedding -> layers -> final RMSNorm -> tied lm_head
 * -> int32 logits ([README] intro: ids to int32 logits with no float), for the
 * last row of every sequence (all rows when all_rows != 0), and the greedy
 * token = lowest id among the maxima ([BLOG] "DetLLM": ties go to the smallest
 * token id). Logits: R(acc * m_r * m_v, k_r + w_k - f_l), must fit int32. */
int orc_forward(const orc_model *md, const int32_t *ids, int64_t R_,
                const int32_t *cu, const int32_t *start, const int32_t *slot, int64_t S,
                int8_t *kc, int8_t *vc, int64_t slots, int32_t all_rows,
                int32_t *logits, int32_t *next_tok) {
  const int64_t H = md->hidden, V = md->vocab;
  int32_t *h = malloc(4 * R_ * H);
  orc_embed(md, ids, R_, h);
  for (int64_t l = 0; l < md->n_layers && !g_err; l++)
    orc_layer_forward(md, l, h, R_, cu, start, slot, S, kc, vc, slots, NULL);
  if (g_err) { free(h); return g_err; }
  int64_t nout = all_rows ? R_ : S;
  int32_t *hs = malloc(4 * nout * H);
  for (int64_t o = 0; o < nout; o++) {
    int64_t r = all_rows ? o : cu[o + 1] - 1;
    memcpy(hs + o * H, h + r * H, 4 * H);
  }
  int8_t *x8 = malloc(nout * H);
  int32_t *xm = malloc(4 * nout), *xk = malloc(4 * nout);
  int64_t *acc = malloc(8 * nout * V);
  orc_rmsnorm(hs, md->final_norm, nout, H, x8, xm, xk);
  orc_gemm(x8, md->wide ? NULL : md->emb, md->wide ? md->emb16 : NULL, nout, V, H, acc);
  orc_epilogue(acc, nout, V, xm, xk, md->emb_m, md->w_k, md->f_l, ORC_FIX, logits);
  if (next_tok) orc_argmax(logits, nout, V, next_tok);
  free(h); free(hs); free(x8); free(xm); free(xk); free(acc);
  return g_err;
}
