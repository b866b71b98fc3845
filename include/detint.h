/*
 * detint.h - C ABI of libdetint, an integer-only transformer forward pass for
 * AMD Instinct MI355X (gfx950). Every op from token ids to int32 logits is
 * exact integer arithmetic, so results are bit-identical for any batch
 * composition, prefill/decode split and summation order.
 *
 * Sources (page title, section):
 *   DetLLM README ("DetLLM - Fully Deterministic LLM Inference"): intro and
 *     "Layout" (integer primitives with frozen rounding, dyadic (data, m, k)
 *     requant, the int8 GEMM as the one hardware-dispatched call, DI-Exp /
 *     DI-Softmax / DI-RMSNorm / DI-SwiGLU / integer RoPE).
 *   DetLLM blog (integer-arithmetic post), section "DetLLM": dyadic scales
 *     m/2^k with one rounding rule, shift-based nonlinears, int16 sin/cos
 *     tables, per-token activation quantisation, fixed-scale int8 KV cache,
 *     lowest-id argmax; footnote 8: 15-bit attention probabilities and P.V
 *     as two int8 GEMMs.
 *   BitExact LLM blog, "Fix the arithmetic": 16-bit fixed-point weights as
 *     integer limbs with wide accumulators; explicit rounding rules and
 *     bounds.
 *
 * Conventions for every call:
 *   - Pointers to tensors are DEVICE pointers owned by the caller; arrays are
 *     row-major and contiguous. int8 matrices that feed a GEMM need a 16-byte
 *     aligned base and a row length that is a multiple of 16.
 *   - Sizes are int64_t; no float type appears anywhere in this ABI.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Calls only enqueue work: no allocation, no synchronisation, no memset,
 *     so every call may be captured into a hipGraph.
 *   - Return value: DETINT_OK, or an error code (the call enqueued nothing);
 *     detint_last_error() gives the message. Device faults surface at the
 *     caller's next synchronisation.
 *   - Rounding rule used everywhere: R(x, s) = floor(x / 2^s + 1/2) for s >= 1
 *     (round half up via an arithmetic shift), x for s = 0, x * 2^-s for s < 0.
 *   - Per-token dynamic quantisation DQ(y) over a row: A = max |y_i|,
 *     e = max(0, bitlen(A) - 7), q_i = clamp(R(y_i, e), -127, 127).
 *   - Results are undefined (but memory-safe) where an input breaks a stated
 *     bound; the CPU oracle of this project reports such inputs as errors.
 */
#ifndef DETINT_H
#define DETINT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t detint_status;
#define DETINT_OK 0
#define DETINT_EINVAL 1        /* bad shape, null pointer, misalignment */
#define DETINT_EUNSUPPORTED 2  /* shape or configuration this build does not handle */
#define DETINT_EHIP 3          /* a HIP launch/runtime call failed */
#define DETINT_EBOUND 4        /* detint_check: an intermediate left its bound */

/* GEMM epilogue modes (DetLLM README "Layout": dyadic requant in dyadic.py). */
#define DETINT_GEMM_RAW 0      /* out int32 = acc                                   */
#define DETINT_GEMM_REQ_I8 1   /* out int8  = clamp8(R(acc*m_r*m_c, k_r + k_c))     */
#define DETINT_GEMM_FIX 2      /* out int32 = R(acc*m_r*m_c, k_r + k_c - frac)      */
#define DETINT_GEMM_RES_ADD 3  /* out int32 += R(acc*m_r*m_c, k_r + k_c - frac)     */

const char *detint_version(void);

/* Device bound checks (BitExact LLM blog, "Reproducibility has a cost":
 * range checks before residual additions, on the final logits and on the
 * linear epilogues). Kernels test their intermediates against the bounds
 * this header states and, on a violation, set a bit in a flag word of the
 * device and finish normally (the affected results are undefined, memory
 * stays safe). Bits:
 *   RESIDUAL  the residual stream left |h| < 2^25 (embedding, O-proj or
 *             down-projection residual add of a model);
 *   INT32     a FIX / logits / standalone RES_ADD result, a q/k/v fixed-point
 *             value or a rotated q/k left int32;
 *   NORM      an RMSNorm row's sum of squares reached 2^62;
 *   SWIGLU    a SwiGLU gate or up value left |x| < 2^24;
 *   ID        a token id outside [0, vocab) (its row is embedded as zeros);
 *   WEIGHT    a bf16 weight exact mode cannot hold (detint_exact_prepare);
 *   PAGE      a KV block-table entry outside the page pool (detint_forward_kv).
 * detint_check waits for `stream` (everything enqueued on it so far), then
 * reads and clears the current device's flags (set by any call on any
 * stream of that device since the last check): *flags (nullable) receives
 * them; returns DETINT_EBOUND when any is set, else DETINT_OK (DETINT_EHIP
 * if the device could not be read). It synchronises, so it is not for use
 * inside a graph capture. */
#define DETINT_BOUND_RESIDUAL 1u
#define DETINT_BOUND_INT32 2u
#define DETINT_BOUND_NORM 4u
#define DETINT_BOUND_SWIGLU 8u
#define DETINT_BOUND_ID 16u
#define DETINT_BOUND_WEIGHT 32u  /* a bf16 weight exact mode cannot hold */
#define DETINT_BOUND_PAGE 64u    /* a KV block-table entry outside the page pool */
detint_status detint_check(void *stream, uint32_t *flags);
/* Message of the last error returned on the calling thread ("" if none). */
const char *detint_last_error(void);

/* ------------------------------------------------------------------------ */
/* GEMM: acc[i][j] = sum_k A[i][k] * W[j][k], exact in int32 (DetLLM blog,
 * "DetLLM": the int8 x int8 -> int32 matmul is the one hardware-dispatched
 * function; integer accumulation is exact, so any tiling gives the same bits).
 *   A      int8 [M, K] activations.          W      int8 [N, K] weights.
 *   row_m  int32 [M], row_k int32 [M]: per-row dyadic scale (ignored in RAW).
 *   col_m  int32 [N], col_k: per-column mantissas, one shift for the tensor.
 *   frac   fractional bits of FIX / RES_ADD outputs.
 *   out    [M, N] int32 (RAW, FIX, RES_ADD; read-modify-write for RES_ADD) or
 *          int8 (REQ_I8).
 * Bounds: K <= 131056 (K * 2^14 < 2^31, so |acc| < 2^31 even when every
 * operand is -128); scaled modes |acc * m_r * m_c| < 2^62,
 * and FIX / RES_ADD results within int32. M, N >= 0; M = 0 or N = 0 is a
 * no-op.
 *   ws, ws_bytes: optional device workspace (16-byte aligned, contents need
 *   not be initialised) of detint_gemm_workspace(M, N, K, limbs) bytes; with
 *   it, shapes that give few output tiles split K over more workgroups (17-64
 *   rows: the last split to arrive sums the partials; int8 weights with more
 *   rows and fewer than 192 tiles of 128 x 64: int32 partials per split, then
 *   one summing epilogue kernel). Integer sums are order-free and stay below
 *   2^31, so the split changes no bit (DetLLM blog, "DetLLM"). NULL, 0 or a
 *   smaller size: no split. Concurrent calls need workspaces of their own. */
int64_t detint_gemm_workspace(int64_t M, int64_t N, int64_t K, int32_t limbs);
detint_status detint_gemm_i8(const int8_t *A, const int8_t *W, int64_t M, int64_t N, int64_t K,
                             const int32_t *row_m, const int32_t *row_k,
                             const int32_t *col_m, int32_t col_k, int32_t frac,
                             int32_t mode, void *out, void *ws, int64_t ws_bytes, void *stream);

/* GEMM with 16-bit fixed-point weights W16 = 256 * hi + lo held as two int8
 * planes: W_hi = W16 >> 8 (signed) and W_lo = (W16 & 255) - 128 (biased so
 * both limbs feed the signed int8 matrix units). The int64 accumulator is
 * 256 * (A.hi) + (A.lo') + 128 * rowsum(A) = A.W16 exactly (BitExact blog,
 * "Fix the arithmetic": limb partial products combined in wide accumulators).
 * Epilogue modes as above with a 128-bit product; RAW writes int64 [M, N].
 * Bound: K <= 65536. ws, ws_bytes as for detint_gemm_i8 (limbs = 1). */
detint_status detint_gemm_w16(const int8_t *A, const int8_t *W_hi, const int8_t *W_lo,
                              int64_t M, int64_t N, int64_t K,
                              const int32_t *row_m, const int32_t *row_k,
                              const int32_t *col_m, int32_t col_k, int32_t frac,
                              int32_t mode, void *out, void *ws, int64_t ws_bytes, void *stream);

/* Exact mode (BitExact LLM blog, "Three execution paths": the linear layers
 * keep their bf16 weights, multiplied with fixed-point activations; "Fix the
 * arithmetic": integer limbs, wide accumulators). A bf16 pattern (sign s,
 * exponent field E, fraction f) is (-1)^s M 2^(E' - 134) with M = 128 + f,
 * E' = E (E >= 1), or M = f, E' = 1 (E = 0). Row j of W [N, K] becomes the
 * integers W_int = (-1)^s M 2^(E' - emin_j), emin_j the smallest E' among the
 * row's nonzero entries (1 for an all-zero row), and the row scale
 * 2^row_exp[j] with row_exp[j] = emin_j - 134: w = W_int 2^row_exp exactly.
 * |W_int| < 2^31: a row may span at most 23 binary orders.
 *
 * detint_exact_prepare: W uint16 [N, K] bf16 bit patterns (device) ->
 *   planes int8 [4][N][K] (P0 = W_int >> 24, P1..P3 = its next bytes minus
 *   128; W_int = 2^24 P0 + 2^16 P1 + 2^8 P2 + P3 + 128 (2^16 + 2^8 + 1)) and
 *   row_exp int32 [N]. A weight the integers cannot hold (infinity, NaN, a
 *   wider span) sets the DETINT_BOUND_WEIGHT flag (see detint_check) and is
 *   written as 0.
 * detint_gemm_exact: acc[i][j] = sum_k A[i][k] W_int[j][k] (int64, exact;
 *   computed as 2^16 (A.H16) + A.L16 + 2^15 rowsum(A) with the two 16-bit
 *   halves on the limb GEMM), then with the activation row scale
 *   x8 m_r 2^-k_r the real output acc m_r 2^(row_exp[j] - k_r):
 *     RAW     out int64 [M, N] = acc
 *     REQ_I8  out int8  = clamp8(R(acc m_r, k_r - row_exp[j]))
 *     FIX     out int32 = R(acc m_r, k_r - row_exp[j] - frac)  (DETINT_BOUND_INT32
 *             when outside int32)
 *   A int8 [M, K] (16-byte aligned, K % 16 == 0, K <= 65536); row_m, row_k
 *   int32 [M] (ignored by RAW); ws: device workspace of
 *   detint_gemm_exact_workspace(M, N) bytes, 16-byte aligned. */
detint_status detint_exact_prepare(const uint16_t *W, int64_t N, int64_t K, int8_t *planes,
                                   int32_t *row_exp, void *stream);
int64_t detint_gemm_exact_workspace(int64_t M, int64_t N);
detint_status detint_gemm_exact(const int8_t *A, const int8_t *planes, const int32_t *row_exp,
                                int64_t M, int64_t N, int64_t K, const int32_t *row_m,
                                const int32_t *row_k, int32_t frac, int32_t mode, void *out,
                                void *ws, int64_t ws_bytes, void *stream);

/* Split int16 weights [n] into the two limb planes used by detint_gemm_w16. */
detint_status detint_split_w16(const int16_t *W16, int64_t n, int8_t *W_hi, int8_t *W_lo,
                               void *stream);

/* ------------------------------------------------------------------------ */
/* Row operations (DetLLM README "Layout", ops/). */

/* Integer RMSNorm of R rows of n (DI-RMSNorm). For each row: S = sum h_i^2,
 * c = max(0, floor((62 - bitlen(S)) / 2)), r = isqrt(floor(S * 4^c / n)),
 * T = bitlen(r) + 14, m = RD(2^T, r) (m = 2^15 -> m = 2^14, T -= 1), where
 * RD(a, b) = floor((2a + b) / 2b); (x8, e) = DQ(h_i * gain_i);
 * row_m = m, row_k = T - c + 12 - e. So x8 * row_m * 2^-row_k approximates
 * h * (gain * 2^-12) / rms(h). A zero row gives x8 = 0, scale (2^14, 26).
 *   h int32 [R, n]; gain int16 [n]; x8 int8 [R, n]; row_m, row_k int32 [R].
 *   n <= 16384. Domain: every row's S = sum h_i^2 < 2^62 and |h| < 2^31,
 *   e.g. |h| < 2^25 (the residual stream's bound) for n <= 4096, or
 *   |h| < 2^24 for n <= 16384. Outside it the row's outputs are undefined. */
detint_status detint_rmsnorm(const int32_t *h, const int16_t *gain, int64_t R, int64_t n,
                             int8_t *x8, int32_t *row_m, int32_t *row_k, void *stream);

/* DQ of each row (per-token dynamic quantisation, DetLLM blog "DetLLM"):
 *   y int32 [R, n] -> q int8 [R, n], row_e int32 [R] with y ~ q * 2^row_e. */
detint_status detint_requant(const int32_t *y, int64_t R, int64_t n, int8_t *q, int32_t *row_e,
                             void *stream);

/* Requantisation at a fixed dyadic scale, the kind the K/V cache uses (DetLLM
 * blog "DetLLM": K and V are quantised once at fixed offline scales):
 *   q[i] = clamp(R(y[i] * m, k), -127, 127) for n elements of y int32 (16-byte
 *   aligned; q 4-byte aligned), 0 <= k <= 62, |m| < 2^31. */
detint_status detint_requant_fixed(const int32_t *y, int64_t n, int32_t m, int32_t k, int8_t *q,
                                   void *stream);

/* Integer RoPE in place on x int32 [R, heads, d] with Q1.14 tables
 * cos_t/sin_t int16 [max_pos, d/2] (DetLLM blog "DetLLM": precomputed int16
 * sin/cos tables). Pairs (i, i + d/2) at position pos[r]:
 *   x_i' = R(x_i C - x_{i+d/2} S, 14), x_{i+d/2}' = R(x_{i+d/2} C + x_i S, 14).
 * d even, d <= 256; 0 <= pos[r] < max_pos; |x| < 2^31 after rotation. */
detint_status detint_rope(int32_t *x, const int32_t *pos, const int16_t *cos_t,
                          const int16_t *sin_t, int64_t R, int64_t heads, int64_t d,
                          int64_t max_pos, void *stream);

/* DI-Softmax with 15-bit probabilities (DetLLM blog footnote 8). Row r has
 * valid[r] (1 <= valid <= C) scores; mx = max of them;
 * u_j = R((s_j - mx) * mult_m, mult_k - shift[r]) (base-2 exponent, Q15);
 * E_j = DI-Exp(u_j): with v = -u_j, n = v >> 15, f = 2^15 - R(v & 32767, 1),
 * E_j = R(f, n) (0 for n > 30); D = sum E_j; Rn = floor(2^46 / D);
 * P_j = min(R(E_j * Rn, 31), 2^15 - 1); P_j = 0 for j >= valid[r].
 *   s int32 [R, C], valid/shift int32 [R], P int16 [R, C]. C <= 65536. */
detint_status detint_softmax(const int32_t *s, const int32_t *valid, const int32_t *shift,
                             int64_t R, int64_t C, int32_t mult_m, int32_t mult_k, int16_t *P,
                             void *stream);

/* DI-SwiGLU of R rows. gu int32 [R, 2n]: gate in [:, :n], up in [:, n:], both
 * with f_a fractional bits, |g|, |u| < 2^24. Integer sigmoid (Q15):
 * E = DI-Exp(-R(|g| * Mg, Kg)) with (Mg, Kg) = detint_swiglu_mult(f_a),
 * s+ = RD(2^30, 2^15 + E), s = s+ (g >= 0) or 2^15 - s+ (g < 0);
 * silu = R(g * s, 15); p = silu * u; (a8, e) = DQ(p);
 * row scale (row_m, row_k) = (2^14, 2 f_a - e + 14).
 *   a8 int8 [R, n]; row_m, row_k int32 [R]. n <= 8192. */
detint_status detint_swiglu(const int32_t *gu, int64_t R, int64_t n, int32_t f_a, int8_t *a8,
                            int32_t *row_m, int32_t *row_k, void *stream);

/* ------------------------------------------------------------------------ */
/* Attention over the int8 KV cache (DetLLM blog "DetLLM": K and V are
 * quantised once at fixed offline scales, so prefill and decode see the same
 * cached bits; footnote 8: 15-bit probabilities, P.V exact).
 * Cache layout, K and V alike: int8 [n_slots][n_kv][max_pos][d] for ONE
 * layer (pass the layer's base). Query head h reads KV head h * n_kv / n_q.
 * Query row r at absolute position p attends positions 0..p of its slot
 * (rows whose position or slot is out of range get zeros):
 *   s_j = q8 . k8_j; P = DI-Softmax(s, mult, shift = e_q[r][h]);
 *   out[r][h][t] = sum_j P_j * v8_j[t]   (int32, exact).
 *   q8 int8 [rows, n_q, d]; e_q int32 [rows, n_q]; out int32 [rows, n_q, d].
 * d in {64, 128}; n_q / n_kv in {1, 2, 4, 8}; max_pos <= 16384.          */

/* Prefill: S packed sequences; sequence s owns rows cu_seqlens[s] ..
 * cu_seqlens[s+1]-1 at positions start_pos[s] + i, cache slot slot[s]
 * (chunked prefill: positions < start_pos[s] come from earlier calls).
 * R = cu_seqlens[S] (host copy of the last entry). */
detint_status detint_attn_prefill(const int8_t *q8, const int32_t *e_q, const int8_t *k_cache,
                                  const int8_t *v_cache, int64_t n_slots, const int32_t *cu_seqlens,
                                  const int32_t *start_pos, const int32_t *slot, int64_t S,
                                  int64_t R, int64_t n_q, int64_t n_kv, int64_t d,
                                  int64_t max_pos, int32_t mult_m, int32_t mult_k,
                                  int32_t *out, void *stream);

/* Decode: B rows, row b at position ctx_len[b] - 1 of slot slot[b]. */
detint_status detint_attn_decode(const int8_t *q8, const int32_t *e_q, const int8_t *k_cache,
                                 const int8_t *v_cache, int64_t n_slots, const int32_t *ctx_len,
                                 const int32_t *slot, int64_t B, int64_t n_q, int64_t n_kv,
                                 int64_t d, int64_t max_pos, int32_t mult_m, int32_t mult_k,
                                 int32_t *out, void *stream);

/* ------------------------------------------------------------------------ */
/* Host-side set-up arithmetic (no device work; table/constant construction
 * is offline work in the pages' design, outside the forward pass). */

/* Q1.14 RoPE tables: C[p][i] = floor(2^14 cos(p * base^(-2i/d)) + 1/2), S
 * likewise with sin, for p < P, i < d/2, evaluated in float64. Host arrays. */
detint_status detint_rope_tables(int16_t *cos_t, int16_t *sin_t, int64_t P, int64_t d,
                                 int64_t base);
/* Softmax exponent multiplier (M, K): M * 2^-K ~ log2(e) / sqrt(d) * 2^15 *
 * (2^kq_k / kq_m) * 2^(-2 f_n), M in [2^14, 2^15). */
detint_status detint_softmax_mult(int32_t kq_m, int32_t kq_k, int64_t d, int32_t f_n,
                                  int32_t *M, int32_t *K);
/* SiLU exponent multiplier: M * 2^-K ~ log2(e) * 2^(15 - f_a). */
detint_status detint_swiglu_mult(int32_t f_a, int32_t *M, int32_t *K);
/* V-cache dequant scale (m, k), the dyadic inverse of the quant scale:
 * m = RD(2^29, vq_m), k = 29 - vq_k (m = 2^15 -> (2^14, 28 - vq_k)). */
detint_status detint_v_dequant(int32_t vq_m, int32_t vq_k, int32_t *m, int32_t *k);

/* ------------------------------------------------------------------------ */
/* Whole model (DetLLM README "Layout": the IntQwen3 runtime; "Usage": greedy
 * generate). The handle only records caller-owned device pointers and
 * integer constants; it copies no tensor and allocates no device memory. */

typedef struct detint_layer_desc {
  /* Linear weights [N, K]; for wide (16-bit) models w* is the high limb and
   * w*_lo the biased low limb (see detint_gemm_w16), else w*_lo is NULL.
   * wqkv rows: n_q*d query, n_kv*d key, n_kv*d value. wgu rows: ffn gate
   * then ffn up. Each *_m is the per-output-channel mantissa [N]; the shift
   * of every weight scale is the model's w_k. */
  const int8_t *wqkv, *wqkv_lo; const int32_t *wqkv_m;
  const int8_t *wo, *wo_lo;     const int32_t *wo_m;
  const int8_t *wgu, *wgu_lo;   const int32_t *wgu_m;
  const int8_t *wd, *wd_lo;     const int32_t *wd_m;
  const int16_t *attn_norm, *ffn_norm;   /* [hidden] gains, value g * 2^-12 */
  const int16_t *q_norm, *k_norm;        /* [d] gains (qk_norm models) or NULL */
  int32_t kq_m, kq_k;                    /* K-cache quant scale: k8 = clamp8(R(k * kq_m, kq_k)) */
  int32_t vq_m, vq_k;                    /* V-cache quant scale */
  /* Per-channel key rescale with the inverse on the query (DetLLM blog
   * footnote 8): device int8 [n_kv][d], each g in [0, 7], or NULL (all 0).
   * Key channel j of KV head h is cached as clamp8(R(k_j * kq_m, kq_k - g))
   * and channel j of every query head sharing h enters its DQ as R(q_j, g),
   * g = k_gain[h * d + j]: the factors 2^g and 2^-g cancel in q.k, so the
   * score scale (and the softmax multiplier) stay those of kq_m / 2^kq_k.
   * Requires kq_k >= 8. */
  const int8_t *k_gain;
} detint_layer_desc;

typedef struct detint_model_desc {
  int64_t n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab, max_pos;
  int32_t qk_norm;   /* 1: per-head RMSNorm on q and k before RoPE (Qwen3) */
  int32_t wide;      /* 1: 16-bit limbed linear weights and embedding        */
  int32_t w_k;       /* shift of every weight / embedding scale              */
  int32_t f_res;     /* fractional bits of the int32 residual stream         */
  int32_t f_n;       /* fractional bits of q/k/v before quantisation         */
  int32_t f_a;       /* fractional bits of SwiGLU gate/up                    */
  int32_t f_l;       /* fractional bits of the int32 logits                  */
  int32_t reserved;
  const int8_t *emb, *emb_lo;   /* tied embedding / lm_head [vocab, hidden]; may be
                                   NULL with vocab = 0 (layer-only models) */
  const int32_t *emb_m;         /* [vocab] mantissas                          */
  const int16_t *final_norm;    /* [hidden]                                   */
  const int16_t *rope_cos, *rope_sin;  /* device [max_pos, d/2] Q1.14 tables  */
  const detint_layer_desc *layers;     /* HOST array [n_layers], copied       */
} detint_model_desc;

typedef struct detint_model detint_model;

detint_status detint_model_create(const detint_model_desc *desc, detint_model **out);
void detint_model_destroy(detint_model *m);

/* Bytes of device workspace detint_forward needs for up to max_rows packed
 * rows in up to max_seqs sequences. */
int64_t detint_workspace_size(const detint_model *m, int64_t max_rows, int64_t max_seqs);

/* Forward pass: ids -> embedding -> n_layers decoder layers -> final RMSNorm
 * -> tied lm_head -> int32 logits of the LAST row of each sequence, and the
 * greedy next token (lowest id among the maxima; DetLLM blog "DetLLM").
 *   k_cache, v_cache: int8 [n_layers][n_slots][n_kv][max_pos][d].
 *   ids int32 [R]; cu_seqlens int32 [S+1]; start_pos, slot int32 [S]
 *   (device); R and max_seqlen are host copies (rows in total, longest
 *   sequence) used for launch sizes.
 *   logits int32 [S, vocab]: written at row (logit_row_base ? *logit_row_base
 *   : 0) + s, so a captured decode graph can append to a history buffer.
 *   next_tok int32 [S] (may alias ids for decode).
 *   flags: DETINT_FWD_ADVANCE - after the step, for every s: ids[s] =
 *   next_tok[s], start_pos[s] += 1, and *logit_row_base += S (decode only:
 *   requires R == S). Positions and lengths are read from device memory, so
 *   one captured graph serves every decode step.
 *   ws: device workspace of ws_bytes >= detint_workspace_size(m, R, S).     */
#define DETINT_FWD_ADVANCE 1
detint_status detint_forward(const detint_model *m, int8_t *k_cache, int8_t *v_cache,
                             int64_t n_slots, int32_t *ids, int64_t R,
                             const int32_t *cu_seqlens, int32_t *start_pos,
                             const int32_t *slot, int64_t S, int64_t max_seqlen,
                             int32_t *logits, int32_t *logit_row_base, int32_t *next_tok,
                             int32_t flags, void *ws, int64_t ws_bytes, void *stream);

/* A KV cache described for detint_forward_kv: either the contiguous layout
 * of detint_forward or pages through a block table (BitExact LLM blog, "What
 * the checks actually compare": KV-cache reuse, shared prefixes, preemption
 * and chunked prefill must not change a bit; the cached int8 rows are the
 * same, only their addresses differ).
 *   k, v: device int8, 16-byte aligned, caller-owned.
 *   block_table == NULL: k, v are [n_layers][n_slots][n_kv][max_pos][d]
 *     (page_size, n_pages, max_blocks ignored).
 *   block_table != NULL: device int32 [n_slots][max_blocks]; position p of
 *     slot s is row p & (page_size - 1) of page block_table[s][p / page_size]
 *     of the pools k, v = [n_layers][n_pages][n_kv][page_size][d].
 *     page_size: a power of two in [16, max_pos]; max_blocks * page_size >=
 *     max_pos; n_pages * n_kv * page_size * d < 2^31. Several slots may name
 *     the same page (a shared prefix is then stored once); a row is written
 *     by the call whose sequence reaches its position, so slots that share a
 *     page must not write it differently. Entries past a sequence's length
 *     are not read. An entry outside [0, n_pages) raises
 *     DETINT_BOUND_PAGE (see detint_check) and is read and written as page 0. */
typedef struct detint_kv_desc {
  int8_t *k, *v;
  int64_t n_slots;
  int64_t n_pages;
  int64_t page_size;
  const int32_t *block_table;
  int64_t max_blocks;
} detint_kv_desc;

/* Bytes of each of k and v the descriptor addresses (-1 if it is invalid
 * for the model). */
int64_t detint_kv_bytes(const detint_model *m, const detint_kv_desc *kv);

/* detint_forward over a described (contiguous or paged) KV cache; every other
 * argument as in detint_forward. */
detint_status detint_forward_kv(const detint_model *m, const detint_kv_desc *kv, int32_t *ids,
                                int64_t R, const int32_t *cu_seqlens, int32_t *start_pos,
                                const int32_t *slot, int64_t S, int64_t max_seqlen,
                                int32_t *logits, int32_t *logit_row_base, int32_t *next_tok,
                                int32_t flags, void *ws, int64_t ws_bytes, void *stream);

/* Tied lm_head for up to 16 rows, as one kernel: logits int32 [S, V] =
 * R(x8 . E^T * row_m * emb_m, row_k + w_k - f_l), plus for every row the
 * partial greedy-argmax keys of each of the kernel's waves in
 * part int64 [S, detint_lm_head_parts(V)] (key = logit * 2^32 + 2^32 - 1 - id:
 * the largest key is the largest logit at the lowest id). x8 [S, H] int8;
 * E = emb [V, H] int8, or 16-bit limbs emb/emb_lo as in detint_gemm_w16.
 * DetLLM README intro: int32 logits; DetLLM blog "DetLLM": ties go to the
 * smallest token id. */
int64_t detint_lm_head_parts(int64_t V);
detint_status detint_lm_head(const int8_t *x8, const int8_t *emb, const int8_t *emb_lo, int64_t S,
                             int64_t V, int64_t H, const int32_t *row_m, const int32_t *row_k,
                             const int32_t *emb_m, int32_t w_k, int32_t f_l, int32_t *logits,
                             int64_t *part, void *stream);
/* Greedy token of each row from detint_lm_head's partials: next_tok int32 [S]. */
detint_status detint_argmax_parts(const int64_t *part, int64_t S, int64_t nparts,
                                  int32_t *next_tok, void *stream);

/* Integer temperature / top-k / top-p sampling of R rows of int32 logits [R, V]
 * (BitExact blog intro: sampling rules in integer arithmetic; DetLLM blog,
 * limits: integer sampling left open; the pages give no formula). Per row:
 * keep the top_k highest-ranked ids, ranked by larger logit first and, among
 * equal logits, lower id first (top_k <= 0 or >= V keeps all); weight kept id
 * j by E_j = DI-Exp(R((l_j - l_max) * t_m, t_k)) (the softmax's exponential:
 * t_m / 2^t_k is log2(e) / (2^(f_l - 15) T) for temperature T and logits with
 * f_l fractional bits); top-p then keeps the shortest prefix of the ranking
 * whose weight reaches P = ceil(top_p * D_k / 2^16), D_k the weight of the
 * top-k ids (top_p = p in units of 2^-16, 1..65536; 65536 keeps all); D = sum
 * of the kept E_j; with the caller's uniform draw r,
 * t = floor(r * D / 2^32); tokens[row] = the smallest id j with
 * E_0 + ... + E_j > t. top_k = 1 gives the greedy token for every draw.
 *   logits int32 [R, V], device; draws uint32 [R], device (the randomness is
 *   the caller's: any generator, so a stream of draws replays exactly);
 *   tokens int32 [R], device. 1 <= V <= 262144, 1 <= t_m < 2^24, 0 <= t_k <= 62.
 *   ws: optional device workspace (16-byte aligned) of ws_bytes >=
 *   detint_sample_workspace(R, V), owned by the caller, contents need not be
 *   initialised (under R * 136 KiB for V <= 262144). With it, work spreads
 *   over slices of the row across the GPU:
 *   - every id kept, top-p off: 1024-id slices;
 *   - top-k (with or without top-p) where the 2048-id slices give at most
 *     8192 candidates, ceil(V / 2048) * min(k, 2048) <= 8192: each slice
 *     selects its top ids first;
 *   - top-p alone: each 2048-id slice offers its top min(2048, 16384 /
 *     ceil(V / 2048)) ids; a row whose nucleus reaches below what a slice
 *     offered is sampled by the one-workgroup algorithm in the same kernel.
 *   Other calls, ws = NULL, or ws_bytes below the size above, take one
 *   workgroup per row. Same tokens either way. Calls that may run at the
 *   same time (other streams) need workspaces of their own. */
int64_t detint_sample_workspace(int64_t R, int64_t V);
detint_status detint_sample(const int32_t *logits, int64_t R, int64_t V, int64_t top_k,
                            int32_t top_p, int32_t t_m, int32_t t_k, const uint32_t *draws,
                            int32_t *tokens, void *ws, int64_t ws_bytes, void *stream);

/* The model's last step for S rows of the int32 residual h [S, H]: final
 * RMSNorm with gain int16 [H] (scale 2^-12), tied lm_head logits int32
 * [S, V] = R(x8 . E^T * m_r * emb_m, k_r + w_k - f_l), and the greedy token
 * next_tok int32 [S] (lowest id among maxima). E is emb [V, H] int8, or
 * 16-bit limbs emb/emb_lo as in detint_gemm_w16. For S <= 8 rows of int8
 * weights (H <= 8192) it is the decode step's single streaming kernel (norm in
 * its prologue, logits and per-wave argmax keys in its epilogue) plus one
 * reduction; otherwise RMSNorm, lm_head and argmax run as separate launches.
 * next_tok may be NULL: logits only (one launch on the fused path).
 * ws: device scratch of detint_final_head_workspace(S, V, H) bytes.
 * DetLLM README intro: int32 logits; DetLLM blog "DetLLM": DI-RMSNorm and
 * the lowest-id tie rule. */
int64_t detint_final_head_workspace(int64_t S, int64_t V, int64_t H);
detint_status detint_final_head(const int32_t *h, int64_t S, int64_t H, const int16_t *gain,
                                const int8_t *emb, const int8_t *emb_lo, const int32_t *emb_m,
                                int64_t V, int32_t w_k, int32_t f_l, int32_t *logits,
                                int32_t *next_tok, void *ws, int64_t ws_bytes, void *stream);

/* detint_final_head for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and arguments, without a workspace. Its
 * scratch is a fixed DETINT_NOALLOC_SCRATCH_BYTES array in the library's
 * device storage, one per GPU, held until the process ends; the call
 * allocates nothing. It returns DETINT_EINVAL when
 * detint_final_head_workspace(S, V, H) exceeds that size (e.g. up to 16 rows
 * fit for V <= 262144, H <= 8192). Every call on one GPU shares that GPU's
 * scratch: calls that may overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. */
#define DETINT_NOALLOC_SCRATCH_BYTES (4 << 20)
detint_status detint_final_head_noalloc(const int32_t *h, int64_t S, int64_t H,
                                        const int16_t *gain, const int8_t *emb,
                                        const int8_t *emb_lo, const int32_t *emb_m, int64_t V,
                                        int32_t w_k, int32_t f_l, int32_t *logits,
                                        int32_t *next_tok, void *stream);

/* One decoder layer in place on the int32 residual h [R, hidden] (|h| <
 * 2^25), same sequence/cache arguments and workspace as detint_forward:
 * RMSNorm -> QKV -> (q/k-norm) -> RoPE -> q DQ, K/V into the cache ->
 * attention -> DQ -> O-proj + residual -> RMSNorm -> gate/up -> DI-SwiGLU ->
 * down + residual (DetLLM README "Layout"; DetLLM blog "DetLLM"). Works on
 * models without a vocabulary (vocab = 0). */
detint_status detint_layer_forward(const detint_model *m, int64_t layer, int32_t *h,
                                   int8_t *k_cache, int8_t *v_cache, int64_t n_slots, int64_t R,
                                   const int32_t *cu_seqlens, const int32_t *start_pos,
                                   const int32_t *slot, int64_t S, int64_t max_seqlen, void *ws,
                                   int64_t ws_bytes, void *stream);

/* Measurement, not part of the forward pass: runs `rounds` device-wide
 * barriers between 256 resident workgroups (one per CU) on `stream`, each
 * round exchanging a 64-int row per workgroup, so that the barrier's cost
 * (kernel time / rounds) can be set against a graph node per decode phase.
 * mode 0: per-workgroup generation flags, release store and acquire fence;
 * 1: one arrival counter (release RMW); 2: two levels of flags (8 groups,
 * then their leaders); 3: mode 0's flags with relaxed stores and no fences
 * (a hardware lower bound, not a barrier the memory model guarantees).
 * Every wait is bounded: when one runs out of polls its workgroup returns.
 * When `result` is non-null the call waits for the stream and writes the
 * run's failure bits (1: a wait ran out, 2: a row read back wrong).
 * DETINT_EUNSUPPORTED on a device with fewer than 256 CUs. */
detint_status detint_probe_barrier(int32_t mode, int32_t rounds, uint32_t *result, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DETINT_H */
