// C ABI of libdetint (declared in include/detint.h): argument checks, the
// host-side set-up arithmetic, the model handle, and the forward pass as a
// sequence of kernel launches on the caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "detint.h"
#include "internal.h"

using namespace detint;

namespace detint {

hipError_t set_max_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, hipError_t> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel);
  const auto it = done.find(key);
  if (it != done.end()) return it->second;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  done[key] = e;
  return e;
}

}  // namespace detint

namespace {

thread_local std::string g_err;

detint_status fail(detint_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

detint_status ok() {
  g_err.clear();
  return DETINT_OK;
}

detint_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DETINT_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

hipStream_t S_(void* s) { return (hipStream_t)s; }

#define REQUIRE(cond, ...)                               \
  do {                                                   \
    if (!(cond)) return fail(DETINT_EINVAL, __VA_ARGS__); \
  } while (0)

detint_status check_gemm(const int8_t* A, const int8_t* W, int64_t M, int64_t N, int64_t K,
                         const int32_t* row_m, const int32_t* row_k, const int32_t* col_m,
                         int32_t mode, const void* out, int64_t kmax) {
  REQUIRE(M >= 0 && N >= 0 && K > 0, "gemm: bad shape M=%lld N=%lld K=%lld", (long long)M,
          (long long)N, (long long)K);
  REQUIRE(K % 16 == 0, "gemm: K=%lld must be a multiple of 16", (long long)K);
  REQUIRE(K <= kmax, "gemm: K=%lld exceeds %lld (int32 accumulator bound)", (long long)K,
          (long long)kmax);
  REQUIRE(M <= (int64_t)1 << 30 && N <= (int64_t)1 << 30, "gemm: M or N too large");
  REQUIRE(mode >= DETINT_GEMM_RAW && mode <= DETINT_GEMM_RES_ADD, "gemm: bad mode %d", mode);
  if (M == 0 || N == 0) return ok();
  REQUIRE(A && W && out, "gemm: null pointer");
  REQUIRE(aligned16(A) && aligned16(W), "gemm: A and W must be 16-byte aligned");
  if (mode != DETINT_GEMM_RAW) REQUIRE(row_m && row_k && col_m, "gemm: null scale pointer");
  return ok();
}

}  // namespace

extern "C" {

const char* detint_version(void) { return "libdetint 0.1 gfx950"; }
const char* detint_last_error(void) { return g_err.c_str(); }

detint_status detint_check(void* stream, uint32_t* flags) {
  uint32_t f = 0;
  hipError_t e = bound_flags_gemm(&f, S_(stream));
  if (e == hipSuccess) e = bound_flags_decode(&f, S_(stream));
  if (e == hipSuccess) e = bound_flags_rowops(&f, S_(stream));
  if (e == hipSuccess) e = bound_flags_attention(&f, S_(stream));
  if (flags) *flags = f;
  if (e != hipSuccess) return hip_status(e, "check: reading the bound flags");
  if (f)
    return fail(DETINT_EBOUND, "check: bound flags 0x%x (residual %d, int32 %d, norm %d, "
                "swiglu %d, id %d)", f, !!(f & DETINT_BOUND_RESIDUAL), !!(f & DETINT_BOUND_INT32),
                !!(f & DETINT_BOUND_NORM), !!(f & DETINT_BOUND_SWIGLU), !!(f & DETINT_BOUND_ID));
  return ok();
}

// ------------------------------------------------------------------- GEMMs

int64_t detint_gemm_workspace(int64_t M, int64_t N, int64_t K, int32_t limbs) {
  if (M < 0 || N < 0 || K < 0) return -1;
  return gemm_workspace_bytes(M, N, K, limbs != 0);
}

// Split-K workspace of a standalone GEMM: the skinny kernel's arrival
// counters (cleared by a kernel first), then the partials.
static detint_status gemm_with_ws(const int8_t* A, const int8_t* W, const int8_t* W_lo, int64_t M,
                                  int64_t N, int64_t K, const Epi& e, void* out, void* ws,
                                  int64_t ws_bytes, hipStream_t st, const char* what) {
  const int64_t need = gemm_workspace_bytes(M, N, K, W_lo != nullptr);
  if (!ws || need == 0 || ws_bytes < need)
    return hip_status(launch_gemm(A, W, W_lo, M, N, K, e, out, st), what);
  REQUIRE(aligned16(ws), "%s: workspace must be 16-byte aligned", what);
  const int64_t tiles = (N + 31) / 32;
  const int64_t cnt_bytes = ((4 * tiles + 255) / 256) * 256;
  SplitWs sp{(int32_t*)((char*)ws + cnt_bytes), (int32_t*)ws, kSplitPairsStandalone, tiles,
             (ws_bytes - cnt_bytes) / 4};
  if (gemm_takes_skinny(M, N, K, W_lo != nullptr)) {
    const hipError_t z = launch_zero_i32(sp.cnt, tiles, st);
    if (z != hipSuccess) return hip_status(z, what);
  }
  return hip_status(launch_gemm(A, W, W_lo, M, N, K, e, out, st, &sp), what);
}

detint_status detint_gemm_i8(const int8_t* A, const int8_t* W, int64_t M, int64_t N, int64_t K,
                             const int32_t* row_m, const int32_t* row_k, const int32_t* col_m,
                             int32_t col_k, int32_t frac, int32_t mode, void* out, void* ws,
                             int64_t ws_bytes, void* stream) {
  // K * 2^14 < 2^31 even when every operand is -128
  detint_status s = check_gemm(A, W, M, N, K, row_m, row_k, col_m, mode, out, 131056);
  if (s != DETINT_OK || M == 0 || N == 0) return s;
  Epi e{row_m, row_k, col_m, col_k, frac, mode, nullptr};
  return gemm_with_ws(A, W, nullptr, M, N, K, e, out, ws, ws_bytes, S_(stream), "gemm_i8 launch");
}

detint_status detint_gemm_w16(const int8_t* A, const int8_t* W_hi, const int8_t* W_lo, int64_t M,
                              int64_t N, int64_t K, const int32_t* row_m, const int32_t* row_k,
                              const int32_t* col_m, int32_t col_k, int32_t frac, int32_t mode,
                              void* out, void* ws, int64_t ws_bytes, void* stream) {
  detint_status s = check_gemm(A, W_hi, M, N, K, row_m, row_k, col_m, mode, out, 65536);
  if (s != DETINT_OK || M == 0 || N == 0) return s;
  REQUIRE(W_lo && aligned16(W_lo), "gemm_w16: W_lo null or misaligned");
  Epi e{row_m, row_k, col_m, col_k, frac, mode, nullptr};
  return gemm_with_ws(A, W_hi, W_lo, M, N, K, e, out, ws, ws_bytes, S_(stream), "gemm_w16 launch");
}

detint_status detint_exact_prepare(const uint16_t* W, int64_t N, int64_t K, int8_t* planes,
                                   int32_t* row_exp, void* stream) {
  REQUIRE(N >= 0 && K > 0 && N * K < ((int64_t)1 << 40), "exact_prepare: bad shape");
  if (N == 0) return ok();
  REQUIRE(W && planes && row_exp, "exact_prepare: null pointer");
  return hip_status(launch_exact_prepare(W, N, K, planes, row_exp, S_(stream)),
                    "exact_prepare launch");
}

int64_t detint_gemm_exact_workspace(int64_t M, int64_t N) {
  if (M < 0 || N < 0) return -1;
  return 8 * (2 * M * N + M) + 256;
}

detint_status detint_gemm_exact(const int8_t* A, const int8_t* planes, const int32_t* row_exp,
                                int64_t M, int64_t N, int64_t K, const int32_t* row_m,
                                const int32_t* row_k, int32_t frac, int32_t mode, void* out,
                                void* ws, int64_t ws_bytes, void* stream) {
  REQUIRE(mode == DETINT_GEMM_RAW || mode == DETINT_GEMM_REQ_I8 || mode == DETINT_GEMM_FIX,
          "gemm_exact: mode must be RAW, REQ_I8 or FIX");
  detint_status s = check_gemm(A, planes, M, N, K, row_m, row_k, row_exp, mode, out, 65536);
  if (s != DETINT_OK || M == 0 || N == 0) return s;
  REQUIRE(M < ((int64_t)1 << 31) && N < ((int64_t)1 << 31) && M * N < ((int64_t)1 << 40),
          "gemm_exact: M or N too large");
  REQUIRE(row_exp, "gemm_exact: null row_exp");
  REQUIRE(ws && aligned16(ws) && ws_bytes >= detint_gemm_exact_workspace(M, N),
          "gemm_exact: workspace of %lld bytes needed", (long long)detint_gemm_exact_workspace(M, N));
  REQUIRE(aligned16(planes + N * K), "gemm_exact: N * K must keep the planes 16-byte aligned");
  return hip_status(launch_gemm_exact(A, planes, row_exp, M, N, K, row_m, row_k, frac, mode, out,
                                      (int64_t*)ws, S_(stream)),
                    "gemm_exact launch");
}

detint_status detint_split_w16(const int16_t* W16, int64_t n, int8_t* W_hi, int8_t* W_lo,
                               void* stream) {
  REQUIRE(n >= 0, "split_w16: n < 0");
  if (n == 0) return ok();
  REQUIRE(W16 && W_hi && W_lo, "split_w16: null pointer");
  return hip_status(launch_split_w16(W16, n, W_hi, W_lo, S_(stream)), "split_w16 launch");
}

// ---------------------------------------------------------------- row ops

detint_status detint_rmsnorm(const int32_t* h, const int16_t* gain, int64_t R, int64_t n,
                             int8_t* x8, int32_t* row_m, int32_t* row_k, void* stream) {
  REQUIRE(R >= 0 && n > 0 && n <= 16384, "rmsnorm: bad shape R=%lld n=%lld", (long long)R,
          (long long)n);
  if (R == 0) return ok();
  REQUIRE(h && gain && x8 && row_m && row_k, "rmsnorm: null pointer");
  return hip_status(launch_rmsnorm(h, nullptr, gain, R, n, x8, row_m, row_k, S_(stream)),
                    "rmsnorm launch");
}

detint_status detint_requant(const int32_t* y, int64_t R, int64_t n, int8_t* q, int32_t* row_e,
                             void* stream) {
  REQUIRE(R >= 0 && n > 0 && n <= (int64_t)1 << 24, "requant: bad shape");
  if (R == 0) return ok();
  REQUIRE(y && q && row_e, "requant: null pointer");
  return hip_status(launch_requant(y, R, n, q, row_e, nullptr, nullptr, 0, 0, S_(stream)),
                    "requant launch");
}

detint_status detint_requant_fixed(const int32_t* y, int64_t n, int32_t m, int32_t k, int8_t* q,
                                   void* stream) {
  REQUIRE(n >= 0 && k >= 0 && k <= 62, "requant_fixed: bad n or shift");
  if (n == 0) return ok();
  REQUIRE(y && q && aligned16(y) && ((uintptr_t)q & 3) == 0, "requant_fixed: null or misaligned");
  return hip_status(launch_requant_fixed(y, n, m, k, q, S_(stream)), "requant_fixed launch");
}

detint_status detint_rope(int32_t* x, const int32_t* pos, const int16_t* cos_t,
                          const int16_t* sin_t, int64_t R, int64_t heads, int64_t d,
                          int64_t max_pos, void* stream) {
  REQUIRE(R >= 0 && heads >= 0 && d > 0 && d % 2 == 0 && d <= 256 && max_pos > 0,
          "rope: bad shape");
  if (R == 0 || heads == 0) return ok();
  REQUIRE(x && pos && cos_t && sin_t, "rope: null pointer");
  return hip_status(launch_rope(x, pos, cos_t, sin_t, R, heads, d, max_pos, S_(stream)),
                    "rope launch");
}

detint_status detint_softmax(const int32_t* s, const int32_t* valid, const int32_t* shift,
                             int64_t R, int64_t C, int32_t mult_m, int32_t mult_k, int16_t* P,
                             void* stream) {
  REQUIRE(R >= 0 && C > 0 && C <= 65536, "softmax: bad shape");
  if (R == 0) return ok();
  REQUIRE(s && valid && shift && P, "softmax: null pointer");
  REQUIRE(mult_m > 0 && mult_m < (1 << 16), "softmax: mult_m out of range");
  return hip_status(launch_softmax(s, valid, shift, R, C, mult_m, mult_k, P, S_(stream)),
                    "softmax launch");
}

detint_status detint_swiglu(const int32_t* gu, int64_t R, int64_t n, int32_t f_a, int8_t* a8,
                            int32_t* row_m, int32_t* row_k, void* stream) {
  REQUIRE(R >= 0 && n > 0 && n <= 8192 && f_a >= 0 && f_a <= 24, "swiglu: bad shape (n <= 8192)");
  if (R == 0) return ok();
  REQUIRE(gu && a8 && row_m && row_k, "swiglu: null pointer");
  int32_t Mg, Kg;
  detint_swiglu_mult(f_a, &Mg, &Kg);
  return hip_status(launch_swiglu(gu, R, n, f_a, Mg, Kg, a8, row_m, row_k, S_(stream)),
                    "swiglu launch");
}

// -------------------------------------------------------------- attention

static detint_status check_attn(const int8_t* q8, const int32_t* e_q, const int8_t* kc,
                                const int8_t* vc, int64_t nq, int64_t nkv, int64_t d,
                                int64_t max_pos, const int32_t* out) {
  REQUIRE(nq > 0 && nkv > 0 && nq % nkv == 0, "attention: n_q must be a multiple of n_kv");
  REQUIRE(max_pos > 0 && max_pos <= 16384, "attention: max_pos out of range");
  if (!attention_supported(d, nq / nkv, max_pos))
    return fail(DETINT_EUNSUPPORTED, "attention: unsupported d=%lld group=%lld max_pos=%lld",
                (long long)d, (long long)(nq / nkv), (long long)max_pos);
  REQUIRE(q8 && e_q && kc && vc && out, "attention: null pointer");
  REQUIRE(aligned16(q8) && aligned16(kc) && aligned16(vc), "attention: q8/cache misaligned");
  return ok();
}

detint_status detint_attn_prefill(const int8_t* q8, const int32_t* e_q, const int8_t* k_cache,
                                  const int8_t* v_cache, int64_t n_slots, const int32_t* cu_seqlens,
                                  const int32_t* start_pos, const int32_t* slot, int64_t S,
                                  int64_t R, int64_t n_q, int64_t n_kv, int64_t d,
                                  int64_t max_pos, int32_t mult_m, int32_t mult_k, int32_t* out,
                                  void* stream) {
  REQUIRE(S >= 0 && R >= 0, "attn_prefill: bad sizes");
  if (R == 0) return ok();
  REQUIRE(S > 0 && cu_seqlens && start_pos && slot, "attn_prefill: null sequence arrays");
  detint_status s = check_attn(q8, e_q, k_cache, v_cache, n_q, n_kv, d, max_pos, out);
  if (s != DETINT_OK) return s;
  REQUIRE(n_slots > 0, "attn_prefill: n_slots must be positive");
  RowMap rows{cu_seqlens, start_pos, slot, (int32_t)S, nullptr, 0, nullptr};
  // R bounds the longest sequence
  return hip_status(launch_attention_seqs(q8, e_q, k_cache, v_cache, rows, R, R, n_q, n_kv, d,
                                          n_slots, max_pos, mult_m, mult_k, out, S_(stream)),
                    "attn_prefill launch");
}

detint_status detint_attn_decode(const int8_t* q8, const int32_t* e_q, const int8_t* k_cache,
                                 const int8_t* v_cache, int64_t n_slots, const int32_t* ctx_len,
                                 const int32_t* slot, int64_t B, int64_t n_q, int64_t n_kv,
                                 int64_t d, int64_t max_pos, int32_t mult_m, int32_t mult_k,
                                 int32_t* out, void* stream) {
  REQUIRE(B >= 0, "attn_decode: bad sizes");
  if (B == 0) return ok();
  REQUIRE(ctx_len && slot, "attn_decode: null ctx_len/slot");
  detint_status s = check_attn(q8, e_q, k_cache, v_cache, n_q, n_kv, d, max_pos, out);
  if (s != DETINT_OK) return s;
  REQUIRE(n_slots > 0, "attn_decode: n_slots must be positive");
  RowMap rows{nullptr, nullptr, nullptr, 0, ctx_len, -1, slot};
  return hip_status(launch_attention(q8, e_q, k_cache, v_cache, rows, B, n_q, n_kv, d, n_slots,
                                     max_pos, mult_m, mult_k, out, S_(stream)),
                    "attn_decode launch");
}

// ------------------------------------------------------------- lm_head

constexpr int64_t kArgmaxParts = 64;

int64_t detint_lm_head_parts(int64_t V) { return V > 0 ? logits_argmax_parts(V) : 0; }

detint_status detint_lm_head(const int8_t* x8, const int8_t* emb, const int8_t* emb_lo, int64_t S,
                             int64_t V, int64_t H, const int32_t* row_m, const int32_t* row_k,
                             const int32_t* emb_m, int32_t w_k, int32_t f_l, int32_t* logits,
                             int64_t* part, void* stream) {
  detint_status s = check_gemm(x8, emb, S, V, H, row_m, row_k, emb_m, DETINT_GEMM_FIX, logits,
                               emb_lo ? 65536 : 131056);
  if (s != DETINT_OK || S == 0 || V == 0) return s;
  REQUIRE(S <= 16, "lm_head: at most 16 rows (S=%lld)", (long long)S);
  REQUIRE(part, "lm_head: null partials");
  if (emb_lo) REQUIRE(aligned16(emb_lo), "lm_head: emb_lo misaligned");
  Epi e{row_m, row_k, emb_m, w_k, f_l, MODE_FIX, nullptr};
  return hip_status(launch_logits_argmax(x8, emb, emb_lo, S, V, H, e, logits, part, S_(stream)),
                    "lm_head launch");
}

static int64_t final_head_parts(int64_t S, int64_t V) {
  int64_t np = logits_argmax_parts(V);
  if (fused_decode_parts(V, S) > np) np = fused_decode_parts(V, S);
  if (kArgmaxParts > np) np = kArgmaxParts;
  return S * np;
}

int64_t detint_final_head_workspace(int64_t S, int64_t V, int64_t H) {
  if (S < 0 || V < 0 || H < 0) return -1;
  const int64_t a = 8 * final_head_parts(S, V > 0 ? V : 1);
  const int64_t b = ((S * H + 255) / 256) * 256;
  return a + b + 8 * S + 256;
}

detint_status detint_final_head(const int32_t* h, int64_t S, int64_t H, const int16_t* gain,
                                const int8_t* emb, const int8_t* emb_lo, const int32_t* emb_m,
                                int64_t V, int32_t w_k, int32_t f_l, int32_t* logits,
                                int32_t* next_tok, void* ws, int64_t ws_bytes, void* stream) {
  REQUIRE(S >= 0 && H > 0 && V >= 0, "final_head: bad sizes");
  if (S == 0 || V == 0) return ok();
  REQUIRE(h && gain && emb && emb_m && logits && ws, "final_head: null pointer");
  REQUIRE(H % 16 == 0 && aligned16(emb) && (!emb_lo || aligned16(emb_lo)),
          "final_head: hidden must be a multiple of 16 with 16-byte aligned tables");
  REQUIRE(H <= (emb_lo ? 65536 : 131056), "final_head: hidden too large");
  REQUIRE(ws_bytes >= detint_final_head_workspace(S, V, H), "final_head: workspace too small");
  hipStream_t st = S_(stream);
  int64_t* part = (int64_t*)ws;
  int8_t* x8 = (int8_t*)ws + 8 * final_head_parts(S, V);
  int32_t* rm = (int32_t*)(x8 + ((S * H + 255) / 256) * 256);
  int32_t* rk = rm + S;
  hipError_t e;
  if (!emb_lo && fused_decode_supported(S, H)) {
    // the decode step's kernel: RMSNorm prologue, logits, argmax partials
    e = launch_fused_lm_head(h, nullptr, gain, emb, emb_m, w_k, f_l, S, V, H, logits, nullptr, part, st);
    if (e != hipSuccess || !next_tok) return hip_status(e, "final_head fused launch");
    return hip_status(launch_argmax_final(part, S, fused_decode_parts(V, S), next_tok, st),
                      "final_head argmax");
  }
  e = launch_rmsnorm(h, nullptr, gain, S, H, x8, rm, rk, st);
  if (e != hipSuccess) return hip_status(e, "final_head rmsnorm");
  Epi ep{rm, rk, emb_m, w_k, f_l, MODE_FIX, nullptr};
  if (S <= 16) {
    e = launch_logits_argmax(x8, emb, emb_lo, S, V, H, ep, logits, part, st);
    if (e != hipSuccess || !next_tok) return hip_status(e, "final_head lm_head");
    return hip_status(launch_argmax_final(part, S, logits_argmax_parts(V), next_tok, st),
                      "final_head argmax");
  }
  e = launch_gemm(x8, emb, emb_lo, S, V, H, ep, logits, st);
  if (e != hipSuccess || !next_tok) return hip_status(e, "final_head lm_head");
  return hip_status(launch_argmax(logits, nullptr, S, V, part, kArgmaxParts, next_tok, st),
                    "final_head argmax");
}

// ------------------------------------------------ allocation-free final head

// Scratch of detint_final_head_noalloc: file-scope device storage, one copy
// on every GPU the library runs on, held until the process ends. Host code
// never uses this name as an address: each device's address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) char scratch[DETINT_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// This device's address of `scratch` (looked up on the first call per device).
detint_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "final_head_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DETINT_EUNSUPPORTED, "final_head_noalloc: device %d beyond %d", dev, kMaxDevices);
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess || !s.ptr)
    return hip_status(s.err != hipSuccess ? s.err : hipErrorInvalidSymbol,
                      "final_head_noalloc: hipGetSymbolAddress(scratch)");
  *ptr = s.ptr;
  return ok();
}
}  // namespace

detint_status detint_final_head_noalloc(const int32_t* h, int64_t S, int64_t H,
                                        const int16_t* gain, const int8_t* emb,
                                        const int8_t* emb_lo, const int32_t* emb_m, int64_t V,
                                        int32_t w_k, int32_t f_l, int32_t* logits,
                                        int32_t* next_tok, void* stream) {
  REQUIRE(S >= 0 && H > 0 && V >= 0, "final_head_noalloc: bad sizes");
  if (S == 0 || V == 0) return ok();
  const int64_t need = detint_final_head_workspace(S, V, H);
  if (need < 0 || need > DETINT_NOALLOC_SCRATCH_BYTES)
    return fail(DETINT_EINVAL,
                "final_head_noalloc: S=%lld V=%lld H=%lld needs %lld scratch bytes, more than "
                "the %lld held per device (use detint_final_head with a workspace)",
                (long long)S, (long long)V, (long long)H, (long long)need,
                (long long)DETINT_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const detint_status st = scratch_of_current_device(&ws);
  if (st != DETINT_OK) return st;
  // every kernel of the final head writes the scratch it later reads (argmax
  // partials for all parts, the normalised rows and their scales), so
  // nothing needs clearing between calls
  return detint_final_head(h, S, H, gain, emb, emb_lo, emb_m, V, w_k, f_l, logits, next_tok, ws,
                           DETINT_NOALLOC_SCRATCH_BYTES, stream);
}

detint_status detint_argmax_parts(const int64_t* part, int64_t S, int64_t nparts,
                                  int32_t* next_tok, void* stream) {
  REQUIRE(S >= 0 && nparts > 0, "argmax_parts: bad sizes");
  if (S == 0) return ok();
  REQUIRE(part && next_tok, "argmax_parts: null pointer");
  return hip_status(launch_argmax_final(part, S, nparts, next_tok, S_(stream)),
                    "argmax_parts launch");
}

int64_t detint_sample_workspace(int64_t R, int64_t V) {
  if (R < 0 || V < 1 || V > 262144) return -1;
  return sample_workspace_bytes(R, V);
}

detint_status detint_sample(const int32_t* logits, int64_t R, int64_t V, int64_t top_k,
                            int32_t top_p, int32_t t_m, int32_t t_k, const uint32_t* draws,
                            int32_t* tokens, void* ws, int64_t ws_bytes, void* stream) {
  REQUIRE(R >= 0 && V >= 1 && V <= 262144, "sample: V must be in [1, 262144]");
  REQUIRE(t_m >= 1 && t_m < (1 << 24) && t_k >= 0 && t_k <= 62, "sample: t_m or t_k out of range");
  REQUIRE(top_p >= 1 && top_p <= 65536, "sample: top_p must be in [1, 65536]");
  if (R == 0) return ok();
  REQUIRE(logits && draws && tokens, "sample: null pointer");
  const int64_t keep = (top_k <= 0 || top_k >= V) ? V : top_k;
  REQUIRE(ws_bytes >= 0 && (!ws || aligned16(ws)), "sample: workspace misaligned");
  return hip_status(launch_sample(logits, R, V, keep, top_p, t_m, t_k, draws, tokens, ws, ws_bytes,
                                  S_(stream)),
                    "sample launch");
}

// ------------------------------------------------------ host set-up arithmetic

detint_status detint_rope_tables(int16_t* cos_t, int16_t* sin_t, int64_t P, int64_t d,
                                 int64_t base) {
  REQUIRE(cos_t && sin_t && P > 0 && d > 0 && d % 2 == 0 && base > 1, "rope_tables: bad args");
  const int64_t half = d / 2;
  for (int64_t i = 0; i < half; ++i) {
    const double theta = std::pow((double)base, -(double)(2 * i) / (double)d);
    for (int64_t p = 0; p < P; ++p) {
      const double a = (double)p * theta;
      cos_t[p * half + i] = (int16_t)std::floor(16384.0 * std::cos(a) + 0.5);
      sin_t[p * half + i] = (int16_t)std::floor(16384.0 * std::sin(a) + 0.5);
    }
  }
  return ok();
}

// A positive real as (m, k) with m in [2^14, 2^15) and m * 2^-k nearest.
static void to_dyadic(double x, int32_t* M, int32_t* K) {
  int ex = 0;
  const double f = std::frexp(x, &ex);  // x = f * 2^ex, f in [0.5, 1)
  long long m = (long long)std::floor(std::ldexp(f, 15) + 0.5);
  int k = 15 - ex;
  if (m == 32768) {
    m = 16384;
    --k;
  }
  *M = (int32_t)m;
  *K = k;
}

detint_status detint_softmax_mult(int32_t kq_m, int32_t kq_k, int64_t d, int32_t f_n,
                                  int32_t* M, int32_t* K) {
  REQUIRE(M && K && kq_m > 0 && d > 0, "softmax_mult: bad args");
  const double log2e = 1.4426950408889634;
  to_dyadic(std::ldexp(log2e, 15 + kq_k - 2 * f_n) / ((double)kq_m * std::sqrt((double)d)), M, K);
  return ok();
}

detint_status detint_swiglu_mult(int32_t f_a, int32_t* M, int32_t* K) {
  REQUIRE(M && K, "swiglu_mult: null");
  to_dyadic(std::ldexp(1.4426950408889634, 15 - f_a), M, K);
  return ok();
}

detint_status detint_v_dequant(int32_t vq_m, int32_t vq_k, int32_t* m, int32_t* k) {
  REQUIRE(m && k && vq_m > 0, "v_dequant: bad args");
  const long long a = 1LL << 29;
  long long q = (2 * a + vq_m) / (2LL * vq_m);  // RD(2^29, vq_m)
  int kk = 29 - vq_k;
  if (q == 32768) {
    q = 16384;
    --kk;
  }
  *m = (int32_t)q;
  *k = kk;
  return ok();
}

}  // extern "C"

// ------------------------------------------------------------------ model

struct detint_model {
  detint_model_desc d;
  std::vector<detint_layer_desc> layers;
  std::vector<int32_t> sm_m, sm_k, vd_m, vd_k;
  int32_t mg, kg;
};

namespace {


int64_t al(int64_t x) { return (x + 255) & ~(int64_t)255; }

struct WsLayout {
  int64_t pos_of, slot_of, last_row, h, x8, rm, rk, qkv, q8, eq, att, gu, p64, part, sk_part,
      sk_cnt, sk_tiles, total;
};
constexpr int64_t kSplitPairs = 1024;  // (tile, split) pairs of split-K partials

WsLayout ws_layout(const detint_model_desc& d, int64_t R, int64_t S) {
  WsLayout w{};
  const int64_t nqd = d.n_q * d.head_dim;
  const int64_t nqkv = (d.n_q + 2 * d.n_kv) * d.head_dim;
  int64_t kmax = d.hidden;
  if (d.ffn > kmax) kmax = d.ffn;
  if (nqd > kmax) kmax = nqd;
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o += al(bytes);
    return at;
  };
  const int64_t Rm = R > S ? R : S;
  w.pos_of = take(4 * R);
  w.slot_of = take(4 * R);
  w.last_row = take(4 * S);
  w.h = take(4 * R * d.hidden);
  w.x8 = take(Rm * kmax);
  w.rm = take(4 * Rm);
  w.rk = take(4 * Rm);
  w.qkv = take(4 * R * nqkv);
  w.q8 = take(R * nqd);
  w.eq = take(4 * R * d.n_q);
  w.att = take(4 * R * nqd);
  w.gu = take(4 * R * 2 * d.ffn);
  w.p64 = take(8 * R * d.ffn);
  int64_t np = logits_argmax_parts(d.vocab > 0 ? d.vocab : 1);
  for (int64_t mrows : {int64_t(1), int64_t(8)}) {  // the fused lm_head's partials for any R <= 8
    const int64_t npf = fused_decode_parts(d.vocab > 0 ? d.vocab : 1, mrows);
    if (npf > np) np = npf;
  }
  w.part = take(8 * S * (np > kArgmaxParts ? np : kArgmaxParts));
  // split-K partials and counters of the skinny (<= 64-row) GEMMs
  int64_t nmax = nqkv > d.hidden ? nqkv : d.hidden;
  if (2 * d.ffn > nmax) nmax = 2 * d.ffn;
  w.sk_tiles = (nmax + 31) / 32;
  w.sk_part = R <= 64 ? take(4 * kSplitPairs * kSplitTileInts) : 0;
  w.sk_cnt = R <= 64 ? take(4 * w.sk_tiles) : 0;
  if (R > 64) w.sk_tiles = 0;
  w.total = o;
  return w;
}

}  // namespace

extern "C" {

detint_status detint_model_create(const detint_model_desc* desc, detint_model** out) {
  REQUIRE(desc && out, "model_create: null");
  const detint_model_desc& d = *desc;
  REQUIRE(d.n_layers > 0 && d.hidden > 0 && d.n_q > 0 && d.n_kv > 0 && d.head_dim > 0 &&
              d.ffn > 0 && d.vocab >= 0 && d.max_pos > 0,
          "model_create: bad dimensions");
  REQUIRE(d.n_q % d.n_kv == 0, "model_create: n_q must be a multiple of n_kv");
  REQUIRE(d.hidden % 16 == 0 && d.ffn % 16 == 0 && (d.n_q * d.head_dim) % 16 == 0,
          "model_create: hidden, ffn and n_q*d must be multiples of 16");
  // the residual bound |h| < 2^25 keeps RMSNorm's sum of squares below 2^62
  // only while hidden <= 4096
  REQUIRE(d.head_dim <= 128 && d.hidden <= 4096 && d.ffn <= 8192,
          "model_create: head_dim/hidden/ffn too large (hidden <= 4096, ffn <= 8192)");
  if (!attention_supported(d.head_dim, d.n_q / d.n_kv, d.max_pos))
    return fail(DETINT_EUNSUPPORTED, "model_create: attention does not support d=%lld group=%lld max_pos=%lld",
                (long long)d.head_dim, (long long)(d.n_q / d.n_kv), (long long)d.max_pos);
  REQUIRE(d.layers && d.rope_cos && d.rope_sin, "model_create: null tensor pointer");
  if (d.vocab > 0) {
    REQUIRE(d.emb && d.emb_m && d.final_norm, "model_create: null embedding/final norm");
    if (d.wide) REQUIRE(d.emb_lo, "model_create: wide model needs emb_lo");
  }
  for (int64_t l = 0; l < d.n_layers; ++l) {
    const detint_layer_desc& L = d.layers[l];
    REQUIRE(L.wqkv && L.wqkv_m && L.wo && L.wo_m && L.wgu && L.wgu_m && L.wd && L.wd_m &&
                L.attn_norm && L.ffn_norm,
            "model_create: layer %lld has a null pointer", (long long)l);
    if (d.qk_norm) REQUIRE(L.q_norm && L.k_norm, "model_create: qk_norm needs q/k gains");
    if (d.wide) REQUIRE(L.wqkv_lo && L.wo_lo && L.wgu_lo && L.wd_lo, "model_create: wide limbs");
    if (L.k_gain) REQUIRE(L.kq_k >= 8, "model_create: key gains need kq_k >= 8 (layer %lld)",
                          (long long)l);
  }
  REQUIRE(!(d.wide && d.qk_norm), "model_create: wide weights with q/k-norm not supported");
  detint_model* m = new detint_model();
  m->d = d;
  m->layers.assign(d.layers, d.layers + d.n_layers);
  m->d.layers = nullptr;
  for (auto& L : m->layers) {
    int32_t a, b;
    detint_softmax_mult(L.kq_m, L.kq_k, d.head_dim, d.f_n, &a, &b);
    m->sm_m.push_back(a);
    m->sm_k.push_back(b);
    detint_v_dequant(L.vq_m, L.vq_k, &a, &b);
    m->vd_m.push_back(a);
    m->vd_k.push_back(b);
  }
  detint_swiglu_mult(d.f_a, &m->mg, &m->kg);
  *out = m;
  return ok();
}

void detint_model_destroy(detint_model* m) { delete m; }

int64_t detint_workspace_size(const detint_model* m, int64_t max_rows, int64_t max_seqs) {
  if (!m || max_rows < 0 || max_seqs < 0) return -1;
  return ws_layout(m->d, max_rows, max_seqs).total;
}

// One decoder layer in place on h [R, H] (workspace buffers from w).
// A KV cache as the kernels see it: per-layer bases at k / v + l layer_stride,
// contiguous or paged (see KvPages).
struct Kv {
  int8_t* k;
  int8_t* v;
  int64_t n_slots;
  int64_t layer_stride;
  KvPages pages;
};

Kv contiguous_kv(const detint_model_desc& d, int8_t* k, int8_t* v, int64_t n_slots) {
  return Kv{k, v, n_slots, n_slots * d.n_kv * d.max_pos * d.head_dim, KvPages{nullptr, 0, 0, 0}};
}

static detint_status run_layer(const detint_model* m, int64_t l, int32_t* h, const Kv& kv,
                               int64_t R, const RowMap& seqs,
                               int64_t max_seqlen, char* base, const WsLayout& w, hipStream_t st) {
  const detint_model_desc& d = m->d;
  const detint_layer_desc& L = m->layers[l];
  int32_t* pos_of = (int32_t*)(base + w.pos_of);
  int32_t* slot_of = (int32_t*)(base + w.slot_of);
  int8_t* x8 = (int8_t*)(base + w.x8);
  int32_t* rm = (int32_t*)(base + w.rm);
  int32_t* rk = (int32_t*)(base + w.rk);
  int32_t* qkv = (int32_t*)(base + w.qkv);
  int8_t* q8 = (int8_t*)(base + w.q8);
  int32_t* eq = (int32_t*)(base + w.eq);
  int32_t* att = (int32_t*)(base + w.att);
  int32_t* gu = (int32_t*)(base + w.gu);
  const int64_t H = d.hidden, nq = d.n_q, nkv = d.n_kv, hd = d.head_dim, F = d.ffn;
  const int64_t nqd = nq * hd, nqkv = (nq + 2 * nkv) * hd;
  const int64_t n_slots = kv.n_slots;
  const int32_t wk = d.w_k;
  const SplitWs spw{w.sk_tiles ? (int32_t*)(base + w.sk_part) : nullptr,
                    w.sk_tiles ? (int32_t*)(base + w.sk_cnt) : nullptr, kSplitPairs, w.sk_tiles};
  const SplitWs* sp = w.sk_tiles ? &spw : nullptr;
  int8_t* kc = kv.k + l * kv.layer_stride;
  int8_t* vc = kv.v + l * kv.layer_stride;
  hipError_t e;
#define LAUNCH(x)                                  \
  do {                                             \
    e = (x);                                       \
    if (e != hipSuccess) return hip_status(e, #x); \
  } while (0)
  // attention block: RMSNorm -> QKV -> q/k-norm, RoPE, q DQ, K/V cache ->
  // attention -> DQ -> O-proj + residual
  LAUNCH(launch_rmsnorm(h, nullptr, L.attn_norm, R, H, x8, rm, rk, st));
  {
    Epi ep{rm, rk, L.wqkv_m, wk, d.qk_norm ? 0 : d.f_n, d.qk_norm ? MODE_RAW : MODE_FIX, nullptr};
    LAUNCH(launch_gemm(x8, L.wqkv, d.wide ? L.wqkv_lo : nullptr, R, nqkv, H, ep, qkv, st, sp));
  }
  QkvPost qp{d.qk_norm, rm, rk, L.wqkv_m, wk, L.q_norm, L.k_norm, d.f_n, L.kq_m, L.kq_k,
             L.vq_m, L.vq_k, d.rope_cos, d.rope_sin, L.k_gain};
  if (max_seqlen == 1 && seqs.cu && (int64_t)seqs.S == R) {
    // one row per sequence (decode rows): post-processing fused into the
    // attention kernel, which reads row r's position and slot from
    // start[r] and seq_slot[r]
    LAUNCH(launch_attention_decode_fused(qkv, qp, seqs.start, seqs.seq_slot, R, nq, nkv, hd,
                                         n_slots, d.max_pos, kc, vc, m->sm_m[l], m->sm_k[l], att,
                                         st, kv.pages));
  } else {
    LAUNCH(launch_qkv_post(qkv, R, nq, nkv, hd, pos_of, slot_of, qp, q8, eq, kc, vc, n_slots,
                           d.max_pos, st, kv.pages));
    LAUNCH(launch_attention_seqs(q8, eq, kc, vc, seqs, R, max_seqlen, nq, nkv, hd, n_slots,
                                 d.max_pos, m->sm_m[l], m->sm_k[l], att, st, kv.pages));
  }
  LAUNCH(launch_requant(att, R, nqd, x8, nullptr, rm, rk, m->vd_m[l], m->vd_k[l] + 15 + d.f_n, st));
  {
    Epi ep{rm, rk, L.wo_m, wk, d.f_res, MODE_RES_ADD, nullptr, 0, 0, 25};
    LAUNCH(launch_gemm(x8, L.wo, d.wide ? L.wo_lo : nullptr, R, H, nqd, ep, h, st, sp));
  }
  // FFN block: RMSNorm -> gate/up -> DI-SwiGLU -> down + residual
  LAUNCH(launch_rmsnorm(h, nullptr, L.ffn_norm, R, H, x8, rm, rk, st));
  if (gemm_takes_skinny(R, 2 * F, H, d.wide) && F % 16 == 0 && F % 4 == 0 && F <= 8192) {
    // decode-sized batches: the SwiGLU product in the gate/up GEMM's
    // epilogue (spread over all its workgroups), then only the row DQ
    int64_t* p64 = (int64_t*)(base + w.p64);
    Epi ep{rm, rk, L.wgu_m, wk, d.f_a, MODE_SWIGLU, nullptr, m->mg, m->kg};
    LAUNCH(launch_gemm(x8, L.wgu, d.wide ? L.wgu_lo : nullptr, R, 2 * F, H, ep, p64, st, sp));
    LAUNCH(launch_dq64(p64, R, F, d.f_a, x8, rm, rk, st));
  } else {
    Epi ep{rm, rk, L.wgu_m, wk, d.f_a, MODE_FIX, nullptr};
    LAUNCH(launch_gemm(x8, L.wgu, d.wide ? L.wgu_lo : nullptr, R, 2 * F, H, ep, gu, st, sp));
    LAUNCH(launch_swiglu(gu, R, F, d.f_a, m->mg, m->kg, x8, rm, rk, st));
  }
  {
    Epi ep{rm, rk, L.wd_m, wk, d.f_res, MODE_RES_ADD, nullptr, 0, 0, 25};
    LAUNCH(launch_gemm(x8, L.wd, d.wide ? L.wd_lo : nullptr, R, H, F, ep, h, st, sp));
  }
#undef LAUNCH
  return ok();
}

// Decode-shaped forward (R == S rows, one per sequence at position
// start_pos[s]): embedding, then per layer fused [RMSNorm + QKV],
// [q/k-norm + RoPE + KV write + attention], [DQ + O-proj + residual],
// [RMSNorm + gate/up + SwiGLU product], [DQ + down + residual]; then
// [RMSNorm + lm_head + argmax partials] and [greedy token + advance].
static detint_status run_decode(const detint_model* m, const Kv& kv, int32_t* ids, int64_t R,
                                int32_t* start_pos,
                                const int32_t* slot, int32_t* logits, int32_t* row_base,
                                int32_t* next_tok, bool advance, char* base, const WsLayout& w,
                                hipStream_t st) {
  const detint_model_desc& d = m->d;
  int32_t* h = (int32_t*)(base + w.h);
  int32_t* rm = (int32_t*)(base + w.rm);
  int32_t* rk = (int32_t*)(base + w.rk);
  int32_t* qkv = (int32_t*)(base + w.qkv);
  int32_t* att = (int32_t*)(base + w.att);
  int64_t* p64 = (int64_t*)(base + w.p64);
  int64_t* part = (int64_t*)(base + w.part);
  const int64_t H = d.hidden, nq = d.n_q, nkv = d.n_kv, hd = d.head_dim, F = d.ffn;
  const int64_t nqd = nq * hd, nqkv = (nq + 2 * nkv) * hd;
  const int64_t n_slots = kv.n_slots;
  const int32_t wk = d.w_k;
  hipError_t e;
#define LAUNCH(x)                                  \
  do {                                             \
    e = (x);                                       \
    if (e != hipSuccess) return hip_status(e, #x); \
  } while (0)
  LAUNCH(launch_embed(ids, R, d.emb, nullptr, d.emb_m, H, d.vocab, wk - d.f_res, h, st));
  for (int64_t l = 0; l < d.n_layers; ++l) {
    const detint_layer_desc& L = m->layers[l];
    int8_t* kc = kv.k + l * kv.layer_stride;
    int8_t* vc = kv.v + l * kv.layer_stride;
    LAUNCH(launch_fused_qkv(h, L.attn_norm, L.wqkv, L.wqkv_m, wk, d.qk_norm ? 0 : d.f_n,
                            d.qk_norm != 0, R, nqkv, H, qkv, rm, rk, st));
    QkvPost qp{d.qk_norm, rm, rk, L.wqkv_m, wk, L.q_norm, L.k_norm, d.f_n, L.kq_m, L.kq_k,
               L.vq_m, L.vq_k, d.rope_cos, d.rope_sin, L.k_gain};
    LAUNCH(launch_attention_decode_fused(qkv, qp, start_pos, slot, R, nq, nkv, hd, n_slots,
                                         d.max_pos, kc, vc, m->sm_m[l], m->sm_k[l], att, st,
                                         kv.pages));
    LAUNCH(launch_fused_oproj(att, m->vd_m[l], m->vd_k[l] + 15 + d.f_n, L.wo, L.wo_m, wk, d.f_res,
                              R, H, nqd, h, st));
    LAUNCH(launch_fused_gateup(h, L.ffn_norm, L.wgu, L.wgu_m, wk, d.f_a, m->mg, m->kg, R, F, H, p64,
                               st));
    LAUNCH(launch_fused_down(p64, d.f_a, L.wd, L.wd_m, wk, d.f_res, R, H, F, h, st));
  }
  LAUNCH(launch_fused_lm_head(h, nullptr, d.final_norm, d.emb, d.emb_m, wk, d.f_l, R, d.vocab, H,
                              logits, row_base, part, st));
  LAUNCH(launch_argmax_advance(part, R, fused_decode_parts(d.vocab, R), next_tok, ids, start_pos,
                               row_base, advance, st));
#undef LAUNCH
  return ok();
}

static detint_status check_run(const detint_model* m, const Kv& kv, int64_t R,
                               const int32_t* cu_seqlens, const int32_t* start_pos,
                               const int32_t* slot, int64_t S, int64_t max_seqlen, void* ws,
                               int64_t ws_bytes) {
  REQUIRE(m, "forward: null model");
  REQUIRE(R >= 0 && S >= 0 && kv.n_slots > 0, "forward: bad sizes");
  REQUIRE(S > 0 && R >= S, "forward: need 1 <= S <= R (every sequence has a row)");
  REQUIRE(kv.k && kv.v && cu_seqlens && start_pos && slot && ws, "forward: null pointer");
  REQUIRE(aligned16(kv.k) && aligned16(kv.v) && aligned16(ws), "forward: misaligned buffer");
  REQUIRE(max_seqlen >= 1 && max_seqlen <= R, "forward: bad max_seqlen");
  const WsLayout w = ws_layout(m->d, R, S);
  REQUIRE(ws_bytes >= w.total, "forward: workspace %lld < %lld bytes", (long long)ws_bytes,
          (long long)w.total);
  return ok();
}

// A caller's descriptor as the kernels' view (validated).
static detint_status kv_from_desc(const detint_model* m, const detint_kv_desc* kd, Kv* out) {
  REQUIRE(m && kd, "kv: null model or descriptor");
  const detint_model_desc& d = m->d;
  REQUIRE(kd->n_slots > 0 && kd->n_slots < ((int64_t)1 << 31), "kv: n_slots out of range");
  if (!kd->block_table) {
    *out = contiguous_kv(d, kd->k, kd->v, kd->n_slots);
    return ok();
  }
  const int64_t P = kd->page_size;
  REQUIRE(P >= 16 && P <= d.max_pos && (P & (P - 1)) == 0,
          "kv: page_size must be a power of two in [16, max_pos]");
  REQUIRE(kd->max_blocks * P >= d.max_pos && kd->max_blocks < ((int64_t)1 << 24),
          "kv: max_blocks * page_size must cover max_pos");
  REQUIRE(kd->n_pages > 0 && kd->n_pages * d.n_kv * P * d.head_dim < ((int64_t)1 << 31),
          "kv: a layer's pool must hold under 2^31 bytes");
  int shift = 0;
  while ((int64_t(1) << shift) < P) ++shift;
  *out = Kv{kd->k, kd->v, kd->n_slots, kd->n_pages * d.n_kv * P * d.head_dim,
            KvPages{kd->block_table, (int32_t)kd->max_blocks, shift, (int32_t)kd->n_pages}};
  return ok();
}

int64_t detint_kv_bytes(const detint_model* m, const detint_kv_desc* kv) {
  Kv v;
  if (kv_from_desc(m, kv, &v) != DETINT_OK) return -1;
  return v.layer_stride * m->d.n_layers;
}

static detint_status layer_forward_impl(const detint_model* m, int64_t layer, int32_t* h,
                                        const Kv& kv, int64_t R, const int32_t* cu_seqlens,
                                        const int32_t* start_pos, const int32_t* slot, int64_t S,
                                        int64_t max_seqlen, void* ws, int64_t ws_bytes,
                                        void* stream) {
  if (R == 0 && S == 0) return ok();
  detint_status s = check_run(m, kv, R, cu_seqlens, start_pos, slot, S, max_seqlen, ws, ws_bytes);
  if (s != DETINT_OK) return s;
  REQUIRE(h && layer >= 0 && layer < m->d.n_layers, "layer_forward: bad layer or null h");
  const WsLayout w = ws_layout(m->d, R, S);
  char* base = (char*)ws;
  hipStream_t st = S_(stream);
  hipError_t e = launch_rows_meta(cu_seqlens, start_pos, slot, S, (int32_t*)(base + w.pos_of),
                                  (int32_t*)(base + w.slot_of), (int32_t*)(base + w.last_row), st,
                                  w.sk_tiles ? (int32_t*)(base + w.sk_cnt) : nullptr, w.sk_tiles);
  if (e != hipSuccess) return hip_status(e, "rows_meta");
  const RowMap seqs{cu_seqlens, start_pos, slot, (int32_t)S, nullptr, 0, nullptr};
  return run_layer(m, layer, h, kv, R, seqs, max_seqlen, base, w, st);
}

detint_status detint_layer_forward(const detint_model* m, int64_t layer, int32_t* h,
                                   int8_t* k_cache, int8_t* v_cache, int64_t n_slots, int64_t R,
                                   const int32_t* cu_seqlens, const int32_t* start_pos,
                                   const int32_t* slot, int64_t S, int64_t max_seqlen, void* ws,
                                   int64_t ws_bytes, void* stream) {
  REQUIRE(m, "layer_forward: null model");
  return layer_forward_impl(m, layer, h, contiguous_kv(m->d, k_cache, v_cache, n_slots), R,
                            cu_seqlens, start_pos, slot, S, max_seqlen, ws, ws_bytes, stream);
}

static detint_status forward_impl(const detint_model* m, const Kv& kv, int32_t* ids, int64_t R,
                                  const int32_t* cu_seqlens, int32_t* start_pos,
                                  const int32_t* slot, int64_t S, int64_t max_seqlen,
                                  int32_t* logits, int32_t* logit_row_base, int32_t* next_tok,
                                  int32_t flags, void* ws, int64_t ws_bytes, void* stream) {
  if (R == 0 && S == 0) return ok();
  detint_status s = check_run(m, kv, R, cu_seqlens, start_pos, slot, S, max_seqlen, ws, ws_bytes);
  if (s != DETINT_OK) return s;
  REQUIRE(ids && logits && next_tok, "forward: null ids/logits/next_tok");
  REQUIRE(m->d.vocab > 0 && m->d.emb, "forward: model has no vocabulary");
  if (flags & DETINT_FWD_ADVANCE) REQUIRE(R == S, "forward: ADVANCE needs one row per sequence");
  const detint_model_desc& d = m->d;
  const WsLayout w = ws_layout(d, R, S);
  hipStream_t st = S_(stream);
  char* base = (char*)ws;
  int32_t* last_row = (int32_t*)(base + w.last_row);
  int32_t* h = (int32_t*)(base + w.h);
  int8_t* x8 = (int8_t*)(base + w.x8);
  int32_t* rm = (int32_t*)(base + w.rm);
  int32_t* rk = (int32_t*)(base + w.rk);
  int64_t* part = (int64_t*)(base + w.part);
  hipError_t e;
#define LAUNCH(x)                                  \
  do {                                             \
    e = (x);                                       \
    if (e != hipSuccess) return hip_status(e, #x); \
  } while (0)
  int64_t kmax = d.hidden;
  if (d.ffn > kmax) kmax = d.ffn;
  if (d.n_q * d.head_dim > kmax) kmax = d.n_q * d.head_dim;
  if (R == S && !d.wide && fused_decode_supported(R, kmax)) {
    // decode-shaped call (one row per sequence): 5 fused kernels per layer
    return run_decode(m, kv, ids, R, start_pos, slot, logits, logit_row_base, next_tok,
                      (flags & DETINT_FWD_ADVANCE) != 0, base, w, st);
  }
  LAUNCH(launch_rows_meta(cu_seqlens, start_pos, slot, S, (int32_t*)(base + w.pos_of),
                          (int32_t*)(base + w.slot_of), last_row, st,
                          w.sk_tiles ? (int32_t*)(base + w.sk_cnt) : nullptr, w.sk_tiles));
  LAUNCH(launch_embed(ids, R, d.emb, d.wide ? d.emb_lo : nullptr, d.emb_m, d.hidden, d.vocab,
                      d.w_k - d.f_res, h, st));
  const RowMap seqs{cu_seqlens, start_pos, slot, (int32_t)S, nullptr, 0, nullptr};
  for (int64_t l = 0; l < d.n_layers; ++l) {
    s = run_layer(m, l, h, kv, R, seqs, max_seqlen, base, w, st);
    if (s != DETINT_OK) return s;
  }
  // final norm on each sequence's last row, tied lm_head, greedy token
  LAUNCH(launch_rmsnorm(h, last_row, d.final_norm, S, d.hidden, x8, rm, rk, st));
  {
    Epi ep{rm, rk, d.emb_m, d.w_k, d.f_l, MODE_FIX, logit_row_base};
    const int8_t* lo = d.wide ? d.emb_lo : nullptr;
    if (S <= 16) {  // decode-sized: logits GEMV with fused argmax partials
      LAUNCH(launch_logits_argmax(x8, d.emb, lo, S, d.vocab, d.hidden, ep, logits, part, st));
      LAUNCH(launch_argmax_final(part, S, logits_argmax_parts(d.vocab), next_tok, st));
    } else {
      LAUNCH(launch_gemm(x8, d.emb, lo, S, d.vocab, d.hidden, ep, logits, st));
      LAUNCH(launch_argmax(logits, logit_row_base, S, d.vocab, part, kArgmaxParts, next_tok, st));
    }
  }
  if (flags & DETINT_FWD_ADVANCE)
    LAUNCH(launch_advance(ids, next_tok, start_pos, logit_row_base, S, st));
#undef LAUNCH
  return ok();
}

detint_status detint_forward(const detint_model* m, int8_t* k_cache, int8_t* v_cache,
                             int64_t n_slots, int32_t* ids, int64_t R, const int32_t* cu_seqlens,
                             int32_t* start_pos, const int32_t* slot, int64_t S,
                             int64_t max_seqlen, int32_t* logits, int32_t* logit_row_base,
                             int32_t* next_tok, int32_t flags, void* ws, int64_t ws_bytes,
                             void* stream) {
  REQUIRE(m, "forward: null model");
  return forward_impl(m, contiguous_kv(m->d, k_cache, v_cache, n_slots), ids, R, cu_seqlens,
                      start_pos, slot, S, max_seqlen, logits, logit_row_base, next_tok, flags, ws,
                      ws_bytes, stream);
}

detint_status detint_forward_kv(const detint_model* m, const detint_kv_desc* kv, int32_t* ids,
                                int64_t R, const int32_t* cu_seqlens, int32_t* start_pos,
                                const int32_t* slot, int64_t S, int64_t max_seqlen,
                                int32_t* logits, int32_t* logit_row_base, int32_t* next_tok,
                                int32_t flags, void* ws, int64_t ws_bytes, void* stream) {
  Kv v;
  detint_status s = kv_from_desc(m, kv, &v);
  if (s != DETINT_OK) return s;
  return forward_impl(m, v, ids, R, cu_seqlens, start_pos, slot, S, max_seqlen, logits,
                      logit_row_base, next_tok, flags, ws, ws_bytes, stream);
}

}  // extern "C"

extern "C" detint_status detint_probe_barrier(int32_t mode, int32_t rounds, uint32_t* result,
                                              void* stream) {
  REQUIRE(mode >= 0 && mode <= 3 && rounds >= 0 && rounds <= (1 << 20),
          "probe_barrier: mode in 0..3 and rounds in 0..2^20");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e, "probe_barrier");
  if (cus < 256)
    return fail(DETINT_EUNSUPPORTED, "probe_barrier: needs 256 CUs (one resident workgroup each), found %d", cus);
  return hip_status(launch_probe_barrier(mode, rounds, result, S_(stream)), "probe_barrier");
}
