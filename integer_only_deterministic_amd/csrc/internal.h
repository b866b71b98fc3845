// Internal launchers shared by the libdetint translation units (host side).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace detint {

enum { MODE_RAW = 0, MODE_REQ_I8 = 1, MODE_FIX = 2, MODE_RES_ADD = 3, MODE_SWIGLU = 4 };

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device,
// once per (device, kernel): thread-safe (a mutex-guarded registry), and the
// attribute call is not a stream operation, so a first launch inside a graph
// capture records only the kernel. Returns the attribute call's status.
hipError_t set_max_lds(const void* kernel, int bytes);

// Dyadic epilogue parameters of a GEMM (see detint.h, detint_gemm_i8).
struct Epi {
  const int32_t* row_m;
  const int32_t* row_k;
  const int32_t* col_m;
  int32_t col_k;
  int32_t frac;
  int32_t mode;
  const int32_t* out_row_base;  // nullable: output row i goes to row *base + i
  // MODE_SWIGLU (skinny GEMMs only): W holds F gate rows then F up rows
  // (N = 2F, F % 16 == 0); gate and up go through the FIX epilogue (frac =
  // f_a) and the int64 DI-SwiGLU product R(g sigmoid(g), 15) u is stored to
  // out [M, F]. Sigmoid multiplier (sw_mg, sw_kg).
  int32_t sw_mg, sw_kg;
  // RES_ADD bound: a result with |h| >= 2^res_bits raises the residual bound
  // flag (the model's residual stream: 25); 0 checks only the int32 range.
  int32_t res_bits;
};

// Bound flags of each translation unit (see detint_check): wait for the
// stream, OR the unit's flag word into *acc and clear it.
hipError_t bound_flags_gemm(uint32_t* acc, hipStream_t st);
hipError_t bound_flags_decode(uint32_t* acc, hipStream_t st);
hipError_t bound_flags_rowops(uint32_t* acc, hipStream_t st);
hipError_t bound_flags_attention(uint32_t* acc, hipStream_t st);

// C = A[M,K] . W[N,K]^T with epilogue; W_lo != nullptr selects 16-bit limbs.
// Workspace for split-K skinny GEMMs: int32 partials for up to
// max_tile_splits (tile, split) pairs of up to 2 x 64 x 32 values each plus
// row sums, and one arrival counter per 32-column tile (max_tiles), which must
// be zero before the first use (every use leaves them zero).
// part_ints > 0 also lets the pipelined int8 GEMM split K over workgroup
// rows for shapes with few tiles: part then holds ks M N int32 partials.
struct SplitWs {
  int32_t* part;
  int32_t* cnt;
  int64_t max_tile_splits;
  int64_t max_tiles;
  int64_t part_ints;
};
constexpr int64_t kSplitTileInts = 2 * 2 * 1024 + 2 * 32;
constexpr int64_t kSplitPairsStandalone = 1024;
// Workspace bytes a standalone GEMM uses for split-K (0: none), and the
// kernel that clears int32 counters.
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, bool limbs);
hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t st);

hipError_t launch_gemm(const int8_t* A, const int8_t* W, const int8_t* W_lo, int64_t M,
                       int64_t N, int64_t K, const Epi& e, void* out, hipStream_t st,
                       const SplitWs* sp = nullptr);
// true when launch_gemm runs this shape on the skinny kernel (the only one
// with MODE_SWIGLU)
bool gemm_takes_skinny(int64_t M, int64_t N, int64_t K, bool limbs);
hipError_t launch_split_w16(const int16_t* W16, int64_t n, int8_t* hi, int8_t* lo,
                            hipStream_t st);
// Exact mode (bf16 weights as integers): planes int8 [4][N][K], row_exp [N];
// the GEMM's workspace holds 2 M N + M int64 (two limb products, row sums).
hipError_t launch_exact_prepare(const uint16_t* W, int64_t N, int64_t K, int8_t* planes,
                                int32_t* row_exp, hipStream_t st);
hipError_t launch_gemm_exact(const int8_t* A, const int8_t* planes, const int32_t* row_exp,
                             int64_t M, int64_t N, int64_t K, const int32_t* row_m,
                             const int32_t* row_k, int32_t frac, int32_t mode, void* out,
                             int64_t* ws, hipStream_t st);
// lm_head for M <= 16 rows: FIX-mode logits plus per-wave greedy-argmax
// partials part[M][logits_argmax_parts(N)] (reduce with launch_argmax_final).
int64_t logits_argmax_parts(int64_t N);
hipError_t launch_logits_argmax(const int8_t* A, const int8_t* W, const int8_t* W_lo, int64_t M,
                                int64_t N, int64_t K, const Epi& e, int32_t* logits,
                                int64_t* part, hipStream_t st);
hipError_t launch_argmax_final(const int64_t* part, int64_t S, int64_t nparts, int32_t* out,
                               hipStream_t st);

// Row ops.
hipError_t launch_rmsnorm(const int32_t* h, const int32_t* row_index, const int16_t* gain,
                          int64_t R, int64_t n, int8_t* x8, int32_t* row_m, int32_t* row_k,
                          hipStream_t st);
// DQ of each row; optionally also a row scale (fold_m, fold_k - e) into
// row_m / row_k (the attention output's scale folds the V dequant scale).
hipError_t launch_requant(const int32_t* y, int64_t R, int64_t n, int8_t* q, int32_t* row_e,
                          int32_t* row_m, int32_t* row_k, int32_t fold_m, int32_t fold_k,
                          hipStream_t st);
// q = clamp8(R(y m, k)) elementwise (16-byte aligned y, 4-byte aligned q)
hipError_t launch_requant_fixed(const int32_t* y, int64_t n, int32_t m, int32_t k, int8_t* q,
                                hipStream_t st);
hipError_t launch_rope(int32_t* x, const int32_t* pos, const int16_t* cos_t,
                       const int16_t* sin_t, int64_t R, int64_t heads, int64_t d, int64_t max_pos,
                       hipStream_t st);
hipError_t launch_softmax(const int32_t* s, const int32_t* valid, const int32_t* shift,
                          int64_t R, int64_t C, int32_t M, int32_t K, int16_t* P,
                          hipStream_t st);
// Temperature / top-k / top-p sampling of R rows of V logits (keep in [1, V],
// top_p in [1, 2^16], 2^16 = off).
// With a workspace of sample_workspace_bytes(R, V) and every id kept, plain
// temperature sampling runs over 1024-id slices in three kernels.
hipError_t launch_sample(const int32_t* logits, int64_t R, int64_t V, int64_t keep, int32_t top_p,
                         int32_t t_m, int32_t t_k, const uint32_t* draws, int32_t* out, void* ws,
                         int64_t ws_bytes, hipStream_t st);
int64_t sample_workspace_bytes(int64_t R, int64_t V);
hipError_t launch_swiglu(const int32_t* gu, int64_t R, int64_t n, int32_t f_a, int32_t Mg,
                         int32_t Kg, int8_t* a8, int32_t* row_m, int32_t* row_k, hipStream_t st);
// DQ of int64 SwiGLU products [R, n] -> int8, row scale (2^14, 2 f_a - e + 14)
hipError_t launch_dq64(const int64_t* p, int64_t R, int64_t n, int32_t f_a, int8_t* a8,
                       int32_t* row_m, int32_t* row_k, hipStream_t st);
hipError_t launch_embed(const int32_t* ids, int64_t R, const int8_t* emb, const int8_t* emb_lo,
                        const int32_t* emb_m, int64_t H, int64_t V, int32_t shift, int32_t* h,
                        hipStream_t st);

// Per-row metadata of packed sequences: pos_of/slot_of [R], last_row [S];
// also zeroes zero[0 .. nzero) (the split-K arrival counters).
hipError_t launch_rows_meta(const int32_t* cu, const int32_t* start, const int32_t* slot,
                            int64_t S, int32_t* pos_of, int32_t* slot_of, int32_t* last_row,
                            hipStream_t st, int32_t* zero = nullptr, int64_t nzero = 0);
hipError_t launch_decode_meta(const int32_t* ctx_len, const int32_t* slot, int64_t B,
                              int32_t* pos_of, int32_t* slot_of, hipStream_t st);

// Where the cached rows of a (slot, KV head) live. bt == nullptr: the
// contiguous layout [n_slots][n_kv][max_pos][d] per layer. Otherwise a paged
// pool [n_pages][n_kv][2^shift][d] per layer: position j of slot s is row
// j & (2^shift - 1) of page bt[s * max_blocks + (j >> shift)]. A page index
// outside [0, n_pages) raises the PAGE bound flag and is read and written as
// page 0 (memory-safe, results undefined).
struct KvPages {
  const int32_t* bt;
  int32_t max_blocks, shift, n_pages;
};

// QKV post-processing: q/k-norm (or fixed-point input), RoPE, q DQ, K/V cache
// writes. qkv int32 [R, (nq + 2 nkv) d].
struct QkvPost {
  int32_t qk_norm;            // 1: qkv holds raw accumulators; 0: f_n fixed point
  const int32_t* row_m;       // row scale of the GEMM input (raw mode, V)
  const int32_t* row_k;
  const int32_t* col_m;       // column mantissas of Wqkv (raw mode)
  int32_t col_k;
  const int16_t* q_norm;
  const int16_t* k_norm;
  int32_t f_n;
  int32_t kq_m, kq_k, vq_m, vq_k;
  const int16_t* cos_t;
  const int16_t* sin_t;
  const int8_t* k_gain;       // [nkv][d] per-channel key gains in [0, 7], or null
};
hipError_t launch_qkv_post(const int32_t* qkv, int64_t R, int64_t nq, int64_t nkv, int64_t d,
                           const int32_t* pos_of, const int32_t* slot_of, const QkvPost& p,
                           int8_t* q8, int32_t* e_q, int8_t* kc, int8_t* vc, int64_t n_slots,
                           int64_t max_pos, hipStream_t st, KvPages kp = KvPages{});

// Where a row sits: either packed sequences (cu != nullptr: row r belongs to
// the sequence s with cu[s] <= r < cu[s+1], position start[s] + r - cu[s],
// slot seq_slot[s]) or per-row arrays (position pos[r] + bias, slot slot[r]).
struct RowMap {
  const int32_t* cu;
  const int32_t* start;
  const int32_t* seq_slot;
  int32_t S;
  const int32_t* pos;
  int32_t bias;
  const int32_t* slot;
};

// Attention for R rows packed as S sequences (seqs.cu / start / seq_slot):
// the MFMA prefill kernel when the longest sequence has 16 or more rows and
// the head shape allows, else the per-row kernel. Same results either way.
hipError_t launch_attention_seqs(const int8_t* q8, const int32_t* e_q, const int8_t* kc,
                                 const int8_t* vc, const RowMap& seqs, int64_t R,
                                 int64_t max_seqlen, int64_t nq, int64_t nkv, int64_t d,
                                 int64_t n_slots, int64_t max_pos, int32_t M, int32_t K,
                                 int32_t* out, hipStream_t st, KvPages kp = KvPages{});

// Attention over the cache for R rows.
hipError_t launch_attention(const int8_t* q8, const int32_t* e_q, const int8_t* kc,
                            const int8_t* vc, const RowMap& rows, int64_t R, int64_t nq,
                            int64_t nkv, int64_t d, int64_t n_slots, int64_t max_pos, int32_t M,
                            int32_t K, int32_t* out, hipStream_t st, KvPages kp = KvPages{});
// Decode (one row per sequence at position start_pos[b] of slot slot[b]):
// QKV post-processing of each (row, KV head)'s own heads fused with attention.
hipError_t launch_attention_decode_fused(const int32_t* qkv, const QkvPost& p,
                                         const int32_t* start_pos, const int32_t* slot, int64_t B,
                                         int64_t nq, int64_t nkv, int64_t d, int64_t n_slots,
                                         int64_t max_pos, int8_t* kc, int8_t* vc, int32_t M,
                                         int32_t K, int32_t* out, hipStream_t st,
                                         KvPages kp = KvPages{});
// true when the attention kernel supports (d, n_q / n_kv, max_pos)
bool attention_supported(int64_t d, int64_t group, int64_t max_pos);

// Greedy argmax over rows of int32 logits (lowest index among maxima).
hipError_t launch_argmax(const int32_t* logits, const int32_t* row_base, int64_t S, int64_t V,
                         int64_t* part, int64_t nparts, int32_t* out, hipStream_t st);
hipError_t launch_advance(int32_t* ids, const int32_t* next_tok, int32_t* start_pos,
                          int32_t* row_base, int64_t S, hipStream_t st);
hipError_t launch_argmax_advance(const int64_t* part, int64_t S, int64_t nparts, int32_t* next_tok,
                                 int32_t* ids, int32_t* start_pos, int32_t* row_base, bool advance,
                                 hipStream_t st);

// Fused decode kernels (decode.hip), M <= 8 rows of 8-bit weights.
bool fused_decode_supported(int64_t M, int64_t K);
// argmax partials per row of the fused lm_head for M rows (at most
// fused_decode_parts(V, 8) for any M <= 8)
int fused_decode_parts(int64_t V, int64_t M);
hipError_t launch_fused_qkv(const int32_t* h, const int16_t* gain, const int8_t* W,
                            const int32_t* col_m, int32_t col_k, int32_t frac, bool raw, int64_t M,
                            int64_t N, int64_t K, int32_t* out, int32_t* rm_out, int32_t* rk_out,
                            hipStream_t st);
hipError_t launch_fused_oproj(const int32_t* att, int32_t fold_m, int32_t fold_k, const int8_t* W,
                              const int32_t* col_m, int32_t col_k, int32_t frac, int64_t M,
                              int64_t N, int64_t K, int32_t* h, hipStream_t st);
hipError_t launch_fused_gateup(const int32_t* h, const int16_t* gain, const int8_t* W,
                               const int32_t* col_m, int32_t col_k, int32_t f_a, int32_t Mg,
                               int32_t Kg, int64_t M, int64_t F, int64_t K, int64_t* prod,
                               hipStream_t st);
hipError_t launch_fused_down(const int64_t* prod, int32_t f_a, const int8_t* W, const int32_t* col_m,
                             int32_t col_k, int32_t frac, int64_t M, int64_t N, int64_t K,
                             int32_t* h, hipStream_t st);
// Standalone int8 GEMM for M <= 8 rows on the decode GEMV (8-bit weights,
// K <= 8192, K % 16 == 0, N K < 2^31, 4-byte aligned A; any epilogue mode,
// no out_row_base).
hipError_t launch_fgemv_i8(const int8_t* A, const int8_t* W, int64_t M, int64_t N, int64_t K,
                           const int32_t* row_m, const int32_t* row_k, const int32_t* col_m,
                           int32_t col_k, int32_t frac, int mode, void* out, hipStream_t st,
                           int32_t res_bits = 0);
hipError_t launch_fused_lm_head(const int32_t* h, const int32_t* row_index, const int16_t* gain,
                                const int8_t* E, const int32_t* emb_m, int32_t w_k, int32_t f_l,
                                int64_t M, int64_t V, int64_t K, int32_t* logits,
                                const int32_t* row_base, int64_t* part, hipStream_t st);

// Device-wide barrier measurement (256 resident workgroups; mode 0..3; the
// failure bits of the last run into *result after a stream sync, if given).
hipError_t launch_probe_barrier(int mode, int rounds, uint32_t* result, hipStream_t st);

}  // namespace detint
