// Per-head QKV post-processing shared by the standalone QKV kernel and the
// fused decode attention kernel. One wave handles one head of one row; lane
// i < d/2 owns the RoPE pair (i, i + d/2).
//
// q and k: per-head RMSNorm of acc * m_c (Qwen3 q/k-norm, placed before RoPE
// per DetLLM blog footnote 8; the column shift and the row scale cancel in
// the normalisation) or, without q/k-norm, the f_n fixed point the GEMM
// epilogue already produced; then RoPE with the Q1.14 tables. q -> DQ per
// head (q8, e_q). k, v -> int8 at the layer's fixed cache scales, written once
// into the cache (DetLLM blog "DetLLM": prefill and decode read the same
// cached bits).
#pragma once
#include "dev_int.h"
#include "internal.h"

namespace detint {

// Byte offset, within one layer's paged pool, of position j of (slot, KV
// head kvh); see KvPages. A page index outside the pool sets kBoundPage in
// `bad` and addresses page 0.
__device__ __forceinline__ int64_t page_row_off(const KvPages& kp, int slot, int kvh, int nkv, int d,
                                                int j, uint32_t& bad) {
  int page = kp.bt[(int64_t)slot * kp.max_blocks + (j >> kp.shift)];
  if ((unsigned)page >= (unsigned)kp.n_pages) {
    bad |= kBoundPage;
    page = 0;
  }
  return ((((int64_t)page * nkv + kvh) << kp.shift) + (j & ((1 << kp.shift) - 1))) * d;
}

// The same offset for either layout, from the layer's cache base.
__device__ __forceinline__ int64_t kv_row_off(const KvPages& kp, int slot, int kvh, int nkv,
                                              int max_pos, int d, int j, uint32_t& bad) {
  if (!kp.bt) return (((int64_t)slot * nkv + kvh) * max_pos + j) * d;
  return page_row_off(kp, slot, kvh, nkv, d, j, bad);
}

__device__ __forceinline__ void qkv_head(const int32_t* __restrict__ row, int hh, int nq, int nkv,
                                         int d, int pos, int slot, bool ok, int32_t rm, int32_t rk,
                                         const QkvPost& p, int8_t* q_dst, int32_t* e_dst,
                                         int8_t* __restrict__ kc, int8_t* __restrict__ vc,
                                         int max_pos, const KvPages& kp) {
  const int lane = threadIdx.x & 63;
  const int half = d >> 1;
  const bool act = lane < half;
  const int j0 = lane, j1 = lane + half;
  const int c0 = hh * d;
  if (hh >= nq + nkv) {  // V
    if (!act || !ok) return;
    const int kvh = hh - nq - nkv;
    uint32_t bad = 0;
    int8_t* dst = vc + kv_row_off(kp, slot, kvh, nkv, max_pos, d, pos, bad);
    bound_raise(bad);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = t ? j1 : j0;
      int64_t vf = row[c0 + j];
      if (p.qk_norm) vf = R(vf * rm * p.col_m[c0 + j], rk + p.col_k - p.f_n);
      bound_raise(i32_check(vf));
      dst[j] = clamp8(R(vf * p.vq_m, p.vq_k));
    }
    return;
  }
  int64_t x0 = 0, x1 = 0;
  if (act) {
    x0 = row[c0 + j0];
    x1 = row[c0 + j1];
  }
  if (p.qk_norm) {
    const int16_t* gn = hh < nq ? p.q_norm : p.k_norm;
    int64_t a0 = act ? x0 * p.col_m[c0 + j0] : 0, a1 = act ? x1 * p.col_m[c0 + j1] : 0;
    const int b = wave_bitlen_max(uabs64(a0), uabs64(a1));
    const int sh0 = b > 24 ? b - 24 : 0;
    a0 = R(a0, sh0);
    a1 = R(a1, sh0);
    const int64_t S = wave_sum(a0 * a0 + a1 * a1);
    if (S == 0) {
      x0 = x1 = 0;
    } else {
      int32_t m, sh;
      irms_wave(S, d, m, sh);
      if (act) {
        x0 = R(a0 * gn[j0] * m, sh + 12 - p.f_n);
        x1 = R(a1 * gn[j1] * m, sh + 12 - p.f_n);
      }
    }
  }
  int64_t y0 = 0, y1 = 0;
  if (act && ok) {
    const int64_t c = p.cos_t[(size_t)pos * half + lane], s = p.sin_t[(size_t)pos * half + lane];
    y0 = R(x0 * c - x1 * s, 14);
    y1 = R(x1 * c + x0 * s, 14);
    bound_raise(i32_check(y0) | i32_check(y1));  // rotated q / k within int32
  }
  if (hh < nq) {
    if (p.k_gain && act) {  // the inverse of the key gain of the shared KV head
      // query heads per KV head is a power of two: hh / (nq / nkv) as a shift
      const int8_t* g = p.k_gain + (size_t)(hh >> (__builtin_ctz(nq) - __builtin_ctz(nkv))) * d;
      y0 = R(y0, g[j0] & 7);
      y1 = R(y1, g[j1] & 7);
    }
    const int bl = wave_bitlen_max(uabs64(y0), uabs64(y1));
    const int e = bl > 7 ? bl - 7 : 0;  // dq_exp of the maximum
    if (act) {
      q_dst[j0] = clamp8(R(y0, e));
      q_dst[j1] = clamp8(R(y1, e));
    }
    if (lane == 0) *e_dst = e;
  } else if (act && ok) {
    const int kvh = hh - nq;
    uint32_t bad = 0;
    int8_t* dst = kc + kv_row_off(kp, slot, kvh, nkv, max_pos, d, pos, bad);
    bound_raise(bad);
    const int8_t* g = p.k_gain ? p.k_gain + (size_t)kvh * d : nullptr;
    dst[j0] = clamp8(R(y0 * p.kq_m, p.kq_k - (g ? g[j0] & 7 : 0)));
    dst[j1] = clamp8(R(y1 * p.kq_m, p.kq_k - (g ? g[j1] & 7 : 0)));
  }
}

}  // namespace detint
