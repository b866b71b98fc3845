// Causal attention over the int8 KV cache with DI-Softmax (15-bit
// probabilities) for gfx950.
//
// One 256-thread workgroup per (query row, KV head) handles the G = n_q/n_kv
// query heads that share that KV head (grouped-query attention), so every
// cached K/V row is read once per query row. Exactness rules out the online
// (flash) rescaling: DI-Exp must see the true row maximum and P needs the
// full sum first (DetLLM blog, footnote 8: 15-bit probabilities, P.V exact),
// so the row is processed in passes over an LDS copy of its scores:
//   1. s_j = q8 . k8_j (v_dot4), kept in LDS; row max per head;
//   2. E_j = DI-Exp(R((s_j - max) M, K - e_q)) in place; D = sum E_j;
//   3. P_j = min(R(E_j floor(2^46 / D), 31), 2^15 - 1) on the fly while
//      4. out[t] = sum_j P_j v8_j[t]: a lane owns a 16-byte column chunk of a
//         V row (rows read whole, coalesced) and the partial sums are reduced
//         over lanes and waves - an exact integer sum in any order.
// Prefill and decode both use it (row position and slot come per row), which
// is what makes prefill and token-by-token decode produce the same bits.
#include "dev_int.h"
#include "internal.h"
#include "qkv_dev.h"

namespace detint {
namespace {

constexpr int TPB = 256;

__device__ __forceinline__ int sbyte(int w, int b) { return (w << (24 - 8 * b)) >> 24; }

__device__ __forceinline__ int dot16(const v4i& a, const v4i& b, int c) {
  c = __builtin_amdgcn_sdot4(a.x, b.x, c, false);
  c = __builtin_amdgcn_sdot4(a.y, b.y, c, false);
  c = __builtin_amdgcn_sdot4(a.z, b.z, c, false);
  c = __builtin_amdgcn_sdot4(a.w, b.w, c, false);
  return c;
}

__device__ __forceinline__ void row_info(const RowMap& m, int r, int& pos, int& slot) {
  if (m.cu) {
    int lo = 0, hi = m.S - 1;  // last s with cu[s] <= r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (m.cu[mid] <= r)
        lo = mid;
      else
        hi = mid - 1;
    }
    pos = m.start[lo] + r - m.cu[lo];
    slot = m.seq_slot[lo];
  } else {
    pos = m.pos[r] + m.bias;
    slot = m.slot[r];
  }
}

// Attention of one query row for the G query heads sharing one KV head.
// sq: the G q8 vectors (LDS, 16-byte chunks); eqv: their DQ exponents;
// K, V: the (slot, KV head) cache block; keys 0..ctx-1; sc: LDS [G][ld].
template <int D, int G, int NT = TPB>
__device__ __forceinline__ void attend(const v4i* sq, const int32_t* eqv, const int8_t* __restrict__ K,
                                       const int8_t* __restrict__ V, int ctx, int ld, int32_t Ms,
                                       int32_t Ks, int32_t* __restrict__ orow, int32_t* sc,
                                       int64_t* red, int32_t (*sred)[G * D]) {
  constexpr int CH = D / 16;        // 16-byte chunks per row
  constexpr int RG = NT / CH;       // V rows in flight per pass-4 step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % CH, rg = tid / CH;

  // pass 1: scores and per-head max
  int64_t mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = INT64_MIN;
  auto score = [&](const v4i (&kv)[CH], int j) {
    int s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = dot16(sq[g * CH + c], kv[c], s[g]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sc[g * ld + j] = s[g];
      mx[g] = s[g] > mx[g] ? s[g] : mx[g];
    }
  };
  int j1 = tid;
  for (; j1 + NT < ctx; j1 += 2 * NT) {  // two key rows in flight
    v4i ka[CH], kb[CH];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      ka[cc] = ((const v4i*)(K + (size_t)j1 * D))[cc];
      kb[cc] = ((const v4i*)(K + (size_t)(j1 + NT) * D))[cc];
    }
    score(ka, j1);
    score(kb, j1 + NT);
  }
  if (j1 < ctx) {
    v4i ka[CH];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) ka[cc] = ((const v4i*)(K + (size_t)j1 * D))[cc];
    score(ka, j1);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = block_max(mx[g], red);

  // pass 2: exponentials and their sum
  int sh[G];
  int64_t den[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    sh[g] = Ks - eqv[g];
    den[g] = 0;
  }
  for (int j = tid; j < ctx; j += NT) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int32_t E = diexp(R(((int64_t)sc[g * ld + j] - mx[g]) * Ms, sh[g]));
      sc[g * ld + j] = E;
      den[g] += E;
    }
  }
  int64_t rn[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    den[g] = block_sum(den[g], red);  // also orders pass-2 LDS writes before pass 4
    rn[g] = (int64_t)udiv_wave<32>(uint64_t(1) << 46, (uint64_t)den[g]);  // D >= 2^15
  }

  // passes 3+4: probabilities and P.V
  int acc[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int b = 0; b < 16; ++b) acc[g][b] = 0;
  auto pv = [&](const v4i& v, int j) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      int64_t p = R((int64_t)sc[g * ld + j] * rn[g], 31);
      const int P = (int)(p > 32767 ? 32767 : p);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[g][b] += P * sbyte(v.x, b);
        acc[g][4 + b] += P * sbyte(v.y, b);
        acc[g][8 + b] += P * sbyte(v.z, b);
        acc[g][12 + b] += P * sbyte(v.w, b);
      }
    }
  };
  int j = rg;
  for (; j + 3 * RG < ctx; j += 4 * RG) {  // four independent row loads in flight
    const v4i v0 = *(const v4i*)(V + (size_t)j * D + c * 16);
    const v4i v1 = *(const v4i*)(V + (size_t)(j + RG) * D + c * 16);
    const v4i v2 = *(const v4i*)(V + (size_t)(j + 2 * RG) * D + c * 16);
    const v4i v3 = *(const v4i*)(V + (size_t)(j + 3 * RG) * D + c * 16);
    pv(v0, j);
    pv(v1, j + RG);
    pv(v2, j + 2 * RG);
    pv(v3, j + 3 * RG);
  }
  for (; j < ctx; j += RG) pv(*(const v4i*)(V + (size_t)j * D + c * 16), j);
  // reduce over the lanes of a wave that share chunk c
#pragma unroll
  for (int off = CH; off < 64; off <<= 1)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int b = 0; b < 16; ++b) acc[g][b] += __shfl_xor(acc[g][b], off);
  if (lane < CH) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int b = 0; b < 16; ++b) sred[wave][g * D + c * 16 + b] = acc[g][b];
  }
  __syncthreads();
  for (int t = tid; t < G * D; t += NT) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += sred[w][t];
    orow[t] = s;
  }
}

template <int D, int G>
__global__ __launch_bounds__(TPB) void attn_rows(const int8_t* __restrict__ q8,
                                                 const int32_t* __restrict__ e_q,
                                                 const int8_t* __restrict__ kc,
                                                 const int8_t* __restrict__ vc, RowMap rows,
                                                 int nq, int nkv, int n_slots, int max_pos,
                                                 int32_t Ms, int32_t Ks,
                                                 int32_t* __restrict__ out) {
  constexpr int CH = D / 16;
  extern __shared__ int32_t sc[];   // [G][max_pos]: scores -> E
  __shared__ v4i sq[G * CH];
  __shared__ int32_t seq[G];
  __shared__ int64_t red[16];
  __shared__ int32_t sred[TPB / 64][G * D];
  const int r = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x;
  const int h0 = kvh * G;
  int pos, slot;
  row_info(rows, r, pos, slot);
  int32_t* orow = out + ((size_t)r * nq + h0) * D;
  if (pos < 0 || pos >= max_pos || slot < 0 || slot >= n_slots) {
    for (int t = tid; t < G * D; t += TPB) orow[t] = 0;
    return;
  }
  const size_t base = ((size_t)slot * nkv + kvh) * max_pos * D;
  if (tid < G * CH) sq[tid] = *(const v4i*)(q8 + ((size_t)r * nq + h0) * D + tid * 16);
  if (tid < G) seq[tid] = e_q[(size_t)r * nq + h0 + tid];
  __syncthreads();
  attend<D, G>(sq, seq, kc + base, vc + base, pos + 1, max_pos, Ms, Ks, orow, sc, red, sred);
}

// Decode: one row per sequence. The workgroup of (row, KV head) first does
// the QKV post-processing of its own heads (G query heads -> q8 in LDS, the
// key and value -> int8 into the cache at the row's position), then attends
// over positions 0..pos, which include the key it just wrote.
template <int D, int G>
__global__ __launch_bounds__(TPB) void attn_decode_fused(
    const int32_t* __restrict__ qkv, QkvPost p, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ slot_arr, int nq, int nkv, int n_slots, int max_pos,
    int8_t* __restrict__ kc, int8_t* __restrict__ vc, int32_t Ms, int32_t Ks,
    int32_t* __restrict__ out) {
  constexpr int CH = D / 16;
  extern __shared__ int32_t sc[];
  __shared__ v4i sq[G * CH];
  __shared__ int32_t seq[G];
  __shared__ int64_t red[16];
  constexpr int DEC_NT = TPB;
  __shared__ int32_t sred[DEC_NT / 64][G * D];
  const int r = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x, wave = tid >> 6;
  const int h0 = kvh * G;
  const int pos = start_pos[r], slot = slot_arr[r];
  int32_t* orow = out + ((size_t)r * nq + h0) * D;
  if (pos < 0 || pos >= max_pos || slot < 0 || slot >= n_slots) {
    for (int t = tid; t < G * D; t += DEC_NT) orow[t] = 0;
    return;
  }
  const int nh = nq + 2 * nkv;
  const int32_t* row = qkv + (size_t)r * nh * D;
  const int32_t rm = p.qk_norm ? p.row_m[r] : 0, rk = p.qk_norm ? p.row_k[r] : 0;
  for (int t = wave; t < G + 2; t += DEC_NT / 64) {
    const int hh = t < G ? h0 + t : (t == G ? nq + kvh : nq + nkv + kvh);
    int8_t* qd = (int8_t*)sq + (t < G ? t : 0) * D;
    qkv_head(row, hh, nq, nkv, D, pos, slot, true, rm, rk, p, qd, &seq[t < G ? t : 0], kc, vc,
             max_pos);
  }
  __syncthreads();
  const size_t base = ((size_t)slot * nkv + kvh) * max_pos * D;
  attend<D, G, DEC_NT>(sq, seq, kc + base, vc + base, pos + 1, max_pos, Ms, Ks, orow, sc, red,
                          sred);
}

template <int D, int G>
hipError_t launch_t(const int8_t* q8, const int32_t* e_q, const int8_t* kc, const int8_t* vc,
                    const RowMap& rows, int64_t R, int64_t nq, int64_t nkv, int64_t n_slots,
                    int64_t max_pos, int32_t M, int32_t K, int32_t* out, hipStream_t st) {
  const size_t lds = (size_t)G * max_pos * sizeof(int32_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)attn_rows<D, G>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        96 * 1024);
    attr_set = true;
  }
  attn_rows<D, G><<<dim3((unsigned)R, (unsigned)nkv), TPB, lds, st>>>(
      q8, e_q, kc, vc, rows, (int)nq, (int)nkv, (int)n_slots, (int)max_pos, M, K, out);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_fused_t(const int32_t* qkv, const QkvPost& p, const int32_t* start_pos,
                          const int32_t* slot, int64_t B, int64_t nq, int64_t nkv, int64_t n_slots,
                          int64_t max_pos, int8_t* kc, int8_t* vc, int32_t M, int32_t K, int32_t* out,
                          hipStream_t st) {
  const size_t lds = (size_t)G * max_pos * sizeof(int32_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)attn_decode_fused<D, G>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    attr_set = true;
  }
  attn_decode_fused<D, G><<<dim3((unsigned)B, (unsigned)nkv), TPB, lds, st>>>(
      qkv, p, start_pos, slot, (int)nq, (int)nkv, (int)n_slots, (int)max_pos, kc, vc, M, K, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_decode_fused(const int32_t* qkv, const QkvPost& p,
                                         const int32_t* start_pos, const int32_t* slot, int64_t B,
                                         int64_t nq, int64_t nkv, int64_t d, int64_t n_slots,
                                         int64_t max_pos, int8_t* kc, int8_t* vc, int32_t M,
                                         int32_t K, int32_t* out, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const int64_t G = nq / nkv;
#define DETINT_ATTF(DD, GG)                                                                      \
  if (d == DD && G == GG)                                                                        \
    return launch_fused_t<DD, GG>(qkv, p, start_pos, slot, B, nq, nkv, n_slots, max_pos, kc, vc, \
                                  M, K, out, st);
  DETINT_ATTF(64, 1) DETINT_ATTF(64, 2) DETINT_ATTF(64, 4) DETINT_ATTF(64, 8)
  DETINT_ATTF(128, 1) DETINT_ATTF(128, 2) DETINT_ATTF(128, 4) DETINT_ATTF(128, 8)
#undef DETINT_ATTF
  return hipErrorInvalidValue;
}

bool attention_supported(int64_t d, int64_t group, int64_t max_pos) {
  if (d != 64 && d != 128) return false;
  if (group != 1 && group != 2 && group != 4 && group != 8) return false;
  return (size_t)group * max_pos * sizeof(int32_t) <= 96 * 1024;
}

hipError_t launch_attention(const int8_t* q8, const int32_t* e_q, const int8_t* kc,
                            const int8_t* vc, const RowMap& rows, int64_t R, int64_t nq,
                            int64_t nkv, int64_t d, int64_t n_slots, int64_t max_pos, int32_t M,
                            int32_t K, int32_t* out, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const int64_t G = nq / nkv;
#define DETINT_ATT(DD, GG)                                                                   \
  if (d == DD && G == GG)                                                                    \
    return launch_t<DD, GG>(q8, e_q, kc, vc, rows, R, nq, nkv, n_slots, max_pos, M, K, out, \
                            st);
  DETINT_ATT(64, 1) DETINT_ATT(64, 2) DETINT_ATT(64, 4) DETINT_ATT(64, 8)
  DETINT_ATT(128, 1) DETINT_ATT(128, 2) DETINT_ATT(128, 4) DETINT_ATT(128, 8)
#undef DETINT_ATT
  return hipErrorInvalidValue;
}

}  // namespace detint
