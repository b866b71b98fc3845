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

template <int D, int G>
__global__ __launch_bounds__(TPB) void attn_rows(const int8_t* __restrict__ q8,
                                                 const int32_t* __restrict__ e_q,
                                                 const int8_t* __restrict__ kc,
                                                 const int8_t* __restrict__ vc, RowMap rows,
                                                 int nq, int nkv, int n_slots, int max_pos,
                                                 int32_t Ms, int32_t Ks,
                                                 int32_t* __restrict__ out) {
  constexpr int CH = D / 16;        // 16-byte chunks per row
  constexpr int RG = TPB / CH;      // V rows in flight per pass-4 step
  extern __shared__ int32_t sc[];   // [G][max_pos]: scores -> E
  __shared__ v4i sq[G * CH];
  __shared__ int64_t red[16];
  __shared__ int32_t sred[TPB / 64][G * D];

  const int r = blockIdx.x, kvh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h0 = kvh * G;
  int pos, slot;
  row_info(rows, r, pos, slot);
  int32_t* orow = out + ((size_t)r * nq + h0) * D;
  if (pos < 0 || pos >= max_pos || slot < 0 || slot >= n_slots) {
    for (int t = tid; t < G * D; t += TPB) orow[t] = 0;
    return;
  }
  const int ctx = pos + 1;
  const size_t base = ((size_t)slot * nkv + kvh) * max_pos * D;
  const int8_t* K = kc + base;
  const int8_t* V = vc + base;
  if (tid < G * CH) sq[tid] = *(const v4i*)(q8 + ((size_t)r * nq + h0) * D + tid * 16);
  __syncthreads();

  // pass 1: scores and per-head max
  int64_t mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = INT64_MIN;
  for (int j = tid; j < ctx; j += TPB) {
    const v4i* kr = (const v4i*)(K + (size_t)j * D);
    int s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const v4i kv = kr[c];
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = dot16(sq[g * CH + c], kv, s[g]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sc[g * max_pos + j] = s[g];
      mx[g] = s[g] > mx[g] ? s[g] : mx[g];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = block_max(mx[g], red);

  // pass 2: exponentials and their sum
  int sh[G];
  int64_t den[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    sh[g] = Ks - e_q[(size_t)r * nq + h0 + g];
    den[g] = 0;
  }
  for (int j = tid; j < ctx; j += TPB) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int32_t E = diexp(R(((int64_t)sc[g * max_pos + j] - mx[g]) * Ms, sh[g]));
      sc[g * max_pos + j] = E;
      den[g] += E;
    }
  }
  int64_t rn[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    den[g] = block_sum(den[g], red);  // also orders pass-2 LDS writes before pass 4
    rn[g] = (int64_t)udiv_q<32>(uint64_t(1) << 46, (uint64_t)den[g]);  // D >= 2^15
  }

  // passes 3+4: probabilities and P.V
  const int c = tid % CH, rg = tid / CH;
  int acc[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int b = 0; b < 16; ++b) acc[g][b] = 0;
  for (int j = rg; j < ctx; j += RG) {
    const v4i v = *(const v4i*)(V + (size_t)j * D + c * 16);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      int64_t p = R((int64_t)sc[g * max_pos + j] * rn[g], 31);
      const int P = (int)(p > 32767 ? 32767 : p);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[g][b] += P * sbyte(v.x, b);
        acc[g][4 + b] += P * sbyte(v.y, b);
        acc[g][8 + b] += P * sbyte(v.z, b);
        acc[g][12 + b] += P * sbyte(v.w, b);
      }
    }
  }
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
  for (int t = tid; t < G * D; t += TPB) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < TPB / 64; ++w) s += sred[w][t];
    orow[t] = s;
  }
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

}  // namespace

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
