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

#define DETINT_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int TPB = 256;

__device__ __forceinline__ int sbyte(int w, int b) { return (w << (24 - 8 * b)) >> 24; }

__device__ __forceinline__ int dot16(const v4i& a, const v4i& b, int c) {
  c = __builtin_amdgcn_sdot4(a.x, b.x, c, false);
  c = __builtin_amdgcn_sdot4(a.y, b.y, c, false);
  c = __builtin_amdgcn_sdot4(a.z, b.z, c, false);
  c = __builtin_amdgcn_sdot4(a.w, b.w, c, false);
  return c;
}

// exp_delta in 32-bit arithmetic: v >= 31 * 2^15 (E = 0) exactly when
// delta * M >= T = 31 * 2^(15 + sh) - 2^(sh - 1) + 1, i.e. delta >= d0 =
// ceil(T / M); clamping delta to d0 keeps that outcome and bounds the product
// by T + M < 2^32 when 1 <= sh <= 11 and 2^10 <= M < 2^15 (then d0 < 2^22, so
// one 24-bit multiply is exact, and v < 32 * 2^15 keeps every shift below
// 32). exp32_limit gives d0 for a lane's (M, sh), or 0 when the lane is
// outside that range.
__device__ __forceinline__ uint32_t exp32_limit(int32_t M, int sh) {
  if (sh < 1 || sh > 11 || M < (1 << 10) || M >= (1 << 15)) return 0;
  const uint64_t T = (uint64_t(31) << (15 + sh)) - (uint64_t(1) << (sh - 1)) + 1;
  return (uint32_t)udiv_q<23>(T + (uint64_t)M - 1, (uint64_t)M);  // ceil(T / M) < 2^22
}

// Transposed partial reduction of N int32 values per lane over the lane
// offsets O, O/2, ..., OMIN: each step keeps half of the values and adds the
// partner's copy of them, so N - N / 2^steps exchanges replace
// N * steps. Afterwards lane l holds, in v[0 .. N / (64 / OMIN)), the totals
// (over the lanes that differ from l in those offset bits) of value indices
// base(l) + i, base(l) = sum over steps of bit(l, O_s) * N / 2^(s+1).
template <int N, int O, int OMIN>
struct HalveTo {
  __device__ __forceinline__ static void run(int* v, int lane) {
    if constexpr (O >= OMIN && N > 1) {
      const bool upper = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const int keep = upper ? v[i + N / 2] : v[i];
        const int give = upper ? v[i] : v[i + N / 2];
        v[i] = keep + lane_xor<O>(give);
      }
      HalveTo<N / 2, O / 2, OMIN>::run(v, lane);
    }
  }
};

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
// KU key rows and VU value rows are in flight per thread in passes 1 and 4.
// off(j): byte offset of cached position j from K and V (the same for both).
template <int D, int G, int NT = TPB, int KU = 4, int VU = 8, class Off>
__device__ __forceinline__ void attend(const v4i* sq, const int32_t* eqv, const int8_t* __restrict__ K,
                                       const int8_t* __restrict__ V, int ctx, int ld, int32_t Ms,
                                       int32_t Ks, int32_t* __restrict__ orow, int32_t* sc,
                                       int64_t* red, int32_t (*sred)[G * D], Off off) {
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
  for (; j1 + (KU - 1) * NT < ctx; j1 += KU * NT) {  // KU key rows in flight
    v4i kk[KU][CH];
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) kk[u][cc] = ((const v4i*)(K + off(j1 + u * NT)))[cc];
#pragma unroll
    for (int u = 0; u < KU; ++u) score(kk[u], j1 + u * NT);
  }
  for (; j1 < ctx; j1 += NT) {
    v4i ka[CH];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) ka[cc] = ((const v4i*)(K + off(j1)))[cc];
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
  for (; j + (VU - 1) * RG < ctx; j += VU * RG) {  // VU independent row loads in flight
    v4i vv[VU];
#pragma unroll
    for (int u = 0; u < VU; ++u) vv[u] = *(const v4i*)(V + off(j + u * RG) + c * 16);
#pragma unroll
    for (int u = 0; u < VU; ++u) pv(vv[u], j + u * RG);
  }
  for (; j < ctx; j += RG) pv(*(const v4i*)(V + off(j) + c * 16), j);
  // reduce over the lanes of a wave that share chunk c
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int b = 0; b < 16; ++b) acc[g][b] = xor_sum_from<CH>(acc[g][b]);
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
                                                 int32_t* __restrict__ out, KvPages kp) {
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
  if (!kp.bt) {
    attend<D, G>(sq, seq, kc + base, vc + base, pos + 1, max_pos, Ms, Ks, orow, sc, red, sred,
                 [](int j) { return (int64_t)j * D; });
  } else {
    uint32_t bad = 0;
    attend<D, G>(sq, seq, kc, vc, pos + 1, max_pos, Ms, Ks, orow, sc, red, sred,
                 [&](int j) { return page_row_off(kp, slot, kvh, nkv, D, j, bad); });
    bound_raise(bad);
  }
}

// Decode: one row per sequence. The workgroup of (row, KV head) does the QKV
// post-processing of its own heads (G query heads -> q8 in LDS, the new key
// and value -> int8 into the cache at the row's position and into LDS), then
// attends over positions 0..pos. The row position is the only input the
// cached rows 0..pos-1 depend on, so their first PRE keys and values are
// loaded into registers before the post-processing (its own loads go first:
// loads complete in order) and arrive while it computes; the new row at pos
// is taken from LDS. Later cached rows, if any, are streamed as in `attend`.
// Same passes and the same integer results as `attend`. A workgroup takes G
// of the gq query heads that share a KV head (G = gq, or G = 1 to spread a
// small batch over more CUs; the key and value rows are then written by
// each of the gq workgroups, with identical bytes).
// (qkv is not __restrict__: loads through a restrict-qualified read-only
// pointer may be sunk to their first use, past the cache loads)
template <int D, int G, bool QKN, int NT>
__global__ __launch_bounds__(NT) void attn_decode_fused(
    const int32_t* qkv, QkvPost p, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ slot_arr, int nq, int nkv, int n_slots, int max_pos,
    int8_t* __restrict__ kc, int8_t* __restrict__ vc, int32_t Ms, int32_t Ks,
    int32_t* __restrict__ out, int gq, KvPages kp) {
  constexpr int CH = D / 16;              // 16-byte chunks per row
  constexpr int NW = NT / 64;
  constexpr int PRE = G <= 2 && NT == 256 ? 768 : 512;  // cached rows loaded up front
  constexpr int KU = PRE / NT;           // key rows per thread (one row each)
  constexpr int RG = NT / CH;            // value rows per pass-4 step
  constexpr int VU = PRE / RG;            // value chunks per thread
  constexpr int NH = G + 2;               // heads post-processed here
  constexpr int HR = (NH + NW - 1) / NW;  // rounds of NW waves
  constexpr int half = D / 2;
  extern __shared__ int32_t sc[];         // [G][max_pos]: scores -> E
  __shared__ v4i sq[G * CH];
  __shared__ v4i snew[2 * CH];            // new key row, new value row (int8)
  __shared__ int32_t seq[G];
  __shared__ int64_t rmax[NW][G], rsum[NW][G], rnv[G];
  __shared__ int32_t sred[NW][G * D];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h0 = blockIdx.y * G, kvh = h0 >> (__builtin_ctz(gq));  // gq: a power of two

  // 1. loads of the post-processing, which do not depend on the row's
  //    position: per head this wave handles, lane i < d/2 holds elements i
  //    and i + d/2 (addresses clamped, lanes past d/2 idle)
  const int nh = nq + 2 * nkv;
  const int32_t* row = qkv + (size_t)r * nh * D;
  const bool act = lane < half;
  const int jl = act ? lane : 0;
  int32_t hx0[HR], hx1[HR], hm0[HR], hm1[HR], hg0[HR], hg1[HR];
#pragma unroll
  for (int u = 0; u < HR; ++u) {
    const int t = min(wave + NW * u, NH - 1);
    const int hh = t < G ? h0 + t : (t == G ? nq + kvh : nq + nkv + kvh);
    const int c0 = hh * D;
    hx0[u] = row[c0 + jl];
    hx1[u] = row[c0 + jl + half];
    if (QKN) {
      hm0[u] = p.col_m[c0 + jl];
      hm1[u] = p.col_m[c0 + jl + half];
      const int16_t* gn = t < G ? p.q_norm : p.k_norm;
      hg0[u] = gn[jl];
      hg1[u] = gn[jl + half];
    }
  }
  const int32_t rm = QKN ? p.row_m[r] : 0, rk = QKN ? p.row_k[r] : 0;
  // per-channel key gains of this KV head (2^-g on the query, 2^g on the key)
  int gk0 = 0, gk1 = 0;
  if (p.k_gain) {
    gk0 = p.k_gain[(size_t)kvh * D + jl] & 7;
    gk1 = p.k_gain[(size_t)kvh * D + jl + half] & 7;
  }
  asm volatile("" ::: "memory");  // keep these loads ahead of the ones below
  const int pos = start_pos[r], slot = slot_arr[r];
  int32_t* orow = out + ((size_t)r * nq + h0) * D;
  if (pos < 0 || pos >= max_pos || slot < 0 || slot >= n_slots) {
    for (int t = tid; t < G * D; t += NT) orow[t] = 0;
    return;
  }
  const int nold = pos, ctx = pos + 1, ld = max_pos;
  const int64_t cs = p.cos_t[(size_t)pos * half + jl], sn = p.sin_t[(size_t)pos * half + jl];
  asm volatile("" ::: "memory");

  // 2. cached keys and values 0..min(pos, PRE)-1 into registers. Loads are
  //    issued only where a row lies below pos - per wave for keys, per step
  //    for values and for the first later batch (a uniform test each): a row
  //    past the end would read zeros without touching memory but still cost
  //    the texture unit 16 cycles per load, which on a short context is most
  //    of the preload. Their number thus varies with pos, so the
  //    post-processing inputs are waited for before them (a wait after them
  //    could not count only the older loads); their latency then overlaps
  //    the post-processing arithmetic. Lanes whose row is past the end read
  //    zeros through an out-of-range offset.
#pragma unroll
  for (int u = 0; u < HR; ++u) asm volatile("" ::"v"(hx0[u]), "v"(hx1[u]));
  if (QKN) {
#pragma unroll
    for (int u = 0; u < HR; ++u) asm volatile("" ::"v"(hm0[u]), "v"(hm1[u]), "v"(hg0[u]), "v"(hg1[u]));
  }
  asm volatile("" ::"v"(gk0), "v"(gk1), "v"(cs), "v"(sn));
  // contiguous: a buffer over this (slot, KV head) block, row j at j D;
  // paged: a buffer over the layer's pool, row j where the block table puts it
  const bool paged = kp.bt != nullptr;
  const size_t base = paged ? 0 : ((size_t)slot * nkv + kvh) * max_pos * D;
  const int cbytes = paged ? (kp.n_pages * nkv * D) << kp.shift : max_pos * D;
  uint32_t pbad = 0;
  auto roff = [&](int j) -> int {
    return paged ? (int)page_row_off(kp, slot, kvh, nkv, D, j, pbad) : j * D;
  };
  const __amdgpu_buffer_rsrc_t rsk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kc + base), (short)0, cbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vc + base), (short)0, cbytes, 0x00020000);
  const int c = tid % CH, rg = tid / CH;
  const int wave_row0 = __builtin_amdgcn_readfirstlane(wave * 64);
  const v4i zero4 = {0, 0, 0, 0};
  v4i kpre[KU][CH], vpre[VU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int j = tid + u * NT;
    if (wave_row0 + u * NT < nold) {
      const int off = j < nold ? roff(j) : cbytes;
#pragma unroll
      for (int cc = 0; cc < CH; ++cc)
        kpre[u][cc] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rsk, off + cc * 16, 0, 0));
    } else {
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) kpre[u][cc] = zero4;
    }
  }
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int j = rg + u * RG;
    vpre[u] = u * RG < nold ? __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rsv, j < nold ? roff(j) + c * 16 : cbytes, 0, 0))
                            : zero4;
  }
  // the first batch of later cached keys too (long contexts; rows past the
  // end read zeros without touching memory)
  constexpr int SK = D == 64 && NT == 256 ? 4 : 2;
  v4i ka[SK][CH], kb[SK][CH];
  auto kload = [&](v4i (&kr)[SK][CH], int b0) {
#pragma unroll
    for (int u = 0; u < SK; ++u) {
      const int j = b0 + tid + u * NT;
      const int off = j < nold ? roff(j) : cbytes;
#pragma unroll
      for (int cc = 0; cc < CH; ++cc)
        kr[u][cc] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rsk, off + cc * 16, 0, 0));
    }
  };
  if (PRE < nold) {
    kload(ka, PRE);
  } else {
#pragma unroll
    for (int u = 0; u < SK; ++u)
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) ka[u][cc] = zero4;
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. post-processing (the integer steps of qkv_head): q -> q8, e_q (LDS);
  //    k, v -> int8 at the cache scales, into the cache and LDS
  int8_t* snk = (int8_t*)snew;
  int8_t* snv = (int8_t*)snew + D;
  uint32_t bad = 0;
#pragma unroll
  for (int u = 0; u < HR; ++u) {
    const int t = wave + NW * u;
    if (t >= NH) break;
    const int j0 = lane, j1 = lane + half;
    if (t == G + 1) {  // value head
      const int c0 = (nq + nkv + kvh) * D;
      int8_t* dst = vc + base + roff(pos);
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        int64_t vf = e2 ? hx1[u] : hx0[u];
        if (QKN) vf = R(vf * rm * (e2 ? hm1[u] : hm0[u]), rk + p.col_k - p.f_n);
        if (act) bad |= i32_check(vf);
        const int8_t v8 = clamp8(R(vf * p.vq_m, p.vq_k));
        if (act) {
          dst[e2 ? j1 : j0] = v8;
          snv[e2 ? j1 : j0] = v8;
        }
      }
      (void)c0;
      continue;
    }
    int64_t x0 = act ? hx0[u] : 0, x1 = act ? hx1[u] : 0;
    if (QKN) {
      int64_t a0 = act ? x0 * hm0[u] : 0, a1 = act ? x1 * hm1[u] : 0;
      const int b = wave_bitlen_max(uabs64(a0), uabs64(a1));
      const int sh0 = b > 24 ? b - 24 : 0;
      a0 = R(a0, sh0);
      a1 = R(a1, sh0);
      const int64_t S = wave_sum(a0 * a0 + a1 * a1);
      if (S == 0) {
        x0 = x1 = 0;
      } else {
        int32_t m, sh;
        irms_wave(S, D, m, sh);
        x0 = R(a0 * hg0[u] * m, sh + 12 - p.f_n);
        x1 = R(a1 * hg1[u] * m, sh + 12 - p.f_n);
      }
    }
    int64_t y0 = act ? R(x0 * cs - x1 * sn, 14) : 0;
    int64_t y1 = act ? R(x1 * cs + x0 * sn, 14) : 0;
    bad |= i32_check(y0) | i32_check(y1);  // rotated q / k within int32
    const int g0 = act ? gk0 : 0, g1 = act ? gk1 : 0;
    if (t < G) {
      y0 = R(y0, g0);
      y1 = R(y1, g1);
      const int bl = wave_bitlen_max(uabs64(y0), uabs64(y1));
      const int e = bl > 7 ? bl - 7 : 0;  // dq_exp of the maximum
      int8_t* qd = (int8_t*)sq + t * D;
      if (act) {
        qd[j0] = clamp8(R(y0, e));
        qd[j1] = clamp8(R(y1, e));
      }
      if (lane == 0) seq[t] = e;
    } else if (act) {  // key head
      int8_t* dst = kc + base + roff(pos);
      const int8_t k0 = clamp8(R(y0 * p.kq_m, p.kq_k - g0));
      const int8_t k1 = clamp8(R(y1 * p.kq_m, p.kq_k - g1));
      dst[j0] = k0;
      dst[j1] = k1;
      snk[j0] = k0;
      snk[j1] = k1;
    }
  }
  bound_raise(bad | pbad);
  lds_barrier();

  // 4. pass 1: scores into LDS, per-head maxima
  // scores are int32 (|q . k| <= 2^14 d), and so are the maxima and, below
  // max_pos <= 16384 keys of E <= 2^15, the sums: reductions in 32 bits
  int32_t mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = INT32_MIN;
  auto score = [&](const v4i (&kv)[CH], int j) {
    int s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0;
#pragma unroll
    for (int cc = 0; cc < CH; ++cc)
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = dot16(sq[g * CH + cc], kv[cc], s[g]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sc[g * ld + j] = s[g];
      mx[g] = s[g] > mx[g] ? s[g] : mx[g];
    }
  };
#pragma unroll
  for (int u = 0; u < KU; ++u)
    if (tid + u * NT < nold) score(kpre[u], tid + u * NT);
  if (PRE < nold) {
    // later cached keys in batches of SK rows per thread (the first one is
    // already in flight), two batches in flight (rows past pos read zeros
    // and are skipped); the loop body is straight-line so each wait counts
    // only the older batch
    auto kuse = [&](v4i (&kr)[SK][CH], int b0) {
#pragma unroll
      for (int u = 0; u < SK; ++u)
        if (b0 + tid + u * NT < nold) score(kr[u], b0 + tid + u * NT);
    };
    for (int b0 = PRE; b0 < nold; b0 += 2 * SK * NT) {
      kload(kb, b0 + SK * NT);
      kuse(ka, b0);
      kload(ka, b0 + 2 * SK * NT);
      kuse(kb, b0 + SK * NT);
    }
  }
  if (tid == NT - 1) {  // the new key
    v4i kn[CH];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) kn[cc] = snew[cc];
    score(kn, pos);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int m = wave_max32(mx[g]);
    if (lane == 0) rmax[wave][g] = m;
  }
  lds_barrier();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    int64_t m = rmax[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = rmax[w][g] > m ? rmax[w][g] : m;
    mx[g] = (int32_t)m;
  }

  // the first batch of later cached values, in flight during passes 2-3
  constexpr int SU = NT == 256 ? 8 : 4;
  v4i va[SU], vb[SU];
  auto vload = [&](v4i (&vr)[SU], int b0) {
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int j = b0 + rg + u * RG;
      vr[u] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(rsv, j < nold ? roff(j) + c * 16 : cbytes, 0, 0));
    }
  };
  if (PRE < nold) vload(va, PRE);

  // 5. pass 2: exponentials in place and their sums; 2^46 / D per head
  int32_t den[G];
#pragma unroll
  for (int g = 0; g < G; ++g) den[g] = 0;
  {
    int shg[G];
    bool fast = Ms > 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      shg[g] = __builtin_amdgcn_readfirstlane(Ks - seq[g]);
      fast = fast && shg[g] >= 1 && shg[g] <= 62;
    }
    if (fast) {  // uniform: the branch-free form of DI-Exp (exp_delta)
      for (int j = tid; j < ctx; j += NT) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int32_t E = exp_delta((uint32_t)(mx[g] - sc[g * ld + j]), (uint32_t)Ms, shg[g]);
          sc[g * ld + j] = E;
          den[g] += E;
        }
      }
    } else {
      for (int j = tid; j < ctx; j += NT) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int32_t E = diexp(R(((int64_t)sc[g * ld + j] - mx[g]) * Ms, shg[g]));
          sc[g * ld + j] = E;
          den[g] += E;
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int d = wave_sum32(den[g]);
    if (lane == 0) rsum[wave][g] = d;
  }
  lds_barrier();
  // rn = floor(2^46 / D) per head (D >= 2^15): with one or two heads every
  // wave divides for itself, else one head per wave, in parallel, through LDS
  uint32_t rn[G];
  if constexpr (G <= 2) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      int64_t d = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) d += rsum[w][g];
      rn[g] = (uint32_t)udiv_wave<32>(uint64_t(1) << 46, (uint64_t)d);
    }
  } else {
    for (int g = wave; g < G; g += NW) {
      int64_t d = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) d += rsum[w][g];
      const int64_t q = (int64_t)udiv_wave<32>(uint64_t(1) << 46, (uint64_t)d);
      if (lane == 0) rnv[g] = q;
    }
    lds_barrier();
#pragma unroll
    for (int g = 0; g < G; ++g) rn[g] = (uint32_t)rnv[g];
  }

  // 6. P.V with P = min(R(E rn, 31), 2^15 - 1) formed as each value row is
  //    used (the lanes sharing a row repeat it); a lane owns a 16-byte
  //    chunk c of value rows rg, rg + RG, ...
  int acc[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int b = 0; b < 16; ++b) acc[g][b] = 0;
  auto pv = [&](const v4i& v, int j) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint64_t pp = ((((uint64_t)(uint32_t)sc[g * ld + j] * rn[g]) >> 30) + 1) >> 1;
      const int P = (int)(pp > 32767 ? 32767 : pp);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[g][b] += P * sbyte(v.x, b);
        acc[g][4 + b] += P * sbyte(v.y, b);
        acc[g][8 + b] += P * sbyte(v.z, b);
        acc[g][12 + b] += P * sbyte(v.w, b);
      }
    }
  };
#pragma unroll
  for (int u = 0; u < VU; ++u)
    if (rg + u * RG < nold) pv(vpre[u], rg + u * RG);
  if (PRE < nold) {  // later cached values, as the keys: SU rows per batch, two in flight
    auto vuse = [&](v4i (&vr)[SU], int b0) {
#pragma unroll
      for (int u = 0; u < SU; ++u)
        if (b0 + rg + u * RG < nold) pv(vr[u], b0 + rg + u * RG);
    };
    for (int b0 = PRE; b0 < nold; b0 += 2 * SU * RG) {
      vload(vb, b0 + SU * RG);
      vuse(va, b0);
      vload(va, b0 + 2 * SU * RG);
      vuse(vb, b0 + SU * RG);
    }
  }
  if (rg == RG - 1) pv(snew[CH + c], pos);  // the new value row
  // reduce over the 64 / CH lanes of a wave that share chunk c, transposed:
  // each halving step sends half of the values to the partner lane, so lane
  // l ends with NV / (64 / CH) totals, value indices (l / CH) NV CH / 64 + i;
  // then over waves through LDS
  constexpr int NV = 16 * G, NL = NV * CH / 64;
  int* av = &acc[0][0];
  HalveTo<NV, 32, CH>::run(av, lane);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int vi = (lane / CH) * NL + i, g = vi / 16, b = vi % 16;
    sred[wave][g * D + c * 16 + b] = av[i];
  }
  lds_barrier();
  for (int t = tid; t < G * D; t += NT) {
    int s2 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) s2 += sred[w][t];
    orow[t] = s2;
  }
  bound_raise(pbad);  // pages of the later cached rows
}

// ------------------------------------------------------ prefill on MFMA
//
// Prefill rows of a sequence are consecutive positions, so a workgroup takes
// a block of QP query positions of one sequence and the G query heads of one
// KV head, and walks the causal key range in chunks of 32 keys three times:
//   1. S^T = K . Q^T (v_mfma_i32_32x32x32_i8, exact int32): row maxima;
//   2. recompute S^T; E = DI-Exp(...) as above; D = sum E;
//   3. recompute S^T and E; P = min(R(E floor(2^46 / D), 31), 2^15 - 1);
//      O^T += V^T . P^T on MFMA with P split into int8 limbs:
//      P = 256 Ph + Pl + 128, Ph in [0, 127], Pl in [-128, 127]
//      (DetLLM blog, footnote 8: 15-bit probabilities, P.V as two int8
//      GEMMs), so O = 256 (Ph.V) + (Pl.V) + 128 colsum(V).
// Computing S^T rather than S leaves each lane with 16 keys of one query in
// its accumulator registers (lane l: query l % 32; register r: key
// 8 (r / 4) + 4 (l / 32) + r % 4), which is exactly a 16-byte MFMA operand of
// P^T once the contraction runs over keys in that order; the V^T operand is
// read from the row-major V tile with LDS transpose reads in the same key
// order. Row statistics become per-lane values plus one exchange between the
// two half-waves. Masked keys (past the query's position, or past the
// chunk's end) get P = 0, i.e. Ph = 0, Pl = -128, which the colsum term
// cancels exactly; the column sums are taken over the chunks each wave
// actually multiplies.
template <int G>
struct PfCfg {
  static constexpr int PT = 4 / G;       // 32-position tiles per workgroup
  static constexpr int QP = 32 * PT;     // query positions per workgroup
};

template <int D, int G>
struct PfLds {
  static constexpr int BK = 256;           // keys per staged batch (8 chunks)
  static constexpr int KB = BK * D;        // bytes of K (or V) per batch
  static constexpr int bytes = 4 * KB;     // K and V, each double-buffered
};

// K and V rows in LDS: 16-byte chunk c of key row r sits at chunk c ^ swz(r).
// The 16 rows one MFMA operand read of K touches per LDS cycle then hit 16
// distinct slots of the 256-byte bank window, and the transposed reads of V
// below spread their 128 dwords evenly over the banks (two per bank).
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}

typedef int v2i_t __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b8: within each group of 16 lanes, lane j receives byte
// j % 8 of the 8 bytes read by lanes 2 m + j / 8 (m = 0..7), as byte m.
__device__ __forceinline__ v2i_t lds_read_tr8(const int8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i_t*)(p));
}

// d = 64 fits two workgroups per CU in LDS (64 KiB each): keep the registers
// within 256 so that both are resident
template <int D, int G>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void attn_prefill_mfma(
    const int8_t* __restrict__ q8, const int32_t* __restrict__ e_q, const int8_t* __restrict__ kc,
    const int8_t* __restrict__ vc, const int32_t* __restrict__ cu, const int32_t* __restrict__ start,
    const int32_t* __restrict__ seq_slot, int nq, int nkv, int n_slots, int max_pos, int nblk,
    int32_t Ms, int32_t Ks, int32_t* __restrict__ out, KvPages kp) {
  constexpr int QP = PfCfg<G>::QP, KS = D / 32, CPR = D / 16;
  using L = PfLds<D, G>;
  constexpr int BK = L::BK, KB = L::KB;
  constexpr int LPB = KB / 4096;  // DMA loads per thread per batch and operand
  extern __shared__ __attribute__((aligned(1024))) int8_t smem[];
  int8_t* sK = smem;                 // [2][KB]
  int8_t* sV = smem + 2 * KB;        // [2][KB]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, ql = lane & 31;
  const int qb = nblk - 1 - (int)blockIdx.x, sq = blockIdx.y, kvh = blockIdx.z;
  const int r0 = cu[sq], len = cu[sq + 1] - r0;
  if (qb * QP >= len) return;
  const int p0 = start[sq], slot = seq_slot[sq];
  const int nrow = min(QP, len - qb * QP);
  const int hq = kvh * G + wave % G, qi = (wave / G) * 32 + ql;
  const int row = r0 + qb * QP + qi, pos = p0 + qb * QP + qi;
  const bool rvalid = qi < nrow;
  int32_t* orow = out + ((size_t)row * nq + hq) * D;
  if (slot < 0 || slot >= n_slots) {
    if (rvalid)
      for (int d = hh; d < D; d += 2) orow[d] = 0;  // lanes l and l + 32 split the row
    return;
  }
  const bool live = rvalid && pos >= 0 && pos < max_pos;
  const int kend = min(p0 + qb * QP + nrow, max_pos);
  const int nch = (kend + 31) >> 5, nbt = (kend + BK - 1) / BK;
  // contiguous: a buffer over this (slot, KV head) block; paged: over the
  // layer's pool, each key row where the block table puts it
  const bool paged = kp.bt != nullptr;
  const size_t base = paged ? 0 : ((size_t)slot * nkv + kvh) * max_pos * D;
  const int cbytes = paged ? (kp.n_pages * nkv * D) << kp.shift : max_pos * D;
  uint32_t pbad = 0;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + base), (short)0,
                                                                      cbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + base), (short)0,
                                                                      cbytes, 0x00020000);
  // batch bt of K and, for pass 3, V (both swizzled) into buffer bt & 1:
  // load q of thread t moves chunk g = 256 q + t, LDS bytes [16 g, 16 g + 16)
  auto issue = [&](int bt, bool withv) {
    const int buf = bt & 1;
#pragma unroll
    for (int q = 0; q < LPB; ++q) {
      const int g = q * 256 + tid, r = g / CPR, ph = g % CPR;
      const int key = bt * BK + r;
      const int goff = !paged ? key * D
                              : (key < kend ? (int)page_row_off(kp, slot, kvh, nkv, D, key, pbad) : cbytes);
      // a template call written straight into the builtin's argument list
      // leaves the kernel uninstantiated on the host side (no host stub)
      const int soff = goff + ((ph ^ kswz<D>(r)) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, DETINT_LDS(sK + buf * KB + (q * 256 + wave * 64) * 16),
                                               16, soff, 0, 0, 0);
      if (withv)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, DETINT_LDS(sV + buf * KB + (q * 256 + wave * 64) * 16),
                                                 16, soff, 0, 0, 0);
    }
  };

  v4i qf[KS];
  const v4i z4 = {0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = rvalid ? *(const v4i*)(q8 + ((size_t)row * nq + hq) * D + 32 * ks + 16 * hh) : z4;
  const int sh = Ks - (rvalid ? e_q[(size_t)row * nq + hq] : 0);
  const bool fast = sh >= 1 && sh <= 62 && Ms > 0;
  const uint32_t d0 = exp32_limit(Ms, sh);
  const bool wfast32 = __all(d0 != 0);  // every lane of the wave on the 32-bit form
  // chunks below every query of this wave's tile need no causal mask
  const int pmin = p0 + qb * QP + (wave / G) * 32;

  // S^T of chunk c (keys 32 c ..) from the staged batch: its K fragments,
  // then the MFMAs on them
  auto kfrag = [&](int c, v4i (&kf)[KS]) {
    const int8_t* kb = sK + ((c / (BK / 32)) & 1) * KB;
    const int r = (c * 32) % BK + ql;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const v4i*)(kb + r * D + (((2 * ks + hh) ^ kswz<D>(r)) << 4));
  };
  auto smma = [&](const v4i (&kf)[KS]) {
    v16i acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[ks], qf[ks], acc, 0, 0, 0);
    return acc;
  };
  // key offset within its chunk of accumulator register r
  auto koff = [&](int r) { return 8 * (r >> 2) + 4 * hh + (r & 3); };
  // Each pass walks the chunks with batches staged one ahead: at a batch's
  // start, wait for it, then a barrier (which also retires every wave's
  // reads of the buffer the next issue overwrites), then issue the next.
  auto batch_begin = [&](int bt, bool withv) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (bt + 1 < nbt) issue(bt + 1, withv);
  };
  auto sweep_end = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  constexpr int CPB = BK / 32;  // chunks per batch

  // Every pass takes a batch's chunks with their scores one chunk ahead and
  // their K fragments two ahead: the MFMAs of chunk c + 1 and the LDS reads
  // of chunk c + 2 are issued before chunk c's integer work, which then runs
  // under them (near the batch's end the last chunk is taken again).
  auto sweep = [&](bool withv, auto body) {
    issue(0, withv);
    for (int bt = 0; bt < nbt; ++bt) {
      batch_begin(bt, withv);
      const int c0 = bt * CPB, c1 = min(nch, (bt + 1) * CPB);
      v4i kn[KS];
      kfrag(c0, kn);
      v16i sacc = smma(kn);
      kfrag(min(c0 + 1, c1 - 1), kn);
      for (int c = c0; c < c1; ++c) {
        const v16i snext = smma(kn);
        kfrag(min(c + 2, c1 - 1), kn);
        body(c, sacc);
        sacc = snext;
      }
    }
    sweep_end();
  };

  // pass 1: maxima. Its per-chunk work (16 maxima) is too short to cover a
  // chunk's two chained MFMAs, so chunks go in pairs: both pairs' MFMA
  // chains issued together, the next pair's K fragments read under them.
  int mx = INT32_MIN;
  auto max_chunk = [&](int c, const v16i& sacc) {
    if (c * 32 + 31 <= pmin) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = max(mx, sacc[r]);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (c * 32 + koff(r) <= pos) mx = max(mx, sacc[r]);
    }
  };
  issue(0, false);
  for (int bt = 0; bt < nbt; ++bt) {
    batch_begin(bt, false);
    const int c0 = bt * CPB, c1 = min(nch, (bt + 1) * CPB);
    v4i ka[KS], kb[KS];
    kfrag(c0, ka);
    kfrag(min(c0 + 1, c1 - 1), kb);
    for (int c = c0; c < c1; c += 2) {
      const v16i sa = smma(ka), sb = smma(kb);
      kfrag(min(c + 2, c1 - 1), ka);
      kfrag(min(c + 3, c1 - 1), kb);
      max_chunk(c, sa);
      if (c + 1 < c1) max_chunk(c + 1, sb);
    }
  }
  sweep_end();
  mx = max(mx, lane_xor<32>(mx));
  if (!live) mx = 0;  // its values are never used; keep the arithmetic tame

  // E(s) = DI-Exp(R((s - mx) Ms, sh)) for s <= mx. The 32-bit form is
  // exp_delta of mx - s with the clamp at d0 moved onto the score: v =
  // (mx - max(s, mx - d0)) Ms + 2^(sh-1) - 1, shifted by sh, evaluated as
  // C - max(s, slo) Ms mod 2^32 (its value is below 2^31); then n = v >> 15
  // <= 31, f = (2^16 - v mod 2^15) >> 1 = 2^15 - R(v mod 2^15, 1), and
  // E = R(f, n), which is 0 from n = 17 on. Other waves take the 64-bit
  // forms.
  // Per score: one 24-bit multiply-add gives x = C - max(s, slo) Ms, then
  // n = x >> (sh + 15) and v mod 2^15 = bits sh .. sh + 14 of x.
  const int32_t slo = mx - (int32_t)d0;
  const uint32_t c32 = (uint32_t)mx * (uint32_t)Ms + ((1u << ((sh - 1) & 31)) - 1u);
  const int32_t nMs = -Ms;
  const uint32_t sh15 = (uint32_t)(sh + 15) & 31u, shb = (uint32_t)sh & 31u;
  auto e32 = [&](int32_t s) -> uint32_t {
    const uint32_t x = (uint32_t)__mul24(max(s, slo), nMs) + c32;
    const uint32_t n = x >> sh15, f = (65536u - __builtin_amdgcn_ubfe(x, shb, 15u)) >> 1;
    return (f + ((1u << n) >> 1)) >> n;
  };
  // E = 0 exactly when v >= 16 2^15 + 1 (n = 16 leaves 1 only for v mod
  // 2^15 = 0), i.e. when (mx - s) Ms >= T1 = (2^19 + 1) 2^sh - 2^(sh-1) + 1:
  // for s <= szero = mx - ceil(T1 / Ms). On the 32-bit form (sh <= 11,
  // 2^10 <= Ms) T1 < 2^31 and the quotient is below 2^21.
  const int shz = d0 != 0 ? sh : 1;  // keeps the shifts in range on the other lanes
  const uint64_t Mz = d0 != 0 ? (uint64_t)Ms : 1u << 10;
  const int32_t szero = d0 != 0 ? mx - (int32_t)udiv_q<21>(((uint64_t)524289 << shz) -
                                                               (uint64_t(1) << (shz - 1)) + Mz, Mz)
                                : INT32_MIN;
  auto e64 = [&](int32_t s) -> uint32_t {
    return (uint32_t)(fast ? exp_delta((uint32_t)(mx - s), (uint32_t)Ms, sh)
                           : diexp(R(((int64_t)s - mx) * Ms, sh)));
  };
  // A chunk's 32 x 32 tile is dead when every exponential in it is 0. E
  // does not increase as the score falls (Ms > 0), so E at the lane's
  // largest score of the chunk being 0 (masked keys included, and that
  // score no larger than the row maximum) clears the lane's 16 keys; lanes
  // without a live query are dead. A wave skips a dead tile in passes 2
  // and 3: it adds nothing to D, to P.V or to the column sums below.
  auto dead = [&](const v16i& sacc, auto ef) {
    int32_t cm = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) cm = max(cm, sacc[r]);
    if constexpr (std::is_same_v<decltype(ef), decltype(e32)>)
      return __all(!live || cm <= szero);  // the same test through the threshold
    else
      return __all(!live || (Ms > 0 && cm <= mx && ef(cm) == 0u));
  };

  // pass 2: sum of exponentials
  int64_t den = 0;
  auto sum_chunk = [&](int c, const v16i& sacc, auto ef) {
    uint32_t part = 0;  // 16 terms of at most 2^15
    if (c * 32 + 31 <= pmin) {
#pragma unroll
      for (int r = 0; r < 16; ++r) part += ef(sacc[r]);
    } else {
      const int lim = pos - c * 32;  // key offsets <= lim are causal
#pragma unroll
      for (int r = 0; r < 16; ++r) part += koff(r) <= lim ? ef(sacc[r]) : 0u;
    }
    den += part;
  };
  sweep(false, [&](int c, const v16i& sacc) {
    if (wfast32) {
      if (!dead(sacc, e32)) sum_chunk(c, sacc, e32);
    } else if (!dead(sacc, e64)) {
      sum_chunk(c, sacc, e64);
    }
  });
  den += lane_xor<32>(den);
  if (!live) den = 0;
  const uint32_t rn = den > 0 ? (uint32_t)udiv_q<32>(uint64_t(1) << 46, (uint64_t)den) : 0u;  // D >= 2^15
  // P = min(R(E rn, 31), 2^15 - 1) from 24-bit products: with rn = 2^16 rh
  // + rl, E rn + 2^30 = 2^16 (E rh + (t >> 16)) + (t mod 2^16) for t = E rl
  // + 2^30 < 2^32 (E <= 2^15, rl < 2^16), so R(E rn, 31) = (E rh + (t >>
  // 16)) >> 15. Rows without a live query have rn = 0, hence P = 0.
  const uint32_t rh = rn >> 16, rl = rn & 0xFFFFu;
  auto pr = [&](uint32_t E) -> uint32_t {
    const uint32_t t = __umul24(E, rl) + (1u << 30);
    return min((__umul24(E, rh) + (t >> 16)) >> 15, 32767u);
  };

  // pass 3: probabilities and P.V, O^T += V^T . P^T. The V^T operand of
  // d-tile t comes from two transposed reads of the staged V rows: in the
  // group of 16 lanes g = lane / 16 (query columns 16 (g % 2) .., keys of
  // half-wave g / 2), lanes 2 m and 2 m + 1 read the two 8-byte halves of
  // d = 32 t + 16 (g % 2) .. + 15 in the row of key 8 (m / 4) + 4 (g / 2) +
  // m % 4 (+ 16 for the second read), so lane j of the group receives d =
  // 32 t + 16 (g % 2) + j at the 16 keys its P^T operand bytes stand for.
  // The same bytes give this wave's column sums of V over the chunks it
  // processes, for d = 32 t + lane % 32 (half of the keys in each half-wave).
  int voff[2][KS];
  {
    const int g = lane >> 4, i = lane & 15, m = i >> 1;
    const int key = 8 * (m >> 2) + 4 * hh + (m & 3);
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int l2 = 0; l2 < 2; ++l2)
        voff[l2][t] = (key + 16 * l2) * D + (((2 * t + (g & 1)) ^ kswz<D>(key)) << 4) + 8 * (i & 1);
  }
  v16i oh[KS], ol[KS];
  int cs[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    cs[t] = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) oh[t][r] = ol[t][r] = 0;
  }
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  auto pv_chunk = [&](int c, const v16i& sacc, auto ef) {
    // V^T fragments first: the LDS reads complete under the P arithmetic
    const int8_t* vb = sV + ((c / CPB) & 1) * KB + ((c * 32) % BK) * D;
    v2i_t vlo[KS], vhi[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      vlo[t] = lds_read_tr8(vb + voff[0][t]);
      vhi[t] = lds_read_tr8(vb + voff[1][t]);
    }
    uint32_t P[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) P[r] = pr(ef(sacc[r]));
    if (c * 32 + 31 > pmin) {
      const int lim = pos - c * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) P[r] = koff(r) <= lim ? P[r] : 0u;
    }
    // limbs, byte r of a fragment = register r: Ph = P >> 8, Pl = (P & 255) - 128
    v4i fph, fpl;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const uint32_t p01 = P[4 * r4] | (P[4 * r4 + 1] << 16), p23 = P[4 * r4 + 2] | (P[4 * r4 + 3] << 16);
      fph[r4] = (int)__builtin_amdgcn_perm(p23, p01, 0x07050301u);
      fpl[r4] = (int)(__builtin_amdgcn_perm(p23, p01, 0x06040200u) ^ 0x80808080u);
    }
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const v4i fv = {vlo[t].x, vlo[t].y, vhi[t].x, vhi[t].y};
      oh[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fv, fph, oh[t], 0, 0, 0);
      ol[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fv, fpl, ol[t], 0, 0, 0);
      cs[t] = dot16(fv, ones, cs[t]);
    }
  };
  sweep(true, [&](int c, const v16i& sacc) {
    if (wfast32) {
      if (!dead(sacc, e32)) pv_chunk(c, sacc, e32);
    } else if (!dead(sacc, e64)) {
      pv_chunk(c, sacc, e64);
    }
  });
  // the wave's column sums into LDS (the K/V buffers are free now), d-major
  int32_t* s_cs = (int32_t*)smem + wave * D;
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    const int tot = cs[t] + lane_xor<32>(cs[t]);
    if (hh == 0) s_cs[32 * t + ql] = tot;
  }
  __syncthreads();
  bound_raise(pbad);
  if (!rvalid) return;
  // O^T layout: lane l holds query l % 32; register r of d-tile t is
  // d = 32 t + 8 (r / 4) + 4 (l / 32) + r % 4
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int db = 32 * t + 8 * r4 + 4 * hh;
      v4i o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * r4 + i;
        o[i] = live ? (int)(256 * (int64_t)oh[t][r] + ol[t][r] + 128 * (int64_t)s_cs[db + i]) : 0;
      }
      *(v4i*)(orow + db) = o;
    }
}

template <int D, int G>
hipError_t launch_pf(const int8_t* q8, const int32_t* e_q, const int8_t* kc, const int8_t* vc,
                     const RowMap& seqs, int64_t max_seqlen, int64_t nq, int64_t nkv,
                     int64_t n_slots, int64_t max_pos, int32_t M, int32_t K, int32_t* out,
                     hipStream_t st, KvPages kp) {
  constexpr int lds = PfLds<D, G>::bytes;
  const hipError_t err = set_max_lds((const void*)attn_prefill_mfma<D, G>, lds);
  if (err != hipSuccess) return err;
  const int nblk = (int)((max_seqlen + PfCfg<G>::QP - 1) / PfCfg<G>::QP);
  attn_prefill_mfma<D, G><<<dim3((unsigned)nblk, (unsigned)seqs.S, (unsigned)nkv), 256, lds, st>>>(
      q8, e_q, kc, vc, seqs.cu, seqs.start, seqs.seq_slot, (int)nq, (int)nkv, (int)n_slots,
      (int)max_pos, nblk, M, K, out, kp);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_t(const int8_t* q8, const int32_t* e_q, const int8_t* kc, const int8_t* vc,
                    const RowMap& rows, int64_t R, int64_t nq, int64_t nkv, int64_t n_slots,
                    int64_t max_pos, int32_t M, int32_t K, int32_t* out, hipStream_t st,
                    KvPages kp) {
  const size_t lds = (size_t)G * max_pos * sizeof(int32_t);
  const hipError_t err = set_max_lds((const void*)attn_rows<D, G>, 96 * 1024);
  if (err != hipSuccess) return err;
  attn_rows<D, G><<<dim3((unsigned)R, (unsigned)nkv), TPB, lds, st>>>(
      q8, e_q, kc, vc, rows, (int)nq, (int)nkv, (int)n_slots, (int)max_pos, M, K, out, kp);
  return hipGetLastError();
}

template <int D, int G, int NT>
hipError_t launch_fused_g(const int32_t* qkv, const QkvPost& p, const int32_t* start_pos,
                          const int32_t* slot, int64_t B, int64_t nq, int64_t nkv, int64_t n_slots,
                          int64_t max_pos, int8_t* kc, int8_t* vc, int32_t M, int32_t K, int32_t* out,
                          hipStream_t st, KvPages kp) {
  const size_t lds = (size_t)G * max_pos * sizeof(int32_t);
  hipError_t err = set_max_lds((const void*)attn_decode_fused<D, G, true, NT>, 96 * 1024);
  if (err == hipSuccess) err = set_max_lds((const void*)attn_decode_fused<D, G, false, NT>, 96 * 1024);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)B, (unsigned)(nq / G));
  const int gq = (int)(nq / nkv);
  if (p.qk_norm)
    attn_decode_fused<D, G, true, NT><<<grid, NT, lds, st>>>(qkv, p, start_pos, slot, (int)nq, (int)nkv,
                                                         (int)n_slots, (int)max_pos, kc, vc, M, K,
                                                         out, gq, kp);
  else
    attn_decode_fused<D, G, false, NT><<<grid, NT, lds, st>>>(qkv, p, start_pos, slot, (int)nq, (int)nkv,
                                                          (int)n_slots, (int)max_pos, kc, vc, M, K,
                                                          out, gq, kp);
  return hipGetLastError();
}

// A workgroup per (row, KV head) from 128 such pairs up, else one per (row,
// query head): a small batch has few workgroups' worth of work and is
// latency-bound, so halving or quartering each workgroup's arithmetic
// matters more than reading the cache rows once (batch 8 with 8 KV heads:
// 4.7% faster decode steps with a workgroup per query head). A single
// 128-wide head takes 512 threads: its passes are latency chains, and twice
// the waves halve each one (batch 1: 4.9% faster steps, batch 8: 2.8%).
template <int D, int G>
hipError_t launch_fused_t(const int32_t* qkv, const QkvPost& p, const int32_t* start_pos,
                          const int32_t* slot, int64_t B, int64_t nq, int64_t nkv, int64_t n_slots,
                          int64_t max_pos, int8_t* kc, int8_t* vc, int32_t M, int32_t K, int32_t* out,
                          hipStream_t st, KvPages kp) {
  if (G > 1 && B * nkv < 128)
    return launch_fused_g<D, 1, D == 128 ? 512 : 256>(qkv, p, start_pos, slot, B, nq, nkv, n_slots,
                                                      max_pos, kc, vc, M, K, out, st, kp);
  // four heads per workgroup with 64-wide heads: the passes are
  // VALU-bound, so two waves per SIMD instead of one
  constexpr int NT = D == 64 && G == 4 ? 512 : 256;
  return launch_fused_g<D, G, NT>(qkv, p, start_pos, slot, B, nq, nkv, n_slots, max_pos, kc, vc, M,
                                  K, out, st, kp);
}

}  // namespace

DETINT_BOUND_READER(bound_flags_attention)

hipError_t launch_attention_decode_fused(const int32_t* qkv, const QkvPost& p,
                                         const int32_t* start_pos, const int32_t* slot, int64_t B,
                                         int64_t nq, int64_t nkv, int64_t d, int64_t n_slots,
                                         int64_t max_pos, int8_t* kc, int8_t* vc, int32_t M,
                                         int32_t K, int32_t* out, hipStream_t st, KvPages kp) {
  if (B == 0) return hipSuccess;
  const int64_t G = nq / nkv;
#define DETINT_ATTF(DD, GG)                                                                      \
  if (d == DD && G == GG)                                                                        \
    return launch_fused_t<DD, GG>(qkv, p, start_pos, slot, B, nq, nkv, n_slots, max_pos, kc, vc, \
                                  M, K, out, st, kp);
  DETINT_ATTF(64, 1) DETINT_ATTF(64, 2) DETINT_ATTF(64, 4) DETINT_ATTF(64, 8)
  DETINT_ATTF(128, 1) DETINT_ATTF(128, 2) DETINT_ATTF(128, 4) DETINT_ATTF(128, 8)
#undef DETINT_ATTF
  return hipErrorInvalidValue;
}

hipError_t launch_attention_seqs(const int8_t* q8, const int32_t* e_q, const int8_t* kc,
                                 const int8_t* vc, const RowMap& seqs, int64_t R,
                                 int64_t max_seqlen, int64_t nq, int64_t nkv, int64_t d,
                                 int64_t n_slots, int64_t max_pos, int32_t M, int32_t K,
                                 int32_t* out, hipStream_t st, KvPages kp) {
  if (R == 0) return hipSuccess;
  const int64_t G = nq / nkv;
  if (max_seqlen >= 16) {
#define DETINT_PF(DD, GG)                                                                     \
    if (d == DD && G == GG)                                                                   \
      return launch_pf<DD, GG>(q8, e_q, kc, vc, seqs, max_seqlen, nq, nkv, n_slots, max_pos, M, \
                               K, out, st, kp);
    DETINT_PF(64, 1) DETINT_PF(64, 2) DETINT_PF(64, 4)
    DETINT_PF(128, 1) DETINT_PF(128, 2) DETINT_PF(128, 4)
#undef DETINT_PF
  }
  return launch_attention(q8, e_q, kc, vc, seqs, R, nq, nkv, d, n_slots, max_pos, M, K, out, st, kp);
}

bool attention_supported(int64_t d, int64_t group, int64_t max_pos) {
  if (d != 64 && d != 128) return false;
  if (group != 1 && group != 2 && group != 4 && group != 8) return false;
  return (size_t)group * max_pos * sizeof(int32_t) <= 96 * 1024;
}

hipError_t launch_attention(const int8_t* q8, const int32_t* e_q, const int8_t* kc,
                            const int8_t* vc, const RowMap& rows, int64_t R, int64_t nq,
                            int64_t nkv, int64_t d, int64_t n_slots, int64_t max_pos, int32_t M,
                            int32_t K, int32_t* out, hipStream_t st, KvPages kp) {
  if (R == 0) return hipSuccess;
  const int64_t G = nq / nkv;
#define DETINT_ATT(DD, GG)                                                                   \
  if (d == DD && G == GG)                                                                    \
    return launch_t<DD, GG>(q8, e_q, kc, vc, rows, R, nq, nkv, n_slots, max_pos, M, K, out, \
                            st, kp);
  DETINT_ATT(64, 1) DETINT_ATT(64, 2) DETINT_ATT(64, 4) DETINT_ATT(64, 8)
  DETINT_ATT(128, 1) DETINT_ATT(128, 2) DETINT_ATT(128, 4) DETINT_ATT(128, 8)
#undef DETINT_ATT
  return hipErrorInvalidValue;
}

}  // namespace detint
