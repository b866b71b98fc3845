// Row kernels of libdetint for gfx950: DI-RMSNorm, per-token DQ, integer
// RoPE, DI-Softmax, DI-SwiGLU, embedding, QKV post-processing with the int8
// KV-cache writes, greedy argmax. One workgroup (or wave) per row; row
// statistics (sum of squares, absolute maximum, exponential sums) are exact
// int64 reductions across lanes with shuffles and LDS, so their order cannot
// matter (DetLLM README, "Why ...": integer sums are associative).
#include "dev_int.h"
#include "internal.h"
#include "qkv_dev.h"

namespace detint {
namespace {

constexpr int TPB = 256;

// DI-RMSNorm (DetLLM README "Layout", ops/): x8 * m * 2^-k ~ h * g/2^12 / rms(h).
__global__ __launch_bounds__(TPB) void rmsnorm_k(const int32_t* __restrict__ h,
                                                 const int32_t* __restrict__ row_index,
                                                 const int16_t* __restrict__ g, int n,
                                                 int8_t* __restrict__ x8,
                                                 int32_t* __restrict__ rm,
                                                 int32_t* __restrict__ rk) {
  __shared__ int64_t red[16];
  const int r = blockIdx.x;
  const int src = row_index ? row_index[r] : r;
  const int32_t* hr = h + (size_t)src * n;
  int64_t S = 0, A = 0;
  for (int i = threadIdx.x; i < n; i += TPB) {
    const int64_t v = hr[i];
    S += v * v;
    const int64_t p = (int64_t)uabs64(v * g[i]);
    A = p > A ? p : A;
  }
  S = block_sum(S, red);
  A = block_max(A, red);
  if (threadIdx.x == 0) bound_raise((uint64_t)S >> 62 ? kBoundNorm : 0u);
  int8_t* xr = x8 + (size_t)r * n;
  if (S == 0) {
    for (int i = threadIdx.x; i < n; i += TPB) xr[i] = 0;
    if (threadIdx.x == 0) {
      rm[r] = 1 << 14;
      rk[r] = 26;
    }
    return;
  }
  int32_t m, sh;
  irms_wave(S, n, m, sh);
  const int e = dq_exp((uint64_t)A);
  for (int i = threadIdx.x; i < n; i += TPB) xr[i] = clamp8(R((int64_t)hr[i] * g[i], e));
  if (threadIdx.x == 0) {
    rm[r] = m;
    rk[r] = sh + 12 - e;
  }
}

// Row-in-registers forms of the row kernels (n % 4 == 0, n <= 4 NT U, 16-byte
// aligned rows): thread t owns elements u 4 NT + 4 t .. + 3 for u < U. Every
// load is issued before any is used (clamped addresses, so none sits behind
// a branch; elements past n are zeroed afterwards) and the second pass works
// on the registers instead of re-reading the row. Same integer results as
// the loop forms above and below.
template <int NT, int U>
struct RowRegs {
  __device__ __forceinline__ static int first(int u) { return u * 4 * NT + 4 * (int)threadIdx.x; }
  __device__ __forceinline__ static int at(int u, int n) { return min(first(u), n - 4); }
};

__device__ __forceinline__ uint32_t pack4(int64_t a, int64_t b, int64_t c, int64_t d) {
  return (uint32_t)(uint8_t)clamp8(a) | (uint32_t)(uint8_t)clamp8(b) << 8 |
         (uint32_t)(uint8_t)clamp8(c) << 16 | (uint32_t)(uint8_t)clamp8(d) << 24;
}

template <int U>
__global__ __launch_bounds__(TPB) void rmsnorm_rk(const int32_t* __restrict__ h,
                                                  const int32_t* __restrict__ row_index,
                                                  const int16_t* __restrict__ g, int n,
                                                  int8_t* __restrict__ x8,
                                                  int32_t* __restrict__ rm,
                                                  int32_t* __restrict__ rk) {
  using RR = RowRegs<TPB, U>;
  __shared__ int64_t red[32];
  const int r = blockIdx.x;
  const int src = row_index ? row_index[r] : r;
  const int32_t* hr = h + (size_t)src * n;
  v4i hv[U];
  int2 gw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    hv[u] = *(const v4i*)(hr + RR::at(u, n));
    gw[u] = *(const int2*)(g + RR::at(u, n));
  }
  int64_t v[U][4], gv[U][4], S = 0;
  uint64_t A = 0;  // OR of the magnitudes: the bit length of their maximum
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool ok = RR::first(u) < n;
    v[u][0] = ok ? hv[u].x : 0; v[u][1] = ok ? hv[u].y : 0;
    v[u][2] = ok ? hv[u].z : 0; v[u][3] = ok ? hv[u].w : 0;
    gv[u][0] = (int16_t)(gw[u].x & 0xFFFF); gv[u][1] = (int16_t)(gw[u].x >> 16);
    gv[u][2] = (int16_t)(gw[u].y & 0xFFFF); gv[u][3] = (int16_t)(gw[u].y >> 16);
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      S += v[u][e4] * v[u][e4];
      A |= uabs64(v[u][e4] * gv[u][e4]);
    }
  }
  int B = bitlen64(A);
  block_sum_maxbits(S, B, red);
  if (threadIdx.x == 0) bound_raise((uint64_t)S >> 62 ? kBoundNorm : 0u);
  int8_t* xr = x8 + (size_t)r * n;
  int32_t m = 1 << 14, sh = 26;
  int e = 0;
  if (S != 0) {
    irms_wave(S, n, m, sh);
    e = B > 7 ? B - 7 : 0;  // dq_exp of the largest magnitude
    sh = sh + 12 - e;
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (RR::first(u) < n)  // an all-zero row quantises to zeros with e = 0
      *(uint32_t*)(xr + RR::first(u)) =
          pack4(R_nn(v[u][0] * gv[u][0], e), R_nn(v[u][1] * gv[u][1], e),
                R_nn(v[u][2] * gv[u][2], e), R_nn(v[u][3] * gv[u][3], e));
  if (threadIdx.x == 0) {
    rm[r] = m;
    rk[r] = sh;
  }
}

template <int U>
__global__ __launch_bounds__(TPB) void requant_rk(const int32_t* __restrict__ y, int n,
                                                  int8_t* __restrict__ q, int32_t* row_e,
                                                  int32_t* row_m, int32_t* row_k, int32_t fm,
                                                  int32_t fk) {
  using RR = RowRegs<TPB, U>;
  __shared__ int64_t red[16];
  const int r = blockIdx.x;
  const int32_t* yr = y + (size_t)r * n;
  v4i yv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) yv[u] = *(const v4i*)(yr + RR::at(u, n));
  int64_t A = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool ok = RR::first(u) < n;
    if (!ok) yv[u] = v4i{0, 0, 0, 0};
    const uint64_t a = uabs64(yv[u].x) > uabs64(yv[u].y) ? uabs64(yv[u].x) : uabs64(yv[u].y);
    const uint64_t b = uabs64(yv[u].z) > uabs64(yv[u].w) ? uabs64(yv[u].z) : uabs64(yv[u].w);
    const int64_t c = (int64_t)(a > b ? a : b);
    A = c > A ? c : A;
  }
  A = block_max(A, red);
  const int e = dq_exp((uint64_t)A);
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (RR::first(u) < n)
      *(uint32_t*)(q + (size_t)r * n + RR::first(u)) =
          pack4(R_nn(yv[u].x, e), R_nn(yv[u].y, e), R_nn(yv[u].z, e), R_nn(yv[u].w, e));
  if (threadIdx.x == 0) {
    if (row_e) row_e[r] = e;
    if (row_m) {
      row_m[r] = fm;
      row_k[r] = fk - e;
    }
  }
}

// Per-token DQ (DetLLM blog "DetLLM": a token's activations are quantised
// from its own values): q = clamp8(R(y, e)), e from the row's |max|.
__global__ __launch_bounds__(TPB) void requant_k(const int32_t* __restrict__ y, int n,
                                                 int8_t* __restrict__ q, int32_t* row_e,
                                                 int32_t* row_m, int32_t* row_k, int32_t fm,
                                                 int32_t fk) {
  __shared__ int64_t red[16];
  const int r = blockIdx.x;
  const int32_t* yr = y + (size_t)r * n;
  int64_t A = 0;
  for (int i = threadIdx.x; i < n; i += TPB) {
    const int64_t a = (int64_t)uabs64(yr[i]);
    A = a > A ? a : A;
  }
  A = block_max(A, red);
  const int e = dq_exp((uint64_t)A);
  for (int i = threadIdx.x; i < n; i += TPB) q[(size_t)r * n + i] = clamp8(R(yr[i], e));
  if (threadIdx.x == 0) {
    if (row_e) row_e[r] = e;
    if (row_m) {
      row_m[r] = fm;
      row_k[r] = fk - e;
    }
  }
}

// Integer RoPE on pairs (i, i + d/2) with Q1.14 tables.
__global__ void rope_k(int32_t* __restrict__ x, const int32_t* __restrict__ pos,
                       const int16_t* __restrict__ ct, const int16_t* __restrict__ stab,
                       int heads, int d, int max_pos) {
  const int r = blockIdx.x, hh = blockIdx.y, i = threadIdx.x;
  const int half = d >> 1;
  if (i >= half || pos[r] < 0 || pos[r] >= max_pos) return;  // out of table: untouched
  int32_t* v = x + ((size_t)r * heads + hh) * d;
  const int64_t a = v[i], b = v[i + half];
  const int64_t c = ct[(size_t)pos[r] * half + i], s = stab[(size_t)pos[r] * half + i];
  v[i] = (int32_t)R(a * c - b * s, 14);
  v[i + half] = (int32_t)R(b * c + a * s, 14);
}

// DI-Softmax with 15-bit probabilities (DetLLM blog, footnote 8).
__global__ __launch_bounds__(TPB) void softmax_k(const int32_t* __restrict__ s,
                                                 const int32_t* __restrict__ valid,
                                                 const int32_t* __restrict__ shift, int C,
                                                 int32_t Mm, int32_t Kk, int16_t* __restrict__ P) {
  __shared__ int64_t red[16];
  const int r = blockIdx.x;
  const int32_t* sr = s + (size_t)r * C;
  int v = valid[r];
  v = v < 1 ? 1 : (v > C ? C : v);
  const int sh = Kk - shift[r];
  int64_t mx = INT64_MIN;
  for (int j = threadIdx.x; j < v; j += TPB) mx = sr[j] > mx ? sr[j] : mx;
  mx = block_max(mx, red);
  int64_t D = 0;
  for (int j = threadIdx.x; j < v; j += TPB) D += diexp(R((sr[j] - mx) * Mm, sh));
  D = block_sum(D, red);
  const int64_t Rn = (int64_t)udiv_wave<32>(uint64_t(1) << 46, (uint64_t)D);  // D >= 2^15
  for (int j = threadIdx.x; j < C; j += TPB) {
    int64_t p = 0;
    if (j < v) {
      p = R((int64_t)diexp(R((sr[j] - mx) * Mm, sh)) * Rn, 31);
      p = p > 32767 ? 32767 : p;
    }
    P[(size_t)r * C + j] = (int16_t)p;
  }
}

// DI-SwiGLU (DetLLM README "Layout"): a8 * 2^(e - 2 f_a) ~ silu(g) * u.
__device__ __forceinline__ int64_t swiglu_p(int64_t g, int64_t u, int32_t Mg, int32_t Kg) {
  return R(g * sigmoid_q15(g, Mg, Kg), 15) * u;
}

constexpr int SWT = 1024, SWPER = 8;  // n <= SWT * SWPER

__global__ __launch_bounds__(SWT) void swiglu_k(const int32_t* __restrict__ gu, int n, int32_t f_a,
                                                int32_t Mg, int32_t Kg, int8_t* __restrict__ a8,
                                                int32_t* __restrict__ rm, int32_t* __restrict__ rk) {
  __shared__ int64_t red[16];
  const int r = blockIdx.x;
  const int32_t* g = gu + (size_t)r * 2 * n;
  const int32_t* u = g + n;
  int64_t p[SWPER];
  int64_t A = 0;
  uint32_t bad = 0;
#pragma unroll
  for (int i = 0; i < SWPER; ++i) {
    const int j = threadIdx.x + i * SWT;
    p[i] = j < n ? swiglu_p(g[j], u[j], Mg, Kg) : 0;
    if (j < n) bad |= out_of32(g[j], 24) | out_of32(u[j], 24);
    const int64_t a = (int64_t)uabs64(p[i]);
    A = a > A ? a : A;
  }
  bound_raise(bad ? kBoundSwiglu : 0u);
  A = block_max(A, red);
  const int e = dq_exp((uint64_t)A);
#pragma unroll
  for (int i = 0; i < SWPER; ++i) {
    const int j = threadIdx.x + i * SWT;
    if (j < n) a8[(size_t)r * n + j] = clamp8(R(p[i], e));
  }
  if (threadIdx.x == 0) {
    rm[r] = 1 << 14;
    rk[r] = 2 * f_a - e + 14;
  }
}

template <int U>
__global__ __launch_bounds__(SWT) void swiglu_rk(const int32_t* __restrict__ gu, int n, int32_t f_a,
                                                 int32_t Mg, int32_t Kg, int8_t* __restrict__ a8,
                                                 int32_t* __restrict__ rm, int32_t* __restrict__ rk) {
  using RR = RowRegs<SWT, U>;
  __shared__ int64_t red[16];
  const int r = blockIdx.x;
  const int32_t* g = gu + (size_t)r * 2 * n;
  const int32_t* up = g + n;
  v4i gv[U], uv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    gv[u] = *(const v4i*)(g + RR::at(u, n));
    uv[u] = *(const v4i*)(up + RR::at(u, n));
  }
  int64_t p[U][4], A = 0;
  uint32_t bad = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool ok = RR::first(u) < n;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      p[u][e4] = ok ? swiglu_p(gv[u][e4], uv[u][e4], Mg, Kg) : 0;
      if (ok) bad |= out_of32(gv[u][e4], 24) | out_of32(uv[u][e4], 24);
      const int64_t a = (int64_t)uabs64(p[u][e4]);
      A = a > A ? a : A;
    }
  }
  bound_raise(bad ? kBoundSwiglu : 0u);
  A = block_max(A, red);
  const int e = dq_exp((uint64_t)A);
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (RR::first(u) < n)
      *(uint32_t*)(a8 + (size_t)r * n + RR::first(u)) =
          pack4(R_nn(p[u][0], e), R_nn(p[u][1], e), R_nn(p[u][2], e), R_nn(p[u][3], e));
  if (threadIdx.x == 0) {
    rm[r] = 1 << 14;
    rk[r] = 2 * f_a - e + 14;
  }
}

// Quotients of the integer sigmoid, q(E) = RD(2^30, 2^15 + E) for every
// DI-Exp output E in [0, 2^15] (the same rounded division sigmoid_q15 runs
// bit-serially), evaluated by the compiler as exact integer constant
// expressions. 32769 entries, padded to a whole number of 16-byte chunks.
constexpr int kSigEntries = 32769, kSigPad = 32776;
struct alignas(16) SigTable {
  uint16_t q[kSigPad];
};
constexpr SigTable make_sig_table() {
  SigTable t{};
  for (uint32_t E = 0; E < (uint32_t)kSigEntries; ++E) {
    const uint64_t b = 32768u + E;
    t.q[E] = (uint16_t)(((uint64_t(1) << 31) + b) / (2 * b));
  }
  return t;
}
__device__ const SigTable kSigTable = make_sig_table();
constexpr size_t kSigLds = sizeof(SigTable);  // 65552 bytes

// DI-SwiGLU for many rows (prefill): a persistent grid whose workgroups copy
// the sigmoid quotients into LDS once and then take rows w, w + G, ...; the
// sigmoid's division becomes one LDS lookup. One 1024-thread workgroup per
// CU, 4 waves per SIMD (up to 128 VGPRs), which holds the next row's
// gate/up values in flight while it computes the current row. Same integer
// function as swiglu_rk, row for row.
template <int U>
__global__ __launch_bounds__(SWT, 4) void swiglu_tab_rk(const int32_t* __restrict__ gu, int rows, int n,
                                                     int32_t f_a, int32_t Mg, int32_t Kg, uint32_t g0,
                                                     int8_t* __restrict__ a8,
                                                     int32_t* __restrict__ rm,
                                                     int32_t* __restrict__ rk) {
  using RR = RowRegs<SWT, U>;
  extern __shared__ __attribute__((aligned(16))) uint16_t tab[];  // kSigPad entries
  __shared__ int64_t red[16];
  for (int i = threadIdx.x; i < kSigPad / 8; i += SWT)
    ((v4i*)tab)[i] = ((const v4i*)kSigTable.q)[i];
  const int G = (int)gridDim.x;
  int r = blockIdx.x;
  v4i gv[U], uv[U];
  auto load = [&](int row, v4i (&gg)[U], v4i (&uu)[U]) {
    const int32_t* g = gu + (size_t)row * 2 * n;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      gg[u] = *(const v4i*)(g + RR::at(u, n));
      uu[u] = *(const v4i*)(g + n + RR::at(u, n));
    }
  };
  __syncthreads();  // table resident
  // one row: silu and the DQ'd product, in place in gv / uv
  auto body = [&](int r, v4i (&gv)[U], v4i (&uv)[U]) {
    if (g0) {
      // 32-bit form (g0 > 0: 1 <= Kg <= 12, 2^10 <= Mg < 2^15). The sigmoid's
      // DI-Exp input v = R(|g| Mg, Kg) reaches 31 * 2^15 (E = 0) exactly from
      // |g| = g0 on, so |g| is clamped there: the product then stays below
      // 31 * 2^(15 + Kg) + Mg < 2^32 and v >> 15 <= 31. With v = 2^15 n + r,
      // DI-Exp's fraction 2^15 - R(r, 1) is (2^16 - r) >> 1. In range |g|,
      // |u| < 2^24 (checked), so the magnitudes enter unsigned 24-bit
      // products: with a = |g| sig (sig >= 0), |R(g sig, 15)| is
      // (a + 2^14) >> 15 for g >= 0 and (a + 2^14 - 1) >> 15 for g < 0
      // (round half up on a negative value), and the row's DQ exponent comes
      // from the OR of the exact |silu| |u| (the bit length of the OR is that
      // of the maximum).
      // silu and the 24-bit u replace g and u in the row's own registers
      uint32_t amax = 0, lo_or = 0, hi_or = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = RR::first(u) < n;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int32_t g = ok ? gv[u][e4] : 0, uv0 = ok ? uv[u][e4] : 0;
          const uint32_t ag = (uint32_t)max(g, -g), au = (uint32_t)max(uv0, -uv0);
          amax = max(amax, max(ag, au));
          const uint32_t v = (__umul24(min(ag, g0), (uint32_t)Mg) + (1u << (Kg - 1))) >> Kg;
          const uint32_t nn = v >> 15, f = (65536u - (v & 32767u)) >> 1;
          const uint32_t E = (f + ((1u << nn) >> 1)) >> nn;
          const int32_t q = tab[E];
          const int32_t sig = g >= 0 ? q : 32768 - q;
          const uint64_t a = (uint64_t)(ag & 0xFFFFFFu) * ((uint32_t)sig & 0xFFFFu);
          const uint32_t as = (uint32_t)((a + (1u << 14) - (g < 0 ? 1u : 0u)) >> 15);
          const uint32_t au24 = au & 0xFFFFFFu;
          lo_or |= __umul24(as, au24);
          hi_or |= __umulhi(as, au24);
          gv[u][e4] = g < 0 ? -(int32_t)as : (int32_t)as;  // silu
          uv[u][e4] = uv0;
        }
      }
      bound_raise(amax >= (1u << 24) ? kBoundSwiglu : 0u);
      const int64_t A = block_max((int64_t)(((uint64_t)hi_or << 32) | lo_or), red);
      const int e = dq_exp((uint64_t)A);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (RR::first(u) < n) {
          int64_t pq[4];
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) pq[e4] = R_nn((int64_t)gv[u][e4] * uv[u][e4], e);
          *(uint32_t*)(a8 + (size_t)r * n + RR::first(u)) = pack4(pq[0], pq[1], pq[2], pq[3]);
        }
      if (threadIdx.x == 0) {
        rm[r] = 1 << 14;
        rk[r] = 2 * f_a - e + 14;
      }
      return;
    }
    int64_t p[U][4], A = 0;
    uint32_t bad = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = RR::first(u) < n;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int64_t g = gv[u][e4];
        if (ok) bad |= out_of32((int32_t)g, 24) | out_of32(uv[u][e4], 24);
        const int64_t ag = g < 0 ? -g : g;
        const int E = min(diexp(-R(ag * Mg, Kg)), kSigEntries - 1);
        const int32_t q = tab[E];
        const int32_t sig = g >= 0 ? q : 32768 - q;
        p[u][e4] = ok ? R(g * sig, 15) * (int64_t)uv[u][e4] : 0;
        const int64_t a = (int64_t)uabs64(p[u][e4]);
        A = a > A ? a : A;
      }
    }
    bound_raise(bad ? kBoundSwiglu : 0u);
    A = block_max(A, red);
    const int e = dq_exp((uint64_t)A);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (RR::first(u) < n)
        *(uint32_t*)(a8 + (size_t)r * n + RR::first(u)) =
            pack4(R_nn(p[u][0], e), R_nn(p[u][1], e), R_nn(p[u][2], e), R_nn(p[u][3], e));
    if (threadIdx.x == 0) {
      rm[r] = 1 << 14;
      rk[r] = 2 * f_a - e + 14;
    }
  };
  // the next row's loads in flight under this row's arithmetic (rows past
  // the end load the last row again; its values are not used)
  v4i gb[U], ub[U];
  if (r < rows) load(r, gv, uv);
  for (; r < rows; r += 2 * G) {
    load(min(r + G, rows - 1), gb, ub);
    body(r, gv, uv);
    if (r + G >= rows) break;
    load(min(r + 2 * G, rows - 1), gv, uv);
    body(r + G, gb, ub);
  }
}

// The DQ half of DI-SwiGLU for products already formed (by a GEMM
// epilogue): int64 rows -> int8, row scale (2^14, 2 f_a - e + 14).
template <int U>
__global__ __launch_bounds__(TPB) void dq64_rk(const int64_t* __restrict__ p, int n, int32_t f_a,
                                               int8_t* __restrict__ a8, int32_t* __restrict__ rm,
                                               int32_t* __restrict__ rk) {
  using RR = RowRegs<TPB, U>;
  typedef int64_t v2l __attribute__((ext_vector_type(2)));
  __shared__ int64_t red[16];
  const int r = blockIdx.x;
  const int64_t* pr = p + (size_t)r * n;
  v2l lo[U], hi[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    lo[u] = *(const v2l*)(pr + RR::at(u, n));
    hi[u] = *(const v2l*)(pr + RR::at(u, n) + 2);
  }
  int64_t A = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (RR::first(u) >= n) lo[u] = hi[u] = v2l{0, 0};
    const uint64_t a = uabs64(lo[u].x) > uabs64(lo[u].y) ? uabs64(lo[u].x) : uabs64(lo[u].y);
    const uint64_t b = uabs64(hi[u].x) > uabs64(hi[u].y) ? uabs64(hi[u].x) : uabs64(hi[u].y);
    const int64_t c = (int64_t)(a > b ? a : b);
    A = c > A ? c : A;
  }
  A = block_max(A, red);
  const int e = dq_exp((uint64_t)A);
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (RR::first(u) < n)
      *(uint32_t*)(a8 + (size_t)r * n + RR::first(u)) =
          pack4(R_nn(lo[u].x, e), R_nn(lo[u].y, e), R_nn(hi[u].x, e), R_nn(hi[u].y, e));
  if (threadIdx.x == 0) {
    rm[r] = 1 << 14;
    rk[r] = 2 * f_a - e + 14;
  }
}

// Embedding rounded once onto the residual grid (BitExact blog, "Three
// execution paths"): h = R(E[id] * m_v[id], w_k - f_res).
__global__ __launch_bounds__(TPB) void embed_k(const int32_t* __restrict__ ids,
                                               const int8_t* __restrict__ emb,
                                               const int8_t* __restrict__ emb_lo,
                                               const int32_t* __restrict__ emb_m, int H, int V,
                                               int shift, int32_t* __restrict__ h) {
  const int r = blockIdx.x;
  const int64_t id = ids[r];
  if (id < 0 || id >= V) {  // out-of-vocabulary id: zero row, flagged
    if (threadIdx.x == 0) bound_raise(kBoundId);
    for (int i = threadIdx.x; i < H; i += TPB) h[(size_t)r * H + i] = 0;
    return;
  }
  const int64_t m = emb_m[id];
  uint32_t bad = 0;
  for (int i = threadIdx.x; i < H; i += TPB) {
    int64_t e = emb[id * H + i];
    if (emb_lo) e = 256 * e + (int64_t)emb_lo[id * H + i] + 128;
    const int64_t v = R(e * m, shift);
    bad |= out_of(v, 25);
    h[(size_t)r * H + i] = (int32_t)v;
  }
  bound_raise(bad ? kBoundResidual : 0u);
}

__global__ void rows_meta_k(const int32_t* __restrict__ cu, const int32_t* __restrict__ start,
                            const int32_t* __restrict__ slot, int32_t* pos_of, int32_t* slot_of,
                            int32_t* last_row, int32_t* zero, int nzero) {
  const int s = blockIdx.x;
  if (s == 0)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0;
  const int b = cu[s], e = cu[s + 1];
  for (int r = b + threadIdx.x; r < e; r += blockDim.x) {
    pos_of[r] = start[s] + (r - b);
    slot_of[r] = slot[s];
  }
  if (threadIdx.x == 0 && last_row) last_row[s] = e - 1;
}

__global__ void decode_meta_k(const int32_t* __restrict__ ctx, const int32_t* __restrict__ slot,
                              int B, int32_t* pos_of, int32_t* slot_of) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    pos_of[b] = ctx[b] - 1;
    slot_of[b] = slot[b];
  }
}

// QKV post-processing, one wave per (row, head) - four heads per workgroup,
// grid (rows, heads / 4); the per-head arithmetic is qkv_head (qkv_dev.h).
__global__ __launch_bounds__(TPB) void qkv_post_k(const int32_t* __restrict__ qkv, int nq, int nkv,
                                                  int d, const int32_t* __restrict__ pos_of,
                                                  const int32_t* __restrict__ slot_of, QkvPost p,
                                                  int8_t* __restrict__ q8, int32_t* __restrict__ e_q,
                                                  int8_t* __restrict__ kc, int8_t* __restrict__ vc,
                                                  int n_slots, int max_pos, KvPages kp) {
  const int r = blockIdx.x;
  const int hh = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int nh = nq + 2 * nkv;
  if (hh >= nh) return;
  const int pos = pos_of[r], slot = slot_of[r];
  const bool ok = pos >= 0 && pos < max_pos && slot >= 0 && slot < n_slots;
  const int32_t rm = p.qk_norm ? p.row_m[r] : 0, rk = p.qk_norm ? p.row_k[r] : 0;
  qkv_head(qkv + (size_t)r * nh * d, hh, nq, nkv, d, pos, slot, ok, rm, rk, p,
           q8 + ((size_t)r * nq + (hh < nq ? hh : 0)) * d, e_q + (size_t)r * nq + (hh < nq ? hh : 0),
           kc, vc, max_pos, kp);
}

// Without q/k-norm and with 64-wide heads a head needs only 32 lanes (lane i
// owns the RoPE pair (i, i + 32)), so a wave takes two: the 32-lane half h
// handles head 2 w + h. The same integer steps as qkv_head without q/k-norm;
// the query's DQ maximum is reduced over its half only (xor offsets below
// 32 stay within a half). Every lane takes part in the reduction; a half
// past the last head stores nothing. A workgroup takes RPW consecutive rows
// (their loads all issued before the first wait, then their RoPE table
// rows), so that the two dependent round trips (position, then table row)
// are paid once per RPW rows rather than per row.
template <int RPW>
__global__ __launch_bounds__(TPB) void qkv_post_pair_k(const int32_t* __restrict__ qkv, int rows, int nq,
                                                       int nkv, const int32_t* __restrict__ pos_of,
                                                       const int32_t* __restrict__ slot_of,
                                                       QkvPost p, int8_t* __restrict__ q8,
                                                       int32_t* __restrict__ e_q,
                                                       int8_t* __restrict__ kc,
                                                       int8_t* __restrict__ vc, int n_slots,
                                                       int max_pos, KvPages kp) {
  constexpr int d = 64, half = 32;
  const int li = threadIdx.x & 31;
  const int nh = nq + 2 * nkv;
  const int hh = (blockIdx.y * (TPB / 64) + (threadIdx.x >> 6)) * 2 + ((threadIdx.x >> 5) & 1);
  const bool live = hh < nh;
  const int hc = live ? hh : nh - 1;
  const bool isq = hc < nq, isv = hc >= nq + nkv;
  const int kvh = isq ? hc >> (__builtin_ctz(nq) - __builtin_ctz(nkv)) : (isv ? 0 : hc - nq);
  const int j0 = li, j1 = li + half;
  // rows past the last repeat it (loads only; nothing is stored for them)
  int pos[RPW], slot[RPW];
  int64_t x0[RPW], x1[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int rr = min((int)blockIdx.x * RPW + i, rows - 1);
    pos[i] = pos_of[rr];
    slot[i] = slot_of[rr];
    const int32_t* row = qkv + (size_t)rr * nh * d + (size_t)hc * d;
    x0[i] = row[j0];  // f_n fixed point from the GEMM epilogue
    x1[i] = row[j1];
  }
  int64_t c[RPW], sn[RPW];
  bool ok[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    ok[i] = (int)blockIdx.x * RPW + i < rows && pos[i] >= 0 && pos[i] < max_pos && slot[i] >= 0 &&
            slot[i] < n_slots;
    const int pc = ok[i] ? pos[i] : 0;
    c[i] = p.cos_t[(size_t)pc * half + li];
    sn[i] = p.sin_t[(size_t)pc * half + li];
  }
  const int g0 = p.k_gain && !isv ? p.k_gain[(size_t)kvh * d + j0] & 7 : 0;
  const int g1 = p.k_gain && !isv ? p.k_gain[(size_t)kvh * d + j1] & 7 : 0;
  uint32_t bad = 0;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = (int)blockIdx.x * RPW + i;
    if (isv && live && ok[i]) {
      int8_t* dst = vc + kv_row_off(kp, slot[i], hc - nq - nkv, nkv, max_pos, d, pos[i], bad);
      dst[j0] = clamp8(R(x0[i] * p.vq_m, p.vq_k));
      dst[j1] = clamp8(R(x1[i] * p.vq_m, p.vq_k));
    }
    int64_t y0 = ok[i] ? R(x0[i] * c[i] - x1[i] * sn[i], 14) : 0;
    int64_t y1 = ok[i] ? R(x1[i] * c[i] + x0[i] * sn[i], 14) : 0;
    if (live && !isv) bad |= i32_check(y0) | i32_check(y1);  // rotated q / k within int32
    if (isq) {  // the inverse of the key gain
      y0 = R(y0, g0);
      y1 = R(y1, g1);
    }
    uint64_t u = uabs64(y0) > uabs64(y1) ? uabs64(y0) : uabs64(y1);
    auto umax = [](uint64_t x, uint64_t y) { return x > y ? x : y; };
    u = umax(u, lane_xor<16>(u));
    u = umax(u, lane_xor<8>(u));
    u = umax(u, lane_xor<4>(u));
    u = umax(u, lane_xor<2>(u));
    u = umax(u, lane_xor<1>(u));
    if (!live || isv || r >= rows) continue;
    if (isq) {
      const int e = dq_exp(u);
      int8_t* qd = q8 + ((size_t)r * nq + hc) * d;
      qd[j0] = clamp8(R(y0, e));
      qd[j1] = clamp8(R(y1, e));
      if (li == 0) e_q[(size_t)r * nq + hc] = e;
    } else if (ok[i]) {
      int8_t* dst = kc + kv_row_off(kp, slot[i], kvh, nkv, max_pos, d, pos[i], bad);
      dst[j0] = clamp8(R(y0 * p.kq_m, p.kq_k - g0));
      dst[j1] = clamp8(R(y1 * p.kq_m, p.kq_k - g1));
    }
  }
  bound_raise(bad);
}

// Greedy argmax with the lowest index among maxima (DetLLM blog "DetLLM").
// Key = value << 32 | (2^32 - 1 - index): the largest key is the largest
// value at the smallest index, and max is order-free.
__device__ __forceinline__ int64_t amax_key(int32_t v, int64_t j) {
  return ((int64_t)v * 4294967296LL) | (int64_t)(0xFFFFFFFFu - (uint32_t)j);
}

__global__ __launch_bounds__(TPB) void argmax_part_k(const int32_t* __restrict__ logits,
                                                     const int32_t* row_base, int V, int nparts,
                                                     int chunk, int64_t* part) {
  __shared__ int64_t red[16];
  const int s = blockIdx.y, pi = blockIdx.x;
  const int64_t base = row_base ? *row_base : 0;
  const int32_t* L = logits + (base + s) * (int64_t)V;
  const int lo = pi * chunk, hi = lo + chunk < V ? lo + chunk : V;
  int64_t best = INT64_MIN;
  for (int j = lo + threadIdx.x; j < hi; j += TPB) {
    const int64_t k = amax_key(L[j], j);
    best = k > best ? k : best;
  }
  best = block_max(best, red);
  if (threadIdx.x == 0) part[(size_t)s * nparts + pi] = best;
}

__global__ __launch_bounds__(1024) void argmax_final_k(const int64_t* __restrict__ part, int nparts,
                                                      int32_t* out) {
  __shared__ int64_t red[16];
  const int s = blockIdx.x;
  int64_t best = INT64_MIN;
  for (int i = threadIdx.x; i < nparts; i += 1024) {
    const int64_t k = part[(size_t)s * nparts + i];
    best = k > best ? k : best;
  }
  best = block_max(best, red);
  if (threadIdx.x == 0) out[s] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFLL));
}

// Final greedy reduction of the lm_head partials fused with the decode-step
// advance: next_tok[s]; with advance, ids[s] = next_tok[s], start_pos[s] += 1
// and the logits history row base moves on by S.
__global__ __launch_bounds__(1024) void argmax_advance_k(const int64_t* __restrict__ part, int nparts,
                                                        int32_t* next_tok, int32_t* ids,
                                                        int32_t* start_pos, int32_t* row_base, int S,
                                                        int advance) {
  __shared__ int64_t red[16];
  const int s = blockIdx.x;
  int64_t best = INT64_MIN;
  for (int i = threadIdx.x; i < nparts; i += 1024) {
    const int64_t k = part[(size_t)s * nparts + i];
    best = k > best ? k : best;
  }
  best = block_max(best, red);
  if (threadIdx.x == 0) {
    const int32_t tok = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFLL));
    next_tok[s] = tok;
    if (advance) {
      ids[s] = tok;
      start_pos[s] += 1;
      if (s == 0 && row_base) *row_base += S;
    }
  }
}

__global__ void advance_k(int32_t* ids, const int32_t* next_tok, int32_t* start_pos,
                          int32_t* row_base, int S) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < S) {
    ids[s] = next_tok[s];
    start_pos[s] += 1;
  }
  if (s == 0 && row_base) *row_base += S;
}

bool aligned_to(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

namespace {
// q = clamp8(R(y m, k)), four elements per thread (n % 4 == 0 handled by
// the tail loop of the last thread block)
__global__ __launch_bounds__(256) void requant_fixed_k(const int32_t* __restrict__ y, int64_t n,
                                                       int32_t m, int32_t k, int8_t* __restrict__ q) {
  const int64_t i = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (i + 4 <= n) {
    const v4i v = *(const v4i*)(y + i);
    *(uint32_t*)(q + i) = pack4(R((int64_t)v.x * m, k), R((int64_t)v.y * m, k),
                                R((int64_t)v.z * m, k), R((int64_t)v.w * m, k));
  } else {
    for (int64_t t = i; t < n; ++t) q[t] = clamp8(R((int64_t)y[t] * m, k));
  }
}
}  // namespace

hipError_t launch_requant_fixed(const int32_t* y, int64_t n, int32_t m, int32_t k, int8_t* q,
                                hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 1023) / 1024;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  requant_fixed_k<<<(unsigned)blocks, 256, 0, st>>>(y, n, m, k, q);
  return hipGetLastError();
}

DETINT_BOUND_READER(bound_flags_rowops)

hipError_t launch_rmsnorm(const int32_t* h, const int32_t* row_index, const int16_t* gain,
                          int64_t R, int64_t n, int8_t* x8, int32_t* row_m, int32_t* row_k,
                          hipStream_t st) {
  if (R == 0) return hipSuccess;
  if (n % 4 == 0 && n >= 4 && n <= 32 * TPB && aligned_to(h, 16) && aligned_to(gain, 8) &&
      aligned_to(x8, 4)) {
    const int u = (int)((n + 4 * TPB - 1) / (4 * TPB));
    if (u <= 1)
      rmsnorm_rk<1><<<(unsigned)R, TPB, 0, st>>>(h, row_index, gain, (int)n, x8, row_m, row_k);
    else if (u <= 2)
      rmsnorm_rk<2><<<(unsigned)R, TPB, 0, st>>>(h, row_index, gain, (int)n, x8, row_m, row_k);
    else if (u <= 4)
      rmsnorm_rk<4><<<(unsigned)R, TPB, 0, st>>>(h, row_index, gain, (int)n, x8, row_m, row_k);
    else
      rmsnorm_rk<8><<<(unsigned)R, TPB, 0, st>>>(h, row_index, gain, (int)n, x8, row_m, row_k);
    return hipGetLastError();
  }
  rmsnorm_k<<<(unsigned)R, TPB, 0, st>>>(h, row_index, gain, (int)n, x8, row_m, row_k);
  return hipGetLastError();
}

hipError_t launch_requant(const int32_t* y, int64_t R, int64_t n, int8_t* q, int32_t* row_e,
                          int32_t* row_m, int32_t* row_k, int32_t fold_m, int32_t fold_k,
                          hipStream_t st) {
  if (R == 0) return hipSuccess;
  if (n % 4 == 0 && n >= 4 && n <= 32 * TPB && aligned_to(y, 16) && aligned_to(q, 4)) {
    const int u = (int)((n + 4 * TPB - 1) / (4 * TPB));
#define DETINT_RQ(UU) \
  requant_rk<UU><<<(unsigned)R, TPB, 0, st>>>(y, (int)n, q, row_e, row_m, row_k, fold_m, fold_k)
    if (u <= 1)
      DETINT_RQ(1);
    else if (u <= 2)
      DETINT_RQ(2);
    else if (u <= 4)
      DETINT_RQ(4);
    else
      DETINT_RQ(8);
#undef DETINT_RQ
    return hipGetLastError();
  }
  requant_k<<<(unsigned)R, TPB, 0, st>>>(y, (int)n, q, row_e, row_m, row_k, fold_m, fold_k);
  return hipGetLastError();
}

hipError_t launch_rope(int32_t* x, const int32_t* pos, const int16_t* cos_t,
                       const int16_t* sin_t, int64_t R, int64_t heads, int64_t d, int64_t max_pos,
                       hipStream_t st) {
  if (R == 0 || heads == 0) return hipSuccess;
  const int thr = (int)((d / 2 + 63) / 64 * 64);
  rope_k<<<dim3((unsigned)R, (unsigned)heads), thr, 0, st>>>(x, pos, cos_t, sin_t, (int)heads,
                                                              (int)d, (int)max_pos);
  return hipGetLastError();
}

hipError_t launch_softmax(const int32_t* s, const int32_t* valid, const int32_t* shift,
                          int64_t R, int64_t C, int32_t M, int32_t K, int16_t* P,
                          hipStream_t st) {
  if (R == 0) return hipSuccess;
  softmax_k<<<(unsigned)R, TPB, 0, st>>>(s, valid, shift, (int)C, M, K, P);
  return hipGetLastError();
}

hipError_t launch_swiglu(const int32_t* gu, int64_t R, int64_t n, int32_t f_a, int32_t Mg,
                         int32_t Kg, int8_t* a8, int32_t* row_m, int32_t* row_k, hipStream_t st) {
  if (R == 0) return hipSuccess;
  if (n > SWT * SWPER) return hipErrorInvalidValue;
  if (n % 4 == 0 && n >= 4 && aligned_to(gu, 16) && aligned_to(a8, 4)) {
    if (R > 64) {
      // persistent, one workgroup per CU (the table takes 64 KiB of LDS),
      // each row's loads issued under the previous row's arithmetic: 150
      // against 163 us per layer for two workgroups per CU without the
      // prefetch (their 64 VGPRs leave no room for it)
      hipError_t err = set_max_lds((const void*)swiglu_tab_rk<1>, kSigLds);
      if (err == hipSuccess) err = set_max_lds((const void*)swiglu_tab_rk<2>, kSigLds);
      if (err != hipSuccess) return err;
      const unsigned grid = (unsigned)(R < 256 ? R : 256);
      // clamp of the 32-bit form: the least |g| with R(|g| Mg, Kg) >= 31 2^15,
      // ceil((31 2^(15 + Kg) - 2^(Kg - 1)) / Mg); 0 (the 64-bit form) outside
      // 1 <= Kg <= 12, 2^10 <= Mg < 2^15
      uint32_t g0 = 0;
      if (Kg >= 1 && Kg <= 12 && Mg >= (1 << 10) && Mg < (1 << 15)) {
        const uint64_t T = (uint64_t(31) << (15 + Kg)) - (uint64_t(1) << (Kg - 1));
        g0 = (uint32_t)((T + (uint64_t)Mg - 1) / (uint64_t)Mg);
      }
      if (n <= 4 * SWT)
        swiglu_tab_rk<1><<<grid, SWT, kSigLds, st>>>(gu, (int)R, (int)n, f_a, Mg, Kg, g0, a8, row_m, row_k);
      else
        swiglu_tab_rk<2><<<grid, SWT, kSigLds, st>>>(gu, (int)R, (int)n, f_a, Mg, Kg, g0, a8, row_m, row_k);
      return hipGetLastError();
    }
    if (n <= 4 * SWT)
      swiglu_rk<1><<<(unsigned)R, SWT, 0, st>>>(gu, (int)n, f_a, Mg, Kg, a8, row_m, row_k);
    else
      swiglu_rk<2><<<(unsigned)R, SWT, 0, st>>>(gu, (int)n, f_a, Mg, Kg, a8, row_m, row_k);
    return hipGetLastError();
  }
  swiglu_k<<<(unsigned)R, SWT, 0, st>>>(gu, (int)n, f_a, Mg, Kg, a8, row_m, row_k);
  return hipGetLastError();
}

hipError_t launch_dq64(const int64_t* p, int64_t R, int64_t n, int32_t f_a, int8_t* a8,
                       int32_t* row_m, int32_t* row_k, hipStream_t st) {
  if (R == 0) return hipSuccess;
  if (n % 4 != 0 || n < 4 || n > 32 * TPB || !aligned_to(p, 16) || !aligned_to(a8, 4))
    return hipErrorInvalidValue;
  const int u = (int)((n + 4 * TPB - 1) / (4 * TPB));
#define DETINT_DQ(UU) dq64_rk<UU><<<(unsigned)R, TPB, 0, st>>>(p, (int)n, f_a, a8, row_m, row_k)
  if (u <= 1)
    DETINT_DQ(1);
  else if (u <= 2)
    DETINT_DQ(2);
  else if (u <= 4)
    DETINT_DQ(4);
  else
    DETINT_DQ(8);
#undef DETINT_DQ
  return hipGetLastError();
}

hipError_t launch_embed(const int32_t* ids, int64_t R, const int8_t* emb, const int8_t* emb_lo,
                        const int32_t* emb_m, int64_t H, int64_t V, int32_t shift, int32_t* h,
                        hipStream_t st) {
  if (R == 0) return hipSuccess;
  embed_k<<<(unsigned)R, TPB, 0, st>>>(ids, emb, emb_lo, emb_m, (int)H, (int)V, shift, h);
  return hipGetLastError();
}

hipError_t launch_rows_meta(const int32_t* cu, const int32_t* start, const int32_t* slot,
                            int64_t S, int32_t* pos_of, int32_t* slot_of, int32_t* last_row,
                            hipStream_t st, int32_t* zero, int64_t nzero) {
  if (S == 0) return hipSuccess;
  rows_meta_k<<<(unsigned)S, 256, 0, st>>>(cu, start, slot, pos_of, slot_of, last_row, zero,
                                           (int)nzero);
  return hipGetLastError();
}

hipError_t launch_decode_meta(const int32_t* ctx_len, const int32_t* slot, int64_t B,
                              int32_t* pos_of, int32_t* slot_of, hipStream_t st) {
  if (B == 0) return hipSuccess;
  decode_meta_k<<<(unsigned)((B + 255) / 256), 256, 0, st>>>(ctx_len, slot, (int)B, pos_of, slot_of);
  return hipGetLastError();
}

hipError_t launch_qkv_post(const int32_t* qkv, int64_t R, int64_t nq, int64_t nkv, int64_t d,
                           const int32_t* pos_of, const int32_t* slot_of, const QkvPost& p,
                           int8_t* q8, int32_t* e_q, int8_t* kc, int8_t* vc, int64_t n_slots,
                           int64_t max_pos, hipStream_t st, KvPages kp) {
  if (R == 0) return hipSuccess;
  if (!p.qk_norm && d == 64) {  // two heads per wave
    const unsigned hp = (unsigned)((nq + 2 * nkv + 2 * (TPB / 64) - 1) / (2 * (TPB / 64)));
    constexpr int RPW = 4;
    qkv_post_pair_k<RPW><<<dim3((unsigned)((R + RPW - 1) / RPW), hp), TPB, 0, st>>>(
        qkv, (int)R, (int)nq, (int)nkv, pos_of, slot_of, p, q8, e_q, kc, vc, (int)n_slots,
        (int)max_pos, kp);
    return hipGetLastError();
  }
  const unsigned hb = (unsigned)((nq + 2 * nkv + 3) / 4);  // 4 heads (waves) per workgroup
  qkv_post_k<<<dim3((unsigned)R, hb), TPB, 0, st>>>(qkv, (int)nq, (int)nkv, (int)d, pos_of, slot_of,
                                                     p, q8, e_q, kc, vc, (int)n_slots, (int)max_pos,
                                                     kp);
  return hipGetLastError();
}

hipError_t launch_argmax(const int32_t* logits, const int32_t* row_base, int64_t S, int64_t V,
                         int64_t* part, int64_t nparts, int32_t* out, hipStream_t st) {
  if (S == 0) return hipSuccess;
  const int chunk = (int)((V + nparts - 1) / nparts);
  argmax_part_k<<<dim3((unsigned)nparts, (unsigned)S), TPB, 0, st>>>(logits, row_base, (int)V,
                                                                      (int)nparts, chunk, part);
  argmax_final_k<<<(unsigned)S, 1024, 0, st>>>(part, (int)nparts, out);
  return hipGetLastError();
}

hipError_t launch_argmax_final(const int64_t* part, int64_t S, int64_t nparts, int32_t* out,
                               hipStream_t st) {
  if (S == 0) return hipSuccess;
  argmax_final_k<<<(unsigned)S, 1024, 0, st>>>(part, (int)nparts, out);
  return hipGetLastError();
}

hipError_t launch_argmax_advance(const int64_t* part, int64_t S, int64_t nparts, int32_t* next_tok,
                                 int32_t* ids, int32_t* start_pos, int32_t* row_base, bool advance,
                                 hipStream_t st) {
  if (S == 0) return hipSuccess;
  argmax_advance_k<<<(unsigned)S, 1024, 0, st>>>(part, (int)nparts, next_tok, ids, start_pos,
                                                 row_base, (int)S, advance ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_advance(int32_t* ids, const int32_t* next_tok, int32_t* start_pos,
                          int32_t* row_base, int64_t S, hipStream_t st) {
  if (S == 0) return hipSuccess;
  advance_k<<<(unsigned)((S + 255) / 256), 256, 0, st>>>(ids, next_tok, start_pos, row_base, (int)S);
  return hipGetLastError();
}

// ------------------------------------------------------------- sampling

// Integer temperature / top-k sampling, one 1024-thread workgroup per row
// (BitExact blog intro: sampling rules in integer arithmetic; DetLLM blog,
// limits: integer sampling left open). Same function as detint.h states:
// keep the k highest-ranked ids (larger logit first, lower id on ties),
// weight each by E = DI-Exp(R((l - l_max) t_m, t_k)), draw t = floor(r D /
// 2^32) from the caller's uniform 32-bit r, and return the smallest id whose
// running weight exceeds t. Every reduction is an integer max, count or sum,
// so the thread layout changes no result.
//
// Layout: wave w owns ids [w Cw, (w + 1) Cw) in steps of 256 ids, lane i
// taking ids i, 64 + i, 128 + i, 192 + i of a step (each load reads 256
// contiguous bytes), and issues the loads of UB steps before using any (one
// workgroup per row needs many loads in flight). Each step's
// sum (weights, or ties at the top-k boundary) goes to LDS, where the wave
// holding a running-sum crossing finds its step with one ballot and reloads
// only that step. The k-th largest logit comes from a radix select on
// key - key_min (key the order-preserving unsigned form) in 8-bit digits
// aligned to the top bit of the row's span (so the first histogram spreads
// over 256 bins), with per-wave LDS histograms.
constexpr int SMT = 1024, SMW = SMT / 64, SPS = 256, SMS = 64, UB = 4;  // V <= SMW * SPS * SMS

__device__ __forceinline__ uint32_t okey(int32_t v) { return (uint32_t)v ^ 0x80000000u; }

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// The step q of a wave's range (n steps with sums s[0..n)) where the running
// sum first exceeds x (0 <= x < sum of all), and x minus the sum of the steps
// before q. Lane i scans steps i, i + 64, ... in rounds of 64.
__device__ __forceinline__ void step_of(const int64_t* s, int n, int64_t x, int lane, int& q,
                                        int64_t& rest) {
  int64_t run = 0;
  for (int b = 0; b < n; b += 64) {
    const int64_t inc = wave_incl_scan(b + lane < n ? s[b + lane] : 0, lane);
    const uint64_t m = __ballot(run + inc > x);
    if (m) {
      const int i = __builtin_ctzll(m);
      q = b + i;
      rest = x - run - (__shfl(inc, i) - s[b + i]);
      return;
    }
    run += __shfl(inc, 63);
  }
  q = n - 1;  // not reached for x below the total
  rest = 0;
}

// The offset, inside one step (value c[e] at offset 64 e + lane: counts or
// weights), where the running sum over the step first exceeds x.
__device__ __forceinline__ int crossing_in_step(const int64_t (&c)[4], int64_t x, int lane) {
  int64_t run = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t inc = run + wave_incl_scan(c[e], lane);
    const uint64_t m = __ballot(inc > x);
    if (m) return 64 * e + __builtin_ctzll(m);
    run = __shfl(inc, 63);
  }
  return 255;  // not reached for x below the step's sum
}

// One row (blockIdx.x) by one SMT-thread workgroup; also the in-kernel
// fallback of the sliced top-p pick.
__device__ __forceinline__ void sample_row(const int32_t* __restrict__ logits, int V, int keep,
                                           int32_t top_p, int32_t t_m, int32_t t_k,
                                           const uint32_t* __restrict__ draws,
                                           int32_t* __restrict__ out) {
  __shared__ int32_t hw[SMW][256];                // per-wave histograms (counts)
  __shared__ unsigned long long hm[SMW][256];     // per-wave histograms (weights, top-p)
  __shared__ int32_t hist[256];
  __shared__ int64_t histm[256];
  __shared__ int64_t red[16], wsum[SMW];
  __shared__ int64_t ssum[SMW][SMS];  // per-step sums of each wave's range
  __shared__ int64_t s_sel[3];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* l = logits + (size_t)r * V;
  const int Cw = ((V + SMW - 1) / SMW + SPS - 1) / SPS * SPS;
  const int wlo = min(V, wave * Cw), whi = min(V, wlo + Cw);
  const int nst = (whi - wlo + SPS - 1) / SPS;
  // f(step, values[4], valid[4]) over this wave's steps, UB steps of loads in
  // flight at a time (addresses clamped into the row; invalid ids flagged);
  // value e of a step is id wlo + step SPS + 64 e + lane
  auto sweep = [&](auto f) {
    for (int s0 = 0; s0 < nst; s0 += UB) {
      int32_t x[UB][4];
#pragma unroll
      for (int u = 0; u < UB; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[u][e] = l[min(wlo + (s0 + u) * SPS + 64 * e + lane, V - 1)];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        if (s0 + u >= nst) break;
        bool ok[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ok[e] = wlo + (s0 + u) * SPS + 64 * e + lane < whi;
        f(s0 + u, x[u], ok);
      }
    }
  };
  int32_t mx = INT32_MIN, mn = INT32_MAX;
  sweep([&](int, const int32_t(&x)[4], const bool(&ok)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ok[e]) {
        mx = max(mx, x[e]);
        mn = min(mn, x[e]);
      }
  });
  mx = (int32_t)block_max(mx, red);
  mn = (int32_t)(-block_max(-(int64_t)mn, red));
  const uint32_t kmin = okey(mn), span = okey(mx) - kmin;
  const int B = span ? 32 - __builtin_clz(span) : 0;
  // DI-Exp of the scaled gap: the branch-free exp_delta whenever t_k >= 1
  // (the same value), else as written
  auto expw = [&](int32_t v) -> int32_t {
    return t_k >= 1 ? exp_delta((uint32_t)((int64_t)mx - v), (uint32_t)t_m, t_k)
                    : diexp(R((int64_t)(v - (int64_t)mx) * t_m, t_k));
  };
  // kept(j): l_j > Lk, or l_j == Lk and j <= idk
  int32_t Lk = INT32_MIN;
  int idk = V - 1;
  auto kept = [&](int j, int32_t v) { return v > Lk || (v == Lk && j <= idk); };
  // the rem-th lowest id (rem >= 1) among the values equal to L
  auto nth_tie = [&](int32_t L, int64_t rem) -> int {
    int64_t wc = 0;
    __syncthreads();  // ssum / wsum / s_sel free
    sweep([&](int q, const int32_t(&x)[4], const bool(&ok)[4]) {
      int c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += ok[e] && x[e] == L;
      const int32_t st = wave_sum32(c);
      if (lane == 0) ssum[wave][q] = st;
      wc += st;
    });
    if (lane == 0) wsum[wave] = wc;
    __syncthreads();
    int64_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (before < rem && before + wsum[wave] >= rem) {
      int q;
      int64_t rest;
      step_of(ssum[wave], nst, rem - before - 1, lane, q, rest);
      const int base = wlo + q * SPS + lane;
      int64_t c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = base + 64 * e < whi && l[min(base + 64 * e, V - 1)] == L;
      const int at = crossing_in_step(c, rest, lane);
      if (lane == 0) s_sel[2] = wlo + q * SPS + at;
    }
    __syncthreads();
    return (int)s_sel[2];
  };
  // bucket from the top (lane i: bins 255 - 4i .. 252 - 4i) whose running
  // total first reaches rem; s_sel = (bucket, rem minus the bins above it)
  auto pick_bucket = [&](auto bins, int64_t rem) {
    if (wave == 0) {
      int64_t h[4], mine = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) mine += h[e] = bins(255 - 4 * lane - e);
      const int64_t inc = wave_incl_scan(mine, lane);
      const int i = __builtin_ctzll(__ballot(inc >= rem));  // the total reaches rem
      if (lane == i) {
        int64_t c = inc - mine;
        int e = 0;
        for (; e < 3; ++e) {
          if (c + h[e] >= rem) break;
          c += h[e];
        }
        s_sel[0] = 255 - 4 * i - e;
        s_sel[1] = rem - c;
      }
    }
    __syncthreads();
  };
  if (keep < V) {
    // radix select of the keep-th largest value on the order-preserving key
    uint32_t prefix = 0, pmask = 0;
    int64_t rem = keep;  // rank (from the top, 1-based) inside the current bucket
    for (int hi = B; hi > 0; hi -= 8) {  // digit = bits [lo, hi) of key - key_min
      const int lo = hi > 8 ? hi - 8 : 0;
      const uint32_t dm = (1u << (hi - lo)) - 1;
      for (int i = lane; i < 256; i += 64) hw[wave][i] = 0;
      __syncthreads();
      sweep([&](int, const int32_t(&x)[4], const bool(&ok)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t d = okey(x[e]) - kmin;
          if (ok[e] && (d & pmask) == prefix) atomicAdd(&hw[wave][(d >> lo) & dm], 1);
        }
      });
      __syncthreads();
      if (tid < 256) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < SMW; ++w) c += hw[w][tid];
        hist[tid] = c;
      }
      __syncthreads();
      pick_bucket([&](int d) { return (int64_t)hist[d]; }, rem);
      prefix |= (uint32_t)s_sel[0] << lo;
      pmask |= dm << lo;
      rem = s_sel[1];
    }
    Lk = (int32_t)((prefix + kmin) ^ 0x80000000u);
    idk = nth_tie(Lk, rem);
  }
  if (top_p < 65536) {
    // D_k, then the shortest prefix of the ranking whose weight reaches
    // P = ceil(top_p D_k / 2^16): a radix select on weight sums
    int64_t mine = 0;
    sweep([&](int q, const int32_t(&x)[4], const bool(&ok)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = wlo + q * SPS + 64 * e + lane;
        if (ok[e] && kept(j, x[e])) mine += expw(x[e]);
      }
    });
    const int64_t Dk = block_sum(mine, red);
    uint32_t prefix = 0, pmask = 0;
    int64_t rem = ((int64_t)top_p * Dk + 65535) >> 16;  // weight still to reach
    for (int hi = B; hi > 0; hi -= 8) {  // digit = bits [lo, hi) of key - key_min
      const int lo = hi > 8 ? hi - 8 : 0;
      const uint32_t dm = (1u << (hi - lo)) - 1;
      for (int i = lane; i < 256; i += 64) hm[wave][i] = 0;
      __syncthreads();
      sweep([&](int q, const int32_t(&x)[4], const bool(&ok)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = wlo + q * SPS + 64 * e + lane;
          const uint32_t d = okey(x[e]) - kmin;
          if (ok[e] && (d & pmask) == prefix && kept(j, x[e]))
            atomicAdd(&hm[wave][(d >> lo) & dm], (unsigned long long)expw(x[e]));
        }
      });
      __syncthreads();
      if (tid < 256) {
        unsigned long long c = 0;
#pragma unroll
        for (int w = 0; w < SMW; ++w) c += hm[w][tid];
        histm[tid] = (int64_t)c;
      }
      __syncthreads();
      pick_bucket([&](int d) { return histm[d]; }, rem);
      prefix |= (uint32_t)s_sel[0] << lo;
      pmask |= dm << lo;
      rem = s_sel[1];
    }
    const int32_t Lp = (int32_t)((prefix + kmin) ^ 0x80000000u);
    // every id at Lp weighs expw(Lp) > 0: ceil(rem / weight) of them, lowest ids first
    const uint64_t wp = (uint64_t)expw(Lp);
    const int64_t need = (int64_t)udiv64((uint64_t)rem + wp - 1, wp);
    idk = nth_tie(Lp, need);
    Lk = Lp;
  }
  int64_t ws = 0;
  __syncthreads();  // ssum / wsum free
  sweep([&](int q, const int32_t(&x)[4], const bool(&ok)[4]) {
    int32_t sm = 0;  // at most 4 * 2^15 per lane, 2^23 per step
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = wlo + q * SPS + 64 * e + lane;
      sm += ok[e] && kept(j, x[e]) ? expw(x[e]) : 0;
    }
    const int32_t st = wave_sum32(sm);
    if (lane == 0) ssum[wave][q] = st;
    ws += st;
  });
  if (lane == 0) wsum[wave] = ws;
  __syncthreads();
  int64_t before = 0, D = 0;
#pragma unroll
  for (int w = 0; w < SMW; ++w) {
    before += w < wave ? wsum[w] : 0;
    D += wsum[w];
  }
  const int64_t t = (int64_t)(((unsigned __int128)draws[r] * (uint64_t)D) >> 32);  // in [0, D)
  if (before <= t && t < before + wsum[wave]) {
    int q;
    int64_t rest;
    step_of(ssum[wave], nst, t - before, lane, q, rest);
    const int base = wlo + q * SPS + lane;
    int64_t c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = base + 64 * e;
      const int32_t v = l[min(j, V - 1)];
      c[e] = j < whi && kept(j, v) ? expw(v) : 0;
    }
    const int at = crossing_in_step(c, rest, lane);
    if (lane == 0) out[r] = wlo + q * SPS + at;
  }
}

__global__ __launch_bounds__(SMT) void sample_k(const int32_t* __restrict__ logits, int V, int keep,
                                               int32_t top_p, int32_t t_m, int32_t t_k,
                                               const uint32_t* __restrict__ draws,
                                               int32_t* __restrict__ out) {
  sample_row(logits, V, keep, top_p, t_m, t_k, draws, out);
}

// Plain temperature sampling (every id kept) spread over the chip: slices of
// 1024 ids, one 256-thread workgroup each, wave w of a slice owning its
// w-th 256-id step (ids 64 e + lane within it, as in sample_k).
//   1. slice maxima;  2. each slice reduces the maxima and writes its
//   per-step DI-Exp weight sums;  3. one workgroup per row scans the step
//   sums in id order, places the draw and reloads that step.
// The same integer function as sample_k with all ids kept.
constexpr int SLC = 1024, SLT = 256;

__global__ __launch_bounds__(SLT) void sample_max_k(const int32_t* __restrict__ logits, int V,
                                                    int P, int32_t* __restrict__ smax) {
  __shared__ int64_t red[16];
  const int r = blockIdx.y, p = blockIdx.x;
  const int32_t* l = logits + (size_t)r * V;
  int32_t m = INT32_MIN;
#pragma unroll
  for (int i = 0; i < SLC / SLT; ++i) {
    const int j = p * SLC + i * SLT + threadIdx.x;
    m = max(m, l[min(j, V - 1)]);  // clamped ids repeat a real value
  }
  m = (int32_t)block_max(m, red);
  if (threadIdx.x == 0) smax[(size_t)r * P + p] = m;
}

__device__ __forceinline__ int32_t row_max_of(const int32_t* smax, int P, int64_t* red) {
  int32_t m = INT32_MIN;
  for (int i = threadIdx.x; i < P; i += blockDim.x) m = max(m, smax[i]);
  return (int32_t)block_max(m, red);
}

__device__ __forceinline__ int32_t expw_of(int32_t v, int32_t mx, int32_t t_m, int32_t t_k) {
  return t_k >= 1 ? exp_delta((uint32_t)((int64_t)mx - v), (uint32_t)t_m, t_k)
                  : diexp(R((int64_t)(v - (int64_t)mx) * t_m, t_k));
}

__global__ __launch_bounds__(SLT) void sample_wsum_k(const int32_t* __restrict__ logits, int V,
                                                     int P, int32_t t_m, int32_t t_k,
                                                     const int32_t* __restrict__ smax,
                                                     int32_t* __restrict__ ssum) {
  __shared__ int64_t red[16];
  const int r = blockIdx.y, p = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int32_t* l = logits + (size_t)r * V;
  const int32_t mx = row_max_of(smax + (size_t)r * P, P, red);
  const int base = p * SLC + w * 256 + lane;
  int32_t sm = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = base + 64 * e;
    const int32_t v = l[min(j, V - 1)];
    sm += j < V ? expw_of(v, mx, t_m, t_k) : 0;
  }
  sm = wave_sum32(sm);
  if (lane == 0) ssum[((size_t)r * P + p) * 4 + w] = sm;
}

__global__ __launch_bounds__(SLT) void sample_pick_k(const int32_t* __restrict__ logits, int V,
                                                     int P, int32_t t_m, int32_t t_k,
                                                     const int32_t* __restrict__ smax,
                                                     const int32_t* __restrict__ ssum,
                                                     const uint32_t* __restrict__ draws,
                                                     int32_t* __restrict__ out) {
  __shared__ int64_t red[16], wtot[SLT / 64];
  __shared__ int s_step;
  __shared__ int64_t s_rest;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* l = logits + (size_t)r * V;
  const int32_t mx = row_max_of(smax + (size_t)r * P, P, red);
  const int32_t* sr = ssum + (size_t)r * P * 4;
  const int n = 4 * P;  // steps of 256 ids, in id order
  // thread t holds steps 4t .. 4t + 3 (n <= 1024)
  int64_t c[4], mine = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c[e] = 4 * tid + e < n ? sr[4 * tid + e] : 0;
    mine += c[e];
  }
  const int64_t inc = wave_incl_scan(mine, lane);
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  int64_t before = 0, D = 0;
#pragma unroll
  for (int w = 0; w < SLT / 64; ++w) {
    before += w < wave ? wtot[w] : 0;
    D += wtot[w];
  }
  const int64_t t = (int64_t)(((unsigned __int128)draws[r] * (uint64_t)D) >> 32);  // in [0, D)
  const int64_t lo = before + inc - mine;  // weight before this thread's steps
  if (lo <= t && t < lo + mine) {
    int64_t run = lo;
    int e = 0;
    for (; e < 3; ++e) {
      if (run + c[e] > t) break;
      run += c[e];
    }
    s_step = 4 * tid + e;
    s_rest = t - run;
  }
  __syncthreads();
  if (wave == 0) {
    const int base = s_step * 256 + lane;
    int64_t cw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = base + 64 * e;
      cw[e] = j < V ? expw_of(l[min(j, V - 1)], mx, t_m, t_k) : 0;
    }
    const int at = crossing_in_step(cw, s_rest, lane);
    if (lane == 0) out[r] = s_step * 256 + at;
  }
}

// Top-k (and top-p after it) sampling spread over the chip. A global top-k id is
// among the top min(k, n) of its own slice, so:
//   1. each 2048-id slice selects its top min(k, slice) ids (radix select on
//      the order key, ties to the lowest ids) and writes them, in id order,
//      as (key << 32 | ~id) into a row-private candidate list (kc entries per
//      slice, padded with 0, which no id's entry equals);
//   2. one workgroup per row selects the top k among the candidates, weighs
//      them against the row maximum, keeps the top-p nucleus of those and
//      places the draw in id order.
// The same integer function as sample_k.
constexpr int TKS = 2048, TKT = 512, TKN = TKS / TKT;  // ids per slice, threads, ids per thread
constexpr int TPT = 1024;             // pick threads
constexpr int TKC = 16 * TPT;         // candidate row stride: 16 a thread for top-p alone
constexpr int TKK = 8 * TPT;          // top-k: 8 a thread

// Inclusive prefix sum over the workgroup in thread order; also the total.
template <int NT>
__device__ __forceinline__ int64_t block_incl_scan(int64_t v, int64_t* wt, int64_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t inc = wave_incl_scan(v, lane);
  __syncthreads();  // wt free from its previous use
  if (lane == 63) wt[wave] = inc;
  __syncthreads();
  int64_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    before += w < wave ? wt[w] : 0;
    tot += wt[w];
  }
  total = tot;
  return before + inc;
}

// The same in 32 bits (half the lane exchanges), for sums below 2^31.
__device__ __forceinline__ int32_t wave_incl_scan32(int32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

template <int NT>
__device__ __forceinline__ int32_t block_incl_scan32(int32_t v, int32_t* wt, int32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t inc = wave_incl_scan32(v, lane);
  __syncthreads();  // wt free from its previous use
  if (lane == 63) wt[wave] = inc;
  __syncthreads();
  int32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    before += w < wave ? wt[w] : 0;
    tot += wt[w];
  }
  total = tot;
  return before + inc;
}

// Radix select over the valid keys held by the workgroup, key e weighing
// wv(e) (all 1: the n-th largest key), on digits of key - (smallest key) taken 8
// bits a pass from the top of that span (so the first pass already spreads
// keys that share their high bits over the bins). Finds
// the largest T such that the keys at or above T weigh at least n
// (1 <= n <= total weight, total below 2^31), and returns in tneed the
// weight still needed from the keys equal to T (>= 1) beyond those above it.
template <int NT, int N, typename WF>
__device__ __forceinline__ void radix_nth(const uint32_t (&key)[N], uint32_t okm, WF wv, int n,
                                          int32_t (*hw)[256],
                                          int32_t* wt, int64_t* red, int* sel, uint32_t& T,
                                          int& tneed) {
  uint32_t kmx = 0, kmn = 0xFFFFFFFFu;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const bool ok = okm >> e & 1;
    kmx = ok && key[e] > kmx ? key[e] : kmx;
    kmn = ok && key[e] < kmn ? key[e] : kmn;
  }
  kmx = (uint32_t)block_max((int64_t)kmx, red);
  kmn = ~(uint32_t)block_max((int64_t)(~kmn), red);
  const int B = 32 - __clz(kmx - kmn);  // span bits (0: one distinct key)
  uint32_t prefix = 0, pmask = 0;
  int rem = n;
  for (int hi = B; hi > 0; hi -= 8) {  // digit = bits [lo, hi) of key - kmn
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint32_t dm = (1u << (hi - lo)) - 1;
    for (int i = threadIdx.x; i < NT / 64 * 256; i += NT) hw[i >> 8][i & 255] = 0;
    __syncthreads();
    int32_t* mh = hw[threadIdx.x >> 6];  // this wave's histogram
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const uint32_t d = key[e] - kmn;
      if ((okm >> e & 1) && (d & pmask) == prefix) atomicAdd(&mh[(d >> lo) & dm], wv(e));
    }
    __syncthreads();
    // bins from the top down: thread i holds bin 255 - i
    int32_t c = 0;  // at most the total weight, below 2^31
    if (threadIdx.x < 256)
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) c += hw[w][255 - threadIdx.x];
    int32_t tot;
    const int32_t inc = block_incl_scan32<NT>(c, wt, tot);
    if (inc - c < rem && rem <= inc) {
      sel[0] = 255 - (int)threadIdx.x;
      sel[1] = rem - (inc - c);
    }
    __syncthreads();
    prefix |= (uint32_t)sel[0] << lo;
    pmask |= dm << lo;
    rem = sel[1];
  }
  T = prefix + kmn;
  tneed = rem;
}

// Bit e of the result: valid key e above T, or equal to T and among the
// first tneed such keys in thread-major order (which is id order).
template <int NT, int N>
__device__ __forceinline__ uint32_t take_top(const uint32_t (&key)[N], uint32_t okm, uint32_t T,
                                             int tneed, int32_t* wt) {
  int ties = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) ties += (okm >> e & 1) && key[e] == T;
  int32_t tt;
  int tb = block_incl_scan32<NT>(ties, wt, tt) - ties;
  uint32_t tm = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const bool ok = okm >> e & 1, eq = ok && key[e] == T;
    tm |= (uint32_t)(ok && (key[e] > T || (eq && tb < tneed))) << e;
    tb += eq;
  }
  return tm;
}

__global__ __launch_bounds__(TKT) void topk_slice_k(const int32_t* __restrict__ logits, int V,
                                                    int kc, uint64_t* __restrict__ cand,
                                                    uint32_t* __restrict__ sT) {
  __shared__ int32_t hw[TKT / 64][256];
  __shared__ int32_t wt[TKT / 64];
  __shared__ int64_t red[16];
  __shared__ int sel[2];
  const int r = blockIdx.y, p = blockIdx.x, tid = threadIdx.x;
  const int32_t* l = logits + (size_t)r * V;
  const int j0 = p * TKS + TKN * tid;
  uint32_t key[TKN], okm = 0;
#pragma unroll
  for (int e = 0; e < TKN; ++e) {
    okm |= (uint32_t)(j0 + e < V) << e;
    key[e] = okey(l[min(j0 + e, V - 1)]);
  }
  const int kk = min(kc, V - p * TKS);  // ids kept from this slice
  uint32_t T;
  int tneed;
  radix_nth<TKT, TKN>(key, okm, [](int) { return 1; }, kk, hw, wt, red, sel, T, tneed);
  const uint32_t take = take_top<TKT, TKN>(key, okm, T, tneed, wt);
  const int nt = __popc(take);
  int32_t tot;
  int at = block_incl_scan32<TKT>(nt, wt, tot) - nt;
  uint64_t* dst = cand + (size_t)r * TKC + (size_t)p * kc;
#pragma unroll
  for (int e = 0; e < TKN; ++e)
    if ((take >> e & 1) && at < kk) dst[at++] = (uint64_t)key[e] << 32 | (uint32_t)~(uint32_t)(j0 + e);
  for (int i = kk + tid; i < kc; i += TKT) dst[i] = 0;
  // the cut key of a slice that had more ids than it kept (0: kept them all)
  if (sT && tid == 0) sT[(size_t)r * gridDim.x + p] = min(TKS, V - p * TKS) > kc ? T : 0;
}

// NUC: top-p over the whole row (no top-k). Every candidate is kept, the
// nucleus target comes from the weight of the whole row (the per-step sums
// of sample_wsum_k), and the result stands only if the nucleus threshold
// key lies above every cut key sT of a slice that had more ids than it
// kept: then the candidates hold every id at or above that key, so the
// nucleus, its ties and the draw are the whole row's. Otherwise the
// workgroup samples the row from its logits as sample_k does.
template <bool NUC, int PT>
__global__ __launch_bounds__(PT) void topk_pick_k(const uint64_t* __restrict__ cand, int nc,
                                                   int keep, int32_t top_p, int32_t t_m, int32_t t_k,
                                                   const uint32_t* __restrict__ draws,
                                                   int32_t* __restrict__ out,
                                                   const int32_t* __restrict__ ssum, int P,
                                                   const uint32_t* __restrict__ sT, int P2,
                                                   const int32_t* __restrict__ logits) {
  constexpr int N = NUC ? TKC / PT : TKK / TPT;  // candidates a thread
  __shared__ int32_t hw[PT / 64][256];
  __shared__ int32_t wl[N][PT];  // candidate weights, element-major
  __shared__ int32_t wt[PT / 64];
  __shared__ int64_t wt64[PT / 64], red[16];
  __shared__ int sel[2];
  const int r = blockIdx.x, tid = threadIdx.x;
  const uint64_t* c = cand + (size_t)r * TKC + N * tid;  // this thread's entries
  const int nmine = min(N, max(0, nc - N * tid));
  uint32_t key[N], km = 0, okm = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const uint64_t cv = e < nmine ? c[e] : 0;
    okm |= (uint32_t)(cv != 0) << e;
    key[e] = (uint32_t)(cv >> 32);
    km = cv != 0 && key[e] > km ? key[e] : km;
  }
  const int32_t mx = (int32_t)((uint32_t)block_max((int64_t)km, red) ^ 0x80000000u);
  // each weight computed once, kept in LDS (not registers: pressure)
#pragma unroll
  for (int e = 0; e < N; ++e)
    wl[e][tid] = okm >> e & 1 ? expw_of((int32_t)(key[e] ^ 0x80000000u), mx, t_m, t_k) : 0;
  auto wgt = [&](int e) -> int32_t { return wl[e][tid]; };
  uint32_t take = okm;
  if constexpr (!NUC) {
    uint32_t T;
    int tneed;
    radix_nth<PT, N>(key, okm, [](int) { return 1; }, keep, hw, wt, red, sel, T, tneed);
    take = take_top<PT, N>(key, okm, T, tneed, wt);
  }
  auto weight_of = [&](uint32_t m) {  // candidate weights total below 2^30
    int32_t s = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) s += m >> e & 1 ? wgt(e) : 0;
    return s;
  };
  int32_t mine = weight_of(take);
  if (NUC || top_p < 65536) {
    // the shortest prefix of the ranking whose weight reaches
    // ceil(top_p D / 2^16), D the weight of the kept ids (of the whole row
    // for NUC): a weighted select over the candidates (their weight is below
    // 2^30), then ceil(rest / weight of that key) of its ties, lowest ids first
    int32_t Wc;
    block_incl_scan32<PT>(mine, wt, Wc);
    int64_t Dk = Wc;
    uint32_t tc = 0;
    if constexpr (NUC) {
      int64_t ds = 0;
      for (int i = tid; i < 4 * P; i += PT) ds += ssum[(size_t)r * P * 4 + i];
      block_incl_scan<PT>(ds, wt64, Dk);
      for (int i = tid; i < P2; i += PT) tc = max(tc, sT[(size_t)r * P2 + i]);
      tc = (uint32_t)block_max((int64_t)tc, red);
    }
    const int64_t need = ((int64_t)top_p * Dk + 65535) >> 16;
    uint32_t Lp = 0;
    int rest = 0;
    bool good = need <= Wc;  // uniform over the workgroup
    if (good) {
      radix_nth<PT, N>(key, take, wgt, (int)need, hw, wt, red, sel, Lp, rest);
      good = !NUC || Lp > tc;
    }
    if constexpr (NUC) {
      if (!good) {  // uniform: the whole row, one workgroup
        sample_row(logits, keep, keep, top_p, t_m, t_k, draws, out);
        return;
      }
    }
    const int wp = expw_of((int32_t)(Lp ^ 0x80000000u), mx, t_m, t_k);  // > 0
    take = take_top<PT, N>(key, take, Lp, (int)udiv32((uint32_t)(rest + wp - 1), (uint32_t)wp), wt);
    mine = weight_of(take);
  }
  int32_t D;
  int32_t run = block_incl_scan32<PT>(mine, wt, D) - mine;  // weight of earlier ids
  const int32_t t = (int32_t)(((uint64_t)draws[r] * (uint64_t)D) >> 32);  // in [0, D)
  if (run <= t && t < run + mine) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const int32_t w = take >> e & 1 ? wgt(e) : 0;
      if (run + w > t) {
        out[r] = (int32_t)~(uint32_t)c[e];  // reload the entry for its id
        break;
      }
      run += w;
    }
  }
}

// Workspace: candidates [R][TKC] u64 | slice maxima [R][P] | step sums
// [R][P][4] | slice cut keys [R][P2]  (P = 1024-id slices, P2 = 2048-id
// slices); the plain path uses maxima and step sums only.
int64_t sample_workspace_bytes(int64_t R, int64_t V) {
  const int64_t P = (V + SLC - 1) / SLC, P2 = (V + TKS - 1) / TKS;
  return R * (TKC * 8 + P * 4 * (1 + 4) + P2 * 4);
}

hipError_t launch_sample(const int32_t* logits, int64_t R, int64_t V, int64_t keep, int32_t top_p,
                         int32_t t_m, int32_t t_k, const uint32_t* draws, int32_t* out, void* ws,
                         int64_t ws_bytes, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const int64_t P = (V + SLC - 1) / SLC, P2 = (V + TKS - 1) / TKS;
  const bool fits = ws && ws_bytes >= sample_workspace_bytes(R, V) && R <= 65535;
  uint64_t* cand = (uint64_t*)ws;
  int32_t* smax = (int32_t*)(cand + R * TKC);
  int32_t* ssum = smax + R * P;
  uint32_t* sT = (uint32_t*)(ssum + R * P * 4);
  if (fits && keep >= V && top_p >= 65536) {
    sample_max_k<<<dim3((unsigned)P, (unsigned)R), SLT, 0, st>>>(logits, (int)V, (int)P, smax);
    sample_wsum_k<<<dim3((unsigned)P, (unsigned)R), SLT, 0, st>>>(logits, (int)V, (int)P, t_m, t_k,
                                                                  smax, ssum);
    sample_pick_k<<<(unsigned)R, SLT, 0, st>>>(logits, (int)V, (int)P, t_m, t_k, smax, ssum, draws,
                                               out);
    return hipGetLastError();
  }
  const int64_t kc = std::min<int64_t>(keep, TKS);
  if (fits && keep < V && P2 * kc <= TKK) {
    topk_slice_k<<<dim3((unsigned)P2, (unsigned)R), TKT, 0, st>>>(logits, (int)V, (int)kc, cand,
                                                                  nullptr);
    // up to 4096 candidates: 512 threads (the pick is a chain of workgroup
    // scans and barriers, each cheaper with half the waves)
    if (P2 * kc <= 4096)
      topk_pick_k<false, 512><<<(unsigned)R, 512, 0, st>>>(cand, (int)(P2 * kc), (int)keep, top_p,
                                                          t_m, t_k, draws, out, nullptr, 0, nullptr,
                                                          0, nullptr);
    else
      topk_pick_k<false, TPT><<<(unsigned)R, TPT, 0, st>>>(cand, (int)(P2 * kc), (int)keep, top_p,
                                                          t_m, t_k, draws, out, nullptr, 0, nullptr,
                                                          0, nullptr);
    return hipGetLastError();
  }
  if (fits && keep >= V) {
    // top-p alone: each slice's top kn ids as candidates, the whole row's
    // weight from the step sums; a row whose nucleus reaches below a slice's
    // cut is sampled from its logits by its pick workgroup
    const int64_t kn = std::min<int64_t>(TKS, TKC / P2);
    sample_max_k<<<dim3((unsigned)P, (unsigned)R), SLT, 0, st>>>(logits, (int)V, (int)P, smax);
    sample_wsum_k<<<dim3((unsigned)P, (unsigned)R), SLT, 0, st>>>(logits, (int)V, (int)P, t_m, t_k,
                                                                  smax, ssum);
    topk_slice_k<<<dim3((unsigned)P2, (unsigned)R), TKT, 0, st>>>(logits, (int)V, (int)kn, cand, sT);
    topk_pick_k<true, TPT><<<(unsigned)R, TPT, 0, st>>>(cand, (int)(P2 * kn), (int)V, top_p, t_m, t_k,
                                                   draws, out, ssum, (int)P, sT, (int)P2, logits);
    return hipGetLastError();
  }
  sample_k<<<(unsigned)R, SMT, 0, st>>>(logits, (int)V, (int)keep, top_p, t_m, t_k, draws, out);
  return hipGetLastError();
}

}  // namespace detint
