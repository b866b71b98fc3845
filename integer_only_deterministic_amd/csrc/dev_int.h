// Device integer primitives for gfx950 kernels of libdetint.
//
// Everything here is integer arithmetic. Division and square root are
// bit-serial integer routines rather than the compiler's `/`, whose AMDGPU
// lowering seeds its quotient with a float reciprocal; these run once per row
// (or once per element on 16-bit quotients) and keep the ISA float-free.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace detint {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Round-half-up shift R(x, s): floor(x / 2^s + 1/2) for s >= 1, x for s = 0,
// x * 2^-s for s < 0 (DetLLM blog "DetLLM": one fixed rounding rule for every
// dyadic rescale). Shifts past 62 give 0 (inputs here stay below 2^61).
__device__ __forceinline__ int64_t R(int64_t x, int s) {
  if (s > 0) {
    if (s > 62) return 0;
    return (x + (int64_t(1) << (s - 1))) >> s;
  }
  return x * (int64_t(1) << (-s));
}

__device__ __forceinline__ int64_t R128(__int128 x, int s) {
  if (s > 0) {
    if (s > 126) return 0;
    return (int64_t)((x + ((__int128)1 << (s - 1))) >> s);
  }
  return (int64_t)(x * ((__int128)1 << (-s)));
}

__device__ __forceinline__ int bitlen64(uint64_t x) { return x ? 64 - __builtin_clzll(x) : 0; }

// ------------------------------------------------------------------------
// Device bound flags (BitExact LLM blog, "Reproducibility has a cost": range
// checks before residual additions, on the final logits and on the linear
// epilogues). A kernel that sees an intermediate outside its written bound
// ORs a bit into a flag word and carries on (memory-safe, result undefined);
// detint_check reads and clears the words. The bits are the DETINT_BOUND_*
// values of detint.h. One word per translation unit: static device storage
// on each GPU, no allocation.
enum : uint32_t {
  kBoundResidual = 1u,  // residual stream |h| >= 2^25 (adds, embedding)
  kBoundInt32 = 2u,     // a FIX / logits / RES_ADD result outside int32
  kBoundNorm = 4u,      // RMSNorm row with sum of squares >= 2^62
  kBoundSwiglu = 8u,    // SwiGLU gate or up outside (-2^24, 2^24)
  kBoundId = 16u,       // token id outside [0, vocab)
  kBoundWeight = 32u,   // a bf16 weight the exact-mode integers cannot hold
  kBoundPage = 64u,     // a KV block-table entry outside the page pool
};
static __device__ uint32_t g_bound_flags;

// OR `bits` into the flag word when nonzero (rare: only on a violation).
__device__ __forceinline__ void bound_raise(uint32_t bits) {
  if (bits) atomicOr(&g_bound_flags, bits);
}
// 1 when |t| >= 2^b (0 < b <= 62)
__device__ __forceinline__ uint32_t out_of(int64_t t, int b) {
  return (uint64_t)(t + (int64_t(1) << b) - 1) >= (uint64_t(1) << (b + 1)) - 1 ? 1u : 0u;
}
// 1 when |t| >= 2^b for an int32 t (0 < b <= 30), in 32-bit arithmetic
__device__ __forceinline__ uint32_t out_of32(int32_t t, int b) {
  return (uint32_t)t + ((1u << b) - 1u) >= (2u << b) - 1u ? 1u : 0u;
}
// flag bit of a residual-add result t with bound 2^res_bits (0: int32)
__device__ __forceinline__ uint32_t res_check(int64_t t, int res_bits) {
  return res_bits > 0 ? (out_of(t, res_bits) ? kBoundResidual : 0u)
                      : ((uint64_t)(t + 2147483648LL) >> 32 ? kBoundInt32 : 0u);
}
// flag bit of a FIX result outside int32
__device__ __forceinline__ uint32_t i32_check(int64_t y) {
  return (uint64_t)(y + 2147483648LL) >> 32 ? kBoundInt32 : 0u;
}

// R(x, e) for a shift e >= 0 known to be the same across the wave (a DQ
// exponent): branch-free, the rounding half is 2^e >> 1 (0 for e = 0).
__device__ __forceinline__ int64_t R_nn(int64_t x, int e) {
  e = __builtin_amdgcn_readfirstlane(e);
  return (x + ((int64_t(1) << e) >> 1)) >> e;
}

__device__ __forceinline__ int8_t clamp8(int64_t x) {
  return (int8_t)(x > 127 ? 127 : (x < -127 ? -127 : x));
}

__device__ __forceinline__ uint64_t uabs64(int64_t x) {
  return x < 0 ? (uint64_t)0 - (uint64_t)x : (uint64_t)x;
}

// floor(n / d) for d > 0 by restoring binary long division.
__device__ __forceinline__ uint64_t udiv64(uint64_t n, uint64_t d) {
  uint64_t q = 0, r = 0;
  for (int i = bitlen64(n) - 1; i >= 0; --i) {
    r = (r << 1) | ((n >> i) & 1);
    if (r >= d) {
      r -= d;
      q |= uint64_t(1) << i;
    }
  }
  return q;
}

// floor(n / d) for 32-bit n and d >= 1, restoring division from the top bit
// of n: index arithmetic (tile numbers, head groups, tie counts) without the
// compiler's `/`, whose expansion goes through a float reciprocal.
__device__ __forceinline__ uint32_t udiv32(uint32_t n, uint32_t d) {
  uint32_t q = 0, r = 0;
  for (int i = 31 - __builtin_clz(n | 1); i >= 0; --i) {
    r = (r << 1) | ((n >> i) & 1u);
    if (r >= d) {
      r -= d;
      q |= 1u << i;
    }
  }
  return q;
}

// floor(n / d) when the quotient is known to be below 2^QB: QB restoring
// steps on the shifted divisor (d << (QB - 1) must not overflow).
template <int QB>
__device__ __forceinline__ uint64_t udiv_q(uint64_t n, uint64_t d) {
  uint64_t q = 0;
#pragma unroll
  for (int i = QB - 1; i >= 0; --i) {
    const uint64_t t = d << i;
    if (n >= t) {
      n -= t;
      q |= uint64_t(1) << i;
    }
  }
  return q;
}

// RD(a, b) = floor((2a + b) / 2b), a >= 0, b > 0.
__device__ __forceinline__ int64_t div_round(int64_t a, int64_t b) {
  return (int64_t)udiv64(2 * (uint64_t)a + (uint64_t)b, 2 * (uint64_t)b);
}

// floor(sqrt(n)), digit-by-digit from the highest even bit of n.
__device__ __forceinline__ uint64_t isqrt64(uint64_t n) {
  if (n == 0) return 0;
  uint64_t res = 0;
  uint64_t bit = uint64_t(1) << ((bitlen64(n) - 1) & ~1);
  while (bit) {
    if (n >= res + bit) {
      n -= res + bit;
      res = (res >> 1) + bit;
    } else {
      res >>= 1;
    }
    bit >>= 2;
  }
  return res;
}

// Inverse RMS of n entries with sum of squares S > 0: 1/sqrt(S/n) ~ m * 2^-sh,
// m in [2^14, 2^15) (DetLLM README "Layout": DI-RMSNorm). The same integer
// function as the definition in detint.h; the division by n is a shift when
// n is a power of two, and RD(2^T, r) has a quotient <= 2^15.
__device__ __forceinline__ void irms(int64_t S, int64_t n, int32_t& m, int32_t& sh) {
  const int b = bitlen64((uint64_t)S);
  const int c = b < 62 ? (62 - b) >> 1 : 0;
  const uint64_t num = (uint64_t)S << (2 * c);
  const uint64_t u = (n & (n - 1)) == 0 ? num >> (__builtin_ctzll((uint64_t)n)) : udiv64(num, (uint64_t)n);
  const uint64_t r = isqrt64(u);
  int T = bitlen64(r) + 14;
  int64_t mm = (int64_t)udiv_q<16>((uint64_t(1) << (T + 1)) + r, 2 * r);
  if (mm == (1 << 15)) {
    mm = 1 << 14;
    T -= 1;
  }
  m = (int32_t)mm;
  sh = T - c;
}

// ------------------------------------------------------ wave-parallel forms
// Same integer functions as isqrt64 / udiv_q / irms, computed by a whole
// wave (all 64 lanes active, uniform inputs): the result is found 6 bits at a
// time, lane l testing the candidate with l in the current 6-bit digit; the
// test is monotone in l, so the highest passing lane (ballot + clz) gives the
// digit. About 6 rounds replace 31-47 dependent serial steps.

// A wave-uniform 64-bit value moved to scalar registers, so that the
// bookkeeping below runs on the scalar unit.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// floor(sqrt(u)) for u < 2^64: six rounds at fixed digit positions 30, 24,
// ..., 0 (a round above the root's top bit finds digit 0), branch-free. In
// the first round only candidates below 2^32 (lanes 0..3) take part.
__device__ __forceinline__ uint64_t isqrt_wave(uint64_t u) {
  const uint32_t lane = threadIdx.x & 63;
  u = uniform64(u);
  uint32_t r = 0;
#pragma unroll
  for (int s = 30; s >= 0; s -= 6) {
    const uint32_t c = r | (lane << s);  // exact for the lanes that take part
    const bool ok = (s < 30 || lane < 4) & ((uint64_t)c * c <= u);
    r |= (uint32_t)(63 - __builtin_clzll(__ballot(ok))) << s;
  }
  return r;
}

// floor(n / d), d > 0, when the quotient is known to be below 2^QB and
// 2^QB * d < 2^64 (so every candidate product fits 64 bits); branch-free.
template <int QB>
__device__ __forceinline__ uint64_t udiv_wave(uint64_t n, uint64_t d) {
  const uint64_t lane = threadIdx.x & 63;
  n = uniform64(n);
  d = uniform64(d);
  uint64_t q = 0;
#pragma unroll
  for (int s = ((QB - 1) / 6) * 6; s >= 0; s -= 6) {
    const uint64_t c = q | (lane << s);
    const bool ok = (QB - s >= 6 || lane < (uint64_t(1) << (QB - s))) & (c * d <= n);
    q |= (uint64_t)(63 - __builtin_clzll(__ballot(ok))) << s;
  }
  return q;
}

// irms (see above) by a whole wave.
__device__ __forceinline__ void irms_wave(int64_t S, int64_t n, int32_t& m, int32_t& sh) {
  S = (int64_t)uniform64((uint64_t)S);
  const int b = bitlen64((uint64_t)S);
  const int c = b < 62 ? (62 - b) >> 1 : 0;
  const uint64_t num = (uint64_t)S << (2 * c);
  const uint64_t u = (n & (n - 1)) == 0 ? num >> (__builtin_ctzll((uint64_t)n)) : udiv64(num, (uint64_t)n);
  const uint64_t r = isqrt_wave(u);
  int T = bitlen64(r) + 14;
  int64_t mm = (int64_t)udiv_wave<16>((uint64_t(1) << (T + 1)) + r, 2 * r);
  if (mm == (1 << 15)) {
    mm = 1 << 14;
    T -= 1;
  }
  m = (int32_t)mm;
  sh = T - c;
}

// DI-Exp (DetLLM README "Layout"; shift-based exp as in I-ViT's Shiftmax):
// u <= 0 is a base-2 exponent in Q15; returns E ~ 2^15 * 2^(u / 2^15), using
// 2^(-r/2^15) ~ 1 - r/2^16 on the fractional part and a shift for the rest.
__device__ __forceinline__ int32_t diexp(int64_t u) {
  const int64_t v = -u;
  const int64_t n = v >> 15;
  const int64_t r = v & 32767;
  const int64_t f = 32768 - ((r + 1) >> 1);
  if (n > 30) return 0;
  return (int32_t)R(f, (int)n);
}

// E = DI-Exp(R((s - mx) M, sh)) for s <= mx, written for x = (mx - s) M >= 0:
// R(-x, sh) = -((x + 2^(sh-1) - 1) >> sh) for sh >= 1, so DI-Exp's
// magnitude is v = (x + 2^(sh-1) - 1) >> sh and E = R(2^15 - R(v mod 2^15, 1),
// v >> 15), zero once v >> 15 > 30. Needs 1 <= sh <= 62 and M > 0; other
// rows take diexp(R(...)) as written.
__device__ __forceinline__ int32_t exp_delta(uint32_t delta, uint32_t M, int sh) {
  const uint64_t x = (uint64_t)delta * M;
  const uint64_t v = (x + (uint64_t(1) << (sh - 1)) - 1) >> sh;
  const uint32_t vv = (uint32_t)v, n = min(vv >> 15, 31u);
  const uint32_t f = 32768u - (((vv & 32767u) + 1u) >> 1);
  return v >= (uint64_t(31) << 15) ? 0 : (int32_t)((f + ((1u << n) >> 1)) >> n);
}

// Integer sigmoid in Q15 of a gate g with f_a fractional bits, given the
// exponent multiplier (Mg, Kg): E = DI-Exp(-R(|g| Mg, Kg)),
// s+ = RD(2^30, 2^15 + E) = floor((2^31 + b) / 2b) with b = 2^15 + E, a
// quotient in [2^14, 2^15]: 15 restoring steps in 32 bits (b = 2^16 exactly,
// i.e. E = 2^15, gives 2^14 directly), s = s+ or 2^15 - s+ by the sign of g.
__device__ __forceinline__ int32_t sigmoid_q15(int64_t g, int32_t Mg, int32_t Kg) {
  const int64_t ag = g < 0 ? -g : g;
  const uint32_t E = (uint32_t)diexp(-R(ag * Mg, Kg));
  uint32_t q;
  if (E >= 32768u) {
    q = 16384u;
  } else {
    const uint32_t b2 = 2u * (32768u + E);        // 2b in [2^16, 2^17)
    uint32_t num = (1u << 31) + (32768u + E);     // 2a + b
    q = 0;
    if (num >= (b2 << 15)) {                      // quotient bit 15 (b2 << 15 < 2^32)
      num -= b2 << 15;
      q = 1u << 15;
    }
#pragma unroll
    for (int i = 14; i >= 0; --i) {
      const uint32_t t = b2 << i;
      if (num >= t) {
        num -= t;
        q |= 1u << i;
      }
    }
  }
  return (int32_t)(g >= 0 ? q : 32768 - q);
}

// sigmoid_q15 for a wave-uniform gate, the quotient found by the whole wave
// (three 6-bit digit rounds instead of 16 serial restoring steps).
__device__ __forceinline__ int32_t sigmoid_q15_wave(int64_t g, int32_t Mg, int32_t Kg) {
  g = (int64_t)uniform64((uint64_t)g);
  const int64_t ag = g < 0 ? -g : g;
  const uint64_t b = 32768u + (uint32_t)diexp(-R(ag * Mg, Kg));  // in [2^15, 2^16]
  const int32_t q = (int32_t)udiv_wave<16>((uint64_t(1) << 31) + b, 2 * b);  // RD(2^30, b)
  return g >= 0 ? q : 32768 - q;
}

// ---------------------------------------------------------------- reductions
//
// Lane exchanges on the VALU rather than through the LDS crossbar
// (ds_bpermute, which __shfl_xor compiles to): DPP quad permutes and row
// mirrors / rotates inside 16-lane rows, and gfx950's permlane16 / permlane32
// swaps across rows. Each step costs a few cycles instead of an LDS round
// trip, which matters on the latency chains of the batch-1 decode kernels.
// Workgroups are one-dimensional with a multiple of 64 threads, and every
// lane of the wave must be active (uniform control flow).

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppRev4 = 0x1B,        // quad_perm [3,2,1,0]: lane i ^ 3
  kDppHalfMirror = 0x141, // lane i ^ 7 within 8
  kDppMirror = 0x140,     // lane i ^ 15 within 16
  kDppRor8 = 0x128,       // lane i ^ 8 within 16
};

// (a, b) with a = v of the even and b = v of the odd 16-lane rows (O = 16),
// or of the lower and upper 32 lanes (O = 32), in every lane of the pair
template <int O>
__device__ __forceinline__ void row_pair(uint32_t v, uint32_t& a, uint32_t& b) {
  static_assert(O == 16 || O == 32, "row_pair: 16 or 32");
  if constexpr (O == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = s[0];
    b = s[1];
  } else {
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = s[0];
    b = s[1];
  }
}

// v of lane (lane ^ O), O a power of two below 64
template <int O>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (O == 1) {
    return dpp_u32<kDppXor1>(v);
  } else if constexpr (O == 2) {
    return dpp_u32<kDppXor2>(v);
  } else if constexpr (O == 4) {
    return dpp_u32<kDppHalfMirror>(dpp_u32<kDppRev4>(v));  // i ^ 4 = (i ^ 3) ^ 7
  } else if constexpr (O == 8) {
    return dpp_u32<kDppRor8>(v);
  } else {
    uint32_t a, b;
    row_pair<O>(v, a, b);
    return (threadIdx.x & O) ? a : b;
  }
}
template <int O>
__device__ __forceinline__ int lane_xor(int v) {
  return (int)lane_xor<O>((uint32_t)v);
}
template <int O>
__device__ __forceinline__ int64_t lane_xor(int64_t v) {
  const uint32_t lo = lane_xor<O>((uint32_t)(uint64_t)v);
  const uint32_t hi = lane_xor<O>((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <int O>
__device__ __forceinline__ uint64_t lane_xor(uint64_t v) {
  return (uint64_t)lane_xor<O>((int64_t)v);
}

// Whole-wave reduction of 64-bit values by an associative, commutative op;
// every lane receives the result. After the two quad steps a quad holds one
// value, so the half-row and row mirrors pair it with the other quad / half
// row; the permlane swaps then pair rows.
template <class Op>
__device__ __forceinline__ uint64_t wave_reduce64(uint64_t v, Op op) {
  auto step = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    const uint64_t w = ((uint64_t)dpp_u32<C>((uint32_t)(v >> 32)) << 32) | dpp_u32<C>((uint32_t)v);
    v = op(v, w);
  };
  step(std::integral_constant<int, kDppXor1>{});
  step(std::integral_constant<int, kDppXor2>{});
  step(std::integral_constant<int, kDppHalfMirror>{});
  step(std::integral_constant<int, kDppMirror>{});
  uint32_t al, bl, ah, bh;
  row_pair<16>((uint32_t)v, al, bl);
  row_pair<16>((uint32_t)(v >> 32), ah, bh);
  v = op(((uint64_t)ah << 32) | al, ((uint64_t)bh << 32) | bl);
  row_pair<32>((uint32_t)v, al, bl);
  row_pair<32>((uint32_t)(v >> 32), ah, bh);
  return op(((uint64_t)ah << 32) | al, ((uint64_t)bh << 32) | bl);
}

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
  return (int64_t)wave_reduce64((uint64_t)v, [](uint64_t a, uint64_t b) { return a + b; });
}
__device__ __forceinline__ int64_t wave_max(int64_t v) {
  return (int64_t)wave_reduce64(
      (uint64_t)v, [](uint64_t a, uint64_t b) { return (int64_t)a > (int64_t)b ? a : b; });
}
__device__ __forceinline__ uint64_t wave_max_u(uint64_t v) {
  return wave_reduce64(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}

// Maximum / sum over the wave of a 32-bit value (one exchange per step).
template <class Op>
__device__ __forceinline__ int wave_reduce32(int v, Op op) {
  v = op(v, (int)dpp_u32<kDppXor1>((uint32_t)v));
  v = op(v, (int)dpp_u32<kDppXor2>((uint32_t)v));
  v = op(v, (int)dpp_u32<kDppHalfMirror>((uint32_t)v));
  v = op(v, (int)dpp_u32<kDppMirror>((uint32_t)v));
  uint32_t a, b;
  row_pair<16>((uint32_t)v, a, b);
  v = op((int)a, (int)b);
  row_pair<32>((uint32_t)v, a, b);
  return op((int)a, (int)b);
}
__device__ __forceinline__ int wave_max32(int v) {
  return wave_reduce32(v, [](int a, int b) { return max(a, b); });
}
__device__ __forceinline__ int wave_sum32(int v) {
  return wave_reduce32(v, [](int a, int b) { return a + b; });
}

// Bit length of the wave's largest magnitude among 64-bit u0, u1: the bit
// length of a maximum is the maximum of the bit lengths, so the exchange
// carries 32-bit lengths instead of 64-bit values.
__device__ __forceinline__ int wave_bitlen_max(uint64_t u0, uint64_t u1) {
  return wave_max32(bitlen64(u0 | u1));
}

// Sum over the lanes that differ from this one in bits O, O / 2, ..., 1
template <int O>
__device__ __forceinline__ int xor_sum_to(int v) {
  if constexpr (O == 0) {
    return v;
  } else {
    return xor_sum_to<O / 2>(v + lane_xor<O>(v));
  }
}
// Sum (or maximum) of 64-bit values over the lanes that differ in bits O .. 1
template <int O, bool MAX>
__device__ __forceinline__ int64_t xor_fold_to(int64_t v) {
  if constexpr (O == 0) {
    return v;
  } else {
    const int64_t w = lane_xor<O>(v);
    return xor_fold_to<O / 2, MAX>(MAX ? (w > v ? w : v) : v + w);
  }
}
// Sum over the lanes that differ from this one in bits O, 2 O, ..., 32
template <int O>
__device__ __forceinline__ int xor_sum_from(int v) {
  if constexpr (O >= 64) {
    return v;
  } else {
    return xor_sum_from<2 * O>(v + lane_xor<O>(v));
  }
}

// Block-wide reductions for blockDim.x a multiple of 64 (<= 1024); `red` is
// shared scratch of >= 16 entries. All threads receive the result.
__device__ __forceinline__ int64_t block_sum(int64_t v, int64_t* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int64_t t = 0;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
// A row's sum of squares and the bit length of its largest magnitude in
// one exchange through LDS (`red` >= 32 entries): the sum in 64 bits, the
// bit length as a 32-bit maximum. All threads receive both.
__device__ __forceinline__ void block_sum_maxbits(int64_t& s, int& b, int64_t* red) {
  s = wave_sum(s);
  b = wave_max32(b);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[w] = s;
    red[16 + w] = b;
  }
  __syncthreads();
  int64_t ts = 0;
  int tb = 0;
  for (int i = 0; i < nw; ++i) {
    ts += red[i];
    tb = max(tb, (int)red[16 + i]);
  }
  s = ts;
  b = tb;
}
__device__ __forceinline__ int64_t block_max(int64_t v, int64_t* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int64_t t = red[0];
  for (int i = 1; i < nw; ++i) t = red[i] > t ? red[i] : t;
  return t;
}

// Workgroup barrier that orders LDS accesses only. __syncthreads also drains
// every outstanding global load of the wave (vmcnt(0)); this one waits for
// the wave's LDS (and scalar) operations alone, so global loads issued before
// it - weights streamed ahead of their use - stay in flight across it. The
// compiler still waits for those loads before their registers are used.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// DQ exponent from the absolute maximum: e = max(0, bitlen(A) - 7).
__device__ __forceinline__ int dq_exp(uint64_t A) {
  const int b = bitlen64(A);
  return b > 7 ? b - 7 : 0;
}

// Host side: defines `hipError_t NAME(uint32_t* acc, hipStream_t st)`, which
// waits for the stream, ORs this translation unit's flag word into *acc and
// clears it (copies, no memset, outside any graph capture).
#define DETINT_BOUND_READER(NAME)                                                         \
  hipError_t NAME(uint32_t* acc, hipStream_t st) {                                        \
    uint32_t v = 0;                                                                        \
    static const uint32_t zero = 0;                                                        \
    hipError_t e = hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_bound_flags), sizeof v, 0,    \
                                            hipMemcpyDeviceToHost, st);                    \
    if (e == hipSuccess) e = hipStreamSynchronize(st);                                     \
    if (e == hipSuccess && v)                                                              \
      e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_bound_flags), &zero, sizeof zero, 0,         \
                                 hipMemcpyHostToDevice, st);                               \
    if (e == hipSuccess && v) e = hipStreamSynchronize(st);                                \
    *acc |= v;                                                                             \
    return e;                                                                              \
  }

}  // namespace detint
