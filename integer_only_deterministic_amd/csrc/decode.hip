// Fused weight-streaming kernels for decode-sized batches (M <= 8 rows).
//
// A decode step is a chain of small GEMVs whose cost on this GPU is set by
// the number of kernels and by memory latency, not by bytes: a graph node
// costs ~1.6 us and a kernel with two dependent memory round trips a few us
// more. Each kernel here therefore (1) issues its first weight loads before
// touching activations (weights never depend on them), (2) recomputes the
// row-wise prologue its input needs in every workgroup - RMSNorm of the
// residual, or DQ of the attention output / SwiGLU product (DetLLM blog
// "DetLLM": per-token quantisation from the token's own values) - into LDS,
// and (3) fuses the dyadic epilogue: fixed point, residual add, the SwiGLU
// product of a (gate j, up j) column pair, or int32 logits with greedy-argmax
// partials. Every step is the same integer function as the unfused kernels.
#include "dev_int.h"
#include "internal.h"

namespace detint {
namespace {

constexpr int TPB = 256;

__device__ __forceinline__ int dot16(const v4i& a, const v4i& b, int c) {
  c = __builtin_amdgcn_sdot4(a.x, b.x, c, false);
  c = __builtin_amdgcn_sdot4(a.y, b.y, c, false);
  c = __builtin_amdgcn_sdot4(a.z, b.z, c, false);
  c = __builtin_amdgcn_sdot4(a.w, b.w, c, false);
  return c;
}

__device__ __forceinline__ int64_t amax_key(int64_t v, int64_t j) {
  return (v * 4294967296LL) | (int64_t)(0xFFFFFFFFu - (uint32_t)j);
}

// Transposed wave reduction of NV (a power of two <= 64) int32 values per
// lane: each halving step exchanges half of the values with the lane `O`
// apart, so NV sums take NV - 1 + log2(64 / NV) shuffles instead of 6 NV.
// Afterwards lane l holds the wave total of value index
//   idx(l) = sum_s bit(l, 5 - s) * (NV >> (s + 1)),
// identical in the 64 / NV lanes that differ only in their low bits. Sizes
// and lane offsets are template constants, so every register index is static
// and the exchanges compile to fixed-pattern lane swizzles.
template <int N, int O>
struct Halve {
  __device__ __forceinline__ static int run(int* v, int lane) {
    const bool upper = (lane & O) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const int keep = upper ? v[i + N / 2] : v[i];
      const int give = upper ? v[i] : v[i + N / 2];
      v[i] = keep + lane_xor<O>(give);
    }
    return Halve<N / 2, O / 2>::run(v, lane);
  }
};
template <int O>
struct Halve<1, O> {
  __device__ __forceinline__ static int run(int* v, int) {
    return xor_sum_to<O>(v[0]);
  }
};

template <int NV>
__device__ __forceinline__ int wave_reduce_t(int (&v)[NV], int lane) {
  return Halve<NV, 32>::run(v, lane);
}

// The same transposed reduction with a maximum (bit lengths).
template <int O>
__device__ __forceinline__ int xor_max_to(int v) {
  if constexpr (O == 0) {
    return v;
  } else {
    return xor_max_to<O / 2>(max(v, lane_xor<O>(v)));
  }
}
template <int N, int O>
struct HalveMax {
  __device__ __forceinline__ static int run(int* v, int lane) {
    const bool upper = (lane & O) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const int keep = upper ? v[i + N / 2] : v[i];
      const int give = upper ? v[i] : v[i + N / 2];
      v[i] = max(keep, lane_xor<O>(give));
    }
    return HalveMax<N / 2, O / 2>::run(v, lane);
  }
};
template <int O>
struct HalveMax<1, O> {
  __device__ __forceinline__ static int run(int* v, int) {
    return xor_max_to<O>(v[0]);
  }
};

// The same transposed reduction for int64 values with a sum or a max.
template <int N, int O, bool MAX>
struct Halve64 {
  __device__ __forceinline__ static int64_t run(int64_t* v, int lane) {
    const bool upper = (lane & O) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const int64_t keep = upper ? v[i + N / 2] : v[i];
      const int64_t give = upper ? v[i] : v[i + N / 2];
      const int64_t got = lane_xor<O>(give);
      v[i] = MAX ? (got > keep ? got : keep) : keep + got;
    }
    return Halve64<N / 2, O / 2, MAX>::run(v, lane);
  }
};
template <int O, bool MAX>
struct Halve64<1, O, MAX> {
  __device__ __forceinline__ static int64_t run(int64_t* v, int) {
    return xor_fold_to<O, MAX>(v[0]);
  }
};

template <int NV>
__device__ __forceinline__ int reduce_index(int lane) {
  int idx = 0, h = NV >> 1, b = 5;
#pragma unroll
  for (int n = NV; n > 1; n >>= 1, h >>= 1, --b) idx += ((lane >> b) & 1) * h;
  return idx;
}

enum { PRO_NORM = 1, PRO_DQ32 = 2, PRO_DQ64 = 3, PRO_I8 = 4 };
enum { EPI_RAW = 0, EPI_FIX = 1, EPI_RES = 2, EPI_SWIGLU = 3, EPI_LOGITS = 4, EPI_REQ = 5 };

struct FG {
  const int32_t* h;          // PRO_NORM: residual rows [*, K]
  const int16_t* gain;
  const int32_t* row_index;  // PRO_NORM: input row of output row m (nullable)
  const int32_t* in32;       // PRO_DQ32: [M, K]
  int32_t fold_m, fold_k;    //   row scale (fold_m, fold_k - e)
  const int64_t* in64;       // PRO_DQ64: [M, K]; row scale (2^14, 2 f_a - e + 14)
  int32_t f_a;
  const int8_t* a8;          // PRO_I8: int8 rows [M, K] with scales rm_in / rk_in (nullable: RAW)
  const int32_t* rm_in;
  const int32_t* rk_in;
  const int8_t* W;           // [N, K] ([2N, K] for SWIGLU: gate rows then up rows)
  const int32_t* col_m;
  int32_t col_k, frac;
  int32_t Mg, Kg;            // SWIGLU sigmoid multiplier
  int32_t M, N, K;
  void* out;
  const int32_t* out_row_base;
  int64_t* part;
  int32_t* rm_out;           // nullable: row scales written by workgroup 0
  int32_t* rk_out;
  int32_t res_bits;          // EPI_RES bound 2^res_bits (0: int32 range only)
};

template <int MT, int CPW, int KC, int PRO, int EPI>
__global__ __launch_bounds__(TPB, (EPI == EPI_LOGITS && MT == 1 && KC == 1 ? (CPW == 4 ? 6 : 8) : 1)) void fgemv(FG p) {
  extern __shared__ __attribute__((aligned(16))) int8_t sx[];  // [MT][K] int8 input rows
  __shared__ int64_t sred[TPB / 64][2 * MT];
  __shared__ int32_t s_m[MT], s_k[MT], s_e[MT];
  constexpr int NV = CPW * MT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gw = blockIdx.x * (TPB / 64) + wave, nw = gridDim.x * (TPB / 64);
  const int M = p.M, N = p.N, K = p.K;
  const int ngroups = EPI == EPI_SWIGLU ? N : (N + CPW - 1) / CPW;
  const int64_t obase = EPI == EPI_LOGITS && p.out_row_base ? *p.out_row_base : 0;
  uint32_t bad = 0;  // bound flags seen by this thread

  // 1. Loads. Every load below uses a clamped, always-valid address and
  //    its register is left untouched until all of them are in flight:
  //    activations first, then the weights of the wave's first two groups
  //    (a register ring of two buffers, with their column mantissas). Loads
  //    complete in order, so the prologue arithmetic waits for the
  //    activations only, and the LDS-only barriers below do not drain the
  //    weights. Out-of-range elements are zeroed after the loads (inputs) or
  //    multiply the zero padding of the LDS rows / land in discarded columns
  //    (weights).
  v4i w[2][CPW][KC];
  int32_t cmv[2][CPW];
  // weights and mantissas through buffer resources: a group past the end
  // (and lanes past K) get out-of-range offsets, which read zeros without
  // touching memory, so no load sits behind a branch
  const int wrows = EPI == EPI_SWIGLU ? 2 * N : N;
  const int wbytes = wrows * K;  // < 2^31 and (rows + 2^16) K < 2^32 (checked at launch)
  const __amdgpu_buffer_rsrc_t wsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.W, (short)0, wbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t csrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.col_m, (short)0, wrows * 4, 0x00020000);
  auto load_w = [&](int g, int b) {
    // rows of a group past the end fall past the buffer (for SWIGLU the
    // group index is moved there), lanes past K read a clamped chunk whose
    // products with the zero padding of the LDS rows vanish; all offsets are
    // formed before the first load is issued
    const uint32_t gg = EPI == EPI_SWIGLU && g >= ngroups ? 2u * N : (uint32_t)g;
    uint32_t roff[CPW], koff[KC];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      roff[c] = EPI == EPI_SWIGLU ? (c == 0 ? gg : N + gg) : gg * CPW + c;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) koff[kc] = (uint32_t)min(kc * 1024 + lane * 16, K - 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if (EPI != EPI_RAW)
        cmv[b][c] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(csrc, (int)(roff[c] * 4u), 0, 0);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        w[b][c][kc] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(wsrc, (int)(roff[c] * (uint32_t)K + koff[kc]), 0, 0));
    }
  };
  int g = gw;
  // every wave streams at most one group (the decode shapes): the refills
  // two groups ahead would all fall past the end, and a load past the end,
  // though it reads zeros without touching memory, still costs the texture
  // unit 16 cycles per instruction - issue none of them
  const bool one = nw >= ngroups;

  if constexpr (PRO == PRO_I8) {
    // int8 rows given (a standalone GEMM): rows and their scales into LDS
    uint32_t ar[MT][KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int i = min(kc * 1024 + 4 * tid, K - 4);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        ar[m][kc] = *(const uint32_t*)(p.a8 + (size_t)(m < M ? m : M - 1) * K + i);
    }
    load_w(g, 0);
    if (!one) load_w(g + nw, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (tid < MT) {
      const int mc = tid < M ? tid : M - 1;
      s_m[tid] = p.rm_in ? p.rm_in[mc] : 0;
      s_k[tid] = p.rk_in ? p.rk_in[mc] : 0;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bool ok = m < M && kc * 1024 + 4 * tid < K;
        *(uint32_t*)(sx + (size_t)m * (KC * 1024) + kc * 1024 + 4 * tid) = ok ? ar[m][kc] : 0u;
      }
    lds_barrier();
  } else {
    typedef int64_t v4l __attribute__((ext_vector_type(4)));
    constexpr bool WIDE_IN = PRO == PRO_DQ64;
    v4i xr[MT][KC];        // int32 inputs as loaded
    v4l xw[WIDE_IN ? MT : 1][KC];  // int64 inputs as loaded
    int2 graw[KC];
  #pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int i = min(kc * 1024 + 4 * tid, K - 4);
      if (PRO == PRO_NORM) graw[kc] = *(const int2*)(p.gain + i);  // four int16 gains
  #pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int mc = m < M ? m : M - 1;
        if (PRO == PRO_NORM) {
          const int src = p.row_index ? p.row_index[mc] : mc;
          xr[m][kc] = *(const v4i*)(p.h + (size_t)src * K + i);
        } else if (!WIDE_IN) {
          xr[m][kc] = *(const v4i*)(p.in32 + (size_t)mc * K + i);
        } else {
          xw[m][kc] = *(const v4l*)(p.in64 + (size_t)mc * K + i);
        }
      }
    }
    load_w(g, 0);
    if (!one) load_w(g + nw, 1);
    __builtin_amdgcn_sched_barrier(0);

    // 2. prologue: int8 input rows and their scales into LDS. Thread t owns
    //    elements kc * 1024 + 4 t .. + 3 of every row (zero past K, and rows
    //    past M are zero).
    int64_t xv[MT][KC][4];
    int32_t gv[KC][4];
  #pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const bool iv = kc * 1024 + 4 * tid < K;
      if (PRO == PRO_NORM) {
        gv[kc][0] = iv ? (int16_t)(graw[kc].x & 0xFFFF) : 0;
        gv[kc][1] = iv ? (int16_t)(graw[kc].x >> 16) : 0;
        gv[kc][2] = iv ? (int16_t)(graw[kc].y & 0xFFFF) : 0;
        gv[kc][3] = iv ? (int16_t)(graw[kc].y >> 16) : 0;
      }
  #pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bool ok = iv && m < M;
        if (!WIDE_IN) {
          xv[m][kc][0] = ok ? xr[m][kc].x : 0;
          xv[m][kc][1] = ok ? xr[m][kc].y : 0;
          xv[m][kc][2] = ok ? xr[m][kc].z : 0;
          xv[m][kc][3] = ok ? xr[m][kc].w : 0;
        } else {
          xv[m][kc][0] = ok ? xw[m][kc].x : 0;
          xv[m][kc][1] = ok ? xw[m][kc].y : 0;
          xv[m][kc][2] = ok ? xw[m][kc].z : 0;
          xv[m][kc][3] = ok ? xw[m][kc].w : 0;
        }
      }
    }
    // per row: the sum of squares and the bit length of the largest
    // magnitude (all the DQ exponent needs; the bit length of the OR of the
    // magnitudes is that of their maximum), so the maxima travel as 32 bits
    int64_t Sv[MT];
    int Bv[MT];
  #pragma unroll
    for (int m = 0; m < MT; ++m) {
      int64_t S = 0;
      uint64_t A = 0;
  #pragma unroll
      for (int kc = 0; kc < KC; ++kc)
  #pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int64_t v = xv[m][kc][e4];
          if (PRO == PRO_NORM) S += v * v;
          A |= uabs64(PRO == PRO_NORM ? v * gv[kc][e4] : v);
        }
      Sv[m] = S;
      Bv[m] = bitlen64(A);
    }
    {
      // wave totals of every row at once: lane l ends with row idx(l)'s totals
      const int At = HalveMax<MT, 32>::run(Bv, lane);
      const int64_t St = PRO == PRO_NORM ? Halve64<MT, 32, false>::run(Sv, lane) : 0;
      const int r = reduce_index<MT>(lane);
      if ((lane & (64 / MT - 1)) == 0) {
        sred[wave][2 * r] = St;
        sred[wave][2 * r + 1] = At;
      }
    }
    lds_barrier();
    // row scales: wave w finishes rows w, w + 4, ... (irms needs a whole
    // wave); a single row is finished by every wave, which then needs no
    // barrier before quantising its own elements (wave 0 publishes the
    // scales for the epilogue, read after the barrier below)
    constexpr bool SOLO = MT == 1;
    int e_solo = 0;
    for (int r = SOLO ? 0 : wave; r < M; r += SOLO ? M : TPB / 64) {
      int64_t St = 0, At = 0;
  #pragma unroll
      for (int w2 = 0; w2 < TPB / 64; ++w2) {
        St += sred[w2][2 * r];
        At = sred[w2][2 * r + 1] > At ? sred[w2][2 * r + 1] : At;
      }
      const int e = At > 7 ? (int)At - 7 : 0;  // dq_exp of the rows' largest magnitude
      int32_t sm, sk;
      if (PRO == PRO_NORM && (uint64_t)St >> 62) bad |= kBoundNorm;
      if (PRO == PRO_NORM) {
        if (St == 0) {
          sm = 1 << 14;
          sk = 26;
        } else {
          int32_t mm, sh;
          irms_wave(St, K, mm, sh);
          sm = mm;
          sk = sh + 12 - e;
        }
      } else if (PRO == PRO_DQ32) {
        sm = p.fold_m;
        sk = p.fold_k - e;
      } else {
        sm = 1 << 14;
        sk = 2 * p.f_a - e + 14;
      }
      const int eq = (PRO == PRO_NORM && St == 0) ? 0 : e;
      if (lane == 0 && (!SOLO || wave == 0)) {
        s_m[r] = sm;
        s_k[r] = sk;
        s_e[r] = eq;
      }
      e_solo = eq;
    }
    if (!SOLO) lds_barrier();
    // quantised rows, zero-padded to KC * 1024 bytes (the weight loads of
    // lanes past K read clamped addresses; their products with the padding
    // are zero)
  #pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int e = SOLO ? e_solo : s_e[m < M ? m : 0];
  #pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int i = kc * 1024 + 4 * tid;
        uint32_t packed = 0;
  #pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int64_t v = PRO == PRO_NORM ? xv[m][kc][e4] * gv[kc][e4] : xv[m][kc][e4];
          // |R(v, e)| <= 128 by the choice of e, so the clamp can run in 32 bits
          const int32_t q = (int32_t)R_nn(v, e);
          packed |= (uint32_t)(uint8_t)(q > 127 ? 127 : (q < -127 ? -127 : q)) << (8 * e4);
        }
        *(uint32_t*)(sx + (size_t)m * (KC * 1024) + i) = packed;
      }
    }
    if (p.rm_out && blockIdx.x == 0 && tid < M) {
      p.rm_out[tid] = s_m[tid];
      p.rk_out[tid] = s_k[tid];
    }
    lds_barrier();
  }

  // 3. stream the weights: per group, dot products from LDS, reduce, epilogue
  const int idx = reduce_index<NV>(lane);
  const bool leader = (lane & (64 / NV - 1)) == 0;
  const int cc = idx / MT, mm = idx % MT;  // the (column, row) this lane finishes
  int64_t bestk = INT64_MIN;
  // b and refill are constants at each call; g may be past the end
  auto group = [&](int g, int b, bool refill) {
    int32_t cm[CPW];  // this group's mantissas, before buffer b is refilled
#pragma unroll
    for (int c = 0; c < CPW; ++c) cm[c] = cmv[b][c];
    // residual value to add to, loaded before the refill below so that
    // waiting for it does not wait for the refill (clamped address)
    int32_t old = 0;
    if (EPI == EPI_RES)
      old = ((const int32_t*)p.out)[(size_t)(mm < M ? mm : M - 1) * N + min(g * CPW + cc, N - 1)];
    int v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = 0;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int k = kc * 1024 + lane * 16;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const v4i x = *(const v4i*)(sx + (size_t)m * (KC * 1024) + k);
#pragma unroll
        for (int c = 0; c < CPW; ++c) v[c * MT + m] = dot16(x, w[b][c][kc], v[c * MT + m]);
      }
    }
    // two groups ahead, into the buffer just consumed (kept apart from the
    // dot products so the loads reuse its registers: a copy would have to
    // wait for them)
    __builtin_amdgcn_sched_barrier(0);
    if (refill) load_w(g + 2 * nw, b);
    __builtin_amdgcn_sched_barrier(0);
    const int tot = wave_reduce_t<NV>(v, lane);
    if (EPI == EPI_SWIGLU && MT == 1) {
      // one row: the gate total sits in lanes 0..31, the up total in lanes
      // 32..63; the whole wave computes the (uniform) epilogue
      const int gt = __builtin_amdgcn_readfirstlane(tot);
      const int ut = __builtin_amdgcn_readlane(tot, 32);
      if (g < ngroups) {
        const int sh = s_k[0] + p.col_k - p.f_a;
        const int64_t gv = R((int64_t)gt * s_m[0] * cm[0], sh);
        const int64_t uv = R((int64_t)ut * s_m[0] * cm[1], sh);
        const int64_t res = R(gv * sigmoid_q15_wave(gv, p.Mg, p.Kg), 15) * uv;
        bad |= out_of(gv, 24) | out_of(uv, 24) ? kBoundSwiglu : 0u;
        if (lane == 0) ((int64_t*)p.out)[g] = res;
      }
    } else if (EPI == EPI_SWIGLU) {
      const int up = lane_xor<32>(tot);  // column 1 (up) sits in the lane 32 apart
      if (leader && cc == 0 && mm < M && g < ngroups) {
        const int j = g;
        const int sh = s_k[mm] + p.col_k - p.f_a;
        const int64_t gv = R((int64_t)tot * s_m[mm] * cm[0], sh);
        const int64_t uv = R((int64_t)up * s_m[mm] * cm[1], sh);
        bad |= out_of(gv, 24) | out_of(uv, 24) ? kBoundSwiglu : 0u;
        ((int64_t*)p.out)[(size_t)mm * N + j] = R(gv * sigmoid_q15(gv, p.Mg, p.Kg), 15) * uv;
      }
    } else if (leader && mm < M) {
      const int col = g * CPW + cc;
      if (col < N) {
        if (EPI == EPI_RAW) {
          ((int32_t*)p.out)[(size_t)mm * N + col] = tot;
        } else {
          const int64_t y = R((int64_t)tot * s_m[mm] * cm[cc], s_k[mm] + p.col_k - p.frac);
          if (EPI == EPI_FIX) {
            bad |= i32_check(y);
            ((int32_t*)p.out)[(size_t)mm * N + col] = (int32_t)y;
          } else if (EPI == EPI_REQ) {
            ((int8_t*)p.out)[(size_t)mm * N + col] = clamp8(y);
          } else if (EPI == EPI_RES) {
            const int64_t t = (int64_t)old + y;
            bad |= res_check(t, p.res_bits);
            ((int32_t*)p.out)[(size_t)mm * N + col] = (int32_t)t;
          } else {
            bad |= i32_check(y);
            ((int32_t*)p.out)[(size_t)(obase + mm) * N + col] = (int32_t)y;
            const int64_t key = amax_key(y, col);
            bestk = key > bestk ? key : bestk;
          }
        }
      }
    }
  };
  // several groups per wave: both calls unconditional (the second group may
  // be past the end: its loads read zeros and its results are dropped), so
  // the loop body is straight-line code and the wait for a buffer counts
  // only older loads
  if (one) {
    if (g < ngroups) group(g, 0, false);
  } else {
    for (; g < ngroups; g += 2 * nw) {
      group(g, 0, true);
      group(g + nw, 1, true);
    }
  }
  if (EPI == EPI_LOGITS) {
    // the column leaders' best keys into lane 0 (leaders 16 apart for four
    // columns, 32 apart for two)
    if (CPW == 4) {
      const int64_t o1 = lane_xor<16>(bestk);
      bestk = o1 > bestk ? o1 : bestk;
    }
    if (CPW >= 2) {
      const int64_t o2 = lane_xor<32>(bestk);
      bestk = o2 > bestk ? o2 : bestk;
    }
    if (leader && cc == 0 && mm < M) p.part[(size_t)mm * nw + gw] = bestk;
  }
  bound_raise(bad);
}

// Workgroups of a launch: one group per wave where that fits, else a cap -
// for one row 1024 (four per CU, each wave then streaming ~18 lm_head column
// pairs: fewer prologues than eight per CU, and measured 5-6% faster than
// 768, 1280 or 2048), otherwise 2048.
int cap_blocks(int64_t groups, int mt) {
  const int64_t cap = mt == 1 ? 1024 : 2048;
  const int64_t b = (groups + 3) / 4;
  return (int)(b < cap ? (b > 0 ? b : 1) : cap);
}

template <int MT, int CPW, int PRO, int EPI>
hipError_t launch_kc(const FG& p, hipStream_t st) {
  const int64_t groups = EPI == EPI_SWIGLU ? p.N : (p.N + CPW - 1) / CPW;
  const int blocks = cap_blocks(groups, MT);
  // weight offsets are 32-bit buffer offsets; those of groups up to two
  // rounds past the end (at most 2^16 rows) must not wrap
  if ((int64_t)(EPI == EPI_SWIGLU ? 2 : 1) * p.N * p.K >= (int64_t(1) << 31) || p.K > 8192)
    return hipErrorInvalidValue;
  const int kc = (p.K + 1023) / 1024;
#define DETINT_KC(KK)                                                         \
  if (kc <= KK) {                                                             \
    const size_t lds = (size_t)MT * KK * 1024;                                \
    fgemv<MT, CPW, KK, PRO, EPI><<<blocks, TPB, lds, st>>>(p);                \
    return hipGetLastError();                                                 \
  }
  DETINT_KC(1) DETINT_KC(2) DETINT_KC(3) DETINT_KC(8)
#undef DETINT_KC
  return hipErrorInvalidValue;
}

template <int CPW, int PRO, int EPI>
hipError_t launch_mt(const FG& p, hipStream_t st) {
  if (p.M <= 1) return launch_kc<1, CPW, PRO, EPI>(p, st);
  if (p.M <= 4) return launch_kc<4, CPW, PRO, EPI>(p, st);
  return launch_kc<8, CPW, PRO, EPI>(p, st);
}

}  // namespace

DETINT_BOUND_READER(bound_flags_decode)

// column groups of the vocabulary head: four columns per wave for one row,
// two otherwise
constexpr int head_cpw(int64_t M) { return M <= 1 ? 4 : 2; }

int fused_decode_parts(int64_t V, int64_t M) {
  return cap_blocks((V + head_cpw(M) - 1) / head_cpw(M), M <= 1 ? 1 : (M <= 4 ? 4 : 8)) * 4;
}

bool fused_decode_supported(int64_t M, int64_t K) { return M >= 1 && M <= 8 && K <= 8192 && K % 16 == 0; }

hipError_t launch_fused_qkv(const int32_t* h, const int16_t* gain, const int8_t* W,
                            const int32_t* col_m, int32_t col_k, int32_t frac, bool raw, int64_t M,
                            int64_t N, int64_t K, int32_t* out, int32_t* rm_out, int32_t* rk_out,
                            hipStream_t st) {
  FG p{};
  p.h = h; p.gain = gain; p.W = W; p.col_m = col_m; p.col_k = col_k; p.frac = frac;
  p.M = (int)M; p.N = (int)N; p.K = (int)K; p.out = out; p.rm_out = rm_out; p.rk_out = rk_out;
  return raw ? launch_mt<2, PRO_NORM, EPI_RAW>(p, st) : launch_mt<2, PRO_NORM, EPI_FIX>(p, st);
}

hipError_t launch_fused_oproj(const int32_t* att, int32_t fold_m, int32_t fold_k, const int8_t* W,
                              const int32_t* col_m, int32_t col_k, int32_t frac, int64_t M,
                              int64_t N, int64_t K, int32_t* h, hipStream_t st) {
  FG p{};
  p.in32 = att; p.fold_m = fold_m; p.fold_k = fold_k; p.W = W; p.col_m = col_m; p.col_k = col_k;
  p.frac = frac; p.M = (int)M; p.N = (int)N; p.K = (int)K; p.out = h; p.res_bits = 25;
  return launch_mt<1, PRO_DQ32, EPI_RES>(p, st);
}

hipError_t launch_fused_gateup(const int32_t* h, const int16_t* gain, const int8_t* W,
                               const int32_t* col_m, int32_t col_k, int32_t f_a, int32_t Mg,
                               int32_t Kg, int64_t M, int64_t F, int64_t K, int64_t* prod,
                               hipStream_t st) {
  FG p{};
  p.h = h; p.gain = gain; p.W = W; p.col_m = col_m; p.col_k = col_k; p.f_a = f_a; p.Mg = Mg;
  p.Kg = Kg; p.M = (int)M; p.N = (int)F; p.K = (int)K; p.out = prod;
  return launch_mt<2, PRO_NORM, EPI_SWIGLU>(p, st);
}

hipError_t launch_fused_down(const int64_t* prod, int32_t f_a, const int8_t* W, const int32_t* col_m,
                             int32_t col_k, int32_t frac, int64_t M, int64_t N, int64_t K,
                             int32_t* h, hipStream_t st) {
  FG p{};
  p.in64 = prod; p.f_a = f_a; p.W = W; p.col_m = col_m; p.col_k = col_k; p.frac = frac;
  p.M = (int)M; p.N = (int)N; p.K = (int)K; p.out = h; p.res_bits = 25;
  return launch_mt<1, PRO_DQ64, EPI_RES>(p, st);
}

hipError_t launch_fgemv_i8(const int8_t* A, const int8_t* W, int64_t M, int64_t N, int64_t K,
                           const int32_t* row_m, const int32_t* row_k, const int32_t* col_m,
                           int32_t col_k, int32_t frac, int mode, void* out, hipStream_t st,
                           int32_t res_bits) {
  FG p{};
  p.a8 = A; p.rm_in = row_m; p.rk_in = row_k; p.W = W; p.col_m = col_m; p.col_k = col_k;
  p.res_bits = res_bits;
  p.frac = mode == MODE_REQ_I8 ? 0 : frac;
  p.M = (int)M; p.N = (int)N; p.K = (int)K; p.out = out;
  switch (mode) {
    case MODE_RAW: return launch_mt<2, PRO_I8, EPI_RAW>(p, st);
    case MODE_REQ_I8: return launch_mt<2, PRO_I8, EPI_REQ>(p, st);
    case MODE_FIX: return launch_mt<2, PRO_I8, EPI_FIX>(p, st);
    default: return launch_mt<2, PRO_I8, EPI_RES>(p, st);
  }
}

hipError_t launch_fused_lm_head(const int32_t* h, const int32_t* row_index, const int16_t* gain,
                                const int8_t* E, const int32_t* emb_m, int32_t w_k, int32_t f_l,
                                int64_t M, int64_t V, int64_t K, int32_t* logits,
                                const int32_t* row_base, int64_t* part, hipStream_t st) {
  FG p{};
  p.h = h; p.row_index = row_index; p.gain = gain; p.W = E; p.col_m = emb_m; p.col_k = w_k;
  p.frac = f_l; p.M = (int)M; p.N = (int)V; p.K = (int)K; p.out = logits;
  p.out_row_base = row_base; p.part = part;
  // one row: four columns per wave, twice the weight bytes in flight per
  // wave with the same workgroups
  if (head_cpw(M) == 4) return launch_kc<1, 4, PRO_NORM, EPI_LOGITS>(p, st);
  return launch_mt<2, PRO_NORM, EPI_LOGITS>(p, st);
}

}  // namespace detint
