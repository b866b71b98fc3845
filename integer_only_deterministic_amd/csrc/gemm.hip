// int8 x int8 -> int32 GEMMs for gfx950 with the dyadic epilogue fused.
//
// out = epilogue(A[M,K] . W[N,K]^T). Integer accumulation is exact, so the
// tiling, the K order and the choice between the two kernels below cannot
// change a single bit (DetLLM blog, "DetLLM": the int8 matmul is the only
// hardware-dispatched function and exactness makes it backend-independent).
//
//  * gemm_mfma: M > 16. 128x128 output tile per 256-thread workgroup, K in
//    steps of 64 bytes staged through LDS (double buffered, rows padded to
//    80 bytes so 16-byte fragment reads spread over the banks); each wave
//    owns a 64x64 quadrant = 2x2 v_mfma_i32_32x32x32_i8 tiles.
//  * gemv: M <= 16 (decode). Weight streaming: one wave per output column,
//    16 bytes per lane per step (1 KiB contiguous per wave), v_dot4 on the
//    activation rows, wave reduction, epilogue by lane 0.
//
// 16-bit weights (BitExact blog, "Fix the arithmetic": limb products into
// wide accumulators) arrive as hi = W16 >> 8 and lo' = (W16 & 255) - 128:
// acc64 = 256 * (A.hi) + (A.lo') + 128 * rowsum(A).
#include "dev_int.h"
#include "internal.h"

namespace detint {
namespace {

template <bool WIDE>
__device__ __forceinline__ void epi_store(int64_t acc, int64_t i, int64_t j, int64_t N,
                                          const Epi& e, void* out) {
  const int64_t o = (i + (e.out_row_base ? *e.out_row_base : 0)) * N + j;
  if (e.mode == MODE_RAW) {
    if (WIDE)
      ((int64_t*)out)[o] = acc;
    else
      ((int32_t*)out)[o] = (int32_t)acc;
    return;
  }
  const int s = e.row_k[i] + e.col_k - (e.mode == MODE_REQ_I8 ? 0 : e.frac);
  int64_t y;
  if (WIDE)
    y = R128((__int128)(acc * e.row_m[i]) * e.col_m[j], s);
  else
    y = R(acc * e.row_m[i] * e.col_m[j], s);
  if (e.mode == MODE_REQ_I8)
    ((int8_t*)out)[o] = clamp8(y);
  else if (e.mode == MODE_FIX)
    ((int32_t*)out)[o] = (int32_t)y;
  else
    ((int32_t*)out)[o] += (int32_t)y;
}

__device__ __forceinline__ int dot16(const v4i& a, const v4i& b, int c) {
  c = __builtin_amdgcn_sdot4(a.x, b.x, c, false);
  c = __builtin_amdgcn_sdot4(a.y, b.y, c, false);
  c = __builtin_amdgcn_sdot4(a.z, b.z, c, false);
  c = __builtin_amdgcn_sdot4(a.w, b.w, c, false);
  return c;
}

// ---------------------------------------------------------------- MFMA GEMM

constexpr int BM = 128, BN = 128, BK = 64, LDS_STRIDE = 80;

template <bool WIDE>
__global__ __launch_bounds__(256) void gemm_mfma(const int8_t* __restrict__ A,
                                                 const int8_t* __restrict__ W,
                                                 const int8_t* __restrict__ Wlo, int M, int N,
                                                 int K, Epi e, void* out) {
  constexpr int NB = WIDE ? 2 : 1;  // weight planes
  __shared__ __attribute__((aligned(16))) int8_t sA[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) int8_t sB[2][NB][BN * LDS_STRIDE];
  __shared__ int32_t sRowSum[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int nk = (K + BK - 1) / BK;

  // global -> register staging: 2 chunks of 16 bytes per operand per thread
  v4i ra[2], rb[NB][2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int id = tid + 256 * c;
      const int row = id >> 2, col = (id & 3) * 16;
      const int k = kt * BK + col;
      const v4i z = {0, 0, 0, 0};
      const int gm = m0 + row, gn = n0 + row;
      ra[c] = (gm < M && k < K) ? *(const v4i*)(A + (size_t)gm * K + k) : z;
      rb[0][c] = (gn < N && k < K) ? *(const v4i*)(W + (size_t)gn * K + k) : z;
      if (WIDE) rb[NB - 1][c] = (gn < N && k < K) ? *(const v4i*)(Wlo + (size_t)gn * K + k) : z;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int id = tid + 256 * c;
      const int row = id >> 2, col = (id & 3) * 16;
      *(v4i*)(&sA[buf][row * LDS_STRIDE + col]) = ra[c];
#pragma unroll
      for (int p = 0; p < NB; ++p) *(v4i*)(&sB[buf][p][row * LDS_STRIDE + col]) = rb[p][c];
    }
  };

  v16i acc[NB][2][2];
#pragma unroll
  for (int p = 0; p < NB; ++p)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[p][a][b][r] = 0;
  int rowsum = 0;  // WIDE: thread tid < BM sums row tid of A
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    if (WIDE && tid < BM) {
#pragma unroll
      for (int c = 0; c < 4; ++c) rowsum = dot16(*(const v4i*)(&sA[cur][tid * LDS_STRIDE + c * 16]), ones, rowsum);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kb = ks * 32 + (lane >> 5) * 16;
      v4i fa[2], fb[NB][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        fa[t] = *(const v4i*)(&sA[cur][(wm * 64 + t * 32 + (lane & 31)) * LDS_STRIDE + kb]);
#pragma unroll
        for (int p = 0; p < NB; ++p)
          fb[p][t] = *(const v4i*)(&sB[cur][p][(wn * 64 + t * 32 + (lane & 31)) * LDS_STRIDE + kb]);
      }
#pragma unroll
      for (int p = 0; p < NB; ++p)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[p][a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[a], fb[p][b], acc[p][a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }
  if (WIDE) {
    if (tid < BM) sRowSum[tid] = rowsum;
    __syncthreads();
  }

  // accumulator layout of a 32x32 tile: lane l, register r ->
  // row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int li = wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int i = m0 + li;
        const int j = n0 + wn * 64 + b * 32 + (lane & 31);
        if (i < M && j < N) {
          int64_t v = acc[0][a][b][r];
          if (WIDE) v = 256 * v + (int64_t)acc[NB - 1][a][b][r] + 128 * (int64_t)sRowSum[li];
          epi_store<WIDE>(v, i, j, N, e, out);
        }
      }
}

// ---------------------------------------------------------------- GEMV

// Key of a logit for the greedy argmax: larger value first, then the lower
// index (DetLLM blog "DetLLM": ties go to the smallest token id); max over
// keys is order-free.
__device__ __forceinline__ int64_t amax_key(int64_t v, int64_t j) {
  return (v * 4294967296LL) | (int64_t)(0xFFFFFFFFu - (uint32_t)j);
}

// ARGMAX: FIX-mode logits epilogue that also keeps, per row, the best key
// over the columns this wave produced and writes it to part[m * nwaves + wave]
// (the final reduction over waves is argmax_final in rowops.hip).
template <int MT, bool WIDE, bool ARGMAX>
__global__ __launch_bounds__(256) void gemv(const int8_t* __restrict__ A,
                                            const int8_t* __restrict__ W,
                                            const int8_t* __restrict__ Wlo, int M, int N, int K,
                                            Epi e, void* out, int64_t* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  int64_t best[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) best[m] = INT64_MIN;
  for (int j0 = wave * 2; j0 < N; j0 += nwaves * 2) {
    int acc[2][MT], accl[2][MT], rs[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      acc[0][m] = acc[1][m] = accl[0][m] = accl[1][m] = 0;
      rs[m] = 0;
    }
    const bool two = j0 + 1 < N;
    for (int k = lane * 16; k < K; k += 1024) {
      const v4i w0 = *(const v4i*)(W + (size_t)j0 * K + k);
      const v4i w1 = two ? *(const v4i*)(W + (size_t)(j0 + 1) * K + k) : w0;
      v4i l0 = w0, l1 = w1;
      if (WIDE) {
        l0 = *(const v4i*)(Wlo + (size_t)j0 * K + k);
        l1 = two ? *(const v4i*)(Wlo + (size_t)(j0 + 1) * K + k) : l0;
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          const v4i x = *(const v4i*)(A + (size_t)m * K + k);
          acc[0][m] = dot16(x, w0, acc[0][m]);
          acc[1][m] = dot16(x, w1, acc[1][m]);
          if (WIDE) {
            accl[0][m] = dot16(x, l0, accl[0][m]);
            accl[1][m] = dot16(x, l1, accl[1][m]);
            rs[m] = dot16(x, ones, rs[m]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        int64_t s0 = wave_sum(acc[0][m]), s1 = wave_sum(acc[1][m]);
        if (WIDE) {
          const int64_t r = 128 * wave_sum(rs[m]);
          s0 = 256 * s0 + wave_sum(accl[0][m]) + r;
          s1 = 256 * s1 + wave_sum(accl[1][m]) + r;
        }
        if (ARGMAX) {
          // logits: R(acc * m_r * m_c, k_r + k_c - frac), as epi_store's FIX
          const int sh = e.row_k[m] + e.col_k - e.frac;
          const int64_t y0 = WIDE ? R128((__int128)(s0 * e.row_m[m]) * e.col_m[j0], sh)
                                  : R(s0 * e.row_m[m] * e.col_m[j0], sh);
          int64_t k0 = amax_key(y0, j0);
          const int64_t base = (e.out_row_base ? *e.out_row_base : 0) + m;
          if (lane == 0) ((int32_t*)out)[base * N + j0] = (int32_t)y0;
          if (two) {
            const int64_t y1 = WIDE ? R128((__int128)(s1 * e.row_m[m]) * e.col_m[j0 + 1], sh)
                                    : R(s1 * e.row_m[m] * e.col_m[j0 + 1], sh);
            if (lane == 0) ((int32_t*)out)[base * N + j0 + 1] = (int32_t)y1;
            const int64_t k1 = amax_key(y1, j0 + 1);
            k0 = k1 > k0 ? k1 : k0;
          }
          best[m] = k0 > best[m] ? k0 : best[m];
        } else if (lane == 0) {
          epi_store<WIDE>(s0, m, j0, N, e, out);
          if (two) epi_store<WIDE>(s1, m, j0 + 1, N, e, out);
        }
      }
    }
  }
  if (ARGMAX && lane == 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < M) part[(size_t)m * nwaves + wave] = best[m];
  }
}

int gemv_blocks(int64_t N) {
  const int64_t want = (N + 7) / 8;  // 8 columns per workgroup pass
  return (int)(want < 4096 ? want : 4096);
}

template <int MT>
hipError_t gemv_launch(const int8_t* A, const int8_t* W, const int8_t* Wlo, int M, int N, int K,
                       const Epi& e, void* out, int64_t* part, hipStream_t st) {
  const int blocks = gemv_blocks(N);
  if (part) {
    if (Wlo)
      gemv<MT, true, true><<<blocks, 256, 0, st>>>(A, W, Wlo, M, N, K, e, out, part);
    else
      gemv<MT, false, true><<<blocks, 256, 0, st>>>(A, W, Wlo, M, N, K, e, out, part);
  } else {
    if (Wlo)
      gemv<MT, true, false><<<blocks, 256, 0, st>>>(A, W, Wlo, M, N, K, e, out, nullptr);
    else
      gemv<MT, false, false><<<blocks, 256, 0, st>>>(A, W, Wlo, M, N, K, e, out, nullptr);
  }
  return hipGetLastError();
}

hipError_t gemv_dispatch(const int8_t* A, const int8_t* W, const int8_t* W_lo, int64_t M,
                         int64_t N, int64_t K, const Epi& e, void* out, int64_t* part,
                         hipStream_t st) {
  const int m = (int)M, n = (int)N, k = (int)K;
  if (M <= 1) return gemv_launch<1>(A, W, W_lo, m, n, k, e, out, part, st);
  if (M <= 2) return gemv_launch<2>(A, W, W_lo, m, n, k, e, out, part, st);
  if (M <= 4) return gemv_launch<4>(A, W, W_lo, m, n, k, e, out, part, st);
  if (M <= 8) return gemv_launch<8>(A, W, W_lo, m, n, k, e, out, part, st);
  return gemv_launch<16>(A, W, W_lo, m, n, k, e, out, part, st);
}

__global__ void split_w16(const int16_t* __restrict__ w, int64_t n, int8_t* __restrict__ hi,
                          int8_t* __restrict__ lo) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int v = w[i];
    hi[i] = (int8_t)(v >> 8);
    lo[i] = (int8_t)((v & 255) - 128);
  }
}

}  // namespace

hipError_t launch_gemm(const int8_t* A, const int8_t* W, const int8_t* W_lo, int64_t M,
                       int64_t N, int64_t K, const Epi& e, void* out, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (M <= 16) return gemv_dispatch(A, W, W_lo, M, N, K, e, out, nullptr, st);
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (W_lo)
    gemm_mfma<true><<<grid, 256, 0, st>>>(A, W, W_lo, (int)M, (int)N, (int)K, e, out);
  else
    gemm_mfma<false><<<grid, 256, 0, st>>>(A, W, W_lo, (int)M, (int)N, (int)K, e, out);
  return hipGetLastError();
}

int64_t logits_argmax_parts(int64_t N) { return (int64_t)gemv_blocks(N) * 4; }

hipError_t launch_logits_argmax(const int8_t* A, const int8_t* W, const int8_t* W_lo, int64_t M,
                                int64_t N, int64_t K, const Epi& e, int32_t* logits,
                                int64_t* part, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  return gemv_dispatch(A, W, W_lo, M, N, K, e, logits, part, st);
}

hipError_t launch_split_w16(const int16_t* W16, int64_t n, int8_t* hi, int8_t* lo,
                            hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  split_w16<<<(unsigned)blocks, 256, 0, st>>>(W16, n, hi, lo);
  return hipGetLastError();
}

}  // namespace detint
