// int8 x int8 -> int32 GEMMs for gfx950 with the dyadic epilogue fused.
//
// out = epilogue(A[M,K] . W[N,K]^T). Integer accumulation is exact, so the
// tiling, the K order and the choice between the two kernels below cannot
// change a single bit (DetLLM blog, "DetLLM": the int8 matmul is the only
// hardware-dispatched function and exactness makes it backend-independent).
//
//  * gemm_pipe: M > 16 and K a multiple of 128. BMxBN output tile (256x256,
//    128x256, 128x128 or 128x64, chosen by how many tiles the shape gives) per
//    workgroup of a WGM x WGN grid of waves (2 x 2, or 2 x 4 for the 256x256
//    int8 tiling); each wave owns a (BM/WGM)x(BN/WGN) block of
//    v_mfma_i32_32x32x32_i8 tiles with the accumulators in registers. K advances
//    128 bytes per tile through an ST-deep LDS ring filled by buffer loads
//    that write LDS directly (no register staging; rows past M or N read as
//    zero through the buffer bounds). 16-byte chunks are XOR-swizzled by row
//    so that both the DMA writes and the MFMA fragment reads are free of
//    bank conflicts on the 64-bank LDS. MFMA fragments are double-buffered
//    in registers and the block barrier sits one k-step before the end of a
//    tile, so the next tile's first fragments load under the last MFMAs.
//  * gemm_skinny: 16 < M <= 64 (32 with limbs), K a multiple of 512: weight
//    streaming with MFMA; see the kernel.
//  * gemm_mfma: other M > 16 shapes (K not a multiple of 128). 128x128 tile,
//    K in steps of 64 bytes staged through registers into padded LDS rows.
//  * gemv: M <= 16 (decode). Weight streaming: one wave per output column,
//    16 bytes per lane per step (1 KiB contiguous per wave), v_dot4 on the
//    activation rows, wave reduction, epilogue by lane 0.
//
// 16-bit weights (BitExact blog, "Fix the arithmetic": limb products into
// wide accumulators) arrive as hi = W16 >> 8 and lo' = (W16 & 255) - 128:
// acc64 = 256 * (A.hi) + (A.lo') + 128 * rowsum(A).
#include "dev_int.h"
#include "internal.h"
#include <type_traits>

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
  if (e.mode == MODE_REQ_I8) {
    ((int8_t*)out)[o] = clamp8(y);
  } else if (e.mode == MODE_FIX) {
    bound_raise(i32_check(y));
    ((int32_t*)out)[o] = (int32_t)y;
  } else {
    const int64_t t = (int64_t)((int32_t*)out)[o] + y;
    bound_raise(res_check(t, e.res_bits));
    ((int32_t*)out)[o] = (int32_t)t;
  }
}

// epi_store with the output index, the row and column scales and (RES_ADD)
// the residual already loaded
template <bool WIDE>
__device__ __forceinline__ void epi_store_pre(int64_t acc, int64_t o, int32_t rm, int32_t rk,
                                              int32_t cm, int32_t res, const Epi& e, void* out) {
  if (e.mode == MODE_RAW) {
    if (WIDE)
      ((int64_t*)out)[o] = acc;
    else
      ((int32_t*)out)[o] = (int32_t)acc;
    return;
  }
  const int s = rk + e.col_k - (e.mode == MODE_REQ_I8 ? 0 : e.frac);
  const int64_t y = WIDE ? R128((__int128)(acc * rm) * cm, s) : R(acc * rm * cm, s);
  if (e.mode == MODE_REQ_I8) {
    ((int8_t*)out)[o] = clamp8(y);
  } else if (e.mode == MODE_FIX) {
    bound_raise(i32_check(y));
    ((int32_t*)out)[o] = (int32_t)y;
  } else {
    const int64_t t = (int64_t)res + y;
    bound_raise(res_check(t, e.res_bits));
    ((int32_t*)out)[o] = (int32_t)t;
  }
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

// ------------------------------------------------------- pipelined MFMA GEMM

#define DETINT_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int PBK = 128;  // K bytes per pipeline tile

// Physical 16-byte chunk of logical chunk c in LDS row r (128-byte rows): two
// rows share a 256-byte bank window, so 16 consecutive rows must land on 16
// distinct chunk slots.
__device__ __forceinline__ int pswz(int c, int r) { return c ^ ((r >> 1) & 7); }

// buffer resource over [base, base + bytes): loads past the end return zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// Epilogue helper: hands one 32x32 sub-tile's accumulators (both limb planes)
// to the epilogue where it is used. The empty volatile asm is a point the
// compiler cannot move their reads or their widening to 64 bits across, so it
// no longer converts every accumulator of the tile at the end of the K loop
// (256 values that do not fit the register file and went to scratch).
template <int NB, typename Acc>
__device__ __forceinline__ void pin_acc(Acc& acc, int a, int t) {
  asm volatile("" : "+v"(acc[0][a][t]));
  if (NB > 1) asm volatile("" : "+v"(acc[NB - 1][a][t]));
}

template <int BM, int BN, int ST, bool WIDE, int MODE, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_pipe(const int8_t* __restrict__ A,
                                                 const int8_t* __restrict__ W,
                                                 const int8_t* __restrict__ Wlo, int M, int N,
                                                 int K, Epi e, void* out, int kspan) {
  // Split-K (RAW only): workgroup row blockIdx.y covers K range
  // [blockIdx.y kspan, (blockIdx.y + 1) kspan) and writes its partial sums to
  // the int32 slice blockIdx.y of out ([gridDim.y][M][N]); kspan = K otherwise.
  constexpr int NB = WIDE ? 2 : 1;             // weight planes
  constexpr int CPR = PBK / 16;                // chunks per row
  constexpr int SA = BM * PBK, SB = BN * PBK;  // bytes per stage and operand
  constexpr int NT = 64 * WGM * WGN;           // threads: a WGM x WGN grid of waves
  constexpr int LA = SA / (16 * NT), LB = SB / (16 * NT);  // buffer loads per thread per stage
  constexpr int LT = LA + NB * LB;
  static_assert(LA * 16 * NT == SA && LB * 16 * NT == SB, "stage must split evenly over the threads");
  constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 32, TN = WN / 32;
  constexpr int NS = PBK / 32;                 // MFMA k-steps per tile
  static_assert(NS % 2 == 0, "fragment double buffer assumes an even step count");
  extern __shared__ __attribute__((aligned(1024))) int8_t smem[];
  int8_t* sA = smem;
  int8_t* sB = smem + ST * SA;  // [ST][NB][SB]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: LDS DMA bases in SGPRs
  const int wm = wave / WGN, wn = wave % WGN;
  // Tile order. Workgroups are dealt round-robin to the 8 XCDs: give each XCD
  // a contiguous run of logical tiles, then sweep groups of 8 tile rows
  // column by column, so an XCD's L2 holds the A rows and W columns it reuses.
  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN, nb = nbm * nbn;
  int b = blockIdx.x;
  const int q8 = nb >> 3;
  if (b < 8 * q8) b = (b & 7) * q8 + (b >> 3);
  constexpr int G = 8;
  const int grp = (int)udiv32((uint32_t)b, (uint32_t)(G * nbn)), first = grp * G,
            gm = min(nbm - first, G);
  const int inr = b - grp * G * nbn, tn = (int)udiv32((uint32_t)inr, (uint32_t)gm);
  const int tm = first + inr - tn * gm;
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = kspan / PBK, kbase = blockIdx.y * kspan;
  if (MODE == MODE_RAW && gridDim.y > 1) out = (int32_t*)out + (int64_t)blockIdx.y * M * N;

  const __amdgpu_buffer_rsrc_t ra = brsrc(A, (int64_t)M * K);
  const __amdgpu_buffer_rsrc_t rb = brsrc(W, (int64_t)N * K);
  const __amdgpu_buffer_rsrc_t rl = brsrc(WIDE ? Wlo : W, (int64_t)N * K);
  // stage kt % ST <- tile kt. Load q of thread t moves chunk g = NT q + t of
  // the stage: LDS bytes [16g, 16g + 16) = row g / 8, physical chunk g % 8.
  // Loads 0 .. LA-1 fill A, the rest the weight plane(s).
  auto issue_one = [&](int kt, int i) {
    const int st = kt % ST, k0 = kbase + kt * PBK;
    if (i < LA) {
      const int g = i * NT + tid, r = g / CPR;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, DETINT_LDS(sA + st * SA + (i * NT + wave * 64) * 16), 16,
          (m0 + r) * K + k0 + pswz(g % CPR, r) * 16, 0, 0, 0);
    } else {
      const int p = (i - LA) / LB, q = (i - LA) % LB;
      const int g = q * NT + tid, r = g / CPR;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          p ? rl : rb, DETINT_LDS(sB + (st * NB + p) * SB + (q * NT + wave * 64) * 16), 16,
          (n0 + r) * K + k0 + pswz(g % CPR, r) * 16, 0, 0, 0);
    }
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LT; ++i) issue_one(kt, i);
  };

  v16i acc[NB][TM][TN];
#pragma unroll
  for (int p = 0; p < NB; ++p)
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[p][a][t][r] = 0;
  int rsum[TM];  // WIDE: partial row sums of A over this lane's fragment bytes
#pragma unroll
  for (int a = 0; a < TM; ++a) rsum[a] = 0;

  v4i fa[2][TM], fb[2][NB][TN];
  auto frag = [&](int kt, int s, int buf) {
    const int8_t* a_s = sA + (kt % ST) * SA;
    const int c = 2 * s + (lane >> 5);
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int r = wm * WM + a * 32 + (lane & 31);
      fa[buf][a] = *(const v4i*)(a_s + r * PBK + (pswz(c, r) << 4));
    }
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = wn * WN + t * 32 + (lane & 31);
        fb[buf][p][t] = *(const v4i*)(sB + ((kt % ST) * NB + p) * SB + r * PBK + (pswz(c, r) << 4));
      }
  };
  // The MFMAs of one k-step; when kt_load >= 0 the LT loads of that tile go
  // out one after each MFMA, so their issue overlaps matrix work.
  // first: MFMAs with index (p TM + a) TN + t below it are issued by an
  // earlier call (mma_first) for the same step.
  auto mma = [&](int buf, int kt_load, auto first_c) {
    constexpr int first = decltype(first_c)::value;
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const int i = (p * TM + a) * TN + t;
          if (i < first) continue;
          acc[p][a][t] =
              __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[buf][a], fb[buf][p][t], acc[p][a][t], 0, 0, 0);
          if (i < LT && kt_load >= 0) issue_one(kt_load, i);
        }
#pragma unroll
    for (int i = NB * TM * TN; i < LT; ++i)
      if (kt_load >= 0) issue_one(kt_load, i);
    if (WIDE) {
      const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
      for (int a = 0; a < TM; ++a) rsum[a] = dot16(fa[buf][a], ones, rsum[a]);
    }
  };

  // The first two MFMAs of a step, issued before that step's reads of the
  // next step's fragments, so no MFMA waits on a read issued in its own step.
  constexpr int PRE = 2;
  static_assert(NB * TM * TN >= PRE, "fewer MFMAs per step than the lead-in");
  auto mma_first = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PRE; ++i) {
      const int p = i / (TM * TN), a = (i / TN) % TM, t = i % TN;
      acc[p][a][t] =
          __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[buf][a], fb[buf][p][t], acc[p][a][t], 0, 0, 0);
    }
  };

  // every stage in flight, then wait for tile 0
#pragma unroll
  for (int s = 0; s < ST; ++s)
    if (s < nk) issue(s);
  if (ST - 1 < nk)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((ST - 1) * LT) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  frag(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int buf = s & 1;
      if (s + 1 < NS) {
        mma_first(buf);
        __builtin_amdgcn_sched_barrier(0);
        frag(kt, s + 1, buf ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(buf, -1, std::integral_constant<int, PRE>{});
        __builtin_amdgcn_sched_barrier(0);
        continue;
      } else if (kt + 1 < nk) {
        // Tile kt+1 resident (own loads counted, others' by the barrier) and
        // every wave's reads of tile kt issued and complete, so its stage can
        // be refilled with tile kt+ST.
        if (ST > 2 && kt + ST - 1 < nk)
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((ST > 2 ? ST - 2 : 0) * LT) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        frag(kt + 1, 0, buf ^ 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      mma(buf, kt + ST < nk ? kt + ST : -1, std::integral_constant<int, 0>{});
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Epilogue straight from the accumulators (fully unrolled so they stay
  // statically indexed). Loads use clamped indices and are unconditional, so
  // each tile's are issued together; only the stores are guarded. Accumulator
  // layout of a 32x32 tile: lane l, register r -> row 8 * (r / 4) + 4 * (l / 32)
  // + r % 4, column l % 32.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();  // every wave done with the LDS ring
  // per row r of the tile, ints 4 r .. 4 r + 3: {WIDE: row sum of A, row
  // scale, total shift, shift - 33}, stored one int at a time (a store to one
  // lane of a 16-byte vector would rewrite all four) and read as one vector
  int32_t* s_row = (int32_t*)smem;
  if (WIDE && wn == 0) {
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int v = rsum[a] + __shfl_xor(rsum[a], 32);
      if (lane < 32) s_row[4 * (wm * WM + a * 32 + lane)] = v;  // |v| <= 128 K
    }
  }
  // The fast path needs every scale in [0, 2^15) and every shift in [1, 62]
  // (int8 weights) or [33, 94] with K < 2^16 (limbs); anything else takes
  // the general per-element path below.
  const int csh = e.col_k - (MODE == MODE_REQ_I8 ? 0 : e.frac);
  int slow = 0, narrow = 0;
  if (MODE != MODE_RAW) {
    for (int t = tid; t < BM; t += NT) {
      const int i = min(m0 + t, M - 1);
      const int rm = e.row_m[i], sh = e.row_k[i] + csh;
      s_row[4 * t + 1] = rm;
      s_row[4 * t + 2] = sh;
      s_row[4 * t + 3] = sh - 33;
      slow |= (unsigned)rm >= 32768u || (WIDE ? sh < 33 || sh > 94 || K >= 65536 : sh < 1 || sh > 62);
      narrow |= sh < 33;
    }
    for (int t = tid; t < BN; t += NT) slow |= (unsigned)e.col_m[min(n0 + t, N - 1)] >= 32768u;
  }
  const int64_t obase = e.out_row_base ? *e.out_row_base : 0;
  slow = __syncthreads_or(slow);
  // int8 weights with every shift >= 33: R(p, s) = (hi(p) + 2^(s-33)) >> (s-32)
  // exactly, hi(p) the upper 32 bits of the 64-bit product p (the low word
  // cannot carry into the floor), so the product needs one mul_hi
  const bool hi_only = !WIDE && !__syncthreads_or(narrow);
  if (MODE != MODE_RAW && !slow && m0 + BM <= M && n0 + BN <= N &&
      (int64_t)BM * N * (MODE == MODE_REQ_I8 ? 1 : 4) < (int64_t(1) << 31)) {
    // Interior tile, in-range scales: no bounds checks, branch-free rounding.
    // int8 weights: |m_r * m_c| < 2^30, so acc * m_r * m_c is one 32 x 32 ->
    // 64-bit product. For a shift s >= 33, R(p, s) = (floor(p / 2^32) +
    // 2^(s-33)) >> (s-32) exactly (p's low word cannot carry into the floor).
    // Limbs: v = 256 hi + w with w = lo + 128 rowsum = sum A (W & 255), |w| <
    // 2^15 K < 2^31; M = m_r m_c < 2^30; with v = vh 2^32 + vl (0 <= vl <
    // 2^32), floor(v M / 2^32) = vh M + mulhi(vl, M).
    auto tiles = [&](auto hi) {  // hi: every shift >= 33 (compile-time flag)
      constexpr bool HI = decltype(hi)::value;
      constexpr int EB = MODE == MODE_REQ_I8 ? 1 : 4;  // output element bytes
      // the tile's output block through a buffer resource (it spans fewer
      // than 2^31 bytes): a lane offset per 32x32 sub-tile in a VGPR, the
      // offsets of its 16 rows as scalars
      const __amdgpu_buffer_rsrc_t ro =
          brsrc((const int8_t*)out + ((m0 + obase) * N + n0) * EB, (int64_t)BM * N * EB);
      // bound checks as OR-accumulated words (no per-element compares):
      // nonzero when a result left int32 / when a residual sum t had
      // |t| >= 2^res_bits (t + 2^b - 1 < 0 or t - 2^b >= 0)
      uint32_t ovf = 0, ovr = 0;
      const int rb = e.res_bits;
      const int64_t rlo = rb > 0 ? (int64_t(1) << rb) - 1 : 0, rhi = rb > 0 ? int64_t(1) << rb : 0;
#pragma clang loop unroll(full)
      for (int a = 0; a < TM; ++a)
#pragma clang loop unroll(full)
        for (int t = 0; t < TN; ++t) {
          if constexpr (WIDE) pin_acc<NB>(acc, a, t);
          const int jj = wn * WN + t * 32 + (lane & 31);
          const int32_t cm = e.col_m[n0 + jj];
          const int lb = wm * WM + a * 32 + 4 * (lane >> 5);
          const int vo = (lb * N + jj) * EB;
          int32_t old[16];
          if (MODE == MODE_RES_ADD) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              old[r] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ro, vo, (8 * (r >> 2) + (r & 3)) * N * EB, 0);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int li = lb + 8 * (r >> 2) + (r & 3);
            const int so = (8 * (r >> 2) + (r & 3)) * N * EB;
            const v4i rw = *(const v4i*)(s_row + 4 * li);
            const uint32_t Mrc = (uint32_t)__mul24(rw[1], cm);
            // R(x, s) = ((x >> (s - 1)) + 1) >> 1 for s >= 1, and the
            // floor(p / 2^32) form above: R(p, s) = ((floor(p / 2^32) >> (s -
            // 33)) + 1) >> 1 for s >= 33 (rw[3] = s - 33)
            int64_t y;
            if (WIDE) {
              const int32_t w = acc[NB - 1][a][t][r] + rw[0] * 128;
              const int64_t v = (int64_t)acc[0][a][t][r] * 256 + w;
              const int64_t q = (int64_t)(int32_t)(v >> 32) * (int64_t)(int32_t)Mrc +
                                (int64_t)__umulhi((uint32_t)v, Mrc);
              y = ((q >> rw[3]) + 1) >> 1;
            } else if (HI) {
              const int32_t ph = __mulhi(acc[0][a][t][r], (int32_t)Mrc);
              y = ((ph >> rw[3]) + 1) >> 1;
            } else {
              const int64_t pr = (int64_t)acc[0][a][t][r] * (int64_t)Mrc;
              y = ((pr >> (rw[2] - 1)) + 1) >> 1;
            }
            if (MODE == MODE_REQ_I8) {
              __builtin_amdgcn_raw_buffer_store_b8((uint8_t)clamp8(y), ro, vo, so, 0);
            } else if (MODE == MODE_FIX) {
              if (!HI) ovf |= (uint32_t)((uint64_t)(y + 2147483648LL) >> 32);  // mul_hi results fit
              __builtin_amdgcn_raw_buffer_store_b32((uint32_t)y, ro, vo, so, 0);
            } else {
              const int64_t tsum = (int64_t)old[r] + y;
              if (rb > 0)
                ovr |= (uint32_t)((uint64_t)(tsum + rlo) >> 63) | (uint32_t)(~(uint64_t)(tsum - rhi) >> 63);
              else
                ovf |= (uint32_t)((uint64_t)(tsum + 2147483648LL) >> 32);
              __builtin_amdgcn_raw_buffer_store_b32((uint32_t)tsum, ro, vo, so, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      bound_raise((ovf ? (uint32_t)kBoundInt32 : 0u) | (ovr ? (uint32_t)kBoundResidual : 0u));
    };
    // one copy of the unrolled tile loop per case (a per-element branch
    // would interleave both and double the code the loop runs through)
    if constexpr (!WIDE) {
      if (hi_only) {
        tiles(std::true_type{});
        return;
      }
    }
    tiles(std::false_type{});
    return;
  }
  uint32_t bad = 0;
#pragma clang loop unroll(full)
  for (int a = 0; a < TM; ++a)
#pragma clang loop unroll(full)
    for (int t = 0; t < TN; ++t) {
      if constexpr (WIDE) pin_acc<NB>(acc, a, t);
      const int j = n0 + wn * WN + t * 32 + (lane & 31), jc = min(j, N - 1);
      const int32_t cm = MODE != MODE_RAW ? e.col_m[jc] : 0;
      const int lb = wm * WM + a * 32 + 4 * (lane >> 5);
      int32_t old[16];
      if (MODE == MODE_RES_ADD) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = min(m0 + lb + 8 * (r >> 2) + (r & 3), M - 1);
          old[r] = ((const int32_t*)out)[(i + obase) * N + jc];
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int li = lb + 8 * (r >> 2) + (r & 3), i = m0 + li;
        int64_t v = acc[0][a][t][r];
        if (WIDE) v = 256 * v + (int64_t)acc[NB - 1][a][t][r] + 128 * (int64_t)s_row[4 * li];
        const int64_t o = (i + obase) * N + j;
        if (MODE == MODE_RAW) {
          if (i < M && j < N) {
            if (WIDE)
              ((int64_t*)out)[o] = v;
            else
              ((int32_t*)out)[o] = (int32_t)v;
          }
          continue;
        }
        const int sh = s_row[4 * li + 2];
        const int64_t y = WIDE ? R128((__int128)(v * s_row[4 * li + 1]) * cm, sh)
                               : R((int64_t)(int32_t)v * s_row[4 * li + 1] * cm, sh);
        if (i < M && j < N) {
          if (MODE == MODE_REQ_I8) {
            ((int8_t*)out)[o] = clamp8(y);
          } else if (MODE == MODE_FIX) {
            bad |= i32_check(y);
            ((int32_t*)out)[o] = (int32_t)y;
          } else {
            const int64_t tsum = (int64_t)old[r] + y;
            bad |= res_check(tsum, e.res_bits);
            ((int32_t*)out)[o] = (int32_t)tsum;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep tiles' live ranges apart
    }
  bound_raise(bad);
}

template <int BM, int BN, int ST, bool WIDE, int MODE, int WGM, int WGN>
hipError_t pipe_launch_m(const int8_t* A, const int8_t* W, const int8_t* Wlo, int M, int N, int K,
                         const Epi& e, void* out, hipStream_t st) {
  constexpr int lds = ST * (BM + (WIDE ? 2 : 1) * BN) * PBK;
  static_assert(lds <= 160 * 1024, "LDS ring exceeds the workgroup limit");
  const hipError_t err = set_max_lds((const void*)gemm_pipe<BM, BN, ST, WIDE, MODE, WGM, WGN>, lds);
  if (err != hipSuccess) return err;
  const int nb = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  gemm_pipe<BM, BN, ST, WIDE, MODE, WGM, WGN><<<nb, 64 * WGM * WGN, lds, st>>>(A, W, Wlo, M, N, K, e,
                                                                              out, K);
  return hipGetLastError();
}

// Split-K over ks workgroup rows (int8 weights, RAW partials into part
// [ks][M][N]), then one kernel sums the ks partials (exact: |sum| < 2^31 by
// the K bound) and applies the epilogue.
__global__ __launch_bounds__(256) void splitk_reduce_k(const int32_t* __restrict__ part, int ks,
                                                       int M, int N, Epi e, void* out) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= N) return;
  const int64_t plane = (int64_t)M * N;
  for (int i = blockIdx.y; i < M; i += gridDim.y) {
    int64_t v = 0;
    for (int s = 0; s < ks; ++s) v += part[s * plane + (int64_t)i * N + j];
    epi_store<false>(v, i, j, N, e, out);
  }
}

hipError_t pipe_splitk(const int8_t* A, const int8_t* W, int M, int N, int K, int ks,
                       const Epi& e, void* out, int32_t* part, hipStream_t st) {
  constexpr int BMs = 128, BNs = 64, STs = 4;
  constexpr int lds = STs * (BMs + BNs) * PBK;
  const hipError_t err = set_max_lds((const void*)gemm_pipe<BMs, BNs, STs, false, MODE_RAW, 2, 2>, lds);
  if (err != hipSuccess) return err;
  const int nb = ((M + BMs - 1) / BMs) * ((N + BNs - 1) / BNs);
  const Epi raw{nullptr, nullptr, nullptr, 0, 0, MODE_RAW, nullptr};
  gemm_pipe<BMs, BNs, STs, false, MODE_RAW, 2, 2><<<dim3((unsigned)nb, (unsigned)ks), 256, lds, st>>>(
      A, W, nullptr, M, N, K, raw, part, K / ks);
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)(M < 65535 ? M : 65535));
  splitk_reduce_k<<<grid, 256, 0, st>>>(part, ks, M, N, e, out);
  return hipGetLastError();
}

template <int BM, int BN, int ST, bool WIDE, int WGM = 2, int WGN = 2>
hipError_t pipe_launch(const int8_t* A, const int8_t* W, const int8_t* Wlo, int M, int N, int K,
                       const Epi& e, void* out, hipStream_t st) {
  switch (e.mode) {
    case MODE_RAW:
      return pipe_launch_m<BM, BN, ST, WIDE, MODE_RAW, WGM, WGN>(A, W, Wlo, M, N, K, e, out, st);
    case MODE_REQ_I8:
      return pipe_launch_m<BM, BN, ST, WIDE, MODE_REQ_I8, WGM, WGN>(A, W, Wlo, M, N, K, e, out, st);
    case MODE_FIX:
      return pipe_launch_m<BM, BN, ST, WIDE, MODE_FIX, WGM, WGN>(A, W, Wlo, M, N, K, e, out, st);
    default:
      return pipe_launch_m<BM, BN, ST, WIDE, MODE_RES_ADD, WGM, WGN>(A, W, Wlo, M, N, K, e, out, st);
  }
}

// Largest tile that still gives the chip most of a wave of workgroups (int8
// weights fall back to 128x64, which fills the chip where 128x128 leaves
// half of it idle, e.g. M = 2048, N = 1024: 20% faster). Every tiling that
// fills the LDS runs 8 waves, two per SIMD, so one wave's barrier and load
// waits run under the other's MFMAs: the 256x256 int8 tiling (2 x 4 waves of
// 128x64) measured 3-16% faster than 4 waves, the 256x128 limb tiling (4 x 2
// waves of 64x64, both planes, 128 accumulators each) 9-13% faster, the
// 128x256 int8 tiling 14% at M = 2048, N = 4096. The 128x64 fallback keeps
// 4 waves (8 would leave each a single 32x32 tile); where even it leaves a
// quarter of the CUs idle, 64x64 tiles of two waves take twice the
// workgroups (M = 512, N = 1024: K = 2048 10.9 -> 9.8 us, K = 3072 14.1
// -> 12.5 us, graph-replayed; a split of K over workgroups was slower
// there, 14.1 us).
template <bool WIDE>
hipError_t pipe_dispatch(const int8_t* A, const int8_t* W, const int8_t* Wlo, int M, int N,
                         int K, const Epi& e, void* out, hipStream_t st) {
  auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  constexpr int64_t FILL = 192;  // 3/4 of the 256 CUs
  if (WIDE) {
    if (tiles(256, 128) >= FILL) return pipe_launch<256, 128, 2, true, 4, 2>(A, W, Wlo, M, N, K, e, out, st);
    return pipe_launch<128, 128, 3, true, 4, 2>(A, W, Wlo, M, N, K, e, out, st);
  }
  if (tiles(256, 256) >= FILL) return pipe_launch<256, 256, 2, false, 2, 4>(A, W, Wlo, M, N, K, e, out, st);
  if (tiles(128, 256) >= FILL) return pipe_launch<128, 256, 3, false, 4, 2>(A, W, Wlo, M, N, K, e, out, st);
  if (tiles(128, 128) >= FILL) return pipe_launch<128, 128, 4, false, 4, 2>(A, W, Wlo, M, N, K, e, out, st);
  if (tiles(128, 64) < FILL) return pipe_launch<64, 64, 4, false, 2, 1>(A, W, Wlo, M, N, K, e, out, st);
  return pipe_launch<128, 64, 4, false>(A, W, Wlo, M, N, K, e, out, st);
}

// ------------------------------------------------------------- skinny GEMM

// M <= 64 rows (batched decode, short prompts): weight streaming. A
// workgroup of SK_W waves owns 32 NC output columns for all rows; its waves
// split K into SK_W chunks, each streaming its chunk of the weight rows from
// HBM straight into MFMA fragments (buffer loads, one group of SK_G k-steps
// in flight while the previous group is multiplied) against A fragments that
// stay L2-resident. Per-wave partial sums meet in LDS; integer sums are
// order-free, so the split changes no bit. Limb planes are reduced
// separately in int32 (|sum| <= 2^14 K < 2^31) and combined in int64 at the
// end. SK_W = 4 waves where the column tiles alone fill the chip (each wave
// streams a quarter of K and several workgroups share a CU: lm_head 235 ->
// 163 us at batch 32), 16 where few tiles need K split over waves and
// workgroups to fill it (4 waves there left a CU a quarter of the loads).
// Where 64-column tiles still give 256 workgroups, a workgroup takes two
// adjacent 32-column tiles (NC = 2): each A fragment, reloaded per tile
// otherwise, feeds both tiles' MFMAs (64 x 1024 x 151936, cache-cold: 107
// -> 88 us; batch-32 limb gate/up 26.6 -> 25.4 us; not the limb lm_head,
// see skinny_launch).
constexpr int SK_KQ = 512;  // K granularity of the skinny path (and of its splits)

// Split-K across workgroups (grid.y = ks > 1, given a workspace): split s
// covers K range [s K / ks, (s + 1) K / ks); each split writes its partial
// sums for the tile to sp.part, and the last split to arrive (counted in
// sp.cnt[tile], which it resets to 0) adds the ks partials - an exact integer
// sum, so the split changes no bit - and runs the epilogue.
template <bool WIDE, int MR, int SK_W, int NC>
__global__ __launch_bounds__(64 * SK_W) void gemm_skinny(const int8_t* __restrict__ A,
                                                         const int8_t* __restrict__ W,
                                                         const int8_t* __restrict__ Wlo, int M, int N,
                                                         int K, Epi e, void* out, SplitWs sp) {
  constexpr int SK_T = 64 * SK_W;
  constexpr int SK_O = 1024 / SK_T;  // outputs of a 32 x 32 tile per thread
  // k-steps per load group: 16 waves keep 2 (128 registers each), 4 waves
  // stream four times the K range and take 4, or 2 with two column tiles
  constexpr int SK_G = SK_W == 16 || NC == 2 ? 2 : 4;
  constexpr int NB = WIDE ? 2 : 1;
  constexpr int TE = NB * MR * 1024 + MR * 32;       // partial ints per (tile, split)
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  int32_t* part = (int32_t*)smem;                   // [SK_W][NC][NB][MR][32 * 32]
  int32_t* prs = part + SK_W * NC * NB * MR * 1024;  // [SK_W][MR * 32] row sums
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 32 * NC, ks = gridDim.y, split = blockIdx.y;
  const int kspl = (int)udiv32((uint32_t)K, (uint32_t)ks);  // K range of one split
  const int kc = kspl / SK_W, nst = kc / 32;
  const int kb = split * kspl + wave * kc + (lane >> 5) * 16;
  const __amdgpu_buffer_rsrc_t ra = brsrc(A, (int64_t)M * K);
  const __amdgpu_buffer_rsrc_t rb = brsrc(W, (int64_t)N * K);
  const __amdgpu_buffer_rsrc_t rl = brsrc(WIDE ? Wlo : W, (int64_t)N * K);
  // weight row of this lane's output column in column tile t (columns n0 +
  // 32 t ..); in SWIGLU mode a tile's 32 columns are gate columns j0 .. j0 +
  // 15 then up columns j0 .. j0 + 15 (j0 = n0t / 2), so each gate/up pair
  // meets in one workgroup. With NC = 2 tiles every A fragment serves two
  // tiles' MFMAs, halving the A loads per weight load.
  const bool swg = e.mode == MODE_SWIGLU;
  const int cl = lane & 31;
  const int aoff = (lane & 31) * K + kb;
  int woff[NC];
#pragma unroll
  for (int t = 0; t < NC; ++t) {
    const int n0t = n0 + 32 * t;
    const int wrow = swg ? (cl < 16 ? (n0t >> 1) + cl : (N >> 1) + (n0t >> 1) + cl - 16) : n0t + cl;
    woff[t] = wrow * K + kb;
  }

  v16i acc[NC][NB][MR];
#pragma unroll
  for (int t = 0; t < NC; ++t)
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][p][m][r] = 0;
  int rsum[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) rsum[m] = 0;
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

  v4i fa[2][SK_G][MR], fw[2][SK_G][NC][NB];
  auto load = [&](int g, int buf) {
#pragma unroll
    for (int s = 0; s < SK_G; ++s) {
      const int k = (g * SK_G + s) * 32;
      if (g * SK_G + s < nst) {
#pragma unroll
        for (int t = 0; t < NC; ++t)
#pragma unroll
          for (int p = 0; p < NB; ++p)
            fw[buf][s][t][p] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_raw_buffer_load_b128(p ? rl : rb, woff[t] + k, 0, 0));
#pragma unroll
        for (int m = 0; m < MR; ++m)
          fa[buf][s][m] = __builtin_bit_cast(
              v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff + m * 32 * K + k, 0, 0));
      }
    }
  };
  // Epilogue operands, loaded before the weights so that their latency
  // hides under the streaming (loaded inside the epilogue, each output's
  // scales would wait behind the previous output's store, which may alias
  // them): per output of this thread, the row and column scales and, for
  // RES_ADD, the residual it adds to; the output row base once. Thread t
  // finishes outputs o = t + SK_T q of each 32 x 32 block m: row m 32 +
  // o / 32, column o % 32 of the tile (in SWIGLU mode the weight row of
  // that gate or up column).
  // The rows' scales come from one load per lane (lane l: row min(l, M - 1),
  // M <= 64), handed out by lane reads after the stream (a read here would
  // wait for the load before the weights go out): output o of block m sits
  // in row m 32 + 2 wave + 2 SK_W q + (lane >= 32), so two wave-uniform lane
  // reads serve each (m, q) - per-output loads would cost the texture unit
  // as much as a third of the weight stream. The column's mantissa is the
  // same for every (m, q) of a thread (column o % 32 = lane % 32).
  const int64_t orb = e.out_row_base ? *e.out_row_base : 0;
  int32_t eres[NC][MR][SK_O];
  int32_t ecm[NC], vrm, vrk;
  const int w2 = 2 * __builtin_amdgcn_readfirstlane(wave);
  {
    const bool scaled = e.mode != MODE_RAW;
    const int lr = lane < M ? lane : M - 1;
    vrm = scaled ? e.row_m[lr] : 0;
    vrk = scaled ? e.row_k[lr] : 0;
    const int c = lane & 31;
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int n0t = n0 + 32 * t;
      int jc;
      if (swg) {
        const int wr = c < 16 ? (n0t >> 1) + c : (N >> 1) + (n0t >> 1) + c - 16;
        jc = wr < N ? wr : N - 1;
      } else {
        jc = n0t + c < N ? n0t + c : N - 1;
      }
      ecm[t] = scaled ? e.col_m[jc] : 0;
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int q = 0; q < SK_O; ++q) {
          const int i = m * 32 + w2 + 2 * SK_W * q + (lane >> 5), ic = i < M ? i : M - 1;
          eres[t][m][q] = e.mode == MODE_RES_ADD ? ((const int32_t*)out)[(orb + ic) * N + jc] : 0;
        }
    }
  }
  const int ng = (nst + SK_G - 1) / SK_G;
  auto group = [&](int g, int buf) {  // buf is a constant at each call
    if (g + 1 < ng) load(g + 1, buf ^ 1);
#pragma unroll
    for (int s = 0; s < SK_G; ++s) {
      if (g * SK_G + s < nst) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
#pragma unroll
          for (int t = 0; t < NC; ++t)
#pragma unroll
            for (int p = 0; p < NB; ++p)
              acc[t][p][m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[buf][s][m], fw[buf][s][t][p],
                                                                   acc[t][p][m], 0, 0, 0);
          if (WIDE) rsum[m] = dot16(fa[buf][s][m], ones, rsum[m]);
        }
      }
    }
  };
  load(0, 0);
  for (int g = 0; g < ng; g += 2) {
    group(g, 0);
    if (g + 1 < ng) group(g + 1, 1);
  }
  // partials to LDS (accumulator layout: lane l, register r -> row
  // 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32)
#pragma unroll
  for (int t = 0; t < NC; ++t)
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          part[(((wave * NC + t) * NB + p) * MR + m) * 1024 + (8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * 32 +
               (lane & 31)] = acc[t][p][m][r];
  if (WIDE) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const int v = rsum[m] + __shfl_xor(rsum[m], 32);
      if (lane < 32) prs[wave * MR * 32 + m * 32 + lane] = v;
    }
  }
  __syncthreads();
  // thread t finishes outputs o = t + SK_T q of each 32 x 32 block m: row
  // m * 32 + o / 32, column o % 32
  int32_t hs[NC][MR][SK_O], ls[NC][MR][SK_O], rss[MR][SK_O];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < SK_O; ++q) {
      const int o = tid + SK_T * q, row = m * 32 + (o >> 5);
      rss[m][q] = 0;
#pragma unroll
      for (int t = 0; t < NC; ++t) hs[t][m][q] = ls[t][m][q] = 0;
#pragma unroll
      for (int w = 0; w < SK_W; ++w) {
#pragma unroll
        for (int t = 0; t < NC; ++t) {
          hs[t][m][q] += part[(((w * NC + t) * NB + 0) * MR + m) * 1024 + o];
          if (WIDE) ls[t][m][q] += part[(((w * NC + t) * NB + NB - 1) * MR + m) * 1024 + o];
        }
        if (WIDE) rss[m][q] += prs[w * MR * 32 + row];
      }
    }
  // (split K runs with one column tile per workgroup: NC = 1)
  if (NC == 1 && ks > 1) {
    // Partials go out as agent-scope atomic stores (coherent across the
    // XCDs' L2 caches). Ordering: every thread's stores happen before the
    // workgroup barrier; thread 0's arrival is a release RMW at agent scope,
    // which publishes them. RMWs continue release sequences, so the split
    // whose RMW reads ks - 1 has read every earlier split's release; its
    // agent-scope acquire fence then synchronises with all of them (only
    // the last split pays for the acquire's cache invalidation). The second
    // barrier carries that to the other threads, which read the partials
    // back with agent-scope atomic loads.
    auto put = [](int32_t* p, int32_t v) {
      __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto get = [](const int32_t* p) {
      return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    int32_t* mine = sp.part + ((size_t)blockIdx.x * ks + split) * TE;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int q = 0; q < SK_O; ++q) {
        const int o = tid + SK_T * q;
        put(&mine[m * 1024 + o], hs[0][m][q]);
        if (WIDE) put(&mine[(MR + m) * 1024 + o], ls[0][m][q]);
        if (WIDE && (o & 31) == 0) put(&mine[NB * MR * 1024 + m * 32 + (o >> 5)], rss[m][q]);
      }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const bool last = __hip_atomic_fetch_add(&sp.cnt[blockIdx.x], 1, __ATOMIC_RELEASE,
                                               __HIP_MEMORY_SCOPE_AGENT) == ks - 1;
      if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    const int32_t* all = sp.part + (size_t)blockIdx.x * ks * TE;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int q = 0; q < SK_O; ++q) {
        const int o = tid + SK_T * q;
        hs[0][m][q] = ls[0][m][q] = rss[m][q] = 0;
        for (int t = 0; t < ks; ++t) {
          hs[0][m][q] += get(&all[t * TE + m * 1024 + o]);
          if (WIDE) {
            ls[0][m][q] += get(&all[t * TE + (MR + m) * 1024 + o]);
            rss[m][q] += get(&all[t * TE + NB * MR * 1024 + m * 32 + (o >> 5)]);
          }
        }
      }
    if (tid == 0) put(&sp.cnt[blockIdx.x], 0);  // ready for the next call
  }
  int32_t erm[MR][SK_O], erk[MR][SK_O];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < SK_O; ++q) {
      const int ib = m * 32 + w2 + 2 * SK_W * q;  // <= 62
      const int32_t m0 = __builtin_amdgcn_readlane(vrm, ib), m1 = __builtin_amdgcn_readlane(vrm, ib + 1);
      const int32_t k0 = __builtin_amdgcn_readlane(vrk, ib), k1 = __builtin_amdgcn_readlane(vrk, ib + 1);
      erm[m][q] = lane < 32 ? m0 : m1;
      erk[m][q] = lane < 32 ? k0 : k1;
    }
  if (swg) {
    // FIX value of this thread's gate or up column, then the gate thread
    // (column c < 16) takes its up partner's from the lane 16 apart
#pragma unroll
    for (int t = 0; t < NC; ++t)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int q = 0; q < SK_O; ++q) {
        const int o = tid + SK_T * q;
        const int i = m * 32 + (o >> 5), c = o & 31;
        int64_t v = hs[t][m][q];
        if (WIDE) v = 256 * v + (int64_t)ls[t][m][q] + 128 * (int64_t)rss[m][q];
        const int s = erk[m][q] + e.col_k - e.frac;
        const int64_t y = WIDE ? R128((__int128)(v * erm[m][q]) * ecm[t], s)
                               : R(v * erm[m][q] * ecm[t], s);
        const int64_t u = lane_xor<16>(y);
        const int j = ((n0 + 32 * t) >> 1) + c;
        if (c < 16 && i < M && j < (N >> 1)) {
          bound_raise(out_of(y, 24) | out_of(u, 24) ? kBoundSwiglu : 0u);
          ((int64_t*)out)[(size_t)i * (N >> 1) + j] = R(y * sigmoid_q15(y, e.sw_mg, e.sw_kg), 15) * u;
        }
      }
    return;
  }
#pragma unroll
  for (int t = 0; t < NC; ++t)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int q = 0; q < SK_O; ++q) {
        const int o = tid + SK_T * q;
        const int i = m * 32 + (o >> 5), j = n0 + 32 * t + (o & 31);
        if (i < M && j < N) {
          int64_t v = hs[t][m][q];
          if (WIDE) v = 256 * v + (int64_t)ls[t][m][q] + 128 * (int64_t)rss[m][q];
          epi_store_pre<WIDE>(v, (orb + i) * N + j, erm[m][q], erk[m][q], ecm[t], eres[t][m][q], e, out);
        }
      }
}

// K splits for a skinny GEMM: the most workgroups that still run as one
// round (one workgroup per CU, 256 CUs: a second round would
// repeat the whole load / reduce / epilogue latency), each split a multiple
// of 512 bytes of K, within the workspace.
int skinny_splits(int64_t N, int64_t K, const SplitWs* sp) {
  if (!sp || !sp->part) return 1;
  const int64_t tiles = (N + 31) / 32;
  if (tiles >= 256) return 1;  // already a workgroup per CU
  int ks = 1;
  for (int c = 2; c <= 16; ++c) {
    if (tiles * c > 256) break;
    if (K % (c * SK_KQ) != 0) continue;
    if (tiles * c > sp->max_tile_splits || tiles > sp->max_tiles) break;
    ks = c;
  }
  return ks;
}

template <bool WIDE, int MR, int SK_W, int NC = 1>
hipError_t skinny_launch_w(const int8_t* A, const int8_t* W, const int8_t* Wlo, int M, int N, int K,
                           const Epi& e, void* out, const SplitWs* sp, int ks, hipStream_t st) {
  constexpr int lds = (SK_W * NC * (WIDE ? 2 : 1) * MR * 1024 + SK_W * MR * 32) * 4;
  static_assert(lds <= 160 * 1024, "skinny partials exceed the workgroup LDS");
  if (NC > 1 && ks > 1) return hipErrorInvalidValue;  // split K takes one column tile
  const hipError_t err = set_max_lds((const void*)gemm_skinny<WIDE, MR, SK_W, NC>, lds);
  if (err != hipSuccess) return err;
  const SplitWs none{};
  gemm_skinny<WIDE, MR, SK_W, NC><<<dim3((unsigned)((N + 32 * NC - 1) / (32 * NC)), (unsigned)ks), 64 * SK_W, lds, st>>>(
      A, W, Wlo, M, N, K, e, out, ks > 1 ? *sp : none);
  return hipGetLastError();
}

template <bool WIDE, int MR>
hipError_t skinny_launch(const int8_t* A, const int8_t* W, const int8_t* Wlo, int M, int N, int K,
                         const Epi& e, void* out, const SplitWs* sp, hipStream_t st) {
  // two tiles per workgroup: limb weights already load two weight
  // fragments per A fragment, so on a vocabulary-wide limb head (4008
  // tiles, already many workgroups per CU) the saving does not pay for the
  // lower occupancy (165.5 against 167.0 us)
  if ((N + 63) / 64 >= 256 && (!WIDE || (N + 31) / 32 < 2048))
    return skinny_launch_w<WIDE, MR, 4, 2>(A, W, Wlo, M, N, K, e, out, sp, 1, st);
  if ((N + 31) / 32 >= 256) return skinny_launch_w<WIDE, MR, 4>(A, W, Wlo, M, N, K, e, out, sp, 1, st);
  return skinny_launch_w<WIDE, MR, 16>(A, W, Wlo, M, N, K, e, out, sp, skinny_splits(N, K, sp), st);
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
          uint32_t bad = i32_check(y0);
          if (lane == 0) ((int32_t*)out)[base * N + j0] = (int32_t)y0;
          if (two) {
            const int64_t y1 = WIDE ? R128((__int128)(s1 * e.row_m[m]) * e.col_m[j0 + 1], sh)
                                    : R(s1 * e.row_m[m] * e.col_m[j0 + 1], sh);
            bad |= i32_check(y1);
            if (lane == 0) ((int32_t*)out)[base * N + j0 + 1] = (int32_t)y1;
            const int64_t k1 = amax_key(y1, j0 + 1);
            k0 = k1 > k0 ? k1 : k0;
          }
          if (lane == 0) bound_raise(bad);
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
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;  // one element a thread
  if (i < n) {
    const int v = w[i];
    hi[i] = (int8_t)(v >> 8);
    lo[i] = (int8_t)((v & 255) - 128);
  }
}

// ------------------------------------------------------------- exact mode
//
// bf16 weights as integers (BitExact blog, "Three execution paths": exact
// mode keeps the bf16 weights and multiplies them with fixed-point
// activations). Row j's values are W_int = +-M * 2^(E' - emin_j) with M the
// 8-bit significand (implicit one for normal numbers), E' the exponent field
// (1 for subnormals) and emin_j the row's smallest E' among nonzero entries;
// the row scale is 2^(emin_j - 134). |W_int| < 2^31 (a row spans at most 23
// binary orders), held as four int8 planes: P0 = W_int >> 24 (signed) and
// P1..P3 = the next bytes minus 128, so that
//   W_int = 2^24 P0 + 2^16 P1 + 2^8 P2 + P3 + 128 (2^16 + 2^8 + 1).
// (P0, P1) and (P2, P3) are the limb planes of the 16-bit GEMM for
// H16 = W_int >> 16 and L16 = (W_int & 65535) - 32768; the product is
// acc = 2^16 (A.H16) + A.L16 + 2^15 rowsum(A), exact in int64.

__device__ __forceinline__ int block_min_int(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int w = __shfl_xor(v, o);
    v = w < v ? w : v;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) v = red[w] < v ? red[w] : v;
    red[0] = v;
  }
  __syncthreads();
  v = red[0];
  __syncthreads();
  return v;
}

// one 256-thread workgroup per weight row
__global__ __launch_bounds__(256) void exact_prepare_k(const uint16_t* __restrict__ W, int K,
                                                       int8_t* __restrict__ planes, int64_t plane,
                                                       int32_t* __restrict__ row_exp) {
  __shared__ int red[4];
  const int64_t j = blockIdx.x;
  const uint16_t* w = W + j * K;
  int emin = 255;
  uint32_t bad = 0;
  for (int k = threadIdx.x; k < K; k += 256) {
    const int b = w[k], E = (b >> 7) & 255, f = b & 127;
    const int Ep = E ? E : 1, M = E ? 128 + f : f;
    if (E == 255) bad = kBoundWeight;
    if (M != 0 && Ep < emin) emin = Ep;
  }
  emin = block_min_int(emin, red);
  if (emin == 255) emin = 1;  // an all-zero row
  for (int k = threadIdx.x; k < K; k += 256) {
    const int b = w[k], E = (b >> 7) & 255, f = b & 127;
    const int Ep = E ? E : 1, M = E ? 128 + f : f;
    int32_t v = 0;
    if (M != 0 && E != 255) {
      if (Ep - emin > 23) bad = kBoundWeight;
      else v = M << (Ep - emin);
    }
    if (b & 0x8000) v = -v;
    const int64_t o = j * K + k;
    planes[o] = (int8_t)(v >> 24);
    planes[plane + o] = (int8_t)(((v >> 16) & 255) - 128);
    planes[2 * plane + o] = (int8_t)(((v >> 8) & 255) - 128);
    planes[3 * plane + o] = (int8_t)((v & 255) - 128);
  }
  bound_raise(bad);
  if (threadIdx.x == 0) row_exp[j] = emin - 134;
}

// rowsum(A) for M rows of K int8 (one workgroup per row)
__global__ __launch_bounds__(256) void exact_rowsum_k(const int8_t* __restrict__ A, int K,
                                                      int64_t* __restrict__ rs) {
  __shared__ int64_t red[16];
  const int8_t* a = A + (int64_t)blockIdx.x * K;
  int64_t s = 0;
  for (int k = threadIdx.x; k < K; k += 256) s += a[k];
  s = block_sum(s, red);
  if (threadIdx.x == 0) rs[blockIdx.x] = s;
}

// acc = 2^16 hi + lo + 2^15 rowsum, then the exact-mode epilogue: the real
// output is acc * m_r * 2^(row_exp[j] - k_r)
__global__ __launch_bounds__(256) void exact_combine_k(const int64_t* __restrict__ hi,
                                                       const int64_t* __restrict__ lo,
                                                       const int64_t* __restrict__ rs, int M, int N,
                                                       const int32_t* __restrict__ row_m,
                                                       const int32_t* __restrict__ row_k,
                                                       const int32_t* __restrict__ row_exp,
                                                       int32_t frac, int mode, void* out) {
  const int j = blockIdx.x * 256 + threadIdx.x;  // column; rows i = y, y + gridDim.y, ...
  if (j >= N) return;
  uint32_t bad = 0;
  for (int i = blockIdx.y; i < M; i += gridDim.y) {
    const int64_t t = (int64_t)i * N + j;
    const int64_t acc = 65536 * hi[t] + lo[t] + 32768 * rs[i];
    if (mode == MODE_RAW) {
      ((int64_t*)out)[t] = acc;
      continue;
    }
    const int s = row_k[i] - row_exp[j] - (mode == MODE_REQ_I8 ? 0 : frac);
    const __int128 p = (__int128)acc * row_m[i];
    int64_t y = 0;
    if (s <= 120) {
      if (s <= -62) bad |= kBoundInt32;
      else y = R128(p, s);
    }
    if (mode == MODE_REQ_I8) {
      ((int8_t*)out)[t] = clamp8(y);
    } else {
      bad |= i32_check(y);
      ((int32_t*)out)[t] = (int32_t)y;
    }
  }
  bound_raise(bad);
}

__global__ void zero_i32_k(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// workgroup rows of the pipelined split-K for a few-tile int8 shape: the
// fewest of 2, 4, 8 that reach 192 workgroups (3/4 of the CUs) with every
// split at least two 128-byte K steps and the partials within part_ints; 1
// when the shape fills the chip or no split fits
int pipe_split_count(int64_t M, int64_t N, int64_t K, int64_t part_ints) {
  const int64_t tiles = ((M + 127) / 128) * ((N + 63) / 64);
  if (tiles >= 192) return 1;
  for (int ks = 2; ks <= 8; ks *= 2)
    if ((K / PBK) % ks == 0 && K / ks >= 2 * PBK && ks * M * N <= part_ints && tiles * ks >= 192)
      return ks;
  for (int ks = 8; ks >= 2; ks /= 2)
    if ((K / PBK) % ks == 0 && K / ks >= 2 * PBK && ks * M * N <= part_ints) return ks;
  return 1;
}

}  // namespace

bool gemm_takes_skinny(int64_t M, int64_t N, int64_t K, bool limbs) {
  const bool off32 = M * K < (int64_t(1) << 31) && N * K < (int64_t(1) << 31);
  return M > 16 && off32 && K % SK_KQ == 0 && (M <= 32 || (M <= 64 && !limbs));
}

DETINT_BOUND_READER(bound_flags_gemm)

hipError_t launch_gemm(const int8_t* A, const int8_t* W, const int8_t* W_lo, int64_t M,
                       int64_t N, int64_t K, const Epi& e, void* out, hipStream_t st,
                       const SplitWs* sp) {
  if (M == 0 || N == 0) return hipSuccess;
  if (e.mode == MODE_SWIGLU && (!gemm_takes_skinny(M, N, K, W_lo != nullptr) || N % 32 != 0))
    return hipErrorInvalidValue;
  if (M <= 8 && K >= 16 && !W_lo && !e.out_row_base && fused_decode_supported(M, K) &&
      N * K < (int64_t(1) << 31) && ((uintptr_t)A & 3) == 0)
    return launch_fgemv_i8(A, W, M, N, K, e.row_m, e.row_k, e.col_m, e.col_k, e.frac, e.mode, out,
                           st, e.res_bits);
  if (M <= 16) return gemv_dispatch(A, W, W_lo, M, N, K, e, out, nullptr, st);
  // buffer offsets are 32-bit
  const bool off32 = M * K < (int64_t(1) << 31) && N * K < (int64_t(1) << 31);
  if (off32 && K % SK_KQ == 0 && (M <= 32 || (M <= 64 && !W_lo))) {
    if (W_lo) return skinny_launch<true, 1>(A, W, W_lo, (int)M, (int)N, (int)K, e, out, sp, st);
    if (M <= 32) return skinny_launch<false, 1>(A, W, W_lo, (int)M, (int)N, (int)K, e, out, sp, st);
    return skinny_launch<false, 2>(A, W, W_lo, (int)M, (int)N, (int)K, e, out, sp, st);
  }
  if (K % PBK == 0 && off32) {
    if (!W_lo && sp && sp->part_ints > 0) {
      const int ks = pipe_split_count(M, N, K, sp->part_ints);
      if (ks > 1) return pipe_splitk(A, W, (int)M, (int)N, (int)K, ks, e, out, sp->part, st);
    }
    if (W_lo) return pipe_dispatch<true>(A, W, W_lo, (int)M, (int)N, (int)K, e, out, st);
    return pipe_dispatch<false>(A, W, W_lo, (int)M, (int)N, (int)K, e, out, st);
  }
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

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  zero_i32_k<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n);
  return hipGetLastError();
}

// Split-K pays for a standalone call only on long K: measured on MI355X
// (REQ_I8), 512 x 1024 rows x columns: K = 2048 11.2 -> 14.0 us (a loss),
// K = 4096 17.1 -> 15.8, K = 8192 29.5 -> 17.8; 256 x 1024 x 16384 52.7 ->
// 18.3 us; skinny 32 x 1024 x 8192 17.5 -> 13.1 us but 64 x 1024 x 3072
// 12.3 -> 13.4. So a workspace is asked for only from K = 4096 up.
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, bool limbs) {
  if (M <= 0 || N <= 0 || K < 4096) return 0;
  int64_t b = 0;
  if (gemm_takes_skinny(M, N, K, limbs)) {
    b = 4 * ((N + 31) / 32) + 256 + 4 * kSplitPairsStandalone * kSplitTileInts;
  } else if (!limbs && K % PBK == 0 && ((M + 127) / 128) * ((N + 63) / 64) < 192) {
    b = 4 * 8 * M * N + 256 + 4 * ((N + 31) / 32);
  }
  return b;
}

hipError_t launch_exact_prepare(const uint16_t* W, int64_t N, int64_t K, int8_t* planes,
                                int32_t* row_exp, hipStream_t st) {
  if (N == 0) return hipSuccess;
  exact_prepare_k<<<(unsigned)N, 256, 0, st>>>(W, (int)K, planes, N * K, row_exp);
  return hipGetLastError();
}

hipError_t launch_gemm_exact(const int8_t* A, const int8_t* planes, const int32_t* row_exp,
                             int64_t M, int64_t N, int64_t K, const int32_t* row_m,
                             const int32_t* row_k, int32_t frac, int32_t mode, void* out,
                             int64_t* ws, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  int64_t* hi = ws;
  int64_t* lo = ws + M * N;
  int64_t* rs = ws + 2 * M * N;
  const int64_t plane = N * K;
  const Epi raw{nullptr, nullptr, nullptr, 0, 0, MODE_RAW, nullptr};
  hipError_t e = launch_gemm(A, planes, planes + plane, M, N, K, raw, hi, st);
  if (e == hipSuccess) e = launch_gemm(A, planes + 2 * plane, planes + 3 * plane, M, N, K, raw, lo, st);
  if (e != hipSuccess) return e;
  exact_rowsum_k<<<(unsigned)M, 256, 0, st>>>(A, (int)K, rs);
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)(M < 65535 ? M : 65535));
  exact_combine_k<<<grid, 256, 0, st>>>(hi, lo, rs, (int)M, (int)N, row_m, row_k, row_exp, frac,
                                        mode, out);
  return hipGetLastError();
}

hipError_t launch_split_w16(const int16_t* W16, int64_t n, int8_t* hi, int8_t* lo,
                            hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  split_w16<<<(unsigned)blocks, 256, 0, st>>>(W16, n, hi, lo);
  return hipGetLastError();
}

}  // namespace detint
