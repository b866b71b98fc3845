// Measurement of a device-wide barrier between 256 resident workgroups (one
// per CU). It decides whether a decode step can run as one persistent kernel
// with a barrier between phases instead of one graph node per phase: the
// barrier has to cost less than a node plus the kernel ramp it replaces.
// Not part of the forward pass.
//
// Each round every workgroup writes a 64-int row into one of two row buffers
// (the round's parity), arrives, waits for all 256 arrivals, then reads
// another workgroup's row of the same round and checks it. Arrival and wait:
//   0  per-workgroup generation flags: release store, wave 0 polls all 256
//      flags with relaxed loads (four per lane), then an acquire fence;
//   1  one arrival counter: release RMW, poll, acquire fence;
//   2  two levels: the 8 leaders (workgroups 0..7) each wait for the flags
//      of workgroups g, g + 8, ... (the same XCD under round-robin
//      placement), acquire, and publish a group flag with a release store;
//      everyone waits for the 8 group flags;
//   3  flags as in 0 with relaxed stores after the row stores have
//      completed and no fences: a lower bound on the hardware's latency,
//      not a barrier the memory model guarantees.
// Every wait gives up after a bounded number of polls: it records the
// failure and its workgroup returns, so all waves exit either way.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace detint {
namespace {

constexpr int PB_WG = 256, PB_T = 256, PB_ROW = 64, PB_POLLS = 1 << 16;

__device__ uint32_t pb_flags[PB_WG];
__device__ uint32_t pb_group[8];
__device__ uint32_t pb_count;
__device__ int32_t pb_rows[2][PB_WG][PB_ROW];
__device__ uint32_t pb_err;

__global__ void probe_clear_k() {
  const int t = threadIdx.x;
  if (t < PB_WG) pb_flags[t] = 0;
  if (t < 8) pb_group[t] = 0;
  if (t == 0) {
    pb_count = 0;
    pb_err = 0;
  }
}

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// wave-wide wait until n words at p[0], p[s], ... (n <= 256, a multiple of
// 64 or below it) are all >= want; false when the poll budget ran out
__device__ bool wait_words(const uint32_t* p, int n, int s, uint32_t want, int lane) {
  for (int polls = 0; polls < PB_POLLS; ++polls) {
    uint32_t lo = 0xFFFFFFFFu;
    for (int i = lane; i < n; i += 64) {
      const uint32_t f = ld_relaxed(p + i * s);
      lo = f < lo ? f : lo;
    }
    if (__all(lo >= want)) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

template <int MODE>
__global__ __launch_bounds__(PB_T) void probe_barrier_k(int rounds) {
  __shared__ int s_quit;
  const int tid = threadIdx.x, lane = tid & 63, wg = blockIdx.x;
  if (tid == 0) s_quit = 0;
  __syncthreads();
  for (int r = 1; r <= rounds; ++r) {
    int32_t* row = pb_rows[r & 1][wg];
    if (tid < PB_ROW) {
      const int32_t v = r * 1000 + wg;
      if (MODE == 3)
        __hip_atomic_store(row + tid, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        row[tid] = v;
    }
    __syncthreads();
    if (tid < 64) {
      bool ok;
      const uint32_t want = (uint32_t)r;
      if (MODE == 0 || MODE == 2) {
        if (tid == 0) __hip_atomic_store(&pb_flags[wg], want, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        if (MODE == 0) {
          ok = wait_words(pb_flags, PB_WG, 1, want, lane);
        } else {
          ok = true;
          if (wg < 8) {
            ok = wait_words(pb_flags + wg, PB_WG / 8, 8, want, lane);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            if (tid == 0) __hip_atomic_store(&pb_group[wg], want, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
          }
          ok = ok && wait_words(pb_group, 8, 1, want, lane);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      } else if (MODE == 1) {
        if (tid == 0) __hip_atomic_fetch_add(&pb_count, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        ok = false;
        for (int polls = 0; polls < PB_POLLS && !ok; ++polls) {
          ok = ld_relaxed(&pb_count) >= want * PB_WG;
          if (!ok) __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (tid == 0) __hip_atomic_store(&pb_flags[wg], want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = wait_words(pb_flags, PB_WG, 1, want, lane);
      }
      if (!ok && lane == 0) {
        atomicOr(&pb_err, 1u);
        s_quit = 1;
      }
    }
    __syncthreads();
    if (s_quit) return;
    if (tid < PB_ROW) {
      const int src = (wg + 1 + r) % PB_WG;
      const int32_t* srow = pb_rows[r & 1][src] + tid;
      const int32_t v = MODE == 3 ? __hip_atomic_load(srow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *srow;
      if (v != r * 1000 + src) atomicOr(&pb_err, 2u);
    }
  }
}

}  // namespace

hipError_t launch_probe_barrier(int mode, int rounds, uint32_t* result, hipStream_t st) {
  probe_clear_k<<<1, PB_WG, 0, st>>>();
  switch (mode) {
    case 0: probe_barrier_k<0><<<PB_WG, PB_T, 0, st>>>(rounds); break;
    case 1: probe_barrier_k<1><<<PB_WG, PB_T, 0, st>>>(rounds); break;
    case 2: probe_barrier_k<2><<<PB_WG, PB_T, 0, st>>>(rounds); break;
    default: probe_barrier_k<3><<<PB_WG, PB_T, 0, st>>>(rounds); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !result) return e;
  e = hipMemcpyFromSymbolAsync(result, HIP_SYMBOL(pb_err), 4, 0, hipMemcpyDeviceToHost, st);
  return e != hipSuccess ? e : hipStreamSynchronize(st);
}

}  // namespace detint
