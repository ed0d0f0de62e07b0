// Device helpers shared by the nanospec kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nanospec.h"

#define NS_WAVE 64

// Ends a batch of independent loads: the compiler may not sink a load of the
// batch below this point (into the block that uses it) nor let the machine
// scheduler interleave the batch with later work, so all of the batch's
// requests are in flight before the first wait.
#define NS_ISSUE_FENCE()                   \
  do {                                     \
    asm volatile("" ::: "memory");         \
    __builtin_amdgcn_sched_barrier(0);     \
  } while (0)

namespace ns {

// ---------------------------------------------------------------------------
// Ordered 64-bit keys: (orderable float32 bits) << 32 | (0xFFFFFFFF - id).
// Larger key = larger value, and for equal values the smaller id.  +0.0 and
// -0.0 map to the same orderable bits.  Key 0 is "empty": it is below every
// key made from a non-NaN value (those have a high word >= 0x007FFFFF).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ord_f32(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t make_key(float v, int32_t id) {
  return ((uint64_t)ord_f32(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ int32_t key_id(uint64_t k) {
  return (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}

__device__ __forceinline__ float key_val(uint64_t k) { return unord_f32((uint32_t)(k >> 32)); }

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
// IEEE binary16 halves of a 32-bit pair, widened exactly to float32.
__device__ __forceinline__ float fp16_lo(uint32_t pair) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(pair & 0xFFFFu));
}
__device__ __forceinline__ float fp16_hi(uint32_t pair) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(pair >> 16));
}

// ---------------------------------------------------------------------------
// Wave-level helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = __shfl_xor((unsigned int)(v & 0xFFFFFFFFull), mask, NS_WAVE);
  uint32_t hi = __shfl_xor((unsigned int)(v >> 32), mask, NS_WAVE);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Running maximum over the 16 lanes of each DPP row (row_shr 1, 2, 4, 8 with
// 0 shifted in, 0 being the empty key): lane 15 of a row ends with the
// row's maximum.
__device__ __forceinline__ uint64_t row16_max_u64(uint64_t v) {
#define NS_ROW_MAX_STEP(CTRL)                                                                              \
  {                                                                                                       \
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);  \
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, \
                                                              false);                                     \
    const uint64_t o = ((uint64_t)hi << 32) | lo;                                                         \
    v = o > v ? o : v;                                                                                    \
  }
  NS_ROW_MAX_STEP(0x111)
  NS_ROW_MAX_STEP(0x112)
  NS_ROW_MAX_STEP(0x114)
  NS_ROW_MAX_STEP(0x118)
#undef NS_ROW_MAX_STEP
  return v;
}

// Maximum over all 64 lanes (every lane must be active): running maxima
// within each 16-lane DPP row, then the four row results read as scalars.
__device__ __forceinline__ float wave_max_f32(float v) {
  const int ninf = __float_as_int(-INFINITY);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x111, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x112, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x114, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x118, 0xf, 0xf, false)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, NS_WAVE);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP lane moves
// (row_shr 1/2/4/8 within each row of 16 lanes, then row_bcast 15 and 31
// carry row totals forward); lanes whose DPP source is out of range add 0.
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64,
// NT <= 64*64).  `sh` is LDS scratch of at least NT/64 + 1 ints.  Returns the
// thread's exclusive prefix; *total receives the block sum.  Contains two
// __syncthreads and must be reached by every thread of the block.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  constexpr int NW = NT / NS_WAVE;
  const int tid = threadIdx.x, lane = tid & (NS_WAVE - 1), w = tid / NS_WAVE;
  int inc = wave_incl_scan(v, lane);
  if (lane == NS_WAVE - 1) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    int t = lane < NW ? sh[lane] : 0;
    int ti = wave_incl_scan(t, lane);
    if (lane < NW) sh[lane] = ti - t;          // exclusive wave offsets
    if (lane == NW - 1) sh[NW] = ti;           // block total
  }
  __syncthreads();
  int r = sh[w] + inc - v;
  *total = sh[NW];
  return r;
}

// ---------------------------------------------------------------------------
// Per-thread sorted (descending) candidate lists of CAP keys, and a block
// merge that pops the k largest keys across all threads' lists.
// ---------------------------------------------------------------------------
template <int CAP>
__device__ __forceinline__ void list_insert(uint64_t (&lst)[CAP], uint64_t key) {
  // Precondition: key > lst[CAP-1].  Shifts smaller entries down by one.
#pragma unroll
  for (int i = CAP - 1; i > 0; --i) {
    uint64_t prev = lst[i - 1];
    uint64_t cur = lst[i];
    lst[i] = key > prev ? prev : (key > cur ? key : cur);
  }
  lst[0] = key > lst[0] ? key : lst[0];
}

template <int CAP>
__device__ __forceinline__ void list_pop(uint64_t (&lst)[CAP]) {
#pragma unroll
  for (int i = 0; i < CAP - 1; ++i) lst[i] = lst[i + 1];
  lst[CAP - 1] = 0;
}

// Pops the k largest keys over all threads of a block of NT threads, in
// descending order, handing each to emit(r, key) on thread 0.  Keys must be
// unique among non-empty entries (ids are distinct).  `sh` is LDS scratch of
// NT/64 uint64.  Every thread of the block must call it.
template <int NT, int CAP, typename Emit>
__device__ __forceinline__ void block_pop_topk(uint64_t (&lst)[CAP], int k, uint64_t* sh, Emit emit) {
  constexpr int NW = NT / NS_WAVE;
  const int tid = threadIdx.x, lane = tid & (NS_WAVE - 1), w = tid / NS_WAVE;
  for (int r = 0; r < k; ++r) {
    uint64_t best = wave_max_u64(lst[0]);
    if (lane == 0) sh[w] = best;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) { uint64_t o = sh[i]; best = o > best ? o : best; }
    __syncthreads();
    if (best != 0 && lst[0] == best) list_pop(lst);
    if (tid == 0) emit(r, best);
  }
}

// Pops the k largest keys over the lists of the 64 lanes of one wave (no
// barriers).  Lane r (r < k) returns the r-th key (0 if there are fewer than
// r+1 non-empty keys).  If several lanes hold the same key at their heads,
// only the lowest such lane pops it.
template <int CAP>
__device__ __forceinline__ uint64_t wave_pop_topk(uint64_t (&lst)[CAP], int k, int lane) {
  uint64_t mine = 0;
  for (int r = 0; r < k; ++r) {
    const uint64_t best = wave_max_u64(lst[0]);
    const unsigned long long ball = __ballot(best != 0 && lst[0] == best);
    const int owner = ball ? (__ffsll((unsigned long long)ball) - 1) : -1;
    if (lane == owner) list_pop(lst);
    if (lane == r) mine = best;
  }
  return mine;
}

}  // namespace ns

// Launch-error helper for host code.
static inline int ns_launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NS_OK : NS_EHIP;
}
