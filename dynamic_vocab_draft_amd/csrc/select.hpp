// Block-wide top-k selection over (value, id) pairs held by a 1024-thread
// block, used by the draft-head merges.
#pragma once
#include "common.hpp"

namespace {

// ---------------------------------------------------------------------------
// Keys are (ordered f32 bits << 32) | ~id, so one 64-bit compare orders by
// (value desc, id asc); 0 is the empty key.
//
// block_select_topk: the k largest (value, id) pairs held by a 1024-thread
// block (U per thread; id < 0 marks an empty slot), by the key order.
// T = the k-th largest of the 16 wave maxima (k <= 16) or of the 64 maxima of
// 16-lane DPP rows (float values, counted with multiplicity).  Each of those
// is a real value, so the k-th largest value overall is >= T and the top k
// are among the pairs with value >= T.  Only those are turned into 64-bit
// keys, collected in LDS and ranked by counting; if more than kCandCap reach
// T, the block falls back to k rounds of block-wide maxima.
// `nlive` (block-uniform) bounds the live slots, which lead: slot u of
// thread t is index t + u * 1024.  The maxima only give a threshold when at
// least k of them are live, so wave maxima are used when more than 64 (k - 1)
// slots may be live, row maxima when more than 16 (k - 1), and otherwise
// every live pair (at most 16 k) is ranked.  emit(r, key) is called once for
// every rank r < k (key 0 when fewer than r + 1 pairs exist).  mid() is
// called by every thread between the first two barriers, while wave 0 looks
// for the threshold (work placed there by waves 1..15 is free; its LDS
// writes are visible to every emit).
// ---------------------------------------------------------------------------
constexpr int kSelectThreads = 1024;
constexpr int kCandCap = 1024;

struct SelectSmem {
  float rmax[NS_WAVE];                             // (1024 / 64 waves) x (4 rows of 16 lanes)
  uint64_t cand[kCandCap];
  uint64_t red[kSelectThreads / NS_WAVE];
  float T;
  int cnt;
};

struct NoMid {
  __device__ void operator()() const {}
};

template <int U, typename Emit, typename Mid = NoMid>
__device__ __forceinline__ void block_select_topk(const float (&val)[U], const int (&id)[U], int k, int nlive,
                                                  SelectSmem& sm, Emit emit, Mid mid = Mid()) {
  static_assert(kSelectThreads / NS_WAVE * 4 == NS_WAVE, "one row maximum per lane of a wave");
  const int tid = threadIdx.x, lane = tid & (NS_WAVE - 1);
  const int ninf = __float_as_int(-INFINITY);
  float best = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (id[u] >= 0) best = fmaxf(best, val[u]);
  best = fmaxf(best, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(best), 0x111, 0xf, 0xf, false)));
  best = fmaxf(best, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(best), 0x112, 0xf, 0xf, false)));
  best = fmaxf(best, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(best), 0x114, 0xf, 0xf, false)));
  best = fmaxf(best, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(best), 0x118, 0xf, 0xf, false)));
  constexpr int NW = kSelectThreads / NS_WAVE;
  // Wave maxima when k <= NW and at least k waves can hold a live pair (fewer
  // compares for wave 0); else row maxima when at least k rows can; else no
  // threshold (T = -inf, all live pairs ranked).
  const bool by_wave = k <= NW && nlive > NS_WAVE * (k - 1);
  const bool by_row = !by_wave && nlive > 16 * (k - 1);
  if (by_wave) {
    const float w0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), 15));
    const float w1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), 31));
    const float w2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), 47));
    const float w3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), 63));
    if (lane == 0) sm.rmax[tid / NS_WAVE] = fmaxf(fmaxf(w0, w1), fmaxf(w2, w3));
  } else if ((lane & 15) == 15) {
    sm.rmax[(tid / NS_WAVE) * 4 + (lane >> 4)] = best;
  }
  if (tid == 0) sm.cnt = 0;
  __syncthreads();
  // Wave 0 finds T: the maximum x with #{> x} < k <= #{>= x}.
  if (tid < NS_WAVE) {
    const int nv = by_wave ? NW : NS_WAVE;
    const float mine = lane < nv ? sm.rmax[lane] : -INFINITY;
    int gt = 0, ge = 0;
    if (by_wave) {
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const float o = sm.rmax[q];
        gt += o > mine;
        ge += o >= mine;
      }
    } else {
#pragma unroll 16
      for (int q = 0; q < NS_WAVE; ++q) {
        const float o = sm.rmax[q];
        gt += o > mine;
        ge += o >= mine;
      }
    }
    const unsigned long long ball = __ballot(mine != -INFINITY && gt < k && ge >= k);
    if (lane == 0) sm.T = (ball && (by_wave || by_row)) ? sm.rmax[__ffsll(ball) - 1] : -INFINITY;
  }
  mid();
  __syncthreads();
  const float T = sm.T;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (id[u] >= 0 && val[u] >= T) {
      const int slot = atomicAdd(&sm.cnt, 1);
      if (slot < kCandCap) sm.cand[slot] = ns::make_key(val[u], id[u]);
    }
  }
  __syncthreads();
  const int C = sm.cnt;
  if (C <= kCandCap) {
    for (int q = tid; q < C; q += kSelectThreads) {
      const uint64_t x = sm.cand[q];
      int r = 0;
#pragma unroll 8
      for (int p = 0; p < C; ++p) r += sm.cand[p] > x;
      if (r < k) emit(r, x);
    }
    for (int r = C + tid; r < k; r += kSelectThreads) emit(r, (uint64_t)0);
  } else {                                         // block-uniform: too many pairs at T
    uint64_t lst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) lst[u] = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (id[u] >= 0) ns::list_insert(lst, ns::make_key(val[u], id[u]));
    ns::block_pop_topk<kSelectThreads, U>(lst, k, sm.red, emit);
  }
}

}  // namespace
