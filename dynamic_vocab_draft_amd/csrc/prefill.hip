// Prefill candidates: P[i] = T_Kpre(z_i) for every prompt position i.
//
// MicroSpec/NanoSpec (arXiv 2605.26444) Sec. 3.2 "Candidate Stream
// Initialization": the stream starts as the prompt followed by the union of
// each position's top-K_pre logits.  The pass reads L x V logits once, so it
// is HBM-bound.  One wave owns one row and streams it with 16-byte loads, in
// batches of four per lane that alternate between two register sets; a block
// holds the waves of four adjacent rows (measured faster than one-wave
// blocks and than several waves sharing a row).  Each lane scans its
// elements in ascending id order and keeps a sorted list of its CAP best
// (value, id) keys; an element that only ties the list's last value has a
// larger id and is dropped.  After every batch the wave shares the
// largest k-th best value held by any lane as a floor (the row's k-th largest
// cannot be below it), so most vectors cost a conversion and one compare of
// their 8-element maximum.  A pop over the wave's lanes (no block barrier)
// then emits the k winners ordered by (value desc, id asc).  Values are the
// stored logits widened to float32, so the result is exact.
#include "common.hpp"

namespace {

constexpr int kPrefillThreads = NS_WAVE;  // lanes per row: one wave per row, all rows resident at once
constexpr int kPrefillRows = 4;           // rows (waves) per block
constexpr int kPrefillUnroll = 4;

template <int CAP>
struct Cands {
  uint64_t lst[CAP];
  float thr;     // value of lst[CAP-1] once the list is full
  float floor;   // lower bound on the row's k-th largest value (shared by the wave)
  int filled;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < CAP; ++i) lst[i] = 0;
    thr = -INFINITY;
    floor = -INFINITY;
    filled = 0;
  }
  // A value below `floor` has k larger values in the row; a value that only
  // ties the full list's last one loses to it on id (ids ascend in the scan).
  __device__ __forceinline__ bool wants(float v) const { return v >= floor && (filled < CAP || v > thr); }
  __device__ __forceinline__ void add(float v, int id) {
    if (!wants(v)) return;
    ns::list_insert(lst, ns::make_key(v, id));
    ++filled;
    if (filled >= CAP) thr = ns::key_val(lst[CAP - 1]);
  }
  // Value of this thread's k-th best so far (-inf if it holds fewer).
  __device__ __forceinline__ float kth(int k) const {
    float r = -INFINITY;
#pragma unroll
    for (int i = 0; i < CAP; ++i)
      if (i == k - 1 && lst[i] != 0) r = ns::key_val(lst[i]);
    return r;
  }
};

// Element types are the NS_* dtype codes: NS_BF16 and NS_FP16 (2 bytes,
// 8 per 16-byte vector) and NS_FP32 (4 bytes, 4 per vector).
__host__ __device__ constexpr int elem_bytes(int ET) { return ET == NS_FP32 ? 4 : 2; }

// Element e of a 32-bit word pair (e = 0: low half) widened to float32.
template <int ET>
__device__ __forceinline__ float half_elem(uint32_t w, int e) {
  if (ET == NS_BF16) return e ? ns::bf16_hi(w) : ns::bf16_lo(w);
  return e ? ns::fp16_hi(w) : ns::fp16_lo(w);
}

// Scans one batch of 16-byte vectors (vector q0 + u * threads for u < U);
// vectors past the row were loaded clamped and are skipped.
template <int ET, int CAP>
__device__ __forceinline__ void scan_batch(const uint4 (&x)[kPrefillUnroll], int q0, int nvec, Cands<CAP>& c) {
  constexpr int EPV = 16 / elem_bytes(ET);
#pragma unroll
  for (int u = 0; u < kPrefillUnroll; ++u) {
    const int q = q0 + u * kPrefillThreads;
    if (q >= nvec) continue;
    const uint32_t wv[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
    float v[EPV];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (ET != NS_FP32) {
        v[2 * e] = half_elem<ET>(wv[e], 0);
        v[2 * e + 1] = half_elem<ET>(wv[e], 1);
      } else {
        v[e] = __uint_as_float(wv[e]);
      }
    }
    float mx = v[0];
#pragma unroll
    for (int e = 1; e < EPV; ++e) mx = fmaxf(mx, v[e]);
    if (c.wants(mx)) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) c.add(v[e], q * EPV + e);
    }
  }
}

template <int ET, bool VEC, int CAP>
__global__ __launch_bounds__(kPrefillThreads * kPrefillRows) void k_prefill(const void* __restrict__ Z, int L, int V,
                                                                            int k, int32_t* __restrict__ out_ids,
                                                                            float* __restrict__ out_vals) {
  const size_t row = (size_t)blockIdx.x * kPrefillRows + threadIdx.x / NS_WAVE;
  const int tid = threadIdx.x & (NS_WAVE - 1);
  if (row >= (size_t)L) return;                        // wave-uniform; no barrier below
  Cands<CAP> c;
  c.init();
  if (VEC) {
    constexpr int EPV = 16 / elem_bytes(ET);   // elements per 16-byte vector
    constexpr int STEP = kPrefillThreads * kPrefillUnroll;
    const int nvec = V / EPV;
    const uint4* __restrict__ p = (const uint4*)((const char*)Z + row * (size_t)V * elem_bytes(ET));
    // Two register batches, a and b, alternate so that the loads of one are
    // in flight while the other is scanned.  Indices are clamped into the row,
    // so every load is in bounds.  The loop trip count is the same for all
    // threads: after each batch the wave raises every thread's floor to the
    // largest k-th best held by any of its lanes, which turns most vectors
    // into a single compare and keeps the lanes from diverging into inserts.
    // The logits are read once: loads carry the non-temporal policy (the
    // `nt` bit), measured 202 -> 186 us on 4096 x 128256 bf16 logits.
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const auto ld = [&](int q) -> uint4 {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)p + q);
      return make_uint4(v.x, v.y, v.z, v.w);
    };
    uint4 a[kPrefillUnroll], b[kPrefillUnroll];
#pragma unroll
    for (int u = 0; u < kPrefillUnroll; ++u) {
      const int q = tid + u * kPrefillThreads;
      a[u] = ld(q < nvec ? q : 0);
    }
    for (int base = 0; base < nvec; base += 2 * STEP) {
#pragma unroll
      for (int u = 0; u < kPrefillUnroll; ++u) {
        const int q = base + STEP + tid + u * kPrefillThreads;
        b[u] = ld(q < nvec ? q : 0);
      }
      NS_ISSUE_FENCE();
      scan_batch<ET, CAP>(a, base + tid, nvec, c);
      c.floor = fmaxf(c.floor, ns::wave_max_f32(c.kth(k)));
      if (base + STEP >= nvec) break;                   // uniform
#pragma unroll
      for (int u = 0; u < kPrefillUnroll; ++u) {
        const int q = base + 2 * STEP + tid + u * kPrefillThreads;
        a[u] = ld(q < nvec ? q : 0);
      }
      NS_ISSUE_FENCE();
      scan_batch<ET, CAP>(b, base + STEP + tid, nvec, c);
      c.floor = fmaxf(c.floor, ns::wave_max_f32(c.kth(k)));
    }
  } else {
    if (ET != NS_FP32) {
      const uint16_t* __restrict__ p = (const uint16_t*)Z + row * (size_t)V;
      for (int e = tid; e < V; e += kPrefillThreads) c.add(half_elem<ET>((uint32_t)p[e], 0), e);
    } else {
      const float* __restrict__ p = (const float*)Z + row * (size_t)V;
      for (int e = tid; e < V; e += kPrefillThreads) c.add(p[e], e);
    }
  }
  const uint64_t key = ns::wave_pop_topk<CAP>(c.lst, k, tid);   // lane r < k holds the r-th winner
  if (tid < k) {
    out_ids[row * k + tid] = key ? ns::key_id(key) : -1;
    out_vals[row * k + tid] = key ? ns::key_val(key) : -INFINITY;
  }
}

template <int ET, bool VEC>
void launch_cap(int cap, const void* Z, int L, int V, int k, int32_t* ids, float* vals, hipStream_t s) {
#define NS_LAUNCH_PREFILL(C)                                                                                  \
  hipLaunchKernelGGL((k_prefill<ET, VEC, C>), dim3((unsigned)(((int64_t)L + kPrefillRows - 1) / kPrefillRows)), \
                     dim3(kPrefillThreads * kPrefillRows), 0, s, Z, L, V, k, ids, vals)
  switch (cap) {
    case 4: NS_LAUNCH_PREFILL(4); break;
    case 8: NS_LAUNCH_PREFILL(8); break;
    case 16: NS_LAUNCH_PREFILL(16); break;
    case 32: NS_LAUNCH_PREFILL(32); break;
    default: NS_LAUNCH_PREFILL(64); break;
  }
#undef NS_LAUNCH_PREFILL
}

}  // namespace

extern "C" int nanospec_prefill_topk(const void* logits, int32_t L, int32_t V, int32_t dtype, int32_t k,
                                     int32_t* out_ids, float* out_vals, hipStream_t stream) {
  if (dtype != NS_BF16 && dtype != NS_FP32 && dtype != NS_FP16) return NS_EDTYPE;
  if (L < 0 || V < 1 || k < 1 || k > NS_MAX_K || k > V) return NS_EINVAL;
  if (L == 0) return NS_OK;
  if (!logits || !out_ids || !out_vals) return NS_EINVAL;
  const int esz = elem_bytes(dtype);
  const bool vec = (((uintptr_t)logits) & 15u) == 0 && (((size_t)V * esz) % 16) == 0;
  const int cap = k <= 4 ? 4 : k <= 8 ? 8 : k <= 16 ? 16 : k <= 32 ? 32 : 64;
  (void)hipGetLastError();
  if (dtype == NS_BF16) {
    if (vec) launch_cap<NS_BF16, true>(cap, logits, L, V, k, out_ids, out_vals, stream);
    else launch_cap<NS_BF16, false>(cap, logits, L, V, k, out_ids, out_vals, stream);
  } else if (dtype == NS_FP16) {
    if (vec) launch_cap<NS_FP16, true>(cap, logits, L, V, k, out_ids, out_vals, stream);
    else launch_cap<NS_FP16, false>(cap, logits, L, V, k, out_ids, out_vals, stream);
  } else {
    if (vec) launch_cap<NS_FP32, true>(cap, logits, L, V, k, out_ids, out_vals, stream);
    else launch_cap<NS_FP32, false>(cap, logits, L, V, k, out_ids, out_vals, stream);
  }
  return ns_launch_status();
}
