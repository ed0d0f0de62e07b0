// Window state of the candidate stream: append (with in-tuple first-occurrence
// dedup), the sliding-window active set as an LDS-built bitmap with ascending
// compaction, and the fused per-step update.
//
// MicroSpec/NanoSpec (arXiv 2605.26444) Sec. 3.2: S_init and S_new are
// concatenations of tuples, and I_{t+1} = Unique(Suffix(S_new, W_max)).
// NanoSpec "Eliminating Overhead via GPU-Resident State Management": the state
// stays on the GPU as a bitmap and is updated by device kernels only.
//
// Device layout of a state (caller-owned, 256-byte aligned):
//   [0, 256)            control: int64 len (|S|), uint32 status, int32 n_cur
//   ring   int32[w_max] S entry p lives at ring[p % w_max] while p >= |S|-w_max
//   first  int32[V]     per-id first position inside the current append
//                       (INT32_MAX between calls)
//   bitmap uint32[ceil(V/32)]  the active set of the latest rebuild
//   cur    int32[w_max] the active set in ascending order (n_cur of them),
//                       as left by the latest nanospec_decode_step
//   next   uint32[ceil(V/32) rounded up to 8]  the bitmap of I_{t+1}, passed
//                       between the two launches of a decode step (words
//                       past ceil(V/32) stay zero)
//
// All state kernels run as ONE workgroup of 1024 threads: the per-step work
// is a few thousand ids and words, so a single CU finishes it in a few
// microseconds, and a single workgroup needs no grid-wide synchronisation
// between the dedup, scan, write and rebuild phases.  Only integer atomics
// (atomicMin, atomicOr) are used, so results do not depend on scheduling.
#include <new>

#include "common.hpp"
#include "state_internal.hpp"
#include "state_fast.hpp"

namespace {

constexpr int kStateThreads = 1024;
constexpr int kNW = kStateThreads / NS_WAVE;

struct StateDev {
  int64_t* len;
  uint32_t* status;
  int32_t* ring;
  int32_t* first;
  uint32_t* bitmap;
  int V;
  int w_max;
};

__device__ __forceinline__ int load_first(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Appends ids[0..n) to the stream (Sec. 3.2 tuple concatenation).  `len` is
// the block-uniform stream length, updated in place.  Returns through *bad
// whether any id was outside [0, V).  Must be called by all threads.
__device__ void block_append(const StateDev& s, const int32_t* __restrict__ ids, int n,
                             bool dedup, int64_t& len, int* sh_scan, int* sh_flag) {
  const int tid = threadIdx.x;
  if (n <= 0) return;
  // Phase 1: first position of each id inside this tuple.
  if (dedup) {
    for (int i = tid; i < n; i += kStateThreads) {
      int id = ids[i];
      if (id >= 0 && id < s.V) atomicMin(&s.first[id], i);
    }
  }
  __syncthreads();
  // Phase 2: number of entries this tuple contributes.
  int c = 0;
  bool bad = false;
  for (int i = tid; i < n; i += kStateThreads) {
    int id = ids[i];
    bool valid = id >= 0 && id < s.V;
    bad |= !valid;
    c += valid && (!dedup || load_first(&s.first[id]) == i);
  }
  if (bad) *sh_flag = 1;
  int total = 0;
  (void)ns::block_excl_scan<kStateThreads>(c, sh_scan, &total);
  const int C = total;
  // Phase 3: ordered positions; only the last w_max kept entries can still
  // be inside the window, so only those are written (no slot collisions).
  int base = 0;
  for (int c0 = 0; c0 < n; c0 += kStateThreads) {
    int i = c0 + tid;
    int id = i < n ? ids[i] : -1;
    bool keep = i < n && id >= 0 && id < s.V && (!dedup || load_first(&s.first[id]) == i);
    int chunk_total = 0;
    int pos = ns::block_excl_scan<kStateThreads>(keep ? 1 : 0, sh_scan, &chunk_total);
    if (keep) {
      int p = base + pos;
      if (p >= C - s.w_max) {
        int64_t q = len + (int64_t)p;
        s.ring[(int)(q % (int64_t)s.w_max)] = id;
      }
    }
    base += chunk_total;
  }
  __syncthreads();
  // Phase 4: restore the first-position table for the next call.
  if (dedup) {
    for (int i = tid; i < n; i += kStateThreads) {
      int id = ids[i];
      if (id >= 0 && id < s.V)
        __hip_atomic_store(&s.first[id], INT32_MAX, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  len += (int64_t)C;
  __syncthreads();
}

// Rebuilds I = Unique(Suffix(S, W_max)) from the ring: bits set in an LDS
// bitmap, then a popcount prefix scan over the words emits ids in ascending
// order.  Must be called by all threads.
__device__ void block_active(const StateDev& s, int64_t len, uint32_t* lds_bm, int32_t* __restrict__ active_ids,
                             int32_t* __restrict__ n_active, uint32_t* __restrict__ bitmap_out, int* sh_scan) {
  const int tid = threadIdx.x;
  const int words = (s.V + 31) >> 5;
  for (int w = tid; w < words; w += kStateThreads) lds_bm[w] = 0u;
  __syncthreads();
  const int cnt = (int)(len < (int64_t)s.w_max ? len : (int64_t)s.w_max);
  // While |S| < w_max the entries sit in ring[0..|S|); afterwards every slot
  // holds one of the last w_max entries.
  for (int e = tid; e < cnt; e += kStateThreads) {
    int id = s.ring[e];
    if (id >= 0 && id < s.V) atomicOr(&lds_bm[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  const int per = (words + kStateThreads - 1) / kStateThreads;
  const int w0 = tid * per;
  const int w1 = min(words, w0 + per);
  int pc = 0;
  for (int w = w0; w < w1; ++w) pc += __popc(lds_bm[w]);
  int total = 0;
  int off = ns::block_excl_scan<kStateThreads>(pc, sh_scan, &total);
  for (int w = w0; w < w1; ++w) {
    uint32_t b = lds_bm[w];
    s.bitmap[w] = b;
    if (bitmap_out) bitmap_out[w] = b;
    while (b) {
      int bit = __ffs(b) - 1;
      active_ids[off++] = (w << 5) + bit;
      b &= b - 1u;
    }
  }
  if (tid == 0) *n_active = total;
}

__device__ __forceinline__ StateDev state_dev(const ns_state_view& v) {
  StateDev s;
  s.len = v.len;
  s.status = v.status;
  s.ring = v.ring;
  s.first = v.first;
  s.bitmap = v.bitmap;
  s.V = v.V;
  s.w_max = v.w_max;
  return s;
}

__device__ __forceinline__ void finish(const StateDev& s, int64_t len, int flag) {
  if (threadIdx.x == 0) {
    *s.len = len;
    if (flag) atomicOr(s.status, NS_STATUS_BAD_ID);
  }
}

__global__ __launch_bounds__(kStateThreads) void k_append(ns_state_view v, const int32_t* __restrict__ ids,
                                                          int n, int dedup) {
  __shared__ int sh_scan[kNW + 1];
  __shared__ int sh_flag;
  __shared__ int64_t sh_len;
  StateDev s = state_dev(v);
  if (threadIdx.x == 0) { sh_flag = 0; sh_len = *s.len; }
  __syncthreads();
  int64_t len = sh_len;
  block_append(s, ids, n, dedup != 0, len, sh_scan, &sh_flag);
  finish(s, len, sh_flag);
}

__global__ __launch_bounds__(kStateThreads) void k_active(ns_state_view v, int32_t* __restrict__ active_ids,
                                                          int32_t* __restrict__ n_active,
                                                          uint32_t* __restrict__ bitmap_out) {
  extern __shared__ uint32_t lds_bm[];
  __shared__ int sh_scan[kNW + 1];
  StateDev s = state_dev(v);
  int64_t len = *s.len;
  block_active(s, len, lds_bm, active_ids, n_active, bitmap_out, sh_scan);
}

__global__ __launch_bounds__(kStateThreads) void k_step(ns_state_view v, const int32_t* __restrict__ draft_ids,
                                                        int n_draft, const int32_t* __restrict__ ver_ids, int n_ver,
                                                        int32_t* __restrict__ active_ids, int32_t* __restrict__ n_active,
                                                        uint32_t* __restrict__ bitmap_out) {
  extern __shared__ uint32_t lds_bm[];
  __shared__ int sh_scan[kNW + 1];
  __shared__ int sh_flag;
  __shared__ int64_t sh_len;
  StateDev s = state_dev(v);
  if (threadIdx.x == 0) { sh_flag = 0; sh_len = *s.len; }
  __syncthreads();
  int64_t len = sh_len;
  block_append(s, draft_ids, n_draft, true, len, sh_scan, &sh_flag);
  block_append(s, ver_ids, n_ver, false, len, sh_scan, &sh_flag);
  block_active(s, len, lds_bm, active_ids, n_active, bitmap_out, sh_scan);
  finish(s, len, sh_flag);
}

template <typename T, int RU>
__global__ __launch_bounds__(kFastThreads) void k_step_fast(ns_state_view v, const int32_t* draft_ids,
                                                            int n_draft, const int32_t* ver_ids, int n_ver,
                                                            int32_t* __restrict__ active_ids,
                                                            int32_t* __restrict__ n_active,
                                                            uint32_t* __restrict__ bitmap_out) {
  extern __shared__ int4 lds4[];
  step_fast_body<T, RU, kFastThreads, 0>(lds4, fast_stage_ints(v.V, v.w_max), v, draft_ids, n_draft, ver_ids, n_ver,
                                         active_ids, n_active, bitmap_out, FuseCtl{});
}

// B sequences, one workgroup each: sequence b's state is sequence 0's moved
// by b * stride bytes; its tuples start at b * {draft,ver}_stride and hold
// n_draft[b] / n_ver[b] ids (device counts, clamped to [0, nd_max] /
// [0, nv_max]); its outputs are the b-th W_max / 1 / ceil(V/32) blocks.
template <typename T, int RU>
__global__ __launch_bounds__(kFastThreads) void k_step_fast_batch(ns_state_view v0, size_t stride,
                                                                  const int32_t* draft_ids, int draft_stride,
                                                                  const int32_t* n_draft, int nd_max,
                                                                  const int32_t* ver_ids, int ver_stride,
                                                                  const int32_t* n_ver, int nv_max,
                                                                  int32_t* __restrict__ active_ids,
                                                                  int32_t* __restrict__ n_active,
                                                                  uint32_t* __restrict__ bitmap_out) {
  const int b = blockIdx.x;
  const size_t off = (size_t)b * stride;
  ns_state_view v = v0;
  v.len = (int64_t*)((char*)v0.len + off);
  v.status = (uint32_t*)((char*)v0.status + off);
  v.ring = (int32_t*)((char*)v0.ring + off);
  v.first = (int32_t*)((char*)v0.first + off);
  v.bitmap = (uint32_t*)((char*)v0.bitmap + off);
  v.cur = (int32_t*)((char*)v0.cur + off);
  v.n_cur = (int32_t*)((char*)v0.n_cur + off);
  v.next_bm = (uint32_t*)((char*)v0.next_bm + off);
  const int nd = min(max(n_draft[b], 0), nd_max);
  const int nv = min(max(n_ver[b], 0), nv_max);
  const int words = (v0.V + 31) >> 5;
  extern __shared__ int4 lds4[];
  step_fast_body<T, RU, kFastThreads, 0>(lds4, fast_stage_ints(v0.V, v0.w_max), v, draft_ids + (size_t)b * draft_stride,
                                         nd, ver_ids + (size_t)b * ver_stride, nv, active_ids + (size_t)b * v0.w_max,
                                         n_active + b, bitmap_out ? bitmap_out + (size_t)b * words : nullptr,
                                         FuseCtl{});
}

size_t fast_lds_bytes(int V, int w_max, int n_draft) {
  return ((size_t)kFastThreads * fast_wpt(V) + (size_t)fast_stage_ints(V, w_max) +
          2 * (size_t)((n_draft + NS_WAVE - 1) & ~(NS_WAVE - 1))) * 4;
}

typedef void (*step_fast_fn)(ns_state_view, const int32_t*, int, const int32_t*, int, int32_t*, int32_t*, uint32_t*);

// Kernel instance holding ring entries of a w_max-slot ring in registers.
typedef void (*step_fast_batch_fn)(ns_state_view, size_t, const int32_t*, int, const int32_t*, int, const int32_t*,
                                   int, const int32_t*, int, int32_t*, int32_t*, uint32_t*);

step_fast_batch_fn pick_step_fast_batch(int w_max) {
  if (w_max > kFastMaxRing) return nullptr;
  if ((w_max & 3) == 0) {
    const int per = (w_max / 4 + kFastThreads - 1) / kFastThreads;
    if (per <= 1) return k_step_fast_batch<int4, 1>;
    if (per <= 2) return k_step_fast_batch<int4, 2>;
    if (per <= 4) return k_step_fast_batch<int4, 4>;
    return k_step_fast_batch<int4, 8>;
  }
  const int per = (w_max + kFastThreads - 1) / kFastThreads;
  if (per <= 1) return k_step_fast_batch<int, 1>;
  if (per <= 2) return k_step_fast_batch<int, 2>;
  if (per <= 4) return k_step_fast_batch<int, 4>;
  if (per <= 8) return k_step_fast_batch<int, 8>;
  if (per <= 16) return k_step_fast_batch<int, 16>;
  return k_step_fast_batch<int, 32>;
}

step_fast_fn pick_step_fast(int w_max) {
  if (w_max > kFastMaxRing) return nullptr;
  if ((w_max & 3) == 0) {
    const int per = (w_max / 4 + kFastThreads - 1) / kFastThreads;
    if (per <= 1) return k_step_fast<int4, 1>;
    if (per <= 2) return k_step_fast<int4, 2>;
    if (per <= 4) return k_step_fast<int4, 4>;
    return k_step_fast<int4, 8>;
  }
  const int per = (w_max + kFastThreads - 1) / kFastThreads;
  if (per <= 1) return k_step_fast<int, 1>;
  if (per <= 2) return k_step_fast<int, 2>;
  if (per <= 4) return k_step_fast<int, 4>;
  if (per <= 8) return k_step_fast<int, 8>;
  if (per <= 16) return k_step_fast<int, 16>;
  return k_step_fast<int, 32>;
}

// Initialisation / reset: empty stream, cleared status, first[] = INT32_MAX,
// empty bitmap.  A grid-stride fill kernel (no memset nodes, so the call can
// be captured in a graph).
__global__ void k_init(ns_state_view v) {
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  const int gs = gridDim.x * blockDim.x;
  if (gt == 0) { *v.len = 0; *v.status = 0u; *v.n_cur = 0; }
  for (int i = gt; i < v.w_max; i += gs) v.ring[i] = -1;
  for (int i = gt; i < v.V; i += gs) v.first[i] = INT32_MAX;
  const int words = (v.V + 31) >> 5;
  for (int i = gt; i < words; i += gs) v.bitmap[i] = 0u;
  for (int i = gt; i < next_words(v.V); i += gs) v.next_bm[i] = 0u;
}

__global__ void k_window(ns_state_view v, int32_t* __restrict__ window, int64_t* __restrict__ len_out) {
  const int64_t len = *v.len;
  const int cnt = (int)(len < (int64_t)v.w_max ? len : (int64_t)v.w_max);
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  const int gs = gridDim.x * blockDim.x;
  if (window) {
    for (int e = gt; e < v.w_max; e += gs) {
      int val = -1;
      if (e < cnt) {
        int64_t p = len - cnt + e;
        val = v.ring[(int)(p % (int64_t)v.w_max)];
      }
      window[e] = val;
    }
  }
  if (len_out && gt == 0) *len_out = len;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool state_dims_ok(int32_t V, int32_t w_max) {
  return V >= 1 && V <= NS_MAX_V && w_max >= 1 && w_max <= NS_MAX_WMAX;
}

size_t lds_bitmap_bytes(int V) { return (size_t)((V + 31) >> 5) * sizeof(uint32_t); }

int set_lds_limit(const void* fn, size_t bytes) {
  if (bytes <= 65536) return NS_OK;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess
             ? NS_OK : NS_EHIP;
}

int fill_grid(const ns_state_view& v) {
  int n = v.V > v.w_max ? v.V : v.w_max;
  int g = (n + 255) / 256;
  return g < 1 ? 1 : (g > 1024 ? 1024 : g);
}

}  // namespace

extern "C" {

const char* nanospec_strerror(int code) {
  switch (code) {
    case NS_OK: return "ok";
    case NS_EINVAL: return "invalid argument (null pointer, bad size or limit exceeded)";
    case NS_EDTYPE: return "unknown dtype or mode";
    case NS_ECAPACITY: return "buffer too small";
    case NS_EHIP: return "HIP launch or runtime error";
    case NS_ESCRATCH: return "request larger than the fixed scratch of the allocation-free draft head";
    default: return "unknown error code";
  }
}

int nanospec_version(void) { return 100; }

size_t nanospec_state_bytes(int32_t V, int32_t w_max) {
  if (!state_dims_ok(V, w_max)) return 0;
  size_t b = 256;
  b += align256((size_t)w_max * 4);
  b += align256((size_t)V * 4);
  b += align256((size_t)((V + 31) >> 5) * 4);
  b += align256((size_t)w_max * 4);
  b += align256((size_t)next_words(V) * 4);
  return b;
}

}  // extern "C"

namespace {

// Device pointers of a state laid out at p (256-byte aligned).
ns_state_view make_view(char* p, int32_t V, int32_t w_max) {
  ns_state_view v;
  v.len = (int64_t*)p;
  v.status = (uint32_t*)(p + 8);
  size_t off = 256;
  v.ring = (int32_t*)(p + off);
  off += align256((size_t)w_max * 4);
  v.first = (int32_t*)(p + off);
  off += align256((size_t)V * 4);
  v.bitmap = (uint32_t*)(p + off);
  off += align256((size_t)((V + 31) >> 5) * 4);
  v.cur = (int32_t*)(p + off);
  off += align256((size_t)w_max * 4);
  v.next_bm = (uint32_t*)(p + off);
  v.n_cur = (int32_t*)(p + 16);
  v.V = V;
  v.w_max = w_max;
  return v;
}

// Sets the dynamic-LDS limits of the state kernels that a state of this
// W_max launches.  The limits are the largest any state may ask for (the
// bitmap of NS_MAX_V ids, kFastLdsMax), not this state's own needs: the
// attribute belongs to the kernel, so a state created later with a smaller V
// must not lower it below what an earlier state still launches with.
int prepare_kernels(int32_t /*V*/, int32_t w_max) {
  int rc = set_lds_limit((const void*)k_active, lds_bitmap_bytes(NS_MAX_V));
  if (rc == NS_OK) rc = set_lds_limit((const void*)k_step, lds_bitmap_bytes(NS_MAX_V));
  step_fast_fn fast_fn = pick_step_fast(w_max);
  if (rc == NS_OK && fast_fn) rc = set_lds_limit((const void*)fast_fn, kFastLdsMax);
  step_fast_batch_fn batch_fn = pick_step_fast_batch(w_max);
  if (rc == NS_OK && batch_fn) rc = set_lds_limit((const void*)batch_fn, kFastLdsMax);
  return rc;
}

}  // namespace

extern "C" {

int nanospec_state_create(nanospec_state** out, int32_t V, int32_t w_max, void* dev_mem, size_t dev_bytes,
                          hipStream_t stream) {
  if (!out || !dev_mem || !state_dims_ok(V, w_max)) return NS_EINVAL;
  if (((uintptr_t)dev_mem & 255u) != 0) return NS_EINVAL;
  size_t need = nanospec_state_bytes(V, w_max);
  if (dev_bytes < need) return NS_ECAPACITY;
  int rc = prepare_kernels(V, w_max);
  if (rc != NS_OK) return rc;
  nanospec_state* st = new (std::nothrow) nanospec_state;
  if (!st) return NS_EINVAL;
  st->view = make_view((char*)dev_mem, V, w_max);
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_init, dim3(fill_grid(st->view)), dim3(256), 0, stream, st->view);
  rc = ns_launch_status();
  if (rc != NS_OK) { delete st; return rc; }
  *out = st;
  return NS_OK;
}

// ---- batches of independent sequences ------------------------------------

size_t nanospec_batch_state_bytes(int32_t B, int32_t V, int32_t w_max) {
  if (B < 1 || B > NS_MAX_BATCH) return 0;
  const size_t one = nanospec_state_bytes(V, w_max);
  return one * (size_t)B;
}

int nanospec_batch_create(nanospec_batch** out, int32_t B, int32_t V, int32_t w_max, void* dev_mem,
                          size_t dev_bytes, hipStream_t stream) {
  if (!out || !dev_mem || B < 1 || B > NS_MAX_BATCH || !state_dims_ok(V, w_max)) return NS_EINVAL;
  if (((uintptr_t)dev_mem & 255u) != 0) return NS_EINVAL;
  if (dev_bytes < nanospec_batch_state_bytes(B, V, w_max)) return NS_ECAPACITY;
  int rc = prepare_kernels(V, w_max);
  if (rc != NS_OK) return rc;
  nanospec_batch* bt = new (std::nothrow) nanospec_batch;
  if (!bt) return NS_EINVAL;
  bt->members = new (std::nothrow) nanospec_state[B];
  if (!bt->members) { delete bt; return NS_EINVAL; }
  bt->B = B;
  bt->stride = nanospec_state_bytes(V, w_max);
  (void)hipGetLastError();
  for (int b = 0; b < B; ++b) {
    bt->members[b].view = make_view((char*)dev_mem + (size_t)b * bt->stride, V, w_max);
    hipLaunchKernelGGL(k_init, dim3(fill_grid(bt->members[b].view)), dim3(256), 0, stream, bt->members[b].view);
  }
  rc = ns_launch_status();
  if (rc != NS_OK) { delete[] bt->members; delete bt; return rc; }
  *out = bt;
  return NS_OK;
}

int nanospec_batch_destroy(nanospec_batch* bt) {
  if (!bt) return NS_EINVAL;
  delete[] bt->members;
  delete bt;
  return NS_OK;
}

int nanospec_batch_member(nanospec_batch* bt, int32_t b, nanospec_state** out) {
  if (!bt || !out || b < 0 || b >= bt->B) return NS_EINVAL;
  *out = &bt->members[b];
  return NS_OK;
}

int nanospec_batch_step_update(nanospec_batch* bt, const int32_t* draft_ids, int32_t draft_stride,
                               const int32_t* n_draft, int32_t nd_max, const int32_t* ver_ids, int32_t ver_stride,
                               const int32_t* n_ver, int32_t nv_max, int32_t* active_ids, int32_t* n_active,
                               uint32_t* bitmap, hipStream_t stream) {
  if (!bt || !draft_ids || !ver_ids || !n_draft || !n_ver || !active_ids || !n_active) return NS_EINVAL;
  if (nd_max < 0 || nv_max < 0 || nd_max > kFastMaxIds || nv_max > kFastMaxIds) return NS_EINVAL;
  if (draft_stride < nd_max || ver_stride < nv_max) return NS_EINVAL;
  for (int b = 0; b < bt->B; ++b)                     // the batched kernel appends for every member
    if (bt->members[b].mode == NS_STREAM_CTX_ONLY) return NS_EINVAL;
  for (int b = 0; b < bt->B; ++b) bt->members[b].drop_cur();
  const ns_state_view& v0 = bt->members[0].view;
  step_fast_batch_fn fn = pick_step_fast_batch(v0.w_max);
  const size_t lds = fast_lds_bytes(v0.V, v0.w_max, nd_max);
  if (!fn || lds > kFastLdsMax) return NS_EINVAL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(fn, dim3(bt->B), dim3(kFastThreads), lds, stream, v0, bt->stride, draft_ids, draft_stride, n_draft,
                     nd_max, ver_ids, ver_stride, n_ver, nv_max, active_ids, n_active, bitmap);
  return ns_launch_status();
}

int nanospec_state_reset(nanospec_state* st, hipStream_t stream) {
  if (!st) return NS_EINVAL;
  st->drop_cur();
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_init, dim3(fill_grid(st->view)), dim3(256), 0, stream, st->view);
  return ns_launch_status();
}

int nanospec_state_set_mode(nanospec_state* st, int32_t mode) {
  if (!st) return NS_EINVAL;
  if (mode != NS_STREAM_FULL && mode != NS_STREAM_CTX_ONLY && mode != NS_STREAM_EXT_ONLY) return NS_EINVAL;
  st->mode = mode;
  return NS_OK;
}

int nanospec_state_destroy(nanospec_state* st) {
  if (!st) return NS_EINVAL;
  delete st;
  return NS_OK;
}

int nanospec_state_status(nanospec_state* st, uint32_t* flags, hipStream_t stream) {
  if (!st || !flags) return NS_EINVAL;
  uint32_t h = 0;
  const uint32_t zero = 0;
  if (hipMemcpyAsync(&h, st->view.status, 4, hipMemcpyDeviceToHost, stream) != hipSuccess) return NS_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return NS_EHIP;
  if (hipMemcpyAsync(st->view.status, &zero, 4, hipMemcpyHostToDevice, stream) != hipSuccess) return NS_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return NS_EHIP;
  *flags = h;
  return NS_OK;
}

int nanospec_state_window(nanospec_state* st, int32_t* window, int64_t* len, hipStream_t stream) {
  if (!st) return NS_EINVAL;
  if (!window && !len) return NS_OK;
  (void)hipGetLastError();
  int g = (st->view.w_max + 255) / 256;
  hipLaunchKernelGGL(k_window, dim3(g > 1024 ? 1024 : g), dim3(256), 0, stream, st->view, window, len);
  return ns_launch_status();
}

int nanospec_stream_append(nanospec_state* st, const int32_t* ids, int32_t n, int32_t dedup_first,
                           hipStream_t stream) {
  if (!st || n < 0 || (n > 0 && !ids)) return NS_EINVAL;
  if (dedup_first != 0 && dedup_first != 1) return NS_EINVAL;
  if (n == 0 || st->mode == NS_STREAM_EXT_ONLY) return NS_OK;   // ext-only: no prompt context
  st->drop_cur();
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_append, dim3(1), dim3(kStateThreads), 0, stream, st->view, ids, n, dedup_first);
  return ns_launch_status();
}

int nanospec_active_vocab(nanospec_state* st, int32_t* active_ids, int32_t* n_active, uint32_t* bitmap,
                          hipStream_t stream) {
  if (!st || !active_ids || !n_active) return NS_EINVAL;
  st->drop_cur();
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_active, dim3(1), dim3(kStateThreads), lds_bitmap_bytes(st->view.V), stream, st->view,
                     active_ids, n_active, bitmap);
  return ns_launch_status();
}

int nanospec_step_update(nanospec_state* st, const int32_t* draft_ids, int32_t n_draft, const int32_t* ver_ids,
                         int32_t n_ver, int32_t* active_ids, int32_t* n_active, uint32_t* bitmap,
                         hipStream_t stream) {
  if (!st || !active_ids || !n_active || n_draft < 0 || n_ver < 0) return NS_EINVAL;
  if ((n_draft > 0 && !draft_ids) || (n_ver > 0 && !ver_ids)) return NS_EINVAL;
  if (st->mode == NS_STREAM_CTX_ONLY) n_draft = n_ver = 0;     // ctx-only: nothing added while decoding
  st->drop_cur();
  (void)hipGetLastError();
  const size_t fast = fast_lds_bytes(st->view.V, st->view.w_max, n_draft);
  step_fast_fn fast_fn = pick_step_fast(st->view.w_max);
  if (fast_fn && n_draft <= kFastMaxIds && n_ver <= kFastMaxIds && fast <= kFastLdsMax) {
    // The kernel reads element 0 of an empty tuple unconditionally.
    const int32_t* dptr = n_draft > 0 ? draft_ids : st->view.ring;
    const int32_t* vptr = n_ver > 0 ? ver_ids : st->view.ring;
    hipLaunchKernelGGL(fast_fn, dim3(1), dim3(kFastThreads), fast, stream, st->view, dptr, n_draft, vptr, n_ver,
                       active_ids, n_active, bitmap);
  } else {
    hipLaunchKernelGGL(k_step, dim3(1), dim3(kStateThreads), lds_bitmap_bytes(st->view.V), stream, st->view,
                       draft_ids, n_draft, ver_ids, n_ver, active_ids, n_active, bitmap);
  }
  return ns_launch_status();
}

}  // extern "C"
