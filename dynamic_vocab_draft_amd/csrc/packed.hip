// Slot-stable packed buffer of active rows.
//
// NanoSpec, Sec. 3.3 "Avoiding Sparse Computation via Asynchronous
// Gathering": a buffer of W_max rows is allocated once, and at each step only
// the rows of tokens that became active are gathered into it, so the head can
// run as a dense product over the buffer.  The pages leave the placement open;
// here a row keeps its slot while its id stays active, the slots of ids that
// left become holes (id -1), and the entering ids, in ascending id order, fill
// the free slots in ascending slot order.  The head then reads slots
// [0, n_slots), n_slots being one past the highest occupied slot, and skips
// holes.  Taking the lowest free slots keeps every occupied slot below the
// largest active-set size seen so far, so n_slots stays close to |I|.
//
// One update is two launches:
//   k_pack_plan  one workgroup: entering ids = active bitmap & ~held bitmap;
//                slots whose id is no longer active become free; one scan
//                ranks both (entering ids ascending, free slots ascending) and
//                pairs the r-th free slot with the r-th entering id; the slot
//                map, the held bitmap, the gather list and n_slots are written.
//   row copy     rows[enter_slot[r], :] = W_head[enter_id[r], :], one wave
//                per row, for the n_enter rows only.
#include <new>

#include "common.hpp"
#include "gather_internal.hpp"
#include "state_internal.hpp"

struct nanospec_packed {
  int V;
  int cap;                 // slots
  int32_t* hdr;            // [0] n_slots, [1] n_enter
  int32_t* slot_ids;       // [cap] id held in each slot, -1 for a hole
  uint32_t* held;          // [ceil(V/32)] ids held, LSB-first
  int32_t* enter_slot;     // [cap] this update's gather list: slots ...
  int32_t* enter_id;       // [cap] ... and the ids copied into them
};

namespace {

constexpr int kPlanThreads = 1024;
// The row copy of an update runs on a small grid that strides over the
// entering rows (a few dozen per step in steady decoding).
constexpr int kCopyBlocks = 64;

struct packed_view {
  int V, cap;
  int32_t* hdr;
  int32_t* slot_ids;
  uint32_t* held;
  int32_t* enter_slot;
  int32_t* enter_id;
};

packed_view view_of(const nanospec_packed* pk) {
  return packed_view{pk->V, pk->cap, pk->hdr, pk->slot_ids, pk->held, pk->enter_slot, pk->enter_id};
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool packed_dims_ok(int32_t V, int32_t cap) {
  return V >= 1 && V <= NS_MAX_V && cap >= 1 && cap <= NS_MAX_SLOTS;
}

// Every slot a hole, nothing held, both counts zero.
__global__ __launch_bounds__(256) void k_pack_init(packed_view p) {
  const int nw = (p.V + 31) >> 5;
  const int stride = gridDim.x * blockDim.x;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < p.cap || i < nw; i += stride) {
    if (i < p.cap) p.slot_ids[i] = -1;
    if (i < nw) p.held[i] = 0u;
  }
  if (blockIdx.x == 0 && threadIdx.x < 2) p.hdr[threadIdx.x] = 0;
}

// Bits of bitmap word w that can hold ids below V (nw words, `last` = the
// valid bits of word nw - 1).
__device__ __forceinline__ uint32_t word_mask(int w, int nw, uint32_t last) {
  return w < nw - 1 ? ~0u : (w == nw - 1 ? last : 0u);
}

// One workgroup plans the update.  All global reads happen in two rounds:
// the thread's run of active/held bitmap words (G 16-byte vectors each) and
// its run of SPT slot ids, then the active word of each slot's id.  Thread t
// owns contiguous runs, so a single block scan over the packed counts
// (entering ids in the low 16 bits, free slots in the high 16) ranks both in
// ascending order.  cap <= 16384 < 2^16 keeps each count in its half.
template <int G, int SPT>
__global__ __launch_bounds__(kPlanThreads) void k_pack_plan(const uint32_t* __restrict__ act, packed_view p) {
  extern __shared__ int32_t ent[];                     // [cap] entering ids, ascending
  __shared__ int sh_scan[kPlanThreads / NS_WAVE + 1];
  __shared__ int sh_top;
  const int tid = threadIdx.x;
  const int nw = (p.V + 31) >> 5;
  const int nv = (nw + 3) >> 2;                        // 16-byte vectors of bitmap words
  const uint4* __restrict__ act4 = (const uint4*)act;
  uint4* __restrict__ held4 = (uint4*)p.held;
  // First load round: bitmap vectors and slot ids (indices clamped, results masked).
  uint4 a[G], h[G];
  int sid[SPT];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int v = min(tid * G + i, nv - 1);
    a[i] = act4[v];
    h[i] = held4[v];
  }
  const int s0 = tid * SPT;
#pragma unroll
  for (int i = 0; i < SPT; ++i) sid[i] = p.slot_ids[min(s0 + i, p.cap - 1)];
  NS_ISSUE_FENCE();
  // A vector may run past the last bitmap word into the allocation's padding,
  // which nobody initialises: words past it, and bits past V, count as zero.
  const uint32_t last = (p.V & 31) ? ((1u << (p.V & 31)) - 1u) : ~0u;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int w0 = (tid * G + i) * 4;
    const uint32_t m0 = word_mask(w0, nw, last), m1 = word_mask(w0 + 1, nw, last);
    const uint32_t m2 = word_mask(w0 + 2, nw, last), m3 = word_mask(w0 + 3, nw, last);
    a[i] = make_uint4(a[i].x & m0, a[i].y & m1, a[i].z & m2, a[i].w & m3);
    h[i] = make_uint4(h[i].x & m0, h[i].y & m1, h[i].z & m2, h[i].w & m3);
  }
  // Second load round: is each slot's id still active?
  uint32_t aw[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int id = sid[i];
    const bool ok = s0 + i < p.cap && id >= 0 && id < p.V;
    aw[i] = act[ok ? (id >> 5) : 0];
  }
  NS_ISSUE_FENCE();
  if (tid == 0) sh_top = 0;
  int n_ent = 0, n_free = 0;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (tid * G + i < nv)
      n_ent += __popc(a[i].x & ~h[i].x) + __popc(a[i].y & ~h[i].y) + __popc(a[i].z & ~h[i].z) +
               __popc(a[i].w & ~h[i].w);
  }
  bool live[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int id = sid[i];
    live[i] = id >= 0 && id < p.V && ((aw[i] >> (id & 31)) & 1u);
    n_free += (s0 + i < p.cap && !live[i]) ? 1 : 0;
  }
  int totals = 0;
  const int offs = ns::block_excl_scan<kPlanThreads>(n_ent | (n_free << 16), sh_scan, &totals);
  const int n_enter = min(totals & 0xFFFF, p.cap);
  const int n_fill = min(n_enter, totals >> 16);
  // Entering ids into LDS in ascending order; the held bitmap becomes the
  // active one.  Bitmap words past V are zero in a valid state.
  int off = offs & 0xFFFF;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int v = tid * G + i;
    if (v < nv) {
      const uint32_t aa[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
      const uint32_t hh[4] = {h[i].x, h[i].y, h[i].z, h[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t e = aa[q] & ~hh[q];
        while (e) {
          const int id = ((v * 4 + q) << 5) | (__ffs(e) - 1);
          if (off < p.cap) ent[off] = id;
          ++off;
          e &= e - 1u;
        }
      }
      held4[v] = a[i];
    }
  }
  __syncthreads();
  // Free slots take the entering ids in rank order.
  int r = offs >> 16;
  int top = 0;                                         // one past the highest occupied slot
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int s = s0 + i;
    if (s < p.cap) {
      if (live[i]) {
        top = s + 1;
      } else {
        if (r < n_fill) {
          const int nid = ent[r];
          p.slot_ids[s] = nid;
          p.enter_slot[r] = s;
          p.enter_id[r] = nid;
          top = s + 1;
        } else if (sid[i] != -1) {
          p.slot_ids[s] = -1;
        }
        ++r;
      }
    }
  }
  const uint64_t wtop = ns::wave_max_u64((uint64_t)top);
  if ((tid & (NS_WAVE - 1)) == 0) atomicMax(&sh_top, (int)wtop);
  __syncthreads();
  if (tid == 0) {
    p.hdr[0] = sh_top;
    p.hdr[1] = n_fill;
  }
}

using plan_fn = void (*)(const uint32_t*, packed_view);

// Smallest instantiation whose per-thread runs cover the bitmap and the slots.
plan_fn pick_plan(int V, int cap) {
  const int nv = (((V + 31) >> 5) + 3) >> 2;
  const bool s4 = cap <= 4 * kPlanThreads;
#define NS_PLAN_CASE(GG)                                                                \
  if (nv <= GG * kPlanThreads) return s4 ? (plan_fn)k_pack_plan<GG, 4> : (plan_fn)k_pack_plan<GG, 16>;
  NS_PLAN_CASE(1)
  NS_PLAN_CASE(2)
  NS_PLAN_CASE(4)
  NS_PLAN_CASE(8)
#undef NS_PLAN_CASE
  return nullptr;
}

}  // namespace

extern "C" {

size_t nanospec_packed_bytes(int32_t V, int32_t w_max) {
  if (!packed_dims_ok(V, w_max)) return 0;
  return 256 + 3 * align256((size_t)w_max * 4) + align256((size_t)((V + 31) >> 5) * 4);
}

int nanospec_packed_reset(nanospec_packed* pk, hipStream_t stream) {
  if (!pk) return NS_EINVAL;
  const int n = pk->cap > pk->V / 32 ? pk->cap : pk->V / 32 + 1;
  int grid = (n + 255) / 256;
  grid = grid < 1 ? 1 : (grid > 1024 ? 1024 : grid);
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_pack_init, dim3(grid), dim3(256), 0, stream, view_of(pk));
  return ns_launch_status();
}

int nanospec_packed_create(nanospec_packed** out, int32_t V, int32_t w_max, void* dev_mem, size_t dev_bytes,
                           hipStream_t stream) {
  if (!out || !dev_mem || !packed_dims_ok(V, w_max)) return NS_EINVAL;
  if (((uintptr_t)dev_mem & 255u) != 0) return NS_EINVAL;
  if (dev_bytes < nanospec_packed_bytes(V, w_max)) return NS_ECAPACITY;
  // The plan keeps the entering ids in LDS (w_max int32 of dynamic LDS).  The
  // limit is a property of the kernel, shared by every slot map, so it is set
  // to what the largest map needs.
  const plan_fn plan = pick_plan(V, w_max);
  if (!plan) return NS_EINVAL;
  if (hipFuncSetAttribute((const void*)plan, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)(NS_MAX_SLOTS * sizeof(int32_t))) != hipSuccess)
    return NS_EHIP;
  nanospec_packed* pk = new (std::nothrow) nanospec_packed;
  if (!pk) return NS_EINVAL;
  char* p = (char*)dev_mem;
  const size_t slots = align256((size_t)w_max * 4);
  pk->V = V;
  pk->cap = w_max;
  pk->hdr = (int32_t*)p;
  pk->slot_ids = (int32_t*)(p + 256);
  pk->enter_slot = (int32_t*)(p + 256 + slots);
  pk->enter_id = (int32_t*)(p + 256 + 2 * slots);
  pk->held = (uint32_t*)(p + 256 + 3 * slots);
  const int rc = nanospec_packed_reset(pk, stream);
  if (rc != NS_OK) {
    delete pk;
    return rc;
  }
  *out = pk;
  return NS_OK;
}

int nanospec_packed_destroy(nanospec_packed* pk) {
  if (!pk) return NS_EINVAL;
  delete pk;
  return NS_OK;
}

int nanospec_packed_slots(const nanospec_packed* pk, const int32_t** slot_ids, const int32_t** n_slots,
                          const int32_t** enter_slots, const int32_t** enter_ids, const int32_t** n_enter) {
  if (!pk) return NS_EINVAL;
  if (slot_ids) *slot_ids = pk->slot_ids;
  if (n_slots) *n_slots = pk->hdr;
  if (enter_slots) *enter_slots = pk->enter_slot;
  if (enter_ids) *enter_ids = pk->enter_id;
  if (n_enter) *n_enter = pk->hdr + 1;
  return NS_OK;
}

int nanospec_packed_update(nanospec_packed* pk, const nanospec_state* st, const void* w, int32_t d,
                           int32_t dtype, void* rows, hipStream_t stream) {
  if (!pk || !st || !w || !rows || d < 8 || d > NS_MAX_D || (d % 8) != 0) return NS_EINVAL;
  if (dtype != NS_BF16 && dtype != NS_FP32 && dtype != NS_FP16) return NS_EDTYPE;
  if ((((uintptr_t)w) & 15u) || (((uintptr_t)rows) & 15u)) return NS_EINVAL;
  if (st->view.V != pk->V || st->view.w_max > pk->cap) return NS_EINVAL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(pick_plan(pk->V, pk->cap), dim3(1), dim3(kPlanThreads), (size_t)pk->cap * sizeof(int32_t),
                     stream, (const uint32_t*)st->view.bitmap, view_of(pk));
  int rc = ns_launch_status();
  if (rc != NS_OK) return rc;
  const int esz = dtype == NS_FP32 ? 4 : 2;
  return ns::launch_row_copy(w, pk->V, d * esz / 16, pk->enter_id, pk->enter_slot, pk->hdr + 1, pk->cap, rows,
                             stream, kCopyBlocks);
}

}  // extern "C"
