// Device pointers and sizes of one window state (passed to kernels by value).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Words of next_bm: the bitmap's ceil(V/32), rounded up to 8 so that a
// thread may read any aligned run of 4 or 8 words that starts inside it.
__host__ __device__ inline int next_words(int V) { return (((V + 31) >> 5) + 7) & ~7; }

struct ns_state_view {
  int64_t* len;       // |S|, the total number of stream entries appended
  uint32_t* status;   // sticky NS_STATUS_* bits
  int32_t* ring;      // [w_max] tail of S
  int32_t* first;     // [V] first-position table (INT32_MAX between calls)
  uint32_t* bitmap;   // [ceil(V/32)] active set of the latest rebuild
  int32_t* cur;       // [w_max] the active set in ascending order, kept by the decode-step call
  int32_t* n_cur;     // its size
  uint32_t* next_bm;  // [ceil(V/32) rounded up to 8 words] the decode step's bitmap of I_{t+1}, between its launches
  int V;
  int w_max;
};

// The opaque host handle behind nanospec_state*.  `mode` is the stream-source
// setting of nanospec_state_set_mode (NS_STREAM_*), applied on the host.
struct nanospec_state {
  ns_state_view view;
  int mode = 0;
  // True while cur / n_cur hold the window's active set: set by
  // nanospec_decode_step, cleared by every other call that changes the
  // window or rebuilds the set without them.
  bool cur_valid = false;
  // A decode step between nanospec_decode_step_project and _select: its
  // form (0 none, 1 three launches, 2 fused) and what select must match.
  struct Pending {
    int form = 0;
    bool keep = false;   // the shapes allow the two-launch form: keep I_{t+1} in cur
    int nt = 0, d = 0, dtype = 0, M = 0, k = 0;
    const void* ws = nullptr;
    const int32_t* ids = nullptr;
    const int32_t* n = nullptr;
  } pending;
  // Every call that changes the window or rebuilds I outside a decode step.
  void drop_cur() {
    cur_valid = false;
    pending.form = 0;
  }
};

// B states laid out back to back at a fixed stride; members[b] is the
// ordinary handle of sequence b.
struct nanospec_batch {
  int B;
  size_t stride;
  nanospec_state* members;
};
