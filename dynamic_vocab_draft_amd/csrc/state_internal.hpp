// Device pointers and sizes of one window state (passed to kernels by value).
#pragma once
#include <stdint.h>

struct ns_state_view {
  int64_t* len;       // |S|, the total number of stream entries appended
  uint32_t* status;   // sticky NS_STATUS_* bits
  int32_t* ring;      // [w_max] tail of S
  int32_t* first;     // [V] first-position table (INT32_MAX between calls)
  uint32_t* bitmap;   // [ceil(V/32)] active set of the latest rebuild
  int V;
  int w_max;
};

// The opaque host handle behind nanospec_state*.  `mode` is the stream-source
// setting of nanospec_state_set_mode (NS_STREAM_*), applied on the host.
struct nanospec_state {
  ns_state_view view;
  int mode = 0;
};

// B states laid out back to back at a fixed stride; members[b] is the
// ordinary handle of sequence b.
struct nanospec_batch {
  int B;
  size_t stride;
  nanospec_state* members;
};
