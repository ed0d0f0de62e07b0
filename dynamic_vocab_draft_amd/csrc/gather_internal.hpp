// Launcher of the row copy kernel shared by the plain gather and the
// slot-stable packed buffer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ns {

// Enqueues out[dst ? dst[j] : j, :] = w[ids[j], :] for j < n, where n is
// *n_dev (n_max when n_dev is NULL) clamped to [0, n_max].  Rows are dvec
// 16-byte vectors long; ids outside [0, V) and destinations outside
// [0, n_max) are skipped.  One wave copies one row at a time; the grid is one
// wave per row up to max_blocks blocks (0: no cap), striding over the rest.
// Returns an NS_* code.
int launch_row_copy(const void* w, int V, int dvec, const int32_t* ids, const int32_t* dst,
                    const int32_t* n_dev, int n_max, void* out, hipStream_t stream, int max_blocks = 0);

}  // namespace ns
