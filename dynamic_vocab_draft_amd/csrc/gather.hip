// Row gather into a packed buffer: out[j, :] = W[ids[j], :] for j < n (or,
// for the slot-stable buffer, out[dst[j], :] = W[ids[j], :]).
//
// NanoSpec "Avoiding Sparse Computation via Asynchronous Gathering": the rows
// W_head[I_t, :] are copied into a preallocated contiguous buffer so the LM
// head becomes a dense product.  On MI355X each row is one contiguous run
// (d * elem bytes, 8 KiB for d = 4096 bf16), so the copy is a plain streaming
// copy: one wave per row, every lane moving 16-byte vectors, with all of a
// lane's loads issued before its stores so a whole row is in flight at once.
#include "common.hpp"
#include "gather_internal.hpp"

namespace {

constexpr int kGatherThreads = 256;
constexpr int kRowsPerBlock = kGatherThreads / NS_WAVE;   // one wave per row
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kGatherThreads) void k_gather(const uint4* __restrict__ w, int V, int dvec,
                                                           const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ dst_rows,
                                                           const int32_t* __restrict__ n_dev, int n_max,
                                                           uint4* __restrict__ out) {
  int n = n_dev ? *n_dev : n_max;
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  const int lane = threadIdx.x & (NS_WAVE - 1);
  const int step = gridDim.x * kRowsPerBlock;
  for (int j = blockIdx.x * kRowsPerBlock + (int)(threadIdx.x / NS_WAVE); j < n; j += step) {
    const int id = ids[j];
    const int row = dst_rows ? dst_rows[j] : j;
    if (id < 0 || id >= V || row < 0 || row >= n_max) continue;
    const uint4* __restrict__ src = w + (size_t)id * dvec;
    uint4* __restrict__ dst = out + (size_t)row * dvec;
    // Full batches: kUnroll unguarded 16-byte loads per lane, then the stores.
    int q0 = 0;
    for (; q0 + NS_WAVE * kUnroll <= dvec; q0 += NS_WAVE * kUnroll) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = src[q0 + u * NS_WAVE + lane];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) dst[q0 + u * NS_WAVE + lane] = v[u];
    }
    for (int q = q0 + lane; q < dvec; q += NS_WAVE) dst[q] = src[q];
  }
}

}  // namespace

int ns::launch_row_copy(const void* w, int V, int dvec, const int32_t* ids, const int32_t* dst,
                        const int32_t* n_dev, int n_max, void* out, hipStream_t stream, int max_blocks) {
  int grid = (int)(((int64_t)n_max + kRowsPerBlock - 1) / kRowsPerBlock);
  if (max_blocks > 0 && grid > max_blocks) grid = max_blocks;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_gather, dim3(grid), dim3(kGatherThreads), 0, stream, (const uint4*)w, V, dvec, ids, dst,
                     n_dev, n_max, (uint4*)out);
  return ns_launch_status();
}

extern "C" int nanospec_gather_rows(const void* w, int32_t V, int32_t d, int32_t dtype, const int32_t* ids,
                                    const int32_t* n_dev, int32_t n_max, void* out, hipStream_t stream) {
  if (!w || !ids || !out || V < 1 || n_max < 1 || d < 8 || d > NS_MAX_D || (d % 8) != 0) return NS_EINVAL;
  if (dtype != NS_BF16 && dtype != NS_FP32 && dtype != NS_FP16) return NS_EDTYPE;
  if ((((uintptr_t)w) & 15u) || (((uintptr_t)out) & 15u)) return NS_EINVAL;
  const int esz = dtype == NS_FP32 ? 4 : 2;
  return ns::launch_row_copy(w, V, d * esz / 16, ids, nullptr, n_dev, n_max, out, stream);
}
