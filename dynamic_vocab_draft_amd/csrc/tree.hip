// Best-k selection over draft-tree candidates.
//
// NanoSpec, Sec. 4.1: the draft tree has depth 5 and at most 60 draft tokens.
// Each depth's draft head (nanospec_draft_logprob_topk) scores the top K
// children of every frontier node as parent score + log-probability over the
// active set; the next frontier is the best F of those children, and the
// final tree the best N of all nodes generated.  Both selections are this
// kernel: one 1024-thread block per sequence ranks up to 4096 (score, flat
// index) candidates with the draft head's block top-k (one 64-bit key orders
// by score descending, then flat index ascending) and writes the winners'
// flat indices, scores and token ids.
#include "common.hpp"
#include "select.hpp"

namespace {

template <int U>
__global__ __launch_bounds__(kSelectThreads) void k_tree_select(const float* __restrict__ vals,
                                                                const int32_t* __restrict__ ids, int C, int k,
                                                                int32_t* __restrict__ out_idx,
                                                                float* __restrict__ out_vals,
                                                                int32_t* __restrict__ out_ids) {
  __shared__ SelectSmem sm;
  const size_t b = blockIdx.x;
  vals += b * C;
  ids += b * C;
  out_idx += b * k;
  out_vals += b * k;
  out_ids += b * k;
  const int tid = threadIdx.x;
  float lv[U];
  int li[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = tid + u * kSelectThreads;
    const int jc = j < C ? j : C - 1;
    lv[u] = vals[jc];
    li[u] = ids[jc];
  }
  NS_ISSUE_FENCE();
  float v[U];
  int g[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = tid + u * kSelectThreads;
    const bool live = j < C && li[u] >= 0;            // id -1: an empty slot
    v[u] = live ? lv[u] : 0.f;
    g[u] = live ? j : -1;
  }
  block_select_topk<U>(v, g, k, C, sm, [&](int r, uint64_t x) {
    const int idx = x ? ns::key_id(x) : -1;
    out_idx[r] = idx;
    out_vals[r] = x ? ns::key_val(x) : -INFINITY;
    out_ids[r] = x ? ids[idx] : -1;
  });
}

}  // namespace

extern "C" int nanospec_tree_select(const float* vals, const int32_t* ids, int32_t C, int32_t B, int32_t k,
                                    int32_t* out_idx, float* out_vals, int32_t* out_ids, hipStream_t stream) {
  if (!vals || !ids || !out_idx || !out_vals || !out_ids) return NS_EINVAL;
  if (C < 1 || C > NS_MAX_TREE_CAND || B < 1 || B > NS_MAX_BATCH || k < 1 || k > NS_MAX_K) return NS_EINVAL;
  (void)hipGetLastError();
  const dim3 grid(B), block(kSelectThreads);
  if (C <= kSelectThreads)
    hipLaunchKernelGGL(k_tree_select<1>, grid, block, 0, stream, vals, ids, C, k, out_idx, out_vals, out_ids);
  else if (C <= 2 * kSelectThreads)
    hipLaunchKernelGGL(k_tree_select<2>, grid, block, 0, stream, vals, ids, C, k, out_idx, out_vals, out_ids);
  else
    hipLaunchKernelGGL(k_tree_select<4>, grid, block, 0, stream, vals, ids, C, k, out_idx, out_vals, out_ids);
  return ns_launch_status();
}
