// Restricted LM head: logits[m, j] = <h[m, :], row_j> over the active rows,
// then T_k per hidden row with the winners mapped back to global ids.
//
// MicroSpec/NanoSpec (arXiv 2605.26444) Sec. 3.1, Eq. 1 (z = W_head h) on the
// sub-matrix W_head[I_t, :]; T_K from Sec. 3.2.  The pages pack the rows
// first ("Avoiding Sparse Computation via Asynchronous Gathering") and name
// the naive indexed product as the slower alternative (ablation, Table 5).
// Here both forms are one kernel with two address modes: NS_PACKED reads the
// packed buffer, NS_INDEXED reads W_head[row_ids[j]] directly (each row is a
// contiguous 16-byte-aligned run, so an indexed row read is as coalesced as a
// packed one); which is faster is decided by measurement.
//
// Kernels:
//   k_proj_valu : VALU projection.  A block stages MT hidden rows in LDS and
//                 its four waves stream rows of W (one row per wave, 16-byte
//                 vectors, all of a lane's loads in flight together); bf16
//                 pairs use v_dot2_f32_bf16.  Grid-stride over rows, grid.y
//                 over chunks of MT hidden rows.
//   k_proj_mfma : bf16 MFMA projection (v_mfma_f32_16x16x32_bf16), for the
//                 wider M where fp32 VALU work would exceed the HBM time.
//   k_topk_merge: one block per hidden row; per-thread sorted candidate lists
//                 of 64-bit keys (orderable value, inverted global id), then a
//                 block-wide pop of the k largest.
#include "common.hpp"

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kProjThreads = 256;
constexpr int kProjWaves = kProjThreads / NS_WAVE;
constexpr int kProjUnroll = 8;
constexpr int kMergeThreads = 256;
constexpr size_t kHLdsBytes = 65536;   // LDS budget for staged hidden rows

__device__ __forceinline__ float dot16(uint4 w, uint4 h, float acc, bool bf16) {
  if (bf16) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, h.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, h.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, h.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, h.w), acc, false);
  } else {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(h.x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(h.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(h.z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(h.w), acc);
  }
  return acc;
}

__device__ __forceinline__ int clamp_n(const int32_t* n_dev, int n_max) {
  int n = n_dev ? *n_dev : n_max;
  return n < 0 ? 0 : (n > n_max ? n_max : n);
}

template <bool BF16, int MT>
__global__ __launch_bounds__(kProjThreads) void k_proj_valu(const uint4* __restrict__ rows, int mode,
                                                            const int32_t* __restrict__ row_ids,
                                                            const int32_t* __restrict__ n_dev, int n_max, int V,
                                                            int dvec, const uint4* __restrict__ h, int M,
                                                            float* __restrict__ logits) {
  extern __shared__ uint4 hs[];   // [mt][dvec]
  const int n = clamp_n(n_dev, n_max);
  if ((int)blockIdx.x * kProjWaves >= n) return;      // block-uniform
  const int m0 = blockIdx.y * MT;
  const int mt = min(MT, M - m0);
  const int tid = threadIdx.x;
  for (int q = tid; q < mt * dvec; q += kProjThreads) hs[q] = h[(size_t)m0 * dvec + q];
  __syncthreads();
  const int wv = tid / NS_WAVE, lane = tid & (NS_WAVE - 1);
  for (int j = blockIdx.x * kProjWaves + wv; j < n; j += gridDim.x * kProjWaves) {
    const int gid = row_ids ? row_ids[j] : j;
    if (gid < 0 || gid >= V) continue;                 // hole
    const uint4* __restrict__ src = rows + (size_t)(mode == NS_INDEXED ? gid : j) * dvec;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
    for (int q0 = 0; q0 < dvec; q0 += NS_WAVE * kProjUnroll) {
      uint4 w[kProjUnroll];
#pragma unroll
      for (int u = 0; u < kProjUnroll; ++u) {
        const int q = q0 + u * NS_WAVE + lane;
        w[u] = q < dvec ? src[q] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kProjUnroll; ++u) {
        const int q = q0 + u * NS_WAVE + lane;
        if (q < dvec) {
#pragma unroll
          for (int m = 0; m < MT; ++m)
            if (m < mt) acc[m] = dot16(w[u], hs[m * dvec + q], acc[m], BF16);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = ns::wave_sum_f32(acc[m]);
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < mt) logits[(size_t)(m0 + m) * n_max + j] = acc[m];
    }
  }
}

template <int CAP>
__global__ __launch_bounds__(kMergeThreads) void k_topk_merge(const float* __restrict__ logits, int n_max,
                                                              const int32_t* __restrict__ row_ids,
                                                              const int32_t* __restrict__ n_dev, int V, int k,
                                                              int32_t* __restrict__ out_ids,
                                                              float* __restrict__ out_vals) {
  __shared__ uint64_t sh[kMergeThreads / NS_WAVE];
  const int m = blockIdx.x;
  const int n = clamp_n(n_dev, n_max);
  uint64_t lst[CAP];
#pragma unroll
  for (int i = 0; i < CAP; ++i) lst[i] = 0;
  const float* __restrict__ lrow = logits + (size_t)m * n_max;
  for (int j = threadIdx.x; j < n; j += kMergeThreads) {
    const int gid = row_ids ? row_ids[j] : j;
    if (gid < 0 || gid >= V) continue;
    const uint64_t key = ns::make_key(lrow[j], gid);
    if (key > lst[CAP - 1]) ns::list_insert(lst, key);
  }
  ns::block_pop_topk<kMergeThreads, CAP>(lst, k, sh, [&](int r, uint64_t key) {
    out_ids[(size_t)m * k + r] = key ? ns::key_id(key) : -1;
    out_vals[(size_t)m * k + r] = key ? ns::key_val(key) : -INFINITY;
  });
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int pick_mt(int M, int d, int esz) {
  int mt = 8;
  while (mt > 1 && (mt >= 2 * M || (size_t)mt * d * esz > kHLdsBytes)) mt >>= 1;
  return ((size_t)mt * d * esz > kHLdsBytes) ? 0 : mt;
}

template <bool BF16>
int launch_valu(int mt, const void* rows, int mode, const int32_t* row_ids, const int32_t* n_dev, int n_max, int V,
                int d, const void* h, int M, float* logits, hipStream_t stream) {
  const int esz = BF16 ? 2 : 4;
  const int dvec = d * esz / 16;
  const int quads = (n_max + kProjWaves - 1) / kProjWaves;
  const int gx = quads < 2048 ? quads : 2048;
  const dim3 grid(gx, (M + mt - 1) / mt);
  const size_t lds = (size_t)mt * dvec * 16;
#define NS_LAUNCH_VALU(MTV)                                                                                     \
  hipLaunchKernelGGL((k_proj_valu<BF16, MTV>), grid, dim3(kProjThreads), lds, stream, (const uint4*)rows, mode, \
                     row_ids, n_dev, n_max, V, dvec, (const uint4*)h, M, logits)
  switch (mt) {
    case 1: NS_LAUNCH_VALU(1); break;
    case 2: NS_LAUNCH_VALU(2); break;
    case 4: NS_LAUNCH_VALU(4); break;
    default: NS_LAUNCH_VALU(8); break;
  }
#undef NS_LAUNCH_VALU
  return ns_launch_status();
}

int launch_merge(const float* logits, int n_max, const int32_t* row_ids, const int32_t* n_dev, int V, int M, int k,
                 int32_t* ids, float* vals, hipStream_t stream) {
#define NS_LAUNCH_MERGE(CAPV)                                                                                 \
  hipLaunchKernelGGL((k_topk_merge<CAPV>), dim3(M), dim3(kMergeThreads), 0, stream, logits, n_max, row_ids, \
                     n_dev, V, k, ids, vals)
  if (k <= 8) NS_LAUNCH_MERGE(8);
  else if (k <= 16) NS_LAUNCH_MERGE(16);
  else if (k <= 32) NS_LAUNCH_MERGE(32);
  else NS_LAUNCH_MERGE(64);
#undef NS_LAUNCH_MERGE
  return ns_launch_status();
}

}  // namespace

extern "C" {

size_t nanospec_draft_workspace_bytes(int32_t n_max, int32_t M, int32_t k) {
  if (n_max < 1 || M < 1 || M > NS_MAX_M || k < 1 || k > NS_MAX_K) return 0;
  return 256 + align256((size_t)M * n_max * sizeof(float));
}

int nanospec_draft_logits_topk(const void* rows, int32_t mode, const int32_t* row_ids, const int32_t* n_dev,
                               int32_t n_max, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M,
                               int32_t k, float* logits, int32_t* topk_ids, float* topk_vals, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  if (mode != NS_PACKED && mode != NS_INDEXED) return NS_EDTYPE;
  if (dtype != NS_BF16 && dtype != NS_FP32) return NS_EDTYPE;
  if (!rows || !h || !topk_ids || !topk_vals || !ws) return NS_EINVAL;
  if (mode == NS_INDEXED && !row_ids) return NS_EINVAL;
  if (n_max < 1 || V < 1 || M < 1 || M > NS_MAX_M || k < 1 || k > NS_MAX_K) return NS_EINVAL;
  if (d < 8 || d > NS_MAX_D || (d % 8) != 0) return NS_EINVAL;
  if ((((uintptr_t)rows) & 15u) || (((uintptr_t)h) & 15u) || (((uintptr_t)ws) & 255u)) return NS_EINVAL;
  if (ws_bytes < nanospec_draft_workspace_bytes(n_max, M, k)) return NS_ECAPACITY;
  const int esz = dtype == NS_BF16 ? 2 : 4;
  const int mt = pick_mt(M, d, esz);
  if (mt == 0) return NS_EINVAL;
  float* lg = logits ? logits : (float*)((char*)ws + 256);
  (void)hipGetLastError();
  int rc = dtype == NS_BF16 ? launch_valu<true>(mt, rows, mode, row_ids, n_dev, n_max, V, d, h, M, lg, stream)
                            : launch_valu<false>(mt, rows, mode, row_ids, n_dev, n_max, V, d, h, M, lg, stream);
  if (rc != NS_OK) return rc;
  return launch_merge(lg, n_max, row_ids, n_dev, V, M, k, topk_ids, topk_vals, stream);
}

}  // extern "C"
