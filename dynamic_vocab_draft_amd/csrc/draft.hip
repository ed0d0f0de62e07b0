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
// Two kernels per call:
//   k_proj_mfma  (bf16) / k_proj_valu (fp32): partial products.  For bf16 a
//       block owns 16*RT active rows (the A operand of
//       v_mfma_f32_16x16x32_bf16, or _f16 for fp16, one row per lane group
//       of 16) and all M
//       hidden rows (the B operand, padded to 16*NMT), over one of S slices
//       of d; its 4 waves split the slice further and their tiles are summed
//       through LDS.  Splitting d across blocks is what puts enough blocks on
//       the 256 CUs: ~1k active rows x 8 KiB is only ~60 row tiles, and one
//       CU alone cannot pull a tile's 128 KiB fast enough.  Both operands
//       reach the matrix cores through per-wave LDS buffers filled by direct
//       global->LDS loads that read each row as a contiguous 128-byte run
//       (double-buffered batches of two k-steps).  Padded B-operand lanes
//       (m >= M) are zeroed.  Each block writes its partial sums
//       (deterministic; no atomics) to partial[s][m][j], slice-major with the
//       column pitch rounded up to 4, so a lane's four rows of one hidden row
//       leave as one 16-byte store and the merge reads each slice with
//       coalesced loads over consecutive columns.  The grid is 1-D, in
//       groups of 8 tiles x S slices per sequence, one tile per XCD: the
//       blocks of the live tiles come first in dispatch order and are dealt
//       evenly over the 8 XCDs and their CUs however large n_max is, and
//       each row is read whole by one XCD.  For 48 < M <= 64 over many rows
//       k_proj_msplit splits M across the waves instead of k.
//   k_merge_cols (+ k_merge_keys past one chunk): per hidden row m and
//       4096-column chunk, a 1024-thread block sums the S partials of each
//       active column in a fixed order and selects the chunk's k best
//       (value, id) keys with a threshold from wave or row maxima and a rank
//       count in LDS; with several chunks a second kernel selects the final
//       k from the chunks' keys, unless every live column is in chunk 0,
//       which then writes the result itself.  No k rounds of cross-lane
//       reductions.
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "select.hpp"
#include "state_fast.hpp"

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// bf16 and fp16 go through the matrix cores; fp32 through the VALU kernel.
__host__ __device__ constexpr bool is_mfma_dtype(int dtype) { return dtype == NS_BF16 || dtype == NS_FP16; }

// Floats between the runs of consecutive hidden rows (and slices) in the
// partial sums: n_max rounded up to 4, so every 4-row group is 16-byte aligned.
__host__ __device__ inline int col_pitch(int n_max) { return (n_max + 3) & ~3; }
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProjThreads = 256;                 // VALU projection block
constexpr int kProjWaves = kProjThreads / NS_WAVE;
constexpr int kProjUnroll = 8;
constexpr size_t kHLdsBytes = 65536;              // LDS budget for staged hidden rows (VALU)

constexpr int kPW = 4;                            // waves per MFMA projection block
constexpr int kPThreads = kPW * NS_WAVE;
constexpr int kTile = 16;                         // rows per MFMA tile
constexpr int kKC = 4;                            // 32-column steps per wave and slice, at least
constexpr int kTargetBlocks = 768;                // MFMA blocks aimed for when choosing S
constexpr int kMaxSplits = 16;
constexpr int kLiveRowsHint = 3072;               // live rows assumed when sizing S without n
constexpr int kBatchLiveRowsHint = 1024;          // rows per sequence a batched launch covers per pass, at most
constexpr int kBatchTargetBlocks = 1024;          // blocks a batched launch aims for


// Per-sequence element strides of a batched call (sequence b = blockIdx.z in
// the merge and the fp32 projection, blockIdx.y in k_merge_keys, decoded from
// the 1-D grid in k_proj_mfma); all zero for a single sequence.
struct BatchStrides {
  size_t rows;     // uint4 units (0: W_head shared by all sequences)
  size_t ids;      // row_ids / n_dev: ids per sequence (n_dev advances by 1)
  size_t h;        // uint4 units
  size_t part;     // floats
  size_t logits;   // floats
  size_t out;      // top-k entries
  size_t cand;     // chunk keys
};

// Log-probability outputs of nanospec_draft_logprob_topk (per sequence b the
// pointers advance by M, or M * C for the chunk statistics).
struct LogProb {
  const float* parent;   // [B][M] score added to each row's log-probabilities (NULL: 0)
  float* lse;            // [B][M] log-sum-exp of the row over the active columns (NULL: not written)
  float2* stats;         // [B][M][C] per chunk: (max, sum of exp(z - max)) when C > 1
  int M;                 // hidden rows per sequence
};

// Sum over the 64 lanes of a wave in a fixed order: an inclusive DPP scan
// (row_shr 1, 2, 4, 8, then row_bcast 15 and 31), read from lane 63.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  const int z = __float_as_int(0.f);
  v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x111, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x112, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x114, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x118, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x142, 0xa, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x143, 0xc, 0xf, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// d-slices for n live rows of each of B sequences: about kTargetBlocks
// blocks, at most s_launch.  When the launch may over-split (n only known on
// the device, n_max above kLiveRowsHint), the projection and the merge both
// derive it from the n they read, so they agree.
__host__ __device__ __forceinline__ int live_splits(int n, int M, int B, int s_launch) {
  const int rt = M <= 16 ? kTile : 2 * kTile;
  const int tiles = ((n > 0 ? n : 1) + rt - 1) / rt * B;
  const int s = (kTargetBlocks + tiles - 1) / tiles;
  return s < 1 ? 1 : (s > s_launch ? s_launch : s);
}

__device__ __forceinline__ int clamp_n(const int32_t* n_dev, int n_max) {
  int n = n_dev ? *n_dev : n_max;
  return n < 0 ? 0 : (n > n_max ? n_max : n);
}

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

// ---------------------------------------------------------------------------
// fp32 VALU projection: a block stages MT hidden rows in LDS and its four
// waves stream rows (one row per wave, 16-byte vectors).  Writes complete dot
// products into part (a single slice).
// ---------------------------------------------------------------------------
template <bool BF16, int MT>
__global__ __launch_bounds__(kProjThreads) void k_proj_valu(const uint4* __restrict__ rows, int mode,
                                                            const int32_t* __restrict__ row_ids,
                                                            const int32_t* __restrict__ n_dev, int n_max, int V,
                                                            int dvec, const uint4* __restrict__ h, int M,
                                                            float* __restrict__ part, BatchStrides bs) {
  extern __shared__ uint4 hs[];   // [mt][dvec]
  {
    const size_t b = blockIdx.z;
    rows += b * bs.rows;
    if (row_ids) row_ids += b * bs.ids;
    if (n_dev) n_dev += b;
    h += b * bs.h;
    part += b * bs.part;
  }
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
        w[u] = src[q < dvec ? q : 0];
      }
      NS_ISSUE_FENCE();
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
        if (m < mt) part[(size_t)(m0 + m) * col_pitch(n_max) + j] = acc[m];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 / fp16 MFMA projection over one slice of d, with both operands staged
// through LDS by direct global->LDS loads (global_load_lds_dwordx4).
//
// A wave owns RT tiles of 16 rows and a range of 32-column k-steps, taken in
// batches of kDmaKC.  One load instruction of a batch fills 16 * 4 kDmaKC
// bytes of LDS: lane L reads row q RPI + L / CPR of the tile at 16-byte
// position p = L % CPR of the batch window, so each row is read as one
// contiguous 16 CPR-byte run (8 rows x 128 B per instruction instead of the
// 16 rows x 64 B that the MFMA lane layout would ask of a direct load; the
// load units then touch half as many cache lines).  The LDS image is
// row-major; position p of row r holds window chunk p ^ (r mod CPR), so the
// ds_read_b128 of an MFMA fragment (lane (i, g) wants chunk 4 kk + g of row
// i) spreads 8 consecutive lanes over distinct banks.  Hidden rows take the
// same route, aliased to row M - 1 past M, except with two hidden tiles
// (17 <= M <= 32), which load them into registers.
//
// Buffers are per wave, NB of them: the wave's first NB batches are
// requested at once and batch b + NB refills batch b's buffers once b is
// multiplied; the waits are explicit vmcnts counting the batches still in
// flight.  With one hidden tile NB = 4, which puts a wave's whole range in
// flight for d = 4096 over four slices (8 KiB of rows instead of two 2 KiB
// batches at a time: 5.12 -> 4.84 us per projection at 1000 live rows of the
// Llama-shaped head, same box, bit-identical results), and the hidden rows
// past M are not fetched at all.  The LDS reads are inline-asm ds_read_b128
// followed by an explicit lgkmcnt(0): the compiler would otherwise wait for
// every load still in flight (it cannot tell the buffers' loads apart across
// the loop).  Hidden rows loaded into registers get such a full wait from the
// compiler before their first use; through LDS they also arrive as whole
// 128-byte runs instead of half lines, which measured faster from three
// hidden tiles up (M = 60: 13.2 -> 12.3 us per call) and slower with two.
// No block barrier until the four waves' tiles are summed.
// ---------------------------------------------------------------------------
constexpr int kDmaKC = 2;                          // k-steps per batch (128-byte row runs)

__device__ __forceinline__ uint32_t lds_addr(const uint4* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint4*)p;
}

__device__ __forceinline__ uint4 lds_read_b128(const uint4* p) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(lds_addr(p)));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Ties a value read by lds_read_b128 to the point after the lgkmcnt wait.
__device__ __forceinline__ void lds_ready(uint4& x) {
  u32x4 v = {x.x, x.y, x.z, x.w};
  asm volatile("" : "+v"(v));
  x = make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void dma16(const uint4* src, uint4* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

// The same load with the non-temporal cache policy (the `nt` bit), for
// W_head rows: each byte of a row is read once per call, so the caches need
// not keep it.  Measured on the full-vocabulary head at M = 8: 189 -> 171 us.
__device__ __forceinline__ void dma16_stream(const uint4* src, uint4* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 2);
}

// vmcnt immediate (gfx9 encoding, expcnt and lgkmcnt left at their maxima).
__host__ __device__ constexpr int vm_imm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

// Waits until at most `left` (< NB) batches of L vector loads each are still
// outstanding: loads complete in issue order, so the oldest batch has landed.
template <int L, int NB>
__device__ __forceinline__ void wait_batches(int left) {
  static_assert(NB >= 1 && NB <= 4 && (NB - 1) * L < 64, "vmcnt range");
  if (NB > 3 && left >= 3) __builtin_amdgcn_s_waitcnt(vm_imm(NB > 3 ? 3 * L : 0));
  else if (NB > 2 && left == 2) __builtin_amdgcn_s_waitcnt(vm_imm(NB > 2 ? 2 * L : 0));
  else if (NB > 1 && left == 1) __builtin_amdgcn_s_waitcnt(vm_imm(L));
  else __builtin_amdgcn_s_waitcnt(vm_imm(0));
}

// The first launch of the fused decode step (nanospec_decode_step): the
// projection with FUSE runs the window-state update in block 0, beside the
// projection in the other blocks, which cannot depend on it.  They project a
// superset of I_{t+1}: columns [0, nd + nv) are the step's tuple entries and
// [cbase, cbase + n_cur) are I_t (the state's cur; cbase is nd + nv rounded
// up to a tile); every id of I_{t+1} is in one of them.  Slice-0 blocks write
// each live column's id to colid and, for a tuple column, whether its id is
// in I_t (the state's bitmap still holds I_t) to told; the update writes
// which columns hold ids of I_{t+1} (FuseCtl).  W_max is at most kPThreads
// kFuseCU and a multiple of 4.
constexpr int kFuseCU = 12;                       // I_t entries per state-update thread
constexpr int kFuseRU = 3;                        // 16-byte ring loads per state-update thread
constexpr int kFuseMaxWmax = kPThreads * kFuseCU;
static_assert(kFuseMaxWmax <= kPThreads * kFuseRU * 4, "ring loads cover W_max");

// The first sequence's arguments; sequence b's state lies st_stride bytes
// further per sequence, its tuples dstride / vstride ids further, and its
// workspace region (flags, hdr, colid, told) ws_stride bytes further.  nd and
// nv are the tuple column counts (the batch's bounds); nd_dev / nv_dev, when
// given, hold each sequence's own counts.
struct FuseArgs {
  ns_state_view v;
  size_t st_stride;
  const int32_t* dids;
  int nd, dstride;
  const int32_t* nd_dev;
  const int32_t* vids;
  int nv, vstride;
  const int32_t* nv_dev;
  FuseCtl fc;
  int32_t* colid;
  uint8_t* told;
  size_t ws_stride;
};

// Sequence b's pointers (the counts nd / nv stay the column bounds).
__device__ __forceinline__ FuseArgs fuse_seq(const FuseArgs& fa, int b) {
  FuseArgs f = fa;
  if (b == 0) return f;
  const size_t so = (size_t)b * fa.st_stride, wo = (size_t)b * fa.ws_stride;
  auto at = [](auto* p, size_t off) { return (decltype(p))((char*)p + off); };
  f.v.len = at(fa.v.len, so);
  f.v.status = at(fa.v.status, so);
  f.v.ring = at(fa.v.ring, so);
  f.v.first = at(fa.v.first, so);
  f.v.bitmap = at(fa.v.bitmap, so);
  f.v.cur = at(fa.v.cur, so);
  f.v.n_cur = at(fa.v.n_cur, so);
  f.v.next_bm = at(fa.v.next_bm, so);
  f.fc.cur = at(fa.fc.cur, so);
  f.fc.n_cur = at(fa.fc.n_cur, so);
  f.fc.next_bm = at(fa.fc.next_bm, so);
  f.fc.flags = at(fa.fc.flags, wo);
  f.fc.hdr = at(fa.fc.hdr, wo);
  f.colid = at(fa.colid, wo);
  f.told = at(fa.told, wo);
  f.dids = fa.dids + (size_t)b * fa.dstride;
  f.vids = fa.vids + (size_t)b * fa.vstride;
  return f;
}

// A sequence's own tuple count: the device count clamped to the bound, or the
// bound when there are no device counts.
__device__ __forceinline__ int fuse_count(const int32_t* dev, int b, int bound) {
  if (!dev) return bound;
  const int c = dev[b];
  return c < 0 ? 0 : (c > bound ? bound : c);
}

// FUSE: 0 the projection alone; 1 the decode step's first launch for one
// sequence (block 0 updates its state); 2 the same for a batch (blocks
// 0..B-1, tuple counts per sequence).  The batch form is an instance of its
// own: its per-sequence offsets and counts in the single form cost the
// decode step 0.3-0.5 us.
template <int NMT, int RT, bool F16, int HI, int NB, bool NT, int FUSE>
__global__ __launch_bounds__(kPThreads) void k_proj_mfma(const uint4* __restrict__ rows, int mode,
                                                         const int32_t* __restrict__ row_ids,
                                                         const int32_t* __restrict__ n_dev, int n_max, int V,
                                                         int dv, const uint4* __restrict__ h, int M,
                                                         int S, int adapt, float* __restrict__ part,
                                                         BatchStrides bs, int B, int tile_step, int dense,
                                                         FuseArgs fa) {
  constexpr int KC = kDmaKC;
  constexpr int CPR = 4 * KC;                      // 16-byte chunks of one row per batch
  constexpr int RPI = NS_WAVE / CPR;               // rows per load instruction
  constexpr int NI = kTile / RPI;                  // load instructions per 16 rows
  constexpr int TB = kTile * CPR;                  // uint4 of one tile's batch window
  // Hidden rows reach the matrix cores through LDS as well, except for two
  // hidden tiles (17 <= M <= 32), where loads into registers measured faster
  // (the LDS copy would cost a block per CU).
  constexpr bool HDMA = NMT != 2;
  // Through LDS, HI load instructions per batch fetch the hidden rows: rows
  // past M are not fetched when HI < NMT NI (their operand lanes are zeroed).
  static_assert(!HDMA || (HI >= 1 && HI <= NMT * NI), "hidden-row loads per batch");
  // NB batch buffers per wave: up to NB batches of one wave are in flight.
  __shared__ uint4 abuf[NB][kPW][RT * TB];
  __shared__ uint4 bbuf[NB][kPW][HDMA ? NMT * TB : 1];
  // The wave tiles of the final sum reuse the staging buffers (RT NMT 4 KiB:
  // within abuf for NMT <= 2, within bbuf otherwise; checked below for every
  // instance).
  static_assert(sizeof(f32x4_t) * kPW * RT * NMT * NS_WAVE <= (NMT <= 2 ? sizeof(abuf) : sizeof(bbuf)),
                "wave tiles fit the reused buffer");
  auto red = reinterpret_cast<f32x4_t (*)[RT][NMT][NS_WAVE]>(NMT <= 2 ? &abuf[0][0][0] : &bbuf[0][0][0]);
  constexpr bool FB = FUSE == 2;
  if constexpr (FUSE == 1) {
    if (blockIdx.x == 0) {                              // the window-state update, in abuf's LDS
      step_fast_body<int4, kFuseRU, kPThreads, kFuseCU>((int4*)&abuf[0][0][0], 0, fa.v, fa.dids, fa.nd, fa.vids, fa.nv,
                                                        nullptr, nullptr, nullptr, fa.fc);
      return;
    }
  }
  if constexpr (FB) {
    if (blockIdx.x < (unsigned)B) {                     // sequence b's window-state update, in abuf's LDS
      const int b = (int)blockIdx.x;
      const FuseArgs f = fuse_seq(fa, b);
      step_fast_body<int4, kFuseRU, kPThreads, kFuseCU>((int4*)&abuf[0][0][0], 0, f.v, f.dids,
                                                        fuse_count(fa.nd_dev, b, fa.nd), f.vids,
                                                        fuse_count(fa.nv_dev, b, fa.nv), nullptr, nullptr, nullptr,
                                                        f.fc);
      return;
    }
  }
  // The 1-D grid is read as (tile group, sequence, slice, XCD lane), tile
  // group slowest: L = ((tg B + b) S + s) 8 + x.  Row tile tg 8 + x of
  // sequence b and slice s.  Dispatch then runs over the low (live) tiles of
  // every sequence before any sequence's high tiles, and every slice of a
  // tile goes to the same XCD (L mod 8).  kblk = (tg S + s) 8 + x is the
  // block's index among its sequence's blocks; for B = 1 it is L.
  const unsigned L = blockIdx.x - (FB ? (unsigned)B : (FUSE ? 1u : 0u));
  const int seq = (int)((L / (8u * (unsigned)S)) % (unsigned)B);
  const unsigned kblk = (L / (8u * (unsigned)S * (unsigned)B)) * (8u * (unsigned)S) + L % (8u * (unsigned)S);
  {
    const size_t b = (size_t)seq;
    rows += b * bs.rows;
    if (row_ids) row_ids += b * bs.ids;
    if (n_dev) n_dev += b;
    h += b * bs.h;
    part += b * bs.part;
  }
  const int tid = threadIdx.x, lane = tid & (NS_WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / NS_WAVE);   // wave-uniform, so branches on it are scalar
  const int i = lane & 15, g = lane >> 4;
  // Workgroups are dealt to the 8 XCDs round-robin (block L to XCD L % 8).
  // Block L takes row tile 8 (L / 8S) + L % 8 and slice (L / 8) % S: each
  // XCD owns whole rows (every slice of its tiles, so a row is read as one
  // 8 KiB run in one L2), and the tiles are dispatched in ascending order,
  // so the live ones (the lowest) come first and spread over every XCD and
  // its CUs, whatever n_max is.
  int r0 = (int)((kblk / (8 * S)) * 8 + (kblk & 7)) * (kTile * RT);
  int split = (int)((kblk >> 3) % S);
  // With dense > 0 (one sequence, a grid of `dense` resident blocks) the
  // blocks take the (tile, slice) items in tile order instead: item q is
  // tile q / S, slice q % S, and block L takes items L, L + dense, ... for as
  // long as they hold live rows, so the live items fill the grid's first
  // blocks whatever the live tile count.
  unsigned q = kblk;
  if (dense > 0) {
    r0 = (int)(q / (unsigned)S) * (kTile * RT);
    split = (int)(q % (unsigned)S);
  }
  // Independent loads first: the active count and this lane's row ids.
  // Fused: |I_t|, the sequence's tuple counts and the ids of the tuple and
  // I_t columns; a column is live iff it holds an entry of either.
  const FuseArgs fs = FB ? fuse_seq(fa, seq) : fa;
  const int cb = fa.fc.cbase, nt = fa.nd + fa.nv;
  int n_old = 0, nd_s = 0, nv_s = 0;
  if constexpr (FUSE != 0) {
    n_old = *fs.fc.n_cur;
    n_old = n_old < 0 ? 0 : (n_old > fa.v.w_max ? fa.v.w_max : n_old);
    if constexpr (FB) {
      nd_s = fuse_count(fa.nd_dev, seq, fa.nd);
      nv_s = fuse_count(fa.nv_dev, seq, fa.nv);
    }
  }
  auto col_id = [&](int row) -> int {
    if (row < nt) return row < fa.nd ? fs.dids[row] : fs.vids[row - fa.nd];
    return (row >= cb && row - cb < fa.v.w_max) ? fs.fc.cur[row - cb] : -1;
  };
  auto col_live = [&](int row) {
    if constexpr (FB) return row < nd_s || (row >= fa.nd && row < fa.nd + nv_s) || (row >= cb && row < cb + n_old);
    else return row < nt || (row >= cb && row < cb + n_old);
  };
  const int n = FUSE ? n_max : clamp_n(n_dev, n_max);
  int gid[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int row = r0 + r * kTile + i;
    if constexpr (FUSE != 0) gid[r] = row < n_max ? col_id(row) : -1;
    else gid[r] = row < n_max ? (row_ids ? row_ids[row] : row) : -1;
  }
  // With `adapt`, S was launched for a few live rows: if n calls for fewer
  // slices, the block maps itself again and reloads its row ids (one more
  // round trip, only when many rows are live).
  if (adapt) {                                          // launch-uniform
    const int S_live = live_splits(n, M, B, S);
    if (S_live != S) {                                  // block-uniform
      S = S_live;
      r0 = (int)((kblk / (8 * S)) * 8 + (kblk & 7)) * (kTile * RT);
      split = (int)((kblk >> 3) % S);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int row = r0 + r * kTile + i;
        gid[r] = row < n_max ? (row_ids ? row_ids[row] : row) : -1;
      }
    }
  }
  // With tile_step > 0 (batches launched for fewer tiles per sequence than
  // n_max holds) the block then takes the tiles tile_step rows further on
  // for as long as they hold live rows.
  for (;;) {
  if (r0 >= n) return;                                  // block-uniform: nothing live here
  if (FUSE && r0 >= nt && (r0 >= cb + n_old || r0 + kTile * RT <= cb)) return;   // block-uniform
  bool ok[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int row = r0 + r * kTile + i;
    ok[r] = (FUSE ? col_live(row) : row < n) && gid[r] >= 0 && gid[r] < V;
  }
  // The merge reads each column's id from colid and, for a tuple column,
  // whether its id is in I_t from told (its word of the I_t bitmap is
  // requested here and written out after the rows).
  uint32_t obits[RT];
  if (FUSE && split == 0 && lane < kTile) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = r0 + r * kTile + i;
      if (row < n_max) fs.colid[row] = ok[r] ? gid[r] : -1;
      obits[r] = (row < nt && ok[r]) ? fs.v.bitmap[gid[r] >> 5] : 0u;
    }
  }
  // Load sources.  Row tr of a tile is requested by the lanes of instruction
  // tr / RPI with L / CPR == tr % RPI; lanes 0..15 hold the tile's row ids.
  // Rows that are not live read row 0 of `rows` (in bounds) and are zeroed
  // as MFMA operands.
  const int rsub = lane / CPR, cpos = lane % CPR;
  const uint4* asrc[RT][NI];
  int apos[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int tr = q * RPI + rsub;
    apos[q] = cpos ^ (tr & (CPR - 1));                  // window chunk this lane fetches
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int gsh = __shfl(gid[r], tr, NS_WAVE);
      const int oks = __shfl((int)ok[r], tr, NS_WAVE);
      asrc[r][q] = rows + (size_t)(oks ? (mode == NS_INDEXED ? gsh : r0 + r * kTile + tr) : 0) * dv;
    }
  }
  // Hidden-row sources: by load instruction for the LDS route (lanes laid out
  // as for the rows, rows past M alias row M - 1), by MFMA lane otherwise
  // (padded lanes alias a real row).  Padded rows are zeroed as operands.
  const uint4* hsrc[HDMA ? HI : 1];
  const uint4* hrow[HDMA ? 1 : NMT];
  bool m_ok[NMT];
#pragma unroll
  for (int t = 0; t < NMT; ++t) {
    m_ok[t] = t * 16 + i < M;
    if constexpr (!HDMA) {
      const int m = t * 16 + i;
      hrow[t] = h + (size_t)(m < M ? m : m % M) * dv;
    }
  }
  if constexpr (HDMA) {
#pragma unroll
    for (int hq = 0; hq < HI; ++hq) {                   // instruction hq: tile hq / NI, rows (hq % NI) RPI ..
      const int m = (hq / NI) * 16 + (hq % NI) * RPI + rsub;
      hsrc[hq] = h + (size_t)(m < M ? m : M - 1) * dv;
    }
  }
  // This wave's 32-column steps: the split's range, divided among the waves.
  const int ksteps = (dv + 3) >> 2;
  const int ks_per_split = (ksteps + S - 1) / S;
  const int kb = split * ks_per_split;
  const int ke = min(ksteps, kb + ks_per_split);
  const int per = (ke - kb + kPW - 1) / kPW;
  const int s_begin = kb + w * per;
  const int s_end = min(ke, s_begin + per);
  f32x4_t acc[RT][NMT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < NMT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint4 z = make_uint4(0, 0, 0, 0);
  const int swz_i = i & (CPR - 1);

  // Requests batch s0 into one set of buffers.  Chunks past the wave's range
  // or past d load column 0 of the same row (their products are zeroed).
  constexpr int HB = HDMA ? NMT * TB : 1;
  auto issue = [&](int s0, uint4 (&ab)[kPW][RT * TB], uint4 (&bb)[kPW][HB], uint4 (&bq)[KC][HDMA ? 1 : NMT]) {
    __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0): earlier reads of these buffers done
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int c = s0 * 4 + apos[q];
      const int cc = (c < s_end * 4 && c < dv) ? c : 0;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        if (NT) dma16_stream(asrc[r][q] + cc, &ab[w][r * TB + q * NS_WAVE]);
        else dma16(asrc[r][q] + cc, &ab[w][r * TB + q * NS_WAVE]);
      }
    }
    if constexpr (HDMA) {
#pragma unroll
      for (int hq = 0; hq < HI; ++hq) {
        const int c = s0 * 4 + apos[hq % NI];
        const int cc = (c < s_end * 4 && c < dv) ? c : 0;
        dma16(hsrc[hq] + cc, &bb[w][(hq / NI) * TB + (hq % NI) * NS_WAVE]);
      }
    }
    if constexpr (!HDMA) {
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const int c8 = (s0 + kk) * 4 + g;
        const int cc = ((s0 + kk) < s_end && c8 < dv) ? c8 : 0;
#pragma unroll
        for (int t = 0; t < NMT; ++t) bq[kk][t] = hrow[t][cc];
      }
    }
  };
  auto compute = [&](int s0, const uint4 (&ab)[kPW][RT * TB], const uint4 (&bb)[kPW][HB],
                     const uint4 (&bq)[KC][HDMA ? 1 : NMT]) {
    uint4 af[KC][RT], bf[KC][HDMA ? NMT : 1];
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const int off = i * CPR + ((4 * kk + g) ^ swz_i);
#pragma unroll
      for (int r = 0; r < RT; ++r) af[kk][r] = lds_read_b128(&ab[w][r * TB + off]);
      if constexpr (HDMA) {
#pragma unroll
        for (int t = 0; t < NMT; ++t) bf[kk][t] = lds_read_b128(&bb[w][t * TB + off]);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
#pragma unroll
      for (int r = 0; r < RT; ++r) lds_ready(af[kk][r]);
      if constexpr (HDMA) {
#pragma unroll
        for (int t = 0; t < NMT; ++t) lds_ready(bf[kk][t]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const int c8 = (s0 + kk) * 4 + g;
      const bool kok = (s0 + kk) < s_end && c8 < dv;
#pragma unroll
      for (int t = 0; t < NMT; ++t) {
        uint4 hv;
        if constexpr (HDMA) hv = bf[kk][t];
        else hv = bq[kk][t];
        const uint4 bv = (kok && m_ok[t]) ? hv : z;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const uint4 av = (kok && ok[r]) ? af[kk][r] : z;
          if (F16)
            acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av),
                                                               __builtin_bit_cast(f16x8_t, bv), acc[r][t], 0, 0, 0);
          else
            acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                __builtin_bit_cast(bf16x8_t, bv), acc[r][t], 0, 0, 0);
        }
      }
    }
  };
  // Loads per batch (vmcnt units), and the wave's batches.  The first NB
  // batches are requested at once (for d = 4096 over four slices that is the
  // wave's whole range, 8 KiB of rows); batch b + NB reuses batch b's buffers
  // as soon as b is multiplied.  The loop over buffers is unrolled, so every
  // buffer (and every register copy of hidden rows) has a fixed index.
  constexpr int NLOADS = NI * RT + (HDMA ? HI : KC * NMT);
  uint4 bq[NB][KC][HDMA ? 1 : NMT];
  const int nb = s_begin < s_end ? (s_end - s_begin + KC - 1) / KC : 0;   // wave-uniform
  // The row ids of this block's next tile (tile_step > 0 or dense > 0) are
  // requested before this tile's rows, so they land while the rows stream
  // (loads complete in issue order, so the batch waits below cover them).
  int gid_next[RT];
  int r0_next = -1, split_next = split;
  if (dense > 0) {
    r0_next = (int)((q + (unsigned)dense) / (unsigned)S) * (kTile * RT);
    split_next = (int)((q + (unsigned)dense) % (unsigned)S);
  } else if (tile_step > 0) {
    r0_next = r0 + tile_step;
  }
  if (r0_next >= 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = r0_next + r * kTile + i;
      if constexpr (FUSE != 0) gid_next[r] = row < n_max ? col_id(row) : -1;
      else gid_next[r] = row < n_max ? (row_ids ? row_ids[row] : row) : -1;
    }
  }
  if (nb > 0) {
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (u < nb) issue(s_begin + u * KC, abuf[u], bbuf[u], bq[u]);
    NS_ISSUE_FENCE();
    for (int b0 = 0; b0 < nb; b0 += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int b = b0 + u;
        if (b < nb) {
          wait_batches<NLOADS, NB>(min(nb - b - 1, NB - 1));
          compute(s_begin + b * KC, abuf[u], bbuf[u], bq[u]);
          if (b + NB < nb) {
            issue(s_begin + (b + NB) * KC, abuf[u], bbuf[u], bq[u]);
            NS_ISSUE_FENCE();
          }
        }
      }
    }
  }
  __syncthreads();                                      // every wave is done with the buffer red reuses
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < NMT; ++t) red[w][r][t][lane] = acc[r][t];
  __syncthreads();
  // Sum the wave tiles.  In a 16x16 result tile, lane L holds rows
  // 4*(L/16) .. +3 (one per register) of column L%16: one 16-byte store into
  // this slice's run of hidden row m (rows that are not live hold zeros and
  // are never read; a quad that starts below n_max ends within the pitch).
  const int NP = col_pitch(n_max);
  for (int e = tid; e < RT * NMT * NS_WAVE; e += kPThreads) {
    const int r = e / (NMT * NS_WAVE);
    const int t = (e / NS_WAVE) % NMT;
    const int l2 = e % NS_WAVE;
    f32x4_t sum = red[0][r][t][l2];
#pragma unroll
    for (int ww = 1; ww < kPW; ++ww) sum += red[ww][r][t][l2];
    const int m = t * 16 + (l2 & 15);
    const int q0 = r0 + r * kTile + (l2 >> 4) * 4;
    if (m < M && q0 < n_max) *(f32x4_t*)(part + ((size_t)split * M + m) * NP + q0) = sum;
  }
  if (FUSE && split == 0 && lane < kTile) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = r0 + r * kTile + i;
      if (row < nt) fs.told[row] = (uint8_t)((obits[r] >> (gid[r] & 31)) & 1u);
    }
  }
  if (r0_next < 0) return;                              // launch-uniform
  r0 = r0_next;
  split = split_next;
  q += (unsigned)dense;
  if (r0 >= n) return;                                  // block-uniform
  __syncthreads();                                      // red is read before the buffers it aliases refill
#pragma unroll
  for (int r = 0; r < RT; ++r) gid[r] = gid_next[r];
  }
}

// ---------------------------------------------------------------------------
// Projection for 48 < M <= 64 over many rows: the four waves split M (wave
// w owns hidden rows 16w .. 16w+15) instead of k, so a block's 16 RT rows
// are read once and shared, and the hidden rows cost one load per row
// tile group instead of one per 32 rows.  Each batch (two k-steps) of the rows is filled into a
// block-shared LDS window by all four waves (RT/4 tiles each, direct
// global->LDS loads, 128-byte row runs, XOR-swizzled as in k_proj_mfma);
// each wave also fills its own hidden-row window.  Three buffers: batch
// it+2 is requested after the barrier of batch it, so two batches are in
// flight while one is multiplied.  Each wave owns complete sums of its
// hidden tile over the block's slice and writes them without a reduction.
// ---------------------------------------------------------------------------
template <int RT, bool F16>
__global__ __launch_bounds__(kPThreads) void k_proj_msplit(const uint4* __restrict__ rows, int mode,
                                                           const int32_t* __restrict__ row_ids,
                                                           const int32_t* __restrict__ n_dev, int n_max, int V,
                                                           int dv, const uint4* __restrict__ h, int M,
                                                           int S, float* __restrict__ part,
                                                           BatchStrides bs, int B) {
  constexpr int KC = kDmaKC;
  constexpr int CPR = 4 * KC;                      // 16-byte chunks of one row per batch
  constexpr int RPI = NS_WAVE / CPR;               // rows per load instruction (8)
  constexpr int NI = kTile / RPI;                  // load instructions per 16 rows (2)
  constexpr int TB = kTile * CPR;                  // uint4 of one tile's batch window
  constexpr int TPW = RT / kPW;                    // row tiles loaded by each wave
  static_assert(RT % kPW == 0, "each wave loads whole tiles");
  constexpr int NBUF = 3;
  __shared__ uint4 ab0[RT * TB], ab1[RT * TB], ab2[RT * TB];
  __shared__ uint4 hb0[kPW][TB], hb1[kPW][TB], hb2[kPW][TB];
  __shared__ int sh_ok[RT * kTile];
  const unsigned L = blockIdx.x;
  const int seq = (int)((L / (8u * (unsigned)S)) % (unsigned)B);
  const unsigned kblk = (L / (8u * (unsigned)S * (unsigned)B)) * (8u * (unsigned)S) + L % (8u * (unsigned)S);
  {
    const size_t b = (size_t)seq;
    rows += b * bs.rows;
    if (row_ids) row_ids += b * bs.ids;
    if (n_dev) n_dev += b;
    h += b * bs.h;
    part += b * bs.part;
  }
  const int tid = threadIdx.x, lane = tid & (NS_WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / NS_WAVE);
  const int i = lane & 15, g = lane >> 4;
  const int r0 = (int)((kblk / (8 * S)) * 8 + (kblk & 7)) * (kTile * RT);
  const int split = (int)((kblk >> 3) % S);
  const int n = clamp_n(n_dev, n_max);
  // This wave loads tiles w TPW .. w TPW + TPW - 1; lanes 0..15 of each hold
  // the tile's row ids.
  int gid[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int row = r0 + (w * TPW + t) * kTile + i;
    gid[t] = row < n_max ? (row_ids ? row_ids[row] : row) : -1;
  }
  if (r0 >= n) return;                                  // block-uniform
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int row = r0 + (w * TPW + t) * kTile + i;
    const bool okv = row < n && gid[t] >= 0 && gid[t] < V;
    if (lane < kTile) sh_ok[(w * TPW + t) * kTile + lane] = okv;
  }
  const int rsub = lane / CPR, cpos = lane % CPR;
  const uint4* asrc[TPW][NI];
  int apos[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int tr = q * RPI + rsub;
    apos[q] = cpos ^ (tr & (CPR - 1));
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int row = r0 + (w * TPW + t) * kTile + tr;
      const int gsh = __shfl(gid[t], tr, NS_WAVE);
      const bool oks = row < n && gsh >= 0 && gsh < V;
      asrc[t][q] = rows + (size_t)(oks ? (mode == NS_INDEXED ? gsh : row) : 0) * dv;
    }
  }
  const uint4* hsrc[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int m = w * kTile + q * RPI + rsub;
    hsrc[q] = h + (size_t)(m < M ? m : M - 1) * dv;
  }
  const bool m_ok = w * kTile + i < M;
  const int ksteps = (dv + 3) >> 2;
  const int ks_per_split = (ksteps + S - 1) / S;
  const int kb = split * ks_per_split;
  const int ke = min(ksteps, kb + ks_per_split);
  f32x4_t acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint4 z = make_uint4(0, 0, 0, 0);
  const int swz_i = i & (CPR - 1);
  auto issue = [&](int s0, uint4 (&ab)[RT * TB], uint4 (&hb)[kPW][TB]) {
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int c = s0 * 4 + apos[q];
      const int cc = (c < ke * 4 && c < dv) ? c : 0;
#pragma unroll
      for (int t = 0; t < TPW; ++t) dma16_stream(asrc[t][q] + cc, &ab[(w * TPW + t) * TB + q * NS_WAVE]);
      dma16(hsrc[q] + cc, &hb[w][q * NS_WAVE]);
    }
  };
  bool okr[RT];
  auto compute = [&](int s0, const uint4 (&ab)[RT * TB], const uint4 (&hb)[kPW][TB]) {
    uint4 af[KC][RT], bf[KC];
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const int off = i * CPR + ((4 * kk + g) ^ swz_i);
#pragma unroll
      for (int r = 0; r < RT; ++r) af[kk][r] = lds_read_b128(&ab[r * TB + off]);
      bf[kk] = lds_read_b128(&hb[w][off]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
#pragma unroll
      for (int r = 0; r < RT; ++r) lds_ready(af[kk][r]);
      lds_ready(bf[kk]);
    }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const int c8 = (s0 + kk) * 4 + g;
      const bool kok = (s0 + kk) < ke && c8 < dv;
      const uint4 bv = (kok && m_ok) ? bf[kk] : z;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const uint4 av = (kok && okr[r]) ? af[kk][r] : z;
        if (F16)
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av),
                                                          __builtin_bit_cast(f16x8_t, bv), acc[r], 0, 0, 0);
        else
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                           __builtin_bit_cast(bf16x8_t, bv), acc[r], 0, 0, 0);
      }
    }
  };
  constexpr int NLOADS = NI * (TPW + 1);                   // this wave's loads of one batch
  constexpr int kWaitOne = (NLOADS & 0xF) | (0x7 << 4) | (0xF << 8) | ((NLOADS >> 4) << 14);
  constexpr int kWaitAll = 0x0F70;
  // Batch b lives in buffer b mod 3.  Iteration it: wait for this wave's
  // loads of batch it (batch it+1 may stay in flight), barrier (every
  // wave's part of batch it has landed, and every wave is done with batch
  // it-1, whose buffer batch it+2 reuses), request batch it+2, multiply.
  if (kb < ke) {                                        // block-uniform
    issue(kb, ab0, hb0);
    if (kb + KC < ke) issue(kb + KC, ab1, hb1);
    NS_ISSUE_FENCE();
    int it = 0;
    for (int s0 = kb; s0 < ke; s0 += KC, ++it) {
      if (s0 + KC < ke) __builtin_amdgcn_s_waitcnt(kWaitOne);
      else __builtin_amdgcn_s_waitcnt(kWaitAll);
      __syncthreads();
      if (it == 0) {
#pragma unroll
        for (int r = 0; r < RT; ++r) okr[r] = sh_ok[r * kTile + i] != 0;
      }
      const int b = it % NBUF;                          // uniform
      if (s0 + 2 * KC < ke) {
        if (b == 0) issue(s0 + 2 * KC, ab2, hb2);
        else if (b == 1) issue(s0 + 2 * KC, ab0, hb0);
        else issue(s0 + 2 * KC, ab1, hb1);
        NS_ISSUE_FENCE();
      }
      if (b == 0) compute(s0, ab0, hb0);
      else if (b == 1) compute(s0, ab1, hb1);
      else compute(s0, ab2, hb2);
    }
  }
  // Lane L of a 16x16 result tile holds rows 4 (L / 16) .. +3 of column L % 16,
  // stored as one 16-byte run (rows that are not live hold zeros and are never
  // read); an empty slice (kb >= ke) writes its zeros so the merge can sum all S.
  const int m = w * kTile + i;
  if (m < M) {
    float* dst = part + ((size_t)split * M + m) * col_pitch(n_max);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int q0 = r0 + r * kTile + g * 4;
      if (q0 < n_max) *(f32x4_t*)(dst + q0) = acc[r];
    }
  }
}

// ---------------------------------------------------------------------------
// Merge (the block selection routine is in select.hpp).
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = kSelectThreads;
constexpr int kMergeCols = 4;                      // columns per thread
constexpr int kMergeChunk = kMergeThreads * kMergeCols;
// One block of 8 columns per thread covers n_max <= 8192 in a single chunk
// (no key merge) when a column's partial sums are at most two 16-byte loads.
constexpr int kMergeColsWide = 8;
// With one or two slices (4-8 bytes of partial sums per column), 16 columns
// per thread cover n_max <= 16384 in a single chunk: one launch instead of
// the per-chunk selection and the key merge.
constexpr int kMergeColsWide16 = 16;

// A column's partial sums of slices 0 .. S-1 (S <= SPT), `stride` floats
// apart (one slice's M runs of NP floats).  Registers past S repeat slice 0
// (the same lines, so no further memory traffic) and are not summed.
template <int SPT>
__device__ __forceinline__ void load_slices(const float* __restrict__ col, size_t stride, int S, float (&p)[SPT]) {
#pragma unroll
  for (int q = 0; q < SPT; ++q) p[q] = col[(q < S ? q : 0) * stride];
}

template <int SPT>
__device__ __forceinline__ float sum_slices(const float (&p)[SPT], int S) {
  float sv = 0.f;                                  // slices summed in a fixed order
#pragma unroll
  for (int q = 0; q < SPT; ++q)
    if (q < S) sv += p[q];
  return sv;
}

// k_merge_cols: block (m, c) sums the S partials of columns
// [c * 1024 U, (c + 1) * 1024 U) of hidden row m (at most U per thread),
// optionally writes the logits, and selects that chunk's top k.  With one
// chunk the winners go straight to the outputs; otherwise each chunk's k
// keys go to cand_out[m][c][k] for k_merge_keys.  The first column of every
// thread is requested in the same round as |I|, so the partial sums are in
// flight before |I| is known (every slice the workspace holds; with `adapt`
// the live count may use fewer).  The further columns follow |I|, and with
// `adapt` they request only the live slices.  With LOGP the emitted values are
// parent[m] + z - lse[m], lse[m] being the log-sum-exp of row m over all
// active columns (a block max and a sum of exp(z - max) per chunk, combined
// by k_merge_keys when there are several); the selection itself runs on z,
// whose order is the same.
template <int SPT, bool FINAL, int U, bool LOGP>
__global__ __launch_bounds__(kMergeThreads) void k_merge_cols(const float* __restrict__ part, int S, int adapt,
                                                              int n_max,
                                                              const int32_t* __restrict__ row_ids,
                                                              const int32_t* __restrict__ n_dev, int V, int k,
                                                              float* __restrict__ logits_out,
                                                              int32_t* __restrict__ out_ids,
                                                              float* __restrict__ out_vals,
                                                              uint64_t* __restrict__ cand_out, BatchStrides bs,
                                                              LogProb lp) {
  constexpr int NT = kMergeThreads, CHUNK = kMergeThreads * U;
  __shared__ SelectSmem sm;
  {
    const size_t b = blockIdx.z;
    part += b * bs.part;
    if (row_ids) row_ids += b * bs.ids;
    if (n_dev) n_dev += b;
    if (logits_out) logits_out += b * bs.logits;
    out_ids += b * bs.out;
    out_vals += b * bs.out;
    cand_out += b * bs.cand;
  }
  const int m = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int col0 = c * CHUNK;
  const int cend = min(n_max, col0 + CHUNK);         // > col0
  const float* prow = part + (size_t)m * col_pitch(n_max);   // slice 0 of hidden row m
  const size_t sstride = (size_t)gridDim.x * col_pitch(n_max);
  const int n_raw = n_dev ? *n_dev : n_max;
  int gv[U];
  float pv[U][SPT];
  const int j0 = col0 + tid;
  const int jc0 = j0 < cend ? j0 : cend - 1;
  // LOGP: the parent score is requested in the first round too, as a vector
  // load (an opaque zero keeps it per lane): a scalar load would share the
  // LDS wait counter and stall the selection's first LDS wait on memory.
  // Without parents it reads a valid partial sum instead.
  const size_t row = (size_t)blockIdx.z * lp.M + m;
  float par_raw = 0.f;
  gv[0] = row_ids ? row_ids[jc0] : jc0;
  load_slices<SPT>(prow + jc0, sstride, SPT, pv[0]);
  if (LOGP) {
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    par_raw = (lp.parent ? lp.parent + row : part)[zero];
  }
  NS_ISSUE_FENCE();
  const float par = (LOGP && lp.parent) ? par_raw : 0.f;
  const int n = n_raw < 0 ? 0 : (n_raw > n_max ? n_max : n_raw);
  if (adapt) S = live_splits(n, (int)gridDim.x, gridDim.z, S);   // as the projection chose (grid: M x chunks x B)
  const int lim = min(n, cend);                      // live columns of this chunk end here
  // With several chunks but every live column in chunk 0, chunk 0 writes the
  // final result and k_merge_keys does nothing; the other chunks are idle.
  const bool final_here = FINAL || n <= CHUNK;
  if (!FINAL && final_here && c > 0) return;         // block-uniform
  const bool more = lim > col0 + NT;                 // block-uniform
  if (more) {
#pragma unroll
    for (int u = 1; u < U; ++u) {
      const int j = col0 + tid + u * NT;
      const int jc = j < lim ? j : lim - 1;
      gv[u] = row_ids ? row_ids[jc] : jc;
      load_slices<SPT>(prow + jc, sstride, adapt ? S : SPT, pv[u]);
    }
    NS_ISSUE_FENCE();
  }
  float val[U];
  int gid[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = col0 + tid + u * NT;
    val[u] = 0.f;
    gid[u] = -1;
    if (u == 0 || more) {
      const float sv = sum_slices<SPT>(pv[u], S);
      if (j < lim && gv[u] >= 0 && gv[u] < V) {
        if (logits_out) logits_out[(size_t)m * n_max + j] = sv;
        val[u] = sv;
        gid[u] = gv[u];
      }
    }
  }
  const int nlive = lim > col0 ? lim - col0 : 0;     // live slots lead: thread t, then t + NT, ...
  // LOGP: each wave's (max, sum of exp(z - max)) goes to LDS before the
  // selection, whose first barrier publishes it; wave 1 combines the 16 pairs
  // in wave order while wave 0 finds the threshold, and the second barrier
  // publishes the result to the emitters.  No barrier of its own.
  __shared__ float sh_mx[NT / NS_WAVE], sh_se[NT / NS_WAVE], sh_lse;
  if (LOGP) {
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (gid[u] >= 0) mx = fmaxf(mx, val[u]);
    mx = ns::wave_max_f32(mx);
    float se = 0.f;
    if (mx != -INFINITY) {                           // wave-uniform
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (gid[u] >= 0) se += expf(val[u] - mx);
    }
    se = wave_sum_dpp(se);
    if ((tid & (NS_WAVE - 1)) == 0) {
      sh_mx[tid / NS_WAVE] = mx;
      sh_se[tid / NS_WAVE] = se;
    }
  }
  const auto mid = [&]() {
    if (LOGP && tid / NS_WAVE == 1) {                // wave 1: lane i takes wave i's pair
      const int lane = tid & (NS_WAVE - 1);
      const float wm = lane < NT / NS_WAVE ? sh_mx[lane] : -INFINITY;
      const float ws = lane < NT / NS_WAVE ? sh_se[lane] : 0.f;
      const float cm = ns::wave_max_f32(wm);
      const float cs = wave_sum_dpp(wm != -INFINITY ? ws * expf(wm - cm) : 0.f);
      if (lane == 0) {
        if (final_here)
          sh_lse = cm == -INFINITY ? -INFINITY : cm + logf(cs);
        else                                         // this chunk's pair for k_merge_keys
          lp.stats[row * gridDim.y + c] = make_float2(cm, cs);
      }
    }
  };
  if (final_here) {
    block_select_topk<U>(val, gid, k, nlive, sm, [&](int r, uint64_t x) {
      out_ids[(size_t)m * k + r] = x ? ns::key_id(x) : -1;
      if (LOGP) {
        const float lse = sh_lse;
        out_vals[(size_t)m * k + r] = x ? ns::key_val(x) + (par - lse) : -INFINITY;
        if (r == 0 && lp.lse) lp.lse[row] = lse;
      } else {
        out_vals[(size_t)m * k + r] = x ? ns::key_val(x) : -INFINITY;
      }
    }, mid);
  } else {
    uint64_t* dst = cand_out + ((size_t)m * gridDim.y + c) * k;
    block_select_topk<U>(val, gid, k, nlive, sm, [&](int r, uint64_t x) { dst[r] = x; }, mid);
  }
}

// k_merge_fused: the merge of the fused decode step (one chunk of at most
// 4096 columns, logits only).  Block m < M sums the S partials of every live
// column of hidden row m (the tuple columns and the I_t columns), keeps
// those the state update flagged as members of I_{t+1}, with the ids the
// projection wrote, and selects their top k exactly as k_merge_cols does.
// The first 2048 columns are requested with |I_t|, the rest only when
// |I_t| reaches them.  Block M turns the update's bitmap of I_{t+1}
// (next_bm) into the state's bitmap and the ascending ids, written to
// active_ids and to the state's cur (with their count to n_active and
// n_cur), and adds the step's appended entries (hdr[1]) to |S|; no other
// block of this launch reads any of them.
constexpr int kFuseCompactWords = 8;                 // bitmap words per thread of block M, at most

// Bitmap words per thread of block M: 4 or 8, as few as cover ceil(V/32).
__host__ __device__ __forceinline__ int fused_compact_wq(int V) {
  return ((V + 31) >> 5) <= 4 * kMergeThreads ? 4 : 8;
}

__device__ __forceinline__ void fused_compact(const uint32_t* __restrict__ next_bm, uint32_t* __restrict__ bitmap,
                                              int V, int w_max, int32_t* __restrict__ ids,
                                              int32_t* __restrict__ n_ids, int32_t* __restrict__ cur,
                                              int32_t* __restrict__ n_cur, int64_t* __restrict__ len, int appended) {
  __shared__ int sh_scan[kMergeThreads / NS_WAVE + 1];
  const int tid = threadIdx.x;
  const int words = (V + 31) >> 5;
  const int wq = fused_compact_wq(V);
  const int w0 = tid * wq;
  uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
  if (w0 < words) {                                   // next_bm has next_words(V) words, zero past ceil(V/32)
    a = *(const uint4*)(next_bm + w0);
    if (wq > 4) b = *(const uint4*)(next_bm + w0 + 4);
  }
  const int pc = __popc(a.x) + __popc(a.y) + __popc(a.z) + __popc(a.w) + __popc(b.x) + __popc(b.y) +
                 __popc(b.z) + __popc(b.w);
  if (w0 < words) {
    if (wq > 4) bm_store8(bitmap, w0, words, a, b, true);
    else bm_store4(bitmap, w0, words, a, true);
  }
  int tot = 0;
  int off = ns::block_excl_scan<kMergeThreads>(pc, sh_scan, &tot);
  // A thread holds a few ids at most, so the stores of one wave fall on
  // nearly consecutive positions.
  auto emit = [&](uint32_t x, int w) {
    while (x) {
      const int id = (w << 5) + (__ffs(x) - 1);
      if (off < w_max) {
        ids[off] = id;
        cur[off] = id;
      }
      ++off;
      x &= x - 1u;
    }
  };
  emit(a.x, w0); emit(a.y, w0 + 1); emit(a.z, w0 + 2); emit(a.w, w0 + 3);
  emit(b.x, w0 + 4); emit(b.y, w0 + 5); emit(b.z, w0 + 6); emit(b.w, w0 + 7);
  if (tid == 0) {
    const int n = tot < w_max ? tot : w_max;
    *n_ids = n;
    *n_cur = n;
    *len += appended;
  }
}

// The merge's buffers for the first sequence; sequence b (blockIdx.z) finds
// its partial sums part_stride floats further per sequence, its workspace
// region (colid, flags, told, hdr) ws_stride bytes further, its state
// st_stride bytes further, its outputs M k (top-k), w_max (ids) and 1
// (count) further.
struct MergeFuseArgs {
  const float* part;
  size_t part_stride;
  const int32_t* colid;
  const uint8_t* flags;
  const uint8_t* told;
  const int32_t* hdr;
  size_t ws_stride;
  int32_t* out_ids;
  float* out_vals;
  const uint32_t* next_bm;
  uint32_t* bitmap;
  int32_t* cur;
  int32_t* n_cur;
  int64_t* len;
  size_t st_stride;
  int32_t* act_ids;
  int32_t* n_act;
};

template <int SPT>
__global__ __launch_bounds__(kMergeThreads) void k_merge_fused(MergeFuseArgs a, int S, int n_max, int M, int cbase,
                                                               int nt, int V, int k, int w_max) {
  constexpr int U = kMergeCols;
  __shared__ SelectSmem sm;
  const int m = blockIdx.x, tid = threadIdx.x;
  const size_t b = blockIdx.z;
  auto at = [](auto* p, size_t off) { return (decltype(p))((char*)p + off); };
  const float* __restrict__ part = a.part + b * a.part_stride;
  const int32_t* __restrict__ colid = at(a.colid, b * a.ws_stride);
  const uint8_t* __restrict__ flags = at(a.flags, b * a.ws_stride);
  const uint8_t* __restrict__ told = at(a.told, b * a.ws_stride);
  const int32_t* __restrict__ hdr = at(a.hdr, b * a.ws_stride);
  int32_t* __restrict__ out_ids = a.out_ids + b * M * k;
  float* __restrict__ out_vals = a.out_vals + b * M * k;
  const uint32_t* __restrict__ next_bm = at(a.next_bm, b * a.st_stride);
  uint32_t* __restrict__ bitmap = at(a.bitmap, b * a.st_stride);
  int32_t* __restrict__ cur = at(a.cur, b * a.st_stride);
  int32_t* __restrict__ n_cur = at(a.n_cur, b * a.st_stride);
  int64_t* __restrict__ len = at(a.len, b * a.st_stride);
  int32_t* __restrict__ act_ids = a.act_ids + b * w_max;
  int32_t* __restrict__ n_act = a.n_act + b;
  if (m == M) {                                       // block-uniform
    fused_compact(next_bm, bitmap, V, w_max, act_ids, n_act, cur, n_cur, len, hdr[1]);
    return;
  }
  const float* prow = part + (size_t)m * col_pitch(n_max);
  const size_t sstride = (size_t)M * col_pitch(n_max);
  // One round of loads: |I_t| and every column's partials, id and flag
  // (indices clamped, so all in bounds).
  constexpr int U1 = 2;                              // columns per thread requested with |I_t|
  const int n_old_raw = hdr[0];
  float pv[U][SPT];
  int gv[U], fv[U];
  auto request = [&](int u) {
    const int j = tid + u * kMergeThreads;
    const int jc = j < n_max ? j : n_max - 1;
    gv[u] = colid[jc];
    fv[u] = flags[jc];
    load_slices<SPT>(prow + jc, sstride, S, pv[u]);
  };
#pragma unroll
  for (int u = 0; u < U1; ++u) request(u);
  const int in_old = tid < nt ? told[tid] : 0;       // tuple columns are all below kMergeThreads
  NS_ISSUE_FENCE();
  const int n_old = n_old_raw < 0 ? 0 : (n_old_raw > w_max ? w_max : n_old_raw);
  const bool more = cbase + n_old > U1 * kMergeThreads;           // block-uniform
  if (more) {
#pragma unroll
    for (int u = U1; u < U; ++u) request(u);
    NS_ISSUE_FENCE();
  }
  float val[U];
  int gid[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = tid + u * kMergeThreads;
    const bool live = (u < U1 || more) && j < n_max && (j < nt ? in_old == 0 : (j >= cbase && j < cbase + n_old)) &&
                      fv[u] != 0 && gv[u] >= 0 && gv[u] < V;
    val[u] = live ? sum_slices<SPT>(pv[u], S) : 0.f;
    gid[u] = live ? gv[u] : -1;
  }
  block_select_topk<U>(val, gid, k, n_max, sm, [&](int r, uint64_t x) {
    out_ids[(size_t)m * k + r] = x ? ns::key_id(x) : -1;
    out_vals[(size_t)m * k + r] = x ? ns::key_val(x) : -INFINITY;
  });
}

// Fallback of the batched decode step: sequence blockIdx.y's cur / n_cur
// from its I_{t+1} (states stride bytes apart).
__global__ void k_copy_cur_batch(ns_state_view v0, size_t stride, const int32_t* __restrict__ ids,
                                 const int32_t* __restrict__ n, int w_max) {
  const size_t b = blockIdx.y;
  int32_t* cur = (int32_t*)((char*)v0.cur + b * stride);
  int32_t* n_cur = (int32_t*)((char*)v0.n_cur + b * stride);
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g == 0) *n_cur = n[b];
  for (int j = g; j < w_max; j += gridDim.x * blockDim.x) cur[j] = ids[b * w_max + j];
}

// Fallback of the decode step: the state's cur / n_cur from I_{t+1}.
__global__ void k_copy_cur(int32_t* __restrict__ cur, int32_t* __restrict__ n_cur, const int32_t* __restrict__ ids,
                           const int32_t* __restrict__ n, int w_max) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g == 0) *n_cur = *n;
  for (int j = g; j < w_max; j += gridDim.x * blockDim.x) cur[j] = ids[j];
}

// k_merge_keys: the final top k of hidden row m over the C chunks' keys
// (nk = C * k of them, at most PER per thread).  With LOGP the chunks'
// (max, sum) pairs give the row's log-sum-exp, combined in chunk order.
template <int PER, bool LOGP>
__global__ __launch_bounds__(kMergeThreads) void k_merge_keys(const uint64_t* __restrict__ cand, int nk, int k,
                                                              const int32_t* __restrict__ n_dev, int n_max,
                                                              int32_t* __restrict__ out_ids,
                                                              float* __restrict__ out_vals, BatchStrides bs,
                                                              LogProb lp) {
  __shared__ SelectSmem sm;
  {
    const size_t b = blockIdx.y;
    cand += b * bs.cand;
    if (n_dev) n_dev += b;
    out_ids += b * bs.out;
    out_vals += b * bs.out;
  }
  if (clamp_n(n_dev, n_max) <= kMergeChunk) return;   // chunk 0 already wrote the result
  const int m = blockIdx.x, tid = threadIdx.x;
  const size_t row = (size_t)blockIdx.y * lp.M + m;
  const float par_raw = *(LOGP && lp.parent ? lp.parent + row : (const float*)cand);
  const float par = (LOGP && lp.parent) ? par_raw : 0.f;
  float shift = 0.f;
  if (LOGP) {
    const int C = nk / k;
    const float2* st = lp.stats + row * C;
    float mx = -INFINITY;
    for (int c = 0; c < C; ++c) mx = fmaxf(mx, st[c].x);
    float se = 0.f;
    if (mx != -INFINITY)
      for (int c = 0; c < C; ++c)
        if (st[c].x != -INFINITY) se += st[c].y * expf(st[c].x - mx);
    const float lse = mx == -INFINITY ? -INFINITY : mx + logf(se);
    shift = par - lse;
    if (lp.lse && tid == 0) lp.lse[row] = lse;
  }
  const uint64_t* src = cand + (size_t)m * nk;
  uint64_t key[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int j = tid + u * kMergeThreads;
    key[u] = src[j < nk ? j : 0];
  }
  NS_ISSUE_FENCE();
  float val[PER];
  int gid[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const bool live = tid + u * kMergeThreads < nk && key[u] != 0;
    val[u] = live ? ns::key_val(key[u]) : 0.f;
    gid[u] = live ? ns::key_id(key[u]) : -1;
  }
  block_select_topk<PER>(val, gid, k, nk, sm, [&](int r, uint64_t x) {
    out_ids[(size_t)m * k + r] = x ? ns::key_id(x) : -1;
    out_vals[(size_t)m * k + r] = x ? (LOGP ? ns::key_val(x) + shift : ns::key_val(x)) : -INFINITY;
  });
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int pick_mt(int M, int d, int esz) {
  int mt = 8;
  while (mt > 1 && (mt >= 2 * M || (size_t)mt * d * esz > kHLdsBytes)) mt >>= 1;
  return ((size_t)mt * d * esz > kHLdsBytes) ? 0 : mt;
}

// The M-split kernel (k_proj_msplit, 64-row groups) serves 48 < M <= 64 once
// the launch spans at least kMsplitMinTiles row groups (over all sequences);
// below that the k-split kernel, with more blocks per row, is faster (at
// ~900 live rows of 3072 it is 11 us against 13 us).
constexpr int kMsplitRT = 4;
constexpr int kMsplitMinTiles = 128;
constexpr int kMsplitTargetBlocks = 512;

bool use_msplit(int n_max, int M, int B) {
  return M > 48 && (long)((n_max + kTile * kMsplitRT - 1) / (kTile * kMsplitRT)) * B >= kMsplitMinTiles;
}

int pick_rt(int M, int n_max, int B) { return use_msplit(n_max, M, B) ? kMsplitRT : (M <= 16 ? 1 : 2); }

// Tile height (16 rt rows) of a batch of B sequences of one slice per tile
// with one hidden tile of at most 8 rows: the largest of 1, 2, 4 that still
// gives about kBatchTargetBlocks blocks for kBatchLiveRowsHint rows each.
int batch_rt(int B) {
  const long per_rt1 = (long)B * (kBatchLiveRowsHint / kTile);
  return per_rt1 >= 4L * kBatchTargetBlocks ? 4 : (per_rt1 >= 2L * kBatchTargetBlocks ? 2 : 1);
}

// Number of d-slices S for the MFMA path: about kTargetBlocks blocks, each
// wave keeping at least kKC k-steps.  When the live row count is
// only known on the device (n_dev given) and M <= 16, S is sized as if at
// most kLiveRowsHint rows of each sequence were live, so a few live rows out
// of a large n_max still spread over the chip; the partial sums then cost at
// most 4 M S / d of the row bytes (3% at d = 4096, M = 8, S = 4).  Larger M
// and calls with n known on the host use n_max: re-mapping the M > 16
// kernel's blocks to the live count measured slower (M = 64 at 3000 of 3072
// rows 22.7 -> 26.7 us per call, M = 20 14.8 -> 20.1 us).  Other dtypes use
// one slice.
int launch_splits(bool n_known, int n_max, int M, int d, int dtype, int B) {
  if (!is_mfma_dtype(dtype)) return 1;
  const int ksteps = (d / 8 + 3) / 4;
  if (use_msplit(n_max, M, B)) {
    // Each wave runs the whole slice; about kMsplitTargetBlocks blocks, so
    // that the partial sums (M S floats per row) stay a small share: two
    // slices over the stress shape's 256 row groups (one: 45.5 -> 64.8 us per
    // call, four: 54.0 us), one over a full vocabulary (two: 327 -> 354 us at
    // V = 151936, M = 64).
    const long tiles = (long)((n_max + kTile * kMsplitRT - 1) / (kTile * kMsplitRT)) * B;
    int s = (int)((kMsplitTargetBlocks + tiles - 1) / tiles);
    const int s_hi = ksteps / kKC < kMaxSplits ? ksteps / kKC : kMaxSplits;
    s = s > s_hi ? s_hi : s;
    return s < 1 ? 1 : s;
  }
  int s_hi = ksteps / (kPW * kKC);
  s_hi = s_hi < 1 ? 1 : (s_hi > kMaxSplits ? kMaxSplits : s_hi);
  const int rt = kTile * pick_rt(M, n_max, B);
  long tiles = (n_max + rt - 1) / rt;
  if (!n_known && M <= 16 && tiles > kLiveRowsHint / rt) tiles = kLiveRowsHint / rt;
  tiles *= B;
  const long s = (kTargetBlocks + tiles - 1) / tiles;
  return s < 1 ? 1 : (s > s_hi ? s_hi : (int)s);
}

// Largest S any call with these dims may launch (sizes the workspace).
int max_splits(int n_max, int M, int d, int B) {
  const int a = launch_splits(false, n_max, M, d, NS_BF16, B);
  const int b = launch_splits(true, n_max, M, d, NS_BF16, B);
  return a > b ? a : b;
}

// Blocks of the single-sequence MFMA projection for M hidden rows that the
// current device holds at once, or 0 when the runtime cannot tell.  Cached
// per device and instance.
int resident_cap(int M) {
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs][5];
  const int inst = M <= 8 ? 0 : (M <= 16 ? 1 : (M <= 32 ? 2 : (M <= 48 ? 3 : 4)));
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) {
    (void)hipGetLastError();
    return 0;
  }
  int c = cache[dev][inst].load(std::memory_order_relaxed);
  if (c != 0) return c > 0 ? c : 0;
  const void* fn = inst == 0   ? (const void*)k_proj_mfma<1, 1, false, 1, 4, true, 0>
                   : inst == 1 ? (const void*)k_proj_mfma<1, 1, false, 2, 4, true, 0>
                   : inst == 2 ? (const void*)k_proj_mfma<2, 2, false, 1, 2, true, 0>
                   : inst == 3 ? (const void*)k_proj_mfma<3, 2, false, 6, 2, true, 0>
                               : (const void*)k_proj_mfma<4, 2, false, 8, 2, true, 0>;
  int cus = 0, bpc = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, fn, kPThreads, 0) != hipSuccess) {
    (void)hipGetLastError();
    c = -1;
  } else {
    c = cus * bpc > 0 ? cus * bpc : -1;
  }
  cache[dev][inst].store(c, std::memory_order_relaxed);
  return c > 0 ? c : 0;
}

template <bool BF16>
int launch_valu(int mt, const void* rows, int mode, const int32_t* row_ids, const int32_t* n_dev, int n_max, int V,
                int d, const void* h, int M, float* part, int B, const BatchStrides& bs, hipStream_t stream) {
  const int esz = BF16 ? 2 : 4;
  const int dvec = d * esz / 16;
  const int quads = (n_max + kProjWaves - 1) / kProjWaves;
  const int gx = quads < 2048 ? quads : 2048;
  const dim3 grid(gx, (M + mt - 1) / mt, B);
  const size_t lds = (size_t)mt * dvec * 16;
#define NS_LAUNCH_VALU(MTV)                                                                                     \
  hipLaunchKernelGGL((k_proj_valu<BF16, MTV>), grid, dim3(kProjThreads), lds, stream, (const uint4*)rows, mode, \
                     row_ids, n_dev, n_max, V, dvec, (const uint4*)h, M, part, bs)
  switch (mt) {
    case 1: NS_LAUNCH_VALU(1); break;
    case 2: NS_LAUNCH_VALU(2); break;
    case 4: NS_LAUNCH_VALU(4); break;
    default: NS_LAUNCH_VALU(8); break;
  }
#undef NS_LAUNCH_VALU
  return ns_launch_status();
}

template <int NMT, int RT, bool F16, int HI, int NB, bool NT, int FUSE>
void launch_mfma_t(unsigned blocks, int B, hipStream_t stream, const void* rows, int mode, const int32_t* row_ids,
                   const int32_t* n_dev, int n_max, int V, int dv, const void* h, int M, int S, int adapt,
                   float* part, const BatchStrides& bs, int tile_step, int dense, const FuseArgs& fa) {
  hipLaunchKernelGGL((k_proj_mfma<NMT, RT, F16, HI, NB, NT, FUSE>), dim3(blocks + (FUSE == 2 ? (unsigned)B : (FUSE ? 1u : 0u))), dim3(kPThreads),
                     0, stream, (const uint4*)rows, mode, row_ids, n_dev, n_max, V, dv, (const uint4*)h, M, S, adapt,
                     part, bs, B, tile_step, dense, fa);
}

template <bool F16>
int launch_mfma(const void* rows, int mode, const int32_t* row_ids, const int32_t* n_dev, int n_max, int V, int d,
                const void* h, int M, int S, int adapt, float* part, int B, const BatchStrides& bs,
                hipStream_t stream, const FuseArgs* fa = nullptr, int max_blocks = 0) {
  const int dv = d / 8;
  const bool msplit = use_msplit(n_max, M, B);
  // Batches of one slice per tile (below) with one hidden tile of at most 8
  // rows take taller tiles as B grows (16 rt rows, rt the largest of 1, 2, 4
  // that still gives about kBatchTargetBlocks blocks for kBatchLiveRowsHint
  // rows per sequence) and a single batch buffer per wave: more blocks per
  // CU (40 KiB of LDS at rt = 4, four blocks) and one hidden-row load per
  // 4 rt row loads.  Measured on the Llama-shaped batch (mean |I| about
  // 780): B = 64 0.56 -> 0.66 of HBM peak, B = 32 0.53 -> 0.59.
  const bool batched = !fa && B > 1 && S == 1 && !adapt && !msplit;
  int rt = pick_rt(M, n_max, B);
  int nb_bufs = 4;
  if (batched && M <= 8) {
    rt = batch_rt(B);
    nb_bufs = rt > 1 ? 1 : 4;
  }
  // Tiles rounded up to a multiple of 8 (padded tiles start past n_max and
  // exit), times S slices, per sequence; one 1-D grid for all B sequences.
  // S > 1 only while tiles x B < kTargetBlocks, or with `adapt` (grid
  // trimmed below), so the grid stays below 2^31.
  unsigned per_seq = (unsigned)(((n_max + kTile * rt - 1) / (kTile * rt) + 7) / 8) * 8u * (unsigned)S;
  if (adapt) {
    // Blocks re-map to the live n with S_live = live_splits(n) slices.  With
    // t = tiles(n) and T = kTargetBlocks: S_live = 1 needs at most
    // tiles_max + 7 blocks per sequence; otherwise t (S_live - 1) < T / B, so
    // the round8(t) S_live blocks it needs stay below T / B + t + 7 S.  The
    // rest of a full tiles x S grid would only exit.
    const unsigned tiles_max = (unsigned)((n_max + kTile * rt - 1) / (kTile * rt));
    const unsigned bound = (unsigned)((kTargetBlocks + B - 1) / B) + tiles_max + 7u * (unsigned)S;
    const unsigned group = 8u * (unsigned)S;
    const unsigned trimmed = (bound + group - 1) / group * group;
    per_seq = trimmed < per_seq ? trimmed : per_seq;
  }
  // Batches of one slice per tile: launch the tiles of kBatchLiveRowsHint
  // rows per sequence and let each block step on by that many rows while
  // its sequence has live rows there.  Launching all of n_max's tiles left
  // most blocks dead (about 850 live rows of 3072 per sequence in the
  // Llama-shaped batch), and each dead block still took a slot for one
  // round trip.
  int tile_step = 0;
  if (batched) {
    // About kBatchTargetBlocks blocks in all, each taking every
    // hint_tiles-th tile of its sequence: at large B a block streams several
    // tiles, the next tile's row ids requested while the current rows stream.
    unsigned hint_tiles = (unsigned)((kBatchLiveRowsHint + kTile * rt - 1) / (kTile * rt) + 7) / 8 * 8;
    const unsigned fill = ((unsigned)kBatchTargetBlocks / (unsigned)B + 7) / 8 * 8;
    hint_tiles = fill > 8 ? (fill < hint_tiles ? fill : hint_tiles) : 8;
    if (hint_tiles < per_seq) {
      per_seq = hint_tiles;
      tile_step = (int)hint_tiles * kTile * rt;
    }
  }
  // With max_blocks (a single sequence whose live row count only the device
  // knows), the grid is cut to a multiple of 8 blocks within max_blocks, all
  // resident at once, and the blocks take the (tile, slice) items in tile
  // order (dense > 0), so the live items, whatever their count, fill the
  // first blocks.  Past the live rows a full grid is mostly blocks that only
  // read the count and exit, and with one block per CU they queue behind the
  // live ones.  Qwen-shaped head (M = 60, one block per CU, S = 7, about
  // 1080 live of 3152 columns): fused decode-step projection 9.0 -> 7.2 us
  // with the grid cut to whole groups of 8 tiles x S slices (the live tiles
  // past 32 then took a second pass), decode step 15.8 -> 12.8 us with the
  // dense order; fewer slices so that 1280 rows fit whole groups (S = 6)
  // measured slower (separate draft head 6.2 -> 7.7 us).
  // Batched fused decode steps: each pass covers the tuple columns and
  // kBatchLiveRowsHint I_t columns per sequence; blocks step on while live.
  if (fa && B > 1 && !adapt) {
    const unsigned hint =
        (unsigned)((fa->fc.cbase + kBatchLiveRowsHint + kTile * rt - 1) / (kTile * rt) + 7) / 8 * 8u;
    if (hint * (unsigned)S < per_seq) {
      per_seq = hint * (unsigned)S;
      tile_step = (int)hint * kTile * rt;
    }
  }
  int dense = 0;
  if (max_blocks > 0 && !batched && !adapt && B == 1) {
    const unsigned lim = (unsigned)max_blocks / 8u * 8u;
    if (lim > 0 && lim < per_seq) {
      per_seq = lim;
      dense = (int)lim;
    }
  }
  const unsigned blocks = per_seq * (unsigned)B;
#define NS_LAUNCH_MFMA_ONLY(NMTV, RTV, HIV, NBV, NTV)                                                         \
  launch_mfma_t<NMTV, RTV, F16, HIV, NBV, NTV, 0>(blocks, B, stream, rows, mode, row_ids, n_dev, n_max, V, dv, h, M, \
                                                  S, adapt, part, bs, tile_step, dense, FuseArgs{})
#define NS_LAUNCH_MFMA(NMTV, RTV, HIV, NBV, NTV)                                                                \
  do {                                                                                                          \
    if (fa && B > 1)                                                                                            \
      launch_mfma_t<NMTV, RTV, F16, HIV, NBV, NTV, 2>(blocks, B, stream, rows, mode, row_ids, n_dev, n_max, V, dv, \
                                                      h, M, S, adapt, part, bs, tile_step, dense, *fa);          \
    else if (fa)                                                                                                \
      launch_mfma_t<NMTV, RTV, F16, HIV, NBV, NTV, 1>(blocks, B, stream, rows, mode, row_ids, n_dev, n_max, V, dv, \
                                                      h, M, S, adapt, part, bs, tile_step, dense, *fa);          \
    else                                                                                                        \
      NS_LAUNCH_MFMA_ONLY(NMTV, RTV, HIV, NBV, NTV);                                                            \
  } while (0)
  if (msplit) {
    hipLaunchKernelGGL((k_proj_msplit<kMsplitRT, F16>), dim3(blocks), dim3(kPThreads), 0, stream, (const uint4*)rows,
                       mode, row_ids, n_dev, n_max, V, dv, (const uint4*)h, M, S, part, bs, B);
    return ns_launch_status();
  }
  // One hidden tile: four batch buffers per wave (64 KiB of LDS per block),
  // and only the hidden rows that exist are fetched (one load instruction per
  // batch covers eight rows).  More tiles keep two buffers (LDS).  Rows are
  // read with the non-temporal policy, except by the tall-tile batch kernels,
  // where it measured slower (B = 64: 102.6 -> 106.4 us per call).
  switch ((M + 15) / 16) {
    case 1:
      if (M <= 8 && nb_bufs == 1) {
        if (rt == 4) NS_LAUNCH_MFMA_ONLY(1, 4, 1, 1, false);
        else NS_LAUNCH_MFMA_ONLY(1, 2, 1, 1, false);
      } else if (M <= 8) {
        NS_LAUNCH_MFMA(1, 1, 1, 4, true);
      } else {
        NS_LAUNCH_MFMA(1, 1, 2, 4, true);
      }
      break;
    case 2: NS_LAUNCH_MFMA(2, 2, 1, 2, true); break;
    case 3: NS_LAUNCH_MFMA(3, 2, 6, 2, true); break;
    default: NS_LAUNCH_MFMA(4, 2, 8, 2, true); break;
  }
#undef NS_LAUNCH_MFMA
#undef NS_LAUNCH_MFMA_ONLY
  return ns_launch_status();
}

int merge_chunks(int n_max) { return (n_max + kMergeChunk - 1) / kMergeChunk; }

// Slices the workspace holds, and the merge requests per column, for S
// slices (monotonic in S, so a workspace sized for the largest S fits every
// smaller one; the merge instances exist for these counts).
int slice_pitch(int S) { return S <= 2 ? S : (S + 3) & ~3; }

// Workspace layout: [0, 256) reserved; partial sums float[B][SP][M][NP]
// (NP = n_max rounded up to 4) at 256; for n_max > kMergeChunk, chunk keys
// uint64[B][M][C][k] after them.
size_t partial_floats(int n_max, int M, int SP) { return (size_t)SP * M * col_pitch(n_max); }
size_t partial_bytes(int n_max, int M, int SP, int B) {
  return align256(partial_floats(n_max, M, SP) * B * sizeof(float));
}

template <bool LOGP>
int launch_merge_t(const float* part, int S, int adapt, int SP, int n_max, const int32_t* row_ids, const int32_t* n_dev, int V,
                   int M, int k, float* logits, int32_t* ids, float* vals, uint64_t* cand, int B,
                   const BatchStrides& bs, const LogProb& lp, hipStream_t stream) {
  const int C = merge_chunks(n_max);
#define NS_LAUNCH_COLS(SPV, FIN, UV)                                                                                 \
  hipLaunchKernelGGL((k_merge_cols<SPV, FIN, UV, LOGP>), dim3(M, (n_max + kMergeThreads * UV - 1) /                 \
                     (kMergeThreads * UV), B), dim3(kMergeThreads), 0, stream, part, S, adapt, n_max, row_ids, n_dev, \
                     V, k, \
                     logits, ids, vals, cand, bs, lp)
#define NS_LAUNCH_COLS_SP(FIN)                        \
  switch (SP) {                                       \
    case 1: NS_LAUNCH_COLS(1, FIN, kMergeCols); break;  \
    case 2: NS_LAUNCH_COLS(2, FIN, kMergeCols); break;  \
    case 4: NS_LAUNCH_COLS(4, FIN, kMergeCols); break;  \
    case 8: NS_LAUNCH_COLS(8, FIN, kMergeCols); break;  \
    case 12: NS_LAUNCH_COLS(12, FIN, kMergeCols); break; \
    default: NS_LAUNCH_COLS(16, FIN, kMergeCols); break; \
  }
  if (C == 1) {
    NS_LAUNCH_COLS_SP(true);
    return ns_launch_status();
  }
  if (C <= 4 && SP <= 2 && C > 2) {                  // one 16384-column chunk: no key merge
    if (SP == 1) NS_LAUNCH_COLS(1, true, kMergeColsWide16);
    else NS_LAUNCH_COLS(2, true, kMergeColsWide16);
    return ns_launch_status();
  }
  if (C == 2 && SP <= 8) {                           // one wide chunk: no key merge
    switch (SP) {
      case 1: NS_LAUNCH_COLS(1, true, kMergeColsWide); break;
      case 2: NS_LAUNCH_COLS(2, true, kMergeColsWide); break;
      case 4: NS_LAUNCH_COLS(4, true, kMergeColsWide); break;
      default: NS_LAUNCH_COLS(8, true, kMergeColsWide); break;
    }
    return ns_launch_status();
  }
  NS_LAUNCH_COLS_SP(false);
#undef NS_LAUNCH_COLS_SP
#undef NS_LAUNCH_COLS
  const int nk = C * k;
  const int per = (nk + kMergeThreads - 1) / kMergeThreads;
#define NS_LAUNCH_KEYS(PERV)                                                                                       \
  hipLaunchKernelGGL((k_merge_keys<PERV, LOGP>), dim3(M, B), dim3(kMergeThreads), 0, stream, cand, nk, k, n_dev, \
                     n_max, ids, vals, bs, lp)
  if (per <= 1) NS_LAUNCH_KEYS(1);
  else if (per <= 2) NS_LAUNCH_KEYS(2);
  else if (per <= 4) NS_LAUNCH_KEYS(4);
  else if (per <= 8) NS_LAUNCH_KEYS(8);
  else NS_LAUNCH_KEYS(16);
#undef NS_LAUNCH_KEYS
  return ns_launch_status();
}

int launch_merge(const float* part, int S, int adapt, int SP, int n_max, const int32_t* row_ids, const int32_t* n_dev, int V,
                 int M, int k, float* logits, int32_t* ids, float* vals, uint64_t* cand, int B,
                 const BatchStrides& bs, const LogProb* lp, hipStream_t stream) {
  if (lp)
    return launch_merge_t<true>(part, S, adapt, SP, n_max, row_ids, n_dev, V, M, k, logits, ids, vals, cand, B, bs, *lp,
                                stream);
  return launch_merge_t<false>(part, S, adapt, SP, n_max, row_ids, n_dev, V, M, k, logits, ids, vals, cand, B, bs,
                               LogProb{nullptr, nullptr, nullptr, M}, stream);
}

// n_max is bounded by the largest vocabulary (a full-vocabulary head has
// n_max = V), which also keeps every grid and pitch computation from it in
// int range.
bool draft_dims_ok(int32_t n_max, int32_t M, int32_t k, int32_t d) {
  return n_max >= 1 && n_max <= NS_MAX_V && M >= 1 && M <= NS_MAX_M && k >= 1 && k <= NS_MAX_K && d >= 8 && d <= NS_MAX_D &&
         (d % 8) == 0;
}

}  // namespace

extern "C" {

// Workspace: partial sums [B x SP x M x NP] float32 (SP = S for S <= 2, else
// S rounded up to 4; NP = n_max rounded up to 4) at offset 256, then, when
// n_max > 4096, the chunk keys and the chunks' log-sum-exp pairs.
size_t nanospec_batch_draft_workspace_bytes(int32_t B, int32_t n_max, int32_t M, int32_t k, int32_t d) {
  if (B < 1 || B > NS_MAX_BATCH || !draft_dims_ok(n_max, M, k, d)) return 0;
  const int SP = slice_pitch(max_splits(n_max, M, d, B));
  const int C = merge_chunks(n_max);
  const size_t keys = C > 1 ? align256((size_t)B * M * C * k * sizeof(uint64_t)) : 0;
  const size_t stats = C > 1 ? align256((size_t)B * M * C * sizeof(float2)) : 0;
  return 256 + partial_bytes(n_max, M, SP, B) + keys + stats;
}

size_t nanospec_draft_workspace_bytes(int32_t n_max, int32_t M, int32_t k, int32_t d) {
  return nanospec_batch_draft_workspace_bytes(1, n_max, M, k, d);
}

}  // extern "C"

namespace {

// Launch plan shared by the whole call and its two stages: slice count,
// partial-sum layout and workspace regions follow from the arguments alone,
// so nanospec_draft_project and nanospec_draft_select agree.
struct DraftPlan {
  int S, SP, adapt, C, max_blocks;
  BatchStrides bs;
  float* part;
  uint64_t* cand;
  float2* stats;
};

int draft_check(const void* rows, int32_t mode, const int32_t* row_ids, int32_t n_max, int32_t B, int32_t V,
                int32_t d, int32_t dtype, const void* h, int32_t M, int32_t k, void* ws, size_t ws_bytes) {
  if (mode != NS_PACKED && mode != NS_INDEXED) return NS_EDTYPE;
  if (dtype != NS_BF16 && dtype != NS_FP32 && dtype != NS_FP16) return NS_EDTYPE;
  if (!rows || !h || !ws) return NS_EINVAL;
  if (mode == NS_INDEXED && !row_ids) return NS_EINVAL;
  if (V < 1 || B < 1 || B > NS_MAX_BATCH || !draft_dims_ok(n_max, M, k, d)) return NS_EINVAL;
  if ((((uintptr_t)rows) & 15u) || (((uintptr_t)h) & 15u) || (((uintptr_t)ws) & 255u)) return NS_EINVAL;
  if (ws_bytes < nanospec_batch_draft_workspace_bytes(B, n_max, M, k, d)) return NS_ECAPACITY;
  return NS_OK;
}

DraftPlan draft_plan(const int32_t* n_dev, int32_t n_max, int32_t B, int32_t d, int32_t dtype, int32_t M, int32_t k,
                     void* ws) {
  DraftPlan p;
  p.S = launch_splits(n_dev == nullptr, n_max, M, d, dtype, B);
  p.SP = slice_pitch(p.S);
  // Only a launch sized by kLiveRowsHint can over-split; the kernels then
  // size S from the live n.
  p.adapt = (is_mfma_dtype(dtype) && n_dev != nullptr && M <= 16 && n_max > kLiveRowsHint) ? 1 : 0;
  // One sequence whose count only the device knows: a grid of resident
  // blocks (launch_mfma's max_blocks).
  p.max_blocks = 0;
  if (is_mfma_dtype(dtype) && n_dev != nullptr && B == 1 && !p.adapt && !use_msplit(n_max, M, B))
    p.max_blocks = resident_cap(M);
  p.C = merge_chunks(n_max);
  const int esz = dtype == NS_FP32 ? 4 : 2;
  p.bs.rows = 0;                                 // W_head (or one packed buffer) shared
  p.bs.ids = (size_t)n_max;
  p.bs.h = (size_t)M * d * esz / 16;
  p.bs.part = partial_floats(n_max, M, p.SP);
  p.bs.logits = (size_t)M * n_max;
  p.bs.out = (size_t)M * k;
  p.bs.cand = (size_t)M * p.C * k;
  p.part = (float*)((char*)ws + 256);
  p.cand = (uint64_t*)((char*)p.part + partial_bytes(n_max, M, p.SP, B));
  p.stats = (float2*)((char*)p.cand + (p.C > 1 ? align256((size_t)B * M * p.C * k * sizeof(uint64_t)) : 0));
  return p;
}

int draft_project(const void* rows, int32_t mode, const int32_t* row_ids, const int32_t* n_dev, int32_t n_max,
                  int32_t B, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M, const DraftPlan& p,
                  hipStream_t stream) {
  (void)hipGetLastError();
  if (dtype == NS_BF16)
    return launch_mfma<false>(rows, mode, row_ids, n_dev, n_max, V, d, h, M, p.S, p.adapt, p.part, B, p.bs,
                              stream, nullptr, p.max_blocks);
  if (dtype == NS_FP16)
    return launch_mfma<true>(rows, mode, row_ids, n_dev, n_max, V, d, h, M, p.S, p.adapt, p.part, B, p.bs,
                             stream, nullptr, p.max_blocks);
  const int mt = pick_mt(M, d, 4);
  if (mt == 0) return NS_EINVAL;
  return launch_valu<false>(mt, rows, mode, row_ids, n_dev, n_max, V, d, h, M, p.part, B, p.bs, stream);
}

int draft_select(const int32_t* row_ids, const int32_t* n_dev, int32_t n_max, int32_t B, int32_t V, int32_t M,
                 int32_t k, float* logits, int32_t* topk_ids, float* topk_vals, const DraftPlan& p, bool logp,
                 const float* parent, float* lse, hipStream_t stream) {
  (void)hipGetLastError();
  const LogProb lp{parent, lse, p.stats, M};
  return launch_merge(p.part, p.S, p.adapt, p.SP, n_max, row_ids, n_dev, V, M, k, logits, topk_ids, topk_vals,
                      p.cand, B, p.bs, logp ? &lp : nullptr, stream);
}

int draft_call(const void* rows, int32_t mode, const int32_t* row_ids, const int32_t* n_dev, int32_t n_max,
               int32_t B, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M, int32_t k, float* logits,
               int32_t* topk_ids, float* topk_vals, void* ws, size_t ws_bytes, hipStream_t stream,
               bool logp = false, const float* parent = nullptr, float* lse = nullptr) {
  int rc = draft_check(rows, mode, row_ids, n_max, B, V, d, dtype, h, M, k, ws, ws_bytes);
  if (rc != NS_OK) return rc;
  if (!topk_ids || !topk_vals) return NS_EINVAL;
  if (!is_mfma_dtype(dtype) && pick_mt(M, d, 4) == 0) return NS_EINVAL;
  const DraftPlan p = draft_plan(n_dev, n_max, B, d, dtype, M, k, ws);
  rc = draft_project(rows, mode, row_ids, n_dev, n_max, B, V, d, dtype, h, M, p, stream);
  if (rc != NS_OK) return rc;
  return draft_select(row_ids, n_dev, n_max, B, V, M, k, logits, topk_ids, topk_vals, p, logp, parent, lse, stream);
}

}  // namespace

extern "C" {

int nanospec_draft_logits_topk(const void* rows, int32_t mode, const int32_t* row_ids, const int32_t* n_dev,
                               int32_t n_max, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M,
                               int32_t k, float* logits, int32_t* topk_ids, float* topk_vals, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  return draft_call(rows, mode, row_ids, n_dev, n_max, 1, V, d, dtype, h, M, k, logits, topk_ids, topk_vals, ws,
                    ws_bytes, stream);
}

int nanospec_batch_draft_logits_topk(const void* w, const int32_t* row_ids, const int32_t* n_dev, int32_t n_max,
                                     int32_t B, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M,
                                     int32_t k, float* logits, int32_t* topk_ids, float* topk_vals, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!n_dev) return NS_EINVAL;
  return draft_call(w, NS_INDEXED, row_ids, n_dev, n_max, B, V, d, dtype, h, M, k, logits, topk_ids, topk_vals, ws,
                    ws_bytes, stream);
}

int nanospec_batch_draft_logprob_topk(const void* w, const int32_t* row_ids, const int32_t* n_dev, int32_t n_max,
                                      int32_t B, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M,
                                      int32_t k, const float* parent, float* lse, float* logits, int32_t* topk_ids,
                                      float* topk_vals, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!n_dev) return NS_EINVAL;
  return draft_call(w, NS_INDEXED, row_ids, n_dev, n_max, B, V, d, dtype, h, M, k, logits, topk_ids, topk_vals, ws,
                    ws_bytes, stream, true, parent, lse);
}

int nanospec_draft_project(const void* rows, int32_t mode, const int32_t* row_ids, const int32_t* n_dev,
                           int32_t n_max, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M, int32_t k,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  const int rc = draft_check(rows, mode, row_ids, n_max, 1, V, d, dtype, h, M, k, ws, ws_bytes);
  if (rc != NS_OK) return rc;
  if (!is_mfma_dtype(dtype) && pick_mt(M, d, 4) == 0) return NS_EINVAL;
  return draft_project(rows, mode, row_ids, n_dev, n_max, 1, V, d, dtype, h, M,
                       draft_plan(n_dev, n_max, 1, d, dtype, M, k, ws), stream);
}

int nanospec_draft_select(const int32_t* row_ids, const int32_t* n_dev, int32_t n_max, int32_t V, int32_t d,
                          int32_t dtype, int32_t M, int32_t k, float* logits, int32_t* topk_ids, float* topk_vals,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dtype != NS_BF16 && dtype != NS_FP32 && dtype != NS_FP16) return NS_EDTYPE;
  if (!topk_ids || !topk_vals || !ws || V < 1 || !draft_dims_ok(n_max, M, k, d)) return NS_EINVAL;
  if (((uintptr_t)ws) & 255u) return NS_EINVAL;
  if (ws_bytes < nanospec_batch_draft_workspace_bytes(1, n_max, M, k, d)) return NS_ECAPACITY;
  return draft_select(row_ids, n_dev, n_max, 1, V, M, k, logits, topk_ids, topk_vals,
                      draft_plan(n_dev, n_max, 1, d, dtype, M, k, ws), false, nullptr, nullptr, stream);
}

int nanospec_draft_logprob_topk(const void* rows, int32_t mode, const int32_t* row_ids, const int32_t* n_dev,
                                int32_t n_max, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M,
                                int32_t k, const float* parent, float* lse, float* logits, int32_t* topk_ids,
                                float* topk_vals, void* ws, size_t ws_bytes, hipStream_t stream) {
  return draft_call(rows, mode, row_ids, n_dev, n_max, 1, V, d, dtype, h, M, k, logits, topk_ids, topk_vals, ws,
                    ws_bytes, stream, true, parent, lse);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The decode step in one call: nanospec_step_update then the INDEXED draft
// head on the new active set, with the same results.  When the state's cur
// holds I_t (the previous call was a decode step on this state) and the
// shapes allow it, the step takes two launches instead of three: the
// projection with the state update in its block 0 (k_proj_mfma with FUSE),
// then k_merge_fused.  Otherwise the three separate launches run and a copy
// refreshes cur (only for shapes that allow the two-launch form).  nanospec_decode_step_project enqueues the first launch
// (the first two of three) and records the form in the state's handle;
// nanospec_decode_step_select enqueues the rest.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kFuseLds = 32768;                  // abuf of every single-sequence MFMA projection instance

struct DecodeLayout {
  int cbase, n_cols, S, SP;
  size_t part, colid, flags, told, total;
};

// Columns: the n_tuple tuple entries, then I_t from the next tile boundary.
// One sequence's region; a batch of B holds B of them back to back, with the
// slices of the separate batched draft head.
DecodeLayout decode_layout(int32_t w_max, int32_t n_tuple, int32_t M, int32_t d, int32_t B = 1) {
  DecodeLayout L;
  L.cbase = ((n_tuple > 0 ? n_tuple : 0) + kTile - 1) / kTile * kTile;
  L.n_cols = L.cbase + w_max;
  L.S = launch_splits(false, w_max, M, d, NS_BF16, B);   // the slices of the separate draft head
  L.SP = slice_pitch(L.S);
  L.part = 256;
  L.colid = L.part + partial_bytes(L.n_cols, M, L.SP, 1);
  L.flags = L.colid + align256((size_t)L.n_cols * 4);
  L.told = L.flags + align256((size_t)L.n_cols);
  L.total = L.told + align256((size_t)(n_tuple > 0 ? n_tuple : 1));
  return L;
}

// LDS of the state-update block of the fused step: the bitmap and the
// tuple ids and first positions.
size_t fused_state_lds(int V, int n_tuple) {
  const int nd64 = (n_tuple + NS_WAVE - 1) & ~(NS_WAVE - 1);
  return ((size_t)kPThreads * fused_wpt<kPThreads>(V) + 2 * (size_t)nd64) * 4;
}

// The merge launch of the fused decode step for B sequences (grid M + 1 by
// B), with the instance of the layout's slice pitch.
int launch_merge_fused(const MergeFuseArgs& ma, const DecodeLayout& L, int M, int B, int nt, int V, int k, int w_max,
                       hipStream_t stream) {
  (void)hipGetLastError();
  const dim3 grid(M + 1, 1, B);
#define NS_LAUNCH_FMERGE(SPV)                                                                                      \
  hipLaunchKernelGGL((k_merge_fused<SPV>), grid, dim3(kMergeThreads), 0, stream, ma, L.S, L.n_cols, M, L.cbase, nt, V, \
                     k, w_max)
  switch (L.SP) {
    case 1: NS_LAUNCH_FMERGE(1); break;
    case 2: NS_LAUNCH_FMERGE(2); break;
    case 4: NS_LAUNCH_FMERGE(4); break;
    case 8: NS_LAUNCH_FMERGE(8); break;
    case 12: NS_LAUNCH_FMERGE(12); break;
    default: NS_LAUNCH_FMERGE(16); break;
  }
#undef NS_LAUNCH_FMERGE
  return ns_launch_status();
}

}  // namespace

extern "C" {

size_t nanospec_decode_step_workspace_bytes(int32_t w_max, int32_t n_tuple, int32_t M, int32_t k, int32_t d) {
  if (w_max < 1 || w_max > NS_MAX_WMAX || n_tuple < 0 || n_tuple > 2 * kFastMaxIds) return 0;
  const size_t sep = nanospec_draft_workspace_bytes(w_max, M, k, d);
  if (sep == 0) return 0;
  const size_t fused = decode_layout(w_max, n_tuple, M, d).total;
  return sep > fused ? sep : fused;
}

int nanospec_decode_step_project(nanospec_state* st, const int32_t* draft_ids, int32_t n_draft,
                                 const int32_t* ver_ids, int32_t n_ver, int32_t* active_ids, int32_t* n_active,
                                 const void* w, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M,
                                 int32_t k, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!st || !active_ids || !n_active || n_draft < 0 || n_ver < 0) return NS_EINVAL;
  if ((n_draft > 0 && !draft_ids) || (n_ver > 0 && !ver_ids)) return NS_EINVAL;
  if (n_draft > kFastMaxIds || n_ver > kFastMaxIds) return NS_EINVAL;
  const ns_state_view& v = st->view;
  if (V != v.V) return NS_EINVAL;
  const int w_max = v.w_max;
  int rc = draft_check(w, NS_INDEXED, active_ids, w_max, 1, V, d, dtype, h, M, k, ws, ws_bytes);
  if (rc != NS_OK) return rc;
  if (ws_bytes < nanospec_decode_step_workspace_bytes(w_max, n_draft + n_ver, M, k, d)) return NS_ECAPACITY;
  st->pending.form = 0;                              // a step this call replaces is not selected any more
  const int nd = st->mode == NS_STREAM_CTX_ONLY ? 0 : n_draft;
  const int nv = st->mode == NS_STREAM_CTX_ONLY ? 0 : n_ver;
  const DecodeLayout L = decode_layout(w_max, nd + nv, M, d);
  // Shapes for which the two-launch form exists; it then needs only the kept
  // I_t (cur_valid).
  const bool fusable = is_mfma_dtype(dtype) && (w_max & 3) == 0 && w_max <= kFuseMaxWmax && nd + nv <= kPThreads &&
                       fused_state_lds(V, nd + nv) <= kFuseLds &&
                       ((V + 31) >> 5) <= kFuseCompactWords * kMergeThreads && !use_msplit(L.n_cols, M, 1) &&
                       L.n_cols <= kMergeChunk && L.SP <= 16;
  const bool fuse = fusable && st->cur_valid;
  nanospec_state::Pending pd;
  pd.keep = fusable;
  pd.nt = nd + nv;
  pd.d = d;
  pd.dtype = dtype;
  pd.M = M;
  pd.k = k;
  pd.ws = ws;
  pd.ids = active_ids;
  pd.n = n_active;
  if (!fuse) {
    rc = nanospec_step_update(st, draft_ids, n_draft, ver_ids, n_ver, active_ids, n_active, nullptr, stream);
    if (rc != NS_OK) return rc;
    const DraftPlan p = draft_plan(n_active, w_max, 1, d, dtype, M, k, ws);
    rc = draft_project(w, NS_INDEXED, active_ids, n_active, w_max, 1, V, d, dtype, h, M, p, stream);
    if (rc != NS_OK) return rc;
    pd.form = 1;
    st->pending = pd;
    return NS_OK;
  }
  char* base = (char*)ws;
  FuseArgs fa{};
  fa.v = v;
  fa.dids = nd > 0 ? draft_ids : v.ring;             // read unconditionally by the update
  fa.nd = nd;
  fa.vids = nv > 0 ? ver_ids : v.ring;
  fa.nv = nv;
  fa.fc = FuseCtl{v.cur, v.n_cur, (uint8_t*)(base + L.flags), (int32_t*)base, v.next_bm, L.cbase, nd, nv};
  fa.told = (uint8_t*)(base + L.told);
  fa.colid = (int32_t*)(base + L.colid);
  BatchStrides bs{};
  bs.part = partial_floats(L.n_cols, M, L.SP);
  // The slices of the separate draft head on I_{t+1} (draft_plan: L.S), so
  // that both forms sum the same partials, and a grid of resident blocks
  // beside the state-update block.
  const int cap = resident_cap(M) - 1;
  float* part = (float*)(base + L.part);
  (void)hipGetLastError();
  rc = dtype == NS_BF16
           ? launch_mfma<false>(w, NS_INDEXED, nullptr, nullptr, L.n_cols, V, d, h, M, L.S, 0, part, 1, bs, stream,
                                &fa, cap)
           : launch_mfma<true>(w, NS_INDEXED, nullptr, nullptr, L.n_cols, V, d, h, M, L.S, 0, part, 1, bs, stream,
                               &fa, cap);
  if (rc != NS_OK) {
    st->drop_cur();
    return rc;
  }
  pd.form = 2;
  st->pending = pd;
  return NS_OK;
}

int nanospec_decode_step_select(nanospec_state* st, int32_t* active_ids, int32_t* n_active, int32_t V, int32_t d,
                                int32_t dtype, int32_t M, int32_t k, int32_t* topk_ids, float* topk_vals, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  if (!st || !topk_ids || !topk_vals) return NS_EINVAL;
  const nanospec_state::Pending pd = st->pending;
  if (pd.form == 0 || pd.ws != ws || pd.ids != active_ids || pd.n != n_active || pd.d != d || pd.dtype != dtype ||
      pd.M != M || pd.k != k)
    return NS_EINVAL;
  const ns_state_view& v = st->view;
  if (V != v.V) return NS_EINVAL;
  const int w_max = v.w_max;
  if (ws_bytes < nanospec_decode_step_workspace_bytes(w_max, pd.nt, M, k, d)) return NS_ECAPACITY;
  st->pending.form = 0;
  int rc;
  if (pd.form == 1) {
    const DraftPlan p = draft_plan(n_active, w_max, 1, d, dtype, M, k, ws);
    rc = draft_select(active_ids, n_active, w_max, 1, V, M, k, nullptr, topk_ids, topk_vals, p, false, nullptr,
                      nullptr, stream);
    if (rc != NS_OK || !pd.keep) return rc;   // shapes without the two-launch form keep no I_t
    (void)hipGetLastError();
    const int g = (w_max + 255) / 256;
    hipLaunchKernelGGL(k_copy_cur, dim3(g > 64 ? 64 : g), dim3(256), 0, stream, v.cur, v.n_cur, active_ids, n_active,
                       w_max);
    rc = ns_launch_status();
    if (rc == NS_OK) st->cur_valid = true;
    return rc;
  }
  // Fused form: unless the merge launches, cur no longer matches the window.
  st->drop_cur();
  const DecodeLayout L = decode_layout(w_max, pd.nt, M, d);
  char* base = (char*)ws;
  (void)hipGetLastError();
  MergeFuseArgs ma{};
  ma.part = (const float*)(base + L.part);
  ma.colid = (const int32_t*)(base + L.colid);
  ma.flags = (const uint8_t*)(base + L.flags);
  ma.told = (const uint8_t*)(base + L.told);
  ma.hdr = (const int32_t*)base;
  ma.out_ids = topk_ids;
  ma.out_vals = topk_vals;
  ma.next_bm = v.next_bm;
  ma.bitmap = v.bitmap;
  ma.cur = v.cur;
  ma.n_cur = v.n_cur;
  ma.len = v.len;
  ma.act_ids = active_ids;
  ma.n_act = n_active;
  rc = launch_merge_fused(ma, L, M, 1, pd.nt, V, k, w_max, stream);
  if (rc == NS_OK) st->cur_valid = true;
  return rc;
}

int nanospec_decode_step(nanospec_state* st, const int32_t* draft_ids, int32_t n_draft, const int32_t* ver_ids,
                         int32_t n_ver, int32_t* active_ids, int32_t* n_active, const void* w, int32_t V, int32_t d,
                         int32_t dtype, const void* h, int32_t M, int32_t k, int32_t* topk_ids, float* topk_vals,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!topk_ids || !topk_vals) return NS_EINVAL;
  const int rc = nanospec_decode_step_project(st, draft_ids, n_draft, ver_ids, n_ver, active_ids, n_active, w, V, d,
                                              dtype, h, M, k, ws, ws_bytes, stream);
  if (rc != NS_OK) return rc;
  return nanospec_decode_step_select(st, active_ids, n_active, V, d, dtype, M, k, topk_ids, topk_vals, ws, ws_bytes,
                                     stream);
}


size_t nanospec_batch_decode_step_workspace_bytes(int32_t B, int32_t w_max, int32_t n_tuple, int32_t M, int32_t k,
                                                  int32_t d) {
  if (B < 1 || B > NS_MAX_BATCH || w_max < 1 || w_max > NS_MAX_WMAX || n_tuple < 0 || n_tuple > 2 * kFastMaxIds)
    return 0;
  const size_t sep = nanospec_batch_draft_workspace_bytes(B, w_max, M, k, d);
  if (sep == 0) return 0;
  const size_t fused = (size_t)B * decode_layout(w_max, n_tuple, M, d, B).total;
  return sep > fused ? sep : fused;
}

int nanospec_batch_decode_step(nanospec_batch* bt, const int32_t* draft_ids, int32_t draft_stride,
                               const int32_t* n_draft, int32_t nd_max, const int32_t* ver_ids, int32_t ver_stride,
                               const int32_t* n_ver, int32_t nv_max, int32_t* active_ids, int32_t* n_active,
                               const void* w, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M,
                               int32_t k, int32_t* topk_ids, float* topk_vals, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (!bt || !draft_ids || !ver_ids || !n_draft || !n_ver || !active_ids || !n_active || !topk_ids || !topk_vals)
    return NS_EINVAL;
  if (nd_max < 0 || nv_max < 0 || nd_max > kFastMaxIds || nv_max > kFastMaxIds) return NS_EINVAL;
  if (draft_stride < nd_max || ver_stride < nv_max) return NS_EINVAL;
  const int B = bt->B;
  const ns_state_view& v0 = bt->members[0].view;
  if (V != v0.V) return NS_EINVAL;
  for (int b = 0; b < B; ++b)                         // as nanospec_batch_step_update
    if (bt->members[b].mode == NS_STREAM_CTX_ONLY) return NS_EINVAL;
  const int w_max = v0.w_max;
  int rc = draft_check(w, NS_INDEXED, active_ids, w_max, B, V, d, dtype, h, M, k, ws, ws_bytes);
  if (rc != NS_OK) return rc;
  if (ws_bytes < nanospec_batch_decode_step_workspace_bytes(B, w_max, nd_max + nv_max, M, k, d)) return NS_ECAPACITY;
  const int nt = nd_max + nv_max;
  const DecodeLayout L = decode_layout(w_max, nt, M, d, B);
  const bool fusable_shape = is_mfma_dtype(dtype) && (w_max & 3) == 0 && w_max <= kFuseMaxWmax && nt <= kPThreads &&
                             fused_state_lds(V, nt) <= kFuseLds &&
                             ((V + 31) >> 5) <= kFuseCompactWords * kMergeThreads && !use_msplit(L.n_cols, M, B) &&
                             L.n_cols <= kMergeChunk && L.SP <= 16;
  // Where the separate batched draft head takes taller tiles (M <= 8, B of
  // 32 and more) the fused projection, which keeps 16-row tiles, measured
  // slower than the three launches (Llama-shaped batch, B = 64: 106.6 against
  // 88.4 us per step, B = 32: 55.6 against 53.8; B = 8: 23.3 against 24.1).
  const bool tall = M <= 8 && B > 1 && L.S == 1 && batch_rt(B) > 1;
  const bool fusable = fusable_shape && !tall;
  bool kept = true;
  for (int b = 0; b < B; ++b) kept = kept && bt->members[b].cur_valid;
  if (!fusable || !kept) {
    rc = nanospec_batch_step_update(bt, draft_ids, draft_stride, n_draft, nd_max, ver_ids, ver_stride, n_ver, nv_max,
                                    active_ids, n_active, nullptr, stream);
    if (rc != NS_OK) return rc;
    rc = nanospec_batch_draft_logits_topk(w, active_ids, n_active, w_max, B, V, d, dtype, h, M, k, nullptr, topk_ids,
                                          topk_vals, ws, ws_bytes, stream);
    if (rc != NS_OK || !fusable) return rc;            // shapes without the two-launch form keep no I_t
    (void)hipGetLastError();
    const int g = (w_max + 255) / 256;
    hipLaunchKernelGGL(k_copy_cur_batch, dim3(g > 64 ? 64 : g, B), dim3(256), 0, stream, v0, bt->stride, active_ids,
                       n_active, w_max);
    rc = ns_launch_status();
    if (rc == NS_OK)
      for (int b = 0; b < B; ++b) bt->members[b].cur_valid = true;
    return rc;
  }
  for (int b = 0; b < B; ++b) bt->members[b].drop_cur();   // until the merge has launched
  char* base = (char*)ws;
  FuseArgs fa{};
  fa.v = v0;
  fa.st_stride = bt->stride;
  fa.dids = draft_ids;
  fa.nd = nd_max;
  fa.dstride = draft_stride;
  fa.nd_dev = n_draft;
  fa.vids = ver_ids;
  fa.nv = nv_max;
  fa.vstride = ver_stride;
  fa.nv_dev = n_ver;
  fa.fc = FuseCtl{v0.cur, v0.n_cur, (uint8_t*)(base + L.flags), (int32_t*)base, v0.next_bm, L.cbase, nd_max, nv_max};
  fa.told = (uint8_t*)(base + L.told);
  fa.colid = (int32_t*)(base + L.colid);
  fa.ws_stride = L.total;
  BatchStrides bs{};
  bs.part = L.total / sizeof(float);                  // each sequence's region, partial sums at L.part
  bs.h = (size_t)M * d * (dtype == NS_FP32 ? 4 : 2) / 16;
  // One sequence: the resident grid in tile order beside the state-update
  // block, as the single-sequence step.
  const int cap = B == 1 ? resident_cap(M) - 1 : 0;
  float* part = (float*)(base + L.part);
  (void)hipGetLastError();
  rc = dtype == NS_BF16
           ? launch_mfma<false>(w, NS_INDEXED, nullptr, nullptr, L.n_cols, V, d, h, M, L.S, 0, part, B, bs, stream,
                                &fa, cap)
           : launch_mfma<true>(w, NS_INDEXED, nullptr, nullptr, L.n_cols, V, d, h, M, L.S, 0, part, B, bs, stream,
                               &fa, cap);
  if (rc != NS_OK) return rc;
  MergeFuseArgs ma{};
  ma.part = part;
  ma.part_stride = L.total / sizeof(float);
  ma.colid = (const int32_t*)(base + L.colid);
  ma.flags = (const uint8_t*)(base + L.flags);
  ma.told = (const uint8_t*)(base + L.told);
  ma.hdr = (const int32_t*)base;
  ma.ws_stride = L.total;
  ma.out_ids = topk_ids;
  ma.out_vals = topk_vals;
  ma.next_bm = v0.next_bm;
  ma.bitmap = v0.bitmap;
  ma.cur = v0.cur;
  ma.n_cur = v0.n_cur;
  ma.len = v0.len;
  ma.st_stride = bt->stride;
  ma.act_ids = active_ids;
  ma.n_act = n_active;
  rc = launch_merge_fused(ma, L, M, B, nt, V, k, w_max, stream);
  if (rc == NS_OK)
    for (int b = 0; b < B; ++b) bt->members[b].cur_valid = true;
  return rc;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free draft head: the workspace (partial sums, chunk keys) is a
// fixed device array of the library instead of a caller buffer.  Each GPU the
// library runs on holds its own copy until the process ends; its address on a
// device is resolved once, on the first call with that device current, and
// kept.  The kernels then receive that address exactly as they receive a
// caller's workspace (the array's name is only a host-side stand-in).
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[NS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (NS_OK), or an error.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return NS_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return NS_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NS_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NS_OK;
}

}  // namespace

extern "C" {

int nanospec_draft_logits_topk_noalloc(const void* rows, int32_t mode, const int32_t* row_ids, const int32_t* n_dev,
                                       int32_t n_max, int32_t V, int32_t d, int32_t dtype, const void* h, int32_t M,
                                       int32_t k, float* logits, int32_t* topk_ids, float* topk_vals,
                                       hipStream_t stream) {
  const size_t need = nanospec_draft_workspace_bytes(n_max, M, k, d);
  if (need == 0) return NS_EINVAL;
  if (need > (size_t)NS_NOALLOC_SCRATCH_BYTES) return NS_ESCRATCH;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != NS_OK) return rc;
  return draft_call(rows, mode, row_ids, n_dev, n_max, 1, V, d, dtype, h, M, k, logits, topk_ids, topk_vals, ws,
                    (size_t)NS_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
