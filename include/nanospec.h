/*
 * nanospec.h -- C ABI of the dynamic-vocabulary draft LM head for AMD MI355X
 * (gfx950).
 *
 * The method (MicroSpec / NanoSpec, arXiv 2605.26444):
 *   Sec. 3.1, Eq. 1         : the LM head z = W_head h, W_head in R^{V x d};
 *                             the draft computes it only on W_head[I_t, :].
 *   Sec. 3.2 (prefill)      : T_K(z) = indices of the K largest logits;
 *                             S_init = prompt (+) tuple(U_i T_Kpre(z_i)).
 *   Sec. 3.2 (decoding)     : S_new = S_old (+) tuple(C_draft) (+) tuple(C_ver).
 *   Sec. 3.2 (sliding window): I_{t+1} = Unique(Suffix(S_new, W_max)).
 *   Sec. 3.3 / NanoSpec "Eliminating Overhead via GPU-Resident State
 *   Management": the window state lives on the GPU as a bitmap and is updated
 *   without host round trips; "Avoiding Sparse Computation via Asynchronous
 *   Gathering": the rows W_head[I_t, :] are packed into a preallocated buffer
 *   on a second stream.
 *
 * Conventions (every entry point):
 *   - Pointers are DEVICE pointers unless the comment says "host".
 *   - Every call enqueues its work on `stream` and returns without waiting
 *     for it; only nanospec_state_status synchronises (the given stream).
 *   - The library never allocates device memory: the caller owns the state
 *     buffer, workspaces and outputs, and must keep them alive until the
 *     enqueued work has finished.  The library owns only the small host
 *     handle made by nanospec_state_create.
 *   - Return value: NS_OK, or an error code.  Argument errors (NS_EINVAL,
 *     NS_EDTYPE, NS_ECAPACITY) are detected on the host before anything is
 *     enqueued.  NS_EHIP reports a failed kernel launch; for calls that
 *     launch more than one kernel, kernels launched before the failure stay
 *     enqueued.
 *   - Errors only the device can see (an id outside [0, V)) set sticky bits
 *     in the state's status word (NS_STATUS_*); the offending entries are
 *     skipped, so results equal the definition applied to the valid entries.
 *   - Tie rule for every top-k: value descending, then id ascending; +0.0 and
 *     -0.0 are equal.  If k exceeds the candidate count, trailing entries are
 *     (id -1, value -INFINITY).
 *   - Calls on one state must be ordered (same stream, or events); calls on
 *     distinct states and buffers may run concurrently.
 */
#ifndef NANOSPEC_H
#define NANOSPEC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------- */
#define NS_OK        0
#define NS_EINVAL    1   /* null pointer, bad size, limit exceeded */
#define NS_EDTYPE    2   /* unknown dtype or mode */
#define NS_ECAPACITY 3   /* state or workspace buffer too small */
#define NS_EHIP      4   /* a HIP launch or runtime call failed */
#define NS_ESCRATCH  5   /* larger than the fixed scratch of nanospec_draft_logits_topk_noalloc */

/* ---- element types of W_head, h and logits ---------------------------- */
#define NS_BF16 0        /* bfloat16, stored as 16-bit patterns */
#define NS_FP32 1        /* IEEE float32 */
#define NS_FP16 2        /* IEEE binary16, stored as 16-bit patterns */

/* ---- row modes of nanospec_draft_logits_topk --------------------------- */
#define NS_PACKED  0     /* rows = packed buffer [n_max x d]; row j is rows[j] */
#define NS_INDEXED 1     /* rows = W_head [V x d]; row j is W_head[row_ids[j]] */

/* ---- stream sources (nanospec_state_set_mode) -------------------------- */
#define NS_STREAM_FULL     0   /* prompt, prefill candidates and decoding tuples */
#define NS_STREAM_CTX_ONLY 1   /* prompt and prefill candidates only */
#define NS_STREAM_EXT_ONLY 2   /* decoding tuples only */

/* ---- sticky device status bits ---------------------------------------- */
#define NS_STATUS_BAD_ID 0x1u   /* an appended id was outside [0, V) and was skipped */

/* ---- limits ------------------------------------------------------------ */
#define NS_MAX_M      64        /* hidden rows per draft-head call */
#define NS_MAX_K      64        /* draft top-k and prefill K_pre */
#define NS_MAX_V      1048576   /* vocabulary size (the bitmap is built in LDS) */
#define NS_MAX_WMAX   1048576   /* sliding-window length */
#define NS_MAX_D      16384     /* hidden size; d % 8 == 0 */
#define NS_MAX_BATCH  4096      /* sequences in one batch */
#define NS_MAX_SLOTS  16384     /* slots of a slot-stable packed buffer */
#define NS_MAX_TREE_CAND 4096   /* candidates of one nanospec_tree_select */

typedef struct nanospec_state nanospec_state;   /* opaque host handle */
typedef struct nanospec_batch nanospec_batch;   /* opaque host handle of B states */
typedef struct nanospec_packed nanospec_packed; /* opaque host handle of a slot map */

/* Human-readable text for a return code (static storage, never NULL). */
const char* nanospec_strerror(int code);

/* Library version, major*10000 + minor*100 + patch. */
int nanospec_version(void);

/* ======================================================================
 * Window state: the tail of the candidate stream S and the active bitmap.
 * Sec. 3.2 "Vocabulary Construction via Sliding Window" needs only the last
 * W_max entries of S, so the state keeps them in a ring of W_max int32 plus
 * the total stream length (int64); the per-id first-position table (int32[V],
 * used for in-tuple dedup) and the active bitmap (uint32[ceil(V/32)]) make up
 * the rest.  Size is O(V + W_max), independent of sequence length.
 * ====================================================================== */

/* Bytes of device memory a state for (V, w_max) needs; 0 if out of limits. */
size_t nanospec_state_bytes(int32_t V, int32_t w_max);

/* Binds a state to caller-owned device memory `dev_mem` (>= state_bytes,
 * 256-byte aligned) and enqueues its initialisation (empty stream, empty
 * active set) on `stream`.  *out (host) receives the handle.
 * Errors: NS_EINVAL (null, V or w_max outside [1, limit], misaligned),
 * NS_ECAPACITY (dev_bytes too small), NS_EHIP. */
int nanospec_state_create(nanospec_state** out, int32_t V, int32_t w_max,
                          void* dev_mem, size_t dev_bytes, hipStream_t stream);

/* Enqueues a reset to the empty stream (status bits cleared). */
int nanospec_state_reset(nanospec_state* st, hipStream_t stream);

/* Frees the host handle (the device memory stays the caller's). */
int nanospec_state_destroy(nanospec_state* st);

/* Stream sources of the ablation study (NanoSpec Sec. 4, ablation, Table 5),
 * a host-side setting of the handle (default NS_STREAM_FULL, kept by reset):
 *   NS_STREAM_CTX_ONLY : I comes from the prompt and the prefill candidates
 *       only; nanospec_step_update appends nothing (it ignores its tuples)
 *       and still rebuilds I and writes its outputs.
 *   NS_STREAM_EXT_ONLY : I comes from the decoding tuples C_draft and C_ver
 *       only; nanospec_stream_append drops its ids and enqueues nothing.
 * The same call sequence then yields each ablation's vocabulary.
 * nanospec_batch_step_update refuses (NS_EINVAL) a batch with a CTX_ONLY
 * member.  Errors: NS_EINVAL (null handle, unknown mode). */
int nanospec_state_set_mode(nanospec_state* st, int32_t mode);

/* Synchronises `stream`, then writes the sticky status bits to *flags (host)
 * and clears them. */
int nanospec_state_status(nanospec_state* st, uint32_t* flags, hipStream_t stream);

/* Enqueues a copy of Suffix(S, W_max) in stream order into window[0..w_max)
 * (entries past min(|S|, W_max) are set to -1) and |S| into *len (int64).
 * Either output may be NULL. */
int nanospec_state_window(nanospec_state* st, int32_t* window, int64_t* len,
                          hipStream_t stream);

/* ======================================================================
 * Stream append.  Sec. 3.2: S_init = prompt (+) tuple(U_i T_Kpre(z_i)) and
 * S_new = S_old (+) tuple(C_draft) (+) tuple(C_ver).
 *   ids[0..n)    : candidate ids (device, int32), read in the given order.
 *   dedup_first  : 0 -> append every id as given (prompt, C_ver);
 *                  1 -> append each distinct id once, at its first occurrence
 *                  (tuple() of the prefill union, C_draft from raw tree ids).
 * Dedup is within this call only; S keeps repeats across calls.  Ids outside
 * [0, V) are skipped and set NS_STATUS_BAD_ID.  n may be 0.
 * Errors: NS_EINVAL (null state, n < 0, ids NULL with n > 0), NS_EHIP. */
int nanospec_stream_append(nanospec_state* st, const int32_t* ids, int32_t n,
                           int32_t dedup_first, hipStream_t stream);

/* ======================================================================
 * Active vocabulary.  Sec. 3.2: I = Unique(Suffix(S, W_max)).
 *   active_ids[0..w_max) : receives I in ascending id order; entries past
 *                          |I| are left untouched.
 *   n_active[1]          : receives |I| (int32, device; no host readback).
 *   bitmap[ceil(V/32)]   : optional (may be NULL) copy of the state's bitmap:
 *                          bit b of word w (LSB first) is set iff 32w+b is
 *                          in I; padding bits are 0.
 * The state's own bitmap is always updated.
 * Errors: NS_EINVAL (null state / active_ids / n_active), NS_EHIP. */
int nanospec_active_vocab(nanospec_state* st, int32_t* active_ids, int32_t* n_active,
                          uint32_t* bitmap, hipStream_t stream);

/* One decode-step state update in a single launch: the same as
 *   stream_append(draft_ids, n_draft, 1); stream_append(ver_ids, n_ver, 0);
 *   active_vocab(active_ids, n_active, bitmap);
 * (Sec. 3.2 decoding phase followed by the sliding-window rebuild). */
int nanospec_step_update(nanospec_state* st,
                         const int32_t* draft_ids, int32_t n_draft,
                         const int32_t* ver_ids, int32_t n_ver,
                         int32_t* active_ids, int32_t* n_active, uint32_t* bitmap,
                         hipStream_t stream);

/* ======================================================================
 * Batches of independent sequences (data parallel over sequences).  Each
 * sequence has its own window state, exactly as above; a batch lays B of them
 * back to back in one caller-owned buffer so that one launch serves all B.
 * nanospec_batch_member returns the ordinary handle of sequence b, which every
 * single-sequence call above accepts (prompt appends, window, status, reset).
 *   nanospec_batch_state_bytes : B * nanospec_state_bytes(V, w_max) (0 if B
 *             is not in [1, NS_MAX_BATCH] or the dims are invalid).
 *   nanospec_batch_create      : as nanospec_state_create for all B members.
 *   nanospec_batch_step_update : nanospec_step_update for every sequence b,
 *             one workgroup per sequence:
 *               draft_ids + b * draft_stride : C_draft ids of sequence b,
 *                   n_draft[b] of them (device int32 [B], clamped to
 *                   [0, nd_max]); the same for ver_ids / ver_stride / n_ver.
 *                   draft_ids and ver_ids must point to readable memory even
 *                   when a count is 0.
 *               active_ids [B x w_max], n_active [B], bitmap [B x ceil(V/32)]
 *                   or NULL: sequence b's outputs are the b-th blocks.
 *             Limits: nd_max, nv_max <= 512, w_max <= 16384 and the bitmap
 *             in LDS (V <= about 1.1M); NS_EINVAL otherwise (use the
 *             single-sequence call per member).
 * Errors: NS_EINVAL, NS_ECAPACITY, NS_EHIP. */
size_t nanospec_batch_state_bytes(int32_t B, int32_t V, int32_t w_max);
int nanospec_batch_create(nanospec_batch** out, int32_t B, int32_t V, int32_t w_max,
                          void* dev_mem, size_t dev_bytes, hipStream_t stream);
int nanospec_batch_destroy(nanospec_batch* bt);
int nanospec_batch_member(nanospec_batch* bt, int32_t b, nanospec_state** out);
int nanospec_batch_step_update(nanospec_batch* bt,
                               const int32_t* draft_ids, int32_t draft_stride,
                               const int32_t* n_draft, int32_t nd_max,
                               const int32_t* ver_ids, int32_t ver_stride,
                               const int32_t* n_ver, int32_t nv_max,
                               int32_t* active_ids, int32_t* n_active, uint32_t* bitmap,
                               hipStream_t stream);

/* ======================================================================
 * Row gather ("pack").  NanoSpec "Avoiding Sparse Computation via
 * Asynchronous Gathering": out[j, :] = w[ids[j], :] for j < n, a bit copy.
 *   w     : W_head, [V x d] row-major, elements of `dtype`, 16-byte aligned.
 *   ids   : [n_max] int32 row ids; ids outside [0, V) leave out[j] untouched.
 *   n_dev : [1] int32 row count on the device (NULL -> n = n_max); n is
 *           clamped to [0, n_max].
 *   out   : [n_max x d] packed buffer, 16-byte aligned; rows j >= n untouched.
 * Meant to run on a copy stream, with an event recorded after it that the
 * compute stream waits on before the projection.
 * Errors: NS_EINVAL (nulls, d % 8 != 0, d > NS_MAX_D, V or n_max < 1),
 * NS_EDTYPE, NS_EHIP. */
int nanospec_gather_rows(const void* w, int32_t V, int32_t d, int32_t dtype,
                         const int32_t* ids, const int32_t* n_dev, int32_t n_max,
                         void* out, hipStream_t stream);

/* ======================================================================
 * Slot-stable packed buffer.  NanoSpec "Avoiding Sparse Computation via
 * Asynchronous Gathering": one buffer of W_max rows is allocated up front and
 * each step gathers into it only the rows of ids that became active.
 * Placement (the pages leave it open): a row stays in its slot while its id
 * stays active; the slots of ids that left become holes (id -1); the entering
 * ids, in ascending id order, take the free slots in ascending slot order.
 * n_slots is one past the highest occupied slot; it never exceeds the
 * largest |I| seen since the last reset.
 *   nanospec_packed_bytes  : device bytes of the slot map for (V, w_max slots):
 *             a 256-byte header (int32 n_slots, int32 n_enter), int32
 *             slot_ids[w_max], int32 enter_slots[w_max], int32
 *             enter_ids[w_max] and the held-id bitmap uint32[ceil(V/32)].
 *             0 if V or w_max is outside [1, NS_MAX_V] / [1, NS_MAX_SLOTS].
 *   nanospec_packed_create : binds a slot map to caller-owned device memory
 *             (256-byte aligned) and enqueues its reset (all holes, nothing
 *             held).  The row buffer itself, [w_max x d] elements, is also
 *             the caller's and is passed to every update.
 *   nanospec_packed_update : for the active set of the state's latest rebuild
 *             (its bitmap), updates the slot map and enqueues the copy
 *             rows[enter_slots[r], :] = w[enter_ids[r], :] for r < n_enter.
 *             Rows of slots that stay occupied are not touched; hole rows hold
 *             whatever they held.  st must have the same V and a w_max no
 *             larger than the slot count; w and rows are 16-byte aligned, d %
 *             8 == 0, and d, dtype and rows must stay the same from one update
 *             to the next (until a reset).
 *   nanospec_packed_slots  : (host call) the device addresses of slot_ids,
 *             n_slots, enter_slots, enter_ids and n_enter (each output may be
 *             NULL).  The head over the buffer is
 *             nanospec_draft_logits_topk(rows, NS_PACKED, slot_ids, n_slots,
 *             w_max, ...), which skips holes.
 *   nanospec_packed_reset / _destroy : reset to empty / free the host handle.
 * The update is two launches (the slot plan on one workgroup, then the row
 * copy); like the plain gather it may run on a copy stream, ordered after the
 * state update that produced the active set.
 * Errors: NS_EINVAL (nulls, limits, misalignment, V / w_max mismatch),
 * NS_EDTYPE, NS_ECAPACITY (dev_bytes too small), NS_EHIP. */
size_t nanospec_packed_bytes(int32_t V, int32_t w_max);
int nanospec_packed_create(nanospec_packed** out, int32_t V, int32_t w_max,
                           void* dev_mem, size_t dev_bytes, hipStream_t stream);
int nanospec_packed_reset(nanospec_packed* pk, hipStream_t stream);
int nanospec_packed_destroy(nanospec_packed* pk);
int nanospec_packed_slots(const nanospec_packed* pk, const int32_t** slot_ids,
                          const int32_t** n_slots, const int32_t** enter_slots,
                          const int32_t** enter_ids, const int32_t** n_enter);
int nanospec_packed_update(nanospec_packed* pk, const nanospec_state* st,
                           const void* w, int32_t d, int32_t dtype, void* rows,
                           hipStream_t stream);

/* ======================================================================
 * Restricted LM head + top-k + map back to global ids.  Sec. 3.1, Eq. 1 on
 * the sub-matrix W_head[I, :] for M hidden rows, then T_k per row.
 *   rows    : NS_PACKED  -> packed rows [n_max x d] (row j = rows[j]);
 *             NS_INDEXED -> W_head [V x d] (row j = W_head[row_ids[j]]).
 *   row_ids : [n_max] global id of row j (a hole if outside [0, V): skipped).
 *             May be NULL in NS_PACKED mode only: then row j has id j (with
 *             rows = W_head and n_max = V this is the full-vocabulary head).
 *   n_dev   : [1] int32 active row count (NULL -> n_max), clamped to n_max.
 *   h       : [M x d] hidden rows, same dtype as rows, 16-byte aligned.
 *   logits  : optional [M x n_max] float32 output (NULL -> not written);
 *             columns j >= n and holes are left untouched.
 *   topk_ids/topk_vals : [M x k] int32 / float32 outputs; row m holds the k
 *             largest logits of hidden row m, ordered by (value desc, global
 *             id asc), with the global ids.
 *   ws      : workspace of >= nanospec_draft_workspace_bytes(n_max, M, k, d)
 *             bytes, 256-byte aligned (partial sums over slices of d and,
 *             when n_max > 4096, room for per-chunk top-k keys and
 *             log-sum-exp pairs; no initialisation needed).  Calls sharing
 *             a workspace must be ordered.
 * Arithmetic: bf16 and fp16 products are exact in float32 and summed in
 * float32 on the matrix cores (v_mfma_f32_16x16x32_bf16 / _f16), in slices of
 * d whose partial sums are added in a fixed order; fp32 inputs use float32
 * FMAs.  No float atomics: the same arguments and inputs give the same
 * results (the slice count depends on n_max, M, d and the live count).
 * row_ids must be distinct apart from holes.
 * Errors: NS_EINVAL (nulls, M not in [1,64], k not in [1,64], d % 8 != 0,
 * n_max not in [1, NS_MAX_V]), NS_EDTYPE, NS_ECAPACITY (ws too small),
 * NS_EHIP.  nanospec_draft_workspace_bytes returns 0 for such dims. */
size_t nanospec_draft_workspace_bytes(int32_t n_max, int32_t M, int32_t k, int32_t d);
int nanospec_draft_logits_topk(const void* rows, int32_t mode, const int32_t* row_ids,
                               const int32_t* n_dev, int32_t n_max, int32_t V,
                               int32_t d, int32_t dtype, const void* h, int32_t M,
                               int32_t k, float* logits, int32_t* topk_ids,
                               float* topk_vals, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* The two stages of nanospec_draft_logits_topk, for callers that place them
 * separately (and to time the projection on its own):
 *   nanospec_draft_project : the projection (Eq. 1 on the active rows) into
 *       the workspace's partial sums; same arguments as the whole call minus
 *       the outputs (k only sizes the workspace).
 *   nanospec_draft_select  : the merge of those partial sums, top-k and the
 *       map to global ids; writes logits / topk_ids / topk_vals exactly as
 *       the whole call.
 * select must follow a project call on the same workspace with the same
 * n_dev (NULL or not), n_max, d, dtype, M and k; the pair then gives
 * bit-identical results to nanospec_draft_logits_topk.  Errors as for the
 * whole call. */
int nanospec_draft_project(const void* rows, int32_t mode, const int32_t* row_ids,
                           const int32_t* n_dev, int32_t n_max, int32_t V, int32_t d,
                           int32_t dtype, const void* h, int32_t M, int32_t k, void* ws,
                           size_t ws_bytes, hipStream_t stream);
int nanospec_draft_select(const int32_t* row_ids, const int32_t* n_dev, int32_t n_max,
                          int32_t V, int32_t d, int32_t dtype, int32_t M, int32_t k,
                          float* logits, int32_t* topk_ids, float* topk_vals, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* Allocation-free variant of nanospec_draft_logits_topk, for callers that
 * cannot allocate device memory around the call (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, rules and results as nanospec_draft_logits_topk, without the
 * workspace: the kernels use a fixed device array of the library of
 * NS_NOALLOC_SCRATCH_BYTES (8 MiB), one copy per GPU, held until the process
 * ends.  The first call on a device (which must be the current device, the
 * device of `stream`) resolves that array's address with hipGetSymbolAddress
 * and keeps it; no call allocates or frees memory.  Every call on one GPU
 * shares the array, and it needs no initialisation; calls that may overlap
 * on one GPU (different streams without ordering between them) race on it
 * and must be ordered by the caller.
 * Errors: as nanospec_draft_logits_topk (but never NS_ECAPACITY), plus
 * NS_ESCRATCH when nanospec_draft_workspace_bytes(n_max, M, k, d) exceeds
 * NS_NOALLOC_SCRATCH_BYTES (nothing is enqueued): e.g. n_max = 3072 fits
 * every M <= 64 at d = 4096, n_max = 16384 fits M <= 16 only. */
#define NS_NOALLOC_SCRATCH_BYTES (8u << 20)
int nanospec_draft_logits_topk_noalloc(const void* rows, int32_t mode, const int32_t* row_ids,
                                       const int32_t* n_dev, int32_t n_max, int32_t V,
                                       int32_t d, int32_t dtype, const void* h, int32_t M,
                                       int32_t k, float* logits, int32_t* topk_ids,
                                       float* topk_vals, hipStream_t stream);

/* ======================================================================
 * The draft head for a batch of B independent sequences sharing W_head, in
 * NS_INDEXED mode: for every b, the result of nanospec_draft_logits_topk on
 * sequence b's inputs.  One pair of launches serves all B sequences, so a
 * call moves B times the bytes of a single-sequence call for the same launch
 * and round-trip latency.
 *   w        : W_head [V x d], shared.
 *   row_ids  : [B x n_max] (sequence b's active ids in row b), holes skipped.
 *   n_dev    : [B] device counts (required), each clamped to n_max.
 *   h        : [B x M x d]; logits : [B x M x n_max] or NULL;
 *   topk_ids, topk_vals : [B x M x k].
 *   ws       : >= nanospec_batch_draft_workspace_bytes(B, n_max, M, k, d)
 *              bytes, 256-byte aligned, no initialisation needed.
 * B in [1, NS_MAX_BATCH]; other limits and errors as for
 * nanospec_draft_logits_topk (NS_EINVAL also for n_dev == NULL). */
size_t nanospec_batch_draft_workspace_bytes(int32_t B, int32_t n_max, int32_t M, int32_t k, int32_t d);
int nanospec_batch_draft_logits_topk(const void* w, const int32_t* row_ids, const int32_t* n_dev,
                                     int32_t n_max, int32_t B, int32_t V, int32_t d, int32_t dtype,
                                     const void* h, int32_t M, int32_t k, float* logits,
                                     int32_t* topk_ids, float* topk_vals, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* ======================================================================
 * Draft head with log-probabilities over the active set, for tree drafting.
 * NanoSpec Sec. 4.1 (draft tree of depth 5) and its results discussion: with
 * a dynamic vocabulary the draft softmax is renormalised over I.  Same
 * arguments and rules as nanospec_draft_logits_topk, plus:
 *   parent : [M] float32 (device) or NULL (zeros): score of hidden row m's
 *            node in the tree;
 *   lse    : [M] float32 output or NULL: log(sum over active j of
 *            exp(z[m, j])), -INFINITY for an empty row;
 * and topk_vals[m, r] = parent[m] + z[m, j_r] - lse[m] for the same top-k
 * ids as the logits version (the shift does not change the order).  logits,
 * when given, receives the raw z.  lse is computed in float32: a max, then a
 * sum of exp(z - max) in a fixed order (per 4096-column chunk, combined in
 * chunk order), so results are deterministic.  The workspace is the same as
 * for nanospec_draft_logits_topk. */
int nanospec_draft_logprob_topk(const void* rows, int32_t mode, const int32_t* row_ids,
                                const int32_t* n_dev, int32_t n_max, int32_t V, int32_t d,
                                int32_t dtype, const void* h, int32_t M, int32_t k,
                                const float* parent, float* lse, float* logits,
                                int32_t* topk_ids, float* topk_vals, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* nanospec_draft_logprob_topk for B independent sequences sharing W_head, in
 * NS_INDEXED mode, with the batch layout of nanospec_batch_draft_logits_topk;
 * parent and lse are [B x M] (parent may be NULL).  Workspace:
 * nanospec_batch_draft_workspace_bytes. */
int nanospec_batch_draft_logprob_topk(const void* w, const int32_t* row_ids, const int32_t* n_dev,
                                      int32_t n_max, int32_t B, int32_t V, int32_t d, int32_t dtype,
                                      const void* h, int32_t M, int32_t k, const float* parent,
                                      float* lse, float* logits, int32_t* topk_ids, float* topk_vals,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/* ======================================================================
 * The decode step in one call (Sec. 3.2 decoding phase and sliding-window
 * rebuild, then Sec. 3.1 Eq. 1 on W_head[I_{t+1}, :] with T_k): the same
 * results as
 *   nanospec_step_update(st, draft_ids, n_draft, ver_ids, n_ver, active_ids,
 *                        n_active, NULL, stream);
 *   nanospec_draft_logits_topk(w, NS_INDEXED, active_ids, n_active, w_max,
 *                              V, d, dtype, h, M, k, NULL, topk_ids,
 *                              topk_vals, ws, ws_bytes, stream);
 * bit for bit (the logits output is not offered).  The state keeps I_t in
 * ascending order (cur) between decode steps.  When it holds I_t, dtype is
 * NS_BF16 or NS_FP16, W_max <= 3072 and a multiple of 4, n_draft + n_ver <=
 * 256 and V <= about 200k, the step takes two launches instead of three: the
 * state update runs beside the projection, which covers I_t and the tuple
 * entries (a superset of I_{t+1}), and the merge keeps only members of
 * I_{t+1}.  Otherwise the three launches run, followed by a copy of I_{t+1}
 * into cur when the shapes allow the two-launch form (and by nothing when
 * they do not: no I_t is kept then).  Any other call that changes the window or rebuilds I
 * (stream_append, active_vocab, step_update, batch_step_update, reset) drops
 * cur until the next decode step.
 *   w, V, d, dtype, h, M, k, topk_ids, topk_vals : as nanospec_draft_logits_topk
 *              in NS_INDEXED mode; V must be the state's V.
 *   ws       : >= nanospec_decode_step_workspace_bytes(w_max, n_draft + n_ver,
 *              M, k, d) bytes, 256-byte aligned.
 * Errors: NS_EINVAL (nulls, counts, limits, V mismatch), NS_EDTYPE,
 * NS_ECAPACITY, NS_EHIP (see the conventions on kernels already enqueued). */
size_t nanospec_decode_step_workspace_bytes(int32_t w_max, int32_t n_tuple, int32_t M, int32_t k, int32_t d);
int nanospec_decode_step(nanospec_state* st, const int32_t* draft_ids, int32_t n_draft,
                         const int32_t* ver_ids, int32_t n_ver, int32_t* active_ids,
                         int32_t* n_active, const void* w, int32_t V, int32_t d, int32_t dtype,
                         const void* h, int32_t M, int32_t k, int32_t* topk_ids, float* topk_vals,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* The two stages of nanospec_decode_step, for callers that place them
 * separately (and to time the first launch on its own):
 *   nanospec_decode_step_project : the state update and the projection
 *       (the fused first launch, or the state update and the projection
 *       stage of the three-launch form); same arguments as the whole call
 *       minus the outputs (k only sizes the workspace).  Records the form
 *       in the state's handle.
 *   nanospec_decode_step_select  : the merge, top-k and map to global ids,
 *       and the state's cur (and, in the fused form, I_{t+1} in active_ids /
 *       n_active, the state's bitmap and |S|); writes topk_ids / topk_vals
 *       exactly as the whole call.
 * select must follow project on the same state, workspace, active_ids and
 * n_active, with the same V, d, dtype, M and k (else NS_EINVAL, nothing
 * enqueued); the pair then gives bit-identical results to
 * nanospec_decode_step.  Between the two the state is mid-update: any other
 * call that changes it drops the pending step (select then returns
 * NS_EINVAL), and a fused project that is not followed by its select leaves
 * the window undefined until nanospec_state_reset.  Errors as for the whole
 * call. */
int nanospec_decode_step_project(nanospec_state* st, const int32_t* draft_ids, int32_t n_draft,
                                 const int32_t* ver_ids, int32_t n_ver, int32_t* active_ids,
                                 int32_t* n_active, const void* w, int32_t V, int32_t d,
                                 int32_t dtype, const void* h, int32_t M, int32_t k, void* ws,
                                 size_t ws_bytes, hipStream_t stream);
int nanospec_decode_step_select(nanospec_state* st, int32_t* active_ids, int32_t* n_active,
                                int32_t V, int32_t d, int32_t dtype, int32_t M, int32_t k,
                                int32_t* topk_ids, float* topk_vals, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* The decode step for B independent sequences in one call: the results of
 *   nanospec_batch_step_update(bt, draft_ids, draft_stride, n_draft, nd_max,
 *                              ver_ids, ver_stride, n_ver, nv_max,
 *                              active_ids, n_active, NULL, stream);
 *   nanospec_batch_draft_logits_topk(w, active_ids, n_active, w_max, B, V, d,
 *                                    dtype, h, M, k, NULL, topk_ids,
 *                                    topk_vals, ws, ws_bytes, stream);
 * bit for bit, for every sequence (Sec. 3.2 decoding phase and window
 * rebuild, then Sec. 3.1 Eq. 1 with T_k, per sequence).  Arguments and
 * layouts as in those two calls: sequence b's tuples at draft_ids + b *
 * draft_stride (n_draft[b] <= nd_max of them, device counts) and ver_ids + b *
 * ver_stride, its I_{t+1} at active_ids + b * w_max, its hidden rows at h + b
 * * M * d, its top-k at topk_ids / topk_vals + b * M * k.  When every member
 * keeps I_t (its previous step was a batched or single decode step) and the
 * shapes allow it (as for nanospec_decode_step, with nd_max + nv_max <= 256;
 * not for M <= 8 with B >= 32, where the separate batched head's taller tiles
 * are faster), the step takes two launches: one state-update block per sequence beside the
 * projection of the sequences' tuple and I_t columns, then the merge.
 * Otherwise the three separate launches run (and a copy of every I_{t+1}
 * into its state when the shapes allow the two-launch form).  A member in the
 * CTX_ONLY stream mode is refused, as by nanospec_batch_step_update.
 *   ws : >= nanospec_batch_decode_step_workspace_bytes(B, w_max,
 *        nd_max + nv_max, M, k, d) bytes, 256-byte aligned.
 * Errors: NS_EINVAL, NS_EDTYPE, NS_ECAPACITY, NS_EHIP (see the conventions on
 * kernels already enqueued). */
size_t nanospec_batch_decode_step_workspace_bytes(int32_t B, int32_t w_max, int32_t n_tuple,
                                                  int32_t M, int32_t k, int32_t d);
int nanospec_batch_decode_step(nanospec_batch* bt, const int32_t* draft_ids, int32_t draft_stride,
                               const int32_t* n_draft, int32_t nd_max, const int32_t* ver_ids,
                               int32_t ver_stride, const int32_t* n_ver, int32_t nv_max,
                               int32_t* active_ids, int32_t* n_active, const void* w, int32_t V,
                               int32_t d, int32_t dtype, const void* h, int32_t M, int32_t k,
                               int32_t* topk_ids, float* topk_vals, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Best-k selection over draft-tree candidates, B independent selections:
 *   vals, ids : [B x C] candidate scores and token ids (device); id -1 marks
 *               an empty candidate, which is never selected;
 *   out_idx   : [B x k] flat candidate indices of the k best, ordered by
 *               (score desc, flat index asc); out_vals / out_ids : their
 *               scores and token ids; padded with (-1, -INFINITY, -1) when
 *               fewer than k candidates exist.
 * Next frontier: the best F of the F x K children a depth's draft head wrote
 * ([F x K] row-major, so flat index / K is the parent slot); final tree: the
 * best N of all nodes kept so far.  C in [1, NS_MAX_TREE_CAND], k in
 * [1, NS_MAX_K], B in [1, NS_MAX_BATCH].
 * Errors: NS_EINVAL, NS_EHIP. */
int nanospec_tree_select(const float* vals, const int32_t* ids, int32_t C, int32_t B,
                         int32_t k, int32_t* out_idx, float* out_vals, int32_t* out_ids,
                         hipStream_t stream);

/* ======================================================================
 * Prefill candidates.  Sec. 3.2 prefill: P[i] = T_Kpre(z_i) for every prompt
 * position i.
 *   logits   : [L x V] target logits, NS_BF16, NS_FP16 or NS_FP32, row-major.
 *   out_ids  : [L x k] int32, out_vals : [L x k] float32 (exact: the stored
 *              logits widened to float32), each row ordered by (value desc,
 *              id asc).  out_ids may be fed to nanospec_stream_append with
 *              dedup_first = 1 to append tuple(U_i T_Kpre(z_i)), which orders
 *              the union position-major, rank-minor.
 * Errors: NS_EINVAL (nulls, L < 0, V < 1, k not in [1, min(64, V)]),
 * NS_EDTYPE, NS_EHIP.  L = 0 enqueues nothing. */
int nanospec_prefill_topk(const void* logits, int32_t L, int32_t V, int32_t dtype,
                          int32_t k, int32_t* out_ids, float* out_vals,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* NANOSPEC_H */
