// Host-side memory and undefined-behaviour checks of libnanospec, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on its host code by
// tests/test_sanitizers.py and run on a machine WITHOUT a GPU.
//
// Three groups of calls, none of which can reach a device:
//  * the size queries over edge and out-of-range arguments;
//  * argument errors, rejected on the host before anything is enqueued;
//  * calls that pass the argument checks with placeholder device addresses,
//    so that the host planning (slice counts, tile shapes, workspace layout,
//    kernel choice) runs for every shape class and stops at the first HIP
//    call, which fails for want of a device (NS_EHIP).
// The placeholder addresses are never dereferenced on the host.  Exit status
// 0 when every check passes.
#include <stdint.h>
#include <stdio.h>

#include "nanospec.h"

#define CHECK(c)                                                                \
  do {                                                                          \
    if (!(c)) {                                                                 \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);     \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

namespace {

// Aligned placeholder device addresses (never dereferenced on the host).
void* fake(uintptr_t i) { return (void*)(uintptr_t)(0x100000u + 0x1000u * i); }

int check_sizes() {
  for (int c = -3; c <= 12; ++c) CHECK(nanospec_strerror(c) != nullptr);
  CHECK(nanospec_version() >= 100);
  const int32_t Vs[] = {INT32_MIN, -1, 0, 1, 31, 32, 33, 70, 2048, 128256, 151936, NS_MAX_V, NS_MAX_V + 1,
                        INT32_MAX};
  const int32_t Ws[] = {INT32_MIN, -1, 0, 1, 3, 512, 3072, 16384, NS_MAX_WMAX, NS_MAX_WMAX + 1, INT32_MAX};
  const int32_t Bs[] = {INT32_MIN, -1, 0, 1, 8, 64, NS_MAX_BATCH, NS_MAX_BATCH + 1, INT32_MAX};
  for (int32_t V : Vs)
    for (int32_t w : Ws) {
      const bool ok = V >= 1 && V <= NS_MAX_V && w >= 1 && w <= NS_MAX_WMAX;
      const size_t b = nanospec_state_bytes(V, w);
      CHECK(ok ? (b > 0 && b % 256 == 0) : b == 0);
      for (int32_t B : Bs) {
        const size_t bb = nanospec_batch_state_bytes(B, V, w);
        CHECK((ok && B >= 1 && B <= NS_MAX_BATCH) ? bb == (size_t)B * b : bb == 0);
      }
      const size_t pb = nanospec_packed_bytes(V, w);
      CHECK((V >= 1 && V <= NS_MAX_V && w >= 1 && w <= NS_MAX_SLOTS) ? pb > 0 : pb == 0);
    }
  const int32_t Ns[] = {INT32_MIN, -1, 0, 1, 15, 16, 17, 1000, 3072, 4096, 4097, 16384, 65536, NS_MAX_WMAX,
                        NS_MAX_WMAX + 1, INT32_MAX};
  const int32_t Ms[] = {-1, 0, 1, 8, 16, 17, 32, 33, 48, 49, 60, 64, 65};
  const int32_t Ks[] = {-1, 0, 1, 8, 16, 64, 65};
  const int32_t Ds[] = {INT32_MIN, -8, 0, 4, 8, 256, 3584, 4096, 4100, NS_MAX_D, NS_MAX_D + 8, INT32_MAX};
  for (int32_t n : Ns)
    for (int32_t M : Ms)
      for (int32_t k : Ks)
        for (int32_t d : Ds) {
          const size_t w = nanospec_draft_workspace_bytes(n, M, k, d);
          if (M < 1 || M > NS_MAX_M || k < 1 || k > NS_MAX_K || d < 8 || d % 8 || d > NS_MAX_D || n < 1 ||
              n > NS_MAX_V)
            CHECK(w == 0);
          else if (n <= 65536)
            CHECK(w >= (size_t)n * M * 4);
          for (int32_t B : Bs) {
            const size_t wb = nanospec_batch_draft_workspace_bytes(B, n, M, k, d);
            if (B < 1 || B > NS_MAX_BATCH || w == 0) CHECK(wb == 0);
            else if (B == 1) CHECK(wb == w);
            // the batched decode step: zero exactly where the separate batched head's is (for a valid
            // tuple bound and n <= NS_MAX_WMAX), else at least as large
            if (n <= NS_MAX_WMAX) {
              const size_t wd = nanospec_batch_decode_step_workspace_bytes(B, n, 68, M, k, d);
              CHECK(wb == 0 ? wd == 0 : (wd >= wb && wd % 256 == 0));
              CHECK(nanospec_batch_decode_step_workspace_bytes(B, n, -1, M, k, d) == 0);
            }
          }
        }
  return 0;
}

int check_rejections() {
  nanospec_state* st = nullptr;
  CHECK(nanospec_state_create(nullptr, 10, 4, fake(0), 1 << 20, nullptr) == NS_EINVAL);
  CHECK(nanospec_state_create(&st, 10, 4, nullptr, 1 << 20, nullptr) == NS_EINVAL);
  CHECK(nanospec_state_create(&st, 0, 4, fake(0), 1 << 20, nullptr) == NS_EINVAL);
  CHECK(nanospec_state_create(&st, 10, 0, fake(0), 1 << 20, nullptr) == NS_EINVAL);
  CHECK(nanospec_state_create(&st, 10, 4, (char*)fake(0) + 16, 1 << 20, nullptr) == NS_EINVAL);
  CHECK(nanospec_state_create(&st, 10, 4, fake(0), 16, nullptr) == NS_ECAPACITY);
  CHECK(st == nullptr);
  CHECK(nanospec_state_reset(nullptr, nullptr) == NS_EINVAL);
  CHECK(nanospec_state_destroy(nullptr) == NS_EINVAL);
  CHECK(nanospec_state_set_mode(nullptr, NS_STREAM_FULL) == NS_EINVAL);
  uint32_t flags = 0;
  CHECK(nanospec_state_status(nullptr, &flags, nullptr) == NS_EINVAL);
  CHECK(nanospec_state_window(nullptr, (int32_t*)fake(1), nullptr, nullptr) == NS_EINVAL);
  CHECK(nanospec_stream_append(nullptr, (const int32_t*)fake(1), 3, 1, nullptr) == NS_EINVAL);
  CHECK(nanospec_active_vocab(nullptr, (int32_t*)fake(1), (int32_t*)fake(2), nullptr, nullptr) == NS_EINVAL);
  CHECK(nanospec_step_update(nullptr, nullptr, 0, nullptr, 0, (int32_t*)fake(1), (int32_t*)fake(2), nullptr,
                             nullptr) == NS_EINVAL);
  nanospec_batch* bt = nullptr;
  CHECK(nanospec_batch_create(&bt, 0, 10, 4, fake(0), 1 << 20, nullptr) == NS_EINVAL);
  CHECK(nanospec_batch_create(&bt, NS_MAX_BATCH + 1, 10, 4, fake(0), 1 << 20, nullptr) == NS_EINVAL);
  CHECK(nanospec_batch_create(&bt, 2, 10, 4, fake(0), 16, nullptr) == NS_ECAPACITY);
  CHECK(nanospec_batch_destroy(nullptr) == NS_EINVAL);
  CHECK(nanospec_batch_member(nullptr, 0, &st) == NS_EINVAL);
  CHECK(nanospec_batch_step_update(nullptr, (const int32_t*)fake(1), 4, (const int32_t*)fake(2), 4,
                                   (const int32_t*)fake(3), 4, (const int32_t*)fake(4), 4, (int32_t*)fake(5),
                                   (int32_t*)fake(6), nullptr, nullptr) == NS_EINVAL);
  CHECK(nanospec_batch_decode_step(nullptr, (const int32_t*)fake(1), 4, (const int32_t*)fake(2), 4,
                                   (const int32_t*)fake(3), 4, (const int32_t*)fake(4), 4, (int32_t*)fake(5),
                                   (int32_t*)fake(6), fake(7), 100, 64, NS_BF16, fake(8), 8, 8, (int32_t*)fake(9),
                                   (float*)fake(10), fake(11), 1 << 20, nullptr) == NS_EINVAL);
  nanospec_packed* pk = nullptr;
  CHECK(nanospec_packed_create(&pk, 10, 0, fake(0), 1 << 20, nullptr) == NS_EINVAL);
  CHECK(nanospec_packed_create(&pk, 10, 4, fake(0), 16, nullptr) == NS_ECAPACITY);
  CHECK(nanospec_packed_reset(nullptr, nullptr) == NS_EINVAL);
  CHECK(nanospec_packed_destroy(nullptr) == NS_EINVAL);
  CHECK(nanospec_packed_slots(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == NS_EINVAL);
  CHECK(nanospec_packed_update(nullptr, nullptr, fake(1), 8, NS_BF16, fake(2), nullptr) == NS_EINVAL);
  // Gather: element type, d and sizes.
  CHECK(nanospec_gather_rows(fake(0), 10, 8, 7, (const int32_t*)fake(1), nullptr, 4, fake(2), nullptr) == NS_EDTYPE);
  CHECK(nanospec_gather_rows(fake(0), 10, 12, NS_BF16, (const int32_t*)fake(1), nullptr, 4, fake(2), nullptr) ==
        NS_EINVAL);
  CHECK(nanospec_gather_rows(nullptr, 10, 8, NS_BF16, (const int32_t*)fake(1), nullptr, 4, fake(2), nullptr) ==
        NS_EINVAL);
  CHECK(nanospec_gather_rows(fake(0), 0, 8, NS_BF16, (const int32_t*)fake(1), nullptr, 4, fake(2), nullptr) ==
        NS_EINVAL);
  // Draft head: mode, element type, limits, alignment, workspace size.
  const size_t ws = nanospec_draft_workspace_bytes(64, 8, 8, 64);
  CHECK(ws > 0);
  int32_t* ids = (int32_t*)fake(3);
  float* vals = (float*)fake(4);
  CHECK(nanospec_draft_logits_topk(fake(0), 5, ids, nullptr, 64, 100, 64, NS_BF16, fake(1), 8, 8, nullptr, ids,
                                   vals, fake(2), ws, nullptr) == NS_EDTYPE);
  CHECK(nanospec_draft_logits_topk(fake(0), NS_INDEXED, ids, nullptr, 64, 100, 64, 9, fake(1), 8, 8, nullptr, ids,
                                   vals, fake(2), ws, nullptr) == NS_EDTYPE);
  CHECK(nanospec_draft_logits_topk(fake(0), NS_INDEXED, nullptr, nullptr, 64, 100, 64, NS_BF16, fake(1), 8, 8,
                                   nullptr, ids, vals, fake(2), ws, nullptr) == NS_EINVAL);
  CHECK(nanospec_draft_logits_topk(fake(0), NS_PACKED, nullptr, nullptr, 64, 100, 64, NS_BF16, fake(1), 65, 8,
                                   nullptr, ids, vals, fake(2), ws, nullptr) == NS_EINVAL);
  CHECK(nanospec_draft_logits_topk(fake(0), NS_PACKED, nullptr, nullptr, 64, 100, 64, NS_BF16, fake(1), 8, 65,
                                   nullptr, ids, vals, fake(2), ws, nullptr) == NS_EINVAL);
  CHECK(nanospec_draft_logits_topk(fake(0), NS_PACKED, nullptr, nullptr, 64, 100, 60, NS_BF16, fake(1), 8, 8,
                                   nullptr, ids, vals, fake(2), ws, nullptr) == NS_EINVAL);
  CHECK(nanospec_draft_logits_topk((char*)fake(0) + 8, NS_PACKED, nullptr, nullptr, 64, 100, 64, NS_BF16, fake(1),
                                   8, 8, nullptr, ids, vals, fake(2), ws, nullptr) == NS_EINVAL);
  CHECK(nanospec_draft_logits_topk(fake(0), NS_PACKED, nullptr, nullptr, 64, 100, 64, NS_BF16, fake(1), 8, 8,
                                   nullptr, ids, vals, (char*)fake(2) + 128, ws, nullptr) == NS_EINVAL);
  CHECK(nanospec_draft_logits_topk(fake(0), NS_PACKED, nullptr, nullptr, 64, 100, 64, NS_BF16, fake(1), 8, 8,
                                   nullptr, ids, vals, fake(2), ws - 1, nullptr) == NS_ECAPACITY);
  CHECK(nanospec_draft_logits_topk(fake(0), NS_PACKED, nullptr, nullptr, 64, 100, 64, NS_BF16, fake(1), 8, 8,
                                   nullptr, nullptr, vals, fake(2), ws, nullptr) == NS_EINVAL);
  CHECK(nanospec_draft_select(ids, nullptr, 64, 100, 64, NS_BF16, 8, 8, nullptr, ids, vals, fake(2), ws - 1,
                              nullptr) == NS_ECAPACITY);
  CHECK(nanospec_batch_draft_logits_topk(fake(0), ids, nullptr, 64, 2, 100, 64, NS_BF16, fake(1), 8, 8, nullptr, ids,
                                         vals, fake(2), ws * 4, nullptr) == NS_EINVAL);
  CHECK(nanospec_draft_logits_topk_noalloc(fake(0), NS_PACKED, nullptr, nullptr, 16384, 100, 4096, NS_BF16,
                                           fake(1), 64, 8, nullptr, ids, vals, nullptr) == NS_ESCRATCH);
  CHECK(nanospec_draft_logits_topk_noalloc(fake(0), NS_PACKED, nullptr, nullptr, 64, 100, 64, NS_BF16, fake(1), 0,
                                           8, nullptr, ids, vals, nullptr) == NS_EINVAL);
  // Tree selection and prefill.
  CHECK(nanospec_tree_select((const float*)fake(0), ids, 0, 1, 4, ids, vals, ids, nullptr) == NS_EINVAL);
  CHECK(nanospec_tree_select((const float*)fake(0), ids, NS_MAX_TREE_CAND + 1, 1, 4, ids, vals, ids, nullptr) ==
        NS_EINVAL);
  CHECK(nanospec_prefill_topk(fake(0), 4, 100, 7, 4, ids, vals, nullptr) == NS_EDTYPE);
  CHECK(nanospec_prefill_topk(fake(0), -1, 100, NS_BF16, 4, ids, vals, nullptr) == NS_EINVAL);
  CHECK(nanospec_prefill_topk(fake(0), 4, 100, NS_BF16, 65, ids, vals, nullptr) == NS_EINVAL);
  CHECK(nanospec_prefill_topk(fake(0), 4, 3, NS_BF16, 4, ids, vals, nullptr) == NS_EINVAL);
  CHECK(nanospec_prefill_topk(nullptr, 0, 100, NS_BF16, 4, ids, vals, nullptr) == NS_OK);   // L = 0: nothing
  return 0;
}

// Calls that pass every argument check: the host plans the launch and the
// first HIP call fails (no device).
int check_plans() {
  const int32_t Ns[] = {1, 15, 16, 17, 100, 967, 1024, 3072, 4096, 4097, 8192, 16384, 40000};
  const int32_t Ms[] = {1, 4, 8, 16, 17, 32, 33, 48, 49, 60, 64};
  const int32_t Ds[] = {8, 24, 256, 3584, 4096, NS_MAX_D};
  const int32_t Ts[] = {NS_BF16, NS_FP16, NS_FP32};
  int planned = 0;
  for (int32_t n : Ns)
    for (int32_t M : Ms)
      for (int32_t d : Ds)
        for (int32_t dt : Ts)
          for (int with_n = 0; with_n < 2; ++with_n) {
            const int32_t k = M % 3 == 0 ? 16 : 8;
            const size_t ws = nanospec_draft_workspace_bytes(n, M, k, d);
            CHECK(ws > 0);
            const int32_t* nd = with_n ? (const int32_t*)fake(5) : nullptr;
            int rc = nanospec_draft_logits_topk(fake(0), NS_INDEXED, (const int32_t*)fake(1), nd, n, 151936, d, dt,
                                                fake(2), M, k, nullptr, (int32_t*)fake(3), (float*)fake(4),
                                                fake(6), ws, nullptr);
            CHECK(rc == NS_EHIP || (dt == NS_FP32 && rc == NS_EINVAL));
            if (rc == NS_EINVAL) continue;
            ++planned;
            rc = nanospec_draft_select((const int32_t*)fake(1), nd, n, 151936, d, dt, M, k, (float*)fake(7),
                                       (int32_t*)fake(3), (float*)fake(4), fake(6), ws, nullptr);
            CHECK(rc == NS_EHIP);
            rc = nanospec_draft_logprob_topk(fake(0), NS_PACKED, nullptr, nd, n, n, d, dt, fake(2), M, k, nullptr,
                                             (float*)fake(8), nullptr, (int32_t*)fake(3), (float*)fake(4), fake(6),
                                             ws, nullptr);
            CHECK(rc == NS_EHIP);
            if (n <= 4097 && d <= 4096) {
              const int32_t B = n <= 1024 ? 64 : 3;
              const size_t wsb = nanospec_batch_draft_workspace_bytes(B, n, M, k, d);
              CHECK(wsb > 0);
              rc = nanospec_batch_draft_logits_topk(fake(0), (const int32_t*)fake(1), (const int32_t*)fake(5), n, B,
                                                    151936, d, dt, fake(2), M, k, nullptr, (int32_t*)fake(3),
                                                    (float*)fake(4), fake(6), wsb, nullptr);
              CHECK(rc == NS_EHIP);
            }
          }
  CHECK(planned > 0);
  for (int32_t dt : Ts) {
    CHECK(nanospec_gather_rows(fake(0), 128256, 4096, dt, (const int32_t*)fake(1), (const int32_t*)fake(2), 3072,
                               fake(3), nullptr) == NS_EHIP);
    CHECK(nanospec_prefill_topk(fake(0), 4096, 128256, dt, 4, (int32_t*)fake(1), (float*)fake(2), nullptr) ==
          NS_EHIP);
    CHECK(nanospec_prefill_topk(fake(0), 7, 101, dt, 64, (int32_t*)fake(1), (float*)fake(2), nullptr) == NS_EHIP);
  }
  // Extreme sizes: grids and pitches computed from them stay in range.
  CHECK(nanospec_gather_rows(fake(0), INT32_MAX, NS_MAX_D, NS_FP32, (const int32_t*)fake(1), nullptr, INT32_MAX,
                             fake(3), nullptr) == NS_EHIP);
  CHECK(nanospec_prefill_topk(fake(0), INT32_MAX, INT32_MAX, NS_FP32, 64, (int32_t*)fake(1), (float*)fake(2),
                              nullptr) == NS_EHIP);
  for (int32_t M : {1, 8, 64}) {
    const size_t ws = nanospec_draft_workspace_bytes(NS_MAX_V, M, 64, NS_MAX_D);
    CHECK(ws > 0);
    CHECK(nanospec_draft_logits_topk(fake(0), NS_PACKED, nullptr, (const int32_t*)fake(5), NS_MAX_V, NS_MAX_V,
                                     NS_MAX_D, NS_BF16, fake(2), M, 64, nullptr, (int32_t*)fake(3), (float*)fake(4),
                                     fake(6), ws, nullptr) == NS_EHIP);
    CHECK(nanospec_draft_logits_topk(fake(0), NS_PACKED, nullptr, nullptr, NS_MAX_V + 1, NS_MAX_V, NS_MAX_D,
                                     NS_BF16, fake(2), M, 64, nullptr, (int32_t*)fake(3), (float*)fake(4), fake(6),
                                     ws, nullptr) == NS_EINVAL);
  }
  CHECK(nanospec_tree_select((const float*)fake(0), (const int32_t*)fake(1), 100, 10, 10, (int32_t*)fake(2),
                             (float*)fake(3), (int32_t*)fake(4), nullptr) == NS_EHIP);
  nanospec_state* st = nullptr;
  CHECK(nanospec_state_create(&st, 128256, 3072, fake(0), nanospec_state_bytes(128256, 3072), nullptr) == NS_EHIP);
  CHECK(st == nullptr);
  nanospec_batch* bt = nullptr;
  CHECK(nanospec_batch_create(&bt, 4, 2048, 512, fake(0), nanospec_batch_state_bytes(4, 2048, 512), nullptr) ==
        NS_EHIP);
  CHECK(bt == nullptr);
  CHECK(nanospec_draft_logits_topk_noalloc(fake(0), NS_PACKED, nullptr, nullptr, 3072, 3072, 4096, NS_BF16, fake(1),
                                           8, 8, nullptr, (int32_t*)fake(2), (float*)fake(3), nullptr) == NS_EHIP);
  return 0;
}

}  // namespace

int main() {
  if (check_sizes()) return 1;
  if (check_rejections()) return 1;
  if (check_plans()) return 1;
  printf("host checks passed\n");
  return 0;
}
