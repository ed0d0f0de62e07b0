"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/nanospec.h, and rejects bad arguments on the host before
anything is enqueued (these calls return before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nanospec.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nanospec_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def ns():
    from dynamic_vocab_draft_amd import nanospec
    return nanospec


def test_header_declares_the_five_calls():
    names = declared_functions()
    for f in ["nanospec_stream_append", "nanospec_active_vocab", "nanospec_gather_rows",
              "nanospec_draft_logits_topk", "nanospec_prefill_topk"]:
        assert f in names


def test_library_exports_every_declared_symbol(ns):
    lib = ctypes.CDLL(ns.LIB_PATH)
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, missing


def test_binding_wraps_every_declared_symbol(ns):
    for f in declared_functions():
        assert f in ns._SIGS, f


def test_codes_and_sizes(ns):
    L = ns._lib
    assert L.nanospec_version() >= 100
    assert L.nanospec_strerror(0) == b"ok"
    assert L.nanospec_strerror(99) == b"unknown error code"
    assert L.nanospec_state_bytes(0, 10) == 0
    assert L.nanospec_state_bytes(10, 0) == 0
    assert L.nanospec_state_bytes(ns.NS_MAX_V + 1, 10) == 0
    b = L.nanospec_state_bytes(128256, 3072)
    # control + ring + first[V] + bitmap + the kept active set + the decode step's next bitmap
    # (ceil(V/32) rounded up to 8 words), each 256-byte aligned
    assert b == 256 + 12288 + 513024 + 16128 + 12288 + 16128
    assert L.nanospec_draft_workspace_bytes(3072, 8, 8, 4096) >= 3072 * 8 * 4
    assert L.nanospec_draft_workspace_bytes(3072, 65, 8, 4096) == 0
    assert L.nanospec_draft_workspace_bytes(3072, 8, 65, 4096) == 0
    assert L.nanospec_draft_workspace_bytes(3072, 8, 8, 4100) == 0      # d % 8 != 0
    # batches: B copies of one state; the batched workspace grows with B
    assert L.nanospec_batch_state_bytes(8, 128256, 3072) == 8 * b
    assert L.nanospec_batch_state_bytes(0, 128256, 3072) == 0
    assert L.nanospec_batch_state_bytes(ns.NS_MAX_BATCH + 1, 128256, 3072) == 0
    w1 = L.nanospec_batch_draft_workspace_bytes(1, 3072, 8, 8, 4096)
    assert w1 == L.nanospec_draft_workspace_bytes(3072, 8, 8, 4096)
    assert L.nanospec_batch_draft_workspace_bytes(8, 3072, 8, 8, 4096) >= 8 * 3072 * 8 * 4
    assert L.nanospec_batch_draft_workspace_bytes(0, 3072, 8, 8, 4096) == 0
    # the decode step: at least the separate draft head's workspace; the tuple bound is checked
    dw = L.nanospec_decode_step_workspace_bytes(3072, 68, 8, 8, 4096)
    assert dw >= L.nanospec_draft_workspace_bytes(3072, 8, 8, 4096) and dw % 256 == 0
    assert L.nanospec_decode_step_workspace_bytes(3072, -1, 8, 8, 4096) == 0
    assert L.nanospec_decode_step_workspace_bytes(3072, 68, 65, 8, 4096) == 0
    # the batched decode step: B regions of the decode step, at least the separate batched head's
    bw = L.nanospec_batch_decode_step_workspace_bytes(8, 3072, 68, 8, 8, 4096)
    assert bw >= L.nanospec_batch_draft_workspace_bytes(8, 3072, 8, 8, 4096) and bw % 256 == 0
    assert bw >= 8 * 3072 * 8 * 4 and bw > L.nanospec_batch_decode_step_workspace_bytes(1, 3072, 68, 8, 8, 4096)
    assert L.nanospec_batch_decode_step_workspace_bytes(0, 3072, 68, 8, 8, 4096) == 0
    assert L.nanospec_batch_decode_step_workspace_bytes(ns.NS_MAX_BATCH + 1, 3072, 68, 8, 8, 4096) == 0
    assert L.nanospec_batch_decode_step_workspace_bytes(8, 3072, -1, 8, 8, 4096) == 0


def test_host_validation_rejects_before_launch(ns):
    L = ns._lib
    fake = ctypes.c_void_p(0x1000)        # never dereferenced: validation fails first
    h = ctypes.c_void_p()
    assert L.nanospec_state_create(None, 10, 4, fake, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_state_create(ctypes.byref(h), 10, 4, None, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_state_create(ctypes.byref(h), 10, 4, ctypes.c_void_p(0x1010), 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_state_create(ctypes.byref(h), 10, 4, fake, 16, None) == ns.NS_ECAPACITY
    assert L.nanospec_stream_append(None, fake, 3, 1, None) == ns.NS_EINVAL
    assert L.nanospec_active_vocab(None, fake, fake, None, None) == ns.NS_EINVAL
    assert L.nanospec_state_status(None, None, None) == ns.NS_EINVAL
    assert L.nanospec_state_destroy(None) == ns.NS_EINVAL
    assert L.nanospec_decode_step(None, fake, 3, fake, 1, fake, fake, fake, 100, 64, ns.NS_BF16, fake, 8, 8, fake,
                                  fake, fake, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_decode_step_project(None, fake, 3, fake, 1, fake, fake, fake, 100, 64, ns.NS_BF16, fake, 8, 8,
                                          fake, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_decode_step_select(None, fake, fake, 100, 64, ns.NS_BF16, 8, 8, fake, fake, fake, 1 << 20,
                                         None) == ns.NS_EINVAL
    assert L.nanospec_batch_decode_step(None, fake, 3, fake, 3, fake, 1, fake, 1, fake, fake, fake, 100, 64,
                                        ns.NS_BF16, fake, 8, 8, fake, fake, fake, 1 << 20, None) == ns.NS_EINVAL
    # gather: null, bad d, bad dtype, misaligned
    assert L.nanospec_gather_rows(None, 10, 8, 0, fake, None, 4, fake, None) == ns.NS_EINVAL
    assert L.nanospec_gather_rows(fake, 10, 12, 0, fake, None, 4, fake, None) == ns.NS_EINVAL
    assert L.nanospec_gather_rows(fake, 10, 8, 7, fake, None, 4, fake, None) == ns.NS_EDTYPE
    assert L.nanospec_gather_rows(ctypes.c_void_p(0x1008), 10, 8, 0, fake, None, 4, fake, None) == ns.NS_EINVAL
    # draft head
    args = dict(rows=fake, mode=0, row_ids=fake, n_dev=None, n_max=16, V=100, d=64, dtype=0, h=fake, M=8, k=8,
                logits=None, ids=fake, vals=fake, ws=fake, ws_bytes=1 << 20)

    def call(**kw):
        a = dict(args, **kw)
        return L.nanospec_draft_logits_topk(a["rows"], a["mode"], a["row_ids"], a["n_dev"], a["n_max"], a["V"],
                                            a["d"], a["dtype"], a["h"], a["M"], a["k"], a["logits"], a["ids"],
                                            a["vals"], a["ws"], a["ws_bytes"], None)
    assert call(mode=5) == ns.NS_EDTYPE
    assert call(dtype=3) == ns.NS_EDTYPE
    assert call(M=0) == ns.NS_EINVAL
    assert call(M=65) == ns.NS_EINVAL
    assert call(k=0) == ns.NS_EINVAL
    assert call(k=65) == ns.NS_EINVAL
    assert call(d=60) == ns.NS_EINVAL
    assert call(mode=1, row_ids=None) == ns.NS_EINVAL
    assert call(h=None) == ns.NS_EINVAL
    assert call(ws_bytes=64) == ns.NS_ECAPACITY
    assert call(ws=ctypes.c_void_p(0x1010)) == ns.NS_EINVAL
    # batches
    assert L.nanospec_batch_create(None, 2, 10, 4, fake, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_batch_create(ctypes.byref(h), 0, 10, 4, fake, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_batch_create(ctypes.byref(h), 2, 10, 4, fake, 16, None) == ns.NS_ECAPACITY
    assert L.nanospec_batch_destroy(None) == ns.NS_EINVAL
    assert L.nanospec_batch_member(None, 0, ctypes.byref(h)) == ns.NS_EINVAL
    assert L.nanospec_batch_step_update(None, fake, 8, fake, 8, fake, 8, fake, 8, fake, fake, None,
                                        None) == ns.NS_EINVAL
    assert L.nanospec_batch_draft_logits_topk(fake, fake, None, 16, 2, 100, 64, 0, fake, 8, 8, None, fake, fake,
                                              fake, 1 << 20, None) == ns.NS_EINVAL       # n_dev required
    assert L.nanospec_batch_draft_logits_topk(fake, fake, fake, 16, 0, 100, 64, 0, fake, 8, 8, None, fake, fake,
                                              fake, 1 << 20, None) == ns.NS_EINVAL       # B = 0
    # two-stage draft head
    assert L.nanospec_draft_project(fake, 0, fake, None, 16, 100, 60, 0, fake, 8, 8, fake, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_draft_project(fake, 1, None, None, 16, 100, 64, 0, fake, 8, 8, fake, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_draft_project(fake, 0, fake, None, 16, 100, 64, 0, fake, 8, 8, fake, 64, None) == ns.NS_ECAPACITY
    assert L.nanospec_draft_select(fake, None, 16, 100, 64, 0, 8, 8, None, None, fake, fake, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_draft_select(fake, None, 16, 100, 64, 3, 8, 8, None, fake, fake, fake, 1 << 20, None) == ns.NS_EDTYPE
    assert L.nanospec_draft_select(fake, None, 16, 100, 64, 0, 8, 8, None, fake, fake, fake, 64, None) == ns.NS_ECAPACITY
    # log-prob head and tree selection
    assert L.nanospec_batch_draft_logprob_topk(fake, fake, None, 16, 2, 100, 64, 0, fake, 8, 8, None, None, None,
                                               fake, fake, fake, 1 << 20, None) == ns.NS_EINVAL   # n_dev required
    assert L.nanospec_draft_logprob_topk(fake, 5, fake, None, 16, 100, 64, 0, fake, 8, 8, None, None, None, fake,
                                         fake, fake, 1 << 20, None) == ns.NS_EDTYPE               # bad mode
    assert L.nanospec_tree_select(fake, fake, 0, 1, 8, fake, fake, fake, None) == ns.NS_EINVAL
    assert L.nanospec_tree_select(fake, fake, ns.NS_MAX_TREE_CAND + 1, 1, 8, fake, fake, fake, None) == ns.NS_EINVAL
    assert L.nanospec_tree_select(fake, fake, 10, 1, 65, fake, fake, fake, None) == ns.NS_EINVAL
    assert L.nanospec_tree_select(None, fake, 10, 1, 8, fake, fake, fake, None) == ns.NS_EINVAL
    # stream modes
    assert L.nanospec_state_set_mode(None, ns.NS_STREAM_CTX_ONLY) == ns.NS_EINVAL
    # slot-stable packed buffer
    pb = L.nanospec_packed_bytes(128256, 3072)
    assert pb == 256 + 3 * 12288 + 16128          # header, three [w_max] int32 arrays, bitmap (256-aligned)
    assert L.nanospec_packed_bytes(0, 16) == 0
    assert L.nanospec_packed_bytes(100, 0) == 0
    assert L.nanospec_packed_bytes(100, ns.NS_MAX_SLOTS + 1) == 0
    assert L.nanospec_packed_bytes(100, ns.NS_MAX_SLOTS) > 0
    assert L.nanospec_packed_create(None, 10, 4, fake, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_packed_create(ctypes.byref(h), 10, 4, None, 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_packed_create(ctypes.byref(h), 10, 4, ctypes.c_void_p(0x1010), 1 << 20, None) == ns.NS_EINVAL
    assert L.nanospec_packed_create(ctypes.byref(h), 10, 4, fake, 16, None) == ns.NS_ECAPACITY
    assert L.nanospec_packed_create(ctypes.byref(h), 10, ns.NS_MAX_SLOTS + 1, fake, 1 << 30, None) == ns.NS_EINVAL
    assert L.nanospec_packed_update(None, fake, fake, 64, 0, fake, None) == ns.NS_EINVAL
    assert L.nanospec_packed_reset(None, None) == ns.NS_EINVAL
    assert L.nanospec_packed_destroy(None) == ns.NS_EINVAL
    assert L.nanospec_packed_slots(None, None, None, None, None, None) == ns.NS_EINVAL
    # prefill
    assert L.nanospec_prefill_topk(fake, 4, 10, 0, 0, fake, fake, None) == ns.NS_EINVAL
    assert L.nanospec_prefill_topk(fake, 4, 10, 0, 11, fake, fake, None) == ns.NS_EINVAL
    assert L.nanospec_prefill_topk(fake, 4, 10, 9, 2, fake, fake, None) == ns.NS_EDTYPE
    assert L.nanospec_prefill_topk(None, 4, 10, 0, 2, fake, fake, None) == ns.NS_EINVAL
    assert L.nanospec_prefill_topk(None, 0, 10, 0, 2, fake, fake, None) == ns.NS_OK   # L = 0: nothing to do


def test_noalloc_rejects_oversize_before_launch(ns):
    """The allocation-free draft head refuses a workspace need above its fixed
    scratch (NS_ESCRATCH) and bad dimensions (NS_EINVAL) before any HIP call."""
    L = ns._lib
    fake = ctypes.c_void_p(0x1000)
    need = L.nanospec_draft_workspace_bytes(16384, 64, 16, 4096)
    assert need > ns.NS_NOALLOC_SCRATCH_BYTES
    assert L.nanospec_draft_logits_topk_noalloc(fake, ns.NS_INDEXED, fake, fake, 16384, 151936, 4096, ns.NS_BF16,
                                                fake, 64, 16, None, fake, fake, None) == ns.NS_ESCRATCH
    assert L.nanospec_draft_logits_topk_noalloc(fake, ns.NS_INDEXED, fake, fake, 3072, 128256, 4096, ns.NS_BF16,
                                                fake, 65, 8, None, fake, fake, None) == ns.NS_EINVAL
    # the workloads the header names as fitting do fit
    for n_max, M, k in ((3072, 64, 16), (3072, 8, 8), (16384, 16, 16)):
        assert L.nanospec_draft_workspace_bytes(n_max, M, k, 4096) <= ns.NS_NOALLOC_SCRATCH_BYTES
    assert L.nanospec_strerror(ns.NS_ESCRATCH) != b"unknown error code"
