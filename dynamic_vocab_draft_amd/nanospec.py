"""Thin ctypes binding of libnanospec.so (include/nanospec.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Functions keep the C names and take torch tensors (device memory)
plus an optional ``torch.cuda.Stream``; they raise ``NanoSpecError`` on a
non-zero return code.  The library must have been built
(``python -m dynamic_vocab_draft_amd.build``); importing this module without
it raises, and there is no fallback.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (same SONAME), and the two share
streams and device memory.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnanospec.so")

NS_OK, NS_EINVAL, NS_EDTYPE, NS_ECAPACITY, NS_EHIP, NS_ESCRATCH = 0, 1, 2, 3, 4, 5
NS_NOALLOC_SCRATCH_BYTES = 8 << 20
NS_BF16, NS_FP32, NS_FP16 = 0, 1, 2
NS_PACKED, NS_INDEXED = 0, 1
NS_STATUS_BAD_ID = 0x1
NS_STREAM_FULL, NS_STREAM_CTX_ONLY, NS_STREAM_EXT_ONLY = 0, 1, 2
NS_MAX_M = NS_MAX_K = 64
NS_MAX_V = NS_MAX_WMAX = 1 << 20
NS_MAX_D = 16384
NS_MAX_BATCH = 4096
NS_MAX_SLOTS = 16384
NS_MAX_TREE_CAND = 4096


class NanoSpecError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {code} ({_strerror(code)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing; build it with `python -m dynamic_vocab_draft_amd.build`")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_LOCAL)
    _check_single_runtime()
    return lib


def _check_single_runtime() -> None:
    """Fails if two different HIP runtimes ended up in this process."""
    try:
        with open("/proc/self/maps") as f:
            paths = {l.split()[-1] for l in f if "libamdhip64" in l}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise ImportError(f"more than one HIP runtime loaded: {sorted(real)}")


_lib = _load()

c_int32, c_size, c_vp, c_u32p = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32)

_SIGS = {
    "nanospec_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "nanospec_version": (ctypes.c_int, []),
    "nanospec_state_bytes": (c_size, [c_int32, c_int32]),
    "nanospec_state_create": (ctypes.c_int, [ctypes.POINTER(c_vp), c_int32, c_int32, c_vp, c_size, c_vp]),
    "nanospec_state_reset": (ctypes.c_int, [c_vp, c_vp]),
    "nanospec_state_destroy": (ctypes.c_int, [c_vp]),
    "nanospec_state_set_mode": (ctypes.c_int, [c_vp, c_int32]),
    "nanospec_state_status": (ctypes.c_int, [c_vp, c_u32p, c_vp]),
    "nanospec_state_window": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp]),
    "nanospec_stream_append": (ctypes.c_int, [c_vp, c_vp, c_int32, c_int32, c_vp]),
    "nanospec_active_vocab": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp]),
    "nanospec_step_update": (ctypes.c_int, [c_vp, c_vp, c_int32, c_vp, c_int32, c_vp, c_vp, c_vp, c_vp]),
    "nanospec_gather_rows": (ctypes.c_int, [c_vp, c_int32, c_int32, c_int32, c_vp, c_vp, c_int32, c_vp, c_vp]),
    "nanospec_draft_workspace_bytes": (c_size, [c_int32, c_int32, c_int32, c_int32]),
    "nanospec_draft_logits_topk": (ctypes.c_int, [c_vp, c_int32, c_vp, c_vp, c_int32, c_int32, c_int32, c_int32,
                                                  c_vp, c_int32, c_int32, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "nanospec_draft_logits_topk_noalloc": (ctypes.c_int, [c_vp, c_int32, c_vp, c_vp, c_int32, c_int32, c_int32,
                                                          c_int32, c_vp, c_int32, c_int32, c_vp, c_vp, c_vp, c_vp]),
    "nanospec_prefill_topk": (ctypes.c_int, [c_vp, c_int32, c_int32, c_int32, c_int32, c_vp, c_vp, c_vp]),
    "nanospec_batch_state_bytes": (c_size, [c_int32, c_int32, c_int32]),
    "nanospec_batch_create": (ctypes.c_int, [ctypes.POINTER(c_vp), c_int32, c_int32, c_int32, c_vp, c_size, c_vp]),
    "nanospec_batch_destroy": (ctypes.c_int, [c_vp]),
    "nanospec_batch_member": (ctypes.c_int, [c_vp, c_int32, ctypes.POINTER(c_vp)]),
    "nanospec_batch_step_update": (ctypes.c_int, [c_vp, c_vp, c_int32, c_vp, c_int32, c_vp, c_int32, c_vp, c_int32,
                                                  c_vp, c_vp, c_vp, c_vp]),
    "nanospec_batch_draft_workspace_bytes": (c_size, [c_int32, c_int32, c_int32, c_int32, c_int32]),
    "nanospec_batch_draft_logits_topk": (ctypes.c_int, [c_vp, c_vp, c_vp, c_int32, c_int32, c_int32, c_int32,
                                                        c_int32, c_vp, c_int32, c_int32, c_vp, c_vp, c_vp, c_vp,
                                                        c_size, c_vp]),
    "nanospec_draft_logprob_topk": (ctypes.c_int, [c_vp, c_int32, c_vp, c_vp, c_int32, c_int32, c_int32, c_int32,
                                                   c_vp, c_int32, c_int32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                   c_size, c_vp]),
    "nanospec_tree_select": (ctypes.c_int, [c_vp, c_vp, c_int32, c_int32, c_int32, c_vp, c_vp, c_vp, c_vp]),
    "nanospec_draft_project": (ctypes.c_int, [c_vp, c_int32, c_vp, c_vp, c_int32, c_int32, c_int32, c_int32, c_vp,
                                              c_int32, c_int32, c_vp, c_size, c_vp]),
    "nanospec_draft_select": (ctypes.c_int, [c_vp, c_vp, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_vp,
                                             c_vp, c_vp, c_vp, c_size, c_vp]),
    "nanospec_batch_draft_logprob_topk": (ctypes.c_int, [c_vp, c_vp, c_vp, c_int32, c_int32, c_int32, c_int32, c_int32,
                                                         c_vp, c_int32, c_int32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                         c_size, c_vp]),
    "nanospec_packed_bytes": (c_size, [c_int32, c_int32]),
    "nanospec_packed_create": (ctypes.c_int, [ctypes.POINTER(c_vp), c_int32, c_int32, c_vp, c_size, c_vp]),
    "nanospec_packed_reset": (ctypes.c_int, [c_vp, c_vp]),
    "nanospec_packed_destroy": (ctypes.c_int, [c_vp]),
    "nanospec_packed_slots": (ctypes.c_int, [c_vp] + [ctypes.POINTER(c_vp)] * 5),
    "nanospec_packed_update": (ctypes.c_int, [c_vp, c_vp, c_vp, c_int32, c_int32, c_vp, c_vp]),
    "nanospec_decode_step_workspace_bytes": (c_size, [c_int32, c_int32, c_int32, c_int32, c_int32]),
    "nanospec_decode_step": (ctypes.c_int, [c_vp, c_vp, c_int32, c_vp, c_int32, c_vp, c_vp, c_vp, c_int32, c_int32,
                                            c_int32, c_vp, c_int32, c_int32, c_vp, c_vp, c_vp, c_size, c_vp]),
    "nanospec_decode_step_project": (ctypes.c_int, [c_vp, c_vp, c_int32, c_vp, c_int32, c_vp, c_vp, c_vp, c_int32,
                                                    c_int32, c_int32, c_vp, c_int32, c_int32, c_vp, c_size, c_vp]),
    "nanospec_decode_step_select": (ctypes.c_int, [c_vp, c_vp, c_vp, c_int32, c_int32, c_int32, c_int32, c_int32, c_vp,
                                                   c_vp, c_vp, c_size, c_vp]),
    "nanospec_batch_decode_step_workspace_bytes": (c_size, [c_int32] * 6),
    "nanospec_batch_decode_step": (ctypes.c_int, [c_vp, c_vp, c_int32, c_vp, c_int32, c_vp, c_int32, c_vp, c_int32,
                                                  c_vp, c_vp, c_vp, c_int32, c_int32, c_int32, c_vp, c_int32, c_int32,
                                                  c_vp, c_vp, c_vp, c_size, c_vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _strerror(code: int) -> str:
    return _lib.nanospec_strerror(code).decode()


def _check(rc: int, where: str) -> None:
    if rc != NS_OK:
        raise NanoSpecError(rc, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return NS_BF16
    if t.dtype == torch.float32:
        return NS_FP32
    if t.dtype == torch.float16:
        return NS_FP16
    raise NanoSpecError(NS_EDTYPE, f"dtype {t.dtype}")


def nanospec_version() -> int:
    return _lib.nanospec_version()


def nanospec_strerror(code: int) -> str:
    return _strerror(code)


# ---------------------------------------------------------------------------
# Window state
# ---------------------------------------------------------------------------


def nanospec_state_bytes(V: int, w_max: int) -> int:
    return _lib.nanospec_state_bytes(V, w_max)


class NanoSpecState:
    """Host handle plus the caller-owned device buffer of one window state."""

    def __init__(self, V: int, w_max: int, device="cuda", stream=None):
        nbytes = nanospec_state_bytes(V, w_max)
        if nbytes == 0:
            raise NanoSpecError(NS_EINVAL, f"nanospec_state_bytes(V={V}, w_max={w_max})")
        self.V, self.w_max = V, w_max
        self.mem = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.mem.data_ptr()) % 256
        self.buf = self.mem[off:off + nbytes]
        h = ctypes.c_void_p()
        _check(_lib.nanospec_state_create(ctypes.byref(h), V, w_max, _ptr(self.buf), nbytes, _stream(stream)),
               "nanospec_state_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            _lib.nanospec_state_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


def nanospec_state_set_mode(st, mode: int) -> None:
    _check(_lib.nanospec_state_set_mode(st.handle, mode), "nanospec_state_set_mode")


def nanospec_state_reset(st: NanoSpecState, stream=None) -> None:
    _check(_lib.nanospec_state_reset(st.handle, _stream(stream)), "nanospec_state_reset")


def nanospec_state_status(st: NanoSpecState, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check(_lib.nanospec_state_status(st.handle, ctypes.byref(flags), _stream(stream)), "nanospec_state_status")
    return flags.value


def nanospec_state_window(st: NanoSpecState, window: Optional[torch.Tensor], length: Optional[torch.Tensor],
                          stream=None) -> None:
    _check(_lib.nanospec_state_window(st.handle, _ptr(window), _ptr(length), _stream(stream)),
           "nanospec_state_window")


def nanospec_stream_append(st: NanoSpecState, ids: Optional[torch.Tensor], n: int, dedup_first: int,
                           stream=None) -> None:
    _check(_lib.nanospec_stream_append(st.handle, _ptr(ids), n, dedup_first, _stream(stream)),
           "nanospec_stream_append")


def nanospec_active_vocab(st: NanoSpecState, active_ids: torch.Tensor, n_active: torch.Tensor,
                          bitmap: Optional[torch.Tensor] = None, stream=None) -> None:
    _check(_lib.nanospec_active_vocab(st.handle, _ptr(active_ids), _ptr(n_active), _ptr(bitmap),
                                      _stream(stream)), "nanospec_active_vocab")


def nanospec_step_update(st: NanoSpecState, draft_ids: Optional[torch.Tensor], n_draft: int,
                         ver_ids: Optional[torch.Tensor], n_ver: int, active_ids: torch.Tensor,
                         n_active: torch.Tensor, bitmap: Optional[torch.Tensor] = None, stream=None) -> None:
    _check(_lib.nanospec_step_update(st.handle, _ptr(draft_ids), n_draft, _ptr(ver_ids), n_ver,
                                     _ptr(active_ids), _ptr(n_active), _ptr(bitmap), _stream(stream)),
           "nanospec_step_update")


def nanospec_decode_step_workspace_bytes(w_max: int, n_tuple: int, M: int, k: int, d: int) -> int:
    return _lib.nanospec_decode_step_workspace_bytes(w_max, n_tuple, M, k, d)


def nanospec_decode_step(st: NanoSpecState, draft_ids: Optional[torch.Tensor], n_draft: int,
                         ver_ids: Optional[torch.Tensor], n_ver: int, active_ids: torch.Tensor,
                         n_active: torch.Tensor, w: torch.Tensor, V: int, d: int, dtype: int, h: torch.Tensor,
                         M: int, k: int, topk_ids: torch.Tensor, topk_vals: torch.Tensor, ws: torch.Tensor,
                         stream=None) -> None:
    _check(_lib.nanospec_decode_step(st.handle, _ptr(draft_ids), n_draft, _ptr(ver_ids), n_ver, _ptr(active_ids),
                                     _ptr(n_active), _ptr(w), V, d, dtype, _ptr(h), M, k, _ptr(topk_ids),
                                     _ptr(topk_vals), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "nanospec_decode_step")


def nanospec_decode_step_project(st: NanoSpecState, draft_ids: Optional[torch.Tensor], n_draft: int,
                                 ver_ids: Optional[torch.Tensor], n_ver: int, active_ids: torch.Tensor,
                                 n_active: torch.Tensor, w: torch.Tensor, V: int, d: int, dtype: int, h: torch.Tensor,
                                 M: int, k: int, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_decode_step_project(st.handle, _ptr(draft_ids), n_draft, _ptr(ver_ids), n_ver,
                                             _ptr(active_ids), _ptr(n_active), _ptr(w), V, d, dtype, _ptr(h), M, k,
                                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "nanospec_decode_step_project")


def nanospec_decode_step_select(st: NanoSpecState, active_ids: torch.Tensor, n_active: torch.Tensor, V: int, d: int,
                                dtype: int, M: int, k: int, topk_ids: torch.Tensor, topk_vals: torch.Tensor,
                                ws: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_decode_step_select(st.handle, _ptr(active_ids), _ptr(n_active), V, d, dtype, M, k,
                                            _ptr(topk_ids), _ptr(topk_vals), _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream)), "nanospec_decode_step_select")


def alloc_decode_workspace(w_max: int, n_tuple: int, M: int, k: int, d: int, device="cuda") -> torch.Tensor:
    """A 256-byte-aligned uint8 workspace of nanospec_decode_step_workspace_bytes."""
    nbytes = nanospec_decode_step_workspace_bytes(w_max, n_tuple, M, k, d)
    if nbytes == 0:
        raise NanoSpecError(NS_EINVAL, "nanospec_decode_step_workspace_bytes")
    mem = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-mem.data_ptr()) % 256
    return mem[off:off + nbytes]


# ---------------------------------------------------------------------------
# Gather, draft head, prefill
# ---------------------------------------------------------------------------


def nanospec_gather_rows(w: torch.Tensor, V: int, d: int, dtype: int, ids: torch.Tensor,
                         n_dev: Optional[torch.Tensor], n_max: int, out: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_gather_rows(_ptr(w), V, d, dtype, _ptr(ids), _ptr(n_dev), n_max, _ptr(out),
                                     _stream(stream)), "nanospec_gather_rows")


def nanospec_draft_workspace_bytes(n_max: int, M: int, k: int, d: int) -> int:
    return _lib.nanospec_draft_workspace_bytes(n_max, M, k, d)


def nanospec_draft_logits_topk(rows: torch.Tensor, mode: int, row_ids: Optional[torch.Tensor],
                               n_dev: Optional[torch.Tensor], n_max: int, V: int, d: int, dtype: int,
                               h: torch.Tensor, M: int, k: int, logits: Optional[torch.Tensor],
                               topk_ids: torch.Tensor, topk_vals: torch.Tensor, ws: torch.Tensor,
                               stream=None) -> None:
    _check(_lib.nanospec_draft_logits_topk(_ptr(rows), mode, _ptr(row_ids), _ptr(n_dev), n_max, V, d, dtype,
                                           _ptr(h), M, k, _ptr(logits), _ptr(topk_ids), _ptr(topk_vals),
                                           _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "nanospec_draft_logits_topk")


def nanospec_draft_logits_topk_noalloc(rows: torch.Tensor, mode: int, row_ids: Optional[torch.Tensor],
                                       n_dev: Optional[torch.Tensor], n_max: int, V: int, d: int, dtype: int,
                                       h: torch.Tensor, M: int, k: int, logits: Optional[torch.Tensor],
                                       topk_ids: torch.Tensor, topk_vals: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_draft_logits_topk_noalloc(_ptr(rows), mode, _ptr(row_ids), _ptr(n_dev), n_max, V, d, dtype,
                                                   _ptr(h), M, k, _ptr(logits), _ptr(topk_ids), _ptr(topk_vals),
                                                   _stream(stream)), "nanospec_draft_logits_topk_noalloc")


def nanospec_draft_logprob_topk(rows: torch.Tensor, mode: int, row_ids: Optional[torch.Tensor],
                                n_dev: Optional[torch.Tensor], n_max: int, V: int, d: int, dtype: int, h: torch.Tensor,
                                M: int, k: int, parent: Optional[torch.Tensor], lse: Optional[torch.Tensor],
                                logits: Optional[torch.Tensor], topk_ids: torch.Tensor, topk_vals: torch.Tensor,
                                ws: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_draft_logprob_topk(_ptr(rows), mode, _ptr(row_ids), _ptr(n_dev), n_max, V, d, dtype, _ptr(h),
                                            M, k, _ptr(parent), _ptr(lse), _ptr(logits), _ptr(topk_ids),
                                            _ptr(topk_vals), _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream)), "nanospec_draft_logprob_topk")


def nanospec_batch_draft_logprob_topk(w: torch.Tensor, row_ids: torch.Tensor, n_dev: torch.Tensor, n_max: int,
                                      B: int, V: int, d: int, dtype: int, h: torch.Tensor, M: int, k: int,
                                      parent: Optional[torch.Tensor], lse: Optional[torch.Tensor],
                                      logits: Optional[torch.Tensor], topk_ids: torch.Tensor, topk_vals: torch.Tensor,
                                      ws: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_batch_draft_logprob_topk(_ptr(w), _ptr(row_ids), _ptr(n_dev), n_max, B, V, d, dtype, _ptr(h),
                                                  M, k, _ptr(parent), _ptr(lse), _ptr(logits), _ptr(topk_ids),
                                                  _ptr(topk_vals), _ptr(ws), ws.numel() * ws.element_size(),
                                                  _stream(stream)), "nanospec_batch_draft_logprob_topk")


def nanospec_draft_project(rows: torch.Tensor, mode: int, row_ids: Optional[torch.Tensor], n_dev: Optional[torch.Tensor],
                           n_max: int, V: int, d: int, dtype: int, h: torch.Tensor, M: int, k: int, ws: torch.Tensor,
                           stream=None) -> None:
    _check(_lib.nanospec_draft_project(_ptr(rows), mode, _ptr(row_ids), _ptr(n_dev), n_max, V, d, dtype, _ptr(h), M, k,
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "nanospec_draft_project")


def nanospec_draft_select(row_ids: Optional[torch.Tensor], n_dev: Optional[torch.Tensor], n_max: int, V: int, d: int,
                          dtype: int, M: int, k: int, logits: Optional[torch.Tensor], topk_ids: torch.Tensor,
                          topk_vals: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_draft_select(_ptr(row_ids), _ptr(n_dev), n_max, V, d, dtype, M, k, _ptr(logits),
                                      _ptr(topk_ids), _ptr(topk_vals), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)), "nanospec_draft_select")


def nanospec_tree_select(vals: torch.Tensor, ids: torch.Tensor, C: int, B: int, k: int, out_idx: torch.Tensor,
                         out_vals: torch.Tensor, out_ids: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_tree_select(_ptr(vals), _ptr(ids), C, B, k, _ptr(out_idx), _ptr(out_vals), _ptr(out_ids),
                                     _stream(stream)), "nanospec_tree_select")


def nanospec_prefill_topk(logits: torch.Tensor, L: int, V: int, dtype: int, k: int, out_ids: torch.Tensor,
                          out_vals: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_prefill_topk(_ptr(logits), L, V, dtype, k, _ptr(out_ids), _ptr(out_vals),
                                      _stream(stream)), "nanospec_prefill_topk")


# ---------------------------------------------------------------------------
# Batches of independent sequences
# ---------------------------------------------------------------------------


def nanospec_batch_state_bytes(B: int, V: int, w_max: int) -> int:
    return _lib.nanospec_batch_state_bytes(B, V, w_max)


class _Member:
    """A borrowed per-sequence handle of a batch (the batch owns it)."""

    def __init__(self, handle, V, w_max):
        self.handle, self.V, self.w_max = handle, V, w_max


class NanoSpecBatch:
    """B window states in one caller-owned device buffer."""

    def __init__(self, B: int, V: int, w_max: int, device="cuda", stream=None):
        nbytes = nanospec_batch_state_bytes(B, V, w_max)
        if nbytes == 0:
            raise NanoSpecError(NS_EINVAL, f"nanospec_batch_state_bytes(B={B}, V={V}, w_max={w_max})")
        self.B, self.V, self.w_max = B, V, w_max
        self.mem = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.mem.data_ptr()) % 256
        self.buf = self.mem[off:off + nbytes]
        h = ctypes.c_void_p()
        _check(_lib.nanospec_batch_create(ctypes.byref(h), B, V, w_max, _ptr(self.buf), nbytes, _stream(stream)),
               "nanospec_batch_create")
        self.handle = h

    def member(self, b: int) -> "_Member":
        out = ctypes.c_void_p()
        _check(_lib.nanospec_batch_member(self.handle, b, ctypes.byref(out)), "nanospec_batch_member")
        return _Member(out, self.V, self.w_max)

    def close(self):
        if getattr(self, "handle", None):
            _lib.nanospec_batch_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


def nanospec_batch_step_update(bt: NanoSpecBatch, draft_ids: torch.Tensor, draft_stride: int, n_draft: torch.Tensor,
                               nd_max: int, ver_ids: torch.Tensor, ver_stride: int, n_ver: torch.Tensor, nv_max: int,
                               active_ids: torch.Tensor, n_active: torch.Tensor,
                               bitmap: Optional[torch.Tensor] = None, stream=None) -> None:
    _check(_lib.nanospec_batch_step_update(bt.handle, _ptr(draft_ids), draft_stride, _ptr(n_draft), nd_max,
                                           _ptr(ver_ids), ver_stride, _ptr(n_ver), nv_max, _ptr(active_ids),
                                           _ptr(n_active), _ptr(bitmap), _stream(stream)),
           "nanospec_batch_step_update")


def nanospec_batch_draft_workspace_bytes(B: int, n_max: int, M: int, k: int, d: int) -> int:
    return _lib.nanospec_batch_draft_workspace_bytes(B, n_max, M, k, d)


def nanospec_batch_draft_logits_topk(w: torch.Tensor, row_ids: torch.Tensor, n_dev: torch.Tensor, n_max: int,
                                     B: int, V: int, d: int, dtype: int, h: torch.Tensor, M: int, k: int,
                                     logits: Optional[torch.Tensor], topk_ids: torch.Tensor,
                                     topk_vals: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_batch_draft_logits_topk(_ptr(w), _ptr(row_ids), _ptr(n_dev), n_max, B, V, d, dtype,
                                                 _ptr(h), M, k, _ptr(logits), _ptr(topk_ids), _ptr(topk_vals),
                                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "nanospec_batch_draft_logits_topk")


# ---------------------------------------------------------------------------
# Slot-stable packed buffer
# ---------------------------------------------------------------------------


def nanospec_packed_bytes(V: int, w_max: int) -> int:
    return _lib.nanospec_packed_bytes(V, w_max)


class NanoSpecPacked:
    """Host handle plus the caller-owned device memory of one slot map.  The
    int32 tensors ``slot_ids`` [w_max], ``n_slots`` [1], ``enter_slots``
    [w_max], ``enter_ids`` [w_max] and ``n_enter`` [1] view that memory at the
    addresses nanospec_packed_slots reports."""

    def __init__(self, V: int, w_max: int, device="cuda", stream=None):
        nbytes = nanospec_packed_bytes(V, w_max)
        if nbytes == 0:
            raise NanoSpecError(NS_EINVAL, f"nanospec_packed_bytes(V={V}, w_max={w_max})")
        self.V, self.w_max = V, w_max
        self.mem = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.mem.data_ptr()) % 256
        self.buf = self.mem[off:off + nbytes]
        h = ctypes.c_void_p()
        _check(_lib.nanospec_packed_create(ctypes.byref(h), V, w_max, _ptr(self.buf), nbytes, _stream(stream)),
               "nanospec_packed_create")
        self.handle = h
        ptrs = [c_vp() for _ in range(5)]
        _check(_lib.nanospec_packed_slots(h, *[ctypes.byref(p) for p in ptrs]), "nanospec_packed_slots")
        base = self.buf.data_ptr()

        def view(p, n):
            o = p.value - base
            return self.buf[o:o + 4 * n].view(torch.int32)

        self.slot_ids = view(ptrs[0], w_max)
        self.n_slots = view(ptrs[1], 1)
        self.enter_slots = view(ptrs[2], w_max)
        self.enter_ids = view(ptrs[3], w_max)
        self.n_enter = view(ptrs[4], 1)

    def close(self):
        if getattr(self, "handle", None):
            _lib.nanospec_packed_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


def nanospec_packed_reset(pk: NanoSpecPacked, stream=None) -> None:
    _check(_lib.nanospec_packed_reset(pk.handle, _stream(stream)), "nanospec_packed_reset")


def nanospec_packed_update(pk: NanoSpecPacked, st, w: torch.Tensor, d: int, dtype: int, rows: torch.Tensor,
                           stream=None) -> None:
    _check(_lib.nanospec_packed_update(pk.handle, st.handle, _ptr(w), d, dtype, _ptr(rows), _stream(stream)),
           "nanospec_packed_update")


def nanospec_batch_decode_step_workspace_bytes(B: int, w_max: int, n_tuple: int, M: int, k: int, d: int) -> int:
    return _lib.nanospec_batch_decode_step_workspace_bytes(B, w_max, n_tuple, M, k, d)


def nanospec_batch_decode_step(bt: "NanoSpecBatch", draft_ids: torch.Tensor, draft_stride: int, n_draft: torch.Tensor,
                               nd_max: int, ver_ids: torch.Tensor, ver_stride: int, n_ver: torch.Tensor, nv_max: int,
                               active_ids: torch.Tensor, n_active: torch.Tensor, w: torch.Tensor, V: int, d: int,
                               dtype: int, h: torch.Tensor, M: int, k: int, topk_ids: torch.Tensor,
                               topk_vals: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.nanospec_batch_decode_step(bt.handle, _ptr(draft_ids), draft_stride, _ptr(n_draft), nd_max,
                                           _ptr(ver_ids), ver_stride, _ptr(n_ver), nv_max, _ptr(active_ids),
                                           _ptr(n_active), _ptr(w), V, d, dtype, _ptr(h), M, k, _ptr(topk_ids),
                                           _ptr(topk_vals), _ptr(ws), ws.numel() * ws.element_size(),
                                           _stream(stream)), "nanospec_batch_decode_step")


def alloc_batch_decode_workspace(B: int, w_max: int, n_tuple: int, M: int, k: int, d: int,
                                 device="cuda") -> torch.Tensor:
    """A 256-byte-aligned uint8 workspace of nanospec_batch_decode_step_workspace_bytes."""
    nbytes = nanospec_batch_decode_step_workspace_bytes(B, w_max, n_tuple, M, k, d)
    if nbytes == 0:
        raise NanoSpecError(NS_EINVAL, "nanospec_batch_decode_step_workspace_bytes")
    mem = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-mem.data_ptr()) % 256
    return mem[off:off + nbytes]


def alloc_batch_workspace(B: int, n_max: int, M: int, k: int, d: int, device="cuda") -> torch.Tensor:
    """A 256-byte-aligned uint8 workspace of nanospec_batch_draft_workspace_bytes."""
    nbytes = nanospec_batch_draft_workspace_bytes(B, n_max, M, k, d)
    if nbytes == 0:
        raise NanoSpecError(NS_EINVAL, "nanospec_batch_draft_workspace_bytes")
    mem = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-mem.data_ptr()) % 256
    return mem[off:off + nbytes]


def alloc_workspace(n_max: int, M: int, k: int, d: int, device="cuda") -> torch.Tensor:
    """A 256-byte-aligned uint8 workspace of nanospec_draft_workspace_bytes."""
    nbytes = nanospec_draft_workspace_bytes(n_max, M, k, d)
    if nbytes == 0:
        raise NanoSpecError(NS_EINVAL, "nanospec_draft_workspace_bytes")
    mem = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-mem.data_ptr()) % 256
    return mem[off:off + nbytes]
