"""ctypes binding of the C++ oracle (oracle/nanospec_oracle.cpp).

TEST INFRASTRUCTURE ONLY, like the numpy oracle: loaded by tests/ and by
bench.py's cpu_baseline leg, never by the product path.  The library is
built from source by oracle/build_oracle.py (when it is missing)."""
from __future__ import annotations

import ctypes

import numpy as np

from oracle.build_oracle import ensure_built

DTYPES = {"bf16": 0, "fp32": 1, "fp16": 2}

_lib = ctypes.CDLL(ensure_built())
_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_lib.nso_seq_new.restype = _vp
_lib.nso_seq_new.argtypes = [ctypes.c_int]
_lib.nso_seq_free.argtypes = [_vp]
_lib.nso_seq_append.argtypes = [_vp, _vp, ctypes.c_int]
_lib.nso_seq_step.argtypes = [_vp, _vp, ctypes.c_int, _vp, ctypes.c_int]
_lib.nso_seq_len.restype = _i64
_lib.nso_seq_len.argtypes = [_vp]
_lib.nso_seq_active.restype = ctypes.c_int
_lib.nso_seq_active.argtypes = [_vp, _vp, ctypes.c_int]
_lib.nso_project.restype = ctypes.c_int
_lib.nso_project.argtypes = [_vp, ctypes.c_int, ctypes.c_int, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, ctypes.c_int]
_lib.nso_topk.argtypes = [_vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp]


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _i32a(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


class Sequence:
    """The full stream S of one sequence (C++), with the window rule."""

    def __init__(self, w_max: int):
        self.w_max = int(w_max)
        self._h = _lib.nso_seq_new(self.w_max)

    def __del__(self):
        if getattr(self, "_h", None):
            _lib.nso_seq_free(self._h)
            self._h = None

    def append_prompt(self, ids) -> None:
        a = _i32a(ids)
        _lib.nso_seq_append(self._h, _p(a), a.size)

    def step(self, tree_ids, ver_ids) -> None:
        t, v = _i32a(tree_ids), _i32a(ver_ids)
        _lib.nso_seq_step(self._h, _p(t), t.size, _p(v), v.size)

    def __len__(self) -> int:
        return int(_lib.nso_seq_len(self._h))

    def active(self) -> np.ndarray:
        out = np.empty(self.w_max, dtype=np.int32)
        n = _lib.nso_seq_active(self._h, _p(out), out.size)
        return out[:n].astype(np.int64)


def project(h: np.ndarray, W: np.ndarray, I, dtype: str, threads: int = 1):
    """(logits [M x n] float64, threads that ran) of Eq. 1 on W[I, :]."""
    W = np.ascontiguousarray(W)
    h = np.ascontiguousarray(h)
    I = _i32a(I)
    M, d = h.shape
    out = np.empty((M, I.size), dtype=np.float64)
    used = _lib.nso_project(_p(W), d, DTYPES[dtype], _p(I), I.size, _p(h), M, _p(out), int(threads))
    return out, used


def topk(logits: np.ndarray, I, k: int):
    """(ids int64 [M x k], vals float64 [M x k]) by (value desc, id asc)."""
    z = np.ascontiguousarray(np.atleast_2d(logits), dtype=np.float64)
    I = _i32a(I)
    M = z.shape[0]
    ids = np.empty((M, k), dtype=np.int64)
    vals = np.empty((M, k), dtype=np.float64)
    _lib.nso_topk(_p(z), _p(I), I.size, M, int(k), _p(ids), _p(vals))
    return ids, vals
