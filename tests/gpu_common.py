"""Shared helpers for the GPU parity tests: device marshalling, the oracle
side of a run, and the comparison rules.

Rules (the oracle is the reference; see oracle/nanospec_oracle.py):
  * ids, windows, active sets, counts, bitmaps, gathered rows and prefill
    top-k: bit-exact;
  * logits: |gpu - ref| <= ATOL + RTOL * |ref| element-wise on valid columns;
  * draft top-k (float sums in different orders may swap near-ties): with O
    the oracle's set and G the GPU's, G holds min(k, n) distinct active ids,
    every id of G xor O has a reference logit within tolerance of the
    oracle's k-th value, every GPU value is within tolerance of the reference
    logit of its id, values are non-increasing, padding is (-1, -inf).
"""
import sys

import numpy as np
import torch

import oracle.nanospec_oracle as O

ATOL = 1e-2
RTOL = 1e-2


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def dev_i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).cuda()


def dev_elems(x: np.ndarray, dtype: str) -> torch.Tensor:
    """bf16 / fp16 bit patterns (uint16) or float32 array -> device tensor."""
    if dtype in ("bf16", "fp16"):
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).cuda()
        return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_elems(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype in ("bf16", "fp16"):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def dcode_of(ns, dtype: str) -> int:
    return {"bf16": ns.NS_BF16, "fp32": ns.NS_FP32, "fp16": ns.NS_FP16}[dtype]


def tol(ref):
    return ATOL + RTOL * np.abs(ref)


def check_logits(gpu: np.ndarray, ref: np.ndarray, what=""):
    gpu = np.asarray(gpu, np.float64)
    bad = np.abs(gpu - ref) > tol(ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} logits out of tolerance, worst " \
                          f"{float(np.max(np.abs(gpu - ref))):.3g}"


def check_topk(g_ids, g_vals, ref_logits, I, o_ids, o_vals, k, what=""):
    """Set rule for the draft top-k (see module docstring).  ref_logits[m, j]
    is the oracle logit of active column j, whose global id is I[j]."""
    I = np.asarray(I, np.int64)
    pos = {int(v): j for j, v in enumerate(I)}
    n = len(I)
    kk = min(k, n)
    for m in range(g_ids.shape[0]):
        gi = g_ids[m].astype(np.int64)
        gv = g_vals[m].astype(np.float64)
        assert (gi[kk:] == -1).all() and np.isneginf(gv[kk:]).all(), f"{what} m={m}: bad padding"
        G, Os = gi[:kk], o_ids[m][:kk]
        assert len(set(G.tolist())) == kk, f"{what} m={m}: duplicate ids"
        assert all(int(x) in pos for x in G), f"{what} m={m}: id outside the active set"
        if kk == 0:
            continue
        vk = o_vals[m][kk - 1]
        for x in set(G.tolist()) ^ set(Os.tolist()):
            r = ref_logits[m, pos[int(x)]]
            assert abs(r - vk) <= tol(vk), f"{what} m={m}: id {x} (ref {r}) is not a near-tie of the k-th {vk}"
        refs = np.array([ref_logits[m, pos[int(x)]] for x in G])
        assert (np.abs(gv[:kk] - refs) <= tol(refs)).all(), f"{what} m={m}: value off its id's logit"
        assert (np.diff(gv[:kk]) <= 0).all(), f"{what} m={m}: values not sorted"


def bitmap_from_ids(I, V):
    return O.bitmap(np.asarray(I), V)
