"""CPU oracle for the dynamic-vocabulary draft head.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: it is used by ``tests/``, by ``__graft_entry__.smoke()`` (to check one
small GPU invocation) and by ``bench.py``'s ``cpu_baseline`` leg.  It shares no
code with the HIP path and imports nothing from the package.

Every result the method reaches has a plain definition, so each function below
is that definition written out with numpy, in float64 where floating point is
involved.  Sources (cited by page title and section/equation):

* MicroSpec/NanoSpec (arXiv 2605.26444), Sec. 3.1 "Preliminaries and Problem
  Formulation", Eq. 1: the LM head z_t = W_head h_t, and its restriction to a
  row subset W_head[I_t, :].
* Sec. 3.2 "Candidate Stream Initialization (Prefill Phase)": the top-K
  operator T_K(z) and S_init = (x_1..x_L) (+) tuple(U_i T_Kpre(z_i)).
* Sec. 3.2 "Dynamic Stream Update (Decoding Phase)": C_draft (unique ids of the
  draft tree), C_ver = T_Kver(z_verify) and
  S_new = S_old (+) tuple(C_draft) (+) tuple(C_ver).
* Sec. 3.2 "Vocabulary Construction via Sliding Window":
  I_{t+1} = Unique(Suffix(S_new, W_max)).
* NanoSpec, "Eliminating Overhead via GPU-Resident State Management": the
  active set is held as a bitmap.
* NanoSpec, "Avoiding Sparse Computation via Asynchronous Gathering": a
  preallocated buffer of W_max rows receives only the rows of newly active ids.

Readings taken where the pages leave a step open (each also listed in the
design notes):

* R1 ``tuple()`` of a set keeps first occurrences in the order the elements
  are produced: position-major, rank-minor for the prefill union; flattened
  tree order for C_draft; rank order for T_Kver.
* R2 dedup happens only *inside* each tuple; S itself keeps repeats (the
  S_new equation appends without filtering).
* R3 the window is over stream *entries*, so |I| <= W_max; when |S| < W_max
  the suffix is all of S.
* R4 ``Unique`` returns ascending ids; ties in T_K go to the lower index
  (for the draft head: the lower *global* id).
* R5 k larger than the candidate count pads with (id -1, value -inf).
* R7 the draft head's values for the tree are log-probabilities renormalised
  over I plus the parent's score; R8 the tree keeps the F best children of
  each depth for expansion and the N best nodes overall (see draft_tree).
* R6 slot-stable packing (see packed_update): rows keep their slot while
  their id stays active; entering ids fill the lowest free slots in ascending
  id order; slots of ids that left are holes.

Parity pins for every function live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

from typing import Iterable, List, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")

# ---------------------------------------------------------------------------
# Input widening
# ---------------------------------------------------------------------------


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of each stored element.

    bf16 elements are given as their 16-bit patterns (uint16); a bf16 value is
    the float32 whose upper half is those bits, and float32 -> float64 is
    exact.  fp16 elements are uint16 patterns of IEEE binary16, decoded from
    their fields.  fp32 elements widen exactly too."""
    if dtype == "bf16":
        b = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32).astype(np.float64)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "fp16":
        # IEEE-754 binary16 from its fields: sign, 5-bit exponent (bias 15),
        # 10-bit fraction; exponent 0 is subnormal (fraction * 2^-24).  Inputs
        # are finite (the generators never make Inf or NaN).
        u = np.asarray(x, dtype=np.uint16).astype(np.int64)
        sign = np.where(u >> 15, -1.0, 1.0)
        e = (u >> 10) & 0x1F
        f = (u & 0x3FF).astype(np.float64)
        mag = np.where(e == 0, f * 2.0 ** -24, (1024.0 + f) * np.exp2((e - 25).astype(np.float64)))
        return sign * mag
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# T_K  (Sec. 3.2, Candidate Stream Initialization: the Top-K operator)
# ---------------------------------------------------------------------------


def top_k(z: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest entries of z, ordered by value descending and,
    among equal values, index ascending (R4).  Returns min(K, len(z)) indices.

    The K largest all lie at or above the K-th largest value, so the entries
    with z >= that value are taken and fully sorted by (-value, index)."""
    z = np.asarray(z, dtype=np.float64)
    n = z.shape[0]
    K = min(int(K), n)
    if K <= 0:
        return np.zeros(0, dtype=np.int64)
    assert not np.isnan(z).any(), "oracle inputs never hold NaN"
    kth = np.partition(z, n - K)[n - K]
    cand = np.nonzero(z >= kth)[0]
    order = np.lexsort((cand, -z[cand]))
    return cand[order[:K]]


# ---------------------------------------------------------------------------
# Prefill: T_Kpre per position, ordered union, S_init
# ---------------------------------------------------------------------------


def prefill_topk(Z: np.ndarray, K: int, dtype: str = "bf16") -> Tuple[np.ndarray, np.ndarray]:
    """P[i] = T_Kpre(z_i) for every prompt position i (Sec. 3.2, prefill).

    Returns (ids int64 [L x K], values float64 [L x K]); K <= V assumed."""
    L = Z.shape[0]
    ids = np.zeros((L, K), dtype=np.int64)
    vals = np.zeros((L, K), dtype=np.float64)
    for i in range(L):
        z = widen(Z[i], dtype)
        t = top_k(z, K)
        ids[i, :len(t)] = t
        vals[i, :len(t)] = z[t]
    return ids, vals


def first_occurrence(ids: Iterable[int]) -> List[int]:
    """tuple() of a set built from a sequence: each distinct id once, in the
    order of its first appearance (R1)."""
    seen = set()
    out: List[int] = []
    for x in ids:
        x = int(x)
        if x not in seen:
            seen.add(x)
            out.append(x)
    return out


def init_stream(prompt: Sequence[int], P: np.ndarray) -> List[int]:
    """S_init = (x_1..x_L) (+) tuple(union_i T_Kpre(z_i))  (Sec. 3.2, prefill).

    The union is ordered position-major, rank-minor (R1) and is not filtered
    against the prompt (R2)."""
    return [int(x) for x in prompt] + first_occurrence(np.asarray(P).reshape(-1))


# ---------------------------------------------------------------------------
# Decode-step stream update (Sec. 3.2, Dynamic Stream Update)
# ---------------------------------------------------------------------------


def draft_candidates(tree_ids: Sequence[int]) -> List[int]:
    """C_draft: every distinct id of the draft tree, in flattened tree order."""
    return first_occurrence(tree_ids)


def stream_update(S: List[int], tree_ids: Sequence[int], ver_ids: Sequence[int]) -> List[int]:
    """S_new = S_old (+) tuple(C_draft) (+) tuple(C_ver).

    ``ver_ids`` is C_ver already in rank order (distinct ids, appended as
    given)."""
    return list(S) + draft_candidates(tree_ids) + [int(x) for x in ver_ids]


# ---------------------------------------------------------------------------
# Sliding-window active set (Sec. 3.2, Vocabulary Construction via Sliding Window)
# ---------------------------------------------------------------------------


def suffix(S: Sequence[int], w_max: int) -> List[int]:
    """The last W_max entries of S (all of S when it is shorter; R3)."""
    assert w_max >= 1
    return list(S[-w_max:]) if len(S) > w_max else list(S)


def active_set(S: Sequence[int], w_max: int) -> np.ndarray:
    """I = Unique(Suffix(S, W_max)), as ascending ids (R4)."""
    return np.unique(np.asarray(suffix(S, w_max), dtype=np.int64))


def bitmap(I: np.ndarray, V: int) -> np.ndarray:
    """The active set as a bitmap of ceil(V/32) uint32 words: bit b of word w
    is set iff id 32*w + b is in I; bits past V stay 0."""
    words = np.zeros((V + 31) // 32, dtype=np.uint32)
    for v in np.asarray(I, dtype=np.int64):
        assert 0 <= v < V
        words[v >> 5] |= np.uint32(1) << np.uint32(v & 31)
    return words


# ---------------------------------------------------------------------------
# Restricted LM head (Sec. 3.1, Eq. 1 restricted to W_head[I_t, :])
# ---------------------------------------------------------------------------


def gather_rows(W: np.ndarray, I: np.ndarray) -> np.ndarray:
    """R[j] = W[I[j]], a bit copy."""
    return np.asarray(W)[np.asarray(I, dtype=np.int64)]


def project(h: np.ndarray, R: np.ndarray, dtype: str) -> np.ndarray:
    """logits[m, j] = sum_c h[m, c] * R[j, c] in float64 (Eq. 1 on the
    gathered rows: z = W_head[I, :] h for each hidden row)."""
    return widen(h, dtype) @ widen(R, dtype).T


def dense_logits(h: np.ndarray, W: np.ndarray, dtype: str) -> np.ndarray:
    """Full-vocabulary LM head z = W_head h for each hidden row (Eq. 1)."""
    return widen(h, dtype) @ widen(W, dtype).T


def draft_topk(logits: np.ndarray, I: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per hidden row m: T_k over the active columns, ordered by (logit
    descending, global id ascending), mapped back to global ids I[j].

    Returns (ids int64 [M x k], vals float64 [M x k]) padded with (-1, -inf)
    when k > |I| (R5)."""
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    I = np.asarray(I, dtype=np.int64)
    M = logits.shape[0]
    ids = np.full((M, k), -1, dtype=np.int64)
    vals = np.full((M, k), NEG_INF, dtype=np.float64)
    for m in range(M):
        order = np.lexsort((I, -logits[m]))[:k]
        ids[m, :len(order)] = I[order]
        vals[m, :len(order)] = logits[m, order]
    return ids, vals


def draft_head(h: np.ndarray, W: np.ndarray, I: np.ndarray, k: int, dtype: str):
    """Gather + projection + top-k + map back, composed.  Returns
    (logits [M x n], ids [M x k], vals [M x k])."""
    logits = project(h, gather_rows(W, I), dtype)
    ids, vals = draft_topk(logits, I, k)
    return logits, ids, vals


# ---------------------------------------------------------------------------
# Log-probabilities over the active set, and the multi-depth draft tree
# ---------------------------------------------------------------------------
#
# NanoSpec, Sec. 4.1 "Experimental Setup": the draft tree has depth 5 and at
# most 60 draft tokens; the results discussion notes that dropping tokens from
# the draft vocabulary renormalises the draft softmax over the active set.
# Readings R7 and R8: a node's children are the top K of its draft head, each
# scored by the node's score plus the child's log-probability over I; the
# next depth expands the F best children of the current depth (score
# descending, then flat index m * K + r ascending); the final tree is the N
# best of all generated nodes in the same order (pool index ascending on ties).


def log_softmax_active(logits: np.ndarray) -> np.ndarray:
    """logp[m, j] = z[m, j] - log(sum over active columns j' of exp(z[m, j'])),
    in float64 (the softmax restricted to, and renormalised over, I)."""
    z = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    if z.shape[1] == 0:
        return z.copy()
    mx = z.max(axis=1, keepdims=True)
    return z - (mx + np.log(np.exp(z - mx).sum(axis=1, keepdims=True)))


def draft_logprob_topk(h: np.ndarray, W: np.ndarray, I: np.ndarray, k: int, dtype: str,
                       parent: np.ndarray = None):
    """The draft head with log-probabilities over I: per hidden row m the top k
    of logp[m] (the same ids as the top k of the logits), valued
    parent[m] + logp.  Returns (logp [M x n], ids [M x k], vals [M x k])."""
    logp = log_softmax_active(project(h, gather_rows(W, I), dtype))
    ids, vals = draft_topk(logp, I, k)
    if parent is not None:
        vals = vals + np.asarray(parent, dtype=np.float64)[:, None]
    return logp, ids, vals


def select_best(vals: np.ndarray, ids: np.ndarray, k: int) -> np.ndarray:
    """Flat indices of the k best candidates (value descending, flat index
    ascending), skipping entries whose id is negative; padded with -1."""
    v = np.asarray(vals, dtype=np.float64).reshape(-1)
    live = np.flatnonzero(np.asarray(ids).reshape(-1) >= 0)
    order = live[np.lexsort((live, -v[live]))][:k]
    out = np.full(k, -1, dtype=np.int64)
    out[:len(order)] = order
    return out


def draft_tree(hs: Sequence[np.ndarray], W: np.ndarray, I: np.ndarray, K: int, F: int, N: int, dtype: str):
    """The multi-depth draft loop on one active set.  hs[t] holds the hidden
    rows of depth t: one row (the root) at depth 0, one per frontier slot
    after that.  Returns a dict with the node pool (ids, scores, parent pool
    index, depth), the frontier of every depth (pool indices) and the final
    N nodes (pool indices)."""
    pool_ids, pool_vals, pool_parent, pool_depth = [], [], [], []
    frontier = np.array([-1], dtype=np.int64)           # the root
    frontiers = []
    for t, h in enumerate(hs):
        h = np.atleast_2d(np.asarray(h))
        parent = np.array([pool_vals[f] if f >= 0 else 0.0 for f in frontier])
        _, ids, vals = draft_logprob_topk(h[:len(frontier)], W, I, K, dtype, parent)
        base = len(pool_ids)
        for m in range(len(frontier)):
            for r in range(K):
                pool_ids.append(int(ids[m, r]))
                pool_vals.append(float(vals[m, r]))
                pool_parent.append(int(frontier[m]))
                pool_depth.append(t)
        best = select_best(vals, ids, F)
        frontier = np.array([base + i for i in best if i >= 0], dtype=np.int64)
        frontiers.append(frontier)
    final = select_best(np.array(pool_vals), np.array(pool_ids), N)
    return {"ids": np.array(pool_ids), "vals": np.array(pool_vals), "parent": np.array(pool_parent),
            "depth": np.array(pool_depth), "frontiers": frontiers, "final": final}


# ---------------------------------------------------------------------------
# Slot-stable packed buffer
# ---------------------------------------------------------------------------
#
# NanoSpec, "Avoiding Sparse Computation via Asynchronous Gathering": a
# preallocated buffer of W_max rows holds W_head[I_t, :]; at each step only the
# rows of ids that became active are gathered into it.  The pages fix neither
# where an entering row goes nor what happens to the rows of ids that left.
# Reading R6: a row stays in its slot for as long as its id stays active; the
# slots of ids that left become holes (id -1); the ids that entered, taken in
# ascending id order, fill the free slots in ascending slot order; the head
# reads slots [0, n_slots), n_slots = 1 + the highest occupied slot (0 when
# none), and skips holes.


def packed_update(slot_ids: np.ndarray, I: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray, int]:
    """One update of the slot map to a new active set I.

    slot_ids: int [n_slot_cap], the global id held in each slot, -1 for a
    hole.  Returns (new slot ids, entering slots, entering ids, n_slots); the
    entering lists are in ascending id order and are the rows to gather."""
    old = np.asarray(slot_ids, dtype=np.int64)
    active = set(int(x) for x in np.asarray(I).reshape(-1))
    new = old.copy()
    for s in range(len(new)):                      # ids that left free their slot
        if new[s] >= 0 and int(new[s]) not in active:
            new[s] = -1
    held = set(int(x) for x in new if x >= 0)
    entering = sorted(active - held)
    free = [s for s in range(len(new)) if new[s] < 0]
    if len(entering) > len(free):
        raise ValueError("active set larger than the buffer")
    slots = np.array(free[:len(entering)], dtype=np.int64)
    new[slots] = np.array(entering, dtype=np.int64)
    occupied = [s for s in range(len(new)) if new[s] >= 0]
    n_slots = occupied[-1] + 1 if occupied else 0
    return new, slots, np.array(entering, dtype=np.int64), n_slots


def packed_draft_head(h: np.ndarray, W: np.ndarray, slot_ids: np.ndarray, n_slots: int, k: int,
                      dtype: str):
    """The draft head over the packed buffer: column j of slots [0, n_slots) is
    W[slot_ids[j]]; holes are not candidates.  Returns (ids, vals) as
    draft_topk."""
    ids = np.asarray(slot_ids, dtype=np.int64)[:n_slots]
    live = ids[ids >= 0]
    logits = project(h, gather_rows(W, live), dtype)
    return draft_topk(logits, live, k)


# ---------------------------------------------------------------------------
# Whole-sequence driver (composition of the above; used by tests and timing)
# ---------------------------------------------------------------------------


STREAM_MODES = ("full", "ctx_only", "ext_only")


class Sequence_:
    """Keeps the full stream S of one sequence and derives each step's active
    set from scratch.

    ``mode`` selects the stream sources of the ablation study (NanoSpec
    Sec. 4, ablation, Table 5): "full" is the method; "ctx_only" keeps only
    the prompt and the prefill candidates, S^(0), and adds nothing while
    decoding; "ext_only" keeps only the decoding tuples C_draft and C_ver and
    ignores the prompt context (the window rule is unchanged)."""

    def __init__(self, w_max: int, mode: str = "full"):
        if mode not in STREAM_MODES:
            raise ValueError(mode)
        self.w_max = int(w_max)
        self.mode = mode
        self.S: List[int] = []

    def append_prompt(self, prompt: Sequence[int]) -> None:
        if self.mode != "ext_only":
            self.S = self.S + [int(x) for x in prompt]

    def append_prefill_union(self, P: np.ndarray) -> None:
        if self.mode != "ext_only":
            self.S = self.S + first_occurrence(np.asarray(P).reshape(-1))

    def step(self, tree_ids: Sequence[int], ver_ids: Sequence[int]) -> None:
        if self.mode != "ctx_only":
            self.S = stream_update(self.S, tree_ids, ver_ids)

    def active(self) -> np.ndarray:
        return active_set(self.S, self.w_max)

    def window(self) -> List[int]:
        return suffix(self.S, self.w_max)
