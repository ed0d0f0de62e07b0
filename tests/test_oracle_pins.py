"""Pins for the CPU oracle: each checks it against something other than itself
(a hand-worked example, textbook/library special cases, brute-force
re-characterisations from a different sentence of the pages, exact integer
arithmetic).  ``test_oracle_mutations.py`` plants plausible mistakes in the
oracle and checks that at least one pin below catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle.nanospec_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _vals(x):
    return np.array([[(-math.inf if v == "-inf" else v) for v in row] for row in x], dtype=np.float64)


# ---------------------------------------------------------------------------
# Pin functions (take the oracle module so mutated copies can be checked)
# ---------------------------------------------------------------------------


def pin_worked_example(o):
    g = _golden()
    Z = np.asarray(g["Z"], dtype=np.float32)
    P_ids, P_vals = o.prefill_topk(Z, g["k_pre"], "fp32")
    assert P_ids.tolist() == g["expect_P_ids"]
    assert P_vals.tolist() == g["expect_P_vals"]
    assert o.first_occurrence(P_ids.reshape(-1)) == g["expect_U"]
    S = o.init_stream(g["prompt"], P_ids)
    assert S == g["expect_S_init"]
    I1 = o.active_set(S, g["w_max"])
    assert I1.tolist() == g["expect_I1"]
    assert o.bitmap(I1, g["V"]).tolist() == g["expect_bitmap1"]
    assert o.draft_candidates(g["tree"]) == g["expect_C_draft"]
    S = o.stream_update(S, g["tree"], g["ver"])
    assert S == g["expect_S_step1"]
    assert o.suffix(S, g["w_max"]) == g["expect_window_step1"]
    I2 = o.active_set(S, g["w_max"])
    assert I2.tolist() == g["expect_I2"]
    assert o.bitmap(I2, g["V"]).tolist() == g["expect_bitmap2"]
    W = np.asarray(g["W"], dtype=np.float32)
    h = np.asarray(g["h"], dtype=np.float32)
    logits = o.project(h, o.gather_rows(W, I2), "fp32")
    assert logits.tolist() == g["expect_logits_I2"]
    ids, vals = o.draft_topk(logits, I2, g["k"])
    assert ids.tolist() == g["expect_topk_ids"]
    assert vals.tolist() == g["expect_topk_vals"]
    ids, vals = o.draft_topk(logits, I2, g["k_pad"])
    assert ids.tolist() == g["expect_topk_ids_pad"]
    np.testing.assert_array_equal(vals, _vals(g["expect_topk_vals_pad"]))
    _, ids2, vals2 = o.draft_head(h, W, I2, g["k"], "fp32")
    assert ids2.tolist() == g["expect_topk_ids"] and vals2.tolist() == g["expect_topk_vals"]
    assert o.dense_logits(h, W, "fp32")[0].tolist() == g["expect_dense_logits_row0"]


def pin_widen_bf16(o):
    # Known bfloat16 bit patterns (IEEE-754 binary32 upper halves).
    cases = {
        0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625, 0x4000: 2.0, 0xC040: -3.0,
        0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,
        0x3C00: 2.0 ** -7, 0x0000: 0.0,
    }
    bits = np.array(list(cases.keys()), dtype=np.uint16)
    got = o.widen(bits, "bf16")
    assert got.dtype == np.float64
    assert got.tolist() == list(cases.values())
    neg0 = o.widen(np.array([0x8000], np.uint16), "bf16")[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0
    f = np.array([1.5, -2.25, 3.0e-40], np.float32)
    assert o.widen(f, "fp32").tolist() == [float(x) for x in f]


def pin_widen_fp16(o):
    # Known IEEE binary16 bit patterns.
    cases = {
        0x3C00: 1.0, 0xBC00: -1.0, 0x4000: 2.0, 0xC200: -3.0, 0x3800: 0.5, 0x3555: 0.25 * (1 + 0x155 / 1024),
        0x7BFF: 65504.0, 0x0400: 2.0 ** -14, 0x03FF: 1023 * 2.0 ** -24, 0x0001: 2.0 ** -24, 0x0000: 0.0,
        0x4248: 3.140625,
    }
    bits = np.array(list(cases.keys()), dtype=np.uint16)
    got = o.widen(bits, "fp16")
    assert got.dtype == np.float64
    assert got.tolist() == list(cases.values())
    neg0 = o.widen(np.array([0x8000], np.uint16), "fp16")[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0


def _rank_topk(z, K):
    """Brute force from the rank characterisation: index i is among the top K
    iff fewer than K entries beat it, where j beats i when z_j > z_i or
    (z_j == z_i and j < i); the result is ordered by that rank."""
    n = len(z)
    rank = [sum(1 for j in range(n) if z[j] > z[i] or (z[j] == z[i] and j < i)) for i in range(n)]
    sel = [i for i in range(n) if rank[i] < K]
    return sorted(sel, key=lambda i: rank[i])


def pin_topk_bruteforce(o):
    rng = np.random.default_rng(11)
    for trial in range(150):
        n = int(rng.integers(1, 24))
        z = rng.integers(-3, 4, size=n).astype(np.float64)   # many ties
        for K in range(0, n + 3):
            got = o.top_k(z, K).tolist()
            assert got == _rank_topk(z.tolist(), K), (z, K, got)
    # +0.0 and -0.0 compare equal, so the lower index wins.
    assert o.top_k(np.array([0.0, -0.0]), 1).tolist() == [0]
    assert o.top_k(np.array([-0.0, 0.0]), 1).tolist() == [0]


def pin_topk_library_cases(o):
    rng = np.random.default_rng(12)
    for _ in range(50):
        z = rng.standard_normal(int(rng.integers(1, 500)))
        assert o.top_k(z, 1).tolist() == [int(np.argmax(z))]          # first maximum
        K = int(rng.integers(1, len(z) + 1))
        t = o.top_k(z, K)
        np.testing.assert_array_equal(z[t], np.sort(z)[::-1][:K])     # values = sorted prefix
        assert len(set(t.tolist())) == K


def pin_prefill_planted(o):
    """Rows with K planted peaks far above the background: T_K returns exactly
    the planted ids, ordered by peak height."""
    rng = np.random.default_rng(13)
    V, K = 300, 5
    Z = rng.uniform(-1, 1, size=(20, V)).astype(np.float32)
    planted = np.stack([rng.choice(V, size=K, replace=False) for _ in range(20)])
    heights = np.arange(K, 0, -1, dtype=np.float32) * 10.0
    for i in range(20):
        Z[i, planted[i]] = heights
    ids, vals = o.prefill_topk(Z, K, "fp32")
    np.testing.assert_array_equal(ids, planted)
    np.testing.assert_array_equal(vals, np.tile(heights, (20, 1)))


def pin_first_occurrence(o):
    assert o.first_occurrence([5, 3, 5, 1, 3, 9]) == [5, 3, 1, 9]
    assert o.first_occurrence([]) == []
    rng = np.random.default_rng(14)
    for _ in range(100):
        x = rng.integers(0, 12, size=int(rng.integers(0, 40))).tolist()
        u = o.first_occurrence(x)
        assert len(u) == len(set(u)) and set(u) == set(x)
        assert [x.index(v) for v in u] == sorted(x.index(v) for v in u)


def pin_stream_update(o):
    """S_new keeps every earlier entry and repeats across tuples (no dedup
    against S or between C_draft and C_ver)."""
    S = [1, 2, 3]
    out = o.stream_update(S, [3, 3, 4], [4, 1])
    assert out == [1, 2, 3, 3, 4, 4, 1]
    assert S == [1, 2, 3]
    assert o.init_stream([2, 2], np.array([[2, 5], [5, 7]])) == [2, 2, 2, 5, 7]


def _last_occurrence_active(S, w_max, V):
    """Recency characterisation (NanoSpec, sliding-window paragraph): an id is
    active iff its most recent occurrence lies inside the last W_max entries."""
    last = {}
    for p, v in enumerate(S):
        last[v] = p
    lo = len(S) - w_max
    return sorted(v for v, p in last.items() if p >= lo)


def pin_active_set_bruteforce(o):
    rng = np.random.default_rng(15)
    for _ in range(200):
        V = int(rng.integers(8, 65))
        S = rng.integers(0, V, size=int(rng.integers(0, 200))).tolist()
        for w_max in (1, 2, 5, 17, 64, 250):
            I = o.active_set(S, w_max)
            assert I.tolist() == _last_occurrence_active(S, w_max, V)
            assert len(I) <= min(w_max, V, len(S))
            bm = o.bitmap(I, V)
            assert sum(bin(int(w)).count("1") for w in bm) == len(I)
            for v in range(V):
                assert bool((int(bm[v >> 5]) >> (v & 31)) & 1) == (v in set(I.tolist()))


def pin_active_full_coverage(o):
    V = 37
    S = list(range(V))[::-1] + [3, 3]
    assert o.active_set(S, len(S)).tolist() == list(range(V))
    assert o.active_set(S, 10**6).tolist() == list(range(V))


def pin_bitmap_tail(o):
    V = 70   # 3 words, 6 bits used in the last one
    I = np.array([0, 31, 32, 63, 64, 69])
    bm = o.bitmap(I, V)
    assert bm.tolist() == [0x80000001, 0x80000001, 0x21]


def pin_projection_exact(o):
    """Integer-valued inputs (exact in bf16 and fp32, sums exact in float64):
    the projection equals exact integer arithmetic.  M, n and d all differ so
    a transposed operand cannot pass."""
    rng = np.random.default_rng(16)
    M, V, d = 3, 40, 24
    Wi = rng.integers(-8, 9, size=(V, d))
    hi = rng.integers(-8, 9, size=(M, d))
    I = np.array([1, 4, 5, 9, 20, 33, 39])
    exact = [[sum(int(hi[m, c]) * int(Wi[v, c]) for c in range(d)) for v in I] for m in range(M)]
    Wf = Wi.astype(np.float32)
    hf = hi.astype(np.float32)
    assert o.project(hf, o.gather_rows(Wf, I), "fp32").tolist() == exact
    Wb = (Wf.view(np.uint32) >> 16).astype(np.uint16)        # small ints are exact bf16
    hb = (hf.view(np.uint32) >> 16).astype(np.uint16)
    assert o.project(hb, o.gather_rows(Wb, I), "bf16").tolist() == exact
    dense = o.dense_logits(hb, Wb, "bf16")
    assert dense.shape == (M, V)
    assert dense[:, I].tolist() == exact


def pin_gather(o):
    W = np.arange(50, dtype=np.uint16).reshape(10, 5)
    I = np.array([0, 3, 9])
    np.testing.assert_array_equal(o.gather_rows(W, I), np.stack([W[0], W[3], W[9]]))


def pin_subset_equals_dense(o):
    """Subset logits are the matching columns of the full-vocabulary head, and
    with every id active the draft top-k is the dense top-k."""
    rng = np.random.default_rng(17)
    V, d, M, k = 97, 40, 5, 7
    W = rng.standard_normal((V, d)).astype(np.float32)
    h = rng.standard_normal((M, d)).astype(np.float32)
    dense = o.dense_logits(h, W, "fp32")
    I = np.sort(rng.choice(V, size=30, replace=False))
    np.testing.assert_allclose(o.project(h, o.gather_rows(W, I), "fp32"), dense[:, I],
                               rtol=0, atol=1e-12)
    S = rng.permutation(V).tolist()
    I_all = o.active_set(S, V)
    assert I_all.tolist() == list(range(V))
    _, ids, vals = o.draft_head(h, W, I_all, k, "fp32")
    for m in range(M):
        ref = _rank_topk(dense[m].tolist(), k)
        assert ids[m].tolist() == ref
        np.testing.assert_allclose(vals[m], dense[m, ref], rtol=0, atol=1e-12)


def pin_draft_topk_global_ids(o):
    """Ties are decided by global id, independent of the column order."""
    logits = np.array([[1.0, 2.0, 1.0, 2.0]])
    I = np.array([40, 7, 3, 9])
    ids, vals = o.draft_topk(logits, I, 3)
    assert ids.tolist() == [[7, 9, 3]] and vals.tolist() == [[2.0, 2.0, 1.0]]


def pin_stream_modes(o):
    """Ablation modes, from their descriptions: with the context only, the
    active set after any number of steps is the prompt's (capped by the window
    over the prompt); with the decoding tuples only, it is the window over the
    concatenated deduplicated tuples, as if the prompt had never been seen."""
    rng = np.random.default_rng(31)
    V, w = 40, 12
    prompt = rng.integers(0, V, size=20).tolist()
    steps = [(rng.integers(0, V, size=7).tolist(), rng.choice(V, size=3, replace=False).tolist())
             for _ in range(6)]
    ctx = o.Sequence_(w, "ctx_only")
    ctx.append_prompt(prompt)
    ext = o.Sequence_(w, "ext_only")
    ext.append_prompt(prompt)
    tail = []
    for tree, ver in steps:
        ctx.step(tree, ver)
        ext.step(tree, ver)
        seen = []
        for x in tree:                              # C_draft: first occurrences
            if x not in seen:
                seen.append(x)
        tail = tail + seen + list(ver)
        assert ctx.active().tolist() == sorted(set(prompt[-w:]))
        assert ext.active().tolist() == sorted(set(tail[-w:]))
    full = o.Sequence_(w)
    full.append_prompt(prompt)
    assert full.active().tolist() == sorted(set(prompt[-w:]))


def pin_log_softmax(o):
    """Closed forms: exp of the row sums to one over I, a constant added to a
    row cancels, and logits (0, ln 2, ln 3) give log(1/6, 2/6, 3/6)."""
    rng = np.random.default_rng(41)
    z = rng.standard_normal((4, 9)) * 3
    lp = o.log_softmax_active(z)
    np.testing.assert_allclose(np.exp(lp).sum(axis=1), 1.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o.log_softmax_active(z + 7.5), lp, rtol=0, atol=1e-12)
    got = o.log_softmax_active(np.array([[0.0, math.log(2), math.log(3)]]))[0]
    np.testing.assert_allclose(got, np.log([1 / 6, 2 / 6, 3 / 6]), rtol=0, atol=1e-12)
    assert (np.argsort(-lp, axis=1, kind="stable") == np.argsort(-z, axis=1, kind="stable")).all()


def pin_select_best(o):
    """Brute-force ranking of candidates with negative ids skipped."""
    rng = np.random.default_rng(43)
    for _ in range(20):
        v = rng.integers(-3, 3, size=30).astype(np.float64)     # many ties
        ids = rng.integers(-1, 5, size=30)
        k = int(rng.integers(1, 35))
        cand = [i for i in range(30) if ids[i] >= 0]
        rank = {i: sum(1 for j in cand if v[j] > v[i] or (v[j] == v[i] and j < i)) for i in cand}
        ref = sorted([i for i in cand if rank[i] < k], key=lambda i: rank[i])
        got = o.select_best(v, ids, k)
        assert got[:len(ref)].tolist() == ref and (got[len(ref):] == -1).all()


GOLDEN_TREE = os.path.join(os.path.dirname(__file__), "golden", "draft_tree.json")


def pin_draft_tree_worked_example(o):
    """The hand-worked tree of tests/golden/draft_tree.json."""
    from fractions import Fraction
    with open(GOLDEN_TREE) as f:
        g = json.load(f)
    sym = {"ln2": math.log(2), "-ln3": -math.log(3), "0": 0.0}
    hs = [np.array([[sym[x]] for x in row]) for row in g["h_symbolic"]]
    W = np.asarray(g["W"], dtype=np.float32)
    r = o.draft_tree(hs, W, np.asarray(g["I"]), g["K"], g["F"], g["N"], "fp32")
    assert r["ids"].tolist() == g["expect_ids"]
    probs = np.array([float(Fraction(p)) for p in g["expect_probs"]])
    np.testing.assert_allclose(np.exp(r["vals"]), probs, rtol=1e-6, atol=0)
    assert r["parent"].tolist() == g["expect_parent"] and r["depth"].tolist() == g["expect_depth"]
    assert [f.tolist() for f in r["frontiers"]] == g["expect_frontiers"]
    assert r["final"].tolist() == g["expect_final"]


def pin_draft_tree_invariants(o):
    """Random trees: every child's score is its parent's score plus its own
    log-probability over I (so it never exceeds the parent's), each depth's
    frontier is the brute-force best F of that depth's children, and the
    final N nodes are closed under taking parents."""
    rng = np.random.default_rng(47)
    V, d, K, F, N = 60, 12, 3, 4, 9
    W = rng.standard_normal((V, d)).astype(np.float32)
    I = np.sort(rng.choice(V, size=25, replace=False))
    hs = [rng.standard_normal((1, d))] + [rng.standard_normal((F, d)) for _ in range(3)]
    r = o.draft_tree(hs, W, I, K, F, N, "fp32")
    dense = W.astype(np.float64) @ np.asarray(hs[0], np.float64)[0].astype(np.float32).astype(np.float64)
    lse = np.log(np.exp(dense[I] - dense[I].max()).sum()) + dense[I].max()
    for i in range(K):
        assert r["parent"][i] == -1 and abs(r["vals"][i] - (dense[r["ids"][i]] - lse)) < 1e-9
    for i, p in enumerate(r["parent"]):
        if p >= 0:
            assert r["vals"][i] <= r["vals"][p] + 1e-12
    for t, fr in enumerate(r["frontiers"]):
        at = np.flatnonzero(r["depth"] == t)
        best = sorted(at, key=lambda i: (-r["vals"][i], i))[:F]
        assert fr.tolist() == best
    chosen = set(r["final"].tolist())
    assert all(r["parent"][i] < 0 or r["parent"][i] in chosen for i in chosen)


GOLDEN_PACKED = os.path.join(os.path.dirname(__file__), "golden", "packed_slots.json")


def pin_packed_worked_example(o):
    """The hand-worked slot placements of tests/golden/packed_slots.json."""
    with open(GOLDEN_PACKED) as f:
        g = json.load(f)
    slots = np.full(g["capacity"], -1, dtype=np.int64)
    for st in g["steps"]:
        slots, es, ei, n = o.packed_update(slots, np.array(st["I"], dtype=np.int64))
        assert slots.tolist() == st["slot_ids"], st["why"]
        assert list(es) == st["enter_slots"] and list(ei) == st["enter_ids"], st["why"]
        assert n == st["n_slots"], st["why"]


def pin_packed_invariants(o):
    """Random churn on a small vocabulary, checked against properties the
    placement rule implies on its own: the held ids are exactly I, an id that
    stays keeps its slot, the entering list is I minus what was held (ascending)
    and is what the update wrote, and every occupied slot lies below the largest
    |I| seen so far (entering ids take the lowest free slots, so the r-th of
    them lands below the count of ids held afterwards)."""
    rng = np.random.default_rng(23)
    V, cap = 60, 24
    slots = np.full(cap, -1, dtype=np.int64)
    peak = 0
    prev = {}
    for _ in range(300):
        n = int(rng.integers(0, cap + 1))
        I = np.sort(rng.choice(V, size=n, replace=False)) if rng.random() < 0.3 or not prev else \
            np.sort(np.array(list(set(rng.choice(list(prev), size=min(len(prev), max(0, n - 4)),
                                                    replace=False).tolist())
                                  | set(rng.choice(V, size=4, replace=False).tolist())))[:cap])
        new, es, ei, n_slots = o.packed_update(slots, I)
        held = {int(x): s for s, x in enumerate(new) if x >= 0}
        assert sorted(held) == I.tolist() and len(held) == int(np.sum(new >= 0))
        for x, s in prev.items():
            if x in held:
                assert held[x] == s
        assert list(ei) == sorted(set(I.tolist()) - set(prev)), "entering ids"
        assert all(new[s] == x for s, x in zip(es, ei))
        assert all(s < len(I) for s in es)
        peak = max(peak, len(I))
        assert all(s < peak for s in held.values())
        assert n_slots == (max(held.values()) + 1 if held else 0)
        slots, prev = new, held


def pin_packed_head(o):
    """The head over a slot map with holes equals the brute-force top-k of the
    dense logits restricted to the held ids, whatever their slots."""
    rng = np.random.default_rng(29)
    V, d, M, k = 70, 24, 3, 6
    W = rng.standard_normal((V, d)).astype(np.float32)
    h = rng.standard_normal((M, d)).astype(np.float32)
    dense = h.astype(np.float64) @ W.astype(np.float64).T
    slot_ids = np.full(40, -1, dtype=np.int64)
    held = rng.choice(V, size=25, replace=False)
    slot_ids[rng.choice(40, size=25, replace=False)] = held
    n_slots = int(np.flatnonzero(slot_ids >= 0).max()) + 1
    ids, vals = o.packed_draft_head(h, W, slot_ids, n_slots, k, "fp32")
    for m in range(M):
        col = np.full(V, -np.inf)
        col[held] = dense[m, held]
        ref = _rank_topk(col.tolist(), k)
        assert ids[m].tolist() == ref
        np.testing.assert_allclose(vals[m], dense[m, ref], rtol=0, atol=1e-9)


PINS = [pin_worked_example, pin_widen_bf16, pin_widen_fp16, pin_topk_bruteforce, pin_topk_library_cases,
        pin_prefill_planted, pin_first_occurrence, pin_stream_update,
        pin_active_set_bruteforce, pin_active_full_coverage, pin_bitmap_tail,
        pin_projection_exact, pin_gather, pin_subset_equals_dense, pin_draft_topk_global_ids,
        pin_packed_worked_example, pin_packed_invariants, pin_packed_head, pin_stream_modes,
        pin_log_softmax, pin_select_best, pin_draft_tree_worked_example, pin_draft_tree_invariants]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(O)
