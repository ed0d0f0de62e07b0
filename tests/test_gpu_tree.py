"""GPU parity of tree drafting: the draft head with log-probabilities over the
active set (values parent + z - lse), the best-k candidate selection, and the
multi-depth loop built from them.

* Head: top-k ids by the set rule and values to the draft-head tolerance
  |d| <= 1e-2 + 1e-2 |ref| (as for the logits head), lse to the same bound.
* Selection: the same float32 inputs on both sides, so indices, values and
  ids are compared exactly (ties by flat index).
* Loop: integer-valued weights and hidden rows make every logit an exact
  integer on both sides, so each row's order (ties by global id) is decided
  identically; only the float32 log-sum-exp and the running parent sums
  differ (below 1e-5 here).  Inputs are used only if the oracle's decisions
  across rows (frontier order and boundary, final boundary) have margins above
  2e-4; the trees are then compared exactly, scores within 1e-4.
* Full-size loop (Llama shapes, bf16): invariants that hold at any size."""
import numpy as np
import pytest
import torch

import oracle.nanospec_oracle as O
from dynamic_vocab_draft_amd import workloads as WL
from tests.gpu_common import dcode_of, check_topk, dev_elems, dev_i32, say, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ns():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocab_draft_amd import nanospec
    return nanospec


def logprob_call(ns, W_dev, I, n_max, V, d, dtype, h, M, k, parent, mode=None, with_lse=True):
    mode = ns.NS_INDEXED if mode is None else mode
    ids = torch.full((n_max,), -1, dtype=torch.int32, device="cuda")
    ids[:len(I)] = dev_i32(I)
    n_dev = torch.tensor([len(I)], dtype=torch.int32, device="cuda")
    dcode = dcode_of(ns, dtype)
    rows = W_dev
    if mode == ns.NS_PACKED:
        rows = torch.zeros((n_max, d), dtype=W_dev.dtype, device="cuda")
        ns.nanospec_gather_rows(W_dev, V, d, dcode, ids, n_dev, n_max, rows)
    lse = torch.full((M,), float("nan"), device="cuda") if with_lse else None
    tids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((M, k), device="cuda")
    ws = ns.alloc_workspace(n_max, M, k, d)
    par = None if parent is None else torch.as_tensor(np.asarray(parent, np.float32)).cuda()
    ns.nanospec_draft_logprob_topk(rows, mode, ids, n_dev, n_max, V, d, dcode, dev_elems(h, dtype), M, k, par, lse,
                                   None, tids, tvals, ws)
    torch.cuda.synchronize()
    return tids.cpu().numpy(), tvals.cpu().numpy(), None if lse is None else lse.cpu().numpy()


def test_logprob_head(ns):
    """Column counts through every merge path (one chunk, one wide chunk,
    several chunks with the key merge, chunk 0 alone), with and without
    parent scores, both row modes and both dtypes, and an empty active set."""
    say("log-prob head")
    rng = np.random.default_rng(51)
    V = 20000
    for dtype in ("bf16", "fp32"):
        for d, M, k, n, n_max, with_parent in ((64, 4, 8, 300, 1024, True), (128, 10, 10, 3000, 3072, True),
                                               (64, 3, 16, 7000, 8192, False), (64, 2, 64, 9000, 12000, True),
                                               (64, 5, 8, 2000, 12000, True), (64, 2, 4, 0, 3072, True),
                                               (64, 1, 1, 1, 1024, True)):
            Wf = (rng.standard_normal((V, d)) * 0.3).astype(np.float32)
            W = WL.f32_to_bf16_bits(Wf) if dtype == "bf16" else Wf
            W_dev = dev_elems(W, dtype)
            hf = rng.standard_normal((M, d)).astype(np.float32)
            h = WL.f32_to_bf16_bits(hf) if dtype == "bf16" else hf
            I = np.sort(rng.choice(V, size=n, replace=False))
            # float32 parent scores, the values both sides use
            parent = rng.uniform(-6, 0, size=M).astype(np.float32).astype(np.float64) if with_parent else None
            for mode in (ns.NS_INDEXED, ns.NS_PACKED):
                what = f"{dtype} d={d} M={M} k={k} n={n} n_max={n_max} parent={with_parent} mode={mode}"
                g_ids, g_vals, g_lse = logprob_call(ns, W_dev, I, n_max, V, d, dtype, h, M, k, parent, mode)
                logp, o_ids, o_vals = O.draft_logprob_topk(h, W, I, k, dtype, parent)
                shift = 0.0 if parent is None else parent[:, None]
                if n == 0:
                    assert (g_ids == -1).all() and np.isneginf(g_vals).all() and np.isneginf(g_lse).all(), what
                    continue
                z = O.project(h, O.gather_rows(W, I), dtype)
                mx = z.max(axis=1)
                lse_ref = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))
                assert (np.abs(g_lse - lse_ref) <= tol(lse_ref)).all(), f"{what}: lse"
                check_topk(g_ids, g_vals, logp + shift, I, o_ids, o_vals, k, what)


def test_tree_select(ns):
    """Exact against the oracle's selection on the same float32 candidates:
    many ties, empty (-1) candidates, -inf scores, every per-thread count."""
    say("tree select")
    rng = np.random.default_rng(53)
    for C in (1, 5, 100, 1024, 1025, 2048, 2049, 4096):
        for k in (1, 10, 60, 64):
            B = 3
            vals = rng.integers(-20, 5, size=(B, C)).astype(np.float32) * np.float32(0.25)
            vals[rng.random((B, C)) < 0.05] = -np.inf
            ids = rng.integers(0, 5000, size=(B, C)).astype(np.int32)
            ids[rng.random((B, C)) < 0.1] = -1
            oi = torch.empty((B, k), dtype=torch.int32, device="cuda")
            ov = torch.empty((B, k), device="cuda")
            od = torch.empty((B, k), dtype=torch.int32, device="cuda")
            ns.nanospec_tree_select(torch.as_tensor(vals).cuda(), dev_i32(ids.reshape(-1)), C, B, k, oi, ov, od)
            torch.cuda.synchronize()
            gi, gv, gd = oi.cpu().numpy(), ov.cpu().numpy(), od.cpu().numpy()
            for b in range(B):
                ref = O.select_best(vals[b], ids[b], k)
                what = f"select C={C} k={k} b={b}"
                assert gi[b].tolist() == ref.tolist(), what
                live = ref >= 0
                assert np.array_equal(gv[b][live], vals[b][ref[live]]) and np.isneginf(gv[b][~live]).all(), what
                assert np.array_equal(gd[b][live], ids[b][ref[live]]) and (gd[b][~live] == -1).all(), what


def gpu_tree(ns, W_dev, I, n_max, V, d, dtype, hs, K, F, N):
    """The multi-depth loop on the GPU: one log-prob head and one selection
    per depth (parents' scores stay on the device), then the final
    selection.  Returns the pool, each depth's frontier (pool indices) and the
    final pool indices."""
    D = len(hs)
    P = K + (D - 1) * F * K
    ids = torch.full((n_max,), -1, dtype=torch.int32, device="cuda")
    ids[:len(I)] = dev_i32(I)
    n_dev = torch.tensor([len(I)], dtype=torch.int32, device="cuda")
    dcode = dcode_of(ns, dtype)
    pool_ids = torch.full((P,), -7, dtype=torch.int32, device="cuda")
    pool_vals = torch.full((P,), float("nan"), device="cuda")
    f_idx = torch.empty((D, F), dtype=torch.int32, device="cuda")
    f_vals = torch.empty((D, F), device="cuda")
    f_ids = torch.empty((D, F), dtype=torch.int32, device="cuda")
    ws = ns.alloc_workspace(n_max, F, K, d)
    base = 0
    bases = []
    for t, h in enumerate(hs):
        M = 1 if t == 0 else F
        parent = None if t == 0 else f_vals[t - 1]
        ns.nanospec_draft_logprob_topk(W_dev, ns.NS_INDEXED, ids, n_dev, n_max, V, d, dcode, dev_elems(h[:M], dtype),
                                       M, K, parent, None, None, pool_ids[base:base + M * K],
                                       pool_vals[base:base + M * K], ws)
        ns.nanospec_tree_select(pool_vals[base:base + M * K], pool_ids[base:base + M * K], M * K, 1, F, f_idx[t],
                                f_vals[t], f_ids[t])
        bases.append(base)
        base += M * K
    fin_idx = torch.empty(N, dtype=torch.int32, device="cuda")
    fin_vals = torch.empty(N, device="cuda")
    fin_ids = torch.empty(N, dtype=torch.int32, device="cuda")
    ns.nanospec_tree_select(pool_vals, pool_ids, P, 1, N, fin_idx, fin_vals, fin_ids)
    torch.cuda.synchronize()
    fi = f_idx.cpu().numpy()
    frontiers = [np.array([bases[t] + i for i in fi[t] if i >= 0]) for t in range(D)]
    parent = np.full(P, -1, np.int64)
    for t in range(1, D):
        for m in range(F):
            parent[bases[t] + m * K: bases[t] + (m + 1) * K] = frontiers[t - 1][m]
    return {"ids": pool_ids.cpu().numpy(), "vals": pool_vals.cpu().numpy(), "parent": parent,
            "frontiers": frontiers, "final": fin_idx.cpu().numpy(), "final_vals": fin_vals.cpu().numpy(),
            "final_ids": fin_ids.cpu().numpy()}


def cross_row_margin(r, K, F, N):
    """Smallest score gap at the oracle's decisions between candidates of
    different rows (different parent or depth): adjacent pairs among each
    depth's best F + 1 children and among the best N + 1 nodes.  Candidates of
    one row share its shift, so their order is decided exactly on both sides
    (equal scores by flat index)."""
    v, depth, parent = r["vals"], r["depth"], r["parent"]
    gaps = [np.inf]

    def scan(idx, top):
        order = sorted(idx, key=lambda i: (-v[i], i))[:top + 1]
        for a, b in zip(order, order[1:]):
            if parent[a] != parent[b] or depth[a] != depth[b]:
                gaps.append(v[a] - v[b])

    for t in range(len(r["frontiers"])):
        scan(np.flatnonzero(depth == t).tolist(), F)
    scan(list(range(len(v))), N)
    return float(np.min(gaps))


def test_draft_tree_loop_exact(ns):
    say("draft tree loop, integer-exact logits")
    V, d, K, F, N, D = 2048, 16, 10, 10, 60, 5
    for dtype in ("fp32", "bf16"):
        found = 0
        for seed in range(40):
            rng = np.random.default_rng(1000 + seed)
            Wf = rng.integers(-1, 2, size=(V, d)).astype(np.float32)
            I = np.sort(rng.choice(V, size=400, replace=False))
            hs = [rng.integers(-1, 2, size=(1 if t == 0 else F, d)).astype(np.float32) for t in range(D)]
            W = WL.f32_to_bf16_bits(Wf) if dtype == "bf16" else Wf      # small integers are exact in bf16
            hq = [WL.f32_to_bf16_bits(h) if dtype == "bf16" else h for h in hs]
            r = O.draft_tree(hq, W, I, K, F, N, dtype)
            if cross_row_margin(r, K, F, N) <= 2e-4:
                continue
            g = gpu_tree(ns, dev_elems(W, dtype), I, 3072, V, d, dtype, hq, K, F, N)
            what = f"{dtype} seed {seed}"
            assert g["ids"].tolist() == r["ids"].tolist(), f"{what}: pool ids"
            assert np.abs(g["vals"] - r["vals"]).max() <= 1e-4, f"{what}: pool scores"
            assert [f.tolist() for f in g["frontiers"]] == [f.tolist() for f in r["frontiers"]], f"{what}: frontiers"
            assert g["parent"].tolist() == r["parent"].tolist(), f"{what}: parents"
            assert g["final"].tolist() == r["final"].tolist(), f"{what}: final"
            found += 1
            if found == 3:
                break
        assert found == 3, f"{dtype}: too few seeds with clear decision margins"


def test_draft_tree_loop_llama_invariants(ns):
    """Depth 5, 10 x 10 children, 60 final nodes on the Llama-shaped workload
    (bf16, |I| from its stream): the head at depth 0 against the oracle, and
    for the whole loop the invariants of the tree rule on the GPU's own
    results."""
    say("draft tree loop, Llama shapes")
    cfg = WL.get_config("llama3_8b")
    K, F, N, D = 10, 10, 60, 5
    W = WL.make_weights(cfg)
    W_dev = dev_elems(W, cfg.dtype)
    script = WL.make_id_script(cfg, 4)
    seq = O.Sequence_(cfg.w_max)
    seq.append_prompt(script.prompt)
    for t in range(4):
        seq.step(script.tree[t], script.ver[t])
    I = seq.active()
    rng = np.random.default_rng(61)
    hs = [WL.f32_to_bf16_bits(rng.standard_normal((1 if t == 0 else F, cfg.d)).astype(np.float32)) for t in range(D)]
    g = gpu_tree(ns, W_dev, I, cfg.w_max, cfg.V, cfg.d, cfg.dtype, hs, K, F, N)
    logp, o_ids, o_vals = O.draft_logprob_topk(hs[0], W, I, K, cfg.dtype)
    check_topk(g["ids"][None, :K], g["vals"][None, :K], logp, I, o_ids, o_vals, K, "depth 0")
    v, p, ids = g["vals"].astype(np.float64), g["parent"], g["ids"]
    Iset = set(I.tolist())
    assert all(int(x) in Iset for x in ids), "pool id outside the active set"
    for blk in range(0, len(ids), K):
        row = ids[blk:blk + K]
        assert len(set(row.tolist())) == K, "repeated child in one row"
        assert (np.diff(v[blk:blk + K]) <= 0).all(), "children not in score order"
    for i in range(len(v)):
        if p[i] >= 0:
            assert v[i] <= v[p[i]] + 1e-5, "child scores above its parent"
    bases = [0] + [K + t * F * K for t in range(D - 1)]
    for t, fr in enumerate(g["frontiers"]):
        lo, hi = bases[t], bases[t] + (K if t == 0 else F * K)
        best = sorted(range(lo, hi), key=lambda i: (-v[i], i))[:F]
        assert fr.tolist() == best, f"frontier {t}"
    assert g["final"].tolist() == sorted(range(len(v)), key=lambda i: (-v[i], i))[:N]
    chosen = set(g["final"].tolist())
    assert all(p[i] < 0 or p[i] in chosen for i in chosen), "final tree not closed under parents"


def test_batched_logprob_and_selection(ns):
    """B sequences in one log-prob head call (different active sets and
    counts, per-sequence parents) against the oracle by the set rule, and one
    batched selection over the head's output, checked as the best F of its
    own inputs."""
    say("batched log-prob head and selection")
    rng = np.random.default_rng(71)
    V, d, M, k, n_max, F = 30000, 128, 6, 10, 9000, 8
    W = WL.f32_to_bf16_bits((rng.standard_normal((V, d)) * 0.3).astype(np.float32))
    W_dev = dev_elems(W, "bf16")
    sizes = (3000, 40, 9000, 0, 5000)
    B = len(sizes)
    Is = [np.sort(rng.choice(V, size=s, replace=False)) for s in sizes]
    ids = np.full((B, n_max), -1, np.int32)
    for b, I in enumerate(Is):
        ids[b, :len(I)] = I
    hs = [WL.f32_to_bf16_bits(rng.standard_normal((M, d)).astype(np.float32)) for _ in range(B)]
    parent = rng.uniform(-5, 0, size=(B, M)).astype(np.float32)
    ws = ns.alloc_batch_workspace(B, n_max, M, k, d)
    tids = torch.empty((B, M, k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((B, M, k), device="cuda")
    lse = torch.empty((B, M), device="cuda")
    ns.nanospec_batch_draft_logprob_topk(W_dev, dev_i32(ids.reshape(-1)), dev_i32(np.array(sizes, np.int32)), n_max,
                                         B, V, d, ns.NS_BF16, dev_elems(np.stack(hs), "bf16"), M, k,
                                         torch.as_tensor(parent).cuda(), lse, None, tids, tvals, ws)
    oi = torch.empty((B, F), dtype=torch.int32, device="cuda")
    ov = torch.empty((B, F), device="cuda")
    od = torch.empty((B, F), dtype=torch.int32, device="cuda")
    ns.nanospec_tree_select(tvals, tids, M * k, B, F, oi, ov, od)
    torch.cuda.synchronize()
    ti, tv, gl = tids.cpu().numpy(), tvals.cpu().numpy(), lse.cpu().numpy()
    gi, gv, gd = oi.cpu().numpy(), ov.cpu().numpy(), od.cpu().numpy()
    for b, I in enumerate(Is):
        what = f"batched log-prob seq {b} n={len(I)}"
        p64 = parent[b].astype(np.float64)
        logp, o_ids, o_vals = O.draft_logprob_topk(hs[b], W, I, k, "bf16", p64)
        if len(I) == 0:
            assert (ti[b] == -1).all() and np.isneginf(tv[b]).all() and np.isneginf(gl[b]).all(), what
        else:
            check_topk(ti[b], tv[b], logp + p64[:, None], I, o_ids, o_vals, k, what)
        # The selection as a property of its own inputs: the best F of the
        # head's candidates by (score desc, index asc), empty ones skipped.
        cv, cid = tv[b].reshape(-1), ti[b].reshape(-1)
        best = sorted([i for i in range(len(cv)) if cid[i] >= 0], key=lambda i: (-cv[i], i))[:F]
        assert gi[b][:len(best)].tolist() == best and (gi[b][len(best):] == -1).all(), what
        assert np.array_equal(gv[b][:len(best)], cv[best]) and np.array_equal(gd[b][:len(best)], cid[best]), what
