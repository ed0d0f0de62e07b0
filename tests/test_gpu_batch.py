"""GPU parity of the batched entry points: B independent sequences, each
checked against its own CPU oracle sequence (window, active ids, bitmap, |S|
exactly; logits and top-k to the draft-head tolerance)."""
import numpy as np
import pytest
import torch

import oracle.nanospec_oracle as O
from dynamic_vocab_draft_amd import workloads as WL
from tests.gpu_common import dcode_of, bitmap_from_ids, check_logits, check_topk, dev_elems, dev_i32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ns():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocab_draft_amd import nanospec
    return nanospec


def member_state(ns, bt, b, V, w_max):
    m = bt.member(b)
    win = torch.empty(w_max, dtype=torch.int32, device="cuda")
    ln = torch.zeros(1, dtype=torch.int64, device="cuda")
    ns.nanospec_state_window(m, win, ln)
    torch.cuda.synchronize()
    L = int(ln.item())
    return L, win[:min(L, w_max)].cpu().numpy().astype(np.int64), win[min(L, w_max):].cpu().numpy()


def pack(lists, width):
    a = np.full((len(lists), max(width, 1)), -1, np.int32)
    for b, x in enumerate(lists):
        a[b, :len(x)] = x
    return dev_i32(a.reshape(-1)), dev_i32(np.array([len(x) for x in lists], np.int32))


def run_batch(ns, name, B, steps, check_steps, dtype=None, vary=False):
    base = WL.get_config(name, **({"dtype": dtype} if dtype else {}))
    cfgs = [WL.get_config(name, seed=base.seed + 100 * b, **({"dtype": dtype} if dtype else {})) for b in range(B)]
    say(f"batch {name} B={B}: generating inputs", base)
    W = WL.make_weights(base)
    W_dev = dev_elems(W, base.dtype)
    V, w_max, d, M, k = base.V, base.w_max, base.d, base.M, base.k
    scripts = [WL.make_id_script(c, steps) for c in cfgs]
    bt = ns.NanoSpecBatch(B, V, w_max)
    seqs = []
    for b in range(B):
        seq = O.Sequence_(w_max)
        seq.append_prompt(scripts[b].prompt)
        seqs.append(seq)
        ns.nanospec_stream_append(bt.member(b), dev_i32(scripts[b].prompt), len(scripts[b].prompt), 0)
    ids = torch.full((B, w_max), -7, dtype=torch.int32, device="cuda")
    n = torch.zeros(B, dtype=torch.int32, device="cuda")
    bm = torch.zeros((B, (V + 31) // 32), dtype=torch.int32, device="cuda")
    ws = ns.alloc_batch_workspace(B, w_max, M, k, d)
    logits = torch.empty((B, M, w_max), device="cuda")
    tids = torch.empty((B, M, k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((B, M, k), device="cuda")
    rng = np.random.default_rng(base.seed)
    for t in range(steps):
        trees = [scripts[b].tree[t] for b in range(B)]
        vers = [scripts[b].ver[t] for b in range(B)]
        if vary:                                   # different tuple sizes per sequence, some empty
            trees = [tr[:int(rng.integers(0, len(tr) + 1))] for tr in trees]
            vers = [vr[:int(rng.integers(0, len(vr) + 1))] for vr in vers]
        nd_max = max(len(x) for x in trees)
        nv_max = max(len(x) for x in vers)
        tr_dev, nd_dev = pack(trees, nd_max)
        vr_dev, nv_dev = pack(vers, nv_max)
        ns.nanospec_batch_step_update(bt, tr_dev, max(nd_max, 1), nd_dev, nd_max, vr_dev, max(nv_max, 1), nv_dev,
                                      nv_max, ids, n, bm)
        hs = [WL.make_hidden(cfgs[b], t) for b in range(B)]
        h_dev = dev_elems(np.stack(hs), base.dtype)
        logits.fill_(float("nan"))
        ns.nanospec_batch_draft_logits_topk(W_dev, ids, n, w_max, B, V, d,
                                            dcode_of(ns, base.dtype), h_dev, M, k, logits,
                                            tids, tvals, ws)
        torch.cuda.synchronize()
        n_h, ids_h, bm_h = n.cpu().numpy(), ids.cpu().numpy(), bm.cpu().numpy().view(np.uint32)
        lg, ti, tv = logits.cpu().numpy(), tids.cpu().numpy(), tvals.cpu().numpy()
        for b in range(B):
            seqs[b].step(trees[b], vers[b])
            I = seqs[b].active()
            what = f"batch {name} B={B} step {t} seq {b}"
            L, win, tail = member_state(ns, bt, b, V, w_max)
            assert L == len(seqs[b].S), what
            assert win.tolist() == seqs[b].window(), f"{what}: window"
            assert (tail == -1).all()
            assert n_h[b] == len(I), f"{what}: n {n_h[b]} vs {len(I)}"
            assert np.array_equal(ids_h[b, :len(I)], I), f"{what}: ids"
            assert np.array_equal(bm_h[b], bitmap_from_ids(I, V)), f"{what}: bitmap"
            if t in check_steps or steps <= 4:
                ref_logits, o_ids, o_vals = O.draft_head(hs[b], W, I, k, base.dtype)
                check_logits(lg[b][:, :len(I)], ref_logits, what)
                assert np.isnan(lg[b][:, len(I):]).all(), f"{what}: columns past n written"
                check_topk(ti[b], tv[b], ref_logits, I, o_ids, o_vals, k, what)
    for b in range(B):
        assert ns.nanospec_state_status(bt.member(b)) == 0


def test_batch_tiny(ns):
    for B in (1, 3, 8):
        run_batch(ns, "tiny", B, 8, set(range(8)), dtype="bf16")
    run_batch(ns, "tiny", 4, 6, set(range(6)))                      # fp32 draft head


def test_batch_varying_tuples(ns):
    run_batch(ns, "tiny", 5, 12, set(range(12)), dtype="bf16", vary=True)


def test_batch_llama3_8b(ns):
    run_batch(ns, "llama3_8b", 8, 24, {0, 23})


def test_batch_qwen25_7b(ns):
    # B = 3: 3 x 48 groups of 64 rows, the M-split projection; B = 2 (96
    # groups) keeps the k-split kernel, hidden rows staged through LDS.
    run_batch(ns, "qwen25_7b", 3, 6, {5})
    run_batch(ns, "qwen25_7b", 2, 4, {3})


def test_batch_many_columns(ns):
    """n_max > 4096 (chunked merge) with several sequences."""
    say("batch: chunked merge")
    rng = np.random.default_rng(31)
    V, d, M, k, B, n_max = 30000, 64, 4, 9, 3, 6000
    W = WL.f32_to_bf16_bits((rng.standard_normal((V, d)) * 0.1).astype(np.float32))
    W_dev = dev_elems(W, "bf16")
    Is = [np.sort(rng.choice(V, size=s, replace=False)) for s in (6000, 4097, 1500)]
    ids = np.full((B, n_max), -1, np.int32)
    for b, I in enumerate(Is):
        ids[b, :len(I)] = I
    hs = [WL.f32_to_bf16_bits(rng.standard_normal((M, d)).astype(np.float32)) for _ in range(B)]
    ws = ns.alloc_batch_workspace(B, n_max, M, k, d)
    tids = torch.empty((B, M, k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((B, M, k), device="cuda")
    logits = torch.full((B, M, n_max), float("nan"), device="cuda")
    ns.nanospec_batch_draft_logits_topk(W_dev, dev_i32(ids.reshape(-1)), dev_i32(np.array([len(I) for I in Is])),
                                        n_max, B, V, d, ns.NS_BF16, dev_elems(np.stack(hs), "bf16"), M, k, logits,
                                        tids, tvals, ws)
    torch.cuda.synchronize()
    for b, I in enumerate(Is):
        ref_logits, o_ids, o_vals = O.draft_head(hs[b], W, I, k, "bf16")
        check_logits(logits[b].cpu().numpy()[:, :len(I)], ref_logits, f"seq {b}")
        check_topk(tids[b].cpu().numpy(), tvals[b].cpu().numpy(), ref_logits, I, o_ids, o_vals, k, f"seq {b}")


def test_batch_member_calls_and_limits(ns):
    """Members accept the single-sequence calls; out-of-limit batched calls are
    rejected before launch."""
    V, w_max, B = 500, 40, 3
    bt = ns.NanoSpecBatch(B, V, w_max)
    seq = O.Sequence_(w_max)
    m1 = bt.member(1)
    ns.nanospec_stream_append(m1, dev_i32([5, 6, 5, 7]), 4, 1)
    seq.append_prompt(O.first_occurrence([5, 6, 5, 7]))
    ids = torch.empty(w_max, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    ns.nanospec_active_vocab(m1, ids, n)
    torch.cuda.synchronize()
    assert ids[:int(n.item())].cpu().tolist() == seq.active().tolist()
    L, win, _ = member_state(ns, bt, 0, V, w_max)                 # other members untouched
    assert L == 0
    z = torch.zeros(B * 600, dtype=torch.int32, device="cuda")
    c = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B * w_max, dtype=torch.int32, device="cuda")
    with pytest.raises(ns.NanoSpecError):
        ns.nanospec_batch_step_update(bt, z, 600, c, 600, z, 8, c, 8, out, c)     # nd_max > 512
    with pytest.raises(ns.NanoSpecError):
        ns.nanospec_batch_step_update(bt, z, 4, c, 8, z, 8, c, 8, out, c)         # stride < nd_max


def test_many_active_ids_staged(ns):
    """More than 4096 active ids (the compaction staged in LDS, then copied
    out), for a single state and for batch members whose active-id outputs
    start off 16-byte alignment (W_max not a multiple of 4): ids, counts and
    bitmaps bit-exact against the oracle at every step."""
    say("many active ids: staged compaction")
    rng = np.random.default_rng(41)
    V = 200000                                        # uniform ids over a large V: nearly all distinct
    for w_max, B in ((4403, 1), (5001, 3)):
        bt = ns.NanoSpecBatch(B, V, w_max)
        seqs = []
        for b in range(B):
            prompt = rng.integers(0, V, size=w_max + 500).astype(np.int32)
            seq = O.Sequence_(w_max)
            seq.append_prompt(prompt)
            seqs.append(seq)
            ns.nanospec_stream_append(bt.member(b), dev_i32(prompt), len(prompt), 0)
        ids = torch.full((B, w_max), -7, dtype=torch.int32, device="cuda")
        n = torch.zeros(B, dtype=torch.int32, device="cuda")
        bm = torch.zeros((B, (V + 31) // 32), dtype=torch.int32, device="cuda")
        for step in range(4):
            trees = [rng.integers(0, V, size=400).astype(np.int32) for _ in range(B)]
            vers = [rng.choice(V, size=8, replace=False).astype(np.int32) for _ in range(B)]
            td, nd = pack(trees, 400)
            tv, nv = pack(vers, 8)
            ns.nanospec_batch_step_update(bt, td, 400, nd, 400, tv, 8, nv, 8, ids, n, bm)
            torch.cuda.synchronize()
            for b in range(B):
                seqs[b].step(trees[b], vers[b])
                I = seqs[b].active()
                got_n = int(n[b].item())
                assert len(I) > 4096, f"W_max={w_max}: only {len(I)} active ids"
                assert got_n == len(I), f"W_max={w_max} seq {b} step {step}: n {got_n} vs {len(I)}"
                assert np.array_equal(ids[b, :got_n].cpu().numpy(), I), f"W_max={w_max} seq {b} step {step}: ids"
                assert np.array_equal(bm[b].cpu().numpy().view(np.uint32), bitmap_from_ids(I, V)), "bitmap"
            if B == 1:
                # the single-sequence entry point on the same state
                m = bt.member(0)
                ids1 = torch.full((w_max,), -7, dtype=torch.int32, device="cuda")
                n1 = torch.zeros(1, dtype=torch.int32, device="cuda")
                tree, ver = rng.integers(0, V, size=300).astype(np.int32), rng.choice(V, size=8, replace=False)
                ns.nanospec_step_update(m, dev_i32(tree), len(tree), dev_i32(ver), len(ver), ids1, n1)
                torch.cuda.synchronize()
                seqs[0].step(tree, ver)
                I = seqs[0].active()
                assert len(I) > 4096, f"few active ids: {len(I)}"
                assert int(n1.item()) == len(I) and np.array_equal(ids1[:len(I)].cpu().numpy(), I), "single-state ids"


@pytest.mark.parametrize("M,dtype,B", [(8, "bf16", 6), (20, "bf16", 6), (16, "fp16", 6), (8, "bf16", 32),
                                       (8, "fp16", 64), (8, "bf16", 64)])
def test_batch_rows_beyond_one_pass(ns, M, dtype, B):
    """A batched head launches the tiles of 1024 rows per sequence and steps
    on by that much while rows are live (tiles of 16, 32 or 64 rows as B
    grows, with M <= 8): sequences with 3072, 2500, 1025, 1024, 17, 0, 777,
    64, 65 and 1 live rows of n_max = 3072, repeated up to B, each checked
    against the oracle (logits to tolerance, top-k by the set rule)."""
    say(f"batched head past one pass: M={M} {dtype} B={B}")
    rng = np.random.default_rng(61 + M + B)
    V, d, k, n_max = 50000, 512, 8, 3072
    pattern = [3072, 2500, 1025, 1024, 17, 0, 777, 64, 65, 1]
    counts = [pattern[b % len(pattern)] for b in range(B)]
    W = WL.to_bits((rng.standard_normal((V, d)) * 0.02).astype(np.float32), dtype)
    W_dev = dev_elems(W, dtype)
    ids = np.full((B, n_max), -1, np.int32)
    Is = []
    for b, c in enumerate(counts):
        I = np.sort(rng.choice(V, size=c, replace=False)).astype(np.int64)
        ids[b, :c] = I
        Is.append(I)
    hs = [WL.to_bits(rng.standard_normal((M, d)).astype(np.float32), dtype) for _ in range(B)]
    ws = ns.alloc_batch_workspace(B, n_max, M, k, d)
    logits = torch.full((B, M, n_max), float("nan"), device="cuda")
    tids = torch.empty((B, M, k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((B, M, k), device="cuda")
    ns.nanospec_batch_draft_logits_topk(W_dev, dev_i32(ids.reshape(-1)), dev_i32(np.array(counts, np.int32)), n_max,
                                        B, V, d, dcode_of(ns, dtype), dev_elems(np.stack(hs), dtype), M, k, logits,
                                        tids, tvals, ws)
    torch.cuda.synchronize()
    lg, ti, tv = logits.cpu().numpy(), tids.cpu().numpy(), tvals.cpu().numpy()
    for b in range(B):
        ref, o_ids, o_vals = O.draft_head(hs[b], W, Is[b], k, dtype)
        c = counts[b]
        check_logits(lg[b][:, :c], ref, f"sequence {b} ({c} live)")
        assert np.isnan(lg[b][:, c:]).all(), f"sequence {b}: columns past n written"
        check_topk(ti[b], tv[b], ref, Is[b], o_ids, o_vals, k, f"sequence {b} ({c} live)")
