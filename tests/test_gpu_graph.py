"""HIP-graph capture of a whole decode step (state update, gather on a second
stream, draft head in both row modes), of the batched calls, of a step with
the slot-stable buffer updated on a second stream, and of a tree-drafting
step: each replay, with eager work and synchronisations between replays, must
give exactly the outputs of the same calls run eagerly on a twin state."""
import numpy as np
import pytest
import torch

from dynamic_vocab_draft_amd import workloads as WL
from tests.gpu_common import dev_elems, dev_i32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ns():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocab_draft_amd import nanospec
    return nanospec


class Side:
    def __init__(self, ns, cfg, W, prompt):
        self.ns, self.cfg, self.W = ns, cfg, W
        self.st = ns.NanoSpecState(cfg.V, cfg.w_max)
        ns.nanospec_stream_append(self.st, prompt, prompt.numel(), 0)
        self.ids = torch.empty(cfg.w_max, dtype=torch.int32, device="cuda")
        self.n = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.bm = torch.zeros((cfg.V + 31) // 32, dtype=torch.int32, device="cuda")
        ns.nanospec_active_vocab(self.st, self.ids, self.n, self.bm)
        self.packed = torch.zeros((cfg.w_max, cfg.d), dtype=W.dtype, device="cuda")
        self.ws = ns.alloc_workspace(cfg.w_max, cfg.M, cfg.k, cfg.d)
        self.out = {m: (torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda"),
                        torch.empty((cfg.M, cfg.k), device="cuda"),
                        torch.empty((cfg.M, cfg.w_max), device="cuda")) for m in (ns.NS_PACKED, ns.NS_INDEXED)}

    def step(self, tree, ver, h, copy_stream):
        ns, cfg = self.ns, self.cfg
        ns.nanospec_step_update(self.st, tree, tree.numel(), ver, ver.numel(), self.ids, self.n, self.bm)
        comp = torch.cuda.current_stream()
        copy_stream.wait_stream(comp)
        ns.nanospec_gather_rows(self.W, cfg.V, cfg.d, ns.NS_BF16, self.ids, self.n, cfg.w_max, self.packed,
                                stream=copy_stream)
        comp.wait_stream(copy_stream)
        for mode, rows in ((ns.NS_PACKED, self.packed), (ns.NS_INDEXED, self.W)):
            tids, tvals, logits = self.out[mode]
            ns.nanospec_draft_logits_topk(rows, mode, self.ids, self.n, cfg.w_max, cfg.V, cfg.d, ns.NS_BF16, h,
                                          cfg.M, cfg.k, logits, tids, tvals, self.ws)

    def snapshot(self):
        n = int(self.n.item())
        r = [self.ids[:n].clone(), self.n.clone(), self.bm.clone()]
        for mode in sorted(self.out):
            tids, tvals, logits = self.out[mode]
            r += [tids.clone(), tvals.clone(), logits[:, :n].clone()]
        return r


def test_graph_replays_match_eager(ns):
    cfg = WL.get_config("tiny", dtype="bf16")
    say("graph capture of a decode step", cfg)
    W = dev_elems(WL.make_weights(cfg), "bf16")
    script = WL.make_id_script(cfg, 8)
    prompt = dev_i32(script.prompt)
    g_side, e_side = Side(ns, cfg, W, prompt), Side(ns, cfg, W, prompt)
    tree_buf = torch.empty(cfg.n_tree, dtype=torch.int32, device="cuda")
    ver_buf = torch.empty(cfg.k_ver, dtype=torch.int32, device="cuda")
    h_buf = torch.empty((cfg.M, cfg.d), dtype=torch.bfloat16, device="cuda")
    copy_stream = torch.cuda.Stream()
    # step 0 runs eagerly on both sides (also warms up every kernel)
    for side in (g_side, e_side):
        tree_buf.copy_(dev_i32(script.tree[0]))
        ver_buf.copy_(dev_i32(script.ver[0]))
        h_buf.copy_(dev_elems(WL.make_hidden(cfg, 0), "bf16"))
        side.step(tree_buf, ver_buf, h_buf, copy_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_side.step(tree_buf, ver_buf, h_buf, copy_stream)
    torch.cuda.synchronize()
    for t in range(1, 8):
        # eager work between replays: new inputs into the captured buffers
        tree_buf.copy_(dev_i32(script.tree[t]))
        ver_buf.copy_(dev_i32(script.ver[t]))
        h = dev_elems(WL.make_hidden(cfg, t), "bf16")
        h_buf.copy_(h)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e_side.step(dev_i32(script.tree[t]), dev_i32(script.ver[t]), h, copy_stream)
        torch.cuda.synchronize()
        for a, b in zip(g_side.snapshot(), e_side.snapshot()):
            assert torch.equal(a, b), f"replay {t} differs from the eager run"
    assert ns.nanospec_state_status(g_side.st) == 0


def test_graph_replays_batched(ns):
    cfg = WL.get_config("tiny", dtype="bf16")
    B = 3
    say("graph capture of a batched step", cfg)
    W = dev_elems(WL.make_weights(cfg), "bf16")
    scripts = [WL.make_id_script(WL.get_config("tiny", dtype="bf16", seed=cfg.seed + b), 6) for b in range(B)]
    sides = []
    for _ in range(2):
        bt = ns.NanoSpecBatch(B, cfg.V, cfg.w_max)
        for b in range(B):
            ns.nanospec_stream_append(bt.member(b), dev_i32(scripts[b].prompt), len(scripts[b].prompt), 0)
        sides.append(dict(bt=bt, ids=torch.empty((B, cfg.w_max), dtype=torch.int32, device="cuda"),
                          n=torch.zeros(B, dtype=torch.int32, device="cuda"),
                          ws=ns.alloc_batch_workspace(B, cfg.w_max, cfg.M, cfg.k, cfg.d),
                          tids=torch.empty((B, cfg.M, cfg.k), dtype=torch.int32, device="cuda"),
                          tvals=torch.empty((B, cfg.M, cfg.k), device="cuda")))
    tree_buf = torch.empty((B, cfg.n_tree), dtype=torch.int32, device="cuda")
    ver_buf = torch.empty((B, cfg.k_ver), dtype=torch.int32, device="cuda")
    nd = torch.full((B,), cfg.n_tree, dtype=torch.int32, device="cuda")
    nv = torch.full((B,), cfg.k_ver, dtype=torch.int32, device="cuda")
    h_buf = torch.empty((B, cfg.M, cfg.d), dtype=torch.bfloat16, device="cuda")

    def step(sd):
        ns.nanospec_batch_step_update(sd["bt"], tree_buf, cfg.n_tree, nd, cfg.n_tree, ver_buf, cfg.k_ver, nv,
                                      cfg.k_ver, sd["ids"], sd["n"])
        ns.nanospec_batch_draft_logits_topk(W, sd["ids"], sd["n"], cfg.w_max, B, cfg.V, cfg.d, ns.NS_BF16, h_buf,
                                            cfg.M, cfg.k, None, sd["tids"], sd["tvals"], sd["ws"])

    def load(t):
        tree_buf.copy_(dev_i32(np.stack([s.tree[t] for s in scripts])))
        ver_buf.copy_(dev_i32(np.stack([s.ver[t] for s in scripts])))
        h_buf.copy_(dev_elems(np.stack([WL.make_hidden(cfg, 10 * t + b) for b in range(B)]), "bf16"))

    load(0)
    for sd in sides:
        step(sd)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(sides[0])
    for t in range(1, 6):
        load(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(sides[1])
        torch.cuda.synchronize()
        for key in ("n", "tids", "tvals"):
            assert torch.equal(sides[0][key], sides[1][key]), f"batched replay {t}: {key} differs"
        for b in range(B):                       # ids past n[b] are never written
            nb = int(sides[1]["n"][b].item())
            assert torch.equal(sides[0]["ids"][b, :nb], sides[1]["ids"][b, :nb]), f"batched replay {t}: ids"


def test_graph_replays_slot_buffer(ns):
    """State update, the slot-stable buffer's update on a second stream (fork
    and join), and the head over the slot map, captured once and replayed
    against an eager twin."""
    cfg = WL.get_config("tiny", dtype="bf16")
    say("graph capture of a slot-buffer step", cfg)
    W = dev_elems(WL.make_weights(cfg), "bf16")
    script = WL.make_id_script(cfg, 8)
    prompt = dev_i32(script.prompt)
    copy_stream = torch.cuda.Stream()

    def side():
        st = ns.NanoSpecState(cfg.V, cfg.w_max)
        ns.nanospec_stream_append(st, prompt, prompt.numel(), 0)
        d = dict(st=st, pk=ns.NanoSpecPacked(cfg.V, cfg.w_max),
                 rows=torch.zeros((cfg.w_max, cfg.d), dtype=torch.bfloat16, device="cuda"),
                 ids=torch.empty(cfg.w_max, dtype=torch.int32, device="cuda"),
                 n=torch.zeros(1, dtype=torch.int32, device="cuda"),
                 ws=ns.alloc_workspace(cfg.w_max, cfg.M, cfg.k, cfg.d),
                 tids=torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda"),
                 tvals=torch.empty((cfg.M, cfg.k), device="cuda"))
        ns.nanospec_active_vocab(st, d["ids"], d["n"])
        ns.nanospec_packed_update(d["pk"], st, W, cfg.d, ns.NS_BF16, d["rows"])
        return d

    def step(d, tree, ver, h):
        ns.nanospec_step_update(d["st"], tree, tree.numel(), ver, ver.numel(), d["ids"], d["n"])
        comp = torch.cuda.current_stream()
        copy_stream.wait_stream(comp)
        ns.nanospec_packed_update(d["pk"], d["st"], W, cfg.d, ns.NS_BF16, d["rows"], stream=copy_stream)
        comp.wait_stream(copy_stream)
        ns.nanospec_draft_logits_topk(d["rows"], ns.NS_PACKED, d["pk"].slot_ids, d["pk"].n_slots, cfg.w_max, cfg.V,
                                      cfg.d, ns.NS_BF16, h, cfg.M, cfg.k, None, d["tids"], d["tvals"], d["ws"])

    g, e = side(), side()
    tree_buf = torch.empty(cfg.n_tree, dtype=torch.int32, device="cuda")
    ver_buf = torch.empty(cfg.k_ver, dtype=torch.int32, device="cuda")
    h_buf = torch.empty((cfg.M, cfg.d), dtype=torch.bfloat16, device="cuda")

    def load(t):
        tree_buf.copy_(dev_i32(script.tree[t]))
        ver_buf.copy_(dev_i32(script.ver[t]))
        h_buf.copy_(dev_elems(WL.make_hidden(cfg, t), "bf16"))

    load(0)
    for d in (g, e):
        step(d, tree_buf, ver_buf, h_buf)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g, tree_buf, ver_buf, h_buf)
    torch.cuda.synchronize()
    for t in range(1, 8):
        load(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(e, tree_buf, ver_buf, h_buf)
        torch.cuda.synchronize()
        for key in ("tids", "tvals"):
            assert torch.equal(g[key], e[key]), f"slot replay {t}: {key}"
        assert torch.equal(g["pk"].slot_ids, e["pk"].slot_ids), f"slot replay {t}: slot map"
        assert torch.equal(g["pk"].n_slots, e["pk"].n_slots), f"slot replay {t}: n_slots"
        occ = (e["pk"].slot_ids >= 0).nonzero().flatten()
        assert torch.equal(g["rows"][occ].view(torch.int16), e["rows"][occ].view(torch.int16)), f"slot replay {t}"


def test_graph_replays_tree(ns):
    """A state update and a 3-depth draft tree (log-prob heads, frontier
    selections, final selection) captured once and replayed against an
    eager twin."""
    cfg = WL.get_config("tiny", dtype="bf16")
    K, F, N, D = 4, 4, 10, 3
    say("graph capture of a tree-drafting step", cfg)
    W = dev_elems(WL.make_weights(cfg), "bf16")
    script = WL.make_id_script(cfg, 6)
    prompt = dev_i32(script.prompt)
    P = K + (D - 1) * F * K

    def side():
        st = ns.NanoSpecState(cfg.V, cfg.w_max)
        ns.nanospec_stream_append(st, prompt, prompt.numel(), 0)
        return dict(st=st, ids=torch.empty(cfg.w_max, dtype=torch.int32, device="cuda"),
                    n=torch.zeros(1, dtype=torch.int32, device="cuda"),
                    ws=ns.alloc_workspace(cfg.w_max, F, K, cfg.d),
                    pid=torch.empty(P, dtype=torch.int32, device="cuda"), pv=torch.empty(P, device="cuda"),
                    fi=torch.empty((D, F), dtype=torch.int32, device="cuda"), fv=torch.empty((D, F), device="cuda"),
                    fd=torch.empty((D, F), dtype=torch.int32, device="cuda"),
                    out=[torch.empty(N, dtype=torch.int32, device="cuda"), torch.empty(N, device="cuda"),
                         torch.empty(N, dtype=torch.int32, device="cuda")])

    hs = [torch.empty((1 if t == 0 else F, cfg.d), dtype=torch.bfloat16, device="cuda") for t in range(D)]
    tree_buf = torch.empty(cfg.n_tree, dtype=torch.int32, device="cuda")
    ver_buf = torch.empty(cfg.k_ver, dtype=torch.int32, device="cuda")

    def step(d):
        ns.nanospec_step_update(d["st"], tree_buf, tree_buf.numel(), ver_buf, ver_buf.numel(), d["ids"], d["n"])
        base = 0
        for t in range(D):
            M = 1 if t == 0 else F
            ti, tv = d["pid"][base:base + M * K], d["pv"][base:base + M * K]
            ns.nanospec_draft_logprob_topk(W, ns.NS_INDEXED, d["ids"], d["n"], cfg.w_max, cfg.V, cfg.d, ns.NS_BF16,
                                           hs[t], M, K, None if t == 0 else d["fv"][t - 1], None, None, ti, tv,
                                           d["ws"])
            ns.nanospec_tree_select(tv, ti, M * K, 1, F, d["fi"][t], d["fv"][t], d["fd"][t])
            base += M * K
        ns.nanospec_tree_select(d["pv"], d["pid"], P, 1, N, *d["out"])

    def load(t):
        tree_buf.copy_(dev_i32(script.tree[t]))
        ver_buf.copy_(dev_i32(script.ver[t]))
        for i, h in enumerate(hs):
            h.copy_(dev_elems(WL.make_hidden(cfg, 10 * t + i, M=h.shape[0]), "bf16"))

    g, e = side(), side()
    load(0)
    for d in (g, e):
        step(d)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g)
    torch.cuda.synchronize()
    for t in range(1, 6):
        load(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(e)
        torch.cuda.synchronize()
        for key in ("pid", "pv", "fi", "fv", "fd"):
            assert torch.equal(g[key], e[key]), f"tree replay {t}: {key}"
        for a, b in zip(g["out"], e["out"]):
            assert torch.equal(a, b), f"tree replay {t}: final"
