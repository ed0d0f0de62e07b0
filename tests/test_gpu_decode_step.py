"""nanospec_decode_step, the decode step in one call (NanoSpec Sec. 3.2,
decoding phase and sliding-window rebuild, then Sec. 3.1 Eq. 1 on
W_head[I_{t+1}, :] with T_k).

Two states run the same id script: one through nanospec_decode_step, the
other through nanospec_step_update and then nanospec_draft_logits_topk
(INDEXED).  At every step the active set, |I| and the top-k ids and values
must be identical bit for bit; on sampled steps both are also checked against
the oracle.  The step takes the two-launch form (state update beside the
projection) once the state holds its active set from a previous decode step;
its first launch then writes |I_t| into the first word of the workspace, which
the tests set to a sentinel before each call to see which form ran.  The
first step, and the step after an append or after a separate rebuild, take
the three-launch form.  Shapes: the Llama- and Qwen-shaped heads (one and four
hidden tiles), two hidden tiles, fp16, a tiny fp32 head (always three
launches), both stream-source modes, a HIP graph of fused steps, the step
split into nanospec_decode_step_project and _select, the state's bitmap after
the steps, and the edge cases of the form: tuples past 256 entries, empty
tuples, W_max not a multiple of 4, and ids outside [0, V).  The batched
decode step (nanospec_batch_decode_step) against the separate batched calls:
Llama-shaped B = 1, 4, 32, M = 12, 40, and 20 in fp16, Qwen-shaped B = 2 and 3,
with per-sequence tuple counts; and batched steps between single-sequence
calls on members (an append, a single decode step)."""
import numpy as np
import pytest
import torch

import oracle.nanospec_oracle as O
from dynamic_vocab_draft_amd import workloads as WL
from tests.gpu_common import check_topk, dcode_of, dev_elems, dev_i32, say

pytestmark = pytest.mark.gpu

SENTINEL = -12345


@pytest.fixture(scope="module")
def ns():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocab_draft_amd import nanospec
    return nanospec


class Pair:
    """The same sequence driven through the one-call step (a) and the
    separate calls (b)."""

    def __init__(self, ns, cfg, W_dev, dcode, M, k, mode=None):
        self.ns, self.cfg, self.W, self.dcode, self.M, self.k = ns, cfg, W_dev, dcode, M, k
        self.st_a = ns.NanoSpecState(cfg.V, cfg.w_max)
        self.st_b = ns.NanoSpecState(cfg.V, cfg.w_max)
        if mode is not None:
            ns.nanospec_state_set_mode(self.st_a, mode)
            ns.nanospec_state_set_mode(self.st_b, mode)
        mk = lambda: (torch.empty(cfg.w_max, dtype=torch.int32, device="cuda"),
                      torch.zeros(1, dtype=torch.int32, device="cuda"),
                      torch.empty((M, k), dtype=torch.int32, device="cuda"),
                      torch.empty((M, k), dtype=torch.float32, device="cuda"))
        self.a, self.b = mk(), mk()
        self.ws_a = ns.alloc_decode_workspace(cfg.w_max, 2 * 256, M, k, cfg.d)
        self.ws_b = ns.alloc_workspace(cfg.w_max, M, k, cfg.d)
        self.ws_b_decode = ns.alloc_decode_workspace(cfg.w_max, 2 * 256, M, k, cfg.d)

    def append(self, ids):
        d = dev_i32(ids)
        for st in (self.st_a, self.st_b):
            self.ns.nanospec_stream_append(st, d, len(ids), 0)

    def rebuild(self):
        for st, (ids, n, _, _) in ((self.st_a, self.a), (self.st_b, self.b)):
            self.ns.nanospec_active_vocab(st, ids, n)

    def step(self, tree, ver, h_dev):
        ns, cfg = self.ns, self.cfg
        td, vd = dev_i32(tree), dev_i32(ver)
        ids, n, ti, tv = self.a
        self.ws_a.view(torch.int32)[0] = SENTINEL
        ns.nanospec_decode_step(self.st_a, td, len(tree), vd, len(ver), ids, n, self.W, cfg.V, cfg.d, self.dcode,
                                h_dev, self.M, self.k, ti, tv, self.ws_a)
        ids, n, ti, tv = self.b
        ns.nanospec_step_update(self.st_b, td, len(tree), vd, len(ver), ids, n)
        ns.nanospec_draft_logits_topk(self.W, ns.NS_INDEXED, ids, n, cfg.w_max, cfg.V, cfg.d, self.dcode, h_dev,
                                      self.M, self.k, None, ti, tv, self.ws_b)

    def fused_ran(self):
        return int(self.ws_a.view(torch.int32)[0].item()) != SENTINEL

    def compare(self, what):
        torch.cuda.synchronize()
        na, nb = int(self.a[1].item()), int(self.b[1].item())
        assert na == nb, f"{what}: |I| {na} != {nb}"
        assert torch.equal(self.a[0][:na], self.b[0][:nb]), f"{what}: active sets differ"
        assert torch.equal(self.a[2], self.b[2]), f"{what}: top-k ids differ"
        assert torch.equal(self.a[3], self.b[3]), f"{what}: top-k values differ"
        return na


def _run(ns, name, steps, check_every, M=None, k=None, dtype=None, mode=None, expect_fused=True):
    cfg = WL.get_config(name)
    M = M or cfg.M
    k = k or cfg.k
    dtype = dtype or cfg.dtype
    say(f"decode step {name} M={M} k={k} {dtype} mode={mode}: generating inputs")
    W = WL.make_weights(cfg)
    if dtype != cfg.dtype:                                 # fp16 copies of the bf16 weights
        W = WL.f32_to_fp16_bits(WL.bf16_bits_to_f32(W))
    W_dev = dev_elems(W, dtype)
    dcode = dcode_of(ns, dtype)
    script = WL.make_id_script(cfg, steps)
    seq = O.Sequence_(cfg.w_max, mode or "full")
    code = {None: None, "ctx_only": ns.NS_STREAM_CTX_ONLY, "ext_only": ns.NS_STREAM_EXT_ONLY}[mode]
    pair = Pair(ns, cfg, W_dev, dcode, M, k, code)
    seq.append_prompt(script.prompt)
    pair.append(script.prompt)
    pair.rebuild()
    fused_steps = 0
    for t, tree, ver in WL.iter_steps(cfg, script):
        h = WL.make_hidden(cfg, t, M=M)
        if dtype != cfg.dtype:
            h = WL.f32_to_fp16_bits(WL.bf16_bits_to_f32(h))
        h_dev = dev_elems(h, dtype)
        seq.step(tree, ver)
        pair.step(tree, ver, h_dev)
        what = f"{name} step {t}"
        nn = pair.compare(what)
        fused = pair.fused_ran()
        fused_steps += fused
        if t == 0:
            assert not fused, f"{what}: the first step has no kept active set"
        elif expect_fused:
            assert fused, f"{what}: expected the two-launch form"
        if t % check_every and t != steps - 1:
            continue
        I = seq.active()
        assert nn == len(I) and np.array_equal(pair.a[0][:nn].cpu().numpy(), I), f"{what}: active set vs oracle"
        ref, o_ids, o_vals = O.draft_head(h, W, I, k, dtype)
        check_topk(pair.a[2].cpu().numpy(), pair.a[3].cpu().numpy(), ref, I, o_ids, o_vals, k, what)
        say(f"{what}: |I| = {nn}, {'two' if fused else 'three'} launches, ok")
    assert ns.nanospec_state_status(pair.st_a) == 0
    # The state's bitmap after the last step holds I exactly: the slot-stable
    # buffer, planned from it, maps exactly I.
    pk = ns.NanoSpecPacked(cfg.V, cfg.w_max)
    ns.nanospec_packed_update(pk, pair.st_a, W_dev, cfg.d, dcode, torch.zeros((cfg.w_max, cfg.d),
                              dtype=torch.bfloat16 if dtype != "fp32" else torch.float32, device="cuda"))
    torch.cuda.synchronize()
    slots = pk.slot_ids.cpu().numpy()
    assert np.array_equal(np.sort(slots[slots >= 0]), seq.active()), f"{name}: the state's bitmap is not I"
    return pair, fused_steps


def test_decode_step_llama3_8b(ns):
    _run(ns, "llama3_8b", steps=48, check_every=8)


def test_decode_step_qwen25_7b(ns):
    _run(ns, "qwen25_7b", steps=24, check_every=8)


def test_decode_step_two_hidden_tiles_fp16(ns):
    _run(ns, "llama3_8b", steps=20, check_every=10, M=20, k=16, dtype="fp16")


def test_decode_step_tiny_fp32_three_launches(ns):
    _run(ns, "tiny", steps=8, check_every=2, expect_fused=False)


@pytest.mark.parametrize("mode", ["ctx_only", "ext_only"])
def test_decode_step_stream_sources(ns, mode):
    _run(ns, "llama3_8b", steps=12, check_every=4, M=4, k=8, mode=mode)


def test_decode_step_after_append_and_rebuild(ns):
    """An append, or a separate rebuild, drops the kept active set: the next
    decode step takes three launches, and the one after it two again."""
    cfg = WL.get_config("llama3_8b")
    W = WL.make_weights(cfg)
    W_dev = dev_elems(W, cfg.dtype)
    script = WL.make_id_script(cfg, 12)
    pair = Pair(ns, cfg, W_dev, ns.NS_BF16, 8, 8)
    seq = O.Sequence_(cfg.w_max)
    seq.append_prompt(script.prompt)
    pair.append(script.prompt)
    pair.rebuild()
    rng = np.random.default_rng(3)
    for t, tree, ver in WL.iter_steps(cfg, script):
        if t == 4:                                   # an append between steps
            extra = rng.integers(0, cfg.V, size=100).astype(np.int32)
            seq.append_prompt(extra)
            pair.append(extra)
        if t == 8:                                   # a separate rebuild
            pair.rebuild()
        h_dev = dev_elems(WL.make_hidden(cfg, t), cfg.dtype)
        seq.step(tree, ver)
        pair.step(tree, ver, h_dev)
        pair.compare(f"step {t}")
        assert pair.fused_ran() == (t not in (0, 4, 8)), f"step {t}: launch form"
        I = seq.active()
        nn = int(pair.a[1].item())
        assert np.array_equal(pair.a[0][:nn].cpu().numpy(), I), f"step {t}: active set vs oracle"


def test_decode_step_graph_replay(ns):
    """Fused steps captured in a HIP graph and replayed give the results of
    the same steps run eagerly on a twin state."""
    cfg = WL.get_config("llama3_8b")
    W = WL.make_weights(cfg)
    W_dev = dev_elems(W, cfg.dtype)
    script = WL.make_id_script(cfg, 16)
    steps = list(WL.iter_steps(cfg, script))
    hs = [dev_elems(WL.make_hidden(cfg, t), cfg.dtype) for t, _, _ in steps]
    trees = [dev_i32(tr) for _, tr, _ in steps]
    vers = [dev_i32(v) for _, _, v in steps]

    def fresh():
        st = ns.NanoSpecState(cfg.V, cfg.w_max)
        ids = torch.empty(cfg.w_max, dtype=torch.int32, device="cuda")
        n = torch.zeros(1, dtype=torch.int32, device="cuda")
        ti = torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda")
        tv = torch.empty((cfg.M, cfg.k), dtype=torch.float32, device="cuda")
        ws = ns.alloc_decode_workspace(cfg.w_max, 512, cfg.M, cfg.k, cfg.d)
        ns.nanospec_stream_append(st, dev_i32(script.prompt), len(script.prompt), 0)
        ns.nanospec_active_vocab(st, ids, n)
        return st, ids, n, ti, tv, ws

    def run(obj, lo, hi):
        st, ids, n, ti, tv, ws = obj
        for i in range(lo, hi):
            ns.nanospec_decode_step(st, trees[i], trees[i].numel(), vers[i], vers[i].numel(), ids, n, W_dev, cfg.V,
                                    cfg.d, ns.NS_BF16, hs[i], cfg.M, cfg.k, ti, tv, ws)

    eager, graphed = fresh(), fresh()
    run(eager, 0, 2)
    run(graphed, 0, 2)                               # both now keep their active sets
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(graphed, 2, 8)
    for rep in range(3):                             # each replay repeats steps 2..7 on the advanced state
        run(eager, 2, 8)
        g.replay()
        torch.cuda.synchronize()
        n = int(eager[2].item())
        assert int(graphed[2].item()) == n, f"replay {rep}: |I| differs"
        for a, b, what in ((eager[1][:n], graphed[1][:n], "active ids"), (eager[3], graphed[3], "top-k ids"),
                           (eager[4], graphed[4], "top-k values")):
            assert torch.equal(a, b), f"replay {rep}: {what} differ"


def test_decode_step_split_calls(ns):
    """nanospec_decode_step_project then _select on one state, the one-call
    step on a twin: identical outputs at every step, in both forms (the
    first step takes three launches).  select is refused without a pending
    project, with other buffers than project's, and after another call on
    the state in between."""
    cfg = WL.get_config("llama3_8b")
    W = WL.make_weights(cfg)
    W_dev = dev_elems(W, cfg.dtype)
    script = WL.make_id_script(cfg, 10)
    M, k = 8, 8
    pair = Pair(ns, cfg, W_dev, ns.NS_BF16, M, k)
    pair.append(script.prompt)
    pair.rebuild()
    st, (ids, n, ti, tv), ws = pair.st_a, pair.a, pair.ws_a
    sel = lambda i=ids, nn=n: ns.nanospec_decode_step_select(st, i, nn, cfg.V, cfg.d, ns.NS_BF16, M, k, ti, tv, ws)
    with pytest.raises(ns.NanoSpecError):                # nothing pending
        sel()
    for t, tree, ver in WL.iter_steps(cfg, script):
        h_dev = dev_elems(WL.make_hidden(cfg, t), cfg.dtype)
        td, vd = dev_i32(tree), dev_i32(ver)
        ws.view(torch.int32)[0] = SENTINEL
        ns.nanospec_decode_step_project(st, td, len(tree), vd, len(ver), ids, n, W_dev, cfg.V, cfg.d, ns.NS_BF16,
                                        h_dev, M, k, ws)
        if t == 3:                                       # select with another active-set buffer
            with pytest.raises(ns.NanoSpecError):
                sel(i=pair.b[0])
        sel()
        b_ids, b_n, b_ti, b_tv = pair.b
        ns.nanospec_decode_step(pair.st_b, td, len(tree), vd, len(ver), b_ids, b_n, W_dev, cfg.V, cfg.d,
                                ns.NS_BF16, h_dev, M, k, b_ti, b_tv, pair.ws_b_decode)
        torch.cuda.synchronize()
        assert pair.fused_ran() == (t > 0), f"step {t}: launch form"
        na = int(n.item())
        assert na == int(b_n.item()) and torch.equal(ids[:na], b_ids[:na]), f"step {t}: active sets differ"
        assert torch.equal(ti, b_ti) and torch.equal(tv, b_tv), f"step {t}: top-k differs"
    # Another call on the state between project and select drops the pending step.
    tree, ver = script.tree[0], script.ver[0]
    ns.nanospec_decode_step_project(st, dev_i32(tree), len(tree), dev_i32(ver), len(ver), ids, n, W_dev, cfg.V,
                                    cfg.d, ns.NS_BF16, dev_elems(WL.make_hidden(cfg, 0), cfg.dtype), M, k, ws)
    ns.nanospec_stream_append(st, dev_i32(tree), len(tree), 0)
    with pytest.raises(ns.NanoSpecError):
        sel()
    torch.cuda.synchronize()


def _edge_run(ns, cfg, steps, expect):
    """Drives a Pair through (tree, ver) steps and checks, at every step,
    identical outputs in both forms, the launch form against `expect`, the
    active set against the oracle, and the state's status bits."""
    W = WL.make_weights(cfg)
    W_dev = dev_elems(W, cfg.dtype)
    script = WL.make_id_script(cfg, 4)
    pair = Pair(ns, cfg, W_dev, ns.NS_BF16, 8, 8)
    seq = O.Sequence_(cfg.w_max)
    seq.append_prompt(script.prompt)
    pair.append(script.prompt)
    pair.rebuild()
    for t, (tree, ver) in enumerate(steps):
        h_dev = dev_elems(WL.make_hidden(cfg, t), cfg.dtype)
        seq.step(tree, ver)
        pair.step(tree, ver, h_dev)
        nn = pair.compare(f"step {t}")
        assert pair.fused_ran() == expect[t], f"step {t}: launch form"
        I = seq.active()
        assert nn == len(I) and np.array_equal(pair.a[0][:nn].cpu().numpy(), I), f"step {t}: active set vs oracle"
    return pair


def test_decode_step_forms_across_tuple_sizes(ns):
    """A step with more than 256 tuple entries has no two-launch form: it
    drops the kept I_t, so the step after it takes three launches and the one
    after that two again.  A step with no tuple entries keeps I_t as it is."""
    cfg = WL.get_config("llama3_8b")
    rng = np.random.default_rng(11)
    small = lambda: (rng.integers(0, cfg.V, 60).astype(np.int32), rng.integers(0, cfg.V, 8).astype(np.int32))
    big = (rng.integers(0, cfg.V, 290).astype(np.int32), rng.integers(0, cfg.V, 8).astype(np.int32))
    empty = (np.zeros(0, np.int32), np.zeros(0, np.int32))
    steps = [small(), small(), big, small(), small(), empty, small()]
    _edge_run(ns, cfg, steps, [False, True, False, False, True, True, True])


def test_decode_step_w_max_not_multiple_of_4(ns):
    """W_max = 3070: never the two-launch form, same results as the separate
    calls."""
    cfg = WL.get_config("llama3_8b", w_max=3070)
    rng = np.random.default_rng(12)
    steps = [(rng.integers(0, cfg.V, 60).astype(np.int32), rng.integers(0, cfg.V, 8).astype(np.int32))
             for _ in range(4)]
    _edge_run(ns, cfg, steps, [False] * 4)


def test_decode_step_bad_ids(ns):
    """Ids outside [0, V) in the tuples are skipped by both forms and set the
    sticky status bit of both states."""
    cfg = WL.get_config("llama3_8b")
    rng = np.random.default_rng(13)
    steps = []
    for t in range(4):
        tree = rng.integers(0, cfg.V, 60).astype(np.int32)
        ver = rng.integers(0, cfg.V, 8).astype(np.int32)
        if t == 2:
            tree[[3, 17]] = [cfg.V, -5]
            ver[1] = cfg.V + 100
        steps.append((tree, ver))
    # The oracle skips the same ids: drop them from its copy of the script.
    W = WL.make_weights(cfg)
    W_dev = dev_elems(W, cfg.dtype)
    script = WL.make_id_script(cfg, 4)
    pair = Pair(ns, cfg, W_dev, ns.NS_BF16, 8, 8)
    seq = O.Sequence_(cfg.w_max)
    seq.append_prompt(script.prompt)
    pair.append(script.prompt)
    pair.rebuild()
    for t, (tree, ver) in enumerate(steps):
        h_dev = dev_elems(WL.make_hidden(cfg, t), cfg.dtype)
        ok = lambda a: a[(a >= 0) & (a < cfg.V)]
        seq.step(ok(tree), ok(ver))
        pair.step(tree, ver, h_dev)
        nn = pair.compare(f"step {t}")
        assert pair.fused_ran() == (t > 0), f"step {t}: launch form"
        I = seq.active()
        assert nn == len(I) and np.array_equal(pair.a[0][:nn].cpu().numpy(), I), f"step {t}: active set vs oracle"
    assert ns.nanospec_state_status(pair.st_a) == ns.nanospec_state_status(pair.st_b) != 0


@pytest.mark.parametrize("name,B,M,dtype,two", [
    ("llama3_8b", 1, None, None, True),       # the single sequence's resident grid
    ("llama3_8b", 4, None, None, True),
    ("llama3_8b", 32, None, None, False),     # the separate batched head's taller tiles
    ("llama3_8b", 3, 12, None, True),         # one hidden tile of 9-16 rows
    ("llama3_8b", 5, 20, "fp16", True),       # two hidden tiles, fp16
    ("llama3_8b", 2, 40, None, True),         # three hidden tiles
    ("qwen25_7b", 2, None, None, True),       # four hidden tiles
    ("qwen25_7b", 3, None, None, False),      # the M-split projection
])
def test_batch_decode_step(ns, name, B, M, dtype, two):
    """B sequences of one workload (`two`: whether the steps after the first
    take two launches; the forms that keep three are the shapes whose
    separate batched head takes taller tiles or the M-split projection):
    nanospec_batch_decode_step on one batch,
    nanospec_batch_step_update and nanospec_batch_draft_logits_topk on a twin,
    identical bit for bit at every step; per-sequence tuple counts differ (so
    the tuple columns are padded), the first step takes three launches and
    the others two, and the first, middle and last sequences' active sets and
    top-k match their own oracle sequences on sampled steps."""
    steps = 10
    cfg = WL.get_config(name)
    M, dtype = M or cfg.M, dtype or cfg.dtype
    V, w_max, d, k = cfg.V, cfg.w_max, cfg.d, cfg.k
    say(f"batch decode step {name} B={B} M={M} {dtype}: generating inputs")
    W = WL.make_weights(cfg)
    if dtype != cfg.dtype:                                 # fp16 copies of the bf16 weights
        W = WL.f32_to_fp16_bits(WL.bf16_bits_to_f32(W))
    W_dev = dev_elems(W, dtype)
    dcode = dcode_of(ns, dtype)
    cfgs = [WL.get_config(name, seed=cfg.seed + 100 * b) for b in range(B)]
    scripts = [WL.make_id_script(c, steps) for c in cfgs]
    nd_max, nv_max = cfg.n_tree, cfg.k_ver
    A, Bt = ns.NanoSpecBatch(B, V, w_max), ns.NanoSpecBatch(B, V, w_max)
    seqs = []
    for b in range(B):
        seq = O.Sequence_(w_max)
        seq.append_prompt(scripts[b].prompt)
        seqs.append(seq)
        for bt in (A, Bt):
            ns.nanospec_stream_append(bt.member(b), dev_i32(scripts[b].prompt), len(scripts[b].prompt), 0)
    mk = lambda: (torch.full((B, w_max), -7, dtype=torch.int32, device="cuda"),
                  torch.zeros(B, dtype=torch.int32, device="cuda"),
                  torch.empty((B, M, k), dtype=torch.int32, device="cuda"),
                  torch.empty((B, M, k), dtype=torch.float32, device="cuda"))
    oa, ob = mk(), mk()
    ws_a = ns.alloc_batch_decode_workspace(B, w_max, nd_max + nv_max, M, k, d)
    ws_b = ns.alloc_batch_workspace(B, w_max, M, k, d)
    rng = np.random.default_rng(21)
    for t in range(steps):
        trees, vers = [], []
        for b in range(B):
            tree, ver = scripts[b].tree[t], scripts[b].ver[t]
            keep_t = len(tree) - int(rng.integers(0, 20)) if b % 2 else len(tree)
            keep_v = len(ver) - int(rng.integers(0, 4)) if b == 3 else len(ver)
            trees.append(tree[:keep_t])
            vers.append(ver[:keep_v])
        dr = np.full((B, nd_max), -1, np.int32)
        vr = np.full((B, nv_max), -1, np.int32)
        for b in range(B):
            dr[b, :len(trees[b])] = trees[b]
            vr[b, :len(vers[b])] = vers[b]
        d_dev, v_dev = dev_i32(dr.reshape(-1)), dev_i32(vr.reshape(-1))
        nd_dev = dev_i32(np.array([len(x) for x in trees], np.int32))
        nv_dev = dev_i32(np.array([len(x) for x in vers], np.int32))
        hs = [WL.make_hidden(cfgs[b], t, M=M) for b in range(B)]
        if dtype != cfg.dtype:
            hs = [WL.f32_to_fp16_bits(WL.bf16_bits_to_f32(x)) for x in hs]
        h_dev = dev_elems(np.stack(hs), dtype)
        ws_a.view(torch.int32)[0] = SENTINEL
        ns.nanospec_batch_decode_step(A, d_dev, nd_max, nd_dev, nd_max, v_dev, nv_max, nv_dev, nv_max, oa[0], oa[1],
                                      W_dev, V, d, dcode, h_dev, M, k, oa[2], oa[3], ws_a)
        ns.nanospec_batch_step_update(Bt, d_dev, nd_max, nd_dev, nd_max, v_dev, nv_max, nv_dev, nv_max, ob[0], ob[1])
        ns.nanospec_batch_draft_logits_topk(W_dev, ob[0], ob[1], w_max, B, V, d, dcode, h_dev, M, k, None,
                                            ob[2], ob[3], ws_b)
        torch.cuda.synchronize()
        fused = int(ws_a.view(torch.int32)[0].item()) != SENTINEL
        assert fused == (t > 0 and two), f"step {t}: launch form"
        assert torch.equal(oa[1], ob[1]), f"step {t}: counts differ"
        for b in range(B):
            nb = int(oa[1][b].item())
            assert torch.equal(oa[0][b, :nb], ob[0][b, :nb]), f"step {t} seq {b}: active sets differ"
        assert torch.equal(oa[2], ob[2]) and torch.equal(oa[3], ob[3]), f"step {t}: top-k differs"
        for b in range(B):
            seqs[b].step(trees[b], vers[b])
        if t % 3 and t != steps - 1:
            continue
        for b in sorted({0, B // 2, B - 1}):
            I = seqs[b].active()
            nb = int(oa[1][b].item())
            assert nb == len(I) and np.array_equal(oa[0][b, :nb].cpu().numpy(), I), f"step {t} seq {b}: vs oracle"
            ref, o_ids, o_vals = O.draft_head(hs[b], W, I, k, dtype)
            check_topk(oa[2][b].cpu().numpy(), oa[3][b].cpu().numpy(), ref, I, o_ids, o_vals, k, f"step {t} seq {b}")
        say(f"batch decode step B={B} t={t}: {'two' if fused else 'three'} launches, ok")
    for b in range(B):
        assert ns.nanospec_state_status(A.member(b)) == 0


def test_batch_decode_step_with_member_calls(ns):
    """Three Llama-shaped sequences through nanospec_batch_decode_step while
    single-sequence calls act on members between the batched steps: an append
    to one member (the next batched step takes three launches, the one after
    two), then a single decode step on member 0 alone (the next batched step
    still takes two).  The twin batch takes the separate calls throughout;
    results agree bit for bit, and every member's active set matches its
    oracle sequence at the end."""
    B, steps = 3, 7
    cfg = WL.get_config("llama3_8b")
    V, w_max, d, M, k = cfg.V, cfg.w_max, cfg.d, cfg.M, cfg.k
    W = WL.make_weights(cfg)
    W_dev = dev_elems(W, cfg.dtype)
    cfgs = [WL.get_config("llama3_8b", seed=cfg.seed + 300 * b) for b in range(B)]
    scripts = [WL.make_id_script(c, steps) for c in cfgs]
    nd, nv = cfg.n_tree, cfg.k_ver
    A, Bt = ns.NanoSpecBatch(B, V, w_max), ns.NanoSpecBatch(B, V, w_max)
    seqs = [O.Sequence_(w_max) for _ in range(B)]
    for b in range(B):
        seqs[b].append_prompt(scripts[b].prompt)
        for bt in (A, Bt):
            ns.nanospec_stream_append(bt.member(b), dev_i32(scripts[b].prompt), len(scripts[b].prompt), 0)
    mk = lambda: (torch.empty((B, w_max), dtype=torch.int32, device="cuda"),
                  torch.zeros(B, dtype=torch.int32, device="cuda"),
                  torch.empty((B, M, k), dtype=torch.int32, device="cuda"),
                  torch.empty((B, M, k), dtype=torch.float32, device="cuda"))
    oa, ob = mk(), mk()
    ws_a = ns.alloc_batch_decode_workspace(B, w_max, nd + nv, M, k, d)
    ws_b = ns.alloc_batch_workspace(B, w_max, M, k, d)
    ws_1 = ns.alloc_decode_workspace(w_max, nd + nv, M, k, d)
    ws_1b = ns.alloc_workspace(w_max, M, k, d)
    counts = lambda x: dev_i32(np.full(B, x, np.int32))
    expect = {0: False, 1: True, 2: False, 3: True, 5: True, 6: True}   # batched steps: two launches?
    for t in range(steps):
        h = [WL.make_hidden(cfgs[b], t) for b in range(B)]
        if t == 2:                                         # an append to member 1 drops its I_t
            extra = np.array([5, 77, 1234, 9], np.int32)
            seqs[1].append_prompt(extra)
            for bt in (A, Bt):
                ns.nanospec_stream_append(bt.member(1), dev_i32(extra), len(extra), 0)
        if t == 4:                                         # member 0 alone, single-sequence calls
            tr, vr = scripts[0].tree[t], scripts[0].ver[t]
            td, vd, hd = dev_i32(tr), dev_i32(vr), dev_elems(h[0], cfg.dtype)
            ns.nanospec_decode_step(A.member(0), td, nd, vd, nv, oa[0][0], oa[1][0:1], W_dev, V, d, ns.NS_BF16, hd,
                                    M, k, oa[2][0], oa[3][0], ws_1)
            ns.nanospec_step_update(Bt.member(0), td, nd, vd, nv, ob[0][0], ob[1][0:1])
            ns.nanospec_draft_logits_topk(W_dev, ns.NS_INDEXED, ob[0][0], ob[1][0:1], w_max, V, d, ns.NS_BF16, hd,
                                          M, k, None, ob[2][0], ob[3][0], ws_1b)
            seqs[0].step(tr, vr)
            torch.cuda.synchronize()
            n0 = int(oa[1][0].item())
            assert n0 == int(ob[1][0].item()) and torch.equal(oa[0][0, :n0], ob[0][0, :n0])
            assert torch.equal(oa[2][0], ob[2][0]) and torch.equal(oa[3][0], ob[3][0]), "member 0 single step"
            continue
        dr = dev_i32(np.stack([scripts[b].tree[t] for b in range(B)]).reshape(-1))
        vr = dev_i32(np.stack([scripts[b].ver[t] for b in range(B)]).reshape(-1))
        h_dev = dev_elems(np.stack(h), cfg.dtype)
        ws_a.view(torch.int32)[0] = SENTINEL
        ns.nanospec_batch_decode_step(A, dr, nd, counts(nd), nd, vr, nv, counts(nv), nv, oa[0], oa[1], W_dev, V, d,
                                      ns.NS_BF16, h_dev, M, k, oa[2], oa[3], ws_a)
        ns.nanospec_batch_step_update(Bt, dr, nd, counts(nd), nd, vr, nv, counts(nv), nv, ob[0], ob[1])
        ns.nanospec_batch_draft_logits_topk(W_dev, ob[0], ob[1], w_max, B, V, d, ns.NS_BF16, h_dev, M, k, None,
                                            ob[2], ob[3], ws_b)
        for b in range(B):
            seqs[b].step(scripts[b].tree[t], scripts[b].ver[t])
        torch.cuda.synchronize()
        fused = int(ws_a.view(torch.int32)[0].item()) != SENTINEL
        assert fused == expect[t], f"step {t}: launch form"
        assert torch.equal(oa[1], ob[1]), f"step {t}: counts differ"
        for b in range(B):
            nb = int(oa[1][b].item())
            assert torch.equal(oa[0][b, :nb], ob[0][b, :nb]), f"step {t} seq {b}: active sets differ"
        assert torch.equal(oa[2], ob[2]) and torch.equal(oa[3], ob[3]), f"step {t}: top-k differs"
        say(f"batch decode with member calls, step {t}: {'two' if fused else 'three'} launches, ok")
    for b in range(B):
        I = seqs[b].active()
        nb = int(oa[1][b].item())
        assert nb == len(I) and np.array_equal(oa[0][b, :nb].cpu().numpy(), I), f"seq {b}: vs oracle"
