"""GPU parity of the ablation stream modes (context only, decoding tuples
only): the same call sequence as a normal run, with the state's mode set,
against the oracle's Sequence_ in the same mode (|S|, window, active ids and
bitmap bit-exactly at every step; the draft head on sampled steps)."""
import numpy as np
import pytest
import torch

import oracle.nanospec_oracle as O
from dynamic_vocab_draft_amd import workloads as WL
from tests.gpu_common import dcode_of, check_logits, check_topk, dev_elems, dev_i32, say
from tests.test_gpu_parity import GpuSeq, check_state

pytestmark = pytest.mark.gpu

MODES = {"full": 0, "ctx_only": 1, "ext_only": 2}


@pytest.fixture(scope="module")
def ns():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocab_draft_amd import nanospec
    return nanospec


def run_mode(ns, name, mode, steps, head_steps, prefill_k=0):
    cfg = WL.get_config(name)
    say(f"modes {name} {mode}: {steps} steps")
    assert ns.NS_STREAM_FULL == MODES["full"] and ns.NS_STREAM_CTX_ONLY == MODES["ctx_only"]
    assert ns.NS_STREAM_EXT_ONLY == MODES["ext_only"]
    script = WL.make_id_script(cfg, steps)
    g = GpuSeq(ns, cfg.V, cfg.w_max)
    ns.nanospec_state_set_mode(g.st, MODES[mode])
    seq = O.Sequence_(cfg.w_max, mode)
    g.append(script.prompt, 0)
    seq.append_prompt(script.prompt)
    if prefill_k:                                   # a prefill union appended with dedup
        rng = np.random.default_rng(cfg.seed + 3)
        P = rng.integers(0, cfg.V, size=(16, prefill_k)).astype(np.int32)
        g.append(P.reshape(-1), 1)
        seq.append_prefill_union(P)
    g.active()
    check_state(g, seq, cfg.V, f"{name} {mode} prompt")
    W = dev = None
    if head_steps:
        Wh = WL.make_weights(cfg)
        dev = dev_elems(Wh, cfg.dtype)
        W = Wh
    ws = ns.alloc_workspace(cfg.w_max, cfg.M, cfg.k, cfg.d)
    for t, tree, ver in WL.iter_steps(cfg, script):
        g.step(tree, ver)
        seq.step(tree, ver)
        what = f"{name} {mode} step {t}"
        I = check_state(g, seq, cfg.V, what)
        if t in head_steps:
            h = WL.make_hidden(cfg, t)
            logits = torch.full((cfg.M, cfg.w_max), float("nan"), device="cuda")
            tids = torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda")
            tvals = torch.empty((cfg.M, cfg.k), device="cuda")
            ns.nanospec_draft_logits_topk(dev, ns.NS_INDEXED, g.ids, g.n, cfg.w_max, cfg.V, cfg.d,
                                          dcode_of(ns, cfg.dtype),
                                          dev_elems(h, cfg.dtype), cfg.M, cfg.k, logits, tids, tvals, ws)
            torch.cuda.synchronize()
            ref, o_ids, o_vals = O.draft_head(h, W, I, cfg.k, cfg.dtype)
            check_logits(logits.cpu().numpy()[:, :len(I)], ref, what)
            check_topk(tids.cpu().numpy(), tvals.cpu().numpy(), ref, I, o_ids, o_vals, cfg.k, what)
    assert ns.nanospec_state_status(g.st) == 0
    return g, seq


def test_modes_tiny(ns):
    for mode in ("ctx_only", "ext_only", "full"):
        run_mode(ns, "tiny", mode, 8, set(range(8)), prefill_k=3)


def test_modes_llama3_8b(ns):
    for mode in ("ctx_only", "ext_only"):
        run_mode(ns, "llama3_8b", mode, 24, {0, 23})


def test_mode_switch_and_reset(ns):
    """The mode is a host setting: switching it changes what later calls
    append, and a reset keeps it."""
    cfg = WL.get_config("tiny")
    script = WL.make_id_script(cfg, 6)
    g = GpuSeq(ns, cfg.V, cfg.w_max)
    seq = O.Sequence_(cfg.w_max, "ctx_only")
    ns.nanospec_state_set_mode(g.st, ns.NS_STREAM_CTX_ONLY)
    g.append(script.prompt, 0)
    seq.append_prompt(script.prompt)
    for t in range(3):
        g.step(script.tree[t], script.ver[t])
        seq.step(script.tree[t], script.ver[t])
        check_state(g, seq, cfg.V, f"ctx step {t}")
    ns.nanospec_state_set_mode(g.st, ns.NS_STREAM_FULL)
    seq.mode = "full"
    for t in range(3, 6):
        g.step(script.tree[t], script.ver[t])
        seq.step(script.tree[t], script.ver[t])
        check_state(g, seq, cfg.V, f"full step {t}")
    ns.nanospec_state_set_mode(g.st, ns.NS_STREAM_EXT_ONLY)
    ns.nanospec_state_reset(g.st)
    seq = O.Sequence_(cfg.w_max, "ext_only")
    g.append(script.prompt, 0)                      # dropped: ext-only survives the reset
    seq.append_prompt(script.prompt)
    g.step(script.tree[0], script.ver[0])
    seq.step(script.tree[0], script.ver[0])
    check_state(g, seq, cfg.V, "ext after reset")
    with pytest.raises(ns.NanoSpecError):
        ns.nanospec_state_set_mode(g.st, 3)


def test_batch_refuses_ctx_only_member(ns):
    cfg = WL.get_config("tiny")
    bt = ns.NanoSpecBatch(2, cfg.V, cfg.w_max)
    ns.nanospec_state_set_mode(bt.member(1), ns.NS_STREAM_CTX_ONLY)
    ids = torch.zeros((2, cfg.w_max), dtype=torch.int32, device="cuda")
    n = torch.zeros(2, dtype=torch.int32, device="cuda")
    tr = dev_i32(np.zeros(2 * 4, np.int32))
    cnt = dev_i32(np.full(2, 4, np.int32))
    with pytest.raises(ns.NanoSpecError):
        ns.nanospec_batch_step_update(bt, tr, 4, cnt, 4, tr, 4, cnt, 4, ids, n)
    ns.nanospec_state_set_mode(bt.member(1), ns.NS_STREAM_FULL)
    ns.nanospec_batch_step_update(bt, tr, 4, cnt, 4, tr, 4, cnt, 4, ids, n)
    torch.cuda.synchronize()
    assert n.cpu().tolist() == [1, 1]                # id 0, appended by both tuples
