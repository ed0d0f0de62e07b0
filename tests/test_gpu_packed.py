"""GPU parity of the slot-stable packed buffer: after every step the slot map,
the gather list and n_slots / n_enter are compared bit-exactly with the
oracle's packed_update run on the oracle's own active sets; on sampled steps
the buffer rows of occupied slots are compared bit-exactly with W_head and the
head over the buffer (PACKED mode, holes skipped) is checked against the
oracle to the draft-head tolerance."""
import numpy as np
import pytest
import torch

import oracle.nanospec_oracle as O
from dynamic_vocab_draft_amd import workloads as WL
from tests.gpu_common import dcode_of, check_logits, check_topk, dev_elems, dev_i32, host_elems, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ns():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocab_draft_amd import nanospec
    return nanospec


def new_rows(cap, d, dtype):
    """A row buffer filled with NaN patterns, so an unwritten row shows."""
    if dtype == "bf16":
        return torch.full((cap, d), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return torch.full((cap, d), float("nan"), dtype=torch.float32, device="cuda")


class Packed:
    """One sequence's state, slot map and row buffer, with the oracle beside it."""

    def __init__(self, ns, cfg, W, W_dev, cap=None, w_max=None):
        self.ns, self.cfg, self.W, self.W_dev = ns, cfg, W, W_dev
        self.V, self.d = cfg.V, cfg.d
        self.w_max = w_max or cfg.w_max
        self.cap = cap or self.w_max
        self.dcode = dcode_of(ns, cfg.dtype)
        self.st = ns.NanoSpecState(self.V, self.w_max)
        self.pk = ns.NanoSpecPacked(self.V, self.cap)
        self.rows = new_rows(self.cap, self.d, cfg.dtype)
        self.seq = O.Sequence_(self.w_max)
        self.slots = np.full(self.cap, -1, np.int64)
        self.ids = torch.empty(self.w_max, dtype=torch.int32, device="cuda")
        self.n = torch.zeros(1, dtype=torch.int32, device="cuda")

    def prompt(self, ids):
        self.seq.append_prompt(ids)
        if len(ids):
            self.ns.nanospec_stream_append(self.st, dev_i32(ids), len(ids), 0)
        self.ns.nanospec_active_vocab(self.st, self.ids, self.n, None)
        return self.update()

    def step(self, tree, ver):
        self.seq.step(tree, ver)
        self.ns.nanospec_step_update(self.st, dev_i32(tree) if len(tree) else None, len(tree),
                                     dev_i32(ver) if len(ver) else None, len(ver), self.ids, self.n, None)
        return self.update()

    def update(self):
        self.ns.nanospec_packed_update(self.pk, self.st, self.W_dev, self.d, self.dcode, self.rows)
        I = self.seq.active()
        self.slots, es, ei, n_slots = O.packed_update(self.slots, I)
        return I, es, ei, n_slots

    def check_slots(self, ref, what):
        I, es, ei, n_slots = ref
        torch.cuda.synchronize()
        g_slots = self.pk.slot_ids.cpu().numpy()
        assert np.array_equal(g_slots, self.slots), f"{what}: slot map"
        assert int(self.pk.n_slots.item()) == n_slots, f"{what}: n_slots"
        ne = int(self.pk.n_enter.item())
        assert ne == len(ei), f"{what}: n_enter {ne} vs {len(ei)}"
        assert np.array_equal(self.pk.enter_slots[:ne].cpu().numpy(), es), f"{what}: enter slots"
        assert np.array_equal(self.pk.enter_ids[:ne].cpu().numpy(), ei), f"{what}: enter ids"

    def check_rows(self, what):
        occ = np.flatnonzero(self.slots >= 0)
        got = host_elems(self.rows, self.cfg.dtype)[occ]
        assert np.array_equal(got, self.W[self.slots[occ]]), f"{what}: buffer rows"

    def check_head(self, h, M, k, what):
        cfg = self.cfg
        ws = self.ns.alloc_workspace(self.cap, M, k, self.d)
        logits = torch.full((M, self.cap), float("nan"), device="cuda")
        tids = torch.empty((M, k), dtype=torch.int32, device="cuda")
        tvals = torch.empty((M, k), device="cuda")
        self.ns.nanospec_draft_logits_topk(self.rows, self.ns.NS_PACKED, self.pk.slot_ids, self.pk.n_slots, self.cap,
                                           self.V, self.d, self.dcode, dev_elems(h, cfg.dtype), M, k, logits, tids,
                                           tvals, ws)
        torch.cuda.synchronize()
        n_slots = int(self.pk.n_slots.item())
        live = np.flatnonzero(self.slots[:n_slots] >= 0)
        held = self.slots[live]
        o_ids, o_vals = O.packed_draft_head(h, self.W, self.slots, n_slots, k, cfg.dtype)
        ref = O.project(h, O.gather_rows(self.W, held), cfg.dtype)
        lg = logits.cpu().numpy()
        check_logits(lg[:, live], ref, what)
        holes = np.setdiff1d(np.arange(self.cap), live)
        assert np.isnan(lg[:, holes]).all(), f"{what}: hole or tail columns written"
        check_topk(tids.cpu().numpy(), tvals.cpu().numpy(), ref, held, o_ids, o_vals, k, what)


def poison_padding(p):
    """Fills the bytes after the last bitmap word (up to the 256-byte padding
    of both allocations) with 0xFF: the update must not read them as ids."""
    nw = (p.V + 31) // 32
    def a256(x):
        return (x + 255) // 256 * 256
    st_bm = 256 + a256(p.w_max * 4) + a256(p.V * 4)
    pk_bm = 256 + 3 * a256(p.cap * 4)
    for buf, off in ((p.st.buf, st_bm), (p.pk.buf, pk_bm)):
        end = off + a256(nw * 4)
        assert end <= buf.numel()
        buf[off + nw * 4:end].fill_(0xFF)
    return a256(nw * 4) - nw * 4


def run_packed(ns, name, steps, rows_steps, head_steps, cap=None, w_max=None, dtype=None, poison=False, **over):
    cfg = WL.get_config(name, **({"dtype": dtype} if dtype else {}), **over)
    say(f"packed {name}: generating inputs (cap={cap}, w_max={w_max}, {over})")
    W = WL.make_weights(cfg)
    W_dev = dev_elems(W, cfg.dtype)
    script = WL.make_id_script(cfg, steps)
    p = Packed(ns, cfg, W, W_dev, cap=cap, w_max=w_max)
    if poison:
        torch.cuda.synchronize()
        assert poison_padding(p) > 0
    ref = p.prompt(script.prompt)
    p.check_slots(ref, f"packed {name} prompt")
    p.check_rows(f"packed {name} prompt")
    entered = 0
    for t, tree, ver in WL.iter_steps(cfg, script):
        what = f"packed {name} step {t}"
        ref = p.step(tree, ver)
        p.check_slots(ref, what)
        entered += len(ref[2])
        if t in rows_steps:
            p.check_rows(what)
        if t in head_steps:
            p.check_head(WL.make_hidden(cfg, t), cfg.M, cfg.k, what)
    p.check_rows(f"packed {name} last step")
    assert ns.nanospec_state_status(p.st) == 0
    say(f"packed {name}: {steps} steps, {entered} rows entered")
    return p


def test_packed_tiny(ns):
    run_packed(ns, "tiny", 8, set(range(8)), set(range(8)))
    run_packed(ns, "tiny", 8, set(range(8)), {0, 7}, dtype="bf16")


def test_packed_slots_beyond_window(ns):
    """More slots than W_max: the extra slots stay holes."""
    run_packed(ns, "tiny", 6, set(range(6)), {5}, cap=512 + 37)


def test_packed_full_turnover(ns):
    """A window shorter than one step's appends: most of the set changes at
    every step, and the slot map is rebuilt from holes each time."""
    run_packed(ns, "tiny", 8, set(range(8)), set(range(8)), w_max=20)


def test_packed_partial_bitmap_vector(ns):
    """V = 1061: 34 bitmap words, so the plan's last 16-byte vector holds two
    words and two words of allocation padding, here set to all ones; V % 32
    = 5 leaves padding bits in the last word too."""
    run_packed(ns, "tiny", 8, set(range(8)), {0, 7}, poison=True, V=1061, w_max=200, prompt_len=150)
    run_packed(ns, "tiny", 6, set(range(6)), {5}, poison=True, V=1061, w_max=20, prompt_len=150)


def test_packed_llama3_8b(ns):
    run_packed(ns, "llama3_8b", 40, {0, 1, 17, 39}, {0, 39})


def test_packed_qwen25_7b(ns):
    run_packed(ns, "qwen25_7b", 6, {5}, {5})


def test_packed_stress_max_slots(ns):
    """W_max = NS_MAX_SLOTS = 16384 slots, |I| of 12-16k and ~60 entering ids a
    step."""
    assert WL.get_config("stress").w_max == ns.NS_MAX_SLOTS
    run_packed(ns, "stress", 3, {2}, {2})


def test_packed_reset_and_empty(ns):
    """A reset empties the map; an empty active set leaves only holes, and the
    head over zero slots returns padding."""
    cfg = WL.get_config("tiny")
    W = WL.make_weights(cfg)
    p = Packed(ns, cfg, W, dev_elems(W, cfg.dtype))
    script = WL.make_id_script(cfg, 2)
    p.check_slots(p.prompt(script.prompt), "prompt")
    p.check_slots(p.step(script.tree[0], script.ver[0]), "step 0")
    # The state empties (reset, rebuild): every id leaves.
    ns.nanospec_state_reset(p.st)
    p.seq = O.Sequence_(p.w_max)
    ref = p.prompt(np.zeros(0, np.int32))
    assert ref[3] == 0
    p.check_slots(ref, "empty set")
    tids = torch.zeros((cfg.M, cfg.k), dtype=torch.int32, device="cuda")
    tvals = torch.zeros((cfg.M, cfg.k), device="cuda")
    ws = ns.alloc_workspace(p.cap, cfg.M, cfg.k, cfg.d)
    ns.nanospec_draft_logits_topk(p.rows, ns.NS_PACKED, p.pk.slot_ids, p.pk.n_slots, p.cap, cfg.V, cfg.d, p.dcode,
                                  dev_elems(WL.make_hidden(cfg, 0), cfg.dtype), cfg.M, cfg.k, None, tids, tvals, ws)
    torch.cuda.synchronize()
    assert (tids.cpu().numpy() == -1).all() and np.isneginf(tvals.cpu().numpy()).all()
    # The same ids again, after a reset of the map too: placement restarts from slot 0.
    ns.nanospec_packed_reset(p.pk)
    p.slots[:] = -1
    ref = p.prompt(script.prompt)
    p.check_slots(ref, "after both resets")
    p.check_rows("after both resets")
    assert p.slots[:len(ref[0])].tolist() == ref[0].tolist()


def test_packed_argument_checks(ns):
    cfg = WL.get_config("tiny")
    W_dev = dev_elems(WL.make_weights(cfg), cfg.dtype)
    st = ns.NanoSpecState(cfg.V, cfg.w_max)
    rows = new_rows(cfg.w_max, cfg.d, cfg.dtype)
    small = ns.NanoSpecPacked(cfg.V, cfg.w_max - 1)
    with pytest.raises(ns.NanoSpecError):              # W_max larger than the slot count
        ns.nanospec_packed_update(small, st, W_dev, cfg.d, ns.NS_FP32, rows)
    other_v = ns.NanoSpecPacked(cfg.V + 1, cfg.w_max)
    with pytest.raises(ns.NanoSpecError):              # different vocabulary
        ns.nanospec_packed_update(other_v, st, W_dev, cfg.d, ns.NS_FP32, rows)
    ok = ns.NanoSpecPacked(cfg.V, cfg.w_max)
    with pytest.raises(ns.NanoSpecError):              # d % 8 != 0
        ns.nanospec_packed_update(ok, st, W_dev, cfg.d - 1, ns.NS_FP32, rows)
    with pytest.raises(ns.NanoSpecError):              # unknown dtype
        ns.nanospec_packed_update(ok, st, W_dev, cfg.d, 7, rows)
    torch.cuda.synchronize()
