"""Draft-head step benchmark on one MI355X.

One step is the whole per-step hot path of the dynamic-vocabulary draft head
on the Llama-3-8B-shaped workload (V=128256, d=4096, W_max=3072, M=8 bf16
hidden rows, top-8, 60 raw draft-tree ids + 8 verify ids appended per step):

  nanospec_step_update        append C_draft (dedup) and C_ver, rebuild I
  nanospec_gather_rows        PACKED mode only, on a second stream
  nanospec_packed_update      SLOTS mode only: slot-stable buffer, entering rows
  nanospec_draft_logits_topk  projection on W_head[I,:], top-k, map back

Inputs are seeded synthetic tensors resident in HBM before timing starts.

Timing: the K timed steps are captured once into a HIP graph and replayed,
with one event pair around the replay (an event record costs microseconds on
the GPU timeline, comparable to a step, so there are none between steps).
Cold mode (the headline) streams a 512 MiB buffer through the caches between
steps (a strided read touching every 128-byte line), so each step's rows come
from HBM, not from L2 or the 256 MB Infinity Cache: in decoding, the target
model reads its weights between draft steps.  The cost of that read is
measured by a graph of the same reads alone and subtracted.  Replayed outputs are checked
against an eager run.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def progress(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--config", default="llama3_8b")
    p.add_argument("--mode", default="auto",
                   help="auto (every mode) or a comma-separated list of packed, indexed, slots, decode")
    p.add_argument("--reps", type=int, default=5, help="graph replays per measurement (median)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-extras", action="store_true", help="skip the prefill, overlap and batch legs")
    p.add_argument("--batches", default="1,8,32,64", help="sequence counts of the batched leg")
    p.add_argument("--sweep", action="store_true",
                   help="only sweep the draft head over |I| x M (cold) and print one JSON line per point")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES (calibrates HBM byte counters) and exit")
    p.add_argument("--overlap-study", action="store_true",
                   help="only run the gather/backbone overlap variants (graph and eager, 13 and 1000 gathered "
                        "rows), separated by host pauses so a kernel trace splits them, and exit")
    p.add_argument("--trace-summary", default="", metavar="CSV",
                   help="only summarize a rocprofv3 kernel-trace CSV of an --overlap-study run (no GPU) and exit")
    p.add_argument("--step-trace-summary", default="", metavar="CSV",
                   help="only summarize a rocprofv3 kernel-trace CSV of a bench run per decode-step kernel (no GPU) "
                        "and exit")
    p.add_argument("--sq-summary", nargs="+", default=None, metavar="CSV",
                   help="only tabulate the per-dispatch counters of rocprofv3 --pmc CSVs of a --head-probe run "
                        "(median over each projection kernel's dispatches; no GPU) and exit")
    p.add_argument("--counter-summary", nargs=5, default=None,
                   metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "BENCH_OUT"),
                   help="only write the draft-head traffic summary (no GPU) from FETCH_SIZE and WRITE_SIZE counter "
                        "CSVs of an indexed bench run, the two counters of a --copy-probe run, and that bench run's "
                        "output (its JSON line gives mean |I| and the algorithmic bytes), and exit")
    p.add_argument("--prefill-probe", action="store_true",
                   help="only run the prefill top-K_pre leg (cold, 12 calls), print its JSON and exit")
    p.add_argument("--prefill-counter-summary", nargs=5, default=None,
                   metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "TRACE_CSV"),
                   help="only write the prefill traffic summary (no GPU) from FETCH_SIZE and WRITE_SIZE counter "
                        "CSVs and a kernel-trace CSV of --prefill-probe runs and the two counters of a --copy-probe "
                        "run, and exit")
    p.add_argument("--head-probe", default="", metavar="M[,M...]",
                   help="only run the full-vocabulary projection (V=151936, d=4096, bf16) three times for each "
                        "M, for hardware counters, and exit")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no multi-GPU "
              f"path.", file=sys.stderr)
        sys.exit(2)

    if args.trace_summary:
        print(overlap_trace_summary(args.trace_summary))
        return
    if args.step_trace_summary:
        print(step_trace_summary(args.step_trace_summary))
        return
    if args.sq_summary:
        print(sq_summary(args.sq_summary))
        return
    if args.counter_summary:
        print(counter_summary(*args.counter_summary, workload=args.config))
        return
    if args.prefill_counter_summary:
        print(prefill_counter_summary(*args.prefill_counter_summary))
        return
    import torch
    if args.copy_probe:
        copy_probe(torch, args.copy_probe)
        return
    from dynamic_vocab_draft_amd import nanospec as ns
    from dynamic_vocab_draft_amd import workloads as WL

    torch.cuda.set_device(0)
    if args.prefill_probe:
        flush = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        lines = flush.view(-1, 128)
        sink = torch.empty(lines.shape[0], dtype=torch.uint8, device="cuda")
        print(json.dumps(prefill_leg(torch, ns, WL, lambda i: sink.copy_(lines[:, i % 128]))))
        return
    if args.head_probe:
        head_probe(torch, ns, [int(x) for x in args.head_probe.split(",")])
        return
    if args.sweep:
        sweep(torch, ns, WL, args)
        return
    if args.overlap_study:
        overlap_study(torch, ns, WL)
        return
    cfg = WL.get_config(args.config)
    K, Wm = args.steps, args.warmup
    # Generous id script: the lead-in (steps until |S| reaches W_max, each
    # step appends at least k_ver ids) plus warm-up and timed steps.
    T_script = Wm + K + -(-max(0, cfg.w_max - cfg.prompt_len) // max(1, cfg.k_ver)) + 1
    dcode = ns.NS_BF16 if cfg.dtype == "bf16" else ns.NS_FP32
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    # ---- inputs, resident on the GPU before timing ------------------------
    W_host = WL.make_weights(cfg)
    W = dev(W_host)
    script = WL.make_id_script(cfg, steps=T_script)
    trees = [torch.as_tensor(t, dtype=torch.int32).cuda() for t in script.tree]
    vers = [torch.as_tensor(v, dtype=torch.int32).cuda() for v in script.ver]
    prompt = torch.as_tensor(script.prompt, dtype=torch.int32).cuda()
    st = ns.NanoSpecState(cfg.V, cfg.w_max)
    ids = torch.empty(cfg.w_max, dtype=torch.int32, device="cuda")
    n_act = torch.zeros(1, dtype=torch.int32, device="cuda")

    # Lead-in: the untimed steps until the window is full (|S| >= W_max, read
    # from the state), so the warm-up and timed steps that follow run at the
    # workload's steady-state |I| whatever --steps is.
    s_len = torch.zeros(1, dtype=torch.int64, device="cuda")
    ns.nanospec_stream_append(st, prompt, prompt.numel(), 0)
    lead = 0
    ns.nanospec_state_window(st, None, s_len)
    while int(s_len.item()) < cfg.w_max:
        ns.nanospec_step_update(st, trees[lead], trees[lead].numel(), vers[lead], vers[lead].numel(), ids, n_act)
        ns.nanospec_state_window(st, None, s_len)
        lead += 1
    t0 = lead + Wm                               # first timed step
    T = t0 + K
    hs = torch.stack([dev(WL.make_hidden(cfg, t)) for t in range(T)])
    progress(f"{cfg.name} inputs resident on the GPU; lead-in {lead} steps, timed steps {t0}..{T - 1}")
    packed = torch.zeros((cfg.w_max, cfg.d), dtype=tdt, device="cuda")
    pk = ns.NanoSpecPacked(cfg.V, cfg.w_max)
    slot_rows = torch.zeros((cfg.w_max, cfg.d), dtype=tdt, device="cuda")
    SLOTS = "slots"
    DECODE = "decode"                            # nanospec_decode_step: state update and draft head in one call
    ws = ns.alloc_workspace(cfg.w_max, cfg.M, cfg.k, cfg.d)
    ws_dec = ns.alloc_decode_workspace(cfg.w_max, cfg.n_tree + cfg.k_ver, cfg.M, cfg.k, cfg.d)
    tids = torch.empty((T, cfg.M, cfg.k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((T, cfg.M, cfg.k), dtype=torch.float32, device="cuda")
    flush = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    flush_lines = flush.view(-1, 128)            # one row per 128-byte cache line
    sink = torch.empty(flush_lines.shape[0], dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()

    def init_state():
        ns.nanospec_state_reset(st)
        ns.nanospec_stream_append(st, prompt, prompt.numel(), 0)
        ns.nanospec_active_vocab(st, ids, n_act)

    def pack_update(stream=None):
        ns.nanospec_packed_update(pk, st, W, cfg.d, dcode, slot_rows, stream=stream)

    def state_part(t):
        ns.nanospec_step_update(st, trees[t], trees[t].numel(), vers[t], vers[t].numel(), ids, n_act)

    # |I|, entering rows and slots in use per step, from an untimed pass.
    init_state()
    ns.nanospec_packed_reset(pk)
    pack_update()
    sizes, enters, n_slots = [], [], []
    for t in range(T):
        state_part(t)
        pack_update()
        sizes.append(int(n_act.item()))
        enters.append(int(pk.n_enter.item()))
        n_slots.append(int(pk.n_slots.item()))
    sizes = np.array(sizes)

    def decode_part(t):
        ns.nanospec_decode_step(st, trees[t], trees[t].numel(), vers[t], vers[t].numel(), ids, n_act, W, cfg.V,
                                cfg.d, dcode, hs[t], cfg.M, cfg.k, tids[t], tvals[t], ws_dec)

    def decode_project(t):                       # the step's first launch alone (timing)
        ns.nanospec_decode_step_project(st, trees[t], trees[t].numel(), vers[t], vers[t].numel(), ids, n_act, W,
                                        cfg.V, cfg.d, dcode, hs[t], cfg.M, cfg.k, ws_dec)

    def draft_part(t, mode):
        comp = torch.cuda.current_stream()
        rows = W
        if mode == "project":                      # the projection stage alone (timing)
            ns.nanospec_draft_project(W, ns.NS_INDEXED, ids, n_act, cfg.w_max, cfg.V, cfg.d, dcode, hs[t], cfg.M,
                                      cfg.k, ws)
            return
        if mode == SLOTS:
            pack_update()
            ns.nanospec_draft_logits_topk(slot_rows, ns.NS_PACKED, pk.slot_ids, pk.n_slots, cfg.w_max, cfg.V, cfg.d,
                                          dcode, hs[t], cfg.M, cfg.k, None, tids[t], tvals[t], ws)
            return
        if mode == ns.NS_PACKED:
            copy_stream.wait_stream(comp)
            ns.nanospec_gather_rows(W, cfg.V, cfg.d, dcode, ids, n_act, cfg.w_max, packed, stream=copy_stream)
            comp.wait_stream(copy_stream)
            rows = packed
        ns.nanospec_draft_logits_topk(rows, mode, ids, n_act, cfg.w_max, cfg.V, cfg.d, dcode, hs[t], cfg.M, cfg.k,
                                      None, tids[t], tvals[t], ws)

    def body(mode, cold, with_state=True, with_draft=True):
        # In the decode mode, with_state alone is the step's first launch
        # (the state update beside the projection).
        def run():
            for t in range(t0, T):
                if cold:
                    sink.copy_(flush_lines[:, (t * 7) % 128])
                if mode == DECODE:
                    if with_state and with_draft:
                        decode_part(t)
                    elif with_state:
                        decode_project(t)
                    continue
                if with_state:
                    state_part(t)
                if with_draft:
                    draft_part(t, mode)
        return run

    def warm_up_state(mode=None):
        init_state()
        if mode == SLOTS:
            ns.nanospec_packed_reset(pk)
            pack_update()
        for t in range(t0):
            if mode == DECODE and t == t0 - 1:
                decode_part(t)                   # the state keeps I_t: the timed steps take the fused form
                continue
            state_part(t)
            if mode == SLOTS:
                pack_update()

    def capture(fn, mode=None):
        warm_up_state(mode)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time_graph(g, needs_state=True, mode=None):
        ts = []
        for _ in range(args.reps):
            if needs_state:
                warm_up_state(mode)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    def time_diff(g1, g2, mode=None):
        """Median over interleaved replay pairs of time(g1) - time(g2), in ms.
        Both graphs carry the same K cache-streaming reads (~0.1 ms each),
        whose run-to-run spread is comparable to the microseconds being
        compared; pairing the replays cancels the slow drift."""
        d = []
        for _ in range(max(3 * args.reps, 15)):
            t = []
            for g in (g1, g2):
                warm_up_state(mode)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                t.append(a.elapsed_time(b))
            d.append(t[0] - t[1])
        return float(np.median(d))

    def time_eager(fn, mode=None):
        warm_up_state(mode)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3

    by_name = {"packed": ns.NS_PACKED, "indexed": ns.NS_INDEXED, "slots": SLOTS, "decode": DECODE}
    names = list(by_name) if args.mode == "auto" else args.mode.split(",")
    if not names or any(n not in by_name for n in names):
        raise SystemExit(f"--mode: auto or a comma-separated list of {', '.join(by_name)}")
    modes = [by_name[n] for n in names]
    mname = {ns.NS_PACKED: "packed", ns.NS_INDEXED: "indexed", SLOTS: "slots", DECODE: "decode"}
    g_flush = capture(body(None, True, False, False))
    t_flush = time_graph(g_flush, needs_state=False)

    res = {}
    decode_fused = False
    for m in modes:
        # eager reference outputs for the replay check
        if m == DECODE:
            ws_dec.view(torch.int32)[0] = -1           # the fused first launch writes |I_t| here
        time_eager(body(m, False), m)
        if m == DECODE:
            decode_fused = int(ws_dec.view(torch.int32)[0].item()) >= 0
        ref_ids, ref_vals = tids.clone(), tvals.clone()
        tids.fill_(-7)
        g_cold = capture(body(m, True), m)
        g_warm = capture(body(m, False), m)
        g_state = capture(body(m, True, True, False), m)
        time_graph(g_cold, mode=m)                     # replays whose outputs the check reads
        ok = bool(torch.equal(tids[t0:], ref_ids[t0:]) and torch.equal(tvals[t0:], ref_vals[t0:]))
        t_warm = time_graph(g_warm, mode=m)
        t_draft = time_diff(g_cold, g_state, mode=m)
        # Step and state update against the reads alone, also over paired
        # replays (the reads' drift between separate medians reached several
        # us per step at K = 200).
        t_step = time_diff(g_cold, g_flush, mode=m)
        t_st = time_diff(g_state, g_flush, mode=m)
        res[m] = dict(cold_ms=t_step / K, warm_ms=t_warm / K,
                      draft_ms=t_draft / K, state_ms=t_st / K,
                      eager_warm_ms=time_eager(body(m, False), m) / K, replay_matches_eager=ok)
        if m == DECODE:                                # first launch, and the merge launch after it
            res[m]["project_ms"] = res[m].pop("state_ms")
            res[m]["select_ms"] = res[m].pop("draft_ms")
        del g_cold, g_warm, g_state
        progress(f"mode {mname[m]}: {res[m]['cold_ms'] * 1e3:.2f} us/step cold")
    best = min(modes, key=lambda m: res[m]["cold_ms"])
    r = res[best]
    # The separate calls' figures (draft call, state update) come from the
    # fastest separate mode, when one ran.
    sep = [m for m in modes if m != DECODE]
    rs = res[min(sep, key=lambda m: res[m]["cold_ms"])] if sep else None
    # The projection stage on its own: the INDEXED projection after the
    # state update, minus the state update alone.
    g_proj = capture(body("project", True))
    g_st = capture(body("project", True, True, False))
    t_proj_ms = time_diff(g_proj, g_st) / K
    del g_proj, g_st

    ms = r["cold_ms"]
    n_mean = float(np.mean(sizes[t0:]))
    s = cfg.elem_bytes
    words = (cfg.V + 31) // 32
    # Algorithmic bytes of one draft-head call: active rows, h, row ids, outputs.
    draft_bytes = n_mean * cfg.d * s + cfg.M * cfg.d * s + n_mean * 4 + cfg.M * cfg.k * 8
    # The projection's own algorithmic bytes: active rows, h and row ids.
    proj_bytes = n_mean * cfg.d * s + cfg.M * cfg.d * s + n_mean * 4
    proj_GBps = proj_bytes / (t_proj_ms * 1e-3) / 1e9
    # The state update's: ring read, tuple ids, bitmap write (and the id list).
    state_bytes = cfg.w_max * 4 + (cfg.n_tree + cfg.k_ver) * 4 + words * 4
    step_bytes = draft_bytes + state_bytes + n_mean * 4
    projection_stage = {"kernel": "nanospec_draft_project (INDEXED; k_proj_mfma, or k_proj_msplit for 48 < M <= 64 "
                                  "over many rows)",
                        "bytes_per_launch": proj_bytes, "avg_launch_us": t_proj_ms * 1e3, "achieved": proj_GBps,
                        "frac": proj_GBps / HBM_PEAK_GBS,
                        "traffic": measured_traffic(cfg.name, "indexed", n_mean, "traffic_bytes_per_projection")}
    draft_call = None
    if rs is not None:
        achieved = draft_bytes / (rs["draft_ms"] * 1e-3) / 1e9
        sname = mname[min(sep, key=lambda m: res[m]["cold_ms"])]
        draft_call = {"kernels": "nanospec_draft_logits_topk = k_proj_mfma + k_merge_cols", "mode": sname,
                      "bytes": draft_bytes, "avg_us": rs["draft_ms"] * 1e3, "achieved": achieved,
                      "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(cfg.name, sname, n_mean)}
    if best == DECODE and decode_fused:
        # The step's dominant kernel is its first launch: the projection of
        # the tuple and I_t columns with the state update in block 0.  Its
        # algorithmic bytes: the projection's (I_{t+1} rows, h, ids) and the
        # state update's.
        a_bytes = proj_bytes + state_bytes
        a_us = r["project_ms"] * 1e3
        a_GBps = a_bytes / (a_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": a_GBps, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": a_GBps / HBM_PEAK_GBS,
                    "traffic": measured_traffic(cfg.name, "decode", n_mean, "traffic_bytes_per_decode_project"),
                    "kernel": "first launch of nanospec_decode_step (nanospec_decode_step_project): k_proj_mfma "
                              "with the window-state update in block 0",
                    "bytes_per_launch": a_bytes, "avg_launch_us": a_us,
                    "projection_stage": projection_stage, "draft_call": draft_call}
    else:
        roofline = {"bound": "hbm", "achieved": proj_GBps, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": proj_GBps / HBM_PEAK_GBS, "traffic": projection_stage["traffic"],
                    "kernel": projection_stage["kernel"], "bytes_per_launch": proj_bytes,
                    "avg_launch_us": t_proj_ms * 1e3, "draft_call": draft_call}

    out = {
        "metric": "draft LM-head steps/s (V=128k,d=4096,W_max=3072) + achieved HBM GB/s vs peak",
        "value": 1000.0 / ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Zipf/pool id streams, N(0,0.02) bf16 W_head, N(0,1) bf16 h)",
        "config": {"workload": f"{cfg.name}: V={cfg.V} d={cfg.d} W_max={cfg.w_max} M={cfg.M} k={cfg.k}, "
                               f"{cfg.n_tree} draft-tree + {cfg.k_ver} verify ids per step",
                   "mode": mname[best], "cache": "cold (512 MiB streamed through the caches between steps)",
                   "decode_two_launch_form": decode_fused if DECODE in modes else None,
                   "mean_active": n_mean, "lead_in_steps": lead, "timed_steps": [t0, T - 1],
                   "timing": "hipGraph replay of the timed steps"},
        "roofline": roofline,
        "step": {"alg_bytes": step_bytes, "step_GBps": step_bytes / (ms * 1e-3) / 1e9,
                 "state_update_us": rs["state_ms"] * 1e3 if rs else None,
                 "draft_us": rs["draft_ms"] * 1e3 if rs else None,
                 "decode_first_launch_us": res[DECODE]["project_ms"] * 1e3 if DECODE in res and decode_fused else None,
                 "decode_merge_us": res[DECODE]["select_ms"] * 1e3 if DECODE in res and decode_fused else None,
                 "warm_ms": r["warm_ms"], "eager_warm_ms": r["eager_warm_ms"],
                 "per_mode": {mname[m]: {k: (round(v, 5) if isinstance(v, float) else v) for k, v in res[m].items()}
                              for m in modes},
                 "flush_ms": t_flush / K,
                 "slots": {"mean_entering_rows": float(np.mean(enters[t0:])),
                           "mean_slots_in_use": float(np.mean(n_slots[t0:])),
                           "gather_bytes_per_step": float(np.mean(enters[t0:])) * 2 * cfg.d * s,
                           "full_gather_bytes_per_step": n_mean * 2 * cfg.d * s}},
        "cpu_baseline": None,
    }
    if not args.no_extras:
        flush_fn = lambda i: sink.copy_(flush_lines[:, i % 128])
        progress("prefill top-K leg")
        out["prefill"] = prefill_leg(torch, ns, WL, flush_fn)
        progress("gather / backbone overlap leg")
        out["overlap"] = overlap_leg(torch, ns, cfg, W, ids, n_act, packed, hs[t0], ws, dcode, copy_stream,
                                     flush_fn)
        progress("decode pipeline leg")
        backbone = make_backbone(torch, cfg)

        class Head:
            def __init__(self, mode, fn, owns_state=False):
                self.mode, self.fn, self.owns_state = mode, fn, owns_state

            def __call__(self, t, comp, copy):
                self.fn(t, comp, copy)

        def head_indexed(t, comp, copy):
            backbone()
            ns.nanospec_draft_logits_topk(W, ns.NS_INDEXED, ids, n_act, cfg.w_max, cfg.V, cfg.d, dcode, hs[t],
                                          cfg.M, cfg.k, None, tids[t], tvals[t], ws)

        def head_slots(overlap):
            def f(t, comp, copy):
                if overlap:
                    copy.wait_stream(comp)
                    pack_update(copy)
                    backbone()
                    comp.wait_stream(copy)
                else:
                    backbone()
                    pack_update()
                ns.nanospec_draft_logits_topk(slot_rows, ns.NS_PACKED, pk.slot_ids, pk.n_slots, cfg.w_max, cfg.V,
                                              cfg.d, dcode, hs[t], cfg.M, cfg.k, None, tids[t], tvals[t], ws)
            return f

        def head_full_gather(t, comp, copy):
            copy.wait_stream(comp)
            ns.nanospec_gather_rows(W, cfg.V, cfg.d, dcode, ids, n_act, cfg.w_max, packed, stream=copy)
            backbone()
            comp.wait_stream(copy)
            ns.nanospec_draft_logits_topk(packed, ns.NS_PACKED, ids, n_act, cfg.w_max, cfg.V, cfg.d, dcode, hs[t],
                                          cfg.M, cfg.k, None, tids[t], tvals[t], ws)

        def head_decode(t, comp, copy):
            backbone()
            decode_part(t)

        heads = {"decode": Head(DECODE, head_decode, owns_state=True),
                 "indexed": Head(ns.NS_INDEXED, head_indexed),
                 "slots_serial": Head(SLOTS, head_slots(False)),
                 "slots_overlap": Head(SLOTS, head_slots(True)),
                 "full_gather_overlap": Head(ns.NS_PACKED, head_full_gather)}
        out["pipeline"] = pipeline_leg(torch, cfg, backbone, warm_up_state, state_part, heads, flush_fn, t0,
                                       min(K, 40), copy_stream)
        progress("tree drafting leg")
        out["tree"] = tree_leg(torch, ns, cfg, W, ids, n_act, dcode, flush_fn)
        progress("stream-source ablation and W_max leg")
        out["ablation"] = ablation_leg(torch, ns, WL, cfg, W, dcode, flush_fn)
        progress("batched-sequences leg")
        out["batched"] = batch_leg(torch, ns, WL, cfg, W, dcode, flush_fn, [int(x) for x in args.batches.split(",")])
        for name in ("qwen25_7b", "stress"):
            progress(f"{name} leg")
            out[name] = config_leg(torch, ns, WL, flush_fn, name)
    # The launch floor of the step's chain: the same cold protocol with three
    # dependent launches that do nothing but touch one element each.
    out["dispatch_floor"] = dispatch_floor(torch, lambda i: sink.copy_(flush_lines[:, i % 128]), K, args.reps)
    if not args.no_dense:
        out["dense"] = dense_compare(torch, ns, cfg, W, hs[t0], dcode, lambda i: sink.copy_(flush_lines[:, i % 128]), ms)
    if not args.no_cpu_baseline:
        progress("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(cfg, W_host, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def copy_probe(torch, nbytes):
    """A plain device-to-device copy of a known size, three times.  Profiled
    with the FETCH_SIZE / WRITE_SIZE counters it gives the factor between what
    those counters read and the bytes a kernel really moves."""
    torch.cuda.set_device(0)
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "copies": 3}), flush=True)


def head_probe(torch, ns, Ms, V=151936, d=4096, k=16):
    """The projection stage alone (nanospec_draft_project, PACKED over all V
    rows of a seeded N(0, 0.02^2) bf16 head), three calls per M: the same
    kernels as the full-vocabulary comparison, for per-kernel hardware
    counters."""
    g = torch.Generator(device="cuda")
    g.manual_seed(1005)
    W = torch.randn((V, d), generator=g, device="cuda").mul_(0.02).to(torch.bfloat16)
    for M in Ms:
        h = torch.randn((M, d), generator=g, device="cuda").to(torch.bfloat16)
        ws = ns.alloc_workspace(V, M, k, d)
        for _ in range(3):
            ns.nanospec_draft_project(W, ns.NS_PACKED, None, None, V, V, d, ns.NS_BF16, h, M, k, ws)
        torch.cuda.synchronize()
        del ws
    print(json.dumps({"head_probe_M": Ms, "V": V, "d": d, "calls_per_M": 3}), flush=True)


DRAFT_SOURCES = ("dynamic_vocab_draft_amd/csrc/draft.hip", "dynamic_vocab_draft_amd/csrc/select.hpp",
                 "dynamic_vocab_draft_amd/csrc/common.hpp", "dynamic_vocab_draft_amd/csrc/state_fast.hpp",
                 "dynamic_vocab_draft_amd/csrc/state_internal.hpp")


PREFILL_SOURCES = ("dynamic_vocab_draft_amd/csrc/prefill.hip", "dynamic_vocab_draft_amd/csrc/common.hpp")


def kernel_source_hash(sources=DRAFT_SOURCES):
    """sha256 of the given kernel sources (the draft head by default) with
    comments and blank space removed, so that only a change to the code
    itself retires the committed counter summary."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, mode, mean_active, key="traffic_bytes_per_call", path=None):
    """HBM bytes per draft-head call (or, with key
    traffic_bytes_per_projection, per k_proj_mfma launch; with
    traffic_bytes_per_decode_project, per first launch of the decode step)
    from the committed counter summary (FETCH_SIZE + WRITE_SIZE, scaled by
    the copy calibration), or None when there is none for this workload and
    mode, the kernel sources changed since the counters were taken, or the
    summary's mean |I| is more than 5% away from this run's (the bytes scale
    with it)."""
    if path is None:
        path = os.path.join(ROOT, "profiles", f"draft_head_{workload}_traffic.txt")
    try:
        with open(path) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != kernel_source_hash() or mode not in kv.get("modes", "").split():
        return None
    try:
        if abs(float(kv["mean_active"]) - mean_active) > 0.05 * mean_active:
            return None
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def _counter_rows(path):
    """Per dispatch (in dispatch order): (kernel name, summed counter value)
    of a rocprofv3 --pmc CSV holding one counter."""
    import csv
    by = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = int(r["Dispatch_Id"])
            name, val = r["Kernel_Name"], float(r["Counter_Value"])
            if key in by:
                by[key][1] += val
            else:
                by[key] = [name, val]
    return [tuple(by[k]) for k in sorted(by)]


def counter_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, bench_out, workload="llama3_8b"):
    """HBM traffic per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch)
    over the cold steps of an indexed (+ decode) bench run: dispatch runs of
    cache-streaming read, k_step_fast, k_proj_mfma, k_merge_cols (indexed)
    and of read, k_proj_mfma, k_merge_fused (the decode step's two launches,
    when the run's fastest mode was decode).  Each counter is scaled by what
    it reads for a plain device copy of known size (the --copy-probe run).
    Mean |I| and the algorithmic bytes come from the bench run's JSON line.
    Returns the summary text that measured_traffic() reads."""
    with open(bench_out) as f:
        line = [l for l in f if l.startswith("{") and '"metric"' in l][-1]
    b = json.loads(line)
    mean_active = float(b["config"]["mean_active"])
    rf = b["roofline"]
    if rf.get("draft_call") is None:
        raise SystemExit(f"{bench_out}: needs a run of the indexed mode")
    with_decode = b["config"]["mode"] == "decode" and bool(b["config"].get("decode_two_launch_form"))
    alg_dec = float(rf["bytes_per_launch"]) if with_decode else None
    alg_proj = float(rf.get("projection_stage", rf)["bytes_per_launch"])
    alg_call = float(rf["draft_call"]["bytes"])
    patterns = {"indexed": (("elementwise_kernel_manual_unroll",), ("k_step_fast",), PROJ_KERNELS, ("k_merge_cols",))}
    if with_decode:
        patterns["decode"] = (("elementwise_kernel_manual_unroll",), PROJ_KERNELS, ("k_merge_fused",))
    per, steps, pname = {}, {}, None
    for tag, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path)
        acc = {(mode, j): [] for mode, pat in patterns.items() for j in range(1, len(pat))}
        for mode, pat in patterns.items():
            for i in range(len(rows) - len(pat) + 1):
                names = [kernel_base_name(rows[i + j][0]) for j in range(len(pat))]
                if all(names[j] in pat[j] for j in range(len(pat))):
                    if mode == "indexed":
                        pname = names[2]
                    for j in range(1, len(pat)):
                        acc[(mode, j)].append(rows[i + j][1])
        for mode in patterns:
            steps[(tag, mode)] = len(acc[(mode, 1)])
            if steps[(tag, mode)] == 0:
                raise SystemExit(f"{path}: no cold {mode} step found")
        per[tag] = {key: float(np.mean(v)) for key, v in acc.items()}
    cal = {}
    for tag, path in (("FETCH_SIZE", copy_fetch_csv), ("WRITE_SIZE", copy_write_csv)):
        cal[tag] = [v for n, v in _counter_rows(path) if "copyBuffer" in kernel_base_name(n)]
    # The copy probe moves COPY_BYTES each way; the calibration is true KiB / counted KiB.
    true_kib = COPY_PROBE_BYTES / 1024.0
    f_cal = true_kib / float(np.median(cal["FETCH_SIZE"]))
    w_cal = true_kib / float(np.median(cal["WRITE_SIZE"]))
    kib = 1024.0
    by = lambda key: (per["FETCH_SIZE"][key] * f_cal + per["WRITE_SIZE"][key] * w_cal) * kib
    proj, merge = by(("indexed", 2)), by(("indexed", 3))
    call = proj + merge
    head = [
        f"# HBM traffic per launch, cold steps of the {workload} workload ({b['config']['workload']};",
        f"# mean |I| = {mean_active:.2f} over the timed steps): "
        + (f"the decode step (nanospec_decode_step: {pname} with the state update in block 0, then "
           f"k_merge_fused) and " if with_decode else "")
        + f"the separate draft-head call ({pname} + k_merge_cols, indexed).",
        f"# bench.py reads the traffic_bytes_* values from this file while source_sha256 matches its kernel",
        f"# sources and its mean |I| is within 5% of this value.",
        f"source_sha256: {kernel_source_hash()}",
        f"modes: indexed" + (" decode" if with_decode else ""),
        f"mean_active: {mean_active:.2f}",
    ]
    if with_decode:
        dproj, dmerge = by(("decode", 1)), by(("decode", 2))
        head += [f"traffic_bytes_per_decode_project: {dproj:.0f}",
                 f"algorithmic_bytes_per_decode_project: {alg_dec:.0f}",
                 f"traffic_bytes_per_decode_step: {dproj + dmerge:.0f}"]
    out = head + [
        f"traffic_bytes_per_call: {call:.0f}",
        f"algorithmic_bytes_per_call: {alg_call:.0f}",
        f"traffic_bytes_per_projection: {proj:.0f}",
        f"algorithmic_bytes_per_projection: {alg_proj:.0f}",
        f"fetch_calibration: {f_cal:.4f}",
        f"write_calibration: {w_cal:.4f}",
        "",
        "Per-dispatch means over the cold steps, KiB as the counters read them:",
    ]
    for tag in ("FETCH_SIZE", "WRITE_SIZE"):
        dec = (f"decode ({steps[(tag, 'decode')]} steps) {pname} (with the state update) "
               f"{per[tag][('decode', 1)]:.1f}, k_merge_fused {per[tag][('decode', 2)]:.1f}; " if with_decode else "")
        out.append(f"  {tag}: {dec}indexed ({steps[(tag, 'indexed')]} steps) k_step_fast "
                   f"{per[tag][('indexed', 1)]:.1f}, {pname} {per[tag][('indexed', 2)]:.1f}, k_merge_cols "
                   f"{per[tag][('indexed', 3)]:.1f}")
    out += [
        f"  copy calibration: a {COPY_PROBE_BYTES}-byte device copy (__amd_rocclr_copyBuffer) reads FETCH_SIZE "
        f"{np.median(cal['FETCH_SIZE']):.1f} KiB and WRITE_SIZE {np.median(cal['WRITE_SIZE']):.1f} KiB",
        f"  (true {true_kib:.0f} KiB each), so FETCH_SIZE is scaled by {f_cal:.4f} and WRITE_SIZE by {w_cal:.4f}.",
    ]
    if with_decode:
        out.append(f"  decode step, first launch: {dproj / 1e6:.3f} MB, {dproj / alg_dec:.3f}x its algorithmic bytes "
                   f"(I_(t+1) rows, h, ids, the state update's ring, tuples and bitmap; it also reads the rows of "
                   f"the tuple and I_t ids that are not in I_(t+1), and writes partial sums); whole step "
                   f"{(dproj + dmerge) / 1e6:.3f} MB.")
    out += [
        f"  draft call: {call / 1e6:.3f} MB per call, {call / alg_call:.3f}x the algorithmic bytes.",
        f"  {pname} alone: {proj / 1e6:.3f} MB per launch, {proj / alg_proj:.3f}x its algorithmic bytes "
        f"(active rows, h, row ids; the partial sums it writes are implementation bytes).",
    ]
    return "\n".join(out)


COPY_PROBE_BYTES = 268435456


def sq_summary(paths, kernels=("k_proj_msplit", "k_proj_mfma")):
    """Markdown table of hardware counters from rocprofv3 --pmc CSVs: per
    dispatch, each counter summed over the rows rocprofv3 reports for it;
    per kernel, the median over its dispatches."""
    import csv
    per = {}                                            # (kernel, counter) -> [values]
    for path in paths:
        acc = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                name = kernel_base_name(r["Kernel_Name"])
                if name not in kernels:
                    continue
                key = (int(r["Dispatch_Id"]), name, r["Counter_Name"])
                acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        for (_, name, counter), v in acc.items():
            per.setdefault((name, counter), []).append(v)
    counters = sorted({c for _, c in per})
    lines = ["| counter | " + " | ".join(kernels) + " |", "|---" * (len(kernels) + 1) + "|"]
    for c in counters:
        cells = [f"{np.median(per[(k, c)]):.0f}" if (k, c) in per else "-" for k in kernels]
        lines.append(f"| {c} | " + " | ".join(cells) + " |")
    return "\n".join(lines)

# The projection stage's kernel: MFMA k-split, MFMA M-split (48 < M <= 64
# over many rows) or the fp32 VALU kernel.
PROJ_KERNELS = ("k_proj_mfma", "k_proj_msplit", "k_proj_valu")

STEP_PATTERNS = {
    "decode": (PROJ_KERNELS, ("k_merge_fused",)),
    "indexed": (("k_step_fast",), PROJ_KERNELS, ("k_merge_cols",)),
    "packed": (("k_step_fast",), ("k_gather",), PROJ_KERNELS, ("k_merge_cols",)),
    "slots": (("k_step_fast",), ("k_pack_plan",), ("k_gather",), PROJ_KERNELS, ("k_merge_cols",)),
}


def kernel_base_name(name):
    """A trace's kernel name without return type, namespaces, template
    arguments and parameters (full or -T truncated names alike)."""
    import re
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    name = re.sub(r"\(.*", "", name).split("<")[0]
    return name.split("::")[-1].strip()


def step_trace_summary(path):
    """Per-kernel spans (End - Start, us) of the cold decode steps in a
    kernel trace of a bench run: dispatch runs of the cache-streaming read
    followed by one mode's step kernels, consecutive on one queue.  Also the
    per-step sums of the decode and indexed steps' kernels."""
    import csv
    ks = []
    with open(path) as f:
        for r in csv.DictReader(f):
            ks.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), kernel_base_name(r["Kernel_Name"]),
                       r["Queue_Id"]))
    ks.sort()
    read = "elementwise_kernel_manual_unroll"
    lines = ["| mode | steps | kernel | mean | median | min | max |", "|---|---|---|---|---|---|---|"]
    step_sums = {"decode": [], "indexed": []}
    for mode, pat in STEP_PATTERNS.items():
        spans = {}                                        # kernel name -> spans, in step order
        n = 0
        for i in range(len(ks) - len(pat)):
            if ks[i][2] != read:
                continue
            seq = ks[i + 1:i + 1 + len(pat)]
            if all(q[2] in p for p, q in zip(pat, seq)) and len({q[3] for q in seq}) == 1:
                n += 1
                for q in seq:
                    spans.setdefault(q[2], []).append((q[1] - q[0]) / 1e3)
                if mode in step_sums:
                    step_sums[mode].append(sum((q[1] - q[0]) / 1e3 for q in seq))
        for name, sp in spans.items():
            v = np.array(sp)
            lines.append(f"| {mode} | {n} | {name} | {v.mean():.3f} | {np.median(v):.3f} | {v.min():.3f} | "
                         f"{v.max():.3f} |")
    for mode, sums in step_sums.items():
        if not sums:
            continue
        v = np.array(sums)
        lines.append("")
        lines.append(f"Per-step kernel time ({mode}, cold; the sum of its kernels' spans over {len(v)} steps): "
                     f"p10 {np.percentile(v, 10):.2f} us, median {np.median(v):.2f} us, "
                     f"p90 {np.percentile(v, 90):.2f} us.")
    return "\n".join(lines)


def prefill_counter_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, trace_csv):
    """The prefill top-K_pre pass's HBM traffic per k_prefill launch from
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch, scaled by the --copy-probe
    calibration) and its duration from a kernel trace, all of --prefill-probe
    runs.  Returns the summary text that measured_prefill_traffic() reads."""
    import csv
    from dynamic_vocab_draft_amd import workloads as WL
    cfg = WL.get_config("prefill")
    alg = cfg.L * cfg.V * 2 + cfg.L * cfg.k_pre * 8
    per = {}
    for tag, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        v = [val for n, val in _counter_rows(path) if kernel_base_name(n) == "k_prefill"]
        if not v:
            raise SystemExit(f"{path}: no k_prefill dispatch")
        per[tag] = v
    cal = {}
    for tag, path in (("FETCH_SIZE", copy_fetch_csv), ("WRITE_SIZE", copy_write_csv)):
        cal[tag] = float(np.median([v for n, v in _counter_rows(path) if "copyBuffer" in kernel_base_name(n)]))
    true_kib = COPY_PROBE_BYTES / 1024.0
    f_cal, w_cal = true_kib / cal["FETCH_SIZE"], true_kib / cal["WRITE_SIZE"]
    fetch = float(np.mean(per["FETCH_SIZE"])) * f_cal * 1024.0
    write = float(np.mean(per["WRITE_SIZE"])) * w_cal * 1024.0
    with open(trace_csv) as f:
        us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in csv.DictReader(f)
              if kernel_base_name(r["Kernel_Name"]) == "k_prefill"]
    if not us:
        raise SystemExit(f"{trace_csv}: no k_prefill dispatch")
    t = float(np.mean(us))
    return "\n".join([
        "# HBM traffic and duration of k_prefill (nanospec_prefill_topk) on the prefill workload:",
        f"# L={cfg.L} positions x V={cfg.V} bf16 logits (N(0, {cfg.sigma:g}^2) plus {cfg.n_peaks} peaks of "
        f"+{cfg.peak:g} per row), K_pre={cfg.k_pre}, cold.",
        "# bench.py reports traffic_bytes_per_call from this file while source_sha256 matches prefill.hip + common.hpp.",
        f"source_sha256: {kernel_source_hash(PREFILL_SOURCES)}",
        f"traffic_bytes_per_call: {fetch + write:.0f}",
        f"algorithmic_bytes_per_call: {alg}",
        f"fetch_calibration: {f_cal:.4f}",
        f"write_calibration: {w_cal:.4f}",
        "",
        f"Per-dispatch counters ({len(per['FETCH_SIZE'])} dispatches each, KiB as read): FETCH_SIZE mean "
        f"{np.mean(per['FETCH_SIZE']):.1f} (min {min(per['FETCH_SIZE']):.1f}, max {max(per['FETCH_SIZE']):.1f}),",
        f"WRITE_SIZE mean {np.mean(per['WRITE_SIZE']):.1f}. Scaled by the copy calibration (a {COPY_PROBE_BYTES}-byte "
        f"device copy reads FETCH_SIZE {cal['FETCH_SIZE']:.1f} KiB and WRITE_SIZE {cal['WRITE_SIZE']:.1f} KiB):",
        f"fetch {fetch / 1e9:.4f} GB + write {write / 1e6:.3f} MB = {(fetch + write) / 1e9:.4f} GB per launch, "
        f"{(fetch + write) / alg:.4f}x the algorithmic bytes (the logits once plus the L x K_pre outputs).",
        "",
        f"Kernel trace ({len(us)} dispatches, cold): mean {t:.1f} us, min {min(us):.1f}, max {max(us):.1f}",
        f"= {alg / (t * 1e-6) / 1e9:.0f} GB/s ({alg / (t * 1e-6) / 1e9 / HBM_PEAK_GBS:.3f} of 8 TB/s).",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp; REPO is the repository root, OUT an output directory):",
        "  rocprofv3 --kernel-trace --stats -T --output-format csv -d $OUT/pkt -o p -- python3 $REPO/bench.py "
        "--prefill-probe",
        "  rocprofv3 --pmc FETCH_SIZE -T --output-format csv -d $OUT/ppf -o p -- python3 $REPO/bench.py --prefill-probe",
        "  rocprofv3 --pmc WRITE_SIZE -T --output-format csv -d $OUT/ppw -o p -- python3 $REPO/bench.py --prefill-probe",
        "  rocprofv3 --pmc FETCH_SIZE -T --output-format csv -d $OUT/cf -o copy -- python3 $REPO/bench.py "
        "--copy-probe 268435456",
        "  rocprofv3 --pmc WRITE_SIZE -T --output-format csv -d $OUT/cw -o copy -- python3 $REPO/bench.py "
        "--copy-probe 268435456",
        "  python3 $REPO/bench.py --prefill-counter-summary $OUT/ppf/p_counter_collection.csv "
        "$OUT/ppw/p_counter_collection.csv $OUT/cf/copy_counter_collection.csv $OUT/cw/copy_counter_collection.csv "
        "$OUT/pkt/p_kernel_trace.csv",
    ])


def measured_prefill_traffic():
    """HBM bytes per k_prefill launch on the prefill workload (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy calibration) from the committed counter
    summary, or None once the prefill sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "prefill_topk_4096x128256_traffic.txt")
    try:
        with open(path) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != kernel_source_hash(PREFILL_SOURCES):
        return None
    try:
        return float(kv["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def _event_time(torch, fn, flush, reps, stream=None):
    """Median of `reps` event-bracketed calls of fn(), each after a cold flush."""
    ts = []
    for i in range(reps + 2):
        flush(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def prefill_leg(torch, ns, WL, flush):
    """a1: per-position top-K_pre over the prefill workload's logits
    (L=4096 x V=128256 bf16, N(0, 3^2) plus 32 peaks of +8 per row), cold.
    The logits are drawn on the GPU from a seeded torch generator (same shape
    and distribution as the test inputs; peak ids uniform here)."""
    cfg = WL.get_config("prefill")
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)
    Z = torch.randn((cfg.L, cfg.V), generator=g, device="cuda", dtype=torch.float32).mul_(cfg.sigma)
    peaks = torch.randint(0, cfg.V, (cfg.L, cfg.n_peaks), generator=g, device="cuda")
    Z.scatter_(1, peaks, Z.gather(1, peaks) + cfg.peak)
    Zb = Z.to(torch.bfloat16)
    del Z
    pid = torch.empty((cfg.L, cfg.k_pre), dtype=torch.int32, device="cuda")
    pval = torch.empty((cfg.L, cfg.k_pre), dtype=torch.float32, device="cuda")
    call = lambda: ns.nanospec_prefill_topk(Zb, cfg.L, cfg.V, ns.NS_BF16, cfg.k_pre, pid, pval)
    ms = _event_time(torch, call, flush, 10)
    nbytes = cfg.L * cfg.V * 2 + cfg.L * cfg.k_pre * 8
    # sanity: the planted ids dominate most rows' top-K
    ref = torch.topk(Zb[:64].float(), cfg.k_pre, dim=1).values
    ok = bool(torch.equal(ref, pval[:64]))
    del Zb
    return {"workload": f"prefill: L={cfg.L} V={cfg.V} bf16, K_pre={cfg.k_pre}", "ms": ms,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes": nbytes, "traffic": measured_prefill_traffic(), "values_match_torch_topk_first_64_rows": ok,
            "cache": "cold"}


def make_backbone(torch, cfg):
    """Stand-in for the draft model's backbone: the seven bf16 GEMMs of one
    Llama-3-8B decoder layer (q, k, v, o, gate, up, down weight shapes) on M
    rows, as one EAGLE-style draft layer would run them."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed + 7)
    shapes = [(4096, 4096), (4096, 4096), (4096, 1024), (4096, 1024), (4096, 14336), (4096, 14336), (14336, 4096)]
    Ws = [(torch.randn((i, o), generator=gen, device="cuda") * 0.02).to(torch.bfloat16) for i, o in shapes]
    xs = {n: torch.randn((cfg.M, n), generator=gen, device="cuda").to(torch.bfloat16) for n in (4096, 14336)}
    outs = [torch.empty((cfg.M, o), dtype=torch.bfloat16, device="cuda") for _, o in shapes]

    def backbone():
        for (i, _), w, o in zip(shapes, Ws, outs):
            torch.matmul(xs[i], w, out=o)
    return backbone


def pipeline_leg(torch, cfg, backbone, warm_up, state_part, heads, flush, Wm, R, copy_stream, reps=5):
    """Decode steps with the state advancing: per step the state update, the
    draft backbone stand-in, and the draft head in one of several variants
    (``heads[name](t, comp, copy)`` enqueues the head's part after the state
    update: it may fork work to the copy stream and must join it before the
    head; a head with ``owns_state`` runs the state update itself and follows
    no separate one).  ``base`` runs the state update and the backbone only,
    ``backbone`` the backbone alone.  Graph replay of R steps, cold, the
    cache-streaming read subtracted; per-step ms."""
    def run_fn(name):
        def run():
            comp = torch.cuda.current_stream()
            for t in range(Wm, Wm + R):
                flush(t)
                if name not in ("flush", "backbone") and not (name in heads and heads[name].owns_state):
                    state_part(t)
                if name == "flush":
                    continue
                if name in ("base", "backbone"):
                    backbone()
                else:
                    heads[name](t, comp, copy_stream)
        return run

    names = ["flush", "base", "backbone"] + list(heads)
    out = {}
    for name in names:
        mode = heads[name].mode if name in heads else None
        warm_up(mode)
        run_fn(name)()                                 # eager pass first
        warm_up(mode)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_fn(name)()
        ts = []
        for _ in range(reps):
            warm_up(mode)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        out[name] = float(np.median(ts)) / R
        del g
    flush_ms = out.pop("flush")
    res = {name: v - flush_ms for name, v in out.items()}
    # A head's cost over the backbone: over base when it follows the separate
    # state update, over the backbone alone when it runs the update itself.
    return {"backbone": "bf16 GEMM chain, Llama-3-8B decoder-layer weight shapes, M rows",
            "steps": R, "step_ms": res,
            "head_cost_ms": {name: res[name] - res["backbone" if heads[name].owns_state else "base"]
                             for name in heads},
            "note": "per step: state update, backbone, draft head variant (decode: backbone, then the decode "
                    "step with its own state update); cold; hipGraph replay"}


def overlap_leg(torch, ns, cfg, W, ids, n_act, packed, h, ws, dcode, copy_stream, flush):
    """a7: the gather on a second stream while a backbone stand-in runs on the
    compute stream (a chain of bf16 GEMMs with one Llama-3-8B decoder layer's
    weight shapes, M rows), then the PACKED draft head after the join.
    Each variant is captured R times (with the cache-streaming read before
    each repetition) into a HIP graph; the read alone is subtracted.
    hidden = (T_serial - T_overlap) / T_gather."""
    M, d = cfg.M, cfg.d
    R = 20
    backbone = make_backbone(torch, cfg)
    tids = torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((cfg.M, cfg.k), dtype=torch.float32, device="cuda")

    def gather(stream):
        ns.nanospec_gather_rows(W, cfg.V, d, dcode, ids, n_act, cfg.w_max, packed, stream=stream)

    def head():
        ns.nanospec_draft_logits_topk(packed, ns.NS_PACKED, ids, n_act, cfg.w_max, cfg.V, d, dcode, h, M, cfg.k,
                                      None, tids, tvals, ws)

    def variant(kind):
        def run():
            comp = torch.cuda.current_stream()
            for i in range(R):
                flush(i)
                if kind == "backbone":
                    backbone()
                elif kind == "gather":
                    gather(comp)
                elif kind == "head":
                    head()
                elif kind == "serial":
                    backbone()
                    gather(comp)
                    head()
                elif kind == "overlap":
                    copy_stream.wait_stream(comp)
                    gather(copy_stream)
                    backbone()
                    comp.wait_stream(copy_stream)
                    head()
                elif kind == "forkjoin":                # the same stream dependencies, no gather
                    copy_stream.wait_stream(comp)
                    backbone()
                    comp.wait_stream(copy_stream)
                    head()
        return run

    kinds = ("flush", "backbone", "gather", "head", "serial", "overlap", "forkjoin")
    for kd in kinds:                                   # warm up every path eagerly first
        variant(kd)()
    torch.cuda.synchronize()
    graphs = {}
    for kd in kinds:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            variant(kd)()
        graphs[kd] = g
    torch.cuda.synchronize()

    def t(kd):
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            graphs[kd].replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    base = t("flush")
    r = {kd: (t(kd) - base) / R for kd in kinds[1:]}
    del graphs
    return {"backbone": "bf16 GEMM chain, Llama-3-8B decoder-layer weight shapes, M rows",
            "T_backbone_ms": r["backbone"], "T_gather_ms": r["gather"], "T_head_ms": r["head"],
            "T_serial_ms": r["serial"], "T_overlap_ms": r["overlap"], "T_forkjoin_no_gather_ms": r["forkjoin"],
            "hidden_fraction": (r["serial"] - r["overlap"]) / r["gather"] if r["gather"] > 0 else None,
            "note": "cold, hipGraph replay of 20 repetitions per variant, cache-streaming read subtracted"}


OVERLAP_VARIANTS = [("flush", 13), ("backbone", 13), ("serial", 13), ("overlap", 13), ("forkjoin", 13),
                    ("serial", 1000), ("overlap", 1000)]


def overlap_study(torch, ns, WL, R=20, reps=3):
    """The overlap leg's variants, for a kernel trace: per repetition the
    cache-streaming read, then the backbone stand-in alone, or with a gather
    of n rows and the PACKED head serially on one stream ("serial"), or the
    gather forked to a second stream beside the backbone and joined before
    the head ("overlap"), or the same fork and join with nothing on the
    second stream ("forkjoin").  n = 13 is the slot-stable buffer's typical
    per-step delta, n = 1000 a whole active set.  Each variant runs R
    repetitions as a graph replay (reps times) and then eagerly (reps times),
    with host pauses between runs so the trace splits into one cluster per
    run.  Prints the per-repetition times (us, the read subtracted)."""
    torch.cuda.set_device(0)
    cfg = WL.get_config("llama3_8b")
    W = torch.from_numpy(WL.make_weights(cfg).view(np.int16)).cuda().view(torch.bfloat16)
    flush_buf = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    lines = flush_buf.view(-1, 128)
    sink = torch.empty(lines.shape[0], dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(cfg.seed + 11)
    ids = torch.as_tensor(np.sort(rng.choice(cfg.V, size=cfg.w_max, replace=False)).astype(np.int32)).cuda()
    counts = {n: torch.tensor([n], dtype=torch.int32, device="cuda") for n in (13, 1000)}
    packed = torch.empty((cfg.w_max, cfg.d), dtype=torch.bfloat16, device="cuda")
    h = torch.randn((cfg.M, cfg.d), device="cuda").to(torch.bfloat16)
    ws = ns.alloc_workspace(cfg.w_max, cfg.M, cfg.k, cfg.d)
    tids = torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((cfg.M, cfg.k), device="cuda")
    backbone = make_backbone(torch, cfg)
    copy = torch.cuda.Stream()

    def gather(stream, n):
        ns.nanospec_gather_rows(W, cfg.V, cfg.d, ns.NS_BF16, ids, counts[n], cfg.w_max, packed, stream=stream)

    def head():
        ns.nanospec_draft_logits_topk(packed, ns.NS_PACKED, ids, counts[1000], cfg.w_max, cfg.V, cfg.d, ns.NS_BF16,
                                      h, cfg.M, cfg.k, None, tids, tvals, ws)

    def variant(kind, n):
        def run():
            comp = torch.cuda.current_stream()
            for i in range(R):
                sink.copy_(lines[:, i % 128])
                if kind == "backbone":
                    backbone()
                elif kind == "serial":
                    backbone()
                    gather(comp, n)
                    head()
                elif kind == "overlap":
                    copy.wait_stream(comp)
                    gather(copy, n)
                    backbone()
                    comp.wait_stream(copy)
                    head()
                elif kind == "forkjoin":
                    copy.wait_stream(comp)
                    backbone()
                    comp.wait_stream(copy)
                    head()
        return run

    def timed(fn):
        ts = []
        for _ in range(reps):
            time.sleep(0.05)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)) / R * 1e3

    for kd, n in OVERLAP_VARIANTS:
        variant(kd, n)()
    torch.cuda.synchronize()
    res = {}
    for kd, n in OVERLAP_VARIANTS:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            variant(kd, n)()
        torch.cuda.synchronize()
        res[f"graph_{kd}_{n}"] = timed(g.replay)
        del g
    for kd, n in OVERLAP_VARIANTS:
        res[f"eager_{kd}_{n}"] = timed(variant(kd, n))
    out = {k: round(v - res[k.split("_")[0] + "_flush_13"], 2) for k, v in res.items()}
    print(json.dumps({"overlap_study_us_per_repetition": out, "R": R, "reps": reps}), flush=True)


def overlap_trace_summary(path, R=20):
    """Markdown table of a kernel trace of an --overlap-study run: the runs
    are the trace's clusters of R cache-streaming reads (split at pauses of
    more than 20 ms), in the study's order (graph replays, then eager runs,
    reps of each variant).  Per repetition, from the end of its read: when
    the first GEMM and the gather start, the GEMMs' summed durations, how
    long after the last GEMM the head starts, the head's span (projection
    start to merge end) and the whole repetition; medians over a run's
    repetitions, then over its reps."""
    import csv
    ks = []
    with open(path) as f:
        for r in csv.DictReader(f):
            nm = r["Kernel_Name"]
            kind = ("gemm" if "Cijk" in nm else "gather" if "k_gather" in nm else
                    "head" if ("k_proj" in nm or "k_merge" in nm) else
                    "read" if ("copy" in nm.lower() and "elementwise" in nm) else "other")
            ks.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), kind, r["Queue_Id"]))
    ks.sort()
    clusters = [[ks[0]]]
    for k in ks[1:]:
        if k[0] - max(x[1] for x in clusters[-1][-8:]) > 20_000_000:
            clusters.append([k])
        else:
            clusters[-1].append(k)
    runs = [c for c in clusters if sum(1 for k in c if k[2] == "read") == R]
    reps = len(runs) // (2 * len(OVERLAP_VARIANTS))
    cols = ["first_gemm_us", "gather_start_us", "gather_us", "gemm_sum_us", "head_after_gemm_us", "head_span_us",
            "repetition_us"]
    lines = ["| run | variant | gathered rows | " + " | ".join(cols) + " |", "|---" * (3 + len(cols)) + "|"]
    for vi, (kd, n) in enumerate(OVERLAP_VARIANTS * 2):
        mode = "graph" if vi < len(OVERLAP_VARIANTS) else "eager"
        meds = []
        for c in runs[vi * reps:(vi + 1) * reps]:
            reads = [k for k in c if k[2] == "read"]
            per = {col: [] for col in cols}
            for i in range(R):
                t0 = reads[i][1]
                t1 = reads[i + 1][0] if i + 1 < R else max(k[1] for k in c)
                inrep = [k for k in c if t0 <= k[0] <= t1]
                g = [k for k in inrep if k[2] == "gemm"]
                ga = [k for k in inrep if k[2] == "gather"]
                hd = [k for k in inrep if k[2] == "head"]
                per["repetition_us"].append((t1 - t0) / 1e3)
                if g:
                    per["first_gemm_us"].append((g[0][0] - t0) / 1e3)
                    per["gemm_sum_us"].append(sum(k[1] - k[0] for k in g) / 1e3)
                if ga:
                    per["gather_start_us"].append((ga[0][0] - t0) / 1e3)
                    per["gather_us"].append((ga[0][1] - ga[0][0]) / 1e3)
                if hd and g:
                    per["head_after_gemm_us"].append((hd[0][0] - g[-1][1]) / 1e3)
                    per["head_span_us"].append((hd[-1][1] - hd[0][0]) / 1e3)
            meds.append({col: (float(np.median(v)) if v else None) for col, v in per.items()})
        cells = []
        for col in cols:
            v = [m[col] for m in meds if m[col] is not None]
            cells.append(f"{np.median(v):.1f}" if v else "-")
        lines.append(f"| {mode} | {kd} | {n} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


def batch_leg(torch, ns, WL, cfg, W, dcode, flush, Bs, steps=48, warm=8):
    """B independent sequences of the same workload (seeds differ), one
    batched step update and one batched draft head (INDEXED) per step, cold,
    graph replay; the step-update-only graph is subtracted for the draft
    time.  Algorithmic bytes of a batched draft call: the sum over sequences
    of n_b*d*s + M*d*s + 4*n_b + 8*M*k.  The same steps through the batched
    decode step (two launches per step once the states hold their active
    sets) are timed the same way."""
    res = []
    s = cfg.elem_bytes
    for B in Bs:
        cfgs = [WL.get_config(cfg.name, seed=cfg.seed + 1000 * (b + 1)) for b in range(B)]
        T = warm + steps
        scripts = [WL.make_id_script(c, steps=T) for c in cfgs]
        nd = cfg.n_tree
        nv = cfg.k_ver
        trees = torch.as_tensor(np.stack([np.stack(sc.tree) for sc in scripts], 1), dtype=torch.int32).cuda()
        vers = torch.as_tensor(np.stack([np.stack(sc.ver) for sc in scripts], 1), dtype=torch.int32).cuda()
        n_d = torch.full((B,), nd, dtype=torch.int32, device="cuda")
        n_v = torch.full((B,), nv, dtype=torch.int32, device="cuda")
        g = torch.Generator(device="cuda")
        g.manual_seed(cfg.seed + 5)
        hs = (torch.randn((T, B, cfg.M, cfg.d), generator=g, device="cuda")).to(W.dtype)
        bt = ns.NanoSpecBatch(B, cfg.V, cfg.w_max)
        ids = torch.empty((B, cfg.w_max), dtype=torch.int32, device="cuda")
        n = torch.zeros(B, dtype=torch.int32, device="cuda")
        wsb = ns.alloc_batch_workspace(B, cfg.w_max, cfg.M, cfg.k, cfg.d)
        tids = torch.empty((B, cfg.M, cfg.k), dtype=torch.int32, device="cuda")
        tvals = torch.empty((B, cfg.M, cfg.k), device="cuda")
        prompts = [torch.as_tensor(sc.prompt, dtype=torch.int32).cuda() for sc in scripts]

        wsd = ns.alloc_batch_decode_workspace(B, cfg.w_max, nd + nv, cfg.M, cfg.k, cfg.d)

        def decode(t):
            ns.nanospec_batch_decode_step(bt, trees[t], nd, n_d, nd, vers[t], nv, n_v, nv, ids, n, W, cfg.V, cfg.d,
                                          dcode, hs[t], cfg.M, cfg.k, tids, tvals, wsd)

        def init(dec=False):
            # dec: the last warm-up step is a decode step, so that the state
            # holds its active set and every timed decode step is fused.
            for b in range(B):
                m = bt.member(b)
                ns.nanospec_state_reset(m)
                ns.nanospec_stream_append(m, prompts[b], prompts[b].numel(), 0)
            for t in range(warm):
                if dec and t == warm - 1:
                    decode(t)
                else:
                    ns.nanospec_batch_step_update(bt, trees[t], nd, n_d, nd, vers[t], nv, n_v, nv, ids, n)

        sizes = []

        def body(with_draft, record=False):
            def run():
                for t in range(warm, T):
                    flush(t)
                    ns.nanospec_batch_step_update(bt, trees[t], nd, n_d, nd, vers[t], nv, n_v, nv, ids, n)
                    if record:
                        sizes.append(n.clone())
                    if with_draft:
                        ns.nanospec_batch_draft_logits_topk(W, ids, n, cfg.w_max, B, cfg.V, cfg.d, dcode, hs[t],
                                                            cfg.M, cfg.k, None, tids, tvals, wsb)
            return run

        init()
        body(False, record=True)()                       # eager pass: |I| per sequence and step
        torch.cuda.synchronize()
        n_mean = float(torch.stack(sizes).float().mean().item())

        def decode_body():
            for t in range(warm, T):
                flush(t)
                decode(t)

        def timed(fn, dec=False):
            init(dec)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                fn()
            ts = []
            for _ in range(3):
                init(dec)
                torch.cuda.synchronize()
                a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                gr.replay()
                b_.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b_))
            del gr
            return float(np.median(ts))

        def flush_only():
            for t in range(warm, T):
                flush(t)

        t_f = timed(flush_only)
        t_s = timed(body(False))
        t_a = timed(body(True))
        t_d = timed(decode_body, dec=True)
        step_us = (t_a - t_f) / steps * 1e3
        dec_us = (t_d - t_f) / steps * 1e3
        draft_us = (t_a - t_s) / steps * 1e3
        draft_bytes = B * (n_mean * cfg.d * s + cfg.M * cfg.d * s + 4 * n_mean + 8 * cfg.M * cfg.k)
        res.append({"B": B, "step_us": step_us, "sequence_steps_per_s": B / (step_us * 1e-6),
                    "state_update_us": (t_s - t_f) / steps * 1e3, "draft_us": draft_us,
                    "draft_GBps": draft_bytes / (draft_us * 1e-6) / 1e9,
                    "draft_frac_of_peak": draft_bytes / (draft_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                    "mean_active": n_mean, "decode_step_us": dec_us,
                    "decode_sequence_steps_per_s": B / (dec_us * 1e-6)})
        del bt, hs, wsb, wsd
    return {"workload": f"{cfg.name} x B independent sequences (seeds differ), batched step update + batched "
                        f"INDEXED draft head, and the batched decode step, cold, hipGraph replay of {steps} steps",
            "per_B": res}


def tree_leg(torch, ns, cfg, W, ids, n_act, dcode, flush, K=10, F=10, N=60, D=5, R=20):
    """Tree drafting on one active set (the state as the main loop left it):
    per depth one log-probability head (1 hidden row at depth 0, F after)
    and one best-F selection, then the best-N selection over all nodes.  The
    cache-streaming read runs before every depth, as the draft backbone's
    weight traffic would.  Graph replay of R trees; the reads alone are
    subtracted.  The same loop with the plain logits head shows what the
    log-softmax costs."""
    P = K + (D - 1) * F * K
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed + 13)
    hs = [torch.randn((1 if t == 0 else F, cfg.d), generator=g, device="cuda").to(W.dtype) for t in range(D)]
    pool_ids = torch.empty(P, dtype=torch.int32, device="cuda")
    pool_vals = torch.empty(P, device="cuda")
    f_idx = torch.empty((D, F), dtype=torch.int32, device="cuda")
    f_vals = torch.empty((D, F), device="cuda")
    f_ids = torch.empty((D, F), dtype=torch.int32, device="cuda")
    fin = [torch.empty(N, dtype=torch.int32, device="cuda"), torch.empty(N, device="cuda"),
           torch.empty(N, dtype=torch.int32, device="cuda")]
    ws = ns.alloc_workspace(cfg.w_max, F, K, cfg.d)

    def tree(kind):
        def run():
            for i in range(R):
                base = 0
                for t in range(D):
                    flush(i * D + t)
                    if kind == "flush":
                        continue
                    M = 1 if t == 0 else F
                    tv, ti = pool_vals[base:base + M * K], pool_ids[base:base + M * K]
                    if kind == "logprob":
                        ns.nanospec_draft_logprob_topk(W, ns.NS_INDEXED, ids, n_act, cfg.w_max, cfg.V, cfg.d, dcode,
                                                       hs[t], M, K, None if t == 0 else f_vals[t - 1], None, None,
                                                       ti, tv, ws)
                    else:
                        ns.nanospec_draft_logits_topk(W, ns.NS_INDEXED, ids, n_act, cfg.w_max, cfg.V, cfg.d, dcode,
                                                      hs[t], M, K, None, ti, tv, ws)
                    ns.nanospec_tree_select(tv, ti, M * K, 1, F, f_idx[t], f_vals[t], f_ids[t])
                    base += M * K
                if kind != "flush":
                    ns.nanospec_tree_select(pool_vals, pool_ids, P, 1, N, fin[0], fin[1], fin[2])
        return run

    out = {}
    for kind in ("flush", "logprob", "logits"):
        tree(kind)()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            tree(kind)()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            gr.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        out[kind] = float(np.median(ts)) / R
        del gr
    n_act_h = int(n_act.item())
    per_tree = out["logprob"] - out["flush"]
    return {"workload": f"{cfg.name}: depth {D}, {K} children per node, frontier {F}, final {N} nodes, "
                        f"|I| = {n_act_h}; cold before every depth; hipGraph replay of {R} trees",
            "tree_us": per_tree * 1e3, "per_depth_us": per_tree * 1e3 / D,
            "tree_with_logits_head_us": (out["logits"] - out["flush"]) * 1e3,
            "logsoftmax_cost_us_per_tree": (out["logprob"] - out["logits"]) * 1e3,
            "draft_nodes_per_s": N / (per_tree * 1e-3)}


def ablation_leg(torch, ns, WL, cfg, W, dcode, flush, steps=48, warm=16):
    """Stream sources of the ablation study (full, context only, decoding
    tuples only) at the workload's W_max, then the full stream over W_max in
    [1024, 8192]: per configuration the mean |I| and the cold per-step times
    of the state update and the INDEXED draft head (graph replay, the
    cache-streaming read and the state-only graph subtracted)."""
    T = warm + steps
    script = WL.make_id_script(cfg, steps=T)
    trees = [torch.as_tensor(t, dtype=torch.int32).cuda() for t in script.tree]
    vers = [torch.as_tensor(v, dtype=torch.int32).cuda() for v in script.ver]
    prompt = torch.as_tensor(script.prompt, dtype=torch.int32).cuda()
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed + 11)
    hs = torch.randn((T, cfg.M, cfg.d), generator=g, device="cuda").to(W.dtype)
    tids = torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((cfg.M, cfg.k), device="cuda")
    s = cfg.elem_bytes
    modes = {"full": ns.NS_STREAM_FULL, "ctx_only": ns.NS_STREAM_CTX_ONLY, "ext_only": ns.NS_STREAM_EXT_ONLY}
    points = [(m, cfg.w_max) for m in modes] + [("full", w) for w in (1024, 2048, 4096, 6144, 8192)
                                                  if w != cfg.w_max]
    out = []
    for mode, w_max in points:
        st = ns.NanoSpecState(cfg.V, w_max)
        ns.nanospec_state_set_mode(st, modes[mode])
        ids = torch.empty(w_max, dtype=torch.int32, device="cuda")
        n = torch.zeros(1, dtype=torch.int32, device="cuda")
        ws = ns.alloc_workspace(w_max, cfg.M, cfg.k, cfg.d)

        def init():
            ns.nanospec_state_reset(st)
            ns.nanospec_stream_append(st, prompt, prompt.numel(), 0)
            ns.nanospec_active_vocab(st, ids, n)
            for t in range(warm):
                ns.nanospec_step_update(st, trees[t], trees[t].numel(), vers[t], vers[t].numel(), ids, n)

        sizes = []

        def body(with_state, with_draft, record=False):
            def run():
                for t in range(warm, T):
                    flush(t)
                    if with_state:
                        ns.nanospec_step_update(st, trees[t], trees[t].numel(), vers[t], vers[t].numel(), ids, n)
                    if record:
                        sizes.append(n.clone())
                    if with_draft:
                        ns.nanospec_draft_logits_topk(W, ns.NS_INDEXED, ids, n, w_max, cfg.V, cfg.d, dcode, hs[t],
                                                      cfg.M, cfg.k, None, tids, tvals, ws)
            return run

        init()
        body(True, False, record=True)()
        torch.cuda.synchronize()
        n_mean = float(torch.stack(sizes).float().mean().item())

        def timed(fn):
            init()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                fn()
            ts = []
            for _ in range(3):
                init()
                torch.cuda.synchronize()
                a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                gr.replay()
                b_.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b_))
            del gr
            return float(np.median(ts))

        t_f = timed(body(False, False))
        t_s = timed(body(True, False))
        t_a = timed(body(True, True))
        draft_us = (t_a - t_s) / steps * 1e3
        draft_bytes = n_mean * cfg.d * s + cfg.M * cfg.d * s + 4 * n_mean + 8 * cfg.M * cfg.k
        out.append({"mode": mode, "w_max": w_max, "mean_active": n_mean,
                    "step_us": (t_a - t_f) / steps * 1e3, "state_update_us": (t_s - t_f) / steps * 1e3,
                    "draft_us": draft_us, "draft_GBps": draft_bytes / (draft_us * 1e-6) / 1e9})
        del st, ws
    return {"workload": f"{cfg.name} id stream under each stream source, and the full stream over W_max; "
                        f"cold, hipGraph replay of {steps} steps", "points": out}


def config_leg(torch, ns, WL, flush, name, steps=32, warm=16):
    """One decode workload besides the headline one, e.g. the stress workload
    (V=151936, d=4096, W_max=16384, M=64, k=16; a uniform id stream keeps
    about 15.5k ids active) or the Qwen-2.5-7B-shaped head (V=151936,
    d=3584, W_max=3072, M=60, k=10): cold per-step times of the state update
    and the INDEXED draft head (graph replay, the cache-streaming read and
    the state-only graph subtracted), of the same step as one
    nanospec_decode_step call (two launches at W_max <= 3072, three above),
    and the full-vocabulary head at the same M.  W and h are drawn on the GPU from a seeded generator with the
    workload's distributions (N(0, 0.02^2) and N(0, 1), bf16)."""
    cfg = WL.get_config(name)
    T = warm + steps
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)
    W = torch.randn((cfg.V, cfg.d), generator=g, device="cuda").mul_(0.02).to(torch.bfloat16)
    hs = torch.randn((T, cfg.M, cfg.d), generator=g, device="cuda").to(torch.bfloat16)
    script = WL.make_id_script(cfg, steps=T)
    trees = [torch.as_tensor(t, dtype=torch.int32).cuda() for t in script.tree]
    vers = [torch.as_tensor(v, dtype=torch.int32).cuda() for v in script.ver]
    prompt = torch.as_tensor(script.prompt, dtype=torch.int32).cuda()
    st = ns.NanoSpecState(cfg.V, cfg.w_max)
    ids = torch.empty(cfg.w_max, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = ns.alloc_workspace(cfg.w_max, cfg.M, cfg.k, cfg.d)
    tids = torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((cfg.M, cfg.k), device="cuda")
    wsdec = ns.alloc_decode_workspace(cfg.w_max, cfg.n_tree + cfg.k_ver, cfg.M, cfg.k, cfg.d)

    def decode(t):
        ns.nanospec_decode_step(st, trees[t], trees[t].numel(), vers[t], vers[t].numel(), ids, n, W, cfg.V, cfg.d,
                                ns.NS_BF16, hs[t], cfg.M, cfg.k, tids, tvals, wsdec)

    def init(with_decode=False):
        ns.nanospec_state_reset(st)
        ns.nanospec_stream_append(st, prompt, prompt.numel(), 0)
        ns.nanospec_active_vocab(st, ids, n)
        for t in range(warm):
            if with_decode and t == warm - 1:
                decode(t)                          # the state keeps I_t for the timed decode steps
            else:
                ns.nanospec_step_update(st, trees[t], trees[t].numel(), vers[t], vers[t].numel(), ids, n)

    sizes = []

    def body(with_state, with_draft, record=False):
        def run():
            for t in range(warm, T):
                flush(t)
                if with_state:
                    ns.nanospec_step_update(st, trees[t], trees[t].numel(), vers[t], vers[t].numel(), ids, n)
                if record:
                    sizes.append(n.clone())
                if with_draft:
                    ns.nanospec_draft_logits_topk(W, ns.NS_INDEXED, ids, n, cfg.w_max, cfg.V, cfg.d, ns.NS_BF16,
                                                  hs[t], cfg.M, cfg.k, None, tids, tvals, ws)
        return run

    init()
    body(True, False, record=True)()
    torch.cuda.synchronize()
    n_mean = float(torch.stack(sizes).float().mean().item())

    def decode_body():
        for t in range(warm, T):
            flush(t)
            decode(t)

    def timed(fn, with_decode=False):
        init(with_decode)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        ts = []
        for _ in range(5):
            init(with_decode)
            torch.cuda.synchronize()
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            gr.replay()
            b_.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b_))
        del gr
        return float(np.median(ts))

    t_f = timed(body(False, False))
    t_s = timed(body(True, False))
    t_a = timed(body(True, True))
    t_d = timed(decode_body, with_decode=True)
    draft_us = (t_a - t_s) / steps * 1e3
    s = cfg.elem_bytes
    draft_bytes = n_mean * cfg.d * s + cfg.M * cfg.d * s + 4 * n_mean + 8 * cfg.M * cfg.k

    # Full-vocabulary head at M = 64: our kernels over every row, and torch.
    wsd = ns.alloc_workspace(cfg.V, cfg.M, cfg.k, cfg.d)
    h0 = hs[warm]

    def ours():
        ns.nanospec_draft_logits_topk(W, ns.NS_PACKED, None, None, cfg.V, cfg.V, cfg.d, ns.NS_BF16, h0, cfg.M,
                                      cfg.k, None, tids, tvals, wsd)

    def vendor():
        z = h0 @ W.t()
        torch.topk(z.float(), cfg.k, dim=1)

    t_ours = _event_time(torch, ours, flush, 10)
    t_vendor = _event_time(torch, vendor, flush, 10)
    step_us = (t_a - t_f) / steps * 1e3
    stream_kind = "uniform id stream" if cfg.prompt_kind == "uniform" else "Zipf/pool id stream"
    res = {"workload": f"{name}: V={cfg.V} d={cfg.d} W_max={cfg.w_max} M={cfg.M} k={cfg.k}, {stream_kind}, "
                       f"cold, hipGraph replay of {steps} steps",
           "mean_active": n_mean, "step_us": step_us, "state_update_us": (t_s - t_f) / steps * 1e3,
           "decode_step_us": (t_d - t_f) / steps * 1e3,
           "draft_us": draft_us, "draft_GBps": draft_bytes / (draft_us * 1e-6) / 1e9,
           "draft_frac_of_peak": draft_bytes / (draft_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
           "dense_ours_ms": t_ours, "dense_torch_ms": t_vendor,
           "dense_ours_GBps": cfg.V * cfg.d * s / (t_ours * 1e-3) / 1e9,
           "speedup_vs_dense": min(t_ours, t_vendor) * 1e3 / min(step_us, (t_d - t_f) / steps * 1e3)}
    del st, ws, wsd, wsdec, W, hs
    return res


def sweep(torch, ns, WL, args):
    """Draft head alone (INDEXED, graph replay) over |I| x M on the
    Llama-3-8B-shaped head; one JSON line per point.  Cold: 512 MiB streamed
    through the caches before every call, the read alone subtracted.  Warm
    (us_warm): the same calls back to back, so the rows a call reads were
    read by the call before (up to 16384 rows x 8 KiB = 128 MiB, within the
    256 MB Infinity Cache): the distance between the two shows whether the
    cold protocol really reads the rows from HBM."""
    cfg = WL.get_config("llama3_8b")
    W_host = WL.make_weights(cfg)
    W = torch.from_numpy(W_host.view(np.int16)).cuda().view(torch.bfloat16)
    del W_host
    flush = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    lines = flush.view(-1, 128)
    sink = torch.empty(lines.shape[0], dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(cfg.seed + 11)
    R = 50
    for n in (512, 1024, 2048, 3072, 8192, 16384):
        I = np.sort(rng.choice(cfg.V, size=n, replace=False)).astype(np.int32)
        ids = torch.as_tensor(I).cuda()
        n_dev = torch.tensor([n], dtype=torch.int32, device="cuda")
        for M in (1, 8, 16, 64):
            k = cfg.k
            h = (torch.randn((M, cfg.d), device="cuda")).to(torch.bfloat16)
            ws = ns.alloc_workspace(n, M, k, cfg.d)
            tids = torch.empty((M, k), dtype=torch.int32, device="cuda")
            tvals = torch.empty((M, k), dtype=torch.float32, device="cuda")

            def body(with_head, cold=True):
                def run():
                    for i in range(R):
                        if cold:
                            sink.copy_(lines[:, (i * 7) % 128])
                        if with_head:
                            ns.nanospec_draft_logits_topk(W, ns.NS_INDEXED, ids, n_dev, n, cfg.V, cfg.d, ns.NS_BF16,
                                                          h, M, k, None, tids, tvals, ws)
                return run

            def capture(fn):
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fn()
                torch.cuda.synchronize()
                return g

            def timed(g):
                ts = []
                for _ in range(3):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    g.replay()
                    b.record()
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                return float(np.median(ts))

            g_all, g_fl, g_warm = capture(body(True)), capture(body(False)), capture(body(True, cold=False))
            us = (timed(g_all) - timed(g_fl)) / R * 1e3
            us_warm = timed(g_warm) / R * 1e3
            nbytes = n * cfg.d * 2 + M * cfg.d * 2 + n * 4 + M * k * 8
            print(json.dumps({"n": n, "M": M, "k": k, "d": cfg.d, "us": us, "bytes": nbytes,
                              "GBps": nbytes / (us * 1e-6) / 1e9,
                              "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                              "us_warm": us_warm}), flush=True)
            del g_all, g_fl, g_warm


def dispatch_floor(torch, flush, K, reps):
    """Graph-replayed chains of three dependent launches that each add 1 to a
    one-element tensor, after the same cache-streaming read as the timed
    steps: the time a three-launch step costs when its kernels do no work.
    Returns microseconds per chain and per launch (the read's graph is
    subtracted)."""
    x = torch.zeros(1, device="cuda")

    def chain(with_launches):
        def run():
            for t in range(K):
                flush(t * 7)
                if with_launches:
                    for _ in range(3):
                        x.add_(1.0)
        return run

    def capture(fn):
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def replay_ms(g):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    # Interleaved replay pairs, as for the steps: the reads' drift between
    # two separate medians is comparable to the chain being measured.
    g_chain, g_read = capture(chain(True)), capture(chain(False))
    diffs = [replay_ms(g_chain) - replay_ms(g_read) for _ in range(max(3 * reps, 15))]
    del g_chain, g_read
    per_chain = float(np.median(diffs)) / K * 1e3
    return {"what": "three dependent one-element launches after the cache-streaming read, graph replay",
            "us_per_chain": per_chain, "us_per_launch": per_chain / 3}


def dense_compare(torch, ns, cfg, W, h, dcode, flush, step_ms):
    """Full-vocabulary head at the same M, cold: our kernel over all V rows and
    torch's bf16 GEMM (hipBLASLt) + torch.topk; the faster is the reference."""
    tids = torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((cfg.M, cfg.k), dtype=torch.float32, device="cuda")
    ws = ns.alloc_workspace(cfg.V, cfg.M, cfg.k, cfg.d)

    def ours():
        ns.nanospec_draft_logits_topk(W, ns.NS_PACKED, None, None, cfg.V, cfg.V, cfg.d, dcode, h, cfg.M, cfg.k,
                                      None, tids, tvals, ws)

    def vendor():
        z = h @ W.t()
        torch.topk(z.float(), cfg.k, dim=1)

    def timeit(fn, reps=20):
        ts = []
        for i in range(reps + 3):
            flush(i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if i >= 3:
                ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    t_ours, t_vendor = timeit(ours), timeit(vendor)
    best = min(t_ours, t_vendor)
    return {"ours_ms": t_ours, "torch_gemm_topk_ms": t_vendor,
            "ours_GBps": cfg.V * cfg.d * cfg.elem_bytes / (t_ours * 1e-3) / 1e9,
            "speedup_vs_dense": best / step_ms, "note": "event-bracketed single calls, cold"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_steps(C, cfg, W, seconds, script, hs, threads):
    """Decode steps of the C++ oracle in about `seconds`: stream update,
    window, sorted unique, float64 projection of W[I, :] (the gather is the
    row reads) and top-k.  Returns (steps, passes, seconds, threads that ran)."""
    done = passes = 0
    used = 1
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        seq = C.Sequence(cfg.w_max)
        seq.append_prompt(script.prompt)
        for t in range(cfg.steps):
            seq.step(script.tree[t], script.ver[t])
            I = seq.active()
            logits, used = C.project(hs[t], W, I, cfg.dtype, threads=threads)
            C.topk(logits, I, cfg.k)
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        passes += 1
    return done, passes, time.perf_counter() - t0, used


def cpu_baseline(cfg, W, seconds):
    """The C++ oracle (oracle/nanospec_oracle.cpp, float64, OpenMP over the
    projection's (m, j) pairs) on a bounded sample of the same workload: as
    many decode steps as fit in about `seconds` on every host core the
    OpenMP runtime is given, then a shorter sample on one thread, and the
    full-vocabulary float64 head once (context for the dense comparison)."""
    import oracle.nanospec_oracle_cpp as C
    from dynamic_vocab_draft_amd import workloads as WL
    script = WL.make_id_script(cfg)
    hs = [WL.make_hidden(cfg, t) for t in range(cfg.steps)]
    done, passes, el, used = _oracle_steps(C, cfg, W, seconds, script, hs, threads=0)
    d1, _, e1, _ = _oracle_steps(C, cfg, W, seconds / 3, script, hs, threads=1)
    t0 = time.perf_counter()
    C.project(hs[0], W, np.arange(cfg.V), cfg.dtype, threads=0)
    dense_s = time.perf_counter() - t0
    return {"value": done / el, "unit": "steps/s", "cores": int(used), "kind": "oracle",
            "sample": f"{done} decode steps of {cfg.name} ({passes} pass(es) over its {cfg.steps} steps: stream "
                      f"update, window, sorted unique, fp64 projection of W[I, :], top-k) in {el:.1f} s by the C++ "
                      f"oracle on {used} OpenMP threads; host has {os.cpu_count()} logical CPUs",
            "single_thread_steps_per_s": d1 / e1, "cpu_model": _cpu_model(),
            "dense_f64_head_s": dense_s, "dense_f64_head_threads": int(used)}


if __name__ == "__main__":
    main()
