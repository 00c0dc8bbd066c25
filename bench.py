#!/usr/bin/env python3
"""SPRINT block-step benchmark on one MI355X.

One benchmark step is one whole SPRINT block over one batch of synthetic
input: the pruning pass (prefix LM-head confidence, key-norm score,
per-modality top-k, compaction, full-prefix attention, block confidence,
unmasking) followed by the pruned denoising steps (attention over the pruned
cache, block confidence, unmasking).  The default workload is the largest
single-GPU one: a bf16 prefix of 32768 positions in 8 alternating text/image
runs (1024 + 3072 each), 16/4 heads of dim 128, vocabulary 163840, pass + 8
steps, r_img = 0.8 against full retention.

Printed: one JSON line.  `value` is denoising block-steps per second
(1 pass + 8 pruned steps = 9 block-steps per block and sequence): the faster
of the whole block replayed as one HIP graph (after checking that a replay
leaves exactly the state an eager run leaves) and the same blocks launched
eagerly from the host; `timing` names which.  The same line carries both
rates, the full-retention baseline, per-call GPU times (each call captured
20 times back to back in a graph, HIP events around 11 replays on the stream
it runs on: median, 10th and 90th percentile of the per-launch means; and
cache-flushed single calls), the roofline of the dominant call, the
image-generation-shaped prefix (16384 positions) pruned against full, the
step counts of a block whose confidences are planted above tau, torch.mm on
the prefix GEMM's shape as a library yardstick, and the CPU oracle timed on
the host (measured on a bounded sample and extrapolated to one block).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector / fp32 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed blocks")
    ap.add_argument("--warmup", type=int, default=5, help="untimed blocks")
    ap.add_argument("--workload", default="interleaved32k")
    ap.add_argument("--cold-iters", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--compare", default="imggen16k",
                    help="second workload timed pruned against full in the same line ('' to skip)")
    ap.add_argument("--no-planted", action="store_true",
                    help="skip the planted-confidence step-count measurement")
    ap.add_argument("--gen-blocks", type=int, default=8,
                    help="blocks of the generation measurement (0: skip it)")
    ap.add_argument("--layers", type=int, default=16,
                    help="layers of the several-layer measurement (0: skip it)")
    ap.add_argument("--moe-experts", type=int, default=256,
                    help="experts of the MoE FFN measurement (0: skip it)")
    ap.add_argument("--profile-call", default=None,
                    help="only launch this call --steps times (for rocprofv3 counter runs); "
                         "'copy' launches a 256 MiB device-to-device copy for calibration")
    return ap.parse_args()


class EventTimer:
    """Records a start/end HIP event pair around named regions on torch's
    current stream (the stream every library call is launched on)."""

    def __init__(self, torch):
        self.torch = torch
        self.records = []

    def __call__(self, name):
        timer = self

        class Ctx:
            def __enter__(self_):
                s = timer.torch.cuda.Event(enable_timing=True)
                s.record()
                self_.s = s

            def __exit__(self_, *a):
                e = timer.torch.cuda.Event(enable_timing=True)
                e.record()
                timer.records.append((name, self_.s, e))
                return False
        return Ctx()

    def summary(self):
        out = {}
        for name, s, e in self.records:
            out.setdefault(name, []).append(s.elapsed_time(e) * 1e3)   # us
        return {k: dict(n=len(v), mean_us=sum(v) / len(v), min_us=min(v), **pctl(v))
                for k, v in out.items()}


def pctl(v):
    """Median, 10th and 90th percentiles (nearest rank) of a list of times."""
    v = sorted(v)
    n = len(v)
    return {"median_us": v[n // 2], "p10_us": v[(n - 1) // 10], "p90_us": v[n - 1 - (n - 1) // 10]}


def work_model(blk):
    """Algorithmic bytes / flops per library call (counted once per launch)."""
    wl, lay = blk.wl, blk.layout
    es, H, V, D, Hq, Hkv, Lq = wl.es, wl.H, wl.vocab, wl.D, wl.Hq, wl.Hkv, wl.Lq
    nseq, L, Lk = lay.nseq, lay.total_L, blk.total_kept
    M = nseq * Lq
    row = Hkv * D * es

    def attn(kv):
        return {"bytes": (kv + nseq * Lq) * row * 2 + 2 * nseq * Lq * Hq * D * es,
                "flops": 4 * Lq * Hq * D * (kv + nseq * Lq)}
    return {
        "lmhead_prefix": {"bytes": V * H * es + L * H * es + L * 8,
                          "flops": 2 * L * H * V, "bound": "mfma"},
        "lmhead_block": {"bytes": V * H * es + M * H * es + M * 8,
                         "flops": 2 * M * H * V, "bound": "hbm"},
        "attend_full": dict(attn(L), bound="hbm"),
        "attend_pruned": dict(attn(Lk), bound="hbm"),
        "score": {"bytes": L * row + 12 * L, "flops": 2 * L * Hkv * D, "bound": "hbm"},
        "prune": {"bytes": 4 * Lk * row + 4 * Lk + 5 * L, "flops": 0, "bound": "hbm"},
        "unmask": {"bytes": M * 14, "flops": 0, "bound": "hbm"},
    }


def src_sha(relpath):
    with open(os.path.join(ROOT, relpath), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(call, workload):
    """HBM bytes per launch of `call` on `workload` from committed rocprofv3
    counter runs, if they were taken on the current kernel source; None
    otherwise (another workload's counters are never reused)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    ent = t.get(f"{call}@{workload}")
    if not ent or ent.get("workload") != workload or ent.get("source_sha") != src_sha(ent["source"]):
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, wl, n_steps):
    """The oracle on the host, on a bounded sample of one block of the same
    workload, extrapolated to the whole block.

    Timed in full, once each: the scoring, top-k and compaction of the whole
    prefix; attention over the full prefix and over the pruned cache; the
    block's LM head (32 rows per sequence); one unmask step.  The prefix-wide
    LM head is timed on two seeded row samples and extrapolated linearly to
    every prefix row (a fixed part per call, converting W, plus a part per
    row).  Block time = prefix LM head + scoring/pruning + full attention +
    (steps + 1) x (LM head + unmask) + steps x pruned attention."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max(i["num_threads"] for i in info) if info else 1
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    lay = x.layout
    nseq, Lq, L = lay.nseq, wl.Lq, int(lay.total_L)
    rng = np.random.default_rng(1)
    t = {}

    def timed(name, fn):
        t0 = time.perf_counter()
        r = fn()
        t[name] = time.perf_counter() - t0
        return r
    n1, n2 = min(L, 256), min(L, 1024)
    rows2 = np.sort(rng.choice(L, n2, replace=False))
    c_s, _, _ = timed("lm_rows_a", lambda: oracle.lmhead_confidence(x.hidden[rows2[:n1]], x.W))
    c_s2, _, _ = timed("lm_rows_b", lambda: oracle.lmhead_confidence(x.hidden[rows2], x.W))
    per_row = max(0.0, (t["lm_rows_b"] - t["lm_rows_a"]) / max(1, n2 - n1))
    fixed = max(0.0, t["lm_rows_a"] - per_row * n1)
    t_prefix_lm = fixed + per_row * L
    # scores from sampled confidences: every row gets the median of the sample
    conf = np.full(L, float(np.median(c_s2)))
    keep = np.array([[oracle.keep_count(wl.r_text, lay.n_text[s]),
                      oracle.keep_count(wl.r_img, lay.n_img[s])] for s in range(nseq)])
    cu_kept = np.concatenate([[0], np.cumsum(keep.sum(1))])

    def prune():
        ib = oracle.key_norm_importance(x.K, lay.cu_len)
        sc = oracle.composite_score(ib, conf, wl.alpha)
        kept = oracle.select_kept(sc, lay.modality, lay.cu_len, keep)
        return oracle.compact(x.K, x.V, kept)
    Kp, Vp = timed("score_topk_compact", prune)
    O = timed("attn_full", lambda: oracle.attention(x.Q, x.K, x.V, lay.cu_len, x.Kb, x.Vb))
    timed("attn_pruned", lambda: oracle.attention(x.Q, Kp, Vp, cu_kept, x.Kb, x.Vb))
    c, a, _ = timed("lm_block", lambda: oracle.lmhead_confidence(
        O.reshape(nseq * Lq, -1), x.W))
    masked = np.ones((nseq, Lq), np.uint8)
    tokens = np.full((nseq, Lq), -1)
    timed("unmask", lambda: oracle.unmask_select(c.reshape(nseq, Lq), a.reshape(nseq, Lq),
                                                masked, tokens, np.float32(wl.tau), n_steps + 1))
    block = (t_prefix_lm + t["score_topk_compact"] + t["attn_full"] +
             (n_steps + 1) * (t["lm_block"] + t["unmask"]) + n_steps * t["attn_pruned"])
    steps = (n_steps + 1) * nseq
    measured = sum(t.values())
    return {"value": steps / block, "unit": "block-steps/s", "cores": int(cores),
            "kind": "oracle", "extrapolated": True,
            "sample": (f"fp64 NumPy oracle, {measured:.1f} s measured: the prefix LM head on "
                       f"{n1} and {n2} seeded prefix rows, extrapolated linearly to all {L} rows "
                       f"({t_prefix_lm:.1f} s); scoring + top-k + compaction of the whole "
                       f"prefix, full and pruned attention, the block LM head and one unmask "
                       f"step timed once each; block = pass + {n_steps} pruned steps "
                       f"({block:.1f} s)"),
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "seconds": {k: round(v, 3) for k, v in t.items()} | {
                "prefix_lm_extrapolated": round(t_prefix_lm, 2), "block": round(block, 2)}}


def profile_call(args, blk, wl, n_steps, torch):
    """Launch one call (or a calibration copy) a few times and exit: a short
    program for rocprofv3 counter passes."""
    if args.profile_call == "copy":
        n = 256 * 1024 * 1024 // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        fn = lambda: b.copy_(a)
        what = "copy of 268435456 bytes"
    else:
        fns = {"lmhead_prefix": blk.prefix_confidence, "score": blk.score_prefix,
               "prune": blk.prune_prefix, "attend_full": lambda: blk.attend(False),
               "attend_pruned": lambda: blk.attend(True), "lmhead_block": blk.block_confidence,
               "unmask": lambda: blk.unmask(1),
               "lmhead_unmask": lambda: blk.confidence_and_unmask(1)}
        blk.run_block(n_steps)
        if args.profile_call == "moe":
            fns["moe"] = moe_call(args, blk, wl, torch)[0]
        fn = fns[args.profile_call]
        what = args.profile_call
    torch.cuda.synchronize()
    for _ in range(args.steps):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"profile_call": what, "launches": args.steps}), flush=True)


def capture_graph(torch, fn):
    """Warm fn up on a side stream, then capture it as a HIP graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_median(torch, g, reps):
    """Median GPU time (s) of one replay, HIP events around each of reps replays."""
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    return sorted(ts)[len(ts) // 2]


def eager_median(torch, fn, reps):
    """Median host wall time (s) of fn launched eagerly, synchronised."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2]


def graph_and_eager(torch, run, state, poison, reps):
    """(graph s, eager s, replay matches eager): run timed eagerly and as a
    graph replay, after checking that a replay, from poisoned outputs,
    leaves exactly the state an eager run leaves."""
    t_e = eager_median(torch, run, reps)
    run()
    torch.cuda.synchronize()
    ref = state()
    g = capture_graph(torch, run)
    poison()
    g.replay()
    torch.cuda.synchronize()
    ok = all(torch.equal(u, v) for u, v in zip(ref, state()))
    t_g = replay_median(torch, g, reps)
    # the last of the timed replays must leave the same state too
    ok = ok and all(torch.equal(u, v) for u, v in zip(ref, state()))
    del g
    return t_g, t_e, ok


def measure_generation(args, x, wl, n_steps, torch, reps=5):
    """B consecutive blocks over a growing prefix (each block's rows join the
    prefix before the next pass), SPRINT vs the unpruned baseline, plus the
    steps each block actually needs under the adaptive schedule."""
    from sparse_prefix_kv_amd.gen import SprintGeneration
    B = args.gen_blocks
    gen = SprintGeneration(x, B, "cuda")
    nseq, Lq = gen.nseq, gen.Lq

    def timed(g_obj, full):
        b = g_obj.blk

        def state():
            return [g_obj.tokens_out.clone(), b.O.clone(), b.kept_idx.clone()]

        def poison():
            g_obj.tokens_out.fill_(-7)
            b.O.zero_()
        return graph_and_eager(torch, lambda: g_obj.run(n_steps, full=full), state, poison, reps)
    t_sp, t_sp_e, ok_sp = timed(gen, False)
    t_full, t_full_e, ok_full = timed(gen, True)
    # steps until every position of the block is accepted (host-checked here,
    # outside the timed runs)
    blk = gen.blk
    finished, max_conf = [], 0.0
    for b in range(B):
        gen.begin_block(b)
        blk.reset()
        blk.pruning_pass(not gen.conf_carried(b))
        t = 0
        max_conf = max(max_conf, float(blk.conf_blk.max().item()))
        while int(blk.masked.sum().item()) > 0 and t < n_steps:
            t += 1
            blk.pruned_step(t)
            max_conf = max(max_conf, float(blk.conf_blk.max().item()))
        finished.append(t + 1)
        gen.finish_block(b)
    # the same generation recomputing every prefix confidence at each pass
    gen_re = SprintGeneration(x, B, "cuda", carry_conf=False)
    t_re, t_re_e, ok_re = timed(gen_re, False)
    del gen_re
    torch.cuda.synchronize()
    T = n_steps + 1
    m0 = Lq
    per_step = -(-m0 // T)
    fixed_steps = -(-m0 // per_step)
    prefix_last = int(np.sum(gen.lens[-1]))
    return {
        "blocks": B, "steps_budget_T": T,
        "prefix_first": int(x.layout.total_L), "prefix_last": prefix_last,
        "timing": "HIP graph replay of the whole generation (eager_ms: host-launched)",
        "replay_matches_eager": bool(ok_sp and ok_full and ok_re),
        "sprint": {"ms": round(t_sp * 1e3, 3), "blocks_per_s": round(B / t_sp, 2),
                   "tokens_per_s": round(B * Lq * nseq / t_sp, 1),
                   "block_steps_per_s": round(B * T * nseq / t_sp, 1),
                   "eager_ms": round(t_sp_e * 1e3, 3)},
        "full_prefix": {"ms": round(t_full * 1e3, 3), "blocks_per_s": round(B / t_full, 2),
                        "tokens_per_s": round(B * Lq * nseq / t_full, 1),
                        "eager_ms": round(t_full_e * 1e3, 3)},
        "sprint_recomputed_conf": {"ms": round(t_re * 1e3, 3),
                                   "blocks_per_s": round(B / t_re, 2),
                                   "eager_ms": round(t_re_e * 1e3, 3),
                                   "note": "every pass runs the LM head over the whole prefix"},
        "speedup": round(t_full / t_sp, 4),
        "adaptive_steps_per_block": finished,
        "fixed_schedule_steps_per_block": fixed_steps,
        "max_block_confidence": round(max_conf, 6), "tau": gen.blk.tau,
        "note": "timed runs launch all T steps of every block (pass + T-1 pruned); the "
                "steps a block needs are counted separately with a host check per step"
                + ("; no confidence exceeds tau with these random weights, so the adaptive "
                   "schedule accepts only its minimum ceil(m/(T-t)) per step"
                   if max_conf <= gen.blk.tau else ""),
    }


def measure_layers(args, x, n_steps, torch, reps=5):
    """A block of an n-layer stand-in (every layer its own prefix cache and
    block inputs; LM head on the last layer): one kept set shared by all
    layers, a set per layer, and the unpruned baseline.  Each is timed as a
    HIP graph replay (GPU time: at 16 attention launches per step the host
    binding, not the GPU, would set an eager rate) after checking that a
    replay leaves what an eager run leaves, and also eagerly from the host."""
    from sparse_prefix_kv_amd.layers import SprintLayers

    def timed_block(b, run):
        def state():
            return [b.tokens.clone(), b.masked.clone(), b.kept_idx.clone(), b.O.clone()]

        def poison():
            b.tokens.fill_(-7)
            b.O.zero_()
        return graph_and_eager(torch, run, state, poison, reps)

    out = {"n_layers": args.layers,
           "note": "layers run in order, one attention launch each; the LM head reads the "
                   "last layer; layer inputs are independent draws (no layer weights); "
                   "block_ms and step_ms are HIP graph replays, eager_* host-launched runs"}
    blk = SprintLayers(x, args.layers, "cuda", mode="shared")
    t_full, t_full_e, all_ok = timed_block(blk, lambda: blk.run_full_block(n_steps))
    blk.run_block(n_steps)
    steps = {}
    for name, pruned in (("full", False), ("pruned", True)):
        fn = (lambda p=pruned: [blk.attend_layers(p), blk.confidence_and_unmask(1)])
        g = capture_graph(torch, fn)
        steps[name] = (replay_median(torch, g, reps), eager_median(torch, fn, reps))
        del g
    for mode in ("shared", "per_layer"):
        if mode != blk.mode:
            del blk
            torch.cuda.synchronize()
            blk = SprintLayers(x, args.layers, "cuda", mode=mode)
        t, t_e, ok = timed_block(blk, lambda: blk.run_block(n_steps))
        all_ok = all_ok and ok
        gp = capture_graph(torch, lambda: [blk.prefix_confidence(), blk.score_and_prune()])
        t_pass = replay_median(torch, gp, reps)
        del gp
        out[mode] = {"block_ms": round(t * 1e3, 4), "pruning_pass_ms": round(t_pass * 1e3, 4),
                     "speedup_vs_full": round(t_full / t, 4),
                     "eager_block_ms": round(t_e * 1e3, 4)}
        if mode == "shared":
            # the same block with its prefix confidences carried from earlier
            # blocks (a generation after its first block): no prefix LM head
            t_c, t_ce, ok = timed_block(blk, lambda: blk.run_block(n_steps, prefix_conf=False))
            all_ok = all_ok and ok
            gp = capture_graph(torch, blk.score_and_prune)
            t_pc = replay_median(torch, gp, reps)
            del gp
            out["shared_carried_conf"] = {
                "block_ms": round(t_c * 1e3, 4), "pruning_pass_ms": round(t_pc * 1e3, 4),
                "speedup_vs_full": round(t_full / t_c, 4), "eager_block_ms": round(t_ce * 1e3, 4),
                "note": "prefix confidences carried (no prefix LM head in the pass)"}
    out["full_prefix"] = {"block_ms": round(t_full * 1e3, 4),
                          "eager_block_ms": round(t_full_e * 1e3, 4)}
    out["step_ms"] = {"pruned": round(steps["pruned"][0] * 1e3, 4),
                      "full": round(steps["full"][0] * 1e3, 4),
                      "speedup": round(steps["full"][0] / steps["pruned"][0], 4),
                      "eager_pruned": round(steps["pruned"][1] * 1e3, 4),
                      "eager_full": round(steps["full"][1] * 1e3, 4)}
    out["replay_matches_eager"] = bool(all_ok)
    del blk
    torch.cuda.synchronize()
    return out


def moe_call(args, blk, wl, torch):
    """One MoE FFN call on the block's attention outputs (M = 32 tokens), with
    synthetic weights drawn on the GPU (the laws of synth.make_moe_weights,
    bf16).  Returns the call, the expert ids it writes, (E, K, I, H, M) and
    the weights (router, bias, gate, up, down)."""
    from sparse_prefix_kv_amd import sprint as sp
    E, K, I, H = args.moe_experts, 8, 512, wl.H
    g = torch.Generator(device="cuda").manual_seed(0)
    bf = torch.bfloat16

    def normal(shape, std):
        return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std).to(bf)
    wr = normal((E, H), H ** -0.5)
    bias = (torch.rand(E, generator=g, device="cuda") - 0.5) * 0.1
    wg = torch.empty((E, I, H), dtype=bf, device="cuda")
    wu = torch.empty_like(wg)
    wd = torch.empty((E, H, I), dtype=bf, device="cuda")
    for e in range(E):            # per expert, to bound the fp32 temporaries
        wg[e] = normal((I, H), H ** -0.5)
        wu[e] = normal((I, H), H ** -0.5)
        wd[e] = normal((H, I), I ** -0.5)
    M = blk.nseq * blk.Lq
    x = blk.O.view(M, H)
    y = torch.empty_like(x)
    ids = torch.empty((M, K), dtype=torch.int32, device="cuda")
    gates = torch.empty((M, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(sp.moe_ffn_ws(M, H, E, K, I), dtype=torch.uint8, device="cuda")

    def call():
        sp.moe_ffn(x, wr, bias, wg, wu, wd, K, residual=x, y=y, expert_ids=ids, gates=gates,
                   ws=ws)
    return call, ids, (E, K, I, H, M), (wr, bias, wg, wu, wd)


def measure_moe(args, blk, x_in, wl, n_steps, torch, reps=20):
    """The MoE FFN (moe_call): 20 back-to-back calls captured in a graph, HIP
    events around the replay.  Algorithmic bytes: every chosen expert's three
    matrices once, the router, and x, the residual and y."""
    call, ids, (E, K, I, H, M), (wr, bias, wg, wu, wd) = moe_call(args, blk, wl, torch)
    call()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            call()
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(5):
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / reps)
    us = sorted(ts)[len(ts) // 2]
    distinct = int(torch.unique(ids).numel())
    alg = distinct * 3 * I * H * 2 + E * H * 2 + 3 * M * H * 2
    del graph

    # a pruned denoising step with the MoE FFN between attention and the LM
    # head, against the same step without it (8 steps captured in a graph)
    from sparse_prefix_kv_amd.block import SprintBlock

    def step_us(b):
        b.run_block(n_steps)
        torch.cuda.synchronize()
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            for t in range(1, n_steps + 1):
                b.pruned_step(t)
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for t in range(1, n_steps + 1):
                b.pruned_step(t)
        gr.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (10 * n_steps)
    blk_moe = SprintBlock(x_in, "cuda", moe=(wr, bias, wg, wu, wd, K, 2.5))
    t_moe = step_us(blk_moe)
    t_plain = step_us(blk)
    del blk_moe, wg, wu, wd
    torch.cuda.synchronize()
    return {"config": f"E {E}, top-{K}, inter {I}, H {H}, M {M} tokens, bf16",
            "us": round(us, 2), "distinct_experts": distinct, "alg_bytes": alg,
            "gbs": round(alg / us / 1e3, 1), "hbm_frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4),
            "bound": "hbm",
            "pruned_step_us": {"with_moe": round(t_moe, 2), "without": round(t_plain, 2)},
            "note": "weights are synthetic (N(0,1/H), N(0,1/I)); the page gives no expert sizes"}


def call_us(torch, fn, reps=20, samples=11):
    """Median per-launch GPU time (us) of fn: reps launches captured in one
    graph, HIP events around each of `samples` replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(samples):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / reps)
    del g
    return sorted(ts)[len(ts) // 2]


def measure_compare(name, n_steps, torch, reps=10):
    """A second workload in the same line: its block pruned (r_img of the
    workload) against full retention (every step on the full prefix), its
    attention call pruned against full, and one denoising step each way."""
    from sparse_prefix_kv_amd import synth
    from sparse_prefix_kv_amd.block import SprintBlock
    wl = synth.WORKLOADS[name]
    x = synth.make_inputs(wl, 0)
    blk = SprintBlock(x, "cuda")
    blk.run_block(n_steps)
    torch.cuda.synchronize()
    g_sp = capture_graph(torch, lambda: blk.run_block(n_steps))
    g_full = capture_graph(torch, lambda: blk.run_full_block(n_steps))
    t_sp = replay_median(torch, g_sp, reps)
    t_full = replay_median(torch, g_full, reps)
    del g_sp, g_full
    att_pr = call_us(torch, lambda: blk.attend(True))
    att_full = call_us(torch, lambda: blk.attend(False))
    conf_un = call_us(torch, lambda: blk.confidence_and_unmask(1))
    work = work_model(blk)
    out = {"workload": name, "desc": wl.desc, "prefix": int(blk.layout.total_L),
           "kept": int(blk.total_kept),
           "block_ms": {"sprint": round(t_sp * 1e3, 4), "full_retention": round(t_full * 1e3, 4)},
           "block_steps_per_s": {"sprint": round((n_steps + 1) * blk.nseq / t_sp, 2),
                                 "full_retention": round((n_steps + 1) * blk.nseq / t_full, 2)},
           "attention_us": {"pruned": round(att_pr, 3), "full": round(att_full, 3)},
           "attention_hbm_frac": {
               "pruned": round(work["attend_pruned"]["bytes"] / att_pr / 1e3 / HBM_PEAK_GBS, 4),
               "full": round(work["attend_full"]["bytes"] / att_full / 1e3 / HBM_PEAK_GBS, 4)},
           "denoising_step_us": {"pruned": round(att_pr + conf_un, 3),
                                 "full": round(att_full + conf_un, 3)},
           "speedup_pruned_vs_full": {"attention_call": round(att_full / att_pr, 4),
                                      "denoising_step": round((att_full + conf_un) /
                                                              (att_pr + conf_un), 4),
                                      "block": round(t_full / t_sp, 4)}}
    del blk
    torch.cuda.synchronize()
    return out


def measure_planted(x, wl, n_steps, torch, fractions=(1.0, 0.5, 0.0), gamma=24.0, reps=5):
    """Steps a block needs under confidence-adaptive unmasking when a known
    fraction of its positions is confident.  After the block's pass, the LM
    head rows of a fraction f of the block's positions are planted along
    their attention outputs (W[v_i] = gamma * O_i / |O_i|^2, so position i's
    logit for token v_i is about gamma = 24 and its confidence about
    1 - V e^-24).  The block then runs with a host check after every step
    and stops once nothing is masked; the fixed schedule always takes
    ceil(m0 / ceil(m0 / T)) steps.  The block's inputs do not change between
    steps here (the model that would refresh them is not on this path), so a
    confidence below tau stays below it and the remaining positions follow
    the minimum ceil(m / (T - t)) rule."""
    from sparse_prefix_kv_amd.block import SprintBlock
    blk = SprintBlock(x, "cuda")
    blk.reset()
    blk.pruning_pass()
    torch.cuda.synchronize()
    M, H, V = blk.nseq * blk.Lq, wl.H, wl.vocab
    O = blk.O.float().view(M, H)
    W0 = blk.W
    T = n_steps + 1
    m0 = blk.Lq
    per_step = -(-m0 // T)
    fixed_steps = -(-m0 // per_step)
    out = {"gamma": gamma, "tau": blk.tau, "steps_budget_T": T,
           "fixed_schedule_steps": fixed_steps, "cases": []}
    for f in fractions:
        n_pl = int(round(f * M))
        pos = torch.arange(n_pl, device="cuda") * M // max(n_pl, 1)
        vocab_rows = (pos * 4099 + 17) % V
        W = W0.clone()
        if n_pl:
            Op = O[pos]
            W[vocab_rows] = (gamma * Op / (Op * Op).sum(1, keepdim=True)).to(W.dtype)
        blk.W = W

        def run_adaptive():
            blk.reset()
            blk.pruning_pass()
            t = 0
            while int(blk.masked.sum().item()) > 0 and t < n_steps:
                t += 1
                blk.pruned_step(t)
            return t + 1
        steps = run_adaptive()
        ts, tf = [], []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run_adaptive()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
            t0 = time.perf_counter()
            blk.run_block(n_steps)
            torch.cuda.synchronize()
            tf.append(time.perf_counter() - t0)
        conf = blk.conf_blk
        out["cases"].append({
            "fraction_planted": f, "adaptive_steps": steps,
            "confident_after_pass": int((conf > blk.tau).sum().item()),
            "block_ms_adaptive": round(sorted(ts)[reps // 2] * 1e3, 4),
            "block_ms_all_T_steps": round(sorted(tf)[reps // 2] * 1e3, 4)})
        del W
    blk.W = W0
    out["timing"] = ("eager with a host check of the mask after every step (both columns); "
                     "all_T_steps launches every step of the budget")
    del blk
    torch.cuda.synchronize()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the SPRINT block step runs on a single MI355X here).", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_prefix_kv_amd import synth
    from sparse_prefix_kv_amd.block import SprintBlock

    wl = synth.WORKLOADS[args.workload]
    n_steps = (wl.T - 1) if wl.T is not None else wl.Lq - 1
    log(f"[bench] workload {wl.name}: {wl.desc}")
    x = synth.make_inputs(wl, 0)
    blk = SprintBlock(x, "cuda")
    lay = blk.layout
    steps_per_block = (n_steps + 1) * lay.nseq
    props = torch.cuda.get_device_properties(0)
    log(f"[bench] device {props.name}, {props.multi_processor_count} CUs; kept "
        f"{blk.total_kept} of {lay.total_L} prefix positions")

    if args.profile_call:
        profile_call(args, blk, wl, n_steps, torch)
        return

    # ---------------------------------------------------------------- warmup
    for _ in range(args.warmup):
        blk.run_block(n_steps)
        blk.run_full_block(n_steps)
    torch.cuda.synchronize()
    log("[bench] warmup done")

    # ---------------------------------------------------------------- eager (host-launched)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        blk.run_block(n_steps)
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / args.steps
    log(f"[bench] eager SPRINT block {t_eager * 1e3:.3f} ms")

    # ---------------------------------------------------------------- graphs
    def capture(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def state():
        return (blk.tokens.clone(), blk.masked.clone(), blk.kept_idx.clone(), blk.O.clone())

    def replay_rate(g, reps):
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps, e0.elapsed_time(e1) * 1e-3 / reps

    g_sprint = capture(lambda: blk.run_block(n_steps))
    g_full = capture(lambda: blk.run_full_block(n_steps))
    # SPRINT with every position kept (r_text = r_img = 1): the pruning pass's
    # overhead without any attention saving
    blk_r1 = SprintBlock(x, "cuda", r_text=1.0, r_img=1.0)
    blk_r1.run_block(n_steps)
    g_r1 = capture(lambda: blk_r1.run_block(n_steps))
    # a replay must leave exactly what an eager run leaves
    blk.run_block(n_steps)
    torch.cuda.synchronize()
    ref = state()
    blk.tokens.fill_(-7)
    blk.O.zero_()
    g_sprint.replay()
    torch.cuda.synchronize()
    graph_ok = all(torch.equal(a, b) for a, b in zip(ref, state()))
    if not graph_ok:
        log("[bench] WARNING: graph replay differs from the eager run; reporting eager")
    _, t_graph = replay_rate(g_sprint, args.steps)
    _, t_full = replay_rate(g_full, args.steps)
    _, t_r1 = replay_rate(g_r1, args.steps)
    # the same verified work launched two ways; the faster is the headline
    t_sprint = min(t_graph, t_eager) if graph_ok else t_eager
    timing = ("HIP graph replay of whole blocks" if graph_ok and t_graph <= t_eager
              else "eager launches (host-queued)")
    log(f"[bench] graph SPRINT block {t_graph * 1e3:.3f} ms, full-retention block "
        f"{t_full * 1e3:.3f} ms")
    del g_sprint, g_full, g_r1, blk_r1

    # ---------------------------------------------------------------- per-call GPU time
    reps = 20
    call_fns = {
        "lmhead_prefix": blk.prefix_confidence,
        "score": blk.score_prefix,
        "prune": blk.prune_prefix,
        "attend_full": lambda: blk.attend(False),
        "attend_pruned": lambda: blk.attend(True),
        "lmhead_block": blk.block_confidence,
        "unmask": lambda: blk.unmask(1),
    }
    calls = {}
    for name, fn in call_fns.items():
        blk.reset()
        g = capture(lambda: [fn() for _ in range(reps)])
        # 11 samples, each the mean launch time over one replay of 20 launches
        ts = [replay_rate(g, 1)[1] / reps * 1e6 for _ in range(11)]
        pc = pctl(ts)
        calls[name] = {"us": pc["median_us"], "min_us": min(ts), "p10_us": pc["p10_us"],
                       "p90_us": pc["p90_us"]}
        del g
    launches = {"lmhead_prefix": 1, "score": 1, "prune": 1, "attend_full": 1,
                "attend_pruned": n_steps, "lmhead_block": n_steps + 1, "unmask": n_steps + 1}
    launches_full = {"attend_full": n_steps + 1, "lmhead_block": n_steps + 1,
                     "unmask": n_steps + 1}

    # ---------------------------------------------------------------- fused step tail
    # The end of a step as one lmhead_confidence_unmask call (the block's
    # default) against lmhead_confidence + unmask_select, and a whole pruned
    # step each way: graph replays of 20 launches, bitwise the same state.
    step_tail = {}
    for fused in (True, False):
        blk.fused_tail = fused
        blk.reset()
        key = "fused" if fused else "two_calls"
        step_tail[key] = {"tail_us": round(call_us(torch, lambda: blk.confidence_and_unmask(1)), 3),
                          "pruned_step_us": round(call_us(torch, lambda: blk.pruned_step(1)), 3)}
    blk.fused_tail = True
    step_tail["note"] = ("tail = the block LM head and the unmasking step of one denoising "
                         "step; fused: one call, two launches (the block that merges a "
                         "sequence's last row runs its unmasking step)")

    # ---------------------------------------------------------------- library yardstick
    # The prefix GEMM's shape through torch.mm (hipBLASLt), for comparison
    # only: logits^T = W . hidden^T, written out in bf16, which the fused
    # kernel never does.  Eager launches, HIP events around 10 at a time.
    yardstick = None
    if wl.dtype == "bf16":
        hT = blk.hidden.t().contiguous()
        lg = torch.empty((wl.vocab, lay.total_L), dtype=blk.W.dtype, device="cuda")
        for _ in range(3):
            torch.mm(blk.W, hT, out=lg)
        ys = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                torch.mm(blk.W, hT, out=lg)
            e1.record()
            torch.cuda.synchronize()
            ys.append(e0.elapsed_time(e1) * 1e3 / 10)
        yus = pctl(ys)["median_us"]
        yfl = 2 * lay.total_L * wl.H * wl.vocab
        yardstick = {"op": "torch.mm(W [V,H], hidden^T [H,L]) -> logits^T [V,L], bf16",
                     "us": round(yus, 3), "tflops": round(yfl / yus / 1e6, 2),
                     "frac": round(yfl / yus / 1e6 / BF16_PEAK_TFLOPS, 4),
                     "note": "a library GEMM that writes the logits; not part of the path"}
        log(f"[bench] torch.mm on the prefix GEMM's shape: {yus:.1f} us "
            f"({yfl / yus / 1e6:.0f} TFLOP/s)")
        del hT, lg

    # ---------------------------------------------------------------- cold per-call timings
    # cold: before each call, read a 512 MB buffer (twice the Infinity Cache)
    # so the call's operands are not cached; a read leaves no dirty lines
    # whose write-back would be charged to the call
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    cold = EventTimer(torch)

    def cold_run(name, fn):
        for i in range(args.cold_iters):
            torch.sum(flush, dim=0, out=sink)
            with cold(name):
                fn()
    blk.reset()
    for name, fn in call_fns.items():
        cold_run(name, fn)
    torch.cuda.synchronize()
    calls_cold = cold.summary()
    del flush

    # ---------------------------------------------------------------- roofline
    work = work_model(blk)
    per_block = {k: calls[k]["us"] * launches[k] for k in calls}
    dominant = max(per_block, key=per_block.get)
    kernels = {}
    for name, st in calls.items():
        w = work[name]
        us = st["us"]
        ent = {"us": round(us, 3), "launches_per_block": launches[name],
               "us_per_block": round(us * launches[name], 2),
               "alg_bytes": w["bytes"], "alg_flops": w["flops"], "bound": w["bound"],
               "p10_us": round(st["p10_us"], 3), "p90_us": round(st["p90_us"], 3),
               "gbs": round(w["bytes"] / us / 1e3, 1),
               "tflops": round(w["flops"] / us / 1e6, 2)}
        # fraction of the roofline the call is bound by
        if w["bound"] == "mfma":
            ent["frac"] = round(w["flops"] / us / 1e6 /
                                (BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS), 4)
        else:
            ent["frac"] = round(w["bytes"] / us / 1e3 / HBM_PEAK_GBS, 4)
        if name in calls_cold:
            cu = calls_cold[name]["median_us"]
            ent["cold_us"] = round(cu, 3)
            ent["cold_p10_us"] = round(calls_cold[name]["p10_us"], 3)
            ent["cold_p90_us"] = round(calls_cold[name]["p90_us"], 3)
            ent["cold_gbs"] = round(w["bytes"] / cu / 1e3, 1)
        kernels[name] = ent
    dw = work[dominant]
    dus = calls[dominant]["us"]
    bf16 = wl.dtype == "bf16"
    if dw["bound"] == "mfma":
        achieved = dw["flops"] / dus / 1e6
        peak = BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS
        unit = "TFLOP/s"
    else:
        achieved = dw["bytes"] / dus / 1e3
        peak = HBM_PEAK_GBS
        unit = "GB/s"
    cus = calls_cold[dominant]["median_us"]
    cold_achieved = (dw["flops"] / cus / 1e6) if dw["bound"] == "mfma" else (dw["bytes"] / cus / 1e3)
    roofline = {"bound": dw["bound"], "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": load_traffic(dominant, wl.name),
                "kernel": dominant, "alg_per_launch": dw["flops"] if dw["bound"] == "mfma"
                else dw["bytes"], "mean_launch_us": round(dus, 3),
                "cold_launch_us": round(cus, 3), "cold_frac": round(cold_achieved / peak, 4)}

    att_pr = calls["attend_pruned"]["us"]
    att_full = calls["attend_full"]["us"]
    step_pr = att_pr + calls["lmhead_block"]["us"] + calls["unmask"]["us"]
    step_full = att_full + calls["lmhead_block"]["us"] + calls["unmask"]["us"]

    # ---------------------------------------------------------------- generation
    generation = None
    if args.gen_blocks > 0:
        generation = measure_generation(args, x, wl, n_steps, torch)
        log(f"[bench] generation of {args.gen_blocks} blocks: "
            f"{generation['sprint']['blocks_per_s']:.1f} blocks/s SPRINT, "
            f"{generation['full_prefix']['blocks_per_s']:.1f} blocks/s full prefix")

    # ---------------------------------------------------------------- several layers
    layers = None
    if args.layers > 0:
        layers = measure_layers(args, x, n_steps, torch)
        log(f"[bench] {args.layers} layers: block {layers['shared']['block_ms']:.3f} ms shared set "
            f"({layers['shared_carried_conf']['block_ms']:.3f} ms with carried confidences), "
            f"{layers['per_layer']['block_ms']:.3f} ms per-layer sets, "
            f"{layers['full_prefix']['block_ms']:.3f} ms full prefix")

    # ---------------------------------------------------------------- MoE FFN
    moe = None
    if args.moe_experts > 0 and bf16:
        moe = measure_moe(args, blk, x, wl, n_steps, torch)
        log(f"[bench] MoE FFN ({moe['config']}): {moe['us']:.1f} us, {moe['gbs']:.0f} GB/s over "
            f"{moe['distinct_experts']} chosen experts")

    # ---------------------------------------------------------------- second workload
    compare = None
    if args.compare and args.compare != wl.name:
        compare = measure_compare(args.compare, n_steps, torch)
        log(f"[bench] {args.compare}: block {compare['block_ms']['sprint']:.3f} ms SPRINT, "
            f"{compare['block_ms']['full_retention']:.3f} ms full retention; attention "
            f"{compare['attention_us']['pruned']:.1f} vs {compare['attention_us']['full']:.1f} us")

    # ---------------------------------------------------------------- planted confidences
    planted = None
    if not args.no_planted:
        planted = measure_planted(x, wl, n_steps, torch)
        log("[bench] planted confidences: " + ", ".join(
            f"f={c['fraction_planted']}: {c['adaptive_steps']} steps" for c in planted["cases"]))

    # ---------------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(x, wl, n_steps)
        log(f"[bench] oracle {cpu['value']:.3f} block-steps/s on {cpu['cores']} threads")

    value = steps_per_block / t_sprint
    rec = {
        "metric": "denoising block-steps/s (pruned vs full prefix), 1 MI355X",
        "value": round(value, 2),
        "unit": "block-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_sprint * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1) activations, lognormal key scales, N(0,0.02) LM head)",
        "config": {"workload": wl.name, "desc": wl.desc, "nseq": lay.nseq,
                   "prefix": int(lay.total_L), "kept": int(blk.total_kept), "block": wl.Lq,
                   "steps_per_block": n_steps + 1, "r_text": blk.r_text, "r_img": blk.r_img,
                   "tau": blk.tau, "step_unit": "one whole block (pass + pruned steps)"},
        "tokens_per_s": round(wl.Lq * lay.nseq / t_sprint, 1),
        "timing": timing,
        "eager": {"block_ms": round(t_eager * 1e3, 4),
                  "block_steps_per_s": round(steps_per_block / t_eager, 2)},
        "graph": {"block_ms": round(t_graph * 1e3, 4),
                  "block_steps_per_s": round(steps_per_block / t_graph, 2),
                  "replay_matches_eager": bool(graph_ok)},
        "full_retention": {"block_ms": round(t_full * 1e3, 4),
                           "block_steps_per_s": round(steps_per_block / t_full, 2)},
        "sprint_keep_all": {"block_ms": round(t_r1 * 1e3, 4),
                            "block_steps_per_s": round(steps_per_block / t_r1, 2),
                            "note": "r_text = r_img = 1: pruning-pass overhead only"},
        "pruning_pass_us": round(calls["lmhead_prefix"]["us"] + calls["score"]["us"] +
                                 calls["prune"]["us"], 2),
        "speedup_pruned_vs_full": {"attention_call": round(att_full / att_pr, 4),
                                   "denoising_step": round(step_full / step_pr, 4),
                                   "block": round(t_full / t_sprint, 4),
                                   "pages_claim_context": "up to 1.6x end to end (model, "
                                                          "hardware and workload not given)"},
        "generation": generation,
        "layers": layers,
        "moe": moe,
        "compare": compare,
        "planted_confidence": planted,
        "roofline": roofline,
        "kernels": kernels,
        "step_tail": step_tail,
        "yardstick": yardstick,
        "cpu_baseline": cpu,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
