"""Throughput of the tree-verify step on one MI355X.

A step is one pass of the whole path over one batch: ancestor mask -> tree-masked
split-KV attention -> vocab argmax + longest-path acceptance -> KV commit, four C-ABI
calls back to back on one stream, inputs resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload long32k] [--splits S]

value = verified tree tokens/s = B*T / seconds per step.  The roofline object covers
the attention call, timed with HIP events on the stream it runs on, against the HBM (or
matrix-core) peak and against a plain device copy timed in the same process;
cpu_baseline times the oracle on whole sequences of the same workload.  Also reported:
each stage on its own, per-stage latencies of the three small workloads (and a chain
verified at once vs node by node), and the batched 8K workload's attention call.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified tree tokens/s + tree-verify attention HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_traffic(inp, depth):
    """Algorithmic bytes and flops of one attention call (what the method must move)."""
    import numpy as np
    w = inp.w
    e = 2 if w.dtype == "bf16" else 4
    P = inp.prefix_len.cpu().numpy().astype(np.int64)
    kv_prefix = int(P.sum()) * w.Hkv * w.D * e * 2
    kv_tree = w.B * w.Hkv * w.T * w.D * e * 2
    q = w.B * w.Hq * w.T * w.D * e
    o = w.B * w.T * w.Hq * w.D * 4
    anc = depth.cpu().numpy().astype(np.int64) + 1            # [B, T] keys from the tree
    keys = (P[:, None] + anc).sum() * w.Hq                      # sum over (b, h, i)
    flops = 4 * w.D * int(keys)
    return kv_prefix + kv_tree + q + o, flops


def _oracle_sequence(orc, O, inp, b, heads, threads):
    """One sequence of a workload through the oracle (mask, attention for the first `heads`
    q heads and every node, accept, commit); returns the seconds of each stage."""
    import numpy as np
    from _support import to_np

    w = inp.w
    _, Hkv, bs, D = inp.k_pool.shape
    nblk = int((inp.block_table[b] >= 0).sum())
    blocks = inp.block_table[b, :nblk].long()
    cache = O.Cache(k=to_np(inp.k_pool.index_select(0, blocks)),
                    v=to_np(inp.v_pool.index_select(0, blocks)),
                    table=np.arange(nblk, dtype=np.int32)[None], block_size=bs,
                    block_stride=Hkv * bs * D, head_stride=bs * D, row_stride=D,
                    num_blocks=nblk, dtype=O.BF16 if w.dtype == "bf16" else O.F32)
    parents = to_np(inp.parents[b:b + 1])
    q, kt, vt = to_np(inp.q[b:b + 1]), to_np(inp.k_tree[b:b + 1]), to_np(inp.v_tree[b:b + 1])
    P = to_np(inp.prefix_len[b:b + 1])
    logits, draft = to_np(inp.logits[b:b + 1]), to_np(inp.draft[b:b + 1])
    rows = np.array([[0, h, i] for h in range(heads) for i in range(w.T)], dtype=np.int32)
    t = {}
    t0 = time.perf_counter()
    mask, _, err = orc.build_tree_mask(parents)
    t["mask"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.tree_verify_attention(q, kt, vt, cache, P, int(P.max()), mask, inp.scale, rows=rows,
                              nthreads=threads)
    t["attention"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    _, L, nodes, _ = orc.accept_longest_path(logits, draft, parents, err)
    t["accept"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.kv_commit(kt, vt, L, nodes, err, cache, P, int(P.max()))
    t["commit"] = time.perf_counter() - t0
    return t


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, seed, budget_s=15.0):
    """The oracle on whole sequences of the workload, one after another, until the time
    budget is spent: mask, attention for every head and node, accept, commit.  Then, with
    one thread, one step of each small workload."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle as O
    from tree_masked_verify_amd import workloads as wl

    w = inp.w
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    orc = O.Oracle()
    done, heads_used = 0, w.Hq
    stages = {"mask": 0.0, "attention": 0.0, "accept": 0.0, "commit": 0.0}
    for b in range(w.B):
        heads = heads_used
        if b == 0:
            # a sequence too large for the budget is sampled by heads (scaled to all heads)
            t_head = _oracle_sequence(orc, O, inp, 0, 1, threads)["attention"]
            heads = heads_used = max(1, min(w.Hq, int(budget_s / max(t_head, 1e-9))))
        t = _oracle_sequence(orc, O, inp, b, heads, threads)
        t["attention"] *= w.Hq / heads                 # that sequence's full step
        for k in stages:
            stages[k] += t[k]
        done += 1
        if heads < w.Hq or sum(stages.values()) >= budget_s:
            break
    spent = sum(stages.values())
    t_step = spent / done * w.B
    # one thread, one whole step of each small workload
    single = {}
    for name in ("tiny", "parity512", "chain2k"):
        sw = wl.WORKLOADS[name]
        sinp = wl.make_inputs(sw, seed=seed, device="cpu")
        tot = {"mask": 0.0, "attention": 0.0, "accept": 0.0, "commit": 0.0}
        for b in range(sw.B):
            for k, v in _oracle_sequence(orc, O, sinp, b, sw.Hq, 1).items():
                tot[k] += v
        single[name] = {k: round(v * 1e3, 3) for k, v in tot.items()}
    return {"value": w.B * w.T / t_step, "unit": "verified tree tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"sequences 0..{done - 1} of {w.B} in full (mask, attention for "
                      f"{heads_used} of {w.Hq} q heads x {w.T} nodes"
                      f"{' scaled to all heads' if heads_used < w.Hq else ''}, accept over "
                      f"{w.V} logits, commit); step time = {w.B} x the mean sequence; "
                      f"{spent:.1f} s of oracle time",
            "stage_s_per_step": {k: round(v / done * w.B, 3) for k, v in stages.items()},
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "single_thread_small_configs_ms": single}


def counter_traffic(workload):
    """HBM bytes per attention call from the committed rocprofv3 counter summary of this
    workload, or None when the kernel sources have changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attention_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for name in fields.get("sources", "").split():
        path = os.path.join(ROOT, "tree_masked_verify_amd", "csrc", name)
        if not os.path.exists(path):
            return None
        with open(path, "rb") as f:
            h.update(f.read())
    if not fields.get("sources") or h.hexdigest() != fields.get("sources_sha256"):
        return None
    return int(fields["hbm_bytes_per_call"])


def _smi_sample():
    """(socket power W, graphics clock MHz) from one `amd-smi metric -p -c` reading, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True,
                           text=True, timeout=10)
        d = json.loads(r.stdout)
    except Exception:
        return None
    d = d[0] if isinstance(d, list) else d
    if isinstance(d, dict) and "gpu_data" in d:
        d = d["gpu_data"][0]

    def val(x):
        x = x.get("value") if isinstance(x, dict) else x
        try:
            return float(x)
        except (TypeError, ValueError):
            return None
    clk = d.get("clock", {})
    gfx = clk.get("gfx_0", clk.get("gfx", {}))
    return val(d.get("power", {}).get("socket_power")), val(gfx.get("clk") if isinstance(gfx, dict) else gfx)


def power_probe(st, seconds):
    """The attention call back to back for `seconds` while amd-smi samples the board's socket
    power and graphics clock (the first second of samples is dropped as ramp-up)."""
    import statistics
    import threading
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        t0 = time.time()
        while not stop.is_set():
            v = _smi_sample()
            if v is not None and time.time() - t0 > 1.0:
                samples.append(v)
            time.sleep(0.25)
    th = threading.Thread(target=sampler)
    th.start()
    t0, n = time.time(), 0
    while time.time() - t0 < seconds:
        for _ in range(50):
            st.attention()
        torch.cuda.synchronize()
        n += 50
    dt = time.time() - t0
    stop.set()
    th.join()
    pw = [p for p, _ in samples if p is not None]
    ck = [c for _, c in samples if c is not None]
    return {"attention_us": round(dt / n * 1e6, 1), "calls": n, "samples": len(samples),
            "socket_power_w_median": statistics.median(pw) if pw else None,
            "socket_power_w_max": max(pw) if pw else None,
            "gfx_clock_mhz_median": statistics.median(ck) if ck else None}


def settle_clock(st, ms):
    """Whole steps, back to back, until `ms` milliseconds have passed.  From idle the
    board's graphics clock first runs high and then throttles to the 1400 W power limit
    over the first ~10-30 ms of load (a call then takes up to 40% longer than settled);
    the warmup and timed steps that follow run at the settled clock a serving loop runs
    at."""
    import torch
    if ms <= 0:
        return 0
    t0, n = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            st.run()
        torch.cuda.synchronize()
        n += 10
    return n


def copy_bandwidth(dev, mib=2048, reps=10):
    """Achievable HBM bandwidth in this process: a plain device-to-device copy of `mib`
    MiB (torch copy_, HIP events on its stream), read + write bytes over the median
    duration."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del src, dst
    return round(2 * n / (sorted(ts)[reps // 2] * 1e-3) / 1e9, 1)


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def small_config_latency(dev, seed, reps=21):
    """Per-stage device latency (us) of the three small workloads.  Cold: median of reps
    with a 512 MiB write before each, so that every rep starts with nothing of its inputs
    in the 256 MB MALL (nor their pages in the address-translation caches).  Warm: the
    mean of reps back to back, queued behind a spin kernel so that host launch gaps do
    not count.  At the 2K chain also one 8-node chain verify against 8 single-node
    verifies with a commit after each (the chain's nodes verified one by one)."""
    import torch
    from tree_masked_verify_amd import workloads as wl
    from tree_masked_verify_amd.step import VerifyStep
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def warm(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(reps * 60_000)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) * 1000.0 / reps, 2)

    def timed(fn):
        ts = []
        for r in range(reps):
            flush.fill_(r & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1000.0)
        return round(_median(ts), 2)

    out = {}
    for name in ("tiny", "parity512", "chain2k"):
        w = wl.WORKLOADS[name]
        inp = wl.make_inputs(w, seed=seed, device=dev)
        st = VerifyStep.from_inputs(inp)
        for _ in range(3):
            st.run()
        torch.cuda.synchronize()
        calls = (("mask", st.build_mask), ("attention", st.attention), ("accept", st.accept),
                 ("commit", st.commit), ("step", st.run))
        res = {stage: timed(fn) for stage, fn in calls}
        res["warm"] = {stage: warm(fn) for stage, fn in calls}
        res["tree_tokens_per_s"] = round(w.B * w.T / (res["step"] * 1e-6), 1)
        res["tree_tokens_per_s_warm"] = round(w.B * w.T / (res["warm"]["step"] * 1e-6), 1)
        out[name] = res
        if name == "chain2k":
            # the same chain node by node: tree = 1 verify + commit, prefix advanced each time
            kp, vp = inp.k_pool.clone(), inp.v_pool.clone()
            P0 = inp.prefix_len.clone()
            prefix = inp.prefix_len.clone()
            one = []
            for i in range(w.T):
                sl = lambda t: t[:, :, i:i + 1].contiguous()
                one.append(VerifyStep(sl(inp.q), sl(inp.k_tree), sl(inp.v_tree), kp, vp,
                                      inp.block_table, prefix, int(inp.max_prefix_len) + i,
                                      torch.full((1, 1), -1, dtype=torch.int32, device=dev),
                                      inp.logits[:, i:i + 1].contiguous(),
                                      inp.draft[:, i:i + 1].contiguous(), inp.scale,
                                      new_prefix_len=prefix))

            def serial():
                for o in one:
                    o.run()
            def serial_from_start():
                prefix.copy_(P0)
                serial()
            serial_from_start()
            ts = []
            for r in range(reps):
                prefix.copy_(P0)
                flush.fill_(r & 0xFF)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                serial()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1000.0)
            res["serial_single_node_steps_us"] = round(_median(ts), 2)
            res["serial_over_chain"] = round(res["serial_single_node_steps_us"] / res["step"], 2)
            res["warm"]["serial_single_node_steps"] = warm(serial_from_start)
            res["warm"]["serial_over_chain"] = round(
                res["warm"]["serial_single_node_steps"] / res["warm"]["step"], 2)
    del flush
    return out


def secondary_workload(name, dev, seed, steps=30, warmup=10):
    """The attention call and whole step of another workload, timed like the main one
    (HIP events on the stream; clock settled first)."""
    import torch
    from tree_masked_verify_amd import workloads as wl
    from tree_masked_verify_amd.step import VerifyStep
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, seed=seed, device=dev)
    st = VerifyStep.from_inputs(inp)
    stream = torch.cuda.current_stream()
    settle_clock(st, 100)
    for _ in range(warmup):
        st.run()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ea = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    e[0].record(stream)
    for k in range(steps):
        st.build_mask()
        ea[k][0].record(stream)
        st.attention()
        ea[k][1].record(stream)
        st.accept()
        st.commit()
    e[1].record(stream)
    torch.cuda.synchronize()
    ms_step = e[0].elapsed_time(e[1]) / steps
    us_attn = sum(a.elapsed_time(b) for a, b in ea) / steps * 1000.0
    nbytes, flops = attention_traffic(inp, st.depth)
    return {"workload": name, "ms_per_step": round(ms_step, 4),
            "verified_tree_tokens_per_s": round(w.B * w.T / (ms_step * 1e-3), 1),
            "attention_us_per_launch": round(us_attn, 2),
            "attention_bytes_per_launch": nbytes, "attention_flops_per_launch": flops,
            "attention_hbm_gbs": round(nbytes / us_attn / 1e3, 1),
            "attention_mfma_tflops": round(flops / us_attn / 1e6, 1),
            "attention_mfma_frac": round(flops / us_attn / 1e6 / BF16_PEAK_TFLOPS, 4),
            "attention_traffic": counter_traffic(name)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="whole steps back to back for this long before the warmup, so that "
                         "the board's clock has settled at its power limit (0: none)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the same-run copy bandwidth, the small workloads' latencies "
                         "and the batched 8K workload")
    ap.add_argument("--workload", default="long32k")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="only loop the attention call this long while sampling board power "
                         "and graphics clock with amd-smi; prints one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of this many MiB --steps "
                         "times (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verify path has no multi-GPU code)", file=sys.stderr)
        sys.exit(2)

    import torch
    from tree_masked_verify_amd import workloads as wl
    from tree_masked_verify_amd.step import VerifyStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": args.steps}), flush=True)
        return
    w = wl.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name} inputs (seed {args.seed})")
    inp = wl.make_inputs(w, seed=args.seed, device=dev)
    st = VerifyStep.from_inputs(inp, num_splits=args.splits)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    if args.power > 0:
        st.build_mask()
        for _ in range(3):
            st.attention()
        torch.cuda.synchronize()
        log(f"[bench] power probe, {args.power} s of attention calls")
        print(json.dumps({"workload": w.name, **power_probe(st, args.power)}), flush=True)
        return
    settled = settle_clock(st, args.settle_ms)
    log(f"[bench] settled the clock with {settled} steps; warmup {args.warmup}")
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ea = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for k in range(args.steps):
        st.build_mask()
        ea[k][0].record(stream)
        st.attention()
        ea[k][1].record(stream)
        st.accept()
        st.commit()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms_step = ev[0].elapsed_time(ev[1]) / args.steps
    ms_attn = sum(a.elapsed_time(b) for a, b in ea) / args.steps

    # the write-before-accept variant of the same step, timed the same way: the tree rows
    # go into the cache first, the attention reads them there, the accepted path is
    # compacted instead of committed
    log(f"[bench] timing {args.steps} write-before-accept steps")
    for _ in range(2):
        st.run_in_cache()
    torch.cuda.synchronize()
    ev[0].record(stream)
    for k in range(args.steps):
        st.run_in_cache()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms_step_in_cache = ev[0].elapsed_time(ev[1]) / args.steps

    # per-stage split (separate pass, one call type at a time); the sampled acceptance
    # (the alternative to the greedy accept stage) is timed here as well
    ua, us = wl.make_uniforms(w.B, w.T, args.seed)
    ua, us = torch.from_numpy(ua).to(dev), torch.from_numpy(us).to(dev)
    # and the tree-position rotary embedding (in place on Q and the tree keys; last, so
    # that the other stages are timed on the unrotated inputs)
    from tree_masked_verify_amd import sv_rope_tree
    # and the builder of the next draft tree (top-K of each drafter row, best-first
    # expansion) on synthetic drafter logits of this batch and tree size
    from tree_masked_verify_amd import (sv_draft_tree, sv_draft_tree_workspace_size,
                                        workspace)
    d_k, d_levels = (w.topk or 8), (w.max_levels or w.T)
    d_logits, d_roots = wl.make_drafter_inputs(w, seed=args.seed, device=dev)
    d_par = torch.empty((w.B, w.T), dtype=torch.int32, device=dev)
    d_tok = torch.empty((w.B, w.T), dtype=torch.int32, device=dev)
    d_cum = torch.empty((w.B, w.T), dtype=torch.float64, device=dev)
    d_ws = workspace(sv_draft_tree_workspace_size(w.B, w.T, d_k), dev)
    stages = {}
    for name, fn in (("mask", st.build_mask), ("attention", st.attention),
                     ("accept", st.accept), ("commit", st.commit),
                     ("accept_sampled", lambda: st.accept_sampled(ua, us, w.temperature)),
                     ("draft_tree", lambda: sv_draft_tree(d_logits, d_roots, d_k, d_levels,
                                                          d_par, d_tok, d_cum, d_ws)),
                     # the write-before-accept variant (tree rows into the cache first,
                     # attention reading them there, compaction instead of the commit)
                     ("append", st.append), ("attention_in_cache", st.attention_in_cache),
                     ("compact", st.compact),
                     ("rope", lambda: sv_rope_tree(st.q, st.k_tree, st.prefix_len, st.depth,
                                                   1e4))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # a spin kernel first keeps the GPU busy while the host queues the calls, so that
        # short stages are timed back to back on the GPU, not at the host's launch rate
        torch.cuda._sleep(args.steps * 120_000)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        stages[name] = round(e0.elapsed_time(e1) / args.steps * 1000.0, 2)

    bytes_attn, flops_attn = attention_traffic(inp, st.depth)
    gbs = bytes_attn / (ms_attn * 1e-3) / 1e9
    tflops = flops_attn / (ms_attn * 1e-3) / 1e12
    # the bound is the side the call's arithmetic intensity puts it on: matrix cores when
    # its flops per algorithmic byte exceed the ratio of the two peaks (2500e12 / 8000e9)
    mfma_bound = flops_attn / bytes_attn > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if w.dtype != "bf16":
        kernel = f"attn_valu_kernel<{w.D}> (chunks merged in the kernel)"
    elif w.D in (128, 256):
        kernel = (f"attn_w4_kernel<{w.D}> (chunks merged in the kernel when the grid fills the "
                  "chip, else by attn_reduce_kernel)")
    else:
        kernel = f"attn_mfma_kernel<{w.D}> + attn_reduce_kernel"
    roofline = {"bound": "mfma" if mfma_bound else "hbm",
                "kernel": kernel,
                "achieved": round(tflops, 1) if mfma_bound else round(gbs, 1),
                "peak": BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
                "unit": "TFLOP/s" if mfma_bound else "GB/s",
                "frac": round(tflops / BF16_PEAK_TFLOPS if mfma_bound else gbs / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic(w.name),
                "bytes_per_launch": bytes_attn, "flops_per_launch": flops_attn,
                "us_per_launch": round(ms_attn * 1e3, 2),
                "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "mfma_tflops": round(tflops, 1),
                "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    bytes_argmax = w.B * w.T * w.V * 4
    tokens = w.B * w.T
    result = {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "verified tree tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "prefix": list(w.prefix), "tree_nodes": w.T,
                   "tree": w.tree, "vocab": w.V, "paged_block": w.block_size,
                   "num_splits": args.splits, "seed": args.seed,
                   "sampled_temperature": w.temperature, "draft_topk": d_k,
                   "draft_levels": d_levels},
        "roofline": roofline,
        "stages_us": stages,
        "accepted_tokens_per_step": int(st.accepted_len.sum()),
        "argmax_gbs": round(bytes_argmax / (stages["accept"] * 1e-6) / 1e9, 1),
        # KV commit: the accepted rows of K and V read from the tree buffers and written to
        # the cache (a few hundred KB per call: latency-bound, not a bandwidth figure)
        "commit_gbs": round(2 * 2 * int(st.accepted_len.sum()) * w.Hkv * w.D
                            * (2 if w.dtype == "bf16" else 4) / (stages["commit"] * 1e-6) / 1e9, 1),
        # sampled acceptance: one read of every logit row (the walk and the draw touch a
        # few more bytes per sequence, not counted)
        "accept_sampled_gbs": round(bytes_argmax / (stages["accept_sampled"] * 1e-6) / 1e9, 1),
        # the whole step with the write-before-accept cache update (append, attention over
        # the cache-resident tree, compaction) instead of delayed write-through
        "ms_per_step_write_before_accept": round(ms_step_in_cache, 4),
        # its append: every tree row of K and V read from the tree buffers and written to
        # the cache
        "append_gbs": round(2 * 2 * w.B * w.Hkv * w.T * w.D * (2 if w.dtype == "bf16" else 4)
                            / (stages["append"] * 1e-6) / 1e9, 1),
        # draft tree: one read of the drafter rows that can be expanded (all but the last)
        "draft_tree_gbs": round(w.B * (w.T - 1) * w.V * 4 / (stages["draft_tree"] * 1e-6) / 1e9,
                                1),
        # rotary embedding: Q and tree keys read and written once
        "rope_gbs": round(2 * w.B * (w.Hq + w.Hkv) * w.T * w.D * (2 if w.dtype == "bf16" else 4)
                          / (stages["rope"] * 1e-6) / 1e9, 1),
    }
    result["settle_ms"] = args.settle_ms
    if not args.no_extras:
        log("[bench] copy bandwidth")
        cbw = copy_bandwidth(dev)
        roofline["copy_gbs"] = cbw
        roofline["frac_of_copy"] = round(gbs / cbw, 4)
        log("[bench] small workloads")
        result["small_configs_latency_us"] = small_config_latency(dev, args.seed)
        if w.name != "batched8k":
            log("[bench] batched8k")
            result["batched8k"] = secondary_workload("batched8k", dev, args.seed)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(inp, args.seed)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
