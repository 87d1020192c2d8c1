#!/usr/bin/env python3
"""Decode-throughput benchmark of the SFI hot path on one MI355X.

One step is one decode step of every layer of the workload (the slow/fast schedule of the
seeded trajectory decides, per sequence, between dense attention + Selector + pack and the
two-segment fast attention).  Inputs (paged K/V of every layer, all queries, schedule
tables) are resident in HBM before the timed region; the timed region issues exactly
--steps steps on the engine's streams, bracketed by a device synchronisation.

Printed: one JSON line.  `value` is layer decode steps per second (steps x layers /
seconds).  `roofline` covers the dominant call, the fast-step attention: algorithmic bytes
(packed rows + recent window of K and V, q in, o out) over its average duration, from HIP
events recorded on the stream it runs on around every fast-step graph replay (all layers'
calls back to back; per call = replay time / layers), or around every n-th layer's call
when graphs are off.  `cpu_baseline` is the fp64 oracle on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def read_ceiling(gib: float) -> float:
    """GB/s (bytes read + bytes written) of a device-to-device copy of `gib` GiB, far larger
    than every cache: the practical HBM ceiling the roofline fraction can be set against."""
    import torch
    n = int(gib * 2 ** 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    gbs = reps * 2 * n * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return round(gbs, 1)


def _parse():
    from workload import BENCH_WORKLOAD
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed decode steps (default: the trajectory length)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default=BENCH_WORKLOAD)
    ap.add_argument("--dense-steps", type=int, default=64,
                    help="steps of the Full-KV dense baseline timed after the main run")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle CPU baseline sample (0 disables it)")
    ap.add_argument("--time-every", type=int, default=9,
                    help="bracket every n-th attention call issued call by call, and every "
                         "n-th fast-step graph replay, with HIP events (0: none)")
    ap.add_argument("--no-graphs", action="store_true",
                    help="issue fast steps call by call instead of replaying the captured "
                         "fast-step graph")
    ap.add_argument("--pace", choices=("auto", "on", "off"), default="auto",
                    help="host queues a Selector stream's wait only once stream 1 has reached "
                         "the attention it waits for (auto: on)")
    ap.add_argument("--sel-lookahead", type=int, default=None,
                    help="with pacing, queue layer i's Selector only after layer i's attention "
                         "has finished, with this many attention calls queued behind it (0: off; "
                         "default: 2 for stacks of more than two layers)")
    ap.add_argument("--sel-streams", type=int, default=2,
                    help="Selector streams (layers alternate between them)")
    ap.add_argument("--one-stream", action="store_true",
                    help="issue the Selector and pack on the attention stream")
    ap.add_argument("--repeats", type=int, default=20,
                    help="after the timed region, run the timed steps this many more times and "
                         "report the median, p10 and p90 of the time per step (0: skip)")
    ap.add_argument("--ceiling-gib", type=float, default=4.0,
                    help="size of the copy that measures the practical HBM ceiling (0: skip)")
    ap.add_argument("--evidence-window", type=int, default=None,
                    help="decode queries pooled into the Selector's evidence at a slow step "
                         "(default: the workload's, 1)")
    ap.add_argument("--lambda-clip", type=float, default=None,
                    help="adaptive fusion weight min(lambda_clip, H(f)/ln N) per (row, KV head) "
                         "instead of the workload's fixed lambda")
    ap.add_argument("--nms-greedy", action="store_true",
                    help="greedy soft-NMS in the Selector instead of the one-pass reading")
    ap.add_argument("--pack", choices=("auto", "full", "incremental"), default="auto",
                    help="full: re-pack every selected row at each slow step (sfi_pack); "
                         "incremental: copy only the newly selected ones (sfi_pack_update); "
                         "auto: the engine's choice (incremental for a stack of layers)")
    ap.add_argument("--device-control", action="store_true",
                    help="decide slow/fast and append K/V on the device every step (token "
                         "ids in, no host schedule); every step is replayed from a graph "
                         "unless --no-graphs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a device copy of known size (for counter calibration)")
    ap.add_argument("--traffic-json", default=None,
                    help="HBM traffic per fast call measured with counters (default: "
                         "profiles/fast_attn_traffic_<workload>.json); used only when its "
                         "workload and attention-kernel source hash match this run")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": 3}))


def cpu_baseline(w, d0, budget_s: float):
    """Oracle (fp64 NumPy) on layer 0, first steps of the trajectory, on the host cores."""
    import numpy as np
    from oracle import sfi_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    b = 0
    q = d0["q"][:, b].double().cpu().numpy()
    K = d0["K"][b].double().cpu().numpy()
    V = d0["V"][b].double().cpu().numpy()
    flags = d0["flags"][b].cpu().numpy()
    mode = O.schedule(flags[None, :], w.refresh_budget)[0]
    norms = O.key_norms(K)
    t0 = time.perf_counter()
    done = 0
    packed, rs = None, 0
    for s in range(w.steps):
        N = w.seq_len(s)
        if mode[s]:
            o, z, lse, p = O.attention(q[s], K[:, :N], V[:, :N])
            sel = O.select(p, norms[:, :N], N, w.num_kv_heads, w.n_sink, w.n_recent, w.top_k,
                           w.nms_radius, w.alpha_soft, w.alpha_cross, w.lam)
            packed = [O.packed_positions(sel.sel[g], w.n_sink) for g in range(w.num_kv_heads)]
            rs = O.recent_start_at(N, w.n_sink, w.n_recent)
        else:
            O.fast_attention(q[s], K, V, packed, rs, N)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    n_slow = int(mode[:done].sum())
    # One layer decode step serves every row of the batch; the sample ran row 0 only, so a
    # whole step costs batch times the sample's time per step (the unit of `value`).
    rows = f"row 0 of {w.batch} (time per step scaled by {w.batch})" if w.batch > 1 else "row 0"
    return {"value": done / (w.batch * dt), "unit": "layer decode steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"layer 0, {rows}, trajectory steps 0..{done - 1} ({n_slow} slow, "
                      f"{done - n_slow} fast) in {dt:.1f} s, fp64 NumPy"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(sequences shard across GPUs with no exchange, see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    from workload import get
    from workload.gen import make_layer
    from sparse_kv_attention_decode_amd.engine import Engine

    w = get(args.workload)
    inc = {"auto": None, "full": False, "incremental": True}[args.pack]
    pace = {"auto": None, "on": True, "off": False}[args.pace]
    if args.evidence_window is not None:
        w = w.replace(evidence_window=args.evidence_window)
    if args.lambda_clip is not None:
        w = w.replace(lambda_clip=args.lambda_clip)
    if args.nms_greedy:
        w = w.replace(nms_greedy=True)
    steps = args.steps if args.steps is not None else w.steps
    t_setup = time.perf_counter()
    d0 = None
    eng = None
    for layer in range(w.layers):
        keep = layer == 0 and args.cpu_seconds > 0
        d = make_layer(w, layer, device="cuda", keep_logical=keep)
        if eng is None:
            if args.device_control:
                from workload.gen import BOUNDARY_TOKENS, gen_tokens
                eng = Engine(w, d["flags"], two_streams=not args.one_stream,
                             sel_streams=args.sel_streams,
                             device_control=True, tokens=gen_tokens(w, d["flags"]),
                             boundary_tokens=BOUNDARY_TOKENS, incremental_pack=inc)
            else:
                eng = Engine(w, d["flags"], two_streams=False if args.one_stream else None,
                             sel_streams=args.sel_streams,
                             incremental_pack=inc, paced=pace,
                             sel_lookahead=args.sel_lookahead)
        eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
        if keep:
            d0 = {k: d[k] for k in ("q", "K", "V", "flags")}
        del d
        if layer % 6 == 5 or layer == w.layers - 1:
            print(f"[bench] layer {layer + 1}/{w.layers} resident "
                  f"({time.perf_counter() - t_setup:.1f} s)", file=sys.stderr, flush=True)
    if not args.no_graphs:
        if args.device_control:
            eng.enable_device_graphs()
        else:
            eng.enable_graphs()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    S = w.steps

    # warm-up: the first steps of the trajectory
    for k in range(args.warmup):
        eng.step(k % S)
    eng.join()
    torch.cuda.synchronize()

    # timed region: exactly `steps` decode steps of every layer; every event it records is
    # created beforehand (at most two sampled calls per layer and step, plus graph replays)
    timer = []
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    if args.time_every > 0:
        eng.reserve_timing_events(steps * (2 * w.layers + 1) // args.time_every + 16)
    torch.cuda.synchronize()
    for k in range(steps):
        step_ev[k].record(eng.stream1)
        if args.time_every > 0:
            eng.step(k % S, timer=timer, time_every=args.time_every)
        else:
            eng.step(k % S)
    eng.join()
    step_ev[steps].record(eng.stream1)
    torch.cuda.synchronize()
    total_ms = step_ev[0].elapsed_time(step_ev[steps])

    step_ms = [step_ev[k].elapsed_time(step_ev[k + 1]) for k in range(steps)]
    slow_step = [bool(eng.plan.mode[:, k % S].any()) for k in range(steps)]
    fast_ms = [t for t, sl in zip(step_ms, slow_step) if not sl]
    slow_ms = [t for t, sl in zip(step_ms, slow_step) if sl]
    # A fast step right after a slow step first waits for that step's Selector and pack (on
    # their own streams); steady fast steps follow a fast step and carry no such tail.
    steady_ms = [t for k, (t, sl) in enumerate(zip(step_ms, slow_step))
                 if not sl and k > 0 and not slow_step[k - 1]]

    def agg(kind):
        ts = [(e0.elapsed_time(e1), nb, nc) for kd, e0, e1, nb, nc in timer if kd == kind]
        if not ts:
            return None
        tot_ms = sum(t for t, _, _ in ts)
        tot_b = sum(b for _, b, _ in ts)
        calls = sum(c for _, _, c in ts)
        return {"calls": calls, "avg_us": 1e3 * tot_ms / calls,
                "gbs": tot_b / (tot_ms * 1e-3) / 1e9, "avg_bytes": tot_b / calls}

    fast = agg("fast")
    slow = agg("slow")

    # Full-KV dense baseline: dense attention of every layer, no Selector
    # spread: the same steps again, several times (after the timed region, not part of it)
    rep_ms = []
    for _ in range(max(0, args.repeats)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(eng.stream1)
        for k in range(steps):
            eng.step(k % S)
        eng.join()
        e1.record(eng.stream1)
        torch.cuda.synchronize()
        rep_ms.append(e0.elapsed_time(e1) / steps)
    repeats = None
    if rep_ms:
        import numpy as np
        q = np.percentile(rep_ms, [10, 50, 90])
        repeats = {"n": len(rep_ms), "ms_per_step_p10": round(float(q[0]), 4),
                   "ms_per_step_median": round(float(q[1]), 4),
                   "ms_per_step_p90": round(float(q[2]), 4),
                   "value_median": round(steps * w.layers / (float(q[1]) * steps * 1e-3), 2)}

    dense = None
    if args.dense_steps > 0:
        # timed like the steps above: one event at each step boundary, created beforehand
        dense_timer = []
        dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.dense_steps + 1)]
        torch.cuda.synchronize()
        for k in range(args.dense_steps):
            dev_ev[k].record(eng.stream1)
            eng.step(k % S, dense_only=True, timer=dense_timer,
                     time_every=max(1, args.time_every))
        dev_ev[args.dense_steps].record(eng.stream1)
        torch.cuda.synchronize()
        dms = [dev_ev[k].elapsed_time(dev_ev[k + 1]) for k in range(args.dense_steps)]
        dk = [(e0.elapsed_time(e1), nb) for _, e0, e1, nb, _ in dense_timer]
        dense = {"step_ms": sum(dms) / len(dms),
                 "gbs": (sum(b for _, b in dk) / (sum(t for t, _ in dk) * 1e-3) / 1e9)
                 if dk else None}

    ceiling = read_ceiling(args.ceiling_gib) if args.ceiling_gib > 0 else None
    ms_per_step = total_ms / steps
    value = steps * w.layers / (total_ms * 1e-3)
    traffic = None
    if args.traffic_json is None:
        args.traffic_json = os.path.join(ROOT, "profiles", f"fast_attn_traffic_{w.name}.json")
    if os.path.exists(args.traffic_json):
        try:
            import hashlib
            tj = json.load(open(args.traffic_json))
            pkg = os.path.join(ROOT, "sparse_kv_attention_decode_amd")
            h = hashlib.sha256()
            for f in (os.path.join(pkg, "csrc", "sfi_attn.hip"), os.path.join(pkg, "build.py")):
                h.update(open(f, "rb").read())
            digest = h.hexdigest()
            # counters taken on another kernel (source or build flags) or workload do not
            # describe this run
            if tj.get("workload") == w.name and tj.get("kernel_source_sha256") == digest:
                traffic = tj.get("bytes_per_call")
        except (OSError, ValueError):
            traffic = None
    # pacing acts on host-scheduled steps with separate Selector streams only
    one_stream = eng.sel_streams[0] is eng.stream1
    paced_on = bool(eng.paced) and not args.device_control and not one_stream
    roof = None
    if fast:
        roof = {"bound": "hbm", "achieved": round(fast["gbs"], 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(fast["gbs"] / PEAK_HBM_GBS, 4),
                "traffic": traffic, "kernel": "sfi_fast_attn (fast-step two-segment attention)",
                "avg_call_us": round(fast["avg_us"], 2),
                "algorithmic_bytes_per_call": int(fast["avg_bytes"])}
    cpu = None
    if args.cpu_seconds > 0 and d0 is not None:
        cpu = cpu_baseline(w, d0, args.cpu_seconds)

    mean = lambda xs: (sum(xs) / len(xs)) if xs else None  # noqa: E731
    line = {
        "metric": "SFI decode steps/s per layer at 8K–128K ctx; achieved HBM GB/s vs peak",
        "value": round(value, 2),
        "unit": "layer decode steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded span-drift generator)",
        "config": {"workload": w.name, "layers": w.layers, "batch": w.batch,
                   "context": w.context, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "top_k": w.top_k, "n_recent": w.n_recent,
                   "streams": 1 if one_stream else 1 + len(eng.sel_streams),
                   "fast_step_graph": eng.graph is not None,
                   "evidence_window": w.evidence_window,
                   "lambda_clip": w.lambda_clip if w.lambda_clip >= 0 else None,
                   "nms_greedy": bool(w.nms_greedy),
                   "device_control": bool(args.device_control),
                   "pack": "incremental" if eng.incremental_pack else "full",
                   "paced": paced_on,
                   "sel_lookahead": int(eng.sel_lookahead or 0) if paced_on else 0},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": {
            "stack_steps_per_s": round(steps / (total_ms * 1e-3), 3),
            "fast_step_ms": mean(fast_ms), "slow_step_ms": mean(slow_ms),
            "steady_fast_step_ms": mean(steady_ms),
            "n_fast_steps": len(fast_ms), "n_slow_steps": len(slow_ms),
            "n_steady_fast_steps": len(steady_ms),
            "fast_attn": fast, "slow_attn": slow,
            "dense_step_ms": dense["step_ms"] if dense else None,
            "dense_attn_gbs": dense["gbs"] if dense else None,
            "fast_vs_dense": (dense["step_ms"] / mean(fast_ms)) if dense and fast_ms else None,
            "steady_fast_vs_dense": (dense["step_ms"] / mean(steady_ms))
            if dense and steady_ms else None,
            "mixed_vs_dense": (dense["step_ms"] / ms_per_step) if dense else None,
            "setup_s": round(setup_s, 1),
            "repeats": repeats,
            "copy_ceiling_gbs": ceiling,
            "fast_call_frac_of_copy_ceiling": (round(fast["gbs"] / ceiling, 4)
                                               if fast and ceiling else None),
            # K/V of one step fit in the 256 MiB Infinity Cache: repeated steps may be served
            # from it rather than from HBM
            "cache_resident": eng.dense_bytes(0, range(w.batch)) < 256 * 2 ** 20,
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
