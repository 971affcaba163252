"""Benchmark of the TriAttention prune step on one MI355X.

One step = one tria_prune call (tria_score, tria_select_topB and tria_compact in sequence) over
every stream of the workload (score every cached key, z-score per query head, GQA max, top-B,
in-place compaction of K, V and positions); --entry separate makes the three calls itself.  Default workload: Qwen3-32B shapes, 64 layers x 8 sequences x 8 KV heads
(4096 streams), 32768 bf16 keys per stream compressed to B = 3072.

Before every step, outside the timed region, K, V and positions are restored from a pristine
device copy and 1 GiB of scratch is written to evict the 256 MB Infinity Cache and the L2, so
each step reads a cold, unpruned cache.  Each step is timed with HIP events on the stream the
kernels run on, enqueued while the restore and flush still run, so that its time is the device's
(the host's enqueue time of the call is reported apart, host_enqueue_us); the library's own HIP
events around each kernel give the per-kernel times and the dominant kernel's duration for the
roofline.

Prints one JSON line (see the keys below).  --gpus above 1 is refused: this path runs on one GPU.

--workload decode measures the decode loop on config 4 (Qwen3-8B shapes, 36 layers x 64
sequences x 8 KV heads, B = 2048; --config 3: one sequence, B = 3072): one step appends the K/V
rows of 128 new tokens to every stream and prunes the full cache (B + 128 rows) back to B
(tria_decode_step).

--workload calib measures instead the calibration-statistics kernel (tria_calib_stats) on the
offline capture it would see for Qwen3-32B: 64 layers x 64 query heads x 10240 captured pre-RoPE
queries in bf16 (about ten thousand calibration tokens), one launch per step.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def measured_traffic(workload: str) -> dict:
    """HBM bytes per launch of each kernel as measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy of known size), from the table in profiles/hbm_traffic.md.
    A row counts only for the workload it was measured on and while the source files the kernel
    was built from are unchanged (their SHA-256 digests are in the row, joined by '+'); otherwise
    the figure is stale and is reported as null."""
    import hashlib

    out = {}
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return out
    for line in lines:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) < 6 or cells[0] != "traffic" or cells[1] != workload:
            continue
        name, nbytes, srcs, shas = cells[2], cells[3], cells[4].split("+"), cells[5].split("+")
        try:
            cur = []
            for src in srcs:
                with open(os.path.join(ROOT, src.strip()), "rb") as fh:
                    cur.append(hashlib.sha256(fh.read()).hexdigest())
        except OSError:
            continue
        if cur == [x.strip() for x in shas]:
            out[name] = int(float(nbytes))
    return out


VARIANTS = ("default", "per_key_phase", "pre_rope", "weight_r", "offset_max")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=None,
                    help="workload id (1..5), see synth.py; default 5 (prune), 4 (decode: 3 or 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--workload", choices=("prune", "decode", "calib"), default="prune",
                    help="prune: the prune step (default); decode: append 128 tokens + prune per step; "
                         "calib: calibration statistics of captured queries")
    ap.add_argument("--graph", action="store_true",
                    help="prune workload: time replays of the step captured once in a HIP graph")
    ap.add_argument("--entry", choices=("prune", "separate"), default="prune",
                    help="prune: one tria_prune call per step (default); separate: tria_score, "
                         "tria_select_topB and tria_compact")
    ap.add_argument("--score-path", choices=("auto", "tiled"), default="auto",
                    help="long-stream bf16 scoring: auto (stream clusters keep raw scores on chip) or tiled")
    ap.add_argument("--variant", choices=VARIANTS, default="default",
                    help="scoring form: default (post-RoPE keys, rotated queries), per_key_phase (post-RoPE "
                         "keys, literal per-key phases), pre_rope (keys cached before RoPE), weight_r (R-weighted "
                         "trigonometric term), offset_max (maximum over the future offsets)")
    return ap.parse_args()


def cpu_model() -> str:
    """The host CPU as lscpu reports it (model name, family / model / stepping numbers), else the
    first model name of /proc/cpuinfo."""
    import subprocess

    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        f = dict(line.split(":", 1) for line in out.splitlines() if ":" in line)
        f = {a.strip(): b.strip() for a, b in f.items()}
        name = f.get("Model name", "")
        if name:
            return f"{name} (family {f.get('CPU family', '?')}, model {f.get('Model', '?')}, " \
                   f"stepping {f.get('Stepping', '?')}; {f.get('Socket(s)', '?')} socket(s))"
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_info() -> dict:
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu": cpu_model(), "os_cpu_count": os.cpu_count(), "cpus_usable": aff}


def copy_bandwidth(torch, T, dev, nbytes: int = 8 << 30, reps: int = 5) -> dict:
    """Read + write GB/s of a plain device-to-device copy of nbytes (the best of reps), each rep
    after a cache flush: the achievable streaming rate the kernels are compared with.  "hip": the
    library's streaming copy kernel (tria_copy, non-temporal 16-byte loads and stores, eight in
    flight per lane); "torch": torch's copy_."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for name, run in (("hip", lambda: T.copy(src, dst)), ("torch", lambda: dst.copy_(src))):
        best = float("inf")
        for _ in range(reps):
            flush.zero_()
            torch.cuda.synchronize()
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        out[name] = 2 * nbytes / (best * 1e-3) / 1e9
    del src, dst, flush
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the prune step runs on one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not "
              "supported: this build measures one GPU (streams are independent, so they would shard across GPUs "
              "with no exchange between them)", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_compression_tria_amd as T
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    T.lib()   # fail loudly if the HIP library is missing
    if args.workload == "calib":
        return bench_calib(args, T, torch)
    if args.workload == "decode":
        return bench_decode(args, T, torch, synth)
    if args.config is None:
        args.config = 5
    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    t0 = time.time()
    pre_rope = args.variant == "pre_rope"
    flags = {"default": 0, "per_key_phase": T.PER_KEY_PHASE, "pre_rope": T.KEYS_PRE_ROPE,
             "weight_r": T.TRIG_WEIGHT_R, "offset_max": T.OFFSET_MAX}[args.variant]
    if args.score_path == "tiled":
        flags |= T.SCORE_TILED
    if args.config >= 4:
        wl = synth.make_device(cfg, dev, pre_rope=pre_rope)
    else:
        wl = synth.to_device(synth.make_host(cfg, pre_rope=pre_rope), dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    # The generated tensors stay as the pristine copy; the timed cache is a fresh allocation made
    # after them.  Measured on MI355X: the first ~68 GB a process allocates are read measurably
    # slower with the scoring access pattern (same data: 7.6 vs 6.8 ms for the 34 GB of keys); in
    # a serving process that region holds the model weights, allocated before the KV cache.
    k0, v0, pos0, t = wl["k"], wl["v"], wl["pos"], wl["t_dev"]
    k, v, pos = k0.clone(), v0.clone(), pos0.clone()
    S, L, Hkv, N, d = k.shape
    B = cfg.budget
    n_streams = S * L * Hkv
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], Hkv, cfg.theta)
    ws = T.workspace(T.prune_workspace_bytes(calib, S, N, B, k.dtype, flags), dev)
    F = torch.empty((S, L, Hkv, N), dtype=torch.float32, device=dev)
    kept = torch.empty((n_streams, min(B, N)), dtype=torch.int32, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def restore(dst=(k, v, pos), src=(k0, v0, pos0)):
        for a, b in zip(dst, src):
            a.copy_(b)
        if not args.no_flush:
            flush.zero_()

    host_us = []
    graph = None                      # --graph: the step on (k, v, pos) captured once

    def step(kk=k, vv=v, pp=pos, replay=False):
        ev[0].record(stream)
        if replay:
            h0 = time.perf_counter()
            graph.replay()
            host_us.append((time.perf_counter() - h0) * 1e6)
            ev[1].record(stream)
            ev[2].record(stream)
        elif args.entry == "prune":
            # the whole step through its own entry point (score, select and compact on one
            # stream); the workspace's error word is checked after the timed loop
            h0 = time.perf_counter()
            T.prune(calib, kk, vv, pp, t, B, F=F, kept=kept, flags=flags, ws=ws, stream=stream, check=False)
            host_us.append((time.perf_counter() - h0) * 1e6)
            ev[1].record(stream)
            ev[2].record(stream)
        else:
            T.score(calib, kk, t, F=F, ws=ws, stream=stream, pos=pp if flags & 3 else None, flags=flags)
            ev[1].record(stream)
            T.select_topB(F, B, kept=kept, stream=stream)
            ev[2].record(stream)
            T.compact(kk, vv, pp, kept, B, stream=stream)
        ev[3].record(stream)

    for _ in range(args.warmup):
        restore()
        step()
    torch.cuda.synchronize()
    if args.warmup > 0:
        T.score_check(ws)    # (the workspace's error word is set by the first step)
    if args.graph:
        if args.entry != "prune":
            sys.exit("bench.py: --graph captures the tria_prune step (--entry prune)")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            # the capture stream is the current one inside the context; nothing runs until replay
            T.prune(calib, k, v, pos, t, B, F=F, kept=kept, flags=flags, ws=ws, check=False)
        torch.cuda.synchronize()

    # the timed steps (the headline), without the library's per-kernel events
    phase = np.zeros((args.steps, 3))
    torch.cuda.synchronize()
    wall0 = time.time()
    host_us.clear()
    for i in range(args.steps):
        # the restore and the cache flush are still running on the stream while the step is
        # enqueued behind them, so the step's time is the device's own (the host's enqueue
        # latency, host_enqueue_us below, is not part of it, as for a caller that enqueues the
        # step behind other work)
        restore()
        step(replay=graph is not None)
        torch.cuda.synchronize()
        phase[i] = [ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]), ev[2].elapsed_time(ev[3])]
    wall_s = time.time() - wall0
    host_enqueue = list(host_us)
    T.score_check(ws)

    # The same steps again with per-kernel HIP-event timing inside the library (events on the
    # stream each kernel runs on): the per-kernel times and the dominant kernel's duration come
    # from here.  The event records between the kernels lengthen a short step (by ~20 us at
    # Qwen3-8B batch-1 shapes), so the headline above runs without them.
    T.timing_read()
    T.timing_enable(True)
    inst_ms = []
    for i in range(args.steps):
        restore()
        step()
        torch.cuda.synchronize()
        inst_ms.append(ev[0].elapsed_time(ev[3]))
    kern = T.timing_read()
    T.timing_enable(False)
    T.score_check(ws)
    moved_kept = kept.clone()

    # The same step on the process's first allocation (the generated cache, allocated before
    # anything else): roles swapped, the timed copy above now serves as the pristine one.
    restore()
    torch.cuda.synchronize()
    first_ms = []
    for i in range(min(args.steps, 5)):
        restore((k0, v0, pos0), (k, v, pos))
        step(k0, v0, pos0)
        torch.cuda.synchronize()
        first_ms.append(ev[0].elapsed_time(ev[3]))
    T.score_check(ws)
    restore((k0, v0, pos0), (k, v, pos))
    copy_rates = copy_bandwidth(torch, T, dev)
    copy_gbs = copy_rates["hip"]

    step_ms = phase.sum(axis=1)
    ms = float(step_ms.mean())
    total_keys = n_streams * N
    ar = torch.arange(kept.shape[1], device=dev, dtype=torch.int32)
    moved = int((moved_kept != ar).sum().item())
    alg = synth.algorithmic_bytes(cfg, moved)
    r = d * cfg.elem_bytes
    # algorithmic bytes per step of each timed kernel (what the method must move, no overheads);
    # on the stream-cluster path the scoring kernel also writes F (no separate normaliser).  Times
    # are summed per step, so a kernel split over several launches would be counted whole.
    on_chip_finish = kern["normalise"]["launches"] == 0
    kern_bytes = {
        "score_keys": n_streams * N * r + (n_streams * N * 4 if on_chip_finish else 0),   # keys read once (+ F)
        "normalise": n_streams * N * 4,         # F written once
        "select": n_streams * N * 4,            # F read once
        "compact": moved * (4 * r + 8),         # moved K, V rows and positions, read + written
        "select_compact": n_streams * N * 4 + moved * (4 * r + 8),   # both, in one kernel (tria_prune)
    }
    kernels = {}
    for name, kv in kern.items():
        if kv["launches"] == 0:
            continue
        per_step = kv["ms"] / args.steps
        kernels[name] = {"ms_per_step": round(per_step, 4), "launches_per_step": kv["launches"] // args.steps,
                         "avg_ms": round(kv["ms"] / kv["launches"], 4), "alg_bytes": int(kern_bytes[name]),
                         "GB_s": round(kern_bytes[name] / (per_step * 1e-3) / 1e9, 1)}
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_step"])
    ph = phase.mean(axis=0)
    out = {
        "metric": "prune step keys/s (scored + selected + compacted)",
        "value": round(total_keys / (ms * 1e-3), 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_median": round(float(np.median(step_ms)), 4),
        "ms_min": round(float(step_ms.min()), 4),
        "ms_max": round(float(step_ms.max()), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "streams": n_streams, "keys_per_stream": N, "budget": B,
                   "layers": L, "seqs": S, "q_heads": cfg.n_q_heads, "kv_heads": Hkv, "head_dim": d,
                   "cache_dtype": cfg.dtype, "score_variant": args.variant, "score_path": args.score_path,
                   "entry": "tria_prune" if args.entry == "prune" else "tria_score+tria_select_topB+tria_compact",
                   "hip_graph": graph is not None, "parallelism": "single-gpu"},
        "alg_bytes_per_step": int(alg),
        "alg_GB_s": round(alg / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "moved_rows": moved,
        "phases_ms": ({"score": round(float(ph[0]), 4), "select": round(float(ph[1]), 4),
                       "compact": round(float(ph[2]), 4)} if args.entry == "separate" else
                      {name: kv["ms_per_step"] for name, kv in kernels.items()}),
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["GB_s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kernels[dom]["GB_s"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic(cfg.name).get(dom)},
        "copy_GB_s": round(copy_gbs, 1),
        "torch_copy_GB_s": round(copy_rates["torch"], 1),
        "alg_frac_of_copy": round(alg / (ms * 1e-3) / 1e9 / copy_gbs, 4),
        "placement": {"timed_cache": "allocated after the generated pristine copy (K, V, positions)",
                      "ms_per_step_first_allocation": round(float(np.mean(first_ms)), 4),
                      "ms_min_first_allocation": round(float(np.min(first_ms)), 4)},
        "host": host_info(),
        "ms_per_step_with_kernel_events": round(float(np.mean(inst_ms)), 4),
        "wall_s_timed_loop_incl_restore": round(wall_s, 3),
        "host_enqueue_us": (round(float(np.mean(host_enqueue)), 1) if host_enqueue else None),
        "gen_s": round(gen_s, 1),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, cfg, wl, k0, v0, pos0, total_keys / (ms * 1e-3), pre_rope,
                                           form="max" if args.variant == "offset_max" else "fac",
                                           weight_r=args.variant == "weight_r")
    calib.free()
    print(json.dumps(out), flush=True)


def bench_decode(args, T, torch, synth):
    """Decode loop on config 4 shapes (Qwen3-8B, batch 64), or with --config 3 on Qwen3-8B batch-1
    shapes: append 128 tokens' rows, prune B + 128 -> B, per step."""
    cid = 4 if args.config is None else args.config
    if cid not in (3, 4):
        sys.exit(f"bench.py: the decode loop runs on config 3 or 4 (a cache of B + 128 keys), not {cid}")
    cfg = synth.CONFIGS[cid]
    dev = torch.device("cuda:0")
    # N = B + 128 keys: a full cache
    wl = synth.make_device(cfg, dev) if cid >= 4 else synth.to_device(synth.make_host(cfg), dev)
    assert cfg.n_keys == cfg.budget + 128
    k, v, pos, t = wl["k"], wl["v"], wl["pos"], wl["t_dev"].clone()
    S, L, Hkv, cap, d = k.shape
    B = cfg.budget
    n_new = cap - B
    streams = S * L * Hkv
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], Hkv, cfg.theta)
    # the rows of 128 new tokens (one draw, appended every step at advancing positions)
    kn = k[:, :, :, B:].clone()
    vn = v[:, :, :, B:].clone()
    pn0 = pos[:, :, :, B:].clone()
    F = torch.empty((S, L, Hkv, cap), dtype=torch.float32, device=dev)
    kept = torch.empty((streams, B), dtype=torch.int32, device=dev)
    ws = T.workspace(T.prune_workspace_bytes(calib, S, cap, B, k.dtype), dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    T.prune(calib, k, v, pos, t, B, F=F, kept=kept, ws=ws, stream=stream)    # start from a pruned cache
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    times = []
    step_no = 0

    def step():
        nonlocal step_no
        step_no += 1
        pn = pn0 + 128 * step_no
        t.add_(128)
        return pn

    for _ in range(args.warmup):
        pn = step()
        T.decode_step(calib, k, v, pos, t, B, B, kn, vn, pn, F=F, kept=kept, ws=ws, stream=stream, check=False)
    torch.cuda.synchronize()

    def timed(out):
        for _ in range(args.steps):
            pn = step()
            if not args.no_flush:
                flush.zero_()
            # enqueued behind the flush: the step's time is the device's own
            ev[0].record(stream)
            n = T.decode_step(calib, k, v, pos, t, B, B, kn, vn, pn, F=F, kept=kept, ws=ws, stream=stream,
                              check=False)
            ev[1].record(stream)
            torch.cuda.synchronize()
            assert n == B
            out.append(ev[0].elapsed_time(ev[1]))

    timed(times)                       # the headline, without the library's per-kernel events
    T.score_check(ws)
    T.timing_read()
    T.timing_enable(True)
    inst = []
    timed(inst)                        # per-kernel times (events between the kernels)
    kern = T.timing_read()
    T.timing_enable(False)
    T.score_check(ws)
    ms = float(np.mean(times))
    kernels = {name: {"ms_per_step": round(kv["ms"] / args.steps, 4), "avg_ms": round(kv["ms"] / kv["launches"], 4),
                      "launches": kv["launches"]}
               for name, kv in kern.items() if kv["launches"]}
    out = {
        "metric": "decode-loop keys/s (128 tokens appended, B+128 keys scored, selected, compacted)",
        "value": round(streams * cap / (ms * 1e-3), 1), "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name + "-decode-loop", "streams": streams, "capacity": cap, "budget": B,
                   "new_tokens_per_step": n_new, "parallelism": "single-gpu"},
        "generated_tokens_per_s": round(S * n_new / (ms * 1e-3), 1),
        "ms_per_step_with_kernel_events": round(float(np.mean(inst)), 4),
        "kernels": kernels,
    }
    calib.free()
    print(json.dumps(out), flush=True)


def bench_calib(args, T, torch):
    """Calibration statistics over a captured-query tensor of Qwen3-32B shapes."""
    L, Hq, n_cal, d = 64, 64, 10240, 128
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    # per head: centre of norm 8 plus N(0, s^2) noise, s ~ U(0.05, 3) (concentrated to diffuse)
    centre = torch.randn((L, Hq, 1, d), generator=gen, device=dev)
    centre = 8.0 * centre / centre.norm(dim=-1, keepdim=True)
    spread = 0.05 + 2.95 * torch.rand((L, Hq, 1, 1), generator=gen, device=dev)
    q = torch.empty((L, Hq, n_cal, d), dtype=torch.bfloat16, device=dev)
    for l in range(L):
        q[l] = (centre[l] + spread[l] * torch.randn((Hq, n_cal, d), generator=gen, device=dev)).to(torch.bfloat16)
    outs = (torch.empty((L, Hq, d), device=dev), torch.empty((L, Hq, d // 2), device=dev),
            torch.empty((L, Hq, d // 2), device=dev))
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        T.calib_stats(q, *outs, stream=stream)
    torch.cuda.synchronize()
    T.timing_read()
    T.timing_enable(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    times = []
    for _ in range(args.steps):
        if not args.no_flush:
            flush.zero_()
        torch.cuda.synchronize()
        ev[0].record(stream)
        T.calib_stats(q, *outs, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        times.append(ev[0].elapsed_time(ev[1]))
    kern = T.timing_read()["calib"]
    T.timing_enable(False)
    ms = float(np.mean(times))
    kms = kern["ms"] / max(kern["launches"], 1)
    nbytes = L * Hq * n_cal * d * 2
    out = {
        "metric": "calibration queries/s (pre-RoPE query statistics)", "value": round(L * Hq * n_cal / (ms * 1e-3), 1),
        "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3-32b-calibration-64layer-64qhead-10240q-bf16", "layers": L, "q_heads": Hq,
                   "queries_per_head": n_cal, "head_dim": d},
        "roofline": {"bound": "hbm", "kernel": "calib", "achieved": round(nbytes / (kms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("qwen3-32b-calibration-64layer-64qhead-10240q-bf16").get("calib")},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle
        oracle.build()

        def run(n_layers):
            qh = q[:n_layers].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            t0 = time.perf_counter()
            oracle.calib_stats(qh)
            return time.perf_counter() - t0

        n_layers = 1
        dt = run(n_layers)
        if dt < args.cpu_seconds / 2:
            n_layers = int(min(16, max(1, args.cpu_seconds / max(dt, 1e-3))))
            if n_layers > 1:
                dt = run(n_layers)
        n_heads = n_layers * Hq
        out["cpu_baseline"] = {"value": round(n_heads * n_cal / dt, 1), "unit": "queries/s", "cores": 1,
                               "kind": "oracle", "sample": f"{n_heads} of {L * Hq} heads ({n_heads * n_cal} queries), "
                                                           f"fp64, single thread, {dt:.2f} s",
                               "cpu": cpu_model()}
    print(json.dumps(out), flush=True)


def cpu_baseline(args, cfg, wl, k0, v0, pos0, gpu_keys_s, pre_rope=False, form="fac", weight_r=False):
    """The fp64 oracle (factored form, OpenMP over streams) on a bounded sample of streams of the
    same workload, timed on the host cores: scores, z-score and GQA max, top-B selection, and the
    oracle's (out-of-place, one stream at a time) compaction of K, V and positions."""
    import synth
    from oracle import oracle

    oracle.build()
    N, d = cfg.n_keys, cfg.head_dim
    kk = k0.reshape(-1, N, d)
    vv = v0.reshape(-1, N, d)
    pp = pos0.reshape(-1, N)
    threads = oracle.max_threads(0)

    def run(ids):
        kh = synth.cache_to_host(kk[ids[0]:ids[-1] + 1])
        vh = synth.cache_to_host(vv[ids[0]:ids[-1] + 1])
        ph = pp[ids[0]:ids[-1] + 1].cpu().numpy()
        t0 = time.perf_counter()
        res = oracle.prune_streams(kh, ph, wl["t"], wl["qc"], wl["qn"], wl["rb"], cfg.budget, cfg.n_kv_heads,
                                   stream_ids=ids, form=form, n_threads=threads, pre_rope=pre_rope,
                                   weight_r=weight_r)
        for i in range(len(ids)):
            for x in (kh, vh, ph):
                oracle.compact_rows(x[i], res["kept"][i])
        return time.perf_counter() - t0

    n = max(1, min(threads, kk.shape[0]))
    dt = run(np.arange(n))
    if dt < args.cpu_seconds / 2:
        n2 = int(min(kk.shape[0], max(n, n * args.cpu_seconds / max(dt, 1e-3))))
        n2 = max(n, (n2 // threads) * threads)
        if n2 > n:
            n = n2
            dt = run(np.arange(n))
    keys = n * N
    return {"value": round(keys / dt, 1), "unit": "keys/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {kk.shape[0]} streams ({keys} keys), fp64 {form} form, score + select + "
                      f"compaction, {dt:.1f} s",
            "cpu": cpu_model(), "os_cpu_count": os.cpu_count(), "gpu_over_cpu": round(gpu_keys_s / (keys / dt), 1)}


if __name__ == "__main__":
    main()
