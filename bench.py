#!/usr/bin/env python3
"""Decode-step benchmark of the MosaicKV hot path on one MI355X.

One step = one mkv_append_decode call: the append of one new token per
request (rotate in float64, top-r, pack, block-key update) and then the decode
(query rotation, block scoring, top-k, sparse attention, merge, inverse
rotation), with the query rotation running inside the append's launch.

Default workload (128K context): GQA layer with 32 query / 8 KV heads, d=128,
batch 4, T=131072 tokens per request, bf16 storage, segments: 64 dense sink,
[64, 63520) packed r=26 keep 5%, [63520, 126976) packed r=38 keep 10%, 4096
dense recent, then a packed update segment (r=38, keep 10%) that receives the
new decode tokens. Inputs are seeded synthetic data (mkv_synth) resident in
HBM before the timed region.

Steps visit --layers distinct caches (same content, distinct addresses) in
turn, as a multi-layer model does: between two visits of one cache several
hundred MB of other layers' data stream through, so no call is served from the
previous call's footprint in the 256 MB last-level cache.

Prints one JSON line (see README of the repository root for fields).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mkv_synth as synth  # noqa: E402

METRIC = "decode-attn effective KV tokens/s/GPU + achieved HBM GB/s vs 8 TB/s peak"
PEAK_FP64_TFLOPS = 78.6  # MI355X fp64 vector peak: 256 CUs x 2.4 GHz x 64 fp64 FMA lanes x 2
PEAK_GBPS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def log(msg):
    print("[bench %s] %s" % (time.strftime("%H:%M:%S"), msg), file=sys.stderr, flush=True)


def workload(cfg: int, scale: int, extra: int):
    w = synth.workload(cfg, scale=scale, extra_cap=extra if cfg == 5 else 0)
    if cfg != 5:
        w = synth.with_update_segment(w, cap=extra)
    return w


def gen_rows(w, t_end):
    """Raw stored K/V [B][Hkv][t_end][d] (bf16 bit patterns or float32)."""
    B, hkv, d, dt = w["batch"], w["n_kv_heads"], w["d"], w["dtype"]
    npdt = np.uint16 if dt == "bf16" else np.float32
    K = np.empty((B, hkv, t_end, d), npdt)
    V = np.empty((B, hkv, t_end, d), npdt)
    for b in range(B):
        for g in range(hkv):
            synth.gen_kv_into(w["cfg"], b, g, 0, 0, t_end, dt, K[b, g], d)
            synth.gen_kv_into(w["cfg"], b, g, 1, 0, t_end, dt, V[b, g], d)
    return K, V


def rotations(L, w, K, V, T):
    B, hkv, d = w["batch"], w["n_kv_heads"], w["d"]
    code = L.MKV_BF16 if w["dtype"] == "bf16" else L.MKV_F32
    R = np.empty((B, hkv, 2, d, d), np.float32)
    for b in range(B):
        for g in range(hkv):
            for kind, arr in ((0, K), (1, V)):
                x = np.ascontiguousarray(arr[b, g, :T[b]])
                L.mkv_rotation_from_prefill(x.ctypes.data, code, int(T[b]), d, R[b, g, kind].ctypes.data, None)
    return R


def dev(torch, a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def union_summary(w, lengths, sel):
    """Per request and segment: filled tokens, blocks and the number of distinct
    blocks the query heads of each KV head selected (summed over KV heads)."""
    from kv_cache_compression_mkv_amd.bytes_model import keep_blocks
    G = w["n_q_heads"] // w["n_kv_heads"]
    out = []
    for b in range(w["batch"]):
        L = int(lengths[b])
        rows, col = [], 0
        for s in w["segs"][b]:
            filled = min(max(L - s["t_begin"], 0), s["t_cap"])
            if s["kind"] == synth.DENSE:
                rows.append(dict(kind="dense", filled=filled))
                continue
            nb = -(-filled // 16)
            k = keep_blocks(nb, s["keep_ppm"], s["k_abs"])
            uni = 0
            for g in range(w["n_kv_heads"]):
                blocks = sel[b, g * G:(g + 1) * G, col:col + k]
                uni += len(np.unique(blocks))
            col += k
            rows.append(dict(kind="packed", filled=filled, r=s["r"], n_blocks=nb, union=uni,
                             bitmap=s["kind"] == synth.BITMAP, key_ch=s.get("key_ch", 0), group=s.get("group", 0)))
        out.append(rows)
    return out


def counter_traffic(kernel_key: str, workload_key: dict):
    """HBM bytes per dispatch from the committed counter summary, or None when it
    is missing, was taken on other kernel sources or on another workload
    (workload_key: config, scale, record layout, key channels, element group)."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    src = os.path.join(ROOT, "kv_cache_compression_mkv_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(src)):
        with open(os.path.join(src, name), "rb") as f:
            h.update(f.read())
    if c.get("source_sha256") != h.hexdigest() or c.get("workload") != workload_key:
        return None
    k = c.get("kernels", {}).get(kernel_key)
    if not k:
        return None
    return (k["fetch_kib"] * c["fetch_factor"] + k["write_kib"] * c["write_factor"]) * 1024.0


def prefill_summary(ms, vectors, d):
    """Bulk append of a whole layer cache (every request's prompt, every KV
    head): each token's K and V are rotated with d x d fp64 multiply-adds, so
    4 d^2 flops per (token, KV head). The rotation keeps one fp64 chain per
    output channel, so it runs on the fp64 vector ALU."""
    flops = 4.0 * d * d * vectors
    tf = flops / (ms * 1e-3) / 1e12
    return {"kernel": "k_compress (bulk append)", "token_heads": vectors, "ms": round(ms, 3),
            "token_heads_per_s": round(vectors / (ms * 1e-3), 1),
            "roofline": {"bound": "alu", "achieved": round(tf, 2), "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP64_TFLOPS, 4), "flops_per_token_head": 4 * d * d}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, scale, R, T0, steps, n_units, workers, steps_1t):
    """The oracle as it stands, on a bounded sample of the workload's
    (request, KV head) units. Each unit is compressed up to its prompt length
    (not timed), then runs decode steps (append one token, then decode its G
    query heads) with one oracle thread per unit:
      * all cores: `workers` units at once, one per thread (the oracle's own
        threading only spans the 4 heads of a unit, so units run side by side);
      * one thread: one unit alone.
    A step of the whole workload is B * Hkv unit-steps; tokens/s = sum_b T_b
    over that step time."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as orc
    w = workload(cfg, scale, 2 * steps + steps_1t + 64)
    G = w["n_q_heads"] // w["n_kv_heads"]
    dt, d, hkv = w["dtype"], w["d"], w["n_kv_heads"]
    n_all = w["batch"] * hkv
    to64 = (lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)) if dt == "bf16" else \
        (lambda a: a.astype(np.float64))
    npdt = np.uint16 if dt == "bf16" else np.float32
    # spread the sample over the workload's units
    units = [divmod(int(u * n_all // n_units), hkv) for u in range(n_units)]
    prep_threads = synth.host_threads()
    states = []
    for b, g in units:
        rows = int(T0[b]) + 2 * steps + steps_1t + 1
        Kb = np.empty((rows, d), npdt)
        Vb = np.empty((rows, d), npdt)
        synth.gen_kv_into(cfg, b, g, 0, 0, rows, dt, Kb, d)
        synth.gen_kv_into(cfg, b, g, 1, 0, rows, dt, Vb, d)
        Kr, Vr = to64(Kb), to64(Vb)
        Rk, Rv = R[b, g, 0].astype(np.float64), R[b, g, 1].astype(np.float64)
        st = orc.compress_unit(Kr, Vr, Rk, Rv, w["segs"][b], int(T0[b]), dt, nthreads=prep_threads)
        qs = [synth.gen_q(cfg, 5000 + s, w["batch"], w["n_q_heads"], dt)[b, g * G:(g + 1) * G].astype(np.float64)
              for s in range(steps + steps_1t)]
        states.append([b, Kr, Vr, Rk, Rv, st, qs])

    def run(i, n, q0):
        b, Kr, Vr, Rk, Rv, st, qs = states[i]
        for s in range(n):
            st = orc.compress_unit(Kr, Vr, Rk, Rv, w["segs"][b], st["length"] + 1, dt, nthreads=1, state=st)
            orc.decode_unit(st, qs[q0 + s], Rk, Rv, nthreads=1)
        states[i][5] = st

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda i: run(i, steps, 0), range(n_units)))
    wall = time.perf_counter() - t0
    unit_steps_per_s = n_units * steps / wall
    t1 = time.perf_counter()
    run(0, steps_1t, steps)
    one = (time.perf_counter() - t1) / steps_1t
    total_T = float(np.sum(T0))
    return dict(value=total_T / (n_all / unit_steps_per_s), unit="tokens/s", cores=min(workers, n_units),
                kind="oracle", cpu_model=cpu_model(), host_cpus_visible=len(os.sched_getaffinity(0)),
                sample="%d of %d (request, KV head) units x %d decode steps each (append 1 token + decode "
                       "its %d query heads) at T=%d, one oracle thread per unit, %d units at once: %.1f s; "
                       "scaled to all %d units" % (n_units, n_all, steps, G, int(T0[0]), min(workers, n_units),
                                                   wall, n_all),
                one_thread={"value": total_T / (n_all * one), "cores": 1,
                            "sample": "1 unit x %d decode steps, %.2f ms per unit-step" % (steps_1t, one * 1e3)},
                seconds=float(wall + one * steps_1t))


def pct(a, q):
    return float(np.percentile(np.asarray(a, np.float64), q))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3,
                    help="workload id: 1 single head 4K fp32, 2 32K layer, 3 128K batch 4 (default), "
                         "4 1M tokens, 5 serving batch 32")
    ap.add_argument("--scale", type=int, default=1, help="divide token counts (1 = full size)")
    ap.add_argument("--cpu-units", type=int, default=-1,
                    help="oracle sample: units run side by side (-1: one per host thread; 0 disables)")
    ap.add_argument("--cpu-steps", type=int, default=-1,
                    help="oracle decode steps per unit (-1: 600 at 128K context, scaled inversely with context)")
    ap.add_argument("--cpu-steps-1t", type=int, default=-1, help="oracle decode steps of the 1-thread run "
                                                                 "(-1: half of --cpu-steps)")
    ap.add_argument("--layers", type=int, default=4,
                    help="distinct layer caches visited round-robin (keeps every call cache-cold)")
    ap.add_argument("--layout", choices=["u8", "bitmap"], default="u8",
                    help="position format of the packed records: u8 channel indices (default) or bitmaps")
    ap.add_argument("--key-ch", type=int, default=0,
                    help="block keys over the leading N rotated channels of every packed segment (0: all)")
    ap.add_argument("--group", type=int, default=0, choices=[0, 1, 2, 4, 8],
                    help="every packed segment keeps whole groups of N adjacent channels (0: single channels)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a streaming scale kernel over this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (requested --gpus %d)."
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    K_steps, W_steps = args.steps, args.warmup
    cap_extra = W_steps + 2 * K_steps + 64
    w = workload(args.config, args.scale, cap_extra)
    if args.layout == "bitmap":
        w["segs"] = synth.as_bitmap(w["segs"])
    if args.key_ch:
        w["segs"] = synth.with_key_channels(w["segs"], args.key_ch)
    if args.group > 1:
        w["segs"] = synth.with_groups(w["segs"], args.group)
    T0 = np.asarray(w["lengths"], np.int64)
    B, hq, hkv, d, dt = w["batch"], w["n_q_heads"], w["n_kv_heads"], w["d"], w["dtype"]
    n_step_total = W_steps + 2 * K_steps + 1
    log("workload cfg=%d scale=%d B=%d T=[%d..%d] dtype=%s" % (args.config, args.scale, B, int(T0.min()),
                                                              int(T0.max()), dt))

    t = time.time()
    K, V = gen_rows(w, int(T0.max()) + n_step_total)
    log("generated inputs in %.1f s" % (time.time() - t))

    import torch  # noqa: E402
    from kv_cache_compression_mkv_amd import _lib as L
    from kv_cache_compression_mkv_amd import bytes_model as bm
    from kv_cache_compression_mkv_amd.cache import Cache

    t = time.time()
    R = rotations(L, w, K, V, T0)
    log("host rotations in %.1f s" % (time.time() - t))

    n_layers = max(1, args.layers)
    kpre = dev(torch, K[:, :, :int(T0.max())])
    vpre = dev(torch, V[:, :, :int(T0.max())])
    caches = []
    prefill_all = []
    # one untimed prefill first: the first bulk append in a process runs cold
    warm = Cache(B, hq, hkv, dt, w["segs"])
    warm.set_rotation(R)
    warm.append(kpre, vpre, [int(x) for x in T0])
    torch.cuda.synchronize()
    del warm
    for _ in range(n_layers):
        c = Cache(B, hq, hkv, dt, w["segs"])
        c.set_rotation(R)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        c.append(kpre, vpre, [int(x) for x in T0])
        e1.record()
        torch.cuda.synchronize()
        prefill_all.append(e0.elapsed_time(e1))
        c.workspace()
        caches.append(c)
    del kpre, vpre
    prefill_ms = float(np.median(prefill_all))
    log("prefill compress of %d (token, KV head) pairs per layer cache: %s ms" % (
        int(T0.sum()) * hkv, ", ".join("%.2f" % t for t in prefill_all)))

    # per-step inputs, resident in HBM before timing
    newk = [dev(torch, np.stack([K[b, :, T0[b] + s:T0[b] + s + 1] for b in range(B)])) for s in range(n_step_total)]
    newv = [dev(torch, np.stack([V[b, :, T0[b] + s:T0[b] + s + 1] for b in range(B)])) for s in range(n_step_total)]
    qs = [torch.from_numpy(synth.gen_q(args.config, s, B, hq, dt)).cuda() for s in range(n_step_total)]
    del K, V
    out = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    ones = [1] * B
    step = 0
    tokens = []

    def run_step():
        nonlocal step
        c = caches[step % n_layers]
        c.append_decode(newk[step], newv[step], ones, qs[step], out=out)
        tokens.append(sum(c.lengths))
        step += 1

    for _ in range(W_steps):
        run_step()
    torch.cuda.synchronize()
    tok0 = len(tokens)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K_steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(K_steps):
        run_step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(K_steps)]
    gpu_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = wall * 1e3 / K_steps
    mean_len = float(np.mean(tokens[tok0:tok0 + K_steps]))
    value = mean_len / (ms_per_step / 1e3)
    log("timed %d steps: %.4f ms/step wall, %.4f ms/step GPU events (p10 %.4f, p50 %.4f, p90 %.4f)" % (
        K_steps, ms_per_step, gpu_ms / K_steps, pct(step_ms, 10), pct(step_ms, 50), pct(step_ms, 90)))

    # per-kernel durations, live: HIP events around every launch of the same steps
    L.mkv_timing_enable(True)
    for _ in range(K_steps):
        run_step()
    torch.cuda.synchronize()
    stages = L.mkv_timing_read()
    L.mkv_timing_enable(False)
    stage_ms = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in stages.items()}
    log("per-launch ms: " + ", ".join("%s %.4f" % (k, v) for k, v in stage_ms.items() if v))

    # algorithmic bytes of one decode call at the current lengths, from its own selections
    c = caches[step % n_layers]
    _, sel = c.decode(qs[step], out=out, want_sel=True)
    torch.cuda.synchronize()
    lens_now = np.asarray(c.lengths)
    summ = union_summary(w, lens_now, sel.cpu().numpy())
    sb = 2 if dt == "bf16" else 4
    call = bm.decode_call_bytes(d, sb, hkv, B, hq, summ)
    r_new = [s["r"] for s in w["segs"][0] if synth.is_packed(s["kind"])][-1]
    append = bm.append_bytes(d, sb, hkv, B, r_new, args.layout == "bitmap", args.key_ch, args.group)
    step_bytes = call["total"] + append
    # algorithmic bytes each kernel of the step must move (the query rotation
    # runs in the append's launch: it reads R_k and the queries, writes q')
    qrot_bytes = B * hkv * d * d * 4 + B * hq * d * 4
    cand = {"attend": call["records"] + call["dense"], "score": call["meta"], "select": 0,
            "merge": B * hkv * d * d * 4 + B * hq * d * 4, "compress": append + qrot_bytes, "q_rotate": qrot_bytes}
    kernels = {}
    for k, ms in stage_ms.items():
        if not ms:
            continue
        a = cand.get(k, 0)
        kernels[k] = {"avg_launch_ms": round(ms, 5), "alg_bytes": int(a),
                      "gbps": round(a / (ms * 1e-3) / 1e9, 1) if a else None,
                      "frac": round(a / (ms * 1e-3) / 1e9 / PEAK_GBPS, 4) if a else None}
    dom = max(("attend", "score"), key=lambda k: stage_ms.get(k, 0.0))
    dom_ms = stage_ms[dom]
    achieved = cand[dom] / (dom_ms * 1e-3) / 1e9
    traffic = counter_traffic(dom, {"config": args.config, "scale": args.scale, "layout": args.layout,
                                    "key_ch": args.key_ch, "group": max(args.group, 1)})
    dense_equiv = bm.dense_kv_bytes(int(np.sum(lens_now)), d, sb) * hkv
    dec_ms = sum(stage_ms.get(k, 0.0) for k in ("q_rotate", "score", "select", "attend", "merge"))
    if not stage_ms.get("q_rotate"):
        # the query rotation ran inside the append's launch: count the decode
        # from score on, and its bytes without the rotation's R_k read
        dec_bytes = call["total"] - B * hkv * d * d * 4
    else:
        dec_bytes = call["total"]
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9

    cpu = None
    if args.cpu_steps < 0:
        args.cpu_steps = int(max(20, min(600, 600 * 131072 / float(np.mean(T0)))))
    if args.cpu_steps_1t < 0:
        args.cpu_steps_1t = max(10, args.cpu_steps // 2)
    if args.cpu_units != 0:
        workers = synth.host_threads()
        n_units = workers if args.cpu_units < 0 else args.cpu_units
        n_units = min(n_units, B * hkv)
        log("oracle CPU baseline: %d units x %d steps on %d threads, then 1 unit x %d steps on 1 thread" % (
            n_units, args.cpu_steps, min(workers, n_units), args.cpu_steps_1t))
        cpu = cpu_baseline(args.config, args.scale, R, T0, args.cpu_steps, n_units, workers, args.cpu_steps_1t)
        log("oracle: %.3g tokens/s on %d threads, %.3g on 1 thread (%.1f s)" % (
            cpu["value"], cpu["cores"], cpu["one_thread"]["value"], cpu["seconds"]))
        cpu.pop("seconds")

    if args.copy_mib > 0:
        # a plain streaming kernel of known traffic: reads n bytes, writes n bytes
        n = args.copy_mib * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        log("calibration kernel: read %d bytes, wrote %d bytes" % (n, n))

    seg_desc = "; ".join("%s[%d,%d)%s" % ("D" if s["kind"] == 0 else "P", s["t_begin"], s["t_begin"] + s["t_cap"],
                                          "" if s["kind"] == 0 else " r=%d keep=%s" % (
                                              s["r"], ("%d blocks" % s["k_abs"]) if s["k_abs"] else
                                              ("%g%%" % (s["keep_ppm"] / 1e4))))
                         for s in w["segs"][0])
    if args.config == 5:
        seg_desc += " (request 0; every request: D[0,64) then one packed segment)"
    names = {1: "single head, T=4096, fp32", 2: "32K-token GQA layer", 3: "128K-token GQA layer, batch 4",
             4: "1M-token GQA layer share", 5: "serving batch 32, T uniform in [16K, 96K]"}
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "%s: GQA %d/%d heads d=%d, batch %d, T=%d..%d/request at start, %s storage; "
                        "step = append 1 token/request + decode attention" % (
                            names.get(args.config, "workload %d" % args.config), hq, hkv, d, B, int(T0.min()),
                            int(T0.max()), dt),
            "global_batch": B,
            "seq_len": int(T0.max()),
            "segments": seg_desc,
            "storage": dt,
            "record_positions": "bitmap" if args.layout == "bitmap" else "u8 indices",
            "key_channels": args.key_ch or d,
            "element_group": max(args.group, 1),
            "parallelism": "single GPU",
            "layer_caches": n_layers,
        },
        "step_ms_p10_p50_p90": [round(pct(step_ms, 10), 4), round(pct(step_ms, 50), 4), round(pct(step_ms, 90), 4)],
        "achieved_step_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_alg_bytes": int(step_bytes),
        "append_alg_bytes": int(append),
        "decode_alg_bytes": {k: int(v) for k, v in call.items()},
        "decode_roofline": {"kernels": "q_rotate+score+select+attend+merge (summed launch times)",
                            "bound": "hbm", "alg_bytes": int(dec_bytes), "ms": round(dec_ms, 5),
                            "achieved": round(dec_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                            "frac": round(dec_gbps / PEAK_GBPS, 4)},
        "kernels": kernels,
        "dense_equiv_bytes": int(dense_equiv),
        "gpu_event_ms_per_step": round(gpu_ms / K_steps, 4),
        "prefill_compress_ms": round(prefill_ms, 3),
        "prefill": prefill_summary(prefill_ms, int(T0.sum()) * hkv, d),
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": int(cand[dom]),
            "avg_launch_ms": round(dom_ms, 5),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
