#!/usr/bin/env python3
"""Benchmark of the Gemma 2 attention layer on one MI355X.

One step = the whole hot path on seeded synthetic inputs shaped like Gemma 2 9B:
  prefill of a local (sliding window 4096) and a global layer at B=2, T=S=8192,
  H=16, KVH=8, d=256, softcap 50, query_scale 1/16; then decode of one token
  for 64 sequences against a global linear cache (L_b uniform on [4096, 8192])
  and a local 4096-slot ring; then the same decode against a paged cache
  (16-token blocks at seeded random pool positions, one block table per
  sequence); and a chunked prefill: the last 2048 queries of the 9B batch
  against its whole 8192-token cache (local and global).  The steps on either
  side of the attention call are timed after the steps, on their own: the
  rotary embedding of the 9B prefill's Q and K, and the final-logit soft-cap
  (30) over the prefill batch's vocabulary logits (2*8192 x 256000, bf16);
  and the backward pass of the 9B local+global pair (dq, dk, dv for a seeded
  upstream gradient), counted as 10*d FLOPs per visible (query head, key) pair
  (S recomputed, dP, dV, dK, dQ: what its kernels execute, dS being stored
  once rather than recomputed); and the local + global prefill pairs of the
  2B-shaped (B=4, H=8, KVH=4, d=256) and 27B-shaped (B=1, H=32, KVH=16,
  d=128, query_scale 1/12) workloads.
  Each of these secondary timings first runs its launches back to back for
  0.25 s: the chip lowers its clock while idle (they follow seconds of
  host-side input generation) and needs ~0.1 s of load to raise it again.
  No decode launch can find its own cache rows in the 256 MB Infinity Cache
  (MALL): the four decode launches of a step read four different buffers
  (ring, linear cache, and the pool twice with different visible rows, each
  2.1-3.2 GB, with non-temporal loads), and about 10 GB of other traffic
  passes between two launches of the same decode.  An explicit 1 GiB stream
  through the caches before each decode launch left decode unchanged (within
  1%) and slowed the prefill launches of the same step by 3-5%, so it is not
  part of the step.

Reported (one JSON line):
  value    prefill effective TFLOP/s = algorithmic FLOPs of the pair / prefill
           kernel time, counting 4*d FLOPs per visible (query head, key) pair
           only (QK^T and PV, 2*d each); masked pairs are not counted;
  decode   KV GB/s = visible K/V bytes (plus q and out) / decode time;
  roofline the prefill kernel against the bf16 dense MFMA peak (2.5 PFLOP/s),
           durations from HIP events on the launch stream over the timed steps;
  cpu_baseline the fp64 oracle on a bounded sample of the same workload, with
           the host's CPU model, usable CPUs and OMP_NUM_THREADS.
The library's baked source hash must equal the sources' hash, else the run
stops: the numbers always describe the code beside this script.
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = ("prefill eff. TFLOP/s (% bf16 MFMA peak) @9B 8K; "
          "decode KV GB/s (% HBM peak)")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_bf16_9b_8k_traffic.txt")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-rows", type=int, default=40960,
                    help="rows per layer of the oracle's bounded CPU sample (0: none)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run one device copy of this many MiB "
                         "(reference kernel for HBM counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no benchmark: read rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
                         "counter CSVs of a run made with --copy-calibration-mib, and "
                         "write the per-launch HBM traffic of the kernels to profiles/")
    ap.add_argument("--calibration-mib", type=int, default=1024,
                    help="size of the calibration copy used in the counter runs")
    return ap.parse_args()


KERNEL_FILES = {  # the sources each measured kernel is built from
    "prefill": ("prefill_bf16.hip", "g2_device.h", "g2_kernels.h", "g2_tiles.h"),
    "decode": ("decode.hip", "g2_device.h", "g2_kernels.h"),
}


def kernel_source_hash(which):
    """sha256 of the sources one measured kernel is built from (the staleness
    key of the committed counter readings)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_g2attn_prefill_amd", "csrc")
    names = KERNEL_FILES[which]
    for name in names:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()


def prefill_pairs(T, S, window, is_local):
    """Visible (query, key) pairs of one (batch, head) slice."""
    tot = 0
    off = S - T
    for t in range(T):
        p = t + off
        lo = max(0, p - window + 1) if is_local else 0
        tot += p - lo + 1
    return tot


def prefill_tile_pairs(T, S, window, is_local, rows_per_wave=32, bn=32):
    """(query, key) pairs the prefill kernel computes for one (batch, head) slice:
    every key tile of bn keys that any of a wave's rows_per_wave positions sees
    is computed whole (masked entries included)."""
    off = S - T
    tot = 0
    for a in range(0, T, rows_per_wave):
        rows = min(rows_per_wave, T - a)
        p_first, p_last = a + off, a + rows - 1 + off
        lo = max(0, p_first - window + 1) if is_local else 0
        tiles = p_last // bn - lo // bn + 1
        tot += tiles * bn * rows
    return tot


def warm(fn, seconds=0.25):
    """Run fn back to back for about `seconds` of GPU time before it is timed.
    The chip lowers its clock while idle (these timings follow seconds of
    host-side input generation) and needs ~0.1 s of load to raise it again."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def gemm_tflops(dev, n=8192, reps=10):
    """bf16 GEMM rate of torch's library path (n x n x n) on this GPU, for context:
    the MFMA rate a tuned library reaches at the clock the chip holds under load."""
    import torch
    a = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    b = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    c = a @ b
    warm(lambda: a @ b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b, c
    return 2.0 * n ** 3 / secs / 1e12


def copy_gbs(dev, mib=1024, reps=5):
    """Device-to-device copy rate (read + write bytes / time) on this GPU, for context."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return 2.0 * n / secs / 1e9


def time_adjacent(g2, qd, kd, dev, stream, reps=10, vocab=256000):
    """HBM rate of the rotary embedding (Q and K in place) and of the final
    soft-cap (logits in place): bytes read + written / kernel time."""
    import torch
    B, T = qd.shape[0], qd.shape[1]
    pos = torch.arange(T, dtype=torch.int32, device=dev).repeat(B, 1).contiguous()
    q2, k2 = qd.clone(), kd.clone()
    logits = torch.randn((B * T, vocab), dtype=torch.bfloat16, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    warm(lambda: (g2.rope_(q2, pos, stream=stream), g2.rope_(k2, pos, stream=stream),
                  g2.softcap_(logits, 30.0, stream=stream)))
    ev[0].record(stream)
    for _ in range(reps):
        g2.rope_(q2, pos, stream=stream)
        g2.rope_(k2, pos, stream=stream)
    ev[1].record(stream)
    for _ in range(reps):
        g2.softcap_(logits, 30.0, stream=stream)
    ev[2].record(stream)
    torch.cuda.synchronize()
    t_rope = ev[0].elapsed_time(ev[1]) * 1e-3 / reps
    t_cap = ev[1].elapsed_time(ev[2]) * 1e-3 / reps
    rope_bytes = 2.0 * (q2.numel() + k2.numel()) * q2.element_size()
    cap_bytes = 2.0 * logits.numel() * logits.element_size()
    del q2, k2, logits
    return {"rope": {"metric": "rotary embedding of Q and K, GB/s",
                     "parity": "partly unpinned: the pair layout (x[i], x[i+d/2]) and base 10000 "
                               "are readings, the pages give no rotary formula",
                     "value": round(rope_bytes / t_rope / 1e9, 1),
                     "frac_of_hbm_peak": round(rope_bytes / t_rope / 1e9 / PEAK_HBM_GBS, 4),
                     "ms": round(t_rope * 1e3, 4), "bytes": rope_bytes},
            "final_softcap": {"metric": "final-logit soft-cap, GB/s",
                              "value": round(cap_bytes / t_cap / 1e9, 1),
                              "frac_of_hbm_peak": round(cap_bytes / t_cap / 1e9 / PEAK_HBM_GBS, 4),
                              "ms": round(t_cap * 1e3, 4), "bytes": cap_bytes,
                              "shape": [int(B * T), vocab]}}


def time_backward(g2, qd, kd, vd, kw, dev, stream, reps=5):
    """Backward pass of the local and global layer (after their forward with
    log-sum-exp, outside the timed region)."""
    import torch
    from attention_g2attn_prefill_amd import synth
    B, T, H, d = qd.shape
    S = kd.shape[1]
    dout = synth.draw(tuple(qd.shape), 17, 3).to(dev)
    res = {}
    total_f, total_t = 0.0, 0.0
    for is_local in (True, False):
        out, lse = g2.prefill_lse(qd, kd, vd, is_local=is_local, stream=stream, **kw)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws = torch.empty(g2.backward_workspace_bytes(B, T, S, H), dtype=torch.uint8, device=dev)
        warm(lambda: g2.prefill_backward(qd, kd, vd, out, dout, lse, is_local=is_local, dq=dq,
                                         dk=dk, dv=dv, workspace=ws, stream=stream, **kw))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g2.prefill_backward(qd, kd, vd, out, dout, lse, is_local=is_local, dq=dq, dk=dk,
                                dv=dv, workspace=ws, stream=stream, **kw)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        f = 10.0 * d * B * H * prefill_pairs(T, S, kw["window"], is_local)
        res["local" if is_local else "global"] = {"ms": round(t * 1e3, 4),
                                                  "tflops": round(f / t / 1e12, 2)}
        total_f += f
        total_t += t
        del out, lse, dq, dk, dv, ws
    tf = total_f / total_t / 1e12
    res.update({"metric": "backward eff. TFLOP/s (10*d per visible pair)", "value": round(tf, 2),
                "unit": "TFLOP/s", "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                "executed_flops_per_pair": 10 * d, "flops": total_f})
    return res


def measured_traffic(which, key):
    """HBM bytes per launch from committed counter runs, if they were taken on
    the current sources of that kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.loads(fh.read())
    except (OSError, ValueError):
        return None
    if rec.get(which + "_source_sha256") != kernel_source_hash(which):
        return None
    return rec.get(key)


def _counter_rows(path, counter):
    import csv
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]),
                             int(r["Grid_Size"])))
    return sorted(rows)


def write_traffic(fetch_csv, write_csv, calib_mib):
    """Per-launch HBM bytes of the prefill and decode kernels from counter runs.

    FETCH_SIZE / WRITE_SIZE are in KiB per dispatch.  Each is scaled by the
    ratio true bytes / counter reading of the calibration copy (the largest
    device copy in the run: it reads and writes calib_mib MiB)."""
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")
    nbytes = calib_mib * 1024.0 * 1024.0
    cf = max((v for _, n, v, _g in fetch if "copyBuffer" in n), default=0.0)
    cw = max((v for _, n, v, _g in write if "copyBuffer" in n), default=0.0)
    if cf <= 0 or cw <= 0:
        raise SystemExit("no calibration copy found in the counter files")
    f_fetch = nbytes / (cf * 1024.0)
    f_write = nbytes / (cw * 1024.0)

    def per_launch(tag, largest_grid=False):
        """Mean over the dispatches of a kernel; with largest_grid, only those
        of its largest grid issued by the step loop (the full-size 9B prefill:
        not the chunked one, nor the 2B pair timed later, whose grid is the
        same size).  The step loop ends with its last chunked-prefill launch."""
        def pick(rows):
            sel = [(d, v, g) for d, n, v, g in rows if tag in n]
            if largest_grid and sel:
                gmax = max(g for _, _, g in sel)
                last_chunk = max((d for d, _, g in sel if g != gmax), default=None)
                sel = [x for x in sel if x[2] == gmax and (last_chunk is None or x[0] < last_chunk)]
            return [v for _, v, _ in sel]
        fv, wv = pick(fetch), pick(write)
        if not fv or not wv:
            return None
        return (sum(fv) / len(fv) * 1024.0 * f_fetch + sum(wv) / len(wv) * 1024.0 * f_write,
                len(fv))
    pre = per_launch("prefill_bf16_kernel<256, 2, 32, 1, true, false>", largest_grid=True)  # cap 50: constant offset, no lse
    dec = per_launch("decode_split_kernelIDF16bLi256ELi2ELb0E")    # linear / ring cache
    pag = per_launch("decode_split_kernelIDF16bLi256ELi2ELb1E")    # paged cache
    rec = {"prefill_source_sha256": kernel_source_hash("prefill"),
           "decode_source_sha256": kernel_source_hash("decode"),
           "calibration_copy_mib": calib_mib,
           "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4),
           "traffic_bytes_per_launch": round(pre[0]) if pre else None,
           "prefill_launches": pre[1] if pre else 0,
           "decode_split_traffic_bytes_per_launch": round(dec[0]) if dec else None,
           "paged_split_traffic_bytes_per_launch": round(pag[0]) if pag else None,
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE -d <dir> -o p --output-format csv -- python3 bench.py "
               f"--steps 20 --warmup 5 --cpu-rows 0 --copy-calibration-mib {calib_mib}",
               "rocprofv3 --pmc WRITE_SIZE -d <dir> -o p --output-format csv -- python3 bench.py "
               f"--steps 20 --warmup 5 --cpu-rows 0 --copy-calibration-mib {calib_mib}",
               "python3 bench.py --write-traffic <fetch csv> <write csv>"]}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec))


def host_description():
    """CPU model, logical CPUs this process may run on, and OMP_NUM_THREADS."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_model": model, "affinity_cpus": affinity,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def time_models(g2, dev, stream, reps=10):
    """Prefill local + global layer pairs of the 2B- and 27B-shaped workloads
    (same kernels as the 9B pair), each layer timed over `reps` launches."""
    import torch
    from attention_g2attn_prefill_amd import synth
    res = {}
    for name in ("2b-8k", "27b-8k"):
        cfg = synth.WORKLOADS[name]
        q, k, v = (x.to(dev) for x in synth.prefill_inputs(cfg))
        out = torch.empty_like(q)
        B, T, H, d = q.shape
        S = k.shape[1]
        kw = dict(query_scale=cfg["query_scale"], softcap=cfg["softcap"], window=cfg["window"])
        row = {"shape": {"B": B, "T": T, "S": S, "H": H, "KVH": k.shape[2], "d": d,
                         "query_scale": cfg["query_scale"], "window": cfg["window"]}}
        tot_f, tot_t = 0.0, 0.0
        for is_local in (True, False):
            warm(lambda: g2.prefill(q, k, v, is_local=is_local, out=out, stream=stream, **kw))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g2.prefill(q, k, v, is_local=is_local, out=out, stream=stream, **kw)
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / reps
            f = 4.0 * d * B * H * prefill_pairs(T, S, cfg["window"], is_local)
            tag = "local" if is_local else "global"
            row[f"{tag}_ms"] = round(t * 1e3, 4)
            row[f"{tag}_tflops"] = round(f / t / 1e12, 2)
            tot_f += f
            tot_t += t
        tf = tot_f / tot_t / 1e12
        row.update({"pair_tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                    "flops": tot_f})
        res[name] = row
        del q, k, v, out
    return res


def cpu_baseline(cfg, q, k, v, rows_per_layer):
    import numpy as np
    import oracle
    from attention_g2attn_prefill_amd import synth

    B, T, H, d = q.shape
    S = k.shape[1]
    qn, kn, vn = (synth.to_f32_numpy(x) for x in (q, k, v))
    rng = np.random.default_rng(0)
    flops, secs = 0.0, 0.0
    for is_local in (True, False):
        rows = rng.integers(0, B * T * H, size=rows_per_layer)
        t = (rows // H) % T
        p = t + (S - T)
        lo = np.maximum(0, p - cfg["window"] + 1) if is_local else np.zeros_like(p)
        flops += float(4 * d * (p - lo + 1).sum())
        t0 = time.perf_counter()
        oracle.prefill(qn, kn, vn, rows=rows, query_scale=cfg["query_scale"],
                       softcap=cfg["softcap"], window=cfg["window"], is_local=is_local)
        secs += time.perf_counter() - t0
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "host": host_description(),
            "sample": (f"{rows_per_layer} seeded random (b,t,h) rows of each layer of the "
                       f"9B 8K local+global pair, every visible key; {secs:.1f} s, "
                       f"{flops / 1e9:.0f} GFLOP counted like the GPU")}


def main():
    args = parse_args()
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.calibration_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library "
              "is single-GPU kernels and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        sys.exit("--steps must be >= 1")

    import numpy as np
    import torch
    import attention_g2attn_prefill_amd as g2
    from attention_g2attn_prefill_amd import build as g2build
    from attention_g2attn_prefill_amd import synth

    # the library must be the one built from the sources beside this script
    lib_id, src_id = g2.build_id(), g2build.source_hash()
    if lib_id != src_id:
        sys.exit(f"{g2.library_path} was built from other sources (id {lib_id}, sources "
                 f"{src_id}): run __graft_entry__.build() first")

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg_p = synth.WORKLOADS["9b-8k"]
    cfg_d = synth.WORKLOADS["9b-decode"]

    # ---- inputs, resident in HBM before timing
    q, k, v = synth.prefill_inputs(cfg_p)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out_l = torch.empty_like(qd)
    out_g = torch.empty_like(qd)
    dq, k_g, v_g, lens, k_l, v_l = synth.decode_inputs(cfg_d)
    dqd = dq.to(dev)
    kgd, vgd, kld, vld = (x.to(dev) for x in (k_g, v_g, k_l, v_l))
    del k_g, v_g, k_l, v_l
    lens_d = torch.from_numpy(lens).to(dev)
    dout_l = torch.empty_like(dqd)
    dout_g = torch.empty_like(dqd)
    B, T, H, d = q.shape
    S, KVH = k.shape[1], k.shape[2]
    DB, DS, DH, DKVH, Dd = dq.shape[0], kgd.shape[1], dq.shape[2], kgd.shape[2], dq.shape[3]
    W = cfg_p["window"]
    ws = torch.empty(g2.decode_workspace_bytes(DB, DH, Dd, DS), dtype=torch.uint8, device=dev)
    # paged cache: the global cache's 16-token blocks scattered over a pool
    PBS = 16
    maxb = DS // PBS
    gen = torch.Generator().manual_seed(16)
    perm = torch.randperm(DB * maxb, generator=gen).to(dev)
    kpool = torch.empty((DB * maxb, PBS, DKVH, Dd), dtype=kgd.dtype, device=dev)
    vpool = torch.empty_like(kpool)
    kpool[perm] = kgd.view(DB * maxb, PBS, DKVH, Dd)
    vpool[perm] = vgd.view(DB * maxb, PBS, DKVH, Dd)
    table = perm.view(DB, maxb).to(torch.int32).contiguous()
    CT = 2048
    qchunk = qd[:, T - CT:].contiguous() if T > CT else qd
    CT = qchunk.shape[1]
    cout = torch.empty_like(qchunk)
    pout_l = torch.empty_like(dqd)
    pout_g = torch.empty_like(dqd)
    pws = torch.empty(g2.decode_paged_workspace_bytes(DB, DH, Dd, maxb, PBS), dtype=torch.uint8,
                      device=dev)
    torch.cuda.synchronize()

    kw_p = dict(query_scale=cfg_p["query_scale"], softcap=cfg_p["softcap"], window=W)
    kw_d = dict(query_scale=cfg_d["query_scale"], softcap=cfg_d["softcap"],
                window=cfg_d["window"])
    stream = torch.cuda.current_stream()

    # The timed launches of one step, in order.
    launches = [
        lambda: g2.prefill(qd, kd, vd, is_local=True, out=out_l, stream=stream, **kw_p),
        lambda: g2.prefill(qd, kd, vd, is_local=False, out=out_g, stream=stream, **kw_p),
        lambda: g2.decode(dqd, kld, vld, lens_d, is_local=True, out=dout_l, workspace=ws,
                          stream=stream, **kw_d),
        lambda: g2.decode(dqd, kgd, vgd, lens_d, is_local=False, out=dout_g, workspace=ws,
                          stream=stream, **kw_d),
        lambda: g2.decode_paged(dqd, kpool, vpool, table, lens_d, is_local=True, out=pout_l,
                                workspace=pws, stream=stream, **kw_d),
        lambda: g2.decode_paged(dqd, kpool, vpool, table, lens_d, is_local=False, out=pout_g,
                                workspace=pws, stream=stream, **kw_d),
        lambda: g2.prefill(qchunk, kd, vd, is_local=True, out=cout, stream=stream, **kw_p),
        lambda: g2.prefill(qchunk, kd, vd, is_local=False, out=cout, stream=stream, **kw_p),
    ]

    def step(ev=None):
        """One pass of the hot path; ev[2i] / ev[2i+1] bracket launch i."""
        for i, launch in enumerate(launches):
            if ev is not None:
                ev[2 * i].record(stream)
            launch()
            if ev is not None:
                ev[2 * i + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(launches))]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    ms = np.array([[events[i][2 * j].elapsed_time(events[i][2 * j + 1]) for j in range(len(launches))]
                   for i in range(args.steps)])  # pl, pg, dl, dg, paged l, paged g, chunk l, chunk g
    t_pl, t_pg, t_dl, t_dg, t_ql, t_qg, t_cl, t_cg = ms.mean(axis=0) * 1e-3
    med = np.median(ms, axis=0)
    mn = ms.min(axis=0)

    adjacent = time_adjacent(g2, qd, kd, dev, stream, reps=10)
    backward = time_backward(g2, qd, kd, vd, kw_p, dev, stream, reps=5)
    models = time_models(g2, dev, stream, reps=10)
    copy_rate = copy_gbs(dev)
    gemm_rate = gemm_tflops(dev)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- algorithmic work
    f_local = 4.0 * d * B * H * prefill_pairs(T, S, W, True)
    f_global = 4.0 * d * B * H * prefill_pairs(T, S, W, False)
    prefill_tflops = (f_local + f_global) / (t_pl + t_pg) / 1e12
    bn = 32 if d > 128 else 64
    ft_local = 4.0 * d * B * H * prefill_tile_pairs(T, S, W, True, bn=bn)
    ft_global = 4.0 * d * B * H * prefill_tile_pairs(T, S, W, False, bn=bn)
    row_bytes = 2 * DKVH * Dd * 2  # K and V bytes per visible position (bf16)
    n_local = np.minimum(lens.astype(np.int64), cfg_d["window"]).sum()
    n_global = lens.astype(np.int64).sum()
    qo_bytes = 2 * DB * DH * Dd * 2
    b_local = float(n_local * row_bytes + qo_bytes)
    b_global = float(n_global * row_bytes + qo_bytes)
    decode_gbs = (b_local + b_global) / (t_dl + t_dg) / 1e9
    paged_gbs = (b_local + b_global) / (t_ql + t_qg) / 1e9
    fc_local = 4.0 * d * B * H * prefill_pairs(CT, S, W, True)
    fc_global = 4.0 * d * B * H * prefill_pairs(CT, S, W, False)
    chunk_tflops = (fc_local + fc_global) / (t_cl + t_cg) / 1e12

    src_hash = lib_id  # baked into the loaded library, equal to the sources' hash
    traffic = measured_traffic("prefill", "traffic_bytes_per_launch")
    roofline = {"bound": "mfma", "achieved": round(prefill_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(prefill_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic}
    mfma_context = {"library_bf16_gemm_tflops": round(gemm_rate, 1), "gemm_shape": [8192, 8192, 8192],
                    "prefill_frac_of_library_gemm": round(prefill_tflops / gemm_rate, 4)}
    decode = {"metric": "decode KV GB/s", "value": round(decode_gbs, 1), "unit": "GB/s",
              "frac_of_hbm_peak": round(decode_gbs / PEAK_HBM_GBS, 4),
              "roofline": {"bound": "hbm", "achieved": round(decode_gbs, 1),
                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(decode_gbs / PEAK_HBM_GBS, 4),
                           "traffic": measured_traffic("decode", "decode_split_traffic_bytes_per_launch")},
              "ms_local": round(t_dl * 1e3, 4), "ms_global": round(t_dg * 1e3, 4),
              "ms_local_median_min": [round(med[2], 4), round(mn[2], 4)],
              "ms_global_median_min": [round(med[3], 4), round(mn[3], 4)],
              "bytes_local": b_local, "bytes_global": b_global,
              "device_copy_gbs_context": round(copy_rate, 1)}
    decode_paged = {"metric": "paged decode KV GB/s", "value": round(paged_gbs, 1), "unit": "GB/s",
                    "block_size": PBS,
                    "roofline": {"bound": "hbm", "achieved": round(paged_gbs, 1),
                                 "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": round(paged_gbs / PEAK_HBM_GBS, 4),
                                 "traffic": measured_traffic("decode", "paged_split_traffic_bytes_per_launch")},
                    "ms_local": round(t_ql * 1e3, 4), "ms_global": round(t_qg * 1e3, 4),
                    "ms_local_median_min": [round(med[4], 4), round(mn[4], 4)],
                    "ms_global_median_min": [round(med[5], 4), round(mn[5], 4)]}
    per_layer = {"prefill_local_ms": round(t_pl * 1e3, 4), "prefill_global_ms": round(t_pg * 1e3, 4),
                 "prefill_local_tflops": round(f_local / t_pl / 1e12, 2),
                 "prefill_global_tflops": round(f_global / t_pg / 1e12, 2),
                 "prefill_local_ms_median_min": [round(med[0], 4), round(mn[0], 4)],
                 "prefill_global_ms_median_min": [round(med[1], 4), round(mn[1], 4)],
                 "prefill_flops_local": f_local, "prefill_flops_global": f_global,
                 "prefill_tile_level_flops_local": ft_local,
                 "prefill_tile_level_flops_global": ft_global,
                 "prefill_tile_level_tflops": round((ft_local + ft_global) / (t_pl + t_pg) / 1e12, 2)}

    cpu = None
    if args.cpu_rows > 0:
        cpu = cpu_baseline(cfg_p, q, k, v, args.cpu_rows)

    rec = {
        "metric": METRIC,
        "value": round(prefill_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the Gemma 2 9B attention layer)",
        "config": {"workload": "gemma2-9b attention: prefill local+global pair B=2 T=S=8192 "
                               "H=16 KVH=8 d=256 W=4096 cap=50; decode B=64 global "
                               "L~U[4096,8192] + local ring 4096",
                   "global_batch": B, "seq_len": T, "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "mfma_context": mfma_context,
        "decode": decode,
        "decode_paged": decode_paged,
        "adjacent": adjacent,
        "backward": backward,
        "prefill_chunk": {"metric": "chunked prefill eff. TFLOP/s", "value": round(chunk_tflops, 2),
                          "unit": "TFLOP/s", "chunk": CT, "cache": S,
                          "frac_of_bf16_peak": round(chunk_tflops / PEAK_BF16_TFLOPS, 4),
                          "ms_local": round(t_cl * 1e3, 4), "ms_global": round(t_cg * 1e3, 4),
                          "flops_local": fc_local, "flops_global": fc_global},
        "per_layer": per_layer,
        "prefill_models": models,
        "kernel_source_sha256": src_hash[:16],
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
