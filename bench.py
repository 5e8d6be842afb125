"""Benchmark of the ReplaySSM decode hot path on one MI355X.

A step is one replay decode step (append + output-only replay, with the fold
fused into the step that fills the 16-record window) for every sequence of one
Mamba-2 layer at serving shape: batch 256, 128 heads, 64 x 128 fp32 state tiles
(4 MiB per sequence), bf16 inputs.  Inputs for every timed step are generated
up front and resident in HBM before the timed region.  The conventional
read-modify-write kernel is timed on the same inputs as the comparison point,
and the fp64 CPU oracle is timed on a bounded sample as a reported baseline.

Prints one JSON line (see the keys at the end of main()).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
METRIC = "SSM decode tokens/s + effective HBM GB/s (% of peak), B=256 H128 P64 N128 fp32"
WORKLOAD = "m2_decode_b256"
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "k_decode_mamba2_b256_h128_p64_n128_counters.txt")
COPY_BYTES = 1 << 30            # size of each calibration copy (read and written)
KERNEL_SOURCES = ["attention_decode_mamba_amd/csrc/rssm_device.hpp",
                  "attention_decode_mamba_amd/csrc/kernels_m2.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- byte model
def step_bytes(wl, h: int) -> dict:
    """Algorithmic HBM bytes of one replay decode step over the whole batch, with h records
    in the window after the append (h == L: the fold step).  Per (sequence, head) tile:
    checkpoint read 4PN (+ write 4PN on the fold step), the h-1 older ring records
    (alpha, v per head; k per key head), the step inputs, the ring append (non-fold steps)
    and the fp32 output row."""
    s = 2 if wl.in_dtype == "bf16" else 4
    B, H, G, P, N = wl.batch, wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    gdn = wl.kind == "gdn"
    flush = h >= wl.L
    head_rec = s * (1 + P + (1 if gdn else 0))          # alpha (+beta) + v per value head
    key_rec = s * N                                      # k per key head (ring reads need no q)
    state_read = B * H * 4 * P * N
    state_write = B * H * 4 * P * N if flush else 0
    ring_read = (h - 1) * (B * H * head_rec + B * G * key_rec)
    inputs = B * H * head_rec + B * G * 2 * s * N
    append = 0 if flush else inputs
    out = B * H * 4 * P
    total = state_read + state_write + ring_read + inputs + append + out
    return dict(state=state_read + state_write, total=total)


def conventional_bytes(wl) -> dict:
    s = 2 if wl.in_dtype == "bf16" else 4
    B, H, G, P, N = wl.batch, wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    state = 2 * B * H * 4 * P * N
    inputs = B * H * s * (1 + P) + B * G * 2 * s * N
    return dict(state=state, total=state + inputs + B * H * 4 * P)


# ----------------------------------------------------------------------------- CPU baseline
def _oracle_worker(args):
    wl, b, steps, barrier_at = args
    import numpy as np  # noqa: F401
    from oracle import ReplayOracle
    from synth import decode_inputs, initial_state
    inps = [decode_inputs(wl, t, [b]) for t in range(steps)]
    orc = ReplayOracle(wl, [b], initial_state(wl, [b]))
    while time.time() < barrier_at:
        time.sleep(0.001)
    t0 = time.time()
    for x in inps:
        orc.decode(x)
    return t0, time.time()


def cpu_baseline(wl, n_seqs: int = 16, steps: int = 64) -> dict:
    """The fp64 oracle on a bounded sample: n_seqs sequences x steps decode steps, one
    sequence per worker process, all starting together; tokens/s = n_seqs*steps / wall."""
    from concurrent.futures import ProcessPoolExecutor
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    workers = max(1, min(16, cores, n_seqs))
    start_at = time.time() + 5.0
    with ProcessPoolExecutor(max_workers=workers) as ex:
        spans = list(ex.map(_oracle_worker, [(wl, b, steps, start_at) for b in range(n_seqs)]))
    wall = max(e for _, e in spans) - min(s for s, _ in spans)
    cpu = sum(e - s for s, e in spans)
    return {"value": n_seqs * steps / wall, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{n_seqs} sequences x {steps} decode steps of the same workload "
                      f"(fp64 stepwise recurrence, all 128 heads), {cpu:.1f} s CPU over {workers} processes",
            "wall_s": round(wall, 3)}


# ----------------------------------------------------------------------------- GPU run
def _gen_inputs(wl, steps, torch):
    """Per-step device inputs, generated in parallel over sequences and copied to HBM."""
    import numpy as np
    from synth.stream import StepSource
    out = []
    with StepSource(wl, range(wl.batch)) as src:
        for t in range(steps):
            d = src.decode(t)
            out.append({k: (torch.from_numpy(np.ascontiguousarray(v).view(np.int16) if v.dtype == np.uint16
                                              else np.ascontiguousarray(v)).cuda()
                            if v is not None else None) for k, v in d.items()})
    return out


def _s0_device(wl, torch):
    import numpy as np
    from concurrent.futures import ProcessPoolExecutor
    from synth import initial_state
    from synth.gen import default_workers
    chunks = np.array_split(np.arange(wl.batch), default_workers())
    s0 = torch.empty(wl.batch, wl.n_heads, wl.dv, wl.dk, dtype=torch.float32, device="cuda")
    with ProcessPoolExecutor(max_workers=len(chunks)) as ex:
        for idx, arr in zip(chunks, ex.map(initial_state, [wl] * len(chunks), [list(c) for c in chunks])):
            if len(idx):
                s0[int(idx[0]): int(idx[-1]) + 1] = torch.from_numpy(arr).cuda()
    return s0


def run(args) -> dict:
    import torch
    from attention_decode_mamba_amd import rssm as R
    from attention_decode_mamba_amd.state import DeviceState, config_of
    from synth import get_workload

    wl = get_workload(WORKLOAD)
    if args.batch:
        wl = wl.replace(batch=args.batch)
    K, W = args.steps, args.warmup
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    print(f"[bench] generating inputs for {W + K} steps", file=sys.stderr, flush=True)
    t0 = time.time()
    s0 = _s0_device(wl, torch)
    inputs = _gen_inputs(wl, W + K, torch)
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    cfg = config_of(wl)
    ds = DeviceState(cfg)
    ds.init(s0, sh)
    conv = s0.clone()
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")

    def replay(t):
        d = inputs[t]
        R.rssm_decode_step(cfg, ds.st, d["alpha"].data_ptr(), None, d["v"].data_ptr(), d["k"].data_ptr(),
                           d["q"].data_ptr(), y.data_ptr(), sh)

    def conventional(t):
        d = inputs[t]
        R.rssm_decode_step_conventional(cfg, conv.data_ptr(), d["alpha"].data_ptr(), None, d["v"].data_ptr(),
                                        d["k"].data_ptr(), d["q"].data_ptr(), y.data_ptr(), sh)

    def timed(fn, first, per_launch):
        """Elapsed ms of K launches (start/end events only), or per-launch durations."""
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if not per_launch:
            torch.cuda.synchronize()
            start.record(stream)
            for i in range(K):
                fn(first + i)
            end.record(stream)
            torch.cuda.synchronize()
            return start.elapsed_time(end), None
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            ev[i][0].record(stream)
            fn(first + i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return None, [a.elapsed_time(b) for a, b in ev]

    # timed region: K steps bracketed by synchronisation, no events in between
    for t in range(W):
        replay(t)
    total_ms, _ = timed(replay, W, False)
    # the same K launches again (same window phases) with an event pair around each launch
    _, per = timed(lambda t: replay(W + (t - W) % K), W + K, True)
    assert ds.error() == 0
    for t in range(W):
        conventional(t)
    conv_ms, _ = timed(conventional, W, False)

    # exact algorithmic bytes: launch i of the timed region sits at window phase
    # h = ((W + i) % L) + 1 records after the append; the per-launch pass continues at W + K
    hs1 = [((W + i) % wl.L) + 1 for i in range(K)]
    alg_total = sum(step_bytes(wl, h)["total"] for h in hs1)
    alg_state = sum(step_bytes(wl, h)["state"] for h in hs1)
    hs = [((W + K + i) % wl.L) + 1 for i in range(K)]
    alg_launch = sum(step_bytes(wl, h)["total"] for h in hs) / K
    kern_ms = sum(per)
    fold = [p for p, h in zip(per, hs) if h == wl.L]
    nonfold = [p for p, h in zip(per, hs) if h != wl.L]
    cb = conventional_bytes(wl)

    # achievable bandwidth of a plain streaming copy (context for the roofline fraction)
    nbytes = COPY_BYTES
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    R.rssm_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh)
    cs, ce = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cs.record(stream)
    for _ in range(5):
        R.rssm_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh)
    ce.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * nbytes / (cs.elapsed_time(ce) * 1e-3) / 1e9
    del src, dst

    B = wl.batch
    avg_launch_s = kern_ms / K * 1e-3
    achieved = alg_launch / avg_launch_s / 1e9
    traffic = None
    if os.path.exists(PROFILE_SUMMARY):
        with open(PROFILE_SUMMARY) as f:
            prof = json.load(f)
        if prof.get("kernel_source_hash") == kernel_source_hash() and prof.get("batch") == B:
            traffic = prof.get("traffic_bytes_per_launch")
    res = {
        "metric": METRIC,
        "value": B * K / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": total_ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"mamba2_replay_decode_b{B}_h128_p64_n128_bf16in_fp32state_L16",
                   "batch": B, "heads": wl.n_heads, "dv": wl.dv, "dk": wl.dk, "window": wl.L,
                   "in_dtype": wl.in_dtype, "state_dtype": "fp32", "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "kernel": "k_decode<mamba2, N=128, RGW=2>",
                     "algorithmic_bytes_per_launch": alg_launch},
        "state_GBps": alg_state / (total_ms * 1e-3) / 1e9,
        "total_GBps": alg_total / (total_ms * 1e-3) / 1e9,
        "state_pct_of_peak": 100.0 * alg_state / (total_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "kernel_ms_per_launch": kern_ms / K,
        "fold_step_ms": sum(fold) / max(len(fold), 1),
        "nonfold_step_ms": sum(nonfold) / max(len(nonfold), 1),
        "conventional": {"tokens_per_s": B * K / (conv_ms * 1e-3), "ms_per_step": conv_ms / K,
                         "state_GBps": cb["state"] / (conv_ms / K * 1e-3) / 1e9,
                         "total_GBps": cb["total"] / (conv_ms / K * 1e-3) / 1e9},
        "speedup_vs_conventional": conv_ms / total_ms,
        "stream_copy_GBps": copy_gbps,
    }
    return res


def _read_counter_csv(path):
    """rocprofv3 counter_collection CSV -> {dispatch_id: (kernel_name, {counter: value})}."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            did = row.get("Dispatch_Id") or row.get("Correlation_Id")
            name = row.get("Kernel_Name", "")
            cn = row.get("Counter_Name")
            val = float(row.get("Counter_Value") or 0.0)
            ent = out.setdefault(did, (name, {}))
            ent[1][cn] = ent[1].get(cn, 0.0) + val
    return out


def summarize_counters(fetch_csv, write_csv, out_path, command, batch, steps):
    """Per-launch HBM traffic of the decode and conventional kernels from two --pmc runs
    (FETCH_SIZE, WRITE_SIZE in KiB per dispatch), each scaled by what the same counter
    reads for the streaming copy of COPY_BYTES bytes."""
    from synth import get_workload
    wl = get_workload(WORKLOAD).replace(batch=batch)
    res = {"kernel_source_hash": kernel_source_hash(), "batch": batch, "command": command}
    fetch = _read_counter_csv(fetch_csv)
    write = _read_counter_csv(write_csv)

    def per_kernel(table, counter, key):
        vals = [c.get(counter, 0.0) for n, c in table.values() if key in n]
        return vals

    cf = per_kernel(fetch, "FETCH_SIZE", "k_stream_copy")
    cw = per_kernel(write, "WRITE_SIZE", "k_stream_copy")
    known_kib = COPY_BYTES / 1024.0
    ff = known_kib / (sum(cf) / len(cf))
    fw = known_kib / (sum(cw) / len(cw))
    res["copy_calibration"] = {"bytes": COPY_BYTES, "fetch_kib_mean": sum(cf) / len(cf),
                               "write_kib_mean": sum(cw) / len(cw), "fetch_scale": ff, "write_scale": fw,
                               "dispatches": len(cf)}
    for key, label in (("k_decode", "replay_decode"), ("k_conventional", "conventional")):
        f = per_kernel(fetch, "FETCH_SIZE", key)
        w = per_kernel(write, "WRITE_SIZE", key)
        if not f or not w:
            continue
        fb = sum(f) / len(f) * 1024.0 * ff
        wb = sum(w) / len(w) * 1024.0 * fw
        res[label] = {"dispatches": len(f), "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                      "fetch_bytes_per_token": fb / batch, "write_bytes_per_token": wb / batch,
                      "write_mib_per_dispatch_min_max": [min(w) / 1024.0 * fw, max(w) / 1024.0 * fw]}
    W = 16
    hs = [((W + i) % wl.L) + 1 for i in range(steps)]
    alg = sum(step_bytes(wl, h)["total"] for h in hs) / steps
    res["algorithmic_bytes_per_launch"] = alg
    if "replay_decode" in res:
        r = res["replay_decode"]
        res["traffic_bytes_per_launch"] = r["fetch_bytes_per_launch"] + r["write_bytes_per_launch"]
        res["traffic_over_algorithmic"] = res["traffic_bytes_per_launch"] / alg
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--batch", type=int, default=0, help="override the batch (default: 256)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-only", action="store_true")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the counter summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--counter-command", default="", help="command recorded in the counter summary")
    args = ap.parse_args()
    if args.summarize_counters:
        r = summarize_counters(args.summarize_counters[0], args.summarize_counters[1], PROFILE_SUMMARY,
                               args.counter_command, args.batch or 256, args.steps)
        print(json.dumps(r, indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the decode path shards over "
                                   "sequences/heads with no exchange, so N GPUs run N independent copies"}))
        sys.exit(2)
    from synth import get_workload
    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline(get_workload(WORKLOAD))))
        return
    res = run(args)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(get_workload(WORKLOAD))
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


if __name__ == "__main__":
    main()
