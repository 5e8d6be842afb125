"""Benchmark of the ReplaySSM decode hot path on one MI355X.

Default (the headline line): a step is one replay decode step (append +
output-only replay, with the fold fused into the step that fills the 16-record
window) for every sequence of one Mamba-2 layer at serving shape: batch 256,
128 heads, 64 x 128 fp32 state tiles (4 MiB per sequence), bf16 inputs.  Inputs
for every timed step are generated up front and resident in HBM before the
timed region.  The conventional read-modify-write kernel is timed on the same
inputs as the comparison point, and the fp64 CPU oracle is timed on a bounded
sample as a reported baseline.  Prints one JSON line.

Other measurements of the path (--workload):
  gdn_b256          Gated DeltaNet replay decode, B=256, 32/16 heads, 128 x 128
  m2_readcopy_b256  Mamba-2 replay decode with an fp8 or MXFP4 read copy (--read-copy)
  m2_verify_b512    speculative verify(T=4) -> commit -> flush(16), B=512 (Mamba-2)
  gdn_verify_b256   the same loop for Gated DeltaNet, B=256
  kda_b256          KDA replay decode (per-channel gates), B=256, 32 heads, 128 x 128
  kda_verify_b256   the speculative loop for KDA, B=256
  --drift           read-copy output drift against the fp32 path over 4096 decode steps
  --sweep-L         window length L in {4, 8, 16, 32}, flushes in lockstep and staggered
  --snapshot        with a verify workload: the snapshot-based speculative comparator
  --tree            with a verify workload: tree-shaped drafts, accepted path committed
  --fused           with a verify workload: verify_fold(L) -> commit (the flush fused into the verify)
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
# the sources of the headline decode kernel (Mamba-2, bf16 records staged in 16-byte chunks)
KERNEL_SOURCES = ["attention_decode_mamba_amd/csrc/rssm_device.hpp",
                  "attention_decode_mamba_amd/csrc/rssm_internal.hpp",
                  "attention_decode_mamba_amd/csrc/kind_launch.hpp",
                  "attention_decode_mamba_amd/csrc/kernels_m2_bf16.hip"]


def kernel_source_hash() -> str:
    """Hash of the kernel sources without their comments: a counter summary stays valid
    across comment edits, which do not change the compiled kernels."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update("\n".join(ln.rstrip() for ln in src.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- byte model
def _es(wl) -> int:
    return 2 if wl.in_dtype == "bf16" else 4


def _rec_bytes(wl):
    """(bytes of one record per value head: alpha (KDA: dk gates) (+beta) + v, per key head: k)."""
    s = _es(wl)
    n_alpha = wl.dk if wl.kind == "kda" else 1
    n_beta = 0 if wl.kind == "mamba2" else 1
    return s * (n_alpha + wl.dv + n_beta), s * wl.dk


def _tile_read_bytes(wl, fold: bool) -> int:
    PN = wl.dv * wl.dk
    if fold or wl.read_copy == "none":
        return 4 * PN
    return PN + PN // 8 if wl.read_copy == "fp8" else PN // 2 + PN // 32


def _copy_write_bytes(wl) -> int:
    PN = wl.dv * wl.dk
    return {"none": 0, "fp8": PN + PN // 8, "mxfp4": PN // 2 + PN // 32}[wl.read_copy]


def step_bytes(wl, h: int) -> dict:
    """Algorithmic HBM bytes of one replay decode step over the whole batch, with h records
    in the window after the append (h == L: the fold step).  Per (sequence, head) tile:
    checkpoint (or read-copy) read, on the fold step the checkpoint write (and the read-copy
    write), the h-1 older ring records (alpha, beta, v per value head; k per key head), the
    step inputs, the ring append (non-fold steps) and the fp32 output row."""
    s = _es(wl)
    B, H, G, P, N = wl.batch, wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    fold = h >= wl.L
    head_rec, key_rec = _rec_bytes(wl)
    state = B * H * _tile_read_bytes(wl, fold)
    if fold:
        state += B * H * (4 * P * N + _copy_write_bytes(wl))
    ring_read = (h - 1) * (B * H * head_rec + B * G * key_rec)
    inputs = B * H * head_rec + B * G * 2 * s * N
    append = 0 if fold else inputs
    out = B * H * 4 * P
    return dict(state=state, total=state + ring_read + inputs + append + out)


def conventional_bytes(wl) -> dict:
    s = _es(wl)
    B, H, G, P, N = wl.batch, wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    head_rec, _ = _rec_bytes(wl)
    state = 2 * B * H * 4 * P * N
    inputs = B * H * head_rec + B * G * 2 * s * N
    return dict(state=state, total=state + inputs + B * H * 4 * P)


def verify_bytes(wl, hs, T: int) -> dict:
    """One verify launch: per tile the checkpoint read, the h committed ring records, T drafts
    read and appended, T output rows.  hs: records in each sequence's window."""
    s = _es(wl)
    H, G, P, N = wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    head_rec, key_rec = _rec_bytes(wl)
    nb = len(hs)
    state = nb * H * 4 * P * N
    ring = int(sum(hs)) * (H * head_rec + G * key_rec)
    drafts = nb * T * (H * head_rec + G * 2 * s * N)
    return dict(state=state, total=state + ring + 2 * drafts + nb * T * H * 4 * P)


def flush_bytes(wl, hs_folded) -> dict:
    """One flush launch: each folding sequence reads its h ring records and reads + writes
    its checkpoint tiles."""
    H, G, P, N = wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    head_rec, key_rec = _rec_bytes(wl)
    state = len(hs_folded) * H * (8 * P * N + _copy_write_bytes(wl))
    ring = int(sum(hs_folded)) * (H * head_rec + G * key_rec)
    return dict(state=state, total=state + ring)


# ----------------------------------------------------------------------------- CPU baseline
def _oracle_worker(args):
    wl, b, steps, barrier_at = args
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)                  # one BLAS thread per worker process
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


def cpu_baseline(wl, n_seqs: int = 16, steps: int = 320) -> dict:
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
                      f"(fp64 stepwise recurrence, all {wl.n_heads} heads), {cpu:.1f} s CPU over {workers} processes",
            "wall_s": round(wall, 3)}


# ----------------------------------------------------------------------------- GPU helpers
def _to_dev(arrs, torch):
    import numpy as np
    out = {}
    for k, v in arrs.items():
        if v is None:
            out[k] = None
        else:
            a = np.ascontiguousarray(v)
            out[k] = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
    return out


def _gen_inputs(wl, steps, torch, drafts_T=0):
    """Per-step device inputs (decode records, or T drafts per sequence), generated in
    parallel over sequences and copied to HBM."""
    from synth.stream import StepSource
    out = []
    with StepSource(wl, range(wl.batch)) as src:
        for t in range(steps):
            out.append(_to_dev(src.drafts(t, drafts_T) if drafts_T else src.decode(t), torch))
    return out


def _s0_device(wl, torch):
    import numpy as np
    from concurrent.futures import ProcessPoolExecutor
    from synth import initial_state
    from synth.gen import default_workers
    chunks = [c for c in np.array_split(np.arange(wl.batch), default_workers()) if len(c)]
    s0 = torch.empty(wl.batch, wl.n_heads, wl.dv, wl.dk, dtype=torch.float32, device="cuda")
    with ProcessPoolExecutor(max_workers=len(chunks)) as ex:
        for idx, arr in zip(chunks, ex.map(initial_state, [wl] * len(chunks), [list(c) for c in chunks])):
            s0[int(idx[0]): int(idx[-1]) + 1] = torch.from_numpy(arr).cuda()
    return s0


def _p(t):
    return None if t is None else t.data_ptr()


class _Timer:
    """Elapsed time of a launch sequence on one stream (start/end events only), or an event
    pair around every launch."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def total_ms(self, fn, n):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        a.record(self.stream)
        for i in range(n):
            fn(i)
        b.record(self.stream)
        t.cuda.synchronize()
        return a.elapsed_time(b)

    def per_launch_ms(self, fns, n):
        """fns: list of callables(i); returns per-callable lists of durations."""
        t = self.torch
        ev = [[(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in fns] for _ in range(n)]
        t.cuda.synchronize()
        for i in range(n):
            for j, fn in enumerate(fns):
                ev[i][j][0].record(self.stream)
                fn(i)
                ev[i][j][1].record(self.stream)
        t.cuda.synchronize()
        return [[ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(n)] for j in range(len(fns))]


def _stream_copy_gbps(R, torch, stream, sh):
    nbytes = COPY_BYTES
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    R.rssm_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        R.rssm_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh)
    b.record(stream)
    torch.cuda.synchronize()
    return 5 * 2 * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9


# ----------------------------------------------------------------------------- decode
def window_phases(wl, n_per_layer: int, staggered: bool):
    """Records each sequence's window holds after the append, at a layer's n-th launch:
    sequence b starts with b mod L records when staggered, with none in lockstep."""
    import numpy as np
    start = np.arange(wl.batch) % wl.L if staggered else np.zeros(wl.batch, np.int64)
    return (start + n_per_layer) % wl.L + 1


def launch_bytes(wl, hs) -> dict:
    """Algorithmic bytes of one decode launch whose sequences hold hs records (after the append)."""
    import numpy as np
    one = wl.replace(batch=1)
    out = {"state": 0, "total": 0}
    for h, c in zip(*np.unique(np.asarray(hs), return_counts=True)):
        sb = step_bytes(one, int(h))
        out["state"] += int(c) * sb["state"]
        out["total"] += int(c) * sb["total"]
    return out


def stagger_windows(R, torch, wl, cfg, ds, drafts, sh):
    """Stagger the windows through the API (untimed): L - 1 rounds of verify(T=1) + commit,
    sequence b accepting its draft in the first b mod L rounds, so it starts with b mod L
    records and B / L sequences fold on every later decode step."""
    import numpy as np
    B = wl.batch
    o = torch.empty(B, 1, wl.n_heads, wl.dv, device="cuda")
    keep = []
    for r in range(wl.L - 1):
        d = drafts[r]
        R.rssm_verify(cfg, ds.st, 1, _p(d["alpha"]), _p(d["beta"]), _p(d["v"]), _p(d["k"]), _p(d["q"]),
                      o.data_ptr(), sh)
        acc = torch.from_numpy((np.arange(B) % wl.L > r).astype(np.int32)).cuda()
        keep.append(acc)
        R.rssm_commit(cfg, ds.st, acc.data_ptr(), 1, sh)
    torch.cuda.synchronize()


def run_decode(args, wl, with_conventional=True) -> dict:
    """Replay decode over `layers` independent layer instances, used round robin (launch n
    steps layer n % layers), so no layer's state or read copy is still cached when it is read
    again.

    Windows are staggered by default (sequence b starts with b mod L records), so every
    launch carries the window-average share of folds (B / L sequences fold on every step)
    and any K measures the window average; --lockstep starts every window together.  Timed:
    `reps` repetitions of K launches each, the median reported; then K more launches with an
    event pair around each (per-launch durations for the roofline).  With staggered windows
    a lockstep pass over whole windows (K rounded up to layers x L launches) gives the fold
    and non-fold step times as well."""
    import statistics
    import torch
    from attention_decode_mamba_amd import rssm as R
    from attention_decode_mamba_amd.state import DeviceState, config_of

    K, W, layers, reps = args.steps, args.warmup, max(1, args.layers), max(1, args.reps)
    staggered = not args.lockstep
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    n_in = W + K if not args.distinct else min(args.distinct, W + K)
    print(f"[bench] {wl.name}: generating inputs for {n_in} steps, {layers} layer instances, "
          f"{'staggered' if staggered else 'lockstep'} windows", file=sys.stderr, flush=True)
    t0 = time.time()
    s0 = _s0_device(wl, torch)
    inputs = _gen_inputs(wl, n_in, torch)
    drafts = _gen_inputs(wl, wl.L - 1, torch, drafts_T=1) if staggered else None
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    cfg = config_of(wl)
    states = [DeviceState(cfg) for _ in range(layers)]
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    count = [0]                                   # launches since the states were set up

    def setup(stag):
        for ds in states:
            ds.init(s0, sh)
            if stag:
                stagger_windows(R, torch, wl, cfg, ds, drafts, sh)
        count[0] = 0

    def replay(t):
        d = inputs[t % n_in]
        ds = states[count[0] % layers]
        count[0] += 1
        R.rssm_decode_step(cfg, ds.st, _p(d["alpha"]), _p(d["beta"]), _p(d["v"]), _p(d["k"]), _p(d["q"]),
                           y.data_ptr(), sh)

    def bytes_of(n, stag):                        # launch n since set-up
        return launch_bytes(wl, window_phases(wl, n // layers, stag))

    tm = _Timer(torch, stream)
    setup(staggered)
    for t in range(W):
        replay(t)
    rep_ms, rep_state, rep_total = [], [], []
    for _ in range(reps):
        n0 = count[0]
        rep_ms.append(tm.total_ms(lambda i: replay(W + i), K))
        bs = [bytes_of(n0 + i, staggered) for i in range(K)]
        rep_state.append(sum(b_["state"] for b_ in bs))
        rep_total.append(sum(b_["total"] for b_ in bs))
    med = sorted(range(reps), key=lambda r: rep_ms[r])[reps // 2]
    total_ms, alg_state, alg_total = rep_ms[med], rep_state[med], rep_total[med]
    n0 = count[0]
    (per,) = tm.per_launch_ms([lambda i: replay(W + i)], K)
    for ds in states:
        assert ds.error() == 0
    alg_launch = alg_total / K                    # the median repetition's launches
    kern_ms = sum(per)
    # the launch duration over the timed region: K back-to-back launches of the one kernel
    # (the event pairs around single launches add their own overhead, reported beside)
    achieved = alg_launch / (total_ms / K * 1e-3) / 1e9
    B = wl.batch
    res = {
        "value": B * K / (total_ms * 1e-3),
        "unit": "tokens/s",
        "ms_per_step": total_ms / K,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
                     "algorithmic_bytes_per_launch": alg_launch},
        "state_GBps": alg_state / (total_ms * 1e-3) / 1e9,
        "total_GBps": alg_total / (total_ms * 1e-3) / 1e9,
        "state_pct_of_peak": 100.0 * alg_state / (total_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "kernel_ms_per_launch": total_ms / K,
        "event_pair_ms_per_launch": kern_ms / K,
        "windows": (f"staggered: sequence b starts with b mod {wl.L} records, so {B // wl.L} of {B} "
                    f"sequences fold on every step" if staggered else "lockstep: every sequence folds on "
                    f"the same step, once per {wl.L} steps"),
        "timing": {"layers": layers, "reps": reps, "rep_ms_per_step": [m / K for m in rep_ms],
                   "median_rep": med, "spread": (max(rep_ms) - min(rep_ms)) / statistics.median(rep_ms),
                   "launch_ms_min": min(per), "launch_ms_max": max(per),
                   "distinct_input_steps": n_in},
    }

    # lockstep over whole windows: every repetition covers the same window phases
    period = layers * wl.L
    Kw = period * max(1, -(-K // period)) if staggered else (K if K % period == 0 else None)
    if Kw:
        if staggered:
            setup(False)
            for t in range(period):
                replay(t)
        lms = [tm.total_ms(lambda i: replay(i), Kw) for _ in range(reps)]
        n0 = count[0]
        (lper,) = tm.per_launch_ms([lambda i: replay(i)], Kw)
        for ds in states:
            assert ds.error() == 0
        hs = [int(window_phases(wl, (n0 + i) // layers, False)[0]) for i in range(Kw)]
        fold = [p for p, h in zip(lper, hs) if h == wl.L]
        nonfold = [p for p, h in zip(lper, hs) if h != wl.L]
        lb = [bytes_of(n0 + i, False) for i in range(Kw)]
        lms_med = statistics.median(lms)
        res["lockstep"] = {
            "ms_per_step": lms_med / Kw, "tokens_per_s": B * Kw / (lms_med * 1e-3), "launches": Kw,
            "fold_step_ms": sum(fold) / max(len(fold), 1),
            "nonfold_step_ms": sum(nonfold) / max(len(nonfold), 1),
            "state_pct_of_peak": 100.0 * sum(b_["state"] for b_ in lb) / (lms_med * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "frac": sum(b_["total"] for b_ in lb) / (sum(lper) * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "spread": (max(lms) - min(lms)) / lms_med}
    if with_conventional:
        convs = [s0.clone() for _ in range(layers)]
        ccount = [0]

        def conventional(t):
            d = inputs[t % n_in]
            conv = convs[ccount[0] % layers]
            ccount[0] += 1
            R.rssm_decode_step_conventional(cfg, conv.data_ptr(), _p(d["alpha"]), _p(d["beta"]), _p(d["v"]),
                                            _p(d["k"]), _p(d["q"]), y.data_ptr(), sh)

        for t in range(W):
            conventional(t)
        conv_ms = statistics.median(tm.total_ms(lambda i: conventional(W + i), K) for _ in range(reps))
        cb = conventional_bytes(wl)
        res["conventional"] = {"tokens_per_s": B * K / (conv_ms * 1e-3), "ms_per_step": conv_ms / K,
                               "state_GBps": cb["state"] / (conv_ms / K * 1e-3) / 1e9,
                               "total_GBps": cb["total"] / (conv_ms / K * 1e-3) / 1e9}
        res["speedup_vs_conventional"] = conv_ms / total_ms
        del convs
    res["stream_copy_GBps"] = _stream_copy_gbps(R, torch, stream, sh)
    return res


def decode_profile(wl) -> str:
    """The counter summary under profiles/ that covers decode workload wl."""
    if wl.read_copy != "none":
        return os.path.join(ROOT, "profiles",
                            f"k_decode_readcopy_{wl.read_copy}_mamba2_b256_h128_p64_n128_counters.txt")
    return {"gdn_b256": os.path.join(ROOT, "profiles", "k_decode_gdn_b256_h32_p128_n128_counters.txt"),
            "kda_b256": os.path.join(ROOT, "profiles", "k_decode_kda_b256_h32_p128_n128_counters.txt")}.get(
                wl.name, PROFILE_SUMMARY)


def decode_traffic(wl):
    """HBM traffic per launch from the counter summary of wl, if it was taken from the current
    kernel sources at this batch, workload and read-copy format; else None."""
    path = decode_profile(wl)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    if (prof.get("kernel_source_hash") != kernel_source_hash() or prof.get("batch") != wl.batch
            or prof.get("workload", WORKLOAD) != wl.name or prof.get("read_copy", "none") != wl.read_copy):
        return None
    return prof.get("traffic_bytes_per_launch")


def decode_kernel_name(wl) -> str:
    kind = {"mamba2": "mamba2", "gdn": "gdn", "kda": "kda"}[wl.kind]
    if wl.read_copy != "none":
        return f"k_decode_rc<mamba2, N={wl.dk}, read copy {wl.read_copy}>"
    return f"k_decode<{kind}, N={wl.dk}, P={wl.dv}>"


def headline(args) -> dict:
    from synth import get_workload
    wl = get_workload(WORKLOAD)
    if args.batch:
        wl = wl.replace(batch=args.batch)
    r = run_decode(args, wl)
    r["roofline"]["traffic"] = decode_traffic(wl)
    r["roofline"]["kernel"] = "k_decode<mamba2, N=128, RGW=2>"
    out = {"metric": METRIC, "value": r.pop("value"), "unit": r.pop("unit"), "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": r.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": f"mamba2_replay_decode_b{wl.batch}_h128_p64_n128_bf16in_fp32state_L16",
                      "batch": wl.batch, "heads": wl.n_heads, "dv": wl.dv, "dk": wl.dk, "window": wl.L,
                      "in_dtype": wl.in_dtype, "state_dtype": "fp32", "parallelism": "single_gpu"}}
    out.update(r)
    return out


# ----------------------------------------------------------------------------- window sweep
def run_sweep(args) -> dict:
    """Window length sweep: Mamba-2 decode at the headline shape for L in {4, 8, 16, 32}
    (ring capacity C = L), with all sequences folding on the same step (lockstep) and with
    the windows staggered so that sequence b starts with b mod L records (about B / L
    sequences fold on every step).  The stagger is set up through the API: L - 1 rounds of
    verify(T=1) + commit, sequence b accepting its draft in the first b mod L rounds."""
    import statistics
    import numpy as np
    import torch
    from attention_decode_mamba_amd import rssm as R
    from attention_decode_mamba_amd.state import DeviceState, config_of
    from synth import get_workload

    K, W, layers, reps = args.steps, args.warmup, max(1, args.layers), max(1, args.reps)
    base = get_workload(WORKLOAD)
    if args.batch:
        base = base.replace(batch=args.batch)
    B = base.batch
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    s0 = _s0_device(base, torch)
    inputs = _gen_inputs(base, W + K, torch)
    drafts = _gen_inputs(base, 31, torch, drafts_T=1)
    y = torch.empty(B, base.n_heads, base.dv, device="cuda")
    o = torch.empty(B, 1, base.n_heads, base.dv, device="cuda")
    tm = _Timer(torch, stream)
    rows = []
    for L in args.sweep_windows:
        wl = base.replace(L=L, capacity=L, t_max=1)
        cfg = config_of(wl)
        for mode in ("lockstep", "staggered"):
            states = [DeviceState(cfg) for _ in range(layers)]
            for ds in states:
                ds.init(s0, sh)
                if mode == "staggered":
                    for r in range(L - 1):
                        d = drafts[r]
                        R.rssm_verify(cfg, ds.st, 1, _p(d["alpha"]), None, _p(d["v"]), _p(d["k"]), _p(d["q"]),
                                      o.data_ptr(), sh)
                        acc = torch.from_numpy((np.arange(B) % L > r).astype(np.int32)).cuda()
                        R.rssm_commit(cfg, ds.st, acc.data_ptr(), 1, sh)
                        R.rssm_flush(cfg, ds.st, L, sh)
            start = np.arange(B) % L if mode == "staggered" else np.zeros(B, np.int64)
            count = [0]

            def replay(t):
                d = inputs[t]
                ds = states[count[0] % layers]
                count[0] += 1
                R.rssm_decode_step(cfg, ds.st, _p(d["alpha"]), None, _p(d["v"]), _p(d["k"]), _p(d["q"]),
                                   y.data_ptr(), sh)

            def launch_bytes(n):                  # algorithmic bytes of launch n, per sequence phase
                hs = (start + n // layers) % L + 1
                one = wl.replace(batch=1)
                tot = st_b = 0
                for h, c in zip(*np.unique(hs, return_counts=True)):
                    sb = step_bytes(one, int(h))
                    tot += c * sb["total"]
                    st_b += c * sb["state"]
                return tot, st_b

            for t in range(W):
                replay(t)
            rep_ms = []
            for _ in range(reps):
                rep_ms.append(tm.total_ms(lambda i: replay(W + i), K))
            n0 = count[0]
            (per,) = tm.per_launch_ms([lambda i: replay(W + i)], K)
            for ds in states:
                assert ds.error() == 0
            ms = statistics.median(rep_ms)
            byts = [launch_bytes(n0 + i) for i in range(K)]
            tot = sum(b_[0] for b_ in byts) / K
            stb = sum(b_[1] for b_ in byts) / K
            row = {"L": L, "mode": mode, "ms_per_step": ms / K, "tokens_per_s": B * K / (ms * 1e-3),
                   "kernel_ms_per_launch": sum(per) / K, "launch_ms_min": min(per), "launch_ms_max": max(per),
                   "algorithmic_GBps": tot / (sum(per) / K * 1e-3) / 1e9,
                   "frac": tot / (sum(per) / K * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                   "state_bytes_per_step": stb, "total_bytes_per_step": tot}
            print(f"[sweep] L={L} {mode}: {row['ms_per_step']:.4f} ms/step, launches "
                  f"{row['launch_ms_min']:.3f}..{row['launch_ms_max']:.3f} ms", file=sys.stderr, flush=True)
            rows.append(row)
            del states
    best = min(rows, key=lambda r: r["ms_per_step"])
    return {"metric": "replay decode window sweep (Mamba-2, B=%d H128 P64 N128 bf16 inputs)" % B,
            "rows": rows, "best": {"L": best["L"], "mode": best["mode"], "ms_per_step": best["ms_per_step"]},
            "config": {"workload": base.name, "batch": B, "layers": layers, "reps": reps, "steps": K}}


# ----------------------------------------------------------------------------- verify loop
def run_verify(args, wl, tree=False, fused=False) -> dict:
    """verify(T) -> commit(a) -> flush(L) per step; a ~ U{0..T} per sequence and step.  With
    tree: the drafts form a random tree per sequence (verify_tree), and a random node's
    root-to-node path is accepted up to a random depth (commit_tree).  With fused: the flush
    is fused into the next verify (verify_fold(L) -> commit per step)."""
    import numpy as np
    import torch
    from attention_decode_mamba_amd import rssm as R
    from attention_decode_mamba_amd.state import DeviceState, config_of
    from synth import accept_counts, draft_tree

    T = wl.t_max
    if fused:                               # the fused call keeps h + T <= C before its fold
        wl = wl.replace(capacity=wl.L + 2 * T - 1)
    K, W = args.steps, args.warmup
    distinct = min(args.distinct or 16, W + K)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    print(f"[bench] {wl.name}: generating {distinct} distinct draft steps (cycled)", file=sys.stderr, flush=True)
    s0 = _s0_device(wl, torch)
    drafts = _gen_inputs(wl, distinct, torch, drafts_T=T)
    if tree:
        trees = [draft_tree(wl, s, T) for s in range(W + K)]
        accept = [tr[2] for tr in trees]
        tree_dev = [(torch.from_numpy(tr[0]).cuda(), torch.from_numpy(tr[1]).cuda()) for tr in trees]
    else:
        accept = [accept_counts(wl, s, T) for s in range(W + K)]
    accept_dev = [torch.from_numpy(a).cuda() for a in accept]
    cfg = config_of(wl)
    ds = DeviceState(cfg)
    ds.init(s0, sh)
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")

    def verify(s):
        d = drafts[s % distinct]
        if fused:
            R.rssm_verify_fold(cfg, ds.st, wl.L, T, tree_dev[s][0].data_ptr() if tree else None, _p(d["alpha"]),
                               _p(d["beta"]), _p(d["v"]), _p(d["k"]), _p(d["q"]), o.data_ptr(), sh)
        elif tree:
            R.rssm_verify_tree(cfg, ds.st, T, tree_dev[s][0].data_ptr(), _p(d["alpha"]), _p(d["beta"]), _p(d["v"]),
                               _p(d["k"]), _p(d["q"]), o.data_ptr(), sh)
        else:
            R.rssm_verify(cfg, ds.st, T, _p(d["alpha"]), _p(d["beta"]), _p(d["v"]), _p(d["k"]), _p(d["q"]),
                          o.data_ptr(), sh)

    def commit(s):
        if tree:
            R.rssm_commit_tree(cfg, ds.st, tree_dev[s][0].data_ptr(), tree_dev[s][1].data_ptr(),
                               accept_dev[s].data_ptr(), T, sh)
        else:
            R.rssm_commit(cfg, ds.st, accept_dev[s].data_ptr(), T, sh)

    def flush(s):
        if not fused:
            R.rssm_flush(cfg, ds.st, wl.L, sh)

    def step(s):
        verify(s)
        commit(s)
        flush(s)

    # host-side cursor bookkeeping for the byte counts (the same integer policy as the kernels)
    # hist[s] = (records each window holds at verify s, records of the windows folded at step s)
    h = np.zeros(wl.batch, np.int64)
    hist = []
    for s in range(W + K):
        if fused:                          # the fold of the last commit happens in this verify
            folded = h >= wl.L
            hist.append((h.copy(), h[folded].copy()))
            h[folded] = 0
            h = h + accept[s]
        else:
            h_before = h.copy()
            h = h + accept[s]
            folded = h >= wl.L
            hist.append((h_before, h[folded].copy()))
            h[folded] = 0

    tm = _Timer(torch, stream)
    for s in range(W):
        step(s)
    total_ms = tm.total_ms(lambda i: step(W + i), K)
    assert ds.error() == 0
    committed = int(sum(int(accept[W + i].sum()) for i in range(K)))
    # per-kernel durations on a second pass over the same steps (cursor restarted)
    ds.init(s0, sh)
    for s in range(W):
        step(s)
    if fused:
        pv, pc = tm.per_launch_ms([lambda i: verify(W + i), lambda i: commit(W + i)], K)
        pf = [0.0] * K
    else:
        pv, pc, pf = tm.per_launch_ms([lambda i: verify(W + i), lambda i: commit(W + i), lambda i: flush(W + i)], K)
    assert ds.error() == 0
    vb = [verify_bytes(wl, hist[W + i][0], T) for i in range(K)]
    fb = [flush_bytes(wl, hist[W + i][1]) for i in range(K)]
    if fused:
        # the verify reads each tile and the folding windows' records anyway: the fold adds
        # the checkpoint (and read-copy) writes of the folding tiles
        for i in range(K):
            nf = len(hist[W + i][1]) * wl.n_heads
            vb[i] = {k: v + nf * (4 * wl.dv * wl.dk + _copy_write_bytes(wl)) for k, v in vb[i].items()}
            fb[i] = {"state": 0, "total": 0}
    v_ach = sum(b["total"] for b in vb) / (sum(pv) * 1e-3) / 1e9
    f_ach = (sum(b["total"] for b in fb) / (sum(pf) * 1e-3) / 1e9) if not fused else None
    copy_gbps = _stream_copy_gbps(R, torch, stream, sh)
    return {
        "stream_copy_GBps": copy_gbps,
        "metric": (f"speculative {'tree ' if tree else ''}" +
                   ("verify_fold->commit" if fused else "verify->commit->flush") +
                   f", committed tokens/s ({wl.name}, T={T})"),
        "value": committed / (total_ms * 1e-3), "unit": "committed tokens/s",
        "ms_per_step": total_ms / K, "steps": K, "warmup": W, "data": "synthetic",
        "draft_inputs": (f"{distinct} distinct draft batches cycled; " +
                         ("random recursive draft trees, a random node's path accepted to a uniform depth"
                          if tree else f"accepted prefix ~ U{{0..{T}}} per step")),
        "mean_accept": committed / (K * wl.batch),
        "verify": {"ms": sum(pv) / K, "GBps": v_ach, "frac": v_ach / PEAK_HBM_GBPS,
                   "bytes_per_launch": sum(b["total"] for b in vb) / K},
        "commit": {"ms": sum(pc) / K},
        "flush": {"ms": sum(pf) / K, "GBps": f_ach, "frac": f_ach / PEAK_HBM_GBPS if f_ach else None,
                  "bytes_per_launch": sum(b["total"] for b in fb) / K,
                  "sequences_folded_per_step": sum(len(hist[W + i][1]) for i in range(K)) / K},
        "roofline": {"bound": "hbm", "kernel": "k_verify", "achieved": v_ach, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": v_ach / PEAK_HBM_GBPS},
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.n_heads, "qk_heads": wl.n_qk_heads,
                   "dv": wl.dv, "dk": wl.dk, "T": T, "window": wl.L, "capacity": wl.capacity},
    }


def snapshot_verify_bytes(wl, T: int) -> dict:
    """One snapshot-verify launch: per tile one state read and T state writes, T drafts read,
    T output rows."""
    s = _es(wl)
    B, H, G, P, N = wl.batch, wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    head_rec, _ = _rec_bytes(wl)
    state = B * H * 4 * P * N * (1 + T)
    drafts = B * T * (H * head_rec + G * 2 * s * N)
    return dict(state=state, total=state + drafts + B * T * H * 4 * P)


def run_verify_snapshot(args, wl) -> dict:
    """The snapshot-based speculative comparator: verify_snapshot(T) -> commit_snapshot(a) per
    step, on the same drafts and acceptance counts as the replay loop."""
    import torch
    from attention_decode_mamba_amd import rssm as R
    from attention_decode_mamba_amd.state import config_of
    from synth import accept_counts

    T = wl.t_max
    K, W = args.steps, args.warmup
    distinct = min(args.distinct or 16, W + K)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    s0 = _s0_device(wl, torch)
    drafts = _gen_inputs(wl, distinct, torch, drafts_T=T)
    accept_dev = [torch.from_numpy(accept_counts(wl, s, T)).cuda() for s in range(W + K)]
    cfg = config_of(wl)
    snap = torch.empty(wl.batch, T + 1, wl.n_heads, wl.dv, wl.dk, device="cuda")
    snap[:, 0] = s0
    del s0
    cur = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")

    def verify(s):
        d = drafts[s % distinct]
        R.rssm_verify_snapshot(cfg, snap.data_ptr(), cur.data_ptr(), T, _p(d["alpha"]), _p(d["beta"]), _p(d["v"]),
                               _p(d["k"]), _p(d["q"]), o.data_ptr(), err.data_ptr(), sh)

    def commit(s):
        R.rssm_commit_snapshot(cfg, cur.data_ptr(), accept_dev[s].data_ptr(), T, err.data_ptr(), sh)

    tm = _Timer(torch, stream)
    for s in range(W):
        verify(s)
        commit(s)
    total_ms = tm.total_ms(lambda i: (verify(W + i), commit(W + i)), K)
    pv, pc = tm.per_launch_ms([lambda i: verify(W + i), lambda i: commit(W + i)], K)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    committed = int(sum(int(accept_dev[W + i].sum().item()) for i in range(K)))
    vb = snapshot_verify_bytes(wl, T)
    v_ach = vb["total"] / (sum(pv) / K * 1e-3) / 1e9
    copy_gbps = _stream_copy_gbps(R, torch, stream, sh)
    return {
        "stream_copy_GBps": copy_gbps,
        "metric": f"snapshot-based speculative verify->commit, committed tokens/s ({wl.name}, T={T})",
        "value": committed / (total_ms * 1e-3), "unit": "committed tokens/s",
        "ms_per_step": total_ms / K, "steps": K, "warmup": W, "data": "synthetic",
        "mean_accept": committed / (K * wl.batch),
        "verify": {"ms": sum(pv) / K, "GBps": v_ach, "frac": v_ach / PEAK_HBM_GBPS,
                   "bytes_per_launch": vb["total"], "state_bytes_per_launch": vb["state"]},
        "commit": {"ms": sum(pc) / K},
        "roofline": {"bound": "hbm", "kernel": "k_verify_snapshot", "achieved": v_ach, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": v_ach / PEAK_HBM_GBPS},
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.n_heads, "qk_heads": wl.n_qk_heads,
                   "dv": wl.dv, "dk": wl.dk, "T": T, "snapshots_per_sequence": T + 1},
    }


# ----------------------------------------------------------------------------- read-copy drift
def run_drift(args) -> dict:
    """Output drift of the fp8 / MXFP4 read copy against the fp32 path on the same inputs:
    normwise relative error per output vector, per 256-step bin, over the decode steps."""
    import numpy as np
    import torch
    from attention_decode_mamba_amd import rssm as R
    from attention_decode_mamba_amd.state import DeviceState, config_of
    from synth import get_workload
    from synth.stream import StepSource

    steps = args.drift_steps
    wl = get_workload("m2_readcopy_b256").replace(batch=args.drift_batch)
    torch.cuda.set_device(0)
    sh = torch.cuda.current_stream().cuda_stream
    s0 = _s0_device(wl, torch)
    states = {}
    for fmt in ("none", "fp8", "mxfp4"):
        ds = DeviceState(config_of(wl.replace(read_copy=fmt)))
        ds.init(s0, sh)
        states[fmt] = ds
    ys = {f: torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda") for f in states}
    bins = {f: [] for f in ("fp8", "mxfp4")}
    cur = {f: [] for f in ("fp8", "mxfp4")}
    with StepSource(wl, range(wl.batch)) as src:
        for t in range(steps):
            d = _to_dev(src.decode(t), torch)
            for f, ds in states.items():
                R.rssm_decode_step(ds.cfg, ds.st, _p(d["alpha"]), None, _p(d["v"]), _p(d["k"]), _p(d["q"]),
                                   ys[f].data_ptr(), sh)
            ref = ys["none"].double()
            den = ref.abs().amax(dim=-1).clamp_min(1e-30)
            for f in ("fp8", "mxfp4"):
                e = (ys[f].double() - ref).abs().amax(dim=-1) / den
                cur[f].append((float(e.mean()), float(e.max())))
            if (t + 1) % 256 == 0:
                for f in ("fp8", "mxfp4"):
                    arr = np.array(cur[f])
                    bins[f].append({"steps": [t - 255, t], "mean": float(arr[:, 0].mean()),
                                    "max": float(arr[:, 1].max())})
                    cur[f] = []
                print(f"[drift] step {t + 1}/{steps}", file=sys.stderr, flush=True)
    for ds in states.values():
        assert ds.error() == 0
    out = {"metric": "read-copy output drift vs the fp32 path (normwise relative error per output vector)",
           "config": {"workload": wl.name, "batch": wl.batch, "steps": steps, "window": wl.L}}
    for f in ("fp8", "mxfp4"):
        means = np.array([b["mean"] for b in bins[f]])
        x = np.arange(len(means))
        slope = float(np.polyfit(x, means, 1)[0]) if len(means) > 1 else 0.0
        out[f] = {"bins": bins[f], "mean_of_means": float(means.mean()),
                  "fitted_slope_per_bin": slope, "slope_over_mean": slope / float(means.mean())}
    return out


# ----------------------------------------------------------------------------- counters
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


def summarize_counters(fetch_csv, write_csv, out_path, command, wl, bench_json, steps, warmup, layers, reps):
    """Per-launch HBM traffic of the kernels of one bench run from two rocprofv3 --pmc runs
    of it (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by what the same
    counter reads for the streaming copy of COPY_BYTES bytes that every bench run ends with.

    Which dispatches are averaged, and against which algorithmic bytes:
    * decode workloads: the launches of the staggered windows (the first warmup + (reps + 1)
      * steps decode dispatches; the lockstep pass follows them), whose algorithmic bytes are
      the same for every launch; the conventional kernel: every dispatch.
    * speculative loops: the last `steps` dispatches of verify, commit and flush (the pass
      with per-launch events, whose mean algorithmic bytes the bench line reports).
    * the snapshot comparator: every dispatch (the same bytes each launch).
    Per token: decode per sequence-step; speculative per committed token."""
    with open(bench_json) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    res = {"kernel_source_hash": kernel_source_hash(), "workload": wl.name, "batch": wl.batch,
           "read_copy": wl.read_copy, "command": command, "steps": steps, "warmup": warmup, "layers": layers,
           "reps": reps}
    fetch = _read_counter_csv(fetch_csv)
    write = _read_counter_csv(write_csv)

    def per_kernel(table, counter, key):               # in dispatch order
        rows = sorted(((int(d), n, c) for d, (n, c) in table.items() if d is not None), key=lambda r: r[0])
        return [c.get(counter, 0.0) for _, n, c in rows if key in n]

    cf = per_kernel(fetch, "FETCH_SIZE", "k_stream_copy")
    cw = per_kernel(write, "WRITE_SIZE", "k_stream_copy")
    known_kib = COPY_BYTES / 1024.0
    ff = known_kib / (sum(cf) / len(cf))
    fw = known_kib / (sum(cw) / len(cw))
    res["copy_calibration"] = {"bytes": COPY_BYTES, "fetch_kib_mean": sum(cf) / len(cf),
                               "write_kib_mean": sum(cw) / len(cw), "fetch_scale": ff, "write_scale": fw,
                               "dispatches": len(cf)}
    B = wl.batch
    if "verify" not in bench:                                          # decode
        alg = launch_bytes(wl, window_phases(wl, 0, True))
        picks = [("k_decode", "replay_decode", slice(0, warmup + (reps + 1) * steps), alg["total"], B),
                 ("k_conventional", "conventional", slice(None), conventional_bytes(wl)["total"], B)]
        res["algorithmic_state_bytes_per_launch"] = alg["state"]
    elif bench["roofline"]["kernel"] == "k_verify_snapshot":
        per_tok = bench["mean_accept"] * B
        picks = [("k_verify_snapshot", "verify_snapshot", slice(None), bench["verify"]["bytes_per_launch"], per_tok),
                 ("k_commit_snapshot", "commit_snapshot", slice(None), None, per_tok)]
    else:
        per_tok = bench["mean_accept"] * B
        picks = [("k_verify", "verify", slice(-steps, None), bench["verify"]["bytes_per_launch"], per_tok),
                 ("k_commit_tree" if "tree" in bench["metric"] else "k_commit", "commit", slice(-steps, None), None,
                  per_tok),
                 ("k_flush", "flush", slice(-steps, None), bench["flush"]["bytes_per_launch"], per_tok)]
    for key, label, sl, alg_b, per in picks:
        f = per_kernel(fetch, "FETCH_SIZE", key)[sl]
        w = per_kernel(write, "WRITE_SIZE", key)[sl]
        if not f or not w:
            continue
        fb = sum(f) / len(f) * 1024.0 * ff
        wb = sum(w) / len(w) * 1024.0 * fw
        ent = {"kernel": key, "dispatches": len(f), "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
               "traffic_bytes_per_launch": fb + wb, "fetch_bytes_per_token": fb / per,
               "write_bytes_per_token": wb / per, "traffic_bytes_per_token": (fb + wb) / per}
        if alg_b:
            ent["algorithmic_bytes_per_launch"] = alg_b
            ent["traffic_over_algorithmic"] = (fb + wb) / alg_b
        res[label] = ent
    res["per_token"] = "per sequence-step" if "verify" not in bench else "per committed token"
    if "replay_decode" in res:                 # the keys the headline bench line reads
        res["algorithmic_bytes_per_launch"] = res["replay_decode"]["algorithmic_bytes_per_launch"]
        res["traffic_bytes_per_launch"] = res["replay_decode"]["traffic_bytes_per_launch"]
        res["traffic_over_algorithmic"] = res["replay_decode"]["traffic_over_algorithmic"]
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--batch", type=int, default=0, help="override the batch of the headline workload")
    ap.add_argument("--layers", type=int, default=4, help="layer instances used round robin (decode workloads)")
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions of K steps; the median is reported")
    ap.add_argument("--lockstep", action="store_true",
                    help="decode workloads: start every window together instead of staggered")
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=[WORKLOAD, "gdn_b256", "kda_b256", "m2_readcopy_b256", "m2_verify_b512",
                             "gdn_verify_b256", "kda_verify_b256"])
    ap.add_argument("--read-copy", default="fp8", choices=["fp8", "mxfp4"])
    ap.add_argument("--distinct", type=int, default=0,
                    help="distinct input batches, cycled (0: every step distinct for decode, 16 for verify)")
    ap.add_argument("--tree", action="store_true", help="verify workloads: tree-shaped drafts (verify_tree/commit_tree)")
    ap.add_argument("--fused", action="store_true", help="verify workloads: flush fused into the next verify")
    ap.add_argument("--snapshot", action="store_true",
                    help="verify workloads: time the snapshot-based comparator instead of the replay loop")
    ap.add_argument("--drift", action="store_true", help="read-copy drift report and exit")
    ap.add_argument("--sweep-L", action="store_true", help="window length sweep (lockstep and staggered) and exit")
    ap.add_argument("--sweep-windows", type=int, nargs="+", default=[4, 8, 16, 32])
    ap.add_argument("--drift-steps", type=int, default=4096)
    ap.add_argument("--drift-batch", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-only", action="store_true")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the counter summary of the bench run with these arguments (two rocprofv3 "
                         "--pmc runs of it) and exit")
    ap.add_argument("--counter-bench", help="the JSON line the FETCH_SIZE run printed (with --summarize-counters)")
    ap.add_argument("--counter-out", default=PROFILE_SUMMARY, help="where the counter summary goes")
    ap.add_argument("--counter-command", default="", help="command recorded in the counter summary")
    args = ap.parse_args()
    if args.summarize_counters:
        from synth import get_workload
        name = {"m2_verify_b512": "m2_verify_b512", "gdn_verify_b256": "gdn_b256",
                "kda_verify_b256": "kda_b256"}.get(args.workload, args.workload)
        wl = get_workload(name)
        if args.batch:
            wl = wl.replace(batch=args.batch)
        if args.workload == "m2_readcopy_b256":
            wl = wl.replace(read_copy=args.read_copy)
        r = summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.counter_out,
                               args.counter_command, wl, args.counter_bench, args.steps, args.warmup,
                               args.layers, args.reps)
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
    if args.drift:
        print(json.dumps(run_drift(args)))
        return
    if args.sweep_L:
        print(json.dumps(run_sweep(args)))
        return
    if args.workload == WORKLOAD:
        res = headline(args)
        if not args.no_cpu_baseline:
            print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
            res["cpu_baseline"] = cpu_baseline(get_workload(WORKLOAD))
        else:
            res["cpu_baseline"] = None
        print(json.dumps(res))
        return
    if args.workload in ("m2_verify_b512", "gdn_verify_b256", "kda_verify_b256"):
        wl = get_workload({"m2_verify_b512": "m2_verify_b512", "gdn_verify_b256": "gdn_b256",
                           "kda_verify_b256": "kda_b256"}[args.workload])
        res = (run_verify_snapshot(args, wl) if args.snapshot
               else run_verify(args, wl, tree=args.tree, fused=args.fused))
    else:
        wl = get_workload(args.workload)
        if args.workload == "m2_readcopy_b256":
            wl = wl.replace(read_copy=args.read_copy)
        res = run_decode(args, wl)
        res["roofline"]["traffic"] = decode_traffic(wl)
        res["roofline"]["kernel"] = decode_kernel_name(wl)
        res["metric"] = f"replay decode tokens/s ({wl.name}, read copy {wl.read_copy})"
        res["config"] = {"workload": wl.name, "batch": wl.batch, "heads": wl.n_heads, "qk_heads": wl.n_qk_heads,
                         "dv": wl.dv, "dk": wl.dk, "window": wl.L, "read_copy": wl.read_copy}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
