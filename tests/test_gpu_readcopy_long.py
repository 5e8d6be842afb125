"""Low-precision read copy over a long decode at serving shape, against the fp64 oracle.

Mamba-2, batch 256, 128 heads, 64 x 128 fp32 checkpoint tiles, bf16 inputs, L = 16,
4096 decode steps (256 folds), with an fp8 E4M3 copy and with an MXFP4 copy of the
checkpoint written at every fold and read by every non-flush step (page 1, section on
what got faster, low-precision paragraph; page 4 "What shipped", quantisation
paragraph).  The GPU runs the whole batch in the launch configuration the benchmark
times; three states step side by side on the same inputs: without a copy, with the
fp8 copy and with the MXFP4 copy.

Sampling.  Heads are independent tiles of the recurrence, so the oracle follows 128
(sequence, head) tiles: 8 sequences spread over the batch, 16 heads each, sequence i
taking heads i, i + 8, ..., i + 120 (together every head index).  These tiles get
their exact seeded inputs at every step; every other tile cycles through the first 16
seeded steps of the full batch (its outputs are not compared, its cursors are).

Checked, per sampled tile and step:
* read-copy outputs against the oracle, which quantises its own fp32 checkpoint: each
  output row within the fp32 tolerance plus the oracle's allowance for codes at a
  rounding boundary (a wrong rounding rule moves codes far from any boundary and fails
  this); every row of either format within 5e-2 normwise.  Reported beside: the share
  of rows that differ by more than the fp32 tolerance (a code differs: the GPU and the
  oracle quantise checkpoints that agree only to fp32 rounding) and their worst error;
* the path without a copy against the exact fp64 recurrence (2e-5), and its
  checkpoints every 256 steps;
and for the whole batch: every cursor replica on every step, and the checkpoints of
the states with a copy bit-identical to the state without one (the copy never feeds
the recurrence).

Drift (reported): normwise relative error of the read-copy outputs against the exact
fp64 recurrence (sampled tiles) and against the GPU path without a copy (all tiles),
mean and max per 256-step bin with the fitted slope.  With RSSM_DRIFT_JSON set, the
report is written there as JSON.
"""
from __future__ import annotations

import json
import os
import time
from concurrent.futures import ProcessPoolExecutor, as_completed

import numpy as np
import pytest
import torch

from oracle import ReplayOracle
from synth import decode_inputs, get_workload, initial_state
from synth.gen import default_workers
from synth.stream import StepSource

from gpu_util import TOL, TOL_READ, decode, new_state, read_copy_excess, relerr, tile_relerr
from oracle_runs import READ_TOL

pytestmark = pytest.mark.gpu

STEPS = 4096
SEQS = [0, 37, 74, 111, 148, 185, 222, 255]
NHS = 16          # sampled heads per sampled sequence
POOL = 16         # seeded full-batch steps the unsampled tiles cycle through
BIN = 256
FIELDS = ("alpha", "v", "k", "q")
_SHARED: dict = {}     # filled before the worker pools fork; read by the workers


def _heads(i):
    return [i + 8 * j for j in range(NHS)]


def _sample_job(i):
    """Exact seeded inputs and initial state of sampled sequence i's tiles, all steps."""
    wl = _SHARED["wl"]
    b, hs = SEQS[i], np.asarray(_heads(i))
    out = {f: np.empty((STEPS, NHS) + (() if f == "alpha" else (wl.dv if f == "v" else wl.dk,)), np.uint16)
           for f in FIELDS}
    for t in range(STEPS):
        x = decode_inputs(wl, t, [b])
        for f in FIELDS:                       # Mamba-2: one key/query head per value head
            out[f][t] = x[f][0][hs]
    out["S0"] = np.ascontiguousarray(initial_state(wl, [b])[0][hs])
    return i, out


def _s0_chunk(seqs):
    return initial_state(_SHARED["wl"], seqs)


def _slope(bins):
    m = np.array([b["mean"] for b in bins])
    return float(np.polyfit(np.arange(len(m)), m, 1)[0]) if len(m) > 1 else 0.0


def _oracle_job(args):
    """fp64 oracle of sampled sequence i with copy format fmt; compares the GPU outputs."""
    i, fmt = args
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    wl = _SHARED["wl"]
    smp = _SHARED["samples"][i]
    gy = _SHARED["gpu_y"][fmt][:, i]           # [STEPS, NHS, P]
    g32 = _SHARED["gpu_y"]["none"][:, i]
    sub = wl.replace(batch=1, n_heads=NHS, n_qk_heads=NHS, read_copy=fmt)
    orc = ReplayOracle(sub, [0], smp["S0"][None], read_tol=READ_TOL)
    err_read = np.empty((STEPS, NHS))          # vs the oracle's read-copy chain
    err_exact = np.empty((STEPS, NHS))         # vs the exact recurrence (drift)
    err_fp32 = np.empty((STEPS, NHS))          # GPU path without a copy vs the exact recurrence
    amb = np.zeros((STEPS, NHS), bool)         # rows with a nonzero allowance
    need = np.zeros((STEPS, NHS), bool)        # rows that differ by more than the fp32 tolerance
    excess = -np.inf
    ck = 0.0
    for t in range(STEPS):
        inp = {f: smp[f][t][None] for f in FIELDS}
        inp["beta"] = None
        y = orc.decode(inp)[0]
        ye = orc.y_exact[0]
        al = orc.allowance[0]
        err_read[t] = relerr(gy[t], y)
        err_exact[t] = relerr(gy[t], ye)
        err_fp32[t] = relerr(g32[t], ye)
        amb[t] = np.max(al, axis=-1) > 0
        need[t] = np.any(np.abs(gy[t] - y) > TOL * np.max(np.abs(y), axis=-1, keepdims=True), axis=-1)
        excess = max(excess, float(np.max(read_copy_excess(gy[t], y, al))))
        if t in _SHARED["ckpt"]:
            ck = max(ck, float(np.max(tile_relerr(_SHARED["ckpt"][t][i], orc.S_ckpt[0]))))
    flush = (np.arange(STEPS) + 1) % wl.L == 0
    return {"i": i, "fmt": fmt, "excess": excess,
            "worst_read": float(err_read.max()),
            "worst_read_zero_allowance": float(err_read[~amb].max()),
            "worst_read_not_needed": float(err_read[~need].max()),
            "worst_read_needed": float(err_read[need].max()) if need.any() else None,
            "allowance_rows": int(amb.sum()), "needed_rows": int(need.sum()), "rows": int(amb.size),
            "worst_fp32": float(err_fp32.max()), "worst_ckpt": ck,
            "flush_steps_worst_exact": float(err_exact[flush].max()),
            "drift_exact": err_exact[~flush].mean(axis=1), "drift_exact_max": err_exact[~flush].max(axis=1),
            "nonflush_steps": np.flatnonzero(~flush)}


def test_read_copy_serving_shape_4096_steps():
    wl = get_workload("m2_readcopy_b256").replace(read_copy="none")
    assert wl.decode_steps == STEPS and wl.batch == 256 and wl.L == 16
    B, H, P, N = wl.batch, wl.n_heads, wl.dv, wl.dk
    _SHARED.clear()
    _SHARED["wl"] = wl
    workers = default_workers()
    t0 = time.time()
    print(f"[read copy 4096] sampled inputs for {len(SEQS)} sequences x {NHS} heads x {STEPS} steps", flush=True)
    with ProcessPoolExecutor(max_workers=min(workers, len(SEQS))) as ex:
        samples = dict(ex.map(_sample_job, range(len(SEQS))))
        chunks = [list(c) for c in np.array_split(np.arange(B), workers) if len(c)]
        s0 = torch.empty(B, H, P, N, dtype=torch.float32, device="cuda")
        for c, arr in zip(chunks, ex.map(_s0_chunk, chunks)):
            s0[c[0]: c[-1] + 1] = torch.from_numpy(arr).cuda()
    with StepSource(wl, range(B)) as src:
        pool = [{f: torch.from_numpy(v.view(np.int16)).cuda() for f, v in src.decode(t).items() if v is not None}
                for t in range(POOL)]
    print(f"[read copy 4096] inputs ready in {time.time() - t0:.1f} s", flush=True)

    states = {fmt: new_state(wl.replace(read_copy=fmt)) for fmt in ("none", "fp8", "mxfp4")}
    for ds in states.values():
        ds.init(s0, torch.cuda.current_stream().cuda_stream)
    del s0
    bidx = torch.tensor([[b] * NHS for b in SEQS], device="cuda")
    hidx = torch.tensor([_heads(i) for i in range(len(SEQS))], device="cuda")
    samp = {f: torch.from_numpy(np.stack([samples[i][f] for i in range(len(SEQS))], axis=1).view(np.int16)).cuda()
            for f in FIELDS}                   # [STEPS, 8, NHS, ...]
    work = {f: torch.empty_like(pool[0][f]) for f in FIELDS}
    ys = {fmt: torch.empty(B, H, P, device="cuda") for fmt in states}
    gy = {fmt: torch.empty(STEPS, len(SEQS), NHS, P, device="cuda") for fmt in states}
    drift32 = {fmt: torch.empty(STEPS, 2, dtype=torch.float64, device="cuda") for fmt in ("fp8", "mxfp4")}
    bad_cursor = torch.zeros((), dtype=torch.int64, device="cuda")
    bad_ident = torch.zeros((), dtype=torch.int64, device="cuda")
    ckpt = {}
    for t in range(STEPS):
        for f in FIELDS:
            work[f].copy_(pool[t % POOL][f])
            work[f][bidx, hidx] = samp[f][t]
        for fmt, ds in states.items():
            decode(ds, dict(work, beta=None), ys[fmt])
            gy[fmt][t] = ys[fmt][bidx, hidx]
            nc, nk = ds.counters()
            bad_cursor += ((nc != t + 1) | (nk != wl.L * ((t + 1) // wl.L))).sum()
        ref = ys["none"].double()
        den = ref.abs().amax(dim=-1).clamp_min(1e-30)
        for fmt in ("fp8", "mxfp4"):
            e = (ys[fmt].double() - ref).abs().amax(dim=-1) / den
            drift32[fmt][t, 0] = e.mean()
            drift32[fmt][t, 1] = e.max()
        if t % BIN == BIN - 1:
            base = states["none"].ckpt()
            for fmt in ("fp8", "mxfp4"):
                bad_ident += (states[fmt].ckpt().view(torch.int32) != base.view(torch.int32)).any().long()
            ckpt[t] = base[bidx, hidx].cpu().numpy()
            print(f"[read copy 4096] GPU step {t + 1}/{STEPS} ({time.time() - t0:.1f} s)", flush=True)
    torch.cuda.synchronize()
    assert int(bad_cursor.item()) == 0, "cursor replicas differ from the integer policy"
    assert int(bad_ident.item()) == 0, "a read copy changed the fp32 checkpoint trajectory"
    for ds in states.values():
        assert ds.error() == 0
    _SHARED["samples"] = samples
    _SHARED["gpu_y"] = {fmt: v.cpu().numpy() for fmt, v in gy.items()}
    _SHARED["ckpt"] = ckpt
    d32 = {fmt: v.cpu().numpy() for fmt, v in drift32.items()}
    del states, pool, samp, work, gy

    jobs = [(i, fmt) for fmt in ("fp8", "mxfp4") for i in range(len(SEQS))]
    res = {"fp8": [], "mxfp4": []}
    with ProcessPoolExecutor(max_workers=min(workers, len(jobs))) as ex:
        futs = [ex.submit(_oracle_job, j) for j in jobs]
        for n, fu in enumerate(as_completed(futs)):
            r = fu.result()
            res[r["fmt"]].append(r)
            print(f"[read copy 4096] oracle {n + 1}/{len(jobs)}: seq {SEQS[r['i']]} {r['fmt']} worst {r['worst_read']:.3g} "
                  f"excess {r['excess']:.3g} ({time.time() - t0:.1f} s)", flush=True)

    report = {"command": "RSSM_DRIFT_JSON=<path> python -m pytest tests/test_gpu_readcopy_long.py -s",
              "workload": "mamba2 read copy, B=256 H=128 P=64 N=128 bf16 inputs, L=16", "steps": STEPS,
              "sampled_tiles": len(SEQS) * NHS, "sampled_sequences": SEQS,
              "heads_per_sequence": "sequence i of the sample: heads i, i+8, ..., i+120", "bin": BIN}
    for fmt in ("fp8", "mxfp4"):
        rs = sorted(res[fmt], key=lambda r: r["i"])
        nf = rs[0]["nonflush_steps"]
        ex_mean = np.mean([r["drift_exact"] for r in rs], axis=0)
        ex_max = np.max([r["drift_exact_max"] for r in rs], axis=0)
        full_mean = np.full(STEPS, np.nan)
        full_mean[nf] = ex_mean
        full_max = np.full(STEPS, np.nan)
        full_max[nf] = ex_max
        b_exact = [{"steps": [s, s + BIN - 1], "mean": float(np.nanmean(full_mean[s:s + BIN])),
                    "max": float(np.nanmax(full_max[s:s + BIN]))} for s in range(0, STEPS, BIN)]
        b_gpu = [{"steps": [s, s + BIN - 1], "mean": float(d32[fmt][s:s + BIN, 0].mean()),
                  "max": float(d32[fmt][s:s + BIN, 1].max())} for s in range(0, STEPS, BIN)]
        amb_rows = sum(r["allowance_rows"] for r in rs)
        need_rows = sum(r["needed_rows"] for r in rs)
        rows = sum(r["rows"] for r in rs)
        worst_need = [r["worst_read_needed"] for r in rs if r["worst_read_needed"] is not None]
        report[fmt] = {
            "parity_vs_oracle": {
                "rows": rows,
                "worst_normwise_rel_err": max(r["worst_read"] for r in rs),
                "rows_with_nonzero_allowance": amb_rows, "share_with_nonzero_allowance": amb_rows / rows,
                "worst_normwise_rel_err_rows_with_zero_allowance": max(r["worst_read_zero_allowance"] for r in rs),
                "rows_that_needed_the_allowance": need_rows, "share_that_needed_the_allowance": need_rows / rows,
                "worst_normwise_rel_err_rows_that_needed_it": max(worst_need) if worst_need else None,
                "worst_normwise_rel_err_other_rows": max(r["worst_read_not_needed"] for r in rs),
                "worst_excess_over_fp32_tolerance_plus_allowance": max(r["excess"] for r in rs)},
            "drift_vs_fp64_oracle": {"tiles": "sampled", "bins": b_exact, "fitted_slope_per_bin": _slope(b_exact),
                                     "mean": float(np.mean(ex_mean))},
            "drift_vs_gpu_fp32_path": {"tiles": "all", "bins": b_gpu, "fitted_slope_per_bin": _slope(b_gpu),
                                       "mean": float(d32[fmt][:, 0].mean())},
        }
    report["fp32_path"] = {"worst_normwise_rel_err_vs_fp64": max(r["worst_fp32"] for f in res for r in res[f]),
                           "worst_checkpoint_rel_err": max(r["worst_ckpt"] for f in res for r in res[f])}
    out = os.environ.get("RSSM_DRIFT_JSON")
    if out:
        with open(out, "w") as f:
            json.dump(report, f, indent=1)
    print("[read copy 4096] " + json.dumps({k: report[k]["parity_vs_oracle"] for k in ("fp8", "mxfp4")}), flush=True)

    for fmt in ("fp8", "mxfp4"):
        pv = report[fmt]["parity_vs_oracle"]
        assert pv["worst_excess_over_fp32_tolerance_plus_allowance"] <= 0, fmt
        assert pv["worst_normwise_rel_err_rows_with_zero_allowance"] <= TOL_READ, fmt
        assert pv["worst_normwise_rel_err_other_rows"] <= TOL_READ, fmt
        assert pv["worst_normwise_rel_err"] <= TOL_READ, fmt
    assert report["fp32_path"]["worst_normwise_rel_err_vs_fp64"] <= TOL
    assert report["fp32_path"]["worst_checkpoint_rel_err"] <= TOL
