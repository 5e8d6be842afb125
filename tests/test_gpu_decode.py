"""GPU parity of replay decode (fused flush) and of the conventional comparator
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from attention_decode_mamba_amd import rssm as R
from oracle import ReplayOracle
from synth import decode_inputs, draft_inputs, get_workload, initial_state
from synth.stream import StepSource

from gpu_util import (TOL, assert_counters, decode, dev, new_state, ptr, relerr, ring_bits, stream,
                      tile_relerr, to_dev_inputs, verify)
from oracle_runs import cursor_run, decode_runs

pytestmark = pytest.mark.gpu


def _check_ring(ds, orc, seqs):
    ring = {k: (None if v is None else ring_bits(v)) for k, v in ds.ring_arrays().items()}
    wl = orc.wl
    for i, b in enumerate(seqs):
        for slot in orc.live_slots(i):
            assert np.array_equal(ring["alpha"][b, :, slot], orc.ring["alpha"][i, slot])
            assert np.array_equal(ring["v"][b, :, slot], orc.ring["v"][i, slot])
            g_lead = np.arange(wl.n_qk_heads)
            assert np.array_equal(ring["k"][b, g_lead, slot], orc.ring["k"][i, slot])
            assert np.array_equal(ring["q"][b, g_lead, slot], orc.ring["q"][i, slot])
            if ring["beta"] is not None:
                assert np.array_equal(ring["beta"][b, :, slot], orc.ring["beta"][i, slot])


def _run_small(wl, steps, check_ring=True):
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    ys = []
    for t in range(steps):
        inp = decode_inputs(wl, t, seqs)
        decode(ds, to_dev_inputs(inp), y)
        yr = orc.decode(inp)
        got = y.cpu().numpy()
        ys.append(got.copy())
        err = relerr(got, yr).max()
        assert err <= TOL, f"step {t}: output rel err {err:.3g}"
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"step {t}")
        if np.all(orc.n_ckpt == orc.n_committed):
            e = tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max()
            assert e <= TOL, f"step {t}: checkpoint rel err {e:.3g}"
        if check_ring:
            _check_ring(ds, orc, seqs)
    assert ds.error() == 0
    return np.array(ys)


@pytest.mark.parametrize("s0", ["normal", "zero"])
def test_tiny_mamba2_decode(s0):
    """64 steps, 4 flushes: every output, checkpoint, cursor and ring record."""
    wl = get_workload("m2_tiny").replace(s0=s0)
    _run_small(wl, wl.decode_steps)


def test_tiny_mamba2_decode_deterministic():
    wl = get_workload("m2_tiny")
    a = _run_small(wl, 20, check_ring=False)
    b = _run_small(wl, 20, check_ring=False)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


SHAPES = [
    # kind, dtype, B, H, G, P, N, L, C
    ("mamba2", "fp32", 5, 3, 3, 17, 32, 5, 5),
    ("mamba2", "bf16", 3, 2, 1, 100, 64, 16, 20),
    ("mamba2", "fp32", 2, 2, 2, 200, 32, 4, 4),
    ("mamba2", "bf16", 2, 3, 3, 64, 256, 8, 8),
    ("mamba2", "fp32", 3, 2, 2, 16, 32, 1, 1),
    ("gdn", "bf16", 3, 4, 2, 40, 64, 6, 6),
    ("gdn", "fp32", 2, 2, 1, 128, 128, 16, 16),
    ("gdn", "bf16", 2, 2, 2, 33, 32, 3, 3),
    ("mamba2", "bf16", 2, 3, 3, 64, 128, 32, 32),   # longest window: records staged in two rounds
    ("gdn", "bf16", 2, 2, 1, 128, 128, 32, 32),
    ("kda", "bf16", 3, 4, 2, 40, 64, 6, 6),
    ("kda", "fp32", 2, 2, 2, 128, 128, 16, 16),
    ("kda", "bf16", 2, 2, 2, 33, 32, 3, 3),         # rows not 16-byte aligned: element-wise staging
    ("kda", "bf16", 2, 2, 1, 128, 128, 32, 32),
    # the widest tiles: 16 row groups of 8 per wave at dk = 32, 8 at dk = 64
    ("mamba2", "bf16", 2, 2, 2, 512, 32, 5, 5),
    ("gdn", "fp32", 2, 2, 1, 512, 32, 4, 4),
    ("kda", "bf16", 2, 2, 2, 500, 32, 4, 4),
    ("mamba2", "fp32", 2, 2, 2, 256, 64, 4, 4),
]

_BASE = {"mamba2": "m2_tiny", "gdn": "gdn_b256", "kda": "kda_b256"}


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_decode_shapes_and_ragged_tails(shape):
    kind, dt, B, H, G, P, N, L, C = shape
    base = get_workload(_BASE[kind])
    wl = base.replace(name="shape", batch=B, n_heads=H, n_qk_heads=G, dv=P, dk=N, in_dtype=dt, L=L,
                      t_max=1, capacity=C, read_copy="none")
    _run_small(wl, 3 * L + 3)


@pytest.mark.parametrize("kind,L", [("mamba2", 4), ("mamba2", 16), ("gdn", 8), ("kda", 8)])
def test_staggered_windows_decode(kind, L):
    """Windows at different phases: sequence b first commits b mod L one-draft verifies
    (verify(T=1) + commit(0 or 1)), so each decode step folds only the sequences whose window
    fills on that step.  Every output, cursor and checkpoint against the oracle for 2L steps."""
    base = get_workload(_BASE[kind])
    wl = base.replace(name="stagger", batch=2 * L + 1, n_heads=3 if kind == "mamba2" else 4,
                      n_qk_heads=3 if kind == "mamba2" else 2, dv=24, dk=64, in_dtype="bf16", L=L, t_max=1,
                      capacity=L, read_copy="none")
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    o = torch.empty(wl.batch, 1, wl.n_heads, wl.dv, device="cuda")
    for r in range(L - 1):
        dr = draft_inputs(wl, r, seqs, 1)
        verify(ds, 1, to_dev_inputs(dr), o)
        orc.verify(dr, 1)
        acc = (np.arange(wl.batch) % L > r).astype(np.int32)
        acc_d = dev(acc)
        R.rssm_commit(ds.cfg, ds.st, ptr(acc_d), 1, stream())
        orc.commit(acc, 1)
        R.rssm_flush(ds.cfg, ds.st, L, stream())
        orc.flush(L)
    assert_counters(ds, orc.n_committed, orc.n_ckpt, "after staggering")
    assert sorted(set((orc.n_committed - orc.n_ckpt).tolist())) == list(range(L))
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    for t in range(2 * L):
        inp = decode_inputs(wl, t, seqs)
        decode(ds, to_dev_inputs(inp), y)
        yr = orc.decode(inp)
        err = relerr(y.cpu().numpy(), yr).max()
        assert err <= TOL, f"step {t}: output rel err {err:.3g}"
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"step {t}")
        folded = orc.n_ckpt == orc.n_committed
        assert 1 <= int(folded.sum()) <= 3           # b mod L hits each phase 2 or 3 times
        e = tile_relerr(ds.ckpt().cpu().numpy()[folded], orc.S_ckpt[folded]).max()
        assert e <= TOL, f"step {t}: checkpoint rel err {e:.3g}"
    assert ds.error() == 0


def test_conventional_comparator_small():
    for name in ("m2_tiny", "gdn_b256", "kda_b256"):
        wl = get_workload(name)
        if name != "m2_tiny":
            wl = wl.replace(batch=3, n_heads=4, n_qk_heads=2, dv=24, dk=32, in_dtype="fp32")
        seqs = list(range(wl.batch))
        S0 = initial_state(wl, seqs)
        orc = ReplayOracle(wl, seqs, S0)
        s = dev(S0)
        cfg = new_state(wl, S0).cfg
        y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
        for t in range(24):
            inp = decode_inputs(wl, t, seqs)
            d = to_dev_inputs(inp)
            R.rssm_decode_step_conventional(cfg, ptr(s), ptr(d["alpha"]), ptr(d.get("beta")), ptr(d["v"]),
                                            ptr(d["k"]), ptr(d["q"]), ptr(y), stream())
            yr = orc.decode(inp)
            assert relerr(y.cpu().numpy(), yr).max() <= TOL
        assert tile_relerr(s.cpu().numpy(), orc.S).max() <= TOL


SAMPLE = [0, 37, 74, 111, 148, 185, 222, 255]


def test_serving_shape_decode_sampled():
    """Mamba-2 at B=256, H=128, P=64, N=128, bf16 inputs, 256 steps (16 flushes), in the
    launch configuration the benchmark times; sampled sequences checked against the oracle at
    every step, every sequence's cursor checked at every step; conventional comparator too."""
    wl = get_workload("m2_decode_b256")
    steps = wl.decode_steps
    seqs = list(range(wl.batch))
    print(f"[serving decode] oracle runs for {SAMPLE}", flush=True)
    ref = decode_runs(wl, SAMPLE, steps, ckpt_every=64)
    cur = cursor_run(wl, steps, verify=False)
    S0 = initial_state(wl, seqs)
    ds = new_state(wl, S0)
    conv = dev(S0)
    del S0
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    yc = torch.empty_like(y)
    idx = torch.tensor(SAMPLE, device="cuda")
    worst = worst_c = 0.0
    with StepSource(wl, seqs) as src:
        for t in range(steps):
            d = to_dev_inputs(src.decode(t))
            decode(ds, d, y)
            R.rssm_decode_step_conventional(ds.cfg, ptr(conv), ptr(d["alpha"]), None, ptr(d["v"]), ptr(d["k"]),
                                            ptr(d["q"]), ptr(yc), stream())
            got = y[idx].cpu().numpy()
            gotc = yc[idx].cpu().numpy()
            for i, b in enumerate(SAMPLE):
                worst = max(worst, relerr(got[i], ref[b]["y"][t]).max())
                worst_c = max(worst_c, relerr(gotc[i], ref[b]["y"][t]).max())
            assert_counters(ds, *cur[t], f"step {t}")
            for b in SAMPLE:
                if t in ref[b]["ckpt"]:
                    e = tile_relerr(ds.ckpt()[b].cpu().numpy(), ref[b]["ckpt"][t]).max()
                    assert e <= TOL, f"step {t} seq {b}: checkpoint rel err {e:.3g}"
            if t % 64 == 63:
                print(f"[serving decode] step {t + 1}/{steps} worst rel err {worst:.3g} conv {worst_c:.3g}",
                      flush=True)
    assert worst <= TOL and worst_c <= TOL
    assert ds.error() == 0
