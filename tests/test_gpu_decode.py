"""GPU parity of replay decode (fused flush) and of the conventional comparator
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from attention_decode_mamba_amd import rssm as R
from oracle import ReplayOracle
from synth import decode_inputs, draft_inputs, get_workload, initial_state
from synth.stream import StepSource

from gpu_util import (TOL, assert_counters, check_ring, decode, dev, new_state, ptr, relerr, stream,
                      tile_relerr, to_dev_inputs, verify)
from oracle_runs import cursor_run, decode_runs

pytestmark = pytest.mark.gpu


def _run_small(wl, steps, ring=True):
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
        if ring:
            check_ring(ds, orc, seqs)
    assert ds.error() == 0
    return np.array(ys)


@pytest.mark.parametrize("s0", ["normal", "zero"])
def test_tiny_mamba2_decode(s0):
    """64 steps, 4 flushes: every output, checkpoint, cursor and ring record."""
    wl = get_workload("m2_tiny").replace(s0=s0)
    _run_small(wl, wl.decode_steps)


def test_tiny_mamba2_decode_deterministic():
    wl = get_workload("m2_tiny")
    a = _run_small(wl, 20, ring=False)
    b = _run_small(wl, 20, ring=False)
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
    # H a multiple of 16: Mamba-2 and KDA append each group of heads (16; Mamba-2 32 where H
    # allows) from the group's last workgroup, dispatched after all others (ragged grids; 8 x 16
    # tiles take the XCD order; key groups of 8 and of 3 heads; fp32 rows; rows not 16-byte
    # aligned; GDN keeps per-tile appends)
    ("mamba2", "bf16", 3, 16, 16, 16, 32, 4, 4),
    ("mamba2", "bf16", 8, 16, 16, 64, 128, 5, 5),
    ("mamba2", "fp32", 2, 32, 4, 8, 32, 3, 3),
    ("mamba2", "bf16", 2, 48, 16, 8, 32, 3, 3),
    ("kda", "bf16", 2, 16, 8, 40, 64, 4, 4),
    ("kda", "bf16", 3, 16, 16, 33, 32, 3, 3),
    ("kda", "fp32", 8, 16, 16, 16, 32, 3, 3),
    ("gdn", "bf16", 2, 16, 8, 16, 32, 4, 4),
]

_BASE = {"mamba2": "m2_tiny", "gdn": "gdn_b256", "kda": "kda_b256"}


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_decode_shapes_and_ragged_tails(shape):
    kind, dt, B, H, G, P, N, L, C = shape
    base = get_workload(_BASE[kind])
    wl = base.replace(name="shape", batch=B, n_heads=H, n_qk_heads=G, dv=P, dk=N, in_dtype=dt, L=L,
                      t_max=1, capacity=C, read_copy="none")
    _run_small(wl, 3 * L + 3)


@pytest.mark.parametrize("kind,L,H,G", [("mamba2", 4, 3, 3), ("mamba2", 16, 3, 3), ("gdn", 8, 4, 2), ("kda", 8, 4, 2),
                                         ("mamba2", 8, 16, 16), ("kda", 4, 16, 8), ("mamba2", 6, 32, 32)])
def test_staggered_windows_decode(kind, L, H, G):
    """Windows at different phases: sequence b first commits b mod L one-draft verifies
    (verify(T=1) + commit(0 or 1)), so each decode step folds only the sequences whose window
    fills on that step.  Every output, cursor and checkpoint against the oracle for 2L steps,
    and every live ring slot bit for bit (with 16 or 32 heads the appends of a sequence's group of
    heads come from its last workgroup, which skips them when the sequence folds)."""
    base = get_workload(_BASE[kind])
    wl = base.replace(name="stagger", batch=2 * L + 1, n_heads=H, n_qk_heads=G, dv=24, dk=64, in_dtype="bf16",
                      L=L, t_max=1, capacity=L, read_copy="none")
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
        check_ring(ds, orc, seqs)
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


@pytest.mark.parametrize("kind,H", [("mamba2", 16), ("mamba2", 32), ("kda", 16), ("kda", 32)])
def test_decode_cursor_error_with_group_appends(kind, H):
    """With H a multiple of 16 the ring appends of a group of heads of a sequence (16 heads;
    Mamba-2 32 where H allows) come from the workgroup of the group's last head.  A broken main tile
    (1, 2) is left out of its group's appends: its cursors, output rows, checkpoint and ring
    rows stay untouched, and the rest of sequence 1 matches a run without the corruption bit
    for bit, ring included.  A broken appender (2, H - 1) sets the error bit and stays
    untouched; its group's other heads still produce the step's outputs, but their records of
    that step are not appended.  Sequence 0 matches the clean run bit for bit throughout."""
    base = get_workload("m2_decode_b256" if kind == "mamba2" else "kda_b256")
    wl = base.replace(name="group_err", batch=3, n_heads=H, n_qk_heads=H, dv=64 if kind == "mamba2" else 32,
                      dk=128 if kind == "mamba2" else 64, in_dtype="bf16", L=6, capacity=6, t_max=1,
                      read_copy="none")
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    ds = new_state(wl, S0)
    ref = new_state(wl, S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    y2 = torch.empty_like(y)
    for t in range(3):
        d = to_dev_inputs(decode_inputs(wl, t, seqs))
        decode(ds, d, y)
        decode(ref, d, y2)
    nc, nk = ds.counters()
    nk[1, 2] = nc[1, 2] + 1                       # h < 0 on a main tile
    nc[2, H - 1] = nk[2, H - 1] + wl.capacity + 1     # h > C on an appender
    bad = [(1, 2), (2, H - 1)]
    keep_nc, keep_nk = nc.clone(), nk.clone()
    keep_ck = ds.ckpt().clone()
    ring0 = {k: (None if v is None else v.clone()) for k, v in ds.ring_arrays().items()}
    good = torch.ones(wl.batch, wl.n_heads, dtype=torch.bool)
    good[1, 2] = False
    good[2, :] = False                            # the broken appender's group
    sentinel = torch.full_like(y, 12345.0)
    for t in range(3, 6):                         # steps 3 and 4 are non-fold steps, step 5 folds
        d = to_dev_inputs(decode_inputs(wl, t, seqs))
        y.copy_(sentinel)
        decode(ds, d, y)
        decode(ref, d, y2)
        torch.cuda.synchronize()
        for b, h in bad:
            assert torch.equal(y[b, h], sentinel[b, h]), f"step {t}: output row of broken tile ({b},{h}) written"
            assert torch.equal(ds.ckpt()[b, h], keep_ck[b, h]), f"step {t}: checkpoint of ({b},{h}) changed"
            assert int(nc[b, h]) == int(keep_nc[b, h]) and int(nk[b, h]) == int(keep_nk[b, h])
        ring = ds.ring_arrays()
        for name in ("alpha", "v", "beta"):
            if ring[name] is not None:
                assert torch.equal(ring[name][1, 2], ring0[name][1, 2]), f"step {t}: ring {name} of (1,2) written"
        for name in ("k", "q"):
            assert torch.equal(ring[name][1, 2], ring0[name][1, 2]), f"step {t}: ring {name} of key head 2 written"
        gy, ry = y.cpu()[good], y2.cpu()[good]
        assert torch.equal(gy.view(torch.int32), ry.view(torch.int32)), f"step {t}: healthy outputs differ"
        if t == 3:                                # the group's records up to step 2 were appended
            assert torch.equal(y[2, :H - 1].cpu().view(torch.int32), y2[2, :H - 1].cpu().view(torch.int32))
        rc, rk = ref.counters()
        assert torch.equal(nc.cpu()[good], rc.cpu()[good]) and torch.equal(nk.cpu()[good], rk.cpu()[good])
        assert torch.equal(ds.ckpt().cpu()[good].view(torch.int32), ref.ckpt().cpu()[good].view(torch.int32))
        rr = ref.ring_arrays()
        for name in ("alpha", "v", "beta"):
            if ring[name] is not None:
                assert torch.equal(ring[name].cpu()[good], rr[name].cpu()[good]), f"step {t}: ring {name} differs"
        for name in ("k", "q"):                   # key head g is led by value head g (G = H)
            assert torch.equal(ring[name].cpu()[good], rr[name].cpu()[good]), f"step {t}: ring {name} differs"
    assert ds.error() == R.RSSM_DEVERR_CURSOR
    assert ref.error() == 0
