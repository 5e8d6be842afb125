"""GPU parity of the speculative path (verify -> commit -> flush) for Mamba-2 and
Gated DeltaNet, rollback invariants and device-side contract errors."""
import numpy as np
import pytest
import torch

from attention_decode_mamba_amd import rssm as R
from oracle import ReplayOracle
from synth import accept_counts, decode_inputs, draft_inputs, draft_tree, get_workload, initial_state
from synth.stream import StepSource

from gpu_util import (TOL, assert_counters, check_ring, counters, decode, dev, new_state, ptr, relerr,
                      stream, tile_relerr, to_dev_inputs, verify)
from oracle_runs import cursor_run, spec_runs

pytestmark = pytest.mark.gpu


def _small(name, **kw):
    wl = get_workload(name)
    if name.startswith(("gdn", "kda")):
        base = dict(batch=6, n_heads=4, n_qk_heads=2, dv=48, dk=64)
    else:
        base = dict(batch=6, n_heads=4, n_qk_heads=4, dv=20, dk=32)
    base.update(kw)
    return wl.replace(name="small", **base)


def _commit(ds, acc, T):
    R.rssm_commit(ds.cfg, ds.st, ptr(acc), T, stream())


def _flush(ds, m):
    R.rssm_flush(ds.cfg, ds.st, m, stream())


def _poison_rejected(ds, nc_before, acc, T):
    """Overwrite the ring slots of rejected drafts with NaN bit patterns (host-side writes)."""
    ring = ds.ring_arrays()
    C = ds.cfg.capacity
    nan = -1 if ring["v"].dtype == torch.int16 else float("nan")     # 0xFFFF is a bf16 NaN
    for b in range(ds.cfg.batch):
        for tau in range(int(acc[b]), T):
            slot = int((nc_before[b] + tau) % C)
            ring["alpha"][b, :, slot] = nan
            ring["v"][b, :, slot] = nan
            ring["k"][b, :, slot] = nan
            ring["q"][b, :, slot] = nan
            if ring["beta"] is not None:
                ring["beta"][b, :, slot] = nan


@pytest.mark.parametrize("name", ["m2_verify_b512", "gdn_b256", "kda_b256"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_spec_small(name, dtype):
    """A few decode steps, then verify(T) / commit(a) / flush(L): outputs, cursors, checkpoints."""
    wl = _small(name, in_dtype=dtype)
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    for t in range(5):
        inp = decode_inputs(wl, t, seqs)
        decode(ds, to_dev_inputs(inp), y)
        assert relerr(y.cpu().numpy(), orc.decode(inp)).max() <= TOL
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    for s in range(40):
        d = draft_inputs(wl, s, seqs, T)
        verify(ds, T, to_dev_inputs(d), o)
        Or = orc.verify(d, T)
        err = relerr(o.cpu().numpy(), Or).max()
        assert err <= TOL, f"verify step {s}: rel err {err:.3g}"
        acc = accept_counts(wl, s, T)[: wl.batch]
        _commit(ds, dev(acc), T)
        orc.commit(acc, T)
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"commit {s}")
        _flush(ds, wl.L)
        orc.flush(wl.L)
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"flush {s}")
        e = tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max()
        assert e <= TOL, f"step {s}: checkpoint rel err {e:.3g}"
    # a decode step after speculation continues from the same cursor
    inp = decode_inputs(wl, 99, seqs)
    decode(ds, to_dev_inputs(inp), y)
    assert relerr(y.cpu().numpy(), orc.decode(inp)).max() <= TOL
    assert_counters(ds, orc.n_committed, orc.n_ckpt, "final decode")
    assert ds.error() == 0


@pytest.mark.parametrize("name", ["m2_verify_b512", "gdn_b256", "kda_b256"])
def test_rejected_slots_are_never_read(name):
    """Poisoning every rejected draft slot with NaN changes no output and no checkpoint bit."""
    wl = _small(name)
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    A, B = new_state(wl, S0), new_state(wl, S0)
    oa = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    ob = torch.empty_like(oa)
    for s in range(30):
        d = to_dev_inputs(draft_inputs(wl, s, seqs, T))
        verify(A, T, d, oa)
        verify(B, T, d, ob)
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32)), f"step {s}"
        acc = accept_counts(wl, s, T)[: wl.batch]
        nc_before = counters(B)[0][:, 0].copy()
        _commit(A, dev(acc), T)
        _commit(B, dev(acc), T)
        torch.cuda.synchronize()
        _poison_rejected(B, nc_before, acc, T)
        _flush(A, wl.L)
        _flush(B, wl.L)
        assert torch.equal(A.ckpt().view(torch.int32), B.ckpt().view(torch.int32)), f"step {s}"
    assert A.error() == 0 and B.error() == 0


def test_device_errors_leave_sequences_untouched():
    wl = _small("m2_verify_b512")
    T = wl.t_max
    seqs = list(range(wl.batch))
    ds = new_state(wl, initial_state(wl, seqs))
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    acc = np.zeros(wl.batch, np.int32)
    acc[0] = T                                   # sequence 0 commits T per step, never flushed
    for s in range(4):
        verify(ds, T, to_dev_inputs(draft_inputs(wl, s, seqs, T)), o)
        _commit(ds, dev(acc), T)
    assert ds.error() == 0
    nc, nk = counters(ds)
    assert np.all(nc[0] == 4 * T) and np.all(nc[1:] == 0)
    ring0 = {k: (None if v is None else v[0].clone()) for k, v in ds.ring_arrays().items()}
    ck_before = ds.ckpt().clone()
    o.fill_(7.0)
    verify(ds, T, to_dev_inputs(draft_inputs(wl, 9, seqs, T)), o)
    err = ds.error()
    assert err & R.RSSM_DEVERR_VERIFY_CAPACITY
    assert torch.all(o[0] == 7.0)                # rows of the refused sequence not written
    assert torch.all(o[1:] != 7.0)
    after = ds.ring_arrays()
    for k, v in ring0.items():                   # the refused sequence's ring rows are unchanged
        if v is not None:
            assert torch.equal(v, after[k][0]), k
    assert torch.equal(ck_before, ds.ckpt())
    # commit of the refused verify is refused too
    acc2 = np.ones(wl.batch, np.int32)
    _commit(ds, dev(acc2), T)
    assert ds.error() & R.RSSM_DEVERR_ACCEPT_RANGE
    nc2, _ = counters(ds)
    assert np.all(nc2[0] == 4 * T) and np.all(nc2[1:] == 1)
    # out-of-range accepted count
    acc3 = np.zeros(wl.batch, np.int32)
    acc3[1] = T + 1
    verify(ds, T, to_dev_inputs(draft_inputs(wl, 10, seqs, T)), o)
    _commit(ds, dev(acc3), T)
    e = ds.error()
    assert e & R.RSSM_DEVERR_ACCEPT_RANGE
    nc3, _ = counters(ds)
    assert np.all(nc3[1] == 1) and np.all(nc3[2:] == 1)
    # flushing repairs sequence 0 and the protocol continues
    _flush(ds, wl.L)
    assert ds.error() == 0
    _, nk4 = counters(ds)
    assert np.all(nk4[0] == 4 * T)


SAMPLE8_512 = [0, 73, 146, 219, 292, 365, 438, 511]
SAMPLE8_256 = [0, 37, 74, 111, 148, 185, 222, 255]


def test_serving_shape_verify_sampled():
    """Mamba-2 verify at B=512, H=128, P=64, N=128, T=4, 128 steps; accepted prefix ~ U{0..4}.
    8 sampled sequences x all heads against the oracle at every step; every cursor of the batch
    at every step; sampled checkpoints every 32 steps."""
    wl = get_workload("m2_verify_b512")
    T, steps = wl.t_max, wl.verify_steps
    seqs = list(range(wl.batch))
    print(f"[serving verify] oracle runs for {SAMPLE8_512}", flush=True)
    ref = spec_runs(wl, SAMPLE8_512, 0, steps, T, ckpt_every=32)
    cur = cursor_run(wl, steps, verify=True, T=T)
    ds = new_state(wl, initial_state(wl, seqs))
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    idx = torch.tensor(SAMPLE8_512, device="cuda")
    worst = 0.0
    with StepSource(wl, seqs) as src:
        for s in range(steps):
            verify(ds, T, to_dev_inputs(src.drafts(s, T)), o)
            got = o[idx].cpu().numpy()
            for i, b in enumerate(SAMPLE8_512):
                worst = max(worst, relerr(got[i], ref[b]["O"][s]).max())
            _commit(ds, dev(accept_counts(wl, s, T)), T)
            _flush(ds, wl.L)
            assert_counters(ds, *cur[s], f"step {s}")
            for b in SAMPLE8_512:
                if s in ref[b]["ckpt"]:
                    e = tile_relerr(ds.ckpt()[b].cpu().numpy(), ref[b]["ckpt"][s]).max()
                    assert e <= TOL, f"step {s} seq {b}: checkpoint rel err {e:.3g}"
            if s % 32 == 31:
                print(f"[serving verify] step {s + 1}/{steps} worst rel err {worst:.3g}", flush=True)
    assert worst <= TOL
    assert ds.error() == 0


@pytest.mark.parametrize("name", ["gdn_b256", "kda_b256"])
def test_serving_shape_gdn_decode_then_verify_sampled(name):
    """Gated DeltaNet at B=256, 32 value / 16 key heads, 128 x 128 tiles (KDA: 32 heads with
    per-channel gates): 256 decode steps, then 256 verify steps with T = 4 drafts.  8 sampled
    sequences x all heads against the oracle at every step of both phases; every cursor of the
    batch at every step of both phases; sampled checkpoints every 64 steps of both phases."""
    wl = get_workload(name)
    T = wl.t_max
    nd, nv = wl.decode_steps, wl.verify_steps
    seqs = list(range(wl.batch))
    sample = SAMPLE8_256
    print(f"[serving {name}] oracle runs for {sample}", flush=True)
    ref = spec_runs(wl, sample, nd, nv, T, ckpt_every=64)
    cur_d = cursor_run(wl, nd, verify=False)
    cur = cursor_run(wl, nv, verify=True, T=T, decode_steps=nd)
    ds = new_state(wl, initial_state(wl, seqs))
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    idx = torch.tensor(sample, device="cuda")
    worst_d = worst_v = 0.0
    with StepSource(wl, seqs) as src:
        for t in range(nd):
            decode(ds, to_dev_inputs(src.decode(t)), y)
            got = y[idx].cpu().numpy()
            for i, b in enumerate(sample):
                worst_d = max(worst_d, relerr(got[i], ref[b]["y"][t]).max())
            assert_counters(ds, *cur_d[t], f"decode step {t}")
            for b in sample:
                if t in ref[b]["ckpt_decode"]:
                    e = tile_relerr(ds.ckpt()[b].cpu().numpy(), ref[b]["ckpt_decode"][t]).max()
                    assert e <= TOL, f"decode step {t} seq {b}: checkpoint rel err {e:.3g}"
        print(f"[serving {name}] decode worst rel err {worst_d:.3g}", flush=True)
        for s in range(nv):
            verify(ds, T, to_dev_inputs(src.drafts(s, T)), o)
            got = o[idx].cpu().numpy()
            for i, b in enumerate(sample):
                worst_v = max(worst_v, relerr(got[i], ref[b]["O"][s]).max())
            _commit(ds, dev(accept_counts(wl, s, T)), T)
            _flush(ds, wl.L)
            assert_counters(ds, *cur[s], f"verify step {s}")
            for b in sample:
                if s in ref[b]["ckpt"]:
                    e = tile_relerr(ds.ckpt()[b].cpu().numpy(), ref[b]["ckpt"][s]).max()
                    assert e <= TOL, f"step {s} seq {b}: checkpoint rel err {e:.3g}"
            if s % 64 == 63:
                print(f"[serving {name}] verify step {s + 1}/{nv} worst rel err {worst_v:.3g}", flush=True)
    assert worst_d <= TOL and worst_v <= TOL
    assert ds.error() == 0


@pytest.mark.parametrize("name", ["m2_verify_b512", "gdn_b256", "kda_b256"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_snapshot_verify_small(name, dtype):
    """The snapshot-based speculative comparator: outputs of every draft against the oracle's
    verify, the committed snapshot against the oracle's committed state after every commit,
    and the committed slot untouched by verify."""
    wl = _small(name, in_dtype=dtype)
    T = wl.t_max
    S_ = T + 1
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    cfg = new_state(wl, S0).cfg
    snap = torch.zeros(wl.batch, S_, wl.n_heads, wl.dv, wl.dk, device="cuda")
    snap[:, 0] = dev(S0)
    cur = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    for s in range(12):
        dr = draft_inputs(wl, s, seqs, T)
        c = cur.cpu().numpy()
        before = torch.stack([snap[b, int(c[b])] for b in seqs]).cpu().numpy()
        d = to_dev_inputs(dr)                     # held until the kernel has run
        R.rssm_verify_snapshot(cfg, ptr(snap), ptr(cur), T, ptr(d["alpha"]), ptr(d.get("beta")), ptr(d["v"]),
                               ptr(d["k"]), ptr(d["q"]), ptr(o), ptr(err), stream())
        ref = orc.verify(dr, T)
        e = relerr(o.cpu().numpy(), ref).max()
        assert e <= TOL, f"step {s}: snapshot verify rel err {e:.3g}"
        after = torch.stack([snap[b, int(c[b])] for b in seqs]).cpu().numpy()
        assert np.array_equal(before.view(np.uint32), after.view(np.uint32))
        acc = accept_counts(wl, s, T)
        acc_d = dev(acc)
        R.rssm_commit_snapshot(cfg, ptr(cur), ptr(acc_d), T, ptr(err), stream())
        orc.commit(acc, T)
        orc.flush(wl.L)
        c = cur.cpu().numpy()
        committed = torch.stack([snap[b, int(c[b])] for b in seqs]).cpu().numpy()
        e = tile_relerr(committed, orc.S).max()
        assert e <= TOL, f"step {s}: committed snapshot rel err {e:.3g}"
    assert int(err.item()) == 0


def test_snapshot_commit_errors():
    """Out-of-range accept counts and slots set the device error word and leave the
    sequence's committed slot unchanged."""
    wl = _small("m2_verify_b512")
    cfg = new_state(wl).cfg
    T = wl.t_max
    cur = torch.tensor([0, 1, 2, 3, 4, 0], dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc = torch.tensor([1, T + 1, -1, 2, 0, 3], dtype=torch.int32, device="cuda")
    R.rssm_commit_snapshot(cfg, ptr(cur), ptr(acc), T, ptr(err), stream())
    torch.cuda.synchronize()
    assert cur.cpu().tolist() == [1, 1, 2, 0, 4, 3]
    assert int(err.item()) == R.RSSM_DEVERR_ACCEPT_RANGE
    err.zero_()
    cur = torch.tensor([T + 1, 0, 0, 0, 0, 0], dtype=torch.int32, device="cuda")
    acc = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
    R.rssm_commit_snapshot(cfg, ptr(cur), ptr(acc), T, ptr(err), stream())
    torch.cuda.synchronize()
    assert cur.cpu().tolist()[0] == T + 1
    assert int(err.item()) == R.RSSM_DEVERR_CURSOR


def _tree_step(ds, orc, wl, s, T, seqs, o, ring=True):
    parent, path, a = draft_tree(wl, s, T)
    dr = draft_inputs(wl, 300 + s, seqs, T)
    d = to_dev_inputs(dr)
    par_d, path_d, acc_d = dev(parent), dev(path), dev(a)
    R.rssm_verify_tree(ds.cfg, ds.st, T, ptr(par_d), ptr(d["alpha"]), ptr(d.get("beta")), ptr(d["v"]),
                       ptr(d["k"]), ptr(d["q"]), ptr(o), stream())
    ref = orc.verify_tree(dr, T, parent)
    e = relerr(o.cpu().numpy(), ref).max()
    assert e <= TOL, f"step {s}: tree verify rel err {e:.3g}"
    R.rssm_commit_tree(ds.cfg, ds.st, ptr(par_d), ptr(path_d), ptr(acc_d), T, stream())
    orc.commit_tree(path, a, T)
    _flush(ds, wl.L)
    orc.flush(wl.L)
    assert_counters(ds, orc.n_committed, orc.n_ckpt, f"step {s}")
    if ring:
        check_ring(ds, orc, seqs)
    folded = orc.n_ckpt == orc.n_committed
    if folded.any():
        e = tile_relerr(ds.ckpt().cpu().numpy()[folded], orc.S_ckpt[folded]).max()
        assert e <= TOL, f"step {s}: checkpoint rel err {e:.3g}"


@pytest.mark.parametrize("name", ["m2_verify_b512", "gdn_b256", "kda_b256"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tree_spec_small(name, dtype):
    """Tree-shaped drafts: verify_tree -> commit_tree(path) -> flush(L) against the oracle:
    every output, cursor, committed (compacted) ring record and checkpoint."""
    wl = _small(name, in_dtype=dtype)
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    for s in range(24):
        _tree_step(ds, orc, wl, s, T, seqs, o)
    assert ds.error() == 0


def test_chain_tree_matches_linear_verify_bits():
    """A tree in which every draft hangs off the previous one is the linear chain: the
    outputs are bit-identical to rssm_verify's."""
    for name in ("m2_verify_b512", "gdn_b256", "kda_b256"):
        wl = _small(name)
        T = wl.t_max
        seqs = list(range(wl.batch))
        S0 = initial_state(wl, seqs)
        lin, tree = new_state(wl, S0), new_state(wl, S0)
        chain = dev(np.tile(np.arange(-1, T - 1, dtype=np.int32), (wl.batch, 1)))
        o1 = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
        o2 = torch.empty_like(o1)
        for s in range(6):
            d = to_dev_inputs(draft_inputs(wl, s, seqs, T))
            verify(lin, T, d, o1)
            R.rssm_verify_tree(tree.cfg, tree.st, T, ptr(chain), ptr(d["alpha"]), ptr(d.get("beta")), ptr(d["v"]),
                               ptr(d["k"]), ptr(d["q"]), ptr(o2), stream())
            assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
            acc_d = dev(accept_counts(wl, s, T))
            _commit(lin, acc_d, T)
            path = np.where(np.arange(T)[None, :] < accept_counts(wl, s, T)[:, None], np.arange(T)[None, :], -1)
            path_d = dev(path.astype(np.int32))
            R.rssm_commit_tree(tree.cfg, tree.st, ptr(chain), ptr(path_d), ptr(acc_d), T, stream())
            _flush(lin, wl.L)
            _flush(tree, wl.L)
        assert torch.equal(lin.ckpt().view(torch.int32), tree.ckpt().view(torch.int32))
        assert lin.error() == 0 and tree.error() == 0


def test_tree_contract_errors():
    """An invalid parent index sets RSSM_DEVERR_TREE and appends nothing; a path that is not
    a chain from the head sets RSSM_DEVERR_ACCEPT_RANGE and moves nothing."""
    wl = _small("m2_verify_b512")
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    ds = new_state(wl, S0)
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    d = to_dev_inputs(draft_inputs(wl, 0, seqs, T))
    parent = np.tile(np.array([-1, 0, 0, 1], np.int32), (wl.batch, 1))
    parent[1, 2] = 2
    par_d = dev(parent)
    ring_before = {k: (None if v is None else v.clone()) for k, v in ds.ring_arrays().items()}
    R.rssm_verify_tree(ds.cfg, ds.st, T, ptr(par_d), ptr(d["alpha"]), None, ptr(d["v"]), ptr(d["k"]), ptr(d["q"]),
                       ptr(o), stream())
    assert ds.error() == R.RSSM_DEVERR_TREE
    ring_after = ds.ring_arrays()
    assert torch.equal(ring_before["v"][1], ring_after["v"][1])
    good = dev(np.tile(np.array([-1, 0, 0, 1], np.int32), (wl.batch, 1)))
    R.rssm_verify_tree(ds.cfg, ds.st, T, ptr(good), ptr(d["alpha"]), None, ptr(d["v"]), ptr(d["k"]), ptr(d["q"]),
                       ptr(o), stream())
    path = np.full((wl.batch, T), -1, np.int32)
    path[0, :2] = [0, 2]
    path[2, :2] = [1, 0]
    path[3, :2] = [0, 3]
    acc = np.array([2, 0, 2, 2, 0, 0], np.int32)
    path_d, acc_d = dev(path), dev(acc)
    R.rssm_commit_tree(ds.cfg, ds.st, ptr(good), ptr(path_d), ptr(acc_d), T, stream())
    assert ds.error() == R.RSSM_DEVERR_ACCEPT_RANGE
    nc, _ = counters(ds)
    assert nc[:, 0].tolist() == [2, 0, 0, 0, 0, 0]


def test_tree_commit_refuses_a_tree_the_verify_refused():
    """A parent row the verify refused (draft 0 hanging off the later draft 1) appended
    nothing, so a commit of it must move nothing either, even for a path that follows that
    row's parent links ([1, 0]): RSSM_DEVERR_ACCEPT_RANGE, cursor and ring unchanged.  The
    oracle refuses the same commit."""
    wl = _small("m2_verify_b512")
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    ds = new_state(wl, S0)
    orc = ReplayOracle(wl, seqs, S0)
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    dr = draft_inputs(wl, 0, seqs, T)
    d = to_dev_inputs(dr)
    parent = np.tile(np.array([-1, 0, 0, 1], np.int32), (wl.batch, 1))
    parent[2] = [1, -1, 0, 1]
    par_d = dev(parent)
    R.rssm_verify_tree(ds.cfg, ds.st, T, ptr(par_d), ptr(d["alpha"]), None, ptr(d["v"]), ptr(d["k"]), ptr(d["q"]),
                       ptr(o), stream())
    orc.verify_tree(dr, T, parent)
    assert ds.error() == R.RSSM_DEVERR_TREE
    ring_before = {k: (None if v is None else v.clone()) for k, v in ds.ring_arrays().items()}
    path = np.full((wl.batch, T), -1, np.int32)
    path[:, :2] = [0, 1]
    path[2, :2] = [1, 0]
    acc = np.full(wl.batch, 2, np.int32)
    path_d, acc_d = dev(path), dev(acc)           # alive until the kernel has run
    R.rssm_commit_tree(ds.cfg, ds.st, ptr(par_d), ptr(path_d), ptr(acc_d), T, stream())
    orc.commit_tree(path, acc, T)
    assert ds.error() == R.RSSM_DEVERR_ACCEPT_RANGE and orc.err
    nc, _ = counters(ds)
    assert nc[:, 0].tolist() == [2, 2, 0, 2, 2, 2] == orc.n_committed.tolist()
    ring_after = ds.ring_arrays()
    for k in ("alpha", "v", "k", "q"):
        assert torch.equal(ring_before[k][2], ring_after[k][2]), k


def test_invalid_tree_in_fused_verify_leaves_sequence_untouched():
    """verify_fold with an invalid draft tree: that sequence is neither folded nor appended
    (checkpoint bits, n_ckpt and ring unchanged), RSSM_DEVERR_TREE is set; the other
    sequences fold and verify as usual."""
    wl = _small("gdn_b256")
    wl = wl.replace(capacity=wl.L + 2 * wl.t_max - 1)
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    ds = new_state(wl, S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    for t in range(3):
        decode(ds, to_dev_inputs(decode_inputs(wl, t, seqs)), y)
    ck_before = ds.ckpt().clone()
    ring_before = {k: (None if v is None else v.clone()) for k, v in ds.ring_arrays().items()}
    parent = np.tile(np.array([-1, 0, 1, 1], np.int32), (wl.batch, 1))
    parent[2, 3] = 3                                   # not an earlier draft
    par_d = dev(parent)
    d = to_dev_inputs(draft_inputs(wl, 0, seqs, T))
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    R.rssm_verify_fold(ds.cfg, ds.st, 3, T, ptr(par_d), ptr(d["alpha"]), ptr(d["beta"]), ptr(d["v"]),
                       ptr(d["k"]), ptr(d["q"]), ptr(o), stream())
    assert ds.error() == R.RSSM_DEVERR_TREE
    nc, nk = counters(ds)
    assert nk[2].tolist() == [0] * wl.n_heads and nc[2].tolist() == [3] * wl.n_heads
    assert torch.equal(ds.ckpt()[2].view(torch.int32), ck_before[2].view(torch.int32))
    ring_after = ds.ring_arrays()
    for f in ("alpha", "beta", "v"):
        assert torch.equal(ring_before[f][2], ring_after[f][2]), f
    others = [b for b in seqs if b != 2]
    assert all(nk[b].tolist() == [3] * wl.n_heads for b in others)
    assert not torch.equal(ds.ckpt()[0].view(torch.int32), ck_before[0].view(torch.int32))


def test_tree_spec_full_heads():
    """Tree speculation at the serving head shape (H=128, P=64, N=128, bf16, C=19) for a
    batch of 12 sequences, 40 steps: every output, cursor and checkpoint."""
    wl = get_workload("m2_verify_b512").replace(batch=12)
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    for s in range(40):
        _tree_step(ds, orc, wl, s, T, seqs, o, ring=(s % 8 == 0))
    assert ds.error() == 0


def _fused_loop(wl, steps, tree, seed0=400):
    """verify_fold(L) -> commit per step against the oracle's flush(L) -> verify -> commit:
    outputs, cursors and checkpoints after every call.  Returns the number of folds of a
    window holding L + T - 1 records (the most a window reaches between folds)."""
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    full = 0
    for s in range(steps):
        nk0 = orc.n_ckpt.copy()
        hb = orc.n_committed - nk0
        fold = hb >= wl.L
        full += int(np.sum(hb == wl.L + T - 1))
        dr = draft_inputs(wl, seed0 + s, seqs, T)
        d = to_dev_inputs(dr)
        if tree:
            parent, path, a = draft_tree(wl, s, T)
        else:
            parent, a = None, np.full(wl.batch, T, np.int32) if s % 3 == 0 else accept_counts(wl, s, T)
            path = None
        par_d = dev(parent) if tree else None
        R.rssm_verify_fold(ds.cfg, ds.st, wl.L, T, ptr(par_d), ptr(d["alpha"]), ptr(d.get("beta")), ptr(d["v"]),
                           ptr(d["k"]), ptr(d["q"]), ptr(o), stream())
        orc.flush(wl.L)
        ref = orc.verify_tree(dr, T, parent) if tree else orc.verify(dr, T)
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"step {s} after verify_fold")
        e = relerr(o.cpu().numpy(), ref).reshape(wl.batch, -1).max(axis=1)
        bad = np.flatnonzero(e > TOL)
        assert bad.size == 0, (f"step {s}: fused verify rel err {e.max():.3g}; sequences {bad.tolist()} "
                               f"(window {hb[bad].tolist()}, folded {fold[bad].tolist()}, "
                               f"n_ckpt before {nk0[bad].tolist()})")
        if fold.any():
            e = tile_relerr(ds.ckpt().cpu().numpy()[fold], orc.S_ckpt[fold]).max()
            assert e <= TOL, f"step {s}: checkpoint rel err {e:.3g}"
        acc_d = dev(a)
        if tree:
            path_d = dev(path)
            R.rssm_commit_tree(ds.cfg, ds.st, ptr(par_d), ptr(path_d), ptr(acc_d), T, stream())
            orc.commit_tree(path, a, T)
        else:
            _commit(ds, acc_d, T)
            orc.commit(a, T)
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"step {s} after commit")
    assert ds.error() == 0
    return full


@pytest.mark.parametrize("name", ["m2_verify_b512", "gdn_b256", "kda_b256"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("tree", [False, True])
def test_verify_with_fused_flush(name, dtype, tree):
    """The fused loop at small shapes, the ring sized C = L + 2T - 1 as the fused call needs;
    the linear loop must fold windows at their largest (L + T - 1 records)."""
    wl = _small(name, in_dtype=dtype)
    wl = wl.replace(capacity=wl.L + 2 * wl.t_max - 1)
    full = _fused_loop(wl, 30, tree)
    if not tree:
        assert full > 0, "no window reached L + T - 1 records before its fold"


def test_verify_with_fused_flush_full_heads():
    """The fused loop at the serving head shape of Gated DeltaNet (32 value heads sharing 16
    key heads: the key records a folding head reads are shared with its sibling head)."""
    wl = get_workload("gdn_b256").replace(batch=8)
    wl = wl.replace(capacity=wl.L + 2 * wl.t_max - 1)
    _fused_loop(wl, 24, tree=False)


def test_verify_fold_capacity_rule():
    """A window that cannot take T drafts before its fold is a capacity error, untouched."""
    wl = _small("m2_verify_b512", in_dtype="fp32")
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    ds = new_state(wl, S0)
    o = torch.zeros(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    full = np.full(wl.batch, T, np.int32)
    for s in range(4):                  # 16 committed records, C = 19
        d = to_dev_inputs(draft_inputs(wl, 500 + s, seqs, T))
        R.rssm_verify(ds.cfg, ds.st, T, ptr(d["alpha"]), None, ptr(d["v"]), ptr(d["k"]), ptr(d["q"]), ptr(o),
                      stream())
        acc_d = dev(full)
        _commit(ds, acc_d, T)
    assert ds.error() == 0
    nc0, nk0 = counters(ds)
    ck0 = ds.ckpt().clone()
    d = to_dev_inputs(draft_inputs(wl, 600, seqs, T))
    o.zero_()
    R.rssm_verify_fold(ds.cfg, ds.st, wl.L, T, None, ptr(d["alpha"]), None, ptr(d["v"]), ptr(d["k"]),
                       ptr(d["q"]), ptr(o), stream())
    assert ds.error() == R.RSSM_DEVERR_VERIFY_CAPACITY
    nc1, nk1 = counters(ds)
    assert np.array_equal(nc0, nc1) and np.array_equal(nk0, nk1)
    assert torch.equal(ck0, ds.ckpt())
    assert not o.any()


MAX_SHAPES = [
    # name, dv, dk: T = 8 drafts (the maximum) and C = 32 ring slots (the maximum), L = C - T + 1
    ("m2_verify_b512", 64, 256),
    ("gdn_b256", 128, 128),
    ("kda_b256", 64, 128),
]


@pytest.mark.parametrize("shape", MAX_SHAPES, ids=lambda s: f"{s[0]}-{s[1]}x{s[2]}")
def test_spec_at_maximum_drafts_and_capacity(shape):
    """The largest draft count (8) and ring (32 slots) the ABI allows, at the widest tiles the
    LDS budget admits: linear verify -> commit -> flush(L), then tree verify -> commit_tree ->
    flush(L), then the flush fused into the verify, each against the oracle."""
    name, P, N = shape
    _spec_linear_tree_fused(_small(name, batch=3, dv=P, dk=N, t_max=8, capacity=32, L=25))


WIDE_SHAPES = [
    # name, dv, dk: the widest tiles the kernels accept (16 row groups of 8 per wave at dk = 32,
    # 8 at dk = 64), ragged row counts included; T = 4, C = 19, L = 16
    ("m2_verify_b512", 512, 32),
    ("gdn_b256", 512, 32),
    ("kda_b256", 500, 32),
    ("m2_verify_b512", 250, 64),
]


@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=lambda s: f"{s[0]}-{s[1]}x{s[2]}")
def test_spec_at_widest_tiles(shape):
    name, P, N = shape
    _spec_linear_tree_fused(_small(name, batch=3, dv=P, dk=N, t_max=4, capacity=19, L=16))


def _spec_linear_tree_fused(wl):
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    for s in range(12):
        d = draft_inputs(wl, s, seqs, T)
        verify(ds, T, to_dev_inputs(d), o)
        err = relerr(o.cpu().numpy(), orc.verify(d, T)).max()
        assert err <= TOL, f"verify step {s}: rel err {err:.3g}"
        acc = accept_counts(wl, s, T)[: wl.batch]
        _commit(ds, dev(acc), T)
        orc.commit(acc, T)
        _flush(ds, wl.L)
        orc.flush(wl.L)
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"step {s}")
        e = tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max()
        assert e <= TOL, f"step {s}: checkpoint rel err {e:.3g}"
    for s in range(12):
        _tree_step(ds, orc, wl, 100 + s, T, seqs, o)
    assert ds.error() == 0
    _fused_loop(wl.replace(L=wl.capacity - 2 * T + 1), 12, tree=False)


@pytest.mark.parametrize("name", ["m2_verify_b512", "kda_b256"])
def test_group_appends_between_speculative_rounds(name):
    """With 16 value heads the decode appends each group's records from the group's last
    workgroup.  Decode steps alternate with verify(T) / commit(a) / flush(L) rounds, so those
    appends land after committed drafts, after folds and at every window phase: every output,
    cursor and checkpoint against the oracle, and every live ring slot bit for bit."""
    wl = _small(name, batch=5, n_heads=16, n_qk_heads=16 if name.startswith("m2") else 8)
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    for s in range(24):
        for t in range(2):
            inp = decode_inputs(wl, 1000 + 2 * s + t, seqs)
            decode(ds, to_dev_inputs(inp), y)
            err = relerr(y.cpu().numpy(), orc.decode(inp)).max()
            assert err <= TOL, f"round {s} decode {t}: rel err {err:.3g}"
            assert_counters(ds, orc.n_committed, orc.n_ckpt, f"round {s} decode {t}")
            check_ring(ds, orc, seqs)
        d = draft_inputs(wl, s, seqs, T)
        verify(ds, T, to_dev_inputs(d), o)
        err = relerr(o.cpu().numpy(), orc.verify(d, T)).max()
        assert err <= TOL, f"round {s}: verify rel err {err:.3g}"
        acc = accept_counts(wl, s, T)[: wl.batch]
        _commit(ds, dev(acc), T)
        orc.commit(acc, T)
        _flush(ds, wl.L)
        orc.flush(wl.L)
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"round {s} after flush")
        check_ring(ds, orc, seqs)
        e = tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max()
        assert e <= TOL, f"round {s}: checkpoint rel err {e:.3g}"
    assert ds.error() == 0
