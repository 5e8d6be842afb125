"""GPU parity of the low-precision read copy (fp8 E4M3 / MXFP4): quantiser bits,
exact readout through the non-flush path, outputs against the oracle, and the
invariant that the fp32 checkpoint trajectory is untouched by the copy."""
import numpy as np
import pytest
import torch

from oracle import (ReplayOracle, dequantize_fp8_blocks, dequantize_mxfp4_blocks,
                    quantize_fp8_blocks, quantize_mxfp4_blocks)
from synth import decode_inputs, draft_inputs, get_workload, initial_state
from synth.stream import StepSource

from gpu_util import (TOL, TOL_READ, assert_counters, check_ring, decode, dev, new_state, ptr, read_copy_excess,
                      relerr, stream, tile_relerr, to_dev_inputs, verify)
from attention_decode_mamba_amd import rssm as R
from oracle_runs import READ_TOL, decode_runs

pytestmark = pytest.mark.gpu


def _wl(fmt, **kw):
    base = dict(name="rc", batch=3, n_heads=4, n_qk_heads=4, dv=40, dk=64, in_dtype="fp32", L=5,
                capacity=5, read_copy=fmt)
    base.update(kw)
    return get_workload("m2_readcopy_b256").replace(**base)


def _special_s0(wl):
    S0 = initial_state(wl, range(wl.batch))
    S0[0, 0, 0, :32] = 0.0                       # all-zero block
    S0[0, 0, 1, :32] = 2.0 ** -140               # tiny block (denormal values)
    S0[0, 1, 2, :] = np.float32(448.0)           # exact maximum
    S0[1, 0, 3, 5] = 1e4                          # one large outlier per block
    return S0


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("dk", [32, 64, 128])
def test_init_quantiser_bits(fmt, dk):
    wl = _wl(fmt, dk=dk)
    S0 = _special_s0(wl)
    ds = new_state(wl, S0)
    codes, scales = ds.read_copy()
    if fmt == "fp8":
        rc, rs = quantize_fp8_blocks(S0)
        assert np.array_equal(codes.cpu().numpy(), rc)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    else:
        rc, rs = quantize_mxfp4_blocks(S0)
        assert np.array_equal(codes.cpu().numpy(), rc)
        assert np.array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_exact_readout_through_decode(fmt):
    """alpha = 1, v = 0, k = 0, q = e_n: a non-flush output is column n of the dequantised
    copy (one rounding of code * scale), a flush output is column n of the fp32 state."""
    wl = _wl(fmt, dk=32, L=5, capacity=5)
    B, H, P, N = wl.batch, wl.n_heads, wl.dv, wl.dk
    S0 = _special_s0(wl)
    ds = new_state(wl, S0)
    if fmt == "fp8":
        deq = dequantize_fp8_blocks(*quantize_fp8_blocks(S0))
    else:
        deq = dequantize_mxfp4_blocks(*quantize_mxfp4_blocks(S0))
    deq32 = deq.astype(np.float32)
    y = torch.empty(B, H, P, device="cuda")
    inp = {"alpha": np.ones((B, H), np.float32), "beta": None, "v": np.zeros((B, H, P), np.float32),
           "k": np.zeros((B, H, N), np.float32)}
    for t in range(5 * N):
        n = t % N
        q = np.zeros((B, H, N), np.float32)
        q[:, :, n] = 1.0
        decode(ds, to_dev_inputs(dict(inp, q=q)), y)
        got = y.cpu().numpy()
        flush = (t + 1) % wl.L == 0
        want = S0[:, :, :, n] if flush else deq32[:, :, :, n]
        # exact equality (a code for -0 reads back as +0 through the FMA chain, so compare values)
        assert np.array_equal(got, want), f"step {t} column {n} flush={flush}"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("shape", [(40, 64, "fp32"), (17, 32, "bf16"), (128, 128, "bf16"), (64, 128, "bf16"),
                                   (64, 128, "fp32"), (24, 128, "bf16"), (8, 64, "bf16"), (48, 128, "fp32")])
def test_decode_with_read_copy_matches_oracle(fmt, shape):
    P, N, dt = shape
    wl = _wl(fmt, dv=P, dk=N, in_dtype=dt, L=6, capacity=6)
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0, read_tol=READ_TOL)
    ds = new_state(wl, S0)
    plain = new_state(wl.replace(read_copy="none"), S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    y2 = torch.empty_like(y)
    for t in range(20):
        inp = decode_inputs(wl, t, seqs)
        d = to_dev_inputs(inp)
        decode(ds, d, y)
        decode(plain, d, y2)
        yr = orc.decode(inp)
        got = y.cpu().numpy()
        err = relerr(got, yr).max()
        if fmt == "fp8":
            assert err <= TOL_READ, f"step {t}: rel err {err:.3g}"
        ex = read_copy_excess(got, yr, orc.allowance).max()
        assert ex <= 0, f"step {t}: output outside fp32 tolerance + quantisation ambiguity by {ex:.3g}"
        # the copy never feeds the recurrence: checkpoints are bit-identical to the plain run
        assert torch.equal(ds.ckpt().view(torch.int32), plain.ckpt().view(torch.int32))
        if (t + 1) % wl.L == 0:
            assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
        if (t + 1) % wl.L == 0:
            assert tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max() <= TOL
    assert ds.error() == 0


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("dt,H,G", [("bf16", 6, 3), ("fp32", 6, 3), ("bf16", 16, 16), ("bf16", 32, 8)])
def test_read_copy_decode_staggered_windows(fmt, dt, H, G):
    """Mamba-2 read-copy decode at P = 64, N = 128 with a 16-record window, the shape served
    with one tile per wave and one head of four sequences per workgroup: 5 sequences x 6
    value heads over 3 key heads (the workgroups of sequence 4 hold one tile), windows
    staggered by verify(T = 1) /
    commit rounds (sequence b holds 3b mod 16 records) so that sequences fold at different
    steps, then 40 decode steps.  Outputs against the oracle (fp32 tolerance plus the
    quantisation ambiguity bound; fp8 also normwise); checkpoints bit-identical to the run
    without a copy at every step, and so are a sequence's outputs at its fold steps; cursors;
    every live ring slot bit for bit (also at 16 and 32 heads, where the decode on the fp32
    tile appends each group of heads, 16 or 32, from its last workgroup); the final read copy equal to
    the quantised final checkpoint."""
    wl = _wl(fmt, batch=5, n_heads=H, n_qk_heads=G, dv=64, dk=128, in_dtype=dt, L=16, capacity=16, t_max=1)
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0, read_tol=READ_TOL)
    ds = new_state(wl, S0)
    plain = new_state(wl.replace(read_copy="none"), S0)
    o1 = torch.empty(wl.batch, 1, wl.n_heads, wl.dv, device="cuda")
    for r in range(wl.L - 1):
        d = draft_inputs(wl, 100 + r, seqs, 1)
        dd = to_dev_inputs(d)
        acc = np.array([1 if r < (3 * b) % wl.L else 0 for b in seqs], np.int32)
        acc_d = dev(acc)                               # stays alive until the commits have run
        for st in (ds, plain):
            verify(st, 1, dd, o1)
            R.rssm_commit(st.cfg, st.st, ptr(acc_d), 1, stream())
        orc.verify(d, 1)
        orc.commit(acc, 1)
    assert_counters(ds, orc.n_committed, orc.n_ckpt, "after staggering")
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    y2 = torch.empty_like(y)
    folds = np.zeros(wl.batch, int)
    for t in range(40):
        fold = orc.h() + 1 >= wl.L
        folds += fold
        inp = decode_inputs(wl, t, seqs)
        d = to_dev_inputs(inp)
        decode(ds, d, y)
        decode(plain, d, y2)
        yr = orc.decode(inp)
        got = y.cpu().numpy()
        ex = read_copy_excess(got, yr, orc.allowance).max()
        assert ex <= 0, f"step {t}: output outside fp32 tolerance + quantisation ambiguity by {ex:.3g}"
        if fmt == "fp8":
            assert relerr(got, yr).max() <= TOL_READ, f"step {t}"
        assert torch.equal(ds.ckpt().view(torch.int32), plain.ckpt().view(torch.int32)), f"step {t}"
        for b in np.nonzero(fold)[0]:
            assert torch.equal(y[b].view(torch.int32), y2[b].view(torch.int32)), f"step {t} fold of sequence {b}"
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"step {t}")
        check_ring(ds, orc, seqs)
    assert folds.min() >= 2
    codes, scales = ds.read_copy()
    ck = ds.ckpt().cpu().numpy()
    if fmt == "fp8":
        rc, rs = quantize_fp8_blocks(ck)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    else:
        rc, rs = quantize_mxfp4_blocks(ck)
        assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert ds.error() == 0 and plain.error() == 0 and not orc.err


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_serving_shape_read_copy_sampled(fmt):
    """Mamba-2 serving shape (B=256, H=128, P=64, N=128, bf16) with a read copy, 512 steps.

    Each output row must match the oracle (which quantises its own fp32 checkpoint) to the fp32
    tolerance plus the oracle's bound on what an element lying within that tolerance of a
    rounding boundary may change; the normwise error is also held to 5e-2 for fp8 and, for
    MXFP4, on every row whose allowance is zero (a single ambiguous E2M1 code moves a row by a
    few percent); the worst MXFP4 error and the share of rows that needed the allowance are
    reported."""
    wl = get_workload("m2_readcopy_b256").replace(read_copy=fmt)
    steps = 512
    seqs = list(range(wl.batch))
    sample = [0, 100, 255]
    print(f"[read copy {fmt}] oracle runs for {sample}", flush=True)
    ref = decode_runs(wl, sample, steps)
    ds = new_state(wl, initial_state(wl, seqs))
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    idx = torch.tensor(sample, device="cuda")
    worst = 0.0
    worst_plain = 0.0                             # rows whose allowance is zero
    excess = -1.0
    rows = needed = 0
    with StepSource(wl, seqs) as src:
        for t in range(steps):
            decode(ds, to_dev_inputs(src.decode(t)), y)
            got = y[idx].cpu().numpy()
            for i, b in enumerate(sample):
                yr, allow = ref[b]["y"][t], np.asarray(ref[b]["allowance"][t])
                err = relerr(got[i], yr)
                worst = max(worst, err.max())
                plain = np.broadcast_to(allow, got[i].shape).max(axis=-1) == 0
                if plain.any():
                    worst_plain = max(worst_plain, err[plain].max())
                ex_fp32 = read_copy_excess(got[i], yr, 0.0).max(axis=-1)
                rows += err.size
                needed += int((ex_fp32 > 0).sum())
                excess = max(excess, read_copy_excess(got[i], yr, allow).max())
            if t % 128 == 127:
                print(f"[read copy {fmt}] step {t + 1}/{steps} worst normwise rel err {worst:.3g} "
                      f"({worst_plain:.3g} on rows without allowance), worst excess over "
                      f"tolerance+ambiguity {excess:.3g}, rows that needed the allowance "
                      f"{needed}/{rows}", flush=True)
    assert excess <= 0
    assert worst_plain <= TOL_READ
    if fmt == "fp8":
        assert worst <= TOL_READ
    assert ds.error() == 0


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_delta_rule_decode_with_read_copy(kind, fmt):
    """Gated DeltaNet and KDA decode with a read copy: non-flush outputs come from the copy
    through the delta-rule sweep.  Each output within 5e-2 (normwise) of the oracle, which
    quantises its own fp32 checkpoint and steps a chain restarted from the dequantised copy
    (the difference left is fp32 rounding and the odd element at a rounding boundary); flush
    steps from the fp32 state to the fp32 tolerance; checkpoints bit-identical to a run
    without the copy."""
    wl = get_workload("gdn_b256" if kind == "gdn" else "kda_b256").replace(
        name="rc", batch=3, n_heads=4, n_qk_heads=2, dv=40, dk=64, in_dtype="bf16", L=5, t_max=1,
        capacity=5, read_copy=fmt)
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    plain = new_state(wl.replace(read_copy="none"), S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    y2 = torch.empty_like(y)
    for t in range(20):
        inp = decode_inputs(wl, t, seqs)
        d = to_dev_inputs(inp)
        decode(ds, d, y)
        decode(plain, d, y2)
        yr = orc.decode(inp)
        err = relerr(y.cpu().numpy(), yr).max()
        flush = (t + 1) % wl.L == 0
        assert err <= (TOL if flush else TOL_READ), f"step {t}: rel err {err:.3g} (flush={flush})"
        assert torch.equal(ds.ckpt().view(torch.int32), plain.ckpt().view(torch.int32))
        if flush:
            assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
            assert tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max() <= TOL
    assert ds.error() == 0


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("L", [2, 3])
def test_read_copy_shortest_windows(fmt, L):
    """The shortest windows through the one-wave read-copy decode (P = 64, N = 128, bf16): with
    L = 2 every non-fold step replays only the step's own record over the copy, and every
    other step folds.  Outputs against the oracle, checkpoints bit-identical to the run
    without a copy, cursors."""
    wl = _wl(fmt, dv=64, dk=128, in_dtype="bf16", L=L, capacity=L, batch=3, n_heads=4, n_qk_heads=2)
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0, read_tol=READ_TOL)
    ds = new_state(wl, S0)
    plain = new_state(wl.replace(read_copy="none"), S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    y2 = torch.empty_like(y)
    for t in range(3 * L + 1):
        inp = decode_inputs(wl, t, seqs)
        d = to_dev_inputs(inp)
        decode(ds, d, y)
        decode(plain, d, y2)
        yr = orc.decode(inp)
        got = y.cpu().numpy()
        assert read_copy_excess(got, yr, orc.allowance).max() <= 0, f"step {t}"
        if fmt == "fp8":
            assert relerr(got, yr).max() <= TOL_READ, f"step {t}"
        assert torch.equal(ds.ckpt().view(torch.int32), plain.ckpt().view(torch.int32)), f"step {t}"
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"step {t}")
    assert ds.error() == 0


@pytest.mark.parametrize("fmt", ["none", "fp8", "mxfp4"])
def test_decode_cursor_error_leaves_the_tile_untouched(fmt):
    """Counters out of range on two tiles (n_ckpt past n_committed; a window longer than the
    ring) set the device error bit and leave those tiles' cursors, output rows and checkpoints
    untouched, over a non-fold step and a fold step of the others.  Every other tile, including
    those that share a workgroup with a broken one in the read-copy kernel, matches a run
    without the corruption bit for bit."""
    wl = _wl(fmt, dv=64, dk=128, in_dtype="bf16", L=6, capacity=6, batch=3, n_heads=4, n_qk_heads=4)
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
    nk[1, 2] = nc[1, 2] + 1                       # h < 0
    nc[2, 0] = nk[2, 0] + wl.capacity + 1         # h > C
    bad = [(1, 2), (2, 0)]
    keep_nc, keep_nk = nc.clone(), nk.clone()
    keep_ck = ds.ckpt().clone()
    good = torch.ones(wl.batch, wl.n_heads, dtype=torch.bool)
    for b, h in bad:
        good[b, h] = False
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
        gy, ry = y.cpu()[good], y2.cpu()[good]
        assert torch.equal(gy.view(torch.int32), ry.view(torch.int32)), f"step {t}: healthy outputs differ"
        rc, rk = ref.counters()
        assert torch.equal(nc.cpu()[good], rc.cpu()[good]) and torch.equal(nk.cpu()[good], rk.cpu()[good])
        assert torch.equal(ds.ckpt().cpu()[good].view(torch.int32), ref.ckpt().cpu()[good].view(torch.int32))
    assert ds.error() == R.RSSM_DEVERR_CURSOR
    assert ref.error() == 0
