"""GPU parity on records carrying the special values of the recurrences.

The oracle pins these cases on the CPU (tests/test_oracle_pins.py,
tests/test_oracle_kda.py).  Here the HIP path must reproduce them through every
kernel of the path:
* alpha = 0, which erases the history: every decay across such a record is 0;
* alpha = 1, with no decay; KDA additionally gets gate rows of all channels 0, all 1,
  or alternating 0 / 1;
* beta = 0 (Gated DeltaNet, KDA), where the record only decays the state;
* beta = 1 with a unit-basis key: the delta rule then overwrites the state's column
  under that key with v (page 4 "Why it matters", the delta-rule update), and with
  q = k the output reads that column back;
* one key repeated in several records of a window, so later writes under the key
  replace earlier ones.

The records come from the seeded special-record recipe in synth.  For each model kind
and input dtype, at a ragged tile shape, the test runs:
* decode through two folds, which leaves the window empty;
* verify(T = 1) at h = 0, whose output must equal the decode step of the same record
  (the oracle gives both);
* 30 rounds of verify(T = 4) / commit / flush with the accepted prefix ~ U{0..4}.

Outputs, cursors and checkpoints are compared with the oracle throughout.

Error measure: normwise per output row, with the denominator floored at 1e-3 of the
call's largest row norm.  alpha = 0 together with beta = 0 makes some rows exactly
zero, and for them the plain relative error is undefined.
"""
import numpy as np
import pytest
import torch

from oracle import ReplayOracle
from synth import accept_counts, get_workload, initial_state, special_decode_inputs, special_draft_inputs

from gpu_util import (TOL, TOL_READ, assert_counters, decode, dev, new_state, ptr, stream, tile_relerr,
                      to_dev_inputs, verify)
from oracle_runs import READ_TOL
from attention_decode_mamba_amd import rssm as R

pytestmark = pytest.mark.gpu


def _wl(name, dtype):
    wl = get_workload(name)
    if name.startswith(("gdn", "kda")):
        base = dict(batch=5, n_heads=4, n_qk_heads=2 if name.startswith("gdn") else 4, dv=40, dk=64)
    else:
        base = dict(batch=5, n_heads=4, n_qk_heads=4, dv=20, dk=32)
    return wl.replace(name="special", in_dtype=dtype, L=16, t_max=4, capacity=19, **base)


def _err(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(x - ref), axis=-1)
    row = np.max(np.abs(ref), axis=-1)
    return num / np.maximum(row, 1e-3 * max(float(row.max()), 1e-30))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("name", ["m2_verify_b512", "gdn_b256", "kda_b256"])
def test_special_records(name, dtype):
    wl = _wl(name, dtype)
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    o = torch.empty(wl.batch, wl.t_max, wl.n_heads, wl.dv, device="cuda")
    for t in range(2 * wl.L):
        inp = special_decode_inputs(wl, t, seqs)
        decode(ds, to_dev_inputs(inp), y)
        e = _err(y.cpu().numpy(), orc.decode(inp)).max()
        assert e <= TOL, f"decode step {t}: rel err {e:.3g}"
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"decode step {t}")
        if (t + 1) % wl.L == 0:
            e = tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max()
            assert e <= TOL, f"fold at step {t}: checkpoint rel err {e:.3g}"
    assert np.all(orc.h() == 0)

    # verify(T = 1) at an empty window is the decode step of the same record
    d1 = special_draft_inputs(wl, 0, seqs, 1)
    o1 = torch.empty(wl.batch, 1, wl.n_heads, wl.dv, device="cuda")
    verify(ds, 1, to_dev_inputs(d1), o1)
    ref1 = orc.verify(d1, 1)
    probe = ReplayOracle(wl, seqs, orc.S.astype(np.float32))   # the same record as a decode step
    yd = probe.decode({k: (None if v is None else v[:, 0]) for k, v in d1.items()})
    assert np.max(np.abs(ref1[:, 0] - yd)) <= 1e-6 * np.max(np.abs(yd))
    e = _err(o1.cpu().numpy(), ref1).max()
    assert e <= TOL, f"verify T=1 at h=0: rel err {e:.3g}"
    acc1 = np.ones(wl.batch, np.int32)
    acc1_d = dev(acc1)                             # device arguments stay alive until their kernels run
    R.rssm_commit(ds.cfg, ds.st, ptr(acc1_d), 1, stream())
    orc.commit(acc1, 1)
    R.rssm_flush(ds.cfg, ds.st, wl.L, stream())
    orc.flush(wl.L)

    T = wl.t_max
    for s in range(1, 31):
        d = special_draft_inputs(wl, s, seqs, T)
        verify(ds, T, to_dev_inputs(d), o)
        e = _err(o.cpu().numpy(), orc.verify(d, T)).max()
        assert e <= TOL, f"verify step {s}: rel err {e:.3g}"
        acc = accept_counts(wl, s, T)[: wl.batch]
        acc_d = dev(acc)
        R.rssm_commit(ds.cfg, ds.st, ptr(acc_d), T, stream())
        orc.commit(acc, T)
        R.rssm_flush(ds.cfg, ds.st, wl.L, stream())
        orc.flush(wl.L)
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"verify step {s}")
        e = tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max()
        assert e <= TOL, f"verify step {s}: checkpoint rel err {e:.3g}"
    assert ds.error() == 0 and not orc.err


def _excess(got, ref, allowance):
    """read_copy_excess with the row scale floored like _err: alpha = 0 records leave rows
    that are small against the call's largest, where fp32 rounding of the surviving terms
    dominates."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    scale = np.maximum(scale, 1e-3 * max(float(scale.max()), 1e-30))
    return np.abs(got - ref) - (TOL * scale + np.asarray(allowance) * (1 + 1e-9))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_special_records_read_copy(fmt, dtype):
    """Special records through the Mamba-2 read-copy decode at the one-wave-per-tile shape
    (P = 64, N = 128, 16-record window; 5 sequences x 4 heads over 2 key heads): two windows of
    decode steps, then 12 rounds of verify(T = 4) / commit with the accepted prefix ~ U{0..4}
    (every fourth round also a standalone flush of windows holding at least 8 records)
    followed by three decode steps, so non-fold steps replay windows that hold committed drafts
    and records with alpha in {0, 1}, unit and repeated keys and q = k.  Outputs against the
    oracle (fp32 tolerance on the floored row scale of _err plus the oracle's quantisation
    ambiguity bound; fp8 also normwise), cursors,
    checkpoints bit-identical to a run without the copy, and against the oracle at every fold."""
    wl = get_workload("m2_readcopy_b256").replace(name="special_rc", batch=5, n_heads=4, n_qk_heads=2, dv=64,
                                                  dk=128, in_dtype=dtype, L=16, t_max=4, capacity=19,
                                                  read_copy=fmt)
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0, read_tol=READ_TOL)
    ds = new_state(wl, S0)
    plain = new_state(wl.replace(read_copy="none"), S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    y2 = torch.empty_like(y)
    o = torch.empty(wl.batch, wl.t_max, wl.n_heads, wl.dv, device="cuda")
    step = [0]

    def decode_step():
        t = step[0]
        step[0] += 1
        inp = special_decode_inputs(wl, t, seqs)
        d = to_dev_inputs(inp)
        decode(ds, d, y)
        decode(plain, d, y2)
        yr = orc.decode(inp)
        got = y.cpu().numpy()
        ex = _excess(got, yr, orc.allowance).max()
        assert ex <= 0, f"decode step {t}: outside fp32 tolerance + quantisation ambiguity by {ex:.3g}"
        if fmt == "fp8":
            assert _err(got, yr).max() <= TOL_READ, f"decode step {t}"
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"decode step {t}")
        assert torch.equal(ds.ckpt().view(torch.int32), plain.ckpt().view(torch.int32)), f"decode step {t}"

    for _ in range(2 * wl.L):
        decode_step()
    e = tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max()
    assert e <= TOL, f"checkpoint rel err {e:.3g}"
    T = wl.t_max
    for r in range(12):
        dr = special_draft_inputs(wl, 100 + r, seqs, T)
        dd = to_dev_inputs(dr)
        acc = accept_counts(wl, r, T)[: wl.batch]
        acc_d = dev(acc)                          # device arguments stay alive until their kernels run
        for st in (ds, plain):
            verify(st, T, dd, o)
            R.rssm_commit(st.cfg, st.st, ptr(acc_d), T, stream())
        orc.verify(dr, T)
        orc.commit(acc, T)
        if r % 4 == 3:                            # a standalone flush of windows holding >= 8 records
            for st in (ds, plain):
                R.rssm_flush(st.cfg, st.st, 8, stream())
            orc.flush(8)
        for _ in range(3):                        # decode folds at h >= 15, so the next verify fits
            decode_step()
        assert_counters(ds, orc.n_committed, orc.n_ckpt, f"round {r}")
        e = tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max()
        assert e <= TOL, f"round {r}: checkpoint rel err {e:.3g}"
    assert ds.error() == 0 and plain.error() == 0 and not orc.err
