"""Checkpoint / resume: the caller-owned buffers (S_ckpt, read copy, ring, cursors) are the whole
state of a sequence batch (page 4 "What shipped": a checkpoint plus the buffered records; page
1, what the method does: the pointer works like a KV cache's).  Copied to the host mid-window
and back into freshly allocated buffers, a state continues bit for bit like the original; and
a flush with min_records = 1 leaves the full state in S_ckpt, equal to the stepwise recurrence."""
import numpy as np
import pytest
import torch

from attention_decode_mamba_amd import rssm as R
from attention_decode_mamba_amd.state import DeviceState
from oracle import ReplayOracle
from synth import accept_counts, decode_inputs, draft_inputs, get_workload, initial_state

from gpu_util import (TOL, assert_counters, decode, dev, new_state, ptr, relerr, stream, tile_relerr,
                      to_dev_inputs, verify)

pytestmark = pytest.mark.gpu

_BUFFERS = ("s_ckpt", "s_read", "s_read_scale", "ring", "n_committed", "n_ckpt")


def _workload(kind, read_copy):
    if kind == "mamba2":
        return get_workload("m2_verify_b512").replace(name="resume", batch=3, n_heads=16, n_qk_heads=16, dv=64,
                                                      dk=128, read_copy=read_copy)
    base = get_workload("gdn_b256" if kind == "gdn" else "kda_b256")
    return base.replace(name="resume", batch=3, n_heads=4, n_qk_heads=2, dv=48, dk=64, read_copy=read_copy)


def _round(ds, wl, s, seqs, o):
    T = wl.t_max
    d = to_dev_inputs(draft_inputs(wl, 500 + s, seqs, T))
    verify(ds, T, d, o)
    acc = dev(accept_counts(wl, s, T)[: wl.batch])
    R.rssm_commit(ds.cfg, ds.st, ptr(acc), T, stream())
    R.rssm_flush(ds.cfg, ds.st, wl.L, stream())
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind,read_copy", [("mamba2", "none"), ("mamba2", "fp8"), ("gdn", "none"), ("kda", "none")])
def test_state_copied_out_and_back_resumes_bit_for_bit(kind, read_copy):
    wl = _workload(kind, read_copy)
    T = wl.t_max
    seqs = list(range(wl.batch))
    ds = new_state(wl, initial_state(wl, seqs))
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    o = torch.empty(wl.batch, T, wl.n_heads, wl.dv, device="cuda")
    for t in range(wl.L // 2 + 3):                      # mid-window, with a speculative round
        decode(ds, to_dev_inputs(decode_inputs(wl, t, seqs)), y)
    _round(ds, wl, 0, seqs, o)
    for t in range(3):
        decode(ds, to_dev_inputs(decode_inputs(wl, 100 + t, seqs)), y)
    torch.cuda.synchronize()
    saved = {n: (None if getattr(ds, n) is None else getattr(ds, n).cpu()) for n in _BUFFERS}

    rs = DeviceState(ds.cfg)                            # fresh buffers, never initialised
    for n in _BUFFERS:
        if saved[n] is not None:
            getattr(rs, n).copy_(saved[n].to("cuda"))
    torch.cuda.synchronize()

    y2 = torch.empty_like(y)
    o2 = torch.empty_like(o)
    for t in range(2 * wl.L):
        d = to_dev_inputs(decode_inputs(wl, 200 + t, seqs))
        decode(ds, d, y)
        decode(rs, d, y2)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32)), f"step {t}: resumed outputs differ"
        if t % 5 == 4:
            _round(ds, wl, 10 + t, seqs, o)
            _round(rs, wl, 10 + t, seqs, o2)
            assert torch.equal(o.view(torch.int32), o2.view(torch.int32)), f"step {t}: resumed verify differs"
    for n in _BUFFERS:
        a, b = getattr(ds, n), getattr(rs, n)
        if a is not None:
            assert torch.equal(a, b), f"{n} differs after resuming"
    assert ds.error() == 0 and rs.error() == 0


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_flush_one_materialises_the_full_state(kind):
    """After flush(min_records = 1) every window is empty and S_ckpt is the state of the stepwise
    recurrence over every record committed so far."""
    wl = _workload(kind, "none")
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    ds = new_state(wl, S0)
    y = torch.empty(wl.batch, wl.n_heads, wl.dv, device="cuda")
    for t in range(wl.L + 5):                            # one fold, then 5 buffered records
        inp = decode_inputs(wl, t, seqs)
        decode(ds, to_dev_inputs(inp), y)
        assert relerr(y.cpu().numpy(), orc.decode(inp)).max() <= TOL
    assert np.all(orc.n_committed - orc.n_ckpt == 5)
    R.rssm_flush(ds.cfg, ds.st, 1, stream())
    orc.flush(1)
    assert_counters(ds, orc.n_committed, orc.n_ckpt, "after flush(1)")
    nc, nk = ds.counters()
    assert torch.equal(nc, nk)
    e = tile_relerr(ds.ckpt().cpu().numpy(), orc.S_ckpt).max()
    assert e <= TOL, f"checkpoint after flush(1): rel err {e:.3g}"
    assert ds.error() == 0
