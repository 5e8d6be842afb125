"""Helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np
import torch

from attention_decode_mamba_amd import rssm as R
from attention_decode_mamba_amd.state import DeviceState, config_of

TOL = 2e-5          # max normwise relative error, fp32 state
TOL_READ = 5e-2     # max normwise relative error, fp8 / MXFP4 read copy


def dev(arr):
    """numpy -> device tensor (bf16 bit patterns travel as int16)."""
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def ptr(t):
    return None if t is None else t.data_ptr()


def stream():
    return torch.cuda.current_stream().cuda_stream


def relerr(x, ref):
    """max |x - ref| / max |ref| along the last axis (normwise, per vector)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return num / np.maximum(den, 1e-30)


def tile_relerr(x, ref):
    """Normwise relative error per P x N tile."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(x - ref), axis=(-2, -1))
    den = np.max(np.abs(ref), axis=(-2, -1))
    return num / np.maximum(den, 1e-30)


def new_state(wl, S0=None):
    ds = DeviceState(config_of(wl))
    ds.init(dev(S0) if S0 is not None else None, stream())
    return ds


def decode(ds, inp, y):
    R.rssm_decode_step(ds.cfg, ds.st, ptr(inp["alpha"]), ptr(inp.get("beta")), ptr(inp["v"]),
                       ptr(inp["k"]), ptr(inp["q"]), ptr(y), stream())


def verify(ds, T, d, o):
    R.rssm_verify(ds.cfg, ds.st, T, ptr(d["alpha"]), ptr(d.get("beta")), ptr(d["v"]), ptr(d["k"]),
                  ptr(d["q"]), ptr(o), stream())


def to_dev_inputs(inp):
    return {k: dev(v) for k, v in inp.items()}


def counters(ds):
    nc, nk = ds.counters()
    return nc.cpu().numpy(), nk.cpu().numpy()


def assert_counters(ds, nc_ref, nk_ref, where=""):
    nc, nk = counters(ds)
    assert np.array_equal(nc, np.broadcast_to(np.asarray(nc_ref)[:, None], nc.shape)), f"n_committed {where}"
    assert np.array_equal(nk, np.broadcast_to(np.asarray(nk_ref)[:, None], nk.shape)), f"n_ckpt {where}"


def ring_bits(arr):
    """A torch ring view -> numpy with the same bit patterns as the stored inputs."""
    a = arr.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def read_copy_excess(got, ref, allowance):
    """Per output row: |got - ref| minus (TOL * ||ref||_inf + the oracle's ambiguity allowance).
    Positive values are violations.  Rows without an ambiguous element must match to fp32 level;
    rows with one may differ by at most the bound on the dequantised change."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    return np.abs(got - ref) - (TOL * scale + np.asarray(allowance) * (1 + 1e-9))


def check_ring(ds, orc, seqs):
    """Every live ring slot of the device state holds the oracle's record bits (alpha, v and
    beta per value head; k and q per key head)."""
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
