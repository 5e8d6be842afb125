"""The bench's algorithmic byte model against the per-unit figures of the decode path (CPU).

Every roofline figure the bench reports divides these bytes by a measured time, so the
model is held to sizes that follow from the shapes alone:
* a ring record per (sequence, head) tile at the Mamba-2 serving shape (B=256, H=G=128,
  P=64, N=128, bf16 inputs): alpha 2 B + v 128 B read per value head, k 256 B per key head
  (386 B), and a step's append adds its q (642 B, 21.0 MB per step);
* the fp32 checkpoint: 32 KiB per tile, 1 GiB per step; a fold writes it back;
* the read copies: 9,216 B (fp8, one fp32 scale per 32 values) and 4,352 B (MXFP4, one
  E8M0 byte per 32) per tile;
* the conventional step reads and writes the state every step.
"""
import numpy as np
import pytest

import bench
from synth import get_workload

MB = 1e6


def _m2():
    return get_workload("m2_decode_b256")


def test_record_and_append_bytes():
    wl = _m2()
    head_rec, key_rec = bench._rec_bytes(wl)
    assert (head_rec, key_rec) == (2 + 128, 256)               # alpha + v, k
    B, H = wl.batch, wl.n_heads
    a = bench.step_bytes(wl, 2)
    b = bench.step_bytes(wl, 3)
    assert b["total"] - a["total"] == B * H * 386              # one more older record per tile
    assert a["state"] == B * H * 32768 == 2 ** 30              # 1 GiB of checkpoint reads
    # inputs read + appended + fp32 output row, per tile: 2 * 642 + 256
    one_older = B * H * 386
    assert a["total"] - a["state"] - one_older == B * H * (2 * 642 + 256)
    assert abs(B * H * 642 / MB - 21.0) < 0.05


def test_fold_step_writes_the_checkpoint_once():
    wl = _m2()
    B, H = wl.batch, wl.n_heads
    f = bench.step_bytes(wl, wl.L)
    assert f["state"] == 2 * B * H * 32768                     # read + write
    nf = bench.step_bytes(wl, wl.L - 1)
    # the fold step appends nothing: its record goes into the checkpoint
    assert f["total"] - f["state"] - (wl.L - 1) * B * H * 386 == B * H * (642 + 256)
    assert nf["total"] - nf["state"] - (wl.L - 2) * B * H * 386 == B * H * (2 * 642 + 256)


def test_window_average_per_token():
    wl = _m2()
    B = wl.batch
    tot = sum(bench.step_bytes(wl, h)["total"] for h in range(1, wl.L + 1)) / wl.L
    per_token = tot / B
    # per tile: 32768 (1 + 1/16) state + 7.5 x 386 older records + 642 inputs + 642 x 15/16
    # appends (none on the fold step) + 256 output = 39,210.875 B; x 128 heads
    assert per_token == 128 * (32768 * 17 / 16 + 7.5 * 386 + 642 + 642 * 15 / 16 + 256) == 5_018_992
    # staggered windows: every launch carries the window average
    hs = bench.window_phases(wl, 0, True)
    assert sorted(np.bincount(hs)[1:].tolist()) == [B // wl.L] * wl.L
    assert bench.launch_bytes(wl, hs)["total"] == pytest.approx(tot, rel=1e-12)


def test_conventional_bytes_per_token():
    wl = _m2()
    c = bench.conventional_bytes(wl)
    assert c["state"] == 2 * 2 ** 30
    assert c["total"] / wl.batch / MB == pytest.approx(8.50, abs=0.01)


@pytest.mark.parametrize("fmt,tile", [("fp8", 9216), ("mxfp4", 4352)])
def test_read_copy_tile_bytes(fmt, tile):
    wl = get_workload("m2_readcopy_b256").replace(read_copy=fmt)
    B, H = wl.batch, wl.n_heads
    nf = bench.step_bytes(wl, 1)
    assert nf["state"] == B * H * tile
    f = bench.step_bytes(wl, wl.L)
    assert f["state"] == B * H * (2 * 32768 + tile)            # fp32 read + write, copy written


def test_verify_bytes():
    wl = get_workload("m2_verify_b512")
    B, H, T = wl.batch, wl.n_heads, 4
    v = bench.verify_bytes(wl, np.zeros(B, np.int64), T)
    assert v["state"] == 2 * 2 ** 30                            # 2 GiB of checkpoint reads
    drafts = B * T * H * 642
    assert abs(drafts / MB - 168.3) < 0.1                       # drafts read, and again appended
    assert v["total"] == v["state"] + 2 * drafts + B * T * H * 4 * wl.dv
