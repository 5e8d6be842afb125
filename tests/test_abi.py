"""Host-side checks of the C ABI: the library loads, exports every declared symbol,
sizes buffers as documented and rejects bad arguments before enqueuing anything.
No call here reaches a kernel launch."""
import ctypes

import pytest

from attention_decode_mamba_amd import rssm as R
from attention_decode_mamba_amd.state import make_config


def _cfg(**kw):
    base = dict(kind="mamba2", batch=256, n_heads=128, n_qk_heads=128, dv=64, dk=128, L=16, t_max=1,
                capacity=16, in_dtype="bf16", read_copy="none")
    base.update(kw)
    return make_config(**base)


def test_exports_every_header_symbol():
    lib = R.lib()
    names = R.header_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
        assert n in R._SIGS, n


def test_version_and_strerror():
    assert R.rssm_version() >= 100
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert isinstance(R.rssm_strerror(code), str) and R.rssm_strerror(code)
    assert "ring" in R.rssm_strerror(R.RSSM_DEVERR_VERIFY_CAPACITY)
    # every device error bit has its own message, alone and as the only bit of a word
    bits = {R.RSSM_DEVERR_VERIFY_CAPACITY: "ring", R.RSSM_DEVERR_ACCEPT_RANGE: "accepted",
            R.RSSM_DEVERR_CURSOR: "cursor", R.RSSM_DEVERR_TREE: "tree"}
    msgs = set()
    for bit, word in bits.items():
        m = R.rssm_strerror(bit)
        assert m.startswith("device:") and word in m, (bit, m)
        msgs.add(m)
    assert len(msgs) == len(bits)
    assert R.rssm_strerror(16) == "unknown error"              # no such bit
    assert R.rssm_strerror(R.RSSM_DEVERR_TREE | 16).startswith("device:")


def test_sizes_serving_shape():
    sz = R.rssm_sizes(_cfg())
    assert sz.s_ckpt == 256 * 128 * 64 * 128 * 4          # 4 MiB per sequence
    assert sz.s_read == 0 and sz.s_read_scale == 0
    assert sz.n_committed == sz.n_ckpt == 256 * 128 * 8
    off = R.rssm_ring_offsets(_cfg())
    es, C = 2, 16
    assert off[0] == 0
    assert off[1] == off[2]                                # no beta region for Mamba-2
    assert off[3] - off[2] >= 256 * 128 * C * 64 * es
    assert sz.ring >= off[4] + 256 * 128 * C * 128 * es
    assert all(o % 256 == 0 for o in off)


def test_sizes_read_copy_and_gdn():
    fp8 = R.rssm_sizes(_cfg(read_copy="fp8"))
    mx = R.rssm_sizes(_cfg(read_copy="mxfp4"))
    tiles, PN = 256 * 128, 64 * 128
    assert fp8.s_read == tiles * PN and fp8.s_read_scale == tiles * PN // 32 * 4
    assert mx.s_read == tiles * PN // 2 and mx.s_read_scale == tiles * PN // 32
    g = _cfg(kind="gdn", n_heads=32, n_qk_heads=16, dv=128, t_max=4, capacity=19)
    off = R.rssm_ring_offsets(g)
    assert off[2] - off[1] >= 256 * 32 * 19 * 2           # beta region present


@pytest.mark.parametrize("kw,code", [
    (dict(kind="mamba2", n_heads=6, n_qk_heads=4), R.RSSM_E_SHAPE),
    (dict(dk=96), R.RSSM_E_SHAPE),
    (dict(dv=200), R.RSSM_E_SHAPE),                      # 200 > 16384 / 128
    (dict(capacity=15), R.RSSM_E_SHAPE),                 # C < L + t_max - 1
    (dict(capacity=40, L=16), R.RSSM_E_SHAPE),           # C > 32
    (dict(t_max=9, capacity=32), R.RSSM_E_RANGE),
    (dict(L=0), R.RSSM_E_RANGE),
    (dict(batch=-1), R.RSSM_E_SHAPE),
])
def test_check_config_rejects(kw, code):
    with pytest.raises(R.RssmError) as e:
        R.rssm_check_config(_cfg(**kw))
    assert e.value.code == code


def test_check_config_bad_enums():
    c = _cfg()
    c.kind = 7
    assert R.lib().rssm_check_config(ctypes.byref(c)) == R.RSSM_E_DTYPE
    c = _cfg()
    c.read_copy = 3
    assert R.lib().rssm_check_config(ctypes.byref(c)) == R.RSSM_E_DTYPE


@pytest.mark.parametrize("dv,dk", [(1, 32), (512, 32), (256, 64), (128, 128), (64, 256), (17, 128)])
def test_check_config_accepts_supported_shapes(dv, dk):
    assert R.rssm_check_config(_cfg(dv=dv, dk=dk, n_heads=4, n_qk_heads=2, batch=3)) == 0


def test_null_and_range_rejected_without_launch():
    c = _cfg(batch=2, n_heads=2, n_qk_heads=2, t_max=4, capacity=19)
    st = R.rssm_state()
    with pytest.raises(R.RssmError) as e:
        R.rssm_decode_step(c, st, 16, None, 16, 16, 16, 16)
    assert e.value.code == R.RSSM_E_NULL
    fake = R.rssm_state(256, None, None, 256, 256, 256, 256)      # aligned, never dereferenced
    with pytest.raises(R.RssmError) as e:
        R.rssm_verify(c, fake, 5, 16, None, 16, 16, 16, 16)         # T > t_max
    assert e.value.code == R.RSSM_E_RANGE
    with pytest.raises(R.RssmError) as e:
        R.rssm_flush(c, fake, -1)
    assert e.value.code == R.RSSM_E_RANGE
    with pytest.raises(R.RssmError) as e:
        R.rssm_commit(c, fake, 16, 0)
    assert e.value.code == R.RSSM_E_RANGE
    with pytest.raises(R.RssmError) as e:
        R.rssm_decode_step(c, fake, 16, None, 17, 16, 16, 16)       # misaligned v (bf16 needs 2 B)
    assert e.value.code == R.RSSM_E_ALIGN
    g = _cfg(kind="gdn", batch=2, n_heads=2, n_qk_heads=1, t_max=4, capacity=19)
    with pytest.raises(R.RssmError) as e:
        R.rssm_decode_step(g, fake, 16, None, 16, 16, 16, 16)       # GDN needs beta
    assert e.value.code == R.RSSM_E_NULL
    with pytest.raises(R.RssmError) as e:
        R.rssm_stream_copy(16, 32, 100)
    assert e.value.code == R.RSSM_E_ALIGN


def test_empty_batch_enqueues_nothing():
    c = _cfg(batch=0)
    fake = R.rssm_state(256, None, None, 256, 256, 256, 256)
    assert R.rssm_decode_step(c, fake, 16, None, 16, 16, 16, 16) == 0
    assert R.rssm_flush(c, fake, 16) == 0
    assert R.rssm_commit(c, fake, 16, 1) == 0
