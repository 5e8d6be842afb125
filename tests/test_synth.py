"""The seeded generator: subsets regenerate identically, dtypes and ranges as stated."""
import numpy as np

from synth import (get_workload, decode_inputs, draft_inputs, initial_state, accept_counts,
                   stack_decode_inputs, bf16_bits_from_f32)


def test_subset_regenerates_identically():
    wl = get_workload("gdn_b256")
    full = decode_inputs(wl.replace(batch=6), 3, range(6))
    part = decode_inputs(wl, 3, [4, 1])
    for k in ("alpha", "beta", "v", "k", "q"):
        np.testing.assert_array_equal(part[k][0], full[k][4])
        np.testing.assert_array_equal(part[k][1], full[k][1])
    np.testing.assert_array_equal(initial_state(wl, [5])[0], initial_state(wl, range(6))[5])


def test_pool_matches_serial():
    wl = get_workload("m2_tiny")
    a = stack_decode_inputs(wl, range(5), [0, 1], workers=1)
    b = stack_decode_inputs(wl, range(5), [0, 1], workers=2)
    for k in a:
        if a[k] is not None:
            np.testing.assert_array_equal(a[k], b[k])


def test_ranges():
    wl = get_workload("m2_decode_b256")
    d = decode_inputs(wl, 0, [0])
    assert d["alpha"].dtype == np.uint16 and d["beta"] is None
    a = (d["alpha"].astype(np.uint32) << 16).view(np.float32)
    assert np.all((a > 0) & (a <= 1))
    g = get_workload("gdn_b256")
    d = draft_inputs(g, 0, [0], 4)
    k = (d["k"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-2)
    acc = accept_counts(g, 0, 4)
    assert acc.shape == (256,) and acc.min() >= 0 and acc.max() <= 4


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    bits = bf16_bits_from_f32(x)
    assert bits.tolist() == [0x3F80, 0x3F82, 0x3F81]
