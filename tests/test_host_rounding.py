"""Host check of the rounding shortcut the 16-bit RoPE paths use (CPU only).

The rotated values are computed in fp64 and must reach bf16 with one rounding
to nearest, ties to even, as the oracle rounds them.  The kernels convert
fp64 -> fp32 -> bf16 (two nearest-even roundings) and redo, with the single
rounding, every group that holds an fp32 value whose low 16 bits are 0x8000
(a bf16 midpoint).  The claim: outside that case the two roundings give the
single rounding's result.  Checked here on random values and on values built
around midpoints, against the oracle's own rounding (oracle_round_sig).
"""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def lib():
    oracle.build.build()
    return oracle.load()


def _rn_bf16_bits(f32):
    """Nearest-even bf16 of finite fp32 values, as bit patterns (uint16)."""
    u = f32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return (u >> 16).astype(np.uint16)


def _single_bits(lib, xs):
    r = np.array([oracle.round_sig(x, 8, lib=lib) for x in xs], dtype=np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def test_double_rounding_differs_only_on_flagged_midpoints(lib):
    rng = np.random.default_rng(7)
    # random fp64 values over a wide range of magnitudes, both signs
    xs = rng.standard_normal(4000) * np.exp2(rng.integers(-20, 20, 4000))
    # values around bf16 midpoints: m +- a fraction of an fp32 ulp (flagged:
    # they round to m in fp32), and +- 1..3 fp32 ulps plus a fraction (not
    # flagged)
    mids = (rng.integers(0x3C00, 0x4400, 600).astype(np.uint32) << 16) | 0x8000
    m = mids.view(np.float32).astype(np.float64)
    ulp = np.spacing(m.astype(np.float32)).astype(np.float64)
    frac = rng.uniform(0.01, 0.49, 600)
    sign = rng.choice([-1.0, 1.0], 600)
    near = [m + sign * frac * ulp, m]
    for k in (1, 2, 3):
        near.append(m + sign * (k + frac) * ulp)
    xs = np.concatenate([xs, *near, -np.concatenate(near)])
    f32 = xs.astype(np.float32)  # fp64 -> fp32, nearest even
    flagged = (f32.view(np.uint32) & 0xFFFF) == 0x8000
    twice = _rn_bf16_bits(f32)
    once = _single_bits(lib, xs)
    assert flagged.sum() >= 1200  # the midpoint cases are exercised
    np.testing.assert_array_equal(twice[~flagged], once[~flagged])
    # the flag is needed: among the flagged values off the midpoint itself,
    # the double rounding is wrong for those on the odd side of the tie
    off = flagged & (f32.astype(np.float64) != xs)
    assert (twice[off] != once[off]).any()
