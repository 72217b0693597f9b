"""Pins for the OCP Microscaling (MX) formats the oracle decodes and datagen
encodes: E2M1 elements, E8M0 block scales, MXFP8 / MXFP4 blocks of 32.

The format values come from the OCP MX definition (not from the pages, which
are silent on block scaling): E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
E8M0 byte b means 2^(b - 127) and 0xFF is NaN.  A problem whose decoded
values equal a bf16 problem's must select exactly what that problem selects,
which ties the MX path to the separately pinned bf16 path.
"""
import numpy as np
import pytest

import datagen
import oracle


def test_e2m1_values_from_the_format():
    got = oracle.decode_e2m1(np.arange(16))
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert np.array_equal(got[:8], want)
    assert np.array_equal(got[8:], -np.array(want, dtype=np.float64))
    assert np.signbit(got[8])  # code 8 is -0
    # every code survives encode(decode(code))
    assert np.array_equal(datagen.f32_to_e2m1(got), np.arange(16, dtype=np.uint8))


def test_e2m1_rounds_to_nearest_even_and_saturates():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.3, 0.26])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, -0.5, 0.5])
    assert np.array_equal(oracle.decode_e2m1(datagen.f32_to_e2m1(x)), want)


def test_e8m0_values_from_the_format():
    v = oracle.decode_e8m0(np.array([127, 0, 254, 128, 126, 255]))
    assert v[0] == 1.0 and v[1] == 2.0 ** -127 and v[2] == 2.0 ** 127
    assert v[3] == 2.0 and v[4] == 0.5 and np.isnan(v[5])


@pytest.mark.parametrize("fmt,emax,maxnorm,rel,sub", [
    ("mxfp8", 8, 448.0, 2.0 ** -4, 2.0 ** -10), ("mxfp4", 2, 6.0, 2.0 ** -2, 0.25)])
def test_mx_block_quantisation(fmt, emax, maxnorm, rel, sub):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((300, 128)) * np.exp2(rng.integers(-20, 20, size=(300, 1)))).astype(np.float32)
    x[7] = 0.0
    codes, scales = datagen.quantize_mx(x, fmt)
    assert scales.shape == (300, 4)
    assert codes.shape == ((300, 128) if fmt == "mxfp8" else (300, 64))
    blocks = x.reshape(300, 4, 32).astype(np.float64)
    amax = np.abs(blocks).max(axis=2)
    nz = amax > 0
    want = np.floor(np.log2(amax[nz])) - emax + 127
    assert np.array_equal(scales[nz].astype(np.float64), want)
    dec = oracle.decode_mx(codes, scales, fmt)
    X = np.repeat(oracle.decode_e8m0(scales), 32, axis=1)
    xd = x.astype(np.float64)
    assert np.all(np.abs(dec / X) <= maxnorm)
    # elements past the format's largest value saturate to it (the block scale
    # comes from floor(log2(amax)), so a block maximum can reach 2^(emax+1) X);
    # the rest obey the round-to-nearest bound of the element format
    sat = np.abs(xd) > maxnorm * X
    assert np.array_equal(dec[sat], np.sign(xd[sat]) * maxnorm * X[sat])
    ok = ~sat
    assert np.all(np.abs(dec[ok] - xd[ok]) <= rel * np.abs(xd[ok]) + sub * X[ok] + 1e-300)
    assert np.all(dec[7] == 0.0)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_integer_values_quantise_exactly_and_select_like_bf16(fmt):
    mx = datagen.make_custom("mxint", 900, 40, 8, 128, 64, dtype=fmt, dist="int", seed=81)
    bf = datagen.make_custom("bfint", 900, 40, 8, 128, 64, dtype="bf16", dist="int", seed=81)
    dm, db = oracle.Decoded(mx), oracle.Decoded(bf)
    assert np.array_equal(dm.keys, db.keys)
    assert np.array_equal(dm.query(3)[0], db.query(3)[0])
    a, b = oracle.select(mx), oracle.select(bf)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
