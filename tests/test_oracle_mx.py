"""Pins of the oracle's MXFP4 decode and encode against the format definition
(OCP MX v1.0 E2M1 elements with E8M0 scales per 32-element block) and against
the generator's independently written quantiser."""

import os

import numpy as np
import pytest
import torch

import oracle
from synth import quantize_mxfp4
from tests.dense_ref import e2m1_from_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def test_e2m1_table_matches_golden_and_bitfields():
    rows = _rows("e2m1_table.txt")
    assert len(rows) == 16
    for code_s, val_s in rows:
        code, val = int(code_s, 16), float(val_s)
        got = oracle.e2m1_value(code)
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)
        assert got == e2m1_from_bits(code)


def test_e8m0_every_finite_scale():
    for s in range(255):
        assert oracle.e8m0_value(s) == 2.0 ** (s - 127), s


def test_decode_every_code_and_scale():
    # one row per scale code; the 32 elements of its block hold codes 0..15 twice
    codes = np.tile(np.array([c | (c2 << 4) for c, c2 in zip(range(0, 16, 2), range(1, 16, 2))],
                             np.uint8), 2)
    codes = np.tile(codes, (255, 1))
    scales = np.arange(255, dtype=np.uint8).reshape(255, 1)
    dec = oracle.mxfp4_decode(codes, scales)
    want = e2m1_from_bits(np.tile(np.arange(16), 2))[None, :] * np.ldexp(1.0, np.arange(255) - 127)[:, None]
    # exact wherever the value fits fp32; only scale codes 253/254 (never
    # produced from finite fp32 input, whose largest scale code is 252) overflow
    fits = np.abs(want) <= np.finfo(np.float32).max
    assert np.array_equal(dec.astype(np.float64)[fits], want[fits])
    assert np.isinf(dec[~fits]).all() and (np.sign(dec[~fits]) == np.sign(want[~fits])).all()
    assert fits[:253].all()
    assert np.array_equal(np.signbit(dec[:, 8]), np.ones(255, bool))  # code 8 is -0


def _block_with(value, lead=4.0):
    blk = np.zeros((1, 32), np.float32)
    blk[0, 0] = lead
    blk[0, 5] = value
    return blk


@pytest.mark.parametrize("quant", ["oracle", "generator"])
def test_rne_golden_elements(quant):
    for val_s, code_s in _rows("mxfp4_rne_elements.txt"):
        v, want = np.float32(float(val_s)), int(code_s, 16)
        if val_s.startswith("-0.0"):
            v = np.float32(-0.0)
        blk = _block_with(v)
        if quant == "oracle":
            codes, scales = oracle.mxfp4_quantize(blk)
        else:
            c, s = quantize_mxfp4(torch.from_numpy(blk))
            codes, scales = c.numpy(), s.numpy()
        assert scales[0, 0] == 127
        got = (codes[0, 2] >> 4) & 15  # element 5 = high nibble of byte 2
        assert got == want, (quant, val_s, hex(got), hex(want))
        assert codes[0, 0] & 15 == 0x6  # the 4.0 lead element


@pytest.mark.parametrize("quant", ["oracle", "generator"])
def test_scale_exponent_golden(quant):
    for amax_s, want_s in _rows("mxfp4_scale_exponents.txt"):
        amax, want = np.float32(float(amax_s)), int(want_s)
        blk = np.zeros((1, 32), np.float32)
        blk[0, 7] = -amax
        if quant == "oracle":
            codes, scales = oracle.mxfp4_quantize(blk)
        else:
            c, s = quantize_mxfp4(torch.from_numpy(blk))
            codes, scales = c.numpy(), s.numpy()
        assert scales[0, 0] == want, (quant, amax_s, scales[0, 0], want)
        if amax == 0:
            assert not codes.any()


def test_all_zero_block_and_negative_zero_block():
    blk = np.zeros((2, 32), np.float32)
    blk[1] = -0.0
    codes, scales = oracle.mxfp4_quantize(blk)
    assert not codes.any() and not scales.any()
    c, s = quantize_mxfp4(torch.from_numpy(blk))
    assert not c.numpy().any() and not s.numpy().any()


def test_roundtrip_codes_survive_decode_then_encode():
    rng = np.random.default_rng(7)
    N = 300
    nib = rng.integers(0, 16, size=(N, 64))
    nib[:, 0] = rng.choice([6, 7, 14, 15], size=N)  # a +-4 or +-6 fixes the scale
    nib[:, 32] = rng.choice([6, 7, 14, 15], size=N)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(20, 235, size=(N, 2)).astype(np.uint8)
    dec = oracle.mxfp4_decode(codes, scales)
    c2, s2 = oracle.mxfp4_quantize(dec)
    assert np.array_equal(s2, scales)
    assert np.array_equal(c2, codes)


def test_generator_quantiser_matches_oracle_bytes():
    rng = np.random.default_rng(3)
    # wide dynamic range: per-row scale factors from 2^-60 to 2^60 plus
    # exact grid points, midpoints and zeros sprinkled in
    w = rng.standard_normal((257, 512)).astype(np.float32)
    w *= np.ldexp(1.0, rng.integers(-60, 60, size=(257, 1))).astype(np.float32)
    grid = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6], np.float32)
    w[::7, ::3] = rng.choice(grid, size=w[::7, ::3].shape) * rng.choice([-1, 1], size=w[::7, ::3].shape)
    w[5, 64:96] = 0.0
    c_o, s_o = oracle.mxfp4_quantize(w)
    c_g, s_g = quantize_mxfp4(torch.from_numpy(w))
    assert np.array_equal(s_o, s_g.numpy())
    assert np.array_equal(c_o, c_g.numpy())


def test_quantised_values_within_half_ulp_of_grid():
    # |decode(encode(v)) - v| <= half the E2M1 spacing at v's magnitude, times
    # the scale, except where v saturates (|v|/scale > 6).
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    codes, scales = oracle.mxfp4_quantize(w)
    dec = oracle.mxfp4_decode(codes, scales).astype(np.float64)
    sc = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    q = np.abs(w.astype(np.float64)) / sc
    spacing = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    err = np.abs(dec - w) / sc
    ok = (err <= spacing / 2 + 1e-12) | (q > 6)
    assert ok.all()
