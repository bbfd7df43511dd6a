"""Pins of the oracle's two-plane MXFP6 carriage of activations (the FP6X2
mode): OCP MX v1.0 E2M3 elements with an E8M0 scale per 32-element block
(shared exponent floor(log2 amax) - 2, round-to-nearest-even, magnitudes
beyond 7.5 clamped), plane 2 carrying the fp32 residual of plane 1.

Independent evaluations used here: the spec's landmark values, a bit-field
decode, an arithmetic rounding (Python's frexp for the binade and its
round-half-even) with an explicit bit-field encoder, closed forms worked by
hand, and the error bound that two planes imply."""

import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m3_landmarks_golden():
    with open(os.path.join(GOLDEN, "e2m3_landmarks.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 15
    for code_s, val_s in rows:
        got, want = oracle.e2m3_value(int(code_s, 16)), float(val_s)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), code_s


def _bitfield_value(c):
    s, e, m = c >> 5, (c >> 3) & 3, c & 7
    v = m * 2.0 ** -3 if e == 0 else 2.0 ** (e - 1) * (1 + m * 2.0 ** -3)
    return -v if s else v


def test_e2m3_every_code_matches_bitfield():
    for c in range(64):
        got, want = oracle.e2m3_value(c), _bitfield_value(c)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), c
    vals = [oracle.e2m3_value(c) for c in range(32)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def _encode(v):
    """E2M3 code of a grid value, from the bit fields."""
    s = 0x20 if math.copysign(1, v) < 0 else 0
    a = abs(v)
    if a < 1:
        return s | int(a * 8)
    e = math.frexp(a)[1] - 1  # a in [2^e, 2^(e+1))
    return s | ((e + 1) << 3) | int((a / 2.0 ** e - 1) * 8)


def mxfp6_reference(v):
    """MXFP6 of [N, K] fp32: frexp for the shared exponent, then each scaled
    element rounded half-to-even on its binade's step (2^(e-3) for |q| >= 1,
    1/8 below), clamped to 7.5, encoded from the bit fields."""
    v = np.asarray(v, np.float32).astype(np.float64)
    N, K = v.shape
    codes = np.zeros((N, K), np.uint8)
    scales = np.zeros((N, K // 32), np.uint8)
    for n in range(N):
        for b in range(K // 32):
            blk = v[n, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            s = min(max(math.frexp(amax)[1] - 1 - 2 + 127, 0), 254)
            scales[n, b] = s
            for i, x in enumerate(blk):
                q = float(np.float32(x / 2.0 ** (s - 127)))
                a = abs(q)
                if a >= 7.5:
                    r = 7.5
                else:
                    step = 0.125 if a < 1 else 2.0 ** (math.frexp(a)[1] - 1 - 3)
                    r = round(a / step) * step
                    r = min(r, 7.5)
                codes[n, 32 * b + i] = _encode(math.copysign(r, q))
    return codes, scales


def _blocks():
    rng = np.random.default_rng(5)
    rows = [rng.standard_normal(64) * np.exp2(rng.integers(-20, 20, 64))]
    for a in (1.0, 2.0 ** -30, 2.0 ** 40, 1.0 - 2.0 ** -24, 7.9):
        r = rng.uniform(-1, 1, 32) * a
        r[5] = a
        rows.append(r)
    # every tie of the grid at amax 4 (scale 2^0): q = (g_i + g_{i+1}) / 2
    grid = np.array([oracle.e2m3_value(c) for c in range(32)])
    mids = (grid[:-1] + grid[1:]) / 2
    r = np.zeros(32)
    r[:31] = mids * np.where(np.arange(31) % 2, -1, 1)
    r[31] = 4.0
    rows.append(r)
    for sgn in (-1, 1):  # either side of the ties
        r = np.zeros(32)
        r[:31] = np.nextafter(mids.astype(np.float32), np.float32(sgn * np.inf))
        r[31] = 4.0
        rows.append(r)
    # the 7.5 clamp: q in [7.5, 8)
    rows.append(np.linspace(7.5, 7.999, 32))
    rows.append(-np.linspace(7.6, 7.76, 32))
    rows.append(np.zeros(32))
    r = np.zeros(32); r[0] = 4.0; r[1] = -2.0 ** -10; r[2] = 2.0 ** -10
    rows.append(r)
    rows.append(np.full(32, 2.0 ** -149) * np.where(np.arange(32) % 3, 1, -1))
    rows.append(np.full(32, np.finfo(np.float32).max))
    return np.concatenate([np.asarray(r, np.float64).reshape(-1, 32) for r in rows]).astype(
        np.float32)


def test_mxfp6_quantize_matches_arithmetic_rounding():
    v = _blocks()
    for arr in (v, v[: (len(v) // 4) * 4].reshape(-1, 128)):
        codes, scales = oracle.mxfp6_quantize(arr)
        rc, rs = mxfp6_reference(arr)
        assert np.array_equal(scales, rs)
        assert np.array_equal(codes, rc), np.argwhere(codes != rc)[:5]


def test_mxfp6_hand_cases():
    # amax 4 -> scale code 127 + 2 - 2 = 127 (X = 1), q = v
    r = np.zeros((1, 32), np.float32)
    r[0, :7] = [4.0, 1.0625, 1.1875, 0.0625, 0.1875, 7.25, -3.0]
    # 1.0625: tie of 1.0 (0x08) and 1.125 (0x09) -> 0x08; 1.1875 -> 1.25 (0x0a);
    # 0.0625: tie of 0 and 0.125 -> 0; 0.1875: tie of 0.125 (0x01) and 0.25
    # (0x02) -> 0x02; 7.25: tie of 7.0 (0x1e) and 7.5 (0x1f) -> 0x1e; -3 -> 0x34
    c, s = oracle.mxfp6_quantize(r)
    assert s[0, 0] == 127
    assert list(c[0, :7]) == [0x18, 0x08, 0x0A, 0x00, 0x02, 0x1E, 0x34]
    # amax 7.9 -> scale code 127 (floor(log2 7.9) = 2); 7.9 clamps to 7.5
    r[0, 0] = 7.9
    c, s = oracle.mxfp6_quantize(r)
    assert s[0, 0] == 127 and c[0, 0] == 0x1F
    assert oracle.mxfp6_decode(c, s)[0, 0] == 7.5


def test_split_closed_form():
    # block [4, 1 + 2^-7, -(2 + 3 * 2^-6), 0, ...]: plane 1 at scale 2^0 holds
    # 4 (0x18), 1 (0x08) and -2 (0x30) (2 + 3 * 2^-6 = 2.046875 lies nearer 2
    # than 2.25); residuals 0, 2^-7, -3 * 2^-6 (amax 0.046875, floor(log2) =
    # -5, scale code 127 - 5 - 2 = 120, X = 2^-7): q = 0, 1 (0x08), -6 (0x3c)
    v = np.zeros((1, 32), np.float32)
    v[0, :3] = [4.0, 1 + 2.0 ** -7, -(2 + 3 * 2.0 ** -6)]
    c, s = oracle.fp6x2_split(v)
    assert s[0, 0, 0] == 127 and list(c[0, 0, :3]) == [0x18, 0x08, 0x30]
    assert s[1, 0, 0] == 120 and list(c[1, 0, :3]) == [0x00, 0x08, 0x3C]
    assert np.array_equal(oracle.fp6x2_value(c, s), v.astype(np.float64))
    # a block already on the plane-1 grid: plane 2 is the all-zero block
    g = np.array([oracle.e2m3_value(i) for i in range(32)], np.float32)[None] * 2.0 ** -3
    c, s = oracle.fp6x2_split(g)
    assert np.array_equal(oracle.mxfp6_decode(c[0], s[0]), g)
    assert not c[1].any() and not s[1].any()


def test_split_error_bound_and_planes():
    """With E = floor(log2 amax) of the block: plane 1 (scale X1 = 2^(E-2))
    leaves residuals below 2^(E-3) (half a top step, 0.25 X1, or up to 0.5 X1
    past the 7.5 clamp), so plane 2's scale is X2 <= 2^(E-6), and plane 2
    leaves at most half its top step or its clamp excess, 0.5 X2. Hence
    |v - carried| <= 0.5 X2 <= 2^(E-7) per element. Plane 2 is each block's
    MXFP6 conversion of the fp32 residual of plane 1."""
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal((64, 256)),
        rng.standard_normal((8, 256)) * np.exp2(rng.integers(-30, 30, (8, 256))),
        _blocks()[:16].reshape(-1, 256),
    ]).astype(np.float32)
    c, s = oracle.fp6x2_split(v)
    carried = oracle.fp6x2_value(c, s)
    v64 = v.astype(np.float64)
    amax = np.abs(v64).reshape(len(v), -1, 32).max(-1)
    E = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    X2 = np.repeat(np.exp2(s[1].astype(np.int64) - 127.0), 32, axis=1)
    bound = np.repeat(np.exp2(E - 7), 32, axis=1)
    # blocks whose plane scales stay above the bottom of the E8M0 range
    # (2^-127); below it, codes round to zero and only the X2 bound holds
    ok = np.repeat((amax > 0) & (E >= -120), 32, axis=1)
    assert ok.sum() > 18000
    assert (X2[ok] <= 2 * bound[ok]).all()
    assert (np.abs(carried - v64) <= 0.5 * X2).all()
    assert (np.abs(carried - v64)[ok] <= bound[ok]).all()
    # plane 2 is the conversion of the residual of plane 1
    r = (v - oracle.mxfp6_decode(c[0], s[0])).astype(np.float32)
    rc, rs = mxfp6_reference(r)
    assert np.array_equal(c[1], rc) and np.array_equal(s[1], rs)
    # plane 1 alone misses the bound: the second plane carries real precision
    one = oracle.mxfp6_decode(c[0], s[0]).astype(np.float64)
    assert (np.abs(one - v64) > bound).any()


def test_split_of_bf16_tokens_rms():
    """On N(0,1) bf16 tokens the carried value is within 1e-3 rms of the
    tokens (two 6-bit planes hold about 10 bits of a block's range)."""
    rng = np.random.default_rng(9)
    x = torch_bf16(rng.standard_normal((64, 3584)))
    c, s = oracle.fp6x2_split(x)
    err = oracle.fp6x2_value(c, s) - x
    assert np.sqrt((err ** 2).mean() / (x.astype(np.float64) ** 2).mean()) < 1e-3


def torch_bf16(a):
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()
