"""Pins of the oracle's block-scaled precision mode (MX8): MXFP8 activations
(OCP MX v1.0 E4M3 elements, E8M0 scale per 32-element block, shared exponent
floor(log2 amax) - 8, round-to-nearest-even, magnitudes beyond 448 clamped)
with MXFP4 weights.

Independent evaluations used here: torch's float8_e4m3fn type (its decode and
its round-to-nearest-even conversion from fp32), Python's frexp for the
shared exponent, a dense fp64 evaluation of every expert, and closed forms of
all-ones weights that land on an E4M3 tie and on the 448 clamp."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import LayerConfig, make_inputs
from tests.dense_ref import decode_bitfield, dense_gate_matrix, max_abs_over_rms, rel_l2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_value(code):
    return float(torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float())


def test_e4m3_landmarks_golden():
    with open(os.path.join(GOLDEN, "e4m3_landmarks.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 16
    for code_s, val_s in rows:
        got = oracle.e4m3_value(int(code_s, 16))
        if val_s == "nan":
            assert math.isnan(got), code_s
        else:
            want = float(val_s)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code_s


def test_e4m3_every_code_matches_torch_float8():
    for c in range(256):
        got, want = oracle.e4m3_value(c), _torch_e4m3_value(c)
        if math.isnan(want):
            assert math.isnan(got), c
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), c
    # 0x00..0x7e strictly increasing: 127 distinct finite non-negative values
    vals = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def mxfp8_reference(v):
    """MXFP8 of [N, K] fp32 with frexp for the shared exponent and torch's
    fp32 -> float8_e4m3fn conversion (round-to-nearest-even) for the elements,
    after clamping to +-448."""
    v = np.asarray(v, np.float32)
    N, K = v.shape
    blocks = v.astype(np.float64).reshape(N, K // 32, 32)
    amax = np.abs(blocks).max(-1)
    s = np.zeros((N, K // 32), np.int64)
    for n in range(N):
        for b in range(K // 32):
            if amax[n, b] != 0:
                s[n, b] = min(max(math.frexp(amax[n, b])[1] - 1 - 8 + 127, 0), 254)
    q = blocks / np.ldexp(1.0, s - 127)[..., None]
    q32 = torch.from_numpy(np.clip(q, -448.0, 448.0).astype(np.float32))
    codes = q32.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    codes[amax == 0] = 0
    return codes.reshape(N, K), s.astype(np.uint8)


def mxfp8_decode_reference(codes, scales):
    vals = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
    return vals * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)


def _blocks():
    rng = np.random.default_rng(11)
    rows = []
    # random magnitudes over many binades, mixed signs
    rows.append(rng.standard_normal(64) * np.exp2(rng.integers(-20, 20, 64)))
    # amax exactly a power of two, and just below one
    for a in (1.0, 2.0 ** -30, 2.0 ** 40, 1.0 - 2.0 ** -24, 2.0 ** 10 * (1 - 2.0 ** -24)):
        r = rng.uniform(-1, 1, 32) * a
        r[5] = a
        rows.append(r)
    # every tie of the E4M3 grid at amax = 1 (scale 2^-8): q = (g_i + g_{i+1}) / 2
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = (grid[:-1] + grid[1:]) / 2
    for chunk in range(0, len(mids), 31):
        r = np.zeros(32)
        m = mids[chunk:chunk + 31] / 256.0
        r[:len(m)] = m * np.where(np.arange(len(m)) % 2, -1, 1)
        r[31] = 1.0  # amax 1 -> scale 2^-8
        rows.append(r)
    # values just either side of the ties
    for sgn in (-1, 1):
        r = np.zeros(32)
        m = mids[40:71] / 256.0
        r[:31] = np.nextafter(m.astype(np.float32), np.float32(sgn * np.inf)).astype(np.float64)
        r[31] = 1.0
        rows.append(r)
    # the 448 clamp: amax in [448, 512) x 2^-8 of a power of two
    rows.append(np.linspace(1.5, 1.999, 32))
    rows.append(-np.linspace(1.74, 1.76, 32))
    # zeros, negative zeros, a negative value rounding to zero, fp32 subnormals
    rows.append(np.zeros(32))
    rows.append(-np.zeros(32))
    r = np.zeros(32); r[0] = 1.0; r[1] = -2.0 ** -20; r[2] = 2.0 ** -20
    rows.append(r)
    rows.append(np.full(32, 2.0 ** -149) * np.where(np.arange(32) % 3, 1, -1))
    rows.append(np.full(32, np.finfo(np.float32).max))
    out = []
    for r in rows:
        r = np.asarray(r, np.float64)
        if r.size % 32:
            r = np.concatenate([r, np.zeros(32 - r.size % 32)])
        out.append(r.reshape(-1, 32))
    return np.concatenate(out).astype(np.float32)


def test_mxfp8_quantize_matches_torch_conversion():
    v = _blocks()
    # one block per row, and the same data as rows of 4 blocks
    for arr in (v, v[: (len(v) // 4) * 4].reshape(-1, 128)):
        codes, scales = oracle.mxfp8_quantize(arr)
        rc, rs = mxfp8_reference(arr)
        assert np.array_equal(scales, rs)
        assert np.array_equal(codes, rc), np.argwhere(codes != rc)[:5]


def test_mxfp8_hand_cases():
    # amax 1 -> scale code 127 - 8 = 119; 1.0 -> q = 256 (0x78)
    r = np.zeros((1, 32), np.float32)
    r[0, 0] = 1.0
    r[0, 1] = 1.0625   # q = 272, tie between 256 (0x78) and 288 (0x79) -> even 0x78
    r[0, 2] = 1.1875   # q = 304, tie between 288 (0x79) and 320 (0x7a) -> even 0x7a
    r[0, 3] = -1.0
    c, s = oracle.mxfp8_quantize(r)
    assert s[0, 0] == 119 and list(c[0, :4]) == [0x78, 0x78, 0x7A, 0xF8]
    # amax 1.9 -> scale 2^-8, q = 486.4 clamps to 448 (0x7e)
    r[0, 0] = 1.9
    c, s = oracle.mxfp8_quantize(r)
    assert s[0, 0] == 119 and c[0, 0] == 0x7E
    dec = oracle.mxfp8_decode(c, s)
    assert dec[0, 0] == 1.75


def test_mxfp8_decode_matches_reference():
    v = _blocks()
    c, s = oracle.mxfp8_quantize(v)
    got = oracle.mxfp8_decode(c, s).astype(np.float64)
    want = mxfp8_decode_reference(c, s)
    fits = np.abs(want) <= np.finfo(np.float32).max
    assert np.array_equal(got[fits], want[fits])
    # quantisation error per element, with X the block's scale: at most half
    # an E4M3 step -- 2^-4 of the value among normals, 2^-10 X among
    # subnormals -- and up to (amax - 448 X) at the clamp
    v64 = v.astype(np.float64)
    X = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    err = np.abs(got - v64)
    clamped = np.abs(v64) >= 448 * X
    bound = np.where(clamped, np.abs(v64) - 448 * X,
                     np.maximum(np.abs(v64) * 2.0 ** -4, X * 2.0 ** -10))
    assert (err <= bound).all()


def dense_masked_layer_mx8(x, idx, w, wts, *, E, e0=0, n_local=None, act=1):
    """The MX8 layer evaluated densely: tokens quantised by mxfp8_reference,
    every expert on every token in fp64, g and u rounded to fp32, h = act in
    fp32 (as the oracle states it), h quantised by mxfp8_reference, y in fp64,
    weighted by the dense gate matrix."""
    x = np.asarray(x, np.float32)
    n_local = E if n_local is None else n_local
    G = dense_gate_matrix(idx, w, E)
    xq = mxfp8_decode_reference(*mxfp8_reference(x))
    out = np.zeros(x.shape, np.float64)
    for le in range(n_local):
        wg = decode_bitfield(wts["gate_codes"][le], wts["gate_scales"][le])
        wu = decode_bitfield(wts["up_codes"][le], wts["up_scales"][le])
        wd = decode_bitfield(wts["down_codes"][le], wts["down_scales"][le])
        g = (xq @ wg.T).astype(np.float32)
        u = (xq @ wu.T).astype(np.float32)
        if act == oracle.ACT_NONE:
            h = g
        else:
            silu = g / (np.float32(1) + np.exp(-g))
            h = (silu * u).astype(np.float32)
        hq = mxfp8_decode_reference(*mxfp8_reference(h))
        y = (hq @ wd.T).astype(np.float32).astype(np.float64)
        out += G[:, e0 + le:e0 + le + 1] * y
    return out


SMALL = [
    LayerConfig("m0", T=7, I=32, d=64, E=8, k=2),
    LayerConfig("m1", T=13, I=64, d=96, E=16, k=4, bias="normal"),
    LayerConfig("m2", T=9, I=32, d=64, E=12, k=3, expert_begin=4, num_local=5),
]


def _np_weights(inp):
    return {k: v.numpy() for k, v in inp.weights.items()}


def _run(inp, act, mx8=True):
    c = inp.cfg
    return oracle.layer(inp.x, inp.w_router.numpy(),
                        None if inp.bias is None else inp.bias.numpy(), _np_weights(inp),
                        E=c.E, k=c.k, I=c.I, e0=c.expert_begin, n_local=c.num_local, act=act,
                        mx8=mx8)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_SILU_MUL])
def test_mx8_layer_vs_dense(cfg, act):
    inp = make_inputs(cfg)
    r = _run(inp, act)
    ref = dense_masked_layer_mx8(inp.x.float().numpy(), r["idx"], r["w"], _np_weights(inp),
                                 E=cfg.E, e0=cfg.expert_begin, n_local=cfg.num_local, act=act)
    # act NONE: the same fp32 g, so the same h codes; SiLU: exp may differ by
    # an ulp, which can move an h element across an E4M3 tie
    tol = 1e-6 if act == oracle.ACT_NONE else 1e-4
    assert rel_l2(r["out"], ref) <= tol
    # routing is the bf16 path's
    r0 = _run(inp, act, mx8=False)
    assert np.array_equal(r0["idx"], r["idx"]) and np.array_equal(r0["w"], r["w"])
    # and the quantisation is really there: an E4M3 step is 2^-3 of the value
    assert 1e-3 < rel_l2(r["out"], r0["out"]) < 0.2


@pytest.mark.parametrize("d,xval,h,hq", [
    (96, 1.0, 96.0 ** 2, 96.0 ** 2),         # 9216 = 288 x 2^5: on the grid
    (160, 1.0, 160.0 ** 2, 24576.0),        # 25600 = 400 x 2^6: tie of 384 and 416 -> 384
    (32, 1.375, 44.0 ** 2, 1792.0),         # 1936 = 484 x 2^2: clamped to 448
])
def test_mx8_all_ones_weights_closed_form(d, xval, h, hq):
    """x constant, every weight 1.0: g = u = d x, h = silu(g) u = g^2 (silu(g)
    = g in fp32 for g >= 32), a constant block that MXFP8 maps to hq, and
    y = I hq in every column."""
    cfg = LayerConfig("ones", T=4, I=64, d=d, E=4, k=2)
    inp = make_inputs(cfg)
    inp.x = torch.full((cfg.T, d), xval, dtype=torch.bfloat16)
    for name, t in inp.weights.items():
        t.fill_(127 if name.endswith("scales") else 0x22)
    r = _run(inp, oracle.ACT_SILU_MUL)
    assert (d * xval) ** 2 == h
    want = cfg.I * hq * r["w"].astype(np.float64).sum(1)
    assert np.allclose(r["out"].astype(np.float64), want[:, None], rtol=1e-6, atol=0)


def test_mx8_token_rows_equal_layer_rows_bitwise():
    cfg = SMALL[2]
    inp = make_inputs(cfg)
    r = _run(inp, oracle.ACT_SILU_MUL)
    toks = [0, 3, 8, 5]
    rows = oracle.token_rows(inp.x, r["idx"], r["w"], toks, _np_weights(inp), I=cfg.I,
                             e0=cfg.expert_begin, n_local=cfg.num_local, mx8=True)
    assert np.array_equal(rows, r["out"][toks])
