"""GPU parity of the FP6X2 carriage (activations as two MXFP6 planes, MXFP4
weights, v_mfma_scale_f32_32x32x64_f8f6f4 at the 6-bit x 4-bit rate).

Stage by stage: the split byte for byte against the oracle's; the grouped
projection elementwise against the exact sum of the planes' values times the
exactly decoded weights; the layer against the oracle's default (bf16
activation) layer on the GPU's routing, within the default contract. The
projection's bound: the products are exact, a one-wave probe of the 6-bit x
4-bit instruction found its 64-long sums exact to fp32 rounding, and the fp32
accumulation of two partial sums per 64-long step adds at most
2 (K/64) 2^-24 of sum|products|; the tests allow 1e-5 sum|a w|."""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, LayerConfig, make_inputs, quantize_mxfp4
from tests.parity_util import (assert_close_layer, block_int16_step, host_weights, np_,
                               oracle_rows, rel_l2, run_gpu_layer, sample_tokens)
from tests.test_oracle_fp6x2 import _blocks

pytestmark = pytest.mark.gpu
DEV = "cuda"
MMA_TOL = 1e-5


@pytest.fixture(scope="module")
def m():
    import mxfp4_expert_top_amd as mod
    return mod


def unpack_split(rec):
    """[N, 2 K] bytes as written by moe_fp6x2_split -> codes [2, N, K] and
    scales [2, N, K/32]. Per 128-byte record s: blocks 2s and 2s+1 at bytes
    0 and 64 (plane 1, then plane 2, 24 bytes each, code i at bits
    6i..6i+5, little-endian), the four scale codes at bytes 48..51 ((2s, 1),
    (2s, 2), (2s+1, 1), (2s+1, 2)) and again at 52..55, 56..59, 60..63,
    zeros at 112..127."""
    N, K2 = rec.shape
    r = rec.reshape(N, K2 // 128, 128)
    assert not r[:, :, 112:].any()
    for c in (52, 56, 60):
        assert np.array_equal(r[:, :, c:c + 4], r[:, :, 48:52])
    blocks = np.stack([r[:, :, 0:48], r[:, :, 64:112]], axis=2).reshape(N, -1, 2, 2, 24)
    bits = np.unpackbits(blocks, axis=-1, bitorder="little").reshape(N, -1, 2, 2, 32, 6)
    codes = (bits * (1 << np.arange(6))).sum(-1).astype(np.uint8)  # [N, s, block, plane, 32]
    codes = codes.transpose(3, 0, 1, 2, 4).reshape(2, N, -1)
    sc = r[:, :, 48:52].reshape(N, -1, 2, 2).transpose(3, 0, 1, 2).reshape(2, N, -1)
    return codes, np.ascontiguousarray(sc)


def _check_split(m, v_dev, v_host):
    rec = m.moe_fp6x2_split(v_dev)
    torch.cuda.synchronize()
    rc, rs = oracle.fp6x2_split(v_host)
    codes, scales = unpack_split(np_(rec))
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc), np.argwhere(codes != rc)[:5]


# ---------------------------------------------------------------- the split
@pytest.mark.parametrize("K", [64, 128, 3584])
def test_fp6x2_split_fp32_bitexact(m, K):
    """Ties of the E2M3 grid and either side of them, the 7.5 clamp, zero
    blocks, a negative value rounding to zero, fp32 subnormals and the fp32
    maximum; random rows of three magnitudes."""
    v = _blocks().reshape(-1)
    v = np.resize(v, ((v.size + K - 1) // K) * K).reshape(-1, K).astype(np.float32)
    rnd = np.random.default_rng(K).standard_normal((7, K)).astype(np.float32)
    v = np.ascontiguousarray(np.concatenate([v, rnd * 3.0, rnd * 1e-30, rnd * 1e30]))
    _check_split(m, torch.from_numpy(v).to(DEV), v)


def test_fp6x2_split_bf16_rows_with_stride(m):
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((33, 3584 + 64)).astype(np.float32)).to(torch.bfloat16)
    x[3, :64] = 0
    x[4] *= 1e-20
    x[5, :32] = torch.tensor(np.float32(2.0) ** -133)  # bf16 subnormals
    _check_split(m, x.to(DEV)[:, :3584], x[:, :3584].float().numpy())


def test_fp6x2_split_grid_stride(m):
    """More blocks (140000 x 32) than the launch's threads (16384 x 256): rows
    on both sides of the first pass's end, against the oracle."""
    N, K = 140000, 1024
    g = torch.Generator(device=DEV).manual_seed(7)
    v = (torch.randn(N, K, generator=g, device=DEV) * 2.0).to(torch.bfloat16)
    rec = m.moe_fp6x2_split(v)
    torch.cuda.synchronize()
    wrap = 16384 * 256 // (K // 32)
    rows = np.r_[0:4, wrap - 4:wrap + 4, N - 4:N]
    rc, rs = oracle.fp6x2_split(v[torch.from_numpy(rows).to(DEV)].float().cpu().numpy())
    codes, scales = unpack_split(np_(rec)[rows])
    assert np.array_equal(scales, rs) and np.array_equal(codes, rc)


# ---------------------------------------------------------------- projection
def _experts(num_local, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    cs = [quantize_mxfp4(torch.randn(N, K, generator=g) / np.sqrt(K)) for _ in range(num_local)]
    return torch.stack([c for c, _ in cs]), torch.stack([s for _, s in cs])


def _bound(a, w):
    return np.abs(a) @ np.abs(w).T


def _split_rows(m, rng, R, K):
    """Random bf16 rows of mixed magnitudes, split on the GPU; the value the
    oracle's split of the same rows carries (fp64)."""
    v = (rng.standard_normal((R, K)) * np.exp2(rng.integers(-3, 4, (R, 1)))).astype(np.float32)
    vb = torch.from_numpy(v).to(torch.bfloat16)
    rec = m.moe_fp6x2_split(vb.to(DEV))
    rc, rs = oracle.fp6x2_split(vb.float().numpy())
    return rec, oracle.fp6x2_value(rc, rs), vb.float().numpy().astype(np.float64)


@pytest.mark.parametrize("act", [0, 1, 2])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("K", [128, 640, 3584, 4096])
def test_grouped_gemm_fp6x2_vs_definition(m, act, packed, K):
    """Experts with 37, 0, 513, 1, 257 and 150 rows (empty, one row, ragged,
    several 256-row groups), a column count that is not a tile multiple,
    gathered rows, fp32 output; rows past the last expert's end untouched."""
    rng = np.random.default_rng(K + 3 * act + 7 * packed)
    nl, N, T = 6, 320, 700
    counts = np.array([37, 0, 513, 1, 257, 150], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    xd, xval, xb = _split_rows(m, rng, T, K)
    a_rows = rng.integers(0, T, size=A).astype(np.int32)
    w1c, w1s = _experts(nl, N, K, 3)
    w2c, w2s = _experts(nl, N, K, 4) if act else (None, None)
    dev = lambda t: None if t is None else t.to(DEV)
    pk = lambda c, s: m.moe_mxfp4_prepack(dev(c), dev(s)) if packed else (dev(c), dev(s))
    g1c, g1s = pk(w1c, w1s)
    g2c, g2s = pk(w2c, w2s) if act else (None, None)
    out = torch.full((A + 3, N), 7.0, dtype=torch.float32, device=DEV)
    ws = m.alloc_workspace(m.moe_grouped_gemm_fp6x2_workspace_size(nl, A), DEV)
    m.moe_grouped_gemm_fp6x2(xd, torch.from_numpy(a_rows).to(DEV), g1c, g1s, g2c, g2s,
                             torch.from_numpy(off).to(DEV), A, act, out, ws,
                             w_layout=m.LAYOUT_PACKED if packed else m.LAYOUT_OCP)
    torch.cuda.synchronize()
    got = np_(out).astype(np.float64)
    assert (got[A:] == 7.0).all()
    xa, xba = xval[a_rows], xb[a_rows]
    for e in range(nl):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            continue
        w1 = oracle.mxfp4_decode(w1c[e].numpy(), w1s[e].numpy()).astype(np.float64)
        g = xa[r0:r1] @ w1.T
        bg = MMA_TOL * _bound(xa[r0:r1], w1)
        if act == 0:
            assert (np.abs(got[r0:r1] - g) <= bg).all(), np.abs(got[r0:r1] - g).max()
            # and the exact bf16 rows' product within what the planes leave
            # out (at most 2^(E-7) per element)
            gb = xba[r0:r1] @ w1.T
            assert rel_l2(got[r0:r1], gb) < 2e-3
        else:
            w2 = oracle.mxfp4_decode(w2c[e].numpy(), w2s[e].numpy()).astype(np.float64)
            u = xa[r0:r1] @ w2.T
            bu = MMA_TOL * _bound(xa[r0:r1], w2)
            if act == 1:
                h = g / (1.0 + np.exp(-g)) * u
                # first-order propagation: |d silu/dg| <= 1.1, |silu(g)| <= |g| + 0.28
                dmax, off_ = 1.1, 0.28
            else:
                # GELU, tanh form: 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3)));
                # |d gelu/dg| <= 1.129, |gelu(g)| <= |g|
                c = np.sqrt(2.0 / np.pi)
                h = 0.5 * g * (1.0 + np.tanh(c * (g + 0.044715 * g ** 3))) * u
                dmax, off_ = 1.13, 0.0
            tol = dmax * np.abs(u) * bg + (np.abs(g) + off_) * bu + 1e-5 * np.abs(h) + 1e-30
            assert (np.abs(got[r0:r1] - h) <= tol).all(), np.abs(got[r0:r1] - h).max()


def test_grouped_gemm_fp6x2_bf16_out_and_direct_rows(m):
    """No gathered rows, bf16 output, the down-projection shape (K = 1024,
    N = 3584 not a multiple of 256)."""
    rng = np.random.default_rng(9)
    nl, N, K = 3, 3584, 1024
    counts = np.array([200, 3, 70], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    hd, hval, _ = _split_rows(m, rng, A, K)
    wc, wsc = _experts(nl, N, K, 8)
    out = torch.empty(A, N, dtype=torch.bfloat16, device=DEV)
    ws = m.alloc_workspace(m.moe_grouped_gemm_fp6x2_workspace_size(nl, A), DEV)
    m.moe_grouped_gemm_fp6x2(hd, None, wc.to(DEV), wsc.to(DEV), None, None,
                             torch.from_numpy(off).to(DEV), A, 0, out, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    for e in range(nl):
        r0, r1 = off[e], off[e + 1]
        w = oracle.mxfp4_decode(wc[e].numpy(), wsc[e].numpy()).astype(np.float64)
        ref = hval[r0:r1] @ w.T
        b = MMA_TOL * _bound(hval[r0:r1], w)
        assert (np.abs(got[r0:r1] - ref) <= 2.0 ** -8 * (np.abs(ref) + b) + b).all()


@pytest.mark.parametrize("counts,K", [([150, 0, 257, 40], 384), ([900, 701], 384),
                                      ([900, 701], 4096)], ids=["16waves", "wide", "wide_k4096"])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("act", [1, 2])
def test_grouped_gemm_fp6x2_record_output_bitexact(m, act, packed, counts, K):
    """Split-record output (the layer's h): byte for byte the oracle's split
    of the fp32 output of the same launch configuration; rows past each
    group's end untouched. With at least 512 rows per expert (the row bound
    over the experts) the records come from the wide-wave tile (8 waves of
    64 x 128), the fp32 rows from the 16-wave one: the same sums either way;
    K = 4096 fills the wide tile's three-stage ring to 152 KB of LDS."""
    rng = np.random.default_rng(30 + act + 2 * packed + 5 * len(counts) + K)
    N, T = 320, 500
    counts = np.array(counts, np.int32)
    nl = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    xd, _, _ = _split_rows(m, rng, T, K)
    a_rows = torch.from_numpy(rng.integers(0, T, size=A).astype(np.int32)).to(DEV)
    w1c, w1s = _experts(nl, N, K, 5)
    w2c, w2s = _experts(nl, N, K, 6)
    dev = lambda t: t.to(DEV)
    pk = lambda c, s: m.moe_mxfp4_prepack(dev(c), dev(s)) if packed else (dev(c), dev(s))
    g1c, g1s = pk(w1c, w1s)
    g2c, g2s = pk(w2c, w2s)
    lay = m.LAYOUT_PACKED if packed else m.LAYOUT_OCP
    args = (xd, a_rows, g1c, g1s, g2c, g2s, torch.from_numpy(off).to(DEV), A, act)
    ws = m.alloc_workspace(m.moe_grouped_gemm_fp6x2_workspace_size(nl, A), DEV)
    f32 = torch.empty(A, N, dtype=torch.float32, device=DEV)
    m.moe_grouped_gemm_fp6x2(*args, f32, ws, w_layout=lay)
    rec = torch.full((A + 2, 2 * N), 0xA5, dtype=torch.uint8, device=DEV)
    m.moe_grouped_gemm_fp6x2(*args, rec, ws, w_layout=lay)
    torch.cuda.synchronize()
    rc, rs = oracle.fp6x2_split(np_(f32))
    codes, scales = unpack_split(np_(rec)[:A])
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc), np.argwhere(codes != rc)[:5]
    assert (np_(rec)[A:] == 0xA5).all()


# ---------------------------------------------------------------- layer
SMALL = [
    LayerConfig("f0", T=37, I=128, d=256, E=64, k=8),
    LayerConfig("f1", T=300, I=256, d=384, E=16, k=4),
    LayerConfig("f2", T=50, I=128, d=256, E=40, k=6, expert_begin=8, num_local=20, bias="normal"),
    LayerConfig("f3", T=700, I=128, d=256, E=100, k=6, bias="normal"),
    LayerConfig("f4", T=2600, I=256, d=512, E=32, k=8, bias="normal"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("packed", [False, True])
def test_small_layer_fp6x2_vs_oracle(m, cfg, packed):
    """The FP6X2 layer on 256-row tiles (tokens and h as two MXFP6 planes)
    against the oracle's bf16-activation layer on the GPU's scores, within the
    default contract; and no further from it than the GPU's bf16 layer (fp32
    outputs), which rounds h to bf16 where the FP6X2 layer carries h from its
    fp32 value."""
    inp = make_inputs(cfg).to(DEV)
    pw = m.prepack_weights(inp.weights) if packed else None
    g = run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=m.MODE_TILE256, packed=pw,
                      out_dtype=torch.float32)
    lg = np_(g["logits"])
    r_idx, _ = oracle.topk_softmax(lg, cfg.k)
    assert np.array_equal(np_(g["idx"]), r_idx)
    ref = oracle.layer(inp.x, np_(inp.w_router), None if inp.bias is None else np_(inp.bias),
                       host_weights(inp.weights), E=cfg.E, k=cfg.k, I=cfg.I,
                       e0=cfg.expert_begin, n_local=cfg.num_local, logits=lg)
    got = np_(g["out"])
    assert_close_layer(got, ref["out"], cfg.name)
    b = run_gpu_layer(inp, mode=m.MODE_TILE256, packed=pw, out_dtype=torch.float32)
    assert torch.equal(b["idx"], g["idx"])
    e6, e16 = rel_l2(got, ref["out"]), rel_l2(np_(b["out"]), ref["out"])
    print(f"{cfg.name}: rel-L2 FP6X2 {e6:.3e}, bf16 {e16:.3e}")
    assert e6 <= max(1.5 * e16, 1e-3)
    assert not torch.equal(b["out"], g["out"])  # the FP6X2 projections ran


@pytest.mark.parametrize("cfg", [SMALL[4], LayerConfig("f5", T=3000, I=256, d=512, E=64, k=8,
                                                       expert_begin=16, num_local=24,
                                                       bias="normal")], ids=lambda c: c.name)
def test_auto_schedule_takes_fp6x2(m, cfg):
    """With the schedule left to the library and a mean of 128 or more rows
    per local expert over the row bound, the FP6X2 layer runs (bitwise the
    explicit 256-row choice, whatever tiles it picks per projection), here
    also on a local expert range."""
    inp = make_inputs(cfg).to(DEV)
    a = run_gpu_layer(inp, precision=m.PREC_FP6X2, out_dtype=torch.float32)
    b = run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=m.MODE_TILE256, out_dtype=torch.float32)
    for key in a:
        assert torch.equal(a[key], b[key]), key
    lg = np_(a["logits"])
    ref = oracle.layer(inp.x, np_(inp.w_router), None if inp.bias is None else np_(inp.bias),
                       host_weights(inp.weights), E=cfg.E, k=cfg.k, I=cfg.I,
                       e0=cfg.expert_begin, n_local=cfg.num_local, logits=lg)
    assert_close_layer(np_(a["out"]), ref["out"], cfg.name)


@pytest.mark.parametrize("cfg", [SMALL[1], SMALL[4]], ids=lambda c: c.name)
def test_fp6x2_layer_block_int16_expert_outputs(m, cfg):
    """Inside the FP6X2 layer the expert outputs Y travel as block-int16 rows
    (per 32 columns the biased exponent e of the largest magnitude; each value
    as the integer nearest 32767 v 2^(126 - e)). Against the same layer built
    from the standalone entry points -- the permutation, the split, the
    gate/up projection's records and the down projection's fp32 rows -- and
    an fp32 combine of those unrounded rows in slot order: every output
    element within sum_j w_j (0.5 + 2^-9) step_j plus fp32 rounding, step_j
    the code spacing of row j's block. A rounding toward zero (errors up to a
    whole step), a wrong exponent or a wrong block would exceed that on many
    of the elements."""
    inp = make_inputs(cfg).to(DEV)
    T, k, d, I, nl = cfg.T, cfg.k, cfg.d, cfg.I, cfg.num_local
    g = run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=m.MODE_TILE256, out_dtype=torch.float32)
    A = T * k
    off = torch.empty(nl + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(A, dtype=torch.int32, device=DEV)
    inv = torch.empty(T, k, dtype=torch.int32, device=DEV)
    pws = m.alloc_workspace(m.moe_permute_workspace_size(T, nl), DEV)
    m.moe_permute(g["idx"], None, cfg.expert_begin, nl, off, perm, inv, pws, E=cfg.E)
    W = inp.weights
    xd = m.moe_fp6x2_split(inp.x)
    ws = m.alloc_workspace(m.moe_grouped_gemm_fp6x2_workspace_size(nl, A), DEV)
    hrec = torch.empty(A, 2 * I, dtype=torch.uint8, device=DEV)
    m.moe_grouped_gemm_fp6x2(xd, perm, W["gate_codes"], W["gate_scales"], W["up_codes"],
                             W["up_scales"], off, A, 1, hrec, ws)
    y = torch.zeros(A, d, dtype=torch.float32, device=DEV)
    m.moe_grouped_gemm_fp6x2(hrec, None, W["down_codes"], W["down_scales"], None, None, off, A, 0,
                             y, ws)
    torch.cuda.synchronize()
    yv, iv, wv = np_(y), np_(inv), np_(g["w"])
    step = block_int16_step(yv)
    ref = np.zeros((T, d), np.float32)
    bound = np.zeros((T, d), np.float64)
    mag = np.zeros((T, d), np.float64)
    for j in range(k):
        r = iv[:, j]
        on = r >= 0
        wj = np.where(on, wv[:, j], 0.0).astype(np.float32)[:, None]
        rows = np.where(on, r, 0)
        ref = ref + wj * yv[rows]
        bound += wj.astype(np.float64) * step[rows]
        mag += np.abs(wj.astype(np.float64) * yv[rows])
    got = np_(g["out"]).astype(np.float64)
    diff = np.abs(got - ref.astype(np.float64))
    lim = (0.5 + 2.0 ** -9) * bound + 4 * k * 2.0 ** -24 * mag
    print(f"{cfg.name}: max |out - fp32-Y out| / sum w step = {(diff / bound).max():.3f}")
    assert (diff <= lim).all(), (diff - lim).max()


@pytest.mark.parametrize("cfg", [SMALL[1], SMALL[2]], ids=lambda c: c.name)
def test_fp6x2_layer_bf16_output_is_fp32_rounded(m, cfg):
    """The FP6X2 layer's bf16 output (the block-int16 combine's bf16 store) is
    exactly its fp32 output rounded to nearest-even, on every element."""
    inp = make_inputs(cfg).to(DEV)
    a = run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=m.MODE_TILE256, out_dtype=torch.float32)
    b = run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=m.MODE_TILE256, out_dtype=torch.bfloat16)
    assert torch.equal(a["idx"], b["idx"])
    assert torch.equal(b["out"], a["out"].to(torch.bfloat16))


def test_fp6x2_layer_determinism_bitwise(m):
    inp = make_inputs(SMALL[4]).to(DEV)
    a = run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=m.MODE_TILE256)
    b = run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=m.MODE_TILE256)
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("cfg,act,packed", [
    # K = 512 and 256: three-stage rings on both tile heights
    (LayerConfig("h0", T=700, I=256, d=512, E=24, k=6, bias="normal"), 1, False),
    # K = 1536 (gate/up) and 2048 (down): two stages on 128-row tiles
    (LayerConfig("h1", T=600, I=2048, d=1536, E=16, k=4, expert_begin=4, num_local=8), 1, True),
    # K = 3584 (two stages) and 1024 (three), about 300 rows per expert
    (LayerConfig("h2", T=1200, I=1024, d=3584, E=16, k=4, bias="normal"), 2, True),
    # K = 4096, the largest taken: 80 KB of LDS on 128-row tiles, 152 KB on 256
    (LayerConfig("h3", T=300, I=2048, d=4096, E=4, k=2), 1, True),
    # 512 rows per expert (the row bound's mean): the 256-row gate/up tiles on
    # wide waves (8 waves of 64 x 128), streaming and canonical weights
    (LayerConfig("h4", T=2048, I=256, d=512, E=8, k=2, bias="normal"), 1, True),
    (LayerConfig("h5", T=1536, I=384, d=640, E=6, k=2), 2, False),
], ids=lambda v: v.name if isinstance(v, LayerConfig) else str(v))
def test_fp6x2_layer_tile_heights_bitwise(m, cfg, act, packed):
    """An output element is the same sum on 256- and 128-row tiles (the same
    K steps and planes in the same order; the tile only decides which
    workgroup computes it): the layer on 128-row tiles (8 waves, two
    workgroups per CU, a two-stage ring where three do not fit 80 KB), on
    256-row tiles (16 waves of 64 x 64, or for gate/up over 512 rows per
    expert 8 waves of 64 x 128) and under the automatic per-projection choice
    agree bit for bit, records, block-int16 rows and all."""
    inp = make_inputs(cfg).to(DEV)
    pw = m.prepack_weights(inp.weights) if packed else None
    runs = [run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=md, act=act, packed=pw,
                          out_dtype=torch.float32)
            for md in (m.MODE_TILE256, m.MODE_TILE128, m.MODE_AUTO)]
    assert runs[0]["out"].abs().max() > 0
    for r in runs[1:]:
        for key in r:
            assert torch.equal(r[key], runs[0][key]), key


@pytest.mark.parametrize("act", [1, 2])
def test_fp6x2_layer_128_row_tiles_vs_oracle(m, act):
    """The FP6X2 layer on 128-row tiles (MOE_SCHED_TILE128, both projections)
    with SiLU and GELU-tanh against the oracle's layer of the same activation
    on the GPU's scores, within the default contract."""
    cfg = SMALL[4]
    inp = make_inputs(cfg).to(DEV)
    g = run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=m.MODE_TILE128, act=act,
                      packed=m.prepack_weights(inp.weights), out_dtype=torch.float32)
    lg = np_(g["logits"])
    r_idx, _ = oracle.topk_softmax(lg, cfg.k)
    assert np.array_equal(np_(g["idx"]), r_idx)
    ref = oracle.layer(inp.x, np_(inp.w_router), None if inp.bias is None else np_(inp.bias),
                       host_weights(inp.weights), E=cfg.E, k=cfg.k, I=cfg.I,
                       e0=cfg.expert_begin, n_local=cfg.num_local, logits=lg, act=act)
    assert_close_layer(np_(g["out"]), ref["out"], f"{cfg.name} act={act}")


def test_fp6x2_streaming_shapes_are_the_bf16_layer(m):
    """Where the schedule streams the weights (few rows per expert) the FP6X2
    precision runs the bf16 kernels: bitwise the bf16 layer."""
    inp = make_inputs(SMALL[0]).to(DEV)
    a = run_gpu_layer(inp, precision=m.PREC_FP6X2, mode=m.MODE_STREAM)
    b = run_gpu_layer(inp, mode=m.MODE_STREAM)
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("name", ["prefill", "ep_share", "long_skewed_prefill"])
def test_full_size_fp6x2(m, name):
    """The prefill-sized workloads with the FP6X2 gate/up projection, in the
    benchmark's launch configuration (streaming-layout weights, schedule
    chosen automatically, fp32 output): routing on every token, 64 sampled
    tokens' rows (segment edges, the hottest expert, seeded random) against
    the oracle's bf16-activation layer, within the default contract."""
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, DEV)
    g = run_gpu_layer(inp, precision=m.PREC_FP6X2, packed=m.prepack_weights(inp.weights),
                      out_dtype=torch.float32)
    r_idx, _ = oracle.topk_softmax(np_(g["logits"]), cfg.k)
    assert np.array_equal(np_(g["idx"]), r_idx)
    toks = sample_tokens(cfg, r_idx, 64, seed=3)
    ref = oracle_rows(inp, r_idx, np_(g["w"]), toks)
    got = g["out"].float().cpu().numpy()[toks]
    print(f"{name}: rel-L2 {rel_l2(got, ref):.3e}")
    assert_close_layer(got, ref, name)
    del inp, g
    torch.cuda.empty_cache()
