"""GPU parity of the block-scaled precision mode (MX8: MXFP8 tokens and h,
MXFP4 weights, v_mfma_scale_f32_32x32x64_f8f6f4) against the oracle's MX8
definition.

Stage by stage: the quantiser byte for byte; the grouped projection
elementwise against the exact sum of exactly decoded operands, within the
instruction's summation bound; the layer against the oracle's MX8 layer on
the GPU's routing. The bound of the projection comes from the instruction:
its products are exact and a one-wave measurement of its 64-long sums put
them within 1.1e-4 of sum|products| (about 13 bits); fp32 accumulation over
K/64 of them adds at most K/64 * 2^-24 of sum|products|. The tests allow
2e-4 * sum|a w|."""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, LayerConfig, make_inputs, quantize_mxfp4
from tests.parity_util import (assert_close_layer, block_int16_step, host_weights, np_,
                               oracle_rows, rel_l2, run_gpu_layer, sample_tokens)
from tests.test_oracle_mx8 import _blocks

pytestmark = pytest.mark.gpu
DEV = "cuda"
MMA_TOL = 2e-4


@pytest.fixture(scope="module")
def m():
    import mxfp4_expert_top_amd as mod
    return mod


# ---------------------------------------------------------------- quantiser
@pytest.mark.parametrize("K", [32, 128, 3584])
def test_mxfp8_quantize_fp32_bitexact(m, K):
    v = _blocks().reshape(-1)
    v = np.resize(v, ((v.size + K - 1) // K) * K).reshape(-1, K).astype(np.float32)
    rnd = np.random.default_rng(K).standard_normal((7, K)).astype(np.float32)
    v = np.ascontiguousarray(np.concatenate([v, rnd * 3.0, rnd * 1e-30]))
    c, s = m.moe_mxfp8_quantize(torch.from_numpy(v).to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.mxfp8_quantize(v)
    assert np.array_equal(np_(s), rs)
    assert np.array_equal(np_(c), rc), np.argwhere(np_(c) != rc)[:5]


def test_mxfp8_quantize_bf16_rows_with_stride(m):
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((33, 3584 + 64)).astype(np.float32)).to(torch.bfloat16)
    x[3, :64] = 0
    x[4] *= 1e-20
    xv = x[:, :3584]
    c, s = m.moe_mxfp8_quantize(x.to(DEV)[:, :3584])  # rows of 3584 at a stride of 3648
    torch.cuda.synchronize()
    rc, rs = oracle.mxfp8_quantize(xv.float().numpy())
    assert np.array_equal(np_(s), rs) and np.array_equal(np_(c), rc)


def test_mxfp8_quantize_grid_stride(m):
    """More 32-element blocks (140000 x 32) than the launch's threads (16384 x 256): the
    threads past the first pass's end and rows on both sides of the wrap, against the oracle."""
    N, K = 140000, 1024
    g = torch.Generator(device=DEV).manual_seed(7)
    v = torch.randn(N, K, generator=g, device=DEV) * 2.0
    c, s = m.moe_mxfp8_quantize(v)
    torch.cuda.synchronize()
    wrap = 16384 * 256 // (K // 32)  # first row of the second pass
    rows = np.r_[0:4, wrap - 4:wrap + 4, N - 4:N]
    rc, rs = oracle.mxfp8_quantize(v[torch.from_numpy(rows).to(DEV)].cpu().numpy())
    assert np.array_equal(np_(s)[rows], rs)
    assert np.array_equal(np_(c)[rows], rc)


# ---------------------------------------------------------------- projection
def _experts(num_local, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    cs = [quantize_mxfp4(torch.randn(N, K, generator=g) / np.sqrt(K)) for _ in range(num_local)]
    return torch.stack([c for c, _ in cs]), torch.stack([s for _, s in cs])


def _mx8_rows(rng, R, K):
    v = (rng.standard_normal((R, K)) * np.exp2(rng.integers(-3, 4, (R, 1)))).astype(np.float32)
    return oracle.mxfp8_quantize(v)


def _bound(a, w):
    """sum_k |a_k w_k| for every (row, weight row)."""
    return np.abs(a) @ np.abs(w).T


@pytest.mark.parametrize("mode", [1, 3, 4])
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("K", [128, 640])
def test_grouped_gemm_mx8_vs_definition(m, act, packed, K, mode):
    """Experts with 0, 1, 37, 150, 257 and 513 rows (empty, one row, ragged,
    several 128- and 256-row groups), a column count that is not a tile
    multiple, gathered rows, fp32 output; both tile heights."""
    rng = np.random.default_rng(K + 3 * act + 7 * packed)
    nl, N, T = 6, 320, 700
    counts = np.array([37, 0, 513, 1, 257, 150], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    xc, xs = _mx8_rows(rng, T, K)
    a_rows = rng.integers(0, T, size=A).astype(np.int32)
    w1c, w1s = _experts(nl, N, K, 3)
    w2c, w2s = _experts(nl, N, K, 4) if act else (None, None)
    dev = lambda t: None if t is None else t.to(DEV)
    pk = lambda c, s: m.moe_mxfp4_prepack(dev(c), dev(s)) if packed else (dev(c), dev(s))
    g1c, g1s = pk(w1c, w1s)
    g2c, g2s = pk(w2c, w2s) if act else (None, None)
    out = torch.full((A + 3, N), 7.0, dtype=torch.float32, device=DEV)
    ws = m.alloc_workspace(m.moe_grouped_gemm_mx8_workspace_size(nl, A), DEV)
    m.moe_grouped_gemm_mx8(torch.from_numpy(xc).to(DEV), torch.from_numpy(xs).to(DEV),
                           torch.from_numpy(a_rows).to(DEV), g1c, g1s, g2c, g2s,
                           torch.from_numpy(off).to(DEV), A, act, out, ws,
                           w_layout=m.LAYOUT_PACKED if packed else m.LAYOUT_OCP, mode=mode)
    torch.cuda.synchronize()
    got = np_(out).astype(np.float64)
    assert (got[A:] == 7.0).all()
    xa = oracle.mxfp8_decode(xc, xs).astype(np.float64)[a_rows]
    for e in range(nl):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            continue
        w1 = oracle.mxfp4_decode(w1c[e].numpy(), w1s[e].numpy()).astype(np.float64)
        g = xa[r0:r1] @ w1.T
        bg = MMA_TOL * _bound(xa[r0:r1], w1)
        if act == 0:
            assert (np.abs(got[r0:r1] - g) <= bg).all(), np.abs(got[r0:r1] - g).max()
        else:
            w2 = oracle.mxfp4_decode(w2c[e].numpy(), w2s[e].numpy()).astype(np.float64)
            u = xa[r0:r1] @ w2.T
            bu = MMA_TOL * _bound(xa[r0:r1], w2)
            sg = 1.0 / (1.0 + np.exp(-g))
            h = g * sg * u
            # first-order propagation: |d silu/dg| <= 1.1, |silu(g)| <= |g| + 0.28
            tol = 1.1 * np.abs(u) * bg + (np.abs(g) + 0.28) * bu + 1e-5 * np.abs(h) + 1e-30
            assert (np.abs(got[r0:r1] - h) <= tol).all(), np.abs(got[r0:r1] - h).max()


@pytest.mark.parametrize("mode", [1, 3, 4])
def test_grouped_gemm_mx8_strided_rows(m, mode):
    """Rows with a stride past K (lda = K + 32, so lda / 32 scale bytes per
    row is not a whole number of dwords); the padding holds E4M3 NaN codes
    and NaN scales, which must never be read."""
    rng = np.random.default_rng(5 + mode)
    nl, N, T, K, lda = 4, 320, 400, 128, 160
    counts = np.array([70, 0, 290, 3], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    xc, xs = _mx8_rows(rng, T, K)
    xc_full = np.full((T, lda), 0x7F, np.uint8)
    xs_full = np.full((T, lda // 32), 0xFF, np.uint8)
    xc_full[:, :K] = xc
    xs_full[:, :K // 32] = xs
    a_rows = rng.integers(0, T, size=A).astype(np.int32)
    w1c, w1s = _experts(nl, N, K, 8)
    w2c, w2s = _experts(nl, N, K, 9)
    out = torch.full((A + 3, N), 7.0, dtype=torch.float32, device=DEV)
    ws = m.alloc_workspace(m.moe_grouped_gemm_mx8_workspace_size(nl, A), DEV)
    gc = torch.from_numpy(xc_full).to(DEV)
    gs = torch.from_numpy(xs_full).to(DEV)
    m.moe_grouped_gemm_mx8(gc[:, :K], gs[:, :K // 32], torch.from_numpy(a_rows).to(DEV),
                           w1c.to(DEV), w1s.to(DEV), w2c.to(DEV), w2s.to(DEV),
                           torch.from_numpy(off).to(DEV), A, 1, out, ws, mode=mode)
    torch.cuda.synchronize()
    got = np_(out).astype(np.float64)
    assert np.isfinite(got).all()
    assert (got[A:] == 7.0).all()
    xa = oracle.mxfp8_decode(xc, xs).astype(np.float64)[a_rows]
    for e in range(nl):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            continue
        w1 = oracle.mxfp4_decode(w1c[e].numpy(), w1s[e].numpy()).astype(np.float64)
        w2 = oracle.mxfp4_decode(w2c[e].numpy(), w2s[e].numpy()).astype(np.float64)
        g, u = xa[r0:r1] @ w1.T, xa[r0:r1] @ w2.T
        bg, bu = MMA_TOL * _bound(xa[r0:r1], w1), MMA_TOL * _bound(xa[r0:r1], w2)
        h = g / (1.0 + np.exp(-g)) * u
        tol = 1.1 * np.abs(u) * bg + (np.abs(g) + 0.28) * bu + 1e-5 * np.abs(h) + 1e-30
        assert (np.abs(got[r0:r1] - h) <= tol).all(), np.abs(got[r0:r1] - h).max()


def test_grouped_gemm_mx8_bf16_out_and_direct_rows(m):
    """No gathered rows (a_rows NULL), bf16 output, the down-projection shape
    (K = 1024, N = 3584 not a tile multiple of 256)."""
    rng = np.random.default_rng(9)
    nl, N, K = 3, 3584, 1024
    counts = np.array([200, 3, 70], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    hc, hs = _mx8_rows(rng, A, K)
    wc, wsc = _experts(nl, N, K, 8)
    out = torch.empty(A, N, dtype=torch.bfloat16, device=DEV)
    ws = m.alloc_workspace(m.moe_grouped_gemm_mx8_workspace_size(nl, A), DEV)
    m.moe_grouped_gemm_mx8(torch.from_numpy(hc).to(DEV), torch.from_numpy(hs).to(DEV), None,
                           wc.to(DEV), wsc.to(DEV), None, None, torch.from_numpy(off).to(DEV),
                           A, 0, out, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ha = oracle.mxfp8_decode(hc, hs).astype(np.float64)
    for e in range(nl):
        r0, r1 = off[e], off[e + 1]
        w = oracle.mxfp4_decode(wc[e].numpy(), wsc[e].numpy()).astype(np.float64)
        ref = ha[r0:r1] @ w.T
        # bf16 rounding of a value within the summation bound of the exact sum
        err = np.abs(got[r0:r1] - ref)
        assert (err <= 2.0 ** -8 * (np.abs(ref) + MMA_TOL * _bound(ha[r0:r1], w))
                + MMA_TOL * _bound(ha[r0:r1], w)).all()


@pytest.mark.parametrize("mode", [3, 4])
@pytest.mark.parametrize("act", [0, 1])
def test_grouped_gemm_mx8_mxfp8_output_bitexact(m, act, mode):
    """MXFP8 output (the layer's h): codes and scales equal the oracle's
    quantiser applied to the fp32 output of the same launch configuration,
    byte for byte; rows past each group's end and columns past N untouched."""
    rng = np.random.default_rng(20 + act)
    nl, N, K, T = 4, 320, 384, 500
    counts = np.array([150, 0, 257, 40], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    xc, xs = _mx8_rows(rng, T, K)
    a_rows = torch.from_numpy(rng.integers(0, T, size=A).astype(np.int32)).to(DEV)
    w1c, w1s = _experts(nl, N, K, 5)
    w2c, w2s = _experts(nl, N, K, 6) if act else (None, None)
    dev = lambda t: None if t is None else t.to(DEV)
    args = (torch.from_numpy(xc).to(DEV), torch.from_numpy(xs).to(DEV), a_rows, dev(w1c),
            dev(w1s), dev(w2c), dev(w2s), torch.from_numpy(off).to(DEV), A, act)
    ws = m.alloc_workspace(m.moe_grouped_gemm_mx8_workspace_size(nl, A), DEV)
    f32 = torch.empty(A, N, dtype=torch.float32, device=DEV)
    m.moe_grouped_gemm_mx8(*args, f32, ws, mode=mode)
    codes = torch.full((A + 2, N), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((A + 2, N // 32), 0x5A, dtype=torch.uint8, device=DEV)
    m.moe_grouped_gemm_mx8(*args, codes, ws, out_scales=scales, mode=mode)
    torch.cuda.synchronize()
    rc, rs = oracle.mxfp8_quantize(np_(f32))
    assert np.array_equal(np_(scales)[:A], rs)
    assert np.array_equal(np_(codes)[:A], rc)
    assert (np_(codes)[A:] == 0xA5).all() and (np_(scales)[A:] == 0x5A).all()


# ---------------------------------------------------------------- layer
SMALL = [
    LayerConfig("x0", T=37, I=128, d=256, E=64, k=8),
    LayerConfig("x1", T=300, I=256, d=384, E=16, k=4),
    LayerConfig("x2", T=50, I=128, d=256, E=40, k=6, expert_begin=8, num_local=20, bias="normal"),
    LayerConfig("x3", T=700, I=128, d=256, E=100, k=6, bias="normal"),
]


def _routing(inp, g):
    c = inp.cfg
    lg = np_(g["logits"])
    r_idx, r_w = oracle.topk_softmax(lg, c.k)
    assert np.array_equal(np_(g["idx"]), r_idx)
    return lg, r_idx, r_w


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("mode", [0, 1, 3, 4])
def test_small_layer_mx8_vs_oracle(m, cfg, packed, mode):
    """The whole MX8 layer against the oracle's MX8 layer on the GPU's scores.
    Both round h to E4M3 from fp32 values that differ by the instruction's
    summation error, so a few h codes may sit one E4M3 step apart; the layer
    bounds (rel-L2 1e-2, max-abs 3e-2 rms) cover that. The routing is the
    bf16 path's, bit for bit."""
    inp = make_inputs(cfg).to(DEV)
    g = run_gpu_layer(inp, precision=m.PREC_MX8, mode=mode,
                      packed=m.prepack_weights(inp.weights) if packed else None)
    lg, _, _ = _routing(inp, g)
    ref = oracle.layer(inp.x, np_(inp.w_router), None if inp.bias is None else np_(inp.bias),
                       host_weights(inp.weights), E=cfg.E, k=cfg.k, I=cfg.I,
                       e0=cfg.expert_begin, n_local=cfg.num_local, logits=lg, mx8=True)
    got = g["out"].float().cpu().numpy()
    assert_close_layer(got, ref["out"], cfg.name)
    # the bf16-activation layer differs by the activation rounding (E4M3 steps
    # are 2^-3 of the value): far more than the parity gap above
    ref16 = oracle.layer(inp.x, np_(inp.w_router), None if inp.bias is None else np_(inp.bias),
                         host_weights(inp.weights), E=cfg.E, k=cfg.k, I=cfg.I,
                         e0=cfg.expert_begin, n_local=cfg.num_local, logits=lg)
    assert rel_l2(got, ref16["out"]) > 2 * rel_l2(got, ref["out"])


def test_mx8_layer_determinism_bitwise(m):
    inp = make_inputs(SMALL[1]).to(DEV)
    a = run_gpu_layer(inp, precision=m.PREC_MX8)
    b = run_gpu_layer(inp, precision=m.PREC_MX8)
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("cfg", [SMALL[1], SMALL[2], SMALL[3]], ids=lambda c: c.name)
def test_mx8_layer_block_int16_expert_outputs(m, cfg):
    """On the 256-row tile the MX8 layer carries the expert outputs Y as
    block-int16 rows (per 32 columns the biased exponent e of the largest
    magnitude, each value the integer nearest 32767 v 2^(126 - e)). Rebuilt
    from the standalone entry points -- the permutation, MXFP8 tokens, the
    gate/up projection's fp32 h, MXFP8 h and the down projection's fp32 rows
    on the same tile -- and combined in fp32 in slot order, every output
    element lies within sum_j w_j (0.5 + 2^-9) step_j plus fp32 rounding,
    step_j the code spacing of row j's block. Rounding toward zero, a wrong
    exponent or a wrong block would exceed that. x2 is an EP share: h rows
    past the local ones are never read."""
    inp = make_inputs(cfg).to(DEV)
    T, k, d, I, nl = cfg.T, cfg.k, cfg.d, cfg.I, cfg.num_local
    g = run_gpu_layer(inp, precision=m.PREC_MX8, mode=m.MODE_TILE256, out_dtype=torch.float32)
    A = T * k
    off = torch.empty(nl + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(A, dtype=torch.int32, device=DEV)
    inv = torch.empty(T, k, dtype=torch.int32, device=DEV)
    pws = m.alloc_workspace(m.moe_permute_workspace_size(T, nl), DEV)
    m.moe_permute(g["idx"], None, cfg.expert_begin, nl, off, perm, inv, pws, E=cfg.E)
    W = inp.weights
    xc, xs = m.moe_mxfp8_quantize(inp.x)
    ws = m.alloc_workspace(m.moe_grouped_gemm_mx8_workspace_size(nl, A), DEV)
    h = torch.zeros(A, I, dtype=torch.float32, device=DEV)
    m.moe_grouped_gemm_mx8(xc, xs, perm, W["gate_codes"], W["gate_scales"], W["up_codes"],
                           W["up_scales"], off, A, 1, h, ws, mode=m.MODE_TILE256)
    hc, hs = m.moe_mxfp8_quantize(h)
    y = torch.zeros(A, d, dtype=torch.float32, device=DEV)
    m.moe_grouped_gemm_mx8(hc, hs, None, W["down_codes"], W["down_scales"], None, None, off, A, 0,
                           y, ws, mode=m.MODE_TILE256)
    torch.cuda.synchronize()
    yv, iv, wv = np_(y), np_(inv), np_(g["w"])
    assert (iv < int(np_(off)[nl])).all()
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
    print(f"{cfg.name}: max |out - fp32-Y out| / sum w step = {(diff / np.maximum(bound, 1e-300)).max():.3f}")
    assert (diff <= lim).all(), (diff - lim).max()
    # the rounding is visible: the block-int16 output is not the fp32-Y one
    assert not np.array_equal(got, ref.astype(np.float64))


@pytest.mark.parametrize("name", ["prefill", "decode", "ep_share", "long_skewed_prefill"])
def test_full_size_mx8(m, name):
    """The workloads in the MX8 mode, in the benchmark's launch configuration
    (fp32 output): 64 sampled tokens' rows (segment edges, the hottest
    expert, seeded random) against the oracle's MX8 rows on the GPU's
    routing."""
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, DEV)
    g = run_gpu_layer(inp, precision=m.PREC_MX8, packed=m.prepack_weights(inp.weights),
                      out_dtype=torch.float32)
    _, r_idx, _ = _routing(inp, g)
    toks = sample_tokens(cfg, r_idx, 64, seed=1)
    ref = oracle_rows(inp, r_idx, np_(g["w"]), toks, mx8=True)
    assert_close_layer(g["out"].float().cpu().numpy()[toks], ref, name)
    del inp, g
    torch.cuda.empty_cache()
