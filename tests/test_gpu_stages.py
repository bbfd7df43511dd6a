"""GPU parity of each C-ABI entry point against the oracle, on seeded inputs
that span several tiles with ragged tails, plus the degenerate cases."""

import numpy as np
import pytest
import torch

import oracle
from synth import LayerConfig, quantize_mxfp4
from tests.dense_ref import ACTS
from tests.parity_util import W_TOL, LOGIT_TOL, bf16_rounding_ok, np_, rel_l2, max_abs_rms

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import mxfp4_expert_top_amd as mod
    return mod


# ---------------------------------------------------------------- decode
def test_dequant_every_code_and_scale_bitexact(m):
    """Every E2M1 code under every finite E8M0 scale code (row s uses scale
    code s, 0..254): subnormal results of codes 0 and 1 and the overflow to
    +-inf of codes 253 and 254 included, bit for bit with the oracle."""
    S = np.arange(0, 255)
    N, K = len(S), 128
    nib = np.tile(np.arange(16), (N, K // 16))
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = np.repeat(S[:, None], K // 32, axis=1).astype(np.uint8)
    out = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)
    m.moe_mxfp4_dequant(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    want = oracle.mxfp4_decode(codes, scales)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # -0 stays -0
    assert (want[:2] != 0).any() and np.isinf(want[253:]).any()  # both edges reached


@pytest.mark.parametrize("sc", [0, 1])
@pytest.mark.parametrize("mode", [1, 3, 4])
def test_grouped_gemm_subnormal_weight_scales(m, sc, mode):
    """Weights whose scale code is 0 or 1 decode to bf16 subnormals; against
    activations of 2^100 their products are ordinary numbers, and the
    grouped GEMM gives them exactly (every product and sum exact in fp32)."""
    rng = np.random.default_rng(sc)
    R, K, N = 32, 128, 64
    wc = rng.integers(0, 256, (1, N, K // 2), dtype=np.uint8)
    ws = np.full((1, N, K // 32), sc, np.uint8)
    a = torch.full((R, K), 2.0 ** 100, dtype=torch.bfloat16)
    off = torch.tensor([0, R], dtype=torch.int32, device=DEV)
    out = torch.empty(R, N, dtype=torch.float32, device=DEV)
    wsb = m.alloc_workspace(m.moe_grouped_gemm_workspace_size(1, R, N), DEV)
    m.moe_grouped_gemm_mxfp4(a.to(DEV), None, torch.from_numpy(wc).to(DEV),
                             torch.from_numpy(ws).to(DEV), None, None, off, R, 0, out, wsb,
                             mode=mode)
    torch.cuda.synchronize()
    ref = a.double().numpy() @ oracle.mxfp4_decode(wc[0], ws[0]).astype(np.float64).T
    assert np.abs(ref).max() > 1e-7
    assert np.array_equal(np_(out).astype(np.float64), ref)


def _quantize_cases():
    """Rows of 64 (two MX blocks each) that reach every branch of the
    encoding: scales from subnormal to huge, exact rounding ties, saturation,
    all-zero and signed-zero blocks."""
    rng = np.random.default_rng(11)
    rows = []
    for k in range(-149, 126, 5):  # amax around 2^k, subnormal to near the fp32 top
        r = rng.standard_normal(64) * np.float64(2.0) ** k
        rows.append(r)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.2499, 0.2501, 0.7499, 5.0001,
                     4.9999, 1.7501, 2.4999, 3.4999, 1.2501])
    for k in (-120, -3, 0, 7, 100):
        for sgn in (1.0, -1.0):
            blk = np.concatenate([[6.0], sgn * ties, -ties[:15]]) * 2.0 ** k  # amax 6 * 2^k
            rows.append(np.concatenate([blk, blk[::-1]]))
    sat = np.array([7.9, 7.0, 6.5, 6.0, 5.9, 5.1, -7.5, -6.01] * 4) * 2.0 ** -5  # |q| up to 7.9
    rows.append(np.concatenate([sat, -sat]))
    rows.append(np.zeros(64))
    rows.append(-np.zeros(64))
    mixed = np.zeros(64)
    mixed[::2] = -0.0
    mixed[5] = 1e-3
    mixed[40] = -3.0
    rows.append(mixed)
    big = np.full(64, 3.0e38)
    big[1::2] = -1.7e38
    rows.append(big)
    sub = np.full(64, 1.4e-45)
    sub[7] = -2.8e-45
    rows.append(sub)
    return np.ascontiguousarray(np.stack(rows).astype(np.float32))


@pytest.mark.parametrize("K", [64, 3584])
def test_quantize_bitexact(m, K):
    w = _quantize_cases()
    if K != 64:  # the same rows spread over long rows, plus random ones
        g = np.random.default_rng(12).standard_normal((9, K)).astype(np.float32) * 0.02
        tiled = np.resize(w, (w.size // K + 1) * K)[: (w.size // K) * K].reshape(-1, K)
        w = np.ascontiguousarray(np.concatenate([tiled, g]))
    codes, scales = m.moe_mxfp4_quantize(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    want_c, want_s = oracle.mxfp4_quantize(w)
    assert np.array_equal(np_(scales), want_s)
    assert np.array_equal(np_(codes), want_c)


def test_quantize_then_decode_round_trip(m):
    # decoding what was quantised gives the nearest grid value: within half an
    # E2M1 step (relative to the block scale) of each input
    g = torch.Generator().manual_seed(13)
    w = (torch.randn(64, 256, generator=g) * 0.05).to(DEV)
    codes, scales = m.moe_mxfp4_quantize(w)
    out = torch.empty(64, 256, dtype=torch.bfloat16, device=DEV)
    m.moe_mxfp4_dequant(codes, scales, out)
    torch.cuda.synchronize()
    err = (out.float() - w).abs().view(64, 8, 32)
    step = torch.pow(2.0, scales.float() - 127).view(64, 8, 1)  # the scale: grid spacing 0.5 .. 2
    assert bool((err <= step * 2.0).all())  # |q| in [6, 8) saturates to 6


def test_dequant_random_weights_bitexact(m):
    g = torch.Generator().manual_seed(5)
    w = torch.randn(300, 512, generator=g) * 0.02
    c, s = quantize_mxfp4(w)
    out = torch.empty(300, 512, dtype=torch.bfloat16, device=DEV)
    m.moe_mxfp4_dequant(c.to(DEV), s.to(DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), oracle.mxfp4_decode(c.numpy(), s.numpy()))


# ---------------------------------------------------------------- routing
def _route_gpu(m, logits_np, k, x=None, w_router=None, bias=None, given=True):
    T, E = logits_np.shape
    lg = torch.from_numpy(np.ascontiguousarray(logits_np)).to(DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    cnt = torch.full((E,), 12345, dtype=torch.int32, device=DEV)
    m.moe_route(x, w_router, bias, lg, given, idx, w, cnt)
    torch.cuda.synchronize()
    return np_(lg), np_(idx), np_(w), np_(cnt)


def _tie_logits(T, E, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[1] = np.round(lg[1] * 2) / 2         # many exact ties
    lg[2] = 0.0
    lg[2, ::3] = -0.0                       # +-0: all tie
    lg[3] = 0.75                            # all equal
    lg[4] = rng.integers(-3, 3, size=E)
    lg[5, E // 2:] = lg[5, : E - E // 2]    # duplicated halves
    if T > 7:
        # experts e with e % 64 < 16 far ahead: many large scores share the
        # same lanes of a 64-wide layout (a kernel that packs candidates per
        # lane sees more than 64 of them)
        lg[6, (np.arange(E) % 64) < 16] += 10.0
        lg[7] = np.arange(E, dtype=np.float32)[::-1] / E  # strictly decreasing by id
    return lg


@pytest.mark.parametrize("T,E,k", [(300, 896, 16), (77, 64, 8), (40, 17, 1), (33, 2048, 32),
                                   (6, 16, 16), (1, 896, 16)])
def test_route_injected_logits_bitexact(m, T, E, k):
    lg = _tie_logits(max(T, 8), E, T * 7 + E)[:T]
    _, idx, w, cnt = _route_gpu(m, lg, k)
    oi, ow = oracle.topk_softmax(lg, k)
    assert np.array_equal(idx, oi)
    assert np.abs(w - ow).max() <= W_TOL
    assert np.array_equal(cnt, oracle.histogram(oi, E))
    if k == 1:
        assert (w == 1.0).all()


def test_route_t0_zeroes_counts(m):
    cnt = torch.full((64,), 7, dtype=torch.int32, device=DEV)
    e = torch.empty(0, 4, dtype=torch.int32, device=DEV)
    m.moe_route(None, None, None, torch.empty(0, 64, device=DEV), True, e,
                torch.empty(0, 4, device=DEV), cnt)
    torch.cuda.synchronize()
    assert (np_(cnt) == 0).all()


@pytest.mark.parametrize("T,d,E,bias", [(77, 3584, 896, False), (130, 256, 40, True),
                                        (1, 3584, 896, True), (16, 3584, 896, False),
                                        (20, 512, 40, True), (64, 3584, 896, True),
                                        (33, 128, 17, False),
                                        # T >= 512 with d % 64 == 0 takes the tiled router:
                                        # ragged token and expert blocks, and d split into
                                        # 28, 8 and 4 partial sums (T=512, 1111, 2600)
                                        (600, 3584, 896, True), (512, 3584, 896, False),
                                        (1111, 256, 300, False), (2600, 128, 17, True)])
def test_router_scores_and_replay(m, T, d, E, bias):
    from synth import make_router, make_tokens
    cfg = LayerConfig("r", T=T, I=128, d=d, E=E, bias="normal" if bias else None)
    x = make_tokens(cfg)
    w_r, b = make_router(cfg)
    lg_ref = oracle.router_logits(x, w_r.numpy(), None if b is None else b.numpy())
    k = min(16, E)
    lg, idx, w, cnt = _route_gpu(m, np.zeros((T, E), np.float32), k, x=x.to(DEV),
                                 w_router=w_r.to(DEV), bias=None if b is None else b.to(DEV),
                                 given=False)
    assert (np.abs(lg - lg_ref) <= LOGIT_TOL * np.maximum(1, np.abs(lg_ref))).all()
    oi, ow = oracle.topk_softmax(lg, k)  # replay on the GPU's scores
    assert np.array_equal(idx, oi)
    assert np.abs(w - ow).max() <= W_TOL
    assert np.array_equal(cnt, oracle.histogram(oi, E))


# ---------------------------------------------------------------- permute
@pytest.mark.parametrize("T,E,k,e0,nl", [(0, 64, 4, 0, 64), (1, 896, 16, 0, 896),
                                         (7, 8, 2, 0, 8), (257, 896, 16, 0, 896),
                                         (1000, 64, 4, 16, 20), (5000, 896, 16, 0, 112),
                                         (700, 896, 16, 784, 112), (513, 32, 32, 0, 32),
                                         (200, 896, 16, 0, 896), (256, 64, 4, 8, 40),
                                         (256, 1100, 16, 0, 1100), (300, 2048, 32, 0, 2048),
                                         # 274 blocks: runs of 18 blocks per column
                                         # scan thread group, two load chunks each
                                         (70000, 64, 4, 8, 40)])
@pytest.mark.parametrize("with_counts", [True, False])
def test_permute_bitexact(m, T, E, k, e0, nl, with_counts):
    rng = np.random.default_rng(T + E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    oi, _ = oracle.topk_softmax(lg, k) if T else (np.zeros((0, k), np.int32), None)
    cnt = oracle.histogram(oi, E) if T else np.zeros(E, np.int32)
    off = oracle.offsets(cnt, e0, nl)
    perm, inv = oracle.permute(oi, off, e0, nl) if T else (np.zeros(0, np.int32),
                                                          np.zeros((0, k), np.int32))
    g_off = torch.full((nl + 1,), -7, dtype=torch.int32, device=DEV)
    g_perm = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    g_inv = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    ws = m.alloc_workspace(m.moe_permute_workspace_size(T, nl), DEV)
    m.moe_permute(torch.from_numpy(oi).to(DEV),
                  torch.from_numpy(cnt).to(DEV) if with_counts else None, e0, nl, g_off,
                  g_perm, g_inv, ws, E=E)
    torch.cuda.synchronize()
    A = int(off[-1])
    assert np.array_equal(np_(g_off), off)
    assert np.array_equal(np_(g_perm)[:A], perm)
    assert (np_(g_perm)[A:] == -7).all()  # untouched beyond the local rows
    assert np.array_equal(np_(g_inv), inv)


# ---------------------------------------------------------------- grouped GEMM
def _experts(num_local, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    out = []
    for _ in range(num_local):
        c, s = quantize_mxfp4(torch.randn(N, K, generator=g) / np.sqrt(K))
        out.append((c, s))
    return torch.stack([c for c, _ in out]), torch.stack([s for _, s in out])


@pytest.mark.parametrize("mode", [1, 3, 4])
@pytest.mark.parametrize("act", [0, 1, 2])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_grouped_gemm_vs_definition(m, mode, act, out_dtype):
    rng = np.random.default_rng(act * 10 + mode)
    nl, N, K, T = 6, 192, 384, 90
    counts = np.array([0, 37, 1, 16, 70, 17], np.int32)  # empty, ragged, exact tiles
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    x = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16)
    a_rows = rng.integers(0, T, size=A).astype(np.int32)
    w1c, w1s = _experts(nl, N, K, 1)
    w2c, w2s = _experts(nl, N, K, 2) if act else (None, None)
    out = torch.full((A + 5, N), 7.0, dtype=out_dtype, device=DEV)
    ws = m.alloc_workspace(m.moe_grouped_gemm_workspace_size(nl, A, N, mode), DEV)
    m.moe_grouped_gemm_mxfp4(x.to(DEV), torch.from_numpy(a_rows).to(DEV), w1c.to(DEV),
                             w1s.to(DEV), None if w2c is None else w2c.to(DEV),
                             None if w2s is None else w2s.to(DEV),
                             torch.from_numpy(off).to(DEV), A, act, out, ws, mode=mode)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert (got[A:] == 7.0).all()  # rows past the last expert untouched
    xa = x.float().numpy().astype(np.float64)[a_rows]
    ref = np.zeros((A, N))
    for e in range(nl):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            continue
        g1 = xa[r0:r1] @ oracle.mxfp4_decode(w1c[e].numpy(), w1s[e].numpy()).astype(np.float64).T
        if act == 0:
            ref[r0:r1] = g1
        else:
            u = xa[r0:r1] @ oracle.mxfp4_decode(w2c[e].numpy(), w2s[e].numpy()).astype(np.float64).T
            ref[r0:r1] = ACTS[act](g1, u)
    tol = 4e-3 if out_dtype == torch.bfloat16 else 1e-5
    assert rel_l2(got[:A], ref) <= tol, rel_l2(got[:A], ref)
    if out_dtype == torch.bfloat16:
        # elementwise: bf16 keeps 8 significant bits, so rounding to nearest
        # moves a value by at most 2^-8 of itself (the GLU output is heavy
        # tailed, so a bound relative to its rms would not hold)
        assert bf16_rounding_ok(got[:A], ref)
    else:
        assert max_abs_rms(got[:A], ref) <= 1e-4


@pytest.mark.parametrize("mode", [1, 3, 4])
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("K", [128, 640])
def test_grouped_gemm_many_rows(m, mode, act, K):
    """Experts with more rows than one tile (300, 513, 256, 257 rows), an
    empty and a single-row expert, one of 200 rows, a column count that is not
    a tile multiple, and the shortest contraction (one 128-wide chunk). With
    256-row tiles the groups hold 1, 128, 129, 150, 171, 200 and 256 rows:
    every count of active 32-row tiles but 2 and 3, and both ways of sharing a
    fifth or sixth row tile between the waves."""
    rng = np.random.default_rng(K + act + 7 * mode)
    nl, N, T = 7, 320, 700
    counts = np.array([300, 0, 513, 1, 256, 257, 200], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    x = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16)
    a_rows = rng.integers(0, T, size=A).astype(np.int32)
    w1c, w1s = _experts(nl, N, K, 3)
    w2c, w2s = _experts(nl, N, K, 4) if act else (None, None)
    out = torch.full((A + 3, N), 7.0, dtype=torch.float32, device=DEV)
    ws = m.alloc_workspace(m.moe_grouped_gemm_workspace_size(nl, A, N, mode), DEV)
    m.moe_grouped_gemm_mxfp4(x.to(DEV), torch.from_numpy(a_rows).to(DEV), w1c.to(DEV),
                             w1s.to(DEV), None if w2c is None else w2c.to(DEV),
                             None if w2s is None else w2s.to(DEV),
                             torch.from_numpy(off).to(DEV), A, act, out, ws, mode=mode)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[A:] == 7.0).all()
    xa = x.float().numpy().astype(np.float64)[a_rows]
    ref = np.zeros((A, N))
    for e in range(nl):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            continue
        g1 = xa[r0:r1] @ oracle.mxfp4_decode(w1c[e].numpy(), w1s[e].numpy()).astype(np.float64).T
        if act == 0:
            ref[r0:r1] = g1
        else:
            u = xa[r0:r1] @ oracle.mxfp4_decode(w2c[e].numpy(), w2s[e].numpy()).astype(np.float64).T
            ref[r0:r1] = ACTS[act](g1, u)
    assert rel_l2(got[:A], ref) <= 1e-5, rel_l2(got[:A], ref)
    assert max_abs_rms(got[:A], ref) <= 1e-4


@pytest.mark.parametrize("mode", [3, 4])
@pytest.mark.parametrize("K", [4096, 4224])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("act", [0, 1])
def test_grouped_gemm_long_contraction(m, mode, K, packed, act):
    """The longest contraction whose scales the 256-row schedule keeps in LDS
    beside its three load stages (4096), and one chunk past it, where that
    schedule stages its loads through registers instead."""
    rng = np.random.default_rng(K + mode)
    nl, N, T = 3, 128, 200
    counts = np.array([40, 0, 150], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    x = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16)
    a_rows = rng.integers(0, T, size=A).astype(np.int32)
    w1c, w1s = _experts(nl, N, K, 5)
    w2c, w2s = _experts(nl, N, K, 6)
    dev = [t.to(DEV) for t in (w1c, w1s, w2c, w2s)]
    if packed:
        dev = [*m.moe_mxfp4_prepack(dev[0], dev[1]), *m.moe_mxfp4_prepack(dev[2], dev[3])]
    if act == 0:
        dev[2:] = [None, None]
    out = torch.full((A + 3, N), 7.0, dtype=torch.float32, device=DEV)
    ws = m.alloc_workspace(m.moe_grouped_gemm_workspace_size(nl, A, N, mode), DEV)
    m.moe_grouped_gemm_mxfp4(x.to(DEV), torch.from_numpy(a_rows).to(DEV), *dev,
                             torch.from_numpy(off).to(DEV), A, act, out, ws, mode=mode,
                             w_layout=m.LAYOUT_PACKED if packed else m.LAYOUT_OCP)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[A:] == 7.0).all()
    xa = x.float().numpy().astype(np.float64)[a_rows]
    ref = np.zeros((A, N))
    for e in range(nl):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            continue
        g1 = xa[r0:r1] @ oracle.mxfp4_decode(w1c[e].numpy(), w1s[e].numpy()).astype(np.float64).T
        if act == 0:
            ref[r0:r1] = g1
            continue
        u = xa[r0:r1] @ oracle.mxfp4_decode(w2c[e].numpy(), w2s[e].numpy()).astype(np.float64).T
        ref[r0:r1] = ACTS[1](g1, u)
    assert rel_l2(got[:A], ref) <= 1e-5, rel_l2(got[:A], ref)
    assert max_abs_rms(got[:A], ref) <= 1e-4


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("y_dtype,out_dtype", [(torch.float32, torch.float32),
                                               (torch.float32, torch.bfloat16),
                                               (torch.bfloat16, torch.float32),
                                               (torch.bfloat16, torch.bfloat16)])
def test_combine_vs_oracle(m, y_dtype, out_dtype):
    rng = np.random.default_rng(3)
    T, k, d, R = 50, 16, 3584, 600
    y = torch.from_numpy(rng.standard_normal((R, d)).astype(np.float32)).to(y_dtype)
    inv = rng.integers(0, R, size=(T, k)).astype(np.int32)
    inv[rng.random((T, k)) < 0.3] = -1
    inv[7] = -1  # a token with no local assignment
    w = rng.random((T, k)).astype(np.float32)
    out = torch.empty(T, d, dtype=out_dtype, device=DEV)
    m.moe_combine(y.to(DEV), torch.from_numpy(inv).to(DEV), torch.from_numpy(w).to(DEV), out)
    torch.cuda.synchronize()
    ref = oracle.combine(y.float().numpy(), inv, w)
    got = out.float().cpu().numpy()
    assert (got[7] == 0).all()
    if out_dtype == torch.float32:
        assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()
    else:
        assert np.abs(got - ref).max() <= 2 ** -8 * np.abs(ref).max()


# ---------------------------------------------------------------- prepack
def _unpack_reference(pc, ps, n, N, K):
    """Inverse of the streaming layout, written from the layout's definition:
    codes [N/16][K/128][4][16][16], scales [N/16][ceil(K/512)][4][16][4]."""
    nch, nc4 = K // 128, (K // 128 + 3) // 4
    codes = pc.reshape(n, N // 16, nch, 4, 16, 16)           # rb, c, g, m, byte
    codes = codes.transpose(0, 1, 4, 2, 3, 5).reshape(n, N, K // 2)  # rb, m, c, g, byte
    sc = ps.reshape(n, N // 16, nc4, 4, 16, 4)               # rb, c4, g, m, cc
    sc = sc.transpose(0, 1, 4, 2, 5, 3).reshape(n, N, nc4 * 16)  # rb, m, c4, cc, g
    return codes, sc[:, :, : K // 32], sc[:, :, K // 32:]


@pytest.mark.parametrize("n,N,K", [(3, 48, 384), (2, 64, 1024), (1, 16, 128), (2, 1024, 3584)])
def test_prepack_is_a_permutation(m, n, N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, size=(n, N, K // 2), dtype=np.uint8)
    scales = rng.integers(2, 253, size=(n, N, K // 32), dtype=np.uint8)
    pc, ps = m.moe_mxfp4_prepack(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    torch.cuda.synchronize()
    c2, s2, pad = _unpack_reference(np_(pc), np_(ps), n, N, K)
    assert np.array_equal(c2, codes)
    assert np.array_equal(s2, scales)
    assert (pad == 0).all()


@pytest.mark.parametrize("mode", [1, 3, 4])
@pytest.mark.parametrize("act", [0, 1])
def test_grouped_gemm_packed_equals_canonical(m, mode, act):
    rng = np.random.default_rng(11 + act)
    nl, N, K, T = 5, 192, 384, 80
    counts = np.array([3, 0, 40, 17, 60], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    x = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    a_rows = torch.from_numpy(rng.integers(0, T, size=A).astype(np.int32)).to(DEV)
    w1c, w1s = [t.to(DEV) for t in _experts(nl, N, K, 3)]
    w2c, w2s = [t.to(DEV) for t in _experts(nl, N, K, 4)] if act else (None, None)
    offd = torch.from_numpy(off).to(DEV)
    ws = m.alloc_workspace(m.moe_grouped_gemm_workspace_size(nl, A, N, mode), DEV)
    outs = []
    for lay in (m.LAYOUT_OCP, m.LAYOUT_PACKED):
        if lay == m.LAYOUT_PACKED:
            p1c, p1s = m.moe_mxfp4_prepack(w1c, w1s)
            p2c, p2s = m.moe_mxfp4_prepack(w2c, w2s) if act else (None, None)
        else:
            p1c, p1s, p2c, p2s = w1c, w1s, w2c, w2s
        out = torch.empty(A, N, dtype=torch.float32, device=DEV)
        m.moe_grouped_gemm_mxfp4(x, a_rows, p1c, p1s, p2c, p2s, offd, A, act, out, ws, mode=mode,
                                 w_layout=lay)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
