"""GPU parity of the fused layer (moe_layer) against the oracle.

Small shapes: the whole oracle layer on all tokens, routing replayed on the
GPU's fp32 scores (routing arrays bit-exact) and the output within the layer
tolerance. Full-size workloads (the launch configuration the benchmark times):
routing of every token replayed bit-exactly, and the output of sampled tokens
(random, segment edges, hottest expert, no local expert) computed one by one
by the oracle."""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, LayerConfig, make_inputs
from tests.parity_util import (LOGIT_TOL, W_TOL, assert_close_layer, host_weights, np_,
                               oracle_rows, oracle_scores, run_gpu_layer, sample_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_routing(inp, g):
    """Replay the oracle's routing on the GPU's scores; compare bit for bit."""
    c = inp.cfg
    lg = np_(g["logits"])
    r_idx, r_w = oracle.topk_softmax(lg, c.k)
    assert np.array_equal(np_(g["idx"]), r_idx)
    assert np.abs(np_(g["w"]) - r_w).max() <= W_TOL
    return lg, r_idx, r_w


def _check_scores(inp, lg, rows=None):
    xb = inp.x if rows is None else inp.x[torch.as_tensor(rows, device=inp.x.device)]
    ref = oracle.router_logits(xb, np_(inp.w_router), None if inp.bias is None else np_(inp.bias))
    got = lg if rows is None else lg[rows]
    assert (np.abs(got - ref) <= LOGIT_TOL * np.maximum(1, np.abs(ref))).all()


SMALL = [
    LayerConfig("g0", T=37, I=128, d=256, E=64, k=8),
    LayerConfig("g1", T=300, I=256, d=384, E=16, k=4),
    LayerConfig("g2", T=50, I=128, d=256, E=40, k=6, expert_begin=8, num_local=20, bias="normal"),
    LayerConfig("g3", T=1, I=128, d=3584, E=896, k=16),
    LayerConfig("g4", T=129, I=256, d=512, E=8, k=8),  # k == E: every expert
    # T >= 512: the tiled router (split-K planes, bias, E not a tile multiple)
    LayerConfig("g5", T=700, I=128, d=256, E=100, k=6, bias="normal"),
    LayerConfig("g6", T=1030, I=256, d=384, E=40, k=4, expert_begin=4, num_local=30),
    # the largest expert count and top-k the ABI takes (E = 2048, k = 32), with
    # a local range, and at T >= 512 on the tiled router
    LayerConfig("g7", T=40, I=128, d=256, E=2048, k=32, expert_begin=1000, num_local=700),
    LayerConfig("g8", T=520, I=128, d=256, E=2048, k=32, bias="normal"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("mode", [0, 1, 3, 4])
def test_small_layer_vs_oracle(cfg, mode):
    inp = make_inputs(cfg)
    g = run_gpu_layer(inp.to(DEV), mode=mode)
    lg, _, _ = _check_routing(inp, g)
    _check_scores(inp, lg)
    ref = oracle.layer(inp.x, np_(inp.w_router), None if inp.bias is None else np_(inp.bias),
                       host_weights(inp.weights), E=cfg.E, k=cfg.k, I=cfg.I,
                       e0=cfg.expert_begin, n_local=cfg.num_local, logits=lg)
    assert_close_layer(g["out"].float().cpu().numpy(), ref["out"], cfg.name)


@pytest.mark.parametrize("act", [1, 2])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_layer_act_and_dtype(act, out_dtype):
    cfg = SMALL[0]
    inp = make_inputs(cfg)
    g = run_gpu_layer(inp.to(DEV), out_dtype=out_dtype, act=act)
    lg, _, _ = _check_routing(inp, g)
    ref = oracle.layer(inp.x, np_(inp.w_router), None, host_weights(inp.weights), E=cfg.E,
                       k=cfg.k, I=cfg.I, logits=lg, act=act)
    assert_close_layer(g["out"].float().cpu().numpy(), ref["out"], f"act={act}")


@pytest.fixture(scope="module")
def tiny():
    return make_inputs(CONFIGS["tiny"])


def test_tiny_workload_full_oracle(tiny):
    cfg = tiny.cfg
    g = run_gpu_layer(tiny.to(DEV))
    lg, _, _ = _check_routing(tiny, g)
    _check_scores(tiny, lg)
    ref = oracle.layer(tiny.x, np_(tiny.w_router), None, host_weights(tiny.weights), E=cfg.E,
                       k=cfg.k, I=cfg.I, logits=lg)
    assert ref["A"] == cfg.T * cfg.k
    assert_close_layer(g["out"].float().cpu().numpy(), ref["out"], "tiny")


@pytest.mark.parametrize("cfg", [SMALL[0], SMALL[1], SMALL[2], SMALL[5]], ids=lambda c: c.name)
@pytest.mark.parametrize("mode", [1, 3, 4])
def test_packed_layout_layer_bitwise(cfg, mode):
    import mxfp4_expert_top_amd as m
    inp = make_inputs(cfg).to(DEV)
    a = run_gpu_layer(inp, mode=mode)
    b = run_gpu_layer(inp, mode=mode, packed=m.prepack_weights(inp.weights))
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("mode", [0, 1, 3, 4])
def test_determinism_bitwise(tiny, mode):
    """No atomics on any value path: two runs agree bit for bit on every
    schedule (the 256-row one with its direct-to-LDS loads included)."""
    gi = tiny.to(DEV)
    a = run_gpu_layer(gi, mode=mode)
    b = run_gpu_layer(gi, mode=mode)
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("mode", [3, 4])
def test_determinism_bitwise_many_rows(mode):
    """The same at a size whose experts hold several 32-row tiles (and,
    T >= 512, the tiled router's split-K planes)."""
    gi = make_inputs(SMALL[6]).to(DEV)
    a = run_gpu_layer(gi, mode=mode)
    b = run_gpu_layer(gi, mode=mode)
    for key in a:
        assert torch.equal(a[key], b[key]), key


# ---------------------------------------------------------------- full sizes
def _check_dispatch(inp, lg, r_idx):
    """The dispatch arrays on every token at full size: moe_route on the
    layer's own fp32 scores (given, not recomputed) and moe_permute -- the
    layer's bitmap counting path, and the path fed the top-k kernel's
    histogram -- against the oracle's histogram, offsets and permutation of
    the replayed routing, bit for bit."""
    import mxfp4_expert_top_amd as m
    c = inp.cfg
    T, k, E = c.T, c.k, c.E
    logits = torch.from_numpy(lg).to(DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    m.moe_route(None, None, None, logits, 1, idx, w, counts)
    torch.cuda.synchronize()
    assert np.array_equal(np_(idx), r_idx)
    r_cnt = oracle.histogram(r_idx, E)
    assert np.array_equal(np_(counts), r_cnt)
    r_off = oracle.offsets(r_cnt, c.expert_begin, c.num_local)
    r_perm, r_inv = oracle.permute(r_idx, r_off, c.expert_begin, c.num_local)
    A = int(r_off[-1])
    ws = m.alloc_workspace(m.moe_permute_workspace_size(T, c.num_local), DEV)
    for cnt in (None, counts):
        off = torch.full((c.num_local + 1,), -7, dtype=torch.int32, device=DEV)
        perm = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
        inv = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
        m.moe_permute(idx, cnt, c.expert_begin, c.num_local, off, perm, inv, ws, E=E)
        torch.cuda.synchronize()
        assert np.array_equal(np_(off), r_off)
        assert np.array_equal(np_(perm)[:A], r_perm[:A])
        assert np.array_equal(np_(inv), r_inv)
    return r_cnt, A


@pytest.mark.parametrize("name", ["decode", "prefill", "ep_share", "long_skewed_prefill"])
def test_full_size_workload(name):
    """The benchmark's launch configuration: weights converted to the streaming
    layout at load, schedule chosen automatically, fp32 output. Routing and
    dispatch arrays on every token; the output on 64 sampled tokens (segment
    edges, the hottest expert, a token with no local expert, seeded random)
    evaluated one by one by the oracle. The bf16 output is then checked, on
    every token, to be exactly the fp32 output rounded to nearest-even: the
    only difference between the two is that final rounding, which on its own
    reaches about 0.024 rms on heavy-tailed rows, most of the 3e-2 rms
    max-abs budget."""
    import mxfp4_expert_top_amd as m
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, DEV)
    packed = m.prepack_weights(inp.weights)
    g = run_gpu_layer(inp, packed=packed, out_dtype=torch.float32)
    lg, r_idx, _ = _check_routing(inp, g)
    # the scores of every token against the oracle's own router product
    ref = oracle_scores(inp.x, np_(inp.w_router), None if inp.bias is None else np_(inp.bias))
    err = np.abs(lg - ref) / np.maximum(1, np.abs(ref))
    assert err.max() <= LOGIT_TOL, (name, float(err.max()))
    print(f"{name}: router scores of all {cfg.T} tokens within {err.max():.2e} max(1, |l|)")
    _, A = _check_dispatch(inp, lg, r_idx)
    assert A > 0
    toks = sample_tokens(cfg, r_idx, 64)
    assert len(toks) == min(64, cfg.T)
    ref = oracle_rows(inp, r_idx, np_(g["w"]), toks)
    got = g["out"].float().cpu().numpy()[toks]
    assert_close_layer(got, ref, name)
    # rows with no local expert are exact zeros
    loc = r_idx - cfg.expert_begin
    none = ~((loc >= 0) & (loc < cfg.num_local)).any(1)
    if none.any():
        assert (g["out"][torch.as_tensor(np.nonzero(none)[0], device=DEV)] == 0).all()
    b = run_gpu_layer(inp, packed=packed, out_dtype=torch.bfloat16)
    assert torch.equal(b["idx"], g["idx"])
    assert torch.equal(b["out"], g["out"].to(torch.bfloat16))
    del inp, g, b, packed
    torch.cuda.empty_cache()
