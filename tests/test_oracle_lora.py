"""Pins of the oracle's LoRA layer (a low-rank increment B A on each frozen
MXFP4 expert projection, P1 "从Kimi K3到MiniMax-H3" section 二, 第五层):
zero B factors reproduce the base layer bit for bit, and the layer matches a
dense fp64 evaluation that folds W + scale * B A into each expert's weights
and shares none of the oracle's code."""

import numpy as np
import pytest
import torch

import oracle
from synth import LayerConfig, make_inputs, make_lora
from tests.dense_ref import ACTS, decode_bitfield, dense_gate_matrix, max_abs_over_rms, rel_l2

CFGS = [
    LayerConfig("l0", T=7, I=32, d=64, E=8, k=2),
    LayerConfig("l1", T=13, I=64, d=96, E=16, k=4, bias="normal"),
    LayerConfig("l2", T=9, I=32, d=64, E=12, k=3, expert_begin=4, num_local=5),
]


def _np(w):
    return {k: v.numpy() for k, v in w.items()}


def _run(inp, lora, rank, scale, act=oracle.ACT_SILU_MUL):
    c = inp.cfg
    return oracle.layer_lora(inp.x, inp.w_router.numpy(),
                             None if inp.bias is None else inp.bias.numpy(), _np(inp.weights),
                             lora, E=c.E, k=c.k, I=c.I, rank=rank, scale=scale,
                             e0=c.expert_begin, n_local=c.num_local, act=act)


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_zero_b_is_the_base_layer_bitwise(cfg):
    inp = make_inputs(cfg)
    lora = make_lora(cfg, 8)
    for n in ("gate_b", "up_b", "down_b"):
        lora[n] = torch.zeros_like(lora[n])
    r = _run(inp, lora, 8, 0.75)
    base = oracle.layer(inp.x, inp.w_router.numpy(),
                        None if inp.bias is None else inp.bias.numpy(), _np(inp.weights),
                        E=cfg.E, k=cfg.k, I=cfg.I, e0=cfg.expert_begin, n_local=cfg.num_local)
    assert np.array_equal(r["out"], base["out"])
    assert np.array_equal(r["idx"], base["idx"])


def dense_lora_layer(x, idx, w, wts, lora, *, E, e0, n_local, scale, act=1):
    """Every local expert on every token in fp64 with W + scale * B A."""
    x = np.asarray(x, np.float64)
    G = dense_gate_matrix(idx, w, E)
    out = np.zeros(x.shape, np.float64)
    f = ACTS[act]
    L = {k: v.float().numpy().astype(np.float64) for k, v in lora.items()}
    for le in range(n_local):
        wg = decode_bitfield(wts["gate_codes"][le], wts["gate_scales"][le]) + scale * L["gate_b"][le] @ L["gate_a"][le]
        wu = decode_bitfield(wts["up_codes"][le], wts["up_scales"][le]) + scale * L["up_b"][le] @ L["up_a"][le]
        wd = decode_bitfield(wts["down_codes"][le], wts["down_scales"][le]) + scale * L["down_b"][le] @ L["down_a"][le]
        h = f(x @ wg.T, x @ wu.T)
        out += G[:, e0 + le:e0 + le + 1] * (h @ wd.T)
    return out


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
@pytest.mark.parametrize("rank", [1, 8, 32])
def test_lora_layer_vs_dense(cfg, rank):
    inp = make_inputs(cfg)
    lora = make_lora(cfg, rank)
    scale = 0.5
    r = _run(inp, lora, rank, scale)
    ref = dense_lora_layer(inp.x.float().numpy(), r["idx"], r["w"], _np(inp.weights), lora,
                           E=cfg.E, e0=cfg.expert_begin, n_local=cfg.num_local, scale=scale)
    assert rel_l2(r["out"], ref) <= 1e-5
    assert max_abs_over_rms(r["out"], ref) <= 1e-4
    # the increment is really there
    base = dense_lora_layer(inp.x.float().numpy(), r["idx"], r["w"], _np(inp.weights), lora,
                            E=cfg.E, e0=cfg.expert_begin, n_local=cfg.num_local, scale=0.0)
    assert rel_l2(r["out"], base) > 1e-2


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_token_rows_lora_vs_dense(cfg):
    """The per-token form (used at workload sizes, where the whole LoRA
    layer is too slow) against the same dense fp64 evaluation, and equal to
    the whole layer's rows: the same sums per token, in the same order."""
    rank, scale = 8, 0.5
    inp = make_inputs(cfg)
    lora = make_lora(cfg, rank)
    r = _run(inp, lora, rank, scale)
    toks = sorted({0, cfg.T // 2, cfg.T - 1})
    rows = oracle.token_rows_lora(inp.x, r["idx"], r["w"], toks, _np(inp.weights), lora, I=cfg.I,
                                  rank=rank, scale=scale, e0=cfg.expert_begin,
                                  n_local=cfg.num_local)
    ref = dense_lora_layer(inp.x.float().numpy(), r["idx"], r["w"], _np(inp.weights), lora,
                           E=cfg.E, e0=cfg.expert_begin, n_local=cfg.num_local, scale=scale)
    assert rel_l2(rows, ref[toks]) <= 1e-5
    assert max_abs_over_rms(rows, ref[toks]) <= 1e-4
    assert np.array_equal(rows, r["out"][toks])
