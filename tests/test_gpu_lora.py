"""GPU parity of LoRA on the MXFP4 base: the grouped low-rank increment
against its definition, and the LoRA layer against the oracle's LoRA layer
(routing replayed on the GPU's scores)."""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, LayerConfig, make_inputs, make_lora
from tests.parity_util import (assert_close_layer, host_weights, np_, oracle_rows, rel_l2,
                               run_gpu_layer, sample_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import mxfp4_expert_top_amd as mod
    return mod


@pytest.mark.parametrize("rank", [1, 16, 24, 64])
@pytest.mark.parametrize("gather", [True, False])
@pytest.mark.parametrize("K,N", [(64, 128), (3584, 1024), (1024, 3584)])
def test_grouped_lora_vs_definition(m, rank, gather, K, N):
    """Experts with 0, 37, 1, 130 and 64 rows; rows past the last expert's
    end are left as they were."""
    rng = np.random.default_rng(rank + K + 7 * gather)
    nl, T = 5, 300
    counts = np.array([0, 37, 1, 130, 64], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    rows = T if gather else A
    x = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16)
    x_rows = rng.integers(0, T, size=A).astype(np.int32) if gather else None
    la = torch.from_numpy(rng.standard_normal((nl, rank, K)).astype(np.float32) / np.sqrt(K))
    lb = torch.from_numpy(rng.standard_normal((nl, N, rank)).astype(np.float32) / np.sqrt(rank))
    la, lb = la.to(torch.bfloat16), lb.to(torch.bfloat16)
    y0 = rng.standard_normal((A + 3, N)).astype(np.float32)
    y = torch.from_numpy(y0).to(DEV)
    ws = m.alloc_workspace(m.moe_grouped_lora_workspace_size(A, rank), DEV)
    scale = 0.75
    m.moe_grouped_lora(x.to(DEV), None if x_rows is None else torch.from_numpy(x_rows).to(DEV),
                       la.to(DEV), lb.to(DEV), scale, torch.from_numpy(off).to(DEV), A, y, ws)
    torch.cuda.synchronize()
    got = np_(y).astype(np.float64)
    assert np.array_equal(got[A:], y0[A:])
    xf = x.float().numpy().astype(np.float64)
    xa = xf[x_rows] if gather else xf
    laf, lbf = la.float().numpy().astype(np.float64), lb.float().numpy().astype(np.float64)
    for e in range(nl):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            continue
        t = scale * xa[r0:r1] @ laf[e].T
        delta = t @ lbf[e].T
        d_got = got[r0:r1] - y0[r0:r1]
        # fp32 sums of K and rank terms, and the fp32 add to y
        bound = 1e-5 * (np.abs(scale * xa[r0:r1]) @ np.abs(laf[e]).T) @ np.abs(lbf[e]).T \
            + 2.0 ** -23 * np.abs(y0[r0:r1] + delta)
        assert (np.abs(d_got - delta) <= bound + 1e-30).all(), np.abs(d_got - delta).max()


def run_gpu_lora_layer(m, inp, lora, rank, scale, mode=0, out_dtype=torch.bfloat16, act=1,
                       packed=None):
    """``packed``: the weights converted to the streaming layout (else the
    canonical ones in ``inp``)."""
    c = inp.cfg
    p = m.layer_params(c.T, c.d, c.E, c.k, c.I, c.expert_begin, c.num_local, act=act,
                       out_dtype=m.DT_F32 if out_dtype == torch.float32 else m.DT_BF16, mode=mode,
                       weight_layout=m.LAYOUT_OCP if packed is None else m.LAYOUT_PACKED)
    ws = m.alloc_workspace(m.moe_layer_lora_workspace_size(p, rank), DEV)
    out = torch.empty(c.T, c.d, dtype=out_dtype, device=DEV)
    logits = torch.empty(c.T, c.E, dtype=torch.float32, device=DEV)
    idx = torch.empty(c.T, c.k, dtype=torch.int32, device=DEV)
    w = torch.empty(c.T, c.k, dtype=torch.float32, device=DEV)
    m.moe_layer_lora(p, lora, rank, scale, inp.x, inp.w_router, inp.bias,
                     inp.weights if packed is None else packed, out, ws, logits, idx, w)
    torch.cuda.synchronize()
    return dict(out=out, logits=logits, idx=idx, w=w)


SMALL = [
    LayerConfig("r0", T=37, I=128, d=256, E=64, k=8),
    LayerConfig("r1", T=300, I=256, d=384, E=16, k=4),
    LayerConfig("r2", T=50, I=128, d=256, E=40, k=6, expert_begin=8, num_local=20, bias="normal"),
    LayerConfig("r3", T=700, I=128, d=256, E=100, k=6, bias="normal"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("mode", [0, 1, 3, 4])
@pytest.mark.parametrize("rank", [8, 16, 32])
def test_small_lora_layer_vs_oracle(m, cfg, mode, rank):
    """Ranks 16 and 32 add the increment inside the GEMMs (every schedule);
    rank 8 takes the unfused path."""
    inp = make_inputs(cfg).to(DEV)
    lora = {k: v.to(DEV) for k, v in make_lora(cfg, rank).items()}
    g = run_gpu_lora_layer(m, inp, lora, rank, 0.5, mode=mode)
    lg = np_(g["logits"])
    r_idx, _ = oracle.topk_softmax(lg, cfg.k)
    assert np.array_equal(np_(g["idx"]), r_idx)
    ref = oracle.layer_lora(inp.x, np_(inp.w_router), None if inp.bias is None else np_(inp.bias),
                            host_weights(inp.weights), {k: v.cpu() for k, v in lora.items()},
                            E=cfg.E, k=cfg.k, I=cfg.I, rank=rank, scale=0.5,
                            e0=cfg.expert_begin, n_local=cfg.num_local, logits=lg)
    assert_close_layer(g["out"].float().cpu().numpy(), ref["out"], cfg.name)


@pytest.mark.parametrize("cfg", SMALL[1:4:2], ids=lambda c: c.name)
@pytest.mark.parametrize("mode", [3, 4])
@pytest.mark.parametrize("rank", [48, 64])
def test_wide_rank_lora_layer_vs_oracle(m, cfg, mode, rank):
    """Rank 48 takes three 32-column tiles for gate and up together; rank 64
    takes one rank-factor pass per adapter."""
    test_small_lora_layer_vs_oracle(m, cfg, mode, rank)


def test_tiny_workload_lora_full_oracle(m):
    """The full-width tiny workload (d = 3584, 896 experts, top-16, I = 128)
    with rank-16 adapters on all 896 experts, increment inside the GEMMs."""
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg).to(DEV)
    lora = {k: v.to(DEV) for k, v in make_lora(cfg, 16).items()}
    g = run_gpu_lora_layer(m, inp, lora, 16, 0.5, mode=4)
    lg = np_(g["logits"])
    ref = oracle.layer_lora(inp.x, np_(inp.w_router), None, host_weights(inp.weights),
                            {k: v.cpu() for k, v in lora.items()}, E=cfg.E, k=cfg.k, I=cfg.I,
                            rank=16, scale=0.5, logits=lg)
    assert_close_layer(g["out"].float().cpu().numpy(), ref["out"], "tiny lora")


@pytest.mark.parametrize("mode,rank", [(1, 8), (4, 8), (1, 16), (3, 16), (4, 16)])
def test_zero_increment_is_the_base_layer(m, mode, rank):
    """Zero B factors: the LoRA layer, unfused (rank 8) or with the increment
    inside the GEMMs (rank 16, streaming or tiled), gives moe_layer's output
    to fp32 rounding of the same sums."""
    cfg = SMALL[1]
    inp = make_inputs(cfg).to(DEV)
    lora = {k: v.to(DEV) for k, v in make_lora(cfg, rank).items()}
    for n in ("gate_b", "up_b", "down_b"):
        lora[n].zero_()
    a = run_gpu_lora_layer(m, inp, lora, rank, 0.5, mode=mode, out_dtype=torch.float32)
    b = run_gpu_layer(inp, mode=mode, out_dtype=torch.float32)
    assert torch.equal(a["idx"], b["idx"])
    assert rel_l2(np_(a["out"]), np_(b["out"])) <= 1e-6


@pytest.mark.parametrize("mode", [1, 3, 4])
@pytest.mark.parametrize("rank", [16, 64])
def test_lora_layer_packed_equals_canonical(m, mode, rank):
    """The benchmark's launch configuration: weights in the streaming layout.
    The layout only permutes bytes, so the LoRA layer's output is bitwise the
    canonical layout's, on every schedule."""
    cfg = SMALL[1]
    inp = make_inputs(cfg).to(DEV)
    lora = {k: v.to(DEV) for k, v in make_lora(cfg, rank).items()}
    a = run_gpu_lora_layer(m, inp, lora, rank, 0.5, mode=mode)
    b = run_gpu_lora_layer(m, inp, lora, rank, 0.5, mode=mode,
                           packed=m.prepack_weights(inp.weights))
    assert torch.equal(a["idx"], b["idx"])
    assert torch.equal(a["out"], b["out"])


@pytest.mark.parametrize("name", ["decode", "prefill"])
@pytest.mark.parametrize("rank", [16, 64])
def test_full_size_lora_layer(m, name, rank):
    """The benchmark's launch configuration with adapters (streaming-layout
    weights, schedule chosen automatically, the increment inside the GEMMs,
    fp32 output):
    routing replayed on every token, and 48 sampled tokens' rows (segment
    edges, the hottest expert's segment, seeded random) against the oracle's
    LoRA layer evaluated token by token."""
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, DEV)
    lora = make_lora(cfg, rank, DEV)
    g = run_gpu_lora_layer(m, inp, lora, rank, 0.5, packed=m.prepack_weights(inp.weights),
                           out_dtype=torch.float32)
    lg = np_(g["logits"])
    r_idx, _ = oracle.topk_softmax(lg, cfg.k)
    assert np.array_equal(np_(g["idx"]), r_idx)
    toks = sample_tokens(cfg, r_idx, 48, seed=2)
    ref = oracle_rows(inp, r_idx, np_(g["w"]), toks, lora=lora, rank=rank, scale=0.5)
    assert_close_layer(g["out"].float().cpu().numpy()[toks], ref, f"{name} rank {rank}")
    del inp, g, lora
    torch.cuda.empty_cache()
