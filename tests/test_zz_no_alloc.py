"""moe_layer_noalloc, the layer entry for callers that cannot allocate (its
scratch is the library's static per-GPU array), against moe_layer on the
same inputs through the C ABI: two calls in a row, the second with a smaller
batch over a local expert range, each bitwise equal to moe_layer's output and
routing (the same kernels, which are deterministic)."""

import pytest
import torch

import mxfp4_expert_top_amd as m
from synth import LayerConfig, make_inputs
from tests.parity_util import run_gpu_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_noalloc(inp, packed, out_dtype, precision=m.PREC_BF16, mode=m.MODE_AUTO):
    c = inp.cfg
    p = m.layer_params(c.T, c.d, c.E, c.k, c.I, c.expert_begin, c.num_local,
                       out_dtype=m.DT_F32 if out_dtype == torch.float32 else m.DT_BF16,
                       mode=mode, weight_layout=m.LAYOUT_PACKED, precision=precision)
    assert m.moe_layer_workspace_size(p) <= m.NOALLOC_SCRATCH_BYTES
    out = torch.empty(c.T, c.d, dtype=out_dtype, device=DEV)
    logits = torch.empty(c.T, c.E, dtype=torch.float32, device=DEV)
    idx = torch.empty(c.T, c.k, dtype=torch.int32, device=DEV)
    w = torch.empty(c.T, c.k, dtype=torch.float32, device=DEV)
    m.moe_layer_noalloc(p, inp.x, inp.w_router, inp.bias, packed, out, logits, idx, w)
    torch.cuda.synchronize()
    return dict(out=out, logits=logits, idx=idx, w=w)


@pytest.mark.parametrize("first,second", [
    # full width, 896 experts, top-16: 200 tokens (the small-batch tiled
    # router), then 24 (the skinny router) with experts 100..399 local
    (LayerConfig("na0", T=200, I=256), LayerConfig("na1", T=24, I=256, expert_begin=100,
                                                   num_local=300, bias="normal")),
], ids=["200-then-24"])
def test_noalloc_equals_moe_layer_two_calls(first, second):
    for cfg, dt in ((first, torch.bfloat16), (second, torch.float32)):
        inp = make_inputs(cfg, DEV)
        packed = m.prepack_weights(inp.weights)
        a = _run_noalloc(inp, packed, dt)
        b = run_gpu_layer(inp, packed=packed, out_dtype=dt)
        for key in ("idx", "w", "logits", "out"):
            assert torch.equal(a[key], b[key]), (cfg.name, key)
        assert bool((a["out"] != 0).any())
        del inp, packed, a, b
        torch.cuda.empty_cache()


def test_noalloc_fp6x2_two_calls():
    """The FP6X2 layer through the same entry: 128 tokens on 128-row tiles,
    then 64 tokens on 256-row tiles over a local expert range, each bitwise
    equal to moe_layer's output and routing."""
    calls = ((LayerConfig("nf0", T=128, I=256), m.MODE_TILE128, torch.float32),
             (LayerConfig("nf1", T=64, I=256, expert_begin=100, num_local=300, bias="normal"),
              m.MODE_TILE256, torch.bfloat16))
    for cfg, mode, dt in calls:
        inp = make_inputs(cfg, DEV)
        packed = m.prepack_weights(inp.weights)
        a = _run_noalloc(inp, packed, dt, precision=m.PREC_FP6X2, mode=mode)
        b = run_gpu_layer(inp, packed=packed, out_dtype=dt, precision=m.PREC_FP6X2, mode=mode)
        for key in ("idx", "w", "logits", "out"):
            assert torch.equal(a[key], b[key]), (cfg.name, key)
        assert bool((a["out"] != 0).any())
        del inp, packed, a, b
        torch.cuda.empty_cache()
