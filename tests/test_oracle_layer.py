"""Pins of the oracle's whole layer (dispatch -> expert compute -> combine)
against evaluations that share none of its code: a dense, gate-matrix
weighted fp64 evaluation of every expert, a textbook dense MLP for E=1, k=1,
and the closed form of all-ones weights."""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, LayerConfig, make_inputs
from tests.dense_ref import decode_bitfield, dense_masked_layer, max_abs_over_rms, rel_l2, silu


def _np_weights(inp):
    return {k: v.numpy() for k, v in inp.weights.items()}


def _run_oracle(inp, act=oracle.ACT_SILU_MUL):
    c = inp.cfg
    return oracle.layer(inp.x, inp.w_router.numpy(),
                        None if inp.bias is None else inp.bias.numpy(),
                        _np_weights(inp), E=c.E, k=c.k, I=c.I, e0=c.expert_begin,
                        n_local=c.num_local, act=act)


SMALL = [
    LayerConfig("s0", T=7, I=32, d=64, E=8, k=2),
    LayerConfig("s1", T=13, I=64, d=96, E=16, k=4, bias="normal"),
    LayerConfig("s2", T=9, I=32, d=64, E=12, k=3, expert_begin=4, num_local=5),
    LayerConfig("s3", T=1, I=32, d=32, E=4, k=4),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("act", [oracle.ACT_SILU_MUL, oracle.ACT_GELU_TANH_MUL])
def test_layer_vs_dense_masked_fp64(cfg, act):
    inp = make_inputs(cfg)
    r = _run_oracle(inp, act)
    ref = dense_masked_layer(inp.x.float().numpy(), r["idx"], r["w"], _np_weights(inp),
                             E=cfg.E, e0=cfg.expert_begin, n_local=cfg.num_local, act=act)
    assert rel_l2(r["out"], ref) <= 1e-5
    assert max_abs_over_rms(r["out"], ref) <= 1e-4
    # routing replayed from the same logits gives the same routing
    idx2, w2 = oracle.topk_softmax(r["logits"], cfg.k)
    assert np.array_equal(idx2, r["idx"]) and np.array_equal(w2, r["w"])


def test_e1_k1_is_a_dense_mlp():
    cfg = LayerConfig("mlp", T=6, I=64, d=128, E=1, k=1)
    inp = make_inputs(cfg)
    r = _run_oracle(inp)
    assert (r["w"] == 1.0).all() and (r["idx"] == 0).all()
    wt = _np_weights(inp)
    wg = torch.from_numpy(decode_bitfield(wt["gate_codes"][0], wt["gate_scales"][0])).float()
    wu = torch.from_numpy(decode_bitfield(wt["up_codes"][0], wt["up_scales"][0])).float()
    wd = torch.from_numpy(decode_bitfield(wt["down_codes"][0], wt["down_scales"][0])).float()
    x = inp.x.float()
    ref = torch.matmul(torch.nn.functional.silu(torch.matmul(x, wg.T)) * torch.matmul(x, wu.T), wd.T)
    assert rel_l2(r["out"], ref.numpy()) <= 1e-5


def test_all_ones_weights_closed_form():
    cfg = LayerConfig("ones", T=5, I=64, d=64, E=6, k=3)
    inp = make_inputs(cfg)
    rng = np.random.default_rng(4)
    xv = rng.integers(-1, 2, size=(cfg.T, cfg.d)).astype(np.float32) / 8  # exact sums
    inp.x = torch.from_numpy(xv).to(torch.bfloat16)
    for name, t in inp.weights.items():
        t.fill_(127 if name.endswith("scales") else 0x22)  # every weight = 1.0
    r = _run_oracle(inp)
    S = xv.astype(np.float64).sum(1)
    want = cfg.I * S * silu(S)
    got = r["out"].astype(np.float64)
    assert np.allclose(got, want[:, None] * r["w"].astype(np.float64).sum(1)[:, None],
                       rtol=2e-6, atol=1e-6)
    assert np.allclose(got, want[:, None], rtol=4e-6, atol=1e-6)


def test_token_rows_equal_layer_rows_bitwise():
    cfg = SMALL[2]
    inp = make_inputs(cfg)
    r = _run_oracle(inp)
    toks = [0, 3, 8, 5]
    rows = oracle.token_rows(inp.x, r["idx"], r["w"], toks, _np_weights(inp), I=cfg.I,
                             e0=cfg.expert_begin, n_local=cfg.num_local)
    assert np.array_equal(rows, r["out"][toks])


def test_injected_logits_replay():
    cfg = SMALL[0]
    inp = make_inputs(cfg)
    lg = np.zeros((cfg.T, cfg.E), np.float32)
    lg[:, 5] = 1.0
    lg[:, 2] = 1.0  # tie between experts 2 and 5 -> 2 first
    r = oracle.layer(inp.x, inp.w_router.numpy(), None, _np_weights(inp), E=cfg.E,
                     k=cfg.k, I=cfg.I, logits=lg)
    assert (r["idx"][:, 0] == 2).all() and (r["idx"][:, 1] == 5).all()
    assert (r["w"] == 0.5).all()


@pytest.fixture(scope="module")
def tiny_inputs():
    return make_inputs(CONFIGS["tiny"])


def test_tiny_config_vs_dense_masked_fp64(tiny_inputs):
    """The full-width tiny workload (T=8, d=3584, 896 experts, top-16, I=128):
    the oracle against the dense fp64 evaluation over every expert that any
    token selected (the gate matrix is zero for the rest)."""
    inp = tiny_inputs
    cfg = inp.cfg
    r = _run_oracle(inp)
    assert r["A"] == cfg.T * cfg.k
    used = np.unique(r["idx"])
    wt = _np_weights(inp)
    sub = {k: v[used] for k, v in wt.items()}
    remap = np.searchsorted(used, r["idx"]).astype(np.int32)
    ref = dense_masked_layer(inp.x.float().numpy(), remap, r["w"], sub, E=len(used))
    assert rel_l2(r["out"], ref) <= 1e-5
    assert max_abs_over_rms(r["out"], ref) <= 1e-4
    # logits against an fp64 product
    ref_l = inp.x.float().numpy().astype(np.float64) @ inp.w_router.numpy().astype(np.float64).T
    assert np.abs(r["logits"] - ref_l).max() <= 1e-4


@pytest.mark.parametrize("cfg", SMALL[:3], ids=lambda c: c.name)
def test_expert_compute_vs_dense_fp64(cfg):
    """The grouped expert step on its own: for every permuted row, h and y
    against an fp64 evaluation of that row's expert from the bit-field
    decode, and combine(y) gives the layer's output bit for bit."""
    inp = make_inputs(cfg)
    r = _run_oracle(inp)
    wts = _np_weights(inp)
    h, y = oracle.expert_compute(inp.x, cfg.I, r["off"], r["perm"], wts)
    assert h.shape == (r["A"], cfg.I) and y.shape == (r["A"], cfg.d)
    x = inp.x.float().numpy().astype(np.float64)
    for le in range(cfg.num_local):
        a, b = r["off"][le], r["off"][le + 1]
        if a == b:
            continue
        wg = decode_bitfield(wts["gate_codes"][le], wts["gate_scales"][le])
        wu = decode_bitfield(wts["up_codes"][le], wts["up_scales"][le])
        wd = decode_bitfield(wts["down_codes"][le], wts["down_scales"][le])
        xe = x[r["perm"][a:b]]
        g, u = xe @ wg.T, xe @ wu.T
        hr = silu(g) * u
        yr = hr @ wd.T
        assert rel_l2(h[a:b], hr) <= 1e-5 and rel_l2(y[a:b], yr) <= 1e-5
    assert np.array_equal(oracle.combine(y, r["inv"], r["w"]), r["out"])
