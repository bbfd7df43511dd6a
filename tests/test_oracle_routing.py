"""Pins of the oracle's routing and dispatch: router scores against an fp64
product, top-k against a brute-force sort, softmax closed forms, and the
permutation's invariants."""

import numpy as np
import pytest
import torch

import oracle


def _brute_topk(l, k):
    # order: larger score first, equal scores by lower expert id; -0 == +0
    return sorted(range(len(l)), key=lambda e: (-float(l[e]) + 0.0, e))[:k]


def test_router_logits_vs_fp64():
    rng = np.random.default_rng(0)
    T, d, E = 5, 256, 40
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    w = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_logits(x, w, b)
    xf = x.float().numpy().astype(np.float64)
    want = xf @ w.astype(np.float64).T + b
    bound = 1e-6 * (np.abs(xf) @ np.abs(w.astype(np.float64)).T + np.abs(b)) + 1e-7
    assert (np.abs(got - want) <= bound).all()
    got_nb = oracle.router_logits(x, w, None)
    assert np.allclose(got_nb + b.astype(np.float32), got, rtol=0, atol=1e-5)


@pytest.mark.parametrize("E,k", [(896, 16), (64, 8), (17, 1), (12, 12)])
def test_topk_matches_sort(E, k):
    rng = np.random.default_rng(E * 31 + k)
    T = 23
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[3] = np.round(logits[3] * 2) / 2          # many exact ties
    logits[4] = 0.0
    logits[4, ::3] = -0.0                            # +-0 mix: all tie
    logits[5] = rng.integers(-2, 3, size=E).astype(np.float32)
    idx, w = oracle.topk_softmax(logits, k)
    for t in range(T):
        assert list(idx[t]) == _brute_topk(logits[t], k), t


def test_all_equal_logits():
    logits = np.full((3, 896), 0.37, np.float32)
    idx, w = oracle.topk_softmax(logits, 16)
    assert (idx == np.arange(16)).all()
    assert (w == np.float32(0.0625)).all()


def test_k_equals_one_and_k_equals_e():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((4, 30)).astype(np.float32)
    idx, w = oracle.topk_softmax(logits, 1)
    assert (w == 1.0).all() and (idx[:, 0] == logits.argmax(1)).all()
    idx, w = oracle.topk_softmax(logits, 30)
    for t in range(4):
        assert sorted(idx[t]) == list(range(30))


def test_softmax_weights():
    rng = np.random.default_rng(2)
    logits = (3 * rng.standard_normal((50, 896))).astype(np.float32)
    idx, w = oracle.topk_softmax(logits, 16)
    assert np.abs(w.sum(1) - 1).max() <= 2e-6
    assert (np.diff(w, axis=1) <= 0).all()
    sel = np.take_along_axis(logits, idx, 1).astype(np.float64)
    ref = np.exp(sel - sel[:, :1])
    ref /= ref.sum(1, keepdims=True)
    assert np.abs(w - ref).max() <= 1e-6


def _routing(T, E, k, seed, bias=0.0):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((T, E)) + bias).astype(np.float32)
    return oracle.topk_softmax(logits, k)


@pytest.mark.parametrize("T,E,k,e0,nl", [(37, 896, 16, 0, 896), (200, 64, 4, 16, 20),
                                         (1, 8, 8, 0, 8), (50, 896, 16, 0, 112)])
def test_permutation_invariants(T, E, k, e0, nl):
    idx, w = _routing(T, E, k, T + E)
    counts = oracle.histogram(idx, E)
    assert counts.sum() == T * k
    assert (counts == np.bincount(idx.reshape(-1), minlength=E)).all()
    off = oracle.offsets(counts, e0, nl)
    assert off[0] == 0 and (np.diff(off) >= 0).all()
    assert (np.diff(off) == counts[e0:e0 + nl]).all()
    perm, inv = oracle.permute(idx, off, e0, nl)
    A = int(off[-1])
    local = (idx >= e0) & (idx < e0 + nl)
    assert A == int(local.sum())
    assert ((inv >= 0) == local).all()
    # inv is a bijection onto [0, A) and perm_token inverts it
    pos = inv[local]
    assert sorted(pos.tolist()) == list(range(A))
    tok = np.repeat(np.arange(T), k).reshape(T, k)
    assert (perm[inv[local]] == tok[local]).all()
    # each position lies in its expert's segment; segments ascend in t
    exp_of = idx[local] - e0
    assert ((pos >= off[exp_of]) & (pos < off[exp_of + 1])).all()
    for le in range(nl):
        seg = perm[off[le]:off[le + 1]]
        assert (np.diff(seg) > 0).all()


def test_permute_then_unpermute_is_identity():
    rng = np.random.default_rng(5)
    T, E, k, d = 40, 32, 4, 16
    idx, _ = _routing(T, E, k, 9)
    off = oracle.offsets(oracle.histogram(idx, E), 0, E)
    perm, inv = oracle.permute(idx, off, 0, E)
    x = rng.integers(0, 2**16, size=(T, d)).astype(np.uint16)  # arbitrary bf16 rows
    x_perm = x[perm]
    back = x_perm[inv]  # [T, k, d]
    assert np.array_equal(back, np.repeat(x[:, None, :], k, axis=1))
    # combine with one-hot weights returns each token's chosen copy exactly
    y = x_perm.astype(np.float32)
    wsel = np.zeros((T, k), np.float32)
    wsel[:, 2] = 1.0
    out = oracle.combine(y, inv, wsel)
    assert np.array_equal(out, x.astype(np.float32))


def test_combine_drops_nonlocal_and_zero_rows():
    y = np.arange(12, dtype=np.float32).reshape(3, 4)
    inv = np.array([[0, -1], [-1, -1], [2, 1]], np.int32)
    w = np.array([[0.5, 0.5], [0.3, 0.7], [0.25, 0.75]], np.float32)
    out = oracle.combine(y, inv, w)
    assert np.array_equal(out[0], 0.5 * y[0])
    assert np.array_equal(out[1], np.zeros(4, np.float32))
    assert np.allclose(out[2], 0.25 * y[2] + 0.75 * y[1])
