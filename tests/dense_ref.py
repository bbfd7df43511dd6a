"""Independent fp64 numpy evaluations used to pin the oracle.

Nothing here is shared with the oracle or the GPU library: MXFP4 values are
decoded from the E2M1 bit fields (not from a table) and the layer output is
evaluated densely -- every expert on every token, weighted by a dense
[T, E] gate matrix -- so no permutation, offset or combine code is involved.
"""

from __future__ import annotations

import numpy as np


def e2m1_from_bits(code):
    """E2M1 value from its bit fields: sign bit 3, exponent bits 2-1 (bias 1),
    mantissa bit 0, exponent 0 subnormal (OCP MX v1.0 FP4 element)."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where((code >> 3) & 1, -1.0, 1.0)
    exp = (code >> 1) & 3
    man = code & 1
    mag = np.where(exp == 0, 0.5 * man, np.ldexp(1.0 + 0.5 * man, exp - 1))
    return sign * mag


def decode_bitfield(codes, scales) -> np.ndarray:
    """[N, K] fp64 from codes [N, K/2] (low nibble = even element) and E8M0
    scales [N, K/32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N = codes.shape[0]
    nib = np.empty((N, codes.shape[1] * 2), dtype=np.int64)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    vals = e2m1_from_bits(nib)
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return vals * np.repeat(sc, 32, axis=1)


def silu(g):
    return g / (1.0 + np.exp(-g))


def gelu_tanh(g):
    return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))


ACTS = {1: lambda g, u: silu(g) * u, 2: lambda g, u: gelu_tanh(g) * u}


def dense_gate_matrix(idx, w, E):
    """Dense [T, E] gate matrix: G[t, idx[t,j]] = w[t,j], zero elsewhere."""
    T, k = idx.shape
    G = np.zeros((T, E), dtype=np.float64)
    rows = np.repeat(np.arange(T), k)
    G[rows, idx.reshape(-1)] = w.reshape(-1).astype(np.float64)
    return G


def dense_masked_layer(x, idx, w, wts, *, E, e0=0, n_local=None, act=1):
    """out[t] = sum_{e local} G[t, e] * FFN_e(x[t]), every expert evaluated on
    every token in fp64. ``x`` is [T, d] (any float dtype, widened exactly)."""
    x = np.asarray(x, dtype=np.float64)
    n_local = E if n_local is None else n_local
    G = dense_gate_matrix(idx, w, E)
    T, d = x.shape
    out = np.zeros((T, d), dtype=np.float64)
    f = ACTS[act]
    for le in range(n_local):
        wg = decode_bitfield(wts["gate_codes"][le], wts["gate_scales"][le])
        wu = decode_bitfield(wts["up_codes"][le], wts["up_scales"][le])
        wd = decode_bitfield(wts["down_codes"][le], wts["down_scales"][le])
        h = f(x @ wg.T, x @ wu.T)
        out += G[:, e0 + le:e0 + le + 1] * (h @ wd.T)
    return out


def rel_l2(a, ref):
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs_over_rms(a, ref):
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(a - ref)) / max(rms, 1e-300))
