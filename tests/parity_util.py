"""Helpers of the GPU parity tests: run the layer through the C ABI, and run
the oracle on exactly the bytes the GPU saw."""

from __future__ import annotations

import numpy as np
import torch

import oracle

# Layer-output bound: relative L2 and max-abs relative to the oracle's rms.
REL_L2 = 1e-2
MAX_ABS_RMS = 3e-2
# Router scores: |gpu - oracle| <= LOGIT_TOL * max(1, |oracle|)
LOGIT_TOL = 1e-4
# Gate weights: |gpu - oracle| <= W_TOL (both computed from the same scores)
W_TOL = 2e-6


def np_(t):
    return t.detach().cpu().numpy()


def rel_l2(a, ref):
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs_rms(a, ref):
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(a - ref)) / max(rms, 1e-300))


def bf16_rounding_ok(got, ref, rel_slack=1e-5):
    """Elementwise check of a bf16 output against the exact result: rounding to
    nearest with 8 significant bits moves a value by at most 2^-8 of itself;
    the slack covers fp32 summation-order differences (rel_slack of each value
    plus 1e-5 of the rms)."""
    a, r = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(r ** 2)))
    return bool(np.all(np.abs(a - r) <= (2.0 ** -8 + rel_slack) * np.abs(r) + 1e-5 * rms))


def assert_close_layer(got, ref, what="", bf16_out=False):
    """rel-L2 <= REL_L2 and every |got - ref| <= MAX_ABS_RMS * rms. With
    ``bf16_out`` each element may also carry the final rounding to bf16, at
    most the unit roundoff 2^-8 of its own magnitude: that error scales with
    the value, the rms term covers the roundings inside the layer."""
    r = rel_l2(got, ref)
    if bf16_out:
        a, b = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        rms = float(np.sqrt(np.mean(b ** 2)))
        m = float(np.max(np.abs(a - b) - 2.0 ** -8 * np.abs(b)) / max(rms, 1e-300))
    else:
        m = max_abs_rms(got, ref)
    assert r <= REL_L2 and m <= MAX_ABS_RMS, f"{what}: rel_l2={r:.3e} max_abs/rms={m:.3e}"
    return r, m


def run_gpu_layer(inp, *, mode=0, out_dtype=torch.bfloat16, act=1, packed=None, precision=0):
    """The fused entry on ``inp`` (tensors already on the GPU). ``packed``: the
    weights already in the streaming layout (``inp.weights`` stay canonical).
    Returns dict of GPU tensors: out, logits, idx, w."""
    import mxfp4_expert_top_amd as m
    c = inp.cfg
    p = m.layer_params(c.T, c.d, c.E, c.k, c.I, c.expert_begin, c.num_local, act=act,
                       out_dtype=m.DT_F32 if out_dtype == torch.float32 else m.DT_BF16, mode=mode,
                       weight_layout=m.LAYOUT_OCP if packed is None else m.LAYOUT_PACKED,
                       precision=precision)
    dev = inp.x.device
    ws = m.alloc_workspace(m.moe_layer_workspace_size(p), dev)
    out = torch.empty(c.T, c.d, dtype=out_dtype, device=dev)
    logits = torch.empty(c.T, c.E, dtype=torch.float32, device=dev)
    idx = torch.empty(c.T, c.k, dtype=torch.int32, device=dev)
    w = torch.empty(c.T, c.k, dtype=torch.float32, device=dev)
    m.moe_layer(p, inp.x, inp.w_router, inp.bias, inp.weights if packed is None else packed, out,
                ws, logits, idx, w)
    torch.cuda.synchronize()
    return dict(out=out, logits=logits, idx=idx, w=w)


def host_weights(weights, local_ids=None):
    """numpy copies of the listed local experts' weights (all if None)."""
    out = {}
    for n, t in weights.items():
        out[n] = np_(t if local_ids is None else t[torch.as_tensor(local_ids, device=t.device)])
    return out


def oracle_rows(inp, idx, w, tokens, act=1, mx8=False):
    """Oracle output rows for `tokens`, given routing (idx, w) as numpy. Only
    the experts these tokens use are copied to the host."""
    c = inp.cfg
    idx = np.asarray(idx)
    sel = idx[tokens]
    loc = sel - c.expert_begin
    used = np.unique(loc[(loc >= 0) & (loc < c.num_local)])
    wts = host_weights(inp.weights, used)
    remap = np.full(c.num_local, -1, np.int64)
    remap[used] = np.arange(len(used))
    # compact routing: non-local experts -> -1 (skipped by the oracle's range test)
    cidx = np.full(idx.shape, -1, np.int32)
    local = (idx - c.expert_begin >= 0) & (idx - c.expert_begin < c.num_local)
    cidx[local] = remap[(idx - c.expert_begin)[local]]
    cidx[cidx < 0] = -1
    return oracle.token_rows(inp.x, cidx, np.asarray(w, np.float32), tokens, wts, I=c.I,
                             e0=0, n_local=max(len(used), 1), act=act, mx8=mx8) if len(used) else \
        np.zeros((len(tokens), c.d), np.float32)


def x_bits(inp):
    return oracle.bf16_bits(inp.x)
