"""Helpers of the GPU parity tests: run the layer through the C ABI, and run
the oracle on exactly the bytes the GPU saw."""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

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


def assert_close_layer(got, ref, what=""):
    """rel-L2 <= REL_L2 and every |got - ref| <= MAX_ABS_RMS * rms(ref)."""
    r = rel_l2(got, ref)
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


def oracle_workers():
    """Threads for the oracle's per-token evaluations (each ctypes call runs
    the single-threaded oracle with the GIL released): the host's cores, at
    most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _compact(inp, idx, tokens):
    """The listed tokens' routing with local experts renumbered over the
    experts they use (non-local -> -1), and those experts' ids."""
    c = inp.cfg
    idx = np.asarray(idx)[np.asarray(tokens)]
    loc = idx - c.expert_begin
    is_loc = (loc >= 0) & (loc < c.num_local)
    used = np.unique(loc[is_loc])
    remap = np.full(c.num_local, -1, np.int64)
    remap[used] = np.arange(len(used))
    cidx = np.full(idx.shape, -1, np.int32)
    cidx[is_loc] = remap[loc[is_loc]]
    return cidx, used


def oracle_rows(inp, idx, w, tokens, act=1, mx8=False, lora=None, rank=0, scale=0.0):
    """Oracle output rows for `tokens`, given routing (idx, w) as numpy: each
    token evaluated on its own (oracle.token_rows, or token_rows_lora with
    ``lora`` adapters indexed by local expert), over chunks of tokens in
    parallel threads. Only the experts these tokens use are copied to the
    host."""
    c = inp.cfg
    tokens = np.asarray(tokens, np.int64)
    cidx, used = _compact(inp, idx, tokens)
    if not len(used):
        return np.zeros((len(tokens), c.d), np.float32)
    wts = host_weights(inp.weights, used)
    ad = None
    if lora is not None:
        ids = torch.as_tensor(used, device=lora["gate_a"].device)
        ad = {n: lora[n][ids].cpu() for n in oracle.LORA_NAMES}
    tsel = torch.as_tensor(tokens, device=inp.x.device)
    xs = inp.x[tsel].cpu()
    ws = np.asarray(w, np.float32)[tokens]
    n = len(tokens)
    nw = min(oracle_workers(), n)
    bounds = np.linspace(0, n, nw + 1).astype(int)

    def part(i):
        a, b = bounds[i], bounds[i + 1]
        if a == b:
            return np.zeros((0, c.d), np.float32)
        rows = np.arange(a, b)
        if ad is not None:
            return oracle.token_rows_lora(xs, cidx, ws, rows, wts, ad, I=c.I, rank=rank,
                                          scale=scale, e0=0, n_local=len(used), act=act)
        return oracle.token_rows(xs, cidx, ws, rows, wts, I=c.I, e0=0, n_local=len(used),
                                 act=act, mx8=mx8)

    with ThreadPoolExecutor(max_workers=nw) as ex:
        return np.concatenate(list(ex.map(part, range(nw))), axis=0)


def oracle_scores(x, w_router, bias):
    """The oracle's router scores of every token of x (a torch bf16 tensor,
    any device) against w_router / bias (numpy), over chunks of tokens in
    parallel threads."""
    T = x.shape[0]
    nw = max(1, min(oracle_workers(), T))
    bounds = np.linspace(0, T, nw + 1).astype(int)
    xs = x.cpu()

    def part(i):
        return oracle.router_logits(xs[bounds[i]:bounds[i + 1]], w_router, bias)

    with ThreadPoolExecutor(max_workers=nw) as ex:
        return np.concatenate(list(ex.map(part, range(nw))), axis=0)


def sample_tokens(cfg, idx, n_total=64, seed=0):
    """Tokens whose layer rows the full-size tests compare: the first and last
    token of the batch; the first and last token of the largest and of the
    smallest non-empty local expert segment; tokens spread through the hottest
    expert's segment; a token with no local expert (if any); seeded random
    tokens for the rest, n_total in all (or every token of a smaller batch)."""
    if cfg.T <= n_total:
        return list(range(cfg.T))
    idx = np.asarray(idx)
    loc = idx - cfg.expert_begin
    is_loc = (loc >= 0) & (loc < cfg.num_local)
    counts = np.bincount(loc[is_loc], minlength=cfg.num_local)
    nz = np.nonzero(counts)[0]
    big, small = int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])])
    toks = {0, cfg.T - 1}
    for e in (big, small):
        users = np.nonzero((loc == e).any(1))[0]
        toks |= {int(users[0]), int(users[-1])}
    hot = np.nonzero((loc == big).any(1))[0]
    toks |= set(int(t) for t in hot[np.linspace(0, len(hot) - 1, 10).astype(int)])
    none = np.nonzero(~is_loc.any(1))[0]
    if len(none):
        toks |= {int(none[0]), int(none[-1])}
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(cfg.T), sorted(toks))
    toks |= set(rng.choice(rest, size=max(0, n_total - len(toks)), replace=False).tolist())
    return sorted(toks)


def x_bits(inp):
    return oracle.bf16_bits(inp.x)


def block_int16_step(y):
    """The spacing of the block-int16 codes of fp32 rows y [R, d]: per 32
    columns, with e the biased exponent of the block's largest magnitude
    (at most 252), 2^(e - 126) / 32767."""
    R, d = y.shape
    mb = (np.abs(y).reshape(R, d // 32, 32).view(np.uint32).max(-1) >> 23).astype(np.int64)
    e = np.minimum(mb, 252)
    return np.repeat(np.exp2(e - 126.0) / 32767.0, 32, axis=1)
