"""CPU oracle for the LatentMoE MXFP4 layer -- TEST INFRASTRUCTURE ONLY.

Plain single-threaded fp32 C (``moe_oracle.c``), loaded through ctypes. Only
the tests, the smoke check and the benchmark's CPU-baseline leg may use it; the
product path never imports it, and it imports nothing from the product.

Every array argument is a numpy array (C-contiguous, the dtype each wrapper
states); outputs are returned as new numpy arrays.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "moe_oracle.c"
# MOE_ORACLE_LIB names another build of moe_oracle.c to load instead (the
# mutation test points the pins at deliberately broken builds this way)
_LIB = Path(os.environ["MOE_ORACLE_LIB"]) if os.environ.get("MOE_ORACLE_LIB") else \
    _HERE / "liboracle.so"

ACT_NONE, ACT_SILU_MUL, ACT_GELU_TANH_MUL = 0, 1, 2

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-fPIC", "-shared"]


def build(force: bool = True) -> Path:
    """Compile liboracle.so with gcc (no BLAS, no OpenMP, no fast-math)."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        subprocess.check_call(["gcc", *CFLAGS, str(_SRC), "-lm", "-o", str(tmp)])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build(force=False)
        L = C.CDLL(str(_LIB))
        p, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        L.oracle_e2m1_value.restype = C.c_float
        L.oracle_e2m1_value.argtypes = [i32]
        L.oracle_e8m0_value.restype = C.c_float
        L.oracle_e8m0_value.argtypes = [i32]
        L.oracle_mxfp4_decode.argtypes = [p, p, i64, i64, p]
        L.oracle_mxfp4_quantize.argtypes = [p, i64, i64, p, p]
        L.oracle_router_logits.argtypes = [p, p, p, i64, i64, i64, p]
        L.oracle_topk_softmax.argtypes = [p, i64, i64, i64, p, p]
        L.oracle_histogram.argtypes = [p, i64, i64, i64, p]
        L.oracle_offsets.argtypes = [p, i64, i64, p]
        L.oracle_permute.argtypes = [p, p, i64, i64, i64, i64, p, p]
        L.oracle_expert_compute.restype = i32
        L.oracle_expert_compute.argtypes = [p, i64, i64, p, p, i64, p, p, p, p, p, p, i32, p, p]
        L.oracle_combine.argtypes = [p, p, p, i64, i64, i64, p]
        L.oracle_layer.restype = i64
        L.oracle_layer.argtypes = [p, p, p, p, i32, i64, i64, i64, i64, i64, i64, i64,
                                   p, p, p, p, p, p, i32, p, p, p, p, p, p, p]
        L.oracle_token_rows.restype = i32
        L.oracle_token_rows.argtypes = [p, i64, i64, i64, p, p, p, i64, i64, i64,
                                        p, p, p, p, p, p, i32, p]
        L.oracle_e4m3_value.restype = C.c_float
        L.oracle_e4m3_value.argtypes = [i32]
        L.oracle_mxfp8_quantize.argtypes = [p, i64, i64, p, p]
        L.oracle_mxfp8_decode.argtypes = [p, p, i64, i64, p]
        L.oracle_e2m3_value.argtypes = [i32]
        L.oracle_e2m3_value.restype = C.c_float
        L.oracle_mxfp6_quantize.argtypes = [p, i64, i64, p, p]
        L.oracle_mxfp6_decode.argtypes = [p, p, i64, i64, p]
        L.oracle_fp6x2_split.argtypes = [p, i64, i64, p, p]
        L.oracle_fp6x2_split.restype = i32
        L.oracle_expert_compute_mx8.restype = i32
        L.oracle_expert_compute_mx8.argtypes = L.oracle_expert_compute.argtypes
        L.oracle_layer_mx8.restype = i64
        L.oracle_layer_mx8.argtypes = L.oracle_layer.argtypes
        L.oracle_token_rows_mx8.restype = i32
        L.oracle_token_rows_mx8.argtypes = L.oracle_token_rows.argtypes
        L.oracle_layer_lora.restype = i64
        L.oracle_layer_lora.argtypes = [p, p, p, p, i32, i64, i64, i64, i64, i64, i64, i64,
                                        p, p, p, p, p, p, i32, p, p, p, p, p, p, i64,
                                        C.c_float, p, p, p, p, p, p, p]
        L.oracle_token_rows_lora.restype = i32
        L.oracle_token_rows_lora.argtypes = [p, i64, i64, i64, p, p, p, i64, i64, i64,
                                             p, p, p, p, p, p, i32, p, p, p, p, p, p, i64,
                                             C.c_float, p]
        _lib = L
    return _lib


def _arr(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def bf16_bits(x) -> np.ndarray:
    """bf16 payload as uint16 bits from a torch bf16 tensor or a uint16 array."""
    if hasattr(x, "dtype") and str(getattr(x, "dtype")) == "torch.bfloat16":
        import torch
        return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return _arr(x, np.uint16)


def e2m1_value(code: int) -> float:
    return float(lib().oracle_e2m1_value(int(code)))


def e8m0_value(s: int) -> float:
    return float(lib().oracle_e8m0_value(int(s)))


def mxfp4_decode(codes, scales) -> np.ndarray:
    codes, scales = _arr(codes, np.uint8), _arr(scales, np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    assert scales.shape == (N, K // 32)
    out = np.empty((N, K), np.float32)
    lib().oracle_mxfp4_decode(_ptr(codes), _ptr(scales), N, K, _ptr(out))
    return out


def mxfp4_quantize(w):
    w = _arr(w, np.float32)
    N, K = w.shape
    assert K % 32 == 0
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // 32), np.uint8)
    lib().oracle_mxfp4_quantize(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def e4m3_value(code: int) -> float:
    """OCP-MX E4M3 element value of a code (NaN for S.1111.111)."""
    return float(lib().oracle_e4m3_value(int(code)))


def mxfp8_quantize(v):
    """[N, K] fp32 -> MXFP8: codes [N, K] u8 (E4M3), scales [N, K/32] u8 (E8M0)."""
    v = _arr(v, np.float32)
    N, K = v.shape
    assert K % 32 == 0
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, K // 32), np.uint8)
    lib().oracle_mxfp8_quantize(_ptr(v), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def mxfp8_decode(codes, scales) -> np.ndarray:
    codes, scales = _arr(codes, np.uint8), _arr(scales, np.uint8)
    N, K = codes.shape
    assert scales.shape == (N, K // 32)
    out = np.empty((N, K), np.float32)
    lib().oracle_mxfp8_decode(_ptr(codes), _ptr(scales), N, K, _ptr(out))
    return out


def e2m3_value(code: int) -> float:
    """OCP-MX E2M3 element value of a code."""
    return float(lib().oracle_e2m3_value(int(code)))


def mxfp6_quantize(v):
    """[N, K] fp32 -> MXFP6: codes [N, K] u8 (E2M3, one per byte), scales
    [N, K/32] u8 (E8M0)."""
    v = _arr(v, np.float32)
    N, K = v.shape
    assert K % 32 == 0
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, K // 32), np.uint8)
    lib().oracle_mxfp6_quantize(_ptr(v), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def mxfp6_decode(codes, scales) -> np.ndarray:
    codes, scales = _arr(codes, np.uint8), _arr(scales, np.uint8)
    N, K = codes.shape
    assert scales.shape == (N, K // 32)
    out = np.empty((N, K), np.float32)
    lib().oracle_mxfp6_decode(_ptr(codes), _ptr(scales), N, K, _ptr(out))
    return out


def fp6x2_split(v):
    """[N, K] fp32 -> the two MXFP6 planes: codes [2, N, K] u8, scales
    [2, N, K/32] u8 (plane 2 carries v - decode(plane 1))."""
    v = _arr(v, np.float32)
    N, K = v.shape
    assert K % 32 == 0
    codes = np.empty((2, N, K), np.uint8)
    scales = np.empty((2, N, K // 32), np.uint8)
    if lib().oracle_fp6x2_split(_ptr(v), N, K, _ptr(codes), _ptr(scales)) != 0:
        raise MemoryError("oracle_fp6x2_split")
    return codes, scales


def fp6x2_value(codes, scales) -> np.ndarray:
    """The value the two planes carry: decode(plane 1) + decode(plane 2), in
    fp64 (exact)."""
    return (mxfp6_decode(codes[0], scales[0]).astype(np.float64) +
            mxfp6_decode(codes[1], scales[1]).astype(np.float64))


def router_logits(x, w_router, bias=None) -> np.ndarray:
    xb = bf16_bits(x)
    w_router = _arr(w_router, np.float32)
    T, d = xb.shape
    E = w_router.shape[0]
    if bias is not None:
        bias = _arr(bias, np.float32)
    out = np.empty((T, E), np.float32)
    lib().oracle_router_logits(_ptr(xb), _ptr(w_router), _ptr(bias), T, d, E, _ptr(out))
    return out


def topk_softmax(logits, k: int):
    logits = _arr(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().oracle_topk_softmax(_ptr(logits), T, E, k, _ptr(idx), _ptr(w))
    return idx, w


def histogram(idx, E: int) -> np.ndarray:
    idx = _arr(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    lib().oracle_histogram(_ptr(idx), T, k, E, _ptr(counts))
    return counts


def offsets(counts, e0: int, n_local: int) -> np.ndarray:
    counts = _arr(counts, np.int32)
    off = np.empty(n_local + 1, np.int32)
    lib().oracle_offsets(_ptr(counts), e0, n_local, _ptr(off))
    return off


def permute(idx, off, e0: int, n_local: int):
    idx, off = _arr(idx, np.int32), _arr(off, np.int32)
    T, k = idx.shape
    perm = np.empty(max(int(off[-1]), 1), np.int32)[: int(off[-1])]
    inv = np.empty((T, k), np.int32)
    lib().oracle_permute(_ptr(idx), _ptr(off), T, k, e0, n_local, _ptr(perm), _ptr(inv))
    return perm, inv


def _weights(wts):
    names = ("gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales")
    return [_arr(wts[n], np.uint8) for n in names]


def expert_compute(x, I, off, perm, wts, act=ACT_SILU_MUL, mx8=False):
    """Grouped expert FFNs over the permuted rows: h [A, I] and y [A, d] fp32.
    With mx8 the tokens and h are MXFP8-quantised (h is returned decoded, as
    it feeds the down projection)."""
    xb = bf16_bits(x)
    T, d = xb.shape
    off, perm = _arr(off, np.int32), _arr(perm, np.int32)
    n_local = off.shape[0] - 1
    A = int(off[-1])
    w6 = _weights(wts)
    h = np.empty((A, I), np.float32)
    y = np.empty((A, d), np.float32)
    fn = lib().oracle_expert_compute_mx8 if mx8 else lib().oracle_expert_compute
    rc = fn(_ptr(xb), d, I, _ptr(off), _ptr(perm), n_local, *[_ptr(a) for a in w6], act,
            _ptr(h), _ptr(y))
    if rc != 0:
        raise MemoryError("oracle_expert_compute failed")
    return h, y


def combine(y, inv, w) -> np.ndarray:
    y, inv, w = _arr(y, np.float32), _arr(inv, np.int32), _arr(w, np.float32)
    T, k = inv.shape
    d = y.shape[1]
    out = np.empty((T, d), np.float32)
    lib().oracle_combine(_ptr(y), _ptr(inv), _ptr(w), T, k, d, _ptr(out))
    return out


def layer(x, w_router, bias, wts, *, E, k, I, e0=0, n_local=None, act=ACT_SILU_MUL,
          logits=None, mx8=False):
    """The whole layer. If ``logits`` is given it is used instead of the router
    GEMM (routing replayed on another implementation's fp32 scores). With mx8
    the expert FFNs run in the block-scaled precision mode (MXFP8 tokens and h).

    Returns a dict: out [T,d] f32, logits, idx, w, counts, off, perm, inv, A.
    """
    xb = bf16_bits(x)
    T, d = xb.shape
    n_local = E - e0 if n_local is None else n_local
    if not (0 <= e0 and e0 + n_local <= E and 1 <= k <= E):
        raise ValueError("bad expert range or k")
    w_router = _arr(w_router, np.float32)
    if bias is not None:
        bias = _arr(bias, np.float32)
    if logits is None:
        lg, given = np.empty((T, E), np.float32), 0
    else:
        lg, given = np.array(_arr(logits, np.float32), copy=True), 1
    w6 = _weights(wts)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    counts = np.empty(E, np.int32)
    off = np.empty(n_local + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty((T, k), np.int32)
    out = np.empty((T, d), np.float32)
    fn = lib().oracle_layer_mx8 if mx8 else lib().oracle_layer
    A = fn(_ptr(xb), _ptr(w_router), _ptr(bias), _ptr(lg), given,
                           T, d, E, k, I, e0, n_local, *[_ptr(a) for a in w6], act,
                           _ptr(idx), _ptr(w), _ptr(counts), _ptr(off), _ptr(perm),
                           _ptr(inv), _ptr(out))
    if A < 0:
        raise MemoryError("oracle_layer failed")
    return dict(out=out, logits=lg, idx=idx, w=w, counts=counts, off=off,
                perm=perm[:A], inv=inv, A=int(A))


def token_rows(x, idx, w, tokens, wts, *, I, e0=0, n_local, act=ACT_SILU_MUL, mx8=False):
    """Layer output rows for the listed tokens only, from their routing."""
    xb = bf16_bits(x)
    T, d = xb.shape
    idx, w = _arr(idx, np.int32), _arr(w, np.float32)
    k = idx.shape[1]
    tokens = _arr(np.asarray(tokens, np.int64), np.int64)
    w6 = _weights(wts)
    out = np.empty((tokens.shape[0], d), np.float32)
    fn = lib().oracle_token_rows_mx8 if mx8 else lib().oracle_token_rows
    rc = fn(_ptr(xb), d, I, k, _ptr(idx), _ptr(w), _ptr(tokens),
                                 tokens.shape[0], e0, n_local, *[_ptr(a) for a in w6],
                                 act, _ptr(out))
    if rc != 0:
        raise MemoryError("oracle_token_rows failed")
    return out


LORA_NAMES = ("gate_a", "gate_b", "up_a", "up_b", "down_a", "down_b")


def layer_lora(x, w_router, bias, wts, lora, *, E, k, I, rank, scale, e0=0, n_local=None,
               act=ACT_SILU_MUL, logits=None):
    """The whole layer with LoRA adapters on every local expert's gate, up
    and down projections. ``lora`` maps gate_a/up_a [n_local, rank, d],
    gate_b/up_b [n_local, I, rank], down_a [n_local, rank, I], down_b
    [n_local, d, rank] to bf16 tensors or uint16 bit arrays."""
    xb = bf16_bits(x)
    T, d = xb.shape
    n_local = E - e0 if n_local is None else n_local
    w_router = _arr(w_router, np.float32)
    if bias is not None:
        bias = _arr(bias, np.float32)
    if logits is None:
        lg, given = np.empty((T, E), np.float32), 0
    else:
        lg, given = np.array(_arr(logits, np.float32), copy=True), 1
    w6 = _weights(wts)
    ad = [bf16_bits(lora[n]) for n in LORA_NAMES]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    counts = np.empty(E, np.int32)
    off = np.empty(n_local + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty((T, k), np.int32)
    out = np.empty((T, d), np.float32)
    A = lib().oracle_layer_lora(_ptr(xb), _ptr(w_router), _ptr(bias), _ptr(lg), given,
                                T, d, E, k, I, e0, n_local, *[_ptr(a) for a in w6], act,
                                *[_ptr(a) for a in ad], rank, float(scale),
                                _ptr(idx), _ptr(w), _ptr(counts), _ptr(off), _ptr(perm),
                                _ptr(inv), _ptr(out))
    if A < 0:
        raise MemoryError("oracle_layer_lora failed")
    return dict(out=out, logits=lg, idx=idx, w=w, counts=counts, off=off,
                perm=perm[:A], inv=inv, A=int(A))


def token_rows_lora(x, idx, w, tokens, wts, lora, *, I, rank, scale, e0=0, n_local,
                    act=ACT_SILU_MUL):
    """The LoRA layer's output rows for the listed tokens only, from their
    routing. ``lora`` as in layer_lora, indexed by local expert."""
    xb = bf16_bits(x)
    T, d = xb.shape
    idx, w = _arr(idx, np.int32), _arr(w, np.float32)
    k = idx.shape[1]
    tokens = _arr(np.asarray(tokens, np.int64), np.int64)
    w6 = _weights(wts)
    ad = [bf16_bits(lora[n]) for n in LORA_NAMES]
    out = np.empty((tokens.shape[0], d), np.float32)
    rc = lib().oracle_token_rows_lora(_ptr(xb), d, I, k, _ptr(idx), _ptr(w), _ptr(tokens),
                                      tokens.shape[0], e0, n_local, *[_ptr(a) for a in w6], act,
                                      *[_ptr(a) for a in ad], rank, float(scale), _ptr(out))
    if rc != 0:
        raise MemoryError("oracle_token_rows_lora failed")
    return out
