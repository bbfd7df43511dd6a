"""Python binding of libmoe_mxfp4.so (the C ABI in include/moe_mxfp4.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library. Tensors are PyTorch device tensors (PyTorch supplies device
memory and streams); each function checks devices, dtypes, contiguity and
shapes on the host -- the C ABI cannot see buffer sizes -- then passes raw
pointers and the current stream. There is no CPU fallback: if the library is
missing, importing this package raises.
"""

from __future__ import annotations

import ctypes as C
from pathlib import Path

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libmoe_mxfp4.so"

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
DT_BF16, DT_F32, DT_MXFP8, DT_FP6X2 = 0, 1, 2, 3
ACT_NONE, ACT_SILU_MUL, ACT_GELU_TANH_MUL = 0, 1, 2
MODE_AUTO, MODE_STREAM, MODE_TILED, MODE_TILE128, MODE_TILE256 = 0, 1, 2, 3, 4
LAYOUT_OCP, LAYOUT_PACKED = 0, 1
PREC_BF16, PREC_MX8, PREC_FP6X2 = 0, 1, 2
MX_BLOCK = 32


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def _load(path=None):
    path = Path(path) if path is not None else _LIB_PATH
    if not path.exists():
        raise ImportError(
            f"{path} is not built; run `python mxfp4_expert_top_amd/build.py` "
            "(there is no fallback path)")
    L = C.CDLL(str(path))
    p, i32, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
    L.moe_status_string.restype = C.c_char_p
    L.moe_status_string.argtypes = [i32]
    L.moe_last_error.restype = C.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_route.restype = i32
    L.moe_route.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, p, p, p, p]
    L.moe_permute_workspace_size.restype = sz
    L.moe_permute_workspace_size.argtypes = [i32, i32]
    L.moe_permute.restype = i32
    L.moe_permute.argtypes = [p, p, i32, i32, i32, i32, i32, p, p, p, p, sz, p]
    L.moe_mxfp4_quantize.restype = i32
    L.moe_mxfp4_quantize.argtypes = [p, i64, i32, p, p, p]
    L.moe_mxfp4_dequant.restype = i32
    L.moe_mxfp4_dequant.argtypes = [p, p, i64, i32, p, p]
    L.moe_grouped_gemm_schedule.restype = i32
    L.moe_grouped_gemm_schedule.argtypes = [i32, i32, i32]
    L.moe_grouped_gemm_workspace_size.restype = sz
    L.moe_grouped_gemm_workspace_size.argtypes = [i32, i32, i32, i32]
    L.moe_grouped_gemm_mxfp4.restype = i32
    L.moe_grouped_gemm_mxfp4.argtypes = [p, i64, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                         i32, p, i32, i64, i32, p, sz, p]
    L.moe_mxfp4_packed_scale_bytes.restype = sz
    L.moe_mxfp4_packed_scale_bytes.argtypes = [i32, i32]
    L.moe_mxfp4_prepack.restype = i32
    L.moe_mxfp4_prepack.argtypes = [p, p, i32, i32, i32, p, p, p]
    L.moe_combine.restype = i32
    L.moe_combine.argtypes = [p, i32, i64, p, p, i32, i32, i32, p, i32, i64, p]
    L.moe_layer_workspace_size.restype = sz
    L.moe_layer_workspace_size.argtypes = [p]
    L.moe_layer.restype = i32
    L.moe_layer.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p, p, p, p, sz, p, p]
    L.moe_layer_noalloc.restype = i32
    L.moe_layer_noalloc.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p, p, p, p]
    L.moe_mxfp8_quantize.restype = i32
    L.moe_mxfp8_quantize.argtypes = [p, i32, i64, i64, i32, p, p, p]
    L.moe_grouped_gemm_mx8_workspace_size.restype = sz
    L.moe_grouped_gemm_mx8_workspace_size.argtypes = [i32, i32]
    L.moe_grouped_lora_workspace_size.restype = sz
    L.moe_grouped_lora_workspace_size.argtypes = [i32, i32]
    L.moe_grouped_lora.restype = i32
    L.moe_grouped_lora.argtypes = [p, i64, p, p, p, i32, C.c_float, p, i32, i32, i32, i32, p,
                                   i64, p, sz, p]
    L.moe_layer_lora_workspace_size.restype = sz
    L.moe_layer_lora_workspace_size.argtypes = [p, i32]
    L.moe_layer_lora.restype = i32
    L.moe_layer_lora.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p, p, p, p, p, sz, p, p]
    L.moe_grouped_gemm_mx8.restype = i32
    L.moe_grouped_gemm_mx8.argtypes = [p, p, i64, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                       i32, p, i32, p, i64, i32, p, sz, p]
    L.moe_fp6x2_split.restype = i32
    L.moe_fp6x2_split.argtypes = [p, i32, i64, i64, i32, p, i64, p]
    L.moe_grouped_gemm_fp6x2_workspace_size.restype = sz
    L.moe_grouped_gemm_fp6x2_workspace_size.argtypes = [i32, i32]
    L.moe_grouped_gemm_fp6x2.restype = i32
    L.moe_grouped_gemm_fp6x2.argtypes = [p, i64, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                         i32, p, i32, i64, p, sz, p]
    return L


lib = _load()

EXPORTED = ("moe_route", "moe_permute", "moe_permute_workspace_size", "moe_mxfp4_dequant",
            "moe_mxfp4_quantize",
            "moe_mxfp4_prepack", "moe_mxfp4_packed_scale_bytes",
            "moe_grouped_gemm_mxfp4", "moe_grouped_gemm_workspace_size",
            "moe_grouped_gemm_schedule", "moe_combine",
            "moe_layer", "moe_layer_workspace_size", "moe_layer_noalloc", "moe_status_string",
            "moe_last_error",
            "moe_mxfp8_quantize", "moe_grouped_gemm_mx8", "moe_grouped_gemm_mx8_workspace_size",
            "moe_grouped_lora", "moe_grouped_lora_workspace_size", "moe_layer_lora",
            "moe_layer_lora_workspace_size", "moe_fp6x2_split", "moe_grouped_gemm_fp6x2",
            "moe_grouped_gemm_fp6x2_workspace_size")


class LayerParams(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("T", "d", "E", "k", "I", "block_size", "expert_begin",
                                        "num_local", "act", "out_dtype", "mode",
                                        "weight_layout", "precision")]


def _check(fn, status):
    if status != MOE_OK:
        msg = lib.moe_status_string(status).decode()
        if status == MOE_ERR_HIP:
            msg += ": " + lib.moe_last_error().decode()
        raise MoeError(fn, status, msg)


def _dev(*ts, strided=()):
    """All tensors on one GPU and contiguous, except those in ``strided``
    (whose strides the caller checks and passes on)."""
    dev = None
    for t in (*ts, *strided):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous() and not any(t is u for u in strided):
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors on different devices")
    return dev


def _ptr(t):
    return None if t is None else t.data_ptr()


def _want(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dt(t):
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def moe_route(x, w_router, bias, logits, logits_given, topk_idx, topk_w, expert_counts,
              stream=None):
    """Router scores (unless ``logits_given``), top-k, softmax, histogram."""
    T, k = topk_idx.shape
    E = expert_counts.shape[0]
    d = x.shape[1] if x is not None else 0
    _dev(x, w_router, bias, logits, topk_idx, topk_w, expert_counts)
    _want(logits, torch.float32, (T, E), "logits")
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(topk_w, torch.float32, (T, k), "topk_w")
    _want(expert_counts, torch.int32, (E,), "expert_counts")
    if not logits_given:
        _want(x, torch.bfloat16, (T, d), "x")
        _want(w_router, torch.float32, (E, d), "w_router")
        if bias is not None:
            _want(bias, torch.float32, (E,), "bias")
    st = lib.moe_route(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits), int(bool(logits_given)),
                       T, d, E, k, _ptr(topk_idx), _ptr(topk_w), _ptr(expert_counts),
                       _stream(stream))
    _check("moe_route", st)


def moe_permute_workspace_size(T, num_local):
    return int(lib.moe_permute_workspace_size(T, num_local))


def moe_permute(topk_idx, expert_counts, expert_begin, num_local, expert_offsets, perm_token,
                inv, ws, stream=None, E=None):
    """expert_counts may be None (counts are then taken from topk_idx); E, the
    expert count, is then required."""
    T, k = topk_idx.shape
    if expert_counts is not None:
        E = expert_counts.shape[0]
        _want(expert_counts, torch.int32, (E,), "expert_counts")
    elif E is None:
        raise ValueError("E is required when expert_counts is None")
    _dev(topk_idx, expert_counts, expert_offsets, perm_token, inv, ws)
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(expert_offsets, torch.int32, (num_local + 1,), "expert_offsets")
    _want(perm_token, torch.int32, (T * k,), "perm_token")
    _want(inv, torch.int32, (T, k), "inv")
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib.moe_permute(_ptr(topk_idx), _ptr(expert_counts), T, k, E, expert_begin, num_local,
                         _ptr(expert_offsets), _ptr(perm_token), _ptr(inv), _ptr(ws), nbytes,
                         _stream(stream))
    _check("moe_permute", st)


def moe_mxfp4_quantize(w, codes=None, scales=None, stream=None):
    """fp32 [N, K] (or [..., N, K]) on the GPU -> (codes uint8 [..., N, K/2],
    scales uint8 [..., N, K/32]) in the canonical MXFP4 layout."""
    if w.dtype != torch.float32:
        raise TypeError(f"w: expected torch.float32, got {w.dtype}")
    K = w.shape[-1]
    N = w.numel() // K if K else 0
    lead = tuple(w.shape[:-1])
    if codes is None:
        codes = torch.empty(*lead, K // 2, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(*lead, K // 32, dtype=torch.uint8, device=w.device)
    _dev(w, codes, scales)
    _want(codes, torch.uint8, lead + (K // 2,), "codes")
    _want(scales, torch.uint8, lead + (K // 32,), "scales")
    _check("moe_mxfp4_quantize", lib.moe_mxfp4_quantize(_ptr(w), N, K, _ptr(codes),
                                                        _ptr(scales), _stream(stream)))
    return codes, scales


def moe_mxfp8_quantize(v, codes=None, scales=None, stream=None):
    """bf16 or fp32 [N, K] on the GPU -> MXFP8 (codes uint8 [N, K] E4M3,
    scales uint8 [N, K/32] E8M0)."""
    if v.dtype not in (torch.bfloat16, torch.float32) or v.dim() != 2:
        raise TypeError("v must be a 2-D bf16 or fp32 tensor")
    N, K = v.shape
    if v.stride(1) != 1:
        raise ValueError("v rows must be contiguous")
    if codes is None:
        codes = torch.empty(N, K, dtype=torch.uint8, device=v.device)
    if scales is None:
        scales = torch.empty(N, K // 32, dtype=torch.uint8, device=v.device)
    _dev(codes, scales)
    if not v.is_cuda or v.device != codes.device:
        raise ValueError("v must be on the GPU of codes and scales")
    _want(codes, torch.uint8, (N, K), "codes")
    _want(scales, torch.uint8, (N, K // 32), "scales")
    _check("moe_mxfp8_quantize", lib.moe_mxfp8_quantize(_ptr(v), _dt(v), v.stride(0), N, K,
                                                        _ptr(codes), _ptr(scales),
                                                        _stream(stream)))
    return codes, scales


def moe_mxfp4_dequant(codes, scales, out, stream=None):
    N, K = out.shape
    _dev(codes, scales, out)
    _want(codes, torch.uint8, (N, K // 2), "codes")
    _want(scales, torch.uint8, (N, K // 32), "scales")
    _want(out, torch.bfloat16, (N, K), "out")
    _check("moe_mxfp4_dequant",
           lib.moe_mxfp4_dequant(_ptr(codes), _ptr(scales), N, K, _ptr(out), _stream(stream)))


def packed_scale_cols(N, K):
    """Per-row width of the packed scale array: moe_mxfp4_packed_scale_bytes / N."""
    return int(lib.moe_mxfp4_packed_scale_bytes(N, K)) // N


def scale_shape(n_mats, N, K, layout):
    return (n_mats, N, K // 32 if layout == LAYOUT_OCP else packed_scale_cols(N, K))


def moe_mxfp4_prepack(codes, scales, stream=None):
    """Streaming layout of stacked MXFP4 matrices: codes [n, N, K/2], scales
    [n, N, K/32] -> new (codes, scales) tensors on the same device."""
    n, N, K2 = codes.shape
    K = 2 * K2
    _dev(codes, scales)
    _want(codes, torch.uint8, (n, N, K // 2), "codes")
    _want(scales, torch.uint8, (n, N, K // 32), "scales")
    pc = torch.empty_like(codes)
    ps = torch.empty(scale_shape(n, N, K, LAYOUT_PACKED), dtype=torch.uint8, device=codes.device)
    _check("moe_mxfp4_prepack", lib.moe_mxfp4_prepack(_ptr(codes), _ptr(scales), n, N, K,
                                                      _ptr(pc), _ptr(ps), _stream(stream)))
    return pc, ps


def prepack_weights(weights, stream=None):
    """The six expert weight arrays of a layer in the streaming layout."""
    out = {}
    for name in ("gate", "up", "down"):
        out[name + "_codes"], out[name + "_scales"] = moe_mxfp4_prepack(
            weights[name + "_codes"], weights[name + "_scales"], stream)
    return out


def moe_grouped_gemm_schedule(num_local, max_rows, mode=MODE_AUTO):
    """The schedule (MODE_STREAM, MODE_TILE128 or MODE_TILE256) `mode` resolves to."""
    r = lib.moe_grouped_gemm_schedule(num_local, max_rows, mode)
    if r < 0:
        raise MoeError("moe_grouped_gemm_schedule", MOE_ERR_INVALID_ARG, "invalid argument")
    return r


def moe_grouped_gemm_workspace_size(num_local, max_rows, N, mode=MODE_AUTO):
    return int(lib.moe_grouped_gemm_workspace_size(num_local, max_rows, N, mode))


def moe_grouped_gemm_mxfp4(a, a_rows, w1_codes, w1_scales, w2_codes, w2_scales,
                           expert_offsets, max_rows, act, out, ws, mode=MODE_AUTO,
                           w_layout=LAYOUT_OCP, stream=None):
    """out[r] = act(a_row(r) @ W1[e].T, a_row(r) @ W2[e].T) for the rows r of
    each local expert e (see the header). ``out`` is [>= rows, N]."""
    num_local = expert_offsets.shape[0] - 1
    N, K = w1_codes.shape[1], w1_codes.shape[2] * 2
    _dev(a, a_rows, w1_codes, w1_scales, w2_codes, w2_scales, expert_offsets, out, ws)
    if a.dtype != torch.bfloat16 or a.dim() != 2 or a.shape[1] != K:
        raise ValueError("a must be [rows, K] bf16")
    _want(w1_codes, torch.uint8, (num_local, N, K // 2), "w1_codes")
    _want(w1_scales, torch.uint8, scale_shape(num_local, N, K, w_layout), "w1_scales")
    if w2_codes is not None:
        _want(w2_codes, torch.uint8, (num_local, N, K // 2), "w2_codes")
        _want(w2_scales, torch.uint8, scale_shape(num_local, N, K, w_layout), "w2_scales")
    if out.dim() != 2 or out.shape[1] != N or out.shape[0] < max_rows:
        raise ValueError("out must be [>= max_rows, N]")
    if a_rows is not None:
        if a_rows.dtype != torch.int32 or a_rows.numel() < max_rows:
            raise ValueError("a_rows must be int32 with >= max_rows entries")
    elif a.shape[0] < max_rows:
        raise ValueError("a must hold >= max_rows rows")
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib.moe_grouped_gemm_mxfp4(
        _ptr(a), K, _ptr(a_rows), _ptr(w1_codes), _ptr(w1_scales), _ptr(w2_codes),
        _ptr(w2_scales), _ptr(expert_offsets), num_local, max_rows, N, K, MX_BLOCK, w_layout, act,
        _ptr(out), _dt(out), N, mode, _ptr(ws), nbytes, _stream(stream))
    _check("moe_grouped_gemm_mxfp4", st)


def moe_grouped_gemm_mx8_workspace_size(num_local, max_rows):
    return int(lib.moe_grouped_gemm_mx8_workspace_size(num_local, max_rows))


def moe_grouped_gemm_mx8(a_codes, a_scales, a_rows, w1_codes, w1_scales, w2_codes, w2_scales,
                         expert_offsets, max_rows, act, out, ws, w_layout=LAYOUT_OCP,
                         out_scales=None, mode=MODE_AUTO, stream=None):
    """moe_grouped_gemm_mxfp4 with MXFP8 rows (a_codes uint8 [rows, K] E4M3,
    a_scales uint8 [rows, K/32]) on the block-scaled matrix cores. ``out`` is
    bf16 or fp32, or uint8 (MXFP8 codes) with ``out_scales`` uint8
    [>= max_rows, N/32]."""
    num_local = expert_offsets.shape[0] - 1
    N, K = w1_codes.shape[1], w1_codes.shape[2] * 2
    _dev(a_rows, w1_codes, w1_scales, w2_codes, w2_scales, expert_offsets, out, ws,
         strided=(a_codes, a_scales))
    if a_codes.dtype != torch.uint8 or a_codes.dim() != 2 or a_codes.shape[1] != K:
        raise ValueError("a_codes must be [rows, K] uint8")
    # rows may be strided (lda = a_codes.stride(0), a multiple of 32); the
    # scales then have lda / 32 per row
    lda = a_codes.stride(0) if a_codes.shape[0] > 1 else K
    if a_codes.stride(1) != 1 or lda % 32 or lda < K:
        raise ValueError("a_codes rows must be contiguous with a row stride that is a "
                         "multiple of 32")
    if (a_scales.dtype != torch.uint8 or a_scales.dim() != 2
            or tuple(a_scales.shape) != (a_codes.shape[0], K // 32) or a_scales.stride(1) != 1
            or (a_scales.shape[0] > 1 and a_scales.stride(0) != lda // 32)):
        raise ValueError(f"a_scales must be uint8 [{a_codes.shape[0]}, {K // 32}] with row "
                         f"stride {lda // 32}")
    _want(w1_codes, torch.uint8, (num_local, N, K // 2), "w1_codes")
    _want(w1_scales, torch.uint8, scale_shape(num_local, N, K, w_layout), "w1_scales")
    if w2_codes is not None:
        _want(w2_codes, torch.uint8, (num_local, N, K // 2), "w2_codes")
        _want(w2_scales, torch.uint8, scale_shape(num_local, N, K, w_layout), "w2_scales")
    if out.dim() != 2 or out.shape[1] != N or out.shape[0] < max_rows:
        raise ValueError("out must be [>= max_rows, N]")
    if a_rows is not None:
        if a_rows.dtype != torch.int32 or a_rows.numel() < max_rows:
            raise ValueError("a_rows must be int32 with >= max_rows entries")
    elif a_codes.shape[0] < max_rows:
        raise ValueError("a_codes must hold >= max_rows rows")
    if out.dtype == torch.uint8:
        if out_scales is None:
            raise ValueError("MXFP8 output needs out_scales")
        _dev(out_scales)
        _want(out_scales, torch.uint8, (out.shape[0], N // 32), "out_scales")
        odt = DT_MXFP8
    else:
        if out_scales is not None:
            raise ValueError("out_scales is only for MXFP8 (uint8) output")
        odt = _dt(out)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib.moe_grouped_gemm_mx8(
        _ptr(a_codes), _ptr(a_scales), lda, _ptr(a_rows), _ptr(w1_codes), _ptr(w1_scales),
        _ptr(w2_codes), _ptr(w2_scales), _ptr(expert_offsets), num_local, max_rows, N, K,
        MX_BLOCK, w_layout, act, _ptr(out), odt, _ptr(out_scales), N, mode, _ptr(ws), nbytes,
        _stream(stream))
    _check("moe_grouped_gemm_mx8", st)


def moe_fp6x2_split(v, out=None, stream=None):
    """bf16 or fp32 [N, K] on the GPU -> the two MXFP6 planes as uint8
    [N, 2 K]: one 128-byte record per 64 elements (the two blocks at bytes 0
    and 64, each plane-1 codes then plane-2 codes, 24 bytes each, code i at
    bits 6i..6i+5; the four scale codes at bytes 48..51, repeated at 52..63;
    zeros at 112..127)."""
    if v.dtype not in (torch.bfloat16, torch.float32) or v.dim() != 2:
        raise TypeError("v must be a 2-D bf16 or fp32 tensor")
    N, K = v.shape
    if v.stride(1) != 1:
        raise ValueError("v rows must be contiguous")
    if out is None:
        out = torch.empty(N, 2 * K, dtype=torch.uint8, device=v.device)
    _dev(out)
    if not v.is_cuda or v.device != out.device:
        raise ValueError("v must be on the GPU of out")
    _want(out, torch.uint8, (N, 2 * K), "out")
    _check("moe_fp6x2_split", lib.moe_fp6x2_split(_ptr(v), _dt(v), v.stride(0), N, K, _ptr(out),
                                                  K, _stream(stream)))
    return out


def moe_grouped_gemm_fp6x2_workspace_size(num_local, max_rows):
    return int(lib.moe_grouped_gemm_fp6x2_workspace_size(num_local, max_rows))


def moe_grouped_gemm_fp6x2(a, a_rows, w1_codes, w1_scales, w2_codes, w2_scales,
                           expert_offsets, max_rows, act, out, ws, w_layout=LAYOUT_OCP,
                           stream=None):
    """moe_grouped_gemm_mxfp4 with rows as two MXFP6 planes (``a`` uint8
    [rows, 2 K] as moe_fp6x2_split writes it) on the block-scaled matrix
    cores, 256-row tiles. ``out`` is bf16 or fp32 [>= max_rows, N], or uint8
    [>= max_rows, 2 N]: the results as split records (GLU acts only)."""
    num_local = expert_offsets.shape[0] - 1
    N, K = w1_codes.shape[1], w1_codes.shape[2] * 2
    _dev(a, a_rows, w1_codes, w1_scales, w2_codes, w2_scales, expert_offsets, out, ws)
    rows = a.shape[0]
    _want(a, torch.uint8, (rows, 2 * K), "a")
    _want(w1_codes, torch.uint8, (num_local, N, K // 2), "w1_codes")
    _want(w1_scales, torch.uint8, scale_shape(num_local, N, K, w_layout), "w1_scales")
    if w2_codes is not None:
        _want(w2_codes, torch.uint8, (num_local, N, K // 2), "w2_codes")
        _want(w2_scales, torch.uint8, scale_shape(num_local, N, K, w_layout), "w2_scales")
    rec = out.dtype == torch.uint8
    if out.dim() != 2 or out.shape[1] != (2 * N if rec else N) or out.shape[0] < max_rows:
        raise ValueError("out must be [>= max_rows, N] (uint8: [>= max_rows, 2 N])")
    if a_rows is not None:
        if a_rows.dtype != torch.int32 or a_rows.numel() < max_rows:
            raise ValueError("a_rows must be int32 with >= max_rows entries")
    elif rows < max_rows:
        raise ValueError("a must hold >= max_rows rows")
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib.moe_grouped_gemm_fp6x2(
        _ptr(a), K, _ptr(a_rows), _ptr(w1_codes), _ptr(w1_scales), _ptr(w2_codes),
        _ptr(w2_scales), _ptr(expert_offsets), num_local, max_rows, N, K, MX_BLOCK, w_layout, act,
        _ptr(out), DT_FP6X2 if rec else _dt(out), N, _ptr(ws), nbytes, _stream(stream))
    _check("moe_grouped_gemm_fp6x2", st)


def moe_combine(y, inv, topk_w, out, stream=None):
    T, k = inv.shape
    d = out.shape[1]
    _dev(y, inv, topk_w, out)
    _want(inv, torch.int32, (T, k), "inv")
    _want(topk_w, torch.float32, (T, k), "topk_w")
    if y.dim() != 2 or y.shape[1] != d or out.shape[0] != T:
        raise ValueError("y must be [rows, d] and out [T, d]")
    st = lib.moe_combine(_ptr(y), _dt(y), d, _ptr(inv), _ptr(topk_w), T, d, k, _ptr(out), _dt(out),
                         d, _stream(stream))
    _check("moe_combine", st)


def layer_params(T, d, E, k, I, expert_begin=0, num_local=None, act=ACT_SILU_MUL,
                 out_dtype=DT_BF16, mode=MODE_AUTO, weight_layout=LAYOUT_OCP,
                 precision=PREC_BF16):
    return LayerParams(T, d, E, k, I, MX_BLOCK, expert_begin,
                       E - expert_begin if num_local is None else num_local, act, out_dtype, mode,
                       weight_layout, precision)


def moe_layer_workspace_size(params: LayerParams) -> int:
    n = int(lib.moe_layer_workspace_size(C.byref(params)))
    if n == 0:
        raise MoeError("moe_layer_workspace_size", MOE_ERR_INVALID_ARG, "invalid parameters")
    return n


def _layer_args(p, x, w_router, bias, weights, out, ws, logits_out, topk_idx_out, topk_w_out,
                stage_events, stream):
    """Checks of the layer's tensors; returns (byte count of ws, event array)."""
    _dev(x, w_router, bias, out, ws, logits_out, topk_idx_out, topk_w_out,
         *[weights[n] for n in _WNAMES])
    _want(x, torch.bfloat16, (p.T, p.d), "x")
    _want(w_router, torch.float32, (p.E, p.d), "w_router")
    if bias is not None:
        _want(bias, torch.float32, (p.E,), "bias")
    lay = p.weight_layout
    for n, shape in (("gate_codes", (p.num_local, p.I, p.d // 2)),
                     ("gate_scales", scale_shape(p.num_local, p.I, p.d, lay)),
                     ("up_codes", (p.num_local, p.I, p.d // 2)),
                     ("up_scales", scale_shape(p.num_local, p.I, p.d, lay)),
                     ("down_codes", (p.num_local, p.d, p.I // 2)),
                     ("down_scales", scale_shape(p.num_local, p.d, p.I, lay))):
        _want(weights[n], torch.uint8, shape, n)
    _want(out, torch.float32 if p.out_dtype == DT_F32 else torch.bfloat16, (p.T, p.d), "out")
    if logits_out is not None:
        _want(logits_out, torch.float32, (p.T, p.E), "logits_out")
    if topk_idx_out is not None:
        _want(topk_idx_out, torch.int32, (p.T, p.k), "topk_idx_out")
    if topk_w_out is not None:
        _want(topk_w_out, torch.float32, (p.T, p.k), "topk_w_out")
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    ev = None
    if stage_events is not None:
        if len(stage_events) != 6:
            raise ValueError("stage_events needs 6 events")
        for e_ in stage_events:
            e_.record(torch.cuda.current_stream() if stream is None else stream)  # materialise
        ev = (C.c_void_p * 6)(*[e_.cuda_event for e_ in stage_events])
    return nbytes, ev


def moe_layer(params: LayerParams, x, w_router, bias, weights, out, ws, logits_out=None,
              topk_idx_out=None, topk_w_out=None, stage_events=None, stream=None):
    """The fused layer. ``weights`` holds gate/up/down codes and scales
    (local experts stacked). ``stage_events``: None or 6 torch.cuda.Event."""
    p = params
    nbytes, ev = _layer_args(p, x, w_router, bias, weights, out, ws, logits_out, topk_idx_out,
                             topk_w_out, stage_events, stream)
    st = lib.moe_layer(C.byref(p), _ptr(x), _ptr(w_router), _ptr(bias),
                       *[_ptr(weights[n]) for n in _WNAMES], _ptr(out), _ptr(logits_out),
                       _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), nbytes, ev,
                       _stream(stream))
    _check("moe_layer", st)


_WNAMES = ("gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales")

# Bytes of the static device scratch of moe_layer_noalloc.
NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_layer_noalloc(params: LayerParams, x, w_router, bias, weights, out, logits_out=None,
                      topk_idx_out=None, topk_w_out=None, stream=None):
    """moe_layer without a workspace: the library's static per-GPU scratch
    (NOALLOC_SCRATCH_BYTES) instead. The tensors' GPU is made current for the
    call, as the scratch is looked up on the current device."""
    p = params
    _layer_args(p, x, w_router, bias, weights, out, None, logits_out, topk_idx_out, topk_w_out,
                None, stream)
    with torch.cuda.device(x.device):
        st = lib.moe_layer_noalloc(C.byref(p), _ptr(x), _ptr(w_router), _ptr(bias),
                                   *[_ptr(weights[n]) for n in _WNAMES], _ptr(out),
                                   _ptr(logits_out), _ptr(topk_idx_out), _ptr(topk_w_out),
                                   _stream(stream))
    if st == MOE_ERR_WORKSPACE:  # the sizes are in the thread's last error message
        raise MoeError("moe_layer_noalloc", st, lib.moe_last_error().decode())
    _check("moe_layer_noalloc", st)


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device byte buffer (torch's allocator returns 256-byte aligned blocks)."""
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws


# ---------------------------------------------------------------- LoRA
LORA_NAMES = ("gate_a", "gate_b", "up_a", "up_b", "down_a", "down_b")


class LoraAdapters(C.Structure):
    _fields_ = [("rank", C.c_int), ("scale", C.c_float)] + [(n, C.c_void_p) for n in LORA_NAMES]


def moe_grouped_lora_workspace_size(max_rows, rank):
    return int(lib.moe_grouped_lora_workspace_size(max_rows, rank))


def moe_grouped_lora(x, x_rows, lora_a, lora_b, scale, expert_offsets, max_rows, y, ws,
                     stream=None):
    """y[r] += scale * (x_row(r) @ A_e.T) @ B_e.T for the rows r of each local
    expert e: x bf16 [rows, K], lora_a [num_local, rank, K], lora_b
    [num_local, N, rank] bf16, y fp32 [>= max_rows, N]."""
    num_local, rank, K = lora_a.shape
    N = lora_b.shape[1]
    _dev(x, x_rows, lora_a, lora_b, expert_offsets, y, ws)
    _want(x, torch.bfloat16, (x.shape[0], K), "x")
    _want(lora_b, torch.bfloat16, (num_local, N, rank), "lora_b")
    if lora_a.dtype != torch.bfloat16:
        raise TypeError("lora_a must be bf16")
    if y.dtype != torch.float32 or y.dim() != 2 or y.shape[1] != N or y.shape[0] < max_rows:
        raise ValueError("y must be fp32 [>= max_rows, N]")
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_grouped_lora", lib.moe_grouped_lora(
        _ptr(x), K, _ptr(x_rows), _ptr(lora_a), _ptr(lora_b), rank, float(scale),
        _ptr(expert_offsets), num_local, max_rows, N, K, _ptr(y), N, _ptr(ws), nbytes,
        _stream(stream)))


def moe_layer_lora_workspace_size(params: LayerParams, rank) -> int:
    n = int(lib.moe_layer_lora_workspace_size(C.byref(params), rank))
    if n == 0:
        raise MoeError("moe_layer_lora_workspace_size", MOE_ERR_INVALID_ARG, "invalid parameters")
    return n


def moe_layer_lora(params: LayerParams, lora, rank, scale, x, w_router, bias, weights, out, ws,
                   logits_out=None, topk_idx_out=None, topk_w_out=None, stage_events=None,
                   stream=None):
    """moe_layer with LoRA adapters (``lora`` maps gate_a .. down_b to bf16
    tensors of the shapes in the header) on every local expert projection."""
    p = params
    nbytes, ev = _layer_args(p, x, w_router, bias, weights, out, ws, logits_out, topk_idx_out,
                             topk_w_out, stage_events, stream)
    shapes = {"gate_a": (p.num_local, rank, p.d), "gate_b": (p.num_local, p.I, rank),
              "up_a": (p.num_local, rank, p.d), "up_b": (p.num_local, p.I, rank),
              "down_a": (p.num_local, rank, p.I), "down_b": (p.num_local, p.d, rank)}
    _dev(*[lora[n] for n in LORA_NAMES])
    for n in LORA_NAMES:
        _want(lora[n], torch.bfloat16, shapes[n], n)
    ad = LoraAdapters(rank, float(scale), *[_ptr(lora[n]) for n in LORA_NAMES])
    st = lib.moe_layer_lora(C.byref(p), C.byref(ad), _ptr(x), _ptr(w_router), _ptr(bias),
                            *[_ptr(weights[n]) for n in _WNAMES], _ptr(out), _ptr(logits_out),
                            _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), nbytes, ev,
                            _stream(stream))
    _check("moe_layer_lora", st)
