"""The C-ABI library loads, exports every entry point include/moe_mxfp4.h
declares, and rejects bad arguments on the host before any HIP call (these
tests need no GPU: every call here fails validation first)."""

import ctypes as C
import os
import re

import pytest

import mxfp4_expert_top_amd as m

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_mxfp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_layer_entry_points():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_grouped_gemm_mxfp4", "moe_combine", "moe_layer"):
        assert n in names


def test_library_exports_every_declared_function():
    for n in declared_functions():
        assert hasattr(m.lib, n), n
    assert set(m.EXPORTED) <= set(declared_functions())


def test_schedule_choice():
    # the decode, prefill, EP-share and long skewed workloads of this repository
    assert m.moe_grouped_gemm_schedule(896, 64 * 16) == m.MODE_STREAM
    assert m.moe_grouped_gemm_schedule(896, 8192 * 16) == m.MODE_TILE256
    assert m.moe_grouped_gemm_schedule(112, 16384 * 16) == m.MODE_TILE128
    assert m.moe_grouped_gemm_schedule(896, 65536 * 16) == m.MODE_TILE256
    # explicit schedules are kept; TILED never streams
    for md in (m.MODE_STREAM, m.MODE_TILE128, m.MODE_TILE256):
        assert m.moe_grouped_gemm_schedule(896, 64, md) == md
    assert m.moe_grouped_gemm_schedule(896, 64, m.MODE_TILED) == m.MODE_TILE128
    # the thresholds: mean rows 16 (stream below), 128 and 256 (256-row tiles
    # between)
    assert m.moe_grouped_gemm_schedule(10, 159) == m.MODE_STREAM
    assert m.moe_grouped_gemm_schedule(10, 160) == m.MODE_TILE128
    assert m.moe_grouped_gemm_schedule(10, 1279) == m.MODE_TILE128
    assert m.moe_grouped_gemm_schedule(10, 1280) == m.MODE_TILE256
    assert m.moe_grouped_gemm_schedule(10, 2560) == m.MODE_TILE256
    assert m.moe_grouped_gemm_schedule(10, 2561) == m.MODE_TILE128
    # and a row bound of 2^19 or more: 256-row tiles whatever the mean
    assert m.moe_grouped_gemm_schedule(112, (1 << 19) - 1) == m.MODE_TILE128
    assert m.moe_grouped_gemm_schedule(112, 1 << 19) == m.MODE_TILE256
    assert m.lib.moe_grouped_gemm_schedule(0, 10, 0) == -1
    assert m.lib.moe_grouped_gemm_schedule(4, 10, 5) == -1


def test_status_strings():
    for s in range(5):
        assert m.lib.moe_status_string(s)
    assert m.lib.moe_status_string(99) == b"unknown status"
    assert m.lib.moe_last_error() == b""


P = C.c_void_p
FAKE = C.c_void_p(0x10000)  # never dereferenced: validation fails first


def test_route_validation():
    L = m.lib
    # k > E
    assert L.moe_route(FAKE, FAKE, None, FAKE, 0, 4, 128, 8, 9, FAKE, FAKE, FAKE, None) == 1
    # k < 1
    assert L.moe_route(FAKE, FAKE, None, FAKE, 0, 4, 128, 8, 0, FAKE, FAKE, FAKE, None) == 1
    # k > 32 unsupported
    assert L.moe_route(FAKE, FAKE, None, FAKE, 0, 4, 128, 896, 33, FAKE, FAKE, FAKE, None) == 2
    # E too large
    assert L.moe_route(FAKE, FAKE, None, FAKE, 0, 4, 128, 4096, 16, FAKE, FAKE, FAKE, None) == 2
    # d not a multiple of 128 when scores are computed
    assert L.moe_route(FAKE, FAKE, None, FAKE, 0, 4, 96, 64, 4, FAKE, FAKE, FAKE, None) == 2
    # missing outputs
    assert L.moe_route(FAKE, FAKE, None, FAKE, 0, 4, 128, 64, 4, None, FAKE, FAKE, None) == 1
    assert L.moe_route(FAKE, FAKE, None, FAKE, 0, 4, 128, 64, 4, FAKE, FAKE, None, None) == 1
    # negative T
    assert L.moe_route(FAKE, FAKE, None, FAKE, 0, -1, 128, 64, 4, FAKE, FAKE, FAKE, None) == 1


def test_permute_validation():
    L = m.lib
    ws = m.moe_permute_workspace_size(100, 64)
    assert ws >= 64 * 4
    # local range outside [0, E)
    assert L.moe_permute(FAKE, FAKE, 100, 4, 64, 60, 8, FAKE, FAKE, FAKE, FAKE, ws, None) == 1
    # workspace too small
    assert L.moe_permute(FAKE, FAKE, 100, 4, 64, 0, 64, FAKE, FAKE, FAKE, FAKE, 16, None) == 3
    # misaligned workspace
    assert L.moe_permute(FAKE, FAKE, 100, 4, 64, 0, 64, FAKE, FAKE, FAKE, C.c_void_p(0x10004),
                         ws, None) == 3


def _gemm(**kw):
    a = dict(a=FAKE, lda=256, a_rows=None, w1c=FAKE, w1s=FAKE, w2c=FAKE, w2s=FAKE, off=FAKE,
             nl=8, max_rows=64, N=128, K=256, bs=32, lay=0, act=1, out=FAKE, odt=0, ldo=128, mode=0,
             ws=None, wsb=0)
    a.update(kw)
    return m.lib.moe_grouped_gemm_mxfp4(*a.values(), None)


def test_grouped_gemm_validation():
    assert _gemm(bs=64) == 2                 # MX block must be 32
    assert _gemm(K=96, lda=96) == 2          # K % 128
    assert _gemm(N=96, ldo=96) == 2          # N % 64
    assert _gemm(w2c=None, w2s=None) == 1    # GLU without the up weight
    assert _gemm(act=0) == 1                 # plain GEMM with a second weight
    assert _gemm(act=7) == 1
    assert _gemm(odt=5) == 1
    assert _gemm(lda=100) == 1               # stride not a multiple of 8
    assert _gemm(mode=5) == 1
    assert _gemm(lay=2) == 1                 # unknown weight layout
    assert _gemm(K=8320, lda=8320) == 2      # K > MOE_MAX_K
    assert _gemm(w1s=C.c_void_p(0x10004)) == 1  # scales not 16-byte aligned
    assert _gemm() == 3                      # no workspace given
    need = m.moe_grouped_gemm_workspace_size(8, 64, 128, 0)
    assert need > 0
    assert _gemm(ws=C.c_void_p(0x10040), wsb=need) == 3  # misaligned


def test_combine_and_dequant_validation():
    L = m.lib
    assert L.moe_combine(FAKE, 0, 96, FAKE, FAKE, 4, 90, 4, FAKE, 0, 96, None) == 2  # d % 8
    assert L.moe_combine(FAKE, 0, 96, FAKE, FAKE, 4, 96, 33, FAKE, 0, 96, None) == 2  # k > 32
    assert L.moe_combine(FAKE, 3, 96, FAKE, FAKE, 4, 96, 4, FAKE, 0, 96, None) == 1
    assert L.moe_combine(FAKE, 0, 90, FAKE, FAKE, 4, 96, 4, FAKE, 0, 96, None) == 1  # ldy < d
    assert L.moe_mxfp4_dequant(FAKE, FAKE, 4, 48, FAKE, None) == 2
    assert L.moe_mxfp4_dequant(FAKE, FAKE, -1, 64, FAKE, None) == 1
    # zero-size requests are no-ops that touch nothing
    assert L.moe_mxfp4_dequant(None, None, 0, 64, None, None) == 0
    assert L.moe_mxfp4_quantize(FAKE, 4, 48, FAKE, FAKE, None) == 2
    assert L.moe_mxfp4_quantize(FAKE, -1, 64, FAKE, FAKE, None) == 1
    assert L.moe_mxfp4_quantize(None, 4, 64, FAKE, FAKE, None) == 1
    assert L.moe_mxfp4_quantize(C.c_void_p(0x10004), 4, 64, FAKE, FAKE, None) == 1
    assert L.moe_mxfp4_quantize(None, 0, 64, None, None, None) == 0
    assert L.moe_combine(None, 0, 96, None, None, 0, 96, 4, None, 0, 96, None) == 0


def test_prepack_validation():
    L = m.lib
    assert L.moe_mxfp4_prepack(FAKE, FAKE, 2, 24, 256, FAKE, FAKE, None) == 2   # N % 16
    assert L.moe_mxfp4_prepack(FAKE, FAKE, 2, 32, 96, FAKE, FAKE, None) == 2    # K % 128
    assert L.moe_mxfp4_prepack(None, None, 0, 32, 256, None, None, None) == 0   # nothing to do
    assert L.moe_mxfp4_prepack(FAKE, FAKE, 2, 32, 256, None, FAKE, None) == 1
    assert m.lib.moe_mxfp4_packed_scale_bytes(1024, 3584) == 1024 * 3584 // 32
    assert m.lib.moe_mxfp4_packed_scale_bytes(3584, 1024) == 3584 * 1024 // 32
    assert m.lib.moe_mxfp4_packed_scale_bytes(128, 128) == 128 * 16  # one padded group
    assert m.lib.moe_mxfp4_packed_scale_bytes(100, 128) == 0


def test_layer_params_and_workspace():
    p = m.layer_params(8, 3584, 896, 16, 128)
    n = m.moe_layer_workspace_size(p)
    assert n >= 8 * 896 * 4 + 8 * 16 * 3584 * 4
    bad = m.layer_params(8, 3584, 896, 16, 96)  # I % 128
    assert m.lib.moe_layer_workspace_size(C.byref(bad)) == 0
    bad = m.layer_params(8, 3584, 896, 16, 128, expert_begin=800, num_local=112)
    assert m.lib.moe_layer_workspace_size(C.byref(bad)) == 0
    bad = m.layer_params(8, 3584, 896, 16, 8320)  # I > MOE_MAX_K
    assert m.lib.moe_layer_workspace_size(C.byref(bad)) == 0
    bad = m.layer_params(8, 3584, 896, 16, 128, act=0)
    assert m.lib.moe_layer_workspace_size(C.byref(bad)) == 0
    # T == 0 is a no-op: returns before looking at any pointer
    p0 = m.layer_params(0, 3584, 896, 16, 128)
    assert m.lib.moe_layer(C.byref(p0), *([None] * 14), 0, None, None) == 0


def test_mx8_validation():
    L = m.lib
    # quantiser: K % 32, dtype, stride, alignment; empty input is a no-op
    assert L.moe_mxfp8_quantize(FAKE, 0, 64, 4, 48, FAKE, FAKE, None) == 2
    assert L.moe_mxfp8_quantize(FAKE, 2, 64, 4, 64, FAKE, FAKE, None) == 1
    assert L.moe_mxfp8_quantize(FAKE, 0, 60, 4, 64, FAKE, FAKE, None) == 1   # ldv < K
    assert L.moe_mxfp8_quantize(FAKE, 0, 68, 4, 64, FAKE, FAKE, None) == 1   # ldv % 8
    assert L.moe_mxfp8_quantize(C.c_void_p(0x10004), 0, 64, 4, 64, FAKE, FAKE, None) == 1
    assert L.moe_mxfp8_quantize(FAKE, 0, 64, 4, 64, None, FAKE, None) == 1
    assert L.moe_mxfp8_quantize(None, 0, 64, 0, 64, None, None, None) == 0
    # grouped GEMM: the bf16 checks plus the scale stride (lda % 32) and scales
    need = m.moe_grouped_gemm_mx8_workspace_size(8, 64)
    assert need > 0 and m.moe_grouped_gemm_mx8_workspace_size(0, 64) == 0

    def gemm(**kw):
        a = dict(ac=FAKE, asc=FAKE, lda=256, rows=None, w1c=FAKE, w1s=FAKE, w2c=FAKE, w2s=FAKE,
                 off=FAKE, nl=8, maxr=64, N=128, K=256, bs=32, lay=0, act=1, out=FAKE, odt=1,
                 osc=None, ldo=128, mode=0, ws=FAKE, wsb=need)
        a.update(kw)
        return L.moe_grouped_gemm_mx8(*a.values(), None)
    assert gemm(bs=64) == 2
    assert gemm(K=96, lda=96) == 2
    assert gemm(lda=264) == 1                 # scale stride lda / 32 not whole
    assert gemm(asc=None) == 1
    assert gemm(w2c=None, w2s=None) == 1
    assert gemm(wsb=need - 1) == 3
    assert gemm(maxr=0, ac=None, asc=None, out=None, ws=None, wsb=0) == 0
    assert gemm(odt=2) == 1                   # MXFP8 output without its scales
    assert gemm(osc=FAKE) == 1                # scales with an fp32 output
    assert gemm(odt=3, osc=FAKE) == 1
    assert gemm(mode=1, odt=2, osc=FAKE, ldo=128) == 2  # MXFP8 output: tiled schedules only
    assert gemm(mode=5) == 1
    # the streaming schedule needs the most plan space (16-row groups)
    assert need >= m.moe_grouped_gemm_workspace_size(8, 64, 128, m.MODE_STREAM)
    st = m.layer_params(8, 3584, 896, 16, 128, precision=m.PREC_MX8, mode=m.MODE_STREAM)
    assert L.moe_layer_workspace_size(C.byref(st)) > 0
    # the layer's precision field
    p = m.layer_params(8, 3584, 896, 16, 128, precision=m.PREC_MX8)
    n_mx8 = m.moe_layer_workspace_size(p)
    n_bf16 = m.moe_layer_workspace_size(m.layer_params(8, 3584, 896, 16, 128))
    # fp32 h in place of bf16, plus MXFP8 tokens and h
    assert n_mx8 >= n_bf16 + 8 * 16 * 128 * 2 + 8 * 3584 + 8 * 16 * 128
    bad = m.layer_params(8, 3584, 896, 16, 128, precision=3)
    assert L.moe_layer_workspace_size(C.byref(bad)) == 0


def test_fp6x2_validation():
    L = m.lib
    sp = L.moe_fp6x2_split
    A128 = C.c_void_p(0x10000)
    assert sp(FAKE, m.DT_BF16, 256, 0, 256, A128, 256, None) == 0  # no rows: a no-op
    assert sp(FAKE, 2, 256, 4, 256, A128, 256, None) == 1          # not bf16 / fp32
    assert sp(FAKE, m.DT_BF16, 256, 4, 224, A128, 256, None) == 2  # K % 64
    assert sp(FAKE, m.DT_BF16, 128, 4, 256, A128, 256, None) == 1  # ldv < K
    assert sp(FAKE, m.DT_BF16, 256, 4, 256, A128, 288, None) == 1  # ldo % 64
    assert sp(FAKE, m.DT_BF16, 256, 4, 256, None, 256, None) == 1
    assert sp(FAKE, m.DT_BF16, 256, 4, 256, C.c_void_p(0x10040), 256, None) == 1  # 64-byte out
    need = m.moe_grouped_gemm_fp6x2_workspace_size(8, 64)
    assert need > 0 and m.moe_grouped_gemm_fp6x2_workspace_size(0, 64) == 0

    def gemm(**kw):
        a = dict(a=A128, lda=256, rows=None, w1c=FAKE, w1s=FAKE, w2c=FAKE, w2s=FAKE,
                 off=FAKE, nl=8, maxr=64, N=128, K=256, bs=32, lay=0, act=1, out=FAKE, odt=0,
                 ldo=128, ws=FAKE, wsb=need)
        a.update(kw)
        return L.moe_grouped_gemm_fp6x2(*a.values(), None)
    assert gemm(a=None) == 1
    assert gemm(lda=192) == 1                 # row stride below K
    assert gemm(lda=288) == 1                 # row stride not a multiple of 64
    assert gemm(a=C.c_void_p(0x10040)) == 1   # records 128-byte aligned
    assert gemm(K=8192, lda=8192) == 2        # beyond the tile's 4096
    assert gemm(K=320, lda=320) == 2          # K % 128
    assert gemm(wsb=need - 1) == 3
    assert gemm(act=0) == 1                   # ACT_NONE takes no second weight
    assert gemm(maxr=0) == 0
    assert gemm(odt=3, act=0, w2c=None, w2s=None) == 2  # records need a GLU act
    assert gemm(odt=3, ldo=160) == 1          # record rows: ldo % 64
    assert gemm(odt=3, out=C.c_void_p(0x10040)) == 1  # records 128-byte aligned
    assert gemm(odt=4) == 1
    # the layer: FP6X2 adds the tokens' and h's planes (2 T d + 2 T k I
    # bytes) where its schedule resolves to 256-row tiles, nothing where it
    # streams
    big = dict(T=8192, d=3584, E=896, k=16, I=1024)
    n6 = m.moe_layer_workspace_size(m.layer_params(**big, precision=m.PREC_FP6X2))
    nb = m.moe_layer_workspace_size(m.layer_params(**big))
    assert n6 >= nb + 8192 * 3584 * 2 + 8192 * 16 * 1024 * 2
    small = dict(T=64, d=3584, E=896, k=16, I=1024)
    assert (m.moe_layer_workspace_size(m.layer_params(**small, precision=m.PREC_FP6X2)) ==
            m.moe_layer_workspace_size(m.layer_params(**small)))


def test_lora_validation():
    L = m.lib

    def glora(**kw):
        a = dict(x=FAKE, ldx=256, rows=None, la=FAKE, lb=FAKE, rank=16, scale=C.c_float(0.5),
                 off=FAKE, nl=4, maxr=64, N=128, K=256, y=FAKE, ldy=128, ws=FAKE,
                 wsb=m.moe_grouped_lora_workspace_size(64, 16))
        a.update(kw)
        return L.moe_grouped_lora(*a.values(), None)
    assert glora(rank=0) == 2 and glora(rank=65) == 2
    assert glora(K=260, ldx=264) == 2          # K % 8
    assert glora(N=130, ldy=132) == 2          # N % 4
    assert glora(ldx=200) == 1                 # ldx < K
    assert glora(ldy=130) == 1                 # ldy % 4
    assert glora(la=None) == 1
    assert glora(x=C.c_void_p(0x10004)) == 1   # misaligned
    assert glora(wsb=16) == 3
    assert glora(maxr=0, x=None, la=None, lb=None, off=None, y=None, ws=None, wsb=0) == 0
    assert m.moe_grouped_lora_workspace_size(64, 65) == 0
    p = m.layer_params(8, 3584, 896, 16, 128)
    assert m.moe_layer_lora_workspace_size(p, 16) > m.moe_layer_workspace_size(p)
    assert L.moe_layer_lora_workspace_size(C.byref(p), 0) == 0
    mx8 = m.layer_params(8, 3584, 896, 16, 128, precision=m.PREC_MX8)
    assert L.moe_layer_lora_workspace_size(C.byref(mx8), 16) == 0
    ad = m.LoraAdapters(16, 0.5, *([None] * 6))
    # no adapters -> INVALID_ARG (checked before any pointer is used)
    assert L.moe_layer_lora(C.byref(p), C.byref(ad), *([FAKE] * 10), None, None, None, FAKE,
                            1 << 30, None, None) == 1
    assert L.moe_layer_lora(C.byref(p), None, *([FAKE] * 10), None, None, None, FAKE,
                            1 << 30, None, None) == 1
    ad2 = m.LoraAdapters(100, 0.5, *([FAKE.value] * 6))
    assert L.moe_layer_lora(C.byref(p), C.byref(ad2), *([FAKE] * 10), None, None, None, FAKE,
                            1 << 30, None, None) == 2


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        m.moe_combine(x, torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2), x)


def test_layer_noalloc_rejects_sizes_beyond_its_scratch():
    """moe_layer_noalloc checks the scratch its parameters need against its
    static maximum before any HIP call, and says why in moe_last_error()."""
    L = m.lib
    big = m.layer_params(4096, 3584, 896, 16, 1024)  # about 1 GB of scratch
    assert m.moe_layer_workspace_size(big) > m.NOALLOC_SCRATCH_BYTES
    # x, w_router, bias, the six weight arrays, out; no routing copies; stream
    args = [FAKE, FAKE, None] + [FAKE] * 6 + [FAKE] + [None] * 4
    assert L.moe_layer_noalloc(C.byref(big), *args) == m.MOE_ERR_WORKSPACE
    msg = L.moe_last_error().decode()
    assert "moe_layer_noalloc" in msg and str(m.NOALLOC_SCRATCH_BYTES) in msg
    # the decode batch fits (the size check passes; no call is made here)
    dec = m.layer_params(64, 3584, 896, 16, 1024)
    assert m.moe_layer_workspace_size(dec) <= m.NOALLOC_SCRATCH_BYTES
    # T == 0: a no-op before any pointer is looked at
    p0 = m.layer_params(0, 3584, 896, 16, 128)
    assert L.moe_layer_noalloc(C.byref(p0), *([None] * 14)) == 0
    # parameters are checked as for moe_layer
    bad = m.layer_params(8, 3584, 896, 16, 96)
    assert L.moe_layer_noalloc(C.byref(bad), *args) == m.MOE_ERR_UNSUPPORTED
