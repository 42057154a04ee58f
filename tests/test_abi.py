"""C ABI checks that need no GPU: the library loads, exports every entry point declared in
include/q6k.h, reports sizes, and rejects bad arguments on the host before touching HIP."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def lib():
    from q6_int8_prefill_amd import _lib
    return _lib._lib


def declared_functions():
    names = set()
    for h in ("q6k.h", "q4k.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(q[46]k_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 21, names
    from q6_int8_prefill_amd import _lib as binding
    assert sorted(binding.EXPORTS) == names
    L = lib()
    for name in names:
        assert hasattr(L, name), name


def test_timeline_library_exports_its_declared_symbols():
    # the workgroup-timeline build of the same source: every product call plus the three calls of
    # its own header; the product library has none of those
    text = open(os.path.join(ROOT, "include", "q6k_timeline.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(q6k_timeline_[a-z_]+)\s*\(", text)))
    assert names == ["q6k_timeline_capacity", "q6k_timeline_clear", "q6k_timeline_read"]
    T = ctypes.CDLL(os.path.join(ROOT, "q6_int8_prefill_amd", "_build", "libq6k_timeline.so"))
    for name in declared_functions() + names:
        assert hasattr(T, name), name
    for name in names:
        assert not hasattr(lib(), name), name
    T.q6k_timeline_capacity.restype = ctypes.c_int64
    assert T.q6k_timeline_capacity() == 16384
    # host-side argument checks (no device needed)
    T.q6k_timeline_read.restype = ctypes.c_int
    T.q6k_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    assert T.q6k_timeline_read(None, 4) == -1
    assert T.q6k_timeline_read(FAKE, -1) == -1
    assert T.q6k_timeline_read(FAKE, 0) == 0


def test_ceilings_library_exports_its_declared_symbols():
    # the measurement library beside the product: every q6c_ call its header declares
    text = open(os.path.join(ROOT, "include", "q6k_ceilings.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(q6c_[a-z0-9_]+)\s*\(", text)))
    assert names == ["q6c_mfma", "q6c_overlap", "q6c_probe_waves", "q6c_stream", "q6c_tileop",
                     "q6c_valu", "q6c_wall_clock_khz"]
    L = ctypes.CDLL(os.path.join(ROOT, "q6_int8_prefill_amd", "_build", "libq6k_ceilings.so"))
    for name in names:
        assert hasattr(L, name), name
    # host-side argument checks (no device needed: they fail before any HIP call)
    f = L.q6c_mfma
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_void_p]
    assert f(9, 10, 1, FAKE, 1 << 20, None) == -1      # unknown kind
    assert f(0, 10, 9, FAKE, 1 << 20, None) == -1      # more than 8 waves per SIMD
    assert f(0, 0, 1, FAKE, 1 << 20, None) == -1       # no rounds
    s = L.q6c_stream
    s.restype = ctypes.c_int
    s.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_size_t, ctypes.c_void_p]
    assert s(0, FAKE, FAKE, 100, 1 << 20, None) == -1   # not a multiple of 16
    assert s(0, FAKE + 8, FAKE, 1 << 20, 1 << 20, None) == -3


def test_size_queries():
    import q6_int8_prefill_amd as q6k
    assert q6k.q6k_act_bytes(1, 256) == (128 * 256, 128 * 8 * 4)
    assert q6k.q6k_act_bytes(3314, 11008) == (3328 * 11008, 3328 * 344 * 4)
    assert q6k.q6k_act_bytes(0, 256) == (0, 0)
    assert q6k.q6k_act_bytes(5, 300) == (0, 0)
    assert q6k.q6k_weight_bytes(40, 512, 1) == 128 * 512 * 5 // 4
    assert q6k.q6k_weight_bytes(40, 512, 0) == 128 * 512
    assert q6k.q6k_weight_bytes(4096, 11008, 0) == 4096 * 11008
    assert q6k.q6k_weight_bytes(40, 512, 2) == 128 * 512 * 2 + 128 * 2 * 4
    assert q6k.q6k_weight_bytes(4096, 11008, 2) == 4096 * 11008 * 2 + 4096 * 43 * 4
    assert q6k.q6k_weight_bytes(40, 512, 3) == 0
    assert q6k.q6k_weight_bytes(40, 0, 1) == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


@pytest.mark.parametrize("args,status", [
    ((FAKE, 4, 300, 300, FAKE, 1 << 30, FAKE, 1 << 30, None), -2),   # k % 256
    ((FAKE, -1, 256, 256, FAKE, 1 << 30, FAKE, 1 << 30, None), -1),  # n < 0
    ((None, 4, 256, 256, FAKE, 1 << 30, FAKE, 1 << 30, None), -1),   # null x
    ((FAKE, 4, 256, 255, FAKE, 1 << 30, FAKE, 1 << 30, None), -1),   # ldx < k
    ((FAKE + 4, 4, 256, 256, FAKE, 1 << 30, FAKE, 1 << 30, None), -3),  # misaligned x
    ((FAKE, 4, 256, 258, FAKE, 1 << 30, FAKE, 1 << 30, None), -3),   # ldx % 4
    ((FAKE, 4, 256, 256, FAKE, 100, FAKE, 1 << 30, None), -4),       # xq too small
    ((FAKE, 4, 256, 256, FAKE, 1 << 30, FAKE, 100, None), -4),       # da too small
    ((None, 0, 256, 256, None, 0, None, 0, None), 0),                # empty: no-op
])
def test_quantize_act_errors(args, status):
    assert lib().q6k_quantize_act(*args) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, 4, 300, 300, FAKE, 1 << 30, FAKE, 1 << 30, FAKE, 1 << 30, None), -2),   # k % 256
    ((FAKE, -1, 256, 256, FAKE, 1 << 30, FAKE, 1 << 30, FAKE, 1 << 30, None), -1),  # n < 0
    ((FAKE, 4, 256, 256, FAKE, 1 << 30, FAKE, 1 << 30, None, 1 << 30, None), -1),   # null das
    ((FAKE, 4, 256, 256, FAKE, 1 << 30, FAKE, 1 << 30, FAKE + 4, 1 << 30, None), -3),  # das align
    ((FAKE, 4, 256, 256, FAKE, 1 << 30, FAKE, 1 << 30, FAKE, 100, None), -4),       # das too small
    ((FAKE, 4, 256, 256, FAKE, 1 << 30, FAKE, 100, FAKE, 1 << 30, None), -4),       # da too small
    ((FAKE, 4, 256, 255, FAKE, 1 << 30, FAKE, 1 << 30, FAKE, 1 << 30, None), -1),   # ldx < k
    ((None, 0, 256, 256, None, 0, None, 0, None, 0, None), 0),                      # empty: no-op
])
def test_q4k_quantize_act_errors(args, status):
    assert lib().q4k_quantize_act(*args) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, 4, 256, 3, FAKE, 1 << 30, None), -1),    # unknown layout
    ((FAKE, 4, 512 + 32, 1, FAKE, 1 << 30, None), -2),
    ((FAKE + 1, 4, 256, 1, FAKE, 1 << 30, None), -3),  # raw must be 2-byte aligned
    ((FAKE, 4, 256, 1, FAKE + 8, 1 << 30, None), -3),
    ((FAKE, 4, 256, 1, FAKE, 10, None), -4),
    ((None, 4, 256, 0, FAKE, 1 << 30, None), -1),
    ((None, 0, 256, 0, None, 0, None), 0),
])
def test_expand_errors(args, status):
    assert lib().q6k_expand_weights(*args) == status


BIG = 1 << 40  # a buffer size that passes every size check


def gemm_args(xq=FAKE, xqb=BIG, da=FAKE, dab=BIG, n=4, w=FAKE, wb=BIG, layout=1, m=8, k=256,
              y=FAKE, yb=BIG, ldy=8):
    # no workspace: every case below fails (or is empty) before the work split is planned
    return (xq, xqb, da, dab, n, w, wb, layout, m, k, y, yb, ldy, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(layout=3), -1),
    (dict(k=0), -2),
    (dict(ldy=7), -1),                 # ldy < m
    (dict(y=FAKE + 2), -3),            # y not 4-byte aligned
    (dict(da=FAKE + 4, ldy=10), -3),   # misaligned da
    (dict(xq=FAKE + 8), -3),
    (dict(xq=None), -1),
    (dict(y=None), -1),
    (dict(n=0), 0),                    # n = 0: no-op
    (dict(m=0), 0),                    # m = 0: no-op
    (dict(n=-4), -1),
    # buffer sizes (n = 4 tokens pad to 128: xq 128*256 B, da 128*8*4 B; m = 8 rows pad to 128)
    (dict(xqb=128 * 256 - 1), -4),
    (dict(dab=128 * 8 * 4 - 1), -4),
    (dict(wb=128 * 256 * 5 // 4 - 1), -4),             # layout 1: 1.25 B per weight
    (dict(layout=2, wb=128 * 256 * 2 + 128 * 4 - 1), -4),
    (dict(layout=0, wb=128 * 256 - 1), -4),                # layout 0: 1 B per weight
    (dict(yb=4 * (3 * 8 + 8) - 1), -4),                # y: (n-1)*ldy + m floats
    (dict(yb=4 * (3 * 10 + 8) - 1, ldy=10), -4),
    (dict(ldy=(1 << 40) + 1), -4),
])
def test_gemm_errors(kw, status):
    assert lib().q6k_gemm(*gemm_args(**kw)) == status


def test_gemm_one_byte_short_weights():
    # every other buffer at its exact size, the weights one byte short (a passing call would
    # launch on these fake pointers, so only the failing side is checked)
    L = lib()
    for layout, wb in ((0, 128 * 256), (1, 128 * 256 * 5 // 4), (2, 128 * 256 * 2 + 128 * 4)):
        assert L.q6k_gemm(*gemm_args(layout=layout, wb=wb - 1, xqb=128 * 256, dab=4096,
                                     yb=4 * 32)) == -4


def test_gemm_size_limits():
    # one 32-bit buffer range per operand tile: layout 2 needs k < 2^25 (k/32 x 2 KiB of digit
    # planes per row tile), layouts 0/1 k < 2^26; dimensions beyond 2^40 are rejected outright
    L = lib()
    for layout, kmax in ((2, 1 << 25), (1, 1 << 26), (0, 1 << 26)):
        assert L.q6k_gemm(*gemm_args(layout=layout, k=kmax)) == -4
    assert L.q6k_gemm_chunkdots(FAKE, BIG, FAKE, BIG, 4, FAKE, BIG, 2, 8, 1 << 25, 0, 4, 0, 8,
                                FAKE, BIG, None) == -4
    assert L.q6k_gemm(*gemm_args(layout=2, n=(1 << 40) + 1)) == -4
    assert L.q6k_gemm(*gemm_args(layout=2, m=(1 << 40) + 1, ldy=(1 << 40) + 1)) == -4
    assert L.q4k_gemm(FAKE, BIG, FAKE, BIG, FAKE, BIG, 4, FAKE, BIG, 8, 1 << 26, FAKE, BIG, 8,
                      None, 0, None) == -4


def test_workspace_query_errors():
    # shape errors come before the device is asked for its compute units; *bytes is 0 on error
    L = lib()
    out = ctypes.c_size_t(123)
    for args, status in (((4, 8, 100, 1), -2), ((4, 8, 256, 3), -1), ((-1, 8, 256, 1), -1),
                         ((4, 8, 1 << 25, 2), -4), ((0, 8, 256, 1), 0), ((4, 0, 256, 2), 0)):
        out.value = 123
        assert L.q6k_gemm_workspace(*args, ctypes.byref(out)) == status, args
        assert out.value == 0, args
    assert L.q6k_gemm_workspace(4, 8, 256, 1, None) == -1
    for args, status in (((4, 8, 100), -2), ((4, 8, 1 << 26), -4), ((0, 8, 256), 0)):
        out.value = 123
        assert L.q4k_gemm_workspace(*args, ctypes.byref(out)) == status, args
        assert out.value == 0, args
    assert L.q4k_gemm_workspace(4, 8, 256, None) == -1


def test_noalloc_errors():
    # the argument rules of q6k_gemm; shape errors come before the device is asked for anything
    L = lib()

    def call(**kw):
        return L.q6k_gemm_noalloc(*(gemm_args(**kw)[:13] + (None,)))
    assert call(layout=3) == -1
    assert call(k=100) == -2
    assert call(n=-1) == -1
    assert call(layout=2, k=1 << 25) == -4
    assert call(n=0) == 0 and call(m=0) == 0
    assert L.q6k_strerror(-6) and b"scratch" in L.q6k_strerror(-6)


def dots_args(layout, win=(0, 4, 0, 8), dots=FAKE, dotsb=BIG, k=256, n=4, m=8):
    return (FAKE, BIG, FAKE, BIG, n, FAKE, BIG, layout, m, k, *win, dots, dotsb, None)


def test_subdots_errors():
    L = lib()
    assert L.q6k_gemm_subdots(*dots_args(1, dots=None)) == -1
    assert L.q6k_gemm_subdots(*dots_args(1, dots=FAKE + 2)) == -3
    assert L.q6k_gemm_subdots(*dots_args(1, k=100)) == -2
    assert L.q6k_gemm_subdots(*dots_args(2)) == -1  # layout 2 never forms them
    # the window must lie inside the problem, and the buffer hold ntok * nrow * k/16 int32
    assert L.q6k_gemm_subdots(*dots_args(1, win=(1, 4, 0, 8))) == -1
    assert L.q6k_gemm_subdots(*dots_args(1, win=(0, 4, 4, 5))) == -1
    assert L.q6k_gemm_subdots(*dots_args(1, win=(-1, 2, 0, 8))) == -1
    assert L.q6k_gemm_subdots(*dots_args(1, win=(2, 2, 3, 5), dotsb=4 * 2 * 5 * 16 - 1)) == -4
    assert L.q6k_gemm_subdots(*dots_args(1, win=(2, 0, 3, 5), dots=None)) == 0  # empty window


def test_chunkdots_errors():
    L = lib()
    assert L.q6k_gemm_chunkdots(*dots_args(2, dots=None)) == -1
    assert L.q6k_gemm_chunkdots(*dots_args(2, dots=FAKE + 2)) == -3
    assert L.q6k_gemm_chunkdots(*dots_args(2, k=100)) == -2
    for layout in (0, 1, 3):  # only layout 2 forms the per-chunk numerators
        assert L.q6k_gemm_chunkdots(*dots_args(layout)) == -1
    assert L.q6k_gemm_chunkdots(*dots_args(2, win=(0, 4, 0, 8), dotsb=4 * 4 * 8 * 8 - 1)) == -4
    assert L.q6k_gemm_chunkdots(*dots_args(2, win=(0, 5, 0, 8))) == -1


def test_strerror_and_stats():
    import q6_int8_prefill_amd as q6k
    for s in (0, -1, -2, -3, -4, -5, 42):
        assert isinstance(q6k.q6k_strerror(s), str) and q6k.q6k_strerror(s)
    counts = q6k.q6k_stats()
    assert len(counts) == 3 and all(c >= 0 for c in counts)


def test_swiglu_errors():
    L = lib()
    good = (FAKE, FAKE, 4, 256, 256, FAKE, 1 << 30, FAKE, 1 << 30, None)
    assert L.q6k_swiglu_quantize_act(*good[:2], 4, 300, 300, *good[5:]) == -2       # k % 256
    assert L.q6k_swiglu_quantize_act(FAKE, None, *good[2:]) == -1                   # null up
    assert L.q6k_swiglu_quantize_act(FAKE, FAKE + 4, *good[2:]) == -3               # misaligned up
    assert L.q6k_swiglu_quantize_act(FAKE + 4, FAKE, *good[2:]) == -3               # misaligned gate
    assert L.q6k_swiglu_quantize_act(FAKE, FAKE, 4, 256, 255, *good[5:]) == -1      # ld < k
    assert L.q6k_swiglu_quantize_act(FAKE, FAKE, 4, 256, 256, FAKE, 100, FAKE, 1 << 30, None) == -4
    assert L.q6k_swiglu_quantize_act(None, None, 0, 256, 256, None, 0, None, 0, None) == 0
    assert L.q6k_swiglu_f32(FAKE, FAKE, 4, 256, 255, FAKE, 256, None) == -1
    assert L.q6k_swiglu_f32(FAKE, FAKE, 4, 256, 256, FAKE + 2, 256, None) == -3
    assert L.q6k_swiglu_f32(FAKE, FAKE, 0, 256, 256, None, 256, None) == 0


def test_q4k_sizes_and_errors():
    import q6_int8_prefill_amd as q6k
    L = lib()
    assert q6k.q4k_weight_bytes(40, 512) == 128 * 512 + 128 * 16 * 8
    assert q6k.q4k_weight_bytes(40, 300) == 0
    assert L.q4k_expand_weights(FAKE, 4, 300, FAKE, 1 << 30, None) == -2
    assert L.q4k_expand_weights(FAKE + 8, 4, 256, FAKE, 1 << 30, None) == -3
    assert L.q4k_expand_weights(FAKE, 4, 256, FAKE, 10, None) == -4
    assert L.q4k_expand_weights(None, 0, 256, None, 0, None) == 0
    assert L.q4k_act_sums(FAKE, FAKE, 4, 256, FAKE, 10, None) == -4
    assert L.q4k_act_sums(FAKE, FAKE + 4, 4, 256, FAKE, 1 << 30, None) == -3
    def q4(xq=FAKE, da=FAKE, das=FAKE, n=4, k=256, ldy=8, wb=BIG, yb=BIG, dab=BIG):
        return L.q4k_gemm(xq, BIG, da, dab, das, dab, n, FAKE, wb, 8, k, FAKE, yb, ldy, None, 0,
                          None)
    assert q4(das=None) == -1                     # null das
    assert q4(ldy=7) == -1                        # ldy < m
    assert q4(k=100) == -2
    assert q4(n=0) == 0
    assert q4(wb=128 * 256 + 128 * 8 * 8 - 1) == -4
    assert q4(dab=128 * 8 * 4 - 1) == -4
    assert q4(yb=4 * (3 * 8 + 8) - 1) == -4
    assert L.q4k_gemm_dots(FAKE, BIG, 4, FAKE, BIG, 8, 256, 0, 4, 0, 8, None, BIG, None) == -1
    assert L.q4k_gemm_dots(FAKE, BIG, 4, FAKE, BIG, 8, 256, 0, 4, 0, 9, FAKE, BIG, None) == -1
    assert L.q4k_gemm_dots(FAKE, BIG, 4, FAKE, BIG, 8, 256, 0, 4, 0, 8, FAKE, 4 * 4 * 8 * 8 - 1,
                           None) == -4
    assert q6k.q4k_launches() >= 0


def test_binding_rejects_views_that_outrun_their_storage():
    # checked in Python before any pointer reaches the library (CPU tensors suffice: the shape
    # checks come before the device check)
    import torch
    import q6_int8_prefill_amd as q6k
    n, m, k = 64, 128, 256
    xb, db = q6k.q6k_act_bytes(n, k)
    wb = q6k.q6k_weight_bytes(m, k, 2)
    one = torch.zeros(1, dtype=torch.uint8)
    xq_exp = one.expand(xb)                     # numel large enough, storage one byte
    da = torch.zeros(db // 4, dtype=torch.float32)
    w = torch.zeros(wb, dtype=torch.uint8)
    y = torch.zeros((n, m), dtype=torch.float32)
    with pytest.raises(ValueError, match="contiguous"):
        q6k.q6k_gemm(xq_exp, da, n, w, 2, m, k, y)
    with pytest.raises(ValueError, match="contiguous"):
        q6k.q6k_gemm(torch.zeros(xb, dtype=torch.uint8), da, n, one.expand(wb), 2, m, k, y)
    with pytest.raises(ValueError, match="contiguous"):
        q6k.q6k_quantize_act(torch.zeros((n, k)), xq_exp, da)
    with pytest.raises(ValueError, match="contiguous"):
        q6k.q4k_act_sums(xq_exp, da, n, k, da.clone())
    with pytest.raises(ValueError, match="row-major"):
        q6k.q6k_gemm(torch.zeros(xb, dtype=torch.uint8), da, n, w, 2, m, k,
                     torch.zeros((m, n), dtype=torch.float32).t())
    # an explicit row stride that runs the activation rows past the tensor's storage
    with pytest.raises(ValueError, match="past its storage"):
        q6k.q6k_quantize_act(torch.zeros((n, k)), torch.zeros(xb, dtype=torch.uint8), da,
                             ldx=2 * k)
