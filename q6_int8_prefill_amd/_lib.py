"""ctypes marshalling for libq6k.so; names match the C entry points of include/q6k.h."""
import ctypes
import os

import torch

LAYOUT_PACKED = 0
LAYOUT_EXPANDED = 1
LAYOUT_FOLDED = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "_build", "libq6k.so")

if not os.path.exists(lib_path):
    raise ImportError(f"libq6k.so is not built ({lib_path}); run __graft_entry__.build()")

_p, _i64, _sz, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
_WIN = [_i64, _i64, _i64, _i64]


def _declare(lib):
    """Result and argument types of every call of q6k.h and q4k.h on a loaded library."""
    lib.q6k_act_bytes.restype = _sz
    lib.q6k_act_bytes.argtypes = [_i64, _i64, ctypes.POINTER(_sz)]
    lib.q6k_quantize_act.restype = _int
    lib.q6k_quantize_act.argtypes = [_p, _i64, _i64, _i64, _p, _sz, _p, _sz, _p]
    lib.q6k_swiglu_quantize_act.restype = _int
    lib.q6k_swiglu_quantize_act.argtypes = [_p, _p, _i64, _i64, _i64, _p, _sz, _p, _sz, _p]
    lib.q6k_swiglu_f32.restype = _int
    lib.q6k_swiglu_f32.argtypes = [_p, _p, _i64, _i64, _i64, _p, _i64, _p]
    lib.q6k_weight_bytes.restype = _sz
    lib.q6k_weight_bytes.argtypes = [_i64, _i64, _int]
    lib.q6k_expand_weights.restype = _int
    lib.q6k_expand_weights.argtypes = [_p, _i64, _i64, _int, _p, _sz, _p]
    lib.q6k_gemm.restype = _int
    lib.q6k_gemm.argtypes = [_p, _sz, _p, _sz, _i64, _p, _sz, _int, _i64, _i64, _p, _sz, _i64, _p,
                             _sz, _p]
    lib.q6k_gemm_noalloc.restype = _int
    lib.q6k_gemm_noalloc.argtypes = [_p, _sz, _p, _sz, _i64, _p, _sz, _int, _i64, _i64, _p, _sz,
                                     _i64, _p]
    lib.q6k_gemm_workspace.restype = _int
    lib.q6k_gemm_workspace.argtypes = [_i64, _i64, _i64, _int, ctypes.POINTER(_sz)]
    lib.q6k_gemm_subdots.restype = _int
    lib.q6k_gemm_subdots.argtypes = [_p, _sz, _p, _sz, _i64, _p, _sz, _int, _i64, _i64] + \
        _WIN + [_p, _sz, _p]
    lib.q6k_gemm_chunkdots.restype = _int
    lib.q6k_gemm_chunkdots.argtypes = [_p, _sz, _p, _sz, _i64, _p, _sz, _int, _i64, _i64] + \
        _WIN + [_p, _sz, _p]
    lib.q4k_weight_bytes.restype = _sz
    lib.q4k_weight_bytes.argtypes = [_i64, _i64]
    lib.q4k_expand_weights.restype = _int
    lib.q4k_expand_weights.argtypes = [_p, _i64, _i64, _p, _sz, _p]
    lib.q4k_quantize_act.restype = _int
    lib.q4k_quantize_act.argtypes = [_p, _i64, _i64, _i64, _p, _sz, _p, _sz, _p, _sz, _p]
    lib.q4k_act_sums.restype = _int
    lib.q4k_act_sums.argtypes = [_p, _p, _i64, _i64, _p, _sz, _p]
    lib.q4k_gemm.restype = _int
    lib.q4k_gemm.argtypes = [_p, _sz, _p, _sz, _p, _sz, _i64, _p, _sz, _i64, _i64, _p, _sz, _i64,
                             _p, _sz, _p]
    lib.q4k_gemm_workspace.restype = _int
    lib.q4k_gemm_workspace.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_sz)]
    lib.q4k_gemm_dots.restype = _int
    lib.q4k_gemm_dots.argtypes = [_p, _sz, _i64, _p, _sz, _i64, _i64] + _WIN + [_p, _sz, _p]
    lib.q4k_launches.restype = ctypes.c_uint64
    lib.q4k_launches.argtypes = []
    lib.q6k_strerror.restype = ctypes.c_char_p
    lib.q6k_strerror.argtypes = [_int]
    lib.q6k_stats.restype = None
    lib.q6k_stats.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    return lib


_lib = _declare(ctypes.CDLL(lib_path))


def use_library(path):
    """Send every call of this module to the library at `path` from now on, and return its
    handle.  For libq6k_timeline.so: a second build of the same source, with the same calls,
    whose GEMM workgroups also record where and when they ran (include/q6k_timeline.h)."""
    global _lib
    _lib = _declare(ctypes.CDLL(path))
    return _lib


EXPORTS = ("q6k_act_bytes", "q6k_quantize_act", "q6k_swiglu_quantize_act", "q6k_swiglu_f32",
           "q6k_weight_bytes", "q6k_expand_weights",
           "q6k_gemm_workspace", "q6k_gemm", "q6k_gemm_noalloc", "q6k_gemm_subdots",
           "q6k_gemm_chunkdots",
           "q6k_strerror", "q6k_stats",
           "q4k_weight_bytes", "q4k_expand_weights", "q4k_quantize_act", "q4k_act_sums",
           "q4k_gemm_workspace", "q4k_gemm", "q4k_gemm_dots", "q4k_launches")


class Q6KError(RuntimeError):
    def __init__(self, status, func):
        self.status = status
        super().__init__(f"{func}: {q6k_strerror(status)} (status {status})")


def _check(status, func):
    if status != 0:
        raise Q6KError(status, func)


def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.numel() and not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    return t.data_ptr() if t.numel() else None


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _span(t):
    """Bytes addressable from a tensor's first element to the end of its storage (the size of a
    row-major operand whose rows are strided views of a larger buffer)."""
    if t is None or not t.numel():
        return 0
    return t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()


def _flat(**bufs):
    """Buffers the kernels address as plain byte ranges from their first element must be
    contiguous (an expanded or strided view would let them run past the tensor's storage)."""
    for name, t in bufs.items():
        if t is not None and t.numel() and not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous buffer")


def _rows_fit(name, t, rows, cols, ld):
    """A row-major [rows][ld] operand: its last row must end inside the tensor's storage."""
    if rows <= 0 or cols <= 0 or t is None or not t.numel():
        return
    span = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    if ((rows - 1) * ld + cols) * t.element_size() > span:
        raise ValueError(f"{name}: {rows} rows of stride {ld} run past its storage")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def q6k_strerror(status):
    return _lib.q6k_strerror(int(status)).decode()


def q6k_act_bytes(n, k):
    """-> (xq bytes, da bytes); (0, 0) for an invalid shape."""
    da = _sz(0)
    xb = _lib.q6k_act_bytes(int(n), int(k), ctypes.byref(da))
    return int(xb), int(da.value)


def q6k_weight_bytes(m, k, layout):
    return int(_lib.q6k_weight_bytes(int(m), int(k), int(layout)))


def _x_operand(x, n, k, ldx):
    """Shape checks of an f32 [n][ldx] activation operand; returns (n, k, ldx)."""
    if x.dtype != torch.float32:
        raise TypeError("x must be float32")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [n][ldx]")
    n = x.shape[0] if n is None else n
    k = x.shape[1] if k is None else k
    ldx = x.stride(0) if ldx is None else ldx
    if x.numel() and x.stride(1) != 1:
        raise ValueError("x must be row-major")
    if x.numel() and (n > x.shape[0] or k > x.shape[1]):
        raise ValueError("n, k exceed the shape of x")
    _rows_fit("x", x, n, k, ldx)
    return n, k, ldx


def q6k_quantize_act(x, xq, da, n=None, k=None, ldx=None, stream=None):
    """x f32 [n][ldx] (device) -> tiled xq (uint8 buffer) and da (f32 buffer)."""
    n, k, ldx = _x_operand(x, n, k, ldx)
    _flat(xq=xq, da=da)
    _check(_lib.q6k_quantize_act(_ptr(x), n, k, ldx, _ptr(xq), _nbytes(xq), _ptr(da),
                                 _nbytes(da), _stream(stream)), "q6k_quantize_act")


def _rows_f32(name, t, n, k):
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [n][ld]")
    if t.numel() and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major")
    if t.numel() and (n > t.shape[0] or k > t.shape[1]):
        raise ValueError(f"n, k exceed the shape of {name}")
    _rows_fit(name, t, n, k, t.stride(0))


def q6k_swiglu_quantize_act(gate, up, xq, da, n=None, k=None, stream=None):
    """gate, up f32 [n][ld] (device, same strides) -> tiled xq, da of h = up * silu(gate)."""
    n = gate.shape[0] if n is None else n
    k = gate.shape[1] if k is None else k
    _rows_f32("gate", gate, n, k)
    _rows_f32("up", up, n, k)
    if gate.stride(0) != up.stride(0):
        raise ValueError("gate and up must share their row stride")
    _flat(xq=xq, da=da)
    _check(_lib.q6k_swiglu_quantize_act(_ptr(gate), _ptr(up), n, k, gate.stride(0), _ptr(xq),
                                        _nbytes(xq), _ptr(da), _nbytes(da), _stream(stream)),
           "q6k_swiglu_quantize_act")


def q6k_swiglu_f32(gate, up, h, stream=None):
    """Test-only: h = up * silu(gate) as the fused producer forms it (f32 [n][k] tensors)."""
    n, k = gate.shape
    _rows_f32("gate", gate, n, k)
    _rows_f32("up", up, n, k)
    _rows_f32("h", h, n, k)
    if gate.stride(0) != up.stride(0):
        raise ValueError("gate and up must share their row stride")
    _check(_lib.q6k_swiglu_f32(_ptr(gate), _ptr(up), n, k, gate.stride(0), _ptr(h), h.stride(0),
                               _stream(stream)), "q6k_swiglu_f32")


def q6k_expand_weights(w_raw, m, k, layout, w_out, stream=None):
    """raw q6_K bytes (device uint8, m*(k/256)*210 B) -> prepared weights in `layout`."""
    _flat(w_raw=w_raw, w_out=w_out)
    if w_raw is not None and w_raw.numel() and _nbytes(w_raw) < m * (k // 256) * 210:
        raise ValueError("raw weight buffer too small")
    _check(_lib.q6k_expand_weights(_ptr(w_raw), m, k, layout, _ptr(w_out), _nbytes(w_out),
                                   _stream(stream)), "q6k_expand_weights")


def _y_operand(y, n, m, ldy):
    """y f32 row-major [n][ldy]; -> ldy."""
    if y is not None and y.dtype != torch.float32:
        raise TypeError("y must be float32")
    if ldy is None:
        ldy = y.stride(0) if y is not None and y.dim() == 2 else m
    if y is not None and y.dim() == 2 and y.numel() and y.stride(1) != 1:
        raise ValueError("y must be row-major")
    return ldy


def q6k_gemm_workspace(n, m, k, layout):
    """-> workspace bytes q6k_gemm needs for this problem on the current device (0: none)."""
    out = _sz(0)
    _check(_lib.q6k_gemm_workspace(int(n), int(m), int(k), int(layout), ctypes.byref(out)),
           "q6k_gemm_workspace")
    return int(out.value)


def _workspace(workspace, need, like):
    """The caller's workspace (a flat device buffer), or a fresh one of `need` bytes on the device
    of `like` (from torch's caching allocator) when none is given."""
    if workspace is None:
        if need == 0:
            return None
        return torch.empty(need, dtype=torch.uint8, device=like.device)
    _flat(workspace=workspace)
    return workspace


def q6k_gemm(xq, da, n, w, layout, m, k, y, ldy=None, stream=None, workspace=None):
    """y f32 [n][ldy] = GEMM of prepared activations and weights.  `workspace`: a device buffer of
    at least q6k_gemm_workspace(n, m, k, layout) bytes, allocated here when not given."""
    ldy = _y_operand(y, n, m, ldy)
    _flat(xq=xq, da=da, w=w)
    need = q6k_gemm_workspace(n, m, k, layout) if workspace is None and y is not None else 0
    ws = _workspace(workspace, need, y)
    _check(_lib.q6k_gemm(_ptr(xq), _nbytes(xq), _ptr(da), _nbytes(da), n, _ptr(w), _nbytes(w),
                         layout, m, k, _ptr(y), _span(y), ldy, _ptr(ws), _nbytes(ws),
                         _stream(stream)), "q6k_gemm")


def q6k_gemm_noalloc(xq, da, n, w, layout, m, k, y, ldy=None, stream=None):
    """q6k_gemm with the split-k workspace in the library's static device array (allocates
    nothing; calls that overlap on one GPU race)."""
    ldy = _y_operand(y, n, m, ldy)
    _flat(xq=xq, da=da, w=w)
    _check(_lib.q6k_gemm_noalloc(_ptr(xq), _nbytes(xq), _ptr(da), _nbytes(da), n, _ptr(w),
                                 _nbytes(w), layout, m, k, _ptr(y), _span(y), ldy,
                                 _stream(stream)), "q6k_gemm_noalloc")


def _window(n, m, tok0, ntok, row0, nrow):
    ntok = n - tok0 if ntok is None else ntok
    nrow = m - row0 if nrow is None else nrow
    return [int(tok0), int(ntok), int(row0), int(nrow)]


def q6k_gemm_subdots(xq, da, n, w, layout, m, k, dots, tok0=0, ntok=None, row0=0, nrow=None,
                     stream=None):
    """Test-only: int32 sub-block dots [ntok][nrow][k/16] of a window of the problem (default: all
    of it), from the GEMM kernel source launched as q6k_gemm launches it."""
    if dots is not None and dots.dtype != torch.int32:
        raise TypeError("dots must be int32")
    _flat(xq=xq, da=da, w=w, dots=dots)
    _check(_lib.q6k_gemm_subdots(_ptr(xq), _nbytes(xq), _ptr(da), _nbytes(da), n, _ptr(w),
                                 _nbytes(w), layout, m, k, *_window(n, m, tok0, ntok, row0, nrow),
                                 _ptr(dots), _nbytes(dots), _stream(stream)), "q6k_gemm_subdots")


def q6k_gemm_chunkdots(xq, da, n, w, layout, m, k, dots, tok0=0, ntok=None, row0=0, nrow=None,
                       stream=None):
    """Test-only: int32 per-chunk numerators [ntok][nrow][k/32] of a window of the problem
    (default: all of it), from the layout-2 kernel source launched as q6k_gemm launches it."""
    if dots is not None and dots.dtype != torch.int32:
        raise TypeError("dots must be int32")
    _flat(xq=xq, da=da, w=w, dots=dots)
    _check(_lib.q6k_gemm_chunkdots(_ptr(xq), _nbytes(xq), _ptr(da), _nbytes(da), n, _ptr(w),
                                   _nbytes(w), layout, m, k,
                                   *_window(n, m, tok0, ntok, row0, nrow), _ptr(dots),
                                   _nbytes(dots), _stream(stream)), "q6k_gemm_chunkdots")


def q6k_stats():
    """-> launch counts per layout (layout 0, 1, 2)."""
    out = (ctypes.c_uint64 * 3)()
    _lib.q6k_stats(out)
    return tuple(int(v) for v in out)


# ------------------------------------------------------------------------------------------------
# q4_K variant (include/q4k.h)
# ------------------------------------------------------------------------------------------------
def q4k_weight_bytes(m, k):
    return int(_lib.q4k_weight_bytes(int(m), int(k)))


def q4k_expand_weights(w_raw, m, k, w_out, stream=None):
    """raw q4_K bytes (device uint8, m*(k/256)*144 B) -> prepared codes + (d*sc, -dmin*m) pairs."""
    _flat(w_raw=w_raw, w_out=w_out)
    if w_raw is not None and w_raw.numel() and _nbytes(w_raw) < m * (k // 256) * 144:
        raise ValueError("raw weight buffer too small")
    _check(_lib.q4k_expand_weights(_ptr(w_raw), m, k, _ptr(w_out), _nbytes(w_out),
                                   _stream(stream)), "q4k_expand_weights")


def q4k_quantize_act(x, xq, da, das, n=None, k=None, ldx=None, stream=None):
    """x f32 [n][ldx] (device) -> tiled xq, da and das = da * (sum of each chunk's codes)."""
    n, k, ldx = _x_operand(x, n, k, ldx)
    _flat(xq=xq, da=da, das=das)
    _check(_lib.q4k_quantize_act(_ptr(x), n, k, ldx, _ptr(xq), _nbytes(xq), _ptr(da),
                                 _nbytes(da), _ptr(das), _nbytes(das), _stream(stream)),
           "q4k_quantize_act")


def q4k_act_sums(xq, da, n, k, das, stream=None):
    """das = da * (sum of each chunk's codes), tiled like da."""
    _flat(xq=xq, da=da, das=das)
    xb, db = q6k_act_bytes(n, k)
    if n > 0 and xb and (_nbytes(xq) < xb or _nbytes(da) < db):
        raise ValueError("activation buffers too small")
    _check(_lib.q4k_act_sums(_ptr(xq), _ptr(da), n, k, _ptr(das), _nbytes(das), _stream(stream)),
           "q4k_act_sums")


def q4k_gemm_workspace(n, m, k):
    """-> workspace bytes q4k_gemm needs for this problem on the current device (0: none)."""
    out = _sz(0)
    _check(_lib.q4k_gemm_workspace(int(n), int(m), int(k), ctypes.byref(out)),
           "q4k_gemm_workspace")
    return int(out.value)


def q4k_gemm(xq, da, das, n, w, m, k, y, ldy=None, stream=None, workspace=None):
    """y f32 [n][ldy] = q4_K GEMM of prepared activations (xq, da, das) and weights; `workspace`
    as for q6k_gemm (q4k_gemm_workspace bytes)."""
    ldy = _y_operand(y, n, m, ldy)
    _flat(xq=xq, da=da, das=das, w=w)
    need = q4k_gemm_workspace(n, m, k) if workspace is None and y is not None else 0
    ws = _workspace(workspace, need, y)
    _check(_lib.q4k_gemm(_ptr(xq), _nbytes(xq), _ptr(da), _nbytes(da), _ptr(das), _nbytes(das), n,
                         _ptr(w), _nbytes(w), m, k, _ptr(y), _span(y), ldy, _ptr(ws), _nbytes(ws),
                         _stream(stream)), "q4k_gemm")


def q4k_gemm_dots(xq, n, w, m, k, dots, tok0=0, ntok=None, row0=0, nrow=None, stream=None):
    """Test-only: int32 chunk dots [ntok][nrow][k/32] of a window of the problem (default: all of
    it) from the q4_K GEMM kernel source."""
    if dots is not None and dots.dtype != torch.int32:
        raise TypeError("dots must be int32")
    _flat(xq=xq, w=w, dots=dots)
    _check(_lib.q4k_gemm_dots(_ptr(xq), _nbytes(xq), n, _ptr(w), _nbytes(w), m, k,
                              *_window(n, m, tok0, ntok, row0, nrow), _ptr(dots), _nbytes(dots),
                              _stream(stream)), "q4k_gemm_dots")


def q4k_launches():
    return int(_lib.q4k_launches())
