"""ctypes binding of libkfac (include/kfac.h): argument marshalling only.

Every function has the name of the C entry point it calls and takes torch tensors
that live on the current HIP device; it passes their data pointers, the sizes and
the current torch stream (or the one given) to the library, and raises KfacError
when the library returns a non-zero status. Nothing here computes any part of the
K-FAC step, and there is no fallback: without the built library, import fails.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkfac.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python fac_second_order_amd/build.py` "
        "(hipcc, gfx950) first. There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

KFAC_F16 = 0
KFAC_F32 = 1
KFAC_F64 = 2
_STATUS = {0: "KFAC_OK", -1: "KFAC_ERR_INVALID", -2: "KFAC_ERR_UNSUPPORTED",
           -3: "KFAC_ERR_WORKSPACE", -4: "KFAC_ERR_HIP"}


class KfacError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.kfac_last_error().decode(errors="replace")
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {msg}")


class kfac_layer(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in
                ("n", "h", "w", "c_in", "h_out", "w_out", "c_out",
                 "kh", "kw", "sh", "sw", "ph", "pw", "bias")]


class kfac_bn(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("hw", ctypes.c_int32), ("c", ctypes.c_int32)]


_c = ctypes
_vp, _i32, _sz, _f32 = _c.c_void_p, _c.c_int32, _c.c_size_t, _c.c_float
_P = _c.POINTER


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("kfac_version", _i32)
_sig("kfac_status_string", _c.c_char_p, _i32)
_sig("kfac_last_error", _c.c_char_p)
_sig("kfac_factors_workspace", _i32, _P(kfac_layer), _i32, _i32, _P(_sz))
_sig("kfac_factors", _i32, _P(kfac_layer), _i32, _i32, _P(_vp), _P(_vp), _P(_vp), _P(_vp), _f32,
     _vp, _sz, _vp)
_sig("kfac_factors_full", _i32, _P(kfac_layer), _i32, _i32, _P(_vp), _P(_vp), _P(_vp), _P(_vp), _P(_vp),
     _P(_vp), _f32, _vp, _sz, _vp)
_sig("kfac_pack_sym_workspace", _i32, _i32, _P(_i32), _P(_sz))
_sig("kfac_pack_sym", _i32, _i32, _P(_i32), _P(_vp), _P(_vp), _i32, _vp, _sz, _vp)
_sig("kfac_invert_workspace", _i32, _i32, _P(_i32), _P(_sz))
_sig("kfac_invert_schedule", _i32, _P(_i32), _P(_i32))
_sig("kfac_invert", _i32, _i32, _P(_i32), _P(_vp), _P(_vp), _P(_f32), _vp, _P(_vp), _vp, _sz, _vp)
_sig("kfac_invert_refine_workspace", _i32, _i32, _P(_i32), _P(_sz))
_sig("kfac_invert_refine", _i32, _i32, _P(_i32), _P(_vp), _P(_f32), _P(_vp), _vp, _sz, _vp)
_sig("kfac_precondition_workspace", _i32, _i32, _P(_i32), _P(_i32), _P(_sz))
_sig("kfac_precondition", _i32, _i32, _P(_i32), _P(_i32), _P(_vp), _P(_vp), _P(_vp), _i32, _P(_vp),
     _vp, _sz, _vp)
_sig("kfac_precondition_update", _i32, _i32, _P(_i32), _P(_i32), _P(_vp), _P(_vp), _P(_vp), _i32,
     _P(_vp), _P(_vp), _f32, _vp, _sz, _vp)
_sig("kfac_precondition_ex", _i32, _i32, _P(_i32), _P(_i32), _P(_vp), _P(_vp), _P(_vp), _i32,
     _P(_vp), _P(_vp), _f32, _i32, _vp, _sz, _vp)
_sig("kfac_bn_diag_workspace", _i32, _P(kfac_bn), _i32, _P(_sz))
_sig("kfac_bn_diag", _i32, _P(kfac_bn), _i32, _i32, _P(_vp), _P(_vp), _P(_vp), _P(_vp), _f32, _f32,
     _vp, _sz, _vp)
_sig("kfac_bn_update", _i32, _P(kfac_bn), _i32, _i32, _P(_vp), _P(_vp), _P(_vp), _P(_vp), _P(_vp),
     _f32, _f32, _f32, _vp, _sz, _vp)
_sig("kfac_bn_diag_noalloc", _i32, _P(kfac_bn), _i32, _i32, _P(_vp), _P(_vp), _P(_vp), _P(_vp), _P(_vp),
     _f32, _f32, _f32, _vp)
_sig("kfac_timing_kernels", _i32)
_sig("kfac_kernel_name", _c.c_char_p, _i32)
_sig("kfac_timing_enable", _i32, _i32)
_sig("kfac_timing_only", _i32, _i32)
_sig("kfac_timing_reset", _i32)
_sig("kfac_timing_read", _i32, _i32, _P(_c.c_double), _P(_c.c_int64))


def _check(status, where):
    if status != 0:
        raise KfacError(status, where)


def _ptrs(tensors):
    arr = (_vp * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i] = None if t is None else t.data_ptr()
    return arr


def _ints(vals):
    arr = (_i32 * max(1, len(vals)))()
    for i, v in enumerate(vals):
        arr[i] = int(v)
    return arr


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float16:
        return KFAC_F16
    if t.dtype == torch.float32:
        return KFAC_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _layers(layers):
    arr = (kfac_layer * max(1, len(layers)))()
    for i, l in enumerate(layers):
        for f, _ in kfac_layer._fields_:
            setattr(arr[i], f, int(getattr(l, f) if not isinstance(l, dict) else l[f]))
    return arr


def _bns(layers):
    arr = (kfac_bn * max(1, len(layers)))()
    for i, l in enumerate(layers):
        for f, _ in kfac_bn._fields_:
            setattr(arr[i], f, int(getattr(l, f) if not isinstance(l, dict) else l[f]))
    return arr


def _ws(workspace, nbytes, device):
    """The caller's workspace, or a fresh torch allocation of nbytes (256-aligned)."""
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    ptr = workspace.data_ptr()
    pad = (-ptr) % 256
    return _vp(ptr + pad), workspace.numel() * workspace.element_size() - pad


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def kfac_version():
    return _lib.kfac_version()


def kfac_factors_workspace(layers, in_dtype=KFAC_F16):
    out = _sz()
    _check(_lib.kfac_factors_workspace(_layers(layers), len(layers), in_dtype, _c.byref(out)),
           "kfac_factors_workspace")
    return out.value


def _factor_call_args(layers, act, gout, workspace):
    first = next(t for t in list(act) + list(gout) if t is not None)
    dt = _dtype_code(first)
    for t in list(act) + list(gout):
        if t is not None and (t.dtype != first.dtype or not t.is_contiguous()):
            raise TypeError("factor inputs must share one dtype and be contiguous")
    need = kfac_factors_workspace(layers, dt)
    ws, wsb = _ws(workspace, need, first.device)
    return dt, ws, wsb


def kfac_factors(layers, act, gout, A_packed, G_packed, ema_decay=0.0, workspace=None, stream=None):
    """A_packed[l], G_packed[l] <- packed factors of layer l (see kfac.h)."""
    dt, ws, wsb = _factor_call_args(layers, act, gout, workspace)
    _check(_lib.kfac_factors(_layers(layers), len(layers), dt, _ptrs(act), _ptrs(gout),
                             _ptrs(A_packed), _ptrs(G_packed), float(ema_decay), ws, wsb,
                             _stream(stream)), "kfac_factors")


def kfac_factors_full(layers, act, gout, A_packed, G_packed, A_full, G_full, ema_decay=0.0, workspace=None,
                      stream=None):
    """kfac_factors that also writes the upper triangle of each factor into A_full[l] /
    G_full[l] (d x d fp32, row-major; None entries skip it; see kfac.h)."""
    dt, ws, wsb = _factor_call_args(layers, act, gout, workspace)
    orders = [(l.c_in * l.kh * l.kw + (1 if l.bias else 0), l.c_out) for l in layers]
    if len(A_full) != len(layers) or len(G_full) != len(layers):
        raise ValueError("A_full and G_full need one entry per layer")
    for (da, dg), fa, fg in zip(orders, A_full, G_full):
        for t, d in ((fa, da), (fg, dg)):
            if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != d * d):
                raise TypeError("full factor outputs must be contiguous float32 d x d")
    _check(_lib.kfac_factors_full(_layers(layers), len(layers), dt, _ptrs(act), _ptrs(gout),
                                  _ptrs(A_packed), _ptrs(G_packed), _ptrs(A_full), _ptrs(G_full),
                                  float(ema_decay), ws, wsb, _stream(stream)), "kfac_factors_full")


def kfac_pack_sym_workspace(n):
    out = _sz()
    _check(_lib.kfac_pack_sym_workspace(len(n), _ints(n), _c.byref(out)), "kfac_pack_sym_workspace")
    return out.value


def kfac_pack_sym(n, full, packed, direction, workspace=None, stream=None):
    """direction 0: packed <- upper(full); 1: full <- symmetric(packed); 2: upper(full)
    <- packed, strict lower triangle of full left as it was."""
    need = kfac_pack_sym_workspace(n)
    ws, wsb = _ws(workspace, need, full[0].device if full else None)
    _check(_lib.kfac_pack_sym(len(n), _ints(n), _ptrs(full), _ptrs(packed), int(direction), ws, wsb,
                              _stream(stream)), "kfac_pack_sym")


def kfac_invert_workspace(n):
    out = _sz()
    _check(_lib.kfac_invert_workspace(len(n), _ints(n), _c.byref(out)), "kfac_invert_workspace")
    return out.value


def kfac_invert_schedule():
    """(block size, block steps per update launch) of kfac_invert."""
    b, g = _i32(), _i32()
    _check(_lib.kfac_invert_schedule(_c.byref(b), _c.byref(g)), "kfac_invert_schedule")
    return b.value, g.value


def kfac_invert_refine_workspace(n):
    out = _sz()
    _check(_lib.kfac_invert_refine_workspace(len(n), _ints(n), _c.byref(out)), "kfac_invert_refine_workspace")
    return out.value


def kfac_invert_refine(n, mat, shift, inv, workspace=None, stream=None):
    """inv[m] <- X + X (I - (mat[m] + shift[m] I) X), X = inv[m] (see kfac.h)."""
    need = kfac_invert_refine_workspace(n)
    ws, wsb = _ws(workspace, need, inv[0].device)
    shifts = (_f32 * len(n))(*[float(v) for v in shift])
    _check(_lib.kfac_invert_refine(len(n), _ints(n), _ptrs(mat), shifts, _ptrs(inv), ws, wsb, _stream(stream)),
           "kfac_invert_refine")


def kfac_invert(n, mat, inv, shift, info, chol=None, workspace=None, stream=None):
    """inv[m] <- (sym(mat[m]) + shift[m] I)^-1; info (int32 device tensor) <- breakdown index."""
    need = kfac_invert_workspace(n)
    ws, wsb = _ws(workspace, need, mat[0].device if mat else None)
    sh = (_f32 * max(1, len(n)))(*[float(s) for s in shift])
    if info.dtype != torch.int32 or info.numel() < len(n):
        raise TypeError("info must be an int32 tensor with one entry per matrix")
    _check(_lib.kfac_invert(len(n), _ints(n), _ptrs(mat), _ptrs(inv), sh, _vp(info.data_ptr()),
                            _ptrs(chol) if chol is not None else None, ws, wsb, _stream(stream)),
           "kfac_invert")


def kfac_precondition_workspace(d_g, d_a):
    out = _sz()
    _check(_lib.kfac_precondition_workspace(len(d_g), _ints(d_g), _ints(d_a), _c.byref(out)),
           "kfac_precondition_workspace")
    return out.value


def kfac_precondition(d_g, d_a, G_inv, A_inv, grad, out, workspace=None, stream=None):
    """out[l] <- G_inv[l] @ grad[l] @ A_inv[l] (fp32)."""
    dt = _dtype_code(grad[0])
    need = kfac_precondition_workspace(d_g, d_a)
    ws, wsb = _ws(workspace, need, grad[0].device)
    _check(_lib.kfac_precondition(len(d_g), _ints(d_g), _ints(d_a), _ptrs(G_inv), _ptrs(A_inv),
                                  _ptrs(grad), dt, _ptrs(out), ws, wsb, _stream(stream)),
           "kfac_precondition")


def kfac_precondition_update(d_g, d_a, G_inv, A_inv, grad, out, w, lr, workspace=None, stream=None):
    """w[l] <- w[l] - lr * G_inv[l] @ grad[l] @ A_inv[l]; out[l] <- the product unless out is None."""
    dt = _dtype_code(grad[0])
    need = kfac_precondition_workspace(d_g, d_a)
    ws, wsb = _ws(workspace, need, grad[0].device)
    _check(_lib.kfac_precondition_update(len(d_g), _ints(d_g), _ints(d_a), _ptrs(G_inv), _ptrs(A_inv),
                                         _ptrs(grad), dt, None if out is None else _ptrs(out), _ptrs(w),
                                         float(lr), ws, wsb, _stream(stream)),
           "kfac_precondition_update")


def kfac_precondition_ex(d_g, d_a, G_inv, A_inv, grad, out, w=None, lr=0.0, accum=KFAC_F32, workspace=None,
                         stream=None):
    """kfac_precondition (w None) or kfac_precondition_update (w given), the products
    summed in fp32 (accum KFAC_F32) or fp64 (KFAC_F64)."""
    dt = _dtype_code(grad[0])
    need = kfac_precondition_workspace(d_g, d_a)
    ws, wsb = _ws(workspace, need, grad[0].device)
    _check(_lib.kfac_precondition_ex(len(d_g), _ints(d_g), _ints(d_a), _ptrs(G_inv), _ptrs(A_inv), _ptrs(grad), dt,
                                     None if out is None else _ptrs(out), None if w is None else _ptrs(w),
                                     float(lr), int(accum), ws, wsb, _stream(stream)), "kfac_precondition_ex")


def kfac_bn_diag_workspace(layers):
    out = _sz()
    _check(_lib.kfac_bn_diag_workspace(_bns(layers), len(layers), _c.byref(out)), "kfac_bn_diag_workspace")
    return out.value


def kfac_bn_diag(layers, xhat, gout, fisher, precond, ema_decay=0.0, shift=1e-3, workspace=None,
                 stream=None):
    """fisher[l], precond[l] ([2, c] fp32) <- BN diagonal Fisher and grad/(F+shift)."""
    dt = _dtype_code(xhat[0])
    need = kfac_bn_diag_workspace(layers)
    ws, wsb = _ws(workspace, need, xhat[0].device)
    _check(_lib.kfac_bn_diag(_bns(layers), len(layers), dt, _ptrs(xhat), _ptrs(gout), _ptrs(fisher),
                             _ptrs(precond), float(ema_decay), float(shift), ws, wsb, _stream(stream)),
           "kfac_bn_diag")


def kfac_bn_update(layers, xhat, gout, fisher, precond, params, lr, ema_decay=0.0, shift=1e-3,
                   workspace=None, stream=None):
    """kfac_bn_diag, then params[l] ([2, c] fp32: gamma, beta) <- params[l] - lr * precond[l]."""
    dt = _dtype_code(xhat[0])
    need = kfac_bn_diag_workspace(layers)
    ws, wsb = _ws(workspace, need, xhat[0].device)
    _check(_lib.kfac_bn_update(_bns(layers), len(layers), dt, _ptrs(xhat), _ptrs(gout), _ptrs(fisher),
                               _ptrs(precond), _ptrs(params), float(lr), float(ema_decay), float(shift),
                               ws, wsb, _stream(stream)), "kfac_bn_update")


KFAC_BN_NOALLOC_SCRATCH_BYTES = 16 << 20


def kfac_bn_diag_noalloc(layers, xhat, gout, fisher, precond, params=None, lr=0.0, ema_decay=0.0, shift=1e-3,
                         stream=None):
    """kfac_bn_diag (params None) or kfac_bn_update (params given) with the library's
    static scratch instead of a workspace: allocates nothing (see kfac.h)."""
    dt = _dtype_code(xhat[0])
    _check(_lib.kfac_bn_diag_noalloc(_bns(layers), len(layers), dt, _ptrs(xhat), _ptrs(gout), _ptrs(fisher),
                                     _ptrs(precond), None if params is None else _ptrs(params), float(lr),
                                     float(ema_decay), float(shift), _stream(stream)), "kfac_bn_diag_noalloc")


# timing -------------------------------------------------------------------

def kfac_timing_kernels():
    return _lib.kfac_timing_kernels()


def kfac_kernel_name(i):
    return _lib.kfac_kernel_name(int(i)).decode()


def kfac_timing_enable(on=True):
    _check(_lib.kfac_timing_enable(1 if on else 0), "kfac_timing_enable")


def kfac_timing_only(i=-1):
    """Time only kernel id i (-1: every kernel)."""
    _check(_lib.kfac_timing_only(int(i)), "kfac_timing_only")


def kfac_timing_reset():
    _check(_lib.kfac_timing_reset(), "kfac_timing_reset")


def kfac_timing_read(i):
    ms = _c.c_double()
    n = _c.c_int64()
    _check(_lib.kfac_timing_read(int(i), _c.byref(ms), _c.byref(n)), "kfac_timing_read")
    return ms.value, n.value
