"""Thin ctypes binding of libfourtune.so (include/fourtune.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI.  PyTorch provides device memory and the stream.  The
functions keep the C names; they take torch tensors (device memory) and
raise FourTuneError on any status other than FT_OK.  bf16 tensors may be
passed as torch.bfloat16 or as int16/uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfourtune.so")

FT_OK, FT_EINVAL, FT_ESHAPE, FT_EALIGN, FT_EWORKSPACE, FT_EDEVICE, FT_EUNSUPPORTED = range(7)
FT_BF16, FT_F32 = 0, 1
FT_Q_ROW32, FT_Q_ROW32_T, FT_Q_TILE32 = 1, 2, 4
FT_MAX_RANK = 128
FT_NOALLOC_SCRATCH_BYTES = 64 << 20
FT_ACT_NONE, FT_ACT_GELU_TANH = 0, 1
FT_W4A4G4, FT_W4A16G4, FT_W4A4G16, FT_W4A16G16 = 0, 1, 2, 3
FT_WBLOCK_TILE32, FT_WBLOCK_ROW32, FT_WBLOCK_TILE32_T = 0, 1, 2
PRECISION_NAMES = {"W4A4G4": FT_W4A4G4, "W4A16G4": FT_W4A16G4, "W4A4G16": FT_W4A4G16,
                   "W4A16G16": FT_W4A16G16}

EXPORTS = ("fourtune_quantize", "fourtune_dequantize", "fourtune_workspace_bytes", "fourtune_linear_fwd",
           "fourtune_linear_fwd_noalloc", "fourtune_linear_bwd", "fourtune_mlp_workspace_bytes",
           "fourtune_mlp_fwd", "fourtune_mlp_bwd_workspace_bytes", "fourtune_mlp_bwd",
           "fourtune_act_fwd", "fourtune_act_bwd",
           "fourtune_status_string", "fourtune_timing_enable", "fourtune_timing_reset",
           "fourtune_timing_read")


class FourTuneError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


class FtLinear(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("r_stab", ctypes.c_int32), ("r_lora", ctypes.c_int32),
                ("w_codes", ctypes.c_void_p), ("w_scales", ctypes.c_void_p),
                ("wt_codes", ctypes.c_void_p), ("wt_scales", ctypes.c_void_p),
                ("L1t", ctypes.c_void_p), ("L2", ctypes.c_void_p),
                ("At", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("act_in", ctypes.c_int32), ("act_out", ctypes.c_int32),
                ("precision", ctypes.c_int32), ("w_block", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfourtune.so once; fail loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.fourtune_quantize.argtypes = [st, vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.fourtune_quantize.restype = st
        L.fourtune_dequantize.argtypes = [st, vp, vp, i64, i64, vp, vp]
        L.fourtune_dequantize.restype = st
        L.fourtune_workspace_bytes.argtypes = [ctypes.POINTER(FtLinear), st]
        L.fourtune_workspace_bytes.restype = ctypes.c_size_t
        L.fourtune_linear_fwd.argtypes = [ctypes.POINTER(FtLinear), vp, vp, vp, vp, vp, vp,
                                          ctypes.c_size_t, vp]
        L.fourtune_linear_fwd.restype = st
        L.fourtune_linear_fwd_noalloc.argtypes = [ctypes.POINTER(FtLinear), vp, vp, vp, vp, vp, vp]
        L.fourtune_linear_fwd_noalloc.restype = st
        L.fourtune_linear_bwd.argtypes = [ctypes.POINTER(FtLinear), vp, vp, vp, vp, vp, vp, vp,
                                          st, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.fourtune_linear_bwd.restype = st
        L.fourtune_mlp_workspace_bytes.argtypes = [ctypes.POINTER(FtLinear), ctypes.POINTER(FtLinear)]
        L.fourtune_mlp_workspace_bytes.restype = ctypes.c_size_t
        L.fourtune_mlp_fwd.argtypes = [ctypes.POINTER(FtLinear), ctypes.POINTER(FtLinear), vp, vp, vp,
                                       vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.fourtune_mlp_fwd.restype = st
        L.fourtune_mlp_bwd_workspace_bytes.argtypes = [ctypes.POINTER(FtLinear), ctypes.POINTER(FtLinear)]
        L.fourtune_mlp_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.fourtune_mlp_bwd.argtypes = [ctypes.POINTER(FtLinear), ctypes.POINTER(FtLinear), vp, vp, vp,
                                       vp, vp, vp, vp, vp, vp, vp, st, vp, ctypes.c_size_t, vp]
        L.fourtune_mlp_bwd.restype = st
        L.fourtune_act_fwd.argtypes = [st, vp, i64, vp, vp]
        L.fourtune_act_fwd.restype = st
        L.fourtune_act_bwd.argtypes = [st, vp, vp, i64, vp, vp]
        L.fourtune_act_bwd.restype = st
        L.fourtune_status_string.argtypes = [st]
        L.fourtune_status_string.restype = ctypes.c_char_p
        L.fourtune_timing_enable.argtypes = [st]
        L.fourtune_timing_enable.restype = None
        L.fourtune_timing_reset.argtypes = []
        L.fourtune_timing_reset.restype = None
        L.fourtune_timing_read.argtypes = [ctypes.POINTER(ctypes.c_char_p),
                                           ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_int64), st]
        L.fourtune_timing_read.restype = st
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().fourtune_status_string(int(s)).decode()


fourtune_status_string = status_string


def _ptr(t) -> int | None:
    """Device address of a tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != FT_OK:
        raise FourTuneError(status, where)


def make_linear(M, K, N, r_stab, r_lora, w_codes, w_scales, wt_codes=None, wt_scales=None,
                L1t=None, L2=None, At=None, B=None, act_in=FT_ACT_NONE,
                act_out=FT_ACT_NONE, precision=FT_W4A4G4,
                w_block=FT_WBLOCK_TILE32) -> FtLinear:
    """Fill the ft_linear descriptor from tensors (device) or raw addresses.

    The factors are rank-major: L1t = L1^T [r_stab, K], L2 [r_stab, N],
    At = A^T [r_lora, K], B [r_lora, N].  precision: FT_W4A4G4 .. FT_W4A16G16
    or its name; w_block: FT_WBLOCK_TILE32, FT_WBLOCK_ROW32 or
    FT_WBLOCK_TILE32_T."""
    if isinstance(precision, str):
        precision = PRECISION_NAMES[precision]
    return FtLinear(int(M), int(K), int(N), int(r_stab), int(r_lora), _ptr(w_codes),
                    _ptr(w_scales), _ptr(wt_codes), _ptr(wt_scales), _ptr(L1t), _ptr(L2),
                    _ptr(At), _ptr(B), int(act_in), int(act_out), int(precision), int(w_block))


def fourtune_quantize(mode, x, rows, cols, ld, codes, scales, codes_t=None, scales_t=None,
                      stream=None):
    s = lib().fourtune_quantize(int(mode), _ptr(x), int(rows), int(cols), int(ld), _ptr(codes),
                                _ptr(scales), _ptr(codes_t), _ptr(scales_t), _stream(stream))
    _check(s, "fourtune_quantize")


def fourtune_dequantize(mode, codes, scales, rows, cols, out, stream=None):
    s = lib().fourtune_dequantize(int(mode), _ptr(codes), _ptr(scales), int(rows), int(cols),
                                  _ptr(out), _stream(stream))
    _check(s, "fourtune_dequantize")


def fourtune_workspace_bytes(layer: FtLinear, is_bwd: bool) -> int:
    return int(lib().fourtune_workspace_bytes(ctypes.byref(layer), int(bool(is_bwd))))


def fourtune_linear_fwd(layer: FtLinear, X, Y, U_save, xq_codes, xq_scales, workspace,
                        ws_bytes, stream=None):
    s = lib().fourtune_linear_fwd(ctypes.byref(layer), _ptr(X), _ptr(Y), _ptr(U_save),
                                  _ptr(xq_codes), _ptr(xq_scales), _ptr(workspace),
                                  int(ws_bytes), _stream(stream))
    _check(s, "fourtune_linear_fwd")


def fourtune_linear_fwd_noalloc(layer: FtLinear, X, Y, U_save, xq_codes, xq_scales, stream=None):
    s = lib().fourtune_linear_fwd_noalloc(ctypes.byref(layer), _ptr(X), _ptr(Y), _ptr(U_save),
                                          _ptr(xq_codes), _ptr(xq_scales), _stream(stream))
    _check(s, "fourtune_linear_fwd_noalloc")


def fourtune_linear_bwd(layer: FtLinear, dY, X, U_save, H, dX, dA, dB, grad_dtype, P_save,
                        gq_codes, gq_scales, workspace, ws_bytes, stream=None):
    s = lib().fourtune_linear_bwd(ctypes.byref(layer), _ptr(dY), _ptr(X), _ptr(U_save), _ptr(H),
                                  _ptr(dX), _ptr(dA), _ptr(dB), int(grad_dtype), _ptr(P_save),
                                  _ptr(gq_codes), _ptr(gq_scales), _ptr(workspace),
                                  int(ws_bytes), _stream(stream))
    _check(s, "fourtune_linear_bwd")


def fourtune_mlp_workspace_bytes(fc1: FtLinear, fc2: FtLinear) -> int:
    return int(lib().fourtune_mlp_workspace_bytes(ctypes.byref(fc1), ctypes.byref(fc2)))


def fourtune_mlp_fwd(fc1: FtLinear, fc2: FtLinear, X, H, Y, U1_save, U2_save, aq_codes, aq_scales,
                     workspace, ws_bytes, stream=None):
    s = lib().fourtune_mlp_fwd(ctypes.byref(fc1), ctypes.byref(fc2), _ptr(X), _ptr(H), _ptr(Y),
                               _ptr(U1_save), _ptr(U2_save), _ptr(aq_codes), _ptr(aq_scales),
                               _ptr(workspace), int(ws_bytes), _stream(stream))
    _check(s, "fourtune_mlp_fwd")


def fourtune_mlp_bwd_workspace_bytes(fc1: FtLinear, fc2: FtLinear) -> int:
    return int(lib().fourtune_mlp_bwd_workspace_bytes(ctypes.byref(fc1), ctypes.byref(fc2)))


def fourtune_mlp_bwd(fc1: FtLinear, fc2: FtLinear, dY, X, H, U1_save, U2_save, dX, dA1, dB1, dA2, dB2,
                     grad_dtype, workspace, ws_bytes, stream=None):
    s = lib().fourtune_mlp_bwd(ctypes.byref(fc1), ctypes.byref(fc2), _ptr(dY), _ptr(X), _ptr(H),
                               _ptr(U1_save), _ptr(U2_save), _ptr(dX), _ptr(dA1), _ptr(dB1),
                               _ptr(dA2), _ptr(dB2), int(grad_dtype), _ptr(workspace),
                               int(ws_bytes), _stream(stream))
    _check(s, "fourtune_mlp_bwd")


def fourtune_act_fwd(act, h, n, out, stream=None):
    _check(lib().fourtune_act_fwd(int(act), _ptr(h), int(n), _ptr(out), _stream(stream)),
           "fourtune_act_fwd")


def fourtune_act_bwd(act, h, g, n, out, stream=None):
    _check(lib().fourtune_act_bwd(int(act), _ptr(h), _ptr(g), int(n), _ptr(out), _stream(stream)),
           "fourtune_act_bwd")


def fourtune_timing_enable(on: bool):
    lib().fourtune_timing_enable(int(bool(on)))


def fourtune_timing_reset():
    lib().fourtune_timing_reset()


def fourtune_timing_read() -> dict:
    """{kernel name: (total ms, launches)} accumulated since the last reset."""
    L = lib()
    n = L.fourtune_timing_read(None, None, None, 0)
    names = (ctypes.c_char_p * max(n, 1))()
    tot = (ctypes.c_double * max(n, 1))()
    cnt = (ctypes.c_int64 * max(n, 1))()
    n = L.fourtune_timing_read(names, tot, cnt, n)
    return {names[i].decode(): (tot[i], cnt[i]) for i in range(n)}
