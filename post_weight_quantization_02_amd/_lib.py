"""ctypes binding of libgptq_mi355x.so (the C ABI in include/gptq.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch provides device memory and streams. If the library is not
built, importing this module raises ImportError: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptq_mi355x.so")

GPTQ_OK = 0
GPTQ_ERR_INVALID_ARG = 1
GPTQ_ERR_WORKSPACE = 2
GPTQ_ERR_NOT_PD = 3
GPTQ_ERR_HIP = 4
GPTQ_ERR_UNSUPPORTED = 5

GPTQ_DTYPE_F16 = 0
GPTQ_DTYPE_F32 = 1

OP_ACCUMULATE = 0
OP_PREPARE = 1
OP_QUANTIZE = 2
OP_QUANTIZE_PERM = 3

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")

# PyTorch-ROCm ships its own libamdhip64.so.7. Importing torch first makes the
# dynamic loader bind the library's libamdhip64.so.7 dependency to that
# already-loaded runtime, so torch's streams and allocations and the
# library's launches live in one HIP runtime.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

lib.gptq_version.restype = _int
lib.gptq_version.argtypes = []
lib.gptq_status_string.restype = ctypes.c_char_p
lib.gptq_status_string.argtypes = [_int]
lib.gptq_workspace_bytes.restype = _sz
lib.gptq_workspace_bytes.argtypes = [_int, _i64, _i64, _i64]
lib.gptq_hessian_accumulate.restype = _int
lib.gptq_hessian_accumulate.argtypes = [_p, _i64, _p, _i64, _i64, ctypes.c_float, _p, _sz, _p]
lib.gptq_prepare_hinv.restype = _int
lib.gptq_prepare_hinv.argtypes = [_p, _i64, ctypes.c_double, _p, _p, _sz,
                                  ctypes.POINTER(ctypes.c_int64), _p]
lib.gptq_quantize_layer.restype = _int
lib.gptq_quantize_layer.argtypes = [_p, _int, _i64, _i64, _i64, _p, _int, _int, _int,
                                    _p, _p, _p, _p, _p, _sz, _p]
lib.gptq_act_order.restype = _int
lib.gptq_act_order.argtypes = [_p, _i64, _p, _p]
lib.gptq_prepare_hinv_three_step.restype = _int
lib.gptq_prepare_hinv_three_step.argtypes = lib.gptq_prepare_hinv.argtypes
lib.gptq_prepare_hinv_perm.restype = _int
lib.gptq_prepare_hinv_perm.argtypes = [_p, _i64, _p, ctypes.c_double, _p, _p, _sz,
                                       ctypes.POINTER(ctypes.c_int64), _p]
lib.gptq_packed_words.restype = _i64
lib.gptq_packed_words.argtypes = [_i64, _int]
lib.gptq_pack_codes.restype = _int
lib.gptq_pack_codes.argtypes = [_p, _i64, _i64, _int, _p, _p]
lib.gptq_dequant_gemm.restype = _int
lib.gptq_dequant_gemm.argtypes = [_p, _i64, _i64, _i64, _p, _int, _i64, _p, _p, _int, _p, _p,
                                  _i64, _p]
lib.gptq_linear_forward.restype = _int
lib.gptq_linear_forward.argtypes = [_p, _i64, _i64, _i64, _p, _int, _i64, _p, _p, _int, _int, _p,
                                    _i64, _p]
lib.gptq_hessian_accumulate_noalloc.restype = _int
lib.gptq_hessian_accumulate_noalloc.argtypes = [_p, _i64, _p, _i64, _i64, ctypes.c_float, _p]
lib.gptq_quantize_layer_perm.restype = _int
lib.gptq_quantize_layer_perm.argtypes = [_p, _int, _i64, _i64, _i64, _p, _p, _int, _int, _int,
                                         _p, _p, _p, _p, _p, _p, _sz, _p]


class GPTQError(RuntimeError):
    def __init__(self, status: int, where: str, info: int = 0):
        name = lib.gptq_status_string(status).decode()
        msg = f"{where}: {name}"
        if info:
            msg += f" (info={info})"
        super().__init__(msg)
        self.status = status
        self.info = info


def status_string(status: int) -> str:
    return lib.gptq_status_string(status).decode()


def version() -> int:
    return lib.gptq_version()


def workspace_bytes(op: int, rows: int, cols: int, n: int) -> int:
    return int(lib.gptq_workspace_bytes(op, rows, cols, n))


# ---------------------------------------------------------------- torch layer
def _torch():
    import torch
    return torch


def _stream_ptr(stream, device) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _workspace(nbytes: int, device, workspace=None, stream=None):
    """The caller's workspace (checked), or a temporary one. A temporary is
    freed when the call returns while its kernels may still run; torch's
    caching allocator keeps it from being reused before the work queued on
    the current stream ends, and record_stream extends that to `stream`."""
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.device != device or workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small or on another device")
        if workspace.data_ptr() % 256:
            raise ValueError("workspace must be 256-byte aligned")
        return workspace, workspace.numel() * workspace.element_size()
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + nbytes]
    return ws, nbytes


def _check_out(t, shape, dtype, device, name):
    """A preallocated output must match exactly: the library writes
    prod(shape) elements of dtype from its data pointer."""
    if t is None or t.dtype != dtype or tuple(t.shape) != tuple(shape) or t.device != device \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}")
    return t


def _check(status: int, where: str, info: int = 0):
    if status != GPTQ_OK:
        raise GPTQError(status, where, info)


def hessian_accumulate(H, X, alpha: float = 2.0, workspace=None, stream=None):
    """H += alpha * X^T X on the GPU. H: d x d fp32 (contiguous), X: n x d fp16
    with unit column stride. Returns H."""
    torch = _torch()
    if H.dtype != torch.float32 or not H.is_cuda or not H.is_contiguous():
        raise ValueError("H must be a contiguous fp32 CUDA tensor")
    if X.dtype != torch.float16 or X.device != H.device or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D fp16 CUDA tensor with unit column stride")
    d = H.shape[0]
    if H.shape != (d, d) or X.shape[1] != d:
        raise ValueError("shape mismatch")
    n = X.shape[0]
    ldx = X.stride(0) if n > 1 else d
    ws, wsb = _workspace(workspace_bytes(OP_ACCUMULATE, 0, d, n), H.device, workspace, stream)
    st = lib.gptq_hessian_accumulate(H.data_ptr(), d, X.data_ptr(), n, ldx, alpha,
                                     ws.data_ptr() if ws is not None else None, wsb,
                                     _stream_ptr(stream, H.device))
    _check(st, "gptq_hessian_accumulate")
    return H


def hessian_accumulate_noalloc(H, X, alpha: float = 2.0, stream=None):
    """H += alpha * X^T X like hessian_accumulate, with no workspace and no
    allocation (gptq_hessian_accumulate_noalloc). Returns H."""
    torch = _torch()
    if H.dtype != torch.float32 or not H.is_cuda or not H.is_contiguous():
        raise ValueError("H must be a contiguous fp32 CUDA tensor")
    if X.dtype != torch.float16 or X.device != H.device or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D fp16 CUDA tensor with unit column stride")
    d = H.shape[0]
    if H.shape != (d, d) or X.shape[1] != d:
        raise ValueError("shape mismatch")
    n = X.shape[0]
    ldx = X.stride(0) if n > 1 else d
    st = lib.gptq_hessian_accumulate_noalloc(H.data_ptr(), d, X.data_ptr(), n, ldx, alpha,
                                             _stream_ptr(stream, H.device))
    _check(st, "gptq_hessian_accumulate_noalloc")
    return H


def _check_H(H):
    torch = _torch()
    if H.dtype != torch.float32 or not H.is_cuda or not H.is_contiguous() or H.dim() != 2:
        raise ValueError("H must be a contiguous fp32 CUDA tensor")
    if H.shape[0] != H.shape[1]:
        raise ValueError("H must be square")
    return H.shape[0]


def _check_perm(perm, n, device):
    torch = _torch()
    if perm is None:
        return None
    if perm.dtype != torch.int32 or perm.device != device or perm.shape != (n,) or \
            not perm.is_contiguous():
        raise ValueError(f"perm must be a contiguous int32 tensor of length {n} on {device}")
    return perm


def prepare_hinv(H, percdamp: float = 0.01, out=None, workspace=None, stream=None):
    """Hinv (d x d fp32, upper triangular) from H. Raises GPTQError with
    status GPTQ_ERR_NOT_PD and the failing pivot in .info."""
    return prepare_hinv_perm(H, None, percdamp, out, workspace, stream)


def prepare_hinv_three_step(H, percdamp: float = 0.01, out=None, workspace=None, stream=None):
    """prepare_hinv through the pages' three steps (Cholesky, inverse through
    the factor, upper Cholesky of the inverse): gptq_prepare_hinv_three_step."""
    torch = _torch()
    d = _check_H(H)
    if out is None:
        out = torch.empty((d, d), dtype=torch.float32, device=H.device)
    _check_out(out, (d, d), torch.float32, H.device, "out")
    ws, wsb = _workspace(workspace_bytes(OP_PREPARE, 0, d, 0), H.device, workspace, stream)
    info = ctypes.c_int64(0)
    st = lib.gptq_prepare_hinv_three_step(H.data_ptr(), d, float(percdamp), out.data_ptr(),
                                          ws.data_ptr(), wsb, ctypes.byref(info),
                                          _stream_ptr(stream, H.device))
    _check(st, "gptq_prepare_hinv_three_step", info.value)
    return out


def act_order(H, out=None, stream=None):
    """perm (d int32): the columns in decreasing order of H's diagonal, ties
    by index (gptq_act_order)."""
    torch = _torch()
    d = _check_H(H)
    if out is None:
        out = torch.empty((d,), dtype=torch.int32, device=H.device)
    _check_perm(out, d, H.device)
    st = lib.gptq_act_order(H.data_ptr(), d, out.data_ptr(), _stream_ptr(stream, H.device))
    _check(st, "gptq_act_order")
    return out


def prepare_hinv_perm(H, perm, percdamp: float = 0.01, out=None, workspace=None, stream=None):
    """Hinv of H with rows and columns taken in the order perm (None: the
    identity, i.e. gptq_prepare_hinv). H must hold both triangles."""
    torch = _torch()
    d = _check_H(H)
    perm = _check_perm(perm, d, H.device)
    if out is None:
        out = torch.empty((d, d), dtype=torch.float32, device=H.device)
    _check_out(out, (d, d), torch.float32, H.device, "out")
    ws, wsb = _workspace(workspace_bytes(OP_PREPARE, 0, d, 0), H.device, workspace, stream)
    info = ctypes.c_int64(0)
    st_ptr = _stream_ptr(stream, H.device)
    if perm is None:
        st = lib.gptq_prepare_hinv(H.data_ptr(), d, float(percdamp), out.data_ptr(),
                                   ws.data_ptr(), wsb, ctypes.byref(info), st_ptr)
        _check(st, "gptq_prepare_hinv", info.value)
    else:
        st = lib.gptq_prepare_hinv_perm(H.data_ptr(), d, perm.data_ptr(), float(percdamp),
                                        out.data_ptr(), ws.data_ptr(), wsb, ctypes.byref(info),
                                        st_ptr)
        _check(st, "gptq_prepare_hinv_perm", info.value)
    return out


def quantize_layer(W, Hinv, bits: int = 4, groupsize: int = 128, blocksize: int = 128,
                   out=None, workspace=None, stream=None):
    """GPTQ sweep. W: rows x cols fp16/fp32 (unit column stride); Hinv from
    prepare_hinv; groupsize <= 0 means one group per row (per-channel).
    Returns (codes uint8, scales fp32, zeros fp32, losses fp32)."""
    torch = _torch()
    if W.dim() != 2 or W.stride(1) != 1 or not W.is_cuda:
        raise ValueError("W must be a 2-D CUDA tensor with unit column stride")
    if W.dtype == torch.float16:
        wdt = GPTQ_DTYPE_F16
    elif W.dtype == torch.float32:
        wdt = GPTQ_DTYPE_F32
    else:
        raise ValueError("W must be fp16 or fp32")
    rows, cols = W.shape
    if Hinv.shape != (cols, cols) or Hinv.dtype != torch.float32 or not Hinv.is_contiguous():
        raise ValueError("Hinv must be a contiguous cols x cols fp32 tensor")
    if groupsize <= 0:  # per-channel: one group over all columns
        groupsize = cols
    g = groupsize
    ng = (cols + g - 1) // g
    dev = W.device
    if out is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, ng), dtype=torch.float32, device=dev)
        zeros = torch.empty((rows, ng), dtype=torch.float32, device=dev)
        losses = torch.empty((cols,), dtype=torch.float32, device=dev)
    else:
        codes, scales, zeros, losses = out
    _check_out(codes, (rows, cols), torch.uint8, dev, "codes")
    _check_out(scales, (rows, ng), torch.float32, dev, "scales")
    _check_out(zeros, (rows, ng), torch.float32, dev, "zeros")
    _check_out(losses, (cols,), torch.float32, dev, "losses")
    ws, wsb = _workspace(workspace_bytes(OP_QUANTIZE, rows, cols, 0), dev, workspace, stream)
    ldw = W.stride(0) if rows > 1 else cols
    st = lib.gptq_quantize_layer(W.data_ptr(), wdt, rows, cols, ldw, Hinv.data_ptr(), bits,
                                 groupsize, blocksize, codes.data_ptr(), scales.data_ptr(),
                                 zeros.data_ptr(), losses.data_ptr(), ws.data_ptr(), wsb,
                                 _stream_ptr(stream, dev))
    _check(st, "gptq_quantize_layer")
    return codes, scales, zeros, losses


def quantize_layer_perm(W, perm, Hinv, bits: int = 4, groupsize: int = 128, blocksize: int = 128,
                        out=None, workspace=None, stream=None):
    """Act-order sweep: W's columns processed in the order perm, with Hinv
    from prepare_hinv_perm(H, perm). Returns (codes, scales, zeros, losses,
    g_idx): codes, losses and g_idx (int32) in W's column order, scales and
    zeros per processing-order group."""
    torch = _torch()
    if W.dim() != 2 or W.stride(1) != 1 or not W.is_cuda:
        raise ValueError("W must be a 2-D CUDA tensor with unit column stride")
    if W.dtype == torch.float16:
        wdt = GPTQ_DTYPE_F16
    elif W.dtype == torch.float32:
        wdt = GPTQ_DTYPE_F32
    else:
        raise ValueError("W must be fp16 or fp32")
    rows, cols = W.shape
    perm = _check_perm(perm, cols, W.device)
    if Hinv.shape != (cols, cols) or Hinv.dtype != torch.float32 or not Hinv.is_contiguous():
        raise ValueError("Hinv must be a contiguous cols x cols fp32 tensor")
    if groupsize <= 0:  # per-channel: one group over all columns
        groupsize = cols
    g = groupsize
    ng = (cols + g - 1) // g
    dev = W.device
    if out is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, ng), dtype=torch.float32, device=dev)
        zeros = torch.empty((rows, ng), dtype=torch.float32, device=dev)
        losses = torch.empty((cols,), dtype=torch.float32, device=dev)
        g_idx = torch.empty((cols,), dtype=torch.int32, device=dev)
    else:
        codes, scales, zeros, losses, g_idx = out
    _check_out(codes, (rows, cols), torch.uint8, dev, "codes")
    _check_out(scales, (rows, ng), torch.float32, dev, "scales")
    _check_out(zeros, (rows, ng), torch.float32, dev, "zeros")
    _check_out(losses, (cols,), torch.float32, dev, "losses")
    if g_idx is not None:
        _check_out(g_idx, (cols,), torch.int32, dev, "g_idx")
    ws, wsb = _workspace(workspace_bytes(OP_QUANTIZE_PERM, rows, cols, 0), dev, workspace,
                         stream)
    ldw = W.stride(0) if rows > 1 else cols
    st = lib.gptq_quantize_layer_perm(W.data_ptr(), wdt, rows, cols, ldw,
                                      perm.data_ptr() if perm is not None else None,
                                      Hinv.data_ptr(), bits, groupsize, blocksize,
                                      codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                      losses.data_ptr(),
                                      g_idx.data_ptr() if g_idx is not None else None,
                                      ws.data_ptr(), wsb, _stream_ptr(stream, dev))
    _check(st, "gptq_quantize_layer_perm")
    return codes, scales, zeros, losses, g_idx


def packed_words(cols: int, bits: int) -> int:
    return int(lib.gptq_packed_words(cols, bits))


def pack_codes(codes, bits: int, out=None, stream=None):
    """rows x packed_words(cols, bits) int32 tensor holding the codes'
    uint32 words (gptq_pack_codes)."""
    torch = _torch()
    if codes.dtype != torch.uint8 or not codes.is_cuda or not codes.is_contiguous() or \
            codes.dim() != 2:
        raise ValueError("codes must be a contiguous 2-D uint8 CUDA tensor")
    rows, cols = codes.shape
    nw = packed_words(cols, bits)
    if out is None:
        out = torch.empty((rows, nw), dtype=torch.int32, device=codes.device)
    _check_out(out, (rows, nw), torch.int32, codes.device, "out")
    st = lib.gptq_pack_codes(codes.data_ptr(), rows, cols, bits, out.data_ptr(),
                             _stream_ptr(stream, codes.device))
    _check(st, "gptq_pack_codes")
    return out


def dequant_gemm(x, packed, bits: int, cols: int, scales, zeros, groupsize: int, g_idx=None,
                 out=None, stream=None):
    """y = x W_hat^T (m x rows fp32) for fp16 x (m x cols) and the packed
    codes with their scales and zeros (gptq_dequant_gemm)."""
    torch = _torch()
    if x.dtype != torch.float16 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1 or \
            x.shape[1] != cols:
        raise ValueError("x must be an m x cols fp16 CUDA tensor with unit column stride")
    rows = packed.shape[0]
    if packed.dtype != torch.int32 or not packed.is_contiguous() or \
            packed.shape[1] != packed_words(cols, bits):
        raise ValueError("packed must come from pack_codes for these cols and bits")
    if groupsize <= 0:
        groupsize = cols
    ng = (cols + groupsize - 1) // groupsize
    for t in (scales, zeros):
        if t.dtype != torch.float32 or t.shape != (rows, ng) or not t.is_contiguous():
            raise ValueError("scales and zeros must be contiguous rows x ngroups fp32")
    g_idx = _check_perm(g_idx, cols, x.device)
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, rows), dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (m, rows) or out.device != x.device \
            or (m > 0 and out.stride(1) != 1):
        raise ValueError(f"out must be an {m} x {rows} fp32 tensor with unit column stride "
                         f"on {x.device}")
    ldx = x.stride(0) if m > 1 else cols
    st = lib.gptq_dequant_gemm(x.data_ptr(), m, cols, ldx, packed.data_ptr(), bits, rows,
                               scales.data_ptr(), zeros.data_ptr(), groupsize,
                               g_idx.data_ptr() if g_idx is not None else None, out.data_ptr(),
                               out.stride(0) if m > 1 else rows, _stream_ptr(stream, x.device))
    _check(st, "gptq_dequant_gemm")
    return out


def linear_forward(x, packed, bits: int, cols: int, scales, zeros, groupsize: int,
                   relu: bool = False, out=None, stream=None):
    """y = x W_hat^T, or max(x W_hat^T, 0) with relu, as m x rows fp16, for
    fp16 x (m x cols) and the 4- or 8-bit packed codes with their scales and
    zeros (gptq_linear_forward: the product for many tokens on MFMA)."""
    torch = _torch()
    if x.dtype != torch.float16 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1 or \
            x.shape[1] != cols:
        raise ValueError("x must be an m x cols fp16 CUDA tensor with unit column stride")
    rows = packed.shape[0]
    if packed.dtype != torch.int32 or not packed.is_contiguous() or \
            packed.shape[1] != packed_words(cols, bits):
        raise ValueError("packed must come from pack_codes for these cols and bits")
    if groupsize <= 0:
        groupsize = cols
    ng = (cols + groupsize - 1) // groupsize
    for t in (scales, zeros):
        if t.dtype != torch.float32 or t.shape != (rows, ng) or not t.is_contiguous():
            raise ValueError("scales and zeros must be contiguous rows x ngroups fp32")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, rows), dtype=torch.float16, device=x.device)
    elif out.dtype != torch.float16 or out.shape != (m, rows) or out.stride(1) != 1 or \
            out.device != x.device:
        raise ValueError("out must be an m x rows fp16 tensor with unit column stride")
    ldx = x.stride(0) if m > 1 else cols
    st = lib.gptq_linear_forward(x.data_ptr(), m, cols, ldx, packed.data_ptr(), bits, rows,
                                 scales.data_ptr(), zeros.data_ptr(), groupsize, 1 if relu else 0,
                                 out.data_ptr(), out.stride(0) if m > 1 else rows,
                                 _stream_ptr(stream, x.device))
    _check(st, "gptq_linear_forward")
    return out
