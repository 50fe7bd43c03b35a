"""Python binding of libtq (include/tq.h): argument marshalling only.

Every computation runs in the HIP kernels of ``libtq.so``; this module checks
tensors, allocates outputs with torch (device memory and streams are the only
things torch provides here) and passes raw pointers plus torch's current HIP
stream to the C ABI.  There is no CPU fallback: if the library is not built
or a tensor is not on the GPU, the call raises.

The names follow the C ABI: quantize, dequantize, rotate, gemv, gemm,
blockfp_quantize, blockfp_gemm, transcode_q8, q8_gemv, codebook, sign_mask_from_seed.
"""

from __future__ import annotations

import ctypes
import os

import torch  # imported before libtq so both bind to the same HIP runtime

__all__ = [
    "TQError", "lib", "codebook", "sign_mask_from_seed", "DEFAULT_SIGN_MASK",
    "quantize", "dequantize", "rotate", "gemv", "gemm",
    "blockfp_quantize", "blockfp_gemm", "transcode_q8", "q8_gemv", "LIB_PATH", "workspace_bytes", "stream_read",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
FORMATS = {"nvfp4": 1, "mxfp6": 2}
_STATUS = {0: "TQ_OK", 1: "TQ_EINVAL", 2: "TQ_ESHAPE", 3: "TQ_EALIGN", 4: "TQ_EDTYPE", 5: "TQ_EDEVICE"}

EXPORTED = [
    "tq_abi_version", "tq_status_str", "tq_codebook", "tq_sign_mask_from_seed", "tq_default_sign_mask",
    "tq_quantize", "tq_quantize_rsf", "tq_dequantize", "tq_rotate", "tq_gemv", "tq_gemm",
    "tq_blockfp_quantize", "tq_blockfp_quantize_rsf", "tq_blockfp_gemm", "tq_transcode_q8", "tq_q8_gemv",
    "tq_kv_sign_from_seed", "tq_kv_quantize_k", "tq_kv_quantize_v", "tq_kv_dequantize_v", "tq_attn_workspace_bytes",
    "tq_attn_decode", "tq_workspace_bytes", "tq_stream_read", "tq_attn_decode_noalloc",
]


class TQError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dequant_gemv_tq_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    i64, u32, p, c_int = ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    L.tq_abi_version.restype = c_int
    L.tq_status_str.restype = ctypes.c_char_p
    L.tq_status_str.argtypes = [c_int]
    L.tq_codebook.restype = c_int
    L.tq_codebook.argtypes = [p, p]
    L.tq_sign_mask_from_seed.restype = u32
    L.tq_sign_mask_from_seed.argtypes = [ctypes.c_uint64]
    L.tq_default_sign_mask.restype = u32
    L.tq_quantize.argtypes = [p, c_int, i64, i64, i64, u32, p, p, p]
    L.tq_quantize_rsf.argtypes = [p, c_int, i64, i64, i64, u32, p, p, p]
    L.tq_dequantize.argtypes = [p, p, i64, i64, u32, p, c_int, i64, p]
    L.tq_rotate.argtypes = [p, c_int, i64, i64, i64, u32, p, c_int, i64, p]
    L.tq_gemv.argtypes = [p, p, i64, i64, u32, p, c_int, c_int, p, p]
    L.tq_gemm.argtypes = [p, p, i64, i64, i64, p, c_int, i64, p, i64, p, ctypes.c_size_t, p]
    L.tq_blockfp_quantize.argtypes = [c_int, p, c_int, i64, i64, p, p, p, p, ctypes.c_size_t, p]
    L.tq_blockfp_quantize_rsf.argtypes = [c_int, p, c_int, i64, i64, p, p, p, p, ctypes.c_size_t, p]
    L.tq_workspace_bytes.argtypes = [c_int, i64, i64, i64]
    L.tq_workspace_bytes.restype = ctypes.c_size_t
    L.tq_attn_decode_noalloc.argtypes = [p, c_int, i64, i64, i64, i64, i64, p, p, p, p, p, p, p, p]
    L.tq_attn_decode_noalloc.restype = c_int
    L.tq_stream_read.argtypes = [p, ctypes.c_size_t, p, p]
    L.tq_stream_read.restype = c_int
    L.tq_blockfp_gemm.argtypes = [c_int, p, p, p, i64, i64, i64, p, c_int, i64, p, i64, p, ctypes.c_size_t, p]
    L.tq_transcode_q8.argtypes = [p, p, i64, i64, u32, p, p, p]
    L.tq_q8_gemv.argtypes = [p, p, i64, i64, p, c_int, p, p]
    L.tq_kv_sign_from_seed.argtypes = [ctypes.c_uint64, p]
    L.tq_kv_quantize_k.argtypes = [p, c_int, i64, i64, p, p, p]
    L.tq_kv_quantize_v.argtypes = [p, c_int, i64, i64, p, p, p, p]
    L.tq_kv_dequantize_v.argtypes = [p, p, i64, i64, p, p, p]
    L.tq_attn_workspace_bytes.argtypes = [i64, i64, i64]
    L.tq_attn_workspace_bytes.restype = ctypes.c_size_t
    L.tq_attn_decode.argtypes = [p, c_int, i64, i64, i64, i64, i64, p, p, p, p, p, p, p, p, ctypes.c_size_t, p]
    for name in ("tq_quantize", "tq_quantize_rsf", "tq_dequantize", "tq_rotate", "tq_gemv", "tq_gemm",
                 "tq_blockfp_quantize", "tq_blockfp_quantize_rsf", "tq_blockfp_gemm", "tq_transcode_q8", "tq_q8_gemv",
                 "tq_kv_sign_from_seed", "tq_kv_quantize_k", "tq_kv_quantize_v", "tq_kv_dequantize_v",
                 "tq_attn_decode"):
        getattr(L, name).restype = c_int
    _lib = L
    return L


def _check(fn: str, status: int):
    if status != 0:
        raise TQError(fn, status, lib().tq_status_str(status).decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU fallback)")


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"{name}: dtype {t.dtype} not supported (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(ok: bool, msg: str):
    if not ok:
        raise ValueError(msg)


def _dense(t: torch.Tensor, name: str, dtypes, shape):
    """Check a tensor the C ABI reads as dense rows: dtype, exact shape, contiguity."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.dtype in dtypes, f"{name}: dtype {t.dtype} not accepted ({', '.join(str(d) for d in dtypes)})")
    _need(tuple(t.shape) == tuple(shape), f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _same_device(ref: torch.Tensor, *named):
    for t, name in named:
        if t is not None:
            _need(t.device == ref.device, f"{name} is on {t.device}, expected {ref.device}")


def _rows(t: torch.Tensor, name: str, dtypes, rows: int, cols: int):
    """Check a 2-D tensor passed with a leading dimension: [rows, cols], unit column stride."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.dtype in dtypes, f"{name}: dtype {t.dtype} not accepted")
    _need(t.dim() == 2 and tuple(t.shape) == (rows, cols), f"{name}: shape {tuple(t.shape)}, expected {(rows, cols)}")
    _need(t.stride(1) == 1 and t.stride(0) >= cols, f"{name} must have unit column stride and row stride >= {cols}")


_SCALE16 = (torch.int16, torch.float16)


def _tq4_weights(packed: torch.Tensor, scales: torch.Tensor):
    """(N, K) of a TQ4_1S pair: packed uint8 [N, K/2], scales fp16 bits [N, K/16], both dense."""
    _need(isinstance(packed, torch.Tensor) and packed.dim() == 2, "packed must be a 2-D uint8 tensor [N, K/2]")
    N, K = packed.shape[0], packed.shape[1] * 2
    _dense(packed, "packed", (torch.uint8,), (N, K // 2))
    _dense(scales, "scales", _SCALE16, (N, K // 16))
    _same_device(packed, (scales, "scales"))
    _dev(packed, "packed")
    return N, K


# ----------------------------------------------------------------------------
# host constants
# ----------------------------------------------------------------------------

def codebook():
    """(centroids float32[16], thresholds float32[15]) as the kernels use them."""
    import numpy as np
    c = (ctypes.c_float * 16)()
    m = (ctypes.c_float * 15)()
    _check("tq_codebook", lib().tq_codebook(c, m))
    return np.frombuffer(c, dtype=np.float32).copy(), np.frombuffer(m, dtype=np.float32).copy()


def sign_mask_from_seed(seed: int) -> int:
    return int(lib().tq_sign_mask_from_seed(seed))


def default_sign_mask() -> int:
    return int(lib().tq_default_sign_mask())


DEFAULT_SIGN_MASK = 0x7B1DCDAF


# ----------------------------------------------------------------------------
# TQ4_1S
# ----------------------------------------------------------------------------

def quantize(W: torch.Tensor, sign_mask: int = DEFAULT_SIGN_MASK, out=None, rsf: bool = False):
    """W [N, K] (fp32/bf16, row stride may exceed K) -> (packed uint8 [N, K/2], scales int16 [N, K/16]).

    ``scales`` holds the fp16 bit patterns of d0, d1 per block (view as float16).
    ``rsf=True`` runs the RSF-lite scale search (tq_quantize_rsf).
    """
    _dev(W, "W")
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be a 2-D tensor with unit column stride")
    N, K = W.shape
    if out is None:
        packed = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
        scales = torch.empty((N, K // 16), dtype=torch.int16, device=W.device)
    else:
        packed, scales = out
        _dense(packed, "out[0]", (torch.uint8,), (N, K // 2))
        _dense(scales, "out[1]", _SCALE16, (N, K // 16))
        _same_device(W, (packed, "out[0]"), (scales, "out[1]"))
    fn = "tq_quantize_rsf" if rsf else "tq_quantize"
    st = getattr(lib(), fn)(_ptr(W), _dtype_code(W, "W"), N, K, W.stride(0), sign_mask & 0xFFFFFFFF,
                            _ptr(packed), _ptr(scales), _stream())
    _check(fn, st)
    return packed, scales


def dequantize(packed: torch.Tensor, scales: torch.Tensor, sign_mask: int = DEFAULT_SIGN_MASK,
               dtype=torch.float32, out=None):
    N, K = _tq4_weights(packed, scales)
    W = torch.empty((N, K), dtype=dtype, device=packed.device) if out is None else out
    _rows(W, "out", (torch.float32, torch.bfloat16), N, K)
    _same_device(packed, (W, "out"))
    st = lib().tq_dequantize(_ptr(packed), _ptr(scales), N, K, sign_mask & 0xFFFFFFFF, _ptr(W),
                             _dtype_code(W, "out"), W.stride(0), _stream())
    _check("tq_dequantize", st)
    return W


def rotate(x: torch.Tensor, sign_mask: int = DEFAULT_SIGN_MASK, dtype=torch.float32, out=None):
    """x [M, K] or [K] -> x' of the same shape (dtype fp32 or bf16); rows may be strided (unit column
    stride), and ``out`` is written in place (a view of it, never a copy)."""
    _dev(x, "x")
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    _need(x2.dim() == 2 and x2.stride(1) == 1, "x must be [M, K] or [K] with unit column stride")
    M, K = x2.shape
    if out is None:
        xr = torch.empty((M, K), dtype=dtype, device=x.device)
    else:
        _need(isinstance(out, torch.Tensor) and out.dim() == x.dim(), "out must have the shape of x")
        _need(out.dim() == 2 or out.is_contiguous(), "a 1-D out must be contiguous")
        xr = out if out.dim() == 2 else out.view(1, -1)
        _rows(xr, "out", (torch.float32, torch.bfloat16), M, K)
        _same_device(x2, (xr, "out"))
    st = lib().tq_rotate(_ptr(x2), _dtype_code(x2, "x"), M, K, x2.stride(0), sign_mask & 0xFFFFFFFF,
                         _ptr(xr), _dtype_code(xr, "out"), xr.stride(0), _stream())
    _check("tq_rotate", st)
    return xr if x.dim() == 2 else xr.reshape(-1)


def gemv(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, rotated: bool = False,
         sign_mask: int = DEFAULT_SIGN_MASK, out=None):
    """y [N] float32 = W_deq x.  x: [K] raw (fp32/bf16) or, with rotated=True, x' (fp32 or bf16) from rotate()."""
    N, K = _tq4_weights(packed, scales)
    _dev(x, "x")
    if x.numel() != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous vector of length K")
    y = torch.empty(N, dtype=torch.float32, device=packed.device) if out is None else out
    _dense(y, "out", (torch.float32,), (N,))
    _same_device(packed, (x, "x"), (y, "out"))
    st = lib().tq_gemv(_ptr(packed), _ptr(scales), N, K, sign_mask & 0xFFFFFFFF, _ptr(x), _dtype_code(x, "x"),
                       1 if rotated else 0, _ptr(y), _stream())
    _check("tq_gemv", st)
    return y


_GEMM_WS = {}      # (device index, stream) -> zero-filled split-K workspace


def _gemm_workspace(op: str, N: int, K: int, M: int, xbf16: bool, device, workspace):
    """The split-K workspace of a GEMM call: the caller's, checked, or one kept per device and stream.

    The library's contract: zero-filled before its first use, left fit for the next call by every
    call, and never used by two calls at once -- hence one buffer per stream.
    """
    need = workspace_bytes(op, N, K, M) if xbf16 else 0
    if workspace is not None:
        _need(isinstance(workspace, torch.Tensor) and workspace.dtype == torch.uint8 and workspace.is_contiguous()
              and workspace.numel() >= need, f"workspace must be a contiguous uint8 buffer of at least {need} bytes")
        _need(workspace.device == device, "workspace must be on the weights' device")
        _need(workspace.data_ptr() % 256 == 0, "workspace must be 256-byte aligned")
        return workspace
    if need == 0:
        return None
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _GEMM_WS.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
        _GEMM_WS[key] = ws
    return ws


def gemm(packed: torch.Tensor, scales: torch.Tensor, x_rot: torch.Tensor, out=None, workspace=None):
    """Y [M, N] float32 = X' Q^T with pre-rotated activations x_rot [M, K] (bf16 or fp32).

    workspace: optional uint8 device buffer for the split-K sums (see tq_gemm); by default one
    zero-filled buffer per device and stream is kept and reused.
    """
    N, K = _tq4_weights(packed, scales)
    _dev(x_rot, "x_rot")
    M = x_rot.shape[0]
    if x_rot.dim() != 2 or x_rot.shape[1] != K or x_rot.stride(1) != 1:
        raise ValueError("x_rot must be [M, K] with unit column stride")
    y = torch.empty((M, N), dtype=torch.float32, device=packed.device) if out is None else out
    _rows(y, "out", (torch.float32,), M, N)
    _same_device(packed, (x_rot, "x_rot"), (y, "out"))
    ws = _gemm_workspace("gemm", N, K, M, x_rot.dtype == torch.bfloat16, packed.device, workspace)
    st = lib().tq_gemm(_ptr(packed), _ptr(scales), N, K, M, _ptr(x_rot), _dtype_code(x_rot, "x_rot"),
                       x_rot.stride(0), _ptr(y), y.stride(0), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    _check("tq_gemm", st)
    return y


# ----------------------------------------------------------------------------
# NVFP4 / MXFP6
# ----------------------------------------------------------------------------

OPS = {"quantize": 1, "dequantize": 2, "rotate": 3, "gemv": 4, "gemm": 5, "nvfp4_quantize": 6,
       "mxfp6_quantize": 7, "blockfp_gemm": 8, "transcode_q8": 9, "q8_gemv": 10, "attn_decode": 11}


def workspace_bytes(op: str, N: int, K: int, M: int = 0) -> int:
    """Device workspace bytes of a call (tq_workspace_bytes); 0 when it takes none."""
    return int(lib().tq_workspace_bytes(OPS[op], N, K, M))


def blockfp_quantize(fmt: str, W: torch.Tensor, rsf: bool = False, workspace=None, out=None):
    """-> (codes uint8, block_scales uint8, tensor_scale float32[1] or None).

    ``rsf=True`` runs the RSF-lite block-scale search (tq_blockfp_quantize_rsf).  NVFP4 needs a
    workspace of workspace_bytes("nvfp4_quantize", N, K) bytes; one is taken from torch's allocator
    when none is given.  ``out`` = (codes, block_scales, tensor_scale) to write into."""
    _dev(W, "W")
    if W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous 2-D tensor")
    f = FORMATS[fmt]
    N, K = W.shape
    cshape = (N, K // 2) if fmt == "nvfp4" else (N, 3 * K // 4)
    sshape = (N, K // 16) if fmt == "nvfp4" else (N, K // 32)
    if out is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=W.device)
        bs = torch.empty(sshape, dtype=torch.uint8, device=W.device)
        ts = torch.empty(1, dtype=torch.float32, device=W.device) if fmt == "nvfp4" else None
    else:
        codes, bs, ts = out
        _dense(codes, "out[0]", (torch.uint8,), cshape)
        _dense(bs, "out[1]", (torch.uint8,), sshape)
        if fmt == "nvfp4":
            _need(ts is not None, "NVFP4 needs a tensor-scale output")
            _dense(ts, "out[2]", (torch.float32,), (1,))
        _same_device(W, (codes, "out[0]"), (bs, "out[1]"), (ts, "out[2]"))
    ws, wsb = None, 0
    if fmt == "nvfp4":
        need = workspace_bytes("nvfp4_quantize", N, K)
        ws = torch.empty(need, dtype=torch.uint8, device=W.device) if workspace is None else workspace
        _need(ws.is_contiguous() and ws.numel() * ws.element_size() >= need,
              f"workspace must be a contiguous buffer of at least {need} bytes")
        _same_device(W, (ws, "workspace"))
        wsb = ws.numel() * ws.element_size()
    fn = "tq_blockfp_quantize_rsf" if rsf else "tq_blockfp_quantize"
    st = getattr(lib(), fn)(f, _ptr(W), _dtype_code(W, "W"), N, K, _ptr(codes), _ptr(bs), _ptr(ts), _ptr(ws), wsb,
                            _stream())
    _check(fn, st)
    return codes, bs, ts


def blockfp_gemm(fmt: str, codes: torch.Tensor, block_scales: torch.Tensor, tensor_scale, x: torch.Tensor,
                 out=None, workspace=None):
    """Y [M, N] float32 = X W_deq^T (x: [M, K] or [K], fp32/bf16); workspace as for gemm()."""
    f = FORMATS[fmt]
    _need(isinstance(codes, torch.Tensor) and codes.dim() == 2, "codes must be a 2-D uint8 tensor")
    N = codes.shape[0]
    K = codes.shape[1] * 2 if fmt == "nvfp4" else codes.shape[1] * 4 // 3
    _dense(codes, "codes", (torch.uint8,), (N, K // 2 if fmt == "nvfp4" else 3 * K // 4))
    _dense(block_scales, "block_scales", (torch.uint8,), (N, K // 16 if fmt == "nvfp4" else K // 32))
    if fmt == "nvfp4":
        _need(tensor_scale is not None, "NVFP4 needs its tensor scale")
        _dense(tensor_scale, "tensor_scale", (torch.float32,), (1,))
    _same_device(codes, (block_scales, "block_scales"), (tensor_scale, "tensor_scale"))
    _dev(codes, "codes")
    _dev(x, "x")
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    _need(x2.shape[1] == K and x2.stride(1) == 1, f"x must be [M, {K}] or [{K}] with unit column stride")
    M = x2.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=codes.device) if out is None else out
    _need(isinstance(y, torch.Tensor) and (y.dim() == 2 or y.is_contiguous()), "a 1-D out must be contiguous")
    y2 = y if y.dim() == 2 else y.view(1, -1)              # a view: the call writes into ``out``
    _rows(y2, "out", (torch.float32,), M, N)
    _same_device(codes, (x2, "x"), (y2, "out"))
    y = y2 if y.dim() == 2 else y
    ws = _gemm_workspace("blockfp_gemm", N, K, M, x2.dtype == torch.bfloat16, codes.device, workspace)
    st = lib().tq_blockfp_gemm(f, _ptr(codes), _ptr(block_scales), _ptr(tensor_scale), N, K, M, _ptr(x2),
                               _dtype_code(x2, "x"), x2.stride(0), _ptr(y2), y2.stride(0), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream())
    _check("tq_blockfp_gemm", st)
    return y if x.dim() == 2 else y.reshape(-1)


# ----------------------------------------------------------------------------
# load-time int8 transcode
# ----------------------------------------------------------------------------

def transcode_q8(packed: torch.Tensor, scales: torch.Tensor, sign_mask: int = DEFAULT_SIGN_MASK, out=None):
    """TQ4_1S (packed, scales) -> (codes int8 [N, K], q8_scales int16 [N, K/32] = fp16 bits per block)."""
    N, K = _tq4_weights(packed, scales)
    if out is None:
        codes = torch.empty((N, K), dtype=torch.int8, device=packed.device)
        qs = torch.empty((N, K // 32), dtype=torch.int16, device=packed.device)
    else:
        codes, qs = out
        _dense(codes, "out[0]", (torch.int8,), (N, K))
        _dense(qs, "out[1]", _SCALE16, (N, K // 32))
        _same_device(packed, (codes, "out[0]"), (qs, "out[1]"))
    st = lib().tq_transcode_q8(_ptr(packed), _ptr(scales), N, K, sign_mask & 0xFFFFFFFF, _ptr(codes), _ptr(qs),
                               _stream())
    _check("tq_transcode_q8", st)
    return codes, qs


def q8_gemv(codes: torch.Tensor, q8_scales: torch.Tensor, x: torch.Tensor, out=None):
    """y [N] float32 from transcoded int8 weights and the activation x [K] (fp32/bf16, not rotated)."""
    _need(isinstance(codes, torch.Tensor) and codes.dim() == 2, "codes must be a 2-D int8 tensor [N, K]")
    N, K = codes.shape
    _dense(codes, "codes", (torch.int8,), (N, K))
    _dense(q8_scales, "q8_scales", _SCALE16, (N, K // 32))
    _same_device(codes, (q8_scales, "q8_scales"))
    _dev(codes, "codes")
    _dev(x, "x")
    if x.numel() != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous vector of length K")
    y = torch.empty(N, dtype=torch.float32, device=codes.device) if out is None else out
    _dense(y, "out", (torch.float32,), (N,))
    _same_device(codes, (x, "x"), (y, "out"))
    st = lib().tq_q8_gemv(_ptr(codes), _ptr(q8_scales), N, K, _ptr(x), _dtype_code(x, "x"), _ptr(y), _stream())
    _check("tq_q8_gemv", st)
    return y


# ----------------------------------------------------------------------------
# turbo4 KV cache and decode attention
# ----------------------------------------------------------------------------

def kv_sign_from_seed(seed: int = 0):
    """The four 32-bit words of the 128 rotation sign bits (host array, ctypes)."""
    out = (ctypes.c_uint32 * 4)()
    _check("tq_kv_sign_from_seed", lib().tq_kv_sign_from_seed(seed, out))
    return out


def kv_quantize_k(K: torch.Tensor, out=None):
    """Keys [..., d] (bf16/fp32, contiguous) -> (int8 codes [..., d], fp16 scales [..., d/32] as int16);
    ``out`` = (codes, scales) of those shapes to write into."""
    _dev(K, "K")
    if not K.is_contiguous():
        raise ValueError("K must be contiguous")
    d = K.shape[-1]
    n = K.numel() // d
    if out is None:
        codes = torch.empty(K.shape, dtype=torch.int8, device=K.device)
        scales = torch.empty(K.shape[:-1] + (d // 32,), dtype=torch.int16, device=K.device)
    else:
        codes, scales = out
        _dense(codes, "out[0]", (torch.int8,), tuple(K.shape))
        _dense(scales, "out[1]", _SCALE16, tuple(K.shape[:-1]) + (d // 32,))
        _same_device(K, (codes, "out[0]"), (scales, "out[1]"))
    st = lib().tq_kv_quantize_k(_ptr(K), _dtype_code(K, "K"), n, d, _ptr(codes), _ptr(scales), _stream())
    _check("tq_kv_quantize_k", st)
    return codes, scales


def kv_quantize_v(V: torch.Tensor, sign=None, out=None):
    """Values [..., 128] (bf16/fp32, contiguous) -> (packed uint8 [..., 64], fp16 norms [...] as int16);
    ``out`` = (packed, norms) of those shapes to write into."""
    _dev(V, "V")
    if not V.is_contiguous():
        raise ValueError("V must be contiguous")
    d = V.shape[-1]
    n = V.numel() // d
    sign = kv_sign_from_seed(0) if sign is None else sign
    if out is None:
        packed = torch.empty(V.shape[:-1] + (d // 2,), dtype=torch.uint8, device=V.device)
        norms = torch.empty(V.shape[:-1], dtype=torch.int16, device=V.device)
    else:
        packed, norms = out
        _dense(packed, "out[0]", (torch.uint8,), tuple(V.shape[:-1]) + (d // 2,))
        _dense(norms, "out[1]", _SCALE16, tuple(V.shape[:-1]))
        _same_device(V, (packed, "out[0]"), (norms, "out[1]"))
    st = lib().tq_kv_quantize_v(_ptr(V), _dtype_code(V, "V"), n, d, sign, _ptr(packed), _ptr(norms), _stream())
    _check("tq_kv_quantize_v", st)
    return packed, norms


def kv_dequantize_v(packed: torch.Tensor, norms: torch.Tensor, sign=None):
    """turbo4 values back to float32 [..., 128]."""
    _dev(packed, "packed")
    d = packed.shape[-1] * 2
    n = packed.numel() // (d // 2)
    _dense(packed, "packed", (torch.uint8,), packed.shape)
    _dense(norms, "norms", _SCALE16, packed.shape[:-1])
    _same_device(packed, (norms, "norms"))
    sign = kv_sign_from_seed(0) if sign is None else sign
    out = torch.empty(packed.shape[:-1] + (d,), dtype=torch.float32, device=packed.device)
    st = lib().tq_kv_dequantize_v(_ptr(packed), _ptr(norms), n, d, sign, _ptr(out), _stream())
    _check("tq_kv_dequantize_v", st)
    return out


def attn_workspace_bytes(B: int, Hq: int, T_max: int) -> int:
    return int(lib().tq_attn_workspace_bytes(B, Hq, T_max))


def attn_decode(q: torch.Tensor, lengths: torch.Tensor, k_codes, k_scales, v_packed, v_norms, sign=None,
                out=None, workspace=None):
    """Decode attention: q [B, Hq, 128] (bf16/fp32), lengths int32 [B], head-major cache tensors
    [B, Hkv, T_max, ...] from kv_quantize_k / kv_quantize_v -> o [B, Hq, 128] float32."""
    for t, name in ((q, "q"), (lengths, "lengths"), (k_codes, "k_codes"), (v_packed, "v_packed")):
        _dev(t, name)
    _need(q.dim() == 3 and q.is_contiguous(), "q must be a contiguous [B, Hq, 128] tensor")
    B, Hq, d = q.shape
    _need(k_codes.dim() == 4 and k_codes.shape[0] == B and k_codes.shape[-1] == d,
          "k_codes must be [B, Hkv, T_max, 128]")
    _, Hkv, T_max, _ = k_codes.shape
    if lengths.dtype != torch.int32 or lengths.numel() != B or not lengths.is_contiguous():
        raise ValueError("lengths must be a contiguous int32 [B] tensor")
    _dense(k_codes, "k_codes", (torch.int8,), (B, Hkv, T_max, d))
    _dense(k_scales, "k_scales", _SCALE16, (B, Hkv, T_max, d // 32))
    _dense(v_packed, "v_packed", (torch.uint8,), (B, Hkv, T_max, d // 2))
    _dense(v_norms, "v_norms", _SCALE16, (B, Hkv, T_max))
    sign = kv_sign_from_seed(0) if sign is None else sign
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device) if out is None else out
    _dense(o, "out", (torch.float32,), (B, Hq, d))
    ws_bytes = attn_workspace_bytes(B, Hq, T_max)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=q.device)
    _need(workspace.is_contiguous() and workspace.numel() * workspace.element_size() >= ws_bytes,
          f"workspace must be a contiguous buffer of at least {ws_bytes} bytes")
    _same_device(q, (lengths, "lengths"), (k_codes, "k_codes"), (k_scales, "k_scales"), (v_packed, "v_packed"),
                 (v_norms, "v_norms"), (o, "out"), (workspace, "workspace"))
    st = lib().tq_attn_decode(_ptr(q), _dtype_code(q, "q"), B, Hq, Hkv, d, T_max, _ptr(lengths), _ptr(k_codes),
                              _ptr(k_scales), _ptr(v_packed), _ptr(v_norms), sign, _ptr(o), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream())
    _check("tq_attn_decode", st)
    return o


# ----------------------------------------------------------------------------
# measurement helper
# ----------------------------------------------------------------------------

STREAM_READ_SINK_WORDS = 16384


def stream_read(buf: torch.Tensor, nbytes: int | None = None, sink: torch.Tensor | None = None):
    """Read the first ``nbytes`` bytes of ``buf`` with the plain streaming-read kernel (tq_stream_read);
    returns the sink of per-wavefront XOR folds."""
    _dev(buf, "buf")
    _need(buf.is_contiguous(), "buf must be contiguous")
    total = buf.numel() * buf.element_size()
    nbytes = total if nbytes is None else nbytes
    _need(0 < nbytes <= total, "nbytes out of range")
    if sink is None:
        sink = torch.empty(STREAM_READ_SINK_WORDS, dtype=torch.int32, device=buf.device)
    _dense(sink, "sink", (torch.int32,), (STREAM_READ_SINK_WORDS,))
    _same_device(buf, (sink, "sink"))
    _check("tq_stream_read", lib().tq_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream()))
    return sink
