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
    "blockfp_quantize", "blockfp_gemm", "transcode_q8", "q8_gemv", "LIB_PATH",
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
    "tq_attn_decode",
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
    L.tq_gemm.argtypes = [p, p, i64, i64, i64, p, c_int, i64, p, i64, p]
    L.tq_blockfp_quantize.argtypes = [c_int, p, c_int, i64, i64, p, p, p, p]
    L.tq_blockfp_quantize_rsf.argtypes = [c_int, p, c_int, i64, i64, p, p, p, p]
    L.tq_blockfp_gemm.argtypes = [c_int, p, p, p, i64, i64, i64, p, c_int, i64, p, i64, p]
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
    fn = "tq_quantize_rsf" if rsf else "tq_quantize"
    st = getattr(lib(), fn)(_ptr(W), _dtype_code(W, "W"), N, K, W.stride(0), sign_mask & 0xFFFFFFFF,
                            _ptr(packed), _ptr(scales), _stream())
    _check(fn, st)
    return packed, scales


def dequantize(packed: torch.Tensor, scales: torch.Tensor, sign_mask: int = DEFAULT_SIGN_MASK,
               dtype=torch.float32, out=None):
    _dev(packed, "packed")
    N, K = packed.shape[0], packed.shape[1] * 2
    W = torch.empty((N, K), dtype=dtype, device=packed.device) if out is None else out
    st = lib().tq_dequantize(_ptr(packed), _ptr(scales), N, K, sign_mask & 0xFFFFFFFF, _ptr(W),
                             _dtype_code(W, "out"), W.stride(0), _stream())
    _check("tq_dequantize", st)
    return W


def rotate(x: torch.Tensor, sign_mask: int = DEFAULT_SIGN_MASK, dtype=torch.float32, out=None):
    """x [M, K] or [K] -> x' of the same shape (dtype fp32 or bf16)."""
    _dev(x, "x")
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    M, K = x2.shape
    xr = torch.empty((M, K), dtype=dtype, device=x.device) if out is None else out.reshape(M, K)
    st = lib().tq_rotate(_ptr(x2), _dtype_code(x2, "x"), M, K, x2.stride(0), sign_mask & 0xFFFFFFFF,
                         _ptr(xr), _dtype_code(xr, "out"), xr.stride(0), _stream())
    _check("tq_rotate", st)
    return xr if x.dim() == 2 else xr.reshape(-1)


def gemv(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, rotated: bool = False,
         sign_mask: int = DEFAULT_SIGN_MASK, out=None):
    """y [N] float32 = W_deq x.  x: [K] raw (fp32/bf16) or, with rotated=True, x' fp32."""
    _dev(packed, "packed")
    _dev(x, "x")
    N, K = packed.shape[0], packed.shape[1] * 2
    if x.numel() != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous vector of length K")
    y = torch.empty(N, dtype=torch.float32, device=packed.device) if out is None else out
    st = lib().tq_gemv(_ptr(packed), _ptr(scales), N, K, sign_mask & 0xFFFFFFFF, _ptr(x), _dtype_code(x, "x"),
                       1 if rotated else 0, _ptr(y), _stream())
    _check("tq_gemv", st)
    return y


def gemm(packed: torch.Tensor, scales: torch.Tensor, x_rot: torch.Tensor, out=None):
    """Y [M, N] float32 = X' Q^T with pre-rotated activations x_rot [M, K] (bf16 or fp32)."""
    _dev(packed, "packed")
    _dev(x_rot, "x_rot")
    N, K = packed.shape[0], packed.shape[1] * 2
    M = x_rot.shape[0]
    if x_rot.dim() != 2 or x_rot.shape[1] != K or x_rot.stride(1) != 1:
        raise ValueError("x_rot must be [M, K] with unit column stride")
    y = torch.empty((M, N), dtype=torch.float32, device=packed.device) if out is None else out
    st = lib().tq_gemm(_ptr(packed), _ptr(scales), N, K, M, _ptr(x_rot), _dtype_code(x_rot, "x_rot"),
                       x_rot.stride(0), _ptr(y), y.stride(0), _stream())
    _check("tq_gemm", st)
    return y


# ----------------------------------------------------------------------------
# NVFP4 / MXFP6
# ----------------------------------------------------------------------------

def blockfp_quantize(fmt: str, W: torch.Tensor, rsf: bool = False):
    """-> (codes uint8, block_scales uint8, tensor_scale float32[1] or None).

    ``rsf=True`` runs the RSF-lite block-scale search (tq_blockfp_quantize_rsf)."""
    _dev(W, "W")
    if not W.is_contiguous():
        raise ValueError("W must be contiguous")
    f = FORMATS[fmt]
    N, K = W.shape
    if fmt == "nvfp4":
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
        bs = torch.empty((N, K // 16), dtype=torch.uint8, device=W.device)
        ts = torch.empty(1, dtype=torch.float32, device=W.device)
    else:
        codes = torch.empty((N, 3 * K // 4), dtype=torch.uint8, device=W.device)
        bs = torch.empty((N, K // 32), dtype=torch.uint8, device=W.device)
        ts = None
    fn = "tq_blockfp_quantize_rsf" if rsf else "tq_blockfp_quantize"
    st = getattr(lib(), fn)(f, _ptr(W), _dtype_code(W, "W"), N, K, _ptr(codes), _ptr(bs), _ptr(ts), _stream())
    _check(fn, st)
    return codes, bs, ts


def blockfp_gemm(fmt: str, codes: torch.Tensor, block_scales: torch.Tensor, tensor_scale, x: torch.Tensor,
                 out=None):
    """Y [M, N] float32 = X W_deq^T (x: [M, K] or [K], fp32/bf16)."""
    _dev(codes, "codes")
    _dev(x, "x")
    f = FORMATS[fmt]
    N = codes.shape[0]
    K = codes.shape[1] * 2 if fmt == "nvfp4" else codes.shape[1] * 4 // 3
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    M = x2.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=codes.device) if out is None else out
    st = lib().tq_blockfp_gemm(f, _ptr(codes), _ptr(block_scales), _ptr(tensor_scale), N, K, M, _ptr(x2),
                               _dtype_code(x2, "x"), x2.stride(0), _ptr(y), y.stride(0), _stream())
    _check("tq_blockfp_gemm", st)
    return y if x.dim() == 2 else y.reshape(-1)


# ----------------------------------------------------------------------------
# load-time int8 transcode
# ----------------------------------------------------------------------------

def transcode_q8(packed: torch.Tensor, scales: torch.Tensor, sign_mask: int = DEFAULT_SIGN_MASK, out=None):
    """TQ4_1S (packed, scales) -> (codes int8 [N, K], q8_scales int16 [N, K/32] = fp16 bits per block)."""
    _dev(packed, "packed")
    N, K = packed.shape[0], packed.shape[1] * 2
    if out is None:
        codes = torch.empty((N, K), dtype=torch.int8, device=packed.device)
        qs = torch.empty((N, K // 32), dtype=torch.int16, device=packed.device)
    else:
        codes, qs = out
    st = lib().tq_transcode_q8(_ptr(packed), _ptr(scales), N, K, sign_mask & 0xFFFFFFFF, _ptr(codes), _ptr(qs),
                               _stream())
    _check("tq_transcode_q8", st)
    return codes, qs


def q8_gemv(codes: torch.Tensor, q8_scales: torch.Tensor, x: torch.Tensor, out=None):
    """y [N] float32 from transcoded int8 weights and the activation x [K] (fp32/bf16, not rotated)."""
    _dev(codes, "codes")
    _dev(x, "x")
    N, K = codes.shape
    if x.numel() != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous vector of length K")
    y = torch.empty(N, dtype=torch.float32, device=codes.device) if out is None else out
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
        if codes.shape != K.shape or scales.shape != K.shape[:-1] + (d // 32,):
            raise ValueError("out shapes do not match K")
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
        if packed.shape != V.shape[:-1] + (d // 2,) or norms.shape != V.shape[:-1]:
            raise ValueError("out shapes do not match V")
    st = lib().tq_kv_quantize_v(_ptr(V), _dtype_code(V, "V"), n, d, sign, _ptr(packed), _ptr(norms), _stream())
    _check("tq_kv_quantize_v", st)
    return packed, norms


def kv_dequantize_v(packed: torch.Tensor, norms: torch.Tensor, sign=None):
    """turbo4 values back to float32 [..., 128]."""
    _dev(packed, "packed")
    d = packed.shape[-1] * 2
    n = packed.numel() // (d // 2)
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
    B, Hq, d = q.shape
    _, Hkv, T_max, _ = k_codes.shape
    if lengths.dtype != torch.int32 or lengths.numel() != B:
        raise ValueError("lengths must be int32 [B]")
    sign = kv_sign_from_seed(0) if sign is None else sign
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device) if out is None else out
    ws_bytes = attn_workspace_bytes(B, Hq, T_max)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=q.device)
    st = lib().tq_attn_decode(_ptr(q), _dtype_code(q, "q"), B, Hq, Hkv, d, T_max, _ptr(lengths), _ptr(k_codes),
                              _ptr(k_scales), _ptr(v_packed), _ptr(v_norms), sign, _ptr(o), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream())
    _check("tq_attn_decode", st)
    return o

