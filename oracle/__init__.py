"""CPU oracle for group-wise quantization and the quantized matmul.

TEST INFRASTRUCTURE ONLY: the independent reference that the HIP library is
checked against. Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. It shares no code with
``quantized_matmul_amd`` and neither package imports the other.

The arithmetic lives in ``qlin_oracle.c`` (plain C loops, fp64 accumulation);
this module only marshals numpy arrays through ctypes. bf16 and f16 arrays
are passed as numpy ``uint16`` bit patterns.

Functions and what they follow (page titles and sections):
  quantize            "EMLX.Quantization" quantize; "Emily.QuantizedWeight"
                      Layout and Microscaled modes table; mlx-rs
                      quantization.rs ``quantize``.
  dequantize          "EMLX.Quantization" dequantize; mlx-rs ``dequantize``.
  quantized_matmul    "EMLX.Quantization" quantized_matmul;
                      "Emily.Quantization.Layers" quantized_dense (layouts);
                      mlx-rs ``quantized_matmul`` and test_quantized_matmul.
  quantized_dense     "Emily.Quantization.Layers" quantized_dense (the bias).
  qqmm                mlx-rs ``qqmm`` (x quantized on the fly, nvfp4/mxfp8).
  gather_qmm          "EMLX.Quantization" gather_quantized_matmul; mlx-rs
                      ``gather_qmm`` and test_gather_qmm.
Readings of points the pages leave open are stated in ``qlin_oracle.c``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "u8": 3}
FORMATS = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3, "e2m1": 4, "e8m0": 5}
ROUNDING = {"nearest_even": 0, "down": 1, "up": 2}
MODE_PAIRING = {"mxfp4": (32, 4), "mxfp8": (32, 8), "nvfp4": (16, 4)}

_lib = None


class OracleError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "qlin_oracle.c")
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    cs = ctypes.c_char_p
    lib.oracle_round.argtypes = [ctypes.c_double, i32, i32]
    lib.oracle_round.restype = ctypes.c_double
    lib.oracle_decode.argtypes = [i32, ctypes.c_uint]
    lib.oracle_decode.restype = ctypes.c_double
    lib.oracle_encode.argtypes = [i32, ctypes.c_double]
    lib.oracle_encode.restype = ctypes.c_uint
    lib.oracle_quantize.argtypes = [vp, i32, i64, i64, i32, i32, cs, vp, vp, vp]
    lib.oracle_dequantize.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, cs, vp, i32]
    lib.oracle_quantized_matmul.argtypes = [vp, i32, i64, i64, vp, vp, vp, i32, i64, i32, i32,
                                            i32, cs, vp]
    lib.oracle_quantized_dense.argtypes = [vp, i32, i64, i64, vp, vp, vp, i32, i64, i32, i32,
                                           i32, cs, vp, i32, ctypes.c_double, vp]
    lib.oracle_qqmm.argtypes = [vp, i32, i64, i64, vp, vp, i64, i32, i32, i32, cs, vp, vp]
    lib.oracle_gather_qmm.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i32, i64, i64, vp, vp,
                                      i64, i32, i32, i32, cs, vp]
    for f in ("oracle_quantize", "oracle_dequantize", "oracle_quantized_matmul",
              "oracle_quantized_dense", "oracle_qqmm", "oracle_gather_qmm"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"oracle {what} rejected its arguments (status {rc})")


def _np_dtype(dt):
    return {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "u8": np.uint8}[dt]


def round_to(v: float, fmt: str, rounding: str = "nearest_even") -> float:
    """Round an exact real to a float format (no overflow handling)."""
    return _load().oracle_round(float(v), FORMATS[fmt], ROUNDING[rounding])


def decode(fmt: str, code: int) -> float:
    return _load().oracle_decode(FORMATS[fmt], int(code))


def encode(fmt: str, v: float) -> int:
    return _load().oracle_encode(FORMATS[fmt], float(v))


def quantize(w: np.ndarray, dtype: str, group_size: int = 64, bits: int = 4,
             mode: str = "affine"):
    """w [..., K] (f32 array, or uint16 bit patterns for bf16/f16).

    Returns (wq uint32 [..., K*bits/32], scales, biases or None); affine scales
    and biases take w's dtype, microscaled scales are uint8 bytes.
    """
    w = np.ascontiguousarray(w)
    K = w.shape[-1]
    rows = int(np.prod(w.shape[:-1])) if w.ndim > 1 else 1
    if w.ndim < 2:
        raise OracleError("quantize needs rank >= 2")
    wq = np.zeros(w.shape[:-1] + (K * bits // 32,), np.uint32)
    G = K // group_size if group_size and K % group_size == 0 else 1
    if mode == "affine":
        scales = np.zeros(w.shape[:-1] + (G,), _np_dtype(dtype))
        biases = np.zeros_like(scales)
    else:
        scales = np.zeros(w.shape[:-1] + (G,), np.uint8)
        biases = None
    rc = _load().oracle_quantize(_ptr(w), DTYPES[dtype], rows, K, group_size, bits,
                                 mode.encode(), _ptr(wq), _ptr(scales), _ptr(biases))
    _check(rc, "quantize")
    return wq, scales, biases


def dequantize(wq, scales, biases, group_size=64, bits=4, mode="affine",
               scale_dtype="f32", out_dtype="f32"):
    """Dense weight [..., K] in out_dtype (f32 array or uint16 bit patterns)."""
    wq = np.ascontiguousarray(wq)
    K = wq.shape[-1] * 32 // bits
    rows = int(np.prod(wq.shape[:-1]))
    out = np.zeros(wq.shape[:-1] + (K,), _np_dtype(out_dtype))
    sd = "u8" if mode != "affine" else scale_dtype
    rc = _load().oracle_dequantize(_ptr(wq), _ptr(np.ascontiguousarray(scales)),
                                   _ptr(None if biases is None else np.ascontiguousarray(biases)),
                                   DTYPES[sd], rows, K, group_size, bits, mode.encode(),
                                   _ptr(out), DTYPES[out_dtype])
    _check(rc, "dequantize")
    return out


def quantized_matmul(x, x_dtype, wq, scales, biases, transpose=True, group_size=64, bits=4,
                     mode="affine", scale_dtype=None):
    """y (float64) = x . dequant(W)^T (transpose) or x . dequant(W).

    x [..., K]; W 2-D: [N, K] packed along K (transpose) or [K, N] packed
    along N. Returns y [..., N] in fp64.
    """
    x = np.ascontiguousarray(x)
    wq = np.ascontiguousarray(wq)
    if transpose:
        N, K = wq.shape[0], wq.shape[1] * 32 // bits
    else:
        K, N = wq.shape[0], wq.shape[1] * 32 // bits
    M = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    y = np.zeros(x.shape[:-1] + (N,), np.float64)
    if x.shape[-1] != K:
        raise OracleError("x's last dim does not match W")
    sd = scale_dtype or ("u8" if mode != "affine" else x_dtype)
    rc = _load().oracle_quantized_matmul(
        _ptr(x), DTYPES[x_dtype], M, x.shape[-1], _ptr(wq), _ptr(np.ascontiguousarray(scales)),
        _ptr(None if biases is None else np.ascontiguousarray(biases)), DTYPES[sd], N,
        int(bool(transpose)), group_size, bits, mode.encode(), _ptr(y))
    _check(rc, "quantized_matmul")
    return y


def quantized_dense(x, x_dtype, wq, scales, biases, bias=None, bias_dtype="f32", bias_value=0.0,
                    transpose=True, group_size=64, bits=4, mode="affine", scale_dtype=None):
    """y (float64) = quantized_matmul(...) + bias.

    bias: N values (one per output column; bf16/f16 as uint16 bits, f32 as
    float32), or None, and then the number bias_value (taken in fp32) is
    added to every output.
    """
    x = np.ascontiguousarray(x)
    wq = np.ascontiguousarray(wq)
    if transpose:
        N, K = wq.shape[0], wq.shape[1] * 32 // bits
    else:
        K, N = wq.shape[0], wq.shape[1] * 32 // bits
    M = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    if x.shape[-1] != K:
        raise OracleError("x's last dim does not match W")
    if bias is not None:
        bias = np.ascontiguousarray(bias)
        if bias.size != N:
            raise OracleError("a tensor bias holds one value per output column")
    y = np.zeros(x.shape[:-1] + (N,), np.float64)
    sd = scale_dtype or ("u8" if mode != "affine" else x_dtype)
    rc = _load().oracle_quantized_dense(
        _ptr(x), DTYPES[x_dtype], M, x.shape[-1], _ptr(wq), _ptr(np.ascontiguousarray(scales)),
        _ptr(None if biases is None else np.ascontiguousarray(biases)), DTYPES[sd], N,
        int(bool(transpose)), group_size, bits, mode.encode(), _ptr(bias), DTYPES[bias_dtype],
        float(bias_value), _ptr(y))
    _check(rc, "quantized_dense")
    return y


def qqmm(x, x_dtype, wq, scales, transpose=True, group_size=16, bits=4, mode="nvfp4",
         return_xhat=False):
    """y (float64) = dequant(quantize(x)) . dequant(W)^T (or . dequant(W)),
    x quantized along its last axis with W's microscaled mode (nvfp4 or
    mxfp8). With return_xhat, also dequant(quantize(x)) as float32."""
    x = np.ascontiguousarray(x)
    wq = np.ascontiguousarray(wq)
    if transpose:
        N, K = wq.shape[0], wq.shape[1] * 32 // bits
    else:
        K, N = wq.shape[0], wq.shape[1] * 32 // bits
    M = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    if x.shape[-1] != K:
        raise OracleError("x's last dim does not match W")
    y = np.zeros(x.shape[:-1] + (N,), np.float64)
    xhat = np.zeros(x.shape, np.float32)
    rc = _load().oracle_qqmm(_ptr(x), DTYPES[x_dtype], M, K, _ptr(wq),
                             _ptr(np.ascontiguousarray(scales)), N, int(bool(transpose)),
                             group_size, bits, mode.encode(), _ptr(xhat), _ptr(y))
    _check(rc, "qqmm")
    return (y, xhat) if return_xhat else y


def gather_qmm(x, x_dtype, wq, scales, biases, rhs_indices, lhs_indices=None, transpose=True,
               group_size=64, bits=4, mode="affine", scale_dtype=None):
    """y[r] = x[lhs[r]] . dequant(W[rhs[r]])^T, fp64.

    Canonical flattened form: x [B, M, K], W [E, N, K] (transpose) or
    [E, K, N]; rhs [R]; lhs [R] or None (then B must equal R). y [R, M, N].
    """
    x = np.ascontiguousarray(x)
    wq = np.ascontiguousarray(wq)
    B, M, Kx = x.shape
    E = wq.shape[0]
    if transpose:
        N, K = wq.shape[1], wq.shape[2] * 32 // bits
    else:
        K, N = wq.shape[1], wq.shape[2] * 32 // bits
    rhs = np.ascontiguousarray(rhs_indices, dtype=np.uint32).ravel()
    lhs = None if lhs_indices is None else np.ascontiguousarray(lhs_indices, np.uint32).ravel()
    R = rhs.size
    y = np.zeros((R, M, N), np.float64)
    if Kx != K:
        raise OracleError("x's last dim does not match W")
    sd = scale_dtype or ("u8" if mode != "affine" else x_dtype)
    rc = _load().oracle_gather_qmm(
        _ptr(x), DTYPES[x_dtype], B, M, Kx, _ptr(wq), _ptr(np.ascontiguousarray(scales)),
        _ptr(None if biases is None else np.ascontiguousarray(biases)), DTYPES[sd], E, N,
        _ptr(lhs), _ptr(rhs), R, int(bool(transpose)), group_size, bits, mode.encode(), _ptr(y))
    _check(rc, "gather_qmm")
    return y
