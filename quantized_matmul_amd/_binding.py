"""ctypes binding of libqlin (argument marshalling only).

Pages followed for the user-facing defaults:
  "Emily.QuantizedWeight" from_dense options: group_size 64, bits 4,
      transpose true, mode "affine"; Microscaled modes table for the
      (group_size, bits) each microscaled mode pins.
  "EMLX.Quantization" gather_quantized_matmul: lhs_indices None takes the
      activation rows in order; sorted_indices lets the kernel skip its sort.
"""
import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqlin.so")

# (group_size, bits) each microscaled mode pins ("Emily.QuantizedWeight")
MODE_DEFAULTS = {"affine": (64, 4), "mxfp4": (32, 4), "mxfp8": (32, 8), "nvfp4": (16, 4)}

_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.uint8: 3}
_STATUS = {1: "invalid argument", 2: "unsupported", 3: "device error"}

_lib = None


class QlinError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"qlin {_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libqlin.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, cs, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_char_p, ctypes.c_size_t
    lib.qlin_quantize.argtypes = [vp, i32, i64, i64, i32, i32, cs, vp, vp, vp, vp]
    lib.qlin_dequantize.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, cs, vp, i32, vp]
    lib.qlin_quantized_matmul.argtypes = [vp, i32, i64, i64, vp, vp, vp, i32, i64, i32, i32, i32,
                                          cs, vp, vp]
    lib.qlin_quantized_dense.argtypes = [vp, i32, i64, i64, vp, vp, vp, i32, i64, i32, i32, i32,
                                         cs, vp, i32, ctypes.c_double, vp, vp]
    lib.qlin_gather_qmm.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i32, i64, i64, vp, vp,
                                    i64, i32, i32, i32, cs, i32, vp, sz, vp, vp]
    lib.qlin_quantized_matmul_ws.argtypes = [vp, i32, i64, i64, vp, vp, vp, i32, i64, i32, i32,
                                             i32, cs, vp, sz, vp, vp]
    lib.qlin_quantized_matmul_ws.restype = i32
    lib.qlin_quantized_matmul_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, cs]
    lib.qlin_quantized_matmul_workspace_bytes.restype = sz
    lib.qlin_qqmm.argtypes = [vp, i32, i64, i64, vp, vp, i64, i32, i32, i32, cs, vp, sz, vp, vp]
    lib.qlin_qqmm.restype = i32
    lib.qlin_qqmm_workspace_bytes.argtypes = [i64, i64]
    lib.qlin_qqmm_workspace_bytes.restype = sz
    lib.qlin_gather_qmm_workspace_bytes.argtypes = [i64, i64]
    lib.qlin_gather_qmm_workspace_bytes.restype = sz
    lib.qlin_gather_qmm_noalloc.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i32, i64, i64,
                                            vp, vp, i64, i32, i32, i32, cs, i32, vp, vp]
    lib.qlin_gather_qmm_noalloc.restype = i32
    lib.qlin_gather_qmm_noalloc_max_rows.restype = sz
    lib.qlin_gather_qmm_noalloc_max_experts.restype = sz
    lib.qlin_last_error.restype = ctypes.c_char_p
    lib.qlin_last_path.restype = ctypes.c_char_p
    for f in ("qlin_quantize", "qlin_dequantize", "qlin_quantized_matmul", "qlin_quantized_dense",
              "qlin_gather_qmm"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def last_path() -> str:
    """Kernel path of this thread's last matmul-type call (qlin_last_path)."""
    return (load_library().qlin_last_path() or b"").decode()


def _check(rc: int):
    if rc != 0:
        raise QlinError(rc, (_lib.qlin_last_error() or b"").decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("qlin tensors live in GPU memory (got a CPU tensor)")
    if not t.is_contiguous():
        raise ValueError("qlin tensors must be contiguous")
    return t.device


@dataclasses.dataclass
class QuantizedWeight:
    """Packed weight plus metadata ("Emily.QuantizedWeight", t() type)."""
    value: torch.Tensor            # uint32 codes, stored as torch.int32
    scales: torch.Tensor
    biases: Optional[torch.Tensor]
    group_size: int
    bits: int
    transpose: bool = True
    mode: str = "affine"

    @property
    def shape(self):
        """Logical (dense) shape."""
        return tuple(self.value.shape[:-1]) + (self.value.shape[-1] * 32 // self.bits,)


def quantize(w: torch.Tensor, group_size: Optional[int] = None, bits: Optional[int] = None,
             mode: str = "affine", transpose: bool = True) -> QuantizedWeight:
    """qlin_quantize on a rank >= 2 tensor, along its last axis."""
    lib = load_library()
    dev = _dev(w)
    if w.dim() < 2:
        raise ValueError("quantize needs a tensor of rank >= 2")
    g0, b0 = MODE_DEFAULTS.get(mode, (64, 4))
    group_size = g0 if group_size is None else group_size
    bits = b0 if bits is None else bits
    if w.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise ValueError("w must be float32, float16 or bfloat16")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    lead = tuple(w.shape[:-1])
    wq = torch.empty(lead + (max(cols * bits // 32, 0),), dtype=torch.int32, device=dev)
    G = cols // group_size if group_size > 0 else 0
    if mode == "affine":
        scales = torch.empty(lead + (G,), dtype=w.dtype, device=dev)
        biases = torch.empty_like(scales)
    else:
        scales = torch.empty(lead + (G,), dtype=torch.uint8, device=dev)
        biases = None
    rc = lib.qlin_quantize(_ptr(w), _DTYPE[w.dtype], rows, cols, group_size, bits, mode.encode(),
                           _ptr(wq), _ptr(scales), _ptr(biases), _stream(dev))
    _check(rc)
    return QuantizedWeight(wq, scales, biases, group_size, bits, transpose, mode)


def dequantize(qw: QuantizedWeight, dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """qlin_dequantize: dense weight of the logical shape (default dtype: the
    scales dtype for affine, float32 for microscaled)."""
    lib = load_library()
    dev = _dev(qw.value)
    if dtype is None:
        dtype = qw.scales.dtype if qw.mode == "affine" else torch.float32
    cols = qw.value.shape[-1] * 32 // qw.bits
    rows = qw.value.numel() // qw.value.shape[-1] if qw.value.shape[-1] else 0
    out = torch.empty(tuple(qw.value.shape[:-1]) + (cols,), dtype=dtype, device=dev)
    rc = lib.qlin_dequantize(_ptr(qw.value), _ptr(qw.scales), _ptr(qw.biases),
                             _DTYPE[qw.scales.dtype], rows, cols, qw.group_size, qw.bits,
                             qw.mode.encode(), _ptr(out), _DTYPE[dtype], _stream(dev))
    _check(rc)
    return out


def _out(out, shape, dtype, dev):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype or not out.is_contiguous() \
            or out.device != dev:
        raise ValueError(f"out must be a contiguous {dtype} tensor of shape {tuple(shape)} on {dev}")
    return out


def quantized_matmul_workspace_bytes(M: int, K: int, N: int, transpose: bool, group_size: int,
                                     bits: int, mode: str = "affine") -> int:
    """qlin_quantized_matmul_workspace_bytes (0: the shape takes none)."""
    return int(load_library().qlin_quantized_matmul_workspace_bytes(
        M, K, N, int(transpose), group_size, bits, mode.encode()))


# Zeroed workspaces for the K-split [in, out] calls, one per (device,
# stream): the library keeps completion counters at the start of the
# workspace, which must be zero before the first call and which every call
# leaves zero, so a workspace is zeroed once (on its stream) and then reused
# by the calls of that stream, which never overlap.
_SPLIT_WS = {}


def _split_workspace(dev: torch.device, nbytes: int) -> torch.Tensor:
    stream = torch.cuda.current_stream(dev)
    key = (dev.index, stream.cuda_stream)
    ws = _SPLIT_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _SPLIT_WS[key] = ws
    return ws


def quantized_matmul(x: torch.Tensor, qw: QuantizedWeight,
                     out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qlin_quantized_matmul: x [..., K] -> y [..., N] in x's dtype.

    W is 2-D: [N, K] packed along K when qw.transpose, else [K, N] packed
    along N ("Emily.Quantization.Layers", quantized_dense). Shapes that take
    a workspace (the [in, out] layout at few bf16 rows, where K is split over
    workgroups) use one zeroed workspace per device and stream, kept for
    later calls, unless `workspace` (a uint8 device tensor whose first 4096
    bytes are zero before its first use) is given; the call then goes to
    qlin_quantized_matmul_ws.
    """
    lib = load_library()
    dev = _dev(x)
    _dev(qw.value)
    if qw.value.dim() != 2:
        raise ValueError("quantized_matmul takes a 2-D quantized weight")
    per = 32 // qw.bits
    if qw.transpose:
        N, K = qw.value.shape[0], qw.value.shape[1] * per
    else:
        K, N = qw.value.shape[0], qw.value.shape[1] * per
    if x.shape[-1] != K:
        raise ValueError(f"x's last dim {x.shape[-1]} does not match the weight's K={K}")
    M = x.numel() // K if K else 0
    y = _out(out, tuple(x.shape[:-1]) + (N,), x.dtype, dev)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
    elif not qw.transpose and x.dtype == torch.bfloat16 and 1 <= M <= 8:
        ws_bytes = quantized_matmul_workspace_bytes(M, K, N, False, qw.group_size, qw.bits, qw.mode)
        if ws_bytes:
            workspace = _split_workspace(dev, ws_bytes)
            ws_bytes = workspace.numel()
    if ws_bytes:
        rc = lib.qlin_quantized_matmul_ws(_ptr(x), _DTYPE[x.dtype], M, K, _ptr(qw.value),
                                          _ptr(qw.scales), _ptr(qw.biases),
                                          _DTYPE[qw.scales.dtype], N, int(qw.transpose),
                                          qw.group_size, qw.bits, qw.mode.encode(),
                                          _ptr(workspace), ws_bytes, _ptr(y), _stream(dev))
    else:
        rc = lib.qlin_quantized_matmul(_ptr(x), _DTYPE[x.dtype], M, K, _ptr(qw.value),
                                       _ptr(qw.scales), _ptr(qw.biases), _DTYPE[qw.scales.dtype],
                                       N, int(qw.transpose), qw.group_size, qw.bits,
                                       qw.mode.encode(), _ptr(y), _stream(dev))
    _check(rc)
    return y


def quantized_dense(x: torch.Tensor, qw: QuantizedWeight, bias=0,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qlin_quantized_dense: x @ W (+ bias) ("Emily.Quantization.Layers",
    quantized_dense). bias is a number, or a float tensor of N values (one
    per output column) on x's device; it is added in fp32 before the output's
    one rounding.
    """
    lib = load_library()
    dev = _dev(x)
    _dev(qw.value)
    if qw.value.dim() != 2:
        raise ValueError("quantized_dense takes a 2-D quantized weight")
    per = 32 // qw.bits
    if qw.transpose:
        N, K = qw.value.shape[0], qw.value.shape[1] * per
    else:
        K, N = qw.value.shape[0], qw.value.shape[1] * per
    if x.shape[-1] != K:
        raise ValueError(f"x's last dim {x.shape[-1]} does not match the weight's K={K}")
    bias_t, bias_value, bias_dt = None, 0.0, _DTYPE[torch.float32]
    if isinstance(bias, torch.Tensor):
        _dev(bias)
        if bias.device != dev:
            raise ValueError("bias must be on x's device")
        if bias.numel() != N or bias.dim() < 1 or bias.shape[-1] != N:
            raise ValueError(f"a tensor bias holds one value per output column ({N})")
        if bias.dtype not in (torch.float32, torch.bfloat16, torch.float16):
            raise ValueError("bias must be float32, bfloat16 or float16")
        bias_t = bias.contiguous()
        bias_dt = _DTYPE[bias_t.dtype]
    else:
        bias_value = float(bias)
    M = x.numel() // K if K else 0
    y = _out(out, tuple(x.shape[:-1]) + (N,), x.dtype, dev)
    rc = lib.qlin_quantized_dense(_ptr(x), _DTYPE[x.dtype], M, K, _ptr(qw.value),
                                  _ptr(qw.scales), _ptr(qw.biases), _DTYPE[qw.scales.dtype], N,
                                  int(qw.transpose), qw.group_size, qw.bits, qw.mode.encode(),
                                  _ptr(bias_t), bias_dt, bias_value, _ptr(y), _stream(dev))
    _check(rc)
    return y


def qqmm_workspace_bytes(M: int, K: int) -> int:
    return int(load_library().qlin_qqmm_workspace_bytes(M, K))


def qqmm(x: torch.Tensor, qw: QuantizedWeight, workspace: Optional[torch.Tensor] = None,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qlin_qqmm (mlx-rs qqmm): bf16 x quantized on the fly with qw's mode
    (nvfp4 or mxfp8), times the quantized weight. x [..., K] -> y [..., N]."""
    lib = load_library()
    dev = _dev(x)
    _dev(qw.value)
    if qw.value.dim() != 2:
        raise ValueError("qqmm takes a 2-D quantized weight")
    per = 32 // qw.bits
    if qw.transpose:
        N, K = qw.value.shape[0], qw.value.shape[1] * per
    else:
        K, N = qw.value.shape[0], qw.value.shape[1] * per
    if x.shape[-1] != K:
        raise ValueError(f"x's last dim {x.shape[-1]} does not match the weight's K={K}")
    M = x.numel() // K if K else 0
    need = qqmm_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    y = _out(out, tuple(x.shape[:-1]) + (N,), x.dtype, dev)
    rc = lib.qlin_qqmm(_ptr(x), _DTYPE[x.dtype], M, K, _ptr(qw.value), _ptr(qw.scales), N,
                       int(qw.transpose), qw.group_size, qw.bits, qw.mode.encode(),
                       _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(y),
                       _stream(dev))
    _check(rc)
    return y


def gather_qmm_workspace_bytes(R: int, E: int) -> int:
    return int(load_library().qlin_gather_qmm_workspace_bytes(R, E))


def _gather_prep(x, qw, rhs_indices, lhs_indices):
    """Shapes and flattened int32 index arrays of a gather call (no copy
    when the indices are already contiguous int32 tensors on x's device and
    lhs, if given, has rhs's shape)."""
    dev = _dev(x)
    if x.dim() != 3 or qw.value.dim() != 3:
        raise ValueError("gather_qmm takes x [B, M, K] and a stacked weight [E, ., .]")
    B, M, K = x.shape
    E = qw.value.shape[0]
    per = 32 // qw.bits
    N = qw.value.shape[1] if qw.transpose else qw.value.shape[2] * per
    Kw = qw.value.shape[2] * per if qw.transpose else qw.value.shape[1]
    if Kw != K:
        raise ValueError(f"x's last dim {K} does not match the weight's K={Kw}")
    rhs = rhs_indices.to(device=dev, dtype=torch.int32)
    shape = tuple(rhs.shape)
    lhs = None
    if lhs_indices is not None:
        lhs_b, rhs_b = torch.broadcast_tensors(lhs_indices.to(device=dev, dtype=torch.int32), rhs)
        shape = tuple(rhs_b.shape)
        lhs = lhs_b.contiguous().reshape(-1)
        rhs = rhs_b.contiguous().reshape(-1)
    else:
        rhs = rhs.contiguous().reshape(-1)
    return dev, B, M, K, E, N, shape, lhs, rhs


def gather_qmm(x: torch.Tensor, qw: QuantizedWeight, rhs_indices: torch.Tensor,
               lhs_indices: Optional[torch.Tensor] = None, sorted_indices: bool = False,
               workspace: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qlin_gather_qmm: y[r] = x[lhs[r]] . W[rhs[r]]^T (or . W[rhs[r]]).

    x [B, M, K]; qw.value stacks experts on its leading axis; rhs_indices
    (and lhs_indices, broadcast against it) of any shape S. Returns
    y of shape S + (M, N). ("EMLX.Quantization", gather_quantized_matmul.)
    """
    lib = load_library()
    dev, B, M, K, E, N, shape, lhs, rhs = _gather_prep(x, qw, rhs_indices, lhs_indices)
    R = rhs.numel()
    need = int(lib.qlin_gather_qmm_workspace_bytes(R, E))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    y = _out(out, shape + (M, N), x.dtype, dev)
    rc = lib.qlin_gather_qmm(_ptr(x), _DTYPE[x.dtype], B, M, K, _ptr(qw.value), _ptr(qw.scales),
                             _ptr(qw.biases), _DTYPE[qw.scales.dtype], E, N, _ptr(lhs), _ptr(rhs),
                             R, int(qw.transpose), qw.group_size, qw.bits, qw.mode.encode(),
                             int(bool(sorted_indices)), _ptr(workspace), workspace.numel(),
                             _ptr(y), _stream(dev))
    _check(rc)
    return y


def gather_qmm_noalloc(x: torch.Tensor, qw: QuantizedWeight, rhs_indices: torch.Tensor,
                       lhs_indices: Optional[torch.Tensor] = None, sorted_indices: bool = False,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qlin_gather_qmm_noalloc: gather_qmm with the library's own fixed
    scratch instead of a workspace (at most 65536 index rows and 4096
    experts). The C call allocates nothing; this wrapper allocates only y
    when `out` is not given and index copies when the indices are not
    contiguous int32 tensors of one shape on x's device."""
    lib = load_library()
    dev, B, M, K, E, N, shape, lhs, rhs = _gather_prep(x, qw, rhs_indices, lhs_indices)
    R = rhs.numel()
    y = _out(out, shape + (M, N), x.dtype, dev)
    rc = lib.qlin_gather_qmm_noalloc(_ptr(x), _DTYPE[x.dtype], B, M, K, _ptr(qw.value),
                                     _ptr(qw.scales), _ptr(qw.biases), _DTYPE[qw.scales.dtype], E,
                                     N, _ptr(lhs), _ptr(rhs), R, int(qw.transpose), qw.group_size,
                                     qw.bits, qw.mode.encode(), int(bool(sorted_indices)), _ptr(y),
                                     _stream(dev))
    _check(rc)
    return y
