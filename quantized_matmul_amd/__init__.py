"""quantized_matmul_amd -- group-wise quantized matmul for AMD MI355X (gfx950).

A thin Python layer over the C ABI in ``include/qlin.h`` (``libqlin.so``,
hand-written HIP kernels). This module only marshals arguments: PyTorch
provides device memory and the current HIP stream, every step of the
computation runs in the library's kernels. There is no CPU fallback: if the
library is not built, every call raises.

Raw ABI calls (same names as the C functions, minus the ``qlin_`` prefix):
``quantize``, ``dequantize``, ``quantized_matmul``, ``quantized_dense``,
``qqmm``, ``gather_qmm`` operate on explicit tensors. ``QuantizedWeight`` bundles the packed weight with its
metadata, mirroring the field set of the "Emily.QuantizedWeight" page
(value, scales, biases, group_size, bits, transpose, mode).
"""
from ._binding import (  # noqa: F401
    QlinError,
    QuantizedWeight,
    dequantize,
    gather_qmm,
    gather_qmm_noalloc,
    gather_qmm_workspace_bytes,
    last_path,
    library_path,
    load_library,
    quantize,
    qqmm,
    qqmm_workspace_bytes,
    quantized_dense,
    quantized_matmul,
    quantized_matmul_workspace_bytes,
    MODE_DEFAULTS,
)
