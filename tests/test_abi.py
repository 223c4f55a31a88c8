"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects every invalid argument before touching the device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")
LIB = os.path.join(ROOT, "quantized_matmul_amd", "libqlin.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libqlin.so not built")

INVALID, UNSUPPORTED = 1, 2
F32, F16, BF16, U8 = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qlin_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from quantized_matmul_amd import _binding
    return _binding.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"qlin_quantize", "qlin_dequantize", "qlin_quantized_matmul",
                          "qlin_quantized_dense", "qlin_gather_qmm",
                          "qlin_gather_qmm_workspace_bytes", "qlin_last_error"}
    for n in names:
        assert hasattr(lib, n), n


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation rejects first


def err(lib):
    return lib.qlin_last_error().decode()


@pytest.mark.parametrize("mode,g,b", [("mxfp4", 64, 4), ("mxfp4", 32, 8), ("mxfp8", 32, 4),
                                      ("nvfp4", 32, 4), ("nvfp4", 16, 8), ("affine", 64, 3),
                                      ("affine", 64, 6), ("affine", 16, 4), ("affine", 48, 4),
                                      ("int4", 64, 4)])
def test_quantize_rejects_bad_mode_pairing(lib, mode, g, b):
    rc = lib.qlin_quantize(FAKE, F32, 4, 256, g, b, mode.encode(), FAKE, FAKE,
                           FAKE if mode == "affine" else None, None)
    assert rc == INVALID
    assert err(lib)


def test_quantize_rejects_bad_shapes_and_pointers(lib):
    assert lib.qlin_quantize(FAKE, F32, 4, 96, 64, 4, b"affine", FAKE, FAKE, FAKE, None) == INVALID
    assert "multiple of group_size" in err(lib)
    assert lib.qlin_quantize(FAKE, U8, 4, 128, 64, 4, b"affine", FAKE, FAKE, FAKE, None) == INVALID
    assert lib.qlin_quantize(FAKE, F32, 4, 128, 64, 4, b"affine", FAKE, FAKE, None, None) == INVALID
    assert "biases" in err(lib)
    assert lib.qlin_quantize(FAKE, F32, 4, 128, 32, 4, b"mxfp4", FAKE, FAKE, FAKE, None) == INVALID
    assert lib.qlin_quantize(None, F32, 4, 128, 64, 4, b"affine", FAKE, FAKE, FAKE, None) == INVALID
    assert lib.qlin_quantize(FAKE, F32, -1, 128, 64, 4, b"affine", FAKE, FAKE, FAKE, None) == INVALID
    assert lib.qlin_quantize(FAKE, F32, 4, 128, 64, 4, None, FAKE, FAKE, FAKE, None) == INVALID
    # empty input is a no-op that touches nothing
    assert lib.qlin_quantize(None, F32, 0, 128, 64, 4, b"affine", None, None, FAKE, None) == 0


def test_dequantize_rejects(lib):
    assert lib.qlin_dequantize(FAKE, FAKE, FAKE, U8, 4, 128, 64, 4, b"affine", FAKE, F32, None) == INVALID
    assert lib.qlin_dequantize(FAKE, FAKE, None, F32, 4, 128, 64, 4, b"affine", FAKE, F32, None) == INVALID
    assert lib.qlin_dequantize(FAKE, FAKE, FAKE, U8, 4, 128, 32, 4, b"mxfp4", FAKE, F32, None) == INVALID
    assert lib.qlin_dequantize(FAKE, FAKE, None, BF16, 4, 128, 32, 4, b"mxfp4", FAKE, F32, None) == INVALID
    assert lib.qlin_dequantize(FAKE, FAKE, None, U8, 4, 128, 32, 4, b"mxfp4", FAKE, U8, None) == INVALID


def test_quantized_matmul_rejects(lib):
    q = lib.qlin_quantized_matmul
    # K not a multiple of the group (transpose: groups run along K)
    assert q(FAKE, BF16, 1, 100, FAKE, FAKE, FAKE, BF16, 64, 1, 64, 4, b"affine", FAKE, None) == INVALID
    # transpose=false: groups run along N
    assert q(FAKE, BF16, 1, 128, FAKE, FAKE, FAKE, BF16, 100, 0, 64, 4, b"affine", FAKE, None) == INVALID
    # affine output follows the scales dtype: x must match it
    assert q(FAKE, F32, 1, 128, FAKE, FAKE, FAKE, BF16, 64, 1, 64, 4, b"affine", FAKE, None) == INVALID
    assert "dtype" in err(lib)
    # microscaled: u8 scales, no biases
    assert q(FAKE, BF16, 1, 128, FAKE, FAKE, FAKE, U8, 64, 1, 32, 4, b"mxfp4", FAKE, None) == INVALID
    assert q(FAKE, BF16, 1, 128, FAKE, FAKE, None, BF16, 64, 1, 32, 4, b"mxfp4", FAKE, None) == INVALID
    assert q(FAKE, BF16, -1, 128, FAKE, FAKE, FAKE, BF16, 64, 1, 64, 4, b"affine", FAKE, None) == INVALID
    assert q(FAKE, BF16, 1, 0, FAKE, FAKE, FAKE, BF16, 64, 1, 64, 4, b"affine", FAKE, None) == INVALID
    assert q(None, BF16, 1, 128, FAKE, FAKE, FAKE, BF16, 64, 1, 64, 4, b"affine", FAKE, None) == INVALID
    # M == 0 is an empty product: no-op, no device call
    assert q(None, BF16, 0, 128, None, None, FAKE, BF16, 64, 1, 64, 4, b"affine", None, None) == 0


def test_quantized_dense_rejects(lib):
    d = lib.qlin_quantized_dense
    base = dict(x=FAKE, xdt=BF16, M=1, K=128, wq=FAKE, s=FAKE, b=FAKE, sdt=BF16, N=64, t=1, g=64,
                bits=4, mode=b"affine", bias=None, bdt=F32, bval=0.0, y=FAKE, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return d(*a.values())

    assert call(bias=FAKE, bdt=U8) == INVALID             # bias dtype: f32, f16 or bf16
    assert "bias" in err(lib)
    assert call(bias=ctypes.c_void_p(0x1002), bdt=F32) == INVALID   # not 4-byte aligned
    assert call(bias=ctypes.c_void_p(0x1001), bdt=BF16) == INVALID  # not 2-byte aligned
    assert call(bval=float("inf")) == INVALID
    assert call(bval=float("nan")) == INVALID
    assert call(bval=1e39) == INVALID                     # finite in fp64, not in fp32
    # the matmul's own checks still apply
    assert call(K=100) == INVALID
    assert call(xdt=F32) == INVALID
    # M == 0: no-op, no device call (the bias is checked first)
    assert call(x=None, M=0, wq=None, s=None, y=None, bias=FAKE, bdt=BF16) == 0


def test_quantized_matmul_ws_sizes_and_rejects(lib):
    """The workspace query names the [in, out] layout at 1..8 rows only, and
    the workspace entry point keeps qlin_quantized_matmul's checks."""
    nb = lib.qlin_quantized_matmul_workspace_bytes
    need = nb(1, 4096, 14336, 0, 64, 4, b"affine")
    # 4096 bytes of completion counters, then whole fp32 partial rows
    assert need > 4096 and (need - 4096) % (14336 * 4) == 0
    assert nb(4, 4096, 14336, 0, 64, 4, b"affine") > 0
    assert nb(8, 4096, 14336, 0, 64, 4, b"affine") == 0  # 5..8 rows: one-pass kernel
    assert nb(1, 4096, 14336, 1, 64, 4, b"affine") == 0  # [out, in] layout: none
    assert nb(0, 4096, 14336, 0, 64, 4, b"affine") == 0
    assert nb(9, 4096, 14336, 0, 64, 4, b"affine") == 0
    assert nb(4, 4096, 14336, 0, 32, 2, b"affine") == 0  # 2-bit codes: one or two rows
    assert nb(1, 4096, 14336, 0, 64, 3, b"affine") == 0  # invalid format
    assert nb(1, 8192, 8192, 0, 32, 4, b"mxfp4") > 0
    f = lib.qlin_quantized_matmul_ws
    WS = ctypes.c_void_p(0x2000)
    base = dict(x=FAKE, xdt=BF16, M=1, K=4096, wq=FAKE, s=FAKE, b=FAKE, sdt=BF16, N=14336, t=0,
                g=64, bits=4, mode=b"affine", ws=WS, wsb=need, y=FAKE, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())

    assert call(ws=ctypes.c_void_p(0x2008)) == INVALID   # 16-byte alignment
    assert "workspace" in err(lib)
    assert call(N=100) == INVALID                        # groups run along N
    assert call(xdt=F32) == INVALID                      # affine: x dtype = scales dtype
    assert call(x=None) == INVALID
    assert call(M=0, x=None, ws=None, wsb=0) == 0        # empty: no-op


def test_qqmm_rejects(lib):
    q = lib.qlin_qqmm
    need = lib.qlin_qqmm_workspace_bytes(2, 128)
    assert need == 2 * 128 * 2
    WS = ctypes.c_void_p(0x2000)
    base = dict(x=FAKE, xdt=BF16, M=2, K=128, wq=FAKE, s=FAKE, N=64, t=1, g=32, bits=8,
                mode=b"mxfp8", ws=WS, wsb=need, y=FAKE, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return q(*a.values())

    assert call(mode=b"mxfp4", g=32, bits=4) == INVALID      # nvfp4 and mxfp8 only
    assert "nvfp4" in err(lib)
    assert call(mode=b"affine", g=64, bits=4) == INVALID
    assert call(mode=b"nvfp4", g=32, bits=4) == INVALID      # pairing
    assert call(xdt=F32) == UNSUPPORTED                      # bf16 x only
    assert call(wsb=need - 1) == INVALID
    assert call(ws=None) == INVALID
    assert call(ws=ctypes.c_void_p(0x2008)) == INVALID       # 16-byte alignment
    assert call(t=0, N=100) == INVALID                       # [K, N] groups run along N
    assert call(t=0, K=100, N=64) == INVALID                 # x's groups run along K
    assert call(x=None) == INVALID
    assert call(M=0, x=None, ws=None, wsb=0) == 0            # empty: no-op


def test_gather_rejects(lib):
    g = lib.qlin_gather_qmm
    need = lib.qlin_gather_qmm_workspace_bytes(8, 4)
    assert need > 0
    args = dict(x=FAKE, xdt=BF16, B=8, M=1, K=128, wq=FAKE, s=FAKE, b=FAKE, sdt=BF16, E=4, N=64,
                lhs=None, rhs=FAKE, R=8, t=1, g=64, bits=4, mode=b"affine", sorted=0, ws=FAKE,
                wsb=need, y=FAKE, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return g(*a.values())

    assert call(B=5) == INVALID                 # lhs NULL needs B == R
    assert "B == R" in err(lib)
    assert call(wsb=need - 1) == INVALID        # workspace too small
    assert call(ws=None) == INVALID
    assert call(rhs=None) == INVALID
    assert call(E=0) == INVALID
    assert call(mode=b"mxfp8", g=32, bits=8, sdt=U8, b=None, K=100) == INVALID
    assert call(R=0, B=0) == 0                  # empty: no-op


def test_gather_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """The allocation-free gather refuses problems its fixed scratch cannot
    hold, before touching any pointer or the device."""
    assert lib.qlin_gather_qmm_noalloc_max_rows() == 65536
    assert lib.qlin_gather_qmm_noalloc_max_experts() == 4096
    args = lambda R, E: (FAKE, BF16, R, 1, 512, FAKE, FAKE, FAKE, BF16, E, 256, None, FAKE, R, 1,
                         64, 4, b"affine", 0, FAKE, None)
    assert lib.qlin_gather_qmm_noalloc(*args(65537, 64)) == INVALID
    assert "at most 65536 index rows" in err(lib)
    assert lib.qlin_gather_qmm_noalloc(*args(16, 4097)) == INVALID
    # empty problem: a no-op that needs no scratch
    assert lib.qlin_gather_qmm_noalloc(FAKE, BF16, 0, 1, 512, FAKE, FAKE, FAKE, BF16, 8, 256, None,
                                       FAKE, 0, 1, 64, 4, b"affine", 0, FAKE, None) == 0


def test_last_path_is_exported(lib):
    assert lib.qlin_last_path() is not None
