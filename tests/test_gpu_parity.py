"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Bars: codes, packed words, scales and biases bit-exact; dequantized values
bit-exact; matmul outputs within normwise max relative error 1e-5*sqrt(K)
(fp32 outputs) or 2e-2 (bf16/f16 outputs). Every input is seeded synthetic
data drawn by ``synth``.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import ORACLE_DT, from_bits, normwise_rel_err, to_oracle, tolerance

pytestmark = pytest.mark.gpu

qm = pytest.importorskip("quantized_matmul_amd")

DEV = "cuda:0"
AFFINE_CASES = [(2, 32), (2, 64), (2, 128), (4, 32), (4, 64), (4, 128), (8, 32), (8, 64), (8, 128)]
MICRO_CASES = [("mxfp4", 32, 4), ("mxfp8", 32, 8), ("nvfp4", 16, 4)]
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(autouse=True)
def _no_forced_path():
    os.environ.pop("QLIN_FORCE_PATH", None)
    yield
    os.environ.pop("QLIN_FORCE_PATH", None)


def gpu_weight(shape, std, wid, dtype):
    t, bits = synth.normal(shape, std, wid, synth.WEIGHT, dtype)
    return t.to(DEV), bits


def quantize_both(w_gpu, w_bits, dtype, g, b, mode, transpose=True):
    qw = qm.quantize(w_gpu, g, b, mode, transpose=transpose)
    ref = oracle.quantize(w_bits, dtype, g, b, mode)
    return qw, ref


# ---------------------------------------------------------------- quantize

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("bits,g", AFFINE_CASES)
def test_quantize_affine_bit_exact(dtype, bits, g):
    print(f"quantize affine {dtype} b{bits} g{g}", flush=True)
    w, wb = gpu_weight((37, 512), 0.02, 11, dtype)      # ragged row count
    qw, (wq, sc, bi) = quantize_both(w, wb, dtype, g, bits, "affine")
    torch.cuda.synchronize()
    assert np.array_equal(to_oracle(qw.value), wq)
    assert np.array_equal(to_oracle(qw.scales), sc)
    assert np.array_equal(to_oracle(qw.biases), bi)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("mode,g,bits", MICRO_CASES)
def test_quantize_micro_bit_exact(dtype, mode, g, bits):
    print(f"quantize {mode} {dtype}", flush=True)
    w, wb = gpu_weight((29, 512), 0.02, 12, dtype)
    qw, (wq, sc, _) = quantize_both(w, wb, dtype, g, bits, mode)
    torch.cuda.synchronize()
    assert qw.biases is None
    assert np.array_equal(to_oracle(qw.scales), sc)
    assert np.array_equal(to_oracle(qw.value), wq)


def test_quantize_special_values_bit_exact():
    """Constant groups, signed zeros, tiny and large magnitudes, exact ties."""
    r = np.random.default_rng(5)
    a = np.zeros((8, 128), np.float32)
    a[0] = 0.25                                   # constant group
    a[1, :64] = -0.0
    a[1, 64:] = 0.0
    a[2] = r.standard_normal(128) * 1e-30         # subnormal-scale groups
    a[3] = r.standard_normal(128) * 1e30
    a[4] = np.tile(np.array([0, 0.5, 1, 1.5, 2, 2.5, 3, 3.5, 5, 6, 7], np.float32), 12)[:128]
    a[5] = np.arange(128, dtype=np.float32) - 64
    a[6] = r.integers(-3, 4, 128)
    a[7] = r.standard_normal(128) * 300
    for dtype in ("f32", "bf16"):
        t, bits = synth.as_dtype(a, dtype)
        for (mode, g, b) in [("affine", 32, 4), ("affine", 64, 2), ("affine", 128, 8)] + MICRO_CASES:
            qw, (wq, sc, bi) = quantize_both(t.to(DEV), bits, dtype, g, b, mode)
            torch.cuda.synchronize()
            assert np.array_equal(to_oracle(qw.value), wq), (dtype, mode)
            assert np.array_equal(to_oracle(qw.scales), sc), (dtype, mode)
            if bi is not None:
                assert np.array_equal(to_oracle(qw.biases), bi), (dtype, mode)


def _nudge(v, k):
    to = np.float32(np.inf if k > 0 else -np.inf)
    v = np.float32(v)
    for _ in range(abs(k)):
        v = np.nextafter(v, to, dtype=np.float32)
    return v


@pytest.mark.parametrize("bits,a,k", [(8, 3, 0), (8, 63, 4), (4, 3, 6), (4, 11, 2), (2, 15, 9), (2, 25, 3)])
def test_quantize_affine_quotient_edges(bits, a, k):
    """The kernels' fp32 quotient d/s (an fp64 reciprocal product rounded
    to fp32) against the oracle's IEEE division where it matters most:
    groups with bias 0 and scale s = a*2^-k, elements on each half-step
    (m + 1/2)*s and 1-2 ulps around it, so the codes turn on the exact
    rounding of the quotient and on ties going to even."""
    n = (1 << bits) - 1
    g = 64
    s = np.float32(a * 2.0 ** -k)
    vals = []
    for m in range(n):
        tie = np.float32((m + 0.5) * s)
        vals += [tie] + [_nudge(tie, d) for d in (-2, -1, 1, 2)]
    per = g - 2
    vals += [vals[-1]] * (-len(vals) % per)
    rows = np.array(vals, np.float32).reshape(-1, per)
    w = np.concatenate([np.zeros((len(rows), 1), np.float32),
                        np.full((len(rows), 1), np.float32(n * s)), rows], axis=1)
    wq, sc, bi = oracle.quantize(w, "f32", g, bits)
    qw = qm.quantize(torch.from_numpy(w).to(DEV), g, bits)
    torch.cuda.synchronize()
    assert np.array_equal(to_oracle(qw.scales), sc)
    assert np.array_equal(to_oracle(qw.value), wq)


def test_quantize_quotient_random_scales():
    """Random fp32 groups whose magnitudes span 2^-120 .. 2^120 (a different
    scale exponent per group, normal and subnormal quotients alike): codes,
    scales and biases bit-exact for affine 2/4/8-bit and nvfp4, whose
    elements divide by the decoded E4M3 scale."""
    r = np.random.default_rng(77)
    rows, K = 512, 512
    mag = np.float32(2.0) ** r.integers(-120, 121, size=(rows, K // 16)).astype(np.float32)
    w = (r.standard_normal((rows, K)).astype(np.float32) * np.repeat(mag, 16, axis=1)).astype(np.float32)
    wt = torch.from_numpy(w).to(DEV)
    for mode, g, bits in [("affine", 64, 4), ("affine", 32, 2), ("affine", 128, 8), ("nvfp4", 16, 4)]:
        wq, sc, bi = oracle.quantize(w, "f32", g, bits, mode)
        qw = qm.quantize(wt, g, bits, mode)
        torch.cuda.synchronize()
        assert np.array_equal(to_oracle(qw.scales), sc), mode
        assert np.array_equal(to_oracle(qw.value), wq), mode
        if bi is not None:
            assert np.array_equal(to_oracle(qw.biases), bi), mode


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode,g,bits", [("affine", 64, 4), ("affine", 32, 2), ("affine", 128, 8)] + MICRO_CASES)
def test_quantize_dequantize_unaligned_pointers(dtype, mode, g, bits):
    """Input and output one element off a 16-byte boundary (element-wise
    loads and stores instead of vector ones): the same bits as aligned."""
    import ctypes
    w, wb = gpu_weight((21, 256), 0.02, 14, dtype)
    buf = torch.empty(w.numel() + 1, dtype=w.dtype, device=DEV)
    wu = buf[1:].view(w.shape)
    wu.copy_(w)
    assert wu.data_ptr() % 16 != 0
    qa = qm.quantize(w, g, bits, mode)
    qu = qm.quantize(wu, g, bits, mode)
    odt = torch.bfloat16
    da = qm.dequantize(qa, odt)
    obuf = torch.empty(da.numel() + 1, dtype=odt, device=DEV)
    lib = qm.load_library()
    vp = ctypes.c_void_p
    rows, cols = w.shape
    rc = lib.qlin_dequantize(vp(qa.value.data_ptr()), vp(qa.scales.data_ptr()),
                             vp(qa.biases.data_ptr()) if qa.biases is not None else None,
                             {torch.float32: 0, torch.bfloat16: 2, torch.float16: 1, torch.uint8: 3}[qa.scales.dtype],
                             rows, cols, g, bits, mode.encode(), vp(obuf[1:].data_ptr()), 2,
                             vp(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(qu.value, qa.value) and torch.equal(qu.scales.view(torch.uint8), qa.scales.view(torch.uint8))
    if qa.biases is not None:
        assert torch.equal(qu.biases.view(torch.uint8), qa.biases.view(torch.uint8))
    assert torch.equal(obuf[1:].view(da.shape).view(torch.int16), da.view(torch.int16))


# ---------------------------------------------------------------- dequantize

@pytest.mark.parametrize("sdtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("odtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("bits,g", [(2, 32), (4, 64), (8, 128)])
def test_dequantize_affine_bit_exact(sdtype, odtype, bits, g):
    w, wb = gpu_weight((19, 256), 0.5, 13, sdtype)
    qw, (wq, sc, bi) = quantize_both(w, wb, sdtype, g, bits, "affine")
    d = qm.dequantize(qw, TDT[odtype])
    ref = oracle.dequantize(wq, sc, bi, g, bits, "affine", sdtype, odtype)
    torch.cuda.synchronize()
    assert np.array_equal(to_oracle(d), ref)


@pytest.mark.parametrize("odtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode,g,bits", MICRO_CASES)
def test_dequantize_micro_bit_exact(odtype, mode, g, bits):
    w, wb = gpu_weight((19, 256), 0.5, 14, "bf16")
    qw, (wq, sc, _) = quantize_both(w, wb, "bf16", g, bits, mode)
    d = qm.dequantize(qw, TDT[odtype])
    ref = oracle.dequantize(wq, sc, None, g, bits, mode, "u8", odtype)
    torch.cuda.synchronize()
    assert np.array_equal(to_oracle(d), ref)


def test_roundtrip_rs_example():
    """mlx-rs test_quantize_dequantize shapes and bound, on the GPU."""
    x = torch.arange(512, dtype=torch.float32).repeat(128, 1).to(DEV)
    for b in (2, 4, 8):
        qw = qm.quantize(x, 128, b)
        assert tuple(qw.value.shape) == (128, 512 // (32 // b))
        assert tuple(qw.scales.shape) == (128, 4) and tuple(qw.biases.shape) == (128, 4)
        xh = qm.dequantize(qw)
        assert float((x - xh).abs().max()) <= 127.0 / (1 << b)


# ---------------------------------------------------------------- matmul

def run_qmm_case(M, N, K, bits, g, mode, xdtype, transpose, path=None, wid=20, std=0.02):
    wdt = xdtype if mode == "affine" else "bf16"
    wshape = (N, K) if transpose else (K, N)
    w, wb = gpu_weight(wshape, std, wid, wdt)
    xt, xb = synth.normal((M, K), 1.0, wid, synth.ACT, xdtype)
    qw, (wq, sc, bi) = quantize_both(w, wb, wdt, g, bits, mode, transpose)
    if path:
        os.environ["QLIN_FORCE_PATH"] = path
    y = qm.quantized_matmul(xt.to(DEV), qw)
    torch.cuda.synchronize()
    os.environ.pop("QLIN_FORCE_PATH", None)
    yref = oracle.quantized_matmul(xb, xdtype, wq, sc, bi, transpose, g, bits, mode,
                                   scale_dtype=(wdt if mode == "affine" else "u8"))
    assert y.shape == (M, N) and y.dtype == TDT[xdtype]
    err = normwise_rel_err(y, yref)
    tol = tolerance(TDT[xdtype], K)
    print(f"qmm M{M} N{N} K{K} b{bits} g{g} {mode} {xdtype} t{int(transpose)} path={path}: "
          f"err {err:.3e} tol {tol:.1e}", flush=True)
    assert err <= tol
    return err


def test_tiny_affine_config():
    """W f32 [256,512] ~N(0,0.02) int4 g64, x f32 [4,512] ~N(0,1):
    quantize -> dequantize -> quantized_matmul."""
    w, wb = gpu_weight((256, 512), 0.02, 1, "f32")
    xt, xb = synth.normal((4, 512), 1.0, 1, synth.ACT, "f32")
    qw, (wq, sc, bi) = quantize_both(w, wb, "f32", 64, 4, "affine")
    d = qm.dequantize(qw)
    y = qm.quantized_matmul(xt.to(DEV), qw)
    torch.cuda.synchronize()
    assert np.array_equal(to_oracle(qw.value), wq)
    assert np.array_equal(to_oracle(d), oracle.dequantize(wq, sc, bi, 64, 4, scale_dtype="f32"))
    yref = oracle.quantized_matmul(xb, "f32", wq, sc, bi, True, 64, 4)
    assert normwise_rel_err(y, yref) <= 1e-5 * np.sqrt(512)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("bits,g", AFFINE_CASES)
def test_decode_kernel_affine(M, bits, g):
    if bits == 2 and g == 32 and M > 8:
        pytest.skip("2-bit g32 decode kernel takes M <= 8 (other paths cover it)")
    run_qmm_case(M, 80, 1024, bits, g, "affine", "bf16", True, path="decode", wid=21 + bits)


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("K", [256, 3072, 8192])
@pytest.mark.parametrize("bits,g", AFFINE_CASES)
def test_decode_kernel_x_group_sums(M, K, bits, g):
    """Up to 4 rows the affine decode kernel sums x per group once (lane
    reductions) instead of a second MFMA: slices of 1-8 groups, 2-16 lanes per
    group, one or several rows per chunk register."""
    if K % (8 * g) or K % (16 * 32 // bits):
        pytest.skip("shape outside the decode kernel's rules")
    if bits == 2 and g == 32:
        pytest.skip("2-bit g32 keeps the MFMA sums (two row slots)")
    run_qmm_case(M, 40, K, bits, g, "affine", "bf16", True, path="decode", wid=24 + bits)


@pytest.mark.parametrize("M", [5, 6, 7, 8])
@pytest.mark.parametrize("N", [80, 1000])
@pytest.mark.parametrize("bits,g", [(4, 64), (4, 128), (8, 32), (2, 32)])
def test_decode_four_column_blocks(M, N, bits, g):
    """5-8 staged activation rows: each wave covers four column blocks
    (ragged rows, a ragged last block of columns, 2-bit g32's two row slots)."""
    run_qmm_case(M, N, 2048, bits, g, "affine", "bf16", True, path="decode", wid=27 + bits)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("N,K", [(48, 1024), (1000, 2048)])
def test_decode_nvfp4_row_slots(M, N, K):
    """nvfp4 at 1-8 rows: a K-step's two 16-element groups in two MFMA row
    slots, codes at unit scale and the E4M3 scales on the accumulator
    (ragged rows and columns, one-, two- and four-block forms)."""
    run_qmm_case(M, N, K, 4, 16, "nvfp4", "bf16", True, path="decode", wid=33)


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("mode,g,bits", MICRO_CASES)
def test_decode_kernel_micro(M, mode, g, bits):
    run_qmm_case(M, 48, 1024, bits, g, mode, "bf16", True, path="decode", wid=31)


@pytest.mark.parametrize("M", [9, 16])
def test_decode_kernel_row_passes(M):
    """x rows too large for one launch's LDS: affine runs several passes,
    microscaled codes take their x fragments straight from global memory."""
    for mode, g, bits in MICRO_CASES:
        run_qmm_case(M, 64, 8192, bits, g, mode, "bf16", True, path="decode", wid=32)
    run_qmm_case(M, 40, 8192, 4, 64, "affine", "bf16", True, path="decode", wid=33)


@pytest.mark.parametrize("M,N,K", [(17, 128, 256), (100, 200, 512), (256, 256, 192), (300, 64, 256)])
@pytest.mark.parametrize("bits,g", AFFINE_CASES)
def test_tiled_kernel_affine(M, N, K, bits, g):
    if K % g:
        pytest.skip("group does not divide K")
    run_qmm_case(M, N, K, bits, g, "affine", "bf16", True, path="tiled", wid=71 + bits)


@pytest.mark.parametrize("M", [17, 260])
@pytest.mark.parametrize("mode,g,bits", MICRO_CASES)
def test_tiled_kernel_micro(M, mode, g, bits):
    run_qmm_case(M, 136, 512, bits, g, mode, "bf16", True, path="tiled", wid=72)


@pytest.mark.parametrize("M,N,K", [(17, 128, 256), (300, 200, 512), (257, 400, 192),
                                   (520, 385, 128), (1, 64, 64)])
@pytest.mark.parametrize("bits,g", AFFINE_CASES)
def test_prefill_kernel_affine(M, N, K, bits, g):
    """Many-row MFMA kernel: several tiles in both directions, ragged M and N."""
    if K % g:
        pytest.skip("group does not divide K")
    run_qmm_case(M, N, K, bits, g, "affine", "bf16", True, path="prefill", wid=91 + bits)


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
@pytest.mark.parametrize("bits,g", [(2, 32), (4, 64), (8, 128)])
def test_prefill_kernel_tile_shapes(tile, bits, g):
    """Every tile shape of the many-row kernel, forced, on ragged M and N."""
    os.environ["QLIN_PREFILL_TILE"] = str(tile)
    try:
        run_qmm_case(300, 330, 256, bits, g, "affine", "bf16", True, path="prefill", wid=93)
    finally:
        os.environ.pop("QLIN_PREFILL_TILE", None)


@pytest.mark.parametrize("M", [17, 600])
@pytest.mark.parametrize("mode,g,bits", MICRO_CASES)
def test_prefill_kernel_micro(M, mode, g, bits):
    run_qmm_case(M, 392, 512, bits, g, mode, "bf16", True, path="prefill", wid=92)


@pytest.mark.parametrize("M,N,K", [(1, 64, 256), (17, 128, 256), (128, 128, 512), (300, 200, 512),
                                   (257, 400, 768), (520, 385, 1024), (1024, 1024, 1024)])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_prefill2_kernel_affine(M, N, K, g):
    """Software-pipelined 4-bit kernel: 1-4 code blocks of 256 k (the ring
    and block prefetch wrap), ragged M and N (N % 4 != 0 takes the scalar
    stores), grids with and without the per-XCD tile blocks."""
    run_qmm_case(M, N, K, 4, g, "affine", "bf16", True, path="prefill2", wid=95)


def test_prefill2_kernel_refuses_other_shapes():
    """K not a multiple of 256, or another bit width: the forced path fails
    with a clear error instead of running."""
    for (K, bits) in ((192, 4), (512, 8)):
        w, _ = gpu_weight((64, K), 0.02, 96, "bf16")
        qw = qm.quantize(w, 64, bits)
        os.environ["QLIN_FORCE_PATH"] = "prefill2"
        try:
            with pytest.raises(RuntimeError, match="pipelined 4-bit prefill"):
                qm.quantized_matmul(torch.ones(300, K, dtype=torch.bfloat16, device=DEV), qw)
        finally:
            os.environ.pop("QLIN_FORCE_PATH", None)


@pytest.mark.parametrize("M", [1, 3, 4, 8])
@pytest.mark.parametrize("bits,g", AFFINE_CASES)
def test_nt_kernel_affine(M, bits, g):
    """[in, out] layout (transpose=false) kernel, ragged N."""
    run_qmm_case(M, 8 * 96 if g != 128 else 640, 512, bits, g, "affine", "bf16", False,
                 path="decode", wid=81 + bits)


@pytest.mark.parametrize("M", [1, 5])
@pytest.mark.parametrize("mode,g,bits", MICRO_CASES)
def test_nt_kernel_micro(M, mode, g, bits):
    run_qmm_case(M, 768, 256, bits, g, mode, "bf16", False, path="decode", wid=82)


@pytest.mark.parametrize("M,N,K", [(1, 1024, 4160), (2, 3072, 1000), (3, 640, 2048), (5, 512, 64),
                                   (8, 1536, 8)])
@pytest.mark.parametrize("bits,g", [(4, 64), (8, 32), (2, 128)])
def test_nt_kernel_k_slices(M, N, K, bits, g):
    """[in, out] layout: K not a multiple of the waves' slices (ragged last
    slice), K shorter than one prefetch ring, a single row of K."""
    if N % g:
        pytest.skip("group does not divide N")
    run_qmm_case(M, N, K, bits, g, "affine", "bf16", False, path="decode", wid=84 + bits)


@pytest.mark.parametrize("mode,g,bits", MICRO_CASES + [("affine", 32, 2)])
def test_nt_kernel_wide_lanes_ragged(mode, g, bits):
    """[in, out] layout, one activation row of microscaled or 2-bit codes
    (each lane loads several words of one group): the last column block is
    part-filled (672 columns) and K is ragged against the waves' slices."""
    run_qmm_case(1, 672, 1000, bits, g, mode, "bf16", False, path="decode", wid=88)


@pytest.mark.parametrize("mode,g,bits", MICRO_CASES + [("affine", 32, 2)])
def test_nt_kernel_unaligned_weight_pointer(mode, g, bits):
    """Packed words that start 4 bytes past a 16-byte boundary take the
    one-word-per-lane form and give the same values."""
    N, K = 768, 512
    w, wb = gpu_weight((K, N), 0.02, 89, "bf16")
    xt, xb = synth.normal((1, K), 1.0, 89, synth.ACT, "bf16")
    qw, (wq, sc, bi) = quantize_both(w, wb, "bf16", g, bits, mode, False)
    flat = torch.empty(qw.value.numel() + 1, dtype=qw.value.dtype, device=DEV)
    shifted = flat[1:].view(qw.value.shape)
    shifted.copy_(qw.value)
    assert shifted.data_ptr() % 16 == 4
    qs = qm.QuantizedWeight(shifted, qw.scales, qw.biases, qw.group_size, qw.bits, qw.transpose, qw.mode)
    x = xt.to(DEV)
    os.environ["QLIN_FORCE_PATH"] = "decode"
    try:
        y = qm.quantized_matmul(x, qs)
        y0 = qm.quantized_matmul(x, qw)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("QLIN_FORCE_PATH", None)
    yref = oracle.quantized_matmul(xb, "bf16", wq, sc, bi, False, g, bits, mode,
                                   scale_dtype=("bf16" if mode == "affine" else "u8"))
    assert normwise_rel_err(y, yref) <= tolerance(torch.bfloat16, K)
    assert normwise_rel_err(y0, yref) <= tolerance(torch.bfloat16, K)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("bits,g", AFFINE_CASES)
def test_nt_split_affine(M, bits, g):
    """[in, out] layout with a workspace: K split over workgroups, partial
    sums added in a second kernel; ragged last superblock (768 columns)."""
    N = 8 * 96 if g != 128 else 640
    if qm.quantized_matmul_workspace_bytes(M, 512, N, False, g, bits) == 0:
        pytest.skip("no K split at this row count (2-bit codes: 1-2 rows; others 1-4)")
    run_qmm_case(M, N, 512, bits, g, "affine", "bf16", False, path="split", wid=91 + bits)


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("mode,g,bits", MICRO_CASES)
def test_nt_split_micro(M, mode, g, bits):
    run_qmm_case(M, 768, 1024, bits, g, mode, "bf16", False, path="split", wid=94)


def test_nt_split_row_limits():
    """The workspace query offers the K split at 1-4 rows (1-2 for 2-bit
    codes) and not at 5-8, where the one-pass kernel is kept."""
    q = qm.quantized_matmul_workspace_bytes
    assert all(q(M, 4096, 14336, False, 64, 4) > 0 for M in (1, 2, 3, 4))
    assert all(q(M, 4096, 14336, False, 64, 4) == 0 for M in (5, 8))
    assert q(2, 4096, 14336, False, 32, 2) > 0 and q(3, 4096, 14336, False, 32, 2) == 0


@pytest.mark.parametrize("M,N,K", [(1, 1024, 4160), (2, 3072, 1000), (3, 640, 2048), (5, 512, 64),
                                   (8, 1536, 8), (1, 14336, 4096)])
@pytest.mark.parametrize("bits,g", [(4, 64), (8, 32), (2, 128)])
def test_nt_split_k_slices(M, N, K, bits, g):
    """K-split form: ragged last slice, K shorter than one slice, a single
    row of K, and the decode workload's full shape at one row."""
    if N % g:
        pytest.skip("group does not divide N")
    if qm.quantized_matmul_workspace_bytes(M, K, N, False, g, bits) == 0:
        pytest.skip("no K split for this shape (one slice, or the row count)")
    run_qmm_case(M, N, K, bits, g, "affine", "bf16", False, path="split", wid=95 + bits)


def test_nt_split_workspace_rules():
    """A caller's workspace that is too small falls back to the one-pass
    kernel; repeated calls agree bit for bit; the result matches the
    one-pass kernel within the matmul bar."""
    K, N = 2048, 4096
    w, wb = gpu_weight((K, N), 0.02, 97, "bf16")
    xt, xb = synth.normal((2, K), 1.0, 97, synth.ACT, "bf16")
    qw, (wq, sc, bi) = quantize_both(w, wb, "bf16", 64, 4, "affine", False)
    x = xt.to(DEV)
    need = qm.quantized_matmul_workspace_bytes(2, K, N, False, 64, 4)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)   # counters start at zero
    ys = [qm.quantized_matmul(x, qw, workspace=ws) for _ in range(3)]
    small = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    y_small = qm.quantized_matmul(x, qw, workspace=small)
    os.environ["QLIN_FORCE_PATH"] = "decode"
    try:
        y_one = qm.quantized_matmul(x, qw)
    finally:
        os.environ.pop("QLIN_FORCE_PATH", None)
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    assert torch.equal(y_small, y_one)                  # fell back to the one-pass kernel
    yref = oracle.quantized_matmul(xb, "bf16", wq, sc, bi, False, 64, 4, "affine",
                                   scale_dtype="bf16")
    tol = tolerance(torch.bfloat16, K)
    assert normwise_rel_err(ys[0], yref) <= tol
    assert normwise_rel_err(y_one, yref) <= tol
    # every call leaves the completion counters at the start of the workspace zero
    assert int(ws[:4096].count_nonzero()) == 0


def test_nt_split_unzeroed_workspace_fails_visibly():
    """A K-split workspace whose completion counters were never zeroed (all
    bytes 0xFF here) makes every output of the call NaN, and of the next
    call on it too; once zeroed, the same workspace gives the oracle's
    result. The kernels run to completion either way."""
    K, N = 2048, 4096
    w, wb = gpu_weight((K, N), 0.02, 96, "bf16")
    xt, xb = synth.normal((1, K), 1.0, 96, synth.ACT, "bf16")
    qw, (wq, sc, bi) = quantize_both(w, wb, "bf16", 64, 4, "affine", False)
    x = xt.to(DEV)
    need = qm.quantized_matmul_workspace_bytes(1, K, N, False, 64, 4)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    for _ in range(2):
        y = qm.quantized_matmul(x, qw, workspace=ws)
        torch.cuda.synchronize()
        assert bool(torch.isnan(y.float()).all())
    ws.zero_()
    y = qm.quantized_matmul(x, qw, workspace=ws)
    torch.cuda.synchronize()
    yref = oracle.quantized_matmul(xb, "bf16", wq, sc, bi, False, 64, 4, "affine", scale_dtype="bf16")
    assert normwise_rel_err(y, yref) <= tolerance(torch.bfloat16, K)


def test_nt_split_shared_workspace_shapes():
    """One zeroed workspace serves K-split calls of different shapes, row
    counts and formats in turn (the completion counters come back to zero
    after each call); each result is bit-identical to the same call with a
    fresh workspace and within the bar against the oracle."""
    cases = [(1, 4096, 2048, 4, 64, 91), (3, 1536, 1024, 8, 32, 92), (2, 8192, 512, 4, 128, 93),
             (1, 768, 4160, 2, 32, 94)]
    prepared = []
    need = 0
    for M, N, K, bits, g, wid in cases:
        w, wb = gpu_weight((K, N), 0.02, wid, "bf16")
        xt, xb = synth.normal((M, K), 1.0, wid, synth.ACT, "bf16")
        qw, ref = quantize_both(w, wb, "bf16", g, bits, "affine", False)
        nb = qm.quantized_matmul_workspace_bytes(M, K, N, False, g, bits)
        assert nb > 0
        need = max(need, nb)
        prepared.append((xt.to(DEV), xb, qw, ref, nb, M, K, g, bits))
    shared = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for _ in range(2):
        for x, xb, qw, (wq, sc, bi), nb, M, K, g, bits in prepared:
            y = qm.quantized_matmul(x, qw, workspace=shared)
            fresh = torch.zeros(nb, dtype=torch.uint8, device=DEV)
            y_fresh = qm.quantized_matmul(x, qw, workspace=fresh)
            torch.cuda.synchronize()
            assert torch.equal(y, y_fresh)
            assert int(shared[:4096].count_nonzero()) == 0
            yref = oracle.quantized_matmul(xb, "bf16", wq, sc, bi, False, g, bits, "affine",
                                           scale_dtype="bf16")
            assert normwise_rel_err(y, yref) <= tolerance(torch.bfloat16, K)


@pytest.mark.parametrize("M", [9, 20, 128])
@pytest.mark.parametrize("mode,g,bits", [("affine", 64, 4), ("affine", 32, 2), ("mxfp4", 32, 4)])
def test_nt_kernel_row_blocks(M, mode, g, bits):
    """[in, out] layout with 9..128 rows: the few-row kernel over blocks of
    8 rows (ragged last block)."""
    run_qmm_case(M, 768, 512, bits, g, mode, "bf16", False, path="decode", wid=98)


def test_nt_kernel_repeat_is_deterministic():
    """Partial sums meet in a fixed order: repeated calls agree bit for bit."""
    w, _ = gpu_weight((4096, 2048), 0.02, 86, "bf16")
    qw = qm.quantize(w, 64, 4, "affine", transpose=False)
    x, _ = synth.normal((3, 4096), 1.0, 86, synth.ACT, "bf16")
    x = x.to(DEV)
    ys = [qm.quantized_matmul(x, qw) for _ in range(4)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


@pytest.mark.parametrize("transpose", [True, False])
@pytest.mark.parametrize("xdtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("bits,g", [(2, 32), (4, 64), (8, 128)])
def test_generic_kernel_affine(transpose, xdtype, bits, g):
    run_qmm_case(5, 128, 256, bits, g, "affine", xdtype, transpose, path="generic", wid=41)


@pytest.mark.parametrize("transpose", [True, False])
@pytest.mark.parametrize("mode,g,bits", MICRO_CASES)
def test_generic_kernel_micro(transpose, mode, g, bits):
    run_qmm_case(3, 128, 256, bits, g, mode, "bf16", transpose, path="generic", wid=42)


def test_rs_quantized_matmul_example_gpu():
    """mlx-rs test_quantized_matmul: transpose=false, g64 b4, max diff < 1e-3."""
    m, n, k = 32, 128, 128
    xt, xb = synth.normal((m, k), 1 / np.sqrt(k), 1001, 1, "f32")
    wt, wb = synth.normal((k, n), 1 / np.sqrt(k), 1001, 0, "f32")
    qw = qm.quantize(wt.to(DEV), 64, 4, transpose=False)
    w_hat = qm.dequantize(qw)
    y_q = qm.quantized_matmul(xt.to(DEV), qw)
    y_hat = xt.to(DEV) @ w_hat
    torch.cuda.synchronize()
    assert y_q.shape == y_hat.shape
    assert float((y_q - y_hat).abs().max()) < 1e-3


def test_page_worked_example_shape():
    """"Emily.Quantization.Layers" example: x iota {2,128} . W iota {4,128} -> {2,4}."""
    w = torch.arange(4 * 128, dtype=torch.float32).reshape(4, 128).to(DEV)
    x = torch.arange(2 * 128, dtype=torch.float32).reshape(2, 128).to(DEV)
    qw = qm.quantize(w)
    y = qm.quantized_matmul(x, qw)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (2, 4)
    wq, sc, bi = oracle.quantize(w.cpu().numpy(), "f32", 64, 4)
    yref = oracle.quantized_matmul(x.cpu().numpy(), "f32", wq, sc, bi, True, 64, 4)
    assert normwise_rel_err(y, yref) <= 1e-5 * np.sqrt(128)


def test_edge_empty_and_ragged():
    w, wb = gpu_weight((50, 256), 0.02, 51, "bf16")          # N = 50: ragged column blocks
    qw, (wq, sc, bi) = quantize_both(w, wb, "bf16", 64, 4, "affine")
    x0 = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    assert qm.quantized_matmul(x0, qw).shape == (0, 50)
    xt, xb = synth.normal((2, 3, 256), 1.0, 51, 1, "bf16")  # batch dims flattened
    y = qm.quantized_matmul(xt.to(DEV), qw)
    torch.cuda.synchronize()
    yref = oracle.quantized_matmul(xb.reshape(6, 256), "bf16", wq, sc, bi, True, 64, 4)
    assert y.shape == (2, 3, 50)
    assert normwise_rel_err(y.reshape(6, 50), yref) <= 2e-2
    # K that the decode kernel's 128-wide units do not tile (falls back)
    run_qmm_case(2, 40, 192, 4, 64, "affine", "bf16", True, wid=52)


# ---------------------------------------------------------------- gather

def run_gather_case(B, M, K, N, E, rhs, lhs, bits=4, g=64, mode="affine", xdtype="bf16",
                    transpose=True, sorted_indices=False, path=None, wid=60):
    wdt = xdtype if mode == "affine" else "bf16"
    wshape = (E, N, K) if transpose else (E, K, N)
    w, wb = gpu_weight(wshape, 0.02, wid, wdt)
    xt, xb = synth.normal((B, M, K), 1.0, wid, synth.ACT, xdtype)
    qw, (wq, sc, bi) = quantize_both(w, wb, wdt, g, bits, mode, transpose)
    rhs_t = torch.tensor(np.asarray(rhs), dtype=torch.int32)
    lhs_t = None if lhs is None else torch.tensor(np.asarray(lhs), dtype=torch.int32)
    if path:
        os.environ["QLIN_FORCE_PATH"] = path
    y = qm.gather_qmm(xt.to(DEV), qw, rhs_t.to(DEV), None if lhs_t is None else lhs_t.to(DEV),
                      sorted_indices=sorted_indices)
    torch.cuda.synchronize()
    os.environ.pop("QLIN_FORCE_PATH", None)
    rhs_f = np.asarray(rhs, np.uint32).ravel()
    lhs_f = None if lhs is None else np.broadcast_to(np.asarray(lhs, np.uint32), np.asarray(rhs).shape).ravel()
    yref = oracle.gather_qmm(xb, xdtype, wq, sc, bi, rhs_f, lhs_f, transpose, g, bits, mode,
                             scale_dtype=(wdt if mode == "affine" else "u8"))
    err = normwise_rel_err(y.reshape(yref.shape), yref)
    print(f"gather B{B} M{M} K{K} N{N} E{E} R{rhs_f.size} {mode} b{bits} t{int(transpose)} "
          f"sorted={sorted_indices} path={path}: err {err:.3e}", flush=True)
    assert err <= tolerance(TDT[xdtype], K)


def test_gather_rs_cases():
    """mlx-rs test_gather_qmm index cases (fp32, allclose 1e-4 there)."""
    run_gather_case(1, 32, 64, 64, 3, [2, 1], [0], xdtype="f32", wid=61)
    run_gather_case(5, 32, 64, 64, 3, [2, 1], [0, 2], xdtype="f32", wid=62)


@pytest.mark.parametrize("sorted_indices", [False, True])
def test_gather_moe_small(sorted_indices):
    T, E, k = 24, 8, 3
    rhs = synth.topk_distinct(T, E, k, 63)
    if sorted_indices:
        order = np.argsort(rhs.ravel(), kind="stable")
        rhs_s = rhs.ravel()[order]
        lhs = (order // k).astype(np.uint32)
        run_gather_case(T, 1, 256, 128, E, rhs_s, lhs, sorted_indices=True, wid=63)
    else:
        lhs = np.repeat(np.arange(T, dtype=np.uint32), k).reshape(T, k)
        run_gather_case(T, 1, 256, 128, E, rhs, lhs, wid=63)


def test_gather_identity_lhs_and_micro():
    run_gather_case(6, 2, 256, 64, 4, [3, 0, 1, 3, 2, 0], None, wid=64)
    run_gather_case(6, 2, 256, 64, 4, [3, 0, 1, 3, 2, 0], None, bits=4, g=32, mode="mxfp4", wid=65)
    run_gather_case(6, 2, 256, 64, 4, [1, 1, 0, 3, 2, 0], None, transpose=False, wid=66)


@pytest.mark.parametrize("path", ["tiled", "prefill"])
@pytest.mark.parametrize("mode,g,bits", [("affine", 64, 4), ("affine", 32, 2), ("affine", 128, 8)] + MICRO_CASES)
def test_gather_mfma_modes(mode, g, bits, path):
    """Both MFMA gather kernels; M = 3 rows per index row, ragged N = 200."""
    T, E, k = 40, 6, 2
    rhs = synth.topk_distinct(T, E, k, 68)
    lhs = np.repeat(np.arange(T, dtype=np.uint32), k).reshape(T, k)
    run_gather_case(T, 3, 256, 200, E, rhs, lhs, bits=bits, g=g, mode=mode, path=path, wid=68)


@pytest.mark.parametrize("mode,g,bits", [("affine", 64, 4), ("affine", 32, 2), ("affine", 128, 8)] + MICRO_CASES)
def test_gather_prefill_tall_tiles(mode, g, bits):
    """48 or more rows per expert on average: the many-row kernel takes
    128-row tiles of one expert (about 150 rows per expert here: one full
    tile and a ragged one each), ragged N = 200."""
    T, E, k = 100, 4, 2
    rhs = synth.topk_distinct(T, E, k, 70)
    lhs = np.repeat(np.arange(T, dtype=np.uint32), k).reshape(T, k)
    run_gather_case(T, 3, 256, 200, E, rhs, lhs, bits=bits, g=g, mode=mode, path="prefill", wid=70)


def test_gather_prefill_tall_tiles_skewed():
    """128-row tiles with a hot expert (400 rows: four tiles), a small one
    and empty ones, unsorted and sorted."""
    rhs = np.array([5] * 400 + [0] * 30 + [2] * 130, np.uint32)
    np.random.default_rng(4).shuffle(rhs)
    run_gather_case(rhs.size, 1, 256, 96, 9, rhs, None, path="prefill", wid=71)
    order = np.argsort(rhs, kind="stable")
    run_gather_case(rhs.size, 1, 256, 96, 9, rhs[order], order.astype(np.uint32),
                    sorted_indices=True, path="prefill", wid=71)


@pytest.mark.parametrize("path", ["tiled", "prefill"])
def test_gather_skewed_experts(path):
    """One hot expert with 150 rows (several row tiles), several empty ones."""
    rhs = np.array([5] * 150 + [0] * 3 + [2] * 70, np.uint32)
    np.random.default_rng(3).shuffle(rhs)
    run_gather_case(rhs.size, 1, 128, 96, 9, rhs, None, path=path, wid=69)
    order = np.argsort(rhs, kind="stable")
    run_gather_case(rhs.size, 1, 128, 96, 9, rhs[order], order.astype(np.uint32),
                    sorted_indices=True, path=path, wid=69)


@pytest.mark.parametrize("mode,g,bits", [("affine", 64, 4), ("affine", 32, 2), ("affine", 128, 8),
                                         ("affine", 32, 4)] + MICRO_CASES)
def test_gather_decode_kernel(mode, g, bits):
    """Small-M kernel's gather form (forced): one tile per index row (far
    fewer rows than experts, no bucketing), row tiles of 4 (few rows per
    expert) and of 16 (8 for 2-bit g32), experts split over several tiles,
    empty experts, 2 activation rows per index row, lhs given or identity,
    indices unsorted and pre-sorted."""
    K, N = 1024, 200
    # decode sizes: 3 tokens x top-4 of 16 experts (tile height 4)
    T, E, k = 3, 16, 4
    rhs = synth.topk_distinct(T, E, k, 71)
    lhs = np.repeat(np.arange(T, dtype=np.uint32), k).reshape(T, k)
    run_gather_case(T, 1, K, N, E, rhs, lhs, bits=bits, g=g, mode=mode, path="decode", wid=71)
    order = np.argsort(rhs.ravel(), kind="stable")
    run_gather_case(T, 1, K, N, E, rhs.ravel()[order], (order // k).astype(np.uint32), bits=bits,
                    g=g, mode=mode, sorted_indices=True, path="decode", wid=71)
    # 2 rows per index row: expert 3 gets 3 index rows = 6 GEMM rows (2 tiles of 4)
    run_gather_case(6, 2, K, N, 8, [3, 0, 3, 5, 3, 1], None, bits=bits, g=g, mode=mode,
                    path="decode", wid=72)
    # far fewer rows than experts: no bucketing, one tile per index row
    # (expert 3 twice, 1 and 2 rows per index row, lhs given or identity)
    run_gather_case(4, 1, K, N, 16, [3, 9, 3, 14, 0, 7], [0, 1, 2, 3, 1, 0], bits=bits, g=g,
                    mode=mode, path="decode", wid=74)
    run_gather_case(3, 2, K, N, 16, [5, 5, 12], None, bits=bits, g=g, mode=mode, path="decode",
                    wid=75)
    # tile height 16: 20 rows over 4 experts, one of them with 17 (2 tiles)
    rhs2 = np.array([2] * 17 + [0, 3, 0], np.uint32)
    np.random.default_rng(4).shuffle(rhs2)
    run_gather_case(5, 1, K, N, 4, rhs2, np.arange(20, dtype=np.uint32) % 5, bits=bits, g=g,
                    mode=mode, path="decode", wid=73)


@pytest.mark.parametrize("mode,g,bits", [("affine", 64, 4), ("affine", 128, 8), ("mxfp4", 32, 4)])
def test_gather_decode_two_blocks(mode, g, bits):
    """Gather grids large enough for two column blocks per wave (forced
    decode path): 12 tokens x top-4 of 16 experts in 16-row tiles, and 8
    index rows in the one-tile-per-row form; N = 4000 leaves the last block
    pair ragged."""
    K, N, E = 1024, 4000, 16
    rhs = synth.topk_distinct(12, E, 4, 76)
    lhs = np.repeat(np.arange(12, dtype=np.uint32), 4).reshape(12, 4)
    run_gather_case(12, 1, K, N, E, rhs, lhs, bits=bits, g=g, mode=mode, path="decode", wid=76)
    run_gather_case(8, 1, K, N, E, [3, 9, 3, 14, 0, 7, 11, 2], None, bits=bits, g=g, mode=mode,
                    path="decode", wid=77)


def test_gather_sorted_flag_is_only_a_hint():
    """Flag set on indices that are not sorted: results must not change."""
    run_gather_case(6, 1, 256, 64, 4, [3, 0, 1, 3, 2, 0], None, sorted_indices=True, wid=67)


# ---------------------------------------------------------------- quantized_dense
# "Emily.Quantization.Layers" quantized_dense: x @ W plus a bias (a tensor of
# one value per output column, or a number), fused into each kernel's output
# stage. Oracle: the fp64 matmul plus the bias, compared at the matmul bar.

DENSE_CASES = [
    # M, N, K, bits, g, mode, x dtype, transpose, forced path
    (1, 512, 1024, 4, 64, "affine", "bf16", True, "decode"),      # decode kernel
    (3, 500, 1024, 4, 64, "affine", "bf16", True, "decode"),      # x group sums, ragged N
    (9, 256, 4096, 8, 128, "affine", "bf16", True, "decode"),     # rows in two passes
    (16, 512, 8192, 4, 32, "mxfp4", "bf16", True, "decode"),      # direct x fragments
    (4, 1024, 512, 4, 64, "affine", "bf16", False, "decode"),     # [in, out] kernel
    (300, 400, 512, 4, 64, "affine", "bf16", True, "prefill"),    # many-row kernel, ragged
    (130, 256, 512, 8, 32, "mxfp8", "bf16", True, "prefill"),
    (300, 402, 512, 4, 32, "affine", "bf16", True, "prefill2"),   # pipelined 4-bit kernel
    (300, 200, 512, 4, 64, "affine", "bf16", True, "tiled"),      # LDS-tiled kernel
    (5, 128, 256, 4, 64, "affine", "f32", True, "generic"),       # fp32 VALU kernels
    (5, 128, 256, 4, 64, "affine", "f16", False, "generic"),
]


@pytest.mark.parametrize("bias_kind", ["bf16", "f32", "f16", "number"])
@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: f"M{c[0]}N{c[1]}K{c[2]}{c[5]}b{c[3]}t{int(c[7])}{c[8]}")
def test_quantized_dense(case, bias_kind):
    M, N, K, bits, g, mode, xdtype, transpose, path = case
    wdt = xdtype if mode == "affine" else "bf16"
    w, wb = gpu_weight((N, K) if transpose else (K, N), 0.02, 41, wdt)
    xt, xb = synth.normal((M, K), 1.0, 41, synth.ACT, xdtype)
    qw, (wq, sc, bi) = quantize_both(w, wb, wdt, g, bits, mode, transpose)
    if bias_kind == "number":
        bias, bias_bits, bval = -0.75, None, -0.75
    else:
        bt, bias_bits = synth.normal((N,), 1.0, 41, synth.BIAS, bias_kind)
        bias, bval = bt.to(DEV), 0.0
    os.environ["QLIN_FORCE_PATH"] = path
    y = qm.quantized_dense(xt.to(DEV), qw, bias)
    torch.cuda.synchronize()
    os.environ.pop("QLIN_FORCE_PATH", None)
    yref = oracle.quantized_dense(xb, xdtype, wq, sc, bi, bias_bits,
                                  bias_kind if bias_kind != "number" else "f32", bval,
                                  transpose, g, bits, mode,
                                  scale_dtype=(wdt if mode == "affine" else "u8"))
    assert y.shape == (M, N) and y.dtype == TDT[xdtype]
    err = normwise_rel_err(y, yref)
    tol = tolerance(TDT[xdtype], K)
    print(f"dense {case} bias={bias_kind}: err {err:.3e} tol {tol:.1e}", flush=True)
    assert err <= tol
    # the bias is really applied: without it the error is far above the bar
    y0 = oracle.quantized_matmul(xb, xdtype, wq, sc, bi, transpose, g, bits, mode,
                                 scale_dtype=(wdt if mode == "affine" else "u8"))
    assert normwise_rel_err(y, y0) > 2 * tol


def test_quantized_dense_zero_bias_is_quantized_matmul():
    """A number bias of 0 is the plain matmul: same kernel, same bits."""
    w, wb = gpu_weight((512, 1024), 0.02, 42, "bf16")
    xt, _ = synth.normal((2, 1024), 1.0, 42, synth.ACT, "bf16")
    qw = qm.quantize(w, 64, 4, "affine")
    x = xt.to(DEV)
    assert torch.equal(qm.quantized_dense(x, qw, 0).view(torch.int16),
                       qm.quantized_matmul(x, qw).view(torch.int16))


# ---------------------------------------------------------------- qqmm
# mlx-rs qqmm: x quantized on the fly (nvfp4 / mxfp8), W already quantized.
# The decoded x is exact in bf16 and the products of decoded values are exact
# in fp32, so the GPU result is the oracle's up to fp32 accumulation order and
# the bf16 rounding of y: normwise 4e-3 (2^-9 rounding plus accumulation),
# tighter than the 2e-2 bar for bf16 outputs.

QQMM_CASES = [
    # M, N, K, mode, transpose, forced path
    (1, 512, 1024, "mxfp8", True, "decode"),
    (1, 500, 1024, "nvfp4", True, "decode"),
    (16, 256, 8192, "nvfp4", True, "decode"),     # direct x fragments
    (5, 1024, 512, "mxfp8", False, "decode"),     # [in, out] kernel
    (300, 384, 512, "mxfp8", True, "prefill"),
    (260, 256, 512, "nvfp4", True, "prefill"),
    (7, 128, 256, "nvfp4", True, "generic"),
]

# mxfp8 on the scaled fp8 MFMA (the workspace holds x's codes and scales)
QQMM_SCALED_CASES = [
    # M, N, K
    (32, 128, 512),          # one tile, one batch of 4 K steps
    (300, 384, 512),         # ragged rows, several tiles
    (130, 200, 1024),        # ragged weight rows (N % 4 != 0 columns stored one by one)
    (512, 1024, 2048),
    (64, 256, 8192),         # long K
]


@pytest.mark.parametrize("case", QQMM_CASES, ids=lambda c: f"M{c[0]}N{c[1]}K{c[2]}{c[3]}t{int(c[4])}{c[5]}")
def test_qqmm(case):
    M, N, K, mode, transpose, path = case
    g, bits = oracle.MODE_PAIRING[mode]
    w, wb = gpu_weight((N, K) if transpose else (K, N), 0.02, 51, "bf16")
    xt, xb = synth.normal((M, K), 1.0, 51, synth.ACT, "bf16")
    qw, (wq, sc, _) = quantize_both(w, wb, "bf16", g, bits, mode, transpose)
    ws = torch.empty(qm.qqmm_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    os.environ["QLIN_FORCE_PATH"] = path
    y = qm.qqmm(xt.to(DEV), qw, workspace=ws)
    torch.cuda.synchronize()
    os.environ.pop("QLIN_FORCE_PATH", None)
    yref, xhat = oracle.qqmm(xb, "bf16", wq, sc, transpose, g, bits, mode, return_xhat=True)
    # the decoded activation in the workspace, bit for bit
    xh_bits = torch.from_numpy(xhat).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(torch.from_numpy(xhat).to(torch.bfloat16).float().numpy(), xhat)
    assert np.array_equal(to_oracle(ws.view(torch.bfloat16).view(M, K)), xh_bits)
    assert y.shape == (M, N) and y.dtype == torch.bfloat16
    err = normwise_rel_err(y, yref)
    print(f"qqmm {case}: err {err:.3e}", flush=True)
    assert err <= 4e-3



@pytest.mark.parametrize("case", QQMM_SCALED_CASES, ids=lambda c: f"M{c[0]}N{c[1]}K{c[2]}")
def test_qqmm_scaled_mfma(case):
    """mlx-rs qqmm in mxfp8 on v_mfma_scale_f32_32x32x64_f8f6f4: x's codes
    and scale bytes in the workspace bit-exact against the oracle's
    quantization of x, y within the qqmm bar of the oracle's product."""
    M, N, K = case
    g, bits = 32, 8
    w, wb = gpu_weight((N, K), 0.02, 52, "bf16")
    xt, xb = synth.normal((M, K), 1.0, 52, synth.ACT, "bf16")
    qw, (wq, sc, _) = quantize_both(w, wb, "bf16", g, bits, "mxfp8", True)
    ws = torch.empty(qm.qqmm_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    os.environ["QLIN_FORCE_PATH"] = "scaled"
    y = qm.qqmm(xt.to(DEV), qw, workspace=ws)
    torch.cuda.synchronize()
    os.environ.pop("QLIN_FORCE_PATH", None)
    assert qm.last_path() == "qqmm_scaled_mfma"
    xq, xs, _ = oracle.quantize(xb, "bf16", g, bits, "mxfp8")
    got = ws.cpu().numpy()
    assert np.array_equal(got[:M * K], xq.view(np.uint8).reshape(-1))
    assert np.array_equal(got[M * K:M * K + M * K // 32], xs.reshape(-1))
    yref = oracle.qqmm(xb, "bf16", wq, sc, True, g, bits, "mxfp8")
    err = normwise_rel_err(y, yref)
    print(f"qqmm scaled M{M} N{N} K{K}: err {err:.3e}", flush=True)
    assert err <= 4e-3


# ---------------------------------------------------------------- debug mode

@pytest.fixture
def lds_nan_fill():
    os.environ["QLIN_DEBUG_LDS_NAN"] = "1"
    yield
    os.environ.pop("QLIN_DEBUG_LDS_NAN", None)


@pytest.mark.parametrize("case", [
    (300, 200, 512, 4, 64, "affine", "prefill", None),    # pipelined form
    (520, 385, 768, 8, 128, "affine", "prefill", "0"),    # 256 x 192 tile, two-step form
    (300, 330, 512, 2, 32, "affine", "prefill", "0"),     # 2-bit, two-step form
    (300, 330, 256, 2, 32, "affine", "prefill", None),    # 2-bit, 16-byte batches, pipelined
    (130, 392, 512, 4, 32, "mxfp4", "prefill", None),
    (600, 392, 512, 4, 16, "nvfp4", "prefill", None),
    (300, 200, 512, 4, 64, "affine", "prefill2", None),   # register-dequantizing kernel
], ids=lambda c: f"M{c[0]}N{c[1]}K{c[2]}{c[5]}b{c[3]}g{c[4]}-{c[6]}-t{c[7]}")
def test_lds_nan_fill_qmm(case, lds_nan_fill):
    """QLIN_DEBUG_LDS_NAN=1 fills each tile's LDS with NaN before the tile
    starts; the outputs stay within the bar (a NaN fails it), so every LDS
    byte an MFMA fragment reads was written by the tile first (ragged M, N)."""
    M, N, K, bits, g, mode, path, tile = case
    if tile is not None:
        os.environ["QLIN_PREFILL_TILE"] = tile
    try:
        run_qmm_case(M, N, K, bits, g, mode, "bf16", True, path=path, wid=97)
    finally:
        os.environ.pop("QLIN_PREFILL_TILE", None)


def test_lds_nan_fill_gather(lds_nan_fill):
    """The gather form under the NaN fill: 128-row tiles (about 150 rows per
    expert) and 64-row tiles (a few rows per expert)."""
    T, E, k = 100, 4, 2
    rhs = synth.topk_distinct(T, E, k, 98)
    lhs = np.repeat(np.arange(T, dtype=np.uint32), k).reshape(T, k)
    run_gather_case(T, 3, 256, 200, E, rhs, lhs, path="prefill", wid=98)
    T, E, k = 40, 6, 2
    rhs = synth.topk_distinct(T, E, k, 99)
    lhs = np.repeat(np.arange(T, dtype=np.uint32), k).reshape(T, k)
    run_gather_case(T, 3, 256, 200, E, rhs, lhs, bits=4, g=32, mode="mxfp4", path="prefill", wid=99)


def test_lds_nan_fill_qqmm_scaled(lds_nan_fill):
    """The scaled fp8 MFMA kernel under the NaN fill (ragged M and N)."""
    test_qqmm_scaled_mfma((130, 200, 1024))
