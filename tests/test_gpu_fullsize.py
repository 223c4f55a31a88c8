"""GPU parity at the full workload sizes, on sampled outputs.

Same shapes, dtypes, seeds and kernel dispatch as the benchmark. The oracle
cannot redo a 14336 x 4096 (or 206 GFLOP) problem in a test, so it computes
sampled outputs one by one: quantization is local to a row (or, for the
[in, out] layout, to a block of group_size columns), so the oracle quantizes
only the sampled weight rows or column blocks, the GPU's codes, scales and
biases for exactly those rows are checked bit-exact against them, and the
sampled outputs are checked against the oracle's fp64 matmul of those rows
(normwise error over the sample <= 2e-2, the bf16-output bound).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import to_oracle

pytestmark = pytest.mark.gpu

qm = pytest.importorskip("quantized_matmul_amd")

DEV = "cuda:0"
TOL_BF16 = 2e-2


def pick(n, k, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=min(k, n), replace=False))


def ix(a: np.ndarray) -> torch.Tensor:
    """Index array for device tensors."""
    return torch.from_numpy(np.asarray(a, dtype=np.int64)).to(DEV)


def sample_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    den = np.abs(y_ref).max()
    return float(np.abs(y_gpu - y_ref).max() / den)


def gpu_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def check_codes(qw_value, qw_scales, qw_biases, ref, mode):
    wq, sc, bi = ref
    assert np.array_equal(to_oracle(qw_value), wq)
    assert np.array_equal(to_oracle(qw_scales), sc)
    if mode == "affine":
        assert np.array_equal(to_oracle(qw_biases), bi)


# ------------------------------------------------------------ decode [out, in]

@pytest.fixture(scope="module")
def decode_weight():
    w, wb = synth.normal((14336, 4096), 0.02, 101, synth.WEIGHT, "bf16")
    return w.to(DEV), wb


@pytest.mark.parametrize("bits,g", [(4, 64), (8, 64), (2, 32)])
@pytest.mark.parametrize("M", [1, 4, 8])
def test_decode_full_size(decode_weight, bits, g, M):
    """x bf16 [M, 4096] . W[14336, 4096]^T, affine, bf16 scales/biases."""
    w, wb = decode_weight
    qw = qm.quantize(w, g, bits, "affine")
    x, xb = synth.normal((M, 4096), 1.0, 101, synth.ACT, "bf16")
    y = qm.quantized_matmul(x.to(DEV), qw)
    torch.cuda.synchronize()
    cols = pick(14336, 64, 7 + bits + M)
    ref = oracle.quantize(wb[cols], "bf16", g, bits)
    check_codes(qw.value[ix(cols)], qw.scales[ix(cols)], qw.biases[ix(cols)], ref, "affine")
    y_ref = oracle.quantized_matmul(xb, "bf16", *ref, True, g, bits)
    err = sample_err(gpu_np(y[:, ix(cols)]), y_ref)
    print(f"decode full M{M} b{bits} g{g}: sampled err {err:.3e}", flush=True)
    assert err <= TOL_BF16


# ------------------------------------------------------------ decode [in, out]

@pytest.fixture(scope="module")
def decode_weight_t():
    w, wb = synth.normal((4096, 14336), 0.02, 111, synth.WEIGHT, "bf16")
    return w.to(DEV), wb


@pytest.mark.parametrize("bits,g", [(4, 64), (8, 64), (2, 32)])
@pytest.mark.parametrize("M", [1, 4, 8])
def test_decode_full_size_in_out_layout(decode_weight_t, bits, g, M):
    """transpose=false: W [4096, 14336] packed along its 14336 outputs."""
    w, wb = decode_weight_t
    qw = qm.quantize(w, g, bits, "affine", transpose=False)
    x, xb = synth.normal((M, 4096), 1.0, 111, synth.ACT, "bf16")
    y = qm.quantized_matmul(x.to(DEV), qw)
    torch.cuda.synchronize()
    per = 32 // bits
    blocks = np.unique(pick(14336, 24, 11 + bits + M) // g)
    for b in blocks:
        c0 = int(b) * g
        ref = oracle.quantize(np.ascontiguousarray(wb[:, c0:c0 + g]), "bf16", g, bits)
        gs = slice(c0 // g, c0 // g + 1)
        check_codes(qw.value[:, c0 // per:(c0 + g) // per], qw.scales[:, gs], qw.biases[:, gs],
                    ref, "affine")
        y_ref = oracle.quantized_matmul(xb, "bf16", *ref, False, g, bits)
        err = sample_err(gpu_np(y[:, c0:c0 + g]), y_ref)
        assert err <= TOL_BF16, (int(b), err)


# ------------------------------------------------------------ prefill

@pytest.fixture(scope="module")
def prefill_inputs():
    w, wb = synth.normal((12288, 4096), 0.02, 201, synth.WEIGHT, "bf16")
    x, xb = synth.normal((2048, 4096), 1.0, 201, synth.ACT, "bf16")
    return w.to(DEV), wb, x.to(DEV), xb


@pytest.mark.parametrize("g", [64, 128])
def test_prefill_full_size(prefill_inputs, g):
    """x bf16 [2048, 4096] . W[12288, 4096]^T, int4, the benchmark's kernel."""
    w, wb, x, xb = prefill_inputs
    qw = qm.quantize(w, g, 4, "affine")
    y = qm.quantized_matmul(x, qw)
    torch.cuda.synchronize()
    rows, cols = pick(2048, 48, 21 + g), pick(12288, 64, 22 + g)
    ref = oracle.quantize(wb[cols], "bf16", g, 4)
    check_codes(qw.value[ix(cols)], qw.scales[ix(cols)], qw.biases[ix(cols)], ref, "affine")
    y_ref = oracle.quantized_matmul(np.ascontiguousarray(xb[rows]), "bf16", *ref, True, g, 4)
    err = sample_err(gpu_np(y[ix(rows)][:, ix(cols)]), y_ref)
    print(f"prefill full g{g}: sampled err {err:.3e}", flush=True)
    assert err <= TOL_BF16


# ------------------------------------------------------------ microscaled

@pytest.fixture(scope="module")
def micro_weight():
    w, wb = synth.normal((8192, 8192), 0.02, 120, synth.WEIGHT, "bf16")
    return w.to(DEV), wb


@pytest.mark.parametrize("mode,g,bits", [("mxfp4", 32, 4), ("nvfp4", 16, 4), ("mxfp8", 32, 8)])
@pytest.mark.parametrize("M", [1, 16, 512])
def test_micro_full_size(micro_weight, mode, g, bits, M):
    """x bf16 [M, 8192] . W[8192, 8192]^T, microscaled (no biases)."""
    w, wb = micro_weight
    qw = qm.quantize(w, g, bits, mode)
    x, xb = synth.normal((M, 8192), 1.0, 120, synth.ACT, "bf16")
    y = qm.quantized_matmul(x.to(DEV), qw)
    torch.cuda.synchronize()
    rows = pick(M, 32, 31 + M)
    cols = pick(8192, 64, 32 + M + bits)
    ref = oracle.quantize(wb[cols], "bf16", g, bits, mode)
    check_codes(qw.value[ix(cols)], qw.scales[ix(cols)], None, ref, mode)
    y_ref = oracle.quantized_matmul(np.ascontiguousarray(xb[rows]), "bf16", *ref, True, g, bits,
                                    mode)
    err = sample_err(gpu_np(y[ix(rows)][:, ix(cols)]), y_ref)
    print(f"micro full {mode} M{M}: sampled err {err:.3e}", flush=True)
    assert err <= TOL_BF16


# ------------------------------------------------------------ MoE gather

@pytest.fixture(scope="module")
def moe_inputs():
    E, N, K, T, k = 64, 1536, 2048, 512, 8
    w, wb = synth.normal((E, N, K), 0.02, 301, synth.WEIGHT, "bf16")
    x, xb = synth.normal((T, 1, K), 1.0, 301, synth.ACT, "bf16")
    rhs = synth.topk_distinct(T, E, k, 301)
    qw = qm.quantize(w.to(DEV), 64, 4, "affine")
    return qw, wb, x.to(DEV), xb, rhs


@pytest.mark.parametrize("sorted_indices", [False, True])
def test_moe_gather_full_size(moe_inputs, sorted_indices):
    """64 experts [1536, 2048] int4 g64, 512 tokens x top-8 distinct experts."""
    qw, wb, x, xb, rhs = moe_inputs
    T, k = rhs.shape
    lhs = np.repeat(np.arange(T, dtype=np.uint32), k).reshape(T, k)
    rhs_f, lhs_f = rhs.reshape(-1), lhs.reshape(-1)
    if sorted_indices:
        order = np.argsort(rhs_f, kind="stable")
        rhs_f, lhs_f = rhs_f[order], lhs_f[order]
    y = qm.gather_qmm(x, qw, torch.from_numpy(rhs_f.astype(np.int32)).to(DEV),
                      torch.from_numpy(lhs_f.astype(np.int32)).to(DEV),
                      sorted_indices=sorted_indices)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T * k, 1, 1536)
    rows, cols = pick(T * k, 48, 41 + int(sorted_indices)), pick(1536, 48, 42)
    yg = gpu_np(y[:, 0, :])
    errs = []
    for r in rows:
        e, t = int(rhs_f[r]), int(lhs_f[r])
        ref = oracle.quantize(np.ascontiguousarray(wb[e][cols]), "bf16", 64, 4)
        check_codes(qw.value[e][ix(cols)], qw.scales[e][ix(cols)], qw.biases[e][ix(cols)], ref,
                    "affine")
        y_ref = oracle.quantized_matmul(np.ascontiguousarray(xb[t]), "bf16", *ref, True, 64, 4)
        errs.append((yg[r, cols], y_ref[0]))
    got = np.stack([a for a, _ in errs])
    want = np.stack([b for _, b in errs])
    err = sample_err(got, want)
    print(f"moe full sorted={sorted_indices}: sampled err {err:.3e}", flush=True)
    assert err <= TOL_BF16


@pytest.mark.parametrize("T", [1, 8])
def test_moe_decode_sizes_full_size(moe_inputs, T):
    """Decode-sized expert batches on the full 64 x [1536, 2048] int4 stack, in
    the launch configuration the benchmark times (automatic path: one tile
    per index row at 1 token, 4-row expert tiles at 8 tokens)."""
    qw, wb, _, _, _ = moe_inputs
    E, K, k = 64, 2048, 8
    x, xb = synth.normal((T, 1, K), 1.0, 305, synth.ACT, "bf16")
    rhs = synth.topk_distinct(T, E, k, 305)
    lhs = np.repeat(np.arange(T, dtype=np.uint32), k).reshape(T, k)
    rhs_f, lhs_f = rhs.reshape(-1), lhs.reshape(-1)
    y = qm.gather_qmm(x.to(DEV), qw, torch.from_numpy(rhs_f.astype(np.int32)).to(DEV),
                      torch.from_numpy(lhs_f.astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T * k, 1, 1536)
    cols = pick(1536, 48, 43 + T)
    yg = gpu_np(y[:, 0, :])
    got, want = [], []
    for r in range(T * k):
        e, t = int(rhs_f[r]), int(lhs_f[r])
        ref = oracle.quantize(np.ascontiguousarray(wb[e][cols]), "bf16", 64, 4)
        y_ref = oracle.quantized_matmul(np.ascontiguousarray(xb[t]), "bf16", *ref, True, 64, 4)
        got.append(yg[r, cols])
        want.append(y_ref[0])
    err = sample_err(np.stack(got), np.stack(want))
    print(f"moe decode T{T}: sampled err {err:.3e}", flush=True)
    assert err <= TOL_BF16
