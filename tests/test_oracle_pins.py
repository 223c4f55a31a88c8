"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, a library routine, a
brute-force search, or a fact the pages print -- never against a retyping of
the oracle's own formula. Runs on the CPU only.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- formats

def test_e2m1_table_matches_spec_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_table.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        c, v = int(code, 16), float(val)
        d = oracle.decode("e2m1", c)
        assert d == v and np.signbit(d) == np.signbit(v), (code, d, v)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        d = oracle.decode("e4m3", c)
        if np.isnan(ref[c]):
            assert np.isnan(d), c
        else:
            assert d == ref[c] and np.signbit(d) == np.signbit(ref[c]), (c, d, ref[c])
    assert oracle.decode("e4m3", 0x7E) == 448.0
    assert oracle.decode("e4m3", 0x01) == 2.0 ** -9


def test_e8m0_decode_closed_form():
    for c in range(255):
        assert oracle.decode("e8m0", c) == 2.0 ** (c - 127)
    assert np.isnan(oracle.decode("e8m0", 255))


def test_encode_inverts_decode_every_code():
    for c in range(16):
        assert oracle.encode("e2m1", oracle.decode("e2m1", c)) == c
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue  # NaN codes
        assert oracle.encode("e4m3", oracle.decode("e4m3", c)) == c


def test_e4m3_encode_matches_torch_in_range():
    r = np.random.default_rng(0)
    vals = np.concatenate([r.standard_normal(4000) * 50, r.standard_normal(2000) * 1e-2,
                           r.uniform(-448, 448, 2000)]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, c in zip(vals, ref):
        assert oracle.encode("e4m3", float(v)) == c, v
    # saturation (torch gives NaN out of range; the reading saturates)
    assert oracle.encode("e4m3", 1000.0) == 0x7E
    assert oracle.encode("e4m3", -1e6) == 0xFE


def _e2m1_nearest_even_bruteforce(v):
    """Nearest E2M1 magnitude by exhaustive search; ties to the even code."""
    mags = [oracle.decode("e2m1", c) for c in range(8)]
    a = min(abs(v), 6.0)
    best = min(range(8), key=lambda c: (abs(mags[c] - a), c & 1))
    return best | (8 if np.signbit(v) else 0)


def test_e2m1_encode_matches_bruteforce():
    r = np.random.default_rng(1)
    vals = list(r.uniform(-8, 8, 3000)) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 7.0,
                                          -0.1, -0.0, 0.0, 6.5, 100.0]
    for v in vals:
        assert oracle.encode("e2m1", v) == _e2m1_nearest_even_bruteforce(v), v
    assert oracle.encode("e2m1", 2.5) == 0x4     # tie 2|3 -> 2 (even mantissa)
    assert oracle.encode("e2m1", 5.0) == 0x6     # tie 4|6 -> 4
    assert oracle.encode("e2m1", -0.1) == 0x8    # sign kept on zero


def test_rne_bf16_f16_match_libraries():
    r = np.random.default_rng(2)
    vals = np.concatenate([r.standard_normal(3000), r.standard_normal(1000) * 1e-5,
                           r.standard_normal(1000) * 1e4]).astype(np.float32)
    tb = torch.from_numpy(vals).to(torch.bfloat16).float().numpy()
    th = vals.astype(np.float16).astype(np.float32)
    for v, b, h in zip(vals, tb, th):
        assert oracle.round_to(float(v), "bf16") == b
        assert oracle.round_to(float(v), "f16") == h


@pytest.mark.parametrize("fmt,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_directed_rounding_brackets(fmt, tdt):
    """RD/RU give the largest representable <= v and smallest >= v."""
    r = np.random.default_rng(3)
    vals = np.concatenate([r.standard_normal(2000) * 0.02, r.standard_normal(500)]).astype(np.float32)
    for v in vals:
        d = oracle.round_to(float(v), fmt, "down")
        u = oracle.round_to(float(v), fmt, "up")
        td = torch.tensor([d], dtype=torch.float64).to(tdt)
        tu = torch.tensor([u], dtype=torch.float64).to(tdt)
        assert float(td) == d and float(tu) == u          # representable
        assert d <= v <= u
        if d != v:
            nxt = torch.nextafter(td, torch.tensor([np.inf], dtype=tdt))
            assert float(nxt) > v and u == float(nxt)


# ---------------------------------------------------------------- affine

def _grid_exact(rows, K, g, bits, seed, smin=-6):
    """w = z + s*q with power-of-two s, integer z, codes 0 and n in every group."""
    r = np.random.default_rng(seed)
    n = (1 << bits) - 1
    G = K // g
    q = r.integers(0, n + 1, size=(rows, K))
    q[:, ::g] = 0
    q[:, 1::g] = n
    s = 2.0 ** r.integers(smin, 1, size=(rows, G))
    z = r.integers(-8, 8, size=(rows, G)).astype(np.float64)
    w = z.repeat(g, 1) + s.repeat(g, 1) * q
    return w.astype(np.float32), q, s, z


def _unpack(wq, bits, K):
    per = 32 // bits
    k = np.arange(K)
    return (wq[..., k // per] >> ((k % per) * bits).astype(np.uint32)) & ((1 << bits) - 1)


@pytest.mark.parametrize("bits,g", [(2, 32), (4, 64), (8, 128), (4, 32), (8, 64), (2, 128)])
def test_affine_grid_exact_closed_form(bits, g):
    w, q, s, z = _grid_exact(6, 256, g, bits, seed=bits * 100 + g)
    wq, sc, bi = oracle.quantize(w, "f32", g, bits)
    assert wq.shape == (6, 256 * bits // 32)
    assert np.array_equal(_unpack(wq, bits, 256), q)
    assert np.array_equal(sc.astype(np.float64), s)
    assert np.array_equal(bi.astype(np.float64), z)
    dq = oracle.dequantize(wq, sc, bi, g, bits, scale_dtype="f32")
    assert np.array_equal(dq, w)


def test_affine_grid_exact_bf16_storage():
    w, q, s, z = _grid_exact(4, 128, 64, 4, seed=7, smin=-2)
    wb = bf16_bits(w)
    assert np.array_equal(bf16_to_f32(wb), w)  # grid values are bf16-exact
    wq, sc, bi = oracle.quantize(wb, "bf16", 64, 4)
    assert np.array_equal(_unpack(wq, 4, 128), q)
    assert np.array_equal(bf16_to_f32(sc).astype(np.float64), s)
    assert np.array_equal(bf16_to_f32(bi).astype(np.float64), z)


def test_packing_word_layout():
    # codes 0..7 then 15 in the first group: the first word is 0x76543210
    w = np.zeros((1, 64), np.float32)
    w[0, :8] = np.arange(8)
    w[0, 8] = 15
    wq, sc, bi = oracle.quantize(w, "f32", 64, 4)
    assert sc[0, 0] == 1.0 and bi[0, 0] == 0.0
    assert wq[0, 0] == 0x76543210 and wq[0, 1] == 0xF
    # 8-bit: a group holding 0..255 maps to itself, little-endian bytes
    w8 = np.tile(np.arange(128, dtype=np.float32), (1, 1))
    w8[0, 1] = 255
    wq8, sc8, bi8 = oracle.quantize(w8, "f32", 128, 8)
    assert sc8[0, 0] == 1.0 and bi8[0, 0] == 0.0
    assert np.array_equal(wq8.view(np.uint8)[0], w8[0].astype(np.uint8))
    # 2-bit: codes 0,1,2,3,3,2,1,0,... -> bits 2k..2k+1
    w2 = np.array([[0, 1, 2, 3, 3, 2, 1, 0] * 4], np.float32)
    wq2, _, _ = oracle.quantize(w2, "f32", 32, 2)
    expect = sum(c << (2 * i) for i, c in enumerate([0, 1, 2, 3, 3, 2, 1, 0, 0, 1, 2, 3, 3, 2, 1, 0]))
    assert wq2[0, 0] == expect


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_rs_quantize_dequantize_roundtrip(bits):
    """mlx-rs test_quantize_dequantize: rows of 0..511, group 128."""
    x = np.tile(np.arange(512, dtype=np.float32), (128, 1))
    wq, sc, bi = oracle.quantize(x, "f32", 128, bits)
    assert wq.shape == (128, 512 // (32 // bits))
    assert sc.shape == (128, 4) and bi.shape == (128, 4)
    xh = oracle.dequantize(wq, sc, bi, 128, bits, scale_dtype="f32")
    assert np.abs(x - xh).max() <= 127.0 / (1 << bits)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("bits,g", [(2, 32), (4, 64), (8, 64), (4, 128)])
def test_affine_error_bound_half_scale(dtype, bits, g):
    t, wbits = synth.normal((16, 512), 0.02, 99, bits * 1000 + g, dtype)
    wf = t.float().numpy()
    wq, sc, bi = oracle.quantize(wbits, dtype, g, bits)
    s = (sc.astype(np.float32) if dtype == "f32" else
         torch.from_numpy(sc.view(np.int16)).view(torch.bfloat16 if dtype == "bf16" else torch.float16).float().numpy())
    dq = oracle.dequantize(wq, sc, bi, g, bits, scale_dtype=dtype)
    err = np.abs(wf - dq).reshape(16, -1, g)
    half = s[..., None] / 2
    # |w - dq| <= s/2 up to the single fp32 rounding of dq
    assert np.all(err <= half * (1 + 2 ** -20) + np.abs(dq).reshape(16, -1, g) * 2 ** -24)


def test_constant_group_is_exact():
    w = np.full((2, 64), 0.3, np.float32)
    wq, sc, bi = oracle.quantize(w, "f32", 64, 4)
    assert sc[0, 0] == 0 and np.all(wq == 0)
    assert np.array_equal(oracle.dequantize(wq, sc, bi, 64, 4, scale_dtype="f32"), w)


def test_dequant_output_dtypes_match_library_rounding():
    t, wbits = synth.normal((8, 256), 1.0, 5, 0, "f32")
    wq, sc, bi = oracle.quantize(wbits, "f32", 64, 4)
    d32 = oracle.dequantize(wq, sc, bi, 64, 4, scale_dtype="f32", out_dtype="f32")
    db = oracle.dequantize(wq, sc, bi, 64, 4, scale_dtype="f32", out_dtype="bf16")
    dh = oracle.dequantize(wq, sc, bi, 64, 4, scale_dtype="f32", out_dtype="f16")
    assert np.array_equal(db, bf16_bits(d32))
    assert np.array_equal(dh, d32.astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------- microscaled

@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8", "nvfp4"])
def test_micro_grid_exact_closed_form(mode):
    """Elements = code values x a chosen scale, with the group maximum present:
    quantize must return those codes and that scale byte exactly."""
    g, bits = oracle.MODE_PAIRING[mode]
    r = np.random.default_rng(11)
    rows, K = 5, 4 * g
    G = K // g
    fmt = "e4m3" if mode == "mxfp8" else "e2m1"
    ncode = 1 << bits
    valid = [c for c in range(ncode) if not (fmt == "e4m3" and (c & 0x7F) == 0x7F)]
    codes = r.choice(valid, size=(rows, K))
    maxcode = 0x7E if fmt == "e4m3" else 0x7
    codes[:, ::g] = maxcode                      # amax present in every group
    vals = np.vectorize(lambda c: oracle.decode(fmt, int(c)))(codes)
    if mode == "nvfp4":
        sbytes = r.integers(0x20, 0x60, size=(rows, G))   # normal e4m3 scales
        scale = np.vectorize(lambda c: oracle.decode("e4m3", int(c)))(sbytes)
    else:
        e = r.integers(-20, 20, size=(rows, G))
        sbytes = e + 127
        scale = 2.0 ** e
    w = (vals * scale.repeat(g, 1)).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), vals * scale.repeat(g, 1))
    wq, sc, bi = oracle.quantize(w, "f32", g, bits, mode)
    assert bi is None and sc.dtype == np.uint8
    assert np.array_equal(sc, sbytes.astype(np.uint8))
    got = _unpack(wq, bits, K)
    # -0 and +0 both decode to 0; compare values, and codes where nonzero
    nz = vals != 0
    assert np.array_equal(got[nz], codes[nz])
    dq = oracle.dequantize(wq, sc, None, g, bits, mode)
    assert np.array_equal(dq, w)


def test_mx_shared_exponent_rule():
    # amax in [4, 8) -> floor(log2 amax) = 2 -> e = 0 for E2M1 (emax 2)
    w = np.zeros((1, 32), np.float32)
    w[0, 0], w[0, 1], w[0, 2] = 7.0, 2.5, -0.1
    wq, sc, _ = oracle.quantize(w, "f32", 32, 4, "mxfp4")
    assert sc[0, 0] == 127
    c = _unpack(wq, 4, 32)[0]
    assert c[0] == 0x7 and c[1] == 0x4 and c[2] == 0x8   # saturate 7->6, tie 2.5->2, -0
    # all zeros -> byte 0, codes 0
    wz = np.zeros((1, 32), np.float32)
    wq, sc, _ = oracle.quantize(wz, "f32", 32, 8, "mxfp8")
    assert sc[0, 0] == 0 and np.all(wq == 0)
    # nvfp4: scale = e4m3(amax/6)
    w = np.zeros((1, 16), np.float32)
    w[0, 0] = 12.0
    wq, sc, _ = oracle.quantize(w, "f32", 16, 4, "nvfp4")
    assert oracle.decode("e4m3", sc[0, 0]) == 2.0 and _unpack(wq, 4, 16)[0, 0] == 0x7


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8", "nvfp4"])
def test_micro_error_bound(mode):
    g, bits = oracle.MODE_PAIRING[mode]
    t, wbits = synth.normal((8, 512), 0.02, 3, 0, "bf16")
    wf = t.float().numpy()
    wq, sc, _ = oracle.quantize(wbits, "bf16", g, bits, mode)
    dq = oracle.dequantize(wq, sc, None, g, bits, mode)
    fmt = "e4m3" if mode == "mxfp8" else "e2m1"
    sfmt = "e4m3" if mode == "nvfp4" else "e8m0"
    scale = np.vectorize(lambda c: oracle.decode(sfmt, int(c)))(sc).repeat(g, 1)
    v = np.abs(wf) / scale
    # half the element-grid spacing at |v| (mantissa bits 1 / 3), plus saturation
    p = 2 if fmt == "e2m1" else 4
    emin = 0 if fmt == "e2m1" else -6
    E = np.maximum(np.floor(np.log2(np.maximum(v, 1e-30))), emin)
    half = 2.0 ** (E - p + 1) / 2 * scale
    maxv = 6.0 if fmt == "e2m1" else 448.0
    sat = np.maximum(np.abs(wf) - maxv * scale, 0)
    assert np.all(np.abs(wf - dq) <= half + sat + 1e-30)


def test_mode_pairing_rejected():
    w = np.zeros((2, 64), np.float32)
    for mode, (g, b) in oracle.MODE_PAIRING.items():
        oracle.quantize(w, "f32", g, b, mode)  # accepted
        for gg, bb in [(64, b), (g, 2), (128, 8)]:
            if (gg, bb) != (g, b):
                with pytest.raises(oracle.OracleError):
                    oracle.quantize(w, "f32", gg, bb, mode)
    for bad in [(64, 3), (64, 6), (16, 4), (48, 4)]:
        with pytest.raises(oracle.OracleError):
            oracle.quantize(w, "f32", bad[0], bad[1], "affine")
    with pytest.raises(oracle.OracleError):
        oracle.quantize(np.zeros((2, 96), np.float32), "f32", 64, 4)   # 64 does not divide 96
    with pytest.raises(oracle.OracleError):
        oracle.quantize(w, "f32", 64, 4, "int4")


# ---------------------------------------------------------------- matmul

@pytest.mark.parametrize("transpose", [True, False])
@pytest.mark.parametrize("bits,g", [(4, 64), (2, 32), (8, 128)])
def test_qmm_grid_exact_equals_integer_matmul(transpose, bits, g):
    N, K, M = 128, 256, 5
    rows, cols = (N, K) if transpose else (K, N)
    w, q, s, z = _grid_exact(rows, cols, g, bits, seed=31 + bits)
    x = np.random.default_rng(4).integers(-3, 4, size=(M, K)).astype(np.float32)
    wq, sc, bi = oracle.quantize(w, "f32", g, bits)
    y = oracle.quantized_matmul(x, "f32", wq, sc, bi, transpose, g, bits)
    W = w.astype(np.float64)
    ref = x.astype(np.float64) @ (W.T if transpose else W)
    assert np.array_equal(y, ref)
    assert y.shape == (M, N)


def test_qmm_bruteforce_tiny():
    """Every output element against an explicit fp64 triple loop."""
    t, wb = synth.normal((8, 64), 0.5, 21, 0, "bf16")
    tx, xb = synth.normal((3, 64), 1.0, 21, 1, "bf16")
    wq, sc, bi = oracle.quantize(wb, "bf16", 32, 4)
    y = oracle.quantized_matmul(xb, "bf16", wq, sc, bi, True, 32, 4)
    q = _unpack(wq, 4, 64).astype(np.float64)
    s = bf16_to_f32(sc).astype(np.float64)
    z = bf16_to_f32(bi).astype(np.float64)
    xf = bf16_to_f32(xb).astype(np.float64)
    for m in range(3):
        for n in range(8):
            acc, bound = 0.0, 0.0
            for k in range(64):
                wv = s[n, k // 32] * q[n, k] + z[n, k // 32]      # exact in fp64
                acc += xf[m, k] * wv
                bound += abs(xf[m, k]) * abs(wv) * 2.0 ** -24       # one fp32 rounding of wv
            assert abs(y[m, n] - acc) <= bound + 1e-12


def test_rs_quantized_matmul_transpose_false():
    """mlx-rs test_quantized_matmul: transpose=false, max diff < 1e-3."""
    m, n, k = 32, 128, 128
    sc_ = 1.0 / np.sqrt(k)
    tx, x = synth.normal((m, k), sc_, 1001, 1, "f32")
    tw, w = synth.normal((k, n), sc_, 1001, 0, "f32")
    wq, sc, bi = oracle.quantize(w, "f32", 64, 4)
    w_hat = oracle.dequantize(wq, sc, bi, 64, 4, scale_dtype="f32")
    y = oracle.quantized_matmul(x, "f32", wq, sc, bi, False, 64, 4)
    y_hat = x.astype(np.float32) @ w_hat
    assert y.shape == y_hat.shape == (m, n)
    assert np.abs(y - y_hat).max() < 1e-3


# ------------------------------------------------------- quantized_dense
# "Emily.Quantization.Layers" quantized_dense: x times the quantized W plus
# a bias (a tensor or a number, 0 by default).

def _bias_bits(vals, dtype):
    v = np.asarray(vals, np.float32)
    if dtype == "f32":
        return v
    t = torch.from_numpy(v).to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    assert np.array_equal(t.float().numpy(), v)      # the values are exact in dtype
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("transpose", [True, False])
@pytest.mark.parametrize("bdtype", ["f32", "bf16", "f16"])
def test_dense_grid_exact_equals_integer_matmul_plus_bias(transpose, bdtype):
    """Exact weights and integer x: y equals x.W^T (or x.W) plus the column
    bias broadcast over the rows, exactly in fp64 (a bias indexed by row, or
    by the wrong layout's axis, fails: M != N and every column differs)."""
    N, K, M = 128, 256, 5
    rows, cols = (N, K) if transpose else (K, N)
    w, q, s, z = _grid_exact(rows, cols, 64, 4, seed=77)
    x = np.random.default_rng(5).integers(-3, 4, size=(M, K)).astype(np.float32)
    b = (np.arange(N) - 40) / 4.0                       # k/4: exact in f32, bf16 and f16
    wq, sc, bi = oracle.quantize(w, "f32", 64, 4)
    y = oracle.quantized_dense(x, "f32", wq, sc, bi, _bias_bits(b, bdtype), bdtype,
                               transpose=transpose, group_size=64, bits=4)
    W = w.astype(np.float64)
    ref = x.astype(np.float64) @ (W.T if transpose else W) + b[None, :]
    assert y.shape == (M, N)
    assert np.array_equal(y, ref)


def test_dense_number_bias_is_taken_in_fp32():
    N, K, M = 32, 128, 3
    w, q, s, z = _grid_exact(N, K, 32, 4, seed=78)
    x = np.random.default_rng(6).integers(-3, 4, size=(M, K)).astype(np.float32)
    wq, sc, bi = oracle.quantize(w, "f32", 32, 4)
    base = x.astype(np.float64) @ w.astype(np.float64).T   # exact small integers
    y = oracle.quantized_dense(x, "f32", wq, sc, bi, None, bias_value=0.1, group_size=32, bits=4)
    d = y - base                                           # exact: base is a small integer
    assert np.all(d == float(np.float32(0.1))) and float(np.float32(0.1)) != 0.1


def test_dense_zero_bias_is_quantized_matmul():
    tw, wb = synth.normal((48, 128), 0.02, 79, 0, "bf16")
    tx, xb = synth.normal((4, 128), 1.0, 79, 1, "bf16")
    wq, sc, bi = oracle.quantize(wb, "bf16", 64, 4)
    y0 = oracle.quantized_matmul(xb, "bf16", wq, sc, bi, True, 64, 4)
    assert np.array_equal(oracle.quantized_dense(xb, "bf16", wq, sc, bi), y0)
    zeros = _bias_bits(np.zeros(48), "bf16")
    assert np.array_equal(oracle.quantized_dense(xb, "bf16", wq, sc, bi, zeros, "bf16"), y0)


def test_dense_zero_input_gives_the_bias():
    """x = 0: every row of y is the bias vector (the broadcast is over rows)."""
    tw, wb = synth.normal((40, 64), 0.02, 80, 0, "bf16")
    wq, sc, bi = oracle.quantize(wb, "bf16", 32, 4)
    tb, bb = synth.normal((40,), 1.0, 80, synth.BIAS, "bf16")
    x = np.zeros((7, 64), np.uint16)                   # bf16 +0
    y = oracle.quantized_dense(x, "bf16", wq, sc, bi, bb, "bf16", group_size=32, bits=4)
    assert np.array_equal(y, np.broadcast_to(bf16_to_f32(bb).astype(np.float64), (7, 40)))


def test_dense_rejects_bad_bias():
    tw, wb = synth.normal((40, 64), 0.02, 81, 0, "bf16")
    wq, sc, bi = oracle.quantize(wb, "bf16", 32, 4)
    x = np.zeros((2, 64), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.quantized_dense(x, "bf16", wq, sc, bi, np.zeros(39, np.float32), group_size=32, bits=4)
    with pytest.raises(oracle.OracleError):
        oracle.quantized_dense(x, "bf16", wq, sc, bi, None, bias_value=float("inf"), group_size=32, bits=4)
    with pytest.raises(oracle.OracleError):      # finite in fp64, not in fp32
        oracle.quantized_dense(x, "bf16", wq, sc, bi, None, bias_value=1e39, group_size=32, bits=4)


# ------------------------------------------------------------------ qqmm
# mlx-rs qqmm: x quantized on the fly (nvfp4 or mxfp8), W already quantized.

def _micro_grid_x(mode, rows, K, seed):
    """x whose groups are already on the mode's grid: code values times a
    chosen scale with the group maximum present (quantize reproduces it)."""
    g, bits = oracle.MODE_PAIRING[mode]
    r = np.random.default_rng(seed)
    fmt = "e4m3" if mode == "mxfp8" else "e2m1"
    valid = [c for c in range(1 << bits) if not (fmt == "e4m3" and (c & 0x7F) == 0x7F)]
    codes = r.choice(valid, size=(rows, K))
    codes[:, ::g] = 0x7E if fmt == "e4m3" else 0x7
    vals = np.vectorize(lambda c: oracle.decode(fmt, int(c)))(codes)
    G = K // g
    if mode == "nvfp4":
        scale = np.vectorize(lambda c: oracle.decode("e4m3", int(c)))(r.integers(0x28, 0x48, size=(rows, G)))
    else:
        scale = 2.0 ** r.integers(-6, 3, size=(rows, G))
    return (vals * scale.repeat(g, 1)).astype(np.float32)


def _micro_weight(mode, N, K, seed):
    g, bits = oracle.MODE_PAIRING[mode]
    tw, wb = synth.normal((N, K), 0.02, seed, synth.WEIGHT, "bf16")
    wq, sc, _ = oracle.quantize(wb, "bf16", g, bits, mode)
    return wq, sc, g, bits


@pytest.mark.parametrize("mode", ["nvfp4", "mxfp8"])
def test_qqmm_grid_x_equals_quantized_matmul(mode):
    """x already on its grid: quantizing it changes nothing, so qqmm is the
    plain quantized matmul of x, exactly."""
    N, K, M = 24, 128, 5
    x = _micro_grid_x(mode, M, K, seed=90)
    wq, sc, g, bits = _micro_weight(mode, N, K, 90)
    y, xhat = oracle.qqmm(x, "f32", wq, sc, True, g, bits, mode, return_xhat=True)
    assert np.array_equal(xhat, x)
    assert np.array_equal(y, oracle.quantized_matmul(x, "f32", wq, sc, None, True, g, bits, mode))


@pytest.mark.parametrize("mode,k", [("nvfp4", 3), ("nvfp4", -2), ("mxfp8", 5), ("mxfp8", -7)])
def test_qqmm_power_of_two_scaling(mode, k):
    """Scaling x by 2^k moves every block scale by 2^k and keeps the codes
    (no scale leaves its normal range here), so y scales exactly."""
    N, K, M = 16, 128, 4
    tx, _ = synth.normal((M, K), 1.0, 91, synth.ACT, "f32")
    x = tx.numpy()
    wq, sc, g, bits = _micro_weight(mode, N, K, 91)
    y = oracle.qqmm(x, "f32", wq, sc, True, g, bits, mode)
    y2 = oracle.qqmm((x * 2.0 ** k).astype(np.float32), "f32", wq, sc, True, g, bits, mode)
    assert np.array_equal(y2, y * 2.0 ** k)


@pytest.mark.parametrize("mode", ["nvfp4", "mxfp8"])
def test_qqmm_error_bound_against_unquantized_x(mode):
    """Each x element moves by at most half a grid step of its group (closed
    form below); y moves by at most the sum of those moves times |W|."""
    N, K, M = 16, 256, 3
    tx, _ = synth.normal((M, K), 1.0, 92, synth.ACT, "f32")
    x = tx.numpy().astype(np.float64)
    wq, sc, g, bits = _micro_weight(mode, N, K, 92)
    y, xhat = oracle.qqmm(tx.numpy(), "f32", wq, sc, True, g, bits, mode, return_xhat=True)
    amax = np.abs(x).reshape(M, K // g, g).max(-1).repeat(g, 1)
    if mode == "mxfp8":   # e4m3 under the shared exponent e = floor(log2 amax) - 8: half an ulp
        E = np.floor(np.log2(amax))   # of the top binade, or the clamp of (448, 512) x 2^e to 448
        bound_x = np.maximum(2.0 ** (E - 4), amax - 448.0 * 2.0 ** (E - 8))
    else:                 # e2m1 grid gap <= 2 at scale ~amax/6 (scale rounded up to 2^-4 relative)
        bound_x = amax / 6.0 * (1 + 2.0 ** -4)
    assert np.all(np.abs(xhat - x) <= bound_x)
    wd = oracle.dequantize(wq, sc, None, g, bits, mode).astype(np.float64)
    y0 = oracle.quantized_matmul(tx.numpy(), "f32", wq, sc, None, True, g, bits, mode)
    assert np.all(np.abs(y - y0) <= bound_x @ np.abs(wd).T + 1e-9)


def test_qqmm_modes():
    wq, sc, g, bits = _micro_weight("mxfp8", 8, 64, 93)
    x = np.zeros((2, 64), np.float32)
    for mode, gg, b in [("affine", 64, 4), ("mxfp4", 32, 4)]:
        with pytest.raises(oracle.OracleError):
            oracle.qqmm(x, "f32", wq, sc, True, gg, b, mode)


def test_page_example_shapes():
    # "Emily.QuantizedWeight" from_dense / to_dense examples
    t, w = synth.iota((4, 64))
    wq, sc, bi = oracle.quantize(w, "f32", 64, 4)
    assert wq.shape == (4, 8)
    assert oracle.dequantize(wq, sc, bi, 64, 4, scale_dtype="f32").shape == (4, 64)
    # "Emily.Quantization.Layers" quantized_dense example: {2,128} . {4,128} -> {2,4}
    t, w = synth.iota((4, 128))
    t, x = synth.iota((2, 128))
    wq, sc, bi = oracle.quantize(w, "f32", 64, 4)
    y = oracle.quantized_matmul(x, "f32", wq, sc, bi, True, 64, 4)
    assert y.shape == (2, 4)
    # each W group is 64 consecutive integers: |y - x.W^T| <= sum|x| * scale/2
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.all(np.abs(y - exact) <= np.abs(x).sum(1, keepdims=True) * (63 / 15) / 2 * 1.0001)
    # "EMLX.Quantization" basic usage: {1,8,4096} . {512,4096} -> {1,8,512}
    t, w = synth.iota((512, 4096))
    t, x = synth.iota((1, 8, 4096))
    wq, sc, bi = oracle.quantize(w, "f32", 64, 4)
    y = oracle.quantized_matmul(x, "f32", wq, sc, bi, True, 64, 4)
    assert y.shape == (1, 8, 512)


# ---------------------------------------------------------------- gather

def test_gather_grid_exact_and_rs_cases():
    E, N, K, M = 3, 64, 64, 32
    ws = [_grid_exact(N, K, 64, 4, seed=50 + e)[0] for e in range(E)]
    w = np.stack(ws)
    wq, sc, bi = oracle.quantize(w, "f32", 64, 4)
    r = np.random.default_rng(8)
    for B, lhs in [(1, [0]), (5, [0, 2])]:
        x = r.integers(-2, 3, size=(B, M, K)).astype(np.float32)
        rhs = [2, 1]
        lhs_b = np.broadcast_to(np.array(lhs), (2,))
        y = oracle.gather_qmm(x, "f32", wq, sc, bi, rhs, lhs_b, True, 64, 4)
        for i in range(2):
            ref = x[lhs_b[i]].astype(np.float64) @ w[rhs[i]].astype(np.float64).T
            assert np.array_equal(y[i], ref)


def test_rs_gather_qmm_cases():
    """mlx-rs test_gather_qmm, both index cases, against gather_mm on w_hat."""
    m, n, k = 32, 64, 64
    tw, w = synth.normal((3, n, k), 1.0, 2002, 0, "f32")
    wq, sc, bi = oracle.quantize(w, "f32", 64, 4)
    w_hat = oracle.dequantize(wq, sc, bi, 64, 4, scale_dtype="f32")
    for B, lhs in [(1, [0, 0]), (5, [0, 2])]:
        tx, x = synth.normal((B, m, k), 1.0, 2002, 1 + B, "f32")
        rhs = [2, 1]
        c1 = np.stack([x[lhs[i]] @ w_hat[rhs[i]].T for i in range(2)])
        c2 = oracle.gather_qmm(x, "f32", wq, sc, bi, rhs, lhs, True, 64, 4)
        assert np.allclose(c1, c2, rtol=1e-4, atol=1e-4)


def test_gather_permutation_and_identity():
    E, N, K, M = 4, 32, 128, 2
    tw, w = synth.normal((E, N, K), 0.02, 7, 0, "bf16")
    tx, x = synth.normal((6, M, K), 1.0, 7, 1, "bf16")
    wq, sc, bi = oracle.quantize(w, "bf16", 64, 4)
    rhs = np.array([3, 0, 1, 3, 2, 0])
    y = oracle.gather_qmm(x, "bf16", wq, sc, bi, rhs, None, True, 64, 4)
    perm = np.array([5, 2, 0, 4, 1, 3])
    yp = oracle.gather_qmm(x, "bf16", wq, sc, bi, rhs[perm], perm, True, 64, 4)
    assert np.array_equal(yp, y[perm])
    # constant rhs = a plain quantized matmul on that expert
    y1 = oracle.gather_qmm(x, "bf16", wq, sc, bi, np.full(6, 2), None, True, 64, 4)
    ref = oracle.quantized_matmul(x.reshape(-1, K), "bf16", wq[2], sc[2], bi[2], True, 64, 4)
    assert np.array_equal(y1.reshape(-1, N), ref)


# ------------------------------------------------- rounding of the codes
# The affine code is the nearest-even integer of the IEEE fp32 quotient
# (w - bias) / scale, and the dequantized value is scale*q + bias with one
# rounding. These pins take the expected values from numpy's IEEE float32
# division, numpy's round-half-even rint, and exact fp64 arithmetic: none of
# them restates the oracle's own code path.

def _ulp_steps(v, k):
    """v moved k float32 ulps (k may be negative)."""
    v = np.float32(v)
    to = np.float32(np.inf if k > 0 else -np.inf)
    for _ in range(abs(k)):
        v = np.nextafter(v, to, dtype=np.float32)
    return v


@pytest.mark.parametrize("bits,a,k", [(8, 3, 0), (8, 63, 4), (4, 3, 6), (4, 11, 2), (2, 15, 9), (2, 25, 3)])
def test_affine_codes_are_ieee_quotient_ties_even(bits, a, k):
    """Groups with bias 0 and scale s = a*2^-k (the group holds 0 and n*s, so
    the stored scale is exactly s); the other elements sit on each half-step
    (m + 1/2)*s and 1-2 ulps around it. Exact half-steps must give the even
    code (numpy rint); the others must give rint of numpy's IEEE fp32
    quotient. A reciprocal multiply d*(1/s) or a half-up floor(t + 1/2)
    changes some of these codes."""
    n = (1 << bits) - 1
    g = 64
    s = np.float32(a * 2.0 ** -k)
    assert np.float32(np.float32(n * s) / np.float32(n)) == s
    vals = []
    for m in range(n):
        tie = np.float32((m + 0.5) * s)
        assert np.float64(tie) == (m + 0.5) * np.float64(s)      # exact half-step
        vals += [tie] + [_ulp_steps(tie, d) for d in (-2, -1, 1, 2)]
    per = g - 2
    vals += [vals[-1]] * (-len(vals) % per)
    rows = np.array(vals, np.float32).reshape(-1, per)
    w = np.concatenate([np.zeros((len(rows), 1), np.float32),
                        np.full((len(rows), 1), np.float32(n * s)), rows], axis=1)
    wq, sc, bi = oracle.quantize(w, "f32", g, bits)
    assert np.all(sc == s) and np.all(bi == 0)
    expect = np.clip(np.rint(w / s), 0, n).astype(np.int64)      # IEEE quotient, ties even
    got = _unpack(wq, bits, g).astype(np.int64)
    assert np.array_equal(got, expect)
    # the exact half-steps really are ties and went to the even neighbour
    ties = (np.float64(w) / np.float64(s)) % 1.0 == 0.5
    assert ties.sum() >= n and np.all(got[ties] % 2 == 0)
    # the reciprocal product disagrees with the quotient on some of these
    # elements, so the test can tell the two apart
    assert np.any(np.rint(w * np.float32(np.float32(1) / s)) != np.rint(w / s))


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_affine_dequant_single_rounding(sdt):
    """dequant = scale*q + bias rounded once to fp32. For the scales and
    biases drawn here s*q + z is exact in fp64 (s*q has at most 32
    significant bits and |z| is within 2^12 of |s|), so np.float32 of the fp64
    value is that one rounding; with fp32 scales, rounding s*q first differs
    on many elements."""
    r = np.random.default_rng(21)
    rows, g, bits = 64, 64, 8
    G = 4
    K = G * g
    s = np.float32(np.abs(r.standard_normal((rows, G))) * 0.01 + 1e-4)
    z = np.float32(r.standard_normal((rows, G)) * 0.3)
    if sdt == "bf16":
        sb, zb = bf16_bits(s), bf16_bits(z)
        s, z = bf16_to_f32(sb), bf16_to_f32(zb)
    elif sdt == "f16":
        sb, zb = s.astype(np.float16).view(np.uint16), z.astype(np.float16).view(np.uint16)
        s, z = sb.view(np.float16).astype(np.float32), zb.view(np.float16).astype(np.float32)
    else:
        sb, zb = s, z
    q = r.integers(0, 256, size=(rows, K))
    per = 32 // bits
    wq = np.zeros((rows, K // per), np.uint32)
    for j in range(per):
        wq |= (q[:, j::per].astype(np.uint32) << np.uint32(bits * j))
    dq = oracle.dequantize(wq, sb, zb, g, bits, scale_dtype=sdt)
    s64, z64 = s.astype(np.float64).repeat(g, 1), z.astype(np.float64).repeat(g, 1)
    expect = (s64 * q + z64).astype(np.float32)
    assert np.array_equal(dq, expect)
    if sdt == "f32":
        # with 16-bit scales s*q is exact in fp32 and the two forms agree;
        # with fp32 scales rounding the product first changes some values
        two = (s.repeat(g, 1) * q.astype(np.float32)).astype(np.float32) + z.repeat(g, 1)
        assert np.count_nonzero(two != expect) > 0


def test_nvfp4_codes_use_ieee_quotient():
    """nvfp4 elements are fl32(w / scale) rounded nearest-even into E2M1.
    Each group holds 6*sc (so the scale byte decodes to exactly sc) and values
    on and 1-2 ulps around the E2M1 midpoints times sc; expected codes come
    from numpy's IEEE float32 division and a brute-force nearest-even search.
    Dividing by way of a reciprocal moves some of them across a midpoint."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    groups, expect_codes, recip_differs = [], [], False
    for sbyte in range(0x30, 0x48):                  # normal e4m3 scales around 1
        sc = np.float32(oracle.decode("e4m3", sbyte))
        vals = []
        for t in mids:
            tie = np.float32(t * sc)
            assert np.float64(tie) == t * np.float64(sc)
            vals += [tie] + [_ulp_steps(tie, d) for d in (-2, -1, 1, 2)]
        vals += [-v for v in vals[:10]]
        for i in range(0, len(vals), 15):
            chunk = vals[i:i + 15]
            chunk += [chunk[-1]] * (15 - len(chunk))
            grp = np.array([6 * sc] + chunk, np.float32)
            groups.append(grp)
            q = grp / sc                               # IEEE float32 division
            expect_codes.append([_e2m1_nearest_even_bruteforce(float(v)) for v in q])
            rq = grp * np.float32(np.float32(1) / sc)
            if any(_e2m1_nearest_even_bruteforce(float(v)) != c
                   for v, c in zip(rq, expect_codes[-1])):
                recip_differs = True
    assert recip_differs
    w = np.stack(groups)
    wq, sc_b, _ = oracle.quantize(w, "f32", 16, 4, "nvfp4")
    got = _unpack(wq, 4, 16)
    assert np.array_equal(got, np.array(expect_codes))


@pytest.mark.parametrize("mode,c,xhat", [
    # mxfp8: amax 1.1 -> shared exponent floor(log2 1.1) - 8 = -8; 1.1*2^8 = 281.6
    # lies between the E4M3 values 256 and 288 (spacing 32 in [256, 512)) and
    # is nearer 288, so x-hat = 288 * 2^-8 = 1.125
    ("mxfp8", 1.1, 1.125),
    # nvfp4: amax/6 = 0.18333 lies between the E4M3 values 0.171875 and 0.1875
    # (spacing 2^-6 in [0.125, 0.25)) -> scale 0.1875; 1.1/0.1875 = 5.87 rounds
    # to the E2M1 value 6 (midpoint 5) -> x-hat = 6 * 0.1875 = 1.125
    ("nvfp4", 1.1, 1.125),
    # nvfp4: 0.7/6 = 0.11667 -> E4M3 0.1171875 (spacing 2^-7 in [2^-4, 2^-3));
    # 0.7/0.1171875 = 5.97 -> 6 -> x-hat = 0.703125
    ("nvfp4", 0.7, 0.703125),
    # mxfp8: amax 0.3 -> exponent floor(log2 0.3) - 8 = -10; 0.3*2^10 = 307.2 ->
    # E4M3 320 (between 288 and 320, nearer 320) -> x-hat = 320 * 2^-10 = 0.3125
    ("mxfp8", 0.3, 0.3125),
])
def test_qqmm_constant_x_closed_form(mode, c, xhat):
    """x constant off the grid: x-hat is the closed-form value above, and with
    W on its grid (dequant(W) = W exactly) y = x-hat * (row sums of W),
    exactly in fp64. Using the unquantized x gives c * (row sums) instead."""
    g, bits = oracle.MODE_PAIRING[mode]
    N, K, M = 12, 4 * g, 3
    W = _micro_grid_x(mode, N, K, seed=95)
    wq, sc, _ = oracle.quantize(W, "f32", g, bits, mode)
    assert np.array_equal(oracle.dequantize(wq, sc, None, g, bits, mode), W)
    x = np.full((M, K), np.float32(c), np.float32)
    y, xh = oracle.qqmm(x, "f32", wq, sc, True, g, bits, mode, return_xhat=True)
    assert np.all(xh == np.float32(xhat))
    rowsum = W.astype(np.float64).sum(1)
    assert np.array_equal(y, np.broadcast_to(xhat * rowsum, (M, N)))
    assert not np.allclose(y, np.float64(np.float32(c)) * rowsum, rtol=1e-3, atol=0)


@pytest.mark.parametrize("mode", ["nvfp4", "mxfp8"])
def test_qqmm_differs_from_unquantized_x(mode):
    """On random x the quantization of x is visible in y: y departs from the
    product with the unquantized x by more than fp64 rounding could explain
    (a lower bound beside the error bound above)."""
    N, K, M = 16, 256, 3
    tx, _ = synth.normal((M, K), 1.0, 96, synth.ACT, "f32")
    wq, sc, g, bits = _micro_weight(mode, N, K, 96)
    y = oracle.qqmm(tx.numpy(), "f32", wq, sc, True, g, bits, mode)
    y0 = oracle.quantized_matmul(tx.numpy(), "f32", wq, sc, None, True, g, bits, mode)
    assert np.abs(y - y0).max() > 1e-3 * np.abs(y0).max()


def test_affine_scale_rounds_up_in_bf16():
    """An int8 bf16 group with minimum -0.75 and maximum 255: the fp32 scale
    is 255.75/255 = 1.00294, which lies below the bf16 midpoint 1.00390625
    between 1 and 1.0078125. Nearest-even storage would give scale 1 and put
    the group maximum 0.75 (> scale/2) away from its dequantized value
    (code 255 -> -0.75 + 255). The stored scale must be the bf16 value just
    above the fp32 scale (torch nextafter) and keep |w - dq| <= s/2 for every
    element (the benchmark spec's bound)."""
    w = np.linspace(-0.75, 255.0, 64, dtype=np.float32)[None, :]
    wb = bf16_bits(w)
    wf = bf16_to_f32(wb)
    assert wf.min() == -0.75 and wf.max() == 255.0
    wq, sc, bi = oracle.quantize(wb, "bf16", 64, 8)
    s = float(bf16_to_f32(sc)[0, 0])
    s32 = np.float32(np.float32(255.75) / np.float32(255))
    rn = torch.tensor(float(s32)).to(torch.bfloat16)
    assert float(rn) == 1.0                       # nearest-even would round down
    up = torch.nextafter(rn, torch.tensor(np.inf, dtype=torch.bfloat16))
    assert s == float(up) == 1.0078125
    assert float(bf16_to_f32(bi)[0, 0]) == -0.75
    dq = oracle.dequantize(wq, sc, bi, 64, 8, scale_dtype="bf16")
    assert np.all(np.abs(wf - dq) <= s / 2 * (1 + 2 ** -20))
    assert 255.0 - (-0.75 + 255 * 1.0) > 1.0 / 2   # the bound the down-rounded scale breaks
