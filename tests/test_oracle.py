"""Pins for the fp64 oracle against facts fixed outside the oracle itself:
hand-worked examples (tests/golden), library routines (numpy float16 casts,
torch bfloat16 casts, numpy float64 matmul, scipy correlate), closed forms
and invariants.  CPU only."""
import itertools

import numpy as np
import pytest
import scipy.signal
import torch

import oracle
from conftest import read_golden

RNG = np.random.default_rng(12345)


def f16_bits(vals):
    return np.asarray(vals, np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(vals):
    return torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def lib_decode(bits, dtype):
    """Independent decode through numpy / torch casts."""
    bits = np.asarray(bits, np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


# ---------------------------------------------------------------- encodings
def test_golden_encodings():
    for row in read_golden("encodings.txt"):
        fmt, bits, expr = row[0], row[1], " ".join(row[2:])
        want = eval(expr, {"__builtins__": {}}, {"float": float})
        got = oracle.decode(np.array([int(bits, 16)], np.uint16), fmt)[0]
        assert got == want and np.signbit(got) == np.signbit(want), (fmt, bits)
        if fmt == "f8e4m3":  # fp8 is an input type only: the oracle never rounds to it
            continue
        back = oracle.round_to(np.array([want]), fmt)[0]
        assert back == int(bits, 16), (fmt, bits, hex(back))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_all_patterns_match_library(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, dtype)
    want = lib_decode(bits, dtype)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_all_e4m3_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode(codes, "f8e4m3")
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert nan.sum() == 2  # S.1111.111 only: the format has no infinities
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_gemm_fp8_brute_force_numpy():
    # fp8 A and B (codes), bf16 C: the oracle against numpy over torch-decoded values
    for M, N, K in [(1, 1, 16), (5, 7, 32), (13, 8, 48)]:
        a = RNG.integers(0, 256, (M, K + 16), dtype=np.uint8)
        b = RNG.integers(0, 256, (N, K + 16), dtype=np.uint8)
        a[(a & 0x7F) == 0x7F] = 0x38  # no NaN codes
        b[(b & 0x7F) == 0x7F] = 0x38
        c = bf16_bits(RNG.standard_normal((M, N)))
        dec = lambda x: torch.from_numpy(x.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        want = 0.5 * dec(a)[:, :K] @ dec(b)[:, :K].T - 2.0 * lib_decode(c, "bf16")
        got = oracle.gemm(a, b, c, K=K, alpha=0.5, beta=-2.0, dtype="f8e4m3")
        assert np.allclose(got, want, rtol=1e-13, atol=1e-13), (M, N, K)


def test_round_f16_matches_numpy_direct_double_to_half():
    # numpy converts float64 -> float16 in one correctly rounded step
    vals = np.concatenate([
        RNG.standard_normal(20000) * 10.0 ** RNG.uniform(-9, 5, 20000),
        RNG.uniform(-70000, 70000, 2000),
        # exact halfway points between neighbouring fp16 values
        (np.arange(0, 4000, dtype=np.float64) + 0.5) * 2.0 ** -24,
        (np.arange(1024, 2048, dtype=np.float64) + 0.5) * 2.0 ** -3,
        np.array([65504.0, 65519.99, 65520.0, -65520.0, 0.0, -0.0, 2.0 ** -25, 3 * 2.0 ** -26]),
    ])
    got = oracle.round_to(vals, "f16")
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_round_bf16_matches_torch_on_float32_values():
    f32 = np.concatenate([
        (RNG.standard_normal(20000) * 10.0 ** RNG.uniform(-30, 30, 20000)).astype(np.float32),
        np.array([3.3895314e38, 3.4e38, 1e-40, -1e-45, 0.0], np.float32),
    ])
    # halfway points: 1 + 2^-8 (tie -> 1.0, even) and 1 + 3*2^-8 (tie -> 1 + 2^-6)
    f32 = np.concatenate([f32, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32)])
    got = oracle.round_to(f32.astype(np.float64), "bf16")
    want = bf16_bits(f32)
    assert np.array_equal(got, want)
    assert got[-3] == 0x3F80 and got[-2] == 0x3F82 and got[-1] == 0xBF80


def test_round_bf16_double_not_rounded_twice():
    # 1 + 2^-8 + 2^-40 is above the tie: RNE from the double gives 1 + 2^-7;
    # rounding to float32 first would land on the tie and give 1.0
    assert oracle.round_to(np.array([1 + 2 ** -8 + 2 ** -40]), "bf16")[0] == 0x3F81


# ---------------------------------------------------------------- GEMM
def test_golden_gemm():
    g = {r[0]: r[1:] for r in read_golden("gemm_2x2x3.txt")}
    M, N, K = int(g["M"][0]), int(g["N"][0]), int(g["K"][0])
    A = f16_bits([float(v) for v in g["A"]]).reshape(M, K)
    B = f16_bits([float(v) for v in g["B"]]).reshape(N, K)
    C = f16_bits([float(v) for v in g["C"]]).reshape(M, N)
    D = oracle.gemm(A, B, C, alpha=float(g["alpha"][0]), beta=float(g["beta"][0]), dtype="f16")
    assert np.array_equal(D, np.array([float(v) for v in g["D"]]).reshape(M, N))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_brute_force_numpy(dtype):
    sizes = [1, 2, 3, 5, 8, 13]
    enc = f16_bits if dtype == "f16" else bf16_bits
    for M, N, K in itertools.product(sizes, sizes, sizes):
        A = enc(RNG.uniform(-2, 2, (M, K)))
        B = enc(RNG.uniform(-2, 2, (N, K)))
        C = enc(RNG.uniform(-2, 2, (M, N)))
        alpha, beta = 0.75, -1.5
        want = alpha * (lib_decode(A, dtype) @ lib_decode(B, dtype).T) + beta * lib_decode(C, dtype)
        got = oracle.gemm(A, B, C, alpha=alpha, beta=beta, dtype=dtype)
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_gemm_leading_dimensions_and_column_major_b():
    M, N, K, lda, ldb, ldc = 5, 7, 9, 16, 24, 8
    A = f16_bits(RNG.uniform(-1, 1, (M, lda)))
    B = f16_bits(RNG.uniform(-1, 1, (N, ldb)))
    C = f16_bits(RNG.uniform(-1, 1, (M, ldc)))
    got = oracle.gemm(A, B, C, K=K, beta=1.0)
    want = lib_decode(A[:, :K], "f16") @ lib_decode(B[:, :K], "f16").T + lib_decode(C[:, :N], "f16")
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_gemm_identity_a_returns_b_transposed():
    K, N = 12, 7
    A = f16_bits(np.eye(K))
    B = f16_bits(RNG.uniform(-4, 4, (N, K)))
    D = oracle.gemm(A, B)
    assert np.array_equal(D, lib_decode(B, "f16").T)


def test_gemm_all_ones_closed_form():
    M, N, K = 6, 5, 37
    C = f16_bits(RNG.uniform(-1, 1, (M, N)))
    D = oracle.gemm(f16_bits(np.ones((M, K))), f16_bits(np.ones((N, K))), C, alpha=1.5, beta=0.5)
    assert np.array_equal(D, 1.5 * K + 0.5 * lib_decode(C, "f16"))


def test_gemm_zero_a_and_k_zero_give_beta_c():
    M, N, K = 4, 3, 8
    C = bf16_bits(RNG.uniform(-1, 1, (M, N)))
    B = bf16_bits(RNG.uniform(-1, 1, (N, K)))
    D = oracle.gemm(bf16_bits(np.zeros((M, K))), B, C, beta=0.25, dtype="bf16")
    assert np.array_equal(D, 0.25 * lib_decode(C, "bf16"))
    D0 = oracle.gemm(np.zeros((M, 0), np.uint16), np.zeros((N, 0), np.uint16), C, beta=0.25, dtype="bf16")
    assert np.array_equal(D0, 0.25 * lib_decode(C, "bf16"))


def test_gemm_beta_zero_ignores_c():
    M, N, K = 3, 4, 5
    A = f16_bits(RNG.uniform(-1, 1, (M, K)))
    B = f16_bits(RNG.uniform(-1, 1, (N, K)))
    nan_c = np.full((M, N), 0x7E00, np.uint16)
    assert np.array_equal(oracle.gemm(A, B, nan_c, beta=0.0), oracle.gemm(A, B))


def test_grouped_per_group_constants():
    # A_g = 1, B_g = g + 1  =>  D_g = (g + 1) * K_g exactly
    for g, (M, N, K) in enumerate([(3, 4, 5), (1, 9, 16), (7, 2, 3)]):
        D = oracle.gemm(f16_bits(np.ones((M, K))), f16_bits(np.full((N, K), g + 1.0)))
        assert np.array_equal(D, np.full((M, N), (g + 1.0) * K))


# ---------------------------------------------------------------- W4A16
def test_golden_w4_dequant_and_gemm():
    g = {r[0]: r[1:] for r in read_golden("w4_dequant_2x4.txt")}
    N, K, grp = int(g["N"][0]), int(g["K"][0]), int(g["group"][0])
    q = np.array([int(v) for v in g["q"]], np.uint8).reshape(N, K)
    z = np.array([int(v) for v in g["z"]], np.uint8).reshape(K // grp, N)
    s = f16_bits([float(v) for v in g["s"]]).reshape(K // grp, N)
    Wp = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    Zp = (z[:, 0::2] | (z[:, 1::2] << 4)).astype(np.uint8)
    w = oracle.dequant_w4(Wp, s, Zp, N, K, grp)
    assert np.array_equal(w, np.array([float(v) for v in g["w"]]).reshape(N, K))
    X = f16_bits([float(v) for v in g["X"]]).reshape(1, K)
    Y = oracle.w4a16(X, Wp, s, Zp, N, K, grp)
    assert np.array_equal(Y, np.array([[float(v) for v in g["Y"]]]))


def _w4_case(M, N, K, grp, seed=7):
    r = np.random.default_rng(seed)
    q = r.integers(0, 16, (N, K), dtype=np.uint8)
    z = r.integers(0, 16, (K // grp, N), dtype=np.uint8)
    s = f16_bits(r.uniform(0.001, 0.01, (K // grp, N)))
    X = f16_bits(r.standard_normal((M, K)))
    pk = lambda a: (a[:, 0::2] | (a[:, 1::2] << 4)).astype(np.uint8)
    return q, z, s, X, pk(q), pk(z)


def test_w4a16_against_numpy_unpack_and_matmul():
    M, N, K, grp = 5, 12, 256, 64
    q, z, s, X, Wp, Zp = _w4_case(M, N, K, grp)
    # independent: numpy nibble extraction and group broadcast
    qn = np.empty((N, K), np.int64)
    qn[:, 0::2] = Wp & 15
    qn[:, 1::2] = Wp >> 4
    zn = np.empty((K // grp, N), np.int64)
    zn[:, 0::2] = Zp & 15
    zn[:, 1::2] = Zp >> 4
    sf = lib_decode(s, "f16")
    w = (qn - np.repeat(zn.T, grp, axis=1)) * np.repeat(sf.T, grp, axis=1)
    want = lib_decode(X, "f16") @ w.T
    np.testing.assert_allclose(oracle.w4a16(X, Wp, s, Zp, N, K, grp), want, rtol=1e-12, atol=1e-12)


def test_w4a16_two_oracle_paths_agree():
    M, N, K, grp = 3, 16, 384, 128
    q, z, s, X, Wp, Zp = _w4_case(M, N, K, grp, seed=9)
    w = oracle.dequant_w4(Wp, s, Zp, N, K, grp)
    via_gemm = lib_decode(X, "f16") @ w.T
    np.testing.assert_allclose(oracle.w4a16(X, Wp, s, Zp, N, K, grp), via_gemm, rtol=1e-12, atol=1e-12)


def test_w4_dequant_special_cases():
    N, K, grp = 4, 128, 128
    q, z, s, X, Wp, Zp = _w4_case(1, N, K, grp, seed=3)
    ones = f16_bits(np.ones((1, N)))
    eights = np.full((1, N // 2), 0x88, np.uint8)
    # s = 1, z = 8  =>  w = q - 8
    assert np.array_equal(oracle.dequant_w4(Wp, ones, eights, N, K, grp), q.astype(np.float64) - 8)
    # z = q  =>  w = 0
    qc = np.full((N, K), 5, np.uint8)
    Wc = np.full((N, K // 2), 0x55, np.uint8)
    assert np.array_equal(oracle.dequant_w4(Wc, s, np.full((1, N // 2), 0x55, np.uint8), N, K, grp),
                          np.zeros((N, K)))
    # s = 2^-e  => exact scaled integers
    sp = f16_bits(np.full((1, N), 2.0 ** -5))
    assert np.array_equal(oracle.dequant_w4(Wp, sp, eights, N, K, grp), (q.astype(np.float64) - 8) * 2.0 ** -5)
    del qc


def test_w4_group_equals_k_is_per_channel():
    N, K = 8, 256
    q, z, s, X, Wp, Zp = _w4_case(2, N, K, K, seed=5)
    w = oracle.dequant_w4(Wp, s, Zp, N, K, K)
    zz = np.empty(N, np.int64)
    zz[0::2] = Zp[0] & 15
    zz[1::2] = Zp[0] >> 4
    assert np.array_equal(w, (q.astype(np.int64) - zz[:, None]) * lib_decode(s, "f16")[0][:, None])


# ------------------------------------------------ conversion modes, int4, bf16
def _nibbles(packed, signed):
    """numpy nibble extraction; int4 by arithmetic-shift sign extension of the nibble placed in a byte's top."""
    n = np.empty((packed.shape[0], packed.shape[1] * 2), np.uint8)
    n[:, 0::2] = packed & 15
    n[:, 1::2] = packed >> 4
    if signed:
        return ((n << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.int64)
    return n.astype(np.int64)


def test_mixed_direct_convert_reads_each_nibble():
    W = np.arange(256, dtype=np.uint8).reshape(1, 256)  # every byte, so every nibble in both positions
    got_u = oracle.dequant_mixed(W, None, None, 1, 512, 512, "uint4")
    got_s = oracle.dequant_mixed(W, None, None, 1, 512, 512, "int4")
    assert np.array_equal(got_u, _nibbles(W, False).astype(np.float64))
    assert np.array_equal(got_s, _nibbles(W, True).astype(np.float64))
    # two's complement: nibble 8 is -8, 15 is -1, 7 is 7
    assert got_s[0, 0x08 * 2] == -8 and got_s[0, 0x0F * 2] == -1 and got_s[0, 0x07 * 2] == 7


def test_mixed_uint4_modes_reduce_to_the_zero_mode():
    N, K, grp = 6, 256, 128
    q, z, s, X, Wp, Zp = _w4_case(2, N, K, grp, seed=11)
    zero_z = np.zeros_like(Zp)
    ones = f16_bits(np.ones((K // grp, N)))
    assert np.array_equal(oracle.dequant_mixed(Wp, s, None, N, K, grp), oracle.dequant_w4(Wp, s, zero_z, N, K, grp))
    assert np.array_equal(oracle.dequant_mixed(Wp, None, None, N, K, grp),
                          oracle.dequant_w4(Wp, ones, zero_z, N, K, grp))
    assert np.array_equal(oracle.dequant_mixed(Wp, s, Zp, N, K, grp), oracle.dequant_w4(Wp, s, Zp, N, K, grp))
    assert np.array_equal(oracle.mixed(X, Wp, s, Zp, N, K, grp), oracle.w4a16(X, Wp, s, Zp, N, K, grp))


def test_mixed_int4_with_zeros_is_offset_binary_uint4():
    # v(q) - v(z) with two's complement nibbles equals (q ^ 8) - (z ^ 8) as unsigned nibbles
    N, K, grp = 8, 256, 64
    q, z, s, X, Wp, Zp = _w4_case(1, N, K, grp, seed=13)
    got = oracle.dequant_mixed(Wp, s, Zp, N, K, grp, "int4")
    assert np.array_equal(got, oracle.dequant_w4(Wp ^ 0x88, s, Zp ^ 0x88, N, K, grp))
    # and without zero points int4 is offset binary with the constant zero 8
    eights = np.full_like(Zp, 0x88)
    assert np.array_equal(oracle.dequant_mixed(Wp, s, None, N, K, grp, "int4"),
                          oracle.dequant_w4(Wp ^ 0x88, s, eights, N, K, grp))


@pytest.mark.parametrize("w_type,mode", [("int4", "zero"), ("int4", "scale"), ("uint4", "direct"),
                                         ("uint4", "zero")])
def test_mixed_bf16_against_numpy(w_type, mode):
    M, N, K, grp = 4, 10, 256, 128
    r = np.random.default_rng(17)
    Wp = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
    Zp = r.integers(0, 256, (K // grp, N // 2), dtype=np.uint8)
    s = bf16_bits(r.uniform(0.001, 0.01, (K // grp, N)))
    X = bf16_bits(r.standard_normal((M, K)))
    signed = w_type == "int4"
    v = _nibbles(Wp, signed)
    if mode == "zero":
        v = v - np.repeat(_nibbles(Zp, signed).T, grp, axis=1)
    w = v * (np.repeat(lib_decode(s, "bf16").T, grp, axis=1) if mode != "direct" else 1.0)
    want = lib_decode(X, "bf16") @ w.T
    got = oracle.mixed(X, Wp, s if mode != "direct" else None, Zp if mode == "zero" else None, N, K, grp, w_type,
                       "bf16")
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.dequant_mixed(Wp, None, Zp, N, K, grp)  # zero points without scales: no such mode


# ---------------------------------------------------------------- conv
def _conv_scipy(x, w, pad, stride, dil, dtype="bf16"):
    xd, wd = lib_decode(x, dtype), lib_decode(w, dtype)
    N, H, W, C = xd.shape
    K, R, S, _ = wd.shape
    xp = np.pad(xd, ((0, 0), (pad[0], pad[0]), (pad[1], pad[1]), (0, 0)))
    # dilated filter: insert (dil - 1) zeros between taps
    Rd, Sd = dil[0] * (R - 1) + 1, dil[1] * (S - 1) + 1
    wdl = np.zeros((K, Rd, Sd, C))
    wdl[:, ::dil[0], ::dil[1], :] = wd
    outs = []
    for n in range(N):
        per_k = []
        for k in range(K):
            acc = sum(scipy.signal.correlate2d(xp[n, :, :, c], wdl[k, :, :, c], mode="valid") for c in range(C))
            per_k.append(acc[::stride[0], ::stride[1]])
        outs.append(np.stack(per_k, axis=-1))
    return np.stack(outs)


def test_golden_conv():
    rows = read_golden("conv_3x3_2x2.txt")
    x = f16_bits([float(v) for v in rows[0][1:]]).reshape(1, 3, 3, 1)
    w = f16_bits([float(v) for v in rows[1][1:]]).reshape(1, 2, 2, 1)
    for r in rows[2:]:
        pad = int(r[1].split("=")[1])
        stride = int(r[2].split("=")[1])
        want = np.array([float(v) for v in r[4:]])
        got = oracle.conv2d_fprop(x, w, pad=(pad, pad), stride=(stride, stride), dtype="f16")
        assert np.array_equal(got.ravel(), want), (pad, stride, got.ravel())


@pytest.mark.parametrize("R,pad,stride,dil", [(1, 0, 1, 1), (3, 1, 1, 1), (3, 0, 2, 1), (3, 1, 2, 1),
                                              (3, 2, 1, 2), (2, 1, 1, 1)])
def test_conv_against_scipy_correlate(R, pad, stride, dil):
    x = bf16_bits(RNG.standard_normal((2, 7, 6, 8))).reshape(2, 7, 6, 8)
    w = bf16_bits(RNG.standard_normal((5, R, R, 8))).reshape(5, R, R, 8)
    got = oracle.conv2d_fprop(x, w, pad=(pad, pad), stride=(stride, stride), dil=(dil, dil))
    want = _conv_scipy(x, w, (pad, pad), (stride, stride), (dil, dil))
    assert got.shape == want.shape
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_conv_against_im2col_numpy_matmul():
    N, H, W, C, K, R, S, pad, st = 2, 5, 7, 16, 4, 3, 3, 1, 2
    x = bf16_bits(RNG.standard_normal(N * H * W * C)).reshape(N, H, W, C)
    w = bf16_bits(RNG.standard_normal(K * R * S * C)).reshape(K, R, S, C)
    xd, wd = lib_decode(x, "bf16"), lib_decode(w, "bf16")
    P = (H + 2 * pad - R) // st + 1
    Q = (W + 2 * pad - S) // st + 1
    cols = np.zeros((N, P, Q, R, S, C))
    for n, p, q, r, s in itertools.product(range(N), range(P), range(Q), range(R), range(S)):
        ih, iw = p * st - pad + r, q * st - pad + s
        if 0 <= ih < H and 0 <= iw < W:
            cols[n, p, q, r, s] = xd[n, ih, iw]
    want = cols.reshape(N * P * Q, R * S * C) @ wd.reshape(K, R * S * C).T
    got = oracle.conv2d_fprop(x, w, pad=(pad, pad), stride=(st, st))
    np.testing.assert_allclose(got.reshape(-1, K), want, rtol=1e-12, atol=1e-12)


def test_conv_1x1_equals_gemm():
    N, H, W, C, K = 2, 4, 3, 24, 6
    x = bf16_bits(RNG.standard_normal(N * H * W * C)).reshape(N, H, W, C)
    w = bf16_bits(RNG.standard_normal(K * C)).reshape(K, 1, 1, C)
    got = oracle.conv2d_fprop(x, w)
    want = oracle.gemm(x.reshape(-1, C), w.reshape(K, C), dtype="bf16")
    assert np.array_equal(got.reshape(-1, K), want)


def test_conv_all_ones_border_counts():
    # 3x3, pad 1: interior sums 9C, edges 6C, corners 4C
    N, H, W, C, K = 1, 6, 5, 16, 2
    got = oracle.conv2d_fprop(bf16_bits(np.ones(N * H * W * C)).reshape(N, H, W, C),
                              bf16_bits(np.ones(K * 9 * C)).reshape(K, 3, 3, C), pad=(1, 1))
    taps = np.full((H, W), 9.0)
    taps[0, :] = taps[-1, :] = 6
    taps[:, 0] = taps[:, -1] = 6
    taps[0, 0] = taps[0, -1] = taps[-1, 0] = taps[-1, -1] = 4
    assert np.array_equal(got[0, :, :, 0], taps * C) and np.array_equal(got[0, :, :, 1], taps * C)


def test_conv_delta_filter_is_identity():
    N, H, W, C = 2, 5, 4, 8
    x = bf16_bits(RNG.standard_normal(N * H * W * C)).reshape(N, H, W, C)
    w = np.zeros((C, 3, 3, C))
    for c in range(C):
        w[c, 1, 1, c] = 1.0
    got = oracle.conv2d_fprop(x, bf16_bits(w.ravel()).reshape(C, 3, 3, C), pad=(1, 1))
    assert np.array_equal(got, lib_decode(x, "bf16"))


@pytest.mark.parametrize("r,s", [(0, 0), (0, 2), (2, 1), (1, 0)])
def test_conv_one_hot_tap_shifts_input(r, s):
    # cross-correlation: y[p][q] = x[p + r - 1][q + s - 1] (zero outside)
    N, H, W, C = 1, 5, 6, 8
    x = bf16_bits(RNG.standard_normal(N * H * W * C)).reshape(N, H, W, C)
    w = np.zeros((C, 3, 3, C))
    for c in range(C):
        w[c, r, s, c] = 1.0
    got = oracle.conv2d_fprop(x, bf16_bits(w.ravel()).reshape(C, 3, 3, C), pad=(1, 1))
    xd = np.pad(lib_decode(x, "bf16"), ((0, 0), (1, 1), (1, 1), (0, 0)))
    assert np.array_equal(got, xd[:, r:r + H, s:s + W, :])


def test_conv_beta_term():
    x = bf16_bits(RNG.standard_normal(1 * 4 * 4 * 8)).reshape(1, 4, 4, 8)
    w = bf16_bits(RNG.standard_normal(3 * 3 * 3 * 8)).reshape(3, 3, 3, 8)
    c = bf16_bits(RNG.standard_normal(1 * 4 * 4 * 3)).reshape(1, 4, 4, 3)
    base = oracle.conv2d_fprop(x, w, pad=(1, 1))
    got = oracle.conv2d_fprop(x, w, pad=(1, 1), C_in=c, alpha=2.0, beta=-0.5)
    np.testing.assert_allclose(got, 2.0 * base - 0.5 * lib_decode(c, "bf16"), rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- conv fused bias / ReLU epilogue
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_conv_bias_relu_zero_input_is_the_bias(dtype):
    # x = 0: every output pixel of channel k is bias[k], then max(bias[k], 0) with ReLU (W != K and C != K, so
    # a bias indexed by column q or by input channel would fail)
    N, H, W, C, K = 2, 4, 5, 8, 6
    enc = bf16_bits if dtype == "bf16" else f16_bits
    x = enc(np.zeros(N * H * W * C)).reshape(N, H, W, C)
    w = enc(RNG.standard_normal(K * 3 * 3 * C)).reshape(K, 3, 3, C)
    b = enc([-2.5, 0.75, 0.0, 3.0, -0.125, 1.5])
    bd = lib_decode(b, dtype)
    got = oracle.conv2d_fprop(x, w, pad=(1, 1), bias=b, dtype=dtype)
    assert np.array_equal(got, np.broadcast_to(bd, (N, H, W, K)))
    got = oracle.conv2d_fprop(x, w, pad=(1, 1), bias=b, act="relu", dtype=dtype)
    assert np.array_equal(got, np.broadcast_to(np.maximum(bd, 0.0), (N, H, W, K)))


def test_conv_bias_relu_delta_filter():
    # identity filter on the first K input channels: y = max(x[..., k] + bias[k], 0), exactly (integer values)
    N, H, W, C, K = 2, 5, 4, 8, 4
    x = _int_bits((N, H, W, C), -6, 7)
    w = np.zeros((K, 3, 3, C))
    for k in range(K):
        w[k, 1, 1, k] = 1.0
    b = bf16_bits([-2.0, 3.0, 0.0, -5.0])
    want = np.maximum(lib_decode(x, "bf16")[..., :K] + lib_decode(b, "bf16"), 0.0)
    got = oracle.conv2d_fprop(x, bf16_bits(w.ravel()).reshape(K, 3, 3, C), pad=(1, 1), bias=b, act="relu")
    assert np.array_equal(got, want)
    assert (got == 0).any() and (got > 0).any()


def test_conv_bias_after_alpha_beta():
    # bias is added after alpha * acc + beta * C (not scaled by alpha), ReLU after the bias
    x = bf16_bits(RNG.standard_normal(1 * 4 * 4 * 8)).reshape(1, 4, 4, 8)
    w = bf16_bits(RNG.standard_normal(3 * 3 * 3 * 8)).reshape(3, 3, 3, 8)
    c = bf16_bits(RNG.standard_normal(1 * 4 * 4 * 3)).reshape(1, 4, 4, 3)
    b = bf16_bits([0.5, -1.0, 2.0])
    base = oracle.conv2d_fprop(x, w, pad=(1, 1))
    want = 2.0 * base - 0.5 * lib_decode(c, "bf16") + lib_decode(b, "bf16")
    got = oracle.conv2d_fprop(x, w, pad=(1, 1), C_in=c, alpha=2.0, beta=-0.5, bias=b)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
    got = oracle.conv2d_fprop(x, w, pad=(1, 1), C_in=c, alpha=2.0, beta=-0.5, bias=b, act="relu")
    np.testing.assert_allclose(got, np.where(want > 0, want, 0.0), rtol=1e-14, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.conv2d_fprop(x, w, pad=(1, 1), act="gelu")


# ---------------------------------------------------------------- conv dgrad
def _int_bits(shape, lo=-3, hi=4):
    return bf16_bits(RNG.integers(lo, hi, shape).astype(np.float64))


@pytest.mark.parametrize("H,R,pad,stride,dil", [(7, 3, 1, 1, 1), (8, 3, 0, 2, 1), (9, 3, 2, 1, 2), (10, 5, 2, 3, 1),
                                                (6, 1, 0, 1, 1)])
def test_dgrad_is_the_adjoint_of_fprop(H, R, pad, stride, dil):
    # <fprop(x, w), dy> == <x, dgrad(dy, w)> for every x, dy: integer-valued operands make both sides exact
    N, C, K = 2, 5, 3
    x = _int_bits((N, H, H + 1, C))
    w = _int_bits((K, R, R, C))
    P = oracle.conv_out_size(H, R, pad, stride, dil)
    Q = oracle.conv_out_size(H + 1, R, pad, stride, dil)
    dy = _int_bits((N, P, Q, K))
    y = oracle.conv2d_fprop(x, w, pad=(pad, pad), stride=(stride, stride), dil=(dil, dil))
    dx = oracle.conv2d_dgrad(dy, w, H, H + 1, pad=(pad, pad), stride=(stride, stride), dil=(dil, dil))
    assert np.sum(y * lib_decode(dy, "bf16")) == np.sum(lib_decode(x, "bf16") * dx)


@pytest.mark.parametrize("R,pad,dil", [(3, 1, 1), (3, 0, 2), (5, 2, 1), (2, 1, 3)])
def test_dgrad_stride_one_is_fprop_with_flipped_filter(R, pad, dil):
    # textbook identity: the transposed stride-1 convolution is a convolution of dy with the filter rotated by
    # 180 degrees, its in / out channels swapped, and padding dil * (R - 1) - pad
    N, H, C, K = 2, 9, 4, 6
    w = bf16_bits(RNG.standard_normal((K, R, R, C))).reshape(K, R, R, C)
    P = oracle.conv_out_size(H, R, pad, 1, dil)
    dy = bf16_bits(RNG.standard_normal((N, P, P, K))).reshape(N, P, P, K)
    wf = np.ascontiguousarray(w[:, ::-1, ::-1, :].transpose(3, 1, 2, 0))  # [C][R][S][K], flipped taps
    pad2 = dil * (R - 1) - pad
    want = oracle.conv2d_fprop(dy, wf, pad=(pad2, pad2), dil=(dil, dil))
    got = oracle.conv2d_dgrad(dy, w, H, H, pad=(pad, pad), dil=(dil, dil))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_dgrad_beta_term_and_shape_checks():
    dy = bf16_bits(RNG.standard_normal(1 * 4 * 4 * 3)).reshape(1, 4, 4, 3)
    w = bf16_bits(RNG.standard_normal(3 * 3 * 3 * 8)).reshape(3, 3, 3, 8)
    c = bf16_bits(RNG.standard_normal(1 * 4 * 4 * 8)).reshape(1, 4, 4, 8)
    base = oracle.conv2d_dgrad(dy, w, 4, 4, pad=(1, 1))
    got = oracle.conv2d_dgrad(dy, w, 4, 4, pad=(1, 1), C_in=c, alpha=2.0, beta=-0.5)
    np.testing.assert_allclose(got, 2.0 * base - 0.5 * lib_decode(c, "bf16"), rtol=1e-14, atol=1e-14)
    with pytest.raises(AssertionError):
        oracle.conv2d_dgrad(dy, w, 5, 4, pad=(1, 1))  # dy does not have the forward output's size


# ---------------------------------------------------------------- conv wgrad
@pytest.mark.parametrize("H,R,pad,stride,dil", [(7, 3, 1, 1, 1), (8, 3, 0, 2, 1), (9, 3, 2, 1, 2), (10, 5, 2, 3, 1),
                                                (6, 1, 0, 1, 1)])
def test_wgrad_is_the_adjoint_of_fprop_in_the_filter(H, R, pad, stride, dil):
    # <fprop(x, w), dy> == <w, wgrad(x, dy)> for every w, dy: integer-valued operands make both sides exact
    N, C, K = 2, 5, 3
    x = _int_bits((N, H, H + 1, C))
    w = _int_bits((K, R, R, C))
    P = oracle.conv_out_size(H, R, pad, stride, dil)
    Q = oracle.conv_out_size(H + 1, R, pad, stride, dil)
    dy = _int_bits((N, P, Q, K))
    y = oracle.conv2d_fprop(x, w, pad=(pad, pad), stride=(stride, stride), dil=(dil, dil))
    dw = oracle.conv2d_wgrad(x, dy, R, R, pad=(pad, pad), stride=(stride, stride), dil=(dil, dil))
    assert np.sum(y * lib_decode(dy, "bf16")) == np.sum(lib_decode(w, "bf16") * dw)


def test_wgrad_1x1_is_a_gemm_over_pixels():
    # a 1x1 filter with stride 1 and no padding: dw[k][c] = sum over pixels of dy[.., k] x[.., c], i.e. dy^T x
    N, H, W, C, K = 2, 5, 6, 7, 4
    x = bf16_bits(RNG.standard_normal((N, H, W, C)))
    dy = bf16_bits(RNG.standard_normal((N, H, W, K)))
    got = oracle.conv2d_wgrad(x, dy, 1, 1)
    want = lib_decode(dy, "bf16").reshape(-1, K).T @ lib_decode(x, "bf16").reshape(-1, C)
    np.testing.assert_allclose(got.reshape(K, C), want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("G", [2, 4])
def test_grouped_wgrad_is_the_wgrad_of_each_channel_slice(G):
    # output channels of group g see only input channels g*C/G ..: the grouped result equals the plain weight
    # gradient of each group's channel slices
    N, H, C, K, R = 2, 7, 8, 12, 3
    x = bf16_bits(RNG.standard_normal((N, H, H, C)))
    dy = bf16_bits(RNG.standard_normal((N, H, H, K)))
    got = oracle.conv2d_wgrad(x, dy, R, R, pad=(1, 1), groups=G)
    assert got.shape == (K, R, R, C // G)
    cg, kg = C // G, K // G
    for g in range(G):
        part = oracle.conv2d_wgrad(np.ascontiguousarray(x[..., g * cg:(g + 1) * cg]),
                                   np.ascontiguousarray(dy[..., g * kg:(g + 1) * kg]), R, R, pad=(1, 1))
        assert np.array_equal(got[g * kg:(g + 1) * kg], part)


def test_wgrad_beta_term():
    x = bf16_bits(RNG.standard_normal((1, 4, 4, 8)))
    dy = bf16_bits(RNG.standard_normal((1, 4, 4, 3)))
    c = bf16_bits(RNG.standard_normal((3, 3, 3, 8)))
    base = oracle.conv2d_wgrad(x, dy, 3, 3, pad=(1, 1))
    got = oracle.conv2d_wgrad(x, dy, 3, 3, pad=(1, 1), C_in=c, alpha=2.0, beta=-0.5)
    np.testing.assert_allclose(got, 2.0 * base - 0.5 * lib_decode(c, "bf16"), rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- prepack
def test_golden_prepack_positions():
    N, K = 32, 256
    for n, k, off, hi in (map(int, r) for r in read_golden("prepack_positions.txt")):
        q = np.zeros((N, K), np.uint8)
        q[n, k] = 0xA
        Wp = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
        pp = oracle.prepack_w4(Wp, N, K)
        nz = np.nonzero(pp)[0]
        assert list(nz) == [off], (n, k, nz)
        assert pp[off] == (0xA0 if hi else 0x0A), (n, k, hex(pp[off]))


def test_prepack_is_a_bijection_by_position_identification():
    # pass j fills nibble (n, k) with digit j of its linear index; reading the
    # digits back from the prepacked bytes recovers every position exactly once
    N, K = 48, 384
    idx = np.arange(N * K).reshape(N, K)
    recovered = np.zeros(N * K // 2 * 2, np.int64)
    for j in range(4):  # 16^4 > N*K
        q = ((idx >> (4 * j)) & 15).astype(np.uint8)
        pp = oracle.prepack_w4((q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8), N, K)
        nibbles = np.empty(pp.size * 2, np.int64)
        nibbles[0::2] = pp & 15
        nibbles[1::2] = pp >> 4
        recovered |= nibbles << (4 * j)
    assert np.array_equal(np.sort(recovered), np.arange(N * K))


def test_prepack_round_trip_and_size():
    N, K = 64, 512
    Wp = RNG.integers(0, 256, (N, K // 2), dtype=np.uint8)
    pp = oracle.prepack_w4(Wp, N, K)
    assert pp.size == N * K // 2
    assert np.array_equal(oracle.unprepack_w4(pp, N, K), Wp)
    # the permutation moves nibbles only: the multiset of nibbles is unchanged
    cnt = lambda a: np.bincount(np.concatenate([a.ravel() & 15, a.ravel() >> 4]), minlength=16)
    assert np.array_equal(cnt(pp), cnt(Wp))


def test_prepack_word_holds_eight_consecutive_k_of_one_row():
    # each 32-bit word = 8 consecutive k of one row, interleaved even/odd
    N, K = 16, 128
    q = np.tile(np.arange(K, dtype=np.int64) % 16, (N, 1)).astype(np.uint8)
    q[:, :] = (np.arange(K) % 8)[None, :]  # element index within its run of 8
    q[3, :] = 15 - q[3, :]
    pp = oracle.prepack_w4((q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8), N, K)
    words = pp.view("<u4")
    slots = [(words >> (4 * p)) & 15 for p in range(8)]
    # slot p holds element e = 2p (p < 4) or 2(p - 4) + 1
    for p in range(8):
        e = 2 * p if p < 4 else 2 * (p - 4) + 1
        vals = slots[p]
        lanes = np.arange(words.size) // 4  # 4 words per lane
        row = lanes % 16
        assert np.all(vals[row != 3] == e)
        assert np.all(vals[row == 3] == 15 - e)


def test_prepack_rejects_unaligned_shapes():
    with pytest.raises(ValueError):
        oracle.prepack_w4(np.zeros((8, 64), np.uint8), 8, 128)
    with pytest.raises(ValueError):
        oracle.prepack_w4(np.zeros((16, 32), np.uint8), 16, 64)
