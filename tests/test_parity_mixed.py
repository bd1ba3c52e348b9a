"""GPU parity of the mixed-input GEMM in every conversion mode (direct, scale,
scale with zero point), for uint4 and int4 weights and fp16 and bf16
activations, against the fp64 oracle.  The decode (M <= 32: one or two 16-row
tiles), skinny (M <= 64) and tiled (larger M, also split over K) kernels are
each covered.

Tolerance: |d - ref| <= 1e-2 |ref| + 1e-2.  With bf16 activations the skinny
and tiled kernels round every dequantised weight to bf16 before the multiply
(as the page's bf16 conversion does), an error of up to half a bf16 ulp,
2^-9 |w|, per weight; that adds at most 2^-9 sum_k |x_k w_k| to an output, and
their bf16 bar adds twice that bound.  The decode kernel feeds the matrix
instruction exact integer weights, so its results (M <= 32) keep the plain
bar."""
import numpy as np
import pytest
import torch

import gmi_inputs as gi
import oracle
from helpers import Guarded, bytes_to_dev, check_close, dev, to_dev

pytestmark = pytest.mark.gpu

MODES = ["direct", "scale", "zero"]


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _case(M, N, K, group, dtype, seed):
    r = np.random.default_rng(seed)
    W = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
    Z = r.integers(0, 256, (K // group, N // 2), dtype=np.uint8)
    S = gi.to_bits(r.uniform(0.001, 0.01, (K // group, N)).astype(np.float32), dtype)
    X = gi.to_bits(r.standard_normal((M, K)).astype(np.float32), dtype)
    return X, W, S, Z


DECODE_ROWS = 32  # calls of at most this many rows run the exact-integer decode kernel


def _check(got, ref, X, W, S, Z, N, K, group, dtype, w_type, mode, what):
    if dtype == "f16" or X.shape[0] <= DECODE_ROWS:
        check_close(got, ref, dtype, what)
        return
    w = oracle.dequant_mixed(W, S if mode != "direct" else None, Z if mode == "zero" else None, N, K, group, w_type,
                             dtype)
    mag = np.abs(oracle.decode(X, dtype)[:, :K]) @ np.abs(w).T
    d = oracle.decode(got, dtype)
    bad = ~(np.abs(d - ref) <= 1e-2 * np.abs(ref) + 1e-2 + 2.0**-8 * mag)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; {i}: got {d[i]:.6g} "
                             f"want {ref[i]:.6g} bound term {2.0**-8 * mag[i]:.3g}")


def _run(gmi, X, W, S, Z, M, N, K, group, dtype, w_type, mode, workspace=None, ldy_pad=8):
    wpp = gmi.prepack_w4(bytes_to_dev(W), N, K)
    s_dev = to_dev(S, dtype) if mode != "direct" else None
    z_dev = bytes_to_dev(Z) if mode == "zero" else None
    out = Guarded(M, N, N + ldy_pad, dtype)
    gmi.gemm_mixed(to_dev(X, dtype), wpp, s_dev, z_dev, group, N, w_type=w_type, Y=out.view, workspace=workspace)
    torch.cuda.synchronize()
    out.check_guards(f"mixed {dtype} {w_type} {mode} M={M}")
    ref = oracle.mixed(X, W, S if mode != "direct" else None, Z if mode == "zero" else None, N, K, group, w_type,
                       dtype)
    return out.bits(), ref


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("w_type", ["uint4", "int4"])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M", [1, 16, 24, 40, 200])
def test_mixed_modes(gmi, dtype, w_type, mode, M):
    N, K, group = 256, 1024, 128
    X, W, S, Z = _case(M, N, K, group, dtype, seed=M * 7 + len(mode))
    got, ref = _run(gmi, X, W, S, Z, M, N, K, group, dtype, w_type, mode)
    _check(got, ref, X, W, S, Z, N, K, group, dtype, w_type, mode, f"mixed {dtype} {w_type} {mode} M={M}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mixed_per_channel_int4_and_group_256(gmi, dtype):
    # group == K (one scale per output channel) and a group spanning two 128-k blocks
    for group, M in ((1024, 8), (1024, 30), (1024, 96), (256, 20), (256, 33)):
        X, W, S, Z = _case(M, 128, 1024, group, dtype, seed=group + M)
        got, ref = _run(gmi, X, W, S, Z, M, 128, 1024, group, dtype, "int4", "zero")
        _check(got, ref, X, W, S, Z, 128, 1024, group, dtype, "int4", "zero",
               f"mixed {dtype} int4 group {group} M={M}")


def test_mixed_bf16_split_k(gmi):
    # M = 128 over N = 2048: 16 output tiles, so K splits (fp32 partials, then the summing launch)
    M, N, K, group = 128, 2048, 4096, 128
    assert gmi.w4a16_workspace_bytes(M, N, K) > 0
    X, W, S, Z = _case(M, N, K, group, "bf16", seed=21)
    ws = torch.empty(gmi.w4a16_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev())
    got, ref = _run(gmi, X, W, S, Z, M, N, K, group, "bf16", "int4", "scale", workspace=ws)
    _check(got, ref, X, W, S, Z, N, K, group, "bf16", "int4", "scale", "mixed bf16 split-K")


def test_mixed_f16_uint4_zero_mode_is_w4a16_bit_for_bit(gmi):
    # gmi_gemm_w4a16 is the fp16 / uint4 / zero-point case of gmi_gemm_mixed
    for M in (8, 48, 160):
        X, W, S, Z = _case(M, 256, 512, 128, "f16", seed=M)
        wpp = gmi.prepack_w4(bytes_to_dev(W), 256, 512)
        args = (to_dev(X, "f16"), wpp, to_dev(S, "f16"), bytes_to_dev(Z), 128, 256)
        a = gmi.gemm_w4a16(*args)
        b = gmi.gemm_mixed(*args, w_type="uint4")
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), M


@pytest.mark.parametrize("M", [16, 128])
def test_mixed_bf16_full_size_sampled(gmi, M):
    # N = K = 8192, group 128, int4 with zero points: the decode kernel (M = 16) and the split tiled path
    # (M = 128); the oracle on 24 sampled output columns
    N, K, group = 8192, 8192, 128
    X, W, S, Z = _case(M, N, K, group, "bf16", seed=M + 5)
    wpp = gmi.prepack_w4(bytes_to_dev(W), N, K)
    Y = gmi.gemm_mixed(to_dev(X, "bf16"), wpp, to_dev(S, "bf16"), bytes_to_dev(Z), group, N, w_type="int4")
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(M).choice(N, 24, replace=False))
    got = Y.cpu().view(torch.int16).numpy().view(np.uint16)[:, cols]
    # the oracle on the sampled weight rows only (rows n of W, columns n of the scales and zeros)
    Ws = W[cols]
    Ss = S[:, cols]
    zn = np.empty((K // group, N), np.uint8)
    zn[:, 0::2] = Z & 15
    zn[:, 1::2] = Z >> 4
    zs = zn[:, cols]
    Zs = (zs[:, 0::2] | (zs[:, 1::2] << 4)).astype(np.uint8)
    ref = oracle.mixed(X, Ws, Ss, Zs, len(cols), K, group, "int4", "bf16")
    _check(got, ref, X, Ws, Ss, Zs, len(cols), K, group, "bf16", "int4", "zero", f"mixed bf16 8192^2 M={M}")


# Outputs that fall exactly on, just above and just below the midpoint of two representable values: the
# stored result must be the oracle's round-to-nearest-even of the exact value, bit for bit.
_TIES = {"f16": [3 * 2.0**-11, 2.0**-11, 2.0**-11 + 2.0**-16, 3 * 2.0**-11 - 2.0**-16],
         "bf16": [3 * 2.0**-8, 2.0**-8, 2.0**-8 + 2.0**-14, 3 * 2.0**-8 - 2.0**-14]}


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [4, 20, 100])
def test_mixed_output_rounding_is_nearest_even(gmi, dtype, M):
    # direct conversion, uint4 weights 1 at k = 0, 1 and 0 elsewhere, X row [1, t, 0, ...]: y = 1 + t exactly
    N, K = 32, 128
    t = np.resize(np.array(_TIES[dtype]), M)
    xv = np.zeros((M, K), np.float64)
    xv[:, 0], xv[:, 1] = 1.0, t
    X = gi.to_bits(xv.astype(np.float32), dtype)
    assert np.array_equal(oracle.decode(X, dtype), xv)  # every input is representable
    W = np.zeros((N, K // 2), np.uint8)
    W[:, 0] = 0x11
    got, ref = _run(gmi, X, W, None, None, M, N, K, 128, dtype, "uint4", "direct")
    assert np.array_equal(ref, np.repeat((1.0 + t)[:, None], N, axis=1))
    assert np.array_equal(got, oracle.round_to(ref, dtype)), dtype
