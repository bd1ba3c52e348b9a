"""GPU parity of the mixed-input GEMM in every conversion mode (direct, scale,
scale with zero point), for uint4 and int4 weights and fp16 and bf16
activations, against the fp64 oracle.  The decode (M <= 48: one to three 16-row
tiles), skinny (M <= 64) and tiled (larger M, also split over K) kernels are
each covered.

Tolerance: |d - ref| <= 1e-2 |ref| + 1e-2 for every kernel and type.  With
bf16 activations every kernel feeds the matrix instruction exact integer
weights (rounding each dequantised weight to bf16 instead, as the page's bf16
conversion does, costs up to 2^-9 |w| per weight, which over K = 8192 terms
reaches this bar) and applies the group scales to fp32 partial sums."""
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


def _check(got, ref, dtype, what):
    check_close(got, ref, dtype, what)


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
    _check(got, ref, dtype, f"mixed {dtype} {w_type} {mode} M={M}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mixed_per_channel_int4_and_group_256(gmi, dtype):
    # group == K (one scale per output channel) and a group spanning two 128-k blocks
    for group, M in ((1024, 8), (1024, 30), (1024, 96), (256, 20), (256, 33)):
        X, W, S, Z = _case(M, 128, 1024, group, dtype, seed=group + M)
        got, ref = _run(gmi, X, W, S, Z, M, 128, 1024, group, dtype, "int4", "zero")
        _check(got, ref, dtype, f"mixed {dtype} int4 group {group} M={M}")


def test_mixed_bf16_split_k(gmi):
    # M = 128 over N = 2048: 16 output tiles, so K splits (fp32 partials, then the summing launch)
    M, N, K, group = 128, 2048, 4096, 128
    assert gmi.w4a16_workspace_bytes(M, N, K) > 0
    X, W, S, Z = _case(M, N, K, group, "bf16", seed=21)
    ws = torch.empty(gmi.w4a16_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev())
    got, ref = _run(gmi, X, W, S, Z, M, N, K, group, "bf16", "int4", "scale", workspace=ws)
    _check(got, ref, "bf16", "mixed bf16 split-K")


def test_mixed_split_ranges_per_type_and_short_workspace(gmi):
    # M = 160, N = 256, K = 4096: four output tiles.  bf16 splits K into eight k-ranges, fp16 into four, and
    # the workspace size covers the larger; a bf16 call given only what fp16 needs runs unsplit.  Every
    # variant meets the oracle on every output.
    M, N, K, group = 160, 256, 4096, 128
    tile = 128 * 128 * 4
    assert gmi.w4a16_workspace_bytes(M, N, K) == 8 * 4 * tile
    for dtype, sizes in (("bf16", (8 * 4 * tile, 4 * 4 * tile, 0)), ("f16", (8 * 4 * tile, 4 * 4 * tile))):
        X, W, S, Z = _case(M, N, K, group, dtype, seed=31 + len(dtype))
        for nbytes in sizes:
            ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=dev())
            got, ref = _run(gmi, X, W, S, Z, M, N, K, group, dtype, "int4", "zero", workspace=ws)
            _check(got, ref, dtype, f"mixed {dtype} workspace {nbytes} bytes")


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


@pytest.mark.parametrize("M", [16, 48, 128, 1024])
def test_mixed_bf16_full_size_sampled(gmi, M):
    # N = K = 8192, group 128, int4 with zero points: the decode kernel (M = 16; M = 48 as three 16-row tiles),
    # the tiled path split over K into fp32 partials (M = 128: 64 output tiles) and unsplit (M = 1024); the
    # oracle on 24 sampled output columns.  Over K = 8192 terms, weights rounded to bf16 would miss the bar on
    # some outputs of this size; the exact integer weights do not.
    N, K, group = 8192, 8192, 128
    X, W, S, Z = _case(M, N, K, group, "bf16", seed=M + 5)
    wpp = gmi.prepack_w4(bytes_to_dev(W), N, K)
    need = gmi.w4a16_workspace_bytes(M, N, K)
    assert (need > 0) == (M == 128)
    ws = torch.empty(need, dtype=torch.uint8, device=dev()) if need else None
    Y = gmi.gemm_mixed(to_dev(X, "bf16"), wpp, to_dev(S, "bf16"), bytes_to_dev(Z), group, N, w_type="int4",
                       workspace=ws)
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
    _check(got, ref, "bf16", f"mixed bf16 8192^2 M={M}")


def test_mixed_bf16_long_k_near_zero_outputs(gmi):
    # the outputs most sensitive to per-weight rounding are those whose exact value is near zero: at K = 8192
    # the bar there is the absolute 1e-2, against a rounding noise of about 3e-3 per output had each weight
    # been rounded to bf16; 128 rows x 256 columns through the split tiled path, every output checked
    M, N, K, group = 128, 256, 8192, 128
    X, W, S, Z = _case(M, N, K, group, "bf16", seed=77)
    ws = torch.empty(gmi.w4a16_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev())
    got, ref = _run(gmi, X, W, S, Z, M, N, K, group, "bf16", "int4", "zero", workspace=ws)
    assert (np.abs(ref) < 1e-2).sum() > 50
    # the case has the power to tell: weights rounded once to bf16 (on the CPU, through the oracle's dequant)
    # would put outputs outside the bar
    w = oracle.dequant_mixed(W, S, Z, N, K, group, "int4", "bf16")
    rounded = oracle.decode(X, "bf16") @ oracle.decode(oracle.round_to(w, "bf16"), "bf16").T
    d = oracle.decode(oracle.round_to(rounded, "bf16"), "bf16")
    assert (~(np.abs(d - ref) <= 1e-2 * np.abs(ref) + 1e-2)).sum() > 20
    _check(got, ref, "bf16", "mixed bf16 K=8192 every output")


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
