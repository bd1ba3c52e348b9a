"""GPU parity of the implicit-GEMM conv2d forward against the direct fp64
oracle."""
import numpy as np
import pytest
import torch

import gmi_inputs as gi
import oracle
from helpers import check_close, dev, host_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _run(gmi, x, w, pad, stride, dil, dtype="bf16", c=None, alpha=1.0, beta=0.0):
    y = gmi.conv2d_fprop(to_dev(x, dtype), to_dev(w, dtype), pad=pad, stride=stride, dil=dil,
                         c_in=None if c is None else to_dev(c, dtype), alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    return host_bits(y)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,H,W,C,K,R,S,pad,stride,dil", [
    (2, 9, 7, 32, 16, 3, 3, 1, 1, 1),
    (1, 17, 19, 64, 72, 3, 3, 1, 2, 1),
    (3, 8, 8, 16, 24, 1, 1, 0, 1, 1),
    (2, 12, 10, 40, 8, 3, 3, 2, 1, 2),
    (1, 30, 30, 8, 136, 5, 5, 2, 3, 1),
    (2, 11, 13, 24, 40, 2, 3, 0, 1, 1),
    (1, 6, 6, 8, 8, 3, 3, 0, 8, 1),
    (2, 10, 9, 128, 24, 3, 3, 1, 1, 1),   # several whole channel blocks per tap: channel-block-major k order
    (1, 12, 12, 96, 40, 3, 3, 1, 1, 2),
])
def test_conv_shapes(gmi, dtype, N, H, W, C, K, R, S, pad, stride, dil):
    r = np.random.default_rng(N * H + C)
    x = gi.to_bits(r.standard_normal((N, H, W, C)).astype(np.float32), dtype)
    w = gi.to_bits((r.standard_normal((K, R, S, C)) / np.sqrt(R * S * C)).astype(np.float32), dtype)
    got = _run(gmi, x, w, (pad, pad), (stride, stride), (dil, dil), dtype)
    ref = oracle.conv2d_fprop(x, w, pad=(pad, pad), stride=(stride, stride), dil=(dil, dil), dtype=dtype)
    check_close(got, ref, dtype, f"conv {N},{H},{W},{C},{K},{R},{S} p{pad} s{stride} d{dil}")


def test_conv_alpha_beta(gmi):
    r = np.random.default_rng(3)
    x = gi.to_bits(r.standard_normal((2, 10, 10, 16)).astype(np.float32), "bf16")
    w = gi.to_bits((r.standard_normal((32, 3, 3, 16)) / 12).astype(np.float32), "bf16")
    c = gi.to_bits(r.standard_normal((2, 10, 10, 32)).astype(np.float32), "bf16")
    got = _run(gmi, x, w, (1, 1), (1, 1), (1, 1), c=c, alpha=0.5, beta=-2.0)
    ref = oracle.conv2d_fprop(x, w, pad=(1, 1), C_in=c, alpha=0.5, beta=-2.0)
    check_close(got, ref, "bf16", "conv alpha/beta")


def test_conv_delta_filter_bit_exact(gmi):
    N, H, W, C = 2, 14, 9, 32
    x = gi.to_bits(np.random.default_rng(1).standard_normal((N, H, W, C)).astype(np.float32), "bf16")
    w = np.zeros((C, 3, 3, C), np.float32)
    w[np.arange(C), 1, 1, np.arange(C)] = 1.0
    got = _run(gmi, x, gi.to_bits(w, "bf16"), (1, 1), (1, 1), (1, 1))
    assert np.array_equal(got, x)


def test_conv_all_ones_borders_bit_exact(gmi):
    # the workload's geometry on one image: interior 9C, edges 6C, corners 4C
    N, H, W, C, K = 1, 56, 56, 256, 256
    ones_x = gi.to_bits(np.ones((N, H, W, C), np.float32), "bf16")
    ones_w = gi.to_bits(np.ones((K, 3, 3, C), np.float32), "bf16")
    got = oracle.decode(_run(gmi, ones_x, ones_w, (1, 1), (1, 1), (1, 1)), "bf16")
    taps = np.full((H, W), 9.0)
    taps[0, :] = taps[-1, :] = 6
    taps[:, 0] = taps[:, -1] = 6
    taps[0, 0] = taps[0, -1] = taps[-1, 0] = taps[-1, -1] = 4
    assert np.array_equal(got[0], np.repeat((taps * C)[:, :, None], K, axis=2))


def test_workload5_full_size_sampled(gmi):
    # N = 32, 56 x 56 x 256 -> 256 filters 3 x 3, pad 1: two whole images checked
    x, w = gi.conv_fprop_bf16()
    got = _run(gmi, x, w, (1, 1), (1, 1), (1, 1))
    for n in (0, 31):
        ref = oracle.conv2d_fprop(x[n:n + 1], w, pad=(1, 1))
        check_close(got[n:n + 1], ref, "bf16", f"workload 5 image {n}")
