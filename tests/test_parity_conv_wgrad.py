"""GPU parity of the implicit-GEMM conv2d weight gradient against the fp64
oracle, which computes it as the adjoint of the forward convolution in the
filter."""
import numpy as np
import pytest
import torch

import gmi_inputs as gi
import oracle
from helpers import SENTINEL, check_close, dev, host_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _case(N, H, W, C, K, R, S, pad, stride, dil, dtype, seed):
    r = np.random.default_rng(seed)
    P = oracle.conv_out_size(H, R, pad, stride, dil)
    Q = oracle.conv_out_size(W, S, pad, stride, dil)
    x = gi.to_bits(r.standard_normal((N, H, W, C)).astype(np.float32), dtype)
    dy = gi.to_bits((r.standard_normal((N, P, Q, K)) / np.sqrt(N * P * Q)).astype(np.float32), dtype)
    return x, dy


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,H,W,C,K,R,S,pad,stride,dil", [
    (2, 9, 7, 32, 16, 3, 3, 1, 1, 1),
    (3, 17, 19, 16, 24, 3, 3, 1, 2, 1),     # batch not a multiple of 8: padded with zero images
    (8, 8, 8, 24, 16, 1, 1, 0, 1, 1),
    (2, 12, 10, 8, 40, 3, 3, 2, 1, 2),
    (1, 30, 30, 16, 8, 5, 5, 2, 3, 1),
    (4, 11, 13, 40, 24, 2, 3, 0, 1, 1),
    (5, 20, 16, 8, 8, 3, 3, 1, 4, 2),
])
def test_wgrad_shapes(gmi, dtype, N, H, W, C, K, R, S, pad, stride, dil):
    x, dy = _case(N, H, W, C, K, R, S, pad, stride, dil, dtype, seed=N * H + C)
    dw = gmi.conv2d_wgrad(to_dev(x, dtype), to_dev(dy, dtype), R, S, pad=(pad, pad), stride=(stride, stride),
                          dil=(dil, dil))
    torch.cuda.synchronize()
    ref = oracle.conv2d_wgrad(x, dy, R, S, pad=(pad, pad), stride=(stride, stride), dil=(dil, dil), dtype=dtype)
    check_close(host_bits(dw), ref, dtype, f"wgrad {N},{H},{W},{C},{K},{R},{S} p{pad} s{stride} d{dil}")


def test_wgrad_alpha_beta_and_guarded_output(gmi):
    N, H, W, C, K, R = 3, 10, 10, 16, 32, 3
    x, dy = _case(N, H, W, C, K, R, R, 1, 1, 1, "bf16", seed=3)
    c = gi.to_bits(np.random.default_rng(4).standard_normal((K, R, R, C)).astype(np.float32), "bf16")
    n = K * R * R * C
    flat = torch.full((n + 128,), SENTINEL, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    dw = flat[64:64 + n].view(K, R, R, C)
    gmi.conv2d_wgrad(to_dev(x, "bf16"), to_dev(dy, "bf16"), R, R, pad=(1, 1), c_in=to_dev(c, "bf16"), alpha=0.5,
                     beta=-2.0, dw=dw)
    torch.cuda.synchronize()
    guard = flat.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.all(guard[:64] == SENTINEL) and np.all(guard[-64:] == SENTINEL), "guard band written"
    ref = oracle.conv2d_wgrad(x, dy, R, R, pad=(1, 1), C_in=c, alpha=0.5, beta=-2.0)
    check_close(host_bits(dw), ref, "bf16", "wgrad alpha/beta")


def test_wgrad_integer_inputs_bit_exact(gmi):
    # small integers: every product, partial and the fixed-order sum of the partials is exact in fp32
    N, H, W, C, K = 4, 12, 9, 24, 16
    r = np.random.default_rng(5)
    x = gi.to_bits(r.integers(-2, 3, (N, H, W, C)).astype(np.float32), "bf16")
    dy = gi.to_bits(r.integers(-2, 3, (N, H, W, K)).astype(np.float32), "bf16")  # 3x3, pad 1: P = H, Q = W
    dw = gmi.conv2d_wgrad(to_dev(x, "bf16"), to_dev(dy, "bf16"), 3, 3, pad=(1, 1))
    torch.cuda.synchronize()
    ref = oracle.conv2d_wgrad(x, dy, 3, 3, pad=(1, 1))
    assert np.array_equal(host_bits(dw), oracle.round_to(ref, "bf16"))


def test_wgrad_full_size_sampled(gmi):
    # the forward workload's layer (32 x 56 x 56 x 256, 3x3x256 -> 256, pad 1) backwards: 100352 output pixels
    # reduced per filter tap; the oracle on 8 of the 256 filters (dw[k] depends only on dy[..., k])
    N, H, W, C, K = 32, 56, 56, 256, 256
    x, _ = gi.conv_fprop_bf16()
    dy = gi.to_bits((np.random.default_rng(6).standard_normal((N, H, W, K)) / 300).astype(np.float32), "bf16")
    dw = gmi.conv2d_wgrad(to_dev(x, "bf16"), to_dev(dy, "bf16"), 3, 3, pad=(1, 1))
    torch.cuda.synchronize()
    ks = [0, 37, 100, 128, 200, 201, 254, 255]
    ref = oracle.conv2d_wgrad(x, np.ascontiguousarray(dy[..., ks]), 3, 3, pad=(1, 1))
    check_close(host_bits(dw)[ks], ref, "bf16", f"wgrad full size filters {ks}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,H,W,C,K,R,pad,stride,groups", [
    (4, 12, 10, 32, 32, 3, 1, 1, 4),     # 8 channels per group in and out (the page's depthwise-like case)
    (2, 9, 9, 64, 64, 3, 1, 2, 2),
    (3, 8, 12, 16, 48, 1, 0, 1, 2),      # 8 in, 24 out per group
    (2, 14, 14, 128, 128, 3, 1, 1, 16),
])
def test_grouped_wgrad(gmi, dtype, N, H, W, C, K, R, pad, stride, groups):
    x, dy = _case(N, H, W, C, K, R, R, pad, stride, 1, dtype, seed=C + groups)
    dw = gmi.conv2d_wgrad(to_dev(x, dtype), to_dev(dy, dtype), R, R, pad=(pad, pad), stride=(stride, stride),
                          groups=groups)
    torch.cuda.synchronize()
    assert dw.shape == (K, R, R, C // groups)
    ref = oracle.conv2d_wgrad(x, dy, R, R, pad=(pad, pad), stride=(stride, stride), dtype=dtype, groups=groups)
    check_close(host_bits(dw), ref, dtype, f"grouped wgrad {N},{H},{W},{C},{K},{R} g{groups}")
