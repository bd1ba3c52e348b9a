"""GPU parity of the implicit-GEMM conv2d data gradient against the fp64
oracle, which computes it as the adjoint of the forward convolution."""
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


def _case(N, H, W, C, K, R, S, pad, dil, dtype, seed, stride=1):
    r = np.random.default_rng(seed)
    P = oracle.conv_out_size(H, R, pad, stride, dil)
    Q = oracle.conv_out_size(W, S, pad, stride, dil)
    dy = gi.to_bits(r.standard_normal((N, P, Q, K)).astype(np.float32), dtype)
    w = gi.to_bits((r.standard_normal((K, R, S, C)) / np.sqrt(R * S * K)).astype(np.float32), dtype)
    return dy, w


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,H,W,C,K,R,S,pad,dil", [
    (2, 9, 7, 32, 16, 3, 3, 1, 1),
    (1, 17, 19, 72, 64, 3, 3, 1, 1),
    (3, 8, 8, 24, 16, 1, 1, 0, 1),
    (2, 12, 10, 8, 40, 3, 3, 2, 2),
    (1, 30, 30, 136, 8, 5, 5, 2, 1),
    (2, 11, 13, 40, 24, 2, 3, 0, 1),
    (1, 6, 6, 8, 8, 3, 3, 0, 1),
    (2, 10, 9, 24, 128, 3, 3, 1, 1),     # the gather runs over dy's 128 channels: several channel blocks per tap
])
def test_dgrad_shapes(gmi, dtype, N, H, W, C, K, R, S, pad, dil):
    dy, w = _case(N, H, W, C, K, R, S, pad, dil, dtype, seed=N * H + C)
    dx = gmi.conv2d_dgrad(to_dev(dy, dtype), to_dev(w, dtype), H, W, pad=(pad, pad), dil=(dil, dil))
    torch.cuda.synchronize()
    ref = oracle.conv2d_dgrad(dy, w, H, W, pad=(pad, pad), dil=(dil, dil), dtype=dtype)
    check_close(host_bits(dx), ref, dtype, f"dgrad {N},{H},{W},{C},{K},{R},{S} p{pad} d{dil}")


def test_dgrad_alpha_beta_and_guarded_output(gmi):
    N, H, W, C, K = 2, 10, 10, 16, 32
    dy, w = _case(N, H, W, C, K, 3, 3, 1, 1, "bf16", seed=3)
    c = gi.to_bits(np.random.default_rng(4).standard_normal((N, H, W, C)).astype(np.float32), "bf16")
    flat = torch.full((N * H * W * C + 128,), SENTINEL, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    dx = flat[64:64 + N * H * W * C].view(N, H, W, C)
    gmi.conv2d_dgrad(to_dev(dy, "bf16"), to_dev(w, "bf16"), H, W, pad=(1, 1), c_in=to_dev(c, "bf16"), alpha=0.5,
                     beta=-2.0, dx=dx)
    torch.cuda.synchronize()
    guard = flat.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.all(guard[:64] == SENTINEL) and np.all(guard[-64:] == SENTINEL), "guard band written"
    ref = oracle.conv2d_dgrad(dy, w, H, W, pad=(1, 1), C_in=c, alpha=0.5, beta=-2.0)
    check_close(host_bits(dx), ref, "bf16", "dgrad alpha/beta")


def test_dgrad_integer_inputs_bit_exact(gmi):
    # small integers: every product and partial sum is exact in fp32, so the result is the RNE of the exact value
    N, H, W, C, K = 2, 12, 9, 24, 16
    r = np.random.default_rng(5)
    P, Q = H, W  # 3x3, pad 1
    dy = gi.to_bits(r.integers(-3, 4, (N, P, Q, K)).astype(np.float32), "bf16")
    w = gi.to_bits(r.integers(-2, 3, (K, 3, 3, C)).astype(np.float32), "bf16")
    dx = gmi.conv2d_dgrad(to_dev(dy, "bf16"), to_dev(w, "bf16"), H, W, pad=(1, 1))
    torch.cuda.synchronize()
    ref = oracle.conv2d_dgrad(dy, w, H, W, pad=(1, 1))
    assert np.array_equal(host_bits(dx), oracle.round_to(ref, "bf16"))


def test_dgrad_full_size_sampled(gmi):
    # the forward workload's shape (32 x 56 x 56 x 256, 3x3x256 -> 256, pad 1) backwards; the oracle on 4 of 32
    # images (the adjoint sum never mixes images)
    N, H, W, C, K = 32, 56, 56, 256, 256
    x, w = gi.conv_fprop_bf16()
    r = np.random.default_rng(6)
    dy = gi.to_bits(r.standard_normal((N, H, W, K)).astype(np.float32), "bf16")
    dx = gmi.conv2d_dgrad(to_dev(dy, "bf16"), to_dev(w, "bf16"), H, W, pad=(1, 1))
    torch.cuda.synchronize()
    pick = [0, 9, 22, 31]
    ref = oracle.conv2d_dgrad(dy[pick], w, H, W, pad=(1, 1))
    check_close(host_bits(dx)[pick], ref, "bf16", f"dgrad full size images {pick}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,H,W,C,K,R,S,pad,stride,dil", [
    (2, 9, 9, 16, 24, 3, 3, 1, 2, 1),     # odd size: the last input row takes fewer taps
    (1, 16, 12, 32, 16, 3, 3, 1, 2, 1),
    (2, 13, 11, 8, 40, 3, 3, 2, 2, 2),
    (1, 17, 17, 24, 8, 5, 5, 2, 4, 1),
    (1, 8, 8, 8, 16, 1, 1, 0, 2, 1),      # 1x1, stride 2: every other input pixel gets no gradient
    (1, 30, 20, 16, 16, 3, 3, 0, 8, 1),
])
def test_dgrad_strided(gmi, dtype, N, H, W, C, K, R, S, pad, stride, dil):
    dy, w = _case(N, H, W, C, K, R, S, pad, dil, dtype, seed=N * H + C + stride, stride=stride)
    dx = gmi.conv2d_dgrad(to_dev(dy, dtype), to_dev(w, dtype), H, W, pad=(pad, pad), dil=(dil, dil),
                          stride=(stride, stride))
    torch.cuda.synchronize()
    ref = oracle.conv2d_dgrad(dy, w, H, W, pad=(pad, pad), stride=(stride, stride), dil=(dil, dil), dtype=dtype)
    check_close(host_bits(dx), ref, dtype, f"dgrad {N},{H},{W},{C},{K},{R},{S} p{pad} s{stride} d{dil}")
