"""GPU parity of the implicit-GEMM conv2d data gradient against the fp64
oracle, which computes it as the adjoint of the forward convolution.  A
stride above 1 runs by output phase (the rows h with h + pad in
one residue class of the stride, crossed with the columns' classes), each
gathering only the filter taps that reach that phase; the strided cases cover
unequal and odd strides, filters narrower than the stride, and dilations that
share a factor with the stride, which leave whole phases without a tap.
Up to 16 phases (strides up to 4 x 4) run as one launch, more as a launch
per phase; the cases cover both."""
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


def _case(N, H, W, C, K, R, S, pad, dil, dtype, seed, stride=1, stride_w=None, pad_w=None, dil_w=None):
    r = np.random.default_rng(seed)
    P = oracle.conv_out_size(H, R, pad, stride, dil)
    Q = oracle.conv_out_size(W, S, pad if pad_w is None else pad_w, stride if stride_w is None else stride_w,
                             dil if dil_w is None else dil_w)
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


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,H,W,C,K,R,S,ph,pw,sh,sw,dh,dw", [
    (2, 11, 10, 16, 24, 3, 3, 1, 1, 2, 3, 1, 1),   # unequal strides: 2 x 3 phases
    (1, 13, 9, 24, 16, 3, 2, 1, 0, 3, 1, 1, 1),    # stride 3 in rows only
    (1, 10, 15, 8, 32, 2, 5, 0, 2, 1, 2, 1, 1),    # stride 2 in columns only
    (2, 12, 12, 16, 16, 2, 2, 0, 0, 3, 3, 1, 1),   # a 2x2 filter at stride 3: a third of the phases have no tap
    (1, 15, 14, 8, 16, 3, 3, 3, 3, 3, 3, 3, 3),    # dilation 3 at stride 3: only one phase per dimension has taps
    (1, 16, 16, 16, 8, 5, 3, 2, 1, 4, 6, 2, 2),    # dilation sharing a factor with strides 4 and 6
    (1, 23, 19, 8, 16, 7, 5, 3, 2, 7, 5, 1, 1),    # strides 7 and 5: one tap per phase
    (1, 20, 17, 32, 8, 3, 3, 1, 1, 8, 8, 1, 1),
])
def test_dgrad_strided_phases(gmi, dtype, N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw):
    dy, w = _case(N, H, W, C, K, R, S, ph, dh, dtype, seed=H * W + sh * 10 + sw, stride=sh, stride_w=sw, pad_w=pw,
                  dil_w=dw)
    dx = gmi.conv2d_dgrad(to_dev(dy, dtype), to_dev(w, dtype), H, W, pad=(ph, pw), dil=(dh, dw), stride=(sh, sw))
    torch.cuda.synchronize()
    ref = oracle.conv2d_dgrad(dy, w, H, W, pad=(ph, pw), stride=(sh, sw), dil=(dh, dw), dtype=dtype)
    check_close(host_bits(dx), ref, dtype, f"dgrad {N},{H},{W},{C},{K},{R},{S} p{ph},{pw} s{sh},{sw} d{dh},{dw}")


def test_dgrad_strided_beta_guarded_and_tapless_phases(gmi):
    # stride 2 with dilation 2: the odd rows and columns receive no tap, so there dx = RN(beta * C) exactly; the
    # phases write through their strided row map inside a guard band
    N, H, W, C, K, R, S = 2, 14, 13, 16, 24, 3, 3
    dy, w = _case(N, H, W, C, K, R, S, 2, 2, "bf16", seed=31, stride=2)
    c = gi.to_bits(np.random.default_rng(32).standard_normal((N, H, W, C)).astype(np.float32), "bf16")
    flat = torch.full((N * H * W * C + 128,), SENTINEL, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    dx = flat[64:64 + N * H * W * C].view(N, H, W, C)
    gmi.conv2d_dgrad(to_dev(dy, "bf16"), to_dev(w, "bf16"), H, W, pad=(2, 2), dil=(2, 2), stride=(2, 2),
                     c_in=to_dev(c, "bf16"), alpha=0.75, beta=-0.5, dx=dx)
    torch.cuda.synchronize()
    guard = flat.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.all(guard[:64] == SENTINEL) and np.all(guard[-64:] == SENTINEL), "guard band written"
    got = host_bits(dx)
    ref = oracle.conv2d_dgrad(dy, w, H, W, pad=(2, 2), stride=(2, 2), dil=(2, 2), C_in=c, alpha=0.75, beta=-0.5)
    check_close(got, ref, "bf16", "strided dgrad alpha/beta")
    # rows h with h + 2 odd (odd h) have no tap: exactly the rounded beta * C
    tapless = got[:, 1::2, :, :]
    assert np.array_equal(tapless, oracle.round_to(-0.5 * oracle.decode(c, "bf16")[:, 1::2], "bf16"))


def test_dgrad_strided_integer_inputs_bit_exact(gmi):
    # small integers: exact fp32 sums, so each phase's result is the RNE of the exact value
    N, H, W, C, K, R, S = 2, 15, 11, 24, 16, 3, 4
    r = np.random.default_rng(33)
    P = oracle.conv_out_size(H, R, 1, 3, 1)
    Q = oracle.conv_out_size(W, S, 2, 2, 1)
    dy = gi.to_bits(r.integers(-3, 4, (N, P, Q, K)).astype(np.float32), "bf16")
    w = gi.to_bits(r.integers(-2, 3, (K, R, S, C)).astype(np.float32), "bf16")
    dx = gmi.conv2d_dgrad(to_dev(dy, "bf16"), to_dev(w, "bf16"), H, W, pad=(1, 2), stride=(3, 2))
    torch.cuda.synchronize()
    ref = oracle.conv2d_dgrad(dy, w, H, W, pad=(1, 2), stride=(3, 2))
    assert np.array_equal(host_bits(dx), oracle.round_to(ref, "bf16"))


def test_dgrad_strided_full_size_sampled(gmi):
    # the workload layer at stride 2 (dy 32 x 28 x 28 x 256) backwards to 56 x 56 x 256; the oracle on 3 images
    N, H, W, C, K = 32, 56, 56, 256, 256
    x, w = gi.conv_fprop_bf16()
    r = np.random.default_rng(34)
    dy = gi.to_bits(r.standard_normal((N, 28, 28, K)).astype(np.float32), "bf16")
    dx = gmi.conv2d_dgrad(to_dev(dy, "bf16"), to_dev(w, "bf16"), H, W, pad=(1, 1), stride=(2, 2))
    torch.cuda.synchronize()
    pick = [0, 17, 31]
    ref = oracle.conv2d_dgrad(dy[pick], w, H, W, pad=(1, 1), stride=(2, 2))
    check_close(host_bits(dx)[pick], ref, "bf16", f"strided dgrad full size images {pick}")
