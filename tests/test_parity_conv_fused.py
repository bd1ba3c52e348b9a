"""GPU parity of the conv2d forward pass with the fused epilogue (bias per
output channel after alpha * acc + beta * C, then ReLU) against the fp64
oracle."""
import numpy as np
import pytest
import torch

import gmi_inputs as gi
import oracle
from helpers import check_close, host_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _run(gmi, x, w, bias, act, pad=(1, 1), stride=(1, 1), dil=(1, 1), dtype="bf16", c=None, alpha=1.0, beta=0.0):
    y = gmi.conv2d_fprop(to_dev(x, dtype), to_dev(w, dtype), pad=pad, stride=stride, dil=dil,
                         c_in=None if c is None else to_dev(c, dtype), alpha=alpha, beta=beta,
                         bias=None if bias is None else to_dev(bias, dtype), act=act)
    torch.cuda.synchronize()
    return host_bits(y)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("act", ["relu", None])
@pytest.mark.parametrize("N,H,W,C,K,R,S,pad,stride,dil", [
    (2, 9, 7, 32, 16, 3, 3, 1, 1, 1),      # K below one tile: the element-wise store path
    (1, 17, 19, 64, 72, 3, 3, 1, 2, 1),    # ragged N tail of a 64-column tile run
    (2, 12, 10, 40, 8, 3, 3, 2, 1, 2),
    (2, 10, 9, 128, 264, 3, 3, 1, 1, 1),   # several N tiles, ragged last one
])
def test_conv_bias_act_shapes(gmi, dtype, act, N, H, W, C, K, R, S, pad, stride, dil):
    r = np.random.default_rng(N * H + C + K)
    x = gi.to_bits(r.standard_normal((N, H, W, C)).astype(np.float32), dtype)
    w = gi.to_bits((r.standard_normal((K, R, S, C)) / np.sqrt(R * S * C)).astype(np.float32), dtype)
    b = gi.conv_bias(seed=K, K=K, dtype=dtype)
    got = _run(gmi, x, w, b, act, (pad, pad), (stride, stride), (dil, dil), dtype)
    ref = oracle.conv2d_fprop(x, w, pad=(pad, pad), stride=(stride, stride), dil=(dil, dil), dtype=dtype, bias=b,
                              act=act)
    check_close(got, ref, dtype, f"fused conv {N},{H},{W},{C},{K} {act}")
    if act == "relu":
        g = oracle.decode(got, dtype)
        assert (g >= 0).all() and (g == 0).mean() > 0.2 and (g > 0).mean() > 0.2


def test_conv_relu_without_bias_and_with_beta(gmi):
    r = np.random.default_rng(3)
    x = gi.to_bits(r.standard_normal((2, 10, 10, 16)).astype(np.float32), "bf16")
    w = gi.to_bits((r.standard_normal((32, 3, 3, 16)) / 12).astype(np.float32), "bf16")
    c = gi.to_bits(r.standard_normal((2, 10, 10, 32)).astype(np.float32), "bf16")
    b = gi.conv_bias(seed=9, K=32)
    got = _run(gmi, x, w, None, "relu", c=c, alpha=0.5, beta=-2.0)
    check_close(got, oracle.conv2d_fprop(x, w, pad=(1, 1), C_in=c, alpha=0.5, beta=-2.0, act="relu"), "bf16",
                "relu, no bias, beta")
    got = _run(gmi, x, w, b, "relu", c=c, alpha=0.5, beta=-2.0)
    check_close(got, oracle.conv2d_fprop(x, w, pad=(1, 1), C_in=c, alpha=0.5, beta=-2.0, bias=b, act="relu"),
                "bf16", "relu, bias, beta")


@pytest.mark.parametrize("K", [32, 20 * 8])
def test_conv_bias_relu_identity_filter_bit_exact(gmi, K):
    # identity filter on the first K of C channels, integer x and bias: v = x[..., k] + bias[k] is exact in fp32,
    # so y == RN(max(v, 0)) bit for bit
    N, H, W, C = 2, 14, 9, 256
    r = np.random.default_rng(K)
    x = gi.to_bits(r.integers(-20, 21, (N, H, W, C)).astype(np.float32), "bf16")
    w = np.zeros((K, 3, 3, C), np.float32)
    w[np.arange(K), 1, 1, np.arange(K)] = 1.0
    b = gi.to_bits(r.integers(-8, 9, K).astype(np.float32), "bf16")
    got = _run(gmi, x, gi.to_bits(w, "bf16"), b, "relu")
    ref = oracle.conv2d_fprop(x, gi.to_bits(w, "bf16"), pad=(1, 1), bias=b, act="relu")
    assert np.array_equal(got, oracle.round_to(ref, "bf16"))


def test_fused_entry_without_epilogue_matches_plain_bit_for_bit(gmi):
    r = np.random.default_rng(5)
    x = gi.to_bits(r.standard_normal((2, 9, 11, 64)).astype(np.float32), "bf16")
    w = gi.to_bits((r.standard_normal((48, 3, 3, 64)) / 24).astype(np.float32), "bf16")
    plain = _run(gmi, x, w, None, None)
    L = gmi.lib()
    xd, wd = to_dev(x, "bf16"), to_dev(w, "bf16")
    y = torch.empty((2, 9, 11, 48), dtype=torch.bfloat16, device=xd.device)
    assert L.gmi_conv2d_fprop_implicit_fused(2, 9, 11, 64, 48, 3, 3, 1, 1, 1, 1, 1, 1, xd.data_ptr(), wd.data_ptr(),
                                             None, None, y.data_ptr(), gmi.GMI_BF16, 1.0, 0.0, 0,
                                             torch.cuda.current_stream().cuda_stream) == gmi.GMI_OK
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), plain)


def test_workload5_bias_relu_full_size_sampled(gmi):
    # N = 32, 56 x 56 x 256 -> 256 filters 3 x 3, pad 1, bias and ReLU fused: two whole images checked
    x, w = gi.conv_fprop_bf16()
    b = gi.conv_bias()
    got = _run(gmi, x, w, b, "relu")
    for n in (0, 31):
        ref = oracle.conv2d_fprop(x[n:n + 1], w, pad=(1, 1), bias=b, act="relu")
        check_close(got[n:n + 1], ref, "bf16", f"workload 5 bias + ReLU, image {n}")
