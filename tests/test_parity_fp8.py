"""GPU parity of the fp8 (OCP E4M3) grouped and pointer-array GEMMs, bf16
results, against the fp64 oracle on the decoded inputs.  Tolerance: the
fp8 bar of 3e-2 relative plus 1e-2 absolute."""
import numpy as np
import pytest
import torch

import gmi_inputs as gi
import oracle
from helpers import Guarded, check_close, dev, to_dev

pytestmark = pytest.mark.gpu
RTOL8 = 3e-2


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _codes(r, shape, scale=1.0):
    return gi.to_bits((r.standard_normal(shape) * scale).astype(np.float32), "f8e4m3")


def _ptr_run(gmi, A, B, M, N, K, lda, ldb, ldd, C=None, alpha=1.0, beta=0.0):
    L = len(A)
    Ad = [to_dev(a, "f8e4m3") for a in A]
    Bd = [to_dev(b, "f8e4m3") for b in B]
    Cd = [to_dev(c, "bf16") for c in C] if C is not None else None
    outs = [Guarded(M, N, ldd, "bf16") for _ in range(L)]
    pa, pb, pd = (gmi.pointer_array(x, dev()) for x in (Ad, Bd, [o.view for o in outs]))
    pc = gmi.pointer_array(Cd, dev()) if Cd is not None else None
    gmi.gemm_ptr_array(L, M, N, K, pa, lda, pb, ldb, pc, ldd, pd, ldd, gmi.GMI_F8E4M3, alpha, beta)
    torch.cuda.synchronize()
    for o in outs:
        o.check_guards(f"fp8 ptr-array {M}x{N}x{K}")
    return [o.bits() for o in outs]


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (33, 47, 48), (130, 300, 272), (257, 129, 512)])
def test_fp8_ptr_array_shapes(gmi, M, N, K):
    r = np.random.default_rng(M + N + K)
    lda = ldb = K + 16
    ldd = (N + 7) // 8 * 8 + 8
    A = [_codes(r, (M, lda)) for _ in range(2)]
    B = [_codes(r, (N, ldb)) for _ in range(2)]
    C = [gi.to_bits(r.standard_normal((M, ldd)).astype(np.float32), "bf16") for _ in range(2)]
    got = _ptr_run(gmi, A, B, M, N, K, lda, ldb, ldd, C=C, alpha=0.75, beta=-0.5)
    for l in range(2):
        ref = oracle.gemm(A[l], B[l], C[l][:, :N], K=K, alpha=0.75, beta=-0.5, dtype="f8e4m3")
        check_close(got[l], ref, "bf16", f"fp8 {M}x{N}x{K} batch {l}", rtol=RTOL8)


def test_fp8_integer_inputs_bit_exact(gmi):
    # A, B in {-2, ..., 2} (exact in E4M3), K = 64: every sum is an integer of magnitude <= 256, exact in fp32 and
    # in bf16, so D == RN_bf16(ref) bit for bit whatever the summation order
    r = np.random.default_rng(5)
    M, N, K = 96, 160, 64
    A = [gi.to_bits(r.integers(-2, 3, (M, K)).astype(np.float32), "f8e4m3")]
    B = [gi.to_bits(r.integers(-2, 3, (N, K)).astype(np.float32), "f8e4m3")]
    got = _ptr_run(gmi, A, B, M, N, K, K, K, N)[0]
    ref = oracle.gemm(A[0], B[0], K=K, dtype="f8e4m3")
    assert np.array_equal(got, oracle.round_to(ref, "bf16"))


@pytest.mark.parametrize("K", [128, 1040])
def test_fp8_grouped_mixed_tile_classes(gmi, K):
    # enough 256 x 256 tiles for the launch to use them, problems of at most 64 rows on the small class and of
    # at most 32 rows on the tiny one
    r = np.random.default_rng(K)
    Ms = [1, 8, 32, 33, 40, 64, 65, 200, 256, 300] + list(r.integers(1, 500, 62))
    N = 1024
    As = [_codes(r, (int(M), K)) for M in Ms]
    Bs = [_codes(r, (N, K)) for _ in Ms]
    outs = [Guarded(int(M), N, N, "bf16") for M in Ms]
    gmi.gemm_grouped([to_dev(a, "f8e4m3") for a in As], [to_dev(b, "f8e4m3") for b in Bs], None,
                     [o.view for o in outs], alpha=2.0)
    torch.cuda.synchronize()
    for M, a, b, o in zip(Ms, As, Bs, outs):
        o.check_guards(f"fp8 grouped M={M}")
        check_close(o.bits(), oracle.gemm(a, b, K=K, alpha=2.0, dtype="f8e4m3"), "bf16", f"fp8 grouped M={M} K={K}",
                    rtol=RTOL8)


def test_fp8_headline_shape_sampled(gmi):
    # 16 x 1024^3 (the pointer-array workload in fp8): 24 sampled rows of two batches against the oracle
    A, B = gi.ptr_array_f8(L=16)
    got = _ptr_run(gmi, A, B, 1024, 1024, 1024, 1024, 1024, 1024)
    rows = np.random.default_rng(2).choice(1024, 24, replace=False)
    for l in (0, 15):
        ref = oracle.gemm(A[l][rows], B[l], K=1024, dtype="f8e4m3")
        check_close(got[l][rows], ref, "bf16", f"fp8 headline batch {l}", rtol=RTOL8)
