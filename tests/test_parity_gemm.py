"""GPU parity of the grouped and pointer-array GEMM against the fp64 oracle."""
import itertools

import numpy as np
import pytest
import torch

import gmi_inputs as gi
import oracle
from helpers import Guarded, bytes_to_dev, check_close, dev, host_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _enc(vals, dtype):
    vals = np.asarray(vals, np.float32)
    return gi.to_bits(vals, dtype)


def run_grouped(gmi, shapes, dtype, alpha, beta, seed=0, ld_pad=0, vals=None):
    """Random problems with padded leading dimensions and guard-banded D;
    returns (D bits, oracle ref, shape) for every non-empty problem."""
    r = np.random.default_rng(seed)
    gen = vals if vals is not None else (lambda shp: r.uniform(-1, 1, shp))
    probs = (gmi.Problem * len(shapes))()
    keep = []
    for i, (M, N, K) in enumerate(shapes):
        lda = ldb = (K + 7) // 8 * 8 + ld_pad
        ldc = ldd = (N + 7) // 8 * 8 + ld_pad
        a, b, c = _enc(gen((M, lda)), dtype), _enc(gen((N, ldb)), dtype), _enc(gen((M, ldc)), dtype)
        ad, bd, cd = to_dev(a, dtype), to_dev(b, dtype), to_dev(c, dtype)
        g = Guarded(M, N, ldd, dtype) if M and N else None
        probs[i] = gmi.Problem(M, N, K, lda, ldb, ldc, ldd, ad.data_ptr(), bd.data_ptr(),
                               cd.data_ptr() if beta != 0 else None, g.view.data_ptr() if g else None)
        keep.append((a, b, c, M, N, K, ad, bd, cd, g))
    ws = torch.empty(gmi.workspace_bytes(len(shapes)), dtype=torch.uint8, device=dev())
    gmi.gemm_grouped_raw(probs, len(shapes), gmi.GMI_F16 if dtype == "f16" else gmi.GMI_BF16, alpha, beta, ws)
    torch.cuda.synchronize()
    out = []
    for (a, b, c, M, N, K, _, _, _, g) in keep:
        if g is None:
            continue
        g.check_guards(f"grouped {M}x{N}x{K}")
        ref = oracle.gemm(a, b, c if beta != 0 else None, K=K, alpha=alpha, beta=beta, dtype=dtype)
        out.append((g.bits(), ref, (M, N, K)))
    return out


def test_workload1_grouped_fp16(gmi):
    probs = gi.grouped_f16()
    As = [to_dev(p["A"], "f16") for p in probs]
    Bs = [to_dev(p["B"], "f16") for p in probs]
    Cs = [to_dev(p["C"], "f16") for p in probs]
    Gs = [Guarded(p["M"], p["N"], p["N"], "f16") for p in probs]
    gmi.gemm_grouped(As, Bs, Cs, [g.view for g in Gs], alpha=1.0, beta=0.5)
    torch.cuda.synchronize()
    for p, g in zip(probs, Gs):
        g.check_guards("workload 1")
        ref = oracle.gemm(p["A"], p["B"], p["C"], alpha=1.0, beta=0.5, dtype="f16")
        check_close(g.bits(), ref, "f16", f"workload 1 group {p['M']}x{p['N']}x{p['K']}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("beta", [0.0, -0.75])
def test_grouped_odd_shapes(gmi, dtype, beta):
    sizes = [1, 7, 31, 33, 65, 127, 129, 300]
    r = np.random.default_rng(11)
    shapes = [tuple(int(v) for v in r.choice(sizes, 3)) for _ in range(12)]
    shapes += [(0, 5, 8), (4, 0, 8), (257, 263, 72), (5, 9, 0)]
    for bits, ref, shp in run_grouped(gmi, shapes, dtype, alpha=1.25, beta=beta, seed=3, ld_pad=8):
        check_close(bits, ref, dtype, f"grouped {dtype} {shp}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_grouped_integer_inputs_bit_exact(gmi, dtype):
    # integers in [-4, 4], K <= 64: every fp32 partial sum is exact, so D must
    # equal the oracle rounded once, whatever the summation order
    r = np.random.default_rng(5)
    ints = lambda shp: r.integers(-4, 5, shp).astype(np.float32)
    shapes = [(64, 48, 64), (33, 70, 40), (300, 290, 64), (1, 1, 8)]
    for bits, ref, shp in run_grouped(gmi, shapes, dtype, alpha=1.0, beta=2.0, seed=5, vals=ints):
        assert np.array_equal(bits, oracle.round_to(ref, dtype)), shp


def test_grouped_per_group_constants(gmi):
    # A_g = 1, B_g = g + 1  =>  D_g = (g + 1) K_g exactly; catches pointer mix-ups
    shapes = [(40, 24, 16), (300, 8, 64), (7, 260, 8), (129, 129, 128), (1, 16, 512)]
    As, Bs, Gs = [], [], []
    for g, (M, N, K) in enumerate(shapes):
        As.append(torch.ones((M, K), dtype=torch.float16, device=dev()))
        Bs.append(torch.full((N, K), g + 1.0, dtype=torch.float16, device=dev()))
        Gs.append(Guarded(M, N, (N + 7) // 8 * 8, "f16"))
    gmi.gemm_grouped(As, Bs, None, [x.view for x in Gs])
    torch.cuda.synchronize()
    for g, ((M, N, K), x) in enumerate(zip(shapes, Gs)):
        x.check_guards("constants")
        assert np.array_equal(oracle.decode(x.bits(), "f16"), np.full((M, N), (g + 1.0) * K)), g


def test_grouped_moe_small_with_empty_groups(gmi):
    # MoE shape at reduced size: 24 experts, skewed counts, some empty; A and D
    # rows contiguous per group in group order
    counts = gi.moe_counts(tokens=1500, groups=24, empty=4)
    N, K = 192, 256
    r = np.random.default_rng(8)
    A = gi.to_bits(r.standard_normal((counts.sum(), K)).astype(np.float32), "bf16")
    Bw = [gi.to_bits(0.02 * r.standard_normal((N, K)).astype(np.float32), "bf16") for _ in counts]
    Ad = to_dev(A, "bf16")
    Dd = torch.full((counts.sum(), N), 0x7BAD, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    off = np.concatenate([[0], np.cumsum(counts)])
    As = [Ad[off[g]:off[g + 1]] for g in range(len(counts))]
    Ds = [Dd[off[g]:off[g + 1]] for g in range(len(counts))]
    Bs = [to_dev(b, "bf16") for b in Bw]
    gmi.gemm_grouped(As, Bs, None, Ds)
    torch.cuda.synchronize()
    got = host_bits(Dd)
    for g in range(len(counts)):
        if counts[g] == 0:
            continue
        ref = oracle.gemm(A[off[g]:off[g + 1]], Bw[g], dtype="bf16")
        check_close(got[off[g]:off[g + 1]], ref, "bf16", f"moe group {g}")


def test_grouped_is_deterministic(gmi):
    a = run_grouped(gmi, [(300, 260, 200), (64, 64, 64)], "bf16", 1.0, 0.5, seed=9)
    b = run_grouped(gmi, [(300, 260, 200), (64, 64, 64)], "bf16", 1.0, 0.5, seed=9)
    for (x, _, _), (y, _, _) in zip(a, b):
        assert np.array_equal(x, y)


def _ptr_array_case(gmi, L, M, N, K, beta, dtype="bf16"):
    A, B = gi.ptr_array_bf16(L=L, M=M, N=N, K=K) if dtype == "bf16" else (None, None)
    r = np.random.default_rng(2)
    C = [gi.to_bits(r.uniform(-1, 1, (M, N)).astype(np.float32), dtype) for _ in range(L)]
    Ad = [to_dev(a, dtype) for a in A]
    Bd = [to_dev(b, dtype) for b in B]
    Cd = [to_dev(c, dtype) for c in C]
    Dd = [torch.empty((M, N), dtype=Ad[0].dtype, device=dev()) for _ in range(L)]
    pa = lambda ts: gmi.pointer_array(ts, dev())
    gmi.gemm_ptr_array(L, M, N, K, pa(Ad), K, pa(Bd), K, pa(Cd) if beta else None, N, pa(Dd), N, Ad[0].dtype,
                       1.0, beta)
    torch.cuda.synchronize()
    return A, B, C, Dd


def test_ptr_array_small_with_beta(gmi):
    L, M, N, K = 5, 200, 136, 320
    A, B, C, Dd = _ptr_array_case(gmi, L, M, N, K, beta=0.5)
    for l in range(L):
        ref = oracle.gemm(A[l], B[l], C[l], alpha=1.0, beta=0.5, dtype="bf16")
        check_close(host_bits(Dd[l]), ref, "bf16", f"ptr-array batch {l}")


def test_workload2_ptr_array_full_size_sampled(gmi):
    # L = 16 separately allocated 1024^3 bf16 problems, beta = 0 (the launch the
    # benchmark times); every batch checked on 64 sampled rows x all columns
    L, M, N, K = 16, 1024, 1024, 1024
    A, B, C, Dd = _ptr_array_case(gmi, L, M, N, K, beta=0.0)
    rows = np.random.default_rng(4).choice(M, 64, replace=False)
    for l in range(L):
        ref = oracle.gemm(A[l][rows], B[l], dtype="bf16")
        check_close(host_bits(Dd[l])[rows], ref, "bf16", f"workload 2 batch {l}")


def test_ptr_array_one_batch_fully_checked(gmi):
    L, M, N, K = 2, 1024, 1024, 1024
    A, B, C, Dd = _ptr_array_case(gmi, L, M, N, K, beta=0.0)
    ref = oracle.gemm(A[1], B[1], dtype="bf16")
    check_close(host_bits(Dd[1]), ref, "bf16", "ptr-array full batch")


def test_timed_launch_matches_untimed_and_is_used_once(gmi):
    # gmi_time_next_gemm sends the next GEMM kernel through hipExtLaunchKernel with the caller's events: the
    # result is the same bits, the pair holds a positive duration no longer than events around the whole call,
    # and the request is consumed (the following call leaves the pair as it was)
    L, M, N, K = 4, 256, 512, 384
    A, B = gi.ptr_array_bf16(L=L, M=M, N=N, K=K)
    Ad = [to_dev(a, "bf16") for a in A]
    Bd = [to_dev(b, "bf16") for b in B]
    D0 = [torch.empty((M, N), dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    D1 = [torch.empty((M, N), dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    pa = lambda ts: gmi.pointer_array(ts, dev())
    pA, pB, p0, p1 = pa(Ad), pa(Bd), pa(D0), pa(D1)
    run = lambda pD: gmi.gemm_ptr_array(L, M, N, K, pA, K, pB, K, None, N, pD, N, torch.bfloat16, 1.0, 0.0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    ev[2].record()
    gmi.time_next_gemm(ev[0], ev[1])
    run(p0)
    ev[3].record()
    torch.cuda.synchronize()
    t_kernel, t_call = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    assert 0.0 < t_kernel <= t_call
    run(p1)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == t_kernel
    for l in range(L):
        assert np.array_equal(host_bits(D0[l]), host_bits(D1[l]))
    ref = oracle.gemm(A[1], B[1], dtype="bf16")
    check_close(host_bits(D0[1]), ref, "bf16", "timed ptr-array launch")


def test_empty_calls_are_noops(gmi):
    D = torch.full((4, 8), 3.0, dtype=torch.float16, device=dev())
    gmi.gemm_grouped([torch.empty((4, 8), dtype=torch.float16, device=dev())],
                     [torch.empty((0, 8), dtype=torch.float16, device=dev())], None, [D[:, :0]])
    z = torch.empty(0, dtype=torch.int64, device=dev())
    gmi.gemm_ptr_array(0, 4, 8, 8, z, 8, z, 8, None, 8, z, 8, torch.float16)
    torch.cuda.synchronize()
    assert torch.all(D == 3.0)


@pytest.mark.parametrize("K", [128, 100])
def test_grouped_mixed_tile_classes(gmi, K):
    # 72 problems with N = 1024 and M from 1 to 600: enough 256 x 256 tiles to fill the device, so the launch
    # uses them, and every problem of at most 64 rows takes the 64 x 256 tile class, of at most 32 rows the
    # 32 x 256 class, in the same kernel.  K = 100 also exercises the K-tail copies in every class.
    r = np.random.default_rng(K)
    Ms = [1, 17, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257, 600] + list(r.integers(1, 600, 59))
    shapes = [(int(M), 1024, K) for M in Ms]
    assert sum((M + 255) // 256 * 4 for M, _, _ in shapes) >= 256
    for got, ref, shp in run_grouped(gmi, shapes, "bf16", 1.5, 0.5, seed=K, ld_pad=8):
        check_close(got, ref, "bf16", f"grouped tile classes {shp}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_output_rounding_is_nearest_even(gmi, dtype):
    # D = A B with A rows [1, t, 0 ...] and B columns [1, 1, 0 ...]: 1 + t exactly in the fp32 accumulator, on,
    # above and below the midpoint of two representable values; the stored bits must be the oracle's RNE
    ties = {"f16": [3 * 2.0**-11, 2.0**-11, 2.0**-11 + 2.0**-16, 3 * 2.0**-11 - 2.0**-16],
            "bf16": [3 * 2.0**-8, 2.0**-8, 2.0**-8 + 2.0**-14, 3 * 2.0**-8 - 2.0**-14]}[dtype]
    M, N, K = 64, 64, 8
    a = np.zeros((M, K), np.float32)
    a[:, 0], a[:, 1] = 1.0, np.resize(np.array(ties, np.float32), M)
    b = np.zeros((N, K), np.float32)
    b[:, :2] = 1.0
    A, B = gi.to_bits(a, dtype), gi.to_bits(b, dtype)
    G = Guarded(M, N, N, dtype)
    gmi.gemm_grouped([to_dev(A, dtype)], [to_dev(B, dtype)], None, [G.view])
    torch.cuda.synchronize()
    ref = oracle.gemm(A, B, dtype=dtype)
    assert np.array_equal(ref, np.repeat(1.0 + a[:, 1:2].astype(np.float64), N, axis=1))
    assert np.array_equal(G.bits(), oracle.round_to(ref, dtype))


def test_grouped_inline_and_staged_tables_agree(gmi):
    # up to 32 problems travel in the kernel arguments, more are staged into the workspace: the same 32 problems
    # with and without a 33rd give identical bits, and both match the oracle
    r = np.random.default_rng(33)
    shapes = [(int(r.integers(1, 300)), int(r.integers(1, 300)), int(r.integers(1, 200))) for _ in range(33)]
    inline = run_grouped(gmi, shapes[:32], "bf16", 1.0, 0.25, seed=12, ld_pad=8)
    staged = run_grouped(gmi, shapes, "bf16", 1.0, 0.25, seed=12, ld_pad=8)
    assert len(inline) == 32 and len(staged) == 33
    for (a, ref, shp), (b, _, _) in zip(inline, staged):
        assert np.array_equal(a, b), shp
        check_close(a, ref, "bf16", f"grouped {shp}")
