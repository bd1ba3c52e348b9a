"""GPU parity of the grouped GEMM whose group sizes are device-held row offsets
(mixture-of-experts layout: the rows of every group stacked in one A and one D,
one weight per group in one B), against the fp64 oracle per group, and bit for
bit against the host-table grouped GEMM on the same problems."""
import numpy as np
import pytest
import torch

import gmi_inputs as gi
import oracle
from helpers import SENTINEL, check_close, dev, host_bits, to_dev

pytestmark = pytest.mark.gpu
RTOL8 = 3e-2


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _case(counts, N, K, dtype="bf16", seed=0, pad=8, extra_rows=0, beta=0.0):
    """Host operands: A [rows][lda], B [G][N][ldb] with a padded expert stride, C [rows][ldc]."""
    r = np.random.default_rng(seed)
    rows = int(np.sum(counts)) + extra_rows
    ld = (K + 15) // 16 * 16 + (16 if dtype == "f8e4m3" else pad)
    scale = 1.0 if dtype == "f8e4m3" else 0.02
    A = gi.to_bits(r.standard_normal((rows, ld)).astype(np.float32), dtype)
    B = gi.to_bits((scale * r.standard_normal((len(counts), N + 1, ld))).astype(np.float32), dtype)
    cdt = "bf16" if dtype == "f8e4m3" else dtype
    C = gi.to_bits(r.uniform(-1, 1, (rows, N + 8)).astype(np.float32), cdt) if beta else None
    return A, B, C, rows, ld, cdt


def _run(gmi, offsets, A, B, C, rows, N, K, dtype, cdt, alpha=1.0, beta=0.0):
    """D [rows][N + 8] pre-filled with a sentinel; returns its bits."""
    Ad = to_dev(A, dtype)
    Bd = to_dev(B.reshape(B.shape[0], -1), dtype)
    Bv = Bd.view(B.shape[0], B.shape[1], B.shape[2])[:, :N, :K]
    Cd = to_dev(C, cdt)[:, :N] if C is not None else None
    Dfull = torch.full((rows, N + 8), SENTINEL, dtype=torch.int16, device=dev()).view(
        torch.bfloat16 if cdt == "bf16" else torch.float16)
    off = torch.tensor(np.asarray(offsets, np.int32), device=dev())
    gmi.gemm_grouped_offsets(off, Ad[:, :K], Bv, Dfull[:, :N], C=Cd, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    got = host_bits(Dfull)
    assert np.all(got[:, N:] == SENTINEL), "padding columns of D written"
    return got[:, :N]


def _check_groups(got, offsets, A, B, C, rows, N, K, dtype, cdt, alpha=1.0, beta=0.0, rtol=1e-2):
    """Each group's rows against the oracle; rows outside every (clipped) group untouched."""
    covered = np.zeros(rows, bool)
    for g in range(len(offsets) - 1):
        lo = min(max(offsets[g], 0), rows)
        hi = min(max(offsets[g + 1], 0), rows)
        if hi <= lo:
            continue
        covered[lo:hi] = True
        ref = oracle.gemm(A[lo:hi, :K], B[g, :N, :K], C[lo:hi, :N] if C is not None else None, alpha=alpha,
                          beta=beta, dtype=dtype, dtype_c=cdt)
        check_close(got[lo:hi], ref, cdt, f"group {g} rows {lo}:{hi}", rtol=rtol)
    assert np.all(got[~covered] == SENTINEL), "rows outside every group written"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_offsets_moe_small_with_empty_groups(gmi, dtype):
    counts = gi.moe_counts(tokens=1500, groups=24, empty=4)
    N, K = 192, 256
    A, B, C, rows, ld, cdt = _case(counts, N, K, dtype, seed=1, extra_rows=40)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    got = _run(gmi, off, A, B, C, rows, N, K, dtype, cdt)
    _check_groups(got, off, A, B, C, rows, N, K, dtype, cdt)


@pytest.mark.parametrize("K", [128, 100])
def test_offsets_tile_classes_with_beta(gmi, K):
    # 96 groups of 0 .. 600 rows, N = 1024: enough rows for the 256 x 256 tiles, so groups of at most 64 rows
    # take the 64 x 256 class; K = 100 adds the K-tail copies; beta != 0 reads C through the group offsets
    r = np.random.default_rng(K)
    counts = np.array([0, 1, 17, 63, 64, 65, 100, 255, 256, 257, 600, 0] + list(r.integers(0, 600, 84)))
    counts[-1] += max(0, 16384 - int(counts.sum()))
    N = 1024
    A, B, C, rows, ld, cdt = _case(counts, N, K, "bf16", seed=K, beta=0.5)
    off = np.concatenate([[0], np.cumsum(counts)])
    got = _run(gmi, off, A, B, C, rows, N, K, "bf16", cdt, alpha=1.5, beta=0.5)
    # the oracle on a sample of groups covering both tile classes and the boundaries
    for g in [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 20, 95]:
        lo, hi = off[g], off[g + 1]
        ref = oracle.gemm(A[lo:hi, :K], B[g, :N, :K], C[lo:hi, :N], alpha=1.5, beta=0.5, dtype="bf16")
        check_close(got[lo:hi], ref, "bf16", f"group {g} ({hi - lo} rows)")
    assert not np.any(got == SENTINEL), "a row of D was not written"


def test_offsets_match_host_table_bit_for_bit(gmi):
    # the same problems through the host-built table: identical bits (same kernel, same k order)
    counts = gi.moe_counts(tokens=3000, groups=40, empty=5)
    N, K = 320, 384
    A, B, C, rows, ld, cdt = _case(counts, N, K, "bf16", seed=5)
    off = np.concatenate([[0], np.cumsum(counts)])
    got = _run(gmi, off, A, B, C, rows, N, K, "bf16", cdt)
    Ad, Bd = to_dev(A, "bf16"), to_dev(B.reshape(len(counts), -1), "bf16")
    Bv = Bd.view(B.shape)[:, :N, :K]
    D2 = torch.empty((rows, N), dtype=torch.bfloat16, device=dev())
    live = [g for g in range(len(counts)) if counts[g]]
    gmi.gemm_grouped([Ad[off[g]:off[g + 1], :K] for g in live], [Bv[g] for g in live], None,
                     [D2[off[g]:off[g + 1]] for g in live])
    torch.cuda.synchronize()
    assert np.array_equal(got, host_bits(D2))


def test_offsets_fp8(gmi):
    counts = gi.moe_counts(tokens=900, groups=12, empty=2)
    N, K = 256, 512
    A, B, C, rows, ld, cdt = _case(counts, N, K, "f8e4m3", seed=6)
    off = np.concatenate([[0], np.cumsum(counts)])
    got = _run(gmi, off, A, B, C, rows, N, K, "f8e4m3", cdt)
    _check_groups(got, off, A, B, C, rows, N, K, "f8e4m3", cdt, rtol=RTOL8)


@pytest.mark.parametrize("offsets", [
    [-10, 40, 100, 5000],     # clipped to [0, rows)
    [0, 40, 100, 60],         # last group reversed: skipped
    [0, 0, 0, 150],           # empty groups first
    [150, 150, 150, 150],     # every group empty
])
def test_offsets_out_of_range_are_clipped(gmi, offsets):
    N, K, rows = 136, 72, 150
    A, B, C, _, ld, cdt = _case([rows], N, K, "bf16", seed=7)
    B = np.concatenate([B] * 3)
    got = _run(gmi, offsets, A, B, C, rows, N, K, "bf16", cdt)
    _check_groups(got, offsets, A, B, C, rows, N, K, "bf16", cdt)


def test_offsets_one_group_many_rows_and_repeat_calls(gmi):
    # one expert gets every row (the other groups empty); a second call gives the same bits
    N, K = 512, 256
    counts = np.array([0, 2048, 0, 0])
    A, B, C, rows, ld, cdt = _case(counts, N, K, "bf16", seed=8)
    off = np.concatenate([[0], np.cumsum(counts)])
    first = _run(gmi, off, A, B, C, rows, N, K, "bf16", cdt)
    second = _run(gmi, off, A, B, C, rows, N, K, "bf16", cdt)
    assert np.array_equal(first, second)
    sample = np.random.default_rng(8).choice(rows, 96, replace=False)
    ref = oracle.gemm(A[sample, :K], B[1, :N, :K], dtype="bf16")
    check_close(first[sample], ref, "bf16", "single group")
