"""The allocation-free grouped call (gmi_gemm_grouped_offsets_noalloc) against
the call it shares its kernels with (gmi_gemm_grouped_offsets, which keeps the
group table in a caller workspace): the same bits on two calls in a row, the
second one smaller, so a table left behind by the first call cannot leak into
the second.  Rows outside every group stay untouched."""
import numpy as np
import pytest
import torch

import oracle
from helpers import SENTINEL, check_close, dev, host_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _case(counts, N, K, dtype, seed, spare=5):
    r = np.random.default_rng(seed)
    rows = int(np.sum(counts)) + spare  # the last rows belong to no group
    A = r.standard_normal((rows, K)).astype(np.float32)
    B = (r.standard_normal((len(counts), N, K)) * 0.05).astype(np.float32)
    C = r.uniform(-1, 1, (rows, N)).astype(np.float32)
    import gmi_inputs as gi

    return rows, gi.to_bits(A, dtype), gi.to_bits(B, dtype), gi.to_bits(C, dtype)


def _both(gmi, counts, N, K, dtype, seed, beta):
    rows, A, B, C = _case(counts, N, K, dtype, seed)
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device=dev())
    Ad, Bd, Cd = to_dev(A, dtype), to_dev(B.reshape(len(counts) * N, K), dtype).view(len(counts), N, K), \
        to_dev(C, dtype)
    tdt = Ad.dtype
    outs = []
    for noalloc in (False, True):
        D = torch.full((rows, N), SENTINEL, dtype=torch.int16, device=dev()).view(tdt)
        if noalloc:
            gmi.gemm_grouped_offsets_noalloc(off, Ad, Bd, D, C=Cd if beta else None, alpha=1.0, beta=beta)
        else:
            gmi.gemm_grouped_offsets(off, Ad, Bd, D, C=Cd if beta else None, alpha=1.0, beta=beta)
        torch.cuda.synchronize()
        outs.append(host_bits(D))
    return rows, A, B, C, np.concatenate([[0], np.cumsum(counts)]), outs


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_noalloc_matches_the_workspace_call_on_two_calls(gmi, dtype):
    # first call: 40 groups over about 3000 rows (empty groups, groups of both tile classes), beta 0.5
    r = np.random.default_rng(1)
    counts1 = r.integers(0, 160, 40)
    counts1[[3, 17, 30]] = 0
    counts1[5], counts1[9] = 700, 64
    # second call: fewer groups, fewer rows, another N and K, beta 0
    counts2 = np.array([33, 0, 2, 250, 64, 9])
    for counts, N, K, beta, seed in ((counts1, 256, 512, 0.5, 2), (counts2, 128, 256, 0.0, 3)):
        rows, A, B, C, off, (ref_bits, got) = _both(gmi, counts, N, K, dtype, seed, beta)
        assert np.array_equal(got, ref_bits), f"noalloc differs from the workspace call ({len(counts)} groups)"
        assert np.all(got[off[-1]:] == SENTINEL), "rows outside every group written"
        # and the oracle on two groups of each call
        for g in [int(np.argmax(counts)), int(np.flatnonzero(counts)[0])]:
            lo, hi = off[g], off[g + 1]
            ref = oracle.gemm(A[lo:hi], B[g], C[lo:hi] if beta else None, alpha=1.0, beta=beta, dtype=dtype)
            check_close(got[lo:hi], ref, dtype, f"noalloc group {g}")
