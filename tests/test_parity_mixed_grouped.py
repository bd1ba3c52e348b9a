"""GPU parity of the grouped (mixture-of-experts) mixed-input GEMM: group sizes
as device row offsets, one prepacked 4-bit weight with its scales and zero
points per group.  Each group is checked against the fp64 oracle on its own
rows and weights, and against the same group launched alone, bit for bit.

Tolerance: |d - ref| <= 1e-2 |ref| + 1e-2 for every group, whichever kernel
runs it: the decode body (16 rows at a time, or a group of 17 to 32 rows as
two tiles at once) and, for a group of more than 32 rows in a call of more
than 256 rows, the tiled kernel.  With bf16 activations both feed the matrix
instruction exact integer weights and scale fp32 partial sums per group."""
import numpy as np
import pytest
import torch

import gmi_inputs as gi
import oracle
from helpers import SENTINEL, bytes_to_dev, check_close, dev, host_bits, to_dev

pytestmark = pytest.mark.gpu

TILED_ROWS = 32  # groups above this many rows run the tiled kernel, the others the two-tile decode kernel ...
TILED_CALL_ROWS = 256  # ... in calls of more than this many rows


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _experts(G, N, K, group, dtype, seed):
    r = np.random.default_rng(seed)
    W = r.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    Z = r.integers(0, 256, (G, K // group, N // 2), dtype=np.uint8)
    S = gi.to_bits(r.uniform(0.001, 0.01, (G, K // group, N)).astype(np.float32), dtype)
    return W, S, Z


def _run(gmi, offsets, rows, X, W, S, Z, N, K, group, dtype, w_type, mode):
    G = W.shape[0]
    wpp = torch.stack([gmi.prepack_w4(bytes_to_dev(W[g]), N, K) for g in range(G)])
    s_dev = to_dev(S.reshape(G, -1), dtype).view(G, K // group, N) if mode != "direct" else None
    z_dev = bytes_to_dev(Z) if mode == "zero" else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    Yfull = torch.full((rows, N + 8), SENTINEL, dtype=torch.int16, device=dev()).view(tdt)
    off = torch.tensor(np.asarray(offsets, np.int32), device=dev())
    gmi.gemm_mixed_grouped(off, to_dev(X, dtype), wpp, s_dev, z_dev, group, N, w_type=w_type, Y=Yfull[:, :N])
    torch.cuda.synchronize()
    got = host_bits(Yfull)
    assert np.all(got[:, N:] == SENTINEL), "padding columns of Y written"
    return got[:, :N], wpp, s_dev, z_dev


def _check_groups(got, offsets, rows, X, W, S, Z, N, K, group, dtype, w_type, mode):
    covered = np.zeros(rows, bool)
    for g in range(len(offsets) - 1):
        lo, hi = min(max(offsets[g], 0), rows), min(max(offsets[g + 1], 0), rows)
        if hi <= lo:
            continue
        covered[lo:hi] = True
        s = S[g] if mode != "direct" else None
        z = Z[g] if mode == "zero" else None
        ref = oracle.mixed(X[lo:hi], W[g], s, z, N, K, group, w_type, dtype)
        check_close(got[lo:hi], ref, dtype, f"group {g} rows {lo}:{hi} {dtype} {w_type} {mode}")
    assert np.all(got[~covered] == SENTINEL), "rows outside every group written"


@pytest.mark.parametrize("dtype,w_type,mode", [("f16", "uint4", "zero"), ("bf16", "int4", "zero"),
                                               ("f16", "int4", "scale"), ("bf16", "uint4", "direct")])
def test_mixed_grouped_moe_decode(gmi, dtype, w_type, mode):
    # 24 experts, a few routed rows each (0 .. 40: the decode body up to 16 rows, the skinny body above)
    r = np.random.default_rng(3)
    counts = r.integers(0, 41, 24)
    counts[[2, 7, 11]] = 0
    counts[5], counts[6] = 16, 17
    N, K, group = 256, 512, 128
    rows = int(counts.sum()) + 24
    X = gi.to_bits(r.standard_normal((rows, K)).astype(np.float32), dtype)
    W, S, Z = _experts(len(counts), N, K, group, dtype, seed=4)
    off = np.concatenate([[0], np.cumsum(counts)])
    got, *_ = _run(gmi, off, rows, X, W, S, Z, N, K, group, dtype, w_type, mode)
    _check_groups(got, off, rows, X, W, S, Z, N, K, group, dtype, w_type, mode)


def test_mixed_grouped_large_groups_in_chunks(gmi):
    # groups of 150 and 64 rows in a call of 217 rows: all through the decode body, 16-row chunks, the last
    # one partial
    counts = np.array([150, 0, 64, 3])
    N, K, group = 128, 1024, 256
    rows = int(counts.sum())
    r = np.random.default_rng(5)
    X = gi.to_bits(r.standard_normal((rows, K)).astype(np.float32), "f16")
    W, S, Z = _experts(len(counts), N, K, group, "f16", seed=6)
    off = np.concatenate([[0], np.cumsum(counts)])
    got, *_ = _run(gmi, off, rows, X, W, S, Z, N, K, group, "f16", "int4", "zero")
    _check_groups(got, off, rows, X, W, S, Z, N, K, group, "f16", "int4", "zero")


@pytest.mark.parametrize("offsets", [[-10, 5, 30, 500], [0, 20, 40, 12], [40, 40, 40, 40]])
def test_mixed_grouped_offsets_are_clipped(gmi, offsets):
    N, K, group, rows = 64, 256, 128, 40
    r = np.random.default_rng(7)
    X = gi.to_bits(r.standard_normal((rows, K)).astype(np.float32), "bf16")
    W, S, Z = _experts(3, N, K, group, "bf16", seed=8)
    got, *_ = _run(gmi, offsets, rows, X, W, S, Z, N, K, group, "bf16", "uint4", "zero")
    _check_groups(got, offsets, rows, X, W, S, Z, N, K, group, "bf16", "uint4", "zero")


def test_mixed_grouped_groups_are_independent(gmi):
    # every group gives the same bits when launched alone (one group, offsets [0, rows of that group])
    counts = np.array([1, 9, 16, 17, 33, 64, 0, 5])
    N, K, group = 256, 1024, 128
    rows = int(counts.sum())
    r = np.random.default_rng(9)
    X = gi.to_bits(r.standard_normal((rows, K)).astype(np.float32), "bf16")
    W, S, Z = _experts(len(counts), N, K, group, "bf16", seed=10)
    off = np.concatenate([[0], np.cumsum(counts)])
    got, wpp, s_dev, z_dev = _run(gmi, off, rows, X, W, S, Z, N, K, group, "bf16", "int4", "zero")
    Xd = to_dev(X, "bf16")
    for g in range(len(counts)):
        if counts[g] == 0:
            continue
        one = torch.tensor([0, int(counts[g])], dtype=torch.int32, device=dev())
        Yg = gmi.gemm_mixed_grouped(one, Xd[off[g]:off[g + 1]], wpp[g:g + 1], s_dev[g:g + 1], z_dev[g:g + 1], group,
                                    N, w_type="int4")
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(Yg), got[off[g]:off[g + 1]]), g


@pytest.mark.parametrize("dtype,w_type,mode", [("f16", "uint4", "zero"), ("bf16", "int4", "zero"),
                                               ("bf16", "uint4", "scale"), ("f16", "int4", "direct")])
def test_mixed_grouped_prefill_groups_tiled(gmi, dtype, w_type, mode):
    # groups above 32 rows run the tiled launch (128 x 128 tiles, ragged in rows and in N; a last row tile
    # of at most 64 rows -- 1 of 129 and of 513, 33, 44 of 300, 64 -- multiplies half the tile, one of at
    # most 96 rows -- 80, 72 of 200 -- three quarters, 100 all of it), the others the two-tile decode
    # launch, in one call; empty groups between them
    counts = np.array([0, 3, 32, 33, 0, 300, 129, 1, 513, 16, 17, 64, 80, 200, 100])
    N, K, group = 320, 512, 128
    rows = int(counts.sum()) + 7
    r = np.random.default_rng(11)
    X = gi.to_bits(r.standard_normal((rows, K)).astype(np.float32), dtype)
    W, S, Z = _experts(len(counts), N, K, group, dtype, seed=12)
    off = np.concatenate([[0], np.cumsum(counts)])
    got, *_ = _run(gmi, off, rows, X, W, S, Z, N, K, group, dtype, w_type, mode)
    _check_groups(got, off, rows, X, W, S, Z, N, K, group, dtype, w_type, mode)


def test_mixed_grouped_tiled_matches_the_plain_call(gmi):
    # a group of 400 rows through the tiled launch gives the bits of gmi_gemm_mixed on the same rows (the
    # same tiled mainloop and epilogue, 128 x 128 tiles, no split); offsets clipped at the end of X
    N, K, group = 256, 1024, 256
    rows = 500
    r = np.random.default_rng(13)
    X = gi.to_bits(r.standard_normal((rows, K)).astype(np.float32), "bf16")
    W, S, Z = _experts(2, N, K, group, "bf16", seed=14)
    off = [0, 100, 900]  # group 1 clipped to rows 100 .. 499
    got, wpp, s_dev, z_dev = _run(gmi, off, rows, X, W, S, Z, N, K, group, "bf16", "int4", "zero")
    _check_groups(got, off, rows, X, W, S, Z, N, K, group, "bf16", "int4", "zero")
    Xd = to_dev(X, "bf16")
    ws = torch.empty(0, dtype=torch.uint8, device=dev())
    Y1 = gmi.gemm_mixed(Xd[100:500], wpp[1], s_dev[1], z_dev[1], group, N, w_type="int4", workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Y1), got[100:500])


@pytest.mark.parametrize("dtype,mode", [("bf16", "zero"), ("f16", "zero"), ("bf16", "scale")])
def test_mixed_grouped_pairs_match_the_decode_body(gmi, dtype, mode):
    # in a call that takes the tiled launch, groups of at most 32 rows run both 16-row tiles at once (the second
    # one empty for a group of at most 16 rows); they give the bits of a small call (at most 256 rows: every
    # group 16 rows at a time through the decode body)
    N, K, group = 336, 1024, 128  # 64-row weight slices, the last one a single 16-row block
    off = [0, 24, 56, 60, 400]  # 24, 32 and 4 rows (two tiles at once), 340 (tiled)
    rows = 400
    r = np.random.default_rng(21)
    X = gi.to_bits(r.standard_normal((rows, K)).astype(np.float32), dtype)
    W, S, Z = _experts(4, N, K, group, dtype, seed=22)
    got = _run(gmi, off, rows, X, W, S, Z, N, K, group, dtype, "uint4", mode)[0]
    _check_groups(got, off, rows, X, W, S, Z, N, K, group, dtype, "uint4", mode)
    small = _run(gmi, off[:4], 60, X[:60], W[:3], S[:3], Z[:3], N, K, group, dtype, "uint4", mode)[0]
    assert np.array_equal(small, got[:60])


def test_mixed_grouped_many_groups_all_decode(gmi):
    # more groups than the tiled launch's table holds, in a call of more than 256 rows: every group, large ones
    # too, runs the decode launch
    G = 1100
    counts = np.zeros(G, np.int64)
    counts[[0, 5, 700, 1099]] = [2, 90, 17, 170]
    N, K, group = 64, 256, 128
    rows = int(counts.sum())
    r = np.random.default_rng(15)
    X = gi.to_bits(r.standard_normal((rows, K)).astype(np.float32), "f16")
    W = r.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    Z = r.integers(0, 256, (G, K // group, N // 2), dtype=np.uint8)
    S = gi.to_bits(r.uniform(0.001, 0.01, (G, K // group, N)).astype(np.float32), "f16")
    off = np.concatenate([[0], np.cumsum(counts)])
    assert rows > TILED_CALL_ROWS
    got, *_ = _run(gmi, off, rows, X, W, S, Z, N, K, group, "f16", "uint4", "zero")
    _check_groups(got, off, rows, X, W, S, Z, N, K, group, "f16", "uint4", "zero")


def test_moe_w4_prefill_full_size_sampled(gmi):
    # the bench's 4-bit MoE prefill layer: 16384 rows routed over 128 experts (N 2048, K 4096, g 128, bf16,
    # int4 with zero points); 8 sampled rows of the four largest experts (tiled launch), of a mid-size one
    # and of every row of one decode-size expert, against the oracle
    N, K, group = 2048, 4096, 128
    counts = gi.moe_w4_counts(rows=16384)
    order = np.argsort(-counts)
    mid = int(order[np.searchsorted(-counts[order], -100)])           # about 100 rows: tiled
    small = int([g for g in order if 0 < counts[g] <= 64][0])         # the largest decode-size group
    picks = [int(g) for g in order[:4]] + [mid, small]
    experts = {g: gi.moe_w4_expert(g) for g in range(len(counts))}
    wpp = torch.stack([gmi.prepack_w4(bytes_to_dev(experts[g][0]), N, K) for g in range(len(counts))])
    Sx = torch.stack([to_dev(experts[g][1], "bf16") for g in range(len(counts))])
    Zx = torch.stack([bytes_to_dev(experts[g][2]) for g in range(len(counts))])
    X = gi.moe_w4_activations(rows=16384)
    off = np.concatenate([[0], np.cumsum(counts)])
    Y = gmi.gemm_mixed_grouped(torch.tensor(off.astype(np.int32), device=dev()), to_dev(X, "bf16"), wpp, Sx, Zx,
                               group, N, w_type="int4")
    torch.cuda.synchronize()
    got = host_bits(Y)
    r = np.random.default_rng(17)
    for g in picks:
        lo, hi = int(off[g]), int(off[g + 1])
        rows = np.arange(lo, hi) if hi - lo <= 64 else np.sort(r.choice(np.arange(lo, hi), 8, replace=False))
        w, s, z = experts[g]
        ref = oracle.mixed(X[rows], w, s, z, N, K, group, "int4", "bf16")
        check_close(got[rows], ref, "bf16", f"prefill expert {g} ({hi - lo} rows)")


def test_mixed_grouped_tiled_is_deterministic_and_covers_every_row(gmi):
    # three calls over Zipf-routed groups (several tiles per workgroup, partial row tiles, both launches):
    # every output element written, the same bits each time
    N, K, group = 512, 1024, 128
    counts = gi.moe_w4_counts(rows=6000, groups=64)
    rows = int(counts.sum())
    r = np.random.default_rng(19)
    X = gi.to_bits(r.standard_normal((rows, K)).astype(np.float32), "bf16")
    W, S, Z = _experts(len(counts), N, K, group, "bf16", seed=20)
    off = np.concatenate([[0], np.cumsum(counts)])
    outs = [_run(gmi, off, rows, X, W, S, Z, N, K, group, "bf16", "int4", "zero")[0] for _ in range(3)]
    assert not np.any(outs[0] == SENTINEL), "output elements left unwritten"
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert (counts > TILED_ROWS).sum() >= 10 and ((counts > 0) & (counts <= TILED_ROWS)).sum() >= 5
