"""GPU parity of the uint4 prepack (bit-exact) and of the W4A16 GEMM against
the fp64 oracle."""
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


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (256, 1024), (8192, 8192)])
def test_prepack_matches_oracle_bit_exact(gmi, N, K):
    w = np.random.default_rng(N + K).integers(0, 256, (N, K // 2), dtype=np.uint8)
    got = gmi.prepack_w4(bytes_to_dev(w), N, K).cpu().numpy()
    assert got.size == N * K // 2
    assert np.array_equal(got, oracle.prepack_w4(w, N, K))
    assert np.array_equal(oracle.unprepack_w4(got, N, K), w)


def _w4_run(gmi, d, ldy_pad=0):
    M, N, K, g = d["M"], d["N"], d["K"], d["group"]
    wpp = gmi.prepack_w4(bytes_to_dev(d["W"]), N, K)
    out = Guarded(M, N, N + ldy_pad, "f16")
    gmi.gemm_w4a16(to_dev(d["X"], "f16"), wpp, to_dev(d["scales"], "f16"), bytes_to_dev(d["zeros"]), g, N, Y=out.view)
    torch.cuda.synchronize()
    out.check_guards(f"w4a16 M={M} N={N} K={K}")
    return out.bits()


@pytest.mark.parametrize("M", [1, 5, 16, 17, 33, 48, 49, 64, 65, 128, 200, 257])
def test_w4a16_shapes(gmi, M):
    d = gi.w4a16(seed=M, M=M, N=512, K=1024, group=128)
    got = _w4_run(gmi, d, ldy_pad=8)
    ref = oracle.w4a16(d["X"], d["W"], d["scales"], d["zeros"], d["N"], d["K"], d["group"])
    check_close(got, ref, "f16", f"w4a16 M={M}")


@pytest.mark.parametrize("group", [256, 1024])
def test_w4a16_group_sizes(gmi, group):
    # group == K (per channel) and a multi-tile group
    for M in (16, 96):
        d = gi.w4a16(seed=7, M=M, N=256, K=1024, group=group)
        ref = oracle.w4a16(d["X"], d["W"], d["scales"], d["zeros"], d["N"], d["K"], group)
        check_close(_w4_run(gmi, d), ref, "f16", f"w4a16 group {group} M={M}")


@pytest.mark.parametrize("M", [16, 100])
def test_w4a16_exact_small_integers(gmi, M):
    # X in {-1, 0, 1}, s = 1, z = 8, K = 128: every product and partial sum is a
    # small integer, exact in fp16 and fp32, so Y == RN16(ref) bit-exactly
    N, K = 64, 128
    r = np.random.default_rng(1)
    q = r.integers(0, 16, (N, K), dtype=np.uint8)
    X = gi.to_bits(r.integers(-1, 2, (M, K)).astype(np.float32), "f16")
    d = dict(M=M, N=N, K=K, group=128, X=X, W=gi.pack_u4(q),
             scales=gi.to_bits(np.ones((1, N), np.float32), "f16"),
             zeros=gi.pack_u4(np.full((1, N), 8, np.uint8)))
    ref = oracle.w4a16(d["X"], d["W"], d["scales"], d["zeros"], N, K, 128)
    assert np.array_equal(_w4_run(gmi, d), oracle.round_to(ref, "f16"))


@pytest.mark.parametrize("M", [16, 48, 128, 1024, 4096])
def test_workload4_full_size(gmi, M):
    # N = K = 8192, g = 128: all rows checked for M = 16, 32 sampled rows otherwise (M = 48 runs the decode
    # body over three token tiles)
    d = gi.w4a16(M=M)
    got = _w4_run(gmi, d)
    rows = np.arange(M) if M <= 16 else np.random.default_rng(M).choice(M, 32, replace=False)
    ref = oracle.w4a16(d["X"][rows], d["W"], d["scales"], d["zeros"], d["N"], d["K"], d["group"])
    check_close(got[rows], ref, "f16", f"workload 4 M={M}")


def test_w4a16_ragged_raster_band_full(gmi):
    # M = 600 is five 128-token row tiles, so the register-sourced launch's bands of four row tiles end in a
    # band of one (N = 2048: 16 weight panels; K = 512 keeps the call unsplit); every output is checked
    d = gi.w4a16(seed=600, M=600, N=2048, K=512, group=128)
    assert gmi.w4a16_workspace_bytes(600, 2048, 512) == 0
    got = _w4_run(gmi, d)
    ref = oracle.w4a16(d["X"], d["W"], d["scales"], d["zeros"], d["N"], d["K"], d["group"])
    check_close(got, ref, "f16", "w4a16 M=600 ragged band")


def test_w4a16_big_tiles_ragged_raster_band_sampled(gmi):
    # M = 2304 at N = K = 8192 takes the 256 x 256 tiles (9 x 32 = 288 of them): bands of four row tiles end
    # in a band of one; 24 sampled rows, 16 of them from that last row tile
    M = 2304
    d = gi.w4a16(seed=2304, M=M, N=8192, K=8192, group=128)
    got = _w4_run(gmi, d)
    r = np.random.default_rng(2304)
    rows = np.concatenate([r.choice(2048, 8, replace=False), 2048 + r.choice(256, 16, replace=False)])
    ref = oracle.w4a16(d["X"][rows], d["W"], d["scales"], d["zeros"], d["N"], d["K"], d["group"])
    check_close(got[rows], ref, "f16", "w4a16 M=2304 last band")


def test_w4a16_prepack_layout_matters(gmi):
    # feeding the plain (un-prepacked) bytes must give a different answer: the
    # kernels really consume the permuted layout
    d = gi.w4a16(seed=3, M=16, N=64, K=256)
    Y = gmi.gemm_w4a16(to_dev(d["X"], "f16"), bytes_to_dev(d["W"]).reshape(-1), to_dev(d["scales"], "f16"),
                       bytes_to_dev(d["zeros"]), 128, 64)
    torch.cuda.synchronize()
    ref = oracle.w4a16(d["X"], d["W"], d["scales"], d["zeros"], 64, 256, 128)
    got = oracle.decode(host_bits(Y), "f16")
    assert not np.all(np.abs(got - ref) <= 1e-2 * np.abs(ref) + 1e-2)


def test_w4a16_split_and_unsplit_agree(gmi):
    # M = 160, N = 256, K = 2048: four output tiles, so with a workspace K is split into four k-ranges whose
    # fp32 partials (a whole 128 x 128 tile each, the ragged second row of tiles included) a second launch
    # sums; without one the same tiles run unsplit.  Both meet the oracle.
    M, N, K = 160, 256, 2048
    assert gmi.w4a16_workspace_bytes(M, N, K) == 4 * 4 * 128 * 128 * 4
    d = gi.w4a16(seed=11, M=M, N=N, K=K, group=128)
    ref = oracle.w4a16(d["X"], d["W"], d["scales"], d["zeros"], N, K, 128)
    wpp = gmi.prepack_w4(bytes_to_dev(d["W"]), N, K)
    args = (to_dev(d["X"], "f16"), wpp, to_dev(d["scales"], "f16"), bytes_to_dev(d["zeros"]), 128, N)
    for ws in (torch.zeros(gmi.w4a16_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev()),
               torch.empty(0, dtype=torch.uint8, device=dev())):
        out = Guarded(M, N, N + 8, "f16")
        gmi.gemm_w4a16(*args, Y=out.view, workspace=ws)
        torch.cuda.synchronize()
        out.check_guards(f"w4a16 split workspace {ws.numel()} bytes")
        check_close(out.bits(), ref, "f16", f"w4a16 workspace {ws.numel()} bytes")
