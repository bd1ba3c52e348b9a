"""GPU parity of the MoE layer at its full size (16384 token rows routed over
128 experts with Zipf(1.1) counts, 8 experts empty; N = 2048, K = 4096, one
weight per expert), in the launches the benchmark times: the host-table
grouped call, the device-offsets call, and the fp8 (E4M3) host-table call.
The expert weights are slices of one allocation here.  The oracle computes
sampled outputs one by one: every live group on up to 6 of its rows (its
first and last among them) times 16 shared columns."""
import numpy as np
import pytest
import torch

import gmi_inputs as gi
import oracle
from helpers import check_close, dev, host_bits, to_dev

pytestmark = pytest.mark.gpu
N, K = 2048, 4096
COLS = np.sort(np.random.default_rng(31).choice(N, 16, replace=False))


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    g.lib()
    return g


def _rows(counts):
    r = np.random.default_rng(32)
    off = np.concatenate([[0], np.cumsum(counts)])
    pick = {}
    for g, c in enumerate(counts):
        if c == 0:
            continue
        mid = r.choice(int(c), min(int(c), 4), replace=False)
        pick[g] = np.unique(np.concatenate([[0, c - 1], mid])) + off[g]
    return off, pick


_LAYERS = {}


def _layer(dtype):
    """Device A [16384][4096] and B [128][2048][4096]; on the host, A and the
    sampled columns of every expert's weight.  Cached for the last element
    type asked for."""
    if dtype in _LAYERS:
        return _LAYERS[dtype]
    _LAYERS.clear()  # one layer's 2 GB of weights on the device at a time
    counts = gi.moe_counts()
    if dtype == "bf16":
        A = gi.moe_activations()
        weight = gi.moe_expert_weight
    else:
        A = gi.moe_activations_f8()
        weight = gi.moe_expert_weight_f8
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float8_e4m3fn
    B3 = torch.empty((len(counts), N, K), dtype=tdt, device=dev())
    cols = []
    for g in range(len(counts)):
        w = weight(g)
        B3[g].copy_(to_dev(w, dtype))
        cols.append(np.ascontiguousarray(w[COLS]))
    _LAYERS[dtype] = (counts, A, to_dev(A, dtype), B3, cols)
    return _LAYERS[dtype]


def _check(got, A, cols, counts, dtype, what):
    off, pick = _rows(counts)
    assert got.shape == (int(counts.sum()), len(COLS))
    rtol = 1e-2 if dtype == "bf16" else 3e-2
    for g, rows in pick.items():
        ref = oracle.gemm(A[rows], cols[g], K=K, dtype=dtype)
        check_close(got[rows], ref, "bf16", f"{what} group {g} ({counts[g]} rows)", rtol=rtol)


@pytest.mark.parametrize("dtype", ["f8e4m3", "bf16"])
def test_moe_layer_full_size_host_table(gmi, dtype):
    counts, A, Ad, B3, cols = _layer(dtype)
    off = np.concatenate([[0], np.cumsum(counts)])
    D = torch.empty((int(counts.sum()), N), dtype=torch.bfloat16, device=dev())
    gmi.gemm_grouped([Ad[off[g]:off[g + 1]] for g in range(len(counts))], [B3[g] for g in range(len(counts))], None,
                     [D[off[g]:off[g + 1]] for g in range(len(counts))])
    torch.cuda.synchronize()
    got = host_bits(D[:, torch.from_numpy(COLS).to(dev())])
    _check(got, A, cols, counts, dtype, f"MoE {dtype} host table")


def test_moe_layer_full_size_device_offsets(gmi):
    counts, A, Ad, B3, cols = _layer("bf16")
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device=dev())
    D = torch.empty((int(counts.sum()), N), dtype=torch.bfloat16, device=dev())
    gmi.gemm_grouped_offsets(offs, Ad, B3, D)
    torch.cuda.synchronize()
    got = host_bits(D[:, torch.from_numpy(COLS).to(dev())])
    _check(got, A, cols, counts, "bf16", "MoE bf16 device offsets")
