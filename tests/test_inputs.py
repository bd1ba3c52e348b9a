"""The seeded input generators: deterministic, shaped as the workloads state,
and the MoE routing recipe (forced-empty groups, Zipf(1.1) ranks)."""
import hashlib

import numpy as np

import gmi_inputs as gi


def _h(*arrays):
    m = hashlib.sha256()
    for a in arrays:
        m.update(np.ascontiguousarray(a).tobytes())
    return m.hexdigest()


def test_generators_are_deterministic_and_seed_sensitive():
    a = gi.grouped_f16()
    b = gi.grouped_f16()
    c = gi.grouped_f16(seed=1)
    for pa, pb, pc in zip(a, b, c):
        assert _h(pa["A"], pa["B"], pa["C"]) == _h(pb["A"], pb["B"], pb["C"])
        assert _h(pa["A"]) != _h(pc["A"])
    x1, w1 = gi.conv_fprop_bf16(N=1, H=4, W=4, C=8, K=8)
    x2, w2 = gi.conv_fprop_bf16(N=1, H=4, W=4, C=8, K=8)
    assert _h(x1, w1) == _h(x2, w2)


def test_workload_shapes():
    probs = gi.grouped_f16()
    assert [(p["M"], p["N"], p["K"]) for p in probs] == gi.W1_SHAPES
    for p in probs:
        assert p["A"].shape == (p["M"], p["K"]) and p["B"].shape == (p["N"], p["K"])
        assert p["C"].shape == (p["M"], p["N"]) and p["A"].dtype == np.uint16
    A, B = gi.ptr_array_bf16(L=2, M=64, N=32, K=16)
    assert len(A) == 2 and A[0].shape == (64, 16) and B[1].shape == (32, 16)
    w = gi.w4a16(M=3, N=32, K=256, group=128)
    assert w["X"].shape == (3, 256) and w["W"].shape == (32, 128)
    assert w["scales"].shape == (2, 32) and w["zeros"].shape == (2, 16)
    assert np.array_equal(gi.unpack_u4(w["W"], 256), w["Wq"])


def test_value_ranges():
    w = gi.w4a16(M=2, N=64, K=256)
    s = w["scales"].view(np.float16).astype(np.float64)
    assert s.min() >= 0.001 - 1e-6 and s.max() <= 0.01 + 1e-5
    assert w["Wq"].max() <= 15 and w["zq"].max() <= 15
    p = gi.grouped_f16()[0]
    a = p["A"].view(np.float16).astype(np.float64)
    assert a.min() >= -1 and a.max() <= 1
    A, _ = gi.ptr_array_bf16(L=1, M=256, N=8, K=1024)
    std = (A[0].astype(np.uint32) << 16).view(np.float32).std()
    assert abs(std - 1 / 32) < 1e-3


def test_moe_counts_recipe():
    c = gi.moe_counts()
    assert c.sum() == 16384 and len(c) == 128
    assert sorted(np.where(c == 0)[0].tolist()) == [1, 72, 87, 96, 106, 107, 122, 124]
    assert c.max() == 3703
    assert (c[c > 0] < 32).sum() == 43


def test_bf16_cast_is_round_to_nearest_even():
    f = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    assert gi.f32_to_bf16_bits(f).tolist() == [0x3F80, 0x3F82, 0x3F81, 0xC020]


def test_e4m3_encoder_matches_torch_and_saturates():
    import torch

    r = np.random.default_rng(3)
    x = np.concatenate([r.standard_normal(50000) * 10.0 ** r.uniform(-4, 2.6, 50000), np.linspace(-448, 448, 4001)])
    x = np.clip(x, -448, 448).astype(np.float32)
    # exact halfway points between neighbouring positive codes (ties go to the even code)
    codes = np.arange(126, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    x = np.concatenate([x, ((vals[:-1] + vals[1:]) / 2).astype(np.float32)])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(gi.to_bits(x, "f8e4m3"), want)
    # beyond the largest finite value (1.75 * 2^8) the encoder saturates
    assert list(gi.to_bits(np.array([1e4, -500.0, 449.0], np.float32), "f8e4m3")) == [0x7E, 0xFE, 0x7E]


def test_fp8_workloads():
    A, B = gi.ptr_array_f8(L=2, M=8, N=16, K=32)
    assert A[0].dtype == np.uint8 and A[0].shape == (8, 32) and B[1].shape == (16, 32)
    assert _h(*A) == _h(*gi.ptr_array_f8(L=2, M=8, N=16, K=32)[0])
    assert gi.moe_expert_weight_f8(3, N=16, K=32).shape == (16, 32)


def test_moe_w4_decode_workload():
    c = gi.moe_w4_counts()
    assert c.sum() == 128 and len(c) == 128 and (c == 0).sum() >= 8
    w, s, z = gi.moe_w4_expert(5, N=32, K=256)
    assert w.shape == (32, 128) and w.dtype == np.uint8
    assert s.shape == (2, 32) and s.dtype == np.uint16 and z.shape == (2, 16)
    sv = (s.astype(np.uint32) << 16).view(np.float32)  # bf16 scales in [0.001, 0.01]
    assert np.all((sv >= 0.000999) & (sv <= 0.0101))
    assert _h(w) == _h(gi.moe_w4_expert(5, N=32, K=256)[0]) and _h(w) != _h(gi.moe_w4_expert(6, N=32, K=256)[0])
    assert gi.moe_w4_activations(rows=7, K=64).shape == (7, 64)
