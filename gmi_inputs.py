"""Seeded synthetic inputs for the grouped / mixed-input / implicit-conv GEMM
workloads.

This module only draws random numbers and stores them in the element formats
the library consumes (fp16 / bf16 bit patterns as uint16, uint4 packed two per
byte).  It holds none of the arithmetic of the method: both the fp64 oracle and
the HIP path read the bytes produced here, and neither imports the other.

Recipe (all workloads):
  * one numpy ``Generator(PCG64(SeedSequence([seed, workload_id, tensor_id])))``
    per tensor, default seed 20261202;
  * floating inputs are drawn in float32 and cast once, round-to-nearest-even,
    to fp16 (numpy) or bf16 (bit manipulation below);
  * ``N(0, s)`` means standard deviation ``s``;
  * uint4 tensors are drawn uniform on {0..15} and packed two per byte, the even
    index in the low nibble.

Workload ids and tensor ids:
  1  grouped fp16, 4 groups      A_g 10g+0, B_g 10g+1, C_g 10g+2   U(-1, 1)
  2  ptr-array bf16, L x 1024^3  A_l 100+l, B_l 200+l              N(0, 1/sqrt(K))
  3  MoE grouped bf16            counts 5, A 0 N(0,1), B_g 1000+g N(0, 0.02)
  4  W4A16                       X 0 N(0,1) fp16, W 1 U{0..15}, scales 3
                                 U(0.001, 0.01) fp16, zeros 4 U{0..15}
  5  conv2d fprop bf16           x 0 N(0,1), w 1 N(0, 1/sqrt(R*S*C))
"""
from __future__ import annotations

import numpy as np

DEFAULT_SEED = 20261202


def rng(seed: int, workload: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, workload, tensor])))


# ----------------------------------------------------------------------------
# storage casts (float32 -> 16-bit patterns, RNE)
# ----------------------------------------------------------------------------
def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32).astype(np.float16)).view(np.uint16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def f32_to_e4m3_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> OCP fp8 E4M3 codes (uint8), round to nearest even, saturating
    at +-448 (the format has no infinities); NaN -> 0x7F.  Written from the
    format: 3 mantissa bits, exponent bias 7, subnormal quantum 2^-9."""
    x = np.asarray(a, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    mag = np.minimum(np.abs(x), 448.0)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    e = np.maximum(e, -6.0)  # below 2^-6 the quantum stays 2^-9 (subnormals)
    q = np.ldexp(1.0, (e - 3).astype(np.int64))
    r = np.minimum(np.round(mag / q) * q, 448.0)  # np.round: ties to even
    normal = r >= 2.0 ** -6
    with np.errstate(divide="ignore"):
        er = np.floor(np.log2(np.where(normal, r, 1.0)))
    mant_n = np.where(normal, r / np.ldexp(1.0, er.astype(np.int64)) * 8 - 8, 0).astype(np.uint8)
    code_n = ((er + 7).astype(np.int64).clip(0, 15).astype(np.uint8) << np.uint8(3)) | mant_n
    code_s = np.where(normal, 0, r / 2.0 ** -9).astype(np.uint8)
    code = np.where(normal, code_n, code_s).astype(np.uint8) | sign
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def to_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f32_to_f16_bits(a)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    if dtype == "f8e4m3":
        return f32_to_e4m3_bits(a)
    raise ValueError(dtype)


def uniform(g: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    u = g.random(shape, dtype=np.float32)
    return np.float32(lo) + np.float32(hi - lo) * u


def normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return g.standard_normal(shape, dtype=np.float32) * np.float32(std)


def pack_u4(q: np.ndarray) -> np.ndarray:
    """[rows][cols] values 0..15 -> [rows][ceil(cols/2)] bytes, even col in the low nibble."""
    q = np.asarray(q, dtype=np.uint8)
    rows, cols = q.shape
    if cols % 2:
        q = np.concatenate([q, np.zeros((rows, 1), np.uint8)], axis=1)
    return np.ascontiguousarray(q[:, 0::2] | (q[:, 1::2] << np.uint8(4)))


def unpack_u4(p: np.ndarray, cols: int) -> np.ndarray:
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & np.uint8(15)
    out[:, 1::2] = p >> np.uint8(4)
    return out[:, :cols]


def uint4(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    return g.integers(0, 16, size=(rows, cols), dtype=np.uint8)


# ----------------------------------------------------------------------------
# workload 1: grouped fp16, 4 small groups, alpha = 1, beta = 0.5
# ----------------------------------------------------------------------------
W1_SHAPES = [(64, 128, 64), (128, 64, 128), (32, 96, 64), (128, 128, 32)]


def grouped_f16(seed: int = DEFAULT_SEED, shapes=W1_SHAPES):
    """Returns a list of dicts {M,N,K,A,B,C}: A [M][K], B column-major as [N][K],
    C [M][N]; all fp16 bit patterns drawn U(-1, 1)."""
    probs = []
    for gi, (m, n, k) in enumerate(shapes):
        a = to_bits(uniform(rng(seed, 1, 10 * gi + 0), (m, k), -1.0, 1.0), "f16")
        b = to_bits(uniform(rng(seed, 1, 10 * gi + 1), (n, k), -1.0, 1.0), "f16")
        c = to_bits(uniform(rng(seed, 1, 10 * gi + 2), (m, n), -1.0, 1.0), "f16")
        probs.append(dict(M=m, N=n, K=k, A=a, B=b, C=c))
    return probs


# ----------------------------------------------------------------------------
# workload 2: pointer-array bf16, L independent M = N = K = 1024 problems
# ----------------------------------------------------------------------------
def ptr_array_bf16(seed: int = DEFAULT_SEED, L: int = 16, M: int = 1024, N: int = 1024, K: int = 1024):
    """Returns (A_list, B_list): A_l [M][K], B_l column-major as [N][K], bf16 bits
    drawn N(0, 1/sqrt(K))."""
    std = 1.0 / np.sqrt(K)
    A = [to_bits(normal(rng(seed, 2, 100 + l), (M, K), std), "bf16") for l in range(L)]
    B = [to_bits(normal(rng(seed, 2, 200 + l), (N, K), std), "bf16") for l in range(L)]
    return A, B


# ----------------------------------------------------------------------------
# workload 3: MoE grouped bf16, Zipf(1.1)-skewed token counts, some groups empty
# ----------------------------------------------------------------------------
def moe_counts(seed: int = DEFAULT_SEED, tokens: int = 16384, groups: int = 128,
               empty: int = 8, s: float = 1.1) -> np.ndarray:
    """Token count per group: `empty` groups forced to zero, the rest drawn
    multinomially with probability proportional to rank^-s over a random rank
    permutation."""
    g = rng(seed, 3, 5)
    empties = g.choice(groups, empty, replace=False)
    live = np.setdiff1d(np.arange(groups), empties)
    rank = g.permutation(len(live)) + 1
    p = rank.astype(np.float64) ** (-s)
    p /= p.sum()
    counts = np.zeros(groups, np.int64)
    counts[live] = g.multinomial(tokens, p)
    return counts


def moe_activations(seed: int = DEFAULT_SEED, tokens: int = 16384, K: int = 4096) -> np.ndarray:
    return to_bits(normal(rng(seed, 3, 0), (tokens, K), 1.0), "bf16")


def moe_expert_weight(group: int, seed: int = DEFAULT_SEED, N: int = 2048, K: int = 4096) -> np.ndarray:
    """Expert `group`'s weight, column-major B stored as [N][K] bf16 bits, N(0, 0.02)."""
    return to_bits(normal(rng(seed, 3, 1000 + group), (N, K), 0.02), "bf16")


# ----------------------------------------------------------------------------
# workload 4: W4A16, Y = X W^T with uint4 W, fp16 scales, uint4 zeros per group
# ----------------------------------------------------------------------------
def w4a16(seed: int = DEFAULT_SEED, M: int = 16, N: int = 8192, K: int = 8192, group: int = 128):
    """Returns dict with X [M][K] fp16 bits, Wq [N][K] uint8 values 0..15 (unpacked),
    W [N][K/2] packed bytes, scales [K/g][N] fp16 bits, zq [K/g][N] values,
    zeros [K/g][N/2] packed bytes."""
    ng = (K + group - 1) // group
    wq = uint4(rng(seed, 4, 1), N, K)
    scales = to_bits(uniform(rng(seed, 4, 3), (ng, N), 0.001, 0.01), "f16")
    zq = uint4(rng(seed, 4, 4), ng, N)
    x = to_bits(normal(rng(seed, 4, 0), (M, K), 1.0), "f16")
    return dict(M=M, N=N, K=K, group=group, X=x, Wq=wq, W=pack_u4(wq), scales=scales,
                zq=zq, zeros=pack_u4(zq))


# ----------------------------------------------------------------------------
# workload 5: implicit-GEMM conv2d fprop, NHWC activation, KRSC filter
# ----------------------------------------------------------------------------
def conv_fprop_bf16(seed: int = DEFAULT_SEED, N: int = 32, H: int = 56, W: int = 56, C: int = 256,
                    K: int = 256, R: int = 3, S: int = 3):
    x = to_bits(normal(rng(seed, 5, 0), (N, H, W, C), 1.0), "bf16")
    w = to_bits(normal(rng(seed, 5, 1), (K, R, S, C), 1.0 / np.sqrt(R * S * C)), "bf16")
    return x, w


def conv_bias(seed: int = DEFAULT_SEED, K: int = 256, dtype: str = "bf16"):
    """Per-output-channel bias of the fused conv epilogue: N(0, 1), the spread of the conv outputs above, so a
    ReLU after it zeroes about half of them."""
    return to_bits(normal(rng(seed, 5, 2), (K,), 1.0), dtype)


# ----------------------------------------------------------------------------
# workload 6: fp8 E4M3 GEMMs (bf16 results) -- the headline pointer-array shape
# and the MoE layer with fp8 operands.  Values are drawn N(0, 1), the range an
# fp8 tensor holds after its per-tensor scaling; the stored codes are the
# inputs.
# ----------------------------------------------------------------------------
def ptr_array_f8(seed: int = DEFAULT_SEED, L: int = 16, M: int = 1024, N: int = 1024, K: int = 1024):
    """Returns (A_list, B_list) of uint8 E4M3 codes: A_l [M][K], B_l column-major as [N][K]."""
    A = [to_bits(normal(rng(seed, 6, 100 + l), (M, K), 1.0), "f8e4m3") for l in range(L)]
    B = [to_bits(normal(rng(seed, 6, 200 + l), (N, K), 1.0), "f8e4m3") for l in range(L)]
    return A, B


def moe_activations_f8(seed: int = DEFAULT_SEED, tokens: int = 16384, K: int = 4096) -> np.ndarray:
    return to_bits(normal(rng(seed, 6, 0), (tokens, K), 1.0), "f8e4m3")


def moe_expert_weight_f8(group: int, seed: int = DEFAULT_SEED, N: int = 2048, K: int = 4096) -> np.ndarray:
    return to_bits(normal(rng(seed, 6, 1000 + group), (N, K), 1.0), "f8e4m3")


# ----------------------------------------------------------------------------
# workload 7: mixture-of-experts decode step with 4-bit expert weights -- 16
# tokens routed to 8 experts each (128 rows) over 128 experts with the MoE
# layer's expert shape (N 2048, K 4096), bf16 activations and scales, int4
# weights with int4 zero points per 128-k group.
# ----------------------------------------------------------------------------
def moe_w4_counts(seed: int = DEFAULT_SEED, rows: int = 128, groups: int = 128) -> np.ndarray:
    """Rows per expert, Zipf(1.1)-skewed like the MoE layer's token counts."""
    return moe_counts(seed, tokens=rows, groups=groups, empty=8)


def moe_w4_expert(group: int, seed: int = DEFAULT_SEED, N: int = 2048, K: int = 4096, g: int = 128):
    """One expert: packed weight [N][K/2], bf16 scales [K/g][N], packed zero points [K/g][N/2]."""
    w = uint4(rng(seed, 7, 1000 + group), N, K)
    s = to_bits(uniform(rng(seed, 7, 3000 + group), (K // g, N), 0.001, 0.01), "bf16")
    z = uint4(rng(seed, 7, 5000 + group), K // g, N)
    return pack_u4(w), s, pack_u4(z)


def moe_w4_activations(seed: int = DEFAULT_SEED, rows: int = 128, K: int = 4096) -> np.ndarray:
    return to_bits(normal(rng(seed, 7, 0), (rows, K), 1.0), "bf16")
