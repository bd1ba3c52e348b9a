"""fp64 CPU oracle for the grouped / mixed-input / implicit-conv GEMM library.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline import this package; the library itself never does, and this package
imports nothing from the library.  The arithmetic lives in ``oracle.c`` (plain
C, fp64, OpenMP over output rows); this module builds it with gcc and marshals
numpy arrays into it.

Inputs are the stored element bytes: fp16 / bf16 bit patterns as ``uint16``
arrays, OCP fp8 E4M3 codes as ``uint8`` arrays ("f8e4m3", A and B of the fp8
GEMM only), uint4 tensors packed two per byte (even index in the low nibble).
Results are unrounded ``float64`` arrays; ``round_to`` rounds them (RNE) only
for bit-exact comparisons.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None

DTYPES = {"f16": 0, "bf16": 1, "f8e4m3": 2}

_d = ctypes.c_double
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build() -> pathlib.Path:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP)."""
    tmp = _LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Werror",
           str(_SRC), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        build()
    lib = ctypes.CDLL(str(_LIB_PATH))
    lib.ora_decode.argtypes = [_p, _i64, _i32, _p]
    lib.ora_decode.restype = None
    lib.ora_round.argtypes = [_p, _i64, _i32, _p]
    lib.ora_round.restype = None
    lib.ora_gemm.argtypes = [_i32, _i32, _i32, _p, _i64, _p, _i64, _p, _i64, _i32, _i32, _d, _d, _p, _i64]
    lib.ora_gemm.restype = ctypes.c_int
    lib.ora_dequant_w4.argtypes = [_i32, _i32, _p, _p, _p, _i32, _p]
    lib.ora_dequant_w4.restype = ctypes.c_int
    lib.ora_w4a16.argtypes = [_i32, _i32, _i32, _p, _i64, _p, _p, _p, _i32, _p]
    lib.ora_w4a16.restype = ctypes.c_int
    lib.ora_dequant_mixed.argtypes = [_i32, _i32, _p, _i32, _p, _i32, _p, _i32, _p]
    lib.ora_dequant_mixed.restype = ctypes.c_int
    lib.ora_mixed.argtypes = [_i32, _i32, _i32, _p, _i64, _i32, _p, _i32, _p, _p, _i32, _p]
    lib.ora_mixed.restype = ctypes.c_int
    lib.ora_conv2d_fprop.argtypes = [_i32] * 13 + [_p, _p, _p, _i32, _d, _d, _p]
    lib.ora_conv2d_fprop.restype = ctypes.c_int
    lib.ora_conv2d_dgrad.argtypes = [_i32] * 13 + [_p, _p, _p, _i32, _d, _d, _p]
    lib.ora_conv2d_wgrad.argtypes = [_i32] * 13 + [_p, _p, _p, _i32, _d, _d, _p]
    lib.ora_conv2d_wgrad.restype = ctypes.c_int
    lib.ora_conv2d_wgrad_grouped.argtypes = [_i32] * 14 + [_p, _p, _p, _i32, _d, _d, _p]
    lib.ora_conv2d_wgrad_grouped.restype = ctypes.c_int
    lib.ora_conv2d_dgrad.restype = ctypes.c_int
    lib.ora_prepack_w4.argtypes = [_i32, _i32, _p, _p]
    lib.ora_prepack_w4.restype = ctypes.c_int
    lib.ora_unprepack_w4.argtypes = [_i32, _i32, _p, _p]
    lib.ora_unprepack_w4.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """fp16 / bf16 bit patterns or fp8 E4M3 codes -> exact float64 values."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    _load().ora_decode(_ptr(b), b.size, DTYPES[dtype], _ptr(out))
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> fp16 / bf16 bit patterns, round to nearest even."""
    v = _c(x, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().ora_round(_ptr(v), v.size, DTYPES[dtype], _ptr(out))
    return out


def gemm(A, B, C=None, *, K=None, alpha=1.0, beta=0.0, dtype="f16", dtype_c=None) -> np.ndarray:
    """D = alpha * A B + beta * C for one problem.

    A: uint16 [M][lda] (row-major, K leading entries used), B: uint16 [N][ldb]
    (column-major B: row n of the array is column n of B), C: uint16 [M][ldc] or
    None.  For dtype "f8e4m3", A and B are uint8 codes and C is dtype_c
    (bf16 by default).  Returns float64 [M][N]."""
    if dtype == "f8e4m3" and dtype_c is None:
        dtype_c = "bf16"
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    M, lda = A.shape
    N, ldb = B.shape
    K = lda if K is None else K
    Cc = None if C is None else _c(C, np.uint16)
    ldc = 0 if Cc is None else Cc.shape[1]
    out = np.empty((M, N), np.float64)
    dc = DTYPES[dtype_c or dtype]
    rc = _load().ora_gemm(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(Cc), ldc, DTYPES[dtype], dc,
                          float(alpha), float(beta), _ptr(out), N)
    if rc:
        raise ValueError("ora_gemm rejected its arguments")
    return out


def dequant_w4(W, scales, zeros, N, K, group) -> np.ndarray:
    """Dequantised weights w[n][k] = (q - z) * s, float64 [N][K]."""
    W = _c(W, np.uint8)
    s = _c(scales, np.uint16)
    z = _c(zeros, np.uint8)
    out = np.empty((N, K), np.float64)
    if _load().ora_dequant_w4(N, K, _ptr(W), _ptr(s), _ptr(z), group, _ptr(out)):
        raise ValueError("ora_dequant_w4 rejected its arguments")
    return out


def w4a16(X, W, scales, zeros, N, K, group) -> np.ndarray:
    """Y = X W^T with uint4 W [N][K/2] packed, fp16 scales [K/g][N], uint4
    zeros [K/g][N/2] packed.  X: uint16 [M][ldx].  Returns float64 [M][N]."""
    X = _c(X, np.uint16)
    M, ldx = X.shape
    W = _c(W, np.uint8)
    s = _c(scales, np.uint16)
    z = _c(zeros, np.uint8)
    out = np.empty((M, N), np.float64)
    if _load().ora_w4a16(M, N, K, _ptr(X), ldx, _ptr(W), _ptr(s), _ptr(z), group, _ptr(out)):
        raise ValueError("ora_w4a16 rejected its arguments")
    return out


W4_SIGNED = {"uint4": 0, "int4": 1}


def dequant_mixed(W, scales, zeros, N, K, group, w_type="uint4", dtype="f16") -> np.ndarray:
    """Dequantised weights in the conversion mode the arguments select: scales None -> v(q); zeros None ->
    v(q) s; both -> (v(q) - v(z)) s, where v() reads a nibble as `w_type` ("uint4" or "int4", two's
    complement) and the scales are `dtype` ("f16" or "bf16") bit patterns.  float64 [N][K]."""
    W = _c(W, np.uint8)
    s = None if scales is None else _c(scales, np.uint16)
    z = None if zeros is None else _c(zeros, np.uint8)
    out = np.empty((N, K), np.float64)
    if _load().ora_dequant_mixed(N, K, _ptr(W), W4_SIGNED[w_type], _ptr(s), DTYPES[dtype], _ptr(z), group,
                                 _ptr(out)):
        raise ValueError("ora_dequant_mixed rejected its arguments")
    return out


def mixed(X, W, scales, zeros, N, K, group, w_type="uint4", dtype="f16") -> np.ndarray:
    """Y = X W^T with the weights of dequant_mixed; X [M][ldx] `dtype` bit patterns.  float64 [M][N]."""
    X = _c(X, np.uint16)
    M, ldx = X.shape
    W = _c(W, np.uint8)
    s = None if scales is None else _c(scales, np.uint16)
    z = None if zeros is None else _c(zeros, np.uint8)
    out = np.empty((M, N), np.float64)
    if _load().ora_mixed(M, N, K, _ptr(X), ldx, DTYPES[dtype], _ptr(W), W4_SIGNED[w_type], _ptr(s), _ptr(z), group,
                         _ptr(out)):
        raise ValueError("ora_mixed rejected its arguments")
    return out


def conv_out_size(H, R, pad, stride, dil):
    return (H + 2 * pad - dil * (R - 1) - 1) // stride + 1


def conv2d_fprop(x, w, *, pad=(0, 0), stride=(1, 1), dil=(1, 1), C_in=None, alpha=1.0, beta=0.0,
                 dtype="bf16", bias=None, act=None) -> np.ndarray:
    """Direct cross-correlation.  x uint16 [N][H][W][C] (NHWC), w uint16
    [K][R][S][C] (KRSC), C_in uint16 [N][P][Q][K] or None.  Returns float64
    [N][P][Q][K].

    Fused epilogue (the conv page's collective epilogue is only a template
    parameter; the reading here): bias uint16 [K] in the output type is added
    per output channel after alpha * acc + beta * C, then act = "relu" takes
    max(v, 0).  Both are applied to the unrounded fp64 value."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    N, H, Wd, C = x.shape
    K, R, S, C2 = w.shape
    assert C == C2
    P = conv_out_size(H, R, pad[0], stride[0], dil[0])
    Q = conv_out_size(Wd, S, pad[1], stride[1], dil[1])
    ci = None if C_in is None else _c(C_in, np.uint16)
    out = np.empty((N, P, Q, K), np.float64)
    rc = _load().ora_conv2d_fprop(N, H, Wd, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
                                  _ptr(x), _ptr(w), _ptr(ci), DTYPES[dtype], float(alpha), float(beta),
                                  _ptr(out))
    if rc:
        raise ValueError("ora_conv2d_fprop rejected its arguments")
    if bias is not None:
        b = decode(_c(bias, np.uint16), dtype)
        assert b.shape == (K,)
        out += b[None, None, None, :]
    if act == "relu":
        np.maximum(out, 0.0, out=out)
    elif act is not None:
        raise ValueError(f"unknown activation {act!r}")
    return out


def conv2d_dgrad(dy, w, H, W, *, pad=(0, 0), stride=(1, 1), dil=(1, 1), C_in=None, alpha=1.0, beta=0.0,
                 dtype="bf16") -> np.ndarray:
    """Data gradient of conv2d_fprop: dy uint16 [N][P][Q][K], w uint16 [K][R][S][C] (KRSC), the forward
    input's spatial size H, W; C_in uint16 [N][H][W][C] or None.  Returns float64 [N][H][W][C]."""
    dy = _c(dy, np.uint16)
    w = _c(w, np.uint16)
    N, P, Q, K = dy.shape
    K2, R, S, C = w.shape
    assert K == K2
    assert P == conv_out_size(H, R, pad[0], stride[0], dil[0]) and Q == conv_out_size(W, S, pad[1], stride[1], dil[1])
    ci = None if C_in is None else _c(C_in, np.uint16)
    out = np.empty((N, H, W, C), np.float64)
    rc = _load().ora_conv2d_dgrad(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
                                  _ptr(dy), _ptr(w), _ptr(ci), DTYPES[dtype], float(alpha), float(beta),
                                  _ptr(out))
    if rc:
        raise ValueError("ora_conv2d_dgrad rejected its arguments")
    return out


def conv2d_wgrad(x, dy, R, S, *, pad=(0, 0), stride=(1, 1), dil=(1, 1), C_in=None, alpha=1.0, beta=0.0,
                 dtype="bf16", groups=1) -> np.ndarray:
    """Filter gradient of conv2d_fprop: x uint16 [N][H][W][C], dy uint16 [N][P][Q][K], the filter size R, S;
    C_in uint16 [K][R][S][C/groups] or None.  With groups, output channel k sees only the input channels of its
    group.  Returns float64 [K][R][S][C/groups]."""
    x = _c(x, np.uint16)
    dy = _c(dy, np.uint16)
    N, H, W, C = x.shape
    N2, P, Q, K = dy.shape
    assert N == N2
    assert P == conv_out_size(H, R, pad[0], stride[0], dil[0]) and Q == conv_out_size(W, S, pad[1], stride[1], dil[1])
    ci = None if C_in is None else _c(C_in, np.uint16)
    out = np.empty((K, R, S, C // groups), np.float64)
    rc = _load().ora_conv2d_wgrad_grouped(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0],
                                          dil[1], groups, _ptr(x), _ptr(dy), _ptr(ci), DTYPES[dtype], float(alpha),
                                          float(beta), _ptr(out))
    if rc:
        raise ValueError("ora_conv2d_wgrad rejected its arguments")
    return out


def prepack_w4(W, N, K) -> np.ndarray:
    """The library's weight permutation applied to packed uint4 W [N][K/2];
    returns N*K/2 bytes."""
    W = _c(W, np.uint8)
    out = np.empty(N * K // 2, np.uint8)
    if _load().ora_prepack_w4(N, K, _ptr(W), _ptr(out)):
        raise ValueError("prepack needs N % 16 == 0 and K % 128 == 0")
    return out


def unprepack_w4(pp, N, K) -> np.ndarray:
    """Inverse permutation: N*K/2 prepacked bytes -> packed W [N][K/2]."""
    pp = _c(pp, np.uint8)
    out = np.empty((N, K // 2), np.uint8)
    if _load().ora_unprepack_w4(N, K, _ptr(pp), _ptr(out)):
        raise ValueError("prepack needs N % 16 == 0 and K % 128 == 0")
    return out
