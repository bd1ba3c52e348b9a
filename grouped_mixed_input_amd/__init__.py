"""grouped_mixed_input_amd -- grouped, mixed-input (W4A16) and implicit-conv GEMM
for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libgmi.so`` (declared in
``include/gmi.h``).  Functions here only marshal torch tensors into device
pointers, sizes and the current HIP stream; every step of the computation runs
in the library's HIP kernels.  There is no fallback: if ``libgmi.so`` has not
been built, importing the binding's functions raises.
"""
from __future__ import annotations

import ctypes
import pathlib

import torch

_PKG = pathlib.Path(__file__).resolve().parent
LIB_PATH = _PKG / "libgmi.so"

GMI_OK, GMI_ERR_INVALID_ARG, GMI_ERR_UNSUPPORTED, GMI_ERR_MISALIGNED, GMI_ERR_WORKSPACE, GMI_ERR_HIP = range(6)
STATUS_NAMES = ["GMI_OK", "GMI_ERR_INVALID_ARG", "GMI_ERR_UNSUPPORTED", "GMI_ERR_MISALIGNED", "GMI_ERR_WORKSPACE",
                "GMI_ERR_HIP"]
GMI_F16, GMI_BF16, GMI_F8E4M3 = 0, 1, 2
_DT = {torch.float16: GMI_F16, torch.bfloat16: GMI_BF16, torch.float8_e4m3fn: GMI_F8E4M3}


class GmiError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {message}")


class Problem(ctypes.Structure):
    """Mirror of gmi_problem."""
    _fields_ = [("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64), ("ldd", ctypes.c_int64),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p)]


_lib = None
_i32, _i64, _f32, _p, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libgmi.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                           "python -m grouped_mixed_input_amd.build")
    L = ctypes.CDLL(str(LIB_PATH))
    L.gmi_last_error.restype = ctypes.c_char_p
    L.gmi_last_error.argtypes = []
    L.gmi_workspace_bytes.restype = _sz
    L.gmi_workspace_bytes.argtypes = [_i32]
    L.gmi_gemm_grouped.restype = ctypes.c_int
    L.gmi_gemm_grouped.argtypes = [ctypes.POINTER(Problem), _i32, ctypes.c_int, _f32, _f32, _p, _sz, _p]
    L.gmi_gemm_grouped_offsets.restype = ctypes.c_int
    L.gmi_gemm_grouped_offsets.argtypes = [_i32, _p, _i32, _i32, _i32, _p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64,
                                           ctypes.c_int, _f32, _f32, _p, _sz, _p]
    L.gmi_gemm_grouped_offsets_noalloc.restype = ctypes.c_int
    L.gmi_gemm_grouped_offsets_noalloc.argtypes = [_i32, _p, _i32, _i32, _i32, _p, _i64, _p, _i64, _i64, _p, _i64, _p,
                                                   _i64, ctypes.c_int, _f32, _f32, _p]
    L.gmi_gemm_ptr_array.restype = ctypes.c_int
    L.gmi_gemm_ptr_array.argtypes = [_i32, _i32, _i32, _i32, _p, _i64, _p, _i64, _p, _i64, _p, _i64, ctypes.c_int,
                                     _f32, _f32, _p]
    L.gmi_prepack_w4_bytes.restype = _sz
    L.gmi_prepack_w4_bytes.argtypes = [_i32, _i32]
    L.gmi_prepack_w4.restype = ctypes.c_int
    L.gmi_prepack_w4.argtypes = [_p, _i32, _i32, _p, _p]
    L.gmi_gemm_w4a16.restype = ctypes.c_int
    L.gmi_gemm_w4a16.argtypes = [_i32, _i32, _i32, _p, _i64, _p, _p, _p, _i32, _p, _i64, _p, _sz, _p]
    L.gmi_gemm_mixed.restype = ctypes.c_int
    L.gmi_gemm_mixed.argtypes = [_i32, _i32, _i32, ctypes.c_int, _p, _i64, _p, ctypes.c_int, _p, _p, _i32, _p, _i64,
                                 _p, _sz, _p]
    L.gmi_gemm_mixed_grouped.restype = ctypes.c_int
    L.gmi_gemm_mixed_grouped.argtypes = [_i32, _p, _i32, _i32, _i32, ctypes.c_int, _p, _i64, _p, _i64, ctypes.c_int,
                                         _p, _i64, _p, _i64, _i32, _p, _i64, _p]
    L.gmi_conv2d_fprop_implicit_fused.restype = ctypes.c_int
    L.gmi_conv2d_fprop_implicit_fused.argtypes = [_i32] * 13 + [_p, _p, _p, _p, _p, ctypes.c_int, _f32, _f32,
                                                               ctypes.c_int, _p]
    L.gmi_conv2d_dgrad_workspace_bytes.restype = _sz
    L.gmi_conv2d_dgrad_workspace_bytes.argtypes = [_i32] * 4
    L.gmi_conv2d_dgrad_implicit.restype = ctypes.c_int
    L.gmi_conv2d_dgrad_implicit.argtypes = [_i32] * 13 + [_p, _p, _p, _p, ctypes.c_int, _f32, _f32, _p, _sz, _p]
    L.gmi_conv2d_wgrad_workspace_bytes.restype = _sz
    L.gmi_conv2d_wgrad_workspace_bytes.argtypes = [_i32] * 14
    L.gmi_conv2d_wgrad_implicit.restype = ctypes.c_int
    L.gmi_conv2d_wgrad_implicit.argtypes = [_i32] * 14 + [_p, _p, _p, _p, ctypes.c_int, _f32, _f32, _p, _sz, _p]
    L.gmi_w4a16_workspace_bytes.restype = _sz
    L.gmi_w4a16_workspace_bytes.argtypes = [_i32, _i32, _i32]
    L.gmi_conv2d_fprop_implicit.restype = ctypes.c_int
    L.gmi_conv2d_fprop_implicit.argtypes = [_i32] * 13 + [_p, _p, _p, _p, ctypes.c_int, _f32, _f32, _p]
    L.gmi_time_next_gemm.restype = ctypes.c_int
    L.gmi_time_next_gemm.argtypes = [_p, _p]
    _lib = L
    return L


def _check(status: int) -> None:
    if status != GMI_OK:
        raise GmiError(status, lib().gmi_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit stride along its rows")
    return t.stride(0)


# ---------------------------------------------------------------- grouped
def time_next_gemm(start, stop) -> None:
    """Let the next GEMM kernel launched on this thread (grouped, grouped-offsets or pointer-array call) record
    `start` and `stop` around itself, so start.elapsed_time(stop) is that kernel's execution time.  Both are
    torch.cuda.Event(enable_timing=True) objects that have been recorded once (torch creates the HIP event on
    its first record); None, None cancels a pending request."""
    if start is None and stop is None:
        _check(lib().gmi_time_next_gemm(None, None))
        return
    _check(lib().gmi_time_next_gemm(start.cuda_event, stop.cuda_event))


def workspace_bytes(count: int) -> int:
    return lib().gmi_workspace_bytes(count)


def make_problems(As, Bs, Cs, Ds) -> "ctypes.Array":
    """gmi_problem array from lists of tensors: A [M][K], B [N][K] (column-major
    B, i.e. row n of the tensor is column n), C / D [M][N] (C may be None)."""
    arr = (Problem * len(As))()
    for i, (a, b, c, d) in enumerate(zip(As, Bs, Cs, Ds)):
        M, N = d.shape
        K = a.shape[1]
        arr[i] = Problem(M, N, K, _ld(a), _ld(b), _ld(c) if c is not None else 0, _ld(d),
                         _ptr(a), _ptr(b), _ptr(c), _ptr(d))
    return arr


def gemm_grouped(As, Bs, Cs, Ds, alpha=1.0, beta=0.0, workspace=None, stream=None):
    """D_g = alpha A_g B_g + beta C_g for every g, in one launch.  The element type is that of A
    (float8_e4m3fn A and B give bfloat16 C and D)."""
    dt = _DT[As[0].dtype]
    probs = make_problems(As, Bs, Cs if Cs is not None else [None] * len(As), Ds)
    need = workspace_bytes(len(As))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=Ds[0].device)
    _check(lib().gmi_gemm_grouped(probs, len(As), dt, alpha, beta, workspace.data_ptr(), workspace.numel(),
                                  _stream(stream)))
    return Ds


def gemm_grouped_raw(problems, count, dtype, alpha, beta, workspace, stream=None):
    """Call with a prepared gmi_problem array (no per-call marshalling)."""
    _check(lib().gmi_gemm_grouped(problems, count, dtype, alpha, beta, workspace.data_ptr(), workspace.numel(),
                                  _stream(stream)))


def _offsets_args(offsets, A, B, D):
    if B.dim() != 3 or B.stride(2) != 1 or B.stride(1) < B.shape[2]:
        raise ValueError("B must be [groups][N][K] with unit stride along K")
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous int32 vector")
    count = B.shape[0]
    if offsets.numel() != count + 1:
        raise ValueError(f"offsets has {offsets.numel()} entries, {count + 1} expected")
    rows, N = D.shape
    K = A.shape[1]
    if A.shape[0] != rows or B.shape[1] != N or B.shape[2] != K:
        raise ValueError("A [rows][K], B [groups][N][K] and D [rows][N] disagree")
    return count, rows, N, K


def gemm_grouped_offsets(offsets: torch.Tensor, A: torch.Tensor, B: torch.Tensor, D: torch.Tensor,
                         C: torch.Tensor | None = None, alpha=1.0, beta=0.0, workspace=None, stream=None):
    """Grouped GEMM with device-held group sizes: group g owns rows offsets[g] .. offsets[g+1] of A [rows][K]
    and D [rows][N] (and C) and multiplies them by B[g] (B is [groups][N][K], each B[g] column-major K x N).
    `offsets` is a device int32 tensor of groups + 1 entries; nothing is read back to the host."""
    count, rows, N, K = _offsets_args(offsets, A, B, D)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(count), dtype=torch.uint8, device=D.device)
    _check(lib().gmi_gemm_grouped_offsets(count, offsets.data_ptr(), rows, N, K, A.data_ptr(), _ld(A),
                                          B.data_ptr(), B.stride(1), B.stride(0), _ptr(C),
                                          _ld(C) if C is not None else 0, D.data_ptr(), _ld(D), _DT[A.dtype],
                                          alpha, beta, workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return D


def gemm_grouped_offsets_noalloc(offsets: torch.Tensor, A: torch.Tensor, B: torch.Tensor, D: torch.Tensor,
                                 C: torch.Tensor | None = None, alpha=1.0, beta=0.0, stream=None):
    """gemm_grouped_offsets without a workspace: the library keeps the group table in its own static device
    array (at most 1024 groups); calls that overlap on one device race on that array."""
    count, rows, N, K = _offsets_args(offsets, A, B, D)
    _check(lib().gmi_gemm_grouped_offsets_noalloc(count, offsets.data_ptr(), rows, N, K, A.data_ptr(), _ld(A),
                                                  B.data_ptr(), B.stride(1), B.stride(0), _ptr(C),
                                                  _ld(C) if C is not None else 0, D.data_ptr(), _ld(D), _DT[A.dtype],
                                                  alpha, beta, _stream(stream)))
    return D


# ---------------------------------------------------------------- ptr-array
def pointer_array(tensors, device) -> torch.Tensor:
    """Device array (int64) of the tensors' device addresses."""
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


def gemm_ptr_array(L, M, N, K, A_ptrs, lda, B_ptrs, ldb, C_ptrs, ldc, D_ptrs, ldd, dtype, alpha=1.0, beta=0.0,
                   stream=None):
    """Pointer-array GEMM; *_ptrs are device int64 tensors of L addresses."""
    _check(lib().gmi_gemm_ptr_array(L, M, N, K, _ptr(A_ptrs), lda, _ptr(B_ptrs), ldb, _ptr(C_ptrs), ldc,
                                    _ptr(D_ptrs), ldd, _DT[dtype] if dtype in _DT else dtype, alpha, beta,
                                    _stream(stream)))


# ---------------------------------------------------------------- W4A16
def prepack_w4(w_u4: torch.Tensor, N: int, K: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Prepack a uint4 weight stored [N][K/2] (uint8) into the kernels' order."""
    if out is None:
        out = torch.empty(lib().gmi_prepack_w4_bytes(N, K), dtype=torch.uint8, device=w_u4.device)
    _check(lib().gmi_prepack_w4(w_u4.data_ptr(), N, K, out.data_ptr(), _stream(stream)))
    return out


def w4a16_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().gmi_w4a16_workspace_bytes(M, N, K)


def gemm_w4a16(X: torch.Tensor, w_prepacked: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
               group_size: int, N: int, Y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """Y = X W^T with X fp16 [M][K], scales fp16 [K/g][N], zeros uint8 [K/g][N/2].  `workspace` (a device
    byte tensor of at least w4a16_workspace_bytes(M, N, K)) enables the split-K path; pass an empty tensor
    (numel 0) to run unsplit.  With None, one is allocated for this call."""
    M, K = X.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    if workspace is None:
        need = w4a16_workspace_bytes(M, N, K)
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    _check(lib().gmi_gemm_w4a16(M, N, K, X.data_ptr(), _ld(X), w_prepacked.data_ptr(), scales.data_ptr(),
                                zeros.data_ptr(), group_size, Y.data_ptr(), _ld(Y),
                                workspace.data_ptr() if workspace.numel() else None, workspace.numel(),
                                _stream(stream)))
    return Y


W4_TYPES = {"uint4": 0, "int4": 1}


def gemm_mixed(X: torch.Tensor, w_prepacked: torch.Tensor, scales: torch.Tensor | None, zeros: torch.Tensor | None,
               group_size: int, N: int, w_type: str = "uint4", Y: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X W^T in any conversion mode: scales None is the direct conversion, zeros None the conversion
    without zero point.  X, scales and Y share one type (float16 or bfloat16); `w_type` is "uint4" or
    "int4" (zero points, if any, have the same type).  Workspace as for gemm_w4a16."""
    M, K = X.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=X.dtype, device=X.device)
    if workspace is None:
        workspace = torch.empty(w4a16_workspace_bytes(M, N, K), dtype=torch.uint8, device=X.device)
    _check(lib().gmi_gemm_mixed(M, N, K, _DT[X.dtype], X.data_ptr(), _ld(X), w_prepacked.data_ptr(),
                                W4_TYPES[w_type], _ptr(scales), _ptr(zeros), group_size, Y.data_ptr(), _ld(Y),
                                workspace.data_ptr() if workspace.numel() else None, workspace.numel(),
                                _stream(stream)))
    return Y


def gemm_mixed_grouped(offsets: torch.Tensor, X: torch.Tensor, w_prepacked: torch.Tensor,
                       scales: torch.Tensor | None, zeros: torch.Tensor | None, group_size: int, N: int,
                       w_type: str = "uint4", Y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Per-group Y_g = X_g W_g^T (mixture of experts): rows offsets[g] .. offsets[g+1] of X [rows][K] and Y
    [rows][N]; w_prepacked [groups][N*K/2] (each row a gmi_prepack_w4 output), scales [groups][K/g][N] or
    None, zeros [groups][K/g][N/2] or None.  `offsets` is a device int32 tensor of groups + 1 entries."""
    rows, K = X.shape
    count = w_prepacked.shape[0]
    if offsets.dtype != torch.int32 or offsets.numel() != count + 1 or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous int32 vector of groups + 1 entries")
    if Y is None:
        Y = torch.empty((rows, N), dtype=X.dtype, device=X.device)
    _check(lib().gmi_gemm_mixed_grouped(count, offsets.data_ptr(), rows, N, K, _DT[X.dtype], X.data_ptr(), _ld(X),
                                        w_prepacked.data_ptr(), w_prepacked.stride(0), W4_TYPES[w_type],
                                        _ptr(scales), scales.stride(0) if scales is not None else 0, _ptr(zeros),
                                        zeros.stride(0) if zeros is not None else 0, group_size, Y.data_ptr(),
                                        _ld(Y), _stream(stream)))
    return Y


# ---------------------------------------------------------------- conv
def conv_out_size(H, R, pad, stride, dil):
    return (H + 2 * pad - dil * (R - 1) - 1) // stride + 1


ACTIVATIONS = {None: 0, "none": 0, "relu": 1}


def conv2d_fprop(x: torch.Tensor, w: torch.Tensor, pad=(0, 0), stride=(1, 1), dil=(1, 1), c_in=None, alpha=1.0,
                 beta=0.0, y: torch.Tensor | None = None, stream=None, bias: torch.Tensor | None = None,
                 act: str | None = None) -> torch.Tensor:
    """Implicit-GEMM cross-correlation: x NHWC, w KRSC -> y NPQK.  With `bias` (K elements of x's type) or
    `act` ("relu"), the fused entry point adds the bias per output channel and applies the activation before
    the output is rounded."""
    N, H, W, C = x.shape
    K, R, S, _ = w.shape
    if y is None:
        P = conv_out_size(H, R, pad[0], stride[0], dil[0])
        Q = conv_out_size(W, S, pad[1], stride[1], dil[1])
        y = torch.empty((N, max(P, 0), max(Q, 0), K), dtype=x.dtype, device=x.device)
    if bias is None and act in (None, "none"):
        _check(lib().gmi_conv2d_fprop_implicit(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0],
                                               dil[1], x.data_ptr(), w.data_ptr(), _ptr(c_in), y.data_ptr(),
                                               _DT[x.dtype], alpha, beta, _stream(stream)))
    else:
        if bias is not None and (bias.numel() != K or bias.dtype != x.dtype):
            raise ValueError("bias must hold K elements of the activation's type")
        _check(lib().gmi_conv2d_fprop_implicit_fused(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1],
                                                     dil[0], dil[1], x.data_ptr(), w.data_ptr(), _ptr(c_in),
                                                     _ptr(bias), y.data_ptr(), _DT[x.dtype], alpha, beta,
                                                     ACTIVATIONS[act], _stream(stream)))
    return y


def conv2d_dgrad(dy: torch.Tensor, w: torch.Tensor, H: int, W: int, pad=(0, 0), dil=(1, 1), c_in=None, alpha=1.0,
                 beta=0.0, dx: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stride=(1, 1),
                 stream=None) -> torch.Tensor:
    """Data gradient of conv2d_fprop: dy NPQK, w KRSC, the forward input's H, W -> dx NHWC (strides 1 .. 8 in
    each dimension)."""
    N, P, Q, K = dy.shape
    K2, R, S, C = w.shape
    if K2 != K:
        raise ValueError("dy and w disagree on K")
    if dx is None:
        dx = torch.empty((N, H, W, C), dtype=dy.dtype, device=dy.device)
    if workspace is None:
        workspace = torch.empty(lib().gmi_conv2d_dgrad_workspace_bytes(C, K, R, S), dtype=torch.uint8,
                                device=dy.device)
    _check(lib().gmi_conv2d_dgrad_implicit(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
                                           dy.data_ptr(), w.data_ptr(), _ptr(c_in), dx.data_ptr(), _DT[dy.dtype],
                                           alpha, beta, workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return dx


def conv2d_wgrad_workspace_bytes(x_shape, dy_shape, R, S, pad=(0, 0), stride=(1, 1), dil=(1, 1), groups=1) -> int:
    N, H, W, C = x_shape
    K = dy_shape[3]
    return lib().gmi_conv2d_wgrad_workspace_bytes(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0],
                                                  dil[1], groups)


def conv2d_wgrad(x: torch.Tensor, dy: torch.Tensor, R: int, S: int, pad=(0, 0), stride=(1, 1), dil=(1, 1),
                 c_in=None, alpha=1.0, beta=0.0, dw: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, groups: int = 1, stream=None) -> torch.Tensor:
    """Filter gradient of conv2d_fprop: x NHWC, dy NPQK, the filter size R, S -> dw K x R x S x C/groups."""
    N, H, W, C = x.shape
    K = dy.shape[3]
    if dw is None:
        dw = torch.empty((K, R, S, C // groups), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.empty(conv2d_wgrad_workspace_bytes(x.shape, dy.shape, R, S, pad, stride, dil, groups),
                                dtype=torch.uint8, device=x.device)
    _check(lib().gmi_conv2d_wgrad_implicit(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
                                           groups, x.data_ptr(), dy.data_ptr(), _ptr(c_in), dw.data_ptr(),
                                           _DT[x.dtype],
                                           alpha, beta, workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return dw
