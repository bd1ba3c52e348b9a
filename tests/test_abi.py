"""The C ABI without a GPU: libgmi.so loads, exports every function that
include/gmi.h declares, and rejects each invalid request with its status and
a message before any HIP call (validation is host code that runs first)."""
import ctypes
import pathlib
import re

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def gmi():
    import grouped_mixed_input_amd as g

    if not g.LIB_PATH.exists():
        from grouped_mixed_input_amd import build

        build.build()
    g.lib()
    return g


def declared_functions():
    text = (ROOT / "include" / "gmi.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gmi_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["gmi_gemm_grouped", "gmi_gemm_ptr_array", "gmi_prepack_w4", "gmi_gemm_w4a16",
                 "gmi_conv2d_fprop_implicit", "gmi_workspace_bytes", "gmi_prepack_w4_bytes", "gmi_last_error",
                 "gmi_gemm_grouped_offsets", "gmi_w4a16_workspace_bytes", "gmi_gemm_mixed",
                 "gmi_gemm_mixed_grouped", "gmi_conv2d_dgrad_implicit", "gmi_conv2d_dgrad_workspace_bytes",
                 "gmi_conv2d_wgrad_implicit", "gmi_conv2d_wgrad_workspace_bytes", "gmi_conv2d_fprop_implicit_fused",
                 "gmi_gemm_grouped_offsets_noalloc", "gmi_time_next_gemm"]:
        assert want in names


def test_library_exports_every_declared_symbol(gmi):
    lib = ctypes.CDLL(str(gmi.LIB_PATH))
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_size_helpers(gmi):
    L = gmi.lib()
    assert L.gmi_workspace_bytes(0) == 256
    assert L.gmi_workspace_bytes(128) == 256 + 80 * 128
    assert L.gmi_workspace_bytes(-1) == 0
    assert L.gmi_prepack_w4_bytes(8192, 8192) == 8192 * 8192 // 2
    assert L.gmi_prepack_w4_bytes(-1, 4) == 0


A16 = 0x10000  # fake, 16-byte aligned device addresses: never dereferenced by a rejected call


def _grouped(gmi, probs, dtype=0, beta=0.0, ws=A16 * 64, ws_bytes=1 << 20):
    arr = (gmi.Problem * len(probs))(*probs) if probs else None
    st = gmi.lib().gmi_gemm_grouped(arr, len(probs), dtype, 1.0, beta, ws, ws_bytes, None)
    return st, gmi.lib().gmi_last_error().decode()


def P(gmi, M=64, N=64, K=64, lda=64, ldb=64, ldc=64, ldd=64, A=A16, B=A16 * 2, C=A16 * 3, D=A16 * 4):
    return gmi.Problem(M, N, K, lda, ldb, ldc, ldd, A, B, C, D)


def test_grouped_validation(gmi):
    ok_ws = 1 << 20
    assert _grouped(gmi, [P(gmi, M=-1)])[0] == gmi.GMI_ERR_INVALID_ARG
    st, msg = _grouped(gmi, [P(gmi, lda=32)])
    assert st == gmi.GMI_ERR_INVALID_ARG and "leading dimension" in msg
    assert _grouped(gmi, [P(gmi, A=None)])[0] == gmi.GMI_ERR_INVALID_ARG
    assert _grouped(gmi, [P(gmi, C=None)], beta=1.0)[0] == gmi.GMI_ERR_INVALID_ARG
    assert _grouped(gmi, [P(gmi, A=A16 + 8)])[0] == gmi.GMI_ERR_MISALIGNED
    assert _grouped(gmi, [P(gmi, lda=68)])[0] == gmi.GMI_ERR_MISALIGNED
    assert _grouped(gmi, [P(gmi, ldc=60, C=A16 * 3)], beta=0.5)[0] == gmi.GMI_ERR_INVALID_ARG
    assert _grouped(gmi, [P(gmi)], dtype=7)[0] == gmi.GMI_ERR_UNSUPPORTED
    assert _grouped(gmi, [P(gmi, K=40, lda=64, ldb=64)], dtype=2)[0] == gmi.GMI_ERR_UNSUPPORTED
    st, msg = _grouped(gmi, [P(gmi), P(gmi)], ws_bytes=100)
    assert st == gmi.GMI_ERR_WORKSPACE and "workspace" in msg
    assert _grouped(gmi, [P(gmi)], ws=0, ws_bytes=ok_ws)[0] == gmi.GMI_ERR_WORKSPACE
    assert _grouped(gmi, [P(gmi)], ws=A16 + 4)[0] == gmi.GMI_ERR_MISALIGNED
    # negative count / NULL table
    assert gmi.lib().gmi_gemm_grouped(None, -1, 0, 1.0, 0.0, A16, ok_ws, None) == gmi.GMI_ERR_INVALID_ARG
    assert gmi.lib().gmi_gemm_grouped(None, 2, 0, 1.0, 0.0, A16, ok_ws, None) == gmi.GMI_ERR_INVALID_ARG


def test_grouped_empty_requests_launch_nothing(gmi):
    # zero problems, or only empty ones with NULL pointers: OK without a GPU call
    assert gmi.lib().gmi_gemm_grouped(None, 0, 0, 1.0, 0.0, None, 0, None) == gmi.GMI_OK
    empty = [P(gmi, M=0, A=None, B=None, C=None, D=None), P(gmi, N=0, A=None, B=None, C=None, D=None)]
    assert _grouped(gmi, empty, ws=0, ws_bytes=0)[0] == gmi.GMI_OK


def _offs(gmi, count=4, offsets=A16 * 5, rows=256, N=64, K=64, A=A16, lda=64, B=A16 * 2, ldb=64, stride_b=64 * 64,
          C=None, ldc=64, D=A16 * 4, ldd=64, dt=1, beta=0.0, ws=A16 * 64, ws_bytes=1 << 20):
    st = gmi.lib().gmi_gemm_grouped_offsets(count, offsets, rows, N, K, A, lda, B, ldb, stride_b, C, ldc, D, ldd, dt,
                                            1.0, beta, ws, ws_bytes, None)
    return st, gmi.lib().gmi_last_error().decode()


def test_grouped_offsets_validation(gmi):
    bad = gmi.GMI_ERR_INVALID_ARG
    for kw in (dict(count=-1), dict(rows=-2), dict(N=-1), dict(K=-5), dict(offsets=None), dict(A=None),
               dict(D=None), dict(beta=0.5), dict(lda=32), dict(ldd=56), dict(stride_b=-64)):
        assert _offs(gmi, **kw)[0] == bad, kw
    st, msg = _offs(gmi, count=1025)
    assert st == gmi.GMI_ERR_UNSUPPORTED and "1024" in msg
    assert _offs(gmi, dt=9)[0] == gmi.GMI_ERR_UNSUPPORTED
    assert _offs(gmi, dt=2, stride_b=64 * 64 + 8)[0] == gmi.GMI_ERR_UNSUPPORTED  # fp8 expert stride
    assert _offs(gmi, dt=2, K=40, lda=48, ldb=48)[0] == gmi.GMI_ERR_UNSUPPORTED
    for kw in (dict(offsets=A16 + 2), dict(A=A16 + 8), dict(stride_b=64 * 64 + 4), dict(lda=68),
               dict(ws=A16 + 4)):
        assert _offs(gmi, **kw)[0] == gmi.GMI_ERR_MISALIGNED, kw
    st, msg = _offs(gmi, ws_bytes=256 + 80 * 4 - 1)
    assert st == gmi.GMI_ERR_WORKSPACE and "workspace" in msg
    assert _offs(gmi, ws=0)[0] == gmi.GMI_ERR_WORKSPACE
    # nothing to do: no groups, no rows or no columns -- OK without a GPU call
    for kw in (dict(count=0), dict(rows=0), dict(N=0)):
        assert _offs(gmi, offsets=None, A=None, B=None, D=None, ws=0, ws_bytes=0, **kw)[0] == gmi.GMI_OK, kw


def test_grouped_offsets_noalloc_validation(gmi):
    # the allocation-free call runs the same checks before it looks anything up on a device; its table holds
    # at most 1024 groups
    L = gmi.lib()

    def noalloc(count=4, offsets=A16 * 5, A=A16, lda=64, dt=1):
        st = L.gmi_gemm_grouped_offsets_noalloc(count, offsets, 256, 64, 64, A, lda, A16 * 2, 64, 64 * 64, None, 64,
                                                A16 * 4, 64, dt, 1.0, 0.0, None)
        return st, L.gmi_last_error().decode()

    st, msg = noalloc(count=1025)
    assert st == gmi.GMI_ERR_UNSUPPORTED and "1024" in msg and "noalloc" in msg
    assert noalloc(count=-1)[0] == gmi.GMI_ERR_INVALID_ARG
    assert noalloc(offsets=None)[0] == gmi.GMI_ERR_INVALID_ARG
    assert noalloc(A=A16 + 8)[0] == gmi.GMI_ERR_MISALIGNED
    assert noalloc(lda=32)[0] == gmi.GMI_ERR_INVALID_ARG
    assert noalloc(dt=9)[0] == gmi.GMI_ERR_UNSUPPORTED
    assert noalloc(count=0, offsets=None, A=None)[0] == gmi.GMI_OK


def _ptr(gmi, L=2, M=64, N=64, K=64, A=A16, lda=64, B=A16, ldb=64, C=None, ldc=64, D=A16, ldd=64, dt=1, beta=0.0):
    return gmi.lib().gmi_gemm_ptr_array(L, M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dt, 1.0, beta, None)


def test_ptr_array_validation(gmi):
    assert _ptr(gmi, L=-1) == gmi.GMI_ERR_INVALID_ARG
    assert _ptr(gmi, K=-3) == gmi.GMI_ERR_INVALID_ARG
    assert _ptr(gmi, dt=5) == gmi.GMI_ERR_UNSUPPORTED
    assert _ptr(gmi, A=None) == gmi.GMI_ERR_INVALID_ARG
    assert _ptr(gmi, beta=1.0) == gmi.GMI_ERR_INVALID_ARG  # C required when beta != 0
    assert _ptr(gmi, ldb=56) == gmi.GMI_ERR_INVALID_ARG
    assert _ptr(gmi, ldd=72 + 4) == gmi.GMI_ERR_MISALIGNED
    assert _ptr(gmi, A=A16 + 4) == gmi.GMI_ERR_MISALIGNED
    # fp8: K and the A / B leading dimensions must be multiples of 16
    assert _ptr(gmi, dt=2, K=72, lda=80, ldb=80) == gmi.GMI_ERR_UNSUPPORTED
    assert _ptr(gmi, dt=2, K=64, lda=72, ldb=64) == gmi.GMI_ERR_UNSUPPORTED
    assert _ptr(gmi, L=0, A=None, B=None, D=None) == gmi.GMI_OK


def test_prepack_validation(gmi):
    L = gmi.lib()
    assert L.gmi_prepack_w4(A16, -16, 128, A16 * 8, None) == gmi.GMI_ERR_INVALID_ARG
    assert L.gmi_prepack_w4(A16, 24, 128, A16 * 8, None) == gmi.GMI_ERR_UNSUPPORTED
    assert L.gmi_prepack_w4(A16, 16, 192, A16 * 8, None) == gmi.GMI_ERR_UNSUPPORTED
    assert L.gmi_prepack_w4(None, 16, 128, A16 * 8, None) == gmi.GMI_ERR_INVALID_ARG
    assert L.gmi_prepack_w4(A16 + 2, 16, 128, A16 * 8, None) == gmi.GMI_ERR_MISALIGNED
    assert L.gmi_prepack_w4(A16, 16, 128, A16 + 512, None) == gmi.GMI_ERR_INVALID_ARG  # overlap
    assert L.gmi_prepack_w4(None, 0, 128, None, None) == gmi.GMI_OK


def _w4(gmi, M=16, N=64, K=256, X=A16, ldx=256, W=A16 * 2, S=A16 * 3, Z=A16 * 4, g=128, Y=A16 * 5, ldy=64, ws=None,
        ws_bytes=0):
    return gmi.lib().gmi_gemm_w4a16(M, N, K, X, ldx, W, S, Z, g, Y, ldy, ws, ws_bytes, None)


def test_w4a16_validation(gmi):
    assert _w4(gmi, M=-1) == gmi.GMI_ERR_INVALID_ARG
    assert _w4(gmi, N=24) == gmi.GMI_ERR_UNSUPPORTED
    assert _w4(gmi, K=200, ldx=200) == gmi.GMI_ERR_UNSUPPORTED
    assert _w4(gmi, g=0) == gmi.GMI_ERR_INVALID_ARG
    assert _w4(gmi, g=96) == gmi.GMI_ERR_INVALID_ARG  # K % g != 0
    assert _w4(gmi, K=384, ldx=384, g=192) == gmi.GMI_ERR_UNSUPPORTED  # neither K nor a multiple of 128
    assert _w4(gmi, Z=None) == gmi.GMI_ERR_INVALID_ARG  # zero points required
    assert _w4(gmi, S=None) == gmi.GMI_ERR_INVALID_ARG
    assert _w4(gmi, ldx=128) == gmi.GMI_ERR_INVALID_ARG
    assert _w4(gmi, ldy=60) == gmi.GMI_ERR_INVALID_ARG
    assert _w4(gmi, ldy=68) == gmi.GMI_ERR_MISALIGNED
    assert _w4(gmi, S=A16 + 2) == gmi.GMI_ERR_MISALIGNED
    assert _w4(gmi, M=0, X=None, W=None, S=None, Z=None, Y=None) == gmi.GMI_OK
    # a workspace that would enable the split must be 16-byte aligned
    need = gmi.lib().gmi_w4a16_workspace_bytes(128, 8192, 8192)
    assert _w4(gmi, M=128, N=8192, K=8192, ldx=8192, ldy=8192, ws=A16 + 4, ws_bytes=need) == gmi.GMI_ERR_MISALIGNED


def _mixed(gmi, M=16, N=64, K=256, xdt=1, X=A16, ldx=256, W=A16 * 2, wt=1, S=A16 * 3, Z=A16 * 4, g=128, Y=A16 * 5,
           ldy=64):
    return gmi.lib().gmi_gemm_mixed(M, N, K, xdt, X, ldx, W, wt, S, Z, g, Y, ldy, None, 0, None)


def test_mixed_validation(gmi):
    assert _mixed(gmi, xdt=2) == gmi.GMI_ERR_UNSUPPORTED  # fp8 activations: not a mixed-input type here
    assert _mixed(gmi, wt=2) == gmi.GMI_ERR_UNSUPPORTED
    assert _mixed(gmi, S=None) == gmi.GMI_ERR_UNSUPPORTED  # zero points without scales
    assert _mixed(gmi, g=96) == gmi.GMI_ERR_INVALID_ARG
    assert _mixed(gmi, N=24) == gmi.GMI_ERR_UNSUPPORTED
    assert _mixed(gmi, W=None) == gmi.GMI_ERR_INVALID_ARG
    assert _mixed(gmi, Z=A16 + 4) == gmi.GMI_ERR_MISALIGNED
    assert _mixed(gmi, S=None, Z=None, ldy=60) == gmi.GMI_ERR_INVALID_ARG  # reaches the shape checks
    assert _mixed(gmi, M=0, S=None, Z=None, g=0) == gmi.GMI_OK  # group size unused without scales


def _mg(gmi, count=4, offsets=A16 * 6, rows=64, N=64, K=256, xdt=0, X=A16, ldx=256, W=A16 * 2, ws=64 * 128, wt=0,
        S=A16 * 3, ss=128, Z=A16 * 4, zs=64, g=128, Y=A16 * 5, ldy=64):
    return gmi.lib().gmi_gemm_mixed_grouped(count, offsets, rows, N, K, xdt, X, ldx, W, ws, wt, S, ss, Z, zs, g, Y,
                                            ldy, None)


def test_mixed_grouped_validation(gmi):
    assert _mg(gmi, count=-1) == gmi.GMI_ERR_INVALID_ARG
    assert _mg(gmi, count=65536) == gmi.GMI_ERR_UNSUPPORTED
    assert _mg(gmi, offsets=None) == gmi.GMI_ERR_INVALID_ARG
    assert _mg(gmi, offsets=A16 + 2) == gmi.GMI_ERR_MISALIGNED
    assert _mg(gmi, ws=64 * 128 - 16) == gmi.GMI_ERR_INVALID_ARG  # weight stride below one expert
    assert _mg(gmi, ss=120) == gmi.GMI_ERR_INVALID_ARG  # scale stride below one expert's scales
    assert _mg(gmi, zs=48) == gmi.GMI_ERR_INVALID_ARG
    assert _mg(gmi, ws=64 * 128 + 8) == gmi.GMI_ERR_MISALIGNED
    assert _mg(gmi, ss=132) == gmi.GMI_ERR_MISALIGNED
    assert _mg(gmi, S=None) == gmi.GMI_ERR_UNSUPPORTED  # zero points without scales
    assert _mg(gmi, xdt=2) == gmi.GMI_ERR_UNSUPPORTED
    assert _mg(gmi, N=24) == gmi.GMI_ERR_UNSUPPORTED
    assert _mg(gmi, ldx=128) == gmi.GMI_ERR_INVALID_ARG
    # nothing to do: no groups, no rows or no columns
    for kw in (dict(count=0), dict(rows=0), dict(N=0)):
        assert _mg(gmi, offsets=None, X=None, W=None, S=None, Z=None, Y=None, **kw) == gmi.GMI_OK, kw


def _dg(gmi, N=2, H=8, W=8, C=16, K=8, R=3, S=3, ph=1, pw=1, sh=1, sw=1, dh=1, dw=1, dy=A16, w=A16 * 2, c=None,
        dx=A16 * 3, dt=1, beta=0.0, ws=A16 * 4, ws_bytes=1 << 20):
    return gmi.lib().gmi_conv2d_dgrad_implicit(N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw, dy, w, c, dx, dt, 1.0,
                                               beta, ws, ws_bytes, None)


def test_conv_dgrad_validation(gmi):
    L = gmi.lib()
    assert L.gmi_conv2d_dgrad_workspace_bytes(16, 8, 3, 3) == 16 * 8 * 9 * 2  # already a multiple of 256
    assert L.gmi_conv2d_dgrad_workspace_bytes(8, 8, 1, 3) == 512  # 384 rounded up
    assert L.gmi_conv2d_dgrad_workspace_bytes(0, 8, 3, 3) == 0
    assert _dg(gmi, H=0) == gmi.GMI_ERR_INVALID_ARG
    assert _dg(gmi, ph=-1) == gmi.GMI_ERR_INVALID_ARG
    assert _dg(gmi, sh=9) == gmi.GMI_ERR_UNSUPPORTED  # strides 1 .. 8, each dimension on its own
    assert _dg(gmi, sw=16) == gmi.GMI_ERR_UNSUPPORTED
    assert _dg(gmi, sh=0) == gmi.GMI_ERR_INVALID_ARG
    assert _dg(gmi, dt=2) == gmi.GMI_ERR_UNSUPPORTED
    assert _dg(gmi, C=12) == gmi.GMI_ERR_MISALIGNED
    assert _dg(gmi, H=1, ph=0) == gmi.GMI_ERR_INVALID_ARG  # a 3x3 filter does not fit a 1-row image
    assert _dg(gmi, beta=1.0) == gmi.GMI_ERR_INVALID_ARG  # c_in required
    assert _dg(gmi, dy=A16 + 2) == gmi.GMI_ERR_MISALIGNED
    assert _dg(gmi, ws_bytes=100) == gmi.GMI_ERR_WORKSPACE
    assert _dg(gmi, ws=None) == gmi.GMI_ERR_WORKSPACE
    assert _dg(gmi, ws=A16 + 8) == gmi.GMI_ERR_MISALIGNED
    assert _dg(gmi, N=0, dy=None, w=None, dx=None, ws=None) == gmi.GMI_OK


def _wg(gmi, N=2, H=8, W=8, C=16, K=8, R=3, S=3, ph=1, pw=1, sh=1, sw=1, dh=1, dw=1, groups=1, x=A16, dy=A16 * 2,
        c=None, out=A16 * 3, dt=1, beta=0.0, ws=A16 * 4, ws_bytes=1 << 26):
    return gmi.lib().gmi_conv2d_wgrad_implicit(N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw, groups, x, dy, c, out, dt,
                                               1.0, beta, ws, ws_bytes, None)


def test_conv_wgrad_validation(gmi):
    L = gmi.lib()
    need = L.gmi_conv2d_wgrad_workspace_bytes(2, 8, 8, 16, 8, 3, 3, 1, 1, 1, 1, 1, 1, 1)
    # at least the two transposed operands (batch padded to 8) and one fp32 partial of the 16 x 3 x 3 x 8 output
    assert need >= 16 * 8 * 8 * 8 * 2 + 8 * 8 * 8 * 8 * 2 + 16 * 9 * 8 * 4
    assert L.gmi_conv2d_wgrad_workspace_bytes(2, 8, 8, 12, 8, 3, 3, 1, 1, 1, 1, 1, 1, 1) == 0  # rejected problem
    assert _wg(gmi, groups=3) == gmi.GMI_ERR_INVALID_ARG  # does not divide C and K
    assert _wg(gmi, C=32, K=32, groups=8) == gmi.GMI_ERR_UNSUPPORTED  # 4 output channels per group
    assert _wg(gmi, N=0) == gmi.GMI_ERR_INVALID_ARG
    assert _wg(gmi, ph=-1) == gmi.GMI_ERR_INVALID_ARG
    assert _wg(gmi, dh=9) == gmi.GMI_ERR_UNSUPPORTED
    assert _wg(gmi, dt=2) == gmi.GMI_ERR_UNSUPPORTED
    assert _wg(gmi, C=12) == gmi.GMI_ERR_MISALIGNED
    assert _wg(gmi, H=1, ph=0) == gmi.GMI_ERR_INVALID_ARG
    assert _wg(gmi, beta=1.0) == gmi.GMI_ERR_INVALID_ARG
    assert _wg(gmi, x=A16 + 2) == gmi.GMI_ERR_MISALIGNED
    assert _wg(gmi, ws_bytes=need - 1) == gmi.GMI_ERR_WORKSPACE
    assert _wg(gmi, ws=None) == gmi.GMI_ERR_WORKSPACE


def test_w4a16_workspace_bytes(gmi):
    # without a device the library assumes 256 CUs, as on MI355X: 128 x 8192 has 64 output tiles of
    # 128 x 128; fp16 splits K into up to four k-ranges (until the items cover 256 CUs), bf16 into up to
    # eight (until they cover 512 workgroup slots), and the size is the larger need: fp32 partials, a whole
    # tile of 128 x 128 floats per range (ragged row counts round up to 128 tokens); decode shapes and
    # shapes that fill the device use none
    L = gmi.lib()
    tile = 128 * 128 * 4
    assert L.gmi_w4a16_workspace_bytes(128, 8192, 8192) == 8 * 64 * tile
    assert L.gmi_w4a16_workspace_bytes(100, 8192, 8192) == 8 * 64 * tile
    assert L.gmi_w4a16_workspace_bytes(200, 8192, 8192) == 4 * 128 * tile  # 128 tiles: four bf16 ranges fill 512
    assert L.gmi_w4a16_workspace_bytes(128, 8000, 8192) == 8 * 63 * tile  # 8000 rows: 63 tiles of 128
    assert L.gmi_w4a16_workspace_bytes(128, 8192, 2048) == 4 * 64 * tile  # eight ranges would hold 256 k
    assert L.gmi_w4a16_workspace_bytes(16, 8192, 8192) == 0
    assert L.gmi_w4a16_workspace_bytes(4096, 8192, 8192) == 0
    assert L.gmi_w4a16_workspace_bytes(128, 8192, 1024) == 2 * 64 * tile  # k-ranges keep >= 512 k each
    assert L.gmi_w4a16_workspace_bytes(-1, 16, 128) == 0
    assert L.gmi_w4a16_workspace_bytes(128, 24, 128) == 0


def _conv(gmi, N=2, H=8, W=8, C=16, K=16, R=3, S=3, ph=1, pw=1, sh=1, sw=1, dh=1, dw=1, x=A16, w=A16 * 2,
          c=None, y=A16 * 3, dt=1, beta=0.0):
    return gmi.lib().gmi_conv2d_fprop_implicit(N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw, x, w, c, y, dt, 1.0,
                                               beta, None)


def test_conv_validation(gmi):
    assert _conv(gmi, N=-1) == gmi.GMI_ERR_INVALID_ARG
    assert _conv(gmi, C=0) == gmi.GMI_ERR_INVALID_ARG
    assert _conv(gmi, ph=-1) == gmi.GMI_ERR_INVALID_ARG
    assert _conv(gmi, sh=0) == gmi.GMI_ERR_INVALID_ARG
    assert _conv(gmi, sw=9) == gmi.GMI_ERR_UNSUPPORTED  # traversal stride limited to 1..8
    assert _conv(gmi, dh=0) == gmi.GMI_ERR_INVALID_ARG
    assert _conv(gmi, C=12) == gmi.GMI_ERR_MISALIGNED
    assert _conv(gmi, K=20) == gmi.GMI_ERR_MISALIGNED
    assert _conv(gmi, dt=3) == gmi.GMI_ERR_UNSUPPORTED
    assert _conv(gmi, H=2, R=5, ph=0) == gmi.GMI_ERR_INVALID_ARG  # filter larger than the padded image
    assert _conv(gmi, x=None) == gmi.GMI_ERR_INVALID_ARG
    assert _conv(gmi, beta=1.0) == gmi.GMI_ERR_INVALID_ARG  # c_in required
    assert _conv(gmi, y=A16 + 8) == gmi.GMI_ERR_MISALIGNED
    assert _conv(gmi, N=0, x=None, w=None, y=None) == gmi.GMI_OK


def test_errors_raise_through_the_binding(gmi):
    import torch

    with pytest.raises(gmi.GmiError, match="GMI_ERR_MISALIGNED"):
        gmi.gemm_w4a16(torch.empty((16, 256), dtype=torch.float16), torch.empty(16384, dtype=torch.uint8),
                       torch.empty((2, 64), dtype=torch.float16), torch.empty((2, 32), dtype=torch.uint8), 128, 64,
                       Y=torch.empty((16, 68), dtype=torch.float16)[:, 2:66], stream=0)


def _conv_fused(gmi, bias=A16 * 5, act=1, N=2, C=16, K=16, dt=1, x=A16, y=A16 * 3):
    return gmi.lib().gmi_conv2d_fprop_implicit_fused(N, 8, 8, C, K, 3, 3, 1, 1, 1, 1, 1, 1, x, A16 * 2, None, bias,
                                                     y, dt, 1.0, 0.0, act, None)


def test_conv_fused_validation(gmi):
    # rejected before any launch: an unknown activation, a misaligned bias, and every rule of the plain call
    assert _conv_fused(gmi, act=2) == gmi.GMI_ERR_INVALID_ARG
    assert _conv_fused(gmi, act=-1) == gmi.GMI_ERR_INVALID_ARG
    assert _conv_fused(gmi, bias=A16 + 2) == gmi.GMI_ERR_MISALIGNED
    assert _conv_fused(gmi, C=12) == gmi.GMI_ERR_MISALIGNED
    assert _conv_fused(gmi, dt=3) == gmi.GMI_ERR_UNSUPPORTED
    assert _conv_fused(gmi, x=None) == gmi.GMI_ERR_INVALID_ARG
    assert _conv_fused(gmi, N=0) == gmi.GMI_OK  # no images: nothing to do, nothing launched


def test_time_next_gemm_checks_its_pair(gmi):
    # no HIP call: both NULL cancels, exactly one NULL is rejected (a real pair is exercised on the GPU)
    import ctypes
    L = gmi.lib()
    assert L.gmi_time_next_gemm(None, None) == 0
    assert L.gmi_time_next_gemm(ctypes.c_void_p(64), None) == gmi.GMI_ERR_INVALID_ARG
    assert L.gmi_time_next_gemm(None, ctypes.c_void_p(64)) == gmi.GMI_ERR_INVALID_ARG
    assert b"both" in L.gmi_last_error()
    assert L.gmi_time_next_gemm(None, None) == 0
