// gmi_internal.hpp -- host-side declarations shared by the C-ABI layer and
// the kernel translation units: launch descriptors and launcher functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmi {

// One problem of a grouped launch, as staged into the device workspace.
struct GroupDesc {
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* C;
  uint16_t* D;
  int64_t lda, ldb, ldc, ldd;
  int32_t M, N, K;
  int32_t tile_start;  // first tile id of this problem (exclusive prefix sum)
};
static_assert(sizeof(GroupDesc) == 80, "descriptor layout is part of the workspace contract");
constexpr size_t kWorkspaceHeader = 256;

// Tile shapes of the dense mainloop (BM x BN, 4 waves).
enum TileShape { TILE_256x256 = 0, TILE_128x128 = 1, TILE_256x128 = 2 };
inline int tile_bm(int s) { return s == TILE_128x128 ? 128 : 256; }
inline int tile_bn(int s) { return s == TILE_256x256 ? 256 : 128; }
inline int tile_wgs_per_cu(int s) { return s == TILE_256x256 ? 1 : 2; }  // matches TileCfg::WGS_PER_CU
// Grouped GEMM with 256x256 tiles: a problem of at most SMALL_M rows takes
// SMALL_M x 256 tiles instead, and one of at most TINY_M rows TINY_M x 256
// tiles (same kernel, their own tile configurations), so short groups -- the
// rare experts of a mixture-of-experts layer -- do not pay for 256 rows of
// matrix work.  Host tile counting, the device table builder and the kernel
// use this rule.
constexpr int SMALL_M = 64, TINY_M = 32;
inline int grouped_tile_rows(int shape, int M) {
  if (shape != TILE_256x256) return tile_bm(shape);
  return M <= TINY_M ? TINY_M : M <= SMALL_M ? SMALL_M : 256;
}

// Grouped launch whose group sizes are device-held row offsets; `desc` and
// `total` point into the caller's workspace.
struct OffsetsLaunch {
  const int32_t* offsets;
  int count, rows, N, K;
  const void* A;
  const void* B;
  const void* C;  // NULL when beta == 0
  void* D;
  int64_t lda, ldb, stride_b, ldc, ldd;
  GroupDesc* desc;
  int32_t* total;
};
constexpr int kMaxOffsetGroupCount = 1024;

struct PtrArrayLaunch {
  const uint16_t* const* A;
  const uint16_t* const* B;
  const uint16_t* const* C;
  uint16_t* const* D;
  int64_t lda, ldb, ldc, ldd;
  int L, M, N, K;
};

struct ConvLaunch {
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* c;
  uint16_t* y;
  int N, H, W, C, K, R, S, P, Q, ph, pw, sh, sw, dh, dw;
  // split over the taps into fp32 partials (see k_conv_fprop); 1 / NULL: none
  int split = 1, kt_split = 1 << 30;
  float* partial = nullptr;
  // independent groups (see k_conv_fprop): offsets per group in elements
  int groups = 1;
  int64_t x_group = 0, w_group = 0, part_group = 0;
  // fused epilogue of the forward pass: per-output-channel bias (NULL: none)
  // and activation (0: none, 1: ReLU); unsplit launches only
  const uint16_t* bias = nullptr;
  int act = 0;
  // output pixels on a strided grid of a larger NHWC tensor (one phase of the
  // strided data gradient): pixel (n, i, j) of the N x P x Q grid goes to
  // element map_off0 + n map_img + i map_rstep + j map_cstep of y (and c),
  // a tensor of map_bytes bytes; map_bytes == 0: the plain NPQK layout
  int64_t map_off0 = 0, map_img = 0, map_rstep = 0, map_cstep = 0;
  uint32_t map_bytes = 0;
};
// tile shape of a convolution launch's GEMM view (M pixels, N channels),
// by the rule of the GEMM calls
int conv_shape(int64_t M, int64_t N);
// the same for one launch over several problems of M[i] rows and N columns
int conv_shape_multi(const int64_t* M, int count, int64_t N);

struct W4Launch {
  int M, N, K, group;
  int dt;  // DT_F16 or DT_BF16: X, the scales and Y
  const uint16_t* X;
  int64_t ldx;
  const uint8_t* w;
  const uint16_t* scales;
  const uint8_t* zeros;
  // Conversion mode, applied as the values are read: missing scales or zero
  // points get a zero-sized buffer range (every read returns 0).
  uint32_t s_bytes, z_bytes;  // buffer ranges of scales and zeros
  uint32_t sor;               // OR-ed into every scale: the type's 1.0 without scales, else 0
  uint32_t wxor;              // XOR on every weight word: 0x88888888 for int4 (to offset binary), else 0
  uint32_t zxor;              // XOR on every zero point: 8 for int4 (the constant 8 without zeros), else 0
  uint16_t* Y;
  int64_t ldy;
  int split;       // k-ranges per output tile (1: no split)
  float* partial;  // split > 1: fp32 partial products, in the layout of the kernel that writes them
};

// Grouped (mixture-of-experts) mixed-input launch: group g owns rows
// [offsets[g], offsets[g + 1]) of X and Y (clipped to [0, rows)) and its own
// weight, scales and zero points at base + g * stride (bytes for the weight
// and the zeros, elements for the scales).  `base` carries every shared field;
// its M is unused.
struct W4Grouped {
  W4Launch base;
  const int32_t* offsets;
  int count, rows;
  int64_t w_stride, s_stride, z_stride;
};

int device_cu_count();  // cached per device

// Event pair that the next GEMM kernel launch on the calling thread records
// around itself (set by gmi_time_next_gemm, cleared when used)
struct LaunchTimer {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTimer& launch_timer();
// k-ranges per output tile the W4A16 GEMM uses for this shape and activation
// type on the current device (1 when the tiles alone fill the device or the
// path is skinny)
int w4a16_split(int M, int N, int K, int dt);
// bytes of fp32 partial products that split needs (0 without a split), for
// one type and the larger of the two
size_t w4a16_workspace_for(int M, int N, int K, int dt);
size_t w4a16_workspace(int M, int N, int K);

hipError_t launch_grouped(const GroupDesc* desc_dev, int count, int total_tiles, int shape, int dtype, bool ktail,
                          float alpha, float beta, hipStream_t stream);
// up to kInlineGroups problems: the table (host memory) is passed in the
// kernel arguments instead of being staged into the workspace
constexpr int kInlineGroups = 32;
// write a host table into device memory through kernel arguments (no copy
// from pageable memory, which would wait for the stream)
hipError_t stage_table(const GroupDesc* desc_host, int count, GroupDesc* dst, hipStream_t stream);
hipError_t launch_grouped_inline(const GroupDesc* desc_host, int count, int total_tiles, int shape, int dtype,
                                 bool ktail, float alpha, float beta, hipStream_t stream);
hipError_t launch_grouped_offsets(const OffsetsLaunch& p, int shape, int dtype, float alpha, float beta,
                                  hipStream_t stream);
hipError_t launch_ptr_array(const PtrArrayLaunch& a, int shape, int dtype, float alpha, float beta,
                            hipStream_t stream);
hipError_t launch_conv_fprop(const ConvLaunch& a, int shape, int dtype, float alpha, float beta, hipStream_t stream);
hipError_t launch_conv_dgrad(const ConvLaunch& a, uint16_t* wt, int dtype, float alpha, float beta,
                             hipStream_t stream);

// Weight gradient as a forward pass over transposed operands (see
// kernels_conv.hip): the plan fixes the view, the split over taps and the
// workspace layout; the workspace size and the launch both use it.
struct WgradPlan {
  int N, H, W, C, K, R, S, P, Q, ph, pw, sh, sw, dh, dw;  // the forward problem
  int groups, cg, kg;    // channel groups; input and output channels per group
  int N8, Rp, Sp;        // batch rounded up to 8; the view's output taps (>= R, S)
  int split, kt_split;   // the view's split over its P*Q*N8 taps (64 per k-tile)
  size_t x_off, dy_off, part_off, bytes;  // workspace layout
};
bool plan_wgrad(int N, int H, int W, int C, int K, int R, int S, int ph, int pw, int sh, int sw, int dh, int dw,
                int groups, WgradPlan& p);
hipError_t launch_conv_wgrad(const WgradPlan& p, const uint16_t* x, const uint16_t* dy, const uint16_t* c_in,
                             uint16_t* dwt, char* workspace, int dtype, float alpha, float beta, hipStream_t stream);
hipError_t launch_prepack_w4(const uint8_t* w, int N, int K, uint8_t* out, hipStream_t stream);
hipError_t launch_w4a16(const W4Launch& a, hipStream_t stream);
hipError_t launch_w4a16_grouped(const W4Grouped& a, hipStream_t stream);

}  // namespace gmi
