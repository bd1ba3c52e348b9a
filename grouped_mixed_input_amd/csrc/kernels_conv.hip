// kernels_conv.hip -- implicit-GEMM conv2d forward.
//
// The linearised problem of the page sm100_implicit_gemm_umma_warpspecialized.hpp
// (get_problem_shape_MNKL for fprop): M = N*P*Q output pixels, N = K filters,
// K = R*S*C taps.  The activation operand is gathered tile by tile from NHWC
// (ConvLoader: padding, traversal stride and dilation folded into the address,
// zero outside the image); the KRSC filter is already the column-major B
// operand with leading dimension R*S*C; the output rows are NPQK.
#include "gmi_device.hpp"
#include "gmi_internal.hpp"

namespace gmi {

struct ConvArgs {
  ConvGeom g;
  const uint16_t* w;
  const uint16_t* c;
  uint16_t* y;
  int M, Nk;  // GEMM M and N
  int tiles_n, total_tiles;
  float alpha, beta;
};

// Tile ids run n-tile fastest: the few n-tiles of a pixel block are
// consecutive, so one XCD gathers each activation panel once into its L2.
template <class Cfg, int DT>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WGS_PER_CU) void k_conv_fprop(ConvArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
  const int G = gridDim.x;
  for (int base = 0; base < a.total_tiles; base += G) {
    const int tile = base + remap_slot(blockIdx.x, G);
    if (tile >= a.total_tiles) break;
    Tile t;
    t.M = a.M;
    t.N = a.Nk;
    t.K = a.g.Kg;
    t.m0 = (tile / a.tiles_n) * Cfg::BM;
    t.n0 = (tile % a.tiles_n) * Cfg::BN;
    t.C = a.c;
    t.ldc = a.Nk;
    t.D = a.y;
    t.ldd = a.Nk;
    ConvLoader<Cfg, Cfg::BM> al;
    DenseLoader<Cfg, Cfg::BN> bl;
    al.init(a.g, t.m0, t.M);
    bl.init(a.w, a.g.Kg, t.n0, t.N, t.K);
    f32x16 acc[Cfg::TM][Cfg::TN];
    mainloop<Cfg, DT>(lds, al, bl, (t.K + Cfg::BK - 1) / Cfg::BK, acc);
    store_tile<Cfg, DT>(t, acc, a.alpha, a.beta, lds);
  }
}

using ConvCfg256 = TileCfg<256, 256, 4, 2, 64, 2, 5>;
using ConvCfg256x128 = TileCfg<256, 128, 2, 2, 32, 3>;
using ConvCfg128 = TileCfg<128, 128, 2, 2, 32, 4>;

hipError_t launch_conv_fprop(const ConvLaunch& p, int shape, int dtype, float alpha, float beta,
                             hipStream_t stream) {
  ConvArgs a;
  a.g = ConvGeom{p.x,   (uint32_t)((int64_t)p.N * p.H * p.W * p.C * 2),
                 p.H,   p.W,
                 p.C,   p.S,
                 p.P,   p.Q,
                 p.ph,  p.pw,
                 p.sh,  p.sw,
                 p.dh,  p.dw,
                 p.R * p.S * p.C,
                 ((p.H - 1) << p.ush) + 1, ((p.W - 1) << p.ush) + 1,
                 p.ush};
  a.w = p.w;
  a.c = p.c;
  a.y = p.y;
  a.M = p.N * p.P * p.Q;
  a.Nk = p.K;
  const int bm = tile_bm(shape), bn = tile_bn(shape);
  a.tiles_n = (p.K + bn - 1) / bn;
  a.total_tiles = ((a.M + bm - 1) / bm) * a.tiles_n;
  a.alpha = alpha;
  a.beta = beta;
  const int resident = device_cu_count() * tile_wgs_per_cu(shape);
  int grid = (a.total_tiles + XCDS - 1) / XCDS * XCDS;
  if (grid > resident) grid = resident / XCDS * XCDS;
  if (grid < XCDS) grid = XCDS;
  if (shape == TILE_256x256) {
    if (dtype == DT_F16)
      hipLaunchKernelGGL((k_conv_fprop<ConvCfg256, DT_F16>), dim3(grid), dim3(ConvCfg256::THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((k_conv_fprop<ConvCfg256, DT_BF16>), dim3(grid), dim3(ConvCfg256::THREADS), 0, stream, a);
  } else if (shape == TILE_256x128) {
    if (dtype == DT_F16)
      hipLaunchKernelGGL((k_conv_fprop<ConvCfg256x128, DT_F16>), dim3(grid), dim3(ConvCfg256x128::THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((k_conv_fprop<ConvCfg256x128, DT_BF16>), dim3(grid), dim3(ConvCfg256x128::THREADS), 0, stream, a);
  } else {
    if (dtype == DT_F16)
      hipLaunchKernelGGL((k_conv_fprop<ConvCfg128, DT_F16>), dim3(grid), dim3(ConvCfg128::THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((k_conv_fprop<ConvCfg128, DT_BF16>), dim3(grid), dim3(ConvCfg128::THREADS), 0, stream, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Data gradient.  The page runs the non-strided dgrad through the same
// im2col operand with the filter-tap strides negated: dx[n][h][w][c] sums
// dy[n][h + ph - r dh][w + pw - s dw][k] w[k][r][s][c], which is the forward
// gather over dy with padding -ph and dilation -dh.  A forward stride s
// (a power of two here) puts dy on every s-th coordinate of a virtual
// zero-inserted image, dy[n][p][q] at (s p, s q): the same gather, which
// reads only coordinates divisible by s (the others are zeros, and their
// products are wasted matrix work, a factor s^2).  The GEMM's B operand is
// the filter with its reduction (r, s, k) contiguous per column c, i.e. w
// transposed to [C][R][S][K]: one 64 x 64 (k, c) block of one tap per
// workgroup, through LDS so reads run along c and writes along k.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_filter_transpose(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt,
                                                          int K, int RS, int C) {
  __shared__ uint16_t t[64][65];
  const int rs = blockIdx.z, k0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int kk = i / 64, cc = i % 64, k = k0 + kk, c = c0 + cc;
    t[kk][cc] = (k < K && c < C) ? w[((int64_t)k * RS + rs) * C + c] : 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, kk = i % 64, k = k0 + kk, c = c0 + cc;
    if (k < K && c < C) wt[((int64_t)c * RS + rs) * K + k] = t[kk][cc];
  }
}

hipError_t launch_conv_dgrad(const ConvLaunch& p, uint16_t* wt, int shape, int dtype, float alpha, float beta,
                             hipStream_t stream) {
  // p describes the forward problem (x: N x H x W x C, y: N x P x Q x K);
  // here p.x is dy, p.y is dx
  const dim3 tgrid((p.C + 63) / 64, (p.K + 63) / 64, p.R * p.S);
  hipLaunchKernelGGL(k_filter_transpose, tgrid, dim3(256), 0, stream, p.w, wt, p.K, p.R * p.S, p.C);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ConvLaunch f;  // the forward view: gather over dy, filter [C][R][S][K]
  f.x = p.x;
  f.w = wt;
  f.c = p.c;
  f.y = p.y;
  f.N = p.N;
  f.H = p.P;
  f.W = p.Q;
  f.C = p.K;
  f.K = p.C;
  f.R = p.R;
  f.S = p.S;
  f.P = p.H;
  f.Q = p.W;
  f.ph = -p.ph;
  f.pw = -p.pw;
  f.sh = 1;
  f.sw = 1;
  f.dh = -p.dh;
  f.dw = -p.dw;
  f.ush = p.sh == 1 ? 0 : p.sh == 2 ? 1 : p.sh == 4 ? 2 : 3;  // sh == sw, a power of two
  return launch_conv_fprop(f, shape, dtype, alpha, beta, stream);
}

}  // namespace gmi
