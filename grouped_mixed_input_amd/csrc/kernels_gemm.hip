// kernels_gemm.hip -- persistent grouped and pointer-array GEMM kernels.
//
// Both follow the persistent work-tile loop of the page
// sm90_gemm_array_tma_warpspecialized_cooperative.hpp (operator(): take the
// initial work tile, exit when it is invalid, and for every tile refresh the
// problem shape of its group / batch before running the k-loop and the
// epilogue).  Grouped problems carry their own shape and strides; the array
// mode shares one shape and one stride per operand over L batches.
#include <type_traits>

#include <hip/hip_ext.h>

#include "gmi_device.hpp"
#include "gmi_internal.hpp"

namespace gmi {

template <class Cfg, int DT, bool KTAIL>
__device__ __forceinline__ void run_tile(char* lds, const Tile& t, float alpha, float beta) {
  DenseLoader<Cfg, Cfg::BM, KTAIL> al;
  DenseLoader<Cfg, Cfg::BN, KTAIL> bl;
  al.init(t.A, t.lda, t.m0, t.M, t.K);
  bl.init(t.B, t.ldb, t.n0, t.N, t.K);
  f32x16 acc[Cfg::TM][Cfg::TN];
  mainloop<Cfg, DT>(lds, al, bl, (t.K + Cfg::BK - 1) / Cfg::BK, acc);
  store_tile<Cfg, out_dt<DT>()>(t, acc, alpha, beta, lds);
}

template <class Cfg>
constexpr int lds_of() {
  if constexpr (std::is_void<Cfg>::value)
    return 0;
  else
    return Cfg::LDS_BYTES;
}

struct GroupedArgs {
  const GroupDesc* desc;
  int count, total_tiles;  // total_tiles < 0: read the total from *total_dev
  const int32_t* total_dev;
  float alpha, beta;
};

// Tile ids are laid out problem after problem, and inside a problem in bands
// of m-tiles (raster), so one XCD's share of a round -- consecutive tiles --
// reuses a few A and B panels, e.g. one expert weight in a mixture-of-experts
// layer.
// Tile configurations a grouped 256x256 launch uses for problems of at most
// SMALL_M and at most TINY_M rows: SMALL_M x 256 and TINY_M x 256 over the
// same 8 waves (one wave row, eight wave columns), four-stage rings.
template <class Cfg>
struct SmallOf {
  using type = void;
};
template <class Cfg>
struct TinyOf {
  using type = void;
};
template <int DT, bool KTAIL, class Cfg>
__device__ __forceinline__ void grouped_tile(char* lds, const GroupDesc& d, int local, float alpha, float beta) {
  int mi, ni;
  raster(local, (d.M + Cfg::BM - 1) / Cfg::BM, (d.N + Cfg::BN - 1) / Cfg::BN, mi, ni);
  Tile t;
  t.M = d.M;
  t.N = d.N;
  t.K = d.K;
  t.m0 = mi * Cfg::BM;
  t.n0 = ni * Cfg::BN;
  t.A = d.A;
  t.lda = d.lda;
  t.B = d.B;
  t.ldb = d.ldb;
  t.C = d.C;
  t.ldc = d.ldc;
  t.D = d.D;
  t.ldd = d.ldd;
  run_tile<Cfg, DT, KTAIL>(lds, t, alpha, beta);
}

// The persistent walk over a problem table `desc` (global memory, or the
// kernel's own arguments for short lists).
template <class Cfg, int DT, bool KTAIL, class Table>
__device__ __forceinline__ void grouped_walk(char* lds, const Table& desc, int count, int total, float alpha,
                                             float beta) {
  using Small = typename SmallOf<Cfg>::type;
  using Tiny = typename TinyOf<Cfg>::type;
  const int G = gridDim.x;
  int g = 0;
  for (int base = 0; base < total; base += G) {
    const int tile = base + remap_slot(blockIdx.x, G);
    if (tile >= total) break;
    while (g + 1 < count && desc[g + 1].tile_start <= tile) ++g;
    const GroupDesc& d = desc[g];
    const int local = tile - d.tile_start;
    if constexpr (!std::is_void<Tiny>::value) {
      if (d.M <= TINY_M) {
        grouped_tile<DT, KTAIL, Tiny>(lds, d, local, alpha, beta);
        continue;
      }
    }
    if constexpr (!std::is_void<Small>::value) {
      if (d.M <= SMALL_M) {
        grouped_tile<DT, KTAIL, Small>(lds, d, local, alpha, beta);
        continue;
      }
    }
    grouped_tile<DT, KTAIL, Cfg>(lds, d, local, alpha, beta);
  }
}

template <class Cfg>
constexpr int grouped_lds() {
  constexpr int a = Cfg::LDS_BYTES, b = lds_of<typename SmallOf<Cfg>::type>(), c = lds_of<typename TinyOf<Cfg>::type>();
  return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

template <class Cfg, int DT, bool KTAIL>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WGS_PER_CU) void k_gemm_grouped(GroupedArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[grouped_lds<Cfg>()];
  // with device-held group sizes the grid is sized for the device, not the
  // tiles: workgroups past the total find no tile and return
  const int total = a.total_tiles >= 0 ? a.total_tiles : *a.total_dev;
  grouped_walk<Cfg, DT, KTAIL>(lds, a.desc, a.count, total, a.alpha, a.beta);
}

// Short problem lists travel in the kernel arguments: no staging copy before
// the launch, which is most of the cost of a call on a few small problems.
struct GroupedInlineArgs {
  GroupDesc desc[kInlineGroups];
  int count, total_tiles;
  float alpha, beta;
};
static_assert(sizeof(GroupedInlineArgs) <= 4096, "kernel arguments are limited to 4 KB");

template <class Cfg, int DT, bool KTAIL>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WGS_PER_CU) void k_gemm_grouped_inline(GroupedInlineArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[grouped_lds<Cfg>()];
  grouped_walk<Cfg, DT, KTAIL>(lds, a.desc, a.count, a.total_tiles, a.alpha, a.beta);
}

// Group table from device-held row offsets (one workgroup, one thread per
// group): group g owns rows [offsets[g], offsets[g + 1]) clipped to
// [0, rows); it gets the tile rows of the grouped rule, and the groups are
// ranked by work per tile (rows a tile actually uses; K is shared), largest
// first, ties in group order -- the same order the host-built table uses.
// The tile prefix sums follow the ranking; the total goes to *total.
struct OffsetsTableArgs {
  const int32_t* offsets;
  int count, rows, N, K;
  const char* A;  // byte pointers; A and B elements are `eb` bytes, C and D two
  const char* B;
  const char* C;
  char* D;
  int64_t lda, ldb, stride_b, ldc, ldd;
  int eb, bm, bn, small_class;
  GroupDesc* desc;
  int32_t* total;
};


__global__ __launch_bounds__(kMaxOffsetGroupCount) void k_group_table(OffsetsTableArgs a) {
  __shared__ int32_t key[kMaxOffsetGroupCount];
  __shared__ int32_t scan[2][kMaxOffsetGroupCount];
  const int g = threadIdx.x;
  const bool live = g < a.count;
  int lo = 0, m = 0, work = -1, tiles = 0;
  if (live) {
    lo = min(max(a.offsets[g], 0), a.rows);
    const int hi = min(max(a.offsets[g + 1], 0), a.rows);
    m = hi > lo ? hi - lo : 0;
    if (m > 0 && a.N > 0) {
      const int tr = !a.small_class ? a.bm : m <= TINY_M ? TINY_M : m <= SMALL_M ? SMALL_M : a.bm;
      tiles = (m + tr - 1) / tr * ((a.N + a.bn - 1) / a.bn);
      work = min(m, tr);
    }
  }
  key[g] = work;
  __syncthreads();
  int rank = g;
  if (live) {
    rank = 0;
    for (int h = 0; h < a.count; ++h) {
      const int kh = key[h];
      rank += (kh > work) || (kh == work && h < g);
    }
  }
  scan[0][g] = 0;
  __syncthreads();
  if (live) scan[0][rank] = tiles;
  __syncthreads();
  int cur = 0;
  for (int d = 1; d < kMaxOffsetGroupCount; d <<= 1) {  // inclusive scan over ranks
    const int v = scan[cur][g] + (g >= d ? scan[cur][g - d] : 0);
    scan[cur ^ 1][g] = v;
    cur ^= 1;
    __syncthreads();
  }
  if (live) {
    GroupDesc d;
    d.A = (const uint16_t*)(a.A + (int64_t)lo * a.lda * a.eb);
    d.B = (const uint16_t*)(a.B + (int64_t)g * a.stride_b * a.eb);
    d.C = a.C ? (const uint16_t*)(a.C + (int64_t)lo * a.ldc * 2) : nullptr;
    d.D = (uint16_t*)(a.D + (int64_t)lo * a.ldd * 2);
    d.lda = a.lda;
    d.ldb = a.ldb;
    d.ldc = a.ldc;
    d.ldd = a.ldd;
    d.M = m;
    d.N = a.N;
    d.K = a.K;
    d.tile_start = scan[cur][rank] - tiles;
    a.desc[rank] = d;
  }
  if (g == 0) *a.total = a.count > 0 ? scan[cur][a.count - 1] : 0;
}

struct PtrArrayArgs {
  PtrArrayLaunch p;
  int tiles_m, tiles_per_batch, total_tiles;
  float alpha, beta;
};

template <class Cfg, int DT, bool KTAIL>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WGS_PER_CU) void k_gemm_ptr_array(PtrArrayArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
  const int G = gridDim.x;
  for (int base = 0; base < a.total_tiles; base += G) {
    const int tile = base + remap_slot(blockIdx.x, G);
    if (tile >= a.total_tiles) break;
    const int l = tile / a.tiles_per_batch, local = tile - l * a.tiles_per_batch;
    int mi, ni;
    raster(local, a.tiles_m, a.tiles_per_batch / a.tiles_m, mi, ni);
    Tile t;
    t.M = a.p.M;
    t.N = a.p.N;
    t.K = a.p.K;
    t.m0 = mi * Cfg::BM;
    t.n0 = ni * Cfg::BN;
    t.A = a.p.A[l];
    t.lda = a.p.lda;
    t.B = a.p.B[l];
    t.ldb = a.p.ldb;
    t.C = a.beta != 0.0f ? a.p.C[l] : nullptr;
    t.ldc = a.p.ldc;
    t.D = a.p.D[l];
    t.ldd = a.p.ldd;
    run_tile<Cfg, DT, KTAIL>(lds, t, a.alpha, a.beta);
  }
}

// 16-bit inputs: 256x256 on a five-slot ring of 64-k single-operand slots
// (one workgroup of 8 waves per CU); 256x128 and 128x128 on rings of three
// 24 KB and four 16 KB 32-k stages (two workgroups of 4 waves per CU).
using Cfg256 = TileCfg<256, 256, 4, 2, 64, 2, 5>;
using Cfg256x128 = TileCfg<256, 128, 2, 2, 32, 3>;
using Cfg128 = TileCfg<128, 128, 2, 2, 32, 4>;
using CfgSmall256 = TileCfg<SMALL_M, 256, 1, 8, 64, 4>;
using CfgTiny256 = TileCfg<TINY_M, 256, 1, 8, 64, 4>;
// fp8 inputs: the same row bytes (128 k per 128-byte row), so the same rings
// where they fit; 256x128 and 128x128 on two stages of 48 KB and 32 KB.
using Cfg256F8 = TileCfg<256, 256, 4, 2, 128, 2, 5, 1>;
using Cfg256x128F8 = TileCfg<256, 128, 2, 2, 128, 2, 0, 1>;
using Cfg128F8 = TileCfg<128, 128, 2, 2, 128, 2, 0, 1>;
using CfgSmall256F8 = TileCfg<SMALL_M, 256, 1, 8, 128, 4, 0, 1>;
using CfgTiny256F8 = TileCfg<TINY_M, 256, 1, 8, 128, 4, 0, 1>;
template <>
struct SmallOf<Cfg256> {
  using type = CfgSmall256;
};
template <>
struct SmallOf<Cfg256F8> {
  using type = CfgSmall256F8;
};
template <>
struct TinyOf<Cfg256> {
  using type = CfgTiny256;
};
template <>
struct TinyOf<Cfg256F8> {
  using type = CfgTiny256F8;
};
static_assert(CfgSmall256::THREADS == Cfg256::THREADS && CfgSmall256F8::THREADS == Cfg256F8::THREADS &&
                  CfgTiny256::THREADS == Cfg256::THREADS && CfgTiny256F8::THREADS == Cfg256F8::THREADS,
              "every tile shape of a grouped launch runs on the same workgroup");

// Persistent grid: a whole number of XCD rounds, no more workgroups than can
// be resident at once and no more than the tiles need.
static int persistent_grid(int total_tiles, int wgs_per_cu) {
  const int resident = device_cu_count() * wgs_per_cu;
  int g = (total_tiles + XCDS - 1) / XCDS * XCDS;
  if (g > resident) g = resident / XCDS * XCDS;
  return g < XCDS ? XCDS : g;
}

// Instantiate and launch KER for the tile shape, element type and K-tail mode
// (KT: some K is not a multiple of 8, so a chunk can straddle K; fp8 requires
// K % 16 == 0 and has no tail mode).
// A pending gmi_time_next_gemm request goes to this launch: the runtime then
// stamps the pair with the kernel's own start and end.
template <class F, class A>
static void launch_gemm(F kernel, dim3 grid, dim3 block, hipStream_t stream, const A& args) {
  LaunchTimer& t = launch_timer();
  if (t.start) {
    const LaunchTimer ev = t;
    t = LaunchTimer{};
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0, args);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args);
  }
}
#define GMI_LAUNCH1(KER, CFG, DT, KT, tiles, args, stream)                                                    \
  launch_gemm(KER<CFG, DT, KT>, dim3(persistent_grid(tiles, CFG::WGS_PER_CU)), dim3(CFG::THREADS), stream, args)
#define GMI_LAUNCH_DT(KER, CFG, CFG8, dtype, kt, tiles, args, stream)                         \
  do {                                                                                       \
    if ((dtype) == DT_F16) {                                                                 \
      if (kt) GMI_LAUNCH1(KER, CFG, DT_F16, true, tiles, args, stream);                      \
      else GMI_LAUNCH1(KER, CFG, DT_F16, false, tiles, args, stream);                        \
    } else if ((dtype) == DT_BF16) {                                                         \
      if (kt) GMI_LAUNCH1(KER, CFG, DT_BF16, true, tiles, args, stream);                     \
      else GMI_LAUNCH1(KER, CFG, DT_BF16, false, tiles, args, stream);                       \
    } else {                                                                                 \
      GMI_LAUNCH1(KER, CFG8, DT_F8, false, tiles, args, stream);                             \
    }                                                                                        \
  } while (0)
#define GMI_DISPATCH(KER, shape, dtype, kt, tiles, args, stream)                                               \
  do {                                                                                                       \
    if ((shape) == TILE_256x256) GMI_LAUNCH_DT(KER, Cfg256, Cfg256F8, dtype, kt, tiles, args, stream);      \
    else if ((shape) == TILE_256x128)                                                                        \
      GMI_LAUNCH_DT(KER, Cfg256x128, Cfg256x128F8, dtype, kt, tiles, args, stream);                          \
    else GMI_LAUNCH_DT(KER, Cfg128, Cfg128F8, dtype, kt, tiles, args, stream);                               \
  } while (0)

hipError_t launch_grouped(const GroupDesc* desc_dev, int count, int total_tiles, int shape, int dtype, bool ktail,
                          float alpha, float beta, hipStream_t stream) {
  GroupedArgs a{desc_dev, count, total_tiles, nullptr, alpha, beta};
  GMI_DISPATCH(k_gemm_grouped, shape, dtype, ktail, total_tiles, a, stream);
  return hipGetLastError();
}

// A host problem table written into the workspace by launches whose
// arguments carry it, kInlineGroups descriptors each: unlike a copy from
// pageable host memory, a launch does not wait for the work already queued
// on the stream, so the host goes on while the previous GEMM runs.
struct TableChunk {
  GroupDesc desc[kInlineGroups];
  GroupDesc* dst;
  int n;
};

__global__ __launch_bounds__(64) void k_write_table(TableChunk c) {
  if ((int)threadIdx.x < c.n) c.dst[threadIdx.x] = c.desc[threadIdx.x];
}

hipError_t stage_table(const GroupDesc* desc, int count, GroupDesc* dst, hipStream_t stream) {
  for (int g0 = 0; g0 < count; g0 += kInlineGroups) {
    TableChunk c;
    c.n = count - g0 < kInlineGroups ? count - g0 : kInlineGroups;
    for (int i = 0; i < c.n; ++i) c.desc[i] = desc[g0 + i];
    c.dst = dst + g0;
    hipLaunchKernelGGL(k_write_table, dim3(1), dim3(64), 0, stream, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_grouped_inline(const GroupDesc* desc, int count, int total_tiles, int shape, int dtype,
                                 bool ktail, float alpha, float beta, hipStream_t stream) {
  GroupedInlineArgs a;
  for (int g = 0; g < count; ++g) a.desc[g] = desc[g];
  a.count = count;
  a.total_tiles = total_tiles;
  a.alpha = alpha;
  a.beta = beta;
  GMI_DISPATCH(k_gemm_grouped_inline, shape, dtype, ktail, total_tiles, a, stream);
  return hipGetLastError();
}

hipError_t launch_grouped_offsets(const OffsetsLaunch& p, int shape, int dtype, float alpha, float beta,
                                  hipStream_t stream) {
  OffsetsTableArgs t;
  t.offsets = p.offsets;
  t.count = p.count;
  t.rows = p.rows;
  t.N = p.N;
  t.K = p.K;
  t.A = (const char*)p.A;
  t.B = (const char*)p.B;
  t.C = (const char*)p.C;
  t.D = (char*)p.D;
  t.lda = p.lda;
  t.ldb = p.ldb;
  t.stride_b = p.stride_b;
  t.ldc = p.ldc;
  t.ldd = p.ldd;
  t.eb = dtype == DT_F8 ? 1 : 2;
  t.bm = tile_bm(shape);
  t.bn = tile_bn(shape);
  t.small_class = shape == TILE_256x256;
  t.desc = p.desc;
  t.total = p.total;
  hipLaunchKernelGGL(k_group_table, dim3(1), dim3(kMaxOffsetGroupCount), 0, stream, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the tile total is known on the device only: size the grid for the
  // device (every resident workgroup), idle ones return at once
  GroupedArgs a{p.desc, p.count, -1, p.total, alpha, beta};
  const int fill = 1 << 20;
  GMI_DISPATCH(k_gemm_grouped, shape, dtype, (p.K % 8) != 0, fill, a, stream);
  return hipGetLastError();
}

hipError_t launch_ptr_array(const PtrArrayLaunch& p, int shape, int dtype, float alpha, float beta,
                            hipStream_t stream) {
  PtrArrayArgs a;
  a.p = p;
  a.tiles_m = (p.M + tile_bm(shape) - 1) / tile_bm(shape);
  a.tiles_per_batch = a.tiles_m * ((p.N + tile_bn(shape) - 1) / tile_bn(shape));
  a.total_tiles = a.tiles_per_batch * p.L;
  a.alpha = alpha;
  a.beta = beta;
  GMI_DISPATCH(k_gemm_ptr_array, shape, dtype, (p.K % 8) != 0, a.total_tiles, a, stream);
  return hipGetLastError();
}

}  // namespace gmi
