// gmi_api.hip -- the C ABI: argument validation (every rule checked on the
// host before any HIP call), descriptor staging, tile-shape choice, launch.
//
// The checks restate the preconditions of the pages' can_implement functions:
// problem mode and rank, 128-bit alignment of every operand
// (sm90_gemm_array_tma_warpspecialized_cooperative.hpp, machete_mainloop.cuh),
// the group-size rules and the presence of scales and zeros
// (machete_mainloop.cuh), and the convolution rules -- channel-innermost
// tensors, traversal stride 1..8, cross-correlation, groups == 1
// (sm100_implicit_gemm_umma_warpspecialized.hpp).
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gmi.h"
#include "gmi_internal.hpp"

namespace gmi {

static thread_local std::string g_last_error;

static gmi_status fail(gmi_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

static gmi_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GMI_OK;
  return fail(GMI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Operands are read through buffer resources with 32-bit byte offsets: a
// 256-row tile of any operand must span less than 2^32 bytes.
constexpr int64_t kMaxLd = int64_t(1) << 22;
static bool dtype_ok(gmi_dtype d) { return d == GMI_F16 || d == GMI_BF16; }
static bool gemm_dtype_ok(gmi_dtype d) { return dtype_ok(d) || d == GMI_F8E4M3; }
// fp8 A and B: 16 elements per 16-byte chunk, so K and their leading
// dimensions must be multiples of 16 (chunks never straddle K)
static bool f8_shape_ok(gmi_dtype d, int64_t K, int64_t lda, int64_t ldb) {
  return d != GMI_F8E4M3 || K == 0 || (K % 16 == 0 && lda % 16 == 0 && ldb % 16 == 0);
}

// Tile shape for a list of problems: 256x256 when it alone fills every CU,
// then 256x128, else 128x128 (two resident workgroups per CU).
// GMI_FORCE_TILE=0|1|2 (256x256, 128x128, 256x128) overrides the choice; it
// exists for tile-shape sweeps in benchmarks.
static int forced_shape() {
  static const int f = [] {
    const char* e = getenv("GMI_FORCE_TILE");
    return (e && e[0] >= '0' && e[0] <= '2' && e[1] == 0) ? e[0] - '0' : -1;
  }();
  return f;
}

template <class F>
static int choose_shape(F tiles_at) {
  if (forced_shape() >= 0) return forced_shape();
  const int64_t cus = device_cu_count();
  if (tiles_at(256, 256) >= cus) return TILE_256x256;
  if (tiles_at(256, 128) >= cus) return TILE_256x128;
  return TILE_128x128;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int conv_shape(int64_t M, int64_t N) {
  return choose_shape([&](int bm, int bn) { return cdiv(M, bm) * cdiv(N, bn); });
}

int conv_shape_multi(const int64_t* M, int count, int64_t N) {
  return choose_shape([&](int bm, int bn) {
    int64_t t = 0;
    for (int i = 0; i < count; ++i) t += cdiv(M[i], bm) * cdiv(N, bn);
    return t;
  });
}

// Scratch of the allocation-free grouped call (gmi_gemm_grouped_offsets_noalloc):
// what gmi_gemm_grouped_offsets keeps in the caller's workspace -- the tile
// total in the header, then one descriptor per group -- for the largest
// group count the call takes.  Each device the library runs on holds its own
// copy from the library's load until the process ends.  Host code never uses
// the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = kWorkspaceHeader + sizeof(GroupDesc) * kMaxOffsetGroupCount;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];
static std::mutex g_scratch_mu;

// the current device's address of `scratch`, looked up on its first use
static gmi_status scratch_address(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GMI_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GMI_ERR_UNSUPPORTED, "%s: device %d, the scratch table is kept for devices 0..%d", who, dev,
                kMaxDevices - 1);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(GMI_ERR_HIP, "%s: hipGetSymbolAddress of the scratch table: %s", who, hipGetErrorString(e));
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GMI_OK;
}

LaunchTimer& launch_timer() {
  static thread_local LaunchTimer t;
  return t;
}

}  // namespace gmi

using namespace gmi;

extern "C" {

const char* gmi_last_error(void) { return g_last_error.c_str(); }

gmi_status gmi_time_next_gemm(void* start, void* stop) {
  g_last_error.clear();
  if ((start == nullptr) != (stop == nullptr))
    return fail(GMI_ERR_INVALID_ARG, "time_next_gemm: start and stop must both be events or both NULL");
  launch_timer() = LaunchTimer{(hipEvent_t)start, (hipEvent_t)stop};
  return GMI_OK;
}

size_t gmi_workspace_bytes(int32_t problem_count) {
  if (problem_count < 0) return 0;
  return kWorkspaceHeader + sizeof(GroupDesc) * (size_t)problem_count;
}

gmi_status gmi_gemm_grouped(const gmi_problem* problems, int32_t count, gmi_dtype dtype, float alpha, float beta,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (count < 0) return fail(GMI_ERR_INVALID_ARG, "gemm_grouped: count %d < 0", count);
  if (count > 0 && !problems) return fail(GMI_ERR_INVALID_ARG, "gemm_grouped: problems is NULL");
  if (!gemm_dtype_ok(dtype)) return fail(GMI_ERR_UNSUPPORTED, "gemm_grouped: dtype %d not supported", (int)dtype);
  const bool use_c = beta != 0.0f;
  int live = 0;
  for (int32_t g = 0; g < count; ++g) {
    const gmi_problem& p = problems[g];
    if (p.M < 0 || p.N < 0 || p.K < 0)
      return fail(GMI_ERR_INVALID_ARG, "gemm_grouped: problem %d has a negative size (%d, %d, %d)", g, p.M, p.N, p.K);
    if (p.M == 0 || p.N == 0) continue;
    ++live;
    if (!p.D || (p.K > 0 && (!p.A || !p.B)) || (use_c && !p.C))
      return fail(GMI_ERR_INVALID_ARG, "gemm_grouped: problem %d has a NULL operand", g);
    if ((p.K > 0 && (p.lda < p.K || p.ldb < p.K)) || p.ldd < p.N || (use_c && p.ldc < p.N))
      return fail(GMI_ERR_INVALID_ARG, "gemm_grouped: problem %d has a leading dimension below its row width", g);
    if (p.lda > kMaxLd || p.ldb > kMaxLd || p.ldd > kMaxLd || (use_c && p.ldc > kMaxLd))
      return fail(GMI_ERR_UNSUPPORTED, "gemm_grouped: problem %d: a leading dimension above 2^22 elements", g);
    if (!f8_shape_ok(dtype, p.K, p.lda, p.ldb))
      return fail(GMI_ERR_UNSUPPORTED, "gemm_grouped: problem %d: fp8 needs K, lda and ldb multiples of 16", g);
    if ((p.K > 0 && (!aligned16(p.A) || !aligned16(p.B) || p.lda % 8 || p.ldb % 8)) || !aligned16(p.D) ||
        p.ldd % 8 || (use_c && (!aligned16(p.C) || p.ldc % 8)))
      return fail(GMI_ERR_MISALIGNED, "gemm_grouped: problem %d: pointers must be 16-byte aligned, ld multiples of 8",
                  g);
  }
  if (live == 0) return GMI_OK;
  if (!workspace || workspace_bytes < gmi_workspace_bytes(live))
    return fail(GMI_ERR_WORKSPACE, "gemm_grouped: workspace of %zu bytes, %zu needed", workspace_bytes,
                gmi_workspace_bytes(live));
  if (!aligned16(workspace)) return fail(GMI_ERR_MISALIGNED, "gemm_grouped: workspace must be 16-byte aligned");

  const int shape = choose_shape([&](int bm, int bn) {
    int64_t t = 0;
    for (int32_t g = 0; g < count; ++g)
      if (problems[g].M > 0 && problems[g].N > 0) t += cdiv(problems[g].M, bm) * cdiv(problems[g].N, bn);
    return t;
  });
  const int bn = tile_bn(shape);
  // Problems are laid out in decreasing order of work per tile (rows of the
  // tile actually used x K; ties keep the caller's order), so the persistent
  // walk hands out the long tiles first and the short ones fill the tail.
  // The order changes nothing in the results: every problem has its own D.
  std::vector<int32_t> order;
  order.reserve(live);
  for (int32_t g = 0; g < count; ++g)
    if (problems[g].M > 0 && problems[g].N > 0) order.push_back(g);
  auto tile_work = [&](int32_t g) {
    const gmi_problem& p = problems[g];
    const int rows = grouped_tile_rows(shape, p.M);
    return (int64_t)std::min<int64_t>(p.M, rows) * (int64_t)std::max(p.K, 1);
  };
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return tile_work(x) > tile_work(y); });
  std::vector<GroupDesc> desc;
  desc.reserve(live);
  int64_t tiles = 0;
  bool ktail = false;
  for (const int32_t g : order) {
    const gmi_problem& p = problems[g];
    ktail = ktail || (p.K % 8) != 0;
    GroupDesc d;
    d.A = (const uint16_t*)p.A;
    d.B = (const uint16_t*)p.B;
    d.C = use_c ? (const uint16_t*)p.C : nullptr;
    d.D = (uint16_t*)p.D;
    d.lda = p.lda;
    d.ldb = p.ldb;
    d.ldc = p.ldc;
    d.ldd = p.ldd;
    d.M = p.M;
    d.N = p.N;
    d.K = p.K;
    d.tile_start = (int32_t)tiles;
    tiles += cdiv(p.M, grouped_tile_rows(shape, p.M)) * cdiv(p.N, bn);
    if (tiles > INT32_MAX) return fail(GMI_ERR_INVALID_ARG, "gemm_grouped: more than 2^31 - 1 output tiles");
    desc.push_back(d);
  }
  hipStream_t s = (hipStream_t)stream;
  if (live <= kInlineGroups)
    return hip_status(launch_grouped_inline(desc.data(), live, (int)tiles, shape, (int)dtype, ktail, alpha, beta, s),
                      "gemm_grouped: launch");
  GroupDesc* dev_desc = (GroupDesc*)((char*)workspace + kWorkspaceHeader);
  // the table travels in launch arguments (copied at enqueue), so the host
  // table may be reused immediately and the host does not wait for the stream
  gmi_status st = hip_status(stage_table(desc.data(), live, dev_desc, s), "gemm_grouped: staging the problem table");
  if (st != GMI_OK) return st;
  return hip_status(launch_grouped(dev_desc, live, (int)tiles, shape, (int)dtype, ktail, alpha, beta, s),
                    "gemm_grouped: launch");
}

}  // extern "C"

// The grouped GEMM with device-held group sizes: every check, then the
// table-building launch and the GEMM launch.  `own_scratch` selects the
// library's static per-device table instead of the caller's workspace (the
// allocation-free call); it is looked up only after every check has passed.
static gmi_status grouped_offsets(const char* who, int32_t count, const int32_t* offsets, int32_t rows, int32_t N,
                                  int32_t K, const void* A, int64_t lda, const void* B, int64_t ldb, int64_t stride_b,
                                  const void* C, int64_t ldc, void* D, int64_t ldd, gmi_dtype dtype, float alpha,
                                  float beta, void* workspace, size_t workspace_bytes, bool own_scratch,
                                  void* stream) {
  if (count < 0 || rows < 0 || N < 0 || K < 0)
    return fail(GMI_ERR_INVALID_ARG, "%s: negative size (count %d, rows %d, N %d, K %d)", who, count,
                rows, N, K);
  if (count > kMaxOffsetGroupCount)
    return fail(GMI_ERR_UNSUPPORTED, "%s: %d groups, at most %d", who, count, kMaxOffsetGroupCount);
  if (!gemm_dtype_ok(dtype))
    return fail(GMI_ERR_UNSUPPORTED, "%s: dtype %d not supported", who, (int)dtype);
  if (count == 0 || rows == 0 || N == 0) return GMI_OK;
  const bool use_c = beta != 0.0f;
  if (!offsets || !D || (K > 0 && (!A || !B)) || (use_c && !C))
    return fail(GMI_ERR_INVALID_ARG, "%s: a NULL operand", who);
  if ((K > 0 && (lda < K || ldb < K)) || ldd < N || (use_c && ldc < N))
    return fail(GMI_ERR_INVALID_ARG, "%s: a leading dimension below its row width", who);
  if (stride_b < 0) return fail(GMI_ERR_INVALID_ARG, "%s: stride_b %lld < 0", who, (long long)stride_b);
  if (lda > kMaxLd || ldb > kMaxLd || ldd > kMaxLd || (use_c && ldc > kMaxLd))
    return fail(GMI_ERR_UNSUPPORTED, "%s: a leading dimension above 2^22 elements", who);
  if (!f8_shape_ok(dtype, K, lda, ldb) || (dtype == GMI_F8E4M3 && stride_b % 16))
    return fail(GMI_ERR_UNSUPPORTED, "%s: fp8 needs K, lda, ldb and stride_b multiples of 16", who);
  if ((K > 0 && (!aligned16(A) || !aligned16(B) || lda % 8 || ldb % 8 || stride_b % 8)) || !aligned16(D) ||
      ldd % 8 || (use_c && (!aligned16(C) || ldc % 8)) || ((uintptr_t)offsets & 3u))
    return fail(GMI_ERR_MISALIGNED,
                "%s: pointers must be 16-byte aligned (offsets 4-byte), ld and stride_b multiples "
                "of 8", who);
  if (own_scratch) {
    const gmi_status st = scratch_address(who, &workspace);
    if (st != GMI_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < gmi_workspace_bytes(count))
    return fail(GMI_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes,
                gmi_workspace_bytes(count));
  if (!aligned16(workspace)) return fail(GMI_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", who);
  // The group sizes are unknown here: the shape is chosen from the fewest
  // tiles the rows can make (all rows in one group), and the tile total is
  // bounded by every group adding at most one partial tile row.
  const int shape = choose_shape([&](int bm, int bn) { return cdiv(rows, bm) * cdiv(N, bn); });
  const int64_t bound = (cdiv(rows, TINY_M) + count) * cdiv(N, tile_bn(shape));
  if (bound > INT32_MAX) return fail(GMI_ERR_INVALID_ARG, "%s: more than 2^31 - 1 output tiles", who);
  OffsetsLaunch p;
  p.offsets = offsets;
  p.count = count;
  p.rows = rows;
  p.N = N;
  p.K = K;
  p.A = A;
  p.B = B;
  p.C = use_c ? C : nullptr;
  p.D = D;
  p.lda = lda;
  p.ldb = ldb;
  p.stride_b = stride_b;
  p.ldc = ldc;
  p.ldd = ldd;
  p.total = (int32_t*)workspace;
  p.desc = (GroupDesc*)((char*)workspace + kWorkspaceHeader);
  return hip_status(launch_grouped_offsets(p, shape, (int)dtype, alpha, beta, (hipStream_t)stream), who);
}

extern "C" {

gmi_status gmi_gemm_grouped_offsets(int32_t count, const int32_t* offsets, int32_t rows, int32_t N, int32_t K,
                                    const void* A, int64_t lda, const void* B, int64_t ldb, int64_t stride_b,
                                    const void* C, int64_t ldc, void* D, int64_t ldd, gmi_dtype dtype,
                                    float alpha, float beta, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  g_last_error.clear();
  return grouped_offsets("gemm_grouped_offsets", count, offsets, rows, N, K, A, lda, B, ldb, stride_b, C, ldc, D, ldd,
                         dtype, alpha, beta, workspace, workspace_bytes, false, stream);
}

gmi_status gmi_gemm_grouped_offsets_noalloc(int32_t count, const int32_t* offsets, int32_t rows, int32_t N,
                                            int32_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                                            int64_t stride_b, const void* C, int64_t ldc, void* D, int64_t ldd,
                                            gmi_dtype dtype, float alpha, float beta, void* stream) {
  g_last_error.clear();
  return grouped_offsets("gemm_grouped_offsets_noalloc", count, offsets, rows, N, K, A, lda, B, ldb, stride_b, C, ldc,
                         D, ldd, dtype, alpha, beta, nullptr, 0, true, stream);
}

gmi_status gmi_gemm_ptr_array(int32_t L, int32_t M, int32_t N, int32_t K, const void* const* A, int64_t lda,
                              const void* const* B, int64_t ldb, const void* const* C, int64_t ldc, void* const* D,
                              int64_t ldd, gmi_dtype dtype, float alpha, float beta, void* stream) {
  g_last_error.clear();
  if (L < 0 || M < 0 || N < 0 || K < 0)
    return fail(GMI_ERR_INVALID_ARG, "gemm_ptr_array: negative size (L %d, M %d, N %d, K %d)", L, M, N, K);
  if (!gemm_dtype_ok(dtype)) return fail(GMI_ERR_UNSUPPORTED, "gemm_ptr_array: dtype %d not supported", (int)dtype);
  if (L == 0 || M == 0 || N == 0) return GMI_OK;
  const bool use_c = beta != 0.0f;
  if (!D || (K > 0 && (!A || !B)) || (use_c && !C))
    return fail(GMI_ERR_INVALID_ARG, "gemm_ptr_array: NULL pointer array");
  if ((K > 0 && (lda < K || ldb < K)) || ldd < N || (use_c && ldc < N))
    return fail(GMI_ERR_INVALID_ARG, "gemm_ptr_array: leading dimension below its row width");
  if ((K > 0 && (lda % 8 || ldb % 8)) || ldd % 8 || (use_c && ldc % 8))
    return fail(GMI_ERR_MISALIGNED, "gemm_ptr_array: leading dimensions must be multiples of 8");
  if (lda > kMaxLd || ldb > kMaxLd || ldd > kMaxLd || (use_c && ldc > kMaxLd))
    return fail(GMI_ERR_UNSUPPORTED, "gemm_ptr_array: a leading dimension above 2^22 elements");
  if (!f8_shape_ok(dtype, K, lda, ldb))
    return fail(GMI_ERR_UNSUPPORTED, "gemm_ptr_array: fp8 needs K, lda and ldb multiples of 16");
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)D | (uintptr_t)(use_c ? C : nullptr)) & 7u)
    return fail(GMI_ERR_MISALIGNED, "gemm_ptr_array: pointer arrays must be 8-byte aligned");
  const int shape = choose_shape([&](int bm, int bn) { return (int64_t)L * cdiv(M, bm) * cdiv(N, bn); });
  if ((int64_t)L * cdiv(M, tile_bm(shape)) * cdiv(N, tile_bn(shape)) > INT32_MAX)
    return fail(GMI_ERR_INVALID_ARG, "gemm_ptr_array: more than 2^31 - 1 output tiles");
  PtrArrayLaunch p;
  p.A = (const uint16_t* const*)A;
  p.B = (const uint16_t* const*)B;
  p.C = use_c ? (const uint16_t* const*)C : nullptr;
  p.D = (uint16_t* const*)D;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.ldd = ldd;
  p.L = L;
  p.M = M;
  p.N = N;
  p.K = K;
  return hip_status(launch_ptr_array(p, shape, (int)dtype, alpha, beta, (hipStream_t)stream),
                    "gemm_ptr_array: launch");
}

size_t gmi_prepack_w4_bytes(int32_t N, int32_t K) {
  if (N < 0 || K < 0) return 0;
  return (size_t)N * (size_t)K / 2;
}

gmi_status gmi_prepack_w4(const uint8_t* w_u4, int32_t N, int32_t K, uint8_t* w_prepacked, void* stream) {
  g_last_error.clear();
  if (N < 0 || K < 0) return fail(GMI_ERR_INVALID_ARG, "prepack_w4: negative size (N %d, K %d)", N, K);
  if (N % 16 || K % 128) return fail(GMI_ERR_UNSUPPORTED, "prepack_w4: needs N %% 16 == 0 and K %% 128 == 0");
  if (N == 0 || K == 0) return GMI_OK;
  if (!w_u4 || !w_prepacked) return fail(GMI_ERR_INVALID_ARG, "prepack_w4: NULL pointer");
  if (!aligned16(w_u4) || !aligned16(w_prepacked))
    return fail(GMI_ERR_MISALIGNED, "prepack_w4: pointers must be 16-byte aligned");
  const size_t bytes = gmi_prepack_w4_bytes(N, K);
  if (w_u4 < w_prepacked + bytes && w_prepacked < w_u4 + bytes)
    return fail(GMI_ERR_INVALID_ARG, "prepack_w4: input and output overlap");
  return hip_status(launch_prepack_w4(w_u4, N, K, w_prepacked, (hipStream_t)stream), "prepack_w4: launch");
}

size_t gmi_w4a16_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || N % 16 || K % 128) return 0;
  return w4a16_workspace(M, N, K);
}

// Shared by the two mixed-input entry points: every rule checked, then one
// launch.  `scales` NULL is the direct conversion (no scale), `zeros` NULL the
// conversion without zero point.
// Checks shared by the mixed-input entry points and the launch record they
// fill (M, split and partial are the caller's).  `M` is the row count, or
// for the grouped call the row capacity.  Returns GMI_OK with `nothing` set
// when there is no work.
static gmi_status mixed_prepare(const char* who, int32_t M, int32_t N, int32_t K, gmi_dtype x_dtype, const void* X,
                                int64_t ldx, const uint8_t* w_prepacked, gmi_w4_type w_type, const void* scales,
                                const uint8_t* zeros, int32_t group_size, void* Y, int64_t ldy, W4Launch& a,
                                bool& nothing) {
  nothing = false;
  if (M < 0 || N < 0 || K < 0) return fail(GMI_ERR_INVALID_ARG, "%s: negative size (%d, %d, %d)", who, M, N, K);
  if (!dtype_ok(x_dtype)) return fail(GMI_ERR_UNSUPPORTED, "%s: activation type %d not supported", who, (int)x_dtype);
  if (w_type != GMI_W4_UINT4 && w_type != GMI_W4_INT4)
    return fail(GMI_ERR_UNSUPPORTED, "%s: weight type %d not supported", who, (int)w_type);
  if (zeros && !scales)
    return fail(GMI_ERR_UNSUPPORTED, "%s: zero points without scales is not a conversion mode", who);
  if (!scales) group_size = K > 0 ? K : 128;  // unused without scales
  if (N % 16 || K % 128)
    return fail(GMI_ERR_UNSUPPORTED, "%s: needs N %% 16 == 0 and K %% 128 == 0 (prepack blocks)", who);
  if (group_size <= 0) return fail(GMI_ERR_INVALID_ARG, "%s: group_size %d <= 0", who, group_size);
  if (K > 0 && K % group_size)
    return fail(GMI_ERR_INVALID_ARG, "%s: K %d is not a multiple of group_size %d", who, K, group_size);
  if (group_size != K && group_size % 128)
    return fail(GMI_ERR_UNSUPPORTED, "%s: group_size must equal K or be a multiple of 128", who);
  if ((int64_t)N * K / 2 > INT32_MAX || (int64_t)M * ldx * 2 > INT32_MAX || ldy > kMaxLd)
    return fail(GMI_ERR_UNSUPPORTED, "%s: W (N*K/2 bytes) and X (M*ldx*2 bytes) must stay below 2^31 bytes", who);
  if (M == 0 || N == 0) {
    nothing = true;
    return GMI_OK;
  }
  if (!Y || (K > 0 && (!X || !w_prepacked))) return fail(GMI_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if ((K > 0 && ldx < K) || ldy < N) return fail(GMI_ERR_INVALID_ARG, "%s: ldx < K or ldy < N", who);
  if (!aligned16(Y) || ldy % 8 ||
      (K > 0 && (!aligned16(X) || !aligned16(w_prepacked) || (scales && !aligned16(scales)) ||
                 (zeros && !aligned16(zeros)) || ldx % 8)))
    return fail(GMI_ERR_MISALIGNED, "%s: pointers must be 16-byte aligned, ld multiples of 8", who);
  a.M = M;
  a.N = N;
  a.K = K;
  a.group = group_size;
  a.dt = (int)x_dtype;  // the kernels number the element types as gmi_dtype does
  a.X = (const uint16_t*)X;
  a.ldx = ldx;
  a.w = w_prepacked;
  a.scales = (const uint16_t*)scales;
  a.zeros = zeros;
  const int64_t groups = K > 0 ? K / group_size : 0;
  a.s_bytes = scales ? (uint32_t)(groups * N * 2) : 0u;
  a.z_bytes = zeros ? (uint32_t)(groups * N / 2) : 0u;
  a.sor = scales ? 0u : (x_dtype == GMI_BF16 ? 0x3F80u : 0x3C00u);  // 1.0
  // int4 (two's complement) read as offset binary: v = (q ^ 8) - 8, and
  // v_q - v_z = (q ^ 8) - (z ^ 8); without zero points z reads as 0, so the
  // zero becomes the constant 8
  a.wxor = w_type == GMI_W4_INT4 ? 0x88888888u : 0u;
  a.zxor = w_type == GMI_W4_INT4 ? 8u : 0u;
  a.Y = (uint16_t*)Y;
  a.ldy = ldy;
  a.split = 1;
  a.partial = nullptr;
  return GMI_OK;
}

static gmi_status mixed_gemm(const char* who, int32_t M, int32_t N, int32_t K, gmi_dtype x_dtype, const void* X,
                             int64_t ldx, const uint8_t* w_prepacked, gmi_w4_type w_type, const void* scales,
                             const uint8_t* zeros, int32_t group_size, void* Y, int64_t ldy, void* workspace,
                             size_t workspace_bytes, void* stream) {
  W4Launch a;
  bool nothing;
  const gmi_status st = mixed_prepare(who, M, N, K, x_dtype, X, ldx, w_prepacked, w_type, scales, zeros, group_size,
                                      Y, ldy, a, nothing);
  if (st != GMI_OK || nothing) return st;
  const size_t need = w4a16_workspace_for(M, N, K, a.dt);
  if (need > 0 && workspace && workspace_bytes >= need) {
    if (!aligned16(workspace)) return fail(GMI_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", who);
    a.split = w4a16_split(M, N, K, a.dt);
    a.partial = (float*)workspace;
  }
  return hip_status(launch_w4a16(a, (hipStream_t)stream), who);
}

gmi_status gmi_gemm_w4a16(int32_t M, int32_t N, int32_t K, const void* X, int64_t ldx, const uint8_t* w_prepacked,
                          const void* scales, const uint8_t* zeros, int32_t group_size, void* Y, int64_t ldy,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (M > 0 && N > 0 && K > 0 && (!scales || !zeros)) return fail(GMI_ERR_INVALID_ARG, "gemm_w4a16: NULL pointer");
  return mixed_gemm("gemm_w4a16", M, N, K, GMI_F16, X, ldx, w_prepacked, GMI_W4_UINT4, scales, zeros, group_size,
                    Y, ldy, workspace, workspace_bytes, stream);
}

gmi_status gmi_gemm_mixed_grouped(int32_t count, const int32_t* offsets, int32_t rows, int32_t N, int32_t K,
                                  gmi_dtype x_dtype, const void* X, int64_t ldx, const uint8_t* w_prepacked,
                                  int64_t w_stride, gmi_w4_type w_type, const void* scales, int64_t s_stride,
                                  const uint8_t* zeros, int64_t z_stride, int32_t group_size, void* Y, int64_t ldy,
                                  void* stream) {
  g_last_error.clear();
  const char* who = "gemm_mixed_grouped";
  if (count < 0) return fail(GMI_ERR_INVALID_ARG, "%s: count %d < 0", who, count);
  if (count > 65535) return fail(GMI_ERR_UNSUPPORTED, "%s: %d groups, at most 65535", who, count);
  if (count == 0) return GMI_OK;
  W4Launch a;
  bool nothing;
  gmi_status st = mixed_prepare(who, rows, N, K, x_dtype, X, ldx, w_prepacked, w_type, scales, zeros, group_size, Y,
                                ldy, a, nothing);
  if (st != GMI_OK) return st;
  if (nothing) return GMI_OK;
  if (!offsets) return fail(GMI_ERR_INVALID_ARG, "%s: offsets is NULL", who);
  if ((uintptr_t)offsets & 3u) return fail(GMI_ERR_MISALIGNED, "%s: offsets must be 4-byte aligned", who);
  const int64_t w_bytes = (int64_t)N * K / 2;
  if (w_stride < 0 || s_stride < 0 || z_stride < 0)
    return fail(GMI_ERR_INVALID_ARG, "%s: negative group stride", who);
  if (count > 1 && (w_stride < w_bytes || (scales && s_stride < (int64_t)a.s_bytes / 2) ||
                    (zeros && z_stride < (int64_t)a.z_bytes)))
    return fail(GMI_ERR_INVALID_ARG, "%s: a group stride is smaller than one group's data", who);
  if (w_stride % 16 || (s_stride * 2) % 16 || z_stride % 16)
    return fail(GMI_ERR_MISALIGNED, "%s: group strides must keep every group's data 16-byte aligned", who);
  W4Grouped gq;
  gq.base = a;
  gq.offsets = offsets;
  gq.count = count;
  gq.rows = rows;
  gq.w_stride = w_stride;
  gq.s_stride = scales ? s_stride : 0;
  gq.z_stride = zeros ? z_stride : 0;
  return hip_status(launch_w4a16_grouped(gq, (hipStream_t)stream), who);
}

gmi_status gmi_gemm_mixed(int32_t M, int32_t N, int32_t K, gmi_dtype x_dtype, const void* X, int64_t ldx,
                          const uint8_t* w_prepacked, gmi_w4_type w_type, const void* scales, const uint8_t* zeros,
                          int32_t group_size, void* Y, int64_t ldy, void* workspace, size_t workspace_bytes,
                          void* stream) {
  g_last_error.clear();
  return mixed_gemm("gemm_mixed", M, N, K, x_dtype, X, ldx, w_prepacked, w_type, scales, zeros, group_size, Y, ldy,
                    workspace, workspace_bytes, stream);
}

// Checks shared by the weight-gradient calls; fills the plan.
static gmi_status wgrad_check(const char* who, int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R,
                              int32_t S, int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w,
                              int32_t dil_h, int32_t dil_w, int32_t groups, WgradPlan& plan) {
  if (N < 1 || H < 1 || W < 1 || C < 1 || K < 1 || R < 1 || S < 1)
    return fail(GMI_ERR_INVALID_ARG, "%s: sizes must be positive", who);
  if (pad_h < 0 || pad_w < 0 || stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1)
    return fail(GMI_ERR_INVALID_ARG, "%s: padding >= 0, stride >= 1 and dilation >= 1 required", who);
  if (dil_h > 8 || dil_w > 8 || stride_h > 8 || stride_w > 8)
    return fail(GMI_ERR_UNSUPPORTED, "%s: stride and dilation must be in [1, 8]", who);
  if (C % 8 || K % 8) return fail(GMI_ERR_MISALIGNED, "%s: C and K must be multiples of 8", who);
  if (groups < 1 || C % groups || K % groups)
    return fail(GMI_ERR_INVALID_ARG, "%s: groups %d must divide C %d and K %d", who, groups, C, K);
  if ((K / groups) % 8)
    return fail(GMI_ERR_UNSUPPORTED, "%s: output channels per group must be a multiple of 8", who);
  if (!plan_wgrad(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, groups, plan))
    return fail(GMI_ERR_INVALID_ARG, "%s: the filter does not fit the padded image", who);
  const int64_t n8 = plan.N8;
  if ((int64_t)C * H * W * n8 * 2 > INT32_MAX || (int64_t)plan.P * plan.Q * n8 > kMaxLd ||
      (int64_t)K * plan.P * plan.Q * n8 * 2 > INT32_MAX ||
      (int64_t)C * plan.Rp * plan.Sp > INT32_MAX || (int64_t)N * H * W * C > INT32_MAX ||
      (int64_t)N * plan.P * plan.Q * K > INT32_MAX)
    return fail(GMI_ERR_UNSUPPORTED, "%s: a transposed operand above 2^31 bytes or P*Q*N above 2^22 taps", who);
  return GMI_OK;
}

size_t gmi_conv2d_wgrad_workspace_bytes(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S,
                                        int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w,
                                        int32_t dil_h, int32_t dil_w, int32_t groups) {
  WgradPlan plan;
  const std::string saved = g_last_error;
  const gmi_status st = wgrad_check("conv2d_wgrad_workspace_bytes", N, H, W, C, K, R, S, pad_h, pad_w, stride_h,
                                    stride_w, dil_h, dil_w, groups, plan);
  g_last_error = saved;
  return st == GMI_OK ? plan.bytes : 0;
}

gmi_status gmi_conv2d_wgrad_implicit(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S,
                                     int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w, int32_t dil_h,
                                     int32_t dil_w, int32_t groups, const void* x, const void* dy, const void* c_in,
                                     void* dw,
                                     gmi_dtype dtype, float alpha, float beta, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  const char* who = "conv2d_wgrad";
  if (!dtype_ok(dtype)) return fail(GMI_ERR_UNSUPPORTED, "%s: dtype %d not supported", who, (int)dtype);
  WgradPlan plan;
  const gmi_status st =
      wgrad_check(who, N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, groups, plan);
  if (st != GMI_OK) return st;
  const bool use_c = beta != 0.0f;
  if (!x || !dy || !dw || (use_c && !c_in)) return fail(GMI_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dw) || (use_c && !aligned16(c_in)))
    return fail(GMI_ERR_MISALIGNED, "%s: pointers must be 16-byte aligned", who);
  if (!workspace || workspace_bytes < plan.bytes)
    return fail(GMI_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes, plan.bytes);
  if (!aligned16(workspace)) return fail(GMI_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", who);
  return hip_status(launch_conv_wgrad(plan, (const uint16_t*)x, (const uint16_t*)dy,
                                      use_c ? (const uint16_t*)c_in : nullptr, (uint16_t*)dw, (char*)workspace,
                                      (int)dtype, alpha, beta, (hipStream_t)stream),
                    who);
}

size_t gmi_conv2d_dgrad_workspace_bytes(int32_t C, int32_t K, int32_t R, int32_t S) {
  if (C < 1 || K < 1 || R < 1 || S < 1) return 0;
  return ((size_t)C * K * R * S * 2 + 255) / 256 * 256;
}

gmi_status gmi_conv2d_dgrad_implicit(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S,
                                     int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w, int32_t dil_h,
                                     int32_t dil_w, const void* dy, const void* w, const void* c_in, void* dx,
                                     gmi_dtype dtype, float alpha, float beta, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  const char* who = "conv2d_dgrad";
  if (N < 0 || H < 1 || W < 1 || C < 1 || K < 1 || R < 1 || S < 1)
    return fail(GMI_ERR_INVALID_ARG, "%s: sizes must be positive (N >= 0)", who);
  if (pad_h < 0 || pad_w < 0 || stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1)
    return fail(GMI_ERR_INVALID_ARG, "%s: padding >= 0, stride >= 1 and dilation >= 1 required", who);
  if (stride_h > 8 || stride_w > 8)
    return fail(GMI_ERR_UNSUPPORTED, "%s: the traversal stride must be in [1, 8]", who);
  if (!dtype_ok(dtype)) return fail(GMI_ERR_UNSUPPORTED, "%s: dtype %d not supported", who, (int)dtype);
  if (C % 8 || K % 8) return fail(GMI_ERR_MISALIGNED, "%s: C and K must be multiples of 8", who);
  const int64_t Ph = (int64_t)H + 2 * (int64_t)pad_h - (int64_t)dil_h * (R - 1) - 1;
  const int64_t Qw = (int64_t)W + 2 * (int64_t)pad_w - (int64_t)dil_w * (S - 1) - 1;
  if (Ph < 0 || Qw < 0) return fail(GMI_ERR_INVALID_ARG, "%s: the filter does not fit the padded image", who);
  const int64_t P = Ph / stride_h + 1, Q = Qw / stride_w + 1;
  if ((int64_t)N * H * W > INT32_MAX || (int64_t)N * P * Q > INT32_MAX || (int64_t)R * S * K > kMaxLd ||
      (int64_t)N * P * Q * K * 2 > INT32_MAX || C > kMaxLd ||
      ((stride_h > 1 || stride_w > 1) && (int64_t)N * H * W * C * 2 > INT32_MAX))
    return fail(GMI_ERR_UNSUPPORTED,
                "%s: dy (or, for a stride above 1, dx) above 2^31 bytes, R*S*K above 2^22 or too many pixels", who);
  if (N == 0) return GMI_OK;
  const bool use_c = beta != 0.0f;
  if (!dy || !w || !dx || (use_c && !c_in)) return fail(GMI_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(dy) || !aligned16(w) || !aligned16(dx) || (use_c && !aligned16(c_in)))
    return fail(GMI_ERR_MISALIGNED, "%s: pointers must be 16-byte aligned", who);
  if (!workspace || workspace_bytes < gmi_conv2d_dgrad_workspace_bytes(C, K, R, S))
    return fail(GMI_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes,
                gmi_conv2d_dgrad_workspace_bytes(C, K, R, S));
  if (!aligned16(workspace)) return fail(GMI_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", who);
  ConvLaunch a;  // the forward problem; x is dy and y is dx here
  a.x = (const uint16_t*)dy;
  a.w = (const uint16_t*)w;
  a.c = use_c ? (const uint16_t*)c_in : nullptr;
  a.y = (uint16_t*)dx;
  a.N = N;
  a.H = H;
  a.W = W;
  a.C = C;
  a.K = K;
  a.R = R;
  a.S = S;
  a.P = (int)P;
  a.Q = (int)Q;
  a.ph = pad_h;
  a.pw = pad_w;
  a.sh = stride_h;
  a.sw = stride_w;
  a.dh = dil_h;
  a.dw = dil_w;
  return hip_status(launch_conv_dgrad(a, (uint16_t*)workspace, (int)dtype, alpha, beta, (hipStream_t)stream), who);
}

// the forward pass, with or without the fused epilogue (bias NULL and act 0)
static gmi_status conv_fprop(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S,
                             int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w, int32_t dil_h,
                             int32_t dil_w, const void* x, const void* w, const void* c_in, const void* bias, void* y,
                             gmi_dtype dtype, float alpha, float beta, int act, void* stream) {
  if (act != GMI_ACT_NONE && act != GMI_ACT_RELU)
    return fail(GMI_ERR_INVALID_ARG, "conv2d_fprop: activation %d is not one of GMI_ACT_NONE, GMI_ACT_RELU", act);
  if (bias && !aligned16(bias)) return fail(GMI_ERR_MISALIGNED, "conv2d_fprop: bias must be 16-byte aligned");
  if (N < 0 || H < 1 || W < 1 || C < 1 || K < 1 || R < 1 || S < 1)
    return fail(GMI_ERR_INVALID_ARG, "conv2d_fprop: sizes must be positive (N >= 0)");
  if (pad_h < 0 || pad_w < 0 || stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1)
    return fail(GMI_ERR_INVALID_ARG, "conv2d_fprop: padding >= 0, stride >= 1 and dilation >= 1 required");
  if (stride_h > 8 || stride_w > 8)
    return fail(GMI_ERR_UNSUPPORTED, "conv2d_fprop: traversal stride must be in [1, 8]");
  if (!dtype_ok(dtype)) return fail(GMI_ERR_UNSUPPORTED, "conv2d_fprop: dtype %d not supported", (int)dtype);
  if (C % 8 || K % 8)
    return fail(GMI_ERR_MISALIGNED, "conv2d_fprop: C and K must be multiples of 8 (128-bit channel runs)");
  const int64_t P = ((int64_t)H + 2 * (int64_t)pad_h - (int64_t)dil_h * (R - 1) - 1) / stride_h + 1;
  const int64_t Q = ((int64_t)W + 2 * (int64_t)pad_w - (int64_t)dil_w * (S - 1) - 1) / stride_w + 1;
  if ((int64_t)H + 2 * (int64_t)pad_h - (int64_t)dil_h * (R - 1) - 1 < 0 ||
      (int64_t)W + 2 * (int64_t)pad_w - (int64_t)dil_w * (S - 1) - 1 < 0 || P < 1 || Q < 1)
    return fail(GMI_ERR_INVALID_ARG, "conv2d_fprop: the filter does not fit the padded image (P, Q < 1)");
  if ((int64_t)N * P * Q > INT32_MAX || (int64_t)N * H * W > INT32_MAX || (int64_t)R * S * C > INT32_MAX)
    return fail(GMI_ERR_INVALID_ARG, "conv2d_fprop: problem too large for 32-bit pixel / tap indices");
  if ((int64_t)N * H * W * C * 2 > INT32_MAX || (int64_t)R * S * C > kMaxLd || K > kMaxLd)
    return fail(GMI_ERR_UNSUPPORTED, "conv2d_fprop: activation above 2^31 bytes or R*S*C above 2^22");
  if (N == 0) return GMI_OK;
  const bool use_c = beta != 0.0f;
  if (!x || !w || !y || (use_c && !c_in)) return fail(GMI_ERR_INVALID_ARG, "conv2d_fprop: NULL pointer");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (use_c && !aligned16(c_in)))
    return fail(GMI_ERR_MISALIGNED, "conv2d_fprop: pointers must be 16-byte aligned");
  ConvLaunch a;
  a.x = (const uint16_t*)x;
  a.w = (const uint16_t*)w;
  a.c = use_c ? (const uint16_t*)c_in : nullptr;
  a.y = (uint16_t*)y;
  a.N = N;
  a.H = H;
  a.W = W;
  a.C = C;
  a.K = K;
  a.R = R;
  a.S = S;
  a.P = (int)P;
  a.Q = (int)Q;
  a.ph = pad_h;
  a.pw = pad_w;
  a.sh = stride_h;
  a.sw = stride_w;
  a.dh = dil_h;
  a.dw = dil_w;
  a.bias = (const uint16_t*)bias;
  a.act = act;
  const int64_t Mg = (int64_t)N * P * Q;
  const int shape = choose_shape([&](int bm, int bn) { return cdiv(Mg, bm) * cdiv(K, bn); });
  return hip_status(launch_conv_fprop(a, shape, (int)dtype, alpha, beta, (hipStream_t)stream),
                    "conv2d_fprop: launch");
}

gmi_status gmi_conv2d_fprop_implicit(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S,
                                     int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w, int32_t dil_h,
                                     int32_t dil_w, const void* x, const void* w, const void* c_in, void* y,
                                     gmi_dtype dtype, float alpha, float beta, void* stream) {
  g_last_error.clear();
  return conv_fprop(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, x, w, c_in, nullptr, y,
                    dtype, alpha, beta, GMI_ACT_NONE, stream);
}

gmi_status gmi_conv2d_fprop_implicit_fused(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R,
                                           int32_t S, int32_t pad_h, int32_t pad_w, int32_t stride_h,
                                           int32_t stride_w, int32_t dil_h, int32_t dil_w, const void* x,
                                           const void* w, const void* c_in, const void* bias, void* y,
                                           gmi_dtype dtype, float alpha, float beta, gmi_activation act,
                                           void* stream) {
  g_last_error.clear();
  return conv_fprop(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, x, w, c_in, bias, y, dtype,
                    alpha, beta, (int)act, stream);
}

}  // extern "C"
