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
  // split over the taps: work item w is tile w % total_tiles, k-tiles
  // (w / total_tiles) * kt_split .. + kt_split -- the tiles of one tap range
  // run together and share its filter slice in L2; with `partial` set,
  // every item stores its fp32 sum to partial[w / total_tiles] ([M][Nk])
  // instead of y
  int split, kt_split;
  float* partial;
  // independent groups (the grouped weight gradient): group j gathers from
  // g.x + j * x_group, reads filters w + j * w_group and writes partials
  // partial + j * part_group; work items run group-major
  int groups;
  int64_t x_group, w_group, part_group;
  // fused epilogue (see Tile): per-output-channel bias, activation
  const uint16_t* bias;
  int act;
  // output rows on a strided pixel grid (MAPPED launches)
  RowMap map;
};

// Tile ids run n-tile fastest: the few n-tiles of a pixel block are
// consecutive, so one XCD gathers each activation panel once into its L2.
template <class Cfg, int DT, bool MAPPED>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WGS_PER_CU) void k_conv_fprop(ConvArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
  const int G = gridDim.x;
  const int per_group = a.total_tiles * a.split;
  const int total = per_group * a.groups;
  const int nkt = (a.g.Kg + Cfg::BK - 1) / Cfg::BK;
  for (int base = 0; base < total; base += G) {
    const int work = base + remap_slot(blockIdx.x, G);
    if (work >= total) break;
    const int grp = work / per_group, rest = work - grp * per_group;
    const int sidx = rest / a.total_tiles, tile = rest - sidx * a.total_tiles;
    const int kt0 = sidx * a.kt_split;
    const int nk = min(a.kt_split, nkt - kt0);
    const int k0 = kt0 * Cfg::BK;
    Tile t;
    t.M = a.M;
    t.N = a.Nk;
    t.K = min(nk * Cfg::BK, a.g.Kg - k0);
    t.m0 = (tile / a.tiles_n) * Cfg::BM;
    t.n0 = (tile % a.tiles_n) * Cfg::BN;
    t.C = a.c;
    t.ldc = a.Nk;
    t.D = a.y;
    t.ldd = a.Nk;
    t.bias = a.bias;
    t.act = a.act;
    ConvGeom gg = a.g;
    gg.x += grp * a.x_group;
    ConvLoader<Cfg, Cfg::BM> al;
    FilterLoader<Cfg, Cfg::BN> bl;
    al.init(gg, t.m0, t.M, kt0);
    bl.init(a.w + grp * a.w_group, gg, t.n0, t.N, kt0);
    f32x16 acc[Cfg::TM][Cfg::TN];
    mainloop<Cfg, DT>(lds, al, bl, nk, acc);
    if (a.partial)
      store_partial<Cfg>(t, acc, a.partial + grp * a.part_group + (int64_t)sidx * a.M * a.Nk);
    else
      store_tile<Cfg, DT, MAPPED>(t, acc, a.alpha, a.beta, lds, a.map);
  }
}

// The phases of a strided data gradient in one persistent launch.  Phase p
// is the forward gather over dy of its own geometry and filter slice,
// writing its strided grid of dx pixels through the row map (off0 its own,
// the strides shared).  Its tiles are ids tile_start .. of the launch, in
// the order the host sorted the phases (longest reduction first, so the
// static walk hands out the long tiles first); a tile finds its phase by a
// scan of the prefix, which every lane does alike.
constexpr int kMaxConvPhases = 16;
struct PhaseDesc {
  ConvGeom g;
  const uint16_t* w;  // the phase's filter slice [C][taps][K]
  int64_t map_off0;
  int M, Hp, Wp;    // GEMM rows N * Hp * Wp: the phase's pixel grid
  int tile_start;  // first tile id of the phase
};
struct PhasesArgs {
  PhaseDesc ph[kMaxConvPhases];
  int count, total_tiles, tiles_n, Nk;
  const uint16_t* c;
  uint16_t* y;
  float alpha, beta;
  int64_t map_img, map_rstep, map_cstep;
  uint32_t map_bytes;
};
static_assert(sizeof(PhasesArgs) <= 4096, "kernel arguments are limited to 4 KB");

template <class Cfg, int DT>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WGS_PER_CU) void k_conv_phases(PhasesArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
  const int G = gridDim.x;
  const PhaseDesc* ph = a.ph;
  for (int base = 0; base < a.total_tiles; base += G) {
    const int work = base + remap_slot(blockIdx.x, G);
    if (work >= a.total_tiles) break;
    int p = 0;
    for (int i = 1; i < a.count; ++i) p = work >= ph[i].tile_start ? i : p;
    const PhaseDesc& d = ph[p];
    const int tile = work - d.tile_start;
    Tile t;
    t.M = d.M;
    t.N = a.Nk;
    t.K = d.g.Kg;
    t.m0 = (tile / a.tiles_n) * Cfg::BM;
    t.n0 = (tile % a.tiles_n) * Cfg::BN;
    t.C = a.c;
    t.ldc = a.Nk;
    t.D = a.y;
    t.ldd = a.Nk;
    t.bias = nullptr;
    t.act = 0;
    ConvLoader<Cfg, Cfg::BM> al;
    FilterLoader<Cfg, Cfg::BN> bl;
    al.init(d.g, t.m0, t.M, 0);
    bl.init(d.w, d.g, t.n0, t.N, 0);
    f32x16 acc[Cfg::TM][Cfg::TN];
    mainloop<Cfg, DT>(lds, al, bl, (d.g.Kg + Cfg::BK - 1) / Cfg::BK, acc);
    const RowMap map{d.Hp, d.Wp, d.map_off0, a.map_img, a.map_rstep, a.map_cstep, a.map_bytes};
    store_tile<Cfg, DT, true>(t, acc, a.alpha, a.beta, lds, map);
  }
}

using ConvCfg256 = TileCfg<256, 256, 4, 2, 64, 2, 5>;
using ConvCfg256x128 = TileCfg<256, 128, 2, 2, 32, 3>;
using ConvCfg128 = TileCfg<128, 128, 2, 2, 32, 4>;

static int conv_bk(int shape) {
  return shape == TILE_256x256 ? ConvCfg256::BK : shape == TILE_256x128 ? ConvCfg256x128::BK : ConvCfg128::BK;
}

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
                 0,     0};
  // channel-block-major k order when the channels fill whole k-tiles and the
  // launch is not split over k (a split keeps each range's taps together)
  const int bk = conv_bk(shape);
  if (p.R * p.S > 1 && p.C % bk == 0 && p.split == 1) {
    a.g.prs = p.R * p.S;
    a.g.pcb = p.C / bk;
  }
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
  a.split = p.split;
  a.kt_split = p.kt_split;
  a.partial = p.partial;
  a.groups = p.groups;
  a.x_group = p.x_group;
  a.w_group = p.w_group;
  a.part_group = p.part_group;
  a.bias = p.bias;
  a.act = p.act;
  const bool mapped = p.map_bytes > 0;
  a.map = RowMap{p.P, p.Q, p.map_off0, p.map_img, p.map_rstep, p.map_cstep, p.map_bytes};
  const int resident = device_cu_count() * tile_wgs_per_cu(shape);
  int grid = (a.total_tiles * a.split * a.groups + XCDS - 1) / XCDS * XCDS;
  if (grid > resident) grid = resident / XCDS * XCDS;
  if (grid < XCDS) grid = XCDS;
#define GMI_CONV_LAUNCH(CFG)                                                                              \
  do {                                                                                                    \
    if (dtype == DT_F16) {                                                                                \
      if (mapped) hipLaunchKernelGGL((k_conv_fprop<CFG, DT_F16, true>), dim3(grid), dim3(CFG::THREADS), 0, stream, a);   \
      else hipLaunchKernelGGL((k_conv_fprop<CFG, DT_F16, false>), dim3(grid), dim3(CFG::THREADS), 0, stream, a);        \
    } else {                                                                                              \
      if (mapped) hipLaunchKernelGGL((k_conv_fprop<CFG, DT_BF16, true>), dim3(grid), dim3(CFG::THREADS), 0, stream, a);  \
      else hipLaunchKernelGGL((k_conv_fprop<CFG, DT_BF16, false>), dim3(grid), dim3(CFG::THREADS), 0, stream, a);       \
    }                                                                                                     \
  } while (0)
  if (shape == TILE_256x256)
    GMI_CONV_LAUNCH(ConvCfg256);
  else if (shape == TILE_256x128)
    GMI_CONV_LAUNCH(ConvCfg256x128);
  else
    GMI_CONV_LAUNCH(ConvCfg128);
#undef GMI_CONV_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Data gradient, the page's dgrad operator:
//   dx[n][h][w][c] = sum over (p, q, k, r, s) with p sh - ph + r dh = h and
//                    q sw - pw + s dw = w of dy[n][p][q][k] w[k][r][s][c].
// For stride 1 the page runs it through the same im2col operand with the
// filter-tap strides negated: the forward gather over dy with padding -ph and
// dilation -dh.  For a stride s > 1 the page's strided dgrad walks, for each
// output pixel, only the taps that reach it: p = (h + ph - r dh) / s must be
// an integer, so the taps of output row h are those with r dh = h + ph
// (mod s).  The rows h with h + ph = a (mod s) form one phase; its taps are
// r = r_a + t s / g (g = gcd(dh, s), r_a the first), and with h = a - ph +
// s (lo + i) the tap t reads dy row p = i + shift - t dh / g.  So each phase
// is a stride-1 forward gather over dy with padding -shift and dilation
// -dh / g over its own slice of the filter, writing the strided grid of dx
// pixels of that phase; the phases partition both the dx pixels and the
// taps, so no multiply touches a tap that misses.  Each dimension splits
// this way; a phase with pixels but no taps writes beta C (or zeros).
// The GEMM's B operand is each phase's filter slice with its reduction
// (t, u, k) contiguous per column c: [C][taps][K].
// ---------------------------------------------------------------------------
// The filter taps of one phase: output tap b (of the phase's Rp x Sp, row
// major) is input tap (r0 + (b / Sp) rstep) S + s0 + (b % Sp) sstep.
struct TapMap {
  int Sp, r0, rstep, s0, sstep, S;
  __device__ __forceinline__ int operator()(int b) const { return (r0 + (b / Sp) * rstep) * S + s0 + (b % Sp) * sstep; }
};

// out[c][b][a] = in[a][taps(b)][c] for a < A, 0 for A <= a < Ap (in holds
// Bin taps per a, out Bout): one 64 x 64 (a, c) block per workgroup, moved
// in 16-byte runs: 8 consecutive c on the way in, 8 consecutive a on the way
// out (C % 8 == 0, Ap % 8 == 0).  When Ap < 64 a block takes nb = 64 / Ap
// consecutive b instead of one, so each of its rows is whole (every a of one
// b) and each c's output run covers nb b: 128 bytes at Ap = 32, a whole
// line, where one b per block wrote half lines from two workgroups.  One
// launch runs a table of such jobs (the filter slices of every phase of a
// strided data gradient, or x and dy of a weight gradient): grid z walks the
// jobs' b groups one after another, and each job ignores the (a, c) blocks
// past its own extent.
constexpr int kMaxTransposeJobs = 16;
struct TransposeJob {
  const uint16_t* in;
  uint16_t* out;
  int A, Bin, Bout, C, Ap;
  TapMap taps;
  int nb;  // b per workgroup
  int z0;  // first b group of the job in the launch's walk
};
struct TransposeJobs {
  TransposeJob job[kMaxTransposeJobs];
  int count, total;  // jobs; sum of their b groups
};
static_assert(sizeof(TransposeJobs) <= 4096, "kernel arguments are limited to 4 KB");

// In LDS the block is held as 32-bit pairs of rows: word (c, p) packs rows
// 2p and 2p + 1 of column c (one v_perm per word on the way in), so a
// column's 8 consecutive rows are one 16-byte read on the way out.  Column c
// holds its 32 words in 16-byte groups whose order is XOR-ed with c / 8: the
// 8 writes of an instruction touch each bank at most twice, and a read
// instruction's 16-lane groups (8 row groups of 2 columns) none twice.
__global__ __launch_bounds__(256) void k_transpose_outer(TransposeJobs jobs) {
  __shared__ __attribute__((aligned(16))) uint32_t t[64 * 32];
  const int hi = threadIdx.x / 8, lo = threadIdx.x % 8;
  const TransposeJob* js = jobs.job;
  for (int z = blockIdx.z; z < jobs.total; z += gridDim.z) {
    int q = 0;
    for (int i = 1; i < jobs.count; ++i) q = z >= js[i].z0 ? i : q;
    const TransposeJob& jb = js[q];
    const int a0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    if (a0 >= jb.Ap || c0 >= jb.C) continue;  // past this job's extent: the whole workgroup skips alike
    // block row r: b = b0 + r / ab, a = a0 + r % ab (ab a multiple of 8, so
    // an 8-row run never spans two b)
    const int ab = jb.Ap < 64 ? jb.Ap : 64, b0 = (z - jb.z0) * jb.nb;
    {
      // rows 2 hi and 2 hi + 1, columns 8 lo .. 8 lo + 7
      u32x4 v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 2 * hi + h, bl = r / ab, a = a0 + r % ab, b = b0 + bl, c = c0 + lo * 8;
        v[h] = u32x4{0, 0, 0, 0};
        if (bl < jb.nb && b < jb.Bout && a < jb.A && c < jb.C)
          v[h] = *(const u32x4*)(jb.in + ((int64_t)a * jb.Bin + jb.taps(b)) * jb.C + c);
      }
      const int slot = (((hi >> 2) ^ lo) << 2) + (hi & 3);
#pragma unroll
      for (int k = 0; k < 8; ++k)  // column 8 lo + k: the two rows' element k
        t[(lo * 8 + k) * 32 + slot] = __builtin_amdgcn_perm(v[1][k / 2], v[0][k / 2], k % 2 ? 0x07060302u : 0x05040100u);
    }
    __syncthreads();
    {
      // rows 8 lo .. 8 lo + 7 of columns hi and hi + 32
      const int r = lo * 8, bl = r / ab, a = a0 + r % ab, b = b0 + bl;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cc = hi + 32 * j, c = c0 + cc;
        if (bl < jb.nb && b < jb.Bout && c < jb.C && a < jb.Ap)
          *(u32x4*)(jb.out + ((int64_t)c * jb.Bout + b) * jb.Ap + a) = *(const u32x4*)(t + cc * 32 + ((lo ^ (cc >> 3)) << 2));
      }
    }
    __syncthreads();
  }
}

// every job of the table in one launch
static hipError_t transpose_jobs(TransposeJobs& jobs, hipStream_t stream) {
  int cmax = 0, amax = 0, z = 0;
  for (int i = 0; i < jobs.count; ++i) {
    TransposeJob& jb = jobs.job[i];
    jb.nb = jb.Ap < 64 ? 64 / jb.Ap : 1;
    jb.z0 = z;
    z += (jb.Bout + jb.nb - 1) / jb.nb;
    cmax = jb.C > cmax ? jb.C : cmax;
    amax = jb.Ap > amax ? jb.Ap : amax;
  }
  jobs.total = z;
  if (z == 0) return hipSuccess;
  const dim3 grid((cmax + 63) / 64, (amax + 63) / 64, z < 65535 ? z : 65535);
  hipLaunchKernelGGL(k_transpose_outer, grid, dim3(256), 0, stream, jobs);
  return hipGetLastError();
}

// out[c][b][a] = in[a][taps(b)][c] as a job (every tap in order by default)
static TransposeJob transpose_job(const uint16_t* in, uint16_t* out, int A, int B, int C, int Ap,
                                  TapMap taps = TapMap{1 << 30, 0, 0, 0, 1, 1}, int Bin = -1) {
  TransposeJob j;
  j.in = in;
  j.out = out;
  j.A = A;
  j.Bin = Bin < 0 ? B : Bin;
  j.Bout = B;
  j.C = C;
  j.Ap = Ap;
  j.taps = taps;
  j.nb = 1;
  j.z0 = 0;
  return j;
}

static int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }  // b > 0
static int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// One dimension of one phase: output rows h = a - pad + stride (lo + i),
// i < size; taps first + t step, t < count; tap t of row i reads input row
// i + shift - t (dil / gcd(dil, stride)).
struct Phase1D {
  int first, step, count, lo, size, shift, dil;
};
static Phase1D phase_1d(int a, int R, int pad, int stride, int dil, int H) {
  Phase1D p;
  const int g = gcd_int(dil, stride);
  p.step = stride / g;
  p.dil = dil / g;
  p.first = -1;
  for (int r = 0; r < R && r < p.step; ++r)
    if ((r * dil) % stride == a) {
      p.first = r;
      break;
    }
  p.count = p.first < 0 ? 0 : (R - 1 - p.first) / p.step + 1;
  p.lo = -floor_div(a - pad, stride);  // the first i with a - pad + stride i >= 0
  const int last = floor_div(H - 1 - a + pad, stride);
  p.size = last >= p.lo ? last - p.lo + 1 : 0;
  p.shift = p.first < 0 ? 0 : p.lo + (a - p.first * dil) / stride;  // an exact quotient
  return p;
}

// The geometry of one phase's forward view: a stride-1 gather over dy with
// padding -shift and dilation -dil, its filter slice [C][taps][K]
static ConvLaunch phase_view(const ConvLaunch& p, const Phase1D& ph, const Phase1D& pw, const uint16_t* wp) {
  ConvLaunch f;
  f.x = p.x;
  f.w = wp;
  f.c = p.c;
  f.y = p.y;
  f.N = p.N;
  f.H = p.P;
  f.W = p.Q;
  f.C = p.K;
  f.K = p.C;
  f.R = ph.count;
  f.S = pw.count;
  f.P = ph.size;
  f.Q = pw.size;
  f.ph = -ph.shift;
  f.pw = -pw.shift;
  f.sh = 1;
  f.sw = 1;
  f.dh = -ph.dil;
  f.dw = -pw.dil;
  return f;
}

template <class Cfg>
static hipError_t launch_phases(PhasesArgs& a, int dtype, hipStream_t stream) {
  const int resident = device_cu_count() * Cfg::WGS_PER_CU;
  int grid = (a.total_tiles + XCDS - 1) / XCDS * XCDS;
  if (grid > resident) grid = resident / XCDS * XCDS;
  if (grid < XCDS) grid = XCDS;
  if (dtype == DT_F16)
    hipLaunchKernelGGL((k_conv_phases<Cfg, DT_F16>), dim3(grid), dim3(Cfg::THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((k_conv_phases<Cfg, DT_BF16>), dim3(grid), dim3(Cfg::THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_conv_dgrad(const ConvLaunch& p, uint16_t* wt, int dtype, float alpha, float beta,
                             hipStream_t stream) {
  // p describes the forward problem (x: N x H x W x C, y: N x P x Q x K);
  // here p.x is dy, p.y is dx and p.c the dx-shaped C
  const bool strided = p.sh > 1 || p.sw > 1;
  struct Phase {
    ConvLaunch f;
    int64_t off0;
  };
  Phase phases[64];
  int count = 0;
  int64_t woff = 0;  // the phases' filter slices, one after another
  TransposeJobs jobs;  // their rearrangement, kMaxTransposeJobs slices per launch
  jobs.count = 0;
  for (int a = 0; a < p.sh; ++a) {
    const Phase1D ph = phase_1d(a, p.R, p.ph, p.sh, p.dh, p.H);
    if (ph.size == 0) continue;
    for (int b = 0; b < p.sw; ++b) {
      const Phase1D pw = phase_1d(b, p.S, p.pw, p.sw, p.dw, p.W);
      if (pw.size == 0) continue;
      uint16_t* wp = wt + woff;
      const int taps = ph.count * pw.count;
      if (taps > 0) {
        if (jobs.count == kMaxTransposeJobs) {
          const hipError_t e = transpose_jobs(jobs, stream);
          if (e != hipSuccess) return e;
          jobs.count = 0;
        }
        jobs.job[jobs.count++] = transpose_job(p.w, wp, p.K, taps, p.C, p.K,
                                               TapMap{pw.count, ph.first, ph.step, pw.first, pw.step, p.S}, p.R * p.S);
        woff += (int64_t)taps * p.C * p.K;
      }
      phases[count].f = phase_view(p, ph, pw, wp);
      phases[count].off0 = ((int64_t)(a - p.ph + p.sh * ph.lo) * p.W + (b - p.pw + p.sw * pw.lo)) * p.C;
      ++count;
    }
  }
  if (jobs.count > 0) {
    const hipError_t e = transpose_jobs(jobs, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t img = (int64_t)p.H * p.W * p.C, rstep = (int64_t)p.sh * p.W * p.C, cstep = (int64_t)p.sw * p.C;
  const uint32_t bytes = (uint32_t)((int64_t)p.N * p.H * p.W * p.C * 2);
  if (strided && count <= kMaxConvPhases) {
    // every phase in one launch, longest reduction first
    int order[kMaxConvPhases];
    for (int i = 0; i < count; ++i) order[i] = i;
    for (int i = 1; i < count; ++i)  // insertion sort: stable, by taps descending
      for (int j = i; j > 0 && phases[order[j]].f.R * phases[order[j]].f.S >
                                   phases[order[j - 1]].f.R * phases[order[j - 1]].f.S;
           --j) {
        const int t = order[j];
        order[j] = order[j - 1];
        order[j - 1] = t;
      }
    int64_t Ms[kMaxConvPhases];
    for (int i = 0; i < count; ++i) Ms[i] = (int64_t)p.N * phases[i].f.P * phases[i].f.Q;
    const int shape = conv_shape_multi(Ms, count, p.C);
    const int bm = tile_bm(shape), bn = tile_bn(shape), bk = conv_bk(shape);
    PhasesArgs a;
    a.count = count;
    a.tiles_n = (p.C + bn - 1) / bn;
    a.Nk = p.C;
    a.c = p.c;
    a.y = p.y;
    a.alpha = alpha;
    a.beta = beta;
    a.map_img = img;
    a.map_rstep = rstep;
    a.map_cstep = cstep;
    a.map_bytes = bytes;
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) {
      const ConvLaunch& f = phases[order[i]].f;
      PhaseDesc& d = a.ph[i];
      d.g = ConvGeom{f.x, (uint32_t)((int64_t)f.N * f.H * f.W * f.C * 2), f.H, f.W, f.C, f.S, f.P, f.Q,
                     f.ph, f.pw, 1, 1, f.dh, f.dw, f.R * f.S * f.C, 0, 0};
      if (f.R * f.S > 1 && f.C % bk == 0) {  // channel-block-major k order, as in the single launch
        d.g.prs = f.R * f.S;
        d.g.pcb = f.C / bk;
      }
      d.w = f.w;
      d.map_off0 = phases[order[i]].off0;
      d.M = f.N * f.P * f.Q;
      d.Hp = f.P;
      d.Wp = f.Q;
      d.tile_start = (int)tiles;
      tiles += (int64_t)((d.M + bm - 1) / bm) * a.tiles_n;
    }
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
    a.total_tiles = (int)tiles;
    if (shape == TILE_256x256) return launch_phases<ConvCfg256>(a, dtype, stream);
    if (shape == TILE_256x128) return launch_phases<ConvCfg256x128>(a, dtype, stream);
    return launch_phases<ConvCfg128>(a, dtype, stream);
  }
  // stride 1, or more phases than one launch carries: a launch per phase
  for (int i = 0; i < count; ++i) {
    ConvLaunch f = phases[i].f;
    if (strided) {
      f.map_off0 = phases[i].off0;
      f.map_img = img;
      f.map_rstep = rstep;
      f.map_cstep = cstep;
      f.map_bytes = bytes;
    }
    const hipError_t e =
        launch_conv_fprop(f, conv_shape((int64_t)p.N * f.P * f.Q, p.C), dtype, alpha, beta, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Weight gradient.  dw[k][r][s][c] sums dy[n][p][q][k] x[n][p sh - ph + r dh]
// [q sw - pw + s dw][c] over images and output pixels.  Read with the images
// as channels, this is itself a forward convolution: each input channel c is
// an "image" of H x W pixels with N channels, each k a "filter" of P x Q taps
// over those N channels, and the forward pass's dilation and stride trade
// places:
//   out[c][r][s][k] = sum_{p,q,n} X[c][r dh - ph + p sh][s dw - pw + q sw][n] F[k][p][q][n]
// with X[c][h][w][n] = x[n][h][w][c] and F[k][p][q][n] = dy[n][p][q][k].  The
// page runs wgrad with the activation as the im2col operand and dy tiled;
// here the two transposes put both in the channel-innermost layout the
// forward kernel gathers, with the batch padded to a multiple of 8 by zeros.
// The view's reduction (P*Q*N taps) is long and its output (C*R*S x K) small,
// so it is split over taps into fp32 partials, which a last launch sums in a
// fixed order, scales, adds beta * C, rounds and transposes to KRSC.
// ---------------------------------------------------------------------------
using WgradCfg = ConvCfg256;

bool plan_wgrad(int N, int H, int W, int C, int K, int R, int S, int ph, int pw, int sh, int sw, int dh, int dw,
                int groups, WgradPlan& p) {
  if (groups < 1 || C % groups || K % groups) return false;
  p.groups = groups;
  p.cg = C / groups;
  p.kg = K / groups;
  p.N = N;
  p.H = H;
  p.W = W;
  p.C = C;
  p.K = K;
  p.R = R;
  p.S = S;
  p.ph = ph;
  p.pw = pw;
  p.sh = sh;
  p.sw = sw;
  p.dh = dh;
  p.dw = dw;
  const int64_t ph2 = (int64_t)H + 2 * ph - (int64_t)dh * (R - 1) - 1, pw2 = (int64_t)W + 2 * pw - (int64_t)dw * (S - 1) - 1;
  if (ph2 < 0 || pw2 < 0) return false;
  p.P = (int)(ph2 / sh + 1);
  p.Q = (int)(pw2 / sw + 1);
  p.N8 = (N + 7) / 8 * 8;
  // the view's output size: (H + 2 ph - sh (P - 1) - 1) / dh + 1 >= R
  p.Rp = (int)(((int64_t)H + 2 * ph - (int64_t)sh * (p.P - 1) - 1) / dh + 1);
  p.Sp = (int)(((int64_t)W + 2 * pw - (int64_t)sw * (p.Q - 1) - 1) / dw + 1);
  if (p.Rp < R || p.Sp < S) return false;
  // per group: M = cg * Rp * Sp view pixels, N = kg filters
  const int64_t Mv = (int64_t)p.cg * p.Rp * p.Sp, Kg = (int64_t)p.P * p.Q * p.N8;
  const int64_t tiles =
      groups * ((Mv + WgradCfg::BM - 1) / WgradCfg::BM * ((p.kg + WgradCfg::BN - 1) / WgradCfg::BN));
  const int64_t nkt = (Kg + WgradCfg::BK - 1) / WgradCfg::BK;
  // as many k-ranges as keep every work item in one round of the resident
  // workgroups (a second round for a few items would double the launch), with
  // at least 8 k-tiles per item
  const int64_t slots = (int64_t)device_cu_count() * WgradCfg::WGS_PER_CU;
  int64_t split = slots / tiles;
  if (split > nkt / 8) split = nkt / 8;
  if (split < 1) split = 1;
  p.kt_split = (int)((nkt + split - 1) / split);
  p.split = (int)((nkt + p.kt_split - 1) / p.kt_split);
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  p.x_off = 0;
  p.dy_off = up((size_t)C * H * W * p.N8 * 2);
  p.part_off = p.dy_off + up((size_t)K * p.P * p.Q * p.N8 * 2);
  p.bytes = p.part_off + up((size_t)groups * p.split * Mv * p.kg * 4);
  return true;
}

// dw[k][r][s][c] = RN(alpha * sum over splits of part[.][(c Rp + r) Sp + s][k]
// + beta * c_in[k][r][s][c]): one 32 x 64 (c, k) block of one tap per
// workgroup, read along k (eight independent sums per thread, so the loads
// of a split are in flight together), written along c.
// With groups, C is the channels per group and output channel k belongs to
// group k / kg, whose partials start at part + (k / kg) * split * plane.
template <int DT>
__global__ __launch_bounds__(256) void k_wgrad_finish(const float* __restrict__ part, int split, int C, int K, int kg,
                                                      int R, int S, int Rp, int Sp, const uint16_t* __restrict__ cin,
                                                      float alpha, float beta, uint16_t* __restrict__ dw) {
  __shared__ float t[32][65];
  const int rs = blockIdx.z, r = rs / S, s = rs % S;
  const int c0 = blockIdx.x * 32, k0 = blockIdx.y * 64;
  const int64_t plane = (int64_t)C * Rp * Sp * kg;
  const int kk = threadIdx.x % 64, cb = threadIdx.x / 64;  // this thread: k0 + kk, rows c0 + cb + 4 j
  const int k = k0 + kk, grp = k / kg, kl = k - grp * kg;
  const float* gpart = part + grp * split * plane;
  float v[8];
  const float* src[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = c0 + cb + 4 * j;
    v[j] = 0.0f;
    src[j] = (c < C && k < K) ? gpart + ((int64_t)(c * Rp + r) * Sp + s) * kg + kl : nullptr;
  }
  // four splits per round trip (32 loads in flight per thread), in order
  int sp = 0;
  for (; sp + 4 <= split; sp += 4) {
    float u[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) u[q][j] = src[j] ? src[j][(sp + q) * plane] : 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] += u[q][j];
  }
  for (; sp < split; ++sp) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (src[j]) v[j] += src[j][sp * plane];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) t[cb + 4 * j][kk] = v[j];
  __syncthreads();
  for (int i = threadIdx.x; i < 32 * 64; i += 256) {
    const int ko = i / 32, cc = i % 32, c = c0 + cc, kx = k0 + ko;
    if (c < C && kx < K) {
      const int64_t o = ((int64_t)(kx * R + r) * S + s) * C + c;
      float x = alpha * t[cc][ko];
      if (cin) x += beta * from_bits<DT>(cin[o]);
      dw[o] = (uint16_t)to_bits<DT>(x);
    }
  }
}

hipError_t launch_conv_wgrad(const WgradPlan& p, const uint16_t* x, const uint16_t* dy, const uint16_t* c_in,
                             uint16_t* dwt, char* workspace, int dtype, float alpha, float beta, hipStream_t stream) {
  uint16_t* xt = (uint16_t*)(workspace + p.x_off);
  uint16_t* gt = (uint16_t*)(workspace + p.dy_off);
  float* part = (float*)(workspace + p.part_off);
  TransposeJobs jobs;  // x and dy to the channel-innermost layout, in one launch
  jobs.count = 2;
  jobs.job[0] = transpose_job(x, xt, p.N, p.H * p.W, p.C, p.N8);
  jobs.job[1] = transpose_job(dy, gt, p.N, p.P * p.Q, p.K, p.N8);
  hipError_t e = transpose_jobs(jobs, stream);
  if (e != hipSuccess) return e;
  ConvLaunch f;  // the forward view, one problem per channel group
  f.x = xt;
  f.w = gt;
  f.c = nullptr;
  f.y = nullptr;
  f.N = p.cg;
  f.H = p.H;
  f.W = p.W;
  f.C = p.N8;
  f.K = p.kg;
  f.R = p.P;
  f.S = p.Q;
  f.P = p.Rp;
  f.Q = p.Sp;
  f.ph = p.ph;
  f.pw = p.pw;
  f.sh = p.dh;
  f.sw = p.dw;
  f.dh = p.sh;
  f.dw = p.sw;
  f.split = p.split;
  f.kt_split = p.kt_split;
  f.partial = part;
  f.groups = p.groups;
  f.x_group = (int64_t)p.cg * p.H * p.W * p.N8;
  f.w_group = (int64_t)p.kg * p.P * p.Q * p.N8;
  f.part_group = (int64_t)p.split * p.cg * p.Rp * p.Sp * p.kg;
  e = launch_conv_fprop(f, TILE_256x256, dtype, 1.0f, 0.0f, stream);
  if (e != hipSuccess) return e;
  const dim3 grid((p.cg + 31) / 32, (p.K + 63) / 64, p.R * p.S);
  if (dtype == DT_F16)
    hipLaunchKernelGGL(k_wgrad_finish<DT_F16>, grid, dim3(256), 0, stream, part, p.split, p.cg, p.K, p.kg, p.R, p.S,
                       p.Rp, p.Sp, c_in, alpha, beta, dwt);
  else
    hipLaunchKernelGGL(k_wgrad_finish<DT_BF16>, grid, dim3(256), 0, stream, part, p.split, p.cg, p.K, p.kg, p.R, p.S,
                       p.Rp, p.Sp, c_in, alpha, beta, dwt);
  return hipGetLastError();
}

}  // namespace gmi
