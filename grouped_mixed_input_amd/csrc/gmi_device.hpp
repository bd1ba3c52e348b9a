// gmi_device.hpp -- device building blocks shared by every kernel of the
// library: element types, gfx950 MFMA wrappers, buffer and direct-to-LDS
// memory access, the LDS tile layout, operand loaders (dense, implicit-conv,
// prepacked uint4), the multi-stage mainloop, the alpha/beta epilogue and the
// persistent tile walk.
//
// The mainloop follows the structure of the persistent grouped GEMM kernel on
// the page sm90_gemm_array_tma_warpspecialized_cooperative.hpp (operator():
// a work-tile loop, a k-tile loop that accumulates in fp32 starting from
// zero, an epilogue store per tile) rebuilt for CDNA4: every wave both loads
// and computes; operand k-tiles stream from memory straight into a ring of
// LDS stages (buffer_load ... lds), several k-tiles ahead of the multiply;
// v_mfma_f32_32x32x16_{f16,bf16} consumes conflict-free 128-bit LDS reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gmi {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Element types of A and B.  fp16 and bf16 results are stored in the input
// type; OCP fp8 E4M3 inputs give a bf16 result.
enum { DT_F16 = 0, DT_BF16 = 1, DT_F8 = 2 };
template <int DT>
constexpr int out_dt() {
  return DT == DT_F8 ? DT_BF16 : DT;
}

// ---------------------------------------------------------------------------
// MFMA.  Operand fragments: lane l holds row (l % 32) and the 8 consecutive k
// of k-group (l / 32) for the 32x32x16 shape; row (l % 16), k-group (l / 16)
// for 16x16x32.  Result of 32x32: lane l, element j holds
// D[8 (j / 4) + 4 (l / 32) + j % 4][l % 32]; of 16x16: D[4 (l / 16) + j][l % 16].
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands OCP fp8 E4M3 (format
// 0) and unit E8M0 block scales (127 = 2^0): a plain fp8 product, fp32
// accumulation.  Lane l holds 32 consecutive-slot bytes of row l % 32, k-half
// l / 32 of the 64-k step.
__device__ __forceinline__ f32x16 mfma32_f8(u32x8 a, u32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b), c,
                                                         0, 0, 0, 127, 0, 127);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// fp32 -> 16-bit storage pattern, round to nearest even (hardware converts).
template <int DT>
__device__ __forceinline__ uint32_t to_bits(float f) {
  if constexpr (DT == DT_F16)
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  else
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// two fp32 -> one 32-bit word of 16-bit patterns (a low, b high), round to
// nearest even; one v_cvt_pk_{f16,bf16}_f32
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  if constexpr (DT == DT_F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), h2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), b2));
}

template <int DT>
__device__ __forceinline__ float from_bits(uint32_t b) {
  if constexpr (DT == DT_F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  else
    return __builtin_bit_cast(float, b << 16);
}

// ---------------------------------------------------------------------------
// Buffer access.  A buffer resource (4 SGPRs: base, size in bytes) is
// wave-uniform; each lane adds a 32-bit byte offset.  A load at or past the
// size returns zeros and a store there is dropped, which zero-fills the rows
// of a tile that lie past the end of an operand and any lane pointed at OOB.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OOB = 0x80000000u;  // offset past every resource this library builds
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // base and size are wave-uniform by construction; readfirstlane makes that
  // visible to the compiler so the resource lives in SGPRs
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

typedef __attribute__((address_space(1))) u32x2 gu32x2;  // global-memory pointer target
typedef __attribute__((address_space(3))) void lds_void;
// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// dst + 16 l (dst wave-uniform).  Completion is counted by vmcnt.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t off, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)off, 0, 0, 0);
}
// as dma16, with a wave-uniform byte offset soff added to the lane offset
__device__ __forceinline__ void dma16s(rsrc_t r, uint32_t off, uint32_t soff, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)off, (int)soff, 0, 0);
}
// as dma16 with 4 bytes per lane (lane l's dword lands at dst + 4 l)
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t off, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, (int)off, 0, 0, 0);
}
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}
// as above, with a wave-uniform byte offset soff (an SGPR) added to the lane
// offset; a lane at OOB stays past the resource for any soff below 2^31
__device__ __forceinline__ u32x2 buf_load8s(rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, 0));
}
__device__ __forceinline__ uint32_t buf_load2s(rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, (int)soff, 0);
}
__device__ __forceinline__ uint32_t buf_load1s(rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, (int)soff, 0);
}
// Output stores are streaming (nt): each result is written once and not read
// back by the kernel, so the L2 sends it on toward memory instead of holding it
// dirty until the end-of-kernel writeback, which would serialize the whole
// output write after the last tile.
constexpr int CPOL_NT = 2;
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, CPOL_NT);
}
// a plain (write-back) 16-byte store: for data written in pieces of a line
// by several instructions and read again soon, which the L2 then merges
// into whole lines instead of sending each piece on
__device__ __forceinline__ void buf_store16_wb(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, CPOL_NT);
}
__device__ __forceinline__ void buf_store2(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, (int)off, 0, CPOL_NT);
}

// s_waitcnt: gfx9 encoding, vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// wait_vm_le<n> for an n known only after unrolling (n <= N): folds to one
// s_waitcnt when n is a constant
template <int N>
__device__ __forceinline__ void wait_vm_le_n(int n) {
  if constexpr (N == 0) {
    wait_vm_le<0>();
  } else {
    if (n >= N)
      wait_vm_le<N>();
    else
      wait_vm_le_n<N - 1>(n);
  }
}
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// Zero the 16-bit elements e >= n (0 <= n < 8) of an 8-element chunk.
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int n) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int e = 2 * w;
    const uint32_t keep = (e + 1 < n) ? 0xffffffffu : (e < n ? 0x0000ffffu : 0u);
    v[w] &= keep;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Tile configuration: BM x BN output tile, 4 waves arranged WAVES_M x
// WAVES_N, BK k per stage, STAGES LDS stages in a ring.
//
// LDS operand tile: rows of BK values (ROWB = 2 BK bytes, CPR 16-byte chunks).
// gfx950's LDS serves 256 bytes (64 four-byte banks) per cycle; a 128-bit
// read is conflict-free when each group of 16 lanes covers all 64 banks.  A
// fragment read has 16 lanes on 16 consecutive rows and one chunk c; a bank
// line holds RPL = 256 / ROWB consecutive rows, so chunk c of row r goes to
// slot c ^ ((r / RPL) % CPR): the rows sharing a bank position within their
// lines get distinct slots.
// ---------------------------------------------------------------------------
// SLOTS_ = 0: a ring of STAGES stages, each holding one k-tile of A and of B.
// SLOTS_ > 0 (BM == BN): a ring of SLOTS_ single-operand slots, A of k-tile
// kt in slot 2 kt and B in slot 2 kt + 1 (mod SLOTS_); STAGES is then unused.
// EB_: bytes per element of A and B (2: fp16 / bf16, 1: fp8); BK counts
// elements, so a k-tile row is BK * EB bytes.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int STAGES_, int SLOTS_ = 0, int EB_ = 2>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, SLOTS = SLOTS_, EB = EB_;
  static constexpr int RING_BYTES =
      SLOTS_ > 0 ? SLOTS_ * BM_ * BK_ * EB_ : STAGES_ * (BM_ + BN_) * BK_ * EB_;
  // workgroups one CU holds: LDS-bound (160 KB); the kernels' launch bounds
  // hold the registers to match (waves per SIMD = workgroups per CU x NW / 4)
  static constexpr int WGS_PER_CU = (160 * 1024) / RING_BYTES >= 2 ? 2 : 1;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N, THREADS = 64 * NW;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;            // 32x32 blocks per wave
  static constexpr int ROWB = BK * EB, CPR = ROWB / 16, RPL = 256 / ROWB;
  static constexpr int CE = 16 / EB;  // elements per 16-byte chunk
  // matrix-instruction step: 16 k (one chunk per lane) for 16-bit inputs,
  // 64 k (two chunks per lane) for fp8
  static constexpr int KSTEP = EB == 2 ? 16 : 64, FC = EB == 2 ? 1 : 2, KK = BK / KSTEP;
  // chunk t of the fragment of step kk for lanes l / 32 == h
  __device__ static __forceinline__ int frag_chunk(int kk, int h, int t) {
    return EB == 2 ? 2 * kk + h : 4 * kk + 2 * h + t;
  }
  static constexpr int RPI = 1024 / ROWB;  // rows moved by one 1 KB wave copy
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int SLOT_BYTES = A_BYTES;
  static constexpr int LDS_BYTES = RING_BYTES;
  static_assert(SLOTS == 0 || (BM == BN && SLOTS >= 5), "split ring: square tile, at least five slots");
  static_assert(EB == 2 || EB == 1, "16-bit or 8-bit elements");
  static_assert(ROWB == 64 || ROWB == 128, "k-tile rows of 64 or 128 bytes");
  static_assert(KK >= 2 && KK % 2 == 0, "an even number of matrix steps per k-tile");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(STAGES >= 2 && LDS_BYTES <= 160 * 1024, "LDS budget");
  __device__ static __forceinline__ int swz(int row) { return (row / RPL) % CPR; }
  __device__ static __forceinline__ int off(int row, int chunk) { return row * ROWB + ((chunk ^ swz(row)) << 4); }
  // direct-to-LDS copies: instruction i of wave w fills rows RPI (NW i + w) + l / CPR;
  // lane l writes slot l % CPR of its row, i.e. k-chunk (l % CPR) ^ swz(row)
  __device__ static __forceinline__ int dma_row(int i, int lane) { return RPI * (NW * i + wave_id()) + lane / CPR; }
  __device__ static __forceinline__ int dma_chunk(int lane) { return (lane % CPR) ^ swz(dma_row(0, lane)); }
  // wave-uniform (scalar) LDS destination of copy i
  __device__ static __forceinline__ char* dma_dst(char* tile, int i) { return tile + (NW * i + wave_id()) * 1024; }
};

// One output tile of one GEMM problem, as the persistent walk hands it out.
struct Tile {
  int M, N, K;  // problem shape
  int m0, n0;   // tile origin
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  const uint16_t* C;
  int64_t ldc;
  uint16_t* D;
  int64_t ldd;
  // fused epilogue: per-column bias (output type, NULL: none) added after
  // alpha * acc + beta * C, then the activation (ACT_NONE / ACT_RELU)
  const uint16_t* bias = nullptr;
  int act = 0;
};
constexpr int ACT_NONE = 0, ACT_RELU = 1;

// Output rows that are the pixels of a strided grid inside a larger
// channel-innermost tensor (one phase of the strided data gradient): GEMM row
// m = (n Hp + i) Wp + j is stored, and C read, at element
// off0 + n img + i rstep + j cstep (the row's N elements contiguous from
// there), inside a tensor of `bytes` bytes that starts at the tile's D (C).
struct RowMap {
  int Hp, Wp;
  int64_t off0, img, rstep, cstep;
  uint32_t bytes;
  __device__ __forceinline__ uint32_t offset(int m) const {
    const int n = m / (Hp * Wp), r = m - n * Hp * Wp, i = r / Wp, j = r - i * Wp;
    return (uint32_t)(off0 + n * img + i * rstep + j * cstep);
  }
};

// ---------------------------------------------------------------------------
// Dense K-contiguous operand (direct to LDS): ROWS rows x BK k per k-tile
// through a buffer resource spanning exactly the tile's rows inside the
// problem, so rows past the end land as zeros.  Chunks at or past K are
// pointed out of range; a chunk that straddles K (K % 8 != 0, KTAIL) is
// masked in LDS after it lands.
// ---------------------------------------------------------------------------
//
// A tile of fewer 1 KB copies than waves (the 32-row grouped class on eight
// waves) is copied by the first COPIES waves, and every further wave repeats
// the copy of wave w % COPIES -- the same bytes to the same LDS addresses --
// so that each wave issues one copy per k-tile and the waits, which count
// copies per wave, stay uniform.
template <class Cfg, int ROWS, bool KTAIL = false>
struct DenseLoader {
  static constexpr bool kDMA = true;
  static constexpr bool kFIX = KTAIL;  // fix_tail may write LDS
  static constexpr int COPIES = ROWS * Cfg::ROWB / 1024;  // 1 KB copies per k-tile
  static constexpr int P = COPIES >= Cfg::NW ? COPIES / Cfg::NW : 1;  // per wave
  static_assert(COPIES >= 1 && (COPIES % Cfg::NW == 0 || Cfg::NW % COPIES == 0) && ROWS % Cfg::RPI == 0,
                "rows must fill whole copy passes");
  // the wave whose copies this one issues, and its rows / LDS destinations
  __device__ static __forceinline__ int copy_wave() {
    return COPIES >= Cfg::NW ? wave_id() : wave_id() % COPIES;
  }
  __device__ static __forceinline__ int row_of(int i, int lane) {
    return Cfg::RPI * (Cfg::NW * i + copy_wave()) + lane / Cfg::CPR;
  }
  __device__ static __forceinline__ int chunk_of(int lane) { return (lane % Cfg::CPR) ^ Cfg::swz(row_of(0, lane)); }
  __device__ static __forceinline__ char* dst_of(char* tile, int i) {
    return tile + (Cfg::NW * i + copy_wave()) * 1024;
  }
  rsrc_t rs;
  uint32_t voff[P];  // lane offset of copy i within k-tile 0, bytes
  int K, nk;
  // per-k-tile state: the scalar k-tile offset (clamped to the last k-tile, so
  // copies past the end re-read valid data), and, for a K that is not a
  // multiple of BK, the lanes whose chunk starts past K
  struct Prep {
    uint32_t soff;
    uint32_t vo[P];  // lane offset of copy i, or OOB for a chunk past K
  };

  static_assert(!KTAIL || Cfg::EB == 2, "K tails are masked for 16-bit elements only");
  // base: the operand's first element; ld and K in elements
  __device__ __forceinline__ void init(const void* base, int64_t ld, int row0, int rows, int K_) {
    int left = rows - row0;
    if (left > ROWS) left = ROWS;
    if (left < 0) left = 0;
    const uint32_t ldb = (uint32_t)ld * Cfg::EB;  // row pitch, bytes
    rs = make_rsrc((const char*)base + (int64_t)row0 * ld * Cfg::EB, (uint32_t)left * ldb);
    const int lane = threadIdx.x & 63;
    const uint32_t v0 = (uint32_t)row_of(0, lane) * ldb + (uint32_t)chunk_of(lane) * 16u;
    const uint32_t step = (uint32_t)(Cfg::NW * Cfg::RPI) * ldb;
#pragma unroll
    for (int i = 0; i < P; ++i) voff[i] = v0 + i * step;
    K = K_;
    nk = (K_ + Cfg::BK - 1) / Cfg::BK;
  }

  __device__ __forceinline__ Prep prep(int kt) const {
    const int ke = kt < nk ? kt : nk - 1;
    Prep p;
    p.soff = (uint32_t)ke * Cfg::ROWB;
    const bool in = (ke * Cfg::BK + chunk_of(threadIdx.x & 63) * Cfg::CE) < K;
#pragma unroll
    for (int i = 0; i < P; ++i) p.vo[i] = in ? voff[i] : OOB;
    return p;
  }
  // copy i of the prepared k-tile: rows past the problem land as zeros (the
  // lane offset is past the resource), and so do chunks at or past K
  __device__ __forceinline__ void issue_one(int i, const Prep& p, char* tile) const {
    dma16s(rs, p.vo[i], p.soff, dst_of(tile, i));
  }
  __device__ __forceinline__ void issue(int kt, char* tile) const {
    const Prep p = prep(kt);
#pragma unroll
    for (int i = 0; i < P; ++i) issue_one(i, p, tile);
  }

  // after k-tile kt has landed: zero the elements >= K of a straddling chunk
  __device__ __forceinline__ void fix_tail(int kt, char* tile) const {
    if constexpr (!KTAIL) return;
    if ((K & 7) == 0 || kt >= nk || (kt + 1) * Cfg::BK <= K) return;
    const int lane = threadIdx.x & 63;
    const int n = K - (kt * Cfg::BK + chunk_of(lane) * 8);
    if (n <= 0 || n >= 8) return;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      u32x4* p = (u32x4*)(dst_of(tile, i) + lane * 16);
      *p = mask_tail(*p, n);
    }
  }
};

// ---------------------------------------------------------------------------
// Implicit-GEMM convolution A operand (fprop, direct to LDS).  GEMM row m is
// output pixel (n, p, q), m = (n P + p) Q + q; GEMM column k is filter tap
// (r, s, c), k = (r S + s) C + c.  Element (m, k) is
// x[n][p sh - ph + r dh][q sw - pw + s dw][c], or 0 outside the image -- the
// im2col view of the activation that the page
// sm100_implicit_gemm_umma_warpspecialized.hpp builds from the padding,
// traversal stride and dilation (get_tma_load_a_instance), formed here by
// address arithmetic instead.  With C % 8 == 0 a 16-byte chunk never
// straddles two taps, so each chunk is one aligned 128-bit copy or zero.
// ---------------------------------------------------------------------------
struct ConvGeom {
  const uint16_t* x;
  uint32_t x_bytes;  // N * H * W * C * 2 (< 2^31)
  int H, W, C, S;
  int P, Q;
  int ph, pw, sh, sw, dh, dw;
  int Kg;  // R * S * C
  // k-tile order.  prs = 0: the GEMM's own order, taps (r, s) outer and
  // channels inner.  prs = R * S (only when C is a whole number pcb of
  // k-tiles): loop step t takes channel block t / prs of tap t % prs, so the
  // R * S taps of one channel block run back to back and re-read input rows
  // that the previous taps just brought into L2.  The k-tiles partition the
  // same sum either way; only the fp32 accumulation order differs.
  int prs, pcb;
};

// GEMM k-tile of loop step lt under the order above (steps past the last
// k-tile map to themselves)
__device__ __forceinline__ int conv_ktile(int lt, int prs, int pcb) {
  return (prs && lt < prs * pcb) ? (lt % prs) * pcb + lt / prs : lt;
}

template <class Cfg, int ROWS>
struct ConvLoader {
  static constexpr bool kDMA = true;
  static constexpr bool kFIX = false;
  static_assert(Cfg::EB == 2, "16-bit activations");
  static constexpr int P = ROWS * Cfg::ROWB / (1024 * Cfg::NW);
  static_assert(P >= 1 && ROWS % (Cfg::NW * Cfg::RPI) == 0, "rows must fill whole copy passes");
  rsrc_t rs;
  int H, W, C, S, dh, dw, Kg, kt0, prs, pcb;
  int pix[P];        // first pixel of the row's image: n * H * W
  int h0[P], w0[P];  // (virtual) input coordinates of tap (0, 0); far negative for rows past M

  // rows m0 .., k-tiles from kt_first on
  __device__ __forceinline__ void init(const ConvGeom& g, int m0, int M, int kt_first = 0) {
    rs = make_rsrc(g.x, g.x_bytes);
    kt0 = kt_first;
    H = g.H;
    W = g.W;
    C = g.C;
    S = g.S;
    dh = g.dh;
    dw = g.dw;
    Kg = g.Kg;
    prs = g.prs;
    pcb = g.pcb;
    const int PQ = g.P * g.Q;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int m = m0 + Cfg::dma_row(i, lane);
      if (m < M) {
        const int n = m / PQ, rem = m - n * PQ;
        const int p = rem / g.Q, q = rem - p * g.Q;
        pix[i] = n * H * W;
        h0[i] = p * g.sh - g.ph;
        w0[i] = q * g.sw - g.pw;
      } else {
        pix[i] = 0;
        h0[i] = -(1 << 29);
        w0[i] = -(1 << 29);
      }
    }
  }

  // per-k-tile state: this lane's tap (r, s) offsets and channel; copies past
  // the last k-tile land as zeros
  struct Prep {
    int dr, ds, c;
    bool kin;
  };
  __device__ __forceinline__ Prep prep(int kt) const {
    const int kc = conv_ktile(kt + kt0, prs, pcb) * Cfg::BK + Cfg::dma_chunk(threadIdx.x & 63) * 8;
    const int rsx = kc / C, c = kc - rsx * C;
    const int r = rsx / S, s = rsx - r * S;
    return Prep{r * dh, s * dw, c, kc < Kg};
  }
  __device__ __forceinline__ void issue_one(int i, const Prep& p, char* tile) const {
    const int ih = h0[i] + p.dr, iw = w0[i] + p.ds;
    const bool in = p.kin && (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W;
    dma16(rs, in ? (uint32_t)((pix[i] + ih * W + iw) * C + p.c) * 2u : OOB,
          Cfg::dma_dst(tile, i));
  }
  __device__ __forceinline__ void issue(int kt, char* tile) const {
    const Prep p = prep(kt);
#pragma unroll
    for (int i = 0; i < P; ++i) issue_one(i, p, tile);
  }
  __device__ __forceinline__ void fix_tail(int, char*) const {}  // C % 8 == 0: chunks never straddle K
};

// The KRSC filter as the column-major B operand (leading dimension R * S * C),
// its k-tiles taken in the gather's order.
template <class Cfg, int ROWS>
struct FilterLoader : DenseLoader<Cfg, ROWS> {
  using Base = DenseLoader<Cfg, ROWS>;
  using typename Base::Prep;
  int kt0, prs, pcb;
  __device__ __forceinline__ void init(const uint16_t* w, const ConvGeom& g, int row0, int rows, int kt_first) {
    Base::init(w, g.Kg, row0, rows, g.Kg);
    kt0 = kt_first;
    prs = g.prs;
    pcb = g.pcb;
  }
  __device__ __forceinline__ Prep prep(int kt) const {
    return Base::prep(conv_ktile(kt + kt0, prs, pcb));
  }
  __device__ __forceinline__ void issue(int kt, char* tile) const {
    const Prep p = prep(kt);
#pragma unroll
    for (int i = 0; i < Base::P; ++i) Base::issue_one(i, p, tile);
  }
};

// ---------------------------------------------------------------------------
// uint4 -> fp16 dequantisation of one prepacked 32-bit word (8 consecutive k
// of one weight row; even elements in nibbles 0-3, odd ones in nibbles 4-7).
// 0x6400 is 1024.0 in binary16 and its ulp is 1, so OR-ing a nibble q into
// its low bits gives 1024 + q exactly; subtracting 1024 + z gives q - z
// exactly, and one fp16 multiply by the group scale rounds (q - z) * s to
// nearest even.  This is the convert -> scale -> zero -> convert chain of
// transform_A_kblock (page machete_mainloop.cuh) with the zero point read as
// an unsigned offset subtracted before the scale.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x2 zero_pair(uint32_t z) {
  return __builtin_bit_cast(f16x2, (0x6400u | z) * 0x00010001u);
}
__device__ __forceinline__ f16x2 scale_pair(uint32_t s_bits) { return __builtin_bit_cast(f16x2, s_bits * 0x00010001u); }

// The integer part only: q - z for the 8 nibbles of w, exact in fp16, for
// kernels that apply the group scale to the fp32 partial sums instead.  The
// OR constant is passed in a VGPR so that mask-and-OR is one v_and_or_b32.
__device__ __forceinline__ u32x4 unpack8_minus_zero(uint32_t w, f16x2 zz, uint32_t magic) {
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_bit_cast(f16x2, ((w >> (4 * i)) & 0x000F000Fu) | magic);
    out[i] = __builtin_bit_cast(uint32_t, h - zz);
  }
  return out;
}

// 128 + q for the 8 nibbles of w as exact bfloat16 values, in the order of
// unpack8_minus_zero: with magic = 0x43004300 each half is 128 (exponent 7)
// whose 7-bit mantissa holds q in its low 4 bits
__device__ __forceinline__ u32x4 unpack8_biased_bf16(uint32_t w, uint32_t magic) {
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = ((w >> (4 * i)) & 0x000F000Fu) | magic;
  return out;
}

// Pairs 1 and 3 (nibble slots 1, 5 and 3, 7) are used in place, four bits
// up: OR-ed into 0x6400 they give 1024 + 16 q exactly, and 1/16 of that
// minus 64 + z is again q - z exactly (64 + z also has ulp 1/16 at most), so
// only one shift is needed per word and every pair costs one mask-and-OR,
// one add or multiply-add, and the scale multiply.  The results are those of
// the shifted form bit for bit.  `magic` is 0x64006400 passed in a VGPR, so
// that mask-and-OR is one v_and_or_b32.
__device__ __forceinline__ u32x4 dequant8(uint32_t w, uint32_t z, f16x2 ss, uint32_t magic = 0x64006400u) {
  const f16x2 zl = zero_pair(z);                                                    // 1024 + z
  const f16x2 zh = __builtin_bit_cast(f16x2, (0x5400u | (z << 4)) * 0x00010001u);  // 64 + z
  const f16x2 sixteenth = __builtin_bit_cast(f16x2, 0x2C002C00u);                   // 1/16
  const uint32_t w8 = w >> 8;
  u32x4 out;
  out[0] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, (w & 0x000F000Fu) | magic) - zl) * ss);
  out[1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, (w & 0x00F000F0u) | magic) * sixteenth - zh) * ss);
  out[2] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, (w8 & 0x000F000Fu) | magic) - zl) * ss);
  out[3] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, (w8 & 0x00F000F0u) | magic) * sixteenth - zh) * ss);
  return out;
}

// bfloat16 counterparts.  bfloat16 has too few mantissa bits for the OR
// construction to stay cheap, so the nibbles go through fp32: spread into
// bytes (even nibbles, odd nibbles), each byte converted by one
// v_cvt_f32_ubyte.  The bytes of w & 0x0F0F0F0F are elements 0, 4, 1, 5 of
// the word, those of (w >> 4) & 0x0F0F0F0F elements 2, 6, 3, 7.
__device__ __forceinline__ float ubyte_f32(uint32_t v, int i) { return (float)((v >> (8 * i)) & 0xFFu); }

// RN_bf16((q - z) s) for the 8 nibbles of w: q s - z s is formed exactly by
// one fma (a 4-bit integer times an 8-bit significand fits fp32; nzs = -z s
// is exact too), then rounded to nearest even by the conversion.
__device__ __forceinline__ u32x4 dequant8_bf16(uint32_t w, float s, float nzs) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  auto d = [&](uint32_t v, int i) { return __builtin_fmaf(ubyte_f32(v, i), s, nzs); };
  u32x4 out;
  out[0] = pack2<DT_BF16>(d(lo, 0), d(lo, 2));
  out[1] = pack2<DT_BF16>(d(hi, 0), d(hi, 2));
  out[2] = pack2<DT_BF16>(d(lo, 1), d(lo, 3));
  out[3] = pack2<DT_BF16>(d(hi, 1), d(hi, 3));
  return out;
}

// q - z for the 8 nibbles of w as exact bfloat16 values (|q - z| <= 15 has
// at most 4 significant bits), in the order of dequant8_bf16: the integer
// part only, for kernels that apply the group scale to fp32 partial sums.
__device__ __forceinline__ u32x4 exact8_bf16(uint32_t w, float zf) {
  uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  // hide the masks from the compiler: knowing each byte's high bits are
  // zero, it extracts every nibble with a bit-field extract before a byte-0
  // convert; opaque, each byte converts with one v_cvt_f32_ubyteN
  asm("" : "+v"(lo), "+v"(hi));
  auto d = [&](uint32_t v, int i) { return ubyte_f32(v, i) - zf; };
  u32x4 out;
  out[0] = pack2<DT_BF16>(d(lo, 0), d(lo, 2));
  out[1] = pack2<DT_BF16>(d(hi, 0), d(hi, 2));
  out[2] = pack2<DT_BF16>(d(lo, 1), d(lo, 3));
  out[3] = pack2<DT_BF16>(d(hi, 1), d(hi, 3));
  return out;
}

// dequantised 16-bit weights of one word in the activation type: s_bits is
// the scale's storage pattern, z the zero point (both after the mode fix-ups)
template <int DT>
__device__ __forceinline__ u32x4 dequant8_dt(uint32_t w, uint32_t s_bits, uint32_t z) {
  if constexpr (DT == DT_F16) {
    return dequant8(w, z, scale_pair(s_bits));
  } else {
    const float s = from_bits<DT_BF16>(s_bits);
    return dequant8_bf16(w, s, -(float)z * s);
  }
}

// Prepacked weight geometry: 16 rows x 128 k per 1024-byte block, block
// (n / 16, k / 128) at ((n / 16) * (K / 128) + k / 128) * 1024; lane L of a
// block owns bytes [16 L, 16 L + 16): row L % 16, word j covering
// k = 32 j + 8 (L / 16) + {0..7}.
struct W4Geom {
  const uint8_t* w;        // prepacked weight
  const uint16_t* scales;  // [K / g][N], the activation type
  const uint8_t* zeros;    // [K / g][N / 2] 4-bit
  int N, K, group;
  uint32_t s_bytes, z_bytes, sor, wxor, zxor;  // conversion mode (see W4Launch)
};

// ---------------------------------------------------------------------------
// Prepacked uint4 weight as the B operand (rows n, BK = 64 k per k-tile): a
// k-tile takes words j = 2 (kt % 2) + {0, 1} of every lane entry of the
// 16-row blocks it covers -- 8 bytes per entry -- plus each entry's scale and
// zero, into registers.  The dequantisation runs when the registers are
// written to LDS, after the multiplies of the current stage have been issued.
//
// fp16: the LDS tile holds RN16((q - z) s), the page's conversion in the
// activation type (its 11-bit significand keeps that rounding far inside the
// parity bar).  bf16 (EXACT): an 8-bit significand would round each weight by
// up to 2^-9 |w|, which over K = 8192 terms reaches the bar, so the tile holds
// the exact integers q - z instead and the mainloop multiplies into fp32
// partial sums that each 128-k-multiple scale group folds into the
// accumulators with its own scale: sum_k x (q - z) s = sum over groups of
// s * sum_k x (q - z), with every product exact and only fp32 sums rounding.
// The scale of each accumulator column is then loaded once per group
// (fold_scales) instead of once per weight entry.
// ---------------------------------------------------------------------------
template <class Cfg, int ROWS, int DT = DT_F16>
struct W4Loader {
  static constexpr bool kDMA = false;
  static constexpr bool kFIX = false;
  static constexpr bool EXACT = DT == DT_BF16;
  static constexpr int ENTRIES = ROWS / 16 * 64;
  static constexpr int P = ENTRIES / Cfg::THREADS;
  // loads one k-tile issues per lane entry: weight bytes, zero point and, for
  // the rounded form, the scale
  static constexpr int LOADS = P * (EXACT ? 2 : 3);
  static_assert(Cfg::BK == 64, "the uint4 loader moves half a 128-k block per k-tile");
  static_assert(ENTRIES % Cfg::THREADS == 0, "rows must cover whole lane-entry passes");
  struct Regs {
    u32x2 w[P];
    uint32_t s[P], z[P];
  };
  rsrc_t rw, rsc, rz;
  uint32_t kblocks, N, group, block0, kt0, sor, wxor, zxor;

  // rows n0 .., k-tiles from kt_first on (kt_first even: whole 128-k blocks)
  __device__ __forceinline__ void init(const W4Geom& g, int n0, int kt_first = 0) {
    rw = make_rsrc(g.w, (uint32_t)((int64_t)g.N * g.K / 2));
    rsc = make_rsrc(g.scales, g.s_bytes);
    rz = make_rsrc(g.zeros, g.z_bytes);
    kblocks = g.K / 128;
    N = g.N;
    group = g.group;
    block0 = n0 / 16;
    kt0 = kt_first;
    sor = g.sor;
    wxor = g.wxor;
    zxor = g.zxor;
  }

  __device__ __forceinline__ void load(int kt_local, Regs& rg) const {
    const uint32_t kt = kt_local + kt0;
    const uint32_t grp = (kt * Cfg::BK) / group;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = threadIdx.x + i * Cfg::THREADS;
      const uint32_t nb = e / 64, L = e % 64;
      const uint32_t n = (block0 + nb) * 16 + (L % 16);
      const bool ok = n < N;
      rg.w[i] = buf_load8(rw, ok ? ((block0 + nb) * kblocks + kt / 2) * 1024u + L * 16u + (kt & 1) * 8u : OOB);
      if constexpr (!EXACT) rg.s[i] = buf_load2(rsc, ok ? (grp * N + n) * 2u : OOB);
      rg.z[i] = buf_load1(rz, ok ? grp * (N / 2) + n / 2 : OOB);
    }
  }

  __device__ __forceinline__ void store(char* lds, const Regs& rg) const {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = threadIdx.x + i * Cfg::THREADS;
      const int nb = e / 64, L = e % 64;
      const int row = nb * 16 + (L % 16), h = L / 16;
      const uint32_t n = (block0 + nb) * 16 + (L % 16);
      const uint32_t z = ((rg.z[i] >> ((n & 1) * 4)) & 15u) ^ zxor;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        u32x4 v;
        if constexpr (EXACT)
          v = exact8_bf16(rg.w[i][jj] ^ wxor, (float)z);
        else
          v = dequant8_dt<DT>(rg.w[i][jj] ^ wxor, (rg.s[i] & 0xffffu) | sor, z);
        *(u32x4*)(lds + Cfg::off(row, 4 * jj + h)) = v;
      }
    }
  }

  // EXACT: the group scales of this lane's accumulator columns for the group
  // holding k-tile kt_local, as bf16 pairs: block j of the wave tile, register
  // group q covers columns n0 + wn + 32 j + 8 q + 4 (lane / 32) + {0..3}
  // (the MFMA result layout with the weight fragment as first operand)
  __device__ __forceinline__ void fold_scales(int kt_local, u32x2 (&sc)[Cfg::TN][4]) const {
    const uint32_t grp = ((kt_local + kt0) * Cfg::BK) / group;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t wn = (wave % Cfg::WAVES_N) * Cfg::WTN;
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t n = block0 * 16 + wn + 32 * j + 8 * q + 4 * (lane >> 5);
        sc[j][q] = buf_load8(rsc, n < N ? (grp * N + n) * 2u : OOB);
      }
  }
  // acc += s * part over the accumulators, then part = 0.  The mode's OR
  // (1.0 without scales) is applied here, where the scale registers are first
  // read: that is after the k-tile's wait, so the compiler's own wait for
  // them holds back nothing younger.
  __device__ __forceinline__ void fold(f32x16 (&acc)[Cfg::TM][Cfg::TN], f32x16 (&part)[Cfg::TM][Cfg::TN],
                                       const u32x2 (&sc)[Cfg::TN][4]) const {
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s = from_bits<DT_BF16>(((sc[j][q][e / 2] >> (16 * (e % 2))) & 0xffffu) | sor);
#pragma unroll
          for (int i = 0; i < Cfg::TM; ++i) acc[i][j][4 * q + e] = __builtin_fmaf(s, part[i][j][4 * q + e], acc[i][j][4 * q + e]);
        }
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) part[i][j] = f32x16{};
  }
  // EXACT: does the group of k-tile kt_local end with it (or does the k-range)?
  __device__ __forceinline__ bool group_ends(int kt_local, int nk) const {
    return kt_local + 1 == nk || (((kt_local + kt0 + 1) * Cfg::BK) % group) == 0;
  }
};

template <class Ld>
constexpr int dma_count() {
  if constexpr (Ld::kDMA)
    return Ld::P;
  else
    return 0;
}

struct NoRegs {};
template <class Ld, bool = Ld::kDMA>
struct RegsOf {
  using type = NoRegs;
};
template <class Ld>
struct RegsOf<Ld, false> {
  using type = typename Ld::Regs;
};
struct NoPrep {};
template <class Ld, bool = Ld::kDMA>
struct PrepOf {
  using type = typename Ld::Prep;
};
template <class Ld>
struct PrepOf<Ld, false> {
  using type = NoPrep;
};

// ---------------------------------------------------------------------------
// Multiply one stage: acc[i][j] += B-fragment j x A-fragment i for every 16-k
// step, the A tile at `sa` and the B tile at `sb`.  The MFMA's first operand
// is the B tile (rows n), its second the A tile (rows m), so each lane's four
// consecutive result registers are four consecutive n of one output row m.
// On entry fa[0] / fb[0] hold this stage's first-step fragments; during step
// kk the fragments of step kk + 1 are read, and during the last step those of
// the first step of the next k-tile at `na` / `nb` (already visible when
// CROSS is set) -- so no step starts by waiting on LDS.  The instruction order
// is fixed slot by slot (each slot closed by a scheduling barrier): one MFMA,
// then one fragment read, then the direct-to-LDS copies that fall in this
// slot -- first those of loader l1 (k-tile k1 into d1), then those of l2 (k2
// into d2) -- spread evenly over the first 1 / SPAN_DIV of the stage so the
// memory pipeline is fed at its own rate instead of receiving a burst that
// would stall the wave (and the matrix core) at issue.
// ---------------------------------------------------------------------------
// Per-lane LDS byte offsets of this wave's fragments, per matrix step and
// operand (one 16-byte chunk per fragment for 16-bit inputs, two for fp8):
// the row of fragment i (j) is 32 i (32 j) past the first and the swizzle
// repeats every RPL * CPR rows, which divides 32, so fragment i sits a
// constant 32 i rows past fragment 0 of the same step.
template <class Cfg>
struct FragAddr {
  static constexpr int KK = Cfg::KK, FC = Cfg::FC;
  static_assert(32 % (Cfg::RPL * Cfg::CPR) == 0, "swizzle period must divide the fragment row step");
  uint32_t a[KK][FC], b[KK][FC];
  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave / Cfg::WAVES_N) * Cfg::WTM, wn = (wave % Cfg::WAVES_N) * Cfg::WTN;
    const int frow = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int t = 0; t < FC; ++t) {
        a[kk][t] = (uint32_t)Cfg::off(wm + frow, Cfg::frag_chunk(kk, h, t));
        b[kk][t] = (uint32_t)Cfg::off(wn + frow, Cfg::frag_chunk(kk, h, t));
      }
  }
};

// the fragment a lane holds for one matrix instruction
template <class Cfg>
using frag_t = typename std::conditional<Cfg::FC == 1, u32x4, u32x8>::type;

template <class Cfg>
__device__ __forceinline__ frag_t<Cfg> frag_at(const char* st, const uint32_t (&base)[Cfg::FC], int blk) {
  if constexpr (Cfg::FC == 1) {
    return *(const u32x4*)(st + base[0] + blk * 32 * Cfg::ROWB);
  } else {
    const u32x4 lo = *(const u32x4*)(st + base[0] + blk * 32 * Cfg::ROWB);
    const u32x4 hi = *(const u32x4*)(st + base[1] + blk * 32 * Cfg::ROWB);
    return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// one accumulator block: acc += B fragment x A fragment
template <class Cfg, int DT>
__device__ __forceinline__ f32x16 mma_block(const frag_t<Cfg>& fb, const frag_t<Cfg>& fa, f32x16 acc) {
  if constexpr (DT == DT_F8)
    return mfma32_f8(fb, fa, acc);
  else
    return mfma32<DT>(fb, fa, acc);
}

template <class Cfg>
__device__ __forceinline__ void read_frags(const FragAddr<Cfg>& fa_, const char* sa, const char* sb, int kk,
                                           frag_t<Cfg> (&fa)[Cfg::TM], frag_t<Cfg> (&fb)[Cfg::TN]) {
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) fa[i] = frag_at<Cfg>(sa, fa_.a[kk], i);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) fb[j] = frag_at<Cfg>(sb, fa_.b[kk], j);
}

// Copies spread over the first SPAN matrix slots of a stage: slot i issues
// copies [ceil(i T / SPAN), ceil((i + 1) T / SPAN)).  The ranges tile [0, T)
// in order, so every copy is issued exactly once and those of the first
// loader (indices below P1) all go out before any of the second's -- the
// order the end-of-stage waits count on.
constexpr int slot_first_copy(int slot, int T, int SPAN) { return slot < SPAN ? (slot * T + SPAN - 1) / SPAN : T; }
constexpr bool copy_slots_tile(int T, int SPAN, int SLOTS) {
  if (SPAN < 1 || SPAN > SLOTS) return false;
  int next = 0;
  for (int i = 0; i < SLOTS; ++i) {
    const int v0 = slot_first_copy(i, T, SPAN), v1 = slot_first_copy(i + 1, T, SPAN);
    if (v0 != next || v1 < v0) return false;
    next = v1;
  }
  return next == T;
}

template <class Cfg, int DT, bool CROSS, int SPAN_DIV, class L1, class L2>
__device__ __forceinline__ void multiply_stage(const FragAddr<Cfg>& ad, const char* sa, const char* sb,
                                               const char* na, const char* nb, f32x16 (&acc)[Cfg::TM][Cfg::TN],
                                               frag_t<Cfg> (&fa)[2][Cfg::TM], frag_t<Cfg> (&fb)[2][Cfg::TN],
                                               const L1& l1, int k1, char* d1, const L2& l2, int k2, char* d2) {
  constexpr int KK = Cfg::KK;
  static_assert(KK % 2 == 0, "fragment double buffer flips once per step");
  constexpr int NMFMA = Cfg::TM * Cfg::TN, NDS = Cfg::TM + Cfg::TN;
  constexpr int P1 = dma_count<L1>(), P2 = dma_count<L2>(), T = P1 + P2;
  constexpr int SPAN = (KK * NMFMA + SPAN_DIV - 1) / SPAN_DIV;  // copy slots
  static_assert(copy_slots_tile(T, SPAN, KK * NMFMA), "each copy of the stage is issued once, in loader order");
  typename PrepOf<L1>::type p1{};
  typename PrepOf<L2>::type p2{};
  if constexpr (P1 > 0) p1 = l1.prep(k1);
  if constexpr (P2 > 0) p2 = l2.prep(k2);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int cur = kk & 1, nx = cur ^ 1;
    const bool rd = CROSS || kk + 1 < KK;  // fragments to read during this step
    const char* ra = (kk + 1 < KK) ? sa : na;
    const char* rb = (kk + 1 < KK) ? sb : nb;
    const int rk = (kk + 1 < KK) ? kk + 1 : 0;
#pragma unroll
    for (int m = 0; m < NMFMA; ++m) {
      const int i = m / Cfg::TN, j = m % Cfg::TN;
      acc[i][j] = mma_block<Cfg, DT>(fb[cur][j], fa[cur][i], acc[i][j]);
      if (rd) {
        if (m < Cfg::TM)
          fa[nx][m] = frag_at<Cfg>(ra, ad.a[rk], m);
        else if (m < NDS)
          fb[nx][m - Cfg::TM] = frag_at<Cfg>(rb, ad.b[rk], m - Cfg::TM);
      }
      const int slot = kk * NMFMA + m;
      const int v0 = slot_first_copy(slot, T, SPAN), v1 = slot_first_copy(slot + 1, T, SPAN);
#pragma unroll
      for (int v = v0; v < v1; ++v) {
        if constexpr (P1 > 0) {
          if (v < P1) l1.issue_one(v, p1, d1);
        }
        if constexpr (P2 > 0) {
          // the second loader's first copy: fenced so that no copy of the
          // first loader can be scheduled after it
          if (v == P1 && P1 > 0) __builtin_amdgcn_sched_barrier(0);
          if (v >= P1) l2.issue_one(v - P1, p2, d2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NMFMA < NDS) {  // more fragments than MFMA slots
      if (rd) {
#pragma unroll
        for (int m = NMFMA; m < NDS; ++m) {
          if (m < Cfg::TM)
            fa[nx][m] = frag_at<Cfg>(ra, ad.a[rk], m);
          else
            fb[nx][m - Cfg::TM] = frag_at<Cfg>(rb, ad.b[rk], m - Cfg::TM);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Mainloop.  Three schemes, picked by the tile configuration:
//
// Split ring (SLOTS > 0, direct-to-LDS operands): single-operand slots, A of
// k-tile kt in slot 2 kt, B in slot 2 kt + 1 (mod SLOTS).  While the waves
// multiply k-tile kt (two slots), the other three or more slots take the
// copies of B of kt + 1 (early in the stage) and A of kt + 2 (late in the
// stage), so the copy stream never drains; at the end of kt each wave waits
// for its copies of B of kt + 1 only (vmcnt counts down in issue order, A of
// kt + 2 stays in flight) and a barrier publishes k-tile kt + 1.
//
// Stage ring (EARLY, STAGES >= 3, direct-to-LDS operands, prefetch distance
// D = STAGES - 1): while the waves multiply k-tile kt, the copies of k-tile
// kt + D stream into the stage freed by k-tile kt - 1; at the end of kt each
// wave waits until its copies of k-tile kt + 2 have landed and a barrier
// publishes them; k-tile kt + 1, published one step earlier, is already
// being read -- its first fragments come in during the last step of kt.
//
// Two stages (register-staged operands such as the uint4 weights, or two
// direct-to-LDS stages): the loads of k-tile kt + 1 are issued during the
// multiply of kt (copies in its first half), written to the other stage and
// waited for in full at the end of kt.
//
// Copies past the last k-tile are issued anyway (they re-read the last
// k-tile or land as zeros), keeping counts uniform and the multiply free of
// branches.
// ---------------------------------------------------------------------------
template <class Cfg, int DT, class ALd, class BLd>
__device__ __forceinline__ void mainloop(char* lds, const ALd& al, const BLd& bl, int nk,
                                         f32x16 (&acc)[Cfg::TM][Cfg::TN]) {
  constexpr int S = Cfg::STAGES, D = S - 1;
  constexpr int PA = dma_count<ALd>(), PB = dma_count<BLd>(), PT = PA + PB;
  constexpr bool DMA = ALd::kDMA && BLd::kDMA;
  constexpr bool SPLIT = Cfg::SLOTS > 0;
  constexpr bool REG = !SPLIT && (!DMA || S == 2);
  constexpr bool FIX = ALd::kFIX || BLd::kFIX;
  static_assert(!SPLIT || DMA, "the split ring takes direct-to-LDS operands");
  static_assert(SPLIT || (REG ? S == 2 : S >= 3), "register-staged operands use two stages");
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = f32x16{};
  // the previous tile's epilogue may still be reading the stages
  __builtin_amdgcn_s_barrier();
  if (nk <= 0) return;
  frag_t<Cfg> fa[2][Cfg::TM], fb[2][Cfg::TN];
  FragAddr<Cfg> ad;
  ad.init();

  // The waits below count outstanding vector-memory operations in issue
  // order (the compiler does not track direct-to-LDS copies), and each leaves
  // in flight exactly the copies issued after the ones it waits for:
  //   split ring: a stage issues B of kt + 1 (multiply_stage's first loader,
  //     PB copies), then A of kt + 2 (its second, PA); waiting down to PA
  //     lands B of kt + 1.  The prologue issues A0, B0, A1: down to PA lands
  //     A0 and B0.
  //   stage ring: a stage issues the PT copies of k-tile kt + D; k-tiles
  //     kt + 3 .. kt + D stay in flight, (D - 2) PT copies.
  //   two stages: everything is waited for (0).
  static_assert(!SPLIT || (PA > 0 && PB > 0), "the split ring waits on the A copies of the next k-tile");
  static_assert(SPLIT || REG || (D - 2) * PT < 64, "the stages in flight fit the vmcnt counter");
  if constexpr (SPLIT) {
    constexpr int NS = Cfg::SLOTS;
    // prologue: A0 -> slot 0, B0 -> 1, A1 -> 2; A0 and B0 landed and published
    al.issue(0, lds);
    bl.issue(0, lds + Cfg::SLOT_BYTES);
    al.issue(1, lds + 2 * Cfg::SLOT_BYTES);
    wait_vm_le<PA>();
    al.fix_tail(0, lds);
    bl.fix_tail(0, lds + Cfg::SLOT_BYTES);
    if constexpr (FIX) wait_lgkm();
    __builtin_amdgcn_s_barrier();
    int sa = 0;  // slot of A of k-tile kt; B follows
    for (int kt = 0; kt < nk; ++kt) {
      const int sb = (sa + 1) % NS, a1 = (sa + 2) % NS, b1 = (sa + 3) % NS, a2 = (sa + 4) % NS;
      const char* pa = lds + sa * Cfg::SLOT_BYTES;
      const char* pb = lds + sb * Cfg::SLOT_BYTES;
      read_frags<Cfg>(ad, pa, pb, 0, fa[0], fb[0]);
      multiply_stage<Cfg, DT, false, 1>(ad, pa, pb, pa, pb, acc, fa, fb, bl, kt + 1, lds + b1 * Cfg::SLOT_BYTES, al,
                                        kt + 2, lds + a2 * Cfg::SLOT_BYTES);
      wait_vm_le<PA>();
      al.fix_tail(kt + 1, lds + a1 * Cfg::SLOT_BYTES);
      bl.fix_tail(kt + 1, lds + b1 * Cfg::SLOT_BYTES);
      if constexpr (FIX) wait_lgkm();  // the masked chunks are in LDS before the barrier
      __builtin_amdgcn_s_barrier();
      sa = a1;
    }
  } else if constexpr (!REG) {
    // prologue: k-tiles 0 .. D - 1; k-tiles 0 and 1 landed and published
#pragma unroll
    for (int s = 0; s < D; ++s) {
      char* st = lds + s * Cfg::STAGE_BYTES;
      al.issue(s, st);
      bl.issue(s, st + Cfg::A_BYTES);
    }
    wait_vm_le<(D - 2) * PT>();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      al.fix_tail(s, lds + s * Cfg::STAGE_BYTES);
      bl.fix_tail(s, lds + s * Cfg::STAGE_BYTES + Cfg::A_BYTES);
    }
    if constexpr (FIX) wait_lgkm();
    __builtin_amdgcn_s_barrier();
    read_frags<Cfg>(ad, lds, lds + Cfg::A_BYTES, 0, fa[0], fb[0]);
    int cs = 0;  // stage of k-tile kt
    // one loop body (a second copy makes the register allocator shuttle the
    // accumulators between AGPRs and VGPRs); stages are picked per k-tile
    for (int kt = 0; kt < nk; ++kt) {
      const int n1 = (cs + 1) % S, n2 = (cs + 2) % S, nd = (cs + D) % S;
      const char* cur = lds + cs * Cfg::STAGE_BYTES;
      const char* nxs = lds + n1 * Cfg::STAGE_BYTES;
      char* dst = lds + nd * Cfg::STAGE_BYTES;
      multiply_stage<Cfg, DT, true, 1>(ad, cur, cur + Cfg::A_BYTES, nxs, nxs + Cfg::A_BYTES, acc, fa, fb, al, kt + D,
                                       dst, bl, kt + D, dst + Cfg::A_BYTES);
      wait_vm_le<(D - 2) * PT>();
      al.fix_tail(kt + 2, lds + n2 * Cfg::STAGE_BYTES);
      bl.fix_tail(kt + 2, lds + n2 * Cfg::STAGE_BYTES + Cfg::A_BYTES);
      if constexpr (FIX) wait_lgkm();  // the masked chunks are in LDS before the barrier
      __builtin_amdgcn_s_barrier();
      cs = n1;
    }
  } else {
    typename RegsOf<ALd>::type ra;
    typename RegsOf<BLd>::type rb;
    if constexpr (ALd::kDMA) al.issue(0, lds); else al.load(0, ra);
    if constexpr (BLd::kDMA) bl.issue(0, lds + Cfg::A_BYTES); else bl.load(0, rb);
    wait_vm_le<0>();
    if constexpr (ALd::kDMA) al.fix_tail(0, lds); else al.store(lds, ra);
    if constexpr (BLd::kDMA) bl.fix_tail(0, lds + Cfg::A_BYTES); else bl.store(lds + Cfg::A_BYTES, rb);
    wait_lgkm();
    __builtin_amdgcn_s_barrier();
    int cs = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const char* cur = lds + cs * Cfg::STAGE_BYTES;
      char* nxt = lds + (cs ^ 1) * Cfg::STAGE_BYTES;
      const bool more = kt + 1 < nk;
      if constexpr (!ALd::kDMA) {
        if (more) al.load(kt + 1, ra);
      }
      if constexpr (!BLd::kDMA) {
        if (more) bl.load(kt + 1, rb);
      }
      read_frags<Cfg>(ad, cur, cur + Cfg::A_BYTES, 0, fa[0], fb[0]);
      multiply_stage<Cfg, DT, false, 2>(ad, cur, cur + Cfg::A_BYTES, cur, cur + Cfg::A_BYTES, acc, fa, fb, al, kt + 1,
                                        nxt, bl, kt + 1, nxt + Cfg::A_BYTES);
      wait_vm_le<0>();
      if (more) {
        if constexpr (ALd::kDMA) al.fix_tail(kt + 1, nxt); else al.store(nxt, ra);
        if constexpr (BLd::kDMA) bl.fix_tail(kt + 1, nxt + Cfg::A_BYTES); else bl.store(nxt + Cfg::A_BYTES, rb);
        wait_lgkm();
      }
      __builtin_amdgcn_s_barrier();
      cs ^= 1;
    }
  }
  // copies past the last k-tile are still landing: drain them before anyone
  // reuses the ring
  wait_vm_le<0>();
  __builtin_amdgcn_s_barrier();
}

// ---------------------------------------------------------------------------
// Epilogue: D[m][n] = RN(alpha * acc + beta * C[m][n]) in fp32, C read only
// when beta != 0.  Lane l of accumulator block (i, j), register group q holds
// row 32 i + l % 32 and columns 32 j + 8 q + 4 (l / 32) + {0..3} of its wave
// tile; written straight to memory those would be 8-byte runs scattered over
// 32 rows.  Instead each wave stages its fp32 accumulators in its own LDS
// region (the stages are free after the last k-tile), PASS blocks of 32 rows
// at a time, and reads them back row-major, 8 floats per lane: every store
// instruction writes whole row segments, 16 bytes per lane.  Region row r
// holds WTN floats in 16-byte chunks, chunk x in slot x ^ (r % 16) ^ bit 4 of
// x: 16 lanes writing one chunk of 16 rows, or reading the even (odd) chunks
// of one row, touch all 64 banks once.  Rows past M are dropped by the
// store's buffer range; a tile that crosses N stores element by element.
// ---------------------------------------------------------------------------

// fp32 partial tile: each lane's accumulator runs (4 consecutive n of one
// row m) stored as they are, rows past M dropped by the buffer range,
// columns past N skipped
template <class Cfg>
__device__ __forceinline__ void store_partial(const Tile& t, const f32x16 (&acc)[Cfg::TM][Cfg::TN], float* P) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave / Cfg::WAVES_N) * Cfg::WTM, wn = (wave % Cfg::WAVES_N) * Cfg::WTN;
  int rows = t.M - t.m0;
  if (rows > Cfg::BM) rows = Cfg::BM;
  const rsrc_t rp = make_rsrc(P + (int64_t)t.m0 * t.N, (uint32_t)rows * (uint32_t)t.N * 4u);
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t row = wm + 32 * i + (lane & 31);
        const int col = t.n0 + wn + 32 * j + 8 * q + 4 * (lane >> 5);
        if (col < t.N)
          buf_store16_wb(rp, (row * (uint32_t)t.N + col) * 4u,
                      __builtin_bit_cast(u32x4, f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                                      acc[i][j][4 * q + 3]}));
      }
}

template <class Cfg, int DT, bool MAPPED = false>
__device__ __forceinline__ void store_tile(const Tile& t, const f32x16 (&acc)[Cfg::TM][Cfg::TN], float alpha,
                                           float beta, char* lds, const RowMap& map = RowMap{}) {
  constexpr int ROWB = Cfg::WTN * 4;  // fp32 row of the wave tile
  constexpr int PASS = (Cfg::NW * 2 * 32 * ROWB <= Cfg::LDS_BYTES && Cfg::TM % 2 == 0) ? 2 : 1;  // 32-row blocks per pass
  constexpr int REGION = PASS * 32 * ROWB;
  static_assert(Cfg::NW * REGION <= Cfg::LDS_BYTES && Cfg::TM % PASS == 0, "the wave regions must fit the stages");
  constexpr int LPR = Cfg::WTN / 8;  // lanes per row on read-back (8 floats each)
  constexpr int RPI = 64 / LPR;      // rows per read-back instruction
  // the staging addresses depend only on the lane; kept opaque here so they
  // are formed per tile instead of being hoisted out of the tile loop and
  // held in registers through the mainloop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave / Cfg::WAVES_N) * Cfg::WTM, wn = (wave % Cfg::WAVES_N) * Cfg::WTN;
  char* reg = lds + wave * REGION;
  // 16-byte slot of chunk x in row r: XOR with up to 4 row bits (as many as
  // the row has chunks), plus bit 4 for rows of 32 or more chunks
  constexpr int CH = Cfg::WTN / 4;
  constexpr int XM = CH >= 16 ? 15 : CH - 1;
  auto slot = [](int r, int x) { return (x ^ (r & XM) ^ (CH >= 32 ? (x >> 4) & 1 : 0)) << 4; };

  int rows = t.M - t.m0;
  if (rows > Cfg::BM) rows = Cfg::BM;
  const bool use_c = beta != 0.0f;
  const bool full_n = t.n0 + Cfg::BN <= t.N;
  // plain rows: resources from the tile's first row, row pitch ld, rows past
  // M outside the range; mapped rows: resources over the whole tensor, each
  // row at its mapped offset, rows past M pointed out of range
  const rsrc_t rd = MAPPED ? make_rsrc(t.D, map.bytes)
                           : make_rsrc(t.D + (int64_t)t.m0 * t.ldd, (uint32_t)rows * (uint32_t)t.ldd * 2u);
  const rsrc_t rc = !use_c ? rd
                    : MAPPED ? make_rsrc(t.C, map.bytes)
                             : make_rsrc(t.C + (int64_t)t.m0 * t.ldc, (uint32_t)rows * (uint32_t)t.ldc * 2u);
  const uint32_t ldd2 = (uint32_t)t.ldd * 2u, ldc2 = (uint32_t)t.ldc * 2u;
  auto row_d = [&](uint32_t row) -> uint32_t {
    if constexpr (MAPPED) return (int)row < rows ? map.offset(t.m0 + (int)row) * 2u : OOB;
    return row * ldd2;
  };
  auto row_c = [&](uint32_t row) -> uint32_t {
    if constexpr (MAPPED) return (int)row < rows ? map.offset(t.m0 + (int)row) * 2u : OOB;
    return row * ldc2;
  };
  const bool use_bias = t.bias != nullptr, relu = t.act == ACT_RELU;
  const rsrc_t rbias = use_bias ? make_rsrc(t.bias, (uint32_t)t.N * 2u) : rd;

#pragma unroll
  for (int p0 = 0; p0 < Cfg::TM; p0 += PASS) {
#pragma unroll
    for (int ii = 0; ii < PASS; ++ii) {
      const int r = ii * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int x = 8 * j + 2 * q + (lane >> 5);  // 16-byte chunk: columns 4x .. 4x + 3
          const f32x4 v{acc[p0 + ii][j][4 * q], acc[p0 + ii][j][4 * q + 1], acc[p0 + ii][j][4 * q + 2],
                        acc[p0 + ii][j][4 * q + 3]};
          *(f32x4*)(reg + r * ROWB + slot(r, x)) = v;
        }
    }
#pragma unroll
    for (int k = 0; k < PASS * 32 / RPI; ++k) {
      const int r = k * RPI + lane / LPR, c = lane % LPR;  // lane stores columns 8c .. 8c + 7
      const f32x4 a0 = *(const f32x4*)(reg + r * ROWB + slot(r, 2 * c));
      const f32x4 a1 = *(const f32x4*)(reg + r * ROWB + slot(r, 2 * c + 1));
      float v[8] = {alpha * a0[0], alpha * a0[1], alpha * a0[2], alpha * a0[3],
                    alpha * a1[0], alpha * a1[1], alpha * a1[2], alpha * a1[3]};
      const uint32_t row = (uint32_t)(wm + p0 * 32 + r);
      const uint32_t od = row_d(row), oc = use_c ? row_c(row) : 0u;
      const int col = t.n0 + wn + 8 * c;
      if (full_n || col + 8 <= t.N) {
        if (use_c) {
          const u32x4 c4 = buf_load16(rc, oc + (uint32_t)col * 2u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] += beta * from_bits<DT>(c4[e] & 0xffffu);
            v[2 * e + 1] += beta * from_bits<DT>(c4[e] >> 16);
          }
        }
        if (use_bias) {
          const u32x4 b4 = buf_load16(rbias, (uint32_t)col * 2u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] += from_bits<DT>(b4[e] & 0xffffu);
            v[2 * e + 1] += from_bits<DT>(b4[e] >> 16);
          }
        }
        if (relu) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] > 0.0f ? v[e] : 0.0f;
        }
        buf_store16(rd, od + (uint32_t)col * 2u,
                    u32x4{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]), pack2<DT>(v[4], v[5]), pack2<DT>(v[6], v[7])});
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (col + e < t.N) {
            float x = v[e];
            if (use_c) x += beta * from_bits<DT>(buf_load2(rc, oc + (uint32_t)(col + e) * 2u));
            if (use_bias) x += from_bits<DT>(buf_load2(rbias, (uint32_t)(col + e) * 2u));
            if (relu) x = x > 0.0f ? x : 0.0f;
            buf_store2(rd, od + (uint32_t)(col + e) * 2u, to_bits<DT>(x));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent walk.  Workgroups are dispatched round-robin over the 8 XCDs;
// slot w of a round of G workgroups (G a multiple of 8) is remapped so that
// the G/8 workgroups of one XCD take G/8 consecutive tiles, which share
// operand panels in that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int XCDS = 8;
__device__ __forceinline__ int remap_slot(int w, int G) { return (w % XCDS) * (G / XCDS) + w / XCDS; }

// Tile order inside one problem of tm x tn tiles: bands of up to RASTER_M
// m-tiles, the m index fastest inside a band.  An XCD's run of consecutive
// tiles then covers a block of at most RASTER_M m-tiles by a few n-tiles, so
// at every k-step its CUs fetch few distinct A and B panel slices into its L2.
constexpr int RASTER_M = 8;
__device__ __forceinline__ void raster(int local, int tm, int tn, int& mi, int& ni, int band_m = RASTER_M) {
  const int band = local / (band_m * tn);
  const int r = local - band * band_m * tn;
  const int left = tm - band * band_m;
  const int rows = left < band_m ? left : band_m;
  mi = band * band_m + r % rows;
  ni = r / rows;
}

}  // namespace gmi
