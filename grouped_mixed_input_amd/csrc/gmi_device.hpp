// gmi_device.hpp -- device building blocks shared by every kernel of the
// library: element types, gfx950 MFMA wrappers, the LDS tile layout, operand
// loaders (dense, implicit-conv, prepacked uint4), the tiled mainloop, the
// alpha/beta epilogue and the persistent tile walk.
//
// The mainloop follows the structure of the persistent grouped GEMM kernel on
// the page sm90_gemm_array_tma_warpspecialized_cooperative.hpp (operator():
// a work-tile loop, a k-tile loop that accumulates in fp32 starting from
// zero, an epilogue store per tile) rebuilt for CDNA4: every wave both loads
// and computes, operands are staged global -> VGPR -> LDS in two ping-pong
// buffers, and v_mfma_f32_32x32x16_{f16,bf16} consumes 128-bit LDS reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmi {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { DT_F16 = 0, DT_BF16 = 1 };

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

template <int DT>
__device__ __forceinline__ float from_bits(uint32_t b) {
  if constexpr (DT == DT_F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  else
    return __builtin_bit_cast(float, b << 16);
}

// ---------------------------------------------------------------------------
// LDS operand tile: rows of 64 k values (128 bytes = eight 16-byte chunks).
// Chunk c of row r lives at chunk slot c ^ (r & 7), so the eight rows read by
// any eight consecutive lanes of a fragment load fall in distinct slots.
// ---------------------------------------------------------------------------
constexpr int BK = 64;
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// ---------------------------------------------------------------------------
// Tile configuration: BM x BN output tile, 4 waves arranged WM_ x WN_.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;            // 32x32 blocks per wave
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
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
};

// ---------------------------------------------------------------------------
// Dense K-contiguous operand loader: ROWS rows x 64 k per k-tile.  Thread t
// moves chunk t % 8 of rows t / 8 + i * (THREADS / 8), 16 bytes each.
// Rows past `rows_valid` and k past K read as zero.
// ---------------------------------------------------------------------------
template <int ROWS, int THREADS>
struct DenseLoader {
  static constexpr int RPP = THREADS / 8;
  static constexpr int P = ROWS / RPP;
  static_assert(ROWS % RPP == 0, "rows must be a multiple of THREADS / 8");
  struct Regs {
    u32x4 v[P];
  };
  const uint16_t* p0;  // row (t / 8) of this tile, or null when no row is valid
  int64_t step;        // RPP rows, in elements
  int nvalid;          // passes whose row is inside the problem
  int K;

  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int row0, int rows, int K_) {
    int r = threadIdx.x / 8;
    int left = rows - row0 - r;  // rows available from this thread's first row
    nvalid = left <= 0 ? 0 : (left + RPP - 1) / RPP;
    if (nvalid > P) nvalid = P;
    p0 = base + (int64_t)(row0 + r) * ld + (threadIdx.x & 7) * 8;
    step = (int64_t)RPP * ld;
    K = K_;
  }

  __device__ __forceinline__ void load(int kt, Regs& rg) const {
    u32x4(&v)[P] = rg.v;
    const int kc = kt * BK + (threadIdx.x & 7) * 8;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint16_t* p = p0 + i * step + kt * BK;
      if (i < nvalid && kc + 8 <= K) {
        v[i] = *(const u32x4*)p;
      } else if (i < nvalid && kc < K) {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (kc + e < K) ? p[e] : 0u;
        v[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      } else {
        v[i] = u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ __forceinline__ void store(char* lds, const Regs& rg) const {
#pragma unroll
    for (int i = 0; i < P; ++i) *(u32x4*)(lds + lds_off(threadIdx.x / 8 + i * RPP, threadIdx.x & 7)) = rg.v[i];
  }
};

// ---------------------------------------------------------------------------
// Implicit-GEMM convolution A operand (fprop).  GEMM row m is output pixel
// (n, p, q), m = (n P + p) Q + q; GEMM column k is filter tap (r, s, c),
// k = (r S + s) C + c.  Element (m, k) is x[n][p sh - ph + r dh][q sw - pw + s dw][c]
// or 0 outside the image -- the im2col view of the activation that the page
// sm100_implicit_gemm_umma_warpspecialized.hpp builds from the padding,
// traversal stride and dilation (get_tma_load_a_instance), formed here by
// address arithmetic instead.  With C % 8 == 0 a 16-byte chunk never
// straddles two taps, so each chunk is one aligned 128-bit load or zero.
// ---------------------------------------------------------------------------
struct ConvGeom {
  const uint16_t* x;
  int H, W, C, S;
  int P, Q;
  int ph, pw, sh, sw, dh, dw;
  int Kg;  // R * S * C
};

template <int ROWS, int THREADS>
struct ConvLoader {
  static constexpr int RPP = THREADS / 8;
  static constexpr int P = ROWS / RPP;
  struct Regs {
    u32x4 v[P];
  };
  const uint16_t* x;
  int H, W, C, S, dh, dw, Kg;
  int pix[P];     // first pixel of the row's image: n * H * W
  int h0[P], w0[P];  // input coordinates of tap (0, 0); far negative for rows past M

  __device__ __forceinline__ void init(const ConvGeom& g, int m0, int M) {
    x = g.x;
    H = g.H;
    W = g.W;
    C = g.C;
    S = g.S;
    dh = g.dh;
    dw = g.dw;
    Kg = g.Kg;
    const int PQ = g.P * g.Q;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int m = m0 + threadIdx.x / 8 + i * RPP;
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

  __device__ __forceinline__ void load(int kt, Regs& rg) const {
    const int kc = kt * BK + (threadIdx.x & 7) * 8;
    if (kc >= Kg) {
#pragma unroll
      for (int i = 0; i < P; ++i) rg.v[i] = u32x4{0, 0, 0, 0};
      return;
    }
    const int rs = kc / C, c = kc - rs * C;
    const int r = rs / S, s = rs - r * S;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int ih = h0[i] + r * dh, iw = w0[i] + s * dw;
      if ((unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W)
        rg.v[i] = *(const u32x4*)(x + (int64_t)(pix[i] + ih * W + iw) * C + c);
      else
        rg.v[i] = u32x4{0, 0, 0, 0};
    }
  }

  __device__ __forceinline__ void store(char* lds, const Regs& rg) const {
#pragma unroll
    for (int i = 0; i < P; ++i) *(u32x4*)(lds + lds_off(threadIdx.x / 8 + i * RPP, threadIdx.x & 7)) = rg.v[i];
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

__device__ __forceinline__ u32x4 dequant8(uint32_t w, f16x2 zz, f16x2 ss) {
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 h = __builtin_bit_cast(f16x2, ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u);
    h = (h - zz) * ss;
    out[i] = __builtin_bit_cast(uint32_t, h);
  }
  return out;
}

// Prepacked weight geometry: 16 rows x 128 k per 1024-byte block, block
// (n / 16, k / 128) at ((n / 16) * (K / 128) + k / 128) * 1024; lane L of a
// block owns bytes [16 L, 16 L + 16): row L % 16, word j covering
// k = 32 j + 8 (L / 16) + {0..7}.
struct W4Geom {
  const uint8_t* w;        // prepacked weight
  const uint16_t* scales;  // [K / g][N] fp16
  const uint8_t* zeros;    // [K / g][N / 2] uint4
  int N, K, group;
};

// ---------------------------------------------------------------------------
// Prepacked uint4 weight as the B operand (rows n, 64 k per k-tile): a k-tile
// takes words j = 2 (kt % 2) + {0, 1} of every lane entry of the 16-row blocks
// it covers -- 8 bytes per entry -- plus each entry's scale and zero.  The
// dequantisation runs when the registers are written to LDS, so it overlaps
// the matrix instructions of the other waves.
// ---------------------------------------------------------------------------
template <int ROWS, int THREADS>
struct W4Loader {
  static constexpr int ENTRIES = ROWS / 16 * 64;
  static constexpr int P = ENTRIES / THREADS;
  static_assert(ENTRIES % THREADS == 0, "rows must cover whole lane-entry passes");
  struct Regs {
    u32x2 w[P];
    uint32_t sz[P];  // scale bits | zero << 16
  };
  W4Geom g;
  int n0;

  __device__ __forceinline__ void init(const W4Geom& g_, int n0_) {
    g = g_;
    n0 = n0_;
  }

  __device__ __forceinline__ void load(int kt, Regs& rg) const {
    const int kblocks = g.K / 128;
    const int grp = (kt * BK) / g.group;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = threadIdx.x + i * THREADS;
      const int nb = e / 64, L = e % 64;
      const int n = n0 + nb * 16 + (L % 16);
      if (n < g.N) {
        const uint8_t* src = g.w + ((int64_t)((n0 / 16 + nb) * kblocks + kt / 2) * 1024 + L * 16 + (kt & 1) * 8);
        rg.w[i] = *(const u32x2*)src;
        const uint32_t s = g.scales[(int64_t)grp * g.N + n];
        const uint32_t z = (g.zeros[(int64_t)grp * (g.N / 2) + n / 2] >> ((n & 1) * 4)) & 15u;
        rg.sz[i] = s | (z << 16);
      } else {
        rg.w[i] = u32x2{0, 0};
        rg.sz[i] = 0;  // scale 0, zero 0: the row dequantises to zeros
      }
    }
  }

  __device__ __forceinline__ void store(char* lds, const Regs& rg) const {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = threadIdx.x + i * THREADS;
      const int nb = e / 64, L = e % 64;
      const int row = nb * 16 + (L % 16), h = L / 16;
      const f16x2 ss = scale_pair(rg.sz[i] & 0xffffu), zz = zero_pair((rg.sz[i] >> 16) & 15u);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) *(u32x4*)(lds + lds_off(row, 4 * jj + h)) = dequant8(rg.w[i][jj], zz, ss);
    }
  }
};

// ---------------------------------------------------------------------------
// Mainloop: acc[tm][tn] += B-fragment x A-fragment over all k-tiles.
// The MFMA's first operand is the B tile (rows n), its second the A tile
// (rows m), so each lane's four consecutive result registers are four
// consecutive n of one output row m: the epilogue writes 8-byte runs.
// Two LDS stages: while the waves multiply stage s, the next k-tile is loaded
// into registers and written into stage s ^ 1; one barrier per k-tile.
// ---------------------------------------------------------------------------
template <class Cfg, int DT, class ALd, class BLd>
__device__ __forceinline__ void mainloop(char* lds, const ALd& al, const BLd& bl, int nk,
                                         f32x16 (&acc)[Cfg::TM][Cfg::TN]) {
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = f32x16{};
  if (nk <= 0) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave / Cfg::WAVES_N) * Cfg::WTM, wn = (wave % Cfg::WAVES_N) * Cfg::WTN;
  const int frow = lane & 31, fchunk = lane >> 5;

  typename ALd::Regs ra;
  typename BLd::Regs rb;
  al.load(0, ra);
  bl.load(0, rb);
  al.store(lds, ra);
  bl.store(lds + Cfg::A_BYTES, rb);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* sa = lds + (kt & 1) * Cfg::STAGE_BYTES;
    char* sb = sa + Cfg::A_BYTES;
    const bool more = kt + 1 < nk;
    if (more) {
      al.load(kt + 1, ra);
      bl.load(kt + 1, rb);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      u32x4 fa[Cfg::TM], fb[Cfg::TN];
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i) fa[i] = *(const u32x4*)(sa + lds_off(wm + i * 32 + frow, kk * 2 + fchunk));
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) fb[j] = *(const u32x4*)(sb + lds_off(wn + j * 32 + frow, kk * 2 + fchunk));
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = mfma32<DT>(fb[j], fa[i], acc[i][j]);
    }
    if (more) {
      char* na = lds + ((kt + 1) & 1) * Cfg::STAGE_BYTES;
      al.store(na, ra);
      bl.store(na + Cfg::A_BYTES, rb);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Epilogue: D[m][n] = RN(alpha * acc + beta * C[m][n]); C is read only when
// beta != 0.  Lane l of block (i, j), register group q holds
// m = wm + 32 i + l % 32, n = wn + 32 j + 8 q + 4 (l / 32) + {0..3}.
// ---------------------------------------------------------------------------
template <class Cfg, int DT>
__device__ __forceinline__ void epilogue(const Tile& t, const f32x16 (&acc)[Cfg::TM][Cfg::TN], float alpha,
                                         float beta) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave / Cfg::WAVES_N) * Cfg::WTM, wn = (wave % Cfg::WAVES_N) * Cfg::WTN;
  const bool use_c = beta != 0.0f;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
    const int m = t.m0 + wm + i * 32 + (lane & 31);
    if (m >= t.M) continue;
    uint16_t* drow = t.D + (int64_t)m * t.ldd;
    const uint16_t* crow = use_c ? t.C + (int64_t)m * t.ldc : nullptr;
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = t.n0 + wn + j * 32 + q * 8 + (lane >> 5) * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = alpha * acc[i][j][q * 4 + e];
        if (n + 4 <= t.N) {
          if (use_c) {
            u32x2 c2 = *(const u32x2*)(crow + n);
            v[0] += beta * from_bits<DT>(c2[0] & 0xffffu);
            v[1] += beta * from_bits<DT>(c2[0] >> 16);
            v[2] += beta * from_bits<DT>(c2[1] & 0xffffu);
            v[3] += beta * from_bits<DT>(c2[1] >> 16);
          }
          *(u32x2*)(drow + n) =
              u32x2{to_bits<DT>(v[0]) | (to_bits<DT>(v[1]) << 16), to_bits<DT>(v[2]) | (to_bits<DT>(v[3]) << 16)};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e < t.N) {
              float r = v[e];
              if (use_c) r += beta * from_bits<DT>(crow[n + e]);
              drow[n + e] = (uint16_t)to_bits<DT>(r);
            }
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

}  // namespace gmi
