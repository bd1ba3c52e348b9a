// kernels_w4a16.hip -- mixed-input GEMM Y = X W^T with prepacked uint4 W.
//
// The page machete_mainloop.cuh computes the transposed problem so that the
// narrow weight becomes the register-sourced operand, prepacks it so that one
// thread's values for several matrix instructions come from one 128-bit load,
// and dequantises it in registers (convert, scale, zero) right before the
// multiply.  Here:
//   * k_prepack_w4 reorders the plain [N][K/2] uint4 weight once.
//   * k_w4a16_skinny (48 < M <= 64) streams the prepacked weight straight from HBM
//     into VGPRs -- one 16-byte load per lane is one 16-row x 128-k block, i.e.
//     four v_mfma_f32_16x16x32_f16 A fragments -- with the weight rows on the
//     MFMA's M side and the tokens on its N side (the same swap as the page).
//     The waves of a workgroup split K and reduce through LDS.
//   * k_w4a16_tiled (M > 64) is the dense mainloop with the weight loader
//     (W4Loader) dequantising into the LDS B tile.

#include <type_traits>

#include "gmi_device.hpp"
#include "gmi_internal.hpp"

namespace gmi {

// ---------------------------------------------------------------------------
// Prepack: one thread per 32-bit output word.  Output word (block b, lane L,
// word j) holds row n = 16 (b / kblocks) + L % 16, k = 128 (b % kblocks) +
// 32 j + 8 (L / 16) + e for e = 0..7: the 4 input bytes of that run, with
// the even elements (low nibbles) gathered into bits 0-15 and the odd ones
// (high nibbles) into bits 16-31.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_prepack_w4(const uint8_t* __restrict__ w, int N, int K,
                                                    uint32_t* __restrict__ out) {
  const int64_t words = (int64_t)N * K / 8;
  const int kblocks = K / 128;
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < words; id += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = id / 256;
    const int within = (int)(id % 256);
    const int L = within / 4, j = within % 4;
    const int64_t n = (b / kblocks) * 16 + (L % 16);
    const int64_t k = (b % kblocks) * 128 + 32 * j + 8 * (L / 16);
    const uint32_t u = *(const uint32_t*)(w + n * (K / 2) + k / 2);
    uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
    lo = (lo | (lo >> 4)) & 0x00FF00FFu;
    lo = (lo | (lo >> 8)) & 0x0000FFFFu;
    hi = (hi | (hi >> 4)) & 0x00FF00FFu;
    hi = (hi | (hi >> 8)) & 0x0000FFFFu;
    out[id] = lo | (hi << 16);
  }
}

hipError_t launch_prepack_w4(const uint8_t* w, int N, int K, uint8_t* out, hipStream_t stream) {
  const int64_t words = (int64_t)N * K / 8;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_prepack_w4, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, K, (uint32_t*)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny-M kernel.  Workgroup = KW waves over NB 16-row weight blocks; wave w
// owns a contiguous range of 128-wide k-blocks.  Per k-block a lane loads, per
// weight block, its 16 prepacked bytes (row L % 16, k-group L / 16 of the four
// 32-k sub-blocks) plus that row's scale and zero, and, per 16-token tile, the
// matching four 16-byte X fragments (token L % 16, same k-groups).  The next
// k-block's loads are issued before the current one is multiplied.
// ---------------------------------------------------------------------------
// bf16 activations take the exact integers q - z into an fp32 partial sum per
// k-block, which the scales of the lane's output rows then fold into the
// accumulators (see W4Loader): `so` holds those four scales per weight block.
template <int NB, int MT>
struct SkinnyStage {
  u32x4 w[NB];
  uint32_t sz[NB];
  u32x2 so[NB];
  u32x4 x[MT][4];
};

struct SkinnyRes {
  rsrc_t w, x, s, z;
  uint32_t kblocks;
};

template <int DT, int NB, int MT>
__device__ __forceinline__ void skinny_load(SkinnyStage<NB, MT>& st, const W4Launch& a, const SkinnyRes& rs,
                                            int n_base, int kb, int lane) {
  constexpr bool EXACT = DT == DT_BF16;
  const uint32_t r = lane & 15, h = lane >> 4;
  const uint32_t grp = (uint32_t)(kb * 128) / (uint32_t)a.group;
  const uint32_t N = a.N;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint32_t blk = n_base / 16 + nb, n = blk * 16 + r;
    const bool ok = n < N;
    st.w[nb] = buf_load16(rs.w, ok ? (blk * rs.kblocks + kb) * 1024u + lane * 16u : OOB);
    const uint32_t s = EXACT ? 0u : buf_load2(rs.s, ok ? (grp * N + n) * 2u : OOB) | a.sor;
    const uint32_t z = ((buf_load1(rs.z, ok ? grp * (N / 2) + n / 2 : OOB) >> ((n & 1) * 4)) & 15u) ^ a.zxor;
    st.sz[nb] = s | (z << 16);
    // output rows blk * 16 + 4 h + {0..3} of this lane (N is a multiple of 16)
    if constexpr (EXACT)
      st.so[nb] = buf_load8(rs.s, blk * 16 < N ? (grp * N + blk * 16 + 4 * h) * 2u : OOB) | (a.sor * 0x00010001u);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t tok = mt * 16 + r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      st.x[mt][j] = buf_load16(rs.x, (int)tok < a.M ? (tok * (uint32_t)a.ldx + kb * 128 + j * 32 + h * 8) * 2u : OOB);
  }
}

template <int DT, int NB, int MT>
__device__ __forceinline__ void skinny_mma(const SkinnyStage<NB, MT>& st, uint32_t wxor, f32x4 (&acc)[NB][MT]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (DT == DT_BF16) {
      f32x4 part[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) part[mt] = f32x4{0, 0, 0, 0};
      const float zf = (float)(st.sz[nb] >> 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 wf = exact8_bf16(st.w[nb][j] ^ wxor, zf);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) part[mt] = mfma16<DT>(wf, st.x[mt][j], part[mt]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float si = from_bits<DT_BF16>((st.so[nb][i / 2] >> (16 * (i % 2))) & 0xffffu);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nb][mt][i] = __builtin_fmaf(si, part[mt][i], acc[nb][mt][i]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 wf = dequant8_dt<DT>(st.w[nb][j] ^ wxor, st.sz[nb] & 0xffffu, st.sz[nb] >> 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = mfma16<DT>(wf, st.x[mt][j], acc[nb][mt]);
      }
    }
  }
}

template <int NB, int KW, int MT>
constexpr int skinny_lds_bytes() {
  return KW * NB * MT * 64 * (int)sizeof(f32x4);
}

// weight rows n_base .. n_base + 16 NB of Y = X W^T for the a.M <= 16 MT
// tokens of X; `lds` holds skinny_lds_bytes<NB, KW, MT>() bytes
template <int DT, int NB, int KW, int MT>
__device__ __forceinline__ void skinny_body(const W4Launch& a, int n_base, char* lds) {
  f32x4(*red)[NB * MT * 64] = (f32x4(*)[NB * MT * 64])lds;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kblocks = a.K / 128;
  const int per = (kblocks + KW - 1) / KW;
  const int kb0 = wave * per;
  const int kb1 = kb0 + per < kblocks ? kb0 + per : kblocks;

  f32x4 acc[NB][MT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = f32x4{0, 0, 0, 0};

  SkinnyRes rs;
  rs.w = make_rsrc(a.w, (uint32_t)((int64_t)a.N * a.K / 2));
  rs.x = make_rsrc(a.X, (uint32_t)((int64_t)a.M * a.ldx * 2));
  rs.s = make_rsrc(a.scales, a.s_bytes);
  rs.z = make_rsrc(a.zeros, a.z_bytes);
  rs.kblocks = kblocks;
  if (kb0 < kb1) {
    SkinnyStage<NB, MT> cur, nxt;
    skinny_load<DT, NB, MT>(cur, a, rs, n_base, kb0, lane);
    for (int kb = kb0; kb < kb1; ++kb) {
      if (kb + 1 < kb1) skinny_load<DT, NB, MT>(nxt, a, rs, n_base, kb + 1, lane);
      skinny_mma<DT, NB, MT>(cur, a.wxor, acc);
      cur = nxt;
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][(nb * MT + mt) * 64 + lane] = acc[nb][mt];
  __syncthreads();

  // lane-quad q of (nb, mt): rows n = n_base + 16 nb + 4 (q / 16) + {0..3}, token 16 mt + q % 16
  for (int idx = threadIdx.x; idx < NB * MT * 64; idx += 64 * KW) {
    f32x4 s = red[0][idx];
#pragma unroll
    for (int w = 1; w < KW; ++w) s += red[w][idx];
    const int nb = idx / (MT * 64), mt = (idx / 64) % MT, q = idx % 64;
    const int n = n_base + nb * 16 + 4 * (q / 16), tok = mt * 16 + (q % 16);
    if (tok < a.M && n < a.N) {
      *(gu32x2*)(a.Y + (int64_t)tok * a.ldy + n) = u32x2{pack2<DT>(s[0], s[1]), pack2<DT>(s[2], s[3])};
    }
  }
}

template <int DT, int NB, int KW, int MT>
__global__ __launch_bounds__(64 * KW) void k_w4a16_skinny(W4Launch a) {
  __shared__ __attribute__((aligned(16))) char lds[skinny_lds_bytes<NB, KW, MT>()];
  skinny_body<DT, NB, KW, MT>(a, blockIdx.x * NB * 16, lds);
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 16, or M <= 48 as two or three 16-row tiles): the weight
// stream is the whole cost (N K / 2 bytes
// against 2 M (N + K) for X and Y), so it is put in flight as early and as
// deep as the LDS allows.  Workgroup = KW waves over NB 16-row weight blocks;
// wave w owns a contiguous range of 128-wide k-blocks, taken R at a time
// (one round), and works alone until the final reduction.  Per round a wave
// issues, without waiting:
//   * two direct-to-LDS copies of the round's scale and zero-point rows
//     (32 rows x R groups);
//   * per k-block, its NB weight blocks of 1 KB each (one block of the
//     prepacked layout per copy) into the wave's own LDS ring, then its X
//     fragments into registers (token L % 16, k-group L / 16 of each 32-k
//     step; L2-resident, shared by every workgroup).
// It then multiplies the k-blocks in order, each after a wait that leaves the
// younger weight copies in flight.  Per k-block (one 128-k scale group) the
// MFMA takes the exact integers q - z as fp16 (the 0x6400 construction of
// transform_A_kblock's conversion without the scale) into a fresh fp32
// partial sum, and each output row's scale multiplies that partial sum:
// sum_k (q - z) s x = sum over groups of s * sum_k (q - z) x, with the scale
// applied in fp32 instead of rounding every weight to fp16 first.  With bf16
// activations the MFMA takes 128 + q (bf16 0x4300 | q, exact) and
// (128 + z) sum_k x, the k-block's activation sum from one more MFMA against
// ones, comes off each output row's partial sum in fp32: a third of the
// unpacking work of forming q - z in bf16.  All loads of a round are issued in
// straight-line code before their first use, slot by slot (weight blocks,
// then X fragments), so the weight stream starts at once and each wait --
// ours or the compiler's for the X registers -- leaves the younger slots in
// flight.  Slots past the wave's
// range are pointed out of bounds (they land as zeros) so every wait counts a
// fixed number of younger copies.
// ---------------------------------------------------------------------------
template <int NB, int R>
struct DecodeLds {
  static constexpr int WSLOT = NB * 1024;  // one k-block of the wave's weight rows
  static constexpr int WRING = R * WSLOT;
  static constexpr int SZ = 2048;           // scales (1 KB) then zero points (1 KB)
  static constexpr int WAVE = WRING + SZ;
  static constexpr int CHUNKS = 2 * NB;     // 8-row chunks per slot: 16 bytes of scales, 4 of zero points
  static constexpr int SROW = NB * 32;      // scale bytes per slot
  static constexpr int ZROW = NB * 8;       // zero-point bytes per slot
  static_assert(R * CHUNKS <= 64, "one copy instruction carries a round's scale rows");
  static_assert(R * SROW <= 1024 && R * ZROW <= 1024, "a round's scale and zero rows fit their 1 KB");
};

// weight rows n_base .. n_base + 16 NB of Y = X W^T for the a.M <= 16 MT
// tokens of X (MT 16-token tiles share each k-block's weights); `lds` holds
// KW * DecodeLds<NB, R>::WAVE bytes
template <int DT, int NB, int KW, int R, int MT = 1>
__device__ __forceinline__ void decode_body(const W4Launch& a, int n_base, char* lds) {
  static_assert(KW * NB * MT * 64 * 16 <= KW * DecodeLds<NB, R>::WAVE, "the reduction reuses the rings");
  using L = DecodeLds<NB, R>;
  // vector-memory operations one ring slot issues, in this order: NB weight
  // copies (direct to LDS, not tracked by the compiler), then 4 MT X loads.
  // The wait before slot s leaves exactly the younger slots' operations in
  // flight, so every slot must issue exactly this many, whatever its range.
  constexpr int SLOT_VM = NB + 4 * MT;
  static_assert((R - 1) * SLOT_VM < 64, "the younger slots fit the vmcnt counter");
  const int lane = threadIdx.x & 63, wave = wave_id();
  char* wring = lds + wave * L::WAVE;
  char* szb = wring + L::WRING;
  const uint32_t N = a.N;
  const int kblocks = a.K / 128;
  const int per = (kblocks + KW - 1) / KW;
  const int kb0 = wave * per;
  const int kb1 = kb0 + per < kblocks ? kb0 + per : kblocks;
  const int rounds = (per + R - 1) / R;

  const rsrc_t rw = make_rsrc(a.w, (uint32_t)((int64_t)a.N * a.K / 2));
  const rsrc_t rx = make_rsrc(a.X, (uint32_t)((int64_t)a.M * a.ldx * 2));
  const rsrc_t rs = make_rsrc(a.scales, a.s_bytes);
  const rsrc_t rz = make_rsrc(a.zeros, a.z_bytes);
  const uint32_t sor2 = a.sor * 0x00010001u;
  const uint32_t r = lane & 15, h = lane >> 4;
  // fp16 pair (1024, 1024): 1024 + q for a nibble q in the low mantissa
  // bits; bf16 pair (128, 128): 128 + q
  uint32_t magic = DT == DT_F16 ? 0x64006400u : 0x43004300u;
  asm volatile("" : "+v"(magic));

  f32x4 acc[NB][MT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = f32x4{0, 0, 0, 0};

  for (int rd = 0; rd < rounds; ++rd) {
    const int base = kb0 + rd * R;
    u32x4 x[R][MT][4];
    {
      // scales: lane -> slot lane / CHUNKS, 8-row chunk lane % CHUNKS (16
      // bytes); zero points: the same slot and chunk, 4 bytes
      const int s = lane / L::CHUNKS, c = lane % L::CHUNKS, ks = base + s;
      const uint32_t gs = (uint32_t)(ks * 128) / (uint32_t)a.group;
      const bool ok = s < R && ks < kb1 && n_base + 8 * c < (int)N;
      dma16(rs, ok ? (gs * N + n_base + 8 * c) * 2u : OOB, szb);
      dma4(rz, ok ? gs * (N / 2) + n_base / 2 + 4 * c : OOB, szb + 1024);
    }
#pragma unroll
    for (int s = 0; s < R; ++s) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t blk = n_base / 16 + nb;
        dma16(rw, base + s < kb1 && blk * 16 < N ? (blk * (uint32_t)kblocks + base + s) * 1024u + lane * 16u : OOB,
              wring + s * L::WSLOT + nb * 1024);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint32_t tok = mt * 16 + r;
        const bool ok = base + s < kb1 && (int)tok < a.M;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          x[s][mt][j] = buf_load16(rx, ok ? (tok * (uint32_t)a.ldx + (base + s) * 128 + j * 32 + h * 8) * 2u : OOB);
      }
      // the waits below count in issue order: no load of a later slot (a
      // plain load the compiler could hoist) may go out before this slot's
      // weight copies (which it does not track)
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int s = 0; s < R; ++s) {
      // weight blocks and X fragments of slot s (and everything older)
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_le_n<(R - 1) * SLOT_VM>((R - 1 - s) * SLOT_VM);
      if (base + s < kb1) {
        // bf16: the k-block's activation sum of each token, by the matrix
        // instruction against a fragment of ones (every output row the same)
        f32x4 sx[MT];
        if constexpr (DT == DT_BF16) {
          const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            sx[mt] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 4; ++j) sx[mt] = mfma16<DT>(ones, x[s][mt][j], sx[mt]);
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          // the MFMA takes the exact integers q - z of weight row `row`; the
          // group scale of each output row multiplies the fp32 partial sum
          const u32x4 wq = *(const u32x4*)(wring + s * L::WSLOT + nb * 1024 + lane * 16) ^ a.wxor;
          f32x4 part[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) part[mt] = f32x4{0, 0, 0, 0};
          if constexpr (DT == DT_F16) {
            const int row = nb * 16 + r;
            const uint32_t zbits =
                ((*(const uint8_t*)(szb + 1024 + s * L::ZROW + row / 2) >> ((row & 1) * 4)) & 15u) ^ a.zxor;
            const f16x2 zz = zero_pair(zbits);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x4 wf = unpack8_minus_zero(wq[j], zz, magic);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) part[mt] = mfma16<DT>(wf, x[s][mt][j], part[mt]);
            }
          } else {
            // sum_k (q - z) x = sum_k (128 + q) x - (128 + z) sum_k x: the
            // biased integers go in exactly, the bias comes off each output
            // row (rows nb * 16 + 4 h + {0..3} of this lane) in fp32
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x4 wf = unpack8_biased_bf16(wq[j], magic);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) part[mt] = mfma16<DT>(wf, x[s][mt][j], part[mt]);
            }
            const uint32_t z4 = *(const uint16_t*)(szb + 1024 + s * L::ZROW + (nb * 16 + 4 * h) / 2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float zb = (float)(128u + (((z4 >> (4 * i)) & 15u) ^ a.zxor));
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) part[mt][i] = __builtin_fmaf(-zb, sx[mt][i], part[mt][i]);
            }
          }
          // output rows of this lane: nb * 16 + 4 h + {0..3}
          const u32x2 sc = *(const u32x2*)(szb + s * L::SROW + (nb * 16 + 4 * h) * 2) | sor2;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float si = from_bits<DT>((sc[i / 2] >> (16 * (i % 2))) & 0xffffu);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[nb][mt][i] = __builtin_fmaf(si, part[mt][i], acc[nb][mt][i]);
          }
        }
      }
    }
  }
  __syncthreads();  // every wave is done with its ring: reuse it for the reduction

  f32x4* red = (f32x4*)lds;  // [KW][NB][MT][64]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[((wave * NB + nb) * MT + mt) * 64 + lane] = acc[nb][mt];
  __syncthreads();
  // lane quad q of block nb, tile mt: rows n_base + 16 nb + 4 (q / 16) + {0..3}, token 16 mt + q % 16
  for (int idx = threadIdx.x; idx < NB * MT * 64; idx += 64 * KW) {
    f32x4 t = red[idx];
#pragma unroll
    for (int w = 1; w < KW; ++w) t += red[w * NB * MT * 64 + idx];
    const int nb = idx / (MT * 64), mt = (idx / 64) % MT, q = idx % 64;
    const int n = n_base + nb * 16 + 4 * (q / 16), tok = mt * 16 + q % 16;
    if (tok < a.M && n < a.N)
      *(gu32x2*)(a.Y + (int64_t)tok * a.ldy + n) = u32x2{pack2<DT>(t[0], t[1]), pack2<DT>(t[2], t[3])};
  }
}

template <int DT, int NB, int KW, int R, int MT = 1>
__global__ __launch_bounds__(64 * KW) void k_w4a16_decode(W4Launch a) {
  __shared__ __attribute__((aligned(16))) char lds[KW * DecodeLds<NB, R>::WAVE];
  decode_body<DT, NB, KW, R, MT>(a, blockIdx.x * NB * 16, lds);
}

// ---------------------------------------------------------------------------
// Large-M kernel: the dense tiles' fragments, multiply stage and epilogue,
// X as the A operand, the prepacked weight (dequantised on its way into LDS)
// as the column-major B operand.
//
// Mainloop of the tiled kernel, prefetch distance D: D + 1 X stages
// (direct-to-LDS copies), two weight stages (dequantised from registers into
// LDS) and D register sets of raw weights.  While k-tile kt is multiplied,
// the X copies and weight loads of kt + D are issued and those of kt + 1 ..
// kt + D - 1 are still landing, so every load has D stage times to arrive;
// the end of step kt waits for k-tile kt + 1 only (the loads of kt + 2 ..
// kt + D are the younger ones), dequantises its weights into the free weight
// stage and publishes both.  Every step issues the same loads (past the last
// k-tile they re-read valid data or land as zeros and are never multiplied),
// so the wait counts are fixed.  D = 2 keeps two workgroups per CU.  (Deeper
// rings, D = 4 and 6 at one workgroup per CU, measured the same at M = 128:
// the k-steps there do not wait on load latency.)
// ---------------------------------------------------------------------------
template <class Cfg, int D>
struct W4Ring {
  static constexpr int A_STAGES = D + 1, B_STAGES = 2;
  static constexpr int BYTES = A_STAGES * Cfg::A_BYTES + B_STAGES * Cfg::B_BYTES;
  static constexpr int WGS = D == 2 ? Cfg::WGS_PER_CU : 1;  // workgroups per CU
  static_assert(D >= 2 && BYTES * WGS <= 160 * 1024, "LDS budget");
  __device__ static __forceinline__ char* a(char* lds, int s) { return lds + s * Cfg::A_BYTES; }
  __device__ static __forceinline__ char* b(char* lds, int s) {
    return lds + A_STAGES * Cfg::A_BYTES + s * Cfg::B_BYTES;
  }
};

template <int J, int D, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (J < D) {
    f(std::integral_constant<int, J>{});
    static_for<J + 1, D>(f);
  }
}

// one k-tile: weights of kt + D into `rl`, multiply kt, then publish kt + 1
// (X already copied, weights from `rs`).  With exact integer weights (bf16)
// the multiply accumulates into `part`, which the last k-tile of each scale
// group folds into `acc` with the group's scales `sc`; those are loaded one
// step ahead, at the start of the step before the fold.
template <class Cfg, int DT, int D, class ALd, class BLd>
__device__ __forceinline__ void w4_step(char* lds, const ALd& al, const BLd& bl, int kt, int nk,
                                        typename BLd::Regs& rl, const typename BLd::Regs& rs, const FragAddr<Cfg>& ad,
                                        f32x16 (&acc)[Cfg::TM][Cfg::TN], f32x16 (&part)[Cfg::TM][Cfg::TN],
                                        u32x2 (&sc)[Cfg::TN][4], frag_t<Cfg> (&fa)[2][Cfg::TM],
                                        frag_t<Cfg> (&fb)[2][Cfg::TN]) {
  using Ring = W4Ring<Cfg, D>;
  constexpr int YOUNG = ALd::P + BLd::LOADS;  // one k-tile's copies and loads
  static_assert((D - 1) * YOUNG < 64, "the k-tiles left in flight fit the vmcnt counter");
  // The wait below counts outstanding loads in issue order, and the compiler
  // does not track the direct-to-LDS copies: the fences keep every load and
  // copy of k-tile kt + D between the previous step's wait and this one's.
  // Scale loads for the next step's fold go out first, before those of
  // k-tile kt + D: the wait then only waits longer (it still leaves at most
  // the (D - 1) YOUNG youngest in flight), and the next step's wait covers
  // them, so the fold itself never waits on a load.
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (BLd::EXACT) {
    if (kt + 1 < nk && bl.group_ends(kt + 1, nk)) bl.fold_scales(kt + 1, sc);
  }
  bl.load(kt + D, rl);
  const char* ca = Ring::a(lds, kt % (D + 1));
  const char* cb = Ring::b(lds, kt & 1);
  read_frags<Cfg>(ad, ca, cb, 0, fa[0], fb[0]);
  multiply_stage<Cfg, DT, false, 2>(ad, ca, cb, ca, cb, BLd::EXACT ? part : acc, fa, fb, al, kt + D,
                                    Ring::a(lds, (kt + D) % (D + 1)), bl, 0, nullptr);
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_le<(D - 1) * YOUNG>();
  if (kt + 1 < nk) bl.store(Ring::b(lds, (kt + 1) & 1), rs);
  if constexpr (BLd::EXACT) {
    if (bl.group_ends(kt, nk)) bl.fold(acc, part, sc);
  }
  wait_lgkm();
  __builtin_amdgcn_s_barrier();
}

template <class Cfg, int DT, int D, class ALd, class BLd>
__device__ __forceinline__ void mainloop_w4(char* lds, const ALd& al, const BLd& bl, int nk,
                                            f32x16 (&acc)[Cfg::TM][Cfg::TN]) {
  using Ring = W4Ring<Cfg, D>;
  static_assert(ALd::kDMA && !BLd::kDMA, "X by direct copies, weights through registers");
  constexpr int YOUNG = ALd::P + BLd::LOADS;
  f32x16 part[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      acc[i][j] = f32x16{};
      part[i][j] = f32x16{};
    }
  // the previous tile's epilogue may still be reading the stages
  __builtin_amdgcn_s_barrier();
  if (nk <= 0) return;
  frag_t<Cfg> fa[2][Cfg::TM], fb[2][Cfg::TN];
  FragAddr<Cfg> ad;
  ad.init();
  typename BLd::Regs r[D];
  u32x2 sc[Cfg::TN][4];  // scales of the next fold (exact integer weights)
  // prologue: k-tiles 0 .. D - 1 in flight; 0 landed and published.  The
  // wait leaves k-tiles 1 .. D - 1 in flight, so all of k-tile 0's loads must
  // be issued before any of theirs (and so on): the compiler may otherwise
  // hoist a weight load of a later k-tile (a plain load into registers) above
  // a copy of an earlier one (which it does not track), and the wait would
  // then release before that copy has landed.
  static_for<0, D>([&](auto j) {
    bl.load(j, r[j]);
    al.issue(j, Ring::a(lds, j));
    __builtin_amdgcn_sched_barrier(0);
  });
  wait_vm_le<(D - 1) * YOUNG>();
  bl.store(Ring::b(lds, 0), r[0]);
  wait_lgkm();
  __builtin_amdgcn_s_barrier();
  // D k-tiles per trip so each register set keeps a fixed name: step kt
  // loads k-tile kt + D into set kt % D and publishes kt + 1 from set
  // (kt + 1) % D
  for (int kt = 0; kt < nk; kt += D) {
    static_for<0, D>([&](auto j) {
      if (kt + j < nk)
        w4_step<Cfg, DT, D>(lds, al, bl, kt + j, nk, r[j], r[(j + 1) % D], ad, acc, part, sc, fa, fb);
    });
  }
  // copies and loads past the last k-tile are still landing: drain them
  // before anyone reuses the stages
  wait_vm_le<0>();
  __builtin_amdgcn_s_barrier();
}

// ---------------------------------------------------------------------------
// Row tiles per raster band of the tiled launches: an XCD's run of
// consecutive work items covers at most this many X row tiles
constexpr int kW4Band = 4;
constexpr int kW4GroupBand = 2;  // the grouped launch, per expert

// One output tile per work item, the whole K, rounded into Y by the
// epilogue: used only where the tiles alone cover every CU, so it never
// splits over K.
template <class Cfg, int DT, int D>
__global__ __launch_bounds__(Cfg::THREADS, (W4Ring<Cfg, D>::WGS)) void k_w4a16_tiled(W4Launch a, int tiles_m,
                                                                                  int total_work) {
  __shared__ __attribute__((aligned(16))) char lds[W4Ring<Cfg, D>::BYTES];
  const int G = gridDim.x;
  const W4Geom g{a.w, a.scales, a.zeros, a.N, a.K, a.group, a.s_bytes, a.z_bytes, a.sor, a.wxor, a.zxor};
  for (int base = 0; base < total_work; base += G) {
    const int tile = base + remap_slot(blockIdx.x, G);
    if (tile >= total_work) break;
    int mi, ni;
    raster(tile, tiles_m, total_work / tiles_m, mi, ni, kW4Band);
    Tile t;
    t.M = a.M;
    t.N = a.N;
    t.K = a.K;
    t.m0 = mi * Cfg::BM;
    t.n0 = ni * Cfg::BN;
    t.C = nullptr;
    t.ldc = 0;
    t.D = a.Y;
    t.ldd = a.ldy;
    DenseLoader<Cfg, Cfg::BM> al;
    W4Loader<Cfg, Cfg::BN, DT> bl;
    al.init(a.X, a.ldx, t.m0, t.M, a.K);
    bl.init(g, t.n0, 0);
    f32x16 acc[Cfg::TM][Cfg::TN];
    mainloop_w4<Cfg, DT, D>(lds, al, bl, a.K / Cfg::BK, acc);
    store_tile<Cfg, DT>(t, acc, 1.0f, 0.0f, lds);
  }
}

// ---------------------------------------------------------------------------
// Register-sourced kernel (the page's design: the narrow weight is the
// operand that lives in registers, dequantised right before the multiply).
// The prepacked 16-row block is laid out so that lane L's 16 bytes are its
// v_mfma_f32_16x16x32 A fragments (row L % 16, k-group L / 16) for the four
// 32-k steps of the 128-k block, so a wave loads its own weight words
// straight into VGPRs, dequantises them there, and multiplies them against
// X fragments (token L % 16, the same k-group) that the workgroup's waves
// share through an LDS ring of X k-tiles.  No weight tile goes through LDS,
// so nothing waits on a dequantised tile being written and published.
//
// Workgroup: 4 waves, 16 MT tokens (an X tile of 16 MT rows x 64 k per
// stage), wave w owning weight blocks WB w .. WB w + WB - 1 of its 64 WB-row
// slice.  Pipeline distance D: the X copies and weight loads of k-tile
// kt + D go out at the start of step kt, into the X stage and register set
// of k-tile kt - 1 (both free after the previous step's barrier); the end
// of step kt waits for k-tile kt + 1 (the loads of kt + 2 .. kt + D stay in
// flight) and a barrier publishes its X stage.  Accumulator lane l, element
// i: weight row 4 (l / 16) + i of block b, token 16 mt + l % 16.
// bf16: exact q - z into a per-group fp32 partial, folded with the scales of
// the lane's four rows at the end of each scale group (or k-range).
// ---------------------------------------------------------------------------
using RsXCfg = TileCfg<128, 128, 2, 2, 64, 2>;  // X tile layout: 4 waves, 64-k rows of 128 bytes

template <int WB>
struct RsRegs {
  u32x2 w[WB];   // words 2 (kt % 2) + {0, 1} of each block's lane entry
  uint32_t z[WB];  // zero point of row L % 16 (after the mode fix-up)
  u32x2 s[WB];   // fp16: scale of row L % 16 in s[b][0]; bf16: scales of rows 4 (L / 16) + {0..3}
};

template <int DT, int WB>
struct RsWeights {
  static constexpr bool EXACT = DT == DT_BF16;
  static constexpr int LOADS = 3 * WB;  // weight words, zero point, scales per block
  rsrc_t rw, rs, rz;
  uint32_t N, group, kt0, sor, wxor, zxor;
  // lane offsets of each block's weight entry, zero point and scales (OOB for
  // a block past N); the k-tile's offsets are wave-uniform and go in soffset
  uint32_t vw[WB], vz[WB], vs[WB];
  __device__ __forceinline__ void init(const W4Launch& a, int n_base, int kt_first) {
    rw = make_rsrc(a.w, (uint32_t)((int64_t)a.N * a.K / 2));
    rs = make_rsrc(a.scales, a.s_bytes);
    rz = make_rsrc(a.zeros, a.z_bytes);
    N = a.N;
    group = a.group;
    kt0 = kt_first;
    sor = a.sor;
    wxor = a.wxor;
    zxor = a.zxor;
    const uint32_t kblocks = a.K / 128, blk0 = n_base / 16 + wave_id() * WB, lane = threadIdx.x & 63;
#pragma unroll
    for (int b = 0; b < WB; ++b) {
      const uint32_t blk = blk0 + b, n = blk * 16 + lane % 16;
      const bool ok = blk * 16 < N;
      vw[b] = ok ? blk * kblocks * 1024u + lane * 16u : OOB;
      vz[b] = ok ? n / 2 : OOB;
      vs[b] = ok ? (EXACT ? (blk * 16 + 4 * (lane / 16)) * 2u : n * 2u) : OOB;
    }
  }
  __device__ __forceinline__ void load(int kt_local, RsRegs<WB>& r) const {
    const uint32_t kt = kt_local + kt0;
    const uint32_t grp = (kt * 64) / group;
    const uint32_t sw = (kt / 2) * 1024u + (kt & 1) * 8u, sz = grp * (N / 2), ss = grp * N * 2u;
#pragma unroll
    for (int b = 0; b < WB; ++b) {
      r.w[b] = buf_load8s(rw, vw[b], sw);
      r.z[b] = buf_load1s(rz, vz[b], sz);
      if constexpr (EXACT)
        r.s[b] = buf_load8s(rs, vs[b], ss);
      else
        r.s[b] = u32x2{buf_load2s(rs, vs[b], ss), 0u};
    }
  }
  __device__ __forceinline__ bool group_ends(int kt_local, int nk) const {
    return kt_local + 1 == nk || (((kt_local + kt0 + 1) * 64) % group) == 0;
  }
};

template <int DT, int WB, int MT, int D>
struct RsRing {
  static constexpr int XSTAGE = MT * 16 * 128;  // X tile bytes per k-tile
  static constexpr int BYTES = (D + 1) * XSTAGE;
  static_assert(MT * 16 == RsXCfg::BM, "the X loader moves 128-row tiles");
  static_assert(2 * BYTES <= 160 * 1024, "two workgroups per CU");
};

// GK: k-tiles per scale group when the caller knows it (0: found per k-tile).
// With GK fixed, the group boundaries fall on fixed steps of the unrolled
// loop: a group's first multiply starts its partial from zero and its last
// k-tile folds the partial in, with no per-step test and no reset.
// MT: 16-token tiles multiplied (the X stages always hold the loader's 128
// rows; a shortened last tile multiplies only the first MT of them).
template <int DT, int WB, int MT, int D, int GK = 0>
__device__ __forceinline__ void rs_mainloop(char* lds, const DenseLoader<RsXCfg, RsXCfg::BM>& xl,
                                            const RsWeights<DT, WB>& wl, int nk, f32x4 (&acc)[WB][MT]) {
  using Ring = RsRing<DT, WB, RsXCfg::BM / 16, D>;
  static_assert(MT >= 1 && MT <= RsXCfg::BM / 16, "the multiplied tiles lie in the X stage");
  constexpr bool EXACT = DT == DT_BF16;
  static_assert(GK == 0 || (EXACT && (D + 1) % GK == 0), "fixed groups align with the unrolled steps");
  constexpr int YOUNG = RsXCfg::NW == 4 ? DenseLoader<RsXCfg, RsXCfg::BM>::P + RsWeights<DT, WB>::LOADS : 0;
  static_assert((D - 1) * YOUNG < 64, "the k-tiles left in flight fit the vmcnt counter");
  const int lane = threadIdx.x & 63;
  f32x4 part[WB][MT];
#pragma unroll
  for (int b = 0; b < WB; ++b)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[b][mt] = f32x4{0, 0, 0, 0};
      part[b][mt] = f32x4{0, 0, 0, 0};
    }
  __builtin_amdgcn_s_barrier();  // the previous item's waves are done with the ring
  if (nk <= 0) return;
  // X fragment of token row (16 mt + lane % 16), 32-k step j: chunk 4 j + lane / 16
  uint32_t xoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) xoff[j] = (uint32_t)RsXCfg::off(lane % 16, 4 * j + lane / 16);
  uint32_t magic = 0x64006400u;  // in a VGPR: the conversion's mask-and-OR is one instruction
  asm volatile("" : "+v"(magic));
  RsRegs<WB> r[D + 1];
  // prologue: k-tiles 0 .. D - 1 in flight, each one's loads before the
  // next one's (the waits count in issue order), k-tile 0 landed and published
  static_for<0, D>([&](auto j) {
    wl.load(j, r[j]);
    xl.issue(j, lds + j * Ring::XSTAGE);
    __builtin_amdgcn_sched_barrier(0);
  });
  wait_vm_le<(D - 1) * YOUNG>();
  __builtin_amdgcn_s_barrier();
  for (int kt0 = 0; kt0 < nk; kt0 += D + 1) {
    static_for<0, D + 1>([&](auto jj) {
      constexpr int J = decltype(jj)::value;
      const int kt = kt0 + J;
      if (kt < nk) {
        // the loads of k-tile kt + D: into the register set and X stage of kt - 1
        __builtin_amdgcn_sched_barrier(0);
        wl.load(kt + D, r[(J + D) % (D + 1)]);
        xl.issue(kt + D, lds + ((kt + D) % (D + 1)) * Ring::XSTAGE);
        __builtin_amdgcn_sched_barrier(0);
        const char* xs = lds + (kt % (D + 1)) * Ring::XSTAGE;
        // this step's weights, loaded D steps ago: passed through an empty asm
        // here so that no arithmetic on them is scheduled next to their loads
        // (where the compiler would wait for loads just issued)
        RsRegs<WB> cur = r[J];
#pragma unroll
        for (int b = 0; b < WB; ++b) asm volatile("" : "+v"(cur.w[b]), "+v"(cur.z[b]), "+v"(cur.s[b]));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 xf[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) xf[mt] = *(const u32x4*)(xs + xoff[j] + mt * 16 * RsXCfg::ROWB);
#pragma unroll
          for (int b = 0; b < WB; ++b) {
            const uint32_t wq = cur.w[b][j] ^ wl.wxor;
            const uint32_t z = ((cur.z[b] >> ((lane & 1) * 4)) & 15u) ^ wl.zxor;
            u32x4 wf;
            if constexpr (EXACT)
              wf = exact8_bf16(wq, (float)z);
            else
              wf = dequant8(wq, z, scale_pair((cur.s[b][0] & 0xffffu) | wl.sor), magic);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              if constexpr (EXACT) {
                if (GK != 0 && J % (GK == 0 ? 1 : GK) == 0 && j == 0)
                  part[b][mt] = mfma16<DT>(wf, xf[mt], f32x4{0, 0, 0, 0});
                else
                  part[b][mt] = mfma16<DT>(wf, xf[mt], part[b][mt]);
              } else {
                acc[b][mt] = mfma16<DT>(wf, xf[mt], acc[b][mt]);
              }
            }
          }
        }
        if constexpr (EXACT && GK != 0) {
          if constexpr (J % (GK == 0 ? 1 : GK) == (GK == 0 ? 0 : GK - 1)) {
#pragma unroll
            for (int b = 0; b < WB; ++b)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float si = from_bits<DT_BF16>(((cur.s[b][i / 2] >> (16 * (i % 2))) & 0xffffu) | wl.sor);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[b][mt][i] = __builtin_fmaf(si, part[b][mt][i], acc[b][mt][i]);
              }
          }
        } else if constexpr (EXACT) {
          if (wl.group_ends(kt, nk)) {
#pragma unroll
            for (int b = 0; b < WB; ++b)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float si = from_bits<DT_BF16>(((cur.s[b][i / 2] >> (16 * (i % 2))) & 0xffffu) | wl.sor);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                  acc[b][mt][i] = __builtin_fmaf(si, part[b][mt][i], acc[b][mt][i]);
                  part[b][mt][i] = 0.0f;
                }
              }
          }
        }
        // k-tile kt + 1 landed (kt + 2 .. kt + D stay in flight), then published
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_le<(D - 1) * YOUNG>();
        __builtin_amdgcn_s_barrier();
      }
    });
  }
  wait_vm_le<0>();  // loads past the last k-tile are still landing
  __builtin_amdgcn_s_barrier();
}

constexpr int kRsTokens = 128;  // tokens per workgroup (MT = 8)
constexpr int kRsDepth = 3;

// Results of one register-sourced tile: lane l, element i of acc[b][mt] is
// weight row n_base + 16 (WB wave + b) + 4 (l / 16) + i and token
// m0 + 16 mt + l % 16; rounded into Y.  When the call is split over K the
// fp32 partials go to the workspace in this register layout instead: work
// item (tile, s) owns kRsTileFloats floats at (tile split + s) kRsTileFloats,
// accumulator (wave, b, mt) the 1 KB run ((wave WB + b) MT + mt) 256 floats
// in, lane l's four values at 4 l -- one contiguous 1 KB store per
// accumulator; k_w4a16_rs_sum reads them back the same way.
constexpr int kRsTileFloats = kRsTokens * 128;  // one 128-token x 128-row tile
template <int DT, int WB, int MT>
__device__ __forceinline__ void rs_store(const W4Launch& a, const f32x4 (&acc)[WB][MT], int m0, int n_base,
                                         int tile, int sidx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // whole tiles only have the split partials' layout (shortened tiles come
  // from the grouped launch, which never splits)
  if constexpr (4 * WB * MT * 256 == kRsTileFloats) {
    if (a.split > 1) {
      float* pt = a.partial + ((int64_t)tile * a.split + sidx) * kRsTileFloats;
#pragma unroll
      for (int b = 0; b < WB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) *(f32x4*)(pt + ((wave * WB + b) * MT + mt) * 256 + 4 * lane) = acc[b][mt];
      return;
    }
  }
#pragma unroll
  for (int b = 0; b < WB; ++b) {
    const int n = n_base + 16 * (WB * wave + b) + 4 * (lane / 16);
    if (n >= a.N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int tok = m0 + 16 * mt + lane % 16;
      if (tok >= a.M) continue;
      const f32x4 v = acc[b][mt];
      *(gu32x2*)(a.Y + (int64_t)tok * a.ldy + n) = u32x2{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
    }
  }
}

// Y = RN(sum over s of the k-ranges' partials) in s order, from the register
// layout of rs_store: one thread per lane quad of one accumulator of one tile
template <int DT, int WB, int MT>
__global__ __launch_bounds__(256) void k_w4a16_rs_sum(const float* __restrict__ P, int split, int tiles_m, int tiles,
                                                      int M, int N, uint16_t* __restrict__ Y, int64_t ldy) {
  constexpr int QUADS = kRsTileFloats / 4;
  const int64_t total = (int64_t)tiles * QUADS;
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int tile = (int)(id / QUADS), r = (int)(id - (int64_t)tile * QUADS);
    const int lane = r % 64, mt = (r / 64) % MT, wb = r / (64 * MT);  // wb = wave WB + b
    const float* src = P + (int64_t)tile * split * kRsTileFloats + 4 * r;
    f32x4 v = *(const f32x4*)src;
    for (int sp = 1; sp < split; ++sp) v += *(const f32x4*)(src + (int64_t)sp * kRsTileFloats);
    const int tok = (tile % tiles_m) * kRsTokens + 16 * mt + lane % 16;
    const int n = (tile / tiles_m) * 128 + 16 * wb + 4 * (lane / 16);
    if (tok < M && n < N)
      *(u32x2*)(Y + (int64_t)tok * ldy + n) = u32x2{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
  }
}

// work item w = s * tiles + tile over tiles of kRsTokens tokens x 64 WB
// weight rows: k-range major, so an XCD's run of consecutive items shares
// one k-range of X in its L2 (each item's weights are its own); inside a
// k-range the tiles go in bands of kW4Band row tiles, row tile fastest, so
// the run covers a few X row tiles by a few weight panels
// GK: k-tiles per scale group, fixed at compile time (2: bf16 with 128-k
// groups, whose k-ranges are whole 128-k blocks), or 0 to test per k-tile
template <int DT, int WB, int GK>
__global__ __launch_bounds__(256, 2) void k_w4a16_rs(W4Launch a, int tiles_m, int total_work) {
  constexpr int MT = kRsTokens / 16, D = kRsDepth;
  __shared__ __attribute__((aligned(16))) char lds[RsRing<DT, WB, MT, D>::BYTES];
  const int G = gridDim.x;
  const int Ks = a.K / a.split;
  for (int base = 0; base < total_work; base += G) {
    const int work = base + remap_slot(blockIdx.x, G);
    if (work >= total_work) break;
    const int tiles = total_work / a.split;
    const int sidx = work / tiles, tile = work - sidx * tiles;
    int mi, ni;
    raster(tile, tiles_m, tiles / tiles_m, mi, ni, kW4Band);
    const int m0 = mi * kRsTokens, n_base = ni * 64 * WB;
    const int k0 = sidx * Ks;
    DenseLoader<RsXCfg, RsXCfg::BM> xl;
    xl.init(a.X + k0, a.ldx, m0, a.M, Ks);
    RsWeights<DT, WB> wl;
    wl.init(a, n_base, k0 / 64);
    f32x4 acc[WB][MT];
    rs_mainloop<DT, WB, MT, D, GK>(lds, xl, wl, Ks / 64, acc);
    rs_store<DT, WB, MT>(a, acc, m0, n_base, tile, sidx);
  }
}

using W4Cfg256 = TileCfg<256, 256, 4, 2, 64, 2>;
using W4Cfg128 = TileCfg<128, 128, 2, 2, 64, 2>;

// Tile shape of the tiled path: 256 x 256 when those tiles alone fill the
// device, else 128 x 128 (two workgroups per CU).
static bool w4_big_tiles(int M, int N, int cus) { return ((M + 255) / 256) * ((N + 255) / 256) >= cus; }

size_t w4a16_workspace_for(int M, int N, int K, int dt) {
  const int split = w4a16_split(M, N, K, dt);
  if (split <= 1) return 0;
  const size_t tiles = (size_t)((M + kRsTokens - 1) / kRsTokens) * (size_t)((N + 127) / 128);
  return (size_t)split * tiles * kRsTileFloats * sizeof(float);
}

size_t w4a16_workspace(int M, int N, int K) {
  const size_t f = w4a16_workspace_for(M, N, K, DT_F16), b = w4a16_workspace_for(M, N, K, DT_BF16);
  return f > b ? f : b;
}

int w4a16_split(int M, int N, int K, int dt) {
  if (M <= 64) return 1;  // decode / skinny kernels
  const int cus = device_cu_count();
  if (w4_big_tiles(M, N, cus)) return 1;
  const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
  // k-ranges of whole 128-k blocks, at least 8 k-tiles each, until the work
  // items cover every CU once (fp16, up to four) or fill both workgroup slots
  // of every CU (bf16, up to eight: its exact conversion and scale folds give
  // a second wave per SIMD more to overlap than the extra partials cost)
  const int most = dt == DT_BF16 ? 8 : 4, items = dt == DT_BF16 ? 2 * cus : cus;
  int split = 1;
  while (split < most && tiles * split < items && K % (128 * split * 2) == 0 && K / (split * 2) >= 512) split *= 2;
  return split;
}

template <int DT>
static hipError_t launch_w4a16_dt(const W4Launch& a, hipStream_t stream) {
  if (a.M <= 16) {
    // 16 waves, each over a sixteenth of K in rounds of four k-blocks (eight
    // waves over an eighth in one round of eight measured 4% slower)
    constexpr int NB = 2, KW = 16, R = 4;
    hipLaunchKernelGGL((k_w4a16_decode<DT, NB, KW, R>), dim3((a.N + NB * 16 - 1) / (NB * 16)), dim3(64 * KW), 0,
                       stream, a);
    return hipGetLastError();
  }
  if (a.M <= 32) {
    // both 16-row tiles through the decode body (exact integer weights);
    // the second tile's X registers leave room for a four-slot ring
    constexpr int NB = 2, KW = 8, R = 4;
    hipLaunchKernelGGL((k_w4a16_decode<DT, NB, KW, R, 2>), dim3((a.N + NB * 16 - 1) / (NB * 16)), dim3(64 * KW), 0,
                       stream, a);
    return hipGetLastError();
  }
  if (a.M <= 48) {
    // three tiles through the decode body: their X registers leave room for a
    // two-slot ring only (a three-slot ring measured 6% slower, the skinny
    // body with three tiles 5%, with four 17%)
    constexpr int NB = 2, KW = 8, R = 2;
    hipLaunchKernelGGL((k_w4a16_decode<DT, NB, KW, R, 3>), dim3((a.N + NB * 16 - 1) / (NB * 16)), dim3(64 * KW), 0,
                       stream, a);
    return hipGetLastError();
  }
  if (a.M <= 64) {
    constexpr int NB = 2, KW = 8;
    const dim3 grid((a.N + NB * 16 - 1) / (NB * 16)), block(64 * KW);
    hipLaunchKernelGGL((k_w4a16_skinny<DT, NB, KW, 4>), grid, block, 0, stream, a);
    return hipGetLastError();
  }
  const int cus = device_cu_count();
  // fp16 with enough rows for 256 x 256 tiles on every CU: the LDS-dequant
  // tiles (their B tile serves 256 rows of X); otherwise the register-sourced
  // kernel, 128 tokens x 128 weight rows per work item, k-ranges as
  // w4a16_split chose them, two workgroups per CU
  if (DT == DT_F16 && w4_big_tiles(a.M, a.N, cus)) {
    const int tiles_m = (a.M + 255) / 256;
    const int total = tiles_m * ((a.N + 255) / 256);  // w4a16_split gave 1
    int grid = (total + XCDS - 1) / XCDS * XCDS;
    if (grid > cus) grid = cus / XCDS * XCDS;
    hipLaunchKernelGGL((k_w4a16_tiled<W4Cfg256, DT_F16, 2>), dim3(grid), dim3(W4Cfg256::THREADS), 0, stream, a,
                       tiles_m, total);
  } else {
    constexpr int WB = 2, MT = kRsTokens / 16;
    const int tiles_m = (a.M + kRsTokens - 1) / kRsTokens;
    const int tiles = tiles_m * ((a.N + 64 * WB - 1) / (64 * WB));
    const int total = tiles * a.split;
    int grid = (total + XCDS - 1) / XCDS * XCDS;
    if (grid > 2 * cus) grid = 2 * cus / XCDS * XCDS;
    if (DT == DT_BF16 && a.group == 128)
      hipLaunchKernelGGL((k_w4a16_rs<DT, WB, DT == DT_BF16 ? 2 : 0>), dim3(grid), dim3(256), 0, stream, a, tiles_m,
                         total);
    else
      hipLaunchKernelGGL((k_w4a16_rs<DT, WB, 0>), dim3(grid), dim3(256), 0, stream, a, tiles_m, total);
    if (a.split > 1) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      int64_t blocks = ((int64_t)tiles * (kRsTileFloats / 4) + 255) / 256;
      if (blocks > 4 * cus) blocks = 4 * cus;
      hipLaunchKernelGGL((k_w4a16_rs_sum<DT, WB, MT>), dim3((unsigned)blocks), dim3(256), 0, stream, a.partial,
                         a.split, tiles_m, tiles, a.M, a.N, a.Y, a.ldy);
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped (mixture-of-experts) kernel: workgroup (x, g) takes weight rows
// 32 x .. 32 x + 31 of group g over that group's rows, whose count only the
// device knows, 16 rows at a time through the decode body (a decode step
// routes a few rows to each expert; a larger group re-reads its weight slice,
// from L2, once per 16 rows).  A group with no rows returns at once.  Each
// workgroup moves only 32 weight rows, so the body runs on 4 waves with a
// 4-slot ring (40 KB of LDS, at most 128 VGPRs): four workgroups share a CU
// and keep its weight stream busy while others reduce and store.
// ---------------------------------------------------------------------------
constexpr int kGroupedWaves = 4, kGroupedRing = 4;
constexpr int kGroupedLds = kGroupedWaves * DecodeLds<2, kGroupedRing>::WAVE;

template <int DT>
__global__ __launch_bounds__(64 * kGroupedWaves, 4) void k_w4a16_grouped(W4Grouped a) {
  __shared__ __attribute__((aligned(16))) char lds[kGroupedLds];
  const int g = blockIdx.y;
  const int lo = min(max(a.offsets[g], 0), a.rows);
  const int hi = min(max(a.offsets[g + 1], 0), a.rows);
  if (hi <= lo) return;
  W4Launch p = a.base;
  p.w = a.base.w + g * a.w_stride;
  p.scales = a.base.scales + g * a.s_stride;
  p.zeros = a.base.zeros + g * a.z_stride;
  const int n_base = blockIdx.x * 32;
  for (int r0 = lo; r0 < hi; r0 += 16) {
    p.M = min(16, hi - r0);
    p.X = a.base.X + (int64_t)r0 * a.base.ldx;
    p.Y = a.base.Y + (int64_t)r0 * a.base.ldy;
    decode_body<DT, 2, kGroupedWaves, kGroupedRing>(p, n_base, lds);
    __syncthreads();  // the next chunk reuses the LDS the reduction just read
  }
}

// ---------------------------------------------------------------------------
// Tiled path of the grouped call, for groups of more than kGroupedDecodeRows
// rows (a prefill-size batch routed to an expert): a persistent walk over the
// 128 x 128 output tiles of those groups through the tiled mainloop (X tiles
// by direct copies, the group's weight dequantised into LDS), so each weight
// panel is read once per 128 rows instead of once per 16.  Group sizes are
// only on the device, so every wave turns the offsets into a tile prefix held
// in its own registers (count <= kMaxOffsetGroupCount: lane l holds the first
// tile of groups 16 l .. 16 l + 15), and finds the group of tile t as the
// number of groups whose first tile is <= t, minus one (first tiles never
// decrease, and an empty group shares its successor's).  No LDS beyond the
// mainloop's, so two workgroups share a CU.  Inside a group the tiles run
// m-fastest, so the workgroups that share a weight panel run together and
// find it in L2.  A group's last row tile of at most 64 (96) rows multiplies
// only its first 4 (6) 16-token tiles (the same products per token, so the
// same bits as the whole tile; a quarter-tile body as well measured slower,
// its registers spilling).
// ---------------------------------------------------------------------------
constexpr int kGroupedDecodeRows = 32;
// calls of at most this many rows run every group through the decode body:
// the tiled launch would cost more than a group of that size saves
constexpr int kGroupedTiledMinRows = 256;
constexpr int kGroupsPerLane = kMaxOffsetGroupCount / 64;

// wave-wide sum of v (every lane gets it)
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}

template <int DT, int GK>
__global__ __launch_bounds__(256, 2) void k_w4a16_grouped_tiled(W4Grouped a) {
  constexpr int WB = 2, MT = kRsTokens / 16, D = kRsDepth, BM = kRsTokens, BN = 64 * WB;
  __shared__ __attribute__((aligned(16))) char lds[RsRing<DT, WB, MT, D>::BYTES];
  const int lane = threadIdx.x & 63;
  const int tn = (a.base.N + BN - 1) / BN;
  auto clip = [&](int v) { return min(max(v, 0), a.rows); };

  // tiles of groups 16 lane .. + 15 (0 for those the decode launch takes),
  // then their first tiles: an exclusive scan over the lanes
  int first[kGroupsPerLane];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kGroupsPerLane; ++i) {
    const int g = lane * kGroupsPerLane + i;
    int c = 0;
    if (g < a.count) {
      const int rows = clip(a.offsets[g + 1]) - clip(a.offsets[g]);
      if (rows > kGroupedDecodeRows) c = ((rows + BM - 1) / BM) * tn;
    }
    first[i] = c;  // the count for now
    sum += c;
  }
  int incl = sum;  // inclusive scan of the lane sums
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  const int total = __shfl(incl, 63, 64);
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < kGroupsPerLane; ++i) {
    const int c = first[i];
    first[i] = run;
    run += c;
  }

  const int G = gridDim.x;
  for (int base = 0; base < total; base += G) {
    const int t = base + remap_slot(blockIdx.x, G);
    if (t >= total) break;
    int below = 0;  // groups of this lane whose first tile is <= t
#pragma unroll
    for (int i = 0; i < kGroupsPerLane; ++i) below += first[i] <= t && lane * kGroupsPerLane + i < a.count;
    const int g = __builtin_amdgcn_readfirstlane(wave_sum(below) - 1);
    int mine = 0;  // first tile of group g, from the lane that holds it
#pragma unroll
    for (int i = 0; i < kGroupsPerLane; ++i) mine = (i == g % kGroupsPerLane) ? first[i] : mine;
    const int g_first = __builtin_amdgcn_readfirstlane(__shfl(mine, g / kGroupsPerLane, 64));
    const int row0 = clip(a.offsets[g]), rows = clip(a.offsets[g + 1]) - row0;
    const int tm = (rows + BM - 1) / BM;
    const int local = t - g_first;
    // the group as a plain call: its rows of X and Y, its weight, scales and zero points
    W4Launch p = a.base;
    p.M = rows;
    p.X = a.base.X + (int64_t)row0 * a.base.ldx;
    p.Y = a.base.Y + (int64_t)row0 * a.base.ldy;
    p.w = a.base.w + g * a.w_stride;
    p.scales = a.base.scales + g * a.s_stride;
    p.zeros = a.base.zeros + g * a.z_stride;
    p.split = 1;
    // bands of RASTER_M row tiles, row tile fastest: an XCD's run of
    // consecutive items shares a few X row tiles and weight panels in its L2
    int mi, ni;
    raster(local, tm, tn, mi, ni, kW4GroupBand);
    const int m0 = mi * BM, n_base = ni * BN;
    DenseLoader<RsXCfg, RsXCfg::BM> xl;
    xl.init(p.X, p.ldx, m0, rows, p.K);
    RsWeights<DT, WB> wl;
    wl.init(p, n_base, 0);
    const int left = rows - m0;
    if (left <= BM / 2) {
      // a group's last row tile: only its 16-token tiles up to the half or
      // three quarters that hold rows
      f32x4 acc[WB][MT / 2];
      rs_mainloop<DT, WB, MT / 2, D, GK>(lds, xl, wl, p.K / 64, acc);
      rs_store<DT, WB, MT / 2>(p, acc, m0, n_base, 0, 0);
    } else if (left <= 3 * BM / 4) {
      f32x4 acc[WB][3 * MT / 4];
      rs_mainloop<DT, WB, 3 * MT / 4, D, GK>(lds, xl, wl, p.K / 64, acc);
      rs_store<DT, WB, 3 * MT / 4>(p, acc, m0, n_base, 0, 0);
    } else {
      f32x4 acc[WB][MT];
      rs_mainloop<DT, WB, MT, D, GK>(lds, xl, wl, p.K / 64, acc);
      rs_store<DT, WB, MT>(p, acc, m0, n_base, 0, 0);
    }
  }
}

// Groups of 1 .. kGroupedDecodeRows rows in a call that takes the tiled
// launch: the decode body over both 16-row tiles of the group at once (each
// k-block's weights unpacked once for the two tiles; a group of at most 16
// rows leaves the second tile empty), so the weight is streamed once instead
// of once per 16 rows, with the same exact-integer arithmetic and the same
// bits as the 16-row passes.  Workgroup (x, g) takes weight rows 64 x ..
// 64 x + 63 of group g (every workgroup of a group reads all of its X, twice
// the bytes of its weight slice, so wider slices halve that traffic); every
// larger or empty group returns at once.  The second tile's X fragments
// double the registers a slot holds, so two workgroups share a CU instead of
// four; a two-slot ring (rounds of two k-blocks per wave) measured faster
// than four slots.
// ---------------------------------------------------------------------------
constexpr int kPairBlocks = 4, kPairRing = 2, kPairWgsPerCu = 2;
constexpr int kPairLds = kGroupedWaves * DecodeLds<kPairBlocks, kPairRing>::WAVE;

template <int DT>
__global__ __launch_bounds__(64 * kGroupedWaves, kPairWgsPerCu) void k_w4a16_grouped_pair(W4Grouped a) {
  __shared__ __attribute__((aligned(16))) char lds[kPairLds];
  const int g = blockIdx.y;
  const int lo = min(max(a.offsets[g], 0), a.rows);
  const int hi = min(max(a.offsets[g + 1], 0), a.rows);
  if (hi <= lo || hi - lo > kGroupedDecodeRows) return;
  W4Launch p = a.base;
  p.w = a.base.w + g * a.w_stride;
  p.scales = a.base.scales + g * a.s_stride;
  p.zeros = a.base.zeros + g * a.z_stride;
  p.M = hi - lo;
  p.X = a.base.X + (int64_t)lo * a.base.ldx;
  p.Y = a.base.Y + (int64_t)lo * a.base.ldy;
  decode_body<DT, kPairBlocks, kGroupedWaves, kPairRing, 2>(p, blockIdx.x * kPairBlocks * 16, lds);
}

hipError_t launch_w4a16_grouped(const W4Grouped& a, hipStream_t stream) {
  // a call of at most kGroupedTiledMinRows rows, or with more groups than the
  // tiled launch's table holds, runs every group through the decode launch;
  // otherwise groups of at most kGroupedDecodeRows rows take the two-tile
  // launch and larger ones the tiled launch
  if (a.count > kMaxOffsetGroupCount || a.rows <= kGroupedTiledMinRows) {
    const dim3 grid((a.base.N + 31) / 32, a.count);
    if (a.base.dt == DT_BF16)
      hipLaunchKernelGGL(k_w4a16_grouped<DT_BF16>, grid, dim3(64 * kGroupedWaves), 0, stream, a);
    else
      hipLaunchKernelGGL(k_w4a16_grouped<DT_F16>, grid, dim3(64 * kGroupedWaves), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 pgrid((a.base.N + kPairBlocks * 16 - 1) / (kPairBlocks * 16), a.count);
  if (a.base.dt == DT_BF16)
    hipLaunchKernelGGL(k_w4a16_grouped_pair<DT_BF16>, pgrid, dim3(64 * kGroupedWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(k_w4a16_grouped_pair<DT_F16>, pgrid, dim3(64 * kGroupedWaves), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int g1 = device_cu_count() * 2 / XCDS * XCDS;
  if (g1 < XCDS) g1 = XCDS;
  if (a.base.dt == DT_BF16 && a.base.group == 128)
    hipLaunchKernelGGL((k_w4a16_grouped_tiled<DT_BF16, 2>), dim3(g1), dim3(256), 0, stream, a);
  else if (a.base.dt == DT_BF16)
    hipLaunchKernelGGL((k_w4a16_grouped_tiled<DT_BF16, 0>), dim3(g1), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_w4a16_grouped_tiled<DT_F16, 0>), dim3(g1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_w4a16(const W4Launch& a, hipStream_t stream) {
  return a.dt == DT_BF16 ? launch_w4a16_dt<DT_BF16>(a, stream) : launch_w4a16_dt<DT_F16>(a, stream);
}

}  // namespace gmi
