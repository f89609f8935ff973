// Exact-operand GEMMs on the gfx950 16-bit MFMAs (v_mfma_f32_32x32x16_bf16/f16):
//   C[m, n] = tA tB * sum_k A_hat[m, k] B_hat[n, k]   ("TN", FP32 output)
//
// Every operand value is formed EXACTLY in a 16-bit format right before the
// matrix core consumes it, and the matrix core accumulates at FP32 precision
// (measured on MI355X: 2^20 + 2^-3 sums exactly at every operand position):
//   * MXFP8 (E4M3, E8M0 per 32 along K): q * 2^(s-127) has 4 significant bits and
//     stays in BF16 range, so the gfx950 scaled convert (which applies the
//     power-of-two scale exactly) yields it in BF16 -> BF16 MFMA.
//   * NVFP4 (E2M1, E4M3 per 16 along K, FP32 per row/tensor/expert): q * S has
//     at most 6 significant bits and lies in [2^-10, 2688], inside FP16's normal
//     range. S = 2^e * m (m = 1..1.875): the scaled convert applies 2^e, a packed
//     FP16 multiply applies m (exact) -> FP16 MFMA; tA tB in the epilogue.
//   * BF16 operands as they are -> BF16 MFMA.
// Definitions: microscaling blocks along the reduction dimension ("Miles
// Blackwell RL", remio.ai, section "Un Cuantizador Compartido Es el Mecanismo
// Real"); two-level NVFP4 (7minutos.es NVFP4 page, section "Que es realmente
// NVFP4"); dequantized-backward BF16 GEMMs and the BF16 shared expert (remio.ai,
// sections "La Compatibilidad ..." and "NVFP4 por token ...").
// The native scaled-FP8 MFMA is not used here: it sums each group of 8
// consecutive K products in a ~13-bit window (measured), which breaks the
// 2e-5 bound on outlier-heavy data (see gemm_mxfp8.hip).
//
// Data movement: raw operand tiles (64 K per stage: 128 B/row BF16, 64 B/row
// MXFP8, 32 B/row NVFP4) go global -> LDS with gfx950's direct loads
// (global_load_lds_dwordx4: lane l of a wave instruction lands at LDS
// base + 16 l), through a 16-byte XOR swizzle chosen so that each 16-lane
// fragment read (ds_read_b128) covers all 64 banks. NS stages (up to 4) keep
// NS - 1 tiles in flight; explicit vmcnt waits + one barrier per K tile.
// Scales (MXFP8/NVFP4) are loaded per lane straight into registers NS - 1
// tiles ahead. Out-of-range rows and K chunks read a 16-byte zero block.
//
// Operand layouts of the 32x32x16 16-bit MFMAs (measured): lane l supplies row
// l % 32 and 8 consecutive K; accumulator r of lane l is
// C[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32].
#include <type_traits>

#include "common.h"

namespace mxq {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __attribute__((aligned(16))) const uint4 kZero16 = {0u, 0u, 0u, 0u};
// E8M0 1.0 (0x7F) bytes: the scale read for MXFP8 blocks past the end of K.
__device__ __attribute__((aligned(16))) const uint4 kE8M0One16 = {0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};

namespace gx {
constexpr int BK = 64;                          // K elements per stage
template <int LD> struct RowBytes;
template <> struct RowBytes<0> { static constexpr int v = 128; };   // BF16
template <> struct RowBytes<1> { static constexpr int v = 64; };    // MXFP8
template <> struct RowBytes<2> { static constexpr int v = 32; };    // NVFP4

// Scale staging per K slice: SU direct loads of SZ bytes per row, each landing in a
// 4-byte LDS slot per row (gfx950 places 1/2/4-byte direct loads at base + 4 lane).
//   MXFP8, K % 64 == 0: one 2-byte load (32-blocks 0, 1); otherwise two 1-byte loads.
//   NVFP4, K % 64 == 0: one 4-byte load (16-blocks 0..3); otherwise two 2-byte loads.
template <int LD, bool AL> struct ScaleDma {
  static constexpr int SU = LD == 0 ? 0 : (AL ? 1 : 2);
  static constexpr int SZ = LD == 1 ? (AL ? 2 : 1) : (AL ? 4 : 2);
};

template <int LD, int BM, int BN, bool AL = true>
struct Cfg {
  static constexpr int RB = RowBytes<LD>::v;
  static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  static constexpr int SU = ScaleDma<LD, AL>::SU, SZ = ScaleDma<LD, AL>::SZ;
  static constexpr int S_BYTES = SU * (BM + BN) * 4;            // scale slots of one stage
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int NS = (4 * STAGE <= 131072) ? 4 : (3 * STAGE <= 131072 ? 3 : 2);
  static constexpr int IA = A_BYTES / 4096, IB = B_BYTES / 4096;   // 1 KiB wave instructions per wave
  static constexpr int IS = SU * (BM + BN) / 256;                  // 64-row scale loads per wave
  static constexpr int TI = BM / 64, TJ = BN / 64;                // 32x32 MFMA tiles per wave
  static constexpr int ROWS256 = 256 / RB;                         // rows per 256-byte bank span
  static constexpr int CHUNKS = RB / 16;
  static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "tile must split into 1 KiB wave loads");
};
}  // namespace gx

struct ExactProblem {
  const uint8_t* A;        // MXFP8: (rows, lda) bytes; NVFP4: (rows, lda/2); BF16: (rows, lda) x 2 bytes
  const uint8_t* sA;       // MXFP8 (rows, lda/32) E8M0; NVFP4 (rows, lda/16) E4M3
  const float* tA;         // NVFP4 decode scales (tA_mode 0 per A row, 1 tensor)
  int tA_mode;
  const int32_t* a_idx;    // optional gather of A rows
  int64_t a_rows, a_base, m_valid, lda;
  const uint8_t* B;
  const uint8_t* sB;
  const float* tB;
  int tB_mode;             // 0 per B row, 1 tensor
  int64_t n_valid, ldb;
  int64_t k_begin, k_end;  // reduction range (elements)
  float* C;
  int64_t ldc;
};

__device__ __forceinline__ int64_t exact_src_row(const ExactProblem& p, int64_t r) {
  if (!p.a_idx) return p.a_base + r;
  const int64_t ar = p.a_idx[p.a_base + r];
  return (ar >= 0 && ar < p.a_rows) ? ar : -1;
}

template <int RB>
__device__ __forceinline__ int swz(int row) {
  return (row / (256 / RB)) % (RB / 16);
}

// s_waitcnt vmcnt(n) leaving lgkmcnt / expcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct global -> LDS loads, issued through inline asm so that the compiler does
// not pair them with its own conservative waits: all ordering is explicit here
// (vmcnt waits before each stage's barrier, and a final vmcnt(0)). M0 holds the
// wave's LDS base; lane l's data lands at M0 + 16 l (4 l for 1/2/4-byte loads).
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}
__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}

template <int LD>
__device__ __forceinline__ int64_t k_bytes(int64_t k) {
  return LD == 0 ? k * 2 : LD == 1 ? k : k / 2;
}

// Per-lane description of the rows this lane streams into LDS (fixed over K).
template <int NI>
struct LoadRows {
  const uint8_t* base[NI];   // row start (or nullptr when the row is out of range)
  int lc[NI];                // logical 16-byte chunk inside the 64-K slice
};

template <int LD, int RB, int NI, int ROWS>
__device__ __forceinline__ void setup_rows(LoadRows<NI>& L, int wave, int lane, int64_t row0, int64_t valid,
                                           const uint8_t* ptr, int64_t ld_bytes, const ExactProblem* pa) {
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int pos = (wave * NI + j) * 1024 + lane * 16;     // byte in the operand tile
    const int row = pos / RB;
    const int pc = (pos % RB) / 16;
    L.lc[j] = pc ^ swz<RB>(row);
    const int64_t r = row0 + row;
    int64_t src = -1;
    if (row < ROWS && r < valid) src = pa ? exact_src_row(*pa, r) : r;
    L.base[j] = src >= 0 ? ptr + src * ld_bytes : nullptr;
  }
}

template <int LD, int NI>
__device__ __forceinline__ void issue_tile(const LoadRows<NI>& L, uint8_t* lds_op, int wave, int64_t k0,
                                           int64_t k_end) {
  constexpr int RB = gx::RowBytes<LD>::v;
  constexpr int EPC = LD == 0 ? 8 : LD == 1 ? 16 : 32;     // elements per 16-byte chunk
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int64_t k = k0 + (int64_t)L.lc[j] * EPC;
    const void* src = (L.base[j] && k < k_end) ? (const void*)(L.base[j] + k_bytes<LD>(k)) : (const void*)&kZero16;
    lds_dma16(src, lds_op + (wave * NI + j) * 1024);
  }
  (void)RB;
}

// 1/2/4-byte direct loads into 4-byte LDS slots.
template <int SZ>
__device__ __forceinline__ void lds_dma_small(const void* src, uint8_t* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  if constexpr (SZ == 1)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
  else if constexpr (SZ == 2)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}

__device__ __forceinline__ uint4 lds_read16(const uint8_t* lds_op, int row, int lchunk, int RB, int sw) {
  return *reinterpret_cast<const uint4*>(lds_op + row * RB + ((lchunk ^ sw) << 4));
}

__device__ __forceinline__ void exact_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 8 E4M3 bytes (two dwords) -> 8 BF16, each exactly q * 2^(s-127).
__device__ __forceinline__ v8bf mx_to_bf16(uint32_t w0, uint32_t w1, float sc) {
  v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
  v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
  v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
  v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
  v8bf r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1]; r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 E2M1 values (one dword, low nibble first) times the E4M3 block scale S -> 8
// FP16, exactly: convert with the power-of-two part of S, multiply by its mantissa.
__device__ __forceinline__ v8h nv_to_f16(uint32_t w, float p2, v2h m2) {
  v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 0);
  v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 1);
  v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 2);
  v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 3);
  a = a * m2; b = b * m2; c = c * m2; d = d * m2;
  v8h r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1]; r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// E4M3 code -> (2^e as float, mantissa factor in [1, 2) as packed FP16). Code 0 -> (0, 1).
__device__ __forceinline__ void e4m3_split(uint32_t code, float& p2, v2h& m2) {
  const float S = e4m3_to_f32(code & 0x7F);
  const uint32_t bits = __float_as_uint(S);
  p2 = __uint_as_float(bits & 0x7F800000u);
  const float m = S == 0.0f ? 1.0f : __uint_as_float((bits & 0x007FFFFFu) | 0x3F800000u);
  const _Float16 mh = (_Float16)m;        // exact: at most 3 mantissa bits
  m2[0] = mh;
  m2[1] = mh;
}

template <int LD, int BM, int BN, bool AL>
__device__ void exact_gemm_tile(const ExactProblem& p, int64_t m0, int64_t n0, uint8_t* lds0, uint8_t* lds1,
                                uint8_t* lds2, uint8_t* lds3) {
  using C = gx::Cfg<LD, BM, BN, AL>;
  constexpr int RB = C::RB, NS = C::NS, TI = C::TI, TJ = C::TJ;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, lr = lane & 31;

  LoadRows<C::IA> LA;
  LoadRows<C::IB> LB;
  setup_rows<LD, RB, C::IA, BM>(LA, wave, lane, m0, p.m_valid, p.A, k_bytes<LD>(p.lda), &p);
  setup_rows<LD, RB, C::IB, BN>(LB, wave, lane, n0, p.n_valid, p.B, k_bytes<LD>(p.ldb), nullptr);

  // Scale rows this lane streams into LDS: scale load instruction q (of IS per wave)
  // covers 64 rows of the concatenated [A rows | B rows] list; unit u of SU.
  constexpr int BS = LD == 1 ? 32 : 16;          // elements per scale block
  const uint8_t* s_src[C::IS > 0 ? C::IS : 1];
#pragma unroll
  for (int q = 0; q < C::IS; ++q) {
    const int item = (wave * C::IS + q) * 64 + lane;        // in [0, SU * (BM + BN))
    const int row = item % (BM + BN);
    const uint8_t* base = nullptr;
    if (row < BM) {
      const int64_t r = m0 + row;
      const int64_t src = r < p.m_valid ? exact_src_row(p, r) : -1;
      if (src >= 0) base = p.sA + src * (p.lda / BS);
    } else {
      const int64_t n = n0 + row - BM;
      if (n < p.n_valid) base = p.sB + n * (p.ldb / BS);
    }
    s_src[q] = base;
  }

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t kb = p.k_begin, ke = p.k_end;
  const int64_t nk = (ke - kb + gx::BK - 1) / gx::BK;
  constexpr int OPS = C::IA + C::IB + C::IS;     // VMEM ops per tile per wave

  // one LDS object per stage: the direct loads into one stage provably never alias
  // the fragment reads of another, so no extra waits are inserted between them
  auto stage = [&](auto SLOT) -> uint8_t* {
    constexpr int S = decltype(SLOT)::value;
    if constexpr (S == 0) return lds0;
    else if constexpr (S == 1) return lds1;
    else if constexpr (S == 2) return lds2;
    else return lds3;
  };

  auto issue = [&](int64_t t, auto SLOT) {
    uint8_t* st = stage(SLOT);
    const int64_t k0 = kb + t * gx::BK;
    if (LD != 0) {
      // scale unit u of a row starts at block k0 / BS + u * (blocks per unit)
      constexpr int BPU = (LD == 1 ? 2 : 4) / (C::SU > 0 ? C::SU : 1);   // blocks per unit
      const uint8_t* dflt = reinterpret_cast<const uint8_t*>(LD == 1 ? &kE8M0One16 : &kZero16);
#pragma unroll
      for (int q = 0; q < C::IS; ++q) {
        const int item = (wave * C::IS + q) * 64;                     // first item of this instruction
        const int u = item / (BM + BN);
        const int64_t kb0 = k0 + (int64_t)u * BPU * BS;                // first element of the unit
        const void* src = (s_src[q] && kb0 < ke) ? (const void*)(s_src[q] + kb0 / BS) : (const void*)dflt;
        lds_dma_small<C::SZ>(src, st + C::A_BYTES + C::B_BYTES + item * 4);
      }
    }
    issue_tile<LD, C::IA>(LA, st, wave, k0, ke);
    issue_tile<LD, C::IB>(LB, st + C::A_BYTES, wave, k0, ke);
  };

  // scale byte `blk` (block index inside the K slice) of LDS row `row` (B rows follow A rows)
  auto scale_at = [&](const uint8_t* st, int row, int blk) -> uint32_t {
    const uint8_t* sc = st + C::A_BYTES + C::B_BYTES;
    if (C::SU == 1) return sc[row * 4 + blk];
    constexpr int BPU = (LD == 1 ? 2 : 4) / 2;
    return sc[(blk / BPU) * (BM + BN) * 4 + row * 4 + blk % BPU];
  };

  auto compute = [&](auto SLOT) {
    const uint8_t* la = stage(SLOT);
    const uint8_t* lb = la + C::A_BYTES;
    if (LD == 0) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        v8bf fa[TI], fb[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int row = wm * (BM / 2) + i * 32 + lr;
          const uint4 w = lds_read16(la, row, 2 * s + h, RB, swz<RB>(row));
          __builtin_memcpy(&fa[i], &w, 16);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int row = wn * (BN / 2) + j * 32 + lr;
          const uint4 w = lds_read16(lb, row, 2 * s + h, RB, swz<RB>(row));
          __builtin_memcpy(&fb[j], &w, 16);
        }
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    } else if (LD == 1) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        v8bf fa0[TI], fa1[TI];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int row = wm * (BM / 2) + i * 32 + lr;
          const uint4 w = lds_read16(la, row, 2 * u + h, RB, swz<RB>(row));
          const float sc = e8m0_to_float(scale_at(la, row, u));
          fa0[i] = mx_to_bf16(w.x, w.y, sc);
          fa1[i] = mx_to_bf16(w.z, w.w, sc);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int row = wn * (BN / 2) + j * 32 + lr;
          const uint4 w = lds_read16(lb, row, 2 * u + h, RB, swz<RB>(row));
          const float sc = e8m0_to_float(scale_at(la, BM + row, u));
          const v8bf fb0 = mx_to_bf16(w.x, w.y, sc), fb1 = mx_to_bf16(w.z, w.w, sc);
#pragma unroll
          for (int i = 0; i < TI; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[i], fb0, acc[i][j], 0, 0, 0);
#pragma unroll
          for (int i = 0; i < TI; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[i], fb1, acc[i][j], 0, 0, 0);
        }
      }
    } else {
      uint4 ra[TI], rb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = wm * (BM / 2) + i * 32 + lr;
        ra[i] = lds_read16(la, row, h, RB, swz<RB>(row));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int row = wn * (BN / 2) + j * 32 + lr;
        rb[j] = lds_read16(lb, row, h, RB, swz<RB>(row));
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {      // 16-block 2h + half of the lane's chunk
        v8h fa0[TI], fa1[TI];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int row = wm * (BM / 2) + i * 32 + lr;
          float p2;
          v2h m2;
          e4m3_split(scale_at(la, row, 2 * h + half), p2, m2);
          fa0[i] = nv_to_f16(half ? ra[i].z : ra[i].x, p2, m2);
          fa1[i] = nv_to_f16(half ? ra[i].w : ra[i].y, p2, m2);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int row = wn * (BN / 2) + j * 32 + lr;
          float p2;
          v2h m2;
          e4m3_split(scale_at(la, BM + row, 2 * h + half), p2, m2);
          const v8h fb0 = nv_to_f16(half ? rb[j].z : rb[j].x, p2, m2);
          const v8h fb1 = nv_to_f16(half ? rb[j].w : rb[j].y, p2, m2);
#pragma unroll
          for (int i = 0; i < TI; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa0[i], fb0, acc[i][j], 0, 0, 0);
#pragma unroll
          for (int i = 0; i < TI; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa1[i], fb1, acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // One K tile in slot S: wait for its loads (all waves), refill the slot freed by
  // the previous tile, compute. Tiles past the end are still issued (they read the
  // zero / default blocks), so every step has exactly NS - 2 tiles in flight behind
  // tile kt and one unconditional vmcnt wait suffices.
  auto step = [&](int64_t kt, auto SLOT) {
    constexpr int S = decltype(SLOT)::value;
    wait_vmcnt<(NS - 2) * OPS>();
    __builtin_amdgcn_s_barrier();     // LDS of tile kt complete for all waves (no extra fence)
    issue(kt + NS - 1, std::integral_constant<int, (S + NS - 1) % NS>{});
    compute(SLOT);
  };

  // prologue: NS - 1 tiles in flight
  issue(0, std::integral_constant<int, 0>{});
  if constexpr (NS > 2) issue(1, std::integral_constant<int, 1>{});
  if constexpr (NS > 3) issue(2, std::integral_constant<int, 2>{});
  static_assert(NS <= 4, "prologue covers up to 4 stages");

  for (int64_t kt = 0; kt < nk;) {
    step(kt, std::integral_constant<int, 0>{});
    if (++kt >= nk) break;
    step(kt, std::integral_constant<int, 1 % NS>{});
    if (++kt >= nk) break;
    if constexpr (NS > 2) {
      step(kt, std::integral_constant<int, 2 % NS>{});
      if (++kt >= nk) break;
    }
    if constexpr (NS > 3) {
      step(kt, std::integral_constant<int, 3 % NS>{});
      ++kt;
    }
  }
  wait_vmcnt<0>();                    // no direct load may still target this workgroup's LDS
  exact_drain();

#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int64_t col = n0 + wn * (BN / 2) + j * 32 + lr;
    if (col >= p.n_valid) continue;
    float tb = 1.0f;
    if (LD == 2) tb = p.tB_mode == 0 ? p.tB[col] : p.tB[0];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * (BM / 2) + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
        if (row >= p.m_valid) continue;
        float v = acc[i][j][r];
        if (LD == 2) {
          const int64_t arow = exact_src_row(p, row);
          const float ta = arow < 0 ? 0.0f : p.tA_mode == 0 ? p.tA[arow] : p.tA[0];
          v = (v * ta) * tb;
        }
        p.C[row * p.ldc + col] = v;
      }
  }
}

// XCD-aware raster: dispatch order b round-robins over the 8 XCDs; each XCD gets a
// contiguous run of logical tiles, walked in bands of 4 tile rows so the
// workgroups resident on one XCD share operand tiles in its L2.
__device__ __forceinline__ bool exact_map_tile(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  const int64_t T = tiles_m * tiles_n;
  const int64_t T8 = (T + 7) / 8;
  const int64_t L = (b % 8) * T8 + b / 8;
  if (L >= T) return false;
  const int64_t band = L / (4 * tiles_n);
  const int64_t rows_in_band = min((int64_t)4, tiles_m - band * 4);
  const int64_t idx = L - band * 4 * tiles_n;
  tm = band * 4 + idx % rows_in_band;
  tn = idx / rows_in_band;
  return true;
}

#define MXQ_EXACT_LDS(C)                                                              \
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::STAGE];                    \
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::STAGE];                    \
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[C::NS > 2 ? C::STAGE : 16];   \
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[C::NS > 3 ? C::STAGE : 16];

template <int LD, int BM, int BN, bool SU16>
__global__ void __launch_bounds__(256, 1) exact_dense_kernel(ExactProblem p, int64_t tiles_m, int64_t tiles_n) {
  using C = gx::Cfg<LD, BM, BN, SU16>;
  MXQ_EXACT_LDS(C)
  int64_t tm, tn;
  if (!exact_map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  exact_gemm_tile<LD, BM, BN, SU16>(p, tm * BM, tn * BN, lds0, lds1, lds2, lds3);
}

// Grouped: tile_prefix[g] = first tile of group g.
//   vary_k = 0: group g covers slots [off[g], off[g+1]), B_g = expert g of a stacked B;
//   vary_k = 1: group g reduces over k in [off[g], off[g+1]) into C_g = C + g*M*N.
template <int LD, int BM, int BN, bool SU16>
__global__ void __launch_bounds__(256, 1)
exact_grouped_kernel(ExactProblem base, const int64_t* __restrict__ offsets, const int64_t* __restrict__ tile_prefix,
                     int64_t groups, int vary_k, int64_t M, int64_t N, int64_t tiles_n) {
  using C = gx::Cfg<LD, BM, BN, SU16>;
  MXQ_EXACT_LDS(C)
  const int64_t tile = blockIdx.x;
  if (tile >= tile_prefix[groups]) return;
  int64_t lo = 0, hi = groups - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (tile_prefix[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int64_t g = lo;
  const int64_t local = tile - tile_prefix[g];
  const int64_t tm = local / tiles_n, tn = local % tiles_n;
  ExactProblem p = base;
  if (!vary_k) {
    p.a_base = offsets[g];
    p.m_valid = offsets[g + 1] - offsets[g];
    const int64_t b_elems = g * N * base.ldb;
    p.B = base.B + k_bytes<LD>(b_elems);
    if (LD == 1) p.sB = base.sB + b_elems / 32;
    if (LD == 2) {
      p.sB = base.sB + b_elems / 16;
      if (base.tB_mode == 2) { p.tB = base.tB + g; p.tB_mode = 1; }
      else p.tB = base.tB + g * N;
    }
    p.C = base.C + offsets[g] * base.ldc;
  } else {
    p.k_begin = offsets[g];
    p.k_end = offsets[g + 1];
    p.C = base.C + g * M * N;
  }
  exact_gemm_tile<LD, BM, BN, SU16>(p, tm * BM, tn * BN, lds0, lds1, lds2, lds3);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int pick_tile(int ld, int64_t M, int64_t N) {
  // 256 x 256 unless that leaves most of the 256 CUs idle; then 128 x 128.
  // NVFP4 always 128 x 128: its 256-wide variant does not fit the register file.
  if (ld == 2) return 128;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  return t256 >= 192 ? 256 : 128;
}

template <int LD, int BT, bool SU16>
static void launch_dense_t(const ExactProblem& p, int64_t M, int64_t N, hipStream_t st) {
  const int64_t tm = (M + BT - 1) / BT, tn = (N + BT - 1) / BT;
  const int64_t blocks = (tm * tn + 7) / 8 * 8;
  hipLaunchKernelGGL((exact_dense_kernel<LD, BT, BT, SU16>), dim3((unsigned)blocks), dim3(256), 0, st, p, tm, tn);
}

template <int LD>
static void launch_dense_ld(const ExactProblem& p, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const bool su16 = LD == 0 || (K % 64 == 0);      // 64-aligned scale rows and slices
  const int bt = pick_tile(LD, M, N);
  if constexpr (LD != 2) {
    if (bt == 256) {
      if (su16) launch_dense_t<LD, 256, true>(p, M, N, st); else launch_dense_t<LD, 256, false>(p, M, N, st);
      return;
    }
  }
  if (su16) launch_dense_t<LD, 128, true>(p, M, N, st); else launch_dense_t<LD, 128, false>(p, M, N, st);
}

hipError_t launch_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* A, const void* sA, const float* tA,
                       int tA_mode, const void* B, const void* sB, const float* tB, int tB_mode, float* C,
                       int64_t ldc, hipStream_t st) {
  ExactProblem p;
  p.A = (const uint8_t*)A; p.sA = (const uint8_t*)sA; p.tA = tA; p.tA_mode = tA_mode;
  p.a_idx = nullptr; p.a_rows = M; p.a_base = 0; p.m_valid = M; p.lda = K;
  p.B = (const uint8_t*)B; p.sB = (const uint8_t*)sB; p.tB = tB; p.tB_mode = tB_mode; p.n_valid = N; p.ldb = K;
  p.k_begin = 0; p.k_end = K; p.C = C; p.ldc = ldc;
  if (fmt == 1) launch_dense_ld<1>(p, M, N, K, st);
  else if (fmt == 2) launch_dense_ld<2>(p, M, N, K, st);
  else launch_dense_ld<0>(p, M, N, K, st);
  return hipGetLastError();
}

__global__ void tile_prefix_kernel(const int64_t* __restrict__ offsets, int64_t groups, int64_t total, int vary_k,
                                   int64_t align, int64_t bm, int64_t tiles_m_fixed, int64_t tiles_n,
                                   int64_t* __restrict__ prefix) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  // The offsets must describe a partition of [0, total) (aligned to `align` when
  // they split the reduction axis); otherwise no tile runs.
  bool ok = offsets[0] == 0 && offsets[groups] == total;
  for (int64_t g = 0; g < groups && ok; ++g) {
    ok = offsets[g + 1] >= offsets[g];
    if (vary_k) ok = ok && (offsets[g] % align == 0);
  }
  int64_t acc = 0;
  for (int64_t g = 0; g < groups; ++g) {
    prefix[g] = ok ? acc : 0;
    const int64_t mg = vary_k ? tiles_m_fixed : (offsets[g + 1] - offsets[g] + bm - 1) / bm;
    if (ok) acc += mg * tiles_n;
  }
  prefix[groups] = ok ? acc : 0;
}

size_t grouped_gemm_ws_bytes(int64_t groups) { return (size_t)(((groups + 1) * 8 + 255) / 256 * 256); }

template <int LD, int BT, bool SU16>
static void launch_grouped_t(const ExactProblem& p, const int64_t* offsets, const int64_t* prefix, int64_t max_tiles,
                             int64_t groups, int vary_k, int64_t M, int64_t N, hipStream_t st) {
  const int64_t tn = (N + BT - 1) / BT;
  hipLaunchKernelGGL((exact_grouped_kernel<LD, BT, BT, SU16>), dim3((unsigned)max_tiles), dim3(256), 0, st, p, offsets,
                     prefix, groups, vary_k, M, N, tn);
}

hipError_t launch_grouped_gemm(int fmt, int64_t groups, const int64_t* offsets, int vary_k, int64_t total, int64_t M,
                               int64_t N, int64_t K, const int32_t* a_row_index, int64_t a_rows, const void* A,
                               const void* sA, const float* tA, int tA_mode, const void* B, const void* sB,
                               const float* tB, int tB_mode, float* C, void* ws, hipStream_t st) {
  int64_t* prefix = (int64_t*)ws;
  // Expert groups are small (hundreds of rows): 128 x 128 tiles.
  constexpr int BT = 128;
  const int64_t tiles_n = (N + BT - 1) / BT;
  const int64_t tiles_m_fixed = vary_k ? (M + BT - 1) / BT : 0;
  const int64_t align = fmt == 1 ? 32 : fmt == 2 ? 16 : 8;
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(64), 0, st, offsets, groups, total, vary_k, align, (int64_t)BT,
                     tiles_m_fixed, tiles_n, prefix);
  const int64_t max_tiles = vary_k ? groups * tiles_m_fixed * tiles_n : ((total + BT - 1) / BT + groups) * tiles_n;
  if (max_tiles <= 0) return hipGetLastError();
  ExactProblem p;
  p.A = (const uint8_t*)A; p.sA = (const uint8_t*)sA; p.tA = tA; p.tA_mode = tA_mode;
  p.a_idx = a_row_index; p.a_rows = a_rows; p.a_base = 0;
  p.B = (const uint8_t*)B; p.sB = (const uint8_t*)sB; p.tB = tB; p.tB_mode = tB_mode; p.C = C; p.ldc = N;
  if (!vary_k) {
    p.m_valid = 0; p.lda = K; p.n_valid = N; p.ldb = K; p.k_begin = 0; p.k_end = K;
  } else {
    p.m_valid = M; p.lda = total; p.n_valid = N; p.ldb = total; p.k_begin = 0; p.k_end = 0;
  }
  // Scale rows and K slices are 64-aligned unless K % 64 == 32 (or vary_k slices,
  // which start at multiples of 32 only).
  const bool su16 = fmt == 3 || (p.lda % 64 == 0 && !vary_k);
  if (fmt == 1) {
    if (su16) launch_grouped_t<1, BT, true>(p, offsets, prefix, max_tiles, groups, vary_k, M, N, st);
    else launch_grouped_t<1, BT, false>(p, offsets, prefix, max_tiles, groups, vary_k, M, N, st);
  } else if (fmt == 2) {
    if (su16) launch_grouped_t<2, BT, true>(p, offsets, prefix, max_tiles, groups, vary_k, M, N, st);
    else launch_grouped_t<2, BT, false>(p, offsets, prefix, max_tiles, groups, vary_k, M, N, st);
  } else {
    launch_grouped_t<0, BT, true>(p, offsets, prefix, max_tiles, groups, vary_k, M, N, st);
  }
  return hipGetLastError();
}

}  // namespace mxq
