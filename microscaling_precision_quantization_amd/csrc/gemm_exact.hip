// Block-scaled GEMMs with FP32-grade accumulation:
//   C[m, n] = tA tB * sum_k A_hat[m, k] B_hat[n, k]   ("TN", FP32 output)
//
// MXFP8, NVFP4 and BF16 run on the gfx950 16-bit MFMAs (v_mfma_f32_32x32x16_bf16/f16):
// every operand value is formed EXACTLY in a 16-bit format right before the matrix
// core consumes it, and the matrix core accumulates at FP32 precision (measured on
// MI355X: 2^20 + 2^-3 sums exactly at every operand position):
//   * MXFP8 (E4M3, E8M0 per 32 along K): q * 2^(s-127) has 4 significant bits and
//     stays in BF16 range, so the gfx950 scaled convert (which applies the
//     power-of-two scale exactly) yields it in BF16 -> BF16 MFMA.
//   * NVFP4 (E2M1, E4M3 per 16 along K, FP32 per row/tensor/expert): q * S has
//     at most 6 significant bits and lies in [2^-10, 2688], inside FP16's normal
//     range. S = 2^e * m (m = 1..1.875): the scaled convert applies 2^e, a packed
//     FP16 multiply applies m (exact) -> FP16 MFMA; tA tB in the epilogue.
//   * MXFP4 (E2M1, E8M0 per 32 along K) runs on the native FP4 form of the scaled
//     MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), which applies the E8M0 scales itself.
//     Measured on MI355X: lane l supplies row l % 32 and the whole 32-K block h = l / 32
//     of the instruction's 64 K (16 bytes, low nibble first), with that block's scale;
//     products of one block sum exactly, and a result differs from the exact value by
//     at most 2^-23.6 of the sum of the magnitudes of its terms (FP32-grade, unlike the
//     FP8 form's ~2^-13 window), so this path meets the same accuracy bound.
//   * Blockwise FP8 (E4M3, FP32 scale per row and 128-K block of A, per row or per
//     128 x 128 block of B): the E4M3 values are exact in BF16 -> BF16 MFMA into a
//     per-block partial sum; at the end of each 128-K stage the FP32 scales are applied
//     in software (acc += partial * sA sB, one FMA per accumulator).
//   * BF16 operands as they are -> BF16 MFMA.
// Definitions: microscaling blocks along the reduction dimension ("Miles
// Blackwell RL", remio.ai, section "Un Cuantizador Compartido Es el Mecanismo
// Real"); two-level NVFP4 (7minutos.es NVFP4 page, section "Que es realmente
// NVFP4"); dequantized-backward BF16 GEMMs and the BF16 shared expert (remio.ai,
// sections "La Compatibilidad ..." and "NVFP4 por token ...").
// The native scaled-FP8 MFMA (format 0) is not used for gemm_block_scaled: it sums each
// group of 8 consecutive K products of a lane in a fixed-point window about 13 bits
// below the group's largest product, dropping lower bits, and accumulates the group
// sums at FP32 precision (measured on MI355X), which breaks the 2e-5 bound on
// outlier-heavy data. It runs gemm_mxfp8_matrix_core (LD 5 below): the same pipeline
// with 128-K stages, one instruction per 64 K taking both operands' E8M0 bytes.
// Its operand layout (measured): lane l supplies row l % 32; with h = l / 32, bytes
// 0..15 are elements [16h, 16h+16) of the first 32-K block and bytes 16..31 the same
// elements of the second block; the scale of block b comes from lane (l % 32) + 32 b.
//
// Data movement: raw operand tiles go global -> LDS with gfx950's direct loads
// (buffer_load_dwordx4 ... lds: lane l of a wave instruction lands at LDS base +
// 16 l), through a 16-byte XOR swizzle chosen so that each 16-lane fragment read
// (ds_read_b128) covers all 64 banks (measured conflict-free). A stage holds 64 K
// (128 B/row BF16, 64 B/row MXFP8, 32 B/row NVFP4 / MXFP4), or 128 B/row for every
// format in the dense kernels when K allows chunked scales (128 K MXFP8, 256 K NVFP4
// and MXFP4: fewer barriers, larger loads). NS stages keep NS - 1 tiles in flight; explicit
// vmcnt waits + one barrier per stage. Scales travel either per stage into
// 4-byte LDS slots, or as 16-byte chunks per row (16 blocks) double-buffered in
// LDS and read into registers once per chunk. Out-of-range rows and K chunks
// read zeros (buffer range checks).
//
// Operand layouts of the 32x32x16 16-bit MFMAs (measured): lane l supplies row
// l % 32 and 8 consecutive K; accumulator r of lane l is
// C[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32].
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace mxq {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

namespace gx {
constexpr int kLdsBytes = 160 * 1024;           // gfx950 LDS per workgroup
template <int LD> struct RowBytes;
template <> struct RowBytes<0> { static constexpr int v = 128; };   // BF16
template <> struct RowBytes<1> { static constexpr int v = 64; };    // MXFP8
template <> struct RowBytes<2> { static constexpr int v = 32; };    // NVFP4
template <> struct RowBytes<3> { static constexpr int v = 32; };    // MXFP4
template <> struct RowBytes<4> { static constexpr int v = 128; };   // blockwise FP8: one 128-K block per stage
template <> struct RowBytes<5> { static constexpr int v = 128; };   // MXFP8 on the scaled FP8 MFMA: 128 K per stage
template <> struct RowBytes<6> { static constexpr int v = 128; };   // BF16 A x BF16 B built from NVFP4 weights (LDS rows BF16)

// Scale modes (SM):
//   0  general: K tiles may end early; per stage, one direct load per row and scale
//      unit (MXFP8 / MXFP4: 1 byte = one 32-block per unit, NVFP4: 2 bytes = two
//      16-blocks).
//   1  K % 64 == 0: per stage, one load per row of all the stage's blocks (2 / 4 bytes).
//   2  K % 64 == 0 and 16-byte aligned scale rows: 16 bytes per row (8 MXFP8 / 4 NVFP4
//      / 8 MXFP4 narrow stages) in one load, double-buffered in a separate LDS area;
//      cuts the scale cache-line requests by that factor.
// Each per-stage load lands in a 4-byte LDS slot per row (gfx950 places 1/2/4-byte
// direct loads at base + 4 lane); chunked scales in a 16-byte slot per row.
// Blockwise FP8 (LD 4): one FP32 scale per row and 128-K block, one dword load per row
// and stage (SU 1, SZ 4) whatever SM is.
template <int LD, int SM> struct ScaleDma {
  static constexpr int SU = LD == 4 ? 1 : (LD == 0 || LD == 6 || SM == 2) ? 0 : (SM == 1 ? 1 : 2);
  static constexpr int SZ = LD == 4 ? 4 : (LD == 1 || LD == 3) ? (SM >= 1 ? 2 : 1) : (SM >= 1 ? 4 : 2);
};

// OCC = workgroups meant to share one CU: the LDS budget of a workgroup is 1 / OCC of it.
// WIDE (chunked-scale mode only): 128 bytes per row and stage for every format (MXFP8 128 K,
// NVFP4 256 K per stage), i.e. fewer barriers and larger loads per stage.
template <int LD, int BM, int BN, int SM, int OCC = 1, bool WIDE = false>
struct Cfg {
  static constexpr int RB = (WIDE && LD != 0) ? 128 : RowBytes<LD>::v;
  static constexpr int BK = (LD == 0 || LD == 6) ? RB / 2 : (LD == 1 || LD == 4 || LD == 5) ? RB : 2 * RB;   // K per stage
  static constexpr int SBS = LD == 5 ? RB / 64 : RB / 32;                 // sub-blocks per stage
  static_assert(!WIDE || SM == 2, "wide stages need chunked scales");
  static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  static constexpr int SU = ScaleDma<LD, SM>::SU, SZ = ScaleDma<LD, SM>::SZ;
  static constexpr bool CH = SM == 2 && LD != 0 && LD != 4 && LD != 6;      // chunked scales
  // stages per 16-byte scale chunk (16 blocks)
  static constexpr int SPC = (LD == 1 || LD == 3 || LD == 5) ? 16 / (BK / 32) : LD == 2 ? 16 / (BK / 16) : 4;
  // chunk loads per wave: 64 rows of 16 bytes each; rows past BM + BN (a 128 x 256 tile
  // has 384) read zeros into the buffer's tail
  static constexpr int XS = CH ? (BM + BN + 255) / 256 : 0;
  static constexpr int CH_HALF = CH ? XS * 4096 : 0;              // one chunk buffer
  static constexpr int S_BYTES = SU * (BM + BN) * 4;              // scale slots of one stage
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int FREE = kLdsBytes / OCC - 2 * CH_HALF;
  static constexpr int NS_LDS = (4 * STAGE <= FREE) ? 4 : (3 * STAGE <= FREE ? 3 : 2);
  static constexpr int NS = (CH && NS_LDS > SPC + 1) ? SPC + 1 : NS_LDS;
  // 1 KiB wave instructions per wave (LD 6 builds its B tile through registers instead)
  static constexpr int IA = A_BYTES / 4096, IB = LD == 6 ? 0 : B_BYTES / 4096;
  static constexpr int IS = SU * (BM + BN) / 256;                 // 64-row scale loads per wave
  static_assert(SU == 0 || (BM + BN) % 256 == 0, "per-stage scale loads need BM + BN a multiple of 256");
  static constexpr int TI = BM / 64, TJ = BN / 64;                // 32x32 MFMA tiles per wave
  // staged epilogue (NVFP4): per wave 32 rows x (BN/2 + 8) FP32 in LDS
  static constexpr bool EPI_STAGED = LD == 2;
  static constexpr int EPI_PITCH = BN / 2 + 8;
  static constexpr int EPI_BYTES = EPI_STAGED ? 4 * 32 * EPI_PITCH * 4 : 0;
  static constexpr int LDS_MAIN = NS * STAGE + (CH ? 2 * CH_HALF : 0);
  static constexpr int LDS_TOTAL = LDS_MAIN > EPI_BYTES ? LDS_MAIN : EPI_BYTES;
  static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "tile must split into 1 KiB wave loads");
  // chunk c + 1 is issued at stage SPC c ahead of that stage's loads (tile SPC c + NS - 1);
  // the wait for tile SPC (c + 1) must cover it
  static_assert(!CH || NS - 1 <= SPC, "scale chunk must land with the tiles it covers");
};
}  // namespace gx

struct ExactProblem {
  const uint8_t* A;        // MXFP8: (rows, lda) bytes; NVFP4 / MXFP4: (rows, lda/2); BF16: (rows, lda) x 2 bytes
  const uint8_t* sA;       // MXFP8 / MXFP4 (rows, lda/32) E8M0; NVFP4 (rows, lda/16) E4M3
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

// Raw buffer resource (stride 0): reads at offset o (VGPR offset + SGPR offset,
// both counted in the range check) return zeros when o + size > num_records.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)base;
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
  r[3] = __builtin_amdgcn_readfirstlane(0x00020000);     // 32-bit data format, no swizzle
  return r;
}
constexpr uint32_t kOutOfRange = 0x80000000u;            // beyond every num_records used here

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

// Buffer -> LDS direct loads. M0 holds the wave's LDS destination; lane l's data
// lands at M0 + 16 l (dwordx4) or M0 + 4 l (ubyte / ushort / dword, zero-extended).
// Issued through inline asm so that the compiler adds none of its own waits: all
// ordering is explicit (vmcnt waits before each stage barrier, a final vmcnt(0)).
// M0 is not otherwise used by these kernels.
template <int SZ>
__device__ __forceinline__ void buf_dma(v4i rs, uint32_t voff, uint32_t soff, uint32_t m0) {
  soff = __builtin_amdgcn_readfirstlane(soff);           // uniform values, kept in SGPRs
  m0 = __builtin_amdgcn_readfirstlane(m0);
  if constexpr (SZ == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(rs), "s"(soff) : "memory");
  else if constexpr (SZ == 4)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(rs), "s"(soff) : "memory");
  else if constexpr (SZ == 2)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_ushort %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(rs), "s"(soff) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_ubyte %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(rs), "s"(soff) : "memory");
}

// N (1..4) dwordx4 loads sharing one M0 write: load n lands at M0 + 1024 n + 16 lane.
// The instruction offset applies to the LDS destination and to the buffer offset
// alike (32-bit wrap-around), so each VGPR offset is pre-biased by -1024 n.
template <int N>
__device__ __forceinline__ void buf_dma16_group(v4i rs, const uint32_t* vo, uint32_t soff, uint32_t m0) {
  soff = __builtin_amdgcn_readfirstlane(soff);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  if constexpr (N == 1)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0), "v"(vo[0]), "s"(rs), "s"(soff) : "memory");
  else if constexpr (N == 2)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen offset:1024 lds" ::"s"(m0), "v"(vo[0]), "v"(vo[1]), "s"(rs), "s"(soff) : "memory");
  else if constexpr (N == 3)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %4, %5 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %4, %5 offen offset:1024 lds\n\tbuffer_load_dwordx4 %3, %4, %5 offen offset:2048 lds"
                 ::"s"(m0), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "s"(rs), "s"(soff) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\tbuffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
                 "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds"
                 ::"s"(m0), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(rs), "s"(soff) : "memory");
}

template <int LD>
__device__ __forceinline__ int64_t k_bytes(int64_t k) {
  return (LD == 0 || LD == 6) ? k * 2 : (LD == 1 || LD == 4 || LD == 5) ? k : k / 2;
}

typedef __attribute__((address_space(3))) const uint8_t* lds_cptr;
__device__ __forceinline__ lds_cptr as_lds(uint32_t a) { return (lds_cptr)(uintptr_t)a; }
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 lds_ld16(lds_cptr p) { return *(const __attribute__((address_space(3))) u32x4*)p; }

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

// 2 x 16 E4M3 bytes as the A/B operand of the FP8 form of the scaled MFMA.
__device__ __forceinline__ v8i fp8_operand(const u32x4& lo, const u32x4& hi) {
  v8i v;
  v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
  v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
  return v;
}

// 32 E2M1 values (16 bytes) as the A/B operand of the FP4 form of the scaled MFMA, which
// reads the low four dwords.
__device__ __forceinline__ v8i fp4_operand(const u32x4& r) {
  v8i v;
  v[0] = (int)r.x; v[1] = (int)r.y; v[2] = (int)r.z; v[3] = (int)r.w;
  v[4] = 0; v[5] = 0; v[6] = 0; v[7] = 0;
  return v;
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

// The scaled converts use only the exponent field of their FP32 scale operand, an
// exponent field of 0 acting as 2^-127 (measured on MI355X). So an E8M0 code s is
// passed as the bits s << 23 (s = 0 included), and an E4M3 block scale S as S itself.

// E8M0 code -> scale operand of the MXFP8 converts.
__device__ __forceinline__ float mx_cvt_scale(uint32_t s) { return __uint_as_float(s << 23); }

// Byte SEL of `codes` (a positive E4M3 block scale S) -> the converts' scale operand
// (applies the power-of-two part 2^e of S) and the mantissa factor S / 2^e = 1.mmm as
// packed FP16 (exact). E4M3 subnormals are normal in FP32, so the split holds for
// them too; S = 0 scales by 2^-127, which flushes every E2M1 value to zero in FP16.
template <int SEL>
__device__ __forceinline__ void e4m3_split(uint32_t codes, float& p2, v2h& m2) {
  p2 = __builtin_amdgcn_cvt_f32_fp8((int)codes, SEL);
  const uint32_t mh = 0x3C00u | ((__float_as_uint(p2) >> 13) & 0x3FFu);
  const uint32_t pair = mh | (mh << 16);
  __builtin_memcpy(&m2, &pair, 4);
}

// Both bytes of a scale pair at once: p0 / p1 carry 2^e of bytes 0 / 1 as above, and mm holds
// their mantissa factors 1.mmm as packed FP16 (byte 0 low). The E4M3 codes convert to FP16
// exactly (subnormal codes become normal FP16), and forcing the FP16 exponent field to 15
// keeps just the factor S / 2^e -- the same values as the FP32 route.
__device__ __forceinline__ void e4m3_split2(uint32_t codes, float& p0, float& p1, v2h& mm) {
  p0 = __builtin_amdgcn_cvt_f32_fp8((int)codes, 0);
  p1 = __builtin_amdgcn_cvt_f32_fp8((int)codes, 1);
  const v2h s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, false);
  uint32_t b;
  __builtin_memcpy(&b, &s, 4);
  b = (b & 0x03FF03FFu) | 0x3C003C00u;
  __builtin_memcpy(&mm, &b, 4);
}

// nv_to_f16 with half H of a packed mantissa pair broadcast to both lanes of the multiply.
template <int H>
__device__ __forceinline__ v8h nv_to_f16_h(uint32_t w, float p2, v2h mm) {
  const v2h m2 = __builtin_shufflevector(mm, mm, H, H);
  return nv_to_f16(w, p2, m2);
}

template <int I> using ic = std::integral_constant<int, I>;

constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }
constexpr int lcm_int(int a, int b) { return a / gcd_int(a, b) * b; }

// Compile-time loop: f(ic<0>), ..., f(ic<N-1>).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(ic<I>{});
    static_for<I + 1, N>(f);
  }
}

// Tile of BM x BN outputs over K in [k_begin, k_end); 4 waves in a 2 x 2 grid,
// each owning (BM/2) x (BN/2) accumulators.
//
// K advances in stages of 64 (NS stages in LDS, NS - 1 loads in flight); a stage
// splits into SBS sub-blocks of one 16-byte chunk per lane and fragment (BF16: 4
// of 16 K, MXFP8: 2 of 32 K, NVFP4: 1 of 64 K). The raw fragments of the next
// sub-block are read from LDS while the matrix core works on the current one;
// the loads of the stage NS - 1 ahead are interleaved with the first sub-block's
// MFMAs, and the barrier that publishes the next stage sits halfway through the
// last sub-block.
// AKM: A is given K-major -- (k, m) row-major, p.lda = m per row -- as the slot-major
// gradients of a weight-gradient GEMM are; BF16 with per-chunk K tails (SM 0) only.
template <int LD, int BM, int BN, int SM, int OCC = 1, bool WIDE = false, bool AKM = false, bool PART = false>
__device__ __forceinline__ void exact_gemm_tile(const ExactProblem& p, int64_t m0, int64_t n0, uint8_t* lds0,
                                                uint8_t* lds1, uint8_t* lds2, uint8_t* lds3, uint8_t* ldsc) {
  using C = gx::Cfg<LD, BM, BN, SM, OCC, WIDE>;
  constexpr bool AL = SM >= 1;                            // every K tile full and 64-aligned
  constexpr bool CH = C::CH;
  constexpr int XS = C::XS, SPC = C::SPC;
  constexpr int RB = C::RB, NS = C::NS, TI = C::TI, TJ = C::TJ, IA = C::IA, IB = C::IB, IS = C::IS;
  constexpr int SBS = C::SBS;                             // sub-blocks per stage
  constexpr int NF = TI + TJ;                             // fragments per lane and sub-block
  constexpr int BS = LD == 4 ? 128 : (LD == 1 || LD == 3 || LD == 5) ? 32 : 16;   // elements per scale block
  constexpr int SEB = LD == 4 ? 4 : 1;                    // bytes per scale entry
  constexpr int EPC = (LD == 0 || LD == 6) ? 8 : (LD == 1 || LD == 4 || LD == 5) ? 16 : 32;   // elements per 16-byte chunk
  constexpr int OPS = IA + IB + IS;                       // direct loads per stage and wave (chunks aside)
  // stages per unrolled round (LD 6: four, one per B register buffer)
  constexpr int R = CH ? lcm_int(SPC, NS) : (LD == 6 ? 4 : NS);
  static_assert(R % NS == 0 && (!CH || R % SPC == 0), "round must cover whole slot and chunk cycles");
  static_assert((R * SBS) % 2 == 0, "fragment double buffer needs an even sub-block count per round");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, lr = lane & 31;

  const int64_t ldA = k_bytes<LD>(p.lda), ldB = k_bytes<LD>(p.ldb);
  const int64_t a_rows_tile = max((int64_t)0, min((int64_t)BM, p.m_valid - m0));
  const int64_t b_rows_tile = max((int64_t)0, min((int64_t)BN, p.n_valid - n0));

  // --- operand descriptors and per-lane offsets (fixed over K) -------------------
  // A: rebased at the tile's first row, or (gather) at the operand start with
  // per-row offsets; rows outside the tile's valid range read zeros.
  const v4i rsA = p.a_idx ? make_rsrc(p.A, (uint32_t)min(p.a_rows * ldA, (int64_t)0x7FFFFFFF))
                          : make_rsrc(p.A + (p.a_base + m0) * ldA, (uint32_t)(a_rows_tile * ldA));
  const v4i rsB = LD == 6 ? rsA : make_rsrc(p.B + n0 * ldB, (uint32_t)(b_rows_tile * ldB));
  uint32_t voA[IA], voB[IB > 0 ? IB : 1];
  static_assert(!AKM || (LD == 0 && SM == 0 && C::BK == 64), "K-major A: BF16 weight gradients");
  // K-major A: LDS row k of a stage holds the tile's BM values of operand row k0 + k (2 BM
  // bytes), 16-byte chunk c at position c ^ 4 (k % 4) -- so that the transpose reads of one
  // 32-lane half (4 rows x 64 bytes) cover all 64 banks once.
  constexpr int AROW = 2 * BM;
  static_assert(!AKM || AROW >= 256, "K-major A swizzle spans 16 chunks of a row");
#pragma unroll
  for (int j = 0; j < IA; ++j) {
    const int pos = (wave * IA + j) * 1024 + lane * 16;   // byte in the A tile
    uint32_t o;
    if constexpr (AKM) {
      const int row = pos / AROW;
      const int lc = ((pos % AROW) / 16) ^ (4 * (row % 4));
      o = (uint32_t)(row * ldA + lc * 16);
    } else {
      const int row = pos / RB;
      const int lc = ((pos % RB) / 16) ^ swz<RB>(row);    // logical chunk stored at this position
      o = (uint32_t)(row * ldA + lc * 16);
      if (p.a_idx) {
        const int64_t src = row < a_rows_tile ? exact_src_row(p, m0 + row) : -1;
        o = src >= 0 ? (uint32_t)(src * ldA + lc * 16) : kOutOfRange;
      }
    }
    voA[j] = o - 1024u * (uint32_t)(j % 4);                // see buf_dma16_group
  }
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const int pos = (wave * IB + j) * 1024 + lane * 16;
    const int row = pos / RB;
    const int lc = ((pos % RB) / 16) ^ swz<RB>(row);
    voB[j] = (uint32_t)(row * ldB + lc * 16) - 1024u * (uint32_t)(j % 4);
  }
  // Scales: load q of IS per wave covers 64 consecutive items of the [A rows | B rows]
  // list of unit u (SU units per stage); each lands in a 4-byte LDS slot per row.
  constexpr int BPU = ((LD == 1 || LD == 3) ? 2 : 4) / (C::SU > 0 ? C::SU : 1);   // blocks per unit
  v4i rsS[IS > 0 ? IS : 1];
  uint32_t voS[IS > 0 ? IS : 1];
#pragma unroll
  for (int q = 0; q < IS; ++q) {
    const int item0 = (wave * IS + q) * 64;
    const int u = item0 / (BM + BN);
    const int r0 = item0 % (BM + BN);
    const int row = r0 + lane;
    if (r0 < BM) {
      const int64_t lds_ = p.lda / BS * SEB;
      if (p.a_idx) {
        rsS[q] = make_rsrc(p.sA, (uint32_t)min(p.a_rows * lds_, (int64_t)0x7FFFFFFF));
        const int64_t src = row < a_rows_tile ? exact_src_row(p, m0 + row) : -1;
        voS[q] = src >= 0 ? (uint32_t)(src * lds_ + u * BPU) : kOutOfRange;
      } else {
        rsS[q] = make_rsrc(p.sA + (p.a_base + m0) * lds_, (uint32_t)(a_rows_tile * lds_));
        voS[q] = (uint32_t)(row * lds_ + u * BPU);
      }
    } else if (LD == 4 && p.tB_mode == 1) {
      // one scale per 128 x 128 block of B: every row of a 128-row block reads its block's
      // entry (n0 is a multiple of 128)
      const int64_t lds_ = p.ldb / BS * SEB;
      rsS[q] = make_rsrc(p.sB + (n0 / 128) * lds_, (uint32_t)((b_rows_tile + 127) / 128 * lds_));
      voS[q] = (uint32_t)(((row - BM) / 128) * lds_);
    } else {
      const int64_t lds_ = p.ldb / BS * SEB;
      rsS[q] = make_rsrc(p.sB + n0 * lds_, (uint32_t)(b_rows_tile * lds_));
      voS[q] = (uint32_t)((row - BM) * lds_ + u * BPU);
    }
  }

  // Chunked scales: load q of XS per wave covers rows (wave XS + q) 64 + lane of the
  // [A rows | B rows] list, 16 bytes (one chunk) per row; all loads of a wave fall in
  // one operand (BM is a multiple of 64 XS) and share one M0 write.
  v4i rsX = rsA;
  uint32_t voX[XS > 0 ? XS : 1];
  if constexpr (CH) {
    static_assert(BM % (64 * XS) == 0, "chunk loads of a wave must stay in one operand");
    const bool xa = wave * XS * 64 < BM;
    const int64_t lds_ = (xa ? p.lda : p.ldb) / BS;        // scale bytes per row
#pragma unroll
    for (int q = 0; q < XS; ++q) {
      const int row = (wave * XS + q) * 64 + lane;
      uint32_t o;
      if (xa && p.a_idx) {
        const int64_t src = row < a_rows_tile ? exact_src_row(p, m0 + row) : -1;
        o = src >= 0 ? (uint32_t)(src * lds_) : kOutOfRange;
      } else {
        o = (uint32_t)((xa ? row : row - BM) * lds_);
      }
      voX[q] = o - 1024u * (uint32_t)q;
    }
    if (xa) rsX = p.a_idx ? make_rsrc(p.sA, (uint32_t)min(p.a_rows * lds_, (int64_t)0x7FFFFFFF))
                          : make_rsrc(p.sA + (p.a_base + m0) * lds_, (uint32_t)(a_rows_tile * lds_));
    else rsX = make_rsrc(p.sB + n0 * lds_, (uint32_t)(b_rows_tile * lds_));
  }
  const uint32_t lbase_c = lds_addr(ldsc);

  const uint32_t lbase[4] = {lds_addr(lds0), lds_addr(lds1), lds_addr(lds2), lds_addr(lds3)};

  // LD 6: the B tile is made from NVFP4 weight rows W[k][n] (E2M1 pairs along n, one E4M3
  // scale per 16 n, one FP32 decode scale t for the whole group): B[n][k] =
  // RNE_bf16(fl32(fl32(q S) t)), the dequantized weight transposed. It is kept K-major in
  // LDS -- row k of a stage holds the tile's 256 BF16 values of W row k0 + k, 16-byte chunk
  // c at position c ^ 5 (k % 4) -- and the MFMA fragments come out through transpose reads,
  // like a K-major A. Lane (w, l) of the 256 threads owns stage row kr = 16 w + 4 (l / 16) +
  // (l / 2) % 4 and, with q = 2 ((l / 8) % 2) + l % 2, the 32-n pieces q and q + 4 of it: two
  // 16-byte loads of packed E2M1 and four scale bytes per stage (six loads; narrow 8 x 8
  // blocks took sixteen and ran the DeepSeek-shaped dgrads 5-6% slower). Sub-block b
  // converts 16 values (two chunks); the last one writes the block's eight chunks (1% faster
  // than writing each sub-block's pair as it is made). The LDS takes 16-byte writes 8 lanes
  // (128 bytes) at a time: each such group holds 4 rows x 2 adjacent pieces, which the
  // rotation puts on 32 different banks (4 pieces of 2 rows per group, the first lane order,
  // cost 25% of the LDS cycles in bank conflicts); each 32-lane pass of the transpose reads
  // covers all 64 banks.
  const int kb_ = (int)p.k_begin;
  const int nk_ = ((int)p.k_end - kb_ + C::BK - 1) / C::BK;
  constexpr bool NVT = LD == 6;
  static_assert(!NVT || (BN == 256 && C::BK == 64 && C::SBS == 4 && TJ / 2 - 1 == 1 && C::IA == 8),
                "the NVFP4-transposed B path is laid out for 256 x 64 stages of four sub-blocks");
  constexpr int BROW6 = 2 * BN;                           // bytes of one K-major B row in LDS
  constexpr int NB6 = 6;                                  // B loads per lane and stage
  __amdgpu_buffer_rsrc_t rsB6, rsS6;
  uint32_t voB6 = 0, voS6 = 0;
  uint32_t wo6[NVT ? 4 : 1] = {};                         // LDS offset of the lane's chunk c of piece q
  float t6 = 0.0f;
  int64_t rowB6 = 0, rowS6 = 0;
  if constexpr (NVT) {
    const int kr6 = 16 * wave + 4 * (lane >> 4) + ((lane >> 1) & 3), q6 = 2 * ((lane >> 3) & 1) + (lane & 1);
    const int a6 = kr6 & 3;
    rowB6 = p.ldb / 2;                                    // bytes per W row (p.ldb = N elements)
    rowS6 = p.ldb / 16;
    rsB6 = __builtin_amdgcn_make_buffer_rsrc((void*)p.B, (short)0, (int)min(p.k_end * rowB6, (int64_t)0x7FFFFFFF),
                                             0x00020000);
    rsS6 = __builtin_amdgcn_make_buffer_rsrc((void*)p.sB, (short)0, (int)min(p.k_end * rowS6, (int64_t)0x7FFFFFFF),
                                             0x00020000);
    // Columns at or past n_valid read whatever in-range bytes follow, or zeros past the
    // buffer; they only feed accumulator columns the epilogue never stores.
    const int64_t n = n0 + 32 * q6;
    voB6 = (uint32_t)(kr6 * rowB6 + n / 2);               // piece q; piece q + 4 is 64 bytes on
    voS6 = (uint32_t)(kr6 * rowS6 + n / 16);              // its two scale bytes; piece q + 4's at + 8
#pragma unroll
    for (int c = 0; c < 4; ++c) wo6[c] = (uint32_t)(kr6 * BROW6 + 16 * (4 * (q6 ^ a6) + (c ^ a6)));
    t6 = p.tB[0];
  }
  // Four register buffers: the B loads of tile t + 4 go out during stage t, so each block has
  // three stages to arrive before stage t + 3 converts it (16 values in each sub-block) and
  // writes it to its slot (2-4% faster dgrads than two buffers, one stage ahead; rounds of
  // four stages keep the buffer indices static).
  uint32_t bq6[4][NVT ? 8 : 1], bs6[4][NVT ? 4 : 1];
  uint32_t out6[NVT ? 32 : 1];                            // the converted block: chunk pairs of sub-blocks 0..3
  // loads of B tile t into buffer BUF, in the order the sub-blocks use them (rows at or past
  // k_end, and tiles past the end, read zeros)
  auto nvt_issue = [&](int t, auto BUF) {
    if constexpr (NVT) {
      constexpr int bf = decltype(BUF)::value;
      typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
      const int k0 = kb_ + t * C::BK;
      const bool past = t >= nk_;
      const int so = (int)(past ? kOutOfRange : (uint32_t)(k0 * rowB6));
      const int ss = (int)(past ? kOutOfRange : (uint32_t)(k0 * rowS6));
      const v4u_t d0 = __builtin_amdgcn_raw_buffer_load_b128(rsB6, (int)voB6, so, 0);
      bs6[bf][0] = __builtin_amdgcn_raw_buffer_load_b8(rsS6, (int)voS6, ss, 0);
      bs6[bf][1] = __builtin_amdgcn_raw_buffer_load_b8(rsS6, (int)(voS6 + 1), ss, 0);
      const v4u_t d1 = __builtin_amdgcn_raw_buffer_load_b128(rsB6, (int)(voB6 + 64), so, 0);
      bs6[bf][2] = __builtin_amdgcn_raw_buffer_load_b8(rsS6, (int)(voS6 + 8), ss, 0);
      bs6[bf][3] = __builtin_amdgcn_raw_buffer_load_b8(rsS6, (int)(voS6 + 9), ss, 0);
      bq6[bf][0] = d0.x; bq6[bf][1] = d0.y; bq6[bf][2] = d0.z; bq6[bf][3] = d0.w;
      bq6[bf][4] = d1.x; bq6[bf][5] = d1.y; bq6[bf][6] = d1.z; bq6[bf][7] = d1.w;
    }
  };
  // half H (8 values) of sub-block b's 16 values of the block in buffer BUF -> out6[8 b + 4 H ..],
  // BF16 pairs of adjacent n
  auto nvt_conv = [&](auto BUF, auto SB, auto H) {
    if constexpr (NVT) {
      constexpr int bf = decltype(BUF)::value, b = decltype(SB)::value, hh = decltype(H)::value;
      const uint32_t w = bq6[bf][4 * (b / 2) + 2 * (b % 2) + hh];
      const float Sb = __builtin_amdgcn_cvt_f32_fp8((int)bs6[bf][b], 0);   // exact E4M3 decode, no branch
      const v2f_t e0 = e2m1x2_to_f32<0>(w), e1 = e2m1x2_to_f32<1>(w);
      const v2f_t e2 = e2m1x2_to_f32<2>(w), e3 = e2m1x2_to_f32<3>(w);
      out6[8 * b + 4 * hh + 0] = bf16x2_rne((e0.x * Sb) * t6, (e0.y * Sb) * t6);   // q S exact, then * t
      out6[8 * b + 4 * hh + 1] = bf16x2_rne((e1.x * Sb) * t6, (e1.y * Sb) * t6);
      out6[8 * b + 4 * hh + 2] = bf16x2_rne((e2.x * Sb) * t6, (e2.y * Sb) * t6);
      out6[8 * b + 4 * hh + 3] = bf16x2_rne((e3.x * Sb) * t6, (e3.y * Sb) * t6);
    }
  };
  // sub-block b's two chunks (piece q + 4 (b / 2), chunks 2 (b % 2) and 2 (b % 2) + 1) into
  // the B area of slot S
  auto nvt_write = [&](auto SLOT, auto SB) {
    if constexpr (NVT) {
      constexpr int S = decltype(SLOT)::value, b = decltype(SB)::value;
      const uint32_t base = lbase[S] + C::A_BYTES + (uint32_t)(256 * (b / 2));
      const u32x4 v0 = {out6[8 * b + 0], out6[8 * b + 1], out6[8 * b + 2], out6[8 * b + 3]};
      const u32x4 v1 = {out6[8 * b + 4], out6[8 * b + 5], out6[8 * b + 6], out6[8 * b + 7]};
      *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(base + wo6[2 * (b % 2)]) = v0;
      *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(base + wo6[2 * (b % 2) + 1]) = v1;
    }
  };
  auto nvt_store = [&](auto BUF, auto SLOT) {
    static_for<0, 4>([&](auto SB) {
      nvt_conv(BUF, SB, ic<0>{});
      nvt_conv(BUF, SB, ic<1>{});
      nvt_write(SLOT, SB);
    });
  };

  const int kb = (int)p.k_begin, ke = (int)p.k_end;       // K <= 2^22
  const int nk = (ke - kb + C::BK - 1) / C::BK;

  // Uniform load parameters of tile t. Tiles past the end read zeros (out-of-range
  // SGPR offset); in the last tile, chunks and scale units at or beyond k_end are
  // turned out of range per lane.
  struct TileK { uint32_t sod, sos; int k0; bool tail; v4i rsa; };
  auto tile_k = [&](int t) {
    TileK r;
    r.k0 = kb + t * C::BK;
    const bool past = t >= nk;
    if constexpr (AKM) {
      // the stage's rows of the K-major A, clipped at k_end (rows past it read zeros; the
      // columns past m_valid of the last row read bytes that only feed unstored outputs)
      const int64_t rows = past ? 0 : min((int64_t)C::BK, (int64_t)(ke - r.k0));
      const int64_t bytes = rows > 0 ? rows * ldA - m0 * 2 : 0;
      r.rsa = make_rsrc(p.A + (int64_t)r.k0 * ldA + m0 * 2, (uint32_t)min(bytes, (int64_t)0x7FFFFFFF));
    }
    r.sod = past ? kOutOfRange : (uint32_t)((LD == 0 || LD == 6) ? 2 * r.k0 : (LD == 1 || LD == 4 || LD == 5) ? r.k0 : r.k0 / 2);
    r.sos = past ? kOutOfRange : (uint32_t)(r.k0 / BS * SEB);
    r.tail = !AL && !past && r.k0 + C::BK > ke;
    return r;
  };
  // DMA unit d of a tile into slot S: units 0 .. GA-1 are groups of up to 4 A loads,
  // GA .. GA+GB-1 groups of B loads, then the IS scale loads.
  constexpr int GA = (IA + 3) / 4, GB = (IB + 3) / 4, UNITS = GA + GB + IS;
  auto issue_unit = [&](const TileK& tk, auto SLOT, auto D) {
    constexpr int S = decltype(SLOT)::value, d = decltype(D)::value;
    const uint32_t lb = lbase[S];
    if constexpr (d < GA + GB) {
      constexpr bool isA = d < GA;
      constexpr int g = isA ? d : d - GA;
      constexpr int NI = isA ? IA : IB;
      constexpr int N = (NI - 4 * g) < 4 ? NI - 4 * g : 4;
      uint32_t vo[N];
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const int j = 4 * g + n;
        vo[n] = isA ? voA[j] : voB[j];
        if constexpr (!AL && !(AKM && isA)) {
          if (tk.tail) {
            const int pos = (wave * NI + j) * 1024 + lane * 16;
            const int lc = ((pos % RB) / 16) ^ swz<RB>(pos / RB);
            if (tk.k0 + lc * EPC >= ke) vo[n] = kOutOfRange - 1024u * (uint32_t)n;
          }
        }
      }
      const uint32_t m0v = lb + (isA ? 0 : C::A_BYTES) + (uint32_t)(wave * NI + 4 * g) * 1024u;
      if constexpr (AKM && isA) buf_dma16_group<N>(tk.rsa, vo, 0u, m0v);
      else buf_dma16_group<N>(isA ? rsA : rsB, vo, tk.sod, m0v);
    } else if constexpr (IS > 0) {
      constexpr int q = d - GA - GB;
      uint32_t vo = voS[q];
      if constexpr (!AL) {
        const int u = ((wave * IS + q) * 64) / (BM + BN);
        if (tk.tail && tk.k0 + u * BPU * BS >= ke) vo = kOutOfRange;
      }
      const uint32_t m0v = lb + C::A_BYTES + C::B_BYTES + (uint32_t)(wave * IS + q) * 256u;
      buf_dma<C::SZ>(rsS[q], vo, tk.sos, m0v);
    }
  };
  // units [LO, HI) of a tile
  auto issue_range = [&](const TileK& tk, auto SLOT, auto LO, auto HI) {
    static_for<decltype(LO)::value, decltype(HI)::value>([&](auto D) { issue_unit(tk, SLOT, D); });
  };
  // scale chunk c (stages [SPC c, SPC c + SPC)) into chunk buffer c % 2
  auto issue_chunk = [&](int c) {
    if constexpr (CH) {
      const uint32_t so = c * SPC < nk ? (uint32_t)(16 * c) : kOutOfRange;
      const uint32_t m0v = lbase_c + (uint32_t)(c & 1) * C::CH_HALF + (uint32_t)(wave * XS) * 1024u;
      buf_dma16_group<XS>(rsX, voX, so, m0v);
    }
  };

  // --- fragments ---------------------------------------------------------------
  // raw[f]: the lane's 16-byte chunk of fragment f (A rows i = 0..TI-1, then B rows
  // j = 0..TJ-1) for one sub-block; sc[f]: its scale byte(s).
  // LD 5: raw holds K [16h, 16h+16) of the sub-block's first 32-K block, raw2 the same of
  // its second block (the scaled FP8 MFMA's operand layout).
  struct Frag { u32x4 raw[NF]; u32x4 raw2[LD == 5 ? NF : 1]; uint32_t sc[NF]; };
  Frag F[2];

  // LDS addresses of the fragment reads. Fragment rows start at multiples of 32 and
  // the swizzle period is 16 rows, so the swizzle depends on lr alone: the lane part
  // (xo) is one VGPR per sub-block, the wave part is uniform and the fragment part
  // is an instruction offset.
  uint32_t xo[SBS];
#pragma unroll
  for (int b = 0; b < SBS; ++b)
    xo[b] = (uint32_t)(lr * RB + ((((LD == 5 ? 4 : 2) * b + h) ^ swz<RB>(lr)) << 4));
  uint32_t xo2[LD == 5 ? SBS : 1];
  if constexpr (LD == 5) {
#pragma unroll
    for (int b = 0; b < SBS; ++b) xo2[b] = (uint32_t)(lr * RB + (((4 * b + 2 + h) ^ swz<RB>(lr)) << 4));
  }
  const uint32_t wA = (uint32_t)(wm * (BM / 2) * RB), wB = (uint32_t)(C::A_BYTES + wn * (BN / 2) * RB);
  const uint32_t xs = (uint32_t)(lr * 4);                 // scale slot of the lane's row
  const uint32_t wsA = (uint32_t)(C::A_BYTES + C::B_BYTES + wm * (BM / 2) * 4);
  const uint32_t wsB = (uint32_t)(C::A_BYTES + C::B_BYTES + (BM + wn * (BN / 2)) * 4);
  constexpr int SC_UNIT = (BM + BN) * 4;                  // bytes between scale units (SU == 2)

  // Chunked scales: the 16-byte chunk row of each fragment row (one per lane) is read into
  // registers once per chunk (SPC stages), at its first stage, and the stage's bytes are
  // taken from there: row r's byte (MXFP8 block b, MXFP4 block 2b + h) or byte pair (NVFP4
  // blocks 2h, 2h+1) of stage t sits at chunk + 16 r + (t % SPC) * bytes per stage. (Byte-wise LDS reads of
  // 16-byte-strided rows would each take several conflicting passes.)
  const uint32_t wcA = (uint32_t)(wm * (BM / 2) * 16), wcB = (uint32_t)((BM + wn * (BN / 2)) * 16);
  u32x4 chr[CH ? NF : 1];
  // K-major A fragments: two LDS transpose reads (ds_read_b64_tr_b16) per 32 x 16 fragment.
  // In a 16-lane group, lane i receives element i % 4 of the 8-byte rows addressed by
  // lanes i / 4 + 4 j (measured); lane (gq, l16) therefore addresses row 4 q + l16 / 4 of
  // the group's k block (q: first or second 4 k of the lane half) at the 4 m values
  // 4 (l16 % 4) onward, and receives 4 consecutive k of its own m -- the 16-bit MFMA
  // operand. akm_lane[i]: the lane's offset for fragment i, whose 4 chunks are the row's
  // chunk group q = wm TI + i, stored at group q ^ (k % 4).
  uint32_t akm_lane[AKM ? TI : 1] = {};
  if constexpr (AKM) {
    const int gq = lane >> 4, l16 = lane & 15, r = l16 >> 2;
    const int xa = 2 * (gq & 1) + ((l16 & 3) >> 1);
    const uint32_t rowoff = (uint32_t)((8 * (gq >> 1) + r) * AROW) + (uint32_t)((l16 & 1) * 8);
#pragma unroll
    for (int i = 0; i < TI; ++i) akm_lane[i] = rowoff + (uint32_t)((4 * ((wm * TI + i) ^ r) + xa) * 16);
  }
  // LD 6 B fragments, read the same way from the K-major B rows (chunk group q = wn TJ + j
  // of row k at group q ^ (k % 4), its chunk x at x ^ (k % 4)).
  uint32_t bkm_lane[NVT ? TJ : 1] = {};
  if constexpr (NVT) {
    const int gq = lane >> 4, l16 = lane & 15, r = l16 >> 2;
    const int xa = 2 * (gq & 1) + ((l16 & 3) >> 1);
    const uint32_t rowoff = (uint32_t)(C::A_BYTES + (8 * (gq >> 1) + r) * BROW6 + (l16 & 1) * 8);
#pragma unroll
    for (int j = 0; j < TJ; ++j) bkm_lane[j] = rowoff + (uint32_t)(16 * (4 * ((wn * TJ + j) ^ r) + (xa ^ r)));
  }
  // two transpose reads: rows k .. k + 3 of the lane's group at a, k + 4 .. k + 7 at a + 4 rows
  auto tr_frag = [&](uint32_t a, uint32_t row_bytes) {
    typedef short v4s16 __attribute__((ext_vector_type(4)));
    const v4s16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s16*)(uintptr_t)a);
    const v4s16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s16*)(uintptr_t)(a + 4 * row_bytes));
    uint32_t w[4];
    __builtin_memcpy(&w[0], &r0, 8);
    __builtin_memcpy(&w[2], &r1, 8);
    return u32x4{w[0], w[1], w[2], w[3]};
  };
  // TP = t % SPC, known at compile time in the unrolled rounds (R is a multiple of SPC)
  auto read_sub = [&](int t, auto SLOT, auto SB, auto TP, Frag& fr, auto TIAC) {
    constexpr int S = decltype(SLOT)::value, b = decltype(SB)::value, tp = decltype(TP)::value;
    constexpr int TIA = decltype(TIAC)::value;           // A fragments this wave needs
    const lds_cptr pa = as_lds(lbase[S] + wA + xo[b]);
    const lds_cptr pb = as_lds(lbase[S] + wB + xo[b]);
    if constexpr (AKM) {
#pragma unroll
      for (int i = 0; i < TIA; ++i) fr.raw[i] = tr_frag(lbase[S] + akm_lane[i] + (uint32_t)(16 * b * AROW), AROW);
    } else {
#pragma unroll
      for (int i = 0; i < TIA; ++i) fr.raw[i] = lds_ld16(pa + i * 32 * RB);
    }
    if constexpr (NVT) {
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        fr.raw[TI + j] = tr_frag(lbase[S] + bkm_lane[j] + (uint32_t)(16 * b * BROW6), BROW6);
    } else {
#pragma unroll
      for (int j = 0; j < TJ; ++j) fr.raw[TI + j] = lds_ld16(pb + j * 32 * RB);
    }
    if constexpr (LD == 5) {
      const lds_cptr pa2 = as_lds(lbase[S] + wA + xo2[b]);
      const lds_cptr pb2 = as_lds(lbase[S] + wB + xo2[b]);
#pragma unroll
      for (int i = 0; i < TIA; ++i) fr.raw2[i] = lds_ld16(pa2 + i * 32 * RB);
#pragma unroll
      for (int j = 0; j < TJ; ++j) fr.raw2[TI + j] = lds_ld16(pb2 + j * 32 * RB);
    }
    if constexpr (CH) {
      if constexpr (tp == 0 && b == 0) {
        const uint32_t cb = lbase_c + (uint32_t)((t / SPC) & 1) * C::CH_HALF + (uint32_t)(lr * 16);
#pragma unroll
        for (int f = 0; f < NF; ++f)
          chr[f] = lds_ld16(as_lds(cb + (f < TI ? wcA + f * 512 : wcB + (f - TI) * 512)));
      }
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if constexpr (LD == 1) {                      // one block per sub-block
          constexpr int idx = tp * SBS + b;
          fr.sc[f] = (chr[f][idx / 4] >> (8 * (idx % 4))) & 0xFFu;
        } else if constexpr (LD == 3 || LD == 5) {    // two blocks per sub-block, one per lane half
          constexpr int idx = tp * 2 * SBS + 2 * b;    // even: idx % 4 + h stays in its dword
          fr.sc[f] = (chr[f][idx / 4] >> (8 * (idx % 4 + h))) & 0xFFu;
        } else {                                      // four blocks per sub-block, two per lane
          fr.sc[f] = (chr[f][tp * SBS + b] >> (16 * h)) & 0xFFFFu;
        }
      }
    } else if constexpr (LD != 0 && LD != 4 && LD != 6) {
      const lds_cptr sa = as_lds(lbase[S] + wsA + xs), sb = as_lds(lbase[S] + wsB + xs);
      // MXFP8: the byte of block b; NVFP4: the two bytes of blocks 2h, 2h+1; MXFP4 (one
      // sub-block per stage): the byte of block h
      // LD 5 (four blocks per stage, two per sub-block): the byte of block 2b + h
      const int so = LD == 1 ? (C::SU == 1 ? b : b * SC_UNIT)
                   : LD == 2 ? (C::SU == 1 ? 2 * h : h * SC_UNIT)
                   : LD == 5 ? (C::SU == 1 ? 2 * b + h : b * SC_UNIT + h) : (C::SU == 1 ? h : h * SC_UNIT);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const lds_cptr q = (f < TI ? sa + f * 128 : sb + (f - TI) * 128) + so;
        fr.sc[f] = LD != 2 ? (uint32_t)*q : (uint32_t)*(const __attribute__((address_space(3))) uint16_t*)q;
      }
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // Blockwise FP8: the matrix core sums one 128-K block into `part`; at the end of the
  // stage the block's FP32 scales are applied in software, acc += part * (sA[row] sB[col]),
  // and part restarts from zero.
  constexpr int TI4 = LD == 4 ? TI : 1, TJ4 = LD == 4 ? TJ : 1;
  v16f part[TI4][TJ4];
  float sa4[TI4][16], sb4[TJ4];
#pragma unroll
  for (int i = 0; i < TI4; ++i)
#pragma unroll
    for (int j = 0; j < TJ4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[i][j][r] = 0.0f;
  auto dst = [&](int i, int j) -> v16f& {
    if constexpr (LD == 4) return part[i][j];
    else return acc[i][j];
  };
  // the stage's scales (slot S, published by the barrier that ended the previous stage)
  auto read_scales4 = [&](auto SLOT) {
    if constexpr (LD == 4) {
      constexpr int S = decltype(SLOT)::value;
      const uint32_t base = lbase[S] + C::A_BYTES + C::B_BYTES;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {        // accumulator rows 8 g + 4 h + 0..3 of MFMA tile i
          const int row = wm * (BM / 2) + i * 32 + g * 8 + h * 4;
          const u32x4 v4 = lds_ld16(as_lds(base + (uint32_t)(row * 4)));
          sa4[i][4 * g + 0] = __uint_as_float(v4.x);
          sa4[i][4 * g + 1] = __uint_as_float(v4.y);
          sa4[i][4 * g + 2] = __uint_as_float(v4.z);
          sa4[i][4 * g + 3] = __uint_as_float(v4.w);
        }
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        sb4[j] = *(const __attribute__((address_space(3))) float*)as_lds(
            base + (uint32_t)((BM + wn * (BN / 2) + j * 32 + lr) * 4));
    }
  };
  auto promote4 = [&]() {
    if constexpr (LD == 4) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[i][j][r] = __builtin_fmaf(part[i][j][r], sa4[i][r] * sb4[j], acc[i][j][r]);
            part[i][j][r] = 0.0f;
          }
    }
  };

  // Convert + MFMA one sub-block; hook(jj) runs after the MFMAs of B fragment jj.
  auto mma_sub = [&](const Frag& fr, auto TIAC, auto&& hook) {
    constexpr int TIA = decltype(TIAC)::value;
    if constexpr (LD == 0 || LD == 6) {
      v8bf fa[TI];
#pragma unroll
      for (int i = 0; i < TIA; ++i) __builtin_memcpy(&fa[i], &fr.raw[i], 16);
      static_for<0, TJ>([&](auto JJ) {
        constexpr int j = decltype(JJ)::value;
        v8bf fb;
        __builtin_memcpy(&fb, &fr.raw[TI + j], 16);
#pragma unroll
        for (int i = 0; i < TIA; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb, acc[i][j], 0, 0, 0);
        hook(JJ);
      });
    } else if constexpr (LD == 1 || LD == 4) {
      // MXFP8: E4M3 * 2^(s-127); blockwise FP8: the E4M3 values themselves (scale 2^0)
      v8bf fa0[TI], fa1[TI];
#pragma unroll
      for (int i = 0; i < TIA; ++i) {
        const float s = LD == 4 ? 1.0f : mx_cvt_scale(fr.sc[i]);
        fa0[i] = mx_to_bf16(fr.raw[i].x, fr.raw[i].y, s);
        fa1[i] = mx_to_bf16(fr.raw[i].z, fr.raw[i].w, s);
      }
      static_for<0, TJ>([&](auto JJ) {
        constexpr int j = decltype(JJ)::value;
        const float s = LD == 4 ? 1.0f : mx_cvt_scale(fr.sc[TI + j]);
        const v8bf fb0 = mx_to_bf16(fr.raw[TI + j].x, fr.raw[TI + j].y, s);
        const v8bf fb1 = mx_to_bf16(fr.raw[TI + j].z, fr.raw[TI + j].w, s);
#pragma unroll
        for (int i = 0; i < TIA; ++i) dst(i, j) = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[i], fb0, dst(i, j), 0, 0, 0);
#pragma unroll
        for (int i = 0; i < TIA; ++i) dst(i, j) = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[i], fb1, dst(i, j), 0, 0, 0);
        hook(JJ);
      });
    } else if constexpr (LD == 5) {
      // Native E4M3 x E4M3 scaled MFMA, 64 K per instruction: lane half h supplies K
      // [16h, 16h+16) of both 32-K blocks of the sub-block and the E8M0 byte of block h.
      v8i fa[TI];
#pragma unroll
      for (int i = 0; i < TIA; ++i) fa[i] = fp8_operand(fr.raw[i], fr.raw2[i]);
      static_for<0, TJ>([&](auto JJ) {
        constexpr int j = decltype(JJ)::value;
        const v8i fb = fp8_operand(fr.raw[TI + j], fr.raw2[TI + j]);
#pragma unroll
        for (int i = 0; i < TIA; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb, acc[i][j], 0, 0, 0, (int)fr.sc[i], 0,
                                                                     (int)fr.sc[TI + j]);
        hook(JJ);
      });
    } else if constexpr (LD == 3) {
      // Native E2M1 x E2M1 scaled MFMA, 64 K per instruction: lane half h supplies the
      // whole 32-K block of its chunk and that block's E8M0 byte (the operand layout the
      // sub-block reads already have).
      v8i fa[TI];
#pragma unroll
      for (int i = 0; i < TIA; ++i) fa[i] = fp4_operand(fr.raw[i]);
      static_for<0, TJ>([&](auto JJ) {
        constexpr int j = decltype(JJ)::value;
        const v8i fb = fp4_operand(fr.raw[TI + j]);
#pragma unroll
        for (int i = 0; i < TIA; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb, acc[i][j], 4, 4, 0, (int)fr.sc[i], 0,
                                                                     (int)fr.sc[TI + j]);
        hook(JJ);
      });
    } else {
      v8h fa[2][2][TI];        // [half][dword pair][i]
#pragma unroll
      for (int i = 0; i < TIA; ++i)
      {
        float p0, p1;
        v2h mm;
        e4m3_split2(fr.sc[i], p0, p1, mm);
        fa[0][0][i] = nv_to_f16_h<0>(fr.raw[i].x, p0, mm);
        fa[0][1][i] = nv_to_f16_h<0>(fr.raw[i].y, p0, mm);
        fa[1][0][i] = nv_to_f16_h<1>(fr.raw[i].z, p1, mm);
        fa[1][1][i] = nv_to_f16_h<1>(fr.raw[i].w, p1, mm);
      }
      static_for<0, TJ>([&](auto JJ) {
        constexpr int j = decltype(JJ)::value;
        float pb0, pb1;
        v2h mb;
        e4m3_split2(fr.sc[TI + j], pb0, pb1, mb);
        static_for<0, 2>([&](auto HF) {
          constexpr int hf = decltype(HF)::value;
          const float p2 = hf ? pb1 : pb0;
          const v8h fb0 = nv_to_f16_h<hf>(hf ? fr.raw[TI + j].z : fr.raw[TI + j].x, p2, mb);
          const v8h fb1 = nv_to_f16_h<hf>(hf ? fr.raw[TI + j].w : fr.raw[TI + j].y, p2, mb);
#pragma unroll
          for (int i = 0; i < TIA; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[hf][0][i], fb0, acc[i][j], 0, 0, 0);
#pragma unroll
          for (int i = 0; i < TIA; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[hf][1][i], fb1, acc[i][j], 0, 0, 0);
        });
        hook(JJ);
      });
    }
  };

  // The loads of tile t + NS - 1 are spread over the first PJ B-fragment steps of
  // sub-block 0; the barrier comes after B fragment BJ of the last sub-block.
  constexpr int BJ = TJ / 2 - 1;
  constexpr int PJ = SBS == 1 ? BJ + 1 : TJ;

  // Loads issued after tile t+1's data (issued in stage t+2-NS): the data of the
  // NS-2 later tiles, plus the chunk loads of chunk-start stages among the last NS-2
  // stages (issued ahead of their stage's data).
  auto allowed = [](auto RI) constexpr {
    constexpr int ri = decltype(RI)::value;
    int n = (NS - 2) * OPS + (NVT ? NB6 : 0);
    if constexpr (CH)
      for (int d = 0; d <= NS - 3; ++d)
        if (((ri - d) % R + R) % R % SPC == 0) n += XS;
    return n;
  };

  // One stage: tile kt (round position RI) in slot RI % NS.
  auto stage = [&](int kt, auto RI, auto TIAC) {
    constexpr int ri = decltype(RI)::value;
    constexpr int S = ri % NS;
    constexpr int SN = (ri + 1) % NS;                    // slot of the next tile
    constexpr int SL = (ri + NS - 1) % NS;               // slot refilled now
    constexpr int WAIT = allowed(RI);
    static_assert(WAIT < 64, "vmcnt range");
    const TileK tk = tile_k(kt + NS - 1);
    read_scales4(ic<S>{});
    static_for<0, SBS>([&](auto SB) {
      constexpr int b = decltype(SB)::value;
      constexpr int cur = (ri * SBS + b) & 1;
      if constexpr (b + 1 < SBS) {
        read_sub(kt, ic<S>{}, ic<b + 1>{}, ic<ri % SPC>{}, F[cur ^ 1], TIAC);
        __builtin_amdgcn_sched_barrier(0);              // keep the prefetch ahead of this sub-block's MFMAs
      }
      mma_sub(F[cur], TIAC, [&](auto JJ) {
        constexpr int jj = decltype(JJ)::value;
        if constexpr (b == 0 && jj == 0 && CH && ri % SPC == 0) {
          __builtin_amdgcn_sched_barrier(0);
          issue_chunk(kt / SPC + 1);                    // the next chunk, ahead of this stage's data loads
          __builtin_amdgcn_sched_barrier(0);
        }
        // LD 6: the B block of tile kt + 1 was loaded three stages ago, before the A loads that
        // the last barrier waited for, so it has landed (loads return in order). Sub-block b
        // converts its 16 values, interleaved with the matrix work (a scheduling barrier keeps
        // each sub-block's conversion in its sub-block: 1% faster than letting it rise into
        // the previous one). The last sub-block writes the block to tile kt + 1's slot before
        // the barrier. Tile kt + 1's A loads and the B register loads of tile kt + 4 go out
        // during sub-block 0.
        if constexpr (NVT && jj == 0) __builtin_amdgcn_sched_barrier(0);
        if constexpr (b == 0 && jj < PJ) {
          __builtin_amdgcn_sched_barrier(0);
          issue_range(tk, ic<SL>{}, ic<(UNITS * jj) / PJ>{}, ic<(UNITS * (jj + 1)) / PJ>{});
          if constexpr (NVT && jj == PJ - 1) nvt_issue(kt + 4, ic<ri % 4>{});
          __builtin_amdgcn_sched_barrier(0);
        }
        // the first 8 values after fragment 0, the other 8 after fragment 1 (no scheduling
        // barrier: the scheduler interleaves them with the MFMAs)
        if constexpr (NVT && jj == 0) nvt_conv(ic<(ri + 1) % 4>{}, ic<b>{}, ic<0>{});
        if constexpr (NVT && jj == 1) {
          nvt_conv(ic<(ri + 1) % 4>{}, ic<b>{}, ic<1>{});
          if constexpr (b + 1 == SBS) {
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, 4>([&](auto BB) { nvt_write(ic<SL>{}, BB); });
          }
        }
        if constexpr (b + 1 == SBS && jj == BJ) {
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (NVT) __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): B writes have landed
          wait_vmcnt<WAIT>();                           // tile kt + 1 has landed (this wave's loads)
          __builtin_amdgcn_s_barrier();                 // ... and every wave's; slot S fully read
          __builtin_amdgcn_sched_barrier(0);
          read_sub(kt + 1, ic<SN>{}, ic<0>{}, ic<(ri + 1) % SPC>{}, F[cur ^ 1], TIAC);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    });
    promote4();
  };

  // prologue: scale chunk 0, tiles 0 .. NS-2 in flight, then the first sub-block's fragments
  issue_chunk(0);
  static_for<0, NS - 1>([&](auto T) { issue_range(tile_k(T.value), T, ic<0>{}, ic<UNITS>{}); });
  if constexpr (NVT) {
    static_assert(NS == 2 && R == 4, "the B register buffers rotate with rounds of four stages over two slots");
    nvt_issue(0, ic<0>{});
    nvt_store(ic<0>{}, ic<0>{});                        // tile 0 into slot 0 (waits for everything)
    nvt_issue(1, ic<1>{});                              // in flight into the first stages
    nvt_issue(2, ic<2>{});
    nvt_issue(3, ic<3>{});
    __builtin_amdgcn_s_waitcnt(0xC07F);
  }
  wait_vmcnt<(NS - 2) * OPS + (NVT ? NB6 : 0)>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // Whole rounds of R stages: stages past the end multiply zeros (their loads are
  // out of range), which adds nothing to the accumulators.
  const int rounds = (nk + R - 1) / R;
  // BF16 tiles sharing a CU: the workgroup in its main loop issues ahead of one in its
  // prologue or FP32 epilogue (DeepSeek expert wgrads 5% faster; no gain measured for the
  // NVFP4 and MXFP8 kernels, which keep equal priorities)
  constexpr bool PRIO = OCC > 1 && LD == 0;
  // main loop for a wave that needs its first TIA 32-row A fragments (the others cover
  // only rows past m_valid: their MFMAs would multiply zeros into rows never stored)
  auto main_loop = [&](auto TIAC) {
    read_sub(0, ic<0>{}, ic<0>{}, ic<0>{}, F[0], TIAC);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
    for (int r = 0; r < rounds; ++r) {
      const int kt = r * R;
      static_for<0, R>([&](auto RI) { stage(kt + RI.value, RI, TIAC); });
    }
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
  };
  if constexpr (PART) {
    // Row-grouped tiles end where their expert does: in an expert's last row tile a wave
    // whose rows are all or mostly padding runs the loop with fewer A fragments (every
    // wave still does its share of the loads, conversions and barriers).
    const int64_t rows_left = p.m_valid - (m0 + wm * (BM / 2));
    const int vg = rows_left <= 0 ? 0 : (int)min((rows_left + 31) / 32, (int64_t)TI);
    if (vg >= TI) main_loop(ic<TI>{});
    else if (vg == 0) main_loop(ic<0>{});
    else if (vg == 1) main_loop(ic<1>{});
    else if (vg == 2) main_loop(ic<(TI > 2 ? 2 : TI)>{});
    else main_loop(ic<TI>{});
  } else {
    main_loop(ic<TI>{});
  }
  wait_vmcnt<0>();                    // no direct load may still target this workgroup's LDS
  exact_drain();

  if constexpr (C::EPI_STAGED) {
    // NVFP4: C = tA tB acc. Each 32-row strip of the wave's block is scaled into LDS, then
    // leaves as 16-byte row segments (measured: 12-40% faster dense NVFP4 GEMMs than
    // scaling and storing element by element; no gain for the other formats).
    __syncthreads();                    // every wave is done with the stage buffers
    constexpr int P = C::EPI_PITCH;
    float* stg = reinterpret_cast<float*>(lds0) + wave * 32 * P;
    const int64_t col0 = n0 + wn * (BN / 2);
    float tbj[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t col = col0 + j * 32 + lr;
      tbj[j] = col < p.n_valid ? (p.tB_mode == 0 ? p.tB[col] : p.tB[0]) : 0.0f;
    }
    const bool vec_ok = (p.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0);
    // tA of the lane's 16 rows of each strip, all loads issued before the first is used
    float ta[TI][16];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * (BM / 2) + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
        const int64_t arow = row < p.m_valid ? exact_src_row(p, row) : -1;
        ta[i][r] = arow < 0 ? 0.0f : p.tA_mode == 0 ? p.tA[arow] : p.tA[0];
      }
    // interior tile with 16-byte aligned rows: no per-chunk checks; each store instruction
    // covers whole staged rows, lane l taking chunk l % CPR of row l / CPR
    const bool interior = vec_ok && m0 + BM <= p.m_valid && n0 + BN <= p.n_valid;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t rbase = m0 + wm * (BM / 2) + i * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = (r / 4) * 8 + h * 4 + (r % 4);
#pragma unroll
        for (int j = 0; j < TJ; ++j) stg[rl * P + j * 32 + lr] = (acc[i][j][r] * ta[i][r]) * tbj[j];
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): this wave's LDS writes landed
      constexpr int CPR = BN / 8;                    // 16-byte chunks per staged row
      constexpr int RPI = 64 / CPR;                  // staged rows per store instruction
      if (interior) {
        const int lrow = lane / CPR, lch = lane % CPR;
        float* dst = p.C + (rbase + lrow) * p.ldc + col0 + 4 * lch;
        const float* src = stg + lrow * P + 4 * lch;
#pragma unroll
        for (int k = 0; k < 32 / RPI; ++k) {
          const float4 v = *reinterpret_cast<const float4*>(src + k * RPI * P);
          const f32x4_nt vv = {v.x, v.y, v.z, v.w};
          __builtin_nontemporal_store(vv, reinterpret_cast<f32x4_nt*>(dst + k * RPI * p.ldc));
        }
      } else {
#pragma unroll
        for (int k = 0; k < 32 * CPR / 64; ++k) {
          const int idx = k * 64 + lane;
          const int rl = idx / CPR, ch = idx % CPR;
          const int64_t row = rbase + rl, col = col0 + ch * 4;
          if (row >= p.m_valid) continue;
          const float4 v = *reinterpret_cast<const float4*>(stg + rl * P + ch * 4);
          float* dstp = p.C + row * p.ldc + col;
          if (vec_ok && col + 4 <= p.n_valid) {
            const f32x4_nt vv = {v.x, v.y, v.z, v.w};
            __builtin_nontemporal_store(vv, reinterpret_cast<f32x4_nt*>(dstp));
          } else {
            if (col < p.n_valid) dstp[0] = v.x;
            if (col + 1 < p.n_valid) dstp[1] = v.y;
            if (col + 2 < p.n_valid) dstp[2] = v.z;
            if (col + 3 < p.n_valid) dstp[3] = v.w;
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);           // reads done before the next strip overwrites
    }
  } else if (m0 + BM <= p.m_valid && n0 + BN <= p.n_valid) {
    // interior tile (the common case): no per-element bounds checks, one row pointer per
    // accumulator row and the TJ column blocks at fixed offsets from it
    float* cw = p.C + (m0 + wm * (BM / 2) + h * 4) * p.ldc + n0 + wn * (BN / 2) + lr;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float* cr = cw + (int64_t)(i * 32 + (r / 4) * 8 + (r % 4)) * p.ldc;
#pragma unroll
        for (int j = 0; j < TJ; ++j) __builtin_nontemporal_store(acc[i][j][r], cr + j * 32);
      }
  } else {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * (BM / 2) + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
        if (row >= p.m_valid) continue;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int64_t col = n0 + wn * (BN / 2) + j * 32 + lr;
          if (col < p.n_valid) __builtin_nontemporal_store(acc[i][j][r], p.C + row * p.ldc + col);
        }
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

// One LDS block per workgroup, carved into the NS stage slots and the scale-chunk buffers
// (and reused by the staged epilogue once the main loop is done).
#define MXQ_EXACT_LDS(C)                                                                         \
  __shared__ __attribute__((aligned(1024))) uint8_t lds_all[C::LDS_TOTAL];                         \
  uint8_t* lds0 = lds_all;                                                                        \
  uint8_t* lds1 = lds_all + C::STAGE;                                                             \
  uint8_t* lds2 = lds_all + 2 * C::STAGE;                                                         \
  uint8_t* lds3 = lds_all + 3 * C::STAGE;                                                         \
  uint8_t* ldsc = lds_all + C::NS * C::STAGE;

template <int LD, int BM, int BN, int SM, bool WIDE>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) exact_dense_kernel(ExactProblem p, int64_t tiles_m, int64_t tiles_n) {
  using C = gx::Cfg<LD, BM, BN, SM, 1, WIDE>;
  MXQ_EXACT_LDS(C)
  int64_t tm, tn;
  if (!exact_map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  exact_gemm_tile<LD, BM, BN, SM, 1, WIDE>(p, tm * BM, tn * BN, lds0, lds1, lds2, lds3, ldsc);
}

// Two workgroups per CU (each half the LDS, two stages): for the blockwise FP8 tiles, whose
// second accumulator set rules out larger tiles, one workgroup's scale FMAs, prologue and
// epilogue overlap the other's main loop (20-30% faster than one workgroup per CU).
template <int LD, int BM, int BN, int SM>
__global__ void __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) exact_dense_occ2_kernel(ExactProblem p, int64_t tiles_m, int64_t tiles_n) {
  using C = gx::Cfg<LD, BM, BN, SM, 2, false>;
  MXQ_EXACT_LDS(C)
  int64_t tm, tn;
  if (!exact_map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  exact_gemm_tile<LD, BM, BN, SM, 2, false>(p, tm * BM, tn * BN, lds0, lds1, lds2, lds3, ldsc);
}

// Several independent dense problems in one launch (e.g. the fprop, dgrad and wgrad GEMMs
// of a layer): workgroups [block0, block0 + 8 ceil(tiles / 8)) belong to job j. The host
// orders jobs by K, longest first, so the long tiles start first and the epilogue stores of
// finished tiles overlap the main loops of others.
constexpr int kMaxBatch = 8;
struct BatchJob {
  ExactProblem p;
  int64_t tiles_m, tiles_n, block0;
};
struct BatchJobs {
  BatchJob j[kMaxBatch];
  int n;
};

template <int LD, int BM, int BN, int SM, bool WIDE>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) exact_batch_kernel(const BatchJobs jobs) {
  using C = gx::Cfg<LD, BM, BN, SM, 1, WIDE>;
  MXQ_EXACT_LDS(C)
  int jsel = 0;
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (i < jobs.n && (int64_t)blockIdx.x >= jobs.j[i].block0) jsel = i;
  int64_t tm = 0, tn = 0;
  ExactProblem p;
  bool ok = false;
  // static indices only: the table stays in kernel arguments
#pragma unroll
  for (int i = 0; i < kMaxBatch; ++i)
    if (i == jsel) {
      p = jobs.j[i].p;
      ok = exact_map_tile((int64_t)blockIdx.x - jobs.j[i].block0, jobs.j[i].tiles_m, jobs.j[i].tiles_n, tm, tn);
    }
  if (!ok) return;
  exact_gemm_tile<LD, BM, BN, SM, 1, WIDE>(p, tm * BM, tn * BN, lds0, lds1, lds2, lds3, ldsc);
}

// The same over 128 x 256 tiles with two workgroups per CU (each workgroup half the LDS):
// one's prologue and FP32 epilogue overlap the other's main loop.
template <int LD, int SM>
__global__ void __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) exact_batch_rect_kernel(const BatchJobs jobs) {
  using C = gx::Cfg<LD, 128, 256, SM, 2, false>;
  MXQ_EXACT_LDS(C)
  int jsel = 0;
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (i < jobs.n && (int64_t)blockIdx.x >= jobs.j[i].block0) jsel = i;
  int64_t tm = 0, tn = 0;
  ExactProblem p;
  bool ok = false;
#pragma unroll
  for (int i = 0; i < kMaxBatch; ++i)
    if (i == jsel) {
      p = jobs.j[i].p;
      ok = exact_map_tile((int64_t)blockIdx.x - jobs.j[i].block0, jobs.j[i].tiles_m, jobs.j[i].tiles_n, tm, tn);
    }
  if (!ok) return;
  exact_gemm_tile<LD, 128, 256, SM, 2, false>(p, tm * 128, tn * 256, lds0, lds1, lds2, lds3, ldsc);
}

// The same for blockwise FP8 (two accumulator sets): 128 x 128 tiles, two workgroups per CU.
template <int LD, int SM>
__global__ void __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) exact_batch_occ2_kernel(const BatchJobs jobs) {
  using C = gx::Cfg<LD, 128, 128, SM, 2, false>;
  MXQ_EXACT_LDS(C)
  int jsel = 0;
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (i < jobs.n && (int64_t)blockIdx.x >= jobs.j[i].block0) jsel = i;
  int64_t tm = 0, tn = 0;
  ExactProblem p;
  bool ok = false;
#pragma unroll
  for (int i = 0; i < kMaxBatch; ++i)
    if (i == jsel) {
      p = jobs.j[i].p;
      ok = exact_map_tile((int64_t)blockIdx.x - jobs.j[i].block0, jobs.j[i].tiles_m, jobs.j[i].tiles_n, tm, tn);
    }
  if (!ok) return;
  exact_gemm_tile<LD, 128, 128, SM, 2, false>(p, tm * 128, tn * 128, lds0, lds1, lds2, lds3, ldsc);
}

// Group of a tile: the largest g with tile_prefix[g] <= tile (tile_prefix is non-decreasing
// and tile < tile_prefix[groups]). Each wave narrows the range 64-fold per round with one
// load per lane and a ballot (two rounds for up to 4096 groups).
__device__ __forceinline__ int64_t find_group(const int64_t* __restrict__ prefix, int64_t groups, int64_t tile) {
  const int lane = threadIdx.x & 63;
  int64_t lo = 0, span = groups;                 // answer in [lo, lo + span)
  while (span > 1) {
    const int64_t step = (span + 63) / 64;
    const int64_t g = lo + (int64_t)lane * step;
    const bool ok = g < lo + span && prefix[g] <= tile;
    const uint64_t m = __ballot(ok);              // lanes 0 .. last are set (lane 0 always)
    const int last = 63 - __builtin_clzll(m);
    const int64_t nlo = lo + (int64_t)last * step;
    span = min(step, lo + span - nlo);
    lo = nlo;
  }
  return lo;
}

// Grouped: tile_prefix[g] = first tile of group g.
//   vary_k = 0: group g covers slots [off[g], off[g+1]), B_g = expert g of a stacked B;
//   vary_k = 1: group g reduces over k in [off[g], off[g+1]) into C_g = C + g*M*N.
// OCC = 2 gives each workgroup half the LDS, so two share a CU and one's prologue and
// epilogue overlap the other's main loop (expert tiles are short in K or in rows).
//
// Row groups (vary_k = 0) are walked XCD by XCD: dispatch order b goes to XCD b % 8, and
// each XCD takes a contiguous run of the logical tile list, so an expert's tiles share
// one L2. Inside a group the tiles go in column bands of kRowGroupBand row tiles: the row
// tiles that read one weight column slab run side by side (Qwen3-shaped gate_up: L2
// misses 1110 -> 275 MB per launch and 9% faster; DeepSeek-shaped fused dgrads 3-4%
// faster). Weight gradients (vary_k = 1) keep the plain order: there the XCD runs made
// the kernels 2-14% slower (their time goes to the FP32 output stores, not to reads).
constexpr int kRowGroupBand = 4;
template <int LD, int BM, int BN, int SM, int OCC, bool WIDE, bool AKM = false>
__global__ void __launch_bounds__(256, OCC) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
exact_grouped_kernel(ExactProblem base, const int64_t* __restrict__ offsets, const int64_t* __restrict__ tile_prefix,
                     int64_t groups, int vary_k, int64_t M, int64_t N, int64_t tiles_n) {
  using C = gx::Cfg<LD, BM, BN, SM, OCC, WIDE>;
  MXQ_EXACT_LDS(C)
  const int64_t total = tile_prefix[groups];
  int64_t tile = blockIdx.x;
  if (!vary_k) {
    const int64_t T8 = (total + 7) / 8;
    if (tile >= 8 * T8) return;                     // the grid may exceed the tile count
    tile = (tile % 8) * T8 + tile / 8;
  }
  if (tile >= total) return;
  // weight gradients: every group has the same tiles_m x tiles_n tiles (the prefix is g times
  // that, or all zero when the offsets were rejected), so the group needs no search
  const int64_t per_group = (M + BM - 1) / BM * tiles_n;
  const int64_t g = vary_k ? tile / per_group : find_group(tile_prefix, groups, tile);
  const int64_t local = vary_k ? tile - g * per_group : tile - tile_prefix[g];
  int64_t tm = local / tiles_n, tn = local % tiles_n;
  if (!vary_k) {
    const int64_t tiles_m = (tile_prefix[g + 1] - tile_prefix[g]) / tiles_n;
    const int64_t band = local / (kRowGroupBand * tiles_n);
    const int64_t rows_in_band = min((int64_t)kRowGroupBand, tiles_m - band * kRowGroupBand);
    const int64_t idx = local - band * kRowGroupBand * tiles_n;
    tm = band * kRowGroupBand + idx % rows_in_band;
    tn = idx / rows_in_band;
  }
  ExactProblem p = base;
  if (!vary_k) {
    p.a_base = offsets[g];
    p.m_valid = offsets[g + 1] - offsets[g];
    const int64_t b_elems = g * N * base.ldb;
    p.B = base.B + k_bytes<LD>(b_elems);
    if constexpr (LD == 6) {                      // group g's weight: K rows of N (= ldb) NVFP4 elements
      const int64_t w_elems = g * base.k_end * base.ldb;
      p.B = base.B + w_elems / 2;
      p.sB = base.sB + w_elems / 16;
      p.tB = base.tB + g;
    }
    if (LD == 1 || LD == 3) p.sB = base.sB + b_elems / 32;
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
  // the expert-tail specialization pays on the converting forward formats (NVFP4 gate_up /
  // down 3-6% faster); the BF16 kernels at one workgroup per CU measured no gain from it
  constexpr bool PART = LD != 0 && LD != 6;
  exact_gemm_tile<LD, BM, BN, SM, OCC, WIDE, AKM, PART>(p, tm * BM, tn * BN, lds0, lds1, lds2, lds3, ldsc);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

static int pick_tile(int64_t M, int64_t N) {
  // 256 x 256 unless that leaves most of the 256 CUs idle; then 128 x 128.
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  return t256 >= 192 ? 256 : 128;
}

template <int LD, int BT, int SM>
static void launch_dense_t(const ExactProblem& p, int64_t M, int64_t N, hipStream_t st) {
  const int64_t tm = (M + BT - 1) / BT, tn = (N + BT - 1) / BT;
  const int64_t blocks = (tm * tn + 7) / 8 * 8;
  constexpr bool WIDE = SM == 2 && LD != 0;       // measured: 3-6% faster dense tiles
  hipLaunchKernelGGL((exact_dense_kernel<LD, BT, BT, SM, WIDE>), dim3((unsigned)blocks), dim3(256), 0, st, p, tm, tn);
}

// Scale mode: 2 when K % 64 == 0 and every scale row starts 16-byte aligned
// (K % 512 == 0 for MXFP8 / MXFP4, K % 256 == 0 for NVFP4), 1 when K % 64 == 0, else 0.
static int scale_mode(int ld, int64_t K, bool vary_k) {
  if (ld == 5) return K % 512 == 0 ? 2 : K % 128 == 0 ? 1 : 0;   // 128-K stages
  if (vary_k || K % 64) return 0;
  if ((ld == 1 || ld == 3) && K % 512 == 0) return 2;
  if (ld == 2 && K % 256 == 0) return 2;
  return 1;
}

template <int LD, int BT>
static void launch_dense_bt(const ExactProblem& p, int64_t M, int64_t N, int sm, hipStream_t st) {
  if constexpr (LD != 0) {
    if (sm == 2) { launch_dense_t<LD, BT, 2>(p, M, N, st); return; }
  }
  if (sm == 2) launch_dense_t<LD, BT, 1>(p, M, N, st);
  else if (sm == 1) launch_dense_t<LD, BT, 1>(p, M, N, st);
  else launch_dense_t<LD, BT, 0>(p, M, N, st);
}

template <int LD>
static void launch_dense_ld(const ExactProblem& p, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int sm = scale_mode(LD, K, false);
  if (pick_tile(M, N) == 256) launch_dense_bt<LD, 256>(p, M, N, sm, st);
  else launch_dense_bt<LD, 128>(p, M, N, sm, st);
}

hipError_t launch_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* A, const void* sA, const float* tA,
                       int tA_mode, const void* B, const void* sB, const float* tB, int tB_mode, float* C,
                       int64_t ldc, hipStream_t st) {
  ExactProblem p;
  p.A = (const uint8_t*)A; p.sA = (const uint8_t*)sA; p.tA = tA; p.tA_mode = tA_mode;
  p.a_idx = nullptr; p.a_rows = M; p.a_base = 0; p.m_valid = M; p.lda = K;
  p.B = (const uint8_t*)B; p.sB = (const uint8_t*)sB; p.tB = tB; p.tB_mode = tB_mode; p.n_valid = N; p.ldb = K;
  p.k_begin = 0; p.k_end = K; p.C = C; p.ldc = ldc;
  // fmt: 1 MXFP8, 2 NVFP4, 3 BF16, 4 MXFP4, 5 blockwise FP8 (tB_mode: 0 per B row, 1 per
  // 128 x 128 block; 128 x 128 tiles, K % 128 == 0), 6 MXFP8 on the scaled FP8 MFMA
  if (fmt == 5) {
    const int64_t tm = (M + 127) / 128, tn = (N + 127) / 128;
    hipLaunchKernelGGL((exact_dense_occ2_kernel<4, 128, 128, 1>), dim3((unsigned)((tm * tn + 7) / 8 * 8)), dim3(256), 0,
                       st, p, tm, tn);
  }
  else if (fmt == 6) launch_dense_ld<5>(p, M, N, K, st);      // MXFP8 on the scaled FP8 MFMA
  else if (fmt == 1) launch_dense_ld<1>(p, M, N, K, st);
  else if (fmt == 2) launch_dense_ld<2>(p, M, N, K, st);
  else if (fmt == 4) launch_dense_ld<3>(p, M, N, K, st);
  else launch_dense_ld<0>(p, M, N, K, st);
  return hipGetLastError();
}

hipError_t launch_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* A, const void* sA, const float* tA,
                       int tA_mode, const void* B, const void* sB, const float* tB, int tB_mode, float* C,
                       int64_t ldc, hipStream_t st);

// Batched dense GEMMs of one format: one launch, jobs ordered by K (longest first), one
// tile size and scale mode for all (the largest the batch allows). With 256 x 256 tiles, a
// job that would cover fewer than 128 of them (too few to share the CUs with the others
// for long) runs as its own launch with the single-problem tile rule instead.
hipError_t launch_gemm_batch(int fmt, int n, const int64_t* M, const int64_t* N, const int64_t* K,
                             const void* const* A, const void* const* sA, const float* const* tA, const int* tA_mode,
                             const void* const* B, const void* const* sB, const float* const* tB, const int* tB_mode,
                             float* const* C, const int64_t* ldc, hipStream_t st) {
  const int ld = fmt == 1 ? 1 : fmt == 2 ? 2 : fmt == 4 ? 3 : fmt == 5 ? 4 : 0;
  int order[kMaxBatch];
  for (int i = 0; i < n; ++i) order[i] = i;
  for (int i = 1; i < n; ++i)                          // insertion sort, K descending (stable)
    for (int k = i; k > 0 && K[order[k]] > K[order[k - 1]]; --k) std::swap(order[k], order[k - 1]);
  if (ld == 4) {
    // blockwise FP8 (fmt 5, tB_mode = b_blocks): every problem on the single call's 128 x 128
    // tiles at two workgroups per CU, so a long-K problem (a layer's dgrad) shares the CUs
    // with the others instead of leaving half the slots idle
    BatchJobs jobs;
    jobs.n = 0;
    int64_t blocks = 0;
    for (int q = 0; q < n; ++q) {
      const int i = order[q];
      ExactProblem& p = jobs.j[jobs.n].p;
      p.A = (const uint8_t*)A[i]; p.sA = (const uint8_t*)sA[i]; p.tA = nullptr; p.tA_mode = 0;
      p.a_idx = nullptr; p.a_rows = M[i]; p.a_base = 0; p.m_valid = M[i]; p.lda = K[i];
      p.B = (const uint8_t*)B[i]; p.sB = (const uint8_t*)sB[i]; p.tB = nullptr; p.tB_mode = tB_mode[i];
      p.n_valid = N[i]; p.ldb = K[i];
      p.k_begin = 0; p.k_end = K[i]; p.C = C[i]; p.ldc = ldc[i];
      jobs.j[jobs.n].tiles_m = (M[i] + 127) / 128;
      jobs.j[jobs.n].tiles_n = (N[i] + 127) / 128;
      jobs.j[jobs.n].block0 = blocks;
      blocks += (jobs.j[jobs.n].tiles_m * jobs.j[jobs.n].tiles_n + 7) / 8 * 8;
      ++jobs.n;
    }
    if (blocks > 0) hipLaunchKernelGGL((exact_batch_occ2_kernel<4, 1>), dim3((unsigned)blocks), dim3(256), 0, st, jobs);
    return hipGetLastError();
  }
  int64_t t256 = 0;
  for (int i = 0; i < n; ++i) t256 += ((M[i] + 255) / 256) * ((N[i] + 255) / 256);
  const int bt = t256 >= 192 ? 256 : 128;
  // MXFP8 with 16-byte scale chunks (every K % 512 == 0) and a few 256-tiles per CU: every
  // problem on 128 x 256 tiles at two workgroups per CU, none alone (the linear layer's
  // three GEMMs: 6% faster than 256 x 256 tiles plus a separate 128 x 128 dgrad). Batches of
  // four or more 256-tiles per CU (three 8192^3 GEMMs) keep the 256 x 256 tiles.
  int sm_all = 2;
  for (int i = 0; i < n; ++i) sm_all = std::min(sm_all, scale_mode(ld, K[i], false));
  const bool rect = ld == 1 && sm_all == 2 && t256 >= 192 && t256 < 1024;
  bool alone[kMaxBatch];
  int sm = 2, nb = 0;
  for (int i = 0; i < n; ++i) {
    alone[i] = !rect && bt == 256 && ((M[i] + 255) / 256) * ((N[i] + 255) / 256) < 128;
    if (!alone[i]) { sm = std::min(sm, scale_mode(ld, K[i], false)); ++nb; }
  }
  BatchJobs jobs;
  jobs.n = 0;
  int64_t blocks = 0;
  for (int q = 0; q < n; ++q) {
    const int i = order[q];
    if (alone[i]) continue;
    const int qq = jobs.n++;
    ExactProblem& p = jobs.j[qq].p;
    p.A = (const uint8_t*)A[i]; p.sA = (const uint8_t*)sA[i]; p.tA = tA[i]; p.tA_mode = tA_mode[i];
    p.a_idx = nullptr; p.a_rows = M[i]; p.a_base = 0; p.m_valid = M[i]; p.lda = K[i];
    p.B = (const uint8_t*)B[i]; p.sB = (const uint8_t*)sB[i]; p.tB = tB[i]; p.tB_mode = tB_mode[i];
    p.n_valid = N[i]; p.ldb = K[i];
    p.k_begin = 0; p.k_end = K[i]; p.C = C[i]; p.ldc = ldc[i];
    jobs.j[qq].tiles_m = (M[i] + (rect ? 128 : bt) - 1) / (rect ? 128 : bt);
    jobs.j[qq].tiles_n = (N[i] + (rect ? 256 : bt) - 1) / (rect ? 256 : bt);
    jobs.j[qq].block0 = blocks;
    blocks += (jobs.j[qq].tiles_m * jobs.j[qq].tiles_n + 7) / 8 * 8;    // XCD-aware raster per job
  }
  for (int q = 0; q < n; ++q) {                       // the jobs that run alone, longest K first
    const int i = order[q];
    if (!alone[i]) continue;
    const hipError_t e = launch_gemm(fmt, M[i], N[i], K[i], A[i], sA[i], tA[i], tA_mode[i], B[i], sB[i], tB[i],
                                     tB_mode[i], C[i], ldc[i], st);
    if (e != hipSuccess) return e;
  }
  if (nb == 0 || blocks == 0) return hipGetLastError();
  if (rect) {
    hipLaunchKernelGGL((exact_batch_rect_kernel<1, 2>), dim3((unsigned)blocks), dim3(256), 0, st, jobs);
    return hipGetLastError();
  }
  auto go = [&](auto LDC, auto BTC, auto SMC) {
    constexpr int L = decltype(LDC)::value, T = decltype(BTC)::value, S = decltype(SMC)::value;
    constexpr bool WIDE = S == 2 && L != 0;
    hipLaunchKernelGGL((exact_batch_kernel<L, T, T, S, WIDE>), dim3((unsigned)blocks), dim3(256), 0, st, jobs);
  };
  auto by_sm = [&](auto LDC, auto BTC) {
    if constexpr (decltype(LDC)::value != 0) {
      if (sm == 2) { go(LDC, BTC, ic<2>{}); return; }
    }
    if (sm >= 1) go(LDC, BTC, ic<1>{});
    else go(LDC, BTC, ic<0>{});
  };
  auto by_bt = [&](auto LDC) {
    if (bt == 256) by_sm(LDC, ic<256>{});
    else by_sm(LDC, ic<128>{});
  };
  if (ld == 1) by_bt(ic<1>{});
  else if (ld == 2) by_bt(ic<2>{});
  else if (ld == 3) by_bt(ic<3>{});
  else by_bt(ic<0>{});
  return hipGetLastError();
}

// One wave: checks that the offsets partition [0, total) (aligned to `align` when they
// split the reduction axis) and writes the exclusive prefix of the per-group tile counts,
// 64 groups per round (lane scan with shuffles). Invalid offsets give an all-zero prefix,
// so no tile runs.
__global__ void __launch_bounds__(64) tile_prefix_kernel(const int64_t* __restrict__ offsets, int64_t groups,
                                                         int64_t total, int vary_k, int64_t align, int64_t bm,
                                                         int64_t tiles_m_fixed, int64_t tiles_n,
                                                         int64_t* __restrict__ prefix) {
  const int lane = threadIdx.x;
  bool bad = false;
  for (int64_t g0 = 0; g0 < groups; g0 += 64) {
    const int64_t g = g0 + lane;
    if (g < groups) {
      const int64_t a = offsets[g], b = offsets[g + 1];
      bad = bad || b < a || (vary_k && (a % align != 0));
    }
  }
  bad = bad || offsets[0] != 0 || offsets[groups] != total;
  const bool ok = __ballot(bad) == 0;
  int64_t carry = 0;
  for (int64_t g0 = 0; g0 < groups; g0 += 64) {
    const int64_t g = g0 + lane;
    int64_t cnt = 0;
    if (g < groups) cnt = vary_k ? tiles_m_fixed : (offsets[g + 1] - offsets[g] + bm - 1) / bm;
    cnt *= tiles_n;
    int64_t incl = cnt;                                   // inclusive scan over the 64 lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (g < groups) prefix[g] = ok ? carry + incl - cnt : 0;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) prefix[groups] = ok ? carry : 0;
}

size_t grouped_gemm_ws_bytes(int64_t groups) { return (size_t)(((groups + 1) * 8 + 255) / 256 * 256); }

template <int LD, int BT, int SM, bool AKM = false>
static void launch_grouped_t(const ExactProblem& p, const int64_t* offsets, const int64_t* prefix, int64_t max_tiles,
                             int64_t groups, int vary_k, int64_t M, int64_t N, hipStream_t st) {
  const int64_t tn = (N + BT - 1) / BT;
  // expert tiles keep the narrow stages: wide NVFP4 stages leave two LDS stages at half LDS.
  // 128 x 128 tiles run two workgroups per CU, 256 x 256 tiles one.
  constexpr int OCC = BT == 256 ? 1 : 2;
  hipLaunchKernelGGL((exact_grouped_kernel<LD, BT, BT, SM, OCC, false, AKM>), dim3((unsigned)max_tiles), dim3(256), 0, st,
                     p, offsets, prefix, groups, vary_k, M, N, tn);
}

// Row-grouped NVFP4 with chunked scales: 128-row tiles keep the expert padding small,
// 256 columns halve the A re-reads, two workgroups per CU.
template <int SM>
static void launch_grouped_nv_rect(const ExactProblem& p, const int64_t* offsets, const int64_t* prefix,
                                   int64_t max_tiles, int64_t groups, int64_t M, int64_t N, hipStream_t st) {
  const int64_t tn = (N + 255) / 256;
  hipLaunchKernelGGL((exact_grouped_kernel<2, 128, 256, SM, 2, false>), dim3((unsigned)max_tiles), dim3(256), 0, st, p,
                     offsets, prefix, groups, 0, M, N, tn);
}

hipError_t launch_grouped_gemm(int fmt, int64_t groups, const int64_t* offsets, int vary_k, int64_t total, int64_t M,
                               int64_t N, int64_t K, const int32_t* a_row_index, int64_t a_rows, const void* A,
                               const void* sA, const float* tA, int tA_mode, const void* B, const void* sB,
                               const float* tB, int tB_mode, float* C, void* ws, hipStream_t st) {
  int64_t* prefix = (int64_t*)ws;
  // Expert groups are small (hundreds of rows): 128 x 128 tiles. A weight gradient
  // (vary_k) has the full (M, N) output per group: 256 x 256 tiles once that gives each
  // group at least 64 of them. BF16 row groups averaging 384 rows or more also take
  // 256 x 256 tiles: their per-flop speed outweighs the extra row padding there (DeepSeek
  // expert dgrads, ~527 rows per expert: 7% faster). NVFP4 showed no gain.
  const bool big_rows = (fmt == 3 || fmt == 7) && !vary_k && groups > 0 && total / groups >= 384;
  // Row-grouped NVFP4 with chunked scales: 128 x 256 tiles (DeepSeek expert gate_up 12%
  // faster than 128 x 128, Qwen3 8%).
  const bool nv_rect = fmt == 2 && !vary_k && scale_mode(2, K, false) == 2;
  // Weight gradients (vary_k) with large outputs: 256 x 256 tiles. (With the unguarded
  // interior-tile epilogue the DeepSeek expert wgrads run 5% faster on them than on 128 x 256
  // tiles at two workgroups per CU; with per-element guarded stores it was the reverse.)
  const bool wide_out = vary_k && ((M + 255) / 256) * ((N + 255) / 256) >= 64;
  const int BT = fmt == 7 ? 256 : (wide_out || big_rows) ? 256 : 128;
  const int BTN = nv_rect ? 256 : BT;
  const int64_t tiles_n = (N + BTN - 1) / BTN;
  const int64_t tiles_m_fixed = vary_k ? (M + BT - 1) / BT : 0;
  const int64_t align = (fmt == 1 || fmt == 4) ? 32 : fmt == 2 ? 16 : 8;
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(64), 0, st, offsets, groups, total, vary_k, align, (int64_t)BT,
                     tiles_m_fixed, tiles_n, prefix);
  // Row groups: an upper bound on the tiles (the device prefix holds the count), rounded
  // up to a multiple of 8 so that the XCD-contiguous order reaches every logical tile
  // below 8 ceil(tiles / 8) (the kernel maps dispatch index b to (b % 8) ceil(tiles / 8) + b / 8).
  const int64_t max_tiles = vary_k ? groups * tiles_m_fixed * tiles_n
                                   : ((((total + BT - 1) / BT + groups) * tiles_n + 7) / 8) * 8;
  if (max_tiles <= 0) return hipGetLastError();
  ExactProblem p;
  p.A = (const uint8_t*)A; p.sA = (const uint8_t*)sA; p.tA = tA; p.tA_mode = tA_mode;
  p.a_idx = a_row_index; p.a_rows = a_rows; p.a_base = 0;
  p.B = (const uint8_t*)B; p.sB = (const uint8_t*)sB; p.tB = tB; p.tB_mode = tB_mode; p.C = C; p.ldc = N;
  if (!vary_k) {
    p.m_valid = 0; p.lda = K; p.n_valid = N; p.ldb = K; p.k_begin = 0; p.k_end = K;
  } else {
    // vary_k 2: A is given K-major, (total, M) row-major (the slot-major gradient itself)
    p.m_valid = M; p.lda = vary_k == 2 ? M : total; p.n_valid = N; p.ldb = total; p.k_begin = 0; p.k_end = 0;
  }
  if (vary_k == 2) {
    if (BT == 256) launch_grouped_t<0, 256, 0, true>(p, offsets, prefix, max_tiles, groups, vary_k, M, N, st);
    else launch_grouped_t<0, 128, 0, true>(p, offsets, prefix, max_tiles, groups, vary_k, M, N, st);
    return hipGetLastError();
  }
  if (fmt == 7) {
    // BF16 A x the stacked NVFP4 weights (K, N) per group, read transposed: B_g[n][k] is the
    // BF16 dequantization of W_g[k][n], built in the loader (no BF16 weight copy in HBM)
    p.ldb = N;
    const int64_t tn = (N + 255) / 256;
    hipLaunchKernelGGL((exact_grouped_kernel<6, 256, 256, 0, 1, false>), dim3((unsigned)max_tiles), dim3(256), 0, st, p,
                       offsets, prefix, groups, 0, M, N, tn);
    return hipGetLastError();
  }
  const int ld = fmt == 1 ? 1 : fmt == 2 ? 2 : fmt == 4 ? 3 : 0;
  const int sm = scale_mode(ld, p.lda, vary_k != 0);
  auto go = [&](auto LDC, auto SMC) {
    constexpr int L = decltype(LDC)::value, S = decltype(SMC)::value;
    if constexpr (L == 0 || (S == 0 && L != 2)) {   // 256 tiles: BF16, or vary_k (SM 0, never NVFP4)
      if (BT == 256) {
        launch_grouped_t<L, 256, S>(p, offsets, prefix, max_tiles, groups, vary_k, M, N, st);
        return;
      }
    }
    launch_grouped_t<L, 128, S>(p, offsets, prefix, max_tiles, groups, vary_k, M, N, st);
  };
  auto by_sm = [&](auto LDC) {
    if constexpr (decltype(LDC)::value != 0) {
      if (sm == 2) { go(LDC, ic<2>{}); return; }
    }
    if (sm == 2) go(LDC, ic<1>{});
    else if (sm == 1) go(LDC, ic<1>{});
    else go(LDC, ic<0>{});
  };
  if (ld == 1) by_sm(ic<1>{});
  else if (ld == 2 && nv_rect) launch_grouped_nv_rect<2>(p, offsets, prefix, max_tiles, groups, M, N, st);
  else if (ld == 2) by_sm(ic<2>{});
  else if (ld == 3) by_sm(ic<3>{});
  else by_sm(ic<0>{});
  return hipGetLastError();
}

}  // namespace mxq
