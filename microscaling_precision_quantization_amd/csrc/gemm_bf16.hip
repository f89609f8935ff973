// GEMMs on the gfx950 BF16 MFMA (v_mfma_f32_32x32x16_bf16), whose products and
// accumulation are FP32-grade (measured on MI355X: a sum of 2^20 and 2^-3 is
// exact at every operand position). Every operand value is formed EXACTLY in
// BF16 while a tile is staged into LDS, so the results carry only FP32
// accumulation error:
//   * MXFP8 x MXFP8: E4M3 * 2^(s - 127) has 4 significant bits, exact in BF16
//     (the gfx950 scaled convert applies the E8M0 scale), so C = A_hat B_hat^T
//     within FP32 accumulation error. The native scaled FP8 MFMA is faster but
//     sums each group of 8 consecutive K products in a ~13-bit window under the
//     group's largest product (measured), which exceeds the 2e-5 normwise bound
//     on outlier-heavy data; it is offered separately (gemm_mxfp8_matrix_core).
//   * NVFP4 x NVFP4: C[m, n] = tA[m] tB[n] * sum_k (qA SA)[m, k] (qB SB)[n, k].
//     An E2M1 value times its E4M3 block scale has at most 6 significant bits
//     and lies in [2^-10, 2688], so it is EXACT in BF16; the loader forms these
//     products while staging tiles into LDS, the MFMA accumulates them in FP32,
//     and the FP32 second-level scales are applied in the epilogue. (NVFP4's
//     E4M3 scale per 16 values does not match the matrix core's E8M0 scale per
//     32, so the FP4 scaled MFMA cannot consume NVFP4 exactly.) Defined by the
//     two-level NVFP4 format (7minutos.es, section "Que es realmente NVFP4";
//     remio.ai "Miles Blackwell RL", section "La Compatibilidad ...").
//   * BF16 x BF16: the dequantized-backward GEMMs and the higher-precision
//     shared expert (remio.ai, sections "La Compatibilidad ..." and "NVFP4 por
//     token cuestiona el valor predeterminado uniforme de BF16").
//
// BF16 operand layout of the 32x32x16 MFMA (measured): lane l supplies row
// l % 32, elements k = 8 (l / 32) .. +8 (16 bytes). Accumulator layout as for
// every 32x32 MFMA: C[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32].
//
// Tiling: 256 x 256 workgroup tile, four waves of 128 x 128, K tile 64 (BF16 in
// LDS: 128 bytes per row, same 16-byte XOR swizzle as the FP8 kernel), double
// buffered.
#include "common.h"

namespace mxq {

namespace gb {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int ROW_BYTES = BK * 2;                  // 128
constexpr int TILE_BYTES = BM * ROW_BYTES;         // 32 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
}  // namespace gb

struct Bf16Problem {
  int fmt;                 // 1 = MXFP8, 2 = NVFP4, 3 = BF16
  const uint8_t* A;        // MXFP8: E4M3 (rows, lda); NVFP4: packed (rows, lda/2); BF16: (rows, lda) BF16
  const uint8_t* sA;       // MXFP8 E8M0 (rows, lda/32); NVFP4 E4M3 (rows, lda/16)
  const float* tA;         // NVFP4 decode scales
  int tA_mode;             // 0 per A row (after gather), 1 tensor
  const int32_t* a_idx;
  int64_t a_rows;          // gather indices outside [0, a_rows) read as zero rows
  int64_t a_base, m_valid, lda;
  const uint8_t* B;
  const uint8_t* sB;
  const float* tB;
  int tB_mode;             // 0 per B row, 1 tensor, 2 per group (tB already offset to the group)
  int64_t n_valid, ldb;
  int64_t k_begin, k_end;
  float* C;
  int64_t ldc;
};

__device__ __forceinline__ int64_t a_source_row_b(const Bf16Problem& p, int64_t r) {
  if (!p.a_idx) return p.a_base + r;
  const int64_t ar = p.a_idx[p.a_base + r];
  return (ar >= 0 && ar < p.a_rows) ? ar : -1;
}

__device__ __forceinline__ int lds_off_b(int row, int chunk) { return row * gb::ROW_BYTES + ((chunk ^ (row & 7)) << 4); }

// --- loaders: registers hold the raw global data of one K tile -------------
// LD = 0 BF16: thread t loads rows i*32 + t/8 (i = 0..7), 16-byte chunk t % 8.
// LD = 1 MXFP8: thread t loads rows i*64 + t/4 (i = 0..3), the 16 E4M3 bytes
//        of quarter t % 4 and their E8M0 scale byte.
// LD = 2 NVFP4: thread t loads rows i*64 + t/4 (i = 0..3), 8 bytes (16 values,
//        one scale block) at quarter t % 4, plus that block's E4M3 scale byte.
struct RawTile {
  uint4 b[8];
  uint32_t s[4];
};

template <int LD>
__device__ __forceinline__ void load_raw(RawTile& r, const uint8_t* base, const uint8_t* sbase, const int64_t* row_el,
                                         const bool* ok, int64_t ld, int64_t k0, int64_t k_end, int tid) {
  if (LD == 0) {
    const int64_t k = k0 + (tid & 7) * 8;
    const bool kok = k < k_end;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r.b[i] = (ok[i] && kok) ? *reinterpret_cast<const uint4*>(base + (row_el[i] * ld + k) * 2) : make_uint4(0, 0, 0, 0);
  } else if (LD == 1) {
    const int64_t k = k0 + (tid & 3) * 16;
    const bool kok = k < k_end;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool v = ok[i] && kok;
      r.b[i] = v ? *reinterpret_cast<const uint4*>(base + row_el[i] * ld + k) : make_uint4(0, 0, 0, 0);
      r.s[i] = v ? sbase[(row_el[i] * ld + k) / 32] : 127u;
    }
  } else {
    const int64_t k = k0 + (tid & 3) * 16;
    const bool kok = k < k_end;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool v = ok[i] && kok;
      const uint2 d = v ? *reinterpret_cast<const uint2*>(base + (row_el[i] * ld + k) / 2) : make_uint2(0, 0);
      r.b[i] = make_uint4(d.x, d.y, 0, 0);
      r.s[i] = v ? sbase[(row_el[i] * ld + k) / 16] : 0u;
    }
  }
}

// Two E4M3 bytes (word `hi` of w) -> two BF16, each exactly q * 2^(s-127).
__device__ __forceinline__ uint32_t bf16_pair_from_fp8(uint32_t w, float scale, bool hi) {
  v2bf r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, false);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

__device__ __forceinline__ uint32_t bf16_pair_from_fp4(uint32_t byte, float S) {
  const float lo = e2m1_to_f32(byte & 0xF) * S, hi = e2m1_to_f32((byte >> 4) & 0xF) * S;   // exact
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

template <int LD>
__device__ __forceinline__ void store_raw_lds(uint8_t* lds, const RawTile& r, int tid) {
  if (LD == 0) {
    const int chunk = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 32 + (tid >> 3);
      *reinterpret_cast<uint4*>(lds + lds_off_b(row, chunk)) = r.b[i];
    }
  } else if (LD == 1) {
    const int q = tid & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 64 + (tid >> 2);
      const float sc = e8m0_to_float(r.s[i]);
      uint4 c0, c1;
      c0.x = bf16_pair_from_fp8(r.b[i].x, sc, false);
      c0.y = bf16_pair_from_fp8(r.b[i].x, sc, true);
      c0.z = bf16_pair_from_fp8(r.b[i].y, sc, false);
      c0.w = bf16_pair_from_fp8(r.b[i].y, sc, true);
      c1.x = bf16_pair_from_fp8(r.b[i].z, sc, false);
      c1.y = bf16_pair_from_fp8(r.b[i].z, sc, true);
      c1.z = bf16_pair_from_fp8(r.b[i].w, sc, false);
      c1.w = bf16_pair_from_fp8(r.b[i].w, sc, true);
      *reinterpret_cast<uint4*>(lds + lds_off_b(row, 2 * q)) = c0;
      *reinterpret_cast<uint4*>(lds + lds_off_b(row, 2 * q + 1)) = c1;
    }
  } else {
    const int q = tid & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 64 + (tid >> 2);
      const float S = e4m3_to_f32(r.s[i]);
      const uint32_t w0 = r.b[i].x, w1 = r.b[i].y;
      uint4 c0, c1;
      c0.x = bf16_pair_from_fp4(w0 & 0xFF, S);
      c0.y = bf16_pair_from_fp4((w0 >> 8) & 0xFF, S);
      c0.z = bf16_pair_from_fp4((w0 >> 16) & 0xFF, S);
      c0.w = bf16_pair_from_fp4(w0 >> 24, S);
      c1.x = bf16_pair_from_fp4(w1 & 0xFF, S);
      c1.y = bf16_pair_from_fp4((w1 >> 8) & 0xFF, S);
      c1.z = bf16_pair_from_fp4((w1 >> 16) & 0xFF, S);
      c1.w = bf16_pair_from_fp4(w1 >> 24, S);
      *reinterpret_cast<uint4*>(lds + lds_off_b(row, 2 * q)) = c0;
      *reinterpret_cast<uint4*>(lds + lds_off_b(row, 2 * q + 1)) = c1;
    }
  }
}

__device__ __forceinline__ v8bf lds_frag_bf16(const uint8_t* lds, int row, int chunk) {
  const uint4 a = *reinterpret_cast<const uint4*>(lds + lds_off_b(row, chunk));
  v8bf f;
  __builtin_memcpy(&f, &a, 16);
  return f;
}

__device__ __forceinline__ void bf16_mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int LD>
__device__ void gemm_bf16_tile(const Bf16Problem& p, int64_t m0, int64_t n0, uint8_t* lds) {
  using namespace gb;
  constexpr bool NV = LD == 2;
  constexpr bool Q4 = LD != 0;         // quarter-row loaders (4 rows of 64 per thread)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, lr = lane & 31;

  int64_t a_row[8], b_row[8];
  bool a_ok[8], b_ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = m0 + (Q4 ? i * 64 + (tid >> 2) : i * 32 + (tid >> 3));
    const int64_t ar = ((Q4 && i >= 4) || r >= p.m_valid) ? -1 : a_source_row_b(p, r);
    a_ok[i] = ar >= 0;
    a_row[i] = a_ok[i] ? ar : 0;
    const int64_t n = n0 + (Q4 ? i * 64 + (tid >> 2) : i * 32 + (tid >> 3));
    b_ok[i] = (Q4 && i >= 4) ? false : n < p.n_valid;
    b_row[i] = b_ok[i] ? n : 0;
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t kb = p.k_begin, ke = p.k_end;
  const int64_t nk = (ke - kb + BK - 1) / BK;
  RawTile ra, rb;
  if (nk > 0) {
    load_raw<LD>(ra, p.A, p.sA, a_row, a_ok, p.lda, kb, ke, tid);
    load_raw<LD>(rb, p.B, p.sB, b_row, b_ok, p.ldb, kb, ke, tid);
    store_raw_lds<LD>(lds, ra, tid);
    store_raw_lds<LD>(lds + TILE_BYTES, rb, tid);
  }
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * STAGE_BYTES;
    uint8_t* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t k1 = kb + (kt + 1) * BK;
      load_raw<LD>(ra, p.A, p.sA, a_row, a_ok, p.lda, k1, ke, tid);
      load_raw<LD>(rb, p.B, p.sB, b_row, b_ok, p.ldb, k1, ke, tid);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v8bf fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = lds_frag_bf16(cur, wm * 128 + i * 32 + lr, 2 * t + h);
        fb[i] = lds_frag_bf16(cur + TILE_BYTES, wn * 128 + i * 32 + lr, 2 * t + h);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_raw_lds<LD>(nxt, ra, tid);
      store_raw_lds<LD>(nxt + TILE_BYTES, rb, tid);
    }
    __syncthreads();
  }
  bf16_mfma_drain();

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t col = n0 + wn * 128 + j * 32 + lr;
    if (col >= p.n_valid) continue;
    float tb = 1.0f;
    if (NV) tb = p.tB_mode == 0 ? p.tB[col] : p.tB[0];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
        if (row >= p.m_valid) continue;
        float v = acc[i][j][r];
        if (NV) {
          const int64_t arow = a_source_row_b(p, row);
          const float ta = arow < 0 ? 0.0f : p.tA_mode == 0 ? p.tA[arow] : p.tA[0];
          v = (v * ta) * tb;
        }
        p.C[row * p.ldc + col] = v;
      }
  }
}

__device__ __forceinline__ bool map_tile_b(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
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

template <int LD>
__global__ void __launch_bounds__(256, 1) gemm_bf16_dense_kernel(Bf16Problem p, int64_t tiles_m, int64_t tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * gb::STAGE_BYTES];
  int64_t tm, tn;
  if (!map_tile_b(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  gemm_bf16_tile<LD>(p, tm * gb::BM, tn * gb::BN, lds);
}

template <int LD>
__global__ void __launch_bounds__(256, 1)
gemm_bf16_grouped_kernel(Bf16Problem base, const int64_t* __restrict__ offsets, const int64_t* __restrict__ tile_prefix,
                         int64_t groups, int vary_k, int64_t M, int64_t N, int64_t tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * gb::STAGE_BYTES];
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
  Bf16Problem p = base;
  if (!vary_k) {
    p.a_base = offsets[g];
    p.m_valid = offsets[g + 1] - offsets[g];
    const int64_t b_elems = g * N * base.ldb;         // elements before expert g
    p.B = base.B + (LD == 2 ? b_elems / 2 : LD == 1 ? b_elems : b_elems * 2);
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
  gemm_bf16_tile<LD>(p, tm * gb::BM, tn * gb::BN, lds);
}

hipError_t launch_gemm_bf16path(int fmt, int64_t M, int64_t N, int64_t K, const void* A, const void* sA,
                                const float* tA, int tA_mode, const void* B, const void* sB, const float* tB,
                                int tB_mode, float* C, int64_t ldc, hipStream_t st) {
  Bf16Problem p;
  p.fmt = fmt; p.A = (const uint8_t*)A; p.sA = (const uint8_t*)sA; p.tA = tA; p.tA_mode = tA_mode;
  p.a_idx = nullptr; p.a_rows = M; p.a_base = 0; p.m_valid = M; p.lda = K;
  p.B = (const uint8_t*)B; p.sB = (const uint8_t*)sB; p.tB = tB; p.tB_mode = tB_mode; p.n_valid = N; p.ldb = K;
  p.k_begin = 0; p.k_end = K; p.C = C; p.ldc = ldc;
  const int64_t tm = (M + gb::BM - 1) / gb::BM, tn = (N + gb::BN - 1) / gb::BN;
  const int64_t blocks = (tm * tn + 7) / 8 * 8;
  if (fmt == 1) hipLaunchKernelGGL(gemm_bf16_dense_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, p, tm, tn);
  else if (fmt == 2) hipLaunchKernelGGL(gemm_bf16_dense_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, p, tm, tn);
  else hipLaunchKernelGGL(gemm_bf16_dense_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, p, tm, tn);
  return hipGetLastError();
}

hipError_t launch_grouped_bf16path(int fmt, int64_t groups, const int64_t* offsets, const int64_t* tile_prefix,
                                   int64_t max_tiles, int vary_k, int64_t total, int64_t M, int64_t N, int64_t K,
                                   const int32_t* a_idx, int64_t a_rows, const void* A, const void* sA, const float* tA, int tA_mode,
                                   const void* B, const void* sB, const float* tB, int tB_mode, float* C,
                                   hipStream_t st) {
  Bf16Problem p;
  p.fmt = fmt; p.A = (const uint8_t*)A; p.sA = (const uint8_t*)sA; p.tA = tA; p.tA_mode = tA_mode;
  p.a_idx = a_idx; p.a_rows = a_rows; p.a_base = 0;
  p.B = (const uint8_t*)B; p.sB = (const uint8_t*)sB; p.tB = tB; p.tB_mode = tB_mode; p.C = C; p.ldc = N;
  if (!vary_k) {
    p.m_valid = 0; p.lda = K; p.n_valid = N; p.ldb = K; p.k_begin = 0; p.k_end = K;
  } else {
    p.m_valid = M; p.lda = total; p.n_valid = N; p.ldb = total; p.k_begin = 0; p.k_end = 0;
  }
  const int64_t tn = (N + gb::BN - 1) / gb::BN;
  if (fmt == 1)
    hipLaunchKernelGGL(gemm_bf16_grouped_kernel<1>, dim3((unsigned)max_tiles), dim3(256), 0, st, p, offsets,
                       tile_prefix, groups, vary_k, M, N, tn);
  else if (fmt == 2)
    hipLaunchKernelGGL(gemm_bf16_grouped_kernel<2>, dim3((unsigned)max_tiles), dim3(256), 0, st, p, offsets,
                       tile_prefix, groups, vary_k, M, N, tn);
  else
    hipLaunchKernelGGL(gemm_bf16_grouped_kernel<0>, dim3((unsigned)max_tiles), dim3(256), 0, st, p, offsets,
                       tile_prefix, groups, vary_k, M, N, tn);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped-GEMM scheduler: tile_prefix[g] = first tile of group g, computed on
// the device from the offsets (no host synchronisation on group sizes).
// vary_k = 0: group g has ceil(M_g / bm) * tiles_n tiles; vary_k = 1: tiles_m * tiles_n.
// ---------------------------------------------------------------------------
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

hipError_t launch_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* A, const void* sA, const float* tA,
                       int tA_mode, const void* B, const void* sB, const float* tB, int tB_mode, float* C,
                       int64_t ldc, hipStream_t st) {
  return launch_gemm_bf16path(fmt, M, N, K, A, sA, tA, tA_mode, B, sB, tB, tB_mode, C, ldc, st);
}

hipError_t launch_grouped_gemm(int fmt, int64_t groups, const int64_t* offsets, int vary_k, int64_t total, int64_t M,
                               int64_t N, int64_t K, const int32_t* a_row_index, int64_t a_rows, const void* A,
                               const void* sA, const float* tA, int tA_mode, const void* B, const void* sB,
                               const float* tB, int tB_mode, float* C, void* ws, hipStream_t st) {
  int64_t* prefix = (int64_t*)ws;
  const int64_t bm = gb::BM, bn = gb::BN;
  const int64_t tiles_n = (N + bn - 1) / bn;
  const int64_t tiles_m_fixed = vary_k ? (M + bm - 1) / bm : 0;
  const int64_t align = fmt == 1 ? 32 : fmt == 2 ? 16 : 8;
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(64), 0, st, offsets, groups, total, vary_k, align, bm,
                     tiles_m_fixed, tiles_n, prefix);
  const int64_t max_tiles = vary_k ? groups * tiles_m_fixed * tiles_n : ((total + bm - 1) / bm + groups) * tiles_n;
  if (max_tiles <= 0) return hipGetLastError();
  return launch_grouped_bf16path(fmt, groups, offsets, prefix, max_tiles, vary_k, total, M, N, K, a_row_index, a_rows,
                                 A, sA, tA, tA_mode, B, sB, tB, tB_mode, C, st);
}

}  // namespace mxq
