// NVFP4 quantizers: E2M1 elements, one E4M3 scale per 16 values, one FP32
// decode scale per scope (token row, tensor, or group of rows).
//
// Operation (restated from the pages): two-level NVFP4 scaling, where the FP32
// scale keeps the E4M3 block scales in range and the block amax lands next to
// the FP4 maximum (7minutos.es NVFP4 page, section "Que es realmente NVFP4");
// the FP32 scale computed online per token inside the one kernel that emits the
// packed values, block scales and token scales (remio.ai "Miles Blackwell RL",
// section "Un Cuantizador Compartido Es el Mecanismo Real"); no approximate
// math in the FP4 path (same section); optional 16-point random Hadamard
// transform of the quantized axis (7minutos.es, section "La metodologia de
// formacion de cuatro partes").
//
// Binary32 steps, in this order (every division correctly rounded):
//   s_enc = 2688 / A  (A = scope amax; 1 if A == 0; FLT_MAX if it overflows)
//   t     = 1 / s_enc                                (stored decode scale)
//   S_b   = E4M3_RNE_sat((a_b / 6) * s_enc)           (a_b = block amax)
//   r_b   = min(s_enc / S_b, FLT_MAX), 0 when S_b == 0
//   q_i   = E2M1_RNE_sat(x_i * r_b)
#include "common.h"

namespace mxq {

__device__ __forceinline__ void scope_scales(float A, float& s_enc, float& t) {
  float s = 2688.0f / A;
  if (A == 0.0f) s = 1.0f;
  if (__builtin_isinf(s)) s = kFltMax;
  s_enc = s;
  t = 1.0f / s;
}

// Block scale code and element multiplier for a 16-block with amax a_b.
__device__ __forceinline__ uint32_t block_scale(float a_b, float s_enc, float& r_b) {
  float d = (a_b / 6.0f) * s_enc;
  d = fminf(d, kE4M3Max);                                   // saturate (d >= 0)
  const uint32_t code = cvt_fp8x2_f32(0u, d, 0.0f, 1.0f, false) & 0xFFu;
  const float S = e4m3_to_f32(code);
  float r = s_enc / S;
  r = fminf(r, kFltMax);
  r_b = (S == 0.0f) ? 0.0f : r;
  return code;
}

// Eight consecutive values (a 16-block is two lanes) -> 4 packed bytes.
__device__ __forceinline__ uint32_t pack8_e2m1(const float* v, float r) {
  uint32_t o = 0;
  o = cvt_fp4x2_f32<0>(o, v[0] * r, v[1] * r);
  o = cvt_fp4x2_f32<1>(o, v[2] * r, v[3] * r);
  o = cvt_fp4x2_f32<2>(o, v[4] * r, v[5] * r);
  o = cvt_fp4x2_f32<3>(o, v[6] * r, v[7] * r);
  return o;
}

// ---------------------------------------------------------------------------
// Stochastic rounding (gradients only: 7minutos.es NVFP4 page, section "La
// metodologia de formacion de cuatro partes"). Random words come from the
// counter-based Philox4x32-10 generator (Salmon, Moraes, Dror, Shaw, SC 2011):
// element idx of the output tensor (row-major) takes word idx % 4 of the block
// for counter (idx / 4 low, high, 0, 0) and key (seed low, high).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // each 32 x 32 -> 64-bit product in one multiply (high and low words together)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Words of the 8 consecutive elements idx0 .. idx0 + 7 (idx0 % 8 == 0).
__device__ __forceinline__ void philox_words8(uint64_t idx0, uint64_t seed, uint32_t* w) {
  const uint64_t b = idx0 >> 2;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const uint4 a = philox4x32_10(make_uint4((uint32_t)b, (uint32_t)(b >> 32), 0u, 0u), k0, k1);
  const uint4 c = philox4x32_10(make_uint4((uint32_t)(b + 1), (uint32_t)((b + 1) >> 32), 0u, 0u), k0, k1);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = c.x; w[5] = c.y; w[6] = c.z; w[7] = c.w;
}

// E2M1 code of p rounded stochastically: m = |p| between grid neighbours lo < hi
// (spacing d), f = (m - lo) / d (exact); round up iff (word >> 8) < f * 2^24;
// |p| >= 6 saturates to 6; the sign is copied.
__device__ __forceinline__ uint32_t e2m1_sr_code(float p, uint32_t word) {
  const float m = fabsf(p);
  uint32_t lo_i;
  float lo, inv_d;
  if (m >= 6.0f) { lo_i = 7; lo = 6.0f; inv_d = 0.0f; }
  else if (m >= 4.0f) { lo_i = 6; lo = 4.0f; inv_d = 0.5f; }
  else if (m >= 2.0f) { lo = floorf(m); lo_i = lo == 2.0f ? 4u : 5u; inv_d = 1.0f; }
  else { const float h = floorf(m * 2.0f); lo_i = (uint32_t)h; lo = h * 0.5f; inv_d = 2.0f; }
  const float f = (m - lo) * inv_d;                        // exact: m - lo exact, 1/d a power of two
  const bool up = (float)(word >> 8) < f * 16777216.0f;    // both sides exact integers < 2^24 (+1)
  return (lo_i + (up ? 1u : 0u)) | ((__float_as_uint(p) >> 28) & 8u);
}

__device__ __forceinline__ uint32_t pack8_e2m1_sr(const float* v, float r, const uint32_t* w) {
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) o |= e2m1_sr_code(v[i] * r, w[i]) << (4 * i);
  return o;
}

__device__ __forceinline__ void unpack8(const uint4& w, float* f) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// 16-point RHT of a block split over a lane pair (8 values each, even lane
// holds elements 0..7): w = s * v; FWHT stages 1, 2, 4 inside the lane, stage 8
// across the pair; u = w * 0.25.
__device__ __forceinline__ void rht16_pair(float* f, const float* sg, bool odd) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] *= sg[i];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = f[i], b = f[i + h];
      f[i] = a + b;
      f[i + h] = a - b;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float other = __uint_as_float(dpp_xor1(__float_as_uint(f[i])));
    f[i] = odd ? (other - f[i]) : (f[i] + other);
    f[i] *= 0.25f;
  }
}

__device__ __forceinline__ float wave_max_f32(float v) {
  uint32_t u = __float_as_uint(v);  // v >= 0: bits order like values
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = shfl_xor_u32(u, off);
    u = u > o ? u : o;
  }
  return __uint_as_float(u);
}

// ---------------------------------------------------------------------------
// Row-blocked quantizer: one wave per row, the row kept in registers.
//   MODE 0: per-row scope, amax computed here (per-token NVFP4).
//   MODE 1: scope amax read from `scope_amax[row / group_rows]` (tensor/group).
//   MODE 2: pass 1 of MODE 1 -- only the scope amax, by atomic max.
// CH = register chunks of 512 values (the row holds at most CH * 512 values).
// ---------------------------------------------------------------------------
template <int MODE, int CH, bool RHT, bool SR = false>
__global__ void __launch_bounds__(256)
nvfp4_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
                  int64_t group_rows, uint32_t neg_mask,
                  uint32_t* __restrict__ scope_amax,
                  uint8_t* __restrict__ q, uint8_t* __restrict__ s, float* __restrict__ t_out, uint64_t seed) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;   // wave-uniform; with MODE 2 a partial group never syncs
  const uint16_t* xr = x + row * ld_x;
  const bool odd = lane & 1;
  float sg[8];
  if (RHT) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sg[i] = ((neg_mask >> ((odd ? 8 : 0) + i)) & 1u) ? -1.0f : 1.0f;
  }

  uint4 v[CH];
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t e = (int64_t)i * 512 + 8 * lane;
    v[i] = (e < cols) ? load_stream16(xr + e) : make_uint4(0, 0, 0, 0);
    if (!RHT)
      amax_bits = pk_max_u16(amax_bits, pk_max_u16(pk_max_u16(v[i].x & 0x7FFF7FFFu, v[i].y & 0x7FFF7FFFu),
                                                   pk_max_u16(v[i].z & 0x7FFF7FFFu, v[i].w & 0x7FFF7FFFu)));
  }
  float A;
  if (MODE == 1) {
    A = __uint_as_float(scope_amax[row / group_rows]);
  } else if (!RHT) {
    A = __uint_as_float(max_halves(amax_bits) << 16);
    A = wave_max_f32(A);
  } else {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      float f[8];
      unpack8(v[i], f);
      rht16_pair(f, sg, odd);
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[k]));
    }
    A = wave_max_f32(m);
  }
  if (MODE == 2) {
    // One atomic per workgroup when its 4 rows share a scope, else one per row.
    const int64_t row0 = (int64_t)blockIdx.x * 4;
    const bool shared = (row0 + 3 < rows) && (row0 / group_rows == (row0 + 3) / group_rows);
    if (!shared) {
      if (lane == 0 && A > 0.0f) atomicMax(scope_amax + row / group_rows, __float_as_uint(A));
      return;
    }
    __shared__ uint32_t red[4];
    if (lane == 0) red[threadIdx.x >> 6] = __float_as_uint(A);
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t m = max(max(red[0], red[1]), max(red[2], red[3]));
      if (m) atomicMax(scope_amax + row0 / group_rows, m);
    }
    return;
  }
  float s_enc, t;
  scope_scales(A, s_enc, t);
  if (lane == 0) {                     // decode scale: per row, or per scope from its first row
    if (MODE == 0) t_out[row] = t;
    else if (row % group_rows == 0) t_out[row / group_rows] = t;
  }

#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t e = (int64_t)i * 512 + 8 * lane;
    float f[8];
    unpack8(v[i], f);
    if (RHT) rht16_pair(f, sg, odd);
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
    a = fmaxf(a, __uint_as_float(dpp_xor1(__float_as_uint(a))));
    float r;
    const uint32_t code = block_scale(a, s_enc, r);
    uint32_t packed;
    if (SR) {
      uint32_t wd[8];
      philox_words8((uint64_t)row * cols + e, seed, wd);
      packed = pack8_e2m1_sr(f, r, wd);
    } else {
      packed = pack8_e2m1(f, r);
    }
    if (e < cols) {
      // tensor / group scopes (weights, read again only by a later GEMM): non-temporal
      if (MODE == 1) __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(q + row * (cols / 2) + e / 2));
      else *reinterpret_cast<uint32_t*>(q + row * (cols / 2) + e / 2) = packed;
      if (!odd) s[row * (cols / 16) + e / 16] = (uint8_t)code;
    }
  }
}

// ---------------------------------------------------------------------------
// Column-blocked (transposed) quantizer: blocks of 16 consecutive ROWS of x;
// output row c of (cols, rows/2) holds column c of x.
// A workgroup (4 waves) owns a 256-row x 128-column tile; wave w owns rows
// 64w .. 64w+63 of it and lane = 16*m + c16 holds rows 16m .. 16m+15 and
// columns 8*c16 .. 8*c16+7 as sixteen 16-byte loads (each load instruction of
// the wave reads 4 full 256-byte row segments). Every 16-row block of a column
// is then inside one lane: transform, block amax and quantization need no lane
// exchange. The packed bytes (8 per column and lane) and block scales go
// through LDS, so each column of the tile leaves as one 128-byte segment and
// its 16 scale bytes as one 16-byte store.
//   MODE 1: scope amax from scope_amax[c / group_rows]; MODE 2: pass 1 (amax only).
// ---------------------------------------------------------------------------
template <int MODE, bool RHT, bool SR = false>
__global__ void __launch_bounds__(256)
nvfp4_cols_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
                  int64_t group_rows, uint32_t neg_mask,
                  uint32_t* __restrict__ scope_amax,
                  uint8_t* __restrict__ q, uint8_t* __restrict__ s, float* __restrict__ t_out, int64_t col_tiles,
                  int wide_stores, uint64_t seed) {
  // packed tile: column cl at cl * 128, 8-byte granule g = 4w + m at (g ^ 4 * (cl / 8 % 4))
  __shared__ __attribute__((aligned(16))) uint8_t lq[MODE == 1 ? 128 * 128 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ls[MODE == 1 ? 128 * 16 : 16];
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = lane >> 4, c16 = lane & 15;
  const int64_t band = (int64_t)blockIdx.x / col_tiles, ct = (int64_t)blockIdx.x % col_tiles;
  const int64_t R0 = band * 256, C0 = ct * 128;
  const int64_t r0 = R0 + 64 * w + 16 * m;          // first row of the lane's block
  const int64_t c = C0 + 8 * c16;
  const bool ok = c < cols && r0 < rows;            // cols % 8 == 0, rows % 16 == 0: whole blocks
  uint4 v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    // the amax pass leaves x cached for the quantize pass (measured +4% over streaming both)
    v[j] = ok ? (MODE == 2 ? *reinterpret_cast<const uint4*>(x + (r0 + j) * ld_x + c) : load_stream16(x + (r0 + j) * ld_x + c))
              : make_uint4(0, 0, 0, 0);

  if (RHT) {
    // random signs: row j of every block is negated when bit j is set; a dword holds two
    // columns of one row, so one XOR of both sign bits flips them exactly
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t f = ((neg_mask >> j) & 1u) ? 0x80008000u : 0u;
      v[j].x ^= f; v[j].y ^= f; v[j].z ^= f; v[j].w ^= f;
    }
  }
  float mloc = 0.0f;                                 // MODE 2: max over the lane's 8 columns
  float s_enc = 1.0f;
  if (MODE == 1 && ok) {
    float tt;
    scope_scales(__uint_as_float(scope_amax[c / group_rows]), s_enc, tt);   // 8 columns, one scope
    // the decode scale of a scope, from the lane that holds its first column in the first band
    if (band == 0 && w == 0 && m == 0 && c % group_rows == 0) t_out[c / group_rows] = tt;
  }
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    float f[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t wd = (cc >> 1) == 0 ? v[j].x : (cc >> 1) == 1 ? v[j].y : (cc >> 1) == 2 ? v[j].z : v[j].w;
      f[j] = (cc & 1) ? bf16_hi(wd) : bf16_lo(wd);
    }
    if (RHT) {
#pragma unroll
      for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (i & h) continue;
          const float a = f[i], b = f[i + h];
          f[i] = a + b;
          f[i + h] = a - b;
        }
      }
      // the amax pass takes the maximum of the unnormalized sums and scales it once
      // below: rounding is monotonic, so RN(max |f| / 4) = max RN(|f| / 4)
      if (MODE != 2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] *= 0.25f;
      }
    }
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) a = fmaxf(a, fabsf(f[k]));
    if (MODE == 2) {
      mloc = fmaxf(mloc, a);
    } else {
      float r;
      const uint32_t code = block_scale(a, s_enc, r);
      uint32_t lo, hi;
      if (SR) {                                        // output element (col, row): index col * rows + row
        uint32_t wd[16];
        const uint64_t idx0 = (uint64_t)(c + cc) * rows + r0;
        philox_words8(idx0, seed, wd);
        philox_words8(idx0 + 8, seed, wd + 8);
        lo = pack8_e2m1_sr(f, r, wd);
        hi = pack8_e2m1_sr(f + 8, r, wd + 8);
      } else {
        lo = pack8_e2m1(f, r);
        hi = pack8_e2m1(f + 8, r);
      }
      const int cl = 8 * c16 + cc;
      const int g = (4 * w + m) ^ ((c16 & 3) * 4);
      *reinterpret_cast<uint2*>(lq + cl * 128 + g * 8) = make_uint2(lo, hi);
      ls[cl * 16 + 4 * w + m] = (uint8_t)code;
    }
  }

  if (MODE == 2) {
    if (RHT) mloc *= 0.25f;
    // The lane's 8 columns share a scope (group_rows % 8 == 0). Reduce over the
    // workgroup when its whole column tile lies in one scope.
    const int64_t tile_c1 = min(C0 + 128, cols) - 1;
    const bool shared = C0 / group_rows == tile_c1 / group_rows;
    if (!shared) {
      if (ok && mloc > 0.0f) atomicMax(scope_amax + c / group_rows, __float_as_uint(mloc));
      return;
    }
    const float wm = wave_max_f32(mloc);
    if (lane == 0) red[w] = __float_as_uint(wm);
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t mm = max(max(red[0], red[1]), max(red[2], red[3]));
      if (mm) atomicMax(scope_amax + C0 / group_rows, mm);
    }
    return;
  }
  __syncthreads();
  const int t = threadIdx.x;
  const int64_t rb = rows / 2;                       // packed bytes per output row
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = k * 256 + t;                       // 16-byte chunk: column i / 8, rows 32 (i % 8) ..
    const int cl = i >> 3, ch = i & 7;
    const int64_t col = C0 + cl, rr = R0 + 32 * ch;
    if (col >= cols || rr >= rows) continue;
    const int g0 = (2 * ch) ^ (((cl >> 3) & 3) * 4);  // granules 2ch, 2ch+1 stay adjacent
    const uint4 d = *reinterpret_cast<const uint4*>(lq + cl * 128 + g0 * 8);
    uint8_t* dst = q + col * rb + rr / 2;
    if (wide_stores) {                               // rows % 32 == 0: aligned whole chunks
      *reinterpret_cast<uint4*>(dst) = d;
    } else {                                         // 8-byte halves (rows % 16 == 0)
      *reinterpret_cast<uint2*>(dst) = make_uint2(d.x, d.y);
      if (rr + 16 < rows) *reinterpret_cast<uint2*>(dst + 8) = make_uint2(d.z, d.w);
    }
  }
  if (t < 128 && C0 + t < cols) {
    const int64_t sb = rows / 16;                    // scale bytes per output row
    const int64_t nb = min((int64_t)16, sb - band * 16);
    uint8_t* dst = s + (C0 + t) * sb + band * 16;
    const uint4 d = *reinterpret_cast<const uint4*>(ls + t * 16);
    if (wide_stores && (sb % 16) == 0) {
      *reinterpret_cast<uint4*>(dst) = d;
    } else {
      const uint32_t wv[4] = {d.x, d.y, d.z, d.w};
      for (int b = 0; b < nb; ++b) dst[b] = (uint8_t)(wv[b / 4] >> (8 * (b % 4)));
    }
  }
}

// ---------------------------------------------------------------------------
// 2D (16x16-block) NVFP4 for weights: one E4M3 scale per 16x16 block, so the
// forward (rows along K) and the transposed backward use the same codes
// (7minutos.es NVFP4 page, section "La metodologia de formacion de cuatro
// partes", 2D weight scaling). Pass 2 of a two-pass quantizer: the scope amax
// (tensor or group of rows) comes from scope_amax. Tile as nvfp4_cols_kernel:
// 256 rows x 128 columns per workgroup, lane = 16*m + c16 holding rows
// 16m .. 16m+15 of its wave's 64-row slab and columns 8*c16 .. 8*c16+7; a 16x16
// block is the lane pair (c16, c16 ^ 1). Writes the row copy (rows, cols/2) with
// its scales repeated per row (rows, cols/16), and/or the transposed copy
// per scope group (groups, cols, group_rows/2) with (groups, cols, group_rows/16),
// both staged through LDS where rows of the output are short.
// ---------------------------------------------------------------------------
template <bool DO_ROW, bool DO_COL>
__global__ void __launch_bounds__(256)
nvfp4_2d_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x, int64_t group_rows,
                const uint32_t* __restrict__ scope_amax, uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                uint8_t* __restrict__ q_colT, uint8_t* __restrict__ s_colT, float* __restrict__ t_out,
                int64_t col_tiles, int wide_col, int dw_row) {
  __shared__ __attribute__((aligned(16))) uint8_t lq[DO_COL ? 128 * 128 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t lsc[DO_COL ? 128 * 16 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t lsr[DO_ROW ? 256 * 8 : 16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = lane >> 4, c16 = lane & 15;
  const int64_t band = (int64_t)blockIdx.x / col_tiles, ct = (int64_t)blockIdx.x % col_tiles;
  const int64_t R0 = band * 256, C0 = ct * 128;
  const int rl0 = 64 * w + 16 * m;                  // tile row of the lane's first row
  const int64_t r0 = R0 + rl0;
  const int64_t c = C0 + 8 * c16;
  const bool ok = c < cols && r0 < rows;            // cols % 16 == 0, rows % 16 == 0: whole blocks
  uint4 v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    v[j] = ok ? load_stream16(x + (r0 + j) * ld_x + c) : make_uint4(0, 0, 0, 0);
  float s_enc = 1.0f;
  if (ok) {
    float tt;
    scope_scales(__uint_as_float(scope_amax[r0 / group_rows]), s_enc, tt);   // 16 rows, one scope
    // the decode scale of a scope, from the lane that holds its first row in column 0
    if (c == 0 && r0 % group_rows == 0) t_out[r0 / group_rows] = tt;
  }
  uint32_t am = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    am = pk_max_u16(am, pk_max_u16(pk_max_u16(v[j].x & 0x7FFF7FFFu, v[j].y & 0x7FFF7FFFu),
                                   pk_max_u16(v[j].z & 0x7FFF7FFFu, v[j].w & 0x7FFF7FFFu)));
  am = max_halves(am);
  const uint32_t other = dpp_xor1(am);
  am = am > other ? am : other;                     // 16x16 block amax (BF16 bits, exact)
  float r;
  const uint32_t code = block_scale(__uint_as_float(am << 16), s_enc, r);

  if (DO_ROW) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float f[8];
      unpack8(v[j], f);
      const uint32_t packed = pack8_e2m1(f, r);
      if (ok) __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(q_row + (r0 + j) * (cols / 2) + c / 2));
    }
    if ((c16 & 1) == 0)
#pragma unroll
      for (int j = 0; j < 16; ++j) lsr[(rl0 + j) * 8 + (c16 >> 1)] = (uint8_t)code;
  }
  if (DO_COL) {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      float f[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t wd = (cc >> 1) == 0 ? v[j].x : (cc >> 1) == 1 ? v[j].y : (cc >> 1) == 2 ? v[j].z : v[j].w;
        f[j] = (cc & 1) ? bf16_hi(wd) : bf16_lo(wd);
      }
      const uint32_t lo = pack8_e2m1(f, r), hi = pack8_e2m1(f + 8, r);
      const int cl = 8 * c16 + cc;
      const int g = (4 * w + m) ^ ((c16 & 3) * 4);
      *reinterpret_cast<uint2*>(lq + cl * 128 + g * 8) = make_uint2(lo, hi);
      lsc[cl * 16 + 4 * w + m] = (uint8_t)code;
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (DO_ROW && R0 + t < rows) {
    const int64_t sb = cols / 16;
    const int64_t nb = min((int64_t)8, sb - ct * 8);
    uint8_t* dst = s_row + (R0 + t) * sb + ct * 8;
    const uint2 d = *reinterpret_cast<const uint2*>(lsr + t * 8);
    if (dw_row && nb == 8) {
      *reinterpret_cast<uint2*>(dst) = d;
    } else {
      const uint32_t wv[2] = {d.x, d.y};
      for (int b = 0; b < nb; ++b) dst[b] = (uint8_t)(wv[b / 4] >> (8 * (b % 4)));
    }
  }
  if (DO_COL) {
    // transposed copy per scope group: (groups, cols, group_rows / 2) and (groups, cols, group_rows / 16)
    const int64_t rb = group_rows / 2, sb = group_rows / 16;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = k * 256 + t;
      const int cl = i >> 3, ch = i & 7;
      const int64_t col = C0 + cl, rr = R0 + 32 * ch;
      if (col >= cols || rr >= rows) continue;
      const int g0 = (2 * ch) ^ (((cl >> 3) & 3) * 4);
      const uint4 d = *reinterpret_cast<const uint4*>(lq + cl * 128 + g0 * 8);
      const int64_t gi = rr / group_rows, rl = rr - gi * group_rows;
      uint8_t* dst = q_colT + (gi * cols + col) * rb + rl / 2;
      if (wide_col) {                                 // group_rows % 32 == 0: whole aligned chunks
        { const u32x4_nt d4 = {d.x, d.y, d.z, d.w}; __builtin_nontemporal_store(d4, reinterpret_cast<u32x4_nt*>(dst)); }
      } else {                                        // 16-row granules, each inside one group
        *reinterpret_cast<uint2*>(dst) = make_uint2(d.x, d.y);
        const int64_t r2 = rr + 16;
        if (r2 < rows) {
          const int64_t g2 = r2 / group_rows, rl2 = r2 - g2 * group_rows;
          *reinterpret_cast<uint2*>(q_colT + (g2 * cols + col) * rb + rl2 / 2) = make_uint2(d.z, d.w);
        }
      }
    }
    if (t < 128 && C0 + t < cols) {
      const uint4 d = *reinterpret_cast<const uint4*>(lsc + t * 16);
      const int64_t gi = R0 / group_rows, rl = R0 - gi * group_rows;
      if (wide_col && group_rows % 256 == 0 && R0 + 256 <= rows) {   // 16 blocks of one group, aligned
        *reinterpret_cast<uint4*>(s_colT + (gi * cols + C0 + t) * sb + rl / 16) = d;
      } else {
        const uint32_t wv[4] = {d.x, d.y, d.z, d.w};
        for (int b = 0; b < 16; ++b) {
          const int64_t r = R0 + 16 * b;
          if (r >= rows) break;
          const int64_t g2 = r / group_rows, rl2 = r - g2 * group_rows;
          s_colT[(g2 * cols + C0 + t) * sb + rl2 / 16] = (uint8_t)(wv[b / 4] >> (8 * (b % 4)));
        }
      }
    }
  }
}

// t[g] = decode scale of scope g, from the amax in the workspace.
__global__ void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int MODE, bool RHT, bool SR = false>
static void launch_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int64_t group_rows,
                        uint32_t sg, uint32_t* ws, uint8_t* q, uint8_t* s, float* t, hipStream_t st,
                        uint64_t seed = 0) {
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const int64_t ch = (cols + 511) / 512;
  if (ch <= 4)
    hipLaunchKernelGGL((nvfp4_rows_kernel<MODE, 4, RHT, SR>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, sg, ws, q, s, t, seed);
  else if (ch <= 8)
    hipLaunchKernelGGL((nvfp4_rows_kernel<MODE, 8, RHT, SR>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, sg, ws, q, s, t, seed);
  else if (ch <= 12)
    hipLaunchKernelGGL((nvfp4_rows_kernel<MODE, 12, RHT, SR>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, sg, ws, q, s, t, seed);
  else if (ch <= 14)
    hipLaunchKernelGGL((nvfp4_rows_kernel<MODE, 14, RHT, SR>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, sg, ws, q, s, t, seed);
  else if (ch <= 16)
    hipLaunchKernelGGL((nvfp4_rows_kernel<MODE, 16, RHT, SR>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, sg, ws, q, s, t, seed);
  else
    hipLaunchKernelGGL((nvfp4_rows_kernel<MODE, 32, RHT, SR>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, sg, ws, q, s, t, seed);
}

template <int MODE, bool RHT, bool SR = false>
static void launch_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int64_t group_rows,
                        uint32_t sg, uint32_t* ws, uint8_t* q, uint8_t* s, float* t, hipStream_t st,
                        uint64_t seed = 0) {
  const int64_t col_tiles = (cols + 127) / 128;
  const int64_t bands = (rows + 255) / 256;
  // 16-byte stores need 16-byte aligned output rows (and bases)
  const int wide = rows % 32 == 0 && ((uintptr_t)q & 15) == 0 && ((uintptr_t)s & 15) == 0;
  dim3 grid((unsigned)(bands * col_tiles)), block(256);
  hipLaunchKernelGGL((nvfp4_cols_kernel<MODE, RHT, SR>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, sg, ws, q, s,
                     t, col_tiles, wide, seed);
}


// 2D weights: scope amax pass (rows kernel, MODE 2), then the 16x16-block pass.
// Scope maxima of |x| when every scope is one contiguous span of `span` elements (rows
// stored back to back): the first pass of the per-tensor / per-group quantizer as a flat
// streaming reduction. Workgroup b reduces part b % per_scope of scope b / per_scope,
// eight 16-byte loads in flight per lane, and folds its maximum into scope_amax with
// one atomic (BF16 magnitudes compare as their bit patterns).
__global__ void __launch_bounds__(256)
scope_amax_flat_kernel(const uint16_t* __restrict__ x, int64_t span, int per_scope, uint32_t* __restrict__ scope_amax) {
  const int64_t g = blockIdx.x / per_scope;
  const int64_t part = blockIdx.x % per_scope;
  const int64_t units = span / 8;                                    // 16-byte units (span % 8 == 0)
  const int64_t u0 = units * part / per_scope, u1 = units * (part + 1) / per_scope;
  const uint16_t* base = x + g * span;
  uint32_t m = 0;
  int64_t u = u0 + threadIdx.x;
  for (; u + 7 * 256 < u1; u += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load_stream16(base + (u + k * 256) * 8);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      m = pk_max_u16(m, pk_max_u16(pk_max_u16(v[k].x & 0x7FFF7FFFu, v[k].y & 0x7FFF7FFFu),
                                   pk_max_u16(v[k].z & 0x7FFF7FFFu, v[k].w & 0x7FFF7FFFu)));
  }
  for (; u < u1; u += 256) {
    const uint4 v = load_stream16(base + u * 8);
    m = pk_max_u16(m, pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                                 pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu)));
  }
  const float a = wave_max_f32(__uint_as_float(max_halves(m) << 16));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = __float_as_uint(a);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t mm = max(max(red[0], red[1]), max(red[2], red[3]));
    if (mm) atomicMax(scope_amax + g, mm);
  }
}

// First pass of a scope-scaled quantizer (no transform): scope maxima of |x| over row
// groups of gr rows, flat when the rows are stored back to back.
static void launch_scope_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int64_t gr,
                              int64_t n_scopes, uint32_t* ws_amax, hipStream_t st) {
  if (ld_x == cols) {
    const int64_t span = gr * cols, units = span / 8;
    const int64_t want = (2048 + n_scopes - 1) / n_scopes;           // ~2048 workgroups in all
    const int64_t cap = units / 2048 > 0 ? units / 2048 : 1;        // >= 2048 units each
    const int per_scope = (int)(want < cap ? want : cap);
    hipLaunchKernelGGL(scope_amax_flat_kernel, dim3((unsigned)(n_scopes * per_scope)), dim3(256), 0, st, x, span,
                       per_scope, ws_amax);
  } else {
    launch_rows<2, false>(x, rows, cols, ld_x, gr, 0u, ws_amax, nullptr, nullptr, nullptr, st);
  }
}

hipError_t launch_quant_nvfp4_2d(const void* xv, int64_t rows, int64_t cols, int64_t ld_x, int64_t group_rows,
                                 void* q_row, void* s_row, void* q_colT, void* s_colT, float* t, uint32_t* ws_amax,
                                 int64_t n_scopes, hipStream_t st) {
  const uint16_t* x = (const uint16_t*)xv;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n_scopes + 255) / 256)), dim3(256), 0, st, ws_amax, 0u, n_scopes);
  launch_scope_amax(x, rows, cols, ld_x, group_rows, n_scopes, ws_amax, st);
  const int64_t col_tiles = (cols + 127) / 128;
  const int64_t bands = (rows + 255) / 256;
  uint8_t *qr = (uint8_t*)q_row, *sr = (uint8_t*)s_row, *qc = (uint8_t*)q_colT, *sc = (uint8_t*)s_colT;
  const int wide = qc && group_rows % 32 == 0 && ((uintptr_t)qc & 15) == 0 && ((uintptr_t)sc & 15) == 0;
  const int dw_row = sr && (cols / 16) % 8 == 0 && ((uintptr_t)sr & 7) == 0;
  dim3 grid((unsigned)(bands * col_tiles)), block(256);
  if (qr && qc)
    hipLaunchKernelGGL((nvfp4_2d_kernel<true, true>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, ws_amax, qr, sr, qc, sc, t, col_tiles, wide, dw_row);
  else if (qr)
    hipLaunchKernelGGL((nvfp4_2d_kernel<true, false>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, ws_amax, qr, sr, qc, sc, t, col_tiles, wide, dw_row);
  else
    hipLaunchKernelGGL((nvfp4_2d_kernel<false, true>), grid, block, 0, st, x, rows, cols, ld_x, group_rows, ws_amax, qr, sr, qc, sc, t, col_tiles, wide, dw_row);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4_token(const void* x, int64_t tokens, int64_t hidden, int64_t ld_x,
                                    void* q, void* s, float* t, hipStream_t st) {
  launch_rows<0, false>((const uint16_t*)x, tokens, hidden, ld_x, 1, 0u, nullptr, (uint8_t*)q, (uint8_t*)s, t, st);
  return hipGetLastError();
}

// General entry: scope 0 = ROW, 1 = TENSOR, 2 = GROUP. RHT signs are passed as
// a 16-bit mask (bit i set <=> sign i is -1); rht = 0 disables the transform.
// SR = stochastic rounding of the elements with the given seed.
template <bool SR>
static hipError_t quant_nvfp4_impl(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int scope,
                                   int64_t group_rows, int transpose, int rht, uint32_t neg_mask, uint8_t* qp,
                                   uint8_t* sp, float* t, uint32_t* ws_amax, int64_t n_scopes, uint64_t seed,
                                   hipStream_t st) {
  if (scope == 0) {  // per row, one pass (transpose excluded by validation)
    if (rht) launch_rows<0, true, SR>(x, rows, cols, ld_x, 1, neg_mask, nullptr, qp, sp, t, st, seed);
    else launch_rows<0, false, SR>(x, rows, cols, ld_x, 1, 0u, nullptr, qp, sp, t, st, seed);
    return hipGetLastError();
  }
  const int64_t gr = scope == 1 ? (transpose ? cols : rows) : group_rows;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n_scopes + 255) / 256)), dim3(256), 0, st, ws_amax, 0u, n_scopes);
  if (!transpose) {
    if (rht) {
      launch_rows<2, true>(x, rows, cols, ld_x, gr, neg_mask, ws_amax, qp, sp, t, st);
      launch_rows<1, true, SR>(x, rows, cols, ld_x, gr, neg_mask, ws_amax, qp, sp, t, st, seed);
    } else {
      launch_scope_amax(x, rows, cols, ld_x, gr, n_scopes, ws_amax, st);
      launch_rows<1, false, SR>(x, rows, cols, ld_x, gr, 0u, ws_amax, qp, sp, t, st, seed);
    }
  } else {
    if (rht) {
      launch_cols<2, true>(x, rows, cols, ld_x, gr, neg_mask, ws_amax, qp, sp, nullptr, st);
      launch_cols<1, true, SR>(x, rows, cols, ld_x, gr, neg_mask, ws_amax, qp, sp, t, st, seed);
    } else {
      launch_cols<2, false>(x, rows, cols, ld_x, gr, 0u, ws_amax, qp, sp, nullptr, st);
      launch_cols<1, false, SR>(x, rows, cols, ld_x, gr, 0u, ws_amax, qp, sp, t, st, seed);
    }
  }
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const void* xv, int64_t rows, int64_t cols, int64_t ld_x, int scope,
                              int64_t group_rows, int transpose, int rht, uint32_t neg_mask,
                              void* q, void* s, float* t, uint32_t* ws_amax, int64_t n_scopes,
                              int sr, uint64_t seed, hipStream_t st) {
  const uint16_t* x = (const uint16_t*)xv;
  uint8_t *qp = (uint8_t*)q, *sp = (uint8_t*)s;
  if (sr) return quant_nvfp4_impl<true>(x, rows, cols, ld_x, scope, group_rows, transpose, rht, neg_mask, qp, sp, t,
                                        ws_amax, n_scopes, seed, st);
  return quant_nvfp4_impl<false>(x, rows, cols, ld_x, scope, group_rows, transpose, rht, neg_mask, qp, sp, t, ws_amax,
                                 n_scopes, seed, st);
}

}  // namespace mxq
