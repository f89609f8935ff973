// Blockwise FP8 quantizers (DeepSeek-V3 style): E4M3 elements with one FP32 scale
// per 1 x 128 activation / gradient tile or per 128 x 128 weight block.
//
// Operation (restated from the pages): weights use 128 x 128 blocks and activations
// 1 x 128 tiles, with FP32 scales applied in software around the matrix product
// ("Miles Blackwell MXFP8/NVFP4 RL recipes", aib.vote, second paragraph; "Miles
// Blackwell RL", remio.ai, section "NVFP4 por token cuestiona el valor
// predeterminado uniforme de BF16"); gradients use the activation tiles (7minutos.es
// NVFP4 page, the 12B results paragraph). Per block: s = fl32(amax / 448) (0 for an
// all-zero block), q = RNE_sat_E4M3(fl32(x / s)) (signed zero when s = 0).
//
// Work decomposition: a workgroup (4 waves) owns a 128 x 128 BF16 tile, laid out as
// in the MXFP8 quantizer: wave w holds rows 32w .. 32w+31, lane 16m + c16 holds rows
// 8m .. 8m+7 and columns 8 c16 .. 8 c16 + 7 (eight 16-byte loads).
//   AR (1 x 128 row tiles): a row's 128 values sit on the 16 lanes of equal m: amax by
//          two DPP quad exchanges and two lane-xor exchanges; each lane stores its 8
//          bytes; lane c16 = 0 stores the row's scale.
//   AC (128 x 1 column tiles, stored transposed): a column's 128 values span the four
//          waves: per-wave maxima go through LDS; the transposed bytes are staged in
//          LDS and leave as 128-byte column segments. AR and AC together make both
//          activation copies from one read of x.
//   W  (128 x 128 weight blocks): one amax per tile (lane, wave, then LDS across
//          waves); the row copy (WR) is stored directly, the transposed copy (WC)
//          through LDS.
// The quotients are IEEE binary32 x / s, correctly rounded; |x / s| is clamped to 448
// before the E4M3 convert, which equals saturation (the convert itself does not
// saturate). Each block computes r = 1 / s once (correctly rounded division) and each
// element takes Markstein's correction of y = x r: q = fma(-e, r, y) with the residual
// e = fma(y, s, -x). An exhaustive check on MI355X over every binary32 significand of s
// and every BF16 significand of x (both signs; 2^31 cases) found q equal to the
// correctly rounded quotient in all of them; scaling both by powers of two keeps that
// while r, y and the residual stay normal, which holds whenever s >= 2^-92 for every
// element whose E4M3 code is not zero (|x / s| >= 2^-10). Negating x negates y, e and q
// exactly, and the residual's order of operands keeps the sign of a zero x (x = -0
// gives e = +0, q = -0 + -0 = -0). Blocks with a smaller s keep the division. With
// s >= 2^-92 the scale is normal and |x / s| <= 448 (1 + 2^-23), which the convert
// rounds to 448: only the division path needs the clamp.
#include "common.h"

namespace mxq {

// Block scale s -> its reciprocal for the corrected products (0 when s is zero or below
// 2^-92: those blocks divide).
__device__ __forceinline__ float block_recip(float s) { return s >= 0x1p-92f ? 1.0f / s : 0.0f; }

// x / s, correctly rounded, through the reciprocal r of the block (see the file comment)
__device__ __forceinline__ float quot_r(float x, float s, float r) {
  const float y = x * r;
  return __builtin_fmaf(-__builtin_fmaf(y, s, -x), r, y);
}

// Eight BF16 values (one uint4) / s -> eight E4M3 bytes (element 0 in the low byte).
__device__ __forceinline__ uint2 fp8x8_div(const uint4& v, float s, float r) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(w[i]); f[2 * i + 1] = bf16_hi(w[i]); }
  uint32_t o[2] = {0u, 0u};
  if (r != 0.0f) {                       // |q| <= 448 (1 + 2^-23): converts to at most 448
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = quot_r(f[i], s, r);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i / 2] = cvt_fp8x2_f32(o[i / 2], f[2 * i], f[2 * i + 1], 1.0f, (i & 1) != 0);
    return make_uint2(o[0], o[1]);
  }
  if (s > 0.0f) {                        // tiny block scale: divide
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] / s;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] *= 0.0f;     // all-zero block: keep the sign of zero
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = fminf(fmaxf(f[2 * i], -kE4M3Max), kE4M3Max);
    const float b = fminf(fmaxf(f[2 * i + 1], -kE4M3Max), kE4M3Max);
    o[i / 2] = cvt_fp8x2_f32(o[i / 2], a, b, 1.0f, (i & 1) != 0);
  }
  return make_uint2(o[0], o[1]);
}

__device__ __forceinline__ uint32_t amax8(const uint4& v) {
  return max_halves(pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                               pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu)));
}

__device__ __forceinline__ float block_scale(uint32_t amax_bits) {
  return __uint_as_float(amax_bits << 16) / kE4M3Max;     // 0 for an all-zero block
}

template <bool AR, bool AC, bool WR, bool WC>
__global__ void __launch_bounds__(256)
fp8_block_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
                 uint8_t* __restrict__ q_row, float* __restrict__ s_row,
                 uint8_t* __restrict__ q_colT, float* __restrict__ s_colT, int64_t col_tiles) {
  constexpr bool W = WR || WC, DO_COL = AC || WC;
  static_assert(!(W && (AR || AC)), "one kind of tiles per launch");
  __shared__ __attribute__((aligned(16))) uint8_t lcol[DO_COL ? 128 * 128 : 16];
  __shared__ uint32_t lmax[4 * 128];                 // per-wave column maxima (AC) / wave maxima (W)
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int m = lane >> 4, c16 = lane & 15;
  const int64_t band = blockIdx.x / col_tiles, ct = blockIdx.x % col_tiles;
  const int64_t R0 = band * 128, C0 = ct * 128;
  const int rl0 = 32 * w + 8 * m;
  const int64_t c = C0 + 8 * c16;
  const bool col_ok = c < cols;                      // cols % 8 == 0 (% 128 with AR or W)
  uint4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = R0 + rl0 + j;
    v[j] = (col_ok && r < rows) ? load_stream16(x + r * ld_x + c) : make_uint4(0, 0, 0, 0);
  }

  if constexpr (AR) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t a = amax8(v[j]), b;
      b = dpp_xor1(a); a = a > b ? a : b;
      b = dpp_xor2(a); a = a > b ? a : b;
      b = shfl_xor_u32(a, 4); a = a > b ? a : b;
      b = shfl_xor_u32(a, 8); a = a > b ? a : b;
      const float s = block_scale(a);
      const int64_t r = R0 + rl0 + j;
      if (col_ok && r < rows) {
        *reinterpret_cast<uint2*>(q_row + r * cols + c) = fp8x8_div(v[j], s, block_recip(s));
        if (c16 == 0) s_row[r * (cols / 128) + ct] = s;
      }
    }
  }

  float s_tile = 0.0f;                   // W
  float s_col[8];                        // AC: the scales of this lane's 8 columns
  if constexpr (W) {
    uint32_t a = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = max(a, amax8(v[j]));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) a = max(a, shfl_xor_u32(a, d));
    if (lane == 0) lmax[w] = a;
    __syncthreads();
    a = max(max(lmax[0], lmax[1]), max(lmax[2], lmax[3]));
    s_tile = block_scale(a);
  }
  if constexpr (AC) {
    // column maxima over this lane's 8 rows (two columns per dword), then the wave's 32 rows
    uint32_t cm[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t a = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t wd = p == 0 ? v[j].x : p == 1 ? v[j].y : p == 2 ? v[j].z : v[j].w;
        a = pk_max_u16(a, wd & 0x7FFF7FFFu);
      }
      a = pk_max_u16(a, shfl_xor_u32(a, 16));
      a = pk_max_u16(a, shfl_xor_u32(a, 32));
      cm[p] = a;
    }
    if (m == 0) {
#pragma unroll
      for (int p = 0; p < 4; ++p) lmax[w * 128 + 8 * c16 + 2 * p] = cm[p];   // packed pair at the even column
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t a = cm[p];
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) a = pk_max_u16(a, lmax[ww * 128 + 8 * c16 + 2 * p]);
      s_col[2 * p] = block_scale(a & 0xFFFFu);
      s_col[2 * p + 1] = block_scale(a >> 16);
    }
  }

  const float r_tile = block_recip(s_tile);
  if constexpr (WR) {                    // weight row copy, stored directly
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t r = R0 + rl0 + j;
      if (col_ok && r < rows) *reinterpret_cast<uint2*>(q_row + r * cols + c) = fp8x8_div(v[j], s_tile, r_tile);
    }
    if (threadIdx.x == 0) s_row[band * col_tiles + ct] = s_tile;
  }
  if constexpr (DO_COL) {
    // column cc of this lane: its 8 rows -> 8 bytes of the transposed tile (granule
    // swizzle as in the MXFP8 quantizer)
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      float s, rc;
      if constexpr (WC) { s = s_tile; rc = r_tile; }
      else { s = s_col[cc]; rc = block_recip(s); }
      const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
      uint32_t wd[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t p = cc >> 1;
        wd[j] = p == 0 ? v[j].x : p == 1 ? v[j].y : p == 2 ? v[j].z : v[j].w;
      }
      const uint4 col8 = make_uint4(__builtin_amdgcn_perm(wd[1], wd[0], sel), __builtin_amdgcn_perm(wd[3], wd[2], sel),
                                    __builtin_amdgcn_perm(wd[5], wd[4], sel), __builtin_amdgcn_perm(wd[7], wd[6], sel));
      const int cl = 8 * c16 + cc;
      const int g = (4 * w + m) ^ ((c16 & 3) * 4);
      *reinterpret_cast<uint2*>(lcol + cl * 128 + g * 8) = fp8x8_div(col8, s, rc);
    }
    __syncthreads();
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = k * 256 + t;
      const int cl = i / 8, ch = i % 8;
      const int g0 = (ch * 2) ^ (((cl >> 3) & 3) * 4);
      const int64_t col = C0 + cl, r = R0 + 16 * ch;
      if (col < cols && r < rows)
        *reinterpret_cast<uint4*>(q_colT + col * rows + r) = *reinterpret_cast<const uint4*>(lcol + cl * 128 + g0 * 8);
    }
    if constexpr (AC) {
      // lanes with m == 0 of wave 0 hold the scales of all 128 columns (8 each)
      if (w == 0 && m == 0) {
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const int64_t col = C0 + 8 * c16 + cc;
          if (col < cols) s_colT[col * (rows / 128) + band] = s_col[cc];
        }
      }
    } else {
      if (threadIdx.x == 0) s_colT[ct * (rows / 128) + band] = s_tile;
    }
  }
}

// weight = 0: activation tiles, 1 x 128 row copy (q_row, s_row) and/or 128 x 1 transposed
// copy (q_colT, s_colT); weight = 1: 128 x 128 blocks, either or both copies.
hipError_t launch_quant_fp8_block(int weight, const void* x, int64_t rows, int64_t cols, int64_t ld_x, void* q_row,
                                  float* s_row, void* q_colT, float* s_colT, hipStream_t st) {
  const int64_t col_tiles = (cols + 127) / 128;
  const int64_t blocks = (rows + 127) / 128 * col_tiles;
  if (blocks == 0) return hipSuccess;
  dim3 grid((unsigned)blocks), block(256);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint8_t *qr = (uint8_t*)q_row, *qc = (uint8_t*)q_colT;
#define MXQ_FP8B(AR, AC, WR, WC) \
  hipLaunchKernelGGL((fp8_block_kernel<AR, AC, WR, WC>), grid, block, 0, st, xp, rows, cols, ld_x, qr, s_row, qc, s_colT, col_tiles)
  if (!weight) {
    if (qr && qc) MXQ_FP8B(true, true, false, false);
    else if (qr) MXQ_FP8B(true, false, false, false);
    else MXQ_FP8B(false, true, false, false);
  } else {
    if (qr && qc) MXQ_FP8B(false, false, true, true);
    else if (qr) MXQ_FP8B(false, false, true, false);
    else MXQ_FP8B(false, false, false, true);
  }
#undef MXQ_FP8B
  return hipGetLastError();
}

}  // namespace mxq
