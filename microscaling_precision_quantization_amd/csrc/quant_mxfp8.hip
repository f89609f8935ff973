// MXFP8 quantizer: rowwise 1x32 and columnwise 32x1 copies from one HBM read.
//
// Operation (restated from the pages): 32 consecutive E4M3 values share one
// E8M0 scale ("Miles Blackwell RL", remio.ai, section "La Compatibilidad de
// Miles Blackwell Ahora Abarca Todo el Ciclo de RL"); the rowwise and
// columnwise copies are both made from the original BF16 tensor, because each
// GEMM needs its blocks along its own reduction dimension (same page, section
// "Un Cuantizador Compartido Es el Mecanismo Real"; aib.vote, MXFP8 paragraph).
//
// Work decomposition (one wave = 32 rows x 128 columns of BF16 = 8 KiB):
//   lane = 16*m + c16 holds rows 8m .. 8m+7 and columns 8*c16 .. 8*c16+7 of
//   its wave's slab as eight 16-byte loads (each load instruction of the wave
//   reads 4 full 256-byte row segments: fully coalesced).
//   * rowwise block (1 row x 32 cols) = 4 consecutive lanes: amax via two DPP
//     quad exchanges; each lane converts and stores its 8 bytes.
//   * columnwise block (32 rows x 1 col) = the 4 lanes c16, c16+16, c16+32,
//     c16+48: amax via two lane-xor exchanges; each lane converts its 8 rows
//     of a column into 8 consecutive bytes of the transposed copy.
//   No LDS is needed: the register tile of a lane already covers 8 rows.
// The BF16 values are converted straight from their packed form with the
// gfx950 scaled converts (1 instruction per 2 values).
#include "common.h"

namespace mxq {

template <bool DO_ROW, bool DO_COL>
__global__ void __launch_bounds__(256)
quant_mxfp8_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
                   uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                   uint8_t* __restrict__ q_colT, uint8_t* __restrict__ s_colT,
                   int64_t col_tiles) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane >> 4;          // row group of 8 inside the wave slab
  const int c16 = lane & 15;        // column group of 8 inside the 128 columns
  const int64_t slab = (int64_t)blockIdx.x / col_tiles * 4 + wave;   // 32-row slab index
  const int64_t ct = (int64_t)blockIdx.x % col_tiles;
  const int64_t r0 = slab * 32 + 8 * m;
  const int64_t c = ct * 128 + 8 * c16;
  if (slab * 32 >= rows) return;                 // whole wave out of range (uniform)
  const bool col_ok = c < cols;                  // cols % 32 == 0: 4-lane groups agree

  uint4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool ok = col_ok && (r0 + j < rows);
    v[j] = ok ? *reinterpret_cast<const uint4*>(x + (r0 + j) * ld_x + c) : make_uint4(0, 0, 0, 0);
  }

  if (DO_ROW) {
    const int64_t sblocks = cols / 32;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t a = pk_max_u16(pk_max_u16(v[j].x & 0x7FFF7FFFu, v[j].y & 0x7FFF7FFFu),
                              pk_max_u16(v[j].z & 0x7FFF7FFFu, v[j].w & 0x7FFF7FFFu));
      a = max_halves(a);
      uint32_t b = dpp_xor1(a);
      a = a > b ? a : b;
      b = dpp_xor2(a);
      a = a > b ? a : b;
      const uint32_t s = e8m0_from_bf16_amax(a);
      const float sc = e8m0_to_float(s);
      uint32_t lo = cvt_fp8x2_bf16(0u, v[j].x, sc, false);
      lo = cvt_fp8x2_bf16(lo, v[j].y, sc, true);
      uint32_t hi = cvt_fp8x2_bf16(0u, v[j].z, sc, false);
      hi = cvt_fp8x2_bf16(hi, v[j].w, sc, true);
      const int64_t r = r0 + j;
      if (col_ok && r < rows) {
        *reinterpret_cast<uint2*>(q_row + r * cols + c) = make_uint2(lo, hi);
        if ((c16 & 3) == 0) s_row[r * sblocks + c / 32] = (uint8_t)s;
      }
    }
  }

  if (DO_COL) {
    // Column maxima over this lane's 8 rows, two columns per dword.
    uint32_t cm[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t a = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w = p == 0 ? v[j].x : p == 1 ? v[j].y : p == 2 ? v[j].z : v[j].w;
        a = pk_max_u16(a, w & 0x7FFF7FFFu);
      }
      a = pk_max_u16(a, shfl_xor_u32(a, 16));
      a = pk_max_u16(a, shfl_xor_u32(a, 32));
      cm[p] = a;
    }
    const int64_t sblocks = rows / 32;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const uint32_t amax = (cc & 1) ? (cm[cc >> 1] >> 16) : (cm[cc >> 1] & 0xFFFFu);
      const uint32_t s = e8m0_from_bf16_amax(amax);
      const float sc = e8m0_to_float(s);
      const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
      uint32_t w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t p = cc >> 1;
        w[j] = p == 0 ? v[j].x : p == 1 ? v[j].y : p == 2 ? v[j].z : v[j].w;
      }
      // pair (row j, row j+1) of column cc -> one packed BF16x2 dword
      uint32_t out0 = cvt_fp8x2_bf16(0u, __builtin_amdgcn_perm(w[1], w[0], sel), sc, false);
      out0 = cvt_fp8x2_bf16(out0, __builtin_amdgcn_perm(w[3], w[2], sel), sc, true);
      uint32_t out1 = cvt_fp8x2_bf16(0u, __builtin_amdgcn_perm(w[5], w[4], sel), sc, false);
      out1 = cvt_fp8x2_bf16(out1, __builtin_amdgcn_perm(w[7], w[6], sel), sc, true);
      if (col_ok) {
        const int64_t col = c + cc;
        *reinterpret_cast<uint2*>(q_colT + col * rows + r0) = make_uint2(out0, out1);
        if (m == 0) s_colT[col * sblocks + slab] = (uint8_t)s;
      }
    }
  }
}

hipError_t launch_quant_mxfp8(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                              void* q_row, void* s_row, void* q_colT, void* s_colT,
                              hipStream_t stream) {
  const int64_t col_tiles = (cols + 127) / 128;
  const int64_t slabs = (rows + 31) / 32;
  const int64_t blocks = (slabs + 3) / 4 * col_tiles;
  dim3 grid((unsigned)blocks), block(256);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint8_t *qr = (uint8_t*)q_row, *sr = (uint8_t*)s_row, *qc = (uint8_t*)q_colT, *sc = (uint8_t*)s_colT;
  if (q_row && q_colT)
    hipLaunchKernelGGL((quant_mxfp8_kernel<true, true>), grid, block, 0, stream, xp, rows, cols, ld_x, qr, sr, qc, sc, col_tiles);
  else if (q_row)
    hipLaunchKernelGGL((quant_mxfp8_kernel<true, false>), grid, block, 0, stream, xp, rows, cols, ld_x, qr, sr, qc, sc, col_tiles);
  else
    hipLaunchKernelGGL((quant_mxfp8_kernel<false, true>), grid, block, 0, stream, xp, rows, cols, ld_x, qr, sr, qc, sc, col_tiles);
  return hipGetLastError();
}

}  // namespace mxq
