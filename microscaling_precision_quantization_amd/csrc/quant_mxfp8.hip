// MXFP8 / MXFP4 quantizer: rowwise 1x32 and columnwise 32x1 copies from one HBM read.
//
// Operation (restated from the pages): 32 consecutive E4M3 values share one
// E8M0 scale ("Miles Blackwell RL", remio.ai, section "La Compatibilidad de
// Miles Blackwell Ahora Abarca Todo el Ciclo de RL"); the rowwise and
// columnwise copies are both made from the original BF16 tensor, because each
// GEMM needs its blocks along its own reduction dimension (same page, section
// "Un Cuantizador Compartido Es el Mecanismo Real"; aib.vote, MXFP8 paragraph).
//
// Work decomposition: a workgroup (4 waves) owns a 128 x 128 BF16 tile; wave w
// owns rows 32w .. 32w+31 of it. Lane = 16*m + c16 holds rows 8m .. 8m+7 and
// columns 8*c16 .. 8*c16+7 of its wave's 32 x 128 slab as eight 16-byte loads
// (each load instruction of the wave reads 4 full 256-byte row segments).
//   * rowwise block (1 row x 32 cols) = 4 consecutive lanes: amax via two DPP
//     quad exchanges; each lane converts and stores its 8 bytes (16 lanes write
//     one 128-byte row segment).
//   * columnwise block (32 rows x 1 col) = the 4 lanes c16, c16+16, c16+32,
//     c16+48: amax via two lane-xor exchanges; each lane converts its 8 rows of
//     a column into 8 bytes of the transposed copy, which go to LDS first: the
//     workgroup then writes every column of its tile as one 128-byte segment
//     (16 bytes per lane) instead of four scattered 32-byte pieces.
//   * scales: the 4 row scales of a row and the 4 column scales of a column
//     in the tile are gathered in LDS and leave as one dword each.
// The BF16 values are converted straight from their packed form with the
// gfx950 scaled converts (1 instruction per 2 values).
#include "common.h"

namespace mxq {

// Eight BF16 values (one uint4, element 0 first) times 2^(127 - s) (exact) -> eight E2M1
// nibbles, RNE, element 0 in the low nibble.
__device__ __forceinline__ uint32_t fp4x8_scaled(const uint4& v, float inv) {
  uint32_t o = 0;
  o = cvt_fp4x2_f32<0>(o, bf16_lo(v.x) * inv, bf16_hi(v.x) * inv);
  o = cvt_fp4x2_f32<1>(o, bf16_lo(v.y) * inv, bf16_hi(v.y) * inv);
  o = cvt_fp4x2_f32<2>(o, bf16_lo(v.z) * inv, bf16_hi(v.z) * inv);
  o = cvt_fp4x2_f32<3>(o, bf16_lo(v.w) * inv, bf16_hi(v.w) * inv);
  return o;
}

// Up to kMaxQJobs tensors per launch (e.g. the input, weight and gradient of a linear
// layer): workgroups [block0, block0 + blocks) of the grid belong to job j.
constexpr int kMaxQJobs = 8;
struct QJob {
  const uint16_t* x;
  int64_t rows, cols, ld_x;
  uint8_t *q_row, *s_row, *q_colT, *s_colT;
  int64_t col_tiles, block0;
  int row_scale_dw, col_scale_dw;   // dword scale stores allowed (4-byte aligned scale rows)
};
struct QJobs {
  QJob j[kMaxQJobs];
  int n;
};

// FP4 = MXFP4 (E2M1 elements, same E8M0 blocks of 32, packed two per byte, low nibble first).
template <bool DO_ROW, bool DO_COL, bool FP4 = false>
__global__ void __launch_bounds__(256)
quant_mxfp8_kernel(const QJobs jobs) {
  // job of this workgroup (static indices only: the table stays in kernel arguments)
  QJob jb = jobs.j[0];
#pragma unroll
  for (int i = 1; i < kMaxQJobs; ++i)
    if (i < jobs.n && (int64_t)blockIdx.x >= jobs.j[i].block0) jb = jobs.j[i];
  const uint16_t* __restrict__ x = jb.x;
  const int64_t rows = jb.rows, cols = jb.cols, ld_x = jb.ld_x, col_tiles = jb.col_tiles;
  uint8_t* __restrict__ q_row = jb.q_row;
  uint8_t* __restrict__ s_row = jb.s_row;
  uint8_t* __restrict__ q_colT = jb.q_colT;
  uint8_t* __restrict__ s_colT = jb.s_colT;
  const int row_scale_dw = jb.row_scale_dw, col_scale_dw = jb.col_scale_dw;
  const int64_t blk = (int64_t)blockIdx.x - jb.block0;
  // Transposed tile: column cl at cl * CP (128 bytes FP8, 64 FP4); its granule g (rows
  // 8g .. 8g+7: 8 bytes FP8, 4 FP4) sits at granule g ^ 4 * (cl / 8 % 4), which spreads one
  // wave's writes over more banks.
  constexpr int CP = FP4 ? 64 : 128, GB = FP4 ? 4 : 8;
  __shared__ __attribute__((aligned(16))) uint8_t lcol[DO_COL ? 128 * CP : 16];
  __shared__ uint32_t lsrow[DO_ROW ? 128 : 1];     // 4 row-scale bytes per tile row
  __shared__ uint32_t lscol[DO_COL ? 128 : 1];     // 4 column-scale bytes per tile column
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int m = lane >> 4;          // row group of 8 inside the wave slab
  const int c16 = lane & 15;        // column group of 8 inside the 128 columns
  const int64_t band = blk / col_tiles;
  const int64_t ct = blk % col_tiles;
  const int64_t R0 = band * 128, C0 = ct * 128;
  const int rl0 = 32 * w + 8 * m;   // tile row of v[0]
  const int64_t c = C0 + 8 * c16;
  const bool col_ok = c < cols;     // cols % 32 == 0: 4-lane groups agree

  uint4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = R0 + rl0 + j;
    v[j] = (col_ok && r < rows) ? load_stream16(x + r * ld_x + c) : make_uint4(0, 0, 0, 0);
  }

  if (DO_ROW) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t a = pk_max_u16(pk_max_u16(v[j].x & 0x7FFF7FFFu, v[j].y & 0x7FFF7FFFu),
                              pk_max_u16(v[j].z & 0x7FFF7FFFu, v[j].w & 0x7FFF7FFFu));
      a = max_halves(a);
      uint32_t b = dpp_xor1(a);
      a = a > b ? a : b;
      b = dpp_xor2(a);
      a = a > b ? a : b;
      const int64_t r = R0 + rl0 + j;
      uint32_t s;
      if constexpr (FP4) {
        s = e8m0_from_bf16_amax_e2m1(a);
        const uint32_t packed = fp4x8_scaled(v[j], e8m0_inverse(s));
        if (col_ok && r < rows) *reinterpret_cast<uint32_t*>(q_row + r * (cols / 2) + c / 2) = packed;
      } else {
        s = e8m0_from_bf16_amax(a);
        const float sc = e8m0_to_float(s);
        uint32_t lo = cvt_fp8x2_bf16(0u, v[j].x, sc, false);
        lo = cvt_fp8x2_bf16(lo, v[j].y, sc, true);
        uint32_t hi = cvt_fp8x2_bf16(0u, v[j].z, sc, false);
        hi = cvt_fp8x2_bf16(hi, v[j].w, sc, true);
        if (col_ok && r < rows) *reinterpret_cast<uint2*>(q_row + r * cols + c) = make_uint2(lo, hi);
      }
      if ((c16 & 3) == 0) reinterpret_cast<uint8_t*>(lsrow)[(rl0 + j) * 4 + (c16 >> 2)] = (uint8_t)s;
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
        const uint32_t wd = p == 0 ? v[j].x : p == 1 ? v[j].y : p == 2 ? v[j].z : v[j].w;
        a = pk_max_u16(a, wd & 0x7FFF7FFFu);
      }
      a = pk_max_u16(a, shfl_xor_u32(a, 16));
      a = pk_max_u16(a, shfl_xor_u32(a, 32));
      cm[p] = a;
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const uint32_t amax = (cc & 1) ? (cm[cc >> 1] >> 16) : (cm[cc >> 1] & 0xFFFFu);
      const uint32_t s = FP4 ? e8m0_from_bf16_amax_e2m1(amax) : e8m0_from_bf16_amax(amax);
      const float sc = e8m0_to_float(s);
      const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
      uint32_t wd[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t p = cc >> 1;
        wd[j] = p == 0 ? v[j].x : p == 1 ? v[j].y : p == 2 ? v[j].z : v[j].w;
      }
      const int cl = 8 * c16 + cc;
      const int g = (4 * w + m) ^ ((c16 & 3) * 4);
      if constexpr (FP4) {
        // rows j of column cc -> 8 nibbles, row order
        const uint4 col8 = make_uint4(__builtin_amdgcn_perm(wd[1], wd[0], sel), __builtin_amdgcn_perm(wd[3], wd[2], sel),
                                      __builtin_amdgcn_perm(wd[5], wd[4], sel), __builtin_amdgcn_perm(wd[7], wd[6], sel));
        *reinterpret_cast<uint32_t*>(lcol + cl * CP + g * GB) = fp4x8_scaled(col8, e8m0_inverse(s));
      } else {
        // pair (row j, row j+1) of column cc -> one packed BF16x2 dword
        uint32_t out0 = cvt_fp8x2_bf16(0u, __builtin_amdgcn_perm(wd[1], wd[0], sel), sc, false);
        out0 = cvt_fp8x2_bf16(out0, __builtin_amdgcn_perm(wd[3], wd[2], sel), sc, true);
        uint32_t out1 = cvt_fp8x2_bf16(0u, __builtin_amdgcn_perm(wd[5], wd[4], sel), sc, false);
        out1 = cvt_fp8x2_bf16(out1, __builtin_amdgcn_perm(wd[7], wd[6], sel), sc, true);
        *reinterpret_cast<uint2*>(lcol + cl * CP + g * GB) = make_uint2(out0, out1);
      }
      if (m == 0) reinterpret_cast<uint8_t*>(lscol)[cl * 4 + w] = (uint8_t)s;
    }
  }
  __syncthreads();

  const int t = threadIdx.x;
  if (DO_COL) {
    // 16-byte chunk i = k * 256 + t of the tile's transposed copy: column i / NCH, rows
    // (128 / NCH) (i % NCH) .. (FP8: 8 chunks of 16 rows; FP4: 4 chunks of 32 rows).
    // rows % 32 == 0, so a chunk is either wholly inside the tensor or wholly outside.
    constexpr int NCH = CP / 16, RPC = 128 / NCH;
#pragma unroll
    for (int k = 0; k < NCH / 2; ++k) {
      const int i = k * 256 + t;
      const int cl = i / NCH, ch = i % NCH;
      const int g0 = (ch * (16 / GB)) ^ (((cl >> 3) & 3) * 4);   // the chunk's granules stay adjacent
      const int64_t col = C0 + cl, r = R0 + RPC * ch;
      if (col < cols && r < rows)
        *reinterpret_cast<uint4*>(q_colT + col * (FP4 ? rows / 2 : rows) + (FP4 ? r / 2 : r)) =
            *reinterpret_cast<const uint4*>(lcol + cl * CP + g0 * GB);
    }
    if (t < 128 && C0 + t < cols) {
      const int64_t sb = rows / 32;
      uint8_t* dst = s_colT + (C0 + t) * sb + band * 4;
      const int64_t ns = min((int64_t)4, sb - band * 4);
      if (col_scale_dw && ns == 4) {
        *reinterpret_cast<uint32_t*>(dst) = lscol[t];
      } else {
        for (int b = 0; b < ns; ++b) dst[b] = (uint8_t)(lscol[t] >> (8 * b));
      }
    }
  }
  if (DO_ROW && t < 128 && R0 + t < rows) {
    const int64_t sb = cols / 32;
    uint8_t* dst = s_row + (R0 + t) * sb + ct * 4;
    const int64_t nb = min((int64_t)4, sb - ct * 4);
    if (row_scale_dw && nb == 4) {
      *reinterpret_cast<uint32_t*>(dst) = lsrow[t];
    } else {
      for (int b = 0; b < nb; ++b) dst[b] = (uint8_t)(lsrow[t] >> (8 * b));
    }
  }
}

// Tensors of one launch must request the same copies (row, column or both).
template <bool FP4>
static hipError_t launch_quant_mx_multi(int n, const void* const* x, const int64_t* rows, const int64_t* cols,
                                        const int64_t* ld_x, void* const* q_row, void* const* s_row,
                                        void* const* q_colT, void* const* s_colT, hipStream_t stream) {
  QJobs jobs;
  jobs.n = n;
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    QJob& j = jobs.j[i];
    j.x = static_cast<const uint16_t*>(x[i]);
    j.rows = rows[i]; j.cols = cols[i]; j.ld_x = ld_x[i];
    j.q_row = (uint8_t*)q_row[i]; j.s_row = (uint8_t*)s_row[i];
    j.q_colT = (uint8_t*)q_colT[i]; j.s_colT = (uint8_t*)s_colT[i];
    j.col_tiles = (cols[i] + 127) / 128;
    j.block0 = blocks;
    blocks += (rows[i] + 127) / 128 * j.col_tiles;
    j.row_scale_dw = j.s_row && ((uintptr_t)j.s_row & 3) == 0 && (cols[i] / 32) % 4 == 0;
    j.col_scale_dw = j.s_colT && ((uintptr_t)j.s_colT & 3) == 0 && (rows[i] / 32) % 4 == 0;
  }
  if (blocks == 0) return hipSuccess;
  dim3 grid((unsigned)blocks), block(256);
  const bool do_row = q_row[0] != nullptr, do_col = q_colT[0] != nullptr;
  if (do_row && do_col) hipLaunchKernelGGL((quant_mxfp8_kernel<true, true, FP4>), grid, block, 0, stream, jobs);
  else if (do_row) hipLaunchKernelGGL((quant_mxfp8_kernel<true, false, FP4>), grid, block, 0, stream, jobs);
  else hipLaunchKernelGGL((quant_mxfp8_kernel<false, true, FP4>), grid, block, 0, stream, jobs);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp8_multi(int n, const void* const* x, const int64_t* rows, const int64_t* cols,
                                    const int64_t* ld_x, void* const* q_row, void* const* s_row,
                                    void* const* q_colT, void* const* s_colT, hipStream_t stream) {
  return launch_quant_mx_multi<false>(n, x, rows, cols, ld_x, q_row, s_row, q_colT, s_colT, stream);
}

hipError_t launch_quant_mxfp4_multi(int n, const void* const* x, const int64_t* rows, const int64_t* cols,
                                    const int64_t* ld_x, void* const* q_row, void* const* s_row,
                                    void* const* q_colT, void* const* s_colT, hipStream_t stream) {
  return launch_quant_mx_multi<true>(n, x, rows, cols, ld_x, q_row, s_row, q_colT, s_colT, stream);
}

hipError_t launch_quant_mxfp4(const void* x, int64_t rows, int64_t cols, int64_t ld_x, void* q_row, void* s_row,
                              void* q_colT, void* s_colT, hipStream_t stream) {
  return launch_quant_mx_multi<true>(1, &x, &rows, &cols, &ld_x, &q_row, &s_row, &q_colT, &s_colT, stream);
}

hipError_t launch_quant_mxfp8(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                              void* q_row, void* s_row, void* q_colT, void* s_colT,
                              hipStream_t stream) {
  return launch_quant_mxfp8_multi(1, &x, &rows, &cols, &ld_x, &q_row, &s_row, &q_colT, &s_colT, stream);
}

}  // namespace mxq
