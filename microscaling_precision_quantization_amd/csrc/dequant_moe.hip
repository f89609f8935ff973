// Dequantization and the MoE expert-layer glue (SwiGLU + per-row NVFP4 requant,
// weighted top-k combine).
//
// Dequantization serves the dequantized-backward mode: backward GEMMs run in
// BF16 on dequantizations of the exact low-precision forward operands
// ("Miles Blackwell RL", remio.ai, section "La Compatibilidad de Miles
// Blackwell Ahora Abarca Todo el Ciclo de RL"; aib.vote, backward paragraph).
//   v = fl(fl(q * S) * t)  (q * S exact; MXFP8 and MXFP4 have no t), BF16 = RNE(v).
// SwiGLU experts with gate and up in one fused GEMM, and per-token NVFP4 on the
// expert activations: remio.ai, sections "Un Cuantizador Compartido Es el
// Mecanismo Real" and "La Compatibilidad ...".
#include <type_traits>

#include "common.h"

namespace mxq {

typedef float f32x4_nt __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Dequantize: one thread per 16 consecutive elements of a row.
// FMT: 1 MXFP8, 2 NVFP4, 4 MXFP4.
// ---------------------------------------------------------------------------
template <int FMT, bool OUT_F32>
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s, const float* __restrict__ t,
               int t_mode, int64_t group_rows, int64_t rows, int64_t cols, void* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = cols / 16;
  if (idx >= rows * per_row) return;
  const int64_t r = idx / per_row, c0 = (idx % per_row) * 16;
  float v[16];
  // 16 E2M1 codes (8 bytes) -> v[0..15], scaled by sc (exact: E2M1 * E4M3 or * 2^k)
  auto fp4x16 = [&](uint32_t w0, uint32_t w1, float sc) {
    const uint32_t w[2] = {w0, w1};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const v2f_t e0 = e2m1x2_to_f32<0>(w[k]), e1 = e2m1x2_to_f32<1>(w[k]);
      const v2f_t e2 = e2m1x2_to_f32<2>(w[k]), e3 = e2m1x2_to_f32<3>(w[k]);
      v[8 * k + 0] = e0.x * sc; v[8 * k + 1] = e0.y * sc; v[8 * k + 2] = e1.x * sc; v[8 * k + 3] = e1.y * sc;
      v[8 * k + 4] = e2.x * sc; v[8 * k + 5] = e2.y * sc; v[8 * k + 6] = e3.x * sc; v[8 * k + 7] = e3.y * sc;
    }
  };
  if (FMT == 1) {
    const uint4 b = *reinterpret_cast<const uint4*>(q + r * cols + c0);
    const float sc = e8m0_to_float(s[r * (cols / 32) + c0 / 32]);
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = e4m3_to_f32((w[i / 4] >> (8 * (i % 4))) & 0xFF) * sc;
  } else if (FMT == 4) {
    const uint2 b = *reinterpret_cast<const uint2*>(q + r * (cols / 2) + c0 / 2);
    fp4x16(b.x, b.y, e8m0_to_float(s[r * (cols / 32) + c0 / 32]));
  } else {
    const uint2 b = *reinterpret_cast<const uint2*>(q + r * (cols / 2) + c0 / 2);
    const float tt = t_mode == 0 ? t[r] : t_mode == 1 ? t[0] : t[r / group_rows];
    fp4x16(b.x, b.y, e4m3_to_f32(s[r * (cols / 16) + c0 / 16]));   // q * S exact
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= tt;
  }
  if (OUT_F32) {
    float4* o = reinterpret_cast<float4*>((float*)out + r * cols + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  } else {
    uint32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = bf16x2_rne(v[2 * i], v[2 * i + 1]);
    uint4* o = reinterpret_cast<uint4*>((uint16_t*)out + r * cols + c0);
    o[0] = make_uint4(p[0], p[1], p[2], p[3]);
    o[1] = make_uint4(p[4], p[5], p[6], p[7]);
  }
}

// fmt: 1 MXFP8, 2 NVFP4, 4 MXFP4
hipError_t launch_dequant(int fmt, const void* q, const void* s, const float* t, int t_mode, int64_t group_rows,
                          int64_t rows, int64_t cols, void* out, int out_f32, hipStream_t st) {
  const int64_t n = rows * (cols / 16);
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  const uint8_t *qp = (const uint8_t*)q, *sp = (const uint8_t*)s;
  auto go = [&](auto K) {
    if (out_f32) hipLaunchKernelGGL((dequant_kernel<decltype(K)::value, true>), grid, block, 0, st, qp, sp, t, t_mode, group_rows, rows, cols, out);
    else hipLaunchKernelGGL((dequant_kernel<decltype(K)::value, false>), grid, block, 0, st, qp, sp, t, t_mode, group_rows, rows, cols, out);
  };
  if (fmt == 2) go(std::integral_constant<int, 2>{});
  else if (fmt == 4) go(std::integral_constant<int, 4>{});
  else go(std::integral_constant<int, 1>{});
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize + transpose (+ row gather): the BF16 operands of the backward GEMMs
// in the K-contiguous layout the "TN" GEMMs consume.
//   out[g][c][j] = BF16(deq(in[g * group_rows + src(j)][c])),  src(j) = src_row[j]
//   (a gather; -1 gives a zero column) or j. Tile: 64 output columns (j) x 64
//   input columns (c) per workgroup; each thread dequantizes 16 consecutive
//   elements of one input row, the tile is transposed through LDS and leaves as
//   16-byte row segments of the output.
// FMT: 1 MXFP8, 2 NVFP4, 3 BF16 (plain transpose).
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(256)
dequant_t_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s, const float* __restrict__ t,
                 int t_mode, int64_t group_rows, int64_t cols, const int32_t* __restrict__ src_row,
                 int64_t out_cols, uint16_t* __restrict__ out, int64_t ld_out) {
  constexpr int P = 72;                                   // LDS row pitch (BF16), 16-byte aligned rows
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * P];
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.z;
  const int64_t c0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  {
    const int jl = tid >> 2, cl = (tid & 3) * 16;
    const int64_t j = j0 + jl, c = c0 + cl;
    int64_t r = -1;
    if (j < out_cols && c < cols) {
      const int64_t sr = src_row ? (int64_t)src_row[j] : j;
      if (sr >= 0 && sr < group_rows) r = g * group_rows + sr;
    }
    uint32_t p[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (r >= 0) {
      if (FMT == 3) {
        const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) + r * cols + c);
        const uint4 a = src[0], b = src[1];
        p[0] = a.x; p[1] = a.y; p[2] = a.z; p[3] = a.w; p[4] = b.x; p[5] = b.y; p[6] = b.z; p[7] = b.w;
      } else {
        float v[16];
        if (FMT == 1) {
          const uint4 b = *reinterpret_cast<const uint4*>(q + r * cols + c);
          const float sc = e8m0_to_float(s[r * (cols / 32) + c / 32]);
          const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = e4m3_to_f32((w[i / 4] >> (8 * (i % 4))) & 0xFF) * sc;
        } else {
          const uint2 b = *reinterpret_cast<const uint2*>(q + r * (cols / 2) + c / 2);
          const float S = e4m3_to_f32(s[r * (cols / 16) + c / 16]);
          const float tt = t_mode == 0 ? t[r] : t_mode == 1 ? t[0] : t[r / group_rows];
          const uint32_t w[2] = {b.x, b.y};
#pragma unroll
          for (int k = 0; k < 2; ++k) {                     // (q * S) exact, then * t
            const v2f_t e0 = e2m1x2_to_f32<0>(w[k]), e1 = e2m1x2_to_f32<1>(w[k]);
            const v2f_t e2 = e2m1x2_to_f32<2>(w[k]), e3 = e2m1x2_to_f32<3>(w[k]);
            v[8 * k + 0] = (e0.x * S) * tt; v[8 * k + 1] = (e0.y * S) * tt;
            v[8 * k + 2] = (e1.x * S) * tt; v[8 * k + 3] = (e1.y * S) * tt;
            v[8 * k + 4] = (e2.x * S) * tt; v[8 * k + 5] = (e2.y * S) * tt;
            v[8 * k + 6] = (e3.x * S) * tt; v[8 * k + 7] = (e3.y * S) * tt;
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = bf16x2_rne(v[2 * i], v[2 * i + 1]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tile[(cl + 2 * i) * P + jl] = (uint16_t)(p[i] & 0xFFFFu);
      tile[(cl + 2 * i + 1) * P + jl] = (uint16_t)(p[i] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = k * 256 + tid;
    const int cl = i >> 3, jc = (i & 7) * 8;
    const int64_t c = c0 + cl, j = j0 + jc;
    if (c < cols && j < out_cols)
      {
        // non-temporal: the output is not read here, the (gathered) input rows stay in L2
        const uint4 vv = *reinterpret_cast<const uint4*>(tile + cl * P + jc);
        const u32x4_nt v4 = {vv.x, vv.y, vv.z, vv.w};
        __builtin_nontemporal_store(v4, reinterpret_cast<u32x4_nt*>(out + (g * cols + c) * ld_out + j));
      }
  }
}

// NVFP4 without a row gather: 128 output columns (input rows, in pairs) x 128 input
// columns per workgroup, so each input row of the tile is one 64-byte segment and each
// output row one 256-byte segment. Lane (row pair jp, 16-byte unit ul) dequantizes 32
// elements of two rows; the pairs go to LDS as dwords (row 2jp low, 2jp+1 high) at
// 4-dword chunk (jp / 4) ^ sw(c), sw(c) = 2 (c / 32) mod 16, which keeps a wave's pair
// writes on distinct banks. (Measured against the 64 x 64 kernel above: 256 DeepSeek-shaped
// gate_up expert weights (4096 x 7168) 5.04 -> 4.83 ms, 135k x 2048 slot activations
// 0.23 -> 0.17 ms; slower with a gather and for the other formats, which keep that kernel.)
// A workgroup takes two such tiles along the output columns and issues the loads of both
// before the first one's LDS pass and stores, so its reads overlap its own writes (the
// LDS tile limits a CU to five workgroups): 256 gate_up expert weights 4.77 -> 4.12 ms.
__global__ void __launch_bounds__(256)
dequant_t_nv_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s, const float* __restrict__ t,
                    int t_mode, int64_t group_rows, int64_t cols, int64_t out_cols, uint16_t* __restrict__ out,
                    int64_t ld_out) {
  constexpr int EPU = 32, UPR = 4, TC = UPR * EPU;        // 128 input columns
  constexpr int JT = 2;                                    // 128-row tiles per workgroup
  __shared__ __attribute__((aligned(16))) uint32_t tile[TC * 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t g = blockIdx.z;
  const int64_t c0 = (int64_t)blockIdx.y * TC;
  const int rr = lane / UPR, ul = lane % UPR;
  const int jp = w * 16 + rr;                              // 0..63
  const int64_t c = c0 + (int64_t)ul * EPU;
  const bool full = c + 32 <= cols;                        // else only the first 16 columns exist
  uint4 b[JT][2];
  uint32_t sb[JT][2];
  float tt[JT][2];
  bool ok[JT][2];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t j = ((int64_t)blockIdx.x * JT + jt) * 128 + 2 * jp + half;
      ok[jt][half] = j < out_cols && j < group_rows && c < cols;
      b[jt][half] = make_uint4(0, 0, 0, 0); sb[jt][half] = 0; tt[jt][half] = 0.0f;
      if (ok[jt][half]) {
        const int64_t r = g * group_rows + j;
        tt[jt][half] = t_mode == 0 ? t[r] : t_mode == 1 ? t[0] : t[r / group_rows];
        if (full) b[jt][half] = load_stream16(q + r * (cols / 2) + c / 2);
        else { const uint2 b2 = *reinterpret_cast<const uint2*>(q + r * (cols / 2) + c / 2); b[jt][half] = make_uint4(b2.x, b2.y, 0, 0); }
        sb[jt][half] = s[r * (cols / 16) + c / 16] | (full ? (uint32_t)s[r * (cols / 16) + c / 16 + 1] << 8 : 0u);
      }
    }
  const int sw = (2 * ul) & 15;
  const int pos = (((jp >> 2) ^ sw) << 2) | (jp & 3);
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    uint32_t lo[16], hi[16];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = 0;
      if (ok[jt][half]) {
        const float S0 = e4m3_to_f32(sb[jt][half] & 0xFFu);
        const float S1 = full ? e4m3_to_f32(sb[jt][half] >> 8) : 0.0f;
        const float tv = tt[jt][half];
        const uint32_t wd[4] = {b[jt][half].x, b[jt][half].y, b[jt][half].z, b[jt][half].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {                      // (q * S) exact, then * t
          const float S = k < 2 ? S0 : S1;
          const v2f_t e0 = e2m1x2_to_f32<0>(wd[k]), e1 = e2m1x2_to_f32<1>(wd[k]);
          const v2f_t e2 = e2m1x2_to_f32<2>(wd[k]), e3 = e2m1x2_to_f32<3>(wd[k]);
          p[4 * k + 0] = bf16x2_rne((e0.x * S) * tv, (e0.y * S) * tv);
          p[4 * k + 1] = bf16x2_rne((e1.x * S) * tv, (e1.y * S) * tv);
          p[4 * k + 2] = bf16x2_rne((e2.x * S) * tv, (e2.y * S) * tv);
          p[4 * k + 3] = bf16x2_rne((e3.x * S) * tv, (e3.y * S) * tv);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) (half ? hi : lo)[i] = p[i];
    }
    if (jt > 0) __syncthreads();                           // the previous tile's reads are done
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      tile[(ul * EPU + 2 * i) * 64 + pos] = (lo[i] & 0xFFFFu) | (hi[i] << 16);
      tile[(ul * EPU + 2 * i + 1) * 64 + pos] = (lo[i] >> 16) | (hi[i] & 0xFFFF0000u);
    }
    __syncthreads();
    const int64_t j0 = ((int64_t)blockIdx.x * JT + jt) * 128;
#pragma unroll
    for (int k = 0; k < TC * 16 / 256; ++k) {
      const int i = k * 256 + tid;
      const int cl = i >> 4, qq = i & 15;
      const int64_t cc = c0 + cl, j = j0 + 8 * qq;
      const int swc = (2 * (cl / EPU)) & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(tile + cl * 64 + ((qq ^ swc) << 2));
      if (cc < cols && j < out_cols) {
        const u32x4_nt v4 = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(v4, reinterpret_cast<u32x4_nt*>(out + (g * cols + cc) * ld_out + j));
      }
    }
  }
}

hipError_t launch_dequant_t(int fmt, const void* q, const void* s, const float* t, int t_mode, int64_t groups,
                            int64_t group_rows, int64_t cols, const int32_t* src_row, int64_t out_cols, void* out,
                            int64_t ld_out, hipStream_t st) {
  const uint8_t *qp = (const uint8_t*)q, *sp = (const uint8_t*)s;
  uint16_t* o = (uint16_t*)out;
  if (fmt == 2 && !src_row) {
    dim3 g2((unsigned)((out_cols + 255) / 256), (unsigned)((cols + 127) / 128), (unsigned)groups), b2(256);
    hipLaunchKernelGGL(dequant_t_nv_kernel, g2, b2, 0, st, qp, sp, t, t_mode, group_rows, cols, out_cols, o, ld_out);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((out_cols + 63) / 64), (unsigned)((cols + 63) / 64), (unsigned)groups), block(256);
  if (fmt == 1) hipLaunchKernelGGL((dequant_t_kernel<1>), grid, block, 0, st, qp, sp, t, t_mode, group_rows, cols, src_row, out_cols, o, ld_out);
  else if (fmt == 2) hipLaunchKernelGGL((dequant_t_kernel<2>), grid, block, 0, st, qp, sp, t, t_mode, group_rows, cols, src_row, out_cols, o, ld_out);
  else hipLaunchKernelGGL((dequant_t_kernel<3>), grid, block, 0, st, qp, sp, t, t_mode, group_rows, cols, src_row, out_cols, o, ld_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SwiGLU + per-row NVFP4: one wave per slot row; the row stays in registers.
// h = silu(g) * u = g u / (1 + e^(-g)), rounded once to BF16 (nearest, ties to even)
// from its exact value, then the per-token quantizer's arithmetic on the BF16 row.
// ---------------------------------------------------------------------------
// binary64 -> BF16 bits, one rounding: the binary32 conversion is turned into
// round-to-odd (an inexact result is truncated toward zero and gets its last bit set),
// and round-to-odd to 24 bits followed by nearest-even to 8 bits equals nearest-even
// to 8 bits directly (24 >= 8 + 2). Values past the binary32 range come out as
// FLT_MAX | 1 and then round to +-Inf, values below its subnormals as +-2^-149 and
// then to a signed zero, as the direct rounding gives.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  float f = (float)d;
  if ((double)f != d) {
    uint32_t b = __float_as_uint(f);
    if (fabs((double)f) > fabs(d)) b -= 1u;          // magnitude rounded up: step back
    f = __uint_as_float(b | 1u);
  }
  return f32_to_bf16_rne(f);
}

// h in binary64 from P = g u (exact: two 24-bit significands):
//   g >= 0: h = P - C with C = P e / (1 + e), e = e^(-g) <= 1 (so C <= P / 2);
//   g <  0: h = P e / (1 + e) with e = e^g < 1 (a vanishing e gives a zero with the
//           sign of P, which is how the exact value, below 1e-300 in magnitude, rounds).
// Either way h is within a few binary64 ulps of the exact value, so its BF16 rounding is
// the correctly rounded one, except when h itself lands on a BF16 rounding midpoint.
// For g > 0 that happens systematically, not by accident: once C drops below half an
// ulp of P (g above ~37), h = P, and a product of two binary32 values is often a BF16
// midpoint. The exact value is P - C_exact with C_exact > 0, so its side of the midpoint
// is the sign of (|P| - |h|) - |C| (the first difference is exact): the magnitude rounds
// up only if that is positive, else toward zero -- also when C underflowed to 0, since
// the exact value stays strictly inside |P|. For g <= 0 a midpoint can only be hit by
// chance (about 2^-44 per element); it then rounds to even.
__device__ __noinline__ uint32_t swiglu_bf16_f64(float g, float u) {
  const double gd = g, P = (double)g * (double)u;
  double h, C = 0.0;
  if (gd >= 0.0) {
    const double e = exp(-gd);
    C = P * (e / (1.0 + e));
    h = C == 0.0 ? P : P - C;                          // keeps the sign of a zero P
  } else {
    const double e = exp(gd);
    h = P * (e / (1.0 + e));
  }
  if (gd > 0.0 && h != 0.0) {
    // is |h| a midpoint of the BF16 grid (quantum 2^(max(E, -126) - 7), |h| in [2^E, 2^(E+1)))?
    const double a = fabs(h);
    int E;
    frexp(a, &E);                                      // a = f 2^E, f in [0.5, 1)
    const double q = ldexp(1.0, (E - 1 > -126 ? E - 1 : -126) - 7);
    const double t = a / q, lo = floor(t);             // both exact: q is a power of two
    if (t - lo == 0.5) {
      const bool up = (fabs(P) - a) > fabs(C);         // |P| - |h| is exact (Sterbenz)
      const double r = (up ? lo + 1.0 : lo) * q;       // a BF16 value (or 2^128)
      return f32_to_bf16_rne((float)copysign(r, h));   // exact conversions
    }
  }
  return f64_to_bf16_rne(h);
}

// The same BF16 value, mostly from binary32: for |g| <= 80, h32 = (g / (1 + e^-g)) u
// with the accurate expf and correctly rounded division is within 2^-21 of h relative
// (a few roundings of 2^-24 each and the exponential's error), i.e. within 8 binary32
// ulps. Where h32 is a normal number more than 64 ulps away from every BF16 rounding
// midpoint (its 16 bits below the BF16 precision differ from 0x8000 by more than 64),
// the exact h lies on the same side of every midpoint, so rounding h32 gives the
// correctly rounded BF16 value; everything else (about 1 element in 500, plus the
// large gates, infinities and tiny values) takes the binary64 path above.
__device__ __forceinline__ uint32_t swiglu_bf16(float g, float u) {
  if (fabsf(g) <= 80.0f) {
    const float h = g / (1.0f + expf(-g)) * u;
    const uint32_t b = __float_as_uint(h);
    const uint32_t mag = b & 0x7FFFFFFFu;
    const int32_t lowd = (int32_t)(b & 0xFFFFu) - 0x8000;
    if (mag >= 0x0D800000u && mag < 0x7F000000u && (lowd > 64 || lowd < -64))   // 2^-100 <= |h32| < 2^127
      return f32_to_bf16_rne(h);
  }
  return swiglu_bf16_f64(g, u);
}

template <int CH>
__global__ void __launch_bounds__(256)
swiglu_nvfp4_kernel(const float* __restrict__ gu, int64_t rows, int64_t inter, uint16_t* __restrict__ h_out,
                    uint8_t* __restrict__ q, uint8_t* __restrict__ s, float* __restrict__ t_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* g = gu + row * 2 * inter;
  const float* u = g + inter;
  uint4 hb[CH];            // BF16 h, 8 per lane per chunk
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t e = (int64_t)i * 512 + 8 * lane;
    uint32_t p[4] = {0, 0, 0, 0};
    if (e < inter) {
      const float4 g0 = load_stream16f(g + e), g1 = load_stream16f(g + e + 4);
      const float4 u0 = load_stream16f(u + e), u1 = load_stream16f(u + e + 4);
      p[0] = swiglu_bf16(g0.x, u0.x) | (swiglu_bf16(g0.y, u0.y) << 16);
      p[1] = swiglu_bf16(g0.z, u0.z) | (swiglu_bf16(g0.w, u0.w) << 16);
      p[2] = swiglu_bf16(g1.x, u1.x) | (swiglu_bf16(g1.y, u1.y) << 16);
      p[3] = swiglu_bf16(g1.z, u1.z) | (swiglu_bf16(g1.w, u1.w) << 16);
      if (h_out) {                                               // outputs leave with non-temporal stores
        const u32x4_nt h4 = {p[0], p[1], p[2], p[3]};
        __builtin_nontemporal_store(h4, reinterpret_cast<u32x4_nt*>(h_out + row * inter + e));
      }
    }
    hb[i] = make_uint4(p[0], p[1], p[2], p[3]);
    amax_bits = pk_max_u16(amax_bits, pk_max_u16(pk_max_u16(p[0] & 0x7FFF7FFFu, p[1] & 0x7FFF7FFFu),
                                                 pk_max_u16(p[2] & 0x7FFF7FFFu, p[3] & 0x7FFF7FFFu)));
  }
  uint32_t u32 = max_halves(amax_bits) << 16;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = shfl_xor_u32(u32, off);
    u32 = u32 > o ? u32 : o;
  }
  const float A = __uint_as_float(u32);
  float s_enc = 2688.0f / A;
  if (A == 0.0f) s_enc = 1.0f;
  if (__builtin_isinf(s_enc)) s_enc = kFltMax;
  if (lane == 0) t_out[row] = 1.0f / s_enc;
  const bool odd = lane & 1;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t e = (int64_t)i * 512 + 8 * lane;
    const uint32_t w[4] = {hb[i].x, hb[i].y, hb[i].z, hb[i].w};
    float f[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) { f[2 * k] = bf16_lo(w[k]); f[2 * k + 1] = bf16_hi(w[k]); }
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
    a = fmaxf(a, __uint_as_float(dpp_xor1(__float_as_uint(a))));
    float d = fminf((a / 6.0f) * s_enc, kE4M3Max);
    const uint32_t code = cvt_fp8x2_f32(0u, d, 0.0f, 1.0f, false) & 0xFFu;
    const float S = e4m3_to_f32(code);
    const float r = (S == 0.0f) ? 0.0f : fminf(s_enc / S, kFltMax);
    uint32_t o = 0;
    o = cvt_fp4x2_f32<0>(o, f[0] * r, f[1] * r);
    o = cvt_fp4x2_f32<1>(o, f[2] * r, f[3] * r);
    o = cvt_fp4x2_f32<2>(o, f[4] * r, f[5] * r);
    o = cvt_fp4x2_f32<3>(o, f[6] * r, f[7] * r);
    if (e < inter) {
      __builtin_nontemporal_store(o, reinterpret_cast<uint32_t*>(q + row * (inter / 2) + e / 2));
      if (!odd) s[row * (inter / 16) + e / 16] = (uint8_t)code;
    }
  }
}

hipError_t launch_swiglu_nvfp4(const float* gu, int64_t rows, int64_t inter, void* h, void* q, void* s, float* t,
                               hipStream_t st) {
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const int64_t ch = (inter + 511) / 512;
  uint16_t* hp = (uint16_t*)h;
  if (ch <= 2) hipLaunchKernelGGL(swiglu_nvfp4_kernel<2>, grid, block, 0, st, gu, rows, inter, hp, (uint8_t*)q, (uint8_t*)s, t);
  else if (ch <= 4) hipLaunchKernelGGL(swiglu_nvfp4_kernel<4>, grid, block, 0, st, gu, rows, inter, hp, (uint8_t*)q, (uint8_t*)s, t);
  else if (ch <= 8) hipLaunchKernelGGL(swiglu_nvfp4_kernel<8>, grid, block, 0, st, gu, rows, inter, hp, (uint8_t*)q, (uint8_t*)s, t);
  else if (ch <= 16) hipLaunchKernelGGL(swiglu_nvfp4_kernel<16>, grid, block, 0, st, gu, rows, inter, hp, (uint8_t*)q, (uint8_t*)s, t);
  else hipLaunchKernelGGL(swiglu_nvfp4_kernel<32>, grid, block, 0, st, gu, rows, inter, hp, (uint8_t*)q, (uint8_t*)s, t);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: one workgroup per token, float4 per thread, j ascending.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ o, int64_t total_slots, int64_t topk, int64_t hidden,
               const int64_t* __restrict__ slot_of, const float* __restrict__ w, float* __restrict__ y) {
  const int64_t tok = blockIdx.x;
  for (int64_t c = 4 * (int64_t)threadIdx.x; c < hidden; c += 4 * (int64_t)blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t j = 0; j < topk; ++j) {
      const float wj = w[tok * topk + j];
      const int64_t slot = slot_of[tok * topk + j];
      if (slot < 0 || slot >= total_slots) continue;
      const float4 v = load_stream16f(o + slot * hidden + c);
      acc.x += wj * v.x; acc.y += wj * v.y; acc.z += wj * v.z; acc.w += wj * v.w;
    }
    const f32x4_nt a4 = {acc.x, acc.y, acc.z, acc.w};           // output not read here: keep it out of L2
    __builtin_nontemporal_store(a4, reinterpret_cast<f32x4_nt*>(y + tok * hidden + c));
  }
}

hipError_t launch_combine(const float* o, int64_t total_slots, int64_t tokens, int64_t topk, int64_t hidden,
                          const int64_t* slot_of, const float* w, float* y, hipStream_t st) {
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)tokens), dim3(256), 0, st, o, total_slots, topk, hidden, slot_of,
                     w, y);
  return hipGetLastError();
}

}  // namespace mxq
