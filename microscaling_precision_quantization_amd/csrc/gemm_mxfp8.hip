// MXFP8 x MXFP8 block-scaled GEMM on the gfx950 scaled FP8 MFMA (the native
// matrix-core path):  C[m, n] = sum_k A[m, k] B[n, k],  A_hat = E4M3 * 2^(sA - 127)
// per 32 along K.
//
// Accumulation semantics (measured on MI355X): the matrix core sums the
// products of each group of 8 consecutive K of a lane in a fixed-point window
// about 13 bits below the group's largest product, dropping lower bits, and
// accumulates the group sums at FP32 precision. Products within 2^-5 of their
// group maximum are therefore exact; on data whose 8-element groups span more
// than that (outliers, heavy tails) the result differs from the exact sum by up
// to ~2^-13 of the largest product per group. gemm_block_scaled(MXFP8) forms
// exact BF16 operands and accumulates at FP32 precision instead.
//
// The scaling blocks lie along the reduction dimension ("Miles Blackwell RL",
// remio.ai, section "Un Cuantizador Compartido Es el Mecanismo Real"), which is
// exactly what the hardware consumes: v_mfma_scale_f32_32x32x64_f8f6f4 takes
// one E8M0 byte per (row, 32-K block) of each operand, so the E8M0 scales are
// applied inside the matrix core and the FP32 accumulators hold the exact
// scaled sums.
//
// FP8 operand layout of the 32x32x64 scaled MFMA (measured on MI355X): lane l
// supplies row l % 32; with h = l / 32, bytes 0..15 are elements [16h, 16h+16)
// of the first 32-K block and bytes 16..31 the same elements of the second
// block; the scale of block b for that row comes from lane (l % 32) + 32 b.
// A and B use the same layout. Accumulator r of lane l is
// C[(r / 4) * 8 + h * 4 + r % 4][l % 32].
//
// Tiling: workgroup 256 x 256, four waves of 128 x 128 (4 x 4 MFMA tiles),
// K tile 128 bytes, double-buffered LDS (2 x 64 KiB) written from registers with
// a 16-byte XOR swizzle (chunk ^ row % 8) so each 8-row group of a fragment read
// touches all banks. One workgroup per CU (LDS- and register-bound).
#include "common.h"

namespace mxq {

namespace g8 {
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int TILE_BYTES = BM * BK;                // one operand tile: 32 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;        // A + B
}  // namespace g8

struct GemmProblem {
  const uint8_t* A;        // element (row, k) at A[row_off(row) + k]
  const uint8_t* sA;       // scale of (row, k/32) at sA[row_off(row)/32 + k/32] (row_off multiple of lda)
  const int32_t* a_idx;    // optional gather: A row of tile row r = a_idx[a_base + r]
  int64_t a_rows;          // rows of A (gather indices outside [0, a_rows) read as zero rows)
  int64_t a_base;          // first row (slot) of this problem
  int64_t m_valid;         // rows of this problem
  int64_t lda;             // bytes per A row (= K total)
  const uint8_t* B;
  const uint8_t* sB;
  int64_t n_valid;
  int64_t ldb;
  int64_t k_begin, k_end;  // reduction range (elements)
  float* C;                // row 0 of this problem's output
  int64_t ldc;
};

// A row feeding tile row r (r < m_valid), or -1 when a gather index is out of range.
__device__ __forceinline__ int64_t a_source_row(const GemmProblem& p, int64_t r) {
  if (!p.a_idx) return p.a_base + r;
  const int64_t ar = p.a_idx[p.a_base + r];
  return (ar >= 0 && ar < p.a_rows) ? ar : -1;
}

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * g8::BK + ((chunk ^ (row & 7)) << 4); }

// Loads 8 chunks of 16 bytes of a 256 x 128 operand tile into registers.
// Thread t handles rows i * 32 + t / 8 (i = 0..7), chunk t % 8.
__device__ __forceinline__ void load_tile_regs(uint4* r, const int64_t* row_off, const bool* row_ok,
                                               const uint8_t* base, int64_t k0, int64_t k_end, int chunk) {
  const int64_t k = k0 + chunk * 16;
  const bool kok = k < k_end;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    r[i] = (row_ok[i] && kok) ? *reinterpret_cast<const uint4*>(base + row_off[i] + k) : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void store_tile_lds(uint8_t* lds, const uint4* r, int tid) {
  const int chunk = tid & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = i * 32 + (tid >> 3);
    *reinterpret_cast<uint4*>(lds + lds_off(row, chunk)) = r[i];
  }
}

// Scale dword for (row, blocks k0/32 .. k0/32 + 3); blocks past k_end read as 127.
__device__ __forceinline__ uint32_t load_scale4(const uint8_t* srow, int64_t k0, int64_t k_end, bool row_ok) {
  if (!row_ok) return 0x7F7F7F7Fu;
  const int64_t b0 = k0 / 32;
  if (k0 + 128 <= k_end && ((reinterpret_cast<uintptr_t>(srow + b0) & 3) == 0))
    return *reinterpret_cast<const uint32_t*>(srow + b0);
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t b = (k0 + 32 * j < k_end) ? srow[b0 + j] : 0x7Fu;
    v |= b << (8 * j);
  }
  return v;
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* lds, int row, int c0, int c1) {
  const uint4 a = *reinterpret_cast<const uint4*>(lds + lds_off(row, c0));
  const uint4 b = *reinterpret_cast<const uint4*>(lds + lds_off(row, c1));
  v8i f;
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  return f;
}

// Wait states after the last scaled FP8 MFMA before its accumulators are read
// by ordinary instructions: the 16-pass 32x32x64 FP8 form needs more than the
// compiler inserts on its own (observed on MI355X), so 24 are added here.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ void gemm_mxfp8_tile(const GemmProblem& p, int64_t m0, int64_t n0, uint8_t* lds) {
  using namespace g8;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, lr = lane & 31;
  const int chunk = tid & 7;

  // rows this thread loads
  int64_t a_off[8], b_off[8];
  bool a_ok[8], b_ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = m0 + i * 32 + (tid >> 3);
    const int64_t ar = r < p.m_valid ? a_source_row(p, r) : -1;
    a_ok[i] = ar >= 0;
    a_off[i] = (a_ok[i] ? ar : 0) * p.lda;
    const int64_t n = n0 + i * 32 + (tid >> 3);
    b_ok[i] = n < p.n_valid;
    b_off[i] = (b_ok[i] ? n : 0) * p.ldb;
  }
  // rows whose scales this lane feeds to the MFMA (4 row tiles of A, 4 column tiles of B)
  const uint8_t* sa_row[4];
  const uint8_t* sb_row[4];
  bool sa_ok[4], sb_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = m0 + wm * 128 + i * 32 + lr;
    const int64_t ar = r < p.m_valid ? a_source_row(p, r) : -1;
    sa_ok[i] = ar >= 0;
    sa_row[i] = p.sA + (sa_ok[i] ? ar : 0) * (p.lda / 32);
    const int64_t n = n0 + wn * 128 + i * 32 + lr;
    sb_ok[i] = n < p.n_valid;
    sb_row[i] = p.sB + (sb_ok[i] ? n : 0) * (p.ldb / 32);
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
  uint4 ra[8], rb[8];
  uint32_t sa[4], sb[4], sa_n[4], sb_n[4];
  if (nk > 0) {
    load_tile_regs(ra, a_off, a_ok, p.A, kb, ke, chunk);
    load_tile_regs(rb, b_off, b_ok, p.B, kb, ke, chunk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = load_scale4(sa_row[i], kb, ke, sa_ok[i]) >> (8 * h);
      sb[i] = load_scale4(sb_row[i], kb, ke, sb_ok[i]) >> (8 * h);
    }
    store_tile_lds(lds, ra, tid);
    store_tile_lds(lds + TILE_BYTES, rb, tid);
  }
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * STAGE_BYTES;
    uint8_t* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
    const bool more = kt + 1 < nk;
    const int64_t k1 = kb + (kt + 1) * BK;
    if (more) {
      load_tile_regs(ra, a_off, a_ok, p.A, k1, ke, chunk);
      load_tile_regs(rb, b_off, b_ok, p.B, k1, ke, chunk);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa_n[i] = load_scale4(sa_row[i], k1, ke, sa_ok[i]) >> (8 * h);
        sb_n[i] = load_scale4(sb_row[i], k1, ke, sb_ok[i]) >> (8 * h);
      }
    }
    const uint8_t* la = cur;
    const uint8_t* lb = cur + TILE_BYTES;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      v8i fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = lds_frag(la, wm * 128 + i * 32 + lr, 4 * t + h, 4 * t + 2 + h);
        fb[i] = lds_frag(lb, wn * 128 + i * 32 + lr, 4 * t + h, 4 * t + 2 + h);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (t == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 2, sa[i], 2, sb[j]);
        }
    }
    if (more) {
      store_tile_lds(nxt, ra, tid);
      store_tile_lds(nxt + TILE_BYTES, rb, tid);
#pragma unroll
      for (int i = 0; i < 4; ++i) { sa[i] = sa_n[i]; sb[i] = sb_n[i]; }
    }
    __syncthreads();
  }
  mfma_drain();

  // epilogue: FP32 stores, 32 consecutive columns per half-wave
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + j * 32 + lr;
      if (col >= p.n_valid) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
        if (row < p.m_valid) p.C[row * p.ldc + col] = acc[i][j][r];
      }
    }
}

// XCD-aware raster: dispatch order b goes round-robin over the 8 XCDs; give each
// XCD a contiguous run of logical tiles, walked in bands of 4 tile rows so the
// workgroups resident on one XCD share A and B tiles in its L2.
__device__ __forceinline__ bool map_tile(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
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

__global__ void __launch_bounds__(256, 1)
gemm_mxfp8_dense_kernel(GemmProblem p, int64_t tiles_m, int64_t tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * g8::STAGE_BYTES];
  int64_t tm, tn;
  if (!map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  gemm_mxfp8_tile(p, tm * g8::BM, tn * g8::BN, lds);
}

hipError_t launch_gemm_mxfp8_matrix_core(int64_t M, int64_t N, int64_t K, const void* A, const void* sA, const void* B,
                             const void* sB, float* C, int64_t ldc, hipStream_t st) {
  GemmProblem p;
  p.A = (const uint8_t*)A; p.sA = (const uint8_t*)sA; p.a_idx = nullptr; p.a_rows = M; p.a_base = 0; p.m_valid = M;
  p.lda = K;
  p.B = (const uint8_t*)B; p.sB = (const uint8_t*)sB; p.n_valid = N; p.ldb = K;
  p.k_begin = 0; p.k_end = K; p.C = C; p.ldc = ldc;
  const int64_t tm = (M + g8::BM - 1) / g8::BM, tn = (N + g8::BN - 1) / g8::BN;
  const int64_t blocks = (tm * tn + 7) / 8 * 8;
  hipLaunchKernelGGL(gemm_mxfp8_dense_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, tm, tn);
  return hipGetLastError();
}

}  // namespace mxq
