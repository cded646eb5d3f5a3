// Grouped expert GEMMs on gfx950 bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// The expert computation of the MindSpeed Chunk MoE article (core principle /
// timing-diagram sections) is read as a SwiGLU FFN per expert; each expert
// multiplies its contiguous block of permuted rows:
//   gate_up: act[r][i] = silu(x_r . Wg[e][i]) * (x_r . Wu[e][i])   (K = H)
//   down   : y[r][n]   = act_r . Wd[e][n]                          (K = I)
// Both operands are K-contiguous ([rows][K] activations, [cols][K] weights).
//
// Tiling: a 256-thread workgroup computes a 128 x 128 output tile; its four
// waves each own 64 x 64 as 4 x 4 MFMA 16x16 blocks with fp32 accumulators.
// K advances 64 at a time through a double-buffered LDS stage (rows padded by
// 16 bytes); global loads of the next stage are in flight while the matrix
// cores work on the current one.  For gate_up the 128 tile columns hold 64
// gate columns and the 64 matching up columns, arranged so that every lane
// holds the gate and up accumulators of the same (row, i) and the SwiGLU is
// applied in registers: no [rows][2I] intermediate is written.
//
// Grouping: the m-tiles of all experts are numbered expert by expert; each
// workgroup finds its expert from the device-resident offsets (find_m_tile), so
// the host never reads the group sizes.  The grid is bounded from the chunk's
// assignment count; surplus workgroups exit.  Rows past an expert's block are
// loaded from a clamped row and never stored.  The arithmetic of a row does not
// depend on its tile position, so results are identical for any chunking.
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row, in elements
constexpr int kThreads = 256;
constexpr int kVecA = BM * BK / 8 / kThreads;  // 16-byte vectors per thread per stage
constexpr int kVecB = BN * BK / 8 / kThreads;

struct GemmArgs {
  const uint16_t* A;          // [rows][K] bf16
  const uint16_t* B;          // [E][b_rows][K] bf16
  uint16_t* C;                // [rows][ncols] bf16
  const int32_t* off;         // E + 1 offsets of this chunk
  int E, K, I, ncols, n_tiles, b_rows;
  int64_t b_expert_stride;    // elements per expert in B
};

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <bool kGateUp>
__global__ void __launch_bounds__(kThreads) grouped_gemm_bf16(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][(BM + BN) * LDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nt = blockIdx.x % a.n_tiles;
  const int mt = blockIdx.x / a.n_tiles;
  int e, m0, mrows;
  if (!find_m_tile(a.off, a.E, BM, mt, &e, &m0, &mrows)) return;

  const uint16_t* a_src[kVecA];
  const uint16_t* b_src[kVecB];
  int a_dst[kVecA], b_dst[kVecB];
  const uint16_t* Be = a.B + (int64_t)e * a.b_expert_stride;
#pragma unroll
  for (int i = 0; i < kVecA; ++i) {
    const int v = tid + i * kThreads, row = v >> 3, kc = (v & 7) * 8;
    const int r = row < mrows ? row : mrows - 1;
    a_src[i] = a.A + (int64_t)(m0 + r) * a.K + kc;
    a_dst[i] = row * LDK + kc;
  }
#pragma unroll
  for (int i = 0; i < kVecB; ++i) {
    const int v = tid + i * kThreads, row = v >> 3, kc = (v & 7) * 8;
    int brow;
    if constexpr (kGateUp) {
      // tile column `row`: wave half wn = row/64, gate (q=0) or up (q=1), column c
      const int wn = row >> 6, q = (row >> 5) & 1, c = row & 31;
      brow = q * a.I + nt * 64 + wn * 32 + c;
    } else {
      brow = nt * BN + row;
      if (brow > a.ncols - 1) brow = a.ncols - 1;
    }
    b_src[i] = Be + (int64_t)brow * a.K + kc;
    b_dst[i] = (BM + row) * LDK + kc;
  }

  bf16x8 ra[kVecA], rb[kVecB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kVecA; ++i) ra[i] = *(const bf16x8*)(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < kVecB; ++i) rb[i] = *(const bf16x8*)(b_src[i] + k0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kVecA; ++i) *(bf16x8*)&lds[buf][a_dst[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < kVecB; ++i) *(bf16x8*)&lds[buf][b_dst[i]] = rb[i];
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm = wave >> 1, wn = wave & 1;
  const int frag_k = (lane >> 4) * 8;
  const int KT = a.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *(const bf16x8*)&lds[buf][(wm * 64 + i * 16 + (lane & 15)) * LDK + kk + frag_k];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] =
            *(const bf16x8*)&lds[buf][(BM + wn * 64 + j * 16 + (lane & 15)) * LDK + kk + frag_k];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  MFMA 16x16 output: lane holds column (lane & 15) of rows
  // 4 * (lane >> 4) + 0..3 of each 16 x 16 block.
  const int rbase = wm * 64 + (lane >> 4) * 4;
  if constexpr (kGateUp) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = nt * 64 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          if (row < mrows) {
            const float g = acc[i][j][r], u = acc[i][j + 2][r];
            const float act = g / (1.0f + expf(-g)) * u;
            a.C[(int64_t)(m0 + row) * a.ncols + col] = to_bf16_bits(act);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = nt * BN + wn * 64 + j * 16 + (lane & 15);
        if (col >= a.ncols) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          if (row < mrows) a.C[(int64_t)(m0 + row) * a.ncols + col] = to_bf16_bits(acc[i][j][r]);
        }
      }
  }
}

hipError_t launch(bool gate_up, const Shape& s, int64_t rows_bound, const void* A,
                  const int32_t* off, const void* B, void* C, hipStream_t st) {
  if (rows_bound <= 0) return hipSuccess;
  GemmArgs a{};
  a.A = (const uint16_t*)A;
  a.B = (const uint16_t*)B;
  a.C = (uint16_t*)C;
  a.off = off;
  a.E = s.E;
  a.I = s.I;
  if (gate_up) {
    a.K = s.H;
    a.ncols = s.I;
    a.n_tiles = s.I / 64;
    a.b_rows = 2 * s.I;
  } else {
    a.K = s.I;
    a.ncols = s.H;
    a.n_tiles = (s.H + BN - 1) / BN;
    a.b_rows = s.H;
  }
  a.b_expert_stride = (int64_t)a.b_rows * a.K;
  const int64_t grid = m_tiles_bound(rows_bound, s.E, BM) * a.n_tiles;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (gate_up)
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_bf16(const Shape& s, int64_t rows_bound, const void* x_perm,
                               const int32_t* offsets_c, const void* w_gate_up, void* act,
                               hipStream_t st) {
  return launch(true, s, rows_bound, x_perm, offsets_c, w_gate_up, act, st);
}

hipError_t launch_down_bf16(const Shape& s, int64_t rows_bound, const void* act,
                            const int32_t* offsets_c, const void* w_down, void* y,
                            hipStream_t st) {
  return launch(false, s, rows_bound, act, offsets_c, w_down, y, st);
}

}  // namespace moe
