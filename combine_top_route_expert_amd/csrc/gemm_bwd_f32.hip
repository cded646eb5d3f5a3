// Backward grouped products in fp32 (vector FMA), for dtype MOE_F32: the same
// products as gemm_bwd_bf16.hip (gradient of the SwiGLU expert computation of
// the MindSpeed Chunk MoE article, forward recomputed per chunk pair), with one
// fused multiply-add per product in ascending K inside each thread and no
// reduced precision.  64 x 64 tiles, 16-deep LDS stages, 4 x 4 outputs per
// thread.  The small fp32 workloads are latency bound; these kernels aim at
// being plainly correct, not fast.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = 64, BN = 64, BKF = 16;
constexpr int kThreads = 256;

struct SideF {
  const float* p[2];
  int split;
  int64_t ld;
};

__device__ __forceinline__ const float* side_row(const SideF& s, const TileRows& tr, int v) {
  if (s.split) {
    int part;
    const int r = tr.split_row(v, &part);
    return (part ? s.p[1] : s.p[0]) + (int64_t)r * s.ld;
  }
  return s.p[0] + (int64_t)tr.joint_row(v) * s.ld;
}

struct DgradArgsF {
  SideF a;                 // [rows][K]
  const float* B;          // [E][K][N]
  float* C[2];
  int c_split;
  float* gu;               // swiglu epilogue: joint [rows][2I]
  const int32_t* off0;
  const int32_t* off1;
  int E, K, N, I, n_tiles;
};

template <bool kSwiglu>
__global__ void __launch_bounds__(kThreads) dgrad_gemm_f32(DgradArgsF a) {
  __shared__ float As[BM][BKF + 1];
  __shared__ float Bs[BKF][BN];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  MTileMap tm;
  tm.build(a.off0, a.off1, a.E, BM, 1);
  int mt, nt;
  if (!xcd_tile(tm, a.n_tiles, &mt, &nt)) return;
  const TileRows tr = tm.locate(a.off0, a.off1, BM, mt);
  const float* Be = a.B + (int64_t)tr.e * a.K * a.N;

  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[r][q] = 0.0f;

  for (int k0 = 0; k0 < a.K; k0 += BKF) {
    for (int i = tid; i < BM * BKF; i += kThreads) {
      const int r = i / BKF, kk = i % BKF;
      const int rr = r < tr.rows ? r : tr.rows - 1;
      As[r][kk] = (k0 + kk < a.K) ? side_row(a.a, tr, tr.v0 + rr)[k0 + kk] : 0.0f;
    }
    for (int i = tid; i < BKF * BN; i += kThreads) {
      const int kk = i / BN, n = i % BN;
      const int col = nt * BN + n;
      Bs[kk][n] = (k0 + kk < a.K && col < a.N) ? Be[(int64_t)(k0 + kk) * a.N + col] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[r][q] = __builtin_fmaf(As[ty * 4 + r][kk], Bs[kk][tx * 4 + q], acc[r][q]);
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = ty * 4 + r;
    if (row >= tr.rows) continue;
    const int v = tr.v0 + row;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = nt * BN + tx * 4 + q;
      if (col >= a.N) continue;
      if constexpr (kSwiglu) {
        float* gr = a.gu + (int64_t)tr.joint_row(v) * (2 * a.I);
        const float ga = acc[r][q], g = gr[col], u = gr[a.I + col];
        const float s = 1.0f / (1.0f + expf(-g));
        gr[col] = ga * u * (s + g * s * (1.0f - s));
        gr[a.I + col] = ga * (g * s);
      } else {
        float* cr;
        if (a.c_split) {
          int part;
          const int rr = tr.split_row(v, &part);
          cr = a.C[part] + (int64_t)rr * a.N;
        } else {
          cr = a.C[0] + (int64_t)tr.joint_row(v) * a.N;
        }
        cr[col] = acc[r][q];
      }
    }
  }
}

struct WgradArgsF {
  SideF a, b;
  float* C;
  const int32_t* off0;
  const int32_t* off1;
  int E, M, N, m_tiles, n_tiles, accumulate;
  const int32_t* order;  // nullable: experts in dealing order
};

__global__ void __launch_bounds__(kThreads) wgrad_gemm_f32(WgradArgsF a) {
  __shared__ float As[BKF][BM];
  __shared__ float Bs[BKF][BN];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  int emt, nt;
  if (!xcd_tile_rr(a.E * a.m_tiles, a.n_tiles, &emt, &nt)) return;
  const int rank = emt / a.m_tiles, mt = emt - rank * a.m_tiles;
  const int e = a.order ? a.order[rank] : rank;
  TileRows tr;
  tr.e = e;
  tr.v0 = 0;
  tr.lo0 = a.off0[e];
  tr.n0 = a.off0[e + 1] - tr.lo0;
  tr.lo1 = a.off1 ? a.off1[e] : 0;
  const int rows = tr.n0 + (a.off1 ? a.off1[e + 1] - tr.lo1 : 0);
  tr.rows = rows;
  if (rows == 0 && a.accumulate) return;
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[r][q] = 0.0f;
  for (int k0 = 0; k0 < rows; k0 += BKF) {
    for (int i = tid; i < BKF * BM; i += kThreads) {
      const int kk = i / BM, m = i % BM;
      const int col = mt * BM + m;
      As[kk][m] = (k0 + kk < rows && col < a.M) ? side_row(a.a, tr, k0 + kk)[col] : 0.0f;
    }
    for (int i = tid; i < BKF * BN; i += kThreads) {
      const int kk = i / BN, n = i % BN;
      const int col = nt * BN + n;
      Bs[kk][n] = (k0 + kk < rows && col < a.N) ? side_row(a.b, tr, k0 + kk)[col] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[r][q] = __builtin_fmaf(As[kk][ty * 4 + r], Bs[kk][tx * 4 + q], acc[r][q]);
    __syncthreads();
  }
  float* Ce = a.C + (int64_t)e * a.M * a.N;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = mt * BM + ty * 4 + r;
    if (m >= a.M) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = nt * BN + tx * 4 + q;
      if (n >= a.N) continue;
      float* c = Ce + (int64_t)m * a.N + n;
      *c = a.accumulate ? *c + acc[r][q] : acc[r][q];
    }
  }
}

}  // namespace

hipError_t launch_dgrad_f32(const Shape& s, const DgradIO& io, hipStream_t st) {
  if (io.rows_bound <= 0) return hipSuccess;
  DgradArgsF a{};
  a.a.p[0] = (const float*)io.a[0];
  a.a.p[1] = (const float*)(io.a_split ? io.a[1] : io.a[0]);
  a.a.split = io.a_split && io.off[1];
  a.a.ld = io.K;
  a.B = (const float*)io.B;
  a.C[0] = (float*)io.c[0];
  a.C[1] = (float*)(io.c_split ? io.c[1] : io.c[0]);
  a.c_split = io.c_split && io.off[1];
  a.gu = (float*)io.gu;
  a.off0 = io.off[0];
  a.off1 = io.off[1];
  a.E = s.E;
  a.K = io.K;
  a.N = io.N;
  a.I = s.I;
  a.n_tiles = (io.N + BN - 1) / BN;
  const int64_t grid = xcd_grid(m_tiles_bound(io.rows_bound, s.E, BM), a.n_tiles);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (io.gu)
    hipLaunchKernelGGL(dgrad_gemm_f32<true>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(dgrad_gemm_f32<false>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_wgrad_f32(const Shape& s, const WgradIO& io, hipStream_t st) {
  WgradArgsF a{};
  a.a.p[0] = (const float*)io.a[0];
  a.a.p[1] = (const float*)(io.a_split ? io.a[1] : io.a[0]);
  a.a.split = io.a_split && io.off[1];
  a.a.ld = io.M;
  a.b.p[0] = (const float*)io.b[0];
  a.b.p[1] = (const float*)(io.b_split ? io.b[1] : io.b[0]);
  a.b.split = io.b_split && io.off[1];
  a.b.ld = io.N;
  a.C = io.C;
  a.off0 = io.off[0];
  a.off1 = io.off[1];
  a.E = s.E;
  a.M = io.M;
  a.N = io.N;
  a.accumulate = io.accumulate;
  a.order = io.order;
  a.m_tiles = (io.M + BM - 1) / BM;
  a.n_tiles = (io.N + BN - 1) / BN;
  const int64_t grid = xcd_grid_rr((int64_t)s.E * a.m_tiles, a.n_tiles);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(wgrad_gemm_f32, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
