// Grouped expert GEMMs in fp32 (vector FMA), for dtype MOE_F32.
//
// Same contraction and grouping (one chunk, or the two chunks of a pair) as the
// bf16 path (SwiGLU read of the expert computation in the MindSpeed Chunk MoE
// article), in IEEE fp32 with one fused
// multiply-add per product and ascending-k order inside each thread: no
// reduced-precision matrix instruction is involved.
//
// Tiling: 256 threads compute a 64 x 64 tile through a 16-deep LDS stage; each
// thread owns 4 rows x 4 columns.  For gate_up the 64 tile columns are 32 gate
// and the 32 matching up columns, and a thread's four columns are the gate and
// up columns of the same two i, so SwiGLU happens in registers.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = 64, BN = 64, BK = 16;
constexpr int kThreads = 256;

struct GemmArgs {
  const float* A[2];      // A[1]: chunk-1 rows when a_split
  const float* B;
  float* C[2];            // C[1]: chunk-1 rows when c_split
  const int32_t* off0;
  const int32_t* off1;    // second chunk of a pair, or null
  int a_split, c_split;
  int E, K, I, ncols, n_tiles;
  int64_t b_expert_stride;
  float* gu;              // gate_up, optional: g and u of each row, joint [rows][2I]
  const int32_t* gather[2];  // optional: A rows gathered from hidden_states (src_row slices)
  int gather_k;
};

// Address of virtual row v of the tile's expert on one side of the product.
__device__ __forceinline__ const float* row_ptr(const float* const (&base)[2], int split,
                                                const TileRows& tr, int v, int64_t ld) {
  if (split) {
    int part;
    const int r = tr.split_row(v, &part);
    return (part ? base[1] : base[0]) + (int64_t)r * ld;
  }
  return base[0] + (int64_t)tr.joint_row(v) * ld;
}

template <bool kGateUp>
__device__ __forceinline__ int tile_col(int tx, int q) {
  // gate_up: q=0,1 -> gate columns 2tx, 2tx+1; q=2,3 -> the matching up columns
  if constexpr (kGateUp) return q < 2 ? 2 * tx + q : 32 + 2 * tx + (q - 2);
  return 4 * tx + q;
}

template <bool kGateUp>
__global__ void __launch_bounds__(kThreads) grouped_gemm_f32(GemmArgs a) {
  __shared__ float As[BM][BK + 1];
  __shared__ float Bs[BN][BK + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  MTileMap tm;
  tm.build(a.off0, a.off1, a.E, BM, 1);
  int mt, nt;
  if (!xcd_tile(tm, a.n_tiles, &mt, &nt)) return;
  const TileRows tr = tm.locate(a.off0, a.off1, BM, mt);
  const int e = tr.e, mrows = tr.rows;

  // one float4 of A and one of B per thread per stage
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int arow = lrow < mrows ? lrow : mrows - 1;
  const float* a_src;
  if (a.gather[0]) {  // permute fused into the row addressing: chunk row -> token
    int part;
    const int cr = tr.split_row(tr.v0 + arow, &part);
    const int32_t* src = part ? a.gather[1] : a.gather[0];
    a_src = a.A[0] + (int64_t)(src[cr] / a.gather_k) * a.K + lk;
  } else {
    a_src = row_ptr(a.A, a.a_split, tr, tr.v0 + arow, a.K) + lk;
  }
  int brow;
  if constexpr (kGateUp) {
    const int i = nt * 32 + (lrow & 31);
    brow = (i < a.I ? i : a.I - 1) + (lrow >= 32 ? a.I : 0);
  } else {
    brow = nt * BN + lrow;
    if (brow > a.ncols - 1) brow = a.ncols - 1;
  }
  const float* b_src = a.B + (int64_t)e * a.b_expert_stride + (int64_t)brow * a.K + lk;

  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[r][q] = 0.0f;

  for (int k0 = 0; k0 < a.K; k0 += BK) {
    float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = va;
    if (k0 + lk < a.K) {
      va = *(const float4*)(a_src + k0);
      vb = *(const float4*)(b_src + k0);
    }
    As[lrow][lk] = va.x;
    As[lrow][lk + 1] = va.y;
    As[lrow][lk + 2] = va.z;
    As[lrow][lk + 3] = va.w;
    Bs[lrow][lk] = vb.x;
    Bs[lrow][lk + 1] = vb.y;
    Bs[lrow][lk + 2] = vb.z;
    Bs[lrow][lk + 3] = vb.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = As[ty * 4 + r][kk];
#pragma unroll
      for (int q = 0; q < 4; ++q) bv[q] = Bs[tile_col<kGateUp>(tx, q)][kk];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[r][q] = __builtin_fmaf(av[r], bv[q], acc[r][q]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = ty * 4 + r;
    if (row >= mrows) continue;
    const float* const cbase[2] = {a.C[0], a.C[1]};
    float* crow = (float*)row_ptr(cbase, a.c_split, tr, tr.v0 + row, a.ncols);
    if constexpr (kGateUp) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int i = nt * 32 + 2 * tx + q;
        if (i < a.I) {
          const float g = acc[r][q], u = acc[r][q + 2];
          crow[i] = g / (1.0f + expf(-g)) * u;
          if (a.gu) {  // the backward's saved pre-activations
            float* gr = a.gu + (int64_t)tr.joint_row(tr.v0 + row) * (2 * a.I);
            gr[i] = g;
            gr[a.I + i] = u;
          }
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = nt * BN + 4 * tx + q;
        if (col < a.ncols) crow[col] = acc[r][q];
      }
    }
  }
}

hipError_t launch(bool gate_up, const Shape& s, const GroupedIO& io, const void* B,
                  hipStream_t st) {
  if (io.rows_bound <= 0) return hipSuccess;
  GemmArgs a{};
  a.A[0] = (const float*)io.a[0];
  a.A[1] = (const float*)(io.a_split ? io.a[1] : io.a[0]);
  a.C[0] = (float*)io.c[0];
  a.C[1] = (float*)(io.c_split ? io.c[1] : io.c[0]);
  a.off0 = io.off[0];
  a.off1 = io.off[1];
  a.a_split = io.a_split && io.off[1];
  a.c_split = io.c_split && io.off[1];
  a.gu = gate_up ? (float*)io.gu : nullptr;
  a.gather[0] = gate_up ? io.gather[0] : nullptr;
  a.gather[1] = gate_up && io.off[1] ? io.gather[1] : a.gather[0];
  a.gather_k = io.gather_k;
  a.B = (const float*)B;
  a.E = s.E;
  a.I = s.I;
  if (gate_up) {
    a.K = s.H;
    a.ncols = s.I;
    a.n_tiles = (s.I + 31) / 32;
    a.b_expert_stride = (int64_t)2 * s.I * s.H;
  } else {
    a.K = s.I;
    a.ncols = s.H;
    a.n_tiles = (s.H + BN - 1) / BN;
    a.b_expert_stride = (int64_t)s.H * s.I;
  }
  const int64_t grid = xcd_grid(m_tiles_bound(io.rows_bound, s.E, BM), a.n_tiles);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (gate_up)
    hipLaunchKernelGGL(grouped_gemm_f32<true>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(grouped_gemm_f32<false>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_f32(const Shape& s, const GroupedIO& io, const void* w_gate_up,
                              hipStream_t st) {
  return launch(true, s, io, w_gate_up, st);
}

hipError_t launch_down_f32(const Shape& s, const GroupedIO& io, const void* w_down,
                           hipStream_t st) {
  return launch(false, s, io, w_down, st);
}

}  // namespace moe
