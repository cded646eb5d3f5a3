// Permute (dispatch side) and unpermute + weighted combine.
//
// MindSpeed Chunk MoE article, core principle and timing-diagram section:
// tokens are permuted into an expert-contiguous buffer before the expert
// computation and unpermuted back to token order after it, the latter weighted
// by top_k_weights.  The combine reads the dispatch-side dst_row again rather
// than recomputing any routing (MindSpore news page, "# 02": combine reuses
// dispatch's lists).
//
// Both kernels are token-major: one wave owns one token row.
//  * permute reads the token's row once (16-byte vectors, several in flight per
//    lane) and writes it to each of its k destination rows; every destination
//    row is written by exactly one wave, so no atomics are needed.
//  * combine reads the token's k expert-output rows, accumulates
//    w[t,j] * y[row_j] in fp32 in ascending j, and rounds once on the store.
//    Every y row is read once and every out row written once, so the bf16
//    combine uses non-temporal loads and stores (streaming hints): 111.6 -> 98.0
//    us (5.4 TB/s, 67% of HBM peak) on the DeepSeek-V3-shaped layer, 119 -> 103
//    us on the packed 16k-token layer; the permute measured 3% slower with them.
// Both are HBM-bound: permute moves T*H*s + A*H*s bytes, combine A*H*s + T*H*s.
// The backward reuses combine_rows with unit weights (the permute's backward is
// a gather-sum of a token's k rows) and adds combine_backward below.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kVecPerLane = 4;  // 16-byte vectors each lane keeps in flight per pass

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(64 * kWavesPerBlock)
permute_rows(const u32x4* __restrict__ hidden, const int32_t* __restrict__ dst_row,
             u32x4* __restrict__ x_perm, int t0, int t1, int k, int nvec) {
  const int lane = threadIdx.x & 63;
  const int t = t0 + blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= t1) return;
  const u32x4* src = hidden + (size_t)t * nvec;
  // the token's k destination rows, one per lane, fetched in one round trip
  const int my_row = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  for (int v0 = 0; v0 < nvec; v0 += 64 * kVecPerLane) {
    u32x4 buf[kVecPerLane];
#pragma unroll
    for (int i = 0; i < kVecPerLane; ++i) {
      int v = v0 + i * 64 + lane;
      if (v < nvec) buf[i] = src[v];
    }
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_row, j);
      if (r < 0) continue;
      u32x4* dst = x_perm + (size_t)r * nvec;
#pragma unroll
      for (int i = 0; i < kVecPerLane; ++i) {
        int v = v0 + i * 64 + lane;
        if (v < nvec) dst[v] = buf[i];
      }
    }
  }
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4& q, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(q[i] << 16);
    f[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float* f) {
  u32x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __bf16 lo = (__bf16)f[2 * i], hi = (__bf16)f[2 * i + 1];
    q[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return q;
}

// One wave per token; each lane holds kVecPerLane 16-byte vectors of the row.
// Tokens [t0, t_mid) read their rows from y0, tokens [t_mid, t1) from y1 (a
// chunk pair whose expert outputs sit in two slots; row indices are
// chunk-local).
template <bool kBf16>
__global__ void __launch_bounds__(64 * kWavesPerBlock)
combine_rows(const u32x4* __restrict__ y0, const u32x4* __restrict__ y1, int t_mid,
             const int32_t* __restrict__ dst_row, const float* __restrict__ w,
             u32x4* __restrict__ out, int t0, int t1, int k, int nvec) {
  constexpr int kEl = kBf16 ? 8 : 4;  // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int t = t0 + blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= t1) return;
  const u32x4* __restrict__ y = t < t_mid ? y0 : y1;  // wave-uniform
  // the token's k rows and weights, one slot per lane, fetched in one round trip
  const int my_row = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  const float my_w = lane < k ? (w ? w[(size_t)t * k + lane] : 1.0f) : 0.0f;
  for (int v0 = 0; v0 < nvec; v0 += 64 * kVecPerLane) {
    float acc[kVecPerLane][kEl];
#pragma unroll
    for (int i = 0; i < kVecPerLane; ++i)
#pragma unroll
      for (int q = 0; q < kEl; ++q) acc[i][q] = 0.0f;
    // slots in groups of four: the group's row loads are all issued before
    // any is accumulated; accumulation stays in ascending slot order
    for (int j0 = 0; j0 < k; j0 += 4) {
      u32x4 rows[4][kVecPerLane];
      int rj[4];
      float wj[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        rj[g] = j0 + g < k ? __shfl(my_row, j0 + g) : -1;
        wj[g] = __shfl(my_w, (j0 + g) & 63);
        if (rj[g] < 0) continue;
        const u32x4* src = y + (size_t)rj[g] * nvec;
#pragma unroll
        for (int i = 0; i < kVecPerLane; ++i) {
          const int v = v0 + i * 64 + lane;
          if (v < nvec) rows[g][i] = __builtin_nontemporal_load(&src[v]);
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (rj[g] < 0) continue;
#pragma unroll
        for (int i = 0; i < kVecPerLane; ++i) {
          const int v = v0 + i * 64 + lane;
          if (v < nvec) {
            float f[kEl];
            if constexpr (kBf16) {
              unpack_bf16x8(rows[g][i], f);
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) f[q] = __uint_as_float(rows[g][i][q]);
            }
#pragma unroll
            for (int q = 0; q < kEl; ++q) acc[i][q] = __builtin_fmaf(wj[g], f[q], acc[i][q]);
          }
        }
      }
    }
    u32x4* dst = out + (size_t)t * nvec;
#pragma unroll
    for (int i = 0; i < kVecPerLane; ++i) {
      int v = v0 + i * 64 + lane;
      if (v < nvec) {
        if constexpr (kBf16) {
          __builtin_nontemporal_store(pack_bf16x8(acc[i]), &dst[v]);
        } else {
          u32x4 q;
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = __float_as_uint(acc[i][e]);
          dst[v] = q;
        }
      }
    }
  }
}

// Combine backward, one wave per token: for each kept slot j with row r,
// grad_w[t,j] = grad_out[t] . y[r] (fp32, each lane's partial in ascending
// vector order, then a fixed butterfly) and grad_y[r] = w[t,j] grad_out[t]
// (rounded once).  grad_y may alias y: row r is read, then overwritten, by the
// same wave.  Dropped slots get grad_w = 0.
template <bool kBf16>
__global__ void __launch_bounds__(64 * kWavesPerBlock)
combine_backward(const u32x4* __restrict__ grad_out, const u32x4* y, const int32_t* __restrict__ dst_row,
                 const float* __restrict__ w, u32x4* grad_y, float* __restrict__ grad_w, int t0,
                 int t1, int k, int nvec) {
  constexpr int kEl = kBf16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int t = t0 + blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= t1) return;
  const int my_row = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  const float my_w = lane < k ? w[(size_t)t * k + lane] : 0.0f;
  const u32x4* go = grad_out + (size_t)t * nvec;
  for (int j = 0; j < k; ++j) {
    const int r = __shfl(my_row, j);
    const float wj = __shfl(my_w, j);
    if (r < 0) {
      if (lane == 0) grad_w[(size_t)t * k + j] = 0.0f;
      continue;
    }
    const u32x4* yr = y + (size_t)r * nvec;
    u32x4* gy = grad_y + (size_t)r * nvec;
    float dot = 0.0f;
    for (int v = lane; v < nvec; v += 64) {
      const u32x4 gq = go[v], yq = yr[v];
      float gf[kEl], yf[kEl];
      if constexpr (kBf16) {
        unpack_bf16x8(gq, gf);
        unpack_bf16x8(yq, yf);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          gf[q] = __uint_as_float(gq[q]);
          yf[q] = __uint_as_float(yq[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < kEl; ++q) {
        dot = __builtin_fmaf(gf[q], yf[q], dot);
        gf[q] *= wj;
      }
      if constexpr (kBf16) {
        gy[v] = pack_bf16x8(gf);
      } else {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(gf[q]);
        gy[v] = o;
      }
    }
    for (int d = 32; d > 0; d >>= 1) dot += __shfl_xor(dot, d);
    if (lane == 0) grad_w[(size_t)t * k + j] = dot;
  }
}

}  // namespace

hipError_t launch_combine_backward(const Shape& s, int t0, int t1, const void* grad_out,
                                   const void* y, const int32_t* dst_row, const float* w,
                                   void* grad_y, float* grad_w, hipStream_t st) {
  if (t1 <= t0) return hipSuccess;
  const int nvec = (int)((int64_t)s.H * s.elem / 16);
  const unsigned blocks = (unsigned)((t1 - t0 + kWavesPerBlock - 1) / kWavesPerBlock);
  if (s.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_backward<true>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, st,
                       (const u32x4*)grad_out, (const u32x4*)y, dst_row, w, (u32x4*)grad_y,
                       grad_w, t0, t1, s.k, nvec);
  else
    hipLaunchKernelGGL(combine_backward<false>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, st,
                       (const u32x4*)grad_out, (const u32x4*)y, dst_row, w, (u32x4*)grad_y,
                       grad_w, t0, t1, s.k, nvec);
  return hipGetLastError();
}

hipError_t launch_permute(const Shape& s, int t0, int t1, const void* hidden,
                          const int32_t* dst_row, void* x_perm, hipStream_t st) {
  if (t1 <= t0) return hipSuccess;
  const int nvec = (int)((int64_t)s.H * s.elem / 16);
  const unsigned blocks = (unsigned)((t1 - t0 + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(permute_rows, dim3(blocks), dim3(64 * kWavesPerBlock), 0, st,
                     (const u32x4*)hidden, dst_row, (u32x4*)x_perm, t0, t1, s.k, nvec);
  return hipGetLastError();
}

hipError_t launch_combine_pair(const Shape& s, int t0, int t_mid, int t1, const void* y0,
                               const void* y1, const int32_t* dst_row, const float* w,
                               void* out, hipStream_t st) {
  if (t1 <= t0) return hipSuccess;
  const int nvec = (int)((int64_t)s.H * s.elem / 16);
  const unsigned blocks = (unsigned)((t1 - t0 + kWavesPerBlock - 1) / kWavesPerBlock);
  if (s.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_rows<true>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, st,
                       (const u32x4*)y0, (const u32x4*)y1, t_mid, dst_row, w, (u32x4*)out, t0,
                       t1, s.k, nvec);
  else
    hipLaunchKernelGGL(combine_rows<false>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, st,
                       (const u32x4*)y0, (const u32x4*)y1, t_mid, dst_row, w, (u32x4*)out, t0,
                       t1, s.k, nvec);
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& s, int t0, int t1, const void* y,
                          const int32_t* dst_row, const float* w, void* out, hipStream_t st) {
  return launch_combine_pair(s, t0, t1, t1, y, y, dst_row, w, out, st);
}

}  // namespace moe
