// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Validated shape with defaults resolved.
struct Shape {
  int T, H, E, k, I, G, N;
  moe_dtype dtype;
  int Tc;        // ceil(T / N)
  int64_t A;     // T * k
  int elem;      // bytes per hidden/weight element
};

moe_status resolve_shape(const moe_shape* s, Shape* out);

inline void chunk_tokens(const Shape& s, int c, int* t0, int* t1) {
  int64_t a = (int64_t)c * s.Tc, b = (int64_t)(c + 1) * s.Tc;
  *t0 = (int)(a < s.T ? a : s.T);
  *t1 = (int)(b < s.T ? b : s.T);
}

// ---- routing metadata (meta.hip) -------------------------------------------
constexpr int kMaxExperts = 1024;  // largest E the library accepts
constexpr int kMetaSeg = 1024;     // segment granule, in assignments (one wave per segment)
constexpr int kScanStage = 16384;  // ints of one chunk's [segments][E] block staged in LDS

struct MetaPlan {
  int seg;                 // assignments per segment (multiple of kMetaSeg)
  int segs_per_chunk;
  int64_t nseg;            // N * segs_per_chunk
  size_t seg_counts_off;   // int32 [nseg][E]
  size_t seg_invalid_off;  // int32 [nseg]
  size_t bytes;
};
MetaPlan meta_plan(const Shape& s);

hipError_t launch_route_meta(const Shape& s, const int32_t* idx, int32_t* counts,
                             int32_t* offsets, int32_t* splits, int32_t* src_row,
                             int32_t* dst_row, int32_t* dev_error, void* ws, hipStream_t st);

// ---- permute / combine (permute_combine.hip) --------------------------------
hipError_t launch_permute(const Shape& s, int t0, int t1, const void* hidden,
                          const int32_t* dst_row, void* x_perm, hipStream_t st);
hipError_t launch_combine(const Shape& s, int t0, int t1, const void* y,
                          const int32_t* dst_row, const float* w, void* out, hipStream_t st);

// ---- grouped GEMMs (gemm_bf16.hip, gemm_f32.hip) ----------------------------
// `rows_bound` is the chunk's assignment count; `offsets_c` the chunk's E+1 offsets.
hipError_t launch_gate_up_bf16(const Shape& s, int64_t rows_bound, const void* x_perm,
                               const int32_t* offsets_c, const void* w_gate_up, void* act,
                               hipStream_t st);
hipError_t launch_down_bf16(const Shape& s, int64_t rows_bound, const void* act,
                            const int32_t* offsets_c, const void* w_down, void* y,
                            hipStream_t st);
hipError_t launch_gate_up_f32(const Shape& s, int64_t rows_bound, const void* x_perm,
                              const int32_t* offsets_c, const void* w_gate_up, void* act,
                              hipStream_t st);
hipError_t launch_down_f32(const Shape& s, int64_t rows_bound, const void* act,
                           const int32_t* offsets_c, const void* w_down, void* y,
                           hipStream_t st);

// ---- small device helpers ----------------------------------------------------
__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << __lane_id()) - 1ull;
}

// Grouped-GEMM tile lookup.  Expert e owns rows [off[e], off[e+1]) and
// ceil(rows_e / BM) m-tiles; m-tiles are numbered expert by expert.  Every wave
// of the calling workgroup runs this independently (one wave scan over E
// experts, E/64 per lane) and gets the same answer.  Returns false for m-tile
// indices past the last tile (surplus workgroups of the host-bounded grid).
__device__ __forceinline__ bool find_m_tile(const int32_t* __restrict__ off, int E, int BM,
                                            int mt, int* e_out, int* m0_out, int* rows_out) {
  const int lane = __lane_id();
  const int per = (E + 63) >> 6;
  const int e_begin = lane * per;
  const int e_end = e_begin + per < E ? e_begin + per : E;
  int sum = 0;
  for (int e = e_begin; e < e_end; ++e) sum += (off[e + 1] - off[e] + BM - 1) / BM;
  int incl = sum;
  for (int d = 1; d < 64; d <<= 1) {
    int n = __shfl_up(incl, d);
    if (lane >= d) incl += n;
  }
  const int total = __shfl(incl, 63);
  if (mt >= total) return false;
  const int excl = incl - sum;
  const uint64_t own = __ballot(excl <= mt && mt < incl);
  const int owner = __ffsll((unsigned long long)own) - 1;
  int fe = 0, fm0 = 0, frows = 0;
  if (lane == owner) {
    int acc = excl;
    for (int e = e_begin; e < e_end; ++e) {
      const int lo = off[e], n = off[e + 1] - lo;
      const int t = (n + BM - 1) / BM;
      if (mt < acc + t) {
        fe = e;
        fm0 = lo + (mt - acc) * BM;
        frows = lo + n - fm0 < BM ? lo + n - fm0 : BM;
        break;
      }
      acc += t;
    }
  }
  *e_out = __shfl(fe, owner);
  *m0_out = __shfl(fm0, owner);
  *rows_out = __shfl(frows, owner);
  return true;
}

// Upper bound on the m-tiles of a grouped GEMM over `rows` rows split among E
// experts: every expert adds at most one partial tile.
inline int64_t m_tiles_bound(int64_t rows, int E, int BM) {
  int64_t partial = rows < E ? rows : E;
  return rows / BM + partial;
}

}  // namespace moe
