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
constexpr int kMetaSeg = 256;      // segment granule, in assignments (one wave per segment)
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
// w may be null: unit weights (the permute backward, a gather-sum over k rows).
hipError_t launch_combine(const Shape& s, int t0, int t1, const void* y,
                          const int32_t* dst_row, const float* w, void* out, hipStream_t st);

// ---- grouped GEMMs (gemm_bf16.hip, gemm_f32.hip) ----------------------------
// One grouped GEMM over the rows of one chunk, or of the two chunks of a pair.
// Expert e's rows are the chunk-0 block [off0[e], off0[e+1]) followed by the
// chunk-1 block [off1[e], off1[e+1]) (none when off1 is null): the expert is
// multiplied once per launch, so its weights are streamed once for both chunks.
// A side that is "split" holds the two chunks in two buffers at their own
// chunk-local rows; a "joint" side is one buffer in which expert e's rows start
// at off0[e] + off1[e] (the pair's rows grouped by expert; for one chunk this is
// the chunk's own layout).
struct GroupedIO {
  const void* a[2];      // A: [rows][K]; a[1] used when a_split
  void* c[2];            // C: [rows][ncols]; c[1] used when c_split
  const int32_t* off[2]; // E + 1 chunk-local offsets of each chunk; off[1] may be null
  bool a_split, c_split;
  int64_t rows_bound;    // total rows of the launch (host-known bound)
  void* gu = nullptr;    // gate_up only, optional: joint [rows][2I] copy of g and u
  // Gather (gate_up only, optional): A is hidden_states [T][K] (a[0]) and row r
  // of chunk part p is token gather[p][r] / k -- the permute fused into the
  // GEMM's row addressing (gather[p] = the chunk's slice of src_row).
  const int32_t* gather[2] = {nullptr, nullptr};
  int gather_k = 0;
};

// Backward products (gemm_bwd_bf16.hip, gemm_bwd_f32.hip).  Rows follow the
// GroupedIO rules (split or joint sides, one chunk or a pair).
struct DgradIO {         // C[r] = A[r] . B[e]   with B[e] stored [K][N]
  const void* a[2];      // [rows][K]
  bool a_split;
  const void* B;         // [E][K][N]
  int K, N;
  void* c[2];            // [rows][N] (plain epilogue)
  bool c_split;
  void* gu;              // SwiGLU epilogue (N = I): joint [rows][2I] g, u -> grad_g, grad_u
  const int32_t* off[2];
  int64_t rows_bound;
};
struct WgradIO {         // C[e] (+)= sum over e's rows v of A[v]^T B[v]
  const void* a[2];      // [rows][M]
  bool a_split;
  const void* b[2];      // [rows][N]
  bool b_split;
  float* C;              // [E][M][N]
  int M, N;
  int accumulate;        // 0: overwrite (experts without rows get zeros), 1: add
  const int32_t* off[2];
};
hipError_t launch_dgrad_bf16(const Shape& s, const DgradIO& io, hipStream_t st);
hipError_t launch_wgrad_bf16(const Shape& s, const WgradIO& io, hipStream_t st);
hipError_t launch_dgrad_f32(const Shape& s, const DgradIO& io, hipStream_t st);
hipError_t launch_wgrad_f32(const Shape& s, const WgradIO& io, hipStream_t st);
hipError_t launch_combine_backward(const Shape& s, int t0, int t1, const void* grad_out,
                                   const void* y, const int32_t* dst_row, const float* w,
                                   void* grad_y, float* grad_w, hipStream_t st);
hipError_t launch_gate_up_bf16(const Shape& s, const GroupedIO& io, const void* w_gate_up,
                               hipStream_t st);
hipError_t launch_down_bf16(const Shape& s, const GroupedIO& io, const void* w_down,
                            hipStream_t st);
hipError_t launch_gate_up_f32(const Shape& s, const GroupedIO& io, const void* w_gate_up,
                              hipStream_t st);
hipError_t launch_down_f32(const Shape& s, const GroupedIO& io, const void* w_down,
                           hipStream_t st);

// ---- small device helpers ----------------------------------------------------
__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << __lane_id()) - 1ull;
}

// Rows of one m-tile: expert e, virtual rows [v0, v0 + rows) of the expert's
// concatenated block (chunk-0 rows, then chunk-1 rows).
struct TileRows {
  int e, v0, rows;
  int lo0, n0, lo1;  // chunk-0 first row and count; chunk-1 first row (0 if none)

  // Row index of virtual row v on a split side: (buffer, row).
  __device__ __forceinline__ int split_row(int v, int* part) const {
    *part = v >= n0;
    return v < n0 ? lo0 + v : lo1 + (v - n0);
  }
  // Row index of virtual row v on a joint side.
  __device__ __forceinline__ int joint_row(int v) const { return lo0 + lo1 + v; }
};

// Grouped-GEMM tile map.  Expert e owns n_e rows (its rows in one or two
// chunks) and ceil(n_e / BM) m-tiles; m-tiles are numbered expert by expert.
// A map can be restricted to a class of experts by row count, so that one
// launch covers long expert blocks with a large tile and another the short
// ones.  Every wave of a workgroup builds the map independently (one wave scan
// over E experts, E/64 per lane) and gets the same answer.
struct MTileMap {
  int total;              // m-tiles of all experts in the class
  int excl, incl;         // this lane's m-tile range
  int e_begin, e_end;     // this lane's experts
  int lo_rows, hi_rows;   // class: experts with lo_rows <= rows < hi_rows

  __device__ __forceinline__ int tiles_of(int n, int BM) const {
    return (n >= lo_rows && n < hi_rows) ? (n + BM - 1) / BM : 0;
  }

  static __device__ __forceinline__ int rows_of(const int32_t* __restrict__ off0,
                                                const int32_t* __restrict__ off1, int e) {
    int n = off0[e + 1] - off0[e];
    if (off1) n += off1[e + 1] - off1[e];
    return n;
  }

  __device__ __forceinline__ void build(const int32_t* __restrict__ off0,
                                        const int32_t* __restrict__ off1, int E, int BM,
                                        int lo = 1, int hi = 0x7fffffff) {
    lo_rows = lo;
    hi_rows = hi;
    const int lane = __lane_id();
    const int per = (E + 63) >> 6;
    e_begin = lane * per;
    e_end = e_begin + per < E ? e_begin + per : E;
    int sum = 0;
    for (int e = e_begin; e < e_end; ++e) sum += tiles_of(rows_of(off0, off1, e), BM);
    incl = sum;
    for (int d = 1; d < 64; d <<= 1) {
      const int n = __shfl_up(incl, d);
      if (lane >= d) incl += n;
    }
    excl = incl - sum;
    total = __shfl(incl, 63);
  }

  // Rows of m-tile mt (< total), for all lanes.
  __device__ __forceinline__ TileRows locate(const int32_t* __restrict__ off0,
                                             const int32_t* __restrict__ off1, int BM,
                                             int mt) const {
    const int lane = __lane_id();
    const uint64_t own = __ballot(excl <= mt && mt < incl);
    const int owner = __ffsll((unsigned long long)own) - 1;
    int fe = 0, fv0 = 0, frows = 0, flo0 = 0, fn0 = 0, flo1 = 0;
    if (lane == owner) {
      int acc = excl;
      for (int e = e_begin; e < e_end; ++e) {
        const int n = rows_of(off0, off1, e);
        const int t = tiles_of(n, BM);
        if (mt < acc + t) {
          fe = e;
          fv0 = (mt - acc) * BM;
          frows = n - fv0 < BM ? n - fv0 : BM;
          flo0 = off0[e];
          fn0 = off0[e + 1] - flo0;
          flo1 = off1 ? off1[e] : 0;
          break;
        }
        acc += t;
      }
    }
    TileRows r;
    r.e = __shfl(fe, owner);
    r.v0 = __shfl(fv0, owner);
    r.rows = __shfl(frows, owner);
    r.lo0 = __shfl(flo0, owner);
    r.n0 = __shfl(fn0, owner);
    r.lo1 = __shfl(flo1, owner);
    return r;
  }
};

// Workgroup -> (m-tile, n-tile).  Workgroup b runs on XCD b % 8 (checked
// against the hardware XCC id); each XCD gets a contiguous range of
// ceil(total/8) m-tiles with all their n-tiles, in order, so an m-tile's
// activation panel and an expert's weight panels are fetched into one XCD's L2
// instead of up to eight (dealing m-tiles round-robin balances the XCDs better
// but measured no faster: each tile then misses more).  The grid has
// 8 * ceil(bound/8) * n_tiles workgroups; those past their XCD's range exit.
__device__ __forceinline__ bool xcd_tile(int total, int n_tiles, int* mt, int* nt) {
  const int x = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int per = (total + 7) >> 3;
  const int ml = q / n_tiles;
  if (ml >= per) return false;
  *mt = x * per + ml;
  *nt = q - ml * n_tiles;
  return *mt < total;
}

// Round-robin variant: XCD x takes m-tiles x, x + 8, x + 16, ... (each with all
// its n-tiles).  For the weight-gradient products, whose m-tiles are (expert,
// row block) pairs with a reduction as long as the expert's row count, this
// spreads each heavily loaded expert over all eight XCDs instead of queueing
// it on one.  Same grid as xcd_tile.
__device__ __forceinline__ bool xcd_tile_rr(int total, int n_tiles, int* mt, int* nt) {
  const int x = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int ml = q / n_tiles;
  *mt = ml * 8 + x;
  *nt = q - ml * n_tiles;
  return *mt < total;
}

// Host side: grid of xcd_tile for a bound on the m-tiles.
inline int64_t xcd_grid(int64_t m_tiles_bound, int n_tiles) {
  return 8 * ((m_tiles_bound + 7) / 8) * (int64_t)n_tiles;
}

// Upper bound on the m-tiles of a grouped GEMM over `rows` rows split among E
// experts: every expert adds at most one partial tile.
inline int64_t m_tiles_bound(int64_t rows, int E, int BM) {
  int64_t partial = rows < E ? rows : E;
  return rows / BM + partial;
}

}  // namespace moe
