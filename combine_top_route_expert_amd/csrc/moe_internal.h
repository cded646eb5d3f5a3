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

// ---- direct-to-LDS loads through buffer descriptors (GEMM kernels) ----------
// A raw descriptor of the bytes above p (stride 0, the largest record count:
// offsets are computed from in-range rows, as for global loads) and the 16-byte
// direct-to-LDS load through it: lane l's 16 bytes at off + soff land at
// dst + 16 l.  The host pass of the compiler has no buffer builtins (it never
// runs kernels), hence the empty stand-ins there.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t raw_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, -1, 0x00020000);
}
__device__ __forceinline__ void buffer_load_lds16(rsrc_t r, char* dst, uint32_t off, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           off, soff, 0, 0);
}
// The same with the non-temporal cache policy (bytes read once: streamed past
// the caches instead of kept).
__device__ __forceinline__ void buffer_load_lds16_nt(rsrc_t r, char* dst, uint32_t off, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           off, soff, 0, 2);
}
#else
struct rsrc_t {};
__device__ __forceinline__ rsrc_t raw_rsrc(const void*) { return {}; }
__device__ __forceinline__ void buffer_load_lds16(rsrc_t, char*, uint32_t, int) {}
__device__ __forceinline__ void buffer_load_lds16_nt(rsrc_t, char*, uint32_t, int) {}
#endif

// Host: whether rows of ld 2-byte elements in the buffers at p0 and p1 (at
// most `rows` rows each) lie within 4 GiB above the lower base, so that
// descriptor loads from that base reach them with 32-bit offsets.
inline bool rows_fit_4g(const void* p0, const void* p1, int64_t rows, int64_t ld) {
  const uint64_t a = (uint64_t)(uintptr_t)p0, b = (uint64_t)(uintptr_t)p1;
  const uint64_t lo = a < b ? a : b, hi = (a > b ? a : b) + (uint64_t)rows * ld * 2;
  return hi - lo < ((uint64_t)1 << 32);
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
// Both chunks of a pair in one launch: tokens [t0, t_mid) read y0, [t_mid, t1) y1.
hipError_t launch_combine_pair(const Shape& s, int t0, int t_mid, int t1, const void* y0,
                               const void* y1, const int32_t* dst_row, const float* w,
                               void* out, hipStream_t st);

// ---- weight warm-up (prefetch.hip) -------------------------------------------
// Reads the first head_bytes (a multiple of 16) of each of `rows` rows of
// row_bytes so they sit in the caches; writes nothing but, at most, *sink.
hipError_t launch_warm_weights(const void* w, int64_t rows, int64_t row_bytes, int head_bytes,
                               int32_t* sink, hipStream_t st);

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
  // optional [E]: the experts in the order their tiles are dealt out (largest
  // first, from launch_expert_order); null: expert order
  const int32_t* order = nullptr;
};
// order[r] = the expert with the r-th most rows over one chunk or a pair (ties
// to the lower id): one workgroup, E <= 1024.
hipError_t launch_expert_order(const Shape& s, const int32_t* off0, const int32_t* off1,
                               int32_t* order, hipStream_t st);
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
  int single;        // 1 if the tile holds all of its expert's rows (its only m-tile)

  // Row index of virtual row v on a split side: (buffer, row).
  __device__ __forceinline__ int split_row(int v, int* part) const {
    *part = v >= n0;
    return v < n0 ? lo0 + v : lo1 + (v - n0);
  }
  // Row index of virtual row v on a joint side.
  __device__ __forceinline__ int joint_row(int v) const { return lo0 + lo1 + v; }
};

// Grouped-GEMM tile map.  Expert e owns n_e rows (its rows in one or two
// chunks) and ceil(n_e / BM) m-tiles.  Numbering: first the m-tiles of the
// large experts (n_e >= large_min), expert by expert; then the single m-tile
// of each small expert (0 < n_e < large_min <= BM), in four size classes,
// larger first: more than BM/2 rows, more than BM/4, more than BM/8, the rest
// (each class expert by expert).  large_min = 1 gives plain expert order.
// Every wave of a workgroup builds the map independently (wave scans over E
// experts, E/64 per lane) and gets the same answer.
struct MTileMap {
  static constexpr int kClasses = 5;  // 0: large experts' m-tiles; 1..4: small experts by size
  int total;                // m-tiles
  int large;                // m-tiles of large experts (numbers 0 .. large-1)
  int start[kClasses + 1];  // first number of each class; start[kClasses] = total
  int large_min;            // rows that make an expert large
  int excl_large, incl_large;   // this lane's range of large-expert m-tiles
  int excl_small[2], incl_small[2];  // this lane's range within classes 1|2 and
                                     // 3|4, 16 bits per class (E < 65536)
  int e_begin, e_end;       // this lane's experts

  static __device__ __forceinline__ int small_class(int n, int BM) {
    return n > BM / 2 ? 1 : n > BM / 4 ? 2 : n > BM / 8 ? 3 : 4;
  }

  static __device__ __forceinline__ int rows_of(const int32_t* __restrict__ off0,
                                                const int32_t* __restrict__ off1, int e) {
    int n = off0[e + 1] - off0[e];
    if (off1) n += off1[e + 1] - off1[e];
    return n;
  }

  static __device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = __lane_id();
    for (int d = 1; d < 64; d <<= 1) {
      const int n = __shfl_up(v, d);
      if (lane >= d) v += n;
    }
    return v;
  }

  __device__ __forceinline__ void build(const int32_t* __restrict__ off0,
                                        const int32_t* __restrict__ off1, int E, int BM,
                                        int large_rows) {
    large_min = large_rows;
    const int lane = __lane_id();
    const int per = (E + 63) >> 6;
    e_begin = lane * per;
    e_end = e_begin + per < E ? e_begin + per : E;
    int nl = 0, p12 = 0, p34 = 0;  // small-expert counts: classes 1|2 and 3|4, 16 bits each
    for (int e = e_begin; e < e_end; ++e) {
      const int n = rows_of(off0, off1, e);
      if (n >= large_min) {
        nl += (n + BM - 1) / BM;
      } else if (n > 0) {
        const int c = small_class(n, BM);
        const int add = 1 << (16 * ((c - 1) & 1));
        if (c <= 2) p12 += add; else p34 += add;
      }
    }
    incl_large = wave_incl_scan(nl);
    excl_large = incl_large - nl;
    incl_small[0] = wave_incl_scan(p12);
    incl_small[1] = wave_incl_scan(p34);
    excl_small[0] = incl_small[0] - p12;
    excl_small[1] = incl_small[1] - p34;
    large = __shfl(incl_large, 63);
    const int t12 = __shfl(incl_small[0], 63), t34 = __shfl(incl_small[1], 63);
    start[0] = 0;
    start[1] = large;
    start[2] = start[1] + (t12 & 0xFFFF);
    start[3] = start[2] + (t12 >> 16);
    start[4] = start[3] + (t34 & 0xFFFF);
    start[5] = start[4] + (t34 >> 16);
    total = start[5];
  }

  // Rows of m-tile mt (< total), for all lanes.
  __device__ __forceinline__ TileRows locate(const int32_t* __restrict__ off0,
                                             const int32_t* __restrict__ off1, int BM,
                                             int mt) const {
    const int lane = __lane_id();
    // class and range by selects only (no dynamic indexing, which would put
    // the arrays in scratch memory)
    int cls = 0, base = 0;
#pragma unroll
    for (int c = 1; c < kClasses; ++c)
      if (mt >= start[c]) {
        cls = c;
        base = start[c];
      }
    const int local = mt - base;
    int lo, hi;
    if (cls == 0) {
      lo = excl_large;
      hi = incl_large;
    } else {
      const int sh = 16 * ((cls - 1) & 1);
      const int ex = cls <= 2 ? excl_small[0] : excl_small[1];
      const int in = cls <= 2 ? incl_small[0] : incl_small[1];
      lo = (ex >> sh) & 0xFFFF;
      hi = (in >> sh) & 0xFFFF;
    }
    const uint64_t own = __ballot(lo <= local && local < hi);
    const int owner = __ffsll((unsigned long long)own) - 1;
    int fe = 0, fv0 = 0, frows = 0, flo0 = 0, fn0 = 0, flo1 = 0, fsingle = 0;
    if (lane == owner) {
      int acc = lo;
      for (int e = e_begin; e < e_end; ++e) {
        const int n = rows_of(off0, off1, e);
        bool hit = false;
        if (cls == 0) {
          if (n >= large_min) {
            const int t = (n + BM - 1) / BM;
            if (local < acc + t) {
              hit = true;
              fv0 = (local - acc) * BM;
              frows = n - fv0 < BM ? n - fv0 : BM;
            }
            acc += t;
          }
        } else if (n > 0 && n < large_min && small_class(n, BM) == cls) {
          if (local == acc) {
            hit = true;
            fv0 = 0;
            frows = n;
          }
          ++acc;
        }
        if (hit) {
          fsingle = fv0 == 0 && frows == n;
          fe = e;
          flo0 = off0[e];
          fn0 = off0[e + 1] - flo0;
          flo1 = off1 ? off1[e] : 0;
          break;
        }
      }
    }
    // the owner's values, broadcast to the wave, are wave-uniform: kept in
    // scalar registers (as vector registers they stayed live across the K loop)
    TileRows r;
    r.e = __builtin_amdgcn_readfirstlane(__shfl(fe, owner));
    r.v0 = __builtin_amdgcn_readfirstlane(__shfl(fv0, owner));
    r.rows = __builtin_amdgcn_readfirstlane(__shfl(frows, owner));
    r.lo0 = __builtin_amdgcn_readfirstlane(__shfl(flo0, owner));
    r.n0 = __builtin_amdgcn_readfirstlane(__shfl(fn0, owner));
    r.lo1 = __builtin_amdgcn_readfirstlane(__shfl(flo1, owner));
    r.single = __builtin_amdgcn_readfirstlane(__shfl(fsingle, owner));
    return r;
  }
};

// Row split of a compact tile (at most 32, 64, 128 or 160 rows) of the 256 x 256
// grouped GEMM between its two wave rows: wave row 0 takes 32-row blocks
// 0 .. f0-1, wave row 1 the next f1 (rows is the tile's row count, or the
// bound of its class: both give the same split).  A tile that holds its
// expert's whole row block (a weight-streaming tile) spreads its rows over
// both wave rows, so both waves on a SIMD run MFMAs and each hides the other's
// fragment reads (DeepSeek-V3-shaped gate/up: one wave per SIMD holding all of
// a 128-row tile's MFMAs ran them at about half the matrix rate; the layer
// 4.59 -> 4.48 ms).  The tail tile of a larger expert keeps them on wave row 0
// (spreading them there measured 1-3% slower on the MFMA-bound launches).
// Also compiled for the host, where its coverage is checked.
__host__ __device__ constexpr int compact_f0(int rows, bool spread) {
  return spread ? (rows <= 64 ? 1 : rows <= 128 ? 2 : 3) : (rows <= 32 ? 1 : rows <= 64 ? 2 : 4);
}
__host__ __device__ constexpr int compact_f1(int rows, bool spread) {
  return spread ? (rows <= 32 ? 0 : rows <= 64 ? 1 : 2) : (rows <= 128 ? 0 : 1);
}

// Workgroup -> (m-tile, n-tile) for an MTileMap.  Workgroup b runs on XCD
// b % 8 (checked against the hardware XCC id), and an XCD starts its
// workgroups in order of b.  Which m-tiles an XCD gets: a contiguous range of
// the large experts' m-tiles (ceil(large/8) per XCD, fewer for the last
// ones), so an expert's weight panels are fetched into one XCD's L2; then the
// small experts' m-tiles (larger first) top up the XCDs that got fewer large
// ones to ceil(large/8), and the rest are dealt round-robin.  So no XCD gets
// more than ceil(total/8) m-tiles and the work is spread evenly.  In which
// order: the XCD's large and small m-tiles are interleaved evenly, so that
// MFMA-bound large tiles and weight-streaming small tiles run side by side
// (small tiles started all together contend for HBM), except that its last
// `reserve` m-tiles are kept for its smallest ones, to shorten the tail of the
// launch (every caller passes ceil(32/n_tiles), about one workgroup per CU).
// Every m-tile comes with all its n-tiles.  The grid has 8 * ceil(bound/8) * n_tiles workgroups (xcd_grid);
// those past their XCD's share exit.
// xcd_tile_at: the same for position q of XCD x's sequence (a workgroup that
// takes several tiles walks q, q + G, q + 2G, ... with G its XCD's workgroup
// count); false once q is past the XCD's tiles.  Pure integer arithmetic on
// tm.total and tm.large, also compiled for the host so that its coverage
// properties can be checked there.
__host__ __device__ __forceinline__ bool xcd_tile_at(const MTileMap& tm, int n_tiles, int x, int q,
                                                     int reserve, int* mt, int* nt) {
  const int ml = q / n_tiles;
  *nt = q - ml * n_tiles;
  const int per = (tm.large + 7) >> 3;
  int nl = tm.large - x * per;  // large-expert m-tiles of this XCD
  nl = nl < 0 ? 0 : nl > per ? per : nl;
  const int S = tm.total - tm.large;  // small-expert m-tiles, numbered p = 0 .. S-1
  const int D = 8 * per - tm.large;   // slots below `per` over all XCDs
  const int deficit = per - nl;       // this XCD's slots below `per`
  int before = x * per - tm.large;    // slots below `per` on the XCDs before it
  before = before < 0 ? 0 : before;
  int ns = S - before < 0 ? 0 : S - before;  // this XCD's small m-tiles
  ns = ns < deficit ? ns : deficit;
  if (S > D + x) ns += (S - D - x + 7) / 8;
  const int C = nl + ns;
  if (ml >= C) return false;
  const int R = reserve < ns ? reserve : ns;  // small m-tiles kept for the end
  const int C1 = C - R;                       // positions of the even interleave
  int j;                                      // this XCD's j-th small m-tile
  if (ml >= C1) {
    j = ns - R + (ml - C1);
  } else {
    int lb, la;  // large m-tiles before positions ml and ml + 1
    if (C1 < 65536) {  // nl <= C1: the products fit 32 bits
      lb = (int)((unsigned)ml * (unsigned)nl / (unsigned)C1);
      la = (int)((unsigned)(ml + 1) * (unsigned)nl / (unsigned)C1);
    } else {
      lb = (int)((long long)ml * nl / C1);
      la = (int)((long long)(ml + 1) * nl / C1);
    }
    if (la > lb) {
      *mt = x * per + lb;
      return true;
    }
    j = ml - lb;
  }
  const int p = j < deficit ? before + j : D + (j - deficit) * 8 + x;
  *mt = tm.large + p;
  return *mt < tm.total;
}

__device__ __forceinline__ bool xcd_tile(const MTileMap& tm, int n_tiles, int* mt, int* nt) {
  return xcd_tile_at(tm, n_tiles, blockIdx.x & 7, blockIdx.x >> 3, (32 + n_tiles - 1) / n_tiles,
                     mt, nt);
}

// Round-robin variant: XCD x takes m-tiles x, x + 8, x + 16, ... (each with all
// its n-tiles).  For the weight-gradient products, whose m-tiles are (expert,
// row block) pairs with a reduction as long as the expert's row count, this
// spreads each heavily loaded expert over all eight XCDs instead of queueing
// it on one.  Grid: xcd_grid_rr.
__device__ __forceinline__ bool xcd_tile_rr(int total, int n_tiles, int* mt, int* nt) {
  const int x = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int ml = q / n_tiles;
  *mt = ml * 8 + x;
  *nt = q - ml * n_tiles;
  return *mt < total;
}

// Host side: grid of xcd_tile for a bound on the m-tiles (no XCD gets more
// than ceil(total/8) of them).
inline int64_t xcd_grid(int64_t m_tiles_bound, int n_tiles) {
  return 8 * ((m_tiles_bound + 7) / 8) * (int64_t)n_tiles;
}

// Host side: grid of xcd_tile_rr for exactly m_tiles m-tiles.
inline int64_t xcd_grid_rr(int64_t m_tiles, int n_tiles) {
  return 8 * ((m_tiles + 7) / 8) * (int64_t)n_tiles;
}

// Upper bound on the m-tiles of a grouped GEMM over `rows` rows split among E
// experts: every expert adds at most one partial tile.
inline int64_t m_tiles_bound(int64_t rows, int E, int BM) {
  int64_t partial = rows < E ? rows : E;
  return rows / BM + partial;
}

}  // namespace moe
