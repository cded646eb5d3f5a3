// Backward grouped GEMMs on gfx950 bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Gradient of the expert computation of the MindSpeed Chunk MoE article (core
// principle / timing-diagram sections; SwiGLU reading), chunk pair by chunk
// pair with the forward recomputed (the guide's recompute option):
//   dgrad down  : grad_act[r] = grad_y[r] . W_d[e]        ([rows][H] x [H][I])
//                 fused with the SwiGLU backward: grad_g = grad_act u silu'(g),
//                 grad_u = grad_act silu(g), written over the saved g, u
//   dgrad gate/up: grad_x[r] = grad_gu[r] . W_gu[e]      ([rows][2I] x [2I][H])
//   wgrad       : grad_W[e] (+)= sum over e's rows v of A[v]^T B[v]
//                 (W_d: A = grad_y, B = act;  W_gu: A = grad_gu, B = x_perm)
//
// The dgrad B operand (weights [K][N]) and both wgrad operands ([rows][M],
// [rows][N], the reduction running over rows) are stored with the reduction
// index outermost.  Stages are copied global -> LDS row by row with the
// direct-to-LDS load, and the MFMA fragments (8 consecutive K values of one
// column per lane) are read with ds_read_b64_tr_b16: within each group of 16
// lanes, output lane i element j comes from source lane 4j + i/4, element i%4
// (measured), so a source lane that reads 4 consecutive columns of one K row
// delivers a 4 (K) x 16 (column) block already transposed.  The 16-byte chunk c
// of LDS row k sits at slot c ^ 4(k mod 4), which spreads the 4 rows x 4 chunks
// a 32-lane phase reads over 16 distinct bank groups.
//
// The dgrad groups and places tiles like the forward kernels (MTileMap,
// xcd_tile); the wgrad tiles are numbered (expert, m-tile), dealt to the XCDs
// round-robin (xcd_tile_rr), and the K loop runs over the expert's rows of both
// chunks; rows past the expert's block are loaded from a
// clamped row and zeroed in the A fragment.
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BK = 64;
constexpr int wait_vm(int v) { return (v & 0xF) | ((v >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Forces v to be computed at this point (an empty asm that reads it), so the
// compiler cannot sink the arithmetic below later stores; the waits for the
// loads it consumes then come before the first store, not after each one.
__device__ __forceinline__ void pin(uint32_t v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void pin(float v) { asm volatile("" ::"v"(v)); }

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// One operand side of a grouped product: rows of expert e are its chunk-0 rows
// then its chunk-1 rows, either in two buffers (split) or grouped in one (joint).
struct Side {
  const uint16_t* p[2];
  int split;
  int64_t ld;  // elements per row
};

// The two base addresses as wave-uniform integers.  Selecting between them per
// lane as integers keeps the compiler from turning the choice into a per-lane
// load of the pointer from the argument block (whose wait would also drain the
// loads in flight).
struct SideU {
  uint64_t b0, b1;
  int split;
  int64_t ld;
};

__device__ __forceinline__ uint64_t uniform_u64(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ SideU uniform_side(const Side& s) {
  SideU u;
  u.b0 = uniform_u64(s.p[0]);
  u.b1 = uniform_u64(s.p[1]);
  u.split = s.split;
  u.ld = s.ld;
  return u;
}

// Byte address of element `col` of virtual row v of the tile's expert.
__device__ __forceinline__ uint64_t side_addr(const SideU& s, const TileRows& tr, int v, int col) {
  int64_t row;
  uint64_t shift = 0;  // b1 - b0 for rows of the second chunk (added, not selected)
  if (s.split) {
    const bool second = v >= tr.n0;
    row = second ? tr.lo1 + (v - tr.n0) : tr.lo0 + v;
    shift = second ? s.b1 - s.b0 : 0ull;
  } else {
    row = (int64_t)tr.joint_row(v);
  }
  return s.b0 + shift + (uint64_t)(row * s.ld + col) * 2u;
}

// ---- LDS layouts --------------------------------------------------------------
// K-contiguous rows (dgrad A): BM rows x 128 bytes per stage, chunk c of row r at
// slot c ^ ((r >> 1) & 7) (same as the forward kernels).
__device__ __forceinline__ int kfrag_offset(int lane, int kk) {
  const int r = lane & 31;
  const int chunk = 2 * kk + (lane >> 5);
  return r * 128 + ((chunk ^ ((r >> 1) & 7)) << 4);
}

// Column-contiguous rows (K outermost): BK rows x (C * 2) bytes per stage.
template <int C>
struct MnGeom {
  static_assert(C == 128 || C == 256, "column tile");
  static constexpr int ROW_BYTES = C * 2;
  static constexpr int SLOTS = ROW_BYTES / 16;      // 16-byte chunks per row
  static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;
  static constexpr int STAGE_BYTES = BK * ROW_BYTES;
  static __device__ __forceinline__ int swz(int k) { return 4 * (k & 3); }
  // Fragment of the 32 columns starting at cb, K step kk (16 rows), half h (rows
  // 4h..4h+3 of the lane's 8): byte offset of this lane's ds_read_b64_tr_b16.
  static __device__ __forceinline__ int tr_offset(int lane, int cb, int kk, int h) {
    const int g = lane >> 4, s = lane & 15;
    const int k = 16 * kk + 8 * (g >> 1) + 4 * h + (s >> 2);
    const int col = cb + 16 * (g & 1) + 4 * (s & 3);
    return k * ROW_BYTES + (((col >> 3) ^ swz(k)) << 4) + ((col & 7) << 1);
  }
};

__device__ __forceinline__ bf16x8 tr_frag(const char* stage, int off0, int off1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage + off0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage + off1));
  const short v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ---- dgrad ------------------------------------------------------------------------
enum DgradEpi { kDgradPlain = 0, kDgradSwiglu = 1 };

struct DgradArgs {
  Side a;                    // [rows][K], K contiguous
  const uint16_t* B;         // [E][K][N]
  int64_t b_expert_stride;
  uint16_t* C[2];            // plain: [rows][N] (split when c_split)
  int c_split;
  uint16_t* gu;              // swiglu: [rows][2I] joint, g then u; overwritten with grads
  const int32_t* off0;
  const int32_t* off1;
  int E, K, N, I, n_tiles;
};

template <int kEpi, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N) dgrad_gemm_bf16(DgradArgs a) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  using GB = MnGeom<BN>;
  constexpr int A_BYTES = BM * 128;
  constexpr int STAGE = A_BYTES + GB::STAGE_BYTES;
  constexpr int LA = BM / 8 / NW;                        // 1 KB A blocks per wave
  constexpr int LB = GB::STAGE_BYTES / 1024 / NW;        // 1 KB B blocks per wave
  static_assert(LA * 8 * NW == BM && LB * 1024 * NW == GB::STAGE_BYTES, "blocks per wave");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  MTileMap tm;
  tm.build(a.off0, a.off1, a.E, BM, BM);
  int mt, nt;
  if (!xcd_tile(tm, a.n_tiles, &mt, &nt)) return;
  const TileRows tr = tm.locate(a.off0, a.off1, BM, mt);

  // A: lane l of block b holds tile row 8b + l/8, 16-byte slot l % 8
  const char* a_src[LA];
  int live_a = 0;
  const SideU a_u = uniform_side(a.a);
#pragma unroll
  for (int t = 0; t < LA; ++t) {
    const int row = (wave * LA + t) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    const int r = row < tr.rows ? row : tr.rows - 1;
    a_src[t] = (const char*)side_addr(a_u, tr, tr.v0 + r, chunk * 8);
    live_a += (wave * LA + t) * 8 < tr.rows ? 1 : 0;
  }
  // B: lane l of block b holds K row ROWS_PER_KB*b + l/SLOTS, slot l % SLOTS
  const uint16_t* Be = a.B + (int64_t)tr.e * a.b_expert_stride;
  const char* b_src[LB];
#pragma unroll
  for (int t = 0; t < LB; ++t) {
    const int k = (wave * LB + t) * GB::ROWS_PER_KB + lane / GB::SLOTS;
    const int slot = lane % GB::SLOTS;
    int col = nt * BN + 8 * (slot ^ GB::swz(k));
    if (col > a.N - 8) col = a.N - 8;
    b_src[t] = (const char*)(Be + (int64_t)k * a.N + col);
  }
  // a weight panel that only this tile reads (its expert has one m-tile) is
  // streamed with the non-temporal cache policy, as in the forward
  const bool nt_b = __builtin_amdgcn_readfirstlane(tr.single) != 0;
  auto issue = [&](int kt, int buf) {
    char* base = smem + buf * STAGE;
#pragma unroll
    for (int t = 0; t < LA; ++t)
      if (t < live_a)
        __builtin_amdgcn_global_load_lds((const void*)(a_src[t] + (int64_t)kt * 128),
                                         (lds_void*)(base + (wave * LA + t) * 1024), 16, 0, 0);
    if (nt_b) {
#pragma unroll
      for (int t = 0; t < LB; ++t)
        __builtin_amdgcn_global_load_lds((const void*)(b_src[t] + (int64_t)kt * BK * a.N * 2),
                                         (lds_void*)(base + A_BYTES + (wave * LB + t) * 1024), 16,
                                         0, 2);
    } else {
#pragma unroll
      for (int t = 0; t < LB; ++t)
        __builtin_amdgcn_global_load_lds((const void*)(b_src[t] + (int64_t)kt * BK * a.N * 2),
                                         (lds_void*)(base + A_BYTES + (wave * LB + t) * 1024), 16,
                                         0, 0);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  const int KT = a.K / BK;
  // F (<= FM) 32-row blocks of the wave's band take part in the MFMAs; the
  // loop body holds no branch (as in the forward grouped GEMM)
  auto k_loop = [&](auto f_const) {
    constexpr int F = decltype(f_const)::value;
    issue(0, 0);
    for (int kt = 0; kt < KT; ++kt) {
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      __builtin_amdgcn_s_barrier();
      if (kt + 1 < KT) issue(kt + 1, (kt + 1) & 1);
      const char* sa = smem + (kt & 1) * STAGE;
      const char* sb = sa + A_BYTES;
      if constexpr (F > 0) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const int fo = kfrag_offset(lane, kk);
          bf16x8 af[F], bfr[FN];
#pragma unroll
          for (int i = 0; i < F; ++i)
            af[i] = *(const bf16x8*)(sa + (wm * WM + i * 32) * 128 + fo);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int cb = wn * WN + j * 32;
            bfr[j] = tr_frag(sb, GB::tr_offset(lane, cb, kk, 0), GB::tr_offset(lane, cb, kk, 1));
          }
#pragma unroll
          for (int i = 0; i < F; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i][j] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    }
  };
  const int band_rows = tr.rows - wm * WM;
  const int fm_live = band_rows <= 0 ? 0 : (band_rows + 31) / 32;
  static_assert(FM == 4, "band dispatch below assumes four 32-row blocks per wave");
  if (fm_live > 2)
    k_loop(std::integral_constant<int, FM>{});
  else if (fm_live == 2)
    k_loop(std::integral_constant<int, 2>{});
  else if (fm_live == 1)
    k_loop(std::integral_constant<int, 1>{});
  else
    k_loop(std::integral_constant<int, 0>{});

  // epilogue: lane l holds column l % 32 of rows 8(q/4) + 4(l/32) + q%4 of each block
  const int rbase = wm * WM + 4 * (lane >> 5);
  if constexpr (kEpi == kDgradSwiglu) {
    // g and u of the tile's rows go through the freed stage buffers, one wave
    // row (WM tile rows) per pass: read and written back as 16-byte row
    // segments, the gradients computed in place in LDS by the wave row that
    // holds those rows.  Chunk ch of row r at ch ^ 4((r/4) mod 2), as in the
    // forward epilogue.
    static_assert(WAVES_M == 2 && 2 * WM * BN * 2 <= 2 * STAGE && BN / 8 >= 8,
                  "g and u of one wave row in the stage buffers");
    constexpr int CPR = BN / 8;  // 16-byte chunks per row
    char* lg = smem;
    char* lu = smem + WM * BN * 2;
    auto at = [](int r, int c) {
      return r * (BN * 2) + (((c >> 3) ^ (((r >> 2) & 1) << 2)) << 4) + (c & 7) * 2;
    };
#pragma unroll
    for (int h = 0; h < WAVES_M; ++h) {
      __syncthreads();  // the stage buffers (or the previous pass) are free
      for (int ch = threadIdx.x; ch < WM * CPR; ch += blockDim.x) {
        const int r = ch / CPR, c = (ch % CPR) * 8;
        const int row = h * WM + r, col = nt * BN + c;
        if (row >= tr.rows || col >= a.N) continue;
        const uint16_t* gr = a.gu + (int64_t)tr.joint_row(tr.v0 + row) * (2 * a.I);
        *(uint4*)(lg + at(r, c)) = *(const uint4*)(gr + col);
        *(uint4*)(lu + at(r, c)) = *(const uint4*)(gr + a.I + col);
      }
      __syncthreads();
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (h * WM + i * 32 >= tr.rows) break;  // rows past the tile: never stored
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = 4 * (lane >> 5) + i * 32 + 8 * (q >> 2) + (q & 3);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int c = wn * WN + j * 32 + (lane & 31);
              uint16_t* pg = (uint16_t*)(lg + at(r, c));
              uint16_t* pu = (uint16_t*)(lu + at(r, c));
              const float ga = acc[i][j][q];
              const float g = bf16_to_f32(*pg), u = bf16_to_f32(*pu);
              const float sg = 1.0f / (1.0f + expf(-g));
              *pg = to_bf16_bits(ga * u * (sg + g * sg * (1.0f - sg)));
              *pu = to_bf16_bits(ga * (g * sg));
            }
          }
        }
      }
      __syncthreads();
      for (int ch = threadIdx.x; ch < WM * CPR; ch += blockDim.x) {
        const int r = ch / CPR, c = (ch % CPR) * 8;
        const int row = h * WM + r, col = nt * BN + c;
        if (row >= tr.rows || col >= a.N) continue;
        uint16_t* gr = a.gu + (int64_t)tr.joint_row(tr.v0 + row) * (2 * a.I);
        *(uint4*)(gr + col) = *(const uint4*)(lg + at(r, c));
        *(uint4*)(gr + a.I + col) = *(const uint4*)(lu + at(r, c));
      }
    }
    return;
  }
  // plain: the C tile goes through the freed stage buffers as row-major bf16
  // (chunk ch of row r at ch ^ 4((r/4) mod 2), so the rows r and r + 4 of one
  // 2-byte write fall in different banks), then out as 16-byte row segments
  static_assert(BM * BN * 2 <= 2 * STAGE && BN / 8 >= 8, "C tile in the stage buffers");
  constexpr int CPR = BN / 8;
  auto lds_at = [](int r, int c) {
    return r * (BN * 2) + (((c >> 3) ^ (((r >> 2) & 1) << 2)) << 4) + (c & 7) * 2;
  };
  __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (wm * WM + i * 32 >= tr.rows) break;  // blocks past the tile's rows: never stored
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = rbase + i * 32 + 8 * (q >> 2) + (q & 3);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int c = wn * WN + j * 32 + (lane & 31);
        *(uint16_t*)(smem + lds_at(r, c)) = to_bf16_bits(acc[i][j][q]);
      }
    }
  }
  __syncthreads();
  const SideU c_u = uniform_side(Side{{a.C[0], a.C[1]}, a.c_split, a.N});
  for (int ch = threadIdx.x; ch < BM * CPR; ch += blockDim.x) {
    const int r = ch / CPR, c = (ch % CPR) * 8;
    if (r >= tr.rows || nt * BN + c >= a.N) continue;
    const uint4 v = *(const uint4*)(smem + lds_at(r, c));
    *(uint4*)side_addr(c_u, tr, tr.v0 + r, nt * BN + c) = v;
  }
}

// ---- wgrad ------------------------------------------------------------------------
struct WgradArgs {
  Side a;            // [rows][M]
  Side b;            // [rows][N]
  float* C;          // [E][M][N]
  const int32_t* off0;
  const int32_t* off1;
  int E, M, N, m_tiles, n_tiles;
  int accumulate;    // 0: C = sum (experts without rows get zeros); 1: C += sum
  const int32_t* order;  // nullable: experts in dealing order (largest first)
};

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N) wgrad_gemm_bf16(WgradArgs a) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  using GA = MnGeom<BM>;
  using GB = MnGeom<BN>;
  constexpr int STAGE = GA::STAGE_BYTES + GB::STAGE_BYTES;
  constexpr int LA = GA::STAGE_BYTES / 1024 / NW, LB = GB::STAGE_BYTES / 1024 / NW;
  static_assert(LA * 1024 * NW == GA::STAGE_BYTES && LB * 1024 * NW == GB::STAGE_BYTES,
                "blocks per wave");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  int emt, nt;
  if (!xcd_tile_rr(a.E * a.m_tiles, a.n_tiles, &emt, &nt)) return;
  // tiles are dealt expert by expert, largest expert first when an order is
  // given (the longest reductions start first, which shortens the tail)
  const int rank = emt / a.m_tiles, mt = emt - rank * a.m_tiles;
  const int e = a.order ? a.order[rank] : rank;
  TileRows tr;
  tr.e = e;
  tr.v0 = 0;
  tr.lo0 = a.off0[e];
  tr.n0 = a.off0[e + 1] - tr.lo0;
  tr.lo1 = a.off1 ? a.off1[e] : 0;
  const int n1 = a.off1 ? a.off1[e + 1] - tr.lo1 : 0;
  const int rows = tr.n0 + n1;
  tr.rows = rows;
  if (rows == 0 && a.accumulate) return;

  // per lane: the K row (within a stage) and column of each 1 KB block it loads
  int a_k[LA], a_col[LA], b_k[LB], b_col[LB];
#pragma unroll
  for (int t = 0; t < LA; ++t) {
    a_k[t] = (wave * LA + t) * GA::ROWS_PER_KB + lane / GA::SLOTS;
    int col = mt * BM + 8 * ((lane % GA::SLOTS) ^ GA::swz(a_k[t]));
    a_col[t] = col > a.M - 8 ? a.M - 8 : col;
  }
#pragma unroll
  for (int t = 0; t < LB; ++t) {
    b_k[t] = (wave * LB + t) * GB::ROWS_PER_KB + lane / GB::SLOTS;
    int col = nt * BN + 8 * ((lane % GB::SLOTS) ^ GB::swz(b_k[t]));
    b_col[t] = col > a.N - 8 ? a.N - 8 : col;
  }
  const SideU sa_u = uniform_side(a.a), sb_u = uniform_side(a.b);
  auto issue = [&](int kt, int buf) {
    char* base = smem + buf * STAGE;
#pragma unroll
    for (int t = 0; t < LA; ++t) {
      int v = kt * BK + a_k[t];
      v = v < rows ? v : rows - 1;
      __builtin_amdgcn_global_load_lds((const void*)side_addr(sa_u, tr, v, a_col[t]),
                                       (lds_void*)(base + (wave * LA + t) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < LB; ++t) {
      int v = kt * BK + b_k[t];
      v = v < rows ? v : rows - 1;
      __builtin_amdgcn_global_load_lds((const void*)side_addr(sb_u, tr, v, b_col[t]),
                                       (lds_void*)(base + GA::STAGE_BYTES + (wave * LB + t) * 1024),
                                       16, 0, 0);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  const int KT = (rows + BK - 1) / BK;
  const int KF = rows / BK;  // stages whose BK rows all exist
  if (KT > 0) issue(0, 0);
  const int g = lane >> 4;
  // one stage; kTail: the last, partial stage (K rows past the expert's block
  // are zeroed in the A fragments).  Full stages run a body without branches.
  auto stage = [&](int kt, auto tail_const) {
    constexpr bool kTail = decltype(tail_const)::value;
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    __builtin_amdgcn_s_barrier();
    if (kt + 1 < KT) issue(kt + 1, (kt + 1) & 1);
    const char* sa = smem + (kt & 1) * STAGE;
    const char* sb = sa + GA::STAGE_BYTES;
    const int kvalid = rows - kt * BK;  // K rows of this stage that exist
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if constexpr (kTail) {
        if (16 * kk >= kvalid) break;
      }
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int cb = wm * WM + i * 32;
        af[i] = tr_frag(sa, GA::tr_offset(lane, cb, kk, 0), GA::tr_offset(lane, cb, kk, 1));
      }
      if constexpr (kTail) {
        if (16 * kk + 16 > kvalid) {
          // element j of half h is K row 16kk + 8(g/2) + 4h + j: zero rows past the block
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int x = 0; x < 8; ++x)
              if (16 * kk + 8 * (g >> 1) + x >= kvalid) af[i][x] = (__bf16)0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cb = wn * WN + j * 32;
        bfr[j] = tr_frag(sb, GB::tr_offset(lane, cb, kk, 0), GB::tr_offset(lane, cb, kk, 1));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  };
  for (int kt = 0; kt < KF; ++kt) stage(kt, std::false_type{});
  if (KF < KT) stage(KF, std::true_type{});

  // The fp32 C tile goes through the freed stage buffers in two passes of
  // WM rows (the two wave rows), row-major, and out as 16-byte row segments:
  // one global store (and, when accumulating, one load) per 4 elements
  // instead of per element.
  static_assert(WAVES_M == 2 && WM * BN * 4 <= 2 * STAGE, "half C tile in the stage buffers");
  constexpr int CPR = BN / 4;  // 16-byte chunks per row
  float* Ce = a.C + (int64_t)e * a.M * a.N;
  float* cl = (float*)smem;
  // the MFMAs above take the B fragment first, so each block holds C
  // transposed: lane l has row l % 32 and columns 8(q/4) + 4(l/32) + q%4, four
  // consecutive columns per group of q, written as one 16-byte LDS store.
  // 16-byte chunk ch of row r at slot ch ^ (r mod 32): the 32 rows of one
  // store fall in distinct slots.
  auto cl_at = [](int r, int c) { return r * BN + ((((c >> 2) ^ (r & 31))) << 2); };
  const int rq = lane & 31, cq = 4 * (lane >> 5);
#pragma unroll
  for (int h = 0; h < WAVES_M; ++h) {
    __syncthreads();  // the stage buffers (or the previous pass) are free
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const f32x16& x = acc[i][j];
            *(float4*)(cl + cl_at(i * 32 + rq, wn * WN + j * 32 + 8 * g4 + cq)) =
                make_float4(x[4 * g4], x[4 * g4 + 1], x[4 * g4 + 2], x[4 * g4 + 3]);
          }
    }
    __syncthreads();
    for (int ch = threadIdx.x; ch < WM * CPR; ch += blockDim.x) {
      const int r = ch / CPR, c = (ch % CPR) * 4;
      const int m = mt * BM + h * WM + r, n = nt * BN + c;
      if (m >= a.M || n >= a.N) continue;
      float4 v = *(const float4*)(cl + cl_at(r, c));
      float4* dst = (float4*)(Ce + (int64_t)m * a.N + n);
      if (a.accumulate) {
        const float4 old = *dst;
        v.x = old.x + v.x;
        v.y = old.y + v.y;
        v.z = old.z + v.z;
        v.w = old.w + v.w;
        *dst = v;
      } else {
        // written once here and read by nothing later in the layer: streamed
        // (backward 1.44 -> 1.36 ms on the Zipf bench workload with the dgrad
        // weight loads above, 22.4 -> 22.1 ms on the DeepSeek-V3-shaped one)
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(f32x4v{v.x, v.y, v.z, v.w}, (f32x4v*)dst);
      }
    }
  }
}

}  // namespace

hipError_t launch_dgrad_bf16(const Shape& s, const DgradIO& io, hipStream_t st) {
  if (io.rows_bound <= 0) return hipSuccess;
  DgradArgs a{};
  a.a.p[0] = (const uint16_t*)io.a[0];
  a.a.p[1] = (const uint16_t*)(io.a_split ? io.a[1] : io.a[0]);
  a.a.split = io.a_split && io.off[1];
  a.a.ld = io.K;
  a.B = (const uint16_t*)io.B;
  a.b_expert_stride = (int64_t)io.K * io.N;
  a.C[0] = (uint16_t*)io.c[0];
  a.C[1] = (uint16_t*)(io.c_split ? io.c[1] : io.c[0]);
  a.c_split = io.c_split && io.off[1];
  a.gu = (uint16_t*)io.gu;
  a.off0 = io.off[0];
  a.off1 = io.off[1];
  a.E = s.E;
  a.K = io.K;
  a.N = io.N;
  a.I = s.I;
  constexpr int BM = 256, BN = 256;
  a.n_tiles = (io.N + BN - 1) / BN;
  const int64_t grid = xcd_grid(m_tiles_bound(io.rows_bound, s.E, BM), a.n_tiles);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (io.gu)
    hipLaunchKernelGGL((dgrad_gemm_bf16<kDgradSwiglu, BM, BN, 2, 4>), dim3((unsigned)grid),
                       dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((dgrad_gemm_bf16<kDgradPlain, BM, BN, 2, 4>), dim3((unsigned)grid),
                       dim3(512), 0, st, a);
  return hipGetLastError();
}

namespace {

// order[rank] = expert: rank = number of experts with more rows, or as many
// rows and a lower id.  One thread per expert, the row counts staged in LDS.
__global__ void __launch_bounds__(1024) expert_order(const int32_t* __restrict__ off0,
                                                     const int32_t* __restrict__ off1, int E,
                                                     int32_t* __restrict__ order) {
  __shared__ int rows[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    rows[e] = off0[e + 1] - off0[e] + (off1 ? off1[e + 1] - off1[e] : 0);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int n = rows[e];
    int rank = 0;
    for (int f = 0; f < E; ++f) rank += (rows[f] > n || (rows[f] == n && f < e)) ? 1 : 0;
    order[rank] = e;
  }
}

}  // namespace

hipError_t launch_expert_order(const Shape& s, const int32_t* off0, const int32_t* off1,
                               int32_t* order, hipStream_t st) {
  if (s.E > kMaxExperts) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expert_order, dim3(1), dim3(1024), 0, st, off0, off1, s.E, order);
  return hipGetLastError();
}

hipError_t launch_wgrad_bf16(const Shape& s, const WgradIO& io, hipStream_t st) {
  WgradArgs a{};
  a.a.p[0] = (const uint16_t*)io.a[0];
  a.a.p[1] = (const uint16_t*)(io.a_split ? io.a[1] : io.a[0]);
  a.a.split = io.a_split && io.off[1];
  a.a.ld = io.M;
  a.b.p[0] = (const uint16_t*)io.b[0];
  a.b.p[1] = (const uint16_t*)(io.b_split ? io.b[1] : io.b[0]);
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
  constexpr int BM = 256, BN = 256;
  a.m_tiles = (io.M + BM - 1) / BM;
  a.n_tiles = (io.N + BN - 1) / BN;
  const int64_t grid = xcd_grid_rr((int64_t)s.E * a.m_tiles, a.n_tiles);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((wgrad_gemm_bf16<BM, BN, 2, 4>), dim3((unsigned)grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
