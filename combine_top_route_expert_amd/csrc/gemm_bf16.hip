// Grouped expert GEMMs on gfx950 bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// The expert computation of the MindSpeed Chunk MoE article (core principle /
// timing-diagram sections) is read as a SwiGLU FFN per expert; each expert
// multiplies its contiguous block of permuted rows:
//   gate_up: act[r][i] = silu(x_r . Wg[e][i]) * (x_r . Wu[e][i])   (K = H)
//   down   : y[r][n]   = act_r . Wd[e][n]                          (K = I)
// Both operands are K-contiguous ([rows][K] activations, [cols][K] weights).
//
// Pipeline: K advances 64 at a time.  Each stage of the A (rows) and B
// (weight) tiles is copied global -> LDS by the direct-to-LDS load
// (global_load_lds_dwordx4: 64 lanes x 16 bytes land as one contiguous 1 KB
// block), so loads need no VGPRs and STAGES-1 stages are in flight while the
// matrix cores work on the oldest one.  Completion is tracked with explicit
// vmcnt waits plus a plain s_barrier (no fence that would drain every load).
// Inside a 1 KB block lane l holds row l/8 and 16-byte slot l%8; the global
// chunk it fetches is slot ^ ((row >> 1) & 7), which makes the 16-byte fragment
// reads of 16 consecutive rows hit distinct LDS banks.
//
// Tiling: a workgroup computes BM x BN with WAVES_M x WAVES_N waves; each wave
// owns (BM/WAVES_M) x (BN/WAVES_N) as 16 x 16 MFMA blocks with fp32
// accumulators.  For gate_up half of every wave's columns are gate columns and
// the other half the matching up columns, so each lane holds the gate and up
// accumulators of the same (row, i) and SwiGLU runs in registers: no
// [rows][2I] intermediate is written.
//
// Grouping: m-tiles of all experts are numbered expert by expert; every
// workgroup finds its expert from the device-resident offsets (find_m_tile),
// so the host never reads group sizes.  The grid is bounded from the chunk's
// assignment count and surplus workgroups exit.  Rows past an expert's block
// are loaded from a clamped row and never stored.  Two workgroups per CU (or
// eight waves in one) let one wave's barrier and LDS-read bubbles hide behind
// another's MFMAs; a persistent variant with deeper prefetch measured slower.
//
// Instances: a wide 256 x 256 tile with 8 waves for experts with many rows, a
// 128 x 128 tile (two workgroups per CU) for medium blocks and a 64 x 128 tile
// for decode-sized blocks, picked from the average rows per expert.  All use
// the same MFMA instruction and the same order of K steps, so a row gets the
// same bits from any instance or chunking.
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 64;             // K elements per stage
constexpr int ROW_BYTES = BK * 2;  // bytes of one tile row per stage

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14])
constexpr int wait_vm(int v) { return (v & 0xF) | ((v >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

struct GemmArgs {
  const uint16_t* A;          // [rows][K] bf16
  const uint16_t* B;          // [E][b_rows][K] bf16
  uint16_t* C;                // [rows][ncols] bf16
  const int32_t* off;         // E + 1 offsets of this chunk
  int E, K, I, ncols, n_tiles;
  int64_t b_expert_stride;    // elements per expert in B
};

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <bool kGateUp, int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N) grouped_gemm_bf16(GemmArgs a) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int LA = BM / 8 / NW, LB = BN / 8 / NW;  // 1 KB loads per wave per stage
  constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile rows per wave");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");
  static_assert(!kGateUp || WN % 32 == 0, "gate/up halves");
  static_assert(STAGES >= 2, "pipeline depth");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int nt = blockIdx.x % a.n_tiles;
  const int mt = blockIdx.x / a.n_tiles;
  int e, m0, mrows;
  if (!find_m_tile(a.off, a.E, BM, mt, &e, &m0, &mrows)) return;

  // Per-lane source of every direct-to-LDS load (at k = 0).
  const int brow_in_blk = lane >> 3, slot = lane & 7;
  const char* a_src[LA];
  const char* b_src[LB];
#pragma unroll
  for (int t = 0; t < LA; ++t) {
    const int row = (wave * LA + t) * 8 + brow_in_blk;
    const int chunk = slot ^ ((row >> 1) & 7);
    const int r = row < mrows ? row : mrows - 1;
    a_src[t] = (const char*)(a.A + (int64_t)(m0 + r) * a.K + chunk * 8);
  }
  const uint16_t* Be = a.B + (int64_t)e * a.b_expert_stride;
#pragma unroll
  for (int t = 0; t < LB; ++t) {
    const int col = (wave * LB + t) * 8 + brow_in_blk;  // tile column = B row
    const int chunk = slot ^ ((col >> 1) & 7);
    int brow;
    if constexpr (kGateUp) {
      const int cw = col / WN, w = col % WN;
      const int q = w / (WN / 2), c = w % (WN / 2);
      brow = q * a.I + nt * (BN / 2) + cw * (WN / 2) + c;
    } else {
      brow = nt * BN + col;
      if (brow > a.ncols - 1) brow = a.ncols - 1;
    }
    b_src[t] = (const char*)(Be + (int64_t)brow * a.K + chunk * 8);
  }

  auto issue = [&](int kt, int buf) {
    char* base = smem + buf * STAGE_BYTES;
    const int64_t koff = (int64_t)kt * ROW_BYTES;
#pragma unroll
    for (int t = 0; t < LA; ++t)
      __builtin_amdgcn_global_load_lds((const void*)(a_src[t] + koff),
                                       (lds_void*)(base + (wave * LA + t) * 1024), 16, 0, 0);
#pragma unroll
    for (int t = 0; t < LB; ++t)
      __builtin_amdgcn_global_load_lds(
          (const void*)(b_src[t] + koff),
          (lds_void*)(base + BM * ROW_BYTES + (wave * LB + t) * 1024), 16, 0, 0);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment read offset: row (lane & 15), 16-byte chunk (lane >> 4) (+4 for k 32..63)
  const int frag0 = (lane & 15) * ROW_BYTES + (((lane >> 4) ^ ((lane & 15) >> 1)) << 4);
  const int KT = a.K / BK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s, s);

  for (int kt = 0; kt < KT; ++kt) {
    // stage kt has landed once at most STAGES-2 newer stages are still in flight
    if (kt + STAGES - 2 < KT)
      __builtin_amdgcn_s_waitcnt(wait_vm((LA + LB) * (STAGES - 2)));
    else
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    const char* sa = smem + (kt % STAGES) * STAGE_BYTES;
    const char* sb = sa + BM * ROW_BYTES;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int fo = kk ? (frag0 ^ 64) : frag0;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const bf16x8*)(sa + (wm * WM + i * 16) * ROW_BYTES + fo);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *(const bf16x8*)(sb + (wn * WN + j * 16) * ROW_BYTES + fo);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    // this stage's LDS reads are complete before any wave refills its buffer
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }

  // Epilogue.  MFMA 16x16 output: lane holds column (lane & 15) of rows
  // 4 * (lane >> 4) + 0..3 of each 16 x 16 block.
  const int rbase = wm * WM + (lane >> 4) * 4;
  if constexpr (kGateUp) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const int col = nt * (BN / 2) + wn * (WN / 2) + j * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          if (row < mrows) {
            const float g = acc[i][j][r], u = acc[i][j + FN / 2][r];
            const float act = g / (1.0f + expf(-g)) * u;
            a.C[(int64_t)(m0 + row) * a.ncols + col] = to_bf16_bits(act);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = nt * BN + wn * WN + j * 16 + (lane & 15);
        if (col >= a.ncols) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          if (row < mrows) a.C[(int64_t)(m0 + row) * a.ncols + col] = to_bf16_bits(acc[i][j][r]);
        }
      }
  }
}

// Tile instances.  All use the same MFMA instruction and the same order of
// K steps, so any instance gives the same bits for a row; the choice only
// affects speed.
enum Instance { kWide = 1, kMid = 2, kNarrow = 3 };
#ifndef MOE_GEMM_FORCE
#define MOE_GEMM_FORCE 0
#endif
#ifndef MOE_GEMM_MID_STAGES
#define MOE_GEMM_MID_STAGES 2
#endif

// Average rows per expert decides the tile: long blocks of rows amortise each
// weight panel over a 256-row tile, short ones waste less of a 64-row tile.
int choose_instance(int64_t rows_bound, int E) {
  if (MOE_GEMM_FORCE) return MOE_GEMM_FORCE;
  const int64_t avg = rows_bound / (E > 0 ? E : 1);
  if (avg >= 512) return kWide;
  if (avg >= 24) return kMid;
  return kNarrow;
}

template <bool kGateUp, int BM, int BN, int WM_, int WN_, int ST>
hipError_t launch_instance(const GemmArgs& a, int64_t rows_bound, int E, hipStream_t st) {
  constexpr int threads = 64 * WM_ * WN_;
  const int64_t grid = m_tiles_bound(rows_bound, E, BM) * a.n_tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((grouped_gemm_bf16<kGateUp, BM, BN, WM_, WN_, ST>), dim3((unsigned)grid),
                     dim3(threads), 0, st, a);
  return hipGetLastError();
}

template <bool kGateUp>
hipError_t launch_kind(int inst, GemmArgs a, const Shape& s, int64_t rows_bound, hipStream_t st) {
  // n-tiles of the chosen instance; gate_up tiles cover BN/2 intermediate columns
  auto ntiles = [&](int BN) {
    return kGateUp ? s.I / (BN / 2) : (s.H + BN - 1) / BN;
  };
  if (kGateUp && inst == kWide && s.I % 128) inst = kMid;
  switch (inst) {
    case kWide:
      a.n_tiles = ntiles(256);
      return launch_instance<kGateUp, 256, 256, 2, 4, 2>(a, rows_bound, s.E, st);
    case kNarrow:
      a.n_tiles = ntiles(128);
      return launch_instance<kGateUp, 64, 128, 1, 4, 4>(a, rows_bound, s.E, st);
    default:
      a.n_tiles = ntiles(128);
      return launch_instance<kGateUp, 128, 128, 2, 2, MOE_GEMM_MID_STAGES>(a, rows_bound, s.E, st);
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
  const int inst = choose_instance(rows_bound, s.E);
  if (gate_up) {
    a.K = s.H;
    a.ncols = s.I;
    a.b_expert_stride = (int64_t)2 * s.I * s.H;
    return launch_kind<true>(inst, a, s, rows_bound, st);
  }
  a.K = s.I;
  a.ncols = s.H;
  a.b_expert_stride = (int64_t)s.H * s.I;
  return launch_kind<false>(inst, a, s, rows_bound, st);
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
