// Grouped expert GEMMs on gfx950 bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The expert computation of the MindSpeed Chunk MoE article (core principle /
// timing-diagram sections) is read as a SwiGLU FFN per expert; each expert
// multiplies its block of permuted rows:
//   gate_up: act[r][i] = silu(x_r . Wg[e][i]) * (x_r . Wu[e][i])   (K = H)
//   down   : y[r][n]   = act_r . Wd[e][n]                          (K = I)
// Both operands are K-contiguous ([rows][K] activations, [cols][K] weights).
// One launch covers one chunk or both chunks of a pair (GroupedIO): an
// expert's rows are its rows in the first chunk followed by its rows in the
// second, so its weights are streamed once per launch.  gate_up may read its
// rows straight from hidden_states through src_row (GroupedIO::gather): the
// permute fused into the A loader's addresses.
//
// Pipeline: K advances BK (64) at a time.  Each stage of the A (rows) and B
// (weight) tiles is copied HBM -> LDS by the direct-to-LDS load (64 lanes x 16
// bytes land as one contiguous 1 KB block), so loads need no VGPRs and
// STAGES-1 stages are in flight while the matrix cores work on the oldest one
// (the wide 256 x 256 kernel: two A stages and three B stages, k_loop_roles).
// The buffer form of that load (a descriptor per operand, 32-bit offsets) is
// used whenever the rows fit a 4 GiB window: with the global form, a FLAT
// instruction, in flight, the compiler drains every LDS read before each MFMA
// group; with descriptors it waits only for the fragments in use, and each
// 16-deep sub-step's fragment reads overlap the previous sub-step's MFMAs
// (gate/up 4-6% faster on the MFMA-bound workloads).  Completion is tracked
// with explicit vmcnt waits plus a plain s_barrier (no fence that would drain
// every load).  LDS rows are XOR-swizzled (StageGeom) so that 16-byte fragment
// reads are free of bank conflicts (measured).
//
// Matrix instruction: on gfx950 v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_16x16x32_bf16 both occupy the matrix pipe for about 32 cycles, so
// only the 32x32x16 form reaches the chip's dense bf16 peak (measured 2.47
// versus 1.26 PFLOP/s with back-to-back independent MFMAs); every tile here is
// built from 32 x 32 blocks.
//
// Tiling: a workgroup computes BM x BN with WAVES_M x WAVES_N waves; each wave
// owns (BM/WAVES_M) x (BN/WAVES_N) as 32 x 32 MFMA blocks with fp32
// accumulators.  For gate_up half of every wave's columns are gate columns and
// the other half the matching up columns, so each lane holds the gate and up
// accumulators of the same (row, i) and SwiGLU runs in registers: no
// [rows][2I] intermediate is written.
//
// Grouping: every workgroup numbers the m-tiles of all experts from the
// device-resident offsets (MTileMap: the large experts' m-tiles first, then
// the small experts' by size class), so the host never reads group sizes.
// Each XCD takes a contiguous range of the large experts' m-tiles and an even
// share of the small ones, interleaved, each with all its n-tiles (xcd_tile).
// The grid is bounded from the launch's assignment count and surplus
// workgroups exit.  Rows past an expert's block are loaded from a clamped row
// (A blocks wholly past it are not loaded at all) and never stored.
//
// Epilogue: the accumulators go through the freed stage buffers as a
// row-major bf16 tile and leave as 16-byte row segments (store_tile_lds).
//
// Small tiles: an m-tile of at most 32, 64, 128 or 160 rows (a small expert's
// only tile) has little MFMA work and is bound by streaming its weight panel, so
// it runs a K loop with a compact stage layout (its rows of A, then B) and three
// stages, two in flight (k_loop_small): 41 -> 33 us per gate/up tile of at most
// 32 rows on the Zipf workload; the 160-row case (three 52 KB stages, 156 KB of
// LDS) took the DeepSeek-V3-shaped layer, whose experts hold 95-160 rows, from
// 4.89 to 4.79 ms (down 1724 -> 1683 us).  When such a tile holds all of its
// expert's rows its 32-row blocks are split between the two wave rows
// (compact_f0 / compact_f1), so that both waves on each SIMD run MFMAs.
//
// Also measured and dropped, on these launches: a persistent form (one
// workgroup per CU taking its XCD's tiles in sequence, the next tile's first
// stages loaded during the current tile's last steps), for weight-streaming
// and for MFMA-bound launches; two workgroups per CU with 32-deep stages; K
// stages rotated per expert.  The hardware's dynamic dispatch of one-tile
// workgroups balances the tiles better than any fixed sequence per CU.
//
// What bounds it (measured with per-workgroup timestamps): the MFMA loop alone
// (no global loads) runs at ~94% of the matrix peak at the clock it gets, and
// adding the LDS fragment reads costs nothing.  With the operand streaming on
// top, the chip's power management lowers the shader clock (about 2.2 GHz ->
// 1.5-2.1 GHz) and a full 256 x 256 tile takes ~1.45x the cycles of its MFMAs.
// Per-K-step timestamps place the loss at the start of each step: a load
// instruction holds its wave until the texture unit takes it, so while the
// eight waves issued a 64 KB stage no MFMA ran for 800-1150 of ~3300 cycles.
// The wide 256 x 256 kernel therefore gives the two waves of a SIMD different
// load roles (k_loop_roles, with a third weight buffer): 3280 -> 2875 cycles
// per step, of which the power limit returns part as a lower clock (layer
// 2-3% faster on packed16k, the Zipf workload and, in the tile-loop form, the
// two-expert skew; same bits).  Alone, a third
// weight buffer, loads spread over the sub-steps, one wave row issuing every
// load, BK 32 with 4-5 stages, a 256 x 128 tile with three stages,
// register-staged loads, round-robin XCD dealing of all m-tiles and 4-wave
// 128 x 128 wave tiles all measured no faster.  What did help besides: a K
// loop whose body holds no branch, with the wave's count of live 32-row blocks
// chosen once before the loop (5-12% on the larger workloads); the
// size-balanced, interleaved tile order (xcd_tile); the staged epilogue; the
// compact small-tile loop.
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14])
constexpr int wait_vm(int v) { return (v & 0xF) | ((v >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

struct GemmArgs {
  const uint16_t* A[2];       // [rows][K] bf16 (A[1]: chunk-1 rows when a_split)
  const uint16_t* B;          // [E][b_rows][K] bf16
  uint16_t* C[2];             // [rows][ncols] bf16 (C[1]: chunk-1 rows when c_split)
  const int32_t* off0;        // E + 1 offsets of the (first) chunk
  const int32_t* off1;        // E + 1 offsets of the pair's second chunk, or null
  int a_split, c_split;
  int E, K, I, ncols, n_tiles;
  int64_t b_expert_stride;    // elements per expert in B
  uint16_t* gu;               // gate_up, optional: g and u of each row, joint [rows][2I]
  const int32_t* gather[2];   // optional: A rows gathered from hidden_states (src_row slices)
  int gather_k;
  const char* a_base;         // descriptor loads: every A row lies within 4 GiB above it
};


// Address of virtual row v of the tile's expert on one side of the product.
__device__ __forceinline__ const uint16_t* row_ptr(const uint16_t* const (&base)[2], int split,
                                                   const TileRows& tr, int v, int64_t ld) {
  if (split) {
    int part;
    const int r = tr.split_row(v, &part);
    return (part ? base[1] : base[0]) + (int64_t)r * ld;
  }
  return base[0] + (int64_t)tr.joint_row(v) * ld;
}

constexpr int cmax(int x, int y) { return x > y ? x : y; }

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// SwiGLU of one gate/up pair: silu(g) * u = g / (1 + e^-g) * u, with the
// hardware base-2 exponential (__expf) and reciprocal (v_rcp_f32): relative
// error about 1e-7 * (1 + |g|), far below the bf16 rounding of the result.
// e^-g overflowing to infinity gives g * 0 = 0, the limit.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// LDS layout of one stage: BM rows of A then BN rows of B, each row BK bf16
// (ROW_BYTES) holding CH 16-byte chunks; chunk c of row r sits at slot
// c ^ swz(r).  A 16-lane phase of a 16-byte fragment read covers 16
// consecutive rows at one chunk; rows r and r + RB share a position in a
// 256-byte bank line, so swz(r) = (r / RB) mod CH spreads the 16 rows over 16
// distinct 16-byte bank groups (measured: no bank conflicts).
template <int BK>
struct StageGeom {
  static constexpr int ROW_BYTES = BK * 2;
  static constexpr int CH = BK / 8;               // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROW_BYTES;     // rows per 1 KB direct-to-LDS block
  static constexpr int RB = 256 / ROW_BYTES;       // rows per 256-byte bank line
  static_assert(BK == 32 || BK == 64, "stage depth");
  static __device__ __forceinline__ int swz(int r) { return (r / RB) & (CH - 1); }
  // 32x32x16 fragment of a 32-row block: lane l holds row l % 32 and the eight
  // K elements of 16-byte chunk 2*kk + l/32 of the stage.
  static __device__ __forceinline__ int frag_offset(int lane, int kk) {
    const int r = lane & 31;
    const int chunk = 2 * kk + (lane >> 5);
    return r * ROW_BYTES + ((chunk ^ swz(r)) << 4);
  }
};

// Everything a workgroup needs to stream its tile's A and B stages into LDS.
//
// kBuf: the stages are copied with the buffer form of the direct-to-LDS load
// (a descriptor per operand, 32-bit byte offsets per lane) instead of the
// global form.  Same bytes, same LDS layout; but the global form is a FLAT
// instruction, and while one is outstanding the compiler cannot count LDS
// reads in order, so every wait for a fragment read drains all of them.  With
// descriptor loads the K loop waits only for the fragments it is about to use,
// and the next sub-step's reads overlap the current MFMAs.  The host picks the
// global form when the A rows do not fit one 4 GiB window.
template <bool kGateUp, int BM, int BN, int NW, int WN, int BK, bool kBuf>
struct TileLoader {
  using G = StageGeom<BK>;
  static constexpr int LA = BM / G::RPB / NW, LB = BN / G::RPB / NW;  // 1 KB loads per wave
  static constexpr int STAGE_BYTES = (BM + BN) * G::ROW_BYTES;
  static_assert(LA * G::RPB * NW == BM && LB * G::RPB * NW == BN, "tile rows per wave");
  const char* a_src[LA];
  const char* b_src[LB];
  uint32_t a_off[LA], b_off[LB];  // kBuf: byte offsets from the descriptors' bases
  rsrc_t ra, rb;
  int wave, mrows;
  int live_a;  // A blocks of this wave that hold rows of the tile (the rest are skipped)

  __device__ __forceinline__ void init(const GemmArgs& a, const TileRows& tr, int nt, int lane,
                                       int wave_) {
    wave = wave_;
    mrows = tr.rows;
    const int row_in_blk = lane / G::CH, slot = lane % G::CH;
    live_a = 0;
    int rr[LA], ch[LA];
#pragma unroll
    for (int t = 0; t < LA; ++t) {
      const int row = (wave * LA + t) * G::RPB + row_in_blk;
      ch[t] = slot ^ G::swz(row);
      rr[t] = row < mrows ? row : mrows - 1;
      live_a += (wave * LA + t) * G::RPB < mrows ? 1 : 0;
    }
    if (a.gather[0]) {
      // permute fused into the row addressing: chunk row -> token (the LA
      // lookups are issued together and waited for once)
      int src[LA];
#pragma unroll
      for (int t = 0; t < LA; ++t) {
        int part;
        const int cr = tr.split_row(tr.v0 + rr[t], &part);
        src[t] = (part ? a.gather[1] : a.gather[0])[cr];
      }
#pragma unroll
      for (int t = 0; t < LA; ++t)
        a_src[t] = (const char*)(a.A[0] + (int64_t)(src[t] / a.gather_k) * a.K + ch[t] * 8);
    } else {
#pragma unroll
      for (int t = 0; t < LA; ++t)
        a_src[t] = (const char*)(row_ptr(a.A, a.a_split, tr, tr.v0 + rr[t], a.K) + ch[t] * 8);
    }
    // the expert is the same for the whole workgroup: keep its base scalar
    const int e = __builtin_amdgcn_readfirstlane(tr.e);
    const uint16_t* Be = a.B + (int64_t)e * a.b_expert_stride;
#pragma unroll
    for (int t = 0; t < LB; ++t) {
      const int col = (wave * LB + t) * G::RPB + row_in_blk;  // tile column = B row
      const int chunk = slot ^ G::swz(col);
      int brow;
      if constexpr (kGateUp) {
        // each wave's WN columns: gate for the first half, the matching up rows after
        const int cw = col / WN, w = col % WN;
        const int q = w / (WN / 2), c = w % (WN / 2);
        brow = q * a.I + nt * (BN / 2) + cw * (WN / 2) + c;
      } else {
        brow = nt * BN + col;
        if (brow > a.ncols - 1) brow = a.ncols - 1;
      }
      b_src[t] = (const char*)(Be + (int64_t)brow * a.K + chunk * 8);
    }
    if constexpr (kBuf) {
      ra = raw_rsrc(a.a_base);
      rb = raw_rsrc(Be);
#pragma unroll
      for (int t = 0; t < LA; ++t) a_off[t] = (uint32_t)(a_src[t] - a.a_base);
#pragma unroll
      for (int t = 0; t < LB; ++t) b_off[t] = (uint32_t)(b_src[t] - (const char*)Be);
    }
  }

  // One 1 KB block: 64 lanes x 16 bytes at byte koff of their rows into dst.
  __device__ __forceinline__ void load_a(int t, int koff, char* dst) const {
    if constexpr (kBuf)
      buffer_load_lds16(ra, dst, a_off[t], koff);
    else
      __builtin_amdgcn_global_load_lds((const void*)(a_src[t] + koff), (lds_void*)dst, 16, 0, 0);
  }
  // kNt: the weight panel is read by this tile only (its expert has one m-tile),
  // so its bytes are streamed with the non-temporal cache policy.
  template <bool kNt>
  __device__ __forceinline__ void load_b(int t, int koff, char* dst) const {
    if constexpr (kBuf) {
      if constexpr (kNt)
        buffer_load_lds16_nt(rb, dst, b_off[t], koff);
      else
        buffer_load_lds16(rb, dst, b_off[t], koff);
    } else {
      __builtin_amdgcn_global_load_lds((const void*)(b_src[t] + koff), (lds_void*)dst, 16, 0,
                                       kNt ? 2 : 0);
    }
  }

  // Compact stage of a tile with at most SROWS rows: those rows of A (the
  // first blocks, which only the first waves hold) then the BN rows of B.
  template <int SROWS>
  static constexpr int small_a() { return SROWS * G::ROW_BYTES; }
  template <int SROWS>
  static constexpr int small_stage() { return small_a<SROWS>() + BN * G::ROW_BYTES; }
  template <int SROWS, bool kNt>
  __device__ __forceinline__ void issue_small(char* smem, int kt, int buf) const {
    char* base = smem + buf * small_stage<SROWS>();
    const int koff = kt * G::ROW_BYTES;
#pragma unroll
    for (int t = 0; t < LA; ++t)
      if (t < live_a)  // blocks past the tile's (at most SROWS) rows are not live
        load_a(t, koff, base + (wave * LA + t) * 1024);
#pragma unroll
    for (int t = 0; t < LB; ++t)
      load_b<kNt>(t, koff, base + small_a<SROWS>() + (wave * LB + t) * 1024);
  }

  // Rings of the wide 256 x 256 kernel: two A stages, then three B stages.
  static constexpr int A_BYTES = BM * G::ROW_BYTES, B_BYTES = BN * G::ROW_BYTES;
  __device__ __forceinline__ void issue_a(char* smem, int kt, int abuf) const {
    char* base = smem + abuf * A_BYTES;
    const int koff = kt * G::ROW_BYTES;
#pragma unroll
    for (int t = 0; t < LA; ++t)
      if (t < live_a) load_a(t, koff, base + (wave * LA + t) * 1024);
  }
  template <bool kNt>
  __device__ __forceinline__ void issue_b(char* smem, int kt, int bbuf) const {
    char* base = smem + 2 * A_BYTES + bbuf * B_BYTES;
    const int koff = kt * G::ROW_BYTES;
#pragma unroll
    for (int t = 0; t < LB; ++t) load_b<kNt>(t, koff, base + (wave * LB + t) * 1024);
  }

  // Loads one stage.  A blocks of 1 KB that lie wholly past the tile's rows are
  // not loaded (their LDS rows feed only outputs that are never stored), so a
  // wave issues live_a + LB loads per stage.
  template <bool kNt>
  __device__ __forceinline__ void issue(char* smem, int kt, int buf) const {
    char* base = smem + buf * STAGE_BYTES;
    const int koff = kt * G::ROW_BYTES;
#pragma unroll
    for (int t = 0; t < LA; ++t)
      if (t < live_a) load_a(t, koff, base + (wave * LA + t) * 1024);
#pragma unroll
    for (int t = 0; t < LB; ++t)
      load_b<kNt>(t, koff, base + BM * G::ROW_BYTES + (wave * LB + t) * 1024);
  }
};

// Waits until at most n of this wave's vector memory operations are pending
// (s_waitcnt takes an immediate, so n is dispatched over its possible values).
__device__ __forceinline__ void wait_loads(int n) {
#define MOE_WAIT_CASE(v)                    \
  case v:                                   \
    __builtin_amdgcn_s_waitcnt(wait_vm(v)); \
    return;
  switch (n) {
    MOE_WAIT_CASE(1) MOE_WAIT_CASE(2) MOE_WAIT_CASE(3) MOE_WAIT_CASE(4) MOE_WAIT_CASE(5)
    MOE_WAIT_CASE(6) MOE_WAIT_CASE(7) MOE_WAIT_CASE(8) MOE_WAIT_CASE(9) MOE_WAIT_CASE(10)
    MOE_WAIT_CASE(11) MOE_WAIT_CASE(12) MOE_WAIT_CASE(13) MOE_WAIT_CASE(14) MOE_WAIT_CASE(15)
    MOE_WAIT_CASE(16) MOE_WAIT_CASE(17) MOE_WAIT_CASE(18) MOE_WAIT_CASE(19) MOE_WAIT_CASE(20)
    MOE_WAIT_CASE(21) MOE_WAIT_CASE(22) MOE_WAIT_CASE(23) MOE_WAIT_CASE(24)
    default:  // n <= 0, or beyond the table: wait for every load
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      return;
  }
#undef MOE_WAIT_CASE
}

// Epilogue through LDS.  The K loops pass the weight fragment as the MFMA's
// first operand and the row fragment as its second, so each 32x32 block holds
// C transposed: lane l holds row l % 32 of columns 8*(q/4) + 4*(l/32) + q%4,
// q = 0..15 (the products and their order over K are those of the other
// operand order: same bits).  A lane's four consecutive columns of a row go to
// LDS as one 8-byte write (with the rows in each lane's columns, one 2-byte
// write per element had taken four times the LDS writes and twice the
// conversions: down GEMM 2-2.5% slower).  Every wave writes its nblk 32-row
// blocks from row row0 (after SwiGLU for gate_up) as bf16 into a row-major C
// tile in the freed stage buffers, then the workgroup stores the tile 16 bytes
// per lane, one row segment at a time.  PLANES = 3 (gate_up in the backward's
// recompute) also saves g and u into the joint [rows][2I] copy: one plane per
// pass.
template <bool kGateUp, int PLANES, int FM, int FN, int BM, int BN, int WM, int WN, int NT>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& a, const f32x16 (&acc)[FM][FN],
                                               const TileRows& tr, int nt, int row0, int nblk,
                                               int wn, int lane, char* smem) {
  constexpr int CT = kGateUp ? BN / 2 : BN;  // tile columns of C
  constexpr int CPR = CT / 8;                // 16-byte chunks per tile row
  static_assert(CPR >= 8, "chunk swizzle needs 8 chunks per row");
  static_assert(PLANES == 1 || kGateUp, "g and u exist for gate_up only");
  // chunk ch of row r at slot ch ^ (r mod CPR): the 32 rows of one 8-byte
  // write (a row per lane, lanes l and l + 32 the two halves of one chunk)
  // fall in distinct slots
  auto lds_at = [](int r, int c) {
    return r * (CT * 2) + (((c >> 3) ^ (r & (CPR - 1))) << 4) + (c & 7) * 2;
  };
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const int rl = row0 + (lane & 31), cq = 4 * (lane >> 5);
  const int col0 = nt * CT;
  const uint16_t* const cbase[2] = {a.C[0], a.C[1]};
#pragma unroll
  for (int plane = 0; plane < PLANES; ++plane) {
    if (plane > 0) __syncthreads();  // the previous plane's reads are done
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      // blocks past the wave's band or the tile's rows: never stored
      if (i >= nblk || row0 + i * 32 >= tr.rows) break;
      const int r = rl + i * 32;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        if constexpr (kGateUp) {
#pragma unroll
          for (int j = 0; j < FN / 2; ++j) {
            const int c = wn * (WN / 2) + j * 32 + 8 * g4 + cq;
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float g = acc[i][j][4 * g4 + t], u = acc[i][j + FN / 2][4 * g4 + t];
              v[t] = plane == 0 ? swiglu(g, u) : plane == 1 ? g : u;
            }
            *(bf16x4*)(smem + lds_at(r, c)) =
                bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
          }
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int c = wn * WN + j * 32 + 8 * g4 + cq;
            const f32x16& x = acc[i][j];
            *(bf16x4*)(smem + lds_at(r, c)) =
                bf16x4{(__bf16)x[4 * g4], (__bf16)x[4 * g4 + 1], (__bf16)x[4 * g4 + 2],
                       (__bf16)x[4 * g4 + 3]};
          }
        }
      }
    }
    __syncthreads();
    for (int ch = threadIdx.x; ch < BM * CPR; ch += NT) {
      const int r = ch / CPR, c = (ch % CPR) * 8;
      if (r >= tr.rows || col0 + c >= a.ncols) continue;
      typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
      const u32x4v v = *(const u32x4v*)(smem + lds_at(r, c));
      uint16_t* dst;
      if (plane == 0)
        dst = (uint16_t*)row_ptr(cbase, a.c_split, tr, tr.v0 + r, a.ncols);
      else  // g (plane 1) or u (plane 2) of the joint [rows][2I] copy
        dst = a.gu + (int64_t)tr.joint_row(tr.v0 + r) * (2 * a.I) + (plane - 1) * a.I;
      // each output row is written once and read by the next launch: streamed
      // non-temporally in the forward (act, y); the backward's recompute keeps
      // plain stores for the g and u planes it reads back
      if constexpr (PLANES == 1)
        __builtin_nontemporal_store(v, (u32x4v*)(dst + col0 + c));
      else
        *(u32x4v*)(dst + col0 + c) = v;
    }
  }
}

// The K loop of one wave.  F (<= FM) 32-row blocks of the wave's band take
// part in the MFMAs (F = 0: none); the wave still issues its share of every
// stage's loads and joins every barrier.  The loop body holds no branch, so
// the compiler schedules the fragment reads, MFMAs and the next stage's loads
// as one block.
template <int F, int FM, int FN, int WM, int WN, int BM, int BK, int STAGES, bool kNt, class Loader>
__device__ __forceinline__ void k_loop(f32x16 (&acc)[FM][FN], const Loader& ld, char* smem,
                                       int KT, int per_stage, int lane, int wm, int wn) {
  using G = StageGeom<BK>;
  constexpr int KS = BK / 16;  // MFMA sub-steps per stage
  // nothing of the lgkm class (scalar loads included) is pending on entry, so
  // the waits before each sub-step's MFMAs can count the LDS reads in order
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  for (int kt = 0; kt < KT; ++kt) {
    // stage kt has landed once only the newer stages issued so far are pending
    const int newer = KT - 1 - kt < STAGES - 2 ? KT - 1 - kt : STAGES - 2;
    wait_loads(newer * per_stage);
    __builtin_amdgcn_s_barrier();
    const char* sa = smem + (kt % STAGES) * Loader::STAGE_BYTES;
    const char* sb = sa + BM * G::ROW_BYTES;
    if constexpr (F > 0) {
      // fragments in two register sets: sub-step kk + 1 is read while the
      // MFMAs of sub-step kk run
      bf16x8 af[2][F], bfr[2][FN];
      auto frag = [&](int kk, int b) __attribute__((always_inline)) {
        const int fo = G::frag_offset(lane, kk);
#pragma unroll
        for (int i = 0; i < F; ++i)
          af[b][i] = *(const bf16x8*)(sa + (wm * WM + i * 32) * G::ROW_BYTES + fo);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[b][j] = *(const bf16x8*)(sb + (wn * WN + j * 32) * G::ROW_BYTES + fo);
      };
      frag(0, 0);  // ahead of the next stage's loads, so the first MFMAs start sooner
      if (kt + STAGES - 1 < KT)
        ld.template issue<kNt>(smem, kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) frag(kk + 1, (kk + 1) & 1);
        // keeps the compiler from sinking those reads below this sub-step's MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < F; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk & 1][j], af[kk & 1][i],
                                                                acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      if (kt + STAGES - 1 < KT)
        ld.template issue<kNt>(smem, kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    }
    // this stage's LDS reads are complete before any wave refills its buffer
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }
}

// The K loop of the wide 256 x 256 kernel (two waves per SIMD).
// Each load instruction holds its wave in issue until the CU's texture unit
// takes it, at 16-20 cycles per 1 KB; with all eight waves issuing a 64 KB
// stage at the start of a K step, no wave reached its MFMAs for the first
// 800-1150 of about 3300 cycles.  So the two waves of a SIMD take different
// roles.  The second (wave row 1) issues the next step's rows of A at the
// start of the step; the first (wave row 0), which gets the matrix pipe first
// and used to wait about 1000 cycles at the barrier, starts its MFMAs at once
// and issues the weight rows of B two steps ahead once its MFMAs are issued.
// A stays double-buffered and B triple-buffered (2 x 32 + 3 x 32 KB).  Loader
// slot q = wave % 4 of a four-wave loader layout covers the same rows in
// either role.
template <int F, int FM, int FN, int WM, int WN, int BM, int BK, bool kNt, class Loader>
__device__ __forceinline__ void k_loop_roles(f32x16 (&acc)[FM][FN], const Loader& ld, char* smem,
                                             int KT, int lane, int wm, int wn) {
  using G = StageGeom<BK>;
  constexpr int KS = BK / 16;
  const bool a_role = wm != 0;
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  for (int kt = 0; kt < KT; ++kt) {
    // an A wave's newest load is A(kt); a B wave may still have B(kt + 1)
    // pending behind B(kt)
    wait_loads(!a_role && kt + 1 < KT ? Loader::LB : 0);
    __builtin_amdgcn_s_barrier();
    const char* sa = smem + (kt & 1) * Loader::A_BYTES;
    const char* sb = smem + 2 * Loader::A_BYTES + (kt % 3) * Loader::B_BYTES;
    if constexpr (F > 0) {
      bf16x8 af[2][F], bfr[2][FN];
      auto frag = [&](int kk, int b) __attribute__((always_inline)) {
        const int fo = G::frag_offset(lane, kk);
#pragma unroll
        for (int i = 0; i < F; ++i)
          af[b][i] = *(const bf16x8*)(sa + (wm * WM + i * 32) * G::ROW_BYTES + fo);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[b][j] = *(const bf16x8*)(sb + (wn * WN + j * 32) * G::ROW_BYTES + fo);
      };
      frag(0, 0);
      if (a_role && kt + 1 < KT) ld.issue_a(smem, kt + 1, (kt + 1) & 1);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) frag(kk + 1, (kk + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < F; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk & 1][j], af[kk & 1][i],
                                                                acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!a_role && kt + 2 < KT) ld.template issue_b<kNt>(smem, kt + 2, (kt + 2) % 3);
    } else {
      if (a_role && kt + 1 < KT) ld.issue_a(smem, kt + 1, (kt + 1) & 1);
      if (!a_role && kt + 2 < KT) ld.template issue_b<kNt>(smem, kt + 2, (kt + 2) % 3);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }
}

// K loop of a tile on the wide path: the first STAGES - 1 stages, then
// k_loop over the 32-row blocks of this wave's band that hold rows of the
// tile.  Blocks past them feed only outputs that are never stored, so a wide
// tile skips their MFMAs (a band of 1 or 2 live blocks runs the 1- or 2-block
// loop, 3 runs the full one).  A one-block band always runs its MFMAs: a
// wave-uniform branch there measured slower than the wasted work.
// (kRoles: the wide kernel's role split, k_loop_roles.)
template <int FM, int FN, int WM, int WN, int BM, int BK, int STAGES, bool kNt, bool kRoles,
          class Loader>
__device__ __forceinline__ void wide_k(f32x16 (&acc)[FM][FN], const Loader& ld, char* smem, int KT,
                                       int per_stage, int lane, int wm, int wn, int rows) {
  if constexpr (kRoles) {
    // KT >= 1: H and I are positive multiples of 64 (checked at the boundary)
    if (wm != 0) {
      ld.issue_a(smem, 0, 0);
    } else {
      ld.template issue_b<kNt>(smem, 0, 0);
      if (1 < KT) ld.template issue_b<kNt>(smem, 1, 1);
    }
  } else {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < KT) ld.template issue<kNt>(smem, s, s);
  }
  const int band_rows = rows - wm * WM;
  const int fm_live = band_rows <= 0 ? 0 : (band_rows + 31) / 32;
#define MOE_K_LOOP(F)                                                                              \
  do {                                                                                             \
    if constexpr (kRoles)                                                                          \
      k_loop_roles<F, FM, FN, WM, WN, BM, BK, kNt, Loader>(acc, ld, smem, KT, lane, wm, wn);       \
    else                                                                                           \
      k_loop<F, FM, FN, WM, WN, BM, BK, STAGES, kNt, Loader>(acc, ld, smem, KT, per_stage, lane,   \
                                                             wm, wn);                              \
  } while (0)
  if constexpr (FM == 1) {
    MOE_K_LOOP(1);
  } else {
    if (fm_live > 2)
      MOE_K_LOOP(FM);
    else if (fm_live == 2)
      MOE_K_LOOP(2);
    else if (fm_live == 1)
      MOE_K_LOOP(1);
    else
      MOE_K_LOOP(0);
  }
#undef MOE_K_LOOP
}

// MFMAs of one compact stage at sa (rows of A, then B): the wave's F 32-row
// blocks from row0 against its FN 32-column blocks, the fragments of each
// 16-deep sub-step read right before its MFMAs.
template <int F, int SROWS, int FM, int FN, int WN, int BK, class Loader>
__device__ __forceinline__ void compact_mfma(f32x16 (&acc)[FM][FN], const char* sa, int lane,
                                             int wn, int row0) {
  using G = StageGeom<BK>;
  static_assert(F <= FM, "band blocks");
  if constexpr (F > 0) {
    const char* sb = sa + Loader::template small_a<SROWS>();
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int fo = G::frag_offset(lane, kk);
      bf16x8 af[F], bfr[FN];
#pragma unroll
      for (int i = 0; i < F; ++i)
        af[i] = *(const bf16x8*)(sa + (row0 + i * 32) * G::ROW_BYTES + fo);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *(const bf16x8*)(sb + (wn * WN + j * 32) * G::ROW_BYTES + fo);
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }
}

// The K loop of a tile with at most SROWS (32, 64, 128 or 160) rows: such a
// tile (a small expert's only m-tile) is bound by streaming its B panel rather
// than by MFMAs, so it uses the compact stage layout and SSTAGES stages
// (SSTAGES - 1 in flight) to keep more weight bytes in flight.  The wave holds
// F 32-row blocks of the tile's rows starting at row0 (its band); a wave with
// F = 0 only loads and joins the barriers.  (Reading the next sub-step's
// fragments during the current MFMAs, as k_loop does, measured no faster here.)
template <int F, int SROWS, int SSTAGES, int FM, int FN, int WN, int BK, bool kNt, class Loader>
__device__ __forceinline__ void k_loop_small(f32x16 (&acc)[FM][FN], const Loader& ld, char* smem,
                                             int KT, int per_stage, int lane, int wn, int row0) {
  constexpr int STAGE = Loader::template small_stage<SROWS>();
#pragma unroll
  for (int s = 0; s < SSTAGES - 1; ++s)
    if (s < KT) ld.template issue_small<SROWS, kNt>(smem, s, s);
  for (int kt = 0; kt < KT; ++kt) {
    const int newer = KT - 1 - kt < SSTAGES - 2 ? KT - 1 - kt : SSTAGES - 2;
    wait_loads(newer * per_stage);
    __builtin_amdgcn_s_barrier();
    if (kt + SSTAGES - 1 < KT)
      ld.template issue_small<SROWS, kNt>(smem, kt + SSTAGES - 1, (kt + SSTAGES - 1) % SSTAGES);
    compact_mfma<F, SROWS, FM, FN, WN, BK, Loader>(acc, smem + (kt % SSTAGES) * STAGE, lane, wn,
                                                   row0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }
}

// kLoop: the workgroup takes tile after tile of its XCD's sequence (launched
// when the grid is capped below the tile bound); otherwise exactly one.
template <bool kGateUp, bool kSaveGU, int BM, int BN, int WAVES_M, int WAVES_N, int BK,
          int STAGES, bool kBuf, bool kLoop>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N) grouped_gemm_bf16(GemmArgs a) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  using Loader = TileLoader<kGateUp, BM, BN, NW, WN, BK, kBuf>;
  // the wide kernel splits the loads by wave role (k_loop_roles)
  constexpr bool kRoles = NW == 8;
  using RoleLoader = TileLoader<kGateUp, BM, BN, kRoles ? NW / 2 : NW, WN, BK, kBuf>;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
  static_assert(!kGateUp || WN % 64 == 0, "gate/up halves");
  static_assert(STAGES >= 2, "pipeline depth");
  static_assert((STAGES - 2) * (Loader::LA + Loader::LB) <= 24, "wait_loads range");
  constexpr int kSmemBytes =
      cmax(kRoles ? 2 * Loader::A_BYTES + 3 * Loader::B_BYTES : STAGES * Loader::STAGE_BYTES,
           FM >= 4 ? cmax(3 * Loader::template small_stage<160>(),
                          cmax(3 * Loader::template small_stage<32>(),
                               3 * Loader::template small_stage<64>()))
                   : 0);
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];

  const int lane0 = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // Tiles of this workgroup: position q of its XCD's sequence, and with kLoop
  // also q + G, q + 2G, ... (G = the XCD's workgroups: the host then launches
  // fewer workgroups than the tile bound, so that a launch whose row count
  // allows many more tiles than the routing produced does not dispatch
  // thousands of workgroups that find none).
  const int xcd = blockIdx.x & 7, wg_per_xcd = gridDim.x >> 3;
  for (int q = blockIdx.x >> 3;; q += wg_per_xcd) {
    // In the tile loop the compiler hoisted every lane-derived address (loader
    // offsets, fragment offsets) out of the loop and kept them all live: 256
    // VGPRs and spills.  An opaque copy of the lane index per tile keeps them
    // inside (238 VGPRs, no VGPR spills with the load roles).
    int lane = lane0;
    if constexpr (kLoop) asm volatile("" : "+v"(lane));
    // (built per tile: kept across the K loop it would cost registers)
    MTileMap tm;
    // the wide tile (one workgroup per CU) orders small experts' m-tiles by size
    // to balance the XCDs; the narrow tile (three per CU) keeps expert order,
    // which mixes weight-streaming and MFMA-bound tiles on a CU (measured faster)
    tm.build(a.off0, a.off1, a.E, BM, BM >= 128 ? BM : 1);
    int mt, nt;
    if (!xcd_tile_at(tm, a.n_tiles, xcd, q, (32 + a.n_tiles - 1) / a.n_tiles, &mt, &nt)) break;
    const TileRows tr = tm.locate(a.off0, a.off1, BM, mt);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int KT = a.K / BK;
    // tiles of at most 32, 64, 128 or 160 rows: three compact stages (a fourth
    // stage for the 32-row tiles, in 16 KB more LDS, measured no faster; the
    // 128-row case, 144 KB, took the DeepSeek-V3-shaped layer's gate/up from 3.18
    // to 3.01 ms, its experts holding 95-160 rows each, and the 160-row case,
    // 156 KB, the layer from 4.89 to 4.79 ms)
    constexpr bool kSmallPath = FM >= 4 && WAVES_M == 2;
    // The weight panel of a tile that holds all of its expert's rows is read by
    // no other tile of the launch, so it is streamed non-temporally (decode
    // 3.28 -> 2.95 ms with the stores below); panels shared by several m-tiles
    // of one expert stay cached (non-temporal there cost the two-expert skew 13%).
    auto run_k = [&](auto nt_tag) __attribute__((always_inline)) {
    constexpr bool kNt = decltype(nt_tag)::value;
#define MOE_K_SMALL(SR)                                                                          \
  do {                                                                                           \
    constexpr int F0 = compact_f0(SR, kNt), F1 = compact_f1(SR, kNt);                            \
    if (wm == 0)                                                                                 \
      k_loop_small<F0, SR, 3, FM, FN, WN, BK, kNt, Loader>(acc, ld, smem, KT, per_stage, lane,   \
                                                           wn, 0);                               \
    else                                                                                         \
      k_loop_small<F1, SR, 3, FM, FN, WN, BK, kNt, Loader>(acc, ld, smem, KT, per_stage, lane,   \
                                                           wn, F0 * 32);                         \
  } while (0)
    if (kSmallPath && tr.rows <= 160) {
      if constexpr (kSmallPath) {
        Loader ld;
        ld.init(a, tr, nt, lane, wave);
        const int per_stage = ld.live_a + Loader::LB;  // loads this wave issues per stage
        if (tr.rows <= 32)
          MOE_K_SMALL(32);
        else if (tr.rows <= 64)
          MOE_K_SMALL(64);
        else if (tr.rows <= 128)
          MOE_K_SMALL(128);
        else
          MOE_K_SMALL(160);
      }
    } else if constexpr (kRoles) {
      RoleLoader ld;
      ld.init(a, tr, nt, lane, wave % (NW / 2));
      wide_k<FM, FN, WM, WN, BM, BK, STAGES, kNt, true, RoleLoader>(acc, ld, smem, KT, 0, lane, wm,
                                                                    wn, tr.rows);
    } else {
      Loader ld;
      ld.init(a, tr, nt, lane, wave);
      const int per_stage = ld.live_a + Loader::LB;
      wide_k<FM, FN, WM, WN, BM, BK, STAGES, kNt, false, Loader>(acc, ld, smem, KT, per_stage, lane,
                                                                 wm, wn, tr.rows);
    }
#undef MOE_K_SMALL
    };
    if (tr.single)
      run_k(std::true_type{});
    else
      run_k(std::false_type{});
    static_assert(BM * (kGateUp ? BN / 2 : BN) * 2 <= STAGES * Loader::STAGE_BYTES,
                  "C tile fits the stage buffers");
    __syncthreads();  // every wave is done with the stage buffers
    // this wave's rows: its wave row's WM on the wide path, the compact split
    // (recomputed here so that nothing more stays live across the K loop)
    int band0 = wm * WM, nblk = FM;
    if constexpr (kSmallPath) {
      if (tr.rows <= 160) {
        const bool spread = tr.single != 0;
        const int f0 = compact_f0(tr.rows, spread);
        band0 = wm * f0 * 32;
        nblk = wm == 0 ? f0 : compact_f1(tr.rows, spread);
      }
    }
    store_tile_lds<kGateUp, kSaveGU ? 3 : 1, FM, FN, BM, BN, WM, WN, 64 * NW>(a, acc, tr, nt, band0,
                                                                             nblk, wn, lane, smem);
    if constexpr (!kLoop) break;
    __syncthreads();  // the C tile has left LDS before the next tile's stage loads
  }
}

// Tile instances.  Both use the same MFMA instruction and the same order of
// K steps, so either gives the same bits for a row; the choice only affects
// speed.  The wide 256 x 256 tile (8 waves, one workgroup per CU) moves the
// fewest bytes per MFMA; the 64 x 128 tile (three workgroups per CU) wins on
// small launches.  A compile-time override forces one instance.
enum Instance { kAuto = 0, kWide = 1, kNarrow = 2 };
#ifndef MOE_GEMM_FORCE
#define MOE_GEMM_FORCE 0
#endif

// With the small-tile loop and the size-balanced tile order the wide tile also
// wins on launches of a few thousand rows with short expert blocks (8192 rows
// over 54 experts: gate/up 145 against 158 us, down 84 against 100 us); the
// narrow one still wins on decode-sized launches (512 rows), which are pure
// weight streaming.
bool prefer_wide(int64_t rows_bound) { return rows_bound >= 4096; }

template <bool kGateUp, bool kSaveGU, int BM, int BN, int WM_, int WN_, int BK, int ST,
          bool kBuf>
hipError_t launch_instance(GemmArgs a, const Shape& s, int64_t rows_bound, hipStream_t st) {
  constexpr int threads = 64 * WM_ * WN_;
  // gate_up tiles cover BN/2 intermediate columns (gate and up halves)
  a.n_tiles = kGateUp ? s.I / (BN / 2) : (s.H + BN - 1) / BN;
  const int64_t grid = xcd_grid(m_tiles_bound(rows_bound, s.E, BM), a.n_tiles);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  // The bound counts a partial m-tile for each of up to E experts.  When that
  // far exceeds what the rows can fill (few active experts out of many), each
  // surplus workgroup still costs a dispatch of the whole tile's waves and
  // LDS (the two-expert E = 256 launch: 4096 of 4608), so the wide tile caps
  // each XCD at twice its full-tile positions (at least 128 workgroups) and
  // its workgroups take several tiles each: gate/up 410 -> 395 us and down
  // 265 -> 257 us on that launch.  Only where the cap removes more than half
  // the grid: elsewhere the tile loop, with its larger register footprint,
  // measured 0-2% slower than the one-tile kernel.
  if constexpr (BM == 256 && kBuf) {
    const int64_t cap = 8 * std::max<int64_t>(128, 2 * ((rows_bound / BM + 7) / 8) * a.n_tiles);
    if (2 * cap < grid) {
      hipLaunchKernelGGL((grouped_gemm_bf16<kGateUp, kSaveGU, BM, BN, WM_, WN_, BK, ST, kBuf, true>),
                         dim3((unsigned)cap), dim3(threads), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((grouped_gemm_bf16<kGateUp, kSaveGU, BM, BN, WM_, WN_, BK, ST, kBuf, false>),
                     dim3((unsigned)grid), dim3(threads), 0, st, a);
  return hipGetLastError();
}

template <bool kGateUp, bool kSaveGU, bool kBuf>
hipError_t launch_kind(int inst, GemmArgs a, const Shape& s, int64_t rows_bound, hipStream_t st) {
  // a 256-column gate_up tile holds 128 intermediate columns
  const bool wide_ok = !kGateUp || s.I % 128 == 0;
  if (inst == kAuto) {
    inst = prefer_wide(rows_bound) ? kWide : kNarrow;
  }
  if (inst == kWide && wide_ok)
    return launch_instance<kGateUp, kSaveGU, 256, 256, 2, 4, 64, 2, kBuf>(a, s, rows_bound, st);
  return launch_instance<kGateUp, kSaveGU, 64, 128, 2, 2, 64, 2, kBuf>(a, s, rows_bound, st);
}

template <bool kGateUp, bool kSaveGU>
hipError_t launch_kind(bool buf, int inst, GemmArgs a, const Shape& s, int64_t rows_bound,
                       hipStream_t st) {
  return buf ? launch_kind<kGateUp, kSaveGU, true>(inst, a, s, rows_bound, st)
             : launch_kind<kGateUp, kSaveGU, false>(inst, a, s, rows_bound, st);
}

// Descriptor loads take 32-bit byte offsets: every A row (a row of
// hidden_states when gathered, else of one or both row buffers, each bounded
// by the launch's rows) must lie within 4 GiB above the lower base, and each
// expert's weight block within 4 GiB of its start.  Sets a.a_base.
bool descriptor_loads_fit(GemmArgs& a, const Shape& s, int64_t rows_bound) {
  const uint16_t* a1 = a.a_split ? a.A[1] : a.A[0];
  a.a_base = (const char*)std::min(a.A[0], a1);
  return rows_fit_4g(a.A[0], a1, a.gather[0] ? s.T : rows_bound, a.K) &&
         (uint64_t)a.b_expert_stride * 2 < ((uint64_t)1 << 32);
}

hipError_t launch(bool gate_up, const Shape& s, const GroupedIO& io, const void* B,
                  hipStream_t st) {
  const int64_t rows_bound = io.rows_bound;
  if (rows_bound <= 0) return hipSuccess;
  GemmArgs a{};
  a.A[0] = (const uint16_t*)io.a[0];
  a.A[1] = (const uint16_t*)(io.a_split ? io.a[1] : io.a[0]);
  a.C[0] = (uint16_t*)io.c[0];
  a.C[1] = (uint16_t*)(io.c_split ? io.c[1] : io.c[0]);
  a.off0 = io.off[0];
  a.off1 = io.off[1];
  a.a_split = io.a_split && io.off[1];
  a.c_split = io.c_split && io.off[1];
  a.gu = gate_up ? (uint16_t*)io.gu : nullptr;
  a.gather[0] = gate_up ? io.gather[0] : nullptr;
  a.gather[1] = gate_up && io.off[1] ? io.gather[1] : a.gather[0];
  a.gather_k = io.gather_k;
  a.B = (const uint16_t*)B;
  a.E = s.E;
  a.I = s.I;
  const int inst = MOE_GEMM_FORCE;
  if (gate_up) {
    a.K = s.H;
    a.ncols = s.I;
    a.b_expert_stride = (int64_t)2 * s.I * s.H;
    // the backward's recompute also saves g and u (its own instance, so the
    // forward kernel keeps its registers)
    const bool buf = descriptor_loads_fit(a, s, rows_bound);
    if (a.gu) return launch_kind<true, true>(buf, inst, a, s, rows_bound, st);
    return launch_kind<true, false>(buf, inst, a, s, rows_bound, st);
  }
  a.K = s.I;
  a.ncols = s.H;
  a.b_expert_stride = (int64_t)s.H * s.I;
  const bool buf = descriptor_loads_fit(a, s, rows_bound);
  return launch_kind<false, false>(buf, inst, a, s, rows_bound, st);
}

}  // namespace

hipError_t launch_gate_up_bf16(const Shape& s, const GroupedIO& io, const void* w_gate_up,
                               hipStream_t st) {
  return launch(true, s, io, w_gate_up, st);
}

hipError_t launch_down_bf16(const Shape& s, const GroupedIO& io, const void* w_down,
                            hipStream_t st) {
  return launch(false, s, io, w_down, st);
}

}  // namespace moe
