// Routing metadata for every chunk in one pass: per-expert counts, exclusive
// offsets, destination-group send splits and the stable permutation
// (src_row / dst_row).
//
// MindSpeed Chunk MoE article, timing-diagram section: the metadata of all
// chunks is produced once, not per chunk.  MindSpore news page, "# 02
// AlltoAllV收发异构复用特性": the send lists stay on the device and combine
// reuses dispatch's lists (here dst_row), so nothing is copied to the host.
//
// Three launches, deterministic (LDS atomics only add counts, whose sum does
// not depend on order):
//  1. meta_hist : one wave per segment of kMetaSeg assignments (segments never
//     straddle a chunk).  Every lane adds 1 to its expert's LDS counter.
//     Writes seg_counts[seg][E] and the dropped-id count.
//  2. meta_scan : one workgroup per chunk.  Per expert, an exclusive prefix
//     over the chunk's segments (in place), then a block-wide exclusive scan
//     over experts gives offsets; seg_counts becomes each segment's first row
//     per expert.  Also counts, group splits, the -1 tail of src_row, and (in
//     workgroup 0) dev_error.
//  3. meta_rank : one wave per segment again.  Lanes with equal expert id find
//     each other through one LDS word per expert (peer_mask: an OR of lane
//     bits); rank = popcount(peers below me) plus the segment's running base
//     per expert gives dst_row[f] and src_row[chunk_start + row] = f.  Lanes
//     are walked in ascending f, so the permutation is stable.
//
// Chunks of at most kHistScanMaxIds assignments (at most kFusedMaxAll in all)
// fold steps 1 and 2 into one launch, meta_hist_scan: one 1024-thread
// workgroup per chunk counts every segment of the chunk into the staged LDS
// block and scans it in place; meta_rank, spread over the chip, follows.
//
// Chunks of at most kFusedMaxIds assignments (E <= kFusedMaxE, at most
// kFusedMaxAll assignments in all) take one launch instead: meta_fused runs
// the same three steps in one 1024-thread workgroup per chunk.  Wave w owns
// the w-th of 16 contiguous slices of the chunk (at most 512 assignments, held
// in registers with their peer masks from the histogram pass to the rank pass)
// and keeps its per-expert counts and peer words in row w of LDS, so the
// prefix over slices takes the place of the prefix over segments and no step
// waits on another launch.  Workgroup 0 also counts the dropped ids of every
// chunk.  Chunks this small are latency-bound: the two extra launches and the
// round trip of the segment counts through memory cost more than the work.
#include "moe_internal.h"

namespace moe {

namespace {

struct MetaArgs {
  const int32_t* idx;
  int32_t* seg_counts;
  int32_t* seg_invalid;
  int32_t* counts;
  int32_t* offsets;
  int32_t* splits;
  int32_t* src_row;
  int32_t* dst_row;
  int32_t* dev_error;
  int T, k, E, G, N, Tc, spc, seg;
};

// Segment `seg` -> its chunk and flat range [f_lo, f_hi).
__device__ __forceinline__ void seg_range(const MetaArgs& a, int seg, int* chunk, int* f_lo,
                                          int* f_hi, int* chunk_f0) {
  int c = seg / a.spc, j = seg - c * a.spc;
  long long t0 = (long long)c * a.Tc, t1 = (long long)(c + 1) * a.Tc;
  if (t0 > a.T) t0 = a.T;
  if (t1 > a.T) t1 = a.T;
  long long lo = t0 * a.k + (long long)j * a.seg;
  long long hi = lo + a.seg;
  if (hi > t1 * a.k) hi = t1 * a.k;
  if (lo > hi) lo = hi;
  *chunk = c;
  *f_lo = (int)lo;
  *f_hi = (int)hi;
  *chunk_f0 = (int)(t0 * a.k);
}

// Mask of the lanes of this wave whose (valid) expert id equals this lane's,
// through one LDS word per expert: every valid lane ORs its bit into word[e]
// and reads the word back.  One wave's LDS operations complete in program
// order, so the read sees every OR of the instruction before it, and the
// result of an OR does not depend on the order in which the lanes are served.
// The words start at zero; the caller's group leader clears word[e] after the
// read (a later instruction, so every peer has read it by then).  Lanes that
// share a word are served one at a time, so a skewed group costs more than a
// spread one; an earlier form that took one ballot per id bit cost more on
// every workload but the most skewed.
__device__ __forceinline__ uint64_t peer_mask(unsigned long long* word, int e, bool ok) {
  if (ok) atomicOr(&word[e], 1ull << __lane_id());
  return ok ? (uint64_t)word[e] : 0;
}

// Ids of one 1024-assignment batch, 16 per lane, loaded together so their
// latencies overlap; inactive lanes (past the segment) get ok = false.
struct IdBatch {
  int e[16];
  bool active[16];
};

__device__ __forceinline__ void load_batch(const MetaArgs& a, int b0, int f_hi, int lane,
                                           IdBatch* b) {
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    const int f = b0 + g * 64 + lane;
    b->active[g] = f < f_hi;
    b->e[g] = b->active[g] ? a.idx[f] : -1;
  }
}

__global__ void __launch_bounds__(64) meta_hist(MetaArgs a) {
  extern __shared__ int cnt[];
  const int lane = threadIdx.x;
  int c, f_lo, f_hi, cf0;
  seg_range(a, blockIdx.x, &c, &f_lo, &f_hi, &cf0);
  for (int e = lane; e < a.E; e += 64) cnt[e] = 0;
  __syncthreads();
  int invalid = 0;
  for (int b0 = f_lo; b0 < f_hi; b0 += 1024) {
    IdBatch b;
    load_batch(a, b0, f_hi, lane, &b);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      if (b0 + g * 64 >= f_hi) break;
      const int e = b.e[g];
      const bool ok = b.active[g] && e >= 0 && e < a.E;
      invalid += (b.active[g] && !ok) ? 1 : 0;
      if (ok) atomicAdd(&cnt[e], 1);  // counts only: the sum does not depend on order
    }
  }
  __syncthreads();
  int32_t* out = a.seg_counts + (size_t)blockIdx.x * a.E;
  for (int e = lane; e < a.E; e += 64) out[e] = cnt[e];
  for (int d = 32; d > 0; d >>= 1) invalid += __shfl_xor(invalid, d);
  if (lane == 0) a.seg_invalid[blockIdx.x] = invalid;
}

// Exclusive block scan of one value per thread (blockDim.x == 1024).
__device__ int block_exclusive_scan(int v, int* total, int* lds_waves) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int d = 1; d < 64; d <<= 1) {
    int n = __shfl_up(incl, d);
    if (lane >= d) incl += n;
  }
  if (lane == 63) lds_waves[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? lds_waves[lane] : 0;
    int wi = w;
    for (int d = 1; d < 16; d <<= 1) {
      int n = __shfl_up(wi, d);
      if (lane >= d) wi += n;
    }
    if (lane < 16) lds_waves[16 + lane] = wi - w;  // exclusive wave prefix
    if (lane == 15) lds_waves[32] = wi;
  }
  __syncthreads();
  int r = incl - v + lds_waves[16 + wave];
  *total = lds_waves[32];
  __syncthreads();
  return r;
}

// Scan of chunk c's [segments][E] counts, staged in LDS: counts, offsets,
// group splits, the segment bases (to seg_counts) and the -1 tail of src_row.
__device__ void scan_chunk(const MetaArgs& a, int c, int* stage, int* lds_waves, int* off_lds) {
  // P consecutive lanes per expert (P a power of two, P * E <= 1024) share the
  // prefix over the chunk's segments: each sums a contiguous run of segments,
  // the P partial sums are scanned with lane shuffles, then each lane writes
  // its segments' running prefix
  int P = 64;
  while (P > 1 && P * a.E > (int)blockDim.x) P >>= 1;
  const int e = threadIdx.x / P, part = threadIdx.x % P;
  const bool has_e = e < a.E;
  const int n_stage = a.spc * a.E;  // <= kScanStage by the plan
  int32_t* blk = a.seg_counts + (size_t)c * a.spc * a.E;
  const int len = (a.spc + P - 1) / P;
  const int j0 = part * len < a.spc ? part * len : a.spc;
  const int j1 = j0 + len < a.spc ? j0 + len : a.spc;
  int local = 0;
  if (has_e)
    for (int j = j0; j < j1; ++j) local += stage[j * a.E + e];
  int incl = local;
  for (int d = 1; d < P; d <<= 1) {
    const int n = __shfl_up(incl, d, P);
    if (part >= d) incl += n;
  }
  const int count_e = __shfl(incl, P - 1, P);
  int run = incl - local;
  if (has_e)
    for (int j = j0; j < j1; ++j) {
      const int v = stage[j * a.E + e];
      stage[j * a.E + e] = run;
      run += v;
    }
  const bool lead = has_e && part == 0;
  int total;
  const int off = block_exclusive_scan(lead ? count_e : 0, &total, lds_waves);
  if (lead) {
    a.counts[(size_t)c * a.E + e] = count_e;
    a.offsets[(size_t)c * (a.E + 1) + e] = off;
    off_lds[e] = off;
  }
  if (threadIdx.x == 0) {
    a.offsets[(size_t)c * (a.E + 1) + a.E] = total;
    off_lds[a.E] = total;
  }
  __syncthreads();
  // segment bases: chunk offset + prefix over the chunk's earlier segments
  for (int i = threadIdx.x; i < n_stage; i += blockDim.x) blk[i] = stage[i] + off_lds[i % a.E];
  const int per = a.E / a.G;
  for (int g = threadIdx.x; g < a.G; g += blockDim.x)
    a.splits[(size_t)c * a.G + g] = off_lds[(g + 1) * per] - off_lds[g * per];
  // rows past the chunk's valid rows hold no assignment
  long long t0 = (long long)c * a.Tc, t1 = (long long)(c + 1) * a.Tc;
  if (t0 > a.T) t0 = a.T;
  if (t1 > a.T) t1 = a.T;
  const long long f0 = t0 * a.k, ac = (t1 - t0) * a.k;
  for (long long r = total + threadIdx.x; r < ac; r += blockDim.x) a.src_row[f0 + r] = -1;
}

__global__ void __launch_bounds__(1024) meta_scan(MetaArgs a) {
  __shared__ int stage[kScanStage];
  __shared__ int lds_waves[48];
  __shared__ int off_lds[kMaxExperts + 1];
  const int c = blockIdx.x;  // one workgroup per chunk
  const int n_stage = a.spc * a.E;
  const int32_t* blk = a.seg_counts + (size_t)c * a.spc * a.E;
  for (int i = threadIdx.x; i < n_stage; i += blockDim.x) stage[i] = blk[i];
  __syncthreads();
  scan_chunk(a, c, stage, lds_waves, off_lds);
  if (a.dev_error && c == 0) {
    int s = 0;
    const long long nseg = (long long)a.N * a.spc;
    for (long long i = threadIdx.x; i < nseg; i += blockDim.x) s += a.seg_invalid[i];
    int dropped;
    (void)block_exclusive_scan(s, &dropped, lds_waves);
    if (threadIdx.x == 0) *a.dev_error = dropped;
  }
}

// Dropped ids among idx[lo, hi), summed over this thread's share (1024
// threads, 16 loads in flight per thread).
__device__ int count_dropped(const MetaArgs& a, int lo, int hi) {
  int s = 0;
  for (int i0 = lo; i0 < hi; i0 += 16 * 1024) {
    int id[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * 1024 + (int)threadIdx.x;
      id[u] = i < hi ? a.idx[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) s += (id[u] < 0 || id[u] >= a.E) ? 1 : 0;
  }
  return s;
}

// Histogram and scan of one chunk in one workgroup (chunks of up to
// kHistScanMaxIds assignments); meta_rank follows.  Wave w takes a contiguous
// run of the chunk's segments; a 64-id group never straddles two segments
// (segments are multiples of 256 ids), so each group adds to one row of the
// staged [segments][E] block.  Workgroup 0 adds the other chunks' dropped ids
// to its own.
__global__ void __launch_bounds__(1024) meta_hist_scan(MetaArgs a) {
  __shared__ int stage[kScanStage];
  __shared__ int lds_waves[48];
  __shared__ int off_lds[kMaxExperts + 1];
  const int c = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n_stage = a.spc * a.E;
  for (int i = threadIdx.x; i < n_stage; i += blockDim.x) stage[i] = 0;
  __syncthreads();
  long long t0 = (long long)c * a.Tc, t1 = (long long)(c + 1) * a.Tc;
  if (t0 > a.T) t0 = a.T;
  if (t1 > a.T) t1 = a.T;
  const int cf0 = (int)(t0 * a.k), ac = (int)((t1 - t0) * a.k);
  const int spw = (a.spc + 15) / 16;  // segments per wave
  const long long lo_l = (long long)w * spw * a.seg, hi_l = lo_l + (long long)spw * a.seg;
  const int f_lo = cf0 + (int)(lo_l < ac ? lo_l : ac);
  const int f_hi = cf0 + (int)(hi_l < ac ? hi_l : ac);
  int invalid = 0;
  for (int b0 = f_lo; b0 < f_hi; b0 += 1024) {
    IdBatch b;
    load_batch(a, b0, f_hi, lane, &b);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      if (b0 + g * 64 >= f_hi) break;
      int* row = stage + ((b0 + g * 64 - cf0) / a.seg) * a.E;
      const int e = b.e[g];
      const bool ok = b.active[g] && e >= 0 && e < a.E;
      invalid += (b.active[g] && !ok) ? 1 : 0;
      if (ok) atomicAdd(&row[e], 1);  // counts only: the sum does not depend on order
    }
  }
  __syncthreads();
  scan_chunk(a, c, stage, lds_waves, off_lds);
  if (a.dev_error && c == 0) {
    const int s = invalid + count_dropped(a, ac, a.T * a.k);  // chunk 0 holds [0, ac)
    int dropped;
    (void)block_exclusive_scan(s, &dropped, lds_waves);
    if (threadIdx.x == 0) *a.dev_error = dropped;
  }
}

__global__ void __launch_bounds__(64) meta_rank(MetaArgs a) {
  extern __shared__ unsigned long long dyn[];  // [E] peer words, then [E] bases
  unsigned long long* word = dyn;
  int* base = (int*)(dyn + a.E);
  const int lane = threadIdx.x;
  int c, f_lo, f_hi, cf0;
  seg_range(a, blockIdx.x, &c, &f_lo, &f_hi, &cf0);
  (void)c;
  const int32_t* sb = a.seg_counts + (size_t)blockIdx.x * a.E;
  for (int e = lane; e < a.E; e += 64) {
    base[e] = sb[e];
    word[e] = 0;
  }
  __syncthreads();
  const uint64_t lt = lanemask_lt();
  for (int b0 = f_lo; b0 < f_hi; b0 += 1024) {
    IdBatch b;
    load_batch(a, b0, f_hi, lane, &b);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      if (b0 + g * 64 >= f_hi) break;
      const int f = b0 + g * 64 + lane;
      const int e = b.e[g];
      const bool ok = b.active[g] && e >= 0 && e < a.E;
      const uint64_t peers = peer_mask(word, e, ok);
      const int leader = ok ? __ffsll((unsigned long long)peers) - 1 : lane;
      // the leader takes the group's rows from its expert's running base (groups
      // of earlier lanes and earlier iterations come first: program order of
      // one wave); every peer adds its rank among the group's lanes
      int first = 0;
      if (ok && leader == lane) {
        first = atomicAdd(&base[e], (int)__popcll(peers));
        word[e] = 0;
      }
      first = __shfl(first, leader);
      const int row = ok ? first + __popcll(peers & lt) : -1;
      if (b.active[g]) a.dst_row[f] = row;
      if (ok) a.src_row[cf0 + row] = f;
    }
  }
}

constexpr int kFusedWaves = 16;
constexpr int kFusedMaxE = 512;       // LDS: kFusedWaves * E counters
constexpr int kFusedMaxIds = 8192;    // assignments of one chunk
constexpr int64_t kFusedMaxAll = 65536;  // all chunks (workgroup 0 counts dropped ids)
constexpr int kHistScanMaxIds = 32768;   // assignments of one chunk, meta_hist_scan

__global__ void __launch_bounds__(1024) meta_fused(MetaArgs a) {
  __shared__ int cnt[kFusedWaves * kFusedMaxE];  // [slice][E]
  __shared__ unsigned long long pw[kFusedWaves * kFusedMaxE];  // [slice][E] peer words
  __shared__ int off_lds[kFusedMaxE + 1];
  __shared__ int lds_waves[48];
  const int c = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  long long t0 = (long long)c * a.Tc, t1 = (long long)(c + 1) * a.Tc;
  if (t0 > a.T) t0 = a.T;
  if (t1 > a.T) t1 = a.T;
  const int f0 = (int)(t0 * a.k), ac = (int)((t1 - t0) * a.k);
  // slice length: a multiple of 64, 16 slices cover the chunk; a slice holds
  // at most 512 assignments, within one IdBatch, kept in registers for both passes
  const int len = ((ac + kFusedWaves * 64 - 1) / (kFusedWaves * 64)) * 64;
  const int s_lo = f0 + (w * len < ac ? w * len : ac);
  const int s_hi = f0 + ((w + 1) * len < ac ? (w + 1) * len : ac);
  for (int i = threadIdx.x; i < kFusedWaves * a.E; i += blockDim.x) {
    cnt[i] = 0;
    pw[i] = 0;
  }
  IdBatch b;
  load_batch(a, s_lo, s_hi, lane, &b);
  __syncthreads();
  int* mine = cnt + w * a.E;
  unsigned long long* words = pw + w * a.E;
  // 1. per-slice histogram: each group's peer masks, kept for the rank pass,
  // and one add of the group's popcount per expert by its lowest lane
  const int n_groups = (s_hi - s_lo + 63) >> 6;
  int invalid = 0;
  uint64_t peers[16];
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    peers[g] = 0;
    if (g < n_groups) {  // wave-uniform: slices end on a group boundary except the last
      const int e = b.e[g];
      const bool ok = b.active[g] && e >= 0 && e < a.E;
      invalid += (b.active[g] && !ok) ? 1 : 0;
      peers[g] = peer_mask(words, e, ok);
      if (ok && (__ffsll((unsigned long long)peers[g]) - 1) == lane) {
        atomicAdd(&mine[e], (int)__popcll(peers[g]));
        words[e] = 0;
      }
    }
  }
  __syncthreads();
  // 2. per expert (thread e): exclusive prefix over slices, then offsets over experts
  const int e = threadIdx.x;
  const bool has_e = e < a.E;
  int count_e = 0;
  if (has_e)
    for (int v = 0; v < kFusedWaves; ++v) {
      const int x = cnt[v * a.E + e];
      cnt[v * a.E + e] = count_e;
      count_e += x;
    }
  int total;
  const int off = block_exclusive_scan(has_e ? count_e : 0, &total, lds_waves);
  if (has_e) {
    for (int v = 0; v < kFusedWaves; ++v) cnt[v * a.E + e] += off;
    a.counts[(size_t)c * a.E + e] = count_e;
    a.offsets[(size_t)c * (a.E + 1) + e] = off;
    off_lds[e] = off;
  }
  if (threadIdx.x == 0) {
    a.offsets[(size_t)c * (a.E + 1) + a.E] = total;
    off_lds[a.E] = total;
  }
  __syncthreads();
  const int per = a.E / a.G;
  for (int g = threadIdx.x; g < a.G; g += blockDim.x)
    a.splits[(size_t)c * a.G + g] = off_lds[(g + 1) * per] - off_lds[g * per];
  // 3. stable rank within the slice, from the slice's base per expert
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    if (g < n_groups) {
      const int f = s_lo + g * 64 + lane;
      const int ee = b.e[g];
      const bool ok = b.active[g] && ee >= 0 && ee < a.E;
      const int leader = ok ? __ffsll((unsigned long long)peers[g]) - 1 : lane;
      int first = 0;
      if (ok && leader == lane) first = atomicAdd(&mine[ee], (int)__popcll(peers[g]));
      first = __shfl(first, leader);
      const int row = ok ? first + __popcll(peers[g] & lt) : -1;
      if (b.active[g]) a.dst_row[f] = row;
      if (ok) a.src_row[f0 + row] = f;
    }
  }
  if (a.dev_error && c == 0) {
    // dropped ids: this chunk's from the histogram pass, the other chunks' read here
    const int s = invalid + count_dropped(a, ac, a.T * a.k);  // chunk 0 holds [0, ac)
    int dropped;
    (void)block_exclusive_scan(s, &dropped, lds_waves);
    if (threadIdx.x == 0) *a.dev_error = dropped;
  }
  // rows past the chunk's valid rows hold no assignment
  for (int r = total + threadIdx.x; r < ac; r += blockDim.x) a.src_row[f0 + r] = -1;
}

}  // namespace

MetaPlan meta_plan(const Shape& s) {
  MetaPlan p{};
  const int64_t ac = (int64_t)s.Tc * s.k;
  // segment = a multiple of kMetaSeg (256) assignments, large enough that one
  // chunk's [segments][E] counts fit the scan kernel's LDS block
  int64_t seg = kMetaSeg;
  while (((ac + seg - 1) / seg) * s.E > kScanStage) seg += kMetaSeg;
  p.seg = (int)seg;
  p.segs_per_chunk = (int)((ac + seg - 1) / seg);
  if (p.segs_per_chunk < 1) p.segs_per_chunk = 1;
  p.nseg = (int64_t)s.N * p.segs_per_chunk;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.seg_counts_off = 0;
  p.seg_invalid_off = al((size_t)p.nseg * s.E * sizeof(int32_t));
  p.bytes = p.seg_invalid_off + al((size_t)p.nseg * sizeof(int32_t));
  return p;
}

hipError_t launch_route_meta(const Shape& s, const int32_t* idx, int32_t* counts,
                             int32_t* offsets, int32_t* splits, int32_t* src_row,
                             int32_t* dst_row, int32_t* dev_error, void* ws, hipStream_t st) {
  MetaPlan p = meta_plan(s);
  MetaArgs a{};
  a.idx = idx;
  a.seg_counts = (int32_t*)((char*)ws + p.seg_counts_off);
  a.seg_invalid = (int32_t*)((char*)ws + p.seg_invalid_off);
  a.counts = counts;
  a.offsets = offsets;
  a.splits = splits;
  a.src_row = src_row;
  a.dst_row = dst_row;
  a.dev_error = dev_error;
  a.T = s.T;
  a.k = s.k;
  a.E = s.E;
  a.G = s.G;
  a.N = s.N;
  a.Tc = s.Tc;
  a.spc = p.segs_per_chunk;
  a.seg = p.seg;
  if (s.E <= kFusedMaxE && (int64_t)s.Tc * s.k <= kFusedMaxIds &&
      (int64_t)s.T * s.k <= kFusedMaxAll) {
    hipLaunchKernelGGL(meta_fused, dim3((unsigned)s.N), dim3(1024), 0, st, a);
    return hipGetLastError();
  }
  const size_t lds_rank = (size_t)s.E * (sizeof(unsigned long long) + sizeof(int));
  if ((int64_t)s.Tc * s.k <= kHistScanMaxIds && (int64_t)s.T * s.k <= kFusedMaxAll) {
    hipLaunchKernelGGL(meta_hist_scan, dim3((unsigned)s.N), dim3(1024), 0, st, a);
    hipLaunchKernelGGL(meta_rank, dim3((unsigned)p.nseg), dim3(64), lds_rank, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(meta_hist, dim3((unsigned)p.nseg), dim3(64), (size_t)s.E * sizeof(int), st,
                     a);
  hipLaunchKernelGGL(meta_scan, dim3((unsigned)s.N), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(meta_rank, dim3((unsigned)p.nseg), dim3(64), lds_rank, st, a);
  return hipGetLastError();
}

}  // namespace moe
