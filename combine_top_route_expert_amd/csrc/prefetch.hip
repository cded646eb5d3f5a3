// Weight warm-up for the prefetch schedule (MOE_SCHEDULE_PAIR_FUSED_PREFETCH).
//
// The Ascend dual-stream article (section "02 Weight預取雙流並行") prefetches the
// decode stage's expert weights into cache on a second stream while the first
// stream is busy with communication, so that the matrix products find them
// there.  On one GPU the only stretch before the expert GEMMs in which HBM is
// otherwise idle is the routing-metadata pass; this kernel runs beside it on the
// second stream and reads the head (the first head_bytes) of every weight row,
// which is where every gate/up tile starts streaming its panel, so that those
// lines are in the MALL (and the reading XCD's L2) when the GEMM begins.
//
// One 16-byte load per lane, eight consecutive lanes per 128-byte row head, so
// each instruction covers whole lines.  The loaded words are folded into one
// value that is stored to `sink` only if it equals an arbitrary constant, which
// keeps the loads without writing anything in practice (a store, if it ever
// happens, goes to a scratch word nobody reads).
#include "moe_internal.h"

namespace moe {
namespace {

__global__ void __launch_bounds__(256) warm_rows(const char* __restrict__ w, int64_t rows,
                                                 int64_t row_bytes, int pieces,
                                                 int32_t* __restrict__ sink) {
  const int64_t n = rows * pieces;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / pieces;
    const int pc = (int)(i - r * pieces);
    const uint4 v = *(const uint4*)(w + r * row_bytes + (int64_t)pc * 16);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = (int32_t)acc;
}

}  // namespace

hipError_t launch_warm_weights(const void* w, int64_t rows, int64_t row_bytes, int head_bytes,
                               int32_t* sink, hipStream_t st) {
  const int pieces = head_bytes / 16;
  if (rows <= 0 || pieces <= 0) return hipSuccess;
  const int64_t n = rows * pieces;
  int64_t grid = (n + 255) / 256;
  if (grid > 4096) grid = 4096;  // 16 workgroups per CU, grid-stride beyond that
  hipLaunchKernelGGL(warm_rows, dim3((unsigned)grid), dim3(256), 0, st, (const char*)w, rows,
                     row_bytes, pieces, sink);
  return hipGetLastError();
}

}  // namespace moe
