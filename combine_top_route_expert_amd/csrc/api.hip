// C-ABI entry points: argument checks, workspace planning and the Chunk MoE
// two-stream schedules.  Every function only enqueues work; none synchronises
// with the device or copies anything to the host.
#include <mutex>
#include <vector>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kMaxChunks = 4096;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Layout of the moe_chunked_forward workspace.
struct FwdPlan {
  size_t counts, offsets, splits, src_row, dst_row, dev_err, sink, meta_ws;
  size_t slot[2];          // x_perm / y region of each slot
  size_t slot_act[2];      // act region of each slot
  size_t bytes;
  int nslots;
  MetaPlan meta;
};

FwdPlan fwd_plan(const Shape& s) {
  FwdPlan p{};
  size_t o = 0;
  auto take = [&](size_t n) {
    size_t at = o;
    o += align256(n);
    return at;
  };
  p.counts = take((size_t)s.N * s.E * 4);
  p.offsets = take((size_t)s.N * (s.E + 1) * 4);
  p.splits = take((size_t)s.N * s.G * 4);
  p.src_row = take((size_t)s.A * 4);
  p.dst_row = take((size_t)s.A * 4);
  p.dev_err = take(4);
  p.sink = take(4);  // the weight warm-up's scratch word
  p.meta = meta_plan(s);
  p.meta_ws = take(p.meta.bytes);
  const size_t rows = (size_t)s.Tc * s.k;
  p.nslots = s.N >= 2 ? 2 : 1;
  for (int i = 0; i < p.nslots; ++i) p.slot[i] = take(rows * s.H * s.elem);
  // act of both slots back to back: a fused pair uses it as one [2 rows][I] buffer
  const size_t act = take(p.nslots * rows * s.I * s.elem);
  for (int i = 0; i < p.nslots; ++i) p.slot_act[i] = act + i * rows * s.I * s.elem;
  p.bytes = o;
  return p;
}

// Layout of the moe_chunked_backward workspace: the forward's metadata, then
// per slot x_perm and a [rows][H] buffer that holds y, then grad_y, then
// grad_x_perm; act and the saved g/u (later grad_g/grad_u) of both slots back
// to back so a pair uses them as joint buffers.
struct BwdPlan {
  size_t counts, offsets, splits, src_row, dst_row, dev_err, meta_ws;
  size_t xp[2], yg[2], act, gu, order;
  size_t bytes;
  int nslots;
  MetaPlan meta;
};

BwdPlan bwd_plan(const Shape& s) {
  BwdPlan p{};
  size_t o = 0;
  auto take = [&](size_t n) {
    size_t at = o;
    o += align256(n);
    return at;
  };
  p.counts = take((size_t)s.N * s.E * 4);
  p.offsets = take((size_t)s.N * (s.E + 1) * 4);
  p.splits = take((size_t)s.N * s.G * 4);
  p.src_row = take((size_t)s.A * 4);
  p.dst_row = take((size_t)s.A * 4);
  p.dev_err = take(4);
  p.meta = meta_plan(s);
  p.meta_ws = take(p.meta.bytes);
  const size_t rows = (size_t)s.Tc * s.k;
  p.nslots = s.N >= 2 ? 2 : 1;
  for (int i = 0; i < p.nslots; ++i) {
    p.xp[i] = take(rows * s.H * s.elem);
    p.yg[i] = take(rows * s.H * s.elem);
  }
  p.act = take(p.nslots * rows * s.I * s.elem);
  p.gu = take(p.nslots * rows * 2 * s.I * s.elem);
  p.order = take((size_t)s.E * 4);  // experts by rows, for the weight-gradient tiles
  p.bytes = o;
  return p;
}

// Events that order s0 and s1, per device, cached per host thread.  A wait
// refers to the event's latest record at the time of the wait call, so one
// event can be recorded again for every pair.
constexpr int kEvents = 3;
struct DeviceEvents {
  int device = -1;
  hipEvent_t ev[kEvents] = {};
};

hipError_t thread_events(hipEvent_t (&out)[kEvents]) {
  thread_local std::vector<DeviceEvents> cache;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  for (auto& p : cache)
    if (p.device == dev) {
      for (int i = 0; i < kEvents; ++i) out[i] = p.ev[i];
      return hipSuccess;
    }
  DeviceEvents p;
  p.device = dev;
  for (auto& e : p.ev) {
    err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (err != hipSuccess) return err;
  }
  cache.push_back(p);
  for (int i = 0; i < kEvents; ++i) out[i] = p.ev[i];
  return hipSuccess;
}

// s_to waits for all work enqueued so far on s_from.
hipError_t join(hipStream_t s_to, hipStream_t s_from, hipEvent_t ev) {
  hipError_t he = hipEventRecord(ev, s_from);
  if (he == hipSuccess) he = hipStreamWaitEvent(s_to, ev, 0);
  return he;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_chunk(const Shape& s, int chunk, int* t0, int* t1) {
  if (chunk < 0 || chunk >= s.N) return MOE_ERR_INVALID_ARG;
  chunk_tokens(s, chunk, t0, t1);
  return MOE_OK;
}

moe_status gate_up(const Shape& s, const GroupedIO& io, const void* w, hipStream_t st) {
  return hip_status(s.dtype == MOE_BF16 ? launch_gate_up_bf16(s, io, w, st)
                                        : launch_gate_up_f32(s, io, w, st));
}

moe_status down(const Shape& s, const GroupedIO& io, const void* w, hipStream_t st) {
  return hip_status(s.dtype == MOE_BF16 ? launch_down_bf16(s, io, w, st)
                                        : launch_down_f32(s, io, w, st));
}

moe_status dgrad(const Shape& s, const DgradIO& io, hipStream_t st) {
  return hip_status(s.dtype == MOE_BF16 ? launch_dgrad_bf16(s, io, st)
                                        : launch_dgrad_f32(s, io, st));
}

moe_status wgrad(const Shape& s, const WgradIO& io, hipStream_t st) {
  return hip_status(s.dtype == MOE_BF16 ? launch_wgrad_bf16(s, io, st)
                                        : launch_wgrad_f32(s, io, st));
}

// One chunk: A and C are the chunk's own buffers.
GroupedIO single(const Shape& s, int64_t rows, const void* a, const int32_t* off_c, void* c) {
  GroupedIO io{};
  io.a[0] = a;
  io.c[0] = c;
  io.off[0] = off_c;
  io.rows_bound = rows;
  (void)s;
  return io;
}

// gate_up then down over both chunks of a pair (or one chunk when rows1 == 0):
// x_perm and y split over the two slots, act joint.
moe_status pair_ffn(const Shape& s, const int32_t* off0, const int32_t* off1, int64_t rows0,
                    int64_t rows1, const void* x0, const void* x1, const void* w_gate_up,
                    const void* w_down, void* act, void* y0, void* y1, hipStream_t st) {
  GroupedIO io{};
  io.off[0] = off0;
  io.off[1] = rows1 > 0 ? off1 : nullptr;
  io.rows_bound = rows0 + rows1;
  io.a[0] = x0;
  io.a[1] = x1;
  io.a_split = true;
  io.c[0] = act;
  io.c_split = false;
  moe_status r = gate_up(s, io, w_gate_up, st);
  if (r != MOE_OK) return r;
  io.a[0] = act;
  io.a[1] = nullptr;
  io.a_split = false;
  io.c[0] = y0;
  io.c[1] = y1;
  io.c_split = true;
  return down(s, io, w_down, st);
}

}  // namespace

moe_status resolve_shape(const moe_shape* in, Shape* s) {
  if (!in || !s) return MOE_ERR_INVALID_ARG;
  if (in->num_tokens < 0 || in->hidden <= 0 || in->intermediate <= 0 || in->top_k < 1 ||
      in->num_experts < 1)
    return MOE_ERR_INVALID_ARG;
  if (in->dtype != MOE_F32 && in->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  const int G = in->num_groups <= 0 ? 1 : in->num_groups;
  if (in->num_experts % G) return MOE_ERR_INVALID_ARG;
  const int N = in->num_chunks <= 0 ? 1 : in->num_chunks;
  if (in->top_k > 64 || in->num_experts > kMaxExperts || N > kMaxChunks) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)in->num_tokens * in->top_k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (in->dtype == MOE_BF16) {
    if (in->hidden % 64 || in->intermediate % 64) return MOE_ERR_UNSUPPORTED;
  } else {
    if (in->hidden % 4 || in->intermediate % 4) return MOE_ERR_UNSUPPORTED;
  }
  s->T = in->num_tokens;
  s->H = in->hidden;
  s->E = in->num_experts;
  s->k = in->top_k;
  s->I = in->intermediate;
  s->G = G;
  s->N = N;
  s->dtype = (moe_dtype)in->dtype;
  s->Tc = (int)(((int64_t)s->T + N - 1) / N);
  s->A = (int64_t)s->T * s->k;
  s->elem = in->dtype == MOE_BF16 ? 2 : 4;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

int32_t moe_resolve_num_chunks(int32_t num_tokens, int32_t num_chunks, int32_t chunk_size,
                               int32_t* warned) {
  if (warned) *warned = (num_chunks > 0 && chunk_size > 0) ? 1 : 0;
  if (num_chunks > 0) return num_chunks;
  if (chunk_size > 0) {
    const int64_t n = ((int64_t)(num_tokens > 0 ? num_tokens : 0) + chunk_size - 1) / chunk_size;
    return n < 1 ? 1 : (int32_t)n;
  }
  return 1;
}

moe_status moe_chunk_range(const moe_shape* shape, int32_t chunk, int32_t* t0, int32_t* t1) {
  Shape s;
  moe_status st = resolve_shape(shape, &s);
  if (st != MOE_OK) return st;
  if (!t0 || !t1) return MOE_ERR_INVALID_ARG;
  int a, b;
  st = check_chunk(s, chunk, &a, &b);
  if (st != MOE_OK) return st;
  *t0 = a;
  *t1 = b;
  return MOE_OK;
}

moe_status moe_route_meta_workspace_size(const moe_shape* shape, size_t* bytes) {
  Shape s;
  moe_status st = resolve_shape(shape, &s);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = meta_plan(s).bytes;
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes) {
  Shape s;
  moe_status st = resolve_shape(shape, &s);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = fwd_plan(s).bytes;
  return MOE_OK;
}

moe_status moe_route_meta(const moe_shape* shape, const int32_t* top_k_index, int32_t* counts,
                          int32_t* offsets, int32_t* group_splits, int32_t* src_row,
                          int32_t* dst_row, int32_t* dev_error, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  Shape s;
  moe_status st = resolve_shape(shape, &s);
  if (st != MOE_OK) return st;
  if (!counts || !offsets || !group_splits || !ws) return MOE_ERR_INVALID_ARG;
  if (s.A > 0 && (!top_k_index || !src_row || !dst_row)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {top_k_index, counts, offsets, group_splits, src_row, dst_row, dev_error};
  for (const void* p : ptrs)
    if (!aligned(p, 4)) return MOE_ERR_INVALID_ARG;
  if (!aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < meta_plan(s).bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(launch_route_meta(s, top_k_index, counts, offsets, group_splits, src_row,
                                      dst_row, dev_error, ws, stream));
}

moe_status moe_permute(const moe_shape* shape, int32_t chunk, const void* hidden_states,
                       const int32_t* dst_row, void* x_perm, hipStream_t stream) {
  Shape s;
  int t0, t1;
  moe_status st = resolve_shape(shape, &s);
  if (st == MOE_OK) st = check_chunk(s, chunk, &t0, &t1);
  if (st != MOE_OK) return st;
  if (t1 == t0) return MOE_OK;
  if (!hidden_states || !dst_row || !x_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned(hidden_states, 16) || !aligned(x_perm, 16) || !aligned(dst_row, 4))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_permute(s, t0, t1, hidden_states, dst_row, x_perm, stream));
}

moe_status moe_expert_gate_up(const moe_shape* shape, int32_t chunk, const void* x_perm,
                              const int32_t* offsets, const void* w_gate_up, void* act,
                              hipStream_t stream) {
  Shape s;
  int t0, t1;
  moe_status st = resolve_shape(shape, &s);
  if (st == MOE_OK) st = check_chunk(s, chunk, &t0, &t1);
  if (st != MOE_OK) return st;
  if (t1 == t0) return MOE_OK;
  if (!x_perm || !offsets || !w_gate_up || !act) return MOE_ERR_INVALID_ARG;
  if (!aligned(x_perm, 16) || !aligned(w_gate_up, 16) || !aligned(act, 16) ||
      !aligned(offsets, 4))
    return MOE_ERR_INVALID_ARG;
  return gate_up(s, single(s, (int64_t)(t1 - t0) * s.k, x_perm,
                           offsets + (size_t)chunk * (s.E + 1), act),
                 w_gate_up, stream);
}

moe_status moe_expert_down(const moe_shape* shape, int32_t chunk, const void* act,
                           const int32_t* offsets, const void* w_down, void* y,
                           hipStream_t stream) {
  Shape s;
  int t0, t1;
  moe_status st = resolve_shape(shape, &s);
  if (st == MOE_OK) st = check_chunk(s, chunk, &t0, &t1);
  if (st != MOE_OK) return st;
  if (t1 == t0) return MOE_OK;
  if (!act || !offsets || !w_down || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned(act, 16) || !aligned(w_down, 16) || !aligned(y, 16) || !aligned(offsets, 4))
    return MOE_ERR_INVALID_ARG;
  return down(s, single(s, (int64_t)(t1 - t0) * s.k, act, offsets + (size_t)chunk * (s.E + 1), y),
              w_down, stream);
}

moe_status moe_expert_ffn(const moe_shape* shape, int32_t chunk, const void* x_perm,
                          const int32_t* offsets, const void* w_gate_up, const void* w_down,
                          void* act, void* y, hipStream_t stream) {
  moe_status st = moe_expert_gate_up(shape, chunk, x_perm, offsets, w_gate_up, act, stream);
  if (st != MOE_OK) return st;
  return moe_expert_down(shape, chunk, act, offsets, w_down, y, stream);
}

namespace moe {
namespace {

// Checks shared by the pair entry points; fills the pair's offsets and row counts.
moe_status pair_args(const moe_shape* shape, int32_t chunk, Shape* s, const int32_t* offsets,
                     const int32_t** off0, const int32_t** off1, int64_t* rows0,
                     int64_t* rows1) {
  int t0, t1, u0 = 0, u1 = 0;
  moe_status st = resolve_shape(shape, s);
  if (st == MOE_OK) st = check_chunk(*s, chunk, &t0, &t1);
  if (st != MOE_OK) return st;
  if (chunk + 1 < s->N) chunk_tokens(*s, chunk + 1, &u0, &u1);
  *rows0 = (int64_t)(t1 - t0) * s->k;
  *rows1 = (int64_t)(u1 - u0) * s->k;
  if (*rows0 + *rows1 == 0) return MOE_OK;
  if (!offsets || !aligned(offsets, 4)) return MOE_ERR_INVALID_ARG;
  *off0 = offsets + (size_t)chunk * (s->E + 1);
  *off1 = *rows1 > 0 ? *off0 + (s->E + 1) : nullptr;
  return MOE_OK;
}

// A chunk buffer: required and 16-byte aligned when its chunk has rows.
bool buf_ok(const void* p, int64_t rows) { return rows == 0 || (p && aligned(p, 16)); }

}  // namespace
}  // namespace moe

moe_status moe_expert_gate_up_pair(const moe_shape* shape, int32_t chunk, const void* x_perm0,
                                   const void* x_perm1, const int32_t* offsets,
                                   const void* w_gate_up, void* act, hipStream_t stream) {
  Shape s;
  const int32_t *off0 = nullptr, *off1 = nullptr;
  int64_t rows0 = 0, rows1 = 0;
  moe_status st = pair_args(shape, chunk, &s, offsets, &off0, &off1, &rows0, &rows1);
  if (st != MOE_OK || rows0 + rows1 == 0) return st;
  if (!buf_ok(x_perm0, rows0) || !buf_ok(x_perm1, rows1) || !buf_ok(act, 1) ||
      !buf_ok(w_gate_up, 1))
    return MOE_ERR_INVALID_ARG;
  GroupedIO io{};
  io.off[0] = off0;
  io.off[1] = off1;
  io.rows_bound = rows0 + rows1;
  io.a[0] = x_perm0;
  io.a[1] = x_perm1;
  io.a_split = true;
  io.c[0] = act;
  return gate_up(s, io, w_gate_up, stream);
}

moe_status moe_expert_gate_up_gather_pair(const moe_shape* shape, int32_t chunk,
                                          const void* hidden_states, const int32_t* src_row,
                                          const int32_t* offsets, const void* w_gate_up,
                                          void* act, hipStream_t stream) {
  Shape s;
  const int32_t *off0 = nullptr, *off1 = nullptr;
  int64_t rows0 = 0, rows1 = 0;
  moe_status st = pair_args(shape, chunk, &s, offsets, &off0, &off1, &rows0, &rows1);
  if (st != MOE_OK || rows0 + rows1 == 0) return st;
  if (!buf_ok(hidden_states, 1) || !buf_ok(act, 1) || !buf_ok(w_gate_up, 1) || !src_row ||
      !aligned(src_row, 4))
    return MOE_ERR_INVALID_ARG;
  int t0, t1, u0 = 0, u1 = 0;
  chunk_tokens(s, chunk, &t0, &t1);
  if (chunk + 1 < s.N) chunk_tokens(s, chunk + 1, &u0, &u1);
  GroupedIO io{};
  io.off[0] = off0;
  io.off[1] = off1;
  io.rows_bound = rows0 + rows1;
  io.a[0] = hidden_states;
  io.gather[0] = src_row + (size_t)t0 * s.k;
  io.gather[1] = src_row + (size_t)u0 * s.k;
  io.gather_k = s.k;
  io.c[0] = act;
  return gate_up(s, io, w_gate_up, stream);
}

moe_status moe_expert_down_pair(const moe_shape* shape, int32_t chunk, const void* act,
                                const int32_t* offsets, const void* w_down, void* y0, void* y1,
                                hipStream_t stream) {
  Shape s;
  const int32_t *off0 = nullptr, *off1 = nullptr;
  int64_t rows0 = 0, rows1 = 0;
  moe_status st = pair_args(shape, chunk, &s, offsets, &off0, &off1, &rows0, &rows1);
  if (st != MOE_OK || rows0 + rows1 == 0) return st;
  if (!buf_ok(y0, rows0) || !buf_ok(y1, rows1) || !buf_ok(act, 1) || !buf_ok(w_down, 1))
    return MOE_ERR_INVALID_ARG;
  GroupedIO io{};
  io.off[0] = off0;
  io.off[1] = off1;
  io.rows_bound = rows0 + rows1;
  io.a[0] = act;
  io.c[0] = y0;
  io.c[1] = y1;
  io.c_split = true;
  return down(s, io, w_down, stream);
}

moe_status moe_expert_ffn_pair(const moe_shape* shape, int32_t chunk, const void* x_perm0,
                               const void* x_perm1, const int32_t* offsets,
                               const void* w_gate_up, const void* w_down, void* act, void* y0,
                               void* y1, hipStream_t stream) {
  Shape s;
  const int32_t *off0 = nullptr, *off1 = nullptr;
  int64_t rows0 = 0, rows1 = 0;
  moe_status st = pair_args(shape, chunk, &s, offsets, &off0, &off1, &rows0, &rows1);
  if (st != MOE_OK || rows0 + rows1 == 0) return st;
  // every argument of both launches is checked before the first is enqueued
  if (!buf_ok(x_perm0, rows0) || !buf_ok(x_perm1, rows1) || !buf_ok(y0, rows0) ||
      !buf_ok(y1, rows1) || !buf_ok(act, 1) || !buf_ok(w_gate_up, 1) || !buf_ok(w_down, 1))
    return MOE_ERR_INVALID_ARG;
  return pair_ffn(s, off0, off1, rows0, rows1, x_perm0, x_perm1, w_gate_up, w_down, act, y0, y1,
                  stream);
}

moe_status moe_unpermute_combine(const moe_shape* shape, int32_t chunk, const void* y,
                                 const int32_t* dst_row, const float* top_k_weights, void* out,
                                 hipStream_t stream) {
  Shape s;
  int t0, t1;
  moe_status st = resolve_shape(shape, &s);
  if (st == MOE_OK) st = check_chunk(s, chunk, &t0, &t1);
  if (st != MOE_OK) return st;
  if (t1 == t0) return MOE_OK;
  if (!y || !dst_row || !top_k_weights || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(dst_row, 4) || !aligned(top_k_weights, 4))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(s, t0, t1, y, dst_row, top_k_weights, out, stream));
}

moe_status moe_unpermute_combine_backward(const moe_shape* shape, int32_t chunk,
                                          const void* grad_out, const void* y,
                                          const int32_t* dst_row, const float* top_k_weights,
                                          void* grad_y, float* grad_top_k_weights,
                                          hipStream_t stream) {
  Shape s;
  int t0, t1;
  moe_status st = resolve_shape(shape, &s);
  if (st == MOE_OK) st = check_chunk(s, chunk, &t0, &t1);
  if (st != MOE_OK) return st;
  if (t1 == t0) return MOE_OK;
  if (!grad_out || !y || !dst_row || !top_k_weights || !grad_y || !grad_top_k_weights)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(grad_out, 16) || !aligned(y, 16) || !aligned(grad_y, 16) ||
      !aligned(dst_row, 4) || !aligned(top_k_weights, 4) || !aligned(grad_top_k_weights, 4))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine_backward(s, t0, t1, grad_out, y, dst_row, top_k_weights,
                                            grad_y, grad_top_k_weights, stream));
}

moe_status moe_permute_backward(const moe_shape* shape, int32_t chunk, const void* grad_x_perm,
                                const int32_t* dst_row, void* grad_hidden, hipStream_t stream) {
  Shape s;
  int t0, t1;
  moe_status st = resolve_shape(shape, &s);
  if (st == MOE_OK) st = check_chunk(s, chunk, &t0, &t1);
  if (st != MOE_OK) return st;
  if (t1 == t0) return MOE_OK;
  if (!grad_x_perm || !dst_row || !grad_hidden) return MOE_ERR_INVALID_ARG;
  if (!aligned(grad_x_perm, 16) || !aligned(grad_hidden, 16) || !aligned(dst_row, 4))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(s, t0, t1, grad_x_perm, dst_row, nullptr, grad_hidden, stream));
}

moe_status moe_backward_workspace_size(const moe_shape* shape, size_t* bytes) {
  Shape s;
  moe_status st = resolve_shape(shape, &s);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = bwd_plan(s).bytes;
  return MOE_OK;
}

moe_status moe_chunked_backward(const moe_shape* shape, const void* hidden_states,
                                const int32_t* top_k_index, const float* top_k_weights,
                                const void* w_gate_up, const void* w_down, const void* grad_out,
                                void* grad_hidden, float* grad_top_k_weights,
                                float* grad_w_gate_up, float* grad_w_down, int32_t* dev_error,
                                void* ws, size_t ws_bytes, hipStream_t s0, hipStream_t s1) {
  Shape s;
  moe_status st = resolve_shape(shape, &s);
  if (st != MOE_OK) return st;
  if (!ws || !aligned(ws, 256) || !aligned(dev_error, 4)) return MOE_ERR_INVALID_ARG;
  const BwdPlan p = bwd_plan(s);
  if (ws_bytes < p.bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!w_gate_up || !w_down || !grad_w_gate_up || !grad_w_down) return MOE_ERR_INVALID_ARG;
  if (!aligned(w_gate_up, 16) || !aligned(w_down, 16) || !aligned(grad_w_gate_up, 16) ||
      !aligned(grad_w_down, 16))
    return MOE_ERR_INVALID_ARG;
  if (s.T > 0) {
    if (!hidden_states || !top_k_index || !top_k_weights || !grad_out || !grad_hidden ||
        !grad_top_k_weights)
      return MOE_ERR_INVALID_ARG;
    if (!aligned(hidden_states, 16) || !aligned(grad_out, 16) || !aligned(grad_hidden, 16) ||
        !aligned(top_k_index, 4) || !aligned(top_k_weights, 4) ||
        !aligned(grad_top_k_weights, 4))
      return MOE_ERR_INVALID_ARG;
  }
  char* w = (char*)ws;
  int32_t* counts = (int32_t*)(w + p.counts);
  int32_t* offsets = (int32_t*)(w + p.offsets);
  int32_t* splits = (int32_t*)(w + p.splits);
  int32_t* src_row = (int32_t*)(w + p.src_row);
  int32_t* dst_row = (int32_t*)(w + p.dst_row);
  int32_t* err = dev_error ? dev_error : (int32_t*)(w + p.dev_err);
  hipError_t he = launch_route_meta(s, top_k_index, counts, offsets, splits, src_row, dst_row,
                                    err, w + p.meta_ws, s0);
  if (he != hipSuccess) return MOE_ERR_HIP;

  // Every step runs on s0: as in the pair-fused forward, the joins that
  // would let a pair's second permute / combine backward / permute backward
  // run on s1 cost more than that overlap gains.  s1 is accepted for the
  // interface's sake.
  (void)s1;
  bool first = true;
  auto chunk_rows = [&](int c, int* t0, int* t1) {
    *t0 = *t1 = 0;
    if (c < s.N) chunk_tokens(s, c, t0, t1);
    return (int64_t)(*t1 - *t0) * s.k;
  };
  // Pair (c, c+1): both permutes, gate_up (act and the saved g/u), down (y),
  // both combine backwards, the dgrad of down with the SwiGLU backward
  // (grad_g/grad_u over g/u), the W_d wgrad, the gate/up dgrad (grad_x over y's
  // buffer), the W_gu wgrad, then both permute backwards.
  for (int c = 0; c < s.N; c += 2) {
    int t0, t1, u0, u1;
    const int64_t rows0 = chunk_rows(c, &t0, &t1), rows1 = chunk_rows(c + 1, &u0, &u1);
    if (rows0 + rows1 == 0) continue;
    void* xp0 = w + p.xp[0];
    void* xp1 = p.nslots > 1 ? w + p.xp[1] : nullptr;
    void* yg0 = w + p.yg[0];
    void* yg1 = p.nslots > 1 ? w + p.yg[1] : nullptr;
    const int32_t* off0 = offsets + (size_t)c * (s.E + 1);
    const int32_t* off1 = rows1 > 0 ? off0 + (s.E + 1) : nullptr;
    he = launch_permute(s, t0, t1, hidden_states, dst_row, xp0, s0);
    if (he == hipSuccess && rows1 > 0) he = launch_permute(s, u0, u1, hidden_states, dst_row, xp1, s0);
    if (he != hipSuccess) return MOE_ERR_HIP;
    // forward recompute: act + saved g/u, then y
    GroupedIO io{};
    io.off[0] = off0;
    io.off[1] = off1;
    io.rows_bound = rows0 + rows1;
    io.a[0] = xp0;
    io.a[1] = xp1;
    io.a_split = true;
    io.c[0] = w + p.act;
    io.gu = w + p.gu;
    st = gate_up(s, io, w_gate_up, s0);
    if (st != MOE_OK) return st;
    io.gu = nullptr;
    io.a[0] = w + p.act;
    io.a[1] = nullptr;
    io.a_split = false;
    io.c[0] = yg0;
    io.c[1] = yg1;
    io.c_split = true;
    st = down(s, io, w_down, s0);
    if (st != MOE_OK) return st;
    // combine backward: grad_w rows of the pair's tokens, grad_y over y
    he = launch_combine_backward(s, t0, t1, grad_out, yg0, dst_row, top_k_weights, yg0,
                                 grad_top_k_weights, s0);
    if (he == hipSuccess && rows1 > 0)
      he = launch_combine_backward(s, u0, u1, grad_out, yg1, dst_row, top_k_weights, yg1,
                                   grad_top_k_weights, s0);
    if (he != hipSuccess) return MOE_ERR_HIP;
    // dgrad of down with the SwiGLU backward: g/u -> grad_g/grad_u
    DgradIO dd{};
    dd.a[0] = yg0;
    dd.a[1] = yg1;
    dd.a_split = true;
    dd.B = w_down;
    dd.K = s.H;
    dd.N = s.I;
    dd.gu = w + p.gu;
    dd.off[0] = off0;
    dd.off[1] = off1;
    dd.rows_bound = rows0 + rows1;
    st = dgrad(s, dd, s0);
    if (st != MOE_OK) return st;
    // the weight-gradient tiles are dealt largest expert first
    int32_t* order = (int32_t*)(w + p.order);
    he = launch_expert_order(s, off0, off1, order, s0);
    if (he != hipSuccess) return MOE_ERR_HIP;
    // W_d wgrad reads grad_y and act
    WgradIO wd{};
    wd.a[0] = yg0;
    wd.a[1] = yg1;
    wd.a_split = true;
    wd.b[0] = w + p.act;
    wd.C = grad_w_down;
    wd.M = s.H;
    wd.N = s.I;
    wd.accumulate = first ? 0 : 1;
    wd.off[0] = off0;
    wd.off[1] = off1;
    wd.order = order;
    st = wgrad(s, wd, s0);
    if (st != MOE_OK) return st;
    // gate/up dgrad: grad_x over y's (now free) buffer
    DgradIO dg{};
    dg.a[0] = w + p.gu;
    dg.a_split = false;
    dg.B = w_gate_up;
    dg.K = 2 * s.I;
    dg.N = s.H;
    dg.c[0] = yg0;
    dg.c[1] = yg1;
    dg.c_split = true;
    dg.off[0] = off0;
    dg.off[1] = off1;
    dg.rows_bound = rows0 + rows1;
    st = dgrad(s, dg, s0);
    if (st != MOE_OK) return st;
    // W_gu wgrad reads grad_g/grad_u and x_perm
    WgradIO wg{};
    wg.a[0] = w + p.gu;
    wg.a_split = false;
    wg.b[0] = xp0;
    wg.b[1] = xp1;
    wg.b_split = true;
    wg.C = grad_w_gate_up;
    wg.M = 2 * s.I;
    wg.N = s.H;
    wg.accumulate = first ? 0 : 1;
    wg.off[0] = off0;
    wg.off[1] = off1;
    wg.order = order;
    st = wgrad(s, wg, s0);
    if (st != MOE_OK) return st;
    first = false;
    // permute backward: grad_hidden[t] = sum_j grad_x[dst_row[t*k+j]]
    he = rows1 > 0 ? launch_combine_pair(s, t0, u0, u1, yg0, yg1, dst_row, nullptr, grad_hidden,
                                         s0)
                   : launch_combine(s, t0, t1, yg0, dst_row, nullptr, grad_hidden, s0);
    if (he != hipSuccess) return MOE_ERR_HIP;
  }
  if (first) {
    // no rows at all: the weight gradients are zero
    WgradIO z{};
    z.a[0] = w + p.act;
    z.b[0] = w + p.act;
    z.off[0] = offsets;
    z.accumulate = 0;
    z.C = grad_w_down;
    z.M = s.H;
    z.N = s.I;
    st = wgrad(s, z, s0);
    if (st != MOE_OK) return st;
    z.C = grad_w_gate_up;
    z.M = 2 * s.I;
    z.N = s.H;
    st = wgrad(s, z, s0);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_chunked_forward_schedule(const moe_shape* shape, const void* hidden_states,
                                        const int32_t* top_k_index, const float* top_k_weights,
                                        const void* w_gate_up, const void* w_down, void* out,
                                        int32_t* dev_error, void* ws, size_t ws_bytes,
                                        hipStream_t s0, hipStream_t s1, int32_t schedule) {
  Shape s;
  moe_status st = resolve_shape(shape, &s);
  if (st != MOE_OK) return st;
  if (schedule != MOE_SCHEDULE_PAIR_FUSED && schedule != MOE_SCHEDULE_PER_CHUNK &&
      schedule != MOE_SCHEDULE_PAIR_FUSED_PREFETCH && schedule != MOE_SCHEDULE_EXPERT_HALVES)
    return MOE_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
  if (!aligned(dev_error, 4)) return MOE_ERR_INVALID_ARG;
  const FwdPlan p = fwd_plan(s);
  if (ws_bytes < p.bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (s.T > 0) {
    if (!hidden_states || !top_k_index || !top_k_weights || !w_gate_up || !w_down || !out)
      return MOE_ERR_INVALID_ARG;
    if (!aligned(hidden_states, 16) || !aligned(out, 16) || !aligned(w_gate_up, 16) ||
        !aligned(w_down, 16) || !aligned(top_k_index, 4) || !aligned(top_k_weights, 4))
      return MOE_ERR_INVALID_ARG;
  }
  char* w = (char*)ws;
  int32_t* counts = (int32_t*)(w + p.counts);
  int32_t* offsets = (int32_t*)(w + p.offsets);
  int32_t* splits = (int32_t*)(w + p.splits);
  int32_t* src_row = (int32_t*)(w + p.src_row);
  int32_t* dst_row = (int32_t*)(w + p.dst_row);
  int32_t* err = dev_error ? dev_error : (int32_t*)(w + p.dev_err);

  // the prefetch schedule: s1 (ordered after the caller's work on s0) warms the
  // head of every gate/up weight row while s0 runs the metadata pass
  const bool warm = (schedule == MOE_SCHEDULE_PAIR_FUSED_PREFETCH && s1 != nullptr &&
                     s1 != s0 && s.T > 0);
  hipEvent_t ev[kEvents] = {};
  hipError_t he = hipSuccess;
  if (warm) {
    he = thread_events(ev);
    if (he == hipSuccess) he = join(s1, s0, ev[2]);
    const int64_t row_bytes = (int64_t)s.H * s.elem;
    if (he == hipSuccess)
      he = launch_warm_weights(w_gate_up, (int64_t)s.E * 2 * s.I, row_bytes,
                               (int)(row_bytes < 128 ? row_bytes : 128),
                               (int32_t*)(w + p.sink), s1);
    if (he != hipSuccess) return MOE_ERR_HIP;
  }

  // one metadata pass for every chunk, on s0
  he = launch_route_meta(s, top_k_index, counts, offsets, splits, src_row, dst_row, err,
                         w + p.meta_ws, s0);
  if (he != hipSuccess) return MOE_ERR_HIP;
  if (s.T == 0) return MOE_OK;

  // the per-chunk schedule runs odd chunks on s1
  const bool two = (s1 != nullptr && s1 != s0 && s.N >= 2 &&
                    schedule == MOE_SCHEDULE_PER_CHUNK);
  if (two) {
    he = thread_events(ev);
    if (he == hipSuccess) he = join(s1, s0, ev[0]);  // s1 starts after the metadata
    if (he != hipSuccess) return MOE_ERR_HIP;
  }
  // the expert-halves schedule: each pair's expert GEMMs in two launches over
  // experts [0, E/2) and [E/2, E), the first half's down on s1 beside the second
  // half's gate_up on s0
  const bool halves = schedule == MOE_SCHEDULE_EXPERT_HALVES && s1 != nullptr && s1 != s0 &&
                      s.E >= 2;
  if (halves) {
    he = thread_events(ev);
    if (he != hipSuccess) return MOE_ERR_HIP;
  }
  bool used_s1 = false;
  auto chunk_rows = [&](int c, int* t0, int* t1) {
    *t0 = *t1 = 0;
    if (c < s.N) chunk_tokens(s, c, t0, t1);
    return (int64_t)(*t1 - *t0) * s.k;
  };

  if (schedule != MOE_SCHEDULE_PER_CHUNK) {
    // Pair (c, c+1): one gate_up launch over the pair's rows (gathering them
    // from hidden_states), one down launch, one combine launch for both
    // chunks, all on s0.  Every expert's weights are streamed once per pair.
    // (Running the second chunk's steps on s1 measured slower: the stream
    // joins cost more than overlapping two memory-bound kernels gains.)
    for (int c = 0; c < s.N; c += 2) {
      int t0, t1, u0, u1;
      const int64_t rows0 = chunk_rows(c, &t0, &t1), rows1 = chunk_rows(c + 1, &u0, &u1);
      if (rows0 + rows1 == 0) continue;  // empty tail pair
      void* xy0 = w + p.slot[0];
      void* xy1 = p.nslots > 1 ? w + p.slot[1] : nullptr;
      const int32_t* off0 = offsets + (size_t)c * (s.E + 1);
      // gate_up gathers its rows straight from hidden_states through src_row
      // (the permute fused into the GEMM's row addressing: same rows, same
      // bits, no x_perm round trip); down writes y into the slots
      GroupedIO io{};
      io.off[0] = off0;
      io.off[1] = rows1 > 0 ? off0 + (s.E + 1) : nullptr;
      io.rows_bound = rows0 + rows1;
      io.a[0] = hidden_states;
      io.gather[0] = src_row + (size_t)t0 * s.k;
      io.gather[1] = src_row + (size_t)u0 * s.k;
      io.gather_k = s.k;
      io.c[0] = w + p.slot_act[0];
      GroupedIO dn{};
      dn.off[0] = io.off[0];
      dn.off[1] = io.off[1];
      dn.rows_bound = io.rows_bound;
      dn.a[0] = w + p.slot_act[0];
      dn.c[0] = xy0;
      dn.c[1] = xy1;
      dn.c_split = true;
      if (!halves) {
        st = gate_up(s, io, w_gate_up, s0);
        if (st != MOE_OK) return st;
        st = down(s, dn, w_down, s0);
        if (st != MOE_OK) return st;
      } else {
        // Experts [e0, e1) of the same launches: the offsets from e0 on, the
        // weights of expert e0 on (every row index stays absolute).  The halves
        // touch disjoint rows of act and y, so only each half's gate_up -> down
        // order matters; the row bound stays the pair's.
        auto part = [&](const GroupedIO& g, int e0) {
          GroupedIO h = g;
          h.off[0] = g.off[0] + e0;
          h.off[1] = g.off[1] ? g.off[1] + e0 : nullptr;
          return h;
        };
        const int eh = s.E / 2;
        Shape sa = s, sb = s;
        sa.E = eh;
        sb.E = s.E - eh;
        const char* wgu1 = (const char*)w_gate_up + (size_t)eh * 2 * s.I * s.H * s.elem;
        const char* wd1 = (const char*)w_down + (size_t)eh * s.H * s.I * s.elem;
        st = gate_up(sa, part(io, 0), w_gate_up, s0);
        if (st != MOE_OK) return st;
        if (join(s1, s0, ev[0]) != hipSuccess) return MOE_ERR_HIP;  // first half's act ready
        st = down(sa, part(dn, 0), w_down, s1);
        if (st != MOE_OK) return st;
        used_s1 = true;
        st = gate_up(sb, part(io, eh), wgu1, s0);
        if (st != MOE_OK) return st;
        st = down(sb, part(dn, eh), wd1, s0);
        if (st != MOE_OK) return st;
        if (join(s0, s1, ev[1]) != hipSuccess) return MOE_ERR_HIP;  // first half's y ready
      }
      he = rows1 > 0 ? launch_combine_pair(s, t0, u0, u1, xy0, xy1, dst_row, top_k_weights,
                                           out, s0)
                     : launch_combine(s, t0, t1, xy0, dst_row, top_k_weights, out, s0);
      if (he != hipSuccess) return MOE_ERR_HIP;
    }
  } else {
    // Chunk c: permute -> gate_up -> down -> combine on stream s[c % 2], slot c % 2.
    for (int c = 0; c < s.N; ++c) {
      int t0, t1;
      const int64_t rows = chunk_rows(c, &t0, &t1);
      if (rows == 0) continue;  // empty tail chunk: nothing to launch
      const int slot = c % p.nslots;
      hipStream_t st_c = (two && (c & 1)) ? s1 : s0;
      used_s1 |= (st_c == s1 && two);
      void* xy = w + p.slot[slot];
      void* act = w + p.slot_act[slot];
      const int32_t* off_c = offsets + (size_t)c * (s.E + 1);
      he = launch_permute(s, t0, t1, hidden_states, dst_row, xy, st_c);
      if (he != hipSuccess) return MOE_ERR_HIP;
      st = gate_up(s, single(s, rows, xy, off_c, act), w_gate_up, st_c);
      if (st != MOE_OK) return st;
      st = down(s, single(s, rows, act, off_c, xy), w_down, st_c);  // y overwrites x_perm
      if (st != MOE_OK) return st;
      he = launch_combine(s, t0, t1, xy, dst_row, top_k_weights, out, st_c);
      if (he != hipSuccess) return MOE_ERR_HIP;
    }
  }
  if ((two && used_s1) || warm) {
    he = join(s0, s1, ev[1]);  // s0 is ordered after everything on s1
    if (he != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status moe_chunked_forward(const moe_shape* shape, const void* hidden_states,
                               const int32_t* top_k_index, const float* top_k_weights,
                               const void* w_gate_up, const void* w_down, void* out,
                               int32_t* dev_error, void* ws, size_t ws_bytes, hipStream_t s0,
                               hipStream_t s1) {
  return moe_chunked_forward_schedule(shape, hidden_states, top_k_index, top_k_weights,
                                      w_gate_up, w_down, out, dev_error, ws, ws_bytes, s0, s1,
                                      MOE_SCHEDULE_PAIR_FUSED);
}

}  // extern "C"
