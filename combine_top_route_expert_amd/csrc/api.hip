// C-ABI entry points: argument checks, workspace planning and the Chunk MoE
// two-stream schedule.  Every function only enqueues work; none synchronises
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
  size_t counts, offsets, splits, src_row, dst_row, dev_err, meta_ws;
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
  p.meta = meta_plan(s);
  p.meta_ws = take(p.meta.bytes);
  const size_t rows = (size_t)s.Tc * s.k;
  p.nslots = s.N >= 2 ? 2 : 1;
  for (int i = 0; i < p.nslots; ++i) {
    p.slot[i] = take(rows * s.H * s.elem);
    p.slot_act[i] = take(rows * s.I * s.elem);
  }
  p.bytes = o;
  return p;
}

// Two events per device, cached per host thread (used only to order s0/s1).
struct EventPair {
  int device = -1;
  hipEvent_t ev[2] = {nullptr, nullptr};
};

hipError_t thread_events(hipEvent_t* meta_done, hipEvent_t* s1_done) {
  thread_local std::vector<EventPair> cache;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  for (auto& p : cache)
    if (p.device == dev) {
      *meta_done = p.ev[0];
      *s1_done = p.ev[1];
      return hipSuccess;
    }
  EventPair p;
  p.device = dev;
  for (auto& e : p.ev) {
    err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (err != hipSuccess) return err;
  }
  cache.push_back(p);
  *meta_done = p.ev[0];
  *s1_done = p.ev[1];
  return hipSuccess;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_chunk(const Shape& s, int chunk, int* t0, int* t1) {
  if (chunk < 0 || chunk >= s.N) return MOE_ERR_INVALID_ARG;
  chunk_tokens(s, chunk, t0, t1);
  return MOE_OK;
}

moe_status gate_up(const Shape& s, int64_t rows, const void* x, const int32_t* off,
                   const void* w, void* act, hipStream_t st) {
  return hip_status(s.dtype == MOE_BF16 ? launch_gate_up_bf16(s, rows, x, off, w, act, st)
                                        : launch_gate_up_f32(s, rows, x, off, w, act, st));
}

moe_status down(const Shape& s, int64_t rows, const void* act, const int32_t* off,
                const void* w, void* y, hipStream_t st) {
  return hip_status(s.dtype == MOE_BF16 ? launch_down_bf16(s, rows, act, off, w, y, st)
                                        : launch_down_f32(s, rows, act, off, w, y, st));
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
  return gate_up(s, (int64_t)(t1 - t0) * s.k, x_perm, offsets + (size_t)chunk * (s.E + 1),
                 w_gate_up, act, stream);
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
  return down(s, (int64_t)(t1 - t0) * s.k, act, offsets + (size_t)chunk * (s.E + 1), w_down, y,
              stream);
}

moe_status moe_expert_ffn(const moe_shape* shape, int32_t chunk, const void* x_perm,
                          const int32_t* offsets, const void* w_gate_up, const void* w_down,
                          void* act, void* y, hipStream_t stream) {
  moe_status st = moe_expert_gate_up(shape, chunk, x_perm, offsets, w_gate_up, act, stream);
  if (st != MOE_OK) return st;
  return moe_expert_down(shape, chunk, act, offsets, w_down, y, stream);
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

moe_status moe_chunked_forward(const moe_shape* shape, const void* hidden_states,
                               const int32_t* top_k_index, const float* top_k_weights,
                               const void* w_gate_up, const void* w_down, void* out,
                               int32_t* dev_error, void* ws, size_t ws_bytes, hipStream_t s0,
                               hipStream_t s1) {
  Shape s;
  moe_status st = resolve_shape(shape, &s);
  if (st != MOE_OK) return st;
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

  // one metadata pass for every chunk, on s0
  hipError_t he = launch_route_meta(s, top_k_index, counts, offsets, splits, src_row, dst_row,
                                    err, w + p.meta_ws, s0);
  if (he != hipSuccess) return MOE_ERR_HIP;
  if (s.T == 0) return MOE_OK;

  const bool two = (s1 != nullptr && s1 != s0 && s.N >= 2);
  hipEvent_t meta_done = nullptr, s1_done = nullptr;
  if (two) {
    he = thread_events(&meta_done, &s1_done);
    if (he == hipSuccess) he = hipEventRecord(meta_done, s0);
    if (he == hipSuccess) he = hipStreamWaitEvent(s1, meta_done, 0);
    if (he != hipSuccess) return MOE_ERR_HIP;
  }
  bool used_s1 = false;
  for (int c = 0; c < s.N; ++c) {
    int t0, t1;
    chunk_tokens(s, c, &t0, &t1);
    if (t1 == t0) continue;  // empty tail chunk: no rows, nothing to launch
    const int slot = c % p.nslots;
    hipStream_t st_c = (two && (c & 1)) ? s1 : s0;
    used_s1 |= (st_c == s1 && two);
    void* xy = w + p.slot[slot];
    void* act = w + p.slot_act[slot];
    const int64_t rows = (int64_t)(t1 - t0) * s.k;
    const int32_t* off_c = offsets + (size_t)c * (s.E + 1);
    he = launch_permute(s, t0, t1, hidden_states, dst_row, xy, st_c);
    if (he != hipSuccess) return MOE_ERR_HIP;
    st = gate_up(s, rows, xy, off_c, w_gate_up, act, st_c);
    if (st != MOE_OK) return st;
    st = down(s, rows, act, off_c, w_down, xy, st_c);  // y overwrites the dead x_perm
    if (st != MOE_OK) return st;
    he = launch_combine(s, t0, t1, xy, dst_row, top_k_weights, out, st_c);
    if (he != hipSuccess) return MOE_ERR_HIP;
  }
  if (two && used_s1) {
    he = hipEventRecord(s1_done, s1);
    if (he == hipSuccess) he = hipStreamWaitEvent(s0, s1_done, 0);
    if (he != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // extern "C"
