// moe_chunked_forward_noalloc: the whole forward layer for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its workspace is one file-scope device
// array, `scratch`, of kNoAllocScratchBytes, instead of a caller buffer.
//
// Each GPU the library runs on holds its own copy of the array (at its own
// address) until the process ends.  Host code never passes the array's name to
// a kernel or a copy: in host code that name is a host-side stand-in, not a
// device address.  The device address is looked up once per device with
// hipGetSymbolAddress, with that device current, on the entry point's first
// call there, and cached; every later use goes through that pointer.
//
// Every call writes each byte of the scratch that it later reads (routing
// metadata, per-segment counts, act, y), so nothing has to be cleared between
// calls.  All calls on one GPU share the array: calls that overlap in time on
// one GPU (on different streams, or from different host threads without
// ordering) race on it, and must be ordered by the caller.
#include <mutex>
#include <vector>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;  // 64 MiB per GPU

__device__ __align__(256) char scratch[kNoAllocScratchBytes];

struct DeviceScratch {
  int device;
  void* ptr;
};

std::mutex g_scratch_mu;
std::vector<DeviceScratch> g_scratch;  // one entry per device, filled on first use

// Device address of `scratch` on the current device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  for (const auto& d : g_scratch)
    if (d.device == dev) {
      *out = d.ptr;
      return hipSuccess;
    }
  void* ptr = nullptr;
  err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (err != hipSuccess) return err;
  if (!ptr) return hipErrorInvalidSymbol;
  g_scratch.push_back({dev, ptr});
  *out = ptr;
  return hipSuccess;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_chunked_forward_noalloc(const moe_shape* shape,
                                                  const void* hidden_states,
                                                  const int32_t* top_k_index,
                                                  const float* top_k_weights,
                                                  const void* w_gate_up, const void* w_down,
                                                  void* out, int32_t* dev_error,
                                                  hipStream_t stream) {
  size_t need = 0;
  moe_status st = moe_workspace_size(shape, &need);
  if (st != MOE_OK) return st;
  if (need > moe::kNoAllocScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (moe::scratch_address(&ws) != hipSuccess) return MOE_ERR_HIP;
  return moe_chunked_forward_schedule(shape, hidden_states, top_k_index, top_k_weights,
                                      w_gate_up, w_down, out, dev_error, ws,
                                      moe::kNoAllocScratchBytes, stream, nullptr,
                                      MOE_SCHEDULE_PAIR_FUSED);
}
