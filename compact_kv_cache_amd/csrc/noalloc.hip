// Allocation-free form of the fused decode step: the split-K workspace is a
// file-scope device array of fixed size instead of a caller-provided buffer,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// Each device the library runs on holds one copy of `scratch` (kScratchBytes)
// until the process ends. Its address is taken once per device with
// hipGetSymbolAddress while that device is current, and only that address is
// handed to kernels (in host code the array's name is not a device address).
// The arrival counters at its start must be zero before a call; they are
// zero when the code object is loaded, are cleared once more by a small
// kernel at the first call on the device, and every completed call leaves
// them at zero again. All calls on one device share the array: calls that
// overlap in time on one device race (their partials and counters collide).
#include <mutex>

#include "../../include/gva.h"
#include "launch.hpp"

namespace gva {
namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;  // 4 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

// Zero the first `words` 32-bit words (the arrival counters).
__global__ void clear_words_kernel(uint32_t* p, int words) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x) p[i] = 0u;
}

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (set up on first use: the
// symbol address is looked up with the device current, and the counter area
// is cleared on `stream`).
hipError_t scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // every counter the largest accepted shape can use lies in the first
    // ws_counter_bytes(...) bytes; clearing 64 KiB covers B*G + B <= 512
    constexpr int kClearWords = 64 * 1024 / 4;
    clear_words_kernel<<<16, 256, 0, stream>>>(static_cast<uint32_t*>(p), kClearWords);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace gva

extern "C" {

gva_status gva_decode_step_noalloc(const gva_shape* shape, const void* v_new, const void* kr_new,
                                   const void* q_nope, const void* q_rope, const void* M, void* v_cache,
                                   void* kr_cache, int32_t* seq_lens, const int32_t* block_table, float scale,
                                   float rope_base, void* out, hipStream_t stream) {
  const size_t need = gva_decode_step_workspace_bytes(shape);
  if (need == 0) {  // invalid shape: let the regular entry point report why
    return gva_decode_step(shape, v_new, kr_new, q_nope, q_rope, M, v_cache, kr_cache, seq_lens, block_table,
                           scale, rope_base, out, nullptr, 0, stream);
  }
  if (need > gva::kScratchBytes) return gva::refuse_scratch(need, gva::kScratchBytes);
  // the counter area must lie inside the region cleared at set-up
  if (gva::ws_counter_bytes(shape->B, shape->G) > 64 * 1024) return gva::refuse_scratch(need, gva::kScratchBytes);
  void* ws = nullptr;
  const hipError_t e = gva::scratch_for_current_device(stream, &ws);
  if (e != hipSuccess) return gva::hip_failure(e, "gva_decode_step_noalloc scratch set-up");
  return gva_decode_step(shape, v_new, kr_new, q_nope, q_rope, M, v_cache, kr_cache, seq_lens, block_table, scale,
                         rope_base, out, ws, gva::kScratchBytes, stream);
}

}  // extern "C"
