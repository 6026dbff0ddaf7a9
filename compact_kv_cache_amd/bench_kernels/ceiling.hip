// Measurement kernels for the benchmark's ceilings (not part of the GVA
// library): the per-launch floor of an empty kernel, and plain reads in the
// decode's load pattern (every 16-byte load instruction of a wave covers 1 KB
// of contiguous memory; non-temporal buffer loads), each timed as K launches
// captured in one HIP graph and replayed between events on one stream (behind
// a short spin kernel, so the host's submission of the graph is not timed).
//
//   ceiling_empty_us(launches, &us)             empty kernel, 256 x 512 threads
//   ceiling_read_us(bytes, replicas, wgs, launches, &us)
//       each launch reads `bytes` (one of `replicas` distinct buffers, visited
//       in turn so that every launch reads data that is cold in the
//       last-level cache); workgroup i reads bytes/wgs contiguous bytes with
//       8 waves; a wave requests up to 17 KB at once (all of it when its share
//       is that small, as at the mid decode size), else streams with 8 loads
//       in flight.
// Both return 0 on success, a hipError_t value otherwise. The buffers are
// allocated and freed inside the call.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

__global__ void empty_kernel() {}

// One wave that returns once `ticks` of the 100 MHz real-time counter have
// passed: keeps the device busy while the host enqueues the timed launches.
__global__ void spin_kernel(unsigned long long ticks) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) {
  }
}

// All of a wave's loads requested at once (NPW <= 17 per wave).
template <int NPW>
__global__ __launch_bounds__(512) void read_all_kernel(const char* src, unsigned per_wg, unsigned* sink) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const char* base = src + (size_t)blockIdx.x * per_wg;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, (int)per_wg, kWord3);
  u32x4 v[NPW];
#pragma unroll
  for (int i = 0; i < NPW; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (w + 8 * i) * 1024 + 16 * lane, 0, kNonTemporal);
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < NPW; ++i) acc ^= v[i];
  const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9e3779b9u) sink[blockIdx.x] = x;  // keeps the loads; never true for the fill pattern
}

// Streaming: 8 loads in flight per wave.
__global__ __launch_bounds__(512) void read_ring_kernel(const char* src, unsigned per_wg, unsigned* sink) {
  constexpr int D = 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const char* base = src + (size_t)blockIdx.x * per_wg;
  const int nload = (int)(per_wg / 1024);
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, (int)per_wg, kWord3);
  u32x4 ring[D];
#pragma unroll
  for (int i = 0; i < D; ++i) ring[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (w + 8 * i) * 1024 + 16 * lane, 0, kNonTemporal);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int j = 0; w + 8 * D * (j + 1) < nload + 8 * D; ++j) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      acc ^= ring[i];
      ring[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (w + 8 * (D * (j + 1) + i)) * 1024 + 16 * lane, 0, kNonTemporal);
    }
  }
#pragma unroll
  for (int i = 0; i < D; ++i) acc ^= ring[i];
  const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

// K launches back to back on stream s, timed with events: the device spins
// first while the host enqueues them (a C++ loop, a few microseconds per
// launch), so the events bracket the device running the launches back to
// back, as the decode step is timed. Best of three runs, after a warm-up run.
template <typename F>
hipError_t queued_time(hipStream_t s, int launches, F launch, double* us) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  for (int k = 0; k < launches; ++k) launch(k);  // warm-up
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  float best = 1e30f;
  for (int rep = 0; rep < 3 && e == hipSuccess; ++rep) {
    spin_kernel<<<1, 64, 0, s>>>(100000ull);  // about 1 ms
    e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    for (int k = 0; k < launches && e == hipSuccess; ++k) {
      launch(k);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && ms < best) best = ms;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e == hipSuccess) *us = best * 1e3 / launches;
  return e;
}

}  // namespace

extern "C" {

int ceiling_empty_us(int launches, double* us) {
  hipStream_t s = nullptr;
  hipError_t e = hipStreamCreate(&s);
  if (e != hipSuccess) return e;
  e = queued_time(s, launches, [&](int) { empty_kernel<<<256, 512, 0, s>>>(); }, us);
  (void)hipStreamDestroy(s);
  return e;
}

int ceiling_read_us(unsigned long long bytes, int replicas, int wgs, int launches, double* us) {
  if (wgs < 1 || replicas < 1 || launches < 1 || bytes % ((unsigned long long)wgs * 1024) != 0) return hipErrorInvalidValue;
  const unsigned long long per_wg = bytes / wgs;
  if (per_wg > 0x7fffffffull) return hipErrorInvalidValue;
  char* buf = nullptr;
  unsigned* sink = nullptr;
  hipStream_t s = nullptr;
  hipError_t e = hipMalloc(&buf, bytes * replicas);
  if (e == hipSuccess) e = hipMalloc(&sink, sizeof(unsigned) * wgs);
  if (e == hipSuccess) e = hipMemset(buf, 1, bytes * replicas);
  if (e == hipSuccess) e = hipStreamCreate(&s);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  const unsigned pw = (unsigned)per_wg;
  const bool all_at_once = per_wg <= 17 * 8 * 1024;
  if (e == hipSuccess) {
    e = queued_time(s, launches, [&](int k) {
      const char* src = buf + (size_t)(k % replicas) * bytes;
      if (all_at_once)
        read_all_kernel<17><<<wgs, 512, 0, s>>>(src, pw, sink);
      else
        read_ring_kernel<<<wgs, 512, 0, s>>>(src, pw, sink);
    }, us);
  }
  if (s) (void)hipStreamDestroy(s);
  if (sink) (void)hipFree(sink);
  if (buf) (void)hipFree(buf);
  return e;
}

}  // extern "C"
