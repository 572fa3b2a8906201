// Streaming-read rate of the device's HBM, for reporting the sweep's rate beside what the box
// reaches at all (not part of the decode step).
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

// Every 16-byte piece of the buffer read once, eight loads in flight per thread; the values are
// folded into one word that is stored only if it equals a constant, so no load can be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = p[i + e * stride];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc ^= v[e][0] ^ v[e][1] ^ v[e][2] ^ v[e][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace
}  // namespace hs

using namespace hs;

extern "C" hs_status hs_measure_read_gbps(const void* buf, size_t bytes, void* sink, int32_t reps,
                                          double* gbps) {
  if (!buf || !sink || !gbps || reps < 1 || bytes < 16 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return HS_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return HS_ERR_HIP;
  const int64_t n16 = (int64_t)(bytes / 16);
  const dim3 grid((unsigned)(cus * 8));
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return HS_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return HS_ERR_HIP;
  }
  float best_ms = 0.0f;
  hipError_t e = hipSuccess;
  for (int r = 0; r <= reps && e == hipSuccess; ++r) {  // the first launch warms up
    e = hipEventRecord(e0, nullptr);
    hipLaunchKernelGGL(stream_read_kernel, grid, dim3(256), 0, nullptr,
                       static_cast<const u32x4*>(buf), n16, static_cast<uint32_t*>(sink));
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && r > 0 && (best_ms == 0.0f || ms < best_ms)) best_ms = ms;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess || best_ms <= 0.0f) return HS_ERR_HIP;
  *gbps = (double)(n16 * 16) / (best_ms * 1e-3) / 1e9;
  return HS_OK;
}
