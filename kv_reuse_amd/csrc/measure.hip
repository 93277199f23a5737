// Streaming-read ceiling of the device, for the measurement's roofline: the
// dominant decode kernel streams the whole KV cache once, so its bandwidth is
// rated against the datasheet peak and against what a plain streaming read
// reaches on the same part.  Every 16-byte unit of a buffer is read once with
// a non-temporal load (the full layer's load kind); nothing is written except,
// in the practically impossible case that the XOR of everything read equals a
// fixed constant, one flag (so that the compiler keeps every load).

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kSThreads = 256;
constexpr int kSUnroll = 8;   // loads in flight per thread

// Work-group b reads its own contiguous share of the buffer, its threads side
// by side (16 bytes each), kSUnroll loads in flight per thread.  (Measured on
// MI355X: contiguous shares, one work-group of 4 waves per CU, reach about
// 7.2 TB/s; a grid-strided sweep of the whole buffer about 6.2.)
__global__ __launch_bounds__(kSThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                                size_t n16,
                                                                uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = static_cast<size_t>(blockIdx.x) * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  size_t i = b0 + threadIdx.x;
  for (; i + (kSUnroll - 1) * kSThreads < b1; i += kSUnroll * kSThreads) {
    u32x4 v[kSUnroll];
#pragma unroll
    for (int u = 0; u < kSUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kSThreads);
    // every load of the batch is issued before the first is waited on (left to
    // itself the scheduler pulls the first XOR up between the loads)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kSUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < b1; i += kSThreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) atomicOr(sink, 1u);
}

}  // namespace
}  // namespace hs2

using namespace hs2;

extern "C" int hs2_stream_read_ms(const void* buf, size_t bytes, uint32_t* sink, int32_t iters,
                                  void* stream, float* ms_out) {
  if (!buf || !sink || !ms_out || iters < 1 || bytes < 16) return HS2_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return HS2_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0, n_cu = kDefaultCUs;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
    n_cu = kDefaultCUs;
  (void)hipGetLastError();
  const size_t n16 = bytes / 16;
  const int grid = n_cu;   // one work-group per CU
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return HS2_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return HS2_ERR_HIP;
  }
  hipError_t err = hipEventRecord(e0, s);
  for (int it = 0; it < iters && err == hipSuccess; ++it) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kSThreads), 0, s,
                       static_cast<const u32x4*>(buf), n16, sink);
    err = hipGetLastError();
  }
  if (err == hipSuccess) err = hipEventRecord(e1, s);
  if (err == hipSuccess) err = hipEventSynchronize(e1);
  float ms = 0.f;
  if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != hipSuccess) return record_hip_error(err);
  *ms_out = ms / static_cast<float>(iters);
  return HS2_OK;
}
