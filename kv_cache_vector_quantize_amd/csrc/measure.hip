// Measurement helpers: a plain streaming read and a plain streaming write of a
// device buffer, giving the rates at which this device's HBM can be read by a
// kernel that only loads and written by one that only stores (the ceilings
// against which the memory-bound kernels' rates are read).
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

// Grid-stride over 16-byte words, kReadUnroll loads in flight per thread;
// the XOR of everything read is written only if it equals a fixed value, so
// no load can be dropped and (almost) nothing is written.
__global__ void __launch_bounds__(kReadThreads) k_stream_read(const u32x4* __restrict__ buf, int64_t n16,
                                                              uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= buf[i];
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) sink[0] = x;
}

// Grid-stride 16-byte stores of one value.
__global__ void __launch_bounds__(kReadThreads) k_stream_write(u32x4* __restrict__ buf, int64_t n16, uint32_t value) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  const u32x4 v = {value, value, value, value};
  for (int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(v, buf + i);
}

int64_t stream_grid(int64_t n16) {
  const int64_t grid = (n16 + kReadThreads - 1) / kReadThreads;
  return grid > 256 * 16 ? 256 * 16 : grid;    // 16 workgroups per CU, grid-stride beyond
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)stream_grid(n16)), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_stream_write(void* buf, int64_t bytes, uint32_t value, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_write, dim3((unsigned)stream_grid(n16)), dim3(kReadThreads), 0, stream,
                     static_cast<u32x4*>(buf), n16, value);
  return hipGetLastError();
}

}  // namespace tq
