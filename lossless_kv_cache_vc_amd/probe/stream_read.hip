// Streaming-read peak of this GPU (a measurement, not part of the method): every thread reads
// 16-byte pieces of a contiguous buffer with coalesced nontemporal vector loads, 8 in flight;
// work-group b reads 8 consecutive 4 KB chunks, then strides by the grid.  Each work-group
// leaves the XOR of every 32-bit word it read in checksum[group] (a plain store: same-address
// atomics from every wave would serialize in L2 and cost several percent of a launch), so a
// test can check that the whole buffer was read.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void read_kernel(const u32x4* buf, uint64_t n16, uint32_t* checksum) {
  const uint64_t stride = (uint64_t)gridDim.x * 256 * kReadUnroll;
  u32x4 acc = {0, 0, 0, 0};
  for (uint64_t i = (uint64_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x; i < n16; i += stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = i + u * 256 < n16 ? __builtin_nontemporal_load(buf + i + u * 256) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  __shared__ uint32_t x;
  if (threadIdx.x == 0) x = 0;
  __syncthreads();
  atomicXor(&x, acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  __syncthreads();
  if (threadIdx.x == 0) checksum[blockIdx.x] = x;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) of `buf` (device) once with `groups` work-groups of 256 threads
// on `stream`; checksum (device, `groups` words) receives each group's XOR of the 32-bit words it
// read.  Returns 0, -1 for bad arguments (nothing launched) or the HIP error.
int vcprobe_read(const void* buf, uint64_t bytes, int32_t groups, uint32_t* checksum, void* stream) {
  if (!buf || !checksum || bytes == 0 || bytes % 16 || groups < 1 || groups > (1 << 20)) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(groups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, checksum);
  return (int)hipGetLastError();
}

}  // extern "C"
