// GPU fill kernels of the seeded input generator: value(seed, stream, logical index) written
// into dense tensors of up to 6 dimensions with arbitrary logical strides.  Same definition as
// vcsynth/rng.py: SplitMix64 output number idx+1 from the (seed, stream) key; normal variates by
// looking the upper 32 bits up in an inverse-CDF threshold table (built on the host).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth.h"

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct Dims {
  int nd;
  int64_t shape[6];
  int64_t lstride[6];
  int64_t lbase;
  int64_t total;
};

__device__ inline int64_t logical_index(const Dims& d, int64_t e) {
  int64_t li = d.lbase;
  for (int k = d.nd - 1; k >= 0; --k) {
    const int64_t c = e % d.shape[k];
    e /= d.shape[k];
    li += c * d.lstride[k];
  }
  return li;
}

constexpr int kMaxTab = 8192;

__global__ __launch_bounds__(256) void fill_normal_kernel(uint16_t* dst, Dims d, uint64_t key,
                                                          const uint32_t* thr, const uint16_t* val,
                                                          int ntab) {
  __shared__ uint32_t s_thr[kMaxTab];
  __shared__ uint16_t s_val[kMaxTab + 1];
  for (int i = threadIdx.x; i < ntab; i += blockDim.x) s_thr[i] = thr[i];
  for (int i = threadIdx.x; i <= ntab; i += blockDim.x) s_val[i] = val[i];
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < d.total; e += stride) {
    const uint64_t li = (uint64_t)logical_index(d, e);
    const uint32_t u = (uint32_t)(mix64(key + (li + 1) * kGamma) >> 32);
    // number of thresholds <= u
    int lo = 0, hi = ntab;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_thr[mid] <= u) lo = mid + 1;
      else hi = mid;
    }
    dst[e] = s_val[lo];
  }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* dst, Dims d, uint64_t key) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < d.total; e += stride) {
    const uint64_t li = (uint64_t)logical_index(d, e);
    dst[e] = (uint32_t)(mix64(key + (li + 1) * kGamma) >> 32);
  }
}

uint64_t stream_key(uint64_t seed, uint32_t stream) { return mix64(seed * kGamma + stream); }

int make_dims(int ndim, const int64_t* shape, const int64_t* lstride, int64_t lbase, Dims* d) {
  if (ndim < 1 || ndim > 6 || !shape || !lstride) return -1;
  d->nd = ndim;
  d->lbase = lbase;
  d->total = 1;
  for (int k = 0; k < ndim; ++k) {
    if (shape[k] < 0) return -1;
    d->shape[k] = shape[k];
    d->lstride[k] = lstride[k];
    d->total *= shape[k];
  }
  return 0;
}

// grid-stride launches: a few work-groups per CU, so the per-group table load stays cheap
int grid_for(int64_t total, int cap) {
  int64_t g = (total + 255) / 256;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

extern "C" {

int vcs_fill_normal_bf16(void* dst, int ndim, const int64_t* shape, const int64_t* lstride,
                         int64_t lbase, uint64_t seed, uint32_t stream_id, const uint32_t* thresholds,
                         const uint16_t* values, int ntab, void* stream) {
  Dims d;
  if (!dst || !thresholds || !values || ntab < 1 || ntab > kMaxTab) return -1;
  if (make_dims(ndim, shape, lstride, lbase, &d)) return -1;
  if (d.total == 0) return 0;
  hipLaunchKernelGGL(fill_normal_kernel, dim3(grid_for(d.total, 1024)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint16_t*>(dst), d,
                     stream_key(seed, stream_id), thresholds, values, ntab);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int vcs_fill_u32(void* dst, int ndim, const int64_t* shape, const int64_t* lstride, int64_t lbase,
                 uint64_t seed, uint32_t stream_id, void* stream) {
  Dims d;
  if (!dst) return -1;
  if (make_dims(ndim, shape, lstride, lbase, &d)) return -1;
  if (d.total == 0) return 0;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(d.total, 8192)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint32_t*>(dst), d,
                     stream_key(seed, stream_id));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
