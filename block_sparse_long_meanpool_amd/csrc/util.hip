// Small utility kernels: a plain 16-byte copy (used to calibrate hardware
// traffic counters against a known byte count) and an int32 fill, which
// replaces hipMemsetAsync so every stage is an ordinary kernel launch.
#include "moba_internal.hpp"

namespace moba {
namespace {

__global__ void copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void fill_i32(int32_t* __restrict__ p, int32_t v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  copy16<<<(unsigned)blocks, 256, 0, s>>>((const uint4*)src, (uint4*)dst, n);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  size_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_i32<<<(unsigned)blocks, 256, 0, s>>>(p, v, count);
  return hipGetLastError();
}

}  // namespace moba
