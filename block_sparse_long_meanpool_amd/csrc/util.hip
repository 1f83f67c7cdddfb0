// Small utility kernels: a plain 16-byte copy (used to calibrate hardware
// traffic counters against a known byte count, and timed as the HBM stream
// probe), an int32 fill, which replaces hipMemsetAsync so every stage is an
// ordinary kernel launch, a read-only HBM stream probe and a matrix-core
// issue-rate probe.
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

// Matrix-core probe: every wave keeps four independent 32x32 fp32
// accumulators and issues v_mfma_f32_32x32x16_bf16 on them in turn, so the
// issue rate, not the result latency, sets the time. Operands are all 0.125:
// each op adds exactly 16 * 2^-6 = 0.25 to every accumulator element, so the
// per-lane checksum is 4 * 16 * 0.25 * iters = 16 * iters (exact while
// 16 * iters < 2^24), which proves that every op ran.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop(int iters, float* __restrict__ out) {
  bf16x8 a;
  for (int i = 0; i < 8; ++i) a[i] = (__bf16)0.125f;
  f32x16 c0, c1, c2, c3;
  for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c3, 0, 0, 0);
  }
  float sum = 0.f;
  for (int r = 0; r < 16; ++r) sum += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// HBM read probe: per round a workgroup reads 1024 consecutive 16-byte
// words, four per thread, all four in flight before use (lane-consecutive, so
// every load instruction is one contiguous 1 KiB run per wave); the words are
// XOR-folded into one register per lane and each lane writes that value once,
// so the loads stay live and the writes (1 KiB per workgroup) are negligible.
// The XOR of all outputs equals the XOR of every 32-bit word of src.
__global__ __launch_bounds__(256) void read_stream(const uint4* __restrict__ src, size_t n,
                                                   uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 1024;
  for (size_t base = (size_t)blockIdx.x * 1024; base < n; base += stride) {
    uint4 w[4];
    for (int j = 0; j < 4; ++j) {
      const size_t i = base + (size_t)j * 256 + threadIdx.x;
      w[j] = i < n ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    for (int j = 0; j < 4; ++j) acc ^= w[j].x ^ w[j].y ^ w[j].z ^ w[j].w;
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, int workgroups, uint32_t* out,
                             hipStream_t s) {
  read_stream<<<(unsigned)workgroups, 256, 0, s>>>((const uint4*)src, bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int workgroups, int iters, float* out, hipStream_t s) {
  mfma_loop<<<(unsigned)workgroups, 256, 0, s>>>(iters, out);
  return hipGetLastError();
}

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
