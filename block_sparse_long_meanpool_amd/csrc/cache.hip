// Decode cache kernels. Generation appends rows to one sequence; the block
// means (PaperTrace "2.1.3 MoBA", section 1 eq. (3)) of blocks that are
// already full never change, so they are computed once, when the appended
// rows complete a block, and kept (section 5.1 notes that generation needs
// the block means kept current as tokens arrive).
//
// cache_means: fp64 column sums of the B rows of each completed block, one
// workgroup per (block, 256 of the Hkv * d columns); 4 row groups of 256
// threads each sum every 4th row and the groups are added in a fixed order,
// so the result does not depend on timing. Rows are contiguous spans of
// Hkv * d elements, so the 256 threads of a row group read 512 (bf16) or
// 1024 (fp32) contiguous bytes per row.
// kbar_gather: the gate reads the means of the first nh blocks as
// [Hkv][nh][d]; the cache keeps them as [Hkv][nhc][d] for its capacity.
#include "moba_internal.hpp"

namespace moba {
namespace {

constexpr int kCols = 256;
constexpr int kGroups = 4;

template <typename T>
__device__ inline double ld(const T* p);
template <>
__device__ inline double ld<uint16_t>(const uint16_t* p) {
  return (double)__uint_as_float((uint32_t)*p << 16);
}
template <>
__device__ inline double ld<float>(const float* p) {
  return (double)*p;
}

// grid: (count, ceil(Hkv * d / 256)); 1024 threads.
template <typename T>
__global__ __launch_bounds__(kCols * kGroups) void cache_means(const T* __restrict__ K, int Hkv,
                                                               int d, int B, int64_t c0,
                                                               double* __restrict__ kbar,
                                                               int64_t nhc) {
  __shared__ double part[kGroups][kCols];
  const int W = Hkv * d;
  const int col = blockIdx.y * kCols + (threadIdx.x % kCols);
  const int grp = threadIdx.x / kCols;
  const int64_t c = c0 + blockIdx.x;
  double acc = 0.0;
  if (col < W) {
    const T* base = K + (c * B) * (int64_t)W + col;
    for (int r = grp; r < B; r += kGroups) acc += ld<T>(base + (int64_t)r * W);
  }
  part[grp][threadIdx.x % kCols] = acc;
  __syncthreads();
  if (grp == 0 && col < W) {
    double s = part[0][threadIdx.x];
#pragma unroll
    for (int q = 1; q < kGroups; ++q) s += part[q][threadIdx.x];
    const int g = col / d, e = col % d;
    kbar[((int64_t)g * nhc + c) * d + e] = s / (double)B;
  }
}

__global__ void kbar_gather(const double* __restrict__ src, int64_t nhc, double* __restrict__ dst,
                            int64_t nh, int Hkv, int d) {
  const int64_t total = (int64_t)Hkv * nh * d;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = t % d, i = (t / d) % nh, g = t / ((int64_t)d * nh);
    dst[t] = src[(g * nhc + i) * d + e];
  }
}

}  // namespace

hipError_t launch_cache_means(const Prob& P, const void* K, int64_t c0, int64_t count,
                              double* kbar, int64_t nhc, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  dim3 grid((unsigned)count, (unsigned)ceil_div((int64_t)P.Hkv * P.d, kCols));
  if (P.dtype == MOBA_DTYPE_BF16)
    cache_means<uint16_t><<<grid, kCols * kGroups, 0, s>>>((const uint16_t*)K, P.Hkv, P.d, P.B, c0,
                                                           kbar, nhc);
  else
    cache_means<float><<<grid, kCols * kGroups, 0, s>>>((const float*)K, P.Hkv, P.d, P.B, c0, kbar,
                                                        nhc);
  return hipGetLastError();
}

hipError_t launch_kbar_gather(const double* src, int64_t nhc, double* dst, int64_t nh, int Hkv,
                              int d, hipStream_t s) {
  const int64_t total = (int64_t)Hkv * nh * d;
  if (total <= 0) return hipSuccess;
  int64_t nb = ceil_div(total, 256);
  if (nb > 4096) nb = 4096;
  kbar_gather<<<(unsigned)nb, 256, 0, s>>>(src, nhc, dst, nh, Hkv, d);
  return hipGetLastError();
}

}  // namespace moba
