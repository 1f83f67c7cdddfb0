// moba_meanpool — block keys kbar_i = (1/B) sum_{j in block i} k_j
// (PaperTrace "2.1.3 MoBA", section 1, eq. (3); section 3.1 step 1).
//
// HBM-bound streaming reduction. For block i the keys of all KV heads are one
// contiguous span of B * Hkv * d elements, so a workgroup walks rows of that
// span with 16-byte loads (8 bf16 or 4+4 fp32) and keeps fp64 column sums.
// Each block is split over `splits` workgroups to fill the chip; pass 1 writes
// fp64 partial sums per split, pass 2 adds the splits in fixed order, divides
// by B and transposes to kbar[g][i][c]. fp64 sums of bf16 keys are exact, so
// the result does not depend on the summation order.
#include "moba_internal.hpp"

namespace moba {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <typename T>
struct Vec8;
template <>
struct Vec8<__hip_bfloat16> {
  static __device__ inline void load(const __hip_bfloat16* p, double (&x)[8]) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      x[2 * t] = (double)__uint_as_float(w[t] << 16);
      x[2 * t + 1] = (double)__uint_as_float(w[t] & 0xFFFF0000u);
    }
  }
};
template <>
struct Vec8<float> {
  static __device__ inline void load(const float* p, double (&x)[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

// grid: (nh, col chunks, splits). Column groups of 8 elements; CW groups per
// workgroup, R = kThreads / CW rows in flight.
// A block shorter than B (the last one of a sequence) is never history; its
// sums are left at zero.
template <typename T>
__global__ __launch_bounds__(kThreads) void meanpool_partial(const T* __restrict__ K,
                                                             const int32_t* __restrict__ bstart,
                                                             const int32_t* __restrict__ blen,
                                                             double* __restrict__ part, int B,
                                                             int W8, int CW, int splits,
                                                             int64_t nh) {
  __shared__ double red[kThreads * 8];
  const int tid = threadIdx.x;
  const int R = kThreads / CW;
  const int cg = tid % CW;
  const int rr = tid / CW;
  const int64_t blk = blockIdx.x;
  const int colg = blockIdx.y * CW + cg;
  const int s = blockIdx.z;
  const int64_t rows_per_split = (B + splits - 1) / splits;
  const int64_t b0 = bstart[blk];
  const int64_t r0 = b0 + (int64_t)s * rows_per_split;
  int64_t r1 = r0 + rows_per_split;
  if (r1 > b0 + B) r1 = b0 + B;
  if (blen[blk] < B) r1 = r0;
  const int64_t W = (int64_t)W8 * 8;

  double acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.0;
  const bool active = (rr < R) && (colg < W8);
  if (active) {
    const T* base = K + (size_t)colg * 8;
    int64_t r = r0 + rr;
    // kUnroll independent loads in flight per thread.
    for (; r + (kUnroll - 1) * R < r1; r += kUnroll * R) {
      double x[kUnroll][8];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) Vec8<T>::load(base + (size_t)(r + u * R) * W, x[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] += x[u][t];
    }
    for (; r < r1; r += R) {
      double x[8];
      Vec8<T>::load(base + (size_t)r * W, x);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] += x[t];
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) red[tid * 8 + t] = acc[t];
  __syncthreads();
  if (rr == 0 && colg < W8) {
    double sum[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) sum[t] = red[cg * 8 + t];
    for (int q = 1; q < R; ++q)
#pragma unroll
      for (int t = 0; t < 8; ++t) sum[t] += red[(q * CW + cg) * 8 + t];
    double* out = part + ((size_t)s * nh + blk) * W + (size_t)colg * 8;
#pragma unroll
    for (int t = 0; t < 8; ++t) out[t] = sum[t];
  }
}

// kbar[g][i][c] = (sum over splits of part[s][i][g*d + c]) / B
__global__ void meanpool_finish(const double* __restrict__ part, double* __restrict__ kbar,
                                int64_t nh, int Hkv, int d, int B, int splits) {
  const int64_t W = (int64_t)Hkv * d;
  const int64_t total = nh * W;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / W;
    const int64_t col = t % W;
    double s = 0.0;
    for (int q = 0; q < splits; ++q) s += part[((size_t)q * nh + i) * W + col];
    const int64_t g = col / d, c = col % d;
    kbar[(g * nh + i) * d + c] = s / (double)B;
  }
}

}  // namespace

int meanpool_splits(const Prob& P) {
  if (P.nh <= 0) return 1;
  const int W8 = P.Hkv * P.d / 8;
  const int CW = W8 < kThreads ? W8 : kThreads;
  const int R = kThreads / CW;
  const int64_t ncc = ceil_div(W8, CW);
  int64_t want = ceil_div(2048, P.nh * ncc);
  int64_t cap = P.B / (R * 8);
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  return (int)want;
}

hipError_t launch_meanpool(const Prob& P, const Blocks& T, const void* K, double* kbar,
                           double* part, int splits, hipStream_t s) {
  if (P.nh <= 0) return hipSuccess;
  const int W8 = P.Hkv * P.d / 8;
  const int CW = W8 < kThreads ? W8 : kThreads;
  dim3 grid((unsigned)P.nh, (unsigned)ceil_div(W8, CW), (unsigned)splits);
  if (P.dtype == MOBA_DTYPE_BF16)
    meanpool_partial<__hip_bfloat16><<<grid, kThreads, 0, s>>>(
        (const __hip_bfloat16*)K, T.start, T.len, part, P.B, W8, CW, splits, P.nh);
  else
    meanpool_partial<float><<<grid, kThreads, 0, s>>>((const float*)K, T.start, T.len, part, P.B,
                                                      W8, CW, splits, P.nh);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = P.nh * P.Hkv * P.d;
  int64_t nb = ceil_div(total, 256);
  if (nb > 4096) nb = 4096;
  meanpool_finish<<<(unsigned)nb, 256, 0, s>>>(part, kbar, P.nh, P.Hkv, P.d, P.B, splits);
  return hipGetLastError();
}

}  // namespace moba
