// V layout change for the bf16 attention kernels: V [N][Hkv][d] -> per KV
// head, a transposed, block-padded copy Vt[g][d][c * Bpad + pi(r)] holding
// V[start(c) + r][g][d] for the rows r < len(c) of block c. Each block is
// padded to Bpad = ceil(B/64)*64 positions (pads are zero) so 64-key tiles
// never straddle blocks, and inside every 32-key group the key order is
// permuted by pi (swap of bits 2 and 3) so that each lane's 8 keys of the
// P.V matrix-core operand sit in one 16-byte run. One read and one write of
// V; no arithmetic on the values.
#include "moba_internal.hpp"

namespace moba {
namespace {

constexpr int kThreads = 256;
constexpr int kKeys = 64;
constexpr int kStride = kHeadDim + 2;  // odd word stride: column reads spread over banks

__device__ inline int perm32(int r) {  // involution on 0..31 (and on any 32-aligned group)
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// grid: (n * (Bpad / 64), Hkv)
__global__ __launch_bounds__(kThreads) void vt_pack(const uint16_t* __restrict__ V,
                                                    const int32_t* __restrict__ bstart,
                                                    const int32_t* __restrict__ blen,
                                                    uint16_t* __restrict__ Vt, int Hkv,
                                                    int64_t Bpad, int64_t n) {
  __shared__ uint16_t tile[kKeys * kStride];
  const int g = blockIdx.y;
  const int64_t tiles_per_block = Bpad / kKeys;
  const int64_t c = blockIdx.x / tiles_per_block;
  const int64_t t0 = (blockIdx.x % tiles_per_block) * kKeys;  // position offset inside block
  const int64_t row0 = bstart[c], rows_c = blen[c];
  // load 64 key rows (zero past the block)
  {
    const int kk = threadIdx.x >> 2, d0 = (threadIdx.x & 3) * 32;
    const int64_t r = t0 + kk;
    uint32_t w[16];
    if (r < rows_c) {
      const uint4* src = reinterpret_cast<const uint4*>(V + ((row0 + r) * Hkv + g) * kHeadDim + d0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 u = src[i];
        w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = 0u;
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + kk * kStride + d0);
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i] = w[i];
  }
  __syncthreads();
  // write 128 rows of 64 permuted positions: thread -> (d, half of the row)
  {
    const int d = threadIdx.x >> 1, half = threadIdx.x & 1;
    uint32_t out[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p0 = 32 * half + 2 * i;  // output positions p0, p0+1
      const int r0 = perm32(p0 & 31) + 32 * half, r1 = perm32((p0 + 1) & 31) + 32 * half;
      out[i] = (uint32_t)tile[r0 * kStride + d] | ((uint32_t)tile[r1 * kStride + d] << 16);
    }
    const int64_t ld = n * Bpad;
    uint4* dst = reinterpret_cast<uint4*>(Vt + ((int64_t)g * kHeadDim + d) * ld + c * Bpad + t0 +
                                          32 * half);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
  }
}

}  // namespace

hipError_t launch_vt_pack(const Prob& P, const Blocks& T, const void* V, void* Vt, hipStream_t s) {
  const int64_t Bpad = ceil_div(P.B, kKeys) * kKeys;
  dim3 grid((unsigned)(P.n * (Bpad / kKeys)), (unsigned)P.Hkv);
  vt_pack<<<grid, kThreads, 0, s>>>((const uint16_t*)V, T.start, T.len, (uint16_t*)Vt, P.Hkv, Bpad,
                                    P.n);
  return hipGetLastError();
}

}  // namespace moba
