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

// grid: (tiles, Hkv); tile tile0 + blockIdx.x, tiles numbered block by block
// (Bpad / 64 per block). Block starts and lengths come from the block tables,
// or, when bstart is NULL (one sequence of N rows), are c * B and
// min(B, N - c * B). Vt rows are ld_blocks * Bpad long.
__global__ __launch_bounds__(kThreads) void vt_pack(const uint16_t* __restrict__ V,
                                                    const int32_t* __restrict__ bstart,
                                                    const int32_t* __restrict__ blen,
                                                    uint16_t* __restrict__ Vt, int Hkv,
                                                    int64_t Bpad, int64_t ld_blocks,
                                                    int64_t tile0, int B, int64_t N) {
  __shared__ uint16_t tile[kKeys * kStride];
  const int g = blockIdx.y;
  const int64_t tiles_per_block = Bpad / kKeys;
  const int64_t tix = tile0 + blockIdx.x;
  const int64_t c = tix / tiles_per_block;
  const int64_t t0 = (tix % tiles_per_block) * kKeys;  // position offset inside block
  int64_t row0, rows_c;
  if (bstart) {
    row0 = bstart[c];
    rows_c = blen[c];
  } else {
    row0 = c * B;
    rows_c = N - row0 < B ? N - row0 : B;
  }
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
    const int64_t ld = ld_blocks * Bpad;
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
                                    P.vt_blocks, 0, P.B, P.N);
  return hipGetLastError();
}

hipError_t launch_vt_pack_rows(const Prob& P, const void* V, void* Vt, int64_t r0, int64_t r1,
                               hipStream_t s) {
  if (r1 <= r0) return hipSuccess;
  const int64_t Bpad = ceil_div(P.B, kKeys) * kKeys;
  const int64_t tpb = Bpad / kKeys;
  // tiles holding rows r0 .. r1 - 1 (whole tiles are rewritten, from all rows < N)
  const int64_t first = (r0 / P.B) * tpb + (r0 % P.B) / kKeys;
  const int64_t last = ((r1 - 1) / P.B) * tpb + ((r1 - 1) % P.B) / kKeys;
  dim3 grid((unsigned)(last - first + 1), (unsigned)P.Hkv);
  vt_pack<<<grid, kThreads, 0, s>>>((const uint16_t*)V, nullptr, nullptr, (uint16_t*)Vt, P.Hkv,
                                    Bpad, P.vt_blocks, first, P.B, P.N);
  return hipGetLastError();
}

}  // namespace moba
