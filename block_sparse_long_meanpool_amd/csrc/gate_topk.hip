// moba_gate_topk — parameter-free gate and block selection
// (PaperTrace "2.1.3 MoBA": gate s_i = q . kbar_i of section 1 eq. (3); future
// blocks excluded and own block forced, section 2; k counts the own block,
// section 2.1; section 3.1 step 2).
//
// Scores are computed in fp64 on the fp64 matrix cores (v_mfma_f64_16x16x4):
// Q (bf16 or fp32) widens exactly, block keys are fp64, so a selection differs
// from the exact one only where two scores agree to fp64 rounding. Workgroup =
// 64 (row, head) pairs of one KV-head group inside one block c, i.e. pairs
// pi = (row - cB) * G + hh; wave w owns pairs 16w..16w+15 and holds their Q as
// the A operand in registers for the whole kernel. History blocks 0..c-1 are
// streamed through LDS in chunks of 32; after each chunk the scores go to LDS
// and one lane per pair folds them into a running top-(k-1) list kept sorted
// by (score desc, block asc). The own block c is appended and the row is
// written ascending and -1 padded.
#include "moba_internal.hpp"

namespace moba {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPairs = 64;       // pairs per workgroup
constexpr int kChunk = 32;       // history blocks per LDS chunk (two 16-wide MFMA tiles)
constexpr int kSteps = kHeadDim / 4;  // 32 MFMA k-steps of 4 over d = 128
constexpr int kScPad = kChunk + 1;
constexpr int kListCap = kMaxTopk - 1;

template <typename T>
__device__ inline void load_q32(const T* p, double (&q)[kSteps]);
template <>
__device__ inline void load_q32<__hip_bfloat16>(const __hip_bfloat16* p, double (&q)[kSteps]) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 u = v[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      q[8 * i + 2 * t] = (double)__uint_as_float(w[t] << 16);
      q[8 * i + 2 * t + 1] = (double)__uint_as_float(w[t] & 0xFFFF0000u);
    }
  }
}
template <>
__device__ inline void load_q32<float>(const float* p, double (&q)[kSteps]) {
  const float4* v = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 u = v[i];
    q[4 * i] = u.x; q[4 * i + 1] = u.y; q[4 * i + 2] = u.z; q[4 * i + 3] = u.w;
  }
}

// grid.x: (block c in descending order) * tiles_per_block + tile; grid.y: KV head g.
template <typename T>
__global__ __launch_bounds__(kThreads) void gate_topk_kernel(
    const T* __restrict__ Q, const double* __restrict__ kbar, int32_t* __restrict__ sel,
    int64_t N, int Hq, int G, int B, int k, int64_t n, int64_t nh, int tiles_per_block) {
  __shared__ double kb[kSteps * kChunk * 4];     // [ks][blk][grp]: d = grp*32 + ks
  __shared__ double sc[kPairs * kScPad];         // [pair][blk]
  __shared__ double ls[kListCap * kPairs];       // list scores [slot][pair]
  __shared__ int li[kListCap * kPairs];          // list blocks  [slot][pair]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = blockIdx.y;
  const int64_t c = n - 1 - (int64_t)(blockIdx.x / tiles_per_block);
  const int tile = blockIdx.x % tiles_per_block;
  const int64_t row0 = c * B;
  int64_t rows_c = N - row0;
  if (rows_c > B) rows_c = B;
  const int64_t npairs_c = rows_c * G;
  const int64_t pair0 = (int64_t)tile * kPairs;
  if (pair0 >= npairs_c) return;
  const int KH = k - 1;
  const int nsel = (int)(c < KH ? c : KH);  // history blocks this block's rows take

  // ---- scores and running selection (only when there is a choice to make) ----
  const bool rank = (c > KH) && (KH > 0);
  int cnt = 0;
  double thr = -INFINITY;
  const int my_pair = wave * 16 + (lane & 15);  // pair a selecting lane owns (lanes < 16)
  if (rank) {
    double qa[kSteps];
    {
      const int64_t pi = pair0 + wave * 16 + (lane & 15);
      if (pi < npairs_c) {
        const int64_t r = row0 + pi / G;
        const int h = g * G + (int)(pi % G);
        load_q32<T>(Q + ((size_t)r * Hq + h) * kHeadDim + 32 * (lane >> 4), qa);
      } else {
#pragma unroll
        for (int i = 0; i < kSteps; ++i) qa[i] = 0.0;
      }
    }
    const double* kbg = kbar + (size_t)g * nh * kHeadDim;
    for (int64_t cb = 0; cb < c; cb += kChunk) {
      __syncthreads();
      // stage kbar[cb .. cb+32) as [ks][blk][grp]
      {
        const int b = tid >> 3;            // 0..31
        const int d0 = (tid & 7) * 16;     // 16 consecutive d
        const int64_t blk = cb + b;
        if (blk < c) {
          const double2* src = reinterpret_cast<const double2*>(kbg + blk * kHeadDim + d0);
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            double2 v = src[x];
            int dd = d0 + 2 * x;
            kb[((dd & 31) * kChunk + b) * 4 + (dd >> 5)] = v.x;
            kb[(((dd + 1) & 31) * kChunk + b) * 4 + ((dd + 1) >> 5)] = v.y;
          }
        } else {
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            int dd = d0 + x;
            kb[((dd & 31) * kChunk + b) * 4 + (dd >> 5)] = 0.0;
          }
        }
      }
      __syncthreads();
      f64x4 acc0 = {0.0, 0.0, 0.0, 0.0};
      f64x4 acc1 = {0.0, 0.0, 0.0, 0.0};
      const int bl = lane & 15, grp = lane >> 4;
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        double b0 = kb[(ks * kChunk + bl) * 4 + grp];
        double b1 = kb[(ks * kChunk + 16 + bl) * 4 + grp];
        acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], b0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], b1, acc1, 0, 0, 0);
      }
      // D layout of v_mfma_f64_16x16x4: register r of lane l holds row (pair)
      // l/16 + 4r, column (block) l%16
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = wave * 16 + grp + 4 * r;
        sc[p * kScPad + bl] = acc0[r];
        sc[p * kScPad + 16 + bl] = acc1[r];
      }
      __syncthreads();
      if (lane < 16) {
        const int64_t lim = (c - cb < kChunk) ? c - cb : kChunk;
        for (int jj = 0; jj < lim; ++jj) {
          const double s = sc[my_pair * kScPad + jj];
          if (cnt < KH || s > thr) {
            int pos = (cnt < KH) ? cnt : KH - 1;
            while (pos > 0 && ls[(pos - 1) * kPairs + my_pair] < s) {
              ls[pos * kPairs + my_pair] = ls[(pos - 1) * kPairs + my_pair];
              li[pos * kPairs + my_pair] = li[(pos - 1) * kPairs + my_pair];
              --pos;
            }
            ls[pos * kPairs + my_pair] = s;
            li[pos * kPairs + my_pair] = (int)(cb + jj);
            if (cnt < KH) ++cnt;
            thr = ls[(cnt - 1) * kPairs + my_pair];
          }
        }
      }
    }
  }

  // ---- write the selection rows of this wave's 16 pairs ----
  if (lane < 16) {
    const int64_t pi = pair0 + my_pair;
    if (pi < npairs_c) {
      const int64_t r = row0 + pi / G;
      const int h = g * G + (int)(pi % G);
      int32_t* out = sel + ((size_t)r * Hq + h) * k;
      if (rank) {
        // ascending order of the kept blocks (insertion sort of <= 31 entries)
        for (int a = 1; a < cnt; ++a) {
          int v = li[a * kPairs + my_pair];
          int b = a - 1;
          while (b >= 0 && li[b * kPairs + my_pair] > v) {
            li[(b + 1) * kPairs + my_pair] = li[b * kPairs + my_pair];
            --b;
          }
          li[(b + 1) * kPairs + my_pair] = v;
        }
        for (int a = 0; a < cnt; ++a) out[a] = li[a * kPairs + my_pair];
        out[cnt] = (int32_t)c;
        for (int a = cnt + 1; a < k; ++a) out[a] = -1;
      } else {
        for (int a = 0; a < nsel; ++a) out[a] = a;
        out[nsel] = (int32_t)c;
        for (int a = nsel + 1; a < k; ++a) out[a] = -1;
      }
    }
  }
}

}  // namespace

hipError_t launch_gate_topk(const Prob& P, const void* Q, const double* kbar, int32_t* sel,
                            hipStream_t s) {
  const int tiles_per_block = (int)ceil_div((int64_t)P.B * P.G, kPairs);
  dim3 grid((unsigned)(P.n * tiles_per_block), (unsigned)P.Hkv);
  if (P.dtype == MOBA_DTYPE_BF16)
    gate_topk_kernel<__hip_bfloat16><<<grid, kThreads, 0, s>>>(
        (const __hip_bfloat16*)Q, kbar, sel, P.N, P.Hq, P.G, P.B, P.k, P.n, P.nh, tiles_per_block);
  else
    gate_topk_kernel<float><<<grid, kThreads, 0, s>>>((const float*)Q, kbar, sel, P.N, P.Hq, P.G,
                                                      P.B, P.k, P.n, P.nh, tiles_per_block);
  return hipGetLastError();
}

}  // namespace moba
