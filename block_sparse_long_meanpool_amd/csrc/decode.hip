// Attention for a few query rows (decode steps and small chunks). The
// prefill kernels tile 256 routed queries per K/V block; with a handful of
// rows a block has one or two queries, so this path splits the keys instead
// (PaperTrace "2.1.3 MoBA", section 3.1: decode reads the selected blocks for
// very few queries and is bound by memory, not by the matrix cores).
//
// decode_partial: one workgroup per (query row, query head, selection slot,
// 256-key split of the selected block). For each slot's block (eq. (4): the
// top-k history blocks plus the row's own block, causally cut at the row,
// eq. (5)) it computes, in fp32 from the stored inputs, the scores of its 256
// keys, their max m, the sum l of 2^(score - m) and u = sum 2^(score - m) v
// (log2 domain, scores scaled by scale * log2(e)), and stores (m, l, u).
// decode_merge: per (row, head) the partials of all slots and splits are
// merged as in eqs. (7)-(8) (the shared max, rescaled sums) into O, and
// optionally the row's log2-sum-exp M + log2(L).
// K and V are read in place ([N][Hkv][d]): no packed copy is needed.
#include "moba_internal.hpp"

namespace moba {
namespace {

constexpr int kThreads = 256;
constexpr int kSplit = 256;       // keys per partial
constexpr int kPart = kHeadDim + 2;  // m, l, u[128]
constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
__device__ inline float ldf(const T* p);
template <>
__device__ inline float ldf<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}
template <>
__device__ inline float ldf<float>(const float* p) {
  return *p;
}
// Two consecutive elements.
template <typename T>
__device__ inline float2 ld2(const T* p);
template <>
__device__ inline float2 ld2<uint16_t>(const uint16_t* p) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
}
template <>
__device__ inline float2 ld2<float>(const float* p) {
  return *reinterpret_cast<const float2*>(p);
}

// 16 bytes: 8 bf16 or 4 fp32.
__device__ inline void ld16(const uint16_t* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    x[2 * t] = __uint_as_float(w[t] << 16);
    x[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
  }
}
__device__ inline void ld16(const float* p, float (&x)[4]) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  x[0] = u.x;
  x[1] = u.y;
  x[2] = u.z;
  x[3] = u.w;
}

template <typename T>
__device__ inline void st(T* p, float x);
template <>
__device__ inline void st<uint16_t>(uint16_t* p, float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even
  *p = (uint16_t)(u >> 16);
}
template <>
__device__ inline void st<float>(float* p, float x) {
  *p = x;
}

// Sum over each aligned group of 16 lanes, left in every lane of the group,
// with DPP lane moves: swap within pairs, swap pairs within quads, mirror
// within 8 lanes (quad i <-> quad 1 - i), mirror within 16 lanes.
template <int CTRL>
__device__ inline float dpp_mov(float a) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), CTRL, 0xF, 0xF, true));
}
__device__ inline float sum16(float a) {
  a += dpp_mov<0xB1>(a);   // quad_perm [1, 0, 3, 2]
  a += dpp_mov<0x4E>(a);   // quad_perm [2, 3, 0, 1]
  a += dpp_mov<0x141>(a);  // row_half_mirror
  a += dpp_mov<0x140>(a);  // row_mirror
  return a;
}

__device__ inline float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}
__device__ inline float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return v;
}

// items = Nq * Hq * k * splits, item = ((r * Hq + h) * k + slot) * splits + sp
template <typename T>
__global__ __launch_bounds__(kThreads) void decode_partial(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ bstart,
    const int32_t* __restrict__ blen, const int32_t* __restrict__ row_blk, int64_t q0, int Hq,
    int Hkv, int G, int k, int splits, float sl2e, float* __restrict__ part) {
  __shared__ float qs[kHeadDim];
  __shared__ float ps[kSplit];
  __shared__ float red[4];
  __shared__ float us[kThreads / (kHeadDim * sizeof(T) / 16)][kHeadDim];
  const int64_t item = blockIdx.x;
  const int sp = (int)(item % splits);
  const int64_t rhs = item / splits;  // (r * Hq + h) * k + slot
  const int64_t rh = rhs / k;
  const int h = (int)(rh % Hq);
  const int64_t r = rh / Hq;
  const int g = h / G;
  const int tid = threadIdx.x;
  float* out = part + item * kPart;
  const int32_t b = sel[rhs];
  int64_t k0 = 0, k1 = 0;  // keys [k0, k1) of this split
  if (b >= 0) {
    const int64_t start = bstart[b];
    int64_t end = start + blen[b];
    if (b == row_blk[r]) {  // the row's own block: keys up to the row
      const int64_t lim = q0 + r + 1;
      end = end < lim ? end : lim;
    }
    k0 = start + (int64_t)sp * kSplit;
    k1 = k0 + kSplit < end ? k0 + kSplit : end;
  }
  if (k1 <= k0) {  // empty: no weight, u = 0
    if (tid < kHeadDim) out[2 + tid] = 0.f;
    if (tid == 0) {
      out[0] = -INFINITY;
      out[1] = 0.f;
    }
    return;
  }
  if (tid < kHeadDim) qs[tid] = ldf(Q + rh * kHeadDim + tid);
  __syncthreads();
  // scores: the lanes of a group (16 lanes for bf16, 32 for fp32) read one
  // key row together (each its 16-byte chunk), take partial dot products and
  // add them across the group; the group walks its keys, and its lane i keeps
  // the score of its i-th key: key kk + (256 / group) i for group kk
  constexpr int kVec = 16 / sizeof(T);       // elements per 16-byte load
  constexpr int kChunks = kHeadDim / kVec;   // 16-byte chunks per row
  constexpr int kRowsPerPass = kThreads / kChunks;
  const int ch = tid % kChunks, kk = tid / kChunks;
  float qv[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) qv[e] = qs[ch * kVec + e];
  float s = -INFINITY;
  int mykey = -1;  // key offset whose score this thread keeps
#pragma unroll 4
  for (int i = 0; i < kSplit / kRowsPerPass; ++i) {
    const int j = kk + kRowsPerPass * i;
    const int64_t key = k0 + j;
    float x[kVec];
    if (key < k1) {
      ld16(K + (key * Hkv + g) * kHeadDim + ch * kVec, x);
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e) x[e] = 0.f;
    }
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) a = fmaf(qv[e], x[e], a);
    a = sum16(a);
    if (kChunks == 32) a += __shfl_xor(a, 16);  // fp32 rows span 32 lanes
    if (i % kChunks == ch) {
      mykey = j;
      s = key < k1 ? a * sl2e : -INFINITY;
    }
  }
  const float m = block_max(s, red);
  const float p = s > -INFINITY ? __builtin_amdgcn_exp2f(s - m) : 0.f;
  if (mykey >= 0) ps[mykey] = p;
  const float l = block_sum(p, red);  // also publishes ps
  // u: thread (key group kg of 16 keys, 16-byte column group cv) sums its
  // keys' V over the group's columns; the 16 key groups are added in LDS
  constexpr int kColGroups = kChunks;
  constexpr int kKeyGroups = kThreads / kColGroups;
  constexpr int kPerGroup = kSplit / kKeyGroups;
  const int cv = tid % kColGroups, kg = tid / kColGroups;
  float acc[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc[e] = 0.f;
  const int nk = (int)(k1 - k0);
#pragma unroll 4
  for (int j = kg * kPerGroup; j < kg * kPerGroup + kPerGroup; ++j) {
    if (j >= nk) break;
    float x[kVec];
    ld16(V + ((k0 + j) * Hkv + g) * kHeadDim + cv * kVec, x);
    const float pj = ps[j];
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[e] = fmaf(pj, x[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) us[kg][cv * kVec + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    float u = 0.f;
#pragma unroll
    for (int q = 0; q < kKeyGroups; ++q) u += us[q][tid];
    out[2 + tid] = u;
  }
  if (tid == 0) {
    out[0] = m;
    out[1] = l;
  }
}

// One workgroup of 128 threads per (row, head): merge its k * splits
// partials. The max M and the weights 2^(m - M) (0 for empty partials) are
// computed 128 partials at a time by all threads; each thread then adds its
// dimension of u over those partials (independent loads; an empty partial
// has w = 0 and u = 0).
template <typename T>
__global__ __launch_bounds__(kHeadDim) void decode_merge(const float* __restrict__ part,
                                                         int nparts, T* __restrict__ O,
                                                         float* __restrict__ lse_out) {
  __shared__ float ws[kHeadDim];
  __shared__ float red[2];
  const int tid = threadIdx.x;
  const int64_t rh = blockIdx.x;
  const float* p = part + rh * nparts * kPart;
  auto wave_max = [](float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
  };
  auto wave_sum = [](float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
  };
  float M = -INFINITY;
  for (int i = tid; i < nparts; i += kHeadDim)
    if (p[(int64_t)i * kPart + 1] > 0.f) M = fmaxf(M, p[(int64_t)i * kPart]);
  M = wave_max(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  __syncthreads();
  float L = 0.f, u = 0.f;
  for (int i0 = 0; i0 < nparts; i0 += kHeadDim) {
    const int i = i0 + tid;
    float w = 0.f;
    if (i < nparts) {
      const float l = p[(int64_t)i * kPart + 1];
      if (l > 0.f) {  // empty partials carry no weight (and no u)
        w = __builtin_amdgcn_exp2f(p[(int64_t)i * kPart] - M);
        L = fmaf(w, l, L);
      }
    }
    ws[tid] = w;
    __syncthreads();
    const int cnt = nparts - i0 < kHeadDim ? nparts - i0 : kHeadDim;
    // empty partials have w = 0 and u = 0: no branch, independent loads
    float u4[4] = {0.f, 0.f, 0.f, 0.f};
    int j = 0;
    for (; j + 8 <= cnt; j += 8) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p[(int64_t)(i0 + j + e) * kPart + 2 + tid];
#pragma unroll
      for (int e = 0; e < 8; ++e) u4[e & 3] = fmaf(ws[j + e], x[e], u4[e & 3]);
    }
    for (; j < cnt; ++j) u4[0] = fmaf(ws[j], p[(int64_t)(i0 + j) * kPart + 2 + tid], u4[0]);
    u += (u4[0] + u4[1]) + (u4[2] + u4[3]);
    __syncthreads();
  }
  L = wave_sum(L);
  if ((tid & 63) == 0) red[tid >> 6] = L;
  __syncthreads();
  L = red[0] + red[1];
  st(O + rh * kHeadDim + tid, u / L);
  if (lse_out && tid == 0) lse_out[rh] = M + __log2f(L);
}

template <typename T>
hipError_t run(const Prob& P, const Blocks& Tb, const T* q, const T* k, const T* v,
               const int32_t* sel, float* part, T* o, float* lse_out, hipStream_t s) {
  const int splits = decode_splits(P);
  const int64_t items = P.Nq * P.Hq * (int64_t)P.k * splits;
  decode_partial<T><<<(unsigned)items, kThreads, 0, s>>>(q, k, v, sel, Tb.start, Tb.len,
                                                        Tb.row_blk, P.q0, P.Hq, P.Hkv, P.G, P.k,
                                                        splits, P.scale * kLog2e, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_merge<T><<<(unsigned)(P.Nq * P.Hq), kHeadDim, 0, s>>>(part, P.k * splits, o, lse_out);
  return hipGetLastError();
}

}  // namespace

int decode_splits(const Prob& P) { return (int)ceil_div(P.B, kSplit); }

size_t decode_part_bytes(const Prob& P) {
  return sizeof(float) * kPart * (size_t)(P.Nq * P.Hq) * P.k * decode_splits(P);
}

hipError_t launch_decode(const Prob& P, const Blocks& T, const void* q, const void* k,
                         const void* v, const int32_t* sel, float* part, void* o, float* lse_out,
                         hipStream_t s) {
  if (P.dtype == MOBA_DTYPE_BF16)
    return run<uint16_t>(P, T, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sel,
                         part, (uint16_t*)o, lse_out, s);
  return run<float>(P, T, (const float*)q, (const float*)k, (const float*)v, sel, part, (float*)o,
                    lse_out, s);
}

}  // namespace moba
