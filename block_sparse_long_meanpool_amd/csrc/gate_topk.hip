// moba_gate_topk — parameter-free gate and block selection
// (PaperTrace "2.1.3 MoBA": gate s_i = q . kbar_i of section 1 eq. (3); future
// blocks excluded and own block forced, section 2; k counts the own block,
// section 2.1; section 3.1 step 2).
//
// The selection must equal the one defined by exact scores (ties to the lower
// block index). Scores are therefore computed in two tiers:
//
//  1. Fast tier on the bf16 matrix cores. Each fp64 block key is split into
//     three bf16 planes (hi + mid + lo carries 24 significant bits, residual
//     <= 2^-24 |kbar|); Q is exactly bf16, so the three products are exact
//     and only the fp32 accumulation rounds (unit <= u = 2^-23 per rounding,
//     every product counted as a separate rounding). The hi plane sums into
//     two accumulators of 64 products each, the mid and lo planes into one
//     each, then s = (hi_a + hi_b) + (mid + lo). Error, with T = sum_c
//     |q_c kbar_c|: hi chains <= 64 u T (1 + 2^-8); mid chain <= 128 u 2^-8
//     (1 + 2^-8) T = 0.5 u T; lo chain and split residual <= 0.5 u T; three
//     additions <= 3 u T (each result is at most T in magnitude, to first
//     order). So |s_fast - s| <= 68.5 u T <= eps = 8.4e-6 |q| max_b |kbar_b|
//     (Cauchy-Schwarz, max over the KV head's blocks). A lane keeps
//     a sorted top-(KM) list of (score, block) keys for its half of a row's
//     candidates; the two halves merge and the row is certified when the
//     k-1'th and k'th scores differ by more than 2 eps (plus the key
//     truncation): then every exact score of the kept set exceeds every exact
//     score left out, so the kept set is the exact one.
//  2. Exact tier: rows that are not certified (near-ties; about 0.5% of the
//     rows of a 1M-row random layer) are marked in `sel` and a second kernel
//     re-scores each marked row in fp64 with one wave (lane per block, block
//     keys stored transposed so the reads coalesce) and selects exactly
//     (value descending, index ascending). fp32 inputs, diagnostics and
//     calls with a few rows (decode; one workgroup of 4 waves per pair) take
//     this exact path for every row.
//
// Group-shared routing ranks blocks by the group's summed query
// q_g = sum_h q_h (exact in fp64 for bf16 inputs of ordinary range). Its fast
// tier splits q_g into three bf16 planes as well and takes the six plane
// products that reach 2^-16 of the score: hi.hi over dims 0..63 and 64..127
// (two chains of 64), hi.mid + mid.hi (one chain of 256), hi.lo + lo.hi +
// mid.mid (one chain of 384); s = (A + B) + (C + D). With T = sum_c
// |q_g,c kbar_c|: A and B <= 64 u T (1 + 2^-8); C <= 256 u 2^-7 (1 + 2^-8) T
// = 2.01 u T; D <= 384 u 3 2^-16 T = 0.02 u T; the three products left out
// (mid.lo, lo.mid, lo.lo) <= 1.5 u T; the residuals of both splits <= u T;
// three additions <= 3 u T. So |s_fast - s| <= 71.8 u T <= 8.56e-6 |q_g|
// max_b |kbar_b|, and certification is as above.
//
// Workgroup = 4 waves x 32 (row, head) pairs of one KV-head group inside one
// block c (pairs pi = (row - cB) * G + hh). The bf16 planes of 32 history
// blocks (24 KB) are streamed into LDS per chunk with buffer_load ... lds into
// two buffers. The own block c is appended and each row is written ascending
// and -1 padded.
#include "moba_internal.hpp"

namespace moba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kPairs = 32 * kWaves;       // pairs per workgroup
constexpr int kChunk = 32;                // history blocks per LDS chunk
constexpr int kRowBytes = kHeadDim * 2;   // one bf16 plane row of one block
constexpr int kChunkRows = 3 * kChunk;    // (block, plane) rows per chunk
constexpr int kChunkElems = kChunkRows * kHeadDim;
constexpr float kEpsCoef = 8.4e-6f * 1.02f;  // error bound coefficient (see above) with margin
constexpr float kEpsCoefShared = 8.56e-6f * 1.02f;  // the same for group-shared routing
constexpr int kRawBufferFlags = 0x00020000;

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ inline int swz(int row, int c) { return c ^ (row & 15); }

// ---------------------------------------------------------------------------
// Split kernel: kbar fp64 [Hkv][nh][d] -> planes bf16 [Hkv][nh][3][d],
// per-block Euclidean norms fp32 [Hkv][nh] (rounded up) and a transposed fp64
// copy [Hkv][d][nhp] for the exact tier (planes NULL: the copy only).
// ---------------------------------------------------------------------------
__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline double bf16_to_f64(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }

__global__ __launch_bounds__(kHeadDim) void kbar_split(const double* __restrict__ kbar,
                                                       uint16_t* __restrict__ planes,
                                                       float* __restrict__ norms,
                                                       double* __restrict__ kbarT, int64_t nh,
                                                       int64_t nhp) {
  const int64_t blk = blockIdx.x;  // over Hkv * nh
  const int c = threadIdx.x;
  const double x = kbar[blk * kHeadDim + c];
  const int64_t g = blk / nh, b = blk % nh;
  kbarT[(g * kHeadDim + c) * nhp + b] = x;  // [Hkv][d][nhp]: lane-per-block reads coalesce
  if (!planes) return;  // the exact tier alone needs only the transposed copy
  const uint16_t hi = bf16_rne((float)x);
  const double r1 = x - bf16_to_f64(hi);
  const uint16_t mid = bf16_rne((float)r1);
  const double r2 = r1 - bf16_to_f64(mid);
  const uint16_t lo = bf16_rne((float)r2);
  uint16_t* out = planes + blk * 3 * kHeadDim;
  out[c] = hi;
  out[kHeadDim + c] = mid;
  out[2 * kHeadDim + c] = lo;
  __shared__ double sq[kHeadDim];
  sq[c] = x * x;
  __syncthreads();
  if (c == 0) {
    double s = 0.0;
    for (int i = 0; i < kHeadDim; ++i) s += sq[i];
    norms[blk] = (float)(sqrt(s) * (1.0 + 1e-6));
  }
}

// Largest block-key norm per KV head: maxnorm[g] = max_b norms[g][b].
__global__ __launch_bounds__(256) void kbar_maxnorm(const float* __restrict__ norms,
                                                    float* __restrict__ maxnorm, int64_t nh) {
  __shared__ float red[256];
  const int g = blockIdx.x;
  float m = 0.f;
  for (int64_t b = threadIdx.x; b < nh; b += 256) m = fmaxf(m, norms[(size_t)g * nh + b]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  if (threadIdx.x == 0) maxnorm[g] = red[0];
}

// ---------------------------------------------------------------------------
// Candidates travel as one sortable 32-bit key: the fp32 score mapped to an
// order-preserving unsigned integer, its lowest `ib` bits replaced by
// (2^ib - 1 - block) so that equal truncated scores order by lower block.
// Keys are unique, so a descending top-KM list is a plain max/min network
// (two integer ops per slot). Truncation lowers a score by at most 2^ib units
// in its last place; the certification below accounts for that.
// ---------------------------------------------------------------------------
__device__ inline uint32_t score_key(float x, int block, int ib) {
  const uint32_t u = __float_as_uint(x);
  // negative: every bit flipped; otherwise the sign bit set (one bitwise op)
  const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  const uint32_t low = (1u << ib) - 1u;
  return (k & ~low) | (low - (uint32_t)block);
}
__device__ inline float key_score(uint32_t k, int ib) {
  k &= ~((1u << ib) - 1u);
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
__device__ inline int key_block(uint32_t k, int ib) {
  const uint32_t low = (1u << ib) - 1u;
  return (int)(low - (k & low));
}

// Batcher's odd-even merge sort of 16 keys (63 compare-exchanges, against 80
// for the bitonic sort): larger key to the lower position, so the keys end
// in descending order (checked on the host for all 2^16 0-1 inputs, which
// by the 0-1 principle covers every input).
constexpr int kOddEven16[63][2] = {
    {0, 1}, {2, 3}, {4, 5}, {6, 7}, {8, 9}, {10, 11}, {12, 13}, {14, 15}, {0, 2}, {1, 3}, {4,
    6}, {5, 7}, {8, 10}, {9, 11}, {12, 14}, {13, 15}, {1, 2}, {5, 6}, {9, 10}, {13, 14}, {0, 4},
    {1, 5}, {2, 6}, {3, 7}, {8, 12}, {9, 13}, {10, 14}, {11, 15}, {2, 4}, {3, 5}, {10, 12}, {11,
    13}, {1, 2}, {3, 4}, {5, 6}, {9, 10}, {11, 12}, {13, 14}, {0, 8}, {1, 9}, {2, 10}, {3, 11},
    {4, 12}, {5, 13}, {6, 14}, {7, 15}, {4, 8}, {5, 9}, {6, 10}, {7, 11}, {2, 4}, {3, 5}, {6,
    8}, {7, 9}, {10, 12}, {11, 13}, {1, 2}, {3, 4}, {5, 6}, {7, 8}, {9, 10}, {11, 12}, {13, 14},
};

template <int KM>
struct KeyList {
  uint32_t k[KM];  // descending
  __device__ inline void init() {
#pragma unroll
    for (int t = 0; t < KM; ++t) k[t] = 0u;  // below every real key
  }
  __device__ inline void push(uint32_t x) {
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      const uint32_t hi = k[t] > x ? k[t] : x;  // unsigned max / min
      x = k[t] > x ? x : k[t];
      k[t] = hi;
    }
  }
  // Merge another descending list of KM keys (disjoint from this one): the
  // top KM of both are m_t = max(k[t], o[KM-1-t]), a bitonic sequence, which
  // one bitonic merge (with maximal pads first) sorts. Same result as KM
  // push() calls.
  __device__ inline void merge(const uint32_t (&o)[KM]) {
    constexpr int P = KM < 8 ? 8 : KM < 16 ? 16 : KM < 32 ? 32 : 64;  // room for >= 1 pad
    constexpr int PADS = P - KM;
    uint32_t m[P];
#pragma unroll
    for (int t = 0; t < KM; ++t) m[t] = k[t] > o[KM - 1 - t] ? k[t] : o[KM - 1 - t];
#pragma unroll
    for (int t = KM; t < P; ++t) m[t] = 0xFFFFFFFFu;  // above every real key
#pragma unroll
    for (int stride = P >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const uint32_t hi = m[i] > m[j] ? m[i] : m[j], lo = m[i] > m[j] ? m[j] : m[i];
          m[i] = hi;
          m[j] = lo;
        }
      }
#pragma unroll
    for (int t = 0; t < KM; ++t) k[t] = m[PADS + t];
  }
  // Add 16 keys at once: sort them descending (odd-even merge sort); then
  // m_t = max(k[t], c[KM-1-t]) is exactly the top KM of both lists (two
  // sorted lists, one read backwards) and is decreasing-then-increasing, so
  // with maximal keys appended it is bitonic and one bitonic merge of P =
  // 2^ceil(log2(KM + pads)) elements sorts it; the pads come first and are
  // dropped. Same result as 16 push() calls, in fewer operations.
  __device__ inline void push16(uint32_t (&c)[16]) {
#pragma unroll
    for (int q = 0; q < 63; ++q) {
      const int i = kOddEven16[q][0], j = kOddEven16[q][1];
      const uint32_t hi = c[i] > c[j] ? c[i] : c[j], lo = c[i] > c[j] ? c[j] : c[i];
      c[i] = hi;
      c[j] = lo;
    }
    constexpr int P = KM < 8 ? 8 : KM < 16 ? 16 : KM < 32 ? 32 : 64;  // room for >= 1 pad
    constexpr int PADS = P - KM;
    uint32_t m[P];
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      const uint32_t other = KM - 1 - t < 16 ? c[KM - 1 - t] : 0u;
      m[t] = k[t] > other ? k[t] : other;
    }
#pragma unroll
    for (int t = KM; t < P; ++t) m[t] = 0xFFFFFFFFu;  // above every real key
#pragma unroll
    for (int stride = P >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const uint32_t hi = m[i] > m[j] ? m[i] : m[j], lo = m[i] > m[j] ? m[j] : m[i];
          m[i] = hi;
          m[j] = lo;
        }
      }
#pragma unroll
    for (int t = 0; t < KM; ++t) k[t] = m[PADS + t];
  }
};

// out[0..n) = the n block indices of idx[0..n) in ascending order (n <= KM,
// indices distinct): a sorting network over the next power of two (16: the
// odd-even one above; else bitonic), entries past n padded with INT_MAX
// (they sort last and are not written).
template <int KM>
__device__ inline void write_sorted(const int (&idx)[KM], int n, int32_t* out) {
  constexpr int P = KM <= 4 ? 4 : KM <= 8 ? 8 : KM <= 16 ? 16 : 32;
  int a[P];
#pragma unroll
  for (int t = 0; t < P; ++t) a[t] = (t < KM && t < n) ? idx[t < KM ? t : 0] : 0x7FFFFFFF;
  if constexpr (P == 16) {  // the odd-even network, smaller index to the lower position
#pragma unroll
    for (int q = 0; q < 63; ++q) {
      const int i = kOddEven16[q][0], j = kOddEven16[q][1];
      const int lo = a[i] < a[j] ? a[i] : a[j], hi = a[i] < a[j] ? a[j] : a[i];
      a[i] = lo;
      a[j] = hi;
    }
#pragma unroll
    for (int t = 0; t < KM; ++t)
      if (t < n) out[t] = a[t];
    return;
  }
#pragma unroll
  for (int size = 2; size <= P; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const int lo = a[i] < a[j] ? a[i] : a[j], hi = a[i] < a[j] ? a[j] : a[i];
          const bool up = (i & size) == 0;  // the last stage sorts all P ascending
          a[i] = up ? lo : hi;
          a[j] = up ? hi : lo;
        }
      }
#pragma unroll
  for (int t = 0; t < KM; ++t)
    if (t < n) out[t] = a[t];
}

// Issue the copy of planes of blocks [cb, cb + 32) (clamped to nh) into one LDS buffer.
__device__ inline void load_chunk(uint16_t* lds, const uint16_t* __restrict__ planes_g,
                                  int64_t cb, int64_t nblk, int wave, int lane) {
  const int64_t have = (nblk - cb) < kChunk ? nblk - cb : kChunk;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(planes_g + cb * 3 * kHeadDim), 0, (int)(have * 3 * kRowBytes), kRawBufferFlags);
  // 96 rows of 256 B = 24 copies of 1 KB (4 rows each): 6 per wave
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int ii = wave * 6 + i;
    const int row = 4 * ii + (lane >> 4);
    const int c = swz(row, lane & 15);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds + 4 * ii * kHeadDim, 16,
                                             (unsigned)(row * kRowBytes + 16 * c), 0, 0, 0);
  }
}

__device__ inline void wait_chunk() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Scores S^T (32 blocks x 32 pairs) of one chunk: four accumulation chains,
// the hi plane over dims 0..63 and 64..127, the mid and lo planes, summed
// at the end as (hi_a + hi_b) + (mid + lo) (the error bound above).
__device__ inline void chunk_scores(const uint16_t* lds, const bf16x8 (&q)[8], int lane,
                                    f32x16& s) {
  const int h = lane >> 5, lr = lane & 31;
  // the rows' swizzle keys, opaque to the compiler so that it forms the 24
  // operand addresses here, per chunk, instead of keeping them all live
  // across the chunk loop
  int z0 = (3 * lr) & 15, z1 = (3 * lr + 1) & 15, z2 = (3 * lr + 2) & 15;
  asm volatile("" : "+v"(z0), "+v"(z1), "+v"(z2));
  f32x16 a0, a0b, a1, a2;
#pragma unroll
  for (int r = 0; r < 16; ++r) a0[r] = a0b[r] = a1[r] = a2[r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int c = 2 * kk + h;
    const int r0 = 3 * lr, r1 = 3 * lr + 1, r2 = 3 * lr + 2;
    const bf16x8 x0 = as_bf16x8(*reinterpret_cast<const uint4*>(lds + r0 * kHeadDim + 8 * (c ^ z0)));
    const bf16x8 x1 = as_bf16x8(*reinterpret_cast<const uint4*>(lds + r1 * kHeadDim + 8 * (c ^ z1)));
    const bf16x8 x2 = as_bf16x8(*reinterpret_cast<const uint4*>(lds + r2 * kHeadDim + 8 * (c ^ z2)));
    if (kk < 4)
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, q[kk], a0, 0, 0, 0);
    else
      a0b = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, q[kk], a0b, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1, q[kk], a1, 0, 0, 0);
    a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x2, q[kk], a2, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = (a0[r] + a0b[r]) + (a1[r] + a2[r]);
}

// Group-shared scores: the group query in three bf16 planes q[0..2] (hi,
// mid, lo); chains and their sum as in the shared-routing bound above.
__device__ inline void chunk_scores_shared(const uint16_t* lds, const bf16x8 (&q)[3][8], int lane,
                                           f32x16& s) {
  const int h = lane >> 5, lr = lane & 31;
  f32x16 a, b, c2, d;
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = b[r] = c2[r] = d[r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int c = 2 * kk + h;
    const int r0 = 3 * lr, r1 = 3 * lr + 1, r2 = 3 * lr + 2;
    const bf16x8 x0 = as_bf16x8(*reinterpret_cast<const uint4*>(lds + r0 * kHeadDim + 8 * swz(r0, c)));
    const bf16x8 x1 = as_bf16x8(*reinterpret_cast<const uint4*>(lds + r1 * kHeadDim + 8 * swz(r1, c)));
    const bf16x8 x2 = as_bf16x8(*reinterpret_cast<const uint4*>(lds + r2 * kHeadDim + 8 * swz(r2, c)));
    if (kk < 4)
      a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, q[0][kk], a, 0, 0, 0);
    else
      b = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, q[0][kk], b, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1, q[0][kk], c2, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, q[1][kk], c2, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x2, q[0][kk], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, q[2][kk], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1, q[1][kk], d, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = (a[r] + b[r]) + (c2[r] + d[r]);
}

constexpr int32_t kRefine = -2;  // sel marker: this row's history needs the exact tier
// sel record of an uncertified row whose undecided blocks are all in the fast
// tier's list: entry 0 = kBand - (n_in << 8 | n_end), entries 1.. hold the
// list's first n_end block indices, two 16-bit halves per entry, in fast
// order: n_in blocks certainly kept, then the band whose exact scores decide
// the remaining k-1-n_in places (every other block is certainly left out).
constexpr int32_t kBand = -(1 << 20);

template <typename T>
__device__ inline double widen(T x);
template <>
__device__ inline double widen<uint16_t>(uint16_t x) {
  return (double)__uint_as_float((uint32_t)x << 16);
}
template <>
__device__ inline double widen<float>(float x) {
  return (double)x;
}
template <>
__device__ inline double widen<double>(double x) {
  return x;
}

// Exact tier: one wave per ppw consecutive (row, head) pairs (64; a few
// rows use gate_refine_few instead); each marked row
// (or, with all_rows, every row) is re-scored in fp64 (a row with a band
// record only over its band, see kBand) — lane b handles blocks
// b, b+64, ... reading the transposed block keys (coalesced) against q
// staged in LDS — and selected by (value desc, index asc): each lane keeps a
// sorted list of its blocks (they arrive in increasing order), then KH rounds
// of wave arg-max over the list heads pick the kept blocks. Writes the whole
// row: kept blocks ascending, own block, -1 padding.
// Group-shared routing passes pairs (row, KV head) (Hq = Hkv, G = 1) and
// gq = the group size: the scoring query is the fp64 sum of the gq query
// heads ph * gq .. ph * gq + gq - 1 of Q, and the row (and margin) is written
// for each of them; a pair's marker sits in its first head's row.
template <typename T, int KM>
__global__ __launch_bounds__(64) void gate_refine(const T* __restrict__ Q,
                                                  const double* __restrict__ kbarT,
                                                  const int32_t* __restrict__ row_blk,
                                                  const int32_t* __restrict__ blo,
                                                  int32_t* __restrict__ sel,
                                                  float* __restrict__ margin, int64_t N, int Hq,
                                                  int G, int k, int64_t nhp, int all_rows,
                                                  int ppw, int gq) {
  __shared__ double qs[kHeadDim];
  const int lane = threadIdx.x;
  const int KH = k - 1;
  const int64_t nph = N * Hq;
  const int64_t ph0 = (int64_t)blockIdx.x * ppw;
  bool mine = false;
  {
    const int64_t ph = ph0 + lane;
    if (lane < ppw && ph < nph) {
      const int64_t c = row_blk[ph / Hq], lo = blo[c];
      if (c - lo > KH && KH > 0) {
        const int32_t rec = sel[ph * gq * k];
        mine = all_rows || rec == kRefine || (rec <= kBand && rec > kBand - 65536);
      } else if (all_rows) {  // every earlier block of the sequence is taken
        const int nsel = (int)(c - lo < KH ? c - lo : KH);
        for (int hh = 0; hh < gq; ++hh) {
          int32_t* out = sel + (ph * gq + hh) * k;
          if (margin) margin[ph * gq + hh] = __builtin_nanf("");  // nothing left out
          for (int a = 0; a < nsel; ++a) out[a] = (int32_t)(lo + a);
          out[nsel] = (int32_t)c;
          for (int a = nsel + 1; a < k; ++a) out[a] = -1;
        }
      }
    }
  }
  unsigned long long todo = __ballot(mine);
  while (todo) {
    const int l = __ffsll((long long)todo) - 1;
    todo &= todo - 1;
    const int64_t ph = ph0 + l;
    const int64_t c = row_blk[ph / Hq], lo = blo[c];
    const int g = (int)(ph % Hq) / G;
    const T* qrow = Q + ph * gq * kHeadDim;
    double q0 = 0.0, q1 = 0.0;  // the sum of gq bf16 or fp32 values is exact in fp64
    for (int hh = 0; hh < gq; ++hh) {
      q0 += widen<T>(qrow[(int64_t)hh * kHeadDim + 2 * lane]);
      q1 += widen<T>(qrow[(int64_t)hh * kHeadDim + 2 * lane + 1]);
    }
    qs[2 * lane] = q0;
    qs[2 * lane + 1] = q1;
    __syncthreads();
    const double* kt = kbarT + (int64_t)g * kHeadDim * nhp;
    const int32_t rec = all_rows ? 0 : sel[ph * gq * k];
    if (rec <= kBand && rec > kBand - 65536) {
      // Band record: the first n_in listed blocks are kept, and the best
      // KH - n_in of the listed blocks [n_in, n_end) by (exact score desc,
      // index asc) fill the other places. Lane t holds listed block t; the
      // band's lanes score their block in the same order of operations as
      // the full path below, so either path gives the same values.
      const int code = kBand - rec, n_in = code >> 8, n_end = code & 0xFF;
      const int32_t* recp = sel + ph * gq * k;
      int id = 0x7FFFFFFF;
      if (lane < n_end)
        id = (int)(((uint32_t)recp[1 + (lane >> 1)] >> (16 * (lane & 1))) & 0xFFFFu);
      bool cand = lane >= n_in && lane < n_end, kept = lane < n_in;
      double x = -INFINITY;
      if (cand) {
        double acc = 0.0;
#pragma unroll 16
        for (int d = 0; d < kHeadDim; ++d) acc = fma(qs[d], kt[(int64_t)d * nhp + id], acc);
        x = acc;
      }
      for (int rnd = n_in; rnd < KH; ++rnd) {
        double bv = cand ? x : -INFINITY;
        int bi = cand ? id : 0x7FFFFFFF;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const double ov = __shfl_xor(bv, off);
          const int oi = __shfl_xor(bi, off);
          if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
          }
        }
        if (cand && id == bi) {
          cand = false;
          kept = true;
        }
      }
      // each kept block's place in the ascending row: kept blocks below it
      int pos = 0;
      for (int t = 0; t < n_end; ++t) {
        const int oid = __shfl(id, t);
        const int ok = __shfl((int)kept, t);
        pos += (ok && oid < id) ? 1 : 0;
      }
      for (int hh = 0; hh < gq; ++hh) {
        int32_t* out = sel + (ph * gq + hh) * k;
        if (kept) out[pos] = id;
        if (lane == 0) out[KH] = (int32_t)c;
        if (lane > KH && lane < k) out[lane] = -1;
      }
      __syncthreads();  // qs is rewritten for the next row
      continue;
    }
    double v[KM];
    int ix[KM];
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      v[t] = -INFINITY;
      ix[t] = 0x7FFFFFFF;
    }
    for (int64_t b = lo + lane; b < c; b += 64) {
      double acc = 0.0;
#pragma unroll 16
      for (int d = 0; d < kHeadDim; ++d) acc = fma(qs[d], kt[(int64_t)d * nhp + b], acc);
      double x = acc;
      int xi = (int)b;
#pragma unroll
      for (int t = 0; t < KM; ++t) {
        const bool gt = x > v[t];
        const double nv = gt ? x : v[t];
        const int ni = gt ? xi : ix[t];
        x = gt ? v[t] : x;
        xi = gt ? ix[t] : xi;
        v[t] = nv;
        ix[t] = ni;
      }
    }
    int chosen[KM];
#pragma unroll
    for (int t = 0; t < KM; ++t) chosen[t] = 0x7FFFFFFF;
    double last = 0.0, next = 0.0;
    // with a margin output, one more round finds the best block left out
    const int rounds = margin ? KH + 1 : KH;
    for (int rnd = 0; rnd < rounds; ++rnd) {
      const int hi = ix[0];
      double bv = v[0];
      int bi = hi;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (hi == bi) {  // the winning lane pops its head
#pragma unroll
        for (int t = 0; t < KM - 1; ++t) {
          v[t] = v[t + 1];
          ix[t] = ix[t + 1];
        }
        v[KM - 1] = -INFINITY;
        ix[KM - 1] = 0x7FFFFFFF;
      }
#pragma unroll
      for (int t = 0; t < KM; ++t)
        if (t == rnd && rnd < KH) chosen[t] = bi;
      if (rnd == KH - 1) last = bv;
      if (rnd == KH) next = bv;
    }
    if (lane < gq) {
      if (margin) margin[ph * gq + lane] = KH > 0 ? (float)(last - next) : __builtin_nanf("");
      int32_t* out = sel + (ph * gq + lane) * k;
      write_sorted<KM>(chosen, KH, out);
      out[KH] = (int32_t)c;
      for (int a = KH + 1; a < k; ++a) out[a] = -1;
    }
    __syncthreads();  // qs is rewritten for the next row
  }
}

// SHARED: pairs are (row, KV head) (Hq = Hkv, G = 1); the scoring query is
// the fp64 sum of the pair's gq query heads of Q, split into three bf16
// planes here, and the row is written for each of those heads.
// Exact tier for a few rows (decode): a workgroup of 4 waves per (row, head)
// pair, the pair's candidate blocks spread over its 256 lanes (lane t takes
// blocks lo + t, lo + t + 256, ...), each lane keeping a sorted list of its
// blocks; then KH rounds (KH + 1 with margins) of workgroup arg-max by (value
// desc, index asc) — a shuffle reduction per wave, then over the 4 waves in
// LDS — pick the kept blocks. Every pair is written (kept blocks ascending,
// own block, -1 padding); group-shared pairs sum gq heads as gate_refine does.
template <typename T, int KM>
__global__ __launch_bounds__(256) void gate_refine_few(const T* __restrict__ Q,
                                                       const double* __restrict__ kbarT,
                                                       const int32_t* __restrict__ row_blk,
                                                       const int32_t* __restrict__ blo,
                                                       int32_t* __restrict__ sel,
                                                       float* __restrict__ margin, int Hq, int G,
                                                       int k, int64_t nhp, int gq) {
  __shared__ double qs[kHeadDim];
  __shared__ double wbest[4];
  __shared__ int wblk[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int KH = k - 1;
  const int64_t ph = blockIdx.x;
  const int64_t c = row_blk[ph / Hq], lo = blo[c];
  if (!(c - lo > KH && KH > 0)) {  // every earlier block of the sequence is taken
    if (tid < gq) {
      const int nsel = (int)(c - lo < KH ? c - lo : KH);
      int32_t* out = sel + (ph * gq + tid) * k;
      if (margin) margin[ph * gq + tid] = __builtin_nanf("");  // nothing left out
      for (int a = 0; a < nsel; ++a) out[a] = (int32_t)(lo + a);
      out[nsel] = (int32_t)c;
      for (int a = nsel + 1; a < k; ++a) out[a] = -1;
    }
    return;
  }
  const int g = (int)(ph % Hq) / G;
  if (tid < kHeadDim) {
    const T* qrow = Q + ph * gq * kHeadDim;
    double x = 0.0;  // the sum of gq bf16 or fp32 values is exact in fp64
    for (int hh = 0; hh < gq; ++hh) x += widen<T>(qrow[(int64_t)hh * kHeadDim + tid]);
    qs[tid] = x;
  }
  __syncthreads();
  double v[KM];
  int ix[KM];
#pragma unroll
  for (int t = 0; t < KM; ++t) {
    v[t] = -INFINITY;
    ix[t] = 0x7FFFFFFF;
  }
  const double* kt = kbarT + (int64_t)g * kHeadDim * nhp;
  for (int64_t b = lo + tid; b < c; b += 256) {
    double acc = 0.0;
#pragma unroll 32
    for (int d = 0; d < kHeadDim; ++d) acc = fma(qs[d], kt[(int64_t)d * nhp + b], acc);
    double x = acc;
    int xi = (int)b;
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      const bool gt = x > v[t];
      const double nv = gt ? x : v[t];
      const int ni = gt ? xi : ix[t];
      x = gt ? v[t] : x;
      xi = gt ? ix[t] : xi;
      v[t] = nv;
      ix[t] = ni;
    }
  }
  int chosen[KM];
#pragma unroll
  for (int t = 0; t < KM; ++t) chosen[t] = 0x7FFFFFFF;
  double last = 0.0, next = 0.0;
  const int rounds = margin ? KH + 1 : KH;
  for (int rnd = 0; rnd < rounds; ++rnd) {
    double bv = v[0];
    int bi = ix[0];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      wbest[wave] = bv;
      wblk[wave] = bi;
    }
    __syncthreads();
    bv = wbest[0];
    bi = wblk[0];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (wbest[w] > bv || (wbest[w] == bv && wblk[w] < bi)) {
        bv = wbest[w];
        bi = wblk[w];
      }
    __syncthreads();  // the slots are rewritten next round
    if (ix[0] == bi) {  // block indices are unique: exactly one lane pops its head
#pragma unroll
      for (int t = 0; t < KM - 1; ++t) {
        v[t] = v[t + 1];
        ix[t] = ix[t + 1];
      }
      v[KM - 1] = -INFINITY;
      ix[KM - 1] = 0x7FFFFFFF;
    }
#pragma unroll
    for (int t = 0; t < KM; ++t)
      if (t == rnd && rnd < KH) chosen[t] = bi;
    if (rnd == KH - 1) last = bv;
    if (rnd == KH) next = bv;
  }
  if (tid < gq) {
    if (margin) margin[ph * gq + tid] = (float)(last - next);
    int32_t* out = sel + (ph * gq + tid) * k;
    write_sorted<KM>(chosen, KH, out);
    out[KH] = (int32_t)c;
    for (int a = KH + 1; a < k; ++a) out[a] = -1;
  }
}

template <int KM, bool SHARED>
// Per-head routing asks for three waves per SIMD (three workgroups per
// compute unit; 48 KB of LDS each).
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(SHARED ? 1 : 3, SHARED ? 2 : 3))) void gate_topk_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ planes,
    const float* __restrict__ maxnorm, const int32_t* __restrict__ qstart,
    const int32_t* __restrict__ qlen, const int32_t* __restrict__ blo, int32_t* __restrict__ sel,
    int Hq, int G, int gq_arg, int k, int64_t n, int64_t nh, int tiles_per_block) {
  const int gq = SHARED ? gq_arg : 1;  // query heads per pair
  __shared__ __align__(16) uint16_t bufA[kChunkElems];
  __shared__ __align__(16) uint16_t bufB[kChunkElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, lr = lane & 31;
  const int g = blockIdx.y;
  const int64_t c = n - 1 - (int64_t)(blockIdx.x / tiles_per_block);
  const int tile = blockIdx.x % tiles_per_block;
  const int64_t row0 = qstart[c], rows_c = qlen[c];  // query rows of block c
  const int64_t lo = blo[c];  // candidates: blocks [lo, c) of the row's sequence
  const int64_t nc = c - lo;
  const int64_t npairs_c = rows_c * G;
  const int64_t pair0 = (int64_t)tile * kPairs;
  if (pair0 >= npairs_c) return;
  const int KH = k - 1;

  const int64_t pi = pair0 + wave * 32 + lr;
  const bool valid = pi < npairs_c;
  const int64_t r = row0 + (valid ? pi / G : 0);
  const int hq = g * G + (int)(valid ? pi % G : 0);
  // the pair's rows of sel: heads (r * Hq + hq) * gq + 0 .. gq-1
  int32_t* out = sel + ((size_t)r * Hq + hq) * gq * k;
  const int nsel = (int)(nc < KH ? nc : KH);

  if (nc <= KH || KH == 0) {  // every earlier block is taken: nothing to rank
    if (valid && h == 0) {
      for (int hh = 0; hh < gq; ++hh) {
        int32_t* o = out + hh * k;
        for (int a = 0; a < nsel; ++a) o[a] = (int32_t)(lo + a);
        o[nsel] = (int32_t)c;
        for (int a = nsel + 1; a < k; ++a) o[a] = -1;
      }
    }
    return;
  }

  // Q as the B operand: Q[pair][16kk + 8h .. +8]; |q|^2 from the same values
  constexpr int NP = SHARED ? 3 : 1;  // query planes
  const uint16_t* qrow = Q + ((size_t)r * Hq + hq) * gq * kHeadDim;
  bf16x8 q[NP][8];
  float qq = 0.f;
  if constexpr (!SHARED) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 u = valid ? *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * h)
                            : make_uint4(0, 0, 0, 0);
      q[0][kk] = as_bf16x8(u);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)q[0][kk][e];
        qq = fmaf(x, x, qq);
      }
    }
    qq += __shfl_xor(qq, 32);
  } else {
    // group query x = sum of the gq heads (exact in fp64), split like the block keys
    double ss = 0.0;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      double x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.0;
      for (int hh = 0; hh < gq; ++hh) {
        const uint4 u = valid ? *reinterpret_cast<const uint4*>(qrow + hh * kHeadDim + 16 * kk + 8 * h)
                              : make_uint4(0, 0, 0, 0);
        const bf16x8 b = as_bf16x8(u);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += (double)(float)b[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t p0 = bf16_rne((float)x[e]);
        const double r1 = x[e] - bf16_to_f64(p0);
        const uint16_t p1 = bf16_rne((float)r1);
        const uint16_t p2 = bf16_rne((float)(r1 - bf16_to_f64(p1)));
        q[0][kk][e] = __builtin_bit_cast(__bf16, p0);
        q[1][kk][e] = __builtin_bit_cast(__bf16, p1);
        q[2][kk][e] = __builtin_bit_cast(__bf16, p2);
        ss = fma(x[e], x[e], ss);
      }
    }
    ss += __shfl_xor(ss, 32);
    const float qn = (float)(sqrt(ss) * (1.0 + 1e-6));  // |x|, rounded up
    qq = qn * qn;
  }

  // candidates by local index b - lo in [0, nc)
  const uint16_t* planes_g = planes + ((size_t)g * nh + lo) * 3 * kHeadDim;
  const float kmax = maxnorm[g];
  int ib = 1;  // index bits for local blocks 0..nc-1
  while ((1ll << ib) < nc) ++ib;
  KeyList<KM> L;
  L.init();
  const int nchunks = (int)((nc + kChunk - 1) / kChunk);
  auto step = [&](int ch, uint16_t* cur, uint16_t* nxt) {
    if (ch + 1 < nchunks) load_chunk(nxt, planes_g, (int64_t)(ch + 1) * kChunk, nc, wave, lane);
    f32x16 s;
    if constexpr (SHARED)
      chunk_scores_shared(cur, q, lane, s);
    else
      chunk_scores(cur, q[0], lane, s);
    const int64_t cb = (int64_t)ch * kChunk;
    uint32_t c[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {  // blocks past the candidates give key 0, which never enters
      const int b = (int)cb + 8 * (e >> 2) + 4 * h + (e & 3);
      // a mask rather than a conditional, so no slot's key is formed under
      // a branch of its own (gate 7.89 -> 7.83 ms at the 1M-token layer)
      const uint32_t keep = (uint32_t)((b - (int)nc) >> 31);  // all ones for a candidate
      c[e] = score_key(s[e], b, ib) & keep;
    }
    L.push16(c);
    wait_chunk();
  };
  load_chunk(bufA, planes_g, 0, nc, wave, lane);
  wait_chunk();
  for (int ch = 0; ch < nchunks; ch += 2) {
    step(ch, bufA, bufB);
    if (ch + 1 < nchunks) step(ch + 1, bufB, bufA);
  }

  // merge the two halves of each row: both lanes end with the same list
  uint32_t other[KM];  // the partner's list as it was, before any merging
#pragma unroll
  for (int t = 0; t < KM; ++t) other[t] = __shfl_xor(L.k[t], 32);
  L.merge(other);

  // certification: kept (top KH) vs best left out. Decoded scores are at most
  // 2^ib units in the last place below the fp32 ones; the fp32 ones are within
  // eps of the exact ones.
  uint32_t kk_in = 0u, kk_out = 0u;
  int idx[KM];
#pragma unroll
  for (int t = 0; t < KM; ++t) {
    if (t == KH - 1) kk_in = L.k[t];
    if (t == KH) kk_out = L.k[t];
    idx[t] = (int)lo + key_block(L.k[t], ib);
  }
  const float theta = key_score(kk_in, ib), theta_n = key_score(kk_out, ib);
  const float big = fmaxf(fabsf(theta), fabsf(theta_n));
  const float trunc = ldexpf(big, ib - 22);  // >= 2^ib units in the last place of |score| <= big
  const float eps = (SHARED ? kEpsCoefShared : kEpsCoef) * sqrtf(qq) * 1.0001f * kmax;
  const bool certified = (theta - theta_n) > 2.f * eps + trunc + 1e-6f * big;
  // Uncertified: the blocks the exact tier has to decide. With margins as
  // above, list entry t < KH is certainly kept when its score exceeds the
  // (KH+1)-th by more than the certification margin (it beats every block
  // from rank KH+1 on), and entry t >= KH is certainly left out when the
  // KH-th exceeds it by the margin of its own magnitude (every one of the top
  // KH beats it); both sets are runs of the descending list. Blocks outside
  // the list score at most the list's last entry, so they are left out when
  // the left-out run starts inside the list (or the list holds every
  // candidate).
  const float m_in = 2.f * eps + trunc + 1e-6f * big;
  const int n_real = (int)(nc < KM ? nc : KM);
  int n_in = 0, n_end = n_real;
#pragma unroll
  for (int t = 0; t < KM; ++t) {
    const float ph = key_score(L.k[t], ib);
    if (t < KH && t == n_in && ph - theta_n > m_in) n_in = t + 1;
    const float mag = fmaxf(big, fabsf(ph));
    if (t >= KH && t < n_real && n_end == n_real &&
        theta - ph > 2.f * eps + ldexpf(mag, ib - 22) + 1e-6f * mag)
      n_end = t;
  }
  const bool band = (n_end < n_real || nc <= KM) && n_end <= 2 * KH;
  if (valid && h == 0) {
    if (certified) {
      for (int hh = 0; hh < gq; ++hh) {
        int32_t* o = out + hh * k;
        write_sorted<KM>(idx, KH, o);
        o[KH] = (int32_t)c;
        for (int a = KH + 1; a < k; ++a) o[a] = -1;
      }
    } else if (band) {
      out[0] = kBand - ((n_in << 8) | n_end);  // gate_refine writes the pair's rows
#pragma unroll
      for (int t = 0; t < KM; t += 2)
        if (t < n_end)
          out[1 + t / 2] = (int32_t)((uint32_t)idx[t] |
                                     ((t + 1 < n_end ? (uint32_t)idx[t + 1 < KM ? t + 1 : t] : 0u)
                                      << 16));
    } else {
      out[0] = kRefine;  // gate_refine writes the pair's rows
    }
  }

}

// Exact tier over every row of an N x Hq_eff problem with groups of G_eff
// (gq: query heads summed per pair, group-shared routing).
template <typename T>
hipError_t refine_all(const Prob& P, const Blocks& T_, const T* Q, int Hq_eff, int G_eff, int gq,
                      const double* kbarT, int64_t nhp, int32_t* sel, float* margin,
                      hipStream_t s) {
  // a few rows: a workgroup of 4 waves per (row, head) pair; else one wave
  // per 64 consecutive pairs
  const bool few = P.Nq <= kDecodeRows;
  const unsigned grid = (unsigned)(few ? P.Nq * Hq_eff : ceil_div(P.Nq * Hq_eff, 64));
  const int need = P.KH + 1;
#define MOBA_REFINE(KM)                                                                        \
  do {                                                                                         \
    if (few)                                                                                   \
      gate_refine_few<T, KM><<<grid, 256, 0, s>>>(Q, kbarT, T_.row_blk, T_.lo, sel, margin,  \
                                                  Hq_eff, G_eff, P.k, nhp, gq);              \
    else                                                                                       \
      gate_refine<T, KM><<<grid, 64, 0, s>>>(Q, kbarT, T_.row_blk, T_.lo, sel, margin, P.Nq, \
                                             Hq_eff, G_eff, P.k, nhp, 1, 64, gq);            \
  } while (0)
  if (need <= 4) MOBA_REFINE(4);
  else if (need <= 8) MOBA_REFINE(8);
  else if (need <= 12) MOBA_REFINE(12);
  else if (need <= 16) MOBA_REFINE(16);
  else MOBA_REFINE(32);
#undef MOBA_REFINE
  return hipGetLastError();
}

// Fast tier then the exact tier for its uncertified rows, on bf16 Q. Per-head
// routing: pairs (row, query head). Group-shared (SHARED): pairs (row, KV
// head), scored with the sum of the group's G query heads.
template <int KM, bool SHARED>
hipError_t launch_km(const Prob& P, const Blocks& T, const void* Q, const uint16_t* planes,
                     const float* maxnorm, const double* kbarT, int64_t nhp, int32_t* sel,
                     hipStream_t s) {
  const int Hq = SHARED ? P.Hkv : P.Hq, G = SHARED ? 1 : P.G, gq = SHARED ? P.G : 1;
  const int tiles_per_block = (int)ceil_div((int64_t)P.B * G, kPairs);
  // workgroups walk blocks from the last; a chunk's query rows sit in its last blocks
  dim3 grid((unsigned)(query_blocks(P) * tiles_per_block), (unsigned)P.Hkv);
  gate_topk_kernel<KM, SHARED><<<grid, kThreads, 0, s>>>(
      (const uint16_t*)Q, planes, maxnorm, T.qstart, T.qlen, T.lo, sel, Hq, G, gq, P.k, P.n,
      P.nh, tiles_per_block);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.nh <= 0 || P.KH <= 0) return e;
  const unsigned refine_grid = (unsigned)ceil_div(P.Nq * Hq, 64);
  gate_refine<uint16_t, KM><<<refine_grid, 64, 0, s>>>((const uint16_t*)Q, kbarT, T.row_blk, T.lo,
                                                      sel, nullptr, P.Nq, Hq, G, P.k, nhp, 0, 64,
                                                      gq);
  return hipGetLastError();
}

template <bool SHARED>
hipError_t launch_fast(const Prob& P, const Blocks& T, const void* Q, const uint16_t* planes,
                       const float* maxnorm, const double* kbarT, int64_t nhp, int32_t* sel,
                       hipStream_t s) {
  // list length: the k-1 kept blocks plus the best one left out, and two
  // more where the sorting networks cost the same, so that the undecided
  // blocks of an uncertified row usually fit in the list (a band record)
  const int need = P.KH + 1;
#define MOBA_FAST(KM) launch_km<KM, SHARED>(P, T, Q, planes, maxnorm, kbarT, nhp, sel, s)
  if (need <= 6) return MOBA_FAST(6);
  if (need <= 14) return MOBA_FAST(14);
  if (need <= 16) return MOBA_FAST(16);
  return MOBA_FAST(32);
#undef MOBA_FAST
}

int64_t padded_nh(const Prob& P) { return ceil_div(P.nh > 0 ? P.nh : 1, 64) * 64; }

struct GateScratch {
  double* kbarT;
  uint16_t* planes;
  float* norms;
  float* maxnorm;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

GateScratch carve(const Prob& P, void* scratch) {
  GateScratch g{};
  char* base = (char*)scratch;
  g.kbarT = (double*)base;
  base += align256(sizeof(double) * (size_t)P.Hkv * kHeadDim * padded_nh(P));
  g.planes = (uint16_t*)base;
  base += align256((size_t)P.Hkv * P.nh * 3 * kHeadDim * 2);
  g.norms = (float*)base;
  g.maxnorm = g.norms + (size_t)P.Hkv * P.nh;
  return g;
}

// All of the gate: block-key split, then for bf16 inputs with many rows the
// fast tier and the exact tier for its uncertified rows, else (exact_all,
// fp32 inputs, a few rows) the exact tier for every row; margin (nullable)
// receives each row's selection margin. Group-shared routing scores pairs
// (row, KV head) with the group's summed query and writes each head's row.
hipError_t run_gate(const Prob& P, const Blocks& T, const void* Q, const double* kbar,
                    void* scratch, int32_t* sel, float* margin, bool exact_all, hipStream_t s) {
  const GateScratch g = carve(P, scratch);
  const int64_t nhp = padded_nh(P);
  // fp32 inputs, diagnostics and a few rows take the exact tier alone
  const bool exact_only = P.dtype == MOBA_DTYPE_F32 || exact_all || P.Nq <= kDecodeRows;
  if (P.nh > 0 && P.KH > 0) {
    kbar_split<<<(unsigned)(P.Hkv * P.nh), kHeadDim, 0, s>>>(
        kbar, exact_only ? nullptr : g.planes, g.norms, g.kbarT, P.nh, nhp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!exact_only) {
      kbar_maxnorm<<<(unsigned)P.Hkv, 256, 0, s>>>(g.norms, g.maxnorm, P.nh);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  const bool shared = P.routing == MOBA_ROUTING_SHARED;
  const int Hq = shared ? P.Hkv : P.Hq, G = shared ? 1 : P.G, gq = shared ? P.G : 1;
  if (P.dtype == MOBA_DTYPE_F32)
    return refine_all<float>(P, T, (const float*)Q, Hq, G, gq, g.kbarT, nhp, sel, margin, s);
  if (exact_only)
    return refine_all<uint16_t>(P, T, (const uint16_t*)Q, Hq, G, gq, g.kbarT, nhp, sel, margin,
                                s);
  if (shared) return launch_fast<true>(P, T, Q, g.planes, g.maxnorm, g.kbarT, nhp, sel, s);
  return launch_fast<false>(P, T, Q, g.planes, g.maxnorm, g.kbarT, nhp, sel, s);
}

}  // namespace

size_t gate_scratch_bytes(const Prob& P) {
  return align256(sizeof(double) * (size_t)P.Hkv * kHeadDim * padded_nh(P)) +
         align256((size_t)P.Hkv * P.nh * 3 * kHeadDim * 2) +
         align256((size_t)P.Hkv * (P.nh + 1) * 4) + 1024;
}

hipError_t launch_gate_topk(const Prob& P, const Blocks& T, const void* Q, const double* kbar,
                            void* scratch, int32_t* sel, hipStream_t s) {
  return run_gate(P, T, Q, kbar, scratch, sel, nullptr, false, s);
}

hipError_t launch_gate_margin(const Prob& P, const Blocks& T, const void* Q, const double* kbar,
                              void* scratch, int32_t* sel, float* margin, hipStream_t s) {
  return run_gate(P, T, Q, kbar, scratch, sel, margin, true, s);
}

}  // namespace moba
