// moba_attn (bf16) — exact softmax attention over the selected blocks on the
// gfx950 matrix cores (PaperTrace "2.1.3 MoBA": history branch eq. (6) and
// causal own-block branch eq. (5), merged by eqs. (7)-(8); section 3.1 steps
// 4-5; section 5.4 on tiling queries per KV block).
//
// Tile engine shared by both kernels. A wavefront owns 32 queries; a
// workgroup of 4 waves streams one K/V block in 64-key tiles through LDS
// (double buffered, one barrier per tile) so every tile read from HBM/L2
// serves 128 queries. Per tile and wave:
//   S^T = K Q^T   8 x v_mfma_f32_32x32x16_bf16 per 32 keys (keys on rows,
//                 queries on columns, so each lane holds 16 keys of one query
//                 and a softmax row needs one cross-half exchange);
//   online softmax in the exp2 domain, fp32 statistics (m, l);
//   O^T += V^T P^T  the P accumulator registers are reused directly as the B
//                 operand; V is stored transposed in LDS with its keys
//                 permuted to match, so each A operand is one 16-byte read.
// History kernel: one workgroup per 128 routed queries of one (KV head,
// block) list, full (non-causal) block; writes the normalised partial output
// (fp16) and its log2-sum-exp. Own-block kernel: causal inside the block,
// then merges the history partials of its queries (eqs. (7)-(8)) and writes O.
#include "moba_internal.hpp"

namespace moba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int KT = 64;                      // keys per tile
constexpr int KS_STRIDE = kHeadDim + 8;     // bf16 per K row in LDS
constexpr int VT_STRIDE = KT + 8;           // bf16 per V^T row in LDS
constexpr int KS_ELEMS = KT * KS_STRIDE;
constexpr int VT_ELEMS = kHeadDim * VT_STRIDE;
constexpr float kLog2e = 1.4426950408889634f;

struct __align__(16) Smem {
  uint16_t k[2][KS_ELEMS];
  uint16_t v[2][VT_ELEMS];
};

struct Prefetch {
  uint4 k[4];
  uint4 v[4];
};

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Global -> registers for keys [key0, key0 + 64) of KV head g; keys >= nvalid are zero.
__device__ inline void fetch_tile(Prefetch& pf, const uint16_t* __restrict__ K,
                                  const uint16_t* __restrict__ V, int64_t key0, int nvalid,
                                  int Hkv, int g, int tid) {
  const int kk = tid >> 2, dc = (tid & 3) * 32;
  if (kk < nvalid) {
    const uint4* src = reinterpret_cast<const uint4*>(K + ((key0 + kk) * Hkv + g) * kHeadDim + dc);
#pragma unroll
    for (int i = 0; i < 4; ++i) pf.k[i] = src[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) pf.k[i] = make_uint4(0, 0, 0, 0);
  }
  const int kq = tid >> 4, dof = (tid & 15) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = 4 * kq + i;
    if (key < nvalid)
      pf.v[i] = *reinterpret_cast<const uint4*>(V + ((key0 + key) * Hkv + g) * kHeadDim + dof);
    else
      pf.v[i] = make_uint4(0, 0, 0, 0);
  }
}

__device__ inline uint32_t u4_word(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

// Registers -> LDS: K row-major; V transposed to [d][key] with keys permuted
// so that key 16u + 8a + 4h + b of each 32-key half lands at 16u + 8h + 4a + b.
__device__ inline void store_tile(const Prefetch& pf, uint16_t* ks, uint16_t* vt, int tid) {
  const int kk = tid >> 2, dc = (tid & 3) * 32;
  uint4* dst = reinterpret_cast<uint4*>(ks + kk * KS_STRIDE + dc);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = pf.k[i];
  const int kq = tid >> 4, dof = (tid & 15) * 8;
  const int pbase = 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq >> 1) & 1);
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    const int w = dd >> 1, sh = (dd & 1) * 16;
    const uint32_t e0 = (u4_word(pf.v[0], w) >> sh) & 0xFFFFu;
    const uint32_t e1 = (u4_word(pf.v[1], w) >> sh) & 0xFFFFu;
    const uint32_t e2 = (u4_word(pf.v[2], w) >> sh) & 0xFFFFu;
    const uint32_t e3 = (u4_word(pf.v[3], w) >> sh) & 0xFFFFu;
    uint2 pk = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
    *reinterpret_cast<uint2*>(vt + (dof + dd) * VT_STRIDE + pbase) = pk;
  }
}

// Per-wave attention state for 32 queries.
struct Wave {
  bf16x8 q[8];    // B operand of S^T = K Q^T: Q[query][16ks + 8h .. +8]
  f32x16 o[4];    // O^T accumulators, d-blocks of 32
  float m;        // running max (log2 domain)
  float l;        // this lane's partial row sum
};

__device__ inline void wave_init(Wave& W, const uint16_t* qrow, bool valid, int h) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    uint4 u = valid ? *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * h) : make_uint4(0, 0, 0, 0);
    W.q[ks] = as_bf16x8(u);
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) W.o[db][r] = 0.f;
  W.m = -INFINITY;
  W.l = 0.f;
}

// Key row (0..31) of accumulator element r in the 32x32 MFMA output layout.
__device__ inline int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// One 64-key tile for one wave. Mask: key (tile-relative) valid iff < nvalid
// and, when causal, key0 + key <= qrow_abs.
template <bool CAUSAL>
__device__ inline void wave_tile(Wave& W, const uint16_t* ks, const uint16_t* vt, int lane,
                                 int nvalid, int64_t key0, int64_t qrow_abs, float sl2e,
                                 bool need_mask) {
  const int h = lane >> 5, lr = lane & 31;
  f32x16 s[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[sub][r] = 0.f;
    const uint16_t* krow = ks + (sub * 32 + lr) * KS_STRIDE + 8 * h;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 16 * kk));
      s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, W.q[kk], s[sub], 0, 0, 0);
    }
  }
  if (need_mask) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = sub * 32 + acc_row(r, h);
        bool ok = key < nvalid;
        if (CAUSAL) ok = ok && (key0 + key <= qrow_abs);
        if (!ok) s[sub][r] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mnew = fmaxf(W.m, mx * sl2e);
  const float muse = (mnew == -INFINITY) ? 0.f : mnew;
  const float alpha = __builtin_amdgcn_exp2f(W.m - muse);
  W.m = mnew;
  W.l *= alpha;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) W.o[db][r] *= alpha;
  bf16x8 p[2][2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[sub][8 * u + t], sl2e, -muse));
        W.l += e;
        p[sub][u][t] = (__bf16)e;
      }
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint16_t* vcol = vt + lr * VT_STRIDE + 32 * sub + 16 * u + 8 * h;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(vcol + 32 * db * VT_STRIDE));
        W.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[sub][u], W.o[db], 0, 0, 0);
      }
    }
}

// ----------------------------------------------------------------------------
// History attention: one workgroup = up to 128 routed entries of one bin.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void attn_hist_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ tile_map, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ bin_off, const int32_t* __restrict__ scalars,
    const uint32_t* __restrict__ entries, _Float16* __restrict__ part_o,
    float* __restrict__ part_lse, int Hkv, int B, int KH, int64_t nh, float sl2e) {
  __shared__ Smem sm;
  // XCD-aware order: workgroup i runs on XCD i % 8; give each XCD a contiguous
  // range of tiles so the tiles of one K/V block share that XCD's L2. The grid
  // is a multiple of 8, so this is a bijection on [0, gridDim.x).
  const int64_t per = gridDim.x / 8;
  const int64_t w = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= scalars[1]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bin = tile_map[w];
  const int64_t e_begin = bin_off[bin] + (w - tile_off[bin]) * (int64_t)kTileQ;
  const int64_t e_end = bin_off[bin + 1];
  const int g = (int)(bin / nh);
  const int64_t j = bin % nh;

  const int64_t my_e = e_begin + wave * 32 + (lane & 31);
  const bool valid = my_e < e_end;
  const uint32_t ev = valid ? entries[my_e] : 0u;
  const int64_t ph = ev / (uint32_t)KH;
  Wave W;
  wave_init(W, Q + ph * kHeadDim, valid, lane >> 5);

  const int64_t kbase = j * B;
  const int ntiles = (B + KT - 1) / KT;
  Prefetch pf;
  fetch_tile(pf, K, V, kbase, B < KT ? B : KT, Hkv, g, tid);
  store_tile(pf, sm.k[0], sm.v[0], tid);
  __syncthreads();
  const bool wave_live = (e_begin + wave * 32) < e_end;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int nv_next = (kt + 1 < ntiles) ? ((B - (kt + 1) * KT) < KT ? B - (kt + 1) * KT : KT) : 0;
    if (kt + 1 < ntiles) fetch_tile(pf, K, V, kbase + (int64_t)(kt + 1) * KT, nv_next, Hkv, g, tid);
    const int nv = (B - kt * KT) < KT ? B - kt * KT : KT;
    if (wave_live)
      wave_tile<false>(W, sm.k[kt & 1], sm.v[kt & 1], lane, nv, 0, 0, sl2e, nv < KT);
    if (kt + 1 < ntiles) store_tile(pf, sm.k[(kt + 1) & 1], sm.v[(kt + 1) & 1], tid);
    __syncthreads();
  }
  if (!valid) return;
  const float l = W.l + __shfl_xor(W.l, 32);
  const float inv = 1.f / l;
  const int h = lane >> 5;
  _Float16* dst = part_o + (size_t)ev * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * db + 8 * r4 + 4 * h;
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      h4 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = (_Float16)(W.o[db][4 * r4 + t] * inv);
      *reinterpret_cast<h4*>(dst + d0) = v;
    }
  if (h == 0) part_lse[ev] = W.m + __builtin_log2f(l);
}

// ----------------------------------------------------------------------------
// Own-block causal attention + merge. One workgroup = 128 (row, head) pairs of
// one KV-head group inside one block; pairs ordered pi = (row - cB) * G + hh.
// dense: the "block" is the whole sequence and there are no partials.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void attn_self_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const _Float16* __restrict__ part_o, const float* __restrict__ part_lse,
    uint16_t* __restrict__ O, int64_t N, int Hq, int Hkv, int G, int64_t B, int KH,
    int64_t n, int tiles_per_block, float sl2e) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.y;
  // heavier (later) row tiles first
  const int64_t c = n - 1 - (int64_t)(blockIdx.x / tiles_per_block);
  const int tile = tiles_per_block - 1 - (int)(blockIdx.x % tiles_per_block);
  const int64_t row0 = c * B;
  int64_t rows_c = N - row0;
  if (rows_c > B) rows_c = B;
  const int64_t npairs = rows_c * G;
  const int64_t p0 = (int64_t)tile * 128;
  if (p0 >= npairs) return;
  const int64_t plast = (p0 + 127 < npairs) ? p0 + 127 : npairs - 1;
  const int64_t last_row = row0 + plast / G;

  const int64_t my_pi = p0 + wave * 32 + (lane & 31);
  const bool valid = my_pi < npairs;
  const int64_t my_row = valid ? row0 + my_pi / G : -1;
  const int my_h = valid ? g * G + (int)(my_pi % G) : 0;
  const int64_t ph = valid ? my_row * Hq + my_h : 0;
  Wave W;
  wave_init(W, Q + ph * kHeadDim, valid, lane >> 5);

  // row range of this wave (for skipping fully masked tiles / unmasked tiles)
  const int64_t wp0 = p0 + wave * 32;
  const bool wave_live = wp0 < npairs;
  const int64_t wp1 = (wp0 + 31 < npairs) ? wp0 + 31 : npairs - 1;
  const int64_t wrow_min = row0 + wp0 / G;
  const int64_t wrow_max = row0 + wp1 / G;

  const int64_t nkeys = last_row - row0 + 1;
  const int ntiles = (int)((nkeys + KT - 1) / KT);
  Prefetch pf;
  fetch_tile(pf, K, V, row0, nkeys < KT ? (int)nkeys : KT, Hkv, g, tid);
  store_tile(pf, sm.k[0], sm.v[0], tid);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int64_t key0 = row0 + (int64_t)kt * KT;
    if (kt + 1 < ntiles) {
      const int64_t rem = nkeys - (int64_t)(kt + 1) * KT;
      fetch_tile(pf, K, V, key0 + KT, rem < KT ? (int)rem : KT, Hkv, g, tid);
    }
    const int64_t remk = nkeys - (int64_t)kt * KT;
    const int nv = remk < KT ? (int)remk : KT;
    if (wave_live && key0 <= wrow_max) {
      const bool need_mask = (key0 + KT - 1 > wrow_min) || nv < KT;
      wave_tile<true>(W, sm.k[kt & 1], sm.v[kt & 1], lane, nv, key0, my_row, sl2e, need_mask);
    }
    if (kt + 1 < ntiles) store_tile(pf, sm.k[(kt + 1) & 1], sm.v[(kt + 1) & 1], tid);
    __syncthreads();
  }
  if (!valid) return;
  const int h = lane >> 5;
  float l = W.l + __shfl_xor(W.l, 32);
  if (part_o != nullptr && KH > 0) {
    // merge with the history partials of this (row, head): eqs. (7)-(8)
    const int64_t nhist = c < KH ? c : KH;
    const int64_t ebase = ph * KH;
    float M = W.m;
    for (int64_t s = 0; s < nhist; ++s) M = fmaxf(M, part_lse[ebase + s]);
    const float ws = __builtin_amdgcn_exp2f(W.m - M);
    l *= ws;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) W.o[db][r] *= ws;
    for (int64_t s = 0; s < nhist; ++s) {
      const float wgt = __builtin_amdgcn_exp2f(part_lse[ebase + s] - M);
      l += wgt;
      const _Float16* src = part_o + (size_t)(ebase + s) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          const h4 v = *reinterpret_cast<const h4*>(src + 32 * db + 8 * r4 + 4 * h);
#pragma unroll
          for (int t = 0; t < 4; ++t) W.o[db][4 * r4 + t] += wgt * (float)v[t];
        }
    }
  }
  const float inv = 1.f / l;
  uint16_t* dst = O + ph * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      typedef __bf16 b4 __attribute__((ext_vector_type(4)));
      b4 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = (__bf16)(W.o[db][4 * r4 + t] * inv);
      *reinterpret_cast<b4*>(dst + 32 * db + 8 * r4 + 4 * h) = v;
    }
}

}  // namespace

hipError_t launch_attn_hist_bf16(const Prob& P, const BucketPlan& bp, const void* Q, const void* K,
                                 const void* V, const BucketBufs& b, void* part_o, float* part_lse,
                                 hipStream_t s) {
  if (P.nh <= 0 || P.KH <= 0 || bp.max_tiles <= 0) return hipSuccess;
  const float sl2e = P.scale * kLog2e;
  const int64_t grid = ceil_div(bp.max_tiles, 8) * 8;
  attn_hist_bf16<<<(unsigned)grid, kThreads, 0, s>>>(
      (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, b.tile_map, b.tile_off, b.bin_off,
      b.scalars, b.entries, (_Float16*)part_o, part_lse, P.Hkv, P.B, P.KH, P.nh, sl2e);
  return hipGetLastError();
}

hipError_t launch_attn_self_bf16(const Prob& P, const void* Q, const void* K, const void* V,
                                 const void* part_o, const float* part_lse, void* O, bool dense,
                                 hipStream_t s) {
  const float sl2e = P.scale * kLog2e;
  const int64_t B = dense ? P.N : P.B;
  const int64_t n = dense ? 1 : P.n;
  const int tiles_per_block = (int)ceil_div(B * P.G, 128);
  dim3 grid((unsigned)(n * tiles_per_block), (unsigned)P.Hkv);
  attn_self_bf16<<<grid, kThreads, 0, s>>>(
      (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V,
      dense ? nullptr : (const _Float16*)part_o, dense ? nullptr : part_lse, (uint16_t*)O, P.N, P.Hq,
      P.Hkv, P.G, B, dense ? 0 : P.KH, n, tiles_per_block, sl2e);
  return hipGetLastError();
}

}  // namespace moba
