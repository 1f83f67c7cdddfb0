// moba_attn (fp32) — the fp32 build of the history and own-block attention
// stages (PaperTrace "2.1.3 MoBA", eqs. (5)-(8)), used when Q, K, V and O are
// fp32. gfx950 has no fp32 path through the bf16 matrix cores that keeps fp32
// accuracy, so these are vector-ALU kernels: four lanes share one query (32
// head-dim elements each), keys stream through LDS in tiles of 32, and the
// online softmax keeps fp32 statistics. Same inputs, outputs and partial
// layout as the bf16 kernels, with fp32 partials.
#include "moba_internal.hpp"

namespace moba {

hipError_t launch_attn_hist_bf16(const Prob& P, const Blocks& T, const BucketPlan& bp,
                                 const void* Q, const void* K, const void* Vt,
                                 const BucketBufs& b, void* part_o, float* part_lse,
                                 hipStream_t s);
hipError_t launch_attn_self_bf16(const Prob& P, const Blocks& T, const void* Q, const void* K,
                                 const void* Vt, const void* part_o, const float* part_lse,
                                 void* O, float* lse_out, hipStream_t s);

namespace {

constexpr int kQ = 128;                 // queries per workgroup
constexpr int kSub = 4;                 // lanes per query
constexpr int kDim = kHeadDim / kSub;   // 32 elements per lane
constexpr int kThreads = kQ * kSub;     // 512
constexpr int KT = 32;                  // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

struct QState {
  float q[kDim];
  float o[kDim];
  float m, l;
};

__device__ inline void load_tile(float* ks, float* vs, const float* __restrict__ K,
                                 const float* __restrict__ V, int64_t key0, int nvalid, int Hkv,
                                 int g) {
  // 32 keys x 128 floats each for K and V; 512 threads, 8 float4 per thread
  for (int i = threadIdx.x; i < KT * (kHeadDim / 4); i += kThreads) {
    const int key = i / (kHeadDim / 4), c4 = i % (kHeadDim / 4);
    float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
    if (key < nvalid) {
      const size_t off = ((size_t)(key0 + key) * Hkv + g) * kHeadDim + 4 * c4;
      kv = *reinterpret_cast<const float4*>(K + off);
      vv = *reinterpret_cast<const float4*>(V + off);
    }
    reinterpret_cast<float4*>(ks)[i] = kv;
    reinterpret_cast<float4*>(vs)[i] = vv;
  }
}

// Process one staged tile of keys for this lane's query. valid(key) decides the mask.
template <typename MaskFn>
__device__ inline void tile_step(QState& S, const float* ks, const float* vs, int sub, float sl2e,
                                 MaskFn valid) {
  float z[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    const float* kr = ks + t * kHeadDim + sub * kDim;
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < kDim; ++c) a = fmaf(S.q[c], kr[c], a);
    a += __shfl_xor(a, 1);
    a += __shfl_xor(a, 2);
    z[t] = valid(t) ? a * sl2e : -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < KT; ++t) mx = fmaxf(mx, z[t]);
  const float mnew = fmaxf(S.m, mx);
  const float muse = (mnew == -INFINITY) ? 0.f : mnew;
  const float alpha = __builtin_amdgcn_exp2f(S.m - muse);
  S.m = mnew;
  S.l *= alpha;
#pragma unroll
  for (int c = 0; c < kDim; ++c) S.o[c] *= alpha;
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    const float p = __builtin_amdgcn_exp2f(z[t] - muse);
    S.l += p;
    const float* vr = vs + t * kHeadDim + sub * kDim;
#pragma unroll
    for (int c = 0; c < kDim; ++c) S.o[c] = fmaf(p, vr[c], S.o[c]);
  }
}

__device__ inline void init_state(QState& S, const float* qrow, bool valid, int sub) {
#pragma unroll
  for (int c = 0; c < kDim; ++c) {
    S.q[c] = valid ? qrow[sub * kDim + c] : 0.f;
    S.o[c] = 0.f;
  }
  S.m = -INFINITY;
  S.l = 0.f;
}

__global__ __launch_bounds__(kThreads) void attn_hist_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const int32_t* __restrict__ bstart, const int32_t* __restrict__ tile_map,
    const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ bin_off, const int32_t* __restrict__ scalars,
    const uint32_t* __restrict__ entries, float* __restrict__ part_o, float* __restrict__ part_lse,
    int Hkv, int B, int KH, int64_t nh, float sl2e, int Hq, int Hs, int h0, int64_t bin0,
    int64_t bin1) {
  __shared__ float ks[KT * kHeadDim];
  __shared__ float vs[KT * kHeadDim];
  // the tiles of this attention pass's bins [bin0, bin1)
  const int64_t w = tile_off[bin0] + blockIdx.x;
  if (w >= tile_off[bin1]) return;
  const int bin = tile_map[w];
  const int64_t e_begin = bin_off[bin] + (w - tile_off[bin]) * (int64_t)kTileQ;
  const int64_t e_end = bin_off[bin + 1];
  const int g = (int)(bin / nh);
  const int64_t j = bin % nh;
  const int qi = threadIdx.x / kSub, sub = threadIdx.x % kSub;
  for (int64_t base = e_begin; base < e_begin + kTileQ && base < e_end; base += kQ) {
    const int64_t my_e = base + qi;
    const bool valid = my_e < e_end;
    const uint32_t ev = valid ? entries[my_e] : 0u;
    // ev / KH = row * Hs + (head - h0) over the pass's heads; Q row = row * Hq + head
    const int64_t pr = ev / (uint32_t)KH;
    QState S;
    init_state(S, Q + (pr + (pr / Hs) * (Hq - Hs) + h0) * kHeadDim, valid, sub);
    for (int k0 = 0; k0 < B; k0 += KT) {
      const int nv = (B - k0) < KT ? B - k0 : KT;
      __syncthreads();
      load_tile(ks, vs, K, V, (int64_t)bstart[j] + k0, nv, Hkv, g);
      __syncthreads();
      tile_step(S, ks, vs, sub, sl2e, [&](int t) { return t < nv; });
    }
    if (valid) {
      const float inv = 1.f / S.l;
      float* dst = part_o + (size_t)ev * kHeadDim + sub * kDim;
#pragma unroll
      for (int c = 0; c < kDim; ++c) dst[c] = S.o[c] * inv;
      if (sub == 0) part_lse[ev] = S.m + __builtin_log2f(S.l);
    }
  }
}

__global__ __launch_bounds__(kThreads) void attn_self_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const int32_t* __restrict__ bstart, const int32_t* __restrict__ qstart,
    const int32_t* __restrict__ qlen, const int32_t* __restrict__ qpos,
    const int32_t* __restrict__ blo, const float* __restrict__ part_o,
    const float* __restrict__ part_lse, float* __restrict__ O, float* __restrict__ lse_out, int Hq,
    int Hkv, int G, int KH, int64_t n, int tiles_per_block, float sl2e, int g0, int gs) {
  __shared__ float ks[KT * kHeadDim];
  __shared__ float vs[KT * kHeadDim];
  const int g = g0 + (int)blockIdx.y;  // this attention pass's KV heads [g0, g0 + gs)
  const int64_t c = n - 1 - (int64_t)(blockIdx.x / tiles_per_block);
  const int tile = tiles_per_block - 1 - (int)(blockIdx.x % tiles_per_block);
  // keys from the block's first row; query rows and their positions from its query range
  const int64_t key0 = bstart[c], qrow0 = qstart[c], pos0 = qpos[c];
  const int64_t npairs = (int64_t)qlen[c] * G;
  const int64_t p0 = (int64_t)tile * kQ;
  if (p0 >= npairs) return;
  const int64_t plast = (p0 + kQ - 1 < npairs) ? p0 + kQ - 1 : npairs - 1;
  const int64_t last_row = pos0 + plast / G;
  const int qi = threadIdx.x / kSub, sub = threadIdx.x % kSub;
  const int64_t my_pi = p0 + qi;
  const bool valid = my_pi < npairs;
  const int64_t my_row = valid ? pos0 + my_pi / G : -1;
  const int my_h = valid ? g * G + (int)(my_pi % G) : 0;
  const int64_t ph = valid ? (qrow0 + my_pi / G) * Hq + my_h : 0;
  QState S;
  init_state(S, Q + ph * kHeadDim, valid, sub);
  for (int64_t k0 = key0; k0 <= last_row; k0 += KT) {
    const int64_t rem = last_row + 1 - k0;
    const int nv = rem < KT ? (int)rem : KT;
    __syncthreads();
    load_tile(ks, vs, K, V, k0, nv, Hkv, g);
    __syncthreads();
    tile_step(S, ks, vs, sub, sl2e, [&](int t) { return t < nv && k0 + t <= my_row; });
  }
  if (!valid) return;
  float l = S.l;
  float M = S.m;
  if (part_o != nullptr && KH > 0) {
    const int64_t nbefore = c - blo[c];  // earlier blocks of the row's sequence
    const int64_t nhist = nbefore < KH ? nbefore : KH;
    // the pass's partial slots of this (row, head)
    const int64_t ebase = ((qrow0 + my_pi / G) * (gs * G) + (my_h - g0 * G)) * KH;
    for (int64_t s = 0; s < nhist; ++s) M = fmaxf(M, part_lse[ebase + s]);
    const float ws = __builtin_amdgcn_exp2f(S.m - M);
    l *= ws;
#pragma unroll
    for (int cc = 0; cc < kDim; ++cc) S.o[cc] *= ws;
    for (int64_t s = 0; s < nhist; ++s) {
      const float wgt = __builtin_amdgcn_exp2f(part_lse[ebase + s] - M);
      l += wgt;
      const float* src = part_o + (size_t)(ebase + s) * kHeadDim + sub * kDim;
#pragma unroll
      for (int cc = 0; cc < kDim; ++cc) S.o[cc] = fmaf(wgt, src[cc], S.o[cc]);
    }
  }
  if (lse_out && sub == 0) lse_out[ph] = M + __builtin_log2f(l);  // log2-sum-exp of the row
  const float inv = 1.f / l;
  float* dst = O + ph * kHeadDim + sub * kDim;
#pragma unroll
  for (int cc = 0; cc < kDim; ++cc) dst[cc] = S.o[cc] * inv;
}

}  // namespace

hipError_t launch_attn_hist(const Prob& P, const Blocks& T, const BucketPlan& bp, const void* Q,
                            const void* K, const void* V, const void* Vt, const BucketBufs& b,
                            void* part_o, float* part_lse, hipStream_t s) {
  if (P.dtype == MOBA_DTYPE_BF16)
    return attn_hist_q64_supported(P)
               ? launch_attn_hist_q64_bf16(P, T, bp, Q, K, Vt, b, part_o, part_lse, s)
               : launch_attn_hist_bf16(P, T, bp, Q, K, Vt, b, part_o, part_lse, s);
  if (P.nh <= 0 || P.KH <= 0 || bp.max_tiles <= 0) return hipSuccess;
  attn_hist_f32<<<(unsigned)pass_max_tiles(P), kThreads, 0, s>>>(
      (const float*)Q, (const float*)K, (const float*)V, T.start, b.tile_map, b.tile_off,
      b.bin_off, b.scalars, b.entries, (float*)part_o, part_lse, P.Hkv, P.B, P.KH, P.nh,
      P.scale * kLog2e, P.Hq, pass_heads(P), pass_h0(P), (int64_t)P.g0 * P.nh,
      (int64_t)(P.g0 + P.gs) * P.nh);
  return hipGetLastError();
}

hipError_t launch_attn_self(const Prob& P, const Blocks& T, const void* Q, const void* K,
                            const void* V, const void* Vt, const void* part_o,
                            const float* part_lse, void* O, float* lse_out, hipStream_t s) {
  if (P.dtype == MOBA_DTYPE_BF16)
    return launch_attn_self_bf16(P, T, Q, K, Vt, part_o, part_lse, O, lse_out, s);
  const bool merge = part_o != nullptr && P.KH > 0;
  const int tiles_per_block = (int)ceil_div((int64_t)P.B * P.G, kQ);
  dim3 grid((unsigned)(P.n * tiles_per_block), (unsigned)P.gs);
  attn_self_f32<<<grid, kThreads, 0, s>>>(
      (const float*)Q, (const float*)K, (const float*)V, T.start, T.qstart, T.qlen, T.qpos, T.lo,
      merge ? (const float*)part_o : nullptr, merge ? part_lse : nullptr, (float*)O, lse_out, P.Hq,
      P.Hkv, P.G, merge ? P.KH : 0, P.n, tiles_per_block, P.scale * kLog2e, P.g0, P.gs);
  return hipGetLastError();
}

}  // namespace moba
