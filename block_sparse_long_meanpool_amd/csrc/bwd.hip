// Backward pass of MoBA attention with the block selection held fixed: the
// hard top-k gives no gradient to the ranking, so Q, K and V receive
// gradients only through the attended (query, key) pairs (PaperTrace
// "2.1.3 MoBA", section 5.3). For a query with candidate set I (eq. (4)),
// z_j = scale q.k_j, P = softmax(z) over I, o = sum P_j v_j and upstream
// gradient dO:
//   dV_j += P_j dO,  dP_j = dO.v_j,  D = dO.o,  dZ_j = P_j (dP_j - D),
//   dq = scale sum_j dZ_j k_j,  dK_j += scale dZ_j q.
// P_j is rebuilt from the forward's per-row log2-sum-exp (lse2, such that
// P_j = 2^(scale log2(e) q.k_j - lse2)), so no softmax statistics are
// recomputed. fp32 vector arithmetic throughout (4 lanes per query or key,
// 32 head-dim elements each); this is the path for fp32 inputs (bf16 inputs
// take the matrix-core kernels of bwd_bf16.hip, after bwd_delta below).
//   * dK, dV: key-stationary. One workgroup owns 64 keys of one block and
//     one KV head and walks every query that attends to them: the block's
//     routed history entries (the bucketed lists) and the causal rows of
//     the block itself, all G query heads. Each key's gradients are finished
//     in one workgroup and written once.
//   * dQ: query-stationary over the same work lists as the forward kernels
//     (history tiles of one bin, own-block row tiles); a query's pieces from
//     its blocks are summed with fp32 atomics, then scaled and converted.
#include "moba_internal.hpp"

namespace moba {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSub = 4;                // lanes per query (or key)
constexpr int kDim = kHeadDim / kSub;  // 32 elements per lane

template <typename T>
__device__ inline float ldf(const T* p, int64_t i);
template <>
__device__ inline float ldf<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
template <>
__device__ inline float ldf<float>(const float* p, int64_t i) {
  return p[i];
}

template <typename T>
__device__ inline void stf(T* p, int64_t i, float x);
template <>
__device__ inline void stf<uint16_t>(uint16_t* p, int64_t i, float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even
  p[i] = (uint16_t)(u >> 16);
}
template <>
__device__ inline void stf<float>(float* p, int64_t i, float x) {
  p[i] = x;
}

__device__ inline float quad_sum(float a) {  // over the 4 lanes of a query / key
  a += __shfl_xor(a, 1);
  a += __shfl_xor(a, 2);
  return a;
}

// D[ph] = dO[ph] . O[ph]
template <typename T>
__global__ void bwd_delta(const T* __restrict__ O, const T* __restrict__ dO,
                          float* __restrict__ delta, int64_t nph) {
  const int64_t ph = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / kSub;
  const int sub = threadIdx.x % kSub;
  float a = 0.f;
  if (ph < nph)
    for (int c = 0; c < kDim; ++c) {
      const int64_t i = ph * kHeadDim + sub * kDim + c;
      a = fmaf(ldf(O, i), ldf(dO, i), a);
    }
  a = quad_sum(a);
  if (ph < nph && sub == 0) delta[ph] = a;
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup (key tile of 64, block b, KV head g); 256 threads = 64
// keys x 4 lanes. Queries are staged 32 at a time in LDS (q, dO, lse2, D,
// position; position < 0 marks a history query, which sees every key).
// ---------------------------------------------------------------------------
constexpr int kKeysPerWG = 64;
constexpr int kQChunk = 32;

template <typename T>
__global__ __launch_bounds__(256) void bwd_dkv(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ bstart, const int32_t* __restrict__ blen,
    const int32_t* __restrict__ qstart, const int32_t* __restrict__ qlen,
    const int32_t* __restrict__ qpos, const int32_t* __restrict__ bin_off,
    const uint32_t* __restrict__ entries, T* __restrict__ dK, T* __restrict__ dV, int Hq, int Hkv,
    int G, int KH, int64_t nh, int tiles_per_block, float scale) {
  __shared__ float sq[kQChunk][kHeadDim];
  __shared__ float sdo[kQChunk][kHeadDim];
  __shared__ float slse[kQChunk], sdel[kQChunk];
  __shared__ int64_t spos[kQChunk];
  const int g = blockIdx.y;
  const int64_t b = blockIdx.x / tiles_per_block;
  const int kt = blockIdx.x % tiles_per_block;
  const int64_t key_first = bstart[b];
  const int nk = blen[b];
  const int key_local = kt * kKeysPerWG + (int)(threadIdx.x / kSub);
  const int sub = threadIdx.x % kSub;
  if (kt * kKeysPerWG >= nk) return;
  const bool kvalid = key_local < nk;
  const int64_t key = key_first + (kvalid ? key_local : 0);
  const float sl2e = scale * kLog2e;
  float kr[kDim], vr[kDim], dk[kDim], dv[kDim];
  for (int c = 0; c < kDim; ++c) {
    const int64_t i = (key * Hkv + g) * kHeadDim + sub * kDim + c;
    kr[c] = ldf(K, i);
    vr[c] = ldf(V, i);
    dk[c] = dv[c] = 0.f;
  }
  // query list: history entries of bin (g, b), then the block's own rows
  const int64_t e0 = b < nh ? bin_off[g * nh + b] : 0;
  const int64_t e1 = b < nh ? bin_off[g * nh + b + 1] : 0;
  const int64_t nhq = e1 - e0;
  const int64_t nown = (int64_t)qlen[b] * G;
  const int64_t total = nhq + nown;
  for (int64_t base = 0; base < total; base += kQChunk) {
    __syncthreads();  // the previous chunk is consumed
    // stage up to 32 queries: thread t loads element t of each row
    for (int qi = 0; qi < kQChunk; ++qi) {
      const int64_t idx = base + qi;
      int64_t ph = -1, pos = -1;
      if (idx < nhq) {
        ph = (int64_t)(entries[e0 + idx] / (uint32_t)KH);
      } else if (idx < total) {
        const int64_t pi = idx - nhq;
        const int64_t r = qstart[b] + pi / G;
        ph = r * Hq + g * G + (int)(pi % G);
        pos = qpos[b] + pi / G;
      }
      if (threadIdx.x < kHeadDim) {
        sq[qi][threadIdx.x] = ph >= 0 ? ldf(Q, ph * kHeadDim + threadIdx.x) : 0.f;
        sdo[qi][threadIdx.x] = ph >= 0 ? ldf(dO, ph * kHeadDim + threadIdx.x) : 0.f;
      }
      if (threadIdx.x == 0) {
        slse[qi] = ph >= 0 ? lse2[ph] : INFINITY;  // an absent query has weight 0
        sdel[qi] = ph >= 0 ? delta[ph] : 0.f;
        spos[qi] = ph >= 0 ? pos : INT64_MAX;
      }
    }
    __syncthreads();
    for (int qi = 0; qi < kQChunk; ++qi) {
      float z = 0.f, dp = 0.f;
      for (int c = 0; c < kDim; ++c) {
        z = fmaf(sq[qi][sub * kDim + c], kr[c], z);
        dp = fmaf(sdo[qi][sub * kDim + c], vr[c], dp);
      }
      z = quad_sum(z);
      dp = quad_sum(dp);
      const int64_t pos = spos[qi];
      // history queries (pos < 0) see every key; own-block rows see keys <= their position
      const bool on = kvalid && (pos < 0 || (pos != INT64_MAX && key <= pos));
      const float p = on ? __builtin_amdgcn_exp2f(fmaf(z, sl2e, -slse[qi])) : 0.f;
      const float ds = p * (dp - sdel[qi]);
      for (int c = 0; c < kDim; ++c) {
        dv[c] = fmaf(p, sdo[qi][sub * kDim + c], dv[c]);
        dk[c] = fmaf(ds, sq[qi][sub * kDim + c], dk[c]);
      }
    }
  }
  if (!kvalid) return;
  for (int c = 0; c < kDim; ++c) {
    const int64_t i = (key * Hkv + g) * kHeadDim + sub * kDim + c;
    stf(dK, i, scale * dk[c]);
    stf(dV, i, dv[c]);
  }
}

// ---------------------------------------------------------------------------
// dQ pieces. A query (4 lanes) walks one block's keys through LDS tiles of
// 32 keys and adds scale-free sum_j dZ_j k_j to dq_acc with atomics.
// ---------------------------------------------------------------------------
constexpr int kQ = 128;                 // queries per workgroup
constexpr int kThreadsQ = kQ * kSub;    // 512
constexpr int KT = 32;                  // keys per LDS tile

template <typename T>
__device__ inline void stage_kv(float* ks, float* vs, const T* __restrict__ K,
                                const T* __restrict__ V, int64_t key0, int nvalid, int Hkv,
                                int g) {
  for (int i = threadIdx.x; i < KT * kHeadDim; i += kThreadsQ) {
    const int key = i / kHeadDim, c = i % kHeadDim;
    const int64_t off = ((key0 + key) * Hkv + g) * kHeadDim + c;
    ks[i] = key < nvalid ? ldf(K, off) : 0.f;
    vs[i] = key < nvalid ? ldf(V, off) : 0.f;
  }
}

// One query's contribution from keys [key_lo, key_hi] (inclusive) of one block.
template <typename T>
__device__ inline void dq_block(float* ks, float* vs, const T* __restrict__ K,
                                const T* __restrict__ V, int64_t key_lo, int64_t key_last,
                                int64_t my_last, const float (&q)[kDim], const float (&d)[kDim],
                                float lse, float del, float sl2e, int Hkv, int g, int sub,
                                float (&acc)[kDim]) {
  for (int64_t k0 = key_lo; k0 <= key_last; k0 += KT) {
    const int64_t rem = key_last + 1 - k0;
    const int nv = rem < KT ? (int)rem : KT;
    __syncthreads();
    stage_kv(ks, vs, K, V, k0, nv, Hkv, g);
    __syncthreads();
    for (int t = 0; t < KT; ++t) {
      const float* kr = ks + t * kHeadDim + sub * kDim;
      const float* vr = vs + t * kHeadDim + sub * kDim;
      float z = 0.f, dp = 0.f;
      for (int c = 0; c < kDim; ++c) {
        z = fmaf(q[c], kr[c], z);
        dp = fmaf(d[c], vr[c], dp);
      }
      z = quad_sum(z);
      dp = quad_sum(dp);
      const bool on = t < nv && k0 + t <= my_last;
      const float p = on ? __builtin_amdgcn_exp2f(fmaf(z, sl2e, -lse)) : 0.f;
      const float ds = p * (dp - del);
      for (int c = 0; c < kDim; ++c) acc[c] = fmaf(ds, kr[c], acc[c]);
    }
  }
}

template <typename T>
__device__ inline void load_query(const T* __restrict__ Q, const T* __restrict__ dO, int64_t ph,
                                  bool valid, int sub, float (&q)[kDim], float (&d)[kDim]) {
  for (int c = 0; c < kDim; ++c) {
    q[c] = valid ? ldf(Q, ph * kHeadDim + sub * kDim + c) : 0.f;
    d[c] = valid ? ldf(dO, ph * kHeadDim + sub * kDim + c) : 0.f;
  }
}

// History pieces: one workgroup per 256 routed entries of one bin (two rounds of 128).
template <typename T>
__global__ __launch_bounds__(kThreadsQ) void bwd_dq_hist(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ bstart, const int32_t* __restrict__ tile_map,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ bin_off,
    const int32_t* __restrict__ scalars, const uint32_t* __restrict__ entries,
    float* __restrict__ dq_acc, int Hkv, int B, int KH, int64_t nh, float sl2e) {
  __shared__ float ks[KT * kHeadDim];
  __shared__ float vs[KT * kHeadDim];
  const int64_t w = blockIdx.x;
  if (w >= scalars[1]) return;
  const int bin = tile_map[w];
  const int64_t e_begin = bin_off[bin] + (w - tile_off[bin]) * (int64_t)kTileQ;
  const int64_t e_end = bin_off[bin + 1];
  const int g = (int)(bin / nh);
  const int64_t j = bin % nh;
  const int qi = threadIdx.x / kSub, sub = threadIdx.x % kSub;
  for (int64_t base = e_begin; base < e_begin + kTileQ && base < e_end; base += kQ) {
    const int64_t my_e = base + qi;
    const bool valid = my_e < e_end;
    const int64_t ph = valid ? (int64_t)(entries[my_e] / (uint32_t)KH) : 0;
    float q[kDim], d[kDim], acc[kDim];
    load_query(Q, dO, ph, valid, sub, q, d);
    for (int c = 0; c < kDim; ++c) acc[c] = 0.f;
    const float lse = valid ? lse2[ph] : INFINITY, del = valid ? delta[ph] : 0.f;
    const int64_t k0 = bstart[j];
    dq_block(ks, vs, K, V, k0, k0 + B - 1, k0 + B - 1, q, d, lse, del, sl2e, Hkv, g, sub, acc);
    if (valid)
      for (int c = 0; c < kDim; ++c) atomicAdd(&dq_acc[ph * kHeadDim + sub * kDim + c], acc[c]);
  }
}

// Own-block pieces: one workgroup per 128 (row, head) pairs of one block and KV head.
template <typename T>
__global__ __launch_bounds__(kThreadsQ) void bwd_dq_self(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ bstart, const int32_t* __restrict__ qstart,
    const int32_t* __restrict__ qlen, const int32_t* __restrict__ qpos,
    float* __restrict__ dq_acc, int Hq, int Hkv, int G, int64_t n, int tiles_per_block,
    float sl2e) {
  __shared__ float ks[KT * kHeadDim];
  __shared__ float vs[KT * kHeadDim];
  const int g = blockIdx.y;
  const int64_t c = blockIdx.x / tiles_per_block;
  const int tile = blockIdx.x % tiles_per_block;
  const int64_t npairs = (int64_t)qlen[c] * G;
  const int64_t p0 = (int64_t)tile * kQ;
  if (p0 >= npairs) return;
  const int64_t plast = (p0 + kQ - 1 < npairs) ? p0 + kQ - 1 : npairs - 1;
  const int64_t key0 = bstart[c], pos0 = qpos[c], qrow0 = qstart[c];
  const int qi = threadIdx.x / kSub, sub = threadIdx.x % kSub;
  const int64_t pi = p0 + qi;
  const bool valid = pi < npairs;
  const int64_t my_pos = valid ? pos0 + pi / G : -1;
  const int64_t ph = valid ? (qrow0 + pi / G) * Hq + g * G + (int)(pi % G) : 0;
  float q[kDim], d[kDim], acc[kDim];
  load_query(Q, dO, ph, valid, sub, q, d);
  for (int cc = 0; cc < kDim; ++cc) acc[cc] = 0.f;
  const float lse = valid ? lse2[ph] : INFINITY, del = valid ? delta[ph] : 0.f;
  dq_block(ks, vs, K, V, key0, pos0 + plast / G, my_pos, q, d, lse, del, sl2e, Hkv, g, sub, acc);
  if (valid)
    for (int cc = 0; cc < kDim; ++cc) atomicAdd(&dq_acc[ph * kHeadDim + sub * kDim + cc], acc[cc]);
}

template <typename T>
__global__ void bwd_dq_finish(const float* __restrict__ dq_acc, T* __restrict__ dQ, int64_t total,
                              float scale) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x)
    stf(dQ, i, scale * dq_acc[i]);
}

__global__ void zero_f32(float* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 8192) g = 8192;
  return (unsigned)(g > 0 ? g : 1);
}

template <typename T>
hipError_t run(const Prob& P, const Blocks& Tb, const BucketPlan& bp, const BucketBufs& bb,
               const T* q, const T* k, const T* v, const T* o, const float* lse2, const T* dout,
               T* dq, T* dk, T* dv, float* delta, float* dq_acc, hipStream_t s) {
  const int64_t nph = P.Nq * P.Hq;
  const float sl2e = P.scale * kLog2e;
  bwd_delta<T><<<(unsigned)ceil_div(nph * kSub, 256), 256, 0, s>>>(o, dout, delta, nph);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  zero_f32<<<grid_for(nph * kHeadDim), 256, 0, s>>>(dq_acc, nph * kHeadDim);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int key_tiles = (int)ceil_div(P.B, kKeysPerWG);
  bwd_dkv<T><<<dim3((unsigned)(P.n * key_tiles), (unsigned)P.Hkv), 256, 0, s>>>(
      q, k, v, dout, lse2, delta, Tb.start, Tb.len, Tb.qstart, Tb.qlen, Tb.qpos, bb.bin_off,
      bb.entries, dk, dv, P.Hq, P.Hkv, P.G, P.KH > 0 ? P.KH : 1, P.nh > 0 && P.KH > 0 ? P.nh : 0,
      key_tiles, P.scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (P.nh > 0 && P.KH > 0 && bp.max_tiles > 0) {
    bwd_dq_hist<T><<<(unsigned)bp.max_tiles, kThreadsQ, 0, s>>>(
        q, k, v, dout, lse2, delta, Tb.start, bb.tile_map, bb.tile_off, bb.bin_off, bb.scalars,
        bb.entries, dq_acc, P.Hkv, P.B, P.KH, P.nh, sl2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int tpb = (int)ceil_div((int64_t)P.B * P.G, kQ);
  bwd_dq_self<T><<<dim3((unsigned)(P.n * tpb), (unsigned)P.Hkv), kThreadsQ, 0, s>>>(
      q, k, v, dout, lse2, delta, Tb.start, Tb.qstart, Tb.qlen, Tb.qpos, dq_acc, P.Hq, P.Hkv,
      P.G, P.n, tpb, sl2e);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_dq_finish<T><<<grid_for(nph * kHeadDim), 256, 0, s>>>(dq_acc, dq, nph * kHeadDim, P.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Prob& P, const Blocks& T, const BucketPlan& bp,
                           const BucketBufs& bb, const void* q, const void* k, const void* v,
                           const void* o, const float* lse2, const void* dout, void* dq, void* dk,
                           void* dv, const BwdScratch& w, hipStream_t s) {
  if (P.dtype == MOBA_DTYPE_BF16) {
    const int64_t nph = P.Nq * P.Hq;
    bwd_delta<uint16_t><<<(unsigned)ceil_div(nph * kSub, 256), 256, 0, s>>>(
        (const uint16_t*)o, (const uint16_t*)dout, w.delta, nph);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_backward_bf16(P, T, bp, bb, q, k, v, lse2, dout, w.delta, w.kt, w.part_dq, dq,
                                dk, dv, s);
  }
  return run<float>(P, T, bp, bb, (const float*)q, (const float*)k, (const float*)v,
                    (const float*)o, lse2, (const float*)dout, (float*)dq, (float*)dk, (float*)dv,
                    w.delta, w.dq_acc, s);
}

}  // namespace moba
