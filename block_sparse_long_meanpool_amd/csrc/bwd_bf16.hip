// Backward pass of MoBA attention on the gfx950 matrix cores (bf16 inputs).
// The block selection is held fixed: the hard top-k passes no gradient to
// the ranking, so Q, K and V get gradients only through the attended
// (query, key) pairs (PaperTrace "2.1.3 MoBA", section 5.3). With
// z_j = scale q.k_j over a query's candidate keys (eq. (4)), P = softmax(z),
// o = sum_j P_j v_j and upstream gradient dO:
//   dV_j += P_j dO,  dP_j = dO.v_j,  D = dO.o,  dZ_j = P_j (dP_j - D),
//   dq = scale sum_j dZ_j k_j,  dK_j += scale dZ_j q.
// P_j = 2^(c q.k_j - lse2) with c = scale log2(e) and lse2 the forward's
// per-row log2-sum-exp, so no softmax statistics are recomputed.
//
// All products are v_mfma_f32_32x32x16_bf16 (fp32 accumulation); P and dZ
// are rounded to bf16 as matrix operands. Two kernels:
//   * dK, dV (key-stationary): a workgroup of 8 waves owns 128 keys of one
//     block and KV head, a wave 16 of them with its K and V rows held as
//     matrix operands (16x16x32 products) in registers. It streams every query that attends the
//     block (the bucketed history entries of (KV head, block), then the
//     block's own causal rows for all G query heads) through LDS in chunks of
//     64, double buffered, copied straight from global memory into a
//     row-major tile: the operand of S = Q K^T and dP = dO V^T is read from
//     it directly, the transposed operand of dK^T = Q^T dZ and dV^T = dO^T P
//     with the transpose reads of gfx950 (ds_read_b64_tr_b16). The score
//     layout puts one key per lane, so P and dZ feed the second pair of
//     products straight from the accumulators. Every key's gradients are
//     finished in one workgroup and written once.
//   * dQ (query-stationary): the tiles of the forward pass (256 routed
//     entries of one history block, or 256 own-block (row, head) pairs);
//     8 waves of 32 queries stream the block's K rows, V rows and a
//     transposed, key-permuted K copy through LDS in 64-key tiles:
//     S^T = K Q^T and dP^T = V dO^T put one query per lane, and
//     dq^T += K^T dZ^T takes dZ from the accumulators. History tiles write
//     one fp32 partial row per routed entry; the own-block kernel adds the
//     partials of each row's history slots to its own part and writes dq,
//     so no atomics are used and the result is deterministic.
#include "moba_internal.hpp"

namespace moba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kD = kHeadDim;  // 128
constexpr int kRawBufferFlags = 0x00020000;

__device__ inline bf16x8 as_b8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline void zero(f32x16& c) {
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = 0.f;
}
// Row (0..31) of accumulator element r of the 32x32 output, for lane half h.
__device__ inline int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Row-major [rows][128] bf16 tiles keep 16-byte chunk c of row r at
// c ^ (r & 15): the 16 lanes of one ds_read_b128 cycle (16 rows, one chunk)
// hit distinct bank quads. Transposed [128][64] tiles (128-byte rows, two per
// bank line) keep chunk c of row d at c ^ ((d >> 1) & 7) ^ ((d >> 4) & 7):
// 16 consecutive rows read at one chunk spread over all 16 bank quads, and
// the staging writes (rows 8 apart, 32 lanes per pass) over all 8 quads of
// their half, two lanes each.
__device__ inline int rm_swz(int r, int c) { return c ^ (r & 15); }
__device__ inline int tr_swz(int d, int c) { return c ^ ((d >> 1) & 7) ^ ((d >> 4) & 7); }
__device__ inline bf16x8 rm_read(const uint16_t* t, int r, int c) {
  return as_b8(*reinterpret_cast<const uint4*>(t + r * kD + (rm_swz(r, c) << 3)));
}
__device__ inline bf16x8 tr_read(const uint16_t* t, int d, int c) {
  return as_b8(*reinterpret_cast<const uint4*>(t + d * 64 + (tr_swz(d, c) << 3)));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16(float a, float b) {  // round to nearest even
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline bf16x8 to_b8(const float* x) {  // 8 consecutive values
  uint4 u;
  u.x = pack_bf16(x[0], x[1]);
  u.y = pack_bf16(x[2], x[3]);
  u.z = pack_bf16(x[4], x[5]);
  u.w = pack_bf16(x[6], x[7]);
  return as_b8(u);
}

// 16-byte load of element idx, or zeros when !ok. The load itself is
// unconditional (element 0 stands in), so it stays one dwordx4 access
// instead of being split and branched around.
__device__ inline uint4 ld16_or_zero(const uint16_t* __restrict__ base, int64_t idx, bool ok) {
  const uint4 u = *reinterpret_cast<const uint4*>(base + (ok ? idx : 0));
  return ok ? u : make_uint4(0, 0, 0, 0);
}

// ===========================================================================
// dK, dV
// ===========================================================================
constexpr int kKW = 8;              // waves
constexpr int kKThreads = 64 * kKW;
constexpr int kKeysWG = 16 * kKW;   // 128 keys per workgroup, 16 per wave
constexpr int kQC = 64;             // queries per staged chunk

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Source of chunk query idx, as a table word: a history entry's slot code
// (row-head * (k-1) + slot, >= 0) is stored as -2 - code, an own-block pair
// as (r << 6) | i with r its row's offset from the block's first query row
// and i < G <= 64 its head inside the KV head's group, an absent query as -1. The history codes are stored raw (the
// division by k-1 happens when the chunk is staged) so nothing in the
// compute loop waits on the entry list.
struct QSrc {
  const uint32_t* entries;
  int64_t e0;
  int nhq, own0, total;  // history entries, first own pair, all queries
  int G;
  // The entry id is loaded here; the word is formed only in `word`, after
  // the chunk's compute, so the load's latency overlaps the matrix work.
  // Branch-free (a branch here makes the compiler form the word, and wait
  // for the load, right away): the index is clamped into the list, and a
  // list-less launch passes a valid one-element stand-in.
  __device__ inline uint32_t load(int idx) const {
    const int i = idx < nhq ? idx : nhq - 1;
    return entries[e0 + (i > 0 ? i : 0)];
  }
  __device__ inline int64_t word(int idx, uint32_t raw) const {
    if (idx < nhq) return -2 - (int64_t)raw;
    if (idx < total) {
      const uint32_t pi = (uint32_t)(own0 + (idx - nhq));
      const uint32_t r = pi / (uint32_t)G;
      return ((int64_t)r << 6) | (int64_t)(pi - r * (uint32_t)G);
    }
    return -1;
  }
};

// Decode a table word: row-head index (-1 absent) and last visible key.
struct Dec {
  int KH, Hq, qrel, head0;  // head0 = first query head of the KV head's group
  int64_t qstart;
};

__device__ inline int64_t decode(int64_t w, const Dec& dc, int32_t& lim) {
  if (w <= -2) {
    lim = 0x7FFFFFFF;  // a history query sees the whole block
    return (int64_t)((uint32_t)(-2 - w) / (uint32_t)dc.KH);
  }
  if (w < 0) {
    lim = -1;
    return -1;
  }
  const int r = (int)(w >> 6);  // own row: offset r, head head0 + (w & 63)
  lim = dc.qrel + r;
  return (dc.qstart + r) * dc.Hq + dc.head0 + (int)(w & 63);
}

// Chunk query table [64] of words, filled two chunks ahead by the first 64
// threads: the entry id is loaded before a chunk's compute, the word formed
// and stored after it.
struct TabFill {
  int idx;
  uint32_t raw;
};
__device__ inline void fill_load(TabFill& f, const QSrc& src, int base) {
  f.idx = base + (int)threadIdx.x;  // every thread loads (clamped), the first 64 store
  f.raw = src.load(f.idx);
}
__device__ inline void fill_store(const TabFill& f, const QSrc& src, int64_t* tab) {
  if (threadIdx.x < kQC) tab[threadIdx.x] = src.word(f.idx, f.raw);
}

// One staged chunk of 64 queries in LDS.
struct QBuf {
  uint16_t* q;   // [64][128] Q rows, 16-byte chunk c of row r at c ^ (r & 15)
  uint16_t* o;   // [64][128] dO rows, same layout
  float* lse;    // [64] log2-sum-exp
  float* dd;     // [64] D = dO.o
  int32_t* lim;  // [64] last visible key (relative to the block start), -1 none
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Stage a chunk with direct global -> LDS copies (no registers in between):
// each of the 8 waves copies 2 x 1 KB of Q rows and of dO rows (4 rows of 16
// chunks per copy, the source chunk chosen so that the LDS position is
// swizzled), wave 0 the 64 lse values, wave 1 the 64 D values; wave 2 writes
// the key limits. An absent query reads row 0 (finite values; its limit -1
// masks it).
__device__ inline void stage(QBuf B, const int64_t* tab, const Dec& dc,
                             const uint16_t* __restrict__ Q, const uint16_t* __restrict__ dO,
                             const float* __restrict__ lse2, const float* __restrict__ delta) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ii = 2 * wave + i;
    const int r = 4 * ii + (lane >> 4);
    int32_t lim;
    int64_t ph = decode(tab[r], dc, lim);
    ph = ph >= 0 ? ph : 0;
    const int64_t off = ph * kD + 8 * rm_swz(r, lane & 15);  // the swizzle is an involution
    __builtin_amdgcn_global_load_lds(Q + off, (__attribute__((address_space(3))) void*)(B.q + 4 * ii * kD), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(dO + off, (__attribute__((address_space(3))) void*)(B.o + 4 * ii * kD), 16, 0, 0);
  }
  if (wave < 3) {
    int32_t lim;
    int64_t ph = decode(tab[lane], dc, lim);
    ph = ph >= 0 ? ph : 0;
    if (wave == 0)
      __builtin_amdgcn_global_load_lds(lse2 + ph, (__attribute__((address_space(3))) void*)B.lse, 4, 0, 0);
    else if (wave == 1)
      __builtin_amdgcn_global_load_lds(delta + ph, (__attribute__((address_space(3))) void*)B.dd, 4, 0, 0);
    else
      B.lim[lane] = lim;
  }
}

// A operand [16 dims][32 queries] of dK^T = Q^T dZ or dV^T = dO^T P from the
// row-major tile by two transpose reads (ds_read_b64_tr_b16: in each group
// of 16 lanes, lane j receives element j % 4 of the 8-byte reads of lanes
// 4e + j / 4, e = 0..3). Group a = l / 16, lane 4e + b of it reads dims
// 16 mb + 4b .. +3 of query row 4a + e (first read) and 16 + 4a + e
// (second) of the 32-query step, so lane l receives dim 16 mb + l % 16 of
// queries 4a + 0..3 and 16 + 4a + 0..3: the order in which the score
// accumulators of two 16-query blocks hold them.
__device__ inline bf16x8 tr_pair(const uint16_t* p0, const uint16_t* p1) {
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B operand from two 16-query blocks of accumulators: queries 4a + 0..3 of
// the first and of the second block.
__device__ inline bf16x8 pack_pair(const f32x4& x, const f32x4& y) {
  const float v[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return to_b8(v);
}

// grid: 1D, a multiple of 8 covering Hkv * n * ceil(B / 128) items; 512 threads.
// Products are v_mfma_f32_16x16x32_bf16 (lane l: A[l % 16][8 (l / 16) + 0..7],
// B[8 (l / 16) + 0..7][l % 16], C[4 (l / 16) + i][l % 16]).
__global__ __launch_bounds__(kKThreads) void bwd_dkv_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ bstart, const int32_t* __restrict__ blen,
    const int32_t* __restrict__ qstart, const int32_t* __restrict__ qlen,
    const int32_t* __restrict__ qpos, const int32_t* __restrict__ bin_off,
    const uint32_t* __restrict__ entries, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int Hq, int Hkv, int G, int KH, int64_t n, int64_t nh, int tiles_per_block, float scale) {
  // two chunk buffers, each part its own array: the copies into one buffer
  // visibly never alias the reads from the other
  __shared__ __align__(16) uint16_t s_q0[kQC * kD], s_q1[kQC * kD];
  __shared__ __align__(16) uint16_t s_o0[kQC * kD], s_o1[kQC * kD];
  __shared__ __align__(16) float s_l0[kQC], s_l1[kQC], s_d0[kQC], s_d1[kQC];
  __shared__ __align__(16) int32_t s_m0[kQC], s_m1[kQC];
  __shared__ int64_t s_t0[kQC], s_t1[kQC];
  // Items w = (g * n + b) * tiles_per_block + kt. Workgroup i runs on XCD
  // i % 8 and each XCD takes a contiguous range of items, so the key tiles
  // of one (KV head, block), which stage the same query rows, share an L2.
  const int64_t per = gridDim.x / 8;
  const int64_t w = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= (int64_t)Hkv * n * tiles_per_block) return;
  const int kt = (int)(w % tiles_per_block);
  const int64_t b = (w / tiles_per_block) % n;
  const int g = (int)(w / ((int64_t)tiles_per_block * n));
  const int nk = blen[b];
  if (kt * kKeysWG >= nk) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ln16 = lane & 15, a4 = lane >> 4;
  const int64_t key_first = bstart[b];
  const int key_rel = kt * kKeysWG + 16 * wave + ln16;  // this lane's key in the block
  const bool kvalid = key_rel < nk;
  const float sl2e = scale * kLog2e;

  // this lane's key as the B operand: dims 32 kk + 8 a4 .. +7
  bf16x8 kb[4], vb[4];
  {
    const int64_t off = ((key_first + (kvalid ? key_rel : 0)) * Hkv + g) * kD + 8 * a4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      kb[kk] = as_b8(ld16_or_zero(K, off + 32 * kk, kvalid));
      vb[kk] = as_b8(ld16_or_zero(V, off + 32 * kk, kvalid));
    }
    // complete before the chunk loop, whose counter waits then only cover
    // the staging copies
    __builtin_amdgcn_s_waitcnt(0);
  }

  QSrc src;
  src.entries = entries;
  src.e0 = b < nh ? bin_off[g * nh + b] : 0;
  src.nhq = b < nh ? (int)(bin_off[g * nh + b + 1] - src.e0) : 0;
  const int qrel = qpos[b] - bstart[b];  // first query row's position in the block
  // own rows before this key tile see none of its keys
  const int own_all = qlen[b] * G;
  const int first_row = kt * kKeysWG - qrel;  // own row holding key kt * 128
  src.own0 = first_row > 0 ? first_row * G : 0;
  if (src.own0 > own_all) src.own0 = own_all;
  src.total = src.nhq + (own_all - src.own0);
  src.G = G;
  const Dec dc{KH, Hq, qrel, g * G, (int64_t)qstart[b]};

  f32x4 dk[8], dv[8];  // dims 16 mb + 4 a4 + i of this lane's key
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dk[mb][i] = dv[mb][i] = 0.f;

  auto compute = [&](QBuf cur) {
    // Per-lane element offsets inside a tile; query blocks, 32-query steps
    // and the Q / dO tiles differ by constants (the reads' immediate
    // offsets). The lane id goes through an empty asm statement so the
    // offsets are rebuilt per chunk rather than hoisted out of the loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int l16 = ln & 15, la = ln >> 4;
    int rmo[4];  // row l16 (of a 16-query block), dims 32 kk + 8 la
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) rmo[kk] = l16 * kD + (rm_swz(l16, 4 * kk + la) << 3);
    int tro[8];  // row 4 la + e, dims 16 mb + 4 bb of a 32-query step
    {
      const int e = l16 >> 2, bb = l16 & 3, row = 4 * la + e;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
        tro[mb] = row * kD + (rm_swz(row, 2 * mb + (bb >> 1)) << 3) + (bb & 1) * 4;
    }
    // scores and dP of the chunk's 4 query blocks (lane: key; register i:
    // query 16 qb + 4 la + i)
    f32x4 sc[4], dp[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[qb][i] = dp[qb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int o = qb * 16 * kD + rmo[kk];
        sc[qb] = mfma16(as_b8(*reinterpret_cast<const uint4*>(cur.q + o)), kb[kk], sc[qb]);
        dp[qb] = mfma16(as_b8(*reinterpret_cast<const uint4*>(cur.o + o)), vb[kk], dp[qb]);
      }
    }
    // P = 2^(c s - lse) (masked), dZ = P (dP - D)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int q = 16 * qb + 4 * la;
      const float4 l4 = *reinterpret_cast<const float4*>(cur.lse + q);
      const float4 d4 = *reinterpret_cast<const float4*>(cur.dd + q);
      const int4 m4 = *reinterpret_cast<const int4*>(cur.lim + q);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
      const int mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = fmaf(sc[qb][i], sl2e, -lv[i]);
        const float pr = __builtin_amdgcn_exp2f(key_rel <= mv[i] ? x : -INFINITY);
        sc[qb][i] = pr;
        dp[qb][i] = pr * (dp[qb][i] - dv4[i]);
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dZ over two 32-query steps
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x8 pb = pack_pair(sc[2 * j], sc[2 * j + 1]);
      const bf16x8 zb = pack_pair(dp[2 * j], dp[2 * j + 1]);
      const int rows = 32 * j * kD;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const int o = rows + tro[mb];
        dv[mb] = mfma16(tr_pair(cur.o + o, cur.o + o + 16 * kD), pb, dv[mb]);
        dk[mb] = mfma16(tr_pair(cur.q + o, cur.q + o + 16 * kD), zb, dk[mb]);
      }
    }
  };

  const QBuf buf0{s_q0, s_o0, s_l0, s_d0, s_m0}, buf1{s_q1, s_o1, s_l1, s_d1, s_m1};
  const int nchunks = (src.total + kQC - 1) / kQC;
  TabFill tf{0, 0u};
  // Prologue: tables of chunks 0 and 1; chunk 0 staged into buffer 0.
  if (nchunks > 0) {
    fill_load(tf, src, 0);
    fill_store(tf, src, s_t0);
    fill_load(tf, src, kQC);
    fill_store(tf, src, s_t1);
    __syncthreads();
    stage(buf0, s_t0, dc, Q, dO, lse2, delta);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // Iteration t: stage chunk t + 1 (table slot (t + 1) & 1) into the other
  // buffer, load the entry ids of chunk t + 2, compute chunk t, store chunk
  // t + 2's table into slot t & 1, wait for this wave's copies, barrier.
  auto iter = [&](int t, QBuf cur, QBuf nxt, int64_t* tab_cur, int64_t* tab_nxt) {
    if (t + 1 < nchunks) stage(nxt, tab_nxt, dc, Q, dO, lse2, delta);
    fill_load(tf, src, (t + 2) * kQC);  // words past the last query are -1
    compute(cur);
    fill_store(tf, src, tab_cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int t = 0; t < nchunks; t += 2) {
    iter(t, buf0, buf1, s_t0, s_t1);
    if (t + 1 < nchunks) iter(t + 1, buf1, buf0, s_t1, s_t0);
  }
  if (!kvalid) return;
  // lane: key key_rel; register i of block mb: dim 16 mb + 4 a4 + i
  const int64_t off = ((key_first + key_rel) * Hkv + g) * kD + 4 * a4;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    *reinterpret_cast<uint2*>(dK + off + 16 * mb) =
        make_uint2(pack_bf16(scale * dk[mb][0], scale * dk[mb][1]),
                   pack_bf16(scale * dk[mb][2], scale * dk[mb][3]));
    *reinterpret_cast<uint2*>(dV + off + 16 * mb) =
        make_uint2(pack_bf16(dv[mb][0], dv[mb][1]), pack_bf16(dv[mb][2], dv[mb][3]));
  }
}

// ===========================================================================
// dQ
// ===========================================================================
constexpr int kQW = 8;              // waves
constexpr int kQThreads = 64 * kQW;
constexpr int KT = 64;              // keys per LDS tile
static_assert(kQW * 32 == kTileQ, "a history tile is one workgroup");

struct KTile {
  uint16_t* k;   // [64][128] K rows
  uint16_t* v;   // [64][128] V rows
  uint16_t* t;   // [128][64] K^T, keys permuted per 32-group
};

// global -> LDS copies of keys [key0, key0 + 64) (rows past nvalid read as
// zero); each of the 8 waves copies 2 KB of K, of V and of K^T.
__device__ inline void load_ktile(KTile dst, const uint16_t* __restrict__ K,
                                  const uint16_t* __restrict__ V, int64_t key0, int nvalid,
                                  int Hkv, int g, const uint16_t* __restrict__ kt_col, int64_t ldk,
                                  int wave, int lane) {
  const int64_t krow = (int64_t)Hkv * kD;
  const int range = (int)(((int64_t)(nvalid - 1) * krow + kD) * 2);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(K + (key0 * Hkv + g) * kD), 0, range, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(V + (key0 * Hkv + g) * kD), 0, range, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)kt_col, 0, (int)(((int64_t)(kD - 1) * ldk + KT) * 2), kRawBufferFlags);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ii = 2 * wave + i;  // 4 rows per copy
    const int r = 4 * ii + (lane >> 4);
    const int c = rm_swz(r, lane & 15);  // the swizzle is an involution in c
    const unsigned vo = (unsigned)((r * krow + 8 * c) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, dst.k + 4 * ii * kD, 16, vo, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, dst.v + 4 * ii * kD, 16, vo, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ii = 2 * wave + i;  // 8 K^T rows per copy
    const int d = 8 * ii + (lane >> 3);
    const int c = tr_swz(d, lane & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tr, dst.t + 8 * ii * KT, 16,
                                             (unsigned)((d * ldk + 8 * c) * 2), 0, 0, 0);
  }
}

__device__ inline void wait_tile() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// One wave's 32 queries (lane: query lr) over keys [key0, key0 + nkeys) of one
// block, accumulating dq^T (unscaled) in acc. CAUSAL: key <= the query's
// position. Positions are relative to key0 (32-bit): qrel is the lane's
// query, wmin / wmax the wave's first and last query.
template <bool CAUSAL>
__device__ inline void dq_block(KTile b0, KTile b1, const uint16_t* __restrict__ K,
                                const uint16_t* __restrict__ V, int64_t key0, int nkeys,
                                int Hkv, int g, const uint16_t* __restrict__ kt_col, int64_t ldk,
                                const bf16x8 (&qb)[8], const bf16x8 (&ob)[8], float lse, float dd,
                                int qrel, int wmin, int wmax, bool live, float sl2e,
                                f32x16 (&acc)[4]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 31, h = lane >> 5;
  const int nt = (nkeys + KT - 1) / KT;
  auto issue = [&](int t, KTile dst) {
    const int rem = nkeys - t * KT;
    load_ktile(dst, K, V, key0 + (int64_t)t * KT, rem < KT ? rem : KT, Hkv, g, kt_col + t * KT,
               ldk, wave, lane);
  };
  issue(0, b0);
  wait_tile();
  for (int t = 0; t < nt; ++t) {
    const KTile cur = (t & 1) ? b1 : b0;
    if (t + 1 < nt) issue(t + 1, (t & 1) ? b0 : b1);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int k0 = t * KT + 32 * sub;  // relative to key0
      const int rem = nkeys - k0;
      const int nv = rem <= 0 ? 0 : (rem < 32 ? rem : 32);
      if (!live || nv == 0 || (CAUSAL && k0 > wmax)) continue;
      f32x16 s, dp;
      zero(s);
      zero(dp);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        s = mfma(rm_read(cur.k, 32 * sub + lr, 2 * kk + h), qb[kk], s);
        dp = mfma(rm_read(cur.v, 32 * sub + lr, 2 * kk + h), ob[kk], dp);
      }
      // lane: query; element r: key k0 + acc_row(r, h)
      const bool need_mask = nv < 32 || (CAUSAL && k0 + 31 > wmin);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = acc_row(r, h);
        float x = fmaf(s[r], sl2e, -lse);
        if (need_mask) x = (key < nv && (!CAUSAL || k0 + key <= qrel)) ? x : -INFINITY;
        const float p = __builtin_amdgcn_exp2f(x);
        ds[r] = p * (dp[r] - dd);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 b = to_b8(ds + 8 * u);
        const int c = 4 * sub + 2 * u + h;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = mfma(tr_read(cur.t, 32 * db + lr, c), b, acc[db]);
      }
    }
    wait_tile();
  }
}

__device__ inline void load_query(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ dO,
                                  int64_t ph, bool valid, int h, bf16x8 (&qb)[8],
                                  bf16x8 (&ob)[8]) {
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int64_t i = ph * kD + 16 * kk + 8 * h;
    qb[kk] = as_b8(ld16_or_zero(Q, i, valid));
    ob[kk] = as_b8(ld16_or_zero(dO, i, valid));
  }
}

#define MOBA_DQ_TILES                                                            \
  __shared__ __align__(16) uint16_t s_k0[KT * kD], s_k1[KT * kD];               \
  __shared__ __align__(16) uint16_t s_v0[KT * kD], s_v1[KT * kD];               \
  __shared__ __align__(16) uint16_t s_t0[kD * KT], s_t1[kD * KT];               \
  KTile b0{s_k0, s_v0, s_t0}, b1{s_k1, s_v1, s_t1};

// History pieces: one workgroup per 256 routed entries of one (KV head,
// block) list; writes scale * sum_j dZ_j k_j per entry into part_dq [code][d].
__global__ __launch_bounds__(kQThreads) void bwd_dq_hist_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const uint16_t* __restrict__ Kt, const int32_t* __restrict__ bstart,
    const int32_t* __restrict__ tile_map, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ bin_off, const int32_t* __restrict__ scalars,
    const uint32_t* __restrict__ entries, float* __restrict__ part_dq, int Hkv, int B, int KH,
    int64_t nh, int64_t Bpad, int64_t ldk, float scale) {
  MOBA_DQ_TILES
  // XCD-aware order (as in the forward): each XCD takes a contiguous range
  // of tiles, so the tiles of one K/V block share its L2. The grid is a
  // multiple of 8.
  const int64_t per = gridDim.x / 8;
  const int64_t w = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= scalars[1]) return;
  const int bin = tile_map[w];
  const int64_t e_begin = bin_off[bin] + (w - tile_off[bin]) * (int64_t)kTileQ;
  const int64_t e_end = bin_off[bin + 1];
  const int g = (int)(bin / nh);
  const int64_t j = bin % nh;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 31, h = lane >> 5;
  const int64_t my_e = e_begin + 32 * wave + lr;
  const bool valid = my_e < e_end;
  const uint32_t code = valid ? entries[my_e] : 0u;
  const int64_t ph = (int64_t)(code / (uint32_t)KH);
  bf16x8 qb[8], ob[8];
  load_query(Q, dO, ph, valid, h, qb, ob);
  const float lse = valid ? lse2[ph] : INFINITY, dd = valid ? delta[ph] : 0.f;
  const bool live = e_begin + 32 * wave < e_end;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) zero(acc[db]);
  dq_block<false>(b0, b1, K, V, bstart[j], B, Hkv, g, Kt + (int64_t)g * kD * ldk + j * Bpad, ldk,
                  qb, ob, lse, dd, 0, 0, 0, live, scale * kLog2e, acc);
  if (!valid) return;
  float* dst = part_dq + (int64_t)code * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = 32 * db + 8 * jj + 4 * h;
      *reinterpret_cast<float4*>(dst + d) =
          make_float4(scale * acc[db][4 * jj], scale * acc[db][4 * jj + 1],
                      scale * acc[db][4 * jj + 2], scale * acc[db][4 * jj + 3]);
    }
}

// Own-block pieces plus the history partials: one workgroup per 256 (row,
// head) pairs of one block and KV head; writes dq.
__global__ __launch_bounds__(kQThreads) void bwd_dq_self_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const uint16_t* __restrict__ Kt, const int32_t* __restrict__ bstart,
    const int32_t* __restrict__ qstart, const int32_t* __restrict__ qlen,
    const int32_t* __restrict__ qpos, const int32_t* __restrict__ blo,
    const float* __restrict__ part_dq, uint16_t* __restrict__ dQ, int Hq, int Hkv, int G, int KH,
    int64_t n, int tiles_per_block, int64_t Bpad, int64_t ldk, float scale) {
  MOBA_DQ_TILES
  // Items w = (g * n + c) * tiles_per_block + tile, a contiguous range per
  // XCD (the grid is a multiple of 8), so the row tiles of one (KV head,
  // block) share its L2 copy of K/V.
  const int64_t per = gridDim.x / 8;
  const int64_t w = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= (int64_t)Hkv * n * tiles_per_block) return;
  const int tile = (int)(w % tiles_per_block);
  const int64_t c = (w / tiles_per_block) % n;
  const int g = (int)(w / ((int64_t)tiles_per_block * n));
  const int64_t npairs = (int64_t)qlen[c] * G;
  const int64_t p0 = (int64_t)tile * kTileQ;
  if (p0 >= npairs) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 31, h = lane >> 5;
  const int64_t key0 = bstart[c], pos0 = qpos[c], qrow0 = qstart[c];
  const int64_t plast = (p0 + kTileQ - 1 < npairs) ? p0 + kTileQ - 1 : npairs - 1;
  const int64_t pi = p0 + 32 * wave + lr;
  const bool valid = pi <= plast;
  const int64_t qpos_me = pos0 + (valid ? pi : plast) / G;
  const int64_t ph = (qrow0 + (valid ? pi : plast) / G) * Hq + (int64_t)g * G +
                     (int)((valid ? pi : plast) % G);
  // the wave's row range (for skipping and masking subtiles)
  const int64_t wp0 = p0 + 32 * wave;
  const bool live = wp0 <= plast;
  const int64_t wp1 = (wp0 + 31 < plast) ? wp0 + 31 : plast;
  const int64_t wrow_min = pos0 + (live ? wp0 : plast) / G, wrow_max = pos0 + wp1 / G;
  bf16x8 qb[8], ob[8];
  load_query(Q, dO, ph, valid, h, qb, ob);
  const float lse = valid ? lse2[ph] : INFINITY, dd = valid ? delta[ph] : 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) zero(acc[db]);
  const int nkeys = (int)(pos0 + plast / G - key0 + 1);
  dq_block<true>(b0, b1, K, V, key0, nkeys, Hkv, g, Kt + (int64_t)g * kD * ldk + c * Bpad, ldk,
                 qb, ob, lse, dd, (int)(qpos_me - key0), (int)(wrow_min - key0),
                 (int)(wrow_max - key0), live, scale * kLog2e, acc);
  if (!valid) return;
  // the row's history slots: min(k - 1, earlier blocks of its sequence)
  const int64_t avail = c - blo[c];
  const int nhist = (int)(avail < KH ? avail : KH);
  uint16_t* dst = dQ + ph * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = 32 * db + 8 * jj + 4 * h;
      float x0 = scale * acc[db][4 * jj], x1 = scale * acc[db][4 * jj + 1];
      float x2 = scale * acc[db][4 * jj + 2], x3 = scale * acc[db][4 * jj + 3];
      for (int sl = 0; sl < nhist; ++sl) {
        const float4 pp = *reinterpret_cast<const float4*>(part_dq + (ph * KH + sl) * kD + d);
        x0 += pp.x;
        x1 += pp.y;
        x2 += pp.z;
        x3 += pp.w;
      }
      *reinterpret_cast<uint2*>(dst + d) = make_uint2(pack_bf16(x0, x1), pack_bf16(x2, x3));
    }
}

}  // namespace

hipError_t launch_backward_bf16(const Prob& P, const Blocks& T, const BucketPlan& bp,
                                const BucketBufs& bb, const void* q, const void* k, const void* v,
                                const float* lse2, const void* dout, const float* delta,
                                void* kt, float* part_dq, void* dq, void* dk, void* dv,
                                hipStream_t s) {
  const uint16_t* Q = (const uint16_t*)q;
  const uint16_t* K = (const uint16_t*)k;
  const uint16_t* V = (const uint16_t*)v;
  const uint16_t* dO = (const uint16_t*)dout;
  hipError_t e = launch_vt_pack(P, T, k, kt, s);  // K^T in the V^T layout
  if (e != hipSuccess) return e;
  const int64_t Bpad = vt_padded_block(P.B), ldk = P.n * Bpad;
  const bool hist = P.nh > 0 && P.KH > 0;
  auto grid8 = [](int64_t items) { return (unsigned)(ceil_div(items, 8) * 8); };
  if (hist && bp.max_tiles > 0) {
    bwd_dq_hist_bf16<<<grid8(bp.max_tiles), kQThreads, 0, s>>>(
        Q, K, V, dO, lse2, delta, (const uint16_t*)kt, T.start, bb.tile_map, bb.tile_off,
        bb.bin_off, bb.scalars, bb.entries, part_dq, P.Hkv, P.B, P.KH, P.nh, Bpad, ldk, P.scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int key_tiles = (int)ceil_div(P.B, kKeysWG);
  bwd_dkv_bf16<<<grid8(P.n * key_tiles * P.Hkv), kKThreads, 0, s>>>(
      Q, K, V, dO, lse2, delta, T.start, T.len, T.qstart, T.qlen, T.qpos, bb.bin_off,
      hist ? bb.entries : (const uint32_t*)T.start, (uint16_t*)dk, (uint16_t*)dv, P.Hq, P.Hkv,
      P.G, P.KH > 0 ? P.KH : 1, P.n, hist ? P.nh : 0, key_tiles, P.scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int tpb = (int)ceil_div((int64_t)P.B * P.G, kTileQ);
  bwd_dq_self_bf16<<<grid8(P.n * tpb * P.Hkv), kQThreads, 0, s>>>(
      Q, K, V, dO, lse2, delta, (const uint16_t*)kt, T.start, T.qstart, T.qlen, T.qpos, T.lo,
      part_dq, (uint16_t*)dq, P.Hq, P.Hkv, P.G, P.KH, P.n, tpb, Bpad, ldk, P.scale);
  return hipGetLastError();
}

}  // namespace moba
