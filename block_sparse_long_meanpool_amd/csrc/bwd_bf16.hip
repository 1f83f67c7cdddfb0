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
//   * dK, dV (key-stationary): a workgroup of 4 waves owns 128 keys of one
//     block and KV head, a wave 32 of them with its K and V rows held as
//     matrix operands in registers. It streams every query that attends the
//     block (the bucketed history entries of (KV head, block), then the
//     block's own causal rows for all G query heads) through LDS in chunks of
//     64, double buffered, each chunk staged both row-major (operand of
//     S = Q K^T and dP = dO V^T) and transposed (operand of dK^T = Q^T dZ and
//     dV^T = dO^T P). The score layout puts one key per lane, so P and dZ
//     feed the second pair of products straight from the accumulators.
//     Every key's gradients are finished in one workgroup and written once.
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
// Position of row q inside its 32-group in a transposed operand: swapping
// bits 2 and 3 puts the 8 rows a lane contracts over into one 16-byte run.
__device__ inline int perm32(int q) { return (q & ~12) | ((q & 4) << 1) | ((q & 8) >> 1); }

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
constexpr int kKW = 4;              // waves
constexpr int kKThreads = 64 * kKW;
constexpr int kKeysWG = 32 * kKW;   // 128 keys per workgroup
constexpr int kQC = 64;             // queries per staged chunk

struct QChunk {
  uint16_t* qr;   // [64][128] Q rows
  uint16_t* dr;   // [64][128] dO rows
  uint16_t* qt;   // [128][64] Q^T, rows permuted per 32-group
  uint16_t* dt;   // [128][64] dO^T
  float* lse;     // [64] log2-sum-exp
  float* dd;      // [64] D = dO.o
  int32_t* lim;   // [64] last visible key (relative to the block start), -1 none
};

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

// Per thread: 2 staging tasks of (tensor, 4 consecutive queries, 8 dims);
// threads < 64 also carry one query's lse, D and key limit.
struct Stage {
  uint4 v[2][4];
  float lse, dd;
  int32_t lim;
};

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

__device__ inline void stage_load(Stage& st, const int64_t* tab, const Dec& dc,
                                  const uint16_t* __restrict__ Q, const uint16_t* __restrict__ dO,
                                  const float* __restrict__ lse2, const float* __restrict__ delta) {
  const int tid = threadIdx.x;
  if (tid < kQC) {
    // an absent query has lim = -1, which masks all its weights, so its lse
    // and D may be any finite values: row 0's stand in (no select on them)
    const int64_t ph = decode(tab[tid], dc, st.lim);
    const int64_t pc = ph >= 0 ? ph : 0;
    st.lse = lse2[pc];
    st.dd = delta[pc];
  }
  const int q4 = (tid >> 4) & 15, c = tid & 15;  // both tasks: same queries, Q then dO
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int32_t lim;
    const int64_t ph = decode(tab[4 * q4 + i], dc, lim);
    st.v[0][i] = ld16_or_zero(Q, ph * kD + 8 * c, ph >= 0);
    st.v[1][i] = ld16_or_zero(dO, ph * kD + 8 * c, ph >= 0);
  }
}

__device__ inline void stage_store(const Stage& st, QChunk b) {
  const int tid = threadIdx.x;
  const int q4 = (tid >> 4) & 15, c = tid & 15;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint16_t* rm = k ? b.dr : b.qr;
    uint16_t* tr = k ? b.dt : b.qt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 4 * q4 + i;
      *reinterpret_cast<uint4*>(rm + q * kD + (rm_swz(q, c) << 3)) = st.v[k][i];
    }
    // transposed: 8 dims x 4 consecutive (permuted) positions, 8 bytes each
    const int q0 = 4 * q4;
    const int pos = 32 * (q0 >> 5) + perm32(q0 & 31);  // positions pos..pos+3
    const uint32_t w0[4] = {st.v[k][0].x, st.v[k][0].y, st.v[k][0].z, st.v[k][0].w};
    const uint32_t w1[4] = {st.v[k][1].x, st.v[k][1].y, st.v[k][1].z, st.v[k][1].w};
    const uint32_t w2[4] = {st.v[k][2].x, st.v[k][2].y, st.v[k][2].z, st.v[k][2].w};
    const uint32_t w3[4] = {st.v[k][3].x, st.v[k][3].y, st.v[k][3].z, st.v[k][3].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * c + e;
      // byte selectors: low halves (e even) or high halves (e odd) of two words
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint2 out = make_uint2(__builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel),
                                   __builtin_amdgcn_perm(w3[e >> 1], w2[e >> 1], sel));
      *reinterpret_cast<uint2*>(tr + d * 64 + (tr_swz(d, pos >> 3) << 3) + (pos & 7)) = out;
    }
  }
  if (tid < kQC) {
    b.lse[tid] = st.lse;
    b.dd[tid] = st.dd;
    b.lim[tid] = st.lim;
  }
}

// grid: 1D, a multiple of 8 covering Hkv * n * ceil(B / 128) items; 256 threads.
__global__ __launch_bounds__(kKThreads, 1) void bwd_dkv_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ bstart, const int32_t* __restrict__ blen,
    const int32_t* __restrict__ qstart, const int32_t* __restrict__ qlen,
    const int32_t* __restrict__ qpos, const int32_t* __restrict__ bin_off,
    const uint32_t* __restrict__ entries, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int Hq, int Hkv, int G, int KH, int64_t n, int64_t nh, int tiles_per_block, float scale) {
  __shared__ __align__(16) uint16_t s_qr[2][kQC * kD], s_dr[2][kQC * kD];
  __shared__ __align__(16) uint16_t s_qt[2][kD * kQC], s_dt[2][kD * kQC];
  __shared__ __align__(16) float s_lse[2][kQC], s_dd[2][kQC];
  __shared__ __align__(16) int32_t s_lim[2][kQC];
  __shared__ int64_t s_tab[2][kQC];
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
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 31, h = lane >> 5;
  const int64_t key_first = bstart[b];
  const int key_rel = kt * kKeysWG + 32 * wave + lr;  // this lane's key in the block
  const bool kvalid = key_rel < nk;
  const float sl2e = scale * kLog2e;

  // this lane's key as the B operand: dims 16kk + 8h .. +7
  bf16x8 kb[8], vb[8];
  {
    const int64_t off = ((key_first + (kvalid ? key_rel : 0)) * Hkv + g) * kD + 8 * h;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 zk = ld16_or_zero(K, off + 16 * kk, kvalid);
      const uint4 zv = ld16_or_zero(V, off + 16 * kk, kvalid);
      kb[kk] = as_b8(zk);
      vb[kk] = as_b8(zv);
    }
    // complete before the chunk loop, whose counter waits then only cover
    // the staging loads
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

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    zero(dk[db]);
    zero(dv[db]);
  }

  const int nchunks = (src.total + kQC - 1) / kQC;
  Stage st;
  TabFill tf{0, 0u};
  auto buf = [&](int i) {
    return QChunk{s_qr[i], s_dr[i], s_qt[i], s_dt[i], s_lse[i], s_dd[i], s_lim[i]};
  };
  // Prologue: tables of chunks 0 and 1, chunk 0 staged in LDS buffer 0, chunk
  // 1 in flight to the registers, table of chunk 2 in slot 0.
  if (nchunks > 0) {
    fill_load(tf, src, 0);
    fill_store(tf, src, s_tab[0]);
    fill_load(tf, src, kQC);
    fill_store(tf, src, s_tab[1]);
    __syncthreads();
    stage_load(st, s_tab[0], dc, Q, dO, lse2, delta);
    stage_store(st, buf(0));
    if (nchunks > 1) stage_load(st, s_tab[1], dc, Q, dO, lse2, delta);
    fill_load(tf, src, 2 * kQC);
    __syncthreads();  // slot 0 is read by everyone; buffer 0 is complete
    fill_store(tf, src, s_tab[0]);
    __syncthreads();
  }
  // Iteration t computes chunk t from LDS buffer t & 1; then stores chunk
  // t + 1 (loaded into registers during iteration t - 1) into buffer
  // (t + 1) & 1, issues the loads of chunk t + 2 (table slot t & 1) and
  // stores the table of chunk t + 3 (entry ids loaded at the start) into slot
  // (t + 1) & 1. The staging loads thus have a whole iteration of matrix work
  // to land in; one barrier per chunk.
  for (int t = 0; t < nchunks; ++t) {
    const int cb = t & 1;
    fill_load(tf, src, (t + 3) * kQC);  // words past the last query are -1
    const uint16_t* qr = s_qr[cb];
    const uint16_t* dr = s_dr[cb];
    const uint16_t* qt = s_qt[cb];
    const uint16_t* dt = s_dt[cb];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 s, dp;
      zero(s);
      zero(dp);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        s = mfma(rm_read(qr, 32 * sub + lr, 2 * kk + h), kb[kk], s);
        dp = mfma(rm_read(dr, 32 * sub + lr, 2 * kk + h), vb[kk], dp);
      }
      // lane: key key_rel; element r: query 32 sub + acc_row(r, h)
      float p[16], ds[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q = 32 * sub + 8 * j + 4 * h;
        const float4 l4 = *reinterpret_cast<const float4*>(&s_lse[cb][q]);
        const float4 d4 = *reinterpret_cast<const float4*>(&s_dd[cb][q]);
        const int4 m4 = *reinterpret_cast<const int4*>(&s_lim[cb][q]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
        const int mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * j + i;
          const float x = fmaf(s[r], sl2e, -lv[i]);
          const float pr = __builtin_amdgcn_exp2f(key_rel <= mv[i] ? x : -INFINITY);
          p[r] = pr;
          ds[r] = pr * (dp[r] - dv4[i]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pb = to_b8(p + 8 * u), db8 = to_b8(ds + 8 * u);
        const int c = 4 * sub + 2 * u + h;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          dv[db] = mfma(tr_read(dt, 32 * db + lr, c), pb, dv[db]);
          dk[db] = mfma(tr_read(qt, 32 * db + lr, c), db8, dk[db]);
        }
      }
    }
    if (t + 1 < nchunks) stage_store(st, buf(cb ^ 1));
    if (t + 2 < nchunks) stage_load(st, s_tab[cb], dc, Q, dO, lse2, delta);
    fill_store(tf, src, s_tab[cb ^ 1]);
    __syncthreads();
  }
  if (!kvalid) return;
  // lane: key key_rel; element r of block db: dim 32 db + acc_row(r, h)
  const int64_t off = ((key_first + key_rel) * Hkv + g) * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * db + 8 * j + 4 * h;
      const int r = 4 * j;
      *reinterpret_cast<uint2*>(dK + off + d) =
          make_uint2(pack_bf16(scale * dk[db][r], scale * dk[db][r + 1]),
                     pack_bf16(scale * dk[db][r + 2], scale * dk[db][r + 3]));
      *reinterpret_cast<uint2*>(dV + off + d) =
          make_uint2(pack_bf16(dv[db][r], dv[db][r + 1]), pack_bf16(dv[db][r + 2], dv[db][r + 3]));
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
