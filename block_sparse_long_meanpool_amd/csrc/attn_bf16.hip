// moba_attn (bf16) — exact softmax attention over the selected blocks on the
// gfx950 matrix cores (PaperTrace "2.1.3 MoBA": history branch eq. (6) and
// causal own-block branch eq. (5), merged by eqs. (7)-(8); section 3.1 steps
// 4-5; section 5.4 on tiling queries per KV block).
//
// Tile engine shared by both kernels. A wavefront owns 32 queries (one
// 32-column block; QB blocks in general); a workgroup of 8 waves streams one
// K/V block in 64-key tiles through LDS (three buffers, one barrier per
// tile), so each K/V byte read from L2 serves 256 queries, and two waves
// share each SIMD. Tiles move global -> LDS with buffer_load ... lds (no
// register staging); rows are stored with their 16-byte chunks XOR-swizzled
// by the row index so the operand reads below are bank-conflict free.
// Per 32-key subtile and wave:
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, keys on rows and queries on
//                   columns: a lane holds 16 keys of one query, so a softmax
//                   row needs a single cross-half exchange;
//   softmax         exp2 domain, fp32 statistics. The reference max of a
//                   query is fixed by its first unmasked subtile and never
//                   moves, so the output accumulators stay in matrix-core
//                   registers untouched by vector code for the whole loop.
//                   Later scores may exceed it; if any exceeds it by more
//                   than 2^64 (an overflow risk) the workgroup re-runs the
//                   block starting from the true maximum (never for ordinary
//                   data; the result is identical either way up to rounding);
//   O^T += V^T P^T  P stays in the accumulator registers' layout and is the B
//                   operand directly; V comes pre-transposed and key-permuted
//                   (vt_pack) so each A operand is one 16-byte LDS read.
// History kernel: one workgroup per 256 routed queries of one (KV head,
// block) list, whole block (non-causal); writes the normalised partial output
// (fp16) and its log2-sum-exp. Own-block kernel: causal inside the block,
// then merges its queries' history partials (eqs. (7)-(8)) and writes O.
#include <type_traits>

#include "moba_internal.hpp"

namespace moba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef MOBA_ATTN_QB
#define MOBA_ATTN_QB 1
#endif
#ifndef MOBA_ATTN_WAVES
#define MOBA_ATTN_WAVES 8
#endif
constexpr int QB = MOBA_ATTN_QB;            // 32-query blocks per wave
constexpr int NW = MOBA_ATTN_WAVES;         // waves per workgroup
constexpr int kThreads = 64 * NW;
constexpr int kWaveQ = 32 * QB;             // queries per wave
constexpr int kGroupQ = NW * kWaveQ;        // queries per workgroup
constexpr int kLoadsPerWave = 16 / NW;      // 1 KB tile copies per wave (K and V each)
static_assert(kGroupQ == kTileQ, "history tiles are one workgroup");
constexpr int KT = 64;                      // keys per LDS tile
constexpr int KS_ROW = kHeadDim;            // bf16 per K row in LDS (256 B, swizzled)
constexpr int VT_ROW = KT;                  // bf16 per V^T row in LDS (128 B, swizzled)
constexpr int KS_ELEMS = KT * KS_ROW;
constexpr int VT_ELEMS = kHeadDim * VT_ROW;
constexpr float kLog2e = 1.4426950408889634f;

// One LDS tile buffer: a K part and a V^T part. The kernels declare each part
// of each of the three buffers as its own __shared__ array and unroll the key
// loop by three, so the compiler can see that the copies into one buffer never
// alias the operand reads from another (and need not wait for them).
struct Tile {
  uint16_t* k;  // [KT][KS_ROW]
  uint16_t* v;  // [kHeadDim][VT_ROW]
};
#define MOBA_DECLARE_TILES                                                  \
  __shared__ __align__(16) uint16_t lds_k0[KS_ELEMS], lds_k1[KS_ELEMS],    \
      lds_k2[KS_ELEMS];                                                     \
  __shared__ __align__(16) uint16_t lds_v0[VT_ELEMS], lds_v1[VT_ELEMS],    \
      lds_v2[VT_ELEMS];                                                     \
  Tile tA{lds_k0, lds_v0}, tB{lds_k1, lds_v1}, tC{lds_k2, lds_v2};

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// K row r keeps 16-byte chunk c at position c ^ (r & 15); V^T row d (two rows
// per 64 banks) keeps chunk c at c ^ (d & 7) ^ ((d >> 3) & 1). With these, the
// 16 lanes served together by one ds_read_b128 cycle hit 16 distinct bank quads.
__device__ inline int k_swz(int row, int c) { return c ^ (row & 15); }
__device__ inline int vt_swz(int d, int c) { return c ^ (d & 7) ^ ((d >> 3) & 1); }
__device__ inline const uint16_t* k_chunk(const uint16_t* ks, int row, int c) {
  return ks + row * KS_ROW + (k_swz(row, c) << 3);
}
__device__ inline const uint16_t* vt_chunk(const uint16_t* vt, int d, int c) {
  return vt + d * VT_ROW + (vt_swz(d, c) << 3);
}

// Buffer-resource word 3 for plain (untyped, raw) buffer accesses.
constexpr int kRawBufferFlags = 0x00020000;

// Issue the global -> LDS copies of one tile: keys [key0, key0+64) of K and
// the 64 matching packed V^T columns (block pads are zero). Each wave copies
// 16/NW KB of K and of V^T, 1 KB (64 lanes x 16 B) per buffer_load ... lds;
// the buffer resources are rebased per tile on the scalar side, so the
// per-lane offsets are loop invariant, and K rows past nvalid fall outside
// the resource's range and read as zero. The caller waits and barriers.
__device__ inline void load_tile(Tile t, const uint16_t* __restrict__ K, int64_t key0,
                                 int nvalid, int Hkv, int g, const uint16_t* __restrict__ vt_col,
                                 int64_t ldv, int wave, int lane) {
  const int64_t krow = (int64_t)Hkv * kHeadDim;  // elements between consecutive keys
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(K + (key0 * Hkv + g) * kHeadDim), 0,
      (int)(((int64_t)(nvalid - 1) * krow + kHeadDim) * 2), kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)vt_col, 0, (int)(((int64_t)(kHeadDim - 1) * ldv + KT) * 2), kRawBufferFlags);
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int ii = wave * kLoadsPerWave + i;  // 4 K rows per copy
    const int r = 4 * ii + (lane >> 4);
    const int c = k_swz(r, lane & 15);  // the swizzle is an involution in c
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, t.k + 4 * ii * KS_ROW, 16,
                                             (unsigned)((r * krow + 8 * c) * 2), 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int ii = wave * kLoadsPerWave + i;  // 8 V^T rows per copy
    const int d = 8 * ii + (lane >> 3);
    const int c = vt_swz(d, lane & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, t.v + 8 * ii * VT_ROW, 16,
                                             (unsigned)((d * ldv + 8 * c) * 2), 0, 0, 0);
  }
}

// Wait for this wave's outstanding loads (all counters), then a workgroup barrier.
__device__ inline void wait_tile() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Per-wave attention state; lane l holds query 32*qb + l%32 of each block.
struct Wave {
  bf16x8 q[QB][8];   // B operand of S^T = K Q^T: Q[query][16kk + 8h .. +8]
  f32x16 o[QB][4];   // O^T accumulators, d-blocks of 32
  float m[QB];       // reference max (log2 domain), fixed for the whole pass
  float l[QB];       // this lane's partial row sum
  float mx[QB];      // max-only pass: this lane's largest masked score
};

__device__ inline void wave_load_q(Wave& W, const uint16_t* const (&qrow)[QB],
                                   const bool (&valid)[QB], int h) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 u = valid[qb] ? *reinterpret_cast<const uint4*>(qrow[qb] + 16 * kk + 8 * h)
                          : make_uint4(0, 0, 0, 0);
      W.q[qb][kk] = as_bf16x8(u);
    }
}

__device__ inline void wave_reset(Wave& W, const float (&mstart)[QB]) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) W.o[qb][db][r] = 0.f;
    W.m[qb] = mstart[qb];
    W.l[qb] = 0.f;
    W.mx[qb] = -INFINITY;
  }
}

// Weights are 2^(score - m) with m fixed by the first subtile; their sum bounds
// every single weight. A pass is redone from the true maximum when some valid
// query's partial sum reaches 2^64 (or is not finite), so no weight or output
// accumulator can overflow in a pass that is kept.
constexpr float kLMax = 18446744073709551616.f;  // 2^64
__device__ inline bool wave_needs_redo(const Wave& W, const bool (&valid)[QB]) {
  bool r = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) r |= valid[qb] && !(W.l[qb] < kLMax);
  return r;
}

// After a max-only pass: each query's true maximum scaled score (log2 domain),
// 0 for queries with no unmasked key.
__device__ inline void wave_true_max(const Wave& W, float sl2e, float (&m)[QB]) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float v = fmaxf(W.mx[qb], __shfl_xor(W.mx[qb], 32)) * sl2e;
    m[qb] = (v == -INFINITY) ? 0.f : v;
  }
}

// Key row (0..31) of accumulator element r in the 32x32 MFMA output layout.
__device__ inline int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// S^T for 32-key subtile `sub` of an LDS tile: 8 matrix-core ops per query block.
__device__ inline void wave_qk(const Wave& W, Tile t, int sub, int lane, f32x16 (&s)[QB]) {
  const int h = lane >> 5, lr = lane & 31;
  const uint16_t* ks = t.k + sub * 32 * KS_ROW;  // the row swizzle uses (row & 15): same for row+32
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[qb][r] = 0.f;
  // The wave issuing these matrix ops gets the SIMD's issue priority, so
  // they reach the matrix core ahead of the other wave's softmax work (which
  // then fills the gaps); measured 0.6-1.4% faster than equal priority, while
  // raising it for the P.V ops or the exponentials instead was slower.
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(k_chunk(ks, lr, 2 * kk + h)));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, W.q[qb][kk], s[qb], 0, 0, 0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Mask one subtile's scores: keys >= nvalid (from the subtile start) and,
// when CAUSAL, keys with key0 + key > qrow get -inf.
template <bool CAUSAL>
__device__ inline void wave_mask(f32x16 (&s)[QB], int lane, int nvalid, int64_t key0,
                                 const int64_t (&qrow)[QB]) {
  const int h = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = acc_row(r, h);
      bool ok = key < nvalid;
      if (CAUSAL) ok = ok && (key0 + key <= qrow[qb]);
      if (!ok) s[qb][r] = -INFINITY;
    }
}

// Fix each query's reference max from its first subtile's (masked) scores.
__device__ inline void wave_set_reference(Wave& W, const f32x16 (&s)[QB], float sl2e) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float v = s[qb][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) v = fmaxf(v, s[qb][r]);
    v = fmaxf(v, __shfl_xor(v, 32)) * sl2e;
    W.m[qb] = (v == -INFINITY) ? 0.f : v;
  }
}

// Softmax of one subtile's scores against the fixed reference max, and its
// P.V product. MAXONLY: only track the largest masked score (no P.V).
template <bool CAUSAL, bool MAXONLY>
__device__ inline void wave_smpv(Wave& W, f32x16 (&s)[QB], Tile t, int sub, int lane,
                                 int nvalid, int64_t key0, const int64_t (&qrow)[QB], float sl2e,
                                 bool need_mask) {
  const int h = lane >> 5, lr = lane & 31;
  if (need_mask) wave_mask<CAUSAL>(s, lane, nvalid, key0, qrow);
  if (MAXONLY) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) W.mx[qb] = fmaxf(W.mx[qb], s[qb][r]);
    return;
  }
  bf16x8 p[QB][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float mneg = -W.m[qb];
    float lsum = W.l[qb];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x2 pr[4];  // weight pairs, each converted by one packed instruction
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f32x2 f;
        f[0] = __builtin_amdgcn_exp2f(fmaf(s[qb][8 * u + 2 * e], sl2e, mneg));
        f[1] = __builtin_amdgcn_exp2f(fmaf(s[qb][8 * u + 2 * e + 1], sl2e, mneg));
        pr[e] = __builtin_convertvector(f, bf16x2);
        // the row sum adds the fp32 weights (their bf16 rounding is unbiased;
        // a bf16 dot instruction here would stall the SIMD's matrix ops)
        lsum += f[0] + f[1];
      }
      const bf16x4 lo = __builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3);
      const bf16x4 hi = __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3);
      p[qb][u] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    W.l[qb] = lsum;
  }
  const int csub = 4 * sub;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16x8 a = as_bf16x8(
          *reinterpret_cast<const uint4*>(vt_chunk(t.v, 32 * db + lr, csub + 2 * u + h)));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        W.o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[qb][u], W.o[qb][db], 0, 0, 0);
    }
}

// Stream keys [key0, key0 + nkeys) of one block (K rows from K, V^T columns
// from vt_col) through three LDS tile buffers and run the wave pipeline:
// the scores of the next subtile are issued to the matrix cores before the
// softmax of the current one, so exponentials overlap matrix work inside
// each wave. One barrier per 64-key tile; the copy of tile t+2 starts right
// after the barrier that publishes tile t+1 and lands in the buffer tile t-1
// used (every wave is past it by then). Waves whose rows start after a
// subtile (CAUSAL) or that hold no queries skip its compute, never a barrier.
template <bool CAUSAL, bool FULL, bool MAXONLY>
__device__ inline void run_block(Wave& W, Tile b0, Tile b1, Tile b2,
                                 const uint16_t* __restrict__ K, int64_t key0, int64_t nkeys,
                                 int Hkv, int g, const uint16_t* __restrict__ vt_col, int64_t ldv,
                                 int wave, int lane, const int64_t (&qrow)[QB], int64_t wrow_min,
                                 int64_t wrow_max, bool wave_live, float sl2e, bool set_m) {
  const int nt = (int)((nkeys + KT - 1) / KT);
  // FULL: every subtile has 32 keys and every wave computes (the caller checked)
  auto nvs_of = [&](int t, int sub) -> int {
    if (FULL) return 32;
    const int64_t rem = nkeys - (int64_t)t * KT - 32 * sub;
    return rem <= 0 ? 0 : (rem < 32 ? (int)rem : 32);
  };
  auto active = [&](int t, int sub) -> bool {
    if (FULL) return true;
    if (!wave_live || nvs_of(t, sub) == 0) return false;
    return !CAUSAL || key0 + (int64_t)t * KT + 32 * sub <= wrow_max;
  };
  auto issue = [&](int t, Tile dst) {
    const int64_t rem = nkeys - (int64_t)t * KT;
    load_tile(dst, K, key0 + (int64_t)t * KT, rem < KT ? (int)rem : KT, Hkv, g, vt_col + t * KT,
              ldv, wave, lane);
  };
  auto smpv = [&](f32x16 (&s)[QB], Tile cur, int t, int sub) {
    const int nv = nvs_of(t, sub);
    const int64_t k0 = key0 + (int64_t)t * KT + 32 * sub;
    const bool need_mask = nv < 32 || (CAUSAL && k0 + 31 > wrow_min);
    wave_smpv<CAUSAL, MAXONLY>(W, s, cur, sub, lane, nv, k0, qrow, sl2e, need_mask);
  };
  f32x16 sa[QB], sb[QB];
  auto step = [&](int t, Tile cur, Tile nxt, Tile spare) {
    // entering: sa holds the scores of (t, 0) when that subtile is active.
    // Scheduling barriers keep each phase's matrix ops next to the vector
    // work they are meant to overlap instead of letting later phases hoist.
    if (active(t, 1)) wave_qk(W, cur, 1, lane, sb);
    if (active(t, 0)) smpv(sa, cur, t, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < nt) {
      wait_tile();
      if (t + 2 < nt) issue(t + 2, spare);
      if (active(t + 1, 0)) wave_qk(W, nxt, 0, lane, sa);
    }
    if (active(t, 1)) smpv(sb, cur, t, 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  issue(0, b0);
  wait_tile();
  if (nt > 1) issue(1, b1);
  if (active(0, 0)) {
    wave_qk(W, b0, 0, lane, sa);
    // The first subtile holds an unmasked key of every valid query: the causal
    // block starts at or before each row, and history blocks are never empty.
    if (!MAXONLY && set_m) {
      const int nv = nvs_of(0, 0);
      if (nv < 32 || (CAUSAL && key0 + 31 > wrow_min)) wave_mask<CAUSAL>(sa, lane, nv, key0, qrow);
      wave_set_reference(W, sa, sl2e);
    }
  }
  for (int t = 0; t < nt; t += 3) {
    step(t, b0, b1, b2);
    if (t + 1 < nt) step(t + 1, b1, b2, b0);
    if (t + 2 < nt) step(t + 2, b2, b0, b1);
  }
  __syncthreads();  // all waves are done with the buffers before they are reused
}

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// Final outputs of R (row, head) pairs for the 8 head-dim elements
// [8 c16, 8 c16 + 8): each pair's own-block result (normalised `own`,
// log2-sum-exp own_lse) merged with its nhist >= 1 history partials
// (normalised rows po[s], log2-sum-exps lse[s]) by PaperTrace "2.1.3 MoBA"
// eqs. (7)-(8). NH >= nhist is a compile-time bound so the loads of a group
// of partials of all R pairs are in flight before their values are used;
// slots past nhist are not loaded (they count as log2-sum-exp -inf, weight
// 0), so every load reads one of the pair's own partials once.
template <int NH, int R>
__device__ inline void merge_rows(const h8 (&own)[R], const float (&own_lse)[R],
                                  const float* const (&lse_src)[R],
                                  const _Float16* const (&po_src)[R], int nhist, int c16,
                                  b8 (&out)[R], float (&lse_out)[R]) {
  constexpr int GRP = NH < 16 ? NH : 16;  // partial rows of a pair in flight together
  float lse[R][NH];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int s = 0; s < NH; ++s) lse[i][s] = s < nhist ? lse_src[i][s] : -INFINITY;
  float M[R], L[R], acc[R][8];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    M[i] = own_lse[i];
#pragma unroll
    for (int s = 0; s < NH; ++s) M[i] = fmaxf(M[i], lse[i][s]);  // slots past nhist hold -inf
    L[i] = __builtin_amdgcn_exp2f(own_lse[i] - M[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = L[i] * (float)own[i][e];
  }
#pragma unroll
  for (int s0 = 0; s0 < NH; s0 += GRP) {
    if (s0 >= nhist) break;
    h8 v[R][GRP];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        v[i][j] = s0 + j < nhist
                      ? *reinterpret_cast<const h8*>(po_src[i] + (size_t)(s0 + j) * kHeadDim + 8 * c16)
                      : h8{};
      }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const float w = s0 + j < nhist ? __builtin_amdgcn_exp2f(lse[i][s0 + j] - M[i]) : 0.f;
        L[i] += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(w, (float)v[i][j][e], acc[i][e]);
      }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float inv = 1.f / L[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[i][e] = (__bf16)(acc[i][e] * inv);
    lse_out[i] = M[i] + __builtin_log2f(L[i]);  // the row's log2-sum-exp over all its keys
  }
}

// ----------------------------------------------------------------------------
// History attention: one workgroup = up to 256 routed entries of one bin.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void attn_hist_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ Vt,
    const int32_t* __restrict__ bstart, const int32_t* __restrict__ tile_map,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ bin_off,
    const int32_t* __restrict__ scalars, const uint32_t* __restrict__ entries,
    _Float16* __restrict__ part_o, float* __restrict__ part_lse, int Hkv, int B, int64_t Bpad,
    int64_t ldv, int KH, int64_t nh, float sl2e, int Hq, int Hs, int h0, int64_t bin0,
    int64_t bin1) {
  MOBA_DECLARE_TILES
  // XCD-aware order: workgroup i runs on XCD i % 8; each XCD takes a
  // contiguous range of tiles so the tiles of one K/V block share its L2.
  // The grid is a multiple of 8, so this is a bijection on [0, gridDim.x).
  // The tiles are those of this attention pass's bins [bin0, bin1).
  const int64_t per = gridDim.x / 8;
  const int64_t first = tile_off[bin0];
  const int64_t w = first + (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= tile_off[bin1]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int bin = tile_map[w];
  const int64_t e_begin = bin_off[bin] + (w - tile_off[bin]) * (int64_t)kTileQ;
  const int64_t e_end = bin_off[bin + 1];
  const int g = (int)(bin / nh);
  const int64_t j = bin % nh;

  uint32_t ev[QB];
  bool valid[QB];
  const uint16_t* qrow[QB];
  int64_t dummy_row[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t e = e_begin + wave * kWaveQ + qb * 32 + (lane & 31);
    valid[qb] = e < e_end;
    ev[qb] = valid[qb] ? entries[e] : 0u;
    // e / KH = row * Hs + (head - h0) over the pass's heads; Q row = row * Hq + head
    const uint32_t pr = ev[qb] / (uint32_t)KH;
    qrow[qb] = Q + ((int64_t)pr + (int64_t)(pr / (uint32_t)Hs) * (Hq - Hs) + h0) * kHeadDim;
    dummy_row[qb] = 0;
  }
  Wave W;
  wave_load_q(W, qrow, valid, h);

  const int64_t kbase = bstart[j];  // history blocks are always full
  const uint16_t* vt_col = Vt + (int64_t)g * kHeadDim * ldv + j * Bpad;
  const int ntiles = (B + KT - 1) / KT;
  const bool wave_live = (e_begin + wave * kWaveQ) < e_end;
  float mstart[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mstart[qb] = 0.f;
  wave_reset(W, mstart);
  if (B % KT == 0 && e_begin + kGroupQ <= e_end)
    run_block<false, true, false>(W, tA, tB, tC, K, kbase, B, Hkv, g, vt_col, ldv, wave, lane,
                                  dummy_row, 0, 0, wave_live, sl2e, true);
  else
    run_block<false, false, false>(W, tA, tB, tC, K, kbase, B, Hkv, g, vt_col, ldv, wave, lane,
                                   dummy_row, 0, 0, wave_live, sl2e, true);
  // workgroup-uniform: if some weight could have overflowed, find the true
  // maxima with a max-only pass and redo the block from them (weights <= 1)
  if (__syncthreads_or(wave_needs_redo(W, valid))) {
    wave_reset(W, mstart);
    run_block<false, false, true>(W, tA, tB, tC, K, kbase, B, Hkv, g, vt_col, ldv, wave, lane,
                                  dummy_row, 0, 0, wave_live, sl2e, false);
    wave_true_max(W, sl2e, mstart);
    wave_reset(W, mstart);
    run_block<false, false, false>(W, tA, tB, tC, K, kbase, B, Hkv, g, vt_col, ldv, wave, lane,
                                   dummy_row, 0, 0, wave_live, sl2e, false);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = W.l[qb] + __shfl_xor(W.l[qb], 32);
    if (!valid[qb]) continue;
    const float inv = 1.f / l;
    _Float16* dst = part_o + (size_t)ev[qb] * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        h4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (_Float16)(W.o[qb][db][4 * r4 + t] * inv);
        *reinterpret_cast<h4*>(dst + 32 * db + 8 * r4 + 4 * h) = v;
      }
    if (h == 0) part_lse[ev[qb]] = W.m[qb] + __builtin_log2f(l);
  }
}

// ----------------------------------------------------------------------------
// Own-block causal attention + merge. One workgroup = 256 (row, head) pairs
// of one KV-head group inside one block; pairs ordered pi = (row - cB)*G + hh.
// dense: the "block" is the whole sequence and there are no partials.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void attn_self_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ Vt,
    const int32_t* __restrict__ bstart, const int32_t* __restrict__ qstart,
    const int32_t* __restrict__ qlen, const int32_t* __restrict__ qpos,
    const int32_t* __restrict__ blo, const _Float16* __restrict__ part_o,
    const float* __restrict__ part_lse, uint16_t* __restrict__ O, float* __restrict__ lse_out,
    int Hq, int Hkv, int G, int64_t Bpad, int64_t ldv, int KH, int64_t n, int64_t nqb,
    int tiles_per_block, float sl2e, int g0, int gs) {
  MOBA_DECLARE_TILES
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  // Work items w = ((c' * gs) + g - g0) * tiles_per_block + t' over this
  // attention pass's KV heads [g0, g0 + gs), in order of blocks from the last
  // (only the last nqb blocks hold query rows), and inside a block heavier
  // (later) row tiles first. Workgroup i runs on XCD i % 8 and each XCD takes
  // a contiguous range of items, so the row tiles of one (block, KV head)
  // share its L2 copy of K/V.
  const int64_t items = nqb * gs * (int64_t)tiles_per_block;
  const int64_t per = gridDim.x / 8;  // the grid is a multiple of 8
  const int64_t w = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= items) return;
  const int tile = tiles_per_block - 1 - (int)(w % tiles_per_block);
  const int g = g0 + (int)((w / tiles_per_block) % gs);
  const int64_t c = n - 1 - w / ((int64_t)tiles_per_block * gs);
  const int Hs = gs * G, h0 = g0 * G;  // the pass's query heads, for its partials
  // keys from the block's first row; query rows (of Q and O) and their
  // positions (for the causal mask) from the block's query range
  const int64_t key0 = bstart[c], qrow0 = qstart[c], pos0 = qpos[c];
  const int64_t npairs = (int64_t)qlen[c] * G;
  const int64_t p0 = (int64_t)tile * kGroupQ;
  if (p0 >= npairs) return;
  const int64_t plast = (p0 + kGroupQ - 1 < npairs) ? p0 + kGroupQ - 1 : npairs - 1;
  const int64_t last_row = pos0 + plast / G;

  bool valid[QB];
  int64_t my_row[QB], ph[QB];
  const uint16_t* qrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t pi = p0 + wave * kWaveQ + qb * 32 + (lane & 31);
    valid[qb] = pi < npairs;
    my_row[qb] = valid[qb] ? pos0 + pi / G : -1;
    ph[qb] = valid[qb] ? (qrow0 + pi / G) * Hq + g * G + (int)(pi % G) : 0;
    qrow[qb] = Q + ph[qb] * kHeadDim;
  }
  Wave W;
  wave_load_q(W, qrow, valid, h);

  const int64_t wp0 = p0 + wave * kWaveQ;
  const bool wave_live = wp0 < npairs;
  const int64_t wp1 = (wp0 + kWaveQ - 1 < npairs) ? wp0 + kWaveQ - 1 : npairs - 1;
  const int64_t wrow_min = pos0 + wp0 / G;
  const int64_t wrow_max = pos0 + wp1 / G;

  const int64_t nkeys = last_row - key0 + 1;
  const int ntiles = (int)((nkeys + KT - 1) / KT);
  const uint16_t* vt_col = Vt + (int64_t)g * kHeadDim * ldv + c * Bpad;
  // Whole 64-key tiles before the workgroup's first row are unmasked for every
  // one of its queries: they go through the unmasked engine, the rest causally.
  const int64_t nfull = ((pos0 + p0 / G - key0 + 1) / KT) * KT;
  auto pass = [&](auto maxonly, bool set_m) {
    constexpr bool MO = decltype(maxonly)::value;
    if (nfull > 0)
      run_block<false, true, MO>(W, tA, tB, tC, K, key0, nfull, Hkv, g, vt_col, ldv, wave, lane,
                                 my_row, 0, 0, true, sl2e, set_m);
    if (nkeys > nfull)
      run_block<true, false, MO>(W, tA, tB, tC, K, key0 + nfull, nkeys - nfull, Hkv, g,
                                 vt_col + nfull, ldv, wave, lane, my_row, wrow_min, wrow_max,
                                 wave_live, sl2e, set_m && nfull == 0);
  };
  float mstart[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mstart[qb] = 0.f;
  wave_reset(W, mstart);
  pass(std::false_type{}, true);
  if (__syncthreads_or(wave_needs_redo(W, valid))) {
    wave_reset(W, mstart);
    pass(std::true_type{}, false);
    wave_true_max(W, sl2e, mstart);
    wave_reset(W, mstart);
    pass(std::false_type{}, false);
  }
  const int64_t nbefore = c - blo[c];  // earlier blocks of the row's sequence
  const int nhist = part_o != nullptr ? (int)(nbefore < KH ? nbefore : KH) : 0;  // uniform
  if (nhist == 0) {
    // no history: O = own-block result, straight from the accumulators
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = W.l[qb] + __shfl_xor(W.l[qb], 32);
      if (!valid[qb]) continue;
      if (lse_out && h == 0) lse_out[ph[qb]] = W.m[qb] + __builtin_log2f(l);
      const float inv = 1.f / l;
      uint16_t* dst = O + ph[qb] * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          b4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = (__bf16)(W.o[qb][db][4 * r4 + t] * inv);
          *reinterpret_cast<b4*>(dst + 32 * db + 8 * r4 + 4 * h) = v;
        }
    }
    return;
  }
  // Stage each wave's own-block results in the (now idle) tile buffers as
  // normalised fp16 rows plus log2-sum-exps, then merge with 16 lanes per
  // (row, head) so each partial row is one coalesced 256-byte read. Staged
  // row j keeps its 16-byte chunk c at position c ^ (j & 15), so the stores
  // (one chunk of 32 rows at a time) spread over the banks.
  uint16_t* const wbuf = wave < 2 ? lds_k0 : wave < 4 ? lds_k1 : wave < 6 ? lds_k2 : lds_v0;
  _Float16* const stage = reinterpret_cast<_Float16*>(wbuf) + (wave & 1) * kWaveQ * kHeadDim;
  float* const stage_lse = reinterpret_cast<float*>(lds_v1) + wave * kWaveQ;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = W.l[qb] + __shfl_xor(W.l[qb], 32);
    const float inv = 1.f / l;
    const int j = qb * 32 + (lane & 31);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        h4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (_Float16)(W.o[qb][db][4 * r4 + t] * inv);
        *reinterpret_cast<h4*>(stage + j * kHeadDim + 8 * ((4 * db + r4) ^ (j & 15)) + 4 * h) = v;
      }
    if (h == 0) stage_lse[j] = W.m[qb] + __builtin_log2f(l);
  }
  __syncthreads();
  const int q4 = lane >> 4, c16 = lane & 15;
  // R passes (4 pairs each, 16 lanes per pair) merged together: two while a
  // pair's partials fit the registers comfortably, else one
  auto merge_passes = [&](auto nh_tag, auto r_tag) {
    constexpr int NH = decltype(nh_tag)::value, R = decltype(r_tag)::value;
    for (int pass = 0; pass < kWaveQ / 4; pass += R) {
      int64_t pi[R], phj[R];
      h8 own[R];
      float own_lse[R];
      const float* ls[R];
      const _Float16* po[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int j = (pass + i) * 4 + q4;
        pi[i] = p0 + wave * kWaveQ + j;
        const int64_t pic = pi[i] < npairs ? pi[i] : npairs - 1;  // clamped: loads stay in bounds
        phj[i] = (qrow0 + pic / G) * Hq + g * G + (int)(pic % G);
        // the pass's partial slots of this (row, head)
        const int64_t pslot = ((qrow0 + pic / G) * Hs + (g * G - h0) + (int)(pic % G)) * KH;
        own[i] = *reinterpret_cast<const h8*>(stage + j * kHeadDim + 8 * (c16 ^ (j & 15)));
        own_lse[i] = stage_lse[j];
        ls[i] = part_lse + pslot;
        po[i] = part_o + (size_t)pslot * kHeadDim;
      }
      b8 out[R];
      float lse_row[R];
      merge_rows<NH, R>(own, own_lse, ls, po, nhist, c16, out, lse_row);
#pragma unroll
      for (int i = 0; i < R; ++i)
        if (pi[i] < npairs) {
          *reinterpret_cast<b8*>(O + phj[i] * kHeadDim + 8 * c16) = out[i];
          if (lse_out && c16 == 0) lse_out[phj[i]] = lse_row[i];
        }
    }
  };
  using one = std::integral_constant<int, 1>;
  using two = std::integral_constant<int, 2>;
  static_assert((kWaveQ / 4) % 2 == 0, "whole pairs of passes");
  if (nhist <= 4)
    merge_passes(std::integral_constant<int, 4>{}, two{});
  else if (nhist <= 8)
    merge_passes(std::integral_constant<int, 8>{}, two{});
  else if (nhist <= 12)
    merge_passes(std::integral_constant<int, 12>{}, two{});
  else if (nhist <= 16)
    merge_passes(std::integral_constant<int, 16>{}, one{});
  else
    merge_passes(std::integral_constant<int, kMaxTopk>{}, one{});
}

}  // namespace

int64_t vt_padded_block(int64_t B) { return ceil_div(B, KT) * KT; }

hipError_t launch_attn_hist_bf16(const Prob& P, const Blocks& T, const BucketPlan& bp,
                                 const void* Q, const void* K, const void* Vt,
                                 const BucketBufs& b, void* part_o, float* part_lse,
                                 hipStream_t s) {
  if (P.nh <= 0 || P.KH <= 0 || bp.max_tiles <= 0) return hipSuccess;
  const float sl2e = P.scale * kLog2e;
  const int64_t Bpad = vt_padded_block(P.B);
  const int64_t ldv = P.vt_blocks * Bpad;
  const int64_t grid = ceil_div(pass_max_tiles(P), 8) * 8;
  attn_hist_bf16<<<(unsigned)grid, kThreads, 0, s>>>(
      (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)Vt, T.start, b.tile_map,
      b.tile_off, b.bin_off, b.scalars, b.entries, (_Float16*)part_o, part_lse, P.Hkv, P.B, Bpad,
      ldv, P.KH, P.nh, sl2e, P.Hq, pass_heads(P), pass_h0(P), (int64_t)P.g0 * P.nh,
      (int64_t)(P.g0 + P.gs) * P.nh);
  return hipGetLastError();
}

hipError_t launch_attn_self_bf16(const Prob& P, const Blocks& T, const void* Q, const void* K,
                                 const void* Vt, const void* part_o, const float* part_lse,
                                 void* O, float* lse_out, hipStream_t s) {
  const float sl2e = P.scale * kLog2e;
  const int64_t Bpad = vt_padded_block(P.B);
  const int64_t ldv = P.vt_blocks * Bpad;
  const int tiles_per_block = (int)ceil_div((int64_t)P.B * P.G, kGroupQ);
  const int64_t nqb = query_blocks(P);
  const int64_t grid = ceil_div(nqb * tiles_per_block * P.gs, 8) * 8;
  const bool merge = part_o != nullptr && P.KH > 0;
  attn_self_bf16<<<(unsigned)grid, kThreads, 0, s>>>(
      (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)Vt, T.start, T.qstart, T.qlen,
      T.qpos, T.lo, merge ? (const _Float16*)part_o : nullptr, merge ? part_lse : nullptr,
      (uint16_t*)O, lse_out, P.Hq,
      P.Hkv, P.G, Bpad, ldv, merge ? P.KH : 0, P.n, nqb, tiles_per_block, sl2e, P.g0, P.gs);
  return hipGetLastError();
}

}  // namespace moba
