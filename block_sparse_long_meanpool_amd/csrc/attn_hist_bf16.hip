// moba_attn history branch (bf16), wide-wave engine — the dominant kernel of
// the path: exact softmax attention of the routed queries of one (KV head,
// history block) list over that whole block (PaperTrace "2.1.3 MoBA": the
// history branch of eq. (6), section 3.1 step 4; section 5.4 on tiling the
// queries that share a KV block).
//
// One workgroup = 4 waves, one per SIMD, 64 queries per wave = 256 routed
// entries. Each 32x32x16 matrix op reads its K or V^T operand from LDS once
// and applies it to both 32-query halves of the wave, so the LDS bytes per
// matrix op are half those of a 32-query wave; the vector work per op is
// unchanged. With one wave per SIMD the wave hides its own softmax behind its
// matrix ops: per 32-key subtile j it issues, with no data dependence among
// them,
//   the scores of subtile j+2      S^T = K Q^T   (16 ops),
//   the output update of subtile j O^T += V^T P^T (16 ops),
//   the softmax of subtile j+1     (exp2 against a fixed reference max),
// so scores are two subtiles and weights one subtile ahead of their use.
// Registers: Q 64 and two score sets 64 and two weight sets 32 VGPRs, the
// output 128 accumulation registers.
//
// K and V^T move global -> LDS in 64-key tiles through four buffers
// (buffer_load ... lds, no register staging). One barrier per tile, placed
// inside the tile's second subtile once the wave has read the tile's last
// V^T chunk: after it, the tile's buffer is refilled with the tile four
// ahead, so two tiles are always in flight, and the barrier sits between
// matrix ops instead of at a point where the matrix pipe has drained. K rows
// keep their 16-byte chunks XOR-swizzled by row and V^T rows by d, so every
// operand read is
// bank-conflict free. V^T comes from vt_pack: per KV head [d][block-padded
// keys], keys permuted inside each 32-key group (bits 2 and 3 swapped) so a
// lane's 8 weights of the P operand meet one 16-byte V^T chunk.
//
// Softmax: weights are 2^(s - m) with m, per query, the largest score of the
// first subtile (every query has 32 unmasked keys there). The output
// accumulators are never rescaled; if some later score exceeds m by enough
// that a row sum reaches 2^64, the tile is listed and a second kernel
// recomputes it from the true maxima found by a score-only pass (never for
// ordinary data; the result is the same up to rounding). Each normalised
// partial is stored in fp16 with its log2-sum-exp in fp32, at the entry's
// slot.
//
// Workgroups are persistent (one per compute unit) and walk their XCD's
// history tiles; the K/V tile stream and the Q rows of the next history tile
// are fetched during the current tile's last steps, so the pipeline does not
// drain between tiles.
//
// Used when the block size is a multiple of 256 (whole groups of four tiles:
// every tile full, static buffer roles in an unrolled loop); other block
// sizes take the 32-query engine of attn_bf16.hip.
#include <algorithm>

#include "moba_internal.hpp"

namespace moba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;                 // waves per workgroup, one per SIMD
constexpr int kThreads = 64 * NW;
constexpr int kWaveQ = 64;            // queries per wave (two 32-column blocks)
static_assert(NW * kWaveQ == kTileQ, "a history tile is one workgroup");
constexpr int KT = 64;                // keys per LDS tile (two 32-key subtiles)
constexpr int KS_ROW = kHeadDim;      // bf16 per K row in LDS
constexpr int VT_ROW = KT;            // bf16 per V^T row in LDS
constexpr int KS_ELEMS = KT * KS_ROW;
constexpr int VT_ELEMS = kHeadDim * VT_ROW;
constexpr int kCopies = 16 / NW;      // 1 KB copies of K and of V^T per wave and tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLMax = 18446744073709551616.f;  // 2^64
constexpr int kRawBufferFlags = 0x00020000;      // buffer resource word 3, raw access

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// K row r keeps 16-byte chunk c at c ^ (r & 15); V^T row d keeps chunk c at
// c ^ (d & 7) ^ ((d >> 3) & 1): the 16 lanes served by one ds_read_b128
// cycle then hit 16 distinct bank quads.
__device__ inline int k_swz(int row, int c) { return c ^ (row & 15); }
__device__ inline int vt_swz(int d, int c) { return c ^ (d & 7) ^ ((d >> 3) & 1); }

struct Tile {
  uint16_t* k;  // [KT][KS_ROW]
  uint16_t* v;  // [kHeadDim][VT_ROW]
};

// The copies of one tile: keys [key0, key0 + 64) of K (row stride krow
// elements) and V^T columns [col0, col0 + 64) of every d row (row stride
// ldv). Each wave makes 8 copies of 1 KB (64 lanes x 16 B), copy i < 4: four
// K rows, copy i >= 4: eight V^T rows; rows keep the LDS swizzle. The buffer
// resources are rebased per tile on the scalar side, so the per-lane offsets
// are loop invariant.
struct TileSrc {
  __amdgpu_buffer_rsrc_t kr, vr;
};
__device__ inline TileSrc tile_src(const uint16_t* __restrict__ kbase, int64_t krow,
                                   const uint16_t* __restrict__ vbase, int64_t ldv) {
  TileSrc t;
  t.kr = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0,
                                           (int)(((int64_t)(KT - 1) * krow + kHeadDim) * 2),
                                           kRawBufferFlags);
  t.vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)vbase, 0, (int)(uint32_t)(((int64_t)(kHeadDim - 1) * ldv + KT) * 2), kRawBufferFlags);
  return t;
}
__device__ inline void copy_part(Tile dst, const TileSrc& src, int64_t krow, int64_t ldv, int i,
                                 int wave, int lane) {
  if (i < kCopies) {
    const int ii = wave * kCopies + i;  // 4 K rows per copy
    const int r = 4 * ii + (lane >> 4);
    const int c = k_swz(r, lane & 15);  // the swizzle is an involution in c
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.kr, dst.k + 4 * ii * KS_ROW, 16,
                                             (unsigned)((r * krow + 8 * c) * 2), 0, 0, 0);
  } else {
    const int ii = wave * kCopies + (i - kCopies);  // 8 V^T rows per copy
    const int d = 8 * ii + (lane >> 3);
    const int c = vt_swz(d, lane & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.vr, dst.v + 8 * ii * VT_ROW, 16,
                                             (unsigned)((d * ldv + 8 * c) * 2), 0, 0, 0);
  }
}
__device__ inline void load_tile(Tile dst, const TileSrc& src, int64_t krow, int64_t ldv,
                                 int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2 * kCopies; ++i) copy_part(dst, src, krow, ldv, i, wave, lane);
}

// Wait until at most `left` of this wave's tile copies are outstanding and
// its LDS reads have completed, then a workgroup barrier: every wave's copies
// of the older tiles have landed and no wave still reads a buffer that is
// about to be refilled.
template <int left>
__device__ inline void wait_tiles() {
  static_assert(left == 0 || left == kCopies * 2 || left == kCopies * 4 || left == 63, "");
  // s_waitcnt: vmcnt = left (bits 3:0 and 15:14), expcnt not waited on, lgkmcnt 0
  constexpr int imm = (left & 15) | ((left >> 4) << 14) | (7 << 4) | (0 << 8);
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
}

// Per-wave state; lane l holds query l % 32 of each 32-query block qb.
struct Wave {
  bf16x8 q[2][8];  // B operand of S^T = K Q^T: Q[query][16 kk + 8 h .. +8]
  f32x16 o[2][4];  // O^T accumulators, d blocks of 32
  float m[2];      // reference max (log2 domain)
  float l[2];      // this lane's partial row sum (16 of the 32 keys of each subtile)
};

// LDS operand reads: K chunk kk of row lr of a subtile (chunk 2 kk + h), and
// V^T chunk i = 4 u + db (row 32 db + lr, chunk 4 sub + 2 u + h).
__device__ inline bf16x8 read_k(const uint16_t* ks, int sub, int kk, int lane) {
  const int h = lane >> 5, lr = lane & 31;
  const uint16_t* row = ks + (sub * 32 + lr) * KS_ROW;  // the row swizzle uses (row & 15)
  return as_bf16x8(*reinterpret_cast<const uint4*>(row + (k_swz(lr, 2 * kk + h) << 3)));
}
__device__ inline bf16x8 read_v(const uint16_t* vt, int sub, int i, int lane) {
  const int h = lane >> 5, lr = lane & 31;
  const int d = 32 * (i & 3) + lr;
  return as_bf16x8(*reinterpret_cast<const uint4*>(
      vt + d * VT_ROW + (vt_swz(d, 4 * sub + 2 * (i >> 2) + h) << 3)));
}

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Scores of one subtile for both query blocks, in program order (no overlap).
__device__ inline void qk_plain(const Wave& W, const uint16_t* ks, int sub, int lane,
                                f32x16 (&s)[2]) {
  const f32x16 zero = {};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 a = read_k(ks, sub, kk, lane);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) s[qb] = mfma(a, W.q[qb][kk], kk ? s[qb] : zero);
  }
}

// The softmax of one subtile is 16 units (qb, u, e), unit = 8 qb + 4 u + e:
// two scores -> two weights 2^(s sl2e - m) -> one bf16 pair for the P.V
// product, and the fp32 weights added to the row sum (the bf16 rounding of
// the weights is unbiased, so the normalisation does not need the rounded
// values; a bf16 dot instruction for the sum would stall the wave's matrix
// ops). A unit has five stages, each reading only what an earlier stage
// wrote:
//   F0: t0 = s0 sl2e - m      F1E0: t1 = s1 sl2e - m, e0 = 2^t0
//   E1: e1 = 2^t1             C: pair = bf16(e0, e1), e01 = e0 + e1
//   D: lsum += e01
struct Unit {
  float t0, t1, e0, e1, e01;
};
// Pins a value to this point of the instruction stream: an empty statement
// that the compiler must treat as reading and rewriting the register, so the
// arithmetic producing the value stays before it and the arithmetic
// consuming it stays after it (keeps each stage in its slot).
template <typename T>
__device__ inline void pin(T& v) {
  asm volatile("" : "+v"(v));
}
__device__ inline void st_f0(const f32x16 (&s)[2], const Wave& W, int u, float sl2e, Unit& x) {
  const int qb = u >> 3, r = 2 * (u & 7);
  float a = s[qb][r];
  pin(a);
  x.t0 = fmaf(a, sl2e, -W.m[qb]);
  pin(x.t0);
}
__device__ inline void st_f1e0(const f32x16 (&s)[2], const Wave& W, int u, float sl2e, Unit& x) {
  const int qb = u >> 3, r = 2 * (u & 7) + 1;
  float a = s[qb][r];
  pin(a);
  x.t1 = fmaf(a, sl2e, -W.m[qb]);
  pin(x.t1);
  x.e0 = __builtin_amdgcn_exp2f(x.t0);
  pin(x.e0);
}
__device__ inline void st_e1(Unit& x) {
  x.e1 = __builtin_amdgcn_exp2f(x.t1);
  pin(x.e1);
}
__device__ inline void st_c(Unit& x, int u, bf16x2 (&pr)[2][2][4]) {
  f32x2 f;
  f[0] = x.e0;
  f[1] = x.e1;
  bf16x2 p = __builtin_convertvector(f, bf16x2);
  pin(p);
  pr[u >> 3][(u >> 2) & 1][u & 3] = p;
  x.e01 = x.e0 + x.e1;
  pin(x.e01);
}
__device__ inline void st_d(const Unit& x, int u, float (&lsum)[2]) {
  lsum[u >> 3] += x.e01;
  pin(lsum[u >> 3]);
}
__device__ inline bf16x8 gather_p(const bf16x2 (&pr)[4]) {
  const bf16x4 lo = __builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3);
  const bf16x4 hi = __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The softmax of one subtile in program order (pipeline start).
__device__ inline void softmax_plain(Wave& W, const f32x16 (&s)[2], float sl2e,
                                     bf16x8 (&p)[2][2]) {
  bf16x2 pr[2][2][4];
  float lsum[2] = {W.l[0], W.l[1]};
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    Unit x;
    st_f0(s, W, u, sl2e, x);
    st_f1e0(s, W, u, sl2e, x);
    st_e1(x);
    st_c(x, u, pr);
    st_d(x, u, lsum);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    p[qb][0] = gather_p(pr[qb][0]);
    p[qb][1] = gather_p(pr[qb][1]);
    W.l[qb] = lsum[qb];
  }
}

// One pipeline iteration, issued in a fixed order of 32 slots, each one
// matrix op followed by the vector work of that slot:
//   the output update of subtile j, 16 ops m = 0..15 (V^T chunk m / 2, query
//     block m % 2, weights pc): slots 0-5 and 22-31;
//   the scores of subtile j+2 into sn, 16 ops n = 0..15 (K chunk n / 2,
//     query block n % 2): slots 6-21. The two query blocks' accumulation
//     chains alternate, so no matrix op waits on the result of the one just
//     before it, and both chains end ten slots before the next iteration
//     reads them;
//   the softmax of subtile j+1 (scores sc, final since the previous
//     iteration) into pn: unit u runs F0 at slot 2u, F1E0 at 2u+1, E1 at
//     2u+2, C at 2u+3, D at 2u+4, so a slot's vector instructions (about 16
//     cycles of issue each) never wait on one another; the stages past slot
//     31 of the last two units are issued at slot 31.
// Operand reads run six slots ahead of their matrix ops: K chunk kk at slot
// 2 kk, V^T chunk i >= 3 at slot 2 i + 10; V^T chunks 0-2 come from the
// previous iteration (vpre), which reads the next iteration's at slots 26,
// 28, 30 from (vn, sv). In the first iteration of a tile only those V^T
// chunks precede the barrier. A scheduling fence after every slot keeps the
// order.
struct Slot {
  int8_t pv, qk, rk, rv;  // output-update op m, score op n, K chunk read, V^T chunk read (-1: none)
};
constexpr Slot kSlots[32] = {
    {0, -1, 0, -1},   {1, -1, -1, -1},  {2, -1, 1, -1},   {3, -1, -1, -1},
    {4, -1, 2, -1},   {5, -1, -1, -1},  {-1, 0, 3, -1},   {-1, 1, -1, -1},
    {-1, 2, 4, -1},   {-1, 3, -1, -1},  {-1, 4, 5, -1},   {-1, 5, -1, -1},
    {-1, 6, 6, -1},   {-1, 7, -1, -1},  {-1, 8, 7, -1},   {-1, 9, -1, -1},
    {-1, 10, -1, 3},  {-1, 11, -1, -1}, {-1, 12, -1, 4},  {-1, 13, -1, -1},
    {-1, 14, -1, 5},  {-1, 15, -1, -1}, {6, -1, -1, 6},   {7, -1, -1, -1},
    {8, -1, -1, 7},   {9, -1, -1, -1},  {10, -1, -1, -1}, {11, -1, -1, -1},
    {12, -1, -1, -1}, {13, -1, -1, -1}, {14, -1, -1, -1}, {15, -1, -1, -1},
};

// Tile hand-over at slot 26 of a tile's second iteration: by then this wave
// has read the tile's last V^T chunk, so after a barrier (with this wave's
// copies older than the last WAITK landed first; WAITK 63: no wait on
// copies) the tile's buffer may take another tile (COPY), whose eight copies
// are issued over slots 26-31. WAITK < 0: no hand-over.
constexpr int8_t kCopySlot[8] = {26, 26, 27, 28, 28, 29, 30, 31};

template <bool QK, bool SM, bool PREF, int WAITK = -1, bool COPY = false>
__device__ inline void iterate(Wave& W, const uint16_t* kq, int sq, const uint16_t* vp, int sp,
                               const uint16_t* vn, int sv, f32x16 (&sn)[2],
                               const f32x16 (&sc)[2], const bf16x8 (&pc)[2][2],
                               bf16x8 (&pn)[2][2], bf16x8 (&vpre)[3], float sl2e, int lane,
                               Tile fresh = Tile{}, const TileSrc* fsrc = nullptr,
                               int64_t krow = 0, int64_t ldv = 0, int wave = 0) {
  const f32x16 zero = {};
  bf16x8 av[8], ak[8];
  av[0] = vpre[0];
  av[1] = vpre[1];
  av[2] = vpre[2];
  bf16x2 pr[2][2][4];
  float lsum[2] = {W.l[0], W.l[1]};
  Unit x[16];
#pragma unroll
  for (int slot = 0; slot < 32; ++slot) {
    const Slot S = kSlots[slot];
    if (WAITK >= 0 && slot == 26) wait_tiles<(WAITK >= 0 ? WAITK : 0)>();
    if (COPY) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (kCopySlot[i] == slot) copy_part(fresh, *fsrc, krow, ldv, i, wave, lane);
    }
    if (QK && S.rk >= 0) ak[S.rk] = read_k(kq, sq, S.rk, lane);
    if (S.rv >= 0) av[S.rv] = read_v(vp, sp, S.rv, lane);
    if (PREF && slot >= 26 && (slot & 1) == 0)
      vpre[(slot - 26) / 2] = read_v(vn, sv, (slot - 26) / 2, lane);
    if (S.pv >= 0) {
      const int i = S.pv >> 1, qb = S.pv & 1;
      W.o[qb][i & 3] = mfma(av[i], pc[qb][i >> 2], W.o[qb][i & 3]);
    } else if (QK) {
      const int kk = S.qk >> 1, qb = S.qk & 1;
      sn[qb] = mfma(ak[kk], W.q[qb][kk], kk ? sn[qb] : zero);
    }
    if (SM) {
      const int v = slot >> 1;
      if ((slot & 1) == 0) {
        st_f0(sc, W, v, sl2e, x[v]);
        if (v >= 1) st_e1(x[v - 1]);
        if (v >= 2) st_d(x[v - 2], v - 2, lsum);
      } else {
        st_f1e0(sc, W, v, sl2e, x[v]);
        if (v >= 1) st_c(x[v - 1], v - 1, pr);
        if (slot == 31) {
          st_e1(x[15]);
          st_c(x[15], 15, pr);
          st_d(x[14], 14, lsum);
          st_d(x[15], 15, lsum);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (SM) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      pn[qb][0] = gather_p(pr[qb][0]);
      pn[qb][1] = gather_p(pr[qb][1]);
      W.l[qb] = lsum[qb];
    }
  }
}

// Where an attention pass's entries point: e / KH = row * Hs + (head - h0)
// over the pass's Hs query heads from h0; the Q (and O) row of that (row,
// head) is row * Hq + head.
struct PassHeads {
  int KH, Hq, Hs, h0;
};
__device__ inline int64_t entry_qrow(uint32_t e, const PassHeads& ph) {
  const uint32_t pr = e / (uint32_t)ph.KH;
  return (int64_t)pr + (int64_t)(pr / (uint32_t)ph.Hs) * (ph.Hq - ph.Hs) + ph.h0;
}

// The wave's Q rows (B operand of the scores): lane l holds the row of
// entry ev[qb] (query l % 32 of block qb), chunks 16 kk + 8 h; rows of
// invalid entries are zero.
__device__ inline void load_q(Wave& W, const uint16_t* __restrict__ Q, const uint32_t* ev,
                              const bool* valid, const PassHeads& ph, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const uint16_t* qrow = Q + entry_qrow(ev[qb], ph) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 u = valid[qb] ? *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * h)
                                : make_uint4(0, 0, 0, 0);
      W.q[qb][kk] = as_bf16x8(u);
    }
  }
}

// The whole block for one workgroup: keys [key0, key0 + B) of K and the
// matching V^T columns, B a multiple of 256, weights against W.m (set from
// the first subtile when set_m). Tile t sits in buffer t % 4; tile t+4 is
// copied right after the hand-over barrier in step t.
//   STREAM = false: tiles 0-3 are copied here first.
//   STREAM = true (persistent workgroups): on entry tiles 0-2 of this block
//     and the wave's Q rows have been requested by the caller (or by the
//     previous block's pass); tile 3 is copied here once every wave is past
//     the previous block. The last steps hand the freed buffers 0-2 to tiles
//     0-2 of the next block (nkbase, nvbase) and, once no score remains to
//     be made, request the next block's Q rows (entries nev, nvalid) into W.q.
template <bool STREAM>
__device__ inline void run_block(Wave& W, const uint16_t* __restrict__ kbase, int64_t krow,
                                 const uint16_t* __restrict__ vbase, int64_t ldv, int B,
                                 float sl2e, bool set_m, int wave, int lane, uint16_t* k0,
                                 uint16_t* k1, uint16_t* k2, uint16_t* k3, uint16_t* v0,
                                 uint16_t* v1, uint16_t* v2, uint16_t* v3,
                                 const uint16_t* __restrict__ nkbase = nullptr,
                                 const uint16_t* __restrict__ nvbase = nullptr,
                                 const uint16_t* __restrict__ Q = nullptr,
                                 const uint32_t* nev = nullptr, const bool* nvalid = nullptr,
                                 PassHeads ph = PassHeads{1, 1, 1, 0}) {
  const Tile T0{k0, v0}, T1{k1, v1}, T2{k2, v2}, T3{k3, v3};
  const int nt = B / KT;  // a multiple of 4
  auto src_of = [&](int t) {
    return tile_src(kbase + (int64_t)t * KT * krow, krow, vbase + (int64_t)t * KT, ldv);
  };
  auto nsrc_of = [&](int t) {
    return tile_src(nkbase + (int64_t)t * KT * krow, krow, nvbase + (int64_t)t * KT, ldv);
  };
  f32x16 sa[2], sb[2];
  bf16x8 pa[2][2], pb[2][2], vpre[3];
  if (STREAM) {
    wait_tiles<0>();  // tiles 0-2 and the Q rows; every wave is past the previous block
    load_tile(T3, src_of(3), krow, ldv, wave, lane);
  } else {
    const Tile T[4] = {T0, T1, T2, T3};
#pragma unroll
    for (int t = 0; t < 4; ++t) load_tile(T[t], src_of(t), krow, ldv, wave, lane);
    wait_tiles<kCopies * 4>();  // tiles 0 and 1
  }
  qk_plain(W, T0.k, 0, lane, sa);
  qk_plain(W, T0.k, 1, lane, sb);
  if (set_m) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float v = sa[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) v = fmaxf(v, sa[qb][r]);
      W.m[qb] = fmaxf(v, __shfl_xor(v, 32)) * sl2e;
    }
  }
  softmax_plain(W, sa, sl2e, pa);
#pragma unroll
  for (int i = 0; i < 3; ++i) vpre[i] = read_v(T0.v, 0, i, lane);
  // Step t: the output updates of subtiles 2t and 2t+1 (tile t), the scores
  // of tile t+1, the weights of subtiles 2t+1 and 2t+2. Tag: 0 while tile
  // t+4 exists (hand-over with its copies); 1 for t = nt-4 and 2 for t =
  // nt-3 (hand-over publishing tile t+2; STREAM: copies of the next block's
  // tile 0, 1); 3 for t = nt-2 (STREAM: hand-over with the copies of the
  // next block's tile 2); 4 for the final tile (no scores of a next tile;
  // STREAM: the next block's Q rows are requested first).
  auto step = [&](int t, Tile cur, Tile nxt, auto tag) {
    constexpr int TAG = decltype(tag)::value;
    if (TAG <= 3) {
      iterate<true, true, true>(W, nxt.k, 0, cur.v, 0, cur.v, 1, sa, sb, pa, pb, vpre, sl2e, lane);
      constexpr int WAITK = TAG <= 1 ? kCopies * 2 : TAG == 2 ? (STREAM ? kCopies * 2 : 0)
                                                              : (STREAM ? 63 : -1);
      constexpr bool COPY = TAG == 0 || STREAM;
      const TileSrc fs = TAG == 0 ? src_of(t + 4) : STREAM ? nsrc_of(TAG - 1) : src_of(0);
      iterate<true, true, true, WAITK, COPY>(W, nxt.k, 1, cur.v, 1, nxt.v, 0, sb, sa, pb, pa,
                                             vpre, sl2e, lane, cur, &fs, krow, ldv, wave);
    } else {
      if (STREAM) load_q(W, Q, nev, nvalid, ph, lane);
      iterate<false, true, true>(W, nxt.k, 0, cur.v, 0, cur.v, 1, sa, sb, pa, pb, vpre, sl2e, lane);
      iterate<false, false, false>(W, nxt.k, 1, cur.v, 1, nxt.v, 0, sb, sa, pb, pa, vpre, sl2e,
                                   lane);
    }
  };
  using L0 = std::integral_constant<int, 0>;
  int t = 0;
  for (; t + 4 < nt; t += 4) {
    step(t, T0, T1, L0{});
    step(t + 1, T1, T2, L0{});
    step(t + 2, T2, T3, L0{});
    step(t + 3, T3, T0, L0{});
  }
  // the last four tiles (t = nt - 4)
  step(t, T0, T1, std::integral_constant<int, 1>{});
  step(t + 1, T1, T2, std::integral_constant<int, 2>{});
  step(t + 2, T2, T3, std::integral_constant<int, 3>{});
  step(t + 3, T3, T0, std::integral_constant<int, 4>{});
  if (!STREAM) __syncthreads();  // every wave is done with the buffers before they are reused
}

// Score-only pass for the rare re-run: the largest score of each query over
// the block (lane-local half), tiles copied one at a time into T0.
__device__ inline void block_max(const Wave& W, const uint16_t* __restrict__ kbase, int64_t krow,
                                 const uint16_t* __restrict__ vbase, int64_t ldv, int B, int wave,
                                 int lane, uint16_t* k0, uint16_t* v0, float (&mx)[2]) {
  const Tile T0{k0, v0};
  for (int t = 0; t < B / KT; ++t) {
    load_tile(T0, tile_src(kbase + (int64_t)t * KT * krow, krow, vbase + (int64_t)t * KT, ldv),
              krow, ldv, wave, lane);
    wait_tiles<0>();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 s[2];
      qk_plain(W, T0.k, sub, lane, s);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx[qb] = fmaxf(mx[qb], s[qb][r]);
    }
    __syncthreads();
  }
}

}  // namespace

// ----------------------------------------------------------------------------
// History attention. A history tile is up to 256 routed entries of one bin
// (KV head g, history block j): the entries [e_begin, e_end) of the bin's
// list, attended over the whole block.
// ----------------------------------------------------------------------------
struct HistTile {
  int64_t e_begin, e_end;
  const uint16_t* kbase;  // K rows of block j, KV head g
  const uint16_t* vbase;  // V^T columns of block j, KV head g
};

__device__ inline HistTile hist_tile(int64_t w, const uint16_t* __restrict__ K,
                                     const uint16_t* __restrict__ Vt,
                                     const int32_t* __restrict__ bstart,
                                     const int32_t* __restrict__ tile_map,
                                     const int32_t* __restrict__ tile_off,
                                     const int32_t* __restrict__ bin_off, int Hkv, int64_t Bpad,
                                     int64_t ldv, int64_t nh) {
  HistTile t;
  const int bin = tile_map[w];
  t.e_begin = bin_off[bin] + (w - tile_off[bin]) * (int64_t)kTileQ;
  t.e_end = bin_off[bin + 1];
  const int g = (int)(bin / nh);
  const int64_t j = bin % nh;
  t.kbase = K + (bstart[j] * (int64_t)Hkv + g) * kHeadDim;  // history blocks are full
  t.vbase = Vt + (int64_t)g * kHeadDim * ldv + j * Bpad;
  return t;
}

// The two entries of this lane (query l % 32 of each 32-query block of its
// wave) and whether they exist.
__device__ inline void tile_entries(const HistTile& t, const uint32_t* __restrict__ entries,
                                    int wave, int lane, uint32_t (&ev)[2], bool (&valid)[2]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t e = t.e_begin + wave * kWaveQ + qb * 32 + (lane & 31);
    valid[qb] = e < t.e_end;
    ev[qb] = valid[qb] ? entries[e] : 0u;
  }
}

__device__ inline void reset_acc(Wave& W) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) W.o[qb][db][r] = 0.f;
  W.l[0] = W.l[1] = 0.f;
}

// Normalised partial outputs (fp16) and log2-sum-exps of the valid entries.
__device__ inline void store_partials(const Wave& W, const uint32_t (&ev)[2],
                                      const bool (&valid)[2], _Float16* __restrict__ part_o,
                                      float* __restrict__ part_lse, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
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

// True when some valid query's row sum reached 2^64 (or is not finite): its
// weights, taken against the first subtile's maximum, may have overflowed.
__device__ inline bool wave_overflow(const Wave& W, const bool (&valid)[2]) {
  bool r = false;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) r |= valid[qb] && !(W.l[qb] < kLMax);
  return r;
}

// Persistent workgroups, one per compute unit: workgroup i runs on XCD i % 8
// and each XCD walks a contiguous range of history tiles, its 32 workgroups
// taking every 32nd tile, so the tiles in flight on an XCD share the K/V
// blocks in its L2. While a tile's last steps run, the next tile's first
// three K/V tiles and its Q rows are already being fetched. A tile whose
// weights could have overflowed is appended to redo_list (counter
// scalars[2]) and recomputed by attn_hist_q64_redo_bf16.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void
attn_hist_q64_bf16(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ Vt, const int32_t* __restrict__ bstart,
                   const int32_t* __restrict__ tile_map, const int32_t* __restrict__ tile_off,
                   const int32_t* __restrict__ bin_off, int32_t* __restrict__ scalars,
                   const uint32_t* __restrict__ entries, _Float16* __restrict__ part_o,
                   float* __restrict__ part_lse, int32_t* __restrict__ redo_list, int Hkv, int B,
                   int64_t Bpad, int64_t ldv, int64_t nh, float sl2e, PassHeads ph, int64_t bin0,
                   int64_t bin1) {
  __shared__ __align__(16) uint16_t lds_k0[KS_ELEMS], lds_k1[KS_ELEMS], lds_k2[KS_ELEMS],
      lds_k3[KS_ELEMS];
  __shared__ __align__(16) uint16_t lds_v0[VT_ELEMS], lds_v1[VT_ELEMS], lds_v2[VT_ELEMS],
      lds_v3[VT_ELEMS];
  // this attention pass's tiles: those of its bins [bin0, bin1)
  const int64_t first = tile_off[bin0];
  const int64_t total = tile_off[bin1] - first;
  const int64_t nloc = gridDim.x / 8;  // workgroups per XCD (the grid is a multiple of 8)
  const int64_t per = (total + 7) / 8;
  const int64_t lo = first + (blockIdx.x % 8) * per;
  const int64_t hi = lo + per < first + total ? lo + per : first + total;
  int64_t w = lo + blockIdx.x / 8;
  if (w >= hi) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t krow = (int64_t)Hkv * kHeadDim;
  auto tile_of = [&](int64_t x) {
    return hist_tile(x, K, Vt, bstart, tile_map, tile_off, bin_off, Hkv, Bpad, ldv, nh);
  };
  HistTile cur = tile_of(w);
  uint32_t ev[2];
  bool valid[2];
  tile_entries(cur, entries, wave, lane, ev, valid);
  Wave W;
  load_q(W, Q, ev, valid, ph, lane);
  load_tile(Tile{lds_k0, lds_v0}, tile_src(cur.kbase, krow, cur.vbase, ldv), krow, ldv, wave, lane);
  load_tile(Tile{lds_k1, lds_v1},
            tile_src(cur.kbase + KT * krow, krow, cur.vbase + KT, ldv), krow, ldv, wave, lane);
  load_tile(Tile{lds_k2, lds_v2},
            tile_src(cur.kbase + 2 * KT * krow, krow, cur.vbase + 2 * KT, ldv), krow, ldv, wave,
            lane);
  for (;;) {
    const int64_t wn = w + nloc;
    const bool has_next = wn < hi;
    // without a next tile the last steps re-request this tile's first K/V
    // tiles and Q rows (unused), which keeps them free of branches
    const HistTile nxt = has_next ? tile_of(wn) : cur;
    uint32_t evn[2];
    bool validn[2];
    tile_entries(nxt, entries, wave, lane, evn, validn);
    reset_acc(W);
    run_block<true>(W, cur.kbase, krow, cur.vbase, ldv, B, sl2e, true, wave, lane, lds_k0, lds_k1,
                    lds_k2, lds_k3, lds_v0, lds_v1, lds_v2, lds_v3, nxt.kbase, nxt.vbase, Q, evn,
                    validn, ph);
    // workgroup-uniform, so each tile is listed at most once
    if (__syncthreads_or(wave_overflow(W, valid)) && tid == 0)
      redo_list[atomicAdd(&scalars[2], 1)] = (int32_t)w;
    store_partials(W, ev, valid, part_o, part_lse, lane);
    if (!has_next) break;
    w = wn;
    cur = nxt;
    ev[0] = evn[0];
    ev[1] = evn[1];
    valid[0] = validn[0];
    valid[1] = validn[1];
  }
  __builtin_amdgcn_s_waitcnt(0);  // the last re-requested copies land before the LDS is released
}

// Recomputation of the tiles the persistent kernel listed: a score-only
// pass finds each query's true maximum and the block is redone from it
// (weights <= 1). Normally the list is empty and every workgroup returns at
// once.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void
attn_hist_q64_redo_bf16(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ Vt, const int32_t* __restrict__ bstart,
                        const int32_t* __restrict__ tile_map,
                        const int32_t* __restrict__ tile_off,
                        const int32_t* __restrict__ bin_off, const int32_t* __restrict__ scalars,
                        const uint32_t* __restrict__ entries, _Float16* __restrict__ part_o,
                        float* __restrict__ part_lse, const int32_t* __restrict__ redo_list,
                        int Hkv, int B, int64_t Bpad, int64_t ldv, int64_t nh, float sl2e,
                        PassHeads ph) {
  __shared__ __align__(16) uint16_t lds_k0[KS_ELEMS], lds_k1[KS_ELEMS], lds_k2[KS_ELEMS],
      lds_k3[KS_ELEMS];
  __shared__ __align__(16) uint16_t lds_v0[VT_ELEMS], lds_v1[VT_ELEMS], lds_v2[VT_ELEMS],
      lds_v3[VT_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t krow = (int64_t)Hkv * kHeadDim;
  const int64_t count = scalars[2];
  for (int64_t i = blockIdx.x; i < count; i += gridDim.x) {
    const HistTile cur =
        hist_tile(redo_list[i], K, Vt, bstart, tile_map, tile_off, bin_off, Hkv, Bpad, ldv, nh);
    uint32_t ev[2];
    bool valid[2];
    tile_entries(cur, entries, wave, lane, ev, valid);
    Wave W;
    load_q(W, Q, ev, valid, ph, lane);
    float mx[2] = {-INFINITY, -INFINITY};
    block_max(W, cur.kbase, krow, cur.vbase, ldv, B, wave, lane, lds_k0, lds_v0, mx);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) W.m[qb] = fmaxf(mx[qb], __shfl_xor(mx[qb], 32)) * sl2e;
    reset_acc(W);
    run_block<false>(W, cur.kbase, krow, cur.vbase, ldv, B, sl2e, false, wave, lane, lds_k0,
                     lds_k1, lds_k2, lds_k3, lds_v0, lds_v1, lds_v2, lds_v3);
    store_partials(W, ev, valid, part_o, part_lse, lane);
  }
}

bool attn_hist_q64_supported(const Prob& P) { return P.B % 256 == 0; }

hipError_t launch_attn_hist_q64_bf16(const Prob& P, const Blocks& T, const BucketPlan& bp,
                                     const void* Q, const void* K, const void* Vt,
                                     const BucketBufs& b, void* part_o, float* part_lse,
                                     hipStream_t s) {
  if (P.nh <= 0 || P.KH <= 0 || bp.max_tiles <= 0) return hipSuccess;
  const float sl2e = P.scale * kLog2e;
  const int64_t Bpad = vt_padded_block(P.B);
  const int64_t ldv = P.vt_blocks * Bpad;
  const PassHeads ph{P.KH, P.Hq, pass_heads(P), pass_h0(P)};
  // one workgroup per compute unit (256 on MI355X), fewer for small problems
  const int64_t grid = std::min<int64_t>(256, ceil_div(pass_max_tiles(P), 8) * 8);
  // the redo list starts empty in every attention pass (the bucketing clears
  // it for the first)
  if (P.g0 > 0) {
    hipError_t e = launch_fill_i32(b.scalars + 2, 0, 1, s);
    if (e != hipSuccess) return e;
  }
  attn_hist_q64_bf16<<<(unsigned)grid, kThreads, 0, s>>>(
      (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)Vt, T.start, b.tile_map,
      b.tile_off, b.bin_off, b.scalars, b.entries, (_Float16*)part_o, part_lse, b.redo, P.Hkv,
      P.B, Bpad, ldv, P.nh, sl2e, ph, (int64_t)P.g0 * P.nh, (int64_t)(P.g0 + P.gs) * P.nh);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_hist_q64_redo_bf16<<<64, kThreads, 0, s>>>(
      (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)Vt, T.start, b.tile_map,
      b.tile_off, b.bin_off, b.scalars, b.entries, (_Float16*)part_o, part_lse, b.redo, P.Hkv,
      P.B, Bpad, ldv, P.nh, sl2e, ph);
  return hipGetLastError();
}

}  // namespace moba
