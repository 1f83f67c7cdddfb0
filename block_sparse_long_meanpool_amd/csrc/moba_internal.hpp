// Internal declarations shared by the kernels and the host runtime of libmoba.so.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include <cstddef>
#include <cstdint>

#include "moba.h"

namespace moba {

constexpr int kHeadDim = 128;       // head_dim compiled in
constexpr int kMaxTopk = 32;        // topk limit (selection lists live in LDS)
constexpr int64_t kMaxHist = 8192;  // history-capable blocks (bucket bitmaps live in LDS)
constexpr int kTileQ = 256;         // routed queries per history-attention tile
constexpr int kMaxGroup = 64;       // Hq / Hkv limit

// Problem with derived sizes; built and validated on the host. The rows are
// one sequence or several packed ones; blocks are numbered globally, each
// sequence's blocks consecutively from its first row, and only blocks of a
// row's own sequence are candidates for it.
struct Prob {
  int64_t N;          // key rows (all sequences)
  int64_t Nq;         // query rows: the last Nq positions of the sequence (= N unless a chunk)
  int64_t q0;         // position of query row 0 (= N - Nq)
  int Hq, Hkv, G, d, B, k;
  int KH;             // history slots per (row, head) = k - 1
  int64_t nseq;       // sequences
  int64_t n;          // blocks over all sequences (a sequence's last one may be partial)
  int64_t nh;         // blocks that can be history anywhere = n - 1
  int64_t hist_rows;  // sum over query rows of min(k - 1, earlier blocks of the row's sequence)
  float scale;
  int dtype;          // MOBA_DTYPE_*
  int routing;        // MOBA_ROUTING_*
  int64_t vt_blocks;  // blocks of the packed V^T layout read by the bf16 kernels (n, or a
                      // decode cache's capacity in blocks)
  int kvpp;           // KV heads per attention pass (1..Hkv)
  int g0, gs;         // this attention pass: KV heads [g0, g0 + gs) (whole problem: 0, Hkv)
};

// History partial results are indexed per attention pass: the history slot s
// of (row r, query head h) of the pass holding h is
//   ((r * Hs + (h - h0)) * KH + s),  h0 = g0 * G, Hs = gs * G,
// for the pass of h's KV head. These give a pass's h0 and Hs.
inline int pass_h0(const Prob& P) { return P.g0 * P.G; }
inline int pass_heads(const Prob& P) { return P.gs * P.G; }
// Bound on the history tiles of an attention pass (its bins' lists in
// tiles of kTileQ entries).
inline int64_t pass_max_tiles(const Prob& P) {
  const int64_t entries = P.hist_rows * (int64_t)pass_heads(P);
  return (entries + kTileQ - 1) / kTileQ + (int64_t)P.gs * P.nh;
}

// Block and row tables in device memory (built by launch_tables):
//   start[b], len[b]: first key row and key count of global block b (len <= B);
//   lo[b]: first block of b's sequence, so b's rows may select [lo[b], b);
//   qstart[b], qlen[b], qpos[b]: first query row, query row count and the
//     position of that first query row inside block b (qlen may be 0);
//   row_blk[r]: global block of query row r.
// For a full prefill query rows are key rows: qstart = qpos = start, qlen = len.
struct Blocks {
  int32_t* start;
  int32_t* len;
  int32_t* lo;
  int32_t* qstart;
  int32_t* qlen;
  int32_t* qpos;
  int32_t* row_blk;
  int32_t* seq_base;  // [nseq + 1] first block of each sequence (scratch of the build)
};

// Fill the tables; cu = device row offsets [nseq + 1] of packed sequences, or
// NULL for one sequence of P.N rows.
hipError_t launch_tables(const Prob& P, const int64_t* cu, const Blocks& t, hipStream_t s);

// Bucketing (per KV head, history block) of the selected (row, head, slot) entries.
struct BucketPlan {
  int rows_per_chunk;  // rows of one KV head group per counting chunk
  int64_t nchunk;      // chunks per KV head = ceil(N / rows_per_chunk)
  int words;           // 32-bit bitmap words per bin in a chunk
  int ws;              // their row stride in LDS (odd where it fits)
  int64_t nbins;       // Hkv * nh
  int64_t max_entries; // Hq * sum_p min(k-1, c(p))
  int64_t max_tiles;   // bound on sum_b ceil(count_b / kTileQ)
};

struct BucketBufs {
  int32_t* chunk_base;  // [Hkv][nchunk][nh] counts, then exclusive bases
  int32_t* bin_total;   // [nbins]
  int32_t* bin_off;     // [nbins + 1]
  int32_t* tile_off;    // [nbins + 1]
  int32_t* tile_map;    // [max_tiles]
  int32_t* scalars;     // [4]: total entries, total tiles, tiles listed in redo, unused
  uint32_t* entries;    // [max_entries]
  int32_t* redo;        // [max_tiles] history tiles to recompute (bf16 history attention)
};

BucketPlan plan_bucket(const Prob& P);

// Stage launchers (each enqueues on `s`; return hipSuccess or the launch error).
hipError_t launch_meanpool(const Prob& P, const Blocks& T, const void* K, double* kbar,
                           double* part, int splits, hipStream_t s);
int meanpool_splits(const Prob& P);

// Gate + selection; `scratch` holds the bf16 split of the block keys and their
// norms (gate_scratch_bytes).
size_t gate_scratch_bytes(const Prob& P);
hipError_t launch_gate_topk(const Prob& P, const Blocks& T, const void* Q, const double* kbar,
                            void* scratch, int32_t* sel, hipStream_t s);
// The exact tier for every row, also writing each row's selection margin
// (last kept minus best left-out history score; NaN when nothing is left out).
hipError_t launch_gate_margin(const Prob& P, const Blocks& T, const void* Q, const double* kbar,
                              void* scratch, int32_t* sel, float* margin, hipStream_t s);
// Per-(KV head, block) history selection counts [Hkv][n] and per-(row, KV
// head) sizes of the union of the group's history selections [N][Hkv]
// (either output may be NULL).
hipError_t launch_routing_reductions(const Prob& P, const Blocks& T, const int32_t* sel,
                                     int32_t* counts, int32_t* union_size, hipStream_t s);

hipError_t launch_bucket(const Prob& P, const Blocks& T, const BucketPlan& bp, const int32_t* sel,
                         const BucketBufs& b, hipStream_t s);

// bf16 kernels read V through a transposed, block-padded, key-permuted copy
// Vt [Hkv][d][n * Bpad] (see vpack.hip); fp32 kernels read V directly.
// Vt rows are P.vt_blocks * Bpad long.
int64_t vt_padded_block(int64_t B);
hipError_t launch_vt_pack(const Prob& P, const Blocks& T, const void* V, void* Vt, hipStream_t s);
// Pack only the 64-key tiles holding rows [r0, r1) of one sequence of P.N rows
// (no tables needed: block c starts at c * B).
hipError_t launch_vt_pack_rows(const Prob& P, const void* V, void* Vt, int64_t r0, int64_t r1,
                               hipStream_t s);

// Decode cache (cache.hip): fp64 means of the full blocks c0 .. c0 + count - 1
// of one sequence into kbar [Hkv][nhc][d]; and the copy of the first nh
// blocks' means from that layout into the [Hkv][nh][d] layout the gate reads.
hipError_t launch_cache_means(const Prob& P, const void* K, int64_t c0, int64_t count,
                              double* kbar, int64_t nhc, hipStream_t s);
hipError_t launch_kbar_gather(const double* src, int64_t nhc, double* dst, int64_t nh, int Hkv,
                              int d, hipStream_t s);

// bf16 history attention kernels: the 64-query-per-wave engine
// (attn_hist_bf16.hip) for block sizes that are multiples of 256, the
// 32-query engine (attn_bf16.hip) otherwise.
bool attn_hist_q64_supported(const Prob& P);
hipError_t launch_attn_hist_q64_bf16(const Prob& P, const Blocks& T, const BucketPlan& bp,
                                     const void* Q, const void* K, const void* Vt,
                                     const BucketBufs& b, void* part_o, float* part_lse,
                                     hipStream_t s);
hipError_t launch_attn_hist_bf16(const Prob& P, const Blocks& T, const BucketPlan& bp,
                                 const void* Q, const void* K, const void* Vt,
                                 const BucketBufs& b, void* part_o, float* part_lse,
                                 hipStream_t s);

// History-block attention over the bucketed entries; writes normalised partials
// part_o [entry][d] and log2-sum-exp part_lse [entry].
hipError_t launch_attn_hist(const Prob& P, const Blocks& T, const BucketPlan& bp, const void* Q,
                            const void* K, const void* V, const void* Vt, const BucketBufs& b,
                            void* part_o, float* part_lse, hipStream_t s);

// Own-block causal attention fused with the merge of the history partials
// (part_o == NULL: no partials, e.g. the dense baseline, whose problem is one
// block spanning the sequence). lse_out (nullable) [Nq][Hq] receives each
// row's log2-sum-exp: P_j = 2^(scale log2(e) q.k_j - lse) over its keys.
hipError_t launch_attn_self(const Prob& P, const Blocks& T, const void* Q, const void* K,
                            const void* V, const void* Vt, const void* part_o,
                            const float* part_lse, void* O, float* lse_out, hipStream_t s);

// Backward with the selection held fixed: dq [Nq][Hq][d], dk and dv
// [N][Hkv][d] in the input dtype from o, lse2 (the forward's lse_out) and
// dout; bp/bb must hold the bucketed selection of the same problem. Scratch:
// delta [Nq][Hq] fp32 always; fp32 inputs (vector kernels, bwd.hip) use
// dq_acc [Nq][Hq][d] fp32; bf16 inputs (matrix-core kernels, bwd_bf16.hip)
// use kt (vt_pack layout of K) and part_dq [Nq][Hq][k-1][d] fp32.
struct BwdScratch {
  float* delta;
  float* dq_acc;
  void* kt;
  float* part_dq;
};
hipError_t launch_backward(const Prob& P, const Blocks& T, const BucketPlan& bp,
                           const BucketBufs& bb, const void* q, const void* k, const void* v,
                           const void* o, const float* lse2, const void* dout, void* dq, void* dk,
                           void* dv, const BwdScratch& w, hipStream_t s);
hipError_t launch_backward_bf16(const Prob& P, const Blocks& T, const BucketPlan& bp,
                                const BucketBufs& bb, const void* q, const void* k, const void* v,
                                const float* lse2, const void* dout, const float* delta,
                                void* kt, float* part_dq, void* dq, void* dk, void* dv,
                                hipStream_t s);

// Few query rows (decode steps, small chunks): split-K attention over each
// row's selected blocks read in place, then the merge (decode.hip). Used
// instead of bucketing + the tiled kernels when Nq <= kDecodeRows; part holds
// decode_part_bytes(P); lse_out (nullable) as for launch_attn_self.
constexpr int64_t kDecodeRows = 16;
int decode_splits(const Prob& P);
size_t decode_part_bytes(const Prob& P);
hipError_t launch_decode(const Prob& P, const Blocks& T, const void* q, const void* k,
                         const void* v, const int32_t* sel, float* part, void* o, float* lse_out,
                         hipStream_t s);

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t count, hipStream_t s);
hipError_t launch_mfma_probe(int workgroups, int iters, float* out, hipStream_t s);
hipError_t launch_read_probe(const void* src, size_t bytes, int workgroups, uint32_t* out,
                             hipStream_t s);

// Element type of the partial outputs of history attention.
inline size_t part_elem_bytes(const Prob& P) { return P.dtype == MOBA_DTYPE_F32 ? 4 : 2; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Blocks holding query rows, counted from the last: a chunk of one sequence
// has its rows in the blocks from q0 / B on; otherwise every block.
inline int64_t query_blocks(const Prob& P) { return P.nseq == 1 ? P.n - P.q0 / P.B : P.n; }

}  // namespace moba
