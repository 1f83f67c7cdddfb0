// moba_bucket — invert (query, block) selections into per-KV-block query lists
// (PaperTrace "2.1.3 MoBA", section 3.1 step 3: queries are regrouped by the
// KV block they read so that one contiguous K/V block serves a batch of
// queries; section 5.4 on the sort / prefix-sum / reorder this costs).
//
// Bins are (KV head g, history block b). An entry is the index of the
// query's history slot among the partial results of its attention pass (the
// group of kvpp KV heads holding g, query heads h0 .. h0 + Hs - 1):
// e = (row * Hs + head - h0) * (k - 1) + slot, which is where history
// attention writes that query's partial result (one pass of all heads:
// e = (row * Hq + head) * (k - 1) + slot). The lists come out ordered by
// (row, head) within each bin, independently of scheduling:
//   1. count:   per chunk of rows (one KV-head group) an LDS histogram;
//   2. scan:    exclusive scan of the counts down the chunks of every bin,
//               then over bins -> bin offsets and history-tile offsets;
//   3. scatter: per chunk, an LDS bitmap per bin over the chunk's pairs gives
//               each entry its rank by popcount; entries land at
//               bin offset + chunk base + rank;
//   4. tile map: tile index -> bin, for the history-attention grid.
#include "moba_internal.hpp"

namespace moba {
namespace {

constexpr int kThreads = 256;
// Count and scatter: 8 waves per workgroup, so with two workgroups' bitmaps
// in a compute unit's LDS 16 waves keep its selection-row loads in flight
// (4 waves per workgroup: 3.46 ms for the stage at the 1M-token layer, 8:
// 3.27 ms, 16: 3.73 ms).
constexpr int kRowThreads = 512;
constexpr int kScanRowGroups = 16;

// Valid history entry of a selection row of block c: a block b < c at slot
// s < k-1 (the row's own block, always its largest, and -1 pads are not).
__device__ inline bool hist_entry(int32_t b, int64_t c) { return b >= 0 && b < c; }

// The KH history slots of one selection row into registers, every load
// issued before any value is used (one memory latency per row, not KH).
__device__ inline void load_row(const int32_t* __restrict__ row, int KH,
                                int32_t (&bs)[kMaxTopk]) {
#pragma unroll
  for (int s = 0; s < kMaxTopk; ++s) bs[s] = s < KH ? row[s] : -1;
}

// Chunk of rows and KV head of workgroup w (1-D grid of ceil(nchunk / 8) * 8
// * Hkv). Workgroup w runs on XCD w % 8; in each run of 8 * Hkv workgroups
// XCD x takes the Hkv heads of chunk 8 * run + x, so the workgroups that
// read the same selection rows (each its head group's part of every row)
// share one L2 and fetch each cache line of those rows from memory once.
__device__ inline bool chunk_of(int64_t w, int Hkv, int64_t nchunk, int64_t& chunk, int& g) {
  const int64_t run = w / (8 * Hkv), in = w % (8 * Hkv);
  g = (int)(in / 8);
  chunk = run * 8 + in % 8;
  return chunk < nchunk;
}

__global__ __launch_bounds__(kRowThreads) void bucket_count(const int32_t* __restrict__ sel,
                                                         const int32_t* __restrict__ row_blk,
                                                         int32_t* __restrict__ chunk_base,
                                                         int64_t N, int Hq, int G, int k,
                                                         int64_t nh, int rows_per_chunk,
                                                         int64_t nchunk, int Hkv) {
  extern __shared__ int32_t hist[];
  int g;
  int64_t chunk;
  if (!chunk_of(blockIdx.x, Hkv, nchunk, chunk, g)) return;
  for (int64_t b = threadIdx.x; b < nh; b += kRowThreads) hist[b] = 0;
  __syncthreads();
  const int KH = k - 1;
  const int npairs = rows_per_chunk * G;
  for (int pi = threadIdx.x; pi < npairs; pi += kRowThreads) {
    const int64_t r = chunk * rows_per_chunk + pi / G;
    if (r >= N) break;
    const int h = g * G + pi % G;
    const int64_t c = row_blk[r];
    int32_t bs[kMaxTopk];
    load_row(sel + ((size_t)r * Hq + h) * k, KH, bs);
#pragma unroll
    for (int s = 0; s < kMaxTopk; ++s)
      if (s < KH && hist_entry(bs[s], c)) atomicAdd(&hist[bs[s]], 1);
  }
  __syncthreads();
  int32_t* out = chunk_base + ((size_t)g * nchunk + chunk) * nh;
  for (int64_t b = threadIdx.x; b < nh; b += kRowThreads) out[b] = hist[b];
}

// Column-wise exclusive scan of chunk_base over chunks; 16 columns per
// workgroup, each column split into 16 contiguous chunk ranges.
__global__ __launch_bounds__(kThreads) void bucket_scan_cols(int32_t* __restrict__ chunk_base,
                                                             int32_t* __restrict__ bin_total,
                                                             int64_t nbins, int64_t nh,
                                                             int64_t nchunk) {
  __shared__ int32_t part[kScanRowGroups][16];
  const int cl = threadIdx.x % 16;
  const int rg = threadIdx.x / 16;
  const int64_t col = blockIdx.x * 16LL + cl;
  const bool ok = col < nbins;
  const int64_t g = ok ? col / nh : 0, b = ok ? col % nh : 0;
  const int64_t cs = (nchunk + kScanRowGroups - 1) / kScanRowGroups;
  const int64_t c0 = rg * cs;
  const int64_t c1 = (c0 + cs < nchunk) ? c0 + cs : nchunk;
  int32_t* base = chunk_base + (size_t)g * nchunk * nh + b;
  int32_t sum = 0;
  if (ok)
    for (int64_t ch = c0; ch < c1; ++ch) sum += base[(size_t)ch * nh];
  part[rg][cl] = sum;
  __syncthreads();
  int32_t run = 0;
  for (int q = 0; q < rg; ++q) run += part[q][cl];
  if (ok && rg == kScanRowGroups - 1) bin_total[col] = run + sum;
  if (ok)
    for (int64_t ch = c0; ch < c1; ++ch) {
      const int32_t v = base[(size_t)ch * nh];
      base[(size_t)ch * nh] = run;
      run += v;
    }
}

// Exclusive scans over bins: entry offsets and history-tile offsets.
__global__ __launch_bounds__(1024) void bucket_scan_bins(const int32_t* __restrict__ bin_total,
                                                         int32_t* __restrict__ bin_off,
                                                         int32_t* __restrict__ tile_off,
                                                         int32_t* __restrict__ scalars,
                                                         int64_t nbins, int tile_q) {
  __shared__ int32_t se[1024];
  __shared__ int32_t st[1024];
  __shared__ int32_t carry[2];
  const int t = threadIdx.x;
  if (t == 0) carry[0] = carry[1] = 0;
  __syncthreads();
  for (int64_t base = 0; base < nbins; base += 1024) {
    const int64_t i = base + t;
    const int32_t v = i < nbins ? bin_total[i] : 0;
    const int32_t tv = (v + tile_q - 1) / tile_q;
    se[t] = v;
    st[t] = tv;
    __syncthreads();
    // Hillis-Steele inclusive scan
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t a = t >= off ? se[t - off] : 0;
      const int32_t b = t >= off ? st[t - off] : 0;
      __syncthreads();
      se[t] += a;
      st[t] += b;
      __syncthreads();
    }
    if (i < nbins) {
      bin_off[i] = carry[0] + se[t] - v;
      tile_off[i] = carry[1] + st[t] - tv;
    }
    __syncthreads();
    if (t == 1023) {
      carry[0] += se[1023];
      carry[1] += st[1023];
    }
    __syncthreads();
  }
  if (t == 0) {
    bin_off[nbins] = carry[0];
    tile_off[nbins] = carry[1];
    scalars[0] = carry[0];
    scalars[1] = carry[1];
    scalars[2] = 0;  // history tiles listed for recomputation
    scalars[3] = 0;
  }
}

__global__ __launch_bounds__(kRowThreads) void bucket_scatter(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ row_blk,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ bin_off,
    uint32_t* __restrict__ entries, int64_t N, int Hq, int Hkv, int G, int k, int64_t nh,
    int rows_per_chunk, int64_t nchunk, int words, int ws, int kvpp) {
  // [nh][ws] bitmaps, then [nh][ws] prefix counts. The row stride ws is odd
  // where that fits (it spreads the words of different bins over the banks:
  // with stride 32 the 64 lanes of one slot's atomics, each at a random bin
  // but one of two words, land on at most four banks).
  extern __shared__ uint32_t bm[];
  int g;
  int64_t chunk;
  if (!chunk_of(blockIdx.x, Hkv, nchunk, chunk, g)) return;
  // the attention pass of KV head g: query heads [h0, h0 + Hs)
  const int g0 = (g / kvpp) * kvpp;
  const int h0 = g0 * G;
  const int64_t Hs = (int64_t)(Hkv - g0 < kvpp ? Hkv - g0 : kvpp) * G;
  const int64_t nw = nh * ws;
  uint32_t* pre = bm + nw;  // pre[b][w] = where the entries of bin b in word w start
  for (int64_t i = threadIdx.x; i < nw; i += kRowThreads) bm[i] = 0u;
  __syncthreads();
  const int KH = k - 1;
  const int npairs = rows_per_chunk * G;
  for (int pi = threadIdx.x; pi < npairs; pi += kRowThreads) {
    const int64_t r = chunk * rows_per_chunk + pi / G;
    if (r >= N) break;
    const int h = g * G + pi % G;
    const int64_t c = row_blk[r];
    int32_t bs[kMaxTopk];
    load_row(sel + ((size_t)r * Hq + h) * k, KH, bs);
#pragma unroll
    for (int s = 0; s < kMaxTopk; ++s)
      if (s < KH && hist_entry(bs[s], c))
        atomicOr(&bm[(size_t)bs[s] * ws + (pi >> 5)], 1u << (pi & 31));
  }
  __syncthreads();
  const int32_t* cb = chunk_base + ((size_t)g * nchunk + chunk) * nh;
  const int32_t* bo = bin_off + (size_t)g * nh;
  for (int64_t b = threadIdx.x; b < nh; b += kRowThreads) {
    uint32_t run = (uint32_t)(bo[b] + cb[b]);  // the chunk's first entry of bin b
    for (int w = 0; w < words; ++w) {
      pre[b * ws + w] = run;
      run += __popc(bm[b * ws + w]);
    }
  }
  __syncthreads();
  for (int pi = threadIdx.x; pi < npairs; pi += kRowThreads) {
    const int64_t r = chunk * rows_per_chunk + pi / G;
    if (r >= N) break;
    const int h = g * G + pi % G;
    const int64_t c = row_blk[r];
    int32_t bs[kMaxTopk];
    load_row(sel + ((int64_t)r * Hq + h) * k, KH, bs);
    const int64_t pslot = ((int64_t)r * Hs + (h - h0)) * KH;
#pragma unroll
    for (int s = 0; s < kMaxTopk; ++s) {
      const int32_t b = bs[s];
      if (s >= KH || !hist_entry(b, c)) continue;
      const size_t wi = (size_t)b * ws + (pi >> 5);
      const uint32_t at = pre[wi] + __popc(bm[wi] & ((1u << (pi & 31)) - 1u));
      entries[at] = (uint32_t)(pslot + s);
    }
  }
}

__global__ __launch_bounds__(kThreads) void bucket_tile_map(const int32_t* __restrict__ tile_off,
                                                            int32_t* __restrict__ tile_map) {
  const int64_t b = blockIdx.x;
  const int32_t t0 = tile_off[b], t1 = tile_off[b + 1];
  for (int32_t t = t0 + threadIdx.x; t < t1; t += kThreads) tile_map[t] = (int32_t)b;
}

}  // namespace

BucketPlan plan_bucket(const Prob& P) {
  BucketPlan bp{};
  const int64_t nh = P.nh > 0 ? P.nh : 1;
  int64_t wmax = 8192 / nh - 1;  // room for a padded stride (at least one word)
  if (wmax > 32) wmax = 32;
  if (wmax < 1) wmax = 1;
  int64_t rpc = (32 * wmax) / P.G;
  if (rpc < 1) rpc = 1;
  bp.rows_per_chunk = (int)rpc;
  bp.words = (int)ceil_div(rpc * P.G, 32);
  // an odd bitmap stride (padded by one word when even) while the two
  // arrays stay within 64 KB
  bp.ws = nh * (bp.words | 1) <= 8192 ? (bp.words | 1) : bp.words;
  bp.nchunk = ceil_div(P.Nq, rpc);
  bp.nbins = (int64_t)P.Hkv * P.nh;
  bp.max_entries = P.hist_rows * P.Hq;
  bp.max_tiles = ceil_div(bp.max_entries, kTileQ) + bp.nbins;
  return bp;
}

hipError_t launch_bucket(const Prob& P, const Blocks& T, const BucketPlan& bp, const int32_t* sel,
                         const BucketBufs& b, hipStream_t s) {
  if (P.nh <= 0 || P.KH <= 0) {
    // No history anywhere: empty lists.
    hipError_t e = launch_fill_i32(b.bin_off, 0, bp.nbins + 1, s);
    if (e == hipSuccess) e = launch_fill_i32(b.tile_off, 0, bp.nbins + 1, s);
    if (e == hipSuccess) e = launch_fill_i32(b.scalars, 0, 4, s);
    return e;
  }
  const unsigned grid = (unsigned)(ceil_div(bp.nchunk, 8) * 8 * P.Hkv);
  bucket_count<<<grid, kRowThreads, sizeof(int32_t) * P.nh, s>>>(
      sel, T.row_blk, b.chunk_base, P.Nq, P.Hq, P.G, P.k, P.nh, bp.rows_per_chunk, bp.nchunk,
      P.Hkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bucket_scan_cols<<<(unsigned)ceil_div(bp.nbins, 16), kThreads, 0, s>>>(b.chunk_base, b.bin_total,
                                                                         bp.nbins, P.nh, bp.nchunk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bucket_scan_bins<<<1, 1024, 0, s>>>(b.bin_total, b.bin_off, b.tile_off, b.scalars, bp.nbins,
                                      kTileQ);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bucket_scatter<<<grid, kRowThreads, 2 * sizeof(uint32_t) * P.nh * bp.ws, s>>>(
      sel, T.row_blk, b.chunk_base, b.bin_off, b.entries, P.Nq, P.Hq, P.Hkv, P.G, P.k, P.nh,
      bp.rows_per_chunk, bp.nchunk, bp.words, bp.ws, P.kvpp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (b.tile_map) {
    bucket_tile_map<<<(unsigned)bp.nbins, kThreads, 0, s>>>(b.tile_off, b.tile_map);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace moba
