// Host runtime and C ABI of libmoba.so: argument checks, workspace plan and
// the launch sequence of the five stages on the caller's stream. The
// operation and every entry point are specified in include/moba.h.
#include <climits>
#include <mutex>
#include <cmath>
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>

#include "moba_internal.hpp"

namespace moba {
namespace {

thread_local std::string g_last_error;

int fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return MOBA_ERR_HIP;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// KV heads per attention pass: as asked, else the largest group whose
// history partials fit kPassPartialBytes (at least one KV head).
constexpr double kPassPartialBytes = 16.0 * (1u << 30);
int passes_kvpp(const Prob& P, int asked) {
  if (asked > 0) return asked;
  const double per_kv = (double)P.hist_rows * P.G *
                        ((double)part_elem_bytes(P) * P.d + sizeof(float));
  const double fit = per_kv > 0 ? std::floor(kPassPartialBytes / per_kv) : (double)P.Hkv;
  return fit < 1 ? 1 : fit > P.Hkv ? P.Hkv : (int)fit;
}
int num_passes(const Prob& P) { return (int)ceil_div(P.Hkv, P.kvpp); }
Prob pass_of(const Prob& P, int i) {
  Prob Q = P;
  Q.g0 = i * P.kvpp;
  Q.gs = P.Hkv - Q.g0 < P.kvpp ? P.Hkv - Q.g0 : P.kvpp;
  return Q;
}

// The bf16 kernels read the packed V^T (and, in the backward, K^T) of one
// KV head through a buffer resource whose per-lane byte offsets are 32-bit:
// head-dim row d starts at d * ldv elements with ldv = blocks * Bpad, so the
// last row's 64-key tile must end below 2^32 bytes. Beyond that the offsets
// would wrap and read the wrong rows, so such problems are refused.
int check_vt_extent(const Prob& P, int64_t blocks) {
  if (P.dtype != MOBA_DTYPE_BF16) return MOBA_OK;
  const double ldv = (double)blocks * (double)vt_padded_block(P.B);
  if (2.0 * ((kHeadDim - 1) * ldv + 64.0) >= 4294967296.0)
    return fail(MOBA_ERR_UNSUPPORTED,
                "bf16: ceil(N/B) * ceil(B/64) * 64 must stay below 16,909,320 rows of packed V");
  return MOBA_OK;
}

// Checks the problem; fills *P. Returns MOBA_OK or an error code (with text).
int make_prob(const moba_problem_t* p, Prob* P) {
  if (!p) return fail(MOBA_ERR_INVALID_ARGUMENT, "problem pointer is NULL");
  if (p->seqlen < 1) return fail(MOBA_ERR_INVALID_ARGUMENT, "seqlen must be >= 1");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
  if (p->num_q_heads % p->num_kv_heads)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "num_q_heads must be a multiple of num_kv_heads");
  if (p->head_dim < 1) return fail(MOBA_ERR_INVALID_ARGUMENT, "head_dim must be >= 1");
  if (p->block_size < 1) return fail(MOBA_ERR_INVALID_ARGUMENT, "block_size must be >= 1");
  if (p->topk < 1) return fail(MOBA_ERR_INVALID_ARGUMENT, "topk must be >= 1");
  if (!std::isfinite(p->scale) || !(p->scale > 0.f))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (p->dtype != MOBA_DTYPE_BF16 && p->dtype != MOBA_DTYPE_F32)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "dtype must be MOBA_DTYPE_BF16 or MOBA_DTYPE_F32");
  if (p->routing != MOBA_ROUTING_PER_HEAD && p->routing != MOBA_ROUTING_SHARED)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "routing must be MOBA_ROUTING_PER_HEAD or _SHARED");
  if (p->kv_heads_per_pass < 0 || p->kv_heads_per_pass > p->num_kv_heads)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "kv_heads_per_pass must be in [0, num_kv_heads]");
  if (p->head_dim != kHeadDim) return fail(MOBA_ERR_UNSUPPORTED, "only head_dim == 128 is built");
  if (p->topk > kMaxTopk) return fail(MOBA_ERR_UNSUPPORTED, "topk > 32 is not supported");
  const int G = p->num_q_heads / p->num_kv_heads;
  if (G > kMaxGroup) return fail(MOBA_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads > 64");
  if ((double)p->seqlen * p->num_q_heads * p->topk >= 2147483648.0)
    return fail(MOBA_ERR_UNSUPPORTED, "seqlen * num_q_heads * topk must be < 2^31");
  P->N = p->seqlen;
  P->Nq = p->seqlen;
  P->q0 = 0;
  P->Hq = p->num_q_heads;
  P->Hkv = p->num_kv_heads;
  P->G = G;
  P->d = p->head_dim;
  P->B = p->block_size;
  P->k = p->topk;
  P->KH = p->topk - 1;
  P->scale = p->scale;
  P->dtype = p->dtype;
  P->routing = p->routing;
  // one sequence of all rows; make_prob_varlen overrides the sequence layout
  P->nseq = 1;
  P->n = (P->N + P->B - 1) / P->B;
  P->nh = P->n - 1;
  P->vt_blocks = P->n;
  P->g0 = 0;
  P->gs = P->Hkv;
  P->hist_rows = 0;
  for (int64_t c = 0; c < P->n; ++c) {
    const int64_t rows = P->N - c * P->B < P->B ? P->N - c * P->B : P->B;
    P->hist_rows += rows * (c < P->KH ? c : P->KH);
  }
  P->kvpp = passes_kvpp(*P, p->kv_heads_per_pass);
  if (P->nh > kMaxHist) return fail(MOBA_ERR_UNSUPPORTED, "more than 8192 history blocks");
  return check_vt_extent(*P, P->n);
}

// Chunk of the last q_rows positions of one sequence of p->seqlen rows: the
// queries are rows [seqlen - q_rows, seqlen), the keys all seqlen rows.
int make_prob_chunk(const moba_problem_t* p, int64_t q_rows, Prob* P) {
  int rc = make_prob(p, P);
  if (rc) return rc;
  if (q_rows < 1 || q_rows > P->N)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "q_rows must be in [1, seqlen]");
  P->Nq = q_rows;
  P->q0 = P->N - q_rows;
  P->hist_rows = 0;
  for (int64_t c = P->q0 / P->B; c < P->n; ++c) {
    const int64_t a = c * P->B > P->q0 ? c * P->B : P->q0;
    const int64_t e = (c + 1) * P->B < P->N ? (c + 1) * P->B : P->N;
    P->hist_rows += (e - a) * (c < P->KH ? c : P->KH);
  }
  P->kvpp = passes_kvpp(*P, p->kv_heads_per_pass);
  return MOBA_OK;
}

// Packed sequences: row offsets cu[0..nseq] on the host (cu[0] = 0,
// nondecreasing, cu[nseq] = seqlen). Blocks restart at every sequence.
int make_prob_varlen(const moba_problem_t* p, int64_t nseq, const int64_t* cu, Prob* P) {
  if (!cu) return fail(MOBA_ERR_INVALID_ARGUMENT, "cu_seqlens (host) is NULL");
  if (nseq < 1) return fail(MOBA_ERR_INVALID_ARGUMENT, "nseq must be >= 1");
  if (!p) return fail(MOBA_ERR_INVALID_ARGUMENT, "problem pointer is NULL");
  if (cu[0] != 0) return fail(MOBA_ERR_INVALID_ARGUMENT, "cu_seqlens[0] must be 0");
  for (int64_t i = 0; i < nseq; ++i)
    if (cu[i + 1] < cu[i]) return fail(MOBA_ERR_INVALID_ARGUMENT, "cu_seqlens must be nondecreasing");
  if (cu[nseq] != p->seqlen)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "cu_seqlens[nseq] must equal seqlen");
  int rc = make_prob(p, P);
  if (rc) return rc;
  if (nseq > INT32_MAX) return fail(MOBA_ERR_UNSUPPORTED, "too many sequences");
  P->nseq = nseq;
  P->n = 0;
  P->hist_rows = 0;
  for (int64_t i = 0; i < nseq; ++i) {
    const int64_t L = cu[i + 1] - cu[i];
    const int64_t nb = (L + P->B - 1) / P->B;
    for (int64_t c = 0; c < nb; ++c) {
      const int64_t rows = L - c * P->B < P->B ? L - c * P->B : P->B;
      P->hist_rows += rows * (c < P->KH ? c : P->KH);
    }
    P->n += nb;
  }
  P->nh = P->n - 1;
  P->vt_blocks = P->n;
  P->kvpp = passes_kvpp(*P, p->kv_heads_per_pass);
  if (P->nh > kMaxHist) return fail(MOBA_ERR_UNSUPPORTED, "more than 8192 history blocks");
  return check_vt_extent(*P, P->n);
}

size_t elem_bytes(const Prob& P) { return P.dtype == MOBA_DTYPE_BF16 ? 2 : 4; }


struct Layout {
  size_t blk_start, blk_len, blk_lo, qstart, qlen, qpos, row_blk, seq_base;
  size_t kbar, mp_part, gate, sel, chunk_base, bin_total, bin_off, tile_off, scalars, tile_map, entries,
      redo, part_lse, part_o, vt, dec_part, delta, dq_acc, part_dq, kt, total;
};

// Bytes of the packed V^T copy the bf16 kernels read (0 for fp32).
size_t vt_bytes(const Prob& P) {
  if (P.dtype != MOBA_DTYPE_BF16) return 0;
  return sizeof(uint16_t) * (size_t)P.Hkv * P.d * (size_t)(P.n * vt_padded_block(P.B));
}

// Block and row tables (first in every workspace).
void take_tables(const Prob& P, Layout& L, size_t& off) {
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.blk_start = take(sizeof(int32_t) * (size_t)P.n);
  L.blk_len = take(sizeof(int32_t) * (size_t)P.n);
  L.blk_lo = take(sizeof(int32_t) * (size_t)P.n);
  L.qstart = take(sizeof(int32_t) * (size_t)P.n);
  L.qlen = take(sizeof(int32_t) * (size_t)P.n);
  L.qpos = take(sizeof(int32_t) * (size_t)P.n);
  L.row_blk = take(sizeof(int32_t) * (size_t)P.Nq);
  L.seq_base = take(sizeof(int32_t) * (size_t)(P.nseq + 1));
}

// Backward workspace: tables, block means, gate, selection, buckets, then the
// fp32 row terms D = dO.O and, for fp32 inputs, the dq accumulator; for bf16
// inputs, the per-slot dq partials and the transposed K copy.
Layout plan_ws_bwd(const Prob& P) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  take_tables(P, L, off);
  const int splits = meanpool_splits(P);
  L.kbar = take(sizeof(double) * (size_t)(P.Hkv * P.nh * P.d));
  L.mp_part = take(sizeof(double) * (size_t)splits * P.nh * P.Hkv * P.d);
  L.gate = take(gate_scratch_bytes(P));
  const BucketPlan bp = plan_bucket(P);
  L.sel = take(sizeof(int32_t) * (size_t)(P.Nq * P.Hq * P.k));
  L.chunk_base = take(sizeof(int32_t) * (size_t)(P.Hkv * bp.nchunk * P.nh));
  L.bin_total = take(sizeof(int32_t) * (size_t)(bp.nbins + 1));
  L.bin_off = take(sizeof(int32_t) * (size_t)(bp.nbins + 1));
  L.tile_off = take(sizeof(int32_t) * (size_t)(bp.nbins + 1));
  L.scalars = take(sizeof(int32_t) * 4);
  L.tile_map = take(sizeof(int32_t) * (size_t)bp.max_tiles);
  L.entries = take(sizeof(uint32_t) * (size_t)bp.max_entries);
  L.delta = take(sizeof(float) * (size_t)(P.Nq * P.Hq));
  if (P.dtype == MOBA_DTYPE_BF16) {
    L.part_dq = take(sizeof(float) * (size_t)(P.Nq * P.Hq) * P.KH * P.d);
    L.kt = take(vt_bytes(P));
  } else {
    L.dq_acc = take(sizeof(float) * (size_t)(P.Nq * P.Hq) * P.d);
  }
  L.total = off;
  return L;
}

// Workspace layout; `full` = prefill (all stages), else select only;
// `cached` = block means and packed V come from a decode cache (no mean
// partials, no V^T copy).
Layout plan_ws(const Prob& P, bool full, bool cached = false) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  take_tables(P, L, off);
  const int splits = meanpool_splits(P);
  L.kbar = take(sizeof(double) * (size_t)(P.Hkv * P.nh * P.d));
  L.mp_part = cached ? off : take(sizeof(double) * (size_t)splits * P.nh * P.Hkv * P.d);
  L.gate = take(gate_scratch_bytes(P));
  if (full) {
    const BucketPlan bp = plan_bucket(P);
    L.sel = take(sizeof(int32_t) * (size_t)(P.Nq * P.Hq * P.k));
    L.chunk_base = take(sizeof(int32_t) * (size_t)(P.Hkv * bp.nchunk * P.nh));
    L.bin_total = take(sizeof(int32_t) * (size_t)(bp.nbins + 1));
    L.bin_off = take(sizeof(int32_t) * (size_t)(bp.nbins + 1));
    L.tile_off = take(sizeof(int32_t) * (size_t)(bp.nbins + 1));
    L.scalars = take(sizeof(int32_t) * 4);
    L.tile_map = take(sizeof(int32_t) * (size_t)bp.max_tiles);
    L.entries = take(sizeof(uint32_t) * (size_t)bp.max_entries);
    if (P.Nq <= kDecodeRows) {  // few rows: split-K partials instead of the tiled path
      L.part_lse = L.part_o = L.vt = off;
      L.dec_part = take(decode_part_bytes(P));
    } else {
      // history partials of one attention pass (kvpp KV heads)
      const size_t slots = (size_t)P.Nq * (size_t)(P.kvpp * P.G) * (size_t)P.KH;
      L.redo = take(sizeof(int32_t) * (size_t)bp.max_tiles);
      L.part_lse = take(sizeof(float) * slots);
      L.part_o = take(part_elem_bytes(P) * slots * P.d);
      L.vt = cached ? off : take(vt_bytes(P));
    }
  }
  L.total = off;
  return L;
}

// A decode cache seen by one call: means of the cache's full blocks
// [Hkv][nhc][d] and (bf16) the packed V^T of its capacity in blocks.
struct CacheView {
  const double* kbar;
  int64_t nhc;
  const void* vt;
  int64_t vt_blocks;
};

// Cache layout for `capacity` rows: kbar [Hkv][ncap - 1][d] fp64, then V^T
// [Hkv][d][ncap * Bpad] for bf16.
struct CacheLayout {
  int64_t ncap, nhc;
  size_t kbar, vt, total;
};
CacheLayout cache_layout(const Prob& P, int64_t capacity) {
  CacheLayout C{};
  C.ncap = (capacity + P.B - 1) / P.B;
  C.nhc = C.ncap > 0 ? C.ncap - 1 : 0;
  size_t off = 0;
  C.kbar = off;
  off = align_up(off + sizeof(double) * (size_t)P.Hkv * C.nhc * P.d);
  C.vt = off;
  if (P.dtype == MOBA_DTYPE_BF16)
    off = align_up(off + sizeof(uint16_t) * (size_t)P.Hkv * P.d *
                             (size_t)(C.ncap * vt_padded_block(P.B)));
  C.total = off;
  return C;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_ptrs(const void* const* ptrs, int n, const char* what) {
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(MOBA_ERR_INVALID_ARGUMENT, what);
    if (!aligned(ptrs[i], 16))
      return fail(MOBA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  }
  return MOBA_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) return fail(MOBA_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than required");
  if (need > 0 && !ws) return fail(MOBA_ERR_INVALID_ARGUMENT, "workspace pointer is NULL");
  if (ws && !aligned(ws, kAlign))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return MOBA_OK;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

Blocks tables(void* ws, const Layout& L) {
  Blocks t{};
  t.start = at<int32_t>(ws, L.blk_start);
  t.len = at<int32_t>(ws, L.blk_len);
  t.lo = at<int32_t>(ws, L.blk_lo);
  t.qstart = at<int32_t>(ws, L.qstart);
  t.qlen = at<int32_t>(ws, L.qlen);
  t.qpos = at<int32_t>(ws, L.qpos);
  t.row_blk = at<int32_t>(ws, L.row_blk);
  t.seq_base = at<int32_t>(ws, L.seq_base);
  return t;
}

BucketBufs bucket_bufs(void* ws, const Layout& L) {
  BucketBufs b{};
  b.chunk_base = at<int32_t>(ws, L.chunk_base);
  b.bin_total = at<int32_t>(ws, L.bin_total);
  b.bin_off = at<int32_t>(ws, L.bin_off);
  b.tile_off = at<int32_t>(ws, L.tile_off);
  b.tile_map = at<int32_t>(ws, L.tile_map);
  b.scalars = at<int32_t>(ws, L.scalars);
  b.entries = at<uint32_t>(ws, L.entries);
  b.redo = L.redo ? at<int32_t>(ws, L.redo) : nullptr;
  return b;
}

int record(void* const* events, int i, hipStream_t s) {
  if (!events) return MOBA_OK;
  hipError_t e = hipEventRecord((hipEvent_t)events[i], s);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "hipEventRecord");
}

// Tables, block means, gate + top-k. cu: device row offsets or NULL.
int run_select(const Prob& P, const int64_t* cu, const void* q, const void* k, int32_t* sel,
               void* ws, const Layout& L, hipStream_t s, void* const* events,
               const CacheView* cv = nullptr) {
  int rc;
  const Blocks T = tables(ws, L);
  hipError_t e = launch_tables(P, cu, T, s);
  if (e != hipSuccess) return hip_fail(e, "block tables");
  if (cv)
    e = launch_kbar_gather(cv->kbar, cv->nhc, at<double>(ws, L.kbar), P.nh, P.Hkv, P.d, s);
  else
    e = launch_meanpool(P, T, k, at<double>(ws, L.kbar), at<double>(ws, L.mp_part),
                        meanpool_splits(P), s);
  if (e != hipSuccess) return hip_fail(e, "moba_meanpool");
  if ((rc = record(events, 1, s))) return rc;
  e = launch_gate_topk(P, T, q, at<double>(ws, L.kbar), at<void>(ws, L.gate), sel, s);
  if (e != hipSuccess) return hip_fail(e, "moba_gate_topk");
  return record(events, 2, s);
}

// The whole path on prepared problem and workspace.
int run_prefill(const Prob& P0, const int64_t* cu, const void* q, const void* k, const void* v,
                void* o, void* workspace, const Layout& L, hipStream_t s, void* const* events,
                float* lse = nullptr, const CacheView* cv = nullptr) {
  int rc;
  Prob P = P0;
  if (cv) P.vt_blocks = cv->vt_blocks;
  if ((rc = record(events, 0, s))) return rc;
  int32_t* sel = at<int32_t>(workspace, L.sel);
  if ((rc = run_select(P, cu, q, k, sel, workspace, L, s, events, cv))) return rc;
  const Blocks T = tables(workspace, L);
  if (P.Nq <= kDecodeRows) {  // few rows: split-K over the selected blocks
    const int nev = 5 + 2 * num_passes(P);
    for (int i = 3; i < nev - 1; ++i)
      if ((rc = record(events, i, s))) return rc;
    hipError_t e = launch_decode(P, T, q, k, v, sel, at<float>(workspace, L.dec_part), o, lse, s);
    if (e != hipSuccess) return hip_fail(e, "moba_attn (few rows)");
    return record(events, nev - 1, s);
  }
  const BucketPlan bp = plan_bucket(P);
  const BucketBufs bb = bucket_bufs(workspace, L);
  hipError_t e = launch_bucket(P, T, bp, sel, bb, s);
  if (e != hipSuccess) return hip_fail(e, "moba_bucket");
  if ((rc = record(events, 3, s))) return rc;
  void* part_o = at<void>(workspace, L.part_o);
  float* part_lse = at<float>(workspace, L.part_lse);
  const void* vt = cv ? cv->vt : at<void>(workspace, L.vt);
  if (P.dtype == MOBA_DTYPE_BF16 && !cv) {
    e = launch_vt_pack(P, T, v, at<void>(workspace, L.vt), s);
    if (e != hipSuccess) return hip_fail(e, "V pack");
  }
  if ((rc = record(events, 4, s))) return rc;
  // attention passes over groups of kvpp KV heads; the partials of one pass
  // live in the workspace at a time
  for (int i = 0; i < num_passes(P); ++i) {
    const Prob Pi = pass_of(P, i);
    e = launch_attn_hist(Pi, T, bp, q, k, v, vt, bb, part_o, part_lse, s);
    if (e != hipSuccess) return hip_fail(e, "moba_attn (history)");
    if ((rc = record(events, 5 + 2 * i, s))) return rc;
    e = launch_attn_self(Pi, T, q, k, v, vt, part_o, part_lse, o, lse, s);
    if (e != hipSuccess) return hip_fail(e, "moba_attn (own block) + moba_merge");
    if ((rc = record(events, 6 + 2 * i, s))) return rc;
  }
  return MOBA_OK;
}

int check_events(const Prob& P, void* const* events) {
  if (events)
    for (int i = 0; i < 5 + 2 * num_passes(P); ++i)
      if (!events[i]) return fail(MOBA_ERR_INVALID_ARGUMENT, "stage event handle is NULL");
  return MOBA_OK;
}

int check_cu_dev(const int64_t* cu_dev) {
  if (!cu_dev) return fail(MOBA_ERR_INVALID_ARGUMENT, "cu_seqlens (device) is NULL");
  if (!aligned(cu_dev, 8))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "cu_seqlens (device) must be 8-byte aligned");
  return MOBA_OK;
}

}  // namespace
}  // namespace moba

using namespace moba;

extern "C" {

size_t moba_workspace_size(const moba_problem_t* p) {
  Prob P;
  if (make_prob(p, &P) != MOBA_OK) return 0;
  return plan_ws(P, true).total;
}

size_t moba_stage_events(const moba_problem_t* p) {
  Prob P;
  if (make_prob(p, &P) != MOBA_OK) return 0;
  return (size_t)(5 + 2 * num_passes(P));
}

size_t moba_select_workspace_size(const moba_problem_t* p) {
  Prob P;
  if (make_prob(p, &P) != MOBA_OK) return 0;
  const size_t t = plan_ws(P, false).total;
  return t > 0 ? t : kAlign;
}

int moba_prefill_ex(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                    void* workspace, size_t ws_bytes, void* stream, void* const* events) {
  Prob P;
  int rc = make_prob(p, &P);
  if (rc) return rc;
  const void* ptrs[4] = {q, k, v, o};
  if ((rc = check_ptrs(ptrs, 4, "q, k, v and o must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, true);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  if ((rc = check_events(P, events))) return rc;
  return run_prefill(P, nullptr, q, k, v, o, workspace, L, (hipStream_t)stream, events);
}

int moba_prefill(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                 void* workspace, size_t ws_bytes, void* stream) {
  return moba_prefill_ex(p, q, k, v, o, workspace, ws_bytes, stream, nullptr);
}

int moba_select(const moba_problem_t* p, const void* q, const void* k, int32_t* sel,
                void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob(p, &P);
  if (rc) return rc;
  const void* ptrs[3] = {q, k, sel};
  if ((rc = check_ptrs(ptrs, 3, "q, k and sel must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, false);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  return run_select(P, nullptr, q, k, sel, workspace, L, (hipStream_t)stream, nullptr);
}

// Routing statistics: the select workspace, then room for a selection.
static size_t stats_ws(const Prob& P, const Layout& L, size_t* sel_off) {
  *sel_off = L.total;
  return align_up(L.total + sizeof(int32_t) * (size_t)(P.Nq * P.Hq * P.k));
}

size_t moba_routing_stats_workspace_size(const moba_problem_t* p) {
  Prob P;
  if (make_prob(p, &P) != MOBA_OK) return 0;
  size_t off;
  return stats_ws(P, plan_ws(P, false), &off);
}

int moba_routing_stats(const moba_problem_t* p, const void* q, const void* k, int32_t* sel,
                       float* margin, int32_t* counts, int32_t* union_size, void* workspace,
                       size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob(p, &P);
  if (rc) return rc;
  const void* ptrs[2] = {q, k};
  if ((rc = check_ptrs(ptrs, 2, "q and k must be non-NULL"))) return rc;
  const void* outs[4] = {sel, margin, counts, union_size};
  for (const void* o : outs)
    if (o && !aligned(o, 4)) return fail(MOBA_ERR_INVALID_ARGUMENT, "outputs must be 4-byte aligned");
  const Layout L = plan_ws(P, false);
  size_t sel_off;
  if ((rc = check_ws(workspace, ws_bytes, stats_ws(P, L, &sel_off)))) return rc;
  hipStream_t s = (hipStream_t)stream;
  int32_t* selw = sel ? sel : at<int32_t>(workspace, sel_off);
  const Blocks T = tables(workspace, L);
  hipError_t e = launch_tables(P, nullptr, T, s);
  if (e == hipSuccess)
    e = launch_meanpool(P, T, k, at<double>(workspace, L.kbar), at<double>(workspace, L.mp_part),
                        meanpool_splits(P), s);
  if (e == hipSuccess)
    e = launch_gate_margin(P, T, q, at<double>(workspace, L.kbar), at<void>(workspace, L.gate),
                           selw, margin, s);
  if (e == hipSuccess) e = launch_routing_reductions(P, T, selw, counts, union_size, s);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "routing statistics");
}

// ---------------------------------------------------------------------------
// Allocation-free prefill: the workspace is a fixed device array of this
// library (one per GPU, held until the process ends) instead of a caller
// buffer. Its device address is looked up once per device.
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {
constexpr size_t kScratchBytes = (size_t)512 << 20;  // 512 MiB per device
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};  // per device id, from hipGetSymbolAddress

int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MOBA_ERR_UNSUPPORTED, "device id >= 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOBA_OK;
}
}  // namespace

extern "C" {

size_t moba_noalloc_max_workspace(void) { return kScratchBytes; }

int moba_prefill_noalloc(const moba_problem_t* p, const void* q, const void* k, const void* v,
                         void* o, void* stream) {
  Prob P;
  int rc = make_prob(p, &P);
  if (rc) return rc;
  const void* ptrs[4] = {q, k, v, o};
  if ((rc = check_ptrs(ptrs, 4, "q, k, v and o must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, true);
  if (L.total > kScratchBytes)
    return fail(MOBA_ERR_UNSUPPORTED,
                "problem needs more workspace than the library's 512 MiB allocation-free scratch");
  void* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  return run_prefill(P, nullptr, q, k, v, o, ws, L, (hipStream_t)stream, nullptr);
}

int moba_prefill_train(const moba_problem_t* p, const void* q, const void* k, const void* v,
                       void* o, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob(p, &P);
  if (rc) return rc;
  const void* ptrs[5] = {q, k, v, o, lse};
  if ((rc = check_ptrs(ptrs, 5, "q, k, v, o and lse must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, true);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  return run_prefill(P, nullptr, q, k, v, o, workspace, L, (hipStream_t)stream, nullptr, lse);
}

size_t moba_backward_workspace_size(const moba_problem_t* p) {
  Prob P;
  if (make_prob(p, &P) != MOBA_OK) return 0;
  P.kvpp = P.Hkv;
  return plan_ws_bwd(P).total;
}

static int run_backward(const Prob& P0, const int64_t* cu_dev, const void* q, const void* k,
                        const void* v, const void* o, const float* lse, const void* dout,
                        void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                        void* stream) {
  int rc;
  // the backward kernels take the bucket lists of all heads in one pass
  Prob P = P0;
  P.kvpp = P.Hkv;
  const void* ptrs[10] = {q, k, v, o, lse, dout, dq, dk, dv, nullptr};
  if ((rc = check_ptrs(ptrs, 9, "q, k, v, o, lse, dout, dq, dk and dv must be non-NULL")))
    return rc;
  const Layout L = plan_ws_bwd(P);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  hipStream_t s = (hipStream_t)stream;
  int32_t* sel = at<int32_t>(workspace, L.sel);
  if ((rc = run_select(P, cu_dev, q, k, sel, workspace, L, s, nullptr))) return rc;
  const Blocks T = tables(workspace, L);
  const BucketPlan bp = plan_bucket(P);
  const BucketBufs bb = bucket_bufs(workspace, L);
  hipError_t e = launch_bucket(P, T, bp, sel, bb, s);
  if (e != hipSuccess) return hip_fail(e, "moba_bucket");
  BwdScratch w{};
  w.delta = at<float>(workspace, L.delta);
  if (P.dtype == MOBA_DTYPE_BF16) {
    w.part_dq = at<float>(workspace, L.part_dq);
    w.kt = at<void>(workspace, L.kt);
  } else {
    w.dq_acc = at<float>(workspace, L.dq_acc);
  }
  e = launch_backward(P, T, bp, bb, q, k, v, o, lse, dout, dq, dk, dv, w, s);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "moba_backward");
}

int moba_backward(const moba_problem_t* p, const void* q, const void* k, const void* v,
                  const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                  void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob(p, &P);
  if (rc) return rc;
  return run_backward(P, nullptr, q, k, v, o, lse, dout, dq, dk, dv, workspace, ws_bytes, stream);
}

int moba_prefill_train_varlen(const moba_problem_t* p, int64_t nseq,
                              const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
                              const void* q, const void* k, const void* v, void* o, float* lse,
                              void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob_varlen(p, nseq, cu_seqlens_host, &P);
  if (rc) return rc;
  if ((rc = check_cu_dev(cu_seqlens_dev))) return rc;
  const void* ptrs[5] = {q, k, v, o, lse};
  if ((rc = check_ptrs(ptrs, 5, "q, k, v, o and lse must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, true);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  return run_prefill(P, cu_seqlens_dev, q, k, v, o, workspace, L, (hipStream_t)stream, nullptr,
                     lse);
}

size_t moba_backward_varlen_workspace_size(const moba_problem_t* p, int64_t nseq,
                                           const int64_t* cu_seqlens_host) {
  Prob P;
  if (make_prob_varlen(p, nseq, cu_seqlens_host, &P) != MOBA_OK) return 0;
  return plan_ws_bwd(P).total;
}

int moba_backward_varlen(const moba_problem_t* p, int64_t nseq, const int64_t* cu_seqlens_host,
                         const int64_t* cu_seqlens_dev, const void* q, const void* k,
                         const void* v, const void* o, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                         void* stream) {
  Prob P;
  int rc = make_prob_varlen(p, nseq, cu_seqlens_host, &P);
  if (rc) return rc;
  if ((rc = check_cu_dev(cu_seqlens_dev))) return rc;
  return run_backward(P, cu_seqlens_dev, q, k, v, o, lse, dout, dq, dk, dv, workspace, ws_bytes,
                      stream);
}

size_t moba_chunk_workspace_size(const moba_problem_t* p, int64_t q_rows) {
  Prob P;
  if (make_prob_chunk(p, q_rows, &P) != MOBA_OK) return 0;
  return plan_ws(P, true).total;
}

int moba_prefill_chunk(const moba_problem_t* p, int64_t q_rows, const void* q, const void* k,
                       const void* v, void* o, void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob_chunk(p, q_rows, &P);
  if (rc) return rc;
  const void* ptrs[4] = {q, k, v, o};
  if ((rc = check_ptrs(ptrs, 4, "q, k, v and o must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, true);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  return run_prefill(P, nullptr, q, k, v, o, workspace, L, (hipStream_t)stream, nullptr);
}

int moba_select_chunk(const moba_problem_t* p, int64_t q_rows, const void* q, const void* k,
                      int32_t* sel, void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob_chunk(p, q_rows, &P);
  if (rc) return rc;
  const void* ptrs[3] = {q, k, sel};
  if ((rc = check_ptrs(ptrs, 3, "q, k and sel must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, false);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  return run_select(P, nullptr, q, k, sel, workspace, L, (hipStream_t)stream, nullptr);
}

static int check_capacity(const Prob& P, int64_t capacity) {
  if (capacity < P.N) return fail(MOBA_ERR_INVALID_ARGUMENT, "capacity must be >= seqlen");
  if ((double)capacity * P.Hq * P.k >= 2147483648.0)
    return fail(MOBA_ERR_UNSUPPORTED, "capacity * num_q_heads * topk must be < 2^31");
  if ((capacity + P.B - 1) / P.B - 1 > kMaxHist)
    return fail(MOBA_ERR_UNSUPPORTED, "more than 8192 history blocks in the capacity");
  return check_vt_extent(P, (capacity + P.B - 1) / P.B);
}

size_t moba_cache_bytes(const moba_problem_t* p, int64_t capacity) {
  Prob P;
  if (make_prob(p, &P) != MOBA_OK) return 0;
  if (capacity < 1) return 0;
  moba_problem_t c = *p;
  c.seqlen = capacity;
  if (make_prob(&c, &P) != MOBA_OK) return 0;
  return cache_layout(P, capacity).total;
}

int moba_cache_append(const moba_problem_t* p, int64_t capacity, int64_t rows_before,
                      const void* k, const void* v, void* cache, void* stream) {
  Prob P;
  int rc = make_prob(p, &P);
  if (rc) return rc;
  if ((rc = check_capacity(P, capacity))) return rc;
  if (rows_before < 0 || rows_before > P.N)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "rows_before must be in [0, seqlen]");
  const void* ptrs[3] = {k, v, cache};
  if ((rc = check_ptrs(ptrs, 3, "k, v and cache must be non-NULL"))) return rc;
  if (!aligned(cache, kAlign)) return fail(MOBA_ERR_INVALID_ARGUMENT, "cache must be 256-byte aligned");
  const CacheLayout C = cache_layout(P, capacity);
  P.vt_blocks = C.ncap;
  hipStream_t s = (hipStream_t)stream;
  // blocks completed by rows [rows_before, N) that can be history within the capacity
  int64_t c0 = rows_before / P.B, c1 = P.N / P.B;
  if (c1 > C.nhc) c1 = C.nhc;
  hipError_t e = launch_cache_means(P, k, c0, c1 - c0, at<double>(cache, C.kbar), C.nhc, s);
  if (e != hipSuccess) return hip_fail(e, "decode cache: block means");
  if (P.dtype == MOBA_DTYPE_BF16) {
    e = launch_vt_pack_rows(P, v, at<void>(cache, C.vt), rows_before, P.N, s);
    if (e != hipSuccess) return hip_fail(e, "decode cache: V pack");
  }
  return MOBA_OK;
}

size_t moba_cached_workspace_size(const moba_problem_t* p, int64_t q_rows) {
  Prob P;
  if (make_prob_chunk(p, q_rows, &P) != MOBA_OK) return 0;
  return plan_ws(P, true, true).total;
}

int moba_prefill_cached(const moba_problem_t* p, int64_t capacity, int64_t q_rows, const void* q,
                        const void* k, const void* v, const void* cache, void* o,
                        void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob_chunk(p, q_rows, &P);
  if (rc) return rc;
  if ((rc = check_capacity(P, capacity))) return rc;
  const void* ptrs[5] = {q, k, v, o, cache};
  if ((rc = check_ptrs(ptrs, 5, "q, k, v, o and cache must be non-NULL"))) return rc;
  if (!aligned(cache, kAlign)) return fail(MOBA_ERR_INVALID_ARGUMENT, "cache must be 256-byte aligned");
  const Layout L = plan_ws(P, true, true);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  const CacheLayout C = cache_layout(P, capacity);
  const CacheView cv{at<double>(const_cast<void*>(cache), C.kbar), C.nhc,
                     at<void>(const_cast<void*>(cache), C.vt), C.ncap};
  return run_prefill(P, nullptr, q, k, v, o, workspace, L, (hipStream_t)stream, nullptr, nullptr,
                     &cv);
}

size_t moba_varlen_workspace_size(const moba_problem_t* p, int64_t nseq,
                                  const int64_t* cu_seqlens_host) {
  Prob P;
  if (make_prob_varlen(p, nseq, cu_seqlens_host, &P) != MOBA_OK) return 0;
  return plan_ws(P, true).total;
}

size_t moba_varlen_select_workspace_size(const moba_problem_t* p, int64_t nseq,
                                         const int64_t* cu_seqlens_host) {
  Prob P;
  if (make_prob_varlen(p, nseq, cu_seqlens_host, &P) != MOBA_OK) return 0;
  return plan_ws(P, false).total;
}

int moba_prefill_varlen(const moba_problem_t* p, int64_t nseq, const int64_t* cu_seqlens_host,
                        const int64_t* cu_seqlens_dev, const void* q, const void* k,
                        const void* v, void* o, void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob_varlen(p, nseq, cu_seqlens_host, &P);
  if (rc) return rc;
  if ((rc = check_cu_dev(cu_seqlens_dev))) return rc;
  const void* ptrs[4] = {q, k, v, o};
  if ((rc = check_ptrs(ptrs, 4, "q, k, v and o must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, true);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  return run_prefill(P, cu_seqlens_dev, q, k, v, o, workspace, L, (hipStream_t)stream, nullptr);
}

int moba_select_varlen(const moba_problem_t* p, int64_t nseq, const int64_t* cu_seqlens_host,
                       const int64_t* cu_seqlens_dev, const void* q, const void* k, int32_t* sel,
                       void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob_varlen(p, nseq, cu_seqlens_host, &P);
  if (rc) return rc;
  if ((rc = check_cu_dev(cu_seqlens_dev))) return rc;
  const void* ptrs[3] = {q, k, sel};
  if ((rc = check_ptrs(ptrs, 3, "q, k and sel must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, false);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  return run_select(P, cu_seqlens_dev, q, k, sel, workspace, L, (hipStream_t)stream, nullptr);
}

static int dense_prob(const moba_problem_t* p, Prob* P) {
  if (!p) return fail(MOBA_ERR_INVALID_ARGUMENT, "problem pointer is NULL");
  // block_size and topk do not apply: one block spanning the sequence, no history
  moba_problem_t d = *p;
  d.block_size = p->seqlen > 0 && p->seqlen < INT32_MAX ? (int32_t)p->seqlen : 1;
  d.topk = 1;
  return make_prob(&d, P);
}

// Dense workspace: block tables of the one-block problem, then V^T.
static size_t dense_ws(const Prob& P, Layout* L) {
  size_t off = 0;
  take_tables(P, *L, off);
  L->vt = off;
  return align_up(off + vt_bytes(P));
}

size_t moba_dense_workspace_size(const moba_problem_t* p) {
  Prob P;
  if (dense_prob(p, &P) != MOBA_OK) return 0;
  Layout L{};
  return dense_ws(P, &L);
}

int moba_dense_causal(const moba_problem_t* p, const void* q, const void* k, const void* v,
                      void* o, void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = dense_prob(p, &P);
  if (rc) return rc;
  const void* ptrs[4] = {q, k, v, o};
  if ((rc = check_ptrs(ptrs, 4, "q, k, v and o must be non-NULL"))) return rc;
  Layout L{};
  if ((rc = check_ws(workspace, ws_bytes, dense_ws(P, &L)))) return rc;
  hipStream_t s = (hipStream_t)stream;
  const Blocks T = tables(workspace, L);
  hipError_t e = launch_tables(P, nullptr, T, s);
  if (e != hipSuccess) return hip_fail(e, "block tables");
  void* vt = at<void>(workspace, L.vt);
  if (P.dtype == MOBA_DTYPE_BF16) {
    e = launch_vt_pack(P, T, v, vt, s);
    if (e != hipSuccess) return hip_fail(e, "V pack");
  }
  e = launch_attn_self(P, T, q, k, v, vt, nullptr, nullptr, o, nullptr, s);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "dense causal attention");
}

const char* moba_status_string(int status) {
  switch (status) {
    case MOBA_OK: return "MOBA_OK";
    case MOBA_ERR_INVALID_ARGUMENT: return "MOBA_ERR_INVALID_ARGUMENT";
    case MOBA_ERR_UNSUPPORTED: return "MOBA_ERR_UNSUPPORTED";
    case MOBA_ERR_WORKSPACE_TOO_SMALL: return "MOBA_ERR_WORKSPACE_TOO_SMALL";
    case MOBA_ERR_HIP: return "MOBA_ERR_HIP";
    default: return "MOBA_ERR_UNKNOWN";
  }
}

const char* moba_last_error(void) { return g_last_error.c_str(); }

int moba_debug_meanpool(const moba_problem_t* p, const void* k, double* kbar, void* workspace,
                        size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob(p, &P);
  if (rc) return rc;
  const void* ptrs[2] = {k, kbar};
  if ((rc = check_ptrs(ptrs, 2, "k and kbar must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, false);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  const Blocks T = tables(workspace, L);
  hipError_t e = launch_tables(P, nullptr, T, (hipStream_t)stream);
  if (e == hipSuccess)
    e = launch_meanpool(P, T, k, kbar, at<double>(workspace, L.mp_part), meanpool_splits(P),
                        (hipStream_t)stream);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "moba_meanpool");
}

size_t moba_debug_bucket_capacity(const moba_problem_t* p) {
  Prob P;
  if (make_prob(p, &P) != MOBA_OK) return 0;
  return (size_t)plan_bucket(P).max_entries;
}

int moba_debug_bucket(const moba_problem_t* p, const int32_t* sel, int32_t* offsets,
                      uint32_t* entries, void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = make_prob(p, &P);
  if (rc) return rc;
  const void* ptrs[3] = {sel, offsets, entries};
  if ((rc = check_ptrs(ptrs, 3, "sel, offsets and entries must be non-NULL"))) return rc;
  const Layout L = plan_ws(P, true);
  if ((rc = check_ws(workspace, ws_bytes, L.total))) return rc;
  P.kvpp = P.Hkv;  // entries numbered over all heads: ((row * Hq + head) * (k - 1) + slot)
  BucketBufs bb = bucket_bufs(workspace, L);
  bb.bin_off = offsets;
  bb.entries = entries;
  const Blocks T = tables(workspace, L);
  hipError_t e = launch_tables(P, nullptr, T, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_bucket(P, T, plan_bucket(P), sel, bb, (hipStream_t)stream);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "moba_bucket");
}

int moba_debug_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return fail(MOBA_ERR_INVALID_ARGUMENT, "src and dst must be non-NULL");
  if (!aligned(src, 16) || !aligned(dst, 16) || bytes % 16)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "copy needs 16-byte aligned pointers and sizes");
  hipError_t e = launch_copy(src, dst, bytes, (hipStream_t)stream);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "copy");
}

int moba_debug_read_peak(const void* src, size_t bytes, int32_t workgroups, uint32_t* out,
                         void* stream) {
  if (!src || !out) return fail(MOBA_ERR_INVALID_ARGUMENT, "src and out must be non-NULL");
  if (!aligned(src, 16) || bytes % 16 || !aligned(out, 4))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "read probe needs a 16-byte aligned src and size");
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "workgroups must lie in [1, 2^20]");
  hipError_t e = launch_read_probe(src, bytes, workgroups, out, (hipStream_t)stream);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "read probe");
}

int moba_debug_mfma_peak(int32_t workgroups, int32_t iters, float* out, void* stream) {
  if (!out || !aligned(out, 4)) return fail(MOBA_ERR_INVALID_ARGUMENT, "out must be a non-NULL float pointer");
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 20))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "workgroups and iters must lie in [1, 2^20]");
  hipError_t e = launch_mfma_probe(workgroups, iters, out, (hipStream_t)stream);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "mfma probe");
}

}  // extern "C"
