// Host runtime and C ABI of libmoba.so: argument checks, workspace plan and
// the launch sequence of the five stages on the caller's stream. The
// operation and every entry point are specified in include/moba.h.
#include <climits>
#include <cmath>
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
  if (p->head_dim != kHeadDim) return fail(MOBA_ERR_UNSUPPORTED, "only head_dim == 128 is built");
  if (p->topk > kMaxTopk) return fail(MOBA_ERR_UNSUPPORTED, "topk > 32 is not supported");
  const int G = p->num_q_heads / p->num_kv_heads;
  if (G > kMaxGroup) return fail(MOBA_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads > 64");
  const int64_t n = (p->seqlen + p->block_size - 1) / p->block_size;
  if (n - 1 > kMaxHist) return fail(MOBA_ERR_UNSUPPORTED, "more than 8192 history blocks");
  if ((double)p->seqlen * p->num_q_heads * p->topk >= 2147483648.0)
    return fail(MOBA_ERR_UNSUPPORTED, "seqlen * num_q_heads * topk must be < 2^31");
  P->N = p->seqlen;
  P->Hq = p->num_q_heads;
  P->Hkv = p->num_kv_heads;
  P->G = G;
  P->d = p->head_dim;
  P->B = p->block_size;
  P->k = p->topk;
  P->KH = p->topk - 1;
  P->n = n;
  P->nh = n - 1;
  P->scale = p->scale;
  P->dtype = p->dtype;
  return MOBA_OK;
}

size_t elem_bytes(const Prob& P) { return P.dtype == MOBA_DTYPE_BF16 ? 2 : 4; }

struct Layout {
  size_t kbar, mp_part, gate, sel, chunk_base, bin_total, bin_off, tile_off, scalars, tile_map, entries,
      part_lse, part_o, vt, total;
};

// Bytes of the packed V^T copy the bf16 kernels read (0 for fp32).
size_t vt_bytes(const Prob& P, int64_t B) {
  if (P.dtype != MOBA_DTYPE_BF16) return 0;
  const int64_t n = ceil_div(P.N, B);
  return sizeof(uint16_t) * (size_t)P.Hkv * P.d * (size_t)(n * vt_padded_block(B));
}

// Workspace layout; `full` = prefill (all stages), else select only.
Layout plan_ws(const Prob& P, bool full) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const int splits = meanpool_splits(P);
  L.kbar = take(sizeof(double) * (size_t)(P.Hkv * P.nh * P.d));
  L.mp_part = take(sizeof(double) * (size_t)splits * P.nh * P.Hkv * P.d);
  L.gate = take(gate_scratch_bytes(P));
  if (full) {
    const BucketPlan bp = plan_bucket(P);
    L.sel = take(sizeof(int32_t) * (size_t)(P.N * P.Hq * P.k));
    L.chunk_base = take(sizeof(int32_t) * (size_t)(P.Hkv * bp.nchunk * P.nh));
    L.bin_total = take(sizeof(int32_t) * (size_t)(bp.nbins + 1));
    L.bin_off = take(sizeof(int32_t) * (size_t)(bp.nbins + 1));
    L.tile_off = take(sizeof(int32_t) * (size_t)(bp.nbins + 1));
    L.scalars = take(sizeof(int32_t) * 4);
    L.tile_map = take(sizeof(int32_t) * (size_t)bp.max_tiles);
    L.entries = take(sizeof(uint32_t) * (size_t)bp.max_entries);
    const size_t slots = (size_t)(P.N * P.Hq) * (size_t)P.KH;
    L.part_lse = take(sizeof(float) * slots);
    L.part_o = take(part_elem_bytes(P) * slots * P.d);
    L.vt = take(vt_bytes(P, P.B));
  }
  L.total = off;
  return L;
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

BucketBufs bucket_bufs(void* ws, const Layout& L) {
  BucketBufs b{};
  b.chunk_base = at<int32_t>(ws, L.chunk_base);
  b.bin_total = at<int32_t>(ws, L.bin_total);
  b.bin_off = at<int32_t>(ws, L.bin_off);
  b.tile_off = at<int32_t>(ws, L.tile_off);
  b.tile_map = at<int32_t>(ws, L.tile_map);
  b.scalars = at<int32_t>(ws, L.scalars);
  b.entries = at<uint32_t>(ws, L.entries);
  return b;
}

int record(void* const* events, int i, hipStream_t s) {
  if (!events) return MOBA_OK;
  hipError_t e = hipEventRecord((hipEvent_t)events[i], s);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "hipEventRecord");
}

int run_select(const Prob& P, const void* q, const void* k, int32_t* sel, void* ws,
               const Layout& L, hipStream_t s, void* const* events) {
  int rc;
  hipError_t e = launch_meanpool(P, k, at<double>(ws, L.kbar), at<double>(ws, L.mp_part),
                                 meanpool_splits(P), s);
  if (e != hipSuccess) return hip_fail(e, "moba_meanpool");
  if ((rc = record(events, 1, s))) return rc;
  e = launch_gate_topk(P, q, at<double>(ws, L.kbar), at<void>(ws, L.gate), sel, s);
  if (e != hipSuccess) return hip_fail(e, "moba_gate_topk");
  return record(events, 2, s);
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
  if (events)
    for (int i = 0; i < MOBA_STAGE_EVENTS; ++i)
      if (!events[i]) return fail(MOBA_ERR_INVALID_ARGUMENT, "stage event handle is NULL");
  hipStream_t s = (hipStream_t)stream;
  if ((rc = record(events, 0, s))) return rc;
  int32_t* sel = at<int32_t>(workspace, L.sel);
  if ((rc = run_select(P, q, k, sel, workspace, L, s, events))) return rc;
  const BucketPlan bp = plan_bucket(P);
  const BucketBufs bb = bucket_bufs(workspace, L);
  hipError_t e = launch_bucket(P, bp, sel, bb, s);
  if (e != hipSuccess) return hip_fail(e, "moba_bucket");
  if ((rc = record(events, 3, s))) return rc;
  void* part_o = at<void>(workspace, L.part_o);
  float* part_lse = at<float>(workspace, L.part_lse);
  void* vt = at<void>(workspace, L.vt);
  if (P.dtype == MOBA_DTYPE_BF16) {
    e = launch_vt_pack(v, vt, P.N, P.Hkv, P.B, s);
    if (e != hipSuccess) return hip_fail(e, "V pack");
  }
  if ((rc = record(events, 4, s))) return rc;
  e = launch_attn_hist(P, bp, q, k, v, vt, bb, part_o, part_lse, s);
  if (e != hipSuccess) return hip_fail(e, "moba_attn (history)");
  if ((rc = record(events, 5, s))) return rc;
  e = launch_attn_self(P, q, k, v, vt, part_o, part_lse, o, false, s);
  if (e != hipSuccess) return hip_fail(e, "moba_attn (own block) + moba_merge");
  return record(events, 6, s);
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
  return run_select(P, q, k, sel, workspace, L, (hipStream_t)stream, nullptr);
}

static int dense_prob(const moba_problem_t* p, Prob* P) {
  if (!p) return fail(MOBA_ERR_INVALID_ARGUMENT, "problem pointer is NULL");
  // block_size and topk do not apply: one block spanning the sequence, no history
  moba_problem_t d = *p;
  d.block_size = p->seqlen > 0 && p->seqlen < INT32_MAX ? (int32_t)p->seqlen : 1;
  d.topk = 1;
  return make_prob(&d, P);
}

size_t moba_dense_workspace_size(const moba_problem_t* p) {
  Prob P;
  if (dense_prob(p, &P) != MOBA_OK) return 0;
  const size_t t = align_up(vt_bytes(P, P.N));
  return t > 0 ? t : kAlign;
}

int moba_dense_causal(const moba_problem_t* p, const void* q, const void* k, const void* v,
                      void* o, void* workspace, size_t ws_bytes, void* stream) {
  Prob P;
  int rc = dense_prob(p, &P);
  if (rc) return rc;
  const void* ptrs[4] = {q, k, v, o};
  if ((rc = check_ptrs(ptrs, 4, "q, k, v and o must be non-NULL"))) return rc;
  if ((rc = check_ws(workspace, ws_bytes, align_up(vt_bytes(P, P.N))))) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (P.dtype == MOBA_DTYPE_BF16) {
    hipError_t e = launch_vt_pack(v, workspace, P.N, P.Hkv, P.N, s);
    if (e != hipSuccess) return hip_fail(e, "V pack");
  }
  hipError_t e = launch_attn_self(P, q, k, v, workspace, nullptr, nullptr, o, true, s);
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
  hipError_t e = launch_meanpool(P, k, kbar, at<double>(workspace, L.mp_part), meanpool_splits(P),
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
  BucketBufs bb = bucket_bufs(workspace, L);
  bb.bin_off = offsets;
  bb.entries = entries;
  hipError_t e = launch_bucket(P, plan_bucket(P), sel, bb, (hipStream_t)stream);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "moba_bucket");
}

int moba_debug_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return fail(MOBA_ERR_INVALID_ARGUMENT, "src and dst must be non-NULL");
  if (!aligned(src, 16) || !aligned(dst, 16) || bytes % 16)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "copy needs 16-byte aligned pointers and sizes");
  hipError_t e = launch_copy(src, dst, bytes, (hipStream_t)stream);
  return e == hipSuccess ? MOBA_OK : hip_fail(e, "copy");
}

}  // extern "C"
