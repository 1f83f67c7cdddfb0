/*
 * moba.h — C ABI of the MI355X (gfx950) MoBA prefill library, libmoba.so.
 *
 * MoBA (Mixture of Block Attention) prefill forward for one attention layer.
 * The operation is the one on the PaperTrace page "2.1.3 MoBA"
 * (yayajjiang.github.io/PaperTrace, sparse-attention 2.1.3):
 *   - keys are cut into contiguous blocks of block_size tokens (section 1,
 *     eq. (2)); each block is summarised by the mean of its keys (eq. (3));
 *   - a query scores each earlier block with the unscaled dot product
 *     q . kbar_i (eq. (3)); blocks after its own block are excluded; its own
 *     block is always taken and never ranked (section 2); top-k counts that
 *     own block, so at most topk-1 earlier blocks are taken (section 2.1);
 *     ties go to the lower block index;
 *   - the output is one softmax over the union of the taken tokens — the own
 *     block causally (keys j <= p), earlier blocks whole (eqs. (4)-(6)) — with
 *     the two branches merged through (m, l, u) statistics (eqs. (7)-(8)).
 * The MoonshotAI/MoBA README names the public interface of the original:
 * Q, K, V, block size and top-k, as a drop-in for full attention.
 *
 * Conventions for every entry point below:
 *   - Layout is token-major and contiguous: Q and O are [N][Hq][d], K and V
 *     are [N][Hkv][d]; query head h reads KV head h / (Hq / Hkv).
 *   - Positions and blocks are 0-based: block i holds rows [i*B, (i+1)*B); a
 *     last partial block (B not dividing N) is only ever a query's own block.
 *   - All tensor and workspace pointers are DEVICE pointers on the current HIP
 *     device; problem structs are HOST pointers. The caller owns every buffer;
 *     the library never allocates, frees or synchronises.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     asynchronously; results are valid once the stream has been synchronised.
 *   - Inputs are read-only; outputs must not alias inputs or the workspace.
 *   - Calls return a status code and never throw. All argument checks run on
 *     the host before anything is enqueued, so an error leaves outputs and
 *     the workspace untouched and costs no HIP call.
 *   - Calls that overlap on one stream are ordered; calls that share one
 *     workspace on different streams race.
 */
#ifndef MOBA_H
#define MOBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported symbols (the library is built with hidden default visibility). */
#if defined(__GNUC__) || defined(__clang__)
#define MOBA_API __attribute__((visibility("default")))
#else
#define MOBA_API
#endif

/* Status codes. */
#define MOBA_OK 0
#define MOBA_ERR_INVALID_ARGUMENT 1 /* null pointer, sizes < 1, Hq % Hkv != 0, bad scale/dtype */
#define MOBA_ERR_UNSUPPORTED 2      /* valid but not compiled in (head_dim != 128, size limits) */
#define MOBA_ERR_WORKSPACE_TOO_SMALL 3
#define MOBA_ERR_HIP 4 /* a HIP launch/runtime error; text from moba_last_error() */

/* Element type of Q, K, V and O. */
typedef enum { MOBA_DTYPE_BF16 = 0, MOBA_DTYPE_F32 = 1 } moba_dtype_t;

/*
 * Block routing under grouped-query attention (PaperTrace section 5.5 asks
 * that the choice be stated: each query head routes on its own, or a head
 * group shares one routing).
 *   MOBA_ROUTING_PER_HEAD: every query head ranks the blocks with its own
 *     query against its KV head's block keys (the default).
 *   MOBA_ROUTING_SHARED: the Hq/Hkv query heads of a KV head share one
 *     selection, ranked by the group's summed gate score
 *     sum_h q_h . kbar_i = (sum_h q_h) . kbar_i (same ties rule); attention
 *     still uses each head's own query. The group query is summed in fp64
 *     (exact unless the group's values differ in magnitude by more than
 *     2^45); bf16 inputs are ranked by the certified matrix-core tier with
 *     the fp64 tier for the rows it cannot certify, fp32 inputs by the fp64
 *     tier, so the selection is the exact one either way.
 */
typedef enum { MOBA_ROUTING_PER_HEAD = 0, MOBA_ROUTING_SHARED = 1 } moba_routing_t;

typedef struct {
  int64_t seqlen;       /* N >= 1 */
  int32_t num_q_heads;  /* Hq >= 1 */
  int32_t num_kv_heads; /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;     /* d; 128 is compiled in */
  int32_t block_size;   /* B >= 1 */
  int32_t topk;         /* k >= 1, counting the own block; k >= ceil(N/B) = causal full attention */
  float scale;          /* finite and > 0; multiplies attention logits only (the gate is unscaled) */
  int32_t dtype;        /* moba_dtype_t of Q, K, V and O */
  int32_t routing;      /* moba_routing_t; 0 = per head */
  int32_t kv_heads_per_pass; /* 0: the library's choice; else 1..Hkv (see below) */
} moba_problem_t;

/*
 * Attention passes. After the selection, the history and own-block
 * attention (with the merge) run in passes over groups of
 * kv_heads_per_pass KV heads and their query heads; the workspace holds the
 * history partial results (one per selected history block, fp16 + fp32 in
 * bf16 problems, fp32 in fp32 ones) of one pass only. With 0 the library
 * takes the largest group whose partials fit 16 GiB (at least one KV head):
 * for the 1M-token, 32/8-head, k = 12 layer that is one KV head per pass,
 * ~12 GB of partials instead of ~96 GB. The result does not depend on the
 * pass size. Values outside [0, Hkv] give MOBA_ERR_INVALID_ARGUMENT. The
 * backward entry points and moba_debug_bucket ignore the field (one pass
 * over all heads).
 */

/*
 * Size limits of this library (MOBA_ERR_UNSUPPORTED beyond them):
 *   head_dim == 128; topk <= 32; ceil(N/B) - 1 <= 8192 history-capable blocks
 *   (for packed sequences: all their blocks together minus one);
 *   N * Hq * topk < 2^31; Hq / Hkv <= 64; bf16 only: ceil(N/B) * ceil(B/64) * 64
 *   < 16,909,320 (a KV head's packed V^T is addressed with 32-bit byte
 *   offsets; for packed sequences the blocks of all sequences count, for a
 *   decode cache its capacity does).
 * Value range: the bf16 path keeps normalised partial outputs in fp16, so
 * |V| must stay below 65504.
 */

/* Bytes of device workspace moba_prefill needs for *p; 0 if *p is invalid or unsupported. */
MOBA_API size_t moba_workspace_size(const moba_problem_t *p);

/* Bytes of device workspace moba_select needs for *p; 0 if *p is invalid or unsupported. */
MOBA_API size_t moba_select_workspace_size(const moba_problem_t *p);

/*
 * MoBA prefill forward: O = MoBA-attention(Q, K, V) as defined above.
 *   q  [N][Hq][d], k [N][Hkv][d], v [N][Hkv][d] (device, dtype of p)
 *   o  [N][Hq][d] (device, dtype of p), written in full
 *   workspace / ws_bytes: device scratch of at least moba_workspace_size(p)
 *     bytes, 256-byte aligned; contents on entry are ignored.
 * Numerics: bf16 inputs use bf16 matrix-core products with fp32 accumulation
 * and fp32 softmax statistics; block means and gate scores are fp64, so the
 * selection equals the exact one except where scores tie to fp64 rounding.
 * fp32 inputs use fp32 arithmetic throughout the attention.
 */
MOBA_API int moba_prefill(const moba_problem_t *p, const void *q, const void *k, const void *v, void *o,
                 void *workspace, size_t ws_bytes, void *stream);

/*
 * Number of stage events moba_prefill_ex records for *p: 5 + 2 x (attention
 * passes); 0 if *p is invalid or unsupported.
 */
MOBA_API size_t moba_stage_events(const moba_problem_t *p);

/*
 * moba_prefill with optional per-stage timing: if `events` is not NULL it
 * points to moba_stage_events(p) caller-created hipEvent_t handles, recorded
 * on `stream`: [0] before the first stage, then after each of [1] meanpool,
 * [2] gate_topk, [3] bucket, [4] the V layout pack (bf16 only; empty for
 * fp32), and for pass i: [5 + 2i] history attention, [6 + 2i] own-block
 * attention with merge. Otherwise identical to moba_prefill.
 */
MOBA_API int moba_prefill_ex(const moba_problem_t *p, const void *q, const void *k, const void *v, void *o,
                    void *workspace, size_t ws_bytes, void *stream, void *const *events);

/*
 * Block selection only (debug call): sel [N][Hq][topk] int32 (device), per
 * (row, head) the selected blocks in ascending order — the chosen earlier
 * blocks, then the own block — padded with -1.
 */
MOBA_API int moba_select(const moba_problem_t *p, const void *q, const void *k, int32_t *sel,
                void *workspace, size_t ws_bytes, void *stream);

/*
 * Packed variable-length batches. The N rows of q, k, v and o hold nseq
 * sequences back to back; sequence i is rows [cu[i], cu[i+1]). Every
 * sequence is cut into its own blocks from its first row, and a row only
 * sees blocks of its own sequence: block means, the gate, the top-k and the
 * attention never cross a sequence boundary (PaperTrace section 5.1: with
 * packed documents the blocks, their summaries and the gate must share the
 * document boundaries; section 3.1: variable-length attention kernels). The
 * result for each sequence is exactly moba_prefill on that sequence alone.
 *   nseq >= 1; cu_seqlens_host: HOST int64 [nseq + 1] with cu[0] = 0,
 *     nondecreasing (empty sequences allowed), cu[nseq] = p->seqlen;
 *   cu_seqlens_dev: the same values in DEVICE memory (8-byte aligned), read
 *     by the kernels; the caller keeps both copies equal.
 * The history-capable block limit applies to the blocks of all sequences
 * together. Selections (moba_select_varlen) hold global block ids: the
 * sequences' blocks are numbered consecutively in sequence order.
 */
MOBA_API size_t moba_varlen_workspace_size(const moba_problem_t *p, int64_t nseq,
                                           const int64_t *cu_seqlens_host);
MOBA_API size_t moba_varlen_select_workspace_size(const moba_problem_t *p, int64_t nseq,
                                                  const int64_t *cu_seqlens_host);
MOBA_API int moba_prefill_varlen(const moba_problem_t *p, int64_t nseq,
                                 const int64_t *cu_seqlens_host, const int64_t *cu_seqlens_dev,
                                 const void *q, const void *k, const void *v, void *o,
                                 void *workspace, size_t ws_bytes, void *stream);
MOBA_API int moba_select_varlen(const moba_problem_t *p, int64_t nseq,
                                const int64_t *cu_seqlens_host, const int64_t *cu_seqlens_dev,
                                const void *q, const void *k, int32_t *sel, void *workspace,
                                size_t ws_bytes, void *stream);

/*
 * Training: forward with saved statistics, and the backward pass.
 *   moba_prefill_train: moba_prefill plus lse [N][Hq] fp32 (DEVICE): each
 *     row's log2-sum-exp over its keys, lse = log2(sum_j 2^(c q.k_j)) with
 *     c = scale * log2(e), so its attention weights are 2^(c q.k_j - lse).
 *     Same workspace as moba_prefill.
 *   moba_backward: gradients of sum(dout * O) — dq [N][Hq][d], dk and dv
 *     [N][Hkv][d], in the dtype of p, overwritten — from q, k, v, the forward
 *     output o, its lse and dout [N][Hq][d]. The block selection is held
 *     fixed: the hard top-k passes no gradient to the ranking, so Q, K and V
 *     get gradients only through the attended pairs (PaperTrace section
 *     5.3); the selection is recomputed from q and k exactly as in the
 *     forward pass. Workspace: moba_backward_workspace_size(p).
 * Numerics: weights are rebuilt from lse. bf16 inputs run on the matrix
 * cores (fp32 accumulation, the weights P and dZ = P (dP - D) rounded to
 * bf16 as operands); dq sums per-slot partials, so results are
 * deterministic. fp32 inputs run in fp32 on the vector units and sum dq
 * with atomics (the last bits of dq may vary between runs).
 */
MOBA_API int moba_prefill_train(const moba_problem_t *p, const void *q, const void *k,
                                const void *v, void *o, float *lse, void *workspace,
                                size_t ws_bytes, void *stream);
MOBA_API size_t moba_backward_workspace_size(const moba_problem_t *p);
MOBA_API int moba_backward(const moba_problem_t *p, const void *q, const void *k, const void *v,
                           const void *o, const float *lse, const void *dout, void *dq,
                           void *dk, void *dv, void *workspace, size_t ws_bytes, void *stream);

/*
 * Training on packed sequences: moba_prefill_train and moba_backward for the
 * packed layout of moba_prefill_varlen (same nseq / cu_seqlens arguments and
 * rules). Each sequence's result equals the single-sequence call on that
 * sequence alone. Workspaces: moba_varlen_workspace_size (forward) and
 * moba_backward_varlen_workspace_size (backward).
 */
MOBA_API int moba_prefill_train_varlen(const moba_problem_t *p, int64_t nseq,
                                       const int64_t *cu_seqlens_host,
                                       const int64_t *cu_seqlens_dev, const void *q,
                                       const void *k, const void *v, void *o, float *lse,
                                       void *workspace, size_t ws_bytes, void *stream);
MOBA_API size_t moba_backward_varlen_workspace_size(const moba_problem_t *p, int64_t nseq,
                                                    const int64_t *cu_seqlens_host);
MOBA_API int moba_backward_varlen(const moba_problem_t *p, int64_t nseq,
                                  const int64_t *cu_seqlens_host, const int64_t *cu_seqlens_dev,
                                  const void *q, const void *k, const void *v, const void *o,
                                  const float *lse, const void *dout, void *dq, void *dk,
                                  void *dv, void *workspace, size_t ws_bytes, void *stream);

/*
 * Chunked prefill and decode: the queries are the last q_rows positions of
 * one sequence whose keys and values (all p->seqlen rows, the new ones
 * included) are already in k and v — a KV cache. q and o hold only those
 * q_rows rows: [q_rows][Hq][d]. Every output row equals the row at the same
 * position of moba_prefill over the whole sequence: a row never depends on
 * later rows, so a long prefill can be split into chunks, and q_rows = 1 is
 * one decode step (PaperTrace section 3.1 contrasts prefill and decode;
 * section 5.1 notes that generation needs block means kept up to date).
 * Block means are recomputed from k on every call; a generation loop keeps
 * them in a decode cache instead (moba_prefill_cached below).
 *   1 <= q_rows <= seqlen; the selection (moba_select_chunk) is
 *   [q_rows][Hq][topk]. The workspace of moba_chunk_workspace_size serves
 *   both calls.
 */
MOBA_API size_t moba_chunk_workspace_size(const moba_problem_t *p, int64_t q_rows);
MOBA_API int moba_prefill_chunk(const moba_problem_t *p, int64_t q_rows, const void *q,
                                const void *k, const void *v, void *o, void *workspace,
                                size_t ws_bytes, void *stream);
MOBA_API int moba_select_chunk(const moba_problem_t *p, int64_t q_rows, const void *q,
                               const void *k, int32_t *sel, void *workspace, size_t ws_bytes,
                               void *stream);

/*
 * Decode cache: the state a generation loop keeps for one sequence of at
 * most `capacity` rows, so that a chunk or decode step reads the block means
 * and the packed V copy instead of recomputing them from the whole KV cache
 * (PaperTrace section 5.1: generation needs the block means kept current as
 * tokens arrive; a full block's mean never changes, so each block's mean is
 * computed once, when the rows appended complete it).
 *   moba_cache_bytes(p, capacity): bytes of the cache (DEVICE, 256-byte
 *     aligned, caller-owned; no initialisation needed); p->seqlen is not
 *     used beyond validation. 0 if the problem or capacity is invalid.
 *     Holds fp64 means [Hkv][ceil(capacity/B) - 1][d] and, for bf16, the V
 *     copy [Hkv][d][ceil(capacity/B) * ceil(B/64) * 64].
 *   moba_cache_append(p, capacity, rows_before, k, v, cache, stream): k and
 *     v (the KV cache, [capacity][Hkv][d], rows [0, p->seqlen) valid) have
 *     gained rows [rows_before, p->seqlen); computes the means of the blocks
 *     those rows complete and packs those rows of V into the cache. Appends
 *     go in order: rows_before is the previous append's p->seqlen (0 for the
 *     first); 0 <= rows_before <= p->seqlen <= capacity. No workspace.
 *   moba_prefill_cached(p, capacity, q_rows, q, k, v, cache, o, workspace,
 *     ws_bytes, stream): moba_prefill_chunk (same arguments and result) with
 *     the block means and packed V taken from `cache`, which must hold every
 *     row of k and v up to p->seqlen. Workspace:
 *     moba_cached_workspace_size(p, q_rows) bytes.
 * Errors as elsewhere; capacity < p->seqlen is MOBA_ERR_INVALID_ARGUMENT.
 */
MOBA_API size_t moba_cache_bytes(const moba_problem_t *p, int64_t capacity);
MOBA_API int moba_cache_append(const moba_problem_t *p, int64_t capacity, int64_t rows_before,
                               const void *k, const void *v, void *cache, void *stream);
MOBA_API size_t moba_cached_workspace_size(const moba_problem_t *p, int64_t q_rows);
MOBA_API int moba_prefill_cached(const moba_problem_t *p, int64_t capacity, int64_t q_rows,
                                 const void *q, const void *k, const void *v, const void *cache,
                                 void *o, void *workspace, size_t ws_bytes, void *stream);

/*
 * Routing diagnostics (PaperTrace section 5.3: log the gap between the
 * k-th and (k+1)-th block scores, candidate overlap and per-block selection
 * frequency). Runs the block means and the exact (fp64) gate for every row
 * under p->routing, then fills whichever outputs are non-NULL (DEVICE):
 *   sel        int32 [N][Hq][topk]: the selection, as moba_select;
 *   margin     fp32 [N][Hq]: last kept minus best left-out history score
 *              (gate scores, unscaled), NaN where no history block is left
 *              out (topk == 1 or fewer earlier blocks than topk);
 *   counts     int32 [Hkv][ceil(N/B)]: how many (row, query head) pairs of
 *              each KV head selected each block as history;
 *   union_size int32 [N][Hkv]: distinct history blocks selected by the query
 *              heads of each KV head at each row (topk-1 under shared
 *              routing once enough blocks precede the row).
 * Workspace: moba_routing_stats_workspace_size(p) bytes.
 */
MOBA_API size_t moba_routing_stats_workspace_size(const moba_problem_t *p);
MOBA_API int moba_routing_stats(const moba_problem_t *p, const void *q, const void *k,
                                int32_t *sel, float *margin, int32_t *counts,
                                int32_t *union_size, void *workspace, size_t ws_bytes,
                                void *stream);

/*
 * Dense causal softmax attention on the same tensors (PaperTrace section 1,
 * eq. (1) with a causal mask): the full-attention baseline MoBA is measured
 * against. block_size and topk of *p are ignored. The workspace (device,
 * 256-byte aligned) holds a transposed copy of V for bf16 inputs.
 */
MOBA_API size_t moba_dense_workspace_size(const moba_problem_t *p);
MOBA_API int moba_dense_causal(const moba_problem_t *p, const void *q, const void *k, const void *v,
                               void *o, void *workspace, size_t ws_bytes, void *stream);

/*
 * Allocation-free prefill, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): moba_prefill with the workspace taken from a fixed device
 * array of the library (moba_noalloc_max_workspace() bytes, 512 MiB, one
 * per GPU, held until the process ends) instead of a caller buffer. Nothing
 * is allocated or freed by the call.
 *   q, k, v, o: as moba_prefill; stream: the caller's HIP stream.
 * Returns MOBA_ERR_UNSUPPORTED, before any HIP call, when
 * moba_workspace_size(p) exceeds the array. All calls on one GPU share its
 * array: calls that overlap on one GPU (other streams, or another host
 * thread) race and must be serialised by the caller. The array's contents on
 * entry are ignored (every kernel writes what it later reads).
 */
MOBA_API size_t moba_noalloc_max_workspace(void);
MOBA_API int moba_prefill_noalloc(const moba_problem_t *p, const void *q, const void *k,
                                  const void *v, void *o, void *stream);

/* Static text for a status code. */
MOBA_API const char *moba_status_string(int status);

/* Thread-local text of the last MOBA_ERR_HIP (or other error) on this thread. */
MOBA_API const char *moba_last_error(void);

/*
 * Stage-level debug exports (used by the tests to check one stage at a time).
 *   moba_debug_meanpool: kbar [Hkv][max(n-1,0)][d] fp64 (device) = block means
 *     of K (eq. (3)) for the blocks that can be history. workspace as for
 *     moba_select.
 *   moba_debug_bucket: from a selection sel [N][Hq][topk] (device), build the
 *     per-(KV head, block) lists: offsets [Hkv*(n-1)+1] int32 and entries
 *     uint32 (capacity moba_debug_bucket_capacity(p)); entry value
 *     ((row*Hq + head)*(topk-1) + slot), slot = position in the sel row.
 *     Lists are ordered by (row, head). workspace as for moba_prefill.
 *   moba_debug_copy: plain device copy of `bytes` bytes (a traffic calibration
 *     kernel for hardware counters, and the HBM stream probe: it moves
 *     2 * bytes through HBM per call). src and dst: device, 16-byte aligned,
 *     non-overlapping; bytes a multiple of 16.
 *   moba_debug_read_peak: read-only HBM stream probe (the measured
 *     denominator for read-bound stages): `workgroups` workgroups of 256
 *     threads read all `bytes` of src (device, 16-byte aligned, bytes a
 *     multiple of 16) once, 16 bytes per load, four loads in flight per
 *     thread; out: device, workgroups * 256 uint32 values whose XOR equals
 *     the XOR of every 32-bit word of src. workgroups in [1, 2^20], else
 *     MOBA_ERR_INVALID_ARGUMENT; nothing is allocated.
 *   moba_debug_mfma_peak: matrix-core issue-rate probe, the measured
 *     denominator beside the published bf16 peak. `workgroups` workgroups of
 *     four waves each run `iters` rounds of four v_mfma_f32_32x32x16_bf16 per
 *     wave on register operands: FLOP per call = workgroups * 4 * iters * 4 *
 *     32768. out: device fp32, workgroups * 256 values, one per lane, each
 *     exactly 16 * iters (a checksum that every op ran). workgroups and iters
 *     in [1, 2^20], else MOBA_ERR_INVALID_ARGUMENT; nothing is allocated.
 */
MOBA_API int moba_debug_meanpool(const moba_problem_t *p, const void *k, double *kbar, void *workspace,
                        size_t ws_bytes, void *stream);
MOBA_API size_t moba_debug_bucket_capacity(const moba_problem_t *p);
MOBA_API int moba_debug_bucket(const moba_problem_t *p, const int32_t *sel, int32_t *offsets,
                      uint32_t *entries, void *workspace, size_t ws_bytes, void *stream);
MOBA_API int moba_debug_copy(const void *src, void *dst, size_t bytes, void *stream);
MOBA_API int moba_debug_read_peak(const void *src, size_t bytes, int32_t workgroups, uint32_t *out,
                                  void *stream);
MOBA_API int moba_debug_mfma_peak(int32_t workgroups, int32_t iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H */
