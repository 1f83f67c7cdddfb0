// Block and row tables of a (possibly packed) problem. Each sequence is cut
// into contiguous blocks of B rows from its own first row (PaperTrace
// "2.1.3 MoBA", section 1 eq. (2)); sequences never share a block, and a
// row's candidates are the earlier blocks of its own sequence: with packed
// sequences the blocks, their means and the gate must all stop at document
// boundaries (section 5.1), as the variable-length kernels of section 3.1 do.
// Global block ids run over the sequences in order.
#include "moba_internal.hpp"

namespace moba {
namespace {

// Row offset of sequence s: cu[s], or the one sequence [0, N) when cu is NULL.
__device__ inline int64_t cu_at(const int64_t* cu, int64_t s, int64_t N) {
  return cu ? cu[s] : (s == 0 ? 0 : N);
}

// seq_base[s] = first block of sequence s (exclusive scan of its block
// counts), seq_base[nseq] = all blocks. One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void seq_block_base(const int64_t* __restrict__ cu,
                                                       int64_t nseq, int64_t N, int B,
                                                       int32_t* __restrict__ seq_base) {
  __shared__ int32_t sc[1024];
  __shared__ int32_t carry;
  const int t = threadIdx.x;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < nseq; base += 1024) {
    const int64_t s = base + t;
    int32_t v = 0;
    if (s < nseq) v = (int32_t)((cu_at(cu, s + 1, N) - cu_at(cu, s, N) + B - 1) / B);
    sc[t] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
      const int32_t a = t >= off ? sc[t - off] : 0;
      __syncthreads();
      sc[t] += a;
      __syncthreads();
    }
    if (s < nseq) seq_base[s] = carry + sc[t] - v;
    __syncthreads();
    if (t == 1023) carry += sc[1023];
    __syncthreads();
  }
  if (t == 0) seq_base[nseq] = carry;
}

// Largest s in [0, nseq) with key(s) <= x, for a nondecreasing key.
template <typename F>
__device__ inline int64_t last_le(F key, int64_t nseq, int64_t x) {
  int64_t lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (key(mid) <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Query rows are positions [q0, q0 + Nq) (all rows for a full prefill).
__global__ void block_rows(const int64_t* __restrict__ cu, const int32_t* __restrict__ seq_base,
                           int64_t nseq, int64_t N, int B, int64_t nblk, int64_t q0, int64_t Nq,
                           int32_t* __restrict__ start, int32_t* __restrict__ len,
                           int32_t* __restrict__ lo, int32_t* __restrict__ qstart,
                           int32_t* __restrict__ qlen, int32_t* __restrict__ qpos) {
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    // empty sequences share their base with the next one: the last match owns b
    const int64_t s = last_le([&](int64_t i) { return (int64_t)seq_base[i]; }, nseq, b);
    const int64_t r0 = cu_at(cu, s, N) + (b - seq_base[s]) * (int64_t)B;
    const int64_t r1 = cu_at(cu, s + 1, N);
    const int64_t re = r1 < r0 + B ? r1 : r0 + B;  // end of the block's rows
    start[b] = (int32_t)r0;
    len[b] = (int32_t)(re - r0);
    lo[b] = seq_base[s];
    const int64_t a = r0 > q0 ? r0 : q0;  // first query position in the block
    const int64_t e = re < q0 + Nq ? re : q0 + Nq;
    qpos[b] = (int32_t)a;
    qstart[b] = (int32_t)(a - q0);
    qlen[b] = (int32_t)(e > a ? e - a : 0);
  }
}

__global__ void row_blocks(const int64_t* __restrict__ cu, const int32_t* __restrict__ seq_base,
                           int64_t nseq, int64_t N, int B, int64_t q0, int64_t Nq,
                           int32_t* __restrict__ row_blk) {
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < Nq;
       r += (int64_t)gridDim.x * blockDim.x) {
    const int64_t pos = q0 + r;
    const int64_t s = last_le([&](int64_t i) { return cu_at(cu, i, N); }, nseq, pos);
    row_blk[r] = (int32_t)(seq_base[s] + (pos - cu_at(cu, s, N)) / B);
  }
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  return (unsigned)(g > 0 ? g : 1);
}

}  // namespace

hipError_t launch_tables(const Prob& P, const int64_t* cu, const Blocks& t, hipStream_t s) {
  seq_block_base<<<1, 1024, 0, s>>>(cu, P.nseq, P.N, P.B, t.seq_base);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  block_rows<<<grid_for(P.n), 256, 0, s>>>(cu, t.seq_base, P.nseq, P.N, P.B, P.n, P.q0, P.Nq,
                                          t.start, t.len, t.lo, t.qstart, t.qlen, t.qpos);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  row_blocks<<<grid_for(P.Nq), 256, 0, s>>>(cu, t.seq_base, P.nseq, P.N, P.B, P.q0, P.Nq,
                                           t.row_blk);
  return hipGetLastError();
}

}  // namespace moba
