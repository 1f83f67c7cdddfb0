// Routing diagnostics (PaperTrace "2.1.3 MoBA", section 5.3: log the margin
// between the k-th and (k+1)-th block scores, the overlap of candidates and
// how often each block is selected). The margins come from the exact gate
// tier (run_gate with a margin output); this file holds the two reductions
// over a finished selection.
#include "moba_internal.hpp"

namespace moba {
namespace {

// counts[g][b] += 1 for every history selection of block b by a query head of
// KV head g (own blocks and -1 pads excluded).
__global__ void history_counts(const int32_t* __restrict__ sel,
                               const int32_t* __restrict__ row_blk, int32_t* __restrict__ counts,
                               int64_t N, int Hq, int G, int k, int64_t n) {
  const int64_t total = N * Hq;
  for (int64_t ph = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; ph < total;
       ph += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = row_blk[ph / Hq];
    const int g = (int)(ph % Hq) / G;
    for (int a = 0; a + 1 < k; ++a) {
      const int32_t b = sel[ph * k + a];
      if (b >= 0 && b < c) atomicAdd(&counts[(int64_t)g * n + b], 1);
    }
  }
}

// union_size[row][g] = number of distinct history blocks selected by the G
// query heads of KV head g at that row.
__global__ void group_union(const int32_t* __restrict__ sel, const int32_t* __restrict__ row_blk,
                            int32_t* __restrict__ union_size, int64_t N, int Hq, int G, int k) {
  const int Hkv = Hq / G;
  const int64_t total = N * Hkv;
  for (int64_t rg = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; rg < total;
       rg += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = rg / Hkv, c = row_blk[r];
    const int g = (int)(rg % Hkv);
    const int32_t* base = sel + (r * Hq + (int64_t)g * G) * k;
    int cnt = 0;
    for (int i = 0; i < G * (k - 1); ++i) {
      const int32_t b = base[(i / (k - 1)) * k + i % (k - 1)];
      if (b < 0 || b >= c) continue;
      bool seen = false;
      for (int j = 0; j < i && !seen; ++j) seen = base[(j / (k - 1)) * k + j % (k - 1)] == b;
      cnt += seen ? 0 : 1;
    }
    union_size[rg] = cnt;
  }
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  return (unsigned)(g > 0 ? g : 1);
}

}  // namespace

hipError_t launch_routing_reductions(const Prob& P, const Blocks& T, const int32_t* sel,
                                     int32_t* counts, int32_t* union_size, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (counts) {
    e = launch_fill_i32(counts, 0, (size_t)(P.Hkv * P.n), s);
    if (e != hipSuccess) return e;
    if (P.k > 1) {
      history_counts<<<grid_for(P.Nq * P.Hq), 256, 0, s>>>(sel, T.row_blk, counts, P.Nq, P.Hq, P.G,
                                                          P.k, P.n);
      e = hipGetLastError();
    }
  }
  if (e == hipSuccess && union_size) {
    if (P.k > 1) {
      group_union<<<grid_for(P.Nq * P.Hkv), 256, 0, s>>>(sel, T.row_blk, union_size, P.Nq, P.Hq,
                                                        P.G, P.k);
      e = hipGetLastError();
    } else {
      e = launch_fill_i32(union_size, 0, (size_t)(P.Nq * P.Hkv), s);
    }
  }
  return e;
}

}  // namespace moba
