// Expert histogram, scan and stable token permutation.
//
// The routed slots (t, j) are placed into expert-contiguous order, expert
// ascending and token ascending inside an expert, so that each expert's rows
// form one contiguous segment for the grouped expert products.  The pages
// route each token to its top-k experts ("Top-12 routing", skill card
// "Reversible Sparse MoE Single Node", Architecture Details) but say nothing
// of the data movement; the placement here is this library's design.
//
// Determinism without atomic ordering: inside a 256-token block every wave
// builds, per expert, a 64-bit mask of its lanes (tokens) that chose that
// expert (bitwise OR, order-free).  A slot's rank inside the block is the
// popcount of lower lanes in its own wave's mask plus the popcounts of the
// lower waves' masks; the scan then orders blocks.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PB = 256;  // tokens per histogram block

__global__ __launch_bounds__(PB) void perm_hist_kernel(const int32_t *__restrict__ idx, int Tn,
                                                       int E, int k,
                                                       int32_t *__restrict__ block_counts,
                                                       int32_t *__restrict__ rank) {
  extern __shared__ unsigned long long masks[];  // [4][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x * PB + tid;
  for (int i = tid; i < 4 * E; i += PB) masks[i] = 0ull;
  __syncthreads();
  if (t < Tn)
    for (int j = 0; j < k; ++j) atomicOr(&masks[wave * E + idx[(size_t)t * k + j]], 1ull << lane);
  __syncthreads();
  if (t < Tn) {
    const unsigned long long lower = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      int e = idx[(size_t)t * k + j];
      int r = __popcll(masks[wave * E + e] & lower);
      for (int w = 0; w < wave; ++w) r += __popcll(masks[w * E + e]);
      rank[(size_t)t * k + j] = r;
    }
  }
  for (int e = tid; e < E; e += PB) {
    int c = 0;
    for (int w = 0; w < 4; ++w) c += __popcll(masks[w * E + e]);
    block_counts[(size_t)blockIdx.x * E + e] = c;
  }
}

// One block of 1024 threads: per expert, exclusive scan of the block counts
// in block order (in place), the expert totals and their exclusive scan.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t *__restrict__ block_counts,
                                                         int nb, int E,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets) {
  __shared__ int32_t sc[1024];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int b = 0; b < nb; ++b) {
      int c = block_counts[(size_t)b * E + e];
      block_counts[(size_t)b * E + e] = run;
      run += c;
    }
    counts[e] = run;
  }
  sc[e] = e < E ? run : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over 1024 entries
  for (int off = 1; off < 1024; off <<= 1) {
    int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e] = sc[e] - run;
  if (e == E - 1) offsets[E] = sc[e];
}

__global__ void perm_scatter_kernel(const int32_t *__restrict__ idx, int S, int E, int k,
                                    const int32_t *__restrict__ block_off,
                                    const int32_t *__restrict__ offsets,
                                    const int32_t *__restrict__ rank,
                                    int32_t *__restrict__ perm_src, int32_t *__restrict__ slot_pos) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  int t = s / k, b = t / PB, e = idx[s];
  int p = offsets[e] + block_off[(size_t)b * E + e] + rank[s];
  perm_src[p] = s;
  slot_pos[s] = p;
}

// x_perm[p] = x[perm_src[p] / k]: one wave per row, 16-byte vectors.
__global__ void perm_copy_kernel(const uint4 *__restrict__ x, const int32_t *__restrict__ perm_src,
                                 int S, int k, int vec_per_row, uint4 *__restrict__ x_perm) {
  int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= S) return;
  int t = perm_src[p] / k;
  const uint4 *src = x + (size_t)t * vec_per_row;
  uint4 *dst = x_perm + (size_t)p * vec_per_row;
  for (int v = threadIdx.x & 63; v < vec_per_row; v += 64) dst[v] = src[v];
}

size_t permute_ws_bytes(int T, int E, int k) {
  size_t nb = (T + PB - 1) / PB;
  return nb * E * sizeof(int32_t) + (size_t)T * k * sizeof(int32_t) + 256;
}

void launch_permute(const int32_t *idx, int Tn, int E, int k, int32_t *counts, int32_t *offsets,
                    int32_t *perm_src, int32_t *slot_pos, const void *x, void *x_perm,
                    int row_bytes, void *ws, hipStream_t st) {
  int nb = (Tn + PB - 1) / PB;
  int S = Tn * k;
  int32_t *block_counts = (int32_t *)ws;
  int32_t *rank = (int32_t *)((char *)ws + (((size_t)nb * E * 4 + 255) & ~(size_t)255));
  perm_hist_kernel<<<nb, PB, 4 * E * sizeof(unsigned long long), st>>>(idx, Tn, E, k,
                                                                       block_counts, rank);
  perm_scan_kernel<<<1, 1024, 0, st>>>(block_counts, nb, E, counts, offsets);
  perm_scatter_kernel<<<(S + 255) / 256, 256, 0, st>>>(idx, S, E, k, block_counts, offsets, rank,
                                                       perm_src, slot_pos);
  if (x_perm)
    perm_copy_kernel<<<(S + 3) / 4, 256, 0, st>>>((const uint4 *)x, perm_src, S, k,
                                                  row_bytes / 16, (uint4 *)x_perm);
}

}  // namespace moe
