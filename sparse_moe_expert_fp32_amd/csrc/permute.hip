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

// Caller-supplied indices may be out of range or repeat within a token
// (the router always writes k distinct valid ones).  Each token's entries are
// first made canonical, in j order: an index outside [0, E) is clamped into
// range and an index a lower j already took is replaced by the lowest expert
// the token does not use yet (k <= E, so one exists).  Valid input passes
// through unchanged; invalid input still yields a bijective placement with
// every access inside the buffers.  canon[t k + j] holds the result.
//
// SINGLE (T <= 256, one block): the block also does what perm_scan_kernel and
// perm_scatter_kernel do for several blocks -- counts, offsets and the
// placement -- so a short batch is permuted in one launch.
template <bool SINGLE>
__global__ __launch_bounds__(PB) void perm_hist_kernel(const int32_t *__restrict__ idx, int Tn,
                                                       int E, int k,
                                                       int32_t *__restrict__ block_counts,
                                                       int32_t *__restrict__ rank,
                                                       int32_t *__restrict__ canon,
                                                       int32_t *__restrict__ counts,
                                                       int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ perm_src,
                                                       int32_t *__restrict__ slot_pos) {
  extern __shared__ unsigned long long masks[];  // [4][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x * PB + tid;
  for (int i = tid; i < 4 * E; i += PB) masks[i] = 0ull;
  // the token's canonical experts, held in registers (k <= 32: the loops
  // over j are unrolled, so every index into ce is a constant)
  int ce[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) ce[j] = 0;
  if (t < Tn) {
    const int32_t *it = idx + (size_t)t * k;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j >= k) break;
      int e = min(max(it[j], 0), E - 1);
      bool dup = false;
#pragma unroll
      for (int i = 0; i < j; ++i) dup |= ce[i] == e;
      if (dup) {   // (never for the router's output)
        for (e = 0;; ++e) {
          bool u = false;
#pragma unroll
          for (int i = 0; i < j; ++i) u |= ce[i] == e;
          if (!u) break;
        }
      }
      ce[j] = e;
      canon[(size_t)t * k + j] = e;
    }
  }
  __syncthreads();
  if (t < Tn) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j >= k) break;
      atomicOr(&masks[wave * E + ce[j]], 1ull << lane);
    }
  }
  __syncthreads();
  int rk[32];   // (SINGLE: the ranks stay in registers)
  if (t < Tn) {
    const unsigned long long lower = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j >= k) break;
      const int e = ce[j];
      int r = __popcll(masks[wave * E + e] & lower);
      for (int w = 0; w < wave; ++w) r += __popcll(masks[w * E + e]);
      if (SINGLE) rk[j] = r;
      else rank[(size_t)t * k + j] = r;
    }
  }
  if (!SINGLE) {
    for (int e = tid; e < E; e += PB) {
      int c = 0;
      for (int w = 0; w < 4; ++w) c += __popcll(masks[w * E + e]);
      block_counts[(size_t)blockIdx.x * E + e] = c;
    }
    return;
  }
  // counts and their exclusive scan: thread tid takes experts 4 tid .. 4 tid + 3
  // (E <= 4 PB), then a scan of the per-thread sums
  __shared__ int tot[PB];
  __shared__ int off_lds[4 * PB];
  int c4[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    int c = 0;
    if (e < E)
      for (int w = 0; w < 4; ++w) c += __popcll(masks[w * E + e]);
    c4[q] = c;
    sum += c;
  }
  tot[tid] = sum;
  __syncthreads();
  for (int off = 1; off < PB; off <<= 1) {   // Hillis-Steele inclusive scan
    const int v = tid >= off ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  int run = tot[tid] - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    if (e < E) {
      counts[e] = c4[q];
      offsets[e] = run;
      off_lds[e] = run;
    }
    run += c4[q];
  }
  if (tid == PB - 1) offsets[E] = tot[PB - 1];
  __syncthreads();
  if (t < Tn) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j >= k) break;
      const int s = t * k + j, p = off_lds[ce[j]] + rk[j];
      perm_src[p] = s;
      slot_pos[s] = p;
    }
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

__global__ void perm_scatter_kernel(const int32_t *__restrict__ canon, int S, int E, int k,
                                    const int32_t *__restrict__ block_off,
                                    const int32_t *__restrict__ offsets,
                                    const int32_t *__restrict__ rank,
                                    int32_t *__restrict__ perm_src, int32_t *__restrict__ slot_pos) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  int t = s / k, b = t / PB, e = canon[s];
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

// workspace: block counts [nb][E] | rank [S] | canonical indices [S], each
// 256-byte aligned
size_t permute_ws_bytes(int T, int E, int k) {
  const size_t nb = (T + PB - 1) / PB, S = (size_t)T * k;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return al(nb * E * sizeof(int32_t)) + al(S * sizeof(int32_t)) + al(S * sizeof(int32_t));
}

void launch_permute(const int32_t *idx, int Tn, int E, int k, int32_t *counts, int32_t *offsets,
                    int32_t *perm_src, int32_t *slot_pos, const void *x, void *x_perm,
                    int row_bytes, void *ws, hipStream_t st) {
  int nb = (Tn + PB - 1) / PB;
  int S = Tn * k;
  int32_t *block_counts = (int32_t *)ws;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  int32_t *rank = (int32_t *)((char *)ws + al((size_t)nb * E * 4));
  int32_t *canon = (int32_t *)((char *)rank + al((size_t)S * 4));
  const size_t lds = 4 * E * sizeof(unsigned long long);
  if (nb == 1) {
    perm_hist_kernel<true><<<1, PB, lds, st>>>(idx, Tn, E, k, block_counts, rank, canon, counts,
                                               offsets, perm_src, slot_pos);
  } else {
    perm_hist_kernel<false><<<nb, PB, lds, st>>>(idx, Tn, E, k, block_counts, rank, canon,
                                                 nullptr, nullptr, nullptr, nullptr);
    perm_scan_kernel<<<1, 1024, 0, st>>>(block_counts, nb, E, counts, offsets);
    perm_scatter_kernel<<<(S + 255) / 256, 256, 0, st>>>(canon, S, E, k, block_counts, offsets,
                                                         rank, perm_src, slot_pos);
  }
  if (x_perm)
    perm_copy_kernel<<<(S + 3) / 4, 256, 0, st>>>((const uint4 *)x, perm_src, S, k,
                                                  row_bytes / 16, (uint4 *)x_perm);
}

}  // namespace moe
