// Few -> many expert growth: every expert of the grown layer is a copy of one
// of the original experts, and the router is re-initialised around the copied
// columns ("Reversible Sparse MoE Single Node" skill card, Principle 2
// "State-Preserving Growth": few to many, duplicate experts and reinitialise
// routing; Pattern 2 "State-Preserving Expansion").
//
// Grown expert e F + c (c = 0 .. F-1) is original expert e.  With unperturbed
// router columns and F k experts per token the grown layer computes the same
// function: the F copies of each selected expert tie, are all selected, and
// share its gate equally.  Copies c >= 1 get their router column moved by
// s * z (caller-drawn z), which breaks the ties so the copies can diverge.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

// dst block e F + c = src block e; VEC: 16-byte units (sizes and pointers
// 16-byte aligned), else bytes.  One thread per unit of the destination.
template <bool VEC>
__global__ __launch_bounds__(256) void grow_copy_kernel(const uint8_t *__restrict__ src,
                                                        uint8_t *__restrict__ dst, size_t units,
                                                        int F, size_t total) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t o = (size_t)blockIdx.x * 256 + threadIdx.x; o < total; o += stride) {
    const size_t blk = o / units, u = o - blk * units;
    const size_t s = (blk / F) * units + u;
    if (VEC)
      reinterpret_cast<uint4 *>(dst)[o] = reinterpret_cast<const uint4 *>(src)[s];
    else
      dst[o] = src[s];
  }
}

void launch_grow_copy(const void *src, void *dst, size_t block_bytes, int E, int F,
                      hipStream_t st) {
  const bool vec = ((block_bytes | (uintptr_t)src | (uintptr_t)dst) & 15) == 0;
  const size_t units = vec ? block_bytes / 16 : block_bytes;
  const size_t total = units * (size_t)E * F;
  const unsigned grid = (unsigned)std::max<size_t>(1, std::min<size_t>((total + 255) / 256, 16384));
  if (vec)
    grow_copy_kernel<true><<<grid, 256, 0, st>>>((const uint8_t *)src, (uint8_t *)dst, units, F,
                                                 total);
  else
    grow_copy_kernel<false><<<grid, 256, 0, st>>>((const uint8_t *)src, (uint8_t *)dst, units, F,
                                                  total);
}

// w_out[i][e F + c] = w[i][e] (+ s * z[i][e F + c] for c >= 1, one rounding),
// b_out[e F + c] = b[e].  One thread per output column, block rows striding
// over the rows of w.
__global__ __launch_bounds__(256) void grow_router_kernel(const float *__restrict__ w,
                                                          const float *__restrict__ b,
                                                          const float *__restrict__ z, float s,
                                                          int d, int E, int F,
                                                          float *__restrict__ w_out,
                                                          float *__restrict__ b_out) {
  const int EF = E * F;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= EF) return;
  const int e = j / F, c = j - e * F;
  for (int i = blockIdx.y; i < d; i += gridDim.y) {   // rows of w
    const float v = w[(size_t)i * E + e];
    w_out[(size_t)i * EF + j] = (c > 0 && z) ? fmaf(s, z[(size_t)i * EF + j], v) : v;
  }
  if (blockIdx.y == 0 && b) b_out[j] = b[e];
}

void launch_grow_router(const float *w, const float *b, const float *z, float s, int d, int E,
                        int F, float *w_out, float *b_out, hipStream_t st) {
  dim3 grid((E * F + 255) / 256, std::min(d, 4096));
  grow_router_kernel<<<grid, 256, 0, st>>>(w, b, z, s, d, E, F, w_out, b_out);
}

}  // namespace moe
