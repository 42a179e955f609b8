// Bodies of the small set-up kernels (tile lists, group row sums, rank-16
// adapter transposes), shared by their own kernels and by the batched set-up
// launch of prep.hip, which runs the independent ones of a call together.
#pragma once
#include "common.h"

namespace moe {

// Tile list of a grouped product: each expert's rows in tiles of BM (the last
// one partial), expert order.  One block of 1024 threads (E <= 1024).
// first (optional, 2E + 1 ints): index of each expert's first tile, then the
// number of experts not covered by exactly one tile (empty or split), then
// those experts in ascending order.  ntiles[1 .. nzero-1] are zeroed (work
// counters of the products that read the list).
DEV void build_tiles_body(const int32_t *__restrict__ offsets, int E, int BM,
                          int2 *__restrict__ tiles, int *__restrict__ ntiles,
                          int *__restrict__ first_out, int nzero) {
  __shared__ int sc[1024];
  const int e = threadIdx.x;
  if (e >= 1 && e < nzero) ntiles[e] = 0;
  int c = 0, lo = 0;
  if (e < E) {
    lo = offsets[e];
    c = (offsets[e + 1] - lo + BM - 1) / BM;
  }
  sc[e] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  int first = sc[e] - c;
  for (int i = 0; i < c; ++i) tiles[first + i] = make_int2(e, lo + i * BM);
  if (first_out && e < E) first_out[e] = first;
  if (e == 1023) ntiles[0] = sc[e];
  if (!first_out) return;
  __syncthreads();
  const int f = e < E && c != 1 ? 1 : 0;
  sc[e] = f;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (f) first_out[E + sc[e]] = e;   // position 1 + (exclusive prefix)
  if (e == 1023) first_out[E] = sc[e];
}

// Element i of the group row sums of a bf16 matrix [rows][K], groups of G
// along K: out[i] = scale * sum of group i % ng of row i / ng (ng = K / G).
// split: out has 2 ng entries per row, scale * sum then scale2 * sum.
DEV void group_rowsum_elem(size_t i, const bf16_t *__restrict__ a, int rows, int K, int G,
                           float scale, float *__restrict__ out, bool split, float scale2) {
  const int ng = K / G;
  if (i >= (size_t)rows * ng) return;
  const size_t row = i / ng;
  const int g = (int)(i % ng);
  const uint4 *p = reinterpret_cast<const uint4 *>(a + row * K + (size_t)g * G);
  float s = 0.f;
  auto add = [&](const uint4 u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s += __uint_as_float(w[j] << 16);
      s += __uint_as_float(w[j] & 0xFFFF0000u);
    }
  };
  if (G == 128) {   // (all of the group's loads in flight together)
    uint4 u[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) u[v] = p[v];
#pragma unroll
    for (int v = 0; v < 16; ++v) add(u[v]);
  } else {
    for (int v = 0; v < G / 8; ++v) add(p[v]);
  }
  if (split) {
    out[row * 2 * ng + g] = scale * s;
    out[row * 2 * ng + ng + g] = scale2 * s;
  } else {
    out[i] = scale * s;
  }
}

// Rank-16 adapter transpose of a bf16 matrix, one column n of expert e per
// thread (16-byte loads on the [E][N][16] side, which must be 16-byte
// aligned): nr16 [E][N][16] -> [E][16][N].
DEV void transpose_nr16_elem(const uint16_t *__restrict__ in, int N, int e, int n,
                             uint16_t *__restrict__ out) {
  if (n >= N) return;
  const uint4 *src = reinterpret_cast<const uint4 *>(in + ((size_t)e * N + n) * 16);
  const uint4 a = src[0], b = src[1];
  const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint16_t *dst = out + (size_t)e * 16 * N + n;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    dst[(2 * j) * (size_t)N] = (uint16_t)(v[j] & 0xFFFFu);
    dst[(2 * j + 1) * (size_t)N] = (uint16_t)(v[j] >> 16);
  }
}

// out [cols][rows] = in [rows][cols] transposed, float32: the 32 x 32 tile
// whose first input row is by and first input column bx, through LDS (any
// block size that is a multiple of 32).
DEV void transpose_f32_tile(const float *__restrict__ in, int rows, int cols,
                            float *__restrict__ out, int bx, int by) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5, ny = blockDim.x >> 5;
  for (int i = ty; i < 32; i += ny) {
    const int r = by + i, c = bx + tx;
    tile[i][tx] = (r < rows && c < cols) ? in[(size_t)r * cols + c] : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += ny) {
    const int r = bx + i, c = by + tx;  // out row = input column
    if (r < cols && c < rows) out[(size_t)r * rows + c] = tile[tx][i];
  }
}

}  // namespace moe
