// Batched set-up launch: the independent small jobs of one call (tile lists,
// group row sums, rank-16 adapter transposes) run as one grid instead of one
// launch each, so that short calls do not pay a launch per job.  Each job
// owns a contiguous range of the 1024-thread blocks.
#include <cstdio>
#include <cstdlib>

#include "common.h"
#include "kernels.h"
#include "prep.h"

namespace moe {

__global__ __launch_bounds__(1024) void prep_kernel(const PrepBatch B) {
  // the block's job (a uniform choice; constant indices into the argument)
  PrepBatch::Job J{};
  int lb = -1, base = 0;
#pragma unroll
  for (int j = 0; j < PrepBatch::kMax; ++j) {
    const int nb = j < B.n ? B.job[j].nblocks : 0;
    if ((int)blockIdx.x >= base && (int)blockIdx.x < base + nb) {
      J = B.job[j];
      lb = (int)blockIdx.x - base;
    }
    base += nb;
  }
  if (lb < 0) return;
  const int tid = threadIdx.x;
  switch (J.kind) {
    case PrepBatch::kTiles:
      build_tiles_body(J.offsets, J.E, J.BM, J.tiles, J.ntiles, J.first, J.nzero);
      break;
    case PrepBatch::kRowsum:
      group_rowsum_elem((size_t)lb * 1024 + tid, (const bf16_t *)J.src, J.rows, J.K, J.G, J.scale,
                        (float *)J.dst, J.split != 0, J.scale2);
      break;
    case PrepBatch::kTransposeNR16: {
      // four units of (256 columns, expert) per block
      const int units = (J.N + 255) / 256;
      const int u = lb * 4 + (tid >> 8);
      const int e = u / units, n = (u - e * units) * 256 + (tid & 255);
      if (e >= J.E) break;
      transpose_nr16_elem((const uint16_t *)J.src, J.N, e, n, (uint16_t *)J.dst);
      break;
    }
    case PrepBatch::kTransposeF32: {
      const int tcols = (J.K + 31) / 32;   // K: the input's columns
      const int ty = lb / tcols;
      transpose_f32_tile((const float *)J.src, J.rows, J.K, (float *)J.dst, (lb - ty * tcols) * 32,
                         ty * 32);
      break;
    }
    default:
      break;
  }
}

PrepBatch::Job &PrepBatch::next() {
  if (n >= kMax) {
    fprintf(stderr, "moe_tqp: more than %d set-up jobs in one batch\n", kMax);
    abort();
  }
  job[n] = Job{};
  return job[n++];
}

void PrepBatch::tiles(const int32_t *offsets, int E, int BM, int2 *tl, int *nt, int *first,
                      int nzero) {
  Job &J = next();
  J.kind = kTiles; J.nblocks = 1;
  J.offsets = offsets; J.E = E; J.BM = BM; J.tiles = tl; J.ntiles = nt; J.first = first;
  J.nzero = nzero;
}

void PrepBatch::rowsum(const void *a, int rows, int K, int G, float scale, float *out, bool split,
                       float scale2) {
  Job &J = next();
  const size_t elems = (size_t)rows * (K / G);
  J.kind = kRowsum; J.nblocks = (int)((elems + 1023) / 1024);
  J.src = a; J.dst = out; J.rows = rows; J.K = K; J.G = G; J.scale = scale; J.scale2 = scale2;
  J.split = split;
}

void PrepBatch::transpose_nr(const void *in, int E, int N, int r, void *out, hipStream_t st) {
  if (r != 16 || ((uintptr_t)in & 15) != 0) {    // (16-byte loads)
    launch_transpose_nr(in, E, N, r, out, st);
    return;
  }
  Job &J = next();
  J.kind = kTransposeNR16; J.nblocks = (E * ((N + 255) / 256) + 3) / 4;
  J.src = in; J.dst = out; J.E = E; J.N = N;
}

void PrepBatch::transpose_f32(const float *in, int rows, int cols, float *out) {
  Job &J = next();
  J.kind = kTransposeF32; J.nblocks = ((rows + 31) / 32) * ((cols + 31) / 32);
  J.src = in; J.dst = out; J.rows = rows; J.K = cols;
}

void launch_prep(const PrepBatch &b, hipStream_t st) {
  int blocks = 0;
  for (int j = 0; j < b.n; ++j) blocks += b.job[j].nblocks;
  if (blocks > 0) prep_kernel<<<blocks, 1024, 0, st>>>(b);
}

}  // namespace moe
