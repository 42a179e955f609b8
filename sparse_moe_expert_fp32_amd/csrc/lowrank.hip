// Rank-r adapter products on the matrix cores.
//
// TQP trains low-rank adapters on top of the frozen expert base ("Reversible
// Sparse MoE Single Node" skill card, Principle 3; LoRA under Related
// Methods).  Besides the adapter term folded into the expert GEMMs, the layer
// needs the thin projections Z = X A^T (forward) and dZ = lam dOut B
// (backward), and the adapter gradients, which are per-expert reductions over
// that expert's rows:  out[e][a][b] = s * sum_p W[p][a] R[p][b]  with one wide
// operand W (x, H, dO, dG or dU) and one rank-wide operand R (Z or dZ).
//
// Both run bf16 operands with float32 accumulation.  The reductions keep a
// fixed row order (no atomics), so gradients are reproducible bit for bit.
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

// ------------------------------------------------------------ projections --
// Z_s[p][j] = scale * sum_k A(p, k) M_s[e][j][k] for sources s < nsrc, j < r.
// A(p, k) = a[(GATHER ? perm_src[p] / kk : p) * lda + k]; M_s is [E][r][K].
// One wave per 16 rows, 4 waves per 64-row tile of the tile list.
template <bool GATHER>
__global__ __launch_bounds__(256) void proj_mfma_kernel(const ProjMArgs P) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  if ((int)blockIdx.x >= P.ntiles[0]) return;
  const int2 tile = P.tiles[blockIdx.x];
  const int e = tile.x, p0 = tile.y + 16 * w;
  const int p_end = P.offsets[e + 1];
  if (p0 >= p_end) return;
  const int prow = min(p0 + lr, p_end - 1);
  const size_t arow = GATHER ? (size_t)(P.perm_src[prow] / P.kk) : (size_t)prow;
  const uint16_t *ap = P.a + arow * P.lda + 8 * lg;
  const int nj = (P.r + 15) >> 4;           // 16-column fragments per source
  const int nf = nj * P.nsrc;               // <= 4
  // fragment f covers rank columns 16*jf .. 16*jf+15 of source src
  const uint16_t *mp[4];
  bool mv[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int src = nj == 1 ? f : f >> 1;
    const int jf = nj == 1 ? 0 : f & 1;
    const int j = 16 * jf + lr;
    mv[f] = f < nf && j < P.r;
    const uint16_t *m = (f < nf && src == 1) ? P.m1 : P.m0;
    mp[f] = m + ((size_t)e * P.r + (mv[f] ? j : 0)) * P.K + 8 * lg;
  }
  f32x4_t acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint4 zero = {0u, 0u, 0u, 0u};
  for (int k0 = 0; k0 < P.K; k0 += 128) {
    uint4 av[4], bv[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      av[s] = *reinterpret_cast<const uint4 *>(ap + k0 + 32 * s);
#pragma unroll
      for (int f = 0; f < 4; ++f)
        bv[s][f] = mv[f] ? *reinterpret_cast<const uint4 *>(mp[f] + k0 + 32 * s) : zero;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int f = 0; f < 4; ++f)
        if (f < nf) acc[f] = mfma32(av[s], bv[s][f], acc[f]);
  }
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    if (f >= nf) continue;
    const int src = nj == 1 ? f : f >> 1;
    const int j = (nj == 1 ? 0 : 16 * (f & 1)) + lr;
    if (j >= P.r) continue;
    float *Z = src ? P.Z1 : P.Z0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + 4 * lg + i;
      if (p < p_end) Z[(size_t)p * P.ldz + j] = P.scale * acc[f][i];
    }
  }
}

// ------------------------------------------------------ adapter gradients --
// out[e*oe + a*oa + b*ob] = scale * sum_{p in expert e} W(p, a) R[p][b],
// a < wide, b < r.  One block per (64 wide columns, expert); rows of the
// expert in chunks of 32 (ascending): W staged in LDS row-major, R staged
// transposed as bf16; MFMA with K = rows.
constexpr int WG_LDW = 66;  // padded LDS row of 64 bf16 (conflict-free column reads)

template <bool GATHER>
__global__ __launch_bounds__(256) void wgrad_mfma_kernel(const WgradMArgs G) {
  __shared__ __attribute__((aligned(16))) uint16_t wl[32 * WG_LDW];
  __shared__ __attribute__((aligned(16))) uint16_t rl[32 * 32];   // [b][p]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int e = blockIdx.y, a0 = blockIdx.x * 64;
  const int lo = G.offsets[e], hi = G.offsets[e + 1];
  const int nj = (G.r + 15) >> 4;
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  // staging roles
  const int sw_row = tid >> 3, sw_ch = tid & 7;        // W: 32 rows x 8 chunks of 8
  const int sr_row = tid >> 3, sr_c4 = (tid & 7) * 4;  // R: 32 rows x 8 groups of 4
  for (int pc = lo; pc < hi; pc += 32) {
    {
      const int p = pc + sw_row;
      uint4 v = {0u, 0u, 0u, 0u};
      const int a = a0 + sw_ch * 8;
      if (p < hi && a < G.wide) {
        const size_t row = GATHER ? (size_t)(G.perm_src[p] / G.kk) : (size_t)p;
        v = *reinterpret_cast<const uint4 *>(G.w + row * G.ldw + a);
      }
      uint32_t *dst = reinterpret_cast<uint32_t *>(&wl[sw_row * WG_LDW + sw_ch * 8]);
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
    {
      const int p = pc + sr_row;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = sr_c4 + i;
        const float v = (p < hi && b < G.r) ? G.rr[(size_t)p * G.ldr + b] : 0.f;
        rl[b * 32 + sr_row] = f2bf(v);
      }
    }
    __syncthreads();
    uint4 av;
    {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = wl[(8 * lg + i) * WG_LDW + 16 * w + lr];
      av.x = h[0] | (h[1] << 16);
      av.y = h[2] | (h[3] << 16);
      av.z = h[4] | (h[5] << 16);
      av.w = h[6] | (h[7] << 16);
    }
#pragma unroll
    for (int jf = 0; jf < 2; ++jf) {
      if (jf >= nj) break;
      const uint4 bv = *reinterpret_cast<const uint4 *>(&rl[(16 * jf + lr) * 32 + 8 * lg]);
      acc[jf] = mfma32(av, bv, acc[jf]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int jf = 0; jf < 2; ++jf) {
    if (jf >= nj) break;
    const int b = 16 * jf + lr;
    if (b >= G.r) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = a0 + 16 * w + 4 * lg + i;
      if (a < G.wide) G.out[(size_t)e * G.oe + (size_t)a * G.oa + (size_t)b * G.ob] = G.scale * acc[jf][i];
    }
  }
}

// out[e][j][n] = in[e][n][j] for bf16 [E][N][r] -> [E][r][N]
__global__ void transpose_nr_kernel(const uint16_t *__restrict__ in, int E, int N, int r,
                                    uint16_t *__restrict__ out) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)E * N) return;
  const size_t e = i / N, n = i % N;
  for (int j = 0; j < r; ++j) out[(e * r + j) * N + n] = in[i * r + j];
}

void launch_proj_mfma(const ProjMArgs &P, int max_tiles, bool gather, hipStream_t st) {
  if (gather) proj_mfma_kernel<true><<<max_tiles, 256, 0, st>>>(P);
  else proj_mfma_kernel<false><<<max_tiles, 256, 0, st>>>(P);
}

void launch_wgrad_mfma(const WgradMArgs &G, bool gather, hipStream_t st) {
  dim3 grid((G.wide + 63) / 64, G.E);
  if (gather) wgrad_mfma_kernel<true><<<grid, 256, 0, st>>>(G);
  else wgrad_mfma_kernel<false><<<grid, 256, 0, st>>>(G);
}

void launch_transpose_nr(const void *in, int E, int N, int r, void *out, hipStream_t st) {
  size_t n = (size_t)E * N;
  transpose_nr_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>((const uint16_t *)in, E, N, r,
                                                                   (uint16_t *)out);
}

}  // namespace moe
