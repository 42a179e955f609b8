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
// fixed order (no atomics), so results are reproducible bit for bit.
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

// ------------------------------------------------------------ projections --
// Z_s[p][j] = scale * sum_k A(p, k) M_s[e][j][k] for sources s < nsrc, j < r.
// A(p, k) = a[(GATHER ? perm_src[p] / kk : p) * lda + k]; M_s is [E][r][K].
// One block per 64-row tile of the tile list.  The reduction is split over
// the four waves (wave w takes the 64-wide k-chunks w, w + 4, ...), so each
// block reads its rows and the expert's M once; each wave holds the whole
// 64 x (16 nf) partial, and the partials are summed through LDS in wave order.
constexpr int PJ_KC = 64;

template <bool GATHER>
__global__ __launch_bounds__(256) void proj_mfma_kernel(const ProjMArgs P) {
  __shared__ float red[3][16 * 4 * 64];   // partials of waves 1..3: [m*4+f][i][lane]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  if ((int)blockIdx.x >= P.ntiles[0]) return;
  const int2 tile = P.tiles[blockIdx.x];
  const int e = tile.x, p0 = tile.y;
  const int p_end = P.offsets[e + 1];
  const int nj = (P.r + 15) >> 4;           // 16-column fragments per source
  const int nf = nj * P.nsrc;               // <= 4
  // rows: fragment m covers rows p0 + 16 m .. +15 (clamped to the expert)
  const uint16_t *ap[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int prow = min(p0 + 16 * m + lr, p_end - 1);
    const size_t arow = GATHER ? (size_t)(P.perm_src[prow] / P.kk) : (size_t)prow;
    ap[m] = P.a + arow * P.lda + 8 * lg;
  }
  // columns: fragment f covers rank columns 16 jf .. 16 jf + 15 of source src
  const uint16_t *mp[4];
  bool mv[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int src = nj == 1 ? f : f >> 1;
    const int jf = nj == 1 ? 0 : f & 1;
    const int j = 16 * jf + lr;
    mv[f] = f < nf && j < P.r;
    const uint16_t *mm = (f < nf && src == 1) ? P.m1 : P.m0;
    mp[f] = mm + ((size_t)e * P.r + (mv[f] ? j : 0)) * P.K + 8 * lg;
  }
  f32x4_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint4 zero = {0u, 0u, 0u, 0u};
  for (int k0 = w * PJ_KC; k0 < P.K; k0 += 4 * PJ_KC) {
    uint4 av[4][2], bv[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int m = 0; m < 4; ++m) av[m][s] = *reinterpret_cast<const uint4 *>(ap[m] + k0 + 32 * s);
#pragma unroll
      for (int f = 0; f < 4; ++f)
        bv[s][f] = mv[f] ? *reinterpret_cast<const uint4 *>(mp[f] + k0 + 32 * s) : zero;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (f >= nf) continue;
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m][f] = mfma32(av[m][s], bv[s][f], acc[m][f]);
      }
  }
  // partial sums of waves 1..3 to LDS, summed by wave 0 in wave order
  if (w > 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (f >= nf) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w - 1][((m * 4 + f) * 4 + i) * 64 + lane] = acc[m][f][i];
      }
  }
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    if (f >= nf) continue;
    const int src = nj == 1 ? f : f >> 1;
    const int j = (nj == 1 ? 0 : 16 * (f & 1)) + lr;
    float *Z = src ? P.Z1 : P.Z0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = ((m * 4 + f) * 4 + i) * 64 + lane;
        const float v = ((acc[m][f][i] + red[0][o]) + red[1][o]) + red[2][o];
        const int p = p0 + 16 * m + 4 * lg + i;
        if (j < P.r && p < p_end) Z[(size_t)p * P.ldz + j] = P.scale * v;
      }
  }
}

// ------------------------------------------------------ adapter gradients --
// out_s[e*oe + a*oa + b*ob] = scale * sum_{p in expert e} W(p, a) R_s[p][b],
// a < wide, b < r, for one or two R sources sharing W.
//
// Work items are (256-row tile of an expert, 256 wide columns), so a heavily
// loaded expert is spread over many blocks.  An expert that fits one tile
// writes its result directly; otherwise each tile writes an unscaled partial
// and a second kernel sums the partials in tile order (deterministic, no
// atomics).  Inside a tile the rows go in ascending chunks of 64.  MFMA
// operands need 8 consecutive rows per lane, so W is transposed on the way
// into LDS: each thread loads an 8 row x 8 column bf16 block and transposes it
// in registers (v_perm), storing each column's 8 rows as one 16-byte LDS
// chunk ([row octet][column], column index XOR-swizzled); R is staged
// transposed as bf16.  D = R^T W: A operand rows are rank columns, B operand
// columns are wide columns.
constexpr int WG_COLS = 256, WG_ROWS = 64, WG_TILE = 256;

DEV int wg_sw(int c) { return c ^ ((c >> 3) & 7); }

template <bool GATHER>
__global__ __launch_bounds__(256) void wgrad_mfma_kernel(const WgradMArgs G) {
  __shared__ uint4 wl[WG_ROWS / 8][WG_COLS];                          // 32 KB
  __shared__ __attribute__((aligned(16))) uint16_t rl[2][32][WG_ROWS + 8];
  const int ti = blockIdx.y;
  if (ti >= G.ntiles[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int2 tile = G.tiles[ti];
  const int e = tile.x, p0 = tile.y, a0 = blockIdx.x * WG_COLS;
  const int lo_e = G.offsets[e], hi_e = G.offsets[e + 1];
  const int hi = min(p0 + WG_TILE, hi_e);
  const bool single = hi_e - lo_e <= WG_TILE;
  const int nj = (G.r + 15) >> 4, nm = nj * G.nsrc;   // A fragments (<= 4)
  f32x4_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // staging role: row octet oct, columns a0 + 8 cg .. + 7
  const int oct = tid >> 5, cg = tid & 31;
  const bool col_ok = a0 + 8 * cg < G.wide;   // wide is a multiple of 8
  const int rcols = nj * 16 * G.nsrc;         // 16, 32 or 64
  const int rper = rcols >> 2;                // R values per thread and chunk (<= 16)
  for (int pc = p0; pc < hi; pc += WG_ROWS) {
    // issue every load of the chunk first: W block, then R values
    uint4 in[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = min(pc + 8 * oct + i, hi - 1);   // rows past the end meet R = 0
      const size_t row = GATHER ? (size_t)(G.perm_src[p] / G.kk) : (size_t)p;
      in[i] = col_ok ? *reinterpret_cast<const uint4 *>(G.w + row * G.ldw + a0 + 8 * cg)
                     : uint4{0u, 0u, 0u, 0u};
    }
    float rv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      rv[u] = 0.f;
      if (u < rper) {
        const int idx = tid + 256 * u, pp = idx / rcols, cc = idx - pp * rcols;
        const int src = cc / (nj * 16), b = cc - src * nj * 16;
        const int p = min(pc + pp, hi - 1);
        const float *R = src ? G.rr1 : G.rr;
        rv[u] = R[(size_t)p * G.ldr + min(b, G.r - 1)];
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u < rper) {
        const int idx = tid + 256 * u, pp = idx / rcols, cc = idx - pp * rcols;
        const int src = cc / (nj * 16), b = cc - src * nj * 16;
        rl[src][b][pp] = f2bf(pc + pp < hi && b < G.r ? rv[u] : 0.f);
      }
    }
    // 8 x 8 transpose of 16-bit elements: column j gets rows 0..7
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      auto dw = [&](int i) {
        const uint4 v = in[i];
        return (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
      };
      uint4 o;
      o.x = __builtin_amdgcn_perm(dw(1), dw(0), sel);
      o.y = __builtin_amdgcn_perm(dw(3), dw(2), sel);
      o.z = __builtin_amdgcn_perm(dw(5), dw(4), sel);
      o.w = __builtin_amdgcn_perm(dw(7), dw(6), sel);
      wl[oct][wg_sw(8 * cg + j)] = o;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 bw[4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) bw[nf] = wl[4 * s + lg][wg_sw(64 * w + 16 * nf + lr)];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m >= nm) break;
        const int src = m / nj, b = 16 * (m - src * nj) + lr;
        const uint4 ar = *reinterpret_cast<const uint4 *>(&rl[src][b][32 * s + 8 * lg]);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[m][nf] = mfma32(ar, bw[nf], acc[m][nf]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m >= nm) break;
    const int src = m / nj;
    float *out = src ? G.out1 : G.out;
    float *part = G.part + ((size_t)ti * G.nsrc + src) * G.wide * G.r;
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int a = a0 + 64 * w + 16 * nf + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 16 * (m - src * nj) + 4 * lg + i;
        if (a < G.wide && b < G.r) {
          if (single) out[(size_t)e * G.oe + (size_t)a * G.oa + (size_t)b * G.ob] = G.scale * acc[m][nf][i];
          else part[(size_t)a * G.r + b] = acc[m][nf][i];
        }
      }
    }
  }
}

// Experts spread over several tiles: sum their partials in tile order.
// Experts without rows (no tiles at all) get zeros here.  Each thread handles
// WR_PER consecutive outputs, so the grid stays small.
constexpr int WR_PER = 1;

__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const WgradMArgs G) {
  __shared__ int red[256];
  const int e = blockIdx.y, tid = threadIdx.x;
  const int count = G.offsets[e + 1] - G.offsets[e];
  if (count > 0 && count <= WG_TILE) return;   // written directly by its single tile
  const size_t per = (size_t)G.wide * G.r;
  const size_t i0 = ((size_t)blockIdx.x * 256 + tid) * WR_PER;
  int t0 = 0, nt = 0;
  if (count > 0) {
    // index of the expert's first tile: tiles are listed expert by expert
    int c = 0;
    for (int x = tid; x < e; x += 256)
      c += (G.offsets[x + 1] - G.offsets[x] + WG_TILE - 1) / WG_TILE;
    red[tid] = c;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    t0 = red[0];
    nt = (count + WG_TILE - 1) / WG_TILE;
  }
#pragma unroll
  for (int u = 0; u < WR_PER; ++u) {
    const size_t idx = i0 + u;
    if (idx >= per * G.nsrc) return;
    const int src = (int)(idx / per);
    const size_t ab = idx - (size_t)src * per;
    const int a = (int)(ab / G.r), b = (int)(ab - (size_t)a * G.r);
    float sum = 0.f;
    for (int t = 0; t < nt; ++t) sum += G.part[((size_t)(t0 + t) * G.nsrc + src) * per + ab];
    float *out = src ? G.out1 : G.out;
    out[(size_t)e * G.oe + (size_t)a * G.oa + (size_t)b * G.ob] = G.scale * sum;
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

int proj_tile_rows() { return 64; }

void launch_proj_mfma(const ProjMArgs &P, int max_tiles, bool gather, hipStream_t st) {
  if (gather) proj_mfma_kernel<true><<<max_tiles, 256, 0, st>>>(P);
  else proj_mfma_kernel<false><<<max_tiles, 256, 0, st>>>(P);
}

void launch_wgrad_mfma(const WgradMArgs &G, int max_tiles, bool gather, hipStream_t st) {
  dim3 grid((G.wide + WG_COLS - 1) / WG_COLS, max_tiles);
  if (gather) wgrad_mfma_kernel<true><<<grid, 256, 0, st>>>(G);
  else wgrad_mfma_kernel<false><<<grid, 256, 0, st>>>(G);
  dim3 rgrid((unsigned)(((size_t)G.wide * G.r * G.nsrc + 256 * WR_PER - 1) / (256 * WR_PER)), G.E);
  wgrad_reduce_kernel<<<rgrid, 256, 0, st>>>(G);
}

int wgrad_tile_rows() { return WG_TILE; }

void launch_transpose_nr(const void *in, int E, int N, int r, void *out, hipStream_t st) {
  size_t n = (size_t)E * N;
  transpose_nr_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>((const uint16_t *)in, E, N, r,
                                                                   (uint16_t *)out);
}

}  // namespace moe
