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
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "prep.h"
#include "mfma.h"

namespace moe {

// ------------------------------------------------------------ projections --
// Z_s[p][j] = scale * g_p * sum_k A(p, k) M_s[e][j][k] for sources s < nsrc,
// j < r.  A(p, k) = a[(GATHER ? perm_src[p] / kk : p) * lda + k]; M_s is
// [E][r][K]; g_p = gsc[perm_src[p]] when gsc is given (GATHER), else 1.
// NF = nsrc * ceil(r / 16) 16-column fragments.  One block per tile of 64
// rows (16 for short batches); the tiles are spread so that each XCD takes a
// contiguous run of the list (the tiles of one expert share that XCD's L2
// copy of M).  The reduction is split over the NW waves (wave w takes the
// 64-wide k-chunks w, w + NW, ...) and every wave keeps the next chunk's
// loads in flight while it multiplies the current one; the wave partials are
// summed through LDS in wave order.
// Columns j >= r of a fragment read a valid row of M (row r - 1): column j of
// the product depends only on column j of M, and those columns are not stored.
constexpr int PJ_KC = 64;

// NMR: 16-row fragments per tile (4: 64-row tiles; 1: 16-row tiles for short
// batches, with NW = 8 waves splitting the reduction so that each wave has
// fewer chunks to wait for).
template <bool GATHER, int NF, int NMR, int NW>
__global__ __launch_bounds__(64 * NW, NF == 4 ? 1 : 2) void proj_mfma_kernel(const ProjMArgs P) {
  __shared__ float red[NW - 1][NMR * NF * 4 * 64];   // partials of waves 1..NW-1: [m*NF+f][i][lane]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int nt = P.ntiles[0], per = (nt + 7) >> 3;
  const int ti = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (ti >= nt) return;
  const int2 tile = P.tiles[ti];
  const int e = tile.x, p0 = tile.y;
  const int p_end = P.offsets[e + 1];
  const int nj = (P.r + 15) >> 4;           // 16-column fragments per source
  // rows: fragment m covers rows p0 + 16 m .. +15 (clamped to the expert)
  const uint16_t *ap[NMR];
#pragma unroll
  for (int m = 0; m < NMR; ++m) {
    const int prow = min(p0 + 16 * m + lr, p_end - 1);
    const size_t arow = GATHER ? (size_t)(P.perm_src[prow] / P.kk) : (size_t)prow;
    ap[m] = P.a + arow * P.lda + 8 * lg;
  }
  // columns: fragment f covers rank columns 16 (f % nj) .. + 15 of source f / nj
  const uint16_t *mp[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int src = f / nj, j = 16 * (f - src * nj) + lr;
    mp[f] = (src ? P.m1 : P.m0) + ((size_t)e * P.r + min(j, P.r - 1)) * P.K + 8 * lg;
  }
  f32x4_t acc[NMR][NF];
#pragma unroll
  for (int m = 0; m < NMR; ++m)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  using Av = uint4[NMR][2];
  using Bv = uint4[2][NF];
  auto load = [&](Av &av, Bv &bv, int k0) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int m = 0; m < NMR; ++m) av[m][s] = *reinterpret_cast<const uint4 *>(ap[m] + k0 + 32 * s);
#pragma unroll
      for (int f = 0; f < NF; ++f) bv[s][f] = *reinterpret_cast<const uint4 *>(mp[f] + k0 + 32 * s);
    }
  };
  auto comp = [&](const Av &av, const Bv &bv) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int m = 0; m < NMR; ++m) acc[m][f] = mfma32(av[m][s], bv[s][f], acc[m][f]);
  };
  // chunks w, w + NW, ... of K (K is a multiple of 64; with K < 64 NW some
  // waves have none); two register sets.  Each branch issues the next
  // chunk's loads before multiplying the current one, so the wait before the
  // multiplication leaves the new loads in flight.
  const int nk = (P.K / PJ_KC - w + NW - 1) / NW;
  if (nk > 0) {
    Av a0, a1;
    Bv b0, b1;
    int k0 = w * PJ_KC;
    load(a0, b0, k0);
    for (int c = 1;; c += 2, k0 += 2 * NW * PJ_KC) {
      if (c >= nk) {
        comp(a0, b0);
        break;
      }
      load(a1, b1, k0 + NW * PJ_KC);
      comp(a0, b0);
      if (c + 1 >= nk) {
        comp(a1, b1);
        break;
      }
      load(a0, b0, k0 + 2 * NW * PJ_KC);
      comp(a1, b1);
    }
  }
  // partial sums of waves 1..NW-1 to LDS, summed by wave 0 in wave order
  if (w > 0) {
#pragma unroll
    for (int m = 0; m < NMR; ++m)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w - 1][((m * NF + f) * 4 + i) * 64 + lane] = acc[m][f][i];
  }
  __syncthreads();
  if (w > 0) return;
  float gs[NMR][4];
#pragma unroll
  for (int m = 0; m < NMR; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = min(p0 + 16 * m + 4 * lg + i, p_end - 1);
      gs[m][i] = GATHER && P.gsc ? P.scale * P.gsc[P.perm_src[p]] : P.scale;
    }
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int src = f / nj, j = 16 * (f - src * nj) + lr;
    float *Z = src ? P.Z1 : P.Z0;
#pragma unroll
    for (int m = 0; m < NMR; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = ((m * NF + f) * 4 + i) * 64 + lane;
        float v = acc[m][f][i];
#pragma unroll
        for (int q = 0; q < NW - 1; ++q) v += red[q][o];
        const int p = p0 + 16 * m + 4 * lg + i;
        if (j < P.r && p < p_end) Z[(size_t)p * P.ldz + j] = gs[m][i] * v;
      }
  }
}

// ------------------------------------------------------ adapter gradients --
// out_s[e*oe + a*oa + b*ob] = scale * sum_{p in expert e} W(p, a) g_p R_s[p][b],
// a < wide, b < r, for one or two R sources sharing W (NM = nsrc *
// ceil(r / 16) fragments of 16 R columns); W(p, a) = w[(GATHER ? perm_src[p]
// / kk : p) * ldw + a], g_p = gsc[perm_src[p]] when gsc is given (GATHER),
// else 1.
//
// Work items are (512-row tile of an expert, 256 wide columns), so a heavily
// loaded expert is spread over many blocks.  An expert that fits one tile
// writes its result directly; otherwise each tile writes an unscaled partial
// and a second kernel sums the partials in tile order (deterministic, no
// atomics).  Inside a tile the rows go in ascending chunks of 64.  MFMA
// operands need 8 consecutive rows per lane, so W is transposed on the way
// into LDS: each thread loads an 8 row x 8 column bf16 block and transposes it
// in registers (v_perm), storing each column's 8 rows as one 16-byte LDS
// chunk ([row octet][column], column index XOR-swizzled); R is staged
// transposed as bf16.  D = R^T W: A operand rows are R columns, B operand
// columns are wide columns.  A chunk's registers are free once it is in LDS,
// so the next chunk's loads are issued right then and stay in flight across
// the barriers and matrix work of the current one (barriers wait for LDS
// operations only).
//
// PROJ (one source of rank 16, wide a multiple of 256): the same pass also
// forms the projection of the rows onto the adapter B = [E][wide][16] of the
// matrix, Z'_q[p][j] = sum over the block's 256 columns (column range q) of
// W(p, a) B[e][a][j], as partials zpart[q][p][j]; launch_lowrank_reduce adds
// the ranges.  The staged chunk is also stored as it came (rows of 16-byte
// pieces, piece index XOR-swizzled by row), and each wave multiplies 16 of
// its rows by B, staged in LDS transposed (ml[j][a], from its rows of 16
// rank values as stored).
constexpr int WG_COLS = 256, WG_ROWS = 64, WG_TILE = 512;

DEV int wg_sw(int c) { return c ^ ((c >> 3) & 7); }

// all of this wave's LDS operations done, then the workgroup barrier (global
// loads stay in flight)
DEV void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt untouched
  block_barrier();
}

template <bool GATHER, int NM, bool PROJ>
__global__ __launch_bounds__(256, 2) void wgrad_mfma_kernel(const WgradMArgs G) {
  static_assert(!PROJ || NM == 1, "the projection takes one source of rank 16");
  __shared__ uint4 wl[WG_ROWS / 8][WG_COLS];                          // 32 KB
  // PROJ: M of the block's columns, rows padded by 16 bytes (conflict-free
  // reads), and the chunk's rows as loaded (32 KB)
  __shared__ __attribute__((aligned(16))) uint16_t ml[PROJ ? 16 : 1][PROJ ? WG_COLS + 8 : 8];
  __shared__ uint4 wrow[PROJ ? WG_ROWS : 1][PROJ ? WG_COLS / 8 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t rl[16 * NM][WG_ROWS + 8];
  __shared__ int srow[WG_TILE];                                       // source row per tile row
  __shared__ float sgam[WG_TILE];                                     // its R scale
  const int ti = blockIdx.y;
  if (ti >= G.ntiles[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int2 tile = G.tiles[ti];
  const int e = tile.x, p0 = tile.y, a0 = blockIdx.x * WG_COLS;
  const int lo_e = G.offsets[e], hi_e = G.offsets[e + 1];
  const int hi = min(p0 + WG_TILE, hi_e);
  const bool single = hi_e - lo_e <= WG_TILE;
  const int nj = (G.r + 15) >> 4;   // R fragments per source (NM = nj * nsrc)
  constexpr int RC = 16 * NM;       // staged R columns (all sources)
  constexpr int RPER = RC / 4;      // R values per thread and chunk
  if constexpr (PROJ) {   // B[e][a0 + a][jh .. jh + 7] -> ml[jh ..][a]
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + 256 * u, a = idx >> 1, jh = 8 * (idx & 1);
      const uint4 v = *reinterpret_cast<const uint4 *>(G.pm + ((size_t)e * G.wide + a0 + a) * 16 + jh);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ml[jh + 2 * i][a] = (uint16_t)(wv[i] & 0xFFFFu);
        ml[jh + 2 * i + 1][a] = (uint16_t)(wv[i] >> 16);
      }
    }
  }
  if (GATHER) {
    for (int t = tid; t < hi - p0; t += 256) {
      const int ps = G.perm_src[p0 + t];
      srow[t] = ps / G.kk;
      sgam[t] = G.gsc ? G.gsc[ps] : 1.f;
    }
  }
  if (GATHER || PROJ) __syncthreads();
  f32x4_t acc[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // staging role: row octet oct, columns a0 + 8 cg .. + 7
  const int oct = tid >> 5, cg = tid & 31;
  const bool col_ok = a0 + 8 * cg < G.wide;   // wide is a multiple of 8
  const uint16_t *wcol = G.w + a0 + 8 * cg;
  uint4 in[8];
  float rv[RPER];
  // loads of the chunk at rows pc .. pc + 63 (rows past the end repeat the
  // last row; they meet R = 0)
  auto load = [&](int pc) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = min(pc + 8 * oct + i, hi - 1);
      const size_t row = GATHER ? (size_t)srow[p - p0] : (size_t)p;
      in[i] = col_ok ? *reinterpret_cast<const uint4 *>(wcol + row * G.ldw) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < RPER; ++u) {
      const int idx = tid + 256 * u, pp = idx / RC, cc = idx - pp * RC;
      const int src = cc / (nj * 16), b = cc - src * nj * 16;
      const float *R = src ? G.rr1 : G.rr;
      const int p = min(pc + pp, hi - 1);
      rv[u] = R[(size_t)p * G.ldr + min(b, G.r - 1)];
      if (GATHER) rv[u] *= sgam[p - p0];
    }
  };
  load(p0);
  for (int pc = p0; pc < hi; pc += WG_ROWS) {
#pragma unroll
    for (int u = 0; u < RPER; ++u) {
      const int idx = tid + 256 * u, pp = idx / RC, cc = idx - pp * RC;
      const int b = cc - (cc / (nj * 16)) * nj * 16;
      rl[cc][pp] = f2bf(pc + pp < hi && b < G.r ? rv[u] : 0.f);
    }
    if constexpr (PROJ) {   // (piece cg of row r at cg ^ (r & 15))
#pragma unroll
      for (int i = 0; i < 8; ++i) wrow[8 * oct + i][cg ^ ((8 * oct + i) & 15)] = in[i];
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
    if (pc + WG_ROWS < hi) load(pc + WG_ROWS);
    lds_barrier();
    if constexpr (PROJ) {
      // D[j][p] = sum_a M[j][a] W(p, a): lane (lr, lg) ends with rank
      // columns 4 lg .. 4 lg + 3 of row 16 w + lr
      f32x4_t zp = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int rr = 16 * w + lr;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        zp = mfma32(*reinterpret_cast<const uint4 *>(&ml[lr][32 * ks + 8 * lg]),
                    wrow[rr][(4 * ks + lg) ^ (rr & 15)], zp);
      const int p = pc + rr;
      if (p < hi)
        *reinterpret_cast<f32x4_t *>(G.zpart + ((size_t)blockIdx.x * G.S + p) * 16 + 4 * lg) = zp;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 bw[4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) bw[nf] = wl[4 * s + lg][wg_sw(64 * w + 16 * nf + lr)];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 ar = *reinterpret_cast<const uint4 *>(&rl[16 * m + lr][32 * s + 8 * lg]);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[m][nf] = mfma32(ar, bw[nf], acc[m][nf]);
      }
    }
    lds_barrier();
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
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
// Experts without rows (no tiles at all) get zeros here.  Each thread
// handles WR_PER consecutive outputs.
constexpr int WR_PER = 4;

// Only the experts on the list (empty ones, which get zeros, and split ones);
// block row by (of ny) takes list entries by, by + ny, ...
DEV void wgrad_reduce_body(const WgradMArgs &G, int bx, int by, int ny) {
  const int tid = threadIdx.x;
  const size_t per = (size_t)G.wide * G.r;
  const size_t i0 = ((size_t)bx * 256 + tid) * WR_PER;
  const int nl = G.multi[0];
  for (int q = by; q < nl; q += ny) {
    const int e = G.multi[1 + q];
    const int count = G.offsets[e + 1] - G.offsets[e];
    const int t0 = count > 0 ? G.tfirst[e] : 0;
    const int nt = (count + WG_TILE - 1) / WG_TILE;
#pragma unroll
    for (int u = 0; u < WR_PER; ++u) {
      const size_t idx = i0 + u;
      if (idx >= per * G.nsrc) break;
      const int src = (int)(idx / per);
      const size_t ab = idx - (size_t)src * per;
      const int a = (int)(ab / G.r), b = (int)(ab - (size_t)a * G.r);
      float sum = 0.f;
      for (int t = 0; t < nt; ++t) sum += G.part[((size_t)(t0 + t) * G.nsrc + src) * per + ab];
      float *out = src ? G.out1 : G.out;
      out[(size_t)e * G.oe + (size_t)a * G.oa + (size_t)b * G.ob] = G.scale * sum;
    }
  }
}

__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const WgradMArgs G) {
  wgrad_reduce_body(G, blockIdx.x, blockIdx.y, gridDim.y);
}

// blocks of the reduction of one pass: (wide r nsrc / 1024) x min(E, 64)
__host__ __device__ inline int wgrad_reduce_cols(const WgradMArgs &G) {
  return (int)(((size_t)G.wide * G.r * G.nsrc + 256 * WR_PER - 1) / (256 * WR_PER));
}
__host__ __device__ inline int wgrad_reduce_rows(const WgradMArgs &G) { return G.E < 64 ? G.E : 64; }

// out[e][j][n] = in[e][n][j] for bf16 [E][N][r] -> [E][r][N].  One block per
// (256 values of n, expert): the block's input is one contiguous run of
// 256 r values, read in order, and every output row segment is 512
// contiguous bytes; the transposition goes through LDS.
constexpr int TN_N = 256;

__global__ __launch_bounds__(256) void transpose_nr_kernel(const uint16_t *__restrict__ in, int N,
                                                           int r, uint16_t *__restrict__ out) {
  __shared__ uint16_t t[TN_N * 33];   // [n][j], j < r <= 32, padded
  const int e = blockIdx.y, n0 = blockIdx.x * TN_N, tid = threadIdx.x;
  const int nn = min(TN_N, N - n0);
  const uint16_t *src = in + ((size_t)e * N + n0) * r;
  for (int i = tid; i < nn * r; i += 256) {
    const int n = i / r, j = i - n * r;
    t[n * 33 + j] = src[i];
  }
  __syncthreads();
  for (int i = tid; i < nn * r; i += 256) {
    const int j = i / nn, n = i - j * nn;
    out[((size_t)e * r + j) * N + n0 + n] = t[n * 33 + j];
  }
}

int proj_tile_rows(bool short_rows) { return short_rows ? 16 : 64; }

void launch_proj_mfma(const ProjMArgs &P, int max_tiles, bool gather, hipStream_t st,
                      bool short_rows) {
  const int nf = P.nsrc * ((P.r + 15) / 16);
  const unsigned grid = (unsigned)((max_tiles + 7) / 8 * 8);   // every XCD the same share
#define MOE_PROJ2(NF, NMR, NW)                                                  \
  if (gather) proj_mfma_kernel<true, NF, NMR, NW><<<grid, 64 * NW, 0, st>>>(P);  \
  else proj_mfma_kernel<false, NF, NMR, NW><<<grid, 64 * NW, 0, st>>>(P);
#define MOE_PROJ(NF)            \
  if (short_rows) {             \
    MOE_PROJ2(NF, 1, 8)         \
  } else {                      \
    MOE_PROJ2(NF, 4, 4)         \
  }
  if (nf == 1) {
    MOE_PROJ(1)
  } else if (nf == 2) {
    MOE_PROJ(2)
  } else {
    MOE_PROJ(4)
  }
#undef MOE_PROJ
#undef MOE_PROJ2
}

void launch_wgrad_mfma(const WgradMArgs &G, int max_tiles, bool gather, hipStream_t st,
                       bool reduce) {
  const int nm = G.nsrc * ((G.r + 15) / 16);
  dim3 grid((G.wide + WG_COLS - 1) / WG_COLS, max_tiles);
  const bool proj = G.pm != nullptr;
#define MOE_WG(NM)                                                             \
  if (gather) wgrad_mfma_kernel<true, NM, false><<<grid, 256, 0, st>>>(G);     \
  else wgrad_mfma_kernel<false, NM, false><<<grid, 256, 0, st>>>(G);
  if (proj) {
    if (gather) wgrad_mfma_kernel<true, 1, true><<<grid, 256, 0, st>>>(G);
    else wgrad_mfma_kernel<false, 1, true><<<grid, 256, 0, st>>>(G);
  } else if (nm == 1) {
    MOE_WG(1)
  } else if (nm == 2) {
    MOE_WG(2)
  } else {
    MOE_WG(4)
  }
#undef MOE_WG
  if (!reduce) return;
  dim3 rgrid((unsigned)wgrad_reduce_cols(G), (unsigned)wgrad_reduce_rows(G));
  wgrad_reduce_kernel<<<rgrid, 256, 0, st>>>(G);
}

bool wgrad_can_project(const WgradMArgs &G) {
  return G.nsrc == 1 && G.r == 16 && G.wide % WG_COLS == 0;
}

// dZ_s[p * ldz + j] = scale * g_p * sum_q zpart_s[q][p][j] (q ascending, q <
// nq), j < 16, for source src; g_p = gsc[perm_src[p]] when gsc is given,
// else 1.  Element i: row i / 4, rank columns 4 (i % 4) .. + 3.
DEV void zpart_reduce_elem(const ZpartJob &Z, size_t i, int src) {
  if (i >= (size_t)Z.S * 4) return;
  const int p = (int)(i >> 2), j = 4 * (int)(i & 3);
  const float *zp = src ? Z.zp1 : Z.zp0;
  f32x4_t v = *reinterpret_cast<const f32x4_t *>(zp + (size_t)p * 16 + j);
  for (int q = 1; q < Z.nq; ++q) {
    const f32x4_t u = *reinterpret_cast<const f32x4_t *>(zp + ((size_t)q * Z.S + p) * 16 + j);
    v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
  }
  const float g = Z.scale * (Z.gsc ? Z.gsc[Z.perm_src[p]] : 1.f);
  float *z = (src ? Z.z1 : Z.z0) + (size_t)p * Z.ldz + j;
  z[0] = g * v[0]; z[1] = g * v[1]; z[2] = g * v[2]; z[3] = g * v[3];
}

// The deferred reductions of up to three adapter-gradient passes and one set
// of projection partials in one launch: pass i takes the first cols_i rows_i
// blocks after the passes before it, then the projection partials (S * 4 /
// 256 blocks per source).
struct LowrankReduceArgs {
  WgradMArgs w[3];
  int nw;
  ZpartJob z;
  int has_z;
};

__global__ __launch_bounds__(256) void lowrank_reduce_kernel(const LowrankReduceArgs R) {
  int b = (int)blockIdx.x;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (i < R.nw) {
      const int cols = wgrad_reduce_cols(R.w[i]), rows = wgrad_reduce_rows(R.w[i]);
      if (b < cols * rows) {
        wgrad_reduce_body(R.w[i], b % cols, b / cols, rows);
        return;
      }
      b -= cols * rows;
    }
  }
  if (R.has_z) {
    const int zb = (int)(((size_t)R.z.S * 4 + 255) / 256);
    zpart_reduce_elem(R.z, (size_t)(b % zb) * 256 + threadIdx.x, b / zb);
  }
}

void launch_lowrank_reduce(const WgradMArgs *w, int nw, const ZpartJob *z, hipStream_t st) {
  LowrankReduceArgs R{};
  int blocks = 0;
  R.nw = std::min(nw, 3);
  for (int i = 0; i < R.nw; ++i) {
    R.w[i] = w[i];
    blocks += wgrad_reduce_cols(w[i]) * wgrad_reduce_rows(w[i]);
  }
  if (z) {
    R.z = *z;
    R.has_z = 1;
    blocks += (int)(((size_t)z->S * 4 + 255) / 256) * (z->zp1 ? 2 : 1);
  }
  if (blocks > 0) lowrank_reduce_kernel<<<blocks, 256, 0, st>>>(R);
}

int wgrad_tile_rows() { return WG_TILE; }

// Rank 16: one thread per n, 16 values of 2 bytes each way; the column
// side moves as two 16-byte accesses, the row side as coalesced 2-byte
// accesses across the wave.
__global__ __launch_bounds__(256) void transpose_nr16_kernel(const uint16_t *__restrict__ in, int N,
                                                             uint16_t *__restrict__ out) {
  transpose_nr16_elem(in, N, blockIdx.y, blockIdx.x * 256 + threadIdx.x, out);
}

void launch_transpose_nr(const void *in, int E, int N, int r, void *out, hipStream_t st) {
  dim3 grid((N + TN_N - 1) / TN_N, E);
  if (r == 16 && ((uintptr_t)in & 15) == 0)    // (16-byte loads)
    transpose_nr16_kernel<<<grid, 256, 0, st>>>((const uint16_t *)in, N, (uint16_t *)out);
  else
    transpose_nr_kernel<<<grid, 256, 0, st>>>((const uint16_t *)in, N, r, (uint16_t *)out);
}

}  // namespace moe
