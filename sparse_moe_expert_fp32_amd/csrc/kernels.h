// Host-side launchers of the HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- router (route.hip)
size_t route_ws_bytes(int T, int d, int E);
void launch_router_logits(bool bf16, const void *x, const float *wr, int T, int d, int E,
                          void *ws, int *splits_out, hipStream_t st);
void launch_router_topk(const void *ws, int splits, const float *bias, int T, int E, int k,
                        int32_t *topk_idx, float *gates, float *logits, hipStream_t st);

// ---- permutation (permute.hip)
size_t permute_ws_bytes(int T, int E, int k);
void launch_permute(const int32_t *idx, int T, int E, int k, int32_t *counts, int32_t *offsets,
                    int32_t *perm_src, int32_t *slot_pos, const void *x, void *x_perm,
                    int row_bytes, void *ws, hipStream_t st);

// ---- per-token kernels (combine.hip)
void launch_combine(bool bf16, const void *e_out, const int32_t *slot_pos, const float *gates,
                    int T, int d, int k, void *y, hipStream_t st);
void launch_transpose_f32(const float *in, int rows, int cols, float *out, hipStream_t st);
void launch_gate_grad(bool bf16, const void *dy, const void *e_out, const int32_t *topk_idx,
                      const float *gates, const int32_t *slot_pos, const float *wr_t, int T,
                      int d, int k, int E, float *dx_r, void *dO, hipStream_t st);
// matrix-core path (bf16, no dO): the gate gradient and the gather of dX in
// one pass per token, dx[t] = sum_j dl_j W_r[:, e_j] + sum_j dxp[p_j]; returns
// false (nothing launched) when the shape is not covered (d % 8, k > 16)
bool token_bwd_covers(int d, int k);   // the shapes launch_token_bwd takes
// dgp (optional): the partials of the dH product (nq per slot, [nq][S]),
// from which dgamma = sum / g replaces the pass over e_out where g >= 1e-30
bool launch_token_bwd(const void *dy, const void *e_out, const int32_t *topk_idx,
                      const float *gates, const int32_t *slot_pos, const float *wr_t,
                      const void *dxp, int T, int d, int k, int E, void *dx, hipStream_t st,
                      const float *dgp = nullptr, int nq = 0);
void launch_unpermute_sum(bool bf16, bool dxp_f32, const float *dx_r, const void *dxp,
                          const int32_t *slot_pos, int T, int d, int k, void *dx,
                          hipStream_t st);

// out = x + sign * m over n act-dtype values (float32 arithmetic, one rounding)
void launch_rev_couple(bool bf16, const void *x, const void *m, void *out, size_t n, float sign,
                       hipStream_t st);

// ---- few -> many expert growth (grow.hip)
// dst block e F + c = src block e (E source blocks of block_bytes)
void launch_grow_copy(const void *src, void *dst, size_t block_bytes, int E, int F, hipStream_t st);
// w [d][E] -> w_out [d][E F] (copies c >= 1 moved by s z), b [E] -> b_out [E F]
void launch_grow_router(const float *w, const float *b, const float *z, float s, int d, int E,
                        int F, float *w_out, float *b_out, hipStream_t st);

// ---- float32 expert kernels (expert_simple.hip)
// first (optional, 2E + 1 ints): index of each expert's first tile, then the
// number of experts with no tile or more than one, then those experts
// nzero: ntiles[1 .. nzero-1] are set to zero as well (work counters)
void launch_build_tiles(const int32_t *offsets, int E, int BM, int2 *tiles, int *ntiles,
                        hipStream_t st, int *first = nullptr, int nzero = 0);
int simple_tile_rows();

// ---- batched set-up (prep.hip): independent small jobs of one call (tile
// lists, group row sums, rank-16 adapter-B transposes, W_r^T) in one launch of
// 1024-thread blocks; each job takes a contiguous range of the blocks
struct PrepBatch {
  enum Kind { kTiles = 1, kRowsum, kTransposeNR16, kTransposeF32 };
  struct Job {
    int kind, nblocks;
    const int32_t *offsets; int E, BM; int2 *tiles; int *ntiles; int *first; int nzero;
    const void *src; void *dst; int rows, K, G, N; float scale, scale2; int split;
  };
  static constexpr int kMax = 12;
  Job job[kMax];
  int n = 0;
  // launch_build_tiles as a job
  void tiles(const int32_t *offsets, int E, int BM, int2 *tiles, int *ntiles, int *first = nullptr,
             int nzero = 0);
  // launch_group_rowsum as a job
  void rowsum(const void *a, int rows, int K, int G, float scale, float *out, bool split = false,
              float scale2 = 0.f);
  // launch_transpose_nr as a job where the rank-16 kernel applies (else
  // launched on its own now, on st)
  void transpose_nr(const void *in, int E, int N, int r, void *out, hipStream_t st);
  // launch_transpose_f32 as a job
  void transpose_f32(const float *in, int rows, int cols, float *out);

 private:
  Job &next();   // the next free job (aborts past kMax: a fixed number per call)
};
void launch_prep(const PrepBatch &b, hipStream_t st);

struct LinArgs {
  const void *a; int lda; bool gather; const int32_t *perm_src; int kk;
  const int2 *tiles; const int *ntiles; int max_tiles; const int32_t *offsets;
  const uint8_t *q; const uint16_t *scale; int N, K, g; bool trans;
  int bits;                               // base storage: 4 (int4) or 8 (int8)
  const float *Z; int ldz; const void *lmat; size_t l_es; int l_js, l_ns, r; float lam;
  void *out; int ldo; bool acc_out;
};
void launch_lin_simple(bool act_bf16, bool out_f32, const LinArgs &L, hipStream_t st);

struct ProjArgs {
  const void *a; int lda; bool gather; const int32_t *perm_src; int kk;
  const int2 *tiles; const int *ntiles; int max_tiles; const int32_t *offsets;
  const void *m; size_t m_es; int m_cs, m_js; int K, r; float s; float *Z; int ldz;
};
void launch_proj_simple(bool act_bf16, const ProjArgs &P, hipStream_t st);

// out[e][a][b] = s * sum_p L(p,a) R(p,b); exactly one of L, R is float32 (l_f32
// says which); `gather` makes the act-dtype side R read token rows of x.
struct WgradArgs {
  const void *l; int ldl; bool l_f32; bool gather; const int32_t *perm_src; int kk;
  const void *r; int ldr; const int32_t *offsets; int E, Aw, Bw; float s; float *out;
};
void launch_wgrad_simple(bool act_bf16, const WgradArgs &W, hipStream_t st);

void launch_swiglu_fwd(bool act_bf16, const float *G, const float *U, size_t n, void *H,
                       void *Gs, void *Us, hipStream_t st);
void launch_swiglu_bwd(bool act_bf16, const float *dH, const void *Gs, const void *Us, size_t n,
                       void *dG, void *dU, hipStream_t st);

// ---- matrix-core grouped GEMMs (expert_mfma.hip), bf16 activations, group 128
struct MfmaGemmArgs {
  const void *a; int lda;                 // A rows: x [T][d] (mode 0) or H [S][f] (mode 1)
  const int32_t *perm_src; int kk;        // mode 0: token of a permuted row
  const float *rsum; int ld_rsum;         // per A row, per group of 128: -136 * sum of the row
  const int2 *tiles; const int32_t *offsets;   // tile list of launch_build_tiles
  int K, N, NT;                           // reduction, columns per matrix, N-tiles per M-tile
  // ka: the A rows' length.  K for an int4 base; K / 2 for an int8 base split
  // into two int4 planes along K (launch_pack_fwd_int8): the rows are read
  // twice, and the start values of the second plane's groups follow the first's
  int ka;
  // rt: scale ratios [E][K/128][N] of launch_scale_ratio
  const uint8_t *q0; const float *rt0; const uint16_t *B0;   // gate (mode 0) / down (mode 1)
  const uint8_t *q1; const float *rt1; const uint16_t *B1;   // up (mode 0)
  const float *Z0, *Z1; int ldz; int r; float lam;             // X A^T projections (float32)
  // q0, q1 in the stage-major layout of launch_pack_fwd (or null; mode 0
  // reads it only when both matrices have it)
  const uint8_t *qp0, *qp1;
  uint16_t *out; int ldo;                 // H [S][f] (mode 0) or e_out [S][d] (mode 1)
  uint16_t *saveG, *saveU;                // mode 0, optional: U s (1 + G (1 - s)), G s (s = sigmoid G)
  float *rsum_out; int ld_rsum_out;       // mode 0: -136 * group sums of H rows
  int rsum_split;                         // mode 0: also -128 * the sums, at + NT (int8 down)
};
int mfma_tile_rows();
int mfma_blocks_per_cu();      // resident blocks per CU the kernel is built for
// out[row][g] = scale * (sum of group g of the bf16 row), K / G groups; with
// split, out has 2 K / G entries per row and out[row][K / G + g] = scale2 * sum
void launch_group_rowsum(const void *a, int rows, int K, int G, float scale, float *out,
                         hipStream_t st, bool split = false, float scale2 = 0.f);
// scale ratios of a quantized matrix ([E][N][ng] bf16 -> [E][ng'][N] f32):
// rt[e][g][c] = s'[e][c][g-1] / s'[e][c][g] for g >= 1, rt[e][0][c] = s'[e][c][ng'-1],
// s' the scales (ng' = ng), or with split those of the two int4 planes of an
// int8 base, 16 s then s (ng' = 2 ng)
void launch_scale_ratio(const uint16_t *s, int E, int N, int ng, float *rt, hipStream_t st,
                        bool split = false);
// int4 [E][N][K/2] -> stage-major [E][K/64][N][32 B] (K a multiple of 64)
void launch_pack_fwd(const uint8_t *q, int E, int N, int K, uint8_t *qf, hipStream_t st);
// int8 [E][N][K] -> the stage-major int4 layout of its two planes along K
// ([E][2K/64][N][32 B]): q = 16 h + l, plane 1 holds h = q >> 4, plane 2
// l - 8 (l = q & 15), each as a two's-complement nibble
void launch_pack_fwd_int8(const uint8_t *q, int E, int N, int K, uint8_t *qf, hipStream_t st);
// one launch over the tiles of launch_build_tiles (mfma_tile_rows() rows, in
// expert order), each item as the shortest tile class holding its rows (ctr:
// eight counters, zero at launch)
void launch_grouped_gemm(int mode, const MfmaGemmArgs &A, const int *ntiles, int *ctr, int grid,
                         hipStream_t st);
// short batches: one launch over 16-row tiles of launch_build_tiles
// (ntiles: their count), every item a 16-row item
void launch_grouped_gemm_short(int mode, const MfmaGemmArgs &A, const int *ntiles, int grid,
                               hipStream_t st);

// transposed-base products of the backward (expert_mfma_bwd.hip)
struct MfmaGemmTArgs {
  const void *a0, *a1; int lda;           // A rows: dO (mode 0) or dG, dU (mode 1), [S][lda]
  // mode 0 with gsc set: A row p is a0[perm_src[p] / kk] (dy by token) and the
  // product row is scaled by gsc[perm_src[p]] (the gate) before the adapter term
  const int32_t *perm_src; int kk; const float *gsc;
  const int2 *tiles; const int32_t *offsets;   // tile list of launch_build_tiles
  int K, N, NT;                           // reduction per source, output columns, ceil(N / 256)
  // kr: the A rows' length per source.  K for an int4 base; K / 2 for an int8
  // base split into two stacked int4 planes (launch_transpose_q_int8): the rows
  // are read twice, the second plane's offset correction is 128 instead of 136
  int kr;
  const uint8_t *qt0, *qt1;               // int4 base transposed, [E][N][K/2] (qt1: mode 1, up)
  const float *st0, *st1;                 // its scales per column group, [E][N/128][K]
  const float *Z0, *Z1; int ldz; int r;   // dZ = lam dOut B (float32)
  const uint16_t *L0, *L1;                // adapter A of the matrix, [E][r][N]
  const uint16_t *G, *U; uint16_t *dG, *dU;   // mode 0: dG = dH G, dU = dH U ([S][N]; G, U the saved multipliers)
  uint16_t *out; int ldo;                 // mode 1: dX_perm [S][N]
  // mode 0, optional: dgp[q][p] = sum over the q-th 128 columns c of dH[p][c]
  // H[p][c] (H [S][N] the forward's SwiGLU output; q < 2 NT; S rows); with
  // the gate applied to the rows this is g_p times <dy, e_out[p]>
  const uint16_t *H; float *dgp; int S;
};
int mfma_t_tile_rows();         // rows of a full tile (a multiple of 32)
int mfma_t_tile_cols();
int mfma_t_blocks_per_cu();   // resident blocks per CU the kernel is built for
// int4 [E][R][C/2] + scales [E][R][C/128] -> transposed int4 [E][C][R/2] + scales
// [E][C/128][R] (f32), for experts with rows (every expert when offsets is
// null); R, C multiples of 128
void launch_transpose_q(const uint8_t *q, const uint16_t *s, const int32_t *offsets, int E, int R,
                        int C, uint8_t *qt, float *st, hipStream_t stream);
// int8 [E][R][C] + scales [E][R][C/128] -> the transposed int4 layout of its
// two planes stacked along R (2R rows: h = q >> 4 with scale 16 s, then
// l - 8 with scale s, l = q & 15): [E][2R/64][C][32 B] + [E][C/128][2R] f32
void launch_transpose_q_int8(const uint8_t *q, const uint16_t *s, const int32_t *offsets, int E,
                             int R, int C, uint8_t *qt, float *st, hipStream_t stream);

// ---- rank-r adapter products on the matrix cores (lowrank.hip)
struct ProjMArgs {                        // Z_s = scale * A M_s^T over each expert's rows
  const uint16_t *a; int lda; const int32_t *perm_src; int kk;
  const int2 *tiles; const int *ntiles; const int32_t *offsets;   // proj_tile_rows() tiles
  int K, r, nsrc;
  const uint16_t *m0, *m1;                // [E][r][K]
  float scale; float *Z0, *Z1; int ldz;
  const float *gsc;                       // GATHER: row p also scaled by gsc[perm_src[p]] (or null)
};
// short_rows: 16-row tiles with the reduction split over 8 waves (short
// batches: a few rows per expert), else 64-row tiles over 4 waves
void launch_proj_mfma(const ProjMArgs &P, int max_tiles, bool gather, hipStream_t st,
                      bool short_rows = false);
int proj_tile_rows(bool short_rows = false);
struct WgradMArgs {                       // out_s[e][a][b] = scale * sum_p W[p][a] R_s[p][b]
  const uint16_t *w; int ldw; const int32_t *perm_src; int kk;
  const float *rr; int ldr;               // R of source 0
  const float *gsc;                       // GATHER: R row p scaled by gsc[perm_src[p]] (or null)
  const float *rr1; float *out1;          // second source (nsrc = 2): same W, strides, scale
  int nsrc;
  const int32_t *offsets; int E, wide, r; float scale;
  float *out; size_t oe; int oa, ob;
  const int2 *tiles; const int *ntiles;   // wgrad_tile_rows()-row tiles
  const int *tfirst;                      // [E] index of each expert's first tile
  const int *multi;                       // count, then the experts not written by one tile
  float *part;                            // partials: [tiles][nsrc][wide][r]
  // optional (wgrad_can_project): the projection of the same rows onto pm
  // [E][wide][16] (bf16, the adapter B as stored), as partials zpart
  // [wide / 256][S][16] (f32) over the 256-column ranges, for
  // launch_lowrank_reduce
  const uint16_t *pm; float *zpart; int S;
};
int wgrad_tile_rows();
// reduce = false: the per-tile partials are left for launch_lowrank_reduce
void launch_wgrad_mfma(const WgradMArgs &G, int max_tiles, bool gather, hipStream_t st,
                       bool reduce = true);
bool wgrad_can_project(const WgradMArgs &G);
// z_s[p * ldz + j] = scale * g_p * (sum over the nq ranges of zp_s[q][p][j]),
// j < 16, for z0 (from zp0) and, when zp1 is given, z1 (from zp1); g_p =
// gsc[perm_src[p]] when gsc is given, else 1
struct ZpartJob {
  const float *zp0, *zp1; int nq, S;
  const int32_t *perm_src; const float *gsc; float scale;
  float *z0, *z1; int ldz;
};
// the reductions of up to three adapter-gradient passes launched with
// reduce = false (each with its own partial buffer) and, optionally, of one
// set of projection partials, in one launch
void launch_lowrank_reduce(const WgradMArgs *w, int nw, const ZpartJob *z, hipStream_t st);
void launch_transpose_nr(const void *in, int E, int N, int r, void *out, hipStream_t st);
// bf16 [E][r][N] -> [E][N][r]
// one launch over the tiles of launch_build_tiles (mfma_t_tile_rows() rows,
// in expert order), each item as the shortest tile class holding its rows
// (ctr: eight counters, zero at launch, one per XCD)
void launch_grouped_gemm_t(int mode, const MfmaGemmTArgs &A, const int *ntiles, int *ctr, int grid,
                           hipStream_t st);

// ---- fixed device scratch (scratch.hip): the per-device address of the
// library's static scratch array (kStaticScratchBytes), looked up once per
// device with that device current
constexpr size_t kStaticScratchBytes = size_t(64) << 20;

// Work-list block of the persistent products (tile list of 128-row tiles):
// the tile count, then for each of the two products of a call eight work
// counters, one per XCD, each on a 128-byte line of its own, so that the
// atomics of different XCDs do not contend for one line.  The list builder
// zeroes the block (nzero = kWorkListInts).
constexpr int kCtrStride = 32;                               // ints between counters
constexpr int kCtrSet0 = 32, kCtrSet1 = 32 + 8 * kCtrStride;  // first counter of each product
constexpr int kWorkListInts = 32 + 16 * kCtrStride;
hipError_t static_scratch(void **ptr);

// ---- adapter optimizer step (adamw.hip)
struct AdamWArgs {
  size_t n;
  float *p; const float *g; float *m, *v;   // master parameter, gradient, moments
  void *out;                                 // copy of the new parameter, or null
  float lr, beta1, beta2, eps, weight_decay;
  float bc1, bc2;                            // 1 - beta1^t, 1 - beta2^t
};
// out_kind: 0 none, 1 float32 copy, 2 bf16 copy
void launch_adamw(const AdamWArgs &h, int out_kind, hipStream_t st);

}  // namespace moe
