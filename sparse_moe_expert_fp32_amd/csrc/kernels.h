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
                      int d, int k, float *dx_r, void *dO, hipStream_t st);
// matrix-core path (bf16, no dO): the gate gradient and the gather of dX in
// one pass per token, dx[t] = sum_j dl_j W_r[:, e_j] + sum_j dxp[p_j]; returns
// false (nothing launched) when the shape is not covered (d % 8, k > 16)
bool launch_token_bwd(const void *dy, const void *e_out, const int32_t *topk_idx,
                      const float *gates, const int32_t *slot_pos, const float *wr_t,
                      const void *dxp, int T, int d, int k, void *dx, hipStream_t st);
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
void launch_build_tiles(const int32_t *offsets, int E, int BM, int2 *tiles, int *ntiles,
                        hipStream_t st, int *first = nullptr);
int simple_tile_rows();

struct LinArgs {
  const void *a; int lda; bool gather; const int32_t *perm_src; int kk;
  const int2 *tiles; const int *ntiles; int max_tiles; const int32_t *offsets;
  const uint8_t *q; const uint16_t *scale; int N, K, g; bool trans;
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
  const int2 *tiles; const int32_t *offsets;   // tile list of launch_class_tiles
  int K, N, NT;                           // reduction, columns per matrix, N-tiles per M-tile
  // rt: scale ratios [E][K/128][N] of launch_scale_ratio
  const uint8_t *q0; const float *rt0; const uint16_t *B0;   // gate (mode 0) / down (mode 1)
  const uint8_t *q1; const float *rt1; const uint16_t *B1;   // up (mode 0)
  const float *Z0, *Z1; int ldz; int r; float lam;             // X A^T projections (float32)
  // q0, q1 in the stage-major layout of launch_pack_fwd (or null): used by
  // the launches the layout speeds up (mode 1, and the short tile classes of
  // mode 0, whose 128-row kernel needs more registers with it)
  const uint8_t *qp0, *qp1;
  uint16_t *out; int ldo;                 // H [S][f] (mode 0) or e_out [S][d] (mode 1)
  uint16_t *saveG, *saveU;                // mode 0, optional
  float *rsum_out; int ld_rsum_out;       // mode 0: -136 * group sums of H rows
};
int mfma_tile_rows();
int mfma_blocks_per_cu();      // resident blocks per CU the kernel is built for
void launch_group_rowsum(const void *a, int rows, int K, int G, float scale, float *out,
                         hipStream_t st);
// scale ratios of a quantized matrix ([E][N][ng] bf16 -> [E][ng][N] f32):
// rt[e][g][c] = s[e][c][g-1] / s[e][c][g] for g >= 1, rt[e][0][c] = s[e][c][ng-1]
void launch_scale_ratio(const uint16_t *s, int E, int N, int ng, float *rt, hipStream_t st);
// expert tiles of 128 rows, the partial last one of each expert rounded up to
// 32, 64, 96 or 128 rows, grouped by that class; cnt[8]: count and first
// index of each class (128-row class first)
void launch_class_tiles(const int32_t *offsets, int E, int2 *tiles, int *cnt, hipStream_t st);
// int4 [E][N][K/2] -> stage-major [E][K/64][N][32 B] (K a multiple of 64)
void launch_pack_fwd(const uint8_t *q, int E, int N, int K, uint8_t *qf, hipStream_t st);
// the launch of tile class cls (0: 128-row tiles .. 3: 32-row tiles)
void launch_grouped_gemm(int mode, const MfmaGemmArgs &A, const int *cnt, int cls, int grid,
                         hipStream_t st);

// transposed-base products of the backward (expert_mfma_bwd.hip)
struct MfmaGemmTArgs {
  const void *a0, *a1; int lda;           // A rows: dO (mode 0) or dG, dU (mode 1), [S][lda]
  // mode 0 with gsc set: A row p is a0[perm_src[p] / kk] (dy by token) and the
  // product row is scaled by gsc[perm_src[p]] (the gate) before the adapter term
  const int32_t *perm_src; int kk; const float *gsc;
  const int2 *tiles; const int32_t *offsets;   // tile list of launch_class_tiles
  int K, N, NT;                           // reduction per source, output columns, ceil(N / 256)
  const uint8_t *qt0, *qt1;               // int4 base transposed, [E][N][K/2] (qt1: mode 1, up)
  const float *st0, *st1;                 // its scales per column group, [E][N/128][K]
  const float *Z0, *Z1; int ldz; int r;   // dZ = lam dOut B (float32)
  const uint16_t *L0, *L1;                // adapter A of the matrix, [E][r][N]
  const uint16_t *LT0, *LT1;              // the same transposed, [E][N][r] (rank 16; or null)
  const uint16_t *G, *U; uint16_t *dG, *dU;   // mode 0: SwiGLU backward, [S][N]
  uint16_t *out; int ldo;                 // mode 1: dX_perm [S][N]
};
int mfma_t_tile_rows();
int mfma_t_tile_cols();
int mfma_t_blocks_per_cu();   // resident blocks per CU the kernel is built for
// int4 [E][R][C/2] + scales [E][R][C/128] -> transposed int4 [E][C][R/2] + scales
// [E][C/128][R] (f32), for experts with rows (every expert when offsets is
// null); R, C multiples of 128
void launch_transpose_q(const uint8_t *q, const uint16_t *s, const int32_t *offsets, int E, int R,
                        int C, uint8_t *qt, float *st, hipStream_t stream);

// ---- rank-r adapter products on the matrix cores (lowrank.hip)
struct ProjMArgs {                        // Z_s = scale * A M_s^T over each expert's rows
  const uint16_t *a; int lda; const int32_t *perm_src; int kk;
  const int2 *tiles; const int *ntiles; const int32_t *offsets;   // 64-row tiles
  int K, r, nsrc;
  const uint16_t *m0, *m1;                // [E][r][K]
  float scale; float *Z0, *Z1; int ldz;
  const float *gsc;                       // GATHER: row p also scaled by gsc[perm_src[p]] (or null)
};
void launch_proj_mfma(const ProjMArgs &P, int max_tiles, bool gather, hipStream_t st);
int proj_tile_rows();
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
};
int wgrad_tile_rows();
void launch_wgrad_mfma(const WgradMArgs &G, int max_tiles, bool gather, hipStream_t st);
void launch_transpose_nr(const void *in, int E, int N, int r, void *out, hipStream_t st);
// bf16 [E][r][N] -> [E][N][r]
void launch_transpose_rn(const void *in, int E, int r, int N, void *out, hipStream_t st);
// the launch of tile class cls of launch_class_tiles (cnt: counts and starts)
void launch_grouped_gemm_t(int mode, const MfmaGemmTArgs &A, const int *cnt, int cls, int grid,
                           hipStream_t st);

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
