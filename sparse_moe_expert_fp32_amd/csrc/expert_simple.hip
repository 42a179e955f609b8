// Straightforward float32 kernels of the expert FFNs and their adapter-only
// backward.  They serve the float32 activation path (every product computed
// in float32 on the vector ALUs) and hold the pieces that have no matrix-core
// variant: tile lists, element-wise SwiGLU and the adapter reductions.
//
// The computation is TQP's expert under "Reversible Sparse MoE Single Node"
// (skill card), Principle 3 and Implementation Considerations "TQP
// Quantization": a frozen quantized base plus a trained low-rank adapter on
// every matrix (LoRA, Related Methods), so W_eff = W_hat + lam * B A, the
// base gets no gradient.  The SwiGLU form of the expert is this library's
// reading; the pages do not name the FFN.
#include "common.h"
#include "kernels.h"
#include "prep.h"

namespace moe {

// ------------------------------------------------------------ tile list --
// One entry per (expert, BM-row block); entries ordered by expert.  tiles[i]
// = (e, first row); ntiles[0] = count; first (when given) [e] = index of the
// expert's first entry; ntiles[1 .. nzero-1] = 0 (counters of the kernels
// that consume the list).  Launched with one 1024-thread block.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t *__restrict__ offsets,
                                                           int E, int BM, int2 *__restrict__ tiles,
                                                           int *__restrict__ ntiles,
                                                           int *__restrict__ first_out, int nzero) {
  build_tiles_body(offsets, E, BM, tiles, ntiles, first_out, nzero);
}

// ------------------------------------------------------ int4 expert GEMM --
// out[p][n] = (ACC ? out[p][n] : 0) + sum_c A(p, c) W(e, n, c)
//             + lam * sum_j Z[p][j] L(e, j, n)
// A(p, c): GATHER ? a[perm_src[p] / kk][c] : a[p][c].
// W: !TRANS: q [E][N][K/2], scale [E][N][K/g]  (W(e,n,c) = stored[n][c])
//     TRANS: q [E][K][N/2], scale [E][K][N/g]  (W(e,n,c) = stored[c][n])
//     (bits = 8: q holds one two's-complement byte per value, rows of K or N bytes)
// L(e, j, n) = lmat[e * l_es + j * l_js + n * l_ns] (act dtype), Z float32.
constexpr int SB_M = 16, SB_N = 64, SB_K = 32;

template <typename TA, typename TO, bool GATHER, bool TRANS>
__global__ __launch_bounds__(256) void lin_simple_kernel(
    const TA *__restrict__ a, int lda, const int32_t *__restrict__ perm_src, int kk,
    const int2 *__restrict__ tiles, const int *__restrict__ ntiles,
    const int32_t *__restrict__ offsets, const uint8_t *__restrict__ q,
    const uint16_t *__restrict__ scale, int N, int K, int g, int bits, const float *__restrict__ Z,
    int ldz,
    const TA *__restrict__ lmat, size_t l_es, int l_js, int l_ns, int r, float lam,
    TO *__restrict__ out, int ldo, bool acc_out) {
  __shared__ float As[SB_M][SB_K + 1];
  __shared__ float Ws[SB_N][SB_K + 1];
  __shared__ int rows[SB_M];
  if ((int)blockIdx.x >= ntiles[0]) return;
  const int2 tile = tiles[blockIdx.x];
  const int e = tile.x, p0 = tile.y, p_end = offsets[e + 1];
  const int n0 = blockIdx.y * SB_N;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  if (tid < SB_M) {
    int p = p0 + tid;
    rows[tid] = p < p_end ? (GATHER ? perm_src[p] / kk : p) : -1;
  }
  __syncthreads();
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < K; c0 += SB_K) {
    for (int i = tid; i < SB_M * SB_K; i += 256) {
      int rr = i / SB_K, cc = i % SB_K, row = rows[rr];
      As[rr][cc] = (row >= 0 && c0 + cc < K) ? Elem<TA>::ld(a, (size_t)row * lda + c0 + cc) : 0.f;
    }
    for (int i = tid; i < SB_N * SB_K; i += 256) {
      int nn = i / SB_K, cc = i % SB_K, n = n0 + nn, c = c0 + cc;
      float w = 0.f;
      if (n < N && c < K) {
        // the stored row and the position in it
        const size_t rowi = TRANS ? (size_t)e * K + c : (size_t)e * N + n;
        const int L = TRANS ? N : K, at = TRANS ? n : c;
        const int qv = bits == 8 ? (int)(int8_t)q[rowi * L + at] : int4_at(q + rowi * (L / 2), at);
        w = (float)qv * bf2f(scale[rowi * (L / g) + at / g]);
      }
      Ws[nn][cc] = w;
    }
    __syncthreads();
#pragma unroll 8
    for (int cc = 0; cc < SB_K; ++cc) {
      float av = As[ty][cc];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(av, Ws[tx + 16 * i][cc], acc[i]);
    }
    __syncthreads();
  }
  const int p = p0 + ty;
  if (p >= p_end) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int n = n0 + tx + 16 * i;
    if (n >= N) continue;
    float v = acc[i];
    if (Z) {
      float s = 0.f;
      for (int j = 0; j < r; ++j)
        s = fmaf(Z[(size_t)p * ldz + j],
                 Elem<TA>::ld(lmat, (size_t)e * l_es + (size_t)j * l_js + (size_t)n * l_ns), s);
      v = fmaf(lam, s, v);
    }
    size_t o = (size_t)p * ldo + n;
    if (acc_out) v += Elem<TO>::ld(out, o);
    Elem<TO>::st(out, o, v);
  }
}

// --------------------------------------------------- low-rank projections --
// Z[p][j] = s * sum_c A(p, c) M(e, c, j),  M(e,c,j) = m[e*m_es + c*m_cs + j*m_js]
template <typename TA, bool GATHER>
__global__ __launch_bounds__(256) void proj_simple_kernel(
    const TA *__restrict__ a, int lda, const int32_t *__restrict__ perm_src, int kk,
    const int2 *__restrict__ tiles, const int *__restrict__ ntiles,
    const int32_t *__restrict__ offsets, const TA *__restrict__ m, size_t m_es, int m_cs,
    int m_js, int K, int r, float s, float *__restrict__ Z, int ldz) {
  __shared__ float As[SB_M][65];
  __shared__ float Ms[64][33];
  __shared__ int rows[SB_M];
  if ((int)blockIdx.x >= ntiles[0]) return;
  const int2 tile = tiles[blockIdx.x];
  const int e = tile.x, p0 = tile.y, p_end = offsets[e + 1];
  const int tid = threadIdx.x;
  if (tid < SB_M) {
    int p = p0 + tid;
    rows[tid] = p < p_end ? (GATHER ? perm_src[p] / kk : p) : -1;
  }
  __syncthreads();
  // thread -> (row, j) pairs: row = tid / 16, j = tid % 16 and j + 16
  const int rr = tid >> 4, j0 = tid & 15;
  float acc[2] = {0.f, 0.f};
  for (int c0 = 0; c0 < K; c0 += 64) {
    for (int i = tid; i < SB_M * 64; i += 256) {
      int ro = i / 64, cc = i % 64, row = rows[ro];
      As[ro][cc] = (row >= 0 && c0 + cc < K) ? Elem<TA>::ld(a, (size_t)row * lda + c0 + cc) : 0.f;
    }
    for (int i = tid; i < 64 * 32; i += 256) {
      int cc = i / 32, j = i % 32, c = c0 + cc;
      Ms[cc][j] = (c < K && j < r)
                      ? Elem<TA>::ld(m, (size_t)e * m_es + (size_t)c * m_cs + (size_t)j * m_js)
                      : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int cc = 0; cc < 64; ++cc) {
      float av = As[rr][cc];
      acc[0] = fmaf(av, Ms[cc][j0], acc[0]);
      acc[1] = fmaf(av, Ms[cc][j0 + 16], acc[1]);
    }
    __syncthreads();
  }
  const int p = p0 + rr;
  if (p >= p_end) return;
  if (j0 < r) Z[(size_t)p * ldz + j0] = s * acc[0];
  if (j0 + 16 < r) Z[(size_t)p * ldz + j0 + 16] = s * acc[1];
}

// ----------------------------------------------------- adapter gradients --
// out[e][a][b] = s * sum_{p in expert e} L(p, a) R(p, b), rows in ascending p.
// L(p, a) = l[row_L(p) * ldl + a],  R(p, b) = rr[row_R(p) * ldr + b], where a
// side marked "gather" reads row perm_src[p] / kk (a token row) instead of p.
template <typename TL, typename TR, bool GL, bool GR>
__global__ __launch_bounds__(256) void wgrad_simple_kernel(
    const TL *__restrict__ l, int ldl, const int32_t *__restrict__ perm_src, int kk,
    const TR *__restrict__ rr, int ldr, const int32_t *__restrict__ offsets, int Aw, int Bw,
    float s, float *__restrict__ out) {
  __shared__ float Ls[16][17];
  __shared__ float Rs[16][17];
  const int e = blockIdx.z, a0 = blockIdx.y * 16, b0 = blockIdx.x * 16;
  const int tid = threadIdx.x, ta = tid >> 4, tb = tid & 15;
  const int lo = offsets[e], hi = offsets[e + 1];
  float acc = 0.f;
  for (int p0 = lo; p0 < hi; p0 += 16) {
    {
      int i = tid >> 4, j = tid & 15, p = p0 + i;
      int src = p < hi ? perm_src[p] / kk : -1;
      int rowl = p < hi ? (GL ? src : p) : -1;
      int rowr = p < hi ? (GR ? src : p) : -1;
      Ls[i][j] = (rowl >= 0 && a0 + j < Aw) ? Elem<TL>::ld(l, (size_t)rowl * ldl + a0 + j) : 0.f;
      Rs[i][j] = (rowr >= 0 && b0 + j < Bw) ? Elem<TR>::ld(rr, (size_t)rowr * ldr + b0 + j) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = fmaf(Ls[i][ta], Rs[i][tb], acc);
    __syncthreads();
  }
  if (a0 + ta < Aw && b0 + tb < Bw) out[((size_t)e * Aw + a0 + ta) * Bw + b0 + tb] = s * acc;
}

// ---------------------------------------------------------- SwiGLU --
// H = silu(G) * U; the pre-activations are also stored in the act dtype.
template <typename T>
__global__ void swiglu_fwd_kernel(const float *__restrict__ G, const float *__restrict__ U,
                                  size_t n, T *__restrict__ H, T *__restrict__ Gs,
                                  T *__restrict__ Us) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float g = G[i], u = U[i];
  Elem<T>::st(H, i, silu_f(g) * u);
  Elem<T>::st(Gs, i, g);
  Elem<T>::st(Us, i, u);
}

// dG = dH * U * s * (1 + G (1 - s)),  dU = dH * G * s,  s = sigmoid(G)
template <typename T>
__global__ void swiglu_bwd_kernel(const float *__restrict__ dH, const T *__restrict__ Gs,
                                  const T *__restrict__ Us, size_t n, T *__restrict__ dG,
                                  T *__restrict__ dU) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float g = Elem<T>::ld(Gs, i), u = Elem<T>::ld(Us, i), dh = dH[i];
  float sg = sigmoid_f(g);
  Elem<T>::st(dG, i, dh * u * sg * (1.f + g * (1.f - sg)));
  Elem<T>::st(dU, i, dh * g * sg);
}

// ------------------------------------------------------------- launchers --

void launch_build_tiles(const int32_t *offsets, int E, int BM, int2 *tiles, int *ntiles,
                        hipStream_t st, int *first, int nzero) {
  build_tiles_kernel<<<1, 1024, 0, st>>>(offsets, E, BM, tiles, ntiles, first, nzero);
}

int simple_tile_rows() { return SB_M; }

template <typename TA, typename TO>
static void lin_dispatch(const LinArgs &L, hipStream_t st) {
  dim3 grid(L.max_tiles, (L.N + SB_N - 1) / SB_N);
#define LIN_CALL(G, TR)                                                                        \
  lin_simple_kernel<TA, TO, G, TR><<<grid, 256, 0, st>>>(                                      \
      (const TA *)L.a, L.lda, L.perm_src, L.kk, L.tiles, L.ntiles, L.offsets, L.q, L.scale,    \
      L.N, L.K, L.g, L.bits, L.Z, L.ldz, (const TA *)L.lmat, L.l_es, L.l_js, L.l_ns, L.r, L.lam, \
      (TO *)L.out, L.ldo, L.acc_out)
  if (L.gather) {
    if (L.trans) LIN_CALL(true, true); else LIN_CALL(true, false);
  } else {
    if (L.trans) LIN_CALL(false, true); else LIN_CALL(false, false);
  }
#undef LIN_CALL
}

void launch_lin_simple(bool act_bf16, bool out_f32, const LinArgs &L, hipStream_t st) {
  if (act_bf16) {
    if (out_f32) lin_dispatch<bf16_t, float>(L, st);
    else lin_dispatch<bf16_t, bf16_t>(L, st);
  } else {
    lin_dispatch<float, float>(L, st);
  }
}

void launch_proj_simple(bool act_bf16, const ProjArgs &P, hipStream_t st) {
#define PROJ_CALL(TA, G)                                                                       \
  proj_simple_kernel<TA, G><<<P.max_tiles, 256, 0, st>>>(                                      \
      (const TA *)P.a, P.lda, P.perm_src, P.kk, P.tiles, P.ntiles, P.offsets, (const TA *)P.m, \
      P.m_es, P.m_cs, P.m_js, P.K, P.r, P.s, P.Z, P.ldz)
  if (act_bf16) {
    if (P.gather) PROJ_CALL(bf16_t, true); else PROJ_CALL(bf16_t, false);
  } else {
    if (P.gather) PROJ_CALL(float, true); else PROJ_CALL(float, false);
  }
#undef PROJ_CALL
}

void launch_wgrad_simple(bool act_bf16, const WgradArgs &W, hipStream_t st) {
  dim3 grid((W.Bw + 15) / 16, (W.Aw + 15) / 16, W.E);
#define WG_CALL(TL, TR, GL, GR)                                                                \
  wgrad_simple_kernel<TL, TR, GL, GR><<<grid, 256, 0, st>>>(                                   \
      (const TL *)W.l, W.ldl, W.perm_src, W.kk, (const TR *)W.r, W.ldr, W.offsets, W.Aw, W.Bw, \
      W.s, W.out)
  // one side is float32 (a low-rank projection), the other the act dtype
  if (act_bf16) {
    if (W.l_f32) {
      if (W.gather) WG_CALL(float, bf16_t, false, true); else WG_CALL(float, bf16_t, false, false);
    } else {
      WG_CALL(bf16_t, float, false, false);
    }
  } else {
    if (W.gather) WG_CALL(float, float, false, true); else WG_CALL(float, float, false, false);
  }
#undef WG_CALL
}

void launch_swiglu_fwd(bool act_bf16, const float *G, const float *U, size_t n, void *H,
                       void *Gs, void *Us, hipStream_t st) {
  unsigned blocks = (unsigned)((n + 255) / 256);
  if (act_bf16)
    swiglu_fwd_kernel<bf16_t><<<blocks, 256, 0, st>>>(G, U, n, (bf16_t *)H, (bf16_t *)Gs,
                                                      (bf16_t *)Us);
  else
    swiglu_fwd_kernel<float><<<blocks, 256, 0, st>>>(G, U, n, (float *)H, (float *)Gs,
                                                     (float *)Us);
}

void launch_swiglu_bwd(bool act_bf16, const float *dH, const void *Gs, const void *Us, size_t n,
                       void *dG, void *dU, hipStream_t st) {
  unsigned blocks = (unsigned)((n + 255) / 256);
  if (act_bf16)
    swiglu_bwd_kernel<bf16_t><<<blocks, 256, 0, st>>>(dH, (const bf16_t *)Gs, (const bf16_t *)Us,
                                                      n, (bf16_t *)dG, (bf16_t *)dU);
  else
    swiglu_bwd_kernel<float><<<blocks, 256, 0, st>>>(dH, (const float *)Gs, (const float *)Us, n,
                                                     (float *)dG, (float *)dU);
}

}  // namespace moe
