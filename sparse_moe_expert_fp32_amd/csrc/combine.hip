// Per-token kernels: gate-weighted combine, the gate/router part of the
// backward, and the final gather of the expert input-gradients.
//
// Each token gathers its own k rows in ascending slot order with a float32
// accumulator, so no float atomics are needed and results are reproducible
// bit for bit.  The mixing of the selected experts' outputs by the routing
// weights is the routed-expert layer of the skill card "Reversible Sparse
// MoE Single Node" (Architecture Details, top-k routing); the gradient
// through the gates into the router input follows from the full-precision
// router of the same card (Implementation Considerations, TQP Quantization),
// whose own weights are not trained here.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "prep.h"

namespace moe {

// Vector of VEC elements of T loaded as 16 bytes.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static DEV void ld(const float *p, float *v) {
    float4 a = *reinterpret_cast<const float4 *>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
  static DEV void st(float *p, const float *v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static DEV void ld(const bf16_t *p, float *v) {
    uint4 a = *reinterpret_cast<const uint4 *>(p);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static DEV void st(bf16_t *p, const float *v) {
    uint4 a;
    a.x = pack2bf(v[0], v[1]); a.y = pack2bf(v[2], v[3]);
    a.z = pack2bf(v[4], v[5]); a.w = pack2bf(v[6], v[7]);
    *reinterpret_cast<uint4 *>(p) = a;
  }
};

// y[t] = sum_j gates[t][j] * e_out[slot_pos[t*k+j]]
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ e_out,
                                                      const int32_t *__restrict__ slot_pos,
                                                      const float *__restrict__ gates, int d,
                                                      int k, T *__restrict__ y) {
  constexpr int V = Vec16<T>::N;
  const int t = blockIdx.x;
  for (int c = threadIdx.x * V; c < d; c += 256 * V) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      float g = gates[(size_t)t * k + j];
      int p = slot_pos[(size_t)t * k + j];
      float v[V];
      Vec16<T>::ld(e_out + (size_t)p * d + c, v);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(g, v[i], acc[i]);
    }
    Vec16<T>::st(y + (size_t)t * d + c, acc);
  }
}

// out[e][c] = in[c][e]   (W_r [d][E] -> [E][d] so that a token's router
// columns are read with unit stride)
__global__ void transpose_f32_kernel(const float *__restrict__ in, int rows, int cols,
                                     float *__restrict__ out) {
  transpose_f32_tile(in, rows, cols, out, blockIdx.x * 32, blockIdx.y * 32);
}

// Block-wide sum of KMAX-wide partial vectors in a fixed tree order.
template <int KMAX>
DEV void block_sum(float (&v)[KMAX], int k, float *red /*[4][KMAX]*/) {
  int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      float s = v[j];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) red[wave * KMAX + j] = s;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) v[j] = (red[j] + red[KMAX + j]) + (red[2 * KMAX + j] + red[3 * KMAX + j]);
  __syncthreads();
}

// Per token t (one block):
//   dgamma_j = <dy_t, e_out[p_j]>,  dl_j = gamma_j (dgamma_j - sum_i gamma_i dgamma_i)
//   dx_r[t]  = sum_j dl_j * W_r[:, e_j]      (float32)
//   dO[p_j]  = gamma_j * dy_t                (act dtype, permuted order; skipped
//                                            when dO is null)
template <typename T>
__global__ __launch_bounds__(256) void gate_grad_kernel(
    const T *__restrict__ dy, const T *__restrict__ e_out, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ gates, const int32_t *__restrict__ slot_pos,
    const float *__restrict__ wr_t, int d, int k, int E, float *__restrict__ dx_r,
    T *__restrict__ dO) {
  constexpr int V = Vec16<T>::N;
  __shared__ float red[4 * 32];
  __shared__ int sp[32], se[32];
  __shared__ float sg[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    sp[threadIdx.x] = slot_pos[(size_t)t * k + threadIdx.x];
    // (clamped: a caller-supplied index outside [0, E) must not read past W_r)
    se[threadIdx.x] = min(max(topk_idx[(size_t)t * k + threadIdx.x], 0), E - 1);
    sg[threadIdx.x] = gates[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  float part[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) part[j] = 0.f;
  for (int c = threadIdx.x * V; c < d; c += 256 * V) {
    float g[V];
    Vec16<T>::ld(dy + (size_t)t * d + c, g);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j < k) {
        float o[V];
        Vec16<T>::ld(e_out + (size_t)sp[j] * d + c, o);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) s = fmaf(g[i], o[i], s);
        part[j] += s;
      }
    }
  }
  block_sum<32>(part, k, red);
  float mean = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j)
    if (j < k) mean = fmaf(sg[j], part[j], mean);
  for (int c = threadIdx.x * V; c < d; c += 256 * V) {
    float g[V], acc[V];
    Vec16<T>::ld(dy + (size_t)t * d + c, g);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j >= k) break;
      float dl = sg[j] * (part[j] - mean);
      const float *w = wr_t + (size_t)se[j] * d + c;
      float o[V];
#pragma unroll
      for (int i = 0; i < V; ++i) { acc[i] = fmaf(dl, w[i], acc[i]); o[i] = sg[j] * g[i]; }
      if (dO) Vec16<T>::st(dO + (size_t)sp[j] * d + c, o);
    }
#pragma unroll
    for (int i = 0; i < V; ++i) dx_r[(size_t)t * d + c + i] = acc[i];
  }
}

// ---- one wave per token (bf16 activations, d a multiple of 8)
//
// A wave walks its token's row in chunks of 512 columns (8 per lane, 16-byte
// accesses); the k slots are taken in KB batches of 4, fully unrolled, so all
// of a chunk's row loads are independent and in flight together.  Slots past
// k read slot k-1's row again (in bounds, from cache) and are masked out.

// The backward's per-token tail on the matrix-core path (dO is never formed
// there), after the expert input-gradients dX_perm:
//   dgamma_j = <dy_t, e_out[p_j]>,  dl_j = gamma_j (dgamma_j - sum_i gamma_i dgamma_i)
//   dx[t]    = sum_j dl_j * W_r[:, e_j] + sum_j dX_perm[p_j]   (j ascending, float32)
// The same sums as gate_grad_kernel followed by unpermute_sum_kernel, without
// the float32 router-gradient rows between them.
//
// With dgp (the dH product's per-slot partials of g_p <dy_t, e_out[p]>, nq
// of them in column order) dgamma_j is their sum divided by gamma_j (the sum
// in a fixed lane order: lane groups of every fourth partial, then the groups
// pairwise), and the pass over e_out is made only for a token with a gate
// below 1e-30 (where that division would lose precision).
template <int KB>
__global__ __launch_bounds__(256) void token_bwd_wave_kernel(
    const bf16_t *__restrict__ dy, const bf16_t *__restrict__ e_out,
    const int32_t *__restrict__ topk_idx, const float *__restrict__ gates,
    const int32_t *__restrict__ slot_pos, const float *__restrict__ wr_t,
    const bf16_t *__restrict__ dxp, int T, int d, int k, int E, bf16_t *__restrict__ dx,
    const float *__restrict__ dgp, int nq) {
  constexpr int KM = 4 * KB;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  int p[KM], e[KM];
  float g[KM], part[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int jc = j < k ? j : k - 1;
    p[j] = slot_pos[(size_t)t * k + jc];
    e[j] = min(max(topk_idx[(size_t)t * k + jc], 0), E - 1);   // in range (see gate_grad_kernel)
    g[j] = gates[(size_t)t * k + jc];
    part[j] = 0.f;
  }
  bool direct = dgp == nullptr;
  if (!direct) {
    // the partials on the lanes, all loads in one round trip: lane l takes
    // slot j = l % 16 and the partials q = l / 16, l / 16 + 4, ... in order;
    // the four lane groups are then added by shuffles (a fixed order)
    const size_t S = (size_t)T * k;
    const int jl = lane & 15;
    float s = 0.f;
    if (jl < k) {
      const int pj = slot_pos[(size_t)t * k + jl];
      for (int q = lane >> 4; q < nq; q += 4) s += dgp[(size_t)q * S + pj];
    }
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < k) {
        part[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), j)) / g[j];
        direct |= !(g[j] >= 1e-30f);
      }
    }
    if (direct) {
#pragma unroll
      for (int j = 0; j < KM; ++j) part[j] = 0.f;
    }
  }
  if (direct)
  for (int c = lane * 8; c < d; c += 512) {
    float gy[8], v[KM][8];
    Vec16<bf16_t>::ld(dy + (size_t)t * d + c, gy);
#pragma unroll
    for (int j = 0; j < KM; ++j) Vec16<bf16_t>::ld(e_out + (size_t)p[j] * d + c, v[j]);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(gy[i], v[j][i], s);
      part[j] += s;
    }
  }
  float mean = 0.f;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    float s = part[j];
    if (direct) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    }
    part[j] = s;
    if (j < k) mean = fmaf(g[j], s, mean);
  }
  float dl[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) dl[j] = g[j] * (part[j] - mean);
  // 4 columns per lane here (256-column chunks): the float32 W_r rows make
  // this pass twice as wide in registers as the first
  for (int c = lane * 4; c < d; c += 256) {
    float4 w[KM];
    uint2 v[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      w[j] = *reinterpret_cast<const float4 *>(wr_t + (size_t)e[j] * d + c);
      v[j] = *reinterpret_cast<const uint2 *>(dxp + (size_t)p[j] * d + c);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k) {
        acc[0] = fmaf(dl[j], w[j].x, acc[0]);
        acc[1] = fmaf(dl[j], w[j].y, acc[1]);
        acc[2] = fmaf(dl[j], w[j].z, acc[2]);
        acc[3] = fmaf(dl[j], w[j].w, acc[3]);
      }
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k) {
        acc[0] += __uint_as_float(v[j].x << 16);
        acc[1] += __uint_as_float(v[j].x & 0xFFFF0000u);
        acc[2] += __uint_as_float(v[j].y << 16);
        acc[3] += __uint_as_float(v[j].y & 0xFFFF0000u);
      }
    *reinterpret_cast<uint2 *>(dx + (size_t)t * d + c) =
        make_uint2(pack2bf(acc[0], acc[1]), pack2bf(acc[2], acc[3]));
  }
}

// Reversible coupling around the layer: out = x + sign * m elementwise, in
// float32 with one rounding to T.  With m the layer's output for the other
// stream y1 this is the additive coupling of a reversible residual block
// (skill card "Reversible Sparse MoE Single Node", Pattern 1: addition and
// subtraction as the invertible operations; Implementation Considerations:
// reversible residual blocks, stateless routing): sign +1 gives
// y2 = x2 + MoE(y1), sign -1 recovers x2 = y2 - MoE(y1).  VEC: 16-byte
// accesses (every pointer 16-byte aligned), the grid strides over the data.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void rev_couple_kernel(const T *__restrict__ x,
                                                         const T *__restrict__ m, T *out,
                                                         size_t n, float sign) {
  constexpr int V = Vec16<T>::N;
  const size_t stride = (size_t)gridDim.x * 256;
  const size_t t0 = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (VEC) {
    for (size_t i = t0; i < n / V; i += stride) {
      float a[V], b[V];
      Vec16<T>::ld(x + i * V, a);
      Vec16<T>::ld(m + i * V, b);
#pragma unroll
      for (int u = 0; u < V; ++u) a[u] = fmaf(sign, b[u], a[u]);
      Vec16<T>::st(out + i * V, a);
    }
  }
  for (size_t i = (VEC ? n / V * V : 0) + t0; i < n; i += stride)
    Elem<T>::st(out, i, fmaf(sign, Elem<T>::ld(m, i), Elem<T>::ld(x, i)));
}

void launch_rev_couple(bool bf16, const void *x, const void *m, void *out, size_t n, float sign,
                       hipStream_t st) {
  const bool vec = (((uintptr_t)x | (uintptr_t)m | (uintptr_t)out) & 15) == 0;
  const size_t work = (n + 7) / 8;
  const unsigned grid = (unsigned)std::max<size_t>(1, std::min<size_t>((work + 255) / 256, 8192));
#define MOE_RC(TY)                                                                              \
  if (vec) rev_couple_kernel<TY, true><<<grid, 256, 0, st>>>((const TY *)x, (const TY *)m,      \
                                                             (TY *)out, n, sign);               \
  else rev_couple_kernel<TY, false><<<grid, 256, 0, st>>>((const TY *)x, (const TY *)m,         \
                                                          (TY *)out, n, sign);
  if (bf16) {
    MOE_RC(bf16_t)
  } else {
    MOE_RC(float)
  }
#undef MOE_RC
}

// dx[t] = dx_r[t] + sum_j dxp[slot_pos[t*k+j]]   (j ascending)
template <typename T, typename TP>
__global__ __launch_bounds__(256) void unpermute_sum_kernel(const float *__restrict__ dx_r,
                                                            const TP *__restrict__ dxp,
                                                            const int32_t *__restrict__ slot_pos,
                                                            int d, int k, T *__restrict__ dx) {
  constexpr int V = Vec16<T>::N;
  const int t = blockIdx.x;
  for (int c = threadIdx.x * V; c < d; c += 256 * V) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = dx_r[(size_t)t * d + c + i];
    for (int j = 0; j < k; ++j) {
      int p = slot_pos[(size_t)t * k + j];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += Elem<TP>::ld(dxp, (size_t)p * d + c + i);
    }
    Vec16<T>::st(dx + (size_t)t * d + c, acc);
  }
}

void launch_combine(bool bf16, const void *e_out, const int32_t *slot_pos, const float *gates,
                    int Tn, int d, int k, void *y, hipStream_t st) {
  if (bf16)
    combine_kernel<bf16_t><<<Tn, 256, 0, st>>>((const bf16_t *)e_out, slot_pos, gates, d, k,
                                               (bf16_t *)y);
  else
    combine_kernel<float><<<Tn, 256, 0, st>>>((const float *)e_out, slot_pos, gates, d, k,
                                              (float *)y);
}

void launch_transpose_f32(const float *in, int rows, int cols, float *out, hipStream_t st) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  transpose_f32_kernel<<<grid, 256, 0, st>>>(in, rows, cols, out);
}

void launch_gate_grad(bool bf16, const void *dy, const void *e_out, const int32_t *topk_idx,
                      const float *gates, const int32_t *slot_pos, const float *wr_t, int Tn,
                      int d, int k, int E, float *dx_r, void *dO, hipStream_t st) {
  if (bf16)
    gate_grad_kernel<bf16_t><<<Tn, 256, 0, st>>>((const bf16_t *)dy, (const bf16_t *)e_out,
                                                 topk_idx, gates, slot_pos, wr_t, d, k, E, dx_r,
                                                 (bf16_t *)dO);
  else
    gate_grad_kernel<float><<<Tn, 256, 0, st>>>((const float *)dy, (const float *)e_out,
                                                topk_idx, gates, slot_pos, wr_t, d, k, E, dx_r,
                                                (float *)dO);
}

bool token_bwd_covers(int d, int k) { return d % 8 == 0 && k <= 16; }

bool launch_token_bwd(const void *dy, const void *e_out, const int32_t *topk_idx,
                      const float *gates, const int32_t *slot_pos, const float *wr_t,
                      const void *dxp, int Tn, int d, int k, int E, void *dx, hipStream_t st,
                      const float *dgp, int nq) {
  if (!token_bwd_covers(d, k)) return false;
  const int wgrid = (Tn + 3) / 4;
  const bf16_t *a = (const bf16_t *)dy, *b = (const bf16_t *)e_out, *c = (const bf16_t *)dxp;
  bf16_t *o = (bf16_t *)dx;
#define MOE_TB(KB) token_bwd_wave_kernel<KB><<<wgrid, 256, 0, st>>>(a, b, topk_idx, gates, slot_pos, wr_t, c, Tn, d, k, E, o, dgp, nq)
  switch ((k + 3) / 4) {
    case 1: MOE_TB(1); break;
    case 2: MOE_TB(2); break;
    case 3: MOE_TB(3); break;
    default: MOE_TB(4); break;
  }
#undef MOE_TB
  return true;
}

void launch_unpermute_sum(bool bf16, bool dxp_f32, const float *dx_r, const void *dxp,
                          const int32_t *slot_pos, int Tn, int d, int k, void *dx,
                          hipStream_t st) {
  if (bf16) {
    if (dxp_f32)
      unpermute_sum_kernel<bf16_t, float><<<Tn, 256, 0, st>>>(dx_r, (const float *)dxp, slot_pos,
                                                              d, k, (bf16_t *)dx);
    else
      unpermute_sum_kernel<bf16_t, bf16_t><<<Tn, 256, 0, st>>>(dx_r, (const bf16_t *)dxp,
                                                               slot_pos, d, k, (bf16_t *)dx);
  } else {
    unpermute_sum_kernel<float, float><<<Tn, 256, 0, st>>>(dx_r, (const float *)dxp, slot_pos, d,
                                                           k, (float *)dx);
  }
}

}  // namespace moe
