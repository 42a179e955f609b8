// Full-precision router, softmax and top-k.
//
// Router: "Router: Full precision (critical for routing quality)" -- skill
// card "Reversible Sparse MoE Single Node", Implementation Considerations,
// TQP Quantization.  Top-k over routed experts (460 experts, top-12 at the
// largest stage): same card, Architecture Details.  The selection order
// (logit descending, lower expert index first on exact ties) and the gates
// (softmax over the selected logits) are this library's reading; the pages
// state neither.
//
// Two kernels:
//   router_logits  fp32 FMA on the vector ALUs (no matrix cores), a 128-token
//                  x 128-expert tile per 256-thread block, d optionally split
//                  across blocks so that small token counts still fill the
//                  chip; each split writes its own partial.
//   router_topk    one wave per token: sums the partials in split order, adds
//                  the bias, then k rounds of a wave-wide argmax on the key
//                  (logit desc, index asc) and the softmax of the k winners.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int RT_TM = 128;  // tokens per block
constexpr int RT_TE = 128;  // experts per block
constexpr int RT_KC = 16;   // d-chunk staged in LDS per step

// Block tile 128 tokens x 128 experts, 256 threads, each an 8 x 8 register
// tile; x is staged transposed ([k][token]) and W_r as is ([k][expert]) so
// that every thread reads its 8 + 8 operands with four 16-byte LDS loads per
// k and issues 64 FMAs.  blockIdx.z splits d; each split writes a partial.
template <typename T>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const T *__restrict__ x, const float *__restrict__ wr, int Tn, int d, int E,
    int split_len, float *__restrict__ partial) {
  __shared__ __attribute__((aligned(16))) float xs[2][RT_KC][RT_TM];
  __shared__ __attribute__((aligned(16))) float ws[2][RT_KC][RT_TE];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int t0 = blockIdx.x * RT_TM, e0 = blockIdx.y * RT_TE;
  const int c_begin = blockIdx.z * split_len;
  const int c_end = min(d, c_begin + split_len);
  // staging roles: x: token tid/2, 8 consecutive k; W: row tid/16, 8 experts
  const int xt = tid >> 1, xk = (tid & 1) * 8;
  const int wk = tid >> 4, we = (tid & 15) * 8;
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

  auto stage = [&](int c0, int buf) {
    {
      const int t = t0 + xt;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = c0 + xk + i;
        xs[buf][xk + i][xt] = (t < Tn && c < c_end) ? Elem<T>::ld(x, (size_t)t * d + c) : 0.f;
      }
    }
    {
      const int c = c0 + wk;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = e0 + we + i;
        ws[buf][wk][we + i] = (c < c_end && e < E) ? wr[(size_t)c * E + e] : 0.f;
      }
    }
  };

  int buf = 0;
  stage(c_begin, 0);
  __syncthreads();
  for (int c0 = c_begin; c0 < c_end; c0 += RT_KC) {
    if (c0 + RT_KC < c_end) stage(c0 + RT_KC, buf ^ 1);
#pragma unroll
    for (int kk = 0; kk < RT_KC; ++kk) {
      const float4 xa = *reinterpret_cast<const float4 *>(&xs[buf][kk][ty * 8]);
      const float4 xb = *reinterpret_cast<const float4 *>(&xs[buf][kk][ty * 8 + 4]);
      const float4 wa = *reinterpret_cast<const float4 *>(&ws[buf][kk][tx * 8]);
      const float4 wb = *reinterpret_cast<const float4 *>(&ws[buf][kk][tx * 8 + 4]);
      const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
      const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
    buf ^= 1;
  }
  float *out = partial + (size_t)blockIdx.z * Tn * E;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + ty * 8 + i;
    if (t >= Tn) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + tx * 8 + j;
      if (e < E) out[(size_t)t * E + e] = acc[i][j];
    }
  }
}

// (v, e) beats (v2, e2): larger logit, or equal logit and lower index.
DEV bool beats(float v, int e, float v2, int e2) { return v > v2 || (v == v2 && e < e2); }

__global__ __launch_bounds__(256) void router_topk_kernel(
    const float *__restrict__ partial, int splits, const float *__restrict__ bias,
    int Tn, int E, int k, int32_t *__restrict__ topk_idx, float *__restrict__ gates,
    float *__restrict__ logits_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int NE = (E + 63) >> 6;
  float l[16];
  uint32_t taken = 0;
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    int e = lane + 64 * n;
    float v = -INFINITY;
    if (n < NE && e < E) {
      v = 0.f;
      for (int s = 0; s < splits; ++s) v += partial[((size_t)s * Tn + t) * E + e];
      if (bias) v += bias[e];
      if (logits_out) logits_out[(size_t)t * E + e] = v;
    } else {
      taken |= 1u << n;  // padding never wins
    }
    l[n] = v;
  }
  float sel_v = 0.f;  // lane j keeps the j-th winner
  int sel_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      int e = lane + 64 * n;
      if (!((taken >> n) & 1u) && beats(l[n], e, bv, be)) { bv = l[n]; be = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oe = __shfl_xor(be, off);
      if (beats(ov, oe, bv, be)) { bv = ov; be = oe; }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) { sel_v = bv; sel_e = be; }
  }
  // softmax over the k selected logits, relative to the largest (lane 0)
  float top = __shfl(sel_v, 0);
  float z = lane < k ? expf(sel_v - top) : 0.f;
  float sum = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = sel_e;
    gates[(size_t)t * k + lane] = z / sum;
  }
}

int route_splits(int T, int d, int E) {
  const int blocks = ((T + RT_TM - 1) / RT_TM) * ((E + RT_TE - 1) / RT_TE);
  const int max_splits = (d + RT_KC - 1) / RT_KC;
  int s = (512 + blocks - 1) / blocks;
  if (s > max_splits) s = max_splits;
  if (s < 1) s = 1;
  return s;
}

size_t route_ws_bytes(int T, int d, int E) {
  return (size_t)route_splits(T, d, E) * T * E * sizeof(float);
}

void launch_router_logits(bool bf16, const void *x, const float *wr, int Tn, int d, int E,
                          void *ws, int *splits_out, hipStream_t st) {
  int splits = route_splits(Tn, d, E);
  const int chunks = (d + RT_KC - 1) / RT_KC;
  const int split_len = ((chunks + splits - 1) / splits) * RT_KC;
  splits = (d + split_len - 1) / split_len;
  float *partial = (float *)ws;
  dim3 grid((Tn + RT_TM - 1) / RT_TM, (E + RT_TE - 1) / RT_TE, splits);
  if (bf16)
    router_logits_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t *)x, wr, Tn, d, E, split_len,
                                                       partial);
  else
    router_logits_kernel<float><<<grid, 256, 0, st>>>((const float *)x, wr, Tn, d, E, split_len,
                                                      partial);
  *splits_out = splits;
}

void launch_router_topk(const void *ws, int splits, const float *bias, int Tn, int E, int k,
                        int32_t *topk_idx, float *gates, float *logits, hipStream_t st) {
  router_topk_kernel<<<(Tn + 3) / 4, 256, 0, st>>>((const float *)ws, splits, bias, Tn, E, k,
                                                   topk_idx, gates, logits);
}

}  // namespace moe
