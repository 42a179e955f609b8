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
//   router_logits  fp32 FMA on the vector ALUs (no matrix cores), a 32-token
//                  x (64*NE)-expert register tile per 256-thread block, d
//                  optionally split across blocks so that small token counts
//                  still fill the chip; each split writes its own partial.
//   router_topk    one wave per token: sums the partials in split order, adds
//                  the bias, then k rounds of a wave-wide argmax on the key
//                  (logit desc, index asc) and the softmax of the k winners.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int RT_TM = 32;   // tokens per block (8 per wave)
constexpr int RT_KC = 16;   // d-chunk staged in LDS

// The d-chunk staged per step: 16 rows of W_r, 8 when E > 512 (LDS budget).
template <typename T, int NE>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const T *__restrict__ x, const float *__restrict__ wr, int Tn, int d, int E,
    int split_len, float *__restrict__ partial) {
  constexpr int KC = NE <= 8 ? RT_KC : RT_KC / 2;
  __shared__ float xs[RT_TM][KC + 1];
  __shared__ float ws[KC][NE * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_TM;
  const int c_begin = blockIdx.y * split_len;
  const int c_end = min(d, c_begin + split_len);
  float acc[8][NE];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int n = 0; n < NE; ++n) acc[i][n] = 0.f;

  for (int c0 = c_begin; c0 < c_end; c0 += KC) {
    // stage x[t0:t0+32, c0:c0+KC] and W_r[c0:c0+KC, :]
    for (int i = tid; i < RT_TM * KC; i += 256) {
      int tt = i / KC, cc = i % KC;
      int t = t0 + tt, c = c0 + cc;
      xs[tt][cc] = (t < Tn && c < c_end) ? Elem<T>::ld(x, (size_t)t * d + c) : 0.f;
    }
    for (int i = tid; i < KC * NE * 64; i += 256) {
      int cc = i / (NE * 64), e = i % (NE * 64);
      int c = c0 + cc;
      ws[cc][e] = (c < c_end && e < E) ? wr[(size_t)c * E + e] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) {
      float wv[NE];
#pragma unroll
      for (int n = 0; n < NE; ++n) wv[n] = ws[cc][lane + 64 * n];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float xv = xs[wave * 8 + i][cc];
#pragma unroll
        for (int n = 0; n < NE; ++n) acc[i][n] = fmaf(xv, wv[n], acc[i][n]);
      }
    }
    __syncthreads();
  }
  float *out = partial + (size_t)blockIdx.y * Tn * E;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int t = t0 + wave * 8 + i;
    if (t >= Tn) continue;
#pragma unroll
    for (int n = 0; n < NE; ++n) {
      int e = lane + 64 * n;
      if (e < E) out[(size_t)t * E + e] = acc[i][n];
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

int route_splits(int T, int d) {
  int nbx = (T + RT_TM - 1) / RT_TM;
  int max_splits = (d + RT_KC - 1) / RT_KC;
  int s = (256 + nbx - 1) / nbx;
  if (s > max_splits) s = max_splits;
  if (s < 1) s = 1;
  return s;
}

size_t route_ws_bytes(int T, int d, int E) {
  return (size_t)route_splits(T, d) * T * E * sizeof(float);
}

template <typename T, int NE>
static void launch_logits(const void *x, const float *wr, int Tn, int d, int E, int splits,
                          int split_len, float *partial, hipStream_t st) {
  dim3 grid((Tn + RT_TM - 1) / RT_TM, splits);
  router_logits_kernel<T, NE><<<grid, 256, 0, st>>>((const T *)x, wr, Tn, d, E, split_len,
                                                    partial);
}

template <typename T>
static void launch_logits_ne(int NE, const void *x, const float *wr, int Tn, int d, int E,
                             int splits, int split_len, float *partial, hipStream_t st) {
  if (NE <= 1) launch_logits<T, 1>(x, wr, Tn, d, E, splits, split_len, partial, st);
  else if (NE <= 2) launch_logits<T, 2>(x, wr, Tn, d, E, splits, split_len, partial, st);
  else if (NE <= 4) launch_logits<T, 4>(x, wr, Tn, d, E, splits, split_len, partial, st);
  else if (NE <= 8) launch_logits<T, 8>(x, wr, Tn, d, E, splits, split_len, partial, st);
  else launch_logits<T, 16>(x, wr, Tn, d, E, splits, split_len, partial, st);
}

void launch_router_logits(bool bf16, const void *x, const float *wr, int Tn, int d, int E,
                          void *ws, int *splits_out, hipStream_t st) {
  int splits = route_splits(Tn, d);
  int chunks = (d + RT_KC - 1) / RT_KC;
  int split_len = ((chunks + splits - 1) / splits) * RT_KC;
  splits = (d + split_len - 1) / split_len;
  float *partial = (float *)ws;
  int NE = (E + 63) / 64;
  if (bf16) launch_logits_ne<bf16_t>(NE, x, wr, Tn, d, E, splits, split_len, partial, st);
  else launch_logits_ne<float>(NE, x, wr, Tn, d, E, splits, split_len, partial, st);
  *splits_out = splits;
}

void launch_router_topk(const void *ws, int splits, const float *bias, int Tn, int E, int k,
                        int32_t *topk_idx, float *gates, float *logits, hipStream_t st) {
  router_topk_kernel<<<(Tn + 3) / 4, 256, 0, st>>>((const float *)ws, splits, bias, Tn, E, k,
                                                   topk_idx, gates, logits);
}

}  // namespace moe
