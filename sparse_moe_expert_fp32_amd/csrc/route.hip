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
//   router_logits  float32 matrix cores (v_mfma_f32_16x16x4_f32: float32
//                  operands, products and sums), a 128-token x 128-expert
//                  tile per 256-thread block fed by an LDS-DMA ring, d
//                  optionally split across blocks so that small token counts
//                  still fill the chip; each split writes its own partial.
//   router_topk    one wave per token (four when a short batch has many
//                  splits): sums the partials in a fixed order, adds the
//                  bias, then k rounds of a wave-wide argmax on the key
//                  (logit desc, index asc) and the softmax of the k winners.
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

constexpr int RT_TM = 128;  // tokens per block
constexpr int RT_TE = 128;  // experts per block

// Block tile 128 tokens x 128 experts, 256 threads = 4 waves as 2 x 2, each
// wave 64 tokens x 64 experts in 4 x 4 v_mfma_f32_16x16x4_f32 tiles (float32
// operands, float32 products and sums: the router stays full precision).
// d runs in 32-deep chunks through a 3-deep LDS ring filled by LDS-DMA:
// x rows as stored ([token][k], bf16 or f32, 16 bytes per lane) and W_r rows
// ([k][expert], one float per lane, so any E works).  Lane group lg takes
// k = 8 lg .. 8 lg + 7 of a chunk, one per MFMA k-step, on both operands.
// Rows past T and experts past E are clamped to valid memory and never
// stored.  blockIdx.z splits d; each split writes its own partial.
typedef float f32x4r_t __attribute__((ext_vector_type(4)));
constexpr int RT_KS = 32;   // d per pipeline stage

DEV float2 ld2f(const float *p) { return *reinterpret_cast<const float2 *>(p); }

template <typename T>
__global__ __launch_bounds__(256, 2) void router_logits_kernel(
    const T *__restrict__ x, const float *__restrict__ wr, int Tn, int d, int E,
    int split_len, float *__restrict__ partial) {
  constexpr int XB = RT_TM * RT_KS * (int)sizeof(T);   // x bytes per stage
  constexpr int WB = RT_KS * RT_TE * 4;                // W bytes per stage
  __shared__ __attribute__((aligned(16))) uint8_t st0[XB + WB];
  __shared__ __attribute__((aligned(16))) uint8_t st1[XB + WB];
  __shared__ __attribute__((aligned(16))) uint8_t st2[XB + WB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4, wm = w & 1, wn = w >> 1;
  const int t0 = blockIdx.x * RT_TM, e0 = blockIdx.y * RT_TE;
  const int c_begin = blockIdx.z * split_len;
  const int c_end = min(d, c_begin + split_len);
  const int NC = (c_end - c_begin) / RT_KS;   // d and split_len are multiples of RT_KS

  // x staging: a row of a stage is RT_KS * sizeof(T) bytes = 16-byte pieces;
  // piece p of the block (p < XB / 16) is row p / PR, piece p % PR
  constexpr int PR = RT_KS * (int)sizeof(T) / 16;
  constexpr int XOPS = XB / 16 / 256;                 // 16-byte DMA per thread
  uint32_t xoff[XOPS];
#pragma unroll
  for (int i = 0; i < XOPS; ++i) {
    const int pc = (w * XOPS + i) * 64 + lane, row = pc / PR, piece = pc % PR;
    xoff[i] = (uint32_t)min(t0 + row, Tn - 1) * (uint32_t)(d * sizeof(T)) + piece * 16;
  }
  // W staging: RT_KS rows of 128 experts, one float per lane: 2 ops per row
  // pair of waves; wave w takes rows w, w + 4, ...
  constexpr int WOPS = RT_KS * 2 / 4;
  const uint32_t woff = (uint32_t)min(e0 + (lane & 63), E - 1) * 4u;
  const uint32_t woff2 = (uint32_t)min(e0 + 64 + (lane & 63), E - 1) * 4u;
  const uint32_t wu = __builtin_amdgcn_readfirstlane(w);
  auto stage = [&](int jr, uint8_t *S) {
    const int j = min(jr, NC - 1);
    const int c0 = c_begin + j * RT_KS;
    const uint32_t base = lds_addr(S);
    const char *xb = reinterpret_cast<const char *>(x) + (size_t)c0 * sizeof(T);
#pragma unroll
    for (int i = 0; i < XOPS; ++i) dma16(xb, xoff[i], base + (wu * XOPS + i) * 1024);
#pragma unroll
    for (int i = 0; i < WOPS / 2; ++i) {
      const int row = (int)wu + 4 * i;
      const float *wrow = wr + (size_t)(c0 + row) * E;
      dma4(wrow, woff, base + XB + (row * RT_TE) * 4);
      dma4(wrow, woff2, base + XB + (row * RT_TE + 64) * 4);
    }
  };

  f32x4r_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4r_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t *S) {
    const T *xs = reinterpret_cast<const T *>(S);
    const float *ws = reinterpret_cast<const float *>(S + XB);
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // k = 8 lg + 4 h .. + 3
      float av[4][4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const T *xr = xs + (64 * wm + 16 * m + lr) * RT_KS + 8 * lg + 4 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) av[m][q] = Elem<T>::ld(xr, q);
      }
      float bv[4][4];
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) bv[n][q] = ws[(8 * lg + 4 * h + q) * RT_TE + 64 * wn + 16 * n + lr];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int n = 0; n < 4; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m][q], bv[n][q], acc[m][n], 0, 0, 0);
    }
  };

  // 3-deep ring: step j computes from slot j % 3 while the loads of step
  // j + 2 are in flight; each step ends with a wait for all of the wave's
  // loads and a block barrier
  stage(0, st0);
  stage(1, st1);
  __builtin_amdgcn_s_waitcnt(kWaitVm);
  block_barrier();
  for (int j = 0; j < NC; j += 3) {
#define MOE_R_STEP(JJ, CUR, NXT)                 \
  {                                              \
    const int jj = (JJ);                         \
    stage(jj + 2, NXT);                          \
    if (jj < NC) compute(CUR);                   \
    __builtin_amdgcn_s_waitcnt(kWaitVm);         \
    block_barrier();                             \
  }
    MOE_R_STEP(j, st0, st2)
    MOE_R_STEP(j + 1, st1, st0)
    MOE_R_STEP(j + 2, st2, st1)
#undef MOE_R_STEP
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);

  float *out = partial + (size_t)blockIdx.z * Tn * E;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int e = e0 + 64 * wn + 16 * n + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 64 * wm + 16 * m + 4 * lg + i;
        if (t < Tn && e < E) out[(size_t)t * E + e] = acc[m][n][i];
      }
    }
}

// (v, e) beats (v2, e2): larger logit, or equal logit and lower index.
DEV bool beats(float v, int e, float v2, int e2) { return v > v2 || (v == v2 && e < e2); }

// The wave's best (v, e) by that order, in every lane (all 64 lanes active):
// DPP exchanges inside each row of 16 lanes (pairs, quads, halves, rows),
// then the four row winners read as scalars.  Every candidate index is
// distinct, so the order is total and the result does not depend on the
// exchange pattern.
template <int CTRL>
DEV void argmax_dpp(float &bv, int &be) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xF, 0xF, false);
  if (beats(ov, oe, bv, be)) { bv = ov; be = oe; }
}
DEV void wave_argmax(float &bv, int &be) {
  argmax_dpp<0xB1>(bv, be);    // quad_perm [1, 0, 3, 2]
  argmax_dpp<0x4E>(bv, be);    // quad_perm [2, 3, 0, 1]
  argmax_dpp<0x141>(bv, be);   // row_half_mirror
  argmax_dpp<0x140>(bv, be);   // row_mirror
  float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int e = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
    const int oe = __builtin_amdgcn_readlane(be, 16 * r);
    if (beats(ov, oe, v, e)) { v = ov; e = oe; }
  }
  bv = v;
  be = e;
}

// WPT waves per token: 1, or 4 for short batches with many splits (wave w
// adds splits w, w + 4, ..., and wave 0 adds the four sums in wave order).
// NEM: logit slots per lane (expert e = lane + 64 n, n < NEM; E <= 64 NEM).
// The partial loads go in batches of NS splits with clamped, unconditional
// addresses, so a batch is one round trip to memory; the sums skip the
// clamped repeats and keep split order.
template <int WPT, int NEM>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float *__restrict__ partial, int splits, const float *__restrict__ bias,
    int Tn, int E, int k, int32_t *__restrict__ topk_idx, float *__restrict__ gates,
    float *__restrict__ logits_out) {
  constexpr int NS = WPT == 1 ? 4 : 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = WPT == 1 ? blockIdx.x * 4 + w : blockIdx.x;
  if (t >= Tn) return;
  float acc[NEM];
#pragma unroll
  for (int n = 0; n < NEM; ++n) acc[n] = 0.f;
  int eoff[NEM];   // clamped expert of each slot
#pragma unroll
  for (int n = 0; n < NEM; ++n) eoff[n] = min(lane + 64 * n, E - 1);
  for (int s0 = WPT == 1 ? 0 : w; s0 < splits; s0 += NS * WPT) {
    float pv[NS][NEM];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int s = min(s0 + i * WPT, splits - 1);
      const float *ps = partial + ((size_t)s * Tn + t) * E;
#pragma unroll
      for (int n = 0; n < NEM; ++n) pv[i][n] = ps[eoff[n]];
    }
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (s0 + i * WPT < splits) {
#pragma unroll
        for (int n = 0; n < NEM; ++n) acc[n] += pv[i][n];
      }
  }
  if constexpr (WPT > 1) {
    __shared__ float red[WPT - 1][NEM][64];
    if (w > 0) {
#pragma unroll
      for (int n = 0; n < NEM; ++n) red[w - 1][n][lane] = acc[n];
    }
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int n = 0; n < NEM; ++n)
#pragma unroll
      for (int i = 0; i < WPT - 1; ++i) acc[n] += red[i][n][lane];
  }
  float l[NEM];
  uint32_t taken = 0;
#pragma unroll
  for (int n = 0; n < NEM; ++n) {
    const int e = lane + 64 * n;
    float v = -INFINITY;
    if (e < E) {
      v = acc[n];
      if (bias) v += bias[e];
      if (logits_out) logits_out[(size_t)t * E + e] = v;
      // a NaN logit (from non-finite x, W_r or bias) competes as -inf, so the
      // selection always takes k distinct experts in [0, E): the order would
      // otherwise never pick it and could run out of candidates
      if (v != v) v = -INFINITY;
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
    for (int n = 0; n < NEM; ++n) {
      const int e = lane + 64 * n;
      if (!((taken >> n) & 1u) && beats(l[n], e, bv, be)) { bv = l[n]; be = e; }
    }
    wave_argmax(bv, be);
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
  const int max_splits = d / RT_KS;   // d is a multiple of the quantization group (>= 32)
  int s = (512 + blocks - 1) / blocks;
  if (s > max_splits) s = max_splits;
  if (s > 32) s = 32;   // (the top-k pass adds the splits of every logit)
  if (s < 1) s = 1;
  return s;
}

size_t route_ws_bytes(int T, int d, int E) {
  return (size_t)route_splits(T, d, E) * T * E * sizeof(float);
}

void launch_router_logits(bool bf16, const void *x, const float *wr, int Tn, int d, int E,
                          void *ws, int *splits_out, hipStream_t st) {
  int splits = route_splits(Tn, d, E);
  const int chunks = d / RT_KS;
  const int split_len = ((chunks + splits - 1) / splits) * RT_KS;
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
  const float *p = (const float *)ws;
#define MOE_TK(WPT, NEM, GRID) \
  router_topk_kernel<WPT, NEM><<<GRID, 256, 0, st>>>(p, splits, bias, Tn, E, k, topk_idx, gates, logits)
  if (splits > 4) {
    if (E <= 512) MOE_TK(4, 8, Tn); else MOE_TK(4, 16, Tn);
  } else {
    if (E <= 512) MOE_TK(1, 8, (Tn + 3) / 4); else MOE_TK(1, 16, (Tn + 3) / 4);
  }
#undef MOE_TK
}

}  // namespace moe
