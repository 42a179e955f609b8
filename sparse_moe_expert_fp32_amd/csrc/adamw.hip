// Adapter optimizer step: AdamW on float32 master copies of the adapters.
//
// The pages keep optimizer state on the low-rank adapters only, the quantized
// base being fixed ("Reversible Sparse MoE Single Node" skill card, Principle
// 3 "TQP Optimizer Strategy" and Pattern 3).  They do not name the optimizer;
// this library reads it as AdamW ("Decoupled Weight Decay Regularization",
// Loshchilov and Hutter): two float32 moments per parameter, bias-corrected,
// with the decay applied to the parameter itself.
//
// Elementwise and bound by HBM: per element 16 bytes read (parameter,
// gradient, two moments) and 12 written (+2 or 4 for the optional copy of the
// parameter in the activation dtype that the next forward reads).  Each thread
// handles 4 consecutive elements per pass with 16-byte nontemporal accesses
// (when every pointer is 16-byte aligned; 15 % faster than cached ones at the
// 62M-parameter shape), the grid strides over the tensor.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

// 16-byte streaming accesses: each element of the step is touched once, so
// the loads and stores bypass cache retention (nontemporal)
typedef float f32x4n_t __attribute__((ext_vector_type(4)));
DEV float4 ld_stream(const float *q, size_t j) {
  const f32x4n_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4n_t *>(q) + j);
  return make_float4(t.x, t.y, t.z, t.w);
}
DEV void st_stream(float *q, size_t j, float4 t) {
  const f32x4n_t u = {t.x, t.y, t.z, t.w};
  __builtin_nontemporal_store(u, reinterpret_cast<f32x4n_t *>(q) + j);
}

// one element: returns the new parameter; m, v updated in place
DEV float adamw_elem(float p, float g, float &m, float &v, const AdamWArgs &h) {
  m = h.beta1 * m + (1.0f - h.beta1) * g;
  v = h.beta2 * v + (1.0f - h.beta2) * (g * g);
  const float denom = sqrtf(v / h.bc2) + h.eps;
  return p - h.lr * ((m / h.bc1) / denom + h.weight_decay * p);
}

// OUT: 0 no copy, 1 float32 copy, 2 bf16 copy (round to nearest even)
template <int OUT, bool VEC>
__global__ __launch_bounds__(256) void adamw_kernel(AdamWArgs h) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (VEC) {
    const size_t n4 = h.n / 4;
    for (size_t i = t0; i < n4; i += stride) {
      float4 p = ld_stream(h.p, i);
      const float4 g = ld_stream(h.g, i);
      float4 m = ld_stream(h.m, i), v = ld_stream(h.v, i);
      p.x = adamw_elem(p.x, g.x, m.x, v.x, h);
      p.y = adamw_elem(p.y, g.y, m.y, v.y, h);
      p.z = adamw_elem(p.z, g.z, m.z, v.z, h);
      p.w = adamw_elem(p.w, g.w, m.w, v.w, h);
      st_stream(h.p, i, p);
      st_stream(h.m, i, m);
      st_stream(h.v, i, v);
      if (OUT == 1) reinterpret_cast<float4 *>(h.out)[i] = p;
      if (OUT == 2)
        reinterpret_cast<uint2 *>(h.out)[i] = make_uint2(pack2bf(p.x, p.y), pack2bf(p.z, p.w));
    }
  }
  // scalar path: the whole tensor, or the last n % 4 elements of the vector path
  for (size_t i = (VEC ? h.n / 4 * 4 : 0) + t0; i < h.n; i += stride) {
    float m = h.m[i], v = h.v[i];
    const float p = adamw_elem(h.p[i], h.g[i], m, v, h);
    h.p[i] = p;
    h.m[i] = m;
    h.v[i] = v;
    if (OUT == 1) reinterpret_cast<float *>(h.out)[i] = p;
    if (OUT == 2) reinterpret_cast<uint16_t *>(h.out)[i] = f2bf(p);
  }
}

void launch_adamw(const AdamWArgs &h, int out_kind, hipStream_t st) {
  const bool vec = ((reinterpret_cast<uintptr_t>(h.p) | reinterpret_cast<uintptr_t>(h.g) |
                     reinterpret_cast<uintptr_t>(h.m) | reinterpret_cast<uintptr_t>(h.v) |
                     (out_kind == 1 ? reinterpret_cast<uintptr_t>(h.out) : 0) |
                     (out_kind == 2 ? reinterpret_cast<uintptr_t>(h.out) << 1 : 0)) & 15) == 0;
  const size_t work = vec ? (h.n + 3) / 4 : h.n;
  const unsigned grid = (unsigned)std::max<size_t>(1, std::min<size_t>((work + 255) / 256, 8192));
#define MOE_ADAMW(O)                                                          \
  if (vec) adamw_kernel<O, true><<<grid, 256, 0, st>>>(h);                    \
  else adamw_kernel<O, false><<<grid, 256, 0, st>>>(h);
  if (out_kind == 1) {
    MOE_ADAMW(1)
  } else if (out_kind == 2) {
    MOE_ADAMW(2)
  } else {
    MOE_ADAMW(0)
  }
#undef MOE_ADAMW
}

}  // namespace moe
