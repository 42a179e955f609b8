// Device helpers shared by the HIP kernels of the TQP expert layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 carried as raw bits

#define DEV __device__ __forceinline__

// ---------------------------------------------------------------- bf16 --
DEV float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even (inputs here are finite).
DEV uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// two floats -> packed bf16 pair (lo in bits 0..15)
DEV uint32_t pack2bf(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// Typed element access: float storage or bf16 storage, float arithmetic.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static DEV float ld(const float *p, size_t i) { return p[i]; }
  static DEV void st(float *p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static DEV float ld(const bf16_t *p, size_t i) { return bf2f(p[i]); }
  static DEV void st(bf16_t *p, size_t i, float v) { p[i] = f2bf(v); }
};

// Round a float through the storage type (identity for float).
template <typename T> DEV float through(float v);
template <> DEV float through<float>(float v) { return v; }
template <> DEV float through<bf16_t>(float v) { return bf2f(f2bf(v)); }

// ---------------------------------------------------------------- int4 --
// Element c of a packed int4 row (see moe_qlora in moe_tqp.h): word c/8,
// nibble slot (c%8)/2 for even c%8 and (c%8)/2 + 4 for odd.
DEV int int4_at(const uint8_t *row, int c) {
  uint32_t w = reinterpret_cast<const uint32_t *>(row)[c >> 3];
  int m = c & 7;
  int slot = (m >> 1) + ((m & 1) << 2);
  int nib = (w >> (4 * slot)) & 0xF;
  return (nib ^ 8) - 8;
}

DEV float silu_f(float z) { return z / (1.0f + __expf(-z)); }
DEV float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }

DEV int ceil_div(int a, int b) { return (a + b - 1) / b; }
