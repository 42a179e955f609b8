// Input-gradient products of the adapter-only backward, on the matrix cores.
//
// Under TQP the base is frozen ("Reversible Sparse MoE Single Node" skill card,
// Principle 3), so the backward only needs the input gradients through each
// expert matrix, i.e. products with the base itself (not its transpose):
//   mode 0:  dH = dO W_d + dZ_d A_d, then the SwiGLU backward
//            dG = dH U s (1 + G (1 - s)), dU = dH G s, s = sigmoid(G)
//   mode 1:  dX_perm = dG W_g + dU W_u + dZ_g A_g + dZ_u A_u
// (dZ = lam dOut B of the same matrix, computed beforehand).
//
// Here the reduction runs over the storage rows of the int4 base and the
// group scale changes with every reduction step, so the exact per-group
// scaling of the forward does not apply.  A pre-pass dequantises the frozen
// base of every expert that received rows into bf16(s * q) (one rounding per
// weight) laid out [E][N_out][K] with the reduction contiguous; the product
// then runs like the forward kernel: A rows through LDS (LDS-DMA, XOR
// swizzle), B straight from global memory into registers one group ahead,
// v_mfma_f32_16x16x32_bf16 into float32 accumulators, persistent
// XCD-partitioned work list, two blocks per CU.
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

constexpr int GT_BM = 64, GT_KG = 128, GT_BN = 256;

// ------------------------------------------------------------ dequantise --
// out[e][c][n] = bf16(s[e][n][c/128] * q[e][n][c]) for experts with rows.
// q: [E][R][C/2] (storage rows R = reduction of the backward), s: [E][R][C/128].
// Block: 64 storage rows x 64 columns; LDS transpose; 16-byte stores along n.
__global__ __launch_bounds__(256) void dequant_t_kernel(const uint8_t *__restrict__ q,
                                                        const uint16_t *__restrict__ s,
                                                        const int32_t *__restrict__ offsets,
                                                        int R, int C, uint16_t *__restrict__ out) {
  __shared__ uint16_t t[64][72];   // [c][n], padded rows
  const int e = blockIdx.z;
  if (offsets[e + 1] == offsets[e]) return;   // no rows routed to this expert
  const int n0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  // read: 64 rows x 8 words; each thread 2 words (row tid/4, words (tid%4)*2 +{0,1})
  {
    const int rr = tid >> 2, wq = (tid & 3) * 2;
    const size_t row = (size_t)e * R + n0 + rr;
    const uint32_t *qw = reinterpret_cast<const uint32_t *>(q + row * (C / 2)) + (c0 >> 3);
    const float sc = bf2f(s[row * (C / 128) + (c0 >> 7)]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t wv = qw[wq + h];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = (wq + h) * 8 + j;
        t[c][rr] = f2bf((float)int4_of_word(wv, j) * sc);
      }
    }
  }
  __syncthreads();
  // write: 64 columns x 8 chunks of 8 n; each thread 2 chunks
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = tid * 2 + h, c = idx >> 3, ch = idx & 7;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(&t[c][ch * 8]);
    uint4 v;
    v.x = src[0]; v.y = src[1]; v.z = src[2]; v.w = src[3];
    *reinterpret_cast<uint4 *>(out + ((size_t)e * C + c0 + c) * R + n0 + ch * 8) = v;
  }
}

// ------------------------------------------------------------ bf16 GEMM --
template <int MODE>
__global__ __launch_bounds__(256, 2) void grouped_gemm_t_kernel(const MfmaGemmTArgs A) {
  // two distinct arrays, so that reads of one are not ordered behind the
  // LDS-DMA writes into the other
  __shared__ __attribute__((aligned(16))) bf16_t lds0[GT_BM * GT_KG];
  __shared__ __attribute__((aligned(16))) bf16_t lds1[GT_BM * GT_KG];
  const int Kh = A.K, N = A.N;
  const int NGh = Kh / GT_KG;
  const int NG = MODE == 1 ? 2 * NGh : NGh;   // mode 1 reduces over [dG | dU]
  const int total = A.ntiles[0] * A.NT;
  const int nper = gridDim.x >> 3, xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int wbeg = (int)(((long long)total * xcd) >> 3);
  const int wend = (int)(((long long)total * (xcd + 1)) >> 3);

  for (int wi = wbeg + bi; wi < wend; wi += nper) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // keep tid-only arithmetic inside the loop
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int ti = wi / A.NT, nt = wi - ti * A.NT;
    const int2 tile = A.tiles[ti];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(GT_BM, A.offsets[e + 1] - p0);
    const int c0 = nt * GT_BN;
    __syncthreads();  // LDS of the previous item is free

    // A staging: 64 rows x 16 chunks, 4 per thread per group (rows p0 + r)
    uint32_t aoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * (w * 4 + j) + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      aoff[j] = (uint32_t)(p0 + min(r, rows - 1)) * (uint32_t)(A.lda * 2) + c * 16;
    }
    auto stage = [&](int g, bf16_t *buf) {
      const bool second = MODE == 1 && g >= NGh;
      const char *base = reinterpret_cast<const char *>(second ? A.a1 : A.a0);
      const size_t koff = (size_t)(second ? g - NGh : g) * GT_KG * 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) load_lds16(base + aoff[j] + koff, buf + (w * 4 + j) * 512);
    };
    // B: this wave's 64 columns, 16 bytes (8 k) per lane per k-step and fragment
    const int cw = min(c0 + w * 64 + lr, N - 1);
    uint4 b0[4][4], b1[4][4];
    auto load_b = [&](int g, uint4 (&b)[4][4]) {
      const bool second = MODE == 1 && g >= NGh;
      const uint16_t *wt = second ? A.w1 : A.w0;
      const int kg = second ? g - NGh : g;
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int c = min(cw + nf * 16, N - 1);
        const uint16_t *col = wt + ((size_t)e * N + c) * Kh + kg * GT_KG + 32 * lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) b[s][nf] = *reinterpret_cast<const uint4 *>(col + 8 * s);
      }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // one k-group: 4 m-fragments x 4 k-steps x 4 column fragments
    auto compute = [&](const bf16_t *al, const uint4 (&b)[4][4]) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 av = *reinterpret_cast<const uint4 *>(
              al + (16 * m + lr) * GT_KG + (((lg * 4 + s) ^ lr) << 3));
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) acc[m][nf] = mfma32(av, b[s][nf], acc[m][nf]);
        }
    };

    // double buffer: even groups in (lds0, b0), odd groups in (lds1, b1)
    stage(0, lds0);
    load_b(0, b0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int g = 0; g < NG; g += 2) {
      if (g + 1 < NG) {
        stage(g + 1, lds1);
        load_b(g + 1, b1);
      }
      compute(lds0, b0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (g + 1 >= NG) break;
      if (g + 2 < NG) {
        stage(g + 2, lds0);
        load_b(g + 2, b0);
      }
      compute(lds1, b1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }

    // adapter term: acc += dZ L with L = A of the matrix ([r][N]), K = rank
    const int nsrc = MODE == 1 ? 2 : 1;
    for (int src = 0; src < nsrc; ++src) {
      const float *Zp = src ? A.Z1 : A.Z0;
      const uint16_t *Lm = src ? A.L1 : A.L0;
      for (int j0 = 0; j0 < A.r; j0 += 16) {
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const int c = min(cw + nf * 16, N - 1);
          short4_t bv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = j0 + 4 * lg + i;
            bv[i] = j < A.r ? (short)Lm[((size_t)e * A.r + j) * N + c] : (short)0;
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int p = p0 + min(16 * m + lr, rows - 1);
            short4_t av;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = j0 + 4 * lg + i;
              av[i] = j < A.r ? (short)f2bf(Zp[(size_t)p * A.ldz + j]) : (short)0;
            }
            acc[m][nf] = mfma16(av, bv, acc[m][nf]);
          }
        }
      }
    }

    // epilogue: results to LDS (two 64 x 128 tiles), then 16-byte stores
    __syncthreads();
    bf16_t *t0 = lds0, *t1 = lds1;
    auto tidx = [](int r, int c) { return r * 128 + ((((c >> 3) ^ (r & 15))) << 3) + (c & 7); };
    bf16_t *tw = w < 2 ? t0 : t1;
    if (MODE == 0) {
      // dG -> tiles, dU kept in registers for a second round
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * m + 4 * lg + i;
          const size_t p = (size_t)(p0 + min(r, rows - 1));
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) {
            const int c = min(cw + nf * 16, N - 1);
            const size_t o = p * N + c;
            const float dh = acc[m][nf][i];
            const float gv = bf2f(A.G[o]), uv = bf2f(A.U[o]);
            const float sg = sigmoid_f(gv);
            tw[tidx(r, (w & 1) * 64 + nf * 16 + lr)] = f2bf(dh * uv * sg * (1.f + gv * (1.f - sg)));
            acc[m][nf][i] = dh * gv * sg;   // dU
          }
          asm volatile("" ::: "memory");   // bound the number of G/U loads in flight
        }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * m + 4 * lg + i;
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
            tw[tidx(r, (w & 1) * 64 + nf * 16 + lr)] = f2bf(acc[m][nf][i]);
        }
    }
    __syncthreads();
    uint16_t *dst = MODE == 0 ? A.dG : A.out;
    const int ldo = MODE == 0 ? N : A.ldo;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int idx = it * 256 + tid, r = idx >> 5, ch = idx & 31;
      const int c = c0 + ch * 8;
      const bf16_t *tr = ch < 16 ? t0 : t1;
      const int chl = ch & 15;
      if (r < rows && c < N)
        *reinterpret_cast<uint4 *>(&dst[(size_t)(p0 + r) * ldo + c]) =
            *reinterpret_cast<const uint4 *>(&tr[r * 128 + ((chl ^ (r & 15)) << 3)]);
    }
    if (MODE == 0) {
      __syncthreads();
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * m + 4 * lg + i;
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
            tw[tidx(r, (w & 1) * 64 + nf * 16 + lr)] = f2bf(acc[m][nf][i]);
        }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + tid, r = idx >> 5, ch = idx & 31;
        const int c = c0 + ch * 8;
        const bf16_t *tr = ch < 16 ? t0 : t1;
        const int chl = ch & 15;
        if (r < rows && c < N)
          *reinterpret_cast<uint4 *>(&A.dU[(size_t)(p0 + r) * N + c]) =
              *reinterpret_cast<const uint4 *>(&tr[r * 128 + ((chl ^ (r & 15)) << 3)]);
      }
    }
  }
}

int mfma_t_tile_rows() { return GT_BM; }
int mfma_t_tile_cols() { return GT_BN; }

void launch_dequant_t(const uint8_t *q, const uint16_t *s, const int32_t *offsets, int E, int R,
                      int C, uint16_t *out, hipStream_t st) {
  dim3 grid(C / 64, R / 64, E);
  dequant_t_kernel<<<grid, 256, 0, st>>>(q, s, offsets, R, C, out);
}

void launch_grouped_gemm_t(int mode, const MfmaGemmTArgs &A, int grid, hipStream_t st) {
  if (mode == 0) grouped_gemm_t_kernel<0><<<grid, 256, 0, st>>>(A);
  else grouped_gemm_t_kernel<1><<<grid, 256, 0, st>>>(A);
}

}  // namespace moe
