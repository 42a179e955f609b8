// Grouped int4 x bf16 GEMMs of the adapter-only backward, on the matrix cores.
//
// Under TQP the base is frozen ("Reversible Sparse MoE Single Node" skill card,
// Principle 3), so the backward only needs the input gradients of the expert
// matrices, i.e. products with the TRANSPOSED base:
//   mode 0:  dH = dO W_d + dZ_d A_d, then the SwiGLU backward
//            dG = dH U s (1 + G (1 - s)), dU = dH G s, s = sigmoid(G)
//   mode 1:  dX_perm = dG W_g + dU W_u + dZ_g A_g + dZ_u A_u
// (dZ = lam dOut B of the same matrix, computed beforehand; adapters are
// stored out x in).
//
// Transposed use of the int4 storage: the reduction index is the storage row
// n and the output column c is the packed dimension, and the group scale
// s[n][c/128] changes with every reduction step.  Each work item (128 rows x
// 128 output columns, one scale group) therefore dequantises its weight
// block into LDS: a thread takes an 8 x 8 (rows x columns) nibble block,
// forms bf16(s[n] * q[n][c]) (one rounding per weight) and writes the eight
// columns as 16-byte K-runs, XOR-swizzled like the A rows.  The A rows stream
// through LDS with global_load_lds_dwordx4 as in the forward.  Both operands
// are double buffered; a persistent grid walks an XCD-partitioned work list.
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

constexpr int GT_BM = 128, GT_BN = 128, GT_KG = 128;

template <int MODE>
__global__ __launch_bounds__(256, 1) void grouped_gemm_t_kernel(const MfmaGemmTArgs A) {
  __shared__ __attribute__((aligned(16))) bf16_t a_lds[2][GT_BM * GT_KG];
  __shared__ __attribute__((aligned(16))) bf16_t b_lds[2][GT_BN * GT_KG];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int Kh = A.K, N = A.N;
  const int NGh = Kh / GT_KG;                 // chunks per source
  const int NG = MODE == 1 ? 2 * NGh : NGh;   // mode 1 reduces over [dG | dU]
  const int NS = N / 128;                     // scale groups per storage row
  const int total = A.ntiles[0] * A.NT;
  const int nper = gridDim.x >> 3, xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int wbeg = (int)(((long long)total * xcd) >> 3);
  const int wend = (int)(((long long)total * (xcd + 1)) >> 3);
  // B staging role: rows 8*rb .. 8*rb+7 of the chunk, columns 8*cb .. 8*cb+7
  const int rb = tid & 15, cb = tid >> 4;

  for (int wi = wbeg + bi; wi < wend; wi += nper) {
    const int ti = wi / A.NT, nt = wi - ti * A.NT;
    const int2 tile = A.tiles[ti];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(GT_BM, A.offsets[e + 1] - p0);
    const int c0 = nt * GT_BN;

    // A staging: 8 chunks of 16 bytes per thread per K-chunk (rows p0 + r)
    size_t aoff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * (w * 8 + j) + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      aoff[j] = (size_t)(p0 + min(r, rows - 1)) * A.lda * 2 + c * 16;
    }
    auto stage_a = [&](int g, int buf) {
      const char *base = reinterpret_cast<const char *>(MODE == 1 && g >= NGh ? A.a1 : A.a0);
      const size_t koff = (size_t)(MODE == 1 && g >= NGh ? g - NGh : g) * GT_KG * 2;
#pragma unroll
      for (int j = 0; j < 8; ++j) load_lds16(base + aoff[j] + koff, &a_lds[buf][(w * 8 + j) * 512]);
    };
    // B staging: 8 words (rows) and 8 scales of this thread's block
    uint32_t bw[8];
    float bs[8];
    auto load_b = [&](int g) {
      const uint8_t *q = MODE == 1 && g >= NGh ? A.q1 : A.q0;
      const uint16_t *s = MODE == 1 && g >= NGh ? A.s1 : A.s0;
      const int n0 = (MODE == 1 && g >= NGh ? g - NGh : g) * GT_KG + 8 * rb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const size_t row = (size_t)e * Kh + n0 + i;
        bw[i] = reinterpret_cast<const uint32_t *>(q + row * (N / 2))[(c0 >> 3) + cb];
        bs[i] = bf2f(s[row * NS + nt]);
      }
    };
    auto store_b = [&](int buf) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)int4_of_word(bw[i], j) * bs[i];
        uint4 o;
        o.x = cvt_pk_bf16(v[0], v[1]);
        o.y = cvt_pk_bf16(v[2], v[3]);
        o.z = cvt_pk_bf16(v[4], v[5]);
        o.w = cvt_pk_bf16(v[6], v[7]);
        const int c = 8 * cb + j;
        *reinterpret_cast<uint4 *>(&b_lds[buf][c * GT_KG + ((rb ^ (c & 15)) << 3)]) = o;
      }
    };

    f32x4_t acc[8][2];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int nf = 0; nf < 2; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // LDS of the previous item is free
    stage_a(0, 0);
    load_b(0);
    store_b(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int g = 0; g < NG; ++g) {
      const int cur = g & 1;
      if (g + 1 < NG) {
        stage_a(g + 1, cur ^ 1);
        load_b(g + 1);
      }
      // this wave's B fragments for the 4 k-steps and 2 column fragments
      uint4 bf[4][2];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const int c = w * 32 + nf * 16 + lr;
          bf[s][nf] = *reinterpret_cast<const uint4 *>(
              &b_lds[cur][c * GT_KG + (((4 * lg + s) ^ (c & 15)) << 3)]);
        }
      const bf16_t *al = a_lds[cur];
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 av = *reinterpret_cast<const uint4 *>(
              al + (16 * m + lr) * GT_KG + (((lg * 4 + s) ^ lr) << 3));
#pragma unroll
          for (int nf = 0; nf < 2; ++nf) acc[m][nf] = mfma32(av, bf[s][nf], acc[m][nf]);
        }
      if (g + 1 < NG) store_b(cur ^ 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }

    // adapter term: acc += dZ L^T with L = A of the matrix ([r][N]), K = rank
    const int nsrc = MODE == 1 ? 2 : 1;
    for (int src = 0; src < nsrc; ++src) {
      const float *Zp = src ? A.Z1 : A.Z0;
      const uint16_t *Lm = src ? A.L1 : A.L0;
      for (int j0 = 0; j0 < A.r; j0 += 16) {
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const int c = c0 + w * 32 + nf * 16 + lr;
          short4_t bv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = j0 + 4 * lg + i;
            bv[i] = j < A.r ? (short)Lm[((size_t)e * A.r + j) * N + c] : (short)0;
          }
#pragma unroll
          for (int m = 0; m < 8; ++m) {
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

    // epilogue
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * m + 4 * lg + i;
        if (rr >= rows) continue;
        const size_t p = (size_t)(p0 + rr);
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const int c = c0 + w * 32 + nf * 16 + lr;
          const float v = acc[m][nf][i];
          if (MODE == 0) {
            const size_t o = p * N + c;
            const float gv = bf2f(A.G[o]), uv = bf2f(A.U[o]);
            const float sg = sigmoid_f(gv);
            A.dG[o] = f2bf(v * uv * sg * (1.f + gv * (1.f - sg)));
            A.dU[o] = f2bf(v * gv * sg);
          } else {
            A.out[p * A.ldo + c] = f2bf(v);
          }
        }
      }
  }
}

int mfma_t_tile_rows() { return GT_BM; }

void launch_grouped_gemm_t(int mode, const MfmaGemmTArgs &A, int grid, hipStream_t st) {
  if (mode == 0) grouped_gemm_t_kernel<0><<<grid, 256, 0, st>>>(A);
  else grouped_gemm_t_kernel<1><<<grid, 256, 0, st>>>(A);
}

}  // namespace moe
