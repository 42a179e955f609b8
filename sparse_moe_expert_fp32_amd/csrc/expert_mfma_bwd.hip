// Input-gradient products of the adapter-only backward, on the matrix cores.
//
// Under TQP the base is frozen ("Reversible Sparse MoE Single Node" skill card,
// Principle 3), so the backward only needs the input gradients through each
// expert matrix, i.e. products with the base itself (the forward uses its
// transpose):
//   mode 0:  dH = dO W_d + dZ_d A_d, then the SwiGLU backward
//            dG = dH U s (1 + G (1 - s)), dU = dH G s, s = sigmoid(G)
//   mode 1:  dX_perm = dG W_g + dU W_u + dZ_g A_g + dZ_u A_u
// (dZ = lam dOut B of the same matrix, computed beforehand).
//
// The reduction runs over the storage rows n of the int4 base, and the group
// scale s[n][c/128] changes with every reduction step but is constant over
// 128 output columns.  So the scale moves onto the other operand:
//   sum_n A[p][n] s[n][g] q[n][c] = sum_n A'_g[p][n] q[n][c],
//   A'_g[p][n] = bf16(A[p][n] s[n][g]),   g = c / 128,
// and the int4 operand stays int4 all the way to the matrix cores, unpacked
// exactly as 136 + q (nibble in the mantissa of 128.0).  The offset is taken
// out by one more MFMA per row fragment against a constant 136 operand, which
// accumulates 136 sum_n A'_g[p][n] from exactly the values the main products
// used.
//
// A pre-pass transposes the int4 nibbles so that each output column holds its
// reduction run as packed words (the same 8-per-word order as the forward
// operand) and lays the scales out per column group.  The GEMM: 128 x 256
// output tile per block, four waves as 2 x 2, 64 x 128 per wave (one column
// group per wave); A rows through a 3-deep LDS ring (LDS-DMA, XOR swizzle),
// scales through LDS, int4 words straight into registers two steps ahead,
// v_mfma_f32_16x16x32_bf16 into float32 accumulators, persistent
// XCD-partitioned work list, one block per CU.
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

constexpr int GT_BM = 128, GT_BN = 256, GT_KS = 128;

// ------------------------------------------------------------ transpose --
// q: [E][R][C/2] (packed along C), s: [E][R][C/128] bf16  ->
// qt: [E][C][R/2] (packed along R, same in-word order), st: [E][C/128][R] f32.
// Experts without rows are skipped.  Block: 128 storage rows x 128 columns;
// each thread transposes one 8 x 8 nibble block in registers (8 words read
// from 8 rows -> 8 words of 8 columns), then the words are re-laid out
// through LDS so that every column is written as 64 contiguous bytes.
DEV int nib_slot(int j) { return (j >> 1) + ((j & 1) << 2); }   // slot of element j

__global__ __launch_bounds__(256) void transpose_q_kernel(const uint8_t *__restrict__ q,
                                                          const uint16_t *__restrict__ s,
                                                          const int32_t *__restrict__ offsets,
                                                          int R, int C, uint8_t *__restrict__ qt,
                                                          float *__restrict__ st) {
  __shared__ uint32_t lw[128][17];   // [column][row block of 8], padded
  const int e = blockIdx.z;
  if (offsets[e + 1] == offsets[e]) return;
  const int n0 = blockIdx.y * 128, c0 = blockIdx.x * 128;
  const int tid = threadIdx.x, wq = tid & 15, a = tid >> 4;
  uint32_t in[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    in[i] = reinterpret_cast<const uint32_t *>(q + ((size_t)e * R + n0 + 8 * a + i) * (C / 2) +
                                               c0 / 2)[wq];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) o |= ((in[i] >> (4 * nib_slot(j))) & 15u) << (4 * nib_slot(i));
    lw[8 * wq + j][a] = o;
  }
  if (tid < 128) {
    const int G = C / 128, g = c0 >> 7;
    st[((size_t)e * G + g) * R + n0 + tid] = bf2f(s[((size_t)e * R + n0 + tid) * G + g]);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = tid * 2 + h, c = idx >> 2, q4 = idx & 3;
    uint4 v;
    v.x = lw[c][4 * q4]; v.y = lw[c][4 * q4 + 1]; v.z = lw[c][4 * q4 + 2]; v.w = lw[c][4 * q4 + 3];
    *reinterpret_cast<uint4 *>(qt + ((size_t)e * C + c0 + c) * (R / 2) + n0 / 2 + 16 * q4) = v;
  }
}

// ------------------------------------------------------------------ GEMM --
// A bf16x8 fragment times 8 per-k scales, rounded back to bf16.
DEV uint4 scale_frag(uint4 a, const float (&sc)[8]) {
  uint4 r;
  r.x = cvt_pk_bf16(__uint_as_float(a.x << 16) * sc[0], __uint_as_float(a.x & 0xffff0000u) * sc[1]);
  r.y = cvt_pk_bf16(__uint_as_float(a.y << 16) * sc[2], __uint_as_float(a.y & 0xffff0000u) * sc[3]);
  r.z = cvt_pk_bf16(__uint_as_float(a.z << 16) * sc[4], __uint_as_float(a.z & 0xffff0000u) * sc[5]);
  r.w = cvt_pk_bf16(__uint_as_float(a.w << 16) * sc[6], __uint_as_float(a.w & 0xffff0000u) * sc[7]);
  return r;
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8).  vmcnt_imm(n): at most n vector memory operations
// (loads, LDS-DMA, stores) of this wave outstanding; kWaitAll: none, and no
// LDS operation either.
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitAll = 0x0070;

template <int MODE>
__global__ __launch_bounds__(256, 1) void grouped_gemm_t_kernel(const MfmaGemmTArgs A) {
  // three distinct ring slots, so that reads of one are not ordered behind
  // the LDS-DMA writes into the others
  __shared__ __attribute__((aligned(16))) bf16_t al0[GT_BM * GT_KS];
  __shared__ __attribute__((aligned(16))) bf16_t al1[GT_BM * GT_KS];
  __shared__ __attribute__((aligned(16))) bf16_t al2[GT_BM * GT_KS];
  __shared__ __attribute__((aligned(16))) float sl0[2 * GT_KS];
  __shared__ __attribute__((aligned(16))) float sl1[2 * GT_KS];
  __shared__ __attribute__((aligned(16))) float sl2[2 * GT_KS];

  const int Kh = A.K, N = A.N, G = N / 128;
  const int NKh = Kh / GT_KS;
  const int NK = MODE == 1 ? 2 * NKh : NKh;   // mode 1 reduces over [dG | dU]
  const int total = A.ntiles[0] * A.NT;
  const int nper = gridDim.x >> 3, xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int wbeg = (int)(((long long)total * xcd) >> 3);
  const int wend = (int)(((long long)total * (xcd + 1)) >> 3);
  const uint4 c136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};   // bf16 136
  // int4 unpack: each bf16 pair of 136 + q is one shift and one three-input
  // logic op, ((w >> 4i) & 0x000F000F) ^ 0x43084308 (constants in registers)
  const uint32_t kMask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t kMagic;
  asm volatile("v_mov_b32 %0, 0x43084308" : "=v"(kMagic));

  for (int wi = wbeg + bi; wi < wend; wi += nper) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // keep tid-only arithmetic inside the loop
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int wm = w & 1, wn = w >> 1;
    const int ti = wi / A.NT, nt = wi - ti * A.NT;
    const int2 tile = A.tiles[ti];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(GT_BM, A.offsets[e + 1] - p0);
    const int c0 = nt * GT_BN;

    // A staging: wave w, instruction i covers rows 4 (8w + i) .. +3
    uint32_t aoff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * (w * 8 + i) + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      aoff[i] = (uint32_t)(p0 + min(r, rows - 1)) * (uint32_t)(A.lda * 2) + c * 16;
    }
    // scale staging: wave w: column group (w >> 1), k 64 (w & 1) + lane
    const int sg = min(c0 / 128 + (w >> 1), G - 1);
    const int sk = 64 * (w & 1) + lane;
    // int4 words: this wave's 128 columns, words 4 lg .. 4 lg + 3 of each step
    const int cb = c0 + 128 * wn + lr;
    auto stage = [&](int jr, bf16_t *abuf, float *sbuf) {
      const int j = min(jr, NK - 1);
      const bool second = MODE == 1 && j >= NKh;
      const int kj = second ? j - NKh : j;
      const char *base = reinterpret_cast<const char *>(second ? A.a1 : A.a0);
      const uint32_t koff = (uint32_t)kj * GT_KS * 2;
#pragma unroll
      for (int i = 0; i < 8; ++i) load_lds16(base + aoff[i] + koff, abuf + (w * 8 + i) * 512);
      const float *sp = second ? A.st1 : A.st0;
      load_lds4(sp + ((size_t)e * G + sg) * Kh + kj * GT_KS + sk, sbuf + w * 64);
    };
    auto load_b = [&](int jr, uint4 (&b)[8]) {
      const int j = min(jr, NK - 1);
      const bool second = MODE == 1 && j >= NKh;
      const int kj = second ? j - NKh : j;
      const uint8_t *qp = second ? A.qt1 : A.qt0;
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) {
        const int c = min(cb + 16 * nf, N - 1);
        b[nf] = *reinterpret_cast<const uint4 *>(qp + ((size_t)e * N + c) * (Kh / 2) +
                                                 kj * (GT_KS / 2) + 16 * lg);
      }
    };

    f32x4_t acc[4][8], corr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      corr[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // one 128-deep step: 4 k-substeps x 4 row fragments x (8 + 1) MFMAs.
    // Lane group lg takes k = 32 lg + 8 s .. + 7 in substep s (A chunk
    // 4 lg + s, int4 word 4 lg + s), the same permutation on both operands.
    auto compute = [&](const bf16_t *abuf, const float *sbuf, const uint4 (&b)[8]) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float sc[8];
        {
          const float4 s0 = *reinterpret_cast<const float4 *>(sbuf + wn * GT_KS + 32 * lg + 8 * s);
          const float4 s1 =
              *reinterpret_cast<const float4 *>(sbuf + wn * GT_KS + 32 * lg + 8 * s + 4);
          sc[0] = s0.x; sc[1] = s0.y; sc[2] = s0.z; sc[3] = s0.w;
          sc[4] = s1.x; sc[5] = s1.y; sc[6] = s1.z; sc[7] = s1.w;
        }
        uint4 av[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = 64 * wm + 16 * m + lr;
          const uint4 araw = *reinterpret_cast<const uint4 *>(
              abuf + r * GT_KS + (((4 * lg + s) ^ (r & 15)) << 3));
          av[m] = scale_frag(araw, sc);
          corr[m] = mfma32(av[m], c136, corr[m]);
        }
#pragma unroll
        for (int nf = 0; nf < 8; ++nf) {
          const uint32_t x = s == 0 ? b[nf].x : s == 1 ? b[nf].y : s == 2 ? b[nf].z : b[nf].w;
          uint4 bu;
          bu.x = __builtin_amdgcn_bitop3_b32(x, kMask, kMagic, 0x6A);
          bu.y = __builtin_amdgcn_bitop3_b32(x >> 4, kMask, kMagic, 0x6A);
          bu.z = __builtin_amdgcn_bitop3_b32(x >> 8, kMask, kMagic, 0x6A);
          bu.w = __builtin_amdgcn_bitop3_b32(x >> 12, kMask, kMagic, 0x6A);
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[m][nf] = mfma32(av[m], bu, acc[m][nf]);
        }
      }
    };

    // 3-deep pipeline: step j computes from ring slot j % 3 while the loads
    // of step j + 2 are in flight.  Per thread and step: 8 word loads, 8 + 1
    // LDS-DMA (the same count in every wave), so "step j + 1 has landed" is
    // vmcnt(17).  The loop runs in groups of three steps; steps past the end
    // compute nothing (uniform branch) but still issue their loads, clamped to
    // the last real step (cache hits into a slot nobody reads), so that every
    // wait is the same and the compiler's own wait tracking stays exact.  The
    // scheduling barriers keep each step's loads ahead of the MFMAs, where
    // the scheduler would otherwise sink them next to their wait.
    constexpr int kOps = 17;
    uint4 b0[8], b1[8], b2[8];
    __syncthreads();  // LDS of the previous item is free
    load_b(0, b0);
    stage(0, al0, sl0);
    load_b(1, b1);
    stage(1, al1, sl1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kOps));
    block_barrier();
    for (int j = 0; j < NK; j += 3) {
#define MOE_T_STEP(JJ, CUR_A, CUR_S, CUR_B, NXT_A, NXT_S, NXT_B) \
  {                                                              \
    const int jj = (JJ);                                         \
    load_b(jj + 2, NXT_B);                                       \
    stage(jj + 2, NXT_A, NXT_S);                                 \
    __builtin_amdgcn_sched_barrier(0);                           \
    if (jj < NK) compute(CUR_A, CUR_S, CUR_B);                   \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kOps));                 \
    block_barrier();                                             \
  }
      MOE_T_STEP(j, al0, sl0, b0, al2, sl2, b2)
      MOE_T_STEP(j + 1, al1, sl1, b1, al0, sl0, b0)
      MOE_T_STEP(j + 2, al2, sl2, b2, al1, sl1, b1)
#undef MOE_T_STEP
    }
    // drain the trailing (clamped) loads before the ring is reused below
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    block_barrier();

    // remove the 136 offset of the int4 operand
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) acc[m][nf] -= corr[m];

    // adapter term: acc += dZ L with L = A of the matrix ([r][N]), K = rank.
    // Loads are unconditional (clamped indices) so that they issue together;
    // rank columns beyond r are zeroed afterwards.
    const int nsrc = MODE == 1 ? 2 : 1;
    for (int src = 0; src < nsrc; ++src) {
      const float *Zp = src ? A.Z1 : A.Z0;
      const uint16_t *Lm = src ? A.L1 : A.L0;
      for (int j0 = 0; j0 < A.r; j0 += 16) {
        float zv[4][4];
        uint16_t lv[8][4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int p = p0 + min(64 * wm + 16 * m + lr, rows - 1);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            zv[m][i] = Zp[(size_t)p * A.ldz + min(j0 + 4 * lg + i, A.r - 1)];
        }
#pragma unroll
        for (int nf = 0; nf < 8; ++nf) {
          const int c = min(cb + 16 * nf, N - 1);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            lv[nf][i] = Lm[((size_t)e * A.r + min(j0 + 4 * lg + i, A.r - 1)) * N + c];
        }
        short4_t av[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            av[m][i] = j0 + 4 * lg + i < A.r ? (short)f2bf(zv[m][i]) : (short)0;
#pragma unroll
        for (int nf = 0; nf < 8; ++nf) {
          short4_t bv;
#pragma unroll
          for (int i = 0; i < 4; ++i) bv[i] = j0 + 4 * lg + i < A.r ? (short)lv[nf][i] : (short)0;
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[m][nf] = mfma16(av[m], bv, acc[m][nf]);
        }
      }
    }

    // epilogue: per 16-row fragment, through a wave-private 16 x 128 LDS tile
    // (slot 0 of the ring is free: every wave passed the loop's last barrier)
    bf16_t *tw = al0 + w * (16 * 128);
    const bool cols_ok = c0 + 128 * wn < N;   // N is a multiple of 128
    auto tidx = [](int r, int c) { return r * 128 + (((c >> 3) ^ r) << 3) + (c & 7); };
    auto flush = [&](int m, uint16_t *dst, int ldo) {
      // 16 rows x 16 chunks of 8 columns: 4 chunks per lane
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int idx = it * 64 + lane, r = idx >> 4, ch = idx & 15;
        const int rr = 64 * wm + 16 * m + r;
        const uint4 v = *reinterpret_cast<const uint4 *>(&tw[r * 128 + ((ch ^ r) << 3)]);
        if (cols_ok && rr < rows)
          *reinterpret_cast<uint4 *>(&dst[(size_t)(p0 + rr) * ldo + c0 + 128 * wn + ch * 8]) = v;
      }
    };
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (MODE == 0) {
        float du[8][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 64 * wm + 16 * m + 4 * lg + i;
          const size_t p = (size_t)(p0 + min(rr, rows - 1));
#pragma unroll
          for (int nf = 0; nf < 8; ++nf) {
            const size_t o = p * N + min(cb + 16 * nf, N - 1);
            const float dh = acc[m][nf][i];
            const float gv = bf2f(A.G[o]), uv = bf2f(A.U[o]);
            const float sgm = sigmoid_f(gv);
            tw[tidx(4 * lg + i, 16 * nf + lr)] = f2bf(dh * uv * sgm * (1.f + gv * (1.f - sgm)));
            du[nf][i] = dh * gv * sgm;
          }
        }
        flush(m, A.dG, N);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nf = 0; nf < 8; ++nf) tw[tidx(4 * lg + i, 16 * nf + lr)] = f2bf(du[nf][i]);
        flush(m, A.dU, N);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nf = 0; nf < 8; ++nf) tw[tidx(4 * lg + i, 16 * nf + lr)] = f2bf(acc[m][nf][i]);
        flush(m, A.out, A.ldo);
      }
    }
  }
}

int mfma_t_tile_rows() { return GT_BM; }
int mfma_t_tile_cols() { return GT_BN; }

void launch_transpose_q(const uint8_t *q, const uint16_t *s, const int32_t *offsets, int E, int R,
                        int C, uint8_t *qt, float *st, hipStream_t stream) {
  dim3 grid(C / 128, R / 128, E);
  transpose_q_kernel<<<grid, 256, 0, stream>>>(q, s, offsets, R, C, qt, st);
}

void launch_grouped_gemm_t(int mode, const MfmaGemmTArgs &A, int grid, hipStream_t st) {
  if (mode == 0) grouped_gemm_t_kernel<0><<<grid, 256, 0, st>>>(A);
  else grouped_gemm_t_kernel<1><<<grid, 256, 0, st>>>(A);
}

}  // namespace moe
