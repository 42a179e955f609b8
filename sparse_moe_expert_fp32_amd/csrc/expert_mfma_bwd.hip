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
// operand), blocked by 64 reduction steps, and lays the scales out per column
// group.  The GEMM: 128 x 256 output tile per block, four waves as 2 x 2,
// 64 x 128 per wave (one column group per wave); A rows, int4 words and
// scales stream through a 3-deep LDS ring (LDS-DMA, A XOR-swizzled) in steps
// of 64; v_mfma_f32_16x16x32_bf16 into float32 accumulators; persistent
// XCD-partitioned work list; two blocks per CU, so that one block's VALU work
// (scaling, unpacking) overlaps the other's matrix work.
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

constexpr int GT_BM = 128, GT_BN = 256, GT_KS = 64, GT_BPC = 2;   // GT_BPC: blocks per CU

// ------------------------------------------------------------ transpose --
// q: [E][R][C/2] (packed along C), s: [E][R][C/128] bf16  ->
// qt: [E][R/64][C][32 bytes] (each column's run of 64 storage rows as 8 words,
//     same in-word order as the forward operand), st: [E][C/128][R] f32.
// Experts without rows are skipped.  Block: 64 storage rows x 256 columns, so
// every row is read as one 128-byte run and every output block is one 8 KB
// run; each thread transposes one 8 x 8 nibble block in registers (8 words
// read from 8 rows -> 8 words of 8 columns), re-laid out through LDS.
DEV int nib_slot(int j) { return (j >> 1) + ((j & 1) << 2); }   // slot of element j

__global__ __launch_bounds__(256) void transpose_q_kernel(const uint8_t *__restrict__ q,
                                                          const uint16_t *__restrict__ s,
                                                          const int32_t *__restrict__ offsets,
                                                          int R, int C, uint8_t *__restrict__ qt,
                                                          float *__restrict__ st) {
  __shared__ uint32_t lw[256][9];   // [column][row octet], padded
  const int e = blockIdx.z;
  if (offsets[e + 1] == offsets[e]) return;
  const int n0 = blockIdx.y * 64, c0 = blockIdx.x * 256;
  const int tid = threadIdx.x, cg = tid & 31, a = tid >> 5;   // 8-column group, row octet
  const bool ok = c0 + 8 * cg < C;                           // C is a multiple of 128
  if (ok) {
    uint32_t in[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      in[i] = reinterpret_cast<const uint32_t *>(q + ((size_t)e * R + n0 + 8 * a + i) * (C / 2) +
                                                 c0 / 2)[cg];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t o = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) o |= ((in[i] >> (4 * nib_slot(j))) & 15u) << (4 * nib_slot(i));
      lw[8 * cg + j][a] = o;
    }
  }
  if (tid < 128) {
    const int G = C / 128, g = (c0 >> 7) + (tid >> 6), n = n0 + (tid & 63);
    if (g < G) st[((size_t)e * G + g) * R + n] = bf2f(s[((size_t)e * R + n) * G + g]);
  }
  __syncthreads();
  // 256 columns x 32 bytes, contiguous in the output block: 2 x 16 bytes per thread
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = tid * 2 + h, c = idx >> 1, q2 = idx & 1;
    if (c0 + c >= C) continue;
    uint4 v;
    v.x = lw[c][4 * q2]; v.y = lw[c][4 * q2 + 1]; v.z = lw[c][4 * q2 + 2]; v.w = lw[c][4 * q2 + 3];
    const size_t blk = (size_t)e * (R / 64) + n0 / 64;
    *reinterpret_cast<uint4 *>(qt + (blk * C + c0 + c) * 32 + 16 * q2) = v;
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


template <int MODE>
__global__ __launch_bounds__(256, GT_BPC) void grouped_gemm_t_kernel(const MfmaGemmTArgs A) {
  // a 3-deep ring of stages, each with its A rows, int4 words and scales
  // (filled by LDS-DMA issued from inline asm, with explicit waits)
  __shared__ __attribute__((aligned(16))) bf16_t al0[GT_BM * GT_KS];
  __shared__ __attribute__((aligned(16))) bf16_t al1[GT_BM * GT_KS];
  __shared__ __attribute__((aligned(16))) bf16_t al2[GT_BM * GT_KS];
  __shared__ __attribute__((aligned(16))) uint8_t bl0[GT_BN * GT_KS / 2];
  __shared__ __attribute__((aligned(16))) uint8_t bl1[GT_BN * GT_KS / 2];
  __shared__ __attribute__((aligned(16))) uint8_t bl2[GT_BN * GT_KS / 2];
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

    // A staging: wave w, op i covers rows 8 (4w + i) .. +7 (8 chunks of 16 B each)
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * (w * 4 + i) + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);
      aoff[i] = (uint32_t)(p0 + min(r, rows - 1)) * (uint32_t)(A.lda * 2) + c * 16;
    }
    // int4 staging: wave w, op i covers columns 32 (2w + i) .. +31, 32 bytes each
    uint32_t boff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int col = min(c0 + 32 * (2 * w + i) + (lane >> 1), N - 1);
      boff[i] = (uint32_t)col * 32 + 16 * (lane & 1);
    }
    // scale staging: wave w, lanes < 32: column group (w >> 1), k 32 (w & 1) + lane
    const int sg = min(c0 / 128 + (w >> 1), G - 1);
    const int sk = 32 * (w & 1) + lane;
    // this wave's LDS destinations within a stage (wave-uniform byte offsets)
    const uint32_t wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t la = wu * 4 * 1024, lb = wu * 2 * 1024,
                   ls = ((wu >> 1) * GT_KS + 32 * (wu & 1)) * 4;
    const uint32_t soff = (uint32_t)(sg * Kh + sk) * 4u;
    auto stage = [&](int jr, bf16_t *abuf, uint8_t *bbuf, float *sbuf) {
      const int j = min(jr, NK - 1);   // past the end: a harmless copy of the last step
      const bool second = MODE == 1 && j >= NKh;
      const int kj = second ? j - NKh : j;
      const char *abase = reinterpret_cast<const char *>(second ? A.a1 : A.a0);
      const uint32_t koff = (uint32_t)kj * GT_KS * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(abase + koff, aoff[i], lds_addr(abuf) + la + i * 1024);
      const uint8_t *qb = (second ? A.qt1 : A.qt0) + ((size_t)e * NKh + kj) * N * 32;
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(qb, boff[i], lds_addr(bbuf) + lb + i * 1024);
      const float *sp = (second ? A.st1 : A.st0) + (size_t)e * G * Kh + kj * GT_KS;
      if (lane < 32) dma4(sp, soff, lds_addr(sbuf) + ls);
    };

    f32x4_t acc[4][8], corr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      corr[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // one 64-deep step: 2 k-substeps x 4 row fragments x (8 + 1) MFMAs.
    // Lane group lg takes k = 16 lg + 8 s .. + 7 in substep s (A chunk
    // 2 lg + s, int4 word 2 lg + s), the same permutation on both operands.
    auto compute = [&](const bf16_t *abuf, const uint8_t *bbuf, const float *sbuf) {
      __builtin_amdgcn_sched_barrier(0);
      uint2 bw[8];
#pragma unroll
      for (int nf = 0; nf < 8; ++nf)
        bw[nf] = *reinterpret_cast<const uint2 *>(bbuf + (128 * wn + 16 * nf + lr) * 32 + 8 * lg);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float sc[8];
        {
          const float4 s0 = *reinterpret_cast<const float4 *>(sbuf + wn * GT_KS + 16 * lg + 8 * s);
          const float4 s1 =
              *reinterpret_cast<const float4 *>(sbuf + wn * GT_KS + 16 * lg + 8 * s + 4);
          sc[0] = s0.x; sc[1] = s0.y; sc[2] = s0.z; sc[3] = s0.w;
          sc[4] = s1.x; sc[5] = s1.y; sc[6] = s1.z; sc[7] = s1.w;
        }
        uint4 av[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = 64 * wm + 16 * m + lr;
          const uint4 araw = *reinterpret_cast<const uint4 *>(
              abuf + r * GT_KS + (((2 * lg + s) ^ (r & 7)) << 3));
          av[m] = scale_frag(araw, sc);
          corr[m] = mfma32(av[m], c136, corr[m]);
        }
#pragma unroll
        for (int nf = 0; nf < 8; ++nf) {
          const uint32_t x = s ? bw[nf].y : bw[nf].x;
          uint4 bu;
          bu.x = __builtin_amdgcn_bitop3_b32(x, kMask, kMagic, 0x6A);
          bu.y = __builtin_amdgcn_bitop3_b32(x >> 4, kMask, kMagic, 0x6A);
          bu.z = __builtin_amdgcn_bitop3_b32(x >> 8, kMask, kMagic, 0x6A);
          bu.w = __builtin_amdgcn_bitop3_b32(x >> 12, kMask, kMagic, 0x6A);
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[m][nf] = mfma32(av[m], bu, acc[m][nf]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // 3-deep pipeline: step j computes from ring slot j % 3 while the loads
    // of steps j + 1 and j + 2 are in flight.  Per thread and step: 4 + 2 + 1
    // LDS-DMA (the same count in every wave), so "step j + 1 has landed" is
    // vmcnt(7).  The loop runs in groups of three steps; steps past the end
    // compute nothing (uniform branch) but still issue their loads, clamped to
    // the last real step (cache hits into a slot nobody reads), so that every
    // wait is the same and the compiler's own wait tracking stays exact.
    constexpr int kOps = 7;
    __syncthreads();  // LDS of the previous item is free
    stage(0, al0, bl0, sl0);
    stage(1, al1, bl1, sl1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kOps));
    block_barrier();
    for (int j = 0; j < NK; j += 3) {
#define MOE_T_STEP(JJ, CA, CB, CS, NA, NB, NS)              \
  {                                                         \
    const int jj = (JJ);                                    \
    stage(jj + 2, NA, NB, NS);                              \
    if (jj < NK) compute(CA, CB, CS);                       \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kOps));            \
    block_barrier();                                        \
  }
      MOE_T_STEP(j, al0, bl0, sl0, al2, bl2, sl2)
      MOE_T_STEP(j + 1, al1, bl1, sl1, al0, bl0, sl0)
      MOE_T_STEP(j + 2, al2, bl2, sl2, al1, bl1, sl1)
#undef MOE_T_STEP
    }
    // drain the trailing (clamped) loads before the ring is reused below
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    block_barrier();

    const int cb = c0 + 128 * wn + lr;   // this lane's first output column

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
int mfma_t_blocks_per_cu() { return GT_BPC; }

void launch_transpose_q(const uint8_t *q, const uint16_t *s, const int32_t *offsets, int E, int R,
                        int C, uint8_t *qt, float *st, hipStream_t stream) {
  dim3 grid((C + 255) / 256, R / 64, E);
  transpose_q_kernel<<<grid, 256, 0, stream>>>(q, s, offsets, R, C, qt, st);
}

void launch_grouped_gemm_t(int mode, const MfmaGemmTArgs &A, int grid, hipStream_t st) {
  if (mode == 0) grouped_gemm_t_kernel<0><<<grid, 256, 0, st>>>(A);
  else grouped_gemm_t_kernel<1><<<grid, 256, 0, st>>>(A);
}

}  // namespace moe
