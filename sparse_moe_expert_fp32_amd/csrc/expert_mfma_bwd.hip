// Input-gradient products of the adapter-only backward, on the matrix cores.
//
// Under TQP the base is frozen ("Reversible Sparse MoE Single Node" skill card,
// Principle 3), so the backward only needs the input gradients through each
// expert matrix, i.e. products with the base itself (the forward uses its
// transpose):
//   mode 0:  dH = dO W_d + dZ_d A_d, then the SwiGLU backward
//            dG = dH U s (1 + G (1 - s)), dU = dH G s, s = sigmoid(G)
//   mode 1:  dX_perm = dG W_g + dU W_u + dZ_g A_g + dZ_u A_u
// (dZ = lam dOut B of the same matrix, computed beforehand).  The output
// gradient of a permuted row p is its gate times the upstream gradient of its
// token, dO[p] = g_p dy[t(p)], so mode 0 reads the rows of dy by token and
// multiplies the product's row by g_p (dZ_d already carries it): dO is never
// materialised.
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
// Experts without rows are skipped (all are transposed when offsets is null).  Block: 64 storage rows x 256 columns, so
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
  if (offsets && offsets[e + 1] == offsets[e]) return;
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

// One pipeline stage in LDS, one array per kind (each read is a per-lane base
// register plus a compile-time offset): A rows (128 x 64 bf16, 16-byte chunks
// XOR-swizzled by row), int4 words (256 columns x 32 bytes), the scales of the
// stage's 64 reduction steps for the block's two column groups.
constexpr int TS_B = GT_BN * GT_KS / 2, TS_S = 2 * GT_KS * 4;   // (the A stage holds the class's rows)
// blocks per CU of tile class NMH, as LDS (the A ring holds 32 NMH rows) and
// registers allow: 32-row tiles four, 64-row tiles three, the others two
constexpr int gt_bpc(int NMH) { return NMH <= 1 ? 4 : NMH == 2 ? 3 : GT_BPC; }

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

// NMH: row fragments of 16 per wave; the item's tile class has 32 NMH rows
// (128, 96, 64, 32), each class its own launch.  Waves 2 x 2: wave (wm, wn)
// takes rows 16 NMH wm .. + 16 NMH and the 128 columns of column group wn.
// Products are formed transposed (D^T = W^T A^T: the unpacked weights are the
// first MFMA operand) so a lane holds one row and four consecutive columns and
// the epilogue reads G, U and writes its results 8 bytes at a time.
template <int MODE, int NMH, bool EPL>
__global__ __launch_bounds__(256, gt_bpc(NMH)) void grouped_gemm_t_kernel(
    const MfmaGemmTArgs A, const int *__restrict__ cls_count, const int *__restrict__ cls_start) {
  // a 3-deep ring of stages (filled by LDS-DMA issued from inline asm, with
  // explicit waits)
  // (ringA 32-byte aligned: the second substep's chunk is the first's
  // address with bit 4 flipped)
  constexpr int TS_A = 32 * NMH * GT_KS * 2;   // A stage: the class's rows x 64 K
  __shared__ __attribute__((aligned(32))) uint4 ringA[3][TS_A / 16];
  __shared__ uint4 ringB[3][TS_B / 16];
  __shared__ float ringS[3][TS_S / 4];
  constexpr int AOPS = NMH;   // 8-row A loads per wave and stage

  const int Kh = A.K, N = A.N, G = N / 128;
  const int NKh = Kh / GT_KS;
  const int NK = MODE == 1 ? 2 * NKh : NKh;   // mode 1 reduces over [dG | dU]
  const int total = cls_count[0] * A.NT, tbase = cls_start[0];
  const int nper = gridDim.x >> 3, xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int wbeg = (int)(((long long)total * xcd) >> 3);
  const int wend = (int)(((long long)total * (xcd + 1)) >> 3);
  const uint4 c136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};   // bf16 136
  // int4 unpack: each bf16 pair of 136 + q is one shift and one three-input
  // logic op, ((w >> 4i) & 0x000F000F) ^ 0x43084308 (constants in registers)
  const uint32_t kMask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t kMagic;
  asm volatile("v_mov_b32 %0, 0x43084308" : "=v"(kMagic));
  const uint32_t ldsA = lds_addr(ringA), ldsB = lds_addr(ringB), ldsS = lds_addr(ringS);

  for (int wi = wbeg + bi; wi < wend; wi += nper) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // keep tid-only arithmetic inside the loop
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int wm = w & 1, wn = w >> 1;
    const int ti = wi / A.NT, nt = wi - ti * A.NT;
    const int2 tile = A.tiles[tbase + ti];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(32 * NMH, A.offsets[e + 1] - p0);
    const int c0 = nt * GT_BN;

    // A staging: wave w, load i covers rows 8 (AOPS w + i) .. +7 (8 chunks of
    // 16 B each); chunk c of row r lives at c ^ row_swz(r)
    // (mode 0 with gate scaling: the rows of dy by token)
    const bool tokrows = MODE == 0 && A.gsc != nullptr;
    uint32_t aoff[AOPS];
#pragma unroll
    for (int i = 0; i < AOPS; ++i) {
      const int r = 8 * (w * AOPS + i) + (lane >> 3);
      const int c = (lane & 7) ^ row_swz(r);
      const int p = p0 + min(r, rows - 1);
      const int arow = tokrows ? A.perm_src[p] / A.kk : p;
      aoff[i] = (uint32_t)arow * (uint32_t)(A.lda * 2) + c * 16;
    }
    // int4 staging: wave w, load i covers columns 32 (2w + i) .. +31, 32 bytes each
    uint32_t boff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int col = min(c0 + 32 * (2 * w + i) + (lane >> 1), N - 1);
      boff[i] = (uint32_t)col * 32 + 16 * (lane & 1);
    }
    // scale staging: wave w, lanes < 32: column group (w >> 1), k 32 (w & 1) + lane
    const int sg = min(c0 / 128 + (w >> 1), G - 1);
    const int sk = 32 * (w & 1) + lane;
    const uint32_t soff = (uint32_t)(sg * Kh + sk) * 4u;
    // this wave's LDS-DMA destinations within a stage (wave-uniform)
    const uint32_t wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t la = ldsA + wu * AOPS * 1024, lb = ldsB + wu * 2 * 1024,
                   ls = ldsS + ((wu >> 1) * GT_KS + 32 * (wu & 1)) * 4;
    // per-lane LDS read bases (bytes); the rest of every read address is a
    // compile-time constant
    const uint32_t offA0 = opaque(ldsA + (16 * NMH * wm + lr) * 128 + (((2 * lg) ^ row_swz(lr)) << 4)),
                   offB = opaque(ldsB + (128 * wn + lr) * 32 + 8 * lg),
                   offS = opaque(ldsS + (wn * GT_KS + 16 * lg) * 4);

    // the row gates (mode 0, rows of dy by token), fetched now for the epilogue
    float gm[NMH];
#pragma unroll
    for (int m = 0; m < NMH; ++m) {
      const int r = 16 * NMH * wm + lr + 16 * m;
      gm[m] = MODE == 0 && A.gsc ? A.gsc[A.perm_src[p0 + min(r, rows - 1)]] : 1.f;
    }

    // EPL (rank 16): the epilogue's operands come through the ring as the
    // stages after the last: stage NK brings the rows' dZ (Z_d, or Z_g then
    // Z_u: 64 floats at most, with the A swizzle) into the A array and the
    // transposed adapter A of the block columns (32 bytes each) into the
    // word array; in mode 1 stage NK + 1 brings that of the second matrix.
    auto stage_ep = [&](int part, int slot) {
      uint32_t sa = la, sb = lb;
      asm volatile("" : "+s"(sa), "+s"(sb));
      if (part == 0) {
        const char *zb = reinterpret_cast<const char *>(uniform_ptr(A.Z0));
#pragma unroll
        for (int i = 0; i < AOPS; ++i) {
          const int r = 8 * (w * AOPS + i) + (lane >> 3);
          const int c = ((lane & 7) ^ row_swz(r)) & (MODE == 1 ? 7 : 3);   // Z_d: 4 chunks
          const uint32_t zo = (uint32_t)(p0 + min(r, rows - 1)) * (uint32_t)(A.ldz * 4) + c * 16;
          dma16(zb, zo, sa + slot * TS_A + i * 1024);
        }
      }
      const char *lb16 = reinterpret_cast<const char *>(uniform_ptr((part ? A.LT1 : A.LT0) + (size_t)e * N * 16));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int col = min(c0 + 32 * (2 * w + i) + (lane >> 1), N - 1);
        dma16(lb16, (uint32_t)col * 32u + 16 * (lane & 1), sb + slot * TS_B + i * 1024);
      }
    };
    auto stage = [&](int jr, int slot) {
      if (EPL && jr >= NK) {
        if (jr == NK) stage_ep(0, slot);
        else if (MODE == 1 && jr == NK + 1) stage_ep(1, slot);
        return;
      }
      const int j = min(jr, NK - 1);   // past the end: a harmless copy of the last step
      const bool second = MODE == 1 && j >= NKh;
      const int kj = second ? j - NKh : j;
      const char *abase = reinterpret_cast<const char *>(second ? A.a1 : A.a0);
      const uint32_t koff = (uint32_t)kj * GT_KS * 2;
      // destinations re-derived per stage (scalar adds) rather than held
      uint32_t sa = la, sb = lb, ss = ls;
      asm volatile("" : "+s"(sa), "+s"(sb), "+s"(ss));
#pragma unroll
      for (int i = 0; i < AOPS; ++i) dma16(abase + koff, aoff[i], sa + slot * TS_A + i * 1024);
      const uint8_t *qb = (second ? A.qt1 : A.qt0) + ((size_t)e * NKh + kj) * N * 32;
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(qb, boff[i], sb + slot * TS_B + i * 1024);
      const float *sp = (second ? A.st1 : A.st0) + (size_t)e * G * Kh + kj * GT_KS;
      if (lane < 32) dma4(sp, soff, ss + slot * TS_S);
    };

    f32x4_t acc[NMH][8], corr[NMH];
#pragma unroll
    for (int m = 0; m < NMH; ++m) {
      corr[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // one 64-deep step: 2 k-substeps x NMH row fragments x (8 + 1) MFMAs.
    // Lane group lg takes k = 16 lg + 8 s .. + 7 in substep s (A chunk
    // 2 lg + s, int4 word 2 lg + s), the same permutation on both operands.
    auto compute = [&](int slot) {
      __builtin_amdgcn_sched_barrier(0);
      u32x2_t bw[8];
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) bw[nf] = lds_ld<u32x2_t>(offB + slot * TS_B + nf * 16 * 32);
      // substep 1 reads chunk 2 lg + 1, the neighbouring swizzled chunk
      const uint32_t offA1 = offA0 ^ 16u;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float sc[8];
        {
          const f32x4_t s0 = lds_ld<f32x4_t>(offS + slot * TS_S + 32 * s);
          const f32x4_t s1 = lds_ld<f32x4_t>(offS + slot * TS_S + 32 * s + 16);
          sc[0] = s0[0]; sc[1] = s0[1]; sc[2] = s0[2]; sc[3] = s0[3];
          sc[4] = s1[0]; sc[5] = s1[1]; sc[6] = s1[2]; sc[7] = s1[3];
        }
        uint4 av[NMH];
#pragma unroll
        for (int m = 0; m < NMH; ++m) {
          const u32x4_t a4 = lds_ld<u32x4_t>((s ? offA1 : offA0) + slot * TS_A + m * 2048);
          av[m] = scale_frag(make_uint4(a4.x, a4.y, a4.z, a4.w), sc);
          corr[m] = mfma32(c136, av[m], corr[m]);
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
          for (int m = 0; m < NMH; ++m) acc[m][nf] = mfma32(bu, av[m], acc[m][nf]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // 3-deep ring: step j computes from slot j % 3 while the loads of step
    // j + 2 (issued at the start of the step) are in flight; at the end of the
    // step every wave waits for all of its loads and the block syncs.  The
    // loop runs in groups of three steps; steps past the end compute nothing
    // (uniform branch) but still issue their loads, clamped to the last real
    // step.
    __syncthreads();  // LDS of the previous item is free
    stage(0, 0);
    stage(1, 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm);
    block_barrier();
    for (int j = 0; j < NK; j += 3) {
#define MOE_T_STEP(JJ, CUR, NXT)                 \
  {                                              \
    const int jj = (JJ);                         \
    stage(jj + 2, NXT);                          \
    if (jj < NK) compute(CUR);                   \
    __builtin_amdgcn_s_waitcnt(kWaitVm); \
    block_barrier();                             \
  }
      MOE_T_STEP(j, 0, 2)
      MOE_T_STEP(j + 1, 1, 0)
      MOE_T_STEP(j + 2, 2, 1)
#undef MOE_T_STEP
    }
    // drain the trailing (clamped) loads before the ring is reused
    __builtin_amdgcn_s_waitcnt(kWaitAll);

    // ---- epilogue indices, re-derived from an opaque copy of the thread
    // index: the lane's row in fragment m is rbase + 16 m; its output columns
    // are ocol + 16 nf .. + 3; col is the column of the A-of-the-matrix
    // operand lane lr feeds into the adapter product
    int tid2 = threadIdx.x;
    asm volatile("" : "+v"(tid2));
    const int lr2 = tid2 & 15, lg2 = (tid2 >> 4) & 3, wm2 = (tid2 >> 6) & 1, wn2 = tid2 >> 7;
    const int rbase = 16 * NMH * wm2 + lr2;
    const int ocol = c0 + 128 * wn2 + 4 * lg2, lcol = c0 + 128 * wn2 + lr2;

    // remove the 136 offset of the int4 operand (and apply the row's gate
    // when the rows are dy by token)
#pragma unroll
    for (int m = 0; m < NMH; ++m)
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) acc[m][nf] = (acc[m][nf] - corr[m]) * gm[m];

    // adapter term: acc += dZ L with L = A of the matrix ([r][N]), K = rank.
    const int nsrc = MODE == 1 ? 2 : 1;
    if constexpr (EPL) {
      // from the epilogue stages: dZ rows in the A array of ring slot NK % 3,
      // L^T rows in the word arrays of slots NK % 3 and (mode 1) NK % 3 + 1
      const int es = NK % 3;
      for (int src = 0; src < nsrc; ++src) {
        const int ls = src ? (es == 2 ? 0 : es + 1) : es;
        short4_t lv[8];
#pragma unroll
        for (int nf = 0; nf < 8; ++nf)
          lv[nf] = lds_ld<short4_t>(ldsB + ls * TS_B + (128 * wn2 + 16 * nf + lr2) * 32 + 8 * lg2);
#pragma unroll
        for (int m = 0; m < NMH; ++m) {
          const int r = rbase + 16 * m;
          const f32x4_t z = lds_ld<f32x4_t>(ldsA + es * TS_A + r * 128 + (((4 * src + lg2) ^ row_swz(r)) << 4));
          const short4_t av = __builtin_bit_cast(short4_t, u32x2_t{cvt_pk_bf16(z[0], z[1]), cvt_pk_bf16(z[2], z[3])});
#pragma unroll
          for (int nf = 0; nf < 8; ++nf) acc[m][nf] = mfma16(lv[nf], av, acc[m][nf]);
        }
      }
    } else {
      // Loads use clamped indices so that they issue together; rank positions
      // beyond r are zeroed on the L side.
      for (int src = 0; src < nsrc; ++src) {
        const float *Zp = src ? A.Z1 : A.Z0;
        const uint16_t *Lm = src ? A.L1 : A.L0;
        for (int j0 = 0; j0 < A.r; j0 += 16) {
          uint32_t kmask[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) kmask[i] = j0 + 4 * lg2 + i < A.r ? 0xFFFFu : 0u;
          short4_t lv[8];
#pragma unroll
          for (int nf = 0; nf < 8; ++nf) {
            const int c = min(lcol + 16 * nf, N - 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              lv[nf][i] = (short)(Lm[((size_t)e * A.r + min(j0 + 4 * lg2 + i, A.r - 1)) * N + c] &
                                  kmask[i]);
          }
#pragma unroll
          for (int m = 0; m < NMH; ++m) {
            const size_t p = (size_t)(p0 + min(rbase + 16 * m, rows - 1));
            short4_t av;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              av[i] = (short)f2bf(Zp[p * A.ldz + min(j0 + 4 * lg2 + i, A.r - 1)]);
#pragma unroll
            for (int nf = 0; nf < 8; ++nf) acc[m][nf] = mfma16(lv[nf], av, acc[m][nf]);
          }
        }
      }
    }

    // epilogue: 8-byte loads of G, U and 8-byte stores of the results
    const bool cols_ok = c0 + 128 * wn2 < N;   // N is a multiple of 128
#pragma unroll
    for (int m = 0; m < NMH; ++m) {
      const int r = rbase + 16 * m;
      if (!cols_ok || r >= rows) continue;
      const size_t p = (size_t)(p0 + r);
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) {
        const int c = ocol + 16 * nf;
        const f32x4_t a = acc[m][nf];
        if (MODE == 0) {
          const size_t o = p * N + c;
          const u32x2_t gw = *reinterpret_cast<const u32x2_t *>(&A.G[o]);
          const u32x2_t uw = *reinterpret_cast<const u32x2_t *>(&A.U[o]);
          const float gv[4] = {__uint_as_float(gw.x << 16), __uint_as_float(gw.x & 0xffff0000u),
                               __uint_as_float(gw.y << 16), __uint_as_float(gw.y & 0xffff0000u)};
          const float uv[4] = {__uint_as_float(uw.x << 16), __uint_as_float(uw.x & 0xffff0000u),
                               __uint_as_float(uw.y << 16), __uint_as_float(uw.y & 0xffff0000u)};
          float dg[4], du[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sgm = sigmoid_rcp(gv[i]);
            dg[i] = a[i] * uv[i] * sgm * (1.f + gv[i] * (1.f - sgm));
            du[i] = a[i] * gv[i] * sgm;
          }
          *reinterpret_cast<u32x2_t *>(&A.dG[o]) = u32x2_t{cvt_pk_bf16(dg[0], dg[1]), cvt_pk_bf16(dg[2], dg[3])};
          *reinterpret_cast<u32x2_t *>(&A.dU[o]) = u32x2_t{cvt_pk_bf16(du[0], du[1]), cvt_pk_bf16(du[2], du[3])};
        } else {
          *reinterpret_cast<u32x2_t *>(&A.out[p * A.ldo + c]) =
              u32x2_t{cvt_pk_bf16(a[0], a[1]), cvt_pk_bf16(a[2], a[3])};
        }
      }
    }
  }
}

int mfma_t_tile_rows() { return GT_BM; }
int mfma_t_tile_cols() { return GT_BN; }
int mfma_t_blocks_per_cu() { return GT_BPC; }

// The launch of tile class cls (0: 128 rows, 1: 96, 2: 64, 3: 32); cnt as
// written by launch_class_tiles.
void launch_grouped_gemm_t(int mode, const MfmaGemmTArgs &A, const int *cnt, int cls, int grid,
                           hipStream_t st) {
  const int *c = cnt + cls, *s = cnt + 4 + cls;
  // grid: GT_BPC blocks per CU; the 64- and 32-row classes run more
  if (cls >= 2) grid = (grid / GT_BPC * gt_bpc(cls == 2 ? 2 : 1)) & ~7;
  // operands of the epilogue through the LDS ring: rank 16, dZ rows 16-byte
  // aligned, transposed adapter A given
  const bool epl = A.r == 16 && (A.ldz & 3) == 0 && A.LT0 && (mode == 0 || A.LT1);
#define MOE_GT(MODE, NMH)                                                           \
  if (epl) grouped_gemm_t_kernel<MODE, NMH, true><<<grid, 256, 0, st>>>(A, c, s);   \
  else grouped_gemm_t_kernel<MODE, NMH, false><<<grid, 256, 0, st>>>(A, c, s)
  if (mode == 0) {
    if (cls == 0) MOE_GT(0, 4); else if (cls == 1) MOE_GT(0, 3); else if (cls == 2) MOE_GT(0, 2); else MOE_GT(0, 1);
  } else {
    if (cls == 0) MOE_GT(1, 4); else if (cls == 1) MOE_GT(1, 3); else if (cls == 2) MOE_GT(1, 2); else MOE_GT(1, 1);
  }
#undef MOE_GT
}

void launch_transpose_q(const uint8_t *q, const uint16_t *s, const int32_t *offsets, int E, int R,
                        int C, uint8_t *qt, float *st, hipStream_t stream) {
  dim3 grid((C + 255) / 256, R / 64, E);
  transpose_q_kernel<<<grid, 256, 0, stream>>>(q, s, offsets, R, C, qt, st);
}


}  // namespace moe
