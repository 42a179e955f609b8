// Input-gradient products of the adapter-only backward, on the matrix cores.
//
// Under TQP the base is frozen ("Reversible Sparse MoE Single Node" skill card,
// Principle 3), so the backward only needs the input gradients through each
// expert matrix, i.e. products with the base itself (the forward uses its
// transpose):
//   mode 0:  dH = dO W_d + dZ_d A_d, then the SwiGLU backward
//            dG = dH U s (1 + G (1 - s)), dU = dH G s, s = sigmoid(G)
//            (the two multipliers of dH come from the forward, which has
//            s at hand: the epilogue is two products per element)
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
// exactly as 136 + q (nibble in the mantissa of 128.0).  The scaled operand
// is itself formed on the matrix cores, as a product of a diagonal matrix of
// the scales with the fragment (exact in float32, then rounded once to bf16).
// The offset is taken out by one more MFMA per row fragment against a
// constant 136 operand, which accumulates 136 sum_n A'_g[p][n] from exactly
// the values the main products used.
//
// A pre-pass transposes the int4 nibbles so that each output column holds its
// reduction run as packed words (the same 8-per-word order as the forward
// operand), blocked by 64 reduction steps, and lays the scales out per column
// group.  The GEMM: 128 x 256 output tile per block, four waves as 2 x 2,
// 64 x 128 per wave (one column group per wave); A rows, int4 words and
// scales stream through a 3-deep LDS ring (LDS-DMA, A XOR-swizzled) in steps
// of 64; v_mfma_f32_16x16x32_bf16 into float32 accumulators; persistent
// XCD-partitioned work list; two blocks per CU, so that one block's VALU work
// (unpacking) overlaps the other's matrix work.
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

// An int8 base [E][R][C] (bytes in c order) + scales [E][R][C/128] as two
// int4 planes stacked along R, q = 16 h + l: rows 0 .. R-1 hold h = q >> 4
// with scales 16 s, rows R .. 2R-1 hold l - 8 (l = q & 15) with scales s,
// each in the transposed layout above ([E][2R/64][C][32 B], scales
// [E][C/128][2R] f32).  Summed with the matrix cores' 136 offset removed as
// 136 on the first plane and 128 on the second, the planes give s q exactly.
// One thread per output word (8 stacked rows of one column); consecutive
// threads take consecutive words of a column, then consecutive columns.
__global__ __launch_bounds__(256) void transpose_q_int8_kernel(const uint8_t *__restrict__ q,
                                                               const uint16_t *__restrict__ s,
                                                               const int32_t *__restrict__ offsets,
                                                               int R, int C, uint8_t *__restrict__ qt,
                                                               float *__restrict__ st) {
  const int e = blockIdx.z;
  if (offsets && offsets[e + 1] == offsets[e]) return;
  const int blk = blockIdx.y;                     // block of 64 stacked rows
  const int t = blockIdx.x * 256 + threadIdx.x;   // (column, word) of the block
  const int c = t >> 3, wd = t & 7;
  if (c >= C) return;
  const int n0 = blk * 64 + 8 * wd;               // first stacked row of the word
  const bool low = n0 >= R;
  const int r0 = low ? n0 - R : n0;
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = q[((size_t)e * R + r0 + i) * C + c];
    const uint32_t nib = low ? ((b & 15u) ^ 8u) : (b >> 4);
    w |= nib << (4 * nib_slot(i));
  }
  reinterpret_cast<uint32_t *>(qt)[(((size_t)e * (2 * R / 64) + blk) * C + c) * 8 + wd] = w;
  // the scales of the block's 64 rows for this column's group (one word's
  // thread per 8 rows writes them)
  if ((c & 127) == 0) {
    const int G = C / 128, g = c >> 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sv = bf2f(s[((size_t)e * R + r0 + i) * G + g]);
      st[((size_t)e * G + g) * 2 * R + n0 + i] = low ? sv : 16.f * sv;
    }
  }
}

// One pipeline stage in LDS, one array per kind (each read is a per-lane base
// register plus a compile-time offset): A rows (128 x 64 bf16, 16-byte chunks
// XOR-swizzled by row), int4 words (256 columns x 32 bytes), the scales of the
// stage's 64 reduction steps for the block's two column groups (wave w loads
// the 32 of group w / 2 from k = 32 (w % 2) into its own 256-byte region;
// its upper 32 lanes repeat the lower lanes' sources into the region's upper
// half, which nothing reads, so the transfer needs no lane mask).
constexpr int TS_B = GT_BN * GT_KS / 2, TS_S = 4 * 64 * 4;   // (the A stage holds the item's rows)

// Output columns of a wave's 128: fragment nf (of 8) and matrix-instruction
// row j hold column gt_col(nf, j) (8 adjacent columns per lane and fragment
// pair, 16-byte accesses in the epilogue); in LDS, column c of the item's 256
// (the int4 words of a stage, and the transposed adapter rows) sits at
// gt_pos(c), halves swapped by gt_half(c).

// ------------------------------------------------------------------ GEMM --
// A bf16x8 fragment (lane: row l % 16, 8 consecutive k of lane group l / 16)
// times its 8 per-k scales, rounded back to bf16, with the products formed on
// the matrix cores: two 16x16x16 products of a diagonal matrix of scales by
// the fragment's two 4-wide halves.  The diagonal operand d_t of lane
// (i, b) holds the scale of k = 16 (i / 4) + 8 s + 4 t + i % 4 at element
// i % 4 when b = i / 4 and zeros elsewhere, so output element u of lane
// (row, b) is that row's value at k = 16 b + 8 s + 4 t + u times its scale:
// the lane's own eight k in order.  A bf16 times a bf16 is exact in float32,
// and the other terms are zeros, so each product is exact and the
// conversion rounds it once, as a vector multiply would; a row holding an
// infinity or NaN turns its neighbours in the same 16 k into NaN (its
// products are non-finite either way).
DEV uint4 scale_frag_mfma(const u32x4_t a, short4_t d0, short4_t d1) {
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  const f32x4_t p0 = mfma16(d0, __builtin_bit_cast(short4_t, u32x2_t{a.x, a.y}), z);
  const f32x4_t p1 = mfma16(d1, __builtin_bit_cast(short4_t, u32x2_t{a.z, a.w}), z);
  return make_uint4(cvt_pk_bf16(p0[0], p0[1]), cvt_pk_bf16(p0[2], p0[3]), cvt_pk_bf16(p1[0], p1[1]),
                    cvt_pk_bf16(p1[2], p1[3]));
}

// Per-launch values every work item uses.
struct GtCtx {
  int Kh, N, G, NKh, NK, NKr;
  uint32_t ldsA, ldsB, ldsS;   // LDS byte addresses of the ring arrays
  uint32_t ldsD;               // 1 KB of LDS that transfers with nothing to load land in
  uint32_t kMask, kMagic;      // int4 unpack constants (held in registers)
};

// One work item: the rows p0 .. p0 + rows - 1 of expert e (rows <= 32 NMH)
// times the 256 output columns from c0.  NMH: row fragments of 16 per wave;
// the item runs as a tile of 32 NMH rows.  Waves 2 x 2: wave (wm, wn) takes
// rows 16 NMH wm .. + 16 NMH and the 128 columns of column group wn.
// Products are formed transposed (D^T = W^T A^T: the unpacked weights are the
// first MFMA operand) so a lane holds one row and four consecutive columns and
// the epilogue reads its multipliers and writes its results 8 bytes at a time.
template <int MODE, int NMH, bool EPL>
DEV void gt_item(const MfmaGemmTArgs &A, const GtCtx &X, int e, int p0, int rows, int c0) {
  // the ring (3 stages, filled by LDS-DMA issued from inline asm, with
  // explicit waits) holds the item's rows: its A stages are 32 NMH rows apart
  constexpr int TS_A = 32 * NMH * GT_KS * 2;   // A stage: the tile's rows x 64 K
  constexpr int AOPS = NMH;   // 8-row A loads per wave and stage
  const int Kh = X.Kh, N = X.N, G = X.G, NKh = X.NKh, NK = X.NK, NKr = X.NKr;
  const uint32_t ldsA = X.ldsA, ldsB = X.ldsB, ldsS = X.ldsS, kMask = X.kMask, kMagic = X.kMagic;
  const uint4 c136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};   // bf16 136
  const uint4 c128 = {0x43004300u, 0x43004300u, 0x43004300u, 0x43004300u};   // bf16 128
  {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // keep tid-only arithmetic inside the item
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int wm = w & 1, wn = w >> 1;

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
    // int4 staging: wave w, load i fills LDS positions 32 (2w + i) .. +31, 32
    // bytes each, lane L half L & 1 of position (L >> 1) (gt_pos, gt_half)
    uint32_t boff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = gt_pos(32 * (2 * w + i) + (lane >> 1));
      const int col = min(c0 + c, N - 1);
      boff[i] = (uint32_t)col * 32 + 16 * ((lane & 1) ^ gt_half(c));
    }
    // scale staging: wave w, lanes < 32: column group (w >> 1), k 32 (w & 1) + lane
    const int sg = min(c0 / 128 + (w >> 1), G - 1);
    const int sk = 32 * (w & 1) + (lane & 31);
    const uint32_t soff = (uint32_t)(sg * Kh + sk) * 4u;
    // this wave's LDS-DMA destinations within a stage (wave-uniform)
    const uint32_t wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t la = ldsA + wu * AOPS * 1024, lb = ldsB + wu * 2 * 1024,
                   ls = ldsS + wu * 256;
    // per-lane LDS read bases (bytes); the rest of every read address is a
    // compile-time constant
    // (fragment nf reads column 128 wn + gt_col(nf, lr): its LDS position is
    // that of fragment nf & 1 plus 32 (nf >> 1) columns)
    // (offD: the scale that lane lr places on the diagonal of the scaling
    // products, k = 16 (lr / 4) + (lr % 4) + a compile-time 8 s + 4 t, in the
    // region of the wave that loaded group wn's k / 32)
    const uint32_t offA0 = opaque(ldsA + (16 * NMH * wm + lr) * 128 + (((2 * lg) ^ row_swz(lr)) << 4)),
                   offB0 = opaque(ldsB + (128 * wn + gt_pos(gt_col(0, lr))) * 32 +
                                  16 * ((lg >> 1) ^ gt_half(gt_col(0, lr))) + 8 * (lg & 1)),
                   offB1 = opaque(ldsB + (128 * wn + gt_pos(gt_col(1, lr))) * 32 +
                                  16 * ((lg >> 1) ^ gt_half(gt_col(1, lr))) + 8 * (lg & 1)),
                   offD = opaque(ldsS + (2 * wn + (lr >> 3)) * 256 + (16 * ((lr >> 2) & 1) + (lr & 3)) * 4);
    // byte selectors that place the bf16 scale (the upper half of its float32
    // word) at element lr % 4 of the lane's 4-element diagonal operand, in
    // the lanes whose lane group is lr / 4, and zeros everywhere else
    // (selector byte 0x0c gives a zero byte)
    uint32_t selLo, selHi;
    {
      const bool on = (lr >> 2) == lg;
      const uint32_t put = (lr & 1) ? 0x03020c0cu : 0x0c0c0302u;
      selLo = on && (lr & 2) == 0 ? put : 0x0c0c0c0cu;
      selHi = on && (lr & 2) != 0 ? put : 0x0c0c0c0cu;
      selLo = opaque(selLo);
      selHi = opaque(selHi);
    }

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
      // the adapter A of the matrix as stored ([E][16][N]): rank row j of
      // the item's 256 columns at j * 512 bytes (wave w, load i: rows
      // 2 (2 w + i) and + 1, 8 columns a lane; a partial tile repeats its
      // last 8 columns)
      const char *lb16 = reinterpret_cast<const char *>(uniform_ptr((part ? A.L1 : A.L0) + (size_t)e * 16 * N));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int j = 2 * (2 * w + i) + (lane >> 5);
        const int col = min(c0 + 8 * (lane & 31), N - 8);
        dma16(lb16, ((uint32_t)j * (uint32_t)N + (uint32_t)col) * 2u, sb + slot * TS_B + i * 1024);
      }
    };
    // The epilogue stages (EPL) are issued whole at the start of their step.
    auto stage = [&](int jr, int slot) {
      if (EPL && jr >= NK) {
        if (jr == NK) stage_ep(0, slot);
        else if (MODE == 1 && jr == NK + 1) stage_ep(1, slot);
      }
    };
    // A reduction stage j (< NK) is NOPS single transfers (the A rows, the
    // int4 words, the scales), which the step computing the stage two before
    // it issues one at a time between its matrix instructions, so that a
    // wave never stalls on a full load queue with its matrix work waiting.
    constexpr int NOPS = AOPS + 3;
    static_assert(NOPS <= 8, "one transfer per column fragment of a substep");
    struct StageSrc {
      const char *a;
      const uint8_t *q;
      const float *s;
    };
    auto stage_src = [&](int j) {
      const bool second = MODE == 1 && j >= NKh;
      const int kj = second ? j - NKh : j;
      const int ka = kj < NKr ? kj : kj - NKr;   // (an int8 base's second plane: the rows again)
      StageSrc r;
      r.a = reinterpret_cast<const char *>(second ? A.a1 : A.a0) + (size_t)ka * GT_KS * 2;
      r.q = (second ? A.qt1 : A.qt0) + ((size_t)e * NKh + kj) * N * 32;
      r.s = (second ? A.st1 : A.st0) + (size_t)e * G * Kh + kj * GT_KS;
      return r;
    };
    // (live = false: the transfer lands in the unread LDS area instead)
    auto stage_op = [&](int op, const StageSrc &src, int slot, bool live = true) {
      // destinations re-derived per transfer (scalar adds) rather than held
      uint32_t sa = la, sb = lb, ss = ls;
      asm volatile("" : "+s"(sa), "+s"(sb), "+s"(ss));
      if (op < AOPS) dma16(src.a, aoff[op], live ? sa + slot * TS_A + op * 1024 : X.ldsD);
      else if (op < AOPS + 2)
        dma16(src.q, boff[op - AOPS], live ? sb + slot * TS_B + (op - AOPS) * 1024 : X.ldsD);
      else dma4(src.s, soff, live ? ss + slot * TS_S : X.ldsD);
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
    // (a step with no stage left to load issues its transfers anyway, from
    // the last stage into the LDS area nothing reads: the step stays one
    // branch-free block that the compiler schedules as a whole)
    auto compute = [&](int slot, int jc, int jl, int nslot) {   // jc: this stage; jl: the stage to load into nslot
      __builtin_amdgcn_sched_barrier(0);
      // the offset the correction removes: 136, or 128 on an int8 base's second plane
      const int kc = MODE == 1 && jc >= NKh ? jc - NKh : jc;
      const uint4 coff = kc < NKr ? c136 : c128;
      const bool ld = jl < NK;
      const StageSrc src = stage_src(ld ? jl : NK - 1);
      u32x2_t bw[8];
#pragma unroll
      for (int nf = 0; nf < 8; ++nf)
        bw[nf] = lds_ld<u32x2_t>((nf & 1 ? offB1 : offB0) + slot * TS_B + (nf >> 1) * 32 * 32);
      // substep 1 reads chunk 2 lg + 1, the neighbouring swizzled chunk
      const uint32_t offA1 = offA0 ^ 16u;
      // the scaling products' diagonal operands, dg[s][t] for k = 16 b + 8 s
      // + 4 t + (0 .. 3) in lane group b
      short4_t dg[2][2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t f = lds_ld<uint32_t>(offD + slot * TS_S + (8 * s + 4 * t) * 4);
          dg[s][t] = __builtin_bit_cast(short4_t, u32x2_t{__builtin_amdgcn_perm(f, f, selLo),
                                                          __builtin_amdgcn_perm(f, f, selHi)});
        }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        uint4 av[NMH];
#pragma unroll
        for (int m = 0; m < NMH; ++m) {
          const u32x4_t a4 = lds_ld<u32x4_t>((s ? offA1 : offA0) + slot * TS_A + m * 2048);
          av[m] = scale_frag_mfma(a4, dg[s][0], dg[s][1]);
          corr[m] = mfma32(coff, av[m], corr[m]);
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
          if (s == 0 && nf < NOPS) stage_op(nf, src, nslot, ld);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // 3-deep ring: step j computes from slot j % 3 and, between its matrix
    // instructions, issues the loads of stage j + 2 into slot (j + 2) % 3; at
    // the end of the step every wave waits for all of its loads and the block
    // syncs.  The loop runs in groups of three steps; steps past the end
    // compute nothing and load nothing (uniform branches).
    __syncthreads();  // LDS of the previous item is free
    {
      const StageSrc s0 = stage_src(0), s1 = stage_src(min(1, NK - 1));
#pragma unroll
      for (int op = 0; op < NOPS; ++op) stage_op(op, s0, 0);
      if (NK > 1) {
#pragma unroll
        for (int op = 0; op < NOPS; ++op) stage_op(op, s1, 1);
      } else {
        stage(1, 1);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm);
    block_barrier();
    for (int j = 0; j < NK; j += 3) {
#define MOE_T_STEP(JJ, CUR, NXT)                                    \
  {                                                                 \
    const int jj = (JJ), jl = jj + 2;                               \
    stage(jl, NXT);                                                 \
    if (jj < NK) compute(CUR, jj, jl, NXT);                         \
    __builtin_amdgcn_s_waitcnt(kWaitVm);                            \
    block_barrier();                                                \
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
    // in fragments 2t and 2t + 1 are ocol + 32 t .. + 7 (gt_col); the
    // A-of-the-matrix operand lane lr feeds into the adapter product of
    // fragment nf is column wcol + gt_col(nf, lr)
    int tid2 = threadIdx.x;
    asm volatile("" : "+v"(tid2));
    const int lr2 = tid2 & 15, lg2 = (tid2 >> 4) & 3, wm2 = (tid2 >> 6) & 1, wn2 = tid2 >> 7;
    const int rbase = 16 * NMH * wm2 + lr2;
    const int wcol = c0 + 128 * wn2, ocol = wcol + 8 * lg2;

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
      // the rank rows of L in the word arrays of slots NK % 3 and (mode 1)
      // NK % 3 + 1 (rank values 4 lg .. 4 lg + 3 of a column: four 16-bit
      // reads 512 bytes apart)
      const int es = NK % 3;
      for (int src = 0; src < nsrc; ++src) {
        const int ls = src ? (es == 2 ? 0 : es + 1) : es;
        short4_t lv[8];
#pragma unroll
        for (int nf = 0; nf < 8; ++nf) {
          const uint32_t la16 = ldsB + ls * TS_B + (128 * wn2 + gt_col(nf, lr2)) * 2 + 4 * lg2 * 512;
#pragma unroll
          for (int i = 0; i < 4; ++i) lv[nf][i] = lds_ld<short>(la16 + i * 512);
        }
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
            const int c = min(wcol + gt_col(nf, lr2), N - 1);
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

    // epilogue: per pair of fragments (2t, 2t + 1) a lane holds 8 adjacent
    // columns of its row: 16-byte loads of G, U (and H) and 16-byte stores
    const bool cols_ok = c0 + 128 * wn2 < N;   // N is a multiple of 128
    // mode 0 with dgp: the row's dot of dH and H over the wave's 128 columns
    const bool want_dg = MODE == 0 && A.dgp != nullptr;
    auto lo = [](uint32_t v) { return __uint_as_float(v << 16); };
    auto hi = [](uint32_t v) { return __uint_as_float(v & 0xffff0000u); };
#pragma unroll
    for (int m = 0; m < NMH; ++m) {
      const int r = rbase + 16 * m;
      float hdot = 0.f;
      if (cols_ok && r < rows) {
        const size_t p = (size_t)(p0 + r);
        // mode 0: every operand of the row fragment is loaded before any of
        // its stores (a load written after a store would wait for it: the
        // compiler cannot tell that they do not overlap), one round trip
        // per fragment
        uint4 gw[4], uw[4], hw[4];
        if (MODE == 0) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const size_t o = p * N + ocol + 32 * t;
            gw[t] = *reinterpret_cast<const uint4 *>(&A.G[o]);
            uw[t] = *reinterpret_cast<const uint4 *>(&A.U[o]);
            if (want_dg) hw[t] = *reinterpret_cast<const uint4 *>(&A.H[o]);
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4_t a0 = acc[m][2 * t], a1 = acc[m][2 * t + 1];
          const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          const int c = ocol + 32 * t;
          if (MODE == 0) {
            // the forward saved the SwiGLU backward's multipliers
            // mG = U s (1 + G (1 - s)) and mU = G s
            const size_t o = p * N + c;
            const uint32_t g4[4] = {gw[t].x, gw[t].y, gw[t].z, gw[t].w},
                           u4[4] = {uw[t].x, uw[t].y, uw[t].z, uw[t].w};
            uint32_t dg[4], du[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              dg[i] = cvt_pk_bf16(a[2 * i] * lo(g4[i]), a[2 * i + 1] * hi(g4[i]));
              du[i] = cvt_pk_bf16(a[2 * i] * lo(u4[i]), a[2 * i + 1] * hi(u4[i]));
            }
            *reinterpret_cast<uint4 *>(&A.dG[o]) = make_uint4(dg[0], dg[1], dg[2], dg[3]);
            *reinterpret_cast<uint4 *>(&A.dU[o]) = make_uint4(du[0], du[1], du[2], du[3]);
            if (want_dg) {
              const uint32_t h4[4] = {hw[t].x, hw[t].y, hw[t].z, hw[t].w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                hdot = fmaf(a[2 * i], lo(h4[i]), hdot);
                hdot = fmaf(a[2 * i + 1], hi(h4[i]), hdot);
              }
            }
          } else {
            *reinterpret_cast<uint4 *>(&A.out[p * A.ldo + c]) =
                make_uint4(cvt_pk_bf16(a[0], a[1]), cvt_pk_bf16(a[2], a[3]),
                           cvt_pk_bf16(a[4], a[5]), cvt_pk_bf16(a[6], a[7]));
          }
        }
      }
      if (want_dg) {
        // the four lanes of the row (lane groups), in a fixed order
        hdot += __shfl_xor(hdot, 16);
        hdot += __shfl_xor(hdot, 32);
        if (lg2 == 0 && r < rows)
          A.dgp[(size_t)(2 * (c0 / 256) + wn2) * A.S + p0 + r] = hdot;
      }
    }
  }
}

// All items of the product in one launch: the tiles of launch_build_tiles
// (each expert's rows in tiles of 128, in expert order) times the column
// tiles, in that order, as a persistent work list split into eight
// contiguous ranges, one per XCD, so that the tiles of one expert, including
// its short last one, run close together in time on one XCD and share its
// weights in that L2.  Within its range a block takes the next item from a
// counter of the XCD (ctr[xcd], zero at launch), so blocks that drew short
// items take more of them, and once its range is used up from the other
// XCDs' ranges (draw_item).  Each item runs as the shortest tile class that
// holds its rows (32, 64, 96 or 128; a wave-uniform branch).  Two blocks per
// CU, so that one block's VALU work (unpacking) overlaps the other's
// matrix work.
template <int MODE, bool EPL>
__global__ __launch_bounds__(256, GT_BPC) void grouped_gemm_t_kernel(const MfmaGemmTArgs A,
                                                                     const int *__restrict__ ntiles,
                                                                     int *__restrict__ ctr) {
  // (ringA 32-byte aligned: the second substep's chunk is the first's
  // address with bit 4 flipped)
  __shared__ __attribute__((aligned(32))) uint4 ringA[3][GT_BM * GT_KS * 2 / 16];
  __shared__ uint4 ringB[3][TS_B / 16];
  __shared__ float ringS[3][TS_S / 4];
  __shared__ uint4 ringD[64];
  GtCtx X;
  X.Kh = A.K;
  X.N = A.N;
  X.G = A.N / 128;
  X.NKh = A.K / GT_KS;
  X.NK = MODE == 1 ? 2 * X.NKh : X.NKh;   // mode 1 reduces over [dG | dU]
  X.NKr = A.kr / GT_KS;   // steps of the A rows per source (NKh, or NKh / 2 for int8)
  X.ldsA = lds_addr(ringA);
  X.ldsB = lds_addr(ringB);
  X.ldsS = lds_addr(ringS);
  X.ldsD = __builtin_amdgcn_readfirstlane(lds_addr(ringD));
  // int4 unpack: each bf16 pair of 136 + q is one shift and one three-input
  // logic op, ((w >> 4i) & 0x000F000F) ^ 0x43084308 (constants in registers)
  X.kMask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  asm volatile("v_mov_b32 %0, 0x43084308" : "=v"(X.kMagic));
  __shared__ int next_item;
  const int total = ntiles[0] * A.NT;
  const int xcd = blockIdx.x & 7;
  int rng = xcd;
  if (threadIdx.x == 0) next_item = draw_item(ctr, total, rng, xcd);
  __syncthreads();
  for (int wi = next_item; wi >= 0; wi = next_item) {
    // every thread has read next_item; the next draw overlaps this item (its
    // value is visible after the item's first barrier)
    __syncthreads();
    if (threadIdx.x == 0) next_item = draw_item(ctr, total, rng, xcd);
    const int ti = wi / A.NT, nt = wi - ti * A.NT;
    const int2 tile = A.tiles[ti];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(GT_BM, A.offsets[e + 1] - p0);
    const int c0 = nt * GT_BN;
    const int nmh = __builtin_amdgcn_readfirstlane((rows + 31) >> 5);
    if (nmh >= 4) gt_item<MODE, 4, EPL>(A, X, e, p0, rows, c0);
    else if (nmh == 3) gt_item<MODE, 3, EPL>(A, X, e, p0, rows, c0);
    else if (nmh == 2) gt_item<MODE, 2, EPL>(A, X, e, p0, rows, c0);
    else gt_item<MODE, 1, EPL>(A, X, e, p0, rows, c0);
  }
}

int mfma_t_tile_rows() { return GT_BM; }
int mfma_t_tile_cols() { return GT_BN; }
int mfma_t_blocks_per_cu() { return GT_BPC; }

// One launch over the tile list of launch_build_tiles (tiles of 128 rows);
// ctr: eight zeroed counters.
void launch_grouped_gemm_t(int mode, const MfmaGemmTArgs &A, const int *ntiles, int *ctr, int grid,
                           hipStream_t st) {
  // operands of the epilogue through the LDS ring: rank 16, dZ rows 16-byte
  // aligned, transposed adapter A given
  // (the epilogue stages load A's rank rows in 16-byte pieces)
  const bool epl = A.r == 16 && (A.ldz & 3) == 0 &&
                   (((uintptr_t)A.L0 | (uintptr_t)(mode == 1 ? A.L1 : A.L0)) & 15) == 0;
#define MOE_GT(MODE)                                                           \
  if (epl) grouped_gemm_t_kernel<MODE, true><<<grid, 256, 0, st>>>(A, ntiles, ctr);   \
  else grouped_gemm_t_kernel<MODE, false><<<grid, 256, 0, st>>>(A, ntiles, ctr)
  if (mode == 0) {
    MOE_GT(0);
  } else {
    MOE_GT(1);
  }
#undef MOE_GT
}

void launch_transpose_q(const uint8_t *q, const uint16_t *s, const int32_t *offsets, int E, int R,
                        int C, uint8_t *qt, float *st, hipStream_t stream) {
  dim3 grid((C + 255) / 256, R / 64, E);
  transpose_q_kernel<<<grid, 256, 0, stream>>>(q, s, offsets, R, C, qt, st);
}

void launch_transpose_q_int8(const uint8_t *q, const uint16_t *s, const int32_t *offsets, int E,
                             int R, int C, uint8_t *qt, float *st, hipStream_t stream) {
  dim3 grid((C * 8 + 255) / 256, 2 * R / 64, E);
  transpose_q_int8_kernel<<<grid, 256, 0, stream>>>(q, s, offsets, R, C, qt, st);
}


}  // namespace moe
