// Grouped int4 x bf16 expert GEMMs on the CDNA4 matrix cores (gfx950).
//
// TQP keeps each expert's base matrix quantized and frozen and adds a trained
// low-rank adapter ("Reversible Sparse MoE Single Node" skill card,
// Principle 3 and Implementation Considerations "TQP Quantization"; LoRA under
// Related Methods).  Per expert segment of the expert-contiguous rows:
//   gate/up:  G = X W_g^T + lam (X A_g^T) B_g^T, U likewise, H = silu(G) * U
//   down:     O = H W_d^T + lam (H A_d^T) B_d^T
// The SwiGLU form is this library's reading; the pages do not name the FFN.
//
// Design (one 256-thread block = 4 waves, 128 rows x 256 columns per item):
//  * Work items (M-tile, N-tile) are processed by a persistent grid.  Each of
//    the 8 XCDs takes a contiguous eighth of the item list, so the rows and
//    weights of neighbouring tiles stay in that XCD's L2.
//  * K streams through a 2-slot LDS ring in half-group stages (64 of K): the
//    A rows (x gathered by token, or H), the int4 words of the block's 256
//    columns and, per group, the per-row start values and per-column scale
//    ratios, all by LDS-DMA (global_load_lds_*).  The stage after the last
//    one brings the epilogue's operands the same way (adapter projections
//    Z, adapter B rows, last scales), so the epilogue reads only LDS.
//  * Each wave owns 64 output columns for all 128 rows, so every unpacked
//    weight fragment feeds eight matrix instructions.  A nibble u (offset by
//    8) becomes the bf16 bit pattern 0x4300 | u, the exact value 136 + q; the
//    weights enter the matrix cores exactly (no rounding of s*q).
//  * Group scales without a second accumulator: with s_g the scale of group
//    g of a column, the accumulator holds Q_g = (sum over groups g' <= g of
//    s_g' P_g') / s_g, advanced per group as Q <- Q * (s_{g-1} / s_g) + P_g.
//    The ratios are precomputed per call (scale_ratio_kernel), and the final
//    multiplication by the last scale happens in the epilogue.  P_g itself
//    starts at -136 * (the row's sum over the group), which removes the 136
//    offset; the per-row start values are precomputed too.
//  * MFMA v_mfma_f32_16x16x32_bf16 with the weights as the first operand
//    (D^T = W X^T): a lane's accumulator holds one row and four consecutive
//    columns, so the epilogue writes 8-byte packed bf16 stores.
//  * Within a stage the LDS reads of the A fragments run a few fragments
//    ahead of the matrix instructions and the VALU work (unpacking, group
//    update) sits between them, pinned by scheduling-group barriers.
//  * Epilogue: the adapter term (lam Z) B^T is one more MFMA (K = rank) into
//    the same accumulator; gate/up applies SwiGLU in registers (a lane holds
//    the matching gate and up columns), writes H (bf16) and, for the down
//    product, the start values -136 * (row sum of H) per group.
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "prep.h"
#include "mfma.h"

namespace moe {

constexpr int GM_BM = 128;   // rows per tile
constexpr int GM_BPC = 2;    // resident blocks per CU
constexpr int GM_KG = 128;   // quantization group
constexpr int GM_KS = 64;    // K per pipeline stage (half a group)

// One pipeline stage in LDS, one array per kind (each read is a per-lane base
// register plus a compile-time offset below 64 KB): A rows (128 x 64 bf16,
// 16-byte chunks XOR-swizzled by row_swz), int4 words (32 bytes per block
// column), and the group data: the scale ratio per block column (256
// floats), the per-row start values (128 floats) and a copy of those (128
// floats, so that every wave issues the same number of loads).
constexpr int ST_B = 256 * GM_KS / 2, ST_X = 512 * 4;   // (the A stage holds the class's rows)

// ---------------------------------------------------------------- row sums --
// out[row][g] = scale * (sum of a[row][g*G .. g*G+G), bf16 values, float32 sum
// in k order); with split the row of out has 2 K/G entries and
// out[row][K/G + g] = scale2 * the same sum
__global__ void group_rowsum_kernel(const bf16_t *__restrict__ a, int rows, int K, int G,
                                    float scale, float *__restrict__ out, bool split,
                                    float scale2) {
  group_rowsum_elem((size_t)blockIdx.x * blockDim.x + threadIdx.x, a, rows, K, G, scale, out,
                    split, scale2);
}

// ------------------------------------------------------------ scale ratios --
// Per column c of a quantized matrix [E][N] with ng groups, group-major:
// rt[e][g][c] = s'[g-1] / s'[g] for g >= 1 and rt[e][0][c] = s'[ng-1] (the
// final multiplier).  s' is the bf16 scale s with every magnitude below the
// column's floor m 2^-24 (m = the column's largest |s|, and the floor at
// least 2^-100) raised to that floor.  So no ratio exceeds 2^24 and the
// telescoped accumulator stays within 2^24 times the sum of the partial
// products, far from the float32 range, however zero or widely spread the
// scales are; a raised group contributes at most floor * |its partial sum|
// instead of s times it, i.e. an error of one float32 rounding of the
// column's largest group.  One thread per column: its ng scales are one
// contiguous run, and each group's writes are contiguous across the wave.
// With split the column's scale sequence is that of the two int4 planes of
// an int8 base, 16 s[0 .. ng) then s[0 .. ng) (2 ng groups; 16 s is exact).
__global__ __launch_bounds__(256) void scale_ratio_kernel(const uint16_t *__restrict__ s, int E,
                                                          int N, int ng, float *__restrict__ rt,
                                                          bool split) {
  const int e = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c >= N) return;
  const uint16_t *sc = s + ((size_t)e * N + c) * ng;
  const int ngo = split ? 2 * ng : ng;
  auto sv = [&](int g) { return g < ng ? (split ? 16.f : 1.f) * bf2f(sc[g]) : bf2f(sc[g - ng]); };
  float m = 0.f;
  for (int g = 0; g < ngo; ++g) m = fmaxf(m, fabsf(sv(g)));
  const float floor_v = fmaxf(m * 0x1p-24f, 0x1p-100f);
  auto guard = [&](float v) { return fabsf(v) < floor_v ? floor_v : v; };
  float *out = rt + (size_t)e * ngo * N + c;
  float prev = guard(sv(0));
  for (int g = 1; g < ngo; ++g) {
    const float cur = guard(sv(g));
    out[(size_t)g * N] = prev / cur;
    prev = cur;
  }
  out[0] = prev;   // the last scale
}

// ------------------------------------------------------- stage schedule --
// Scheduling groups of one forward pipeline stage (see compute() in
// grouped_gemm_kernel): DS reads (mask 0x100), VALU (0x2), matrix
// instructions (0x8), in the order the stage is written.
template <int NM, int NF, bool EVEN, int PD, int I>
DEV void fwd_frag_sched() {
  constexpr int sub = I / NM, m = I % NM;
  if constexpr (I + PD < 2 * NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, NF, 0);
  constexpr int nvalu = ((EVEN && sub == 0 && m + 1 < NM) ? 4 * NF : 0) + (I == NM / 2 ? 7 * NF : 0);
  if constexpr (nvalu > 0) __builtin_amdgcn_sched_group_barrier(0x002, nvalu, 0);
}
template <int NM, int NF, bool EVEN, int PD, int... I>
DEV void fwd_stage_sched(std::integer_sequence<int, I...>) {
  // prologue: B words (+ ratios and start values), the first PD A reads;
  // unpacking of substep 0 (+ the update of row fragment 0)
  __builtin_amdgcn_sched_group_barrier(0x100, NF + (EVEN ? NF + (NM > 4 ? 2 : 1) : 0) + PD, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 7 * NF + (EVEN ? 4 * NF : 0), 0);
  (fwd_frag_sched<NM, NF, EVEN, PD, I>(), ...);
}

// ------------------------------------------------------------ grouped GEMM --
// MODE 0: gate/up with SwiGLU epilogue (A = x rows gathered by token); a work
//         item covers up to 128 rows x 128 columns of both gate and up.
// MODE 1: down (A = H rows in permuted order); up to 128 rows x 256 columns.
// WAVES (4) waves per block, each with all rows of the item and NF column
// fragments of 16 (mode 0: half gate, half up, so SwiGLU pairs up in a lane),
// so each unpacked weight fragment feeds NM matrix instructions.  NM (2, 4,
// 6, 8) is the number of 16-row fragments of the item: a tile runs as the
// shortest class that holds its rows, so a short tail tile costs only its
// rows.  Two resident blocks per CU (the 16-row kernel of short batches:
// short_bpc).
constexpr int gm_bpc(int NM) { return NM <= 2 ? 4 : GM_BPC; }
// resident blocks per CU of the short-batch kernel (16-row items)
constexpr int short_bpc(int MODE) { return MODE == 0 ? 5 : 4; }

// Per-launch values every work item uses.
struct GmCtx {
  uint32_t ldsA, ldsB, ldsX;   // LDS byte addresses of the ring arrays
  uint32_t kMask, kMagic;      // int4 unpack constants (held in registers)
  int *tok;                    // [GM_BM] LDS: the A row of each tile row
  float *red;                  // [WAVES][GM_BM] LDS (inside the A ring): row sums
};

// One work item: rows p0 .. p0 + rows - 1 of expert e (rows <= 16 NM) times
// column tile nt.  QP: the base in the stage-major packed layout
// (launch_pack_fwd, A.qp0 / A.qp1), else the storage layout (A.q0 / A.q1).
template <int MODE, int WAVES, int NM, bool EPL, bool QP>
DEV void gm_item(const MfmaGemmArgs &A, const GmCtx &X, int e, int p0, int rows, int nt) {
  constexpr int NF = 16 / WAVES;                 // column fragments per wave
  constexpr int BOPS = 8 / WAVES;                // int4-word loads per wave and stage
  constexpr int NT_ = 64 * WAVES;                // threads
  constexpr int WCOLS = (MODE == 0 ? 128 : 256) / WAVES;   // block column slots per wave (per matrix in mode 0)
  constexpr int AOPS = (2 * NM + WAVES - 1) / WAVES;       // 8-row A loads per wave and stage
  constexpr int XOPS = 8 / WAVES;                // group-data loads per wave (even stages)
  // Block column slots (mode 0: gate 0..127, then up 128..255; mode 1:
  // 0..255).  Matrix-instruction row j of fragment nf is slot w WCOLS +
  // fpair(nf) + gt_col(nf & 1, j): fragments 0-1 (mode 0: gate) and 2-3 (up)
  // are pairs whose lanes hold 8 adjacent columns each.
  static_assert(NF == 4, "the column permutation pairs fragments 0-1 and 2-3");
  constexpr auto fpair = [](int nf) { return MODE == 0 ? (nf >> 1) * 128 : (nf >> 1) * 32; };
  // a 2-slot ring of half-group stages, its A stages 16 NM rows apart; after
  // the K loop the first 2 KB of the A ring hold the cross-wave row sums of H.
  constexpr int ST_A = 16 * NM * GM_KS * 2;     // A stage: the tile's rows x 64 K
  static_assert(2 * ST_A >= WAVES * GM_BM * 4, "the row-sum exchange lives in the A ring");
  const int K = A.K, N = A.N, NG = K / GM_KG, NS = 2 * NG;   // NS: half-group stages
  const int NSA = A.ka / GM_KS;   // stages of the A rows (NS, or NS / 2 for an int8 base)
  const int BNO = MODE == 0 ? 128 : 256;   // output columns per item (per matrix)
  const uint32_t kMask = X.kMask, kMagic = X.kMagic;
  const uint32_t ldsA = X.ldsA, ldsB = X.ldsB, ldsX = X.ldsX;
  int *tok_lds = X.tok;
  {
    // thread indices are re-derived per item through an opaque copy so that
    // the compiler does not keep tid-only address arithmetic live across the
    // whole persistent loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int c0 = nt * BNO;
    __syncthreads();  // LDS of the previous item is free
    for (int t = tid; t < GM_BM; t += NT_) {
      const int p = p0 + min(t, rows - 1);
      tok_lds[t] = MODE == 0 ? A.perm_src[p] / A.kk : p;
    }
    __syncthreads();

    // ---- LDS-DMA sources.  A: 8 rows x 8 chunks of 16 B per wave load; wave
    // w, load i covers rows 8 (AOPS w + i) .. +7 (rows past the tile repeat
    // its last row); chunk c of row r lives at c ^ row_swz(r).
    uint32_t src_off[AOPS];
#pragma unroll
    for (int i = 0; i < AOPS; ++i) {
      const int r = min(8 * (AOPS * w + i) + (lane >> 3), GM_BM - 1);
      const int c = (lane & 7) ^ row_swz(r);
      src_off[i] = (uint32_t)tok_lds[r] * (uint32_t)(A.lda * 2) + c * 16;
    }
    const char *abase = reinterpret_cast<const char *>(A.a);
    // int4 words: 8 loads of 32 block columns x 32 B; wave w takes loads
    // BOPS w .. BOPS w + BOPS - 1 (each all gate or all up)
    // (all of a wave's word loads are of one matrix: gate for waves 0-1,
    // up for waves 2-3 in mode 0)
    const uint8_t *q0 = QP ? A.qp0 : A.q0, *q1 = QP ? A.qp1 : A.q1;
    const uint8_t *qbase =
        (const uint8_t *)uniform_ptr((MODE == 0 && w >= 2 ? q1 : q0) + (size_t)e * N * (K / 2));
    uint32_t qoff[BOPS];
#pragma unroll
    for (int i = 0; i < BOPS; ++i) {
      // lane L fills half L & 1 of LDS position 32 (BOPS w + i) + L / 2,
      // which holds block column slot gt_pos of it (halves by gt_half)
      const int bc = gt_pos(32 * (BOPS * w + i) + (lane >> 1));
      const int c = min(c0 + (MODE == 0 ? (bc & 127) : bc), N - 1);
      // (packed base: column c of a stage at 32 c; plain: at c K/2)
      qoff[i] = (uint32_t)c * (QP ? 32u : (uint32_t)(K / 2)) + 16 * ((lane & 1) ^ gt_half(bc));
    }
    // group data, 8 loads of 64 floats: loads 0-3 the ratios of block
    // columns 64 q + lane (group g at + g N), loads 4-5 the start values of
    // the 128 rows (group g at + g), row 16 m + l at position 8 l + m (a
    // lane's values are adjacent), loads 6-7 the same start values again
    // (into the spare quarter); wave w takes loads XOPS w .. XOPS w + XOPS - 1
    // (a wave's group-data loads share one base: waves 0-1 the ratios of
    // gate (mode 1: all) columns, wave 1 in mode 0 those of up, waves 2-3 the
    // start values)
    const bool xr = w < 2;   // this wave loads ratios
    const float *xbase = (const float *)uniform_ptr(
        xr ? ((MODE == 0 && w == 1 ? A.rt1 : A.rt0) + (size_t)e * NG * N) : A.rsum);
    const int xstr = __builtin_amdgcn_readfirstlane(xr ? N : 1);
    uint32_t xoff[XOPS];
#pragma unroll
    for (int i = 0; i < XOPS; ++i) {
      const int q = XOPS * w + i;
      if (q < 4) {
        const int bc = 64 * q + lane;
        const int c = min(c0 + (MODE == 0 ? (bc & 127) : bc), N - 1);
        xoff[i] = (uint32_t)c * 4u;
      } else {
        const int pos = 64 * (q & 1) + lane;
        xoff[i] = (uint32_t)tok_lds[16 * (pos & 7) + (pos >> 3)] * (uint32_t)A.ld_rsum * 4u;
      }
    }
    const uint32_t wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t la = ldsA + wu * AOPS * 1024, lb = ldsB + wu * BOPS * 1024,
                   lx = ldsX + wu * XOPS * 256;
    // per-lane LDS read bases (bytes); the rest of every read address is a
    // compile-time constant.  The int4 word lane lr feeds into the first MFMA
    // operand of fragment nf is block column slot w WCOLS + fpair(nf) +
    // gt_col(nf & 1, lr) (offB0 / offB1 by the parity of nf); the lane's
    // accumulator holds the four output columns from slot w WCOLS + fpair(nf)
    // + 8 lg + 4 (nf & 1).
    const int bcol0 = gt_col(0, lr), bcol1 = gt_col(1, lr);
    const uint32_t offA0 = opaque(ldsA + lr * 128 + (((2 * lg) ^ row_swz(lr)) << 4)),
                   offB0 = opaque(ldsB + (w * WCOLS + gt_pos(bcol0)) * 32 +
                                  16 * ((lg >> 1) ^ gt_half(bcol0)) + 8 * (lg & 1)),
                   offB1 = opaque(ldsB + (w * WCOLS + gt_pos(bcol1)) * 32 +
                                  16 * ((lg >> 1) ^ gt_half(bcol1)) + 8 * (lg & 1)),
                   offR = opaque(ldsX + (w * WCOLS + 8 * lg) * 4),
                   offC = opaque(ldsX + 1024 + lr * 32);

    // The epilogue's operands go through the ring too, as the stage after
    // the last one (rank 16): the adapter projections Z of the item's rows
    // in the A array (row r: Z_g then Z_u, or Z_d; 64 floats at most, with
    // the A swizzle), the adapter B rows of its block columns in the word
    // array (32 bytes each), and group 0's ratios, i.e. the last scales, in
    // the group-data array.
    // (EPL: rank 16 and Z rows 16-byte aligned, checked by the launcher)
    constexpr bool ep_lds = EPL;
    auto stage_ep = [&](int slot) {
      uint32_t sa = la, sb = lb, sx = lx;
      asm volatile("" : "+s"(sa), "+s"(sb), "+s"(sx));
      const char *zb = reinterpret_cast<const char *>(uniform_ptr(A.Z0));
#pragma unroll
      for (int i = 0; i < AOPS; ++i) {
        if (AOPS * wu + i >= 2 * NM) continue;   // (16-row items: waves 0-1 only)
        const int r = min(8 * (AOPS * w + i) + (lane >> 3), GM_BM - 1);
        const int c = ((lane & 7) ^ row_swz(r)) & (MODE == 0 ? 7 : 3);   // Z_d: 4 chunks
        const uint32_t zo = (uint32_t)(p0 + min(r, rows - 1)) * (uint32_t)(A.ldz * 4) + c * 16;
        dma16(zb, zo, sa + slot * ST_A + i * 1024);
      }
#pragma unroll
      for (int i = 0; i < BOPS; ++i) {   // (the int4 words' placement)
        const int bc = gt_pos(32 * (BOPS * w + i) + (lane >> 1));
        const bool up = MODE == 0 && bc >= 128;
        const int c = min(c0 + (MODE == 0 ? (bc & 127) : bc), N - 1);
        const char *bb = reinterpret_cast<const char *>(uniform_ptr((up ? A.B1 : A.B0) + (size_t)e * N * 16));
        dma16(bb, (uint32_t)c * 32u + 16 * ((lane & 1) ^ gt_half(bc)), sb + slot * ST_B + i * 1024);
      }
#pragma unroll
      for (int i = 0; i < XOPS; ++i) dma4(xbase, xoff[i], sx + slot * ST_X + i * 256);
    };
    // one stage = half a quantization group (64 of K); a group's first stage
    // also brings the ratios and start values.  The stage after the last is
    // the epilogue's (rank 16); later ones load nothing.
    auto stage = [&](auto evenc, int jr, int slot) {
      if (jr >= NS) {
        if (ep_lds && jr == NS) stage_ep(slot);
        return;
      }
      const int j = jr, g = j >> 1;
      const int ja = j < NSA ? j : j - NSA;   // (an int8 base's second plane reads the rows again)
      // destinations re-derived per stage (scalar adds) rather than held
      uint32_t sa = la, sb = lb;
      asm volatile("" : "+s"(sa), "+s"(sb));
#pragma unroll
      for (int i = 0; i < AOPS; ++i)
        if (AOPS * wu + i < 2 * NM)   // (16-row items: waves 0-1 only)
          dma16(abase + (size_t)ja * GM_KS * 2, src_off[i], sa + slot * ST_A + i * 1024);
      // stage step of the int4 words: 32 bytes (plain), a whole stage of
      // the expert's columns, 32 N bytes (packed)
#pragma unroll
      for (int i = 0; i < BOPS; ++i)
        dma16(qbase + (size_t)j * (QP ? (uint32_t)N * 32u : 32u), qoff[i], sb + slot * ST_B + i * 1024);
      if (decltype(evenc)::value) {
        uint32_t sx = lx;
        asm volatile("" : "+s"(sx));
#pragma unroll
        for (int i = 0; i < XOPS; ++i) dma4(xbase + (size_t)g * xstr, xoff[i], sx + slot * ST_X + i * 256);
      }
    };

    f32x4_t acc[NM][NF];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // one stage: 2 k-substeps x NM row fragments x NF column fragments.  Lane
    // group lg takes k = 16 lg + 8 s .. + 7 of the stage in substep s (A chunk
    // 2 lg + s, int4 word 2 lg + s).  A group's first stage advances the
    // accumulators: Q <- Q * ratio + (-136 * row sum).
    //
    // The stage is written as one software pipeline over its 2 NM A
    // fragments (substep-major): the LDS read of fragment i + PD is issued
    // before the NF matrix instructions of fragment i, and the VALU work (the
    // second substep's unpacking, and in a group's first stage the update of
    // row fragment m + 1) sits between them, so it runs in the shadow of the
    // matrix instructions.  The scheduling-group barriers at the end pin that
    // order (the scheduler would otherwise cluster every read right before
    // its use to save registers, exposing the LDS latency).
    constexpr int PD = NM >= 8 ? 2 : (2 * NM < 3 ? 2 * NM : 3);   // A read distance, in fragments
    auto compute = [&](auto odd, int slot) {   // odd: compile-time stage parity
      constexpr bool EVEN = !decltype(odd)::value;
      __builtin_amdgcn_sched_barrier(0);
      u32x2_t bq[NF];
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
        bq[nf] = lds_ld<u32x2_t>((nf & 1 ? offB1 : offB0) + slot * ST_B + fpair(nf) * 32);
      f32x4_t rv[NF], nv4[2];
      if (EVEN) {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
          rv[nf] = lds_ld<f32x4_t>(offR + slot * ST_X + (fpair(nf) + 4 * (nf & 1)) * 4);
        nv4[0] = lds_ld<f32x4_t>(offC + slot * ST_X);
        if (NM > 4) nv4[1] = lds_ld<f32x4_t>(offC + slot * ST_X + 16);
      }
      // substep 1 reads chunk 2 lg + 1, i.e. the neighbouring swizzled chunk
      const uint32_t offA1 = offA0 ^ 16u;
      auto lda = [&](int i) {
        const int sub = i / NM, m = i % NM;
        const u32x4_t a4 = lds_ld<u32x4_t>((sub ? offA1 : offA0) + slot * ST_A + m * 2048);
        return make_uint4(a4.x, a4.y, a4.z, a4.w);
      };
      auto unpack = [&](int sub, uint4 (&bu)[NF]) {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
          const uint32_t x = sub ? bq[nf].y : bq[nf].x;
          bu[nf].x = __builtin_amdgcn_bitop3_b32(x, kMask, kMagic, 0x6A);
          bu[nf].y = __builtin_amdgcn_bitop3_b32(x >> 4, kMask, kMagic, 0x6A);
          bu[nf].z = __builtin_amdgcn_bitop3_b32(x >> 8, kMask, kMagic, 0x6A);
          bu[nf].w = __builtin_amdgcn_bitop3_b32(x >> 12, kMask, kMagic, 0x6A);
        }
      };
      auto advance = [&](int m) {   // a group's first stage: Q <- Q * ratio + start
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[m][nf][i] = __builtin_fmaf(acc[m][nf][i], rv[nf][i], nv4[m >> 2][m & 3]);
      };
      uint4 a[2 * NM], bu0[NF], bu1[NF];
#pragma unroll
      for (int i = 0; i < PD; ++i) a[i] = lda(i);
      unpack(0, bu0);
      if (EVEN) advance(0);
#pragma unroll
      for (int i = 0; i < 2 * NM; ++i) {
        const int sub = i / NM, m = i % NM;
        if (i + PD < 2 * NM) a[i + PD] = lda(i + PD);
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) acc[m][nf] = mfma32(sub ? bu1[nf] : bu0[nf], a[i], acc[m][nf]);
        if (EVEN && sub == 0 && m + 1 < NM) advance(m + 1);
        if (i == NM / 2) unpack(1, bu1);
      }
      // the order above, as scheduling groups
      fwd_stage_sched<NM, NF, EVEN, PD>(std::make_integer_sequence<int, 2 * NM>());
      __builtin_amdgcn_sched_barrier(0);
    };

    // Two-slot ring: step j computes stage j from slot j % 2 while the loads
    // of stage j + 1 (issued at the start of the step) fill the other slot;
    // at the end of the step every wave waits for all of its loads and the
    // block syncs, so stage j + 1 is in LDS when step j + 1 starts.  (A
    // deeper ring would not let loads run longer: the end-of-step wait
    // covers everything issued in the step.)  Stages come in pairs (NS is
    // even), the even one a group's first; the step after the last loads the
    // epilogue's operands (rank 16).
    using even_t = std::integral_constant<bool, false>;
    using odd_t = std::integral_constant<bool, true>;
    using ev_t = std::integral_constant<bool, true>;
    using od_t = std::integral_constant<bool, false>;
    stage(ev_t(), 0, 0);
    __builtin_amdgcn_s_waitcnt(kWaitVm);
    block_barrier();
    for (int j = 0; j < NS; j += 2) {
#define MOE_F_STEP(JJ, PAR, LD, CUR, NXT)       \
  {                                             \
    stage(LD(), (JJ) + 1, NXT);                 \
    compute(PAR(), CUR);                        \
    __builtin_amdgcn_s_waitcnt(kWaitVm);        \
    block_barrier();                            \
  }
      MOE_F_STEP(j, even_t, od_t, 0, 1)
      MOE_F_STEP(j + 1, odd_t, ev_t, 1, 0)
#undef MOE_F_STEP
    }

    // ---- epilogue columns (in the matrix's own column space), re-derived
    // from an opaque copy of the thread index: col = the B-operand column of
    // lane lr, ocol = the first of the lane's four output columns (those of
    // fragment 2t + 1 follow those of 2t)
    int tid2 = threadIdx.x;
    asm volatile("" : "+v"(tid2));
    const int lr2 = tid2 & 15, lg2 = (tid2 >> 4) & 3, w2 = tid2 >> 6;
    int col[NF], ocol[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
      const int mc = c0 + w2 * WCOLS + (fpair(nf) & (MODE == 0 ? 127 : 255));
      col[nf] = mc + gt_col(nf & 1, lr2);
      ocol[nf] = mc + 8 * lg2 + 4 * (nf & 1);
    }
    // mode 0: fragment nf belongs to the up matrix when nf >= NF / 2
    auto is_up = [](int nf) { return MODE == 0 && nf >= NF / 2; };

    // ---- the last group's scale (group 0's ratio) and the adapter term
    // acc += (lam Z) B^T, K = rank in steps of 16 (mode 0: gate fragments
    // take Z_g and B_g, up fragments Z_u and B_u).  Rank 16: all operands
    // from the epilogue stage in ring slot NS % 2, one row fragment at a
    // time; otherwise from global memory.
    constexpr int NSRC = MODE == 0 ? 2 : 1;
    auto zbf = [&](f32x4_t z) {   // lam z rounded to bf16 (nearest even)
      const uint32_t lo = cvt_pk_bf16(A.lam * z[0], A.lam * z[1]);
      const uint32_t hi = cvt_pk_bf16(A.lam * z[2], A.lam * z[3]);
      return __builtin_bit_cast(short4_t, u32x2_t{lo, hi});
    };
    if constexpr (ep_lds) {
      const int es = NS % 2;
      const int wc = w2 * WCOLS;   // the wave's first block column slot
      short4_t bv[NF];
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const f32x4_t sl =
            lds_ld<f32x4_t>(ldsX + es * ST_X + (wc + fpair(nf) + 8 * lg2 + 4 * (nf & 1)) * 4);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][nf][i] *= sl[i];
        const int bc = gt_col(nf & 1, lr2);   // (placed like the int4 words)
        bv[nf] = lds_ld<short4_t>(ldsB + es * ST_B + (wc + fpair(nf) + gt_pos(bc)) * 32 +
                                  16 * ((lg2 >> 1) ^ gt_half(bc)) + 8 * (lg2 & 1));
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m & 1) __builtin_amdgcn_sched_barrier(0);
        const int r = 16 * m + lr2;
#pragma unroll
        for (int src = 0; src < NSRC; ++src) {
          const f32x4_t z = lds_ld<f32x4_t>(ldsA + es * ST_A + r * 128 + (((4 * src + lg2) ^ row_swz(r)) << 4));
          const short4_t av = zbf(z);
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            if ((is_up(nf) ? 1 : 0) != src) continue;
            acc[m][nf] = mfma16(bv[nf], av, acc[m][nf]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const float *rt = is_up(nf) ? A.rt1 : A.rt0;
        const f32x4_t sl = *reinterpret_cast<const f32x4_t *>(rt + (size_t)e * NG * N + min(ocol[nf], N - 4));
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][nf][i] *= sl[i];
      }
      const bool zvec = ((A.r | A.ldz) & 3) == 0;
      for (int j0 = 0; j0 < A.r; j0 += 16) {
        uint32_t kmask[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kmask[i] = j0 + 4 * lg2 + i < A.r ? 0xFFFFu : 0u;
        short4_t bv[NF];
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
          const uint16_t *Bm = is_up(nf) ? A.B1 : A.B0;
          const size_t rowb = ((size_t)e * N + min(col[nf], N - 1)) * A.r;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            bv[nf][i] = (short)(Bm[rowb + min(j0 + 4 * lg2 + i, A.r - 1)] & kmask[i]);
        }
        // Z side: rank positions j0 + 4 lg2 + i past r are zeroed like the B
        // side (the 16-byte load starts at most at r - 4, so it stays inside
        // the row's r values; what it reads past the rank is never used)
        const int jz = min(j0 + 4 * lg2, A.r - 4);
#pragma unroll
        for (int src = 0; src < NSRC; ++src) {
          const float *Zp = src ? A.Z1 : A.Z0;
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const float *zr = Zp + (size_t)(p0 + min(16 * m + lr2, rows - 1)) * A.ldz;
            f32x4_t z;
            if (zvec) {
              z = *reinterpret_cast<const f32x4_t *>(zr + jz);
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) z[i] = zr[min(j0 + 4 * lg2 + i, A.r - 1)];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) z[i] = kmask[i] ? z[i] : 0.f;
            const short4_t av = zbf(z);
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) {
              if ((is_up(nf) ? 1 : 0) != src) continue;
              acc[m][nf] = mfma16(bv[nf], av, acc[m][nf]);
            }
            if (m & 1) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }

    // ---- epilogue: lane (lr, lg) holds, for row 16 m + lr, the eight
    // consecutive columns ocol[2t] .. + 7 in fragments 2t and 2t + 1; each
    // such pair becomes one 16-byte store.
    __builtin_amdgcn_s_waitcnt(kWaitAll);   // trailing (clamped) stage loads
    if (MODE == 0) {
      // H = silu(G) U (and, when saved, the SwiGLU backward's multipliers
      // U s (1 + G (1 - s)) and G s, s = sigmoid(G)); the row sums of H over this
      // item's 128 columns (one quantization group of the down product) are
      // reduced over lane groups by shuffles and over the waves through LDS,
      // and stored as the down product's start values -136 * sum.
      __syncthreads();                          // every wave is done with the ring
      float *red = X.red;   // [WAVES][128 rows]
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int r = 16 * m + lr2;
        float hs = 0.f;
        // gate fragments 0-1 with up fragments 2-3: columns ocol[0] .. + 7
        float sg[8], sl[8];   // sigmoid(G), silu(G)
        uint32_t hw[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const f32x4_t g = acc[m][h2], u = acc[m][h2 + 2];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sg[4 * h2 + i] = sigmoid_rcp(g[i]);
            sl[4 * h2 + i] = g[i] * sg[4 * h2 + i];
          }
          const uint32_t h0 = cvt_pk_bf16(sl[4 * h2] * u[0], sl[4 * h2 + 1] * u[1]);
          const uint32_t h1 = cvt_pk_bf16(sl[4 * h2 + 2] * u[2], sl[4 * h2 + 3] * u[3]);
          hw[2 * h2] = h0;
          hw[2 * h2 + 1] = h1;
          hs += (__uint_as_float(h0 << 16) + __uint_as_float(h0 & 0xFFFF0000u)) +
                (__uint_as_float(h1 << 16) + __uint_as_float(h1 & 0xFFFF0000u));
        }
        if (r < rows) {
          const size_t o = (size_t)(p0 + r) * A.ldo + ocol[0];
          *reinterpret_cast<uint4 *>(&A.out[o]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          if (A.saveG) {
            // the SwiGLU backward's multipliers: dG = dH mG, dU = dH mU
            float mg[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) {
              const float g = acc[m][v >> 2][v & 3], u = acc[m][2 + (v >> 2)][v & 3];
              mg[v] = u * sg[v] * __builtin_fmaf(g, 1.f - sg[v], 1.f);
            }
            *reinterpret_cast<uint4 *>(&A.saveG[o]) =
                make_uint4(cvt_pk_bf16(mg[0], mg[1]), cvt_pk_bf16(mg[2], mg[3]),
                           cvt_pk_bf16(mg[4], mg[5]), cvt_pk_bf16(mg[6], mg[7]));
            *reinterpret_cast<uint4 *>(&A.saveU[o]) =
                make_uint4(cvt_pk_bf16(sl[0], sl[1]), cvt_pk_bf16(sl[2], sl[3]),
                           cvt_pk_bf16(sl[4], sl[5]), cvt_pk_bf16(sl[6], sl[7]));
          }
        }
        hs += __shfl_xor(hs, 16);
        hs += __shfl_xor(hs, 32);
        if (lg2 == 0) red[w2 * GM_BM + r] = hs;
      }
      __syncthreads();
      if (tid2 < rows && A.rsum_out) {
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < WAVES; ++q) v += red[q * GM_BM + tid2];
        A.rsum_out[(size_t)(p0 + tid2) * A.ld_rsum_out + nt] = -136.f * v;
        if (A.rsum_split) A.rsum_out[(size_t)(p0 + tid2) * A.ld_rsum_out + A.NT + nt] = -128.f * v;
      }
    } else {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int r = 16 * m + lr2;
        if (r < rows) {
#pragma unroll
          for (int t = 0; t < NF / 2; ++t) {
            if (ocol[2 * t] < N)
              *reinterpret_cast<uint4 *>(&A.out[(size_t)(p0 + r) * A.ldo + ocol[2 * t]]) =
                  make_uint4(cvt_pk_bf16(acc[m][2 * t][0], acc[m][2 * t][1]),
                             cvt_pk_bf16(acc[m][2 * t][2], acc[m][2 * t][3]),
                             cvt_pk_bf16(acc[m][2 * t + 1][0], acc[m][2 * t + 1][1]),
                             cvt_pk_bf16(acc[m][2 * t + 1][2], acc[m][2 * t + 1][3]));
          }
        }
      }
    }
  }
}

#define MOE_GM_CTX(ringA, ringB, ringX, tokarr)                     \
  GmCtx X;                                                          \
  X.ldsA = lds_addr(ringA);                                         \
  X.ldsB = lds_addr(ringB);                                         \
  X.ldsX = lds_addr(ringX);                                         \
  X.kMask = __builtin_amdgcn_readfirstlane(0x000F000Fu);            \
  asm volatile("v_mov_b32 %0, 0x43084308" : "=v"(X.kMagic));       \
  X.tok = tokarr;                                                   \
  X.red = reinterpret_cast<float *>(ringA)

// All items of one product in one launch: the tiles of launch_build_tiles
// (each expert's rows in tiles of 128, in expert order) times the column
// tiles, split into eight contiguous ranges, one per XCD, so that an expert's
// tiles, its short last one included, run close together on one XCD and
// share its weights in that L2.  Within its range a block draws its next item
// from a counter of the XCD (ctr[xcd], zero at launch); in the gate/up
// product, once its range is used up, it draws from the other XCDs' ranges
// (draw_item).  Each item runs as the
// shortest tile class that holds its rows (32, 64, 96 or 128; a wave-uniform
// branch).  QP: the base in the packed layout.  Two blocks of four waves per
// CU.
template <int MODE, bool EPL, bool QP>
__global__ __launch_bounds__(256, GM_BPC) void grouped_gemm_kernel(const MfmaGemmArgs A,
                                                                   const int *__restrict__ ntiles,
                                                                   int *__restrict__ ctr) {
  // (ringA 32-byte aligned: the second substep's chunk is the first's
  // address with bit 4 flipped)
  __shared__ __attribute__((aligned(32))) uint4 ringA[2][GM_BM * GM_KS * 2 / 16];
  __shared__ uint4 ringB[2][ST_B / 16];
  __shared__ float ringX[2][ST_X / 4];
  __shared__ int tok_lds[GM_BM];
  __shared__ int next_item;
  MOE_GM_CTX(ringA, ringB, ringX, tok_lds);
  const int total = ntiles[0] * A.NT;
  const int xcd = blockIdx.x & 7;
  // (the down product's items are short, and items taken from other XCDs'
  // ranges cost it more than the balance gains: measured 4 % slower)
  constexpr bool steal = MODE == 0;
  int rng = xcd;
  if (threadIdx.x == 0) next_item = draw_item(ctr, total, rng, xcd, steal);
  __syncthreads();
  for (int wi = next_item; wi >= 0; wi = next_item) {
    // every thread has read next_item; the next draw overlaps this item (its
    // value is visible after the item's first barrier)
    __syncthreads();
    if (threadIdx.x == 0) next_item = draw_item(ctr, total, rng, xcd, steal);
    const int ti = wi / A.NT, nt = wi - ti * A.NT;
    const int2 tile = A.tiles[ti];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(GM_BM, A.offsets[e + 1] - p0);
    const int cls = __builtin_amdgcn_readfirstlane((rows + 31) >> 5);   // 32-row units
    if (cls >= 4) gm_item<MODE, 4, 8, EPL, QP>(A, X, e, p0, rows, nt);
    else if (cls == 3) gm_item<MODE, 4, 6, EPL, QP>(A, X, e, p0, rows, nt);
    else if (cls == 2) gm_item<MODE, 4, 4, EPL, QP>(A, X, e, p0, rows, nt);
    else gm_item<MODE, 4, 2, EPL, QP>(A, X, e, p0, rows, nt);
  }
}

// Short batches (decode): every expert's rows in tiles of 16 (a list of
// launch_build_tiles), all of them 16-row items.  The ring holds only 16
// rows, so more blocks are resident per CU (short_bpc: five for gate/up, whose
// six column tiles per expert then fill two rounds instead of leaving most of
// a third empty at decode sizes; four for down), which keeps more weight loads
// in flight where the products stream the weights of many experts for a few
// rows each.  The items are split into eight contiguous ranges, one per XCD,
// dealt round-robin to the XCD's blocks.
template <int MODE, bool EPL, bool QP>
__global__ __launch_bounds__(256, short_bpc(MODE)) void grouped_gemm_short_kernel(
    const MfmaGemmArgs A, const int *__restrict__ ntiles) {
  constexpr int NM = 1;
  constexpr int ST_A = 16 * NM * GM_KS * 2;
  __shared__ __attribute__((aligned(32))) uint4 ringA[2][ST_A / 16];
  __shared__ uint4 ringB[2][ST_B / 16];
  __shared__ float ringX[2][ST_X / 4];
  __shared__ int tok_lds[GM_BM];
  MOE_GM_CTX(ringA, ringB, ringX, tok_lds);
  const int total = ntiles[0] * A.NT;
  const int nper = gridDim.x >> 3, xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int wbeg = (int)(((long long)total * xcd) >> 3);
  const int wend = (int)(((long long)total * (xcd + 1)) >> 3);
  for (int wi = wbeg + bi; wi < wend; wi += nper) {
    const int ti = wi / A.NT, nt = wi - ti * A.NT;
    const int2 tile = A.tiles[ti];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(16 * NM, A.offsets[e + 1] - p0);
    gm_item<MODE, 4, NM, EPL, QP>(A, X, e, p0, rows, nt);
  }
}
#undef MOE_GM_CTX

// ------------------------------------------------------ forward packing --
// q [E][N][K/2] -> [E][K/64][N][32 B]: each 32-byte K block of a storage row
// moves unchanged to the run of its (expert, 64-wide K step).  One thread per
// 16 bytes, in output order (the writes are contiguous; a wave's reads are 32
// rows x 32 bytes).
__global__ __launch_bounds__(256) void pack_fwd_kernel(const uint4 *__restrict__ q, int N, int K,
                                                       size_t n16, uint4 *__restrict__ qf) {
  const size_t o = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= n16) return;
  const size_t per_e = (size_t)N * K / 32;   // 16-byte units per expert
  const size_t e = o / per_e, r = o - e * per_e;
  const size_t j = r / ((size_t)N * 2), cr = r - j * N * 2;   // cr = 2 c + half
  const size_t c = cr >> 1, h = cr & 1;
  qf[o] = q[e * per_e + c * (K / 32) + j * 2 + h];
}

void launch_pack_fwd(const uint8_t *q, int E, int N, int K, uint8_t *qf, hipStream_t st) {
  const size_t n16 = (size_t)E * N * K / 32;
  pack_fwd_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, st>>>(
      reinterpret_cast<const uint4 *>(q), N, K, n16, reinterpret_cast<uint4 *>(qf));
}

// An int8 base as two int4 planes along K: q = 16 h + l with h = q >> 4
// (-8 .. 7) and l = q & 15 (0 .. 15); plane 1 holds h and plane 2 l - 8, as
// two's-complement nibbles.  With the plane scales 16 s and s, and the
// matrix cores' offset of 136 removed as 136 on plane 1 and 128 on plane 2,
// the products sum 16 s h + s l = s q exactly.  [E][N][K] bytes ->
// [E][2K/64][N][32 B] (stage j < K/64: plane 1, K-step j; then plane 2),
// every 8 values of K one word in the nibble order of the int4 layout (slot
// i holds value 2i for i < 4 and value 2(i-4)+1 for i >= 4).  One thread per
// 16 output bytes (32 values), in output order.
DEV uint32_t int8_plane_word(uint2 v, bool low) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = ((i < 4 ? v.x : v.y) >> (8 * (i & 3))) & 0xFFu;
    const uint32_t nib = low ? ((b & 15u) ^ 8u) : (b >> 4);
    const int slot = (i & 1) ? 4 + (i >> 1) : (i >> 1);
    w |= nib << (4 * slot);
  }
  return w;
}

__global__ __launch_bounds__(256) void pack_fwd_int8_kernel(const uint8_t *__restrict__ q, int N,
                                                            int K, size_t n16,
                                                            uint4 *__restrict__ qf) {
  const size_t o = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= n16) return;
  const size_t per_e = (size_t)N * K / 16;   // 16-byte output units per expert (2K values)
  const size_t e = o / per_e, r = o - e * per_e;
  const size_t j = r / ((size_t)N * 2), cr = r - j * N * 2;   // stage, 2 c + half
  const size_t c = cr >> 1, h = cr & 1;
  const size_t nk = (size_t)K / 64;
  const bool low = j >= nk;
  const size_t k0 = (low ? j - nk : j) * 64 + 32 * h;
  const uint4 *src = reinterpret_cast<const uint4 *>(q + (e * N + c) * K + k0);
  const uint4 a = src[0], b = src[1];
  uint4 out;
  out.x = int8_plane_word(make_uint2(a.x, a.y), low);
  out.y = int8_plane_word(make_uint2(a.z, a.w), low);
  out.z = int8_plane_word(make_uint2(b.x, b.y), low);
  out.w = int8_plane_word(make_uint2(b.z, b.w), low);
  qf[o] = out;
}

void launch_pack_fwd_int8(const uint8_t *q, int E, int N, int K, uint8_t *qf, hipStream_t st) {
  const size_t n16 = (size_t)E * N * K / 16;
  pack_fwd_int8_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, st>>>(
      q, N, K, n16, reinterpret_cast<uint4 *>(qf));
}

int mfma_tile_rows() { return GM_BM; }
int mfma_blocks_per_cu() { return GM_BPC; }

void launch_group_rowsum(const void *a, int rows, int K, int G, float scale, float *out,
                         hipStream_t st, bool split, float scale2) {
  size_t n = (size_t)rows * (K / G);
  group_rowsum_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>((const bf16_t *)a, rows, K, G,
                                                                   scale, out, split, scale2);
}

void launch_scale_ratio(const uint16_t *s, int E, int N, int ng, float *rt, hipStream_t st,
                        bool split) {
  dim3 grid((N + 255) / 256, E);
  scale_ratio_kernel<<<grid, 256, 0, st>>>(s, E, N, ng, rt, split);
}

// One launch per product over the tiles of launch_build_tiles (ctr: eight
// zeroed counters), reading the packed base where it is given (both matrices
// of gate/up, or down).
void launch_grouped_gemm(int mode, const MfmaGemmArgs &A, const int *ntiles, int *ctr, int grid,
                         hipStream_t st) {
  // operands of the epilogue through the LDS ring: rank 16, Z rows 16-byte aligned
  const bool epl = A.r == 16 && (A.ldz & 3) == 0;
  const bool qp = A.qp0 && (mode == 1 || A.qp1);
#define MOE_GG3(MODE, EPL)                                                                 \
  do {                                                                                     \
    if (qp) grouped_gemm_kernel<MODE, EPL, true><<<grid, 256, 0, st>>>(A, ntiles, ctr);      \
    else grouped_gemm_kernel<MODE, EPL, false><<<grid, 256, 0, st>>>(A, ntiles, ctr);        \
  } while (0)
  if (mode == 0) {
    if (epl) MOE_GG3(0, true); else MOE_GG3(0, false);
  } else {
    if (epl) MOE_GG3(1, true); else MOE_GG3(1, false);
  }
#undef MOE_GG3
}

// The short-batch launch over 16-row tiles (ntiles: the count of the list);
// grid: GM_BPC blocks per CU, scaled to short_bpc(mode)
void launch_grouped_gemm_short(int mode, const MfmaGemmArgs &A, const int *ntiles, int grid,
                               hipStream_t st) {
  grid = (grid / GM_BPC * short_bpc(mode)) & ~7;
  const bool epl = A.r == 16 && (A.ldz & 3) == 0;
  // the packed base where given
  const bool qp = A.qp0 && (mode == 1 || A.qp1);
#define MOE_GS(MODE, EPL, QP) grouped_gemm_short_kernel<MODE, EPL, QP><<<grid, 256, 0, st>>>(A, ntiles)
#define MOE_GS2(MODE, EPL)                     \
  do {                                         \
    if (qp) MOE_GS(MODE, EPL, true);           \
    else MOE_GS(MODE, EPL, false);             \
  } while (0)
  if (mode == 0) {
    if (epl) MOE_GS2(0, true); else MOE_GS2(0, false);
  } else {
    if (epl) MOE_GS2(1, true); else MOE_GS2(1, false);
  }
#undef MOE_GS2
#undef MOE_GS
}

}  // namespace moe
