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
//  * K streams through a 3-deep LDS ring in half-group stages (64 of K): the
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
// in k order)
__global__ void group_rowsum_kernel(const bf16_t *__restrict__ a, int rows, int K, int G,
                                    float scale, float *__restrict__ out) {
  const int ng = K / G;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * ng) return;
  size_t row = i / ng;
  int g = (int)(i % ng);
  const uint4 *p = reinterpret_cast<const uint4 *>(a + row * K + (size_t)g * G);
  float s = 0.f;
  for (int v = 0; v < G / 8; ++v) {
    uint4 u = p[v];
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s += __uint_as_float(w[j] << 16);
      s += __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  out[i] = scale * s;
}

// ------------------------------------------------------------ scale ratios --
// Per column c of a quantized matrix [E][N] with ng groups, group-major:
// rt[e][g][c] = s'[g-1] / s'[g] for g >= 1 and rt[e][0][c] = s'[ng-1] (the
// final multiplier), where s' is the bf16 scale with magnitudes below 2^-100
// raised to 2^-100 (so a zero scale leaves a contribution of at most 2^-100
// times its partial sum).  One thread per column: its ng scales are one
// contiguous run, and each group's writes are contiguous across the wave.
__global__ __launch_bounds__(256) void scale_ratio_kernel(const uint16_t *__restrict__ s, int E,
                                                          int N, int ng, float *__restrict__ rt) {
  const int e = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c >= N) return;
  auto guard = [](float v) { return fabsf(v) < 0x1p-100f ? 0x1p-100f : v; };
  const uint16_t *sc = s + ((size_t)e * N + c) * ng;
  float *out = rt + (size_t)e * ng * N + c;
  float prev = guard(bf2f(sc[0]));
  for (int g = 1; g < ng; ++g) {
    const float cur = guard(bf2f(sc[g]));
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
// WAVES waves per block, each with all rows of the item and NF column
// fragments of 16 (mode 0: half gate, half up, so SwiGLU pairs up in a lane).
// Gate/up runs 8 waves x 2 fragments (four waves per SIMD, 128 VGPRs);
// down runs 4 waves x 4 fragments (two waves per SIMD: each A fragment read
// from LDS feeds four matrix instructions).  NM (2, 4, 6, 8) is the number of
// 16-row fragments of the item's tile class: each class of tiles (32, 64, 96,
// 128 rows) is its own launch, so a short tail tile costs only its rows.
// blocks per CU of tile class NM: the 32-row class (A ring of 12 KB, about
// 130 VGPRs) runs three, the others two
constexpr int gm_bpc(int NM) { return NM <= 2 ? 3 : GM_BPC; }

// QP: q0, q1 in the stage-major packed layout (launch_pack_fwd)
template <int MODE, int WAVES, int NM, bool EPL, bool QP>
__global__ __launch_bounds__(64 * WAVES, WAVES / 4 * gm_bpc(NM)) void grouped_gemm_kernel(
    const MfmaGemmArgs A, const int *__restrict__ cls_count, const int *__restrict__ cls_start) {
  // (hip-clang passes the second launch bound through as the minimum number
  // of waves per SIMD: b blocks per CU are b WAVES / 4 waves per SIMD, i.e.
  // at most 256 VGPRs for two blocks of four waves, 168 for three.)
  constexpr int NF = 16 / WAVES;                 // column fragments per wave
  constexpr int BOPS = 8 / WAVES;                // int4-word loads per wave and stage
  constexpr int NT_ = 64 * WAVES;                // threads
  constexpr int WCOLS = (MODE == 0 ? 128 : 256) / WAVES;   // block column slots per wave (per matrix in mode 0)
  constexpr int AOPS = (2 * NM + WAVES - 1) / WAVES;       // 8-row A loads per wave and stage
  constexpr int XOPS = 8 / WAVES;                // group-data loads per wave (even stages)
  // first block column slot of fragment nf relative to the wave's columns:
  // mode 0 gate slots 0..127 then up 128..255, mode 1 0..255
  constexpr auto nfc = [](int nf) {
    return MODE == 0 ? (nf / (NF / 2)) * 128 + (nf % (NF / 2)) * 16 : nf * 16;
  };
  // a 3-deep ring of half-group stages; after the K loop the first 2 KB of
  // the A ring hold the cross-wave row sums of H.
  // (ringA 32-byte aligned: the second substep's chunk is the first's
  // address with bit 4 flipped)
  constexpr int ST_A = 16 * NM * GM_KS * 2;     // A stage: the class's rows x 64 K
  static_assert(3 * ST_A >= WAVES * GM_BM * 4, "the row-sum exchange lives in the A ring");
  __shared__ __attribute__((aligned(32))) uint4 ringA[3][ST_A / 16];
  __shared__ uint4 ringB[3][ST_B / 16];
  __shared__ float ringX[3][ST_X / 4];
  __shared__ int tok_lds[GM_BM];

  const int K = A.K, N = A.N, NG = K / GM_KG, NS = 2 * NG;   // NS: half-group stages
  const int BNO = MODE == 0 ? 128 : 256;   // output columns per item (per matrix)
  const int total = cls_count[0] * A.NT, tbase = cls_start[0];
  const int nper = gridDim.x >> 3, xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int wbeg = (int)(((long long)total * xcd) >> 3);
  const int wend = (int)(((long long)total * (xcd + 1)) >> 3);
  // unpack constants held in registers: each bf16 pair is one shift and one
  // three-input logic op, ((w >> 4i) & 0x000F000F) ^ 0x43084308
  const uint32_t kMask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t kMagic;
  asm volatile("v_mov_b32 %0, 0x43084308" : "=v"(kMagic));
  const uint32_t ldsA = lds_addr(ringA), ldsB = lds_addr(ringB), ldsX = lds_addr(ringX);

  for (int wi = wbeg + bi; wi < wend; wi += nper) {
    // thread indices are re-derived per item through an opaque copy so that
    // the compiler does not keep tid-only address arithmetic live across the
    // whole persistent loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int ti = wi / A.NT, nt = wi - ti * A.NT;
    const int2 tile = A.tiles[tbase + ti];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(16 * NM, A.offsets[e + 1] - p0);
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
    const uint8_t *qbase =
        (const uint8_t *)uniform_ptr((MODE == 0 && w >= 2 ? A.q1 : A.q0) + (size_t)e * N * (K / 2));
    uint32_t qoff[BOPS];
#pragma unroll
    for (int i = 0; i < BOPS; ++i) {
      const int bc = 32 * (BOPS * w + i) + (lane >> 1);
      const int c = min(c0 + (MODE == 0 ? (bc & 127) : bc), N - 1);
      // (packed base: column c of a stage at 32 c; plain: at c K/2)
      qoff[i] = (uint32_t)c * (QP ? 32u : (uint32_t)(K / 2)) + 16 * (lane & 1);
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
    // operand is block column slot w * WCOLS + nfc + lr; the lane's
    // accumulator holds the four output columns from slot w * WCOLS + nfc + 4 lg.
    const uint32_t offA0 = opaque(ldsA + lr * 128 + (((2 * lg) ^ row_swz(lr)) << 4)),
                   offB = opaque(ldsB + (w * WCOLS + lr) * 32 + 8 * lg),
                   offR = opaque(ldsX + (w * WCOLS + 4 * lg) * 4),
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
        const int r = min(8 * (AOPS * w + i) + (lane >> 3), GM_BM - 1);
        const int c = ((lane & 7) ^ row_swz(r)) & (MODE == 0 ? 7 : 3);   // Z_d: 4 chunks
        const uint32_t zo = (uint32_t)(p0 + min(r, rows - 1)) * (uint32_t)(A.ldz * 4) + c * 16;
        dma16(zb, zo, sa + slot * ST_A + i * 1024);
      }
#pragma unroll
      for (int i = 0; i < BOPS; ++i) {
        const int bc = 32 * (BOPS * w + i) + (lane >> 1);
        const bool up = MODE == 0 && bc >= 128;
        const int c = min(c0 + (MODE == 0 ? (bc & 127) : bc), N - 1);
        const char *bb = reinterpret_cast<const char *>(uniform_ptr((up ? A.B1 : A.B0) + (size_t)e * N * 16));
        dma16(bb, (uint32_t)c * 32u + 16 * (lane & 1), sb + slot * ST_B + i * 1024);
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
      // destinations re-derived per stage (scalar adds) rather than held
      uint32_t sa = la, sb = lb;
      asm volatile("" : "+s"(sa), "+s"(sb));
#pragma unroll
      for (int i = 0; i < AOPS; ++i)
        dma16(abase + (size_t)j * GM_KS * 2, src_off[i], sa + slot * ST_A + i * 1024);
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
    constexpr int PD = NM >= 8 ? 2 : 3;   // A read distance, in fragments
    auto compute = [&](auto odd, int slot) {   // odd: compile-time stage parity
      constexpr bool EVEN = !decltype(odd)::value;
      __builtin_amdgcn_sched_barrier(0);
      u32x2_t bq[NF];
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) bq[nf] = lds_ld<u32x2_t>(offB + slot * ST_B + nfc(nf) * 32);
      f32x4_t rv[NF], nv4[2];
      if (EVEN) {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) rv[nf] = lds_ld<f32x4_t>(offR + slot * ST_X + nfc(nf) * 4);
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

    // 3-deep ring: step j computes from slot j % 3 while the loads of stage
    // j + 2 (issued at the start of the step) are in flight; at the end of
    // the step every wave waits for all of its loads and the block syncs, so
    // stage j + 1 is in LDS when step j + 1 starts and slot j % 3 is free for
    // stage j + 3.  The loop runs in groups of six stages (three ring slots,
    // two parities); stages past the end compute nothing (uniform branch)
    // but still issue their (clamped) loads.
    using even_t = std::integral_constant<bool, false>;
    using odd_t = std::integral_constant<bool, true>;
    using ev_t = std::integral_constant<bool, true>;
    using od_t = std::integral_constant<bool, false>;
    stage(ev_t(), 0, 0);
    stage(od_t(), 1, 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm);
    block_barrier();
    for (int j = 0; j < NS; j += 6) {
#define MOE_F_STEP(JJ, PAR, LD, CUR, NXT)       \
  {                                             \
    const int jj = (JJ);                        \
    stage(LD(), jj + 2, NXT);                   \
    if (jj < NS) compute(PAR(), CUR);           \
    __builtin_amdgcn_s_waitcnt(kWaitVm); \
    block_barrier();                            \
  }
      MOE_F_STEP(j, even_t, ev_t, 0, 2)
      MOE_F_STEP(j + 1, odd_t, od_t, 1, 0)
      MOE_F_STEP(j + 2, even_t, ev_t, 2, 1)
      MOE_F_STEP(j + 3, odd_t, od_t, 0, 2)
      MOE_F_STEP(j + 4, even_t, ev_t, 1, 0)
      MOE_F_STEP(j + 5, odd_t, od_t, 2, 1)
#undef MOE_F_STEP
    }

    // ---- epilogue columns (in the matrix's own column space), re-derived
    // from an opaque copy of the thread index: col = the B-operand column of
    // lane lr, ocol = the first of the lane's four output columns
    int tid2 = threadIdx.x;
    asm volatile("" : "+v"(tid2));
    const int lr2 = tid2 & 15, lg2 = (tid2 >> 4) & 3, w2 = tid2 >> 6;
    int col[NF], ocol[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
      const int mc = c0 + w2 * WCOLS + (MODE == 0 ? nfc(nf) & 127 : nfc(nf));
      col[nf] = mc + lr2;
      ocol[nf] = mc + 4 * lg2;
    }
    // mode 0: fragment nf belongs to the up matrix when nf >= NF / 2
    auto is_up = [](int nf) { return MODE == 0 && nf >= NF / 2; };

    // ---- the last group's scale (group 0's ratio) and the adapter term
    // acc += (lam Z) B^T, K = rank in steps of 16 (mode 0: gate fragments
    // take Z_g and B_g, up fragments Z_u and B_u).  Rank 16: all operands
    // from the epilogue stage in ring slot NS % 3, one row fragment at a
    // time; otherwise from global memory.
    constexpr int NSRC = MODE == 0 ? 2 : 1;
    auto zbf = [&](f32x4_t z) {   // lam z rounded to bf16 (nearest even)
      const uint32_t lo = cvt_pk_bf16(A.lam * z[0], A.lam * z[1]);
      const uint32_t hi = cvt_pk_bf16(A.lam * z[2], A.lam * z[3]);
      return __builtin_bit_cast(short4_t, u32x2_t{lo, hi});
    };
    if constexpr (ep_lds) {
      const int es = NS % 3;
      const int wc = w2 * WCOLS;   // the wave's first block column slot
      short4_t bv[NF];
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const f32x4_t sl = lds_ld<f32x4_t>(ldsX + es * ST_X + (wc + nfc(nf) + 4 * lg2) * 4);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][nf][i] *= sl[i];
        bv[nf] = lds_ld<short4_t>(ldsB + es * ST_B + (wc + nfc(nf) + lr2) * 32 + 8 * lg2);
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
        const int jz = min(j0 + 4 * lg2, A.r - 1);
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

    // ---- epilogue: lane (lr, lg) holds, for row 16 m + lr, the four
    // consecutive columns ocol[nf] .. + 3; each becomes one 8-byte store.
    __builtin_amdgcn_s_waitcnt(kWaitAll);   // trailing (clamped) stage loads
    if (MODE == 0) {
      // H = silu(G) U (and G, U when saved); the row sums of H over this
      // item's 128 columns (one quantization group of the down product) are
      // reduced over lane groups by shuffles and over the waves through LDS,
      // and stored as the down product's start values -136 * sum.
      __syncthreads();                          // every wave is done with the ring
      float *red = reinterpret_cast<float *>(ringA);   // [WAVES][128 rows]
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int r = 16 * m + lr2;
        float hs = 0.f;
#pragma unroll
        for (int nf = 0; nf < NF / 2; ++nf) {
          const f32x4_t g = acc[m][nf], u = acc[m][nf + NF / 2];
          u32x2_t h;
          h.x = cvt_pk_bf16(silu_rcp(g[0]) * u[0], silu_rcp(g[1]) * u[1]);
          h.y = cvt_pk_bf16(silu_rcp(g[2]) * u[2], silu_rcp(g[3]) * u[3]);
          hs += (__uint_as_float(h.x << 16) + __uint_as_float(h.x & 0xFFFF0000u)) +
                (__uint_as_float(h.y << 16) + __uint_as_float(h.y & 0xFFFF0000u));
          if (r < rows) {
            const size_t o = (size_t)(p0 + r) * A.ldo + ocol[nf];
            *reinterpret_cast<u32x2_t *>(&A.out[o]) = h;
            if (A.saveG)
              *reinterpret_cast<u32x2_t *>(&A.saveG[o]) =
                  u32x2_t{cvt_pk_bf16(g[0], g[1]), cvt_pk_bf16(g[2], g[3])};
            if (A.saveU)
              *reinterpret_cast<u32x2_t *>(&A.saveU[o]) =
                  u32x2_t{cvt_pk_bf16(u[0], u[1]), cvt_pk_bf16(u[2], u[3])};
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
      }
    } else {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int r = 16 * m + lr2;
        if (r < rows) {
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            if (ocol[nf] < N)
              *reinterpret_cast<u32x2_t *>(&A.out[(size_t)(p0 + r) * A.ldo + ocol[nf]]) =
                  u32x2_t{cvt_pk_bf16(acc[m][nf][0], acc[m][nf][1]),
                          cvt_pk_bf16(acc[m][nf][2], acc[m][nf][3])};
          }
        }
      }
    }
  }
}

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

// ------------------------------------------------------------ tile classes --
// The work list of the grouped GEMMs: each expert's rows in tiles of 128,
// the last (partial) one rounded up to 32, 64, 96 or 128 rows.  tiles holds
// the 128-row class first, then 96, 64, 32 (each in expert order); cnt[c] and
// cnt[4 + c] are the count and first index of class c (c = 0: 128 rows ..
// c = 3: 32 rows).  One 1024-thread block (E <= 1024).
__global__ __launch_bounds__(1024) void build_class_tiles_kernel(const int32_t *__restrict__ offsets,
                                                                 int E, int2 *__restrict__ tiles,
                                                                 int *__restrict__ cnt) {
  __shared__ int sc[4][1024];
  const int e = threadIdx.x;
  int lo = 0, n = 0;
  if (e < E) {
    lo = offsets[e];
    n = offsets[e + 1] - lo;
  }
  const int nfull = n >> 7, tail = n & 127;
  const int tcls = tail == 0 ? -1 : 3 - ((tail - 1) >> 5);   // 97..127 -> 0, 1..32 -> 3
  int c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) c[k] = (k == 0 ? nfull : 0) + (tcls == k ? 1 : 0);
#pragma unroll
  for (int k = 0; k < 4; ++k) sc[k][e] = c[k];
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = e >= off ? sc[k][e - off] : 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) sc[k][e] += v[k];
    __syncthreads();
  }
  int start[4], s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    start[k] = s;
    s += sc[k][1023];
  }
  // class 0: the full tiles, then a 97..127-row tail
  int pos = start[0] + sc[0][e] - c[0];
  for (int i = 0; i < c[0]; ++i) tiles[pos + i] = make_int2(e, lo + 128 * i);
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (c[k]) tiles[start[k] + sc[k][e] - 1] = make_int2(e, lo + 128 * nfull);
  if (e == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cnt[k] = sc[k][1023];
      cnt[4 + k] = start[k];
    }
  }
}

int mfma_tile_rows() { return GM_BM; }
int mfma_blocks_per_cu() { return GM_BPC; }

void launch_group_rowsum(const void *a, int rows, int K, int G, float scale, float *out,
                         hipStream_t st) {
  size_t n = (size_t)rows * (K / G);
  group_rowsum_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>((const bf16_t *)a, rows, K, G,
                                                                   scale, out);
}

void launch_scale_ratio(const uint16_t *s, int E, int N, int ng, float *rt, hipStream_t st) {
  dim3 grid((N + 255) / 256, E);
  scale_ratio_kernel<<<grid, 256, 0, st>>>(s, E, N, ng, rt);
}

void launch_class_tiles(const int32_t *offsets, int E, int2 *tiles, int *cnt, hipStream_t st) {
  build_class_tiles_kernel<<<1, 1024, 0, st>>>(offsets, E, tiles, cnt);
}

// The launch of tile class cls (0: 128 rows, 1: 96, 2: 64, 3: 32); cnt as
// written by launch_class_tiles.
void launch_grouped_gemm(int mode, const MfmaGemmArgs &A, const int *cnt, int cls, int grid,
                         hipStream_t st) {
  const int *c = cnt + cls, *s = cnt + 4 + cls;
  // grid: GM_BPC blocks per CU; the 32-row class runs gm_bpc(2) per CU
  if (cls == 3) grid = (grid / GM_BPC * gm_bpc(2)) & ~7;
  // operands of the epilogue through the LDS ring: rank 16, Z rows 16-byte aligned
  const bool epl = A.r == 16 && (A.ldz & 3) == 0;
  // the packed base where given and used (P.q0 null: plain layout)
  MfmaGemmArgs P = A;
  const bool use_p = A.qp0 && (mode == 1 || (A.qp1 && cls != 0));
  P.q0 = use_p ? A.qp0 : nullptr;
  P.q1 = use_p ? A.qp1 : nullptr;
#define MOE_GG2(MODE, NM, QP)                                                        \
  if (epl) grouped_gemm_kernel<MODE, 4, NM, true, QP><<<grid, 256, 0, st>>>(QP ? P : A, c, s);  \
  else grouped_gemm_kernel<MODE, 4, NM, false, QP><<<grid, 256, 0, st>>>(QP ? P : A, c, s)
#define MOE_GG(MODE, NM)                                                \
  do {                                                                  \
    if (P.q0) { MOE_GG2(MODE, NM, true); } else { MOE_GG2(MODE, NM, false); } \
  } while (0)
  if (mode == 0) {
    if (cls == 0) MOE_GG(0, 8); else if (cls == 1) MOE_GG(0, 6); else if (cls == 2) MOE_GG(0, 4); else MOE_GG(0, 2);
  } else {
    if (cls == 0) MOE_GG(1, 8); else if (cls == 1) MOE_GG(1, 6); else if (cls == 2) MOE_GG(1, 4); else MOE_GG(1, 2);
  }
#undef MOE_GG
#undef MOE_GG2
}

}  // namespace moe
