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
// Design (one 256-thread block = 4 waves, 128 rows x N-tile per work item):
//  * Work items (M-tile, N-tile) are processed by a persistent grid.  Each of
//    the 8 XCDs takes a contiguous eighth of the item list, so the rows and
//    weights of neighbouring tiles stay in that XCD's L2.
//  * The A rows (x gathered by token, or H) stream through LDS one
//    quantization group (128 of K) at a time, double buffered, loaded with
//    global_load_lds_dwordx4 straight into LDS in an XOR-swizzled layout
//    (16-byte chunk c of row r lives at chunk c ^ (r & 15)) so the MFMA
//    operand reads are bank-conflict free.
//  * Each wave owns 64 output columns for all 128 rows.  Its int4 weights are
//    read straight from global memory (16 bytes per lane per group and 16
//    columns) and unpacked in registers: a nibble u (offset by 8) becomes the
//    bf16 bit pattern 0x4300 | u, i.e. the exact value 136 + q.  The offset is
//    removed exactly by starting every group's accumulation at
//    -136 * (sum of that group's A row), a per-row value precomputed in
//    float32; then the group's partial product is scaled by the bf16 group
//    scale into the float32 accumulator.  The weights therefore enter the
//    matrix cores exactly (no rounding of s*q).
//  * MFMA v_mfma_f32_16x16x32_bf16: within a group, lane group lg = lane/16
//    covers K offsets [32 lg, 32 lg + 32), k-step s the 8 values 32 lg + 8 s.
//    A and B use the same mapping, so the products pair up correctly.
//  * Epilogue: the adapter term (lam Z) B^T is one more MFMA (K = rank) into
//    the same accumulator; gate/up applies SwiGLU in registers (a lane holds
//    the matching gate and up columns), writes H (bf16) and, for the down
//    product's offset correction, the row sums of H per group.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

constexpr int GM_BM = 64;    // rows per tile
constexpr int GM_BPC = 2;    // resident blocks per CU
constexpr int GM_KG = 128;   // quantization group
constexpr int GM_KS = 64;    // K per pipeline stage (half a group)


// One pipeline stage in LDS (byte offsets within the stage): A rows (64 x 64
// bf16, 16-byte chunks XOR-swizzled by row), int4 words (32 bytes per block
// column), the A row sums of the stage's group, the group scale per block
// column (bf16 in the low half of a 4-byte slot).
constexpr int FS_A = 0, FS_B = FS_A + GM_BM * GM_KS * 2, FS_C = FS_B + 256 * GM_KS / 2,
              FS_S = FS_C + GM_BM * 4, FS_BYTES = FS_S + 256 * 4;

// ---------------------------------------------------------------- row sums --
// out[row][g] = sum of a[row][g*G .. g*G+G) (bf16 values, float32 sum in k order)
__global__ void group_rowsum_kernel(const bf16_t *__restrict__ a, int rows, int K, int G,
                                    float *__restrict__ out) {
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
  out[i] = s;
}

// ------------------------------------------------------------ grouped GEMM --
// MODE 0: gate/up with SwiGLU epilogue (A = x rows gathered by token); a work
//         item covers 64 rows x 128 columns of both gate and up.
// MODE 1: down (A = H rows in permuted order); 64 rows x 256 columns.
// 4 waves, each with all 64 rows and a quarter of the columns (MODE 0: 32 gate
// + the same 32 up columns, MODE 1: 64 columns).  Two blocks share a CU so
// that one block's memory waits overlap the other's matrix work.
//
// The products are formed transposed, D^T = W X^T: the unpacked weights are
// the first MFMA operand and the A rows the second, so a lane's accumulator
// holds one row and four consecutive output columns.  The epilogue then packs
// four bf16 results into one 8-byte store and the per-row group sums (the
// -136 start value) are one broadcast value per lane.
template <int MODE>
__global__ __launch_bounds__(256, GM_BPC) void grouped_gemm_kernel(const MfmaGemmArgs A) {
  // a 3-deep ring of half-group stages (A rows, int4 words, A row sums and
  // scales of the group) in one LDS array; after the K loop its first 1 KB
  // holds the cross-wave row sums of H.
  __shared__ uint4 ring[3 * FS_BYTES / 16];
  __shared__ int tok_lds[GM_BM];

  const int K = A.K, N = A.N, NG = K / GM_KG, NS = 2 * NG;   // NS: half-group stages
  const int BNO = MODE == 0 ? 128 : 256;   // output columns per item (per matrix)
  const int total = A.ntiles[0] * A.NT;
  const int nper = gridDim.x >> 3, xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int wbeg = (int)(((long long)total * xcd) >> 3);
  const int wend = (int)(((long long)total * (xcd + 1)) >> 3);
  // unpack constants held in registers: each bf16 pair is one shift and one
  // three-input logic op, ((w >> 4i) & 0x000F000F) ^ 0x43084308
  const uint32_t kMask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t kMagic;
  asm volatile("v_mov_b32 %0, 0x43084308" : "=v"(kMagic));
  const uint32_t ring_lds = lds_addr(ring);

  for (int wi = wbeg + bi; wi < wend; wi += nper) {
    // thread indices are re-derived per item through an opaque copy so that
    // the compiler does not keep tid-only address arithmetic live (and
    // spilled) across the whole persistent loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int ti = wi / A.NT, nt = wi - ti * A.NT;
    const int2 tile = A.tiles[ti];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(GM_BM, A.offsets[e + 1] - p0);
    const int c0 = nt * BNO;
    __syncthreads();  // LDS of the previous item is free
    if (tid < GM_BM) {
      const int p = p0 + min(tid, rows - 1);
      tok_lds[tid] = MODE == 0 ? A.perm_src[p] / A.kk : p;
    }
    __syncthreads();

    // ---- A staging: 64 rows x 8 chunks of 16 B per stage; wave w, op i
    // covers rows 8 (2w + i) .. +7; chunk c of row r lives at c ^ (r & 7)
    uint32_t src_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * (w * 2 + i) + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);
      src_off[i] = (uint32_t)tok_lds[r] * (uint32_t)(A.lda * 2) + c * 16;
    }
    const char *abase = reinterpret_cast<const char *>(A.a);

    // ---- this wave's columns: 4 fragments of 16.  Block column slots: mode 0
    // gate 0..127 then up 128..255, mode 1 0..255.  bslot / col: the column
    // whose int4 word lane (lr) feeds into the first MFMA operand; oslot: the
    // first of the four consecutive output columns the lane accumulates.
    int col[4], bslot[4], oslot[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int base = MODE == 0 ? (nf >> 1) * 128 + w * 32 + (nf & 1) * 16 : w * 64 + nf * 16;
      bslot[nf] = base + lr;
      oslot[nf] = base + 4 * lg;
      col[nf] = c0 + (MODE == 0 ? (base & 127) : base) + lr;
    }
    const uint16_t *sb0 = A.s0, *sb1 = MODE == 0 ? A.s1 : A.s0;
    // int4 staging: wave w, op i covers block columns 32 (2w + i) .. +31, 32 B
    // each (all gate or all up within one op)
    const uint8_t *qbase[2];
    uint32_t qoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int bc = 32 * (2 * w + i) + (lane >> 1);
      const bool up = MODE == 0 && bc >= 128;
      const int c = min(c0 + (MODE == 0 ? (bc & 127) : bc), N - 1);
      qbase[i] = (const uint8_t *)uniform_ptr((up ? A.q1 : A.q0) + (size_t)e * N * (K / 2));
      qoff[i] = (uint32_t)c * (uint32_t)(K / 2) + 16 * (lane & 1);
    }
    // scale staging: wave w, lane l -> block column 64 w + l (mode 0: gate
    // columns first, then up), one bf16 per lane into a 4-byte LDS slot
    const uint16_t *sbase;
    uint32_t soff;
    {
      const int bc = 64 * w + lane;
      const bool up = MODE == 0 && bc >= 128;
      const int c = min(c0 + (MODE == 0 ? (bc & 127) : bc), N - 1);
      sbase = (const uint16_t *)uniform_ptr((up ? sb1 : sb0) + (size_t)e * N * NG);
      soff = (uint32_t)c * (uint32_t)NG * 2u;
    }
    const uint32_t rsoff = (uint32_t)tok_lds[16 * w + (lane & 15)] * (uint32_t)A.ld_rsum * 4u;
    // one stage = half a quantization group (64 of K); stages past the end
    // load a harmless copy of the last one.  This wave's LDS destinations
    // within a stage are wave-uniform byte offsets.
    const uint32_t wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t la = FS_A + wu * 2 * 1024, lb = FS_B + wu * 2 * 1024, lc = FS_C + wu * 64,
                   ls = FS_S + wu * 256;
    auto stage = [&](int jr, int slot) {
      const int j = min(jr, NS - 1), g = j >> 1;
      const uint32_t base = ring_lds + slot * FS_BYTES;
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(abase + (size_t)j * GM_KS * 2, src_off[i], base + la + i * 1024);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma16(qbase[i] + (size_t)j * (GM_KS / 2), qoff[i], base + lb + i * 1024);
      if (lane < 16) dma4(A.rsum + g, rsoff, base + lc);
      dma2(sbase + g, soff, base + ls);
    };

    f32x4_t acc[4][4], P[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // one stage: 2 k-substeps x 4 row fragments x 4 column fragments.  Lane
    // group lg takes k = 16 lg + 8 s .. + 7 of the stage in substep s (A chunk
    // 2 lg + s, int4 word 2 lg + s).  The group's partial products P start
    // at -136 * (row sum of the group) in its first stage and are scaled into
    // the accumulators after its second.
    auto compute = [&](auto odd, int slot) {   // odd: compile-time stage parity
      const char *sp = reinterpret_cast<const char *>(ring) + slot * FS_BYTES;
      const bf16_t *al = reinterpret_cast<const bf16_t *>(sp + FS_A);
      const uint8_t *bb = reinterpret_cast<const uint8_t *>(sp + FS_B);
      const float *cb = reinterpret_cast<const float *>(sp + FS_C);
      const uint32_t *sb = reinterpret_cast<const uint32_t *>(sp + FS_S);
      __builtin_amdgcn_sched_barrier(0);
      constexpr bool first = !decltype(odd)::value;
      f32x4_t ci[4];
      if (first) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float v = -136.f * cb[16 * m + lr];
          ci[m] = f32x4_t{v, v, v, v};
        }
      }
      uint2 bq[4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        bq[nf] = *reinterpret_cast<const uint2 *>(bb + bslot[nf] * 32 + 8 * lg);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint4 bu[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const uint32_t x = s ? bq[nf].y : bq[nf].x;
          bu[nf].x = __builtin_amdgcn_bitop3_b32(x, kMask, kMagic, 0x6A);
          bu[nf].y = __builtin_amdgcn_bitop3_b32(x >> 4, kMask, kMagic, 0x6A);
          bu[nf].z = __builtin_amdgcn_bitop3_b32(x >> 8, kMask, kMagic, 0x6A);
          bu[nf].w = __builtin_amdgcn_bitop3_b32(x >> 12, kMask, kMagic, 0x6A);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = 16 * m + lr;
          const uint4 av = *reinterpret_cast<const uint4 *>(
              al + r * GM_KS + (((2 * lg + s) ^ (r & 7)) << 3));
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
            P[m][nf] = mfma32(bu[nf], av, (s == 0 && first) ? ci[m] : P[m][nf]);
        }
      }
      if (!first) {
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const uint4 sv = *reinterpret_cast<const uint4 *>(sb + oslot[nf]);
          const float sc[4] = {__uint_as_float(sv.x << 16), __uint_as_float(sv.y << 16),
                               __uint_as_float(sv.z << 16), __uint_as_float(sv.w << 16)};
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][nf][i] += sc[i] * P[m][nf][i];
        }
      }
    };

    // 3-deep pipeline: stage j computes from ring slot j % 3 while the loads
    // of stages j + 1 and j + 2 are in flight.  Per thread and stage: 2 + 2 +
    // 1 + 1 LDS-DMA (the same count in every wave), so "stage j + 1 has
    // landed" is vmcnt(6).  The loop runs in groups of six stages (three ring
    // slots, two parities); stages past the end compute nothing (uniform
    // branch) but still issue their (clamped) loads, so every wait is alike.
    constexpr int kOps = 6;
    using even_t = std::integral_constant<bool, false>;
    using odd_t = std::integral_constant<bool, true>;
    stage(0, 0);
    stage(1, 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kOps));
    block_barrier();
    for (int j = 0; j < NS; j += 6) {
#define MOE_F_STEP(JJ, PAR, CUR, NXT)            \
  {                                              \
    const int jj = (JJ);                         \
    stage(jj + 2, NXT);                          \
    if (jj < NS) compute(PAR(), CUR);            \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kOps)); \
    block_barrier();                             \
  }
      MOE_F_STEP(j, even_t, 0, 2)
      MOE_F_STEP(j + 1, odd_t, 1, 0)
      MOE_F_STEP(j + 2, even_t, 2, 1)
      MOE_F_STEP(j + 3, odd_t, 0, 2)
      MOE_F_STEP(j + 4, even_t, 1, 0)
      MOE_F_STEP(j + 5, odd_t, 2, 1)
#undef MOE_F_STEP
    }

    // ---- adapter term: acc += (lam Z) B^T, K = rank in steps of 16.  All
    // loads are unconditional (clamped indices) so that they issue together;
    // rank positions beyond r are zeroed on the B side with a bit mask.
    constexpr int NSRC = MODE == 0 ? 2 : 1;
    for (int j0 = 0; j0 < A.r; j0 += 16) {
      float zv[NSRC][4][4];
      uint16_t bl[4][4];
#pragma unroll
      for (int src = 0; src < NSRC; ++src) {
        const float *Zp = src ? A.Z1 : A.Z0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int p = p0 + min(16 * m + lr, rows - 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) zv[src][m][i] = Zp[(size_t)p * A.ldz + min(j0 + 4 * lg + i, A.r - 1)];
        }
      }
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const uint16_t *Bm = MODE == 0 && nf >= 2 ? A.B1 : A.B0;
        const size_t rowb = ((size_t)e * N + min(col[nf], N - 1)) * A.r;
#pragma unroll
        for (int i = 0; i < 4; ++i) bl[nf][i] = Bm[rowb + min(j0 + 4 * lg + i, A.r - 1)];
      }
      short4_t av[NSRC][4];
#pragma unroll
      for (int src = 0; src < NSRC; ++src)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) av[src][m][i] = (short)f2bf(A.lam * zv[src][m][i]);
      uint32_t kmask[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kmask[i] = j0 + 4 * lg + i < A.r ? 0xFFFFu : 0u;
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        short4_t bv;
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[i] = (short)(bl[nf][i] & kmask[i]);
        const int src = MODE == 0 && nf >= 2 ? 1 : 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m][nf] = mfma16(bv, av[src][m], acc[m][nf]);
      }
    }

    // ---- epilogue: lane (lr, lg) holds, for row 16 m + lr, the four
    // consecutive columns oslot[nf] .. + 3; each becomes one 8-byte store.
    __builtin_amdgcn_s_waitcnt(kWaitAll);   // trailing (clamped) stage loads
    if (MODE == 0) {
      // H = silu(G) U (and G, U when saved); the row sums of H over this
      // item's 128 columns (one quantization group of the down product) are
      // reduced over lane groups by shuffles and over waves through LDS.
      __syncthreads();                        // every wave is done with the ring
      float *red = reinterpret_cast<float *>(ring);   // [4 waves][64 rows]
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 16 * m + lr;
        const bool ok = r < rows;
        const size_t ro = (size_t)(p0 + min(r, rows - 1)) * A.ldo;
        float hs = 0.f;
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const f32x4_t g = acc[m][nf], u = acc[m][nf + 2];
          uint2 h;
          h.x = cvt_pk_bf16(silu_rcp(g[0]) * u[0], silu_rcp(g[1]) * u[1]);
          h.y = cvt_pk_bf16(silu_rcp(g[2]) * u[2], silu_rcp(g[3]) * u[3]);
          hs += (__uint_as_float(h.x << 16) + __uint_as_float(h.x & 0xFFFF0000u)) +
                (__uint_as_float(h.y << 16) + __uint_as_float(h.y & 0xFFFF0000u));
          const size_t o = ro + c0 + oslot[nf];
          if (ok) {
            *reinterpret_cast<uint2 *>(&A.out[o]) = h;
            if (A.saveG)
              *reinterpret_cast<uint2 *>(&A.saveG[o]) =
                  uint2{cvt_pk_bf16(g[0], g[1]), cvt_pk_bf16(g[2], g[3])};
            if (A.saveU)
              *reinterpret_cast<uint2 *>(&A.saveU[o]) =
                  uint2{cvt_pk_bf16(u[0], u[1]), cvt_pk_bf16(u[2], u[3])};
          }
        }
        hs += __shfl_xor(hs, 16);
        hs += __shfl_xor(hs, 32);
        if (lg == 0) red[w * 64 + r] = hs;
      }
      __syncthreads();
      if (tid < rows && A.rsum_out)
        A.rsum_out[(size_t)(p0 + tid) * A.ld_rsum_out + nt] =
            (red[tid] + red[64 + tid]) + (red[128 + tid] + red[192 + tid]);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 16 * m + lr;
        if (r < rows) {
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) {
            const int c = c0 + oslot[nf];
            if (c < N)
              *reinterpret_cast<uint2 *>(&A.out[(size_t)(p0 + r) * A.ldo + c]) =
                  uint2{cvt_pk_bf16(acc[m][nf][0], acc[m][nf][1]),
                        cvt_pk_bf16(acc[m][nf][2], acc[m][nf][3])};
          }
        }
      }
    }
  }
}

int mfma_tile_rows() { return GM_BM; }
int mfma_blocks_per_cu() { return GM_BPC; }

void launch_group_rowsum(const void *a, int rows, int K, int G, float *out, hipStream_t st) {
  size_t n = (size_t)rows * (K / G);
  group_rowsum_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>((const bf16_t *)a, rows, K, G,
                                                                   out);
}

void launch_grouped_gemm(int mode, const MfmaGemmArgs &A, int grid, hipStream_t st) {
  if (mode == 0) grouped_gemm_kernel<0><<<grid, 256, 0, st>>>(A);
  else grouped_gemm_kernel<1><<<grid, 256, 0, st>>>(A);
}

}  // namespace moe
