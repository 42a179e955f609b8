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
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

constexpr int GM_BM = 64;    // rows per tile
constexpr int GM_BPC = 2;    // resident blocks per CU
constexpr int GM_KG = 128;   // K per staged chunk = quantization group

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
template <int MODE>
__global__ __launch_bounds__(256, GM_BPC) void grouped_gemm_kernel(const MfmaGemmArgs A) {
  __shared__ __attribute__((aligned(16))) bf16_t a_lds[2][GM_BM * GM_KG];
  __shared__ __attribute__((aligned(16))) float corr_lds[2][GM_BM];
  __shared__ int tok_lds[GM_BM];

  const int K = A.K, N = A.N, NG = K / GM_KG;
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

    // ---- staging: 64 rows x 16 chunks = 1024 chunks, 4 per thread per group
    uint32_t src_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * (w * 4 + j) + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      src_off[j] = (uint32_t)tok_lds[r] * (uint32_t)(A.lda * 2) + c * 16;
    }
    const char *abase = reinterpret_cast<const char *>(A.a);
    const float *rs_row = A.rsum + (size_t)tok_lds[tid & (GM_BM - 1)] * A.ld_rsum;
    float rs_pref = tid < GM_BM ? rs_row[0] : 0.f;

    // ---- this wave's columns: 4 fragments of 16
    int col[4];
    uint32_t qoff[4], soff[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int c = MODE == 0 ? c0 + w * 32 + (nf & 1) * 16 + lr : c0 + w * 64 + nf * 16 + lr;
      col[nf] = c;
      const uint32_t row = (uint32_t)e * N + min(c, N - 1);
      qoff[nf] = row * (uint32_t)(K / 2) + lg * 16;
      soff[nf] = row * (uint32_t)NG;
    }
    const uint8_t *qb0 = A.q0, *qb1 = MODE == 0 ? A.q1 : A.q0;
    const uint16_t *sb0 = A.s0, *sb1 = MODE == 0 ? A.s1 : A.s0;

    auto stage = [&](int g, int buf) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        load_lds16(abase + src_off[j] + (size_t)g * GM_KG * 2, &a_lds[buf][(w * 4 + j) * 512]);
      if (tid < GM_BM) {
        corr_lds[buf][tid] = -136.f * rs_pref;
        if (g + 1 < NG) rs_pref = rs_row[g + 1];
      }
    };
    auto load_b = [&](int g, uint4 (&bq)[4], float (&sc)[4]) {
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const uint8_t *qb = nf >= 2 ? qb1 : qb0;
        const uint16_t *sb = nf >= 2 ? sb1 : sb0;
        bq[nf] = *reinterpret_cast<const uint4 *>(qb + qoff[nf] + (size_t)g * (GM_KG / 2));
        sc[nf] = bf2f(sb[soff[nf] + g]);
      }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[m][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 bq[4];
    float sc[4];
    stage(0, 0);
    load_b(0, bq, sc);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int g = 0; g < NG; ++g) {
      const int cur = g & 1;
      if (g + 1 < NG) stage(g + 1, cur ^ 1);
      uint4 bu[4][4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const uint32_t wd[4] = {bq[nf].x, bq[nf].y, bq[nf].z, bq[nf].w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t x = wd[s];
          bu[s][nf].x = __builtin_amdgcn_bitop3_b32(x, kMask, kMagic, 0x6A);
          bu[s][nf].y = __builtin_amdgcn_bitop3_b32(x >> 4, kMask, kMagic, 0x6A);
          bu[s][nf].z = __builtin_amdgcn_bitop3_b32(x >> 8, kMask, kMagic, 0x6A);
          bu[s][nf].w = __builtin_amdgcn_bitop3_b32(x >> 12, kMask, kMagic, 0x6A);
        }
      }
      float scg[4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) scg[nf] = sc[nf];
      if (g + 1 < NG) load_b(g + 1, bq, sc);   // registers of the unpacked words are free
      const bf16_t *al = a_lds[cur];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4_t ci = *reinterpret_cast<const f32x4_t *>(&corr_lds[cur][16 * m + 4 * lg]);
        f32x4_t P[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 av = *reinterpret_cast<const uint4 *>(
              al + (16 * m + lr) * GM_KG + (((lg * 4 + s) ^ lr) << 3));
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) P[nf] = mfma32(av, bu[s][nf], s == 0 ? ci : P[nf]);
        }
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[m][nf] += scg[nf] * P[nf];
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }

    // ---- adapter term: acc += (lam Z) B^T, K = rank in steps of 16
    for (int j0 = 0; j0 < A.r; j0 += 16) {
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const uint16_t *Bm = MODE == 0 && nf >= 2 ? A.B1 : A.B0;
        const int cc = min(col[nf], N - 1);
        short4_t bv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 4 * lg + i;
          bv[i] = j < A.r ? (short)Bm[((size_t)e * N + cc) * A.r + j] : (short)0;
        }
        const float *Zp = MODE == 0 && nf >= 2 ? A.Z1 : A.Z0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int p = p0 + min(16 * m + lr, rows - 1);
          short4_t av;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = j0 + 4 * lg + i;
            av[i] = j < A.r ? (short)f2bf(A.lam * Zp[(size_t)p * A.ldz + j]) : (short)0;
          }
          acc[m][nf] = mfma16(av, bv, acc[m][nf]);
        }
      }
    }

    // ---- epilogue through LDS (16-byte chunks XOR-swizzled per row) so that
    // every global store is a full 16-byte vector
    __syncthreads();  // all waves are done reading a_lds
    bf16_t *t0 = a_lds[0], *t1 = a_lds[1];
    auto tidx = [](int r, int c, int RW) {
      return r * RW + ((((c >> 3) ^ (r & 15))) << 3) + (c & 7);
    };
    if (MODE == 0) {
      // H -> t0, G -> t1 (64 x 128 each); then U -> t0
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * m + 4 * lg + i;
#pragma unroll
          for (int nf = 0; nf < 2; ++nf) {
            const int c = w * 32 + nf * 16 + lr;
            const float gv = acc[m][nf][i], uv = acc[m][nf + 2][i];
            t0[tidx(r, c, 128)] = f2bf(silu_f(gv) * uv);
            t1[tidx(r, c, 128)] = f2bf(gv);
          }
        }
      __syncthreads();
      // 64 rows x 16 chunks: thread -> (row, chunk); row sums of H on the way
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int idx = it * 256 + tid, r = idx >> 4, ch = idx & 15;
        const int li = r * 128 + ((ch ^ (r & 15)) << 3);
        const uint4 hv = *reinterpret_cast<const uint4 *>(&t0[li]);
        const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v += __uint_as_float(hw[q] << 16) + __uint_as_float(hw[q] & 0xFFFF0000u);
        const int c = c0 + ch * 8;
        const bool ok = r < rows && c < N;
        if (ok) {
          const size_t o = (size_t)(p0 + r) * A.ldo + c;
          *reinterpret_cast<uint4 *>(&A.out[o]) = hv;
          if (A.saveG) *reinterpret_cast<uint4 *>(&A.saveG[o]) = *reinterpret_cast<const uint4 *>(&t1[li]);
        }
        v = ok ? v : 0.f;
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        if ((lane & 15) == 0 && r < rows && A.rsum_out)
          A.rsum_out[(size_t)(p0 + r) * A.ld_rsum_out + nt] = v;
      }
      if (A.saveU) {
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * m + 4 * lg + i;
#pragma unroll
            for (int nf = 0; nf < 2; ++nf)
              t0[tidx(r, w * 32 + nf * 16 + lr, 128)] = f2bf(acc[m][nf + 2][i]);
          }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int idx = it * 256 + tid, r = idx >> 4, ch = idx & 15;
          const int c = c0 + ch * 8;
          if (r < rows && c < N)
            *reinterpret_cast<uint4 *>(&A.saveU[(size_t)(p0 + r) * A.ldo + c]) =
                *reinterpret_cast<const uint4 *>(&t0[r * 128 + ((ch ^ (r & 15)) << 3)]);
        }
      }
    } else {
      // 64 x 256 tile over both buffers (contiguous)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * m + 4 * lg + i;
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
            t0[tidx(r, w * 64 + nf * 16 + lr, 256)] = f2bf(acc[m][nf][i]);
        }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + tid, r = idx >> 5, ch = idx & 31;
        const int c = c0 + ch * 8;
        if (r < rows && c < N)
          *reinterpret_cast<uint4 *>(&A.out[(size_t)(p0 + r) * A.ldo + c]) =
              *reinterpret_cast<const uint4 *>(&t0[r * 256 + ((ch ^ (r & 15)) << 3)]);
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
