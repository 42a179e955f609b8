// C ABI of the TQP routed-expert layer: host-side validation, workspace
// carving and the kernel sequence of every call.  See include/moe_tqp.h.
#include "moe_tqp.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const std::string &msg) {
  g_last_error = msg;
  return s;
}

#define REQUIRE(cond, msg) \
  do {                     \
    if (!(cond)) return fail(MOE_ERR_INVALID, msg); \
  } while (0)

moe_status check_dims(const moe_dims *d) {
  if (!d) return fail(MOE_ERR_INVALID, "dims is NULL");
  REQUIRE(d->T >= 1, "T must be >= 1");
  REQUIRE(d->n_experts >= 1 && d->n_experts <= 1024, "n_experts must be in [1, 1024]");
  REQUIRE(d->top_k >= 1 && d->top_k <= 32 && d->top_k <= d->n_experts,
          "top_k must be in [1, min(n_experts, 32)]");
  REQUIRE(d->d_model >= 1 && d->d_model <= 65536, "d_model must be in [1, 65536]");
  REQUIRE(d->d_ff >= 1 && d->d_ff <= 65536, "d_ff must be in [1, 65536]");
  REQUIRE(d->rank >= 1 && d->rank <= 32, "rank must be in [1, 32]");
  REQUIRE((int64_t)d->T * d->top_k <= (int64_t(1) << 26), "T * top_k must be <= 2^26");
  REQUIRE(std::isfinite(d->lora_scale), "lora_scale must be finite");
  if (d->act != MOE_F32 && d->act != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "act must be MOE_F32 or MOE_BF16");
  if (d->group != 32 && d->group != 64 && d->group != 128)
    return fail(MOE_ERR_UNSUPPORTED, "group must be 32, 64 or 128");
  REQUIRE(d->d_model % d->group == 0, "d_model must be a multiple of group");
  REQUIRE(d->d_ff % d->group == 0, "d_ff must be a multiple of group");
  if (d->base_bits != 0 && d->base_bits != 4 && d->base_bits != 8)
    return fail(MOE_ERR_UNSUPPORTED, "base_bits must be 4 or 8 (0 means 4)");
  return MOE_OK;
}

// storage width of the frozen base: 4 (int4) or 8 (int8)
int base_bits(const moe_dims *d) { return d->base_bits == 8 ? 8 : 4; }
// the matrix-core path treats an int8 base as two int4 planes: twice the
// reduction of an int4 base (forward: along K; backward: along N)
int plane_mult(const moe_dims *d) { return base_bits(d) / 4; }

moe_status check_qlora(const moe_qlora &m, const char *name) {
  if (!m.q || !m.scale || !m.A || !m.B)
    return fail(MOE_ERR_INVALID, std::string(name) + ": q, scale, A and B must be non-NULL");
  // (the products stream q, A and B in 16-byte pieces)
  if ((((uintptr_t)m.q | (uintptr_t)m.A | (uintptr_t)m.B) & 15) != 0)
    return fail(MOE_ERR_INVALID, std::string(name) + ": q, A and B must be 16-byte aligned");
  if (((uintptr_t)m.qt & 15) != 0)
    return fail(MOE_ERR_INVALID, std::string(name) + ": qt must be 16-byte aligned");
  if (((uintptr_t)m.qf & 15) != 0)
    return fail(MOE_ERR_INVALID, std::string(name) + ": qf must be 16-byte aligned");
  return MOE_OK;
}

moe_status hip_status(const char *where) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
  return MOE_OK;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  }
};

size_t act_bytes(const moe_dims *d) { return d->act == MOE_BF16 ? 2 : 4; }

// ---- save buffer: Z [S][3r] f32 | G [S][f] act | U [S][f] act | H [S][f] act
// (the matrix-core path keeps the SwiGLU backward's multipliers in the G and U
// regions: U s (1 + G (1 - s)) and G s with s = sigmoid(G), rounded to bf16)
struct SaveLayout {
  size_t Z, G, U, H, total;
  explicit SaveLayout(const moe_dims *d) {
    size_t S = (size_t)d->T * d->top_k, f = d->d_ff, ab = act_bytes(d);
    Carve c;
    Z = c.take(S * 3 * d->rank * 4);
    G = c.take(S * f * ab);
    U = c.take(S * f * ab);
    H = c.take(S * f * ab);
    total = c.off;
  }
};

size_t max_tiles(const moe_dims *d, int BM) {
  return ((size_t)d->T * d->top_k + BM - 1) / BM + d->n_experts;
}

// The matrix-core path: bf16 activations, quantization group 128, d and f
// multiples of 128.  Everything else runs the float32 kernels.
bool use_mfma(const moe_dims *d) {
  return d->act == MOE_BF16 && d->group == 128 && d->d_model % 128 == 0 && d->d_ff % 128 == 0;
}

// Workspace flags of a call (the bits above the call id in
// moe_workspace_size): what the caller supplies, so that the call needs no
// room for it.
bool ws_save_given(int flags) { return (flags & MOE_WS_SAVE_GIVEN) != 0; }
bool ws_packed_given(int flags) { return (flags & MOE_WS_PACKED_GIVEN) != 0; }

// one transposed int4 matrix with its f32 scales (d x f or f x d: the same
// size; an int8 base is two such planes)
size_t qt_q_bytes(const moe_dims *d) {
  return (size_t)plane_mult(d) * d->n_experts * d->d_model * d->d_ff / 2;
}
size_t qt_slot_bytes(const moe_dims *d) {
  return qt_q_bytes(d) + (size_t)plane_mult(d) * d->n_experts * d->d_model * d->d_ff / 128 * 4;
}
size_t qf_bytes(const moe_dims *d) { return qt_slot_bytes(d); }

// The forward products of short batches (decode: a few rows per expert) run
// every expert's rows in tiles of 16 in a kernel that holds only 16 rows, so
// more of its blocks are resident and keep more weight loads in flight; from
// 128 tokens they run tiles of 128, each as the shortest class that holds its
// rows.  Either way one launch per product.
constexpr int kFwdShortBelowT = 128;
int fwd_tile_rows(const moe_dims *d) {
  return d->T < kFwdShortBelowT ? 16 : moe::mfma_tile_rows();
}

// ---- expert forward workspace
struct FwdLayout {
  size_t tiles, ntiles, save, G32, U32, tiles_m, ntiles_m, tiles_p, ntiles_p, rs_x, rs_h, rt_g,
      rt_u, rt_d, total;
  FwdLayout(const moe_dims *d, int flags) {
    size_t S = (size_t)d->T * d->top_k, f = d->d_ff, dm = d->d_model, E = d->n_experts;
    Carve c;
    tiles = c.take(max_tiles(d, moe::simple_tile_rows()) * sizeof(int2));
    ntiles = c.take(sizeof(int));
    // Z, G, U, H when the caller passes no save buffer
    save = ws_save_given(flags) ? 0 : c.take(SaveLayout(d).total);
    if (use_mfma(d)) {
      G32 = U32 = 0;
      tiles_m = c.take(max_tiles(d, fwd_tile_rows(d)) * sizeof(int2));
      // (the tile count and eight work counters for each of the two products,
      // one 128-byte line per counter)
      ntiles_m = c.take(moe::kWorkListInts * sizeof(int));
      tiles_p = c.take(max_tiles(d, moe::proj_tile_rows(d->T < kFwdShortBelowT)) * sizeof(int2));
      ntiles_p = c.take(sizeof(int));
      const size_t pm = plane_mult(d);
      rs_x = c.take((size_t)d->T * (dm / 128) * 4 * pm);
      rs_h = c.take(S * (f / 128) * 4 * pm);
      // scale ratios of the three base matrices, [E][N][K/128] f32 (the
      // forward-packed bases carry their own); an int8 base runs only from
      // its packed planes, so without the caller's they are packed here
      const bool pk = ws_packed_given(flags), i8 = base_bits(d) == 8;
      rt_g = pk ? 0 : c.take(i8 ? qf_bytes(d) : E * f * (dm / 128) * 4);
      rt_u = pk ? 0 : c.take(i8 ? qf_bytes(d) : E * f * (dm / 128) * 4);
      rt_d = pk ? 0 : c.take(i8 ? qf_bytes(d) : E * dm * (f / 128) * 4);
    } else {
      G32 = c.take(S * f * 4);
      U32 = c.take(S * f * 4);
      tiles_m = ntiles_m = tiles_p = ntiles_p = rs_x = rs_h = rt_g = rt_u = rt_d = 0;
    }
    total = c.off;
  }
};

// Persistent grids: blocks_per_cu resident blocks on every compute unit
// (rounded to a multiple of the 8 XCDs).
int persistent_grid(int blocks_per_cu = 1) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 8)
    cus = 256;
  return (cus * blocks_per_cu) & ~7;
}

// floats of two [tiles][d_ff][r] adapter-gradient partial buffers
size_t part2_floats(const moe_dims *d) {
  return 2 * max_tiles(d, moe::wgrad_tile_rows()) * (size_t)d->d_ff * d->rank;
}

// ---- adapter backward workspace
struct BwdLayout {
  size_t tiles, ntiles, tiles_m, ntiles_m, tiles_p, ntiles_p, tiles_w, ntiles_w, part, part2, bt,
      wt, wr_t, dx_r, dO, dZ, dH32, dG, dU, dXp, total;
  BwdLayout(const moe_dims *d, int flags) {
    size_t S = (size_t)d->T * d->top_k, f = d->d_ff, dm = d->d_model, ab = act_bytes(d);
    const bool mf = use_mfma(d);
    Carve c;
    tiles = c.take(max_tiles(d, moe::simple_tile_rows()) * sizeof(int2));
    ntiles = c.take(sizeof(int));
    tiles_m = mf ? c.take(max_tiles(d, moe::mfma_t_tile_rows()) * sizeof(int2)) : 0;
    // tile count, then eight work counters for each of the two products (one
    // 128-byte line per counter)
    ntiles_m = mf ? c.take(moe::kWorkListInts * sizeof(int)) : 0;
    tiles_p = mf ? c.take(max_tiles(d, moe::proj_tile_rows()) * sizeof(int2)) : 0;
    ntiles_p = mf ? c.take(sizeof(int)) : 0;
    // adapter-gradient work items and their partial sums ([tiles][2][wide][r] f32)
    tiles_w = mf ? c.take(max_tiles(d, moe::wgrad_tile_rows()) * sizeof(int2)) : 0;
    // count, first tile per expert, then the list of experts the reduction writes
    ntiles_w = mf ? c.take((2 + 2 * (size_t)d->n_experts) * sizeof(int)) : 0;
    part = mf ? c.take(max_tiles(d, moe::wgrad_tile_rows()) * 2 * std::max(dm, f) * d->rank * 4)
              : 0;
    // the partials of the gate and up dB passes, reduced together with dA_d's
    part2 = mf ? c.take(part2_floats(d) * 4) : 0;
    // B of down, gate, up transposed to [E][r][N] (bf16), for projections
    // that do not ride along the dB passes
    bt = mf ? c.take((size_t)d->n_experts * d->rank * (dm + 2 * f) * 2) : 0;
    // transposed int4 base + scales, two slots (down, then gate; up), unless
    // the caller passes every matrix transposed-packed
    wt = mf && !ws_packed_given(flags) ? c.take(2 * qt_slot_bytes(d)) : 0;
    wr_t = c.take((size_t)d->n_experts * dm * 4);
    dx_r = c.take((size_t)d->T * dm * 4);
    dO = mf ? 0 : c.take(S * dm * ab);   // the matrix-core path reads dy by token instead
    dZ = c.take(S * 3 * d->rank * 4);
    dH32 = mf ? 0 : c.take(S * f * 4);
    dG = c.take(S * f * ab);
    dU = c.take(S * f * ab);
    dXp = c.take(S * dm * (mf ? ab : 4));   // bf16 on the matrix-core path
    total = c.off;
  }
};

// call: a moe_call id, optionally OR-ed with MOE_WS_* flags
size_t ws_bytes_for(const moe_dims *d, int call) {
  const int flags = call & ~0xff;
  switch (call & 0xff) {
    case MOE_CALL_ROUTE: return moe::route_ws_bytes(d->T, d->d_model, d->n_experts);
    case MOE_CALL_PERMUTE: return moe::permute_ws_bytes(d->T, d->n_experts, d->top_k);
    case MOE_CALL_EXPERT_FWD: return FwdLayout(d, flags).total;
    case MOE_CALL_COMBINE: return 0;
    case MOE_CALL_ADAPTER_BWD: return BwdLayout(d, flags).total;
    default: return (size_t)-1;
  }
}

// the flags a call's own arguments imply
int fwd_flags(const void *save, const moe_qlora &g, const moe_qlora &u, const moe_qlora &dn) {
  return (save ? MOE_WS_SAVE_GIVEN : 0) | (g.qf && u.qf && dn.qf ? MOE_WS_PACKED_GIVEN : 0);
}
int bwd_flags(const moe_qlora &g, const moe_qlora &u, const moe_qlora &dn) {
  return g.qt && u.qt && dn.qt ? MOE_WS_PACKED_GIVEN : 0;
}

moe_status check_ws(const moe_dims *d, int call, const void *ws, size_t ws_bytes) {
  size_t need = ws_bytes_for(d, call);
  if (need && !ws) return fail(MOE_ERR_WORKSPACE, "workspace pointer is NULL");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                       " bytes, got " + std::to_string(ws_bytes));
  return MOE_OK;
}

template <typename T> T *at(void *base, size_t off) { return (T *)((char *)base + off); }

// ---- kernel timer (instrumentation)
struct KernelTimer {
  int tag = -1;
  int used = 0;
  std::vector<hipEvent_t> ev;  // pairs: start, stop
  ~KernelTimer() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};
thread_local KernelTimer g_timer;
constexpr int kTimerCap = 4096;

void timer_mark(int tag, hipStream_t st, int which) {
  KernelTimer &T = g_timer;
  if (T.tag != tag) return;
  if (which == 0 && T.used >= kTimerCap) return;
  int slot = which == 0 ? T.used : T.used - 1;
  if (which == 0) {
    if ((int)T.ev.size() < 2 * (slot + 1)) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
      T.ev.push_back(a);
      T.ev.push_back(b);
    }
    (void)hipEventRecord(T.ev[2 * slot], st);
    T.used++;
  } else if (slot >= 0) {
    (void)hipEventRecord(T.ev[2 * slot + 1], st);
  }
}

}  // namespace

// Bracket one kernel launch with the armed timer's events.
#define TIMED(tag, st, ...)      \
  do {                           \
    timer_mark(tag, st, 0);      \
    __VA_ARGS__;                 \
    timer_mark(tag, st, 1);      \
  } while (0)

#define TRY(expr)                  \
  do {                             \
    moe_status _s = (expr);        \
    if (_s != MOE_OK) return _s;   \
  } while (0)

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(int32_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_timer_start(int32_t tag) {
  if (tag < 0 || tag >= MOE_KT_COUNT) return fail(MOE_ERR_INVALID, "unknown kernel tag");
  g_timer.tag = tag;
  g_timer.used = 0;
  return MOE_OK;
}

moe_status moe_timer_stop(float *total_ms, int32_t *launches) {
  if (!total_ms || !launches) return fail(MOE_ERR_INVALID, "total_ms and launches are required");
  KernelTimer &T = g_timer;
  double sum = 0.0;
  for (int i = 0; i < T.used; ++i) {
    if (hipEventSynchronize(T.ev[2 * i + 1]) != hipSuccess)
      return fail(MOE_ERR_HIP, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, T.ev[2 * i], T.ev[2 * i + 1]) != hipSuccess)
      return fail(MOE_ERR_HIP, "hipEventElapsedTime failed");
    sum += ms;
  }
  *total_ms = (float)sum;
  *launches = T.used;
  T.tag = -1;
  T.used = 0;
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_dims *dims, int32_t call, size_t *bytes) {
  TRY(check_dims(dims));
  if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
  const int id = call & 0xff, flags = call & ~0xff;
  if (id < MOE_CALL_ROUTE || id > MOE_CALL_ADAPTER_BWD)
    return fail(MOE_ERR_INVALID, "unknown call id");
  if (flags & ~(MOE_WS_SAVE_GIVEN | MOE_WS_PACKED_GIVEN))
    return fail(MOE_ERR_INVALID, "unknown workspace flag");
  *bytes = ws_bytes_for(dims, call);
  return MOE_OK;
}

moe_status moe_save_size(const moe_dims *dims, size_t *bytes) {
  TRY(check_dims(dims));
  if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
  *bytes = SaveLayout(dims).total;
  return MOE_OK;
}

moe_status moe_route(const moe_dims *dims, const void *x, const float *w_router,
                     const float *b_router, int32_t *topk_idx, float *gates, float *logits,
                     void *ws, size_t ws_bytes, void *stream) {
  TRY(check_dims(dims));
  REQUIRE(x && w_router && topk_idx && gates, "moe_route: x, w_router, topk_idx, gates required");
  TRY(check_ws(dims, MOE_CALL_ROUTE, ws, ws_bytes));
  hipStream_t st = (hipStream_t)stream;
  int splits = 1;
  TIMED(MOE_KT_ROUTER_LOGITS, st,
        moe::launch_router_logits(dims->act == MOE_BF16, x, w_router, dims->T, dims->d_model,
                                  dims->n_experts, ws, &splits, st));
  TIMED(MOE_KT_ROUTER_TOPK, st,
        moe::launch_router_topk(ws, splits, b_router, dims->T, dims->n_experts, dims->top_k,
                                topk_idx, gates, logits, st));
  return hip_status("moe_route");
}

moe_status moe_permute(const moe_dims *dims, const int32_t *topk_idx, const void *x,
                       int32_t *counts, int32_t *offsets, int32_t *perm_src, int32_t *slot_pos,
                       void *x_perm, void *ws, size_t ws_bytes, void *stream) {
  TRY(check_dims(dims));
  REQUIRE(topk_idx && counts && offsets && perm_src && slot_pos,
          "moe_permute: topk_idx, counts, offsets, perm_src, slot_pos required");
  REQUIRE(!x_perm || x, "moe_permute: x required when x_perm is requested");
  TRY(check_ws(dims, MOE_CALL_PERMUTE, ws, ws_bytes));
  moe::launch_permute(topk_idx, dims->T, dims->n_experts, dims->top_k, counts, offsets, perm_src,
                      slot_pos, x, x_perm, (int)(dims->d_model * act_bytes(dims)), ws,
                      (hipStream_t)stream);
  return hip_status("moe_permute");
}

moe_status moe_pack_base_t_size(const moe_dims *dims, size_t *bytes) {
  TRY(check_dims(dims));
  if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
  if (!use_mfma(dims))
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_pack_base_t: only the matrix-core path (bf16, group 128, d and f "
                "multiples of 128) has a packed transposed base");
  *bytes = qt_slot_bytes(dims);
  return MOE_OK;
}

moe_status moe_pack_base_t(const moe_dims *dims, int32_t matrix, const uint8_t *q,
                           const uint16_t *scale, void *packed, size_t packed_bytes,
                           void *stream) {
  size_t need = 0;
  TRY(moe_pack_base_t_size(dims, &need));
  if (matrix != MOE_MAT_GATE_UP && matrix != MOE_MAT_DOWN)
    return fail(MOE_ERR_INVALID, "moe_pack_base_t: matrix must be MOE_MAT_GATE_UP or MOE_MAT_DOWN");
  REQUIRE(q && scale && packed, "moe_pack_base_t: q, scale and packed must be non-NULL");
  REQUIRE(((uintptr_t)packed & 15) == 0, "moe_pack_base_t: packed must be 16-byte aligned");
  if (packed_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_pack_base_t: packed buffer too small: need " +
                                       std::to_string(need) + " bytes, got " +
                                       std::to_string(packed_bytes));
  const int E = dims->n_experts, d = dims->d_model, f = dims->d_ff;
  const int R = matrix == MOE_MAT_GATE_UP ? f : d, C = matrix == MOE_MAT_GATE_UP ? d : f;
  uint8_t *qt = (uint8_t *)packed;
  float *st = reinterpret_cast<float *>(qt + qt_q_bytes(dims));
  if (base_bits(dims) == 8)
    moe::launch_transpose_q_int8(q, scale, nullptr, E, R, C, qt, st, (hipStream_t)stream);
  else
    moe::launch_transpose_q(q, scale, nullptr, E, R, C, qt, st, (hipStream_t)stream);
  return hip_status("moe_pack_base_t");
}

// the forward-packed base: int4 words [E][K/64][N][32 B], then the scale
// ratios [E][K/128][N] f32 (the same sizes for gate/up and down; an int8 base
// is packed as its two int4 planes along K, twice both sizes)
float *qf_ratios(const moe_dims *d, const void *qf) {
  return reinterpret_cast<float *>((char *)qf + qt_q_bytes(d));
}

moe_status moe_pack_base_f_size(const moe_dims *dims, size_t *bytes) {
  TRY(check_dims(dims));
  if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
  if (!use_mfma(dims))
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_pack_base_f: only the matrix-core path (bf16, group 128, d and f "
                "multiples of 128) has a packed forward base");
  *bytes = qf_bytes(dims);
  return MOE_OK;
}

moe_status moe_pack_base_f(const moe_dims *dims, int32_t matrix, const uint8_t *q,
                           const uint16_t *scale, void *packed, size_t packed_bytes,
                           void *stream) {
  size_t need = 0;
  TRY(moe_pack_base_f_size(dims, &need));
  if (matrix != MOE_MAT_GATE_UP && matrix != MOE_MAT_DOWN)
    return fail(MOE_ERR_INVALID, "moe_pack_base_f: matrix must be MOE_MAT_GATE_UP or MOE_MAT_DOWN");
  REQUIRE(q && scale && packed, "moe_pack_base_f: q, scale and packed must be non-NULL");
  REQUIRE(((uintptr_t)q & 15) == 0 && ((uintptr_t)packed & 15) == 0,
          "moe_pack_base_f: q and packed must be 16-byte aligned");
  if (packed_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_pack_base_f: packed buffer too small: need " +
                                       std::to_string(need) + " bytes, got " +
                                       std::to_string(packed_bytes));
  const uintptr_t q0 = (uintptr_t)q, p0 = (uintptr_t)packed;
  const size_t qsz = (size_t)dims->n_experts * dims->d_model * dims->d_ff * base_bits(dims) / 8;
  REQUIRE(p0 + need <= q0 || q0 + qsz <= p0, "moe_pack_base_f: packed must not overlap q");
  const int d = dims->d_model, f = dims->d_ff;
  const int N = matrix == MOE_MAT_GATE_UP ? f : d, K = matrix == MOE_MAT_GATE_UP ? d : f;
  const int E = dims->n_experts;
  const bool i8 = base_bits(dims) == 8;
  if (i8)
    moe::launch_pack_fwd_int8(q, E, N, K, (uint8_t *)packed, (hipStream_t)stream);
  else
    moe::launch_pack_fwd(q, E, N, K, (uint8_t *)packed, (hipStream_t)stream);
  moe::launch_scale_ratio(scale, E, N, K / 128, qf_ratios(dims, packed), (hipStream_t)stream, i8);
  return hip_status("moe_pack_base_f");
}

moe_status moe_adamw_step(const moe_adamw_hparams *h, int64_t n, float *master,
                          const float *grad, float *m, float *v, void *param, int32_t param_dtype,
                          void *stream) {
  REQUIRE(h, "moe_adamw_step: hparams is NULL");
  REQUIRE(n >= 0, "moe_adamw_step: n must be >= 0");
  REQUIRE(h->step >= 1, "moe_adamw_step: step must be >= 1");
  REQUIRE(std::isfinite(h->lr) && std::isfinite(h->weight_decay),
          "moe_adamw_step: lr and weight_decay must be finite");
  REQUIRE(h->beta1 >= 0.f && h->beta1 < 1.f && h->beta2 >= 0.f && h->beta2 < 1.f,
          "moe_adamw_step: beta1 and beta2 must be in [0, 1)");
  REQUIRE(std::isfinite(h->eps) && h->eps > 0.f, "moe_adamw_step: eps must be finite and > 0");
  if (param && param_dtype != MOE_F32 && param_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "moe_adamw_step: param_dtype must be MOE_F32 or MOE_BF16");
  if (n == 0) return MOE_OK;
  REQUIRE(master && grad && m && v, "moe_adamw_step: master, grad, m and v are required");
  REQUIRE((const void *)grad != master && (const void *)grad != m && (const void *)grad != v &&
              master != m && master != v && m != v,
          "moe_adamw_step: master, grad, m and v must be distinct buffers");
  moe::AdamWArgs a{};
  a.n = (size_t)n;
  a.p = master; a.g = grad; a.m = m; a.v = v; a.out = param;
  a.lr = h->lr; a.beta1 = h->beta1; a.beta2 = h->beta2; a.eps = h->eps;
  a.weight_decay = h->weight_decay;
  // bias corrections in double, once per call
  a.bc1 = (float)(1.0 - std::pow((double)h->beta1, (double)h->step));
  a.bc2 = (float)(1.0 - std::pow((double)h->beta2, (double)h->step));
  REQUIRE(a.bc1 > 0.f && a.bc2 > 0.f, "moe_adamw_step: 1 - beta^step underflows to 0");
  moe::launch_adamw(a, !param ? 0 : param_dtype == MOE_F32 ? 1 : 2, (hipStream_t)stream);
  return hip_status("moe_adamw_step");
}

moe_status moe_combine(const moe_dims *dims, const void *e_out, const int32_t *slot_pos,
                       const float *gates, void *y, void *ws, size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  TRY(check_dims(dims));
  REQUIRE(e_out && slot_pos && gates && y, "moe_combine: e_out, slot_pos, gates, y required");
  TIMED(MOE_KT_COMBINE, (hipStream_t)stream,
        moe::launch_combine(dims->act == MOE_BF16, e_out, slot_pos, gates, dims->T,
                            dims->d_model, dims->top_k, y, (hipStream_t)stream));
  return hip_status("moe_combine");
}

moe_status moe_grow_copy(const void *src, void *dst, int64_t block_bytes, int32_t n_experts,
                         int32_t factor, void *stream) {
  REQUIRE(src && dst, "moe_grow_copy: src and dst must be non-NULL");
  REQUIRE(block_bytes > 0, "moe_grow_copy: block_bytes must be positive");
  REQUIRE(n_experts >= 1 && factor >= 1 && (int64_t)n_experts * factor <= 1024,
          "moe_grow_copy: need n_experts >= 1, factor >= 1, n_experts * factor <= 1024");
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  const size_t sb = (size_t)block_bytes * n_experts, db = sb * factor;
  REQUIRE(d0 + db <= s0 || s0 + sb <= d0, "moe_grow_copy: dst must not overlap src");
  moe::launch_grow_copy(src, dst, (size_t)block_bytes, n_experts, factor, (hipStream_t)stream);
  return hip_status("moe_grow_copy");
}

moe_status moe_grow_router(int32_t d, int32_t n_experts, int32_t factor, const float *w_router,
                           const float *b_router, const float *noise, float noise_scale,
                           float *w_out, float *b_out, void *stream) {
  REQUIRE(w_router && w_out, "moe_grow_router: w_router and w_out must be non-NULL");
  REQUIRE(!b_router || b_out, "moe_grow_router: b_out is required with b_router");
  REQUIRE(d >= 1 && d <= 65536, "moe_grow_router: d must be in [1, 65536]");
  REQUIRE(n_experts >= 1 && factor >= 1 && (int64_t)n_experts * factor <= 1024,
          "moe_grow_router: need n_experts >= 1, factor >= 1, n_experts * factor <= 1024");
  REQUIRE(std::isfinite(noise_scale), "moe_grow_router: noise_scale must be finite");
  moe::launch_grow_router(w_router, b_router, noise, noise_scale, d, n_experts, factor, w_out,
                          b_out, (hipStream_t)stream);
  return hip_status("moe_grow_router");
}

moe_status moe_rev_couple(const moe_dims *dims, const void *x, const void *m, void *out,
                          int32_t sign, void *stream) {
  TRY(check_dims(dims));
  REQUIRE(x && m && out, "moe_rev_couple: x, m and out must be non-NULL");
  REQUIRE(sign == 1 || sign == -1, "moe_rev_couple: sign must be +1 or -1");
  REQUIRE(out != m, "moe_rev_couple: out must not alias m");
  moe::launch_rev_couple(dims->act == MOE_BF16, x, m, out, (size_t)dims->T * dims->d_model,
                         (float)sign, (hipStream_t)stream);
  return hip_status("moe_rev_couple");
}

}  // extern "C"

namespace {

moe_status check_expert_fwd(const moe_dims *dims, const void *x, const int32_t *offsets,
                            const int32_t *perm_src, const moe_qlora &gate, const moe_qlora &up,
                            const moe_qlora &down, const void *e_out, const void *save) {
  TRY(check_dims(dims));
  REQUIRE(x && offsets && perm_src && e_out, "moe_expert_fwd: x, offsets, perm_src, e_out required");
  REQUIRE((((uintptr_t)x | (uintptr_t)e_out | (uintptr_t)save) & 15) == 0,
          "moe_expert_fwd: x, e_out and save must be 16-byte aligned");
  TRY(check_qlora(gate, "gate"));
  TRY(check_qlora(up, "up"));
  TRY(check_qlora(down, "down"));
  return MOE_OK;
}

// The kernel sequence of moe_expert_fwd on a validated call; ws holds at
// least FwdLayout(dims, fwd_flags(...)).total bytes.
moe_status expert_fwd_run(const moe_dims *dims, const void *x, const int32_t *offsets,
                          const int32_t *perm_src, moe_qlora gate, moe_qlora up, moe_qlora down,
                          void *e_out, void *save, void *ws, void *stream) {
  hipStream_t st = (hipStream_t)stream;
  const bool bf = dims->act == MOE_BF16;
  const int T = dims->T, d = dims->d_model, E = dims->n_experts, k = dims->top_k, f = dims->d_ff,
            r = dims->rank, g = dims->group;
  const size_t S = (size_t)T * k;
  const float lam = dims->lora_scale;
  FwdLayout L(dims, fwd_flags(save, gate, up, down));
  void *sv = save ? save : at<char>(ws, L.save);
  SaveLayout SL(dims);
  float *Z = at<float>(sv, SL.Z);
  void *Gs = at<char>(sv, SL.G), *Us = at<char>(sv, SL.U), *H = at<char>(sv, SL.H);
  int2 *tiles = at<int2>(ws, L.tiles);
  int *ntiles = at<int>(ws, L.ntiles);
  const int BM = moe::simple_tile_rows();
  const int mt = (int)max_tiles(dims, BM);
  // (the float32 kernels' tile list; the matrix-core path builds its own)
  if (!use_mfma(dims)) moe::launch_build_tiles(offsets, E, BM, tiles, ntiles, st);

  moe::ProjArgs P{};
  P.a = x; P.lda = d; P.gather = true; P.perm_src = perm_src; P.kk = k;
  P.tiles = tiles; P.ntiles = ntiles; P.max_tiles = mt; P.offsets = offsets;
  P.m_es = (size_t)r * d; P.m_cs = 1; P.m_js = d; P.K = d; P.r = r; P.s = 1.f; P.ldz = 3 * r;

  if (use_mfma(dims)) {
    const bool short_t = T < kFwdShortBelowT;
    int2 *tiles_m = at<int2>(ws, L.tiles_m), *tiles_p = at<int2>(ws, L.tiles_p);
    const int mtp = (int)max_tiles(dims, moe::proj_tile_rows(short_t));
    int *ntiles_m = at<int>(ws, L.ntiles_m), *ntiles_p = at<int>(ws, L.ntiles_p);
    float *rs_x = at<float>(ws, L.rs_x), *rs_h = at<float>(ws, L.rs_h);
    float *rt_g = at<float>(ws, L.rt_g), *rt_u = at<float>(ws, L.rt_u), *rt_d = at<float>(ws, L.rt_d);
    // An int8 base runs as its two int4 planes along K (packed here unless the
    // caller packed it): twice the reduction, the rows read twice, and start
    // values -136 (first plane) and -128 (second) times the group sums.
    const bool i8 = base_bits(dims) == 8;
    const int pm = plane_mult(dims);
    // set-up in one launch: the products' tile list (zeroing their work
    // counters), the projections' tile list, and the per-row start values
    // -136 * (row sum per group)
    moe::PrepBatch pb;
    pb.tiles(offsets, E, fwd_tile_rows(dims), tiles_m, ntiles_m, nullptr, moe::kWorkListInts);
    pb.tiles(offsets, E, moe::proj_tile_rows(short_t), tiles_p, ntiles_p);
    pb.rowsum(x, T, d, 128, -136.f, rs_x, i8, -128.f);
    moe::launch_prep(pb, st);
    const void *qf_g = gate.qf, *qf_u = up.qf, *qf_d = down.qf;
    if (i8) {
      auto pack = [&](const moe_qlora &m, int N, int K, float *buf) {
        moe::launch_pack_fwd_int8(m.q, E, N, K, (uint8_t *)buf, st);
        moe::launch_scale_ratio(m.scale, E, N, K / 128, qf_ratios(dims, buf), st, true);
        return (const void *)buf;
      };
      if (!qf_g) qf_g = pack(gate, f, d, rt_g);
      if (!qf_u) qf_u = pack(up, f, d, rt_u);
      if (!qf_d) qf_d = pack(down, d, f, rt_d);
    }
    // (the packed bases carry their ratio tables)
    const bool pk_gu = qf_g && qf_u;
    if (pk_gu) {
      rt_g = qf_ratios(dims, qf_g);
      rt_u = qf_ratios(dims, qf_u);
    } else {
      moe::launch_scale_ratio(gate.scale, E, f, d / 128, rt_g, st);
      moe::launch_scale_ratio(up.scale, E, f, d / 128, rt_u, st);
    }
    if (qf_d)
      rt_d = qf_ratios(dims, qf_d);
    else
      moe::launch_scale_ratio(down.scale, E, d, f / 128, rt_d, st);
    // Z_g = X A_g^T, Z_u = X A_u^T (rows gathered from x)
    moe::ProjMArgs Q{};
    Q.a = (const uint16_t *)x; Q.lda = d; Q.perm_src = perm_src; Q.kk = k;
    Q.tiles = tiles_p; Q.ntiles = ntiles_p; Q.offsets = offsets; Q.K = d; Q.r = r; Q.nsrc = 2;
    Q.m0 = (const uint16_t *)gate.A; Q.m1 = (const uint16_t *)up.A; Q.scale = 1.f;
    Q.Z0 = Z; Q.Z1 = Z + r; Q.ldz = 3 * r;
    moe::launch_proj_mfma(Q, mtp, true, st, short_t);
    const int grid = persistent_grid(moe::mfma_blocks_per_cu());
    moe::MfmaGemmArgs M{};
    M.a = x; M.lda = d; M.perm_src = perm_src; M.kk = k; M.rsum = rs_x; M.ld_rsum = d / 128 * pm;
    M.tiles = tiles_m; M.offsets = offsets;
    M.K = d * pm; M.ka = d; M.N = f; M.NT = (f + 127) / 128;
    // the stage-major packed base where both matrices have one (an int8 base
    // has no plain int4 layout)
    M.q0 = i8 ? nullptr : gate.q; M.rt0 = rt_g; M.B0 = (const uint16_t *)gate.B;
    M.q1 = i8 ? nullptr : up.q; M.rt1 = rt_u; M.B1 = (const uint16_t *)up.B;
    M.qp0 = pk_gu ? (const uint8_t *)qf_g : nullptr;
    M.qp1 = pk_gu ? (const uint8_t *)qf_u : nullptr;
    M.Z0 = Z; M.Z1 = Z + r; M.ldz = 3 * r; M.r = r; M.lam = lam;
    M.out = (uint16_t *)H; M.ldo = f;
    M.saveG = save ? (uint16_t *)Gs : nullptr;
    M.saveU = save ? (uint16_t *)Us : nullptr;
    M.rsum_out = rs_h; M.ld_rsum_out = f / 128 * pm; M.rsum_split = i8;
    TIMED(MOE_KT_GATEUP, st, {
      if (short_t) moe::launch_grouped_gemm_short(0, M, ntiles_m, grid, st);
      else moe::launch_grouped_gemm(0, M, ntiles_m, ntiles_m + moe::kCtrSet0, grid, st);
    });
    // Z_d = H A_d^T
    Q.a = (const uint16_t *)H; Q.lda = f; Q.K = f; Q.nsrc = 1; Q.m0 = (const uint16_t *)down.A;
    Q.m1 = nullptr; Q.Z0 = Z + 2 * r; Q.Z1 = nullptr;
    moe::launch_proj_mfma(Q, mtp, false, st, short_t);
    moe::MfmaGemmArgs D{};
    D.a = H; D.lda = f; D.rsum = rs_h; D.ld_rsum = f / 128 * pm;
    D.tiles = tiles_m; D.offsets = offsets;
    D.K = f * pm; D.ka = f; D.N = d; D.NT = (d + 255) / 256;
    D.q0 = i8 ? nullptr : down.q; D.rt0 = rt_d; D.B0 = (const uint16_t *)down.B;
    D.qp0 = (const uint8_t *)qf_d;
    D.Z0 = Z + 2 * r; D.ldz = 3 * r; D.r = r; D.lam = lam;
    D.out = (uint16_t *)e_out; D.ldo = d;
    TIMED(MOE_KT_DOWN, st, {
      if (short_t) moe::launch_grouped_gemm_short(1, D, ntiles_m, grid, st);
      else moe::launch_grouped_gemm(1, D, ntiles_m, ntiles_m + moe::kCtrSet1, grid, st);
    });
    return hip_status("moe_expert_fwd");
  }

  // Z_g = X A_g^T, Z_u = X A_u^T (rows gathered from x)
  P.m = gate.A; P.Z = Z;
  moe::launch_proj_simple(bf, P, st);
  P.m = up.A; P.Z = Z + r;
  moe::launch_proj_simple(bf, P, st);

  // G, U in float32, then SwiGLU
  float *G32 = at<float>(ws, L.G32), *U32 = at<float>(ws, L.U32);
  moe::LinArgs A{};
  A.a = x; A.lda = d; A.gather = true; A.perm_src = perm_src; A.kk = k;
  A.tiles = tiles; A.ntiles = ntiles; A.max_tiles = mt; A.offsets = offsets;
  A.N = f; A.K = d; A.g = g; A.trans = false; A.bits = base_bits(dims); A.ldz = 3 * r;
  A.l_es = (size_t)f * r; A.l_js = 1; A.l_ns = r; A.r = r; A.lam = lam; A.ldo = f;
  A.acc_out = false;
  A.q = gate.q; A.scale = gate.scale; A.Z = Z; A.lmat = gate.B; A.out = G32;
  TIMED(MOE_KT_GATEUP, st, moe::launch_lin_simple(bf, true, A, st));
  A.q = up.q; A.scale = up.scale; A.Z = Z + r; A.lmat = up.B; A.out = U32;
  TIMED(MOE_KT_GATEUP, st, moe::launch_lin_simple(bf, true, A, st));
  moe::launch_swiglu_fwd(bf, G32, U32, S * f, H, Gs, Us, st);

  // Z_d = H A_d, then O = H W_d^T + lam Z_d B_d
  P.a = H; P.lda = f; P.gather = false; P.m = down.A; P.m_es = (size_t)r * f; P.m_cs = 1;
  P.m_js = f; P.K = f; P.Z = Z + 2 * r;
  moe::launch_proj_simple(bf, P, st);
  A.a = H; A.lda = f; A.gather = false; A.N = d; A.K = f; A.q = down.q; A.scale = down.scale;
  A.Z = Z + 2 * r; A.lmat = down.B; A.l_es = (size_t)d * r; A.l_js = 1; A.l_ns = r;
  A.out = e_out; A.ldo = d;
  TIMED(MOE_KT_DOWN, st, moe::launch_lin_simple(bf, false, A, st));
  return hip_status("moe_expert_fwd");
}

}  // namespace

extern "C" {

moe_status moe_expert_fwd(const moe_dims *dims, const void *x, const int32_t *offsets,
                          const int32_t *perm_src, moe_qlora gate, moe_qlora up, moe_qlora down,
                          void *e_out, void *save, void *ws, size_t ws_bytes, void *stream) {
  TRY(check_expert_fwd(dims, x, offsets, perm_src, gate, up, down, e_out, save));
  TRY(check_ws(dims, MOE_CALL_EXPERT_FWD | fwd_flags(save, gate, up, down), ws, ws_bytes));
  return expert_fwd_run(dims, x, offsets, perm_src, gate, up, down, e_out, save, ws, stream);
}

moe_status moe_expert_fwd_noalloc(const moe_dims *dims, const void *x, const int32_t *offsets,
                                  const int32_t *perm_src, moe_qlora gate, moe_qlora up,
                                  moe_qlora down, void *e_out, void *save, void *stream) {
  TRY(check_expert_fwd(dims, x, offsets, perm_src, gate, up, down, e_out, save));
  const size_t need = ws_bytes_for(dims, MOE_CALL_EXPERT_FWD | fwd_flags(save, gate, up, down));
  if (need > moe::kStaticScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_expert_fwd_noalloc: this call needs " + std::to_string(need) +
                    " bytes of scratch, more than the fixed " +
                    std::to_string(moe::kStaticScratchBytes) +
                    " bytes (pass save and the packed bases, or call moe_expert_fwd with a "
                    "workspace)");
  void *ws = nullptr;
  const hipError_t e = moe::static_scratch(&ws);
  if (e != hipSuccess)
    return fail(MOE_ERR_HIP, std::string("moe_expert_fwd_noalloc: hipGetSymbolAddress: ") +
                                 hipGetErrorString(e));
  return expert_fwd_run(dims, x, offsets, perm_src, gate, up, down, e_out, save, ws, stream);
}

moe_status moe_adapter_bwd(const moe_dims *dims, const void *dy, const void *x,
                           const int32_t *topk_idx, const float *gates, const int32_t *offsets,
                           const int32_t *perm_src, const int32_t *slot_pos,
                           const float *w_router, moe_qlora gate, moe_qlora up, moe_qlora down,
                           const void *e_out, const void *save, void *dx, float *dA_gate,
                           float *dB_gate, float *dA_up, float *dB_up, float *dA_down,
                           float *dB_down, void *ws, size_t ws_bytes, void *stream) {
  TRY(check_dims(dims));
  REQUIRE(dy && x && topk_idx && gates && offsets && perm_src && slot_pos && w_router && e_out &&
              save && dx,
          "moe_adapter_bwd: every tensor argument is required");
  REQUIRE(dA_gate && dB_gate && dA_up && dB_up && dA_down && dB_down,
          "moe_adapter_bwd: all six adapter-gradient outputs are required");
  TRY(check_qlora(gate, "gate"));
  TRY(check_qlora(up, "up"));
  TRY(check_qlora(down, "down"));
  TRY(check_ws(dims, MOE_CALL_ADAPTER_BWD | bwd_flags(gate, up, down), ws, ws_bytes));
  hipStream_t st = (hipStream_t)stream;
  const bool bf = dims->act == MOE_BF16;
  const int T = dims->T, d = dims->d_model, E = dims->n_experts, k = dims->top_k, f = dims->d_ff,
            r = dims->rank, g = dims->group;
  const size_t S = (size_t)T * k;
  const float lam = dims->lora_scale;
  BwdLayout L(dims, bwd_flags(gate, up, down));
  SaveLayout SL(dims);
  const float *Z = at<const float>((void *)save, SL.Z);
  const void *Gs = at<const char>((void *)save, SL.G), *Us = at<const char>((void *)save, SL.U),
             *H = at<const char>((void *)save, SL.H);
  int2 *tiles = at<int2>(ws, L.tiles);
  int *ntiles = at<int>(ws, L.ntiles);
  float *wr_t = at<float>(ws, L.wr_t), *dx_r = at<float>(ws, L.dx_r);
  // dO = gamma * dy in permuted order: materialised only for the float32
  // kernels (the matrix-core path reads dy by token and applies the gates)
  void *dO = use_mfma(dims) ? nullptr : at<char>(ws, L.dO);
  float *dZ = at<float>(ws, L.dZ);
  void *dXp = at<char>(ws, L.dXp);
  void *dG = at<char>(ws, L.dG), *dU = at<char>(ws, L.dU);

  // gate path: W_r^T for the router-input gradient; the float32 kernels also
  // take dO from this pass, the matrix-core path runs it last (below)
  if (!use_mfma(dims)) {
    moe::launch_transpose_f32(w_router, d, E, wr_t, st);
    TIMED(MOE_KT_GATE_GRAD, st,
          moe::launch_gate_grad(bf, dy, e_out, topk_idx, gates, slot_pos, wr_t, T, d, k, E, dx_r,
                                dO, st));
  }

  if (use_mfma(dims)) {
    int2 *tiles_m = at<int2>(ws, L.tiles_m), *tiles_p = at<int2>(ws, L.tiles_p);
    int *ntiles_m = at<int>(ws, L.ntiles_m), *ntiles_p = at<int>(ws, L.ntiles_p);
    int2 *tiles_w = at<int2>(ws, L.tiles_w);
    int *ntiles_w = at<int>(ws, L.ntiles_w);
    const int grid = persistent_grid(moe::mfma_t_blocks_per_cu());
    const int mtp = (int)max_tiles(dims, moe::proj_tile_rows());
    const int mtw = (int)max_tiles(dims, moe::wgrad_tile_rows());
    uint16_t *bt_d = at<uint16_t>(ws, L.bt);
    uint16_t *bt_g = bt_d + (size_t)E * r * d, *bt_u = bt_g + (size_t)E * r * f;
    // The projections dZ = lam dO B ride along the dB reductions (rank 16,
    // 256-column ranges, partials in the dX_perm buffer) and read B as
    // stored; otherwise they run on their own over B as [E][r][N].
    const size_t dxp_bytes = (size_t)S * d * 2;
    const size_t zq = (size_t)(f / 256) * S * 16;   // floats of one matrix's partials
    // (B is read there in 16-byte pieces)
    const bool fuse_d = r == 16 && d % 256 == 0 && (size_t)(d / 256) * S * 64 <= dxp_bytes &&
                        ((uintptr_t)down.B & 15) == 0;
    const bool fuse_gu = r == 16 && f % 256 == 0 && 2 * zq * 4 <= dxp_bytes &&
                         (((uintptr_t)gate.B | (uintptr_t)up.B) & 15) == 0;
    // set-up in one launch: W_r^T; the tile lists of the input-gradient
    // products (zeroing their work counters), of the projections and of the
    // adapter-gradient reductions (with the experts they split); B of each
    // matrix as [E][r][N] where its projection runs on its own
    moe::PrepBatch pb;
    pb.transpose_f32(w_router, d, E, wr_t);
    pb.tiles(offsets, E, moe::mfma_t_tile_rows(), tiles_m, ntiles_m, nullptr, moe::kWorkListInts);
    pb.tiles(offsets, E, moe::proj_tile_rows(), tiles_p, ntiles_p);
    pb.tiles(offsets, E, moe::wgrad_tile_rows(), tiles_w, ntiles_w, ntiles_w + 1);
    if (!fuse_d) pb.transpose_nr(down.B, E, d, r, bt_d, st);
    if (!fuse_gu) {
      pb.transpose_nr(gate.B, E, f, r, bt_g, st);
      pb.transpose_nr(up.B, E, f, r, bt_u, st);
    }
    moe::launch_prep(pb, st);
    // An int8 base runs as its two int4 planes stacked along N: twice the
    // reduction, the rows read twice (transposed here unless the caller packed it)
    const bool i8 = base_bits(dims) == 8;
    const int pm = plane_mult(dims);
    auto transpose = [&](const moe_qlora &m, int R, int C, uint8_t *qt, float *stt) {
      if (i8) moe::launch_transpose_q_int8(m.q, m.scale, offsets, E, R, C, qt, stt, st);
      else moe::launch_transpose_q(m.q, m.scale, offsets, E, R, C, qt, stt, st);
    };
    const size_t qsz = qt_q_bytes(dims), slot = qt_slot_bytes(dims);
    uint8_t *qt0 = at<uint8_t>(ws, L.wt), *qt1 = qt0 + slot;
    float *st0 = reinterpret_cast<float *>(qt0 + qsz), *st1 = reinterpret_cast<float *>(qt1 + qsz);
    const uint16_t *H16 = (const uint16_t *)H;

    // The projections dZ = lam dOut B ride along the passes that form dB over
    // the same rows (rank 16, widths multiples of 256): each writes per
    // 256-column partials, which launch_lowrank_reduce adds (together with
    // the adapter-gradient partials of the passes before it).  The dZ
    // partials live in the dX_perm buffer, which is written only at the end.
    float *zpart = reinterpret_cast<float *>(dXp);
    moe::ProjMArgs Q{};
    Q.perm_src = perm_src; Q.kk = k; Q.tiles = tiles_p; Q.ntiles = ntiles_p; Q.offsets = offsets;
    Q.r = r; Q.nsrc = 1; Q.scale = lam; Q.ldz = 3 * r;
    moe::WgradMArgs W{};
    W.perm_src = perm_src; W.kk = k; W.offsets = offsets; W.E = E; W.r = r; W.nsrc = 1;
    W.tiles = tiles_w; W.ntiles = ntiles_w; W.tfirst = ntiles_w + 1; W.multi = ntiles_w + 1 + E;
    W.part = at<float>(ws, L.part);
    W.S = (int)S;
    // dB_d [d][r] = lam sum_p dO[p][n] Z_d[p][j] (= lam sum_p dy[t(p)][n] g_p Z_d[p][j])
    // and dZ_d = lam dO B_d = lam g_p (dy[t(p)] B_d)
    W.w = (const uint16_t *)dy; W.ldw = d; W.rr = Z + 2 * r; W.ldr = 3 * r; W.wide = d;
    W.gsc = gates;
    W.scale = lam; W.out = dB_down; W.oe = (size_t)d * r; W.oa = r; W.ob = 1;
    if (fuse_d) {
      W.pm = (const uint16_t *)down.B; W.zpart = zpart;
      moe::launch_wgrad_mfma(W, mtw, true, st, false);
      const moe::ZpartJob zj{zpart, nullptr, d / 256, (int)S, perm_src, gates, lam, dZ + 2 * r,
                             nullptr, 3 * r};
      moe::launch_lowrank_reduce(&W, 1, &zj, st);
    } else {
      Q.a = (const uint16_t *)dy; Q.lda = d; Q.gsc = gates; Q.K = d; Q.m0 = bt_d;
      Q.Z0 = dZ + 2 * r;
      moe::launch_proj_mfma(Q, mtp, true, st);
      moe::launch_wgrad_mfma(W, mtw, true, st);
    }
    W.gsc = nullptr; W.pm = nullptr; W.zpart = nullptr;
    Q.gsc = nullptr;
    // dH = dO W_d + dZ_d A_d with the SwiGLU backward in the epilogue
    moe::MfmaGemmTArgs M{};
    M.a0 = dy; M.lda = d; M.perm_src = perm_src; M.kk = k; M.gsc = gates;
    M.tiles = tiles_m; M.offsets = offsets;
    // the transposed base: the caller's packing, else this call's own
    const uint8_t *qd = qt0;
    const float *sd = st0;
    if (down.qt) {
      qd = (const uint8_t *)down.qt;
      sd = reinterpret_cast<const float *>(qd + qsz);
    } else {
      transpose(down, d, f, qt0, st0);
    }
    M.K = d * pm; M.kr = d; M.N = f; M.NT = (f + 255) / 256; M.qt0 = qd; M.st0 = sd;
    M.Z0 = dZ + 2 * r; M.ldz = 3 * r; M.r = r; M.L0 = (const uint16_t *)down.A;
    M.G = (const uint16_t *)Gs; M.U = (const uint16_t *)Us;
    M.dG = (uint16_t *)dG; M.dU = (uint16_t *)dU;
    // the gate gradient's dots <dy, e_out[p]> come from this product: per row
    // and 128 columns, dH . H = g_p times their share (in the router-gradient
    // buffer, which the per-token pass leaves unused)
    const int nq = 2 * ((f + 255) / 256);
    float *dgp = moe::token_bwd_covers(d, k) && (size_t)nq * S <= (size_t)T * d ? dx_r : nullptr;
    M.H = H16; M.dgp = dgp; M.S = (int)S;
    TIMED(MOE_KT_BWD_DOWN, st, moe::launch_grouped_gemm_t(0, M, ntiles_m, ntiles_m + moe::kCtrSet0, grid, st));
    // dA_d [r][f] = sum_p dZ_d[p][j] H[p][c]
    moe::WgradMArgs Wd = W;
    Wd.w = H16; Wd.ldw = f; Wd.rr = dZ + 2 * r; Wd.wide = f; Wd.scale = 1.f; Wd.out = dA_down;
    Wd.oe = (size_t)r * f; Wd.oa = 1; Wd.ob = f;
    // dB [f][r] = lam sum_p dG[p][n] Z[p][j] and dZ_g = lam dG B_g (up: dU, Z_u, B_u)
    W.w = (const uint16_t *)dG; W.ldw = f; W.rr = Z; W.wide = f; W.scale = lam; W.out = dB_gate;
    W.oe = (size_t)f * r; W.oa = r; W.ob = 1;
    if (fuse_gu) {
      // dA_d, dB_g and dB_u keep their partials apart (dA_d in the shared
      // buffer, dB_g and dB_u in their own), reduced in one launch with dZ
      moe::launch_wgrad_mfma(Wd, mtw, false, st, false);
      moe::WgradMArgs Wg = W, Wu = W;
      Wg.pm = (const uint16_t *)gate.B; Wg.zpart = zpart; Wg.part = at<float>(ws, L.part2);
      Wu.w = (const uint16_t *)dU; Wu.rr = Z + r; Wu.out = dB_up; Wu.pm = (const uint16_t *)up.B;
      Wu.zpart = zpart + zq; Wu.part = Wg.part + part2_floats(dims) / 2;
      moe::launch_wgrad_mfma(Wg, mtw, false, st, false);
      moe::launch_wgrad_mfma(Wu, mtw, false, st, false);
      const moe::WgradMArgs three[3] = {Wd, Wg, Wu};
      const moe::ZpartJob zj{zpart, zpart + zq, f / 256, (int)S, nullptr, nullptr, lam, dZ,
                             dZ + r, 3 * r};
      moe::launch_lowrank_reduce(three, 3, &zj, st);
    } else {
      moe::launch_wgrad_mfma(Wd, mtw, false, st);
      Q.a = (const uint16_t *)dG; Q.lda = f; Q.K = f; Q.m0 = bt_g; Q.Z0 = dZ;
      moe::launch_proj_mfma(Q, mtp, false, st);
      Q.a = (const uint16_t *)dU; Q.m0 = bt_u; Q.Z0 = dZ + r;
      moe::launch_proj_mfma(Q, mtp, false, st);
      moe::launch_wgrad_mfma(W, mtw, false, st);
      W.w = (const uint16_t *)dU; W.rr = Z + r; W.out = dB_up;
      moe::launch_wgrad_mfma(W, mtw, false, st);
    }
    // dA [r][d] = sum_p dZ[p][j] X[token(p)][c], gate and up in one pass over X
    W.w = (const uint16_t *)x; W.ldw = d; W.rr = dZ; W.wide = d; W.scale = 1.f; W.out = dA_gate;
    W.oe = (size_t)r * d; W.oa = 1; W.ob = d;
    W.nsrc = 2; W.rr1 = dZ + r; W.out1 = dA_up;
    moe::launch_wgrad_mfma(W, mtw, true, st);
    // dX_perm = dG W_g + dZ_g A_g + dU W_u + dZ_u A_u
    moe::MfmaGemmTArgs X{};
    X.a0 = dG; X.a1 = dU; X.lda = f; X.tiles = tiles_m;
    X.offsets = offsets; X.K = f * pm; X.kr = f; X.N = d; X.NT = (d + 255) / 256;
    X.qt0 = qt0; X.st0 = st0; X.qt1 = qt1; X.st1 = st1;
    if (gate.qt) {
      X.qt0 = (const uint8_t *)gate.qt;
      X.st0 = reinterpret_cast<const float *>(X.qt0 + qsz);
    } else {
      transpose(gate, f, d, qt0, st0);
    }
    if (up.qt) {
      X.qt1 = (const uint8_t *)up.qt;
      X.st1 = reinterpret_cast<const float *>(X.qt1 + qsz);
    } else {
      transpose(up, f, d, qt1, st1);
    }
    X.Z0 = dZ; X.Z1 = dZ + r; X.ldz = 3 * r; X.r = r;
    X.L0 = (const uint16_t *)gate.A; X.L1 = (const uint16_t *)up.A;
    X.out = (uint16_t *)dXp; X.ldo = d;
    TIMED(MOE_KT_BWD_GATEUP, st, moe::launch_grouped_gemm_t(1, X, ntiles_m, ntiles_m + moe::kCtrSet1, grid, st));
    // gate gradient and the per-token sum of dX_perm, one pass per token
    TIMED(MOE_KT_GATE_GRAD, st, {
      if (!moe::launch_token_bwd(dy, e_out, topk_idx, gates, slot_pos, wr_t, dXp, T, d, k, E, dx,
                                 st, dgp, nq)) {
        moe::launch_gate_grad(bf, dy, e_out, topk_idx, gates, slot_pos, wr_t, T, d, k, E, dx_r,
                              nullptr, st);
        moe::launch_unpermute_sum(bf, false, dx_r, dXp, slot_pos, T, d, k, dx, st);
      }
    });
    return hip_status("moe_adapter_bwd");
  }

  // ---- float32 kernels
  float *dH32 = at<float>(ws, L.dH32);
  const int BM = moe::simple_tile_rows();
  const int mt = (int)max_tiles(dims, BM);
  moe::launch_build_tiles(offsets, E, BM, tiles, ntiles, st);
  // down: dZ_d = lam dO B_d; dB_d = lam dO^T Z_d; dH = dO W_d + dZ_d A_d
  moe::ProjArgs P{};
  P.a = dO; P.lda = d; P.gather = false; P.perm_src = perm_src; P.kk = k;
  P.tiles = tiles; P.ntiles = ntiles; P.max_tiles = mt; P.offsets = offsets;
  P.m = down.B; P.m_es = (size_t)d * r; P.m_cs = r; P.m_js = 1; P.K = d; P.r = r; P.s = lam;
  P.Z = dZ + 2 * r; P.ldz = 3 * r;
  moe::launch_proj_simple(bf, P, st);
  moe::WgradArgs W{};
  W.perm_src = perm_src; W.kk = k; W.offsets = offsets; W.E = E;
  // dB_d [d][r] = lam * sum_p dO[p][n] Z_d[p][j]
  W.l = dO; W.ldl = d; W.l_f32 = false; W.gather = false;
  W.r = Z + 2 * r; W.ldr = 3 * r; W.Aw = d; W.Bw = r; W.s = lam; W.out = dB_down;
  moe::launch_wgrad_simple(bf, W, st);
  moe::LinArgs A{};
  A.a = dO; A.lda = d; A.gather = false; A.perm_src = perm_src; A.kk = k;
  A.tiles = tiles; A.ntiles = ntiles; A.max_tiles = mt; A.offsets = offsets;
  A.q = down.q; A.scale = down.scale; A.N = f; A.K = d; A.g = g; A.trans = true;
  A.bits = base_bits(dims);
  A.Z = dZ + 2 * r; A.ldz = 3 * r; A.lmat = down.A; A.l_es = (size_t)r * f; A.l_js = f;
  A.l_ns = 1; A.r = r; A.lam = 1.f; A.out = dH32; A.ldo = f; A.acc_out = false;
  TIMED(MOE_KT_BWD_DOWN, st, moe::launch_lin_simple(bf, true, A, st));
  moe::launch_swiglu_bwd(bf, dH32, Gs, Us, S * f, dG, dU, st);
  // dA_d [r][f] = sum_p dZ_d[p][j] H[p][c]
  W.l = dZ + 2 * r; W.ldl = 3 * r; W.l_f32 = true; W.r = H; W.ldr = f; W.Aw = r; W.Bw = f;
  W.s = 1.f; W.out = dA_down;
  moe::launch_wgrad_simple(bf, W, st);
  // gate / up: dZ = lam dG B; dB = lam dG^T Z; dA = dZ^T X
  P.m_es = (size_t)f * r; P.m_cs = r; P.m_js = 1; P.K = f; P.lda = f;
  P.a = dG; P.m = gate.B; P.Z = dZ;
  moe::launch_proj_simple(bf, P, st);
  P.a = dU; P.m = up.B; P.Z = dZ + r;
  moe::launch_proj_simple(bf, P, st);
  // dB [f][r] = lam * sum_p dG[p][n] Z[p][j]
  W.l = dG; W.ldl = f; W.l_f32 = false; W.r = Z; W.ldr = 3 * r; W.Aw = f; W.Bw = r; W.s = lam;
  W.out = dB_gate;
  moe::launch_wgrad_simple(bf, W, st);
  W.l = dU; W.r = Z + r; W.out = dB_up;
  moe::launch_wgrad_simple(bf, W, st);
  // dA [r][d] = sum_p dZ[p][j] X[token(p)][c]
  W.l = dZ; W.ldl = 3 * r; W.l_f32 = true; W.gather = true; W.r = x; W.ldr = d; W.Aw = r;
  W.Bw = d; W.s = 1.f; W.out = dA_gate;
  moe::launch_wgrad_simple(bf, W, st);
  W.l = dZ + r; W.out = dA_up;
  moe::launch_wgrad_simple(bf, W, st);
  // dX_perm = dG W_g + dZ_g A_g + dU W_u + dZ_u A_u   (float32)
  A.a = dG; A.lda = f; A.q = gate.q; A.scale = gate.scale; A.N = d; A.K = f;
  A.Z = dZ; A.lmat = gate.A; A.l_es = (size_t)r * d; A.l_js = d; A.l_ns = 1;
  A.out = dXp; A.ldo = d; A.acc_out = false;
  TIMED(MOE_KT_BWD_GATEUP, st, moe::launch_lin_simple(bf, true, A, st));
  A.a = dU; A.q = up.q; A.scale = up.scale; A.Z = dZ + r; A.lmat = up.A; A.acc_out = true;
  TIMED(MOE_KT_BWD_GATEUP, st, moe::launch_lin_simple(bf, true, A, st));
  moe::launch_unpermute_sum(bf, true, dx_r, dXp, slot_pos, T, d, k, dx, st);
  return hip_status("moe_adapter_bwd");
}

}  // extern "C"
