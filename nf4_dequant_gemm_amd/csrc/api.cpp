// Host side of the C ABI declared in include/nf4qlora.h: argument validation (before any HIP
// call), the NF4 tables, workspace layout and kernel launches.
#include "nf4qlora.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return NF4_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(NF4_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------- NF4 codebook
// The 16 NF4 levels follow the QLoRA construction of 4-bit NormalFloat (the pages name NF4 but
// print no levels [Unsloth v0.1.463-beta release article, "About the Unsloth Project"]):
// normal quantiles of 8 (positive side) and 7 (negative side) evenly spaced probabilities between
// delta = 1 - (1/30 + 1/32)/2 and 1/2, plus an exact zero, normalised by the largest. The
// quantile is solved here by Newton's method on erfc in double precision, then rounded to float.
double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_ppf(double p) {
  // Phi is concave on x > 0, so Newton's iteration from 0 rises monotonically to the root.
  double x = 0.0;
  for (int it = 0; it < 200; ++it) {
    const double f = normal_cdf(x) - p;
    const double d = std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
    const double step = f / d;
    const double nx = x - step;
    if (nx == x || std::fabs(step) <= 1e-17 * std::fabs(nx)) {
      x = nx;
      break;
    }
    x = nx;
  }
  return x;
}

struct TablesHolder {
  nf4q::Tables t;
  TablesHolder() {
    const double delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
    double v[16];
    int n = 0;
    for (int j = 0; j < 8; ++j) v[n++] = normal_ppf(delta + (0.5 - delta) * j / 8.0);
    for (int j = 0; j < 7; ++j) v[n++] = -normal_ppf(delta + (0.5 - delta) * j / 7.0);
    v[n++] = 0.0;
    std::sort(v, v + 16);
    double top = 0.0;
    for (double x : v) top = std::max(top, std::fabs(x));
    for (int i = 0; i < 16; ++i) t.level[i] = (float)(v[i] / top);
    for (int i = 0; i < 15; ++i) {
      const double mid = ((double)t.level[i] + (double)t.level[i + 1]) / 2.0;  // exact
      float th = (float)mid;
      if ((double)th > mid) th = std::nextafter(th, -INFINITY);
      t.thresh[i] = th;
    }
  }
};

const nf4q::Tables &tables() {
  static const TablesHolder h;
  return h.t;
}

// ------------------------------------------------------------------------------ validation
int check_weight(const nf4_tensor *q) {
  if (!q) return fail(NF4_EINVAL, "weight descriptor is NULL");
  if (q->n < 1) return fail(NF4_EINVAL, "weight n must be >= 1 (got %lld)", (long long)q->n);
  if (q->k < 64 || q->k % 64)
    return fail(NF4_EUNSUPPORTED, "weight k must be a positive multiple of 64 (got %lld)",
                (long long)q->k);
  if (q->block != 64 && q->block != 16)
    return fail(NF4_EUNSUPPORTED, "block must be 64 (NF4) or 16 (E2M1) (got %d)", q->block);
  if (q->block == 16 && q->dq_block != 0)
    return fail(NF4_EUNSUPPORTED, "the E2M1 format (block 16) takes dq_block 0 (got %d)", q->dq_block);
  if (q->dq_block != 0 && q->dq_block != 256)
    return fail(NF4_EUNSUPPORTED, "dq_block must be 0 or 256 (got %d)", q->dq_block);
  if (q->n > (int64_t(1) << 40) / q->k)
    return fail(NF4_EUNSUPPORTED, "n*k must be below 2^40");
  if (!q->codes || !q->absmax) return fail(NF4_EINVAL, "codes/absmax pointer is NULL");
  const bool scale_used = q->dq_block || q->block == 16;
  if (scale_used && !q->absmax_scale) return fail(NF4_EINVAL, "absmax_scale is NULL");
  if (!aligned16(q->codes) || !aligned16(q->absmax) || (scale_used && !aligned16(q->absmax_scale)))
    return fail(NF4_EINVAL, "weight buffers must be 16-byte aligned");
  return NF4_OK;
}

nf4q::WDesc desc(const nf4_tensor *q) {
  nf4q::WDesc w;
  w.codes = q->codes;
  w.absmax = q->absmax;
  w.scale = q->absmax_scale;
  w.n = q->n;
  w.k = q->k;
  w.dq = q->dq_block ? 1 : 0;
  w.fp4 = q->block == 16 ? 1 : 0;
  return w;
}

int check_layer(const void *X, int64_t m, const nf4_tensor *W, const void *A, const void *B,
                int32_t r) {
  int st = check_weight(W);
  if (st) return st;
  if (m < 1) return fail(NF4_EINVAL, "m must be >= 1 (got %lld)", (long long)m);
  if (m > (int64_t(1) << 24)) return fail(NF4_EUNSUPPORTED, "m must be <= 2^24");
  if (W->n % 8) return fail(NF4_EUNSUPPORTED, "n must be a multiple of 8 (got %lld)", (long long)W->n);
  // the GEMM kernels address the codes, X and dY tiles with 32-bit buffer offsets
  if (W->n * W->k >= (int64_t(1) << 32) || W->k > (int64_t(1) << 22) || W->n > (int64_t(1) << 22))
    return fail(NF4_EUNSUPPORTED, "n*k must be below 2^32 and n, k at most 2^22 for the GEMM calls");
  if (r < 0 || r > 128) return fail(NF4_EINVAL, "r must lie in [0, 128] (got %d)", r);
  if (!X) return fail(NF4_EINVAL, "X is NULL");
  if (!aligned16(X)) return fail(NF4_EINVAL, "X must be 16-byte aligned");
  if (r > 0) {
    if (!A || !B) return fail(NF4_EINVAL, "A and B must be non-NULL when r > 0");
    if (!aligned16(A) || !aligned16(B)) return fail(NF4_EINVAL, "A and B must be 16-byte aligned");
  }
  return NF4_OK;
}

hipError_t launch_dx(const uint16_t *dy, int64_t m, const nf4_tensor *W, const uint16_t *U,
                     const uint16_t *A, int32_t r, float s, uint16_t *dX, hipStream_t sm) {
  nf4q::GemmArgs g;
  g.a_side = dy;
  g.lda = W->n;
  g.lora_a = U;
  g.lora_b = A;
  g.w = desc(W);
  g.M = m;
  g.C = W->k;
  g.R = W->n;
  g.r = r;
  g.s = s;
  g.out = dX;
  g.ldo = W->k;
  g.t = tables();
  return nf4q::launch_gemm_dx(g, sm);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct FwdWs {
  int splits = 1;
  size_t part = 0, total = 0;
};

FwdWs fwd_ws(int64_t m, int64_t k, int32_t r) {
  FwdWs w;
  if (r <= 0) return w;
  w.splits = nf4q::rowproj_splits(m, k);
  if (w.splits > 1) w.part = align256((size_t)w.splits * m * r * 4);
  w.total = w.part;
  return w;
}

struct BwdWs {
  int splits_u = 1, splits_a = 1, splits_b = 1, splits_t = 1;
  // byte sizes: U at 0, Bt at u, T (recomputed when the caller passes none) at u + bt, partials
  // at u + bt + t
  size_t u = 0, bt = 0, t = 0, part = 0, total = 0;
};

BwdWs bwd_ws(int64_t m, int64_t n, int64_t k, int32_t r) {
  BwdWs w;
  if (r <= 0) return w;
  w.u = align256((size_t)m * r * 2);
  w.bt = align256((size_t)r * n * 2);
  w.t = align256((size_t)m * r * 2);
  w.splits_u = nf4q::rowproj_splits(m, n);
  w.splits_t = nf4q::rowproj_splits(m, k);
  w.splits_a = nf4q::mreduce_splits(m, k, r);
  w.splits_b = nf4q::mreduce_splits(m, n, r);
  size_t p = 0;
  if (w.splits_u > 1) p = std::max(p, (size_t)w.splits_u * m * r * 4);
  if (w.splits_t > 1) p = std::max(p, (size_t)w.splits_t * m * r * 4);
  p = std::max(p, (size_t)w.splits_a * r * k * 4);
  p = std::max(p, (size_t)w.splits_b * r * n * 4);
  w.part = align256(p);
  w.total = w.u + w.bt + w.t + w.part;
  return w;
}

// Gate/up SwiGLU pair: B2 [2n, 2r] (block-diagonal up projection) first; then, for the forward,
// T (when the caller keeps none) and qlora_fwd's workspace of the stacked layer; for the
// backward, dY2 [m, 2n], dB2 [2n, 2r] and qlora_bwd's workspace of the stacked layer.
struct SwiWs {
  size_t b2 = 0, t = 0, fwd = 0, dy2 = 0, db2 = 0, bwd = 0, total = 0;
};

SwiWs swi_ws(int64_t m, int64_t n, int64_t k, int32_t r) {
  SwiWs w;
  if (r > 0) {
    w.b2 = align256((size_t)(2 * n) * (2 * r) * 2);
    w.t = align256((size_t)m * (2 * r) * 2);
    w.fwd = fwd_ws(m, k, 2 * r).total;
    w.db2 = w.b2;
  }
  w.dy2 = align256((size_t)m * (2 * n) * 2);
  w.bwd = bwd_ws(m, 2 * n, k, 2 * r).total;
  w.total = w.b2 + std::max(w.t + w.fwd, w.dy2 + w.db2 + w.bwd);
  return w;
}

int check_swiglu(const void *X, int64_t m, const nf4_tensor *Wgu, const void *Agu, const void *Bg,
                 const void *Bu, int32_t r, void *ws, size_t ws_bytes, size_t *need) {
  int st = check_weight(Wgu);
  if (st) return st;
  if (Wgu->n % 2) return fail(NF4_EINVAL, "Wgu must hold 2n rows (got %lld)", (long long)Wgu->n);
  const int64_t n = Wgu->n / 2;
  if (n % 8) return fail(NF4_EUNSUPPORTED, "n must be a multiple of 8 (got %lld)", (long long)n);
  if (r < 0 || r > 64) return fail(NF4_EINVAL, "r must lie in [0, 64] (got %d)", r);
  st = check_layer(X, m, Wgu, Agu, Agu, 2 * r);   // X, the stacked weight, Agu
  if (st) return st;
  if (r > 0) {
    if (!Bg || !Bu) return fail(NF4_EINVAL, "Bg and Bu must be non-NULL when r > 0");
    if (!aligned16(Bg) || !aligned16(Bu)) return fail(NF4_EINVAL, "Bg and Bu must be 16-byte aligned");
  }
  *need = swi_ws(m, n, Wgu->k, r).total;
  if (ws_bytes < *need || !ws)
    return fail(NF4_EINVAL, "workspace of %zu bytes is smaller than the %zu required", ws_bytes,
                *need);
  if (!aligned16(ws)) return fail(NF4_EINVAL, "ws must be 16-byte aligned");
  return NF4_OK;
}

// Mixture of experts: E experts, rows grouped in expert order, stacked tensors W [E n, k],
// A [E r, k], B [E n, r]. The routing (rows per expert) is either given on the host (counts[e],
// summed into off) or held in device memory (the row total m given on the host; the group table
// is then built on the device, in the workspace).
struct Moe {
  int64_t off[nf4q::kMaxExperts + 1];   // host routing
  int64_t n = 0, mtotal = 0;
  const int64_t *dcounts = nullptr;     // device routing: counts [E] in device memory
};

int check_moe_shape(const void *X, int32_t E, const nf4_tensor *W, const void *A, const void *B,
                    int32_t r, Moe *mo) {
  int st = check_weight(W);
  if (st) return st;
  if (W->n % E) return fail(NF4_EINVAL, "W must hold E*n rows (got %lld for E = %d)", (long long)W->n, E);
  mo->n = W->n / E;
  if (mo->n % 8) return fail(NF4_EUNSUPPORTED, "n must be a multiple of 8 (got %lld)", (long long)mo->n);
  return check_layer(X, mo->mtotal, W, A, B, r);   // m >= 1, the GEMM limits, X, A, B
}

int check_moe(const void *X, const int64_t *counts, int32_t E, const nf4_tensor *W, const void *A,
              const void *B, int32_t r, Moe *mo) {
  if (E < 1 || E > nf4q::kMaxExperts)
    return fail(NF4_EINVAL, "E must lie in [1, %d] (got %d)", nf4q::kMaxExperts, E);
  if (!counts) return fail(NF4_EINVAL, "counts is NULL");
  mo->off[0] = 0;
  for (int e = 0; e < E; ++e) {
    if (counts[e] < 0) return fail(NF4_EINVAL, "counts[%d] is negative", e);
    mo->off[e + 1] = mo->off[e] + counts[e];
  }
  mo->mtotal = mo->off[E];
  return check_moe_shape(X, E, W, A, B, r, mo);
}

int check_moe_dev(const void *X, int64_t m, const int64_t *dcounts, int32_t E, const nf4_tensor *W,
                  const void *A, const void *B, int32_t r, Moe *mo) {
  if (E < 1 || E > nf4q::kMaxExperts)
    return fail(NF4_EINVAL, "E must lie in [1, %d] (got %d)", nf4q::kMaxExperts, E);
  if (!dcounts || (reinterpret_cast<uintptr_t>(dcounts) & 7))
    return fail(NF4_EINVAL, "counts must be a non-NULL, 8-byte aligned device pointer");
  mo->mtotal = m;
  mo->dcounts = dcounts;
  return check_moe_shape(X, E, W, A, B, r, mo);
}

// Launch plan of the grouped layer's rank-r products: the row projections (T = X_e A_e^T,
// U = dY_e B_e) run over every expert's 64-row blocks in one launch, split over the reduction
// like the single layer's; the M-reductions (dA_e, dB_e) run over (expert, column tile, split)
// in one launch (mreduce_splits over E experts), each expert's rows cut into that many splits. The split counts depend on the row total only, so the same routing
// gives the same sums in the same order whether it is given on the host or on the device, and
// one expert gives the single layer's.
struct MoePlan {
  int sp_k = 1, sp_n = 1, sa = 1, sb = 1;
};

MoePlan moe_plan(int64_t mtotal, int32_t E, int64_t n, int64_t k, int32_t r) {
  MoePlan pl;
  pl.sp_k = nf4q::rowproj_splits(mtotal, k);
  pl.sp_n = nf4q::rowproj_splits(mtotal, n);
  pl.sa = nf4q::mreduce_splits(mtotal, k, r, E);
  pl.sb = nf4q::mreduce_splits(mtotal, n, r, E);
  return pl;
}

// Workspace of the grouped layer: with device routing the group table first (table bytes),
// then U [m, r], the transposed stacked B [r, E n], T (recomputed when the caller passes none),
// then float partials of the row projections or of the M-reductions (never both at once).
struct MoeWs {
  size_t table = 0, u = 0, bt = 0, t = 0, part = 0, total = 0;
};

MoeWs moe_ws_layout(int64_t mtotal, int32_t E, int64_t n, int64_t k, int32_t r, bool dev) {
  MoeWs w;
  if (dev) w.table = align256(nf4q::moe_table_bytes(E));
  // the grouped dX's split tail tiles: at most kDxMaxWidth pieces, and at most kDxMaxPieces per
  // tile of the launch (row blocks bounded as in moe_groups)
  const int64_t blocks = std::min<int64_t>((mtotal + 255 * (int64_t)E) / 256, mtotal);
  const int64_t pieces = std::min<int64_t>(nf4q::kDxMaxWidth, nf4q::kDxMaxPieces * blocks * ((k + 255) / 256));
  size_t p = (size_t)pieces * nf4q::kDxPieceFloats * 4;
  if (r > 0) {
    const MoePlan pl = moe_plan(mtotal, E, n, k, r);
    w.u = align256((size_t)mtotal * r * 2);
    w.bt = align256((size_t)r * E * n * 2);
    w.t = w.u;
    if (pl.sp_k > 1) p = std::max(p, (size_t)pl.sp_k * mtotal * r * 4);
    if (pl.sp_n > 1) p = std::max(p, (size_t)pl.sp_n * mtotal * r * 4);
    p = std::max(p, (size_t)E * pl.sa * r * k * 4);
    p = std::max(p, (size_t)E * pl.sb * r * n * 4);
  }
  w.part = align256(p);
  w.total = w.table + w.u + w.bt + w.t + w.part;
  return w;
}

// Groups of a grouped launch whose tiles are `rows` rows of an expert times tiles_c column tiles.
// Host routing: the experts' row offsets and first tiles by value, the grid exact. Device
// routing: the device table (`which`: 0 forward tiles, 1 dX tiles, 2 64-row blocks) and a grid
// bounded by the row total (sum of ceil(rows_e / rows) <= (m + (rows - 1) E) / rows, and <= m).
int moe_groups(const Moe &mo, int32_t E, int64_t tiles_c, nf4q::GroupArgs *gr, int64_t rows,
               void *table, int which) {
  gr->E = E;
  if (mo.dcounts) {
    gr->dm_off = nf4q::moe_table_m_off(table);
    gr->dtile_off = nf4q::moe_table_tiles(table, E, which);
    const int64_t blocks = std::min<int64_t>((mo.mtotal + (rows - 1) * E) / rows, mo.mtotal);
    gr->grid = blocks * tiles_c;
    if (gr->grid >= (int64_t(1) << 31)) return fail(NF4_EUNSUPPORTED, "too many tiles");
    return NF4_OK;
  }
  gr->dm_off = nullptr;
  gr->dtile_off = nullptr;
  gr->tile_off[0] = 0;
  for (int e = 0; e <= E; ++e) gr->m_off[e] = mo.off[e];
  for (int e = 0; e < E; ++e) {
    const int64_t me = mo.off[e + 1] - mo.off[e];
    const int64_t t = gr->tile_off[e] + (me + rows - 1) / rows * tiles_c;
    if (t >= (int64_t(1) << 31)) return fail(NF4_EUNSUPPORTED, "too many tiles");
    gr->tile_off[e + 1] = (int32_t)t;
  }
  gr->grid = gr->tile_off[E];
  return NF4_OK;
}

// Device routing: the group tables, built from the device counts into the workspace.
hipError_t moe_build_table(const Moe &mo, int32_t E, int64_t k, void *table, hipStream_t sm) {
  if (!mo.dcounts) return hipSuccess;
  return nf4q::launch_moe_plan(mo.dcounts, E, mo.mtotal, (mo.n + 255) / 256, (k + 255) / 256, table, sm);
}

// ------------------------------------------------------------------ no-allocation forward
// The workspace of qlora_fwd_noalloc: a static device array, one per GPU the library runs on
// (each holds its own copy until the process ends). Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, looked up once per device with
// that device current, and is what the kernels receive.
constexpr size_t kNoAllocScratchBytes = NF4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "qlora_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(NF4_EUNSUPPORTED, "qlora_fwd_noalloc: device %d beyond the %d it serves", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "qlora_fwd_noalloc: hipGetSymbolAddress");
    if (!p) return fail(NF4_EHIP, "qlora_fwd_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NF4_OK;
}

}  // namespace

extern "C" {

const char *nf4_last_error(void) { return g_err.c_str(); }

int nf4_codebook(float *levels, float *thresholds) {
  if (!levels) return fail(NF4_EINVAL, "levels is NULL");
  const nf4q::Tables &t = tables();
  for (int i = 0; i < 16; ++i) levels[i] = t.level[i];
  if (thresholds)
    for (int i = 0; i < 15; ++i) thresholds[i] = t.thresh[i];
  return ok();
}

int nf4_quantize(const void *w, int w_dtype, const nf4_tensor *q, void *stream) {
  int st = check_weight(q);
  if (st) return st;
  if (!w) return fail(NF4_EINVAL, "w is NULL");
  if (!aligned16(w)) return fail(NF4_EINVAL, "w must be 16-byte aligned");
  if (w_dtype != NF4_BF16 && w_dtype != NF4_F32) return fail(NF4_EINVAL, "unknown w_dtype %d", w_dtype);
  if (q->block == 16)
    return hip_status(nf4q::launch_fp4_quantize(w, w_dtype == NF4_F32, q->n * q->k, q->codes,
                                                (uint8_t *)q->absmax, q->absmax_scale,
                                                (hipStream_t)stream),
                      "nf4_quantize launch");
  const int64_t nblk = q->n * q->k / 64;
  return hip_status(nf4q::launch_quantize(w, w_dtype == NF4_F32, q->codes, q->absmax,
                                          q->absmax_scale, nblk, q->dq_block ? 1 : 0, tables(),
                                          (hipStream_t)stream),
                    "nf4_quantize launch");
}

int nf4_dequantize(const nf4_tensor *q, void *out, int out_dtype, void *stream) {
  int st = check_weight(q);
  if (st) return st;
  if (!out) return fail(NF4_EINVAL, "out is NULL");
  if (!aligned16(out)) return fail(NF4_EINVAL, "out must be 16-byte aligned");
  if (out_dtype != NF4_BF16 && out_dtype != NF4_F32)
    return fail(NF4_EINVAL, "unknown out_dtype %d", out_dtype);
  if (q->block == 16)
    return hip_status(nf4q::launch_fp4_dequantize(desc(q), out, out_dtype == NF4_F32,
                                                  (hipStream_t)stream),
                      "nf4_dequantize launch");
  return hip_status(nf4q::launch_dequantize(desc(q), out, out_dtype == NF4_F32, tables(),
                                            (hipStream_t)stream),
                    "nf4_dequantize launch");
}

size_t qlora_fwd_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r) {
  (void)n;
  if (m < 1 || k < 1 || r < 0) return 0;
  return fwd_ws(m, k, r).total;
}

int qlora_lora_down(const void *X, int64_t m, int64_t k, const void *A, int32_t r, void *T,
                    void *ws, size_t ws_bytes, void *stream) {
  if (m < 1) return fail(NF4_EINVAL, "m must be >= 1 (got %lld)", (long long)m);
  if (m > (int64_t(1) << 24)) return fail(NF4_EUNSUPPORTED, "m must be <= 2^24");
  if (k < 64 || k % 64)
    return fail(NF4_EUNSUPPORTED, "k must be a positive multiple of 64 (got %lld)", (long long)k);
  if (r < 1 || r > 128) return fail(NF4_EINVAL, "r must lie in [1, 128] (got %d)", r);
  if (!X || !A || !T) return fail(NF4_EINVAL, "X, A and T must be non-NULL");
  if (!aligned16(X) || !aligned16(A) || !aligned16(T))
    return fail(NF4_EINVAL, "X, A and T must be 16-byte aligned");
  const FwdWs lay = fwd_ws(m, k, r);
  if (ws_bytes < lay.total || (lay.total && !ws))
    return fail(NF4_EINVAL, "workspace of %zu bytes is smaller than the %zu required", ws_bytes,
                lay.total);
  if (lay.total && !aligned16(ws)) return fail(NF4_EINVAL, "ws must be 16-byte aligned");
  return hip_status(nf4q::launch_rowproj((const uint16_t *)X, k, (const uint16_t *)A, k, m, k, r,
                                         lay.splits, (float *)ws, (uint16_t *)T,
                                         (hipStream_t)stream),
                    "qlora_lora_down launch");
}

// Shapes of the M <= 16 stream kernel: double-quantised NF4 or E2M1 codes, K a multiple of 256.
static bool stream16_shape(int64_t m, const nf4_tensor *W) {
  return m <= 16 && (W->dq_block > 0 || W->block == 16) && W->k % 256 == 0;
}

int qlora_fwd_fused(const void *X, int64_t m, const nf4_tensor *W, const void *T, const void *B,
                    int32_t r, float s, void *Y, void *stream) {
  int st = check_layer(X, m, W, T, B, r);
  if (st) return st;
  if (!Y || !aligned16(Y)) return fail(NF4_EINVAL, "Y must be non-NULL and 16-byte aligned");
  nf4q::GemmArgs g;
  g.a_side = (const uint16_t *)X;
  g.lda = W->k;
  g.lora_a = (const uint16_t *)T;
  g.lora_b = (const uint16_t *)B;
  g.w = desc(W);
  g.M = m;
  g.C = W->n;
  g.R = W->k;
  g.r = r;
  g.s = s;
  g.out = (uint16_t *)Y;
  g.ldo = W->n;
  g.t = tables();
  if (stream16_shape(m, W))
    return hip_status(nf4q::launch_decode16_fwd(g, (hipStream_t)stream), "qlora_fwd_fused launch");
  if (m <= (W->block == 64 ? nf4q::kDecodeMaxM : 16) && W->k % 256 == 0)
    return hip_status(nf4q::launch_decode_fwd(g, (hipStream_t)stream), "qlora_fwd_fused launch");
  return hip_status(nf4q::launch_gemm_fwd(g, (hipStream_t)stream), "qlora_fwd_fused launch");
}

int qlora_fwd(const void *X, int64_t m, const nf4_tensor *W, const void *A, const void *B,
              int32_t r, float s, void *Y, void *T, void *ws, size_t ws_bytes, void *stream) {
  int st = check_layer(X, m, W, A, B, r);
  if (st) return st;
  if (!Y || !aligned16(Y)) return fail(NF4_EINVAL, "Y must be non-NULL and 16-byte aligned");
  // Decode shapes (the M <= 16 kernel): up to rank 64 (NF4) or 16 (E2M1) the fused kernel forms
  // T = X A^T itself from the X slices it streams (one launch, no workspace); otherwise the split
  // partials of T are added inside it (its prologue hides them under the first weight copies),
  // saving the separate reduction launch. Either way workgroup 0 of the fused kernel writes T.
  const int64_t k = W->k;
  const int tin_max = W->block == 16 ? nf4q::kDecode16MaxTinRankE2M1 : nf4q::kDecode16MaxTinRank;
  if (r > 0 && stream16_shape(m, W) && r % 8 == 0 && r <= tin_max) {
    if (!T || !aligned16(T)) return fail(NF4_EINVAL, "T must be non-NULL and 16-byte aligned");
    nf4q::GemmArgs g;
    g.a_side = (const uint16_t *)X;
    g.lda = k;
    g.lora_a = nullptr;
    g.lora_b = (const uint16_t *)B;
    g.w = desc(W);
    g.M = m;
    g.C = W->n;
    g.R = k;
    g.r = r;
    g.s = s;
    g.out = (uint16_t *)Y;
    g.ldo = W->n;
    g.t = tables();
    return hip_status(nf4q::launch_decode16_fwd_tin(g, (const uint16_t *)A, (uint16_t *)T, (hipStream_t)stream),
                      "qlora_fwd launch");
  }
  if (r > 0 && stream16_shape(m, W) && r % 8 == 0) {
    const FwdWs lay = fwd_ws(m, k, r);
    if (lay.splits > 1 && (int64_t)r * lay.splits <= 1024) {
      if (!T || !aligned16(T)) return fail(NF4_EINVAL, "T must be non-NULL and 16-byte aligned");
      if (ws_bytes < lay.total || !ws)
        return fail(NF4_EINVAL, "workspace of %zu bytes is smaller than the %zu required", ws_bytes,
                    lay.total);
      if (!aligned16(ws)) return fail(NF4_EINVAL, "ws must be 16-byte aligned");
      hipStream_t sm = (hipStream_t)stream;
      hipError_t e = nf4q::launch_rowproj((const uint16_t *)X, k, (const uint16_t *)A, k, m, k, r,
                                          lay.splits, (float *)ws, nullptr, sm);
      if (e != hipSuccess) return hip_status(e, "qlora_fwd launch");
      nf4q::GemmArgs g;
      g.a_side = (const uint16_t *)X;
      g.lda = k;
      g.lora_a = nullptr;
      g.lora_b = (const uint16_t *)B;
      g.w = desc(W);
      g.M = m;
      g.C = W->n;
      g.R = k;
      g.r = r;
      g.s = s;
      g.out = (uint16_t *)Y;
      g.ldo = W->n;
      g.t = tables();
      return hip_status(nf4q::launch_decode16_fwd_tpart(g, (const float *)ws, lay.splits,
                                                        (uint16_t *)T, sm),
                        "qlora_fwd launch");
    }
  }
  if (r > 0) {
    st = qlora_lora_down(X, m, k, A, r, T, ws, ws_bytes, stream);
    if (st) return st;
  }
  return qlora_fwd_fused(X, m, W, T, B, r, s, Y, stream);
}

int qlora_fwd_noalloc(const void *X, int64_t m, const nf4_tensor *W, const void *A, const void *B,
                      int32_t r, float s, void *Y, void *T, void *stream) {
  // every check before any HIP call (the scratch lookup included)
  int st = check_layer(X, m, W, A, B, r);
  if (st) return st;
  if (!Y || !aligned16(Y)) return fail(NF4_EINVAL, "Y must be non-NULL and 16-byte aligned");
  if (r > 0 && (!T || !aligned16(T))) return fail(NF4_EINVAL, "T must be non-NULL and 16-byte aligned");
  const size_t need = fwd_ws(m, W->k, r).total;
  if (need > kNoAllocScratchBytes)
    return fail(NF4_EUNSUPPORTED,
                "qlora_fwd_noalloc: these sizes need %zu bytes of scratch, its static array holds %zu "
                "(call qlora_fwd with a workspace instead)",
                need, kNoAllocScratchBytes);
  void *ws = nullptr;
  if (need) {
    st = scratch_of_current_device(&ws);
    if (st) return st;
  }
  return qlora_fwd(X, m, W, A, B, r, s, Y, T, ws, need ? kNoAllocScratchBytes : 0, stream);
}

size_t qlora_bwd_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r) {
  if (m < 1 || n < 1 || k < 1 || r < 0) return 0;
  return bwd_ws(m, n, k, r).total;
}

int qlora_bwd(const void *dY, const void *X, int64_t m, const nf4_tensor *W, const void *A,
              const void *B, int32_t r, float s, const void *T, void *dX, void *dA, void *dB,
              void *ws, size_t ws_bytes, void *stream) {
  int st = check_layer(X, m, W, A, B, r);
  if (st) return st;
  if (!dY || !aligned16(dY)) return fail(NF4_EINVAL, "dY must be non-NULL and 16-byte aligned");
  if (dX && !aligned16(dX)) return fail(NF4_EINVAL, "dX must be 16-byte aligned");
  if (r > 0) {
    if (!dA || !dB) return fail(NF4_EINVAL, "dA and dB must be non-NULL when r > 0");
    if ((T && !aligned16(T)) || !aligned16(dA) || !aligned16(dB))
      return fail(NF4_EINVAL, "T, dA and dB must be 16-byte aligned");
  }
  if (!dX && r == 0) return ok();
  const int64_t n = W->n, k = W->k;
  const BwdWs lay = bwd_ws(m, n, k, r);
  if (ws_bytes < lay.total || (lay.total && !ws))
    return fail(NF4_EINVAL, "workspace of %zu bytes is smaller than the %zu required", ws_bytes,
                lay.total);
  if (lay.total && !aligned16(ws)) return fail(NF4_EINVAL, "ws must be 16-byte aligned");
  hipStream_t sm = (hipStream_t)stream;
  char *base = (char *)ws;
  uint16_t *U = (uint16_t *)base;
  uint16_t *Bt = (uint16_t *)(base + lay.u);
  float *part = (float *)(base + lay.u + lay.bt + lay.t);
  const uint16_t *dy = (const uint16_t *)dY;
  hipError_t e;
  if (r > 0 && !T) {   // T = X A^T recomputed into the workspace, as qlora_lora_down computes it
    uint16_t *Tw = (uint16_t *)(base + lay.u + lay.bt);
    e = nf4q::launch_rowproj((const uint16_t *)X, k, (const uint16_t *)A, k, m, k, r, lay.splits_t,
                             part, Tw, sm);
    if (e != hipSuccess) return hip_status(e, "qlora_bwd T launch");
    T = Tw;
  }
  if (r > 0) {
    e = nf4q::launch_transpose((const uint16_t *)B, n, r, Bt, sm);
    if (e != hipSuccess) return hip_status(e, "qlora_bwd transpose launch");
    e = nf4q::launch_rowproj(dy, n, Bt, n, m, n, r, lay.splits_u, part, U, sm);
    if (e != hipSuccess) return hip_status(e, "qlora_bwd U launch");
  }
  if (dX) {
    e = launch_dx(dy, m, W, U, (const uint16_t *)A, r, s, (uint16_t *)dX, sm);
    if (e != hipSuccess) return hip_status(e, "qlora_bwd dX launch");
  }
  if (r > 0) {
    e = nf4q::launch_mreduce(U, (const uint16_t *)X, k, m, k, r, s, lay.splits_a, part,
                             (uint16_t *)dA, false, sm);
    if (e != hipSuccess) return hip_status(e, "qlora_bwd dA launch");
    e = nf4q::launch_mreduce((const uint16_t *)T, dy, n, m, n, r, s, lay.splits_b, part,
                             (uint16_t *)dB, true, sm);
    if (e != hipSuccess) return hip_status(e, "qlora_bwd dB launch");
  }
  return ok();
}

size_t qlora_swiglu_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r) {
  if (m < 1 || n < 1 || k < 1 || r < 0) return 0;
  return swi_ws(m, n, k, r).total;
}

// One launch of the fused kernel in its pair form: Yg, Yu and, in the epilogue, H; the up
// projection is the block-diagonal [[Bg, 0], [0, Bu]] applied by the kernel.
static int swiglu_pair_launch(const void *X, int64_t m, const nf4_tensor *Wgu, const void *T,
                              const void *Bg, const void *Bu, int32_t r, float s, void *H, void *Ygu,
                              hipStream_t sm, const char *what) {
  const int64_t n = Wgu->n / 2, k = Wgu->k;
  nf4q::GemmArgs g;
  g.a_side = (const uint16_t *)X;
  g.lda = k;
  g.lora_a = r > 0 ? (const uint16_t *)T : nullptr;
  g.lora_b = r > 0 ? (const uint16_t *)Bg : nullptr;
  g.lora_b2 = r > 0 ? (const uint16_t *)Bu : nullptr;
  g.w = desc(Wgu);
  g.M = m;
  g.C = n;
  g.R = k;
  g.r = 2 * r;
  g.s = s;
  g.out = (uint16_t *)Ygu;
  g.ldo = 2 * n;
  g.t = tables();
  g.hout = (uint16_t *)H;
  g.ldh = n;
  return hip_status(nf4q::launch_gemm_fwd_pair(g, sm), what);
}

int qlora_swiglu_fwd(const void *X, int64_t m, const nf4_tensor *Wgu, const void *Agu,
                     const void *Bg, const void *Bu, int32_t r, float s, void *H, void *Ygu,
                     void *Tgu, void *ws, size_t ws_bytes, void *stream) {
  size_t need = 0;
  int st = check_swiglu(X, m, Wgu, Agu, Bg, Bu, r, ws, ws_bytes, &need);
  if (st) return st;
  if (!H || !aligned16(H) || !Ygu || !aligned16(Ygu))
    return fail(NF4_EINVAL, "H and Ygu must be non-NULL and 16-byte aligned");
  if (Tgu && !aligned16(Tgu)) return fail(NF4_EINVAL, "Tgu must be 16-byte aligned");
  const int64_t n = Wgu->n / 2;
  const SwiWs lay = swi_ws(m, n, Wgu->k, r);
  hipStream_t sm = (hipStream_t)stream;
  char *base = (char *)ws;
  void *T = r > 0 ? (Tgu ? Tgu : (void *)(base + lay.b2)) : nullptr;
  const int64_t k = Wgu->k;
  // shapes the stacked layer sends to the decode kernels (M <= 48): the stacked forward with the
  // block-diagonal up projection built in the workspace, then the activation kernel
  if (m <= (Wgu->block == 64 ? nf4q::kDecodeMaxM : 16) && k % 256 == 0) {
    uint16_t *B2 = r > 0 ? (uint16_t *)base : nullptr;
    if (r > 0) {
      hipError_t e = nf4q::launch_blockdiag((const uint16_t *)Bg, (const uint16_t *)Bu, n, r, B2, sm);
      if (e != hipSuccess) return hip_status(e, "qlora_swiglu_fwd launch");
    }
    st = qlora_fwd(X, m, Wgu, r > 0 ? Agu : nullptr, B2, 2 * r, s, Ygu, T,
                   lay.fwd ? base + lay.b2 + lay.t : nullptr, lay.fwd, stream);
    if (st) return st;
    return hip_status(nf4q::launch_swiglu_fwd((const uint16_t *)Ygu, m, n, (uint16_t *)H, sm),
                      "qlora_swiglu_fwd launch");
  }
  // otherwise T = X Agu^T, then the pair's one fused launch
  if (r > 0) {
    st = qlora_lora_down(X, m, k, Agu, 2 * r, T, lay.fwd ? base + lay.b2 + lay.t : nullptr, lay.fwd,
                         stream);
    if (st) return st;
  }
  return swiglu_pair_launch(X, m, Wgu, T, Bg, Bu, r, s, H, Ygu, sm, "qlora_swiglu_fwd launch");
}

int qlora_swiglu_fwd_fused(const void *X, int64_t m, const nf4_tensor *Wgu, const void *Tgu,
                           const void *Bg, const void *Bu, int32_t r, float s, void *H, void *Ygu,
                           void *stream) {
  int st = check_weight(Wgu);
  if (st) return st;
  if (Wgu->n % 2) return fail(NF4_EINVAL, "Wgu must hold 2n rows (got %lld)", (long long)Wgu->n);
  const int64_t n = Wgu->n / 2;
  if (n % 8) return fail(NF4_EUNSUPPORTED, "n must be a multiple of 8 (got %lld)", (long long)n);
  if (r < 0 || r > 64) return fail(NF4_EINVAL, "r must lie in [0, 64] (got %d)", r);
  st = check_layer(X, m, Wgu, Tgu, Tgu, 2 * r);   // X, the stacked weight, Tgu
  if (st) return st;
  if (r > 0) {
    if (!Bg || !Bu) return fail(NF4_EINVAL, "Bg and Bu must be non-NULL when r > 0");
    if (!aligned16(Bg) || !aligned16(Bu)) return fail(NF4_EINVAL, "Bg and Bu must be 16-byte aligned");
  }
  if (!H || !aligned16(H) || !Ygu || !aligned16(Ygu))
    return fail(NF4_EINVAL, "H and Ygu must be non-NULL and 16-byte aligned");
  return swiglu_pair_launch(X, m, Wgu, Tgu, Bg, Bu, r, s, H, Ygu, (hipStream_t)stream,
                            "qlora_swiglu_fwd_fused launch");
}

int qlora_swiglu_bwd(const void *dH, const void *X, int64_t m, const nf4_tensor *Wgu,
                     const void *Agu, const void *Bg, const void *Bu, int32_t r, float s,
                     const void *Ygu, const void *Tgu, void *dX, void *dAgu, void *dBg, void *dBu,
                     void *ws, size_t ws_bytes, void *stream) {
  size_t need = 0;
  int st = check_swiglu(X, m, Wgu, Agu, Bg, Bu, r, ws, ws_bytes, &need);
  if (st) return st;
  if (!dH || !aligned16(dH) || !Ygu || !aligned16(Ygu))
    return fail(NF4_EINVAL, "dH and Ygu must be non-NULL and 16-byte aligned");
  if (dX && !aligned16(dX)) return fail(NF4_EINVAL, "dX must be 16-byte aligned");
  if (r > 0) {
    if (!dAgu || !dBg || !dBu) return fail(NF4_EINVAL, "dAgu, dBg and dBu must be non-NULL when r > 0");
    if ((Tgu && !aligned16(Tgu)) || !aligned16(dAgu) || !aligned16(dBg) || !aligned16(dBu))
      return fail(NF4_EINVAL, "Tgu, dAgu, dBg and dBu must be 16-byte aligned");
  }
  if (!dX && r == 0) return ok();
  const int64_t n = Wgu->n / 2;
  const SwiWs lay = swi_ws(m, n, Wgu->k, r);
  hipStream_t sm = (hipStream_t)stream;
  char *base = (char *)ws;
  uint16_t *B2 = r > 0 ? (uint16_t *)base : nullptr;
  uint16_t *dY2 = (uint16_t *)(base + lay.b2);
  uint16_t *dB2 = r > 0 ? (uint16_t *)(base + lay.b2 + lay.dy2) : nullptr;
  hipError_t e = nf4q::launch_swiglu_bwd((const uint16_t *)dH, (const uint16_t *)Ygu, m, n, dY2, sm);
  if (e != hipSuccess) return hip_status(e, "qlora_swiglu_bwd launch");
  if (r > 0) {
    e = nf4q::launch_blockdiag((const uint16_t *)Bg, (const uint16_t *)Bu, n, r, B2, sm);
    if (e != hipSuccess) return hip_status(e, "qlora_swiglu_bwd launch");
  }
  st = qlora_bwd(dY2, X, m, Wgu, r > 0 ? Agu : nullptr, B2, 2 * r, s, r > 0 ? Tgu : nullptr, dX,
                 r > 0 ? dAgu : nullptr, dB2, base + lay.b2 + lay.dy2 + lay.db2, lay.bwd, stream);
  if (st) return st;
  if (r > 0)
    return hip_status(nf4q::launch_diagblocks(dB2, n, r, (uint16_t *)dBg, (uint16_t *)dBu, sm),
                      "qlora_swiglu_bwd launch");
  return ok();
}

int qlora_merge(const nf4_tensor *W, const void *A, const void *B, int32_t r, float s, void *Wout,
                void *stream) {
  int st = check_weight(W);
  if (st) return st;
  if (W->n * W->k >= (int64_t(1) << 32))
    return fail(NF4_EUNSUPPORTED, "n*k must be below 2^32 for qlora_merge");
  if (r < 0 || r > 128) return fail(NF4_EINVAL, "r must lie in [0, 128] (got %d)", r);
  if (r > 0) {
    if (!A || !B) return fail(NF4_EINVAL, "A and B must be non-NULL when r > 0");
    if (!aligned16(A) || !aligned16(B)) return fail(NF4_EINVAL, "A and B must be 16-byte aligned");
  }
  if (!Wout || !aligned16(Wout)) return fail(NF4_EINVAL, "Wout must be non-NULL and 16-byte aligned");
  return hip_status(nf4q::launch_merge(desc(W), (const uint16_t *)A, (const uint16_t *)B, r, s,
                                       tables(), (uint16_t *)Wout, (hipStream_t)stream),
                    "qlora_merge launch");
}

size_t qlora_moe_workspace_bytes(const int64_t *counts, int32_t E, int64_t n, int64_t k, int32_t r) {
  if (!counts || E < 1 || E > nf4q::kMaxExperts || n < 1 || k < 1 || r < 0) return 0;
  int64_t m = 0;
  for (int e = 0; e < E; ++e) m += std::max<int64_t>(counts[e], 0);
  return moe_ws_layout(m, E, n, k, r, false).total;
}

size_t qlora_moe_workspace_bytes_dev(int64_t m, int32_t E, int64_t n, int64_t k, int32_t r) {
  if (m < 1 || E < 1 || E > nf4q::kMaxExperts || n < 1 || k < 1 || r < 0) return 0;
  return moe_ws_layout(m, E, n, k, r, true).total;
}

}  // extern "C"

namespace {

// Every expert's tiles in one launch of the fused forward kernel.
int moe_fused_impl(const void *X, const Moe &mo, int32_t E, const nf4_tensor *W, const void *T,
                   const void *B, int32_t r, float s, void *Y, void *table, hipStream_t sm) {
  nf4q::GroupArgs gr;
  int st = moe_groups(mo, E, (mo.n + 255) / 256, &gr, 256, table, 0);
  if (st) return st;
  nf4q::GemmArgs g;
  g.a_side = (const uint16_t *)X;
  g.lda = W->k;
  g.lora_a = r > 0 ? (const uint16_t *)T : nullptr;
  g.lora_b = (const uint16_t *)B;
  g.w = desc(W);
  g.M = mo.mtotal;
  g.C = mo.n;
  g.R = W->k;
  g.r = r;
  g.s = s;
  g.out = (uint16_t *)Y;
  g.ldo = mo.n;
  g.t = tables();
  return hip_status(nf4q::launch_gemm_fwd_grouped(g, gr, sm), "grouped forward launch");
}

int check_moe_ws(const MoeWs &lay, void *ws, size_t ws_bytes) {
  if (ws_bytes < lay.total || (lay.total && !ws))
    return fail(NF4_EINVAL, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, lay.total);
  if (lay.total && !aligned16(ws)) return fail(NF4_EINVAL, "ws must be 16-byte aligned");
  return NF4_OK;
}

// T = X_e A_e^T for every expert's rows (one grouped row projection), then the fused launch.
int moe_fwd_impl(const void *X, const Moe &mo, int32_t E, const nf4_tensor *W, const void *A,
                 const void *B, int32_t r, float s, void *Y, void *T, void *ws, size_t ws_bytes,
                 hipStream_t sm) {
  if (!Y || !aligned16(Y)) return fail(NF4_EINVAL, "Y must be non-NULL and 16-byte aligned");
  if (r > 0 && (!T || !aligned16(T))) return fail(NF4_EINVAL, "T must be non-NULL and 16-byte aligned");
  const int64_t k = W->k;
  const bool dev = mo.dcounts != nullptr;
  const MoeWs lay = moe_ws_layout(mo.mtotal, E, mo.n, k, r, dev);
  int st = check_moe_ws(lay, ws, ws_bytes);
  if (st) return st;
  char *base = (char *)ws;
  void *table = dev ? base : nullptr;
  hipError_t he = moe_build_table(mo, E, k, table, sm);
  if (he != hipSuccess) return hip_status(he, "grouped forward plan launch");
  if (r > 0) {
    nf4q::GroupArgs g64;
    st = moe_groups(mo, E, 1, &g64, 64, table, 2);
    if (st) return st;
    const MoePlan pl = moe_plan(mo.mtotal, E, mo.n, k, r);
    he = nf4q::launch_rowproj_grouped((const uint16_t *)X, k, (const uint16_t *)A, (int64_t)r * k, k,
                                      mo.mtotal, k, r, pl.sp_k,
                                      (float *)(base + lay.table + lay.u + lay.bt + lay.t), (uint16_t *)T,
                                      g64, sm);
    if (he != hipSuccess) return hip_status(he, "grouped forward T launch");
  }
  return moe_fused_impl(X, mo, E, W, T, B, r, s, Y, table, sm);
}

int moe_bwd_impl(const void *dY, const void *X, const Moe &mo, int32_t E, const nf4_tensor *W,
                 const void *A, const void *B, int32_t r, float s, const void *T, void *dX, void *dA,
                 void *dB, void *ws, size_t ws_bytes, hipStream_t sm) {
  if (!dY || !aligned16(dY)) return fail(NF4_EINVAL, "dY must be non-NULL and 16-byte aligned");
  if (dX && !aligned16(dX)) return fail(NF4_EINVAL, "dX must be 16-byte aligned");
  if (r > 0) {
    if (!dA || !dB) return fail(NF4_EINVAL, "dA and dB must be non-NULL when r > 0");
    if ((T && !aligned16(T)) || !aligned16(dA) || !aligned16(dB))
      return fail(NF4_EINVAL, "T, dA and dB must be 16-byte aligned");
  }
  const int64_t k = W->k, n = mo.n;
  const bool dev = mo.dcounts != nullptr;
  const MoeWs lay = moe_ws_layout(mo.mtotal, E, n, k, r, dev);
  int st = check_moe_ws(lay, ws, ws_bytes);
  if (st) return st;
  if (!dX && r == 0) return ok();
  char *base = (char *)ws;
  void *table = dev ? base : nullptr;
  uint16_t *U = (uint16_t *)(base + lay.table);
  uint16_t *Bt = (uint16_t *)(base + lay.table + lay.u);
  float *part = (float *)(base + lay.table + lay.u + lay.bt + lay.t);
  const uint16_t *dy = (const uint16_t *)dY, *x = (const uint16_t *)X;
  const uint16_t *a = (const uint16_t *)A;
  hipError_t he = moe_build_table(mo, E, k, table, sm);
  if (he != hipSuccess) return hip_status(he, "grouped backward plan launch");
  // U = dY_e B_e for every expert's rows in one grouped row projection (and T = X_e A_e^T the
  // same way when the caller keeps none), B_e from one transpose of the stacked B: Bt [r, E n],
  // expert e's columns e n .. e n + n - 1
  const MoePlan pl = moe_plan(mo.mtotal, E, n, k, r);
  nf4q::GroupArgs g64;
  st = moe_groups(mo, E, 1, &g64, 64, table, 2);
  if (st) return st;
  if (r > 0) {
    he = nf4q::launch_transpose((const uint16_t *)B, E * n, r, Bt, sm);
    if (he != hipSuccess) return hip_status(he, "grouped backward transpose launch");
    if (!T) {
      uint16_t *Tw = (uint16_t *)(base + lay.table + lay.u + lay.bt);
      he = nf4q::launch_rowproj_grouped(x, k, a, (int64_t)r * k, k, mo.mtotal, k, r, pl.sp_k, part, Tw,
                                        g64, sm);
      if (he != hipSuccess) return hip_status(he, "grouped backward T launch");
      T = Tw;
    }
    he = nf4q::launch_rowproj_grouped(dy, n, Bt, n, E * n, mo.mtotal, n, r, pl.sp_n, part, U, g64, sm);
    if (he != hipSuccess) return hip_status(he, "grouped backward U launch");
  }
  // dX of every expert in one launch
  if (dX) {
    nf4q::GroupArgs gr;
    st = moe_groups(mo, E, (k + 255) / 256, &gr, 256, table, 1);
    if (st) return st;
    nf4q::GemmArgs g;
    g.a_side = dy;
    g.lda = n;
    g.lora_a = U;
    g.lora_b = a;
    g.w = desc(W);
    g.M = mo.mtotal;
    g.C = k;
    g.R = n;
    g.r = r;
    g.s = s;
    g.out = (uint16_t *)dX;
    g.ldo = k;
    g.t = tables();
    // split the tiles of a last, partly filled round (one workgroup per CU at a time)
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) {
      gr.width = std::min(cus, nf4q::kDxMaxWidth);
      gr.smax = nf4q::kDxMaxPieces;
      gr.part = part;
    }
    he = nf4q::launch_gemm_dx_grouped(g, gr, sm);
    if (he != hipSuccess) return hip_status(he, "grouped backward dX launch");
  }
  // dA_e = s U_e^T X_e, dB_e = s dY_e^T T_e over each expert's own rows, every expert in one
  // launch each (an expert with no rows sums nothing: zero gradients)
  if (r > 0) {
    he = nf4q::launch_mreduce_grouped(U, x, k, k, r, s, pl.sa, part, (uint16_t *)dA, false, g64, sm);
    if (he != hipSuccess) return hip_status(he, "grouped backward dA launch");
    he = nf4q::launch_mreduce_grouped((const uint16_t *)T, dy, n, n, r, s, pl.sb, part, (uint16_t *)dB,
                                      true, g64, sm);
    if (he != hipSuccess) return hip_status(he, "grouped backward dB launch");
  }
  return ok();
}

}  // namespace

extern "C" {

int qlora_moe_fwd_fused(const void *X, const int64_t *counts, int32_t E, const nf4_tensor *W,
                        const void *T, const void *B, int32_t r, float s, void *Y, void *stream) {
  Moe mo;
  int st = check_moe(X, counts, E, W, T, B, r, &mo);   // T [sum(counts), r] in A's place
  if (st) return st;
  if (!Y || !aligned16(Y)) return fail(NF4_EINVAL, "Y must be non-NULL and 16-byte aligned");
  return moe_fused_impl(X, mo, E, W, T, B, r, s, Y, nullptr, (hipStream_t)stream);
}

int qlora_moe_fwd(const void *X, const int64_t *counts, int32_t E, const nf4_tensor *W,
                  const void *A, const void *B, int32_t r, float s, void *Y, void *T, void *ws,
                  size_t ws_bytes, void *stream) {
  Moe mo;
  int st = check_moe(X, counts, E, W, A, B, r, &mo);
  if (st) return st;
  return moe_fwd_impl(X, mo, E, W, A, B, r, s, Y, T, ws, ws_bytes, (hipStream_t)stream);
}

int qlora_moe_fwd_dev(const void *X, int64_t m, const int64_t *counts, int32_t E, const nf4_tensor *W,
                      const void *A, const void *B, int32_t r, float s, void *Y, void *T, void *ws,
                      size_t ws_bytes, void *stream) {
  Moe mo;
  int st = check_moe_dev(X, m, counts, E, W, A, B, r, &mo);
  if (st) return st;
  return moe_fwd_impl(X, mo, E, W, A, B, r, s, Y, T, ws, ws_bytes, (hipStream_t)stream);
}

int qlora_moe_bwd(const void *dY, const void *X, const int64_t *counts, int32_t E,
                  const nf4_tensor *W, const void *A, const void *B, int32_t r, float s,
                  const void *T, void *dX, void *dA, void *dB, void *ws, size_t ws_bytes,
                  void *stream) {
  Moe mo;
  int st = check_moe(X, counts, E, W, A, B, r, &mo);
  if (st) return st;
  return moe_bwd_impl(dY, X, mo, E, W, A, B, r, s, T, dX, dA, dB, ws, ws_bytes, (hipStream_t)stream);
}

int qlora_moe_bwd_dev(const void *dY, const void *X, int64_t m, const int64_t *counts, int32_t E,
                      const nf4_tensor *W, const void *A, const void *B, int32_t r, float s,
                      const void *T, void *dX, void *dA, void *dB, void *ws, size_t ws_bytes,
                      void *stream) {
  Moe mo;
  int st = check_moe_dev(X, m, counts, E, W, A, B, r, &mo);
  if (st) return st;
  return moe_bwd_impl(dY, X, mo, E, W, A, B, r, s, T, dX, dA, dB, ws, ws_bytes, (hipStream_t)stream);
}

int qlora_bwd_dx(const void *dY, int64_t m, const nf4_tensor *W, const void *U, const void *A,
                 int32_t r, float s, void *dX, void *stream) {
  // dY [m, n] plays the part of X in the layer checks, U [m, r] and A [r, k] that of A and B
  int st = check_layer(dY, m, W, U, A, r);
  if (st) return st;
  if (!dX || !aligned16(dX)) return fail(NF4_EINVAL, "dX must be non-NULL and 16-byte aligned");
  return hip_status(launch_dx((const uint16_t *)dY, m, W, (const uint16_t *)U, (const uint16_t *)A,
                              r, s, (uint16_t *)dX, (hipStream_t)stream),
                    "qlora_bwd_dx launch");
}

}  // extern "C"
