// Host side of the C ABI: argument validation, work partitioning, workspace layout and
// launches. Every entry point validates its arguments completely before the first HIP call.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "qg_kernels.hpp"
#include "qgalore.h"

using qg::LayerDev;
using qg::StepArgs;

namespace {

thread_local std::string g_last_error;

qg_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
  return QG_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
bool finite(float x) { return std::isfinite(x); }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int kK = 32;       // K per stage of the MFMA kernels
constexpr int kKSlab = 64;   // split-K slab granularity: whole K stages of both tile sizes

qg_status device_present() {
  static int cached = -1;
  if (cached < 0) {
    int n = 0;
    const hipError_t e = hipGetDeviceCount(&n);
    cached = (e == hipSuccess && n > 0) ? 1 : 0;
  }
  return cached ? QG_OK : QG_ERR_NO_DEVICE;
}

// Kernels address every tensor of a layer through 32-bit buffer offsets: the fp32 ones
// (R: r x n, U: m x n) must stay below 2 GiB, hence m*n and r*n below 2^29 elements; the
// projection (m x r, up to 4 bytes per element where a kernel stages it) likewise.
constexpr int64_t kMaxElems = int64_t(1) << 29;

qg_status check_shape(int64_t m, int64_t n, int64_t r) {
  if (m < 1 || n < 1 || r < 1 || m > kMaxDim || n > kMaxDim || r > kMaxDim) return QG_ERR_SHAPE;
  if (r > m || r % 8 != 0) return QG_ERR_SHAPE;
  if (m * n > kMaxElems || r * n > kMaxElems || m * r > kMaxElems) return QG_ERR_SHAPE;
  return QG_OK;
}

// Tile configuration of the MFMA kernels: the larger tiles once the rank exceeds 128.
bool big_tiles(int64_t r) { return r > 128; }
int64_t proj_tiles(int64_t n, int64_t r) {
  return cdiv(r, qg::kProjTileM) * cdiv(n, qg::kProjTileN);
}
// With one K split and rows of whole 256-element groups, each projection tile row is a
// complete Adam group and the projection kernel finishes Adam itself.
bool fused_adam(int64_t n, int split) { return split == 1 && n % qg::kGroup == 0; }

// K-splits of the projection R = P~^T G for one layer launched on its own: enough
// workgroups to cover the chip, bounded so the fp32 partial sums stay small next to G.
int choose_split(int64_t m, int64_t n, int64_t r) {
  const int64_t tiles = proj_tiles(n, r);
  const int64_t kchunks = cdiv(m, kKSlab);
  int64_t s = cdiv(512, tiles);
  s = std::min<int64_t>(s, std::max<int64_t>(1, m / (8 * r)));
  s = std::min<int64_t>(s, kchunks);
  s = std::max<int64_t>(s, 1);
  const int64_t kslab = cdiv(kchunks, s) * kKSlab;
  return (int)cdiv(m, kslab);
}
int64_t kslab_for(int64_t m, int split) { return cdiv(cdiv(m, kKSlab), split) * kKSlab; }

// Whether a layer's INT4 projection is dequantized inside the MFMA kernels' stagers (no bf16
// copy in the workspace, no dequant pass): the method's INT4 format, a rank whose tile rows
// lie inside single scale groups, and the INLINE mode. The automatic choice is the separate
// pass: on MI355X it is the faster of the two at every rank measured (the stagers convert
// each projection element once per column tile, n / 256 times a step, where the pass
// converts it once), and INLINE is the choice that saves the workspace's bf16 copy.
bool p_inline(int32_t p_format, int64_t r, int32_t mode) {
  return p_format == QG_P_INT4 && qg::inline_rank(r) && mode == QG_DEQUANT_INLINE;
}
bool valid_dequant_mode(int32_t mode) {
  return mode == QG_DEQUANT_AUTO || mode == QG_DEQUANT_INLINE || mode == QG_DEQUANT_PASS;
}

// Row pitch of N~ in the workspace (elements): 16-byte aligned rows for any n.
int64_t n_pitch(int64_t n) { return round_up(n, 8); }

// alpha = 2^k with -126 < k <= 0. Scaling by such a power of two is exact in fp32 except for
// results in the subnormal range, so fl(fl(alpha S) * inv) = fl(S * fl(alpha inv)) whenever
// alpha S is normal or zero and alpha inv is normal, zero or infinite; elsewhere the two differ
// by less than 2^-21 (one rounding in the subnormal range, at most 2^-150, times an inv below
// 2^128, plus the roundings of the two products).
bool alpha_folds(float alpha) {
  int e = 0;
  const float f = std::frexp(alpha, &e);   // alpha = f 2^e, 0.5 <= f < 1
  return f == 0.5f && e - 1 <= 0 && e - 1 > -126;
}

// Per-layer workspace: split-K partial sums of R (fp32; absent when Adam is fused into the
// projection), the bf16 update N~ (r x n) and, for projections the MFMA kernels do not
// dequantize themselves, the bf16 dequantized projection P~ (m x r) that both read.
struct WsLayout {
  int64_t rpitch, off_r, off_n, off_p, bytes;
};
WsLayout ws_layout(int64_t m, int64_t n, int64_t r, int split, int64_t base,
                   int32_t p_format = QG_P_INT4, bool inl = false) {
  WsLayout w;
  w.rpitch = round_up(r * n, 64);
  w.off_r = base;
  const int64_t rbytes = fused_adam(n, split) ? 0 : (int64_t)split * w.rpitch * 4;
  w.off_n = base + round_up(rbytes, 256);
  w.off_p = w.off_n + round_up(r * n_pitch(n) * 2, 256);
  // a bf16 projection is staged from the caller's tensor, an inline INT4 one from its codes:
  // no dequantized copy
  const bool copy = p_format != QG_P_BF16 && !inl;
  w.bytes = (w.off_p - base) + (copy ? round_up(m * r * 2, 256) : 0);
  return w;
}

struct Hyper {
  float lr, beta1, beta2, eps, alpha;
};
qg_status check_hyper(const qg_layer_desc* d) {
  if (!finite(d->lr) || !finite(d->beta1) || !finite(d->beta2) || !finite(d->eps) ||
      !finite(d->alpha))
    return QG_ERR_ARG;
  if (d->beta1 < 0.f || d->beta1 >= 1.f || d->beta2 < 0.f || d->beta2 >= 1.f || d->eps < 0.f)
    return QG_ERR_ARG;
  return QG_OK;
}

bool valid_format(int32_t f) { return f == QG_P_INT4 || f == QG_P_INT8 || f == QG_P_BF16; }

// A projection in format f: codes with group scales (INT4, INT8: 4-byte aligned) or bf16
// values that the MFMA kernels read directly (16-byte aligned, no scales).
qg_status check_p(int32_t f, const void* P_q, const float* P_scale) {
  if (!valid_format(f)) return QG_ERR_ARG;
  if (!P_q || (f != QG_P_BF16 && !P_scale)) return QG_ERR_NULL;
  if (!aligned(P_q, f == QG_P_BF16 ? 16 : 4) || !aligned(P_scale, 4)) return QG_ERR_ALIGN;
  return QG_OK;
}

qg_status check_layer(const qg_layer_desc* d, const uint16_t* G, int8_t* W_q, const float* W_scale,
                      const uint8_t* P_q, const float* P_scale, int8_t* M_q, int8_t* V_q) {
  if (!d || !G || !W_q || !W_scale || !M_q || !V_q || !d->M_scale || !d->V_scale)
    return QG_ERR_NULL;
  qg_status st = check_shape(d->m, d->n, d->r);
  if (st != QG_OK) return st;
  if ((st = check_p(d->p_format, P_q, P_scale)) != QG_OK) return st;
  if (!valid_dequant_mode(d->dequant_mode)) return QG_ERR_ARG;
  if (!aligned(G, 16) || !aligned(W_q, 16) || !aligned(M_q, 16) || !aligned(V_q, 16) ||
      !aligned(d->R_out, 16) || !aligned(d->U_out, 16) || !aligned(W_scale, 4) ||
      !aligned(d->M_scale, 4) || !aligned(d->V_scale, 4))
    return QG_ERR_ALIGN;
  return check_hyper(d);
}

qg_status check_step(int64_t step) {
  return (step >= 1 && step < (int64_t(1) << 32)) ? QG_OK : QG_ERR_ARG;
}

// Adam's per-step constants: computed in double from the fp32 hyperparameters and rounded
// once to fp32 (pow from the C library).
void step_constants(float beta1, float beta2, int64_t step, StepArgs& a) {
  const double b1 = beta1, b2 = beta2;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.c1 = (float)(1.0 - b1);
  a.c2 = (float)(1.0 - b2);
  a.bc1 = (float)(1.0 - std::pow(b1, (double)step));
  a.bc2 = (float)(1.0 - std::pow(b2, (double)step));
  // reciprocals of the fp32 bias corrections, correctly rounded in fp64 (the kernels divide
  // by bc1 and bc2 through them); bc is positive for 0 <= beta < 1 and step >= 1
  a.ibc1 = 1.0 / (double)a.bc1;
  a.ibc2 = 1.0 / (double)a.bc2;
  a.step = (uint32_t)step;
}

LayerDev make_layer(const qg_layer_desc* d, const uint16_t* G, int8_t* W_q, const float* W_scale,
                    const uint8_t* P_q, const float* P_scale, int8_t* M_q, int8_t* V_q,
                    int split, int64_t ws_base, bool big) {
  LayerDev L;
  std::memset(&L, 0, sizeof(L));
  L.G = G;
  L.Wq = W_q;
  L.Ws = W_scale;
  L.Pq = P_q;
  L.Ps = P_scale;
  L.Mq = M_q;
  L.Ms = d->M_scale;
  L.Vq = V_q;
  L.Vs = d->V_scale;
  L.R_out = d->R_out;
  L.U_out = d->U_out;
  L.m = d->m;
  L.n = d->n;
  L.r = d->r;
  L.ldn = n_pitch(d->n);
  const bool inl = p_inline(d->p_format, d->r, d->dequant_mode);
  const WsLayout w = ws_layout(d->m, d->n, d->r, split, ws_base, d->p_format, inl);
  L.rpitch = w.rpitch;
  L.off_r = w.off_r;
  L.off_n = w.off_n;
  L.off_p = w.off_p;
  L.layer_id = d->layer_id;
  L.p_format = d->p_format;
  L.p_inline = inl ? 1 : 0;
  L.split = split;
  L.fuse_adam = fused_adam(d->n, split) ? 1 : 0;
  L.kslab = (int32_t)kslab_for(d->m, split);
  L.p_tiles_i = (int32_t)cdiv(d->r, qg::kProjTileM);
  L.p_tiles_j = (int32_t)cdiv(d->n, qg::kProjTileN);
  L.b_tiles_i = (int32_t)cdiv(d->m, qg::kBackTileM(big));
  L.b_tiles_j = (int32_t)cdiv(d->n, qg::kBackTileN(big));
  L.lr = d->lr;
  L.eps = d->eps;
  L.alpha = d->alpha;
  L.fold_alpha = (d->U_out == nullptr && alpha_folds(d->alpha)) ? 1 : 0;
  return L;
}

int grid_project(const LayerDev& L) { return L.split * L.p_tiles_i * L.p_tiles_j; }
int grid_adam(const LayerDev& L) {
  return L.fuse_adam ? 0 : (int)cdiv(cdiv(L.r * L.n, qg::kGroup), 4);
}
int grid_back(const LayerDev& L) { return L.b_tiles_i * L.b_tiles_j; }
int grid_dequant(const LayerDev& L) {
  return (L.p_format == QG_P_BF16 || L.p_inline) ? 0
                                                 : (int)cdiv(L.m * L.r, qg::kThreads * qg::kDeqCodes);
}

qg_status launch_step(const StepArgs& a, const int grid[4], bool big, int pmode, bool fold,
                      hipStream_t s) {
  hipError_t e = hipSuccess;
  if (grid[3] > 0 && (e = qg::launch_dequant(a, grid[3], s)) != hipSuccess)
    return hip_fail(e, "dequant kernel launch");
  e = qg::launch_project(a, grid[0], pmode, s);
  if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
  if (grid[1] > 0 && (e = qg::launch_adam(a, grid[1], s)) != hipSuccess)
    return hip_fail(e, "Adam kernel launch");
  e = qg::launch_backproject(a, grid[2], big, pmode, fold, s);
  if (e != hipSuccess) return hip_fail(e, "back-projection kernel launch");
  return QG_OK;
}

}  // namespace

// ===================================================================== single layer ===

extern "C" size_t qgalore_workspace_bytes(int64_t m, int64_t n, int64_t r) {
  if (check_shape(m, n, r) != QG_OK) return 0;
  return (size_t)ws_layout(m, n, r, choose_split(m, n, r), 0).bytes;
}

extern "C" size_t qgalore_layer_workspace_bytes(const qg_layer_desc* d) {
  if (!d || check_shape(d->m, d->n, d->r) != QG_OK || !valid_format(d->p_format) ||
      !valid_dequant_mode(d->dequant_mode))
    return 0;
  return (size_t)ws_layout(d->m, d->n, d->r, choose_split(d->m, d->n, d->r), 0, d->p_format,
                           p_inline(d->p_format, d->r, d->dequant_mode))
      .bytes;
}

extern "C" qg_status qgalore_step(const qg_layer_desc* d, const uint16_t* G, int8_t* W_q,
                                  const float* W_scale, const uint8_t* P_q, const float* P_scale,
                                  int8_t* M_q, int8_t* V_q, int64_t step, uint64_t seed) {
  qg_status st = check_layer(d, G, W_q, W_scale, P_q, P_scale, M_q, V_q);
  if (st != QG_OK) return st;
  if ((st = check_step(step)) != QG_OK) return st;
  const int split = choose_split(d->m, d->n, d->r);
  const WsLayout w = ws_layout(d->m, d->n, d->r, split, 0, d->p_format,
                               p_inline(d->p_format, d->r, d->dequant_mode));
  if (!d->workspace) return QG_ERR_NULL;
  if (!aligned(d->workspace, 16)) return QG_ERR_ALIGN;
  if (d->workspace_bytes < (size_t)w.bytes) return QG_ERR_WORKSPACE;
  if ((st = device_present()) != QG_OK) return st;

  StepArgs a;
  std::memset(&a, 0, sizeof(a));
  const bool big = big_tiles(d->r);
  a.one = make_layer(d, G, W_q, W_scale, P_q, P_scale, M_q, V_q, split, 0, big);
  a.ws = static_cast<char*>(d->workspace);
  a.table = nullptr;
  a.wg_layer = nullptr;
  step_constants(d->beta1, d->beta2, step, a);
  a.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  a.seed_hi = (uint32_t)(seed >> 32);
  const int grid[4] = {grid_project(a.one), grid_adam(a.one), grid_back(a.one),
                       grid_dequant(a.one)};
  return launch_step(a, grid, big, a.one.p_inline ? qg::kPInline : qg::kPStaged,
                     a.one.fold_alpha != 0, static_cast<hipStream_t>(d->stream));
}

// ============================================= single layer without a workspace argument ===
// For callers that cannot allocate device memory: the step's scratch (split-K partial sums of
// R, N~ and the dequantized projection) lives in a file-scope device array of fixed size, one
// per GPU, kept until the process ends. Every call on a GPU shares that GPU's array, so calls
// that overlap on one GPU (different streams, or threads) race on it. The step writes every
// scratch element it later reads, so nothing needs clearing between calls.
constexpr size_t kNoAllocScratchBytes = QG_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current GPU's scratch array, looked up once per device (with
// that device current). The array's name on the host is only a stand-in for the symbol.
qg_status device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "device index beyond the scratch table";
    return QG_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QG_OK;
}
}  // namespace

extern "C" qg_status qgalore_step_noalloc(const qg_layer_desc* d, const uint16_t* G,
                                          int8_t* W_q, const float* W_scale, const uint8_t* P_q,
                                          const float* P_scale, int8_t* M_q, int8_t* V_q,
                                          int64_t step, uint64_t seed) {
  qg_status st = check_layer(d, G, W_q, W_scale, P_q, P_scale, M_q, V_q);
  if (st != QG_OK) return st;
  if ((st = check_step(step)) != QG_OK) return st;
  const int split = choose_split(d->m, d->n, d->r);
  const WsLayout w = ws_layout(d->m, d->n, d->r, split, 0, d->p_format,
                               p_inline(d->p_format, d->r, d->dequant_mode));
  if ((size_t)w.bytes > kNoAllocScratchBytes) {
    g_last_error = "layer needs " + std::to_string(w.bytes) + " bytes of scratch, more than the " +
                   std::to_string(kNoAllocScratchBytes) + " of the no-alloc step";
    return QG_ERR_WORKSPACE;
  }
  if ((st = device_present()) != QG_OK) return st;
  void* ws = nullptr;
  if ((st = device_scratch(&ws)) != QG_OK) return st;

  StepArgs a;
  std::memset(&a, 0, sizeof(a));
  const bool big = big_tiles(d->r);
  a.one = make_layer(d, G, W_q, W_scale, P_q, P_scale, M_q, V_q, split, 0, big);
  a.ws = static_cast<char*>(ws);
  step_constants(d->beta1, d->beta2, step, a);
  a.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  a.seed_hi = (uint32_t)(seed >> 32);
  const int grid[4] = {grid_project(a.one), grid_adam(a.one), grid_back(a.one),
                       grid_dequant(a.one)};
  return launch_step(a, grid, big, a.one.p_inline ? qg::kPInline : qg::kPStaged,
                     a.one.fold_alpha != 0, static_cast<hipStream_t>(d->stream));
}

// ========================================================================= grouped ===

struct qg_plan {
  std::vector<LayerDev> layers;
  LayerDev* d_table = nullptr;
  int32_t* d_map[4] = {nullptr, nullptr, nullptr, nullptr};
  int grid[4] = {0, 0, 0, 0};
  int64_t ws_bytes = 0;
  float beta1 = 0.f, beta2 = 0.f;
  bool big = false;
  int pmode = qg::kPStaged;   // projection paths of the MFMA launches (all staged / inline / mix)
  bool fold = false;          // every layer has fold_alpha
  int device = 0;
  std::vector<hipEvent_t> events;   // 5 per recorded step when timing is enabled
  int timing_cap = 0;
  int timing_used = 0;
  // kept dequantized projections (qgalore_plan_cache_proj): layers whose P changed since
  // the last step, and the workspace that holds the others' bf16 copies
  bool cache_proj = false;
  std::vector<uint8_t> proj_dirty;
  const void* deq_ws = nullptr;
};

namespace {
hipError_t free_events(qg_plan* p) {
  hipError_t e = hipSuccess;
  for (hipEvent_t ev : p->events) {
    const hipError_t e2 = hipEventDestroy(ev);
    if (e == hipSuccess) e = e2;
  }
  p->events.clear();
  p->timing_cap = 0;
  p->timing_used = 0;
  return e;
}
}  // namespace

extern "C" qg_status qgalore_plan_create(const qg_layer* layers, int32_t count, qg_plan** out) {
  if (!layers || !out) return QG_ERR_NULL;
  *out = nullptr;
  if (count < 1) return QG_ERR_ARG;
  for (int32_t l = 0; l < count; ++l) {
    const qg_layer& x = layers[l];
    qg_status st = check_layer(&x.desc, x.G, x.W_q, x.W_scale, x.P_q, x.P_scale, x.M_q, x.V_q);
    if (st != QG_OK) return st;
    if (x.desc.beta1 != layers[0].desc.beta1 || x.desc.beta2 != layers[0].desc.beta2)
      return QG_ERR_ARG;
  }
  qg_status st = device_present();
  if (st != QG_OK) return st;

  // One tile configuration for the whole set (by its largest rank), and one K-split for every
  // layer unless the set has too few projection tiles to fill the chip.
  int64_t rmax = 0;
  for (int32_t l = 0; l < count; ++l) rmax = std::max<int64_t>(rmax, layers[l].desc.r);
  const bool big = big_tiles(rmax);
  int64_t tiles = 0;
  for (int32_t l = 0; l < count; ++l) tiles += proj_tiles(layers[l].desc.n, layers[l].desc.r);
  const bool grouped_fill = tiles >= 1024;

  qg_plan* p = new (std::nothrow) qg_plan();
  if (!p) return QG_ERR_ARG;
  p->big = big;
  p->beta1 = layers[0].desc.beta1;
  p->beta2 = layers[0].desc.beta2;
  int64_t ws = 0;
  int64_t base[4] = {0, 0, 0, 0};
  std::vector<int32_t> map[4];
  for (int32_t l = 0; l < count; ++l) {
    const qg_layer& x = layers[l];
    const int split = grouped_fill ? 1 : choose_split(x.desc.m, x.desc.n, x.desc.r);
    LayerDev L = make_layer(&x.desc, x.G, x.W_q, x.W_scale, x.P_q, x.P_scale, x.M_q, x.V_q,
                            split, ws, big);
    ws += ws_layout(x.desc.m, x.desc.n, x.desc.r, split, ws, x.desc.p_format, L.p_inline != 0)
              .bytes;
    const int g[4] = {grid_project(L), grid_adam(L), grid_back(L), grid_dequant(L)};
    for (int k = 0; k < 4; ++k) {
      if (base[k] + g[k] > kMaxDim) {
        delete p;
        return QG_ERR_SHAPE;
      }
      L.wg_base[k] = (int32_t)base[k];
      map[k].insert(map[k].end(), (size_t)g[k], l);
      base[k] += g[k];
    }
    p->layers.push_back(L);
  }
  p->ws_bytes = ws;
  for (int k = 0; k < 4; ++k) p->grid[k] = (int)base[k];
  int n_inline = 0;
  for (const LayerDev& L : p->layers) n_inline += L.p_inline;
  p->pmode = n_inline == 0 ? qg::kPStaged : n_inline == count ? qg::kPInline : qg::kPMixed;
  int n_fold = 0;
  for (const LayerDev& L : p->layers) n_fold += L.fold_alpha;
  p->fold = n_fold == count;
  p->proj_dirty.assign((size_t)count, 1);

  hipError_t e = hipGetDevice(&p->device);
  if (e == hipSuccess) e = hipMalloc(&p->d_table, sizeof(LayerDev) * count);
  for (int k = 0; k < 4 && e == hipSuccess; ++k)
    e = hipMalloc(&p->d_map[k], sizeof(int32_t) * std::max<size_t>(1, map[k].size()));
  if (e == hipSuccess)
    e = hipMemcpy(p->d_table, p->layers.data(), sizeof(LayerDev) * count, hipMemcpyHostToDevice);
  for (int k = 0; k < 4 && e == hipSuccess; ++k)
    if (!map[k].empty())
      e = hipMemcpy(p->d_map[k], map[k].data(), sizeof(int32_t) * map[k].size(),
                    hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    qgalore_plan_destroy(p);
    return hip_fail(e, "plan upload");
  }
  *out = p;
  return QG_OK;
}

extern "C" size_t qgalore_plan_workspace_bytes(const qg_plan* p) {
  return p ? (size_t)p->ws_bytes : 0;
}

extern "C" qg_status qgalore_plan_step(qg_plan* p, int64_t step, uint64_t seed, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (!p || !workspace) return QG_ERR_NULL;
  qg_status st = check_step(step);
  if (st != QG_OK) return st;
  if (!aligned(workspace, 16)) return QG_ERR_ALIGN;
  if (workspace_bytes < (size_t)p->ws_bytes) return QG_ERR_WORKSPACE;
  StepArgs a;
  std::memset(&a, 0, sizeof(a));
  a.ws = static_cast<char*>(workspace);
  a.table = p->d_table;
  step_constants(p->beta1, p->beta2, step, a);
  a.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  a.seed_hi = (uint32_t)(seed >> 32);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = nullptr;
  if (p->timing_used < p->timing_cap) ev = &p->events[5 * p->timing_used++];
  hipError_t e = hipSuccess;
  if (ev) e = hipEventRecord(ev[0], s);
  if (e != hipSuccess) return hip_fail(e, "timing event");
  a.wg_layer = p->d_map[3];
  // bf16 projections are staged directly: their layers have no dequant workgroups. With
  // kept projections, only the layers marked changed are dequantized, one launch each while
  // they are few.
  if (p->grid[3] > 0) {
    const bool all = !p->cache_proj || p->deq_ws != workspace;
    std::vector<int32_t> dirty;
    if (!all)
      for (size_t l = 0; l < p->layers.size(); ++l)
        if (p->proj_dirty[l] && grid_dequant(p->layers[l]) > 0) dirty.push_back((int32_t)l);
    if (all || dirty.size() > 32) {
      e = qg::launch_dequant(a, p->grid[3], s);
    } else {
      for (const int32_t l : dirty) {
        StepArgs one = a;
        one.table = nullptr;
        one.wg_layer = nullptr;
        one.one = p->layers[(size_t)l];
        if ((e = qg::launch_dequant(one, grid_dequant(one.one), s)) != hipSuccess) break;
      }
    }
    if (e != hipSuccess) return hip_fail(e, "dequant kernel launch");
  }
  if (p->cache_proj) {
    std::fill(p->proj_dirty.begin(), p->proj_dirty.end(), 0);
    p->deq_ws = workspace;
  }
  if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return hip_fail(e, "timing event");
  a.wg_layer = p->d_map[0];
  e = qg::launch_project(a, p->grid[0], p->pmode, s);
  if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
  if (ev && (e = hipEventRecord(ev[2], s)) != hipSuccess) return hip_fail(e, "timing event");
  a.wg_layer = p->d_map[1];
  // layers whose Adam ran inside the projection kernel have no Adam workgroups
  if (p->grid[1] > 0 && (e = qg::launch_adam(a, p->grid[1], s)) != hipSuccess)
    return hip_fail(e, "Adam kernel launch");
  if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return hip_fail(e, "timing event");
  a.wg_layer = p->d_map[2];
  e = qg::launch_backproject(a, p->grid[2], p->big, p->pmode, p->fold, s);
  if (e != hipSuccess) return hip_fail(e, "back-projection kernel launch");
  if (ev && (e = hipEventRecord(ev[4], s)) != hipSuccess) return hip_fail(e, "timing event");
  return QG_OK;
}

extern "C" qg_status qgalore_plan_cache_proj(qg_plan* p, int32_t enable) {
  if (!p) return QG_ERR_NULL;
  if (enable != 0 && enable != 1) return QG_ERR_ARG;
  p->cache_proj = enable == 1;
  p->deq_ws = nullptr;   // the next step dequantizes every layer
  std::fill(p->proj_dirty.begin(), p->proj_dirty.end(), 1);
  return QG_OK;
}

extern "C" qg_status qgalore_plan_proj_changed(qg_plan* p, int32_t layer) {
  if (!p) return QG_ERR_NULL;
  if (layer < 0 || (size_t)layer >= p->proj_dirty.size()) return QG_ERR_ARG;
  p->proj_dirty[(size_t)layer] = 1;
  return QG_OK;
}

extern "C" qg_status qgalore_plan_enable_timing(qg_plan* p, int32_t max_steps) {
  if (!p) return QG_ERR_NULL;
  if (max_steps < 0 || max_steps > 100000) return QG_ERR_ARG;
  hipError_t e = free_events(p);
  if (e != hipSuccess) return hip_fail(e, "timing event destroy");
  p->events.resize(5 * (size_t)max_steps);
  for (size_t k = 0; k < p->events.size(); ++k) {
    e = hipEventCreate(&p->events[k]);
    if (e != hipSuccess) {
      p->events.resize(k);
      free_events(p);
      return hip_fail(e, "timing event create");
    }
  }
  p->timing_cap = max_steps;
  p->timing_used = 0;
  return QG_OK;
}

extern "C" qg_status qgalore_plan_kernel_times(qg_plan* p, float out_ms[4], int32_t* steps) {
  if (!p || !out_ms) return QG_ERR_NULL;
  double acc[4] = {0, 0, 0, 0};
  for (int k = 0; k < p->timing_used; ++k) {
    hipEvent_t* ev = &p->events[5 * k];
    hipError_t e = hipEventSynchronize(ev[4]);
    for (int j = 0; j < 4 && e == hipSuccess; ++j) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, ev[j], ev[j + 1]);
      acc[j] += ms;
    }
    if (e != hipSuccess) return hip_fail(e, "timing event read");
  }
  const int used = p->timing_used;
  for (int j = 0; j < 4; ++j) out_ms[j] = used ? (float)(acc[j] / used) : 0.f;
  if (steps) *steps = used;
  p->timing_used = 0;
  return QG_OK;
}

extern "C" qg_status qgalore_plan_destroy(qg_plan* p) {
  if (!p) return QG_ERR_NULL;
  hipError_t e = free_events(p);
  if (p->d_table) e = hipFree(p->d_table);
  for (int k = 0; k < 4; ++k)
    if (p->d_map[k]) {
      const hipError_t e2 = hipFree(p->d_map[k]);
      if (e == hipSuccess) e = e2;
    }
  delete p;
  return e == hipSuccess ? QG_OK : hip_fail(e, "plan free");
}

// ============================================================ subspace similarity ===

namespace {
// Newton-Schulz schedule of the similarity test: quintic iterations that lift small singular
// values, then cubic ones that converge them to 1 (bf16 operands, then hi/lo split operands).
constexpr int kNsQuintic = 7;
constexpr int kNsCubicBf16 = 4;
constexpr int kNsCubicSplit = 1;

static_assert(kNsCubicBf16 >= 1, "the last bf16 step hands X over in fp32");

struct CosLayout {
  int split, tiles, ctiles, nblk;
  int64_t off_part, off_c, off_x, off_xn, off_a, off_xb0, off_xb1, off_ab, off_bb, off_blk,
      off_norm, stride;
};
CosLayout cos_layout(int64_t r) {
  CosLayout c;
  c.tiles = (int)cdiv(r, qg::kCosTile);
  // the C product: edge cos_ctile(r); enough K splits for about 64 (64-edge tiles) or 256
  // (128-edge tiles) workgroups per pair, at most 8
  c.ctiles = (int)cdiv(r, qg::cos_ctile((int)r));
  const int64_t want = qg::cos_ctile((int)r) == qg::kCosCTile ? 256 : 64;
  c.split = (int)std::min<int64_t>(8, std::max<int64_t>(1, cdiv(want, (int64_t)c.ctiles * c.ctiles)));
  const int64_t n2 = r * r;
  c.nblk = (int)cdiv(n2, (int64_t)qg::kThreads * 4);
  const int64_t mat = round_up(n2 * 4, 256);
  c.off_part = 0;
  c.off_c = round_up((int64_t)c.split * n2 * 4, 256);
  c.off_x = c.off_c + mat;
  c.off_xn = c.off_x + mat;
  c.off_a = c.off_xn + mat;
  const int64_t matb = round_up(n2 * 2, 256);
  c.off_xb0 = c.off_a + mat;
  c.off_xb1 = c.off_xb0 + matb;
  c.off_ab = c.off_xb1 + matb;
  c.off_bb = c.off_ab + matb;
  c.off_blk = c.off_bb + matb;
  c.off_norm = c.off_blk + round_up((int64_t)c.nblk * 4, 256);
  c.stride = c.off_norm + 256;
  return c;
}

qg_status check_proj(const qg_proj* p) {
  if (!p) return QG_ERR_NULL;
  qg_status st = check_p(p->format, p->q, p->scale);
  if (st != QG_OK) return st;
  if (p->m < 1 || p->r < 1 || p->m > kMaxDim || p->r > 8192 || p->r > p->m || p->r % 8 != 0)
    return QG_ERR_SHAPE;
  return QG_OK;
}

qg_status check_pairs(const qg_proj* a, const qg_proj* b, int32_t count) {
  if (!a || !b) return QG_ERR_NULL;
  if (count < 1) return QG_ERR_ARG;
  for (int32_t k = 0; k < count; ++k) {
    qg_status st = check_proj(&a[k]);
    if (st != QG_OK) return st;
    if ((st = check_proj(&b[k])) != QG_OK) return st;
    if (a[k].m != b[k].m || a[k].r != b[k].r || a[k].r != a[0].r) return QG_ERR_SHAPE;
    if (a[k].format != b[k].format) return QG_ERR_ARG;
  }
  return QG_OK;
}
}  // namespace

extern "C" size_t qgalore_cossim_batch_workspace_bytes(int64_t r, int32_t count) {
  if (r < 1 || r > 8192 || r % 8 != 0 || count < 1) return 0;
  const int64_t per = cos_layout(r).stride;
  return (size_t)(per * std::min<int64_t>(count, qg::kCosMaxPairs));
}

extern "C" size_t qgalore_cossim_workspace_bytes(int64_t m, int64_t r) {
  if (m < 1 || r < 1 || r > m || r % 8 != 0 || r > 8192) return 0;
  return (size_t)cos_layout(r).stride + 256;
}

extern "C" qg_status qgalore_cossim_batch(const qg_proj* P_new, const qg_proj* P_old,
                                          int32_t count, void* workspace, size_t workspace_bytes,
                                          void* stream, float* out_dev) {
  qg_status st = check_pairs(P_new, P_old, count);
  if (st != QG_OK) return st;
  if (!workspace || !out_dev) return QG_ERR_NULL;
  if (!aligned(workspace, 16) || !aligned(out_dev, 4)) return QG_ERR_ALIGN;
  const int64_t r = P_new[0].r;
  if (workspace_bytes < qgalore_cossim_batch_workspace_bytes(r, count)) return QG_ERR_WORKSPACE;
  if ((st = device_present()) != QG_OK) return st;
  const CosLayout c = cos_layout(r);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t first = 0; first < count; first += qg::kCosMaxPairs) {
    qg::CosBatch b;
    std::memset(&b, 0, sizeof(b));
    b.count = std::min<int32_t>(qg::kCosMaxPairs, count - first);
    b.r = (int)r;
    b.tiles = c.tiles;
    b.ctiles = c.ctiles;
    b.nblk = c.nblk;
    b.ws = static_cast<char*>(workspace);
    b.pair_stride = c.stride;
    b.off_part = c.off_part;
    b.off_c = c.off_c;
    b.off_x = c.off_x;
    b.off_xn = c.off_xn;
    b.off_a = c.off_a;
    b.off_xb0 = c.off_xb0;
    b.off_xb1 = c.off_xb1;
    b.off_ab = c.off_ab;
    b.off_bb = c.off_bb;
    b.off_blk = c.off_blk;
    b.off_norm = c.off_norm;
    b.iters_quintic = kNsQuintic;
    b.iters_cubic_bf16 = kNsCubicBf16;
    b.iters_cubic_split = kNsCubicSplit;
    int base = 0;
    for (int k = 0; k < b.count; ++k) {
      const qg_proj& pn = P_new[first + k];
      const qg_proj& po = P_old[first + k];
      qg::CosPair& q = b.pair[k];
      q.format = pn.format;
      q.qa = pn.q;
      q.sa = pn.scale;
      q.qb = po.q;
      q.sb = po.scale;
      q.m = pn.m;
      const int64_t kchunks = cdiv(pn.m, kK);
      const int64_t split = std::min<int64_t>(c.split, kchunks);
      q.kslab = (int)(cdiv(kchunks, split) * kK);
      q.split = (int)cdiv(pn.m, q.kslab);
      q.gemm_base = base;
      base += q.split * c.ctiles * c.ctiles;
    }
    const hipError_t e = qg::launch_cossim_batch(b, out_dev + first, s);
    if (e != hipSuccess) return hip_fail(e, "similarity kernels");
  }
  return QG_OK;
}

extern "C" qg_status qgalore_cossim_async(const qg_proj* P_new, const qg_proj* P_old,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          float* out_dev) {
  return qgalore_cossim_batch(P_new, P_old, 1, workspace, workspace_bytes, stream, out_dev);
}

extern "C" qg_status qgalore_cossim(const qg_proj* P_new, const qg_proj* P_old, void* workspace,
                                    size_t workspace_bytes, void* stream, float* out_host) {
  if (!out_host) return QG_ERR_NULL;
  qg_status st = check_pairs(P_new, P_old, 1);
  if (st != QG_OK) return st;
  if (!workspace) return QG_ERR_NULL;
  const int64_t need = cos_layout(P_new->r).stride;
  if (workspace_bytes < (size_t)need + 256) return QG_ERR_WORKSPACE;
  float* dev_out = reinterpret_cast<float*>(static_cast<char*>(workspace) + need);
  st = qgalore_cossim_batch(P_new, P_old, 1, workspace, workspace_bytes, stream, dev_out);
  if (st != QG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(out_host, dev_out, sizeof(float), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? QG_OK : hip_fail(e, "similarity read-back");
}

// ==================================================================== quantize P ===

extern "C" qg_status qgalore_quantize_proj(const float* P, int64_t m, int64_t r, uint8_t* P_q,
                                           float* P_scale, void* stream) {
  if (!P || !P_q || !P_scale) return QG_ERR_NULL;
  if (m < 1 || r < 1 || m > kMaxDim || r > kMaxDim || m * r > kMaxElems) return QG_ERR_SHAPE;
  if (!aligned(P, 16) || !aligned(P_q, 4) || !aligned(P_scale, 4)) return QG_ERR_ALIGN;
  qg_status st = device_present();
  if (st != QG_OK) return st;
  const hipError_t e =
      qg::launch_quantize_int4(P, m * r, P_q, P_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QG_OK : hip_fail(e, "INT4 quantization kernel");
}

extern "C" qg_status qgalore_quantize_proj_int8(const float* P, int64_t m, int64_t r,
                                                int8_t* P_q, float* P_scale, void* stream) {
  if (!P || !P_q || !P_scale) return QG_ERR_NULL;
  if (m < 1 || r < 1 || m > kMaxDim || r > kMaxDim || m * r > kMaxElems) return QG_ERR_SHAPE;
  if (!aligned(P, 16) || !aligned(P_q, 4) || !aligned(P_scale, 4)) return QG_ERR_ALIGN;
  qg_status st = device_present();
  if (st != QG_OK) return st;
  const hipError_t e =
      qg::launch_quantize_int8(P, m * r, P_q, P_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QG_OK : hip_fail(e, "INT8 quantization kernel");
}

// ======================================================================= refresh ===

namespace {
constexpr int kRfMaxPowerIters = 8;
constexpr int64_t kRfGramChunk = 64;     // rows per partial Gram matrix
constexpr float kRfJacobiTol = 1e-6f;    // relative off-diagonal level that ends a sweep
constexpr float kRfShift = 1e-6f;        // diagonal shift (x trace / k) of the first
                                         // CholeskyQR pass
constexpr int64_t kRfBlockW = 128;       // columns per block of the wide orthonormalization
constexpr int kRfSweeps = 16;            // block Jacobi sweeps at most

struct RfGemmPlan {
  int split, tiles_m, tiles_n;
  int64_t kslab;
  int tile = qg::kSgTile;   // fp32 products: output tile edge
};
// Split-K of one product with G: enough workgroups to cover the chip.
RfGemmPlan rf_gemm_plan(int64_t M, int64_t N, int64_t K) {
  RfGemmPlan p;
  p.tiles_m = (int)cdiv(M, qg::kRfTileM);
  p.tiles_n = (int)cdiv(N, qg::kRfTileN);
  const int64_t stages = cdiv(K, kK);
  int64_t sp = std::max<int64_t>(1, cdiv(512, (int64_t)p.tiles_m * p.tiles_n));
  sp = std::min<int64_t>(std::min<int64_t>(sp, 16), stages);
  p.kslab = cdiv(stages, sp) * kK;
  p.split = (int)cdiv(K, p.kslab);
  return p;
}

// Split-K of an fp32 product (qg::SGemm): about 512 workgroups, K slabs of 4 stages or more.
// A product written in place (no split) takes 64 x 64 tiles when 128-edge ones would leave
// most of the chip idle (the M x 128 updates of the block orthonormalization).
RfGemmPlan sg_plan(int64_t M, int64_t N, int64_t K, bool split_k) {
  RfGemmPlan p;
  if (!split_k && cdiv(M, qg::kSgTile) * cdiv(N, qg::kSgTile) < 128) p.tile = 64;
  p.tiles_m = (int)cdiv(M, p.tile);
  p.tiles_n = (int)cdiv(N, p.tile);
  const int64_t stages = cdiv(K, 16);
  int64_t sp = 1;
  if (split_k) {
    sp = std::max<int64_t>(1, cdiv(512, (int64_t)p.tiles_m * p.tiles_n));
    sp = std::max<int64_t>(1, std::min<int64_t>(sp, stages / 4));
  }
  p.kslab = cdiv(stages, sp) * 16;
  p.split = (int)cdiv(K, p.kslab);
  return p;
}
int64_t sg_part_elems(int64_t M, int64_t N, int64_t K) {
  const RfGemmPlan p = sg_plan(M, N, K, true);
  return p.split > 1 ? p.split * M * N : 0;
}

bool rf_wide(int64_t k) { return k > qg::kRfMaxK; }

struct RfLayout {
  int64_t off_part, off_y, off_t, off_qf, off_qb, off_gpart, off_gram, off_wt, off_eval, off_vr,
      off_info, off_amax, off_sgn, off_p, off_gpad, off_spart, off_s, off_bjc, off_bjv, off_bjj,
      off_bjjrot, off_bjtol, off_bjrot, off_bjrank, bytes;
};
RfLayout rf_layout(int64_t m, int64_t n, int64_t r, int64_t k) {
  const int64_t mx = std::max(m, n);
  const bool wide = rf_wide(k);
  int64_t part = 0;
  const int64_t shapes[3][3] = {{m, k, n}, {m, 2 * k, n}, {n, 2 * k, m}};
  for (const auto& sh : shapes)
    part = std::max<int64_t>(part, rf_gemm_plan(sh[0], sh[1], sh[2]).split * sh[0] * sh[1]);
  // partial sums of the split fp32 products: the Gram matrices of column blocks and of the
  // whole basis, and the projections on the finished blocks
  int64_t spart = 0;
  if (wide) {
    for (const int64_t M : {m, n}) {
      spart = std::max(spart, sg_part_elems(kRfBlockW, kRfBlockW, M));
      for (int64_t c0 = kRfBlockW; c0 < k; c0 += kRfBlockW)
        spart = std::max(spart, sg_part_elems(c0, kRfBlockW, M));
    }
    spart = std::max(spart, sg_part_elems(k, k, n));
  }
  const int bjb = qg::rf_bj_block((int)k);
  const int64_t KJ = (int64_t)qg::rf_bj_blocks((int)k, bjb) * bjb;
  RfLayout L;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off += round_up(std::max<int64_t>(bytes, 1), 256);
    return o;
  };
  L.off_part = take(part * 4);
  L.off_y = take(mx * k * 4);
  L.off_t = take(mx * k * 4);
  L.off_qf = take(mx * k * 4);
  L.off_qb = take(mx * 2 * k * 2);
  L.off_gpart = take(wide ? 0 : cdiv(mx, kRfGramChunk) * k * k * 4);
  L.off_gram = take(k * k * 4);
  L.off_wt = take(k * k * 4);
  L.off_eval = take(k * 4);
  L.off_vr = take(k * r * 4);
  L.off_info = take(16);
  L.off_amax = take(cdiv(m, 64) * r * 4);
  L.off_sgn = take(r * 4);
  L.off_p = take(m * r * 4);
  L.off_gpad = take(n % 8 ? m * round_up(n, 8) * 2 : 0);
  L.off_spart = take(spart * 4);
  L.off_s = take(wide ? k * kRfBlockW * 4 : 0);
  L.off_bjc = take(KJ * KJ * 8);
  L.off_bjv = take(KJ * KJ * 8);
  L.off_bjj = take(KJ * 2 * bjb * 8);
  L.off_bjjrot = take(KJ / (2 * bjb) * 4);
  L.off_bjtol = take(4);
  L.off_bjrot = take(kRfSweeps * 4);
  L.off_bjrank = take(k * 4);
  L.bytes = off;
  return L;
}

qg_status check_refresh(int64_t m, int64_t n, int64_t r, int32_t oversample, int32_t iters) {
  if (m < 1 || n < 1 || r < 8 || r % 8 != 0 || m > kMaxDim || n > kMaxDim) return QG_ERR_SHAPE;
  if (oversample < 0 || oversample % 8 != 0 || iters < 0 || iters > kRfMaxPowerIters)
    return QG_ERR_ARG;
  const int64_t k = r + oversample;
  if (k > qg::kRfMaxKWide || k > m || k > n) return QG_ERR_SHAPE;
  // fp32 slabs of up to max(m, n) x 2k (and G itself) stay below 2^29 elements
  if (m * round_up(n, 8) > kMaxElems || std::max(m, n) * 2 * k > kMaxElems) return QG_ERR_SHAPE;
  return QG_OK;
}
}  // namespace

extern "C" size_t qgalore_refresh_workspace_bytes(int64_t m, int64_t n, int64_t r,
                                                  int32_t oversample) {
  if (check_refresh(m, n, r, oversample, 0) != QG_OK) return 0;
  return (size_t)rf_layout(m, n, r, r + oversample).bytes;
}

extern "C" qg_status qgalore_refresh_proj(const uint16_t* G, int64_t m, int64_t n, int64_t r,
                                          const uint16_t* Omega, int32_t oversample,
                                          int32_t power_iters, uint8_t* P_q, float* P_scale,
                                          float* P_out, float* sigma_out, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (!G || !Omega || !P_q || !P_scale || !workspace) return QG_ERR_NULL;
  qg_status st = check_refresh(m, n, r, oversample, power_iters);
  if (st != QG_OK) return st;
  if (!aligned(G, 16) || !aligned(Omega, 16) || !aligned(P_q, 4) || !aligned(P_scale, 4) ||
      !aligned(workspace, 16) || (P_out && !aligned(P_out, 16)) ||
      (sigma_out && !aligned(sigma_out, 4)))
    return QG_ERR_ALIGN;
  const int64_t k = r + oversample;
  const RfLayout lay = rf_layout(m, n, r, k);
  if (workspace_bytes < (size_t)lay.bytes) return QG_ERR_WORKSPACE;
  if ((st = device_present()) != QG_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto at = [&](int64_t off) { return reinterpret_cast<float*>(ws + off); };
  float* part = at(lay.off_part);
  float* Y = at(lay.off_y);
  float* T = at(lay.off_t);
  float* Qf = at(lay.off_qf);
  uint16_t* Qb = reinterpret_cast<uint16_t*>(ws + lay.off_qb);
  float* gpart = at(lay.off_gpart);
  float* gram = at(lay.off_gram);
  float* Wt = at(lay.off_wt);
  float* evals = at(lay.off_eval);
  float* Vr = at(lay.off_vr);
  int* info = reinterpret_cast<int*>(ws + lay.off_info);
  float* amax = at(lay.off_amax);
  float* sgn = at(lay.off_sgn);
  float* P = P_out ? P_out : at(lay.off_p);
  float* spart = at(lay.off_spart);
  float* S = at(lay.off_s);
  const int kk = (int)k;
  const bool wide = rf_wide(k);

  hipError_t e = hipSuccess;
  // G with rows on 16-byte bounds: a zero-padded copy when n is not a multiple of 8 (the
  // padding columns add nothing to the products)
  const uint16_t* Ga = G;
  const int64_t lda = round_up(n, 8);
  if (n % 8) {
    uint16_t* Gp = reinterpret_cast<uint16_t*>(ws + lay.off_gpad);
    e = qg::launch_rf_pad(G, m, n, lda, Gp, s);
    Ga = Gp;
  }
  // out (M x k) = A B, with A = G (M = m, K = n) or G^T (M = n, K = m) and B a basis of
  // width nb (k for the sketch, 2k for the hi/lo parts of an fp32 basis)
  auto product = [&](bool transposed, const uint16_t* B, int64_t nb, float* out) {
    const int64_t M = transposed ? n : m, K = transposed ? m : n;
    const RfGemmPlan pl = rf_gemm_plan(M, nb, K);
    qg::RfGemm g;
    g.A = Ga;
    g.B = B;
    g.part = part;
    g.M = M;
    g.N = nb;
    g.K = K;
    g.lda = lda;
    g.ldb = nb;
    g.kslab = pl.kslab;
    g.tiles_m = pl.tiles_m;
    g.tiles_n = pl.tiles_n;
    g.split = pl.split;
    g.a_kmajor = transposed ? 1 : 0;
    if (e == hipSuccess) e = qg::launch_rf_gemm(g, s);
    if (e == hipSuccess) e = qg::launch_rf_reduce(part, pl.split, M, (int)nb, kk, out, s);
  };
  // fp32 product out op= A B (qg::SGemm). With mode kSgPartial the K slabs' partial products
  // are summed, in order, into the dense out (M x N).
  auto sgemm = [&](const float* A, int64_t lda_, bool a_kmajor, const float* B, int64_t ldb,
                   int64_t M, int64_t N, int64_t K, float* out, int64_t ldo, int mode) {
    const bool reduce = mode == qg::kSgPartial;
    const RfGemmPlan pl = sg_plan(M, N, K, reduce);
    qg::SGemm g;
    g.A = A;
    g.B = B;
    g.M = M;
    g.N = N;
    g.K = K;
    g.lda = lda_;
    g.ldb = ldb;
    g.kslab = pl.kslab;
    g.tiles_m = pl.tiles_m;
    g.tiles_n = pl.tiles_n;
    g.split = pl.split;
    g.tile = pl.tile;
    g.a_kmajor = a_kmajor ? 1 : 0;
    const bool summed = reduce && pl.split > 1;
    g.out = summed ? spart : out;
    g.ldo = ldo;
    g.mode = reduce && !summed ? qg::kSgStore : mode;
    if (e == hipSuccess) e = qg::launch_rf_sgemm(g, s);
    if (summed && e == hipSuccess) e = qg::launch_rf_sum(spart, pl.split, M * N, out, s);
  };
  auto gram_of = [&](const float* X, int64_t M) {
    if (e == hipSuccess)
      e = qg::launch_rf_gram(X, M, kk, kRfGramChunk, (int)cdiv(M, kRfGramChunk), gpart, gram, s);
  };
  // Qf, Qb = orth(Y) for Y of M rows: CholeskyQR with `passes` passes (the first shifted)
  auto orth = [&](int64_t M, int passes) {
    const float* in = Y;
    for (int pass = 0; pass < passes; ++pass) {
      const bool last = pass == passes - 1;
      float* out = last ? Qf : T;
      gram_of(in, M);
      if (e == hipSuccess) e = qg::launch_rf_chol_inv(gram, kk, pass == 0 ? kRfShift : 0.0f, Wt, s);
      if (e == hipSuccess)
        e = qg::launch_rf_smallmul(in, Wt, M, kk, kk, out, last ? Qb : nullptr, nullptr, s);
      in = out;
    }
  };
  // The same for a wide basis, block by block of kRfBlockW columns: the block's projection on
  // the finished blocks removed twice (S = Q^T X, X -= Q S), then CholeskyQR with `passes`
  // passes on the block alone.
  auto orth_wide = [&](int64_t M, int passes) {
    for (int64_t c0 = 0; c0 < k; c0 += kRfBlockW) {
      const int64_t bw = std::min<int64_t>(kRfBlockW, k - c0);
      float* X = Y + c0;
      if (c0 > 0)
        for (int rep = 0; rep < 2; ++rep) {
          sgemm(Qf, k, true, X, k, c0, bw, M, S, bw, qg::kSgPartial);
          sgemm(Qf, k, false, S, bw, M, bw, c0, X, k, qg::kSgSubtract);
        }
      const float* in = X;
      for (int pass = 0; pass < passes; ++pass) {
        float* out = (pass == passes - 1 ? Qf : T) + c0;
        sgemm(in, k, true, in, k, bw, bw, M, gram, bw, qg::kSgPartial);
        if (e == hipSuccess)
          e = qg::launch_rf_chol_inv(gram, (int)bw, pass == 0 ? kRfShift : 0.0f, Wt, s);
        sgemm(in, k, false, Wt, bw, M, bw, bw, out, k, qg::kSgStore);
        in = out;
      }
    }
    if (e == hipSuccess) e = qg::launch_rf_split(Qf, M, kk, Qb, s);
  };
  auto orthogonalize = [&](int64_t M, int passes) {
    if (wide)
      orth_wide(M, passes);
    else
      orth(M, passes);
  };
  product(false, Omega, k, Y);            // Y = G Omega
  orthogonalize(m, power_iters == 0 ? 2 : 1);
  for (int it = 0; it < power_iters; ++it) {
    product(true, Qb, 2 * k, Y);          // G^T Q
    orthogonalize(n, 1);
    product(false, Qb, 2 * k, Y);         // G Z
    orthogonalize(m, it == power_iters - 1 ? 2 : 1);
  }
  product(true, Qb, 2 * k, Y);            // B^T = G^T Q  (n x k)
  // B B^T and its eigen-decomposition
  if (wide)
    sgemm(Y, k, true, Y, k, k, k, n, gram, k, qg::kSgPartial);
  else
    gram_of(Y, n);
  qg::RfBj bj;
  bj.C = reinterpret_cast<double*>(ws + lay.off_bjc);
  bj.V = reinterpret_cast<double*>(ws + lay.off_bjv);
  bj.J = reinterpret_cast<double*>(ws + lay.off_bjj);
  bj.jrot = reinterpret_cast<int*>(ws + lay.off_bjjrot);
  bj.abs_tol = at(lay.off_bjtol);
  bj.rot = reinterpret_cast<int*>(ws + lay.off_bjrot);
  bj.rank_of = reinterpret_cast<int*>(ws + lay.off_bjrank);
  if (e == hipSuccess)
    e = qg::launch_rf_block_jacobi(gram, kk, (int)r, kRfSweeps, kRfJacobiTol, bj, evals, Vr,
                                   sigma_out, info, s);
  // P = Q V_r with the per-tile column maxima of the sign rule
  if (!wide) {
    if (e == hipSuccess) e = qg::launch_rf_smallmul(Qf, Vr, m, kk, (int)r, P, nullptr, amax, s);
  } else {
    sgemm(Qf, k, false, Vr, r, m, r, k, P, r, qg::kSgStore);
    if (e == hipSuccess) e = qg::launch_rf_colmax(P, m, (int)r, amax, s);
  }
  if (e == hipSuccess) e = qg::launch_rf_signs(P, m, (int)r, amax, sgn, s);
  if (e == hipSuccess) e = qg::launch_quantize_int4(P, m * r, P_q, P_scale, s);
  return e == hipSuccess ? QG_OK : hip_fail(e, "subspace refresh kernels");
}

// ========================================================= INT8-weight linear layer ===

namespace {
qg_status check_linear(int64_t T, int64_t m, int64_t n) {
  if (T < 1 || m < 1 || n < 1 || T > kMaxDim || m > kMaxDim || n > kMaxDim) return QG_ERR_SHAPE;
  if (m % 8 != 0 || n % 8 != 0) return QG_ERR_SHAPE;
  if (m * n > kMaxElems || T * m > kMaxElems || T * n > kMaxElems) return QG_ERR_SHAPE;
  return QG_OK;
}

qg_status run_linear(const qg::LinArgs& a, int which, void* stream, const char* what) {
  qg_status st = device_present();
  if (st != QG_OK) return st;
  const hipError_t e = qg::launch_linear(a, which, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QG_OK : hip_fail(e, what);
}
}  // namespace

extern "C" qg_status qgalore_int8_linear_fwd(const uint16_t* X, const int8_t* W_q,
                                             const float* W_scale, int64_t T, int64_t m,
                                             int64_t n, uint16_t* Y, void* stream) {
  if (!X || !W_q || !W_scale || !Y) return QG_ERR_NULL;
  qg_status st = check_linear(T, m, n);
  if (st != QG_OK) return st;
  if (!aligned(X, 16) || !aligned(W_q, 16) || !aligned(W_scale, 4) || !aligned(Y, 16))
    return QG_ERR_ALIGN;
  qg::LinArgs a{X, nullptr, W_q, W_scale, Y, T, m, n};
  return run_linear(a, qg::kLinFwd, stream, "INT8-weight forward kernel");
}

extern "C" qg_status qgalore_int8_linear_bwd_data(const uint16_t* dY, const int8_t* W_q,
                                                  const float* W_scale, int64_t T, int64_t m,
                                                  int64_t n, uint16_t* dX, void* stream) {
  if (!dY || !W_q || !W_scale || !dX) return QG_ERR_NULL;
  qg_status st = check_linear(T, m, n);
  if (st != QG_OK) return st;
  if (!aligned(dY, 16) || !aligned(W_q, 16) || !aligned(W_scale, 4) || !aligned(dX, 16))
    return QG_ERR_ALIGN;
  qg::LinArgs a{dY, nullptr, W_q, W_scale, dX, T, m, n};
  return run_linear(a, qg::kLinBwdData, stream, "INT8-weight data-gradient kernel");
}

extern "C" qg_status qgalore_linear_bwd_weight(const uint16_t* dY, const uint16_t* X, int64_t T,
                                               int64_t m, int64_t n, uint16_t* G,
                                               void* stream) {
  if (!dY || !X || !G) return QG_ERR_NULL;
  qg_status st = check_linear(T, m, n);
  if (st != QG_OK) return st;
  if (!aligned(dY, 16) || !aligned(X, 16) || !aligned(G, 16)) return QG_ERR_ALIGN;
  qg::LinArgs a{dY, X, nullptr, nullptr, G, T, m, n};
  return run_linear(a, qg::kLinBwdWeight, stream, "weight-gradient kernel");
}

// ====================================================================== schedule ===

extern "C" qg_status qgalore_sched_init(qg_sched* s, int64_t delta0, float gamma) {
  if (!s) return QG_ERR_NULL;
  if (delta0 < 1 || !finite(gamma)) return QG_ERR_ARG;
  s->delta = delta0;
  s->next_refresh = 0;
  s->count = 0;
  s->gamma = gamma;
  s->last_cossim = NAN;
  return QG_OK;
}

extern "C" int32_t qgalore_sched_due(const qg_sched* s, int64_t t) {
  if (!s) return -1;
  return t >= s->next_refresh ? 1 : 0;
}

extern "C" qg_status qgalore_sched_refresh(qg_sched* s, int64_t t, float cossim, int32_t* doubled) {
  if (!s) return QG_ERR_NULL;
  int32_t d = 0;
  if (s->count > 0) {
    if (std::isnan(cossim)) return QG_ERR_ARG;
    s->last_cossim = cossim;
    if (cossim > s->gamma) {
      if (s->delta > (int64_t(1) << 61)) return QG_ERR_ARG;
      s->delta *= 2;
      d = 1;
    }
  }
  s->count += 1;
  s->next_refresh = t + s->delta;
  if (doubled) *doubled = d;
  return QG_OK;
}

// ================================================================== calibration ===

extern "C" qg_status qgalore_mfma_probe(const uint16_t* operands, int64_t n_elems, float* out,
                                        int32_t grid, int32_t iters, void* stream) {
  if (!operands || !out) return QG_ERR_NULL;
  if (n_elems < 8 || n_elems % 8 != 0 || n_elems > (int64_t(1) << 32)) return QG_ERR_SHAPE;
  if (grid < 1 || grid > 65536 || iters < 1 || iters > (1 << 20)) return QG_ERR_ARG;
  if (!aligned(operands, 16) || !aligned(out, 4)) return QG_ERR_ALIGN;
  const hipError_t e = qg::launch_mfma_probe(operands, n_elems, out, grid, iters,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QG_OK : hip_fail(e, "mfma probe launch");
}

// ========================================================================= misc ===

extern "C" const char* qgalore_status_str(qg_status s) {
  switch (s) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "null pointer argument";
    case QG_ERR_SHAPE: return "invalid shape";
    case QG_ERR_ALIGN: return "misaligned pointer";
    case QG_ERR_WORKSPACE: return "workspace too small";
    case QG_ERR_ARG: return "invalid argument";
    case QG_ERR_HIP: return "HIP runtime error";
    case QG_ERR_NO_DEVICE: return "no HIP device";
  }
  return "unknown status";
}

extern "C" const char* qgalore_last_error(void) { return g_last_error.c_str(); }
extern "C" const char* qgalore_version(void) { return "qgalore-gfx950 0.1.0"; }
