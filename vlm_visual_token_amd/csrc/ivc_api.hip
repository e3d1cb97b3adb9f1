// Host side of the C ABI declared in include/ivc.h: validation, weight
// ownership, workspace planning and the kernel sequence of each call.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ivc.h"
#include "kernels.h"


using namespace ivc;

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local std::string g_last_error;

static ivc_status fail(ivc_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

// IVC_TRACE=1 (any value but "0"): one line on stderr per entry-point call
// (its shape arguments) and per kernel launch (name, stream; products also
// their M x N x K and kernel family).  Read once, at the first call.
static bool trace_on() {
  static const bool on = [] {
    const char* e = getenv("IVC_TRACE");
    return e != nullptr && *e != 0 && strcmp(e, "0") != 0;
  }();
  return on;
}
// True when the variable is set to "0" (read at every call, so a process can
// switch between forms for comparison).
static bool env_off(const char* name) {
  const char* e = getenv(name);
  return e != nullptr && strcmp(e, "0") == 0;
}

#define TRACE(...)                          \
  do {                                      \
    if (trace_on()) {                       \
      fprintf(stderr, "[ivc] " __VA_ARGS__); \
      fputc('\n', stderr);                  \
    }                                       \
  } while (0)

#define HIP_OK(expr)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return fail(IVC_ERR_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),       \
                  __FILE__, __LINE__);                                                      \
  } while (0)

// Launch wrapper: optional per-kernel timing, then the launch's status.
#define LAUNCH(name, stream, expr)   \
  do {                               \
    TRACE("  launch %s stream=%p", name, (void*)(stream)); \
    prof_begin(name, stream);        \
    hipError_t le_ = (expr);         \
    prof_end(stream);                \
    HIP_OK(le_);                     \
  } while (0)

// ---------------------------------------------------------------------------
// per-kernel timing
// ---------------------------------------------------------------------------
namespace {
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
bool g_prof_on = false;
bool g_prof_keep_fork = false;  // mode 2: the projector chains keep their two streams
std::vector<ProfRec> g_prof_pending;
std::vector<hipEvent_t> g_prof_free;
std::vector<std::string> g_prof_names;
std::vector<double> g_prof_ms;
std::vector<long long> g_prof_n;
hipEvent_t take_event() {
  if (!g_prof_free.empty()) {
    hipEvent_t e = g_prof_free.back();
    g_prof_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  (void)hipEventCreate(&e);
  return e;
}
}  // namespace

namespace ivc {
void prof_begin(const char* name, hipStream_t s) {
  if (!g_prof_on) return;
  ProfRec r{name, take_event(), take_event()};
  (void)hipEventRecord(r.a, s);
  g_prof_pending.push_back(r);
}
void prof_end(hipStream_t s) {
  if (!g_prof_on || g_prof_pending.empty()) return;
  (void)hipEventRecord(g_prof_pending.back().b, s);
}
}  // namespace ivc

static void prof_collect() {
  for (auto& r : g_prof_pending) {
    (void)hipEventSynchronize(r.b);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, r.a, r.b);
    size_t i = 0;
    for (; i < g_prof_names.size(); ++i)
      if (g_prof_names[i] == r.name) break;
    if (i == g_prof_names.size()) {
      g_prof_names.push_back(r.name);
      g_prof_ms.push_back(0.0);
      g_prof_n.push_back(0);
    }
    g_prof_ms[i] += ms;
    g_prof_n[i] += 1;
    g_prof_free.push_back(r.a);
    g_prof_free.push_back(r.b);
  }
  g_prof_pending.clear();
}

extern "C" void ivc_profile_enable(int on) {
  g_prof_on = on != 0;
  g_prof_keep_fork = on == 2;
}
extern "C" void ivc_profile_reset(void) {
  prof_collect();
  g_prof_names.clear();
  g_prof_ms.clear();
  g_prof_n.clear();
}
extern "C" int32_t ivc_profile_read(const char** names, double* total_ms, int64_t* launches,
                                    int32_t cap) {
  prof_collect();
  const int32_t n = (int32_t)g_prof_names.size();
  for (int32_t i = 0; i < n && i < cap; ++i) {
    if (names) names[i] = g_prof_names[i].c_str();
    if (total_ms) total_ms[i] = g_prof_ms[i];
    if (launches) launches[i] = g_prof_n[i];
  }
  return n;
}

// ---------------------------------------------------------------------------
// handle
// ---------------------------------------------------------------------------
struct ivc_connector {
  ivc_config cfg;
  int esz;
  int ncu = 256;  // compute units of the device the connector was created on
  int dev = 0;     // that device
  // second stream (default priority) on which the mlp1 chain runs beside the
  // mlp2 chain; forked from and joined back to the caller's stream by events
  hipStream_t aux = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  hipStream_t aux2 = nullptr;  // side work beside both projector chains
  hipEvent_t ev_side = nullptr;
  char* blob = nullptr;
  // mlp1 / mlp2
  float *m1_ln_w, *m1_ln_b, *m1_b1, *m1_b2;
  void *m1_w1, *m1_w2;
  float *m2_ln_w, *m2_ln_b, *m2_b1, *m2_b2, *m2_b3;
  void *m2_w1, *m2_w2, *m2_w3;
  // ln_fold: m*_w1 hold gamma o W1, m*_b1 the folded bias, m*_cs the column sums
  float *m1_cs = nullptr, *m2_cs = nullptr;
  // router
  void* query;
  float* query_f;  // the learned query widened to fp32 (read by every tile's first layer)
  // folded pooling: the first layer's folded query, the same for every tile
  // (the learned query projected and folded once at create), [16, C] bf16 hi / lo
  void* qt0_hi;
  void* qt0_lo;
  // folded pooling, layers l >= 1: the previous layer's output projection
  // folded into this layer's query projection, Wqo = Wq_l Wo_{l-1} (fp32, as
  // bf16 hi / lo parts) and bqo = Wq_l bo_{l-1} + bq_l; no per-tile q is formed
  // between layers.  (cr_*: scratch of the products made at create.)
  void *wqo_hi[IVC_MAX_POOL_LAYERS], *wqo_lo[IVC_MAX_POOL_LAYERS];
  float* bqo[IVC_MAX_POOL_LAYERS];
  void* cr_woT;
  float* cr_wqo;
  void *wq[IVC_MAX_POOL_LAYERS], *wo[IVC_MAX_POOL_LAYERS];
  float *bq[IVC_MAX_POOL_LAYERS], *bo[IVC_MAX_POOL_LAYERS];
  void* wkv;   // [2 * layers * C, C]: Wk_0; Wv_0; Wk_1; Wv_1; ...
  float* bkv;  // [2 * layers * C]
  void* wkT;   // bf16 only: [layers][C, C], wkT[l][c][j] = Wk_l[j][c] (query fold)
  void *g_w1[IVC_GATE_BLOCKS], *g_w2[IVC_GATE_BLOCKS], *g_cw;
  // Row strides (elements) of the router matrices above: wq, wo, wkv, wkT and
  // wqo rows (C wide) at lr, gate W1 rows (gate_hidden wide) at lg1, gate W2
  // rows at lg2.  With bf16 weights each row is padded by 16 bytes: the
  // router products read 16 rows of one K step per load instruction, and at a
  // power-of-two stride those reads collide (measured: 16-byte padding makes
  // a 208 x 1024 x 1024 product ~25% faster; 128 bytes of padding does not).
  long long lr, lg1, lg2;
  float *g_b1[IVC_GATE_BLOCKS], *g_b2[IVC_GATE_BLOCKS], *g_lw[IVC_GATE_BLOCKS],
      *g_lb[IVC_GATE_BLOCKS], *g_cb;
};

namespace {

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += al256(bytes);
    return p;
  }
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

__global__ void k_widen(const void* src, int dtype, float* dst, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (dtype == DT_BF16) {
    const uint16_t h = ((const uint16_t*)src)[i];
    dst[i] = __uint_as_float(((uint32_t)h) << 16);
  } else {
    dst[i] = ((const float*)src)[i];
  }
}

ivc_status widen(const void* src, int dtype, float* dst, long long n, hipStream_t s) {
  if (n == 0) return IVC_OK;
  hipLaunchKernelGGL(k_widen, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dtype,
                     dst, n);
  HIP_OK(hipGetLastError());
  return IVC_OK;
}

ivc_status copy_mat(const void* src, void* dst, size_t bytes, hipStream_t s) {
  HIP_OK(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s));
  return IVC_OK;
}

// dense [rows, cols] matrix of e-byte elements into rows of stride ld
ivc_status copy_rows(const void* src, void* dst, size_t rows, size_t cols, size_t ld, size_t e,
                     hipStream_t s) {
  HIP_OK(hipMemcpy2DAsync(dst, ld * e, src, cols * e, cols * e, rows, hipMemcpyDeviceToDevice, s));
  return IVC_OK;
}

ivc_status check_cfg(const ivc_config& c) {
  if (c.dtype != IVC_F32 && c.dtype != IVC_BF16) return fail(IVC_ERR_INVALID_ARG, "dtype %d", c.dtype);
  const int esz = c.dtype == IVC_BF16 ? 2 : 4;
  if (c.vit_width <= 0 || c.grid <= 0 || c.llm_width <= 0 || c.mlp1_hidden <= 0)
    return fail(IVC_ERR_INVALID_ARG, "widths and grid must be positive");
  if (c.has_cls != 0 && c.has_cls != 1) return fail(IVC_ERR_INVALID_ARG, "has_cls must be 0 or 1");
  if (c.grid % (c.flash ? 4 : 2) != 0)
    return fail(IVC_ERR_INVALID_ARG, "grid %d not divisible by %d", c.grid, c.flash ? 4 : 2);
  if ((long long)c.vit_width * esz % 16 || (long long)c.llm_width * esz % 16 ||
      (long long)c.mlp1_hidden * esz % 16)
    return fail(IVC_ERR_MISALIGNED, "row widths must be multiples of 16 bytes");
  if (c.vit_width > shuffle_max_width(c.dtype))
    return fail(IVC_ERR_UNSUPPORTED, "vit_width %d above the loader's %d", c.vit_width,
                shuffle_max_width(c.dtype));
  if (!(c.ln_eps >= 0.f)) return fail(IVC_ERR_INVALID_ARG, "ln_eps");
  if (c.ps_version < 0 || c.ps_version > 2)
    return fail(IVC_ERR_INVALID_ARG, "ps_version %d", c.ps_version);
  if (c.shuffle64_order != IVC_SHUFFLE64_DIRECT && c.shuffle64_order != IVC_SHUFFLE64_TWICE_R2)
    return fail(IVC_ERR_INVALID_ARG, "shuffle64_order %d", c.shuffle64_order);
  if (c.ln_fold != 0 && c.ln_fold != 1) return fail(IVC_ERR_INVALID_ARG, "ln_fold %d", c.ln_fold);
  if (c.ln_fold) {
    if (c.dtype != IVC_BF16) return fail(IVC_ERR_UNSUPPORTED, "ln_fold needs bf16");
    if (c.vit_width % 64 || c.mlp1_hidden % 8 || (c.flash && c.mlp2_hidden % 8))
      return fail(IVC_ERR_UNSUPPORTED, "ln_fold needs C %% 64 == 0 and hidden widths %% 8 == 0");
  }
  if (c.flash) {
    if (c.mlp2_hidden <= 0 || (long long)c.mlp2_hidden * esz % 16)
      return fail(IVC_ERR_INVALID_ARG, "mlp2_hidden");
    if (c.pool_layers < 1 || c.pool_layers > IVC_MAX_POOL_LAYERS)
      return fail(IVC_ERR_INVALID_ARG, "pool_layers %d", c.pool_layers);
    if (c.pool_heads <= 0 || c.vit_width % c.pool_heads)
      return fail(IVC_ERR_INVALID_ARG, "pool_heads %d does not divide C", c.pool_heads);
    if (!pool_attn_supported(c.vit_width, c.pool_heads))
      return fail(IVC_ERR_UNSUPPORTED, "pooling with C=%d, heads=%d", c.vit_width, c.pool_heads);
    if (c.gate_hidden != c.vit_width)
      return fail(IVC_ERR_INVALID_ARG, "gate_hidden %d must equal C %d", c.gate_hidden, c.vit_width);
    if (c.gate_hidden > 4096) return fail(IVC_ERR_UNSUPPORTED, "gate_hidden above 4096");
    if (c.gate_expansion < 1) return fail(IVC_ERR_INVALID_ARG, "gate_expansion");
    if (c.pool_mode != IVC_POOL_KV && c.pool_mode != IVC_POOL_FOLDED)
      return fail(IVC_ERR_INVALID_ARG, "pool_mode %d", c.pool_mode);
    if (c.pool_mode == IVC_POOL_FOLDED && !pool_folded_supported(c.dtype, c.vit_width, c.pool_heads))
      return fail(IVC_ERR_UNSUPPORTED,
                  "folded pooling needs bf16, C in {512, 1024} and at most 16 heads");
    if (!(c.rel_quantile >= 0.0 && c.rel_quantile <= 1.0))
      return fail(IVC_ERR_INVALID_ARG, "rel_quantile outside [0, 1]");
  }
  return IVC_OK;
}

// Scratch of the SIMT kernel's split-K reduction.
struct SimtScratch {
  float* part = nullptr;
  size_t part_elems = 0;
  void need(int M, int N, int K, int batch) {
    const int ks = simt_ksplit(M, N, K, batch);
    const size_t pe = simt_part_elems(M, N, batch, ks);
    if (pe > part_elems) part_elems = pe;
  }
  void carve(Carver& cv) { part = (float*)cv.take(part_elems * 4); }
};

// GEMM dispatch: MFMA for bf16 operands with K % 64 == 0, SIMT otherwise
// (split over K when the product is skinny and scratch is available).
void trace_gemm(const char* name, const GemmArgs& g, const char* family) {
  TRACE("    %s: %s M=%d N=%d K=%d batch=%d act=%d fold=%d rowmap=%d leftover-split=%d", name,
        family, g.M, g.N, g.K, g.batch, g.act, g.fold, g.rm.m_dev != nullptr,
        g.tail_part != nullptr);
}

// Whether gemm() runs the product on the 256 x 256 LDS-DMA kernel (the only
// one that honours RowMap::d_map).
bool gemm_takes_dma(GemmArgs g) {
  if (g.batch <= 0) g.batch = 1;
  if (g.c_dtype == DT_F32 && gemm_f32a_supported(g)) return false;
  if (g.batch != 1 || !gemm_mfma_supported(g)) return false;
  const long long big_tiles = (long long)((g.M + 255) / 256) * ((g.N + 255) / 256);
  return big_tiles >= 256 && gemm_dma_supported(g);
}

hipError_t gemm(const char* name, GemmArgs g, hipStream_t s, const SimtScratch* sc = nullptr) {
  if (g.batch <= 0) g.batch = 1;
  if (trace_on()) {
    const char* fam = gemm_takes_dma(g)                                   ? "256x256 LDS-DMA MFMA"
                      : (g.c_dtype == DT_F32 && gemm_f32a_supported(g)) ? "f32a split-bf16 MFMA"
                      : (g.batch == 1 && gemm_mfma_supported(g))        ? "128x128 MFMA"
                                                                        : "SIMT";
    trace_gemm(name, g, fam);
  }
  // 256 x 256 LDS-DMA tiles when they fill the chip (the only kernel that
  // places rows a second time), else 128 x 128 tiles, split-bf16 or SIMT
  if (gemm_takes_dma(g)) return launch_gemm_dma(g, s);
  if (g.rm.d_map != nullptr) return hipErrorInvalidValue;
  if (g.c_dtype == DT_F32 && gemm_f32a_supported(g)) return launch_gemm_f32a(g, 0, nullptr, 1.f, s);
  if (g.batch == 1 && gemm_mfma_supported(g)) return launch_gemm_mfma(g, s);
  g.ksplit = 1;
  if (sc != nullptr && sc->part != nullptr) {
    const int ks = simt_ksplit(g.M, g.N, g.K, g.batch);
    if (ks > 1 && simt_part_elems(g.M, g.N, g.batch, ks) <= sc->part_elems) {
      g.ksplit = ks;
      g.part = sc->part;
    }
  }
  return launch_gemm_simt(g, s);
}

GemmArgs mk_gemm(const void* A, long long lda, int a_dt, const void* W, int w_dt,
                 const float* bias, void* Cm, int c_dt, int M, int N, int K, int act) {
  GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.W = W;
  g.ldw = K;
  g.bias = bias;
  g.Cm = Cm;
  g.ldc = N;
  g.M = M;
  g.N = N;
  g.K = K;
  g.act = act;
  g.a_dtype = a_dt;
  g.w_dtype = w_dt;
  g.c_dtype = c_dt;
  g.batch = 1;
  g.ksplit = 1;
  return g;
}

int pool_splits(int T, int N) {
  // enough workgroups to cover 256 CUs a few times over, at least 64 tokens each
  int s = 1;
  while ((long long)T * s < 1024 && N / (2 * s) >= 64) s *= 2;
  return s;
}

// ---- workspace plans ----
struct RunWs {
  void *a2, *a4, *h1, *g1, *g2;
  float *st2, *st4;  // ln_fold: (mean, rstd) per LayerNorm row instead of a2 / a4
  int *rank, *list256, *list64, *counts;  // route-first run only
  SimtScratch sc;
  // bf16 standard (non-Flash) connectors: leftover-tile pieces of the mlp1
  // products.  Only a product that runs alone gains from cutting its last
  // partial round of tiles into K pieces: in a Flash run the mlp1 and mlp2
  // chains share the chip on two streams and each fills the other's partial
  // rounds, so there the pieces only add partial-tile traffic (measured on
  // the 2B-Flash step: 2.31 ms with pieces against 2.24 ms without).
  char* tail = nullptr;
};

// Workgroups of one whole round of a product: the CU count, a multiple of 8.
int tail_grid(const ivc_connector* h) { return h->ncu >= 8 ? h->ncu & ~7 : 8; }

// A nonzero tag below 2^56, different for every launch of this process: the
// leftover-tile counters compare it with what they hold, so a counter left by
// an earlier launch (or uninitialised workspace) never counts as this one's.
unsigned long long next_ticket() {
  static std::atomic<unsigned long long> ctr{0};
  static const unsigned long long salt = [] {
    const unsigned long long t =
        (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    return (t ^ (t >> 29) ^ (unsigned long long)(uintptr_t)&ctr) & 0xffffffull;
  }();
  const unsigned long long c = ctr.fetch_add(1, std::memory_order_relaxed) % 0xffffffffull + 1;
  return (salt << 32) | c;
}

// Gives a projector product its chain's leftover-tile scratch (bf16 DMA kernels).
void with_tail(GemmArgs& g, const ivc_connector* h, char* region) {
  if (region == nullptr) return;
  const int G = tail_grid(h);
  g.tail_part = reinterpret_cast<float*>(region);
  g.tail_cnt = reinterpret_cast<unsigned long long*>(region + (size_t)2 * G * 256 * 256 * 4);
  g.tail_ticket = next_ticket();
  g.tail_grid = G;
}
size_t plan_run(const ivc_connector* h, int T, void* base, RunWs* w) {
  const ivc_config& c = h->cfg;
  const size_t e = h->esz;
  const size_t S = (size_t)(c.grid / 2) * (c.grid / 2), S4 = (size_t)(c.grid / 4) * (c.grid / 4);
  Carver cv(base);
  RunWs r{};
  if (c.ln_fold)
    r.st2 = (float*)cv.take((size_t)T * S * 2 * 4);
  else
    r.a2 = cv.take((size_t)T * S * 4 * c.vit_width * e);
  r.h1 = cv.take((size_t)T * S * c.mlp1_hidden * e);
  if (c.flash) {
    if (c.ln_fold)
      r.st4 = (float*)cv.take((size_t)T * S4 * 2 * 4);
    else
      r.a4 = cv.take((size_t)T * S4 * 16 * c.vit_width * e);
    r.g1 = cv.take((size_t)T * S4 * c.mlp2_hidden * e);
    r.g2 = cv.take((size_t)T * S4 * c.mlp2_hidden * e);
    r.rank = (int*)cv.take((size_t)T * 4);
    r.list256 = (int*)cv.take((size_t)T * 4);
    r.list64 = (int*)cv.take((size_t)T * 4);
    r.counts = (int*)cv.take(2 * 4);
  }
  if (c.dtype == IVC_BF16 && !c.flash) r.tail = (char*)cv.take(gemm_tail_bytes(tail_grid(h)));
  if (c.dtype == IVC_F32) {  // bf16 products all run on MFMA
    const int M2 = (int)(T * S), M4 = (int)(T * S4);
    r.sc.need(M2, c.mlp1_hidden, 4 * c.vit_width, 1);
    r.sc.need(M2, c.llm_width, c.mlp1_hidden, 1);
    if (c.flash) {
      r.sc.need(M4, c.mlp2_hidden, 16 * c.vit_width, 1);
      r.sc.need(M4, c.mlp2_hidden, c.mlp2_hidden, 1);
      r.sc.need(M4, c.llm_width, c.mlp2_hidden, 1);
    }
    r.sc.carve(cv);
  }
  if (w) *w = r;
  return cv.off;
}

struct RouteWs {
  void *kv, *qt_hi, *qt_lo;
  float *q, *qp, *o, *part, *xbar, *y1, *y2, *x, *x2;
  // one-launch Gating: further per-phase row buffers and the phase counters
  float *y1b[3], *y2b[3], *x3;
  unsigned long long* sync;
  SimtScratch sc;
};
size_t plan_route(const ivc_connector* h, int T, void* base, RouteWs* w) {
  const ivc_config& c = h->cfg;
  const size_t C = c.vit_width, N = (size_t)c.grid * c.grid, L = c.pool_layers;
  const size_t hh = c.gate_hidden, he = hh * c.gate_expansion;
  Carver cv(base);
  RouteWs r{};
  if (!c.flash) return 0;
  const int sp = pool_splits(T, (int)N);
  if (c.pool_mode == IVC_POOL_FOLDED) {
    int G, Q, segmax;
    folded_geometry(T, (int)N, (int)C, h->ncu, &G, &Q, &segmax);
    r.qt_hi = cv.take((size_t)T * 16 * C * 2);
    r.qt_lo = cv.take((size_t)T * 16 * C * 2);
    r.part = (float*)cv.take((size_t)G * segmax * 16 * (2 + C) * 4);
    r.xbar = (float*)cv.take((size_t)T * c.pool_heads * C * 4);
  } else {
    r.kv = cv.take((size_t)T * N * 2 * L * C * h->esz);
    r.part = (float*)cv.take((size_t)T * sp * (2 * c.pool_heads + C) * 4);
  }
  r.q = (float*)cv.take((size_t)T * C * 4);
  r.qp = (float*)cv.take((size_t)T * C * 4);
  r.o = (float*)cv.take((size_t)T * C * 4);
  r.y1 = (float*)cv.take((size_t)T * he * 4);
  r.y2 = (float*)cv.take((size_t)T * hh * 4);
  r.x = (float*)cv.take((size_t)T * hh * 4);
  r.x2 = (float*)cv.take((size_t)T * hh * 4);
  for (int i = 0; i < 3; ++i) {
    r.y1b[i] = (float*)cv.take((size_t)T * he * 4);
    r.y2b[i] = (float*)cv.take((size_t)T * hh * 4);
  }
  r.x3 = (float*)cv.take((size_t)T * hh * 4);
  r.sync = (unsigned long long*)cv.take(gating_fused_sync_words(T) * sizeof(unsigned long long));
  r.sc.need(T, (int)C, (int)C, 1);
  r.sc.need(T, (int)he, (int)hh, 1);
  r.sc.need(T, (int)hh, (int)he, 1);
  r.sc.need(T, (int)C / c.pool_heads, (int)C, c.pool_heads);
  r.sc.carve(cv);
  if (w) *w = r;
  return cv.off;
}

struct CompactWs {
  int32_t *cnt, *off, *rb;
  long long* src;
};
size_t plan_compact(int T, long long L, void* base, CompactWs* w) {
  Carver cv(base);
  CompactWs r{};
  const long long nb = compact_blocks(L);
  r.cnt = (int32_t*)cv.take((size_t)nb * 4);
  r.off = (int32_t*)cv.take((size_t)(nb + 1) * 4);
  r.rb = (int32_t*)cv.take((size_t)(T + 1) * 4);
  r.src = (long long*)cv.take((size_t)L * 8);
  if (w) *w = r;
  return cv.off;
}

struct CompactBatchWs {
  CompactWs c;
  int32_t *seq_img, *seq_ok, *layout_ok;
  long long* total;
};
size_t plan_compact_batch(int T, long long L, int B, void* base, CompactBatchWs* w) {
  CompactBatchWs r{};
  Carver cv(base);
  cv.off = plan_compact(T, L, base, &r.c);
  r.seq_img = (int32_t*)cv.take((size_t)(B + 1) * 4);
  r.seq_ok = (int32_t*)cv.take((size_t)(B + 1) * 4);
  r.total = (long long*)cv.take(8);
  r.layout_ok = (int32_t*)cv.take(4);
  if (w) *w = r;
  return cv.off;
}

}  // namespace

static void noalloc_scratch_init(int dev);

// ---------------------------------------------------------------------------
// create / destroy
// ---------------------------------------------------------------------------
extern "C" ivc_status ivc_connector_create(const ivc_config* cfg, const ivc_weights* w,
                                           void* stream, ivc_connector** out) {
  if (!cfg || !w || !out) return fail(IVC_ERR_INVALID_ARG, "null argument");
  TRACE("create dtype=%d C=%d P=%d has_cls=%d D=%d mlp1_hidden=%d flash=%d mlp2_hidden=%d "
        "pool=%dx%d heads gate=%dx%d pool_mode=%d ps_version=%d shuffle64_order=%d ln_fold=%d",
        cfg->dtype, cfg->vit_width, cfg->grid, cfg->has_cls, cfg->llm_width, cfg->mlp1_hidden,
        cfg->flash, cfg->mlp2_hidden, cfg->pool_layers, cfg->pool_heads, cfg->gate_hidden,
        cfg->gate_expansion, cfg->pool_mode, cfg->ps_version, cfg->shuffle64_order, cfg->ln_fold);
  *out = nullptr;
  ivc_status st = check_cfg(*cfg);
  if (st != IVC_OK) return st;
  const ivc_config& c = *cfg;
  hipStream_t s = (hipStream_t)stream;
  const int dt = c.dtype;
  const size_t e = dt == IVC_BF16 ? 2 : 4;
  const size_t C = c.vit_width, D = c.llm_width, H1 = c.mlp1_hidden, H2 = c.mlp2_hidden;
  const size_t Lp = c.pool_layers, hh = c.gate_hidden, he = hh * c.gate_expansion;

  // required pointers
  const void* req1[] = {w->mlp1_ln_w, w->mlp1_ln_b, w->mlp1_w1, w->mlp1_b1, w->mlp1_w2, w->mlp1_b2};
  for (const void* p : req1) {
    if (!p) return fail(IVC_ERR_INVALID_ARG, "missing mlp1 weight");
    if (!aligned16(p)) return fail(IVC_ERR_MISALIGNED, "weight pointer not 16-byte aligned");
  }
  if (c.flash) {
    const void* req2[] = {w->mlp2_ln_w, w->mlp2_ln_b, w->mlp2_w1, w->mlp2_b1, w->mlp2_w2,
                          w->mlp2_b2,   w->mlp2_w3,   w->mlp2_b3, w->pool_query, w->gate_cls_w,
                          w->gate_cls_b};
    for (const void* p : req2) {
      if (!p) return fail(IVC_ERR_INVALID_ARG, "missing mlp2/router weight");
      if (!aligned16(p)) return fail(IVC_ERR_MISALIGNED, "weight pointer not 16-byte aligned");
    }
    for (size_t l = 0; l < Lp; ++l) {
      const void* pl[] = {w->pool_wq[l], w->pool_bq[l], w->pool_wk[l], w->pool_bk[l],
                          w->pool_wv[l], w->pool_bv[l], w->pool_wo[l], w->pool_bo[l]};
      for (const void* p : pl)
        if (!p) return fail(IVC_ERR_INVALID_ARG, "missing pooling weight of layer %zu", l);
    }
    for (int b = 0; b < IVC_GATE_BLOCKS; ++b) {
      const void* pb[] = {w->gate_w1[b], w->gate_b1[b], w->gate_w2[b],
                          w->gate_b2[b], w->gate_ln_w[b], w->gate_ln_b[b]};
      for (const void* p : pb)
        if (!p) return fail(IVC_ERR_INVALID_ARG, "missing gating weight of block %d", b);
    }
  }

  ivc_connector* h = new ivc_connector();
  h->cfg = c;
  h->esz = (int)e;
  h->lr = (long long)C + (dt == IVC_BF16 ? 8 : 0);
  h->lg1 = (long long)hh + (dt == IVC_BF16 ? 8 : 0);
  h->lg2 = (long long)he + (dt == IVC_BF16 ? 8 : 0);
  {
    // the token pass of folded pooling splits its work over the compute units
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      h->ncu = n;
    h->dev = dev;
    // the device address of this device's copy of the no-allocation scratch
    // (ivc_connector_compact_noalloc); a failure is reported by that call
    noalloc_scratch_init(dev);
  }
  if (c.flash && dt == IVC_BF16) {
    if (hipStreamCreateWithFlags(&h->aux, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess ||
        hipStreamCreateWithFlags(&h->aux2, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_side, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      ivc_connector_destroy(h);
      return fail(IVC_ERR_HIP, "stream/event creation failed");
    }
  }
  Carver plan(nullptr);
  auto layout = [&](Carver& cv) {
    h->m1_ln_w = (float*)cv.take(4 * C * 4);
    h->m1_ln_b = (float*)cv.take(4 * C * 4);
    h->m1_w1 = cv.take(H1 * 4 * C * e);
    h->m1_b1 = (float*)cv.take(H1 * 4);
    h->m1_w2 = cv.take(D * H1 * e);
    h->m1_b2 = (float*)cv.take(D * 4);
    if (c.ln_fold) {
      h->m1_cs = (float*)cv.take(H1 * 4);
      if (c.flash) h->m2_cs = (float*)cv.take(H2 * 4);
    }
    if (c.flash) {
      h->m2_ln_w = (float*)cv.take(16 * C * 4);
      h->m2_ln_b = (float*)cv.take(16 * C * 4);
      h->m2_w1 = cv.take(H2 * 16 * C * e);
      h->m2_b1 = (float*)cv.take(H2 * 4);
      h->m2_w2 = cv.take(H2 * H2 * e);
      h->m2_b2 = (float*)cv.take(H2 * 4);
      h->m2_w3 = cv.take(D * H2 * e);
      h->m2_b3 = (float*)cv.take(D * 4);
      h->query = cv.take(C * e);
      h->query_f = (float*)cv.take(C * 4);
      for (size_t l = 0; l < Lp; ++l) {
        h->wq[l] = cv.take(C * h->lr * e);
        h->bq[l] = (float*)cv.take(C * 4);
        h->wo[l] = cv.take(C * h->lr * e);
        h->bo[l] = (float*)cv.take(C * 4);
      }
      h->wkv = cv.take(2 * Lp * C * h->lr * e);
      h->bkv = (float*)cv.take(2 * Lp * C * 4);
      h->wkT = dt == IVC_BF16 ? cv.take(Lp * C * h->lr * e) : nullptr;
      h->qt0_hi = dt == IVC_BF16 ? cv.take(16 * C * 2) : nullptr;
      h->qt0_lo = dt == IVC_BF16 ? cv.take(16 * C * 2) : nullptr;
      const bool qo = dt == IVC_BF16 && c.pool_mode == IVC_POOL_FOLDED &&
                      fold_query_fused_supported((int)C, c.pool_heads) && Lp > 1;
      for (size_t l = 0; l < Lp; ++l) {
        h->wqo_hi[l] = qo && l > 0 ? cv.take(C * h->lr * 2) : nullptr;
        h->wqo_lo[l] = qo && l > 0 ? cv.take(C * h->lr * 2) : nullptr;
        h->bqo[l] = qo && l > 0 ? (float*)cv.take(C * 4) : nullptr;
      }
      h->cr_woT = qo ? cv.take(C * C * 2) : nullptr;
      h->cr_wqo = qo ? (float*)cv.take(C * C * 4) : nullptr;
      for (int b = 0; b < IVC_GATE_BLOCKS; ++b) {
        h->g_w1[b] = cv.take(he * h->lg1 * e);
        h->g_b1[b] = (float*)cv.take(he * 4);
        h->g_w2[b] = cv.take(hh * h->lg2 * e);
        h->g_b2[b] = (float*)cv.take(hh * 4);
        h->g_lw[b] = (float*)cv.take(hh * 4);
        h->g_lb[b] = (float*)cv.take(hh * 4);
      }
      h->g_cw = cv.take(2 * hh * e);
      h->g_cb = (float*)cv.take(2 * 4);
    }
  };
  layout(plan);
  if (hipMalloc((void**)&h->blob, plan.off) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return fail(IVC_ERR_OOM, "hipMalloc of %zu bytes for weights failed", plan.off);
  }
  Carver real(h->blob);
  layout(real);

#define STEP(x)                   \
  do {                            \
    ivc_status s_ = (x);          \
    if (s_ != IVC_OK) {           \
      ivc_connector_destroy(h);   \
      return s_;                  \
    }                             \
  } while (0)
  auto fold_or_copy = [&](const void* W1, void* dst, size_t N, size_t K, const float* g,
                          const float* b, float* bias, float* cs) -> ivc_status {
    if (!c.ln_fold) return copy_mat(W1, dst, N * K * e, s);
    return launch_ln_fold_weights(W1, (int)N, (int)K, g, b, bias, dst, cs, bias, s) == hipSuccess
               ? IVC_OK
               : fail(IVC_ERR_HIP, "LayerNorm fold launch failed");
  };
  STEP(widen(w->mlp1_ln_w, dt, h->m1_ln_w, 4 * C, s));
  STEP(widen(w->mlp1_ln_b, dt, h->m1_ln_b, 4 * C, s));
  STEP(widen(w->mlp1_b1, dt, h->m1_b1, H1, s));
  STEP(fold_or_copy(w->mlp1_w1, h->m1_w1, H1, 4 * C, h->m1_ln_w, h->m1_ln_b, h->m1_b1, h->m1_cs));
  STEP(copy_mat(w->mlp1_w2, h->m1_w2, D * H1 * e, s));
  STEP(widen(w->mlp1_b2, dt, h->m1_b2, D, s));
  if (c.flash) {
    STEP(widen(w->mlp2_ln_w, dt, h->m2_ln_w, 16 * C, s));
    STEP(widen(w->mlp2_ln_b, dt, h->m2_ln_b, 16 * C, s));
    STEP(widen(w->mlp2_b1, dt, h->m2_b1, H2, s));
    STEP(fold_or_copy(w->mlp2_w1, h->m2_w1, H2, 16 * C, h->m2_ln_w, h->m2_ln_b, h->m2_b1,
                      h->m2_cs));
    STEP(copy_mat(w->mlp2_w2, h->m2_w2, H2 * H2 * e, s));
    STEP(widen(w->mlp2_b2, dt, h->m2_b2, H2, s));
    STEP(copy_mat(w->mlp2_w3, h->m2_w3, D * H2 * e, s));
    STEP(widen(w->mlp2_b3, dt, h->m2_b3, D, s));
    STEP(copy_mat(w->pool_query, h->query, C * e, s));
    STEP(widen(w->pool_query, dt, h->query_f, C, s));
    for (size_t l = 0; l < Lp; ++l) {
      STEP(copy_rows(w->pool_wq[l], h->wq[l], C, C, h->lr, e, s));
      STEP(widen(w->pool_bq[l], dt, h->bq[l], C, s));
      STEP(copy_rows(w->pool_wo[l], h->wo[l], C, C, h->lr, e, s));
      STEP(widen(w->pool_bo[l], dt, h->bo[l], C, s));
      STEP(copy_rows(w->pool_wk[l], (char*)h->wkv + (2 * l) * C * h->lr * e, C, C, h->lr, e, s));
      STEP(copy_rows(w->pool_wv[l], (char*)h->wkv + (2 * l + 1) * C * h->lr * e, C, C, h->lr, e,
                     s));
      if (h->wkT != nullptr)
        STEP(launch_transpose_bf16(w->pool_wk[l], (long long)C, (char*)h->wkT + l * C * h->lr * e,
                                   h->lr, (int)C, (int)C, s)
                     == hipSuccess
                 ? IVC_OK
                 : fail(IVC_ERR_HIP, "weight transpose launch failed"));
      STEP(widen(w->pool_bk[l], dt, h->bkv + (2 * l) * C, C, s));
      STEP(widen(w->pool_bv[l], dt, h->bkv + (2 * l + 1) * C, C, s));
    }
    for (int b = 0; b < IVC_GATE_BLOCKS; ++b) {
      STEP(copy_rows(w->gate_w1[b], h->g_w1[b], he, hh, h->lg1, e, s));
      STEP(widen(w->gate_b1[b], dt, h->g_b1[b], he, s));
      STEP(copy_rows(w->gate_w2[b], h->g_w2[b], hh, he, h->lg2, e, s));
      STEP(widen(w->gate_b2[b], dt, h->g_b2[b], hh, s));
      STEP(widen(w->gate_ln_w[b], dt, h->g_lw[b], hh, s));
      STEP(widen(w->gate_ln_b[b], dt, h->g_lb[b], hh, s));
    }
    STEP(copy_mat(w->gate_cls_w, h->g_cw, 2 * hh * e, s));
    STEP(widen(w->gate_cls_b, dt, h->g_cb, 2, s));
    if (h->qt0_hi != nullptr && c.pool_mode == IVC_POOL_FOLDED &&
        fold_query_fused_supported((int)C, c.pool_heads)) {
      // the first layer's folded query: the same arithmetic as the per-tile
      // launch of a route call, for one tile (every tile's would be equal)
      const int H = c.pool_heads;
      const float qscale = (1.0f / sqrtf((float)((int)C / H))) * 1.4426950408889634f;
      STEP(launch_fold_query_fused(h->query_f, 0, h->wq[0], h->lr, h->bq[0], h->wkT, h->lr,
                                   h->qt0_hi, h->qt0_lo, 1, (int)C, H, qscale, s) == hipSuccess
               ? IVC_OK
               : fail(IVC_ERR_HIP, "query fold launch failed"));
      if (H < 16)
        STEP(launch_zero_heads(h->qt0_hi, h->qt0_lo, 1, H, (int)C, s) == hipSuccess
                 ? IVC_OK
                 : fail(IVC_ERR_HIP, "query fold launch failed"));
    }
    for (size_t l = 1; l < Lp; ++l) {
      if (h->wqo_hi[l] == nullptr) continue;
      // Wqo = Wq_l Wo_{l-1}: A = Wq_l, W rows = columns of Wo_{l-1}; fp32 FMA
      GemmArgs g = mk_gemm(h->wq[l], h->lr, DT_BF16, h->cr_woT, DT_BF16, nullptr, h->cr_wqo,
                           DT_F32, (int)C, (int)C, (int)C, ACT_NONE);
      // bqo = Wq_l bo_{l-1} + bq_l
      GemmArgs gb = mk_gemm(h->bo[l - 1], (long long)C, DT_F32, h->wq[l], DT_BF16, h->bq[l],
                            h->bqo[l], DT_F32, 1, (int)C, (int)C, ACT_NONE);
      gb.ldw = h->lr;
      const bool ok =
          launch_transpose_bf16(h->wo[l - 1], h->lr, h->cr_woT, (long long)C, (int)C, (int)C, s) ==
              hipSuccess &&
          launch_gemm_simt(g, s) == hipSuccess &&
          launch_split_bf16(h->cr_wqo, h->wqo_hi[l], h->wqo_lo[l], (long long)C, (int)C, h->lr,
                            s) == hipSuccess &&
          launch_gemm_simt(gb, s) == hipSuccess;
      STEP(ok ? IVC_OK : fail(IVC_ERR_HIP, "query-output fold launch failed"));
    }
  }
#undef STEP
  if (hipStreamSynchronize(s) != hipSuccess) {
    hipError_t er = hipGetLastError();
    ivc_connector_destroy(h);
    return fail(IVC_ERR_HIP, "weight copy failed: %s", hipGetErrorString(er));
  }
  *out = h;
  return IVC_OK;
}

extern "C" void ivc_connector_destroy(ivc_connector* h) {
  if (!h) return;
  if (h->blob || h->aux) (void)hipDeviceSynchronize();
  if (h->blob) (void)hipFree(h->blob);
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  if (h->aux) (void)hipStreamDestroy(h->aux);
  if (h->ev_side) (void)hipEventDestroy(h->ev_side);
  if (h->aux2) (void)hipStreamDestroy(h->aux2);
  delete h;
}

// LayerNorm-fold statistics through per-token moments (bf16, C of 512 or
// 1024): the moments live past both the run and the route layouts, so the
// first token pass of forward can leave them for the run half.
static bool use_token_stats(const ivc_connector* h) {
  const ivc_config& c = h->cfg;
  return c.ln_fold && token_stats_supported(c.dtype, c.vit_width, c.grid * c.grid);
}
static size_t tokst_offset(const ivc_connector* h, int T) {
  const size_t a = plan_run(h, T, nullptr, nullptr), b = plan_route(h, T, nullptr, nullptr);
  return ((a > b ? a : b) + 255) & ~(size_t)255;
}
static size_t tokst_bytes(const ivc_connector* h, int T) {
  return use_token_stats(h) ? (size_t)T * h->cfg.grid * h->cfg.grid * 8 : 0;
}

extern "C" size_t ivc_connector_workspace_bytes(const ivc_connector* h, int32_t max_tiles,
                                                int64_t max_seq_len) {
  if (!h || max_tiles < 0 || max_seq_len < 0) return 0;
  const size_t m = tokst_offset(h, max_tiles) + tokst_bytes(h, max_tiles);
  const size_t c = plan_compact(max_tiles, max_seq_len, nullptr, nullptr);
  return m > c ? m : c;
}

// ---------------------------------------------------------------------------
// run
// ---------------------------------------------------------------------------
// The LayerNorm-folded products address a tile's gathered ViT rows with 32-bit
// byte offsets (route-first tiles may gather from anywhere in the batch), so a
// call keeps its ViT rows under this many bytes and larger batches run as
// consecutive sub-batches.  IVC_FOLD_CHUNK_BYTES sets a smaller cap (tests).
static long long fold_chunk_cap() {
  const long long def = (1ll << 31) - (1ll << 24);
  const char* e = getenv("IVC_FOLD_CHUNK_BYTES");
  if (e != nullptr && *e != '\0') {
    const long long v = atoll(e);
    if (v > 0 && v < def) return v;
  }
  return def;
}

// tokst_ready: the per-token moments are already in the workspace; lists_ready:
// so are the per-path tile lists of use64 (both left by forward's route half);
// tokst_in: the moments of these T tiles are here instead (a sub-batch of a
// call whose moments were made for the whole batch)
// side: work the caller adds at the point where the projector chains fork
// (on a stream of its own beside both chains when they fork; joined with the
// caller's stream at the end)
using SideWork = std::function<ivc_status(hipStream_t)>;
// Projector rows placed straight into a compacted sequence (forward_compact):
// the last product of each chain also writes every row to its compacted row,
// slot_dst[tile * S + slot] (the compaction's index half, which runs beside
// the chains, fills it; -1: nowhere).  Only the 256 x 256 DMA kernel can; a
// chain whose product runs elsewhere leaves its rows to the row copy.
struct DirectRows {
  const int32_t* slot_dst = nullptr;  // this call's tiles
  void* out = nullptr;                // the compacted embedding rows
  bool side_ordered = false;          // the index half precedes what is enqueued next on the stream
  bool all256 = true, all64 = true;   // every mlp1 / mlp2 last product placed its rows
};
static ivc_status run_impl(ivc_connector* h, const void* vit, int32_t T, const uint8_t* use64,
                           void* out256, void* out64, void* ws, size_t ws_bytes, void* stream,
                           bool tokst_ready = false, bool lists_ready = false,
                           const SideWork* side = nullptr, const float* tokst_in = nullptr,
                           DirectRows* dr = nullptr) {
  if (!h) return fail(IVC_ERR_INVALID_ARG, "null handle");
  TRACE("run%s T=%d vit=%p ws=%zu tokst_ready=%d lists_ready=%d", use64 ? "_routed" : "", T, vit,
        ws_bytes, (int)tokst_ready, (int)lists_ready);
  const ivc_config& c = h->cfg;
  if (T < 0) return fail(IVC_ERR_INVALID_ARG, "T = %d", T);
  if (T == 0) return IVC_OK;
  if (!vit || !out256 || (c.flash && !out64))
    return fail(IVC_ERR_INVALID_ARG, "null vit/out256%s", c.flash ? "/out64" : "");
  if (!aligned16(vit) || !aligned16(out256) || (out64 && !aligned16(out64)) || !aligned16(ws))
    return fail(IVC_ERR_MISALIGNED, "device pointers must be 16-byte aligned");
  const long long S = (long long)(c.grid / 2) * (c.grid / 2);
  if ((long long)T * S * 16 * c.vit_width > (1ll << 40))
    return fail(IVC_ERR_UNSUPPORTED, "T = %d too large", T);
  const bool tstats = use_token_stats(h);
  const size_t need = tstats ? tokst_offset(h, T) + tokst_bytes(h, T) : plan_run(h, T, nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return fail(IVC_ERR_WORKSPACE, "run needs %zu workspace bytes, got %zu", need, ws_bytes);
  const bool fold = c.ln_fold != 0;
  const long long rows_t = (long long)c.has_cls + (long long)c.grid * c.grid;
  const long long tile_bytes = rows_t * c.vit_width * h->esz;
  const long long cap = fold_chunk_cap();
  if (fold && (long long)T * tile_bytes >= cap) {
    // consecutive sub-batches under the cap, one after another on the stream
    // (tiles are independent; each sub-batch builds its own path lists, in the
    // workspace below where the whole batch's moments sit)
    const int per = (int)((cap - 1) / tile_bytes);
    if (per < 1) return fail(IVC_ERR_UNSUPPORTED, "ln_fold: one tile's ViT rows exceed the cap");
    const float* tok = tokst_in != nullptr ? tokst_in
                       : (tstats && tokst_ready) ? (const float*)((char*)ws + tokst_offset(h, T))
                                                 : nullptr;
    const long long S64 = (long long)(c.grid / 4) * (c.grid / 4);
    const size_t row = (size_t)c.llm_width * h->esz;
    for (int t0 = 0; t0 < T; t0 += per) {
      const int n = T - t0 < per ? T - t0 : per;
      DirectRows sub;
      if (dr != nullptr) {
        sub = *dr;
        sub.slot_dst = dr->slot_dst + (size_t)t0 * S;
      }
      const ivc_status st = run_impl(
          h, (const char*)vit + (size_t)t0 * tile_bytes, n, use64 ? use64 + t0 : nullptr,
          (char*)out256 + (size_t)t0 * S * row,
          out64 ? (void*)((char*)out64 + (size_t)t0 * S64 * row) : nullptr, ws, ws_bytes, stream,
          false, false, t0 == 0 ? side : nullptr,
          tok ? tok + (size_t)t0 * c.grid * c.grid * 2 : nullptr, dr != nullptr ? &sub : nullptr);
      if (dr != nullptr) {
        dr->side_ordered = sub.side_ordered;
        dr->all256 = dr->all256 && sub.all256;
        dr->all64 = dr->all64 && sub.all64;
      }
      if (st != IVC_OK) return st;
    }
    return IVC_OK;
  }
  RunWs w;
  plan_run(h, T, ws, &w);
  hipStream_t s = (hipStream_t)stream;
  const int dt = c.dtype;
  const int C = c.vit_width, D = c.llm_width, H1 = c.mlp1_hidden, H2 = c.mlp2_hidden;
  const int S4 = (c.grid / 4) * (c.grid / 4);

  // route-first: per-path tile ranks and lists from the decision
  RowMap rm256, rm64, rmh256, rmh64;
  if (use64 != nullptr) {
    if (!lists_ready)
      LAUNCH("route_lists", s,
             launch_route_lists(use64, T, w.rank, w.list256, w.list64, w.counts, s));
    rmh256.m_dev = w.counts;      // hidden rows of mlp1: n256 * S
    rmh256.m_mult = (int)S;
    rm256 = rmh256;               // final rows scatter back to the tile's slots
    rm256.c_map = w.list256;
    rm256.c_rpg = (int)S;
    rmh64.m_dev = w.counts + 1;
    rmh64.m_mult = S4;
    rm64 = rmh64;
    rm64.c_map = w.list64;
    rm64.c_rpg = S4;
  }

  ShuffleArgs sa{};
  sa.dtype = dt;
  sa.X = vit;
  sa.T = T;
  sa.P = c.grid;
  sa.C = C;
  sa.has_cls = c.has_cls;
  sa.flash = c.flash;
  sa.ln = 1;
  sa.g2 = h->m1_ln_w;
  sa.b2 = h->m1_ln_b;
  sa.out2 = fold ? nullptr : w.a2;
  sa.g4 = h->m2_ln_w;
  sa.b4 = h->m2_ln_b;
  sa.out4 = fold ? nullptr : w.a4;
  sa.st2 = fold ? w.st2 : nullptr;
  sa.st4 = fold && c.flash ? w.st4 : nullptr;
  sa.eps = c.ln_eps;
  sa.ps_v1 = c.ps_version == 1;
  sa.twice_r2 = c.shuffle64_order == IVC_SHUFFLE64_TWICE_R2;
  if (use64 != nullptr) {
    sa.use64 = use64;
    sa.rank = w.rank;
  }
  if (fold && tstats) {
    // per-token moments (unless the first token pass left them), then each
    // shuffled row's (mean, rstd) from its 4 or 16 cells
    float* tokst = tokst_in != nullptr ? const_cast<float*>(tokst_in)
                                       : (float*)((char*)ws + tokst_offset(h, T));
    if (!tokst_ready && tokst_in == nullptr)
      LAUNCH("token_stats", s,
             launch_token_stats(vit, T, c.has_cls + c.grid * c.grid, c.has_cls, c.grid * c.grid,
                                C, tokst, s,
                                c.flash && (C == 512 || C == 1024)));  // as the token pass
    LAUNCH("ln_stats", s, launch_ln_stats(tokst, T, c.grid, C, c.ln_eps, sa.ps_v1, c.flash,
                                          sa.use64, sa.rank, sa.st2, sa.st4, s));
  } else {
    LAUNCH("shuffle_ln", s, launch_shuffle_ln(sa, s));
  }

  // The mlp1 and mlp2 chains are independent: with a second stream the tail
  // workgroups of one chain's products share the chip with the other's
  // instead of leaving compute units idle.  (bf16 only: the fp32 products
  // share one SIMT scratch buffer.)
  // (While per-kernel timing is on, both chains stay on the caller's stream so
  // each kernel's events time it alone.)
  const bool fork = c.flash && h->aux != nullptr && (!g_prof_on || g_prof_keep_fork);
  hipStream_t s1 = s;
  if (fork) {
    HIP_OK(hipEventRecord(h->ev_fork, s));
    HIP_OK(hipStreamWaitEvent(h->aux, h->ev_fork, 0));
    s1 = h->aux;
  }
  // side work starts here too, on a third stream when the chains fork: its
  // small workgroups take compute units as the products' tiles free them
  const bool side_apart = side != nullptr && fork && h->aux2 != nullptr;
  if (side != nullptr) {
    hipStream_t ss = s;
    if (side_apart) {
      HIP_OK(hipStreamWaitEvent(h->aux2, h->ev_fork, 0));
      ss = h->aux2;
    }
    const ivc_status st = (*side)(ss);
    if (side_apart) {  // joined below, or here if the side work failed
      HIP_OK(hipEventRecord(h->ev_side, ss));
      if (st != IVC_OK) (void)hipStreamWaitEvent(s, h->ev_side, 0);
    }
    if (st != IVC_OK) {
      if (fork) {  // nothing was enqueued on the mlp1 chain's stream yet
        (void)hipEventRecord(h->ev_join, s1);
        (void)hipStreamWaitEvent(s, h->ev_join, 0);
      }
      return st;
    }
  }
  // the last products may place their rows in the compacted sequence once the
  // index half is ordered before them (on its own stream: an event wait)
  const bool direct = dr != nullptr && use64 != nullptr &&
                      (dr->side_ordered || (side != nullptr && (side_apart || !fork)));
  auto place = [&](GemmArgs& g, hipStream_t st, bool& all) -> ivc_status {
    GemmArgs t = g;
    t.rm.d_map = direct ? dr->slot_dst : nullptr;
    t.rm.d_stride = (int)S;
    t.rm.d_out = direct ? dr->out : nullptr;
    if (!direct || !gemm_takes_dma(t)) {
      if (dr != nullptr) all = false;
      return IVC_OK;
    }
    if (side_apart) HIP_OK(hipStreamWaitEvent(st, h->ev_side, 0));
    g = t;
    return IVC_OK;
  };
  bool unused = false;
  const int M2 = (int)(T * S);
  // first product of a projector: the LayerNorm'd rows, or (ln_fold) the raw
  // ViT rows gathered in shuffle order with the LayerNorm applied in the epilogue
  auto first_gemm = [&](int r, void* a_rows, const float* st, const int* list, const void* W1,
                        const float* b1, const float* cs, void* out, int M, int N,
                        const RowMap& rm) -> GemmArgs {
    GemmArgs f;
    if (!fold) {
      f = mk_gemm(a_rows, (long long)r * r * C, dt, W1, dt, b1, out, dt, M, N, r * r * C, ACT_GELU);
    } else {
      f = mk_gemm(vit, C, dt, W1, dt, b1, out, dt, M, N, r * r * C, ACT_GELU);
      f.fold = 1;
      f.ag.list = list;
      f.ag.rows = c.has_cls + c.grid * c.grid;
      f.ag.has_cls = c.has_cls;
      f.ag.P = c.grid;
      f.ag.r = r;
      f.ag.C = C;
      f.ag.v1 = c.ps_version == 1;
      f.ag.twice = r == 4 && c.shuffle64_order == IVC_SHUFFLE64_TWICE_R2;
      f.ln_rows = st;
      f.ln_colsum = cs;
    }
    f.rm = rm;
    return f;
  };
  GemmArgs g;
  g = first_gemm(2, w.a2, w.st2, use64 ? w.list256 : nullptr, h->m1_w1, h->m1_b1, h->m1_cs, w.h1,
                 M2, H1, rmh256);
  if (fold) {
    if (!gemm_dma_supported(g)) return fail(IVC_ERR_UNSUPPORTED, "ln_fold: mlp1 product shape");
    with_tail(g, h, w.tail);
    trace_gemm("mlp1_gemm1", g, "256x256 LDS-DMA MFMA, gathered A");
    LAUNCH("mlp1_gemm1", s1, launch_gemm_dma(g, s1));
  } else {
    with_tail(g, h, w.tail);
    LAUNCH("mlp1_gemm1", s1, gemm("mlp1_gemm1", g, s1, &w.sc));
  }
  g = mk_gemm(w.h1, H1, dt, h->m1_w2, dt, h->m1_b2, out256, dt, M2, D, H1, ACT_NONE);
  g.rm = rm256;
  with_tail(g, h, w.tail);
  {
    const ivc_status pst = place(g, s1, dr != nullptr ? dr->all256 : unused);
    if (pst != IVC_OK) return pst;
  }
  LAUNCH("mlp1_gemm2", s1, gemm("mlp1_gemm2", g, s1, &w.sc));
  if (fork) HIP_OK(hipEventRecord(h->ev_join, s1));
  if (c.flash) {
    const int M4 = T * S4;
    g = first_gemm(4, w.a4, w.st4, use64 ? w.list64 : nullptr, h->m2_w1, h->m2_b1, h->m2_cs, w.g1,
                   M4, H2, rmh64);
    if (fold) {
      if (!gemm_dma_supported(g)) return fail(IVC_ERR_UNSUPPORTED, "ln_fold: mlp2 product shape");
      trace_gemm("mlp2_gemm1", g, "256x256 LDS-DMA MFMA, gathered A");
      LAUNCH("mlp2_gemm1", s, launch_gemm_dma(g, s));
    } else {
      LAUNCH("mlp2_gemm1", s, gemm("mlp2_gemm1", g, s, &w.sc));
    }
    g = mk_gemm(w.g1, H2, dt, h->m2_w2, dt, h->m2_b2, w.g2, dt, M4, H2, H2, ACT_GELU);
    g.rm = rmh64;
    LAUNCH("mlp2_gemm2", s, gemm("mlp2_gemm2", g, s, &w.sc));
    g = mk_gemm(w.g2, H2, dt, h->m2_w3, dt, h->m2_b3, out64, dt, M4, D, H2, ACT_NONE);
    g.rm = rm64;
    {
      const ivc_status pst = place(g, s, dr != nullptr ? dr->all64 : unused);
      if (pst != IVC_OK) return pst;
    }
    LAUNCH("mlp2_gemm3", s, gemm("mlp2_gemm3", g, s, &w.sc));
  }
  if (fork) HIP_OK(hipStreamWaitEvent(s, h->ev_join, 0));
  if (side_apart) HIP_OK(hipStreamWaitEvent(s, h->ev_side, 0));
  // whatever is enqueued on s next follows the side work
  if (dr != nullptr && side != nullptr) dr->side_ordered = true;
  return IVC_OK;
}

extern "C" ivc_status ivc_connector_run(ivc_connector* h, const void* vit, int32_t T,
                                        void* out256, void* out64, void* ws, size_t ws_bytes,
                                        void* stream) {
  return run_impl(h, vit, T, nullptr, out256, out64, ws, ws_bytes, stream);
}

extern "C" ivc_status ivc_connector_run_routed(ivc_connector* h, const void* vit, int32_t T,
                                               const uint8_t* use64, void* out256, void* out64,
                                               void* ws, size_t ws_bytes, void* stream) {
  if (!h) return fail(IVC_ERR_INVALID_ARG, "null handle");
  if (!h->cfg.flash) return fail(IVC_ERR_INVALID_ARG, "route-first run needs a flash connector");
  if (T > 0 && !use64) return fail(IVC_ERR_INVALID_ARG, "null use64");
  return run_impl(h, vit, T, use64, out256, out64, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// route
// ---------------------------------------------------------------------------
// tokst: if set, the first token pass also leaves every token's LayerNorm
// moments there (forward; folded pooling, no padding mask)
// lists: if set (rank, list256, list64, counts of the run workspace), the
// decision kernel also writes the per-path tile lists (forward)
static ivc_status route_impl(ivc_connector* h, const void* vit, const int32_t* valid_tokens,
                             int32_t T, float* gate, double* threshold, uint8_t* use64,
                             float* pooled, int32_t* dev_status, void* ws, size_t ws_bytes,
                             void* stream, float* tokst = nullptr, const RunWs* lists = nullptr) {
  if (!h) return fail(IVC_ERR_INVALID_ARG, "null handle");
  TRACE("route T=%d vit=%p valid=%p pool_mode=%d ws=%zu token_moments=%d", T, vit,
        (const void*)valid_tokens, h->cfg.pool_mode, ws_bytes, tokst != nullptr);
  const ivc_config& c = h->cfg;
  if (!c.flash) return fail(IVC_ERR_INVALID_ARG, "route needs a flash connector");
  if (T < 0) return fail(IVC_ERR_INVALID_ARG, "T = %d", T);
  if (T == 0) return IVC_OK;
  if (!vit || !gate || !threshold || !use64)
    return fail(IVC_ERR_INVALID_ARG, "null vit/gate/threshold/use64");
  if (!aligned16(vit) || !aligned16(ws)) return fail(IVC_ERR_MISALIGNED, "vit/ws alignment");
  const size_t need = plan_route(h, T, nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return fail(IVC_ERR_WORKSPACE, "route needs %zu workspace bytes, got %zu", need, ws_bytes);
  RouteWs w;
  plan_route(h, T, ws, &w);
  hipStream_t s = (hipStream_t)stream;
  const int dt = c.dtype;
  const int C = c.vit_width, N = c.grid * c.grid, L = c.pool_layers, H = c.pool_heads;
  const int rows = c.has_cls + N;
  const int hh = c.gate_hidden, he = hh * c.gate_expansion;

  const bool folded = c.pool_mode == IVC_POOL_FOLDED;
  // router product with fp32 activations and one of the connector's router
  // matrices (rows at stride ldw)
  auto rgemm = [&](const float* A, long long lda, const void* W, long long ldw, const float* bias,
                   float* Cout, int M, int Nn, int K, int act) {
    GemmArgs g = mk_gemm(A, lda, DT_F32, W, dt, bias, Cout, DT_F32, M, Nn, K, act);
    g.ldw = ldw;
    return g;
  };
  if (!folded) {
    // K and V of every layer from the raw tokens (CLS skipped by the row remap)
    GemmArgs kv = mk_gemm(vit, C, dt, h->wkv, dt, h->bkv, w.kv, dt, T * N, 2 * L * C, C, ACT_NONE);
    kv.ldw = h->lr;
    kv.a_rpg = N;
    kv.a_gstride = rows;
    kv.a_goff = c.has_cls;
    LAUNCH("pool_kv_gemm", s, gemm("pool_kv_gemm", kv, s));
  }

  // The pooling's last output projection and the Gating network in one
  // launch (IVC_GATING_FUSED=0 selects the launch-per-product form, which
  // does the same arithmetic).
  const bool gate1 = dt == IVC_BF16 && gating_fused_supported(T, (int)hh, (int)he) &&
                     hh == C && !env_off("IVC_GATING_FUSED");
  // query projection and key fold in one launch where the shape allows it;
  // its first layer reads the learned query as a row of stride 0 for every tile
  const bool fq_fused = c.pool_mode == IVC_POOL_FOLDED && h->wkT != nullptr &&
                        fold_query_fused_supported(C, c.pool_heads);
  if (!fq_fused) LAUNCH("pool_query", s, launch_broadcast_rows(dt, h->query, w.q, T, C, s));
  const int splits = pool_splits(T, N);
  const float scale = 1.0f / sqrtf((float)(C / H));
  int fG = 0, fQ = 0, fseg = 0;
  if (folded) folded_geometry(T, N, C, h->ncu, &fG, &fQ, &fseg);
  // A layer's value fold runs in one launch with the next layer's query fold,
  // and the last layer's in the one-launch Gating (IVC_FOLD_MERGED=0 keeps
  // them apart; the same arithmetic either way).
  const bool vq_ok = folded && fq_fused && dt == IVC_BF16 && !env_off("IVC_FOLD_MERGED");
  bool qt_made = false;      // this layer's q~ came with the previous layer's value fold
  bool vf_in_gating = false;  // the last value fold runs as the Gating launch's first phase
  for (int l = 0; l < L; ++l) {
    const void* wk = (const char*)h->wkv + (size_t)(2 * l) * C * h->lr * h->esz;
    const void* wv = (const char*)h->wkv + (size_t)(2 * l + 1) * C * h->lr * h->esz;
    const float* bv = h->bkv + (size_t)(2 * l + 1) * C;
    // q~_h = Wk_h^T q_h * log2(e) / sqrt(d) (scores in log2 units), per head
    // a product [T, d] x [d, C] with the transposed key weights
    const float qscale = scale * 1.4426950408889634f;
    // the first layer's folded query is the same for every tile: made once at create
    const bool qt_shared = fq_fused && l == 0 && h->qt0_hi != nullptr;
    if (fq_fused) {
      if (!qt_shared && !qt_made) {
        // l >= 1: from the previous layer's value-fold output o through the
        // folded output + query projections (or through q when not folded)
        const bool qo = h->wqo_hi[l] != nullptr;
        LAUNCH("pool_query_fold", s,
               launch_fold_query_fused(qo ? w.o : w.q, C, qo ? h->wqo_hi[l] : h->wq[l], h->lr,
                                       qo ? h->bqo[l] : h->bq[l],
                                       (const char*)h->wkT + (size_t)l * C * h->lr * h->esz,
                                       h->lr, w.qt_hi, w.qt_lo, T, C, H, qscale, s,
                                       qo ? h->wqo_lo[l] : nullptr));
      }
      if (l == 0 && H < 16)  // heads H .. 15 of the per-tile buffers, read by the later layers
        LAUNCH("pool_fold_pad", s, launch_zero_heads(w.qt_hi, w.qt_lo, T, H, C, s));
    } else {
      LAUNCH("pool_q_proj", s, gemm("pool_q_proj",
                                   rgemm(w.q, C, h->wq[l], h->lr, h->bq[l], w.qp, T, C, C,
                                         ACT_NONE), s, &w.sc));
    }
    if (folded) {
      if (fq_fused) {
        // q~ already written by the fused launch
      } else if (h->wkT != nullptr) {
        const int d = C / H;
        const void* wkT_l = (const char*)h->wkT + (size_t)l * C * h->lr * h->esz;
        GemmArgs fq = mk_gemm(w.qp, C, DT_F32, wkT_l, DT_BF16, nullptr, w.qt_hi, DT_BF16, T, C, d,
                              ACT_NONE);
        fq.ldw = h->lr;
        fq.ldc = 16ll * C;
        fq.batch = H;
        fq.a_bs = d;
        fq.w_bs = d;
        fq.c_bs = C;
        LAUNCH("pool_fold_query", s, launch_gemm_f32a(fq, 1, w.qt_lo, qscale, s));
        if (l == 0 && H < 16)
          LAUNCH("pool_fold_pad", s, launch_zero_heads(w.qt_hi, w.qt_lo, T, H, C, s));
      } else {
        LAUNCH("pool_fold_query", s,
               launch_fold_query(dt, w.qp, wk, w.qt_hi, w.qt_lo, T, C, H, qscale, s));
      }
      FoldedArgs fa{};
      fa.dtype = dt;
      fa.X = vit;
      fa.rows = rows;
      fa.has_cls = c.has_cls;
      fa.valid = valid_tokens;
      fa.status = dev_status;
      fa.T = T;
      fa.N = N;
      fa.C = C;
      fa.H = H;
      fa.qt_hi = qt_shared ? h->qt0_hi : w.qt_hi;
      fa.qt_lo = qt_shared ? h->qt0_lo : w.qt_lo;
      fa.qt_shared = qt_shared;
      fa.G = fG;
      fa.Q = fQ;
      fa.segmax = fseg;
      fa.part = w.part;
      fa.tokst = l == 0 ? tokst : nullptr;
      // odd layers walk their ranges backwards: they start on the tokens the
      // previous layer read last, which the 256 MB memory-side cache still holds
      fa.reverse = l & 1;
      // o_h = Wv_h xbar_h + bv_h for every head: one batched product over heads,
      // with bf16 weights reading the token pass's partials directly (the merge
      // of a tile's partials happens in its operand load)
      const bool merged_value = dt == IVC_BF16 && fold_value_merged_max_parts(T, N, fQ) <= 4;
      fa.xbar = merged_value ? nullptr : w.xbar;
      // the first layer's pass also writes per-token LayerNorm moments: timed apart
      LAUNCH(fa.tokst ? "pool_folded_stats" : "pool_folded", s, launch_pool_folded(fa, s));
      const bool next_vq = merged_value && vq_ok && l + 1 < L && h->wqo_hi[l + 1] != nullptr &&
                           h->wqo_lo[l + 1] != nullptr &&
                           fold_value_query_supported(T, N, fQ, C, H);
      qt_made = false;
      if (next_vq) {
        FoldVQArgs va;
        va.part = w.part;
        va.valid = valid_tokens;
        va.N = N;
        va.Q = fQ;
        va.segmax = fseg;
        va.Wv = (const uint16_t*)wv;
        va.ldwv = h->lr;
        va.bv = bv;
        va.o = w.o;
        va.Wq = (const uint16_t*)h->wqo_hi[l + 1];
        va.Wq_lo = (const uint16_t*)h->wqo_lo[l + 1];
        va.ldwq = h->lr;
        va.bq = h->bqo[l + 1];
        va.WkT = (const uint16_t*)((const char*)h->wkT + (size_t)(l + 1) * C * h->lr * h->esz);
        va.ldk = h->lr;
        va.qt_hi = (uint16_t*)w.qt_hi;
        va.qt_lo = (uint16_t*)w.qt_lo;
        va.scale = qscale;
        va.T = T;
        va.C = C;
        va.H = H;
        va.sync = w.sync;
        va.tag = next_ticket() & 0xffffffffffffull;
        va.status = dev_status;
        LAUNCH("pool_fold_value_query", s, launch_fold_value_query(va, s));
        qt_made = true;
      } else if (merged_value && vq_ok && gate1 && l == L - 1) {
        vf_in_gating = true;  // made by the Gating launch
      } else if (merged_value) {
        LAUNCH("pool_fold_value", s,
               launch_fold_value_merged(w.part, valid_tokens, N, fQ, fseg, wv, h->lr, bv, w.o, T,
                                        C, H, s));
      } else {
        const int d = C / H;
        GemmArgs fv = mk_gemm(w.xbar, (long long)H * C, DT_F32, wv, dt, bv, w.o, DT_F32, T, d, C,
                              ACT_NONE);
        fv.ldc = C;
        fv.ldw = h->lr;
        fv.batch = H;
        fv.a_bs = C;
        fv.w_bs = (long long)d * h->lr;
        fv.c_bs = d;
        fv.bias_bs = d;
        LAUNCH("pool_fold_value", s, gemm("pool_fold_value", fv, s, &w.sc));
      }
    } else {
      PoolAttnArgs pa{};
      pa.dtype = dt;
      pa.KV = w.kv;
      pa.kv_ld = 2ll * L * C;
      pa.kcol = 2 * l * C;
      pa.vcol = (2 * l + 1) * C;
      pa.Q = w.qp;
      pa.valid = valid_tokens;
      pa.status = dev_status;
      pa.T = T;
      pa.N = N;
      pa.C = C;
      pa.H = H;
      pa.splits = splits;
      pa.part = w.part;
      pa.O = w.o;
      LAUNCH("pool_attn", s, launch_pool_attn(pa, s));
    }
    // the output projection, unless the next layer's query fold reads o itself
    // through the folded weights (only the last layer's q, the pooled vector, is formed)
    if (!(fq_fused && l + 1 < L && h->wqo_hi[l + 1] != nullptr) && !(gate1 && l == L - 1)) {
      float* qn = (l == L - 1 && pooled) ? pooled : w.q;
      LAUNCH("pool_o_proj", s, gemm("pool_o_proj",
                                   rgemm(w.o, C, h->wo[l], h->lr, h->bo[l], qn, T, C, C, ACT_NONE),
                                   s, &w.sc));
    }
  }
  const float* pooled_v = pooled ? pooled : w.q;

  // Gating: x = pooled; 4 x (x += LN(W2 GELU(W1 x + b1) + b2)); softmax(Wc x + bc)
  static_assert(IVC_GATE_BLOCKS >= 2, "the gating chain below alternates two row buffers");
  if (gate1) {
    static_assert(IVC_GATE_BLOCKS == 4, "the one-launch Gating runs four blocks");
    GatingFusedArgs ga;
    if (vf_in_gating) {
      ga.vf_part = w.part;
      ga.vf_valid = valid_tokens;
      ga.vf_N = N;
      ga.vf_Q = fQ;
      ga.vf_segmax = fseg;
      ga.vf_H = H;
      ga.vf_wv = (const uint16_t*)((const char*)h->wkv + (size_t)(2 * (L - 1) + 1) * C * h->lr *
                                                             h->esz);
      ga.vf_ldw = h->lr;
      ga.vf_bv = h->bkv + (size_t)(2 * (L - 1) + 1) * C;
    }
    ga.o = w.o;
    ga.wo = (const uint16_t*)h->wo[L - 1];
    ga.ldwo = h->lr;
    ga.bo = h->bo[L - 1];
    ga.xb[0] = const_cast<float*>(pooled_v);
    ga.xb[1] = w.x;
    ga.xb[2] = w.x2;
    ga.xb[3] = w.x3;
    ga.y1[0] = w.y1;
    ga.y2[0] = w.y2;
    for (int i = 0; i < 3; ++i) {
      ga.y1[i + 1] = w.y1b[i];
      ga.y2[i + 1] = w.y2b[i];
    }
    for (int b = 0; b < 4; ++b) {
      ga.w1[b] = (const uint16_t*)h->g_w1[b];
      ga.w2[b] = (const uint16_t*)h->g_w2[b];
      ga.b1[b] = h->g_b1[b];
      ga.b2[b] = h->g_b2[b];
      ga.lw[b] = h->g_lw[b];
      ga.lb[b] = h->g_lb[b];
    }
    ga.ldw1 = h->lg1;
    ga.ldw2 = h->lg2;
    ga.wc = (const uint16_t*)h->g_cw;
    ga.bc = h->g_cb;
    ga.gate = gate;
    ga.T = T;
    ga.h = (int)hh;
    ga.he = (int)he;
    ga.eps = c.ln_eps;
    ga.sync = w.sync;
    ga.tag = next_ticket() & 0xffffffffffffull;
    ga.status = dev_status;
    LAUNCH("gating", s, launch_gating_fused(ga, s));
  } else if (dt == IVC_BF16 && f32a_ln_rows_supported(hh)) {
    // block b > 0 takes block b-1's residual LayerNorm into its first Linear's
    // prologue (rows alternate between two buffers; block 0 reads the pooled
    // rows in place); the last block's LayerNorm runs with the classifier head
    const float* xb = pooled_v;
    for (int b = 0; b < IVC_GATE_BLOCKS; ++b) {
      if (b == 0) {
        LAUNCH("gate_fc1", s, gemm("gate_fc1",
                                  rgemm(xb, hh, h->g_w1[b], h->lg1, h->g_b1[b], w.y1, T, he, hh,
                                        ACT_GELU), s, &w.sc));
      } else {
        float* xn = (b & 1) ? w.x : w.x2;
        LAUNCH("gate_ln_fc1", s,
               launch_f32a_ln_rows(xb, w.y2, h->g_lw[b - 1], h->g_lb[b - 1], c.ln_eps, xn,
                                   h->g_w1[b], h->lg1, h->g_b1[b], w.y1, T, he, hh, ACT_GELU, s));
        xb = xn;
      }
      LAUNCH("gate_fc2", s, gemm("gate_fc2",
                                rgemm(w.y1, he, h->g_w2[b], h->lg2, h->g_b2[b], w.y2, T, hh, he,
                                      ACT_NONE), s, &w.sc));
    }
    const int b = IVC_GATE_BLOCKS - 1;
    LAUNCH("gate_res_ln_head", s,
           launch_residual_ln_head(dt, const_cast<float*>(xb), w.y2, h->g_lw[b], h->g_lb[b], T,
                                   hh, c.ln_eps, h->g_cw, h->g_cb, gate, s));
  } else {
    HIP_OK(hipMemcpyAsync(w.x, pooled_v, (size_t)T * hh * 4, hipMemcpyDeviceToDevice, s));
    for (int b = 0; b < IVC_GATE_BLOCKS; ++b) {
      LAUNCH("gate_fc1", s, gemm("gate_fc1",
                                rgemm(w.x, hh, h->g_w1[b], h->lg1, h->g_b1[b], w.y1, T, he, hh,
                                      ACT_GELU), s, &w.sc));
      LAUNCH("gate_fc2", s, gemm("gate_fc2",
                                rgemm(w.y1, he, h->g_w2[b], h->lg2, h->g_b2[b], w.y2, T, hh, he,
                                      ACT_NONE), s, &w.sc));
      if (b + 1 < IVC_GATE_BLOCKS)
        LAUNCH("gate_res_ln", s,
               launch_residual_ln(w.x, w.y2, h->g_lw[b], h->g_lb[b], T, hh, c.ln_eps, s));
      else  // the last block's residual LayerNorm and the classifier head in one launch
        LAUNCH("gate_res_ln_head", s,
               launch_residual_ln_head(dt, w.x, w.y2, h->g_lw[b], h->g_lb[b], T, hh, c.ln_eps,
                                       h->g_cw, h->g_cb, gate, s));
    }
  }
  LAUNCH("quantile_decide", s,
         launch_quantile_decide(gate, T, c.rel_quantile, c.abs_threshold, threshold, use64, s,
                                lists ? lists->rank : nullptr, lists ? lists->list256 : nullptr,
                                lists ? lists->list64 : nullptr, lists ? lists->counts : nullptr));
  return IVC_OK;
}

extern "C" ivc_status ivc_connector_route(ivc_connector* h, const void* vit,
                                          const int32_t* valid_tokens, int32_t T, float* gate,
                                          double* threshold, uint8_t* use64, float* pooled,
                                          int32_t* dev_status, void* ws, size_t ws_bytes,
                                          void* stream) {
  return route_impl(h, vit, valid_tokens, T, gate, threshold, use64, pooled, dev_status, ws,
                    ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// forward = route + route-first run in one call
// ---------------------------------------------------------------------------

static ivc_status forward_impl(ivc_connector* h, const void* vit, const int32_t* valid_tokens,
                               int32_t T, float* gate, double* threshold, uint8_t* use64,
                               float* pooled, int32_t* dev_status, void* out256, void* out64,
                               void* ws, size_t ws_bytes, void* stream, const SideWork* side,
                               DirectRows* dr = nullptr) {
  if (!h) return fail(IVC_ERR_INVALID_ARG, "null handle");
  if (!h->cfg.flash) return fail(IVC_ERR_INVALID_ARG, "forward needs a flash connector");
  if (T > 0 && (!out256 || !out64)) return fail(IVC_ERR_INVALID_ARG, "null out256/out64");
  // the LayerNorm-fold statistics come out of the first token pass when it
  // reads every token (folded pooling, no padding mask): one less pass over
  // the ViT tensor
  const ivc_config& c = h->cfg;
  float* tokst = nullptr;
  if (T > 0 && use_token_stats(h) && c.pool_mode == IVC_POOL_FOLDED && valid_tokens == nullptr &&
      pool_folded_supported(c.dtype, c.vit_width, c.pool_heads)) {
    const size_t need = tokst_offset(h, T) + tokst_bytes(h, T);
    if (!ws || ws_bytes < need)
      return fail(IVC_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (!aligned16(ws)) return fail(IVC_ERR_MISALIGNED, "ws alignment");
    tokst = (float*)((char*)ws + tokst_offset(h, T));
  }
  // the decision kernel also leaves the per-path tile lists where the run half
  // reads them (the run layout may overlap the route scratch, which the
  // decision kernel, the route's last, no longer reads)
  RunWs rl{};
  const bool lists = T > 0 && ws != nullptr && ws_bytes >= plan_run(h, T, nullptr, nullptr);
  if (lists) plan_run(h, T, ws, &rl);
  ivc_status st = route_impl(h, vit, valid_tokens, T, gate, threshold, use64, pooled, dev_status,
                             ws, ws_bytes, stream, tokst, lists ? &rl : nullptr);
  if (st != IVC_OK) return st;
  return run_impl(h, vit, T, use64, out256, out64, ws, ws_bytes, stream, tokst != nullptr, lists,
                  side, nullptr, dr);
}

extern "C" ivc_status ivc_connector_forward(ivc_connector* h, const void* vit,
                                            const int32_t* valid_tokens, int32_t T, float* gate,
                                            double* threshold, uint8_t* use64, float* pooled,
                                            int32_t* dev_status, void* out256, void* out64,
                                            void* ws, size_t ws_bytes, void* stream) {
  TRACE("forward T=%d (route, then route-first run)", T);
  return forward_impl(h, vit, valid_tokens, T, gate, threshold, use64, pooled, dev_status, out256,
                      out64, ws, ws_bytes, stream, nullptr);
}

// ---------------------------------------------------------------------------
// compact
// ---------------------------------------------------------------------------
// checks a compaction's arguments and lays out its workspace (nothing launched)
static ivc_status compact_prep(ivc_connector* h, const int32_t* ids, const void* embeds,
                               int64_t L, int32_t img_context_id, const uint8_t* use64,
                               const void* out256, const void* out64, int32_t T, int32_t* out_ids,
                               int32_t* out_pos, int32_t* keep_map, void* out_embeds,
                               int64_t* out_len, int32_t* dev_status, void* ws, size_t ws_bytes,
                               CompactArgs* out) {
  if (!h) return fail(IVC_ERR_INVALID_ARG, "null handle");
  const ivc_config& c = h->cfg;
  if (L < 0 || T < 0) return fail(IVC_ERR_INVALID_ARG, "negative L or T");
  if (L > 0x7fffffffll) return fail(IVC_ERR_UNSUPPORTED, "L above INT32_MAX");
  if (!out_len || !dev_status) return fail(IVC_ERR_INVALID_ARG, "null out_len/dev_status");
  const long long S = (long long)(c.grid / 2) * (c.grid / 2);
  const long long S64 = (long long)(c.grid / 4) * (c.grid / 4);
  if ((long long)T * S >= (1ll << 31)) return fail(IVC_ERR_UNSUPPORTED, "T * S too large");
  if (L > 0 && (!ids || !embeds || !out_ids || !out_pos || !keep_map || !out_embeds))
    return fail(IVC_ERR_INVALID_ARG, "null sequence pointer");
  if (T > 0 && (!use64 || !out256)) return fail(IVC_ERR_INVALID_ARG, "null use64/out256");
  if (T > 0 && !out64 && !c.flash) {
    // a non-flash connector may compact with an all-zero use64 and no out64
  } else if (T > 0 && !out64) {
    return fail(IVC_ERR_INVALID_ARG, "null out64");
  }
  if (!aligned16(embeds) || !aligned16(out256) || !aligned16(out64) || !aligned16(out_embeds) ||
      !aligned16(ws))
    return fail(IVC_ERR_MISALIGNED, "embedding pointers must be 16-byte aligned");
  const size_t need = plan_compact(T, L, nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return fail(IVC_ERR_WORKSPACE, "compact needs %zu workspace bytes, got %zu", need, ws_bytes);
  CompactWs w;
  plan_compact(T, L, ws, &w);
  CompactArgs a{};
  a.dtype = c.dtype;
  a.ids = ids;
  a.embeds = embeds;
  a.L = L;
  a.img_id = img_context_id;
  a.use64 = use64;
  a.out256 = out256;
  a.out64 = out64 ? out64 : out256;
  a.T = T;
  a.S = (int)S;
  a.S64 = c.flash ? (int)S64 : (int)S;
  a.D = c.llm_width;
  a.out_ids = out_ids;
  a.out_pos = out_pos;
  a.keep_map = keep_map;
  a.out_embeds = out_embeds;
  a.out_len = (long long*)out_len;
  a.status = dev_status;
  a.blk_cnt = w.cnt;
  a.blk_off = w.off;
  a.routed_before = w.rb;
  a.src = w.src;
  *out = a;
  return IVC_OK;
}

static ivc_status compact_impl(ivc_connector* h, const int32_t* ids, const void* embeds,
                               int64_t L, int32_t img_context_id, const uint8_t* use64,
                               const void* out256, const void* out64, int32_t T, int32_t* out_ids,
                               int32_t* out_pos, int32_t* keep_map, void* out_embeds,
                               int64_t* out_len, int32_t* dev_status, void* ws, size_t ws_bytes,
                               void* stream) {
  CompactArgs a{};
  const ivc_status st = compact_prep(h, ids, embeds, L, img_context_id, use64, out256, out64, T,
                                     out_ids, out_pos, keep_map, out_embeds, out_len, dev_status,
                                     ws, ws_bytes, &a);
  if (st != IVC_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  LAUNCH("compact", s, launch_compact(a, s));
  return IVC_OK;
}

extern "C" ivc_status ivc_connector_compact(ivc_connector* h, const int32_t* ids,
                                            const void* embeds, int64_t L, int32_t img_context_id,
                                            const uint8_t* use64, const void* out256,
                                            const void* out64, int32_t T, int32_t* out_ids,
                                            int32_t* out_pos, int32_t* keep_map, void* out_embeds,
                                            int64_t* out_len, int32_t* dev_status, void* ws,
                                            size_t ws_bytes, void* stream) {
  TRACE("compact L=%lld T=%d img_context=%d ws=%zu", (long long)L, T, img_context_id, ws_bytes);
  return compact_impl(h, ids, embeds, L, img_context_id, use64, out256, out64, T, out_ids, out_pos,
                      keep_map, out_embeds, out_len, dev_status, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// forward + compact in one call: the compaction's index half needs only the
// decision, so it runs beside the projector chains on a stream of its own,
// with the text rows' copy; the chains' last products write their rows into
// the compacted sequence themselves (what they cannot place is copied after
// the join)
// ---------------------------------------------------------------------------
static size_t forward_ws_bytes(const ivc_connector* h, int T) {
  return (tokst_offset(h, T) + tokst_bytes(h, T) + 255) & ~(size_t)255;
}

// the compaction's scratch, then the compacted row of every image slot
static size_t compact_slots_offset(int T, long long L) {
  return (plan_compact(T, L, nullptr, nullptr) + 255) & ~(size_t)255;
}
static size_t compact_slots_bytes(const ivc_connector* h, int T) {
  const ivc_config& c = h->cfg;
  return (size_t)T * (size_t)(c.grid / 2) * (size_t)(c.grid / 2) * 4;
}

extern "C" size_t ivc_connector_forward_compact_workspace_bytes(const ivc_connector* h,
                                                                int32_t max_tiles,
                                                                int64_t max_seq_len) {
  if (!h || max_tiles < 0 || max_seq_len < 0) return 0;
  return forward_ws_bytes(h, max_tiles) + compact_slots_offset(max_tiles, max_seq_len) +
         compact_slots_bytes(h, max_tiles);
}

extern "C" ivc_status ivc_connector_forward_compact(
    ivc_connector* h, const void* vit, const int32_t* valid_tokens, int32_t T, float* gate,
    double* threshold, uint8_t* use64, float* pooled, int32_t* dev_status, void* out256,
    void* out64, const int32_t* ids, const void* embeds, int64_t L, int32_t img_context_id,
    int32_t* out_ids, int32_t* out_pos, int32_t* keep_map, void* out_embeds, int64_t* out_len,
    void* ws, size_t ws_bytes, void* stream) {
  TRACE("forward_compact T=%d L=%lld img_context=%d ws=%zu", T, (long long)L, img_context_id,
        ws_bytes);
  if (!h) return fail(IVC_ERR_INVALID_ARG, "null handle");
  if (T < 0) return fail(IVC_ERR_INVALID_ARG, "T = %d", T);
  if (!h->cfg.flash) return fail(IVC_ERR_INVALID_ARG, "forward_compact needs a flash connector");
  const size_t fw = forward_ws_bytes(h, T);
  if (L < 0) return fail(IVC_ERR_INVALID_ARG, "negative L");
  const size_t need = fw + compact_slots_offset(T, L) + compact_slots_bytes(h, T);
  if (!ws || ws_bytes < need)
    return fail(IVC_ERR_WORKSPACE, "forward_compact needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  // the compaction's scratch sits after the forward's: the two run at once
  CompactArgs a{};
  ivc_status st = compact_prep(h, ids, embeds, L, img_context_id, use64, out256, out64, T, out_ids,
                               out_pos, keep_map, out_embeds, out_len, dev_status,
                               (char*)ws + fw, ws_bytes - fw, &a);
  if (st != IVC_OK) return st;
  DirectRows dr;
  if (T > 0) {
    a.slot_dst = (int32_t*)((char*)ws + fw + compact_slots_offset(T, L));
    dr.slot_dst = a.slot_dst;
    dr.out = out_embeds;
  }
  const SideWork side = [&](hipStream_t s1) -> ivc_status {
    LAUNCH("compact_index", s1, launch_compact_index(a, s1));
    LAUNCH("compact_copy_text", s1, launch_compact_copy_text(a, s1));
    return IVC_OK;
  };
  st = forward_impl(h, vit, valid_tokens, T, gate, threshold, use64, pooled, dev_status, out256,
                    out64, ws, fw, stream, &side, T > 0 ? &dr : nullptr);
  if (st != IVC_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {  // no run, no side chain: only text rows
    LAUNCH("compact_index", s, launch_compact_index(a, s));
    LAUNCH("compact_copy_text", s, launch_compact_copy_text(a, s));
    return IVC_OK;
  }
  // rows of the chains whose last product could not place them
  const int kinds = (dr.all256 ? 0 : 2) | (dr.all64 ? 0 : 4);
  if (kinds != 0) LAUNCH("compact_copy", s, launch_compact_copy_kinds(a, kinds, s));
  return IVC_OK;
}

// ---------------------------------------------------------------------------
// compaction without allocation or workspace: the same kernels, their scratch
// (per-block IMG_CONTEXT counts and offsets, routed tiles before each tile, a
// source code per output row) in a fixed device array of this library
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[IVC_COMPACT_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};       // device address of `scratch`, per device
hipError_t g_scratch_err[kMaxDevices] = {};  // why it could not be taken
}  // namespace

// Once per device, with that device current: the device address of its copy
// of `scratch`.  (In host code the array's name stands for a host-side
// handle, not a device address; kernels must be given this pointer.)
static void noalloc_scratch_init(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] != nullptr) return;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    g_scratch_err[dev] = e != hipSuccess ? e : hipErrorInvalidSymbol;
    return;
  }
  g_scratch_ptr[dev] = p;
}

extern "C" ivc_status ivc_connector_compact_noalloc(
    ivc_connector* h, const int32_t* ids, const void* embeds, int64_t L, int32_t img_context_id,
    const uint8_t* use64, const void* out256, const void* out64, int32_t T, int32_t* out_ids,
    int32_t* out_pos, int32_t* keep_map, void* out_embeds, int64_t* out_len, int32_t* dev_status,
    void* stream) {
  TRACE("compact_noalloc L=%lld T=%d img_context=%d", (long long)L, T, img_context_id);
  if (!h) return fail(IVC_ERR_INVALID_ARG, "null handle");
  if (L > IVC_COMPACT_NOALLOC_MAX_LEN || T > IVC_COMPACT_NOALLOC_MAX_TILES)
    return fail(IVC_ERR_UNSUPPORTED,
                "compact_noalloc: L = %lld, T = %d beyond its fixed scratch (L <= %d, T <= %d)",
                (long long)L, T, IVC_COMPACT_NOALLOC_MAX_LEN, IVC_COMPACT_NOALLOC_MAX_TILES);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (h->dev >= 0 && h->dev < kMaxDevices) ws = g_scratch_ptr[h->dev];
  }
  if (ws == nullptr)
    return fail(IVC_ERR_HIP, "compact_noalloc: no scratch address for device %d (%s)", h->dev,
                hipGetErrorString(h->dev >= 0 && h->dev < kMaxDevices ? g_scratch_err[h->dev]
                                                                      : hipErrorInvalidDevice));
  if (plan_compact(IVC_COMPACT_NOALLOC_MAX_TILES, IVC_COMPACT_NOALLOC_MAX_LEN, nullptr, nullptr) >
      sizeof(scratch))
    return fail(IVC_ERR_WORKSPACE, "compact_noalloc: scratch smaller than its stated maximum");
  return compact_impl(h, ids, embeds, L, img_context_id, use64, out256, out64, T, out_ids, out_pos,
                      keep_map, out_embeds, out_len, dev_status, ws, sizeof(scratch), stream);
}

extern "C" size_t ivc_connector_compact_batch_workspace_bytes(const ivc_connector* h,
                                                             int32_t max_tiles,
                                                             int64_t max_total_len,
                                                             int32_t max_seqs) {
  if (!h || max_tiles < 0 || max_total_len < 0 || max_seqs < 0) return 0;
  return plan_compact_batch(max_tiles, max_total_len, max_seqs, nullptr, nullptr);
}

extern "C" ivc_status ivc_connector_compact_batch(
    ivc_connector* h, const int32_t* ids, const int32_t* cu_seqlens, int32_t B, const void* embeds,
    int64_t L, int32_t img_context_id, const int32_t* tile_offsets, const uint8_t* use64,
    const void* out256, const void* out64, int32_t T, int32_t* out_ids, int32_t* out_pos,
    int32_t* keep_map, void* out_embeds, int32_t* out_cu_seqlens, int32_t* dev_status, void* ws,
    size_t ws_bytes, void* stream) {
  TRACE("compact_batch B=%d L=%lld T=%d ws=%zu", B, (long long)L, T, ws_bytes);
  if (!h) return fail(IVC_ERR_INVALID_ARG, "null handle");
  const ivc_config& c = h->cfg;
  if (L < 0 || T < 0 || B < 0) return fail(IVC_ERR_INVALID_ARG, "negative L, T or B");
  if (L > 0x7fffffffll) return fail(IVC_ERR_UNSUPPORTED, "L above INT32_MAX");
  if (B == 0 && L > 0) return fail(IVC_ERR_INVALID_ARG, "B = 0 with L = %lld", (long long)L);
  if (!cu_seqlens || !tile_offsets || !out_cu_seqlens || !dev_status)
    return fail(IVC_ERR_INVALID_ARG, "null cu_seqlens/tile_offsets/out_cu_seqlens/dev_status");
  const long long S = (long long)(c.grid / 2) * (c.grid / 2);
  const long long S64 = (long long)(c.grid / 4) * (c.grid / 4);
  if ((long long)T * S >= (1ll << 31)) return fail(IVC_ERR_UNSUPPORTED, "T * S too large");
  if (L > 0 && (!ids || !embeds || !out_ids || !out_pos || !keep_map || !out_embeds))
    return fail(IVC_ERR_INVALID_ARG, "null sequence pointer");
  if (T > 0 && (!use64 || !out256)) return fail(IVC_ERR_INVALID_ARG, "null use64/out256");
  if (T > 0 && !out64 && c.flash) return fail(IVC_ERR_INVALID_ARG, "null out64");
  if (!aligned16(embeds) || !aligned16(out256) || !aligned16(out64) || !aligned16(out_embeds) ||
      !aligned16(ws))
    return fail(IVC_ERR_MISALIGNED, "embedding pointers must be 16-byte aligned");
  const size_t need = plan_compact_batch(T, L, B, nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return fail(IVC_ERR_WORKSPACE, "compact_batch needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  if (B == 0) return IVC_OK;  // nothing to write: out_cu_seqlens[0] is the caller's 0
  CompactBatchWs w;
  plan_compact_batch(T, L, B, ws, &w);
  CompactBatchArgs ba{};
  CompactArgs& a = ba.base;
  a.dtype = c.dtype;
  a.ids = ids;
  a.embeds = embeds;
  a.L = L;
  a.img_id = img_context_id;
  a.use64 = use64;
  a.out256 = out256;
  a.out64 = out64 ? out64 : out256;
  a.T = T;
  a.S = (int)S;
  a.S64 = c.flash ? (int)S64 : (int)S;
  a.D = c.llm_width;
  a.out_ids = out_ids;
  a.out_pos = out_pos;
  a.keep_map = keep_map;
  a.out_embeds = out_embeds;
  a.status = dev_status;
  a.blk_cnt = w.c.cnt;
  a.blk_off = w.c.off;
  a.routed_before = w.c.rb;
  a.src = w.c.src;
  ba.cu = cu_seqlens;
  ba.tile_off = tile_offsets;
  ba.B = B;
  ba.out_cu = out_cu_seqlens;
  ba.seq_img = w.seq_img;
  ba.seq_ok = w.seq_ok;
  ba.total = w.total;
  ba.layout_ok = w.layout_ok;
  hipStream_t s = (hipStream_t)stream;
  LAUNCH("compact_batch", s, launch_compact_batch(ba, s));
  return IVC_OK;
}

extern "C" ivc_status ivc_route_decide(const float* gate, int32_t T, double rel_quantile,
                                       double abs_threshold, double* threshold, uint8_t* use64,
                                       void* stream) {
  TRACE("route_decide T=%d rel_quantile=%g abs_threshold=%g", T, rel_quantile, abs_threshold);
  if (T < 0) return fail(IVC_ERR_INVALID_ARG, "T = %d", T);
  if (!(rel_quantile >= 0.0 && rel_quantile <= 1.0))
    return fail(IVC_ERR_INVALID_ARG, "rel_quantile outside [0, 1]");
  if (T == 0) return IVC_OK;
  if (!gate || !threshold || !use64) return fail(IVC_ERR_INVALID_ARG, "null pointer");
  hipStream_t s = (hipStream_t)stream;
  LAUNCH("quantile_decide", s,
         launch_quantile_decide(gate, T, rel_quantile, abs_threshold, threshold, use64, s));
  return IVC_OK;
}

extern "C" ivc_status ivc_tile_offsets(const int32_t* tiles_per_image, int32_t B, int32_t* offsets,
                                       int32_t* dev_status, void* stream) {
  TRACE("tile_offsets B=%d", B);
  if (B < 0) return fail(IVC_ERR_INVALID_ARG, "B = %d", B);
  if (!offsets || (B > 0 && !tiles_per_image)) return fail(IVC_ERR_INVALID_ARG, "null pointer");
  hipStream_t s = (hipStream_t)stream;
  LAUNCH("tile_offsets", s, launch_tile_offsets(tiles_per_image, B, offsets, dev_status, s));
  return IVC_OK;
}

extern "C" ivc_status ivc_pixel_shuffle(int32_t dtype, const void* vit, int32_t T, int32_t P,
                                        int32_t C, int32_t has_cls, int32_t r,
                                        int32_t ps_version, int32_t shuffle64_order, void* out,
                                        void* stream) {
  TRACE("pixel_shuffle dtype=%d T=%d P=%d C=%d has_cls=%d r=%d ps_version=%d shuffle64_order=%d",
        dtype, T, P, C, has_cls, r, ps_version, shuffle64_order);
  if (dtype != IVC_F32 && dtype != IVC_BF16) return fail(IVC_ERR_INVALID_ARG, "dtype");
  if (ps_version < 0 || ps_version > 2) return fail(IVC_ERR_INVALID_ARG, "ps_version %d", ps_version);
  if (shuffle64_order != IVC_SHUFFLE64_DIRECT && shuffle64_order != IVC_SHUFFLE64_TWICE_R2)
    return fail(IVC_ERR_INVALID_ARG, "shuffle64_order %d", shuffle64_order);
  if (T < 0 || P <= 0 || C <= 0 || (has_cls != 0 && has_cls != 1) || (r != 2 && r != 4))
    return fail(IVC_ERR_INVALID_ARG, "bad shape");
  if (P % r) return fail(IVC_ERR_INVALID_ARG, "P %% r != 0");
  if (T == 0) return IVC_OK;
  const int esz = dtype == IVC_BF16 ? 2 : 4;
  if ((long long)C * esz % 16) return fail(IVC_ERR_MISALIGNED, "row width");
  if (C > shuffle_max_width(dtype)) return fail(IVC_ERR_UNSUPPORTED, "C too large");
  if (!vit || !out) return fail(IVC_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(vit) || !aligned16(out)) return fail(IVC_ERR_MISALIGNED, "alignment");
  ShuffleArgs sa{};
  sa.dtype = dtype;
  sa.X = vit;
  sa.T = T;
  sa.P = P;
  sa.C = C;
  sa.has_cls = has_cls;
  sa.flash = r == 4;
  sa.ln = 0;
  sa.out2 = r == 2 ? out : nullptr;
  sa.out4 = r == 4 ? out : nullptr;
  sa.ps_v1 = ps_version == 1;
  sa.twice_r2 = shuffle64_order == IVC_SHUFFLE64_TWICE_R2;
  hipStream_t s = (hipStream_t)stream;
  LAUNCH("pixel_shuffle", s, launch_shuffle_ln(sa, s));
  return IVC_OK;
}

extern "C" const char* ivc_status_string(ivc_status st) {
  // a C caller may pass any int: read it as one before naming it (loading an
  // out-of-range enum value is undefined behaviour in C++)
  int v;
  memcpy(&v, &st, sizeof v);
  switch (v) {
    case IVC_OK: return "ok";
    case IVC_ERR_INVALID_ARG: return "invalid argument";
    case IVC_ERR_UNSUPPORTED: return "unsupported shape";
    case IVC_ERR_MISALIGNED: return "misaligned pointer or row";
    case IVC_ERR_WORKSPACE: return "workspace too small";
    case IVC_ERR_OOM: return "out of device memory";
    case IVC_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

extern "C" const char* ivc_last_error(void) { return g_last_error.c_str(); }
