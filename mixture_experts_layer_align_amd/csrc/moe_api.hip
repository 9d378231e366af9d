// C ABI of libmoe: argument validation, workspace layout, launch order.
// The ABI itself is documented in include/libmoe.h.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/libmoe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int64_t WS_ALIGN = 256;
// Router GEMM: split d until ~ROUTER_TARGET_WGS two-wave workgroups run, at
// most ROUTER_MAX_SPLIT planes and ROUTER_MIN_STEPS k-steps per split (the
// loads run 3 steps ahead).
constexpr int ROUTER_TARGET_WGS = 1024;
constexpr int ROUTER_MIN_STEPS = 4;
// Token blocks up to which the router's tiles are one slab wide.
constexpr int ROUTER_NARROW_MAX_BLOCKS = 8;
// Expert GEMMs split K only when the blocks x n-tiles work items leave the chip
// under-filled (fewer than SPLIT_BELOW two-wave workgroups); the split then
// balances the compute units (choose_kchunk_balanced) and keeps at least
// MIN_SPLIT_STEPS k-steps each so the 4-stage load ring still streams.
constexpr int SPLIT_BELOW = 192;
// Average routed rows per expert from which the LDS-tiled GEMM (256-row
// blocks, MFMA-bound) replaces the weight-streaming GEMM (32-row blocks).
// 256-row blocks are used even where they pad more than 128-row ones would:
// a 128-row block's 64 x 128 wave tiles need more LDS bytes per MFMA than the
// LDS delivers.
constexpr int TILED_MIN_ROWS = 64;
constexpr int TILED_BM = 256;
constexpr int MIN_SPLIT_STEPS = 8;
constexpr int64_t MAX_ENTRIES = int64_t(1) << 24;

int64_t up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Bump allocator over the caller's workspace (or a size count when base==NULL).
struct Carve {
  char* base;
  int64_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(int64_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = up(off + count * (int64_t)sizeof(T), WS_ALIGN);
    return p;
  }
};

int act_code(int dt) { return dt == MOE_BF16 ? ACT_BF16 : ACT_F32; }
int w_code(int dt) {
  return dt == MOE_FP8_E4M3 ? W_FP8
         : dt == MOE_MXFP4  ? W_FP4
         : dt == MOE_MXFP8  ? W_MXFP8
         : dt == MOE_BF16   ? W_BF16
                            : W_F32;
}
int act_bytes(int dt) { return dt == MOE_BF16 ? 2 : 4; }

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int check_ws(void* ws, size_t* ws_bytes, int64_t need, bool* query) {
  if (ws_bytes == nullptr) return MOE_ERR_INVALID;
  if (ws == nullptr) {
    *ws_bytes = (size_t)need;
    *query = true;
    return MOE_OK;
  }
  *query = false;
  if ((int64_t)*ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % WS_ALIGN != 0) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// Number of k-splits: 1 when `items` workgroups reach `below`, else enough to
// approach `target`, with at least `min_steps` k-steps per split and at most
// max_split splits.  Returns the k-chunk (a multiple of kstep).
int choose_kchunk(int64_t items, int K, int kstep, int* nsplit, int below, int target,
                  int min_steps, int max_split) {
  const int steps = K / kstep;
  items = std::max<int64_t>(items, 1);
  int s = 1;
  if (items < below)
    s = (int)std::min<int64_t>({(target + items - 1) / items, (int64_t)steps / min_steps,
                                (int64_t)max_split});
  s = std::max(s, 1);
  const int chunk_steps = (steps + s - 1) / s;
  *nsplit = (steps + chunk_steps - 1) / chunk_steps;
  return chunk_steps * kstep;
}

// Workgroups of a persistent stream GEMM launch over `items` expected items:
// as many as leave every workgroup the same whole number of items, at most
// one per compute unit; 0 (one workgroup per item) when there are fewer items
// than compute units.
int persistent_wgs(int64_t items, int cus) {
  if (items <= cus) return 0;
  const int64_t per = (items + cus - 1) / cus;
  return (int)((items + per - 1) / per);
}

// Number of k-splits for a weight-streaming GEMM of `items` workgroups when
// fewer than `below` would run: every split adds a workgroup per item, and
// the layer takes as long as its busiest compute unit, whose share of the
// work is ceil(items*s / cus) / s (workgroups of equal size, spread evenly).
// The smallest s with the least share wins; at least min_steps k-steps each.
int choose_kchunk_balanced(int64_t items, int K, int kstep, int* nsplit, int below, int min_steps,
                           int max_split, int cus) {
  const int steps = K / kstep;
  items = std::max<int64_t>(items, 1);
  int best = 1;
  if (items < below) {
    const int smax = std::max(1, std::min(max_split, steps / min_steps));
    double best_cost = 1e30;
    for (int s = 1; s <= smax; ++s) {
      const double cost = (double)((items * s + cus - 1) / cus) / s;
      if (cost < best_cost * (1.0 - 1e-9)) {
        best_cost = cost;
        best = s;
      }
    }
  }
  const int chunk_steps = (steps + best - 1) / best;
  *nsplit = (steps + chunk_steps - 1) / chunk_steps;
  return chunk_steps * kstep;
}

// k-splits of the tiled down GEMM over `tiles` expected tiles: the busiest
// compute unit's share, ceil(tiles*s / cus) / s full-depth tiles, against the
// cost of each further fp32 output plane (written here and read again by the
// combine, 8 bytes per routed row and output column at ~5.5 TB/s, against
// 2*K flops per row and column at ~1.3 PFLOP/s: 945/K of the GEMM's ideal
// time per plane).  Each split is a multiple of 64 and at least
// TILED_MIN_KCHUNK deep; at most 4.
int choose_tiled_split(int64_t tiles, int K, int cus) {
  tiles = std::max<int64_t>(tiles, 1);
  const double ideal = (double)tiles / cus;
  int best = 1;
  double best_t = 1e30;
  for (int s = 1; s <= 4; ++s) {
    if (K % (64 * s) != 0 || K / s < TILED_MIN_KCHUNK) continue;
    const double t = (double)((tiles * s + cus - 1) / cus) / s + (s - 1) * ideal * 945.0 / K;
    if (t < best_t * (1.0 - 1e-9)) {
      best_t = t;
      best = s;
    }
  }
  return best;
}

// ------------------------------------------------------------ router plan
struct RouterPlan {
  StreamGemmArgs g;
  int nsplit;
  int64_t partial_floats;
};

RouterPlan plan_router(const void* x, const void* w_router, int T, int d, int E, int act) {
  RouterPlan r{};
  StreamGemmArgs& g = r.g;
  g.a = x;
  g.a_ld = d;
  g.a_mode = A_DENSE;
  g.m_total = T;
  g.block_expert = nullptr;
  g.num_mblocks = (T + STREAM_BM - 1) / STREAM_BM;
  g.w = w_router;
  g.w_ld = E;
  g.w_estride = 0;
  g.K = d;
  g.n_out = E;
  // few token blocks: one-slab tiles, so twice the workgroups stream the
  // router weight (its two waves split each tile's k-range)
  const int tc = g.num_mblocks <= ROUTER_NARROW_MAX_BLOCKS ? router_slab_cols(act)
                                                          : router_tile_cols(act);
  g.n_tiles = (E + tc - 1) / tc;
  g.kchunk = choose_kchunk((int64_t)g.num_mblocks * g.n_tiles, d, router_kstep(act), &g.ksplit,
                           ROUTER_TARGET_WGS, ROUTER_TARGET_WGS, ROUTER_MIN_STEPS,
                           ROUTER_MAX_SPLIT);
  g.out_ld = E;
  g.out_split_stride = (int64_t)T * E;
  r.nsplit = g.ksplit;
  r.partial_floats = (int64_t)g.ksplit * T * E;
  return r;
}

hipError_t run_router(RouterPlan& r, int act, float* partial, const float* bias, int T, int E,
                      int k, float* logits, int32_t* ids, float* w, hipStream_t st, moe_trace* tr,
                      int* kidx);

// ------------------------------------------------------------ tracing
void trace_mark(moe_trace* tr, int* kidx, const char* name, hipStream_t st) {
  if (tr == nullptr) return;
  if (*kidx < tr->n_events && tr->events != nullptr)
    (void)hipEventRecord(reinterpret_cast<hipEvent_t>(tr->events[*kidx]), st);
  if (name != nullptr && *kidx < 16) tr->names[*kidx] = name;
  ++*kidx;
}

hipError_t run_router(RouterPlan& r, int act, float* partial, const float* bias, int T, int E,
                      int k, float* logits, int32_t* ids, float* w, hipStream_t st, moe_trace* tr,
                      int* kidx) {
  r.g.out = partial;
  trace_mark(tr, kidx, "router_gemm", st);
  hipError_t e = launch_router_gemm(act, r.g, st);
  if (e != hipSuccess) return e;
  trace_mark(tr, kidx, "topk", st);
  return launch_topk(partial, r.nsplit, (int64_t)T * E, bias, T, E, k, logits, ids, w, st);
}

// Shapes and dtypes; data pointers are checked only when work is enqueued
// (a workspace query needs none).
// p is not NULL and not a multiple of a bytes: the 16-byte vector loads and
// stores (and direct-to-LDS loads) of the kernels need their arrays aligned.
bool misaligned(const void* p, uintptr_t a) {
  return p != nullptr && reinterpret_cast<uintptr_t>(p) % a != 0;
}

int validate_route(int T, int d, int E, int k, int act) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID;
  if (k > E || E > MOE_MAX_EXPERTS) return MOE_ERR_INVALID;
  if ((int64_t)T * k >= MAX_ENTRIES) return MOE_ERR_INVALID;
  if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

// The no-allocation forward's workspace: one static device array, which every
// GPU the library runs on holds (its own copy) until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: only the
// address the runtime reports for the current device is ever used.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

// The current device's copy of `scratch`, resolved on its first use there.
int noalloc_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_DEVICE;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

namespace moe {
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  if (dev >= 0 && dev < 64) cached[dev] = cus;
  return cus;
}
}  // namespace moe

extern "C" {

int moe_abi_version(void) { return 2; }

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_DEVICE: return "HIP runtime error";
    case MOE_ERR_SCRATCH: return "call needs more than the no-allocation scratch holds";
    default: return "unknown status";
  }
}

int64_t moe_align_capacity(int T, int E, int k, int bm) {
  if (T < 0 || E <= 0 || k <= 0 || !pow2(bm)) return -1;
  const int64_t n = (int64_t)T * k;
  if (n == 0) return 0;
  return (int64_t)bm * ((n + std::min<int64_t>(E, n) * (bm - 1)) / bm);
}

int moe_qk_norm(void* q, void* k, const void* q_weight, const void* k_weight, int T,
                int n_q_heads, int n_k_heads, int head_dim, int dtype, float weight_bias,
                float eps, void* stream) {
  if (T < 0 || n_q_heads < 0 || n_k_heads < 0) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return MOE_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(weight_bias)) return MOE_ERR_INVALID;
  if ((int64_t)T * (n_q_heads + n_k_heads) >= (int64_t(1) << 31)) return MOE_ERR_INVALID;
  if (T == 0 || n_q_heads + n_k_heads == 0) return MOE_OK;
  if (n_q_heads > 0 && (q == nullptr || q_weight == nullptr)) return MOE_ERR_INVALID;
  if (n_k_heads > 0 && (k == nullptr || k_weight == nullptr)) return MOE_ERR_INVALID;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(q_weight, 16) ||
      misaligned(k_weight, 16))
    return MOE_ERR_INVALID;
  const hipError_t e =
      launch_qk_norm(dtype == MOE_BF16 ? ACT_BF16 : ACT_F32, q, k, q_weight, k_weight, T,
                     n_q_heads, n_k_heads, head_dim, weight_bias, eps,
                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

int moe_rms_norm(const void* x, const void* weight, void* out, int T, int d, int dtype,
                 float weight_bias, float eps, void* stream) {
  if (T < 0 || d <= 0) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)d * (dtype == MOE_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0 || row_bytes > RMS_MAX_ROW_BYTES) return MOE_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(weight_bias)) return MOE_ERR_INVALID;
  if (T == 0) return MOE_OK;
  if (x == nullptr || weight == nullptr || out == nullptr) return MOE_ERR_INVALID;
  if (misaligned(x, 16) || misaligned(weight, 16) || misaligned(out, 16)) return MOE_ERR_INVALID;
  // out is x itself or does not overlap it
  const char* xb = static_cast<const char*>(x);
  const char* ob = static_cast<const char*>(out);
  const int64_t bytes = row_bytes * T;
  if (ob != xb && ob < xb + bytes && xb < ob + bytes) return MOE_ERR_INVALID;
  const hipError_t e = launch_rms_norm(dtype == MOE_BF16 ? ACT_BF16 : ACT_F32, x, weight, out, T,
                                       d, weight_bias, eps, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

int moe_quantize_mxfp8(const void* x, int rows, int n, int dtype, void* codes, void* scales,
                       void* stream) {
  if (rows < 0 || n <= 0) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (n % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return MOE_ERR_INVALID;
  if (misaligned(x, 16) || misaligned(codes, 8) || misaligned(scales, 4)) return MOE_ERR_INVALID;
  // the three regions must not overlap
  const int64_t elems = (int64_t)rows * n;
  const char* r[3] = {static_cast<const char*>(x), static_cast<const char*>(codes),
                      static_cast<const char*>(scales)};
  const int64_t len[3] = {elems * (dtype == MOE_BF16 ? 2 : 4), elems, elems / 32};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (r[i] < r[j] + len[j] && r[j] < r[i] + len[i]) return MOE_ERR_INVALID;
  const hipError_t e = launch_mx_quant(dtype == MOE_BF16 ? ACT_BF16 : ACT_F32, x, codes, scales,
                                       rows, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

int moe_route(const void* x, const void* w_router, const float* logit_bias, int T, int d, int E,
              int k, int act_dtype, float* logits, int32_t* topk_ids, float* topk_w,
              void* workspace, size_t* workspace_bytes, void* stream) {
  int rc = validate_route(T, d, E, k, act_dtype);
  if (rc != MOE_OK) return rc;
  const int act = act_code(act_dtype);
  RouterPlan r = plan_router(x, w_router, T, d, E, act);
  Carve c(workspace);
  float* partial = c.take<float>(std::max<int64_t>(r.partial_floats, 1));
  bool query;
  rc = check_ws(workspace, workspace_bytes, c.off, &query);
  if (rc != MOE_OK || query || T == 0) return rc;
  if (x == nullptr || w_router == nullptr || topk_ids == nullptr || topk_w == nullptr)
    return MOE_ERR_INVALID;
  if (misaligned(x, 16) || misaligned(w_router, 16) || misaligned(logit_bias, 4) ||
      misaligned(logits, 4) || misaligned(topk_ids, 4) || misaligned(topk_w, 4))
    return MOE_ERR_INVALID;
  int kidx = 0;
  hipError_t e = run_router(r, act, partial, logit_bias, T, E, k, logits, topk_ids, topk_w,
                            static_cast<hipStream_t>(stream), nullptr, &kidx);
  return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

int moe_align(const int32_t* topk_ids, int T, int E, int k, int block_m, int32_t* expert_counts,
              int32_t* padded_offsets, int32_t* sorted_ids, int32_t* inv_pos,
              int32_t* block_expert, void* workspace, size_t* workspace_bytes, void* stream) {
  if (T < 0 || E <= 0 || k <= 0 || k > E || E > MOE_MAX_EXPERTS) return MOE_ERR_INVALID;
  if (!pow2(block_m) || block_m < MOE_BLOCK_M_MIN || block_m > MOE_BLOCK_M_MAX)
    return MOE_ERR_INVALID;
  const int64_t n = (int64_t)T * k;
  if (n >= MAX_ENTRIES) return MOE_ERR_INVALID;
  const int64_t need = align_workspace_bytes((int)n, E);
  bool query;
  int rc = check_ws(workspace, workspace_bytes, need, &query);
  if (rc != MOE_OK || query) return rc;
  if (T == 0) return MOE_OK;
  if (topk_ids == nullptr || expert_counts == nullptr || padded_offsets == nullptr ||
      sorted_ids == nullptr || inv_pos == nullptr || block_expert == nullptr)
    return MOE_ERR_INVALID;
  if (misaligned(topk_ids, 4) || misaligned(expert_counts, 4) || misaligned(padded_offsets, 4) ||
      misaligned(sorted_ids, 4) || misaligned(inv_pos, 4) || misaligned(block_expert, 4))
    return MOE_ERR_INVALID;
  AlignArgs a{};
  a.ids = topk_ids;
  a.n = (int)n;
  a.T = T;
  a.E = E;
  a.k = k;
  a.bm = block_m;
  a.cap = moe_align_capacity(T, E, k, block_m);
  a.counts = expert_counts;
  a.offsets = padded_offsets;
  a.sorted_ids = sorted_ids;
  a.inv_pos = inv_pos;
  a.block_expert = block_expert;
  hipError_t e = launch_align(a, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

int moe_forward_traced(const moe_layer* L, const void* x, int T, void* out, void* workspace,
                       size_t* workspace_bytes, moe_routing_out* routing, moe_trace* tr,
                       void* stream) {
  if (L == nullptr) return MOE_ERR_INVALID;
  const int d = L->d, dff = L->d_ff, E = L->E, k = L->k;
  int rc = validate_route(T, d, E, k, L->act_dtype);
  if (rc != MOE_OK) return rc;
  if (dff <= 0) return MOE_ERR_INVALID;
  if (d % 128 != 0 || dff % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const bool pair_ok = (L->act_dtype == MOE_F32 && L->w_dtype == MOE_F32) ||
                       (L->act_dtype == MOE_BF16 && L->w_dtype == MOE_BF16) ||
                       (L->act_dtype == MOE_BF16 && L->w_dtype == MOE_FP8_E4M3) ||
                       (L->act_dtype == MOE_BF16 && L->w_dtype == MOE_MXFP4) ||
                       (L->act_dtype == MOE_BF16 && L->w_dtype == MOE_MXFP8);
  if (!pair_ok) return MOE_ERR_UNSUPPORTED;
  // fp8 and MXFP4 expert slabs are 256 columns wide
  const bool scaled =
      L->w_dtype == MOE_FP8_E4M3 || L->w_dtype == MOE_MXFP4 || L->w_dtype == MOE_MXFP8;
  if (scaled && (d % 256 != 0 || dff % 256 != 0)) return MOE_ERR_UNSUPPORTED;
  if (scaled && (L->scale_gate_up == nullptr || L->scale_down == nullptr))
    return MOE_ERR_INVALID;
  const bool mx = L->w_dtype == MOE_MXFP4 || L->w_dtype == MOE_MXFP8;

  const int act = act_code(L->act_dtype);
  const int wdt = w_code(L->w_dtype);
  const int ab = act_bytes(L->act_dtype);
  const int64_t n = (int64_t)T * k;
  // regime: thick blocks go to the MFMA-tiled GEMM when its shapes fit
  // (MXFP4 weights always take the weight-streaming GEMM)
  const bool tiled = act == ACT_BF16 && (wdt == W_BF16 || wdt == W_FP8) &&
                     n >= (int64_t)TILED_MIN_ROWS * E &&
                     d % TILED_BN == 0 && dff % (TILED_BN / 2) == 0 &&
                     dff >= TILED_MIN_KCHUNK;
  // the tiled GEMM's half tiles pair two 256-column tiles, so experts are
  // padded to 128 rows when both GEMMs have an even number of column tiles
  const bool half_rows = tiled && (dff / (TILED_BN / 2)) % 2 == 0 && (d / TILED_BN) % 2 == 0;
  // fp8 weights on the weight-streaming GEMM, once the batch averages
  // STREAM_HALVES_MIN entries per expert: the gate|up GEMM applies one weight
  // stream to a pair of an expert's 32-row blocks, so a skewed expert
  // streams its weights once per 64 rows (E=256 top-8 T=128, Zipf 1.2: 77
  // blocks in 63 pairs and singles; gate|up 447 -> 332 us).  The down GEMM
  // (short K: one-block items overlap better) keeps one block per item
  // (pairs: 202 -> 282 us)
  const bool halves2 = !tiled && act == ACT_BF16 && wdt == W_FP8 &&
                       n >= (int64_t)STREAM_HALVES_MIN * E;
  const int bm = tiled ? (half_rows ? TILED_BM / 2 : TILED_BM) : STREAM_BM;
  const int64_t cap = moe_align_capacity(T, E, k, bm);
  const int64_t nblocks = cap / bm;

  RouterPlan r = plan_router(x, L->w_router, T, d, E, act);

  // expert GEMM plans
  const int kstep = stream_kstep(wdt);
  const int gu_tc = tiled ? TILED_BN / 2 : stream_tile_cols(wdt, EPI_SILU_MUL);
  const int dn_tc = tiled ? TILED_BN : stream_tile_cols(wdt, EPI_STORE);
  const int gu_tiles = dff / gu_tc;
  const int dn_tiles = (d + dn_tc - 1) / dn_tc;
  // blocks expected to carry rows: one per active expert plus the overflow
  const int64_t est_blocks =
      std::min<int64_t>(nblocks, std::max<int64_t>(std::min<int64_t>(E, n), (n + bm - 1) / bm));
  int gu_split = 1, dn_split = 1, gu_chunk = d, dn_chunk = dff, gu_wgs = 0, dn_wgs = 0;
  if (!tiled) {
    const int cus = device_cus();
    const int64_t gu_items = std::max<int64_t>(est_blocks, 1) * gu_tiles;
    const int64_t dn_items = std::max<int64_t>(est_blocks, 1) * dn_tiles;
    // MX weights (a scale per 32 k to fetch and apply) stream faster with two
    // workgroups per compute unit when K is split for few experts: split as
    // if the chip had twice the units (E=256 top-8 T=1: MXFP8 0.124 -> 0.115
    // ms, MXFP4 0.086 -> 0.083); so do fp8 down GEMMs (their bf16-pair h
    // doubles the MFMAs per weight byte: E=256 top-8 T=1 down 44 -> 35 µs;
    // four per unit: 43 µs), while the fp8 gate|up keeps one (two: 50 -> 52)
    const int wmul = (wdt == W_MXFP8 || wdt == W_FP4) ? 2 : 1;
    const int wmul_dn = wdt == W_BF16 ? 1 : 2;
    gu_chunk = choose_kchunk_balanced(gu_items, d, kstep, &gu_split, wmul * SPLIT_BELOW,
                                      MIN_SPLIT_STEPS, 64, wmul * cus);
    dn_chunk = choose_kchunk_balanced(dn_items, dff, kstep, &dn_split, wmul_dn * SPLIT_BELOW,
                                      MIN_SPLIT_STEPS, 64, wmul_dn * cus);
    // bf16 weights stream fastest with one workgroup per compute unit; fp8
    // weights (twice the math per byte) need the latency hiding of several
    // workgroups per compute unit and keep one workgroup per item
    if (wdt == W_BF16) {
      gu_wgs = persistent_wgs(gu_items * gu_split, cus);
      dn_wgs = persistent_wgs(dn_items * dn_split, cus);
    }
  } else {
    // tile rows: one per 256 routed rows plus about half a row of padding per
    // active expert
    const int64_t rows_est =
        std::min<int64_t>(nblocks, (n + 255) / 256 + std::min<int64_t>(E, n) / 2);
    dn_split = choose_tiled_split(rows_est * dn_tiles, dff, device_cus());
    dn_chunk = dff / dn_split;
  }
  Carve c(workspace);
  float* r_partial = c.take<float>(std::max<int64_t>(r.partial_floats, 1));
  int32_t* ids = c.take<int32_t>(std::max<int64_t>(n, 1));
  float* tw = c.take<float>(std::max<int64_t>(n, 1));
  int32_t* counts = c.take<int32_t>(E);
  int32_t* offs = c.take<int32_t>(E + 1);
  int32_t* sorted = c.take<int32_t>(std::max<int64_t>(cap, 1));
  int32_t* inv = c.take<int32_t>(std::max<int64_t>(n, 1));
  int32_t* bexp = c.take<int32_t>(std::max<int64_t>(nblocks, 1));
  char* al_ws = c.take<char>(std::max<int64_t>(align_workspace_bytes((int)n, E), 1));
  // tiled GEMM row list: at most one row per bm-block
  int32_t* trows = tiled ? c.take<int32_t>(2 * std::max<int64_t>(nblocks, 1)) : nullptr;
  int32_t* tcounts = tiled ? c.take<int32_t>(2 + TILE_COUNTERS) : nullptr;
  // h; on the weight-streaming path with bf16 activations it is carried as a
  // pair of bf16 planes (high halves, then low halves: 16 significant bits),
  // whose second MFMA per weight fragment the decode GEMMs have issue slots
  // for.  A single bf16 rounding of h measured up to 2.19e-2 * RMS on rows
  // of the E=256 top-8 d=7168 layer (the bound is 2e-2), where the output's
  // own rounding alone stays at 1.4e-2.
  const bool h_pair = !tiled && act == ACT_BF16;
  char* h = c.take<char>(std::max<int64_t>(cap * dff * ab, 1));
  char* h_lo = h_pair ? c.take<char>(std::max<int64_t>(cap * dff * 2, 1)) : nullptr;
  // per-slot expert outputs, or their k-split partial sums: fp32 from the
  // weight-streaming GEMM, fp16 from the MFMA-tiled one (the tiled GEMM's
  // fp32 stores were bound by HBM write bandwidth; fp16's 11 bits keep the
  // output within its own rounding, like h's)
  const bool y_f16 = tiled;
  void* y = c.take<char>(std::max<int64_t>(dn_split * cap * d * (y_f16 ? 2 : 4), 1));
  float* gu_part = gu_split > 1 ? c.take<float>(gu_split * cap * 2 * dff) : nullptr;
  bool query;
  rc = check_ws(workspace, workspace_bytes, c.off, &query);
  if (rc != MOE_OK || query) return rc;
  if (routing != nullptr && routing->block_m != nullptr) *routing->block_m = bm;
  if (tr != nullptr) tr->n_kernels = 0;
  if (T == 0) return MOE_OK;
  if (x == nullptr || out == nullptr || L->w_router == nullptr || L->w_gate_up == nullptr ||
      L->w_down == nullptr || out == x)
    return MOE_ERR_INVALID;
  if (misaligned(x, 16) || misaligned(out, 16) || misaligned(L->w_router, 16) ||
      misaligned(L->w_gate_up, 16) || misaligned(L->w_down, 16) ||
      misaligned(L->scale_gate_up, 16) || misaligned(L->scale_down, 16) ||
      misaligned(L->logit_bias, 4))
    return MOE_ERR_INVALID;
  if (routing != nullptr &&
      (misaligned(routing->logits, 4) || misaligned(routing->topk_ids, 4) ||
       misaligned(routing->topk_w, 4) || misaligned(routing->expert_counts, 4) ||
       misaligned(routing->padded_offsets, 4) || misaligned(routing->sorted_ids, 4) ||
       misaligned(routing->inv_pos, 4)))
    return MOE_ERR_INVALID;

  // routing views the caller asked for are written in place
  if (routing != nullptr) {
    if (routing->topk_ids) ids = routing->topk_ids;
    if (routing->topk_w) tw = routing->topk_w;
    if (routing->expert_counts) counts = routing->expert_counts;
    if (routing->padded_offsets) offs = routing->padded_offsets;
    if (routing->sorted_ids) sorted = routing->sorted_ids;
    if (routing->inv_pos) inv = routing->inv_pos;
  }
  float* logits = routing ? routing->logits : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int kidx = 0;

  AlignArgs a{};
  a.ids = ids;
  a.n = (int)n;
  a.T = T;
  a.E = E;
  a.k = k;
  a.bm = bm;
  a.cap = cap;
  a.counts = counts;
  a.offsets = offs;
  a.sorted_ids = sorted;
  a.inv_pos = inv;
  a.block_expert = bexp;
  a.tile_rows = trows;
  a.tile_counts = tcounts;
  hipError_t e;
  if (route_align_small_ok(T, E, k, r.nsplit)) {
    // a few tokens: top-k and alignment in one launch
    r.g.out = r_partial;
    trace_mark(tr, &kidx, "router_gemm", st);
    e = launch_router_gemm(act, r.g, st);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    trace_mark(tr, &kidx, "route_align", st);
    e = launch_route_align_small(r_partial, r.nsplit, (int64_t)T * E, L->logit_bias, logits, ids,
                                 tw, a, st);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  } else {
    e = run_router(r, act, r_partial, L->logit_bias, T, E, k, logits, ids, tw, st, tr, &kidx);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    trace_mark(tr, &kidx, "align", st);
    e = launch_align(a, al_ws, st);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  }

  StreamGemmArgs g{};
  g.a = x;
  g.a_ld = d;
  g.a_mode = A_GATHER;
  g.sorted_ids = sorted;
  g.topk = k;
  g.block_expert = bexp;
  g.num_mblocks = (int)nblocks;
  g.padded_rows = offs + E;
  g.tile_rows = trows;
  g.tile_counts = tcounts;
  g.die_next = tiled ? tcounts + 2 : nullptr;
  g.w = L->w_gate_up;
  g.w_ld = 2 * (int64_t)dff;
  g.w_estride = (int64_t)d * 2 * dff;
  g.scale = static_cast<const float*>(L->scale_gate_up);
  // fp8: one fp32 per column; MXFP4: one byte per column and 32-row block
  g.scale_estride = mx ? (int64_t)(d / 32) * 2 * dff : 2 * (int64_t)dff;
  g.K = d;
  g.n_out = dff;
  g.up_off = dff;
  g.n_tiles = gu_tiles;
  g.ksplit = gu_split;
  g.kchunk = gu_chunk;
  g.wgs = gu_wgs;
  g.halves = halves2 ? 2 : 1;
  g.expert_offsets = offs;
  g.partial = gu_part;
  g.partial_ld = 2 * (int64_t)dff;
  g.partial_split_stride = cap * 2 * dff;
  g.out = h;
  g.out_lo = h_lo;
  g.out_ld = dff;
  trace_mark(tr, &kidx, "gate_up", st);
  e = tiled ? launch_tiled_gemm(EPI_SILU_MUL, wdt, bm, g, st)
            : launch_stream_gemm(act, wdt, EPI_SILU_MUL, g, st);
  if (e != hipSuccess) return MOE_ERR_DEVICE;

  StreamGemmArgs g2{};
  g2.a = h;
  g2.a_lo = h_lo;
  g2.a_ld = dff;
  // a split gate|up leaves fp32 partials: the down GEMM's items add them and
  // apply SiLU*up for their own rows and k-range before using them
  g2.a_part = gu_split > 1 ? gu_part : nullptr;
  g2.a_part_nsplit = gu_split;
  g2.a_part_ld = 2 * (int64_t)dff;
  g2.a_part_stride = cap * 2 * dff;
  g2.a_mode = A_PADDED;
  g2.sorted_ids = sorted;
  g2.topk = k;
  g2.block_expert = bexp;
  g2.num_mblocks = (int)nblocks;
  g2.padded_rows = offs + E;
  g2.tile_rows = trows;
  g2.tile_counts = tcounts;
  g2.die_next = tiled ? tcounts + 2 + TILE_COUNTERS / 2 : nullptr;
  g2.w = L->w_down;
  g2.w_ld = d;
  g2.w_estride = (int64_t)dff * d;
  g2.scale = static_cast<const float*>(L->scale_down);
  g2.scale_estride = mx ? (int64_t)(dff / 32) * d : d;
  g2.K = dff;
  g2.n_out = d;
  g2.n_tiles = dn_tiles;
  g2.ksplit = dn_split;
  g2.kchunk = dn_chunk;
  g2.wgs = dn_wgs;
  g2.halves = 1;
  g2.partial = static_cast<float*>(y);
  g2.partial_ld = d;
  g2.partial_split_stride = cap * d;
  g2.out_split_stride = cap * d;
  g2.out = y;
  g2.out_ld = d;
  trace_mark(tr, &kidx, "down", st);
  e = tiled ? launch_tiled_gemm(EPI_STORE, wdt, bm, g2, st)
            : launch_stream_gemm(act, wdt, EPI_STORE, g2, st);
  if (e != hipSuccess) return MOE_ERR_DEVICE;

  trace_mark(tr, &kidx, "combine", st);
  e = launch_combine(act, y, y_f16, dn_split, cap * d, inv, tw, T, k, d, out, st);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  trace_mark(tr, &kidx, nullptr, st);
  if (tr != nullptr) tr->n_kernels = kidx - 1;
  return MOE_OK;
}

int moe_forward(const moe_layer* L, const void* x, int T, void* out, void* workspace,
                size_t* workspace_bytes, moe_routing_out* routing, void* stream) {
  return moe_forward_traced(L, x, T, out, workspace, workspace_bytes, routing, nullptr, stream);
}

int moe_forward_noalloc(const moe_layer* L, const void* x, int T, void* out,
                        moe_routing_out* routing, void* stream) {
  // the same validation and workspace plan as moe_forward (a query enqueues
  // nothing)
  size_t need = 0;
  int rc = moe_forward(L, x, T, out, nullptr, &need, routing, stream);
  if (rc != MOE_OK) return rc;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  rc = noalloc_scratch(&ws);
  if (rc != MOE_OK) return rc;
  size_t have = MOE_NOALLOC_SCRATCH_BYTES;
  return moe_forward(L, x, T, out, ws, &have, routing, stream);
}

}  // extern "C"
