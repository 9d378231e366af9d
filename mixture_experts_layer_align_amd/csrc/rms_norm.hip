// RMS normalisation of rows: the row RMSNorm over the hidden size
// (moe_rms_norm) and the per-head QK-norm of attention heads (moe_qk_norm).
//
// For a row x of n values and a gain w of n values,
//   y_i = x_i * rsqrt(sum_j x_j^2 / n + eps) * (w_i + weight_bias)
// ("La fusion de noyaux", section 4.2, reduction + elementwise fusion: one
// kernel loads x once, reduces in registers and writes y once, instead of a
// round trip per elementary operation; "CuTeDSL at Perplexity", RMS-norm
// section: heads of 64-256 values, and the weight bias some models add).
//
// gfx950 mapping, one shape for both: a row of R 16-byte pieces belongs to a
// group of L lanes (L = R for a power-of-two R below 64; 64 lanes, one wave,
// for rows of up to 255 pieces; 256 lanes, the whole workgroup, for longer
// rows), each lane holding C = ceil(R / L) pieces: pieces p, p + L, p + 2L,
// ..., so every load of the group is one contiguous run.  The lane sums the
// squares of its pieces in fp32; an xor butterfly over the wave's lanes of
// the row (offsets below L never leave the group) and, for a row of four
// waves, their four partial sums added in wave order through LDS give every
// lane the row's sum; then the scale and the gain, and one 16-byte store per
// piece.  Spreading a long row over the workgroup keeps each lane at a few
// pieces: a copy of the same bytes measured 6.2-6.4 TB/s with one piece in
// flight per lane and 4.7-5.6 TB/s with fourteen.  x is read and y written
// exactly once, with non-temporal loads and stores.
//
// A launch covers up to two row sets (segments), each a contiguous array of
// rows with its own gain: the q heads and the k heads of QK-norm are two
// segments, the row RMSNorm one.  Every workgroup works inside one segment,
// chosen from its block index, so nothing per lane decides which tensor a
// row belongs to.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

struct RowSet {
  const char* x;   // rows [rows][n]
  char* y;         // output rows (may be x: in place)
  const char* w;   // gain [n]
  int64_t rows;
  int64_t blocks;  // workgroups of this segment
};

template <int ACT>
__device__ __forceinline__ void unpack(const u32x4& v, float* f) {
  if constexpr (ACT == ACT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_bits_to_f32(v[i] & 0xFFFFu);
      f[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
}

template <int ACT>
__device__ __forceinline__ u32x4 pack(const float* f) {
  u32x4 v;
  if constexpr (ACT == ACT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
  }
  return v;
}

}  // namespace

// L lanes per row (1..64, or 256), up to C pieces per lane; MASK: pieces
// past R exist in the lane layout (R not a multiple of L) and are skipped.
template <int ACT, int L, int C, bool MASK>
__global__ __launch_bounds__(256) void k_rms_rows(RowSet s0, RowSet s1, int n, int R,
                                                  float weight_bias, float eps) {
  constexpr int V = ACT == ACT_BF16 ? 8 : 4;  // values per 16-byte piece
  constexpr int ROWS_PER_WG = 256 / L;
  constexpr int WAVES_PER_ROW = L > WAVE ? L / WAVE : 1;
  static_assert(L <= WAVE || L == 256, "a row is a lane group or the whole workgroup");
  const bool second = (int64_t)blockIdx.x >= s0.blocks;  // uniform per workgroup
  const RowSet s = second ? s1 : s0;
  const int64_t blk = second ? (int64_t)blockIdx.x - s0.blocks : (int64_t)blockIdx.x;
  const int64_t row = blk * ROWS_PER_WG + threadIdx.x / L;
  const int p0 = threadIdx.x % L;
  const bool live = row < s.rows;
  const int64_t row_bytes = (int64_t)R * 16;
  const char* xr = s.x + (live ? row : 0) * row_bytes;
  char* yr = s.y + (live ? row : 0) * row_bytes;

  u32x4 xv[C];
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int p = p0 + c * L;
    const bool ok = live && (!MASK || p < R);
    xv[c] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + p * 16)) : zero;
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    float f[V];
    unpack<ACT>(xv[c], f);
#pragma unroll
    for (int v = 0; v < V; ++v) ss += f[v] * f[v];
  }
#pragma unroll
  for (int off = (L < WAVE ? L : WAVE) / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if constexpr (WAVES_PER_ROW > 1) {
    // one row per workgroup: the waves' sums, added in wave order
    __shared__ float wave_sum[256 / WAVE];
    if ((threadIdx.x & (WAVE - 1)) == 0) wave_sum[threadIdx.x / WAVE] = ss;
    __syncthreads();
    ss = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES_PER_ROW; ++w) ss += wave_sum[w];
  }
  const float scale = rsqrtf(ss / (float)n + eps);
  if (!live) return;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int p = p0 + c * L;
    if (MASK && p >= R) continue;
    float f[V], g[V];
    unpack<ACT>(xv[c], f);
    unpack<ACT>(ld16(s.w + p * 16), g);
#pragma unroll
    for (int v = 0; v < V; ++v) f[v] = f[v] * scale * (g[v] + weight_bias);
    __builtin_nontemporal_store(pack<ACT>(f), reinterpret_cast<u32x4*>(yr + p * 16));
  }
}

namespace {

template <int ACT, int L, int C, bool MASK>
hipError_t launch_rows(RowSet a, RowSet b, int n, int R, float wb, float eps, hipStream_t st) {
  constexpr int ROWS_PER_WG = 256 / L;
  a.blocks = (a.rows + ROWS_PER_WG - 1) / ROWS_PER_WG;
  b.blocks = (b.rows + ROWS_PER_WG - 1) / ROWS_PER_WG;
  const int64_t grid = a.blocks + b.blocks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_rms_rows<ACT, L, C, MASK>), dim3((unsigned)grid), dim3(256), 0, st, a, b,
                     n, R, wb, eps);
  return hipGetLastError();
}

// pieces per lane, rounded up to the instantiated counts (pieces past R are
// masked)
template <int ACT>
hipError_t launch_rows_any(RowSet a, RowSet b, int n, int R, float wb, float eps,
                           hipStream_t st) {
  if (R <= 0) return hipErrorInvalidValue;
  if (R < WAVE && (R & (R - 1)) == 0) {
    switch (R) {
      case 1: return launch_rows<ACT, 1, 1, false>(a, b, n, R, wb, eps, st);
      case 2: return launch_rows<ACT, 2, 1, false>(a, b, n, R, wb, eps, st);
      case 4: return launch_rows<ACT, 4, 1, false>(a, b, n, R, wb, eps, st);
      case 8: return launch_rows<ACT, 8, 1, false>(a, b, n, R, wb, eps, st);
      case 16: return launch_rows<ACT, 16, 1, false>(a, b, n, R, wb, eps, st);
      default: return launch_rows<ACT, 32, 1, false>(a, b, n, R, wb, eps, st);
    }
  }
  // rows of up to 255 pieces: one wave each; longer rows: the workgroup
  if (R < 256) {
    const int c = (R + WAVE - 1) / WAVE;
    const bool exact = R % WAVE == 0;
#define MOE_ROWS(L_, C_)                                                                      \
  if (c <= C_)                                                                                \
    return (exact && c == C_) ? launch_rows<ACT, L_, C_, false>(a, b, n, R, wb, eps, st)      \
                              : launch_rows<ACT, L_, C_, true>(a, b, n, R, wb, eps, st);
    MOE_ROWS(WAVE, 1)
    MOE_ROWS(WAVE, 2)
    MOE_ROWS(WAVE, 4)
  }
  const int c = (R + 255) / 256;
  const bool exact = R % 256 == 0;
  MOE_ROWS(256, 1)
  MOE_ROWS(256, 2)
  MOE_ROWS(256, 4)
  MOE_ROWS(256, 8)
#undef MOE_ROWS
  return hipErrorInvalidValue;
}

hipError_t launch_rms(int act, RowSet a, RowSet b, int n, float wb, float eps, hipStream_t st) {
  const int esz = act == ACT_BF16 ? 2 : 4;
  if ((int64_t)n * esz % 16 != 0) return hipErrorInvalidValue;
  const int R = (int)((int64_t)n * esz / 16);
  return act == ACT_BF16 ? launch_rows_any<ACT_BF16>(a, b, n, R, wb, eps, st)
                         : launch_rows_any<ACT_F32>(a, b, n, R, wb, eps, st);
}

}  // namespace

hipError_t launch_qk_norm(int act, void* q, void* k, const void* wq, const void* wk, int T,
                          int nq, int nk, int head_dim, float weight_bias, float eps,
                          hipStream_t st) {
  RowSet a{static_cast<const char*>(q), static_cast<char*>(q), static_cast<const char*>(wq),
           (int64_t)T * nq, 0};
  RowSet b{static_cast<const char*>(k), static_cast<char*>(k), static_cast<const char*>(wk),
           (int64_t)T * nk, 0};
  return launch_rms(act, a, b, head_dim, weight_bias, eps, st);
}

hipError_t launch_rms_norm(int act, const void* x, const void* w, void* y, int T, int d,
                           float weight_bias, float eps, hipStream_t st) {
  RowSet a{static_cast<const char*>(x), static_cast<char*>(y), static_cast<const char*>(w),
           (int64_t)T, 0};
  RowSet none{nullptr, nullptr, nullptr, 0, 0};
  return launch_rms(act, a, none, d, weight_bias, eps, st);
}

}  // namespace moe
