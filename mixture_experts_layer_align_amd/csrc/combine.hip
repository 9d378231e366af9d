// Top-k weighted combine: out[t] = sum_j w[t, j] * y[inv_pos[t*k + j]].
//
// "CuTeDSL at Perplexity", MoE dispatch and combine, local kernel: combine
// accumulates each token's expert outputs in registers, vectorised, using the
// routing weights and the positions dispatch assigned.  Here a workgroup
// handles one token and a 2048- (bf16 output) or 1024-element (fp32) chunk:
// each thread owns 8 or 4 consecutive elements, loads the k fp32 expert rows
// with 16-byte loads (first adding a row's k-split partial sums, in split
// order, when the down GEMM was split) and sums them in fp32 in slot order
// j = 0..k-1, then rounds once to the activation dtype.
//
// Few tokens (decode) leave most compute units idle with that shape, and each
// workgroup walks the k-splits one memory round trip after another.  There a
// one-wave workgroup covers 256 elements (4 per lane) and every row load of
// NS splits x JB slots is issued before the first add.
//
// YH: the expert rows are fp16 (the MFMA-tiled down GEMM's outputs) rather
// than fp32; they are widened exactly and summed the same way.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

// N consecutive values of expert row `row` (element offset c) as fp32
template <bool YH, int N>
__device__ __forceinline__ void load_row(const void* base, int64_t elem, float* v) {
  if constexpr (YH) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const char* p = reinterpret_cast<const char*>(base) + elem * 2;
    uint32_t w[N / 2];
    if constexpr (N == 8) {
      const u32x4 r = ld16(p);
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = r[q];
    } else {
      const u32x2 r = ld8(p);
      w[0] = r[0];
      w[1] = r[1];
    }
#pragma unroll
    for (int q = 0; q < N / 2; ++q) {
      const f16x2 h = __builtin_bit_cast(f16x2, w[q]);
      v[2 * q] = (float)h[0];
      v[2 * q + 1] = (float)h[1];
    }
  } else {
    const float* p = reinterpret_cast<const float*>(base) + elem;
#pragma unroll
    for (int h = 0; h < N / 4; ++h) {
      const u32x4 r = ld16(p + 4 * h);
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 * h + q] = __uint_as_float(r[q]);
    }
  }
}

}  // namespace

template <int ACT, int JB, bool YH>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y, int nsplit,
                                                 int64_t split_stride,
                                                 const int32_t* __restrict__ inv_pos,
                                                 const float* __restrict__ w, int k, int d,
                                                 char* __restrict__ out) {
  constexpr int VEC = ACT == ACT_BF16 ? 8 : 4;  // one 16-byte output store
  const int64_t t = blockIdx.x;
  const int32_t* ip = inv_pos + t * k;
  const float* wt = w + t * k;
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * VEC;
  if (c0 < d) {
    float acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
    // JB slots at a time (up to 4): every row load of the batch is issued
    // before any of them is added, so a token costs ~k/JB memory round trips,
    // not 2k
    for (int j0 = 0; j0 < k; j0 += JB) {
      int pos[JB];
      float wj[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const bool ok = j0 + jj < k;
        pos[jj] = ip[ok ? j0 + jj : 0];  // past k: slot 0 again, never added
        wj[jj] = ok ? wt[j0 + jj] : 0.f;
      }
      float ys[JB][VEC];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj)
#pragma unroll
        for (int v = 0; v < VEC; ++v) ys[jj][v] = 0.f;
      for (int s = 0; s < nsplit; ++s) {
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          float r[VEC];
          load_row<YH, VEC>(y, (int64_t)pos[jj] * d + c0 + s * split_stride, r);
#pragma unroll
          for (int v = 0; v < VEC; ++v) ys[jj][v] += r[v];
        }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj)
        if (j0 + jj < k) {
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] += wj[jj] * ys[jj][v];
        }
    }
    u32x4 o;
    if constexpr (ACT == ACT_BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      st16(out + (t * d + c0) * 2, o);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
      st16(out + (t * d + c0) * 4, o);
    }
  }
}

template <int ACT, int JB, int NS, bool YH>
__global__ __launch_bounds__(64) void k_combine_narrow(const void* __restrict__ y, int nsplit,
                                                       int64_t split_stride,
                                                       const int32_t* __restrict__ inv_pos,
                                                       const float* __restrict__ w, int k, int d,
                                                       char* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int32_t* ip = inv_pos + t * k;
  const float* wt = w + t * k;
  const int c0 = (blockIdx.y * 64 + threadIdx.x) * 4;
  if (c0 >= d) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += JB) {
    int pos[JB];
    float wj[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const bool ok = j0 + jj < k;
      pos[jj] = ip[ok ? j0 + jj : 0];  // past k: slot 0 again, never added
      wj[jj] = ok ? wt[j0 + jj] : 0.f;
    }
    float ys[JB][4];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v) ys[jj][v] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += NS) {
      // NS splits per pass; a split past the last reloads the last and is
      // not added (splits are still added in order)
      float r[NS][JB][4];
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        const int64_t so = (int64_t)min(s0 + q, nsplit - 1) * split_stride;
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
          load_row<YH, 4>(y, so + (int64_t)pos[jj] * d + c0, r[q][jj]);
      }
#pragma unroll
      for (int q = 0; q < NS; ++q)
        if (s0 + q < nsplit) {
#pragma unroll
          for (int jj = 0; jj < JB; ++jj)
#pragma unroll
            for (int v = 0; v < 4; ++v) ys[jj][v] += r[q][jj][v];
        }
    }
#pragma unroll
    for (int jj = 0; jj < JB; ++jj)
      if (j0 + jj < k) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] += wj[jj] * ys[jj][v];
      }
  }
  if constexpr (ACT == ACT_BF16) {
    const u32x2 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(out + (t * d + c0) * 2) = o;
  } else {
    const u32x4 o = {__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                     __float_as_uint(acc[3])};
    st16(out + (t * d + c0) * 4, o);
  }
}

// Token x 2048-element chunks below which the one-wave variant is used.
constexpr int NARROW_BELOW = 256;

template <int ACT, int JB, bool YH>
static void launch_narrow(const void* y, int nsplit, int64_t split_stride, const int32_t* inv_pos,
                          const float* w, int T, int k, int d, void* out, hipStream_t st) {
  const dim3 grid((unsigned)T, (unsigned)((d + 255) / 256));
  char* o = reinterpret_cast<char*>(out);
  if (nsplit >= 4)
    hipLaunchKernelGGL((k_combine_narrow<ACT, JB, 4, YH>), grid, dim3(64), 0, st, y, nsplit,
                       split_stride, inv_pos, w, k, d, o);
  else if (nsplit >= 2)
    hipLaunchKernelGGL((k_combine_narrow<ACT, JB, 2, YH>), grid, dim3(64), 0, st, y, nsplit,
                       split_stride, inv_pos, w, k, d, o);
  else
    hipLaunchKernelGGL((k_combine_narrow<ACT, JB, 1, YH>), grid, dim3(64), 0, st, y, nsplit,
                       split_stride, inv_pos, w, k, d, o);
}

template <bool YH>
static hipError_t launch_combine_y(int act, const void* y, int nsplit, int64_t split_stride,
                                   const int32_t* inv_pos, const float* w, int T, int k, int d,
                                   void* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int vec = act == ACT_BF16 ? 8 : 4;
  const dim3 grid((unsigned)T, (unsigned)((d + 256 * vec - 1) / (256 * vec)));
  const int jb = k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : 8;
  if ((int64_t)T * ((d + 2047) / 2048) < NARROW_BELOW) {
#define MOE_NARROW(A_, JB_) \
  launch_narrow<A_, JB_, YH>(y, nsplit, split_stride, inv_pos, w, T, k, d, out, st)
    if (act == ACT_BF16) {
      if (jb == 1) MOE_NARROW(ACT_BF16, 1);
      else if (jb == 2) MOE_NARROW(ACT_BF16, 2);
      else if (jb == 4) MOE_NARROW(ACT_BF16, 4);
      else MOE_NARROW(ACT_BF16, 8);
    } else {
      if (jb == 1) MOE_NARROW(ACT_F32, 1);
      else if (jb == 2) MOE_NARROW(ACT_F32, 2);
      else if (jb == 4) MOE_NARROW(ACT_F32, 4);
      else MOE_NARROW(ACT_F32, 8);
    }
#undef MOE_NARROW
    return hipGetLastError();
  }
  // many tokens: at most 4 slot rows in flight per thread (with 8, more
  // requests outstanding and 3-5 % slower at 8192-16384 tokens, top-8)
  const int jbw = jb > 4 ? 4 : jb;
#define MOE_COMBINE(A_, JB_)                                                                  \
  hipLaunchKernelGGL((k_combine<A_, JB_, YH>), grid, dim3(256), 0, st, y, nsplit, split_stride, \
                     inv_pos, w, k, d, reinterpret_cast<char*>(out))
  if (act == ACT_BF16) {
    if (jbw == 1) MOE_COMBINE(ACT_BF16, 1);
    else if (jbw == 2) MOE_COMBINE(ACT_BF16, 2);
    else MOE_COMBINE(ACT_BF16, 4);
  } else {
    if (jbw == 1) MOE_COMBINE(ACT_F32, 1);
    else if (jbw == 2) MOE_COMBINE(ACT_F32, 2);
    else MOE_COMBINE(ACT_F32, 4);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

hipError_t launch_combine(int act, const void* y, bool y_f16, int nsplit, int64_t split_stride,
                          const int32_t* inv_pos, const float* w, int T, int k, int d, void* out,
                          hipStream_t st) {
  return y_f16 ? launch_combine_y<true>(act, y, nsplit, split_stride, inv_pos, w, T, k, d, out, st)
               : launch_combine_y<false>(act, y, nsplit, split_stride, inv_pos, w, T, k, d, out,
                                         st);
}

}  // namespace moe
