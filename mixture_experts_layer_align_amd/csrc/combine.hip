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
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

template <int ACT, int JB>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y, int nsplit,
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
    // JB slots at a time (JB >= k up to 8): every row load of the batch is
    // issued before any of them is added, so a token costs ~k/JB memory round
    // trips, not 2k
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
          const float* row = y + (int64_t)pos[jj] * d + c0 + s * split_stride;
#pragma unroll
          for (int h = 0; h < VEC / 4; ++h) {
            const u32x4 r = ld16(row + 4 * h);
#pragma unroll
            for (int q = 0; q < 4; ++q) ys[jj][4 * h + q] += __uint_as_float(r[q]);
          }
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

hipError_t launch_combine(int act, const float* y, int nsplit, int64_t split_stride,
                          const int32_t* inv_pos, const float* w, int T, int k, int d, void* out,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int vec = act == ACT_BF16 ? 8 : 4;
  const dim3 grid((unsigned)T, (unsigned)((d + 256 * vec - 1) / (256 * vec)));
  const int jb = k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : 8;
#define MOE_COMBINE(A_, JB_)                                                                  \
  hipLaunchKernelGGL((k_combine<A_, JB_>), grid, dim3(256), 0, st, y, nsplit, split_stride, \
                     inv_pos, w, k, d, reinterpret_cast<char*>(out))
  if (act == ACT_BF16) {
    if (jb == 1) MOE_COMBINE(ACT_BF16, 1);
    else if (jb == 2) MOE_COMBINE(ACT_BF16, 2);
    else if (jb == 4) MOE_COMBINE(ACT_BF16, 4);
    else MOE_COMBINE(ACT_BF16, 8);
  } else {
    if (jb == 1) MOE_COMBINE(ACT_F32, 1);
    else if (jb == 2) MOE_COMBINE(ACT_F32, 2);
    else if (jb == 4) MOE_COMBINE(ACT_F32, 4);
    else MOE_COMBINE(ACT_F32, 8);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
