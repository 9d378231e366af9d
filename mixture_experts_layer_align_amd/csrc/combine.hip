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

template <int ACT>
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
    for (int j = 0; j < k; ++j) {
      const float wj = wt[j];
      const float* row = y + (int64_t)ip[j] * d + c0;
      float ys[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) ys[v] = 0.f;
      for (int s = 0; s < nsplit; ++s) {
#pragma unroll
        for (int h = 0; h < VEC / 4; ++h) {
          const u32x4 r = ld16(row + s * split_stride + 4 * h);
#pragma unroll
          for (int q = 0; q < 4; ++q) ys[4 * h + q] += __uint_as_float(r[q]);
        }
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] += wj * ys[v];
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
  if (act == ACT_BF16)
    hipLaunchKernelGGL(k_combine<ACT_BF16>, grid, dim3(256), 0, st, y, nsplit, split_stride,
                       inv_pos, w, k, d, reinterpret_cast<char*>(out));
  else
    hipLaunchKernelGGL(k_combine<ACT_F32>, grid, dim3(256), 0, st, y, nsplit, split_stride,
                       inv_pos, w, k, d, reinterpret_cast<char*>(out));
  return hipGetLastError();
}

}  // namespace moe
