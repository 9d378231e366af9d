// Per-head RMS normalisation of query and key heads (QK-norm), in place.
//
// "CuTeDSL at Perplexity", section on the RMS-norm kernel specialised for
// small dimensions: for every token and every head of q and of k,
//   x <- (w + weight_bias) * x * rsqrt(sum(x * x) / head_dim + eps),
// w being the tensor's weight (one value per position in the head, shared by
// its heads).  A head of 64-256 elements needs a reduction only among the
// lanes that hold it, never across waves or through LDS.
//
// gfx950 mapping: every lane loads 16 bytes of one head (8 bf16 or 4 fp32
// values), head_dim*esize/16 lanes hold a head (an aligned power-of-two group
// of 8-64 lanes), so a wave normalises 64/group heads at once.  The squares
// are summed in fp32 by an xor butterfly inside the group (xor offsets below
// the group size never leave it), the reciprocal square root scales the
// lane's values, and the biased weight is applied before one 16-byte store.
// Consecutive heads of a token are contiguous in q and in k, so a wave reads
// and writes 1 KB runs: the kernel streams q and k once (HBM-bound), with
// non-temporal loads and stores.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

template <int ACT, int LPH>
__global__ __launch_bounds__(256) void k_qk_norm(char* __restrict__ q, char* __restrict__ k,
                                                 const char* __restrict__ wq,
                                                 const char* __restrict__ wk, int64_t heads,
                                                 int nq, int nk, int head_dim, float weight_bias,
                                                 float eps) {
  constexpr int VEC = ACT == ACT_BF16 ? 8 : 4;  // values in one 16-byte piece
  constexpr int ESZ = ACT == ACT_BF16 ? 2 : 4;
  const int lane = threadIdx.x & (WAVE - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / WAVE;
  const int64_t g = wave * (WAVE / LPH) + lane / LPH;  // head of this lane's group
  const int part = lane % LPH;                          // its 16-byte piece
  const bool ok = g < heads;
  const int nh = nq + nk;
  const int64_t t = ok ? g / nh : 0;
  const int h = ok ? (int)(g % nh) : 0;
  const bool isq = h < nq;
  char* row = isq ? q + (t * nq + h) * (int64_t)head_dim * ESZ
                  : k + (t * nk + (h - nq)) * (int64_t)head_dim * ESZ;
  const char* wrow = isq ? wq : wk;

  const u32x4 zero = {0u, 0u, 0u, 0u};
  // q and k are streamed once: non-temporal load and store (measured 16 %
  // faster than the default cache policy, and faster than a plain copy)
  const u32x4 xr =
      ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + part * 16)) : zero;
  const u32x4 wr = ok ? ld16(wrow + part * 16) : zero;
  float x[VEC], w[VEC];
  if constexpr (ACT == ACT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(xr[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_bits_to_f32(xr[i] >> 16);
      w[2 * i] = bf16_bits_to_f32(wr[i] & 0xFFFFu);
      w[2 * i + 1] = bf16_bits_to_f32(wr[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(xr[i]);
      w[i] = __uint_as_float(wr[i]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < VEC; ++v) ss += x[v] * x[v];
#pragma unroll
  for (int off = LPH / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = rsqrtf(ss / (float)head_dim + eps);
  float y[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) y[v] = (w[v] + weight_bias) * (x[v] * inv);
  if (ok) {
    u32x4 o;
    if constexpr (ACT == ACT_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(y[i]);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(row + part * 16));
  }
}

hipError_t launch_qk_norm(int act, void* q, void* k, const void* wq, const void* wk, int T,
                          int nq, int nk, int head_dim, float weight_bias, float eps,
                          hipStream_t st) {
  const int64_t heads = (int64_t)T * (nq + nk);
  if (heads == 0) return hipSuccess;
  const int esz = act == ACT_BF16 ? 2 : 4;
  const int lph = head_dim * esz / 16;  // 8..64 lanes per head
  const int64_t lanes = heads * lph;
  const int64_t blocks = (lanes + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  char* qc = static_cast<char*>(q);
  char* kc = static_cast<char*>(k);
  const char* wqc = static_cast<const char*>(wq);
  const char* wkc = static_cast<const char*>(wk);
#define MOE_QKN(A_, L_)                                                                        \
  hipLaunchKernelGGL((k_qk_norm<A_, L_>), dim3((unsigned)blocks), dim3(256), 0, st, qc, kc, wqc, \
                     wkc, heads, nq, nk, head_dim, weight_bias, eps)
  if (act == ACT_BF16) {
    if (lph == 8) MOE_QKN(ACT_BF16, 8);
    else if (lph == 16) MOE_QKN(ACT_BF16, 16);
    else if (lph == 32) MOE_QKN(ACT_BF16, 32);
    else return hipErrorInvalidValue;
  } else {
    if (lph == 16) MOE_QKN(ACT_F32, 16);
    else if (lph == 32) MOE_QKN(ACT_F32, 32);
    else if (lph == 64) MOE_QKN(ACT_F32, 64);
    else return hipErrorInvalidValue;
  }
#undef MOE_QKN
  return hipGetLastError();
}

}  // namespace moe
