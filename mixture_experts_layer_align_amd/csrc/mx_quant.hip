// MXFP8 quantisation of activation rows (moe_quantize_mxfp8).
//
// "CuTeDSL at Perplexity", section on Blackwell support: the block-scaled
// formats quantise in blocks of 32 consecutive elements sharing one scale
// found from the block's absmax, an absmax the post takes with sub-warp
// reductions.  With the OCP MX rule for MXFP8 (E4M3 elements, E8M0 scale):
//   s = floor(log2(absmax)) - 8, at least -127 (an all-zero block: -127),
//   code = E4M3(x * 2^-s), nearest with ties to even, saturated at +-448,
//   scale byte = s + 127.
//
// gfx950 mapping: one 16-byte piece per lane (8 bf16 or 4 fp32 values), so a
// 32-element block is 4 (bf16) or 8 (fp32) consecutive, aligned lanes; their
// absmax comes from an xor butterfly over those lanes only.  floor(log2) of
// the fp32 absmax is its biased exponent field E minus 127, so the scale byte
// is max(E - 8, 0) (a zero or fp32-subnormal absmax gives 0, the clamp) and
// 2^-s is the fp32 with exponent field 254 - byte: x * 2^-s is exact.  The
// product is clamped to +-448 and converted by v_cvt_pk_fp8_f32 (OCP E4M3
// on gfx950, round to nearest even), two values per instruction.  Each lane
// stores its codes (8 or 4 bytes, contiguous across the wave); the first lane
// of every four blocks gathers their four scale bytes by shuffles and stores
// one 32-bit word.  x is read once with non-temporal loads.  (Tried: 16-byte
// code stores from lane pairs and non-temporal code stores, neither faster.)
#include <algorithm>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

template <int ACT>
__global__ __launch_bounds__(256) void k_mx_quant(const char* __restrict__ x,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales, int64_t pieces) {
  constexpr int V = ACT == ACT_BF16 ? 8 : 4;  // values per 16-byte piece
  constexpr int LPB = 32 / V;                 // lanes per 32-element block
  // grid-stride over 256-piece runs (the stride keeps blocks lane-aligned)
  for (int64_t base = (int64_t)blockIdx.x * 256; base < pieces;
       base += (int64_t)gridDim.x * 256) {
    const int64_t g = base + threadIdx.x;
    const bool live = g < pieces;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // lanes past the end take part in the shuffles with zeros and store nothing
    const u32x4 raw =
        live ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + g * 16)) : zero;
    float f[V];
    if constexpr (ACT == ACT_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_bits_to_f32(raw[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(raw[i]);
    }
    float amax = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) amax = fmaxf(amax, fabsf(f[v]));
    // the block's absmax: its LPB lanes are consecutive and LPB-aligned
#pragma unroll
    for (int off = 1; off < LPB; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const uint32_t ex = __float_as_uint(amax) >> 23;  // biased exponent (amax >= 0)
    const uint32_t sbyte = ex > 8u ? ex - 8u : 0u;    // s + 127
    const float mult = __uint_as_float((254u - sbyte) << 23);  // 2^-s
    uint32_t out[V / 4];
#pragma unroll
    for (int w = 0; w < V / 4; ++w) {
      float q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) q[j] = fminf(fmaxf(f[4 * w + j] * mult, -448.f), 448.f);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], pk, true);
      out[w] = (uint32_t)pk;
    }
    // scale bytes of the lane's block and of the next three blocks
    const uint32_t b1 = __shfl_down(sbyte, LPB);
    const uint32_t b2 = __shfl_down(sbyte, 2 * LPB);
    const uint32_t b3 = __shfl_down(sbyte, 3 * LPB);
    if (!live) continue;
    if constexpr (V == 8) {
      *reinterpret_cast<u32x2*>(codes + g * 8) = u32x2{out[0], out[1]};
    } else {
      *reinterpret_cast<uint32_t*>(codes + g * 4) = out[0];
    }
    if ((threadIdx.x & (4 * LPB - 1)) == 0) {
      const int64_t blk = g / LPB;  // a multiple of 4
      const int64_t nblk = pieces / LPB;
      if (blk + 4 <= nblk) {
        *reinterpret_cast<uint32_t*>(scales + blk) = sbyte | (b1 << 8) | (b2 << 16) | (b3 << 24);
      } else {
        const uint32_t b[4] = {sbyte, b1, b2, b3};
        for (int j = 0; j < (int)(nblk - blk); ++j) scales[blk + j] = (uint8_t)b[j];
      }
    }
  }
}

hipError_t launch_mx_quant(int act, const void* x, void* codes, void* scales, int64_t rows, int n,
                           hipStream_t st) {
  const int esz = act == ACT_BF16 ? 2 : 4;
  if (n <= 0 || n % 32 != 0 || rows < 0) return hipErrorInvalidValue;
  const int64_t pieces = rows * n * esz / 16;
  if (pieces == 0) return hipSuccess;
  // 64 workgroups per compute unit, each looping over its runs (measured at
  // 16384 x 7168 bf16: 5.6 TB/s, against 5.3 with one workgroup per run and
  // 5.3-5.5 with 32 or 128 per unit)
  const int64_t grid = std::min<int64_t>((pieces + 255) / 256, 64 * (int64_t)device_cus());
  auto* xc = static_cast<const char*>(x);
  auto* cc = static_cast<uint8_t*>(codes);
  auto* sc = static_cast<uint8_t*>(scales);
  if (act == ACT_BF16)
    hipLaunchKernelGGL(k_mx_quant<ACT_BF16>, dim3((unsigned)grid), dim3(256), 0, st, xc, cc, sc,
                       pieces);
  else
    hipLaunchKernelGGL(k_mx_quant<ACT_F32>, dim3((unsigned)grid), dim3(256), 0, st, xc, cc, sc,
                       pieces);
  return hipGetLastError();
}

}  // namespace moe
