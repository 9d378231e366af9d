// Device-side building blocks shared by the libmoe kernels (gfx950 / CDNA4).
//
// Layout facts relied on throughout (CDNA3/CDNA4 MFMA operand layouts, wave64):
//   v_mfma_f32_16x16x32_bf16  A: lane l holds row (l % 16), 8 k-values of group
//                             (l / 16); B: lane l holds column (l % 16), the 8
//                             k-values of group (l / 16); D: lane l holds rows
//                             4*(l/16) + 0..3 of column (l % 16).
//   v_mfma_f32_16x16x4_f32    A: lane l holds A[l % 16][l / 16]; B: B[l / 16][l % 16];
//                             D as above.
// Only the D layout must be exact: A and B fragments are packed with the same
// (lane group, element) -> k map, so any k ordering the hardware uses pairs the
// same products.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Round-to-nearest-even float -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ------------------------------------------------------------ vector loads

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ------------------------------------------------- in-register transposes

// v_perm_b32 selectors: low halves of (b, a) -> (b.lo | a.lo << 16); high halves.
__device__ __forceinline__ uint32_t perm_lo16(uint32_t b_low_row, uint32_t a_high_row) {
  return __builtin_amdgcn_perm(a_high_row, b_low_row, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi16(uint32_t b_low_row, uint32_t a_high_row) {
  return __builtin_amdgcn_perm(a_high_row, b_low_row, 0x07060302u);
}

// 8x8 transpose of 16-bit elements held by one lane.
// in[r]  = row r  : 4 dwords, dword j = (col 2j | col 2j+1 << 16)
// out[c] = col c  : 4 dwords, dword q = (row 2q | row 2q+1 << 16)
__device__ __forceinline__ void transpose8x8_b16(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      out[2 * j][q] = perm_lo16(in[2 * q][j], in[2 * q + 1][j]);
      out[2 * j + 1][q] = perm_hi16(in[2 * q][j], in[2 * q + 1][j]);
    }
  }
}

// ---------------------------------------------------------------- fp8

// 8 OCP e4m3fn codes (one row, 8 columns) -> 8 bf16 (4 dwords, column pairs).
// Every e4m3fn value is exactly representable in bf16, and the scale operand is
// 1.0, so the conversion is exact.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 v) {
  u32x4 r;
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true);
  r[0] = __builtin_bit_cast(uint32_t, a);
  r[1] = __builtin_bit_cast(uint32_t, b);
  r[2] = __builtin_bit_cast(uint32_t, c);
  r[3] = __builtin_bit_cast(uint32_t, d);
  return r;
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// nv values (multiple of 8 for bf16, 4 for fp32) to a 16-byte aligned
// destination in the activation dtype, rounding to nearest even for bf16.
template <int ACT_IS_BF16>
__device__ __forceinline__ void store_act(char* dst, const float* v, int nv) {
  if constexpr (ACT_IS_BF16 == 1) {
    for (int j = 0; j < nv; j += 8) {
      u32x4 o;
      o[0] = pack_bf16x2(v[j + 0], v[j + 1]);
      o[1] = pack_bf16x2(v[j + 2], v[j + 3]);
      o[2] = pack_bf16x2(v[j + 4], v[j + 5]);
      o[3] = pack_bf16x2(v[j + 6], v[j + 7]);
      st16(dst + j * 2, o);
    }
  } else {
    for (int j = 0; j < nv; j += 4) {
      u32x4 o = {__float_as_uint(v[j]), __float_as_uint(v[j + 1]), __float_as_uint(v[j + 2]),
                 __float_as_uint(v[j + 3])};
      st16(dst + j * 4, o);
    }
  }
}

// v as a pair of bf16, hi = bf16(v) and lo = bf16(v - hi) (both round to
// nearest even): hi + lo carries v to 16 significant bits, so a bf16 MFMA fed
// with both halves sees v with a relative error of at most 2^-17.
template <int NV>
__device__ __forceinline__ void store_bf16_pair(char* dst_hi, char* dst_lo, const float* v) {
  static_assert(NV % 8 == 0, "16-byte stores");
  for (int j = 0; j < NV; j += 8) {
    u32x4 oh, ol;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t h0 = f32_to_bf16_bits(v[j + 2 * q]), h1 = f32_to_bf16_bits(v[j + 2 * q + 1]);
      oh[q] = h0 | (h1 << 16);
      ol[q] = pack_bf16x2(v[j + 2 * q] - bf16_bits_to_f32(h0),
                          v[j + 2 * q + 1] - bf16_bits_to_f32(h1));
    }
    st16(dst_hi + j * 2, oh);
    st16(dst_lo + j * 2, ol);
  }
}

// ------------------------------------------------------------ activation

// SiLU(z) = z * sigmoid(z), from the hardware base-2 exponential and
// reciprocal (a few fp32 ulps; h is rounded to bf16 or kept in fp32 against a
// 1e-4 relative tolerance).  Large |z| reach the limits: exp2 overflows to
// inf and the reciprocal to 0 for z << 0, and the sigmoid is 1 for z >> 0.
__device__ __forceinline__ float silu(float z) {
  constexpr float LOG2E = 1.4426950408889634f;
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * LOG2E));
}

// ------------------------------------------------------------ wave helpers

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
