// Router logits GEMM: L[t, e] = sum_i x[t, i] * W_r[i, e] (fp32 accumulation),
// written per k-split as fp32 partial planes that the top-k kernel sums in a
// fixed order.
//
// The router weight [d, E] is stored like an expert weight ([K, N], N
// contiguous, per the A[M,K] x B[K,N] statement of the vLLM fused-MoE post,
// section "Swap-AB"), and is thin in N: E is 8 to 1024.  The same
// operand-swapped MFMA mapping as the expert GEMMs is used — weight columns on
// the MFMA row side, tokens on the column side, an in-register 8x8 transpose of
// 16-byte weight loads into A fragments — with loads staged in registers
// because E need not be a multiple of the 16-byte chunk: columns past E are
// read element by element and zero-filled.  A workgroup is two waves, each
// streaming one 128-column slab (bf16; 64 for fp32) of its k-range for a block
// of 32 tokens (when E fits one slab, or few token blocks leave the chip
// idle, a tile is one slab that the two waves share, splitting the k-range),
// with its loads running three k-steps ahead of its MFMAs.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

template <int WT>
struct RTr;
template <>
struct RTr<W_BF16> {
  static constexpr int CPL = 8;     // columns per lane load
  static constexpr int RPL = 8;     // weight rows per lane per k-step
  static constexpr int KSTEP = 32;
  static constexpr int ESIZE = 2;
};
template <>
struct RTr<W_F32> {
  static constexpr int CPL = 4;
  static constexpr int RPL = 4;
  static constexpr int KSTEP = 16;
  static constexpr int ESIZE = 4;
};

// CPL columns of one weight row starting at `col`; columns at or past n_valid
// read as zero.  `vec_ok`: rows are 16-byte aligned.
template <int WT>
__device__ __forceinline__ u32x4 load_wrow(const char* rowp, int col, int n_valid, bool vec_ok) {
  constexpr int CPL = RTr<WT>::CPL;
  if (vec_ok && col + CPL <= n_valid) return ld16(rowp + (int64_t)col * RTr<WT>::ESIZE);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (col >= n_valid) return v;  // wholly past E: nothing to read
  if constexpr (WT == W_BF16) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(rowp);
    for (int c = 0; c < CPL; ++c)
      if (col + c < n_valid) v[c >> 1] |= (uint32_t)h[col + c] << (16 * (c & 1));
  } else {
    const uint32_t* f = reinterpret_cast<const uint32_t*>(rowp);
    for (int c = 0; c < CPL; ++c)
      if (col + c < n_valid) v[c] = f[col + c];
  }
  return v;
}

}  // namespace

template <int WT>
__global__ __launch_bounds__(128) void k_router_gemm(const StreamGemmArgs p) {
  using Tr = RTr<WT>;
  constexpr int CPL = Tr::CPL;
  constexpr int RPL = Tr::RPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int SW = 16 * CPL;
  constexpr int NV = 4 * CPL;
  constexpr int ASZ = Tr::ESIZE;  // router weight and tokens share the activation dtype

  const int lane = threadIdx.x & 63;
  const int slab = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  int id = blockIdx.x;
  const int split = id % p.ksplit;
  id /= p.ksplit;
  const int nt = id % p.n_tiles;
  const int mb = id / p.n_tiles;
  const int p0 = mb * STREAM_BM;

  const char* arow[2];
  bool rvalid[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int prow = p0 + 16 * q + li;
    rvalid[q] = prow < p.m_total;
    arow[q] = reinterpret_cast<const char*>(p.a) + (int64_t)(rvalid[q] ? prow : 0) * p.a_ld * ASZ;
  }
  const bool use_q1 = ballot(rvalid[1]) != 0;
  // One-slab tiles (n_tiles * SW >= E: E within one slab, or few token
  // blocks, where the plan takes one slab per tile to run more workgroups):
  // both waves take the tile's slab, wave 0 the first half of the split's
  // k-steps and wave 1 the rest (its sums are added to wave 0's afterwards).
  // Otherwise a tile is two slabs, one per wave.
  const bool kpair = p.n_tiles * SW >= p.n_out;
  const int tbase = kpair ? nt * SW : nt * 2 * SW + slab * SW;
  const int wcol = tbase + CPL * li;
  const int ocol = tbase + lg * NV;
  const char* w = reinterpret_cast<const char*>(p.w);
  const int64_t wrow_bytes = p.w_ld * Tr::ESIZE;
  const bool vec_ok = (p.w_ld % CPL) == 0;
  int kb = split * p.kchunk;
  int ke = min(p.K, kb + p.kchunk);
  if (kpair) {
    const int half = ((ke - kb) / KSTEP + 1) / 2 * KSTEP;
    if (slab == 0)
      ke = kb + half;
    else
      kb += half;
  }

  f32x4 acc[2][CPL];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[q][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // k-steps of this split; loads run DEPTH steps ahead of the MFMAs in a
  // register ring (clamped past the end: reloads of the last step, in bounds
  // and never used), so a workgroup is not bound by one memory latency per
  // step
  const int nsteps = (ke - kb) / KSTEP;
  if (ocol - lg * NV < p.n_out && nsteps > 0) {
    constexpr int DEPTH = 3;
    u32x4 raw[DEPTH][RPL], xv[DEPTH][2];
    auto load = [&](int d, int step) __attribute__((always_inline)) {
      const int k0 = kb + min(step, nsteps - 1) * KSTEP;
      const char* base = w + (int64_t)(k0 + lg * RPL) * wrow_bytes;
#pragma unroll
      for (int j = 0; j < RPL; ++j) raw[d][j] = load_wrow<WT>(base + j * wrow_bytes, wcol, p.n_out, vec_ok);
      const int kk = k0 + (WT == W_BF16 ? 8 : 4) * lg;
      const u32x4 z = {0u, 0u, 0u, 0u};
      xv[d][0] = rvalid[0] ? ld16(arow[0] + (int64_t)kk * ASZ) : z;
      xv[d][1] = rvalid[1] ? ld16(arow[1] + (int64_t)kk * ASZ) : z;
    };
    auto compute = [&](int d) __attribute__((always_inline)) {
      const u32x4 x0 = xv[d][0], x1 = xv[d][1];
      if constexpr (WT == W_F32) {
#pragma unroll
        for (int ss = 0; ss < 4; ++ss)
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float a = __uint_as_float(raw[d][ss][c]);
            acc[0][c] = mfma_f32_16x16x4(a, __uint_as_float(x0[ss]), acc[0][c]);
            if (use_q1) acc[1][c] = mfma_f32_16x16x4(a, __uint_as_float(x1[ss]), acc[1][c]);
          }
      } else {
        u32x4 frag[8];
        transpose8x8_b16(raw[d], frag);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          acc[0][c] = mfma_bf16_16x16x32(frag[c], x0, acc[0][c]);
          if (use_q1) acc[1][c] = mfma_bf16_16x16x32(frag[c], x1, acc[1][c]);
        }
      }
    };
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) load(d, d);
    for (int it = 0; it < nsteps; it += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        load((d + DEPTH - 1) % DEPTH, it + d + DEPTH - 1);
        if (it + d < nsteps) compute(d);
      }
    }
  }
  if (kpair) {
    // wave 0's sums + wave 1's, in that order
    __shared__ f32x4 xch[2][CPL][WAVE];
    if (slab == 1) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int c = 0; c < CPL; ++c) xch[q][c][lane] = acc[q][c];
    }
    __syncthreads();
    if (slab == 1) return;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const f32x4 o = xch[q][c][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[q][c][r] += o[r];
      }
  }
  // lane (li, lg) holds, for row group q, columns ocol + r*CPL + c in acc[q][c][r]:
  // CPL consecutive columns per r, stored 16 bytes at a time when rows are
  // 16-byte aligned (E % 4 == 0) and the run lies within E
  const bool vst = (p.out_ld % 4) == 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (!rvalid[q]) continue;
    float* dst = reinterpret_cast<float*>(p.out) + split * p.out_split_stride +
                 (int64_t)(p0 + 16 * q + li) * p.out_ld;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col0 = ocol + r * CPL;
      if (vst && col0 + CPL <= p.n_out) {
#pragma unroll
        for (int c4 = 0; c4 < CPL; c4 += 4) {
          const u32x4 o = {__float_as_uint(acc[q][c4][r]), __float_as_uint(acc[q][c4 + 1][r]),
                           __float_as_uint(acc[q][c4 + 2][r]), __float_as_uint(acc[q][c4 + 3][r])};
          st16(dst + col0 + c4, o);
        }
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          if (col0 + c < p.n_out) dst[col0 + c] = acc[q][c][r];
      }
    }
  }
}

int router_tile_cols(int act_dtype) { return act_dtype == ACT_BF16 ? 256 : 128; }
int router_slab_cols(int act_dtype) { return router_tile_cols(act_dtype) / 2; }
int router_kstep(int act_dtype) { return act_dtype == ACT_BF16 ? 32 : 16; }

hipError_t launch_router_gemm(int act, const StreamGemmArgs& a, hipStream_t st) {
  const int64_t grid = (int64_t)a.num_mblocks * a.n_tiles * a.ksplit;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (act == ACT_BF16)
    hipLaunchKernelGGL(k_router_gemm<W_BF16>, dim3((unsigned)grid), dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL(k_router_gemm<W_F32>, dim3((unsigned)grid), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
