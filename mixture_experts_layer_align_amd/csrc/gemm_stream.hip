// Weight-streaming grouped GEMM for the expert (and router) matmuls.
//
// Expert compute is A[M,K] x B[K,N] -> C[M,N] with M token rows, K the hidden
// size and N the expert's output width (vLLM fused-MoE post, section
// "Swap-AB"); B is the expert weight stored [K, N], N contiguous.  When M is
// thin (decode), the pages' Hopper answer is to swap operands so the large N
// fills the fixed 64-row side of the tensor-core instruction.  The gfx950
// version of that idea:
//
//   * the weight panel is the MFMA A operand (rows = output columns n), the
//     tokens are the B operand (columns = rows of the block), so 16 output
//     columns x 16 tokens are produced per v_mfma_f32_16x16x32_bf16;
//   * each lane loads 8 consecutive weight rows of 16 bytes (8 bf16 columns) —
//     16 lanes cover 256 contiguous bytes of a weight row, fully coalesced —
//     and transposes its 8x8 block in registers (v_perm_b32) into 8 MFMA A
//     fragments, so weights go HBM -> VGPR once with no LDS round trip;
//   * a wave owns (32-row block of one expert, n-tile, k-range) and applies
//     every weight fragment to all rows of its block (weight-stationary), with
//     a 16-row group skipped when it holds no routed row;
//   * tokens are gathered straight from x by the aligned slot list, so the
//     permuted activations are never materialised (the pages copy tokens into
//     padded per-expert buffers first: "CuTeDSL at Perplexity", MoE dispatch
//     and combine, local kernel);
//   * when blocks x n-tiles cannot fill 256 CUs, K is split; each split stores
//     an fp32 partial and the last split to finish (an integer counter decides
//     who, not what) sums all partials in split order, so results do not
//     depend on scheduling;
//   * the epilogue runs on the fp32 accumulators before the single store:
//     SiLU(gate) * up for the concatenated gate|up weight ("La fusion de
//     noyaux", section 4.2, GEMM + epilogue and the SwiGLU concatenation), and
//     the fp8 per-column scale, applied after the dot product.  h is stored in
//     the activation dtype (its rounding errors average out over the down
//     GEMM's K); the down GEMM's per-slot outputs are stored in fp32, because
//     each output element adds k of them directly and a bf16 rounding there
//     would stack on the output's own.
//
// fp8 (OCP e4m3fn) weights are converted exactly to bf16 in registers and run
// on the same bf16 MFMA (activations stay bf16).  fp32 weights use
// v_mfma_f32_16x16x4_f32 with 4 columns per lane and no transpose.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

template <int WT>
struct WTr;

template <>
struct WTr<W_BF16> {
  static constexpr int CPL = 8;     // weight columns per lane load
  static constexpr int KSTEP = 32;  // K rows per step
  static constexpr int ESIZE = 2;
  struct Raw { u32x4 r[8]; };       // 8 rows x 8 columns
};

template <>
struct WTr<W_FP8> {
  static constexpr int CPL = 8;
  static constexpr int KSTEP = 32;
  static constexpr int ESIZE = 1;
  struct Raw { u32x2 r[8]; };
};

template <>
struct WTr<W_F32> {
  static constexpr int CPL = 4;
  static constexpr int KSTEP = 16;
  static constexpr int ESIZE = 4;
  struct Raw { u32x4 r[4]; };       // 4 rows x 4 columns
};

template <int WT>
struct SlabW {
  static constexpr int value = 16 * WTr<WT>::CPL;   // weight columns per slab
};

// Weight chunk of one lane for one row: CPL columns starting at `col`, columns
// at or past n_valid read as zero when MASKED.
// `vec_ok`: rows are 16-byte aligned so a full chunk may use one vector load.
template <int WT, bool MASKED>
__device__ __forceinline__ auto load_wrow(const char* rowp, int col, int n_valid, bool vec_ok) {
  using Tr = WTr<WT>;
  constexpr int CPL = Tr::CPL;
  constexpr int ES = Tr::ESIZE;
  if constexpr (WT == W_FP8) {
    if (!MASKED || (vec_ok && col + CPL <= n_valid)) return ld8(rowp + (int64_t)col * ES);
    u32x2 v = {0u, 0u};
    for (int c = 0; c < CPL; ++c)
      if (col + c < n_valid) {
        uint32_t b = (uint32_t)(uint8_t)rowp[col + c];
        v[c >> 2] |= b << (8 * (c & 3));
      }
    return v;
  } else {
    if (!MASKED || (vec_ok && col + CPL <= n_valid)) return ld16(rowp + (int64_t)col * ES);
    u32x4 v = {0u, 0u, 0u, 0u};
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
}

template <int ACT>
__device__ __forceinline__ void store_chunk(char* dst, const float* v, int nv) {
  // nv values, contiguous, destination 16-byte aligned
  if constexpr (ACT == ACT_BF16) {
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

template <int ACT, int WT, int EPI>
__global__ __launch_bounds__(64) void k_stream_gemm(const StreamGemmArgs p) {
  using Tr = WTr<WT>;
  using Raw = typename Tr::Raw;
  constexpr int CPL = Tr::CPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int SW = SlabW<WT>::value;
  constexpr int ASZ = (ACT == ACT_BF16) ? 2 : 4;
  constexpr bool MASKED = (EPI == EPI_F32);
  constexpr int NV = 4 * CPL;  // contiguous output columns per lane per slab

  const int lane = threadIdx.x;
  const int li = lane & 15;  // MFMA column within a 16-group (token row)
  const int lg = lane >> 4;  // k group

  int id = blockIdx.x;
  const int split = id % p.ksplit;
  id /= p.ksplit;
  const int nt = id % p.n_tiles;
  const int mb = id / p.n_tiles;
  int e = 0;
  if (p.block_expert != nullptr) {
    e = p.block_expert[mb];
    if (e < 0) return;
  }
  const int p0 = mb * STREAM_BM;

  // -------------------------------------------------------- token rows
  const char* arow[2];
  bool rvalid[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int prow = p0 + 16 * q + li;
    int64_t src = prow;
    bool v;
    if (p.a_mode == A_DENSE) {
      v = prow < p.m_total;
    } else {
      const int sid = p.sorted_ids[prow];
      v = sid >= 0;
      if (p.a_mode == A_GATHER) src = v ? sid / p.topk : 0;
    }
    rvalid[q] = v;
    arow[q] = reinterpret_cast<const char*>(p.a) + (v ? src : 0) * p.a_ld * ASZ;
  }
  const bool use_q1 = ballot(rvalid[1]) != 0;

  // -------------------------------------------------------- weight columns
  int wcol[2];
  int ocol0;  // first output column of this lane's chunk in slab 0
  if constexpr (EPI == EPI_SILU_MUL) {
    wcol[0] = nt * SW + CPL * li;
    wcol[1] = p.up_off + nt * SW + CPL * li;
    ocol0 = nt * SW + lg * NV;
  } else {
    wcol[0] = nt * 2 * SW + CPL * li;
    wcol[1] = wcol[0] + SW;
    ocol0 = nt * 2 * SW + lg * NV;
  }
  // EPI_STORE: the second slab of the last tile may lie past the output width
  const bool has_s1 = (EPI != EPI_STORE) || (ocol0 - lg * NV + SW < p.n_out);
  const char* wexp = reinterpret_cast<const char*>(p.w) + (int64_t)e * p.w_estride * Tr::ESIZE;
  const int64_t wrow_bytes = p.w_ld * Tr::ESIZE;
  constexpr int rows_per_lane = (WT == W_F32) ? 4 : 8;
  const bool vec_ok = (p.w_ld % CPL) == 0;
  const int krow_off = lg * rows_per_lane;

  const int kb = split * p.kchunk;
  const int ke = min(p.K, kb + p.kchunk);

  auto load_w = [&](int s, int k0) {
    Raw r;
    if (s == 1 && !has_s1) {
#pragma unroll
      for (int j = 0; j < rows_per_lane; ++j) r.r[j] = {};
      return r;
    }
    const char* base = wexp + (int64_t)(k0 + krow_off) * wrow_bytes;
#pragma unroll
    for (int j = 0; j < rows_per_lane; ++j)
      r.r[j] = load_wrow<WT, MASKED>(base + j * wrow_bytes, wcol[s], p.n_out, vec_ok);
    return r;
  };
  auto load_x = [&](int q, int k0) {
    u32x4 v = {0u, 0u, 0u, 0u};
    const int kk = k0 + (ACT == ACT_BF16 ? 8 : 4) * lg;
    if (rvalid[q]) v = ld16(arow[q] + (int64_t)kk * ASZ);
    return v;
  };

  f32x4 acc[2][2][CPL];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[s][q][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Raw (&w)[2], const u32x4 (&x)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s == 1 && !has_s1) continue;
      if constexpr (WT == W_F32) {
#pragma unroll
        for (int ss = 0; ss < 4; ++ss)
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float a = __uint_as_float(w[s].r[ss][c]);
            acc[s][0][c] = mfma_f32_16x16x4(a, __uint_as_float(x[0][ss]), acc[s][0][c]);
            if (use_q1) acc[s][1][c] = mfma_f32_16x16x4(a, __uint_as_float(x[1][ss]), acc[s][1][c]);
          }
      } else {
        u32x4 rows[8], frag[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (WT == W_FP8) rows[j] = fp8x8_to_bf16x8(w[s].r[j]);
          else rows[j] = w[s].r[j];
        }
        transpose8x8_b16(rows, frag);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          acc[s][0][c] = mfma_bf16_16x16x32(frag[c], x[0], acc[s][0][c]);
          if (use_q1) acc[s][1][c] = mfma_bf16_16x16x32(frag[c], x[1], acc[s][1][c]);
        }
      }
    }
  };

  {
    Raw cw[2] = {load_w(0, kb), load_w(1, kb)};
    u32x4 cx[2] = {load_x(0, kb), use_q1 ? load_x(1, kb) : u32x4{0u, 0u, 0u, 0u}};
    for (int k0 = kb; k0 < ke; k0 += KSTEP) {
      const int kn = min(k0 + KSTEP, ke - KSTEP);  // the last step reloads itself
      Raw nw[2] = {load_w(0, kn), load_w(1, kn)};
      u32x4 nx[2] = {load_x(0, kn), use_q1 ? load_x(1, kn) : u32x4{0u, 0u, 0u, 0u}};
      compute(cw, cx);
#pragma unroll
      for (int s = 0; s < 2; ++s) cw[s] = nw[s];
      cx[0] = nx[0];
      cx[1] = nx[1];
    }
  }

  // -------------------------------------------------------- split-K reduction
  if constexpr (EPI != EPI_F32) {
    if (p.ksplit > 1) {
      constexpr int NREG = 2 * 2 * CPL;  // f32x4 registers per lane
      const int64_t tile = (int64_t)mb * p.n_tiles + nt;
      float* part = p.partial + (tile * p.ksplit) * (NREG * 4 * WAVE);
      float* mine = part + (int64_t)split * (NREG * 4 * WAVE);
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (rvalid[q])
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const int reg = (s * 2 + q) * CPL + c;
              *reinterpret_cast<f32x4*>(mine + ((int64_t)reg * WAVE + lane) * 4) = acc[s][q][c];
            }
      __threadfence();
      int old = 0;
      if (lane == 0) old = atomicAdd(p.counters + tile, 1);
      old = __shfl(old, 0);
      if (old != p.ksplit - 1) return;
      __threadfence();
      f32x4 sum[2][2][CPL];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int c = 0; c < CPL; ++c) sum[s][q][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int sp = 0; sp < p.ksplit; ++sp) {
        const float* src = part + (int64_t)sp * (NREG * 4 * WAVE);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int q = 0; q < 2; ++q)
            if (rvalid[q])
#pragma unroll
              for (int c = 0; c < CPL; ++c) {
                const int reg = (s * 2 + q) * CPL + c;
                const f32x4 v = (sp == split)
                                    ? acc[s][q][c]
                                    : *reinterpret_cast<const f32x4*>(src + ((int64_t)reg * WAVE + lane) * 4);
                sum[s][q][c] += v;
              }
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[s][q][c] = sum[s][q][c];
      if (lane == 0) p.counters[tile] = 0;
    }
  }

  // -------------------------------------------------------- epilogue
  // Lane (li, lg) holds, per slab s and row group q, output columns
  // ocol0 + s*SW(+) + j for j = r*CPL + c in acc[s][q][c][r].
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (!rvalid[q]) continue;
    const int64_t prow = p0 + 16 * q + li;
    float v0[NV], v1[NV];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        v0[r * CPL + c] = acc[0][q][c][r];
        v1[r * CPL + c] = acc[1][q][c][r];
      }
    if constexpr (EPI == EPI_SILU_MUL) {
      if (WT == W_FP8) {
        const float* sg = p.scale + (int64_t)e * p.scale_estride + ocol0;
        const float* su = sg + p.up_off;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          v0[j] *= sg[j];
          v1[j] *= su[j];
        }
      }
      float h[NV];
#pragma unroll
      for (int j = 0; j < NV; ++j) h[j] = silu(v0[j]) * v1[j];
      char* dst = reinterpret_cast<char*>(p.out) + (prow * p.out_ld + ocol0) * ASZ;
      store_chunk<ACT>(dst, h, NV);
    } else if constexpr (EPI == EPI_STORE) {
      if (WT == W_FP8) {
        const float* sd = p.scale + (int64_t)e * p.scale_estride + ocol0;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          v0[j] *= sd[j];
          if (has_s1) v1[j] *= sd[SW + j];
        }
      }
      // per-slot expert outputs stay fp32: the combine sums them without a
      // second rounding before the output's own
      char* dst = reinterpret_cast<char*>(p.out) + (prow * p.out_ld + ocol0) * 4;
      store_chunk<ACT_F32>(dst, v0, NV);
      if (has_s1) store_chunk<ACT_F32>(dst + SW * 4, v1, NV);
    } else {
      float* dst = reinterpret_cast<float*>(p.out) + split * p.out_split_stride + prow * p.out_ld;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        if (ocol0 + j < p.n_out) dst[ocol0 + j] = v0[j];
        if (ocol0 + SW + j < p.n_out) dst[ocol0 + SW + j] = v1[j];
      }
    }
  }
}

int stream_tile_cols(int w_dtype, int epi) {
  const int sw = (w_dtype == W_F32) ? SlabW<W_F32>::value : SlabW<W_BF16>::value;
  return epi == EPI_SILU_MUL ? sw : 2 * sw;
}

int stream_kstep(int w_dtype) {
  return (w_dtype == W_F32) ? WTr<W_F32>::KSTEP : WTr<W_BF16>::KSTEP;
}

int64_t stream_partial_floats_per_tile_split(int w_dtype) {
  const int cpl = (w_dtype == W_F32) ? WTr<W_F32>::CPL : WTr<W_BF16>::CPL;
  return (int64_t)2 * 2 * cpl * 4 * WAVE;
}

template <int ACT, int WT, int EPI>
static hipError_t launch_one(const StreamGemmArgs& a, hipStream_t st) {
  const int64_t grid = (int64_t)a.num_mblocks * a.n_tiles * a.ksplit;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_stream_gemm<ACT, WT, EPI>), dim3((unsigned)grid), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_stream_gemm(int act, int wdt, int epi, const StreamGemmArgs& a, hipStream_t st) {
#define MOE_CASE(A_, W_, E_) \
  if (act == A_ && wdt == W_ && epi == E_) return launch_one<A_, W_, E_>(a, st);
  MOE_CASE(ACT_F32, W_F32, EPI_SILU_MUL)
  MOE_CASE(ACT_F32, W_F32, EPI_STORE)
  MOE_CASE(ACT_F32, W_F32, EPI_F32)
  MOE_CASE(ACT_BF16, W_BF16, EPI_SILU_MUL)
  MOE_CASE(ACT_BF16, W_BF16, EPI_STORE)
  MOE_CASE(ACT_BF16, W_BF16, EPI_F32)
  MOE_CASE(ACT_BF16, W_FP8, EPI_SILU_MUL)
  MOE_CASE(ACT_BF16, W_FP8, EPI_STORE)
#undef MOE_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
