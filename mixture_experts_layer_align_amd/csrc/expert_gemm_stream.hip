// Weight-streaming grouped expert GEMM for thin token blocks (decode regime).
//
// Expert compute is A[M,K] x B[K,N] -> C[M,N] with M token rows, K the hidden
// size and N the expert's output width (vLLM fused-MoE post, section
// "Swap-AB"); B is the expert weight stored [K, N], N contiguous.  With few
// rows per expert the cost is streaming B from HBM once (the decode case of
// "CuTeDSL at Perplexity", section on prefill and decode: DRAM loads of
// weights dominate).  The pages' Hopper answer is to swap operands so the
// large N fills the fixed 64-row side of the tensor-core instruction.  The
// gfx950 version of that idea:
//
//   * the weight panel is the MFMA A operand (rows = output columns n) and the
//     tokens the B operand (columns = rows of the block), so
//     v_mfma_f32_16x16x32_bf16 produces 16 output columns x 16 tokens;
//   * a workgroup owns (32-row block of one expert, n-tile, k-range); each of
//     its two waves streams one slab of the tile (for gate|up: the gate slab
//     and the matching up slab), applying every weight fragment to all rows of
//     the block (weight-stationary); a 16-row group with no routed row is
//     skipped;
//   * weights go HBM -> LDS with direct loads (global_load_lds_dwordx4: no
//     VGPR holds data in flight) through a ring of 8 KB stages per wave (two
//     for bf16, four for fp8);
//     each lane reads back exactly the 16-byte chunks it requested (8
//     consecutive weight rows, 16 lanes covering 256 contiguous bytes of a row)
//     and transposes its 8x8 bf16 block in registers (v_perm_b32) into 8 MFMA A
//     fragments; the wait before each stage is an explicit vmcnt that leaves
//     the later stages in flight;
//   * tokens are gathered straight from x by the aligned slot list, so the
//     permuted activations are never materialised (the pages copy tokens into
//     padded per-expert buffers first: "CuTeDSL at Perplexity", MoE dispatch
//     and combine, local kernel);
//   * bf16 weights with more items than compute units: a persistent grid of
//     at most one workgroup per compute unit, each taking an equal share of
//     whole items (measured faster than one workgroup per item);
//   * when blocks x n-tiles cannot fill the chip, K is split: each split stores
//     fp32 partial sums and the next kernel adds them in split order (fixed
//     order, no atomics, no device-scope fences: on gfx950 a device-scope
//     fence writes back and invalidates the XCD's L2, which hundreds of
//     workgroups streaming through that L2 cannot afford).  For a split
//     gate|up that next kernel is the down GEMM itself: each of its items
//     first adds the partials of its rows and k-range and applies SiLU*up
//     (one launch fewer; the prologue lengthens the down kernel by 3-5 µs,
//     about what a separate reduce launch and its gap cost);
//   * the epilogue runs on the fp32 accumulators before the single store:
//     SiLU(gate) * up for the concatenated gate|up weight ("La fusion de
//     noyaux", section 4.2, GEMM + epilogue and the SwiGLU concatenation), and
//     the fp8 per-column scale, applied after the dot product.  h is stored in
//     the activation dtype (its rounding errors average out over the down
//     GEMM's K); the down GEMM's per-slot outputs are stored in fp32, because
//     each output element adds k of them directly and a bf16 rounding there
//     would stack on the output's own.
//
// fp8 (OCP e4m3fn) and MXFP8 weights: a lane loads 16 codes of each of its 8
// k-rows (slabs of 256 columns); byte permutes pair each column's codes of
// two consecutive k-rows and one conversion per pair gives the column's bf16
// operand word (MXFP8: scaled by the column's E8M0 block scale, exactly), so
// no bf16 transpose is needed; the same bf16 MFMA runs (activations stay
// bf16).  MXFP4: see its trait below.  fp32 weights: 4 columns per lane, no
// transpose, v_mfma_f32_16x16x4_f32.
#include <algorithm>
#include <type_traits>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

template <int WT>
struct DTr;
template <>
struct DTr<W_BF16> {
  static constexpr int CPL = 8;     // weight columns per lane
  static constexpr int RPL = 8;     // weight rows per lane per k-step (one 16 B load each)
  static constexpr int KSTEP = 32;
  static constexpr int ESIZE = 2;
};
template <>
struct DTr<W_FP8> {
  static constexpr int CPL = 16;
  static constexpr int RPL = 8;
  static constexpr int KSTEP = 32;
  static constexpr int ESIZE = 1;
};
// MXFP4: one 16-byte load holds two k-rows (a packed byte per column) of 16
// columns, so 4 loads cover the lane's 8 k-rows; converted, byte c of the 4
// loads is directly the 8 consecutive-k bf16 operand of column c (no
// transpose), scaled by that column's E8M0 block scale during the conversion.
template <>
struct DTr<W_FP4> {
  static constexpr int CPL = 16;
  static constexpr int RPL = 4;
  static constexpr int KSTEP = 32;  // = the MX block: one scale per column per k-step
  static constexpr int ESIZE = 1;   // (bytes per packed row pair and column)
};
// MXFP8: fp8's shape; one E8M0 scale per column per k-step (= the MX block)
template <>
struct DTr<W_MXFP8> : DTr<W_FP8> {};
template <>
struct DTr<W_F32> {
  static constexpr int CPL = 4;
  static constexpr int RPL = 4;
  static constexpr int KSTEP = 16;
  static constexpr int ESIZE = 4;
};

#ifndef STREAM_HV2_STAGES
#define STREAM_HV2_STAGES 8
#endif
// Load-ring stages per wave.  bf16: two — with fewer requests outstanding
// HBM serves the weight stream faster (more stages measured slower on gfx950).
// fp8: four — its heavier per-stage math needs the deeper ring, and the
// larger LDS footprint keeps two workgroups per compute unit.  MXFP4: eight
// stages of 4 KB (the same bytes in flight as fp8; with four its waves spent
// half their time waiting for loads).
//
// Two-half blocks (HV = 2) use more than 256 registers per wave, so one
// workgroup runs per compute unit: eight stages (128 KB) keep as many weight
// bytes in flight per unit as two one-half workgroups with four each.
template <int WT, int HV = 1>
constexpr int stages_of() {
  return HV == 2 ? STREAM_HV2_STAGES : WT == W_BF16 ? 2 : WT == W_FP4 ? 8 : 4;  // fp8, MXFP8: 4
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory
// operations of this wave are outstanding; LDS/scalar and export counters are
// left alone.
constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14);
}

// Two E2M1 codes (byte `sel` of src: low nibble -> low half) to two bf16,
// times `scale` (exact for the power-of-two MX scales).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t src, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scale, SEL));
}
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t src, float scale, int sel) {
  switch (sel) {  // sel is a constant after unrolling
    case 0: return fp4x2_to_bf16x2<0>(src, scale);
    case 1: return fp4x2_to_bf16x2<1>(src, scale);
    case 2: return fp4x2_to_bf16x2<2>(src, scale);
    default: return fp4x2_to_bf16x2<3>(src, scale);
  }
}

// Two e4m3fn codes (bytes 2*HI, 2*HI+1 of src) to two bf16, times `scale`.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t src, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, scale, HI));
}

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

}  // namespace

// h[p, k] = SiLU(sum_s g_s[p, k]) * sum_s u_s[p, k] for the routed rows p of
// the 32 rows at p0 (bit r of `routed`: row p0 + r) and k in [kb, ke), splits
// added in order, from the gate|up k-split partial sums; stored where the
// item's main loop reads its rows (as a bf16 pair when HILO).  The 128
// threads of those rows (tid 0-127) take part: 8 consecutive columns of one routed row per thread and
// pass, the loads of up to FOLD_SPLITS splits in flight at once (the partials
// come from other dies' L2 or HBM: one round trip per group of splits).  The
// workgroups of the block's other n-tiles write the same values to the same
// places.
constexpr int FOLD_SPLITS = 8;
template <int ACT, bool HILO>
__device__ __forceinline__ void fold_split_silu(const StreamGemmArgs& p, uint32_t routed, int p0,
                                                int kb, int ke, int tid) {
  constexpr int ASZ = (ACT == ACT_BF16) ? 2 : 4;
  const int K = p.K;  // gate|up's d_ff: up columns start at K
  const int per_row = (ke - kb) / 8;
  for (int u = tid; u < STREAM_BM * per_row; u += 128) {
    const int r = u / per_row;
    if (!((routed >> r) & 1u)) continue;
    const int c = kb + 8 * (u - r * per_row);
    const int64_t prow = p0 + r;
    float g[8], v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = v[j] = 0.f;
    const float* row = p.a_part + prow * p.a_part_ld + c;
    for (int s0 = 0; s0 < p.a_part_nsplit; s0 += FOLD_SPLITS) {
      u32x4 ld[FOLD_SPLITS][4];
#pragma unroll
      for (int i = 0; i < FOLD_SPLITS; ++i) {
        if (s0 + i < p.a_part_nsplit) {
          const float* src = row + (int64_t)(s0 + i) * p.a_part_stride;
          ld[i][0] = ld16(src);
          ld[i][1] = ld16(src + 4);
          ld[i][2] = ld16(src + K);
          ld[i][3] = ld16(src + K + 4);
        }
      }
#pragma unroll
      for (int i = 0; i < FOLD_SPLITS; ++i) {
        if (s0 + i < p.a_part_nsplit) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            g[j] += __uint_as_float(ld[i][0][j]);
            g[4 + j] += __uint_as_float(ld[i][1][j]);
            v[j] += __uint_as_float(ld[i][2][j]);
            v[4 + j] += __uint_as_float(ld[i][3][j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = silu(g[j]) * v[j];
    char* dst = const_cast<char*>(reinterpret_cast<const char*>(p.a)) + (prow * p.a_ld + c) * ASZ;
    if constexpr (HILO)
      store_bf16_pair<8>(dst, const_cast<char*>(reinterpret_cast<const char*>(p.a_lo)) +
                                  (prow * p.a_ld + c) * 2,
                         v);
    else
      store_act<ACT>(dst, v, 8);
  }
}

// One item = (block, n-tile, k-split) of the launch.  HILO: the token
// rows come as bf16 pairs (p.a high halves, p.a_lo low halves) and every
// weight fragment is applied to both, which carries h into the down GEMM at
// 16 significant bits instead of 8.
//
// HV = 1: one 32-row block per item, two waves (one per slab), each wave
// with a load ring of its own and no workgroup barrier in the k-loop.  HV = 2
// (gate|up with fp8 weights): a pair of consecutive blocks of one expert per
// item, four waves; wave (slab, blk) applies its slab's weights to the rows
// of block `blk` of the pair.  The two waves of a slab share one ring: each
// issues half of every stage's weight rows (the same lane addresses either
// would use), and one workgroup barrier per k-step, after each wave's own
// vmcnt wait, publishes the landed stage and retires the stage read in the
// previous step, which is then refilled.  An expert's weights then stream
// once per two blocks; a half with no routed row loads only its share of the
// weights.
template <int ACT, int WT, int EPI, bool HILO, int HV>
__device__ __forceinline__ void stream_item(const StreamGemmArgs& p, int id, u32x4* lds) {
  using Tr = DTr<WT>;
  constexpr int CPL = Tr::CPL;
  constexpr int RPL = Tr::RPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int SW = 16 * CPL;    // slab width (weight columns per wave)
  constexpr int NV = 4 * CPL;     // contiguous output columns per lane
  constexpr int ASZ = (ACT == ACT_BF16) ? 2 : 4;
  constexpr int XK = (ACT == ACT_BF16) ? 8 : 4;  // k-values per lane per token fragment
  constexpr int S = stages_of<WT, HV>();
  constexpr bool MX = WT == W_FP4 || WT == W_MXFP8;  // E8M0 block scales
  constexpr bool PACK = WT == W_FP4;                  // two codes per byte along K
  static_assert(!HILO || (ACT == ACT_BF16 && WT != W_F32), "bf16 pairs");
  static_assert(HV == 1 || HV == 2, "one or two 32-row halves");
  static_assert(RPL % HV == 0, "the halves split a stage's weight rows");
  constexpr int RPW = RPL / HV;  // weight rows this wave loads per stage
  // vector-memory ops per stage: the wave's weight rows + 2 token loads (4
  // with HILO) (+ the MX scales)
  constexpr int PER = RPW + (HILO ? 4 : 2) + (MX ? 1 : 0);
  static_assert((S - 1) * PER <= 63, "vmcnt field");
  // (a loop whose second row group is known empty issues one token load
  // fewer per stage, two with HILO, and counts accordingly)
  static_assert(HV == 1 || S >= 3, "a shared ring keeps a stage in flight past the barrier");

  const int lane = threadIdx.x & 63;
  const int slab = HV == 1 ? (int)(threadIdx.x >> 6) : (int)(threadIdx.x >> 6) & 1;
  const int blk = HV == 1 ? 0 : (int)(threadIdx.x >> 7);  // block of the pair
  const int li = lane & 15;  // MFMA column within a 16-group (token row)
  const int lg = lane >> 4;  // k group

  const int split = id % p.ksplit;
  id /= p.ksplit;
  const int nt = id % p.n_tiles;
  const int mb = id / p.n_tiles;
  const int e = p.block_expert[mb];
  if (e < 0) return;  // whole workgroup: a block past the routed rows
  // HV = 2: the expert's blocks pair up from its first one; the item of a
  // pair's second block returns (the first covers it), and a last block
  // without a partner leaves the second half empty
  bool half_ok = true;
  if constexpr (HV == 2) {
    const int first = p.expert_offsets[e] / STREAM_BM;
    if ((mb - first) & 1) return;  // whole workgroup
    half_ok = blk == 0 || mb + 1 < p.expert_offsets[e + 1] / STREAM_BM;
  }
  const int p0 = (mb + blk) * STREAM_BM;

  // -------------------------------------------------------- token rows
  const char* arow[2];
  const char* alrow[2];  // HILO: the rows' low halves
  bool rvalid[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int prow = p0 + 16 * q + li;
    const int sid = half_ok ? p.sorted_ids[prow] : -1;
    rvalid[q] = sid >= 0;
    int64_t src = 0;  // invalid rows read row 0 (in bounds) and are zeroed
    if (rvalid[q]) src = (p.a_mode == A_GATHER) ? sid / p.topk : prow;
    arow[q] = reinterpret_cast<const char*>(p.a) + src * p.a_ld * ASZ;
    alrow[q] = HILO ? reinterpret_cast<const char*>(p.a_lo) + src * p.a_ld * ASZ : nullptr;
  }
  const bool use_q1 = ballot(rvalid[1]) != 0;
  // the half has a routed row (its row 0 is then one: an expert's routed
  // slots come first in its range); one half: always
  const bool live = HV == 1 || ballot(rvalid[0]) != 0;

  // -------------------------------------------------------- weight columns
  int wcol, ocol;  // this lane's first weight column; first output column
  if constexpr (EPI == EPI_SILU_MUL) {
    wcol = (slab ? p.up_off : 0) + nt * SW + CPL * li;
    ocol = nt * SW + lg * NV;
  } else {
    wcol = nt * 2 * SW + slab * SW + CPL * li;
    ocol = nt * 2 * SW + slab * SW + lg * NV;
  }
  // the second slab of the last down tile may lie past the output width
  const bool active = (EPI != EPI_STORE) || (nt * 2 * SW + slab * SW < p.n_out);
  // bytes between consecutive weight rows (MXFP4: packed row pairs) and per k-step
  const int64_t wrow_bytes = p.w_ld * Tr::ESIZE;
  const int64_t kstep_bytes = (PACK ? KSTEP / 2 : KSTEP) * wrow_bytes;
  const int kb = split * p.kchunk;
  const int ke = min(p.K, kb + p.kchunk);
  const int nsteps = (ke - kb) / KSTEP;
  const char* wbase =
      PACK ? reinterpret_cast<const char*>(p.w) + (int64_t)e * (p.w_estride / 2) +
               (int64_t)(kb / 2 + lg * RPL) * wrow_bytes + wcol
         : reinterpret_cast<const char*>(p.w) + (int64_t)e * p.w_estride * Tr::ESIZE +
               (int64_t)(kb + lg * RPL) * wrow_bytes + (int64_t)wcol * Tr::ESIZE;
  // MX: the E8M0 scales of the lane's 16 columns for the k-step's block
  const char* sbase = MX ? reinterpret_cast<const char*>(p.scale) + (int64_t)e * p.scale_estride +
                               (int64_t)(kb / KSTEP) * p.w_ld + wcol
                         : nullptr;
  // MX weights: the stage's E8M0 scales come through the ring as one more
  // row (with HV = 2 both waves of a live pair load the same bytes to the
  // same place); register-loaded scales made the compiler drain every load
  // (vmcnt(0)) before their use once per pass of the unrolled loop
  constexpr bool MXL = MX;
  constexpr int RPR = RPL + (MXL ? 1 : 0);  // ring rows per stage
  u32x4* ring = lds + slab * S * RPR * WAVE;
  if constexpr (EPI == EPI_STORE) {
    if (p.a_part != nullptr) {  // uniform
      // lanes 0-15 hold rows 0-15 (q = 0) and 16-31 (q = 1)
      const uint32_t routed = (uint32_t)(ballot(rvalid[0]) & 0xFFFFu) |
                              ((uint32_t)(ballot(rvalid[1]) & 0xFFFFu) << 16);
      fold_split_silu<ACT, HILO>(p, routed, p0, kb, ke, (int)(threadIdx.x & 127));
      __syncthreads();  // h of the item's rows and k-range is in place
    }
  }

  f32x4 acc[2][CPL];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[q][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  static_assert(HV == 1 || EPI == EPI_SILU_MUL, "two halves: gate|up, whose slabs are all active");
  if (active && nsteps > 0) {
    u32x4 xb[S][2];
    u32x4 xl[HILO ? S : 1][2];
    // stage s <- k-step `step` (clamped: steps past the end reload the last);
    // tok (a std::bool_constant): also the wave's token rows (and MX scales),
    // which an empty half does not load; q1 (std::false_type: the second
    // 16-row group is known empty): not its token row — the compiler drops
    // that load anyway once nothing reads it, and the wait counts must then
    // not count it
    auto issue = [&](int s, int step, auto tok, auto q1) {
      const int sc = min(step, nsteps - 1);
      const char* src = wbase + (int64_t)sc * kstep_bytes;
#pragma unroll
      for (int jw = 0; jw < RPW; ++jw) {
        const int j = jw * HV + blk;
        dma16(src + j * wrow_bytes, ring + (s * RPR + j) * WAVE);
      }
      if constexpr (!decltype(tok)::value) return;
      const int64_t kk = (int64_t)(kb + sc * KSTEP + XK * lg) * ASZ;
      constexpr bool Q1 = !std::is_same_v<decltype(q1), std::false_type>;
      xb[s][0] = ld16(arow[0] + kk);
      if constexpr (Q1) xb[s][1] = ld16(arow[1] + kk);
      if constexpr (HILO) {
        xl[s][0] = ld16(alrow[0] + kk);
        if constexpr (Q1) xl[s][1] = ld16(alrow[1] + kk);
      }
      if constexpr (MXL) dma16(sbase + (int64_t)sc * p.w_ld, ring + (s * RPR + RPL) * WAVE);
    };
    // q1: the block's second 16-row group holds routed rows — a runtime bool
    // (a branch per MFMA) or, for MXFP4, std::true_type/false_type (folded)
    auto compute = [&](int s, auto q1) {
      u32x4 raw[RPL];
#pragma unroll
      for (int j = 0; j < RPL; ++j) raw[j] = ring[(s * RPR + j) * WAVE + lane];
      // MX: the lane's 16 E8M0 scale bytes of the k-step
      u32x4 msc = {0u, 0u, 0u, 0u};
      if constexpr (MXL) msc = ring[(s * RPR + RPL) * WAVE + lane];
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 x0 = rvalid[0] ? xb[s][0] : z;
      const u32x4 x1 = rvalid[1] ? xb[s][1] : z;
      const u32x4 x0l = (HILO && rvalid[0]) ? xl[HILO ? s : 0][0] : z;
      const u32x4 x1l = (HILO && rvalid[1]) ? xl[HILO ? s : 0][1] : z;
      // the 8 fragments' products with the high halves, then (HILO) with the
      // low halves, so consecutive MFMAs use different accumulators
      auto mm8 = [&](const u32x4 (&f)[8], int c0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          acc[0][c0 + c] = mfma_bf16_16x16x32(f[c], x0, acc[0][c0 + c]);
          if (q1) acc[1][c0 + c] = mfma_bf16_16x16x32(f[c], x1, acc[1][c0 + c]);
        }
        if constexpr (HILO) {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            acc[0][c0 + c] = mfma_bf16_16x16x32(f[c], x0l, acc[0][c0 + c]);
            if (q1) acc[1][c0 + c] = mfma_bf16_16x16x32(f[c], x1l, acc[1][c0 + c]);
          }
        }
      };
      if constexpr (WT == W_F32) {
#pragma unroll
        for (int ss = 0; ss < 4; ++ss)
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float a = __uint_as_float(raw[ss][c]);
            acc[0][c] = mfma_f32_16x16x4(a, __uint_as_float(x0[ss]), acc[0][c]);
            if (q1) acc[1][c] = mfma_f32_16x16x4(a, __uint_as_float(x1[ss]), acc[1][c]);
          }
      } else if constexpr (WT == W_BF16) {
        u32x4 frag[8];
        transpose8x8_b16(raw, frag);
        mm8(frag, 0);
      } else if constexpr (WT == W_FP4) {
        // E8M0 byte e of column c -> the fp32 2^(e-127) (exponent field e,
        // zero mantissa)
        auto scl_of = [&](int c) {
          return __uint_as_float(((msc[c >> 2] >> (8 * (c & 3))) & 0xFFu) << 23);
        };
        if constexpr (!HILO) {
          // one fragment at a time (fewest live registers)
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float scl = scl_of(c);
            u32x4 frag;
#pragma unroll
            for (int j = 0; j < 4; ++j) frag[j] = fp4x2_to_bf16x2(raw[j][c >> 2], scl, c & 3);
            acc[0][c] = mfma_bf16_16x16x32(frag, x0, acc[0][c]);
            if (q1) acc[1][c] = mfma_bf16_16x16x32(frag, x1, acc[1][c]);
          }
        } else {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 frag[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const int cc = 8 * half + c;
              const float scl = scl_of(cc);
#pragma unroll
              for (int j = 0; j < 4; ++j)
                frag[c][j] = fp4x2_to_bf16x2(raw[j][cc >> 2], scl, cc & 3);
            }
            mm8(frag, 8 * half);
          }
        }
      } else {
        // fp8 / MXFP8 codes, raw[j] = k-row j of the lane's 16 columns: a
        // byte permute pairs the two consecutive-k bytes of two columns, and
        // each pair converts to the column's bf16 operand word — with the
        // column's E8M0 block scale for MXFP8 (exact: a power of two), 1 for
        // fp8 (its per-column scale multiplies the fp32 sums later)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 frag[8];
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              const uint32_t a = raw[2 * m][2 * half + w], b = raw[2 * m + 1][2 * half + w];
              const uint32_t u01 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // cols 0, 1
              const uint32_t u23 = __builtin_amdgcn_perm(b, a, 0x07030602u);  // cols 2, 3
              // the lane's columns 8*half + 4*w + c; MXFP8: their E8M0 bytes,
              // as the fp32 2^(e-127) (exponent field e, zero mantissa)
              float scl[4] = {1.0f, 1.0f, 1.0f, 1.0f};
              if constexpr (WT == W_MXFP8) {
                const uint32_t sw = msc[2 * half + w];
#pragma unroll
                for (int c = 0; c < 4; ++c) scl[c] = __uint_as_float(((sw >> (8 * c)) & 0xFFu) << 23);
              }
              frag[4 * w + 0][m] = fp8x2_to_bf16x2<false>(u01, scl[0]);
              frag[4 * w + 1][m] = fp8x2_to_bf16x2<true>(u01, scl[1]);
              frag[4 * w + 2][m] = fp8x2_to_bf16x2<false>(u23, scl[2]);
              frag[4 * w + 3][m] = fp8x2_to_bf16x2<true>(u23, scl[3]);
            }
          mm8(frag, 8 * half);
        }
      }
    };
    const std::true_type tok;
    // The first S-1 stages are loaded up front.  Step j: this wave's share
    // of stage j % S has landed once at most the S-2 stages issued after it
    // are in flight (steps up to j+S-2); after the barrier every share has,
    // and every wave is done reading the stage of step j-1 (at j = 0: the
    // stage not yet loaded), which is loaded with step j+S-1 before stage j
    // is computed.  Every wave runs every barrier; live_c (a bool_constant):
    // the half has routed rows (else the wave only loads its weight share,
    // so its wait counts those alone).
    auto loop2 = [&](auto q1_c, auto live_c) {
      constexpr bool LIVE = decltype(live_c)::value;
      constexpr int P =
          LIVE ? PER - (std::is_same_v<decltype(q1_c), std::false_type> ? (HILO ? 2 : 1) : 0) : RPW;
#pragma unroll
      for (int s = 0; s < S - 1; ++s) issue(s, s, live_c, q1_c);
      for (int it = 0; it < nsteps; it += S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * P));
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          issue((s + S - 1) % S, it + s + S - 1, live_c, q1_c);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (LIVE) {
            if (it + s < nsteps) compute(s, q1_c);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    auto main_loop = [&](auto q1_c) {
      if constexpr (HV == 1) {
        constexpr int P =
            PER - (std::is_same_v<decltype(q1_c), std::false_type> ? (HILO ? 2 : 1) : 0);
        // the first S stages, with the loop's own loads (a load the loop
        // never reads would have to be drained before its register is reused)
#pragma unroll
        for (int s = 0; s < S; ++s) issue(s, s, tok, q1_c);
        for (int it = 0; it < nsteps; it += S) {
#pragma unroll
          for (int s = 0; s < S; ++s) {
            // stage s complete: only the S-1 later stages may still be in flight
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 1) * P));
            __builtin_amdgcn_sched_barrier(0);
            if (it + s < nsteps) compute(s, q1_c);
            __builtin_amdgcn_sched_barrier(0);
            issue(s, it + s + S, tok, q1_c);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
        if (live)
          loop2(q1_c, std::true_type{});
        else
          loop2(q1_c, std::false_type{});
      }
    };
    // MXFP4 gains from one loop per case (its many conversions leave no issue
    // slots for the branches); bf16 measured slower with two loop copies
    if constexpr (WT == W_FP4) {
      if (use_q1)
        main_loop(std::true_type{});
      else
        main_loop(std::false_type{});
    } else {
      main_loop(use_q1);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  __syncthreads();  // the ring is free from here on

  // -------------------------------------------------------- split-K partials
  // With several k-splits each split stores its (scaled) fp32 sums for the
  // routed rows; a later kernel adds the splits in split order (for gate|up
  // the down GEMM, whose items first form h from them; for down the
  // combine).  The kernel boundary orders the stores before those reads, so
  // no device-scope fence or atomic is needed here.
  if (p.ksplit > 1) {
    if (!active) return;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!rvalid[q]) continue;
      const int64_t prow = p0 + 16 * q + li;
      // column in the weight's N space (gate|up: [0, 2*d_ff); down: [0, d))
      const int col = (EPI == EPI_SILU_MUL) ? (slab ? p.up_off : 0) + ocol : ocol;
      float v[NV];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[r * CPL + c] = acc[q][c][r];
      if (WT == W_FP8) {
        const float* sc = p.scale + (int64_t)e * p.scale_estride + col;
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] *= sc[j];
      }
      char* dst = reinterpret_cast<char*>(p.partial) +
                  ((int64_t)split * p.partial_split_stride + prow * p.partial_ld + col) * 4;
      store_act<ACT_F32>(dst, v, NV);
    }
    return;
  }

  // -------------------------------------------------------- epilogue
  // Lane (li, lg) holds, for row group q, output columns ocol + j with
  // j = r*CPL + c in acc[q][c][r].
  if constexpr (EPI == EPI_SILU_MUL) {
    if (WT == W_FP8) {
      const float* sc = p.scale + (int64_t)e * p.scale_estride + (slab ? p.up_off : 0) + ocol;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float f = sc[r * CPL + c];
          acc[0][c][r] *= f;
          acc[1][c][r] *= f;
        }
    }
    // wave 0 (gate) finishes row group 0 and wave 1 (up) row group 1; each
    // hands the other the accumulators of the group it does not finish
    // (selects, not indexing by the wave number, keep acc in registers)
    f32x4* xch = reinterpret_cast<f32x4*>(lds) + blk * 2 * CPL * WAVE;  // [HV][2][CPL][WAVE]
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      // selects of values (copies), not of the two array elements: a select
      // of element addresses made the compiler keep acc in private memory
      const f32x4 a0 = acc[0][c], a1 = acc[1][c];
      xch[(slab * CPL + c) * WAVE + lane] = slab ? a0 : a1;
    }
    __syncthreads();
    const int keep = slab;
    if (!rvalid[keep]) return;
    const int64_t prow = p0 + 16 * keep + li;
    float h[NV];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const f32x4 a0 = acc[0][c], a1 = acc[1][c];
      const f32x4 mine = slab ? a1 : a0;
      const f32x4 other = xch[((1 - slab) * CPL + c) * WAVE + lane];
      const f32x4 g = slab ? other : mine;
      const f32x4 u = slab ? mine : other;
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r * CPL + c] = silu(g[r]) * u[r];
    }
    char* dst = reinterpret_cast<char*>(p.out) + (prow * p.out_ld + ocol) * ASZ;
    if (ACT == ACT_BF16 && p.out_lo != nullptr)
      store_bf16_pair<NV>(dst, reinterpret_cast<char*>(p.out_lo) + (prow * p.out_ld + ocol) * 2,
                          h);
    else
      store_act<ACT>(dst, h, NV);
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!active || !rvalid[q]) continue;
      const int64_t prow = p0 + 16 * q + li;
      float v[NV];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[r * CPL + c] = acc[q][c][r];
      if (WT == W_FP8) {
        const float* sd = p.scale + (int64_t)e * p.scale_estride + ocol;
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] *= sd[j];
      }
      // per-slot expert outputs stay fp32
      char* dst = reinterpret_cast<char*>(p.out) + (prow * p.out_ld + ocol) * 4;
      store_act<ACT_F32>(dst, v, NV);
    }
  }
}

// Workgroup g takes items g, g + gridDim.x, ...: with as many workgroups as
// compute units and an equal share each, the weight stream runs with one
// front per expert group and no partly filled last round.  Items are numbered
// n-tile fastest, so the blocks in use (a prefix of the m-blocks) make a
// prefix of the items.
template <int ACT, int WT, int EPI, bool HILO, int HV>
__global__ __launch_bounds__(128 * HV) void k_expert_stream(const StreamGemmArgs p) {
  // ring[slab][stage][row][lane]; after an item's main loop the same memory
  // holds its epilogue exchange
  constexpr bool MXL = WT == W_FP4 || WT == W_MXFP8;
  constexpr int RING = 2 * stages_of<WT, HV>() * (DTr<WT>::RPL + (MXL ? 1 : 0)) * WAVE;
  static_assert(EPI != EPI_SILU_MUL || HV * 2 * DTr<WT>::CPL * WAVE <= RING,
                "the epilogue exchange fits the ring");
  __shared__ u32x4 lds[RING];
  int blocks = p.num_mblocks;
  if (p.padded_rows != nullptr) blocks = min(blocks, *p.padded_rows / STREAM_BM);
  const int items = blocks * p.n_tiles * p.ksplit;
  for (int i = blockIdx.x; i < items; i += gridDim.x) {
    __syncthreads();  // the previous item's epilogue is done with the ring
    stream_item<ACT, WT, EPI, HILO, HV>(p, i, lds);
  }
}

int stream_tile_cols(int w_dtype, int epi) {
  const int sw = 16 * (w_dtype == W_F32     ? DTr<W_F32>::CPL
                       : w_dtype == W_FP8   ? DTr<W_FP8>::CPL
                       : w_dtype == W_MXFP8 ? DTr<W_MXFP8>::CPL
                       : w_dtype == W_FP4   ? DTr<W_FP4>::CPL
                                            : DTr<W_BF16>::CPL);
  return epi == EPI_SILU_MUL ? sw : 2 * sw;
}

int stream_kstep(int w_dtype) {
  return (w_dtype == W_F32) ? DTr<W_F32>::KSTEP : DTr<W_BF16>::KSTEP;
}

template <int ACT, int WT, int EPI, int HV>
static hipError_t launch_hv(const StreamGemmArgs& a, int64_t grid, hipStream_t st) {
  if constexpr (ACT == ACT_BF16 && WT != W_F32 && EPI == EPI_STORE) {
    if (a.a_lo != nullptr) {
      hipLaunchKernelGGL((k_expert_stream<ACT, WT, EPI, true, HV>), dim3((unsigned)grid),
                         dim3(128 * HV), 0, st, a);
      return hipGetLastError();
    }
  } else {
    if (a.a_lo != nullptr) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((k_expert_stream<ACT, WT, EPI, false, HV>), dim3((unsigned)grid),
                     dim3(128 * HV), 0, st, a);
  return hipGetLastError();
}

// block pairs for fp8 weights (MXFP8 and MXFP4 pairs measured slower at
// E=256 top-8 T=128: gate|up 484 -> 504 and 264 -> 341 us)
template <int WT>
constexpr bool has_halves() {
  return WT == W_FP8;
}

template <int ACT, int WT, int EPI>
static hipError_t launch_one(const StreamGemmArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.num_mblocks * a.n_tiles * a.ksplit;
  if (items <= 0) return hipSuccess;
  if (items > 0x7FFFFFFF || a.wgs < 0) return hipErrorInvalidValue;
  const int64_t grid = a.wgs > 0 ? std::min<int64_t>(a.wgs, items) : items;
  if (a.halves == 2) {
    // gate|up only (every slab of its n-tiles lies inside the output, so
    // every wave runs the k-loop's barriers)
    if (a.expert_offsets == nullptr || a.block_expert == nullptr) return hipErrorInvalidValue;
    if constexpr (ACT == ACT_BF16 && has_halves<WT>() && EPI == EPI_SILU_MUL)
      return launch_hv<ACT, WT, EPI, 2>(a, grid, st);
    return hipErrorInvalidValue;
  }
  if (a.halves > 2) return hipErrorInvalidValue;
  return launch_hv<ACT, WT, EPI, 1>(a, grid, st);
}

hipError_t launch_stream_gemm(int act, int wdt, int epi, const StreamGemmArgs& a, hipStream_t st) {
#define MOE_CASE(A_, W_, E_) \
  if (act == A_ && wdt == W_ && epi == E_) return launch_one<A_, W_, E_>(a, st);
  MOE_CASE(ACT_F32, W_F32, EPI_SILU_MUL)
  MOE_CASE(ACT_F32, W_F32, EPI_STORE)
  MOE_CASE(ACT_BF16, W_BF16, EPI_SILU_MUL)
  MOE_CASE(ACT_BF16, W_BF16, EPI_STORE)
  MOE_CASE(ACT_BF16, W_FP8, EPI_SILU_MUL)
  MOE_CASE(ACT_BF16, W_FP8, EPI_STORE)
  MOE_CASE(ACT_BF16, W_FP4, EPI_SILU_MUL)
  MOE_CASE(ACT_BF16, W_FP4, EPI_STORE)
  MOE_CASE(ACT_BF16, W_MXFP8, EPI_SILU_MUL)
  MOE_CASE(ACT_BF16, W_MXFP8, EPI_STORE)
#undef MOE_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
