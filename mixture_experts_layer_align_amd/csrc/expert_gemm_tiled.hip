// LDS-tiled grouped expert GEMM for thick token blocks (prefill regime).
//
// With many rows per expert the expert GEMMs are bound by the matrix cores
// ("CuTeDSL at Perplexity", prefill/decode section: prefill GEMMs are
// compute-bound), so the kernel is a classic tiled GEMM on the MFMA units:
//
//   * a workgroup (4 waves) computes one tile of one expert's aligned, padded
//     slot list: a full tile is 256 rows against 256 weight columns (waves
//     2 x 2), a half tile 128 rows against 512 columns (waves 1 x 4) — the
//     alignment pads each expert to 128 rows and cuts its slots into
//     256-row rows plus, where 128 remain, one 128-row row, so an expert's
//     last rows cost half the padding a 256-row tile would; either way each
//     wave owns 128 rows x 128 columns.  For gate|up, 256 weight columns are
//     the 128 gate columns of an h-tile and the matching 128 up columns, so
//     SiLU(g)*u is applied to the fp32 accumulators in registers before the
//     single store of h ("La fusion de noyaux", section 4.2, GEMM +
//     epilogue; the concatenated d x 2*d_ff gate|up);
//   * K advances 32 at a time (one v_mfma_f32_16x16x32_bf16 deep) through a
//     ring of LDS stages (4 for bf16 weights, 6 for fp8; a stage holds the
//     larger shape's tiles) filled by direct
//     loads (global_load_lds_dwordx4): the token tile is gathered row by row
//     from x by slot (the permuted activations are never materialised), the
//     weight tile is copied untransposed ([K, N], N contiguous, the B[K,N] of
//     the vLLM post's A[M,K] x B[K,N]);
//   * the loop is software-pipelined per k-step: while the MFMAs of step j
//     run on fragments already in registers, the same instruction stream
//     reads step j+1's fragments from LDS and issues the direct loads that
//     refill the stage step j-1 used, spread between the MFMAs (and pinned
//     there), so the LDS, the vector memory path and the matrix cores are
//     busy at once; one workgroup barrier per step publishes the stage that
//     landed and frees the one just consumed;
//   * the weight operand's K-contiguous MFMA fragments come from gfx950's
//     transposing LDS reads: bf16 weights with ds_read_b64_tr_b16 (within
//     each 16-lane group, lane i receives element i%4 of the 8-byte pieces
//     addressed by lanes 4v + i/4, v = 0..3 — so lanes that address 4
//     consecutive rows x 16 columns hand lane i column i of those rows), two
//     per fragment; fp8 (e4m3) weights with ds_read_b64_tr_b8 (lane i
//     receives byte i%8 of the pieces addressed by lanes 2v + i/8, v = 0..7:
//     8 rows x 16 one-byte columns), one per fragment, widened exactly to
//     bf16 in registers; the fp8 per-column scale multiplies the fp32 sums in
//     the epilogue (scale factored out of the dot product, the vLLM post's
//     quantised fused-MoE statement);
//   * both LDS tiles are XOR-swizzled per row so the fragment reads hit
//     distinct banks;
//   * workgroups are renumbered so each of the 8 dies (one L2 each) runs a
//     contiguous range of tiles, walking 8 row blocks before the next weight
//     tile: the ~32 workgroups a die runs at once share their weight tiles
//     and token blocks in its L2, and a weight tile is fetched from HBM once
//     for up to 8 row blocks.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int TBN = 256;  // weight columns per weight sub-tile
constexpr int TBK = 32;   // k per step and per LDS stage
constexpr int GROUP_M = 8;
constexpr int NXCD = 8;   // accelerator complex dies; workgroup i runs on die i % 8
constexpr int MI = 8;             // 16-row A fragments per wave (128 rows)
constexpr int NMFMA = MI * 8;     // MFMAs per wave per step

// per weight type: element bytes, 16-byte chunks per weight-tile row, LDS
// reads per fragment, stages
template <int WT>
struct TCfg;
template <>
struct TCfg<W_BF16> {
  static constexpr int ESZ = 2, CHUNKS = 32, RD_PER_FRAG = 2, STAGES = 4;
};
template <>
struct TCfg<W_FP8> {
  static constexpr int ESZ = 1, CHUNKS = 16, RD_PER_FRAG = 1, STAGES = 6;
};
// Tile shapes.  Full: 256 rows x 256 columns, waves 2 x 2.  Half: 128 rows
// x 512 columns (two weight sub-tiles of 256), waves 1 x 4.  Every wave owns
// 128 rows x 128 columns either way.
template <int WT, bool HALF>
struct Cfg : TCfg<WT> {
  using T = TCfg<WT>;
  static constexpr int TM = HALF ? 128 : 256;
  static constexpr int NSUB = HALF ? 2 : 1;
  static constexpr int A_STAGE_BYTES = TM * TBK * 2;
  static constexpr int B_SUB_BYTES = TBK * TBN * T::ESZ;
  static constexpr int A_DPT = A_STAGE_BYTES / (256 * 16);  // direct loads per thread
  static constexpr int B_SUB_DPT = B_SUB_BYTES / (256 * 16);
  static constexpr int B_DPT = NSUB * B_SUB_DPT;
  static constexpr int DPT = A_DPT + B_DPT;
  static constexpr int NREAD = MI + 8 * T::RD_PER_FRAG;      // LDS reads per wave per step
  static_assert((T::STAGES - 2) * DPT < 64, "vmcnt field");
};
// one LDS ring serves both shapes: a stage holds the larger of the two
template <int WT>
struct Ring {
  using F = Cfg<WT, false>;
  using H = Cfg<WT, true>;
  static constexpr int FB = F::A_STAGE_BYTES + F::NSUB * F::B_SUB_BYTES;
  static constexpr int HB = H::A_STAGE_BYTES + H::NSUB * H::B_SUB_BYTES;
  static constexpr int STAGE_BYTES = FB > HB ? FB : HB;
  static constexpr int LDS_BYTES = TCfg<WT>::STAGES * STAGE_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14);
}

// swizzles: LDS chunk position of logical 16-byte chunk c in row r is c ^ swz(r).
//   A rows are 4 chunks (32 k x bf16): the 16 rows of a fragment read land in
//   16 distinct 16-byte bank groups, and any 8 consecutive rows in 8.
//   bf16 weight rows are 32 chunks (256 columns); fp8 weight rows 16 chunks,
//   where r & 15 spreads the 16 rows a fragment read touches over all
//   chunk positions.
__device__ __forceinline__ int swz_a(int r) {
  return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
}
template <int WT>
__device__ __forceinline__ int swz_b(int r) {
  if constexpr (WT == W_FP8)
    return r & 15;
  else
    return 2 * ((r & 3) | ((r >> 1) & 4));
}

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

// Byte offset of a shared-memory pointer within the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// Fragment reads are inline assembly so their completion is waited for with
// explicit counts (the compiler would otherwise wait for every outstanding
// direct load before each, since it cannot tell which LDS bytes those loads
// write).  Each is one LDS operation.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
// transposing reads of 8 bytes: four 16-bit or eight 8-bit elements
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
__device__ __forceinline__ u32x2 lds_read_tr8(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

// weight fragments as read from LDS
template <int WT>
struct BRaw {
  u32x2 lo[8], hi[8];  // k rows 8g..8g+3 and 8g+4..8g+7 of the lane's column
};
template <>
struct BRaw<W_FP8> {
  u32x2 b8[8];  // k rows 8g..8g+7 of the lane's column, one byte each
};
template <int WT>
struct Frags {
  u32x4 a[MI];
  BRaw<WT> b;
};

// s_waitcnt lgkmcnt(0) with the fragment registers tied to it, so nothing
// that reads them can be scheduled before the wait
template <int WT>
__device__ __forceinline__ void wait_frags(Frags<WT>& f) {
#pragma unroll
  for (int i = 0; i < MI; ++i) asm volatile("" : "+v"(f.a[i]));
  if constexpr (WT == W_FP8) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.b.b8[0]), "+v"(f.b.b8[1]), "+v"(f.b.b8[2]), "+v"(f.b.b8[3]),
                   "+v"(f.b.b8[4]), "+v"(f.b.b8[5]), "+v"(f.b.b8[6]), "+v"(f.b.b8[7]));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.b.lo[0]), "+v"(f.b.lo[1]), "+v"(f.b.lo[2]), "+v"(f.b.lo[3]),
                   "+v"(f.b.lo[4]), "+v"(f.b.lo[5]), "+v"(f.b.lo[6]), "+v"(f.b.lo[7]),
                   "+v"(f.b.hi[0]), "+v"(f.b.hi[1]), "+v"(f.b.hi[2]), "+v"(f.b.hi[3]),
                   "+v"(f.b.hi[4]), "+v"(f.b.hi[5]), "+v"(f.b.hi[6]), "+v"(f.b.hi[7]));
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) asm volatile("" : "+v"(f.a[i]));
}

// fp8 fragments widened to bf16 (gate|up) or fp16 (down) MFMA operands, both
// exact: every e4m3fn value is a bf16 and an fp16 normal.  The widening is
// VALU work feeding MFMAs the compiler cannot see, so the registers are tied
// to an s_nop 1 after it: the two wait states a VALU write needs before an
// MFMA reads the register.
template <bool F16>
__device__ __forceinline__ void widen_fp8(const BRaw<W_FP8>& b, u32x4 (&op)[8]) {
#pragma unroll
  for (int ni = 0; ni < 8; ++ni) {
    if constexpr (F16) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        op[ni][2 * h] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.b8[ni][h], 1.0f, false));
        op[ni][2 * h + 1] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.b8[ni][h], 1.0f, true));
      }
    } else {
      op[ni] = fp8x8_to_bf16x8(b.b8[ni]);
    }
  }
  asm volatile("s_nop 1"
               : "+v"(op[0]), "+v"(op[1]), "+v"(op[2]), "+v"(op[3]), "+v"(op[4]), "+v"(op[5]),
                 "+v"(op[6]), "+v"(op[7]));
}

// bf16 weight fragments rewritten in place as fp16 operands of the down
// GEMM: each bf16 is widened to fp32 (its bits in the high half) and
// converted with round toward zero, which is exact for magnitudes in fp16's
// normal range [2^-14, 65504] (bf16 has 8 significant bits, fp16 11); smaller
// ones lose at most 2^-24 as fp16 subnormals, larger ones saturate at 65504.
// Same s_nop tie as widen_fp8.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t d) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(d << 16),
                                                                 __uint_as_float(d & 0xFFFF0000u)));
}
__device__ __forceinline__ void widen_bf16_f16(BRaw<W_BF16>& b) {
#pragma unroll
  for (int ni = 0; ni < 8; ++ni)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      b.lo[ni][j] = bf16x2_to_f16x2(b.lo[ni][j]);
      b.hi[ni][j] = bf16x2_to_f16x2(b.hi[ni][j]);
    }
  asm volatile("s_nop 1"
               : "+v"(b.lo[0]), "+v"(b.lo[1]), "+v"(b.lo[2]), "+v"(b.lo[3]), "+v"(b.lo[4]),
                 "+v"(b.lo[5]), "+v"(b.lo[6]), "+v"(b.lo[7]), "+v"(b.hi[0]), "+v"(b.hi[1]),
                 "+v"(b.hi[2]), "+v"(b.hi[3]), "+v"(b.hi[4]), "+v"(b.hi[5]), "+v"(b.hi[6]),
                 "+v"(b.hi[7]));
}

// h values as a pair of fp16, rounded to nearest even (|h| beyond 65504
// overflows to infinity, which the output then shows).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// The k-loop MFMAs are inline assembly on accumulators pinned to AGPRs
// ("+a"): with builtins the register allocator moves accumulators between
// AGPRs and VGPRs at every loop back-edge once fragments are carried across
// it.  The compiler does not see these as MFMAs, so the code around them
// keeps the hazards away by construction: the accumulators are first written
// by an MFMA with an inline-constant zero C operand (no VALU write precedes
// an MFMA read of them), nothing but these MFMAs touches them inside the
// loop, operands written by VALU instructions are followed by s_nop padding
// (widen_fp8), and s_nop padding separates the last MFMA from the epilogue's
// reads.
// F16: the fp16 form (the down GEMM), else bf16.
template <bool F16>
__device__ __forceinline__ void mfma_acc(f32x4& acc, const u32x4& a, const u32x4& b) {
  if constexpr (F16)
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <bool F16>
__device__ __forceinline__ void mfma_zero(f32x4& acc, const u32x4& a, const u32x4& b) {
  if constexpr (F16)
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}

template <int I>
using IC = std::integral_constant<int, I>;
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(IC<Is>{}), ...);
}
// f(IC<0>{}), ..., f(IC<N-1>{}) in order
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Position of op i of n spread over the first `span` of `slots` MFMAs:
// op i goes right after MFMA (i * span) / n.
constexpr int slot_of(int i, int n, int span) { return (i * span) / n; }

}  // namespace

// One tile: rows [p0, p0 + TM) of expert e's slots against weight sub-tiles
// nt .. nt + NSUB - 1 (256 columns each), over the k-range of split ks (down
// only: the fp32 sums of split ks go to its own output plane, which the
// combine adds up; gate|up always has one split).  Called by all 256 threads after a
// barrier that frees the LDS ring.  Thread 0 claims the workgroup's next tile
// from *next as the tile starts and returns the counter's old value; other
// threads return 0.
// MIL: the wave's 16-row fragments that hold routed slots (the rest are
// padding, their MFMAs and fragment reads left out); MI for every full tile.
template <int EPI, int WT, bool HALF, int MIL>
__device__ __forceinline__ int run_tile(const StreamGemmArgs& p, char* lds, uint32_t lds_base,
                                        int p0, int e, int n_valid, int nt, int ks,
                                        int* next) {
  using C = Cfg<WT, HALF>;
  constexpr int S = C::STAGES;
  static_assert(TILED_MIN_KCHUNK / TBK >= S + 2, "the pipeline needs nk > S (nk even)");
  // the MFMAs compute the transposed blocks (weights as the first operand;
  // the two operands' lane layouts are the same), so a lane ends with 4
  // consecutive output columns of one row: one 8-byte store of 4 fp16 h
  // (gate|up) or y (down) values
  constexpr bool TRANSPOSED = true;
  // the down GEMM runs on fp16 operands: h as the gate|up epilogue stored it
  // (fp16, 11 significant bits) and the weights converted exactly
  constexpr bool F16 = EPI == EPI_STORE;
  constexpr int ESZ = C::ESZ;
  constexpr int CH = C::CHUNKS;    // 16-byte chunks per weight sub-tile row
  constexpr int EPC = 16 / ESZ;    // weight elements per chunk
  constexpr int STB = Ring<WT>::STAGE_BYTES;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // full: 2 x 2 waves; half: 1 x 4, waves 2j and 2j+1 on weight sub-tile j
  const int wm = HALF ? 0 : wave >> 1;
  const int wn = wave & 1;
  const int sub = HALF ? wave >> 1 : 0;
  const int ntw = nt + sub;        // the wave's 256-column tile
  const int lm = lane & 15, lg = lane >> 4;
  const int nk = p.kchunk / TBK;
  const int64_t k0 = (int64_t)ks * p.kchunk;
  // the workgroup's next tile, claimed now so the counter's latency hides
  // behind this tile (before any accumulator is live)
  const int claimed = tid == 0 ? atomicAdd(next, 1) : 0;

  // ---------------------------------------------------- direct-load sources
  // A slot s = (wave*A_DPT + i)*64 + lane -> tile row s/4, position s%4 =
  // lane%4 (64-slot blocks start at multiples of 4 rows).  gate|up gathers
  // token rows of x by slot; down reads h by slot directly (padding slots
  // read their own rows of h, in bounds, and their results are never stored)
  const char* a_src[C::A_DPT];
#pragma unroll
  for (int i = 0; i < C::A_DPT; ++i) {
    const int r = ((wave * C::A_DPT + i) * 64 + lane) >> 2;
    int row = p0 + r;
    if constexpr (EPI == EPI_SILU_MUL) {
      const int sid = p.sorted_ids[p0 + r];
      row = sid >= 0 ? sid / p.topk : 0;  // padding slots read token 0
    }
    const int c = (lane & 3) ^ swz_a(r);
    a_src[i] = reinterpret_cast<const char*>(p.a) + ((int64_t)row * p.a_ld + k0 + 8 * c) * 2;
  }
  // B slot of sub-tile 0: s = (wave*B_SUB_DPT + i)*64 + lane -> k row s/CH,
  // position s%CH; for gate|up the first half of a row's chunks are the
  // h-tile's gate columns, the second half the matching up columns.  Sub-tile
  // j's slots read the same rows SUB_OFF * j bytes further on.
  const char* b_src[C::B_SUB_DPT];
#pragma unroll
  for (int i = 0; i < C::B_SUB_DPT; ++i) {
    const int r = (wave * C::B_SUB_DPT + i) * (64 / CH) + lane / CH;
    const int c = (lane % CH) ^ swz_b<WT>(r);
    int col;
    if constexpr (EPI == EPI_SILU_MUL)
      col = (c < CH / 2) ? nt * 128 + EPC * c : p.up_off + nt * 128 + EPC * (c - CH / 2);
    else
      col = nt * TBN + EPC * c;
    b_src[i] = reinterpret_cast<const char*>(p.w) +
               ((int64_t)e * p.w_estride + (k0 + r) * p.w_ld + col) * ESZ;
  }
  constexpr int SUB_OFF = (EPI == EPI_SILU_MUL ? 128 : TBN) * ESZ;
  const int64_t b_kstep = (int64_t)TBK * p.w_ld * ESZ;  // bytes per k-step of B

  // the d-th direct load (of DPT) of k-step kt into stage st
  auto dma = [&](auto d_c, int st, int kt) __attribute__((always_inline)) {
    constexpr int d = decltype(d_c)::value;
    char* sa = lds + st * STB;
    if constexpr (d < C::A_DPT) {
      dma16(a_src[d] + (int64_t)kt * (TBK * 2), sa + (wave * C::A_DPT + d) * 1024);
    } else {
      constexpr int i = d - C::A_DPT;
      constexpr int j = i / C::B_SUB_DPT, ii = i % C::B_SUB_DPT;
      dma16(b_src[ii] + kt * b_kstep + j * SUB_OFF,
            sa + C::A_STAGE_BYTES + j * C::B_SUB_BYTES + (wave * C::B_SUB_DPT + ii) * 1024);
    }
  };
  auto dma_all = [&](int st, int kt) __attribute__((always_inline)) {
    static_for<C::DPT>([&](auto d) __attribute__((always_inline)) { dma(d, st, kt); });
  };

  // ---------------------------------------------------- fragment addresses
  // A fragment mi: row R = wm*128 + mi*16 + lane%16, chunk lane/16.
  // R%16 = lane%16, so the swizzle is the lane's own and the address is a
  // per-lane base plus the immediate mi*1024.
  const uint32_t a_base = (uint32_t)(((wm * 128 + lm) * 4 + (lg ^ swz_a(lm))) * 16);
  // B fragment ni covers chunk c0(ni) (fp8: 16 columns) or chunks c0(ni),
  // c0(ni)+1 (bf16) of the wave's columns in its sub-tile.
  //   bf16, half h: k row 8*lg + lm/4 + 4h, chunk c0 + (lm%4)/2, 8-byte half
  //   lm&1; swz of that row depends only on lm/4 and lg&1 (the lane's own),
  //   h is the immediate 4 rows.
  //   fp8: k row 8*lg + lm/2, chunk c0, 8-byte half lm&1.
  const uint32_t b_region = (uint32_t)(C::A_STAGE_BYTES + sub * C::B_SUB_BYTES);
  uint32_t b_base[8];
#pragma unroll
  for (int ni = 0; ni < 8; ++ni) {
    if constexpr (WT == W_FP8) {
      int c0;
      if constexpr (EPI == EPI_SILU_MUL)
        c0 = ni < 4 ? wn * 4 + ni : 8 + wn * 4 + (ni - 4);
      else
        c0 = wn * 8 + ni;
      const int row = 8 * lg + (lm >> 1);
      b_base[ni] = (uint32_t)((row * CH + (c0 ^ swz_b<WT>(row))) * 16 + (lm & 1) * 8) + b_region;
    } else {
      int c0;
      if constexpr (EPI == EPI_SILU_MUL)
        c0 = ni < 4 ? 2 * (wn * 4 + ni) : 16 + 2 * (wn * 4 + ni - 4);
      else
        c0 = 2 * (wn * 8 + ni);
      const int row = 8 * lg + (lm >> 2);
      const int xb = swz_b<WT>(row);
      b_base[ni] = (uint32_t)((row * CH + ((c0 ^ xb) + ((lm & 3) >> 1))) * 16 + (lm & 1) * 8) +
                   b_region;
    }
  }

  // r-th fragment read (of NREAD) of the stage at LDS offset st_off into f
  auto read = [&](auto r_c, Frags<WT>& f, uint32_t st_off) __attribute__((always_inline)) {
    constexpr int r = decltype(r_c)::value;
    if constexpr (r < MI) {
      if constexpr (r < MIL) f.a[r] = lds_read_b128<r * 1024>(st_off + a_base);
    } else if constexpr (WT == W_FP8) {
      f.b.b8[r - MI] = lds_read_tr8(st_off + b_base[r - MI]);
    } else {
      constexpr int ni = (r - MI) >> 1;
      if constexpr (((r - MI) & 1) == 0)
        f.b.lo[ni] = lds_read_tr16<0>(st_off + b_base[ni]);
      else
        f.b.hi[ni] = lds_read_tr16<4 * CH * 16>(st_off + b_base[ni]);
    }
  };

  f32x4 acc[MI][8];
  // fp8: bf16 weight operands of the current and the next step
  u32x4 w0[WT == W_FP8 ? 8 : 1], w1[WT == W_FP8 ? 8 : 1];

  // One k-step: MFMAs on `cur` (fp8: on the widened `wcur`); between them,
  // the reads of `nxt` from the stage at nxt_off (within the first 3/4 of the
  // MFMAs, so they land before the step ends) and, with REFILL, the direct
  // loads of k-step refill_kt into stage refill_st.  Every op is pinned where
  // it stands.  FIRST: the accumulators start from zero.
  auto step = [&](auto first_c, auto refill_c, Frags<WT>& cur, const u32x4* wcur,
                  Frags<WT>& nxt, uint32_t nxt_off, int refill_st,
                  int refill_kt) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr bool REFILL = decltype(refill_c)::value;
    static_for<NMFMA>([&](auto i_c) __attribute__((always_inline)) {
      constexpr int i = decltype(i_c)::value;
      constexpr int ni = i / MI, mi = i % MI;
      u32x4 bf;
      if constexpr (WT == W_FP8)
        bf = wcur[ni];
      else
        bf = u32x4{cur.b.lo[ni][0], cur.b.lo[ni][1], cur.b.hi[ni][0], cur.b.hi[ni][1]};
      if constexpr (mi >= MIL)
        ;  // a padding fragment
      else if constexpr (FIRST)
        if constexpr (TRANSPOSED)
          mfma_zero<F16>(acc[mi][ni], bf, cur.a[mi]);
        else
          mfma_zero<F16>(acc[mi][ni], cur.a[mi], bf);
      else
        if constexpr (TRANSPOSED)
          mfma_acc<F16>(acc[mi][ni], bf, cur.a[mi]);
        else
          mfma_acc<F16>(acc[mi][ni], cur.a[mi], bf);
      static_for<C::NREAD>([&](auto r_c) __attribute__((always_inline)) {
        if constexpr (slot_of(decltype(r_c)::value, C::NREAD, (3 * NMFMA) / 4) == i)
          read(r_c, nxt, nxt_off);
      });
      if constexpr (REFILL)
        static_for<C::DPT>([&](auto d_c) __attribute__((always_inline)) {
          if constexpr (slot_of(decltype(d_c)::value, C::DPT, NMFMA) == i)
            dma(d_c, refill_st, refill_kt);
        });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---------------------------------------------------- main loop
  // The stage of k-step kt is kt % S.  At step kt, k-step kt+1 has landed
  // (waited for before the barrier) and every wave has finished reading stage
  // kt%S (fragments kt were read and waited for in step kt-1), so while
  // fragments kt+1 are read during the MFMAs that stage is refilled with
  // k-step kt+S — in the refill steps kt < nk-S.  In the last S steps fp8
  // weights load nothing: at step kt the loads in flight are those of
  // k-steps kt+1 .. min(kt+S-1, nk-1), so "k-step kt+1 landed" is a wait
  // until the min(S-2, nk-2-kt) later k-steps' loads at most are
  // outstanding, a constant in every step.  bf16 weights keep every step's
  // shape there instead (the refill reloads k-step kt, in bounds, never read
  // again, and the wait stays S-2): their registers are at the limit, and
  // the loadless steps cost them a few spills that the saved loads did not
  // pay back.  The last step's reads of the following stage are discarded.
  // The launcher guarantees nk > S.
  constexpr bool LOADLESS_TAIL = WT == W_FP8;
#pragma unroll
  for (int s = 0; s < S; ++s) dma_all(s, s);
  Frags<WT> f0, f1;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 1) * C::DPT));
  __builtin_amdgcn_s_barrier();
  static_for<C::NREAD>([&](auto r) __attribute__((always_inline)) { read(r, f0, lds_base); });
  wait_frags(f0);
  if constexpr (WT == W_FP8)
    widen_fp8<F16>(f0.b, w0);
  else if constexpr (F16)
    widen_bf16_f16(f0.b);

  // LATER: k-steps' loads issued after those of kt+1 that may still be in
  // flight; REFILL false: a tail step (fp8: no loads; bf16: reload k-step kt)
  auto one = [&](auto first_c, auto refill_c, auto later_c, Frags<WT>& cur, const u32x4* wcur,
                 Frags<WT>& nxt, u32x4* wnxt, int kt) __attribute__((always_inline)) {
    constexpr bool REFILL = decltype(refill_c)::value;
    constexpr int LATER = LOADLESS_TAIL ? decltype(later_c)::value : S - 2;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(LATER * C::DPT));
    __builtin_amdgcn_s_barrier();
    step(first_c, std::integral_constant<bool, REFILL || !LOADLESS_TAIL>{}, cur, wcur, nxt,
         lds_base + ((kt + 1) % S) * STB, kt % S, REFILL ? kt + S : kt);
    wait_frags(nxt);
    if constexpr (WT == W_FP8)
      widen_fp8<F16>(nxt.b, *reinterpret_cast<u32x4(*)[8]>(wnxt));
    else if constexpr (F16)
      widen_bf16_f16(nxt.b);
  };
  // nk and S are even (a split is a multiple of 64 deep): step 0, the refill
  // pairs (1, 2) .. (nk-S-3, nk-S-2), step nk-S-1, then the S tail steps
  // unrolled; fragments alternate f0 (even kt) / f1 (odd kt), so only f0 is
  // live where the loop closes
  using T_ = std::true_type;
  using F_ = std::false_type;
  one(T_{}, T_{}, IC<S - 2>{}, f0, w0, f1, w1, 0);
  int kt = 1;
  for (; kt + 1 < nk - S; kt += 2) {
    one(F_{}, T_{}, IC<S - 2>{}, f1, w1, f0, w0, kt);
    one(F_{}, T_{}, IC<S - 2>{}, f0, w0, f1, w1, kt + 1);
  }
  one(F_{}, T_{}, IC<S - 2>{}, f1, w1, f0, w0, kt);  // kt = nk-S-1
  ++kt;
  static_for<S / 2>([&](auto j_c) __attribute__((always_inline)) {
    constexpr int j = decltype(j_c)::value;
    constexpr int l0 = S - 2 - 2 * j, l1 = S - 3 - 2 * j;  // min(S-2, nk-2-kt)
    one(F_{}, F_{}, IC<l0>{}, f0, w0, f1, w1, kt + 2 * j);
    one(F_{}, F_{}, IC<(l1 > 0 ? l1 : 0)>{}, f1, w1, f0, w0, kt + 2 * j + 1);
  });
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  // the last MFMAs' results are complete before anything else reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) asm volatile("" : "+a"(acc[mi][ni]));

  // ---------------------------------------------------- epilogue
  if constexpr (EPI == EPI_SILU_MUL) {
    // gate|up: the MFMAs took the weight fragment as their first operand, so
    // each 16 x 16 block came out transposed: acc[mi][ni] lane (lm, lg) holds
    // token row wm*128 + mi*16 + lm and the 4 consecutive weight columns
    // 4*lg + r of the block — gate columns ntw*128 + wn*64 + 16ni + 4lg + r
    // for ni < 4, the matching up columns for ni + 4.  One 8-byte store of 4
    // h values per block instead of four 2-byte ones (bf16 weights 0-2 %,
    // fp8 2-5 % faster GEMMs).
    const int lrow0 = wm * 128 + lm;
    const int c0 = ntw * 128 + wn * 64 + 4 * lg;
    f32x4 sc[8];  // fp8: scales of the lane's 4 columns of each block
    if constexpr (WT == W_FP8) {
      const float* sb = p.scale + (int64_t)e * p.scale_estride + c0;
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
        const u32x4 v = ld16(sb + (ni < 4 ? 0 : p.up_off) + 16 * (ni & 3));
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[ni][r] = __uint_as_float(v[r]);
      }
    }
    // the lane's row of block row mi holds a routed slot iff mi*16 < vrows
    const int vrows = n_valid - lrow0;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (mi * 16 >= vrows) continue;  // padding slot
      uint16_t* dst =
          reinterpret_cast<uint16_t*>(p.out) + (int64_t)(p0 + lrow0 + mi * 16) * p.out_ld + c0;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float g = acc[mi][ni][r], u = acc[mi][ni + 4][r];
          if constexpr (WT == W_FP8) {
            g *= sc[ni][r];
            u *= sc[ni + 4][r];
          }
          hv[r] = silu(g) * u;
        }
        // h in fp16 for the down GEMM (see F16)
        const u32x2 o = {pack_f16x2(hv[0], hv[1]), pack_f16x2(hv[2], hv[3])};
        *reinterpret_cast<u32x2*>(dst + ni * 16) = o;
      }
    }
  } else {
    // down: acc[mi][ni] lane (lm, lg) holds token row wm*128 + mi*16 + lm and
    // the 4 consecutive output columns ntw*256 + wn*128 + 16ni + 4lg + r,
    // scaled (fp8) and stored as fp16 (its 11 significant bits keep the
    // combine's sum within the output's own rounding; half the bytes of fp32)
    const int lrow0 = wm * 128 + lm;
    const int c0 = ntw * TBN + wn * 128 + 4 * lg;
    f32x4 sc[8];  // fp8: scales of the lane's 4 columns of each block
    if constexpr (WT == W_FP8) {
      const float* sb = p.scale + (int64_t)e * p.scale_estride + c0;
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
        const u32x4 v = ld16(sb + 16 * ni);
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[ni][r] = __uint_as_float(v[r]);
      }
    }
    // The wave's 128 x 128 block goes through LDS (the ring is idle once
    // every wave has read its last fragments): a direct 8-byte store per
    // block writes 32 bytes into each of 16 rows, and those scattered
    // stores cost the short-K down GEMMs 10-25 % of their time; read back
    // row-wise, one instruction stores 4 whole 256-byte row segments.
    // Staged rows are 272 bytes apart, so the 8-byte writes of a half-wave
    // hit 64 distinct banks.
    constexpr int RS = 272;
    static_assert(4 * 128 * RS <= Ring<WT>::LDS_BYTES, "staging fits the ring");
    char* stage = lds + wave * 128 * RS;
    __syncthreads();  // every wave has read its last fragments
    const int vrows = n_valid - lrow0;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (mi * 16 >= vrows) continue;  // padding slot
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[mi][ni][r];
          if constexpr (WT == W_FP8) v[r] *= sc[ni][r];
        }
        const u32x2 o = {pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(stage + (mi * 16 + lm) * RS + ni * 32 + lg * 8) = o;
      }
    }
    // routed rows of the wave's block (a prefix: routed slots come first)
    const int wrows = min(128, n_valid - wm * 128);
    char* gdst = reinterpret_cast<char*>(p.out) +
                 (ks * p.out_split_stride + (int64_t)(p0 + wm * 128) * p.out_ld + ntw * TBN +
                  wn * 128) * 2;
#pragma unroll 4
    for (int j = 0; j < 32; ++j) {
      const int r = 4 * j + (lane >> 4);
      if (r < wrows)
        *reinterpret_cast<u32x4*>(gdst + (int64_t)r * p.out_ld * 2 + (lane & 15) * 16) =
            *reinterpret_cast<const u32x4*>(stage + r * RS + (lane & 15) * 16);
    }
  }
  return claimed;
}

template <int EPI, int WT>
__global__ __launch_bounds__(256) void k_expert_tiled(const StreamGemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const uint32_t lds_base = lds_off(lds);

  // ---------------------------------------------------- tiles of this workgroup
  // Persistent: one workgroup per compute unit takes tiles of the rows the
  // alignment listed (their counts are read from the device, so no
  // workgroups are spent on the worst-case capacity).  Full rows come first,
  // n_tiles tiles each, then half rows, n_tiles/2 tiles each; within each
  // kind, GROUP_M rows are walked before the next weight tile.  The
  // dispatcher deals workgroups to the dies round-robin, each die with its
  // own L2: every die takes a contiguous share of that numbering, so the
  // workgroups a die runs at once share weight tiles and token blocks in its
  // L2 instead of each die fetching every weight tile.  The shares are equal
  // in cost, a half tile counting 5/4 of a full one (its 128 x 512 tile
  // issues more loads per MFMA; measured 1.1-1.3x a full tile's time), and
  // within a die the workgroups claim the share's tiles in order from the
  // die's counter, so unequal tiles still end together.
  // With k-splits (down only) the numbering repeats once per split.
  const int n_full = min(p.tile_counts[0], p.num_mblocks);
  const int n_half = min(p.tile_counts[1], p.num_mblocks - n_full);
  const int nt_half = p.n_tiles / 2;
  const int work_full = n_full * p.n_tiles;
  const int work1 = work_full + n_half * nt_half;  // tiles of one split
  const int64_t cost_full = 4 * (int64_t)work_full;
  const int64_t cost1 = cost_full + 5 * (int64_t)n_half * nt_half;
  const int64_t cost = cost1 * p.ksplit;
  // first tile whose cost range starts at or after c
  auto tile_at = [&](int64_t c) -> int {
    if (cost1 == 0) return 0;
    const int ks = (int)(c / cost1);
    const int64_t r = c - ks * cost1;
    return ks * work1 +
           (r <= cost_full ? (int)((r + 3) / 4) : work_full + (int)((r - cost_full + 4) / 5));
  };
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % NXCD;
  const int q = nwg / NXCD, rem = nwg % NXCD;
  const int on_die = q + (xcd < rem ? 1 : 0);
  const int before = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
  const int w_begin = tile_at(cost * before / nwg);
  const int w_end = tile_at(cost * (before + on_die) / nwg);
  int* next = p.die_next + xcd;
  // thread 0's claim goes to every thread through a word of the (then idle)
  // LDS ring; the second barrier keeps the next tile's loads from
  // overwriting it before every wave has read it
  int* s_claim = reinterpret_cast<int*>(lds);
  auto publish = [&](int v) __attribute__((always_inline)) {
    if (threadIdx.x == 0) s_claim[0] = v;
    __syncthreads();
    // uniform across the workgroup: keep it (and the tile's indices) scalar
    const int r = __builtin_amdgcn_readfirstlane(s_claim[0]);
    __syncthreads();
    return r;
  };
  int id = w_begin + publish(threadIdx.x == 0 ? atomicAdd(next, 1) : 0);
  while (id < w_end) {
    const int ks = id / work1;
    const int t = id - ks * work1;
    const bool full = t < work_full;
    const int rows = full ? n_full : n_half;
    const int nts = full ? p.n_tiles : nt_half;
    const int lid = full ? t : t - work_full;
    const int per_group = GROUP_M * nts;
    const int grp = lid / per_group;
    const int first = grp * GROUP_M;
    const int gm = min(GROUP_M, rows - first);
    const int local = lid - grp * per_group;
    const int row = (full ? 0 : n_full) + first + local % gm;
    const int nt = local / gm;
    const int p0 = p.tile_rows[2 * row];
    const int ev = p.tile_rows[2 * row + 1];
    const int e = ev & 0xFFFF, n_valid = ev >> 16;
    const int claimed =
        full ? run_tile<EPI, WT, false, MI>(p, lds, lds_base, p0, e, n_valid, nt, ks, next)
        // a half row with at most 32 or 64 routed slots (light experts'
        // last rows): two or four live fragments per wave
        : n_valid <= 32
            ? run_tile<EPI, WT, true, 2>(p, lds, lds_base, p0, e, n_valid, 2 * nt, ks, next)
        : n_valid <= 64
            ? run_tile<EPI, WT, true, 4>(p, lds, lds_base, p0, e, n_valid, 2 * nt, ks, next)
            : run_tile<EPI, WT, true, MI>(p, lds, lds_base, p0, e, n_valid, 2 * nt, ks, next);
    // every wave is done with the tile's LDS stages
    __syncthreads();
    id = w_begin + publish(claimed);
  }
}

template <int EPI, int WT>
static hipError_t launch_tiled(const StreamGemmArgs& a, hipStream_t st) {
  const int64_t work = (int64_t)a.num_mblocks * a.n_tiles * a.ksplit;
  if (work <= 0) return hipSuccess;
  if (work > 0x7FFFFFFF) return hipErrorInvalidValue;
  // one resident workgroup per compute unit
  const int64_t grid = std::min<int64_t>(work, device_cus());
  constexpr int lds = Ring<WT>::LDS_BYTES;
  hipError_t e = hipFuncSetAttribute((const void*)k_expert_tiled<EPI, WT>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_expert_tiled<EPI, WT>), dim3((unsigned)grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_tiled_gemm(int epi, int w_dtype, int bm, const StreamGemmArgs& a,
                             hipStream_t st) {
  // half rows (bm = 128) pair two 256-column tiles: n_tiles must be even
  if ((bm != 256 && bm != 128) || a.K % 64 != 0) return hipErrorInvalidValue;
  // k-splits: down only, each a multiple of 64 deep
  if (a.ksplit < 1 || a.kchunk % 64 != 0 || (int64_t)a.ksplit * a.kchunk != a.K ||
      (epi == EPI_SILU_MUL && a.ksplit != 1))
    return hipErrorInvalidValue;
  if (bm == 128 && a.n_tiles % 2 != 0) return hipErrorInvalidValue;
  // more k-steps per split than LDS stages (the pipeline's prologue fills
  // every stage with real k-steps)
  if (a.kchunk < TILED_MIN_KCHUNK) return hipErrorInvalidValue;
  if (a.tile_rows == nullptr || a.tile_counts == nullptr || a.die_next == nullptr)
    return hipErrorInvalidValue;
  // gate|up gathers tokens by slot, down reads its rows by slot
  if (a.a_mode != (epi == EPI_SILU_MUL ? A_GATHER : A_PADDED)) return hipErrorInvalidValue;
  if (w_dtype == W_FP8) {
    if (a.scale == nullptr) return hipErrorInvalidValue;
    return epi == EPI_SILU_MUL ? launch_tiled<EPI_SILU_MUL, W_FP8>(a, st)
                               : launch_tiled<EPI_STORE, W_FP8>(a, st);
  }
  if (w_dtype == W_BF16)
    return epi == EPI_SILU_MUL ? launch_tiled<EPI_SILU_MUL, W_BF16>(a, st)
                               : launch_tiled<EPI_STORE, W_BF16>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
