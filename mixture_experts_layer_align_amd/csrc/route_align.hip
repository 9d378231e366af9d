// Routing (softmax / top-k / renormalisation) and expert alignment.
//
// Routing: one wave per token.  Each lane holds E/64 logits; k rounds of a
// wave-wide butterfly argmax over the experts not yet taken pick the slots
// in descending order with ties to the lower index, and the renormalised
// softmax weight of slot j is exp(L_j - L_max) / sum_j' exp(L_j' - L_max)
// (the softmax denominator over all E cancels in the renormalisation).  The
// butterfly shuffles are the gfx950 form of the sub-warp horizontal
// reductions of "CuTeDSL at Perplexity"
// (section on QK-norm, and the half-/quarter-warp reductions of its Blackwell
// section).
//
// Alignment ("CuTeDSL at Perplexity", MoE dispatch and combine, local kernel:
// count the tokens of each expert and give every token a unique index in its
// expert's list; prefill spreads the routing over many blocks with a global
// aggregation).  The pages assign slots with shared-memory atomic counters,
// which makes the order within an expert depend on scheduling.  Here every
// step is integer and order-preserving, so the permutation is the unique
// stable one:
//   * per 64-entry chunk, lanes holding the same expert find each other with
//     log2(E) ballots (a "match" mask); the lane's rank among equal lanes below
//     it is a popcount; the lowest such lane adds the chunk count to its
//     wave's running per-expert histogram in LDS (one writer per address);
//   * per expert, an exclusive prefix over waves (and, for large inputs, over
//     4096-entry tiles) turns local ranks into ranks within the expert;
//   * an exclusive scan of counts rounded up to the block size gives the padded
//     offsets; entry i lands at offsets[e] + rank.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

// ================================================================ top-k

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Wave-wide argmax under (value desc, index asc): afterwards every lane holds
// the wave's best (value, index).  The first four levels pair lanes inside
// each row of 16 with DPP moves (quad permutes xor 1 and xor 2, then the
// half-row and row mirrors, which pair lanes of the two halves of the
// previous level's groups); the last two cross rows with shuffles.  The
// maximum of a total order does not depend on the pairing.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_mov_dpp(bi, CTRL, 0xF, 0xF, false);
  if (better(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  argmax_dpp<0xB1>(bv, bi);   // quad_perm(1, 0, 3, 2): lane ^ 1
  argmax_dpp<0x4E>(bv, bi);   // quad_perm(2, 3, 0, 1): lane ^ 2
  argmax_dpp<0x141>(bv, bi);  // row_half_mirror: 7 - lane within 8
  argmax_dpp<0x140>(bv, bi);  // row_mirror: 15 - lane within 16
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

// One selection round over a wave's logits v (expert lane + 64j): the best
// expert not yet taken, under (value desc, index asc), in every lane; its
// owner lane marks it taken.  Taken experts are skipped rather than
// overwritten, so logits of -inf (a masking bias) still rank by index after
// the finite ones and no expert is selected twice.  Bits j of `taken` start
// set for experts past E, which are never candidates; k <= E leaves an
// untaken expert in every round.
template <int V>
__device__ __forceinline__ void pick_next(const float (&v)[V], uint32_t& taken, int lane,
                                          float& bv, int& bi) {
  static_assert(V <= 32, "taken mask");
  bv = -INFINITY;
  bi = 0x7FFFFFFF;  // no candidate: loses to any expert, -inf included
#pragma unroll
  for (int j = 0; j < V; ++j)
    if (!((taken >> j) & 1u) && better(v[j], lane + 64 * j, bv, bi)) {
      bv = v[j];
      bi = lane + 64 * j;
    }
  wave_argmax(bv, bi);
  if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
}

// experts past E start out taken
template <int V>
__device__ __forceinline__ uint32_t taken_init(int lane, int E) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < V; ++j)
    if (lane + 64 * j >= E) m |= 1u << j;
  return m;
}

// Router partial planes are added in one fixed order whatever the launch
// shape: four interleaved sums (planes q, q+4, q+8, ... in plane order, for
// q = 0..3), then ((s0 + s1) + s2) + s3.  All V values of a plane are loaded
// together and planes are unrolled, so many loads are in flight (slots past
// E read expert E-1, in bounds, and are discarded).
template <int V>
__device__ __forceinline__ void plane_sums(const float* __restrict__ pp, int nsplit,
                                           int64_t split_stride, int E, int lane,
                                           float (&acc)[4][V]) {
  int eo[V];
#pragma unroll
  for (int j = 0; j < V; ++j) eo[j] = min(lane + 64 * j, E - 1);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < V; ++j) acc[q][j] = 0.f;
  for (int base = 0; base < nsplit; base += 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (base + q >= nsplit) continue;
      const float* p = pp + (base + q) * split_stride;
#pragma unroll
      for (int j = 0; j < V; ++j) acc[q][j] += p[eo[j]];
    }
  }
}
// the interleaved sum q alone (planes q, q+4, ...)
template <int V>
__device__ __forceinline__ void plane_sum_q(const float* __restrict__ pp, int nsplit,
                                            int64_t split_stride, int E, int lane, int q,
                                            float (&acc)[V]) {
  int eo[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    eo[j] = min(lane + 64 * j, E - 1);
    acc[j] = 0.f;
  }
#pragma unroll 4
  for (int sp = q; sp < nsplit; sp += 4) {
    const float* p = pp + sp * split_stride;
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] += p[eo[j]];
  }
}

// Top-k of one token per wave (tokens = 4 per workgroup) or, with WIDE, of
// one token per workgroup whose 4 waves each own one of the 4 plane sums.
// Selection r is kept by lane r (k <= 64), or in LDS with BIGK (k > 64);
// either way the weights are computed from the same values in the same
// order, so the bits do not depend on k's path.
template <int V, bool WIDE, bool BIGK>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ partial, int nsplit,
                                              int64_t split_stride, const float* __restrict__ bias,
                                              int T, int E, int k, float* __restrict__ logits,
                                              int32_t* __restrict__ ids, float* __restrict__ wout) {
  __shared__ float part[WIDE ? 4 : 1][WIDE ? MAX_EXPERTS : 1];
  constexpr int NSEL = BIGK ? (WIDE ? 1 : 4) : 1;
  __shared__ float sel_v[NSEL][BIGK ? MAX_EXPERTS : 1];
  __shared__ int sel_i[NSEL][BIGK ? MAX_EXPERTS : 1];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = WIDE ? blockIdx.x : blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float* pp = partial + (int64_t)t * E;

  float v[V];
  if constexpr (WIDE) {
    float acc[V];
    plane_sum_q<V>(pp, nsplit, split_stride, E, lane, wave, acc);
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (lane + 64 * j < E) part[wave][lane + 64 * j] = acc[j];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int e = min(lane + 64 * j, E - 1);
      v[j] = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
    }
  } else {
    float acc[4][V];
    plane_sums<V>(pp, nsplit, split_stride, E, lane, acc);
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = ((acc[0][j] + acc[1][j]) + acc[2][j]) + acc[3][j];
  }
  const int sw = WIDE ? 0 : wave;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      if (bias != nullptr) v[j] += bias[e];
      if (logits != nullptr) logits[(int64_t)t * E + e] = v[j];
    } else {
      v[j] = -INFINITY;
    }
  }

  float my_v = 0.f, l0 = 0.f;  // !BIGK: selection `lane`; the largest logit
  int my_i = 0;
  uint32_t taken = taken_init<V>(lane, E);
  for (int r = 0; r < k; ++r) {
    float bv;
    int bi;
    pick_next<V>(v, taken, lane, bv, bi);
    if (r == 0) l0 = bv;
    if constexpr (BIGK) {
      if (lane == 0) {
        sel_v[sw][r] = bv;
        sel_i[sw][r] = bi;
      }
    } else if (lane == r) {
      my_v = bv;
      my_i = bi;
    }
  }
  // weights: exp(L_j - L_0) / sum, the sum as a fixed butterfly
  float psum = 0.f;
  if constexpr (BIGK) {
    for (int r = lane; r < k; r += 64) psum += expf(sel_v[sw][r] - l0);
  } else {
    if (lane < k) psum = expf(my_v - l0);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) psum += __shfl_xor(psum, off);
  const float inv = 1.0f / psum;
  if constexpr (BIGK) {
    for (int r = lane; r < k; r += 64) {
      ids[(int64_t)t * k + r] = sel_i[sw][r];
      wout[(int64_t)t * k + r] = expf(sel_v[sw][r] - l0) * inv;
    }
  } else if (lane < k) {
    ids[(int64_t)t * k + lane] = my_i;
    wout[(int64_t)t * k + lane] = expf(my_v - l0) * inv;
  }
}

// tokens from which one wave per token fills the chip better than a
// workgroup per token
constexpr int TOPK_WIDE_MAX_T = 1024;

template <int V, bool WIDE>
static void launch_topk_v(int grid, const float* partial, int nsplit, int64_t split_stride,
                          const float* bias, int T, int E, int k, float* logits, int32_t* ids,
                          float* w, hipStream_t st) {
  if (k > 64)
    hipLaunchKernelGGL((k_topk<V, WIDE, true>), dim3(grid), dim3(256), 0, st, partial, nsplit,
                       split_stride, bias, T, E, k, logits, ids, w);
  else
    hipLaunchKernelGGL((k_topk<V, WIDE, false>), dim3(grid), dim3(256), 0, st, partial, nsplit,
                       split_stride, bias, T, E, k, logits, ids, w);
}

template <int V>
static void launch_topk_w(bool wide, const float* partial, int nsplit, int64_t split_stride,
                          const float* bias, int T, int E, int k, float* logits, int32_t* ids,
                          float* w, hipStream_t st) {
  if (wide)
    launch_topk_v<V, true>(T, partial, nsplit, split_stride, bias, T, E, k, logits, ids, w, st);
  else
    launch_topk_v<V, false>((T + 3) / 4, partial, nsplit, split_stride, bias, T, E, k, logits,
                            ids, w, st);
}

hipError_t launch_topk(const float* partial, int nsplit, int64_t split_stride, const float* bias,
                       int T, int E, int k, float* logits, int32_t* ids, float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const bool wide = T <= TOPK_WIDE_MAX_T;
  if (E <= 64)
    launch_topk_w<1>(wide, partial, nsplit, split_stride, bias, T, E, k, logits, ids, w, st);
  else if (E <= 128)
    launch_topk_w<2>(wide, partial, nsplit, split_stride, bias, T, E, k, logits, ids, w, st);
  else if (E <= 256)
    launch_topk_w<4>(wide, partial, nsplit, split_stride, bias, T, E, k, logits, ids, w, st);
  else if (E <= 512)
    launch_topk_w<8>(wide, partial, nsplit, split_stride, bias, T, E, k, logits, ids, w, st);
  else
    launch_topk_w<16>(wide, partial, nsplit, split_stride, bias, T, E, k, logits, ids, w, st);
  return hipGetLastError();
}

// ================================================================ alignment

constexpr int AL_THREADS = 1024;
constexpr int AL_WAVES = AL_THREADS / 64;
constexpr int AL_CHUNKS_PER_WAVE = ALIGN_TILE / (AL_WAVES * 64);  // 4

static_assert(ALIGN_SINGLE_MAX == ALIGN_TILE, "single-workgroup path covers one tile");

// Block-wide exclusive scan of one int per thread (1024 threads).  Returns the
// exclusive prefix; *total receives the sum.  Fixed order, integer exact.
__device__ int block_exscan(int x, int* sh /* [AL_WAVES + 1] */, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < AL_WAVES; ++w) {
      const int c = sh[w];
      sh[w] = run;
      run += c;
    }
    sh[AL_WAVES] = run;
  }
  __syncthreads();
  const int ex = sh[wave] + inc - x;
  *total = sh[AL_WAVES];
  __syncthreads();
  return ex;
}

// Processes the entries [i0, i0 + cnt) of one tile with 16 waves: fills
// hist[w][e] with each wave's per-expert count and returns, per lane and chunk,
// the entry's expert and its rank among the same-expert entries of its wave
// that precede it.  After return (and a barrier) hist holds per-wave counts.
struct ChunkState {
  int e[AL_CHUNKS_PER_WAVE];
  int r[AL_CHUNKS_PER_WAVE];
};

__device__ ChunkState tile_local_ranks(const int32_t* __restrict__ ids, int64_t i0, int cnt, int E,
                                       int nbits, int* hist /* [AL_WAVES][E] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int x = threadIdx.x; x < AL_WAVES * E; x += AL_THREADS) hist[x] = 0;
  __syncthreads();
  ChunkState cs;
  int* h = hist + wave * E;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int c = 0; c < AL_CHUNKS_PER_WAVE; ++c) {
    const int local = (wave * AL_CHUNKS_PER_WAVE + c) * 64 + lane;
    const bool valid = local < cnt;
    const int e = valid ? ids[i0 + local] : 0;
    uint64_t mask = ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = ballot(valid && bit);
      mask &= bit ? m : ~m;
    }
    const int below = __popcll(mask & lt);
    int r = 0;
    if (valid) r = h[e] + below;
    // all reads of this chunk precede the leader's update (in-order LDS per wave)
    __builtin_amdgcn_wave_barrier();
    if (valid && below == 0) h[e] += __popcll(mask);
    __builtin_amdgcn_wave_barrier();
    cs.e[c] = valid ? e : -1;
    cs.r[c] = r;
  }
  __syncthreads();
  return cs;
}

// Turns hist[w][e] (per-wave counts) into exclusive per-wave prefixes and
// returns the tile total of expert e = threadIdx.x (threads >= E return 0).
__device__ int hist_wave_prefix(int* hist, int E) {
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int w = 0; w < AL_WAVES; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  return run;
}

// counts/offsets known (in LDS): write counts, offsets, padding -1 slots,
// block_expert and, if asked for, the tiled GEMM's row list.  Called by every
// thread of one workgroup (E <= AL_THREADS); sh is scan scratch.  PREFILLED:
// the workgroup already set every slot and block to -1 (prefill_layout,
// ordered before this by a workgroup barrier), so only the experts' blocks
// are written here.
template <bool PREFILLED>
__device__ void write_layout(const AlignArgs& a, const int* s_counts, const int* s_off, int* sh) {
  const int E = a.E, bm = a.bm;
  for (int e = threadIdx.x; e < E; e += AL_THREADS) {
    a.counts[e] = s_counts[e];
    a.offsets[e] = s_off[e];
    if (!PREFILLED)
      for (int s = s_off[e] + s_counts[e]; s < s_off[e + 1]; ++s) a.sorted_ids[s] = -1;
    for (int b = s_off[e] / bm; b < s_off[e + 1] / bm; ++b) a.block_expert[b] = e;
  }
  if (threadIdx.x == 0) a.offsets[E] = s_off[E];
  if (!PREFILLED) {
    for (int64_t s = s_off[E] + threadIdx.x; s < a.cap; s += AL_THREADS) a.sorted_ids[s] = -1;
    for (int64_t b = s_off[E] / bm + threadIdx.x; b < a.cap / bm; b += AL_THREADS)
      a.block_expert[b] = -1;
  }
  if (a.tile_rows == nullptr) return;
  // rows of 256 slots; a remainder (128 slots when bm = 128) is a half row
  const int e = threadIdx.x;
  int nf = 0, nh = 0;
  if (e < E) {
    const int pad = s_off[e + 1] - s_off[e];
    nf = pad / 256;
    nh = pad % 256 != 0 ? 1 : 0;
  }
  int tot_f, tot_h;
  const int bf = block_exscan(nf, sh, &tot_f);
  const int bh = block_exscan(nh, sh, &tot_h);
  // {first slot, expert | routed rows of the row << 16}: the routed slots of
  // an expert come first in its range, so a row's routed slots are a prefix
  if (e < E) {
    const int cnt = s_counts[e];
    for (int r = 0; r < nf; ++r) {
      a.tile_rows[2 * (bf + r)] = s_off[e] + 256 * r;
      a.tile_rows[2 * (bf + r) + 1] = e | (min(max(cnt - 256 * r, 0), 256) << 16);
    }
    if (nh != 0) {
      a.tile_rows[2 * (tot_f + bh)] = s_off[e] + 256 * nf;
      a.tile_rows[2 * (tot_f + bh) + 1] = e | (min(max(cnt - 256 * nf, 0), 128) << 16);
    }
  }
  if (threadIdx.x == 0) {
    a.tile_counts[0] = tot_f;
    a.tile_counts[1] = tot_h;
  }
  if (threadIdx.x < TILE_COUNTERS) a.tile_counts[2 + threadIdx.x] = 0;
}

// Every slot of sorted_ids and every block of block_expert to -1, by all
// threads of a single-workgroup launch, before the routed slots and the
// experts' blocks are written over them after a workgroup barrier (which
// waits for these stores): one coalesced pass instead of per-expert padding
// loops and a tail fill on a few threads.
__device__ void prefill_layout(const AlignArgs& a) {
  for (int64_t s = threadIdx.x; s < a.cap; s += blockDim.x) a.sorted_ids[s] = -1;
  const int64_t nb = a.cap / a.bm;
  for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) a.block_expert[b] = -1;
}

__device__ __forceinline__ int ilog2_ceil(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

// One workgroup aligns all entries (n <= ALIGN_TILE) of `ids` (global or
// LDS memory); lds holds AL_WAVES * E + 2 * E + 1 + AL_WAVES + 1 ints.  The
// layout arrays must have been prefilled (prefill_layout) by the workgroup;
// the barriers below order those stores first.
__device__ void align_one_tile(const AlignArgs& a, const int32_t* ids, int* lds) {
  int* hist = lds;                          // [AL_WAVES][E]
  int* s_counts = hist + AL_WAVES * a.E;    // [E]
  int* s_off = s_counts + a.E;              // [E + 1]
  int* sh = s_off + a.E + 1;                // [AL_WAVES + 1]
  const int E = a.E;
  const ChunkState cs = tile_local_ranks(ids, 0, a.n, E, ilog2_ceil(E), hist);
  const int cnt = hist_wave_prefix(hist, E);
  int padded = 0;
  if ((int)threadIdx.x < E) padded = (cnt + a.bm - 1) / a.bm * a.bm;
  int total;
  const int ex = block_exscan(padded, sh, &total);
  if ((int)threadIdx.x < E) {
    s_counts[threadIdx.x] = cnt;
    s_off[threadIdx.x] = ex;
  }
  if (threadIdx.x == 0) s_off[E] = total;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < AL_CHUNKS_PER_WAVE; ++c) {
    const int e = cs.e[c];
    if (e < 0) continue;
    const int i = (wave * AL_CHUNKS_PER_WAVE + c) * 64 + lane;
    const int pos = s_off[e] + hist[wave * E + e] + cs.r[c];
    a.sorted_ids[pos] = i;
    a.inv_pos[i] = pos;
  }
  write_layout<true>(a, s_counts, s_off, sh);
}

// One wave aligns n <= 64 entries (ids in LDS, E <= 64 * EPL) without the
// workgroup's histogram passes: lane i holds entry i, its rank among equal
// entries below it comes from the match mask, the leader of each expert
// writes the count to LDS, and lane l owns experts EPL*l .. EPL*l + EPL - 1
// (contiguous, so one wave scan of the lanes' padded sums gives the offsets
// in expert order).  Same layout as align_one_tile (prefilled the same way,
// the prefill ordered before this wave's stores by a workgroup barrier).
// cl: E ints of LDS.
template <int EPL>
__device__ void align_one_wave(const AlignArgs& a, const int32_t* ids, int* cl) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, n = a.n, bm = a.bm;
  const bool valid = lane < n;
  const int e = valid ? ids[lane] : 0;
  uint64_t mask = ballot(valid);
  const int nbits = ilog2_ceil(E);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = ballot(valid && bit);
    mask &= bit ? m : ~m;
  }
  const int rank = __popcll(mask & lanemask_lt());
  for (int x = lane; x < E; x += 64) cl[x] = 0;
  __builtin_amdgcn_wave_barrier();
  if (valid && rank == 0) cl[e] = __popcll(mask);
  __builtin_amdgcn_wave_barrier();
  const int e0 = EPL * lane;
  int c[EPL], pad[EPL], off[EPL];
  int lsum = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    c[j] = e0 + j < E ? cl[e0 + j] : 0;
    pad[j] = (c[j] + bm - 1) / bm * bm;
    lsum += pad[j];
  }
  int inc = lsum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  const int total = __shfl(inc, 63);
  int run = inc - lsum;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    off[j] = run;
    run += pad[j];
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int ee = e0 + j;
    if (ee >= E) continue;
    a.counts[ee] = c[j];
    a.offsets[ee] = off[j];
    for (int b = off[j] / bm; b < (off[j] + pad[j]) / bm; ++b) a.block_expert[b] = ee;
  }
  if (lane == 0) a.offsets[E] = total;
  // the entry's expert offset, from its owner lane
  int oe = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int v = __shfl(off[j], e / EPL);
    if (e % EPL == j) oe = v;
  }
  if (valid) {
    a.sorted_ids[oe + rank] = lane;
    a.inv_pos[lane] = oe + rank;
  }
}

__global__ __launch_bounds__(AL_THREADS) void k_align_single(const AlignArgs a) {
  extern __shared__ int lds[];
  prefill_layout(a);
  align_one_tile(a, a.ids, lds);
}

// ================================================================ small batch
// Routing and alignment of a few tokens in one launch: wave w routes tokens
// w, w + 16, ... exactly as k_topk does (same plane order, same selection
// and weight arithmetic, so the same bits), keeping its k <= 64 selections in
// lane registers; the ids also go to LDS, from where the workgroup aligns
// them as k_align_single does.  One launch and one global round trip fewer.

// Token t's top-k from its logits v (expert lane + 64j; experts past E are
// never candidates), as k_topk selects them: k rounds of the wave argmax
// over the experts not yet taken (value descending, index ascending),
// selection r kept in lane r, weights exp(L_r - L_0) over their
// sum.  Writes ids and weights, and the ids to s_ids.
template <int V>
__device__ __forceinline__ void select_topk(const float (&v)[V], int lane, int t, int E, int k,
                                            int32_t* __restrict__ ids, float* __restrict__ wout,
                                            int* s_ids) {
  float myv = 0.f, l0 = 0.f;
  int myi = 0;
  uint32_t taken = taken_init<V>(lane, E);
  for (int r = 0; r < k; ++r) {
    float bv;
    int bi;
    pick_next<V>(v, taken, lane, bv, bi);
    if (r == 0) l0 = bv;
    if (lane == r) {
      myv = bv;
      myi = bi;
    }
  }
  float psum = lane < k ? expf(myv - l0) : 0.f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) psum += __shfl_xor(psum, off);
  const float inv = 1.0f / psum;
  if (lane < k) {
    const int64_t o = (int64_t)t * k + lane;
    ids[o] = myi;
    wout[o] = expf(myv - l0) * inv;
    s_ids[o] = myi;
  }
}

// Plane loads in batches of NB planes (64 values a lane), each batch issued
// before its adds (planes past nsplit reload the last plane and are not
// added); sums in the order of plane_sums.
template <int V, int NSMAX, int NB_ = 0>
__device__ __forceinline__ void plane_sums_all(const float* __restrict__ pp, int nsplit,
                                               int64_t split_stride, int E, int lane,
                                               float (&acc)[4][V]) {
  constexpr int NB = NB_ > 0 ? NB_ : (64 / V < NSMAX) ? 64 / V : NSMAX;
  static_assert(NB % 4 == 0 && NSMAX % NB == 0, "batches keep the plane order");
  int eo[V];
#pragma unroll
  for (int j = 0; j < V; ++j) eo[j] = min(lane + 64 * j, E - 1);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < V; ++j) acc[q][j] = 0.f;
#pragma unroll
  for (int b0 = 0; b0 < NSMAX; b0 += NB) {
    if (b0 >= nsplit) break;
    float val[NB][V];
#pragma unroll
    for (int sp = 0; sp < NB; ++sp) {
      const float* p = pp + (int64_t)min(b0 + sp, nsplit - 1) * split_stride;
#pragma unroll
      for (int j = 0; j < V; ++j) val[sp][j] = p[eo[j]];
    }
#pragma unroll
    for (int sp = 0; sp < NB; ++sp)
      if (b0 + sp < nsplit) {
#pragma unroll
        for (int j = 0; j < V; ++j) acc[sp & 3][j] += val[sp][j];
      }
  }
}

template <int V, int NT>
__global__ __launch_bounds__(NT) void k_route_align_small(
    const float* __restrict__ partial, int nsplit, int64_t split_stride,
    const float* __restrict__ bias, float* __restrict__ logits, int32_t* __restrict__ ids,
    float* __restrict__ wout, const AlignArgs a) {
  extern __shared__ int lds[];
  int* s_ids = lds;             // [n]
  int* al = lds + a.n;          // alignment scratch
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  // every wave's share of the -1 layout first: the stores drain while the
  // routing waits on its loads (the barrier after routing orders them)
  prefill_layout(a);
  // the narrow workgroup (fewer waves, more registers each) loads every
  // plane in one batch: one memory round trip instead of two at V = 4
  constexpr int NBS = NT < AL_THREADS ? ROUTER_MAX_SPLIT : 0;
  for (int t = wave; t < a.T; t += NT / 64) {
    float acc[4][V];
    plane_sums_all<V, ROUTER_MAX_SPLIT, NBS>(partial + (int64_t)t * E, nsplit, split_stride, E,
                                             lane, acc);
    float v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      v[j] = ((acc[0][j] + acc[1][j]) + acc[2][j]) + acc[3][j];
      const int e = lane + 64 * j;
      if (e < E) {
        if (bias != nullptr) v[j] += bias[e];
        if (logits != nullptr) logits[(int64_t)t * E + e] = v[j];
      } else {
        v[j] = -INFINITY;
      }
    }
    select_topk<V>(v, lane, t, E, k, ids, wout, s_ids);
  }
  __syncthreads();
  // up to 64 entries (and no tiled row list): one wave aligns them (always
  // so in the narrow workgroup)
  if (NT < AL_THREADS || (a.n <= 64 && a.tile_rows == nullptr)) {
    if (wave == 0) align_one_wave<V>(a, s_ids, al);
  } else {
    if constexpr (NT == AL_THREADS) align_one_tile(a, s_ids, al);
  }
}

hipError_t launch_route_align_small(const float* partial, int nsplit, int64_t split_stride,
                                    const float* bias, float* logits, int32_t* ids, float* w,
                                    const AlignArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  if (!route_align_small_ok(a.T, a.E, a.k, nsplit)) return hipErrorInvalidValue;
  const size_t lds =
      ((size_t)a.n + (size_t)AL_WAVES * a.E + 2 * a.E + 1 + AL_WAVES + 1) * sizeof(int);
#define MOE_RAS(V_, NT_)                                                                      \
  do {                                                                                        \
    if (lds > 65536) {                                                                        \
      hipError_t e_ = hipFuncSetAttribute((const void*)k_route_align_small<V_, NT_>,          \
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e_ != hipSuccess) return e_;                                                        \
    }                                                                                         \
    hipLaunchKernelGGL((k_route_align_small<V_, NT_>), dim3(1), dim3(NT_), lds, st, partial,  \
                       nsplit, split_stride, bias, logits, ids, w, a);                          \
  } while (0)
  // more than 128 experts (4 logits a lane, planes loaded 16 at a time with
  // 1024 threads), at most 8 tokens and 64 entries: 8 waves, all 32 planes
  // in one batch
  const bool narrow = a.E > 128 && a.T <= 8 && a.n <= 64 && a.tile_rows == nullptr;
  if (a.E <= 64) MOE_RAS(1, AL_THREADS);
  else if (a.E <= 128) MOE_RAS(2, AL_THREADS);
  else if (narrow) MOE_RAS(4, 512);
  else MOE_RAS(4, AL_THREADS);
#undef MOE_RAS
  return hipGetLastError();
}

// Multi-tile pass 1: per-tile histogram and rank of each entry in its tile.
__global__ __launch_bounds__(AL_THREADS) void k_align_hist(const AlignArgs a) {
  extern __shared__ int lds[];
  int* hist = lds;
  const int E = a.E;
  const int64_t i0 = (int64_t)blockIdx.x * ALIGN_TILE;
  const int cnt = (int)min<int64_t>(ALIGN_TILE, a.n - i0);
  const ChunkState cs = tile_local_ranks(a.ids, i0, cnt, E, ilog2_ceil(E), hist);
  const int tot = hist_wave_prefix(hist, E);
  if ((int)threadIdx.x < E) a.tile_hist[(int64_t)blockIdx.x * E + threadIdx.x] = tot;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < AL_CHUNKS_PER_WAVE; ++c) {
    const int e = cs.e[c];
    if (e < 0) continue;
    const int local = (wave * AL_CHUNKS_PER_WAVE + c) * 64 + lane;
    a.rank[i0 + local] = hist[wave * E + e] + cs.r[c];
  }
}

// Multi-tile pass 2: global counts and padded offsets (each workgroup redoes
// the small scan), then the scatter of this tile's entries; workgroup 0 also
// writes the layout arrays.
__global__ __launch_bounds__(AL_THREADS) void k_align_scatter(const AlignArgs a) {
  extern __shared__ int lds[];
  const int E = a.E;
  int* s_counts = lds;            // [E]
  int* s_off = s_counts + E;      // [E + 1]
  int* s_tbase = s_off + E + 1;   // [E]
  int* sh = s_tbase + E;          // [AL_WAVES + 1]
  const int e = threadIdx.x;
  // the tile's entries (ALIGN_TILE / AL_THREADS per thread), loaded before
  // the histogram prefix they do not depend on
  static_assert(ALIGN_TILE % AL_THREADS == 0, "entries per thread");
  constexpr int EPT = ALIGN_TILE / AL_THREADS;
  const int64_t i0 = (int64_t)blockIdx.x * ALIGN_TILE;
  const int cntt = (int)min<int64_t>(ALIGN_TILE, a.n - i0);
  int eid[EPT], erk[EPT];
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    const int l = threadIdx.x + u * AL_THREADS;
    eid[u] = l < cntt ? a.ids[i0 + l] : 0;
    erk[u] = l < cntt ? a.rank[i0 + l] : 0;
  }
  int cnt = 0, before = 0;
  if (e < E) {
    // sixteen tiles' counts in flight at a time (integer sums: any order)
    for (int t0 = 0; t0 < a.ntiles; t0 += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        c[u] = t0 + u < a.ntiles ? a.tile_hist[(int64_t)(t0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (t0 + u < (int)blockIdx.x) before += c[u];
        cnt += c[u];
      }
    }
  }
  const int padded = (e < E) ? (cnt + a.bm - 1) / a.bm * a.bm : 0;
  int total;
  const int ex = block_exscan(padded, sh, &total);
  if (e < E) {
    s_counts[e] = cnt;
    s_off[e] = ex;
    s_tbase[e] = ex + before;
  }
  if (threadIdx.x == 0) s_off[E] = total;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    const int l = threadIdx.x + u * AL_THREADS;
    if (l < cntt) {
      const int64_t i = i0 + l;
      const int pos = s_tbase[eid[u]] + erk[u];
      a.sorted_ids[pos] = (int)i;
      a.inv_pos[i] = pos;
    }
  }
  if (blockIdx.x == 0) write_layout<false>(a, s_counts, s_off, sh);
}

int64_t align_workspace_bytes(int n, int E) {
  if (n <= ALIGN_SINGLE_MAX) return 0;
  const int64_t ntiles = (n + ALIGN_TILE - 1) / ALIGN_TILE;
  const int64_t hist = ntiles * E * 4;
  return ((hist + 255) / 256) * 256 + (int64_t)n * 4;
}

hipError_t launch_align(AlignArgs a, void* ws, hipStream_t st) {
  if (a.n == 0) {
    return hipSuccess;
  }
  if (a.n <= ALIGN_SINGLE_MAX) {
    const size_t lds = ((size_t)AL_WAVES * a.E + 2 * a.E + 1 + AL_WAVES + 1) * 4;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)k_align_single,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_align_single, dim3(1), dim3(AL_THREADS), lds, st, a);
    return hipGetLastError();
  }
  a.ntiles = (a.n + ALIGN_TILE - 1) / ALIGN_TILE;
  const int64_t hist = (int64_t)a.ntiles * a.E * 4;
  a.tile_hist = reinterpret_cast<int32_t*>(ws);
  a.rank = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + ((hist + 255) / 256) * 256);
  const size_t lds1 = (size_t)AL_WAVES * a.E * 4;
  if (lds1 > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k_align_hist,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_align_hist, dim3(a.ntiles), dim3(AL_THREADS), lds1, st, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds2 = ((size_t)3 * a.E + 1 + AL_WAVES + 1) * 4;
  hipLaunchKernelGGL(k_align_scatter, dim3(a.ntiles), dim3(AL_THREADS), lds2, st, a);
  return hipGetLastError();
}

}  // namespace moe
