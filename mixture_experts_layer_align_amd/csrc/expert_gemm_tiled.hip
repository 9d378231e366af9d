// LDS-tiled grouped expert GEMM for thick token blocks (prefill regime).
//
// With many rows per expert the expert GEMMs are bound by the matrix cores
// ("CuTeDSL at Perplexity", prefill/decode section: prefill GEMMs are
// compute-bound), so the kernel is a classic tiled GEMM on the MFMA units:
//
//   * a workgroup (4 waves, 2 x 2) computes a BM-row block of one expert (the
//     aligned, padded slot list; BM = 128 or 256) against 256 weight columns —
//     for gate|up the 128 gate columns of its h-tile and the matching 128 up
//     columns, so SiLU(g)*u is applied to the fp32 accumulators in registers
//     before the single store of h ("La fusion de noyaux", section 4.2, GEMM +
//     epilogue; the concatenated d x 2*d_ff gate|up); each wave owns a
//     (BM/2) x 128 sub-tile;
//   * K advances 64 at a time through an LDS pipeline (2 or 3 stages) filled by
//     direct loads (global_load_lds_dwordx4): the token tile is gathered row
//     by row from x by slot (the permuted activations are never
//     materialised), the weight tile is copied untransposed ([K, N], N
//     contiguous, the B[K,N] of the vLLM post's A[M,K] x B[K,N]);
//   * within a stage the two 32-deep k-steps' fragments are read into two
//     register sets, so the second step's LDS reads run under the first
//     step's MFMAs (reads and waits are counted explicitly);
//   * the weight operand's K-contiguous MFMA fragments come from gfx950's
//     transposing LDS read (ds_read_b64_tr_b16: within each 16-lane group,
//     lane i receives element i%4 of the 8-byte pieces addressed by lanes
//     4v + i/4, v = 0..3 — so lanes that address 4 consecutive rows x 16
//     columns hand lane i column i of those rows), two per
//     v_mfma_f32_16x16x32_bf16 fragment;
//   * both LDS tiles are XOR-swizzled per row so the fragment reads hit
//     distinct banks;
//   * consecutive workgroups walk 8 row blocks before the next weight tile,
//     so a weight tile is fetched from HBM once for up to 8 row blocks and a
//     token block stays resident in its XCD's L2 across its weight tiles.
#include <type_traits>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int TBN = 256;  // weight columns per tile
constexpr int TBK = 64;   // k per pipeline stage
constexpr int GROUP_M = 8;
constexpr int B_STAGE_BYTES = TBK * TBN * 2;            // 32 KB
constexpr int B_DMA_PER_THREAD = TBK * (TBN / 8) / 256;  // 8

template <int BM>
struct TCfg {
  static constexpr int STAGES = BM == 256 ? 2 : 3;
  static constexpr int A_STAGE_BYTES = BM * TBK * 2;
  static constexpr int STAGE_BYTES = A_STAGE_BYTES + B_STAGE_BYTES;
  static constexpr int A_DMA_PER_THREAD = BM * (TBK / 8) / 256;
  static constexpr int DMA_PER_STAGE = A_DMA_PER_THREAD + B_DMA_PER_THREAD;
  static constexpr int MI = BM / 32;                   // 16-row fragments per wave
  static constexpr int READS_PER_KSTEP = MI + 16;      // LDS reads per wave per k-step
};

constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14);
}

// swizzles: chunk position of logical 16-byte chunk c in row r
__device__ __forceinline__ int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_b(int r) { return 2 * ((r & 3) | ((r >> 1) & 4)); }

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
// transposing read of 8 bytes (four 16-bit elements)
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}

template <int MI>
struct Frags {
  u32x4 a[MI];
  u32x2 bl[8], bh[8];
};

// s_waitcnt lgkmcnt(N) with the fragment registers tied to it, so nothing
// that reads them can be scheduled before the wait
template <int N, int MI>
__device__ __forceinline__ void wait_frags(Frags<MI>& f) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
#pragma unroll
  for (int i = 0; i < MI; ++i) asm volatile("" : "+v"(f.a[i]));
  asm volatile("s_waitcnt lgkmcnt(%16)"
               : "+v"(f.bl[0]), "+v"(f.bl[1]), "+v"(f.bl[2]), "+v"(f.bl[3]), "+v"(f.bl[4]),
                 "+v"(f.bl[5]), "+v"(f.bl[6]), "+v"(f.bl[7]), "+v"(f.bh[0]), "+v"(f.bh[1]),
                 "+v"(f.bh[2]), "+v"(f.bh[3]), "+v"(f.bh[4]), "+v"(f.bh[5]), "+v"(f.bh[6]),
                 "+v"(f.bh[7])
               : "n"(N));
#pragma unroll
  for (int i = 0; i < MI; ++i) asm volatile("" : "+v"(f.a[i]));
}

}  // namespace

template <int EPI, int BM>
__global__ __launch_bounds__(256) void k_expert_tiled(const StreamGemmArgs p) {
  using C = TCfg<BM>;
  constexpr int S = C::STAGES;
  constexpr int MI = C::MI;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ---------------------------------------------------- tile of this workgroup
  // groups of GROUP_M row blocks: row block fastest, then weight tile
  const int id = blockIdx.x;
  const int per_group = GROUP_M * p.n_tiles;
  const int grp = id / per_group;
  const int first_mb = grp * GROUP_M;
  const int gm = min(GROUP_M, p.num_mblocks - first_mb);
  const int local = id - grp * per_group;
  const int mb = first_mb + local % gm;
  const int nt = local / gm;
  const int e = p.block_expert[mb];
  if (e < 0) return;
  const int p0 = mb * BM;

  // ---------------------------------------------------- DMA source addresses
  // A: slot s = (wave*A_DMA + i)*64 + lane -> row s/8, position s%8; the
  // lane's row index (token, or h row) is kept, the chunk is recomputed
  int a_row[C::A_DMA_PER_THREAD];
#pragma unroll
  for (int i = 0; i < C::A_DMA_PER_THREAD; ++i) {
    const int r = ((wave * C::A_DMA_PER_THREAD + i) * 64 + lane) >> 3;
    const int sid = p.sorted_ids[p0 + r];
    int row = 0;  // padding rows read row 0; their results are never stored
    if (sid >= 0) row = (p.a_mode == A_GATHER) ? sid / p.topk : p0 + r;
    a_row[i] = row;
  }
  // A rows are 8 chunks, so slot s's row is s/8 and its chunk position s%8 =
  // lane%8 for every i (the 64-lane blocks start at multiples of 8 rows)
  const int a_pos = lane & 7;
  const char* xa = reinterpret_cast<const char*>(p.a);
  const char* wexp = reinterpret_cast<const char*>(p.w) + (int64_t)e * p.w_estride * 2;
  const int nk = p.K / TBK;

  auto issue = [&](int stage, int kt) __attribute__((always_inline)) {
    char* sa = lds + stage * C::STAGE_BYTES;
    char* sb = sa + C::A_STAGE_BYTES;
    const int64_t k0 = (int64_t)kt * TBK;
#pragma unroll
    for (int i = 0; i < C::A_DMA_PER_THREAD; ++i) {
      const int r = ((wave * C::A_DMA_PER_THREAD + i) * 64 + lane) >> 3;
      const int c = a_pos ^ swz_a(r);
      dma16(xa + ((int64_t)a_row[i] * p.a_ld + k0 + 8 * c) * 2,
            sa + (wave * C::A_DMA_PER_THREAD + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < B_DMA_PER_THREAD; ++i) {
      // B slot s = (wave*8 + i)*64 + lane -> row s/32, position s%32
      const int r = (wave * B_DMA_PER_THREAD + i) * 2 + (lane >> 5);
      const int c = (lane & 31) ^ swz_b(r);
      int col;
      if constexpr (EPI == EPI_SILU_MUL)
        col = (c < 16) ? nt * 128 + 8 * c : p.up_off + nt * 128 + 8 * (c - 16);
      else
        col = nt * TBN + 8 * c;
      dma16(wexp + ((k0 + r) * p.w_ld + col) * 2, sb + (wave * B_DMA_PER_THREAD + i) * 1024);
    }
  };

  // ---------------------------------------------------- fragment addresses
  // A fragment mi, k-step ks: row R = wm*BM/2 + mi*16 + lane%16, chunk
  // ks*4 + lane/16.  R%16 = lane%16, so the swizzle is the lane's own and the
  // address is a per-lane base (one per ks) plus the immediate mi*2048.
  const int lm = lane & 15, lg = lane >> 4;
  const uint32_t lds_base = lds_off(lds);
  uint32_t a_base[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    a_base[ks] = (uint32_t)(((wm * (BM / 2) + lm) * 8 + ((ks * 4 + lg) ^ swz_a(lm))) * 16);
  // B fragment ni, k-step ks, half h: row kr = ks*32 + 8*lg + lm/4 + 4h,
  // chunk c0(ni) + (lm%4)/2, 8-byte half lm&1.  swz_b(kr) depends only on
  // lm/4 and lg&1, so it is the lane's own; ks and h are immediates.
  const int xb = swz_b(8 * lg + (lm >> 2));
  uint32_t b_base[8];
#pragma unroll
  for (int ni = 0; ni < 8; ++ni) {
    int c0;
    if constexpr (EPI == EPI_SILU_MUL)
      c0 = ni < 4 ? 2 * (wn * 4 + ni) : 16 + 2 * (wn * 4 + ni - 4);
    else
      c0 = 2 * (wn * 8 + ni);
    const int row = 8 * lg + (lm >> 2);
    b_base[ni] = (uint32_t)((row * 32 + ((c0 ^ xb) + ((lm & 3) >> 1))) * 16 + (lm & 1) * 8);
  }

  auto read_frags = [&](Frags<MI>& f, uint32_t sa, uint32_t sb, auto ks_c)
                        __attribute__((always_inline)) {
    constexpr int ks = decltype(ks_c)::value;
    const uint32_t ab = sa + a_base[ks];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      // unrolled: mi is a compile-time constant, so is the offset
      switch (mi) {
        case 0: f.a[0] = lds_read_b128<0>(ab); break;
        case 1: f.a[1] = lds_read_b128<2048>(ab); break;
        case 2: f.a[2] = lds_read_b128<4096>(ab); break;
        case 3: f.a[3] = lds_read_b128<6144>(ab); break;
        case 4: f.a[4 % MI] = lds_read_b128<8192>(ab); break;
        case 5: f.a[5 % MI] = lds_read_b128<10240>(ab); break;
        case 6: f.a[6 % MI] = lds_read_b128<12288>(ab); break;
        case 7: f.a[7 % MI] = lds_read_b128<14336>(ab); break;
      }
    }
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      const uint32_t bb = sb + b_base[ni];
      f.bl[ni] = lds_read_tr16<ks * 32 * 512>(bb);
      f.bh[ni] = lds_read_tr16<ks * 32 * 512 + 4 * 512>(bb);
    }
  };

  f32x4 acc[MI][8];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfmas = [&](const Frags<MI>& f) __attribute__((always_inline)) {
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      const u32x4 bf = {f.bl[ni][0], f.bl[ni][1], f.bh[ni][0], f.bh[ni][1]};
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) acc[mi][ni] = mfma_bf16_16x16x32(f.a[mi], bf, acc[mi][ni]);
    }
  };

  // ---------------------------------------------------- main loop
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s);
  Frags<MI> f0, f1;
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt landed for every wave (the stages issued after it may still
    // be in flight); a bare barrier, since a full __syncthreads would also
    // wait for those
    if (S == 3 && kt + 1 < nk)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::DMA_PER_STAGE));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    // refill the stage consumed in the previous iteration
    if (kt + S - 1 < nk) issue((kt + S - 1) % S, kt + S - 1);
    const uint32_t sa = lds_base + (kt % S) * C::STAGE_BYTES;
    const uint32_t sb = sa + C::A_STAGE_BYTES;
    read_frags(f0, sa, sb, std::integral_constant<int, 0>{});
    read_frags(f1, sa, sb, std::integral_constant<int, 1>{});
    wait_frags<C::READS_PER_KSTEP < 16 ? C::READS_PER_KSTEP : 15>(f0);
    mfmas(f0);
    wait_frags<0>(f1);
    mfmas(f1);
  }

  // ---------------------------------------------------- epilogue
  // acc[mi][ni]: lane (n = lane%16, g = lane/16) holds rows 4g + r of the 16x16
  // block (mi, ni)
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lrow = wm * (BM / 2) + mi * 16 + 4 * lg + r;
      if (p.sorted_ids[p0 + lrow] < 0) continue;
      const int64_t prow = p0 + lrow;
      if constexpr (EPI == EPI_SILU_MUL) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + prow * p.out_ld + nt * 128 + wn * 64 + lm;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const float hv = silu(acc[mi][ni][r]) * acc[mi][ni + 4][r];
          dst[ni * 16] = (uint16_t)f32_to_bf16_bits(hv);
        }
      } else {
        float* dst = reinterpret_cast<float*>(p.out) + prow * p.out_ld + nt * TBN + wn * 128 + lm;
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) dst[ni * 16] = acc[mi][ni][r];
      }
    }
}

template <int EPI, int BM>
static hipError_t launch_tiled(const StreamGemmArgs& a, hipStream_t st) {
  const int64_t grid = (int64_t)a.num_mblocks * a.n_tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = (size_t)TCfg<BM>::STAGES * TCfg<BM>::STAGE_BYTES;
  hipError_t e = hipFuncSetAttribute((const void*)k_expert_tiled<EPI, BM>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_expert_tiled<EPI, BM>), dim3((unsigned)grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_tiled_gemm(int epi, int bm, const StreamGemmArgs& a, hipStream_t st) {
  if (bm == 256)
    return epi == EPI_SILU_MUL ? launch_tiled<EPI_SILU_MUL, 256>(a, st)
                               : launch_tiled<EPI_STORE, 256>(a, st);
  if (bm == 128)
    return epi == EPI_SILU_MUL ? launch_tiled<EPI_SILU_MUL, 128>(a, st)
                               : launch_tiled<EPI_STORE, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
