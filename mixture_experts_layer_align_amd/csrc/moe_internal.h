// Host-side launch interface between the C ABI (moe_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int MAX_EXPERTS = 1024;

enum { ACT_F32 = 0, ACT_BF16 = 1 };             // activation storage
enum { W_F32 = 0, W_BF16 = 1, W_FP8 = 2, W_FP4 = 3, W_MXFP8 = 4 };  // expert-weight storage
// W_FP4: MXFP4 — E2M1 codes two per byte along K (even k in the low nibble),
// one E8M0 scale byte per 32 consecutive k of a column (`scale` points to
// bytes, scale_estride counts bytes).

// ------------------------------------------------------------ stream GEMMs
//
// Weight-streaming GEMMs: one two-wave workgroup per work item (m-block of 32
// rows, n-tile, k-split).  Every wave streams one column slab of its k-range
// once and multiplies it with all rows of its block.  The expert GEMMs stage
// weights through LDS with direct loads; the router GEMM (N = E, any width)
// stages them in registers.

enum { A_DENSE = 0,    // row p = input row p, valid when p < m_total
       A_GATHER = 1,   // row p = input row sorted_ids[p] / topk, valid when >= 0
       A_PADDED = 2 }; // row p = input row p, valid when sorted_ids[p] >= 0

enum { EPI_SILU_MUL = 0,  // two slabs (gate, up) -> act dtype  h = silu(g)*u
       EPI_STORE = 1 };   // two adjacent slabs -> fp32

struct StreamGemmArgs {
  const void* a;          // row source
  const void* a_lo;       // bf16 rows only: the low halves of rows carried as a pair of
                          //   bf16 (value = a + a_lo, same layout), or NULL
  int64_t a_ld;           // elements
  // EPI_STORE: the gate|up k-split partial sums [a_part_nsplit][rows][a_part_ld]
  // (gate columns [0, K), up columns [K, 2K)), or NULL.  Given, each item first
  // forms h = SiLU(sum of gate partials) * (sum of up partials) for its block's
  // routed rows over its k-range, splits added in order, and writes it into a
  // (and a_lo), where its main loop then reads its rows.
  const float* a_part;
  int a_part_nsplit;
  int64_t a_part_ld;
  int64_t a_part_stride;
  int a_mode;
  const int32_t* sorted_ids;
  int topk;
  int m_total;            // A_DENSE: valid row count
  const int32_t* block_expert;  // NULL: dense, expert 0
  int num_mblocks;
  const int32_t* padded_rows;   // device count of rows in use, or NULL (all)
  const void* w;          // weights [E][K][w_ld]
  int64_t w_ld;
  int64_t w_estride;
  const float* scale;     // fp8: [E][scale_ld] per weight column, else NULL
  int64_t scale_estride;
  int K;
  int n_out;              // output columns
  int up_off;             // EPI_SILU_MUL: column of the first "up" weight column
  int n_tiles;
  int ksplit;
  int kchunk;
  float* partial;         // ksplit > 1: fp32 partial sums [ksplit][rows][partial_ld]
  int64_t partial_ld;     //   (columns in the weight's N space)
  int64_t partial_split_stride;
  void* out;
  void* out_lo;           // EPI_SILU_MUL, bf16: also store h's low halves here
                          //   (bf16(h - bf16(h)), layout of out), or NULL
  int64_t out_ld;
  int64_t out_split_stride;  // router: elements between split planes
  int wgs;                // stream GEMM: workgroups, each looping over items
                          //   g, g + wgs, ...; 0 = one workgroup per item
  int halves;             // stream GEMM: 32-row blocks per item (1, or 2: an item
                          //   applies one weight stream to a pair of its expert's
                          //   blocks, and needs expert_offsets)
  const int32_t* expert_offsets;  // halves == 2: the alignment's padded offsets [E + 1]
  const int32_t* tile_rows;    // tiled GEMM: [rows][2] = {first slot, expert | routed
                               //   slots << 16}, full rows (256 slots) first, then half
                               //   rows (128 slots); routed slots are the row's first ones
  const int32_t* tile_counts;  // tiled GEMM: {full rows, half rows} (device)
  int32_t* die_next;           // tiled GEMM: 8 per-die tile counters, zero at launch
};

// Compute units of the current device (cached per device; 256 if the query
// fails).
int device_cus();

// Rows per m-block of the stream GEMM (two 16-row MFMA column groups).
constexpr int STREAM_BM = 32;
// routed entries per expert (on average) from which fp8 weights take 64-row
// stream blocks
constexpr int STREAM_HALVES_MIN = 4;

// Output columns covered by one n-tile of the stream GEMM.
int stream_tile_cols(int w_dtype, int epi);
// K granularity of one k-step.
int stream_kstep(int w_dtype);

hipError_t launch_stream_gemm(int act_dtype, int w_dtype, int epi, const StreamGemmArgs& a,
                              hipStream_t st);

// LDS-tiled MFMA grouped GEMM (thick blocks): tile rows of 256 (and 128
// with bm = 128) x 256 weight columns, bf16 activations, bf16 or fp8
// weights, K a multiple of 64; EPI_SILU_MUL needs d_ff % 128 == 0 and one
// split, EPI_STORE n_out % 256 == 0; every split at least TILED_MIN_KCHUNK
// deep (more k-steps than the kernel's LDS stages).
constexpr int TILED_BN = 256;
constexpr int TILED_MIN_KCHUNK = 256;
hipError_t launch_tiled_gemm(int epi, int w_dtype, int bm, const StreamGemmArgs& a,
                             hipStream_t st);

// Router logits: A_DENSE rows, weights [K, n_out] with any n_out; split s writes
// the fp32 plane out + s * out_split_stride.
int router_tile_cols(int act_dtype);
int router_slab_cols(int act_dtype);
int router_kstep(int act_dtype);
hipError_t launch_router_gemm(int act_dtype, const StreamGemmArgs& a, hipStream_t st);

// ------------------------------------------------------------ routing

// Sum split-K partial logits, add bias, write logits (optional), select top-k
// with ties to the lower index and renormalised softmax weights.
hipError_t launch_topk(const float* partial, int nsplit, int64_t split_stride, const float* bias,
                       int T, int E, int k, float* logits, int32_t* ids, float* w, hipStream_t st);

// ------------------------------------------------------------ alignment

struct AlignArgs {
  const int32_t* ids;
  int n;             // T * k entries
  int T, E, k, bm;
  int64_t cap;       // padded capacity (rows)
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_ids;
  int32_t* inv_pos;
  int32_t* block_expert;
  // optional (NULL: not written): the row list of the tiled expert GEMM.  An
  // expert's padded slots are cut into 256-slot rows, the last one 128 slots
  // when 128 remain (bm = 128); full rows are listed first, then half rows,
  // each as {first slot, expert | routed slots of the row << 16}; tile_counts = {full rows, half rows, then
  // TILE_COUNTERS zeros: the two tiled GEMMs' per-die tile counters}
  int32_t* tile_rows;
  int32_t* tile_counts;
  // multi-tile scratch
  int32_t* tile_hist;   // [ntiles][E]
  int32_t* rank;        // [n]
  int ntiles;
};

constexpr int TILE_COUNTERS = 16;

constexpr int ALIGN_SINGLE_MAX = 4096;   // entries one workgroup aligns alone
constexpr int ALIGN_TILE = 4096;         // entries per tile of the multi-pass path

int64_t align_workspace_bytes(int n, int E);
hipError_t launch_align(AlignArgs a, void* ws, hipStream_t st);

// Router: at most this many fp32 partial planes over d.
constexpr int ROUTER_MAX_SPLIT = 32;

// Top-k of the router planes and the alignment in one single-workgroup launch
// (ids receives the ids; a.ids is not read); for T <= ROUTE_ALIGN_SMALL_MAX_T,
// E <= 256, k <= 64.  Above 16 tokens the waves route tokens one after another
// and the many-workgroup top-k plus alignment measured faster (T=64: 20.7 vs
// 15.7 us).
constexpr int ROUTE_ALIGN_SMALL_MAX_T = 16;
inline bool route_align_small_ok(int T, int E, int k, int nsplit) {
  return T >= 1 && T <= ROUTE_ALIGN_SMALL_MAX_T && E <= 256 && k <= 64 && nsplit >= 1 &&
         nsplit <= ROUTER_MAX_SPLIT;
}
hipError_t launch_route_align_small(const float* partial, int nsplit, int64_t split_stride,
                                    const float* bias, float* logits, int32_t* ids, float* w,
                                    const AlignArgs& a, hipStream_t st);

// ------------------------------------------------------------ combine

// y: per-slot expert outputs [nsplit][cap, d] (k-split partial sums, added in
// split order before the weighting), fp32 or, with y_f16, fp16
hipError_t launch_combine(int act_dtype, const void* y, bool y_f16, int nsplit,
                          int64_t split_stride, const int32_t* inv_pos, const float* w, int T,
                          int k, int d, void* out, hipStream_t st);

// ------------------------------------------------------------ RMS norms

// In-place per-head RMS normalisation of q [T, nq, head_dim] and k [T, nk,
// head_dim] (weights [head_dim] each, all in the activation dtype).
hipError_t launch_qk_norm(int act_dtype, void* q, void* k, const void* wq, const void* wk, int T,
                          int nq, int nk, int head_dim, float weight_bias, float eps,
                          hipStream_t st);
// Row RMSNorm of x [T, d] into y [T, d] (y may be x), gain [d].  d * element
// size must be a multiple of 16 bytes and at most RMS_MAX_ROW_BYTES.
constexpr int RMS_MAX_ROW_BYTES = 32768;
hipError_t launch_rms_norm(int act_dtype, const void* x, const void* w, void* y, int T, int d,
                           float weight_bias, float eps, hipStream_t st);

// MXFP8 codes [rows][n] and E8M0 scale bytes [rows][n/32] of x [rows][n]
// (bf16 or fp32, n % 32 == 0).
hipError_t launch_mx_quant(int act_dtype, const void* x, void* codes, void* scales, int64_t rows,
                           int n, hipStream_t st);

}  // namespace moe
