/*
 * libmoe — fused Mixture-of-Experts layer forward for AMD Instinct MI355X
 * (gfx950).  C ABI.
 *
 * The layer, per token t with hidden vector x[t] (length d):
 *   1. router logits   L[t, e] = sum_i x[t, i] * W_r[i, e] + bias[e]
 *   2. routing         ids[t, 0..k-1] = the k largest logits, slot j holding the
 *                      j-th largest (ties to the lower expert index), and
 *                      w[t, j] = softmax(L[t])[ids[t, j]] renormalised over the
 *                      k selected experts (so the k weights sum to 1);
 *   3. alignment       a per-expert count of the routed (t, j) entries and a
 *                      unique slot for each entry inside its expert's padded
 *                      range of the expert-sorted row buffer;
 *   4. gate|up GEMM    h[p] = SiLU(x[t] W_gate[e]) * (x[t] W_up[e]) for every
 *                      slot p holding entry (t, j) of expert e;
 *   5. down GEMM       y[p] = h[p] W_down[e];
 *   6. combine         out[t] = sum_j w[t, j] * y[slot of (t, j)].
 *
 * Sources: "CuTeDSL at Perplexity", section on MoE dispatch and combine, local
 * (TP=1) kernel (routing table, per-expert counts, a unique index per token in
 * its expert's list, optionally padded per-expert buffers, a combine that
 * accumulates weighted expert outputs from those positions); the vLLM fused-MoE
 * post, section "Swap-AB" (expert compute A[M,K] x B[K,N] -> C[M,N], so expert
 * weights are stored [K, N]); "La fusion de noyaux", section 4.2 (SwiGLU and the
 * concatenated d x 2*d_ff gate|up GEMM with the activation applied in the GEMM
 * epilogue).  The router rule (softmax, top-k with ties to the lower index,
 * renormalisation) is the workload statement's; the pages leave it open.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise; arrays are dense,
 *     row-major, and 16-byte aligned (routing arrays of int32/fp32 and the
 *     logit bias need only 4, MXFP8 codes 8 and their scale bytes 4); a
 *     misaligned pointer returns MOE_ERR_INVALID.  `stream` is a hipStream_t (NULL: the
 *     default stream).  All work is enqueued on `stream`; the library never
 *     synchronises, never allocates or frees device memory and never prints.
 *     Outputs are valid once the stream reaches that point.
 *   - The caller owns every buffer.  Weights are read-only and must outlive the
 *     enqueued work.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued.  A launch failure reported by the runtime
 *     returns MOE_ERR_DEVICE; faults inside kernels surface at the caller's
 *     next synchronisation.
 *   - T == 0 is valid and enqueues nothing.
 *   - Workspace: entry points that need scratch take (workspace,
 *     workspace_bytes).  With workspace == NULL the call only writes the
 *     required size to *workspace_bytes and returns MOE_OK.  Otherwise
 *     *workspace_bytes must be at least that size (MOE_ERR_WORKSPACE if not)
 *     and the workspace must be 256-byte aligned.  Its contents on entry do not
 *     matter.  Calls that overlap in time must not share a workspace.
 *   - Results are deterministic: integer outputs never depend on scheduling
 *     (no atomics decide an order), and floating-point sums run in a fixed
 *     order, so a repeated call gives bitwise-identical outputs.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,      /* NULL required pointer, bad size or range      */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but not built: dtype mix, shape modulus */
  MOE_ERR_WORKSPACE = -3,    /* workspace smaller than required, or misaligned */
  MOE_ERR_DEVICE = -4,       /* the HIP runtime refused a launch or query     */
  MOE_ERR_SCRATCH = -5       /* moe_forward_noalloc: the call needs more than
                                MOE_NOALLOC_SCRATCH_BYTES of scratch          */
} moe_status;

typedef enum {
  MOE_F32 = 0,        /* IEEE binary32                                       */
  MOE_BF16 = 1,       /* bfloat16                                            */
  MOE_FP8_E4M3 = 2,   /* OCP FP8 E4M3 ("e4m3fn": max 448, no infinities)     */
  MOE_MXFP4 = 3,      /* OCP MX FP4: E2M1 codes + one E8M0 scale per 32 k    */
  MOE_MXFP8 = 4       /* OCP MX FP8: e4m3fn codes + one E8M0 scale per 32 k  */
} moe_dtype;

/* Supported dtype combinations (activation / router weight, expert weight):
 * (F32, F32), (BF16, BF16), (BF16, FP8_E4M3), (BF16, MXFP4), (BF16, MXFP8).
 * FP8 expert
 * weights carry one fp32 scale per expert and output column; the GEMM
 * multiplies its fp32 accumulator by that scale in the epilogue
 * (W = code * scale).
 * MXFP4 (the microscaling variant the CuTeDSL post names, with the OCP MX
 * encodings): W[k, n] = e2m1(code[k, n]) * 2^(s[k/32, n] - 127); codes are
 * stored two per byte along K (byte [k/2, n]: even k in the low nibble,
 * k+1 in the high nibble), so an [K, N] weight is K/2 x N bytes; the E8M0
 * scale bytes s are [K/32, N].  E2M1 codes 0..7 are the magnitudes 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6, code | 8 their negatives.  Scale bytes must lie in
 * [1, 254] (0 is read as a zero scale, 255 is not allowed).
 * MXFP8: W[k, n] = e4m3fn(code[k, n]) * 2^(s[k/32, n] - 127); one code byte
 * per element ([K, N] like FP8), scale bytes [K/32, N] as for MXFP4.
 * The expert GEMMs convert MX codes to bf16 exactly (scale applied in the
 * conversion) and run the bf16 MFMA; MX layers always take the
 * weight-streaming GEMM.                                                     */

/* Allowed alignment block sizes (rows of one padded block). */
#define MOE_BLOCK_M_MIN 16
#define MOE_BLOCK_M_MAX 256
#define MOE_MAX_EXPERTS 1024
/* Routed entries T*k per call must stay below this (int32 slot indices with
 * room for padding); larger calls return MOE_ERR_INVALID. */
#define MOE_MAX_ENTRIES (1 << 24)

/* Rows of the padded, expert-sorted buffer for T tokens, E experts, top-k and
 * block size bm: each active expert pads its count to a multiple of bm and at
 * most min(E, T*k) experts are active, so
 *   capacity = bm * floor((T*k + min(E, T*k) * (bm - 1)) / bm).
 * Host function; returns -1 for invalid arguments.                           */
int64_t moe_align_capacity(int T, int E, int k, int block_m);

/* ---------------------------------------------------------------------------
 * moe_route — steps 1 and 2 (router logits, softmax, top-k, renormalisation).
 * "CuTeDSL at Perplexity", MoE dispatch and combine: the router's routing
 * table that dispatch consumes; rule from the workload statement.
 *
 *   x          [T, d]  act_dtype (MOE_F32 or MOE_BF16)
 *   w_router   [d, E]  act_dtype
 *   logit_bias [E]     fp32, added to every token's logits before selection
 *                      and softmax; NULL for none
 *   logits     [T, E]  fp32 out (bias included), or NULL
 *   topk_ids   [T, k]  int32 out; slot j = j-th largest logit, ties -> lower id
 *   topk_w     [T, k]  fp32 out; softmax over E restricted to the selected
 *                      experts and renormalised to sum 1
 * Logits accumulate in fp32; the top-k decision is taken on those fp32 values.
 * Limits: 1 <= k <= E <= MOE_MAX_EXPERTS, d % 64 == 0, T >= 0,
 * T * k < MOE_MAX_ENTRIES.
 * ------------------------------------------------------------------------- */
int moe_route(const void* x, const void* w_router, const float* logit_bias,
              int T, int d, int E, int k, int act_dtype,
              float* logits, int32_t* topk_ids, float* topk_w,
              void* workspace, size_t* workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_align — step 3 (histogram -> padded exclusive scan -> stable scatter).
 * "CuTeDSL at Perplexity", MoE dispatch and combine, local kernel: count the
 * tokens routed to each expert, give each a unique index in its expert's list,
 * lay the lists out in optionally padded per-expert buffers.
 *
 *   topk_ids       [T, k] int32 in, every id in [0, E), distinct within a row
 *   expert_counts  [E]    int32 out: entries routed to each expert
 *   padded_offsets [E+1]  int32 out: 0, then running sum of counts rounded up
 *                         to a multiple of block_m
 *   sorted_ids     [cap]  int32 out, cap = moe_align_capacity(T, E, k, block_m):
 *                         sorted_ids[padded_offsets[e] + r] = t*k + j for the
 *                         r-th entry (in ascending t*k + j) routed to e; every
 *                         other slot = -1
 *   inv_pos        [T*k]  int32 out: the slot of entry t*k + j
 *   block_expert   [cap/block_m] int32 out: expert owning each block_m-row
 *                         block, -1 for blocks at or past padded_offsets[E]
 * block_m must be a power of two in [MOE_BLOCK_M_MIN, MOE_BLOCK_M_MAX];
 * 1 <= k <= E <= MOE_MAX_EXPERTS, T * k < MOE_MAX_ENTRIES (else MOE_ERR_INVALID).
 * No atomics decide the order: the result is unique and reproducible.
 * Out-of-range ids are a caller error (not checked on the device).
 * ------------------------------------------------------------------------- */
int moe_align(const int32_t* topk_ids, int T, int E, int k, int block_m,
              int32_t* expert_counts, int32_t* padded_offsets,
              int32_t* sorted_ids, int32_t* inv_pos, int32_t* block_expert,
              void* workspace, size_t* workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_forward — the whole layer, steps 1-6.
 * Expert GEMMs follow the A[M,K] x B[K,N] statement of the vLLM fused-MoE post
 * (section "Swap-AB"): B = expert weight [K, N], N contiguous.  Gate and up are
 * concatenated into one [d, 2*d_ff] matrix, gate columns first ("La fusion de
 * noyaux", section 4.2); SiLU(g)*u is applied to the fp32 accumulators before
 * the single store of h.  The top-k weights are applied in the combine.
 * Intermediates: fp32 throughout for fp32 activations.  For bf16
 * activations h keeps more significant bits than bf16 holds: a pair of bf16
 * (h's high and low halves, 16 significant bits) for thin blocks (the
 * weight-streaming GEMMs of decode batches), with the per-slot expert outputs
 * y in fp32; fp16 (11 significant bits) for thick blocks (the MFMA-tiled
 * GEMMs of prefill batches), where y is fp16 too.  On that path |h| and |y|
 * must stay below 65504, beyond which the output shows infinities.  With one bf16 rounding of h, rows of d = 4096 and 7168 layers
 * measured up to 2.2e-2 * RMS off the exact result against a 2e-2 bound,
 * where the output's own rounding alone stays at 1.74e-2.
 * ------------------------------------------------------------------------- */
typedef struct {
  int d, d_ff, E, k;
  int act_dtype;                /* MOE_F32 or MOE_BF16: x, out, w_router      */
  int w_dtype;                  /* MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4,
                                   MOE_MXFP8                                   */
  const void* w_router;         /* [d, E] act_dtype                           */
  const float* logit_bias;      /* [E] fp32 or NULL                           */
  const void* w_gate_up;        /* [E, d, 2*d_ff]; cols [0,d_ff) gate,
                                   [d_ff, 2*d_ff) up  (MXFP4: [E, d/2, 2*d_ff]
                                   bytes)                                      */
  const void* w_down;           /* [E, d_ff, d]  (MXFP4: [E, d_ff/2, d] bytes) */
  const void* scale_gate_up;    /* FP8: [E, 2*d_ff] fp32; MXFP4 and MXFP8:
                                   [E, d/32, 2*d_ff] E8M0 bytes; else NULL     */
  const void* scale_down;       /* FP8: [E, d] fp32; MXFP4 and MXFP8:
                                   [E, d_ff/32, d] E8M0 bytes; else NULL       */
} moe_layer;

/* Optional copies of the routing the forward computed.  Any pointer may be
 * NULL.  Sizes as for moe_route / moe_align with block_m = the value the
 * forward chose, which it writes to *block_m (host pointer) when non-NULL;
 * sorted_ids must hold moe_align_capacity(T, E, k, MOE_BLOCK_M_MAX) entries
 * so it fits whatever block size the forward picks.                          */
typedef struct {
  float* logits;             /* [T, E]   */
  int32_t* topk_ids;         /* [T, k]   */
  float* topk_w;             /* [T, k]   */
  int32_t* expert_counts;    /* [E]      */
  int32_t* padded_offsets;   /* [E+1]    */
  int32_t* sorted_ids;       /* [cap]    */
  int32_t* inv_pos;          /* [T*k]    */
  int* block_m;              /* host out */
} moe_routing_out;

/* Optional per-kernel timing: when non-NULL, `events` holds n_events
 * hipEvent_t handles (created by the caller) and the forward records
 * events[i] on `stream` before its i-th kernel and events[n] after the last;
 * n_kernels receives the number of kernels enqueued.  Used only for
 * measurement; recording adds no work to the kernels themselves.            */
typedef struct {
  void** events;
  int n_events;
  int n_kernels;             /* out */
  const char* names[16];     /* out: kernel names, in launch order */
} moe_trace;

/*   x    [T, d] act_dtype;  out [T, d] act_dtype (may not alias x).
 * Limits: 1 <= k <= E <= MOE_MAX_EXPERTS, d % 128 == 0, d_ff % 128 == 0,
 * T * k < MOE_MAX_ENTRIES, a supported dtype pair, FP8 / MXFP4 scales present
 * for FP8 / MXFP4 weights. */
int moe_forward(const moe_layer* layer, const void* x, int T, void* out,
                void* workspace, size_t* workspace_bytes,
                moe_routing_out* routing, void* stream);

int moe_forward_traced(const moe_layer* layer, const void* x, int T, void* out,
                       void* workspace, size_t* workspace_bytes,
                       moe_routing_out* routing, moe_trace* trace, void* stream);

/* ---------------------------------------------------------------------------
 * moe_forward_noalloc — moe_forward for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, kernels and results as moe_forward, with
 * the workspace taken from a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.
 *
 *   Arguments as for moe_forward, without (workspace, workspace_bytes).  The
 *   current device must be the device of `stream` and of every pointer.
 *   A call whose workspace (moe_forward's query for the same layer and T)
 *   exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_SCRATCH before
 *   anything is enqueued; at 256 MiB this admits, e.g., every decode batch of
 *   up to 64 tokens of an E=8 top-2 d=4096 d_ff=14336 layer and of up to 16
 *   tokens of an E=256 top-8 d=7168 d_ff=2048 fp8 layer.  No allocation or
 *   free of any kind happens in the call.  The array is set up on the first
 *   call on each device (MOE_ERR_DEVICE if the runtime cannot resolve it).
 *   All calls on one GPU share that GPU's array: calls that overlap in time
 *   on one GPU (different streams, or host threads) race and corrupt each
 *   other's results; serialise them.  The array's contents on entry do not
 *   matter (nothing in it must start at zero).
 * ------------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int moe_forward_noalloc(const moe_layer* layer, const void* x, int T, void* out,
                        moe_routing_out* routing, void* stream);

/* ---------------------------------------------------------------------------
 * moe_rms_norm — row RMS normalisation over the hidden size (RMSNorm).
 * "La fusion de noyaux", section 4.2, reduction + elementwise: for every row
 * t of x,
 *   out[t, i] = x[t, i] / sqrt(sum_j x[t, j]^2 / d + eps) * (weight[i] + weight_bias),
 * in one pass (x read once, out written once), sums in fp32, rounded once to
 * the element type.  weight_bias is the constant some models add to the gain
 * ("CuTeDSL at Perplexity", RMS-norm remarks); 0 gives the plain formula.
 *
 *   x       [T, d]  dtype
 *   weight  [d]     dtype (the gain g)
 *   out     [T, d]  dtype; may be x itself (in place), must not otherwise
 *                   overlap it
 *   dtype   MOE_BF16 or MOE_F32
 * Limits: T >= 0, d * element size a multiple of 16 bytes and at most 32 KiB
 * (bf16: d % 8 == 0, d <= 16384; fp32: d % 4 == 0, d <= 8192; else
 * MOE_ERR_UNSUPPORTED), eps >= 0 and finite, weight_bias finite (else
 * MOE_ERR_INVALID).  No workspace.
 * ------------------------------------------------------------------------- */
int moe_rms_norm(const void* x, const void* weight, void* out, int T, int d, int dtype,
                 float weight_bias, float eps, void* stream);

/* ---------------------------------------------------------------------------
 * moe_qk_norm — per-head RMS normalisation of query and key heads (QK-norm),
 * in place.  "CuTeDSL at Perplexity", section on the RMS-norm kernel
 * specialised for small dimensions: the norm above applied to every head of
 * q (with q_weight) and of k (with k_weight) of every token, over the head's
 * head_dim values:
 *   x <- x * rsqrt(sum(x * x) / head_dim + eps) * (w + weight_bias),
 * rounded once to the element type.  (The section's one-line formula omits
 * the reciprocal square root; its kernel applies one, as does the RMSNorm of
 * "La fusion de noyaux".)
 *
 *   q         [T, n_q_heads, head_dim]  dtype, read and overwritten
 *   k         [T, n_k_heads, head_dim]  dtype, read and overwritten
 *   q_weight  [head_dim] dtype, shared by all q heads
 *   k_weight  [head_dim] dtype, shared by all k heads
 *   dtype     MOE_BF16 or MOE_F32
 * Sums, the root and the weighting run in fp32.  q/q_weight may be NULL when
 * n_q_heads == 0, k/k_weight when n_k_heads == 0; q and k must not overlap.
 * Limits: head_dim in {64, 128, 256} (else MOE_ERR_UNSUPPORTED), T >= 0,
 * head counts >= 0, T * (n_q_heads + n_k_heads) < 2^31, eps >= 0 and finite,
 * weight_bias finite (else MOE_ERR_INVALID).  No workspace.
 * ------------------------------------------------------------------------- */
int moe_qk_norm(void* q, void* k, const void* q_weight, const void* k_weight, int T,
                int n_q_heads, int n_k_heads, int head_dim, int dtype, float weight_bias,
                float eps, void* stream);

/* ---------------------------------------------------------------------------
 * moe_quantize_mxfp8 — MXFP8 quantisation of activation rows.  "CuTeDSL at
 * Perplexity", section on Blackwell support: the block-scaled formats share
 * one scale per block of 32 consecutive elements, found from the block's
 * absmax.  With the OCP MX rule for MXFP8, for every block of 32 consecutive
 * elements of a row:
 *   s     = floor(log2(max |x|)) - 8, at least -127 (an all-zero block: -127)
 *   code  = E4M3 ("fn") of x * 2^-s, rounded to nearest with ties to even,
 *           magnitudes above 448 saturated to 448, the sign bit that of x
 *   scale = s + 127 (an E8M0 byte, 0..246)
 * so that x ~ e4m3(code) * 2^(scale - 127), the MOE_MXFP8 encoding with the
 * blocks along the row.
 *
 *   x       [rows, n]     dtype (device)
 *   codes   [rows, n]     bytes (device, written)
 *   scales  [rows, n/32]  bytes (device, written)
 *   dtype   MOE_BF16 or MOE_F32
 * Limits: rows >= 0, n > 0 (else MOE_ERR_INVALID); n % 32 == 0 and dtype as
 * above (else MOE_ERR_UNSUPPORTED); the three regions must not overlap
 * (MOE_ERR_INVALID).  Inputs must be finite (a NaN or infinity gives
 * unspecified codes and scale for its block).  One launch, no workspace;
 * x is read once.
 * ------------------------------------------------------------------------- */
int moe_quantize_mxfp8(const void* x, int rows, int n, int dtype, void* codes, void* scales,
                       void* stream);

/* Static description of a status code (host). */
const char* moe_status_string(int status);

/* ABI version, bumped on any incompatible change (2: MXFP4 weights; the
 * scale fields of moe_layer became untyped pointers). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOE_H */
