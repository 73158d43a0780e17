/*
 * moe_mi355x.h -- C ABI of a one-GPU mixture-of-experts SwiGLU layer forward
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (page "Mixture of Experts in vLLM - From First Principles to
 * fused_moe", sections "One expert, and one token" through "How vLLM runs
 * the layer: two index lists and no copies"):
 *
 *   logits = W_r x                                   router, one linear layer
 *   p      = softmax(logits) over all E experts
 *   ids, w = the top_k largest p (slot 0 the largest; exact ties -> lower id),
 *            rescaled to sum to 1 when renormalize is set
 *   pair p = t*top_k + j  for token t, slot j
 *   index lists: pair ids sorted by expert, each expert's group padded with
 *            the id P = M*top_k up to a multiple of block_m, one expert per
 *            block of block_m entries
 *   act[p] = SiLU(h_gate) * h_up,  h = W13[id] x_t,  gate = rows 0..I-1,
 *            up = rows I..2I-1 of the stacked [2I, H] matrix
 *   out[t] = sum_j w[t, j] * (W2[id[t, j]] act[t*top_k + j])
 *
 * Conventions for every call below.
 *   - bf16 tensors are passed as raw uint16_t bit patterns.
 *   - Every pointer is a DEVICE pointer unless marked "host".  All tensors
 *     are dense, row-major, and 16-byte aligned (the GEMM calls and
 *     moe_forward return MOE_ERR_INVALID_ARG for a misaligned operand,
 *     index list, output or workspace).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call is asynchronous on that stream: it never allocates, frees or
 *     synchronizes, and returns as soon as its kernels are queued.
 *   - The caller owns every buffer.  Scratch memory comes from a caller
 *     workspace sized by moe_workspace_size(); a workspace may be reused by
 *     later calls on the same stream, but two calls in flight at once
 *     (different streams) need two workspaces.
 *   - Argument errors are detected on the host before anything is launched
 *     and return a negative moe_status; nothing is written then.  M == 0 is
 *     valid and launches nothing.  A failed launch returns MOE_ERR_HIP.
 *   - Device-side preconditions are the caller's: expert ids given to
 *     moe_align and the GEMM calls must lie in [0, E), and index lists given
 *     to the GEMM calls must be ones moe_align produced for the same
 *     (topk_ids, E, block_m).  Breaking them is undefined behaviour.
 *   - Supported sizes: 1 <= E <= 512; 1 <= top_k <= min(E, 32); H and I
 *     positive multiples of 8; M*top_k < 2^24.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad flag   */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside the supported sizes   */
  MOE_ERR_WORKSPACE = -3,    /* workspace missing or too small          */
  MOE_ERR_HIP = -4           /* a HIP launch failed                     */
} moe_status;

/* Which kernel family ran; filled by the GEMM calls and moe_forward.
 * (host struct)  A caller can check what ran instead of inferring it from
 * timing. */
#define MOE_VARIANT_TILED 0   /* LDS-tiled MFMA grouped GEMM (many rows per expert) */
#define MOE_VARIANT_STREAM 1  /* weight-streaming MFMA kernel (about one row per expert) */
#define MOE_VARIANT_PAIR_GEMV 2  /* per-pair GEMVs (block_m 1; moe_forward uses them,
                                    with no index lists, when M*top_k*4 <= E) */
#define MOE_VARIANT_PAIR_GEMV_QUANT 3  /* moe_forward_quantized: per-pair GEMVs on
                                          group-quantized weights */
#define MOE_VARIANT_TILED_MXFP8 4  /* moe_forward_mxfp8: LDS-tiled scaled-MFMA GEMMs on
                                      MXFP8 operands */
#define MOE_VARIANT_STREAM_MXFP8 5  /* moe_forward_mxfp8: weight-streaming scaled-MFMA
                                       GEMMs on MXFP8 operands (block_m 16) */
#define MOE_VARIANT_PAIR_GEMV_MXFP8 6  /* moe_forward_mxfp8: per-pair GEMVs on MXFP8
                                          weights and inputs (M*top_k*4 <= E, no lists) */
#define MOE_VARIANT_STREAM_QUANT 7  /* moe_forward_quantized: weight-streaming MFMA
                                       GEMMs on group-quantized weights (block_m 16) */
#define MOE_VARIANT_TILED_QUANT 8  /* moe_forward_quantized: LDS-tiled MFMA GEMMs, the
                                      codes widened to bf16 tiles in LDS (block_m 128) */
typedef struct moe_dispatch_info {
  int variant;   /* MOE_VARIANT_* of the GEMMs                                   */
  int block_m;   /* rows (pairs) per block of the index lists                    */
  int block_n;   /* output features per workgroup tile of GEMM 1 (gate + up)     */
  int block_k;   /* K elements per pipeline step                                 */
  int k_tail;    /* 1 if some K (H for GEMM 1, I for GEMM 2) is not a multiple of block_k */
  int launches;  /* kernels this call queued                                     */
  int sorted;    /* moe_forward: 1 = pairs sorted by expert into index lists;
                    0 = no lists, one GEMV per pair (MOE_VARIANT_PAIR_GEMV)      */
} moe_dispatch_info;

/* Bytes of workspace that moe_forward needs for any M <= M_max with these
 * layer sizes (it also covers moe_route and moe_grouped_gemm_w2_combine).
 * Returns 0 for unsupported sizes. */
size_t moe_workspace_size(int M_max, int E, int top_k, int H, int I);

/* Static text of a moe_status value. */
const char* moe_strerror(int status);

/* The block size (block_m) moe_forward uses for a batch of M tokens: the
 * compiled tile table.  Returns 1 (per-pair GEMVs) when M >= 1 and
 * M*top_k*4 <= E; otherwise, keyed on the mean number of pairs per expert
 * (M*top_k/E): 16 (weight-streaming kernels) up to 8 pairs per expert, then
 * the tiled kernels: 64 up to 48, 128 below 128, 256 below 192, 128 from 192
 * on (measured per shape). */
int moe_pick_block_m(int M, int E, int top_k);

/*
 * moe_route -- router logits, softmax over all experts, top-k, renormalize.
 * Page "Mixture of Experts in vLLM ...", section "One expert, and one token",
 * sub-section "One token uses only 8 experts"; the output format is that of
 * section "A batch: (token, expert) pairs" (topk_ids, topk_weights [M, k]).
 *
 *   x            [M, H] bf16      token rows
 *   w_router     [E, H] bf16      router weights
 *   logit_bias   [E] fp32 or NULL added to every token's logits (a prior)
 *   topk_ids     [M, top_k] int32 out: expert ids, slot 0 = largest
 *   topk_weights [M, top_k] fp32  out: the kept softmax probabilities,
 *                                 rescaled to sum 1 if renormalize != 0
 *   logits_out   [M, E] fp32 or NULL  out: the fp32 logits (+ bias)
 *   workspace    device scratch of ws_bytes >= M*E*4 (holds the logits when
 *                logits_out is NULL; may be NULL when logits_out is given).
 * Logits accumulate bf16 x bf16 products in fp32; the top-k decision is
 * taken on those fp32 values.
 */
int moe_route(const uint16_t* x, const uint16_t* w_router, const float* logit_bias,
              int M, int H, int E, int top_k, int renormalize,
              int32_t* topk_ids, float* topk_weights, float* logits_out,
              void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_align -- the two index lists (moe_align_block_size).
 * Page "Mixture of Experts in vLLM ...", section "How vLLM runs the layer:
 * two index lists and no copies", sub-section "The two index lists"; pair
 * ids as in section "A batch: (token, expert) pairs".
 *
 *   topk_ids             [M*top_k] int32  expert of pair p = t*top_k + j
 *   block_m              rows per block, 1..256
 *   sorted_token_ids     out [P + min(E,P)*(block_m-1)] int32: pair ids
 *                        grouped by expert (ascending expert; inside a
 *                        group ascending pair id), each group padded with
 *                        P = M*top_k to a multiple of block_m.  Only the
 *                        first num_blocks*block_m entries are written.
 *   expert_ids           out [ceil(P/block_m) + min(E,P)] int32: expert of
 *                        each block; only the first num_blocks are written.
 *   expert_block_offsets out [E+1] int32: first block of each expert;
 *                        entry E = num_blocks.  It stays in device memory;
 *                        later calls read it there, so no host sync is needed.
 *   expert_counts        out [E] int32 (pairs per expert) or NULL.
 *   workspace            device scratch of ws_bytes >=
 *                        moe_align_workspace_size(M, top_k, E) (that size is
 *                        0 for small batches; NULL is then allowed).
 * The result is deterministic (the same bits on every run).
 */
size_t moe_align_workspace_size(int M, int top_k, int E);
int moe_align(const int32_t* topk_ids, int M, int top_k, int E, int block_m,
              int32_t* sorted_token_ids, int32_t* expert_ids,
              int32_t* expert_block_offsets, int32_t* expert_counts,
              void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm_w13_act -- grouped GEMM 1 with SiLU(gate)*up fused.
 * Page "Mixture of Experts in vLLM ...", sub-sections "One GEMM 1 program,
 * step by step" (block -> expert, pad mask, input row p // top_k, output row
 * p) and "The rest of the layer stays in pair order" (SiLU and multiply row
 * by row).  The [M*top_k, 2I] GEMM 1 output never exists in memory.
 *
 *   x      [M, H] bf16;  w13 [E, 2I, H] bf16 (gate rows first)
 *   index lists from moe_align with the same block_m (1, 16, 64, 128 or
 *   256; 1 selects the per-pair GEMV, one pair per block, which reads its
 *   expert's weights once per pair and suits only very small batches; 16
 *   the weight-streaming kernel; the others the tiled kernel)
 *   act    out [M*top_k, I] bf16 in pair order (row p = t*top_k + j)
 *   info   host, optional: which kernel ran
 * Accumulation is fp32; act is rounded to bf16 once.
 */
int moe_grouped_gemm_w13_act(const uint16_t* x, const uint16_t* w13,
                             const int32_t* sorted_token_ids, const int32_t* expert_ids,
                             const int32_t* expert_block_offsets,
                             int M, int top_k, int E, int H, int I, int block_m,
                             uint16_t* act, moe_dispatch_info* info, void* stream);

/*
 * moe_grouped_gemm_w2_combine -- grouped GEMM 2 and the weighted top-k
 * combine.  Page "Mixture of Experts in vLLM ...", sections "The rest of the
 * layer stays in pair order" (GEMM 2 reads act row p in place and writes
 * row p of the pair-order product, the page's cache3) and "Put the results
 * back, and combine them per token" (moe_sum with the routed weights).
 *
 *   act          [M*top_k, I] bf16 in pair order
 *   w2           [E, H, I] bf16
 *   topk_weights [M*top_k] fp32
 *   out          out [M, H] bf16 in token order
 *   workspace    holds the pair-order product [M*top_k, H] (block_m 1 and
 *                16: fp32, already scaled by topk_weights; 64, 128, 256:
 *                bf16, scaled in the sum), ws_bytes >= moe_workspace_size(M,
 *                E, top_k, H, I)
 * A second kernel adds each token's top_k rows in slot order in fp32 and
 * rounds once to bf16, so results are bitwise repeatable.
 */
int moe_grouped_gemm_w2_combine(const uint16_t* act, const uint16_t* w2,
                                const float* topk_weights,
                                const int32_t* sorted_token_ids, const int32_t* expert_ids,
                                const int32_t* expert_block_offsets,
                                int M, int top_k, int E, int H, int I, int block_m,
                                uint16_t* out, void* workspace, size_t ws_bytes,
                                moe_dispatch_info* info, void* stream);

/*
 * moe_forward -- the whole layer: route -> align -> GEMM 1 + act -> GEMM 2 +
 * combine, all queued on `stream` with no host synchronization.  Every
 * intermediate lives in the caller's workspace, allocated once and reused
 * across layers (page "MoE Execution Path Analysis", "Memory allocation per
 * step" and "What we can actually change"); block_m comes from
 * moe_pick_block_m (the same page's per-batch-size BLOCK_SIZE_M choice).
 * Very small batches, M*top_k*4 <= E, build no index lists: each pair runs
 * as its own GEMV against its expert's weights, read from the top-k ids
 * (page "Mixture of Experts in vLLM ...", sub-section "Small batches skip
 * the sort"), and GEMM 2 sums the weighted rows per token in the same
 * launch; info->variant then reads MOE_VARIANT_PAIR_GEMV, info->sorted 0.
 *
 *   x [M, H], w_router [E, H], w13 [E, 2I, H], w2 [E, H, I]: bf16
 *   logit_bias       [E] fp32 or NULL
 *   out              out [M, H] bf16
 *   topk_ids_out     out [M, top_k] int32 or NULL
 *   topk_weights_out out [M, top_k] fp32 or NULL
 *   workspace        ws_bytes >= moe_workspace_size(M, E, top_k, H, I)
 *   info             host, optional
 */
int moe_forward(const uint16_t* x, const uint16_t* w_router, const float* logit_bias,
                const uint16_t* w13, const uint16_t* w2,
                int M, int E, int top_k, int H, int I, int renormalize,
                uint16_t* out, int32_t* topk_ids_out, float* topk_weights_out,
                void* workspace, size_t ws_bytes, moe_dispatch_info* info, void* stream);

/*
 * moe_forward_noalloc -- moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same layer, kernels and results, with the
 * scratch memory in a device array of this library
 * (MOE_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends) instead of a caller workspace.  The caller still
 * passes inputs and outputs, as for moe_forward; nothing is allocated,
 * freed or synchronized.
 *   - A batch whose moe_workspace_size(M, E, top_k, H, I) exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE before any launch
 *     (Qwen3-30B-A3B shape: up to about 850 tokens).
 *   - Every call on one GPU uses that GPU's one array, which keeps the last
 *     call's contents (the kernels clear what must start at zero).  Calls
 *     that overlap on one GPU (other streams, other threads) race on it:
 *     serialize them, or use moe_forward with separate workspaces.
 *   - MOE_ERR_HIP if the array's address cannot be looked up.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const uint16_t* x, const uint16_t* w_router, const float* logit_bias,
                        const uint16_t* w13, const uint16_t* w2, int M, int E, int top_k, int H,
                        int I, int renormalize, uint16_t* out, int32_t* topk_ids_out,
                        float* topk_weights_out, moe_dispatch_info* info, void* stream);

/*
 * Where moe_forward leaves the index lists of a batch in its workspace
 * (host struct): byte offsets from the workspace start, valid after a
 * moe_forward call with the same (M, E, top_k, H, I) on that workspace
 * has completed.  The lists are the ones of moe_align (page "Mixture of
 * Experts in vLLM ...", sub-section "The two index lists") for the
 * routing moe_forward chose, with block_m = moe_pick_block_m(M, E, top_k);
 * only the first num_blocks entries of expert_ids and num_blocks*block_m of
 * sorted_token_ids are written (num_blocks = expert_block_offsets[E]).
 * A caller can read them back to see how the batch was dispatched.
 */
typedef struct moe_forward_lists {
  int block_m;                  /* rows per block of the lists                */
  int sorted;                   /* 0: this M runs per-pair GEMVs, no lists     */
  size_t sorted_token_ids;      /* int32 [M*top_k + min(E, P)*(block_m-1)]    */
  size_t expert_ids;            /* int32 [ceil(P/block_m) + min(E, P)]        */
  size_t expert_block_offsets;  /* int32 [E+1]                                */
  size_t expert_counts;         /* int32 [E]                                  */
} moe_forward_lists;

/* Fills *out for a batch of M tokens; returns MOE_OK, or a negative status
 * (nothing written) for unsupported sizes or a null out. */
int moe_forward_list_offsets(int M, int E, int top_k, int H, int I, moe_forward_lists* out);

/*
 * Group-quantized expert weights (host struct of device pointers): the
 * affine group format in the MLX part of the page "SGLang issue #22283"
 * (GitHub thread): its kernels read 64-element-group, 4-bit weights
 * (affine_qmv ... gs_64_b_4); 6 and 8 bits are discussed too.  Each row of
 * W13 [E, 2I, H] and W2 [E, H, I] holds K codes q in [0, 2^bits), packed
 * least significant first into 32-bit words (element i of a row is bits
 * [bits*i, bits*(i+1)) of the row's bit stream); each group of 64
 * consecutive elements of a row has one bf16 scale s and one bf16 bias b,
 * and the weight is w = s*q + b.
 */
typedef struct moe_quantized_weights {
  int bits;                      /* 4 or 8                                   */
  int group_size;                /* 64                                       */
  const uint32_t* w13_q;         /* [E, 2I, H*bits/32] packed codes          */
  const uint16_t* w13_scales;    /* [E, 2I, H/64] bf16                       */
  const uint16_t* w13_biases;    /* [E, 2I, H/64] bf16                       */
  const uint32_t* w2_q;          /* [E, H, I*bits/32]                        */
  const uint16_t* w2_scales;     /* [E, H, I/64] bf16                        */
  const uint16_t* w2_biases;     /* [E, H, I/64] bf16                        */
} moe_quantized_weights;

/*
 * moe_forward_quantized -- the layer of moe_forward with group-quantized
 * expert weights (the router stays bf16).  Up to E/2 pairs
 * (M*top_k*2 <= E), every pair runs as its own GEMV against
 * its expert's dequantized rows (page "Mixture of Experts in vLLM ...",
 * sub-section "Small batches skip the sort"; no index lists), the group's
 * scale and bias applied per 16-byte unit of codes; GEMV 2 adds the
 * weighted top_k rows per token in one launch (four launches: router
 * logits, top-k, GEMV 1, GEMV 2; info->variant MOE_VARIANT_PAIR_GEMV_QUANT,
 * info->sorted 0).  Larger batches build index lists with block_m 16 (the
 * same route and align launches as moe_forward) and run weight-streaming
 * MFMA GEMMs that read each expert's codes once per block: within a
 * 64-element group, sum w x = s * sum q x + b * sum x, with the codes
 * widened exactly to bf16 MFMA operands and the scale and bias applied in
 * fp32 per group; GEMM 2 writes fp32 weighted pair-order rows and a second
 * kernel sums them per token (info->variant MOE_VARIANT_STREAM_QUANT,
 * info->sorted 1).  The streaming kernels need H and I to be multiples of
 * 128 (other shapes run the per-pair GEMVs there).  Where moe_forward runs
 * its tiles (more than 8 pairs per expert), the quantized layer runs the
 * copy-wave tiles over block_m 128 lists, four more waves per workgroup
 * widening each stage's codes into bf16 weight tiles in LDS (w = s*q + b
 * rounded once to bf16, as a quantized matmul in the activation dtype does),
 * and GEMM 2's bf16 pair-order rows summed per token (info->variant
 * MOE_VARIANT_TILED_QUANT).
 *
 *   x, w_router, logit_bias, out, topk_ids_out, topk_weights_out, workspace:
 *                as for moe_forward (same workspace size)
 *   qw           host struct of device pointers, all 16-byte aligned
 * H and I must be multiples of 64 (MOE_ERR_UNSUPPORTED otherwise); a K that
 * is not a multiple of the kernels' 256- or 512-element passes is fine.
 */
int moe_forward_quantized(const uint16_t* x, const uint16_t* w_router, const float* logit_bias,
                          const moe_quantized_weights* qw, int M, int E, int top_k, int H, int I,
                          int renormalize, uint16_t* out, int32_t* topk_ids_out,
                          float* topk_weights_out, void* workspace, size_t ws_bytes,
                          moe_dispatch_info* info, void* stream);

/*
 * MXFP8 experts (the FP8 layer of page "Mixture of Experts in vLLM - From
 * First Principles to fused_moe", sub-section "The two index lists": the
 * GEMM 1 input qhidden is a quantized copy of x; the MXFP8 format named in
 * the MLX part of the page "SGLang issue #22283"): the OCP microscaling
 * format, blocks of 32 consecutive elements along K, each with one E8M0
 * scale byte c (the value 2^(c - 127)) and 32 E4M3 bytes (sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; 0x7F and 0xFF are NaN).  All arrays
 * row-major, K contiguous, 16-byte aligned.
 */
typedef struct moe_mx_weights {
  const uint8_t* w13_codes;    /* [E, 2I, H] E4M3                              */
  const uint8_t* w13_scales;   /* [E, 2I, H/32] E8M0                           */
  const uint8_t* w2_codes;     /* [E, H, I] E4M3                               */
  const uint8_t* w2_scales;    /* [E, H, I/32] E8M0                            */
} moe_mx_weights;

/*
 * moe_mx_quantize -- MXFP8 codes [rows, K] and scales [rows, K/32] of bf16
 * rows src [rows, K] (K a multiple of 32; device pointers, src and codes
 * 16-byte aligned).  Per block of 32: scale 2^(floor(log2 amax) - 8)
 * clamped to [2^-127, 2^127] (code 0 for an all-zero block); element =
 * v / scale rounded to the nearest E4M3 value, ties to the even code,
 * saturated at 448, sign kept.  One launch; returns MOE_OK, or
 * MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED (K % 32) before any launch.
 */
int moe_mx_quantize(const uint16_t* src, int rows, int K, uint8_t* codes, uint8_t* scales,
                    void* stream);

/* Workspace bytes for every moe_forward_mxfp8 call with M <= M_max (0 if
 * the sizes are unsupported: H or I not a multiple of 128, or as for
 * moe_workspace_size). */
size_t moe_mx_workspace_size(int M_max, int E, int top_k, int H, int I);

/*
 * moe_forward_mxfp8 -- the layer of moe_forward with MXFP8 expert weights
 * and MXFP8 GEMM inputs: routing on the bf16 router as moe_forward; x
 * quantized to MXFP8 as moe_mx_quantize does (by the top-k launch); GEMM 1
 * on the gfx950 scaled MFMA
 * (E4M3 x E4M3, each 32-element block scaled by its E8M0 factor, fp32
 * accumulation) with SiLU(gate)*up, act stored bf16; act quantized to
 * MXFP8; GEMM 2 likewise into bf16 pair-order rows; the weighted top-k sum
 * per token.  Index lists with block_m = moe_pick_block_m(M, E, top_k):
 * weight-streaming kernels at block_m 16, tiled kernels above.  Very small
 * batches (M*top_k*4 <= E, page "Mixture of Experts in vLLM ...",
 * sub-section "Small batches skip the sort") build no lists: the top-k
 * launch also quantizes x, GEMV 1 runs each pair against its expert's
 * MXFP8 rows, and GEMV 2 quantizes each act row to MXFP8 in registers and
 * sums the weighted slots per token (four launches; info->variant
 * MOE_VARIANT_PAIR_GEMV_MXFP8, info->sorted 0).
 *
 *   x, w_router, logit_bias, out, topk_ids_out, topk_weights_out, info,
 *   stream: as for moe_forward;  w: host struct of device pointers
 *   workspace: at least moe_mx_workspace_size(M, ...) bytes, 16-byte aligned
 * H and I must be multiples of 128 (MOE_ERR_UNSUPPORTED otherwise).
 * info->variant reads MOE_VARIANT_PAIR_GEMV_MXFP8, MOE_VARIANT_STREAM_MXFP8 or
 * MOE_VARIANT_TILED_MXFP8.
 */
int moe_forward_mxfp8(const uint16_t* x, const uint16_t* w_router, const float* logit_bias,
                      const moe_mx_weights* w, int M, int E, int top_k, int H, int I,
                      int renormalize, uint16_t* out, int32_t* topk_ids_out,
                      float* topk_weights_out, void* workspace, size_t ws_bytes,
                      moe_dispatch_info* info, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
