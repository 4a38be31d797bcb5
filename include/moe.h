/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts FFN layer, one GPU's expert slice.
 *
 * The layer (per token t with input row x_t):
 *   logits_t = W_r x_t + bias                      router over all E experts (fp32)
 *   S_t      = the k largest logits (lowest expert index first among equal values)
 *   w_tj     = softmax over S_t, or sigmoid(L) / sum over S_t of sigmoid(L)
 *   out_t    = sum_{j : e_tj local} w_tj * FFN_{e_tj}(a_t)  [+ g_t * FFN_shared(a_t)]
 *   FFN_e(a) = W_down,e ( silu(W_gate,e a) * (W_up,e a) )
 *   g_t      = 1 / (1 + exp(-(w_sg . x_t))) for a gated shared expert, else 1
 * where a_t is x_t, or x_t after the activation quantiser for the fp8 / MXFP4 / MXFP8 expert
 * formats.
 *
 * Passages that define the steps (cited by page title and section):
 *   - "Hosting Qwen on Blackwell", section "Prefillers": top-8 routing over 128 experts makes each
 *     expert a dense GEMM problem (~375 tokens each at a 6000-token prefill); section "Expert
 *     parallel": inputs are replicated, the dispatch selects the tokens routed to this rank's
 *     experts and prepares them in buffers for the MoE GEMM, the combine first accumulates the
 *     local contributions (the cross-rank reduction is outside this library).
 *   - "CuTeDSL at Perplexity", section "MoE dispatch and combine": the local kernel counts tokens
 *     per expert from the routing table, gives each token a unique index within its expert's list,
 *     copies tokens into (optionally padded) expert buffers, and the combine accumulates weighted
 *     rows in registers using those positions and the offsets the dispatch computed.
 *     Introduction: the layer adapts to the newer models' additional gate terms (their form is
 *     not given; read here as the per-token logistic gate g_t of the shared expert above).
 *   - "How we served a 397B MoE model with 4.7x speedup on TPU v7", architectural constraints
 *     section: 512 experts, top-10, one always-active shared expert; "Three collectives become two":
 *     routing indices (int) and weights (float) as two arrays of shape [T, k].
 *   - "Driving vLLM WideEP and Large-Scale Serving Toward Maturity on Blackwell (Part I)", section
 *     on lower-precision operations: 4-bit MoE weights packed two per byte with per-group scales,
 *     activations quantised to 4 bits before dispatch.
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers (descriptor structs are host pointers). The caller
 *     owns every buffer, workspaces included; the library never allocates or frees memory and keeps
 *     no pointer after a call returns.
 *   - Work is enqueued on `stream`; calls return without synchronising. Results are valid when the
 *     stream reaches that point. A workspace must not be used by two streams at once.
 *   - Layouts are row-major and contiguous. Matrices are stored [out_features, in_features]
 *     (K contiguous). Expert ids are global ids in [0, E); local expert e' is global id e0 + e'.
 *   - Arguments are validated on the host before anything is launched; on error nothing is
 *     enqueued and a status other than MOE_OK is returned. A failed launch returns MOE_ERR_HIP and
 *     the hipError_t is kept per thread (moe_last_hip_error). Outputs are unspecified after an error.
 *   - Identical inputs give byte-identical outputs (no result depends on atomics' ordering).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* bad size, null or misaligned pointer                         */
  MOE_ERR_UNSUPPORTED = 2,   /* a valid combination this library does not implement          */
  MOE_ERR_WORKSPACE = 3,     /* workspace smaller than the matching *_workspace_bytes query */
  MOE_ERR_HIP = 4            /* a HIP launch failed; see moe_last_hip_error()                 */
} moe_status;

typedef enum {
  MOE_F32 = 0,        /* fp32                                                                  */
  MOE_BF16 = 1,       /* bf16                                                                  */
  MOE_FP8_E4M3 = 2,   /* OCP e4m3 bytes with fp32 block scales                                 */
  MOE_MXFP4 = 3,      /* OCP e2m1, two per byte (element 2i in bits 0-3 of byte i), E8M0 scale
                         byte per 32 consecutive elements along K                             */
  MOE_MXFP8 = 4,      /* OCP e4m3 bytes with an E8M0 scale byte per 32 consecutive elements
                         along K (OCP MX v1.0 MXFP8; the MoE GEMM format of "Hosting Qwen on
                         Blackwell", section "Quantization")                                  */
  MOE_NVFP4 = 5,      /* NVFP4: OCP e2m1, two per byte as MXFP4, with an e4m3 scale per 16
                         consecutive elements along K ("CuTeDSL at Perplexity", section
                         "Blackwell": 16-element absmax groups; "Driving vLLM WideEP ... (Part
                         I)", lower-precision operations: 4-bit weights with FP8 per-group
                         scales) and an fp32 scale per row (NVFP4's second level, per tensor in
                         NVIDIA's recipe, per row here). Element value: e2m1 * s_block * g_row */
  MOE_F16_SCALED = 6  /* expert outputs only (the down projection's y): fp16 values with one fp32
                         power-of-two scale per row per 64 consecutive columns, value = f16 *
                         scale. A row of `cols` values (cols % 64 == 0) is its cols fp16 values
                         followed by its cols / 64 fp32 scales, padded to a multiple of 16 bytes
                         (moe_f16_scaled_row_bytes). A block whose largest magnitude m lies in
                         [2^(e-1), 2^e) gets the scale 2^max(e - 15, -126): its scaled values stay
                         below 2^15, inside fp16's range, and each is rounded (to nearest even) to
                         within 2^-11 m. Written by the grouped GEMM (bf16 experts, STORE), read
                         by the combine: half the bytes of fp32 rows, and at the block maximum
                         four times the precision of bf16 rows */
} moe_dtype;

/* bytes of one MOE_F16_SCALED row of `cols` values (cols % 64 == 0) */
static inline int64_t moe_f16_scaled_row_bytes(int64_t cols) {
  return 2 * cols + (cols / 64 * 4 + 15) / 16 * 16;
}

typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_scoring;
typedef enum { MOE_EPI_STORE = 0, MOE_EPI_SWIGLU = 1 } moe_epilogue;

/* Shape and formats of one layer call. */
typedef struct {
  int32_t T;            /* tokens (>= 0; T = 0 is a no-op)                                     */
  int32_t H;            /* hidden size                                                         */
  int32_t E;            /* experts in the model (router width), 1..1024                        */
  int32_t e0;           /* first local expert (global id)                                      */
  int32_t E_loc;        /* local experts, e0 + E_loc <= E                                      */
  int32_t I;            /* expert intermediate size                                            */
  int32_t k;            /* experts per token, 1 <= k <= min(E, 16)                             */
  int32_t I_s;          /* shared expert intermediate size, 0 = no shared expert; any multiple
                           of the expert format's K granularity (64 bf16 / fp32, 128 fp8 and
                           MXFP8, 256 MXFP4 and NVFP4). I_s == I runs the shared expert inside
                           the routed experts' GEMM launches, other sizes in launches of their
                           own                                                                 */
  int32_t scoring;      /* moe_scoring                                                         */
  int32_t renormalize;  /* 1: weights renormalised over the k chosen experts                   */
  int32_t io_dtype;     /* x and the router weight: MOE_F32 or MOE_BF16                        */
  int32_t out_dtype;    /* out: MOE_F32 or MOE_BF16. out is this GPU's partial sum over its
                           local experts; fp32 keeps it unrounded for the reduction across
                           expert-parallel ranks that follows the layer                        */
  int32_t expert_dtype; /* expert weights and GEMM activations: MOE_F32 (io F32 only),
                           MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4, MOE_MXFP8, MOE_NVFP4              */
} moe_desc;

/* Expert weights of one layer, in expert_dtype:
 *   F32 / BF16:  gate, up [E_loc, I, H]; down [E_loc, H, I]; *_scales NULL.
 *   FP8_E4M3:    codes as above; fp32 scales per 128x128 block: gate/up [E_loc, I/128, H/128],
 *                down [E_loc, H/128, I/128].
 *   MXFP4:       packed codes gate/up [E_loc, I, H/2], down [E_loc, H, I/2]; E8M0 scales
 *                gate/up [E_loc, I, H/32], down [E_loc, H, I/32].
 *   MXFP8:       codes gate/up [E_loc, I, H], down [E_loc, H, I]; E8M0 scales as for MXFP4.
 *   NVFP4:       packed codes as for MXFP4; *_scales: one record per expert (E_loc records back to
 *                back) of an [N, K] matrix: e4m3 block scales [N, K/16], then fp32 row scales [N]
 *                (N*K/16 + 4*N bytes; gate/up N = I, K = H; down N = H, K = I).
 * The shared expert (sh_*) has the same layouts with E_loc = 1 and I = I_s; NULL when I_s = 0.
 * w_router is [E, H] in io_dtype. w_shared_gate is the shared expert's gate vector w_sg [H] in
 * io_dtype, or NULL for an ungated shared expert (g_t = 1); ignored when I_s = 0. Produce
 * quantised weights with moe_quantize. */
typedef struct {
  const void* w_router;
  const void* w_gate;  const void* w_gate_scales;
  const void* w_up;    const void* w_up_scales;
  const void* w_down;  const void* w_down_scales;
  const void* sh_gate; const void* sh_gate_scales;
  const void* sh_up;   const void* sh_up_scales;
  const void* sh_down; const void* sh_down_scales;
  const void* w_shared_gate;
} moe_weights;

/* ---- routing (router logits, scores, top-k, renormalisation) ---------------------------------
 * Defining passages: "How we served a 397B MoE model with 4.7x speedup on TPU v7", section on the
 * architectural constraints (top-10 of 512 experts) and "Three collectives become two" (the
 * routing result is an int index array and a float weight array, both [T, k]); "Hosting Qwen on
 * Blackwell", section "Prefillers" (top-8 of 128). The router function itself (softmax or sigmoid
 * with renormalisation) is not on the pages; it is the layer configuration's.
 * If x != NULL: logits[T,E] = x . w_router^T + bias (fp32 accumulation) are written, then used.
 * If x == NULL: logits[T,E] (fp32) are read as given and w_router is ignored.
 * topk_ids[T,k] (int32, global ids, rank order: topk_ids[t,0] is the largest logit; equal values
 * rank the lower id first; -0 equals +0) and topk_w[T,k] (fp32). The selection is made on exactly
 * the fp32 values in `logits`. bias[E] (fp32) may be NULL. Pointers: 16-byte aligned.
 * ws: moe_route_workspace_bytes(d) bytes of device scratch (the K-split partial sums of a
 * few-token bf16 router); may be NULL when that size is 0 or x is NULL, else MOE_ERR_WORKSPACE. */
moe_status moe_route(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                     float* logits, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                     hipStream_t stream);
size_t moe_route_workspace_bytes(const moe_desc* d);

/* ---- routing blob --------------------------------------------------------------------------------
 * The routing result as one 32-bit array [2][P], P = T*k rounded up to a multiple of 4 (so that
 * each plane starts 16-byte aligned): plane 0 holds topk_ids, plane 1 the bits of topk_w. This is
 * the stacked, bitcast form in which one all-gather moves indices and weights together ("How we
 * served a 397B MoE model with 4.7x speedup on TPU v7", section "Three collectives become two").
 * Pass topk_ids = blob and topk_w = (float*)(blob + P) to moe_route or moe_layer, and the same
 * planes to moe_permute and moe_combine. Returns P (0 for an invalid descriptor). */
int64_t moe_routing_blob_plane(const moe_desc* d);

/* ---- dispatch (count, offsets, unique row per local slot, copy) ------------------------------
 * Defining passage: "CuTeDSL at Perplexity", section "MoE dispatch and combine", local kernel:
 * count the tokens of each expert, give each token a unique index within its expert, copy the
 * tokens into the expert buffers; "Hosting Qwen on Blackwell", section "Expert parallel": the
 * dispatch prepares the tokens routed to this rank's experts as the MoE GEMM's input. The order
 * inside an expert is fixed here (ascending flat slot) where the pages use atomic counters.
 * counts[E_loc]: local slots per expert. offsets[E_loc+1]: exclusive prefix sum, offsets[E_loc] = R.
 * slot_to_row[T,k]: row of slot (t,j) in the expert-contiguous buffer, -1 if e_tj is not local.
 * row_to_flat[T*k]: flat slot t*k+j of each row (entries >= R untouched).
 * Rows of one expert are in ascending flat slot order (a unique, deterministic placement).
 * a_in: the activations in token order in the GEMM input format:
 *   F32 / BF16: [T, H] values; a_in_scales NULL.
 *   FP8_E4M3:   e4m3 [T, H] + fp32 a_in_scales [ceil(T/128), H/128] (128x128 blocks);
 *               a_perm_scales receives [T*k, H/128] (the block row of each token).
 *   MXFP4:      packed [T, H/2] + E8M0 [T, H/32]; a_perm_scales receives [T*k, H/32].
 *   MXFP8:      e4m3 [T, H] + E8M0 [T, H/32]; a_perm_scales receives [T*k, H/32].
 *   NVFP4:      packed [T, H/2] + one scale record (e4m3 [T, H/16], then fp32 [T]); the copy
 *               dequantises: a_perm receives the block values e2m1 * s_block as bf16 [T*k, H]
 *               (exact) and a_perm_scales the fp32 row scales [T*k], the grouped GEMM's A and
 *               A_scales. H % 64 == 0.
 * a_perm: [T*k, row bytes] (R rows written), or NULL to produce only the maps.
 * ws: moe_permute_workspace_bytes(d) bytes of device scratch. */
moe_status moe_permute(const moe_desc* d, const int32_t* topk_ids, const void* a_in,
                       const void* a_in_scales, int32_t* counts, int32_t* offsets,
                       int32_t* slot_to_row, int32_t* row_to_flat, void* a_perm,
                       void* a_perm_scales, void* ws, size_t ws_bytes, hipStream_t stream);
size_t moe_permute_workspace_bytes(const moe_desc* d);

/* ---- grouped GEMM ------------------------------------------------------------------------------
 * Defining passages: "Hosting Qwen on Blackwell", sections "Prefillers" (every expert's tokens
 * form one dense GEMM problem) and "MoE GEMM" (the grouped expert GEMM, decode-limited by loading
 * the weights); "Driving vLLM WideEP and Large-Scale Serving Toward Maturity on Blackwell
 * (Part I)", section on lower-precision operations (4-bit weights with per-group scales,
 * dequantised inside the GEMM). SwiGLU (silu(gate) * up) is the layer configuration's.
 * For every group g with rows [group_offsets[g], group_offsets[g+1]) (device array, ascending,
 * group_offsets[G] <= max_rows):
 *   STORE:  C[r, :N]  = A[a(r), :K] . B[g]^T                       (B[g]: [N, K])
 *   SWIGLU: C[r, :N]  = silu(A[a(r)] . B[g]^T) * (A[a(r)] . B2[g]^T) (B[g], B2[g]: [N, K])
 * where a(r) = r, or a(r) = a_rows[r] / a_row_div when a_rows != NULL (gathering rows of A).
 * dtype is the format of A and B (see moe_weights for B and its scales; A and its scales follow
 * moe_permute's a_perm). out_dtype: STORE -> MOE_F32 | MOE_BF16 (bf16 A and B also
 * MOE_F16_SCALED: C rows of moe_f16_scaled_row_bytes(N) bytes); SWIGLU -> MOE_F32 | MOE_BF16, or
 * the next GEMM's input format (MOE_FP8_E4M3: fp32 C_scales [max_rows, N/128] per 1x128 block;
 * MOE_MXFP4 and MOE_MXFP8: C_scales [max_rows, N/32]). a_scale_rows: 128 when A's fp8 scales
 * are per 128-row block of A (a token-order x), else 1. Rows outside every group are not written.
 * NVFP4: B and B2 as in moe_weights (B_scales / B2_scales: one scale record per group); A holds
 * bf16 block values [rows, K] (as moe_permute writes them) and A_scales fp32 row scales [rows of
 * A] (NULL: 1); every product q * s is exact in bf16 and runs on the bf16 MFMA, the row scales
 * multiply the result; out_dtype MOE_F32 or MOE_BF16.
 * Preconditions: K % 128 == 0 (K % 256 for MXFP4 and NVFP4, K % 64 for BF16/F32), N % 64 == 0
 * (N % 128 for the quantised formats); dtype F32 needs out F32. */
typedef struct {
  int32_t G;            /* groups (experts)                                                   */
  int32_t max_rows;     /* rows of C (and of A when a_rows == NULL)                           */
  int32_t K, N;
  int32_t dtype;        /* moe_dtype of A and B                                               */
  int32_t epilogue;     /* moe_epilogue                                                       */
  int32_t out_dtype;    /* moe_dtype of C                                                     */
  int32_t a_row_div;    /* divisor applied to a_rows entries (>= 1)                            */
  int32_t a_scale_rows; /* 1 or 128 (FP8 only)                                                 */
} moe_gemm_desc;

moe_status moe_grouped_gemm(const moe_gemm_desc* g, const void* A, const void* A_scales,
                            const int32_t* a_rows, const void* B, const void* B_scales,
                            const void* B2, const void* B2_scales, const int32_t* group_offsets,
                            void* C, void* C_scales, hipStream_t stream);

/* ---- combine (weighted un-permute) -------------------------------------------------------------
 * Defining passages: "CuTeDSL at Perplexity", section "MoE dispatch and combine": the combine
 * accumulates each token's weighted expert rows using the routing information and the offsets
 * the dispatch computed; "Hosting Qwen on Blackwell", section "Expert parallel": the local
 * contributions are summed first, before the cross-rank reduction (outside this library).
 * out[t, :] = sum_{j ascending, slot_to_row[t,j] >= 0} topk_w[t,j] * y[slot_to_row[t,j], :]
 *             (+ g_t * shared[t, :] if shared != NULL, g_t = shared_w[t], or 1 when shared_w is
 *             NULL), accumulated in fp32, rounded once to out_dtype.
 * y: [T*k, H] and shared: [T, H] (or NULL) in y_dtype (MOE_F32, MOE_BF16, or MOE_F16_SCALED
 * with rows of moe_f16_scaled_row_bytes(H) bytes, whose values are taken as f16 * scale, exact in
 * fp32); shared_w: [T] fp32
 * (or NULL; must be NULL when shared is); out: [T, H] in d->out_dtype. A token with no local
 * expert and no shared expert gets zeros. Pointers: 16-byte aligned. */
moe_status moe_combine(const moe_desc* d, int32_t y_dtype, const void* y, const float* topk_w,
                       const int32_t* slot_to_row, const void* shared, const float* shared_w,
                       void* out, hipStream_t stream);

/* ---- gate of the shared expert -------------------------------------------------------------------
 * shared_w[t] = 1 / (1 + exp(-(x_t . w_shared_gate))), the dot accumulated in fp32 over the H
 * columns of the unquantised token ("Hosting Qwen on Blackwell", introduction: the newer models'
 * additional gate terms; this per-token logistic gate of the shared expert is the reading taken).
 * x [T, H] and w_shared_gate [H] in d->io_dtype; shared_w [T] fp32, the combine's per-token factor
 * of the shared rows. Pointers: 16-byte aligned. */
moe_status moe_shared_gate(const moe_desc* d, const void* x, const void* w_shared_gate,
                           float* shared_w, hipStream_t stream);

/* ---- activation / weight quantiser -------------------------------------------------------------
 * Defining passages: "Hosting Qwen on Blackwell", section "Quantization" (block scaling as used for
 * DeepSeek-style models; MXFP8 for the MoE GEMMs); "CuTeDSL at Perplexity", section "Blackwell"
 * (scales from the absolute maximum of each small element group); "Driving vLLM WideEP and
 * Large-Scale Serving Toward Maturity on Blackwell (Part I)", lower-precision operations
 * (activations quantised before dispatch). The number formats are OCP 8-bit FP and OCP MX v1.0.
 * src [rows, cols] (src_dtype MOE_F32 or MOE_BF16) -> dst_dtype:
 *   MOE_FP8_E4M3: codes [rows, cols]; one fp32 scale per block_rows x 128 block
 *                 (scales [ceil(rows/block_rows), cols/128]): s = amax/448 (1 if amax = 0),
 *                 code = e4m3(v / s) rounded to nearest even with an IEEE fp32 division,
 *                 saturated to +-448. block_rows is 1 or 128.
 *   MOE_MXFP4:    packed [rows, cols/2], E8M0 scales [rows, cols/32]: per 32 elements
 *                 e = floor(log2(amax)) - 2 clamped to [-127,127] (-127 if amax = 0),
 *                 code = e2m1(v * 2^-e) rounded to nearest even, saturated to +-6 (OCP MX v1.0).
 *   MOE_MXFP8:    codes [rows, cols], E8M0 scales [rows, cols/32]: per 32 elements
 *                 e = floor(log2(amax)) - 8 clamped to [-127,127] (-127 if amax = 0),
 *                 code = e4m3(v * 2^-e) rounded to nearest even, saturated to +-448.
 *   MOE_NVFP4:    packed [rows, cols/2]; scales: one record per matrix (e4m3 block scales
 *                 [rows, cols/16], then fp32 row scales [rows]). Per row g = amax/2688 (1 if
 *                 that is 0); per 16 elements the scale code c = e4m3(bamax / (6 g)) (nearest
 *                 even, saturated), s its value, d = s * g; code = e2m1(v / d) (nearest even,
 *                 saturated to +-6; signed zeros when d = 0). Each step one IEEE fp32 operation.
 * Element signs are kept (a value rounding to zero keeps its sign bit). cols % 128 == 0 (FP8),
 * cols % 32 == 0 (MXFP4, MXFP8) or cols % 64 == 0 (NVFP4). `batch` stacked matrices are quantised independently (weights of
 * E_loc experts): src, codes and scales are then [batch, ...] of the shapes above. */
moe_status moe_quantize(int32_t dst_dtype, int32_t src_dtype, int32_t batch, int32_t rows,
                        int32_t cols, int32_t block_rows, const void* src, void* codes,
                        void* scales, hipStream_t stream);

/* ---- the whole layer ---------------------------------------------------------------------------
 * Defining passages: the steps above in the pages' order, route -> dispatch -> MoE GEMM ->
 * combine ("Hosting Qwen on Blackwell", section "Expert parallel"; "CuTeDSL at Perplexity",
 * section "MoE dispatch and combine"), plus the always-active shared expert of "How we served a
 * 397B MoE model with 4.7x speedup on TPU v7" (architectural constraints). The decode or prefill
 * kernel variants are chosen inside from the table sizes, as "CuTeDSL at Perplexity" chooses its
 * dispatch kernels (section on grid synchronisation).
 * Routing, dispatch, expert GEMMs (gate/up with the SwiGLU epilogue, then down), shared expert and
 * combine, all enqueued on `stream` with no host synchronisation. x [T, H] is io_dtype, out [T, H]
 * is out_dtype. logits [T,E], topk_ids [T,k], topk_w [T,k] are optional outputs (NULL: kept in the
 * workspace). out is this GPU's partial sum over its local experts plus the shared expert (times
 * its gate g_t when w->w_shared_gate is given).
 * Intermediate formats: h (the down projection's input) is in the expert format (bf16 for bf16
 * and NVFP4 experts); the per-slot expert outputs y are fp32 for fp32 experts, MOE_F16_SCALED for
 * bf16 experts and bf16 for fp8/MXFP4/MXFP8/NVFP4. NVFP4 layers quantise x per token (moe_quantize's rule) and run the
 * GEMMs on its block values with the row scales applied after each dot product.
 * ws: moe_layer_workspace_bytes(d) bytes. */
moe_status moe_layer(const moe_desc* d, const moe_weights* w, const void* x, const float* bias,
                     void* out, float* logits, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, hipStream_t stream);
size_t moe_layer_workspace_bytes(const moe_desc* d);

/* ---- the whole layer without a caller workspace --------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): moe_layer with the workspace taken from a fixed device
 * array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the process ends.
 * Arguments and results are those of moe_layer (inputs and outputs are still the caller's). Layers
 * whose moe_layer_workspace_bytes(d) exceeds MOE_NOALLOC_SCRATCH_BYTES (decode-sized layers fit;
 * e.g. 64 tokens of the Qwen3-235B slice need ~10 MiB) return MOE_ERR_WORKSPACE before anything is
 * launched. No device memory is allocated or freed. Every call on one GPU uses that GPU's array:
 * calls that overlap on one GPU (several streams, or host threads) race and must be ordered by the
 * caller. The array keeps the last call's contents; the layer writes every workspace byte it reads
 * within the call, so nothing needs clearing between calls. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_noalloc(const moe_desc* d, const moe_weights* w, const void* x,
                             const float* bias, void* out, float* logits, int32_t* topk_ids,
                             float* topk_w, hipStream_t stream);

const char* moe_status_str(moe_status s);
int32_t moe_last_hip_error(void);     /* hipError_t of the calling thread's last failed launch */

#ifdef __cplusplus
}
#endif
#endif
