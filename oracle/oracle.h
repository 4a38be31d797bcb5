/*
 * oracle.h -- plain, slow CPU reference of the MoE FFN layer (one GPU's expert slice).
 *
 * TEST INFRASTRUCTURE ONLY. This library is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg; the GPU library never links, loads or calls it, and it shares no
 * code with the GPU library.
 *
 * Every function works on host memory, in double precision unless a step's decision is defined in
 * fp32 (top-k selection on fp32 logits; the quantisers, whose codes are fp32 decisions).
 *
 * Sources (the pages, cited by title and section):
 *   [P1] "Hosting Qwen on Blackwell" (Perplexity): sections "Prefillers", "Expert parallel",
 *        "MoE GEMM", "Quantization".
 *   [P2] "How we served a 397B MoE model with 4.7x speedup on TPU v7" (infolabhq): sections on the
 *        architectural constraints (512 experts, top-10, shared expert), "Three collectives become
 *        two" (routing arrays [T,k] int + float), "Roofline validation".
 *   [P3] "CuTeDSL at Perplexity": section "MoE dispatch and combine" (local kernel: per-expert
 *        counts, unique index per token within its expert, copy into expert buffers, weighted
 *        combine using those positions), and the Blackwell section (absmax over 32 elements for
 *        MX formats).
 *   [P4] "Driving vLLM WideEP and Large-Scale Serving Toward Maturity on Blackwell (Part I)":
 *        section on lower-precision operations (4-bit MoE weights, two values per byte with
 *        per-group scales; activations quantised before dispatch).
 * The router function (softmax / sigmoid), SwiGLU, e4m3, e2m1 and E8M0 are not named on the pages;
 * they come from the workload definitions. e4m3 and e2m1/E8M0 follow the OCP 8-bit floating point
 * specification and the OCP Microscaling (MX) v1.0 specification. NVFP4 (e2m1 elements, one e4m3
 * scale per 16 along K: [P3] "Blackwell" section for the 16-element absmax groups, [P4] for 4-bit
 * weights with FP8 per-group scales) takes its second-level fp32 scale from NVIDIA's published
 * NVFP4 recipe (per tensor there; one per row here, see oracle_quant_nv4).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_SOFTMAX = 0, ORACLE_SIGMOID = 1 };

/* formats of a weight / activation matrix */
enum {
  ORACLE_F32 = 0,   /* float values (fp32 and bf16 workloads)                                   */
  ORACLE_BF16 = 1,  /* activation format only: h rounded to bf16 before the down projection      */
  ORACLE_FP8 = 2,   /* e4m3 codes [G,N,K] + fp32 scales [G, ceil(N/bn), ceil(K/bk)]           */
  ORACLE_MX4 = 3,   /* e2m1 codes, 2 per byte, [G,N,K/2] + E8M0 scales [G, N, K/32]            */
  ORACLE_MX8 = 4,   /* e4m3 codes [G,N,K] + E8M0 scales [G, N, K/32] (MXFP8)                    */
  ORACLE_NV4 = 5    /* NVFP4: e2m1 codes, 2 per byte, [G,N,K/2] + e4m3 block scales [G, N, K/16]
                       + fp32 row scales [G, N] (as an activation format: x arrives in NVFP4,
                       h is rounded to bf16)                                                    */
};

/* A stack of G matrices of shape [N, K] (K contiguous) in one of the formats above. */
typedef struct {
  int fmt;
  int G, N, K;
  int bn, bk;             /* fp8 block shape (rows x cols); ignored otherwise                     */
  const void* q;          /* float values, e4m3 codes, or packed e2m1 codes                       */
  const void* s;          /* NULL, fp32 block scales, E8M0 scale bytes or e4m3 scale bytes (NV4)   */
  const void* r;          /* NV4: fp32 row scales [G, N]; NULL otherwise                          */
} oracle_mat;

/* ---- number formats ------------------------------------------------------------------------ */
double  oracle_e4m3_value(uint8_t code);              /* OCP e4m3 code -> value (NaN for S.1111.111) */
uint8_t oracle_e4m3_encode(float v);                  /* round to nearest even, saturate to +-448    */
double  oracle_e2m1_value(uint8_t nibble);            /* OCP e2m1 code (4 bits) -> value             */
uint8_t oracle_e2m1_encode(float v);                  /* round to nearest even, saturate to +-6      */
double  oracle_e8m0_value(uint8_t code);              /* 2^(code-127)                                */
float   oracle_bf16_round(float v);                   /* nearest bf16 value, ties to even (finite v) */

/* fp8 quantiser: one fp32 scale per bn x bk block of a [rows, cols] matrix: s = amax/448 (1 if
 * amax = 0), code = e4m3(v / s) with an fp32 division. scales: [ceil(rows/bn), ceil(cols/bk)]. */
void oracle_quant_fp8(int rows, int cols, int bn, int bk, const float* src,
                      uint8_t* codes, float* scales);
/* MXFP4 quantiser: per row, per 32 consecutive columns: shared exponent
 * e = floor(log2(amax)) - 2 (clamped to [-127, 127]; -127 when amax = 0), E8M0 code e + 127,
 * element code = e2m1(v * 2^-e). Element 2i sits in bits 0-3 of byte i, element 2i+1 in bits 4-7.
 * cols % 32 == 0. packed: [rows, cols/2]; scales: [rows, cols/32]. */
void oracle_quant_mx4(int rows, int cols, const float* src, uint8_t* packed, uint8_t* scales);
/* MXFP8 (E4M3) quantiser: per row, per 32 consecutive columns: shared exponent
 * e = floor(log2(amax)) - 8 (8 is the largest e4m3 exponent; clamped to [-127, 127], -127 when
 * amax = 0), E8M0 code e + 127, element code = e4m3(v * 2^-e) rounded to nearest even and
 * saturated to +-448 (scaled values reach up to 2^9). cols % 32 == 0. codes: [rows, cols];
 * scales: [rows, cols/32]. */
void oracle_quant_mx8(int rows, int cols, const float* src, uint8_t* codes, uint8_t* scales);
/* NVFP4 quantiser, per row (cols % 16 == 0), every step an fp32 operation:
 *   g  = amax_row / 2688 (2688 = 6 * 448, so the largest block scale lands on e4m3's largest
 *        value; g = 1 when that quotient is 0, i.e. amax_row = 0), d6 = 6 * g;
 *   per 16 consecutive columns: scale code c_b = e4m3(bamax / d6) (nearest even, saturated),
 *        s = value of c_b, d = s * g;
 *   element code = e2m1(v / d) (nearest even, saturated to +-6); when d = 0 the codes are
 *        zeros that keep the element's sign.
 * The value of an element is e2m1(code) * s * g. packed: [rows, cols/2] (element 2i in bits 0-3
 * of byte i); bscales: [rows, cols/16] e4m3 codes; rscales: [rows] fp32 g. */
void oracle_quant_nv4(int rows, int cols, const float* src, uint8_t* packed, uint8_t* bscales,
                      float* rscales);

/* value of element (g, n, kk) of a matrix stack */
double oracle_mat_at(const oracle_mat* m, int g, int n, int kk);
/* dequantise a whole stack into doubles [G, N, K] */
void oracle_mat_dequant(const oracle_mat* m, double* out);

/* ---- routing --------------------------------------------------------------------------------- */
/* logits[t,e] = sum_h x[t,h] * w_r[e,h] + bias[e] in double; absdot[t,e] = sum |x*w| + |bias|
 * (both may be computed for a subset of tokens: tok = NULL means all T tokens, else n_tok token
 * indices; rows of the outputs follow the subset order). */
void oracle_logits(int T, int H, int E, const float* x, const float* w_r, const float* bias,
                   int n_tok, const int32_t* tok, double* logits, double* absdot);

/* top-k on fp32 logits [T,E]: the k largest values, equal values ranked by lower expert index,
 * listed in rank order; weights per scoring / renormalisation in double. */
void oracle_topk(int T, int E, int k, const float* logits, int scoring, int renormalize,
                 int32_t* ids, double* w);

/* ---- dispatch (permutation) -------------------------------------------------------------------- */
/* Stable, expert-major placement of the local slots: rows of local expert e' (0 <= e' < E_loc,
 * global id e0+e') appear in ascending flat index t*k+j. Returns R. slot_to_row = -1 for slots
 * whose expert is not local. row_to_flat must hold T*k entries (R are written). */
int oracle_permute(int T, int k, int e0, int E_loc, const int32_t* ids, int32_t* counts,
                   int32_t* offsets, int32_t* slot_to_row, int32_t* row_to_flat);

/* ---- expert FFN and the whole layer --------------------------------------------------------------- */
typedef struct {
  int T, H, E, e0, E_loc, I, k, I_s;
  int scoring, renormalize;
  int act_fmt;            /* format of h, the input of the down projection: ORACLE_F32: as
                             computed; ORACLE_BF16: rounded to bf16; ORACLE_FP8: e4m3 with 1x128
                             fp32 scales; ORACLE_MX4: MXFP4; ORACLE_MX8: MXFP8; ORACLE_NV4: rounded
                             to bf16 (x arrives pre-quantised in `xa` for the quantised formats) */
} oracle_desc;

/* SwiGLU FFN of one activation row a[H] through matrix g of the gate/up/down stacks:
 * h = silu(a . Wg^T) * (a . Wu^T), h quantised per act_fmt, y = h . Wd^T. y: [H]. */
void oracle_ffn_row(const oracle_desc* d, int I, const double* a, const oracle_mat* gate,
                    const oracle_mat* up, const oracle_mat* down, int g, double* y);

/* Gate of the shared expert, for n_tok tokens (tok = NULL: all T in order):
 *   g[i] = 1 / (1 + exp(-(x_t . w_sg))), t = tok[i], the dot over the H columns in double.
 * [P1], introduction: the layer adapts to the newer models' additional gate terms, whose form
 * the pages leave open; read as one learned projection of the unquantised token, through the
 * logistic function, scaling the always-active shared expert's output. */
void oracle_shared_gate(int T, int H, const float* x, const float* w_sg, int n_tok,
                        const int32_t* tok, double* g);

/* The layer for n_tok tokens (tok = NULL: all T in order):
 *   logits from the unquantised x and w_r (double, rounded to fp32 for the selection),
 *   top-k, then out[t] = sum_j w_tj * FFN_{e_tj}(a_t) over local slots (j ascending)
 *                        + g_t * FFN_shared(a_t) if I_s > 0,
 * where a_t is row t of `xa` (x itself, or x after the activation quantiser), and g_t is
 * oracle_shared_gate's value for token t if w_sg != NULL, else 1.
 * Optional outputs (NULL to skip): logits64 [n,E], logits32 [n,E], ids [n,k], w [n,k]. */
void oracle_moe_layer(const oracle_desc* d, const float* x, const float* w_r, const float* bias,
                      const oracle_mat* xa, const oracle_mat* gate, const oracle_mat* up,
                      const oracle_mat* down, const oracle_mat* sh_gate, const oracle_mat* sh_up,
                      const oracle_mat* sh_down, const float* w_sg, int n_tok,
                      const int32_t* tok, double* out, double* logits64, float* logits32,
                      int32_t* ids, double* w);

/* The expert part of the layer for a GIVEN routing: for i < n_tok, token t = tok[i] with chosen
 * experts ids[i, 0..k) and weights w[i, 0..k) (fp32, used as given),
 *   out[i] = sum_j w[i,j] * FFN_{ids[i,j]}(a_t) over local slots (j ascending)
 *            + g_t * FFN_shared(a_t) if I_s > 0,
 * with a_t and g_t as in oracle_moe_layer. Checks a GPU layer output on tokens whose routing the
 * GPU's fp32 logits decided differently from the oracle's fp64 logits (a near tie). */
void oracle_moe_layer_routed(const oracle_desc* d, const float* x, const oracle_mat* xa,
                             const oracle_mat* gate, const oracle_mat* up,
                             const oracle_mat* down, const oracle_mat* sh_gate,
                             const oracle_mat* sh_up, const oracle_mat* sh_down,
                             const float* w_sg, int n_tok, const int32_t* tok,
                             const int32_t* ids, const float* w, double* out);

/* ---- the grouped GEMM and the combine on their own ---------------------------------------------- */
/* For each group g and row r in [offsets[g], offsets[g+1]): with a(r) = a_rows ? a_rows[r] / div : r,
 *   d_n = sum_k A(a(r), k) * B(g, n, k) (+ bias[n]);  out[r, n] = d_n            (B2 == NULL)
 *   out[r, n] = silu(d_n) * sum_k A(a(r), k) * B2(g, n, k)                         (B2 != NULL)
 * A is a one-matrix stack [1, rows_a, K]; out is double [offsets[G], N]. */
void oracle_grouped_gemm(int G, const int32_t* offsets, const oracle_mat* A, const int32_t* a_rows,
                         int a_row_div, const oracle_mat* B, const oracle_mat* B2,
                         const float* bias, double* out);

/* out[t, :] = sum_{j ascending, slot_to_row[t,j] >= 0} w[t,j] * y[slot_to_row[t,j], :]
 *             (+ g_t * shared[t, :] if shared != NULL, g_t = shared_w[t], or 1 if shared_w is
 *             NULL); y, shared, shared_w float; out double [T, H]. */
void oracle_combine(int T, int H, int k, const float* y, const float* w, const int32_t* slot_to_row,
                    const float* shared, const float* shared_w, double* out);

int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
