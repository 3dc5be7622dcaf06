/*
 * qlora.h -- C ABI of the NF4 + double-quantisation + LoRA linear library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is QLoRA as described on these pages:
 *   [P2] "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com
 *        paper text), section "Method", paragraphs "4-bit NormalFloat
 *        Quantization" and "Double Quantization"; the abstract.
 *   [P1] "QLoRA: Efficient Fine-Tuning of Quantized Language Models"
 *        (mbrenndoerfer.com), section "Low-Rank Adaptation (LoRA)".
 *   [P3] "Efficient Language Model Fine-Tuning with QLoRA on
 *        Resource-Constrained Hardware" (marciocunha.net), the LoraConfig
 *        example (r, lora_alpha).
 *
 * Conventions shared by every call:
 *  - Pointers marked "device" are HIP device pointers; the library never
 *    allocates, frees or retains memory and keeps no pointer after return.
 *    Outputs are overwritten, never accumulated into.
 *  - Device work is enqueued asynchronously on `stream` (a hipStream_t;
 *    NULL means the default stream). A return of QLORA_OK means the work was
 *    enqueued; faults inside kernels surface at the caller's next
 *    synchronisation.
 *  - Arguments are validated before any HIP call. On any error nothing is
 *    launched and no output is touched. No C++ exception crosses the ABI.
 *  - Weights W are [N, K] row-major (out x in), flattened in C order for the
 *    blockwise format below. Activations are rows of tokens: X [M, K],
 *    Y [M, N]. LoRA adapters: A [r, K], B [N, r]. All bf16 row-major,
 *    contiguous. The layer is Y = X W~^T + s (X A^T) B^T.
 *  - Stored NF4 + DQ format of n weights (blocks of 64 weights, groups of
 *    256 blocks):
 *      codes  uint8[ceil(n/2)]   4-bit level indices, element 2i in the low
 *                                nibble of byte i (pad nibble 0 when n odd)
 *      c2     uint8[ceil(n/64)]  OCP FP8 E4M3 code of absmax_b / c1_g
 *      c1     float[ceil(ceil(n/64)/256)]  per-group max of absmax_b
 *    Dequantised weight: W^_i = fp32( q[code_i] * fp32( e4m3(c2_b) * c1_g ) );
 *    the matmul operand is W~ = bf16(W^) (round to nearest even).
 *
 * Thread safety: every call may be made concurrently from several host
 * threads; the only global state is immutable tables built once.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,        /* a required pointer is NULL                 */
  QLORA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent     */
  QLORA_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned           */
  QLORA_ERR_UNSUPPORTED = 4, /* a valid but unsupported mode or value      */
  QLORA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than needed   */
  QLORA_ERR_DEVICE = 6,      /* a HIP call failed (launch or device query) */
  QLORA_ERR_SCRATCH = 7      /* sizes need more than the fixed scratch of
                                qlora_linear_fwd_noalloc                  */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;

/* A quantised weight [rows=N, cols=K]: views into caller-owned device
 * memory holding the stored format above for n = rows * cols. */
typedef struct {
  const uint8_t* codes;
  const uint8_t* c2_fp8;
  const float* c1;
  int64_t rows; /* N, out features */
  int64_t cols; /* K, in features  */
} qlora_nf4_weight;

/* The 16 NF4 levels in ascending order, as float32 (code 0 = -1, code 7 = 0,
 * code 15 = +1). [P2] "4-bit NormalFloat Quantization": quantiles of N(0,1)
 * -- 9 on the positive side and 8 on the negative side, one of the two zeros
 * dropped -- normalised into [-1, 1]. The outermost quantile is taken at
 * probability 1 - (1/32 + 1/30)/2, a reading (the pages omit the value).
 * `out`: host memory, 16 floats. Synchronous, no GPU use.
 * Errors: QLORA_ERR_NULL if out is NULL. */
int qlora_nf4_levels(float out[16]);

/* Quantise n bf16 weights to NF4 with double quantisation.
 * [P2] "4-bit NormalFloat Quantization" step (3): each block of 64 is
 * divided by its absolute maximum (IEEE float32 division) and mapped to the
 * nearest level (a tie goes to the lower code; an all-zero block to code 7).
 * [P2] "Double Quantization": the block absmaxes are quantised again, to
 * FP8 E4M3 (round to nearest even) relative to the max of their group of
 * 256; a group whose max is 0 stores c1 = 0 and c2 = 0.
 * w_bf16: device, n bf16 (16-byte aligned). codes / c2_fp8 / c1: device
 * outputs sized as in the stored format (codes and c2 16-byte aligned,
 * c1 4-byte aligned). Weights must be finite (non-finite input gives
 * unspecified codes). Errors: NULL, SHAPE (n < 1 or n > 2^45 - 2^14), ALIGN,
 * DEVICE. */
int qlora_quantize_nf4_dq(const void* w_bf16, int64_t n, uint8_t* codes,
                          uint8_t* c2_fp8, float* c1, void* stream);

/* Dequantise n weights of the stored format: [P2] "Method": a stored weight
 * is dequantised to BFloat16 whenever it is used. out_dtype QLORA_F32 writes
 * W^ (float32, bit-exact per the formula above); QLORA_BF16 writes W~.
 * codes / c2_fp8 / c1: device inputs; out: device output of n elements,
 * 16-byte aligned. Errors: NULL, SHAPE (n < 1 or n > 2^43), ALIGN,
 * UNSUPPORTED (dtype), DEVICE. */
int qlora_dequant(const uint8_t* codes, const uint8_t* c2_fp8, const float* c1,
                  int64_t n, int out_dtype, void* out, void* stream);

/* Base product on the frozen weight alone (no adapters), dequantised in
 * LDS: [P2] "Method": dequantise to BFloat16, then matrix multiplication in
 * 16-bit (float32 accumulate, bf16 result).
 *   transposed == 0:  out [M, N] = act [M, K] W~^T   (forward orientation)
 *   transposed == 1:  out [M, K] = act [M, N] W~     (input-gradient orientation)
 * W: host struct of device views (K % 64 == 0). act, out: device bf16,
 * 16-byte aligned. One kernel launch, no workspace. Limits as for
 * qlora_linear_fwd. Errors: NULL, SHAPE, ALIGN, DEVICE. */
int qlora_nf4_matmul(const qlora_nf4_weight* W, const void* act, int64_t M, int transposed,
                     void* out, void* stream);

/* Workspace bytes needed by qlora_linear_fwd and qlora_linear_bwd for these
 * sizes (the larger of the two; 0 on invalid sizes). When a product has few
 * output tiles (M of a few hundred tokens), its reduction is split and the
 * float32 partial products live in the workspace; they are summed in a fixed
 * order, so results stay bit-identical from run to run. Calls that run
 * concurrently must not share a workspace. */
size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);

/* LoRA linear forward on the frozen quantised weight:
 *   T = X A^T (float32 [M, r]);  Y = X W~^T + scale * T B^T  (bf16 [M, N]).
 * [P1] "Low-Rank Adaptation (LoRA)": x_out = (W_q + B A) x_in with B d x r
 * and A r x d; [P2] "Method": W~ is the bf16 dequantised weight and the
 * product runs in 16-bit with float32 accumulation. scale = lora_alpha / r
 * ([P3] LoraConfig; a reading, the pages show no formula).
 * W: host struct of device views (rows N, cols K; K % 64 == 0).
 * X [M, K], A [r, K], B [N, r]: device bf16. Y [M, N]: device bf16 output.
 * T_save: device float32 [M, r] output, or NULL. ws: device workspace of at
 * least qlora_linear_workspace_bytes(M, N, K, r) bytes, 256-byte aligned.
 * Limits: 1 <= M, 1 <= N, 64 <= K, K % 64 == 0, 1 <= r <= 256, scale finite,
 * max(Mp, rp) * max(N, K, rp) < 2^31 with Mp = 64 ceil(M / 64),
 * rp = 64 ceil(r / 64) (32-bit indexing of every operand). Errors: NULL, SHAPE, ALIGN, UNSUPPORTED,
 * WORKSPACE, DEVICE. */
int qlora_linear_fwd(const qlora_nf4_weight* W, const void* X, const void* A,
                     const void* B, int64_t M, int64_t r, float scale, void* Y,
                     float* T_save, void* ws, size_t ws_bytes, void* stream);

/* qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The library's own scratch takes the
 * workspace's place: a fixed 64 MiB array per GPU, held from the library's
 * load until the process ends; this call allocates nothing and frees nothing.
 * Sizes whose forward workspace (qlora_linear_workspace_bytes covers it)
 * exceeds 64 MiB return QLORA_ERR_SCRATCH before any HIP call. `stream` must
 * belong to the current device (else QLORA_ERR_DEVICE). Every call on a GPU
 * shares that GPU's scratch, so calls that overlap in time on one GPU (other
 * streams, other host threads) race; calls ordered on one stream do not.
 * Results are those of qlora_linear_fwd bit for bit. Other arguments, limits
 * and errors as for qlora_linear_fwd. */
int qlora_linear_fwd_noalloc(const qlora_nf4_weight* W, const void* X, const void* A,
                             const void* B, int64_t M, int64_t r, float scale, void* Y,
                             float* T_save, void* stream);

/* Backward of qlora_linear_fwd for the upstream gradient dY [M, N] (bf16).
 * [P2] abstract: gradients flow through the frozen 4-bit weight into the
 * adapters only, so there is no weight gradient:
 *   U  = dY B                      (float32, internal)
 *   dX = dY W~ + scale * U A       (bf16 [M, K]; skipped when dX is NULL)
 *   dA = scale * U^T X             (bf16 [r, K])
 *   dB = scale * dY^T T            (bf16 [N, r]), T = X A^T
 * T_saved: the T_save of the forward (float32 [M, r]) or NULL to recompute.
 * Other arguments and limits as for qlora_linear_fwd. dA/dB are reduced in a
 * fixed order: results are bit-identical from run to run. */
int qlora_linear_bwd(const qlora_nf4_weight* W, const void* X, const void* A,
                     const void* B, const void* dY, const float* T_saved,
                     int64_t M, int64_t r, float scale, void* dX, void* dA,
                     void* dB, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Other 4-bit data types and the format without double quantisation.
 *
 * [P2] Introduction, contribution (1), compares NF4 with 4-bit Integers and
 * 4-bit Floats; [P2] "Double Quantization" prices fp32 block constants at
 * 32/64 = 0.5 bit per weight. The pages define neither comparison type; the
 * library takes the plainest common forms (readings), normalised like NF4
 * by the block absmax, with the exact zero at code 7 and the same nearest-
 * value rule (a tie goes to the lower code):
 *   QLORA_CB_NF4   the NF4 levels of qlora_nf4_levels
 *   QLORA_CB_INT4  k / 7 for k = -7 .. 7 at code k + 7
 *   QLORA_CB_FP4   the 15 distinct OCP E2M1 values (+-{0, .5, 1, 1.5, 2, 3,
 *                  4, 6}) over 6, ascending
 * Int4 and FP4 have 15 values; their code 15 repeats +1 and is never
 * produced by the quantiser.
 * Without double quantisation (double_quant = 0) the constants are the exact
 * block absmax, float32[ceil(n/64)], and W^_i = fp32(q[code_i] * absmax_b).
 * With it (double_quant = 1) they are c2 / c1 exactly as in the NF4 + DQ
 * format above. The codes are the same either way.
 * ------------------------------------------------------------------------- */
typedef enum { QLORA_CB_NF4 = 0, QLORA_CB_INT4 = 1, QLORA_CB_FP4 = 2 } qlora_codebook;

/* A quantised weight [rows=N, cols=K] in any supported format: views into
 * caller-owned device memory for n = rows * cols.
 *   consts: double_quant ? uint8 c2[ceil(n/64)] : float absmax[ceil(n/64)]
 *   c1:     double_quant ? float[ceil(ceil(n/64)/256)] : unused (may be NULL) */
typedef struct {
  const uint8_t* codes;
  const void* consts;
  const float* c1;
  int64_t rows;         /* N, out features */
  int64_t cols;         /* K, in features  */
  int32_t codebook;     /* qlora_codebook  */
  int32_t double_quant; /* 1 or 0          */
} qlora_4bit_weight;

/* The 16 levels of a data type, ascending, as float32 (host memory).
 * Synchronous, no GPU use. Errors: NULL, UNSUPPORTED (codebook). */
int qlora_levels(int codebook, float out[16]);

/* Quantise n bf16 weights with the given data type, with or without double
 * quantisation of the block constants. Codes as for qlora_quantize_nf4_dq
 * with the data type's levels. consts: device output, uint8[ceil(n/64)] (c2)
 * or float[ceil(n/64)] (absmax); c1: device output float[ceil(ceil(n/64)/256)]
 * when double_quant, else ignored. Alignment: w, codes, consts 16 bytes, c1
 * 4 bytes. Errors: NULL, SHAPE (n < 1 or n > 2^45 - 2^14), ALIGN,
 * UNSUPPORTED (codebook or double_quant out of range), DEVICE. */
int qlora_quantize_4bit(const void* w_bf16, int64_t n, int codebook, int double_quant,
                        uint8_t* codes, void* consts, float* c1, void* stream);

/* Quantise count (1 .. 16) tensors with one launch, as qlora_quantize_4bit
 * would quantise each (bulk quantisation of a model: one launch per layer
 * instead of one per tensor). w_bf16, n, codes, consts, c1: host arrays of
 * count entries holding each tensor's device pointers and size (c1 ignored,
 * and may be NULL, without double quantisation). Errors: NULL, SHAPE (count
 * out of range, an n < 1, more than 2^31 - 1 groups of 16384 in all),
 * ALIGN, UNSUPPORTED, DEVICE; nothing is launched on any error. */
int qlora_quantize_4bit_batch(int count, const void* const* w_bf16, const int64_t* n,
                              int codebook, int double_quant, uint8_t* const* codes,
                              void* const* consts, float* const* c1, void* stream);

/* Dequantise n weights of a stored 4-bit format to float32 (W^) or bf16
 * (W~): [P2] "Method". Inputs as written by qlora_quantize_4bit with the
 * same codebook and double_quant. Errors: NULL, SHAPE (n < 1 or n > 2^43),
 * ALIGN, UNSUPPORTED, DEVICE. */
int qlora_dequant_4bit(const uint8_t* codes, const void* consts, const float* c1, int64_t n,
                       int codebook, int double_quant, int out_dtype, void* out, void* stream);

/* qlora_nf4_matmul, qlora_linear_fwd and qlora_linear_bwd for a weight in
 * any supported format; arguments, limits, workspace and errors as there,
 * plus UNSUPPORTED for a codebook or double_quant out of range. */
int qlora_4bit_matmul(const qlora_4bit_weight* W, const void* act, int64_t M, int transposed,
                      void* out, void* stream);

/* The base product with a rank term fused into its epilogue:
 *   transposed = 0:  out = act W~^T + L R^T   (act [M, K], out [M, N])
 *   transposed = 1:  out = act W~   + L R^T   (act [M, N], out [M, K])
 * L [M, rp] and R [Nout, rp] are bf16 (Nout = N, or K when transposed), rp a
 * multiple of 64; float32 accumulation of both products, one bf16 rounding.
 * This is the kernel the linear layer runs from 17 tokens on: the forward's
 * epilogue adds (scale T) B^T and the input gradient's (scale U) A ([P1]
 * "Low-Rank Adaptation (LoRA)"; [P2] "Method" for the bf16 product); callers
 * that hold their own rank factors, and timing of the fused GEMM alone, use it
 * directly. One kernel launch, no workspace (the reduction is never split
 * here). W: host struct of device views (K % 64 == 0); act, L, R, out:
 * device, 16-byte aligned, row-major, contiguous. Limits as qlora_nf4_matmul
 * plus 64 <= rp <= 4096, rp % 64 == 0, max(M, Nout) rp < 2^31.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, DEVICE. */
int qlora_4bit_matmul_lora(const qlora_4bit_weight* W, const void* act, int64_t M, int transposed,
                           const void* L, const void* R, int64_t rp, void* out, void* stream);
int qlora_linear_fwd_4bit(const qlora_4bit_weight* W, const void* X, const void* A,
                          const void* B, int64_t M, int64_t r, float scale, void* Y,
                          float* T_save, void* ws, size_t ws_bytes, void* stream);
int qlora_linear_bwd_4bit(const qlora_4bit_weight* W, const void* X, const void* A,
                          const void* B, const void* dY, const float* T_saved,
                          int64_t M, int64_t r, float scale, void* dX, void* dA,
                          void* dB, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Grouped linears: several LoRA linears that share one input, as q / k / v
 * (and gate / up) of a decoder layer do.
 *
 * [P2] Introduction (adapters at every network layer) with the layer rule of
 * qlora_linear_fwd: g segments, segment i with weight W_i [Ns, K] and its own
 * adapters A_i [r, K], B_i [Ns, r]:
 *   Y_i = X W_i~^T + scale (X A_i^T) B_i^T             (Y = [Y_1 .. Y_g])
 *   dX  = sum_i (dY_i W_i~ + scale U_i A_i),  U_i = dY_i B_i
 *   dA_i = scale U_i^T X,  dB_i = scale dY_i^T T_i,  T_i = X A_i^T
 * Layouts: W stacks the segments' weights by rows, [g Ns, K], in one stored
 * 4-bit format (quantising the stacked bf16 weight gives the same codes and
 * constants as quantising each W_i when Ns K % 16384 == 0). A stacks the
 * A_i: [g r, K]. B stacks the B_i: [g Ns, r]. X [M, K]; Y and dY [M, g Ns];
 * T_save / T_saved float32 [M, g r] (T_i in columns i r ..); dX [M, K];
 * dA [g r, K]; dB [g Ns, r]. The input is read once for all segments (the
 * projections X A^T and the dA pass), the summed dX comes from one GEMM.
 * Limits: 1 <= groups <= 16; for groups > 1, Ns % 256 == 0 and r % 64 == 0;
 * otherwise as for qlora_linear_fwd (with N = g Ns). groups == 1 is
 * qlora_linear_fwd / _bwd. Errors as there.
 * ------------------------------------------------------------------------- */
size_t qlora_linear_grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r,
                                            int64_t groups);
int qlora_linear_fwd_grouped(const qlora_4bit_weight* W, int64_t groups, const void* X,
                             const void* A, const void* B, int64_t M, int64_t r, float scale,
                             void* Y, float* T_save, void* ws, size_t ws_bytes, void* stream);
int qlora_linear_bwd_grouped(const qlora_4bit_weight* W, int64_t groups, const void* X,
                             const void* A, const void* B, const void* dY,
                             const float* T_saved, int64_t M, int64_t r, float scale,
                             void* dX, void* dA, void* dB, void* ws, size_t ws_bytes,
                             void* stream);

/* Merged weight for deployment: [P1] "Low-Rank Adaptation (LoRA)": the
 * adapted layer is x_out = (W_q + B A) x_in, so the adapters can be folded
 * into one dense weight:
 *   out[n][k] = bf16( fp32( W^[n][k] + fp32(scale * sum_j B[n][j] A[j][k]) ) )
 * with W^ the exact float32 dequantised weight of W (any stored format), the
 * sum over j in float32 (K % 64 == 0: on the matrix cores, bf16 products
 * exact, sums in their order; otherwise ascending j with fused multiply-
 * add; either way within (r + 2) u (|W^| + scale sum_j |B A|) of the exact
 * value, u = 2^-24), one final rounding to bf16 (nearest even). A [r, K], B [N, r]: device bf16; out:
 * device bf16 [N, K]. 1 <= r <= 256. Errors: NULL, SHAPE, ALIGN,
 * UNSUPPORTED (format or non-finite scale), DEVICE. */
int qlora_merge_lora(const qlora_4bit_weight* W, const void* A, const void* B, int64_t r,
                     float scale, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Optimizer step of the adapters, with paged optimizer state.
 *
 * [P1] "Paged Optimizers" and [P2] Introduction, contribution (3): optimizer
 * state may be moved to CPU memory while GPU memory is short. The pages name
 * no update rule; the library implements AdamW (a reading): per parameter,
 *   m <- beta1 m + (1 - beta1) g;   v <- beta2 v + (1 - beta2) g^2
 *   p <- p - lr (weight_decay p + m_hat / (sqrt(v_hat) + eps)),
 *   m_hat = m / (1 - beta1^step),   v_hat = v / (1 - beta2^step)
 * in float32 (each operation rounded to nearest), with g the bf16 gradient
 * as qlora_linear_bwd writes it (dA, dB).
 * "Paged": every array may be device memory or pinned host memory
 * (hipHostMalloc); the kernel then reads and writes the host copy in place
 * over the host link, so optimizer state paged out to the host needs no copy
 * back before a step. Pageable (unregistered) and managed memory are
 * refused (QLORA_ERR_UNSUPPORTED): this GPU configuration does not take page
 * faults, so nothing migrates on demand.
 * ------------------------------------------------------------------------- */
typedef struct {
  float lr;           /* >= 0 */
  float beta1;        /* in [0, 1) */
  float beta2;        /* in [0, 1) */
  float eps;          /* > 0 */
  float weight_decay; /* >= 0 */
  int64_t step;       /* 1 for the first step */
} qlora_adamw_params;

/* One AdamW step over n parameters, in place.
 * param_f32: float32 master weights [n] (updated). param_bf16: bf16 [n]
 * receiving bf16(updated weight) for the next forward, or NULL. grad_bf16:
 * bf16 gradient [n]. m, v: float32 moments [n] (updated; zero before step
 * 1). All 16-byte aligned; device or pinned host memory; the arrays must not
 * overlap. Errors: NULL, SHAPE (n < 1 or n > 2^40), ALIGN, UNSUPPORTED (a
 * parameter out of range, or memory that is neither device nor pinned host), DEVICE. */
int qlora_adamw_step(float* param_f32, void* param_bf16, const void* grad_bf16, float* m,
                     float* v, int64_t n, const qlora_adamw_params* h, void* stream);

/* Static text for a status code ("unknown status" for other values). */
const char* qlora_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
