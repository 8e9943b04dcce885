/*
 * qlora_nf4.h - C ABI of the MI355X (gfx950) QLoRA frozen-NF4 linear library.
 *
 * The library implements the storage and compute types of "QLoRA: Efficient
 * Finetuning of Quantized LLMs" (Dettmers et al., arXiv 2305.14314; cited
 * below as QLoRA, by section and equation):
 *   - blockwise 4-bit NormalFloat quantisation of a weight (section 2
 *     "Block-wise k-bit Quantization", Eq. 1; section 3 "4-bit NormalFloat
 *     Quantization"; Appendix E for the 16 values);
 *   - double quantisation of the per-block constants (section 3 "Double
 *     Quantization");
 *   - dequantisation to fp32 or bf16 (Eq. 2 read as multiplication by the
 *     block absmax, and Eq. 6);
 *   - the forward and backward of one linear layer with a LoRA adapter over
 *     the frozen NF4 weight (section 2 "Low-rank Adapters", Eq. 3; section 3
 *     "QLoRA", Eq. 5 and the paragraph after Eq. 6: gradients for the
 *     adapter and the input only, none for the weight).
 *
 * Conventions shared by every entry point
 *   Pointers.   Every buffer pointer is a DEVICE pointer into memory the
 *               caller allocated and owns; the library never allocates,
 *               frees, or keeps a pointer after a call returns.  Host-only
 *               outputs (sizes, the codebook) are host pointers and say so.
 *   Streams.    `stream` is a hipStream_t passed as void* (NULL = the null
 *               stream).  Every device entry point only enqueues kernels on
 *               that stream and returns without synchronising; results are
 *               ready when the stream reaches that point.
 *   Layouts.    Matrices are dense row-major with no padding between rows.
 *               The weight is [rows, cols] = [N, K] = [out, in]; its
 *               elements are taken in that flattened order for blocking.
 *   Types.      bf16 tensors are IEEE bfloat16 bit patterns (uint16).
 *   Alignment.  Every tensor pointer must be 16-byte aligned.
 *   Errors.     Every function returns QLORA_OK (0) or a negative
 *               qlora_status.  Arguments are validated on the host before
 *               anything is enqueued; on any validation failure nothing is
 *               enqueued and no buffer is touched.  QLORA_ERR_HIP reports a
 *               failed kernel launch (the HIP error text is kept).
 *               qlora_last_error() returns a message for the calling
 *               thread's most recent failure.
 *   Threads.    Calls on different streams are independent; the library
 *               holds no mutable global state besides the per-thread error
 *               message.
 *   Non-finite weights give undefined (but in-range) codes.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_ARG = -1,        /* null pointer, bad size, shape or flag   */
  QLORA_ERR_UNSUPPORTED_DTYPE = -2,  /* dtype code not accepted by this call     */
  QLORA_ERR_WORKSPACE_TOO_SMALL = -3,/* ws_bytes below what the call needs        */
  QLORA_ERR_MISALIGNED = -4,         /* a tensor pointer not 16-byte aligned      */
  QLORA_ERR_HIP = -5,                /* a kernel launch failed                     */
  QLORA_ERR_INTERNAL = -6            /* a library-internal table failed its check  */
} qlora_status;

typedef enum {
  QLORA_DTYPE_F32 = 0,
  QLORA_DTYPE_BF16 = 1
} qlora_dtype;

/* The 4-bit codebook a quantised weight's codes index (qlora_nf4_t's
 * code_type).  NF4 is QLoRA Appendix E (code 0 = -1.0, 7 = 0.0, 15 = 1.0).
 * The other three are the types QLoRA section 3 compares NF4 with (Table 2:
 * Int4, Float4 (E2M1), Float4 (E3M0)); the page gives no values, so each is
 * its bit-field definition with the largest magnitude normalised to 1:
 *   FP4_E2M1  code = s e1 e0 m, magnitude (m/2 for e = 0, else
 *             2^(e-1) (1 + m/2)) / 6 (the OCP microscaling 4-bit float);
 *   FP4_E3M0  code = s e2 e1 e0, magnitude 0 for e = 0, else 2^(e-7);
 *   INT4      code = two's-complement k, value k / 7 (Eq. 1 with 7 levels
 *             per side; code 8 = -8/7 is never produced by quantisation).
 * INT8 is the 8-bit type of QLoRA section 2, Eq. 1 (absmax scaling into
 * [-127, 127]) that section 3's Table 3 compares with NF4, read
 * blockwise with the same 64-blocks and double quantisation: one byte per
 * weight, the two's complement of k, value k / 127 (256 entries; byte 0x80,
 * -128/127, is never produced by quantisation).  Every entry point accepts
 * INT8 weights; the linear layer runs them on its 256 x 256 GEMM kernel
 * at every token count (the few-token weight-streaming kernel takes 4-bit
 * codes only).
 * Values are fp32 (the ratios rounded to nearest); qlora_codebook() returns
 * them. */
typedef enum {
  QLORA_CODE_NF4 = 0,
  QLORA_CODE_FP4_E2M1 = 1,
  QLORA_CODE_FP4_E3M0 = 2,
  QLORA_CODE_INT4 = 3,
  QLORA_CODE_INT8 = 4
} qlora_code_type;

/* Block sizes fixed by QLoRA section 3 ("QLoRA": block size 64 for W,
 * 256 for the first-level constants). */
#define QLORA_NF4_BLOCKSIZE 64
#define QLORA_NF4_BLOCKSIZE2 256
/* Largest LoRA rank accepted by the linear entry points. */
#define QLORA_MAX_RANK 256

/*
 * Descriptor of one 4-bit-quantised weight (the quantisation state).  Plain
 * data: the caller fills it and owns every buffer it points to.
 *
 *   rows, cols     weight shape [N, K]; numel = rows*cols, 0 < numel < 2^37.
 *   blocksize      must be 64;  nb = ceil(numel / 64) blocks, a short last
 *                  block takes its absmax over the elements that exist.
 *   blocksize2     must be 256; ng = ceil(nb / 256) groups of constants.
 *   double_quant   1: constants stored double-quantised (absmax_q, scale2,
 *                  offset used, absmax ignored); 0: absmax used.
 *   codes          u8[ceil(numel/2)]: two NF4 codes per byte, element 2j in
 *                  the low nibble, element 2j+1 in the high nibble; an odd
 *                  last element leaves the high nibble 0.  Code i stands for
 *                  the i-th Appendix E value (0 = -1.0, 7 = 0.0, 15 = 1.0).
 *   absmax_q       u8[nb]: OCP FP8 E4M3FN byte of (c2_b - mu) * 448 / c1_g,
 *                  nearest-even, saturating (QLoRA c2^FP8).
 *   absmax         f32[nb]: the block absmax c2_b (no double quantisation).
 *   scale2         f32[ng]: c1_g / 448 with c1_g = max |c2_b - mu| over the
 *                  group (QLoRA's second-level constant c1^FP32); 0 when the
 *                  group is constant.
 *   offset         f32[1]: mu, the mean of all c2_b, exact and rounded once
 *                  to fp32 (nearest-even).
 *   code_type      qlora_code_type of the codes (0 = NF4, the default).
 *                  The codes description above is NF4's; for the other 4-bit
 *                  types code i stands for value i of that type's codebook.
 *                  INT8: codes is u8[numel], one byte per element in order,
 *                  byte c standing for value c of the INT8 codebook.
 */
typedef struct qlora_nf4 {
  int64_t rows;
  int64_t cols;
  int32_t blocksize;
  int32_t blocksize2;
  int32_t double_quant;
  int32_t code_type;  /* qlora_code_type; 0 = NF4 */
  uint8_t* codes;
  uint8_t* absmax_q;
  float* absmax;
  float* scale2;
  float* offset;
} qlora_nf4_t;

/* ------------------------------------------------------------- host queries */

/* Host only.  Bytes of each buffer of the descriptor for `numel` weights:
 * bytes[0] codes, [1] absmax_q, [2] absmax, [3] scale2, [4] offset (entries
 * not used by the chosen double_quant are 0).  `bytes` is a host array of 5.
 * The total is the storage cost QLoRA section 3 "Double Quantization"
 * accounts: 4 + 32/64 bits per weight without double quantisation,
 * 4 + 8/64 + 32/(64*256) (+32/numel for mu) with it. */
int qlora_nf4_storage_bytes(int64_t numel, int32_t double_quant, int64_t* bytes);

/* Host only.  As qlora_nf4_storage_bytes for a weight of type `code_type`:
 * the same constants, and codes of ceil(numel / 2) bytes for the 4-bit types
 * or numel bytes for QLORA_CODE_INT8 (8 + 8/64 + 32/(64*256) bits per weight
 * with double quantisation). */
int qlora_storage_bytes(int64_t numel, int32_t double_quant, int32_t code_type, int64_t* bytes);

/* Host only.  Workspace bytes qlora_nf4_quantize needs (0 without double
 * quantisation).  Written to the host pointer *ws_bytes. */
int qlora_nf4_quantize_workspace(int64_t numel, int32_t double_quant, int64_t* ws_bytes);

/* Host only.  Workspace bytes qlora_linear_fwd / qlora_linear_bwd need for
 * an [M, K] x [N, K]^T layer of LoRA rank r (host pointers; either may be
 * NULL). */
int qlora_linear_workspace(int64_t M, int64_t N, int64_t K, int32_t r,
                           int64_t* fwd_bytes, int64_t* bwd_bytes);

/* Host only.  Copies the 16 NF4 values the library quantises against
 * (QLoRA Appendix E, code order) into the host array out[16]. */
int qlora_nf4_codebook(float* out);

/* Host only.  Copies the values of codebook `code_type` (a qlora_code_type,
 * code order) into the host array out: 16 values, or 256 for
 * QLORA_CODE_INT8 (out[256]). */
int qlora_codebook(int32_t code_type, float* out);

/* Text for a status code; never NULL. */
const char* qlora_status_string(int32_t status);

/* Message for the calling thread's last failed call ("" if none). */
const char* qlora_last_error(void);

/* ----------------------------------------------------------- quantisation */

/*
 * qlora_nf4_quantize - NF4-quantise a weight, optionally double-quantising
 * the block constants (QLoRA section 2 Eq. 1 and chunking; section 3
 * "4-bit NormalFloat Quantization" steps (1)-(3); section 3 "Double
 * Quantization").
 *
 *   w        device, [q->rows, q->cols] row-major, dtype w_dtype
 *            (QLORA_DTYPE_F32 or QLORA_DTYPE_BF16).
 *   q        host pointer to a filled descriptor; writes q->codes and either
 *            q->absmax (double_quant = 0) or q->absmax_q, q->scale2,
 *            q->offset (double_quant = 1).
 *   ws       device workspace of ws_bytes >= qlora_nf4_quantize_workspace
 *            (may be NULL when that is 0); contents on entry are ignored.
 *
 * Per block b of 64 flattened weights: c2_b = max |w| (exact); each weight
 * x = fp32(w * fp32(1/c2_b)) gets the code of the nearest value of the
 * q->code_type codebook, ties to the smaller value (for NF4, the lower
 * index); an all-zero block gets the code of 0.0 throughout (NF4: 7).  For
 * QLORA_CODE_INT8 this is Eq. 1 per block: the byte of k = round(127 x),
 * ties to the smaller k.  With double quantisation, mu = mean(c2) and each
 * group of 256 constants is stored as described for qlora_nf4_t.
 */
int qlora_nf4_quantize(const void* w, int32_t w_dtype, const qlora_nf4_t* q,
                       void* ws, int64_t ws_bytes, void* stream);

/*
 * qlora_nf4_quantize_batched - qlora_nf4_quantize of `count` weights in one
 * call (a model's weights at load time): the same codes and constants as
 * `count` separate calls, bit for bit, with one quantisation launch and one
 * double-quantisation launch per 32 weights instead of two launches per
 * weight.
 *
 *   w        host array of `count` device pointers; w[i] is weight i
 *            ([q[i].rows, q[i].cols], dtype w_dtype).
 *   q        host array of `count` descriptors; all must share code_type and
 *            double_quant (else QLORA_ERR_INVALID_ARG).
 *   count    0 <= count <= 4096 (0 enqueues nothing).
 *   ws       device workspace of ws_bytes >= qlora_nf4_quantize_batched_
 *            workspace(q, count) (the sum of the weights' own workspaces).
 * Every descriptor and pointer is validated before anything is enqueued.
 */
int qlora_nf4_quantize_batched_workspace(const qlora_nf4_t* q, int32_t count, int64_t* ws_bytes);
int qlora_nf4_quantize_batched(const void* const* w, int32_t w_dtype, const qlora_nf4_t* q,
                               int32_t count, void* ws, int64_t ws_bytes, void* stream);

/*
 * qlora_nf4_dequantize - doubleDequant of QLoRA Eq. 6 (or the single
 * dequant of Eq. 2 without double quantisation).
 *
 *   q        host pointer to a descriptor whose buffers hold a quantised
 *            weight.
 *   out      device, [rows, cols] row-major, dtype out_dtype (F32 or BF16).
 *
 * c2_hat_b = fp32(fp32(fp8(absmax_q_b) * scale2_g) + mu) (two roundings,
 * no fused multiply-add), or absmax_b; w_hat = fp32(value[code] * c2_hat_b)
 * with the q->code_type codebook;
 * bf16 output is w_hat rounded to nearest-even.
 */
int qlora_nf4_dequantize(const qlora_nf4_t* q, void* out, int32_t out_dtype, void* stream);

/* ----------------------------------------------------------- linear layer */

/*
 * qlora_linear_fwd - QLoRA Eq. 5 with the adapter scale of Eq. 3:
 *     Y = X * W_bf16^T + s * (X * A) * B
 * where W_bf16 is exactly what qlora_nf4_dequantize writes as BF16.
 *
 *   X        device bf16 [M, K]; M >= 0 (M = 0 enqueues nothing).
 *   W        host pointer to the descriptor of the frozen weight [N, K];
 *            K % 64 == 0 and N % 64 == 0; any code type (INT8 weights
 *            of 1-16 tokens run on the 256 x 256 GEMM kernel with split
 *            tiles, slower than the 4-bit weight-streaming path).
 *   A        device bf16 [K, r]  (QLoRA L1).
 *   B        device bf16 [r, N]  (QLoRA L2).
 *   r        LoRA rank, 1 <= r <= QLORA_MAX_RANK.
 *   s        adapter scale (alpha / r).
 *   Y        device bf16 [M, N], written.
 *   XA       device bf16 [M, r] or NULL; when given, receives X * A (fp32
 *            accumulation rounded to bf16) for the backward.
 *   ws       device workspace, ws_bytes >= the fwd figure of
 *            qlora_linear_workspace.
 * Products accumulate in fp32; the adapter term runs through bf16(s*X*A).
 * For 1 <= M <= 16 the weight term is computed by a weight-streaming kernel
 * that rounds the codebook value (not its product with c2_hat) to bf16 and
 * applies c2_hat in fp32 to each 64-term block product: the same size of
 * error, but not bit-identical to the product with W_bf16.
 */
int qlora_linear_fwd(const void* X, int64_t M, const qlora_nf4_t* W,
                     const void* A, const void* B, int32_t r, float s,
                     void* Y, void* XA, void* ws, int64_t ws_bytes, void* stream);

/*
 * qlora_linear_bwd - gradients of qlora_linear_fwd for an upstream dY
 * (QLoRA section 3 "QLoRA", paragraph after Eq. 6: only the adapter
 * gradients are needed, not dE/dW, and the input gradient goes through the
 * weight dequantised to BF16):
 *     T  = dY * B^T
 *     dX = dY * W_bf16 + s * T * A^T
 *     dA = s * X^T * T
 *     dB = s * XA^T * dY
 *
 *   dY       device bf16 [M, N].
 *   X        device bf16 [M, K] (the forward input).
 *   XA       device bf16 [M, r] as written by qlora_linear_fwd, or NULL: the
 *            call then recomputes X * A itself, bit-identical to what the
 *            forward writes for the same X, A and M (it costs one more
 *            read of X; the forward need not keep XA).
 *   W, A, B, r, s, M   as for qlora_linear_fwd.
 *   dX       device bf16 [M, K] or NULL (input gradient not wanted); always
 *            written, never added to.
 *   dA       device bf16 [K, r].
 *   dB       device bf16 [r, N].
 *   accumulate  0: dA and dB are written; 1: the gradients of this batch are
 *            added to the values dA and dB hold on entry, dA = bf16(dA +
 *            s X^T T) and likewise dB, so the gradients of several
 *            micro-batches (QLoRA Appendix B.2, Table 9 trains with batch
 *            sizes 16 to 64) sum in place with no caller-side temporary.
 *            Any other value is QLORA_ERR_INVALID_ARG.
 *   ws       device workspace, ws_bytes >= the bwd figure of
 *            qlora_linear_workspace (which includes the room for a
 *            recomputed XA).
 * With M = 0, dA and dB are set to zero (left as they are when
 * accumulating).  Products accumulate in fp32; T enters the products as
 * bf16(s * T).
 */
int qlora_linear_bwd(const void* dY, const void* X, const void* XA, int64_t M,
                     const qlora_nf4_t* W, const void* A, const void* B,
                     int32_t r, float s, void* dX, void* dA, void* dB,
                     int32_t accumulate, void* ws, int64_t ws_bytes, void* stream);

/*
 * qlora_linear_fwd_noalloc - qlora_linear_fwd for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, arguments and
 * results, with no workspace argument.  The workspace comes from a fixed
 * 96 MiB array of device memory the library holds on every GPU it runs on
 * (from the first use on that GPU until the process ends); the call itself
 * allocates and frees nothing.  Calls whose workspace (the fwd figure of
 * qlora_linear_workspace) exceeds 96 MiB return
 * QLORA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  The array is
 * shared by every call on one GPU: calls that overlap on the same GPU (on
 * different streams, or from different threads) race on it; serialise them.
 * The current HIP device must be the one `stream` belongs to.
 */
int qlora_linear_fwd_noalloc(const void* X, int64_t M, const qlora_nf4_t* W,
                             const void* A, const void* B, int32_t r, float s,
                             void* Y, void* XA, void* stream);

/* ------------------------------------------------- LoRA dropout variants */

/*
 * qlora_linear_fwd_dropout / qlora_linear_bwd_dropout - the layer with LoRA
 * dropout on the adapter input (QLoRA Appendix B.2 trains with LoRA dropout
 * 0.1 up to 13B and 0.05 for 33B and 65B; it is read as the usual dropout
 * of the adapter's input with inverted scaling):
 *     Y  = X * W_bf16^T + s * (drop(X) * A) * B,
 *     drop(X) = X * keep / (1 - p)
 *     dX = dY * W_bf16 + s * (T * A^T) * keep / (1 - p),  T = dY * B^T
 *     dA = s * drop(X)^T * T,   dB = s * XA^T * dY,   XA = drop(X) * A
 * The caller draws the mask (the library holds no random state):
 *   keep_mask  device u8 [M, K/8]: bit j of byte (m, c) is 1 when X[m, 8c + j]
 *              is kept; the backward must get the forward's mask.
 *   p          drop probability, 0 <= p < 1; kept elements are scaled by
 *              fp32(1 / (1 - p)).
 * Every other argument, the workspace size and the error behaviour are those
 * of qlora_linear_fwd / qlora_linear_bwd; XA returned by the forward (and
 * recomputed by the backward when XA is NULL) is drop(X) * A.  A null
 * keep_mask is QLORA_ERR_INVALID_ARG.
 */
int qlora_linear_fwd_dropout(const void* X, int64_t M, const qlora_nf4_t* W,
                             const void* A, const void* B, int32_t r, float s,
                             const void* keep_mask, float p,
                             void* Y, void* XA, void* ws, int64_t ws_bytes, void* stream);

int qlora_linear_bwd_dropout(const void* dY, const void* X, const void* XA, int64_t M,
                             const qlora_nf4_t* W, const void* A, const void* B,
                             int32_t r, float s, const void* keep_mask, float p,
                             void* dX, void* dA, void* dB, int32_t accumulate,
                             void* ws, int64_t ws_bytes, void* stream);

/*
 * qlora_dropout_mask - draws the keep mask of the dropout entry points on the
 * device (QLoRA Appendix B.2's LoRA dropout; each element kept with
 * probability 1 - p).  The draw is Philox4x64-10 (Salmon, Moraes, Dror,
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) and fully
 * determined by (seed, offset): byte b = m * (K/8) + c of the mask takes key
 * (seed, 0) and counter (b, offset, 0, 0); the generator's four 64-bit
 * outputs o_0..o_3 give eight 32-bit words u_j = o_{j/2} >> (32 (j % 2)),
 * and bit j (element X[m, 8c + j]) is 1 (kept) iff u_j >= floor(p * 2^32).
 * Use a new offset (or seed) for every layer and step; the backward must get
 * the forward's mask.
 *
 *   seed, offset  the key and the second counter word.
 *   M, K          the shape of the adapter input X [M, K]; K % 8 == 0.
 *   p             drop probability, 0 <= p < 1.
 *   keep_mask     device u8 [M, K/8], written (the layout the dropout entry
 *                 points take).
 * M = 0 enqueues nothing.  Bad sizes or p are QLORA_ERR_INVALID_ARG.
 */
int qlora_dropout_mask(uint64_t seed, uint64_t offset, int64_t M, int64_t K, float p,
                       void* keep_mask, void* stream);

/* --------------------------------------------- LoRA-only optimizer step */

/*
 * The update of the adapters (QLoRA section 3 "Paged Optimizers" and
 * Appendix B.2: Adam beta2 = 0.999, maximum gradient norm 0.3, constant
 * learning rate; only the LoRA parameters are trained).  Read as AdamW with
 * decoupled weight decay and global gradient-norm clipping, over one flat
 * buffer holding all LoRA parameters (their gradients can be the dA / dB
 * outputs of qlora_linear_bwd written into slices of one flat buffer).
 *
 * qlora_clip_scale_workspace - host only: workspace bytes of
 *   qlora_clip_scale for n gradient elements.
 *
 * qlora_clip_scale - device scalar *scale = min(1, max_norm / (||g||_2 +
 *   1e-6)) for the bf16 gradient grad [n] (device).  The sum of squares is
 *   taken in fp64 in a fixed order (bit-reproducible).  max_norm > 0.
 *
 * qlora_adamw_step - one step t = step (>= 1) of
 *     g' = g * (*grad_scale, or 1 when grad_scale is NULL)
 *     m = beta1 m + (1 - beta1) g';  v = beta2 v + (1 - beta2) g'^2
 *     p = p (1 - lr weight_decay) - (lr / (1 - beta1^t)) m /
 *         (sqrt(v) / sqrt(1 - beta2^t) + eps)
 *   in fp32 over n elements: param, exp_avg (m), exp_avg_sq (v) fp32 [n],
 *   updated in place; grad bf16 [n]; param_bf16 (bf16 [n] or NULL) receives
 *   the updated parameters rounded to bf16 (the operands of the next
 *   forward).  exp_avg and exp_avg_sq may be pinned host memory (the paged
 *   optimizer's evicted state): the kernel reads and writes them in place
 *   over the host link.  Requires 0 <= beta1, beta2 < 1, eps > 0, lr >= 0,
 *   weight_decay >= 0.
 */
int qlora_clip_scale_workspace(int64_t n, int64_t* ws_bytes);
int qlora_clip_scale(const void* grad, int64_t n, float max_norm, float* scale,
                     void* ws, int64_t ws_bytes, void* stream);
int qlora_adamw_step(float* param, void* param_bf16, const void* grad,
                     float* exp_avg, float* exp_avg_sq, int64_t n,
                     const float* grad_scale, float lr, float beta1, float beta2,
                     float eps, float weight_decay, int32_t step, void* stream);

/*
 * qlora_adamw_step_paged - qlora_adamw_step with the optimizer states paged
 * (QLoRA section 3 "Paged Optimizers": the states are evicted to CPU RAM
 * and paged back to the GPU for the update).  exp_avg and exp_avg_sq live
 * in pinned host memory (allocated pinned, e.g. hipHostMalloc; never
 * registered after the fact); the call pages them through the device
 * staging buffer in chunks: each chunk is copied in, updated by the same
 * kernel as device-resident states (so the results are bit-identical to
 * qlora_adamw_step on device states), and copied back.  param, param_bf16,
 * grad and grad_scale are device pointers as for qlora_adamw_step.
 *
 *   staging        device workspace of staging_bytes >= 4096: two slots of
 *                  (m, v) chunks; chunk = staging_bytes / 16 rounded down to
 *                  a multiple of 256 elements.
 *   copy_stream    a second stream (hipStream_t as void*) for the copies, or
 *                  NULL: with it the copies of one chunk overlap the update
 *                  of the other (ordered by events the call creates and
 *                  releases); without it everything runs in order on
 *                  `stream`.
 * In both cases `stream` reaches the end of the call only after the last
 * state is back in host memory.  Other arguments and errors as for
 * qlora_adamw_step; a staging buffer below 4096 bytes is
 * QLORA_ERR_WORKSPACE_TOO_SMALL.
 */
int qlora_adamw_step_paged(float* param, void* param_bf16, const void* grad,
                           float* exp_avg, float* exp_avg_sq, int64_t n,
                           const float* grad_scale, float lr, float beta1, float beta2,
                           float eps, float weight_decay, int32_t step,
                           void* staging, int64_t staging_bytes, void* stream, void* copy_stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
