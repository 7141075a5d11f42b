/*
 * fourtune.h - C ABI of libfourtune.so: FourTune's W4A4G4 triple-branch
 * linear layer on AMD Instinct MI355X (gfx950).
 *
 * Method: FourTune (arXiv 2607.05711).  "3.1 Triple-Branch Hybrid-Precision
 * Pipeline", Eq. (2): the forward adds a 4-bit product of the quantized
 * input and the quantized frozen residual weight, a frozen high-precision
 * low-rank stabilizer L1 L2 and a trainable LoRA adapter A B, all reading
 * the same input.  "3.2 4-Bit Backward Pass via Block-Quantization", Eq. (3):
 * the input gradient runs through the same three branches, the 4-bit
 * backbone with the *same* block-quantized weight read transposed, and only
 * the adapter receives weight gradients.  "3.3 Kernel Fusion": quantization
 * and the low-rank down-projections share one read of the input, and the
 * up-projections are accumulated inside the 4-bit GEMM.
 *
 * Number format: MXFP4 (OCP Microscaling v1.0, cited by the paper in "2.3
 * Model Quantization"): E2M1 elements, one E8M0 power-of-two scale per
 * block, scale exponent floor(log2(amax)) - 2, round to nearest with ties
 * to even, saturating at 6.  Blocks are 1x32 along the reduction dimension
 * for activations and gradients, and 32x32 square tiles (one scale per
 * tile) for the frozen residual weight.
 *
 * Shapes (the method's notation):
 *   X   [M, K] bf16      input             dY  [M, N] bf16  incoming gradient
 *   W_res [N, K]         frozen residual (like torch.nn.Linear.weight),
 *                        given as MXFP4 32x32 tiles
 *   L1  [K, r_stab], L2 [r_stab, N]        frozen stabilizer, bf16
 *   A   [K, r_lora], B  [r_lora, N]        trainable adapter, bf16
 *   D = [L1 | A]  [K, R],  V = [L2 ; B]  [R, N],  R = r_stab + r_lora <= 128
 *
 *   forward : Y  = deq(Qrow(X)) deq(Qtile(W_res))^T + U V,   U = bf16(X D)
 *   backward: dX = deq(Qrow(dY)) deq(Qtile(W_res)) + P D^T,  P = bf16(dY V^T)
 *             dA = X^T P[:, r_stab:]          dB = U[:, r_stab:]^T dY
 *
 * Every product accumulates in fp32 and is rounded once to the output type.
 *
 * Storage of the factors: every low-rank factor is stored rank-major, one
 * row per rank: L1 and A as their transposes L1^T [r_stab, K] and A^T
 * [r_lora, K] (the torch.nn.Linear.weight orientation of the
 * down-projections), L2 [r_stab, N] and B [r_lora, N] as they are.  The
 * adapter gradients come back the same way: dA^T [r_lora, K] and dB
 * [r_lora, N].  The weight is stored once, as MXFP4 32x32 tiles [N, K/2]
 * with tile scales [N/32, K/32]: the forward reads its rows, the input
 * gradient reads the same bytes transposed (one scale per tile, so the
 * transpose of the quantized weight is exactly these numbers).
 *
 * Memory layouts (all row-major, no padding between rows):
 *   bf16 tensors are arrays of uint16_t bit patterns.
 *   MXFP4 codes: byte i of a row holds element 2i in its low nibble and
 *   element 2i+1 in its high nibble; bit 3 of a nibble is the sign.
 *   Row-block scales [rows, cols/32]; tile scales [rows/32, cols/32]; one
 *   E8M0 byte each (value 2^(byte-127)).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers owned by the caller, except the ft_linear
 *     descriptor itself, which is host memory read during the call only.
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = default stream);
 *     the call returns without synchronizing.  The library allocates and
 *     frees nothing and keeps no pointer after it returns (exceptions: the
 *     opt-in per-kernel timing helpers at the end, which create events and
 *     wait for them, and the scratch array of fourtune_linear_fwd_noalloc,
 *     set up on its first call on a GPU).
 *   - All checks run on the host before anything is enqueued: a call that
 *     returns an error has enqueued no work and written no device memory.
 *   - Device pointers must be 16-byte aligned.  Inputs must be finite; NaN
 *     or Inf inputs give unspecified (but in-bounds) results.
 *   - Calls on different streams must use distinct workspaces and outputs.
 */
#ifndef FOURTUNE_H
#define FOURTUNE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FT_OK = 0,
  FT_EINVAL = 1,       /* null pointer where one is required, bad enum value   */
  FT_ESHAPE = 2,       /* size not allowed (K or N not multiple of 32, R > 128) */
  FT_EALIGN = 3,       /* device pointer not 16-byte aligned, or bad row stride */
  FT_EWORKSPACE = 4,   /* workspace smaller than fourtune_workspace_bytes       */
  FT_EDEVICE = 5,      /* a HIP launch failed                                   */
  FT_EUNSUPPORTED = 6  /* no GPU of the supported architecture (gfx950)         */
} ft_status;

typedef enum { FT_BF16 = 0, FT_F32 = 1 } ft_dtype;

typedef enum {
  FT_Q_ROW32 = 1,    /* 1x32 blocks along each row                                   */
  FT_Q_ROW32_T = 2,  /* ROW32 of the input and, from the same read, ROW32 of its
                        transpose                                                     */
  FT_Q_TILE32 = 4    /* 32x32 square tiles, one scale per tile (weights)             */
} ft_qmode;

/* Activation next to a linear (FourTune, "3.3 Kernel Fusion for Efficiency /
 * MLP Fusion": the GeLU between the two linears of an MLP block). */
typedef enum {
  FT_ACT_NONE = 0,
  FT_ACT_GELU_TANH = 1   /* gelu(h) = h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3))) / 2,
                            evaluated in fp32, rounded to bf16 once                  */
} ft_act;

/* Precision of the two backbone products (FourTune, "4.3 Ablation Study /
 * Impact of Precision Configurations", Table 4).  The weight is 4-bit in
 * all four; A16 keeps the forward's input in bf16 in the backbone product,
 * G16 the incoming gradient in the input-gradient product.  A 16-bit side
 * multiplies bf16 by the weight's MXFP4 tiles dequantized to bf16 (exact:
 * every dequantized value is a short bf16 number), made in the workspace by
 * each call; the low-rank branches and the adapter gradients are the same
 * in all four.  Only W4A4G4 runs both products on the 4-bit matrix cores. */
typedef enum {
  FT_W4A4G4 = 0,
  FT_W4A16G4 = 1,    /* bit 0: A16 */
  FT_W4A4G16 = 2,    /* bit 1: G16 */
  FT_W4A16G16 = 3
} ft_precision;

/* Storage of the residual weight (FourTune, "3.2 4-Bit Backward Pass via
 * Block-Quantization"; "4.3 Ablation Study / Impact of Quantization
 * Granularity", Table 5).
 * TILE32 is the method: 32x32 tiles stored once, [N, K/2] codes and
 * [N/32, K/32] scales; the dgrad reads the same bytes transposed.
 * TILE32_T: the same tiles plus a stored transposed layout copy of them
 * (wt_codes [K, N/2], wt_scales [K/32, N/32], as FT_Q_TILE32 writes into
 * codes_t / scales_t), which the dgrad reads row-wise instead; a measured
 * alternative that holds the 4-bit weight twice.
 * ROW32 is the group-wise alternative: 1x32 blocks along the reduction of
 * each product, so the forward reads Qrow32(W_res) and the dgrad a separate
 * quantization Qrow32(W_res^T) (which FT_Q_ROW32_T of W_res writes beside
 * the first from one read).  ROW32 requires precision FT_W4A4G4. */
typedef enum {
  FT_WBLOCK_TILE32 = 0,
  FT_WBLOCK_ROW32 = 1,
  FT_WBLOCK_TILE32_T = 2
} ft_wblock;

#define FT_MAX_RANK 128

/* One triple-branch linear layer.  Host struct; the pointers in it are device
 * pointers.  Either rank may be 0 (then its two pointers may be NULL). */
typedef struct {
  int64_t M, K, N;            /* tokens, input features, output features            */
  int32_t r_stab, r_lora;     /* stabilizer and adapter ranks, r_stab + r_lora <= 128 */
  const uint8_t* w_codes;     /* Qtile(W_res) codes  [N, K/2] (ROW32: Qrow32(W_res))  */
  const uint8_t* w_scales;    /* Qtile(W_res) scales [N/32, K/32]; ROW32: [N, K/32]   */
  const uint8_t* wt_codes;    /* the dgrad's separately stored weight, read only by a */
  const uint8_t* wt_scales;   /*   backward with dX: NULL for TILE32 (the method);   */
                              /*   TILE32_T: transposed copy [K, N/2], [K/32, N/32];  */
                              /*   ROW32: Qrow32(W_res^T) [K, N/2], scales [K, N/32]  */
  const uint16_t* L1t;        /* bf16 [r_stab, K] = L1^T  (frozen)                    */
  const uint16_t* L2;         /* bf16 [r_stab, N]  (frozen)                           */
  const uint16_t* At;         /* bf16 [r_lora, K] = A^T  (trainable)                  */
  const uint16_t* B;          /* bf16 [r_lora, N]  (trainable)                        */
  int32_t act_in;             /* FT_ACT_*: the layer's input is act_in(X): X given to the
                                 forward and backward is the pre-activation h, and act(h)
                                 is recomputed wherever it is read, never stored         */
  int32_t act_out;            /* FT_ACT_*: an activation follows this layer: the backward's
                                 dY is the gradient of act_out(Y), and H = Y is required */
  int32_t precision;          /* FT_W4A4G4 (0, the method) .. FT_W4A16G16                */
  int32_t w_block;            /* FT_WBLOCK_TILE32 (0, the method), _ROW32 or _TILE32_T */
} ft_linear;

/* Quantize a bf16 matrix `in` [rows, cols] with row stride ld_in elements.
 *
 * Paper: "2.3 Model Quantization" (Round(W/s) with a block scale, MXFP4);
 * "3.2 4-Bit Backward Pass via Block-Quantization" (square blocks whose
 * scales stay local, so the weight serves the transposed product as is).
 *
 * mode FT_Q_ROW32:   codes [rows, cols/2], scales [rows, cols/32];
 *                    codes_t and scales_t must be NULL.
 * mode FT_Q_ROW32_T: as ROW32, plus codes_t [cols, rows/2] and
 *                    scales_t [cols, rows/32] = ROW32 of in^T; rows % 32 == 0.
 * mode FT_Q_TILE32:  codes [rows, cols/2], scales [rows/32, cols/32];
 *                    rows % 32 == 0; codes_t [cols, rows/2] and scales_t
 *                    [cols/32, rows/32] are optional (both NULL or both set)
 *                    and receive the transposed copy.
 * Requirements: cols % 32 == 0, rows >= 0, ld_in >= cols, ld_in % 8 == 0.
 * rows == 0 is a no-op.
 * Errors: FT_EINVAL (mode, NULLs), FT_ESHAPE, FT_EALIGN. */
ft_status fourtune_quantize(int mode, const uint16_t* in, int64_t rows, int64_t cols,
                            int64_t ld_in, uint8_t* codes, uint8_t* scales,
                            uint8_t* codes_t, uint8_t* scales_t, void* stream);

/* MXFP4 back to bf16: each value is its E2M1 element times its block's
 * power-of-two scale (FourTune, "2.3 Model Quantization"; the 16-bit
 * precision settings of "4.3 Ablation Study" multiply by the weight in this
 * form).
 * mode FT_Q_TILE32 only: codes [rows, cols/2] and tile scales [rows/32,
 * cols/32] in, out bf16 [rows, cols].  Exact for every code and scale byte
 * (bf16 subnormals included) except scale bytes 253 and 254, which no finite
 * bf16 input is quantized to and whose largest elements overflow to Inf.
 * Requirements: rows % 32 == 0, cols % 32 == 0, rows, cols >= 0,
 * rows * cols * 2 < 2^31, pointers 16-byte aligned.  rows == 0 is a no-op.
 * Errors: FT_EINVAL (mode, NULLs), FT_ESHAPE, FT_EALIGN, FT_EDEVICE,
 * FT_EUNSUPPORTED. */
ft_status fourtune_dequantize(int mode, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                              int64_t cols, uint16_t* out, void* stream);

/* Bytes of device workspace fwd (is_bwd = 0) or bwd (is_bwd = 1) needs for
 * layer L (shapes, ranks, precision and w_block only are read).  Returns 0
 * for invalid shapes or enum values. */
size_t fourtune_workspace_bytes(const ft_linear* L, int is_bwd);

/* Forward, Eq. (2), with the fusions of "3.3 Kernel Fusion":
 *   kernel 1 reads X once and writes Qrow(X) and U = bf16(X D);
 *   kernel 2 computes deq(Qrow(X)) deq(Qtile(W_res))^T + U V in fp32 and
 *   writes Y (bf16 [M, N]) once.
 * With act_in != FT_ACT_NONE, X is the pre-activation h and kernel 1 applies
 * act_in to every value as it reads it (the quantized input and U are those
 * of act_in(h)).
 * Under A16 (precision bit 0) kernel 1 computes U only, the weight's tiles
 * are dequantized to bf16 in the workspace, and kernel 2 multiplies bf16 X
 * (act_in(X) when set, made in the workspace first) by them.
 * U_save  : bf16 [M, R], written; the backward needs it.  May be NULL if R == 0.
 * xq_codes, xq_scales: optional outputs [M, K/2], [M, K/32]; NULL = keep
 *   them in the workspace.  Must be NULL under A16 (there are no codes).
 * workspace: device memory of at least fourtune_workspace_bytes(L, 0) bytes;
 *   contents on entry are ignored and on return unspecified.
 * Requirements: M >= 1, K % 32 == 0, N % 32 == 0, R <= 128, and every
 *   activation padded to 256 more rows below 2^31 bytes:
 *   (M + 256) * max(K, N) * 2 < 2^31 (the kernels use 32-bit offsets);
 *   under A16 or G16 the same for the dequantized weight,
 *   (max(K, N) + 256) * min(K, N) * 2 < 2^31; precision in 0..3; w_block
 *   FT_WBLOCK_TILE32 or FT_WBLOCK_ROW32 (ROW32 with FT_W4A4G4 only).
 * Errors: FT_EINVAL, FT_ESHAPE, FT_EALIGN, FT_EWORKSPACE, FT_EDEVICE. */
ft_status fourtune_linear_fwd(const ft_linear* L, const uint16_t* X, uint16_t* Y,
                              uint16_t* U_save, uint8_t* xq_codes, uint8_t* xq_scales,
                              void* workspace, size_t ws_bytes, void* stream);

/* The forward above for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and checks as fourtune_linear_fwd
 * without workspace and ws_bytes: the workspace is a device array of
 * FT_NOALLOC_SCRATCH_BYTES that the library holds on each GPU until the
 * process ends, located on the first call made with that GPU current.
 * The call itself allocates nothing (no hipMalloc, no library routine that
 * allocates; the per-kernel timing below is skipped for it).
 * Layers whose forward workspace (fourtune_workspace_bytes(L, 0)) exceeds
 * FT_NOALLOC_SCRATCH_BYTES are refused with FT_EWORKSPACE before anything
 * is enqueued.  Every call on one GPU shares that GPU's array and leaves
 * it in an unspecified state (nothing in it needs clearing between
 * calls): calls that overlap on one GPU (different streams, or host
 * threads racing) race on it and give unspecified results; calls in order
 * on one stream are safe.
 * Errors: as fourtune_linear_fwd; FT_EDEVICE also if the array cannot be
 * located on the current GPU. */
#define FT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ft_status fourtune_linear_fwd_noalloc(const ft_linear* L, const uint16_t* X, uint16_t* Y,
                                      uint16_t* U_save, uint8_t* xq_codes, uint8_t* xq_scales,
                                      void* stream);

/* Backward, Eq. (3) and the adapter gradients of section 3.2:
 *   kernel 1 reads dY once and writes Qrow(dY) (1x32 blocks along N, the
 *   reduction dimension of the input gradient) and P = bf16(dY V^T); for
 *   r_lora <= 64 it also makes per-workgroup partial sums of dB from the dY
 *   it holds, so dY is read once for the whole backward;
 *   kernel 2 computes deq(Qrow(dY)) deq(Qtile(W_res)) + P D^T, reading the
 *   forward's 32x32-tile codes and scales (w_codes, w_scales) transposed,
 *   and writes dX (bf16 [M, K]) once;
 *   kernel 3 writes the adapter gradients, rank-major like At and B:
 *   dA^T = P[:, r_stab:]^T X ([r_lora, K]) and dB = U[:, r_stab:]^T dY
 *   ([r_lora, N]), in grad_dtype (FT_BF16 or FT_F32); every partial sum is
 *   added in a fixed order, so the gradients are deterministic.  When
 *   kernel 2's tiles leave CUs free (from the start or for its last round)
 *   and dB's partials come from kernel 1, act_in is none and r_lora <= 64,
 *   kernel 2's launch has extra workgroups on those CUs that compute kernel
 *   3's results, with the same bits, and kernel 3 does not run.
 * X and U_save are the forward's input and saved U.  H: bf16 [M, N], this
 * layer's forward output Y; required when act_out != FT_ACT_NONE (then the
 * incoming gradient is dY * act_out'(H), recomputed wherever it is read),
 * else ignored.  With act_in != FT_ACT_NONE, X is the pre-activation h and
 * dA uses act_in(h), recomputed as X is read; dX is still the gradient of
 * the layer's input act_in(h) (the caller applies act_in'(h), e.g. with
 * fourtune_act_bwd).  dX may be NULL (no input gradient; then wt_codes and
 * wt_scales may be NULL for every w_block).  dA, dB may be NULL only when
 * r_lora == 0.
 * Under G16 (precision bit 1) kernel 1 computes P and the dB partials
 * only, the weight tiles are dequantized to bf16 in the workspace in
 * transposed order ([K, N]), and kernel 2 multiplies bf16 dY
 * (dY * act_out'(H) when set, made in the workspace first) by them.
 * P_save : optional bf16 [M, R] output of P; NULL = workspace only.
 * gq_codes, gq_scales: optional outputs [M, N/2], [M, N/32]; must be NULL
 *   under G16.
 * workspace: at least fourtune_workspace_bytes(L, 1) bytes.
 * No gradient is produced for W_res, L1 or L2 (frozen).
 * Requirements: as for the forward.
 * Errors: FT_EINVAL, FT_ESHAPE, FT_EALIGN, FT_EWORKSPACE, FT_EDEVICE. */
ft_status fourtune_linear_bwd(const ft_linear* L, const uint16_t* dY, const uint16_t* X,
                              const uint16_t* U_save, const uint16_t* H, uint16_t* dX, void* dA,
                              void* dB,
                              ft_dtype grad_dtype, uint16_t* P_save, uint8_t* gq_codes,
                              uint8_t* gq_scales, void* workspace, size_t ws_bytes,
                              void* stream);

/* The forward of an MLP block's two linears with the GeLU between them,
 * FC1's GEMM fused with FC2's quantization (FourTune, "3.3 Kernel Fusion for
 * Efficiency / MLP Fusion"):
 *   fc1: X [M, K1] -> H [M, N1], the pre-activation h, written for the
 *        backward (fc1->act_out is not read here);
 *   fc2: gelu(H) [M, N1] -> Y [M, N2]; fc2->act_in must be
 *        FT_ACT_GELU_TANH, fc2->M == fc1->M, fc2->K == fc1->N.
 * Kernels: fc1's kernel 1 (as fourtune_linear_fwd); fc1's GEMM, whose
 * epilogue also applies the GeLU to the rounded h it holds and writes FC2's
 * quantized input Qrow(gelu(h)) and the fp32 sums of FC2's down-projection
 * gelu(h) [L1|A] over each 256 columns of h; a kernel that adds those sums
 * in column order and rounds them to U2; FC2's GEMM.  So FC2's kernel 1,
 * a second full read of H, does not run.
 * Results: H, U1_save, U2_save, Y and the optional aq_codes [M, N1/2] and
 * aq_scales [M, N1/32] (FC2's quantized input) are those of
 * fourtune_linear_fwd(fc1, X) followed by fourtune_linear_fwd(fc2, H): the
 * same bits where FC2's kernel 1 would sum 256-column splits (when
 * ceil(M/64) * ceil(N1/256) is at least the device's CU count), else U2
 * (and so Y) up to the order of U2's fp32 sums.
 * The epilogue fusion applies when both layers are FT_W4A4G4, fc1's
 * w_block is TILE32 or TILE32_T, K1 % 128 == 0, M > 16, FC1's GEMM runs in
 * one pass over its reduction (it splits the reduction only for outputs
 * of at most 128 tiles of 256 x 256, by a cost model of the shapes), and
 * R2 = fc2 ranks <= 64; otherwise the two forwards run one after the
 * other (the same results).
 * workspace: at least fourtune_mlp_workspace_bytes(fc1, fc2) bytes.
 * Requirements and errors: those of fourtune_linear_fwd for each layer;
 * FT_ESHAPE if the layers do not chain; FT_EINVAL if fc2->act_in is not
 * FT_ACT_GELU_TANH. */
size_t fourtune_mlp_workspace_bytes(const ft_linear* fc1, const ft_linear* fc2);
ft_status fourtune_mlp_fwd(const ft_linear* fc1, const ft_linear* fc2, const uint16_t* X,
                           uint16_t* H, uint16_t* Y, uint16_t* U1_save, uint16_t* U2_save,
                           uint8_t* aq_codes, uint8_t* aq_scales, void* workspace,
                           size_t ws_bytes, void* stream);

/* The backward of the same MLP block, mirrored: FC2's input-gradient GEMM
 * (on FC2's tiles read transposed, section 3.2) holds dX2 = dL/d gelu(h) in
 * its registers; its epilogue reads the matching rows of H, forms FC1's
 * incoming gradient dY1 = bf16(dX2 * gelu'(H)) and writes it (dX2 itself is
 * not written), and from the same values writes FC1's quantized gradient
 * Qrow(dY1) and the fp32 sums of FC1's down-projection dY1 V1^T over each
 * 256 columns, so FC1's backward quantize kernel, a read of dX2 and H, does
 * not run.  Then: those sums added in order into P1 (and FC1's padded rank
 * operands), FC2's adapter gradients, FC1's input-gradient GEMM and FC1's
 * adapter gradients (dB1 = U1[:, r_stab:]^T dY1 from dY1).
 *   dY: bf16 [M, N2], the gradient of Y; X: FC1's input [M, K1]; H: FC1's
 *   output h [M, N1] from fourtune_mlp_fwd (or fourtune_linear_fwd);
 *   U1_save, U2_save: the forward's U of each layer.
 *   dX: bf16 [M, K1], FC1's input gradient; dA1, dB1, dA2, dB2: the adapter
 *   gradients, rank-major as in fourtune_linear_bwd, in grad_dtype.
 * Requirements: fc1->act_out and fc2->act_in FT_ACT_GELU_TANH, the layers
 * chain as for fourtune_mlp_fwd, and those of fourtune_linear_bwd for each
 * layer (dX required).  The mirror applies when both layers are FT_W4A4G4,
 * fc2's w_block is TILE32 (the method), N2 % 128 == 0, M > 16, FC2's
 * input-gradient GEMM runs in one pass, and R1 <= 64; otherwise the two
 * backwards run one after the other through dX2 (the same results up to
 * the order of dB1's fp32 sums, which the mirror forms from dY1 in
 * 512-token chunks).
 * workspace: at least fourtune_mlp_bwd_workspace_bytes(fc1, fc2) bytes.
 * Errors: those of fourtune_linear_bwd for each layer; FT_ESHAPE if the
 * layers do not chain; FT_EINVAL for the activations or a missing dX. */
size_t fourtune_mlp_bwd_workspace_bytes(const ft_linear* fc1, const ft_linear* fc2);
ft_status fourtune_mlp_bwd(const ft_linear* fc1, const ft_linear* fc2, const uint16_t* dY,
                           const uint16_t* X, const uint16_t* H, const uint16_t* U1_save,
                           const uint16_t* U2_save, uint16_t* dX, void* dA1, void* dB1, void* dA2,
                           void* dB2, ft_dtype grad_dtype, void* workspace, size_t ws_bytes,
                           void* stream);

/* The activation on its own, with the same device functions the fused
 * kernels apply to their inputs (so that a caller, or a test, can see the
 * exact bf16 values the layers consume).  n elements, contiguous.
 *   fourtune_act_fwd: out = bf16(act(h))
 *   fourtune_act_bwd: out = bf16(g * act'(h))   (the input gradient of act)
 * act must be FT_ACT_GELU_TANH.  Pointers 16-byte aligned; n >= 0.
 * Errors: FT_EINVAL, FT_ESHAPE, FT_EALIGN, FT_EDEVICE, FT_EUNSUPPORTED. */
ft_status fourtune_act_fwd(int act, const uint16_t* h, int64_t n, uint16_t* out, void* stream);
ft_status fourtune_act_bwd(int act, const uint16_t* h, const uint16_t* g, int64_t n,
                           uint16_t* out, void* stream);

/* Static, human-readable text for a status code. */
const char* fourtune_status_string(ft_status s);

/* Per-kernel timing for benchmarks (process-wide, off by default).  While
 * enabled, every kernel the entry points above enqueue is bracketed by two
 * hipEvents recorded on the call's stream; the events come from a pool the
 * library creates on first use and keeps.  fourtune_timing_read waits for the
 * recorded events, adds their elapsed times per kernel name and returns the
 * number of distinct kernels; it fills up to max_entries entries of names
 * (static strings owned by the library), total_ms and counts (any of the
 * three may be NULL).  fourtune_timing_reset clears the totals. */
void fourtune_timing_enable(int on);
void fourtune_timing_reset(void);
int fourtune_timing_read(const char** names, double* total_ms, int64_t* counts, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* FOURTUNE_H */
