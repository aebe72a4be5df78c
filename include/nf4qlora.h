/*
 * nf4qlora.h -- C ABI of the fused NF4 QLoRA linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer is the QLoRA linear layer of Unsloth-style fine-tuning: a frozen base weight W [n,k]
 * stored as 4-bit NormalFloat (NF4) codes with per-block absmax constants that may themselves be
 * quantised ("double quantisation"), and trainable bf16 LoRA adapters A [r,k], B [n,r] with
 * Delta W = B A at rank r [Unsloth v0.1.463-beta release article, "About the Unsloth Project";
 * v0.1.47-beta article, section on lowering the fine-tuning barrier]. NF4 dequantisation, the
 * matmul and the LoRA correction are computed together, without materialising a dequantised
 * copy of W ["Inside Unsloth" book listing, "What You'll Learn", "LoRA and QLoRA"; pyshine
 * Unsloth code tour, "Why You Need This"]:
 *
 *     T  = X A^T                 Y  = X deq(W)^T + s T B^T
 *     U  = dY B                  dX = dY deq(W) + s U A
 *     dA = s U^T X               dB = s dY^T T              (W is frozen: no dW)
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers, owned and allocated by the caller; the library never
 *     allocates or frees device memory. Matrices are dense row-major. bf16 is IEEE bfloat16
 *     stored as 16-bit words. Base pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls are asynchronous on it; the
 *     outputs are ready once the stream has reached the call.
 *   - Every argument is validated on the host before anything is launched, so a call that
 *     returns an error has launched nothing. A launch failure returns NF4_EHIP. Faults inside a
 *     kernel surface at the caller's next synchronisation. The library never aborts.
 *   - nf4_last_error() returns a thread-local message describing the last non-OK status.
 *   - Inputs must be finite; results for NaN or Inf inputs are not specified.
 *   - Results are deterministic: the same inputs give bitwise-identical outputs on every call.
 *
 * NF4 format (the pages name NF4 and double quantisation but fix no constants; these are the
 * QLoRA constructions):
 *   - levels: the 16 NF4 levels from standard-normal quantiles (7 negative, an exact 0,
 *     8 positive, ends -1 and +1), float32; nf4_codebook() returns them.
 *   - blocks of 64 consecutive elements of the row-major W (k % 64 == 0, so a block never
 *     straddles a row); block constant a = max |w| over the block (float32).
 *   - code = index of the level nearest to fl32(w / a), ties to the lower index; an all-zero
 *     block has a = 0 and every code 7 (the exact zero level).
 *   - packing: byte i of `codes` holds element 2i in bits 7..4 and element 2i+1 in bits 3..0.
 *   - dq_block == 0: absmax is float[n*k/64] holding a.
 *     dq_block == 256: absmax is int8_t[n*k/64] and absmax_scale is float[ceil(n*k/64/256)];
 *     run j of 256 consecutive block constants (flattened order; the last run may be short)
 *     has S_j = fl32(max a / 127) and q = rint(fl32(a / S_j)) in [0,127] (S_j == 0 gives q = 0);
 *     blocks decode with a' = fl32(q * S_j). Codes are always taken against the exact a.
 *   - dequantised element: w' = fl32(level[code] * a'); the GEMMs consume w' rounded to bf16
 *     (round-to-nearest-even) and accumulate in float32.
 *
 * E2M1 format (block == 16), the 4-bit floating-point variant of the same layer [NVFP4 update
 * article, "NVFP4: A Quantization Format for the Next Generation of Hardware": E2M1 elements with
 * 1 sign, 2 exponent and 1 mantissa bits up to +-6, groups of 16 or 32 sharing an FP8 scale]:
 *   - element values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives; code = sign << 3 | index.
 *   - groups of 16 consecutive elements (k % 64 == 0 as for NF4); `absmax` holds one FP8 E4M3 byte
 *     per group (bias 7, largest value 448), `absmax_scale` points to ONE float32 tensor scale.
 *   - S = fl32(max |w| / 2688); group scale s = E4M3(fl32(max_g |w| / fl32(6 S))), nearest, ties
 *     to even, saturating at 448 (S == 0: every s and code 0); code = E2M1(fl32(w / fl32(s S))),
 *     nearest, ties to the even mantissa, saturating at 6, sign bit set for negative values.
 *   - packing as NF4 (first element in the high nibble); dequantised w' = fl32(fl32(e2m1 * s) * S).
 *   - the GEMMs consume e2m1 * s, which is exact in bf16, and multiply the float32 sums by S.
 */
#ifndef NF4QLORA_H
#define NF4QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NF4_OK = 0,
  NF4_EINVAL = -1,       /* a pointer, size, alignment or workspace argument is invalid */
  NF4_EUNSUPPORTED = -2, /* a well-formed request outside what the library implements */
  NF4_EHIP = -3          /* the HIP runtime reported an error at launch */
} nf4_status;

typedef enum { NF4_BF16 = 0, NF4_F32 = 1 } nf4_dtype;

/* An NF4-quantised weight W [n,k]. The struct itself is a host object; its pointers are device
 * pointers owned by the caller. */
typedef struct {
  int64_t n, k;         /* logical shape of W; n >= 1, k >= 64, k % 64 == 0                  */
  int32_t block;        /* 64: NF4; 16: E2M1 (see above)                                     */
  int32_t dq_block;     /* NF4: 0 (float32 absmax) or 256 (int8 absmax + float32 run scale);
                           E2M1: 0                                                            */
  uint8_t *codes;       /* [n*k/2] packed codes                                              */
  void *absmax;         /* NF4: float[n*k/64] if dq_block == 0, else int8_t[n*k/64];
                           E2M1: uint8_t[n*k/16] E4M3 group scales                           */
  float *absmax_scale;  /* NF4: float[ceil(n*k/64/dq_block)] if dq_block > 0, else ignored;
                           E2M1: float[1], the tensor scale (written by nf4_quantize)        */
} nf4_tensor;

/* Quantise W (bf16 or float32, [q->n, q->k]) into the buffers of *q, as described above (NF4
 * for block 64, E2M1 for block 16) [the frozen base stored as 4-bit NormalFloat with double
 * quantisation of its constants: Unsloth v0.1.463-beta release article, "About the Unsloth
 * Project"; E2M1: NVFP4 update article, "NVFP4: A Quantization Format for the Next Generation
 * of Hardware"]. NF4: one kernel launch (the double quantisation of a run of 256 constants is
 * finished by the workgroup that computes them, so no staging workspace is needed); E2M1: four
 * (the tensor maximum, then the groups). No workspace. w_dtype is an nf4_dtype value.
 * Bit-exact: the codes, block constants and scales equal those of the
 * definition for every finite input.
 * Errors: NF4_EINVAL for a NULL pointer, a misaligned pointer or n < 1;
 *         NF4_EUNSUPPORTED for k % 64 != 0, block not in {64, 16}, dq_block not in {0, 256}
 *         (0 for E2M1), or n*k >= 2^40. */
int nf4_quantize(const void *w, int w_dtype, const nf4_tensor *q, void *stream);

/* Write deq(W) to out [n,k] as float32 (w', exact) or bf16 (w' rounded to nearest-even).
 * Diagnostic and ablation path; the fused calls never materialise it.
 * Errors: as nf4_quantize, plus NF4_EINVAL for an unknown out_dtype. */
int nf4_dequantize(const nf4_tensor *q, void *out, int out_dtype, void *stream);

/* Host-only: copy the 16 float32 NF4 levels (ascending) into levels[16] and, when thresholds is
 * not NULL, the 15 float32 decision thresholds into thresholds[15] (thresholds[i] is the largest
 * float32 not above the midpoint of levels i and i+1; code = number of thresholds below v).
 * No device access. Returns NF4_EINVAL when levels is NULL. */
int nf4_codebook(float *levels, float *thresholds);

/* Bytes of device workspace qlora_fwd needs for these sizes (0 when r == 0). */
size_t qlora_fwd_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r);

/* Forward of the QLoRA layer:  T = bf16(X A^T),  Y = bf16(X deq(W)^T + s T B^T)  [the
 * layer with the low-rank correction Delta W = B A: Unsloth v0.1.463-beta release article,
 * "About the Unsloth Project"; dequantisation, matmul and LoRA correction computed together:
 * "Inside Unsloth" listing, "What You'll Learn", "LoRA and QLoRA"; pyshine Unsloth code tour,
 * "Why You Need This"].
 *   X  bf16 [m, k]   input activations                     (k == W->k)
 *   W  NF4 [n, k]    frozen base weight
 *   A  bf16 [r, k]   LoRA down-projection; B bf16 [n, r] LoRA up-projection (NULL when r == 0)
 *   s  LoRA scaling (lora_alpha / r by the usual convention)
 *   Y  bf16 [m, n]   output
 *   T  bf16 [m, r]   output: X A^T, kept for qlora_bwd (NULL when r == 0)
 *   ws workspace of at least qlora_fwd_workspace_bytes(m, n, k, r) bytes (NULL when that is 0):
 *      the float32 split-K partial sums of T = X A^T, owned by the caller, free after the call
 * The LoRA term uses T as rounded to bf16 and s*B rounded to bf16 (exact when s is a power of
 * two). Requires m >= 1, n % 8 == 0, 0 <= r <= 128.
 * Decode shapes (m <= 16, k % 256 == 0) with r % 8 == 0 and r <= 64 for a double-quantised NF4
 * weight, r <= 16 for an E2M1 weight, run as ONE launch that forms T from the X slices it
 * streams, and leave ws untouched.
 * Each of its workgroups adds T over k in its own order (start points staggered across the
 * workgroups); the T written is that of the workgroup starting at k = 0, and the T another
 * workgroup uses for its columns of Y may differ from it in the last bf16 bit of an entry.
 * Errors: NF4_EINVAL for NULL/misaligned pointers, m < 1, r out of range, a short workspace;
 *         NF4_EUNSUPPORTED for n % 8 != 0 and the NF4 format limits of nf4_quantize. */
int qlora_fwd(const void *X, int64_t m, const nf4_tensor *W, const void *A, const void *B,
              int32_t r, float s, void *Y, void *T, void *ws, size_t ws_bytes, void *stream);

/* The two launches qlora_fwd is made of, for callers that already hold T or that time them:
 *
 * qlora_lora_down: T = bf16(X A^T), X bf16 [m, k], A bf16 [r, k], T bf16 [m, r], 1 <= r <= 128.
 * ws: at least qlora_fwd_workspace_bytes(m, n, k, r) bytes (float partial sums over k).
 * Errors: NF4_EINVAL for NULL/misaligned pointers, m < 1, r out of range, a short workspace;
 *         NF4_EUNSUPPORTED for k not a positive multiple of 64. */
int qlora_lora_down(const void *X, int64_t m, int64_t k, const void *A, int32_t r, void *T,
                    void *ws, size_t ws_bytes, void *stream);

/* qlora_fwd_fused: Y = bf16(X deq(W)^T + s T B^T) in ONE kernel launch: the NF4 weight is decoded
 * on the fly inside the GEMM and the rank-r term runs as extra reduction steps of the same output
 * tile. T bf16 [m, r] as produced by qlora_lora_down (NULL when r == 0). No workspace.
 * Errors: as qlora_fwd. */
int qlora_fwd_fused(const void *X, int64_t m, const nf4_tensor *W, const void *T, const void *B,
                    int32_t r, float s, void *Y, void *stream);

/* Bytes of device workspace qlora_bwd needs for these sizes. */
size_t qlora_bwd_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r);

/* Backward of the QLoRA layer [only the adapters train, the 4-bit base is frozen: Unsloth
 * v0.1.463-beta release article, "About the Unsloth Project"; the rewritten backward pass:
 * same article and pyshine Unsloth code tour, "Why You Need This"], given the upstream gradient
 * dY bf16 [m, n] and T from qlora_fwd
 * (T may be NULL: it is then recomputed as X A^T into the workspace, exactly as qlora_fwd and
 * qlora_lora_down compute it):
 *   U  = bf16(dY B)                               (left in the workspace: see below)
 *   dX = bf16(dY deq(W) + s U A)      bf16 [m, k]  (skipped when dX is NULL)
 *   dA = bf16(s U^T X)                bf16 [r, k]
 *   dB = bf16(s dY^T T)               bf16 [n, r]
 * Sums over m are taken in float32 in a fixed order (deterministic). With r == 0, A, B, T, dA
 * and dB are ignored and only dX is produced.
 * When r > 0 the call leaves U (bf16 [m, r], row-major) in the first m*r*2 bytes of ws, where
 * qlora_bwd_dx can take it: qlora_bwd with dX == NULL followed by qlora_bwd_dx is the same work
 * as one qlora_bwd call.
 * Non-finite inputs: when n % 64 != 0, dX row i may also multiply zeros by the first
 * 64 - n % 64 values of dY row i + 1 (the last 64-column step of the reduction reads whole
 * 128-byte lines); an Inf or NaN among those values turns dX row i into NaN. With finite dY the
 * result is as stated.
 * Errors: as qlora_fwd, plus NF4_EINVAL when ws is smaller than qlora_bwd_workspace_bytes. */
int qlora_bwd(const void *dY, const void *X, int64_t m, const nf4_tensor *W, const void *A,
              const void *B, int32_t r, float s, const void *T, void *dX, void *dA, void *dB,
              void *ws, size_t ws_bytes, void *stream);

/* The input-gradient launch of qlora_bwd on its own, for callers that hold U or that time it:
 * dX = bf16(dY deq(W) + s U A) in ONE kernel launch (the NF4 weight decoded on the fly, read
 * along n; the rank-r term as extra reduction steps). dY bf16 [m, n], U bf16 [m, r] (= dY B),
 * A bf16 [r, k], dX bf16 [m, k]; U and A may be NULL when r == 0. No workspace.
 * Errors: as qlora_fwd (dY, U, A checked where qlora_fwd checks X, A, B). */
int qlora_bwd_dx(const void *dY, int64_t m, const nf4_tensor *W, const void *U, const void *A,
                 int32_t r, float s, void *dX, void *stream);

/* ---- Gate/up pair with SwiGLU -------------------------------------------------------------
 * The gated MLP's gate and up projections, two QLoRA layers on the same input, joined by the
 * SwiGLU activation (the pages name a fused gated-MLP activation kernel beside the fused LoRA
 * matmul [pyshine Unsloth code tour, "Why You Need This"; "Inside Unsloth" listing, "What You'll
 * Learn", "Triton Kernel Internals"]; the activation is read as the Llama gated MLP):
 *   Yg = X deq(Wg)^T + s (X Ag^T) Bg^T,   Yu = X deq(Wu)^T + s (X Au^T) Bu^T,
 *   H  = silu(Yg) * Yu,                   silu(x) = x / (1 + exp(-x)).
 * Layout: Wgu is ONE NF4 tensor [2n, k] quantised from the stacked weight [Wg; Wu] (rows 0 .. n-1
 * gate, n .. 2n-1 up: the usual fused gate_up layout); Agu bf16 [2r, k] is [Ag; Au]; Bg and Bu
 * are bf16 [n, r] each. The pair runs as one stacked QLoRA layer with the block-diagonal up
 * projection [[Bg, 0], [0, Bu]] (applied by the pair's fused launch as it stages B; built in the
 * workspace for the decode shapes and the backward), so its GEMMs are qlora_fwd's and
 * qlora_bwd's kernels on [2n, k]. Requires n % 8 == 0 and 0 <= r <= 64 (2r <= 128).
 *
 * Bytes of device workspace qlora_swiglu_fwd and qlora_swiglu_bwd need (the same for both). */
size_t qlora_swiglu_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r);

/* Forward: H bf16 [m, n] = bf16(silu(Yg) * Yu), computed in float32, and Ygu bf16 [m, 2n] (each
 * row: Yg then Yu), kept for the backward; Tgu bf16
 * [m, 2r] = [X Ag^T | X Au^T] (may be NULL: the backward then recomputes it). Agu, Bg, Bu, Tgu
 * NULL when r == 0. ws: at least qlora_swiglu_workspace_bytes(m, n, k, r) bytes, 16-byte aligned.
 * Above the decode shapes (m > 48, or k % 256 != 0, or m > 16 with an E2M1 weight) the GEMM and
 * the activation are ONE launch of the fused kernel, H computed in its epilogue from the float32
 * sums of Yg and Yu (one rounding); the decode shapes run the stacked forward, then the
 * activation kernel (H from the bf16 Ygu by the same float32 expression).
 * Errors: as qlora_fwd; NF4_EINVAL also when Wgu->n is odd, r > 64 or H / Ygu is NULL. */
int qlora_swiglu_fwd(const void *X, int64_t m, const nf4_tensor *Wgu, const void *Agu,
                     const void *Bg, const void *Bu, int32_t r, float s, void *H, void *Ygu,
                     void *Tgu, void *ws, size_t ws_bytes, void *stream);

/* qlora_swiglu_fwd_fused: the pair's forward in ONE kernel launch given Tgu bf16 [m, 2r]
 * (= [X Ag^T | X Au^T], as qlora_swiglu_fwd returns it; NULL when r == 0): Yg and Yu with the
 * NF4 decode inside the GEMM and the rank-r terms as extra reduction steps of the same tile, and
 * H = silu(Yg) * Yu from their float32 sums in the epilogue [same passages as qlora_swiglu_fwd].
 * Any m >= 1 (this is the launch qlora_swiglu_fwd makes above the decode shapes, whose H and Ygu
 * it reproduces bit for bit for the same Tgu). No workspace.
 * Errors: as qlora_swiglu_fwd (no workspace checks). */
int qlora_swiglu_fwd_fused(const void *X, int64_t m, const nf4_tensor *Wgu, const void *Tgu,
                           const void *Bg, const void *Bu, int32_t r, float s, void *H, void *Ygu,
                           void *stream);

/* Backward for the upstream gradient dH bf16 [m, n], given Ygu and Tgu from the forward (Tgu may
 * be NULL: recomputed):
 *   dYg = dH * Yu * silu'(Yg),  dYu = dH * silu(Yg)      (float32, rounded to bf16)
 *   dX  bf16 [m, k]  = the sum of both projections' input gradients  (skipped when NULL)
 *   dAgu bf16 [2r, k] = [dAg; dAu],  dBg, dBu bf16 [n, r]
 * computed as qlora_bwd of the stacked layer with dY = [dYg | dYu]; sums in a fixed order
 * (deterministic). dAgu, dBg, dBu are ignored when r == 0.
 * Errors: as qlora_bwd; NF4_EINVAL also when dH or Ygu is NULL. */
int qlora_swiglu_bwd(const void *dH, const void *X, int64_t m, const nf4_tensor *Wgu,
                     const void *Agu, const void *Bg, const void *Bu, int32_t r, float s,
                     const void *Ygu, const void *Tgu, void *dX, void *dAgu, void *dBg, void *dBu,
                     void *ws, size_t ws_bytes, void *stream);

/* ---- LoRA merge ----------------------------------------------------------------------------
 * The adapters folded into the base for a merged save [pyshine Unsloth code tour, the save.py
 * walkthrough; NVFP4 update article, "A More Flexible Quantization Export Pipeline"]:
 *   Wout bf16 [n, k] = bf16(deq(W) + s B A)       W NF4 [n, k], A bf16 [r, k], B bf16 [n, r]
 * so that X Wout^T is the layer's X deq(W)^T + s (X A^T) B^T up to the rounding of Wout. One
 * launch: the rank-r product on the matrix cores, deq(W) = fl32(level * a') added in float32,
 * rounded once to bf16. With r == 0 (A, B NULL) Wout equals nf4_dequantize's bf16 output bit for
 * bit. Re-quantising for export is nf4_quantize of Wout (a new NF4 tensor [n, k]).
 * An E2M1 weight (block 16) merges the same way with w' its E2M1 dequantisation; re-quantising
 * Wout with block 16 gives a compressed FP4 export of the merged layer.
 * Errors: NF4_EINVAL for NULL/misaligned pointers or r outside [0, 128]; NF4_EUNSUPPORTED for the
 * format limits of nf4_quantize or n*k >= 2^32. */
int qlora_merge(const nf4_tensor *W, const void *A, const void *B, int32_t r, float s, void *Wout,
                void *stream);

/* ---- Grouped (mixture-of-experts) layer -------------------------------------------------------
 * E experts (1 <= E <= 256), each a QLoRA layer with its own frozen NF4 base and adapters
 * [NVFP4 update article, "Comprehensive Improvements in Training Performance and Stability":
 * grouped MoE, LoRA on the experts' MLP layers; pyshine Unsloth code tour, "Why You Need This":
 * the grouped-GEMM interface for MoE experts]. The routing is given: the rows of X (and of Y, T,
 * dY, dX) are grouped by expert in expert order, counts[e] >= 0 of them for expert e (a HOST
 * array of E values), and
 *   Y[rows of e] = X[rows of e] deq(W_e)^T + s (X[rows of e] A_e^T) B_e^T.
 * The experts' tensors are stacked in expert order: W ONE NF4 tensor [E n, k] (quantised from the
 * stacked bf16 weights), A bf16 [E r, k], B bf16 [E n, r]; T bf16 [sum(counts), r].
 *
 * Bytes of device workspace qlora_moe_fwd and qlora_moe_bwd need for these counts. */
size_t qlora_moe_workspace_bytes(const int64_t *counts, int32_t E, int64_t n, int64_t k, int32_t r);

/* Forward: T = X_e A_e^T for every expert's rows (ONE grouped row-projection launch) and Y
 * [sum(counts), n] in ONE launch of the fused kernel for all experts (each workgroup finds its
 * expert's rows and weight). T must be non-NULL when r > 0. Errors: as qlora_fwd; NF4_EINVAL
 * also for E out of range, a negative count, W->n not a multiple of E. */
int qlora_moe_fwd(const void *X, const int64_t *counts, int32_t E, const nf4_tensor *W,
                  const void *A, const void *B, int32_t r, float s, void *Y, void *T, void *ws,
                  size_t ws_bytes, void *stream);

/* The grouped fused launch alone, given T [sum(counts), r] (NULL when r == 0): what qlora_moe_fwd
 * runs after its row projections. No workspace. Errors: as qlora_moe_fwd. */
int qlora_moe_fwd_fused(const void *X, const int64_t *counts, int32_t E, const nf4_tensor *W,
                        const void *T, const void *B, int32_t r, float s, void *Y, void *stream);

/* Backward for dY [sum(counts), n]: dX [sum(counts), k] (skipped when NULL), dA [E r, k] and
 * dB [E n, r], each expert's adapter gradients summed over its own rows (zero for an expert with
 * no rows); T from the forward or NULL (recomputed). dX of every expert comes from ONE launch of
 * the fused dX kernel (when its tiles fill at least one round of the GPU's CUs and leave a partly
 * filled last round, the tiles of that round are split along the reduction into float32 pieces
 * kept in ws, and a second small launch adds them in a fixed order: results are deterministic
 * and the same for host and device routing); U = dY_e B_e is one grouped row projection, dA and
 * dB one grouped M-reduction each (every expert summing over its own rows only).
 * Errors: as qlora_bwd and qlora_moe_fwd. */
int qlora_moe_bwd(const void *dY, const void *X, const int64_t *counts, int32_t E,
                  const nf4_tensor *W, const void *A, const void *B, int32_t r, float s,
                  const void *T, void *dX, void *dA, void *dB, void *ws, size_t ws_bytes,
                  void *stream);

/* ---- No-allocation forward -------------------------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. qlora_fwd_noalloc is qlora_fwd (same arguments, same
 * kernels, same results bit for bit) without the workspace argument: its scratch (the float32
 * split-K partial sums of T = X A^T) is a static device array of NF4_NOALLOC_SCRATCH_BYTES on
 * each GPU, which that GPU holds until the process ends. The call allocates nothing; its first
 * call on a device looks the array's device address up (hipGetSymbolAddress) with that device
 * current. The stream must belong to the current device.
 * Every call on one GPU shares that GPU's array, which keeps the last call's partial sums (none
 * needs it cleared): calls that overlap on one GPU (on different streams or host threads) race
 * on it and give undefined results; serialise them.
 * Errors: as qlora_fwd; NF4_EUNSUPPORTED when the sizes need more scratch than the array holds
 * (qlora_fwd_workspace_bytes(m, n, k, r) > NF4_NOALLOC_SCRATCH_BYTES), checked before any HIP
 * call. */
#define NF4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int qlora_fwd_noalloc(const void *X, int64_t m, const nf4_tensor *W, const void *A, const void *B,
                      int32_t r, float s, void *Y, void *T, void *stream);

/* ---- Grouped layer with the routing in device memory ------------------------------------------
 * The same layer when the router runs on the GPU: counts is a DEVICE pointer to E int64 values
 * (8-byte aligned) and m, the number of routed rows (the rows of X, Y, T, dY, dX), is given on the
 * host, so nothing waits for the device and the calls can be captured in a HIP graph whose
 * replays route differently [NVFP4 update article, "Comprehensive Improvements in Training
 * Performance and Stability": grouped MoE training]. Each call first builds the group tables
 * (row offsets and first tiles) from the counts into its workspace with one small kernel; the
 * grouped launches are then sized by bounds from m and E, and workgroups past the last tile exit
 * at once. Results equal those of qlora_moe_fwd / qlora_moe_bwd for the same counts bit for bit
 * (the same split counts, which depend on m only). The counts should sum to m; the experts' row
 * ranges are clipped at m (no row past m is read or written), negative counts count as 0, and
 * rows past the counts' sum are left unwritten.
 *
 * Bytes of device workspace qlora_moe_fwd_dev and qlora_moe_bwd_dev need (any counts summing to
 * at most m). */
size_t qlora_moe_workspace_bytes_dev(int64_t m, int32_t E, int64_t n, int64_t k, int32_t r);

/* Forward (T and Y), as qlora_moe_fwd. Errors: as qlora_moe_fwd (checked on the host; the
 * device counts are not read there), NF4_EINVAL also for a NULL or misaligned counts pointer. */
int qlora_moe_fwd_dev(const void *X, int64_t m, const int64_t *counts, int32_t E, const nf4_tensor *W,
                      const void *A, const void *B, int32_t r, float s, void *Y, void *T, void *ws,
                      size_t ws_bytes, void *stream);

/* Backward (dX, dA, dB), as qlora_moe_bwd. Errors: as qlora_moe_fwd_dev. */
int qlora_moe_bwd_dev(const void *dY, const void *X, int64_t m, const int64_t *counts, int32_t E,
                      const nf4_tensor *W, const void *A, const void *B, int32_t r, float s,
                      const void *T, void *dX, void *dA, void *dB, void *ws, size_t ws_bytes,
                      void *stream);

/* Thread-local description of the last non-OK status returned on this thread ("" if none). */
const char *nf4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NF4QLORA_H */
