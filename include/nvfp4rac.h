/*
 * nvfp4rac.h - NVFP4 W4A4 MoE expert GEMM with Residual Activation
 * Compensation, for AMD Instinct MI355X (CDNA4, gfx950).
 *
 * The method is QUADS (arXiv 2607.15810).  Its rollout side quantizes
 * activations online to FP4 every forward, runs the W4A4 GEMM against
 * weights that came through the same quantize-dequantize (QDQ) path the
 * trainer fake-quantizes with, and adds back the quantization residual of
 * the few activation channels where it is largest (arXiv abstract; the
 * gist.science technical summary, sections 2.1 and 2.2, in Italian and
 * Korean).  This library is that hot path, one call per step.
 *
 * Formats (the public NVFP4 definition; the pages only name the E2M1 grid
 * and "fine-grained scaling"):
 *   - element: E2M1 code, 4 bits = sign | 3-bit magnitude index into
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Two codes per byte, element 2j in bits
 *     3:0 and element 2j+1 in bits 7:4.  Row-major [rows][K/2].
 *   - block scale: one OCP FP8 E4M3 byte per 16 consecutive elements along
 *     K, row-major [rows][K/16].
 *   - tensor scale: one float32 g per tensor (per expert for weights).
 *   - value = e2m1(code) * e4m3(scale) * g.
 *
 * Conventions for every call:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or synchronises; it keeps no pointer
 *     after returning.  Device pointers must be 16-byte aligned unless noted.
 *   - bf16 tensors are passed as void* holding IEEE bfloat16 bit patterns.
 *   - `stream` is a hipStream_t (NULL: the legacy default stream).  All work
 *     is enqueued on it in order.
 *   - `ws` is caller-owned device scratch of at least the size returned by
 *     the matching *_workspace_size query; its contents need not be
 *     initialised and are clobbered.  Calls that share a ws must not
 *     overlap in time.
 *   - Return: NVFP4_OK, or an error status for bad arguments (nothing is
 *     enqueued) or for a failed launch.  nvfp4_last_error() then holds a
 *     message (per thread).  Device faults surface at the caller's next
 *     synchronisation, as usual in HIP.
 *   - Value contract: finite inputs whose tensor absolute maximum is 0 or lies
 *     in [2^-100, 2^100].  NaN/Inf inputs give unspecified outputs.
 */
#ifndef NVFP4RAC_H
#define NVFP4RAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL                     */
  NVFP4_ERR_SHAPE = 2,       /* a size is out of range (K % 16, k > K, ...)    */
  NVFP4_ERR_ALIGN = 3,       /* a device pointer or stride is misaligned       */
  NVFP4_ERR_WORKSPACE = 4,   /* ws_bytes smaller than the workspace query      */
  NVFP4_ERR_UNSUPPORTED = 5, /* valid, but outside what the kernels implement  */
  NVFP4_ERR_HIP = 6          /* a HIP runtime or launch call failed            */
} nvfp4_status;

/* Library version, major*10000 + minor*100 + patch. */
int nvfp4_version(void);
/* Static name of a status code. */
const char* nvfp4_status_str(int status);
/* Detail message of the last failing call on this thread ("" if none). */
const char* nvfp4_last_error(void);

/* ------------------------------------------------------------------------
 * Weight QDQ (shared quantize-dequantize path).
 * Weights are synchronised from trainer to rollout through one QDQ path, so
 * the rollout's FP4 weights and the trainer's fake-quantized weights are the
 * same numbers (arXiv abstract; gist.science summary §2.1 "weights" and
 * §2.2 A, asymmetric W4A16 QAT).
 *
 * w      [E][N][K] bf16, K contiguous (each expert's weight, out x in).
 * codes  [E][N][K/2] packed E2M1, row-major: byte j of row n holds columns
 *        2j (bits 3:0) and 2j+1 (bits 7:4).
 * scales [E][N][K/16] E4M3, row-major: the scale of columns 16b .. 16b+15.
 * g_w    [E] float32: per-expert tensor scale g = fp32(amax_e / 2688).
 * w_qdq  [E][N][K] bf16 or NULL: bf16(fp32(e2m1 * e4m3) * g), the weight the
 *        trainer's forward sees.
 * packed_codes, packed_scales (both or neither; NULL: not written): the same
 *        codes and scales in the grouped GEMMs' packed layout (E*N*K and
 *        E*N*K/8 bytes), the w_codes and w_scales the GEMM calls take.  An
 *        opaque pre-pack, two copies of the row-major bytes per expert: a
 *        permutation that lets a GEMM k-step of a row block read whole cache
 *        lines, then a channel-major copy from which the residual correction
 *        gathers the weight columns of its selected channels
 *        (nvfp4_pack_weights makes it from row-major codes and scales).
 * Scale recipe per 16-block (all float32, round to nearest even):
 *   s = e4m3((blockmax * 448) / amax);  code = e2m1(x * (2688 / (s * amax)))
 *   (s == 0 gives magnitude 0); the sign bit of a code is the sign of x.
 * Requires 1 <= E <= 65535, N % 16 == 0, K % 64 == 0; codes 8-byte, scales
 * and packed_scales 4-byte, packed_codes 16-byte aligned.
 * ---------------------------------------------------------------------- */
size_t nvfp4_qdq_weights_workspace_size(int64_t E);
int nvfp4_qdq_weights(const void* w, int64_t E, int64_t N, int64_t K,
                      uint8_t* codes, uint8_t* scales, float* g_w, void* w_qdq,
                      uint8_t* packed_codes, uint8_t* packed_scales,
                      void* ws, size_t ws_bytes, void* stream);

/* The grouped GEMMs' packed copy of row-major NVFP4 weights (codes
 * [E][N][K/2], scales [E][N][K/16], as nvfp4_qdq_weights writes them), for
 * weights quantized elsewhere: packed_codes (E*N*K bytes) and packed_scales
 * (E*N*K/8 bytes) as described under nvfp4_qdq_weights.  Byte moves, no
 * arithmetic.  Requires 1 <= E <= 65535, N % 16 == 0, K % 64 == 0; codes
 * and packed_codes 16-byte, scales and packed_scales 4-byte aligned.  No
 * workspace. */
int nvfp4_pack_weights(const uint8_t* codes, const uint8_t* scales, int64_t E, int64_t N,
                       int64_t K, uint8_t* packed_codes, uint8_t* packed_scales, void* stream);

/* E2M1 encoding of float32 values with unit scale, the element conversion
 * every quantizer here applies to x * (2688 / (s * amax)) (the E2M1 grid of
 * gist.science summary §1): codes[i] (one code per byte, bits 3:0) = sign of
 * v[i] | index of the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6} to |v[i]|, ties
 * to the even index, saturating at 6.  v [n] float32 (finite), codes [n]
 * bytes; v 4-byte aligned, codes unaligned.  No workspace. */
int nvfp4_e2m1_encode_f32(const float* v, int64_t n, uint8_t* codes, void* stream);

/* ------------------------------------------------------------------------
 * Online activation quantization (activations are recomputed and quantized
 * every forward: arXiv abstract; gist.science summary §2.1), with the
 * per-channel residual statistic that Residual Activation Compensation ranks
 * channels by (summary §2.2 B).
 *
 * x      glu == 0: [M][K] bf16, row stride ldx elements (ldx >= K).
 *        glu == 1: [M][2K] bf16 = [gate | up], row stride ldx (>= 2K); the
 *        tensor quantized is h = bf16(silu(gate) * up), evaluated in float32.
 * codes  [M][K/2], scales [M][K/16], g_x [1] float32 (dynamic, per call).
 * score  [K] uint64 or NULL: score_j = sum over rows of
 *        floor(|r_ij| * 2^(31 - E_A)), r = bf16(fp32(x - dequant(x))), E_A the
 *        binary exponent of the tensor amax A (A = m 2^E_A, m in [0.5, 1)).
 *        An exact integer sum: bitwise reproducible in any order.
 * x_used [M][K] bf16 or NULL: the tensor that was quantized (required for
 *        glu == 1, where it receives h; for glu == 0 it is not written).
 * Requires M >= 0, K >= 32, K % 32 == 0, ldx % 8 == 0.  M == 0 writes
 * g_x = 0 and zero scores.
 * ---------------------------------------------------------------------- */
size_t nvfp4_quantize_act_workspace_size(int64_t M, int64_t K);
int nvfp4_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, int glu,
                       uint8_t* codes, uint8_t* scales, float* g_x,
                       uint64_t* score, void* x_used,
                       void* ws, size_t ws_bytes, void* stream);

/* nvfp4_quantize_act without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, outputs and requirements as
 * nvfp4_quantize_act minus ws/ws_bytes.  Scratch is a fixed 4 MiB array in
 * device memory, one copy per device, held until the process ends; its
 * address is looked up on the first call on each device.  The call allocates
 * and frees nothing.  K above 65536 returns NVFP4_ERR_UNSUPPORTED; any M is
 * taken (fewer row groups share the work when the scratch would overflow).
 * Calls on one device share the array: calls that overlap in time there
 * (other streams, other threads) race; calls in stream order do not. */
int nvfp4_quantize_act_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx, int glu,
                               uint8_t* codes, uint8_t* scales, float* g_x,
                               uint64_t* score, void* x_used, void* stream);

/* ------------------------------------------------------------------------
 * High-residual channel selection (the binary channel mask of Residual
 * Activation Compensation, gist.science summary §2.2 B, both languages).
 *
 * Picks the k channels with the largest score (ties: lower index), returns
 * them ascending in S [k] int32, and gathers the residual of those channels,
 * R_S [M][k] bf16 = bf16(fp32(x - dequant(x))), from x_used (row stride ldx),
 * codes, scales and g_x as produced by nvfp4_quantize_act.
 * k == 0 enqueues nothing.  Requires 0 <= k <= K <= 16384, K % 32 == 0.
 * ---------------------------------------------------------------------- */
size_t select_residual_channels_workspace_size(int64_t M, int64_t K, int64_t k);
int select_residual_channels(const void* x_used, int64_t ldx, const uint8_t* codes,
                             const uint8_t* scales, const float* g_x,
                             const uint64_t* score, int64_t M, int64_t K, int64_t k,
                             int32_t* S, void* R_S, void* ws, size_t ws_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * Gate+up GEMM with SwiGLU fused into its output: grouped_w4a4_gemm_rac on
 * weights whose N = 2 I rows are [gate | up], writing h [M_total][I] bf16,
 *   h[p][i] = bf16(silu(y[p][i]) * y[p][I + i]),  silu(g) = g / (1 + e^-g),
 * from the bf16-rounded products y (the same bits as the plain call followed
 * by the SwiGLU of nvfp4_quantize_act with glu = 1; float32 arithmetic).  On
 * large problems the SwiGLU runs in the GEMM's epilogue, whose column tiles
 * pair gate and up columns, so the [M_total][2 I] product is never written.
 * Same arguments as grouped_w4a4_gemm_rac with y -> h; requires N % 32 == 0.
 * h_amax [1] uint32 (device, nullable) receives max |h| as bf16 bits, the
 * tensor amax nvfp4_quantize_act_amax takes, so h is not read again for it.
 * Workspace: grouped_w4a4_gemm_rac_swiglu_workspace_size (the plain GEMM's
 * plus M_total * N * 2 bytes).
 * ---------------------------------------------------------------------- */
size_t grouped_w4a4_gemm_rac_swiglu_workspace_size(int64_t E, int64_t M_src, int64_t M_total,
                                                   int64_t N, int64_t K, int64_t k);
int grouped_w4a4_gemm_rac_swiglu(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const float* g_x, const int32_t* a_rows, int64_t M_src,
                                 const void* R_S, const int32_t* S, int64_t k,
                                 const uint8_t* w_codes, const uint8_t* w_scales,
                                 const float* g_w, const int32_t* expert_offsets, int64_t E,
                                 int64_t M_total, int64_t N, int64_t K, void* h,
                                 uint32_t* h_amax, void* ws, size_t ws_bytes, void* stream);

/* nvfp4_quantize_act (glu == 0) with the tensor amax given: amax [1] uint32
 * (device) holds max |x| as bf16 bits, e.g. from grouped_w4a4_gemm_rac_swiglu,
 * and x is read once.  The outputs are those nvfp4_quantize_act gives when the
 * amax is right; the call does not check it.  Same workspace query. */
int nvfp4_quantize_act_amax(const void* x, int64_t M, int64_t K, int64_t ldx,
                            const uint32_t* amax, uint8_t* codes, uint8_t* scales, float* g_x,
                            uint64_t* score, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Per-expert compensation: the variant of Residual Activation Compensation
 * in which each expert ranks the channels by the residual of its own rows
 * (the binary channel mask of gist.science summary §2.2 B, one per expert).
 *
 * select_residual_channels_per_expert: for expert e with permuted rows p in
 * [off[e], off[e+1]) taking activation rows t = a_rows ? a_rows[p] : p,
 *   score_e[j] = sum over those rows of floor(|r[t][j]| * 2^(31 - E_A))
 * (the nvfp4_quantize_act statistic restricted to the expert's rows; E_A the
 * binary exponent of the tensor amax, recovered exactly from g_x), S [E][k]
 * int32 = the k channels of largest score_e (ties: lower index), ascending,
 * and R [M_total][k] bf16, R[p][j] = bf16(fp32(x - dequant(x))) of row t on
 * channel S[e][j].  An expert with no rows gets channels 0 .. k-1.
 * x_used (row stride ldx), codes, scales, g_x as from nvfp4_quantize_act.
 * Requires 1 <= E <= 1024, 0 <= k <= K <= 16384, K % 32 == 0, ldx % 8 == 0;
 * k == 0 enqueues nothing.  ws: the per-expert scores, E * K * 8 bytes.
 *
 * grouped_w4a4_gemm_rac_per_expert: grouped_w4a4_gemm_rac with S_E [E][k]
 * (expert e corrects its rows on S_E[e]) and R_P [M_total][k] indexed by
 * permuted row p, as select_residual_channels_per_expert writes them:
 *   y[p][n] = bf16( g_w[e] * ( g_x * sum_k x~[t][k] w~e[n][k]
 *                              + sum_{j<k} R_P[p][j] w~e[n][S_E[e][j]] ) )
 * Same arguments, requirements and workspace query as grouped_w4a4_gemm_rac.
 * ---------------------------------------------------------------------- */
size_t select_residual_channels_per_expert_workspace_size(int64_t E, int64_t K);
int select_residual_channels_per_expert(const void* x_used, int64_t ldx, const uint8_t* codes,
                                        const uint8_t* scales, const float* g_x,
                                        const int32_t* a_rows, const int32_t* expert_offsets,
                                        int64_t E, int64_t M_src, int64_t M_total, int64_t K,
                                        int64_t k, int32_t* S, void* R, void* ws,
                                        size_t ws_bytes, void* stream);
int grouped_w4a4_gemm_rac_per_expert(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const float* g_x, const int32_t* a_rows, int64_t M_src,
                                     const void* R_P, const int32_t* S_E, int64_t k,
                                     const uint8_t* w_codes, const uint8_t* w_scales,
                                     const float* g_w, const int32_t* expert_offsets, int64_t E,
                                     int64_t M_total, int64_t N, int64_t K, void* y, void* ws,
                                     size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Trainer-side W4A16 product: the forward of asymmetric W4A16 QAT, bf16
 * activations against weights that went through the shared QDQ path
 * (gist.science summary §2.2 A; arXiv abstract).  Same expert grouping,
 * gather, weight layout and workspace rules as grouped_w4a4_gemm_rac; the
 * activation is not quantized and there is no correction.
 *
 * x      [M_src][K] bf16, contiguous.
 * y[p][n] (bf16, [M_total][N]) = bf16(sum_k x[t][k] * e2m1 * e4m3 * g_w[e])
 *        for row p of expert e, t = a_rows ? a_rows[p] : p: exact products
 *        (q * s decoded exactly to bf16), float32 accumulation, g_w applied
 *        in float32, one rounding to bf16.
 * Requires 1 <= E <= 1024, N % 16 == 0, K % 128 == 0, K <= 16384,
 * M_src * K * 2 < 2^32; a_rows == NULL needs M_src >= M_total.
 * ---------------------------------------------------------------------- */
size_t grouped_w4a16_gemm_workspace_size(int64_t E);
int grouped_w4a16_gemm(const void* x, const int32_t* a_rows, int64_t M_src,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* g_w,
                       const int32_t* expert_offsets, int64_t E, int64_t M_total,
                       int64_t N, int64_t K, void* y, void* ws, size_t ws_bytes,
                       void* stream);

/* ------------------------------------------------------------------------
 * Second-pass quantization of the compensated residual: the variant of
 * Residual Activation Compensation in which the selected residual is itself
 * quantized to NVFP4 before it is added back (gist.science summary §2.2 B,
 * "second-pass quantization").  The residual goes through the same QDQ path
 * as the weights.
 *
 * r      [M][k] bf16, contiguous: R_S from select_residual_channels.
 * codes  [M][k/2] packed E2M1; scales [M][k/16] E4M3, row-major (blocks of
 *        16 along the selected channels, in the ascending order of S).
 * g_r    [1] float32 = fp32(amax(r) / 2688), amax over the whole [M][k].
 * r_qdq  [M][k] bf16 = bf16(fp32(e2m1 * e4m3) * g_r): pass it as R_S to
 *        grouped_w4a4_gemm_rac to add the quantized residual back.
 * Same scale recipe as nvfp4_qdq_weights.  Requires M >= 0, k >= 16,
 * k % 16 == 0.  M == 0 writes g_r = 0 only.
 * ---------------------------------------------------------------------- */
size_t nvfp4_qdq_residual_workspace_size(int64_t M, int64_t k);
int nvfp4_qdq_residual(const void* r, int64_t M, int64_t k, uint8_t* codes,
                       uint8_t* scales, float* g_r, void* r_qdq,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * MoE routing and expert-major permutation (the MoE model of the pages,
 * gist.science summary §4; the router itself is not described there).
 *
 * logits [T][E] float32, bias [E] float32 or NULL.  Per token: the tk experts
 * of largest l = fp32(logit + bias) (ties: lower expert index), weights =
 * softmax over those tk values (float64, rounded to float32).
 * topk_ids [T][tk] int32, topk_w [T][tk] float32,
 * expert_offsets [E+1] int32 (rows of expert e are [off[e], off[e+1])),
 * perm_token [T*tk] int32 (token of each permuted row; tokens ascending within
 * an expert), inv_perm [T][tk] int32 (row of each (token, slot)).
 * Requires T >= 0, 1 <= tk <= E <= 1024, tk <= 32, T*tk < 2^31.
 * ---------------------------------------------------------------------- */
size_t moe_permute_workspace_size(int64_t T, int64_t E);
int moe_permute(const float* logits, const float* bias, int64_t T, int64_t E, int64_t tk,
                int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                int32_t* perm_token, int32_t* inv_perm,
                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Expert-grouped W4A4 GEMM with Residual Activation Compensation: the native
 * FP4 product over all of K plus the residual of the selected channels
 * multiplied by the same FP4 weights (gist.science summary §2.2 B; arXiv
 * abstract).  For permuted row p of expert e (off[e] <= p < off[e+1]) and
 * activation row t = a_rows ? a_rows[p] : p:
 *
 *   y[p][n] = bf16( g_w[e] * ( g_x * sum_k x~[t][k] w~e[n][k]
 *                              + sum_{j<k} R_S[t][j] w~e[n][S[j]] ) )
 *
 * with x~ = e2m1 * e4m3 of the activation, w~ likewise of the weight (exact
 * in the bf16/fp16 operands of the matrix cores), float32 accumulation.
 * a_codes [M_src][K/2], a_scales [M_src][K/16], g_x [1]; a_rows [M_total] or
 * NULL (then M_src >= M_total); R_S [M_src][k] bf16 (NULL iff k == 0);
 * S [k] int32 ascending; w_codes, w_scales: the packed copy of the weight
 * codes and scales (nvfp4_qdq_weights' packed outputs, or nvfp4_pack_weights), g_w [E];
 * expert_offsets [E+1] (device; off[0] = 0, off[E] = M_total); y [M_total][N]
 * bf16.  Requires K % 128 == 0, N % 16 == 0, 0 <= k <= K.
 * The workspace holds the per-expert tile prefix, an exact f16 image of the
 * activation (2 bytes per element) and, for a
 * problem too small to fill the chip, float32 partial products of up to 4
 * slices of K (slices * M_total * N * 4 bytes), summed in slice order, so
 * results do not depend on timing.  A workspace smaller than the query
 * returns NVFP4_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t grouped_w4a4_gemm_rac_workspace_size(int64_t E, int64_t M_src, int64_t M_total,
                                            int64_t N, int64_t K, int64_t k);
int grouped_w4a4_gemm_rac(const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                          const int32_t* a_rows, int64_t M_src,
                          const void* R_S, const int32_t* S, int64_t k,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* g_w,
                          const int32_t* expert_offsets, int64_t E, int64_t M_total,
                          int64_t N, int64_t K, void* y,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Un-permute and combine: out[t][n] = bf16( sum_j topk_w[t][j] *
 * y[inv_perm[t][j]][n] ), float32 accumulation in slot order j = 0..tk-1.
 * y [T*tk][N] bf16, out [T][N] bf16.  Requires N % 8 == 0.  No workspace.
 * ---------------------------------------------------------------------- */
int moe_unpermute_combine(const void* y, const int32_t* inv_perm, const float* topk_w,
                          int64_t T, int64_t tk, int64_t N, void* out, void* stream);

/* ------------------------------------------------------------------------
 * FP8 (E4M3) W8A8 baseline: the low-precision rollout format the pages
 * compare NVFP4 against (arXiv abstract; gist.science summary §1 and §4,
 * throughput).  The pages give no FP8 recipe; this is OCP E4M3 for both
 * operands with one float32 scale per tensor (per expert for weights).
 *
 * fp8_quantize: x bf16 [E][M][K] contiguous, E tensors of [M][K] each with
 * its own scale (E = 1 for an activation, E experts for weights).  Per
 * tensor, A = max |x|, g[e] = float32(A / 448), and codes [E][M][K] (u8)
 * hold sign(x) << 7 | E4M3(float32(|x| / g[e])) (round to nearest, ties to
 * the even code, saturating at 448; magnitude 0 for every element when
 * A = 0, then g[e] = 0).  Requires 1 <= E <= 65535, M >= 0, K % 8 == 0;
 * x 16-byte and codes 8-byte aligned.  Workspace: E 32-bit amax slots.
 *
 * grouped_fp8_gemm: a [M_src][K] E4M3 codes with scale *g_x (device),
 * w [E][N][K] E4M3 codes with scales g_w [E], expert_offsets [E+1]
 * (device), a_rows [M_total] or NULL (identity).  For output row p of
 * expert e, t = a_rows ? a_rows[p] : p:
 *   y[p][n] = bf16( g_x * g_w[e] * sum_k a[t][k] * w[e][n][k] )
 * (exact products, float32 accumulation, one rounding to bf16).  Requires
 * 1 <= E <= 1024, N % 16 == 0, K % 128 == 0, M_src * K < 2^32,
 * N * K < 2^32; a, w and y 16-byte aligned.  Workspace: the per-expert
 * tile prefix.
 * ---------------------------------------------------------------------- */
size_t fp8_quantize_workspace_size(int64_t E);
int fp8_quantize(const void* x, int64_t E, int64_t M, int64_t K, uint8_t* codes, float* g,
                 void* ws, size_t ws_bytes, void* stream);
size_t grouped_fp8_gemm_workspace_size(int64_t E);
int grouped_fp8_gemm(const uint8_t* a, const float* g_x, const int32_t* a_rows, int64_t M_src,
                     const uint8_t* w, const float* g_w, const int32_t* expert_offsets, int64_t E,
                     int64_t M_total, int64_t N, int64_t K, void* y, void* ws, size_t ws_bytes,
                     void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4RAC_H */
