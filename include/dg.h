/*
 * dg.h -- C ABI of libdg, an FP8 (E4M3 / E5M2) block-scaled NT GEMM for AMD Instinct
 * MI355X (gfx950) with BF16 output, in a dense form and two MoE grouped forms.
 *
 * What every call computes (for each written output element):
 *
 *   C[m,n] = bf16( sum_kb  sA[m,kb] * sB_g[n/128, kb] *
 *                  sum_{k = 128kb}^{128kb+127}  A[m,k] * B_g[n,k] )
 *
 * The operation and its conventions come from the DeepGEMM pages:
 *   - FP8 inputs, BF16 output; the call names gemm_fp8_fp8_bf16_nt,
 *     m_grouped_gemm_fp8_fp8_bf16_nt_contiguous and ..._masked, and the alignment
 *     query get_m_alignment_for_contiguous_layout: aisharenet.com/ja usage guide,
 *     sections 1-3 of "main functions".
 *   - NT layout only (LHS not transposed, RHS transposed, i.e. B stored N x K); casting
 *     and transposition are the caller's job: turtlesai.it summary, technical paragraph.
 *   - fine-grained scaling and two-level accumulation: same paragraph, and the
 *     chattools.cn article, section on core design ideas.  Each 128-deep K block's
 *     product is formed on its own, multiplied by sA*sB and added into a separate fp32
 *     accumulator; the result is rounded to bf16 with round-to-nearest-even.
 *   - grouping on the M axis only, every group sharing N and K: aisharenet.com/ja usage
 *     guide, section 2; contiguous layout for training / prefill and masked layout for
 *     decode, usable under graph capture: flashmla.org/zh page, section "DeepGEMM
 *     performance".
 *
 * Conventions shared by every call:
 *   - Memory: every pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates and frees nothing.  C is an output the library writes in place.
 *   - Layouts (all row-major, densely packed):
 *       A  e4m3fn bytes,   rows x K         sA fp32, rows x (K/128)
 *       B  e4m3fn bytes,   G x N x K        sB fp32, G x ceil(N/128) x (K/128)
 *       C  bf16 bits,      rows x N
 *     e4m3fn is the OCP 8-bit format E4M3 (bias 7, max 448, no infinities, NaN = S.1111.111);
 *     the _ex calls also take E5M2 for either operand.
 *     Column n of C uses row n/128 of its group's sB; N need not be a multiple of 128.
 *   - Preconditions checked on the host, before any device work, in this order:
 *       shapes: 0 < K <= 2^22 and K % 128 == 0, M/N >= 0, G >= 1,
 *       cap >= 0, fewer than 2^31 64x64 output tiles              -> DG_ERR_SHAPE
 *       operand formats (the _ex calls) DG_FP8_E4M3 or DG_FP8_E5M2  -> DG_ERR_FORMAT
 *       an empty output (no rows or N == 0) returns DG_OK without touching anything
 *       pointers non-NULL                                         -> DG_ERR_NULL
 *       A, B, C 16-byte aligned; sA, sB, group_idx, masked_m 4-byte -> DG_ERR_ALIGN
 *       workspace_bytes >= dg_workspace_bytes(...) and workspace
 *       non-NULL when that is > 0                                 -> DG_ERR_WORKSPACE
 *       current device is a gfx950 GPU                            -> DG_ERR_DEVICE
 *     A failed launch returns DG_ERR_HIP.  Values that live in device memory
 *     (group_idx, masked_m) are never read on the host; their rules are stated per call.
 *   - Execution: every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     null stream), never synchronises, and performs no host readback, so it may be
 *     captured in a HIP graph.  Faults inside kernels surface at the caller's next
 *     synchronisation.  Results are deterministic: the same inputs give the same bits.
 *   - Range: each K block's partial, the factor sA*sB and the accumulator are fp32, so a
 *     result is exact up to fp32 rounding as long as they stay inside the fp32 range.
 *     Scales from the quantisation calls below keep sA*sB finite whenever the two
 *     blocks' maxima multiply to less than about 6.8e43 (448^2 * FLT_MAX); beyond that
 *     the factor is +inf and the element becomes +-inf or NaN (0 * inf, inf - inf).
 *   - Workspace: device memory the caller lends for split-K partial sums, at least
 *     dg_workspace_bytes(...) bytes, 16-byte aligned.  It must be zero filled before
 *     its first use; every call leaves it zero filled again (a zero word marks a partial
 *     not yet written), so one workspace can serve calls of any shape in stream order.
 *     Two calls that may run concurrently must not share one workspace.
 *   - Split-K calls (those with a workspace) never depend on one another's workgroups
 *     making progress: the workgroups sharing an output tile reduce it together when
 *     they all run at once, and the last of them to finish its share completes whatever
 *     is left, summing the tile's partials in a fixed order.  So the result does not
 *     depend on scheduling or on other work sharing the GPU.
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int dg_status;
#define DG_OK 0
#define DG_ERR_NULL 1
#define DG_ERR_SHAPE 2
#define DG_ERR_ALIGN 3
#define DG_ERR_WORKSPACE 4
#define DG_ERR_DEVICE 5
#define DG_ERR_HIP 6
#define DG_ERR_FORMAT 7

/* 8-bit operand formats (OCP): E4M3 ("fn": bias 7, max 448, no infinities) and E5M2
 * (bias 15, max 57344, with infinities).  The usage guide allows either for the inputs
 * (aisharenet.com/ja usage guide, main functions, section 1). */
#define DG_FP8_E4M3 0
#define DG_FP8_E5M2 1

#define DG_DENSE 0
#define DG_CONTIGUOUS 1
#define DG_MASKED 2

/* Row alignment that each group's segment must have in the contiguous layout
 * (aisharenet.com/ja usage guide, section 2: group sizes aligned to the GEMM M block).
 * Returns 128. */
int dg_get_m_alignment_for_contiguous_layout(void);

/* Static, human-readable name of a status code ("DG_OK", ...); never NULL. */
const char *dg_status_string(dg_status status);

/* Workspace bytes the call of kind `kind` (DG_DENSE / DG_CONTIGUOUS / DG_MASKED) needs
 * for these sizes; rows_or_cap is M, M_total or cap.  0 when none is needed.  Returns
 * 0 for invalid shapes (the call itself then reports DG_ERR_SHAPE). */
size_t dg_workspace_bytes(int kind, int64_t rows_or_cap, int64_t N, int64_t K, int64_t G);

/* Name of the kernel instance the call of kind `kind` would use for these sizes
 * (a static string), or "none" for invalid or empty shapes.  Host-only; for logging
 * and tests. */
const char *dg_instance_name(int kind, int64_t rows_or_cap, int64_t N, int64_t K, int64_t G);

/* Dense NT GEMM: C (M x N) = A (M x K) x B (N x K)^T with sA (M x K/128) and
 * sB (ceil(N/128) x K/128).  Every element of C is written.
 * (aisharenet.com/ja usage guide, section 1: gemm_fp8_fp8_bf16_nt.) */
dg_status dg_gemm_fp8_nt(const uint8_t *A, const float *sA,
                         const uint8_t *B, const float *sB,
                         uint16_t *C, int64_t M, int64_t N, int64_t K,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Contiguous grouped NT GEMM (MoE training forward / prefill).  The rows of all groups
 * are concatenated into A (M_total x K); B holds G matrices N x K back to back.
 * group_idx (DEVICE, M_total int32) names the group of each row.  Segments are
 * expected to be 128-row aligned (dg_get_m_alignment_for_contiguous_layout); the
 * defined rule for any content is: row m is written with B[group_idx[m]] iff
 * 0 <= group_idx[m] < G and group_idx[m] == group_idx[128*floor(m/128)]; every other
 * row of C is left untouched (so -1 can mark padding rows).  Segments may come in any
 * group order.  (aisharenet.com/ja usage guide, section 2.) */
dg_status dg_grouped_gemm_fp8_contiguous(const uint8_t *A, const float *sA,
                                         const uint8_t *B, const float *sB,
                                         const int32_t *group_idx, uint16_t *C,
                                         int64_t M_total, int64_t N, int64_t K, int64_t G,
                                         void *workspace, size_t workspace_bytes,
                                         void *stream);

/* Masked grouped NT GEMM (MoE decode).  A is G x cap x K (sA G x cap x K/128), B is
 * G x N x K, C is G x cap x N.  masked_m (DEVICE, G int32) gives each group's count of
 * valid leading rows, clamped to [0, cap] on the device; group g writes rows
 * [0, masked_m[g]) of its C block and never writes the others, and A rows at or past
 * masked_m[g] are never read (they may hold anything).  Nothing is read back to the
 * host, so the call can be captured once and replayed with new counts.
 * (aisharenet.com/ja usage guide, section 3; flashmla.org/zh, "DeepGEMM performance".) */
dg_status dg_grouped_gemm_fp8_masked(const uint8_t *A, const float *sA,
                                     const uint8_t *B, const float *sB,
                                     const int32_t *masked_m, uint16_t *C,
                                     int64_t G, int64_t cap, int64_t N, int64_t K,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* dg_gemm_fp8_nt for callers that cannot allocate device memory (code under graph
 * capture, serving loops that must not call hipMalloc): no workspace argument and no
 * allocation of any kind.  Split-K calls use instead a workspace the library holds in a
 * statically sized device array, one per GPU, kept until the process ends: at most
 * 32 MiB + 64 KiB (enough for every shape this library accepts; a shape needing more
 * would return DG_ERR_WORKSPACE).  On the first call for a device the array's address
 * is looked up and, unless `stream` is being captured, the array is zeroed by a kernel
 * on `stream` (make that first call outside graph capture); every call leaves it zero
 * filled.  All calls on one GPU share the array:
 * two such calls that may overlap in time (on different streams, or from different
 * host threads without ordering) race and give undefined results; calls in one stream's
 * order are fine.  Otherwise as dg_gemm_fp8_nt (E4M3 operands, same errors; DG_ERR_HIP
 * if the array's address cannot be had). */
dg_status dg_gemm_fp8_nt_noalloc(const uint8_t *A, const float *sA,
                                 const uint8_t *B, const float *sB,
                                 uint16_t *C, int64_t M, int64_t N, int64_t K, void *stream);

/* The same three calls with explicit operand formats: a_format / b_format are
 * DG_FP8_E4M3 or DG_FP8_E5M2 (any pair), else DG_ERR_FORMAT.  The calls above are these
 * with both formats DG_FP8_E4M3.  Everything else (layouts, scales, routing, workspace,
 * errors, execution) is as described there; the choice of kernel instance, and hence
 * dg_workspace_bytes / dg_instance_name, does not depend on the formats.
 * (aisharenet.com/ja usage guide, main functions, section 1: E4M3 or E5M2 inputs.) */
dg_status dg_gemm_fp8_nt_ex(const uint8_t *A, int a_format, const float *sA,
                            const uint8_t *B, int b_format, const float *sB,
                            uint16_t *C, int64_t M, int64_t N, int64_t K,
                            void *workspace, size_t workspace_bytes, void *stream);
dg_status dg_grouped_gemm_fp8_contiguous_ex(const uint8_t *A, int a_format, const float *sA,
                                            const uint8_t *B, int b_format, const float *sB,
                                            const int32_t *group_idx, uint16_t *C,
                                            int64_t M_total, int64_t N, int64_t K, int64_t G,
                                            void *workspace, size_t workspace_bytes,
                                            void *stream);
dg_status dg_grouped_gemm_fp8_masked_ex(const uint8_t *A, int a_format, const float *sA,
                                        const uint8_t *B, int b_format, const float *sB,
                                        const int32_t *masked_m, uint16_t *C,
                                        int64_t G, int64_t cap, int64_t N, int64_t K,
                                        void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * fp8 quantisation with block scales: the casting step in front of the GEMM, which the
 * pages leave to the caller (turtlesai.it summary, technical paragraph), in the two
 * block shapes of the method's fine-grained scaling (chattools.cn, core design ideas):
 * one scale per 1x128 block of a row (activations, the sA layout) and one per 128x128
 * block (weights, the sB layout).
 *
 * Per block: amax = max |x| in fp32; scale = amax / FMAX in fp32 (FMAX = 448 for E4M3,
 * 57344 for E5M2; 1 for an all-zero block); each code is x / scale, an IEEE fp32
 * division, rounded to the nearest value of `format`, ties to even, saturating at
 * +-FMAX.  So Q * S reproduces X to within half an fp8 step of each block's scale.
 *
 * Inputs: X rows x K (row-major, DEVICE, 16-byte aligned), x_dtype DG_IN_F32 or
 * DG_IN_BF16; values must be finite (non-finite inputs give unspecified codes and
 * scales, never a fault).  K > 0, K % 128 == 0 (DG_ERR_SHAPE); rows >= 0 (0: nothing
 * to do).  Outputs (DEVICE, caller-owned): Q rows x K codes (8-byte aligned); S rows x
 * K/128 (1x128) or ceil(rows/128) x K/128 (128x128) fp32 (4-byte aligned).
 * Errors: DG_ERR_SHAPE, DG_ERR_FORMAT (format or x_dtype), DG_ERR_NULL, DG_ERR_ALIGN,
 * DG_ERR_DEVICE, DG_ERR_HIP, checked in that order.  Asynchronous on `stream`,
 * graph-capturable, deterministic. */
#define DG_IN_F32 0
#define DG_IN_BF16 1

dg_status dg_quantize_fp8_1x128(const void *X, int x_dtype, uint8_t *Q, float *S,
                                int64_t rows, int64_t K, int format, void *stream);
dg_status dg_quantize_fp8_128x128(const void *X, int x_dtype, uint8_t *Q, float *S,
                                  int64_t rows, int64_t K, int format, void *stream);

/* Transposition of a byte matrix (fp8 codes): Y (cols x rows) = X (rows x cols)^T, both
 * row-major DEVICE buffers, 16-byte aligned, rows and cols multiples of 16.  The calls
 * above take the NT layout only and leave transposition to the caller (turtlesai.it
 * summary, technical paragraph); this turns a K x N operand into the N x K one they
 * take.  (Its 128x128 scale matrix transposes as an ordinary small fp32 matrix.)
 * Errors: DG_ERR_SHAPE, DG_ERR_NULL, DG_ERR_ALIGN, DG_ERR_DEVICE, DG_ERR_HIP, in that
 * order; rows or cols 0: nothing to do.  Asynchronous on `stream`. */
dg_status dg_transpose_fp8(const uint8_t *X, uint8_t *Y, int64_t rows, int64_t cols,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DG_H_ */
