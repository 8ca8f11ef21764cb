/*
 * qmm.h — 4-bit weight-quantized matmul Y = X·Wᵀ on AMD MI355X (gfx950).
 *
 * X[T, D] holds bf16 activations, W[N, D] holds 4-bit codes (one output
 * feature per row of W), Y[T, N] is stored as bf16 (row-vector convention of
 * Kapitsa 源码拆解 02：权重、矩阵与 Metal, section "矩阵乘法中数据和参数").
 *
 * Weight formats
 *   QMM_AFFINE4_G64  groups of 64 codes along D, one bf16 scale and one bf16
 *                    bias per group, w = scale·q + bias with q in 0..15
 *                    (same page, section "权重怎样存储": 32 bytes of codes plus
 *                    two bf16, 36 bytes per 64 weights).
 *   QMM_MXFP4_G32    groups of 32 E2M1 codes along D sharing one E8M0
 *                    exponent, w = E2M1(c)·2^(E-127) (Kimi K3 迁移到 Google TPU
 *                    的可行性评估（v2）, section 2 模型解剖, quantisation row:
 *                    W4 group 32 + E8M0, 4.25 bit; element encoding per the
 *                    OCP Microscaling Formats v1.0 specification).
 *
 * Canonical (input) layouts, row-major:
 *   affine codes  uint32[N][D/8]: code k of row n is bits 4(k%8)..4(k%8)+3 of
 *                 word k/8 (lowest nibble first);
 *   affine scale, bias  bf16[N][D/64];
 *   MXFP4 codes   uint8[N][D/2]: code k of row n is the low nibble of byte k/2
 *                 for even k, the high nibble for odd k;
 *   MXFP4 E8M0    uint8[N][D/32].
 *
 * Conventions for every call
 *   - Pointers are caller-owned DEVICE memory unless stated otherwise; the
 *     library never allocates, frees or retains them.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls are
 *     asynchronous on it and return after the kernels are enqueued, except
 *     where a call says it synchronizes.  Reading results on the host needs a
 *     stream or event synchronization first (the non-blocking commit + explicit
 *     wait of Kapitsa 源码拆解 02, section "C++ 代码如何提交 GPU 计算").
 *   - Validation happens on the host before any launch; a rejected call
 *     launches nothing and touches no memory.  Nothing aborts, throws or
 *     exits across this interface.  QMM_E_HIP reports a HIP runtime error
 *     (launch failure, no device); qmm_last_error() then holds the HIP text.
 *   - Alignment (QMM_E_ALIGN otherwise): `packed` 256 bytes, x 16 bytes,
 *     codes and routing tables 4 bytes, y, scales and biases 2 bytes.
 *   - The kernels trust that `packed` holds a blob of this (format, n, d);
 *     only qmm_unpack reads the header back to check it.
 *   - Summation order is fixed per shape and launch configuration, so
 *     repeated calls give bitwise identical results (no float atomics).
 *   - Calls on different streams may run concurrently; the only process
 *     state is a per-device cache of device properties.
 *   - The matmul, routing and combine calls only enqueue kernels on `stream`
 *     (no allocation, copy, memset or synchronization), so a sequence of them
 *     can be recorded into a HIP graph by stream capture and replayed; the
 *     buffers are then fixed at capture and the host scalars (sizes,
 *     max_seg_rows) with them.  qmm_pack and qmm_unpack synchronize and
 *     cannot be captured.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QMM_OK = 0,
  QMM_E_ARG = 1,          /* NULL pointer, bad enum, negative size, inconsistent argument */
  QMM_E_SHAPE = 2,        /* D not a multiple of the group, size out of supported range */
  QMM_E_ALIGN = 3,        /* pointer misaligned for the call */
  QMM_E_UNSUPPORTED = 4,  /* valid request the library does not implement */
  QMM_E_WORKSPACE = 5,    /* workspace NULL or smaller than qmm_workspace_bytes() */
  QMM_E_HIP = 6,          /* HIP runtime error; see qmm_last_error() */
  QMM_E_LAYOUT = 7,       /* packed blob header does not match (format, n, d, version) */
  QMM_E_VALUE = 8         /* input value outside the supported range (see qmm_pack) */
} qmm_status;

typedef enum { QMM_AFFINE4_G64 = 1, QMM_MXFP4_G32 = 2 } qmm_format;

typedef uint16_t qmm_bf16; /* raw bf16 bits */

/* Supported ranges: 1 <= n <= 2^28; group <= d <= 65536 with d % group == 0;
 * 1 <= t <= 2^24 rows for qmm_gemm. */

/* Bytes of the packed device blob for a W[n, d] (a 256-byte header followed by
 * the codes and the per-group metadata; 36 payload bytes per 64 affine
 * weights, 17 per 32 MXFP4 weights), rounded up to 256.  0 if the shape or
 * format is invalid.  Host only; touches no device. */
size_t qmm_packed_bytes(qmm_format f, int64_t n, int64_t d);

/* Workspace of qmm_gemm(f, t, n, d) in bytes (0 = none used; 0 also for
 * t = 1 and for an invalid shape).  Every caller buffer has its size stated
 * per format and shape by a call like this one, as the explicit per-format
 * byte counts that fixed the NULL-scale crash of "Colibri Kimi K3 Metal
 * 后端实现全解析", Phase 10 (fmt_scale_bytes).
 *   2 <= t <= 64 rows on the multi-row kernel (see qmm_gemm: for t <= 16
 *     d <= 3072, MXFP4 weights with n >= 5120 or t <= 8, or affine weights
 *     with n >= 8192, while the t rows fit the kernel's LDS; for 17 <= t <= 64
 *     d <= 2048, n >= 6912 with d <= 5120, or n >= 10240): 0.
 *   other 2 <= t <= 64 rows: one fp32 [t][n] plane per 512-code slab of d,
 *     ceil(d/512)·t·n·4 bytes (0.66 MB for t = 4, n = 4096, d = 5120).
 *   t > 64, affine weights: the activations converted to fp16 (t·d·2 bytes),
 *     one int32 exponent per row and per weight column, each rounded up to
 *     256 bytes (21.0 MB for t = 2048, n = 13824, d = 5120), plus, while the
 *     tile kernel has few tiles (128-row tiles over at most 128 workgroups)
 *     and d is a multiple of 512, up to eight K-split planes of t·n·4 bytes.
 *   t > 64, MXFP4 weights: those K-split planes, else 0.
 * Affine weights REQUIRE this workspace where it is not 0 (QMM_E_WORKSPACE
 * without one).  For MXFP4 it is optional: ws = NULL runs the tile kernel,
 * several times slower for 2 <= t <= 64.  A non-NULL ws must be 16-byte aligned and
 * hold at least this many bytes (QMM_E_ALIGN, QMM_E_WORKSPACE).  Its contents
 * on entry do not matter, and calls sharing one workspace must be ordered on
 * one stream.  Under a forced kernel (qmm_set_kernel) the size is that
 * kernel's.  Host only. */
size_t qmm_workspace_bytes(qmm_format f, int64_t t, int64_t n, int64_t d);

/* Pack canonical weights into the MI355X device layout.  The codes are the
 * 4-bit values of "Kapitsa 源码拆解 02：权重、矩阵与 Metal", section "权重怎样存储"
 * (eight codes per 32-bit word, one bf16 scale and one bf16 bias per group of
 * 64), or the MXFP4 U8-packed codes with one E8M0 exponent per 32 of "Kimi K3
 * 迁移到 Google TPU 的可行性评估（v2）", sections 2 and 3.1.
 *   codes   canonical codes (see above), device
 *   scales  affine: bf16 scales [n][d/64]; MXFP4: uint8 E8M0 [n][d/32], device
 *   biases  affine: bf16 biases [n][d/64]; MXFP4: must be NULL
 *   packed  device buffer of qmm_packed_bytes(f, n, d) bytes, written whole
 * A pure bit/byte permutation plus header: no arithmetic on values.  The
 * call SYNCHRONIZES `stream` to report values outside the supported range as
 * QMM_E_VALUE, and the blob is then marked invalid: for MXFP4 an E8M0 byte of
 * 255 (NaN scale); for affine a scale that is not finite or whose magnitude is
 * 2^100 or more, or a bias that is not finite (the MFMA kernels scale s by
 * 2^24 while dequantising, which must not overflow).  One-time preparation,
 * not a hot-path call. */
qmm_status qmm_pack(qmm_format f, int64_t n, int64_t d, const void* codes, const void* scales,
                    const void* biases, void* packed, void* stream);

/* Inverse of qmm_pack (test support): rewrites the canonical arrays from a
 * blob, so that the layout of "Kapitsa 源码拆解 02：权重、矩阵与 Metal", section
 * "权重怎样存储", can be checked to survive packing bit for bit (every primitive
 * checked against the CPU before it is used: "Colibri Kimi K3 Metal 后端实现全解析",
 * Phase 5).  SYNCHRONIZES `stream` to check the blob header first
 * (QMM_E_LAYOUT on a mismatch or an invalid blob). */
qmm_status qmm_unpack(qmm_format f, int64_t n, int64_t d, const void* packed, void* codes,
                      void* scales, void* biases, void* stream);

/* Decode GEMV: y[n] = Σ_k x[k]·ŵ[n,k] for one activation row.
 *   packed  blob from qmm_pack(f, n, d); x bf16[d]; y bf16[n] (written whole).
 * fp32 accumulation, bf16 round-to-nearest-even output.  n·d/2 must be
 * below 2^31 (32-bit addressing; QMM_E_SHAPE).  Several matrices
 * that share x (a Q/K/V triple, a gate/up pair: the fused dispatches of
 * "LLM Decode / Prefill 优化案例（Metal）", Steps 8-9) run as one launch when
 * packed as one matrix with their rows concatenated: y then holds their
 * outputs back to back, each bit-identical to its own call.  The same holds
 * for qmm_gemm. */
qmm_status qmm_gemv(qmm_format f, const void* packed, int64_t n, int64_t d, const qmm_bf16* x,
                    qmm_bf16* y, void* ws, size_t ws_bytes, void* stream);

/* Deferred-dequantisation decode GEMV (an approximation; affine weights
 * only): the deferred dequantisation of "LLM Decode / Prefill 优化案例（Metal）",
 * Step 2.  The activation row is quantised to int8 by its absolute maximum
 * (s = absmax/127 and x_q = round-half-even(x/s), both in fp32), the 4-bit
 * codes meet it in exact int32 sums per 32-code chunk, and
 *   y[n] = s·Σ_chunks (scale·Σ x_q·q + bias·Σ x_q),
 * fp32 from the integer sums on, rounded once to bf16.  The loss of the
 * activations' low bits makes it differ from qmm_gemv by up to ~s/2 per
 * activation.  Limits as for qmm_gemv, plus d <= 57344 and n·d/2 < 2^31;
 * MXFP4 returns QMM_E_UNSUPPORTED.  No workspace. */
qmm_status qmm_gemv_int8(qmm_format f, const void* packed, int64_t n, int64_t d, const qmm_bf16* x,
                         qmm_bf16* y, void* stream);

/* Prefill GEMM: Y[t][n] = Σ_k X[t][k]·ŵ[n,k], the multi-row product of
 * "Kapitsa 源码拆解 02：权重、矩阵与 Metal", section "矩阵乘法中数据和参数" (many
 * activation rows share each weight read, unlike the one-row decode).
 *   x bf16[t][d] row-major; y bf16[t][n] row-major (written whole);
 *   ws, ws_bytes: the workspace of qmm_workspace_bytes(f, t, n, d), required
 *   for affine weights where that is not 0 (see there), optional for MXFP4.
 * t = 1 runs the GEMV kernel.  Otherwise MFMA with fp32 accumulation, every
 * output rounded once to bf16:
 *   2 <= t <= 16, multi-row kernel (d <= 3072, MXFP4 weights with n >= 5120
 *     or t <= 8, or affine weights with n >= 8192, while its LDS fits 160 KiB: the t rows
 *     padded to whole 512-code slabs, t·ceil(d/512) KiB (one row more for
 *     affine weights with t <= 8), plus 6 KiB, plus ceil(d/512)/2 KiB for
 *     affine weights; at d = 5120 affine t <= 14, MXFP4 t <= 15): every
 *     weight read once for all rows, no workspace, one kernel.  Affine codes enter bf16 MFMAs as the exact
 *     values 128 + q and each group's scale and bias follow in fp32.
 *   17 <= t <= 64 with d <= 2048, n >= 6912 and d <= 5120, or n >= 10240: the same
 *     kernel with the rows streamed through LDS one 512-code slab at a
 *     time (two buffers of 16·ceil(t/16) rows, at most 132 KiB): every
 *     weight read once for all rows, no workspace, one kernel.
 *   other 2 <= t <= 64 (with the workspace): split along d, each 512-code slab's
 *     fp32 partial sums in the workspace, added in slab order by a second
 *     kernel.  Affine codes enter bf16 MFMAs as the exact values 128 + q and
 *     each group's scale and bias follow in fp32, so no weight is rounded.
 *   t > 64, affine: a first kernel converts x to fp16 in the workspace, each
 *     row scaled by a power of two (exact for every element within 2^-30 of
 *     its row's largest), and finds a power of two per weight column; the
 *     tile kernel forms each weight fp16(2^f·(s·q + b)), rounded once
 *     (relative error <= 2^-11 wherever the scaled weight is a normal fp16:
 *     every weight within 2^-27 of its column's largest), runs fp16 MFMAs
 *     and removes both powers of two exactly.  With few tiles the tile kernel
 *     is split along d into up to eight fp32 planes summed in order.
 *   MXFP4: the weights are bf16 MFMA operands, exact for E8M0 in [2, 252]
 *     (at 253 and 254 the largest codes reach 2^128: not representable).
 * Profiling events armed by qmm_profile_next bracket every kernel of the
 * call. */
qmm_status qmm_gemm(qmm_format f, const void* packed, int64_t t, int64_t n, int64_t d,
                    const qmm_bf16* x, qmm_bf16* y, void* ws, size_t ws_bytes, void* stream);

/* qmm_gemm without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels and results as qmm_gemm
 * given a workspace of qmm_workspace_bytes(f, t, n, d) bytes: bitwise the same
 * outputs.  What that workspace holds (split-K partial sums; for affine
 * weights with t > 64 the fp16 activations and the exponents) goes to a
 * static 64 MiB device array inside the library instead (one per GPU,
 * allocated with the library's code object and held until the process ends;
 * its address is looked up on the first call on each device).  Limit: qmm_workspace_bytes(f, t, n, d) <= 64 MiB
 * (67108864 bytes), else QMM_E_WORKSPACE and nothing launched.  The call
 * allocates and frees nothing.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, unordered threads) race on
 * it and must be serialised by the caller.  Nothing in the array needs to
 * start at zero (everything read from it is written first in the same call). */
qmm_status qmm_gemm_noalloc(qmm_format f, const void* packed, int64_t t, int64_t n, int64_t d,
                            const qmm_bf16* x, qmm_bf16* y, void* stream);

/* Routed-expert grouped matmul (all experts in one launch, or two when the
 * row bound splits the segments between two kernels, see max_seg_rows): the
 * per-expert GEMM of the MoE block of "Colibri Kimi K3 Metal 后端实现全解析",
 * Phase 6, whose experts all run in one submission so the launch cost is
 * paid once per kernel, not per expert.
 *   packed_stack        n_experts blobs of qmm_packed_bytes(f, n, d) bytes,
 *                       blob e at packed_stack + e·expert_stride_bytes
 *                       (stride a multiple of 256, >= the blob size)
 *   x                   bf16[t_x][d] activation rows
 *   row_index           int32[m_total]: grouped row r reads x row row_index[r];
 *                       or NULL: row r reads x row r (x already in grouped
 *                       order, e.g. the activated rows of the expert FFN;
 *                       never the decode GEMV path)
 *   seg_expert          int32[n_seg]: expert of segment s
 *   seg_offsets         int32[n_seg + 1]: segment s owns grouped rows
 *                       [seg_offsets[s], seg_offsets[s+1])
 *   max_seg_rows        host upper bound on segment sizes; it selects the
 *                       kernel, never memory bounds: 1 = the decode GEMV
 *                       path; 2..8 = the multi-row kernel (each expert's
 *                       weights read once per pass of up to max_seg_rows
 *                       rows; a longer segment takes several passes);
 *                       more = two launches that split the segments on
 *                       the device: those of at most 8 rows to the
 *                       multi-row kernel, the longer ones to the matmul
 *                       kernel (which takes all of them when forced with
 *                       QMM_KERNEL_GROUPED_MATMUL, or where the multi-row
 *                       kernel's LDS or offsets do not fit the shape)
 *   y                   bf16[m_total][n]: row r = x[row_index[r]]·Ŵ_eᵀ
 * row_index, seg_expert, seg_offsets are device arrays; n_seg, m_total,
 * max_seg_rows, t_x, n_experts are host scalars.  The kernels clamp segment
 * bounds to [0, m_total] and never read outside x or the stack: a segment
 * whose expert is outside [0, n_experts), or a row whose row_index is outside
 * [0, t_x), gets NaN outputs.  Rows covered by no segment are not written. */
qmm_status qmm_grouped_gemm(qmm_format f, const void* packed_stack, int64_t expert_stride_bytes,
                            int32_t n_experts, int64_t n, int64_t d, const qmm_bf16* x,
                            int64_t t_x, const int32_t* row_index, const int32_t* seg_expert,
                            const int32_t* seg_offsets, int32_t n_seg, int32_t m_total,
                            int32_t max_seg_rows, qmm_bf16* y, void* ws, size_t ws_bytes,
                            void* stream);

/* Routed-expert gate_up matmul with the SwiGLU activation fused into its
 * epilogue (the per-expert SwiGLU of "Colibri Kimi K3 Metal 后端实现全解析":
 * the silu_mul operation of its Metal API table, fused into the MoE block in
 * Phase 6).  Arguments as for qmm_grouped_gemm, with the stack's n rows read
 * as the gate (rows [0, n/2)) followed by the up projection (rows [n/2, n)):
 *   h   bf16[m_total][n/2]: h[r][j] = silu(g)·u, g = (x_r·Ŵ_eᵀ)[j],
 *       u = (x_r·Ŵ_eᵀ)[n/2 + j], silu(v) = v / (1 + e^-v); g and u are the
 *       fp32 accumulations (never rounded), h is rounded once to bf16.
 * n must be even (QMM_E_SHAPE).  max_seg_rows selects the kernels as for
 * qmm_grouped_gemm, except that a bound of 1 takes the multi-row kernel too
 * (there is no GEMV form with the activation).  Error rows are NaN as for
 * qmm_grouped_gemm. */
qmm_status qmm_grouped_gemm_swiglu(qmm_format f, const void* packed_stack,
                                   int64_t expert_stride_bytes, int32_t n_experts, int64_t n,
                                   int64_t d, const qmm_bf16* x, int64_t t_x,
                                   const int32_t* row_index, const int32_t* seg_expert,
                                   const int32_t* seg_offsets, int32_t n_seg, int32_t m_total,
                                   int32_t max_seg_rows, qmm_bf16* h, void* ws, size_t ws_bytes,
                                   void* stream);

/* MoE combine: each token's expert outputs weighted and summed back into
 * token space (the weighted scatter-add of "Colibri Kimi K3 Metal 后端实现全解析",
 * Phase 6), the weights being the chosen experts' routing weights
 * renormalised to sum to one ("Kimi K3 迁移到 Google TPU 的可行性评估（v2）", §2:
 * sigmoid + renormalize).
 *   o            bf16[m_total][d], device: expert outputs in the grouped order
 *   topk         int32[t][k], device: each token's experts (qmm_route)
 *   weights      fp32[t][n_experts], device: routing weights (qmm_route's scores)
 *   seg_offsets  int32[n_experts + 1], device: dense per-expert segments
 *   row_index    int32[m_total], device: the token of each grouped row,
 *                ascending inside a segment (qmm_route's tables)
 *   out          bf16[t][d], device, written:
 *                out[t] = Σ_j w_j·o[r_j] with w_j = weights[t][e_j] /
 *                Σ_j' weights[t][e_j'] (summed in slot order), r_j the row of
 *                token t in expert e_j's segment; fp32, rounded once to bf16.
 * One workgroup per token; the sums run in slot order, so results do not
 * depend on timing.  A slot whose expert is out of range or whose token is
 * missing from that expert's segment makes the token's outputs NaN.
 * Limits: 1 <= k <= 64, d a multiple of 8 in [8, 65536], t·k < 2^31; o and
 * out 16-byte aligned, the tables 4-byte aligned (QMM_E_* otherwise). */
qmm_status qmm_moe_combine(const qmm_bf16* o, int32_t m_total, int64_t d, int64_t t, int32_t k,
                           const int32_t* topk, const float* weights, int32_t n_experts,
                           const int32_t* seg_offsets, const int32_t* row_index, qmm_bf16* out,
                           void* stream);

/* MoE router (the step before qmm_grouped_gemm for routed prefill): a sigmoid
 * router with a selection-only bias, top-k per token, tokens grouped by expert
 * ("Colibri Kimi K3 Metal 后端实现全解析", introduction: router with a
 * score-correction bias; "Kimi K3 迁移到 Google TPU 的可行性评估（v2）", §2:
 * sigmoid scoring, top-16 of 896 routed experts).
 *   x        bf16 [t][d], row-major, device, 16-byte aligned
 *   r        bf16 [n_experts][d], the router weights, device, 16-byte aligned
 *   bias     fp32 [n_experts], device, or NULL for none; it changes which
 *            experts are chosen and nothing else
 *   scores   fp32 [t][n_experts], device, written: sigmoid(x·rᵀ), products
 *            accumulated in fp32 -- the routing weights (qmm_moe_combine
 *            renormalises the chosen ones)
 *   topk     int32 [t][k], device, written: each token's experts by the
 *            selection score fp32(scores + bias), highest first, equal
 *            selection scores to the lower expert id; -inf ranks below every
 *            finite value and NaN below -inf (-0 equals +0)
 *   seg_expert  int32 [n_experts], written 0 .. n_experts-1
 *   seg_offsets int32 [n_experts + 1], written: segment e (expert e, possibly
 *            empty) covers grouped rows [seg_offsets[e], seg_offsets[e+1])
 *   row_index   int32 [t*k], written: the tokens of each segment, ascending
 * The three tables feed qmm_grouped_gemm directly (n_seg = n_experts,
 * m_total = t*k, max_seg_rows = t): no count has to come back to the host.
 * Limits: t >= 1; 1 <= n_experts <= 1024; 1 <= k <= min(64, n_experts);
 * d a multiple of 8, 8 <= d <= 65536; t*d*2 and n_experts*d*2 below 2^31;
 * t*k below 2^30 (QMM_E_SHAPE / QMM_E_ARG / QMM_E_ALIGN otherwise, nothing
 * launched).  Three kernel launches on `stream`, asynchronous; armed
 * profiling events bracket all three.  The library allocates nothing. */
qmm_status qmm_route(const qmm_bf16* x, int64_t t, int64_t d, const qmm_bf16* r, int32_t n_experts,
                     const float* bias, int32_t k, float* scores, int32_t* topk,
                     int32_t* seg_expert, int32_t* seg_offsets, int32_t* row_index, void* stream);

/* Per-kernel GPU timing (per-op GPU timestamps, as in the op profiling of
 * "LLM Decode / Prefill 优化案例（Metal）", Step 1).  Arms two caller-owned
 * hipEvent_t handles for the next qmm_gemv / qmm_gemm / qmm_grouped_gemm /
 * qmm_grouped_gemm_swiglu / qmm_moe_combine / qmm_route / qmm_stream_read call
 * on this thread: its kernels are launched with hipExtLaunchKernel so `start`
 * is stamped by the dispatch of its first kernel and `stop` by that of its last
 * (calls of several kernels: qmm_route, qmm_gemm split along K), and their
 * elapsed time is the call's execution time.  Either may be NULL.  The arming
 * is consumed by that next call; a call rejected by validation leaves it armed. */
qmm_status qmm_profile_next(void* start_event, void* stop_event);

/* Kernel override for A/B runs: one matmul kernel forced in place of the
 * library's own choice, so that each can be timed and checked on its own.
 * The pages switch fused paths off or on from the environment for exactly
 * this ("LLM Decode / Prefill 优化案例（Metal）", Steps 9 and 11), and run only
 * some kernels on the GPU to check them in isolation ("Colibri Kimi K3 Metal
 * 后端实现全解析", Phase 10).
 *   QMM_KERNEL_AUTO            the library's choice (the default).
 *   QMM_KERNEL_TILE            qmm_gemm / qmm_gemm_noalloc run the tile GEMM
 *                              for every t >= 1 (t = 1 included), with its
 *                              own tile height and K split.
 *   QMM_KERNEL_TILE_UNSPLIT    the same, never split along K.
 *   QMM_KERNEL_FEW_ROW         qmm_gemm runs the few-row split-K kernel; a
 *                              shape it does not take (t = 1 or t > 64)
 *                              returns QMM_E_UNSUPPORTED, and it needs a
 *                              workspace for both formats.
 *   QMM_KERNEL_GROUPED_MATMUL  qmm_grouped_gemm runs the matmul kernel also
 *                              where every segment has one row.
 *   QMM_KERNEL_MULTI_ROW       qmm_gemm runs the multi-row kernel for every
 *                              shape it takes (2 <= t <= 16 with the rows
 *                              within its LDS, or 17 <= t <= 64 streamed),
 *                              others return QMM_E_UNSUPPORTED; no
 *                              workspace.
 * A setting that does not concern a call leaves it as under AUTO.
 * qmm_workspace_bytes reports the workspace of the kernel the setting
 * selects, so size workspaces after changing it.  The setting is
 * process-wide and takes effect for calls that start after it returns.  Its
 * initial value comes from the environment variable QMM_FORCE_KERNEL, read
 * once at the first call that consults it: unset, "" or "auto", "tile",
 * "tile_unsplit", "few_row", "grouped_matmul", "multi_row", or the digits
 * 0..5.  Any other
 * value makes qmm_gemm, qmm_gemm_noalloc and the grouped calls fail with
 * QMM_E_ARG (a mistyped switch is reported, not ignored) until qmm_set_kernel
 * is called.  qmm_set_kernel returns QMM_E_ARG for a value outside the enum;
 * qmm_get_kernel returns the current setting, -1 for an invalid environment
 * value.  Host only. */
typedef enum {
  QMM_KERNEL_AUTO = 0,
  QMM_KERNEL_TILE = 1,
  QMM_KERNEL_TILE_UNSPLIT = 2,
  QMM_KERNEL_FEW_ROW = 3,
  QMM_KERNEL_GROUPED_MATMUL = 4,
  QMM_KERNEL_MULTI_ROW = 5
} qmm_kernel;
qmm_status qmm_set_kernel(qmm_kernel k);
int qmm_get_kernel(void);

/* Measurement support: the achievable HBM read rate.  Reads every byte of the
 * device buffer `src` once (16-byte non-temporal loads, four in flight per
 * thread, 2048 workgroups of 256 threads, grid-stride) and stores one word per
 * workgroup to `sink` (device,
 * >= 2048 uint32): the XOR of the words it read, so the XOR of all 2048
 * stored words equals the XOR of the buffer.  `src` 16-byte aligned, `bytes`
 * a multiple of 16, 0 < bytes < 2^31 (QMM_E_ALIGN / QMM_E_SHAPE otherwise).
 * Asynchronous on `stream`; armed profiling events apply to it as to the
 * matmul calls.  Not part of the matmul path: a ceiling to report its
 * HBM-bound kernels against. */
qmm_status qmm_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Static description of a status code.  Every entry point reports failure
 * as a status the caller can act on (the stubs of "Colibri Kimi K3 Metal
 * 后端实现全解析", Phase 4, return NOT IMPLEMENTED and the caller falls back;
 * Phase 10's crash came from a size that was not checked). */
const char* qmm_status_string(qmm_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char* qmm_last_error(void);

/* Layout version stamped into packed blobs. */
uint32_t qmm_layout_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
