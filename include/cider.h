/*
 * cider.h - C ABI of the MI355X (gfx950) online-quantized W8A8 / W4A8 linear layer.
 *
 * The operation follows the top-level Cider README:
 *   - section "架构 / Metal Kernel 流水线" (kernel pipeline): a prefill linear is
 *     two device steps, fp16 activations -> int8 codes + one scale per token,
 *     then an INT8 x INT8 -> INT32 matmul whose store stage applies the scales
 *     and writes fp16; for W4A8 the int4 weights are unpacked to int8 while the
 *     matmul loads its fragments;
 *   - section "量化" (Quantization) table: symmetric INT8 weights (per output
 *     channel or per group of 64/128), symmetric INT4 weights with zero point 8,
 *     symmetric INT8 per-token activations, INT32 accumulation, and
 *     C_fp16 = C_int32 * s_act * s_weight per element;
 *   - section "W8A8 量化粒度" (quantization granularity) table: per-channel,
 *     per-group gs = 128, per-group gs = 64;
 *   - section "底层 API" (low-level API): weight quantizers return
 *     (codes, scale); the linear takes (x, codes, scale).
 *
 * Readings of details the page leaves open (fixed here, identical in the CPU
 * oracle that the tests compare against):
 *   - scale = max|v| / qmax in fp32 (one correctly rounded division), qmax = 127
 *     for int8 and 7 for int4; a group whose max|v| is 0 gets scale 0, codes 0;
 *   - code = clamp(round_half_even(v / scale), -qmax, qmax) where v / scale is
 *     one correctly rounded fp32 division; -128 never appears;
 *   - per-group (group_size 64 or 128) groups run along K for the activation
 *     AND the weight: y[m,n] = sum_g acc_g[m,n] * s_a[m,g] * s_w[n,g];
 *   - int4: code c stored as nibble c + 8, byte j of a weight row holds code 2j
 *     in its low nibble and code 2j+1 in its high nibble ([N, K/2] bytes);
 *   - dequant: ((float)acc * s_a) * s_w in fp32 (per group: summed over groups
 *     in fp32), rounded to nearest-even fp16. Outputs that overflow fp16 become
 *     +-inf. Non-finite inputs give unspecified results.
 *
 * Conventions for every call below:
 *   - All tensor arguments are DEVICE pointers to contiguous row-major arrays,
 *     owned by the caller, and must be 16-byte aligned. The library never
 *     allocates, frees, retains or synchronizes; it enqueues kernels on
 *     `stream` (a hipStream_t; NULL = the legacy default stream) and returns.
 *   - Arguments are validated before any HIP call is made. A bad argument
 *     returns CIDER_ERROR_INVALID_VALUE and enqueues nothing; a device that is
 *     not gfx950 returns CIDER_ERROR_NOT_SUPPORTED; a failed launch returns
 *     CIDER_ERROR_LAUNCH. A kernel fault surfaces at the caller's next
 *     synchronization, as usual in HIP.
 *   - Zero-sized work (M == 0 or N == 0) returns CIDER_SUCCESS and launches
 *     nothing; the pointers may then be NULL. Size queries (int64_t results)
 *     return -1 for invalid arguments.
 *   - K is at most CIDER_MAX_K, which keeps |acc| = |sum of K products of
 *     codes| <= 127*127*K below 2^31. The per-channel calls (cider_quant_act
 *     and cider_quant_weight with group_size 0, cider_w8a8_gemm[_dt/_ex/
 *     _noalloc] and cider_gemm_acc_i32 with group_size 0, cider_linear[_dt]
 *     with group_size 0) accept any K >= 1 for int8 codes and any even K for
 *     packed int4 weights; rows whose length is not a multiple of 16 code
 *     bytes (32 codes for int4) start at unaligned addresses and take a
 *     general, slower path with the same results. Per-group calls need
 *     K % group_size == 0. cider_int8_mv, cider_w8a8_gemm_token_group[_dt],
 *     cider_w8a8_gemm_split[_dt], cider_quant_weight_clip and the stack
 *     driver need K a multiple of 16 (32 for int4 weights).
 *   - Calls are reentrant; concurrent calls on different streams do not share
 *     any library state (there is none beyond a cached device-architecture flag).
 */
#ifndef CIDER_H
#define CIDER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CIDER_MAX_K 133120 /* multiple of 128; 127*127*133120 < 2^31 */

typedef enum {
  CIDER_SUCCESS = 0,
  CIDER_ERROR_INVALID_VALUE = 1,
  CIDER_ERROR_NOT_SUPPORTED = 2,
  CIDER_ERROR_LAUNCH = 3,
  CIDER_ERROR_SCRATCH_LIMIT = 4, /* cider_w8a8_gemm_noalloc: the shape needs more scratch */
} cider_status_t;

/* Element types of fp inputs and outputs (the README's roadmap: automatic
 * float16 / bfloat16 handling). bf16 values quantize by the same rule (their
 * fp32 images are exact); a bf16 output is the fp32 dequant value of the
 * fp16 output's arithmetic rounded to bf16 (nearest, ties to even). */
typedef enum {
  CIDER_DTYPE_F16 = 0,
  CIDER_DTYPE_BF16 = 1,
} cider_dtype_t;

/* 1 if the current HIP device is a gfx950 (MI355X-class) GPU, else 0.
 * Mirrors the README's is_available() gate (section "条件编译"). */
int cider_is_available(void);

/* Static, NUL-terminated description of a status code. */
const char* cider_status_string(cider_status_t status);

/* Library version as major*10000 + minor*100 + patch. */
int cider_version(void);

/* Online activation quantization (pipeline step "quantize_per_token").
 *   x_f16   : fp16 [M, K] activations.
 *   group_size : 0 = one scale per token (row); 64 or 128 = one scale per
 *                run of group_size consecutive K elements of a row.
 *   x_q     : int8 [M, K] codes (output).
 *   x_scale : fp32 [M] (group_size 0) or [M, K/group_size] (output).
 */
cider_status_t cider_quant_act(const void* x_f16, int64_t M, int64_t K, int32_t group_size,
                               int8_t* x_q, float* x_scale, void* stream);
/* The same for fp16 or bf16 rows (x_dtype, a cider_dtype_t). */
cider_status_t cider_quant_act_dt(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                                  int32_t group_size, int8_t* x_q, float* x_scale, void* stream);

/* Weight quantization (the README runs it offline in numpy; here it is a
 * device kernel with the same rule, not part of the timed linear).
 *   w_f16   : fp16 [N, K] weights, row = output channel.
 *   bits    : 8 or 4. bits 4 requires group_size 0 and an even K.
 *   w_q     : bits 8: int8 [N, K] codes; bits 4: uint8 [N, K/2] packed nibbles.
 *   w_scale : fp32 [N] (group_size 0) or [N, K/group_size].
 */
cider_status_t cider_quant_weight(const void* w_f16, int64_t N, int64_t K, int32_t bits,
                                  int32_t group_size, void* w_q, float* w_scale, void* stream);
/* The same for fp16 or bf16 weights (w_dtype, a cider_dtype_t). */
cider_status_t cider_quant_weight_dt(const void* w, int32_t w_dtype, int64_t N, int64_t K, int32_t bits,
                                     int32_t group_size, void* w_q, float* w_scale, void* stream);

/* Weight quantization with percentile-clipped scales (the README's notes
 * section: scales by min-max by default, or by a percentile of the
 * magnitudes, clip_percentile=99.9). Per group (a row, or group_size
 * elements of it) the clip threshold t is the `percentile`-th percentile of
 * the magnitudes |w| by linear interpolation between order statistics:
 * h = (n-1) * (percentile/100), i = floor(h), j = min(i+1, n-1),
 * t = a_i + (h-i) * (a_j - a_i) over the ascending magnitudes a, each step
 * one rounded fp64 operation, then rounded to fp32 (percentile 100 gives
 * max|w|, i.e. cider_quant_weight). s = t / qmax; codes as for
 * cider_quant_weight, so magnitudes above t saturate at +-qmax; s == 0
 * gives codes 0. Outputs and layouts as cider_quant_weight.
 *   w_dtype    : CIDER_DTYPE_F16 or CIDER_DTYPE_BF16 (the weights' type).
 *   percentile : in [0, 100] (99.9 on the pages).
 * Sizes and errors as for cider_quant_weight; also N * (K/group_size) < 2^31.
 */
cider_status_t cider_quant_weight_clip(const void* w_f16, int32_t w_dtype, int64_t N, int64_t K,
                                       int32_t bits, int32_t group_size, double percentile, void* w_q,
                                       float* w_scale, void* stream);

/* W8A8 GEMM with fused dequant (pipeline step "matmul_fused_dequant"):
 *   y[m,n] = fp16( sum over groups of ((float)acc_g[m,n] * x_scale[m,g]) * w_scale[n,g] )
 *   acc_g[m,n] = sum_{k in group g} x_q[m,k] * w_q[n,k] (exact int32).
 *   x_q [M, K] int8, x_scale fp32 [M] or [M, K/gs]; w_q [N, K] int8,
 *   w_scale fp32 [N] or [N, K/gs]; y_f16 fp16 [M, N] (output).
 *   group_size must equal the one used to quantize both operands.
 */
cider_status_t cider_w8a8_gemm(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                               const float* w_scale, int64_t M, int64_t N, int64_t K,
                               int32_t group_size, void* y_f16, void* stream);
/* The same with the output type chosen by y_dtype (a cider_dtype_t):
 * bf16: y = bf16(((float)acc * x_scale[m]) * w_scale[n]) (per group: the
 * fp32 sum), i.e. the fp16 path's fp32 value rounded to bf16. */
cider_status_t cider_w8a8_gemm_dt(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K,
                                  int32_t group_size, void* y, int32_t y_dtype, void* stream);

/* W4A8 GEMM with fused dequant: the int4 weights are unpacked to int8 codes
 * (nibble - 8) inside the matmul's operand loads; per-channel scales only.
 *   w_packed uint8 [N, K/2] (K even), w_scale fp32 [N]; the rest as above.
 */
cider_status_t cider_w4a8_gemm(const int8_t* x_q, const float* x_scale, const uint8_t* w_packed,
                               const float* w_scale, int64_t M, int64_t N, int64_t K,
                               void* y_f16, void* stream);
/* Split-K for medium M with long K (too few output tiles to fill the GPU):
 * the _ex GEMMs take a caller workspace and, where the dispatch's plan says
 * so, cut K into ranges (whole 128-code stages) whose partial sums go to the
 * workspace as [splits][M][N] slabs before a second kernel adds them in
 * split order and stores y. Per-channel and W4A8 partials are exact int32
 * sums, so y is bit-identical to the unsplit GEMM; per-group partials are
 * the fp32 group sums of each range (without the per-token scale for
 * cider_w8a8_gemm_token_group), so only the fp32 summation order changes
 * (within the per-group error bound).
 *   cider_gemm_workspace_size: the bytes the plan needs at this shape, 0 when
 *   it does not split, -1 for invalid sizes. The library never allocates.
 *   workspace may be NULL (no split); otherwise 16-byte aligned with at
 *   least the queried bytes, else CIDER_ERROR_INVALID_VALUE. Its contents are
 *   scratch; calls that share one workspace must not overlap in time.
 * Everything else as for cider_w8a8_gemm_dt / cider_w4a8_gemm_dt. */
int64_t cider_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t bits, int32_t group_size);
cider_status_t cider_w8a8_gemm_ex(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K,
                                  int32_t group_size, void* y, int32_t y_dtype, void* workspace,
                                  int64_t workspace_bytes, void* stream);
cider_status_t cider_w4a8_gemm_ex(const int8_t* x_q, const float* x_scale, const uint8_t* w_packed,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                                  int32_t y_dtype, void* workspace, int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * GEMM as cider_w8a8_gemm_ex (per-channel or per-group, fp16 or bf16 y, the
 * same dispatch and the same bits), with the split-K scratch taken from a
 * library-owned device array of CIDER_NOALLOC_SCRATCH_BYTES instead of a
 * caller workspace. The call allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine); on a device's first call it looks up the
 * array's device address (hipGetSymbolAddress) and keeps it.
 *   - Every GPU that runs the library holds its own array until the process
 *     ends. All calls on one GPU share it, so calls that overlap in time on
 *     one GPU (different streams, or several host threads) race and must be
 *     serialized by the caller; calls in one stream's order are safe.
 *   - A shape whose split-K plan needs more than the array holds
 *     (cider_gemm_workspace_size(M, N, K, 8, group_size) >
 *     CIDER_NOALLOC_SCRATCH_BYTES) returns CIDER_ERROR_SCRATCH_LIMIT and
 *     enqueues nothing; every plan of the current dispatch needs at most
 *     42 MiB. Shapes that do not split use no scratch.
 * Arguments, sizes and other errors as for cider_w8a8_gemm_dt. */
#define CIDER_NOALLOC_SCRATCH_BYTES (48ll * 1024 * 1024)
cider_status_t cider_w8a8_gemm_noalloc(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                       const float* w_scale, int64_t M, int64_t N, int64_t K,
                                       int32_t group_size, void* y, int32_t y_dtype, void* stream);

/* The same with the output type chosen by y_dtype (a cider_dtype_t). */
cider_status_t cider_w4a8_gemm_dt(const int8_t* x_q, const float* x_scale, const uint8_t* w_packed,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                                  int32_t y_dtype, void* stream);

/* The whole linear layer in one call, fp16 x in and fp16 y out (the README's
 * perchannel_linear / w4a8_linear take fp16 activations): the activation
 * quantization of cider_quant_act followed by cider_w8a8_gemm (bits 8) or
 * cider_w4a8_gemm (bits 4), with identical results.
 *   w : bits 8: int8 [N, K] codes, w_scale fp32 [N] or [N, K/group_size];
 *       bits 4: packed uint8 [N, K/2], w_scale fp32 [N] (group_size 0).
 *   For group_size 0, M <= 2 and K a multiple of 16 (32 for bits 4), when
 *   the M activation rows' codes fit the GEMV kernel's 64 KiB staging area
 *   (M * ceil(K/256)*256 <= 65536), it is
 *   ONE kernel launch that quantizes the activations itself and needs no
 *   workspace. Otherwise the codes and
 *   scales go through `workspace` (device, 16-byte aligned, at least
 *   cider_linear_workspace_size(M, N, K, bits, group_size) bytes; its
 *   contents after the call are the activation codes [M, K] at offset 0 and
 *   the scales at the next 256-byte boundary, then the GEMM's split-K slabs
 *   when its shape uses them, see cider_gemm_workspace_size).
 * Sizes, alignment and errors as for cider_quant_act / cider_w8a8_gemm;
 * `workspace` may be NULL when the size query returns 0.
 */
int64_t cider_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t bits, int32_t group_size);
cider_status_t cider_linear(const void* x_f16, const void* w, const float* w_scale, int64_t M, int64_t N,
                            int64_t K, int32_t bits, int32_t group_size, void* workspace,
                            int64_t workspace_bytes, void* y_f16, void* stream);
/* The same for bf16 activations and a bf16 output (dtype a cider_dtype_t,
 * for both x and y): the codes are those of cider_quant_act_dt on the bf16
 * rows and y is the GEMMs' bf16 output (cider_w8a8_gemm_dt /
 * cider_w4a8_gemm_dt arithmetic); the one-launch rule and the workspace size
 * are unchanged. */
cider_status_t cider_linear_dt(const void* x, int32_t dtype, const void* w, const float* w_scale, int64_t M,
                               int64_t N, int64_t K, int32_t bits, int32_t group_size, void* workspace,
                               int64_t workspace_bytes, void* y, void* stream);

/* W8A8 GEMM with per-token activation scales and per-group weight scales
 * (the README's "量化" table quantizes activations per token in every mode,
 * while its "W8A8 量化粒度" table offers per-group weights):
 *   y[m,n] = fp16( x_scale[m] * sum_g (float)acc_g[m,n] * w_scale[n,g] ),
 *   acc_g as above. The group sum is accumulated in fp32 (one fma per group,
 *   in group order; for M <= 16 per-wave partial sums are then added in wave
 *   order), multiplied by x_scale[m] in fp32 and rounded to fp16. Its error
 *   is within (K/group_size + 17) * 2^-24 * x_scale[m] * sum_g |acc_g *
 *   w_scale[n,g]| plus the fp16 rounding; results are deterministic.
 *   x_q [M, K] int8 with x_scale fp32 [M] (cider_quant_act with group_size 0);
 *   w_q [N, K] int8 with w_scale fp32 [N, K/group_size]; group_size 64 or 128.
 * workspace / workspace_bytes: an optional split-K workspace as for
 * cider_w8a8_gemm_ex (size from cider_gemm_workspace_size(M, N, K, 8,
 * group_size); NULL: no split).
 * K, alignment and errors as for cider_w8a8_gemm.
 */
cider_status_t cider_w8a8_gemm_token_group(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                           const float* w_scale, int64_t M, int64_t N, int64_t K,
                                           int32_t group_size, void* y_f16, void* workspace,
                                           int64_t workspace_bytes, void* stream);
/* The same with the output type chosen by y_dtype (a cider_dtype_t): bf16
 * rounds the same fp32 value x_scale[m] * sum to bfloat16 (nearest, ties to
 * even) instead of fp16. */
cider_status_t cider_w8a8_gemm_token_group_dt(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                              const float* w_scale, int64_t M, int64_t N, int64_t K,
                                              int32_t group_size, void* y, int32_t y_dtype, void* workspace,
                                              int64_t workspace_bytes, void* stream);

/* Same-input projections as one GEMM (the README's experimental SplitLinear
 * page prepares the input of the Q/K/V and gate/up projections once): the
 * per-channel W8A8 GEMM of x_q against the row-concatenation of n_parts
 * weight matrices, each part's output columns written to its own matrix.
 *   w_q     : int8 [N, K] with N = sum(part_n), part i = rows
 *             [sum(part_n[<i]), sum(part_n[<=i])); w_scale fp32 [N].
 *   part_n  : HOST array of n_parts widths, each > 0 and a multiple of 16,
 *             1 <= n_parts <= CIDER_SPLIT_MAX_PARTS.
 *   y_parts : HOST array of n_parts DEVICE pointers, y_parts[i] fp16
 *             [M, part_n[i]] (output).
 * Every output equals the one cider_w8a8_gemm computes for that part alone,
 * bit for bit (per-channel dequant as above). x_q, x_scale, K and errors as
 * for cider_w8a8_gemm (group_size 0).
 */
#define CIDER_SPLIT_MAX_PARTS 4
cider_status_t cider_w8a8_gemm_split(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                     const float* w_scale, int64_t M, int64_t K, int32_t n_parts,
                                     const int64_t* part_n, void* const* y_parts, void* stream);
/* The same with the outputs' type chosen by y_dtype (a cider_dtype_t): bf16
 * parts hold what cider_w8a8_gemm_dt stores for each part alone. */
cider_status_t cider_w8a8_gemm_split_dt(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                        const float* w_scale, int64_t M, int64_t K, int32_t n_parts,
                                        const int64_t* part_n, void* const* y_parts, int32_t y_dtype,
                                        void* stream);

/* Decode matrix-vector product, the README's int8_mv (section "架构 / Metal
 * Kernel 流水线", Decode (M = 1): the activations are not quantized; the int8
 * weights are dequantized on the fly; the file list names a per-channel and a
 * per-group MV kernel):
 *   y[m,n] = fp16( sum_k x[m,k] * w_q[n,k] * w_scale[n, g(k)] ),
 *   g(k) = k / group_size (group_size 0: one scale per row, w_scale[n]).
 *   x_f16   : fp16 [M, K] activations, 0 <= M <= CIDER_MV_MAX_M.
 *   w_q     : int8 [N, K] weight codes (as cider_quant_weight makes them).
 *   w_scale : fp32 [N] (group_size 0) or [N, K/group_size].
 *   y_f16   : fp16 [M, N] (output).
 * The sum is accumulated in fp32 (each fp16 x int8 product is exact in fp32);
 * its order is fixed, so results are deterministic, and its error is within
 * the fp32 summation bound (K/32 + 24) * 2^-24 * sum_k |x*w_q*w_scale|. The
 * per-channel scale multiplies the fp32 sum (fp32 product, then fp16).
 * K, group_size, alignment and errors as for cider_w8a8_gemm.
 */
#define CIDER_MV_MAX_M 4
cider_status_t cider_int8_mv(const void* x_f16, const int8_t* w_q, const float* w_scale, int64_t M,
                             int64_t N, int64_t K, int32_t group_size, void* y_f16, void* stream);

/* Test hook: the same matmul main loops with an int32 store instead of the
 * dequant, so the accumulators can be compared bit-exactly.
 *   mode 0: w = int8 [N, K] codes; mode 1: w = packed int4 [N, K/2] (group_size 0).
 *   acc: int32 [M, N] for group_size 0, else [K/group_size, M, N] (one slab per group).
 */
cider_status_t cider_gemm_acc_i32(int32_t mode, const int8_t* x_q, const void* w, int64_t M,
                                  int64_t N, int64_t K, int32_t group_size, int32_t* acc,
                                  void* stream);

/* Measurement helper (not part of the method): reads `bytes` (a multiple of
 * 16) of the device buffer `buf` once, in one launch, the way a pure weight
 * stream would (16-byte loads, contiguous per workgroup). Its duration on a
 * buffer that is not cache resident is the single-launch HBM read ceiling
 * the bandwidth-bound small-M kernels are held against. `sink` (device,
 * 16-byte aligned, 4 bytes) is written only for an impossible data pattern.
 * Errors as for the other calls. */
cider_status_t cider_read_probe(const void* buf, int64_t bytes, int32_t* sink, void* stream);

/* ---- Linear-stack driver ----------------------------------------------------
 * The prefill linear layers of a decoder stack shaped like the Qwen3-VL-2B
 * model of the README's end-to-end VLM section, chained so that each layer's
 * inputs are produced by the previous GEMM. Per layer, with per-channel W8A8:
 *   quant(h)    -> Q = h Wq^T, K = h Wk^T, V = h Wv^T   (one shared quant; the
 *                  README's experimental SplitLinear page shares the input
 *                  preparation of same-input projections the same way)
 *   quant(Q)    -> O = Q Wo^T
 *   quant(O)    -> G = O Wg^T, U = O Wu^T               (one shared quant)
 *   quant(U)    -> h' = U Wd^T                          (the next layer's input)
 * i.e. 4 activation quantizations and 7 GEMMs per layer. When a layer's q, k
 * and v codes are adjacent in memory in that order (w[1] == w[0] +
 * q_dim*hidden, w[2] == w[1] + kv_dim*hidden) and so are their scales, the
 * three run as one GEMM over the concatenated rows (cider_w8a8_gemm_split);
 * likewise gate and up. The results are bit-identical either way. K, V and G are
 * computed and kept in the workspace but not consumed (there is no attention
 * or activation function: this is the linear-layer work of the stack only).
 * Shapes: Wq [q_dim, hidden], Wk/Wv [kv_dim, hidden], Wo [hidden, q_dim],
 * Wg/Wu [mlp_dim, hidden], Wd [hidden, mlp_dim]; all dims multiples of 16.
 */
typedef struct {
  const int8_t* w[7]; /* int8 codes, order q, k, v, o, gate, up, down (device) */
  const float* s[7];  /* per-output-channel fp32 scales, same order (device) */
} cider_stack_layer_t;

/* Workspace regions, in this order, each starting at a 256-byte aligned
 * offset: 0 codes int8 [M, max(hidden, q_dim, mlp_dim)], 1 scales fp32 [M],
 * 2 Q fp16 [M, q_dim], 3 K fp16 [M, kv_dim], 4 V fp16 [M, kv_dim],
 * 5 O fp16 [M, hidden], 6 G fp16 [M, mlp_dim], 7 U fp16 [M, mlp_dim],
 * 8 h fp16 [M, hidden] (layer output ping buffer), then a region not listed
 * in `offsets`: the int32 partial sums of the per-projection GEMMs whose K is
 * split (as cider_gemm_workspace_size plans it; e.g. the down projection at
 * M = 1024, mlp_dim = 6144), sized for the largest of them (may be empty).
 * Writes the 9 byte offsets into `offsets` (may be NULL) and returns the total
 * size in bytes (0 for invalid dims). Host-only, no HIP call. */
int64_t cider_stack_workspace_layout(int64_t M, int64_t hidden, int64_t q_dim, int64_t kv_dim,
                                     int64_t mlp_dim, int64_t* offsets);

/* Runs n_layers layers on x_f16 [M, hidden]; the last layer's output goes to
 * y_f16 [M, hidden]. `layers` is a HOST array of n_layers descriptors holding
 * device pointers. `workspace` is a device buffer of at least
 * cider_stack_workspace_layout(...) bytes; after the call its regions hold the
 * last layer's intermediates. All work is enqueued on `stream`. */
cider_status_t cider_stack_forward(const void* x_f16, int64_t M, int64_t hidden, int64_t q_dim,
                                   int64_t kv_dim, int64_t mlp_dim, int32_t n_layers,
                                   const cider_stack_layer_t* layers, void* workspace,
                                   int64_t workspace_bytes, void* y_f16, void* stream);
/* The same chain in bf16 (dtype a cider_dtype_t): x, every intermediate
 * region and y hold bfloat16; each quantization reads bf16 rows
 * (cider_quant_act_dt) and each GEMM stores bf16 (cider_w8a8_gemm_dt
 * arithmetic). The workspace layout is the same (2 bytes per element). */
cider_status_t cider_stack_forward_dt(const void* x, int32_t dtype, int64_t M, int64_t hidden, int64_t q_dim,
                                      int64_t kv_dim, int64_t mlp_dim, int32_t n_layers,
                                      const cider_stack_layer_t* layers, void* workspace,
                                      int64_t workspace_bytes, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CIDER_H */
