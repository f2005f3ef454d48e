/*
 * mnb.h -- C ABI of libmnb: block-wise int4 weight-only matmul in the ONNX
 * MatMulNBits layout, on AMD MI355X (gfx950).
 *
 *   Y[M,N] = A[M,K] . dequant(B)^T,
 *   dequant(B)[n,k] = (code[n,k] - zp[n, k/group]) * scale[n, k/group]
 *
 * The operation and the input format are those of the module doc of
 * onnx-runtime-ep-cuda 0.1.0-dev.6, src/kernels/marlin_gemm.rs, section
 * "ONNX MatMulNBits int4 format (input to the repack)":
 *   packed       u8 [N, k_blocks, group/2]; the nibble of (n,k) is in byte
 *                (n*k_blocks + k/group)*(group/2) + (k%group)/2, low nibble
 *                for even k, high nibble for odd k; code in 0..15.
 *   scales       [N, k_blocks], fp16 or fp32 (a flat [N*k_blocks] array has
 *                the same memory).
 *   zero_points  optional u8 [N, ceil(k_blocks/2)]; the nibble of (n,block) is
 *                in byte n*ceil(k_blocks/2) + block/2, low nibble for even
 *                block.  When absent every zero point is 8.
 * with k_blocks = ceil(K/group).  onnx-runtime-ep-cuda 0.1.0-dev.3,
 * src/kernels/matmul_nbits.rs (MatMulNBitsFactory::create, run, run_f16)
 * fixes the operand dtypes: A is fp16 or fp32, Y has A's dtype, scales are
 * fp16 or fp32 independently of A, bits = 4 only.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named "device" are HIP device pointers (any allocation visible
 *   to the current device); descriptors are host pointers.  Device buffers
 *   must be 16-byte aligned, except y, which needs element alignment.  All
 *   arrays are dense and row-major.
 * - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *   Every call only enqueues work on `stream` and returns; it never
 *   allocates, frees, synchronises, or copies between host and device, and
 *   its grid depends on the shapes only, so a call can be recorded into a
 *   HIP graph (the capture-safety convention of the MatMulNBits kernels on
 *   the onnx-runtime-ep-cuda pages: static grid, no per-call allocation).
 * - The caller owns every buffer.  A repacked buffer is immutable once the
 *   repack that wrote it has completed; calls that read it may overlap.
 * - All arguments are validated on the host before any HIP call.  A failing
 *   check returns an error status and enqueues nothing; mnb_last_error()
 *   then gives the reason ("mnb: ..."), in the calling thread.
 *   MNB_ERR_INVALID_ARGUMENT: a malformed request (null pointer, bad size or
 *     enum, misalignment, workspace too small, size overflow).
 *   MNB_ERR_UNSUPPORTED: a valid MatMulNBits request this library does not
 *     implement (K not a multiple of group, group outside 16/32/64/128, a
 *     dtype pairing other than the ones below, a K beyond the limit a call
 *     documents).  The library never computes
 *     something else instead (the "Unsupported" convention of ferrox-cuda
 *     gpu.rs, enum CudaError), and never falls back internally.
 *   MNB_ERR_DEVICE: no usable gfx950 device, or the launch failed.
 * - m == 0 or n == 0 is a no-op returning MNB_OK.
 * - Offsets are computed in 64-bit; sizes whose byte counts overflow are
 *   rejected.
 *
 * Repacked layout (written by mnb_repack, read by every other call)
 * -----------------------------------------------------------------
 * A permutation of the ONNX nibbles plus a re-indexing of scales and zero
 * points (no expansion: the same bytes plus padding to whole tiles).  Let
 *   T = ceil(N/16)   column tiles of 16 columns,
 *   C = ceil(K/128)  k-chunks of 128 k,
 *   Q = 128/group    groups per k-chunk (8, 4, 2 or 1),
 *   ss = 2 (fp16 scales) or 4 (fp32 scales),
 *   align(x) = x rounded up to a multiple of 256.
 * Section CODES, offset 0, T*C*1024 bytes.  Chunk (t,c) is the 1024 bytes at
 *   ((t*C) + c) * 1024.  Inside it, lane L in 0..63 owns bytes
 *   [16L, 16L+16) = four little-endian 32-bit words D_j, j = 0..3.  D_j holds
 *   column n = 16t + (L mod 16) and the 8 values k = 128c + 32j + 8*(L div 16)
 *   + i, i = 0..7; the code of offset i is the nibble at bits [4p, 4p+4) with
 *   p = (0,4,1,5,2,6,3,7)[i] (nibble slots 0..7 hold i = 0,2,4,6,1,3,5,7).
 *   Columns n >= N and k >= K hold code 0.
 * Section SCALES, offset S0 = align(T*C*1024), T*C*16*Q scale values of the
 *   scale dtype.  Chunk (t,c) owns elements [((t*C)+c)*16Q, +16Q).  The scale
 *   of column i = n mod 16 and in-chunk group q = (k mod 128)/group sits at
 *   slot s(i,q) = i*Q + q when Q <= 4, and s(i,q) = ((q mod 2)*16 + i)*4 +
 *   q div 2 when Q = 8.  Columns n >= N and groups >= K/group hold 0.
 * Section ZERO_POINTS, present iff has_zero_points, offset
 *   Z0 = align(S0 + T*C*16*Q*ss), T*C*8*Q bytes.  Chunk (t,c) owns bytes
 *   [((t*C)+c)*8Q, +8Q); the zero point of slot s is the nibble of byte s/2,
 *   low nibble for even s.  Padding holds 0.
 * Section RANGE_FLAGS, offset F0 = align(end of the last section above), T
 *   bytes: byte t is 1 when tile t's scales are in the range class of the
 *   prefill GEMM's single rescaled accumulator, else 0.  The class: every
 *   scale of the tile's columns that is neither zero nor NaN has magnitude
 *   in [2^-100, 2^100], and in each column the largest such magnitude is at
 *   most 2^64 times the smallest (finite fp16 scales always qualify).  The
 *   prefill GEMM computes a workgroup with a tile outside the class by a
 *   slower path with a fresh partial per group; results meet the same bound
 *   either way.
 * Total size mnb_repacked_bytes() = align(F0 + T).
 * The 16-lane x 8-k ownership is the B-operand distribution of the gfx950
 * v_mfma_f32_16x16x32_f16 instruction, so the same bytes feed the decode
 * GEMVs (one 128-bit load per lane per chunk) and the MFMA GEMMs.
 */
#ifndef MNB_H
#define MNB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MNB_OK = 0,
    MNB_ERR_INVALID_ARGUMENT = 1,
    MNB_ERR_UNSUPPORTED = 2,
    MNB_ERR_DEVICE = 3
} mnb_status;

typedef enum { MNB_F32 = 0, MNB_F16 = 1 } mnb_dtype;

/* One quantized weight B[N,K].  group_size in {16,32,64,128} and K % group
 * == 0 (the GEMM tiles of marlin_gemm.rs demand the same); scale_dtype is an
 * mnb_dtype; has_zero_points is 0 or 1. */
typedef struct {
    int64_t n;
    int64_t k;
    int32_t group_size;
    int32_t has_zero_points;
    int32_t scale_dtype;
    int32_t reserved; /* must be 0 */
} mnb_weight_desc;

/* Byte offsets of the repacked sections (see "Repacked layout"). */
typedef struct {
    int64_t tiles, chunks, groups_per_chunk;
    int64_t codes_offset, codes_bytes;
    int64_t scales_offset, scales_bytes;
    int64_t zero_points_offset, zero_points_bytes; /* 0, 0 without zero points */
    int64_t range_flags_offset, range_flags_bytes;
    int64_t total_bytes;
} mnb_layout;

/* Size in bytes of the repacked buffer for `w`; 0 if `w` is invalid or
 * unsupported (mnb_last_error() says why).  Host only, no HIP call.  The
 * size-query convention of marlin_gemm.rs, fn repacked_bytes. */
size_t mnb_repacked_bytes(const mnb_weight_desc* w);

/* Section offsets of the repacked buffer for `w` into *out.  Host only. */
mnb_status mnb_repacked_layout(const mnb_weight_desc* w, mnb_layout* out);

/* Offline repack (the weight reordering of marlin_gemm.rs, fn
 * repack_int4_weights and kernel matmul_nbits_marlin_repack, re-targeted to
 * the layout above).  Reads the ONNX operands from device memory:
 *   packed       u8 [N, k_blocks, group/2]
 *   scales       [N, k_blocks] in w->scale_dtype
 *   zero_points  u8 [N, ceil(k_blocks/2)]; must be NULL iff
 *                !w->has_zero_points
 * and writes every byte of `repacked` (device, mnb_repacked_bytes(w) bytes,
 * 256-byte aligned), padding included.  Asynchronous on `stream`. */
mnb_status mnb_repack(const mnb_weight_desc* w, const uint8_t* packed, const void* scales,
                      const uint8_t* zero_points, void* repacked, void* stream);

/* Decode GEMV, M = 1 (the f32 GEMV and the fp16 GEMVs of matmul_nbits.rs):
 *   y[n] = sum_k a[k] * dequant(B)[n,k]   for n < N,
 * with a (device, [K]) and y (device, [N]) both of a_dtype (MNB_F16 or
 * MNB_F32).  Products accumulate in fp32; fp16 outputs are rounded once
 * (round to nearest even).  The activation is staged on chip: K <= 31744
 * for fp16 activations, K <= 15872 for fp32 (else MNB_ERR_UNSUPPORTED). */
mnb_status mnb_gemv(const mnb_weight_desc* w, const void* repacked, const void* a,
                    int32_t a_dtype, void* y, void* stream);

/* Fused gate/up projection + SwiGLU, M = 1 (kernel
 * matmul_nbits_gemv_f16_gate_up_swiglu of matmul_nbits.rs):
 *   y[n] = silu(g[n]) * u[n],  g = a . dequant(B_gate)^T,
 *   u = a . dequant(B_up)^T,   silu(x) = x / (1 + e^-x).
 * Gate and up share the descriptor `w` (same N, K, group, dtypes).  a is
 * [K], y is [N], both of a_dtype; g and u are kept in fp32 (not rounded)
 * before the activation. */
mnb_status mnb_gemv_gate_up_swiglu(const mnb_weight_desc* w, const void* gate_repacked,
                                   const void* up_repacked, const void* a, int32_t a_dtype,
                                   void* y, void* stream);

/* Workspace in bytes that mnb_gemm needs for (w, m) with fp16 activations;
 * 0 when none.  Host only.  Like splitk_partials_len of marlin_gemm.rs. */
size_t mnb_gemm_workspace_bytes(const mnb_weight_desc* w, int64_t m);

/* The same for activations of a_dtype (MNB_F16 or MNB_F32): fp32
 * activations with M > 1 need 4*M*K bytes plus the row scales (see
 * mnb_gemm).  0 on an invalid argument (mnb_last_error() says why). */
size_t mnb_gemm_workspace_bytes_for(const mnb_weight_desc* w, int64_t m, int32_t a_dtype);

/* GEMM for any M >= 1 (marlin_gemm.rs, kernels matmul_nbits_marlin_gemm_f16
 * and its split-K form, re-designed for gfx950):
 *   Y[m,n] = sum_k A[m,k] * dequant(B)[n,k],
 * A (device, [M,K]) and Y (device, [M,N]) of a_dtype.  M = 1 runs the decode
 * GEMV (its K limit applies); 2 <= M <= 16 a weight-streaming MFMA kernel
 * whose workgroups split K among their waves and reduce in a fixed order,
 * for K <= 33554432 (its 32-bit buffer ranges; else MNB_ERR_UNSUPPORTED),
 * and the same kernel up to 48 fp16 rows (M with fp16 A), once per slice
 * of at most 16 rows;
 * larger M the MFMA prefill GEMM, for K <= 16777088 (its 32-bit buffer
 * offsets; else MNB_ERR_UNSUPPORTED).  Products are fp16 x fp16 on the
 * matrix cores with fp32 accumulation; each group's partial sum is
 * multiplied by its scale after that group's accumulation.  fp32 A with
 * M > 1 (the fp32 operator of matmul_nbits.rs, MatMulNBitsKernel::run, at
 * any M): each row m is scaled by a power of two 2^-e_m that puts its largest
 * finite magnitude in [2^14, 2^15) and written as two fp16 rows, hi =
 * fp16(a 2^-e_m) and lo = fp16(a 2^-e_m - hi); the fp16 GEMM runs on the 2M
 * rows (the small-M kernel for 2M <= 48, in slices of 8 rows of A, else
 * the prefill kernel, whose K limit then applies) and y[m,n] = 2^e_m * (acc[2m,n] + acc[2m+1,n]) in fp32.
 * The split errs by at most 2^-22 |a| + 2^-39 max|a| per element; NaN and
 * infinities pass whole.  `workspace` (device) must hold
 * mnb_gemm_workspace_bytes_for(w, m, a_dtype) bytes: none for fp16 (it may be
 * NULL), and for fp32 with M > 1 the row scales (fp32 [M]) at offset 0 and the
 * row pairs (fp16 [2M, K]) at the next 256-byte boundary (256-byte aligned).
 * Results are deterministic. */
mnb_status mnb_gemm(const mnb_weight_desc* w, const void* repacked, const void* a, int64_t m,
                    int32_t a_dtype, void* y, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Bias epilogue conventions (onnx-runtime-ep-cuda 0.1.0-dev.3,
 * src/kernels/matmul_nbits.rs, the fp16 GEMV bias epilogue fold_bias_f16 and
 * its dispatch records; marlin_gemm.rs (dev.6), fold_bias with a per-row
 * bias stride). */
typedef enum {
    /* the operator's own bias: acc + b in fp32, rounded once, fp16(acc + b) */
    MNB_BIAS_FUSED = 0,
    /* a folded elementwise Add: the accumulator rounded to fp16 first, then
     * + b in fp32 and rounded again, fp16(fp16(acc) + b); byte-identical to
     * the GEMM's output followed by a separate fp16 add */
    MNB_BIAS_AFTER_ROUND = 1
} mnb_bias_mode;

/* mnb_gemm followed by a bias, in one pass (any M >= 1, every path):
 *   y[m,n] = epilogue(acc[m,n], bias[m*bias_row_stride + n]),
 * acc the fp32 result of mnb_gemm before its output rounding.  bias (device,
 * a_dtype, element-aligned) holds (M-1)*bias_row_stride + N elements:
 * bias_row_stride = 0 adds one [N] vector to every row, N (or more) adds a
 * per-row residual [M, stride].  bias_mode is an mnb_bias_mode; for fp32
 * outputs (fp32 activations) both modes are acc + b in fp32.
 * bias = NULL is mnb_gemm.  Every other argument, the workspace and the
 * error behaviour are as for mnb_gemm; a negative stride or an unknown mode
 * is MNB_ERR_INVALID_ARGUMENT. */
mnb_status mnb_gemm_bias(const mnb_weight_desc* w, const void* repacked, const void* a, int64_t m,
                         int32_t a_dtype, const void* bias, int64_t bias_row_stride,
                         int32_t bias_mode, void* y, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Act-order weights: the optional group-index input g_idx of MatMulNBits
 * (onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs, the
 * g_idx checks of MatMulNBitsFactory and the dequant kernel with
 * group_indices): int32 [K], the code at k keeps its place in the ONNX
 * layout and takes the scale and zero point of group g_idx[k]:
 *   dequant(B)[n,k] = (code[n,k] - zp[n, g_idx[k]]) * scale[n, g_idx[k]].
 * The repack sorts k by group, so every group becomes contiguous, and the
 * GEMM takes A's columns in the same order; the product is the same sum over
 * k in another order.  Three steps, and a fourth for any g_idx:
 *
 * 1. mnb_act_order_permutation (host only, host pointers, no HIP call):
 *    checks g_idx (every value in 0..k_blocks-1, else
 *    MNB_ERR_INVALID_ARGUMENT; every group with exactly group_size members,
 *    else MNB_ERR_UNSUPPORTED, and step 4 below serves that g_idx) and
 *    writes perm [K]: the positions of group 0 in increasing k, then those
 *    of group 1, and so on; perm is written only on MNB_OK. */
mnb_status mnb_act_order_permutation(const mnb_weight_desc* w, const int32_t* g_idx, int32_t* perm);

/* 2. mnb_repack_act_order: mnb_repack of the same ONNX operands with the
 *    codes taken in perm order (perm: device int32 [K], from step 1; a
 *    buffer repacked this way serves only mnb_gemm_act_order with the same
 *    perm).  Arguments and errors as mnb_repack.  Indices outside 0..K-1 in
 *    perm give wrong codes, never an out-of-range read. */
mnb_status mnb_repack_act_order(const mnb_weight_desc* w, const uint8_t* packed, const void* scales,
                                const uint8_t* zero_points, const int32_t* perm, void* repacked,
                                void* stream);

/* 3. mnb_gemm_act_order: mnb_gemm on an act-order repacked buffer, any
 *    M >= 1.  perm: device int32 [K], the one used by the repack.  The
 *    workspace (device, 256-byte aligned) holds A with its columns in perm
 *    order, then mnb_gemm's own workspace:
 *    mnb_gemm_act_order_workspace_bytes(w, m, a_dtype) bytes.  At M = 1
 *    with a 16-byte aligned perm and K <= 15872 (fp16 activations) or
 *    K <= 7936 (fp32) the GEMV reorders A itself while staging it and the
 *    workspace goes unused (its size is still checked); both routes give the
 *    same bits.  Indices outside 0..K-1 in perm give wrong results, never an
 *    out-of-range read.  Other arguments, dtypes and errors as mnb_gemm. */
size_t mnb_gemm_act_order_workspace_bytes(const mnb_weight_desc* w, int64_t m, int32_t a_dtype);
mnb_status mnb_gemm_act_order(const mnb_weight_desc* w, const void* repacked, const void* a, int64_t m,
                              int32_t a_dtype, const int32_t* perm, void* y, void* workspace,
                              size_t workspace_bytes, void* stream);

/* 4. Any g_idx, groups of any size: the general route of the fp32
 *    operator (matmul_nbits.rs, MatMulNBitsKernel::run with group_indices:
 *    the dequant kernel with group_indices, then the dense GEMM with its
 *    bias), for a g_idx that mnb_act_order_permutation answers with
 *    MNB_ERR_UNSUPPORTED, or any other:
 *      Y[m,n] = epilogue(sum_k A[m,k] * (code[n,k] - zp[n,G]) * scale[n,G]),
 *    G = g_idx[k], the sum in fp32 over k in increasing order, each weight
 *    (code - zp) * scale formed in fp32 (exact for fp16 scales).  repacked:
 *    the plain mnb_repack buffer (codes at their ONNX positions).  g_idx:
 *    device int32 [K], 16-byte aligned; a value outside 0..k_blocks-1 gives
 *    the weight 0 at that k, as the dequant kernel does (the operator
 *    rejects such a g_idx on the host beforehand;
 *    mnb_act_order_permutation makes that check, MNB_ERR_INVALID_ARGUMENT).
 *    A (device, [M,K], 16-byte aligned) and Y (device, [M,N], element-
 *    aligned) of a_dtype; bias, bias_row_stride and bias_mode as for
 *    mnb_gemm_bias (bias NULL for none).  Any M >= 1 up to 65535*64 (else
 *    MNB_ERR_UNSUPPORTED), no workspace, K below 2^31 - 128.  The weight is
 *    streamed once per block of up to 16 rows (M <= 16) or 64 rows, each
 *    weight dequantized in registers from a per-tile table of (zero point,
 *    scale) pairs; products by fp32 fma at M = 1, else on the fp32 matrix
 *    cores (v_mfma_f32_16x16x4_f32).  Deterministic. */
mnb_status mnb_gemm_group_indices(const mnb_weight_desc* w, const void* repacked, const void* a, int64_t m,
                                  int32_t a_dtype, const int32_t* g_idx, const void* bias,
                                  int64_t bias_row_stride, int32_t bias_mode, void* y, void* stream);

/* int8 activations: accuracy_level = 4 of the fp32 operator
 * (onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs, kernels
 * matmul_nbits_accuracy4, matmul_nbits_quantize_accuracy4_block32 and
 * matmul_nbits_gemv_accuracy4_block32).  A is fp32 [M, K] (16-byte aligned),
 * Y fp32 [M, N]; the weight is any repacked buffer (fp16 or fp32 scales, with
 * or without zero points).  Each row of A is quantized with one binary32
 * scale s = max|a| / 127 (NaN skipped): q = round(clamp(a * (1/s), -127,
 * 127)), halves away from zero, in binary32 steps; then
 *   Y[m,n] = s[m] * sum_b scale[n,b] * sum_{k in b} q[m,k] * (code[n,k] - zp[n,b])
 *            (+ bias[n]),
 * the inner sums exact integers; a row with s = 0 gives bias[n] (or 0).
 * bias: fp32 [N] or NULL.
 *
 * Workspace (device, 256-byte aligned), mnb_gemm_accuracy4_workspace_bytes(w,
 * m) bytes: it receives the scales s (fp32 [M]) at offset 0 and the codes q
 * (as fp16 integers, [M, K] row-major) at the next 256-byte boundary; the rest
 * is the library's.  Required for M > 1; optional for M = 1 (NULL: the codes
 * stay on chip).  M = 1 needs K <= 32768 (else MNB_ERR_UNSUPPORTED).  Errors
 * otherwise as mnb_gemm. */
size_t mnb_gemm_accuracy4_workspace_bytes(const mnb_weight_desc* w, int64_t m);
mnb_status mnb_gemm_accuracy4(const mnb_weight_desc* w, const void* repacked, const float* a, int64_t m,
                              const float* bias, float* y, void* workspace, size_t workspace_bytes,
                              void* stream);

/* mnb_gemm_accuracy4 without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (less the workspace),
 * same kernels, same results.  For M > 1 the int8 codes and row scales go to
 * a scratch array the library keeps in device memory,
 * MNB_NOALLOC_SCRATCH_BYTES per device, held until the process ends; its
 * device address is looked up on the first call on each device (that call
 * must have the device current, as every call does).  A request whose
 * workspace (mnb_gemm_accuracy4_workspace_bytes) exceeds the array returns
 * MNB_ERR_UNSUPPORTED before any HIP call.  No call allocates or frees
 * memory.  All calls on one device share the array and each leaves its
 * contents behind: calls that overlap on one device (other streams or
 * threads) race and give wrong results; calls on different devices do not
 * interact. */
#define MNB_NOALLOC_SCRATCH_BYTES (32u << 20)
mnb_status mnb_gemm_accuracy4_noalloc(const mnb_weight_desc* w, const void* repacked, const float* a,
                                      int64_t m, const float* bias, float* y, void* stream);

/* Test-only: decode a repacked buffer with the production unpack code.
 * codes: device u8 [N,K] (the stored nibbles); w_f32: device f32 [N,K], the
 * dequantized weights (code - zp) * scale rounded once to fp32.  Either
 * output may be NULL. */
mnb_status mnb_unpack_debug(const mnb_weight_desc* w, const void* repacked, uint8_t* codes,
                            float* w_f32, void* stream);

/* Test-only: the tile height of the prefill GEMM (M > 16) for groups of
 * 128 or 64 k.  rows = 0 (the default): chosen per call from the shape and
 * the device's compute units; 64, 96 or 128: that height for every later
 * call in the process, from any thread (128 only for groups of 128 k; a
 * height the group size does not offer leaves its default).  Returns the
 * previous setting; any other value changes nothing and returns -1.  All
 * heights give bit-identical results; this lets tests run each form at any
 * size. */
int32_t mnb_debug_prefill_rows(int32_t rows);

/* Static string naming a status. */
const char* mnb_status_string(int32_t status);

/* Reason for the last non-OK status returned in this thread ("" if none). */
const char* mnb_last_error(void);

/* Name of the kernel variant the last successful call in this thread
 * enqueued (the dispatch record of matmul_nbits.rs, record_kernel_variant),
 * e.g. "gemv_f16" or "gemm_small_m"; "" if none. */
const char* mnb_last_variant(void);

#ifdef __cplusplus
}
#endif

#endif /* MNB_H */
