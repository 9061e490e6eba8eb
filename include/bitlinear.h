/*
 * bitlinear.h -- C ABI of libbitlinear, the BitLinear W1.58A8 forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * The pass (page "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs"):
 *   1. absmean ternary weight quantization -- section "Ternary Weight
 *      Quantization: absmean Scaling": gamma = mean |W| over the whole tensor,
 *      W~ = Clip(Round(W / (gamma + eps)), -1, 1);
 *   2. per-token absmax int8 activation quantization -- section "8-Bit
 *      Activation Quantization: absmax Scaling": s = 127 / max|x|,
 *      x~ = Clip(Round(x * s), -128, 127);
 *   3. the integer product x~ W~^T with an integer accumulator and
 *   4. the rescale by beta*gamma/127 = gamma/s -- section "Matrix
 *      Multiplication as Pure Integer Addition".
 * Weights are stored two bits each (winbuzzer.com, "Microsoft Releases
 * BitNet b1.58 2B4T", section "The Catch": GPU kernels pack and unpack the
 * weights); the up projection of the FFN is followed by ReLU^2 (same page,
 * section "Under the Hood: The BitNet Approach"), offered here as a fused
 * epilogue.
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers on the current HIP device, owned
 *     by the caller; the library allocates nothing and frees nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work and return; results are ready when the stream
 *     is synchronised.  No entry point synchronises or copies to the host.
 *   - Arguments are checked on the host before any launch.  On a non-BL_OK
 *     return nothing has been enqueued, except BL_ERR_HIP, which reports an
 *     error from the HIP runtime when a kernel was launched.  Faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - Inputs must be finite.  Outputs for NaN/Inf inputs are unspecified.
 *   - Matrices are row-major and dense.  Shapes follow W in R^{N x K}
 *     (N = d_out, K = d_in) and x in R^{M x K} (M = tokens).
 *   - Sizes are int64_t.  1 <= N, K;  K <= BL_MAX_K;  0 <= M.
 */
#ifndef BITLINEAR_H_
#define BITLINEAR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_ABI_VERSION 4

/* Largest K: the kernels accumulate 64 * x~ * W~ in int32, so
 * 64 * 127 * K must stay below 2^31. */
#define BL_MAX_K 262144
/* Largest M and N accepted (grid and index limits). */
#define BL_MAX_MN 16777216

typedef enum {
  BL_OK = 0,
  BL_ERR_INVALID_ARG = 1,       /* null pointer, size < allowed minimum, bad enum, bad eps */
  BL_ERR_UNSUPPORTED_SHAPE = 2, /* size above BL_MAX_K or BL_MAX_MN, or a matrix-core
                                   GEMM of more than 2^31 - 1 output tiles */
  BL_ERR_MISALIGNED = 3,        /* pointer below its documented alignment */
  BL_ERR_WORKSPACE = 4,         /* workspace pointer NULL or smaller than required */
  BL_ERR_HIP = 5                /* the HIP runtime reported an error at launch */
} bl_status;

typedef enum { BL_F32 = 0, BL_BF16 = 1 } bl_dtype;
typedef enum { BL_EPI_NONE = 0, BL_EPI_RELU2 = 1 } bl_epilogue;

/* ------------------------------------------------------------------------
 * Packed ternary weight layout (version 1)
 *
 *   N_pad = 64 * ceil(N / 64)     (row blocks of 64 output rows)
 *   K_pad = 256 * ceil(K / 256)   (super-chunks of 256 inputs), NC = K_pad/256
 *   buffer = N_pad * K_pad / 4 bytes = array of little-endian uint32 words.
 *
 *   Weight (n, k): b = n / 64, r = n % 64, c = k / 256, and
 *   k % 256 = 64*j + 16*q + t  (j, q in 0..3, t in 0..15).  Its code is in
 *       word  (((b*NC + c)*4 + q)*64 + r)*4 + j
 *       bits  [8*(t%4) + 2*(t/4), +2)
 *   as a 2-bit two's complement number: 0 -> 00, +1 -> 01, -1 -> 11 (10 is
 *   never written).  Rows n >= N and columns k >= K hold code 0.
 *
 *   So each 4 KiB block (b, c) holds 64 rows x 256 inputs; inside it, byte
 *   offset q*1024 + r*16 + 4*j.  Shifting a word left by 6-2i and masking
 *   with 0xC0C0C0C0 yields four int8 values 64*W~ for t = 4i..4i+3 in byte
 *   order, i.e. for consecutive inputs k.
 * ---------------------------------------------------------------------- */

/* Size queries return 0 for sizes the entry points refuse (n or m outside
 * 1..BL_MAX_MN, k outside 1..BL_MAX_K). */
/* Row count rounded up to 64. */
int64_t bitlinear_padded_n(int64_t n);
/* Input count rounded up to 256; also the row stride (bytes) of x~. */
int64_t bitlinear_padded_k(int64_t k);
/* Bytes of the packed weight buffer for an N x K matrix. */
size_t bitlinear_packed_bytes(int64_t n, int64_t k);
/* Bytes of the quantized activation buffer x~: m * padded_k(k). */
size_t bitlinear_xq_bytes(int64_t m, int64_t k);

/* ------------------------------------------------------------------------
 * bitlinear_pack_weights -- absmean ternarization and 2-bit packing.
 * Defines: "Ternary Weight Quantization: absmean Scaling" (both equations).
 *
 *   w          [n][k] fp32 (w_dtype = BL_F32) or bf16 (BL_BF16), 16-byte aligned.
 *   eps        >= 0 and finite; the pages use 1e-5.
 *   gamma_in   NULL: gamma = mean|w| is computed on the device (fp64
 *              partial sums in a fixed order, rounded once to fp32; the
 *              result does not depend on the launch or the run).
 *              non-NULL: one fp32 on the device, used as gamma as is (for a
 *              tensor split across devices, or to re-pack with a known
 *              gamma); the workspace is then not touched.
 *   packed     out, bitlinear_packed_bytes(n, k) bytes, 256-byte aligned.
 *   gamma_out  out, one fp32 on the device (may equal gamma_in).
 *   workspace  bitlinear_pack_workspace_bytes(n, k) bytes, 8-byte aligned,
 *              contents ignored; may be NULL when gamma_in is given.
 * Codes: W~ = Clip(rint(fp32(w / fp32(gamma + eps))), -1, 1), ties to even.
 * ---------------------------------------------------------------------- */
size_t bitlinear_pack_workspace_bytes(int64_t n, int64_t k);
bl_status bitlinear_pack_weights(const void* w, int w_dtype, int64_t n, int64_t k,
                                 float eps, const float* gamma_in, void* packed,
                                 float* gamma_out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bitlinear_quant_act -- per-token absmax int8 activation quantization.
 * Defines: "8-Bit Activation Quantization: absmax Scaling".
 *
 *   x       [m][k] fp32 or bf16 (x_dtype), 4-byte aligned (16 for speed).
 *   eps     > 0 with fp32(127 / eps) finite, i.e. eps >= about 3.74e-37
 *           (1e-5 on the pages); 0, negative, NaN/Inf and smaller values
 *           return BL_ERR_INVALID_ARG.  Then s is finite for every token and
 *           an all-zero token gives x~ = 0 (and y = 0).
 *   xq      out, int8 [m][padded_k(k)], 16-byte aligned.  Columns k..K_pad-1
 *           are written as 0.
 *   scale   out, fp32 [m]:  s_m = fp32(127 / max(beta_m, eps)),
 *           beta_m = max_j |x_mj|.
 * x~ = clamp(rint(fp32(x * s_m)), -128, 127) (ties to even); |x~| <= 127.
 * m == 0 is a no-op.
 * ---------------------------------------------------------------------- */
bl_status bitlinear_quant_act(const void* x, int x_dtype, int64_t m, int64_t k,
                              float eps, int8_t* xq, float* scale, void* stream);

/* ------------------------------------------------------------------------
 * bitlinear_rmsnorm_quant_act -- RMSNorm of each token, then the per-token
 * absmax int8 quantization of the normalized activations.  Defines: the
 * BitLinear listing of "End-to-End Implementation: Building a Native
 * BitLinear Layer" (nn.RMSNorm(in_features) applied to x before
 * quantize_activations_int8); "8-Bit Activation Quantization: absmax
 * Scaling" for the quantization.
 *
 *   x            [m][k] fp32 or bf16 (x_dtype), 4-byte aligned.
 *   norm_weight  NULL (a gain of ones, the listing's initial value) or fp32
 *                [k] on the device, 4-byte aligned.
 *   norm_eps     > 0 and finite (nn.RMSNorm's default: fp32 machine epsilon,
 *                2^-23).
 *   eps, xq, scale  as in bitlinear_quant_act, for the normalized y.
 * Per token: ms = fp32(sum_j x_j^2 / k) with the sum accumulated in fp64 in a
 * fixed order (deterministic; equal to the exactly rounded mean unless that
 * lies within fp64 rounding of an fp32 rounding boundary); r = fp32(1 /
 * sqrt(fp32(ms + norm_eps))) evaluated in fp64; y_j = fp32(fp32(x_j * r) *
 * w_j); then s and x~ from y exactly as bitlinear_quant_act.  m == 0 is a
 * no-op.
 * ---------------------------------------------------------------------- */
bl_status bitlinear_rmsnorm_quant_act(const void* x, int x_dtype, int64_t m, int64_t k,
                                      const float* norm_weight, float norm_eps, float eps,
                                      int8_t* xq, float* scale, void* stream);

/* ------------------------------------------------------------------------
 * bitlinear_forward -- y = (x~ W~^T) * gamma / s, with an optional fused
 * ReLU^2.  Defines: "Matrix Multiplication as Pure Integer Addition"
 * (integer accumulator; rescale by beta*gamma/127).
 *
 *   xq, scale  from bitlinear_quant_act (same m, k).
 *   packed     from bitlinear_pack_weights (same n, k); 16-byte aligned.
 *   gamma      one fp32 on the device (gamma_out of the pack call).
 *   epilogue   BL_EPI_NONE or BL_EPI_RELU2 (y <- y > 0 ? y*y : 0, in fp32).
 *   y_dtype    BL_F32 or BL_BF16 (round to nearest even); y is [m][n],
 *              4-byte aligned.
 *   acc_out    NULL, or int32 [m][n] that receives the exact integer
 *              accumulator x~ W~^T (for verification).
 *   workspace  bitlinear_forward_workspace_bytes(m, n, k) bytes, 256-byte
 *              aligned, zero-filled once before its first use (see
 *              bitlinear_workspace_init).  Every completed call leaves it
 *              zero-filled again (each 64-bit split-K slot is cleared by
 *              the contribution that completes it), so one workspace
 *              serves any sequence of calls without clearing.
 *              Calls that share a workspace must be ordered (one stream, or
 *              events); concurrent calls on one workspace race.  May be NULL
 *              when the required size is 0.
 * The accumulator is exact (int32); y is acc * fp32(gamma/s_m) in fp32.
 * m == 0 is a no-op.  The result is the same for every launch and run.
 * ---------------------------------------------------------------------- */
size_t bitlinear_forward_workspace_bytes(int64_t m, int64_t n, int64_t k);
bl_status bitlinear_forward(const int8_t* xq, const float* scale, const void* packed,
                            const float* gamma, int64_t m, int64_t n, int64_t k,
                            int epilogue, int y_dtype, void* y, int32_t* acc_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bitlinear_forward_multi -- several BitLinear products that read the same
 * quantized activations (e.g. the q, k and v projections of one token
 * batch), each y_i = (x~ W~_i^T) * gamma_i / s as in bitlinear_forward
 * ("Matrix Multiplication as Pure Integer Addition"), with the same
 * numbers as one bitlinear_forward per entry.  When the products together
 * are wide enough for the matrix-core GEMM (more than 64 tokens), they run
 * as one launch whose output tiles cover all entries; otherwise one launch
 * per entry.
 *
 *   xq, scale  from bitlinear_quant_act (m tokens, k inputs), shared.
 *   ops        host array of nops (1..BL_MAX_MULTI) entries: packed
 *              weights (n_i, k) 16-byte aligned, gamma_i, epilogue, y
 *              dtype, y_i [m][n_i], acc_out_i (nullable), as in
 *              bitlinear_forward.  The summed padded widths (64 *
 *              ceil(n_i / 64)) must not exceed BL_MAX_MN.
 *   workspace  bitlinear_forward_multi_workspace_bytes(ops, nops, m, k)
 *              bytes, with the contract of bitlinear_forward's workspace
 *              (the entries run in order and share it).
 * m == 0 is a no-op.  Errors as bitlinear_forward, checked for every entry
 * before any launch.
 * ---------------------------------------------------------------------- */
#define BL_MAX_MULTI 16
typedef struct {
  const void* packed;   /* packed weights (n, k), 16-byte aligned */
  const float* gamma;   /* device fp32 */
  int64_t n;
  int epilogue;         /* BL_EPI_NONE or BL_EPI_RELU2 */
  int y_dtype;          /* BL_F32 or BL_BF16 */
  void* y;              /* [m][n] */
  int32_t* acc_out;     /* nullable, int32 [m][n] */
} bl_product;
size_t bitlinear_forward_multi_workspace_bytes(const bl_product* ops, int nops, int64_t m,
                                               int64_t k);
bl_status bitlinear_forward_multi(const int8_t* xq, const float* scale, int64_t m, int64_t k,
                                  const bl_product* ops, int nops, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bitlinear_forward_fused -- the decode step of several BitLinear layers that
 * read the same token batch size, in one launch (but see long rows below):
 * for each entry, per-token
 * absmax int8 quantization of its activations ("8-Bit Activation
 * Quantization: absmax Scaling") and y = (x~ W~^T) * gamma / s ("Matrix
 * Multiplication as Pure Integer Addition"), with the same numbers as
 * bitlinear_quant_act followed by bitlinear_forward.
 *
 *   ops        host array of nops (1..BL_MAX_FUSED) entries; entries may
 *              share x (e.g. the q, k and v projections).
 *   m          tokens, 0..BL_FUSED_MAX_M (0 is a no-op).
 *   eps        as in bitlinear_quant_act (the same values are refused).
 *   workspace  bitlinear_forward_fused_workspace_bytes(ops, nops, m) bytes,
 *              with the contract of bitlinear_forward's workspace.
 * Every workgroup recomputes its entry's per-token absmax from the whole row
 * of x (all workgroups get the same s and x~), so each workgroup reads the
 * activations of its tokens (one block of up to 16 from 3 tokens) from
 * cache once, or twice when a row does not fit its registers; meant for
 * decode-sized batches.  From 3 tokens no workspace is needed (the size
 * query returns 0), except for tables with an activation row of more than
 * 16 KiB (bf16 K > 8192, fp32 K > 4096), and for a single RMSNorm entry
 * with rows of more than 8 KiB: there every distinct input is
 * quantized once by its own launch (into xq_out / scale_out when the entry
 * gives them, else into the workspace), each product then runs its
 * bitlinear_forward plan, and a last launch clears the workspace scratch, so
 * the workspace contract holds (BL_KERNEL_TWO_PASS).
 * Entries with rmsnorm set normalize x first (same numbers as
 * bitlinear_rmsnorm_quant_act followed by bitlinear_forward: the
 * multi-token kernel and the two-pass plan add the squares in fp64 in
 * bitlinear_rmsnorm_quant_act's order; the streaming kernel (1-2 tokens)
 * and the fused matrix-core kernel in fixed orders of their own, so there a
 * token whose mean square lies within the last place of that sum of an fp32
 * rounding boundary may get the neighbouring fp32 mean square).  At 1-2
 * tokens such a table runs on the streaming kernel when every entry has
 * rows of whole 16-byte units at 16-byte alignment, one activation dtype,
 * and x~ of every token within 64 KiB (2 * padded_k <= 65536 at two
 * tokens), and on the fused matrix-core kernel otherwise; every table the
 * checks above accept has a kernel.
 * ---------------------------------------------------------------------- */
#define BL_MAX_FUSED 16
#define BL_FUSED_MAX_M 64
typedef struct {
  const void* x;        /* [m][k] fp32 or bf16 activations, 4-byte aligned */
  int x_dtype;          /* BL_F32 or BL_BF16 */
  const void* packed;   /* packed weights (n, k), 16-byte aligned */
  const float* gamma;   /* device fp32 */
  int64_t n, k;
  int epilogue;         /* BL_EPI_NONE or BL_EPI_RELU2 */
  int y_dtype;          /* BL_F32 or BL_BF16 */
  void* y;              /* [m][n] */
  int32_t* acc_out;     /* nullable: int32 [m][n] accumulator */
  int8_t* xq_out;       /* nullable: int8 [m][padded_k(k)], 16-byte aligned */
  float* scale_out;     /* nullable: fp32 [m] */
  int rmsnorm;          /* nonzero: RMSNorm of x first, as bitlinear_rmsnorm_quant_act */
  float norm_eps;       /* with rmsnorm: > 0 and finite */
  const float* norm_weight;  /* with rmsnorm: NULL (ones) or fp32 [k], 16-byte aligned */
} bl_linear;
size_t bitlinear_forward_fused_workspace_bytes(const bl_linear* ops, int nops, int64_t m);
bl_status bitlinear_forward_fused(const bl_linear* ops, int nops, int64_t m, float eps,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bitlinear_forward_noalloc -- bitlinear_forward for callers that cannot
 * allocate device memory or own a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * checks, kernels and results as bitlinear_forward, without the workspace:
 * the split-K slots live in a scratch array of BL_NOALLOC_SCRATCH_BYTES
 * that the library's code object holds on each device until the process
 * ends.  Nothing is allocated or freed.
 *
 *   - Products whose plan needs more than BL_NOALLOC_SCRATCH_BYTES of
 *     split-K slots return BL_ERR_WORKSPACE before any launch (every split
 *     plan of a matrix with fewer than 16384 rows fits).
 *   - The first call on a device that needs the scratch, and every such call
 *     made under stream capture until one outside capture has run, first
 *     enqueues a small zero-fill kernel on `stream`; every completed call
 *     leaves the scratch zero-filled again.
 *   - All calls on one device share its scratch: calls that overlap in time
 *     on one device (different streams without ordering) race and may return
 *     wrong results.  Order them on one stream or with events.
 * ---------------------------------------------------------------------- */
#define BL_NOALLOC_SCRATCH_BYTES 262144
bl_status bitlinear_forward_noalloc(const int8_t* xq, const float* scale, const void* packed,
                                    const float* gamma, int64_t m, int64_t n, int64_t k,
                                    int epilogue, int y_dtype, void* y, int32_t* acc_out,
                                    void* stream);

/* ------------------------------------------------------------------------
 * bitlinear_forward_kernel, bitlinear_forward_fused_kernel -- which kernel
 * bitlinear_forward (and bitlinear_forward_noalloc) or
 * bitlinear_forward_fused would launch for these arguments: the host-side
 * plan only, nothing is launched and no device memory is touched.  Every
 * kernel gives the same numbers; the choice is speed only.  Returns one of
 * the BL_KERNEL_* values, or a negative bl_status when the arguments would
 * be refused (sizes as the call checks them; for the fused step the
 * pointers' alignment too, since it decides the kernel).
 * ---------------------------------------------------------------------- */
#define BL_KERNEL_DOT4_GEMV 0      /* 1-2 tokens, v_dot4 (fused: the dot4 decode step) */
#define BL_KERNEL_GEMM 1           /* matrix-core GEMM, more than 64 tokens */
#define BL_KERNEL_MFMA_GEMV 2      /* windowed matrix-core GEMV (fused: its fused form) */
#define BL_KERNEL_STREAM_GEMV 3    /* streaming matrix-core GEMV, 1-2 tokens */
#define BL_KERNEL_STREAM_MT 4      /* streaming matrix-core GEMV, blocks of 16 tokens */
#define BL_KERNEL_TWO_PASS 5       /* fused step only: activation quant launches, then each
                                      product's bitlinear_forward plan */
int bitlinear_forward_kernel(int64_t m, int64_t n, int64_t k);
int bitlinear_forward_fused_kernel(const bl_linear* ops, int nops, int64_t m);

/* Zero-fill a forward workspace with a device kernel (no hipMemset, so it can
 * be captured in a HIP graph).  bytes must be a multiple of 4. */
bl_status bitlinear_workspace_init(void* workspace, size_t bytes, void* stream);

/* Static description of a status code. */
const char* bitlinear_status_string(int status);

/* BITLINEAR_ABI_VERSION of the loaded library. */
int bitlinear_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H_ */
