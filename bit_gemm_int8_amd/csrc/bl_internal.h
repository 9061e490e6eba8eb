// Host-side launchers of the libbitlinear kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <stddef.h>
#include <stdint.h>

namespace bl {

// Activation quantization: one workgroup per token.
hipError_t launch_quant_act(const void* x, bool bf16, int64_t m, int64_t k, int64_t kpad,
                            float eps, int8_t* xq, float* scale, hipStream_t stream);

// RMSNorm + activation quantization: one workgroup per token.
hipError_t launch_rmsnorm_quant(const void* x, bool bf16, int64_t m, int64_t k, int64_t kpad,
                                const float* norm_weight, float norm_eps, float eps, int8_t* xq,
                                float* scale, hipStream_t stream);

// Weight absmean partial sums + ternarize/pack.
struct PackPlan {
  int64_t total;       // n * k
  int64_t per_block;   // elements per partial-sum workgroup
  int nparts;          // partial sums written
};
PackPlan pack_plan(int64_t n, int64_t k);
size_t pack_workspace_bytes(int64_t n, int64_t k);
hipError_t launch_pack(const void* w, bool bf16, int64_t n, int64_t k, float eps,
                       const float* gamma_in, uint32_t* packed, float* gamma_out,
                       double* partial, hipStream_t stream);

// Forward: dispatch plan shared by the workspace query and the launch.
struct FwdPlan {
  int kind;            // 0 = dot4 GEMV, 1 = MFMA GEMM, 2 = MFMA GEMV, 3 = stream GEMV,
                       // 4 = multi-token stream GEMV
  int variant;         // dot4 GEMV: waves per workgroup; otherwise the kernel variant
  int pf;              // GEMV: super-chunks in flight per wave
  int qpl;             // GEMV: 16-byte q-parts per lane (4: 64 rows per group, 1: 16 rows);
                       // stream GEMV: workgroups; multi-token stream GEMV: row ranges
  int splits;          // split-K factor
  size_t slots;        // 64-bit split-K slots in the workspace (splits > 1)
  size_t ws_bytes;     // total workspace bytes
};
FwdPlan forward_plan(int64_t m, int64_t n, int64_t k);
hipError_t launch_forward(const FwdPlan& plan, const int8_t* xq, const float* scale,
                          const uint32_t* packed, const float* gamma, int64_t m, int64_t n,
                          int64_t k, bool relu2, bool bf16, void* y, int32_t* acc_out,
                          void* workspace, hipStream_t stream);

hipError_t launch_fill_zero(uint32_t* p, size_t words, hipStream_t stream);

// GEMM over a table of products that share x~ and s (each with its own
// packed weights, gamma, N and output): one launch, the products' column
// tiles side by side.  A single bitlinear_forward is the one-entry table.
constexpr int kMaxMulti = 16;
struct GemmProduct {
  const void* packed;
  const float* gamma;
  int64_t n;
  bool relu2, bf16;
  void* y;
  int32_t* acc_out;       // nullable
};
hipError_t launch_gemm_multi(int variant, const int8_t* xq, const float* scale, int64_t m,
                             int64_t k, const GemmProduct* ops, int nops, hipStream_t stream);

// Fused decode step: a table of BitLinear products that share a token batch
// (M <= 64), each quantizing its own activations in the kernel prologue.
constexpr int kMaxFused = 16;
// One entry of the fused decode step.  The fields a workgroup needs first
// share the first 64-byte line (one scalar load after the entry is known);
// the optional outputs sit in the second line and are read at the end.
struct alignas(64) FusedSeg {
  const void* x;          // [m][k] activations (fp32 or bf16)
  const void* packed;     // packed weights (n, k)
  const float* gamma;
  void* y;                // [m][n]
  int64_t* slots;         // split-K slots, [row block][m][64] (splits > 1)
  int n, k, nc, splits, wg_begin;
  int flags;              // bit 0: ReLU^2, bit 1: y bf16, bit 2: x bf16, bit 3: RMSNorm
  int32_t* acc_out;       // nullable
  int8_t* xq_out;         // nullable, [m][padded_k(k)]
  float* scale_out;       // nullable, [m]
  const float* norm_weight;  // RMSNorm gain (nullable: ones), with flags bit 3
  float norm_eps;
  __host__ __device__ bool relu2() const { return (flags & 1) != 0; }
  __host__ __device__ bool rmsnorm() const { return (flags & 8) != 0; }
  __host__ __device__ bool y_bf16() const { return (flags & 2) != 0; }
  __host__ __device__ bool x_bf16() const { return (flags & 4) != 0; }
};
// The entries' first workgroups share one 64-byte line, so a workgroup
// finds its entry with one scalar load.
struct FusedArgs {
  int wg_begin[kMaxFused];
  int nseg;
  float eps;
  int nsub_alloc;         // stream kernel: 16-row sub-blocks per workgroup, at most
  FusedSeg seg[kMaxFused];
};
static_assert(kMaxFused * sizeof(int) == 64, "entry starts in one line");
static_assert(offsetof(FusedSeg, acc_out) == 64, "first-use fields in the first line");
hipError_t launch_gemv_mfma(int variant, const int8_t* xq, const float* scale,
                            const uint32_t* packed, const float* gamma, int64_t m, int64_t n,
                            int64_t k, bool relu2, bool bf16, void* y, int32_t* acc_out,
                            hipStream_t stream);
hipError_t launch_gemv_mfma_fused(const FusedArgs& args, int m, int variant, bool all_bf16,
                                  bool all_fast, bool norm, int groups, hipStream_t stream);
hipError_t launch_gemv_fused(const FusedArgs& args, int m, int waves, int qpl, bool long_rows,
                             int groups, size_t lds, hipStream_t stream);

// Streaming one/two-token GEMV on the matrix cores (whole 16-row sub-blocks
// per workgroup, x~ of every token in LDS).
size_t stream_lds_bytes(int m, int64_t nc, int nsub_alloc);
void stream_shape(int m, int64_t nc, int* waves, int* depth);
void stream_fused_shape(bool wide, int* waves, int* depth);
hipError_t launch_gemv_stream(int m, const int8_t* xq, const float* scale,
                              const uint32_t* packed, const float* gamma, int64_t n, int64_t k,
                              int grid, bool relu2, bool bf16, void* y, int32_t* acc_out,
                              hipStream_t stream);
hipError_t launch_gemv_stream_fused(const FusedArgs& args, int m, bool wide, bool x_bf16,
                                    bool norm, int xr, int groups, size_t lds,
                                    hipStream_t stream);

// Multi-token streaming GEMV on the matrix cores (x~ of a block of up to 16
// tokens in LDS -- 8 or 16 in the fused form, `tok` --, whole 16-row
// sub-blocks per row range, P row ranges x ceil(m / tok) token blocks of
// workgroups).  gain_k: fp32 RMSNorm gain values staged in LDS (the longest
// row of an entry with a gain; 0 for none).
size_t stream_mt_lds_bytes(int64_t m, int64_t nc, int nsub_alloc, int tok, int64_t gain_k);
hipError_t launch_gemv_stream_mt(const int8_t* xq, const float* scale, const uint32_t* packed,
                                 const float* gamma, int64_t m, int64_t n, int64_t k, int P,
                                 bool relu2, bool bf16, void* y, int32_t* acc_out,
                                 hipStream_t stream);
hipError_t launch_gemv_stream_mt_fused(const FusedArgs& args, int m, int tok, bool x_bf16,
                                       bool norm, int xr, int groups, size_t lds,
                                       hipStream_t stream);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t padded_n(int64_t n) { return 64 * cdiv(n, 64); }
inline int64_t padded_k(int64_t k) { return 256 * cdiv(k, 256); }

}  // namespace bl
