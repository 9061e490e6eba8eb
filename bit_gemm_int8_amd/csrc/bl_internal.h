// Host-side launchers of the libbitlinear kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

// Activation quantization: one workgroup per token.
hipError_t launch_quant_act(const void* x, bool bf16, int64_t m, int64_t k, int64_t kpad,
                            float eps, int8_t* xq, float* scale, hipStream_t stream);

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
  int kind;            // 0 = dot4 GEMV, 1 = MFMA GEMM, 2 = MFMA GEMV
  int variant;         // dot4 GEMV: waves per workgroup; otherwise the kernel variant
  int pf;              // GEMV: super-chunks in flight per wave
  int qpl;             // GEMV: 16-byte q-parts per lane (4: 64 rows per group, 1: 16 rows)
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

// Fused decode step: a table of BitLinear products that share a token batch
// (M <= 4), each quantizing its own activations in the kernel prologue.
constexpr int kMaxFused = 16;
struct FusedSeg {
  const void* x;          // [m][k] activations (fp32 or bf16)
  const void* packed;     // packed weights (n, k)
  const float* gamma;
  void* y;                // [m][n]
  int32_t* acc_out;       // nullable
  int8_t* xq_out;         // nullable, [m][padded_k(k)]
  float* scale_out;       // nullable, [m]
  int64_t* slots;         // split-K slots, [row block][m][64] (splits > 1)
  int n, k, nc, splits, wg_begin, relu2, y_bf16, x_bf16;
};
struct FusedArgs {
  FusedSeg seg[kMaxFused];
  int nseg;
  float eps;
};
hipError_t launch_gemv_mfma(int variant, const int8_t* xq, const float* scale,
                            const uint32_t* packed, const float* gamma, int64_t m, int64_t n,
                            int64_t k, bool relu2, bool bf16, void* y, int32_t* acc_out,
                            hipStream_t stream);
hipError_t launch_gemv_fused(const FusedArgs& args, int m, int waves, int qpl, bool long_rows,
                             int groups, size_t lds, hipStream_t stream);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t padded_n(int64_t n) { return 64 * cdiv(n, 64); }
inline int64_t padded_k(int64_t k) { return 256 * cdiv(k, 256); }

}  // namespace bl
