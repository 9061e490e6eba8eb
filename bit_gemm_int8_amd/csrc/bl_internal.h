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
  int kind;            // 0 = dot4 GEMV, 1 = MFMA GEMM
  int variant;         // tile variant
  int splits;          // split-K factor
  int tiles;           // output tiles that own a counter
  size_t partial_ints; // int32 partial elements in the workspace
  size_t ws_bytes;     // total workspace bytes
};
FwdPlan forward_plan(int64_t m, int64_t n, int64_t k);
hipError_t launch_forward(const FwdPlan& plan, const int8_t* xq, const float* scale,
                          const uint32_t* packed, const float* gamma, int64_t m, int64_t n,
                          int64_t k, bool relu2, bool bf16, void* y, int32_t* acc_out,
                          void* workspace, hipStream_t stream);

hipError_t launch_fill_zero(uint32_t* p, size_t words, hipStream_t stream);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t padded_n(int64_t n) { return 64 * cdiv(n, 64); }
inline int64_t padded_k(int64_t k) { return 256 * cdiv(k, 256); }

}  // namespace bl
