// Host-only exercise of the libbitlinear C ABI for the sanitizer build:
// every size query, plan query and host-side refusal, with edge values.
// Nothing here launches a kernel or needs a GPU (every call returns before
// any HIP call); a failed expectation exits with status 1, a sanitizer
// report with its own status.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <initializer_list>

#include "../../include/bitlinear.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

// distinct fake device addresses (never dereferenced: the calls below are
// refused on the host before any launch)
static void* fake(uintptr_t i, uintptr_t off = 0) { return (void*)(0x100000000ull * i + off); }

int main() {
  EXPECT(bitlinear_abi_version() == BITLINEAR_ABI_VERSION);
  for (int s = -3; s < 12; ++s) EXPECT(bitlinear_status_string(s) != nullptr);

  const int64_t sizes[] = {-5, -1, 0, 1, 2, 63, 64, 65, 255, 256, 257, 4100, 65536,
                           BL_MAX_K, BL_MAX_K + 1, BL_MAX_MN, BL_MAX_MN + 1, INT64_MAX / 2};
  for (int64_t a : sizes) {
    (void)bitlinear_padded_n(a);
    (void)bitlinear_padded_k(a);
    for (int64_t b : sizes) {
      (void)bitlinear_packed_bytes(a, b);
      (void)bitlinear_xq_bytes(a, b);
      (void)bitlinear_pack_workspace_bytes(a, b);
      for (int64_t c : {(int64_t)0, (int64_t)1, (int64_t)2, (int64_t)3, (int64_t)64,
                        (int64_t)65, (int64_t)512, (int64_t)2048, (int64_t)BL_MAX_MN}) {
        (void)bitlinear_forward_workspace_bytes(c, a, b);
        const int k = bitlinear_forward_kernel(c, a, b);
        EXPECT(k >= -BL_ERR_HIP && k <= BL_KERNEL_STREAM_MT);
      }
    }
  }
  EXPECT(bitlinear_forward_kernel(0, 10, 10) == -BL_ERR_INVALID_ARG);

  // bitlinear_pack_weights refusals
  EXPECT(bitlinear_pack_weights(nullptr, BL_F32, 4, 4, 1e-5f, nullptr, fake(2), (float*)fake(3),
                                fake(4), 1 << 20, nullptr) == BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_pack_weights(fake(1), 7, 4, 4, 1e-5f, nullptr, fake(2), (float*)fake(3),
                                fake(4), 1 << 20, nullptr) == BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_pack_weights(fake(1), BL_F32, 4, BL_MAX_K + 1, 1e-5f, nullptr, fake(2),
                                (float*)fake(3), fake(4), 1 << 20, nullptr) ==
         BL_ERR_UNSUPPORTED_SHAPE);
  EXPECT(bitlinear_pack_weights(fake(1, 4), BL_F32, 4, 4, 1e-5f, nullptr, fake(2),
                                (float*)fake(3), fake(4), 1 << 20, nullptr) == BL_ERR_MISALIGNED);
  EXPECT(bitlinear_pack_weights(fake(1), BL_F32, 4, 4, 1e-5f, nullptr, fake(2), (float*)fake(3),
                                nullptr, 0, nullptr) == BL_ERR_WORKSPACE);
  EXPECT(bitlinear_pack_weights(fake(1), BL_F32, 4, 4, -1.0f, nullptr, fake(2), (float*)fake(3),
                                fake(4), 1 << 20, nullptr) == BL_ERR_INVALID_ARG);

  // bitlinear_quant_act / rmsnorm refusals (eps rule included)
  const float bad_eps[] = {0.0f, -1e-5f, 1e-38f, 1.0f / 0.0f};
  for (float e : bad_eps)
    EXPECT(bitlinear_quant_act(fake(1), BL_BF16, 2, 256, e, (int8_t*)fake(2), (float*)fake(3),
                               nullptr) == BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_quant_act(nullptr, BL_BF16, 2, 256, 1e-5f, (int8_t*)fake(2), (float*)fake(3),
                             nullptr) == BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_quant_act(fake(1), BL_BF16, 2, 256, 1e-5f, (int8_t*)fake(2, 8),
                             (float*)fake(3), nullptr) == BL_ERR_MISALIGNED);
  EXPECT(bitlinear_quant_act(fake(1), BL_F32, 2, BL_MAX_K + 1, 1e-5f, (int8_t*)fake(2),
                             (float*)fake(3), nullptr) == BL_ERR_UNSUPPORTED_SHAPE);
  EXPECT(bitlinear_quant_act(fake(1), BL_F32, 0, 256, 1e-5f, (int8_t*)fake(2), (float*)fake(3),
                             nullptr) == BL_OK);
  EXPECT(bitlinear_rmsnorm_quant_act(fake(1), BL_BF16, 2, 256, nullptr, 0.0f, 1e-5f,
                                     (int8_t*)fake(2), (float*)fake(3), nullptr) ==
         BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_rmsnorm_quant_act(fake(1), BL_BF16, 2, 256, (const float*)fake(4, 2), 1e-6f,
                                     1e-5f, (int8_t*)fake(2), (float*)fake(3), nullptr) ==
         BL_ERR_MISALIGNED);

  // bitlinear_forward / noalloc refusals
  EXPECT(bitlinear_forward((int8_t*)fake(1), (float*)fake(2), fake(3), (float*)fake(4), 2, 100,
                           256, 9, BL_F32, fake(5), nullptr, nullptr, 0, nullptr) ==
         BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_forward((int8_t*)fake(1), (float*)fake(2), fake(3, 4), (float*)fake(4), 2,
                           100, 256, BL_EPI_NONE, BL_F32, fake(5), nullptr, nullptr, 0,
                           nullptr) == BL_ERR_MISALIGNED);
  EXPECT(bitlinear_forward((int8_t*)fake(1), (float*)fake(2), fake(3), (float*)fake(4), 2, 300,
                           40000, BL_EPI_NONE, BL_F32, fake(5), nullptr, nullptr, 0, nullptr) ==
         BL_ERR_WORKSPACE);
  EXPECT(bitlinear_forward_noalloc((int8_t*)fake(1), (float*)fake(2), fake(3), (float*)fake(4),
                                   2, 16448, 65536, BL_EPI_NONE, BL_F32, fake(5), nullptr,
                                   nullptr) == BL_ERR_WORKSPACE);
  EXPECT(bitlinear_forward_noalloc(nullptr, (float*)fake(2), fake(3), (float*)fake(4), 2, 100,
                                   256, BL_EPI_NONE, BL_F32, fake(5), nullptr, nullptr) ==
         BL_ERR_INVALID_ARG);

  // fused and multi tables
  bl_linear ops[BL_MAX_FUSED + 1];
  for (int i = 0; i < BL_MAX_FUSED + 1; ++i) {
    ops[i] = bl_linear{};
    ops[i].x = fake(10 + i);
    ops[i].x_dtype = BL_BF16;
    ops[i].packed = fake(40 + i);
    ops[i].gamma = (const float*)fake(70 + i);
    ops[i].n = 64 * (i + 1) + 3;
    ops[i].k = 256 * (i + 1) + 8;
    ops[i].epilogue = i % 2;
    ops[i].y_dtype = BL_BF16;
    ops[i].y = fake(100 + i);
    ops[i].rmsnorm = i % 3 == 0;
    ops[i].norm_eps = 1e-6f;
  }
  for (int nops = 0; nops <= BL_MAX_FUSED + 1; ++nops)
    for (int64_t m : {(int64_t)-1, (int64_t)0, (int64_t)1, (int64_t)2, (int64_t)3, (int64_t)17,
                      (int64_t)64, (int64_t)65}) {
      (void)bitlinear_forward_fused_workspace_bytes(ops, nops, m);
      const int k = bitlinear_forward_fused_kernel(ops, nops, m);
      EXPECT(k >= -BL_ERR_HIP && k <= BL_KERNEL_STREAM_MT);
    }
  EXPECT(bitlinear_forward_fused(ops, 3, 4, 0.0f, nullptr, 0, nullptr) == BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_forward_fused(ops, BL_MAX_FUSED + 1, 4, 1e-5f, nullptr, 0, nullptr) ==
         BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_forward_fused(ops, 3, BL_FUSED_MAX_M + 1, 1e-5f, nullptr, 0, nullptr) ==
         BL_ERR_UNSUPPORTED_SHAPE);
  ops[0].norm_eps = 0.0f;                    // an RMSNorm entry with a bad norm eps
  EXPECT(ops[0].rmsnorm != 0);
  EXPECT(bitlinear_forward_fused(ops, 3, 4, 1e-5f, nullptr, 0, nullptr) == BL_ERR_INVALID_ARG);

  bl_product prods[BL_MAX_FUSED + 1];
  for (int i = 0; i < BL_MAX_FUSED + 1; ++i) {
    prods[i] = bl_product{};
    prods[i].packed = fake(40 + i);
    prods[i].gamma = (const float*)fake(70 + i);
    prods[i].n = 100 + 37 * i;
    prods[i].y_dtype = BL_F32;
    prods[i].y = fake(100 + i);
  }
  for (int nops = 0; nops <= BL_MAX_FUSED + 1; ++nops)
    for (int64_t m : {(int64_t)0, (int64_t)1, (int64_t)64, (int64_t)512, (int64_t)4096})
      (void)bitlinear_forward_multi_workspace_bytes(prods, nops, m, 2560);
  EXPECT(bitlinear_forward_multi(nullptr, (float*)fake(2), 4, 256, prods, 2, nullptr, 0,
                                 nullptr) == BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_workspace_init(fake(1), 6, nullptr) == BL_ERR_INVALID_ARG);
  EXPECT(bitlinear_workspace_init(nullptr, 0, nullptr) == BL_OK);

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi_driver: all host-side checks passed\n");
  return 0;
}
