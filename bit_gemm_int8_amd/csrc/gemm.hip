// Ternary x int8 GEMM on int8 MFMA (v_mfma_i32_16x16x64_i8) with the fused
// dequant, for M > 4 tokens (prefill and batched decode).
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T (integer), then
// y = acc * gamma / s.  With many tokens the product is a dense contraction,
// so it runs on the matrix cores: the 2-bit codes are expanded to int8
// (64 * W~) in registers right before each MFMA.
//
// Tile: BM x BN outputs per workgroup, waves in a WM x WN grid, each wave
// FM x FN fragments of 16x16.  Per 256-input super-chunk the workgroup stages
//   A: x~ rows m0..m0+BM-1, 256 bytes each, into LDS; the 16-byte unit u of
//      row r is stored at unit u ^ (r % 16) so that the 16 lanes reading one
//      MFMA operand column hit 16 different bank groups;
//   B: BN/64 packed 4 KiB blocks, copied as they are.
// MFMA operands: lane l = r + 16 g (r = l % 16, g = l / 16) supplies, for
// k-step j of the super-chunk, the 16 inputs 64 j + 16 g + (0..15): A from x~
// row r of the fragment, B from packed word (q = g, j) of row r, unpacked to
// four dwords.  Byte e of operand dword i is input 4 i + e on both sides, so
// the lane-to-k assignment agrees between A and B, which is all the sum needs.
// The 16x16 int32 result holds row 4 g + i, column r in element i of lane l.
//
// Global loads of super-chunk c+1 are issued before the MFMAs of c (register
// staging, one LDS buffer).  Split-K over super-chunks adds tiles into the
// workspace with device-scope atomics, as in the GEMV.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

template <int FM, int FN, int WM, int WN>
struct Tile {
  static constexpr int BM = 16 * FM * WM;
  static constexpr int BN = 16 * FN * WN;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BNB = BN / 64;              // packed blocks per tile
  static constexpr int UA = BM * 16 / NT;          // 16-byte A units per thread
  static constexpr int UB = BNB * kBlockU4 / NT;   // 16-byte B units per thread
  static_assert(BN % 64 == 0, "tile width must hold whole packed blocks");
  static_assert(BM * 16 % NT == 0 && BNB * kBlockU4 % NT == 0, "staging split");
};

template <int FM, int FN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ scale,
    const uint4* __restrict__ packed, const float* __restrict__ gamma, int m, int n,
    int nb, int nc, int64_t kpad, int splits, int tiles_n, int relu2, int bf16,
    void* __restrict__ y, int32_t* __restrict__ acc_out, int32_t* __restrict__ ws_acc,
    uint32_t* __restrict__ counters) {
  using T = Tile<FM, FN, WM, WN>;
  constexpr int BM = T::BM, BN = T::BN, NT = T::NT, BNB = T::BNB, UA = T::UA, UB = T::UB;
  __shared__ __attribute__((aligned(16))) uint8_t As[BM * 256];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[BNB * 4096];
  __shared__ float fac[BM];
  __shared__ uint32_t flag;

  const int tile = blockIdx.x / splits;
  const int s = blockIdx.x - tile * splits;
  const int tm = tile / tiles_n;
  const int tn = tile - tm * tiles_n;
  const int m0 = tm * BM;
  const int b0 = tn * BNB;
  const int c0 = (int)((int64_t)s * nc / splits);
  const int c1 = (int)((int64_t)(s + 1) * nc / splits);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave / WN;
  const int wn = wave - wm * WN;
  const int r = lane & 15;
  const int g = lane >> 4;

  uint4 ra[UA], rb[UB];
  auto load_tile = [&](int c) {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int p = tid + NT * u;
      const int row = p >> 4, unit = p & 15;
      const int gm = m0 + row;
      ra[u] = gm < m ? *reinterpret_cast<const uint4*>(xq + (int64_t)gm * kpad +
                                                       (int64_t)c * 256 + unit * 16)
                     : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int p = tid + NT * u;
      const int bb = p >> 8, within = p & 255;
      const int blk = b0 + bb;
      rb[u] = blk < nb ? packed[((int64_t)blk * nc + c) * kBlockU4 + within]
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int p = tid + NT * u;
      const int row = p >> 4, unit = p & 15;
      *reinterpret_cast<uint4*>(As + row * 256 + ((unit ^ (row & 15)) << 4)) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int p = tid + NT * u;
      *reinterpret_cast<uint4*>(Bs + (p >> 8) * 4096 + (p & 255) * 16) = rb[u];
    }
  };

  bl_v4i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = bl_v4i{0, 0, 0, 0};

  if (c0 < c1) load_tile(c0);
  for (int c = c0; c < c1; ++c) {
    store_tile();
    __syncthreads();
    if (c + 1 < c1) load_tile(c + 1);

    uint4 bw[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = wn * 16 * FN + 16 * fn + r;
      bw[fn] = *reinterpret_cast<const uint4*>(Bs + (col >> 6) * 4096 + g * 1024 + (col & 63) * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bl_v4i a[FM];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int row = wm * 16 * FM + 16 * fm + r;
        a[fm] = *reinterpret_cast<const bl_v4i*>(As + row * 256 + (((4 * j + g) ^ r) << 4));
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint32_t wj = j == 0 ? bw[fn].x : j == 1 ? bw[fn].y : j == 2 ? bw[fn].z : bw[fn].w;
        const bl_v4i bop = {(int)unpack_x64(wj, 0), (int)unpack_x64(wj, 1),
                            (int)unpack_x64(wj, 2), (int)unpack_x64(wj, 3)};
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[fm], bop, acc[fm][fn], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (splits > 1) {
    // Split-K: add this group's tile into the workspace accumulator with
    // device-scope atomics (each returns, so it has been performed before
    // the tile's counter is bumped); the group that completes the count reads
    // the totals and leaves the accumulator and the counter at zero.
    constexpr int NE = FM * FN * 4;
    int32_t* slot = ws_acc + (int64_t)tile * (BM * BN) + tid;
    int done = 0;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          done |= __hip_atomic_fetch_add(slot + ((fm * FN + fn) * 4 + i) * NT, acc[fm][fn][i],
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(done));
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      flag = prev == (uint32_t)(splits - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (flag == 0u) return;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int32_t* p = slot + ((fm * FN + fn) * 4 + i) * NT;
          acc[fm][fn][i] = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    if (tid == 0)
      __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    (void)NE;
  }

  const float gam = *gamma;
  for (int t = tid; t < BM; t += NT) {
    const int gm = m0 + t;
    fac[t] = gm < m ? gamma_over_s(gam, scale[gm]) : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 16 * FM + 16 * fm + 4 * g + i;
      const int gm = m0 + row;
      if (gm >= m) continue;
      const float f = fac[row];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int gn = b0 * 64 + wn * 16 * FN + 16 * fn + r;
        if (gn >= n) continue;
        const int a = acc[fm][fn][i] >> 6;
        const int64_t idx = (int64_t)gm * n + gn;
        if (acc_out != nullptr) acc_out[idx] = a;
        store_out(y, idx, a, f, relu2 != 0, bf16 != 0);
      }
    }
  }
}

template <int FM, int FN, int WM, int WN>
hipError_t run(const int8_t* xq, const float* scale, const uint32_t* packed, const float* gamma,
               int64_t m, int64_t n, int64_t k, int splits, bool relu2, bool bf16, void* y,
               int32_t* acc_out, int32_t* partial, uint32_t* counters, hipStream_t stream) {
  using T = Tile<FM, FN, WM, WN>;
  const int nb = (int)cdiv(n, kRowBlock);
  const int nc = (int)cdiv(k, kSuperK);
  const int tiles_m = (int)cdiv(m, T::BM);
  const int tiles_n = (int)cdiv(padded_n(n), T::BN);
  const int64_t grid = (int64_t)tiles_m * tiles_n * splits;
  gemm_kernel<FM, FN, WM, WN><<<(unsigned)grid, T::NT, 0, stream>>>(
      xq, scale, reinterpret_cast<const uint4*>(packed), gamma, (int)m, (int)n, nb, nc,
      padded_k(k), splits, tiles_n, relu2, bf16, y, acc_out, partial, counters);
  return hipGetLastError();
}

}  // namespace

// Tile variants: rows per tile and columns per tile.
//   0: 16 x 256   1: 32 x 256   2: 64 x 256   3: 128 x 128
void gemm_tile_shape(int variant, int* bm, int* bn) {
  switch (variant) {
    case 0: *bm = Tile<1, 4, 1, 4>::BM; *bn = Tile<1, 4, 1, 4>::BN; break;
    case 1: *bm = Tile<2, 4, 1, 4>::BM; *bn = Tile<2, 4, 1, 4>::BN; break;
    case 2: *bm = Tile<4, 4, 1, 4>::BM; *bn = Tile<4, 4, 1, 4>::BN; break;
    default: *bm = Tile<4, 4, 2, 2>::BM; *bn = Tile<4, 4, 2, 2>::BN; break;
  }
}

hipError_t launch_gemm(int variant, const int8_t* xq, const float* scale, const uint32_t* packed,
                       const float* gamma, int64_t m, int64_t n, int64_t k, int splits,
                       bool relu2, bool bf16, void* y, int32_t* acc_out, int32_t* partial,
                       uint32_t* counters, hipStream_t stream) {
  switch (variant) {
    case 0: return run<1, 4, 1, 4>(xq, scale, packed, gamma, m, n, k, splits, relu2, bf16, y, acc_out, partial, counters, stream);
    case 1: return run<2, 4, 1, 4>(xq, scale, packed, gamma, m, n, k, splits, relu2, bf16, y, acc_out, partial, counters, stream);
    case 2: return run<4, 4, 1, 4>(xq, scale, packed, gamma, m, n, k, splits, relu2, bf16, y, acc_out, partial, counters, stream);
    default: return run<4, 4, 2, 2>(xq, scale, packed, gamma, m, n, k, splits, relu2, bf16, y, acc_out, partial, counters, stream);
  }
}

}  // namespace bl
