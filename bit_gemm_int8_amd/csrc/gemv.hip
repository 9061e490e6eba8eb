// Decode ternary GEMV for a few tokens (M <= 4) with the fused dequant.
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T in an integer
// accumulator, then y = acc * beta*gamma/127 = acc * gamma / s.
//
// At batch 1 the product reads every packed weight once and does two integer
// ops per 1/4 byte, so the kernel is bound by HBM bandwidth.  Layout of the
// work (the packed layout is in include/bitlinear.h):
//   - a workgroup owns one 64-row packed block (lane = row) and WAVES waves
//     split its 256-input super-chunks into contiguous ranges;
//   - per super-chunk a lane loads its row's 64 bytes as four 128-bit loads
//     q = 0..3; each load instruction of a wave reads 1 KiB of contiguous
//     memory, and PF super-chunks per wave are in flight at once;
//   - all lanes of a wave work on the same inputs: the workgroup stages its
//     slice of x~ in LDS once (after issuing its first weight loads) and the
//     lanes read it at one shared address, which the LDS broadcasts;
//   - a word unpacks to four int8 lanes of 64*W~ with one shift and one mask;
//     acc = sum >> 6 at the end (every term is a multiple of 64);
//   - the waves' sums meet in LDS; when the row blocks alone cannot fill the
//     chip, `splits` workgroups share a row block and combine through the
//     workspace with device-scope atomics (no cache-wide fences).
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

// One super-chunk: w = the lane's four 16-byte loads q = 0..3 (word (q, j) =
// w[q].{x,y,z,w}[j], inputs 64j + 16q + 4i + (0..3)), xs = this super-chunk's
// 256 bytes of x~ for each token in LDS (token stride xs_stride dwords).  All
// lanes read the same LDS address, which the LDS broadcasts.
template <int M>
__device__ __forceinline__ void accumulate_chunk(const uint4 (&w)[4], const uint32_t* xs,
                                                 int xs_stride, int (&acc)[M]) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wq[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + m * xs_stride + 16 * j + 4 * q);
        acc[m] = dot4(unpack_x64(wq[j], 0), xv.x, acc[m]);
        acc[m] = dot4(unpack_x64(wq[j], 1), xv.y, acc[m]);
        acc[m] = dot4(unpack_x64(wq[j], 2), xv.z, acc[m]);
        acc[m] = dot4(unpack_x64(wq[j], 3), xv.w, acc[m]);
      }
    }
  }
}

template <int M, int WAVES, int PF>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ scale,
    const uint4* __restrict__ packed, const float* __restrict__ gamma, int n, int nc,
    int64_t kpad, int splits, int relu2, int bf16, void* __restrict__ y,
    int32_t* __restrict__ acc_out, int32_t* __restrict__ ws_acc,
    uint32_t* __restrict__ counters) {
  __shared__ int red[WAVES > 1 ? WAVES - 1 : 1][M][64];
  extern __shared__ uint4 xs_lds[];                 // x~ of this group's inputs, per token
  const int b = blockIdx.x / splits;
  const int s = blockIdx.x - b * splits;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  // this workgroup's super-chunks, then this wave's contiguous share
  const int g0 = (int)((int64_t)s * nc / splits);
  const int g1 = (int)((int64_t)(s + 1) * nc / splits);
  const int c0 = g0 + (int)((int64_t)wave * (g1 - g0) / WAVES);
  const int c1 = g0 + (int)((int64_t)(wave + 1) * (g1 - g0) / WAVES);
  const uint4* blk = packed + (int64_t)b * nc * kBlockU4 + lane;

  // epilogue operands, loaded now so their latency hides under the stream
  const float g = *gamma;
  float fac[M];
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = scale[m];

  int acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0;

  // first weight loads in flight before staging x~
  uint4 buf[PF][4];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    if (c0 + p < c1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) buf[p][q] = blk[(int64_t)(c0 + p) * kBlockU4 + q * 64];
    }
  }
  // stage x~[m][256*g0 .. 256*g1) for every token (16 units of 16 bytes per
  // super-chunk and token)
  const int span = (g1 - g0) * 16;                  // uint4 per token
  for (int u = threadIdx.x; u < span * M; u += 64 * WAVES) {
    const int m = u / span, v = u - m * span;
    xs_lds[u] = reinterpret_cast<const uint4*>(xq + (int64_t)m * kpad + (int64_t)g0 * 256)[v];
  }
  __syncthreads();
  const uint32_t* xs = reinterpret_cast<const uint32_t*>(xs_lds);
  const int xs_stride = span * 4;                   // dwords per token
  for (int c = c0; c < c1; c += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (c + p < c1) {
        accumulate_chunk<M>(buf[p], xs + (c + p - g0) * 64, xs_stride, acc);
        if (c + p + PF < c1) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            buf[p][q] = blk[(int64_t)(c + p + PF) * kBlockU4 + q * 64];
        }
      }
    }
  }

  // waves of the workgroup meet in LDS; wave 0 keeps the sum
  if (WAVES > 1) {
    if (wave > 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave - 1][m][lane] = acc[m];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < WAVES - 1; ++w)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] += red[w][m][lane];
  }

  if (splits > 1) {
    // Workgroups that share a row block add their sums into the workspace
    // accumulator with device-scope atomics; each add returns, so it has
    // been performed before this group bumps the block's counter.  The group
    // that brings the counter to `splits` reads the totals with device-scope
    // atomic loads, clears them and the counter for the next call.
    int32_t* slot = ws_acc + (int64_t)b * (M * 64) + lane;
    int done = 0;
#pragma unroll
    for (int m = 0; m < M; ++m)
      done |= __hip_atomic_fetch_add(slot + m * 64, acc[m], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(done));                  // the returned values are in
    uint32_t prev = 0;
    if (lane == 0) {
      __builtin_amdgcn_s_waitcnt(0);
      prev = __hip_atomic_fetch_add(&counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
    if (prev != (uint32_t)(splits - 1)) return;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      acc[m] = __hip_atomic_load(slot + m * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(slot + m * 64, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0)
      __hip_atomic_store(&counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  const int64_t row = (int64_t)b * 64 + lane;
  if (row >= n) return;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int a = acc[m] >> 6;                       // exact: every term is a multiple of 64
    if (acc_out != nullptr) acc_out[(int64_t)m * n + row] = a;
    store_out(y, (int64_t)m * n + row, a, gamma_over_s(g, fac[m]), relu2 != 0, bf16 != 0);
  }
}

template <int M, int WAVES, int PF>
hipError_t run_gemv(const int8_t* xq, const float* scale, const uint32_t* packed,
                    const float* gamma, int64_t n, int64_t k, int splits, bool relu2, bool bf16,
                    void* y, int32_t* acc_out, int32_t* ws_acc, uint32_t* counters,
                    hipStream_t stream) {
  const int nb = (int)cdiv(n, kRowBlock);
  const int nc = (int)cdiv(k, kSuperK);
  dim3 grid((unsigned)((int64_t)nb * splits)), block(64 * WAVES);
  const size_t lds = (size_t)M * cdiv(nc, splits) * 256;
  gemv_kernel<M, WAVES, PF><<<grid, block, lds, stream>>>(
      xq, scale, reinterpret_cast<const uint4*>(packed), gamma, (int)n, nc, padded_k(k), splits,
      relu2, bf16, y, acc_out, ws_acc, counters);
  return hipGetLastError();
}

}  // namespace

// Waves per workgroup for a given shape: enough that one row block's
// workgroup keeps several super-chunks in flight per wave.
hipError_t launch_gemv(int m, int waves, const int8_t* xq, const float* scale,
                       const uint32_t* packed, const float* gamma, int64_t n, int64_t k,
                       int splits, bool relu2, bool bf16, void* y, int32_t* acc_out,
                       int32_t* ws_acc, uint32_t* counters, hipStream_t stream) {
#define BL_GEMV(MM, WW)                                                                        \
  return run_gemv<MM, WW, (WW >= 16 ? 1 : 2)>(xq, scale, packed, gamma, n, k, splits, relu2, bf16, y, acc_out, \
                             ws_acc, counters, stream)
#define BL_GEMV_W(MM)            \
  switch (waves) {               \
    case 1: BL_GEMV(MM, 1);      \
    case 2: BL_GEMV(MM, 2);      \
    case 4: BL_GEMV(MM, 4);      \
    case 8: BL_GEMV(MM, 8);      \
    default: BL_GEMV(MM, 16);    \
  }
  switch (m) {
    case 1: BL_GEMV_W(1);
    case 2: BL_GEMV_W(2);
    case 3: BL_GEMV_W(3);
    case 4: BL_GEMV_W(4);
    default: return hipErrorInvalidValue;
  }
#undef BL_GEMV_W
#undef BL_GEMV
}

}  // namespace bl
