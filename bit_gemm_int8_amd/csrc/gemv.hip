// Decode ternary GEMV for a few tokens (M <= 4) with the fused dequant.
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T in an integer
// accumulator, then y = acc * beta*gamma/127 = acc * gamma / s.
//
// At batch 1 the product reads every packed weight once and does two integer
// ops per 1/4 byte, so the kernel is bound by HBM bandwidth.  Layout of the
// work (the packed layout is in include/bitlinear.h):
//   - one wave = 64 output rows (one packed row block), lane = row;
//   - per 256-input super-chunk a lane loads its row's 64 bytes as four
//     128-bit loads q = 0..3; each load instruction of the wave reads 1 KiB
//     of contiguous memory;
//   - all lanes work on the same inputs at the same time, so x~ comes from
//     uniform (scalar-cache) loads into SGPRs, used directly by v_dot4;
//   - a word unpacks to four int8 lanes of 64*W~ with one shift and one
//     mask, and v_dot4_i32_i8 accumulates; acc = sum >> 6 at the end;
//   - the grid splits K over `splits` waves per row block so that enough
//     waves stream at once; partial sums go to the workspace and the last
//     wave of the row block adds them and applies the epilogue.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

template <int M>
__device__ __forceinline__ void accumulate_chunk(const uint4 (&w)[4], const int* __restrict__ x32,
                                                 int64_t xstride, int acc[M]) {
  // word (q, j) = w[q].{x,y,z,w}[j]; inputs 64j + 16q + 4i + (0..3) of the
  // super-chunk; x~ dword index 16j + 4q + i.
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int* xr = x32 + m * xstride;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wq[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[m] = dot4(unpack_x64(wq[j], i), (uint32_t)xr[16 * j + 4 * q + i], acc[m]);
      }
    }
  }
}

template <int M>
__global__ __launch_bounds__(64) void gemv_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ scale,
    const uint4* __restrict__ packed, const float* __restrict__ gamma, int n, int nc,
    int64_t kpad, int splits, int relu2, int bf16, void* __restrict__ y,
    int32_t* __restrict__ acc_out, int32_t* __restrict__ partial,
    uint32_t* __restrict__ counters) {
  __shared__ uint32_t flag;
  const int b = blockIdx.x / splits;
  const int s = blockIdx.x - b * splits;
  const int lane = threadIdx.x;
  const int c0 = (int)((int64_t)s * nc / splits);
  const int c1 = (int)((int64_t)(s + 1) * nc / splits);
  const int64_t xstride = kpad / 4;                 // dwords per x~ row
  const int* x32 = reinterpret_cast<const int*>(xq);
  const uint4* blk = packed + (int64_t)b * nc * kBlockU4 + lane;

  int acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0;

  // two super-chunks in flight: load c+1 while c is consumed
  uint4 cur[4], nxt[4];
  if (c0 < c1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) cur[q] = blk[(int64_t)c0 * kBlockU4 + q * 64];
  }
  for (int c = c0; c < c1; ++c) {
    if (c + 1 < c1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) nxt[q] = blk[(int64_t)(c + 1) * kBlockU4 + q * 64];
    }
    accumulate_chunk<M>(cur, x32 + (int64_t)c * 64, xstride, acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
  }

  if (splits > 1) {
    int32_t* part = partial + ((int64_t)b * splits + s) * (M * 64);
#pragma unroll
    for (int m = 0; m < M; ++m) part[m * 64 + lane] = acc[m];
    if (!splitk_last_arrival(&counters[b], splits, &flag)) return;
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0;
    const int32_t* all = partial + (int64_t)b * splits * (M * 64);
    for (int t = 0; t < splits; ++t) {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] += __builtin_nontemporal_load(&all[(t * M + m) * 64 + lane]);
    }
  }

  const int64_t row = (int64_t)b * 64 + lane;
  if (row >= n) return;
  const float g = *gamma;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int a = acc[m] >> 6;                       // exact: every term is a multiple of 64
    if (acc_out != nullptr) acc_out[(int64_t)m * n + row] = a;
    store_out(y, (int64_t)m * n + row, a, gamma_over_s(g, scale[m]), relu2 != 0, bf16 != 0);
  }
}

}  // namespace

hipError_t launch_gemv(int m, const int8_t* xq, const float* scale, const uint32_t* packed,
                       const float* gamma, int64_t n, int64_t k, int splits, bool relu2,
                       bool bf16, void* y, int32_t* acc_out, int32_t* partial,
                       uint32_t* counters, hipStream_t stream) {
  const int nb = (int)cdiv(n, kRowBlock);
  const int nc = (int)cdiv(k, kSuperK);
  const int64_t kpad = padded_k(k);
  dim3 grid((unsigned)((int64_t)nb * splits)), block(64);
  const uint4* pk = reinterpret_cast<const uint4*>(packed);
#define BL_GEMV(MM)                                                                        \
  gemv_kernel<MM><<<grid, block, 0, stream>>>(xq, scale, pk, gamma, (int)n, nc, kpad,      \
                                              splits, relu2, bf16, y, acc_out, partial,   \
                                              counters)
  switch (m) {
    case 1: BL_GEMV(1); break;
    case 2: BL_GEMV(2); break;
    case 3: BL_GEMV(3); break;
    case 4: BL_GEMV(4); break;
    default: return hipErrorInvalidValue;
  }
#undef BL_GEMV
  return hipGetLastError();
}

}  // namespace bl
