// Decode ternary GEMV for a few tokens (M <= 4) with the fused dequant, and
// the fused decode step (activation quantization + GEMV for several matrices
// in one launch).
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T in an integer
// accumulator, then y = acc * beta*gamma/127 = acc * gamma / s; section
// "8-Bit Activation Quantization: absmax Scaling" for x~ and s.
//
// At batch 1 the product reads every packed weight once and does two integer
// ops per 1/4 byte, so the kernel is bound by HBM bandwidth.  Layout of the
// work (the packed layout is in include/bitlinear.h):
//   - a workgroup owns one 64-row packed block (lane = row) and WAVES waves
//     split its 256-input super-chunks into contiguous ranges;
//   - per super-chunk a lane loads its row's 64 bytes as four 128-bit loads
//     q = 0..3; each load instruction of a wave reads 1 KiB of contiguous
//     memory, and PF super-chunks per wave are in flight at once;
//   - all lanes of a wave work on the same inputs: the workgroup puts its
//     slice of x~ in LDS once (after issuing its first weight loads) and the
//     lanes read it at one shared address, which the LDS broadcasts;
//   - a word unpacks to four int8 lanes of 64*W~ with one shift and one mask;
//     acc = sum >> 6 at the end (every term is a multiple of 64);
//   - the waves' sums meet in LDS; when the row blocks alone cannot fill the
//     chip, `splits` workgroups share a row block and add into the workspace
//     with device-scope atomics (no cache-wide fences).
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

// One super-chunk: w = the lane's four 16-byte loads q = 0..3 (word (q, j) =
// w[q].{x,y,z,w}[j], inputs 64j + 16q + 4i + (0..3)), xs = this super-chunk's
// 256 bytes of x~ for each token in LDS (token stride xs_stride dwords).
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

template <int PF>
__device__ __forceinline__ void prefetch_first(uint4 (&buf)[PF][4], const uint4* blk, int c0,
                                               int c1) {
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    if (c0 + p < c1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) buf[p][q] = blk[(int64_t)(c0 + p) * kBlockU4 + q * 64];
    }
  }
}

// Stream super-chunks c0..c1-1 (the first PF already in buf); x~ in LDS
// starts at super-chunk g0.
template <int M, int PF>
__device__ __forceinline__ void stream_chunks(uint4 (&buf)[PF][4], const uint4* blk, int c0,
                                              int c1, int g0, const uint32_t* xs, int xs_stride,
                                              int (&acc)[M]) {
  for (int c = c0; c < c1; c += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (c + p < c1) {
        accumulate_chunk<M>(buf[p], xs + (c + p - g0) * 64, xs_stride, acc);
        if (c + p + PF < c1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) buf[p][q] = blk[(int64_t)(c + p + PF) * kBlockU4 + q * 64];
        }
      }
    }
  }
}

// Sum the waves' accumulators into wave 0.  Returns false in other waves.
template <int M, int WAVES>
__device__ __forceinline__ bool reduce_waves(int (&acc)[M], int (*red)[M][64], int wave,
                                             int lane) {
  if (WAVES == 1) return true;
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) red[wave - 1][m][lane] = acc[m];
  }
  __syncthreads();
  if (wave > 0) return false;
#pragma unroll
  for (int w = 0; w < WAVES - 1; ++w)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] += red[w][m][lane];
  return true;
}

// Workgroups that share a row block add their sums into the workspace
// accumulator with device-scope atomics; each add returns, so it has been
// performed before this group bumps the block's counter.  The group that
// brings the counter to `splits` reads the totals with device-scope atomic
// loads and clears them and the counter for the next call.  Wave 0 only;
// returns true in the group that finishes the block.
template <int M>
__device__ __forceinline__ bool combine_splits(int (&acc)[M], int32_t* slot, uint32_t* counter,
                                               int splits, int lane) {
  int done = 0;
#pragma unroll
  for (int m = 0; m < M; ++m)
    done |= __hip_atomic_fetch_add(slot + m * 64, acc[m], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::"v"(done));                    // the returned values are in
  uint32_t prev = 0;
  if (lane == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
  if (prev != (uint32_t)(splits - 1)) return false;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    acc[m] = __hip_atomic_load(slot + m * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slot + m * 64, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

template <int M>
__device__ __forceinline__ void write_rows(const int (&acc)[M], const float (&fac)[M], int64_t row,
                                           int n, void* y, int32_t* acc_out, bool relu2,
                                           bool bf16) {
  if (row >= n) return;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int a = acc[m] >> 6;                       // exact: every term is a multiple of 64
    if (acc_out != nullptr) acc_out[(int64_t)m * n + row] = a;
    store_out(y, (int64_t)m * n + row, a, fac[m], relu2, bf16);
  }
}

// ------------------------------------------------------------ plain GEMV --
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

  uint4 buf[PF][4];
  prefetch_first<PF>(buf, blk, c0, c1);
  // epilogue operands, loaded now so their latency hides under the stream
  const float g = *gamma;
  float fac[M];
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = scale[m];
  int acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0;

  // stage x~[m][256*g0 .. 256*g1) for every token (16 units of 16 bytes per
  // super-chunk and token)
  const int span = (g1 - g0) * 16;                  // uint4 per token
  for (int u = threadIdx.x; u < span * M; u += 64 * WAVES) {
    const int m = u / span, v = u - m * span;
    xs_lds[u] = reinterpret_cast<const uint4*>(xq + (int64_t)m * kpad + (int64_t)g0 * 256)[v];
  }
  __syncthreads();
  stream_chunks<M, PF>(buf, blk, c0, c1, g0, reinterpret_cast<const uint32_t*>(xs_lds), span * 4,
                       acc);
  if (!reduce_waves<M, WAVES>(acc, red, wave, lane)) return;
  if (splits > 1 &&
      !combine_splits<M>(acc, ws_acc + (int64_t)b * (M * 64) + lane, &counters[b], splits, lane))
    return;
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = gamma_over_s(g, fac[m]);
  write_rows<M>(acc, fac, (int64_t)b * 64 + lane, n, y, acc_out, relu2 != 0, bf16 != 0);
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

// ---------------------------------------------------- fused decode step --
// Each workgroup reads its segment's activations x (fp32/bf16), computes the
// token's absmax over all K with DPP wave reductions and LDS, s = 127/max(beta,
// eps), and writes x~ = clamp(rint(x*s)) for its own super-chunks straight
// into LDS: every group of a segment computes the same s and x~ bit for bit.

template <int WAVES>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) r = r > red[w] ? r : red[w];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t quant1(float v, float s) {
  float r = rintf(v * s);                            // one fp32 multiply, half to even
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (uint32_t)(uint8_t)(int8_t)(int)r;
}

__device__ __forceinline__ uint32_t quant4(const float (&f)[4], float s) {
  return quant1(f[0], s) | (quant1(f[1], s) << 8) | (quant1(f[2], s) << 16) |
         (quant1(f[3], s) << 24);
}

template <int M, int WAVES>
__device__ __forceinline__ void quantize_into_lds(const FusedSeg& sg, int g0, int g1, float eps,
                                                  uint32_t* xs_words, float (&sv)[M],
                                                  uint32_t* red) {
  const int k = sg.k;
  const bool bf16 = sg.x_bf16 != 0;
  // vector path: 4 consecutive elements per access, aligned
  const bool vec = (k % 4 == 0) && (((uintptr_t)sg.x % (bf16 ? 8 : 16)) == 0);
  const int span_w = (g1 - g0) * 64;                // dwords of x~ per token
  for (int m = 0; m < M; ++m) {
    const char* row = reinterpret_cast<const char*>(sg.x) + (int64_t)m * k * (bf16 ? 2 : 4);
    uint32_t mx = 0;
    if (vec) {
      for (int v = threadIdx.x; v < k / 4; v += 64 * WAVES) {
        uint32_t e[4];
        if (bf16) {
          const uint2 u = reinterpret_cast<const uint2*>(row)[v];
          e[0] = u.x << 16; e[1] = u.x & 0xFFFF0000u; e[2] = u.y << 16; e[3] = u.y & 0xFFFF0000u;
        } else {
          const uint4 u = reinterpret_cast<const uint4*>(row)[v];
          e[0] = u.x; e[1] = u.y; e[2] = u.z; e[3] = u.w;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t a = e[t] & 0x7FFFFFFFu;
          mx = mx > a ? mx : a;
        }
      }
    } else {
      for (int i = threadIdx.x; i < k; i += 64 * WAVES) {
        const float f = bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[i])
                             : reinterpret_cast<const float*>(row)[i];
        const uint32_t a = __float_as_uint(f) & 0x7FFFFFFFu;
        mx = mx > a ? mx : a;
      }
    }
    const float beta = __uint_as_float(group_max_u32<WAVES>(mx, red));
    const float s = (float)(127.0 / (double)fmaxf(beta, eps));
    sv[m] = s;
    // x~ for inputs 256*g0 + 4*d .. +3, d < span_w; zero past K
    for (int d = threadIdx.x; d < span_w; d += 64 * WAVES) {
      const int k0 = g0 * 256 + 4 * d;
      float f[4];
      if (vec) {
        if (k0 < k) {
          if (bf16) {
            const uint2 u = reinterpret_cast<const uint2*>(row)[k0 / 4];
            f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xFFFF0000u);
            f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xFFFF0000u);
          } else {
            const float4 u = reinterpret_cast<const float4*>(row)[k0 / 4];
            f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
          }
        } else {
          f[0] = f[1] = f[2] = f[3] = 0.0f;
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kk = k0 + t;
          f[t] = kk < k ? (bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[kk])
                                : reinterpret_cast<const float*>(row)[kk])
                        : 0.0f;
        }
      }
      xs_words[m * span_w + d] = quant4(f, s);
    }
  }
}

template <int M, int WAVES, int PF>
__global__ __launch_bounds__(64 * WAVES) void gemv_fused_kernel(FusedArgs args) {
  __shared__ int red[WAVES > 1 ? WAVES - 1 : 1][M][64];
  __shared__ uint32_t red_max[WAVES];
  extern __shared__ uint4 xs_lds[];
  // segment of this workgroup
  int si = 0;
  for (int i = 1; i < args.nseg; ++i)
    if ((int)blockIdx.x >= args.seg[i].wg_begin) si = i;
  const FusedSeg& sg = args.seg[si];
  const int local = (int)blockIdx.x - sg.wg_begin;
  const int splits = sg.splits;
  const int b = local / splits;
  const int s = local - b * splits;
  const int nc = sg.nc;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g0 = (int)((int64_t)s * nc / splits);
  const int g1 = (int)((int64_t)(s + 1) * nc / splits);
  const int c0 = g0 + (int)((int64_t)wave * (g1 - g0) / WAVES);
  const int c1 = g0 + (int)((int64_t)(wave + 1) * (g1 - g0) / WAVES);
  const uint4* blk =
      reinterpret_cast<const uint4*>(sg.packed) + (int64_t)b * nc * kBlockU4 + lane;

  uint4 buf[PF][4];
  prefetch_first<PF>(buf, blk, c0, c1);
  const float g = *sg.gamma;
  int acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0;

  uint32_t* xs_words = reinterpret_cast<uint32_t*>(xs_lds);
  float sv[M];
  quantize_into_lds<M, WAVES>(sg, g0, g1, args.eps, xs_words, sv, red_max);
  __syncthreads();
  const int span_w = (g1 - g0) * 64;
  // optional copies of x~ and s (row block 0's groups cover all of K_pad)
  if (b == 0 && sg.xq_out != nullptr) {
    const int64_t kpad = (int64_t)nc * 256;
    for (int m = 0; m < M; ++m)
      for (int d = threadIdx.x; d < span_w; d += 64 * WAVES)
        reinterpret_cast<uint32_t*>(sg.xq_out + (int64_t)m * kpad + (int64_t)g0 * 256)[d] =
            xs_words[m * span_w + d];
  }
  if (b == 0 && s == 0 && sg.scale_out != nullptr && threadIdx.x == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) sg.scale_out[m] = sv[m];
  }

  stream_chunks<M, PF>(buf, blk, c0, c1, g0, xs_words, span_w, acc);
  if (!reduce_waves<M, WAVES>(acc, red, wave, lane)) return;
  if (splits > 1 &&
      !combine_splits<M>(acc, sg.ws_acc + (int64_t)b * (M * 64) + lane, &sg.counters[b], splits,
                         lane))
    return;
  float fac[M];
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = gamma_over_s(g, sv[m]);
  write_rows<M>(acc, fac, (int64_t)b * 64 + lane, sg.n, sg.y, sg.acc_out, sg.relu2 != 0,
                sg.y_bf16 != 0);
}

}  // namespace

// Plain GEMV: x~ and s given.
hipError_t launch_gemv(int m, int waves, const int8_t* xq, const float* scale,
                       const uint32_t* packed, const float* gamma, int64_t n, int64_t k,
                       int splits, bool relu2, bool bf16, void* y, int32_t* acc_out,
                       int32_t* ws_acc, uint32_t* counters, hipStream_t stream) {
#define BL_GEMV(MM, WW)                                                                        \
  return run_gemv<MM, WW, (WW >= 16 ? 1 : 2)>(xq, scale, packed, gamma, n, k, splits, relu2, \
                                              bf16, y, acc_out, ws_acc, counters, stream)
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

// Fused decode step over a complete segment table (wg_begin, splits and
// workspace pointers filled in).
hipError_t launch_gemv_fused(const FusedArgs& args, int m, int waves, int groups, size_t lds,
                             hipStream_t stream) {
#define BL_FUSED(MM, WW)                                                             \
  do {                                                                               \
    gemv_fused_kernel<MM, WW, 2><<<(unsigned)groups, 64 * WW, lds, stream>>>(args); \
    return hipGetLastError();                                                        \
  } while (0)
#define BL_FUSED_W(MM)     \
  if (waves == 4)          \
    BL_FUSED(MM, 4);       \
  else                     \
    BL_FUSED(MM, 8)
  switch (m) {
    case 1: BL_FUSED_W(1);
    case 2: BL_FUSED_W(2);
    case 3: BL_FUSED_W(3);
    case 4: BL_FUSED_W(4);
    default: return hipErrorInvalidValue;
  }
#undef BL_FUSED_W
#undef BL_FUSED
}

}  // namespace bl
