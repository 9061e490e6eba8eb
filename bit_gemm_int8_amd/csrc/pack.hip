// Absmean ternary weight quantization and 2-bit packing.
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Ternary
// Weight Quantization: absmean Scaling": gamma = mean |W_ij| over the whole
// d_out x d_in tensor, W~ = Clip(Round(W / (gamma + eps)), -1, 1).  The
// packed layout is the one in include/bitlinear.h.
//
// Two launches, no host synchronisation:
//   1. absum_partial_kernel: each workgroup sums |W| over a fixed contiguous
//      slice in fp64 (fixed per-thread order, then a fixed shuffle/LDS tree)
//      and writes one partial.
//   2. pack_kernel: every workgroup sums the partials in the same fixed order
//      (so all agree on gamma bit for bit), derives the decision threshold,
//      and packs one 4 KiB block (64 rows x 256 inputs).
//
// Code decision without a division.  For fp32 w >= 0 and d = fp32(gamma+eps),
// rint(fp32(w/d)) >= 1 exactly when fp32(w/d) > 0.5, and fp32(q) > 0.5 exactly
// when q > 0.5 + 2^-25 (the fp32 neighbours of 0.5 are 0.5 - 2^-25 and
// 0.5 + 2^-24; the midpoint 0.5 + 2^-25 rounds to 0.5, whose significand is
// even).  So the code is +1 iff w > T with T = d * (0.5 + 2^-25), a product
// that is exact in fp64 (24 + 25 significant bits).  As w is fp32, w > T iff
// w > T32, T32 = the largest fp32 <= T.  Negative weights mirror this
// (division and round-half-even are odd functions), and a clip at +-1 means
// larger ratios change nothing.  If d == 0 (eps = 0, gamma = 0) all codes are 0.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxParts = 1024;

__device__ __forceinline__ double block_sum_f64(double v, double* lds) {
  // wave: fixed butterfly
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) lds[tid >> 6] = v;
  __syncthreads();
  double s = (lds[0] + lds[1]) + (lds[2] + lds[3]);
  __syncthreads();
  return s;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void absum_partial_kernel(
    const void* __restrict__ w, int64_t total, int64_t per_block, double* __restrict__ partial) {
  __shared__ double lds[kThreads / 64];
  const int64_t beg = (int64_t)blockIdx.x * per_block;
  const int64_t end = beg + per_block < total ? beg + per_block : total;
  constexpr int V = BF16 ? 8 : 4;   // elements per 16-byte vector
  double acc = 0.0;
  for (int64_t e = beg + (int64_t)threadIdx.x * V; e < end; e += (int64_t)kThreads * V) {
    if (e + V <= end) {
      uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(w) +
                                                 e * (BF16 ? 2 : 4));
      uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (BF16) {
          acc += (double)fabsf(__uint_as_float(ww[t] << 16));
          acc += (double)fabsf(__uint_as_float(ww[t] & 0xFFFF0000u));
        } else {
          acc += (double)fabsf(__uint_as_float(ww[t]));
        }
      }
    } else {
      for (int64_t i = e; i < end; ++i) {
        float f = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(w)[i])
                       : reinterpret_cast<const float*>(w)[i];
        acc += (double)fabsf(f);
      }
    }
  }
  double s = block_sum_f64(acc, lds);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

__device__ __forceinline__ uint32_t field_of(float v, float t32) {
  // +1 -> 01, -1 -> 11, 0 -> 00
  return v > t32 ? 1u : (v < -t32 ? 3u : 0u);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void pack_kernel(
    const void* __restrict__ w, int64_t n, int64_t k, int nc, float eps,
    const float* __restrict__ gamma_in, const double* __restrict__ partial, int nparts,
    int64_t total, float* __restrict__ gamma_out, uint32_t* __restrict__ packed) {
  __shared__ double lds[kThreads / 64];
  float gamma;
  if (gamma_in != nullptr) {
    gamma = *gamma_in;
  } else {
    double a = 0.0;
    for (int i = threadIdx.x; i < nparts; i += kThreads) a += partial[i];
    double s = block_sum_f64(a, lds);
    gamma = (float)(s / (double)total);
  }
  const int64_t blk = blockIdx.x;           // = b * nc + c
  if (blk == 0 && threadIdx.x == 0) *gamma_out = gamma;

  const float d = gamma + eps;               // fp32 addition
  float t32;
  if (!(d > 0.0f)) {
    t32 = __builtin_huge_valf();             // d == 0: every code is 0
  } else {
    const double T = (double)d * (0.5 + 0x1p-25);
    t32 = (float)T;
    if ((double)t32 > T) t32 = __uint_as_float(__float_as_uint(t32) - 1u);
  }

  const int b = (int)(blk / nc);
  const int c = (int)(blk % nc);
  const int r = threadIdx.x >> 2;            // row in block
  const int j = threadIdx.x & 3;             // 64-input group in the super-chunk
  const int64_t row = (int64_t)b * kRowBlock + r;
  const int64_t k0 = (int64_t)c * kSuperK + 64 * j;

  // 64 consecutive weights of one row: k0 .. k0+63
  float v[64];
  const bool full = row < n && k0 + 64 <= k && (BF16 ? (k % 8 == 0) : (k % 4 == 0));
  if (full) {
    const char* base = reinterpret_cast<const char*>(w) + (row * k + k0) * (BF16 ? 2 : 4);
    if (BF16) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        uint4 u = reinterpret_cast<const uint4*>(base)[p];
        uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[8 * p + 2 * t] = __uint_as_float(ww[t] << 16);
          v[8 * p + 2 * t + 1] = __uint_as_float(ww[t] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        float4 f = reinterpret_cast<const float4*>(base)[p];
        v[4 * p] = f.x; v[4 * p + 1] = f.y; v[4 * p + 2] = f.z; v[4 * p + 3] = f.w;
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 64; ++t) {
      const int64_t kk = k0 + t;
      float f = 0.0f;
      if (row < n && kk < k)
        f = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(w)[row * k + kk])
                 : reinterpret_cast<const float*>(w)[row * k + kk];
      v[t] = f;
    }
  }

  // word (q) holds inputs 16q + t of this 64-group, t at bits 8(t%4) + 2(t/4)
  uint32_t* out = packed + blk * 1024;       // 4 KiB block = 1024 words
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      word |= field_of(v[16 * q + t], t32) << (8 * (t & 3) + 2 * (t >> 2));
    out[(q * 64 + r) * 4 + j] = word;
  }
}

}  // namespace

PackPlan pack_plan(int64_t n, int64_t k) {
  PackPlan p;
  p.total = n * k;
  int64_t parts = cdiv(p.total, 8192);
  if (parts > kMaxParts) parts = kMaxParts;
  if (parts < 1) parts = 1;
  int64_t per = cdiv(p.total, parts);
  per = cdiv(per, 2048) * 2048;              // multiple of 256 threads x 8 elements
  p.per_block = per;
  p.nparts = (int)cdiv(p.total, per);
  return p;
}

size_t pack_workspace_bytes(int64_t, int64_t) { return (size_t)kMaxParts * sizeof(double); }

hipError_t launch_pack(const void* w, bool bf16, int64_t n, int64_t k, float eps,
                       const float* gamma_in, uint32_t* packed, float* gamma_out,
                       double* partial, hipStream_t stream) {
  const PackPlan p = pack_plan(n, k);
  const int nb = (int)cdiv(n, kRowBlock);
  const int nc = (int)cdiv(k, kSuperK);
  if (gamma_in == nullptr) {
    if (bf16)
      absum_partial_kernel<true><<<p.nparts, kThreads, 0, stream>>>(w, p.total, p.per_block, partial);
    else
      absum_partial_kernel<false><<<p.nparts, kThreads, 0, stream>>>(w, p.total, p.per_block, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = (int64_t)nb * nc;
  if (bf16)
    pack_kernel<true><<<(unsigned)blocks, kThreads, 0, stream>>>(
        w, n, k, nc, eps, gamma_in, partial, p.nparts, p.total, gamma_out, packed);
  else
    pack_kernel<false><<<(unsigned)blocks, kThreads, 0, stream>>>(
        w, n, k, nc, eps, gamma_in, partial, p.nparts, p.total, gamma_out, packed);
  return hipGetLastError();
}

}  // namespace bl
