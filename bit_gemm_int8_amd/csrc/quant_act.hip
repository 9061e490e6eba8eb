// Per-token absmax int8 activation quantization.
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "8-Bit
// Activation Quantization: absmax Scaling": beta = max_j |x_j| per token and
// x~ = Clip(Round(x * 127 / beta)); the page's listing clamps beta below at
// 1e-5, multiplies by 127/beta, rounds half to even and clamps to [-128, 127].
//
// One workgroup (4 waves) per token.  Pass 1 reduces max|x| with DPP inside
// each wave and LDS across waves; pass 2 re-reads the token (L2-resident: at
// most 2*K bytes) and writes x~ and the zero tail up to the padded row stride.
// The max is taken on the fp32 bit patterns with the sign cleared, which
// order like the magnitudes for finite values.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kThreads = 256;

template <bool BF16, bool VEC>
struct Row {
  // Elements per vector access: 16 bytes.
  static constexpr int kVec = VEC ? (BF16 ? 8 : 4) : 1;
};

__device__ __forceinline__ float load_elem(const void* x, int64_t i, bool bf16) {
  if (bf16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[i]);
  return reinterpret_cast<const float*>(x)[i];
}

__device__ __forceinline__ int8_t quantize(float v, float s) {
  float r = rintf(v * s);                 // one fp32 multiply, round half to even
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (int8_t)(int)r;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(
    const void* __restrict__ x, int64_t k, int64_t kpad, float eps,
    int8_t* __restrict__ xq, float* __restrict__ scale) {
  constexpr int V = Row<BF16, VEC>::kVec;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const char* xrow = reinterpret_cast<const char*>(x) + row * k * (BF16 ? 2 : 4);
  int8_t* qrow = xq + row * kpad;
  __shared__ uint32_t red[kThreads / 64];

  // ---- pass 1: max |x| ----
  uint32_t mx = 0;
  if (VEC) {
    const int64_t nvec = k / V;
    for (int64_t v = tid; v < nvec; v += kThreads) {
      uint4 u = reinterpret_cast<const uint4*>(xrow)[v];
      if (BF16) {
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t lo = (w[e] << 16) & 0x7FFFFFFFu;
          uint32_t hi = w[e] & 0x7FFF0000u;
          mx = mx > lo ? mx : lo;
          mx = mx > hi ? mx : hi;
        }
      } else {
        uint32_t w[4] = {u.x & 0x7FFFFFFFu, u.y & 0x7FFFFFFFu, u.z & 0x7FFFFFFFu,
                         u.w & 0x7FFFFFFFu};
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = mx > w[e] ? mx : w[e];
      }
    }
  } else {
    for (int64_t i = tid; i < k; i += kThreads) {
      uint32_t b = __float_as_uint(load_elem(xrow, i, BF16)) & 0x7FFFFFFFu;
      mx = mx > b ? mx : b;
    }
  }
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  uint32_t m01 = red[0] > red[1] ? red[0] : red[1];
  uint32_t m23 = red[2] > red[3] ? red[2] : red[3];
  const float beta = __uint_as_float(m01 > m23 ? m01 : m23);
  // s = 127 / max(beta, eps), correctly rounded to fp32.
  const float s = (float)(127.0 / (double)fmaxf(beta, eps));
  if (tid == 0) scale[row] = s;

  // ---- pass 2: quantize ----
  if (VEC) {
    const int64_t nvec = k / V;
    for (int64_t v = tid; v < nvec; v += kThreads) {
      uint4 u = reinterpret_cast<const uint4*>(xrow)[v];
      if (BF16) {
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
        uint32_t out[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t o = 0;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            uint32_t ww = w[2 * h + e];
            int8_t q0 = quantize(__uint_as_float(ww << 16), s);
            int8_t q1 = quantize(__uint_as_float(ww & 0xFFFF0000u), s);
            o |= ((uint32_t)(uint8_t)q0) << (16 * e);
            o |= ((uint32_t)(uint8_t)q1) << (16 * e + 8);
          }
          out[h] = o;
        }
        reinterpret_cast<uint2*>(qrow)[v] = make_uint2(out[0], out[1]);
      } else {
        float f[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                      __uint_as_float(u.w)};
        uint32_t o = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) o |= ((uint32_t)(uint8_t)quantize(f[e], s)) << (8 * e);
        reinterpret_cast<uint32_t*>(qrow)[v] = o;
      }
    }
  } else {
    for (int64_t i = tid; i < k; i += kThreads) qrow[i] = quantize(load_elem(xrow, i, BF16), s);
  }
  // zero tail up to the padded stride
  for (int64_t i = k + tid; i < kpad; i += kThreads) qrow[i] = 0;
}

}  // namespace

hipError_t launch_quant_act(const void* x, bool bf16, int64_t m, int64_t k, int64_t kpad,
                            float eps, int8_t* xq, float* scale, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  const size_t esz = bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)x % 16 == 0) && ((k * esz) % 16 == 0);
  dim3 grid((unsigned)m), block(kThreads);
  if (bf16) {
    if (vec)
      quant_act_kernel<true, true><<<grid, block, 0, stream>>>(x, k, kpad, eps, xq, scale);
    else
      quant_act_kernel<true, false><<<grid, block, 0, stream>>>(x, k, kpad, eps, xq, scale);
  } else {
    if (vec)
      quant_act_kernel<false, true><<<grid, block, 0, stream>>>(x, k, kpad, eps, xq, scale);
    else
      quant_act_kernel<false, false><<<grid, block, 0, stream>>>(x, k, kpad, eps, xq, scale);
  }
  return hipGetLastError();
}

}  // namespace bl
