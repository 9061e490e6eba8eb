// Per-token absmax int8 activation quantization.
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "8-Bit
// Activation Quantization: absmax Scaling": beta = max_j |x_j| per token and
// x~ = Clip(Round(x * 127 / beta)); the page's listing clamps beta below at
// 1e-5, multiplies by 127/beta, rounds half to even and clamps to [-128, 127].
//
// One workgroup (4 waves) per token.  max|x| is reduced with DPP inside each
// wave and LDS across waves, then x~ and the zero tail up to the padded row
// stride are written.  Rows of up to 16 16-byte vectors per thread (K <=
// 32768 bf16 or 16384 fp32, 16-byte aligned) are loaded into registers all at
// once and quantized from there (quant_act_reg_kernel); longer or unaligned
// rows are read twice, the second time from L2 (quant_act_kernel).  The max
// is taken on the fp32 bit patterns with the sign cleared, which order like
// the magnitudes for finite values.
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

// max of the sign-cleared fp32 bit patterns of one 16-byte vector
template <bool BF16>
__device__ __forceinline__ uint32_t vec_absmax_bits(const uint4& u, uint32_t mx) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (BF16) {
      const uint32_t lo = (w[e] << 16) & 0x7FFFFFFFu;
      const uint32_t hi = w[e] & 0x7FFF0000u;
      mx = mx > lo ? mx : lo;
      mx = mx > hi ? mx : hi;
    } else {
      const uint32_t b = w[e] & 0x7FFFFFFFu;
      mx = mx > b ? mx : b;
    }
  }
  return mx;
}

// x~ of one 16-byte input vector (vector index v of the row) into qrow
template <bool BF16>
__device__ __forceinline__ void vec_quant_store(const uint4& u, float s, int8_t* qrow,
                                                int64_t v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  if (BF16) {
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t o = 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t ww = w[2 * h + e];
        const int8_t q0 = quantize(__uint_as_float(ww << 16), s);
        const int8_t q1 = quantize(__uint_as_float(ww & 0xFFFF0000u), s);
        o |= ((uint32_t)(uint8_t)q0) << (16 * e);
        o |= ((uint32_t)(uint8_t)q1) << (16 * e + 8);
      }
      out[h] = o;
    }
    reinterpret_cast<uint2*>(qrow)[v] = make_uint2(out[0], out[1]);
  } else {
    uint32_t o = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o |= ((uint32_t)(uint8_t)quantize(__uint_as_float(w[e]), s)) << (8 * e);
    reinterpret_cast<uint32_t*>(qrow)[v] = o;
  }
}

// beta over the workgroup from each thread's partial max; s = 127 /
// max(beta, eps), correctly rounded to fp32
__device__ __forceinline__ float row_scale(uint32_t mx, float eps, uint32_t* red) {
  const int tid = threadIdx.x;
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  const uint32_t m01 = red[0] > red[1] ? red[0] : red[1];
  const uint32_t m23 = red[2] > red[3] ? red[2] : red[3];
  const float beta = __uint_as_float(m01 > m23 ? m01 : m23);
  return (float)(127.0 / (double)fmaxf(beta, eps));
}

// Rows of at most R vectors per thread, 16-byte aligned.
template <bool BF16, int R>
__global__ __launch_bounds__(kThreads) void quant_act_reg_kernel(
    const void* __restrict__ x, int64_t k, int64_t kpad, float eps,
    int8_t* __restrict__ xq, float* __restrict__ scale) {
  constexpr int V = BF16 ? 8 : 4;                   // elements per vector
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint4* xrow = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) +
                                                     row * k * (BF16 ? 2 : 4));
  int8_t* qrow = xq + row * kpad;
  __shared__ uint32_t red[kThreads / 64];
  const int nvec = (int)(k / V);
  uint4 u[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int v = tid + kThreads * i;
    u[i] = v < nvec ? xrow[v] : make_uint4(0, 0, 0, 0);
  }
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) mx = vec_absmax_bits<BF16>(u[i], mx);
  const float s = row_scale(mx, eps, red);
  if (tid == 0) scale[row] = s;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int v = tid + kThreads * i;
    if (v < nvec) vec_quant_store<BF16>(u[i], s, qrow, v);
  }
  for (int64_t i = k + tid; i < kpad; i += kThreads) qrow[i] = 0;
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
    for (int64_t v = tid; v < nvec; v += kThreads)
      mx = vec_absmax_bits<BF16>(reinterpret_cast<const uint4*>(xrow)[v], mx);
  } else {
    for (int64_t i = tid; i < k; i += kThreads) {
      uint32_t b = __float_as_uint(load_elem(xrow, i, BF16)) & 0x7FFFFFFFu;
      mx = mx > b ? mx : b;
    }
  }
  const float s = row_scale(mx, eps, red);
  if (tid == 0) scale[row] = s;

  // ---- pass 2: quantize ----
  if (VEC) {
    const int64_t nvec = k / V;
    for (int64_t v = tid; v < nvec; v += kThreads)
      vec_quant_store<BF16>(reinterpret_cast<const uint4*>(xrow)[v], s, qrow, v);
  } else {
    for (int64_t i = tid; i < k; i += kThreads) qrow[i] = quantize(load_elem(xrow, i, BF16), s);
  }
  // zero tail up to the padded stride
  for (int64_t i = k + tid; i < kpad; i += kThreads) qrow[i] = 0;
}

// ---------------------------------------------------------------- RMSNorm --
// x -> y = x * r * w with r = 1 / sqrt(mean(x^2) + norm_eps) per token, then
// the absmax quantization of y.  "BitNet b1.58 2B4T Guide", the BitLinear
// listing in "End-to-End Implementation: Building a Native BitLinear Layer"
// normalises x with RMSNorm before quantize_activations_int8.  One workgroup
// per token, three passes over the row (the second and third from cache):
// the fp64 sum of squares, max|y|, and x~ = clamp(rint(fp32(y * s))).
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  const int tid = threadIdx.x;
  v = wave_sum_f64(v);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  double t = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) t += red[w];
  return t;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void rmsnorm_quant_kernel(
    const void* __restrict__ x, int64_t k, int64_t kpad, const float* __restrict__ nw,
    float neps, float eps, int8_t* __restrict__ xq, float* __restrict__ scale) {
  constexpr int V = Row<BF16, VEC>::kVec;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const char* xrow = reinterpret_cast<const char*>(x) + row * k * (BF16 ? 2 : 4);
  int8_t* qrow = xq + row * kpad;
  __shared__ double red64[kThreads / 64];
  __shared__ uint32_t red[kThreads / 64];
  auto xval = [&](int64_t i) __attribute__((always_inline)) { return load_elem(xrow, i, BF16); };
  auto wval = [&](int64_t i) __attribute__((always_inline)) { return nw ? nw[i] : 1.0f; };

  // ---- pass 1: sum of squares (fp64) ----
  double ss = 0.0;
  for (int64_t i = (int64_t)tid * V; i < k; i += (int64_t)kThreads * V) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const double v = (double)xval(i + e);
      ss += v * v;
    }
  }
  const float r = rms_factor(block_sum_f64(ss, red64), (int)k, neps);

  // ---- pass 2: max |y| ----
  uint32_t mx = 0;
  for (int64_t i = (int64_t)tid * V; i < k; i += (int64_t)kThreads * V) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const uint32_t b = __float_as_uint(rms_apply(xval(i + e), r, wval(i + e))) & 0x7FFFFFFFu;
      mx = mx > b ? mx : b;
    }
  }
  const float s = row_scale(mx, eps, red);
  if (tid == 0) scale[row] = s;

  // ---- pass 3: quantize y ----
  for (int64_t i = (int64_t)tid * V; i < k; i += (int64_t)kThreads * V) {
#pragma unroll
    for (int e = 0; e < V; ++e) qrow[i + e] = quantize(rms_apply(xval(i + e), r, wval(i + e)), s);
  }
  for (int64_t i = k + tid; i < kpad; i += kThreads) qrow[i] = 0;
}

// The same for rows of whole 16-byte vectors at 16-byte alignment, at most R
// per thread, with a 16-byte aligned gain (or none): each thread loads its
// vectors (and their gain) once and keeps them in registers, so the three
// passes wait for memory once.  The fp64 sum runs in the same order as
// rmsnorm_quant_kernel's (vector v of the row on thread v % 256, each
// thread's vectors and their elements in order, then block_sum_f64), and
// every other step is the same, so the two give the same bits.
template <bool BF16, int R>
__global__ __launch_bounds__(kThreads) void rmsnorm_quant_reg_kernel(
    const void* __restrict__ x, int64_t k, int64_t kpad, const float* __restrict__ nw,
    float neps, float eps, int8_t* __restrict__ xq, float* __restrict__ scale) {
  constexpr int V = BF16 ? 8 : 4;                   // elements per vector
  constexpr int G = V / 4;                          // gain vectors per input vector
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint4* xrow = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) +
                                                     row * k * (BF16 ? 2 : 4));
  int8_t* qrow = xq + row * kpad;
  __shared__ double red64[kThreads / 64];
  __shared__ uint32_t red[kThreads / 64];
  const int nvec = (int)(k / V);
  // loads with clamped indices and no branch (past the row the values are
  // replaced by zeros below); without a gain the gain loads read x, unused
  const uint4* gsrc = nw != nullptr ? reinterpret_cast<const uint4*>(nw) : xrow;
  uint4 u[R], gv[R][G];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int v = min(tid + kThreads * i, nvec - 1);
    u[i] = xrow[v];
#pragma unroll
    for (int h = 0; h < G; ++h) gv[i][h] = gsrc[nw != nullptr ? v * G + h : 0];
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (tid + kThreads * i >= nvec) u[i] = make_uint4(0u, 0u, 0u, 0u);
  auto vals = [&](int i, float (&f)[8]) __attribute__((always_inline)) {
    const uint32_t w[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (BF16) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      } else {
        f[e] = __uint_as_float(w[e]);
      }
    }
  };
  auto gains = [&](int i, float (&g)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      g[4 * h] = __uint_as_float(gv[i][h].x); g[4 * h + 1] = __uint_as_float(gv[i][h].y);
      g[4 * h + 2] = __uint_as_float(gv[i][h].z); g[4 * h + 3] = __uint_as_float(gv[i][h].w);
    }
    if (nw == nullptr) {
#pragma unroll
      for (int e = 0; e < V; ++e) g[e] = 1.0f;
    }
  };

  // ---- pass 1: sum of squares (fp64) ----
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (tid + kThreads * i < nvec) {
      float f[8];
      vals(i, f);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const double d = (double)f[e];
        ss += d * d;
      }
    }
  }
  const float r = rms_factor(block_sum_f64(ss, red64), (int)k, neps);

  // ---- pass 2: max |y| ----
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float f[8], g[8];
    vals(i, f);
    gains(i, g);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const uint32_t b = __float_as_uint(rms_apply(f[e], r, g[e])) & 0x7FFFFFFFu;
      mx = mx > b ? mx : b;
    }
  }
  const float s = row_scale(mx, eps, red);
  if (tid == 0) scale[row] = s;

  // ---- pass 3: quantize y (recomputed from the held row, not kept) ----
#pragma unroll
  for (int i = 0; i < R; ++i)
    asm volatile("" : "+v"(u[i].x), "+v"(u[i].y), "+v"(u[i].z), "+v"(u[i].w));
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int v = tid + kThreads * i;
    if (v < nvec) {
      float f[8], g[8];
      vals(i, f);
      gains(i, g);
      uint32_t o[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < V; ++e)
        o[e >> 2] |= ((uint32_t)(uint8_t)quantize(rms_apply(f[e], r, g[e]), s)) << (8 * (e & 3));
      if (BF16)
        reinterpret_cast<uint2*>(qrow)[v] = make_uint2(o[0], o[1]);
      else
        reinterpret_cast<uint32_t*>(qrow)[v] = o[0];
    }
  }
  for (int64_t i = k + tid; i < kpad; i += kThreads) qrow[i] = 0;
}

}  // namespace

hipError_t launch_rmsnorm_quant(const void* x, bool bf16, int64_t m, int64_t k, int64_t kpad,
                                const float* norm_weight, float norm_eps, float eps, int8_t* xq,
                                float* scale, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  dim3 grid((unsigned)m), block(kThreads);
  // V elements per thread and step when a row splits into whole groups of V
  const bool vec = (k % (bf16 ? 8 : 4)) == 0;
  // rows held in registers: whole aligned vectors, an aligned gain (or none)
  if (vec && (uintptr_t)x % 16 == 0 && (uintptr_t)norm_weight % 16 == 0) {
    const int64_t per = cdiv(k / (bf16 ? 8 : 4), kThreads);   // vectors per thread
#define BL_RQREG(R)                                                                       \
  do {                                                                                    \
    if (bf16)                                                                             \
      rmsnorm_quant_reg_kernel<true, R><<<grid, block, 0, stream>>>(                      \
          x, k, kpad, norm_weight, norm_eps, eps, xq, scale);                             \
    else                                                                                  \
      rmsnorm_quant_reg_kernel<false, R><<<grid, block, 0, stream>>>(                     \
          x, k, kpad, norm_weight, norm_eps, eps, xq, scale);                             \
    return hipGetLastError();                                                             \
  } while (0)
    if (per <= 1) BL_RQREG(1);
    if (per <= 2) BL_RQREG(2);
    if (per <= 4) BL_RQREG(4);
    if (per <= 8) BL_RQREG(8);
    if (per <= 16) BL_RQREG(16);
#undef BL_RQREG
  }
  if (bf16) {
    if (vec)
      rmsnorm_quant_kernel<true, true><<<grid, block, 0, stream>>>(x, k, kpad, norm_weight,
                                                                   norm_eps, eps, xq, scale);
    else
      rmsnorm_quant_kernel<true, false><<<grid, block, 0, stream>>>(x, k, kpad, norm_weight,
                                                                    norm_eps, eps, xq, scale);
  } else {
    if (vec)
      rmsnorm_quant_kernel<false, true><<<grid, block, 0, stream>>>(x, k, kpad, norm_weight,
                                                                    norm_eps, eps, xq, scale);
    else
      rmsnorm_quant_kernel<false, false><<<grid, block, 0, stream>>>(x, k, kpad, norm_weight,
                                                                     norm_eps, eps, xq, scale);
  }
  return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, bool bf16, int64_t m, int64_t k, int64_t kpad,
                            float eps, int8_t* xq, float* scale, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  const size_t esz = bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)x % 16 == 0) && ((k * esz) % 16 == 0);
  dim3 grid((unsigned)m), block(kThreads);
  if (vec) {
    const int64_t per = cdiv(k * (int64_t)esz / 16, kThreads);   // vectors per thread
#define BL_QREG(R)                                                                           \
  do {                                                                                       \
    if (bf16)                                                                                \
      quant_act_reg_kernel<true, R><<<grid, block, 0, stream>>>(x, k, kpad, eps, xq, scale); \
    else                                                                                     \
      quant_act_reg_kernel<false, R><<<grid, block, 0, stream>>>(x, k, kpad, eps, xq, scale); \
    return hipGetLastError();                                                                \
  } while (0)
    if (per <= 1) BL_QREG(1);
    if (per <= 2) BL_QREG(2);
    if (per <= 4) BL_QREG(4);
    if (per <= 8) BL_QREG(8);
    if (per <= 16) BL_QREG(16);
#undef BL_QREG
  }
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
