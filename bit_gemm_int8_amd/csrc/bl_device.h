// Device helpers shared by the libbitlinear kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

typedef int32_t bl_v4i __attribute__((ext_vector_type(4)));
typedef int32_t bl_v16i __attribute__((ext_vector_type(16)));
typedef uint16_t bl_u16x2 __attribute__((ext_vector_type(2)));

namespace bl {

// f(std::integral_constant<int, 0>{}), ..., f(<N - 1>): array slots chosen
// at compile time stay in registers
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// 16 bytes of packed weights, which a product reads exactly once: a
// non-temporal load (the "nt" cache policy), so the stream does not
// displace reusable lines from the caches.  Measured on MI355X: a 58.7 MB
// read in the GEMV's access pattern streams at 6.1 TB/s this way against
// 5.7 TB/s with ordinary loads.
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
  const bl_v4i v = __builtin_nontemporal_load(reinterpret_cast<const bl_v4i*>(p));
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

constexpr int kRowBlock = 64;     // rows per packed block
constexpr int kSuperK = 256;      // inputs per packed super-chunk
constexpr int kBlockU4 = 256;     // uint4 per 4 KiB packed block

// Four weights t = 4i..4i+3 of a packed word, as int8 lanes holding 64*W~.
// Code t sits at bits 8*(t%4) + 2*(t/4); shifting left by 6-2i brings the
// pair for t = 4i+e to the top two bits of byte e, and the mask drops the
// rest.  A two's complement 2-bit field at the top of a byte reads as
// 64 * field when the byte is taken as int8: 01 -> 64, 11 -> -64, 00 -> 0.
__device__ __forceinline__ uint32_t unpack_x64(uint32_t w, int i) {
  return (w << (6 - 2 * i)) & 0xC0C0C0C0u;
}

// Signed int8 dot product of four byte lanes, accumulated into c.
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// fp32 -> bf16 bits, round to nearest even (finite input).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> two bf16 (round to nearest even) packed low/high, one
// v_cvt_pk_bf16_f32.
typedef __bf16 bl_bf16x2 __attribute__((ext_vector_type(2)));
typedef float bl_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bl_f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bl_bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Max over each row of 16 lanes with DPP lane permutations; every lane of
// the row ends with the row's maximum.
__device__ __forceinline__ uint32_t dpp_row_max_u32(uint32_t v) {
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row_mirror
  v = v > t ? v : t;
  return v;
}

// Max over the whole wave (result uniform).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_row_max_u32(v);
  uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}

// Sum over the wave in fp64 in a fixed order (xor butterfly): every lane
// ends with the same value, the same for every run.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// RMSNorm factor from the fp64 sum of squares of a row of k activations:
// ms = fp32(sum / k), v = fp32(ms + eps), r = fp32(1 / sqrt(v)) evaluated in
// fp64 (division and square root correctly rounded there) and rounded once.
__device__ __forceinline__ float rms_factor(double sumsq, int k, float norm_eps) {
  const float ms = (float)(sumsq / (double)k);
  const float v = __fadd_rn(ms, norm_eps);
  return (float)(1.0 / sqrt((double)v));
}

// y = fp32(fp32(x * r) * w): two separately rounded multiplies.
__device__ __forceinline__ float rms_apply(float x, float r, float w) {
  return __fmul_rn(__fmul_rn(x, r), w);
}

// Four activations (fp32 bit patterns) to four int8 codes rint(fp32(v * s))
// packed in byte order, for s = fp32(127 / b) with b = max(beta, eps) >= |v|
// (the activation quant of a row whose absmax is beta).  The clamp to
// [-128, 127] is left out: it never binds for finite inputs, since
// |v s| <= 127 (1 + 2^-24), whose fp32 rounding is at most 127 + 2^-17, so
// rint stays within [-127, 127].  Adding 1.5 * 2^23 rounds a product of
// magnitude below 2^22 to the nearest integer, ties to even, in the low
// mantissa bits; three v_perm pack the low bytes.  The product must be
// rounded to fp32 before that add: contracted into one fma, rint would see
// the exact product (__fmul_rn is a plain multiply, and device code
// contracts by default), hence contract(off).
__device__ __forceinline__ uint32_t quant4_rne(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                               float s) {
#pragma clang fp contract(off)
  uint32_t q[4] = {a, b, c, d};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    q[i] = __float_as_uint(__fmul_rn(__uint_as_float(q[i]), s) + 12582912.0f);
  const uint32_t lo = __builtin_amdgcn_perm(q[1], q[0], 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(q[3], q[2], 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Rescale factor gamma / s as the correctly rounded fp32 quotient (the fp64
// quotient of two fp32 values rounds to the same fp32 as the exact one).
__device__ __forceinline__ float gamma_over_s(float gamma, float s) {
  return (float)((double)gamma / (double)s);
}

// Split-K combine in one device-scope round trip.  Every contribution to an
// output adds 2^40 + its partial sum to the output's 64-bit workspace slot;
// the atomic returns the previous value, so the contribution that raises the
// count (bits 40 and up) to `splits` already holds the total, and it clears
// the slot for the next call.  The partial sums of any subset of
// contributions stay below 2^31 in magnitude (64 * 127 * K < 2^31), so the
// count never mixes with the sum.
constexpr int64_t kSplitCount = int64_t(1) << 40;

// Add one contribution; returns the slot's previous value.
__device__ __forceinline__ int64_t split_add(int64_t* slot, int partial) {
  return __hip_atomic_fetch_add(slot, kSplitCount + (int64_t)partial, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}

// From split_add's return value: true for the contribution that completes
// the slot (which it then clears), with the total in `total`.
__device__ __forceinline__ bool split_done(int64_t* slot, int64_t old, int partial, int splits,
                                           int& total) {
  const int64_t count = (old + (kSplitCount >> 1)) >> 40;
  if (count != (int64_t)(splits - 1)) return false;
  total = (int)(old - count * kSplitCount + (int64_t)partial);
  __hip_atomic_store(slot, int64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// The total for the completing contribution, else 1 (never a total: every
// accumulator here is a multiple of 64).
__device__ __forceinline__ int split_finish(int64_t* slot, int64_t old, int partial, int splits) {
  int total = 1;
  return split_done(slot, old, partial, splits, total) ? total : 1;
}

// y = acc * f, then ReLU^2 if asked; stored as fp32 or bf16.
__device__ __forceinline__ void store_out(void* y, int64_t idx, int acc, float f,
                                          bool relu2, bool bf16) {
  float v = (float)acc * f;
  if (relu2) v = v > 0.0f ? v * v : 0.0f;
  if (bf16)
    reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16(v);
  else
    reinterpret_cast<float*>(y)[idx] = v;
}

}  // namespace bl
