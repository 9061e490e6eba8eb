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
// mantissa bits, whose low byte is the code in two's complement; each add
// writes that byte straight into its byte of the result (SDWA dst_sel
// BYTE_i, the other bytes kept), so a value costs two VALU operations and
// no byte permutes.  The product must be rounded to fp32 before that add:
// contracted into one fma, rint would see the exact product (__fmul_rn is a
// plain multiply, and device code contracts by default), hence
// contract(off) -- the add sits in asm, which no contraction crosses anyway.
__device__ __forceinline__ uint32_t quant4_rne(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                               float s) {
#pragma clang fp contract(off)
  const float magic = 12582912.0f;
  const float p0 = __fmul_rn(__uint_as_float(a), s), p1 = __fmul_rn(__uint_as_float(b), s);
  const float p2 = __fmul_rn(__uint_as_float(c), s), p3 = __fmul_rn(__uint_as_float(d), s);
  uint32_t r;
  asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD "
      "src1_sel:DWORD" : "=v"(r) : "v"(p0), "s"(magic));
  asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
      "src1_sel:DWORD" : "+v"(r) : "v"(p1), "s"(magic));
  asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
      "src1_sel:DWORD" : "+v"(r) : "v"(p2), "s"(magic));
  asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
      "src1_sel:DWORD" : "+v"(r) : "v"(p3), "s"(magic));
  return r;
}

// Running max of |x| over the two bf16 values of a word, one VALU operation
// per word: v_pk_maximum3_f16(acc, w, -w) reads each 16-bit lane as fp16.
// Both formats put sign, exponent and mantissa in that order, so for bit
// patterns that are finite in fp16 (fp16 denormals included: the mode keeps
// them) the fp16 order of the magnitudes is the bf16 order.  A bf16
// magnitude above 0x7C00 (|x| > 2^121, or not finite) is a NaN in fp16 and
// makes the accumulator a NaN, which absmax_bf16x2_bits reports.
__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t acc, uint32_t w) {
  uint32_t r;
  asm("v_pk_maximum3_f16 %0, %1, %2, %2 neg_lo:[0,0,1] neg_hi:[0,0,1]"
      : "=v"(r) : "v"(acc), "v"(w));
  return r;
}
constexpr uint32_t kAbsmaxInexact = 0xFFFFFFFFu;
// The larger lane of an absmax_bf16x2 accumulator (started at 0) as fp32
// bits (a bf16 is the top half of its fp32), or kAbsmaxInexact when a lane
// saw a magnitude that fp16 cannot order; that flag exceeds every result,
// so it survives a max reduction, and the caller then takes the exact
// sign-cleared 16-bit max.
__device__ __forceinline__ uint32_t absmax_bf16x2_bits(uint32_t acc) {
  const uint32_t m = max(acc & 0xFFFFu, acc >> 16);
  return m > 0x7C00u ? kAbsmaxInexact : m << 16;
}
// Exact running max of the sign-cleared 16-bit lanes (the path for the
// flagged case).
__device__ __forceinline__ bl_u16x2 absmax_bf16x2_exact(bl_u16x2 acc, uint32_t w) {
  return __builtin_elementwise_max(acc, __builtin_bit_cast(bl_u16x2, w & 0x7FFF7FFFu));
}
// Running max of |x| over fp32 values, two per VALU operation
// (v_max3_f32 with |.| on the new operands); for finite values the result's
// bits are the largest sign-cleared bit pattern.
__device__ __forceinline__ uint32_t absmax_f32x2(uint32_t acc, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(acc), "v"(a), "v"(b));
  return r;
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
