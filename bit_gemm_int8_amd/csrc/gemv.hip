// Decode ternary GEMV for one or two tokens with the fused dequant, and the
// fused decode step (activation quantization + products of several matrices
// in one launch): v_dot4 for 1-2 tokens, int8 matrix cores for 3-64.
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T in an integer
// accumulator, then y = acc * beta*gamma/127 = acc * gamma / s; section
// "8-Bit Activation Quantization: absmax Scaling" for x~ and s.
//
// At batch 1 the product reads every packed weight once and does two integer
// ops per 1/4 byte, so the kernel is bound by HBM bandwidth.  Layout of the
// work (the packed layout is in include/bitlinear.h):
//   - a workgroup owns a group of rows, either 16 rows with four lanes per
//     row (QPL = 1) or a 64-row packed block with one lane per row
//     (QPL = 4), and WAVES waves split its 256-input super-chunks into
//     contiguous ranges;
//   - per super-chunk a lane loads QPL of the four 16-byte parts q of its
//     row's 64 bytes; each load instruction of a wave reads 1 KiB of
//     contiguous memory, non-temporally (the weights are read once), and PF
//     super-chunks per wave are in flight at once;
//   - all lanes of a wave work on the same inputs: the workgroup puts its
//     slice of x~ in LDS once (after issuing its first weight loads) and the
//     lanes read it at one shared address, which the LDS broadcasts;
//   - a word unpacks to four int8 lanes of 64*W~ with one shift and one mask;
//     acc = sum >> 6 at the end (every term is a multiple of 64);
//   - the waves' sums meet in LDS; when the row blocks alone cannot fill the
//     chip, `splits` workgroups share a row block and combine through one
//     64-bit device-scope atomic per output (no counters, no fences).
#include <climits>

#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

// One super-chunk: w = the lane's QPL 16-byte loads, q = q0 .. q0+QPL-1
// (word (q, j) = w[q - q0].{x,y,z,w}[j], inputs 64j + 16q + 4i + (0..3)),
// xs = this super-chunk's 256 bytes of x~ for each token in LDS (token
// stride xs_stride dwords).  With all four q in a lane the loop runs in two
// halves with a scheduling barrier between them, so at most 8 x~ loads (32
// registers) are held at once.
template <int M, int QPL>
__device__ __forceinline__ void accumulate_chunk(const uint4 (&w)[QPL], const uint32_t* xs,
                                                 int xs_stride, int q0, int (&acc)[M]) {
  constexpr int HALVES = QPL >= 2 ? 2 : 1;
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
#pragma unroll
      for (int qi = h * QPL / HALVES; qi < (h + 1) * QPL / HALVES; ++qi) {
        const uint32_t wq[4] = {w[qi].x, w[qi].y, w[qi].z, w[qi].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 xv =
              *reinterpret_cast<const uint4*>(xs + m * xs_stride + 16 * j + 4 * (q0 + qi));
          acc[m] = dot4(unpack_x64(wq[j], 0), xv.x, acc[m]);
          acc[m] = dot4(unpack_x64(wq[j], 1), xv.y, acc[m]);
          acc[m] = dot4(unpack_x64(wq[j], 2), xv.z, acc[m]);
          acc[m] = dot4(unpack_x64(wq[j], 3), xv.w, acc[m]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The first PF super-chunks of a wave's range.  Slots past the range load
// a super-chunk this workgroup reads anyway (the wave's last, or the group's
// first for a wave with none), never used: with no branches around the
// loads the compiler can count them and wait for older loads without
// waiting for these.
template <int PF, int QPL>
__device__ __forceinline__ void prefetch_first(uint4 (&buf)[PF][QPL], const uint4* blk, int c0,
                                               int c1, int g0) {
  const int last = c1 > c0 ? c1 - 1 : g0;
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int c = c0 + p < c1 ? c0 + p : last;
#pragma unroll
    for (int q = 0; q < QPL; ++q) buf[p][q] = load_stream16(blk + (int64_t)c * kBlockU4 + q * 64);
  }
}

// Stream super-chunks c0..c1-1 (the first PF already in buf); x~ in LDS
// starts at super-chunk g0.  The steady-state loop loads without conditions
// (so the compiler need not keep old buffer values alive); the last fewer
// than 2*PF chunks drain after it.
template <int M, int PF, int QPL>
__device__ __forceinline__ void stream_chunks(uint4 (&buf)[PF][QPL], const uint4* blk, int c0,
                                              int c1, int g0, const uint32_t* xs, int xs_stride,
                                              int q0, int (&acc)[M]) {
  int c = c0;
  for (; c + 2 * PF <= c1; c += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      accumulate_chunk<M, QPL>(buf[p], xs + (c + p - g0) * 64, xs_stride, q0, acc);
#pragma unroll
      for (int q = 0; q < QPL; ++q) buf[p][q] = load_stream16(blk + (int64_t)(c + p + PF) * kBlockU4 + q * 64);
    }
  }
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    if (c + p < c1) {
      accumulate_chunk<M, QPL>(buf[p], xs + (c + p - g0) * 64, xs_stride, q0, acc);
      if (c + p + PF < c1) {
#pragma unroll
        for (int q = 0; q < QPL; ++q)
          buf[p][q] = load_stream16(blk + (int64_t)(c + p + PF) * kBlockU4 + q * 64);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (c + PF + p < c1)
      accumulate_chunk<M, QPL>(buf[p], xs + (c + PF + p - g0) * 64, xs_stride, q0, acc);
}

// Lanes that share a row (lane = r + RPW g, RPW = 16 QPL) add up their
// q-parts; afterwards every lane of the row holds the row's sum.
template <int M, int QPL>
__device__ __forceinline__ void reduce_lane_groups(int (&acc)[M]) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (QPL <= 2) acc[m] += __shfl_xor(acc[m], 32);
    if (QPL == 1) acc[m] += __shfl_xor(acc[m], 16);
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

// Workgroups that share a row block combine per (token, row) through a
// 64-bit workspace slot (split_add, split_done); the lane whose contribution
// completes a slot writes that output.  Wave 0 only.
template <int M>
__device__ __forceinline__ void combine_splits(int (&acc)[M], bool (&own)[M], int64_t* slot,
                                               int splits) {
  int64_t old[M];
#pragma unroll
  for (int m = 0; m < M; ++m) old[m] = split_add(slot + m * 64, acc[m]);
#pragma unroll
  for (int m = 0; m < M; ++m) own[m] = split_done(slot + m * 64, old[m], acc[m], splits, acc[m]);
}

template <int M>
__device__ __forceinline__ void write_rows(const int (&acc)[M], const bool (&own)[M],
                                           const float (&fac)[M], int64_t row, int n, void* y,
                                           int32_t* acc_out, bool relu2, bool bf16) {
  if (row >= n) return;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (!own[m]) continue;
    const int a = acc[m] >> 6;                       // exact: every term is a multiple of 64
    if (acc_out != nullptr) acc_out[(int64_t)m * n + row] = a;
    store_out(y, (int64_t)m * n + row, a, fac[m], relu2, bf16);
  }
}

// ------------------------------------------------------------ plain GEMV --
// 16-byte x~ units per thread loaded ahead of the weights: 1024 per group.
template <int WAVES>
constexpr int kXR = WAVES >= 16 ? 1 : 16 / WAVES;

// A workgroup owns RPW = 16*QPL rows of a 64-row packed block (sub-block
// `sub`) and a range of super-chunks; lane l = r + RPW g reads row r's
// q-parts QPL*g .. QPL*g+QPL-1, so one wave instruction still reads whole
// 256-byte runs, and the lanes of a row add up their parts at the end.
// Fewer rows per group give more groups without splitting K.
template <int M, int WAVES, int PF, int QPL>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ scale,
    const uint4* __restrict__ packed, const float* __restrict__ gamma, int n, int nc,
    int64_t kpad, int splits, int relu2, int bf16, void* __restrict__ y,
    int32_t* __restrict__ acc_out, int64_t* __restrict__ ws_slots) {
  constexpr int RPW = 16 * QPL, SUBS = 4 / QPL;
  __shared__ int red[WAVES > 1 ? WAVES - 1 : 1][M][64];
  extern __shared__ uint4 xs_lds[];                 // x~ of this group's inputs, per token
  const int bs = blockIdx.x / splits;
  const int s = blockIdx.x - bs * splits;
  const int b = bs / SUBS, sub = bs - b * SUBS;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar control
  const int lane = threadIdx.x & 63;
  const int r = lane % RPW, q0 = QPL * (lane / RPW);
  // this workgroup's super-chunks, then this wave's contiguous share
  const int g0 = (int)((int64_t)s * nc / splits);
  const int g1 = (int)((int64_t)(s + 1) * nc / splits);
  const int c0 = g0 + (int)((int64_t)wave * (g1 - g0) / WAVES);
  const int c1 = g0 + (int)((int64_t)(wave + 1) * (g1 - g0) / WAVES);
  const uint4* blk = packed + (int64_t)b * nc * kBlockU4 + q0 * 64 + sub * RPW + r;

  // x~[m][256*g0 .. 256*g1) for every token (16 units of 16 bytes per
  // super-chunk and token) goes to LDS.  Its first loads are issued before
  // the weights: loads retire in issue order, so the staging then waits only
  // for them, not for the weight stream.
  constexpr int NT = 64 * WAVES;
  const int span = (g1 - g0) * 16;                  // uint4 per token
  auto x_unit = [&](int u) {
    const int m = u / span, v = u - m * span;
    return reinterpret_cast<const uint4*>(xq + (int64_t)m * kpad + (int64_t)g0 * 256)[v];
  };
  // Slots past the range (span * M units) wrap around and rewrite a unit
  // with its own value: no branch, so the compiler keeps these loads ahead of
  // the weights, and no two lanes of a wave hit one LDS address.
  constexpr int XR = kXR<WAVES>;
  const int units = span * M;
  uint4 xr[XR];
  int xu[XR];
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    xu[r] = ((int)threadIdx.x + NT * r) % units;
    xr[r] = x_unit(xu[r]);
  }

  uint4 buf[PF][QPL];
  prefetch_first<PF, QPL>(buf, blk, c0, c1, g0);
  // epilogue operands, loaded now so their latency hides under the stream
  const float g = *gamma;
  float fac[M];
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = scale[m];
  int acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0;

#pragma unroll
  for (int r = 0; r < XR; ++r) xs_lds[xu[r]] = xr[r];
  for (int u = threadIdx.x + NT * XR; u < units; u += NT) xs_lds[u] = x_unit(u);
  __syncthreads();
  stream_chunks<M, PF, QPL>(buf, blk, c0, c1, g0, reinterpret_cast<const uint32_t*>(xs_lds),
                            span * 4, q0, acc);
  reduce_lane_groups<M, QPL>(acc);
  if (!reduce_waves<M, WAVES>(acc, red, wave, lane)) return;
  if (lane >= RPW) return;
  const int rb = sub * RPW + r;                     // row within the 64-row block
  bool own[M];
#pragma unroll
  for (int m = 0; m < M; ++m) own[m] = true;
  if (splits > 1) combine_splits<M>(acc, own, ws_slots + (int64_t)b * (M * 64) + rb, splits);
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = gamma_over_s(g, fac[m]);
  write_rows<M>(acc, own, fac, (int64_t)b * 64 + rb, n, y, acc_out, relu2 != 0, bf16 != 0);
}

template <int M, int WAVES, int PF, int QPL>
hipError_t run_gemv(const int8_t* xq, const float* scale, const uint32_t* packed,
                    const float* gamma, int64_t n, int64_t k, int splits, bool relu2, bool bf16,
                    void* y, int32_t* acc_out, int64_t* ws_slots, hipStream_t stream) {
  const int nb = (int)cdiv(n, kRowBlock);
  const int nc = (int)cdiv(k, kSuperK);
  dim3 grid((unsigned)((int64_t)nb * (4 / QPL) * splits)), block(64 * WAVES);
  const size_t lds = (size_t)M * cdiv(nc, splits) * 256;
  gemv_kernel<M, WAVES, PF, QPL><<<grid, block, lds, stream>>>(
      xq, scale, reinterpret_cast<const uint4*>(packed), gamma, (int)n, nc, padded_k(k), splits,
      relu2, bf16, y, acc_out, ws_slots);
  return hipGetLastError();
}

// ---------------------------------------------------- fused decode step --
// Each workgroup reads its segment's activations x (fp32/bf16), computes the
// token's absmax over all K with DPP wave reductions and LDS, s = 127/max(beta,
// eps), and writes x~ = clamp(rint(x*s)) for its own super-chunks straight
// into LDS: every group of a segment computes the same s and x~ bit for bit.
//
// Order matters: vector-memory loads retire in issue order, so a load issued
// after the weight stream cannot be waited for without waiting for the
// weights.  The activation loads therefore go out first (x_load_first, raw
// 16-byte units into registers, nothing computed on them yet), then the
// weights; the absmax and the quantization run while the weights are in
// flight.  A unit holds epu = 8 (bf16) or 4 (fp32) activations, i.e. epu/4
// dwords of x~.  Thread t holds units u = (ubase + t + NT*j) mod nu, j < kXV,
// where ubase is the first unit of this workgroup's super-chunks and nu the
// units in a row: together they cover the row when NT*kXV >= nu (else a
// second pass reads the rest), and unit ubase + t + NT*j of this workgroup's
// range is slot j of thread t, ready for the quantization.

// Activation units per thread and token issued first: 1024 per group, or
// 4096 (rows up to 64 KiB) in the long-row instance (one token only).
template <int NT, bool LONGX>
constexpr int kXV = (LONGX ? 4096 : 1024) / NT;

struct XRow {
  int epu;      // activations per 16-byte unit
  int nu;       // units per row
  bool fast;    // whole 16-byte units (row bytes % 16 == 0, x 16-byte aligned)
};

__device__ __forceinline__ XRow x_row_info(const FusedSeg& sg) {
  XRow r;
  const int esize = sg.x_bf16() ? 2 : 4;
  r.epu = 16 / esize;
  r.nu = (sg.k + r.epu - 1) / r.epu;
  r.fast = ((int64_t)sg.k * esize % 16 == 0) && ((uintptr_t)sg.x % 16 == 0);
  return r;
}

__device__ __forceinline__ const char* x_row(const FusedSeg& sg, int m) {
  return reinterpret_cast<const char*>(sg.x) + (int64_t)m * sg.k * (sg.x_bf16() ? 2 : 4);
}

// Unit u of a row as it lies in memory (elements past K read as 0).
__device__ __forceinline__ uint4 load_unit(const FusedSeg& sg, const XRow& xr, const char* row,
                                           int u) {
  if (xr.fast) return reinterpret_cast<const uint4*>(row)[u];
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int i = 0; i < xr.epu; ++i) {
    const int kk = u * xr.epu + i;
    if (kk >= sg.k) break;
    if (sg.x_bf16())
      w[i >> 1] |= ((uint32_t)reinterpret_cast<const uint16_t*>(row)[kk]) << (16 * (i & 1));
    else
      w[i] = reinterpret_cast<const uint32_t*>(row)[kk];
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The epu activations of a unit as fp32 bit patterns.
__device__ __forceinline__ void expand_unit(bool bf16, const uint4& r, uint32_t (&e)[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  if (bf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[2 * i] = w[i] << 16;
      e[2 * i + 1] = w[i] & 0xFFFF0000u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { e[i] = w[i]; e[4 + i] = 0u; }
  }
}

__device__ __forceinline__ uint32_t absmax_unit(bool bf16, const uint4& r) {
  uint32_t e[8];
  expand_unit(bf16, r, e);
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = max(mx, e[i] & 0x7FFFFFFFu);
  return mx;
}

template <int M, int NT, bool LONGX>
__device__ __forceinline__ void x_load_first(const FusedSeg& sg, int g0,
                                             uint4 (&raw)[M][kXV<NT, LONGX>]) {
  constexpr int XV = kXV<NT, LONGX>;
  const XRow xr = x_row_info(sg);
  const int ubase = g0 * 256 / xr.epu;
  int u = (int)(((int64_t)ubase + threadIdx.x) % xr.nu);
  const int step = NT % xr.nu;
#pragma unroll
  for (int j = 0; j < XV; ++j) {
#pragma unroll
    for (int m = 0; m < M; ++m) raw[m][j] = load_unit(sg, xr, x_row(sg, m), u);
    u += step;
    if (u >= xr.nu) u -= xr.nu;
  }
}

__device__ __forceinline__ uint32_t quant1(uint32_t bits, float s) {
  float r = rintf(__uint_as_float(bits) * s);        // one fp32 multiply, half to even
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (uint32_t)(uint8_t)(int8_t)(int)r;
}

__device__ __forceinline__ uint32_t quant4(const uint32_t* e, float s) {
  return quant1(e[0], s) | (quant1(e[1], s) << 8) | (quant1(e[2], s) << 16) |
         (quant1(e[3], s) << 24);
}

// The same four codes with fewer instructions: the product (one fp32
// multiply, as above), clamped to [-128, 127], plus 1.5 * 2^23 lands in
// [2^23, 2^24) where the spacing is 1, so the add rounds it to an integer
// (half to even, like rintf; clamping first is the same since the bounds
// are integers) held in the low mantissa bits: their low byte is the code
// in two's complement.  Three byte permutes pack the four.
__device__ __forceinline__ uint32_t quant4_magic(const uint32_t* e, float s) {
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float p = __fmul_rn(__uint_as_float(e[i]), s);
    p = fminf(fmaxf(p, -128.0f), 127.0f);
    b[i] = __float_as_uint(p + 12582912.0f);
  }
  const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);   // b0.byte0, b1.byte0
  const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// x~ dwords of one unit (relative unit q of this workgroup's range) into LDS.
__device__ __forceinline__ void store_unit_q(bool bf16, const uint4& r, float s, bool live,
                                             uint32_t* xs_token, int q) {
  uint32_t e[8];
  expand_unit(bf16, r, e);
  if (bf16) {
    xs_token[2 * q] = live ? quant4(e, s) : 0u;
    xs_token[2 * q + 1] = live ? quant4(e + 4, s) : 0u;
  } else {
    xs_token[q] = live ? quant4(e, s) : 0u;
  }
}

// Per-token scales s[m] and x~ of super-chunks g0..g1-1 into LDS (token
// stride span_w dwords, zero past K), from the units x_load_first holds.
template <int M, int WAVES, bool LONGX>
__device__ __forceinline__ void quantize_into_lds(const FusedSeg& sg, int g0, int g1, float eps,
                                                  const uint4 (&raw)[M][kXV<64 * WAVES, LONGX>],
                                                  uint32_t* xs_words, float (&sv)[M],
                                                  uint32_t (*red)[M]) {
  constexpr int NT = 64 * WAVES;
  constexpr int XV = kXV<NT, LONGX>;
  const XRow xr = x_row_info(sg);
  const bool bf16 = sg.x_bf16();
  const int ubase = g0 * 256 / xr.epu;
  uint32_t mx[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    mx[m] = 0;
#pragma unroll
    for (int j = 0; j < XV; ++j) mx[m] = max(mx[m], absmax_unit(bf16, raw[m][j]));
  }
  if (NT * XV < xr.nu) {                            // long rows: the units not held
    int u = (int)(((int64_t)ubase + threadIdx.x + (int64_t)NT * XV) % xr.nu);
    for (int i = NT * XV; i < xr.nu; i += NT) {
#pragma unroll
      for (int m = 0; m < M; ++m)
        mx[m] = max(mx[m], absmax_unit(bf16, load_unit(sg, xr, x_row(sg, m), u)));
      u += NT % xr.nu;
      if (u >= xr.nu) u -= xr.nu;
    }
  }
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t w = wave_max_u32(mx[m]);
    if ((threadIdx.x & 63) == 0) red[wave][m] = w;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < M; ++m) {
    uint32_t r = red[0][m];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) r = max(r, red[w][m]);
    sv[m] = (float)(127.0 / (double)fmaxf(__uint_as_float(r), eps));
  }
  const int span_w = (g1 - g0) * 64;                 // dwords of x~ per token
  const int span_u = (g1 - g0) * 256 / xr.epu;       // units per token
#pragma unroll
  for (int j = 0; j < XV; ++j) {
    const int q = threadIdx.x + NT * j;
    if (q < span_u) {
      const bool live = ubase + q < xr.nu;
#pragma unroll
      for (int m = 0; m < M; ++m) store_unit_q(bf16, raw[m][j], sv[m], live, xs_words + m * span_w, q);
    }
  }
  for (int q = threadIdx.x + NT * XV; q < span_u; q += NT) {   // ranges beyond the held slots
    const bool live = ubase + q < xr.nu;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4 r = live ? load_unit(sg, xr, x_row(sg, m), ubase + q) : make_uint4(0, 0, 0, 0);
      store_unit_q(bf16, r, sv[m], live, xs_words + m * span_w, q);
    }
  }
}

template <int M, int WAVES, int PF, int QPL, bool LONGX>
// The entry count and the first workgroup of entries 1..13 lead the kernel
// arguments as plain ints (entries past nseg: INT_MAX), which the hardware
// can preload into scalar registers: a workgroup then finds its entry with
// no memory access and reads that entry's fields with a single load.
__global__ __launch_bounds__(64 * WAVES) void gemv_fused_kernel(
    int nseg, int wb1, int wb2, int wb3, int wb4, int wb5, int wb6, int wb7, int wb8, int wb9,
    int wb10, int wb11, int wb12, int wb13, FusedArgs args) {
  constexpr int RPW = 16 * QPL, SUBS = 4 / QPL;     // rows per group, groups per row block
  __shared__ int red[WAVES > 1 ? WAVES - 1 : 1][M][64];
  __shared__ uint32_t red_max[WAVES][M];
  extern __shared__ uint4 xs_lds[];
  // segment of this workgroup
  const int bid = (int)blockIdx.x;
  const int wb[13] = {wb1, wb2, wb3, wb4, wb5, wb6, wb7, wb8, wb9, wb10, wb11, wb12, wb13};
  int si = 0;
#pragma unroll
  for (int i = 0; i < 13; ++i) si = bid >= wb[i] ? i + 1 : si;
  if (nseg > 14) {
#pragma unroll
    for (int i = 14; i < kMaxFused; ++i)
      if (i < nseg && bid >= args.wg_begin[i]) si = i;
  }
  const FusedSeg& sg = args.seg[si];
  const int local = (int)blockIdx.x - sg.wg_begin;
  const int splits = sg.splits;
  const int bs = local / splits;
  const int s = local - bs * splits;
  const int b = bs / SUBS, sub = bs - b * SUBS;
  const int nc = sg.nc;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar control
  const int lane = threadIdx.x & 63;
  const int r = lane % RPW, q0 = QPL * (lane / RPW);
  const int g0 = (int)((int64_t)s * nc / splits);
  const int g1 = (int)((int64_t)(s + 1) * nc / splits);
  const int c0 = g0 + (int)((int64_t)wave * (g1 - g0) / WAVES);
  const int c1 = g0 + (int)((int64_t)(wave + 1) * (g1 - g0) / WAVES);
  const uint4* blk = reinterpret_cast<const uint4*>(sg.packed) + (int64_t)b * nc * kBlockU4 +
                     q0 * 64 + sub * RPW + r;

  uint4 xraw[M][kXV<64 * WAVES, LONGX>];
  x_load_first<M, 64 * WAVES, LONGX>(sg, g0, xraw);        // activations first (see above)
  uint4 buf[PF][QPL];
  prefetch_first<PF, QPL>(buf, blk, c0, c1, g0);
  const float g = *sg.gamma;
  int acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0;

  uint32_t* xs_words = reinterpret_cast<uint32_t*>(xs_lds);
  float sv[M];
  quantize_into_lds<M, WAVES, LONGX>(sg, g0, g1, args.eps, xraw, xs_words, sv, red_max);
  __syncthreads();
  const int span_w = (g1 - g0) * 64;
  // optional copies of x~ and s (the groups of row block 0, sub-block 0
  // cover all of K_pad)
  if (b == 0 && sub == 0 && sg.xq_out != nullptr) {
    const int64_t kpad = (int64_t)nc * 256;
    for (int m = 0; m < M; ++m)
      for (int d = threadIdx.x; d < span_w; d += 64 * WAVES)
        reinterpret_cast<uint32_t*>(sg.xq_out + (int64_t)m * kpad + (int64_t)g0 * 256)[d] =
            xs_words[m * span_w + d];
  }
  if (b == 0 && sub == 0 && s == 0 && sg.scale_out != nullptr && threadIdx.x == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) sg.scale_out[m] = sv[m];
  }

  stream_chunks<M, PF, QPL>(buf, blk, c0, c1, g0, xs_words, span_w, q0, acc);
  reduce_lane_groups<M, QPL>(acc);
  if (!reduce_waves<M, WAVES>(acc, red, wave, lane)) return;
  if (lane >= RPW) return;
  const int rb = sub * RPW + r;                     // row within the 64-row block
  bool own[M];
#pragma unroll
  for (int m = 0; m < M; ++m) own[m] = true;
  if (splits > 1) combine_splits<M>(acc, own, sg.slots + (int64_t)b * (M * 64) + rb, splits);
  float fac[M];
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = gamma_over_s(g, sv[m]);
  write_rows<M>(acc, own, fac, (int64_t)b * 64 + rb, sg.n, sg.y, sg.acc_out, sg.relu2(),
                sg.y_bf16());
}

// ----------------------------------------------------- fused MFMA decode --
// The fused decode step for 3 to 64 tokens: the entries' products on
// v_mfma_i32_16x16x64_i8 as in the windowed MFMA GEMV (unpacked weights of
// 16 rows as the first operand, x~ of 16 tokens as the second, x~ through
// two LDS windows per K-slice, one barrier per super-chunk), in token
// blocks of 16 on blockIdx.y, with the activation quant of each entry's
// block done by every workgroup of the block:
//   1. the first weight loads are issued;
//   2. max|x| per token over its whole row (every thread reads units of
//      every token; idempotent, so loads past the row or past token m-1
//      read a valid unit again), reduced with DPP and across waves in LDS,
//      and s = 127 / max(beta, eps) exactly as bitlinear_quant_act;
//   3. each window is staged from x itself: the 16 inputs of an x~ unit are
//      loaded (two bf16 or four fp32 16-byte units), quantized with the
//      token's s and stored to LDS (and to xq_out by the entry's first
//      workgroup).
// Workgroup g of an entry owns WR row groups of SB 16-row sub-blocks; its
// WK waves per group split the super-chunks and meet in LDS at the end.
// With NORM, entries flagged for RMSNorm normalize each token first (the
// BitLinear listing of "End-to-End Implementation: Building a Native BitLinear
// Layer" applies nn.RMSNorm before quantize_activations_int8): the token's
// wave sums x^2 over the row in fp64 (lanes, then the xor butterfly),
// r = rms_factor(sum, K, eps), and y = fp32(fp32(x * r) * w) replaces x in
// the absmax and in the staging.
template <int WR, int WK, int SB, int PF, int RPU, int MT, bool FAST, bool NORM>
// Leading scalar arguments (preloadable into SGPRs, as in gemv_fused_kernel):
// the token count, the entry count and the first workgroup of entries 1..12
// (INT_MAX past nseg).
__global__ __launch_bounds__(64 * WR * WK) void gemv_mfma_fused_kernel(
    int m_all, int nseg, int wb1, int wb2, int wb3, int wb4, int wb5, int wb6, int wb7, int wb8,
    int wb9, int wb10, int wb11, int wb12, FusedArgs args) {
  static_assert(RPU == 2 || RPU == 4, "16-byte activation units per x~ unit: 2 (bf16 only), 4");
  // FAST: every entry's rows are whole 16-byte units at 16-byte alignment,
  // so the activation loads are plain vector loads with no branch (a load
  // behind a branch makes the compiler wait for every load in flight)
  static_assert(SB == 1 || SB == 2 || SB == 4, "a wave's sub-blocks lie in one packed block");
  static_assert(PF == 2 || PF == 4, "the loop is unrolled by PF, an even number");
  static_assert(MT == 8 || MT == 16, "tokens handled: m <= MT");
  constexpr int WAVES = WR * WK, NT = 64 * WAVES;
  constexpr int NTS = 64 * WR;                      // threads staging one slice
  constexpr int XU = MT * 16 / NTS;                 // x~ units per staging thread and step
  static_assert(MT * 16 % NTS == 0, "x~ staging split");
  __shared__ bl_v4i xs[WK][2][256];
  __shared__ int red[WK > 1 ? (WK - 1) * WR : 1][SB * 4][64];
  __shared__ uint32_t bmax[MT];
  __shared__ float s_lds[16];
  __shared__ float fac_lds[16];
  __shared__ float rn_lds[NORM ? MT : 1];
  // token block blockIdx.y: tokens t0 .. t0 + m - 1 (16 per block)
  const int t0 = 16 * (int)blockIdx.y;
  const int m = min(m_all - t0, MT);
  const int bid = (int)blockIdx.x;
  const int wgb[12] = {wb1, wb2, wb3, wb4, wb5, wb6, wb7, wb8, wb9, wb10, wb11, wb12};
  int si = 0;
#pragma unroll
  for (int i = 0; i < 12; ++i) si = bid >= wgb[i] ? i + 1 : si;
  if (nseg > 13) {
#pragma unroll
    for (int i = 13; i < kMaxFused; ++i)
      if (i < nseg && bid >= args.wg_begin[i]) si = i;
  }
  const FusedSeg& sg = args.seg[si];
  const int local = (int)blockIdx.x - sg.wg_begin;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave / WK, wk = wave - wr * WK;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int nc = sg.nc;
  const int nsub = (sg.n + kRowBlock - 1) / kRowBlock * 4;
  int u0 = (local * WR + wr) * SB;
  const bool live = u0 < nsub;
  if (!live) u0 = nsub - SB;
  const int b = u0 >> 2, sub0 = u0 & 3;
  const int L = (nc + WK - 1) / WK;
  const int c0 = wk * L;
  const int c1 = min(c0 + L, nc);
  const int clast = c1 > c0 ? c1 - 1 : nc - 1;
  const uint4* blk = reinterpret_cast<const uint4*>(sg.packed) + (int64_t)b * nc * kBlockU4 +
                     g * 64 + sub0 * 16 + r;

  // 1. weights of the first PF super-chunks (ordinary loads, unlike the
  // one-pass GEMVs: the token blocks of an entry read the same weights
  // again, and non-temporal loads measured 5-6% slower from 32 tokens)
  uint4 wb[PF][SB];
  static_for<PF>([&](auto P) {
    constexpr int p = decltype(P)::value;
    const int c = min(c0 + p, clast);
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) wb[p][sb] = blk[(int64_t)c * kBlockU4 + sb * 16];
  });
  const float gam = *sg.gamma;

  // 2. per-token max|x|: wave w reduces tokens w, w + WAVES, ... below m,
  //    eight 16-byte loads per lane in flight (past the row they repeat the
  //    last unit: the max is idempotent)
  const XRow xrow = x_row_info(sg);
  const bool xbf = sg.x_bf16();
  const bool nrm = NORM && sg.rmsnorm();
  const float* gain = sg.norm_weight;
  // RMSNorm gain of input i (ones when absent; i past K clamped, where x is 0)
  auto gain_at = [&](int i) __attribute__((always_inline)) {
    return gain != nullptr ? gain[min(i, sg.k - 1)] : 1.0f;
  };
  for (int t = wave; t < m; t += WAVES) {
    const char* row = x_row(sg, t0 + t);
    float rn = 1.0f;
    if (NORM && nrm) {                               // sum of squares (fp64), this wave
      double ss = 0.0;
      for (int u = lane; u < xrow.nu; u += 64) {
        uint32_t e[8];
        expand_unit(xbf, FAST ? reinterpret_cast<const uint4*>(row)[u]
                              : load_unit(sg, xrow, row, u), e);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double d = (double)__uint_as_float(e[i]);
          ss += d * d;
        }
      }
      rn = rms_factor(wave_sum_f64(ss), sg.k, sg.norm_eps);
      if (lane == 0) rn_lds[t] = rn;
    }
    uint32_t mx = 0;
    for (int ub = 0; ub < xrow.nu; ub += 64 * 8) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int u = min(ub + lane + 64 * j, xrow.nu - 1);
        v[j] = FAST ? reinterpret_cast<const uint4*>(row)[u] : load_unit(sg, xrow, row, u);
      }
      if (NORM && nrm) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int u = min(ub + lane + 64 * j, xrow.nu - 1);
          uint32_t e[8];
          expand_unit(xbf, v[j], e);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (i >= xrow.epu) break;
            const float y = rms_apply(__uint_as_float(e[i]), rn, gain_at(u * xrow.epu + i));
            mx = max(mx, __float_as_uint(y) & 0x7FFFFFFFu);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = max(mx, absmax_unit(xbf, v[j]));
      }
    }
    mx = wave_max_u32(mx);
    if (lane == 0) bmax[t] = mx;
  }
  __syncthreads();
  if (threadIdx.x < MT) {
    // tokens >= m (whose columns are dropped) take token m-1's scale
    const uint32_t bt = bmax[min((int)threadIdx.x, m - 1)];
    const float sv = (float)(127.0 / (double)fmaxf(__uint_as_float(bt), args.eps));
    s_lds[threadIdx.x] = sv;
    fac_lds[threadIdx.x] = gamma_over_s(gam, sv);
    if (local == 0 && sg.scale_out != nullptr && (int)threadIdx.x < m)
      sg.scale_out[t0 + threadIdx.x] = sv;
  }
  __syncthreads();

  // 3. this thread's x~ units of its slice: token t = q / 16, unit q % 16
  //    (inputs 16 (q % 16) .. + 15 of each super-chunk)
  const int epu = xrow.epu;                         // activations per 16-byte unit: 8 or 4
  const char* xsrc[XU];
  int xdst[XU], xtok[XU], xq16[XU];
  float xsc[XU], xrn[XU];
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int q = wr * 64 + lane + NTS * i;
    const int t = q >> 4, u = q & 15;
    xtok[i] = t;
    xq16[i] = u;
    xsrc[i] = x_row(sg, t0 + min(t, m - 1));
    xdst[i] = t * 16 + (u ^ (t & 15));
    xsc[i] = s_lds[t];
    xrn[i] = NORM && nrm ? rn_lds[min(t, m - 1)] : 1.0f;
  }
  // gains of a step's units (16 inputs each), RMSNorm entries only
  float xg[NORM ? PF : 1][NORM ? XU : 1][16];
  auto load_g = [&](auto P, int c) __attribute__((always_inline)) {
    if (NORM && nrm) {
      constexpr int p = decltype(P)::value;
#pragma unroll
      for (int i = 0; i < XU; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) xg[p][i][e] = gain_at(c * 256 + xq16[i] * 16 + e);
    }
  };
  // raw activations of a step's units: RPU 16-byte units each (bf16 uses
  // the first two of four)
  uint4 xr[PF][XU][RPU];
  auto load_x = [&](auto P, int c) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int i = 0; i < XU; ++i)
#pragma unroll
      for (int e = 0; e < RPU; ++e) {
        const int u = (c * 256 + xq16[i] * 16) / epu + e;
        xr[p][i][e] = FAST ? reinterpret_cast<const uint4*>(xsrc[i])[min(u, xrow.nu - 1)]
                           : load_unit(sg, xrow, xsrc[i], min(u, xrow.nu - 1));
      }
  };
  // x~ of one unit from its raw activations (zero past the row); with
  // RMSNorm, of y = (x r) w
  auto quant_unit = [&](const uint4 (&raw)[RPU], float sc, int c, int q16, float rnv,
                        const float* gv) __attribute__((always_inline)) {
    const int k0 = c * 256 + q16 * 16;
    uint32_t d[4];
    if (NORM && nrm) {
      uint32_t v[16];
      if (xbf) {
        uint32_t e0[8], e1[8];
        expand_unit(true, raw[0], e0);
        expand_unit(true, raw[1 < RPU ? 1 : 0], e1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[i] = e0[i];
          v[8 + i] = e1[i];
        }
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t e[8];
          expand_unit(false, raw[h < RPU ? h : 0], e);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * h + i] = e[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = __float_as_uint(rms_apply(__uint_as_float(v[i]), rnv, gv[i]));
#pragma unroll
      for (int h = 0; h < 4; ++h) d[h] = quant4_magic(v + 4 * h, sc);
    } else if (xbf) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t e[8];
        expand_unit(true, raw[h], e);
        d[2 * h] = quant4_magic(e, sc);
        d[2 * h + 1] = quant4_magic(e + 4, sc);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint32_t e[8];
        expand_unit(false, raw[h < RPU ? h : 0], e);
        d[h] = quant4_magic(e, sc);
      }
    }
    bl_v4i out = {(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
    if (k0 >= sg.k) out = bl_v4i{0, 0, 0, 0};
    else if (k0 + 16 > sg.k) {                      // the row ends inside this unit
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = k0 + 4 * j;                  // bytes of dword j: inputs kk .. kk+3
        const int keep = max(0, min(4, sg.k - kk));
        const uint32_t mask = keep >= 4 ? 0xFFFFFFFFu : (1u << (8 * keep)) - 1u;
        out[j] = (int)((uint32_t)out[j] & mask);
      }
    }
    return out;
  };
  static_for<PF>([&](auto P) {
    load_x(P, min(c0 + (int)P, clast));
    load_g(P, min(c0 + (int)P, clast));
  });

  bl_v4i acc[SB];
#pragma unroll
  for (int sb = 0; sb < SB; ++sb) acc[sb] = bl_v4i{0, 0, 0, 0};
  const bool write_xq = local == 0 && sg.xq_out != nullptr;
  const int64_t kpad = (int64_t)nc * 256;
  auto step = [&](auto P, int c) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    bl_v4i* win = xs[wk][p & 1];
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const bl_v4i qv = quant_unit(xr[p][i], xsc[i], c, xq16[i], xrn[i], xg[NORM ? p : 0][NORM ? i : 0]);
      win[xdst[i]] = qv;
      if (write_xq && c < c1 && xtok[i] < m)
        *reinterpret_cast<bl_v4i*>(sg.xq_out + (int64_t)(t0 + xtok[i]) * kpad + c * 256 + xq16[i] * 16) =
            qv;
    }
    __syncthreads();
    const int cn = min(c + PF, clast);
    load_x(P, cn);
    load_g(P, cn);
    __builtin_amdgcn_sched_barrier(0);
    if (c < c1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bl_v4i xv = win[r * 16 + ((4 * j + g) ^ r)];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          const uint32_t wj = j == 0 ? wb[p][sb].x : j == 1 ? wb[p][sb].y
                            : j == 2 ? wb[p][sb].z : wb[p][sb].w;
          const bl_v4i a = {(int)unpack_x64(wj, 0), (int)unpack_x64(wj, 1),
                            (int)unpack_x64(wj, 2), (int)unpack_x64(wj, 3)};
          acc[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, xv, acc[sb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) wb[p][sb] = blk[(int64_t)cn * kBlockU4 + sb * 16];
    __builtin_amdgcn_sched_barrier(0);
  };
  int t = 0;
  for (; t + PF <= L; t += PF) static_for<PF>([&](auto P) { step(P, c0 + t + (int)P); });
  static_for<PF - 1>([&](auto P) {
    if (t + (int)P < L) step(P, c0 + t + (int)P);
  });

  // the slices' sums into the group's first wave
  if (WK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wr * (WK - 1) + wk - 1][sb * 4 + i][lane] = acc[sb][i];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int w = 0; w < WK - 1; ++w)
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[sb][i] += red[wr * (WK - 1) + w][sb * 4 + i][lane];
  }
  // lane (r, g) holds rows 4g..4g+3 of each sub-block for token r (columns
  // of tokens >= MT read window slots never staged; they are dropped)
  if (!live || r >= m) return;
  const float f = fac_lds[r];
  const bool relu2 = sg.relu2(), ybf = sg.y_bf16();
#pragma unroll
  for (int sb = 0; sb < SB; ++sb) {
    const int row0 = b * 64 + (sub0 + sb) * 16 + 4 * g;
    const int64_t idx = (int64_t)(t0 + r) * sg.n + row0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (row0 + i >= sg.n) continue;
      const int a = acc[sb][i] >> 6;
      if (sg.acc_out != nullptr) sg.acc_out[idx + i] = a;
      store_out(sg.y, idx + i, a, f, relu2, ybf);
    }
  }
}

}  // namespace

// Plain GEMV: x~ and s given.
hipError_t launch_gemv(int m, int waves, int pf, int qpl, const int8_t* xq, const float* scale,
                       const uint32_t* packed, const float* gamma, int64_t n, int64_t k,
                       int splits, bool relu2, bool bf16, void* y, int32_t* acc_out,
                       int64_t* ws_slots, hipStream_t stream) {
#define BL_GEMV(MM, WW, PP, QQ)                                                                 \
  return run_gemv<MM, WW, PP, QQ>(xq, scale, packed, gamma, n, k, splits, relu2, bf16, y,       \
                                  acc_out, ws_slots, stream)
  // 64 rows per group (qpl 4): 1 or 2 super-chunks in flight per wave;
  // 16 rows (qpl 1, a quarter of the bytes per super-chunk): 4 or 8
#define BL_GEMV_W(MM)                                                   \
  if (qpl == 1) {                                                       \
    if (waves == 8) {                                                   \
      if (pf >= 8) { BL_GEMV(MM, 8, 8, 1); } else { BL_GEMV(MM, 8, 4, 1); } \
    } else {                                                            \
      if (pf >= 8) { BL_GEMV(MM, 4, 8, 1); } else { BL_GEMV(MM, 4, 4, 1); } \
    }                                                                   \
  } else if (waves == 8) {                                              \
    if (pf == 2) { BL_GEMV(MM, 8, 2, 4); } else { BL_GEMV(MM, 8, 1, 4); } \
  } else {                                                              \
    if (pf == 2) { BL_GEMV(MM, 4, 2, 4); } else { BL_GEMV(MM, 4, 1, 4); } \
  }
  switch (m) {
    case 1: BL_GEMV_W(1);
    case 2: BL_GEMV_W(2);
    default: return hipErrorInvalidValue;
  }
#undef BL_GEMV_W
#undef BL_GEMV
}

// Fused decode step for 3 to 64 tokens on the matrix cores, token blocks of
// 16 on grid.y: variant 0 = two 16-row groups x 4 K-slices, 1 = four 32-row
// groups (whole K per wave).
// all_bf16: every entry's x is bf16 (two 16-byte loads per x~ unit, not
// four); all_fast: every entry's rows are whole, aligned 16-byte units.
hipError_t launch_gemv_mfma_fused(const FusedArgs& args, int m, int variant, bool all_bf16,
                                  bool all_fast, bool norm, int groups, hipStream_t stream) {
  if (m < 1 || m > 64) return hipErrorInvalidValue;
  const dim3 grid((unsigned)groups, (unsigned)((m + 15) / 16));   // token blocks of 16
  int wb[13];
  for (int i = 1; i < 13; ++i) wb[i] = i < args.nseg ? args.wg_begin[i] : INT_MAX;
#define BL_MF1(WR, WK, SB, PF, RPU, MT, FAST, NORM)                                   \
  gemv_mfma_fused_kernel<WR, WK, SB, PF, RPU, MT, FAST, NORM>                        \
      <<<grid, 64 * WR * WK, 0, stream>>>(m, args.nseg, wb[1], wb[2], wb[3], wb[4], wb[5],  \
                                          wb[6], wb[7], wb[8], wb[9], wb[10], wb[11], wb[12],  \
                                          args)
#define BL_MF(WR, WK, SB, PF, RPU, MT, FAST)                  \
  do {                                                        \
    if (norm) BL_MF1(WR, WK, SB, PF, RPU, MT, FAST, true);    \
    else BL_MF1(WR, WK, SB, PF, RPU, MT, FAST, false);        \
  } while (0)
#define BL_MF_X(WR, WK, SB, PF, MT)               \
  if (all_fast && all_bf16) BL_MF(WR, WK, SB, PF, 2, MT, true); \
  else if (all_fast) BL_MF(WR, WK, SB, PF, 4, MT, true);       \
  else BL_MF(WR, WK, SB, PF, 4, MT, false)
  if (variant == 0) {
    if (m <= 8) {
      BL_MF_X(2, 4, 1, 2, 8);
    } else {
      BL_MF_X(2, 4, 1, 2, 16);
    }
  } else {
    BL_MF_X(4, 1, 2, 4, 16);
  }
#undef BL_MF_X
#undef BL_MF
#undef BL_MF1
  return hipGetLastError();
}

// Fused decode step over a complete segment table (wg_begin, splits and
// workspace pointers filled in).  long_rows: one token and some row longer
// than 1024 16-byte units.
hipError_t launch_gemv_fused(const FusedArgs& args, int m, int waves, int qpl, bool long_rows,
                             int groups, size_t lds, hipStream_t stream) {
  int wb[14];
  for (int i = 1; i < 14; ++i) wb[i] = i < args.nseg ? args.wg_begin[i] : INT_MAX;
#define BL_FUSED(MM, WW, QQ, LL)                                                       \
  do {                                                                                 \
    gemv_fused_kernel<MM, WW, (QQ == 1 ? 4 : 2), QQ, LL>                               \
        <<<(unsigned)groups, 64 * WW, lds, stream>>>(                                  \
            args.nseg, wb[1], wb[2], wb[3], wb[4], wb[5], wb[6], wb[7], wb[8], wb[9],     \
            wb[10], wb[11], wb[12], wb[13], args);                                         \
    return hipGetLastError();                                                          \
  } while (0)
#define BL_FUSED_Q(MM, WW, LL) \
  if (qpl == 1)                \
    BL_FUSED(MM, WW, 1, LL);   \
  else                         \
    BL_FUSED(MM, WW, 4, LL)
#define BL_FUSED_W(MM, LL)   \
  if (waves == 4) {          \
    BL_FUSED_Q(MM, 4, LL);   \
  } else {                   \
    BL_FUSED_Q(MM, 8, LL);   \
  }
  switch (m) {
    case 1:
      if (long_rows) {
        BL_FUSED_W(1, true);
      }
      BL_FUSED_W(1, false);
    case 2: BL_FUSED_W(2, false);
    default: return hipErrorInvalidValue;
  }
#undef BL_FUSED_W
#undef BL_FUSED_Q
#undef BL_FUSED
}

}  // namespace bl
