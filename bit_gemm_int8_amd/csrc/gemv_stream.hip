// One- and two-token ternary GEMV on the int8 matrix cores, streaming whole
// 16-row sub-blocks, with the fused dequant; and the same kernel with the
// activation quantization in its prologue (the fused decode step).
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T in an integer
// accumulator, y = acc * gamma / s; section "8-Bit Activation Quantization:
// absmax Scaling" for x~ and s.
//
// At one or two tokens the product reads every packed weight once, so the
// kernel is bound by HBM.  What limits it on MI355X is keeping enough bytes
// in flight per CU while the lanes unpack and multiply, so the work is laid
// out for the memory system and the VALU load is kept low:
//   - a workgroup (8 or 16 waves, about one per CU) owns whole 16-row
//     sub-blocks of one product, all of K, so no K split crosses workgroups:
//     no workspace and no atomics in memory;
//   - the workgroup's 1 KiB units (sub-block t, super-chunk c) are taken in
//     memory order and cut into one contiguous run per wave; each wave keeps
//     D units (one 16-byte non-temporal load per lane each) in flight, issuing
//     the load of unit v + D right after it consumes unit v;
//   - lane (r, g) holds row r, inputs 64j + 16g .. + 15 of word j: exactly the
//     first operand of v_mfma_i32_16x16x64_i8 after the shift-and-mask unpack,
//     so one MFMA per packed word does what four v_dot4 did (the matrix core
//     is idle otherwise; the VALU keeps only the unpack);
//   - the second operand is x~ of token r for lanes r < M (from LDS) and zero
//     for the other lanes, so result column r is token r: lanes r < M hold
//     rows 4g .. 4g + 3 of their token;
//   - a wave adds its sums into LDS (per sub-block, row and token) each time
//     it leaves a sub-block; after one barrier the workgroup writes its rows.
// x~ (all of K, every token) sits in LDS: the plain kernel copies it there
// (loads issued before the weights), the fused kernel computes it there from
// the activations (see gemv_stream_fused_kernel).
#include <climits>

#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

// Load cursor over a wave's units: unit v is sub-block tl, super-chunk cl;
// it stops at the wave's last unit, so loads past the run repeat that unit
// (no branch around the loads, which keeps them in flight).
struct Cursor {
  const uint4* base;      // the lane's record in super-chunk 0 of sub-block tl
  int vl, tl, cl, ulast;
};

__device__ __forceinline__ const uint4* sub_base(const uint4* packed, int nc, int t, int g,
                                                 int r) {
  return packed + ((int64_t)(t >> 2) * nc * 4 + g) * 64 + (t & 3) * 16 + r;
}

__device__ __forceinline__ Cursor cursor_at(const uint4* packed, int nc, int t0, int u0, int u1,
                                            int g, int r) {
  Cursor c;
  c.ulast = u1 > 0 ? u1 - 1 : 0;
  c.vl = min(u0, c.ulast);
  c.tl = t0 + c.vl / nc;
  c.cl = c.vl - (c.vl / nc) * nc;
  c.base = sub_base(packed, nc, c.tl, g, r);
  return c;
}

__device__ __forceinline__ void cursor_next(Cursor& c, const uint4* packed, int nc, int g,
                                            int r) {
  if (c.vl < c.ulast) {
    ++c.vl;
    if (++c.cl == nc) {
      c.cl = 0;
      ++c.tl;
      c.base = sub_base(packed, nc, c.tl, g, r);
    }
  }
}

template <int D>
__device__ __forceinline__ void prefetch_units(uint4 (&buf)[D], Cursor& cur, const uint4* packed,
                                               int nc, int g, int r) {
  static_for<D>([&](auto P) {
    buf[(int)P] = load_stream16(cur.base + (int64_t)cur.cl * kBlockU4);
    cursor_next(cur, packed, nc, g, r);
  });
}

// Stream units [u0, u1) of this workgroup (sub-blocks from t0, nc
// super-chunks each; the first D already in buf) and add each sub-block's
// sums into sums[sub - t0][token][row].  x~ of token m, super-chunk c,
// inputs 64j + 16g .. +15 is LDS uint4 m * kp16 + 16c + 4j + g; zero_idx
// holds 16 zero uint4.
template <int M, int D>
__device__ __forceinline__ void stream_units(uint4 (&buf)[D], Cursor& cur, const uint4* packed,
                                             int nc, int t0, int u0, int u1, int g, int r,
                                             const uint4* xs, int kp16, int zero_idx, int* sums) {
  bl_v4i acc = {0, 0, 0, 0};
  int tc = t0 + u0 / nc, cc = u0 - (u0 / nc) * nc;   // unit being consumed
  auto flush = [&]() __attribute__((always_inline)) {
    if (r < M) {
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&sums[((tc - t0) * M + r) * 16 + 4 * g + i], acc[i]);
    }
    acc = bl_v4i{0, 0, 0, 0};
  };
  // x~ of the unit being consumed, read from LDS one unit ahead so that the
  // MFMAs do not wait for LDS (the read past the last unit is in range: it
  // wraps to super-chunk 0)
  auto x_addr = [&](int c) __attribute__((always_inline)) {
    return r < M ? r * kp16 + c * 16 + g : zero_idx + g;
  };
  uint4 xn[4];
  {
    const int xa = x_addr(cc);
#pragma unroll
    for (int j = 0; j < 4; ++j) xn[j] = xs[xa + 4 * j];
  }
  auto consume = [&](const uint4& w) __attribute__((always_inline)) {
    uint4 xc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xc[j] = xn[j];
    {
      const int xa = x_addr(cc + 1 == nc ? 0 : cc + 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) xn[j] = xs[xa + 4 * j];
    }
    const uint32_t wj[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bl_v4i xv = {(int)xc[j].x, (int)xc[j].y, (int)xc[j].z, (int)xc[j].w};
      const bl_v4i a = {(int)unpack_x64(wj[j], 0), (int)unpack_x64(wj[j], 1),
                        (int)unpack_x64(wj[j], 2), (int)unpack_x64(wj[j], 3)};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, xv, acc, 0, 0, 0);
    }
    if (++cc == nc) {
      flush();
      cc = 0;
      ++tc;
    }
  };
  int v = u0;
  for (; v + D <= u1; v += D) {
    static_for<D>([&](auto P) {
      constexpr int p = decltype(P)::value;
      consume(buf[p]);
      buf[p] = load_stream16(cur.base + (int64_t)cur.cl * kBlockU4);
      cursor_next(cur, packed, nc, g, r);
    });
  }
  static_for<D>([&](auto P) {
    constexpr int p = decltype(P)::value;
    if (v + p < u1) consume(buf[p]);
  });
  if (u1 > u0 && cc != 0) flush();
}

// Rows t0*16 .. t1*16-1 of every token from the LDS sums (64 * acc, exact).
template <int M>
__device__ __forceinline__ void stream_epilogue(const int* sums, int t0, int nsub, int n,
                                                const float (&fac)[M], bool relu2, bool ybf16,
                                                void* y, int32_t* acc_out, int nt) {
  const int rows = nsub * 16;
  for (int i = threadIdx.x; i < rows * M; i += nt) {
    const int m = i / rows, rr = i - m * rows;
    const int row = t0 * 16 + rr;
    if (row >= n) continue;
    const int a = sums[((rr >> 4) * M + m) * 16 + (rr & 15)] >> 6;
    if (acc_out != nullptr) acc_out[(int64_t)m * n + row] = a;
    store_out(y, (int64_t)m * n + row, a, fac[m], relu2, ybf16);
  }
}

// LDS of a workgroup: x~ [M][kp16] uint4, sums [nsub_alloc][M][16] int,
// 16 zero uint4.
__host__ __device__ constexpr int stream_zero_idx(int m, int kp16, int nsub_alloc) {
  return m * kp16 + nsub_alloc * m * 4;
}

// Whether a launch stages x~ before it requests any weight (XF).  At the
// start of a launch every workgroup asks for its x~ and its first weight
// units together: some 12 MB of weight requests queue at the memory
// channels, and x~, which every workgroup needs before its first MFMA,
// waits behind them.  On rows of >= 64 super-chunks at one or two tokens
// (x~ >= 16 KiB per workgroup) that delay measured longer than what the
// early weight requests save: workgroup timestamps put x~ in LDS 2.1-3.0 us after the
// start on 8192 x 28672, and landing x~ first takes the launch from 12.5 to
// 12.0 us at one token, 13.0 to 12.4 us at two (the fused form at one token,
// whose activation row is 56 KiB, from 12.9 to 12.45 us; at two tokens the
// fused form did not move, so it keeps the early requests there); on
// 28672 x 8192 (x~ 8 KiB) it measured 0.1-0.3 us slower.  (MI355X, medians
// of 25 graph replays over 11 rotating weight copies.)
__host__ __device__ constexpr bool gemv_stream_xfirst(int m, int nc) { return m <= 2 && nc >= 64; }

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt = 0 only.
constexpr int kWaitVmcnt0 = 0x0F70;

// ------------------------------------------------------------ plain GEMV --
// x~ and s given.  Workgroup w owns sub-blocks [S w / G, S (w + 1) / G).
template <int M, int WAVES, int D, int XR, bool XF>
__global__ __launch_bounds__(64 * WAVES) void gemv_stream_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ scale,
    const uint4* __restrict__ packed, const float* __restrict__ gamma, int n, int nc, int S,
    int G, int nsub_alloc, int relu2, int ybf16, void* __restrict__ y,
    int32_t* __restrict__ acc_out) {
  constexpr int NT = 64 * WAVES;
  extern __shared__ uint4 lds[];
  const int wg = blockIdx.x;
  const int t0 = (int)((int64_t)S * wg / G), t1 = (int)((int64_t)S * (wg + 1) / G);
  const int nsub = t1 - t0, units = nsub * nc;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int kp16 = nc * 16;
  const int u0 = (int)((int64_t)units * wave / WAVES);
  const int u1 = (int)((int64_t)units * (wave + 1) / WAVES);
  int* sums = reinterpret_cast<int*>(lds + M * kp16);
  const int zero_idx = stream_zero_idx(M, kp16, nsub_alloc);

  // x~ first (loads retire in issue order, so staging it then waits for it
  // alone), clamped so that no load sits behind a branch.  Without XF the
  // first weight units are requested right behind it; with XF (long rows)
  // x~ is in LDS before any weight is requested (see gemv_stream_xfirst).
  const int xu = M * kp16;
  const uint4* xg = reinterpret_cast<const uint4*>(xq);
  uint4 xr[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) xr[j] = xg[min((int)threadIdx.x + NT * j, xu - 1)];
  uint4 buf[D];
  Cursor cur = cursor_at(packed, nc, t0, u0, u1, g, r);
  if constexpr (!XF) prefetch_units<D>(buf, cur, packed, nc, g, r);
  const float gm = *gamma;
  float fac[M];
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = scale[m];

#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int i = (int)threadIdx.x + NT * j;
    if (i < xu) lds[i] = xr[j];
  }
  for (int i = (int)threadIdx.x + NT * XR; i < xu; i += NT) lds[i] = xg[i];
  if constexpr (XF) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    prefetch_units<D>(buf, cur, packed, nc, g, r);
  }
  for (int i = threadIdx.x; i < nsub * M * 16; i += NT) sums[i] = 0;
  if (threadIdx.x < 16) lds[zero_idx + threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  stream_units<M, D>(buf, cur, packed, nc, t0, u0, u1, g, r, lds, kp16, zero_idx, sums);
  __syncthreads();
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = gamma_over_s(gm, fac[m]);
  stream_epilogue<M>(sums, t0, nsub, n, fac, relu2 != 0, ybf16 != 0, y, acc_out, NT);
}

// ----------------------------------------------------- fused decode step --
// A table of products sharing the token count (the entries of FusedArgs;
// `splits` of an entry holds its workgroup count here).  Each workgroup
// quantizes its entry's whole activation rows into LDS before streaming:
//   1. the activations are loaded first (XR 16-byte units per thread and
//      token, clamped: the units past the row repeat the last one, which the
//      max ignores), then the first D weight units (on long one-token rows
//      once the activations have arrived);
//   2. beta = max|x| per token (absmax_bf16x2 / absmax_f32x2, DPP in the
//      wave, LDS across waves) and s = fp32(127 / max(beta, eps)) exactly as
//      bitlinear_quant_act computes it;
//   3. x~ = clamp(rint(fp32(x * s))) of every held unit into LDS
//      (quant4_rne, whose clamp cannot bind), zero past K; every workgroup
//      of an entry computes the same s and x~ bit for bit.
// Rows must be whole 16-byte units at 16-byte alignment (checked on the host).
// With NORM, entries flagged for RMSNorm first normalize each token (the
// BitLinear listing of "End-to-End Implementation: Building a Native
// BitLinear Layer" applies nn.RMSNorm before quantize_activations_int8):
// the fp64 sum of squares of the held units, reduced in a fixed order (xor
// butterfly in the wave, waves in order), r = rms_factor(sum, K, eps), and
// y = fp32(fp32(x * r) * w) replaces x in steps 2 and 3.
template <int M, int WAVES, int D, int XR, bool BF16, bool NORM>
__global__ __launch_bounds__(64 * WAVES) void gemv_stream_fused_kernel(
    int nseg, int wb1, int wb2, int wb3, int wb4, int wb5, int wb6, int wb7, int wb8, int wb9,
    int wb10, int wb11, int wb12, int wb13, FusedArgs args) {
  constexpr int NT = 64 * WAVES;
  constexpr int EPU = BF16 ? 8 : 4;                  // activations per 16-byte unit
  constexpr int WPU = EPU / 4;                       // 16-byte gain units per activation unit
  extern __shared__ uint4 lds[];
  __shared__ uint32_t red[WAVES][M];
  __shared__ double red64[NORM ? WAVES : 1][M];
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
  const int local = bid - sg.wg_begin;
  const int G = sg.splits;
  const int nc = sg.nc, n = sg.n, k = sg.k;
  const int S = ((n + kRowBlock - 1) / kRowBlock) * 4;
  const int t0 = (int)((int64_t)S * local / G), t1 = (int)((int64_t)S * (local + 1) / G);
  const int nsub = t1 - t0, units = nsub * nc;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int kp16 = nc * 16;
  const int u0 = (int)((int64_t)units * wave / WAVES);
  const int u1 = (int)((int64_t)units * (wave + 1) / WAVES);
  const int nsub_alloc = args.nsub_alloc;
  int* sums = reinterpret_cast<int*>(lds + M * kp16);
  const int zero_idx = stream_zero_idx(M, kp16, nsub_alloc);
  const uint4* packed = reinterpret_cast<const uint4*>(sg.packed);

  // 1. activations (and the RMSNorm gain), then weights
  const int nu = k / EPU;                             // units per row (whole units)
  uint4 xr[M][XR];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint4* row = reinterpret_cast<const uint4*>(sg.x) + (int64_t)m * nu;
#pragma unroll
    for (int j = 0; j < XR; ++j) xr[m][j] = row[min((int)threadIdx.x + NT * j, nu - 1)];
  }
  const bool nrm = NORM && sg.rmsnorm();
  const bool have_w = nrm && sg.norm_weight != nullptr;
  uint4 wr[NORM ? XR : 1][WPU];
  if (NORM) {
    // without a gain the loads read the packed weights instead (at least as
    // long as the gain would be), which are never used: no load behind a branch
    const uint4* wsrc = have_w ? reinterpret_cast<const uint4*>(sg.norm_weight) : packed;
#pragma unroll
    for (int j = 0; j < XR; ++j)
#pragma unroll
      for (int h = 0; h < WPU; ++h)
        wr[j][h] = wsrc[min((int)threadIdx.x + NT * j, nu - 1) * WPU + h];
  }
  // one token with 8 units a thread (rows past 16384 inputs at 8 waves):
  // the activations land before any weight is requested (gemv_stream_xfirst)
  if constexpr (M == 1 && XR >= 8) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_sched_barrier(0);
  }
  uint4 buf[D];
  Cursor cur = cursor_at(packed, nc, t0, u0, u1, g, r);
  prefetch_units<D>(buf, cur, packed, nc, g, r);
  const float gm = *sg.gamma;
  for (int i = threadIdx.x; i < nsub * M * 16; i += NT) sums[i] = 0;
  if (threadIdx.x < 16) lds[zero_idx + threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);

  // the EPU activations of held unit j of token m as fp32 bit patterns
  auto raw_vals = [&](int m, int j, uint32_t (&v)[8]) __attribute__((always_inline)) {
    const uint4 x = xr[m][j];
    if (BF16) {
      v[0] = x.x << 16; v[1] = x.x & 0xFFFF0000u; v[2] = x.y << 16; v[3] = x.y & 0xFFFF0000u;
      v[4] = x.z << 16; v[5] = x.z & 0xFFFF0000u; v[6] = x.w << 16; v[7] = x.w & 0xFFFF0000u;
    } else {
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    }
  };
  float rn[M];                                        // RMSNorm factors
#pragma unroll
  for (int m = 0; m < M; ++m) rn[m] = 1.0f;
  if (nrm) {
    double ss[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      ss[m] = 0.0;
#pragma unroll
      for (int j = 0; j < XR; ++j) {
        if ((int)threadIdx.x + NT * j < nu) {
          uint32_t v[8];
          raw_vals(m, j, v);
#pragma unroll
          for (int e = 0; e < EPU; ++e) {
            const double d = (double)__uint_as_float(v[e]);
            ss[m] += d * d;
          }
        }
      }
    }
    // the tokens' xor butterflies step by step together (each token's sum
    // takes the same additions as a butterfly of its own)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      double s[M];
#pragma unroll
      for (int m = 0; m < M; ++m) s[m] = __shfl_xor(ss[m], o);
#pragma unroll
      for (int m = 0; m < M; ++m) ss[m] += s[m];
    }
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) red64[wave][m] = ss[m];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      double t = red64[0][m];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) t += red64[w][m];
      rn[m] = rms_factor(t, k, sg.norm_eps);
    }
  }
  // the values the quantization sees: x, or y = (x r) w
  auto vals = [&](int m, int j, uint32_t (&v)[8]) __attribute__((always_inline)) {
    raw_vals(m, j, v);
    if (NORM && nrm) {
      const uint32_t wv[8] = {wr[j][0].x, wr[j][0].y, wr[j][0].z, wr[j][0].w,
                              wr[j][WPU - 1].x, wr[j][WPU - 1].y, wr[j][WPU - 1].z,
                              wr[j][WPU - 1].w};
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const float w = have_w ? __uint_as_float(wv[e]) : 1.0f;
        v[e] = __float_as_uint(rms_apply(__uint_as_float(v[e]), rn[m], w));
      }
    }
  };

  // 2. beta and s per token: bf16 without RMSNorm one v_pk_maximum3_f16 per
  //    word (absmax_bf16x2; a magnitude above 2^121 flags the block, which
  //    then takes the exact sign-cleared 16-bit max), fp32 values two per
  //    v_max3_f32 (absmax_f32x2); DPP in the wave, LDS across waves
  const bool pk = BF16 && !(NORM && nrm);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    uint32_t mx = 0;
    if (pk) {
      uint32_t acc[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < XR; ++j) {
        acc[0] = absmax_bf16x2(acc[0], xr[m][j].x); acc[1] = absmax_bf16x2(acc[1], xr[m][j].y);
        acc[0] = absmax_bf16x2(acc[0], xr[m][j].z); acc[1] = absmax_bf16x2(acc[1], xr[m][j].w);
      }
      mx = absmax_bf16x2_bits(absmax_bf16x2(acc[0], acc[1]));
    } else {
#pragma unroll
      for (int j = 0; j < XR; ++j) {
        uint32_t v[8];
        vals(m, j, v);
#pragma unroll
        for (int e = 0; e < EPU; e += 2) mx = absmax_f32x2(mx, v[e], v[e + 1]);
      }
    }
    mx = wave_max_u32(mx);
    if (lane == 0) red[wave][m] = mx;
  }
  __syncthreads();
  uint32_t bmax[M];
  bool inexact = false;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    uint32_t b = red[0][m];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) b = max(b, red[w][m]);
    bmax[m] = b;
    inexact = inexact || (pk && b == kAbsmaxInexact);
  }
  if (inexact) {                                      // uniform: every thread read the same
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      bl_u16x2 m16 = {0, 0};
#pragma unroll
      for (int j = 0; j < XR; ++j) {
        m16 = absmax_bf16x2_exact(m16, xr[m][j].x); m16 = absmax_bf16x2_exact(m16, xr[m][j].y);
        m16 = absmax_bf16x2_exact(m16, xr[m][j].z); m16 = absmax_bf16x2_exact(m16, xr[m][j].w);
      }
      const uint32_t mx = wave_max_u32((uint32_t)max(m16[0], m16[1]) << 16);
      if (lane == 0) red[wave][m] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      uint32_t b = red[0][m];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) b = max(b, red[w][m]);
      bmax[m] = b;
    }
  }
  float sv[M];
#pragma unroll
  for (int m = 0; m < M; ++m)
    sv[m] = (float)(127.0 / (double)fmaxf(__uint_as_float(bmax[m]), args.eps));

  // 3. x~ into LDS (bytes EPU*u .. of token m), zero from K to K_pad
  uint32_t* xw = reinterpret_cast<uint32_t*>(lds);
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const int u = (int)threadIdx.x + NT * j;
      if (u < nu) {
        uint32_t v[8];
        vals(m, j, v);
        if (BF16) {
          const uint32_t d0 = quant4_rne(v[0], v[1], v[2], v[3], sv[m]);
          const uint32_t d1 = quant4_rne(v[4], v[5], v[6], v[7], sv[m]);
          reinterpret_cast<uint2*>(xw + m * kp16 * 4)[u] = make_uint2(d0, d1);
        } else {
          xw[m * kp16 * 4 + u] = quant4_rne(v[0], v[1], v[2], v[3], sv[m]);
        }
      }
    }
    for (int d = k / 4 + (int)threadIdx.x; d < kp16 * 4; d += NT) xw[m * kp16 * 4 + d] = 0u;
  }
  __syncthreads();
  if (local == 0) {                                   // optional copies of x~ and s
    if (sg.xq_out != nullptr)
      for (int m = 0; m < M; ++m)
        for (int i = threadIdx.x; i < kp16; i += NT)
          reinterpret_cast<uint4*>(sg.xq_out + (int64_t)m * kp16 * 16)[i] = lds[m * kp16 + i];
    if (sg.scale_out != nullptr && threadIdx.x < M) sg.scale_out[threadIdx.x] = sv[threadIdx.x];
  }

  stream_units<M, D>(buf, cur, packed, nc, t0, u0, u1, g, r, lds, kp16, zero_idx, sums);
  __syncthreads();
  float fac[M];
#pragma unroll
  for (int m = 0; m < M; ++m) fac[m] = gamma_over_s(gm, sv[m]);
  stream_epilogue<M>(sums, t0, nsub, n, fac, sg.relu2(), sg.y_bf16(), sg.y, sg.acc_out, NT);
}

template <int M, int WAVES, int D, int XR>
void run_stream(const int8_t* xq, const float* scale, const uint32_t* packed,
                const float* gamma, int n, int nc, int S, int G, int nsub_alloc, bool relu2,
                bool bf16, void* y, int32_t* acc_out, size_t lds, hipStream_t stream) {
  if (gemv_stream_xfirst(M, nc))
    gemv_stream_kernel<M, WAVES, D, XR, true><<<G, 64 * WAVES, lds, stream>>>(
        xq, scale, reinterpret_cast<const uint4*>(packed), gamma, n, nc, S, G, nsub_alloc,
        relu2, bf16, y, acc_out);
  else
    gemv_stream_kernel<M, WAVES, D, XR, false><<<G, 64 * WAVES, lds, stream>>>(
        xq, scale, reinterpret_cast<const uint4*>(packed), gamma, n, nc, S, G, nsub_alloc,
        relu2, bf16, y, acc_out);
}

template <int M, int WAVES, int D>
void run_stream_xr(int xr, const int8_t* xq, const float* scale, const uint32_t* packed,
                   const float* gamma, int n, int nc, int S, int G, int nsub_alloc, bool relu2,
                   bool bf16, void* y, int32_t* acc_out, size_t lds, hipStream_t stream) {
  if (xr <= 1)
    run_stream<M, WAVES, D, 1>(xq, scale, packed, gamma, n, nc, S, G, nsub_alloc, relu2, bf16, y,
                               acc_out, lds, stream);
  else if (xr <= 2)
    run_stream<M, WAVES, D, 2>(xq, scale, packed, gamma, n, nc, S, G, nsub_alloc, relu2, bf16, y,
                               acc_out, lds, stream);
  else if (xr <= 4)
    run_stream<M, WAVES, D, 4>(xq, scale, packed, gamma, n, nc, S, G, nsub_alloc, relu2, bf16, y,
                               acc_out, lds, stream);
  else
    run_stream<M, WAVES, D, 8>(xq, scale, packed, gamma, n, nc, S, G, nsub_alloc, relu2, bf16, y,
                               acc_out, lds, stream);
}

template <int M, int WAVES, int D, int XR, bool NORM>
void run_stream_fused(const FusedArgs& args, const int (&wb)[14], int groups, size_t lds,
                      bool bf16, hipStream_t stream) {
#define BL_SF(B)                                                                             \
  gemv_stream_fused_kernel<M, WAVES, D, XR, B, NORM><<<groups, 64 * WAVES, lds, stream>>>(   \
      args.nseg, wb[1], wb[2], wb[3], wb[4], wb[5], wb[6], wb[7], wb[8], wb[9], wb[10],      \
      wb[11], wb[12], wb[13], args)
  if (bf16)
    BL_SF(true);
  else
    BL_SF(false);
#undef BL_SF
}

template <int M, int WAVES, int D, bool NORM>
void run_stream_fused_xr(int xr, const FusedArgs& args, const int (&wb)[14], int groups,
                         size_t lds, bool bf16, hipStream_t stream) {
  // the plan keeps M * xr <= 8 (the activation registers), and xr <= 4 with
  // RMSNorm (the gain registers)
  if (xr <= 2) {
    run_stream_fused<M, WAVES, D, 2, NORM>(args, wb, groups, lds, bf16, stream);
  } else if constexpr (M > 1 && NORM) {
    // unreachable: the plan keeps M * xr <= 4 with RMSNorm
    run_stream_fused<M, WAVES, D, 2, NORM>(args, wb, groups, lds, bf16, stream);
  } else if constexpr (M > 1 || NORM) {
    run_stream_fused<M, WAVES, D, 4, NORM>(args, wb, groups, lds, bf16, stream);
  } else {
    if (xr <= 4)
      run_stream_fused<M, WAVES, D, 4, NORM>(args, wb, groups, lds, bf16, stream);
    else  // 8 waves x 5 units on these long rows (100B-class down 12.57 -> 12.45 us
          // against 6 in alternating runs on MI355X; 5 on the 8192-input rows
          // made q/k/v and o slower)
      run_stream_fused<M, WAVES, (WAVES == 8 && D == 6 ? 5 : D), 8, NORM>(args, wb, groups, lds,
                                                                         bf16, stream);
  }
}

template <int M, int WAVES, int D>
void run_stream_fused_n(bool norm, int xr, const FusedArgs& args, const int (&wb)[14],
                        int groups, size_t lds, bool bf16, hipStream_t stream) {
  if (norm)
    run_stream_fused_xr<M, WAVES, D, true>(xr, args, wb, groups, lds, bf16, stream);
  else
    run_stream_fused_xr<M, WAVES, D, false>(xr, args, wb, groups, lds, bf16, stream);
}

}  // namespace

size_t stream_lds_bytes(int m, int64_t nc, int nsub_alloc) {
  return (size_t)stream_zero_idx(m, (int)(nc * 16), nsub_alloc) * 16 + 16 * 16;
}

// Waves per workgroup and units in flight per wave: 8 x 4 at one token on
// rows of fewer than 64 super-chunks, else 16 x 3.  (Swept on MI355X over
// the 100B-class shapes at one and two tokens: 8 x 4, 16 x 2/3/4, 8 x 6.)
void stream_shape(int m, int64_t nc, int* waves, int* depth) {
  if (m == 1 && nc < 64) {
    *waves = 8;
    *depth = 4;
  } else {
    *waves = 16;
    *depth = 3;
  }
}

// The fused form: 8 waves x 6 units in flight (wide = false), or 16 x 3 when
// a token's activation row does not fit the registers of 8 waves (the plan
// decides); one-token rows of 8 units a thread take 5 units in flight
// (run_stream_fused_xr).  (Swept on MI355X over the 100B-class products and
// q/k/v at one and two tokens: 8 x 6 against the plain shapes 2-3.5% faster
// at one token, 7-14% at two; 8 x 5 and 8 x 7 against 8 x 6 on the whole
// one-token layer step.)
void stream_fused_shape(bool wide, int* waves, int* depth) {
  *waves = wide ? 16 : 8;
  *depth = wide ? 3 : 6;
}

hipError_t launch_gemv_stream(int m, const int8_t* xq, const float* scale,
                              const uint32_t* packed, const float* gamma, int64_t n, int64_t k,
                              int grid, bool relu2, bool bf16, void* y, int32_t* acc_out,
                              hipStream_t stream) {
  const int nc = (int)cdiv(k, kSuperK);
  const int S = (int)(cdiv(n, kRowBlock) * 4);
  const int G = grid < S ? grid : S;
  const int nsub_alloc = (int)cdiv(S, G);
  const size_t lds = stream_lds_bytes(m, nc, nsub_alloc);
  int waves, depth;
  stream_shape(m, nc, &waves, &depth);
  const int xr = (int)cdiv((int64_t)m * nc * 16, 64 * waves);
  if (m == 1) {
    if (waves == 8)
      run_stream_xr<1, 8, 4>(xr, xq, scale, packed, gamma, (int)n, nc, S, G, nsub_alloc, relu2,
                             bf16, y, acc_out, lds, stream);
    else
      run_stream_xr<1, 16, 3>(xr, xq, scale, packed, gamma, (int)n, nc, S, G, nsub_alloc, relu2,
                              bf16, y, acc_out, lds, stream);
  } else if (m == 2) {
    run_stream_xr<2, 16, 3>(xr, xq, scale, packed, gamma, (int)n, nc, S, G, nsub_alloc, relu2,
                            bf16, y, acc_out, lds, stream);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_stream_fused(const FusedArgs& args, int m, bool wide, bool x_bf16,
                                    bool norm, int xr, int groups, size_t lds,
                                    hipStream_t stream) {
  int wb[14];
  for (int i = 1; i < 14; ++i) wb[i] = i < args.nseg ? args.wg_begin[i] : INT_MAX;
  if (m == 1) {
    if (wide)
      run_stream_fused_n<1, 16, 3>(norm, xr, args, wb, groups, lds, x_bf16, stream);
    else
      run_stream_fused_n<1, 8, 6>(norm, xr, args, wb, groups, lds, x_bf16, stream);
  } else if (m == 2) {
    if (wide)
      run_stream_fused_n<2, 16, 3>(norm, xr, args, wb, groups, lds, x_bf16, stream);
    else
      run_stream_fused_n<2, 8, 6>(norm, xr, args, wb, groups, lds, x_bf16, stream);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bl
