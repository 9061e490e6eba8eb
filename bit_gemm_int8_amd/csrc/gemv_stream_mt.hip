// Decode products for 3 to 64 tokens (and larger batches whose outputs are
// few) on the int8 matrix cores: the streaming GEMV of whole 16-row
// sub-blocks, with x~ of a block of up to 16 tokens in LDS; plain (x~ and s
// given) and fused (the activation quantization in the prologue, for a
// table of products).
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T in an integer
// accumulator, y = acc * gamma / s; section "8-Bit Activation Quantization:
// absmax Scaling" for x~ and s.
//
// v_mfma_i32_16x16x64_i8 has 16 result columns, so one instruction per
// packed word serves 16 tokens as easily as one: the weight stream of the
// one/two-token kernel carries over and the second operand becomes x~ of 16
// real tokens.  The work of a product is cut into (row range, token block):
//   - token block b holds tokens 16 b .. 16 b + 15 (fewer in the last); its
//     x~ (all of K) sits in LDS, 16-byte unit q of token t's row at
//     q ^ (t % 16), so the 16 tokens of one operand read fall on 16
//     different bank groups;
//   - a row range is whole 16-row sub-blocks over all of K (no K split: no
//     workspace, no atomics in memory), its 1 KiB units cut into one
//     contiguous run per wave, D units in flight per wave;
//   - the token blocks of one row range run on one XCD (workgroup w of a
//     launch runs on XCD w % 8), so after one block has read a weight from
//     HBM the others find it in that XCD's L2.
// Every workgroup reads its block's whole x~ (fused: its activations), so
// more row ranges fill the chip better and re-read more; the plans take
// about one workgroup per CU.
#include <climits>

#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kTokBlock = 16;   // tokens per block of the plain form (the fused form: TBK)
// Word 3 of a raw buffer resource on gfx9 (untyped 32-bit data; loads past
// num_records return zero).
constexpr int kBufferDword3 = 0x00020000;

// (row range, token block) of workgroup w of a product with P row ranges and
// TB token blocks.  With P a multiple of 8, the TB workgroups of a row range
// are w = 8 TB a + 8 b + (p % 8), all on XCD p % 8.
struct MtWork {
  int p, tb;
};
__device__ __forceinline__ MtWork mt_work(int w, int P, int TB) {
  if (TB == 1) return {w, 0};
  if ((P & 7) == 0) return {(w / (8 * TB)) * 8 + (w & 7), (w >> 3) % TB};
  return {w % P, w / P};
}

// Wave cursor over 1 KiB units: unit v is sub-block tl, super-chunk cl;
// loads past the wave's last unit repeat it (no branch around the loads).
struct MtCursor {
  const uint4* base;
  int vl, tl, cl, ulast;
};

__device__ __forceinline__ const uint4* mt_sub_base(const uint4* packed, int nc, int t, int g,
                                                    int r) {
  return packed + ((int64_t)(t >> 2) * nc * 4 + g) * 64 + (t & 3) * 16 + r;
}

__device__ __forceinline__ MtCursor mt_cursor(const uint4* packed, int nc, int t0, int u0, int u1,
                                              int g, int r) {
  MtCursor c;
  c.ulast = u1 > 0 ? u1 - 1 : 0;
  c.vl = min(u0, c.ulast);
  c.tl = t0 + c.vl / nc;
  c.cl = c.vl - (c.vl / nc) * nc;
  c.base = mt_sub_base(packed, nc, c.tl, g, r);
  return c;
}

__device__ __forceinline__ void mt_next(MtCursor& c, const uint4* packed, int nc, int g, int r) {
  if (c.vl < c.ulast) {
    ++c.vl;
    if (++c.cl == nc) {
      c.cl = 0;
      ++c.tl;
      c.base = mt_sub_base(packed, nc, c.tl, g, r);
    }
  }
}

template <int D>
__device__ __forceinline__ void mt_prefetch(uint4 (&buf)[D], MtCursor& cur, const uint4* packed,
                                            int nc, int g, int r) {
  static_for<D>([&](auto P) {
    buf[(int)P] = load_stream16(cur.base + (int64_t)cur.cl * kBlockU4);
    mt_next(cur, packed, nc, g, r);
  });
}

// Stream units [u0, u1) (sub-blocks from t0, nc super-chunks each; the first
// D already in buf) and add each sub-block's sums into
// sums[sub - t0][token][row].  Lane (r, g): token min(r, mb - 1) as the
// second operand (columns of tokens >= mb are dropped), inputs 64 j + 16 g
// .. + 15 of super-chunk cc, i.e. x~ unit 16 cc + ((4 j + g) ^ token).
template <int D, int TBK>
__device__ __forceinline__ void mt_stream(uint4 (&buf)[D], MtCursor& cur, const uint4* packed,
                                          int nc, int t0, int u0, int u1, int g, int r, int mb,
                                          const uint4* xs, int kp16, int* sums) {
  const int tr = min(r, mb - 1);
  const uint4* xrow = xs + tr * kp16;
  bl_v4i acc = {0, 0, 0, 0};
  int tc = t0 + u0 / nc, cc = u0 - (u0 / nc) * nc;
  auto flush = [&]() __attribute__((always_inline)) {
    if (r < mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        atomicAdd(&sums[((tc - t0) * TBK + r) * 16 + 4 * g + i], acc[i]);
    }
    acc = bl_v4i{0, 0, 0, 0};
  };
  auto consume = [&](const uint4& w) __attribute__((always_inline)) {
    const uint32_t wj[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 x4 = xrow[cc * 16 + ((4 * j + g) ^ tr)];
      const bl_v4i xv = {(int)x4.x, (int)x4.y, (int)x4.z, (int)x4.w};
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
      mt_next(cur, packed, nc, g, r);
    });
  }
  static_for<D>([&](auto P) {
    constexpr int p = decltype(P)::value;
    if (v + p < u1) consume(buf[p]);
  });
  if (u1 > u0 && cc != 0) flush();
}

// Outputs of sub-blocks t0 .. t0 + nsub - 1 for tokens tok0 .. tok0 + mb - 1
// from the LDS sums (64 * acc, exact), four consecutive rows per thread.
template <int TBK>
__device__ __forceinline__ void mt_epilogue(const int* sums, const float* fac, int t0, int nsub,
                                            int mb, int tok0, int n, bool relu2, bool ybf16,
                                            bool vec, void* y, int32_t* acc_out, int nt) {
  const int quads = nsub * 4;
  for (int i = threadIdx.x; i < quads * mb; i += nt) {
    const int m = i / quads, qd = i - m * quads;
    const int sub = qd >> 2, rr = (qd & 3) * 4;
    const int row0 = (t0 + sub) * 16 + rr;
    if (row0 >= n) continue;
    const bl_v4i a4 = *reinterpret_cast<const bl_v4i*>(sums + (sub * TBK + m) * 16 + rr);
    const float f = fac[m];
    const int64_t idx = (int64_t)(tok0 + m) * n + row0;
    int v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = a4[e] >> 6;
    if (vec && row0 + 3 < n) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = (float)v[e] * f;
        if (relu2) o[e] = o[e] > 0.0f ? o[e] * o[e] : 0.0f;
      }
      if (acc_out != nullptr)
        *reinterpret_cast<int4*>(acc_out + idx) = make_int4(v[0], v[1], v[2], v[3]);
      if (ybf16)
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + idx) =
            make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      else
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + idx) =
            make_float4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (row0 + e >= n) continue;
        if (acc_out != nullptr) acc_out[idx + e] = v[e];
        store_out(y, idx + e, v[e], f, relu2, ybf16);
      }
    }
  }
}

// ------------------------------------------------------------ plain GEMV --
// x~ [m][K_pad] and s given.  LDS: x~ [mba][kp16] uint4 (mba = min(16, m)
// rows, swizzled), sums [nsub_alloc][16][16] int, fac [16] float.
template <int WAVES, int D, int XR>
__global__ __launch_bounds__(64 * WAVES) void gemv_stream_mt_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ scale,
    const uint4* __restrict__ packed, const float* __restrict__ gamma, int m, int n, int nc,
    int S, int P, int TB, int nsub_alloc, int mba, int relu2, int ybf16, int vec_out,
    void* __restrict__ y, int32_t* __restrict__ acc_out) {
  constexpr int NT = 64 * WAVES;
  extern __shared__ uint4 lds[];
  const MtWork wk = mt_work((int)blockIdx.x, P, TB);
  const int tok0 = kTokBlock * wk.tb;
  const int mb = min(kTokBlock, m - tok0);
  const int t0 = (int)((int64_t)S * wk.p / P), t1 = (int)((int64_t)S * (wk.p + 1) / P);
  const int nsub = t1 - t0, units = nsub * nc;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int kp16 = nc * 16;
  const int u0 = (int)((int64_t)units * wave / WAVES);
  const int u1 = (int)((int64_t)units * (wave + 1) / WAVES);
  int* sums = reinterpret_cast<int*>(lds + mba * kp16);
  float* fac = reinterpret_cast<float*>(sums + nsub_alloc * kTokBlock * 16);

  // x~ of the block first (loads retire in issue order), clamped so no load
  // sits behind a branch
  const int xu = mb * kp16;
  const uint4* xg = reinterpret_cast<const uint4*>(xq) + (int64_t)tok0 * kp16;
  uint4 xr[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) xr[j] = xg[min((int)threadIdx.x + NT * j, xu - 1)];
  uint4 buf[D];
  MtCursor cur = mt_cursor(packed, nc, t0, u0, u1, g, r);
  mt_prefetch<D>(buf, cur, packed, nc, g, r);
  const float gm = *gamma;
  if ((int)threadIdx.x < mb) fac[threadIdx.x] = gamma_over_s(gm, scale[tok0 + threadIdx.x]);
  for (int i = threadIdx.x; i < nsub * kTokBlock * 16; i += NT) sums[i] = 0;
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int i = (int)threadIdx.x + NT * j;
    if (i < xu) {
      const int t = i / kp16, q = i - t * kp16;
      lds[t * kp16 + (q ^ (t & 15))] = xr[j];
    }
  }
  for (int i = (int)threadIdx.x + NT * XR; i < xu; i += NT) {
    const int t = i / kp16, q = i - t * kp16;
    lds[t * kp16 + (q ^ (t & 15))] = xg[i];
  }
  __syncthreads();

  mt_stream<D, kTokBlock>(buf, cur, packed, nc, t0, u0, u1, g, r, mb, lds, kp16, sums);
  __syncthreads();
  mt_epilogue<kTokBlock>(sums, fac, t0, nsub, mb, tok0, n, relu2 != 0, ybf16 != 0, vec_out != 0,
                         y, acc_out, NT);
}

// ----------------------------------------------------- fused decode step --
// A table of products sharing the tokens (FusedArgs; `splits` of an entry
// holds its workgroup count, P row ranges x TB token blocks).  A workgroup
// quantizes its block's activation rows into LDS, one wave per token:
//   1. an RMSNorm entry's gain, then the token's row (XR 16-byte units per
//      lane by range-checked buffer loads: units past the row read as zeros,
//      which change neither the max nor the sum of squares), then the first
//      D weight units;
//   2. with RMSNorm (entries flagged for it; the BitLinear listing of
//      "End-to-End Implementation: Building a Native BitLinear Layer"
//      applies nn.RMSNorm before quantize_activations_int8), from the held
//      row: the fp64 sum of squares in the order bitlinear_rmsnorm_quant_act
//      takes (so both get the same r), r = rms_factor(sum, K, eps), and
//      y = fp32(fp32(x * r) * w) replaces x below, the gain w staged in LDS
//      once per workgroup;
//   3. beta = max|x| (absmax_bf16x2 / absmax_f32x2, then a wave max) and
//      s = fp32(127 / max(beta, eps)) exactly as bitlinear_quant_act;
//   4. x~ = clamp(rint(fp32(x * s))) (quant4_rne, whose clamp cannot bind)
//      into LDS, zero past K; the entry's first row range also writes x~
//      and s out when asked.
// Rows must be whole 16-byte units at 16-byte alignment (checked on the host).
template <int TBK, int WAVES, int D, int XR, bool BF16, bool NORM>
__global__ __launch_bounds__(64 * WAVES) void gemv_stream_mt_fused_kernel(
    int m_all, int nseg, int wb1, int wb2, int wb3, int wb4, int wb5, int wb6, int wb7, int wb8,
    int wb9, int wb10, int wb11, int wb12, FusedArgs args) {
  constexpr int NT = 64 * WAVES;
  constexpr int EPU = BF16 ? 8 : 4;                  // activations per 16-byte unit
  extern __shared__ uint4 lds[];
  const int bid = (int)blockIdx.x;
  const int wb[12] = {wb1, wb2, wb3, wb4, wb5, wb6, wb7, wb8, wb9, wb10, wb11, wb12};
  int si = 0;
#pragma unroll
  for (int i = 0; i < 12; ++i) si = bid >= wb[i] ? i + 1 : si;
  if (nseg > 13) {
#pragma unroll
    for (int i = 13; i < kMaxFused; ++i)
      if (i < nseg && bid >= args.wg_begin[i]) si = i;
  }
  const FusedSeg& sg = args.seg[si];
  const int TB = (m_all + TBK - 1) / TBK;
  const int P = sg.splits / TB;
  const MtWork wk = mt_work(bid - sg.wg_begin, P, TB);
  const int tok0 = TBK * wk.tb;
  const int mb = min(TBK, m_all - tok0);
  const int mba = min(TBK, m_all);
  const int nc = sg.nc, n = sg.n, k = sg.k;
  const int S = ((n + kRowBlock - 1) / kRowBlock) * 4;
  const int t0 = (int)((int64_t)S * wk.p / P), t1 = (int)((int64_t)S * (wk.p + 1) / P);
  const int nsub = t1 - t0, units = nsub * nc;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int kp16 = nc * 16;
  const int u0 = (int)((int64_t)units * wave / WAVES);
  const int u1 = (int)((int64_t)units * (wave + 1) / WAVES);
  int* sums = reinterpret_cast<int*>(lds + mba * kp16);
  float* fac = reinterpret_cast<float*>(sums + args.nsub_alloc * TBK * 16);
  float* gl = fac + TBK;                              // RMSNorm gain (entries with one)
  const uint4* packed = reinterpret_cast<const uint4*>(sg.packed);
  const int nu = k / EPU;                             // units per row (whole units)
  const bool nrm = NORM && sg.rmsnorm();
  const uint4* gw = reinterpret_cast<const uint4*>(sg.norm_weight);
  const bool have_w = nrm && gw != nullptr;
  const bool first = wk.p == 0;

  // 1. this wave's first token (waves past the block load its last token
  //    again: no load behind a branch), then the weights
  //    (a buffer load past the row's nu units returns zeros, which the max
  //    ignores and which are never stored; the whole offset is in the
  //    range-checked vector offset)
  auto load_row = [&](int t, uint4 (&xr)[XR]) __attribute__((always_inline)) {
    const uint4* row = reinterpret_cast<const uint4*>(sg.x) + (int64_t)(tok0 + t) * nu;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(row), 0, nu * 16, kBufferDword3);
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const bl_v4i v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + j * 1024, 0, 0);
      xr[j] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
    }
  };
  // an RMSNorm entry's gain (k floats as whole 16-byte pieces: rows are
  // whole units) is loaded first, so that waiting for it does not wait for
  // the row and weight loads issued after it (loads complete in order); it
  // goes to LDS below
  constexpr int GPT = (XR * 64 * EPU / 4 + NT - 1) / NT;   // gain pieces per thread, at most
  uint4 gv[NORM ? GPT : 1];
  if (NORM) {
    // no load behind a branch (its wait would come at once): indices
    // clamped, and without a gain the loads read the packed weights, unused
    const uint4* gsrc = have_w ? gw : packed;
    const int gn = have_w ? k / 4 : 1;
#pragma unroll
    for (int h = 0; h < GPT; ++h) gv[h] = gsrc[min((int)threadIdx.x + NT * h, gn - 1)];
  }
  uint4 xr[XR];
  load_row(min(wave, mb - 1), xr);
  uint4 buf[D];
  MtCursor cur = mt_cursor(packed, nc, t0, u0, u1, g, r);
  mt_prefetch<D>(buf, cur, packed, nc, g, r);
  const float gm = *sg.gamma;
  for (int i = threadIdx.x; i < nsub * TBK * 16; i += NT) sums[i] = 0;

  // the EPU values of a 16-byte activation unit as fp32 bit patterns
  auto expand = [&](const uint4& x, uint32_t (&v)[8]) __attribute__((always_inline)) {
    if (BF16) {
      v[0] = x.x << 16; v[1] = x.x & 0xFFFF0000u; v[2] = x.y << 16; v[3] = x.y & 0xFFFF0000u;
      v[4] = x.z << 16; v[5] = x.z & 0xFFFF0000u; v[6] = x.w << 16; v[7] = x.w & 0xFFFF0000u;
    } else {
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    }
  };
  // running max of |value| over units, two accumulators: bf16 words one
  // v_pk_maximum3_f16 each (absmax_bf16x2), fp32 pairs one v_max3_f32
  auto unit_max = [&](uint32_t (&acc)[2], const uint4& x) __attribute__((always_inline)) {
    if (BF16) {
      acc[0] = absmax_bf16x2(acc[0], x.x); acc[1] = absmax_bf16x2(acc[1], x.y);
      acc[0] = absmax_bf16x2(acc[0], x.z); acc[1] = absmax_bf16x2(acc[1], x.w);
    } else {
      acc[0] = absmax_f32x2(acc[0], x.x, x.y); acc[1] = absmax_f32x2(acc[1], x.z, x.w);
    }
  };
  auto max_bits = [&](const uint32_t (&acc)[2]) __attribute__((always_inline)) {
    return BF16 ? absmax_bf16x2_bits(absmax_bf16x2(acc[0], acc[1]))
                : absmax_f32x2(acc[0], acc[1], acc[1]);
  };
  // x~ of unit u (values v) into the token's LDS row (swizzled) and out
  uint32_t* xw = reinterpret_cast<uint32_t*>(lds);
  const int64_t kpad = (int64_t)kp16 * 16;
  auto put = [&](int t, int u, const uint32_t (&v)[8], float sv, uint32_t* rowo)
      __attribute__((always_inline)) {
    uint32_t* rowl = xw + t * kp16 * 4;
    if (BF16) {
      const uint32_t d0 = quant4_rne(v[0], v[1], v[2], v[3], sv);
      const uint32_t d1 = quant4_rne(v[4], v[5], v[6], v[7], sv);
      const int q = u >> 1;                           // x~ unit, half u & 1
      *reinterpret_cast<uint2*>(rowl + ((q ^ t) << 2) + ((u & 1) << 1)) = make_uint2(d0, d1);
      if (rowo != nullptr) *reinterpret_cast<uint2*>(rowo + 2 * u) = make_uint2(d0, d1);
    } else {
      const uint32_t d0 = quant4_rne(v[0], v[1], v[2], v[3], sv);
      const int q = u >> 2;
      rowl[((q ^ t) << 2) + (u & 3)] = d0;
      if (rowo != nullptr) rowo[u] = d0;
    }
  };
  // y = fp32(fp32(x * r) * w) of held unit j (RMSNorm); past the row x is 0
  // and so is y
  auto normed = [&](int j, float rn, uint32_t (&v)[8]) __attribute__((always_inline)) {
    expand(xr[j], v);
    float w[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
    if (have_w) {
      const int u = min(lane + 64 * j, nu - 1);
      const uint4* g4 = reinterpret_cast<const uint4*>(gl) + u * (EPU / 4);
#pragma unroll
      for (int h = 0; h < EPU / 4; ++h) {
        const uint4 g = g4[h];
        w[4 * h] = __uint_as_float(g.x); w[4 * h + 1] = __uint_as_float(g.y);
        w[4 * h + 2] = __uint_as_float(g.z); w[4 * h + 3] = __uint_as_float(g.w);
      }
    }
#pragma unroll
    for (int e = 0; e < EPU; ++e) v[e] = __float_as_uint(rms_apply(__uint_as_float(v[e]), rn, w[e]));
  };

  // one token per wave (TBK <= WAVES): wave t's row was loaded at the start
  static_assert(TBK <= WAVES, "one token per wave");
  const int t = wave;
  const bool has_tok = t < mb;
  // 2. with RMSNorm, the fp64 sum of squares of the held row, before the
  //    gain is needed.  bitlinear_rmsnorm_quant_act puts unit u on thread
  //    u % 256 of 256, each thread adding its units' squares in order, then
  //    sums each 64-thread wave by xor butterfly and the four waves in
  //    order; lane l holds units l + 64 j, the units of thread l + 64 (j % 4)
  //    in order, so four partial sums give the same fp64 total, bit for bit
  //    (units past the row add +0).
  float rn = 1.0f;
  if (NORM && nrm && has_tok) {
    double part[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      uint32_t v[8];
      expand(xr[j], v);
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const double d = (double)__uint_as_float(v[e]);
        part[j & 3] += d * d;
      }
    }
    // the four xor butterflies step by step together (each partial sum
    // takes the same additions as a butterfly of its own; the four
    // exchanges of a step are in flight at once), then added in order
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      double s[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) s[c] = __shfl_xor(part[c], o);
#pragma unroll
      for (int c = 0; c < 4; ++c) part[c] += s[c];
    }
    rn = rms_factor(((part[0] + part[1]) + part[2]) + part[3], k, sg.norm_eps);
  }
  // the gain into LDS (its loads were issued first and have had the sums'
  // time to arrive), before any wave normalizes
  if (NORM && have_w) {
    uint4* g4 = reinterpret_cast<uint4*>(gl);
#pragma unroll
    for (int h = 0; h < GPT; ++h) {
      const int i = (int)threadIdx.x + NT * h;
      if (i < k / 4) g4[i] = gv[h];
    }
    __syncthreads();
  }
  if (has_tok) {
    const bool out = first && sg.xq_out != nullptr;
    uint32_t* rowo = out ? reinterpret_cast<uint32_t*>(sg.xq_out + (int64_t)(tok0 + t) * kpad)
                         : nullptr;
    float sv;
    if (NORM && nrm) {
      // 3-4 with RMSNorm: beta = max|y|, then x~ of y
      uint32_t mx = 0;
#pragma unroll
      for (int j = 0; j < XR; ++j) {
        uint32_t v[8];
        normed(j, rn, v);
#pragma unroll
        for (int e = 0; e < EPU; e += 2) mx = absmax_f32x2(mx, v[e], v[e + 1]);
      }
      mx = wave_max_u32(mx);
      sv = (float)(127.0 / (double)fmaxf(__uint_as_float(mx), args.eps));
      // y again from the held row rather than all of it kept from the max
      // (the compiler would, and spill): the row counts as rewritten here
#pragma unroll
      for (int j = 0; j < XR; ++j)
        asm volatile("" : "+v"(xr[j].x), "+v"(xr[j].y), "+v"(xr[j].z), "+v"(xr[j].w));
#pragma unroll
      for (int j = 0; j < XR; ++j) {
        const int u = lane + 64 * j;
        if (u < nu) {
          uint32_t v[8];
          normed(j, rn, v);
          put(t, u, v, sv, rowo);
        }
      }
    } else {
      // 3-4 from the held row
      uint32_t acc[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < XR; ++j) unit_max(acc, xr[j]);
      uint32_t mx = wave_max_u32(max_bits(acc));
      if (BF16 && mx == kAbsmaxInexact) {             // |x| > 2^121 somewhere: exact max
        bl_u16x2 m16 = {0, 0};
#pragma unroll
        for (int j = 0; j < XR; ++j) {
          m16 = absmax_bf16x2_exact(m16, xr[j].x); m16 = absmax_bf16x2_exact(m16, xr[j].y);
          m16 = absmax_bf16x2_exact(m16, xr[j].z); m16 = absmax_bf16x2_exact(m16, xr[j].w);
        }
        mx = wave_max_u32((uint32_t)max(m16[0], m16[1]) << 16);
      }
      sv = (float)(127.0 / (double)fmaxf(__uint_as_float(mx), args.eps));
#pragma unroll
      for (int j = 0; j < XR; ++j) {
        const int u = lane + 64 * j;
        if (u < nu) {
          uint32_t v[8];
          expand(xr[j], v);
          put(t, u, v, sv, rowo);
        }
      }
    }
    uint32_t* rowl = xw + t * kp16 * 4;
    for (int d = k / 4 + lane; d < kp16 * 4; d += 64) {
      rowl[(((d >> 2) ^ t) << 2) + (d & 3)] = 0u;
      if (out) rowo[d] = 0u;
    }
    if (lane == 0) {
      fac[t] = gamma_over_s(gm, sv);
      if (first && sg.scale_out != nullptr) sg.scale_out[tok0 + t] = sv;
    }
  }
  __syncthreads();

  mt_stream<D, TBK>(buf, cur, packed, nc, t0, u0, u1, g, r, mb, lds, kp16, sums);
  __syncthreads();
  const bool ybf = sg.y_bf16();
  const bool vec = (n & 3) == 0 && ((uintptr_t)sg.y & (ybf ? 7 : 15)) == 0 &&
                   (sg.acc_out == nullptr || ((uintptr_t)sg.acc_out & 15) == 0);
  mt_epilogue<TBK>(sums, fac, t0, nsub, mb, tok0, n, sg.relu2(), ybf, vec, sg.y, sg.acc_out, NT);
}

template <int WAVES, int D, int XR>
void run_mt(const int8_t* xq, const float* scale, const uint32_t* packed, const float* gamma,
            int m, int n, int nc, int S, int P, int TB, int nsub_alloc, int mba, bool relu2,
            bool bf16, int vec_out, void* y, int32_t* acc_out, size_t lds, hipStream_t stream) {
  gemv_stream_mt_kernel<WAVES, D, XR><<<P * TB, 64 * WAVES, lds, stream>>>(
      xq, scale, reinterpret_cast<const uint4*>(packed), gamma, m, n, nc, S, P, TB, nsub_alloc,
      mba, relu2, bf16, vec_out, y, acc_out);
}

template <int TBK, int WAVES, int D, int XR, bool NORM>
void run_mt_fused(const FusedArgs& args, int m, const int (&wb)[13], int groups, size_t lds,
                  bool bf16, hipStream_t stream) {
#define BL_MF(B)                                                                               \
  gemv_stream_mt_fused_kernel<TBK, WAVES, D, XR, B, NORM><<<groups, 64 * WAVES, lds, stream>>>( \
      m, args.nseg, wb[1], wb[2], wb[3], wb[4], wb[5], wb[6], wb[7], wb[8], wb[9], wb[10],     \
      wb[11], wb[12], args)
  if (bf16)
    BL_MF(true);
  else
    BL_MF(false);
#undef BL_MF
}

}  // namespace

size_t stream_mt_lds_bytes(int64_t m, int64_t nc, int nsub_alloc, int tok, int64_t gain_k) {
  const int64_t mba = m < tok ? m : tok;
  return (size_t)(mba * nc * 256) + (size_t)nsub_alloc * tok * 16 * 4 + tok * 4 +
         (size_t)gain_k * 4;
}

hipError_t launch_gemv_stream_mt(const int8_t* xq, const float* scale, const uint32_t* packed,
                                 const float* gamma, int64_t m, int64_t n, int64_t k, int P,
                                 bool relu2, bool bf16, void* y, int32_t* acc_out,
                                 hipStream_t stream) {
  const int nc = (int)cdiv(k, kSuperK);
  const int S = (int)(cdiv(n, kRowBlock) * 4);
  const int TB = (int)cdiv(m, kTokBlock);
  if (P < 1 || P > S || m < 1) return hipErrorInvalidValue;
  const int nsub_alloc = (int)cdiv(S, P);
  const int mba = (int)(m < kTokBlock ? m : kTokBlock);
  const size_t lds = stream_mt_lds_bytes(m, nc, nsub_alloc, kTokBlock, 0);
  const int vec_out = n % 4 == 0 && (uintptr_t)y % (bf16 ? 8 : 16) == 0 &&
                      (acc_out == nullptr || (uintptr_t)acc_out % 16 == 0);
  const int xr = (int)cdiv((int64_t)mba * nc * 16, 64 * 16);
#define BL_MT(XR)                                                                          \
  run_mt<16, 3, XR>(xq, scale, packed, gamma, (int)m, (int)n, nc, S, P, TB, nsub_alloc, mba, \
                    relu2, bf16, vec_out, y, acc_out, lds, stream)
  if (xr <= 2)
    BL_MT(2);
  else if (xr <= 4)
    BL_MT(4);
  else
    BL_MT(8);
#undef BL_MT
  return hipGetLastError();
}

hipError_t launch_gemv_stream_mt_fused(const FusedArgs& args, int m, int tok, bool x_bf16,
                                       bool norm, int xr, int groups, size_t lds,
                                       hipStream_t stream) {
  int wb[13];
  for (int i = 1; i < 13; ++i) wb[i] = i < args.nseg ? args.wg_begin[i] : INT_MAX;
  wb[0] = 0;
  if (tok != 8 && tok != 16) return hipErrorInvalidValue;
#define BL_MTT(T, XR)                                                              \
  if (norm)                                                                        \
    run_mt_fused<T, 16, 3, XR, true>(args, m, wb, groups, lds, x_bf16, stream);    \
  else                                                                             \
    run_mt_fused<T, 16, 3, XR, false>(args, m, wb, groups, lds, x_bf16, stream)
#define BL_MTF(XR)                                                                 \
  if (tok == 8) {                                                                  \
    BL_MTT(8, XR);                                                                 \
  } else {                                                                         \
    BL_MTT(16, XR);                                                                \
  }
  if (xr <= 4) {
    BL_MTF(4);
  } else if (xr <= 8) {
    BL_MTF(8);
  } else if (xr <= 16) {
    BL_MTF(16);
  } else {
    return hipErrorInvalidValue;
  }
#undef BL_MTF
#undef BL_MTT
  return hipGetLastError();
}

}  // namespace bl
