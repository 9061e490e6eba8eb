// Decode products for 3 to 64 tokens on the int8 matrix cores, with the
// fused dequant (the windowed MFMA GEMV).
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T in an integer
// accumulator, then y = acc * gamma / s.  With a handful of tokens the
// product still reads every packed weight once for few operations per byte,
// so it is bound by HBM like the batch-1 GEMV; the matrix core does the
// multiply-adds for up to 16 tokens per instruction, which leaves the 2-bit
// unpack as the only VALU work per weight.
//
// v_mfma_i32_16x16x64_i8 operands: lane l = r + 16 g (r = l % 16, g = l / 16)
// supplies row r of the first operand and column r of the second for the 16
// inputs 64 j + 16 g + (0..15) of k-step j of a 256-input super-chunk.  The
// first operand is the unpacked weights (packed word (q = g, j) of row r: one
// 16-byte load per lane and super-chunk holds all four steps j), the second
// x~ of token r.  Byte e of operand dword i is input 4 i + e on both sides.
// The 16 x 16 result holds row 4 g + i, token r in element i of lane l, so a
// lane ends with four consecutive output rows of one token.
//
// x~ passes through LDS one super-chunk at a time, shared by the waves of a
// workgroup, so the rows may be of any length and K is never split over
// workgroups.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

// ---------------------------------------------------- windowed MFMA GEMV --
// Up to 16 * TG tokens.  A workgroup has WR x WK waves: WR row groups,
// group w owning the SB 16-row sub-blocks from (blockIdx * WR + w) * SB,
// and WK contiguous slices of the super-chunks, one per wave of a group (the
// slices' sums meet in LDS at the end).  Per
// super-chunk each slice stages x~[:, c] (16 * TG tokens x 256 bytes; tokens
// past m repeat the last token and their columns are dropped) in one of two
// LDS windows, with one workgroup barrier per step; each wave keeps PF
// super-chunks of its weights and of its share of x~ in flight in registers.
// In LDS the 16-byte unit u of token t sits at unit u ^ (t % 16), so the 16
// tokens of one operand read hit 16 different bank groups.  More tokens than
// 16 * TG run as token blocks of 16 * TG on blockIdx.y.
template <int WR, int WK, int SB, int TG, int PF>
__global__ __launch_bounds__(64 * WR * WK) void gemv_mfma_win_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ scale,
    const uint4* __restrict__ packed, const float* __restrict__ gamma, int m, int n, int nb,
    int nc, int64_t kpad, int relu2, int bf16, int vec_out, void* __restrict__ y,
    int32_t* __restrict__ acc_out) {
  static_assert(SB == 1 || SB == 2 || SB == 4, "a wave's sub-blocks lie in one packed block");
  static_assert(PF == 2 || PF == 4, "the loop is unrolled by PF, an even number");
  constexpr int NTS = 64 * WR;                      // threads staging one slice
  constexpr int MT = 16 * TG;                       // token columns
  // token block blockIdx.y: tokens MT * blockIdx.y .. + MT - 1
  {
    const int t0 = MT * (int)blockIdx.y;
    xq += (int64_t)t0 * kpad;
    scale += t0;
    y = reinterpret_cast<uint8_t*>(y) + (int64_t)t0 * n * (bf16 ? 2 : 4);
    if (acc_out != nullptr) acc_out += (int64_t)t0 * n;
    m = min(m - t0, MT);
  }
  constexpr int XU = MT * 16 / NTS;                 // x~ units per thread and super-chunk
  static_assert(MT * 16 % NTS == 0, "x~ staging split");
  __shared__ bl_v4i xs[WK][2][MT * 16];
  __shared__ int red[WK > 1 ? (WK - 1) * WR : 1][SB * TG * 4][64];
  __shared__ float fac_lds[MT];
  const int bs = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave / WK, wk = wave - wr * WK;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  int u0 = (bs * WR + wr) * SB;
  const bool live = u0 < nb * 4;
  if (!live) u0 = nb * 4 - SB;
  const int b = u0 >> 2, sub0 = u0 & 3;
  // this wave's slice [c0, c1) of the nc >= 1 super-chunks, L steps for
  // every wave (a short or empty last slice idles through the rest), and
  // the chunk its idle steps load
  const int L = (nc + WK - 1) / WK;
  const int c0 = wk * L;
  const int c1 = min(c0 + L, nc);
  const int clast = c1 > c0 ? c1 - 1 : nc - 1;
  const uint4* blk = packed + (int64_t)b * nc * kBlockU4 + g * 64 + sub0 * 16 + r;

  // this thread's x~ units of its slice: token t = q / 16 (clamped to
  // m - 1), unit q % 16
  const bl_v4i* xsrc[XU];
  int xdst[XU];
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int q = wr * 64 + lane + NTS * i;
    const int t = q >> 4, u = q & 15;
    xsrc[i] = reinterpret_cast<const bl_v4i*>(xq + (int64_t)min(t, m - 1) * kpad) + u;
    xdst[i] = t * 16 + (u ^ (t & 15));
  }
  bl_v4i xr[PF][XU];
  uint4 wb[PF][SB];
  auto load_chunk = [&](auto P, int c) {
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int i = 0; i < XU; ++i) xr[p][i] = xsrc[i][(int64_t)c * 16];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) wb[p][sb] = load_stream16(blk + (int64_t)c * kBlockU4 + sb * 16);
  };
  static_for<PF>([&](auto P) { load_chunk(P, min(c0 + (int)P, clast)); });
  if (threadIdx.x < MT) {
    const int t = threadIdx.x;
    fac_lds[t] = t < m ? gamma_over_s(*gamma, scale[t]) : 0.0f;
  }

  bl_v4i acc[SB][TG];
#pragma unroll
  for (int sb = 0; sb < SB; ++sb)
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) acc[sb][tg] = bl_v4i{0, 0, 0, 0};

  // one step: super-chunk c from slot p (its x~ window is LDS buffer p & 1)
  auto step = [&](auto P, int c) {
    constexpr int p = decltype(P)::value;
    bl_v4i* win = xs[wk][p & 1];
#pragma unroll
    for (int i = 0; i < XU; ++i) win[xdst[i]] = xr[p][i];
    __syncthreads();
    // the next loads into this slot stay where they are issued: moved
    // below a later wait they would drain the pipeline
    const int cn = min(c + PF, clast);
#pragma unroll
    for (int i = 0; i < XU; ++i) xr[p][i] = xsrc[i][(int64_t)cn * 16];
    __builtin_amdgcn_sched_barrier(0);
    if (c < c1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bl_v4i xv[TG];
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) xv[tg] = win[(16 * tg + r) * 16 + ((4 * j + g) ^ r)];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          const uint32_t wj = j == 0 ? wb[p][sb].x : j == 1 ? wb[p][sb].y
                            : j == 2 ? wb[p][sb].z : wb[p][sb].w;
          const bl_v4i a = {(int)unpack_x64(wj, 0), (int)unpack_x64(wj, 1),
                            (int)unpack_x64(wj, 2), (int)unpack_x64(wj, 3)};
#pragma unroll
          for (int tg = 0; tg < TG; ++tg)
            acc[sb][tg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, xv[tg], acc[sb][tg], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) wb[p][sb] = load_stream16(blk + (int64_t)cn * kBlockU4 + sb * 16);
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
        for (int tg = 0; tg < TG; ++tg)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            red[wr * (WK - 1) + wk - 1][(sb * TG + tg) * 4 + i][lane] = acc[sb][tg][i];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int w = 0; w < WK - 1; ++w)
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[sb][tg][i] += red[wr * (WK - 1) + w][(sb * TG + tg) * 4 + i][lane];
  }

  // lane (r, g) holds rows 4g..4g+3 of each sub-block for token 16 tg + r
  if (!live) return;
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int tk = 16 * tg + r;
    if (tk >= m) continue;
    const float f = fac_lds[tk];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      const int rb = (sub0 + sb) * 16 + 4 * g;      // first of 4 rows within the block
      int v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc[sb][tg][i] >> 6;
      const int row0 = b * 64 + rb;
      const int64_t idx = (int64_t)tk * n + row0;
      if (vec_out && row0 + 3 < n) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = (float)v[i] * f;
          if (relu2) o[i] = o[i] > 0.0f ? o[i] * o[i] : 0.0f;
        }
        if (acc_out != nullptr)
          *reinterpret_cast<int4*>(acc_out + idx) = make_int4(v[0], v[1], v[2], v[3]);
        if (bf16)
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + idx) =
              make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        else
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + idx) =
              make_float4(o[0], o[1], o[2], o[3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (row0 + i >= n) continue;
          if (acc_out != nullptr) acc_out[idx + i] = v[i];
          store_out(y, idx + i, v[i], f, relu2 != 0, bf16 != 0);
        }
      }
    }
  }
}

template <int WR, int WK, int SB, int TG, int PF>
hipError_t run_gemv_mfma_win(const int8_t* xq, const float* scale, const uint32_t* packed,
                             const float* gamma, int64_t m, int64_t n, int64_t k, bool relu2,
                             bool bf16, void* y, int32_t* acc_out, hipStream_t stream) {
  const int nb = (int)cdiv(n, kRowBlock);
  const int nc = (int)cdiv(k, kSuperK);
  if (m < 1 || nc < 1) return hipErrorInvalidValue;
  dim3 grid((unsigned)cdiv((int64_t)nb * 4, WR * SB), (unsigned)cdiv(m, 16 * TG)),
      block(64 * WR * WK);
  const int vec_out = n % 4 == 0 && (uintptr_t)y % (bf16 ? 8 : 16) == 0 &&
                      (acc_out == nullptr || (uintptr_t)acc_out % 16 == 0);
  gemv_mfma_win_kernel<WR, WK, SB, TG, PF><<<grid, block, 0, stream>>>(
      xq, scale, reinterpret_cast<const uint4*>(packed), gamma, (int)m, (int)n, nb, nc,
      padded_k(k), relu2, bf16, vec_out, y, acc_out);
  return hipGetLastError();
}

}  // namespace

// Windowed MFMA GEMV variants (waves per row group x slices x sub-blocks,
// token groups, super-chunks in flight):
//   0: 2 x 4 x 1, 1 group, 2     1: 1 x 8 x 1, 1 group, 2    2: 4 x 1 x 2, 1 group, 4
//   3: 2 x 4 x 1, 2 groups, 2    4: 8 x 1 x 1, 2 groups, 4
//   5: 4 x 2 x 1, 4 groups, 2    6: 8 x 1 x 1, 4 groups, 2    7: 2 x 4 x 1, 4 groups, 2
hipError_t launch_gemv_mfma(int variant, const int8_t* xq, const float* scale,
                            const uint32_t* packed, const float* gamma, int64_t m, int64_t n,
                            int64_t k, bool relu2, bool bf16, void* y, int32_t* acc_out,
                            hipStream_t stream) {
#define BL_WIN(WR, WK, SB, TG, PF)                                                       \
  return run_gemv_mfma_win<WR, WK, SB, TG, PF>(xq, scale, packed, gamma, m, n, k, relu2, bf16, \
                                               y, acc_out, stream)
  switch (variant) {
    case 0: BL_WIN(2, 4, 1, 1, 2);
    case 1: BL_WIN(1, 8, 1, 1, 2);
    case 2: BL_WIN(4, 1, 2, 1, 4);
    case 3: BL_WIN(2, 4, 1, 2, 2);
    case 4: BL_WIN(8, 1, 1, 2, 4);
    case 5: BL_WIN(4, 2, 1, 4, 2);
    case 6: BL_WIN(8, 1, 1, 4, 2);
    case 7: BL_WIN(2, 4, 1, 4, 2);
    default: return hipErrorInvalidValue;
  }
#undef BL_WIN
}

}  // namespace bl
