// Ternary x int8 GEMM on int8 MFMA (v_mfma_i32_16x16x64_i8) with the fused
// dequant, for M > 4 tokens (prefill and batched decode).
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T (integer), then
// y = acc * gamma / s.  With many tokens the product is a dense contraction,
// so it runs on the matrix cores: the 2-bit codes are expanded to int8
// (64 * W~) in registers right before each MFMA.
//
// Tile: BM x BN outputs per workgroup, waves in a WM x WN grid, each wave
// FM x FN fragments of 16x16.  Per 256-input super-chunk the workgroup stages
//   A: x~ rows m0..m0+BM-1, 256 bytes each, into LDS; the 16-byte unit u of
//      row r is stored at unit u ^ (r % 16) so that the 16 lanes reading one
//      MFMA operand column hit 16 different bank groups;
//   B: BN/64 packed 4 KiB blocks, copied as they are.
// MFMA operands: lane l = r + 16 g (r = l % 16, g = l / 16) supplies, for
// k-step j of the super-chunk, the 16 inputs 64 j + 16 g + (0..15): A from x~
// row r of the fragment, B from packed word (q = g, j) of row r, unpacked to
// four dwords.  Byte e of operand dword i is input 4 i + e on both sides, so
// the lane-to-k assignment agrees between A and B, which is all the sum needs.
// The 16x16 int32 result holds row 4 g + i, column r in element i of lane l.
//
// Two LDS stages: global loads of super-chunk c+1 are issued before the
// MFMAs of c and stored to the other stage afterwards (one barrier each).
// Split-K over super-chunks combines each element through a 64-bit
// workspace slot with one device-scope atomic, as in the GEMV.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

template <int FM, int FN, int WM, int WN>
struct Tile {
  static constexpr int BM = 16 * FM * WM;
  static constexpr int BN = 16 * FN * WN;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BNB = BN / 64;              // packed blocks per tile
  static constexpr int UA = BM * 16 / NT;          // 16-byte A units per thread
  static constexpr int UB = BNB * kBlockU4 / NT;   // 16-byte B units per thread
  static constexpr int A_BYTES = BM * 256;         // one LDS stage of A
  static constexpr int B_BYTES = BNB * 4096;       // one LDS stage of B
  static constexpr int LDS = 2 * (A_BYTES + B_BYTES) + BM * 4;
  static_assert(BN % 64 == 0, "tile width must hold whole packed blocks");
  static_assert(BM * 16 % NT == 0 && BNB * kBlockU4 % NT == 0, "staging split");
};

template <int FM, int FN, int WM, int WN, bool SPLIT>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ scale,
    const uint4* __restrict__ packed, const float* __restrict__ gamma, int m, int n,
    int nb, int nc, int64_t kpad, int splits, int tiles_n, int relu2, int bf16,
    void* __restrict__ y, int32_t* __restrict__ acc_out, int64_t* __restrict__ ws_slots) {
  using T = Tile<FM, FN, WM, WN>;
  constexpr int BM = T::BM, BN = T::BN, NT = T::NT, UA = T::UA, UB = T::UB;
  // two LDS stages of A and B, then the per-row rescale factors
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* const As0 = lds;
  uint8_t* const Bs0 = lds + 2 * T::A_BYTES;
  float* const fac = reinterpret_cast<float*>(lds + 2 * (T::A_BYTES + T::B_BYTES));
  __shared__ uint32_t flag;

  const int tile = blockIdx.x / splits;
  const int s = blockIdx.x - tile * splits;
  const int tm = tile / tiles_n;
  const int tn = tile - tm * tiles_n;
  const int m0 = tm * BM;
  const int b0 = tn * T::BNB;
  const int c0 = (int)((int64_t)s * nc / splits);
  const int c1 = (int)((int64_t)(s + 1) * nc / splits);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave / WN;
  const int wn = wave - wm * WN;
  const int r = lane & 15;
  const int g = lane >> 4;

  uint4 ra[UA], rb[UB];
  auto load_tile = [&](int c) {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int p = tid + NT * u;
      const int row = p >> 4, unit = p & 15;
      const int gm = m0 + row;
      ra[u] = gm < m ? *reinterpret_cast<const uint4*>(xq + (int64_t)gm * kpad +
                                                       (int64_t)c * 256 + unit * 16)
                     : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int p = tid + NT * u;
      const int bb = p >> 8, within = p & 255;
      const int blk = b0 + bb;
      rb[u] = blk < nb ? packed[((int64_t)blk * nc + c) * kBlockU4 + within]
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int stage) {
    uint8_t* As = As0 + stage * T::A_BYTES;
    uint8_t* Bs = Bs0 + stage * T::B_BYTES;
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int p = tid + NT * u;
      const int row = p >> 4, unit = p & 15;
      *reinterpret_cast<uint4*>(As + row * 256 + ((unit ^ (row & 15)) << 4)) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int p = tid + NT * u;
      *reinterpret_cast<uint4*>(Bs + (p >> 8) * 4096 + (p & 255) * 16) = rb[u];
    }
  };

  bl_v4i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = bl_v4i{0, 0, 0, 0};

  // Two LDS stages: while the MFMAs read stage cur, the next super-chunk's
  // global loads are in flight in registers and land in the other stage;
  // one barrier per super-chunk.
  if (c0 < c1) {
    load_tile(c0);
    store_tile(0);
  }
  __syncthreads();
  for (int c = c0; c < c1; ++c) {
    const int cur = (c - c0) & 1;
    if (c + 1 < c1) load_tile(c + 1);
    const uint8_t* As = As0 + cur * T::A_BYTES;
    const uint8_t* Bs = Bs0 + cur * T::B_BYTES;

    uint4 bw[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = wn * 16 * FN + 16 * fn + r;
      bw[fn] = *reinterpret_cast<const uint4*>(Bs + (col >> 6) * 4096 + g * 1024 + (col & 63) * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bl_v4i a[FM];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int row = wm * 16 * FM + 16 * fm + r;
        a[fm] = *reinterpret_cast<const bl_v4i*>(As + row * 256 + (((4 * j + g) ^ r) << 4));
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint32_t wj = j == 0 ? bw[fn].x : j == 1 ? bw[fn].y : j == 2 ? bw[fn].z : bw[fn].w;
        const bl_v4i bop = {(int)unpack_x64(wj, 0), (int)unpack_x64(wj, 1),
                            (int)unpack_x64(wj, 2), (int)unpack_x64(wj, 3)};
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[fm], bop, acc[fm][fn], 0, 0, 0);
      }
    }
    if (c + 1 < c1) store_tile(cur ^ 1);
    __syncthreads();
  }

  if constexpr (SPLIT) {
    // Split-K: each element goes through its 64-bit workspace slot
    // (split_add, split_finish), a batch of fragment rows at a time with all
    // adds of a batch issued before any result is used.  Elements another
    // group completes are set to 1, which no total equals (totals are
    // multiples of 64), and skipped below.
    constexpr int BF = FN * 4 >= 32 ? 1 : 32 / (FN * 4);   // fragment rows per batch
    int64_t* slot = ws_slots + (int64_t)tile * (BM * BN) + tid;
#pragma unroll
    for (int f0 = 0; f0 < FM; f0 += BF) {
      int64_t old[BF][FN][4];
#pragma unroll
      for (int fm = f0; fm < f0 + BF && fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            old[fm - f0][fn][i] = split_add(slot + ((fm * FN + fn) * 4 + i) * NT, acc[fm][fn][i]);
#pragma unroll
      for (int fm = f0; fm < f0 + BF && fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[fm][fn][i] = split_finish(slot + ((fm * FN + fn) * 4 + i) * NT,
                                          old[fm - f0][fn][i], acc[fm][fn][i], splits);
    }
  }

  const float gam = *gamma;
  for (int t = tid; t < BM; t += NT) {
    const int gm = m0 + t;
    fac[t] = gm < m ? gamma_over_s(gam, scale[gm]) : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 16 * FM + 16 * fm + 4 * g + i;
      const int gm = m0 + row;
      if (gm >= m) continue;
      const float f = fac[row];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int gn = b0 * 64 + wn * 16 * FN + 16 * fn + r;
        if (gn >= n || (acc[fm][fn][i] & 63) != 0) continue;
        const int a = acc[fm][fn][i] >> 6;
        const int64_t idx = (int64_t)gm * n + gn;
        if (acc_out != nullptr) acc_out[idx] = a;
        store_out(y, idx, a, f, relu2 != 0, bf16 != 0);
      }
    }
  }
}

template <int FM, int FN, int WM, int WN>
hipError_t run(const int8_t* xq, const float* scale, const uint32_t* packed, const float* gamma,
               int64_t m, int64_t n, int64_t k, int splits, bool relu2, bool bf16, void* y,
               int32_t* acc_out, int64_t* slots, hipStream_t stream) {
  using T = Tile<FM, FN, WM, WN>;
  static bool lds_ready = false;          // allow more than 64 KiB of dynamic LDS once
  if (!lds_ready) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_kernel<FM, FN, WM, WN, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<FM, FN, WM, WN, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
    if (e != hipSuccess) return e;
    lds_ready = true;
  }
  const int nb = (int)cdiv(n, kRowBlock);
  const int nc = (int)cdiv(k, kSuperK);
  const int tiles_m = (int)cdiv(m, T::BM);
  const int tiles_n = (int)cdiv(padded_n(n), T::BN);
  const int64_t grid = (int64_t)tiles_m * tiles_n * splits;
  auto kern = splits > 1 ? gemm_kernel<FM, FN, WM, WN, true> : gemm_kernel<FM, FN, WM, WN, false>;
  kern<<<(unsigned)grid, T::NT, T::LDS, stream>>>(
      xq, scale, reinterpret_cast<const uint4*>(packed), gamma, (int)m, (int)n, nb, nc,
      padded_k(k), splits, tiles_n, relu2, bf16, y, acc_out, slots);
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// 32x32x32 variant (v_mfma_i32_32x32x32_i8) for larger M.  Lane l = c + 32 p
// (c = l % 32, p = l / 32).  A super-chunk is 8 MFMA k-steps (j, h), j = 0..3,
// h = 0..1; in step (j, h) lane half p covers the 16 inputs 64 j + 16 (2h+p)
// + (0..15): A from 16-byte unit 4 j + 2 h + p of x~ row c of the fragment, B
// from packed word (q = 2h + p, j) of output row c.  Result element e of lane
// l is D[8 (e/4) + 4 p + e % 4][c].  A wave covers 32*FM rows, so each
// unpacked weight word feeds FM MFMAs.
//
// Tiles travel from global memory straight into LDS (global_load_lds_dwordx4:
// lane i of a wave instruction lands at the wave's LDS base + 16 i), so no
// registers hold data in flight.  Two LDS stages are separate arrays and the
// loop is unrolled by two, so the compiler sees that the copies into one stage
// do not touch the stage being read and only waits for them at the barrier.
// A unit u of tile row r sits at unit u ^ (r % 16): each lane fetches the
// global unit that belongs in its slot.
// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_wave_base + 16 i (global_load_lds_dwordx4).
__device__ __forceinline__ void lds_copy16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

// One super-chunk of A and B copied global -> LDS (wave instruction u of a
// tile fills 1 KiB at slot u * NT + 64 * wave).
template <int UA, int UB, int NT>
__device__ __forceinline__ void copy_tiles(const int8_t* const (&a_src)[UA],
                                           const uint4* const (&b_src)[UB], uint8_t* As,
                                           uint8_t* Bs, int cc, int wave) {
#pragma unroll
  for (int u = 0; u < UA; ++u)
    lds_copy16(a_src[u] + (int64_t)cc * 256, As + (u * NT + wave * 64) * 16);
#pragma unroll
  for (int u = 0; u < UB; ++u)
    lds_copy16(b_src[u] + (int64_t)cc * kBlockU4, Bs + (u * NT + wave * 64) * 16);
}

template <int FM, int FN, int WM, int WN>
struct Tile32 {
  static constexpr int BM = 32 * FM * WM;
  static constexpr int BN = 32 * FN * WN;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BNB = BN / 64;
  static constexpr int UA = BM * 16 / NT;          // A copy instructions per thread
  static constexpr int UB = BNB * kBlockU4 / NT;   // B copy instructions per thread
  static constexpr int A_BYTES = BM * 256;
  static constexpr int B_BYTES = BNB * 4096;
  static_assert(BN % 64 == 0, "tile width must hold whole packed blocks");
  static_assert(BM * 16 % NT == 0 && BNB * kBlockU4 % NT == 0, "copy split");
};

template <int FM, int FN, int WM, int WN, bool SPLIT>
__global__ __launch_bounds__(64 * WM * WN) void gemm32_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ scale,
    const uint4* __restrict__ packed, const float* __restrict__ gamma, int m, int n,
    int nb, int nc, int64_t kpad, int splits, int tiles_n, int relu2, int bf16,
    void* __restrict__ y, int32_t* __restrict__ acc_out, int64_t* __restrict__ ws_slots) {
  using T = Tile32<FM, FN, WM, WN>;
  constexpr int BM = T::BM, BN = T::BN, NT = T::NT, UA = T::UA, UB = T::UB;
  __shared__ __attribute__((aligned(16))) uint8_t A0[T::A_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t A1[T::A_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t B0[T::B_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t B1[T::B_BYTES];
  __shared__ uint32_t flag;

  const int tile = blockIdx.x / splits;
  const int s = blockIdx.x - tile * splits;
  const int tm = tile / tiles_n;
  const int tn = tile - tm * tiles_n;
  const int m0 = tm * BM;
  const int b0 = tn * T::BNB;
  const int c0 = (int)((int64_t)s * nc / splits);
  const int c1 = (int)((int64_t)(s + 1) * nc / splits);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave / WN;
  const int wn = wave - wm * WN;
  const int c = lane & 31;
  const int ph = lane >> 5;

  // Per-thread source addresses of the copies (super-chunk 0); rows past m
  // and blocks past nb read clamped, valid memory whose results are dropped.
  const int8_t* a_src[UA];
#pragma unroll
  for (int u = 0; u < UA; ++u) {
    const int p = u * NT + tid;                  // LDS slot (16 bytes) this lane fills
    const int row = p >> 4, slot = p & 15;
    const int gm = min(m0 + row, m - 1);
    a_src[u] = xq + (int64_t)gm * kpad + ((slot ^ (row & 15)) << 4);
  }
  const uint4* b_src[UB];
#pragma unroll
  for (int u = 0; u < UB; ++u) {
    const int p = u * NT + tid;
    const int blk = min(b0 + (p >> 8), nb - 1);
    b_src[u] = packed + (int64_t)blk * nc * kBlockU4 + (p & 255);
  }

  bl_v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = bl_v16i{};

  // per-lane LDS offsets: A fragment rows and the swizzled unit of each k-step
  const int a_row = (wm * 32 * FM + c) * 256;
  int a_unit[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) a_unit[st] = ((4 * (st >> 1) + 2 * (st & 1) + ph) ^ (c & 15)) << 4;
  const int bcol = wn * 32 * FN + c;
  const int b_off = (bcol >> 6) * 4096 + ph * 1024 + (bcol & 63) * 16;

  auto compute = [&](const uint8_t* As, const uint8_t* Bs) {
    uint4 bw[FN][2];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int d = ((32 * fn) >> 6) * 4096 + ((32 * fn) & 63) * 16;
      bw[fn][0] = *reinterpret_cast<const uint4*>(Bs + b_off + d);
      bw[fn][1] = *reinterpret_cast<const uint4*>(Bs + b_off + d + 2048);
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) {              // k-step (j, h) = (st / 2, st % 2)
      const int j = st >> 1, h = st & 1;
      bl_v4i a[FM];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        a[fm] = *reinterpret_cast<const bl_v4i*>(As + a_row + fm * 32 * 256 + a_unit[st]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint4 wv = bw[fn][h];
        const uint32_t wj = j == 0 ? wv.x : j == 1 ? wv.y : j == 2 ? wv.z : wv.w;
        const bl_v4i bop = {(int)unpack_x64(wj, 0), (int)unpack_x64(wj, 1),
                            (int)unpack_x64(wj, 2), (int)unpack_x64(wj, 3)};
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[fm], bop, acc[fm][fn], 0, 0, 0);
      }
    }
  };

  if (c0 < c1) copy_tiles<UA, UB, NT>(a_src, b_src, A0, B0, c0, wave);
  __syncthreads();
  for (int cc = c0; cc < c1; cc += 2) {
    if (cc + 1 < c1) copy_tiles<UA, UB, NT>(a_src, b_src, A1, B1, cc + 1, wave);
    compute(A0, B0);
    __syncthreads();
    if (cc + 1 >= c1) break;
    if (cc + 2 < c1) copy_tiles<UA, UB, NT>(a_src, b_src, A0, B0, cc + 2, wave);
    compute(A1, B1);
    __syncthreads();
  }

  if constexpr (SPLIT) {
    // Split-K through 64-bit workspace slots, as in gemm_kernel, one
    // fragment row (FN * 16 elements) per batch.
    int64_t* slot = ws_slots + (int64_t)tile * (BM * BN) + tid;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      int64_t old[FN][16];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          old[fn][e] = split_add(slot + ((fm * FN + fn) * 16 + e) * NT, acc[fm][fn][e]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          acc[fm][fn][e] = split_finish(slot + ((fm * FN + fn) * 16 + e) * NT, old[fn][e],
                                        acc[fm][fn][e], splits);
    }
  }

  // rescale factors per tile row (in the now idle first A stage)
  float* fac = reinterpret_cast<float*>(A0);
  const float gam = *gamma;
  for (int t = tid; t < BM; t += NT) {
    const int gm = m0 + t;
    fac[t] = gm < m ? gamma_over_s(gam, scale[gm]) : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = wm * 32 * FM + 32 * fm + 8 * (e >> 2) + 4 * ph + (e & 3);
      const int gm = m0 + row;
      if (gm >= m) continue;
      const float f = fac[row];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int gn = b0 * 64 + wn * 32 * FN + 32 * fn + c;
        if (gn >= n || (acc[fm][fn][e] & 63) != 0) continue;
        const int a = acc[fm][fn][e] >> 6;
        const int64_t idx = (int64_t)gm * n + gn;
        if (acc_out != nullptr) acc_out[idx] = a;
        store_out(y, idx, a, f, relu2 != 0, bf16 != 0);
      }
    }
  }
}

template <int FM, int FN, int WM, int WN>
hipError_t run32(const int8_t* xq, const float* scale, const uint32_t* packed, const float* gamma,
                 int64_t m, int64_t n, int64_t k, int splits, bool relu2, bool bf16, void* y,
                 int32_t* acc_out, int64_t* slots, hipStream_t stream) {
  using T = Tile32<FM, FN, WM, WN>;
  const int nb = (int)cdiv(n, kRowBlock);
  const int nc = (int)cdiv(k, kSuperK);
  const int tiles_m = (int)cdiv(m, T::BM);
  const int tiles_n = (int)cdiv(padded_n(n), T::BN);
  const int64_t grid = (int64_t)tiles_m * tiles_n * splits;
  auto kern =
      splits > 1 ? gemm32_kernel<FM, FN, WM, WN, true> : gemm32_kernel<FM, FN, WM, WN, false>;
  kern<<<(unsigned)grid, T::NT, 0, stream>>>(
      xq, scale, reinterpret_cast<const uint4*>(packed), gamma, (int)m, (int)n, nb, nc,
      padded_k(k), splits, tiles_n, relu2, bf16, y, acc_out, slots);
  return hipGetLastError();
}

}  // namespace

// Tile variants: rows per tile x columns per tile.
//   0: 16 x 256   1: 32 x 256   2: 64 x 256   3: 64 x 128   (16x16x64 MFMA)
//   4: 128 x 256  (32x32x32 MFMA, tiles copied to LDS by DMA)
void gemm_tile_shape(int variant, int* bm, int* bn) {
  switch (variant) {
    case 0: *bm = Tile<1, 4, 1, 4>::BM; *bn = Tile<1, 4, 1, 4>::BN; break;
    case 1: *bm = Tile<2, 4, 1, 4>::BM; *bn = Tile<2, 4, 1, 4>::BN; break;
    case 2: *bm = Tile<4, 4, 1, 4>::BM; *bn = Tile<4, 4, 1, 4>::BN; break;
    case 3: *bm = Tile<2, 4, 2, 2>::BM; *bn = Tile<2, 4, 2, 2>::BN; break;
    default: *bm = Tile32<2, 2, 2, 4>::BM; *bn = Tile32<2, 2, 2, 4>::BN; break;
  }
}

hipError_t launch_gemm(int variant, const int8_t* xq, const float* scale, const uint32_t* packed,
                       const float* gamma, int64_t m, int64_t n, int64_t k, int splits,
                       bool relu2, bool bf16, void* y, int32_t* acc_out, int64_t* slots,
                       hipStream_t stream) {
  switch (variant) {
    case 0: return run<1, 4, 1, 4>(xq, scale, packed, gamma, m, n, k, splits, relu2, bf16, y, acc_out, slots, stream);
    case 1: return run<2, 4, 1, 4>(xq, scale, packed, gamma, m, n, k, splits, relu2, bf16, y, acc_out, slots, stream);
    case 2: return run<4, 4, 1, 4>(xq, scale, packed, gamma, m, n, k, splits, relu2, bf16, y, acc_out, slots, stream);
    case 3: return run<2, 4, 2, 2>(xq, scale, packed, gamma, m, n, k, splits, relu2, bf16, y, acc_out, slots, stream);
    default: return run32<2, 2, 2, 4>(xq, scale, packed, gamma, m, n, k, splits, relu2, bf16, y, acc_out, slots, stream);
  }
}

}  // namespace bl
