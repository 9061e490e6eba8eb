// Ternary x int8 GEMM on int8 MFMA with the fused dequant, for more than 64
// tokens (prefill): gemmw_kernel on v_mfma_i32_32x32x32_i8 with wide waves.
//
// "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs", section "Matrix
// Multiplication as Pure Integer Addition": acc = x~ W~^T (integer), then
// y = acc * gamma / s.  With many tokens the product is a dense contraction,
// so it runs on the matrix cores: the 2-bit codes are expanded to int8
// (64 * W~) in registers right before each MFMA.  Outputs too small to give
// the chip enough tiles go to the windowed MFMA GEMV in token blocks instead,
// so K is never split here.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_wave_base + 16 i (global_load_lds_dwordx4).  A non-template
// wrapper: the builtin is not accepted inside templates by the host pass.
__device__ __forceinline__ void lds_copy16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

// ------------------------------------------------------------------------
// Waves sit side by side along N (one row of WN waves); each wave owns one
// 64-row packed block (two 32-column fragments) and 32*FM tile rows, so
// every unpacked weight word feeds FM MFMAs and no block is unpacked by two
// waves.  x~, which all waves share, goes global -> LDS by DMA in two
// stages of KS super-chunks each: the copies of the next stage are in
// flight while the current one is computed.  The packed words are private
// to their wave, so they skip LDS: each lane loads its 64 bytes of a
// super-chunk as four 16-byte loads straight into registers, those of the
// next super-chunk early in the current one (no LDS traffic for the
// weights, and the barrier only publishes x~).
//
// v_mfma_i32_32x32x32_i8 lanes: lane l = c + 32 ph (c = l % 32, ph = l / 32)
// supplies row/column c of its operand for 16 inputs; a super-chunk is 8
// k-steps (j, h), j = 0..3, h = 0..1, and in step (j, h) lane half ph covers
// inputs 64 j + 16 (2h+ph) + (0..15): the weights from packed word (q = 2h +
// ph, j) of output row c of the fragment, x~ from 16-byte unit 4 j + 2 h + ph
// of tile row c (an x~ unit u of tile row r sits at unit u ^ (r % 16) in LDS,
// so the lanes of one read hit different banks).  Byte e of operand dword i
// is input 4 i + e on both sides.  The weights are the MFMA's first operand,
// so the result is the transposed tile: element e of lane l holds tile row
// 32fm + c and column 32fn + 8(e/4) + 4ph + e%4, four consecutive columns
// per group of four elements, stored as one vector.
//
// Tile order: with `band` > 0, tiles are numbered band by band (band tile
// rows each, column-major inside a band) and consecutive numbers go to the
// same XCD (workgroups are dispatched to the 8 XCDs round-robin), so the
// workgroups that share an XCD's L2 cover a compact block of the output and
// share its x~ rows and packed columns.  With several products (q, k, v
// sharing x~) their column tiles sit side by side in one grid.

// One product of the table in the kernel arguments; the first column tile
// of every product shares one 64-byte line (tn_begin), so a workgroup finds
// its product with one scalar load.
struct GemmSegK {
  const uint4* packed;
  const float* gamma;
  void* y;
  int32_t* acc_out;
  int n, nb, flags;        // flags: 1 ReLU^2, 2 bf16 y, 4 vector stores, 8 whole-line bf16 rows
};
struct GemmArgs {
  int tn_begin[kMaxMulti];
  const int8_t* xq;
  const float* scale;
  int64_t kpad;
  int m, nc, tiles_m, tiles_n, band, nseg;
  GemmSegK seg[kMaxMulti];
};

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt = 0 only:
// vmcnt[3:0] = 0, expcnt[6:4] = 7, lgkmcnt[11:8] = 15, vmcnt[15:14] = 0.
constexpr int kWaitVmcnt0 = 0x0F70;

template <int FM, int WN, int KS>
struct TileW {
  static constexpr int BM = 32 * FM;
  static constexpr int BN = 64 * WN;
  static constexpr int NT = 64 * WN;
  static constexpr int UA = BM * 16 / NT;          // A copy instructions per thread and chunk
  static constexpr int A_CHUNK = BM * 256;         // x~ bytes per super-chunk
  static constexpr int A_BYTES = KS * A_CHUNK;     // one stage
  static_assert(BM * 16 % NT == 0, "copy split");
  static_assert(2 * A_BYTES <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int tile_of_block(int bid, int tiles, int tiles_m, int tiles_n,
                                             int band) {
  if (band <= 0) return bid;
  // round-robin XCD x = bid % 8 receives the contiguous range of the
  // banded order starting at x * (tiles / 8) + min(x, tiles % 8)
  const int x = bid & 7, li = bid >> 3;
  const int q = tiles >> 3, r = tiles & 7;
  const int lin = x * q + min(x, r) + li;
  const int per_band = band * tiles_n;
  const int b = lin / per_band, w = lin - b * per_band;
  const int rows = min(band, tiles_m - b * band);  // tile rows in this band
  const int tn = w / rows, tm = b * band + (w - tn * rows);
  return tm * tiles_n + tn;
}

// At least two waves per SIMD (registers within 256 per lane): one wave's
// waits are covered by the other's MFMAs.  MULTI: the table may hold
// several products (a scalar lookup finds this workgroup's); otherwise it
// is product 0 at fixed offsets, so its fields load together with the
// other arguments.
template <int FM, int WN, int KS, bool MULTI>
__global__ __launch_bounds__(64 * WN) __attribute__((amdgpu_waves_per_eu(2))) void gemmw_kernel(
    GemmArgs args) {
  using T = TileW<FM, WN, KS>;
  constexpr int BM = T::BM, BN = T::BN, NT = T::NT, UA = T::UA;
  // two stages as separate arrays: the compiler then sees that the copies
  // into one stage do not touch the other and does not wait for them before
  // the LDS reads of the stage being computed
  __shared__ __attribute__((aligned(16))) uint8_t A0[T::A_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t A1[T::A_BYTES];

  // this workgroup's tile over all products' column tiles, then its product
  const int tiles_m = args.tiles_m;
  const int tiles = tiles_m * args.tiles_n;
  const int tile = tile_of_block((int)blockIdx.x, tiles, tiles_m, args.tiles_n, args.band);
  const int tm = tile / args.tiles_n;
  const int tng = tile - tm * args.tiles_n;
  int si = 0;
  if (MULTI) {
#pragma unroll
    for (int i = 1; i < kMaxMulti; ++i)
      if (i < args.nseg && tng >= args.tn_begin[i]) si = i;
  }
  const GemmSegK& sg = args.seg[si];
  const int tn = tng - args.tn_begin[si];
  const int8_t* __restrict__ xq = args.xq;
  const float* __restrict__ scale = args.scale;
  const uint4* __restrict__ packed = sg.packed;
  const float* __restrict__ gamma = sg.gamma;
  void* __restrict__ y = sg.y;
  int32_t* __restrict__ acc_out = sg.acc_out;
  const int m = args.m, n = sg.n, nb = sg.nb, nc = args.nc;
  const int64_t kpad = args.kpad;
  const int relu2 = sg.flags & 1, bf16 = (sg.flags >> 1) & 1, vec_out = (sg.flags >> 2) & 1,
            line_out = (sg.flags >> 3) & 1;
  const int m0 = tm * BM;
  const int c0 = 0, c1 = nc;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane & 31;
  const int ph = lane >> 5;
  const int blk = min(tn * WN + wave, nb - 1);      // this wave's packed block (clamped)

  // x~ copy sources (super-chunk 0); rows past m read row m-1 (dropped)
  const int8_t* a_src[UA];
#pragma unroll
  for (int u = 0; u < UA; ++u) {
    const int p = u * NT + tid;
    const int row = p >> 4, slot = p & 15;
    const int gm = min(m0 + row, m - 1);
    a_src[u] = xq + (int64_t)gm * kpad + ((slot ^ (row & 15)) << 4);
  }
  // this lane's packed words of super-chunk sc: fragment fn, half h, component j
  // at dword ((blk * nc + sc) * 1024 + (2h + ph) * 256 + (32 fn + c) * 4 + j
  const uint32_t* b_words = reinterpret_cast<const uint32_t*>(packed) +
                            (int64_t)blk * nc * 1024 + ph * 256 + c * 4;
  // one stage: super-chunks cc .. cc+KS-1 (those < c1)
  auto copy_stage = [&](uint8_t* As, int cc) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (cc + k < c1) {
#pragma unroll
        for (int u = 0; u < UA; ++u)
          lds_copy16(a_src[u] + (int64_t)(cc + k) * 256,
                     As + k * T::A_CHUNK + (u * NT + wave * 64) * 16);
      }
    }
  };

  bl_v16i acc[FM][2];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = bl_v16i{};

  int a_unit[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) a_unit[st] = ((4 * (st >> 1) + 2 * (st & 1) + ph) ^ (c & 15)) << 4;
  const int a_row = c * 256;

  // One super-chunk: 8 k-steps (j, h) = (st / 2, st % 2), software
  // pipelined: during step st the A operands of step st+RING-1 are read
  // from LDS and the B operands of step st+1 unpacked, while step st's
  // MFMAs run.  A lane's packed words of a super-chunk are four 16-byte
  // loads bw[fn][h] (component j = step j); those of the next super-chunk
  // are issued right after step 1 is unpacked into a second set, which
  // becomes the current one at the end of the super-chunk.
  auto unpack_b = [&](const uint4 (&bw)[2][2], int st, bl_v4i (&bop)[2]) __attribute__((always_inline)) {
    const int j = st >> 1, h = st & 1;
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
      const uint4 wv = bw[fn][h];
      const uint32_t wj = j == 0 ? wv.x : j == 1 ? wv.y : j == 2 ? wv.z : wv.w;
      bop[fn] = bl_v4i{(int)unpack_x64(wj, 0), (int)unpack_x64(wj, 1), (int)unpack_x64(wj, 2),
                       (int)unpack_x64(wj, 3)};
    }
  };
  auto load_b = [&](uint4 (&bw)[2][2], int sc) __attribute__((always_inline)) {
    const int scc = min(sc, c1 - 1);                 // past the end: reload the last (unused)
    const uint32_t* p = b_words + (int64_t)scc * 1024;
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        bw[fn][h] = *reinterpret_cast<const uint4*>(p + 2 * h * 256 + 32 * fn * 4);
  };
  auto read_a = [&](const uint8_t* As, int st, bl_v4i (&a)[FM]) __attribute__((always_inline)) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      a[fm] = *reinterpret_cast<const bl_v4i*>(As + a_row + fm * 32 * 256 + a_unit[st]);
  };
  constexpr int RING = FM >= 4 ? 2 : 3;             // A reads run RING-1 steps ahead
  uint4 bw[2][2], bwn[2][2];
  auto compute = [&](const uint8_t* As, int sc) __attribute__((always_inline)) {
    bl_v4i a[RING][FM];
    bl_v4i bop[2][2];
#pragma unroll
    for (int r = 0; r + 1 < RING; ++r) read_a(As, r, a[r]);
    unpack_b(bw, 0, bop[0]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + RING - 1 < 8) read_a(As, st + RING - 1, a[(st + RING - 1) % RING]);
      if (st + 1 < 8) unpack_b(bw, st + 1, bop[(st + 1) & 1]);
      if (st == 0) load_b(bwn, sc + 1);
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bop[st & 1][fn], a[st % RING][fm],
                                                             acc[fm][fn], 0, 0, 0);
      if (st + 1 < 8) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, FM, 0);     // DS read
#pragma unroll
        for (int i = 1; i < 2 * FM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);    // VALU
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int h = 0; h < 2; ++h) bw[fn][h] = bwn[fn][h];
  };
  auto compute_stage = [&](const uint8_t* As, int cc) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KS; ++k)
      if (cc + k < c1) compute(As + k * T::A_CHUNK, cc + k);
  };

  // The compiler counts a global -> LDS copy as a flat access (global and
  // LDS) and, while one is in flight, waits for every outstanding vector
  // memory operation before any use of a loaded register.  The packed words
  // a stage starts on were loaded a whole super-chunk earlier, so wait for
  // them before the stage's copies are issued: then nothing the stage
  // computes on is still in flight behind the copies, and they stay in
  // flight until the weights of the next super-chunk are needed.
  auto copy_stage_after_b = [&](uint8_t* As, int cc) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    copy_stage(As, cc);
  };

  // Pairs of stages, then an odd last one.
  load_b(bw, c0);
  if (c0 < c1) copy_stage(A0, c0);
  __syncthreads();
  int cc = c0;
  for (; cc + 2 * KS <= c1; cc += 2 * KS) {
    copy_stage_after_b(A1, cc + KS);
    compute_stage(A0, cc);
    __syncthreads();
    if (cc + 2 * KS < c1) copy_stage_after_b(A0, cc + 2 * KS);
    compute_stage(A1, cc + KS);
    __syncthreads();
  }
  if (cc < c1) {
    if (cc + KS < c1) copy_stage_after_b(A1, cc + KS);
    compute_stage(A0, cc);
    __syncthreads();
    if (cc + KS < c1) compute_stage(A1, cc + KS);
  }

  // rescale factors per tile row (in the now idle first A stage)
  float* fac = reinterpret_cast<float*>(A0);
  const float gam = *gamma;
  for (int t = tid; t < BM; t += NT) {
    const int gm = m0 + t;
    fac[t] = gm < m ? gamma_over_s(gam, scale[gm]) : 0.0f;
  }
  __syncthreads();
  // bf16 output in whole lines: a wave's 32*FM x 64 block is one 128-byte
  // line per row.  The scaled values go to LDS (row-major, 16-byte chunk q of
  // row r at q ^ (r % 8), so neither side conflicts on banks) and come back
  // as 16-byte pieces, eight lanes per line: every store instruction writes
  // eight whole lines, which the memory system takes far better than the
  // accumulator layout's 16-byte pieces of 32 rows.  Tall tiles (one round
  // of tiles that all end together) store non-temporally, which measured
  // faster there; the 64-row tiles run in several rounds and keep ordinary
  // stores, which measured faster for them.
  if (line_out) {                                        // uniform
    float fr[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) fr[fm] = fac[32 * fm + c];
    __syncthreads();                                     // all fac reads done
    constexpr int S = 32 * FM * 128;                     // LDS bytes per wave
    constexpr int NA = T::A_BYTES / S;
    static_assert(2 * NA >= WN, "line staging space");
    uint8_t* buf = wave < NA ? A0 + wave * S : A1 + (wave - NA) * S;
    const int col0 = (tn * WN + wave) * 64;
    if (col0 + 64 <= n) {                                // whole block inside the output
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = 32 * fm + c;
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            int v[4];
            float o[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              v[t] = acc[fm][fn][4 * g + t] >> 6;
              o[t] = (float)v[t] * fr[fm];
              if (relu2) o[t] = o[t] > 0.0f ? o[t] * o[t] : 0.0f;
            }
            if (acc_out != nullptr && m0 + r < m)
              *reinterpret_cast<int4*>(acc_out + (int64_t)(m0 + r) * n + col0 + 32 * fn + 8 * g + 4 * ph) =
                  make_int4(v[0], v[1], v[2], v[3]);
            const int q = 4 * fn + g;
            *reinterpret_cast<uint2*>(buf + r * 128 + ((q ^ (r & 7)) << 4) + ph * 8) =
                make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          }
      }
      // the wave reads back only its own block: LDS operations of one wave
      // complete in order, and the barrier keeps the compiler from moving
      // the reads above the writes
      __builtin_amdgcn_wave_barrier();
      const int q = lane & 7;
#pragma unroll
      for (int i = 0; i < 4 * FM; ++i) {
        const int r = 8 * i + (lane >> 3);
        const bl_v4i v = *reinterpret_cast<const bl_v4i*>(buf + r * 128 + ((q ^ (r & 7)) << 4));
        if (m0 + r < m) {
          bl_v4i* dst = reinterpret_cast<bl_v4i*>(reinterpret_cast<uint16_t*>(y) +
                                                 (int64_t)(m0 + r) * n + col0 + 8 * q);
          if (FM >= 3)
            __builtin_nontemporal_store(v, dst);
          else
            *dst = v;
        }
      }
    } else {                                             // the column tail
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int gm = m0 + 32 * fm + c;
        if (gm >= m) continue;
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int gn = col0 + 32 * fn + 8 * g + 4 * ph;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              if (gn + t >= n) continue;
              const int a = acc[fm][fn][4 * g + t] >> 6;
              if (acc_out != nullptr) acc_out[(int64_t)gm * n + gn + t] = a;
              store_out(y, (int64_t)gm * n + gn + t, a, fr[fm], relu2 != 0, true);
            }
          }
      }
    }
    return;
  }
  // Each group of four accumulator elements is four consecutive columns of
  // one row: whole groups go out as one 16-byte (fp32, int32) or 8-byte
  // (bf16) store when vec_out (n % 4 == 0 and aligned outputs); the column
  // tail and unaligned outputs go element by element.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int gm = m0 + 32 * fm + c;
    if (gm >= m) continue;
    const float f = fac[32 * fm + c];
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gn = (tn * WN + wave) * 64 + 32 * fn + 8 * g + 4 * ph;
        const int64_t idx = (int64_t)gm * n + gn;
        int v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = acc[fm][fn][4 * g + t];
        if (vec_out && gn + 3 < n) {
          float o[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            o[t] = (float)(v[t] >> 6) * f;
            if (relu2) o[t] = o[t] > 0.0f ? o[t] * o[t] : 0.0f;
          }
          if (acc_out != nullptr)
            *reinterpret_cast<int4*>(acc_out + idx) =
                make_int4(v[0] >> 6, v[1] >> 6, v[2] >> 6, v[3] >> 6);
          if (bf16)
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + idx) =
                make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          else
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + idx) =
                make_float4(o[0], o[1], o[2], o[3]);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (gn + t >= n) continue;
            const int a = v[t] >> 6;
            if (acc_out != nullptr) acc_out[idx + t] = a;
            store_out(y, idx + t, a, f, relu2 != 0, bf16 != 0);
          }
        }
      }
    }
  }
}

template <int FM, int WN, int KS>
hipError_t runw_multi(const int8_t* xq, const float* scale, int64_t m, int64_t k, int band,
                      const GemmProduct* ops, int nops, hipStream_t stream) {
  using T = TileW<FM, WN, KS>;
  if (nops < 1 || nops > kMaxMulti) return hipErrorInvalidValue;
  GemmArgs a{};
  a.xq = xq;
  a.scale = scale;
  a.kpad = padded_k(k);
  a.m = (int)m;
  a.nc = (int)cdiv(k, kSuperK);
  a.tiles_m = (int)cdiv(m, T::BM);
  a.band = band;
  a.nseg = nops;
  int tn = 0;
  for (int i = 0; i < nops; ++i) {
    const GemmProduct& o = ops[i];
    GemmSegK& sg = a.seg[i];
    sg.packed = reinterpret_cast<const uint4*>(o.packed);
    sg.gamma = o.gamma;
    sg.y = o.y;
    sg.acc_out = o.acc_out;
    sg.n = (int)o.n;
    sg.nb = (int)cdiv(o.n, kRowBlock);
    const bool vec_out = o.n % 4 == 0 && (uintptr_t)o.y % (o.bf16 ? 8 : 16) == 0 &&
                         (o.acc_out == nullptr || (uintptr_t)o.acc_out % 16 == 0);
    // whole 16-byte pieces of bf16 rows: n % 8 == 0 and a 16-byte aligned y
    const bool line_out = o.bf16 && vec_out && o.n % 8 == 0 && (uintptr_t)o.y % 16 == 0;
    sg.flags = (o.relu2 ? 1 : 0) | (o.bf16 ? 2 : 0) | (vec_out ? 4 : 0) | (line_out ? 8 : 0);
    a.tn_begin[i] = tn;
    tn += (int)cdiv(padded_n(o.n), T::BN);
  }
  a.tiles_n = tn;
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
  if (nops > 1)
    gemmw_kernel<FM, WN, KS, true><<<(unsigned)grid, T::NT, 0, stream>>>(a);
  else
    gemmw_kernel<FM, WN, KS, false><<<(unsigned)grid, T::NT, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

// Tile variants: rows per tile x columns per tile (32x32x32 MFMA, wide waves),
// super-chunks per stage.  Eight-wave tiles stage two super-chunks (fewer
// barriers, and room in LDS for their whole-line output staging).
//   0: 128 x 512, 2   1: 64 x 512, 2   2: 64 x 256, 1   3: 96 x 256, 1
void gemm_tile_shape(int variant, int* bm, int* bn) {
  switch (variant) {
    case 0: *bm = TileW<4, 8, 2>::BM; *bn = TileW<4, 8, 2>::BN; break;
    case 1: *bm = TileW<2, 8, 2>::BM; *bn = TileW<2, 8, 2>::BN; break;
    case 2: *bm = TileW<2, 4, 1>::BM; *bn = TileW<2, 4, 1>::BN; break;
    default: *bm = TileW<3, 4, 1>::BM; *bn = TileW<3, 4, 1>::BN; break;
  }
}

// band: tile rows per band of the XCD-grouped order.
constexpr int kBand = 4;

hipError_t launch_gemm_multi(int variant, const int8_t* xq, const float* scale, int64_t m,
                             int64_t k, const GemmProduct* ops, int nops, hipStream_t stream) {
#define BL_GEMMW(FM, WN, KS) \
  return runw_multi<FM, WN, KS>(xq, scale, m, k, kBand, ops, nops, stream)
  switch (variant) {
    case 0: BL_GEMMW(4, 8, 2);
    case 1: BL_GEMMW(2, 8, 2);
    case 2: BL_GEMMW(2, 4, 1);
    case 3: BL_GEMMW(3, 4, 1);
    default: return hipErrorInvalidValue;
  }
#undef BL_GEMMW
}

hipError_t launch_gemm(int variant, const int8_t* xq, const float* scale, const uint32_t* packed,
                       const float* gamma, int64_t m, int64_t n, int64_t k, bool relu2,
                       bool bf16, void* y, int32_t* acc_out, hipStream_t stream) {
  const GemmProduct one{packed, gamma, n, relu2, bf16, y, acc_out};
  return launch_gemm_multi(variant, xq, scale, m, k, &one, 1, stream);
}

}  // namespace bl
