// libbitlinear C ABI: argument checks, dispatch and launches.
// The entry points and their contracts are declared in include/bitlinear.h.
#include <math.h>

#include <mutex>

#include "../../include/bitlinear.h"
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

hipError_t launch_gemv(int m, int waves, int pf, int qpl, const int8_t* xq, const float* scale,
                       const uint32_t* packed, const float* gamma, int64_t n, int64_t k,
                       int splits, bool relu2, bool bf16, void* y, int32_t* acc_out,
                       int64_t* ws_slots, hipStream_t stream);
hipError_t launch_gemm(int variant, const int8_t* xq, const float* scale, const uint32_t* packed,
                       const float* gamma, int64_t m, int64_t n, int64_t k, bool relu2,
                       bool bf16, void* y, int32_t* acc_out, hipStream_t stream);
void gemm_tile_shape(int variant, int* bm, int* bn);

namespace {

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, size_t words) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < words; i += stride) p[i] = 0u;
}

constexpr int64_t kGemvMaxM = 2;           // dot4 GEMV up to here
constexpr int64_t kMfmaGemvMaxM = 64;      // windowed MFMA GEMV up to here (4 token groups)
constexpr int64_t kGemvTargetGroups = 256;  // one token: about one workgroup per CU
constexpr int64_t kGemvMaxLds = 48 * 1024;
constexpr int64_t kCUs = 256;
constexpr int64_t kStreamMinSubs = 64;      // stream GEMV from 1024 rows
constexpr size_t kStreamMaxLds = 64 * 1024;
constexpr size_t kMtMaxLds = 160 * 1024;     // a workgroup's LDS on gfx950

}  // namespace

hipError_t launch_fill_zero(uint32_t* p, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_zero_kernel<<<(unsigned)blocks, 256, 0, stream>>>(p, words);
  return hipGetLastError();
}

// Row ranges of the multi-token streaming GEMV: about one workgroup per CU
// over the ceil(m / 16) token blocks, a multiple of 8 when there are several
// blocks (so a row range's blocks share an XCD), at most one per sub-block.
static int64_t mt_row_ranges(int64_t m, int64_t subs) {
  const int64_t tb = cdiv(m, 16);
  int64_t p = kCUs / tb;
  if (p < 1) p = 1;
  if (tb > 1 && p >= 8) p -= p % 8;
  return p < subs ? p : subs;
}

// The multi-token streaming GEMV for long rows (>= 32 super-chunks) of
// matrices with few row blocks: past 32 tokens up to 128 row blocks, past 16
// tokens up to 16, when x~ of a 16-token block and the sums of a row range
// fit a workgroup's LDS.  Elsewhere the windowed MFMA GEMV measured faster:
// the streaming kernel stages all of its block's x~ before the first MFMA,
// which only pays when every row is long and there are few row ranges to
// feed (MI355X, 100B- and 2B-class shapes at 8 to 64 tokens: 100B q at 64
// tokens 14.8 -> 12.9 us, k/v at 32-64 tokens 7.6 -> 6.7 us).
static bool mt_plan(int64_t m, int64_t n, int64_t k, FwdPlan* p) {
  const int64_t nb = cdiv(n, kRowBlock);
  const int64_t subs = nb * 4;
  const int64_t nc = cdiv(k, kSuperK);
  if (nc < 32 || !((m > 32 && nb <= 128) || (m > 16 && nb <= 16))) return false;
  const int64_t P = mt_row_ranges(m, subs);
  if (stream_mt_lds_bytes(m, nc, (int)cdiv(subs, P), 16, 0) > kMtMaxLds) return false;
  p->kind = 4;
  p->qpl = (int)P;
  p->splits = 1;
  p->slots = 0;
  return true;
}

FwdPlan forward_plan(int64_t m, int64_t n, int64_t k) {
  FwdPlan p{};
  const int64_t nb = cdiv(n, kRowBlock);
  const int64_t nc = cdiv(k, kSuperK);
  if (m <= 0) return p;
  if (m <= kGemvMaxM) {
    // Rows up to 40 super-chunks (K <= 10240) of matrices with fewer than
    // 256 row blocks: 16-row groups (a quarter of a packed block each, four
    // lanes per row), no K split, 8 waves when a group has >= 16
    // super-chunks.  Otherwise 64-row groups, split over up to 4 workgroups
    // when the row blocks alone give fewer than about one workgroup per CU
    // at one token (two at two tokens), each keeping >= 2 super-chunks (one
    // atomic combine per output); 4 waves per group when that leaves >= 128
    // workgroups (at two tokens only without a split: the dot4 work doubles
    // and one wave per SIMD no longer hides it), else 8 once a group has
    // >= 6 super-chunks; two super-chunks in flight per wave once a wave
    // streams >= 4.  Each group's x~ slice must fit LDS.  (Tuned on MI355X
    // over the 2B- and 100B-class decode shapes and other long rows.)
    p.kind = 0;
    int64_t s = 1;
    if (nc <= 40 && m * nc * 256 <= kGemvMaxLds && (nb < 256 || nc < 16)) {
      p.qpl = 1;
      p.variant = nc >= 16 ? 8 : 4;
      p.pf = 4;
    } else {
      if (nb < 256) {
        s = cdiv(m == 1 ? kGemvTargetGroups : 2 * kGemvTargetGroups, nb);
        if (s > 4) s = 4;
        const int64_t smax = nc / 2 > 1 ? nc / 2 : 1;
        if (s > smax) s = smax;
      }
      while (m * cdiv(nc, s) * 256 > kGemvMaxLds) ++s;
      const int64_t per_group = nc / s;
      p.qpl = 4;
      const bool four = nb * s >= 128 && (m == 1 || s == 1);
      p.variant = four || per_group < 6 ? 4 : 8;
      p.pf = per_group / p.variant >= 4 ? 2 : 1;
    }
    p.splits = (int)s;
    p.slots = s > 1 ? (size_t)(nb * m * 64) : 0;
    // The streaming matrix-core GEMV for matrices of >= 1024 rows whose x~
    // (every token, all of K) fits a workgroup's LDS: no K split, about one
    // workgroup per CU.  Rows of at least 12 super-chunks at one token, 8 at
    // two (shorter rows leave its waves too little to stream; measured on
    // MI355X against the plans above, bit for bit).
    const int64_t subs = nb * 4;
    if (subs >= kStreamMinSubs && nc >= (m == 1 ? 12 : 8)) {
      const int64_t grid = subs < kCUs ? subs : kCUs;
      if (stream_lds_bytes((int)m, nc, (int)cdiv(subs, grid)) <= kStreamMaxLds) {
        p.kind = 3;
        p.qpl = (int)grid;
        p.splits = 1;
        p.slots = 0;
      }
    }
  } else if (m <= kMfmaGemvMaxM && mt_plan(m, n, k, &p)) {
    // multi-token streaming GEMV (below)
  } else if (m <= kMfmaGemvMaxM) {
    // Windowed MFMA GEMV: 16, 32 or 64 token columns.  Many row blocks
    // (>= 256): wide row groups, the whole K per wave; fewer: slices of K
    // over the waves of a workgroup, more slices (8 at 16 tokens, 4 at 64)
    // for long rows (>= 24 super-chunks) or few (<= 64) row blocks.  Past
    // 32 tokens, few row blocks keep 32-token blocks (twice the workgroups
    // of 64-token ones: 2560 x 6912 at 64 tokens 12.2 -> 7.3 us).  (Tuned
    // on MI355X over the 2B- and 100B-class decode shapes.)
    p.kind = 2;
    const bool wide = nb >= 256;
    if (m <= 16) p.variant = wide ? 2 : (nb <= 64 && nc >= 24) ? 1 : 0;
    else if (m <= 32) p.variant = wide ? 4 : 3;
    else p.variant = wide ? 6 : nb <= 64 ? 3 : nc >= 24 ? 7 : 5;
    p.splits = 1;
    p.slots = 0;
  } else {
    // MFMA GEMM, wide waves.  The tile shape maximises the work the first
    // rounds of tiles over the 256 CUs keep busy, weighted by how well each
    // shape runs (128 x 512 best, 64 x 512 then 64 x 256 and 96 x 256).
    // When even that leaves more than half the CUs without a tile, the
    // windowed MFMA GEMV takes the product in token blocks of 64, or of 32
    // for few row blocks (it needs no split of K).  (Tuned on MI355X over the 2048- and 512-token
    // prefills and the 100B-class k/v products.)
    static const double kRate[4] = {1.0, 0.9, 0.85, 0.85};
    double best = -1.0;
    int64_t tiles = 0;
    for (int v = 0; v < 4; ++v) {
      int bm, bn;
      gemm_tile_shape(v, &bm, &bn);
      const int64_t t = cdiv(m, bm) * cdiv(nb * 64, bn);
      const double useful = (double)m * (double)(nb * 64) / ((double)bm * bn);
      const double score = kRate[v] * useful / (double)(cdiv(t, kCUs) * kCUs);
      if (score > best) {
        best = score;
        p.variant = v;
        tiles = t;
      }
    }
    // Few tiles on short rows (<= 16 super-chunks): the multi-token
    // streaming GEMV when the matrix has >= 32 row blocks or the batch is
    // >= 512 tokens, else the windowed MFMA GEMV in token blocks (MI355X,
    // 2B-class q and k/v at 128-1024 tokens: q at 512 tokens 12.6 -> 9.5 us,
    // k/v at 1024 tokens 8.9 -> 6.9 us; on rows of 32 super-chunks, the
    // 100B-class k/v, the two tie)
    if (tiles < kCUs / 2 && nc <= 16 && (nb >= 32 || m >= 512)) {
      const int64_t subs = nb * 4;
      const int64_t P = mt_row_ranges(m, subs);
      if (stream_mt_lds_bytes(m, nc, (int)cdiv(subs, P), 16, 0) <= kMtMaxLds) {
        p.kind = 4;
        p.qpl = (int)P;
        p.splits = 1;
        p.slots = 0;
        p.ws_bytes = 0;
        return p;
      }
    }
    if (tiles < kCUs / 2) {
      p.kind = 2;
      p.variant = nb >= 256 ? 6 : nb <= 64 ? 3 : nc >= 24 ? 7 : 5;
    } else {
      p.kind = 1;
    }
    p.splits = 1;
    p.slots = 0;
  }
  p.ws_bytes = p.slots * 8;
  return p;
}

hipError_t launch_forward(const FwdPlan& plan, const int8_t* xq, const float* scale,
                          const uint32_t* packed, const float* gamma, int64_t m, int64_t n,
                          int64_t k, bool relu2, bool bf16, void* y, int32_t* acc_out,
                          void* workspace, hipStream_t stream) {
  int64_t* slots = plan.splits > 1 ? reinterpret_cast<int64_t*>(workspace) : nullptr;
  if (plan.kind == 0)
    return launch_gemv((int)m, plan.variant, plan.pf, plan.qpl, xq, scale, packed, gamma, n, k,
                       plan.splits, relu2, bf16, y, acc_out, slots, stream);
  if (plan.kind == 3)
    return launch_gemv_stream((int)m, xq, scale, packed, gamma, n, k, plan.qpl, relu2, bf16, y,
                              acc_out, stream);
  if (plan.kind == 4)
    return launch_gemv_stream_mt(xq, scale, packed, gamma, m, n, k, plan.qpl, relu2, bf16, y,
                                 acc_out, stream);
  if (plan.kind == 2)
    return launch_gemv_mfma(plan.variant, xq, scale, packed, gamma, m, n, k, relu2, bf16, y,
                            acc_out, stream);
  return launch_gemm(plan.variant, xq, scale, packed, gamma, m, n, k, relu2, bf16, y, acc_out,
                     stream);
}

struct FusedPlan {
  bool norm = false;                    // some entry has RMSNorm
  bool stream = false;                  // 1..2 tokens: the streaming matrix-core kernel
  bool stream_wide = false;             // its 16-wave shape (rows past 8 waves' registers)
  int xr = 0;                           // its activation units per thread and token
  int nsub_alloc = 0;                   // its sub-blocks per workgroup, at most
  int64_t nc_max = 0;
  bool mt = false;                      // the multi-token streaming kernel
  int mt_tok = 16;                      // its tokens per block: 8 or 16
  bool mfma = false;                    // 3..64 tokens: the fused MFMA kernel
  int variant = 0;                      // its wave layout
  int waves = 8;
  int qpl = 4;                          // 16-byte q-parts per lane (rows per group / 16)
  int groups = 0;
  size_t lds = 0;
  size_t ws_bytes = 0;
  int splits[kMaxFused] = {};
  size_t slot_off[kMaxFused] = {};      // bytes
  bool two_pass = false;                // quantize each input once, then each product's forward
  int src[kMaxFused] = {};              // two_pass: the entry whose x~ and s an entry reads
  size_t xq_off[kMaxFused] = {};        // two_pass: workspace offsets of a source's x~ and s
  size_t s_off[kMaxFused] = {};         //   (unused where the entry gives xq_out / scale_out)
  size_t scratch_off = 0;               // two_pass: where the x~ / s scratch starts
};

// The fused step on the streaming kernel: every entry's rows whole aligned
// 16-byte units of one activation dtype, every entry's x~ within the LDS, the
// activation rows within 8 units per thread and token, and some entry with
// rows of at least 8 super-chunks.  Workgroups are
// shared out in proportion to each entry's packed bytes, about one per CU in
// all, each entry at least one and at most one per 16-row sub-block.
static bool stream_fused_plan(const bl_linear* ops, int nops, int64_t m, bool norm,
                              FusedPlan* p) {
  const int xdt = ops[0].x_dtype;
  int64_t units = 0, nc_max = 0, nu_max = 0;
  for (int i = 0; i < nops; ++i) {
    const int64_t esize = ops[i].x_dtype == BL_BF16 ? 2 : 4;
    if (ops[i].x_dtype != xdt || (ops[i].k * esize) % 16 != 0 || ((uintptr_t)ops[i].x % 16) != 0)
      return false;
    const int64_t nc = cdiv(ops[i].k, kSuperK);
    units += cdiv(ops[i].n, kRowBlock) * 4 * nc;
    if (nc > nc_max) nc_max = nc;
    const int64_t nu = ops[i].k * esize / 16;
    if (nu > nu_max) nu_max = nu;
  }
  if (nc_max < 8 && !norm) return false;
  // 8 waves when every token's row fits their registers, else 16
  bool wide = false;
  int64_t xr = 0;
  for (int pass = 0; pass < 2; ++pass) {
    wide = pass == 1;
    int waves, depth;
    stream_fused_shape(wide, &waves, &depth);
    xr = cdiv(nu_max, 64 * waves);
    if (!(m * xr > 8 || (norm && m * xr > 4))) break;
    if (wide) return false;
  }
  // one workgroup per CU at most: a 16-wave workgroup fills a CU, so a
  // workgroup past the 256th would wait for a whole round
  int64_t gs[kMaxFused], total = 0;
  for (int i = 0; i < nops; ++i) {
    const int64_t subs = cdiv(ops[i].n, kRowBlock) * 4;
    const int64_t w = subs * cdiv(ops[i].k, kSuperK);
    int64_t gi = (kCUs * w + units / 2) / units;
    gs[i] = gi < 1 ? 1 : gi > subs ? subs : gi;
    total += gs[i];
  }
  while (total > kCUs) {
    int big = 0;
    for (int i = 1; i < nops; ++i) big = gs[i] > gs[big] ? i : big;
    if (gs[big] <= 1) break;
    --gs[big];
    --total;
  }
  int groups = 0, nsub_alloc = 1;
  for (int i = 0; i < nops; ++i) {
    const int64_t subs = cdiv(ops[i].n, kRowBlock) * 4;
    p->splits[i] = (int)gs[i];
    groups += (int)gs[i];
    const int spw = (int)cdiv(subs, gs[i]);
    if (spw > nsub_alloc) nsub_alloc = spw;
  }
  const size_t lds = stream_lds_bytes((int)m, nc_max, nsub_alloc);
  if (lds > kStreamMaxLds) return false;
  p->stream = true;
  p->stream_wide = wide;
  p->norm = norm;
  p->xr = (int)xr;
  p->nsub_alloc = nsub_alloc;
  p->nc_max = nc_max;
  p->groups = groups;
  p->lds = lds;
  p->ws_bytes = 0;
  return true;
}

// The fused step on the multi-token streaming kernel (faster than the fused
// windowed kernel on every 2B- and 100B-class shape measured at 8 to 64
// tokens on MI355X, e.g. 100B q/k/v at 64 tokens 49.9 -> 21.8 us, 2B q/k/v
// 11.6 -> 8.9 us): every entry's rows
// whole aligned 16-byte units of one activation dtype, a token's row within
// 16 units per lane (bf16 K <= 8192, fp32 K <= 4096), and x~ of a 16-token
// block plus the sums within the LDS.  Row ranges are shared out in
// proportion to each entry's packed bytes, about one workgroup per CU over
// the token blocks, each entry at least one and at most one per sub-block,
// multiples of 8 when there are several token blocks.
static bool mt_fused_plan(const bl_linear* ops, int nops, int64_t m, bool norm, FusedPlan* p) {
  const int xdt = ops[0].x_dtype;
  int64_t units = 0, nc_max = 0, nu_max = 0;
  for (int i = 0; i < nops; ++i) {
    const int64_t esize = ops[i].x_dtype == BL_BF16 ? 2 : 4;
    if (ops[i].x_dtype != xdt || (ops[i].k * esize) % 16 != 0 || ((uintptr_t)ops[i].x % 16) != 0)
      return false;
    const int64_t nc = cdiv(ops[i].k, kSuperK);
    units += cdiv(ops[i].n, kRowBlock) * 4 * nc;
    if (nc > nc_max) nc_max = nc;
    const int64_t nu = ops[i].k * esize / 16;
    if (nu > nu_max) nu_max = nu;
  }
  const int64_t xr = cdiv(nu_max, 64);
  if (xr > 16) return false;
  // Row ranges for tok tokens per block: about one workgroup per CU over the
  // ceil(m / tok) blocks, shared in proportion to the entries' packed bytes,
  // multiples of 8 when there are several blocks.
  auto allocate = [&](int tok, int64_t (&ps)[kMaxFused]) {
    const int64_t tb = cdiv(m, tok);
    const int64_t budget = (kCUs / tb) < 1 ? 1 : kCUs / tb;
    const int64_t step = tb > 1 ? 8 : 1;
    int64_t total = 0;
    for (int i = 0; i < nops; ++i) {
      const int64_t subs = cdiv(ops[i].n, kRowBlock) * 4;
      const int64_t w = subs * cdiv(ops[i].k, kSuperK);
      int64_t pi = (budget * w + units / 2) / units;
      if (pi >= step) pi -= pi % step;
      ps[i] = pi < 1 ? 1 : pi > subs ? subs : pi;
      total += ps[i];
    }
    while (total > budget) {
      int big = 0;
      for (int i = 1; i < nops; ++i) big = ps[i] > ps[big] ? i : big;
      const int64_t dec = ps[big] > step ? step : ps[big] - 1;
      if (dec <= 0) break;
      ps[big] -= dec;
      total -= dec;
    }
  };
  // Tokens per block, 8 or 16: every row range quantizes its block's rows
  // (tok * K elements of VALU work per workgroup), and every block re-reads
  // the weights.  The plan takes the block size whose slowest workgroup
  // costs least, with one 1 KiB weight unit streamed worth 620 elements
  // quantized (fitted to per-launch times on MI355X over the 2B- and
  // 100B-class groups at 16, 32 and 64 tokens, where it picks the faster
  // size every time: 8-token blocks are 9-17% faster on the 2B set at 16-32
  // tokens and win at 64 tokens on short outputs and long rows; 16-token
  // blocks win on the large 100B outputs).  An RMSNorm row costs about three
  // times the VALU work (fp64 squares, two gain multiplies per pass), so its
  // elements count three times (2B-class q/k/v and up with RMSNorm at 64
  // tokens: 8-token blocks 9.9 / 10.4 us against 11.0 / 11.3 us with 16).
  // RMSNorm entries with a gain stage it in LDS (the longest such row)
  int64_t gain_k = 0;
  for (int i = 0; i < nops; ++i)
    if (norm && ops[i].rmsnorm && ops[i].norm_weight != nullptr && ops[i].k > gain_k)
      gain_k = ops[i].k;
  auto lds_of = [&](int t, const int64_t (&q)[kMaxFused]) {
    int na = 1;
    for (int i = 0; i < nops; ++i) {
      const int spw = (int)cdiv(cdiv(ops[i].n, kRowBlock) * 4, q[i]);
      if (spw > na) na = spw;
    }
    return stream_mt_lds_bytes(m, nc_max, na, t, gain_k);
  };
  int tok = 16;
  int64_t ps[kMaxFused];
  double best = -1.0;
  for (int t : {16, 8}) {
    int64_t q[kMaxFused];
    allocate(t, q);
    if (lds_of(t, q) > kMtMaxLds) continue;
    double cost = 0.0;
    for (int i = 0; i < nops; ++i) {
      const int64_t subs = cdiv(ops[i].n, kRowBlock) * 4;
      const double c = (double)(t < m ? t : m) * (double)ops[i].k / (ops[i].rmsnorm ? 207.0 : 620.0) +
                       (double)(cdiv(subs, q[i]) * cdiv(ops[i].k, kSuperK));
      if (c > cost) cost = c;
    }
    if (best < 0.0 || cost < best) {
      best = cost;
      tok = t;
      for (int i = 0; i < nops; ++i) ps[i] = q[i];
    }
  }
  if (best < 0.0) return false;
  const int64_t tb = cdiv(m, tok);
  int groups = 0, nsub_alloc = 1;
  for (int i = 0; i < nops; ++i) {
    const int64_t subs = cdiv(ops[i].n, kRowBlock) * 4;
    p->splits[i] = (int)(ps[i] * tb);
    groups += p->splits[i];
    const int spw = (int)cdiv(subs, ps[i]);
    if (spw > nsub_alloc) nsub_alloc = spw;
  }
  const size_t lds = stream_mt_lds_bytes(m, nc_max, nsub_alloc, tok, gain_k);
  if (lds > kMtMaxLds) return false;
  p->mt = true;
  p->mt_tok = tok;
  p->norm = norm;
  p->xr = (int)xr;
  p->nsub_alloc = nsub_alloc;
  p->nc_max = nc_max;
  p->groups = groups;
  p->lds = lds;
  p->ws_bytes = 0;
  return true;
}

// Two entries read the same activations when x, its dtype, K and the
// RMSNorm settings agree (their x~ and s are then the same).
static bool same_input(const bl_linear& a, const bl_linear& b) {
  if (a.x != b.x || a.x_dtype != b.x_dtype || a.k != b.k || (a.rmsnorm != 0) != (b.rmsnorm != 0))
    return false;
  return a.rmsnorm == 0 || (a.norm_weight == b.norm_weight &&
                            __builtin_bit_cast(uint32_t, a.norm_eps) ==
                                __builtin_bit_cast(uint32_t, b.norm_eps));
}

// The fused step for activation rows of more than 16 KiB at 3 or more
// tokens, which a multi-token workgroup cannot hold in registers and which
// would cost every workgroup tok * K elements of quantization: each distinct
// input is quantized once (the bitlinear_quant_act or
// bitlinear_rmsnorm_quant_act kernel; an entry that asks for xq_out or
// scale_out gets its own quantization, written there), then every product
// runs its bitlinear_forward plan on that x~, and a fill kernel clears the
// x~ / s scratch, so the workspace is left zero-filled as its contract
// requires.  Workspace: the largest forward split-K slot region, then the
// scratch, each 256-byte aligned.
static void two_pass_plan(const bl_linear* ops, int nops, int64_t m, FusedPlan* p) {
  auto up256 = [](size_t b) { return (b + 255) / 256 * 256; };
  size_t slots = 0;
  for (int i = 0; i < nops; ++i) {
    const size_t w = forward_plan(m, ops[i].n, ops[i].k).ws_bytes;
    if (w > slots) slots = w;
  }
  size_t off = up256(slots);
  p->scratch_off = off;
  for (int i = 0; i < nops; ++i) {
    const bl_linear& o = ops[i];
    const bool own = o.xq_out != nullptr || o.scale_out != nullptr;
    int src = i;
    if (!own)
      for (int j = 0; j < i && src == i; ++j)
        if (p->src[j] == j && ops[j].xq_out == nullptr && ops[j].scale_out == nullptr &&
            same_input(ops[j], o))
          src = j;
    p->src[i] = src;
    p->splits[i] = 1;
    if (src != i) continue;
    if (o.xq_out == nullptr) {
      p->xq_off[i] = off;
      off += up256((size_t)(m * padded_k(o.k)));
    }
    if (o.scale_out == nullptr) {
      p->s_off[i] = off;
      off += up256((size_t)(4 * m));
    }
  }
  p->two_pass = true;
  p->ws_bytes = off;
}

// The fused step's plan, in this order: at 1-2 tokens the streaming kernel
// when it takes the table; one RMSNorm product with rows of more than 8 KiB
// from 3 tokens, the two-pass plan; from 3 tokens (and RMSNorm tables at
// 1-2 tokens that the streaming kernel does not take) the multi-token
// kernel; rows of more than 16 KiB from 3 tokens, the two-pass plan; then
// the fused windowed matrix-core kernel from 3 tokens or with RMSNorm, and
// the dot4 decode kernel otherwise.
FusedPlan fused_plan(const bl_linear* ops, int nops, int64_t m) {
  FusedPlan p;
  bool norm = false;
  for (int i = 0; i < nops; ++i) norm = norm || ops[i].rmsnorm != 0;
  if (m <= 2 && stream_fused_plan(ops, nops, m, norm, &p)) return p;
  // One RMSNorm product with activation rows of more than 8 KiB from 3
  // tokens: normalizing tok rows of K in every workgroup of a token block
  // (about three times the VALU work of the plain quantization) costs more
  // than quantizing once in the two-pass plan (measured on MI355X: 2B-class
  // down at 8-64 tokens 14.0-16.2 -> 10.3-13.3 us, 100B-class o and up at
  // 4-48 tokens 14.9-47.2 -> 11.7-27.3 us; 2B-class o and up with 5 KB rows
  // about even, and tables of several products faster fused, e.g. the
  // 100B-class q/k/v at 16 tokens 19.9 fused against 21.7 us).
  if (m >= 3 && nops == 1 && ops[0].rmsnorm &&
      ops[0].k * (ops[0].x_dtype == BL_BF16 ? 2 : 4) > 8 * 1024) {
    p.norm = true;
    two_pass_plan(ops, nops, m, &p);
    return p;
  }
  if ((m >= 3 || norm) && m <= BL_FUSED_MAX_M && mt_fused_plan(ops, nops, m, norm, &p)) return p;
  if (m >= 3) {
    bool long_rows = false;                          // an activation row of more than 16 KiB
    for (int i = 0; i < nops; ++i)
      long_rows = long_rows || ops[i].k * (ops[i].x_dtype == BL_BF16 ? 2 : 4) > 16 * 1024;
    if (long_rows) {
      p.norm = norm;
      two_pass_plan(ops, nops, m, &p);
      return p;
    }
  }
  // RMSNorm tables that none of the kernels above takes run on the
  // matrix-core fused kernel at any token count
  p.norm = norm;
  if (m >= 3 || norm) {
    // Matrix cores: two 16-row groups x 4 K-slices per workgroup, or for
    // sets with >= 256 row blocks in an entry four 32-row groups with the
    // whole K per wave; no K split over workgroups, no workspace.
    int64_t nbmax = 0;
    for (int i = 0; i < nops; ++i) {
      const int64_t nb = cdiv(ops[i].n, kRowBlock);
      if (nb > nbmax) nbmax = nb;
    }
    p.mfma = true;
    p.variant = nbmax >= 256 ? 1 : 0;
    const int rows_per_group = p.variant == 0 ? 2 : 8;   // 16-row sub-blocks per workgroup
    for (int i = 0; i < nops; ++i) {
      p.splits[i] = 1;
      p.groups += (int)cdiv(cdiv(ops[i].n, kRowBlock) * 4, rows_per_group);
    }
    return p;
  }
  // The dot4 decode kernel.  T = super-chunks a workgroup should stream:
  // the set's total over ~512 groups, kept within [8, 32].  Entries with up
  // to 2T super-chunks keep one group per row block; longer ones are split
  // (atomic combine) into ~T-chunk ranges, at two tokens in large sets
  // (T >= 16) at most 2 (each split re-reads both activation rows for the
  // absmax).  4 waves per group, except 8 for large two-token sets with a
  // split entry.  (At one token 4 waves measured 9-18% faster than 8 on the
  // 100B-class up and down; at two tokens, up 4 waves -14%, down 2 splits x
  // 8 waves -23%.)  Rows per group: 16 (four lanes per row) when that keeps
  // the set within 512 groups, else 64 (a lane per row): small sets are
  // bound by each lane's unpack + dot4 work after the data arrive, large
  // ones by the number of groups, each of which reads and quantizes its x
  // range.  (Tuned on MI355X over the 2B- and 100B-class shapes.)
  int64_t units = 0;
  for (int i = 0; i < nops; ++i) units += cdiv(ops[i].n, kRowBlock) * cdiv(ops[i].k, kSuperK);
  int64_t t = cdiv(units, 512);
  t = t < 8 ? 8 : t > 32 ? 32 : t;
  const bool large2 = m > 1 && t >= 16;
  auto splits_of = [&](int64_t nc) {
    int64_t s = nc <= 2 * t ? 1 : cdiv(nc, t);
    if (s > (large2 ? 2 : 8)) s = large2 ? 2 : 8;
    while (m * cdiv(nc, s) * 256 > kGemvMaxLds) ++s;
    return s;
  };
  bool any_split = false;
  for (int i = 0; i < nops; ++i) any_split = any_split || splits_of(cdiv(ops[i].k, kSuperK)) > 1;
  p.waves = large2 && any_split ? 8 : 4;
  int64_t groups16 = 0;                              // groups with 16 rows each
  for (int i = 0; i < nops; ++i)
    groups16 += cdiv(ops[i].n, kRowBlock) * 4 * splits_of(cdiv(ops[i].k, kSuperK));
  p.qpl = groups16 <= 512 ? 1 : 4;
  size_t slots = 0;
  for (int i = 0; i < nops; ++i) {
    const int64_t nb = cdiv(ops[i].n, kRowBlock), nc = cdiv(ops[i].k, kSuperK);
    const int64_t s = splits_of(nc);
    p.splits[i] = (int)s;
    p.groups += (int)(nb * (4 / p.qpl) * s);
    const size_t lds = (size_t)(m * cdiv(nc, s) * 256);
    if (lds > p.lds) p.lds = lds;
    if (s > 1) {
      p.slot_off[i] = slots * 8;
      slots += (size_t)(nb * m * 64);
    }
  }
  p.ws_bytes = slots * 8;
  return p;
}

}  // namespace bl

using namespace bl;

namespace {
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline bool valid_dtype(int d) { return d == BL_F32 || d == BL_BF16; }
inline bool valid_eps(float e) { return isfinite(e) && e >= 0.0f; }
// Activation eps: s = 127 / max(beta, eps) must be a finite fp32 for every
// beta >= 0, so that an all-zero token quantizes to 0 (0 * s = 0) and no
// product x * s is NaN.  That needs eps > 0 with fp32(127 / eps) finite
// (eps >= about 3.74e-37); 0 and smaller values are refused.
inline bool valid_act_eps(float e) {
  if (!(isfinite(e) && e > 0.0f)) return false;
  const volatile float smax = 127.0f / e;
  return isfinite((float)smax);
}
inline bool valid_norm_eps(float e) { return isfinite(e) && e > 0.0f; }
}  // namespace

extern "C" {

int bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

const char* bitlinear_status_string(int status) {
  switch (status) {
    case BL_OK: return "ok";
    case BL_ERR_INVALID_ARG: return "invalid argument";
    case BL_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case BL_ERR_MISALIGNED: return "misaligned pointer";
    case BL_ERR_WORKSPACE: return "workspace missing or too small";
    case BL_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

// Size queries: 0 outside the sizes the entry points accept (1..BL_MAX_MN
// rows and tokens, 1..BL_MAX_K inputs), where every product below fits in
// int64 (2^24 * 2^18 = 2^42).
static bool mn_ok(int64_t v) { return v >= 1 && v <= BL_MAX_MN; }
static bool k_ok(int64_t k) { return k >= 1 && k <= BL_MAX_K; }

int64_t bitlinear_padded_n(int64_t n) { return mn_ok(n) ? padded_n(n) : 0; }
int64_t bitlinear_padded_k(int64_t k) { return k_ok(k) ? padded_k(k) : 0; }

size_t bitlinear_packed_bytes(int64_t n, int64_t k) {
  if (!mn_ok(n) || !k_ok(k)) return 0;
  return (size_t)(padded_n(n) * padded_k(k) / 4);
}

size_t bitlinear_xq_bytes(int64_t m, int64_t k) {
  if (!mn_ok(m) || !k_ok(k)) return 0;
  return (size_t)(m * padded_k(k));
}

size_t bitlinear_pack_workspace_bytes(int64_t n, int64_t k) {
  if (!mn_ok(n) || !k_ok(k)) return 0;
  return pack_workspace_bytes(n, k);
}

size_t bitlinear_forward_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k > BL_MAX_K || n > BL_MAX_MN || m > BL_MAX_MN) return 0;
  return forward_plan(m, n, k).ws_bytes;
}

static bl_status check_fused(const bl_linear* ops, int nops, int64_t m) {
  if (ops == nullptr || nops < 1 || nops > BL_MAX_FUSED) return BL_ERR_INVALID_ARG;
  if (m < 0) return BL_ERR_INVALID_ARG;
  if (m > BL_FUSED_MAX_M) return BL_ERR_UNSUPPORTED_SHAPE;
  for (int i = 0; i < nops; ++i) {
    const bl_linear& o = ops[i];
    if (!valid_dtype(o.x_dtype) || !valid_dtype(o.y_dtype)) return BL_ERR_INVALID_ARG;
    if (o.epilogue != BL_EPI_NONE && o.epilogue != BL_EPI_RELU2) return BL_ERR_INVALID_ARG;
    if (o.n < 1 || o.k < 1) return BL_ERR_INVALID_ARG;
    if (o.n > BL_MAX_MN || o.k > BL_MAX_K) return BL_ERR_UNSUPPORTED_SHAPE;
    if (o.rmsnorm && !valid_norm_eps(o.norm_eps)) return BL_ERR_INVALID_ARG;
    if (m == 0) continue;
    if (o.x == nullptr || o.packed == nullptr || o.gamma == nullptr || o.y == nullptr)
      return BL_ERR_INVALID_ARG;
    if (o.rmsnorm && o.norm_weight != nullptr && !aligned(o.norm_weight, 16))
      return BL_ERR_MISALIGNED;
    if (!aligned(o.x, o.x_dtype == BL_BF16 ? 2 : 4) || !aligned(o.packed, 16) ||
        !aligned(o.gamma, 4) || !aligned(o.y, o.y_dtype == BL_BF16 ? 2 : 4) ||
        (o.acc_out != nullptr && !aligned(o.acc_out, 4)) ||
        (o.xq_out != nullptr && !aligned(o.xq_out, 16)) ||
        (o.scale_out != nullptr && !aligned(o.scale_out, 4)))
      return BL_ERR_MISALIGNED;
  }
  return BL_OK;
}

size_t bitlinear_forward_fused_workspace_bytes(const bl_linear* ops, int nops, int64_t m) {
  if (check_fused(ops, nops, m) != BL_OK || m == 0) return 0;
  return fused_plan(ops, nops, m).ws_bytes;
}

bl_status bitlinear_forward_fused(const bl_linear* ops, int nops, int64_t m, float eps,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const bl_status st = check_fused(ops, nops, m);
  if (st != BL_OK) return st;
  if (!valid_act_eps(eps)) return BL_ERR_INVALID_ARG;
  if (m == 0) return BL_OK;
  const FusedPlan plan = fused_plan(ops, nops, m);
  if (plan.ws_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.ws_bytes) return BL_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return BL_ERR_MISALIGNED;
  }
  if (plan.two_pass) {
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    char* ws = reinterpret_cast<char*>(workspace);
    const int8_t* xq[kMaxFused] = {};
    const float* sc[kMaxFused] = {};
    for (int i = 0; i < nops; ++i) {
      const bl_linear& o = ops[i];
      if (plan.src[i] != i) continue;
      int8_t* q = o.xq_out != nullptr ? o.xq_out : reinterpret_cast<int8_t*>(ws + plan.xq_off[i]);
      float* s = o.scale_out != nullptr ? o.scale_out : reinterpret_cast<float*>(ws + plan.s_off[i]);
      const bool xb = o.x_dtype == BL_BF16;
      const hipError_t e =
          o.rmsnorm ? launch_rmsnorm_quant(o.x, xb, m, o.k, padded_k(o.k), o.norm_weight,
                                           o.norm_eps, eps, q, s, hs)
                    : launch_quant_act(o.x, xb, m, o.k, padded_k(o.k), eps, q, s, hs);
      if (e != hipSuccess) return BL_ERR_HIP;
      xq[i] = q;
      sc[i] = s;
    }
    for (int i = 0; i < nops; ++i) {
      const bl_linear& o = ops[i];
      const int j = plan.src[i];
      const FwdPlan fp = forward_plan(m, o.n, o.k);
      const hipError_t e = launch_forward(fp, xq[j], sc[j], reinterpret_cast<const uint32_t*>(o.packed),
                                          o.gamma, m, o.n, o.k, o.epilogue == BL_EPI_RELU2,
                                          o.y_dtype == BL_BF16, o.y, o.acc_out, workspace, hs);
      if (e != hipSuccess) return BL_ERR_HIP;
    }
    if (plan.ws_bytes > plan.scratch_off &&
        launch_fill_zero(reinterpret_cast<uint32_t*>(ws + plan.scratch_off),
                         (plan.ws_bytes - plan.scratch_off) / 4, hs) != hipSuccess)
      return BL_ERR_HIP;
    return BL_OK;
  }
  FusedArgs args{};
  args.nseg = nops;
  args.eps = eps;
  int begin = 0;
  for (int i = 0; i < nops; ++i) {
    const bl_linear& o = ops[i];
    FusedSeg& sg = args.seg[i];
    sg.x = o.x;
    sg.packed = o.packed;
    sg.gamma = o.gamma;
    sg.y = o.y;
    sg.acc_out = o.acc_out;
    sg.xq_out = o.xq_out;
    sg.scale_out = o.scale_out;
    sg.n = (int)o.n;
    sg.k = (int)o.k;
    sg.nc = (int)cdiv(o.k, kSuperK);
    sg.splits = plan.splits[i];
    sg.wg_begin = begin;
    sg.flags = (o.epilogue == BL_EPI_RELU2 ? 1 : 0) | (o.y_dtype == BL_BF16 ? 2 : 0) |
               (o.x_dtype == BL_BF16 ? 4 : 0) | (o.rmsnorm ? 8 : 0);
    sg.norm_weight = o.norm_weight;
    sg.norm_eps = o.norm_eps;
    args.wg_begin[i] = begin;
    if (sg.splits > 1 && !plan.stream && !plan.mt)
      sg.slots = reinterpret_cast<int64_t*>(reinterpret_cast<char*>(workspace) + plan.slot_off[i]);
    begin += plan.stream || plan.mt ? sg.splits
             : plan.mfma ? (int)cdiv(cdiv(o.n, kRowBlock) * 4, plan.variant == 0 ? 2 : 8)
                         : (int)(cdiv(o.n, kRowBlock) * (4 / plan.qpl) * sg.splits);
  }
  if (plan.stream) {
    args.nsub_alloc = plan.nsub_alloc;
    const hipError_t e = launch_gemv_stream_fused(args, (int)m, plan.stream_wide,
                                                  ops[0].x_dtype == BL_BF16, plan.norm, plan.xr,
                                                  begin, plan.lds,
                                                  reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? BL_OK : BL_ERR_HIP;
  }
  if (plan.mt) {
    args.nsub_alloc = plan.nsub_alloc;
    const hipError_t e = launch_gemv_stream_mt_fused(args, (int)m, plan.mt_tok,
                                                     ops[0].x_dtype == BL_BF16,
                                                     plan.norm, plan.xr, begin, plan.lds,
                                                     reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? BL_OK : BL_ERR_HIP;
  }
  if (plan.mfma) {
    bool all_bf16 = true, all_fast = true;
    for (int i = 0; i < nops; ++i) {
      const int64_t esize = ops[i].x_dtype == BL_BF16 ? 2 : 4;
      all_bf16 = all_bf16 && ops[i].x_dtype == BL_BF16;
      all_fast = all_fast && ops[i].k * esize % 16 == 0 && aligned(ops[i].x, 16);
    }
    const hipError_t e = launch_gemv_mfma_fused(args, (int)m, plan.variant, all_bf16, all_fast,
                                                plan.norm, begin,
                                                reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? BL_OK : BL_ERR_HIP;
  }
  bool long_rows = false;                            // a row of more than 1024 16-byte units
  for (int i = 0; i < nops; ++i)
    if (ops[i].k * (ops[i].x_dtype == BL_BF16 ? 2 : 4) > 1024 * 16) long_rows = true;
  const hipError_t e = launch_gemv_fused(args, (int)m, plan.waves, plan.qpl, long_rows && m == 1,
                                         plan.groups, plan.lds,
                                         reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? BL_OK : BL_ERR_HIP;
}

int bitlinear_forward_kernel(int64_t m, int64_t n, int64_t k) {
  if (m < 1 || n < 1 || k < 1) return -BL_ERR_INVALID_ARG;
  if (m > BL_MAX_MN || n > BL_MAX_MN || k > BL_MAX_K) return -BL_ERR_UNSUPPORTED_SHAPE;
  const FwdPlan p = forward_plan(m, n, k);
  switch (p.kind) {
    case 0: return BL_KERNEL_DOT4_GEMV;
    case 1: return BL_KERNEL_GEMM;
    case 2: return BL_KERNEL_MFMA_GEMV;
    case 3: return BL_KERNEL_STREAM_GEMV;
    default: return BL_KERNEL_STREAM_MT;
  }
}

int bitlinear_forward_fused_kernel(const bl_linear* ops, int nops, int64_t m) {
  const bl_status st = check_fused(ops, nops, m);
  if (st != BL_OK) return -(int)st;
  if (m < 1) return -BL_ERR_INVALID_ARG;
  const FusedPlan p = fused_plan(ops, nops, m);
  if (p.two_pass) return BL_KERNEL_TWO_PASS;
  if (p.stream) return BL_KERNEL_STREAM_GEMV;
  if (p.mt) return BL_KERNEL_STREAM_MT;
  if (p.mfma) return BL_KERNEL_MFMA_GEMV;
  return BL_KERNEL_DOT4_GEMV;
}

bl_status bitlinear_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (bytes == 0) return BL_OK;
  if (workspace == nullptr || bytes % 4 != 0) return BL_ERR_INVALID_ARG;
  if (!aligned(workspace, 4)) return BL_ERR_MISALIGNED;
  if (launch_fill_zero(reinterpret_cast<uint32_t*>(workspace), bytes / 4,
                       reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return BL_ERR_HIP;
  return BL_OK;
}

bl_status bitlinear_pack_weights(const void* w, int w_dtype, int64_t n, int64_t k, float eps,
                                 const float* gamma_in, void* packed, float* gamma_out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (w == nullptr || packed == nullptr || gamma_out == nullptr) return BL_ERR_INVALID_ARG;
  if (!valid_dtype(w_dtype) || !valid_eps(eps)) return BL_ERR_INVALID_ARG;
  if (n < 1 || k < 1) return BL_ERR_INVALID_ARG;
  if (n > BL_MAX_MN || k > BL_MAX_K) return BL_ERR_UNSUPPORTED_SHAPE;
  if (!aligned(w, 16) || !aligned(packed, 256) || !aligned(gamma_out, 4) ||
      (gamma_in != nullptr && !aligned(gamma_in, 4)))
    return BL_ERR_MISALIGNED;
  if (gamma_in == nullptr) {
    if (workspace == nullptr || workspace_bytes < pack_workspace_bytes(n, k))
      return BL_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return BL_ERR_MISALIGNED;
  }
  hipError_t e = launch_pack(w, w_dtype == BL_BF16, n, k, eps, gamma_in,
                             reinterpret_cast<uint32_t*>(packed), gamma_out,
                             reinterpret_cast<double*>(workspace),
                             reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? BL_OK : BL_ERR_HIP;
}

bl_status bitlinear_quant_act(const void* x, int x_dtype, int64_t m, int64_t k, float eps,
                              int8_t* xq, float* scale, void* stream) {
  if (!valid_dtype(x_dtype) || !valid_act_eps(eps)) return BL_ERR_INVALID_ARG;
  if (m < 0 || k < 1) return BL_ERR_INVALID_ARG;
  if (m > BL_MAX_MN || k > BL_MAX_K) return BL_ERR_UNSUPPORTED_SHAPE;
  if (m == 0) return BL_OK;
  if (x == nullptr || xq == nullptr || scale == nullptr) return BL_ERR_INVALID_ARG;
  if (!aligned(x, x_dtype == BL_BF16 ? 2 : 4) || !aligned(xq, 16) || !aligned(scale, 4))
    return BL_ERR_MISALIGNED;
  hipError_t e = launch_quant_act(x, x_dtype == BL_BF16, m, k, padded_k(k), eps, xq, scale,
                                  reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? BL_OK : BL_ERR_HIP;
}

bl_status bitlinear_rmsnorm_quant_act(const void* x, int x_dtype, int64_t m, int64_t k,
                                      const float* norm_weight, float norm_eps, float eps,
                                      int8_t* xq, float* scale, void* stream) {
  if (!valid_dtype(x_dtype) || !valid_act_eps(eps) || !valid_norm_eps(norm_eps))
    return BL_ERR_INVALID_ARG;
  if (m < 0 || k < 1) return BL_ERR_INVALID_ARG;
  if (m > BL_MAX_MN || k > BL_MAX_K) return BL_ERR_UNSUPPORTED_SHAPE;
  if (m == 0) return BL_OK;
  if (x == nullptr || xq == nullptr || scale == nullptr) return BL_ERR_INVALID_ARG;
  if (!aligned(x, x_dtype == BL_BF16 ? 2 : 4) || !aligned(xq, 16) || !aligned(scale, 4) ||
      (norm_weight != nullptr && !aligned(norm_weight, 4)))
    return BL_ERR_MISALIGNED;
  hipError_t e = launch_rmsnorm_quant(x, x_dtype == BL_BF16, m, k, padded_k(k), norm_weight,
                                      norm_eps, eps, xq, scale,
                                      reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? BL_OK : BL_ERR_HIP;
}

// Workgroups of a GEMM launch over products of widths ns[0..count-1]: the
// kernel numbers its tiles with 32-bit ints, so larger grids are refused.
static int64_t gemm_grid(int variant, int64_t m, const int64_t* ns, int count) {
  int bm, bn;
  gemm_tile_shape(variant, &bm, &bn);
  int64_t tn = 0;
  for (int i = 0; i < count; ++i) tn += cdiv(padded_n(ns[i]), bn);
  return cdiv(m, bm) * tn;
}

// A table of products sharing x~: the plan of one product over the summed
// output width decides.  If it is the GEMM, one launch over the table;
// otherwise each product gets its own plan and launch (the same numbers).
static bl_status check_multi(const int8_t* xq, const float* scale, int64_t m, int64_t k,
                             const bl_product* ops, int nops, int64_t* n_total) {
  if (ops == nullptr || nops < 1 || nops > BL_MAX_MULTI) return BL_ERR_INVALID_ARG;
  if (m < 0 || k < 1) return BL_ERR_INVALID_ARG;
  if (m > BL_MAX_MN || k > BL_MAX_K) return BL_ERR_UNSUPPORTED_SHAPE;
  int64_t nt = 0;
  for (int i = 0; i < nops; ++i) {
    const bl_product& o = ops[i];
    if (!valid_dtype(o.y_dtype)) return BL_ERR_INVALID_ARG;
    if (o.epilogue != BL_EPI_NONE && o.epilogue != BL_EPI_RELU2) return BL_ERR_INVALID_ARG;
    if (o.n < 1) return BL_ERR_INVALID_ARG;
    if (o.n > BL_MAX_MN) return BL_ERR_UNSUPPORTED_SHAPE;
    nt += padded_n(o.n);
  }
  if (nt > BL_MAX_MN) return BL_ERR_UNSUPPORTED_SHAPE;
  *n_total = nt;
  if (m == 0) return BL_OK;
  if (xq == nullptr || scale == nullptr) return BL_ERR_INVALID_ARG;
  if (!aligned(xq, 16) || !aligned(scale, 4)) return BL_ERR_MISALIGNED;
  for (int i = 0; i < nops; ++i) {
    const bl_product& o = ops[i];
    if (o.packed == nullptr || o.gamma == nullptr || o.y == nullptr) return BL_ERR_INVALID_ARG;
    if (!aligned(o.packed, 16) || !aligned(o.gamma, 4) ||
        !aligned(o.y, o.y_dtype == BL_BF16 ? 2 : 4) ||
        (o.acc_out != nullptr && !aligned(o.acc_out, 4)))
      return BL_ERR_MISALIGNED;
  }
  return BL_OK;
}

size_t bitlinear_forward_multi_workspace_bytes(const bl_product* ops, int nops, int64_t m,
                                               int64_t k) {
  int64_t nt = 0;
  if (check_multi(nullptr, nullptr, 0, k, ops, nops, &nt) != BL_OK || m <= 0 || m > BL_MAX_MN)
    return 0;
  if (forward_plan(m, nt, k).kind == 1) return 0;
  size_t need = 0;
  for (int i = 0; i < nops; ++i) {
    const size_t b = forward_plan(m, ops[i].n, k).ws_bytes;
    if (b > need) need = b;
  }
  return need;
}

bl_status bitlinear_forward_multi(const int8_t* xq, const float* scale, int64_t m, int64_t k,
                                  const bl_product* ops, int nops, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  int64_t nt = 0;
  const bl_status st = check_multi(xq, scale, m, k, ops, nops, &nt);
  if (st != BL_OK) return st;
  if (m == 0) return BL_OK;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const FwdPlan whole = forward_plan(m, nt, k);
  if (whole.kind == 1) {
    int64_t ns[kMaxMulti];
    for (int i = 0; i < nops; ++i) ns[i] = ops[i].n;
    if (gemm_grid(whole.variant, m, ns, nops) > INT32_MAX) return BL_ERR_UNSUPPORTED_SHAPE;
    GemmProduct g[kMaxMulti];
    for (int i = 0; i < nops; ++i)
      g[i] = GemmProduct{ops[i].packed, ops[i].gamma, ops[i].n, ops[i].epilogue == BL_EPI_RELU2,
                         ops[i].y_dtype == BL_BF16, ops[i].y, ops[i].acc_out};
    return launch_gemm_multi(whole.variant, xq, scale, m, k, g, nops, hs) == hipSuccess
               ? BL_OK : BL_ERR_HIP;
  }
  const size_t need = bitlinear_forward_multi_workspace_bytes(ops, nops, m, k);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return BL_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return BL_ERR_MISALIGNED;
  }
  for (int i = 0; i < nops; ++i) {
    const FwdPlan plan = forward_plan(m, ops[i].n, k);
    if (plan.kind == 1 && gemm_grid(plan.variant, m, &ops[i].n, 1) > INT32_MAX)
      return BL_ERR_UNSUPPORTED_SHAPE;
  }
  for (int i = 0; i < nops; ++i) {
    const bl_product& o = ops[i];
    const FwdPlan plan = forward_plan(m, o.n, k);
    const hipError_t e = launch_forward(plan, xq, scale, reinterpret_cast<const uint32_t*>(o.packed),
                                        o.gamma, m, o.n, k, o.epilogue == BL_EPI_RELU2,
                                        o.y_dtype == BL_BF16, o.y, o.acc_out, workspace, hs);
    if (e != hipSuccess) return BL_ERR_HIP;
  }
  return BL_OK;
}

// Argument checks of bitlinear_forward and bitlinear_forward_noalloc, all
// but the workspace; fills in the plan.
static bl_status check_forward(const int8_t* xq, const float* scale, const void* packed,
                               const float* gamma, int64_t m, int64_t n, int64_t k, int epilogue,
                               int y_dtype, const void* y, const int32_t* acc_out,
                               FwdPlan* plan) {
  if (!valid_dtype(y_dtype)) return BL_ERR_INVALID_ARG;
  if (epilogue != BL_EPI_NONE && epilogue != BL_EPI_RELU2) return BL_ERR_INVALID_ARG;
  if (m < 0 || n < 1 || k < 1) return BL_ERR_INVALID_ARG;
  if (m > BL_MAX_MN || n > BL_MAX_MN || k > BL_MAX_K) return BL_ERR_UNSUPPORTED_SHAPE;
  if (m == 0) return BL_OK;
  if (xq == nullptr || scale == nullptr || packed == nullptr || gamma == nullptr || y == nullptr)
    return BL_ERR_INVALID_ARG;
  if (!aligned(xq, 16) || !aligned(scale, 4) || !aligned(packed, 16) || !aligned(gamma, 4) ||
      !aligned(y, y_dtype == BL_BF16 ? 2 : 4) || (acc_out != nullptr && !aligned(acc_out, 4)))
    return BL_ERR_MISALIGNED;
  *plan = forward_plan(m, n, k);
  if (plan->kind == 1 && gemm_grid(plan->variant, m, &n, 1) > INT32_MAX)
    return BL_ERR_UNSUPPORTED_SHAPE;
  return BL_OK;
}

bl_status bitlinear_forward(const int8_t* xq, const float* scale, const void* packed,
                            const float* gamma, int64_t m, int64_t n, int64_t k, int epilogue,
                            int y_dtype, void* y, int32_t* acc_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  FwdPlan plan{};
  const bl_status st = check_forward(xq, scale, packed, gamma, m, n, k, epilogue, y_dtype, y,
                                     acc_out, &plan);
  if (st != BL_OK || m == 0) return st;
  if (plan.ws_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.ws_bytes) return BL_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return BL_ERR_MISALIGNED;
  }
  hipError_t e = launch_forward(plan, xq, scale, reinterpret_cast<const uint32_t*>(packed), gamma,
                                m, n, k, epilogue == BL_EPI_RELU2, y_dtype == BL_BF16, y, acc_out,
                                workspace, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? BL_OK : BL_ERR_HIP;
}

}  // extern "C"

// ------------------------------------------------------------------------
// bitlinear_forward_noalloc: bitlinear_forward whose split-K slots live in a
// scratch array of this library's code object instead of a caller workspace.
// Each device holds its own copy of the array for the life of the process.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is handed to kernels.
namespace {

static __device__ __align__(256) uint8_t scratch[BL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};     // device address of `scratch`, per device
bool g_scratch_clean[kMaxDevices] = {};    // cleared by a call outside stream capture

// The current device's scratch address, looked up on the first call on the
// device.  When the plan uses the scratch and no call outside stream capture
// has cleared it yet, a fill kernel clears it on `stream` first (a kernel,
// not hipMemsetAsync, so a captured graph replays it correctly); from then
// on every completed call leaves the slots it used zero-filled.
bl_status noalloc_scratch(bool needed, hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BL_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return BL_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  if (needed && !g_scratch_clean[dev]) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return BL_ERR_HIP;
    if (launch_fill_zero(reinterpret_cast<uint32_t*>(g_scratch_ptr[dev]),
                         BL_NOALLOC_SCRATCH_BYTES / 4, stream) != hipSuccess)
      return BL_ERR_HIP;
    if (cs == hipStreamCaptureStatusNone) g_scratch_clean[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return BL_OK;
}

}  // namespace

extern "C" bl_status bitlinear_forward_noalloc(const int8_t* xq, const float* scale,
                                               const void* packed, const float* gamma, int64_t m,
                                               int64_t n, int64_t k, int epilogue, int y_dtype,
                                               void* y, int32_t* acc_out, void* stream) {
  FwdPlan plan{};
  const bl_status st = check_forward(xq, scale, packed, gamma, m, n, k, epilogue, y_dtype, y,
                                     acc_out, &plan);
  if (st != BL_OK || m == 0) return st;
  if (plan.ws_bytes > BL_NOALLOC_SCRATCH_BYTES) return BL_ERR_WORKSPACE;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const bl_status sst = noalloc_scratch(plan.ws_bytes > 0, hs, &ws);
  if (sst != BL_OK) return sst;
  hipError_t e = launch_forward(plan, xq, scale, reinterpret_cast<const uint32_t*>(packed), gamma,
                                m, n, k, epilogue == BL_EPI_RELU2, y_dtype == BL_BF16, y, acc_out,
                                ws, hs);
  return e == hipSuccess ? BL_OK : BL_ERR_HIP;
}
