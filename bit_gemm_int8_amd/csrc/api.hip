// libbitlinear C ABI: argument checks, dispatch and launches.
// The entry points and their contracts are declared in include/bitlinear.h.
#include <math.h>

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

}  // namespace

hipError_t launch_fill_zero(uint32_t* p, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_zero_kernel<<<(unsigned)blocks, 256, 0, stream>>>(p, words);
  return hipGetLastError();
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
  if (plan.kind == 2)
    return launch_gemv_mfma(plan.variant, xq, scale, packed, gamma, m, n, k, relu2, bf16, y,
                            acc_out, stream);
  return launch_gemm(plan.variant, xq, scale, packed, gamma, m, n, k, relu2, bf16, y, acc_out,
                     stream);
}

struct FusedPlan {
  bool mfma = false;                    // 3..64 tokens: the fused MFMA kernel
  int variant = 0;                      // its wave layout
  int waves = 8;
  int qpl = 4;                          // 16-byte q-parts per lane (rows per group / 16)
  int groups = 0;
  size_t lds = 0;
  size_t ws_bytes = 0;
  int splits[kMaxFused] = {};
  size_t slot_off[kMaxFused] = {};      // bytes
};

FusedPlan fused_plan(const bl_linear* ops, int nops, int64_t m) {
  // T = super-chunks a workgroup should stream: the set's total over ~512
  // groups, kept within [8, 32].  Entries with up to 2T super-chunks keep
  // one group per row block; longer ones are split (atomic combine) into
  // ~T-chunk ranges, at two tokens in large sets (T >= 16) at most 2 (each
  // split re-reads both activation rows for the absmax).  4 waves per group,
  // except 8 for large two-token sets with a split entry.  (At one token 4
  // waves measured 9-18% faster than 8 on the 100B-class up and down; at two
  // tokens, up 4 waves -14%, down 2 splits x 8 waves -23%.)  Rows per group:
  // 16 (four lanes per row) when that keeps the set within 512 groups, else
  // 64 (a lane per row): small sets
  // are bound by each lane's unpack + dot4 work after the data arrive, large
  // ones by the number of groups, each of which reads and quantizes its x
  // range.  (Tuned on MI355X over the 2B- and 100B-class shapes.)
  FusedPlan p;
  if (m >= 3) {
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

int64_t bitlinear_padded_n(int64_t n) { return n <= 0 ? 0 : padded_n(n); }
int64_t bitlinear_padded_k(int64_t k) { return k <= 0 ? 0 : padded_k(k); }

size_t bitlinear_packed_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return 0;
  return (size_t)(padded_n(n) * padded_k(k) / 4);
}

size_t bitlinear_xq_bytes(int64_t m, int64_t k) {
  if (m <= 0 || k <= 0) return 0;
  return (size_t)(m * padded_k(k));
}

size_t bitlinear_pack_workspace_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return 0;
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
    if (m == 0) continue;
    if (o.x == nullptr || o.packed == nullptr || o.gamma == nullptr || o.y == nullptr)
      return BL_ERR_INVALID_ARG;
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
  if (!valid_eps(eps)) return BL_ERR_INVALID_ARG;
  if (m == 0) return BL_OK;
  const FusedPlan plan = fused_plan(ops, nops, m);
  if (plan.ws_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.ws_bytes) return BL_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return BL_ERR_MISALIGNED;
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
               (o.x_dtype == BL_BF16 ? 4 : 0);
    args.wg_begin[i] = begin;
    if (sg.splits > 1)
      sg.slots = reinterpret_cast<int64_t*>(reinterpret_cast<char*>(workspace) + plan.slot_off[i]);
    begin += plan.mfma ? (int)cdiv(cdiv(o.n, kRowBlock) * 4, plan.variant == 0 ? 2 : 8)
                       : (int)(cdiv(o.n, kRowBlock) * (4 / plan.qpl) * sg.splits);
  }
  if (plan.mfma) {
    bool all_bf16 = true, all_fast = true;
    for (int i = 0; i < nops; ++i) {
      const int64_t esize = ops[i].x_dtype == BL_BF16 ? 2 : 4;
      all_bf16 = all_bf16 && ops[i].x_dtype == BL_BF16;
      all_fast = all_fast && ops[i].k * esize % 16 == 0 && aligned(ops[i].x, 16);
    }
    const hipError_t e = launch_gemv_mfma_fused(args, (int)m, plan.variant, all_bf16, all_fast,
                                                begin, reinterpret_cast<hipStream_t>(stream));
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
  if (!valid_dtype(x_dtype) || !valid_eps(eps)) return BL_ERR_INVALID_ARG;
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

bl_status bitlinear_forward(const int8_t* xq, const float* scale, const void* packed,
                            const float* gamma, int64_t m, int64_t n, int64_t k, int epilogue,
                            int y_dtype, void* y, int32_t* acc_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
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
  const FwdPlan plan = forward_plan(m, n, k);
  if (plan.kind == 1 && gemm_grid(plan.variant, m, &n, 1) > INT32_MAX)
    return BL_ERR_UNSUPPORTED_SHAPE;
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
