// C ABI of libbam.so: argument validation, workspace carving and kernel launches.
// The declarations, layouts, ownership and error rules are documented in include/bam.h.
#include <stdint.h>

#include <cmath>
#include <mutex>

// The library is built with -fvisibility=hidden: only the entry points declared in bam.h
// are exported.
#pragma GCC visibility push(default)
#include "../../include/bam.h"
#pragma GCC visibility pop
#include "bam_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

int pad64(int n) { return (n + 63) / 64 * 64; }

// Distance-table geometry: causal rows need d in [0, T-1]; non-causal [-(T-1), T-1].
struct TableGeom {
  int d0;
  int n;
  int stride;
};

TableGeom table_geom(int T, bool causal) {
  TableGeom g;
  g.d0 = causal ? 0 : -(T - 1);
  g.n = causal ? T : 2 * T - 1;
  g.stride = pad64(g.n);
  return g;
}

bool dims_ok(int B, int H, int T) { return B > 0 && H > 0 && T > 0; }

bam_status hip_status(hipError_t e) { return e == hipSuccess ? BAM_OK : BAM_EHIP; }

bool prior_ok(const float* alpha, const float* beta, const float* s, unsigned flags) {
  if (alpha == nullptr || beta == nullptr) return false;
  if ((flags & BAM_SSMAX) && s == nullptr) return false;
  if ((flags & BAM_PRIOR_REF) && (flags & BAM_PRIOR_SANDWICH)) return false;
  return true;
}

// Table kind selected by the prior flags (at most one is set; prior_ok checks that).
int prior_kind(unsigned flags) {
  if (flags & BAM_PRIOR_SANDWICH) return bam::kPriorSandwich;
  if (flags & BAM_PRIOR_REF) return bam::kPriorRef;
  return bam::kPriorAlpha;
}

constexpr unsigned kPriorFlags = BAM_PRIOR_REF | BAM_PRIOR_SANDWICH;

// bf16 forward table: reversed, padded with -inf by kFwdTabPad on each side, sqrt(Dh)-scaled
// (entry u holds d = dhi + kFwdTabPad - u).  The fp32 path uses the plain table.
TableGeom fwd_table_geom(int T, bool causal) {
  const TableGeom g = table_geom(T, causal);
  TableGeom r;
  r.d0 = (T - 1) + bam::kFwdTabPad;   // distance held at entry 0
  r.n = g.n + 2 * bam::kFwdTabPad;
  r.stride = pad64(r.n);
  return r;
}

// Forward workspace: the distance table, then (BAM_SKIP_FAR) the skipping plan's arrays.
struct FwdLayout {
  size_t smax_off, rowu_off, rowv_off, kpart_off, first_off, total;
  int nqb, nparts;
};

FwdLayout fwd_layout(int B, int H, int T, int Dh, unsigned flags) {
  FwdLayout L{};
  const bool causal = (flags & BAM_CAUSAL) != 0;
  const TableGeom g = fwd_table_geom(T, causal);
  L.total = align_up((size_t)H * g.stride * sizeof(float));
  if ((flags & BAM_SKIP_FAR) && causal && Dh > 0 && Dh % 8 == 0 && Dh <= 128) {
    const size_t BH = (size_t)B * H;
    L.nqb = (T + bam::fwd_bf16_rows_per_block(Dh, T) - 1) / bam::fwd_bf16_rows_per_block(Dh, T);
    L.nparts = (T + bam::skip_rows_per_block(Dh) - 1) / bam::skip_rows_per_block(Dh);
    L.smax_off = L.total;
    L.rowu_off = L.smax_off + align_up((size_t)H * T * sizeof(float));
    L.rowv_off = L.rowu_off + align_up(BH * T * sizeof(float));
    L.kpart_off = L.rowv_off + align_up(BH * T * sizeof(float));
    L.first_off = L.kpart_off + align_up(BH * L.nparts * sizeof(float));
    L.total = L.first_off + align_up(BH * L.nqb * sizeof(int32_t));
  }
  return L;
}

}  // namespace

extern "C" {

const char* bam_status_string(bam_status status) {
  switch (status) {
    case BAM_OK: return "ok";
    case BAM_EINVAL: return "invalid argument";
    case BAM_EUNSUPPORTED: return "unsupported dtype / head size / flags";
    case BAM_EWORKSPACE: return "workspace too small";
    case BAM_EHIP: return "HIP launch error";
    case BAM_ETOOLARGE: return "problem exceeds the library's static scratch buffer";
    default: return "unknown status";
  }
}

int bam_version(void) { return 100; }

bam_status bam_prior_table(const float* alpha, const float* beta, const float* mu, int H, int d0,
                           int n, float* tab, float* dalpha, float* dbeta, void* stream) {
  if (alpha == nullptr || beta == nullptr || tab == nullptr || H <= 0 || n <= 0) return BAM_EINVAL;
  return hip_status(bam::launch_prior_table(alpha, beta, mu, bam::kPriorAlpha, H, d0, n, n, 1.0f, tab, dalpha, dbeta,
                                            nullptr, (hipStream_t)stream));
}

bam_status bam_prior_table_ex(const float* alpha, const float* beta, const float* mu, int H, int d0,
                              int n, unsigned flags, float* tab, float* dalpha, float* dbeta, float* dmu,
                              void* stream) {
  if (alpha == nullptr || beta == nullptr || tab == nullptr || H <= 0 || n <= 0) return BAM_EINVAL;
  if ((flags & ~kPriorFlags) != 0 || !prior_ok(alpha, beta, nullptr, flags)) return BAM_EINVAL;
  return hip_status(bam::launch_prior_table(alpha, beta, mu, prior_kind(flags), H, d0, n, n, 1.0f,
                                            tab, dalpha, dbeta, dmu, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------
size_t bam_fwd_workspace_size(int B, int H, int T, int Dh, unsigned flags) {
  if (H <= 0 || T <= 0) return 0;
  return fwd_layout(B, H, T, Dh, flags).total;
}

bam_status bam_fwd_skip_plan_offset(int B, int H, int T, int Dh, unsigned flags, size_t* offset,
                                    int* count) {
  if (!dims_ok(B, H, T) || offset == nullptr || count == nullptr) return BAM_EINVAL;
  if (!(flags & BAM_SKIP_FAR) || !(flags & BAM_CAUSAL) || (Dh != 32 && Dh != 64 && Dh != 128))
    return BAM_EUNSUPPORTED;
  const FwdLayout L = fwd_layout(B, H, T, Dh, flags);
  *offset = L.first_off;
  *count = L.nqb * B * H;
  return BAM_OK;
}

bam_status bam_attn_fwd(const void* q, const void* k, const void* v, int in_dtype, int B, int H, int T,
                        int Dh, const float* alpha, const float* beta, const float* mu, const float* s,
                        unsigned flags, void* o, int o_dtype, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!dims_ok(B, H, T) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      lse == nullptr || workspace == nullptr || !prior_ok(alpha, beta, s, flags))
    return BAM_EINVAL;
  if ((flags & ~(BAM_CAUSAL | BAM_SSMAX | BAM_TABLE_READY | kPriorFlags | BAM_SKIP_FAR)) != 0) return BAM_EINVAL;
  if (o_dtype != BAM_BF16 && o_dtype != BAM_F32) return BAM_EUNSUPPORTED;
  if ((flags & BAM_SKIP_FAR) && (in_dtype != BAM_BF16 || !(flags & BAM_CAUSAL))) return BAM_EUNSUPPORTED;
  if (in_dtype == BAM_BF16) {
    if (Dh != 32 && Dh != 64 && Dh != 128) return BAM_EUNSUPPORTED;
  } else if (in_dtype == BAM_F32) {
    if (Dh != 32 && Dh != 64) return BAM_EUNSUPPORTED;
  } else {
    return BAM_EUNSUPPORTED;
  }
  if ((size_t)B * H * (size_t)T * Dh > ((size_t)1 << 40)) return BAM_EUNSUPPORTED;
  // the bf16 kernel addresses one (b, h) slab of Q, K, V with 32-bit buffer offsets
  if (in_dtype == BAM_BF16 && (size_t)T * Dh * 2 > (size_t)0x7fffffff) return BAM_EUNSUPPORTED;
  if (workspace_bytes < bam_fwd_workspace_size(B, H, T, Dh, flags)) return BAM_EWORKSPACE;

  const bool causal = (flags & BAM_CAUSAL) != 0;
  const int kind = prior_kind(flags);
  const bool bf16 = in_dtype == BAM_BF16;
  const TableGeom g = bf16 ? fwd_table_geom(T, causal) : table_geom(T, causal);
  hipStream_t st = (hipStream_t)stream;
  float* tab = (float*)workspace;
  hipError_t e = hipSuccess;
  // Up to kFwdStripT the short-sequence Dh = 64 kernel computes the alpha and reference
  // priors' bias itself; the table is then built only for the skipping plan, which reads it.
  const bool inkernel = bf16 && Dh == 64 && T <= bam::kFwdStripT && kind != bam::kPriorSandwich;
  if (!(flags & BAM_TABLE_READY) && (!inkernel || (flags & BAM_SKIP_FAR))) {
    if (bf16)
      e = bam::launch_prior_table_ex(alpha, beta, mu, kind, H, g.d0, -1, g.n, g.stride, causal ? 0 : -(T - 1), T - 1,
                                     std::sqrt((float)Dh), tab, nullptr, nullptr, nullptr, st);
    else
      e = bam::launch_prior_table(alpha, beta, mu, kind, H, g.d0, g.n, g.stride, 1.0f, tab, nullptr, nullptr,
                                  nullptr, st);
    if (e != hipSuccess) return BAM_EHIP;
  }
  bam::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.tab = tab;
  a.s = s;
  a.tab_d0 = g.d0;
  a.tab_stride = g.stride;
  a.B = B;
  a.H = H;
  a.T = T;
  a.causal = causal;
  a.ssmax = (flags & BAM_SSMAX) != 0;
  a.o = o;
  a.o_f32 = o_dtype == BAM_F32;
  a.lse = lse;
  a.first_tile = nullptr;
  a.bias_inkernel = inkernel;
  a.alpha = alpha;
  a.beta = beta;
  a.mu = mu;
  a.kind = kind;
  a.dlo = causal ? 0 : -(T - 1);
  a.dhi = T - 1;
  if (flags & BAM_SKIP_FAR) {
    const FwdLayout L = fwd_layout(B, H, T, Dh, flags);
    char* ws = (char*)workspace;
    bam::SkipArgs sk;
    sk.q = q;
    sk.k = k;
    sk.tab = tab;
    sk.tab_d0 = g.d0;
    sk.tab_stride = g.stride;
    sk.s = s;
    sk.ssmax = a.ssmax;
    sk.smax = (float*)(ws + L.smax_off);
    sk.rowu = (float*)(ws + L.rowu_off);
    sk.rowv = (float*)(ws + L.rowv_off);
    sk.kpart = (float*)(ws + L.kpart_off);
    sk.first_tile = (int32_t*)(ws + L.first_off);
    e = bam::launch_fwd_skip_plan(sk, B, H, T, Dh, bam::fwd_bf16_rows_per_block(Dh, T), st);
    if (e != hipSuccess) return BAM_EHIP;
    a.first_tile = sk.first_tile;
  }
  e = bf16 ? bam::launch_fwd_bf16(a, Dh, st) : bam::launch_fwd_f32(a, Dh, st);
  return hip_status(e);
}

// ---------------------------------------------------------------------------------------
namespace {
struct DecodeLayout {
  size_t tab_off, part_off, bound_off, total;
  int tab_stride, nsplit, chunk;
};

// workspace: the distance table, the split partials, then two floats per (b, h) for the
// skipping bound
DecodeLayout decode_layout(int B, int H, int Lmax, int Dh) {
  DecodeLayout d;
  d.tab_stride = pad64(Lmax);
  d.chunk = bam::decode_chunk_keys(Lmax, Dh, B * H);
  d.nsplit = (Lmax + d.chunk - 1) / d.chunk;
  d.tab_off = 0;
  d.part_off = align_up((size_t)H * d.tab_stride * sizeof(float));
  d.bound_off = d.part_off + align_up((size_t)B * H * d.nsplit * (Dh + 2) * sizeof(float));
  d.total = d.bound_off + align_up((size_t)B * H * 2 * sizeof(float));
  return d;
}
}  // namespace

size_t bam_decode_workspace_size(int B, int H, int Lmax, int Dh) {
  if (B <= 0 || H <= 0 || Lmax <= 0 || (Dh != 32 && Dh != 64 && Dh != 128)) return 0;
  return decode_layout(B, H, Lmax, Dh).total;
}

namespace {
bam_status decode_common(const void* q, const void* k, const void* v, int in_dtype, const int32_t* block_table,
                         int max_blocks, int num_pages, int page_size, const int32_t* kv_len, int B, int H,
                         int Lmax, int Dh, const float* alpha, const float* beta, const float* mu,
                         const float* s, unsigned flags, void* o, int o_dtype, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream, const float* key_norms = nullptr) {
  if (!dims_ok(B, H, Lmax) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      lse == nullptr || kv_len == nullptr || workspace == nullptr || !prior_ok(alpha, beta, s, flags))
    return BAM_EINVAL;
  if ((flags & ~(BAM_CAUSAL | BAM_SSMAX | BAM_TABLE_READY | kPriorFlags)) != 0) return BAM_EINVAL;
  if (in_dtype != BAM_BF16 || (Dh != 32 && Dh != 64 && Dh != 128)) return BAM_EUNSUPPORTED;
  if (o_dtype != BAM_BF16 && o_dtype != BAM_F32) return BAM_EUNSUPPORTED;
  const DecodeLayout L = decode_layout(B, H, Lmax, Dh);
  if (workspace_bytes < L.total) return BAM_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  float* tab = (float*)((char*)workspace + L.tab_off);
  if (!(flags & BAM_TABLE_READY)) {
    hipError_t e = bam::launch_prior_table(alpha, beta, mu, prior_kind(flags), H, 0, Lmax, L.tab_stride,
                                           1.0f, tab, nullptr, nullptr, nullptr, st);
    if (e != hipSuccess) return BAM_EHIP;
  }
  bam::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.kv_len = kv_len;
  a.tab = tab;
  a.s = s;
  a.tab_stride = L.tab_stride;
  a.B = B;
  a.H = H;
  a.Lmax = Lmax;
  a.ssmax = (flags & BAM_SSMAX) != 0;
  a.nsplit = L.nsplit;
  a.chunk = L.chunk;
  a.part = (float*)((char*)workspace + L.part_off);
  a.o = o;
  a.o_f32 = o_dtype == BAM_F32;
  a.lse = lse;
  a.key_norms = key_norms;
  a.npages = (Lmax + bam::kNormPage - 1) / bam::kNormPage;
  a.bound = (float*)((char*)workspace + L.bound_off);
  return hip_status(bam::launch_decode(a, Dh, st));
}
}  // namespace

bam_status bam_attn_decode(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                           const int32_t* kv_len, int B, int H, int Lmax, int Dh, const float* alpha,
                           const float* beta, const float* mu, const float* s, unsigned flags, void* o,
                           int o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return decode_common(q, k_cache, v_cache, in_dtype, nullptr, 0, 0, 0, kv_len, B, H, Lmax, Dh, alpha, beta, mu, s,
                       flags, o, o_dtype, lse, workspace, workspace_bytes, stream);
}

bam_status bam_decode_partials_layout(int B, int H, int Lmax, int Dh, size_t* offset, int* nsplit, int* chunk) {
  if (offset == nullptr || nsplit == nullptr || chunk == nullptr || bam_decode_workspace_size(B, H, Lmax, Dh) == 0)
    return BAM_EINVAL;
  const DecodeLayout L = decode_layout(B, H, Lmax, Dh);
  *offset = L.part_off;
  *nsplit = L.nsplit;
  *chunk = L.chunk;
  return BAM_OK;
}

int bam_decode_norm_pages(int Lmax) { return Lmax <= 0 ? 0 : (Lmax + bam::kNormPage - 1) / bam::kNormPage; }

bam_status bam_decode_key_norms(const void* k_cache, int in_dtype, int B, int H, int Lmax, int Dh, float* norms,
                                void* stream) {
  if (!dims_ok(B, H, Lmax) || !aligned16(k_cache) || norms == nullptr) return BAM_EINVAL;
  if (in_dtype != BAM_BF16 || (Dh != 32 && Dh != 64 && Dh != 128)) return BAM_EUNSUPPORTED;
  return hip_status(bam::launch_decode_key_norms(k_cache, B, H, Lmax, Dh, norms, (hipStream_t)stream));
}

bam_status bam_attn_decode_skip(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                                const int32_t* kv_len, int B, int H, int Lmax, int Dh, const float* alpha,
                                const float* beta, const float* mu, const float* s, unsigned flags,
                                const float* key_norms, void* o, int o_dtype, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (key_norms == nullptr) return BAM_EINVAL;
  return decode_common(q, k_cache, v_cache, in_dtype, nullptr, 0, 0, 0, kv_len, B, H, Lmax, Dh, alpha, beta, mu, s,
                       flags, o, o_dtype, lse, workspace, workspace_bytes, stream, key_norms);
}

// ---------------------------------------------------------------------------------------
// Decode with no workspace argument, for callers that cannot allocate: the distance table
// and the split partials live in this file's static device array.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current) and kept; host
// code uses only that address, never the array's name.  Every call on a device shares the
// array: calls that overlap on one device race.  Nothing in it needs to start at zero (the
// table kernel writes the whole table and every split writes its whole partial record).
namespace {
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the scratch array on the current device (null on failure).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

size_t bam_decode_static_max_bytes(void) { return kScratchBytes; }

bam_status bam_attn_decode_static(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                                  const int32_t* kv_len, int B, int H, int Lmax, int Dh, const float* alpha,
                                  const float* beta, const float* mu, const float* s, unsigned flags, void* o,
                                  int o_dtype, float* lse, void* stream) {
  if (!dims_ok(B, H, Lmax)) return BAM_EINVAL;
  if (in_dtype != BAM_BF16 || (Dh != 32 && Dh != 64 && Dh != 128)) return BAM_EUNSUPPORTED;
  if (bam_decode_workspace_size(B, H, Lmax, Dh) > kScratchBytes) return BAM_ETOOLARGE;
  void* ws = scratch_ptr();
  if (ws == nullptr) return BAM_EHIP;
  return decode_common(q, k_cache, v_cache, in_dtype, nullptr, 0, 0, 0, kv_len, B, H, Lmax, Dh, alpha, beta, mu, s,
                       flags, o, o_dtype, lse, ws, kScratchBytes, stream);
}

bam_status bam_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, int in_dtype,
                                 const int32_t* block_table, int max_blocks, int num_pages, int page_size,
                                 const int32_t* kv_len, int B, int H, int Dh, const float* alpha,
                                 const float* beta, const float* mu, const float* s, unsigned flags, void* o,
                                 int o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (block_table == nullptr || max_blocks <= 0 || num_pages <= 0 || page_size <= 0) return BAM_EINVAL;
  if (page_size % 64 != 0) return BAM_EUNSUPPORTED;
  if ((long)max_blocks * page_size > (long)INT32_MAX / 2) return BAM_EUNSUPPORTED;
  return decode_common(q, k_pages, v_pages, in_dtype, block_table, max_blocks, num_pages, page_size, kv_len, B, H,
                       max_blocks * page_size, Dh, alpha, beta, mu, s, flags, o, o_dtype, lse, workspace,
                       workspace_bytes, stream);
}

// ---------------------------------------------------------------------------------------
namespace {
// Backward workspace: the four distance tables (forward layout), the per-row scalars of the
// dK / dV kernel (four arrays over rows padded to 64) and the parameter partials; with
// BAM_SKIP_FAR (causal) then the skipping plan's arrays, planned per 128-query block.
struct BwdLayout {
  size_t tab_off, ta_off, tb_off, tm_off, rs_off, part_off, total;
  size_t smax_off, rowu_off, rowv_off, kpart_off, first_off;
  int Tp, nqb, nparts;
  TableGeom g;
};

constexpr int kBwdPlanRows = 128;   // query rows per block of the backward's skipping plan

BwdLayout bwd_layout(int B, int H, int T, int Dh, unsigned flags) {
  const bool causal = (flags & BAM_CAUSAL) != 0;
  BwdLayout L{};
  L.g = fwd_table_geom(T, causal);
  const size_t tabsz = align_up((size_t)H * L.g.stride * sizeof(float));
  L.Tp = (T + 63) / 64 * 64;
  L.tab_off = 0;
  L.ta_off = tabsz;
  L.tb_off = 2 * tabsz;
  L.tm_off = 3 * tabsz;
  L.rs_off = 4 * tabsz;
  L.part_off = L.rs_off + align_up((size_t)4 * B * H * L.Tp * sizeof(float));
  L.total = L.part_off + align_up(bam::bwd_param_partials(B, H, T) * sizeof(float));
  if ((flags & BAM_SKIP_FAR) && causal && Dh > 0 && Dh % 8 == 0 && Dh <= 128) {
    const size_t BH = (size_t)B * H;
    L.nqb = (T + kBwdPlanRows - 1) / kBwdPlanRows;
    L.nparts = (T + bam::skip_rows_per_block(Dh) - 1) / bam::skip_rows_per_block(Dh);
    L.smax_off = L.total;
    L.rowu_off = L.smax_off + align_up((size_t)H * T * sizeof(float));
    L.rowv_off = L.rowu_off + align_up(BH * T * sizeof(float));
    L.kpart_off = L.rowv_off + align_up(BH * T * sizeof(float));
    L.first_off = L.kpart_off + align_up(BH * L.nparts * sizeof(float));
    L.total = L.first_off + align_up(BH * L.nqb * sizeof(int32_t));
  }
  return L;
}
}  // namespace

size_t bam_bwd_workspace_size(int B, int H, int T, int Dh, unsigned flags) {
  if (!dims_ok(B, H, T)) return 0;
  return bwd_layout(B, H, T, Dh, flags).total;
}

bam_status bam_attn_bwd(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                        const float* lse, const void* dout, int in_dtype, int B, int H, int T, int Dh,
                        const float* alpha, const float* beta, const float* mu, const float* s,
                        unsigned flags, void* dq, void* dk, void* dv, int grad_dtype, float* dalpha,
                        float* dbeta, float* ds, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return bam_attn_bwd_ex(q, k, v, o, o_dtype, lse, dout, in_dtype, B, H, T, Dh, alpha, beta, mu, s, flags, dq,
                         dk, dv, grad_dtype, dalpha, dbeta, nullptr, ds, workspace, workspace_bytes, stream);
}

bam_status bam_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                           const float* lse, const void* dout, int in_dtype, int B, int H, int T, int Dh,
                           const float* alpha, const float* beta, const float* mu, const float* s,
                           unsigned flags, void* dq, void* dk, void* dv, int grad_dtype, float* dalpha,
                           float* dbeta, float* dmu, float* ds, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!dims_ok(B, H, T) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || lse == nullptr ||
      dalpha == nullptr || dbeta == nullptr || ds == nullptr || workspace == nullptr ||
      !prior_ok(alpha, beta, s, flags))
    return BAM_EINVAL;
  if ((flags & ~(BAM_CAUSAL | BAM_SSMAX | kPriorFlags | BAM_SKIP_FAR)) != 0) return BAM_EINVAL;
  if (in_dtype != BAM_BF16 || (Dh != 32 && Dh != 64)) return BAM_EUNSUPPORTED;
  if ((flags & BAM_SKIP_FAR) && !(flags & BAM_CAUSAL)) return BAM_EUNSUPPORTED;
  if ((o_dtype != BAM_BF16 && o_dtype != BAM_F32) || (grad_dtype != BAM_BF16 && grad_dtype != BAM_F32))
    return BAM_EUNSUPPORTED;
  // the dK / dV kernel's buffer loads address one (b, h) of Q / dO and all four row-scalar
  // arrays with 32-bit byte ranges
  if ((size_t)T * Dh * 2 > 0x7fffffffu || (size_t)16 * B * H * ((T + 63) / 64 * 64) > 0x7fffffffu)
    return BAM_EUNSUPPORTED;
  const bool causal = (flags & BAM_CAUSAL) != 0;
  const bool skip = (flags & BAM_SKIP_FAR) != 0;
  const BwdLayout L = bwd_layout(B, H, T, Dh, flags);
  if (workspace_bytes < L.total) return BAM_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* tab = (float*)(ws + L.tab_off);
  float* ta = (float*)(ws + L.ta_off);
  float* tb = (float*)(ws + L.tb_off);
  float* tm = dmu ? (float*)(ws + L.tm_off) : nullptr;
  // Up to kFwdStripT both kernels compute the alpha and reference priors' bias and
  // derivatives themselves; no table launch unless the skipping plan needs the table.
  const int kind = prior_kind(flags);
  const bool inkernel = T <= bam::kFwdStripT && kind != bam::kPriorSandwich;
  if (!inkernel || skip) {
    hipError_t e = bam::launch_prior_table_ex(alpha, beta, mu, kind, H, L.g.d0, -1, L.g.n, L.g.stride,
                                              causal ? 0 : -(T - 1), T - 1, std::sqrt((float)Dh), tab, ta, tb, tm,
                                              st);
    if (e != hipSuccess) return BAM_EHIP;
  }
  bam::BwdArgs a;
  a.bias_inkernel = inkernel;
  a.alpha = alpha;
  a.beta = beta;
  a.mu = mu;
  a.kind = kind;
  a.dlo = causal ? 0 : -(T - 1);
  a.dhi = T - 1;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.o_f32 = o_dtype == BAM_F32;
  a.lse = lse;
  a.dout = dout;
  a.tab = tab;
  a.tab_da = ta;
  a.tab_db = tb;
  a.tab_dm = tm;
  a.s = s;
  a.tab_d0 = L.g.d0;
  a.tab_stride = L.g.stride;
  a.B = B;
  a.H = H;
  a.T = T;
  a.causal = causal;
  a.ssmax = (flags & BAM_SSMAX) != 0;
  a.rowsc = (float*)(ws + L.rs_off);
  a.Tp = L.Tp;
  a.dq_acc = nullptr;
  a.param_part = (float*)(ws + L.part_off);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.grad_f32 = grad_dtype == BAM_F32;
  a.dalpha = dalpha;
  a.dbeta = dbeta;
  a.dmu = dmu;
  a.ds = ds;
  a.first_tile = nullptr;
  if (skip) {
    // the forward's plan over 128-query blocks (the dQ kernel's): the first key tile each
    // block needs; the dK / dV kernel leaves out the query tiles of blocks that start
    // beyond its keys
    bam::SkipArgs sk;
    sk.q = q;
    sk.k = k;
    sk.tab = tab;
    sk.tab_d0 = L.g.d0;
    sk.tab_stride = L.g.stride;
    sk.s = s;
    sk.ssmax = a.ssmax;
    sk.smax = (float*)(ws + L.smax_off);
    sk.rowu = (float*)(ws + L.rowu_off);
    sk.rowv = (float*)(ws + L.rowv_off);
    sk.kpart = (float*)(ws + L.kpart_off);
    sk.first_tile = (int32_t*)(ws + L.first_off);
    hipError_t e = bam::launch_fwd_skip_plan(sk, B, H, T, Dh, kBwdPlanRows, st);
    if (e != hipSuccess) return BAM_EHIP;
    a.first_tile = sk.first_tile;
  }
  return hip_status(bam::launch_bwd(a, Dh, st));
}

}  // extern "C"
