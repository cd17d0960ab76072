// Host-side declarations shared between the C-ABI module and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bam {

// Which per-head function of the distance the table holds.
enum PriorKind : int {
  kPriorAlpha = 0,     // -|(d - mu) / alpha|^beta
  kPriorRef = 1,       // -e^theta_alpha (|(j - i) - mu| + eps)^theta_beta
  kPriorSandwich = 2,  // sum_i cos(d w_i) / ratio (alpha = ratio, beta = d_bar)
};

// Launch the distance-table kernel: tab[h*stride + t] = b_h(d0 + t) (and derivatives;
// any derivative pointer may be null).
hipError_t launch_prior_table(const float* alpha, const float* beta, const float* mu, int kind, int H,
                              int d0, int n, int stride, float scale, float* tab, float* dalpha,
                              float* dbeta, float* dmu, hipStream_t stream);
// General form: entry t holds d = d_first + step * t; entries with d outside [dlo, dhi]
// are padding (-inf bias, zero derivatives).  The bias is multiplied by `scale`.
hipError_t launch_prior_table_ex(const float* alpha, const float* beta, const float* mu, int kind, int H,
                                 int d_first, int step, int n, int stride, int dlo, int dhi, float scale,
                                 float* tab, float* dalpha, float* dbeta, float* dmu, hipStream_t stream);

// Forward distance table: reversed (entry u holds d = dhi + kFwdTabPad - u), padded by
// kFwdTabPad entries of -inf on both sides and scaled by sqrt(Dh), so every per-tile
// window of the forward kernel is one contiguous, in-bounds copy.
constexpr int kFwdTabPad = 704;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* tab;   // bf16 path: reversed padded sqrt(Dh)-scaled table; fp32 path: b(d) at d - tab_d0
  const float* s;     // SSMax strength per head (NULL without SSMax)
  int tab_d0;         // distance held at index 0
  int tab_stride;     // floats per head row
  int B, H, T;
  bool causal, ssmax;
  void* o;
  bool o_f32;
  float* lse;
  const int32_t* first_tile;   // per work-group first key tile (prior-aware skipping), or null
  // The short-sequence Dh = 64 kernel computes its bias window itself (bias_inkernel, for
  // T <= kFwdStripT and the alpha and reference priors): the head's parameters, the prior
  // kind and the visible distance range [dlo, dhi]; the table is then not read.
  bool bias_inkernel;
  const float* alpha;
  const float* beta;
  const float* mu;
  int kind, dlo, dhi;
};

// Query rows per work-group of the bf16 forward kernel: two 32-row blocks per wave (256
// rows) for Dh <= 64, one (128 rows) for Dh = 128 and for Dh = 64 up to kFwdShortT.
// Short sequences have few key tiles per work-group, so finer work-groups balance the
// causal triangle better than the operand reuse of two blocks per wave pays.
constexpr int kFwdShortT = 1024;
// Up to this length the short-sequence Dh = 64 kernel computes the alpha and reference
// priors' bias itself (one strip of window entries per work-group, in LDS).
constexpr int kFwdStripT = 512;
constexpr int fwd_bf16_rows_per_block(int Dh, int T) {
  return (Dh == 128 || (Dh == 64 && T <= kFwdShortT)) ? 128 : 256;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int Dh, hipStream_t stream);

// Prior-aware skipping plan (causal bf16 forward): inputs and the workspace arrays it fills.
struct SkipArgs {
  const void* q;          // [B,H,T,Dh] bf16
  const void* k;
  const float* tab;       // the forward's reversed sqrt(Dh)-scaled table
  int tab_d0;             // its entry holding d = 0
  int tab_stride;
  const float* s;         // SSMax strength (null without SSMax)
  bool ssmax;
  float* smax;            // [H][ceil(T / 64)] suffix maximum of the bias at chunk starts
  float* rowu;            // [B*H][T]
  float* rowv;            // [B*H][T]
  float* kpart;           // [B*H][nparts] per-block max |k|
  int32_t* first_tile;    // [nqb * B * H]
};

int skip_rows_per_block(int Dh);
hipError_t launch_fwd_skip_plan(const SkipArgs& a, int B, int H, int T, int Dh, int MQ, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, int Dh, hipStream_t stream);

struct DecodeArgs {
  const void* q;        // [B,H,Dh]
  const void* k;        // [B,H,Lmax,Dh], or pages [num_pages,H,page_size,Dh] with a block table
  const void* v;
  const int32_t* block_table;   // [B, max_blocks] page ids, or null (contiguous caches)
  int max_blocks, num_pages, page_size;
  const int32_t* kv_len;
  const float* tab;     // [H][tab_stride], index = d (0 .. Lmax-1)
  const float* s;
  int tab_stride;
  int B, H, Lmax;
  bool ssmax;
  int nsplit;           // number of key ranges
  int chunk;            // keys per range (multiple of the per-block tile)
  float* part;          // [B,H,nsplit,Dh+2] partial (m, l, o)
  void* o;
  bool o_f32;
  float* lse;
  // prior-aware skipping (contiguous caches): key_norms [B,H,npages] per-64-key-page
  // maxima of |k|, or null (no skipping); bound [B,H,2] written by the bound kernel (a
  // lower bound of each row's largest logit, and |q| log2(e) / sqrt(Dh) rounded up)
  const float* key_norms;
  int npages;
  float* bound;
};

int decode_chunk_keys(int Lmax, int Dh, int BH);
hipError_t launch_decode(const DecodeArgs& a, int Dh, hipStream_t stream);
constexpr int kNormPage = 64;   // keys per page of the key-norm maxima
hipError_t launch_decode_key_norms(const void* k, int B, int H, int Lmax, int Dh, float* norms,
                                   hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  bool o_f32;
  const float* lse;
  const void* dout;
  // Distance tables in the forward's layout: reversed (entry e holds d = tab_d0 - e) and
  // padded by kFwdTabPad entries on both sides; tab holds sqrt(Dh) b(d) (-inf padding), the
  // derivative tables db/dalpha, db/dbeta, db/dmu unscaled (0 padding).
  const float* tab;
  const float* tab_da;   // db/dalpha
  const float* tab_db;   // db/dbeta
  const float* tab_dm;   // db/dmu (null: dmu not wanted)
  const float* s;
  int tab_d0;
  int tab_stride;
  int B, H, T;
  bool causal, ssmax;
  // Per-row scalars of the dK / dV kernel (written by the dQ kernel), four arrays
  // [B*H][Tp] (Tp = T rounded up to 64): Cl = c log2(e) / sqrt(Dh), L2 = lse log2(e),
  // D Cq with D = rowsum(dO * O), Cq = c / sqrt(Dh); rows at or beyond T hold FLT_MIN,
  // +inf, 0, 0.
  float* rowsc;
  int Tp;
  float* dq_acc;         // [B,H,T,Dh] fp32 accumulator
  float* param_part;     // [nparts][3][H] per-block partial sums (or direct)
  void* dq;
  void* dk;
  void* dv;
  bool grad_f32;
  float* dalpha;
  float* dbeta;
  float* dmu;            // null: not computed
  float* ds;
  // Up to kFwdStripT, for the alpha and reference priors, both kernels compute the bias and
  // derivative windows themselves (bias_inkernel): the head's parameters, the prior kind and
  // the visible distance range [dlo, dhi]; the tables are then not read.
  bool bias_inkernel;
  const float* alpha;
  const float* beta;
  const float* mu;
  int kind, dlo, dhi;
  // Prior-aware skipping (causal): per 128-query block of each (b, h), the first 64-key
  // tile that can carry a weight float32 holds (index qb * B * H + b * H + h), or null.
  const int32_t* first_tile;
};

size_t bwd_param_partials(int B, int H, int T);
hipError_t launch_bwd(const BwdArgs& a, int Dh, hipStream_t stream);

}  // namespace bam
