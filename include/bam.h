/*
 * bam.h - C ABI of the BAM attention library (libbam.so) for AMD Instinct MI355X (gfx950).
 *
 * BAM (Bayesian Attention Mechanism) attention is causal scaled-dot-product attention
 * whose logits carry a per-head Generalized-Gaussian positional prior and are then
 * rescaled by Scalable-Softmax (SSMax):
 *
 *   b_h(d)   = -| (d - mu_h) / alpha_h |^beta_h,   d = i - j  (i query, j key)
 *   logit_ij = c_i * ( q_i . k_j / sqrt(Dh) + b_h(i - j) )
 *   c_i      = s_h * ln(n_i) with BAM_SSMAX (n_i = keys visible to query i), else 1
 *   P        = row softmax(logit),  O = P V,  lse_i = ln sum_j exp(logit_ij)
 *
 * Sources: "Bayesian Attention Mechanism" (authors' README), section "Implementation
 * Details" (per-head additive bias from a Generalized Gaussian prior, trained scale and
 * shape); "Résumé Technique : Mécanisme d'Attention Bayésienne (BAM)", section
 * "Solution Proposée : GGD-BAM" (the bias formula with alpha, beta, mu; beta in (0,1)
 * heavy-tailed, beta < 0 inverted; SSMax rescales logits); "ALiBi: Attention with
 * Linear Biases", section "Code" (scores = Q K^T / sqrt(d_k), add the bias, softmax).
 * Conventions where the pages are silent: the offset is taken as (i - j) - mu, there is
 * no epsilon, the SSMax factor is c_i above (the pages give no formula), lse is the
 * natural log.  Special values: u = |d - mu| / alpha; u = 0 and beta > 0 gives 0;
 * beta = 0 gives -1; alpha = +inf gives u = 0.  ALiBi (beta = 1, mu = 0,
 * alpha = 1 / m_h) and NoPE (alpha = +inf) are special cases.
 *
 * Memory and ownership
 *   - Every tensor argument is a DEVICE pointer on the current HIP device, allocated
 *     and owned by the caller.  The library allocates nothing and keeps no mutable
 *     global state; calls on different streams may run concurrently.
 *   - Dense tensors are row-major with the head dimension contiguous:
 *     q, k, v, o, dout, dq, dk, dv: [B, H, T, Dh];  lse: [B, H, T] float32.
 *   - alpha, beta, mu, s: float32[H] on the device.  mu may be NULL (all zero).  s is
 *     read only when BAM_SSMAX is set (it may be NULL otherwise).
 *   - Element types: BAM_BF16 (bfloat16 bits) or BAM_F32.  Data pointers must be 16-byte
 *     aligned.
 *   - workspace: caller-provided device scratch of at least bam_*_workspace_size()
 *     bytes, 256-byte aligned; its contents on entry do not matter.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream).  Calls
 *     return without synchronising; outputs are valid once the stream has reached them.
 *   - Inputs are never written.  Outputs are fully overwritten (dalpha, dbeta, ds too).
 *
 * Errors
 *   Host-checkable problems are reported before anything is enqueued, with no partial
 *   writes: BAM_EINVAL (null or misaligned pointer, non-positive size), BAM_EUNSUPPORTED
 *   (a dtype / head size / flag combination this build has no kernel for), BAM_EWORKSPACE
 *   (workspace too small).  A failed kernel launch returns BAM_EHIP.  Values that live on
 *   the device cannot be checked without a synchronisation and are preconditions:
 *   alpha > 0 (+inf allowed), beta finite, s > 0, 1 <= kv_len[b] <= Lmax, and for
 *   beta < 0 that d - mu != 0 for every visible distance d (otherwise the bias is -inf
 *   and that key is dropped).  q, k, v (and dout) must be finite: the kernels are compiled
 *   on the assumption that no NaN arises (from inputs that meet these preconditions none
 *   does; masked logits are -inf and no exp2 argument is -inf - -inf), so a NaN or
 *   infinite input gives undefined values, not necessarily NaN.  A NaN alpha, beta or mu
 *   likewise; the table entry points make a NaN Sandwich d_bar count as no frequency.
 */
#ifndef BAM_H
#define BAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int bam_status;
#define BAM_OK            0
#define BAM_EINVAL        1
#define BAM_EUNSUPPORTED  2
#define BAM_EWORKSPACE    3
#define BAM_EHIP          4
#define BAM_ETOOLARGE     5   /* bam_attn_decode_static: beyond its static scratch buffer */

/* element types */
#define BAM_BF16 0
#define BAM_F32  1

/* flags */
#define BAM_CAUSAL 1u   /* key j visible to query i only when j <= i */
#define BAM_SSMAX  2u   /* multiply the logits of query i by c_i = s_h ln(n_i) */
/* The workspace already holds the distance table written by an earlier call with the same
 * alpha, beta, mu, shape and flags (and the same workspace): skip rebuilding it.  For
 * callers whose prior parameters do not change between calls (inference); with trained
 * parameters leave it unset.  Accepted by bam_attn_fwd and bam_attn_decode. */
#define BAM_TABLE_READY 4u
/* Reference parameterisation of the prior ("Bayesian Attention Mechanism" README,
 * "Implementation Details", the formula and its AttentionPrior code): the per-head arrays
 * alpha, beta, mu hold theta_alpha, theta_beta, theta_mu and
 *   b_h(d) = -e^theta_alpha * ( |(j - i) - mu| + eps )^theta_beta,   d = i - j,
 *   mu = e^theta_mu - e^-theta_mu,   eps = BAM_REF_EPS.
 * (The page's printed formula writes (i - j) - mu; its code subtracts mu from j - i.  The
 * two agree for theta_mu = 0, the page's default; the code's sign is used.)  mu may be
 * NULL (theta_mu = 0).  Every value is finite for finite thetas (eps > 0), so the
 * beta < 0 precondition does not apply.  Accepted by every entry point. */
#define BAM_PRIOR_REF 8u
#define BAM_REF_EPS 1e-5
/* Sandwich relative-position bias (attention-gym "Score Mods", "Sandwich") in place of the
 * GGD prior: the inner product of two d_bar-dimensional sinusoidal position embeddings,
 * scaled down per head,
 *   b_h(d) = sum_{i = 0}^{d_bar/2 - 1} cos(d / 10000^(2 i / d_bar)) / ratio_h,
 * with alpha[h] = ratio_h (the page uses 8 (h + 1) / H) and beta[h] = d_bar (the page uses
 * 128); mu is ignored.  d_bar above 8192 is taken as 8192 (frequencies included), and the
 * frequency count is trunc(d_bar) / 2: none below 2 (a zero bias).  The bias has no parameters: the
 * backward's dalpha, dbeta and dmu are zero.  Not combinable with BAM_PRIOR_REF
 * (BAM_EINVAL).  Accepted by every entry point. */
#define BAM_PRIOR_SANDWICH 16u
/* Prior-aware key skipping (bam_attn_fwd and the backward, causal bf16 only;
 * BAM_EUNSUPPORTED otherwise).
 * For each block of query rows the call first bounds every logit from above,
 *   l_ij <= c_i (|q_i| max_j |k_j| / sqrt(Dh) + max_{d >= i - j} b(d)),
 * and the row maximum from below by the diagonal logit l_ii, then leaves out the leading
 * 64-key tiles whose every key sits more than 104 (> 150 ln 2) below that lower bound for
 * every row of the block.  Such a key's softmax weight is below 2^-150 of its row's
 * largest, i.e. zero in float32: the result is that of the full computation at float32
 * precision, while a prior that decays with distance (beta > 0 local heads) saves the far
 * tiles.  Rows with c_i <= 0 and non-finite bounds never skip; the bound assumes finite
 * q, k and bias.  Needs the larger workspace that bam_fwd_workspace_size reports for
 * these flags.  The backward plans the same way over 128-query blocks: the dQ pass starts
 * each block's key loop at its first needed tile, and the dK / dV pass leaves out the query
 * tiles of blocks whose first needed tile lies beyond its keys.  Every term it leaves out is
 * zero in float32 (its weight is, so its dZ is), so dQ, dK, dV and the parameter gradients
 * equal those of the full backward bit for bit (bam_bwd_workspace_size with the flag). */
#define BAM_SKIP_FAR 32u

/* Human-readable name of a status code (static storage, never NULL). */
const char* bam_status_string(bam_status status);

/* Library ABI version (major * 100 + minor). */
int bam_version(void);

/*
 * bam_prior_table - the per-head distance table of the GGD prior.
 *
 * Writes tab[h * n + t] = b_h(d0 + t) for t in [0, n), h in [0, H), in float32, where
 * b_h is the bias above (the exponent in float64, the result within about 2 float32 ulps,
 * rounded once to float32).  With dalpha / dbeta
 * non-NULL it also writes the parameter derivatives of the bias,
 *   dalpha[h * n + t] = db/dalpha = beta u^beta / alpha,
 *   dbeta [h * n + t] = db/dbeta  = -u^beta ln u          (both 0 where u = 0).
 * The attention entry points build this table themselves; it is exported so the table
 * can be checked on its own.  Because the bias depends on i - j only, one row of n
 * entries per head replaces the T x T bias matrix that the pages' module materialises
 * ("Bayesian Attention Mechanism", "Implementation Details").
 */
bam_status bam_prior_table(const float* alpha, const float* beta, const float* mu, int H,
                           int d0, int n, float* tab, float* dalpha, float* dbeta,
                           void* stream);

/*
 * bam_prior_table_ex - bam_prior_table for either parameterisation, with the offset
 * derivative.  flags: 0 (alpha-form), BAM_PRIOR_REF or BAM_PRIOR_SANDWICH (whose
 * derivatives are zero).  dalpha, dbeta, dmu may each be NULL.  Alpha-form: dmu = db/dmu = beta u^beta / (d - mu) (0 where u = 0).  Reference
 * form, with x = (j - i) - mu and g = |x| + eps:
 *   dalpha = db/dtheta_alpha = b,   dbeta = db/dtheta_beta = b ln g,
 *   dmu    = db/dtheta_mu    = -b theta_beta sign(x) / g * (e^theta_mu + e^-theta_mu)
 * (sign(0) = 0).
 */
bam_status bam_prior_table_ex(const float* alpha, const float* beta, const float* mu, int H,
                              int d0, int n, unsigned flags, float* tab, float* dalpha,
                              float* dbeta, float* dmu, void* stream);

/*
 * bam_attn_fwd - prefill forward.
 *
 * q, k, v: [B, H, T, Dh] of in_dtype.  flags: BAM_CAUSAL and/or BAM_SSMAX.
 * Without BAM_CAUSAL every query sees all T keys (n_i = T).
 * o: [B, H, T, Dh] of o_dtype (BAM_BF16 output is the round-to-nearest-even of the
 * float32 result).  lse: [B, H, T] float32, natural log.
 * Precision of the bf16 path: Q K^T and P V run on bf16 MFMA with fp32 accumulation; the
 * softmax weights are rounded to bf16 for P V, each at most 1 (the running row maximum is
 * exact), while the row sum and lse use the unrounded fp32 weights.  Any finite bf16 V
 * is accepted.
 * Supported: in_dtype BAM_BF16 with Dh in {32, 64, 128} (bf16 MFMA, fp32 accumulate) and
 * T * Dh * 2 < 2^31 bytes per (b, h); in_dtype BAM_F32 with Dh in {32, 64} (fp32
 * throughout).  Larger requests return BAM_EUNSUPPORTED.  BAM_SKIP_FAR: see above.
 * Bias: for in_dtype BAM_BF16, Dh = 64, T <= 512 and the alpha or reference prior, the
 * kernel computes the bias of each distance itself in float32 arithmetic (within a few
 * float32 ulps of the distance table's value, which is derived in float64) and builds no
 * table unless BAM_SKIP_FAR needs one; BAM_TABLE_READY then changes nothing.  Every other
 * case reads the distance table from the workspace.
 */
size_t bam_fwd_workspace_size(int B, int H, int T, int Dh, unsigned flags);
bam_status bam_attn_fwd(const void* q, const void* k, const void* v, int in_dtype,
                        int B, int H, int T, int Dh,
                        const float* alpha, const float* beta, const float* mu, const float* s,
                        unsigned flags, void* o, int o_dtype, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * bam_fwd_skip_plan_offset - where a BAM_SKIP_FAR forward leaves its skipping plan.
 *
 * After bam_attn_fwd with these flags (which must include BAM_CAUSAL | BAM_SKIP_FAR), the
 * workspace holds, at byte *offset, *count = ceil(T / R) * B * H int32 values, R = 128
 * query rows per block for Dh = 128 and for Dh = 64 with T <= 1024, else R = 256.  Entry qb * B * H + b * H + h
 * is the number of leading 64-key tiles that query block qb of (b, h) left out.  For
 * measuring how much work the prior saved; the plan is rewritten by every such call.
 * Returns BAM_EUNSUPPORTED for flags without BAM_CAUSAL | BAM_SKIP_FAR or an unsupported Dh.
 */
bam_status bam_fwd_skip_plan_offset(int B, int H, int T, int Dh, unsigned flags, size_t* offset,
                                    int* count);

/*
 * bam_attn_decode - one new query row per sequence against a KV cache (split-KV).
 *
 * q: [B, H, Dh]; k_cache, v_cache: [B, H, Lmax, Dh] of in_dtype; kv_len: device
 * int32[B].  The cache already holds the current token, so the query of sequence b sits
 * at position i = kv_len[b] - 1 and sees keys 0 .. kv_len[b] - 1 (causal is implied;
 * n = kv_len[b] for SSMax).  o: [B, H, Dh] of o_dtype; lse: [B, H] float32.
 * flags: BAM_SSMAX, BAM_TABLE_READY and one of BAM_PRIOR_REF / BAM_PRIOR_SANDWICH;
 * BAM_CAUSAL is accepted and changes nothing (decode is causal by construction).
 * Supported: in_dtype BAM_BF16 with Dh in {32, 64, 128}.
 * The key range is cut into splits processed in parallel and merged exactly by their
 * log-sum-exp; the result does not depend on the split count beyond float rounding.
 */
size_t bam_decode_workspace_size(int B, int H, int Lmax, int Dh);
bam_status bam_attn_decode(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                           const int32_t* kv_len, int B, int H, int Lmax, int Dh,
                           const float* alpha, const float* beta, const float* mu, const float* s,
                           unsigned flags, void* o, int o_dtype, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * bam_decode_partials_layout - where a decode call on a workspace of
 * bam_decode_workspace_size(B, H, Lmax, Dh) bytes leaves its per-range partials: float32
 * records [B, H, nsplit, Dh + 2] = (m, l, o[Dh]) from byte *offset, key range s covering
 * keys s * chunk .. s * chunk + chunk - 1.  A range with no visible key, and a range that
 * bam_attn_decode_skip left out, has m = -inf.  BAM_EINVAL for unsupported sizes or NULL
 * outputs.
 */
bam_status bam_decode_partials_layout(int B, int H, int Lmax, int Dh, size_t* offset, int* nsplit, int* chunk);

/*
 * bam_decode_key_norms - per-page maxima of the key norms of a contiguous KV cache, the
 * companion array that bam_attn_decode_skip reads.  Pages are 64 keys: norms (device
 * float32, [B, H, bam_decode_norm_pages(Lmax)], caller-owned) receives, for page p of
 * (b, h), max |k_j|_2 over keys j in 64 p .. 64 p + 63 below Lmax, computed in float32 and
 * rounded up so that it is never below the exact norm.  k_cache: [B, H, Lmax, Dh] of
 * in_dtype (BAM_BF16; Dh in {32, 64, 128}), 16-byte aligned.  The array is kept beside
 * the cache: after keys of a page change, recompute it (this call recomputes every page)
 * before the next skipping decode; pages at or beyond kv_len are never read.
 */
int bam_decode_norm_pages(int Lmax);
bam_status bam_decode_key_norms(const void* k_cache, int in_dtype, int B, int H, int Lmax, int Dh, float* norms,
                                void* stream);

/*
 * bam_attn_decode_skip - bam_attn_decode that leaves out the key ranges whose weights are
 * zero in float32 ("Bayesian Attention Mechanism", "Highlights": retrieval far beyond the
 * training context, where a prior that decays with distance gives far keys no weight).
 * Arguments, flags, workspace and results are those of bam_attn_decode, plus key_norms
 * from bam_decode_key_norms for the same cache (required; BAM_EINVAL if NULL).
 * A first kernel takes the largest logit among the last 256 keys of each sequence, less a
 * rounding margin, as a lower bound M- of its largest logit.  Each key range (split) then
 * bounds its own logits from above, key by key, by c (b(i - j) + |q| |k|_page / sqrt(Dh))
 * (log2 units) and, when that bound is more than 160 below M-, stores the partial of a
 * range with no visible key instead of reading its K and V.  The full computation merges
 * such a range with weight 2^(m_s - M) < 2^-160, which is 0 in float32, so the outputs
 * are bit-for-bit those of bam_attn_decode on the same workspace layout.  The bounds
 * assume finite q, k and table entries; with key norms that no longer bound the cache
 * (stale after the cache changed) the result is undefined.
 */
bam_status bam_attn_decode_skip(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                                const int32_t* kv_len, int B, int H, int Lmax, int Dh,
                                const float* alpha, const float* beta, const float* mu, const float* s,
                                unsigned flags, const float* key_norms, void* o, int o_dtype, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * bam_attn_decode_static - bam_attn_decode with no workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It allocates nothing and calls no allocating routine:
 * the distance table and the split partials live in a static device buffer of
 * bam_decode_static_max_bytes() bytes (32 MiB) inside the library, of which each device
 * the library runs on holds its own copy until the process ends.  Requests whose
 * bam_decode_workspace_size() exceeds that return BAM_ETOOLARGE (the 256,000-token cache
 * with B = 8, H = 12, Dh = 64 needs 15.5 MB).  Arguments, flags and results are those of
 * bam_attn_decode (BAM_TABLE_READY refers to the table the previous static call on this
 * device left behind).  Every call on a device shares that buffer and its contents persist
 * between calls: calls that overlap on one device (concurrent streams or threads) race and
 * give undefined results.
 */
size_t bam_decode_static_max_bytes(void);
bam_status bam_attn_decode_static(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                                  const int32_t* kv_len, int B, int H, int Lmax, int Dh,
                                  const float* alpha, const float* beta, const float* mu, const float* s,
                                  unsigned flags, void* o, int o_dtype, float* lse, void* stream);

/*
 * bam_attn_decode_paged - bam_attn_decode on a paged KV cache.
 *
 * k_pages, v_pages: [num_pages, H, page_size, Dh] of in_dtype; block_table: device
 * int32[B, max_blocks], entry p of sequence b = the page holding its keys
 * p * page_size .. (p + 1) * page_size - 1.  kv_len as for bam_attn_decode, with
 * Lmax = max_blocks * page_size.  page_size must be a multiple of 64 (BAM_EUNSUPPORTED
 * otherwise).  Preconditions: 0 <= block_table entries < num_pages for the pages a
 * sequence uses (out-of-range ids are clamped, so a bad table gives wrong values but
 * never reads outside the pages).  Workspace: bam_decode_workspace_size(B, H,
 * max_blocks * page_size, Dh).  Same result as bam_attn_decode on the gathered cache.
 * Serving systems keep caches in pages so sequences of different lengths share one pool
 * ("Bayesian Attention Mechanism" README, "Highlights": decoding far beyond the
 * training context).
 */
bam_status bam_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, int in_dtype,
                                 const int32_t* block_table, int max_blocks, int num_pages, int page_size,
                                 const int32_t* kv_len, int B, int H, int Dh,
                                 const float* alpha, const float* beta, const float* mu, const float* s,
                                 unsigned flags, void* o, int o_dtype, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * bam_attn_bwd - backward of bam_attn_fwd for L = sum(O * dout).
 *
 * q, k, v, dout: [B, H, T, Dh] of in_dtype; o: the forward output, [B, H, T, Dh] of
 * o_dtype; lse: the forward's [B, H, T].  Same flags as the forward call.
 * dq, dk, dv: [B, H, T, Dh] of grad_dtype.  dalpha, dbeta, ds: device float32[H], the
 * gradients with respect to alpha_h, beta_h and s_h summed over batch, queries and keys
 * (ds is 0 without BAM_SSMAX).  With dP = dout V^T, D_i = sum_e dout_ie O_ie and
 * dZ = P * (dP - D) (the gradient with respect to the logits):
 *   dV = P^T dout,  dQ_i = c_i sum_j dZ_ij k_j / sqrt(Dh),  dK_j = sum_i c_i dZ_ij q_i / sqrt(Dh),
 *   dalpha = sum c_i dZ_ij db/dalpha,  dbeta = sum c_i dZ_ij db/dbeta,
 *   ds = sum dZ_ij ln(n_i) (q_i.k_j / sqrt(Dh) + b_ij).
 * With BAM_PRIOR_REF, dalpha and dbeta are the gradients in theta_alpha and theta_beta.
 * Supported: in_dtype BAM_BF16 with Dh in {32, 64}, T * Dh * 2 <= 2^31 - 1 and
 * 16 * B * H * (T rounded up to 64) <= 2^31 - 1 (the kernels address one head's Q / dO and
 * the per-row scalars with 32-bit byte ranges); BAM_EUNSUPPORTED otherwise.
 * Workspace (bam_bwd_workspace_size): the bias and derivative tables over the padded
 * distance range, four per-row fp32 scalars (D_i c_i / sqrt(Dh) among them) over rows
 * padded to 64, and the per-head partial sums; contents are scratch between calls.  For
 * T <= 512 and the alpha or reference prior the kernels compute the bias and its
 * derivatives themselves in float32 (within a few float32 ulps of the tables'
 * float64-derived values) and the tables are not written.
 */
size_t bam_bwd_workspace_size(int B, int H, int T, int Dh, unsigned flags);
bam_status bam_attn_bwd(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                        const float* lse, const void* dout, int in_dtype,
                        int B, int H, int T, int Dh,
                        const float* alpha, const float* beta, const float* mu, const float* s,
                        unsigned flags, void* dq, void* dk, void* dv, int grad_dtype,
                        float* dalpha, float* dbeta, float* ds,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * bam_attn_bwd_ex - bam_attn_bwd that also returns the gradient with respect to the
 * offset: dmu (device float32[H]) = sum c_i dZ_ij db/dmu (alpha-form) or the gradient in
 * theta_mu (BAM_PRIOR_REF), which the page's training code makes trainable on request.
 * dmu may be NULL (not computed; bam_attn_bwd is this call with dmu = NULL).  Same
 * workspace size as bam_attn_bwd.
 */
bam_status bam_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                           const float* lse, const void* dout, int in_dtype,
                           int B, int H, int T, int Dh,
                           const float* alpha, const float* beta, const float* mu, const float* s,
                           unsigned flags, void* dq, void* dk, void* dv, int grad_dtype,
                           float* dalpha, float* dbeta, float* dmu, float* ds,
                           void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BAM_H */
