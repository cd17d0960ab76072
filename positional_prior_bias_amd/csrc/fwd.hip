// BAM attention prefill forward for gfx950.
//
// Semantics ("ALiBi: Attention with Linear Biases", "Code"; "Résumé Technique :
// Mécanisme d'Attention Bayésienne (BAM)", "Solution Proposée : GGD-BAM"):
//   logit_ij = c_i (q_i.k_j / sqrt(Dh) + b_h(i - j)),  O = softmax_j(logit) V.
// Flash-style: one pass over key tiles with an online softmax in the exp2 domain;
// the exact result of the dense definition up to float rounding.
//
// bf16 kernel design (wave64):
//   * A work-group of 4 waves owns 256 query rows of one (b, h); each wave owns 64 rows as
//     two 32-row blocks that share every K and V^T operand read.  For Dh = 128, and for
//     Dh = 64 with short sequences (finer work-groups balance the causal triangle), a wave
//     owns one 32-row block and a work-group 128 rows.
//   * Key tiles of 64 go straight from HBM to LDS (buffer loads to LDS, issued from inline
//     assembly so the compiler does not make every LDS read wait for them), two tiles in
//     flight ahead of the one being computed (one for 128-row work-groups with Dh = 64), one
//     barrier per tile; rows at or beyond T load as zeros.
//   * S^T = K Q^T (v_mfma_f32_32x32x16_bf16) with keys as MFMA rows and queries as
//     columns: each lane owns one query and 16 keys per 32x32 block, so the row max / sum
//     of the softmax is an in-lane reduction plus one exchange with lane ^ 32.
//   * The bias enters as the MFMA accumulator's initial value: the accumulator is loaded
//     with sqrt(Dh) * b(i - j) from a window of the per-head distance table staged in LDS
//     (stored in reverse distance order, so a lane's values are read in register order),
//     and the MFMA returns q.k + sqrt(Dh) b directly.  Distances the causal mask forbids
//     hold -inf in that window, so masking is free as well.  Up to T = 512 (the training
//     context) a 128-row work-group computes the window entries of all its tiles itself,
//     into an LDS strip, while its first tile loads, and the call launches no table kernel.
//   * The running max of a row is exact, so every weight is at most 1 when it is rounded to
//     bf16 for the PV product (O and l are multiplied by the rescale factor every tile, by
//     1 when the max holds; this keeps the tile one basic block).
//   * O^T = V^T P^T on bf16 MFMA: P^T is fed from the S^T accumulators (rounded to bf16)
//     without any lane exchange (the contraction index runs over the keys in the order the
//     accumulator holds them); V^T comes from transposing LDS reads of the row-major tile.
//     l sums the unrounded fp32 weights, so lse carries fp32 rounding only.
//   * K / V rows in LDS have their 16-byte chunks XOR-swizzled by row so operand reads do
//     not collide in banks.
//   * With a skipping plan (causal only), a work-group starts its key loop at the first
//     key tile whose weights float32 can still hold (the bound is in skip.hip).
#include <float.h>
#include <type_traits>

#include "bam_device.h"
#include "bam_internal.h"
#include "prior_eval.h"

namespace bam {

namespace {

constexpr int kNK = 64;    // keys per tile

// Copies of the reversed distance window, copy c shifted by c entries, so every lane reads
// its runs of consecutive distances with aligned 16-byte (4 copies) or 8-byte (2 copies)
// loads.  Copies are a multiple of 32 floats plus 16 apart: copy c then starts at 16-byte
// bank group 4 c, and the 16 lanes of one LDS cycle (4 consecutive groups of 4 lanes, each
// lane group spanning the copies) hit distinct bank groups.
//
// With four copies every pipeline buffer holds its tile's whole window (TW entries per copy).
// With two copies the window lives in one ring shared by the buffers (kRing below): a tile's
// window is three 64-entry segments, consecutive tiles share two of them, so each tile adds
// one segment.  WN = floats of window per buffer (0 for the ring).
template <int DH, int WN>
struct FwdTile {
  uint16_t k[kNK * DH];
  uint16_t v[kNK * DH];
  float w[WN];
};
template <int DH>
struct FwdTile<DH, 0> {
  uint16_t k[kNK * DH];
  uint16_t v[kNK * DH];
};

// The ring: segment k of local tile t sits in slot (t + k) & 3 (64 entries each), and slots 0
// and 1 are mirrored after slot 3, so tile t's window is the 192 contiguous entries from
// 64 (t & 3).  Per copy 384 entries, copies kRingStride floats apart (400 = 12 * 32 + 16, so
// the two copies start on different banks).  The ring takes 3,200 bytes of LDS for the whole
// pipeline instead of a window per tile buffer; with two 16 KiB K / V buffers a work-group of
// 128 rows (Dh = 64) needs 35,968 bytes (37,120 in the CU's 1,280-byte allocation steps), so
// four fit in a CU's 160 KiB, and its 126 VGPRs allow four waves per SIMD.
constexpr int kRingEntries = 384;
constexpr int kRingStride = 400;
static_assert(kRingStride >= kRingEntries && kRingStride % 32 == 16, "ring copies overlap or share banks");

// The strip: with the bias computed in the kernel (bias_inkernel, T <= kFwdStripT), the
// work-group computes every window entry of all its tiles once, before its first tile:
// 64 (ntiles + 2) <= kStripEntries consecutive entries per copy, so tile t's window is the
// 192 entries from 64 t.  It shares the ring's LDS (whichever the launch uses); copies
// kStripStride floats apart (656 = 20 * 32 + 16) for the same bank spread.  The
// work-group's LDS grows to 38,016 bytes (38,400 allocated): four still fit in a CU.
constexpr int kStripEntries = 64 * (kFwdStripT / kNK + 2);
constexpr int kStripStride = 656;
static_assert(kStripStride >= kStripEntries && kStripStride % 32 == 16, "strip copies overlap or share banks");

// bf16 forward.  NQB = query blocks of 32 rows per wave (2 for Dh <= 64: the K and V^T
// operand reads from LDS are shared by both blocks; 1 for Dh = 128 to bound registers).
// SKIP: the launch carries a prior-aware skipping plan (causal only); a separate
// instantiation, so profiles tell skipping launches from full ones.
template <int DH, bool CAUSAL, int NQB, bool SKIP>
__global__ void __launch_bounds__(256, (DH == 64 && NQB == 1) ? 4 : 2) fwd_bf16_kernel(FwdArgs a, int nqb) {
  static_assert(CAUSAL || !SKIP, "skipping plans are causal only");
  constexpr int QW = 32 * NQB;          // query rows per wave
  constexpr int MQ = 4 * QW;            // query rows per work-group
  constexpr int TW = MQ + kNK;          // distance-window entries per tile (multiple of 64)
  constexpr int KCH = DH / 8;           // 16-byte chunks per K / V row
  constexpr int KS = DH / 16;           // MFMA k-steps over the head dimension
  constexpr int DB = DH / 32;           // 32-row blocks of O^T
  constexpr int CPW = kNK * KCH / 256;  // 1 KiB direct loads per wave per tensor
  // Copies of the window: 4 (each lane's runs of 4 distances are one 16-byte read); 2 for
  // Dh = 64 with one query block per wave (8-byte reads), which keeps the work-group's LDS
  // under a quarter of the CU's so four work-groups (four waves per SIMD) fit.
  constexpr int NCOPY = (DH == 64 && NQB == 1) ? 2 : 4;
  constexpr bool RING = NCOPY == 2;               // two copies: the window is the shared ring
  static_assert(!RING || TW == 192, "the ring holds windows of three 64-entry segments");
  // Four copies: the window lives in an eight-slot ring of 64-entry segments per copy (a
  // tile's TW / 64 segments, consecutive tiles sharing all but one), slots 0 .. NSEG - 2
  // mirrored after slot 7 so every window is contiguous.  Each tile adds one segment per
  // copy: wave w loads copy w's, and its mirror (or the segment again where the slot has
  // none), so every wave issues two window loads per tile.
  constexpr int NSEG = TW / 64;
  constexpr int R4STRIDE = 64 * (8 + NSEG - 1) + 16;   // floats between copies (16 mod 64: 4c bank groups apart)
  static_assert(RING || NSEG + 2 <= 8, "three tiles in flight must fit the eight slots");
  static_assert(R4STRIDE % 64 == 16, "ring copies share banks");
  constexpr int WPW = RING ? 1 : 2;     // window loads per wave per tile
  constexpr int KVL = 2 * CPW;          // K / V direct loads per wave per tile
  constexpr int LPT = KVL + WPW;        // direct-load instructions per wave per tile
  // Two 32-row blocks per wave: each block of MFMAs is issued at raised wave priority, so
  // a wave with matrix work ready goes ahead of the other wave's softmax (about 4% at
  // T = 32768; neutral for one block per wave, where it is left out).
  constexpr bool MFMA_PRIO = NQB == 2;
  static_assert(kNK * KCH % 256 == 0, "tile must split into 1 KiB wave loads");
  static_assert(LPT < 64, "vmcnt range");

  // the buffers as distinct objects: the tile being read, and one (ring) or two being filled
  using Tile = FwdTile<DH, 0>;
  __shared__ __attribute__((aligned(16))) Tile tA, tB;
  typedef typename std::conditional<RING, uint32_t[4], Tile>::type ThirdTile;   // unused with the ring
  __shared__ __attribute__((aligned(16))) ThirdTile tCst;
  Tile& tC = *reinterpret_cast<Tile*>(&tCst);
  // the two-copy ring or strip, or the four-copy ring
  __shared__ __attribute__((aligned(16))) float wring[RING ? NCOPY * kStripStride : NCOPY * R4STRIDE];

  const int BH = a.B * a.H;
  // Work-group i runs on XCD i % 8 (one L2 each).  With B * H a multiple of 8 every query
  // block of a head lands on that head's XCD, so the blocks of a head running together
  // share its K / V tiles in one L2 (spread over four XCDs, they fetched 36% more at T = 512).
  const int bid = blockIdx.x;
  int qb = bid / BH;
  const int bh = bid - qb * BH;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
  const int h = bh % a.H;
  const int T = a.T;
  const size_t base = (size_t)bh * T * DH;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q + base;
  const uint16_t* __restrict__ K = (const uint16_t*)a.k + base;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v + base;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31;
  const int hh = lane >> 5;
  const int i0 = qb * MQ;
  const int iw = i0 + wave * QW;        // first query row of this wave

  // Q^T operands: lane holds q_i[16 ks + 8 hh .. + 7] of its query in each block
  bf16x8 qf[NQB][KS];
  float Cl[NQB], m[NQB], mu[NQB], l[NQB];
  const float sqrtD = __builtin_sqrtf((float)DH);
  const float sh = a.ssmax ? a.s[h] : 1.0f;
  u32x4 qw[NQB][KS];
#pragma unroll
  for (int qb2 = 0; qb2 < NQB; ++qb2) {
    const int i = iw + 32 * qb2 + ql;
    const float c = ssmax_c(a.ssmax, sh, CAUSAL ? i + 1 : T);
    // logit in log2 units = Cl * (q.k + sqrt(Dh) b); c = 0 only when one key is visible
    Cl[qb2] = fmaxf(c * kLog2e / sqrtD, FLT_MIN);
    m[qb2] = kNegInf;
    mu[qb2] = 0.f;
    l[qb2] = 0.f;
  }
  f32x16 oacc[NQB][DB];
#pragma unroll
  for (int qb2 = 0; qb2 < NQB; ++qb2)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int x = 0; x < 16; ++x) oacc[qb2][db][x] = 0.f;

  const int kend = CAUSAL ? min(T, i0 + MQ) : T;
  // key tiles before tf carry no weight float32 can hold (prior-aware plan; causal only)
  int tf = 0;
  if (SKIP && a.first_tile)
    tf = min(max(__builtin_amdgcn_readfirstlane(a.first_tile[qb * BH + bh]), 0), i0 / kNK);
  const int jb = tf * kNK;                          // first key of the loop
  const int ntiles = (kend - jb + kNK - 1) / kNK;   // tiles from jb on
  const float* tabh = a.tab + (size_t)h * a.tab_stride;

  // window value index y of this lane's first accumulator group; the four values of each
  // group are consecutive, read with one 16-byte load from copy (y & 3)
  const int ybase = (MQ - 1) - (QW * wave + ql) + 4 * hh;   // + 32 (kb - qb2) + 8 g
  const int wcopy = ybase & (NCOPY - 1);

  // ---- issue the direct loads of key tile j0.  Chunk position p of K / V holds global
  // chunk (row, (p % KCH) ^ swizzle(row)).  Buffer loads: the per-lane part of each address
  // is a fixed VGPR offset; rows at or beyond T lie outside the K / V buffer ranges and load
  // as zeros (those keys are masked by the table or explicitly).  Every wave issues LPT loads.
  const i32x4 rK = buffer_rsrc(K, (uint32_t)T * DH * 2);
  const i32x4 rV = buffer_rsrc(V, (uint32_t)T * DH * 2);
  const i32x4 rW = buffer_rsrc(tabh, (uint32_t)a.tab_stride * 4);
  // Lane id; in the 128-row kernel read by inline assembly, which the compiler cannot hoist,
  // so the values derived from it (the ring window's offsets, the epilogue's indices) are
  // recomputed where they are used instead of held in registers across the loop.
  auto issue_lane = [&]() {
    int ln = lane;
    if constexpr (NQB == 1) asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    return ln;
  };
  auto kv_voff = [&](int r) {
    const unsigned p = (unsigned)((wave * CPW + r) * 64) + (unsigned)issue_lane();
    const unsigned row = p / KCH;
    return (int)((row * DH + ((p % KCH) ^ (unsigned)vswz<DH>((int)row)) * 8) * 2);
  };
  // Per-lane byte offsets of the K / V direct loads, computed once (unsigned: no rounding
  // fix-up for a negative quotient).  Two registers; recomputing them at each issue cost
  // about 17 VALU instructions per load pair.
  int kvo[CPW];
#pragma unroll
  for (int r = 0; r < CPW; ++r) kvo[r] = kv_voff(r);
  // Four-copy ring: segment g (entries from tile 0's window start + 64 g) of copy wave into
  // slot g & 7, and into its mirror where mirror is set and the slot has one (else the slot
  // again: the same bytes to the same place).
  const int u0_first = a.tab_d0 - (i0 + MQ - 1 - jb);   // tile 0's window start in the reversed table
  auto ring4_load = [&](int g, bool mirror) {
    const int slot = g & 7;
    const int pos = (mirror && slot < NSEG - 1) ? 64 * (8 + slot) : 64 * slot;
    lds_dma4(rW, lane * 4, (u0_first + wave + 64 * g) * 4, &wring[wave * R4STRIDE + pos]);
  };
  // the direct loads of local tile t: its K and V, and (four copies) the segment it adds
  auto issue_tile = [&](Tile& tl, int t) {
    const int j0 = jb + t * kNK;
#pragma unroll
    for (int r = 0; r < CPW; ++r) {
      const int p0 = (wave * CPW + r) * 64;
      const int vo = kvo[r] + j0 * DH * 2;
      lds_dma16(rK, vo, 0, &tl.k[p0 * 8]);
      lds_dma16(rV, vo, 0, &tl.v[p0 * 8]);
    }
    if constexpr (!RING) {
      ring4_load(t + NSEG - 1, false);
      ring4_load(t + NSEG - 1, true);
    }
  };
  // Ring segment k of local tile t (entries from the window start + 64 k) into slot
  // (t + k) & 3 of copy cpy, and into its mirror if mirror is set and the slot is 0 or 1.
  // A wave asked for a mirror that does not exist reloads the slot itself (the same bytes to
  // the same place), so every wave issues the same number of loads.
  auto ring_load = [&](int t, int k, int cpy, bool mirror) {
    const int u0 = a.tab_d0 - (i0 + MQ - 1 - (jb + t * kNK));
    const int slot = (t + k) & 3;
    const int pos = (mirror && slot < 2) ? 256 + 64 * slot : 64 * slot;
    lds_dma4(rW, issue_lane() * 4, (u0 + cpy + 64 * k) * 4, &wring[cpy * kRingStride + pos]);
  };
  // The strip (bias_inkernel): entry x of copy c is table entry u0 + c + x, u0 that of
  // tile 0, that is sqrt(Dh) times the bias at distance tab_d0 - u0 - c - x, computed in
  // float32 (prior_bias_f32: within a few ulps of the table's float64-derived value).
  // Thread l computes table entries u0 + l, u0 + l + 256, ... once and stores each in both
  // copies.  That takes the distance-table launch out of the forward call.
  float pa = 0.f, pb = 0.f, pm = 0.f;   // the head's parameters (scalar loads in the prologue)
  auto fill_strip = [&]() {
    const int u0 = a.tab_d0 - (i0 + MQ - 1 - jb);
    const float sc = __builtin_sqrtf((float)DH);
    for (int x = tid; x <= kStripEntries; x += 256) {
      const int d = a.tab_d0 - (u0 + x);
      const float b = (d >= a.dlo && d <= a.dhi) ? prior_bias_f32(a.kind, pa, pb, pm, d) * sc : kNegInf;
      if (x < kStripEntries) wring[x] = b;
      if (x >= 1) wring[kStripStride + x - 1] = b;
    }
  };
  // the segment tile t adds (k = 2): one load per wave (copy wave & 1, mirror wave >> 1)
  auto ring_next = [&](int t) { ring_load(t, 2, wave & 1, wave >> 1); };

  // Dh = 64: per-lane LDS byte offsets of the K and V^T operand reads, fixed for the whole
  // kernel.  V^T operand rows r0 = 16 st + rb and r1 = r0 + 8, column 32 db + cq: the row
  // swizzle of rb + 16 st does not depend on st and that of r1 is that of r0 with bit 2
  // flipped, so the four (db, r0 / r1) combinations use two offsets, vA and vB, plus
  // immediates.  K operand row 32 kb + ql: the swizzle does not depend on kb.
  int vA = 0, vB = 0, kOff[KS];
  if constexpr (DH == 64) {
    const int G = lane >> 4, gi = lane & 15;
    const int rb = 4 * (G >> 1) + (gi >> 2);
    const int ch0 = (2 * (G & 1) + ((gi & 3) >> 1)) ^ vswz<DH>(rb);
    vA = 128 * rb + 16 * ch0 + 8 * (gi & 1);
    vB = 128 * rb + 16 * (ch0 ^ 4) + 8 * (gi & 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kOff[ks] = 128 * ql + 16 * ((2 * ks + hh) ^ vswz<DH>(ql));
  }

  // Before the barrier that publishes tile t + 1, each wave waits for its own loads of it
  // (tile t + 2's may stay in flight).
  auto wait_next = [&](int t) {
    if (t + 1 >= ntiles) return;
    if constexpr (RING) {
      BAM_WAIT_VMCNT(0);          // two stages: only tile t + 1's loads are in flight
    } else {
      if (t + 2 < ntiles) BAM_WAIT_VMCNT(LPT);   // tile t + 2's stay in flight
      else BAM_WAIT_VMCNT(0);
    }
  };

  auto compute_tile = [&](const Tile& tl, int t) {
    const int j0 = jb + t * kNK;
    // A wave whose rows all precede this tile's keys has nothing to do (causal).  Without
    // the mask the second test never holds (tiles end before T), but the branch splits the
    // tile into its own scheduling region: as one region with the loop around it, the
    // compiler's schedule needs more than the 256 registers of two waves per SIMD.
    if ((CAUSAL && j0 > iw + QW - 1) || (!CAUSAL && j0 >= T)) {
      wait_next(t);
      return;
    }
    // ---- S'^T = K Q^T + sqrt(Dh) b: each accumulator starts from its bias block (read
    // straight into the accumulator registers), then accumulates the contraction.  All
    // LDS reads of the phase are issued before the first MFMA so their latency overlaps.
    f32x16 sacc[NQB][2];
    u32x4 kw[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int qb2 = 0; qb2 < NQB; ++qb2) {
        if constexpr (NCOPY == 4) {
          const f32x4* __restrict__ wv = (const f32x4*)&wring[wcopy * R4STRIDE + 64 * (t & 7)];
          const int y4 = ((ybase - wcopy) >> 2) + 8 * (kb - qb2);   // 16-byte units
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v4 = wv[y4 + 2 * g];
            sacc[qb2][kb][4 * g + 0] = v4[0];
            sacc[qb2][kb][4 * g + 1] = v4[1];
            sacc[qb2][kb][4 * g + 2] = v4[2];
            sacc[qb2][kb][4 * g + 3] = v4[3];
          }
        } else {
          const f32x2* __restrict__ wv = (const f32x2*)&wring[a.bias_inkernel ? wcopy * kStripStride + 64 * t
                                                                               : wcopy * kRingStride + 64 * (t & 3)];
          const int y2 = ((ybase - wcopy) >> 1) + 16 * (kb - qb2);   // 8-byte units
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x2 lo = wv[y2 + 4 * g], hi = wv[y2 + 4 * g + 1];
            sacc[qb2][kb][4 * g + 0] = lo[0];
            sacc[qb2][kb][4 * g + 1] = lo[1];
            sacc[qb2][kb][4 * g + 2] = hi[0];
            sacc[qb2][kb][4 * g + 3] = hi[1];
          }
        }
      }
      if constexpr (DH == 64) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kw[kb][ks] = *(const u32x4*)((const char*)tl.k + kOff[ks] + 4096 * kb);
      } else {
        const int r = 32 * kb + ql;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kw[kb][ks] = *(const u32x4*)(&tl.k[r * DH + ((2 * ks + hh) ^ vswz<DH>(r)) * 8]);
      }
    }
    if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int qb2 = 0; qb2 < NQB; ++qb2)
          sacc[qb2][kb] = mfma32x32x16(as_bf16x8(kw[kb][ks]), qf[qb2][ks], sacc[qb2][kb]);
    if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(0);
    if (!CAUSAL && j0 + kNK > T) {
#pragma unroll
      for (int qb2 = 0; qb2 < NQB; ++qb2)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int kl = 32 * kb + 8 * (x >> 2) + 4 * hh + (x & 3);
            if (j0 + kl >= T) sacc[qb2][kb][x] = kNegInf;
          }
    }

    // ---- online softmax (exp2 domain) with an exact running max
    u32x4 pf[NQB][4];
#pragma unroll
    for (int qb2 = 0; qb2 < NQB; ++qb2) {
      // the 32 values of the lane as a tree of three-input maxima: 16 instructions
      float v[32], t1[11], t2[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) v[16 * kb + x] = sacc[qb2][kb][x];
#pragma unroll
      for (int i = 0; i < 10; ++i) t1[i] = max3(v[3 * i], v[3 * i + 1], v[3 * i + 2]);
      t1[10] = __builtin_fmaxf(v[30], v[31]);
#pragma unroll
      for (int i = 0; i < 3; ++i) t2[i] = max3(t1[3 * i], t1[3 * i + 1], t1[3 * i + 2]);
      t2[3] = max3(t1[9], t1[10], t2[2]);
      const float mx = max_xor32(max3(t2[0], t2[1], t2[3]));
      // The running max is exact (not lazy): the largest weight computed so far is then
      // exactly 1 and every weight is at most 1, so rounding P to bf16 perturbs each weight
      // by at most 2^-8 of itself.  (A lazy max that moved only on jumps of 2^8 let the
      // dominant weight reach 2^8 and round; O's error then reached 2^-9 max|V|.)  O and
      // l are multiplied by the factor every tile, 1 when the max holds: a branch around
      // the multiply made the compiler copy all of O on every tile to merge the two paths.
      //
      // The weights are exp2(fma(Cl, s, -mu)) with mu the exponent reference of the row.  The
      // running max m = round(Cl * max s) differs from the exact product by up to half an
      // ulp of m, which is large when a tile of far keys carries a huge bias (at
      // |m| = 2^34 the max element's exponent could reach +2^9 and its weight overflow).
      // mu = m + 2^-22 |m| lies above every exact product, so every weight is at most 1 at
      // any magnitude; below |m| = 2^13 the dominant weight still rounds to exactly 1.
      const float m_new = fmaxf(m[qb2], Cl[qb2] * mx);
      const float mu_new = (m_new == kNegInf) ? 0.f : fmaf(fabsf(m_new), 0x1p-22f, m_new);
      const float sc = (m[qb2] == kNegInf) ? 0.f : exp2_fast(mu[qb2] - mu_new);
      m[qb2] = m_new;
      mu[qb2] = mu_new;
      l[qb2] *= sc;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) oacc[qb2][db][x] *= sc;
      const float m_use = mu_new;
      // P is rounded to bf16 for the PV product; l sums the unrounded fp32 weights, so lse
      // carries only fp32 rounding and O's error is that of the bf16 weights alone.
      // (the tile's weights are summed from zero, then added to l: accumulated one by one
      // onto a running l near 1, tiny tail weights would each round by a fixed bias)
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; x += 2) {
          const float p0 = exp2_fast(fmaf(Cl[qb2], sacc[qb2][kb][x], -m_use));
          const float p1 = exp2_fast(fmaf(Cl[qb2], sacc[qb2][kb][x + 1], -m_use));
          pf[qb2][2 * kb + (x >> 3)][(x & 7) >> 1] = pack_bf16x2(p0, p1);
          // the first pair starts the sum (0 + y is not folded away for a float y)
          ls = (kb == 0 && x == 0) ? p0 + p1 : ls + (p0 + p1);
        }
      l[qb2] += ls;
    }

    // In the 128-row kernel the wait for the next tile's loads comes after the PV product,
    // which gives the loads a whole tile of lead time.
    if constexpr (NQB != 1) wait_next(t);
    // (128-row kernel: without this scheduling barrier the compiler hoists PV operand reads
    // into the softmax and exceeds the 128 VGPRs of four waves per SIMD)
    if constexpr (NQB == 1) __builtin_amdgcn_sched_barrier(0);

    // ---- O^T += V^T P^T (bf16).  The V^T operand of lane (dh, hh) holds keys
    // {16 st + 4 hh + 0..3, + 8 .. + 11} of column dh: two transposing reads of the
    // row-major V tile (lane i of 16-lane group G reads row key0 + i / 4, columns
    // dh0 + 4 (i % 4) .. + 3, dh0 = 32 db + 16 (G % 2)).
    const int G = lane >> 4, gi = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + 16 * (G & 1) + 4 * (gi & 3);
      bf16x8 av[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        s16x4 v0, v1;
        if constexpr (DH == 64) {
          const char* tv = (const char*)tl.v;
          v0 = lds_read_tr16((const uint16_t*)(tv + (db ? vB : vA) + 2048 * st));
          v1 = lds_read_tr16((const uint16_t*)(tv + (db ? vA : vB) + 2048 * st + 1024));
        } else {
          const int r0 = 16 * st + 4 * (G >> 1) + (gi >> 2);
          const int r1 = r0 + 8;
          v0 = lds_read_tr16(&tl.v[r0 * DH + (((col >> 3) ^ vswz<DH>(r0)) << 3) + (col & 7)]);
          v1 = lds_read_tr16(&tl.v[r1 * DH + (((col >> 3) ^ vswz<DH>(r1)) << 3) + (col & 7)]);
        }
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        av[st] = __builtin_bit_cast(bf16x8, vv);
      }
      if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int qb2 = 0; qb2 < NQB; ++qb2)
          oacc[qb2][db] = mfma32x32x16(av[st], as_bf16x8(pf[qb2][st]), oacc[qb2][db]);
      if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (NQB == 1) wait_next(t);
  };

  // ---- pipeline prologue.  Q must be in registers before any later tile load is issued
  // (the compiler would otherwise wait for it, and so for every load in flight, inside the
  // loop).  Q is loaded after tile 0 with buffer loads the compiler does not track (rows at
  // or beyond T load as zeros); with three stages tile 1 follows, so one wait covers tile 0
  // and Q and tile 1 stays in flight.  The empty asm statements after the wait make Q's
  // registers defined there.
  // With the ring, tile 0's window (segments 0 .. 2 of both copies and the mirrors of slots
  // 0 and 1: ten loads, three per wave, the surplus repeating) goes first; each later tile's
  // segment is issued one tile ahead, after the barrier that frees its slot.  The strip is
  // computed while tile 0 and Q load.
  BAM_WAIT_VMCNT(0);
  if (RING && !a.bias_inkernel) {
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int x = (wave * 3 + r) % 10;
      const int idx = x % 5;
      ring_load(0, idx < 3 ? idx : idx - 3, x / 5, idx >= 3);
    }
  }
  if constexpr (!RING) {   // tile 0's window but its last segment (which issue_tile adds)
#pragma unroll
    for (int g = 0; g < NSEG - 1; ++g) {
      ring4_load(g, false);
      ring4_load(g, true);
    }
  }
  issue_tile(tA, 0);
  {
    const i32x4 rQ = buffer_rsrc(Q, (uint32_t)T * DH * 2);
#pragma unroll
    for (int qb2 = 0; qb2 < NQB; ++qb2) {
      const int i = iw + 32 * qb2 + ql;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t off = (uint32_t)(i * DH + 16 * ks + 8 * hh) * 2u;
        asm volatile(BAM_VMEM_SGPR_NOPS "buffer_load_dwordx4 %0, %1, %2, 0 offen"
                     : "=v"(qw[qb2][ks]) : "v"(off), "s"(rQ) : "memory");
      }
    }
  }
  if (RING && a.bias_inkernel) {
    // scalar loads, issued after tile 0's and Q's: the wait for them (lgkmcnt) leaves those
    // in flight
    pa = uniform_load(a.alpha + h);
    pb = uniform_load(a.beta + h);
    pm = a.mu ? uniform_load(a.mu + h) : 0.f;
    fill_strip();
  }
  if (!RING && ntiles > 1) {
    issue_tile(tB, 1);
    BAM_WAIT_VMCNT(LPT);       // tile 0 and Q landed (tile 1 may be in flight)
  } else {
    BAM_WAIT_VMCNT(0);
  }
#pragma unroll
  for (int qb2 = 0; qb2 < NQB; ++qb2)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      asm volatile("" : "+v"(qw[qb2][ks]));
      qf[qb2][ks] = as_bf16x8(qw[qb2][ks]);
    }
  BAM_BARRIER_VMCNT(63);       // publish tile 0
  // every wave has waited for its loads of tile t + 1 (in compute_tile); publish it
  auto advance = [&]() { BAM_BARRIER_VMCNT(63); };
  if constexpr (RING) {
    // Two stages: tile t + 1 and its ring segment (whose slot held tile t - 1's first
    // segment) load while tile t is computed.  With three or more waves per SIMD, and the keys of a
    // short sequence mostly in L2, one tile of lead time is enough; it was 2% faster than
    // three stages at T = 512 and halves the buffers.  The strip needs no loads.
    const bool ring = !a.bias_inkernel;
    for (int t = 0; t < ntiles; t += 2) {
      if (t + 1 < ntiles) {
        if (ring) ring_next(t + 1);
        issue_tile(tB, t + 1);
      }
      compute_tile(tA, t);
      advance();
      if (t + 1 >= ntiles) break;
      if (t + 2 < ntiles) {
        if (ring) ring_next(t + 2);
        issue_tile(tA, t + 2);
      }
      compute_tile(tB, t + 1);
      advance();
    }
  } else {
    // Three stages: tile t is computed while tiles t + 1 and t + 2 load, from buffer t % 3.
    // Two tiles per iteration, the buffers picked at run time: the compiler keeps O in two
    // register sets that alternate from tile to tile, so a three-tile body (one per buffer)
    // ended with O in the other set and 32 64-bit moves to bring it back; a two-tile body
    // ends where it began.
    auto buf = [&](int t) -> Tile& {
      const int r = t % 3;
      return r == 0 ? tA : (r == 1 ? tB : tC);
    };
    for (int t = 0; t < ntiles; t += 2) {
      if (t + 2 < ntiles) issue_tile(buf(t + 2), t + 2);
      compute_tile(buf(t), t);
      advance();
      if (t + 1 >= ntiles) break;
      if (t + 3 < ntiles) issue_tile(buf(t + 3), t + 3);
      compute_tile(buf(t + 1), t + 1);
      advance();
    }
  }

  // ---- epilogue (the lane's query and half are recomputed here in the 128-row kernel, for
  // the same reason as the load offsets)
  const int eln = issue_lane();
  const int eql = eln & 31, ehh = eln >> 5;
#pragma unroll
  for (int qb2 = 0; qb2 < NQB; ++qb2) {
    const int i = iw + 32 * qb2 + eql;
    const float lt = l[qb2] + xor32(l[qb2]);
    if (i < T) {
      const float inv = 1.0f / lt;
      const size_t orow = base + (size_t)i * DH;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dh0 = 32 * db + 8 * g + 4 * ehh;
          const float o0 = oacc[qb2][db][4 * g + 0] * inv, o1 = oacc[qb2][db][4 * g + 1] * inv;
          const float o2 = oacc[qb2][db][4 * g + 2] * inv, o3 = oacc[qb2][db][4 * g + 3] * inv;
          if (a.o_f32) {
            f32x4 w = {o0, o1, o2, o3};
            *(f32x4*)((float*)a.o + orow + dh0) = w;
          } else {
            u32x2 w = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
            *(u32x2*)((uint16_t*)a.o + orow + dh0) = w;
          }
        }
      if (ehh == 0) a.lse[(size_t)bh * T + i] = (mu[qb2] + __log2f(lt)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------------------------
// fp32 path: one query row per lane, keys and values broadcast from LDS, fp32 FMA.
// ------------------------------------------------------------------------------------
constexpr int kMQ32 = 64;
constexpr int kNK32 = 64;

template <int DH, bool CAUSAL>
__global__ void __launch_bounds__(64) fwd_f32_kernel(FwdArgs a, int nqb) {
  __shared__ __attribute__((aligned(16))) float Ks[kNK32 * DH];
  __shared__ __attribute__((aligned(16))) float Vs[kNK32 * DH];
  __shared__ float tw[kMQ32 + kNK32];
  // the lane's scores of one key tile, column `lane` (a register array indexed in a
  // partially unrolled loop would live in scratch memory)
  __shared__ float scs[kNK32 * kMQ32];

  const int BH = a.B * a.H;
  int qb = blockIdx.x / BH;
  const int bh = blockIdx.x - qb * BH;
  if (CAUSAL) qb = nqb - 1 - qb;
  const int h = bh % a.H;
  const int T = a.T;
  const size_t base = (size_t)bh * T * DH;
  const float* __restrict__ Q = (const float*)a.q + base;
  const float* __restrict__ K = (const float*)a.k + base;
  const float* __restrict__ V = (const float*)a.v + base;
  const int lane = threadIdx.x;
  const int i0 = qb * kMQ32;
  const int i = i0 + lane;

  float qr[DH];
#pragma unroll
  for (int e = 0; e < DH; e += 4) {
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (i < T) w = *(const f32x4*)(Q + (size_t)i * DH + e);
    qr[e] = w[0]; qr[e + 1] = w[1]; qr[e + 2] = w[2]; qr[e + 3] = w[3];
  }
  const int n_i = CAUSAL ? i + 1 : T;
  const float c = ssmax_c(a.ssmax, a.ssmax ? a.s[h] : 1.0f, n_i);
  const float Cs = fmaxf(c * kLog2e / __builtin_sqrtf((float)DH), FLT_MIN);
  const float Cb = fmaxf(c * kLog2e, FLT_MIN);

  float o[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) o[e] = 0.f;
  float m = kNegInf, l = 0.f;
  const int kend = CAUSAL ? min(T, i0 + kMQ32) : T;
  const float* __restrict__ tabh = a.tab + (size_t)h * a.tab_stride;
  const int dlo = CAUSAL ? 0 : -(T - 1);
  const int dhi = T - 1;

  for (int j0 = 0; j0 < kend; j0 += kNK32) {
    __syncthreads();
    for (int x = lane; x < kNK32 * DH / 4; x += 64) {
      const int r = (4 * x) / DH;
      f32x4 kw = {0.f, 0.f, 0.f, 0.f}, vw = {0.f, 0.f, 0.f, 0.f};
      if (j0 + r < T) {
        kw = *(const f32x4*)(K + (size_t)j0 * DH + 4 * x);
        vw = *(const f32x4*)(V + (size_t)j0 * DH + 4 * x);
      }
      *(f32x4*)(Ks + 4 * x) = kw;
      *(f32x4*)(Vs + 4 * x) = vw;
    }
    const int d_min = i0 - j0 - (kNK32 - 1);
    for (int x = lane; x < kMQ32 + kNK32; x += 64) {
      const int d = d_min + x;
      tw[x] = (d >= dlo && d <= dhi) ? tabh[d - a.tab_d0] : kNegInf;
    }
    __syncthreads();
    const int nk = min(kNK32, kend - j0);
    float mx = kNegInf;
#pragma unroll 4
    for (int jj = 0; jj < kNK32; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DH; ++e) dot = fmaf(qr[e], Ks[jj * DH + e], dot);
      const float bv = tw[lane + (kNK32 - 1) - jj];
      float t = fmaf(Cs, dot, Cb * bv);
      if (jj >= nk || bv == kNegInf) t = kNegInf;
      scs[jj * kMQ32 + lane] = t;
      mx = fmaxf(mx, t);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float s0 = exp2_fast(m - m_use);
    m = m_new;
    l *= s0;
#pragma unroll
    for (int e = 0; e < DH; ++e) o[e] *= s0;
#pragma unroll 2
    for (int jj = 0; jj < kNK32; ++jj) {
      const float p = exp2_fast(scs[jj * kMQ32 + lane] - m_use);
      l += p;
#pragma unroll
      for (int e = 0; e < DH; ++e) o[e] = fmaf(p, Vs[jj * DH + e], o[e]);
    }
  }
  if (i < T) {
    const float inv = 1.0f / l;
    const size_t orow = base + (size_t)i * DH;
#pragma unroll
    for (int e = 0; e < DH; e += 4) {
      const float o0 = o[e] * inv, o1 = o[e + 1] * inv, o2 = o[e + 2] * inv, o3 = o[e + 3] * inv;
      if (a.o_f32) {
        f32x4 w = {o0, o1, o2, o3};
        *(f32x4*)((float*)a.o + orow + e) = w;
      } else {
        u32x2 w = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        *(u32x2*)((uint16_t*)a.o + orow + e) = w;
      }
    }
    a.lse[(size_t)bh * T + i] = (m + __log2f(l)) * kLn2;
  }
}

template <int DH, bool CAUSAL, int NQB>
hipError_t launch_bf16_nqb(const FwdArgs& a, hipStream_t stream) {
  constexpr int MQ = 4 * 32 * NQB;
  const int nqb = (a.T + MQ - 1) / MQ;
  const long nblocks = (long)nqb * a.B * a.H;
  if constexpr (CAUSAL) {
    if (a.first_tile != nullptr) {
      hipLaunchKernelGGL((fwd_bf16_kernel<DH, CAUSAL, NQB, true>), dim3((unsigned)nblocks), dim3(256), 0, stream, a,
                         nqb);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<DH, CAUSAL, NQB, false>), dim3((unsigned)nblocks), dim3(256), 0, stream, a, nqb);
  return hipGetLastError();
}

template <int DH, bool CAUSAL>
hipError_t launch_bf16_t(const FwdArgs& a, hipStream_t stream) {
  if constexpr (DH == 128) {
    return launch_bf16_nqb<DH, CAUSAL, 1>(a, stream);
  } else if constexpr (DH == 64) {
    if (fwd_bf16_rows_per_block(DH, a.T) == 128) return launch_bf16_nqb<DH, CAUSAL, 1>(a, stream);
    return launch_bf16_nqb<DH, CAUSAL, 2>(a, stream);
  } else {
    return launch_bf16_nqb<DH, CAUSAL, 2>(a, stream);
  }
}

template <int DH, bool CAUSAL>
hipError_t launch_f32_t(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.T + kMQ32 - 1) / kMQ32;
  const long nblocks = (long)nqb * a.B * a.H;
  hipLaunchKernelGGL((fwd_f32_kernel<DH, CAUSAL>), dim3((unsigned)nblocks), dim3(64), 0, stream, a, nqb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int Dh, hipStream_t stream) {
  switch (Dh) {
    case 32: return a.causal ? launch_bf16_t<32, true>(a, stream) : launch_bf16_t<32, false>(a, stream);
    case 64: return a.causal ? launch_bf16_t<64, true>(a, stream) : launch_bf16_t<64, false>(a, stream);
    case 128: return a.causal ? launch_bf16_t<128, true>(a, stream) : launch_bf16_t<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_f32(const FwdArgs& a, int Dh, hipStream_t stream) {
  switch (Dh) {
    case 32: return a.causal ? launch_f32_t<32, true>(a, stream) : launch_f32_t<32, false>(a, stream);
    case 64: return a.causal ? launch_f32_t<64, true>(a, stream) : launch_f32_t<64, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bam
