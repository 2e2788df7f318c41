// gfx950 (CDNA4) kernels of the linear-memory relation-KL path, bf16 inputs.
//
// Method: "LinearARD: Linear-Memory Attention Distillation for RoPE
// Restoration" (paper-notes page, section "Key designs", items 1 and 3;
// summary page, section "Method").  Phase 1 streams key tiles and keeps only
// the per-row log-sum-exp of the teacher and student logits.  Phase 2
// recomputes the logit tiles on chip, rebuilds both probability tiles from
// the stored statistics, accumulates the row KL and forms the logit gradient
// dZ = (R_s - R_t)/n, which it contracts with the student projections.
//
// Tiling used by every sweep kernel in this file
//   * A workgroup of NW waves owns 32*NW consecutive rows of one head; wave w
//     owns 32 of them.  The owned rows' projections sit in registers as MFMA
//     B operands for the whole sweep.
//   * The other index ("swept") advances in tiles of SW rows (128 by
//     default) that are copied global -> LDS directly (no staging
//     registers), double-buffered, one barrier per tile, the copy split over
//     the NW waves.  Each tile is processed in 32-row blocks.
//   * Logit tiles are computed swept-major: C[swept][owned] =
//     sum_k X[swept][k] X[owned][k] with v_mfma_f32_32x32x16_bf16, so each
//     lane holds one owned index and 16 swept indices per 32x32 block.  Row
//     statistics reduce inside a lane; the lane pair (l, l^32) is combined
//     once at the end.
//   * The gradient contraction  out^T[d][owned] += sum_swept
//     X_s[swept][d] * dZ'[swept][owned]  takes dZ' straight from the logit
//     accumulators as the B operand: the 8 swept values a lane holds per
//     16-step are one B fragment under a fixed permutation of k.  The A
//     operand X_s^T is read from the same row-major LDS tile with the LDS
//     transpose read (ds_read_b64_tr_b16), with the same permutation.
//   * Row-owned sweeps (owned = query row i, swept = key j) give the row KL
//     and the row term dZ X_s; column-owned sweeps (owned = key j, swept =
//     row i) give the column term dZ^T X_s.  Both terms land in dX_s because
//     the relation is a self-relation.
#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace lmr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLog2eD = 1.4426950408889634074;
constexpr double kLn2D = 0.69314718055994530942;

// Waves per workgroup of each sweep (a workgroup of NW waves owns 32*NW
// rows).  Eight waves halve the tile copies per owned row.
#ifndef LMR_W_LSE
#define LMR_W_LSE 8
#endif
#ifndef LMR_W_ROW
#define LMR_W_ROW 8
#endif
#ifndef LMR_W_COL
#define LMR_W_COL 8
#endif
// Swept rows per LDS tile of each sweep (a multiple of 32).  128-row tiles
// halve the tile waits and barriers per block; an 8-wave workgroup has the
// LDS for them (2 x 2 x 32 KiB, one workgroup per CU).
#ifndef LMR_SW_LSE
#define LMR_SW_LSE 128
#endif
#ifndef LMR_SW_ROW
#define LMR_SW_ROW 128
#endif
#ifndef LMR_SW_COL
#define LMR_SW_COL 128
#endif

enum : int { ROLE_ROW = 0, ROLE_COL = 1 };

// Minimum waves per SIMD the sweeps are compiled for (register budget 512/occ).
#ifndef LMR_SWEEP_OCC
#define LMR_SWEEP_OCC 2
#endif
#ifndef LMR_LSE_OCC
#define LMR_LSE_OCC 2
#endif
// Phase 1 also comes in a wide shape: 12 waves (384 owned rows) sweeping
// 96-row tiles in 96 KiB of LDS.  It fits 3 waves per SIMD in its registers
// (the 8-wave shape's 128 KiB of LDS allows only 2), which measured 4% faster
// at n = 16K, but its larger row blocks leave small grids with a long tail,
// so it is used only when its grid has at least LMR_LSE_WIDE_MIN_GRID
// workgroups.
#ifndef LMR_W_LSE_WIDE
#define LMR_W_LSE_WIDE 12
#endif
#ifndef LMR_SW_LSE_WIDE
#define LMR_SW_LSE_WIDE 96
#endif
#ifndef LMR_LSE_WIDE_MIN_GRID
#define LMR_LSE_WIDE_MIN_GRID 1024
#endif
// Whether the forward-only sweep (phase 1 with the KL accumulator) takes the
// wide shape too.  Off: its extra accumulator spills at 3 waves per SIMD, and
// the 8-wave shape measured 2% faster at n = 16K and 8K.
#ifndef LMR_LSE_WIDE_KL
#define LMR_LSE_WIDE_KL 0
#endif

__device__ inline f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 pack8(const float* v) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (__bf16)v[e];
  return f;
}

// Row statistic in log2 units split as hi + lo (hi = its fp32 rounding).
// Phase 2 forms exp2(z*c - hi) with one fma, exact to fp32 rounding of the
// (small) result for the dominant entries.
__device__ inline void split_stat(double lse_nat, float& hi, float& lo) {
  const double l2 = lse_nat * kLog2eD;
  hi = (float)l2;
  lo = (float)(l2 - (double)hi);
}

// Row-major bf16 LDS tile with 16-byte chunks XOR-swizzled by f(row).  f is
// a bijection on 16 consecutive rows (so the 16 rows of a fragment read land
// in 16 distinct bank groups) and maps 4 consecutive rows to 4 different
// 4-chunk blocks (so the 4 rows x 4 chunks of a transpose read are
// conflict free as well).
template <int D, int SW = 64>
struct Tile {
  static constexpr int RB = 2 * D;                // bytes per row
  static constexpr int CH = RB / 16;              // chunks per row: 8 or 16
  static constexpr int RPL = 256 / RB;            // rows per 256-byte bank line
  static constexpr int QB = CH / 4;
  static constexpr int QSH = QB == 4 ? 2 : 1;
  static constexpr int BYTES = SW * RB;           // one tile of SW swept rows
  static_assert(D == 64 || D == 128, "head dim");
  __device__ static inline int f(int r) {
    const int m = r / RPL;
    return ((m & (QB - 1)) << 2) | ((m >> QSH) & 3);
  }
  __device__ static inline int off(int r, int c) { return r * RB + ((c ^ f(r)) << 4); }
  // MFMA operand with k = 16*ks + 8*h + e of row r (A operand of the logits).
  __device__ static inline bf16x8 frag(const char* base, int r, int ks, int h) {
    return *reinterpret_cast<const bf16x8*>(base + off(r, 2 * ks + h));
  }
  // A operand X^T[d][swept] of the contraction for 16-step q and d-block db:
  // lane (d = 32*db + lane%32, half h) gets swept rows 16q+4h+0..3 and
  // 16q+8+4h+0..3.  In each 16-lane group G, input lane L points at row
  // (base row + L/4) and the 4 columns 4*(L%4).. of the group's 16 columns;
  // the transpose read hands lane 4a+b column b of rows a, a+4, a+8, a+12.
  __device__ static inline bf16x8 tr_frag(const char* base, int q, int db, int lane) {
    const int G = lane >> 4, L = lane & 15, h = G >> 1;
    const int row = 16 * q + 4 * h + (L >> 2);
    const int dcol = 32 * db + 16 * (G & 1) + 4 * (L & 3);
    const int c = dcol >> 3, sub = (dcol & 7) * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off(row, c) + sub));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off(row + 8, c) + sub));
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
    return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // Direct global -> LDS copy of SW rows starting at row0 (rows >= n are
  // clamped to row n-1 and masked later).  Every wave-instruction writes 1 KB
  // of consecutive LDS (16 bytes per lane, at base + 16*lane); each lane
  // fetches the logical chunk that the swizzle puts at its physical slot.
  template <int NW>
  __device__ static inline void load(char* lds, const char* g, int row0, int n, int wave, int lane) {
    constexpr int U = BYTES / 1024 / NW;          // instructions per wave
    static_assert(U * 1024 * NW == BYTES, "tile copy split");
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = (wave * U + u) * 1024;
      const int P = blk + 16 * lane;
      const int r = P / RB, pos = (P % RB) >> 4;
      const int c = pos ^ f(r);
      const int gr = min(row0 + r, n - 1);
      const char* src = g + (int64_t)gr * RB + 16 * c;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(lds + blk), 16, 0, 0);
    }
  }
};

__device__ inline void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Owned-row MFMA B operand straight from global memory (null row = zeros).
__device__ inline bf16x8 load_own(const char* row, int ks, int h) {
  if (row == nullptr) return bf16x8{};
  return *reinterpret_cast<const bf16x8*>(row + (16 * ks + 8 * h) * 2);
}

// Both 32x32 logit blocks of swept sub-block sb against the wave's owned rows.
template <int D>
__device__ inline void logits(const char* lt, const char* ls, const bf16x8* Bt, const bf16x8* Bs,
                              f32x16& St, f32x16& Ss, int sb, int lane) {
  constexpr int KS = D / 16;
  const int h = lane >> 5, rr = 32 * sb + (lane & 31);
  St = f32x16{};
  Ss = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    St = mma(Tile<D>::frag(lt, rr, ks, h), Bt[ks], St);
    Ss = mma(Tile<D>::frag(ls, rr, ks, h), Bs[ks], Ss);
  }
}

// Gradient contraction of sub-block sb: acc[db] (out^T[d][owned]) +=
// X_s^T[d][swept] * dZ'[swept][owned], dZ' taken from the logit registers.
template <int D>
__device__ inline void contract(const f32x16& dz, const char* ls, int sb, int lane, f32x16* acc) {
  constexpr int DB = D / 32;
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = dz[8 * q2 + e];
    const bf16x8 bdz = pack8(v);
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = mma(Tile<D>::tr_frag(ls, 2 * sb + q2, db, lane), bdz, acc[db]);
  }
}

// Swept offset within a 32-row block of accumulator element r for half h.
__device__ inline int swept_of(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ---------------------------------------------------------------------------
// Phase 1: per-row LSE of teacher and student (row-owned sweep).
// ---------------------------------------------------------------------------
// Running sums are fp64: a row of 32K keys adds ~1000 block sums into each
// lane's total, and fp32 would let that error reach ~1e-4 of the LSE.
template <bool MASK>
__device__ inline void lse_block(const f32x16& St, const f32x16& Ss, float c, int sw_base, int i, int n,
                                 int causal, int h, float& mt, double& lt, float& ms, double& ls) {
  float zt[16], zs[16];
  float tmt = -INFINITY, tms = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    zt[r] = St[r];
    zs[r] = Ss[r];
    if (MASK) {
      const int j = sw_base + swept_of(r, h);
      const bool ok = (!causal || j <= i) && j < n;
      zt[r] = ok ? zt[r] : -INFINITY;
      zs[r] = ok ? zs[r] : -INFINITY;
    }
    tmt = fmaxf(tmt, zt[r]);
    tms = fmaxf(tms, zs[r]);
  }
  const float mnt = fmaxf(mt, tmt), mns = fmaxf(ms, tms);
  const float mct = mnt == -INFINITY ? 0.f : mnt * c;
  const float mcs = mns == -INFINITY ? 0.f : mns * c;
  float at = 0.f, as = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    at += __builtin_amdgcn_exp2f(fmaf(zt[r], c, -mct));
    as += __builtin_amdgcn_exp2f(fmaf(zs[r], c, -mcs));
  }
  if (mnt != mt) lt *= (double)__builtin_amdgcn_exp2f(fmaf(mt, c, -mct));
  if (mns != ms) ls *= (double)__builtin_amdgcn_exp2f(fmaf(ms, c, -mcs));
  lt += (double)at;
  ls += (double)as;
  mt = mnt;
  ms = mns;
}

// Fixed-shift block sum: sum_r exp2(z_r * c - ref) over one 32x32 block
// (masked entries contribute 0).  KL: also w += sum_r exp2(a_t)(a_t - a_s)
// with a_m = z_m * c - ref_m, the teacher-weighted log-ratio numerator.
template <bool MASK, bool KL>
__device__ inline void lse_block_fixed(const f32x16& St, const f32x16& Ss, float c, float rt, float rs,
                                       int sw_base, int i, int n, int causal, int h, double& lt, double& ls,
                                       double& w) {
  float at = 0.f, as = 0.f, aw = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float xt = fmaf(St[r], c, -rt), xs = fmaf(Ss[r], c, -rs);
    float et = __builtin_amdgcn_exp2f(xt);
    float es = __builtin_amdgcn_exp2f(xs);
    if (MASK) {
      const int j = sw_base + swept_of(r, h);
      const bool ok = (!causal || j <= i) && j < n;
      et = ok ? et : 0.f;
      es = ok ? es : 0.f;
    }
    at += et;
    as += es;
    if (KL) aw = fmaf(et, xt - xs, aw);
  }
  lt += (double)at;
  ls += (double)as;
  if (KL) w += (double)aw;
}

// Teacher-weighted log-ratio against fixed statistics hi_t, hi_s (log2
// units): k += sum_r exp2(a_t) (a_t - a_s), a_m = z_m * c - hi_m.
__device__ inline void kl_block_stat(const f32x16& St, const f32x16& Ss, float c, float ht, float hs,
                                     int sw_base, int i, int n, int causal, int h, double& k) {
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = sw_base + swept_of(r, h);
    const bool ok = (!causal || j <= i) && j < n;
    const float xt = fmaf(St[r], c, -ht), xs = fmaf(Ss[r], c, -hs);
    const float pt = ok ? __builtin_amdgcn_exp2f(xt) : 0.f;
    acc = fmaf(pt, ok ? xt - xs : 0.f, acc);
  }
  k += (double)acc;
}

// Work item of a block in a launch over a map set.  Blocks are ordered by
// map, then within a map so that the workgroups resident on one XCD at a
// time share few heads: workgroups are handed to the 8 XCDs round-robin by
// block index, and the workgroups of one head that run together on one XCD
// sweep the same key tiles, which its L2 then serves once.  When the map's
// head count is a multiple of 8, XCD x (blocks x, x+8, ...) takes its heads
// x, x+8, ... in groups of LMR_XCD_HEADS, and runs each group's row blocks
// rank by rank (longest rows first), heads interleaved.  Other head counts
// use rank-major order over all heads.  The map's arguments are selected
// with a uniform select chain (no indexed copy).
#ifndef LMR_XCD_HEADS
#define LMR_XCD_HEADS 0      // 0: every head of the XCD in one group (rank-major)
#endif
struct WorkItem {
  SweepArgs a;
  int64_t bh;   // head within the map
  int r;        // row-block rank
};

__device__ inline WorkItem decode(const MapSet& S, int nblk) {
  const int64_t bid = blockIdx.x;
  WorkItem w;
  w.a = S.map[0];
  int64_t h0 = 0, h1 = S.head0[1];
#pragma unroll
  for (int k = 1; k < kMaxMaps; ++k) {
    if (k < S.nmaps && bid >= (int64_t)nblk * S.head0[k]) {
      w.a = S.map[k];
      h0 = S.head0[k];
      h1 = S.head0[k + 1];
    }
  }
  const int64_t local = bid - (int64_t)nblk * h0, heads = h1 - h0;
  const int64_t q = heads / 8;                        // heads per XCD
  const int64_t g = LMR_XCD_HEADS > 0 && LMR_XCD_HEADS < q && q % LMR_XCD_HEADS == 0 ? LMR_XCD_HEADS : q;
  if (heads % 8 == 0) {
    const int64_t x = local % 8, slot = local / 8;    // XCD and position in its queue
    const int64_t grp = slot / (g * nblk), rem = slot % (g * nblk);
    w.r = (int)(rem / g);
    w.bh = x + 8 * (grp * g + rem % g);
  } else {
    w.r = (int)(local / heads);
    w.bh = local % heads;
  }
  return w;
}

// End of the phase-1 sweep: combine the lane pair, store LSE (and row KL),
// or, if any row of the workgroup overflowed the fixed shift, redo the
// workgroup's rows with the online maximum.  lds holds two double-buffer
// slots of two tiles; every tile copy of the main sweep has completed.
template <int D, bool KL, int NW, int SW>
__device__ inline void lse_finish(const SweepArgs& a, int64_t bh, const char* yt, const char* ys,
                                  char (*lds)[2][Tile<D, SW>::BYTES], const bf16x8* Bt, const bf16x8* Bs, int ntiles,
                                  int wown0, int i, int n, float c, float ref_t, float ref_s, int wave, int lane,
                                  int h, double lsum_t, double lsum_s, double wkl) {
  lsum_t += __shfl_xor(lsum_t, 32);
  lsum_s += __shfl_xor(lsum_s, 32);
  if (KL) wkl += __shfl_xor(wkl, 32);
  const bool bad = i < n && !(lsum_t > 0.0 && lsum_t < 1e300 && lsum_s > 0.0 && lsum_s < 1e300 &&
                              (!KL || fabs(wkl) < 1e300));
  if (!__syncthreads_or(bad)) {
    // LSE = ln2 * (ref + log2 L), in fp64.
    if (h == 0 && i < n) {
      const double l2t = log2(lsum_t), l2s = log2(lsum_s);
      static_cast<double*>(a.lse_t)[bh * n + i] = ((double)ref_t + l2t) * kLn2D;
      static_cast<double*>(a.lse_s)[bh * n + i] = ((double)ref_s + l2s) * kLn2D;
      if (KL) a.row_kl[bh * n + i] = (float)((wkl / lsum_t + (l2s - l2t)) * kLn2D);
    }
    return;
  }

  // Fallback: online maximum.
  float mt = -INFINITY, ms = -INFINITY;
  lsum_t = 0.0;
  lsum_s = 0.0;
  for (int tI = 0; tI < ntiles; ++tI) {
    const int buf = tI & 1, sw0 = tI * SW;
    __syncthreads();
    Tile<D, SW>::template load<NW>(lds[buf][0], yt, sw0, n, wave, lane);
    Tile<D, SW>::template load<NW>(lds[buf][1], ys, sw0, n, wave, lane);
    wait_loads();
    __syncthreads();
    if (wown0 >= n || (a.causal && sw0 > wown0 + 31)) continue;
#pragma unroll
    for (int sb = 0; sb < SW / 32; ++sb) {
      f32x16 St, Ss;
      logits<D>(lds[buf][0], lds[buf][1], Bt, Bs, St, Ss, sb, lane);
      lse_block<true>(St, Ss, c, sw0 + 32 * sb, i, n, a.causal, h, mt, lsum_t, ms, lsum_s);
    }
  }
  const float mt2 = __shfl_xor(mt, 32), ms2 = __shfl_xor(ms, 32);
  const double lt2 = __shfl_xor(lsum_t, 32), ls2 = __shfl_xor(lsum_s, 32);
  const float Mt = fmaxf(mt, mt2), Ms = fmaxf(ms, ms2);
  const float Mct = Mt * c, Mcs = Ms * c;
  // The shifts Mt*c are exact fp32 values; exp2 of their (small) differences
  // is evaluated in fp64 so the combination adds no fp32 rounding.
  const double Lt = lsum_t * exp2((double)fmaf(mt, c, -Mct)) + lt2 * exp2((double)fmaf(mt2, c, -Mct));
  const double Ls = lsum_s * exp2((double)fmaf(ms, c, -Mcs)) + ls2 * exp2((double)fmaf(ms2, c, -Mcs));
  const double L2t = (double)Mct + log2(Lt), L2s = (double)Mcs + log2(Ls);
  if (h == 0 && i < n) {
    static_cast<double*>(a.lse_t)[bh * n + i] = L2t * kLn2D;
    static_cast<double*>(a.lse_s)[bh * n + i] = L2s * kLn2D;
  }
  if (!KL) return;
  // KL after the fallback: a second sweep against the exact statistics,
  // as the phase-2 row sweep forms it:
  //   KL_i = ln2 * (2^-lo_t * sum_j 2^(a_t)(a_t - a_s) + lo_s - lo_t),
  // a_m = c z_m - hi_m, hi_m the fp32 rounding of L2_m and lo_m the rest.
  const float ht = (float)L2t, hs = (float)L2s;
  const double lot = L2t - (double)ht, los = L2s - (double)hs;
  double kacc = 0.0;
  for (int tI = 0; tI < ntiles; ++tI) {
    const int buf = tI & 1, sw0 = tI * SW;
    __syncthreads();
    Tile<D, SW>::template load<NW>(lds[buf][0], yt, sw0, n, wave, lane);
    Tile<D, SW>::template load<NW>(lds[buf][1], ys, sw0, n, wave, lane);
    wait_loads();
    __syncthreads();
    if (wown0 >= n || (a.causal && sw0 > wown0 + 31)) continue;
#pragma unroll
    for (int sb = 0; sb < SW / 32; ++sb) {
      f32x16 St, Ss;
      logits<D>(lds[buf][0], lds[buf][1], Bt, Bs, St, Ss, sb, lane);
      kl_block_stat(St, Ss, c, ht, hs, sw0 + 32 * sb, i, n, a.causal, h, kacc);
    }
  }
  kacc += __shfl_xor(kacc, 32);
  if (h == 0 && i < n) a.row_kl[bh * n + i] = (float)((exp2(-lot) * kacc + los - lot) * kLn2D);
}

// Phase 1.  Every row's sum is taken against a fixed shift, the row's own
// diagonal logit c*|x_i|^2 (the diagonal is always a kept entry), so the
// inner loop needs no running maximum.  A term can only overflow if
// <x_i, x_j> exceeds |x_i|^2 by more than ~88/scale; if any row of the
// workgroup overflows, the workgroup redoes its rows with the online
// maximum.  The stored statistic is exact either way.
//
// KL (forward-only loss): the same sweep also accumulates
// w_i = sum_j 2^(a_t)(a_t - a_s), a_m = c z_m - ref_m, so that with
// L_m = sum_j 2^(a_m) (log2 units throughout)
//   KL_i / ln2 = sum_j r_t (log2 r_t - log2 r_s) = w_i / L_t + log2(L_s / L_t),
// because log2 r_m = a_m - log2 L_m.  The loss then costs 2 GEMM-units
// instead of phase 1 plus a phase-2 sweep.  Identical inputs give a_t == a_s
// and L_t == L_s bit for bit, hence exactly zero.
template <int D, bool KL, int NW, int SW>
__global__ __launch_bounds__(64 * NW, LMR_LSE_OCC) void lse_fwd_kernel(MapSet maps, int nblk) {
  constexpr int KS = D / 16, RB = 2 * D, TB = Tile<D, SW>::BYTES, kOwn = 32 * NW;
  __shared__ __attribute__((aligned(1024))) char lds[2][2][TB];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const WorkItem wi = decode(maps, nblk);
  const SweepArgs& a = wi.a;
  const int64_t bh = wi.bh;
  const int ob = nblk - 1 - wi.r;                       // longest rows first
  const int n = a.n;
  // Owned rows i come from X, swept tiles (columns j) from Y (== X for a
  // self-relation).
  const char* xt = static_cast<const char*>(a.xt) + bh * (int64_t)n * RB;
  const char* xs = static_cast<const char*>(a.xs) + bh * (int64_t)n * RB;
  const char* yt = static_cast<const char*>(a.yt) + bh * (int64_t)n * RB;
  const char* ys = static_cast<const char*>(a.ys) + bh * (int64_t)n * RB;
  const int own0 = ob * kOwn, wown0 = own0 + 32 * wave, i = wown0 + (lane & 31);

  bf16x8 Bt[KS], Bs[KS];
  {
    const char* rt = i < n ? xt + (int64_t)i * RB : nullptr;
    const char* rs = i < n ? xs + (int64_t)i * RB : nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) { Bt[ks] = load_own(rt, ks, h); Bs[ks] = load_own(rs, ks, h); }
  }
  const int last = a.causal ? min(own0 + kOwn, n) - 1 : n - 1;
  const int ntiles = last / SW + 1;
  const float c = a.scale * kLog2e;

  // Shift: the diagonal logit c * <x_i, y_i> (c * |x_i|^2 for a self-relation),
  // from the row's own fragments (each lane half holds half of d).
  float nt = 0.f, ns = 0.f;
  if (a.cross) {
    const char* qt = i < n ? yt + (int64_t)i * RB : nullptr;
    const char* qs = i < n ? ys + (int64_t)i * RB : nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 yt8 = load_own(qt, ks, h), ys8 = load_own(qs, ks, h);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        nt = fmaf((float)Bt[ks][e], (float)yt8[e], nt);
        ns = fmaf((float)Bs[ks][e], (float)ys8[e], ns);
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float vt = (float)Bt[ks][e], vs = (float)Bs[ks][e];
        nt = fmaf(vt, vt, nt);
        ns = fmaf(vs, vs, ns);
      }
  }
  nt += __shfl_xor(nt, 32);
  ns += __shfl_xor(ns, 32);
  const float ref_t = nt * c, ref_s = ns * c;

  double lsum_t = 0.0, lsum_s = 0.0, wkl = 0.0;
  Tile<D, SW>::template load<NW>(lds[0][0], yt, 0, n, wave, lane);
  Tile<D, SW>::template load<NW>(lds[0][1], ys, 0, n, wave, lane);
  for (int tI = 0; tI < ntiles; ++tI) {
    const int buf = tI & 1, sw0 = tI * SW;
    wait_loads();
    __syncthreads();
    if (tI + 1 < ntiles) {
      Tile<D, SW>::template load<NW>(lds[buf ^ 1][0], yt, sw0 + SW, n, wave, lane);
      Tile<D, SW>::template load<NW>(lds[buf ^ 1][1], ys, sw0 + SW, n, wave, lane);
    }
#pragma unroll
    for (int sb = 0; sb < SW / 32; ++sb) {
      // 32-row block: stop past this wave's diagonal block or past the end.
      const int swb = sw0 + 32 * sb;
      if (wown0 >= n || (a.causal && swb > wown0 + 31) || swb >= n) break;
      const bool need_mask = (a.causal && swb + 31 > wown0) || swb + 32 > n;
      f32x16 St, Ss;
      logits<D>(lds[buf][0], lds[buf][1], Bt, Bs, St, Ss, sb, lane);
      if (need_mask)
        lse_block_fixed<true, KL>(St, Ss, c, ref_t, ref_s, swb, i, n, a.causal, h, lsum_t, lsum_s, wkl);
      else
        lse_block_fixed<false, KL>(St, Ss, c, ref_t, ref_s, swb, i, n, a.causal, h, lsum_t, lsum_s, wkl);
    }
  }
  lse_finish<D, KL, NW, SW>(a, bh, yt, ys, lds, Bt, Bs, ntiles, wown0, i, n, c, ref_t, ref_s, wave, lane, h, lsum_t, lsum_s,
                    wkl);
}

// ---------------------------------------------------------------------------
// Phase 2 sweep.  ROLE_ROW: owned = row i, swept = column j; writes row KL
// and stores the row term.  ROLE_COL: owned = column j, swept = row i; adds
// the column term to what the row sweep stored.
//
// Diagonal entries.  Row i of dZ sums to zero, and dZ(i,i) enters dX_s[i]
// twice (row and column term), so
//   dX_s[i] ~ sum_{j!=i} dZ(i,j) x_j + sum_{j!=i} dZ(j,i) x_j
//             - 2 (sum_{j!=i} dZ(i,j)) x_i.
// Both sweeps skip the diagonal entry and the row sweep adds the last term
// from its running sum of off-diagonal dZ.  The probability of a dominant
// diagonal is ~1 and its fp32 rounding (~6e-8) would otherwise swamp the
// vanishing gradient of very peaky rows.
//
// Probabilities: with the fp64 statistic split as hi + lo (log2 units),
// p = exp2(z*c - hi) is the true probability times 2^lo, |lo| <= one fp32
// ulp of hi.  dZ uses p directly (the factor only moves off-diagonal
// entries by ~1e-6 of themselves); the row KL applies it exactly:
//   KL_i = ln2 * (2^-lo_t * sum_j p_t (a_t - a_s) + lo_s - lo_t),
// using sum_j p_t 2^-lo_t = 1.  Identical teacher and student inputs give
// exactly zero loss and gradient.
// ---------------------------------------------------------------------------

// Per-lane running state of a row sweep: per-block fp32 partials are added
// into fp64 totals (rows of 32K keys add ~1000 blocks per lane).
struct SweepState {
  double kl = 0.0;          // sum_j p_t (a_t - a_s), log2 units
  double dsum = 0.0;        // sum_{j != i} (p_s - p_t)
};

// Elementwise step on one 32x32 block, in place: St <- dZ * n.
// SPECIAL: the block may hold masked or diagonal entries of this wave.
// COL blocks read the swept rows' (hi_t, hi_s) from `stat`.
template <int ROLE, bool SPECIAL>
__device__ inline void block_elementwise(f32x16& St, const f32x16& Ss, float c, int sw_base, int o, int n,
                                         int causal, int h, float l2t, float l2s, const float2* stat,
                                         SweepState& S) {
  float kl = 0.f, dsum = 0.f;
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * g4 + e;
      float bt = l2t, bs = l2s;
      if (ROLE == ROLE_COL) {
        const float2 st = stat[8 * g4 + 4 * h + e];
        bt = st.x;
        bs = st.y;
      }
      float at = fmaf(St[r], c, -bt);
      float as = fmaf(Ss[r], c, -bs);
      float pt = __builtin_amdgcn_exp2f(at);
      float ps = __builtin_amdgcn_exp2f(as);
      float dz;
      if (SPECIAL) {
        const int sw = sw_base + swept_of(r, h);
        const int ii = ROLE == ROLE_ROW ? o : sw;
        const int jj = ROLE == ROLE_ROW ? sw : o;
        const bool ok = (!causal || jj <= ii) && sw < n;
        pt = ok ? pt : 0.f;
        ps = ok ? ps : 0.f;
        at = ok ? at : 0.f;
        as = ok ? as : 0.f;
        dz = (ok && sw != o) ? ps - pt : 0.f;
      } else {
        dz = ps - pt;
      }
      if (ROLE == ROLE_ROW) {
        kl = fmaf(pt, at - as, kl);
        dsum += dz;
      }
      St[r] = dz;
    }
  }
  if (ROLE == ROLE_ROW) {
    S.kl += (double)kl;
    S.dsum += (double)dsum;
  }
}

template <int D, int ROLE, bool WITH_DX, int NW, int SW>
__global__ __launch_bounds__(64 * NW, LMR_SWEEP_OCC) void kl_sweep_kernel(MapSet maps, int nblk) {
  constexpr int KS = D / 16, DB = D / 32, RB = 2 * D, TB = Tile<D, SW>::BYTES, kOwn = 32 * NW;
  static_assert(SW % 32 == 0 && SW <= 64 * NW, "one thread per swept row fetches the statistics");
  constexpr int NSTAT = ROLE == ROLE_COL ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char lds[2][2][TB];
  // COL: per swept row (hi_t, hi_s), double-buffered.
  __shared__ float2 lstat[NSTAT][ROLE == ROLE_COL ? SW : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const WorkItem wi = decode(maps, nblk);
  const SweepArgs& a = wi.a;
  const int64_t bh = wi.bh;
  const int ob = ROLE == ROLE_ROW ? nblk - 1 - wi.r : wi.r;
  const int n = a.n;
  // ROW: owned rows i of X, swept rows j of Y.  COL: owned rows j of Y,
  // swept rows i of X.  (X == Y for a self-relation.)
  const int64_t hoff = bh * (int64_t)n * RB;
  const char* ot = static_cast<const char*>(ROLE == ROLE_ROW ? a.xt : a.yt) + hoff;
  const char* os = static_cast<const char*>(ROLE == ROLE_ROW ? a.xs : a.ys) + hoff;
  const char* wt = static_cast<const char*>(ROLE == ROLE_ROW ? a.yt : a.xt) + hoff;
  const char* ws = static_cast<const char*>(ROLE == ROLE_ROW ? a.ys : a.xs) + hoff;
  const double* glt = static_cast<const double*>(a.lse_t) + bh * n;
  const double* gls = static_cast<const double*>(a.lse_s) + bh * n;
  const int own0 = ob * kOwn, wown0 = own0 + 32 * wave, o = wown0 + (lane & 31);
  const float c = a.scale * kLog2e;

  bf16x8 Bt[KS], Bs[KS];
  {
    const char* rt = o < n ? ot + (int64_t)o * RB : nullptr;
    const char* rs = o < n ? os + (int64_t)o * RB : nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) { Bt[ks] = load_own(rt, ks, h); Bs[ks] = load_own(rs, ks, h); }
  }
  float l2t = 0.f, l2s = 0.f, lot = 0.f, los = 0.f;     // owned-row statistics (ROW)
  if (ROLE == ROLE_ROW && o < n) {
    split_stat(glt[o], l2t, lot);
    split_stat(gls[o], l2s, los);
  }
  int t_begin, t_end;
  if (ROLE == ROLE_ROW) {
    t_begin = 0;
    t_end = (a.causal ? min(own0 + kOwn, n) - 1 : n - 1) / SW + 1;
  } else {
    t_begin = a.causal ? own0 / SW : 0;
    t_end = (n - 1) / SW + 1;
  }

  SweepState S;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // COL statistics: threads 0..63 hold the fp64 LSE of the next tile's rows.
  double nlt = 0.0, nls = 0.0;
  auto fetch_stat = [&](int tile) {
    const int g = tile * SW + tid;
    nlt = g < n ? glt[g] : 0.0;
    nls = g < n ? gls[g] : 0.0;
  };
  auto put_stat = [&](int b, int tile) {
    const int g = tile * SW + tid;
    float ht = 0.f, hs = 0.f, ft, fs;
    if (g < n) {
      split_stat(nlt, ht, ft);
      split_stat(nls, hs, fs);
    }
    lstat[b][tid] = make_float2(ht, hs);
  };

  Tile<D, SW>::template load<NW>(lds[0][0], wt, t_begin * SW, n, wave, lane);
  Tile<D, SW>::template load<NW>(lds[0][1], ws, t_begin * SW, n, wave, lane);
  if (ROLE == ROLE_COL && tid < SW) {
    fetch_stat(t_begin);
    put_stat(0, t_begin);
    if (t_begin + 1 < t_end) fetch_stat(t_begin + 1);
  }
  for (int tI = t_begin; tI < t_end; ++tI) {
    const int buf = (tI - t_begin) & 1, sw0 = tI * SW;
    wait_loads();
    __syncthreads();
    if (tI + 1 < t_end) {
      Tile<D, SW>::template load<NW>(lds[buf ^ 1][0], wt, sw0 + SW, n, wave, lane);
      Tile<D, SW>::template load<NW>(lds[buf ^ 1][1], ws, sw0 + SW, n, wave, lane);
      if (ROLE == ROLE_COL && tid < SW) {
        put_stat(buf ^ 1, tI + 1);
        if (tI + 2 < t_end) fetch_stat(tI + 2);
      }
    }
    const char* lt = lds[buf][0];
    const char* ls = lds[buf][1];
    if constexpr (ROLE == ROLE_ROW) {
#pragma unroll
      for (int sb = 0; sb < SW / 32; ++sb) {
        // 32-row swept block: stop past this wave's diagonal block or past
        // the end.  Blocks with masked entries or with this wave's diagonal
        // take the per-entry path.
        const int swb = sw0 + 32 * sb;
        if ((a.causal && swb > wown0 + 31) || swb >= n) break;
        const bool need_mask = (a.causal && swb + 31 > wown0) || swb + 32 > n;
        f32x16 St, Ss;
        logits<D>(lt, ls, Bt, Bs, St, Ss, sb, lane);
        if (need_mask || swb == wown0)
          block_elementwise<ROLE, true>(St, Ss, c, swb, o, n, a.causal, h, l2t, l2s, nullptr, S);
        else
          block_elementwise<ROLE, false>(St, Ss, c, swb, o, n, a.causal, h, l2t, l2s, nullptr, S);
        if constexpr (WITH_DX) contract<D>(St, ls, sb, lane, acc);
      }
    } else {
      // Column sweep: decided per tile (per-block tests measured slower here).
      if (wown0 >= n || (a.causal && wown0 > sw0 + SW - 1)) continue;        // tile entirely above the diagonal
      const bool need_mask = (a.causal && wown0 + 31 > sw0) || (sw0 + SW > n);
      // Tiles that hold a diagonal entry of this wave take the per-entry path too.
      const bool special = need_mask || (sw0 <= wown0 + 31 && sw0 + SW - 1 >= wown0);
#pragma unroll
      for (int sb = 0; sb < SW / 32; ++sb) {
        const float2* stat = &lstat[buf][32 * sb];
        f32x16 St, Ss;
        logits<D>(lt, ls, Bt, Bs, St, Ss, sb, lane);
        if (special)
          block_elementwise<ROLE, true>(St, Ss, c, sw0 + 32 * sb, o, n, a.causal, h, l2t, l2s, stat, S);
        else
          block_elementwise<ROLE, false>(St, Ss, c, sw0 + 32 * sb, o, n, a.causal, h, l2t, l2s, stat, S);
        if constexpr (WITH_DX) contract<D>(St, ls, sb, lane, acc);
      }
    }
  }

  // ROW: sum_{j!=i} dZ(i,j) * n stands in for -dZ(i,i) * n.  The diagonal
  // entry contributes dZ(i,i) y_s[i] to dX_s[i] and dZ(i,i) x_s[i] to
  // dY_s[i]; for a self-relation both land in dX_s.
  float corr = 0.f;
  if (ROLE == ROLE_ROW) {
    S.kl += __shfl_xor(S.kl, 32);
    S.dsum += __shfl_xor(S.dsum, 32);
    const double klr = exp2(-(double)lot) * S.kl + (double)los - (double)lot;
    if (h == 0 && o < n && a.row_kl != nullptr) a.row_kl[bh * n + o] = (float)(klr * kLn2D);
    corr = (float)((a.cross ? -1.0 : -2.0) * S.dsum);
  }
  auto bf4 = [](const char* row, int d0, float* x4) {     // 4 bf16 of a row as fp32
    const uint2 raw = *reinterpret_cast<const uint2*>(row + 2 * d0);
    x4[0] = __uint_as_float(raw.x << 16);
    x4[1] = __uint_as_float(raw.x & 0xffff0000u);
    x4[2] = __uint_as_float(raw.y << 16);
    x4[3] = __uint_as_float(raw.y & 0xffff0000u);
  };
  const float gs = a.grad_scale;
  if constexpr (WITH_DX) {
    float* out = ROLE == ROLE_COL && a.cross ? a.dy : a.dx;
    if (o < n) {
      float* dst = out + (bh * (int64_t)n + o) * D;
      const char* yo = ws + (int64_t)o * RB;              // ROW: y_s[i] (x_s[i] for a self-relation)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * db + 8 * g4 + 4 * h;
          f32x4 v;
          if (ROLE == ROLE_ROW) {
            float x4[4];
            bf4(yo, d0, x4);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fmaf(corr, x4[e], acc[db][4 * g4 + e]) * gs;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * g4 + e] * gs;
          }
          f32x4* p = reinterpret_cast<f32x4*>(dst + d0);
          if (ROLE == ROLE_ROW) *p = v;
          else *p = *p + v;
        }
      }
    }
  }
  // Cross relation: the row sweep also stores the diagonal part of dY_s[i],
  // dZ(i,i) x_s[i]; the column sweep adds the rest.
  if (ROLE == ROLE_ROW && a.cross && a.dy != nullptr && o < n) {
    float* dst = a.dy + (bh * (int64_t)n + o) * D;
    const char* xo = os + (int64_t)o * RB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * h;
        float x4[4];
        bf4(xo, d0, x4);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = corr * x4[e] * gs;
        *reinterpret_cast<f32x4*>(dst + d0) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused phase 2 of a self-relation: one workgroup owns a block of rows k and
// produces their whole gradient.  It first sweeps the key tiles j <= k (the
// row term sum_j dZ(k,j) x_j, as the row sweep above, with the row KL), then
// the row tiles i >= k (the column term sum_i dZ(i,k) x_i, as the column
// sweep above), adding both into one register accumulator and storing dX_s
// once.  Every workgroup sweeps the same number of tiles (the causal
// triangle of its row term plus the complementary triangle of its column
// term), so the launch has no causal tail; the work executed is the split
// mode's (the logit tiles are computed twice), without its second launch and
// its read-modify-write of dX_s.
// ---------------------------------------------------------------------------
template <int D, int NW, int SW>
__global__ __launch_bounds__(64 * NW, LMR_SWEEP_OCC) void kl_fused_kernel(MapSet maps, int nblk) {
  constexpr int KS = D / 16, DB = D / 32, RB = 2 * D, TB = Tile<D, SW>::BYTES, kOwn = 32 * NW;
  static_assert(SW % 32 == 0 && SW <= 64 * NW, "one thread per swept row fetches the statistics");
  __shared__ __attribute__((aligned(1024))) char lds[2][2][TB];
  __shared__ float2 lstat[2][SW];          // column steps: (hi_t, hi_s) of the swept rows

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const WorkItem wi = decode(maps, nblk);
  const SweepArgs& a = wi.a;
  const int64_t bh = wi.bh;
  const int ob = wi.r;
  const int n = a.n;
  const int64_t hoff = bh * (int64_t)n * RB;
  const char* xt = static_cast<const char*>(a.xt) + hoff;
  const char* xs = static_cast<const char*>(a.xs) + hoff;
  const double* glt = static_cast<const double*>(a.lse_t) + bh * n;
  const double* gls = static_cast<const double*>(a.lse_s) + bh * n;
  const int own0 = ob * kOwn, wown0 = own0 + 32 * wave, o = wown0 + (lane & 31);
  const float c = a.scale * kLog2e;

  bf16x8 Bt[KS], Bs[KS];
  {
    const char* rt = o < n ? xt + (int64_t)o * RB : nullptr;
    const char* rs = o < n ? xs + (int64_t)o * RB : nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) { Bt[ks] = load_own(rt, ks, h); Bs[ks] = load_own(rs, ks, h); }
  }
  float l2t = 0.f, l2s = 0.f, lot = 0.f, los = 0.f;
  if (o < n) {
    split_stat(glt[o], l2t, lot);
    split_stat(gls[o], l2s, los);
  }
  // Steps 0 .. r_end-1 are row tiles 0 .. r_end-1; the following steps are
  // column tiles c_begin .. c_end-1.
  const int r_end = (a.causal ? min(own0 + kOwn, n) - 1 : n - 1) / SW + 1;
  const int c_begin = a.causal ? own0 / SW : 0;
  const int steps = r_end + ((n - 1) / SW + 1 - c_begin);
  auto tile_of = [&](int k) { return k < r_end ? k : c_begin + (k - r_end); };

  SweepState S;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // Column-step statistics: threads 0..SW-1 fetch the fp64 LSE of a column
  // step's swept rows two steps ahead and publish them to LDS one step ahead.
  double nlt = 0.0, nls = 0.0;
  auto fetch_stat = [&](int tile) {
    const int g = tile * SW + tid;
    nlt = g < n ? glt[g] : 0.0;
    nls = g < n ? gls[g] : 0.0;
  };
  auto put_stat = [&](int b, int tile) {
    const int g = tile * SW + tid;
    float ht = 0.f, hs = 0.f, ft, fs;
    if (g < n) {
      split_stat(nlt, ht, ft);
      split_stat(nls, hs, fs);
    }
    lstat[b][tid] = make_float2(ht, hs);
  };

  // Row steps.  The tile of the next step is copied during each step; the
  // statistics of the first column step's rows are published after the last
  // row step (the column steps then run their own two-ahead prefetch).
  Tile<D, SW>::template load<NW>(lds[0][0], xt, 0, n, wave, lane);
  Tile<D, SW>::template load<NW>(lds[0][1], xs, 0, n, wave, lane);
  int k = 0;
  for (; k < r_end; ++k) {
    const int buf = k & 1, sw0 = k * SW;
    wait_loads();
    __syncthreads();
    if (k + 1 < steps) {
      const int nx = tile_of(k + 1) * SW;
      Tile<D, SW>::template load<NW>(lds[buf ^ 1][0], xt, nx, n, wave, lane);
      Tile<D, SW>::template load<NW>(lds[buf ^ 1][1], xs, nx, n, wave, lane);
    }
    const char* lt = lds[buf][0];
    const char* ls = lds[buf][1];
    // 32-row key blocks up to this wave's diagonal block.
#pragma unroll
    for (int sb = 0; sb < SW / 32; ++sb) {
      const int swb = sw0 + 32 * sb;
      if (wown0 >= n || (a.causal && swb > wown0 + 31) || swb >= n) break;
      const bool need_mask = (a.causal && swb + 31 > wown0) || swb + 32 > n;
      f32x16 St, Ss;
      logits<D>(lt, ls, Bt, Bs, St, Ss, sb, lane);
      if (need_mask || swb == wown0)
        block_elementwise<ROLE_ROW, true>(St, Ss, c, swb, o, n, a.causal, h, l2t, l2s, nullptr, S);
      else
        block_elementwise<ROLE_ROW, false>(St, Ss, c, swb, o, n, a.causal, h, l2t, l2s, nullptr, S);
      contract<D>(St, ls, sb, lane, acc);
    }
  }

  // Row KL, and the diagonal term: both off-diagonal sums of dZ(k,.) stand in
  // for -2 dZ(k,k) (see the row sweep).
  S.kl += __shfl_xor(S.kl, 32);
  S.dsum += __shfl_xor(S.dsum, 32);
  const double klr = exp2(-(double)lot) * S.kl + (double)los - (double)lot;
  if (h == 0 && o < n && a.row_kl != nullptr) a.row_kl[bh * n + o] = (float)(klr * kLn2D);
  const float corr = (float)(-2.0 * S.dsum);

  // Column steps.  No column step has run, so lstat is free.
  if (tid < SW && k < steps) {
    fetch_stat(tile_of(k));
    put_stat(k & 1, tile_of(k));
    if (k + 1 < steps) fetch_stat(tile_of(k + 1));
  }
  for (; k < steps; ++k) {
    const int buf = k & 1, sw0 = tile_of(k) * SW;
    wait_loads();
    __syncthreads();
    if (k + 1 < steps) {
      const int nx = tile_of(k + 1) * SW;
      Tile<D, SW>::template load<NW>(lds[buf ^ 1][0], xt, nx, n, wave, lane);
      Tile<D, SW>::template load<NW>(lds[buf ^ 1][1], xs, nx, n, wave, lane);
      if (tid < SW) {
        put_stat(buf ^ 1, tile_of(k + 1));
        if (k + 2 < steps) fetch_stat(tile_of(k + 2));
      }
    }
    const char* lt = lds[buf][0];
    const char* ls = lds[buf][1];
    // Row tiles at or below the diagonal of this wave's rows (as keys).
    if (wown0 >= n || (a.causal && wown0 > sw0 + SW - 1)) continue;
    const bool need_mask = (a.causal && wown0 + 31 > sw0) || (sw0 + SW > n);
    const bool special = need_mask || (sw0 <= wown0 + 31 && sw0 + SW - 1 >= wown0);
#pragma unroll
    for (int sb = 0; sb < SW / 32; ++sb) {
      const float2* stat = &lstat[buf][32 * sb];
      f32x16 St, Ss;
      logits<D>(lt, ls, Bt, Bs, St, Ss, sb, lane);
      if (special)
        block_elementwise<ROLE_COL, true>(St, Ss, c, sw0 + 32 * sb, o, n, a.causal, h, l2t, l2s, stat, S);
      else
        block_elementwise<ROLE_COL, false>(St, Ss, c, sw0 + 32 * sb, o, n, a.causal, h, l2t, l2s, stat, S);
      contract<D>(St, ls, sb, lane, acc);
    }
  }

  const float gs = a.grad_scale;
  if (o < n) {
    float* dst = a.dx + (bh * (int64_t)n + o) * D;
    const char* xo = xs + (int64_t)o * RB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * h;
        const uint2 raw = *reinterpret_cast<const uint2*>(xo + 2 * d0);
        const float x4[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                             __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(corr, x4[e], acc[db][4 * g4 + e]) * gs;
        *reinterpret_cast<f32x4*>(dst + d0) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Deterministic fp64 reduction of row_kl to the loss scalar.
// ---------------------------------------------------------------------------
constexpr int kRedThreads = 256;

__device__ inline double block_sum(double v, double* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
#pragma unroll
  for (int s = kRedThreads / 2; s > 0; s >>= 1) {
    if (tid < s) sh[tid] += sh[tid + s];
    __syncthreads();
  }
  return sh[0];
}

// Per-head weights of a weighted reduction (map m owns heads head0[m] ..).
struct HeadWeights {
  int64_t head0[kMaxMaps + 1];
  float w[kMaxMaps];
  int nmaps;
};

__global__ __launch_bounds__(kRedThreads) void reduce_rows_kernel(const float* row_kl, int n, double* partials,
                                                                  HeadWeights W) {
  __shared__ double sh[kRedThreads];
  const int64_t bh = blockIdx.x;
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kRedThreads) s += (double)row_kl[bh * n + i];
  const double tot = block_sum(s, sh);
  float w = W.w[0];
#pragma unroll
  for (int k = 1; k < kMaxMaps; ++k)
    if (k < W.nmaps && bh >= W.head0[k]) w = W.w[k];
  if (threadIdx.x == 0) partials[bh] = W.nmaps == 1 ? tot : (double)w * tot;
}

__global__ __launch_bounds__(kRedThreads) void reduce_final_kernel(const double* partials, int64_t bh, int n,
                                                                  float loss_scale, float* loss) {
  __shared__ double sh[kRedThreads];
  double s = 0.0;
  for (int64_t k = threadIdx.x; k < bh; k += kRedThreads) s += partials[k];
  const double tot = block_sum(s, sh);
  if (threadIdx.x == 0) *loss = (float)(tot * (double)loss_scale / (double)n);
}

__global__ void zero_scalar_kernel(float* p) { *p = 0.f; }

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
inline int blocks_per_head(int n, int nw) { return (n + 32 * nw - 1) / (32 * nw); }

MapSet single(const SweepArgs& a) {
  MapSet s{};
  s.map[0] = a;
  s.head0[0] = 0;
  s.head0[1] = a.bh;
  s.nmaps = 1;
  return s;
}

template <int D, bool KL>
hipError_t lse_typed(const MapSet& s, hipStream_t st) {
  const int64_t heads = s.head0[s.nmaps];
  const int nbw = blocks_per_head(s.map[0].n, LMR_W_LSE_WIDE);
  if ((!KL || LMR_LSE_WIDE_KL) && (int64_t)nbw * heads >= LMR_LSE_WIDE_MIN_GRID) {
    constexpr int NW = LMR_W_LSE_WIDE;
    hipLaunchKernelGGL((lse_fwd_kernel<D, KL, NW, LMR_SW_LSE_WIDE>), dim3((unsigned)(nbw * heads)), dim3(64 * NW), 0,
                       st, s, nbw);
  } else {
    constexpr int NW = LMR_W_LSE;
    const int nb = blocks_per_head(s.map[0].n, NW);
    hipLaunchKernelGGL((lse_fwd_kernel<D, KL, NW, LMR_SW_LSE>), dim3((unsigned)(nb * heads)), dim3(64 * NW), 0, st,
                       s, nb);
  }
  return hipGetLastError();
}

template <int D, int ROLE>
hipError_t sweep_typed(const MapSet& s, hipStream_t st) {
  constexpr int NW = ROLE == ROLE_ROW ? LMR_W_ROW : LMR_W_COL;
  constexpr int SW = ROLE == ROLE_ROW ? LMR_SW_ROW : LMR_SW_COL;
  const SweepArgs& a = s.map[0];
  const int nb = blocks_per_head(a.n, NW);
  const dim3 grid((unsigned)(nb * s.head0[s.nmaps])), block(64 * NW);
  const bool contract = ROLE == ROLE_COL && a.cross ? a.dy != nullptr : a.dx != nullptr;
  if (contract)
    hipLaunchKernelGGL((kl_sweep_kernel<D, ROLE, true, NW, SW>), grid, block, 0, st, s, nb);
  else
    hipLaunchKernelGGL((kl_sweep_kernel<D, ROLE, false, NW, SW>), grid, block, 0, st, s, nb);
  return hipGetLastError();
}

template <int D>
hipError_t fused_typed(const MapSet& s, hipStream_t st) {
  constexpr int NW = LMR_W_ROW, SW = LMR_SW_ROW;
  const int nb = blocks_per_head(s.map[0].n, NW);
  hipLaunchKernelGGL((kl_fused_kernel<D, NW, SW>), dim3((unsigned)(nb * s.head0[s.nmaps])), dim3(64 * NW), 0, st, s,
                     nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_fwd(const SweepArgs& a, hipStream_t st) {
  if (a.fp32) return launch_wide_lse_fwd(a, st);
  return launch_lse_fwd_multi(single(a), st);
}

hipError_t launch_kl_fwd(const SweepArgs& a, hipStream_t st) {
  if (a.fp32) {
    // Precision mode: the fp64 phase-1 and row-KL kernels, without gradient.
    hipError_t e = launch_wide_lse_fwd(a, st);
    if (e != hipSuccess) return e;
    SweepArgs b = a;
    b.dx = nullptr;
    b.dy = nullptr;
    return launch_wide_kl_row(b, st);
  }
  return launch_kl_fwd_multi(single(a), st);
}

hipError_t launch_kl_row(const SweepArgs& a, hipStream_t st) {
  if (a.fp32) return launch_wide_kl_row(a, st);
  return launch_kl_row_multi(single(a), st);
}

hipError_t launch_kl_col(const SweepArgs& a, hipStream_t st) {
  // The column term only exists with a gradient; without one there is nothing to do.
  if ((a.cross ? a.dy : a.dx) == nullptr) return hipSuccess;
  if (a.fp32) return launch_wide_kl_col(a, st);
  return launch_kl_col_multi(single(a), st);
}

hipError_t launch_kl_fused(const SweepArgs& a, hipStream_t st) { return launch_kl_fused_multi(single(a), st); }

hipError_t launch_kl_fused_multi(const MapSet& s, hipStream_t st) {
  return s.map[0].d == 64 ? fused_typed<64>(s, st) : fused_typed<128>(s, st);
}

hipError_t launch_lse_fwd_multi(const MapSet& s, hipStream_t st) {
  return s.map[0].d == 64 ? lse_typed<64, false>(s, st) : lse_typed<128, false>(s, st);
}

hipError_t launch_kl_fwd_multi(const MapSet& s, hipStream_t st) {
  return s.map[0].d == 64 ? lse_typed<64, true>(s, st) : lse_typed<128, true>(s, st);
}

hipError_t launch_kl_row_multi(const MapSet& s, hipStream_t st) {
  return s.map[0].d == 64 ? sweep_typed<64, ROLE_ROW>(s, st) : sweep_typed<128, ROLE_ROW>(s, st);
}

hipError_t launch_kl_col_multi(const MapSet& s, hipStream_t st) {
  const SweepArgs& a = s.map[0];
  if ((a.cross ? a.dy : a.dx) == nullptr) return hipSuccess;
  return a.d == 64 ? sweep_typed<64, ROLE_COL>(s, st) : sweep_typed<128, ROLE_COL>(s, st);
}

hipError_t launch_reduce(const float* row_kl, int64_t bh, int n, float loss_scale, double* partials,
                         float* loss, hipStream_t st) {
  HeadWeights W{};
  W.head0[0] = 0;
  W.head0[1] = bh;
  W.w[0] = 1.f;
  W.nmaps = 1;
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)bh), dim3(kRedThreads), 0, st, row_kl, n, partials, W);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_final_kernel, dim3(1), dim3(kRedThreads), 0, st, partials, bh, n, loss_scale, loss);
  return hipGetLastError();
}

hipError_t launch_reduce_weighted(const float* row_kl, const int64_t* head0, const float* weight, int nmaps,
                                  int n, float loss_scale, double* partials, float* loss, hipStream_t st) {
  HeadWeights W{};
  for (int m = 0; m <= nmaps; ++m) W.head0[m] = head0[m];
  for (int m = 0; m < nmaps; ++m) W.w[m] = weight[m];
  W.nmaps = nmaps;
  const int64_t bh = head0[nmaps];
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)bh), dim3(kRedThreads), 0, st, row_kl, n, partials, W);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_final_kernel, dim3(1), dim3(kRedThreads), 0, st, partials, bh, n, loss_scale, loss);
  return hipGetLastError();
}

hipError_t launch_zero_scalar(float* loss, hipStream_t st) {
  hipLaunchKernelGGL(zero_scalar_kernel, dim3(1), dim3(1), 0, st, loss);
  return hipGetLastError();
}

}  // namespace lmr
