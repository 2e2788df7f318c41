// gfx950 (CDNA4) kernels of the linear-memory relation-KL path.
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
//   * A workgroup of W waves "owns" 32*W consecutive rows of one head; wave w
//     owns 32 of them.  The owned rows' projections sit in registers as MFMA
//     B operands for the whole sweep.
//   * The other index ("swept") advances in tiles of SW rows that are staged
//     through LDS (row-major, 16-byte XOR swizzle) and shared by all waves.
//   * Logit tiles are computed swept-major: C[swept][owned] =
//     sum_k X[swept][k] X[owned][k] with v_mfma_f32_32x32x16_bf16, so each
//     lane holds one owned index and 16 swept indices per 32x32 block.
//     Row statistics therefore reduce inside a lane; a lane pair (l, l^32)
//     is combined once at the end.
//   * The gradient contraction  out^T[d][owned] += sum_swept
//     X_s[swept][d] * dZ'[swept][owned]  takes dZ' straight from the logit
//     accumulators as the B operand: the 8 swept values a lane holds per
//     16-step are exactly one B fragment under a fixed permutation of k, and
//     the A operand X_s^T is read from a transposed LDS copy with the same
//     permutation.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr double kLog2eD = 1.4426950408889634074;
constexpr double kLn2D = 0.69314718055994530942;

// Row statistic in log2 units split as hi + lo (hi = the fp32 rounding).
// Phase 2 forms exp2(z*c - hi) with one fma, exact to fp32 rounding of the
// (small) result for the dominant entries, and applies 2^-lo as a per-row
// factor on the probabilities that feed dZ.
__device__ inline void split_stat(double lse_nat, float& hi, float& w) {
  const double l2 = lse_nat * kLog2eD;
  hi = (float)l2;
  w = exp2f(-(float)(l2 - (double)hi));
}

enum : int { ROLE_ROW = 0, ROLE_COL = 1 };

// ---------------------------------------------------------------------------
// Element policies: one MFMA "k-step" consumes 16 k values; a lane in half h
// (h = lane / 32) supplies the 8 values k = 16*ks + 8*h + e, e = 0..7.
// ---------------------------------------------------------------------------
template <typename T> struct Ops;

template <> struct Ops<uint16_t> {           // bf16 storage (fp32 inputs use wide.hip)
  using Frag = bf16x8;
  using Group = bf16x4;
  __device__ static inline f32x16 mma(const Frag& a, const Frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline Frag pack(const float* v) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (__bf16)v[e];
    return f;
  }
  __device__ static inline Frag join(const Group& lo, const Group& hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// Row-major LDS tile of ROWS x D elements; 16-byte chunks XOR-swizzled so the
// 16 rows read together by a fragment load hit 16 distinct bank groups.
template <typename T, int D>
struct RowTile {
  static constexpr int RB = D * (int)sizeof(T);          // bytes per row
  static constexpr int CPR = RB / 16;                    // 16-byte chunks per row
  static constexpr int RSH = RB >= 256 ? 0 : 1;          // 128-byte rows: two per bank line
  static constexpr int CMASK = (CPR < 16 ? CPR : 16) - 1;
  static_assert(RB == 128 || RB == 256, "row size");
  __device__ static inline int off(int r, int c) { return r * RB + ((c ^ ((r >> RSH) & CMASK)) << 4); }
  __device__ static inline typename Ops<T>::Frag frag(const char* base, int r, int ks, int h) {
    return *reinterpret_cast<const bf16x8*>(base + off(r, 2 * ks + h));
  }
};

// Transposed LDS copy [D][SW] of a swept tile: 4-element groups of
// consecutive swept rows, XOR-swizzled per d so 32 lanes reading 32 d-rows
// at the same group are conflict free.
template <typename T, int D, int SW>
struct ColTile {
  static constexpr int TRB = SW * (int)sizeof(T);        // bytes per d-row
  static constexpr int GB = 4 * (int)sizeof(T);          // bytes per group
  static constexpr int GMASK = SW / 4 - 1;
  static constexpr int RSH = TRB >= 256 ? 0 : 1;
  static_assert(SW == 64, "swept tile");
  __device__ static inline int off(int d, int g) { return d * TRB + ((g ^ ((d >> RSH) & GMASK)) * GB); }
  // A fragment for 16-step q: swept rows 16q + 4h + 0..3 and 16q + 8 + 4h + 0..3
  __device__ static inline typename Ops<T>::Frag frag(const char* base, int d, int q, int h) {
    using G = typename Ops<T>::Group;
    const G lo = *reinterpret_cast<const G*>(base + off(d, 4 * q + h));
    const G hi = *reinterpret_cast<const G*>(base + off(d, 4 * q + 2 + h));
    return Ops<T>::join(lo, hi);
  }
};

// Owned-row fragment straight from global memory (row pointer may be null = zeros).
template <typename T>
__device__ inline typename Ops<T>::Frag load_own(const char* row, int ks, int h) {
  using F = typename Ops<T>::Frag;
  if (row == nullptr) return F{};
  return *reinterpret_cast<const bf16x8*>(row + (16 * ks + 8 * h) * (int)sizeof(T));
}

// Global -> registers -> LDS staging of one swept tile of X_t and X_s.
template <typename T, int D, int SW, int NT>
struct Stager {
  static constexpr int RB = D * (int)sizeof(T);
  static constexpr int CPR = RB / 16;
  static constexpr int CPT = SW * CPR / NT;               // chunks per thread per matrix
  static constexpr int EPC = 16 / (int)sizeof(T);         // elements per chunk
  static_assert(SW * CPR % NT == 0, "staging split");
  uint4 t[CPT], s[CPT];

  __device__ inline void load(const char* xt, const char* xs, int row0, int n, int tid) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = tid + NT * u, r = q / CPR, c = q % CPR, g = row0 + r;
      if (g < n) {
        t[u] = *reinterpret_cast<const uint4*>(xt + (int64_t)g * RB + c * 16);
        s[u] = *reinterpret_cast<const uint4*>(xs + (int64_t)g * RB + c * 16);
      } else {
        t[u] = make_uint4(0, 0, 0, 0);
        s[u] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ inline void store(char* lt, char* ls, char* lsT, int tid) const {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = tid + NT * u, r = q / CPR, c = q % CPR;
      *reinterpret_cast<uint4*>(lt + RowTile<T, D>::off(r, c)) = t[u];
      *reinterpret_cast<uint4*>(ls + RowTile<T, D>::off(r, c)) = s[u];
      if (lsT != nullptr) {
        const T* e = reinterpret_cast<const T*>(&s[u]);
#pragma unroll
        for (int k = 0; k < EPC; ++k)
          *reinterpret_cast<T*>(lsT + ColTile<T, D, SW>::off(c * EPC + k, r >> 2) + (r & 3) * (int)sizeof(T)) = e[k];
      }
    }
  }
};

// Both logit tiles of one swept LDS tile against the wave's owned rows.
template <typename T, int D, int SW>
__device__ inline void logits(const char* lt, const char* ls, const typename Ops<T>::Frag* Bt,
                              const typename Ops<T>::Frag* Bs, f32x16* St, f32x16* Ss, int lane) {
  constexpr int KS = D / 16, MB = SW / 32;
  const int h = lane >> 5, rr = lane & 31;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    St[mb] = f32x16{};
    Ss[mb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      St[mb] = Ops<T>::mma(RowTile<T, D>::frag(lt, 32 * mb + rr, ks, h), Bt[ks], St[mb]);
      Ss[mb] = Ops<T>::mma(RowTile<T, D>::frag(ls, 32 * mb + rr, ks, h), Bs[ks], Ss[mb]);
    }
  }
}

// Swept offset (within a tile) of accumulator element r of block mb for lane half h.
__device__ inline int swept_of(int mb, int r, int h) { return 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3); }

// ---------------------------------------------------------------------------
// Phase 1: per-row LSE of teacher and student (row-owned sweep).
// ---------------------------------------------------------------------------
template <typename T, int D, int W, int SW>
__global__ __launch_bounds__(W * 64) void lse_fwd_kernel(SweepArgs a, int nblk) {
  constexpr int NT = W * 64, OWN = 32 * W, KS = D / 16, MB = SW / 32;
  constexpr int RB = D * (int)sizeof(T);
  using Frag = typename Ops<T>::Frag;
  __shared__ __attribute__((aligned(16))) char lt[SW * RB];
  __shared__ __attribute__((aligned(16))) char ls[SW * RB];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const int64_t bid = blockIdx.x;
  const int64_t bh = bid % a.bh;
  const int ob = nblk - 1 - (int)(bid / a.bh);          // longest rows first
  const int n = a.n;
  const char* xt = static_cast<const char*>(a.xt) + bh * (int64_t)n * RB;
  const char* xs = static_cast<const char*>(a.xs) + bh * (int64_t)n * RB;
  const int own0 = ob * OWN, wown0 = own0 + 32 * wave, i = wown0 + (lane & 31);

  Frag Bt[KS], Bs[KS];
  {
    const char* rt = i < n ? xt + (int64_t)i * RB : nullptr;
    const char* rs = i < n ? xs + (int64_t)i * RB : nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) { Bt[ks] = load_own<T>(rt, ks, h); Bs[ks] = load_own<T>(rs, ks, h); }
  }
  const int last = a.causal ? min(own0 + OWN, n) - 1 : n - 1;
  const int ntiles = last / SW + 1;
  const float c = a.scale * kLog2e;
  float mt = -INFINITY, lsum_t = 0.f, ms = -INFINITY, lsum_s = 0.f;

  Stager<T, D, SW, NT> stg;
  stg.load(xt, xs, 0, n, tid);
  for (int tI = 0; tI < ntiles; ++tI) {
    const int sw0 = tI * SW;
    __syncthreads();
    stg.store(lt, ls, nullptr, tid);
    __syncthreads();
    if (tI + 1 < ntiles) stg.load(xt, xs, sw0 + SW, n, tid);
    if (a.causal && sw0 > wown0 + 31) continue;          // tile fully above the diagonal
    const bool need_mask = (a.causal && sw0 + SW - 1 > wown0) || (sw0 + SW > n);

    f32x16 St[MB], Ss[MB];
    logits<T, D, SW>(lt, ls, Bt, Bs, St, Ss, lane);
    float tmt = -INFINITY, tms = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (need_mask) {
          const int j = sw0 + swept_of(mb, r, h);
          const bool ok = (!a.causal || j <= i) && j < n;
          St[mb][r] = ok ? St[mb][r] : -INFINITY;
          Ss[mb][r] = ok ? Ss[mb][r] : -INFINITY;
        }
        tmt = fmaxf(tmt, St[mb][r]);
        tms = fmaxf(tms, Ss[mb][r]);
      }
    }
    const float mnt = fmaxf(mt, tmt), mns = fmaxf(ms, tms);
    const float mct = mnt == -INFINITY ? 0.f : mnt * c;
    const float mcs = mns == -INFINITY ? 0.f : mns * c;
    float at = 0.f, as = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        at += __builtin_amdgcn_exp2f(fmaf(St[mb][r], c, -mct));
        as += __builtin_amdgcn_exp2f(fmaf(Ss[mb][r], c, -mcs));
      }
    }
    lsum_t = lsum_t * __builtin_amdgcn_exp2f(fmaf(mt, c, -mct)) + at;
    lsum_s = lsum_s * __builtin_amdgcn_exp2f(fmaf(ms, c, -mcs)) + as;
    mt = mnt;
    ms = mns;
  }
  // Combine the two lane halves that share owned row i.
  const float mt2 = __shfl_xor(mt, 32), lt2 = __shfl_xor(lsum_t, 32);
  const float ms2 = __shfl_xor(ms, 32), ls2 = __shfl_xor(lsum_s, 32);
  const float Mt = fmaxf(mt, mt2), Ms = fmaxf(ms, ms2);
  const float Mct = Mt * c, Mcs = Ms * c;
  const float Lt = lsum_t * __builtin_amdgcn_exp2f(fmaf(mt, c, -Mct)) + lt2 * __builtin_amdgcn_exp2f(fmaf(mt2, c, -Mct));
  const float Ls = lsum_s * __builtin_amdgcn_exp2f(fmaf(ms, c, -Mcs)) + ls2 * __builtin_amdgcn_exp2f(fmaf(ms2, c, -Mcs));
  // LSE = ln2 * (M*c + log2 L), assembled in fp64 from the fp32 shift that
  // the exponentials above actually used, so the stored statistic carries no
  // rounding of M*c.
  if (h == 0 && i < n) {
    static_cast<double*>(a.lse_t)[bh * n + i] = ((double)Mct + (double)log2f(Lt)) * kLn2D;
    static_cast<double*>(a.lse_s)[bh * n + i] = ((double)Mcs + (double)log2f(Ls)) * kLn2D;
  }
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
// from its off-diagonal probability sums.  The probability of a dominant
// diagonal is ~1 and its fp32 rounding (~6e-8) would otherwise swamp the
// vanishing gradient of very peaky rows; the off-diagonal sums carry no
// such cancellation.
//
// Probabilities: p = exp2(z*c - hi) and the true probability is p * w with
// w = 2^-lo per row (split_stat).  The row sweep forms dZ/w_s(i) =
// p_s - p_t * (w_t/w_s) and scales its accumulator by w_s(i) once; the column
// sweep forms (p_s - p_t * w_t/w_s) * w_s per entry.  Identical teacher and
// student inputs therefore give exactly zero.
// ---------------------------------------------------------------------------
template <typename T, int D, int W, int SW, int ROLE, bool WITH_DX>
__global__ __launch_bounds__(W * 64) void kl_sweep_kernel(SweepArgs a, int nblk) {
  constexpr int NT = W * 64, OWN = 32 * W, KS = D / 16, MB = SW / 32, DB = D / 32;
  constexpr int RB = D * (int)sizeof(T);
  using Frag = typename Ops<T>::Frag;
  __shared__ __attribute__((aligned(16))) char lt[SW * RB];
  __shared__ __attribute__((aligned(16))) char ls[SW * RB];
  __shared__ __attribute__((aligned(16))) char lsT[WITH_DX ? D * SW * (int)sizeof(T) : 16];
  // COL: per swept row hi_t, hi_s, w_t/w_s, w_s (see split_stat)
  __shared__ __attribute__((aligned(16))) float llse[ROLE == ROLE_COL ? 4 * SW : 4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const int64_t bid = blockIdx.x;
  const int64_t bh = bid % a.bh;
  const int ob = ROLE == ROLE_ROW ? nblk - 1 - (int)(bid / a.bh) : (int)(bid / a.bh);
  const int n = a.n;
  const char* xt = static_cast<const char*>(a.xt) + bh * (int64_t)n * RB;
  const char* xs = static_cast<const char*>(a.xs) + bh * (int64_t)n * RB;
  const int own0 = ob * OWN, wown0 = own0 + 32 * wave, o = wown0 + (lane & 31);
  const float c = a.scale * kLog2e;

  Frag Bt[KS], Bs[KS];
  {
    const char* rt = o < n ? xt + (int64_t)o * RB : nullptr;
    const char* rs = o < n ? xs + (int64_t)o * RB : nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) { Bt[ks] = load_own<T>(rt, ks, h); Bs[ks] = load_own<T>(rs, ks, h); }
  }
  float l2t = 0.f, l2s = 0.f, wts = 1.f, ws = 1.f;      // owned-row statistics (ROW)
  if (ROLE == ROLE_ROW && o < n) {
    float wt;
    split_stat(static_cast<const double*>(a.lse_t)[bh * n + o], l2t, wt);
    split_stat(static_cast<const double*>(a.lse_s)[bh * n + o], l2s, ws);
    wts = wt / ws;
  }
  int t_begin, t_end;
  if (ROLE == ROLE_ROW) {
    t_begin = 0;
    t_end = (a.causal ? min(own0 + OWN, n) - 1 : n - 1) / SW + 1;
  } else {
    t_begin = a.causal ? own0 / SW : 0;
    t_end = (n - 1) / SW + 1;
  }

  // Row KL in log2 units, accumulated against the stored statistics and
  // renormalised at the end by the row sums of both probability rows, so a
  // rounding error of a stored LSE (a constant shift of the row) cancels.
  // off_t/off_s: off-diagonal probability sums; pd_t/pd_s: diagonal ones.
  float kl = 0.f, off_t = 0.f, off_s = 0.f, pd_t = 0.f, pd_s = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  Stager<T, D, SW, NT> stg;
  stg.load(xt, xs, t_begin * SW, n, tid);
  for (int tI = t_begin; tI < t_end; ++tI) {
    const int sw0 = tI * SW;
    __syncthreads();
    stg.store(lt, ls, WITH_DX ? lsT : nullptr, tid);
    if (ROLE == ROLE_COL && tid < SW) {
      const int g = sw0 + tid;
      float ht = 0.f, hs = 0.f, ft = 1.f, fs = 1.f;
      if (g < n) {
        split_stat(static_cast<const double*>(a.lse_t)[bh * n + g], ht, ft);
        split_stat(static_cast<const double*>(a.lse_s)[bh * n + g], hs, fs);
      }
      llse[tid] = ht;
      llse[SW + tid] = hs;
      llse[2 * SW + tid] = ft / fs;
      llse[3 * SW + tid] = fs;
    }
    __syncthreads();
    if (tI + 1 < t_end) stg.load(xt, xs, sw0 + SW, n, tid);
    bool skip, need_mask;
    if (ROLE == ROLE_ROW) {
      skip = a.causal && sw0 > wown0 + 31;
      need_mask = (a.causal && sw0 + SW - 1 > wown0) || (sw0 + SW > n);
    } else {
      skip = a.causal && wown0 > sw0 + SW - 1;
      need_mask = (a.causal && wown0 + 31 > sw0) || (sw0 + SW > n);
    }
    if (skip) continue;
    // Tiles that hold a diagonal entry of this wave take the per-entry path too.
    const bool special = need_mask || (sw0 <= wown0 + 31 && sw0 + SW - 1 >= wown0);

    f32x16 St[MB], Ss[MB];
    logits<T, D, SW>(lt, ls, Bt, Bs, St, Ss, lane);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 lt4, ls4, rr4, ws4;
        if (ROLE == ROLE_COL) {
          const int rr = 32 * mb + 8 * g4 + 4 * h;
          lt4 = *reinterpret_cast<const f32x4*>(&llse[rr]);
          ls4 = *reinterpret_cast<const f32x4*>(&llse[SW + rr]);
          rr4 = *reinterpret_cast<const f32x4*>(&llse[2 * SW + rr]);
          ws4 = *reinterpret_cast<const f32x4*>(&llse[3 * SW + rr]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          const float bt = ROLE == ROLE_ROW ? l2t : lt4[e];
          const float bs = ROLE == ROLE_ROW ? l2s : ls4[e];
          float at = fmaf(St[mb][r], c, -bt);
          float as = fmaf(Ss[mb][r], c, -bs);
          float pt = __builtin_amdgcn_exp2f(at);
          float ps = __builtin_amdgcn_exp2f(as);
          bool offdiag = true;
          if (special) {
            const int sw = sw0 + swept_of(mb, r, h);
            const int ii = ROLE == ROLE_ROW ? o : sw;
            const int jj = ROLE == ROLE_ROW ? sw : o;
            const bool ok = (!a.causal || jj <= ii) && sw < n;
            const bool diag = ok && sw == o;
            pt = ok ? pt : 0.f;
            ps = ok ? ps : 0.f;
            at = ok ? at : 0.f;
            as = ok ? as : 0.f;
            if (ROLE == ROLE_ROW) {
              pd_t = diag ? pt : pd_t;
              pd_s = diag ? ps : pd_s;
            }
            offdiag = !diag;
          }
          if (ROLE == ROLE_ROW) {
            kl = fmaf(pt, at - as, kl);
            off_t += offdiag ? pt : 0.f;
            off_s += offdiag ? ps : 0.f;
          }
          // dZ * n in place (see the kernel comment for the 2^-lo factors).
          float dz = ROLE == ROLE_ROW ? fmaf(-pt, wts, ps) : fmaf(-pt, rr4[e], ps) * ws4[e];
          St[mb][r] = offdiag ? dz : 0.f;
        }
      }
    }
    if constexpr (WITH_DX) {
#pragma unroll
      for (int q = 0; q < SW / 16; ++q) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = St[q >> 1][8 * (q & 1) + e];
        const Frag bdz = Ops<T>::pack(v);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = Ops<T>::mma(ColTile<T, D, SW>::frag(lsT, 32 * db + (lane & 31), q, h), bdz, acc[db]);
      }
    }
  }

  float corr = 0.f;                                      // ROW: -2 * sum_{j!=i} dZ(i,j) / w_s(i) * n
  if (ROLE == ROLE_ROW) {
    kl += __shfl_xor(kl, 32);
    off_t += __shfl_xor(off_t, 32);
    off_s += __shfl_xor(off_s, 32);
    pd_t += __shfl_xor(pd_t, 32);
    pd_s += __shfl_xor(pd_s, 32);
    const float sum_t = off_t + pd_t, sum_s = off_s + pd_s;
    // KL = sum_j r_t (log2 r_t - log2 r_s) ln2 with r = p / sum p.
    const float klr = kl / sum_t - log2f(sum_t) + log2f(sum_s);
    if (h == 0 && o < n && a.row_kl != nullptr) a.row_kl[bh * n + o] = klr * kLn2;
    corr = -2.f * fmaf(-off_t, wts, off_s);
  }
  if constexpr (WITH_DX) {
    if (o < n) {
      float* dst = a.dx + (bh * (int64_t)n + o) * D;
      const T* xo = reinterpret_cast<const T*>(xs + (int64_t)o * RB);
      const float gs = ROLE == ROLE_ROW ? a.grad_scale * ws : a.grad_scale;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * db + 8 * g4 + 4 * h;
          f32x4 v;
          if (ROLE == ROLE_ROW) {
            const uint2 raw = *reinterpret_cast<const uint2*>(xo + d0);   // 4 bf16 of x_s[i]
            const float x4[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                                 __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
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

__global__ __launch_bounds__(kRedThreads) void reduce_rows_kernel(const float* row_kl, int n, double* partials) {
  __shared__ double sh[kRedThreads];
  const int64_t bh = blockIdx.x;
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kRedThreads) s += (double)row_kl[bh * n + i];
  const double tot = block_sum(s, sh);
  if (threadIdx.x == 0) partials[bh] = tot;
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
constexpr int kW = 4;       // waves per workgroup
constexpr int kSW = 64;     // swept tile rows
constexpr int kOwn = 32 * kW;

inline int blocks_per_head(int n) { return (n + kOwn - 1) / kOwn; }

template <typename T, int D>
hipError_t lse_typed(const SweepArgs& a, hipStream_t st) {
  const int nb = blocks_per_head(a.n);
  hipLaunchKernelGGL((lse_fwd_kernel<T, D, kW, kSW>), dim3((unsigned)(nb * a.bh)), dim3(64 * kW), 0, st, a, nb);
  return hipGetLastError();
}

template <typename T, int D, int ROLE>
hipError_t sweep_typed(const SweepArgs& a, hipStream_t st) {
  const int nb = blocks_per_head(a.n);
  const dim3 grid((unsigned)(nb * a.bh)), block(64 * kW);
  if (a.dx != nullptr)
    hipLaunchKernelGGL((kl_sweep_kernel<T, D, kW, kSW, ROLE, true>), grid, block, 0, st, a, nb);
  else
    hipLaunchKernelGGL((kl_sweep_kernel<T, D, kW, kSW, ROLE, false>), grid, block, 0, st, a, nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_fwd(const SweepArgs& a, hipStream_t st) {
  if (a.fp32) return launch_wide_lse_fwd(a, st);
  return a.d == 64 ? lse_typed<uint16_t, 64>(a, st) : lse_typed<uint16_t, 128>(a, st);
}

hipError_t launch_kl_row(const SweepArgs& a, hipStream_t st) {
  if (a.fp32) return launch_wide_kl_row(a, st);
  return a.d == 64 ? sweep_typed<uint16_t, 64, ROLE_ROW>(a, st) : sweep_typed<uint16_t, 128, ROLE_ROW>(a, st);
}

hipError_t launch_kl_col(const SweepArgs& a, hipStream_t st) {
  if (a.fp32) return launch_wide_kl_col(a, st);
  return a.d == 64 ? sweep_typed<uint16_t, 64, ROLE_COL>(a, st) : sweep_typed<uint16_t, 128, ROLE_COL>(a, st);
}

hipError_t launch_reduce(const float* row_kl, int64_t bh, int n, float loss_scale, double* partials,
                         float* loss, hipStream_t st) {
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)bh), dim3(kRedThreads), 0, st, row_kl, n, partials);
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
