// fp32-input path of the linear-memory relation-KL: the same two phases as
// the bf16 MFMA kernels ("LinearARD: Linear-Memory Attention Distillation
// for RoPE Restoration", paper-notes page, section "Key designs", item 3:
// per-row LSE statistics, then a recompute sweep that rebuilds R_t, R_s and
// contracts dZ = (R_s - R_t)/n), computed in fp64 on the vector ALUs.
//
// Why fp64: every row of dZ sums to zero, so dZ X_s is a small difference of
// two weighted means of the rows of X_s.  fp32 logits and an fp32-rounded LSE
// already move it by ~1e-4 (normwise) on RoPE inputs, so this precision mode
// keeps logits, probabilities, statistics (fp64 LSE buffers) and the
// gradient accumulators in fp64 and rounds only the final outputs to fp32.
// It is a precision mode for small inputs, not a throughput path.
//
// Layout: a workgroup owns WR rows of one head; each owned row is served by
// WS consecutive lanes, each holding D/WS of its components.  Swept rows are
// staged through LDS in tiles of WT rows; every dot product is a partial sum
// per lane followed by a 3-step butterfly across the WS lanes of the row.
#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace lmr {
namespace {

constexpr int WR = 32;                 // owned rows per workgroup
constexpr int WS = 8;                  // lanes per owned row
constexpr int WT = 32;                 // swept rows per LDS tile
constexpr int WTHREADS = WR * WS;      // 256

enum : int { WROW = 0, WCOL = 1 };

__device__ inline double row_sum(double v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  return v;
}

template <int D>
__device__ inline void stage(float (*lt)[D], float (*ls)[D], const float* xt, const float* xs, int row0, int n,
                             int tid) {
  for (int e = tid; e < WT * D; e += WTHREADS) {
    const int r = e / D, k = e % D, g = row0 + r;
    lt[r][k] = g < n ? xt[(int64_t)g * D + k] : 0.f;
    ls[r][k] = g < n ? xs[(int64_t)g * D + k] : 0.f;
  }
}

template <int D>
__global__ __launch_bounds__(WTHREADS) void wide_lse_kernel(SweepArgs a, int nblk) {
  constexpr int KD = D / WS;
  __shared__ float lt[WT][D];
  __shared__ float ls[WT][D];
  const int tid = threadIdx.x, r = tid / WS, q = tid % WS;
  const int64_t bid = blockIdx.x, bh = bid % a.bh;
  const int ob = nblk - 1 - (int)(bid / a.bh);
  const int n = a.n, i = ob * WR + r;
  const float* xt = static_cast<const float*>(a.xt) + bh * (int64_t)n * D;
  const float* xs = static_cast<const float*>(a.xs) + bh * (int64_t)n * D;
  const float* yt = static_cast<const float*>(a.yt) + bh * (int64_t)n * D;   // swept (== x for a self-relation)
  const float* ys = static_cast<const float*>(a.ys) + bh * (int64_t)n * D;
  float ot[KD], os[KD];
#pragma unroll
  for (int k = 0; k < KD; ++k) {
    ot[k] = i < n ? xt[(int64_t)i * D + q * KD + k] : 0.f;
    os[k] = i < n ? xs[(int64_t)i * D + q * KD + k] : 0.f;
  }
  const double s = a.scale;
  const int last = a.causal ? min(ob * WR + WR, n) - 1 : n - 1;
  double mt = -INFINITY, st = 0.0, ms = -INFINITY, ss = 0.0;
  for (int t0 = 0; t0 <= last; t0 += WT) {
    __syncthreads();
    stage<D>(lt, ls, yt, ys, t0, n, tid);
    __syncthreads();
    const int jend = min(t0 + WT, last + 1);
    for (int j = t0; j < jend; ++j) {
      double zt = 0.0, zs = 0.0;
#pragma unroll
      for (int k = 0; k < KD; ++k) {
        zt = fma((double)ot[k], (double)lt[j - t0][q * KD + k], zt);
        zs = fma((double)os[k], (double)ls[j - t0][q * KD + k], zs);
      }
      zt = row_sum(zt) * s;
      zs = row_sum(zs) * s;
      if ((!a.causal || j <= i) && i < n) {
        if (zt > mt) { st = st * exp(mt - zt) + 1.0; mt = zt; } else { st += exp(zt - mt); }
        if (zs > ms) { ss = ss * exp(ms - zs) + 1.0; ms = zs; } else { ss += exp(zs - ms); }
      }
    }
  }
  if (q == 0 && i < n) {
    static_cast<double*>(a.lse_t)[bh * n + i] = mt + log(st);
    static_cast<double*>(a.lse_s)[bh * n + i] = ms + log(ss);
  }
}

template <int D, int ROLE, bool WITH_DX>
__global__ __launch_bounds__(WTHREADS) void wide_sweep_kernel(SweepArgs a, int nblk) {
  constexpr int KD = D / WS;
  __shared__ float lt[WT][D];
  __shared__ float ls[WT][D];
  __shared__ double llt[WT];
  __shared__ double lls[WT];
  const int tid = threadIdx.x, r = tid / WS, q = tid % WS;
  const int64_t bid = blockIdx.x, bh = bid % a.bh;
  const int ob = ROLE == WROW ? nblk - 1 - (int)(bid / a.bh) : (int)(bid / a.bh);
  const int n = a.n, o = ob * WR + r;
  // WROW: owned rows i of X, swept rows j of Y; WCOL: owned rows j of Y,
  // swept rows i of X (X == Y for a self-relation).
  const int64_t hoff = bh * (int64_t)n * D;
  const float* xt = static_cast<const float*>(ROLE == WROW ? a.xt : a.yt) + hoff;
  const float* xs = static_cast<const float*>(ROLE == WROW ? a.xs : a.ys) + hoff;
  const float* wt = static_cast<const float*>(ROLE == WROW ? a.yt : a.xt) + hoff;
  const float* ws = static_cast<const float*>(ROLE == WROW ? a.ys : a.xs) + hoff;
  const double* gl_t = static_cast<const double*>(a.lse_t) + bh * n;
  const double* gl_s = static_cast<const double*>(a.lse_s) + bh * n;
  float ot[KD], os[KD];
#pragma unroll
  for (int k = 0; k < KD; ++k) {
    ot[k] = o < n ? xt[(int64_t)o * D + q * KD + k] : 0.f;
    os[k] = o < n ? xs[(int64_t)o * D + q * KD + k] : 0.f;
  }
  const double s = a.scale;
  const double olt = (ROLE == WROW && o < n) ? gl_t[o] : 0.0;
  const double ols = (ROLE == WROW && o < n) ? gl_s[o] : 0.0;
  int t_begin, t_end;
  if (ROLE == WROW) {
    t_begin = 0;
    t_end = a.causal ? min(ob * WR + WR, n) : n;
  } else {
    t_begin = a.causal ? ob * WR : 0;
    t_end = n;
  }
  double kl = 0.0, sum_t = 0.0, sum_s = 0.0;
  double acc[KD];
#pragma unroll
  for (int k = 0; k < KD; ++k) acc[k] = 0.0;

  for (int t0 = t_begin; t0 < t_end; t0 += WT) {
    __syncthreads();
    stage<D>(lt, ls, wt, ws, t0, n, tid);
    if (ROLE == WCOL && tid < WT) {
      const int g = t0 + tid;
      llt[tid] = g < n ? gl_t[g] : 0.0;
      lls[tid] = g < n ? gl_s[g] : 0.0;
    }
    __syncthreads();
    const int jend = min(t0 + WT, t_end);
    for (int sw = t0; sw < jend; ++sw) {
      const int jj = sw - t0;
      double zt = 0.0, zs = 0.0;
#pragma unroll
      for (int k = 0; k < KD; ++k) {
        zt = fma((double)ot[k], (double)lt[jj][q * KD + k], zt);
        zs = fma((double)os[k], (double)ls[jj][q * KD + k], zs);
      }
      zt = row_sum(zt) * s;
      zs = row_sum(zs) * s;
      const int ii = ROLE == WROW ? o : sw;
      const int cc = ROLE == WROW ? sw : o;
      const bool ok = (!a.causal || cc <= ii) && o < n;
      if (!ok) continue;
      const double at = zt - (ROLE == WROW ? olt : llt[jj]);
      const double as = zs - (ROLE == WROW ? ols : lls[jj]);
      const double pt = exp(at), ps = exp(as);
      if (ROLE == WROW) {
        kl = fma(pt, at - as, kl);
        sum_t += pt;
        sum_s += ps;
      }
      if (WITH_DX) {
        const double dz = ps - pt;
#pragma unroll
        for (int k = 0; k < KD; ++k) acc[k] = fma(dz, (double)ls[jj][q * KD + k], acc[k]);
      }
    }
  }
  if (ROLE == WROW && q == 0 && o < n && a.row_kl != nullptr)
    a.row_kl[bh * n + o] = (float)(kl / sum_t - log(sum_t) + log(sum_s));
  if (WITH_DX && o < n) {
    // The diagonal is an ordinary entry here, so a cross relation's column
    // sweep writes the whole of dY_s; a self-relation's adds to dX_s.
    float* dst = (ROLE == WCOL && a.cross ? a.dy : a.dx) + (bh * (int64_t)n + o) * D + q * KD;
#pragma unroll
    for (int k = 0; k < KD; ++k) {
      const double v = acc[k] * a.grad_scale_d;
      if (ROLE == WROW || a.cross) dst[k] = (float)v;
      else dst[k] = (float)((double)dst[k] + v);
    }
  }
}

inline int wide_blocks(int n) { return (n + WR - 1) / WR; }

template <int ROLE>
hipError_t wide_sweep(const SweepArgs& a, hipStream_t st) {
  const int nb = wide_blocks(a.n);
  const dim3 grid((unsigned)(nb * a.bh)), block(WTHREADS);
  const bool contract = ROLE == WCOL && a.cross ? a.dy != nullptr : a.dx != nullptr;
  if (a.d == 64) {
    if (contract) hipLaunchKernelGGL((wide_sweep_kernel<64, ROLE, true>), grid, block, 0, st, a, nb);
    else hipLaunchKernelGGL((wide_sweep_kernel<64, ROLE, false>), grid, block, 0, st, a, nb);
  } else {
    if (contract) hipLaunchKernelGGL((wide_sweep_kernel<128, ROLE, true>), grid, block, 0, st, a, nb);
    else hipLaunchKernelGGL((wide_sweep_kernel<128, ROLE, false>), grid, block, 0, st, a, nb);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wide_lse_fwd(const SweepArgs& a, hipStream_t st) {
  const int nb = wide_blocks(a.n);
  const dim3 grid((unsigned)(nb * a.bh)), block(WTHREADS);
  if (a.d == 64) hipLaunchKernelGGL(wide_lse_kernel<64>, grid, block, 0, st, a, nb);
  else hipLaunchKernelGGL(wide_lse_kernel<128>, grid, block, 0, st, a, nb);
  return hipGetLastError();
}

hipError_t launch_wide_kl_row(const SweepArgs& a, hipStream_t st) { return wide_sweep<WROW>(a, st); }
hipError_t launch_wide_kl_col(const SweepArgs& a, hipStream_t st) { return wide_sweep<WCOL>(a, st); }

}  // namespace lmr
