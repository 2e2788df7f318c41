// Internal launcher interface between the C ABI (api.cpp) and the gfx950
// kernels (kernels.hip).  Not installed; the public interface is larard.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmr {

// Geometry and arguments of one launch over B*H heads of one relation map.
struct SweepArgs {
  const void* xt;        // [BH, n, d] teacher X, bf16 bits or fp32 (rows i of the relation)
  const void* xs;        // [BH, n, d] student X
  const void* yt;        // [BH, n, d] teacher Y (columns j); == xt for a self-relation
  const void* ys;        // [BH, n, d] student Y; == xs for a self-relation
  int cross;             // 1: Y != X, gradients dX_s and dY_s kept apart
  void* lse_t;           // [BH, n] fp64, natural log
  void* lse_s;           // [BH, n]
  float* row_kl;         // [BH, n]  row KL output (may be null for COL sweeps)
  float* dx;             // [BH, n, d] fp32 gradient dX_s (null = none); self: the whole gradient
  float* dy;             // [BH, n, d] fp32 gradient dY_s (cross only; null = none)
  int64_t bh;            // number of heads B*H
  int n;                 // sequence length
  int d;                 // head dim (64 or 128)
  int fp32;              // 1: fp32 inputs, 0: bf16
  int causal;            // 1: keep j <= i
  float scale;           // logit scale s
  float grad_scale;      // loss_scale * s / n, applied to the dZ contractions
  double grad_scale_d;   // the same factor in fp64 (fp32-input path)
};

// Several relation maps of equal n, d and dtype in one launch (e.g. Q/Q,
// K/K, V/V with their own head counts).  Heads are numbered across maps:
// map m owns heads head0[m] .. head0[m+1]-1 of the launch.
constexpr int kMaxMaps = 8;
struct MapSet {
  SweepArgs map[kMaxMaps];
  int64_t head0[kMaxMaps + 1];
  int nmaps;
};

hipError_t launch_lse_fwd(const SweepArgs& a, hipStream_t st);
// Phase 1 with the KL accumulator: LSE_t, LSE_s and row_kl in one sweep.
hipError_t launch_kl_fwd(const SweepArgs& a, hipStream_t st);
// Row-owned phase-2 sweep: row KL and the row term dZ Y_s (stored, not
// added); cross relations also store the diagonal part of dY_s.
hipError_t launch_kl_row(const SweepArgs& a, hipStream_t st);
// Column-owned phase-2 sweep: adds the column term dZ^T X_s into dx (self)
// or dy (cross).
hipError_t launch_kl_col(const SweepArgs& a, hipStream_t st);
// Fused phase 2 of a self-relation with gradient (bf16): row KL and the whole
// dX_s (row and column terms) stored once; row_kl and dx required, cross == 0.
hipError_t launch_kl_fused(const SweepArgs& a, hipStream_t st);
hipError_t launch_kl_fused_multi(const MapSet& s, hipStream_t st);
// fp32-input path (fp64 arithmetic on the vector ALUs), in wide.hip.
hipError_t launch_wide_lse_fwd(const SweepArgs& a, hipStream_t st);
hipError_t launch_wide_kl_row(const SweepArgs& a, hipStream_t st);
hipError_t launch_wide_kl_col(const SweepArgs& a, hipStream_t st);
// loss = loss_scale/n * sum over heads and rows of row_kl, reduced in fp64
// in a fixed order (deterministic).  partials: [bh] fp64 scratch.
hipError_t launch_reduce(const float* row_kl, int64_t bh, int n, float loss_scale,
                         double* partials, float* loss, hipStream_t st);
// Fused bf16 launches over a map set (row_kl / lse of all maps contiguous,
// map m at head offset head0[m]); every map must have the same kind of
// gradient output (all or none).
hipError_t launch_lse_fwd_multi(const MapSet& s, hipStream_t st);
hipError_t launch_kl_fwd_multi(const MapSet& s, hipStream_t st);
hipError_t launch_kl_row_multi(const MapSet& s, hipStream_t st);
hipError_t launch_kl_col_multi(const MapSet& s, hipStream_t st);
// Weighted reduction: loss = loss_scale/n * sum_m weight[m] * (sum over the
// heads and rows of map m of row_kl).
hipError_t launch_reduce_weighted(const float* row_kl, const int64_t* head0, const float* weight, int nmaps,
                                  int n, float loss_scale, double* partials, float* loss, hipStream_t st);
// Projection backward (proj.hip): dW[dm, H*d] = h^T R^T(dX_s).
struct ProjArgs {
  const uint16_t* h;     // [B*n, dm] bf16 hidden states
  const float* dx;       // [B, H, n, d] fp32 student gradient
  const float* cos;      // [n, d/2] fp32 student rotation tables (null: no rotation)
  const float* sin;
  uint16_t* g;           // workspace: G^T = (R^T dX_s)^T [H*d, kp] bf16 (tokens permuted per 16)
  uint16_t* ht;          // workspace: h^T [dm, kp] bf16, same token order (256-tile path only)
  float* dw;             // [dm, H*d] fp32 output
  int64_t B, n, dm, H, d;
  int64_t kp;            // B*n rounded up to a multiple of 64
};
hipError_t launch_proj_bwd(const ProjArgs& p, hipStream_t st);
// Whether launch_proj_bwd takes the 256 x 256 tile path, which also needs
// the h^T workspace region.
bool proj_uses_256_tiles(int64_t dm, int64_t hd);

// *loss = 0 (used when n == 0).
hipError_t launch_zero_scalar(float* loss, hipStream_t st);

}  // namespace lmr
