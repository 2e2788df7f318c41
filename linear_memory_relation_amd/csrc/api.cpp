// C ABI of liblarard.so (declared in include/larard.h): argument validation,
// workspace carving and kernel dispatch.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "larard.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;
// Fewest rows any sweep kernel assigns to one workgroup (the fp32 kernels own
// 32; the bf16 kernels 128 or 256), so B*H*ceil(n/kOwnRows) bounds every grid.
constexpr int kOwnRows = 32;

larard_status fail(larard_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
larard_status fail(larard_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

larard_status hip_fail(hipError_t e, const char* what) {
  return fail(LARARD_E_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// LSE statistics are fp64 for every input type.
size_t stat_bytes(larard_dtype) { return sizeof(double); }

// Validation shared by every entry point; touches no HIP state.
larard_status check_common(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H,
                           int64_t n, int64_t d, float scale) {
  if (B < 1 || H < 1) return fail(LARARD_E_INVALID, "B and H must be >= 1 (got B=%lld H=%lld)", (long long)B, (long long)H);
  if (n < 0 || n > kMaxN) return fail(LARARD_E_INVALID, "n must be in [0, 2^24] (got %lld)", (long long)n);
  if (B > kMaxGrid / H) return fail(LARARD_E_INVALID, "B*H too large");
  const int64_t bh = B * H;
  const int64_t nblk = (n + kOwnRows - 1) / kOwnRows;
  if (nblk > 0 && bh > kMaxGrid / nblk) return fail(LARARD_E_INVALID, "B*H*ceil(n/32) exceeds the launch grid");
  if (dtype != LARARD_BF16 && dtype != LARARD_FP32) return fail(LARARD_E_UNSUPPORTED, "dtype %d not supported", (int)dtype);
  if (d != 64 && d != 128) return fail(LARARD_E_UNSUPPORTED, "head dim d=%lld not supported (64 or 128)", (long long)d);
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(LARARD_E_INVALID, "scale must be finite and > 0");
  if (n > 0) {
    if (x_t == nullptr || x_s == nullptr) return fail(LARARD_E_INVALID, "x_t / x_s must not be NULL");
    if (!aligned(x_t, 16) || !aligned(x_s, 16)) return fail(LARARD_E_INVALID, "x_t / x_s must be 16-byte aligned");
  }
  return LARARD_OK;
}

lmr::SweepArgs make_args(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H, int64_t n,
                         int64_t d, float scale, int causal) {
  lmr::SweepArgs a{};
  a.xt = x_t;
  a.xs = x_s;
  a.yt = x_t;            // self-relation unless set_cross() replaces Y
  a.ys = x_s;
  a.cross = 0;
  a.bh = B * H;
  a.n = (int)n;
  a.d = (int)d;
  a.fp32 = dtype == LARARD_FP32 ? 1 : 0;
  a.causal = causal ? 1 : 0;
  a.scale = scale;
  return a;
}

// Cross relation: Y tensors of the same shape and dtype as X.
larard_status set_cross(lmr::SweepArgs* a, const void* y_t, const void* y_s, int64_t n) {
  if (n > 0) {
    if (y_t == nullptr || y_s == nullptr) return fail(LARARD_E_INVALID, "y_t / y_s must not be NULL");
    if (!aligned(y_t, 16) || !aligned(y_s, 16)) return fail(LARARD_E_INVALID, "y_t / y_s must be 16-byte aligned");
  }
  a->yt = y_t;
  a->ys = y_s;
  a->cross = 1;
  return LARARD_OK;
}

larard_status check_dx_mode(int dx_mode) {
  if (dx_mode == LARARD_DX_AUTO || dx_mode == LARARD_DX_SPLIT || dx_mode == LARARD_DX_FUSED) return LARARD_OK;
  if (dx_mode == LARARD_DX_ATOMIC) return fail(LARARD_E_UNSUPPORTED, "dx_mode ATOMIC is not built");
  return fail(LARARD_E_INVALID, "unknown dx_mode %d", dx_mode);
}

// Longest sequence for which AUTO takes the fused phase 2.  Measured on
// MI355X (one box, same inputs): fused is 3% faster per step at n = 4K and 2%
// at 8K (GQA), where its equal-length workgroups avoid the split sweeps'
// causal tails, and 1.4% slower at 16K.
constexpr int64_t kFusedMaxN = 8192;

// Whether phase 2 runs as the fused single sweep: bf16 self-relations with a
// gradient, in FUSED mode, or in AUTO mode up to kFusedMaxN.  The fp32
// precision kernels and the cross relation always run split.
bool use_fused(const lmr::SweepArgs& a, int dx_mode) {
  if (a.fp32 || a.cross || a.dx == nullptr) return false;
  return dx_mode == LARARD_DX_FUSED || (dx_mode == LARARD_DX_AUTO && a.n <= kFusedMaxN);
}

// Phase-2 launches (inputs already validated).
larard_status run_kl_bwd(lmr::SweepArgs a, float loss_scale, int dx_mode, hipStream_t st) {
  a.grad_scale = loss_scale * a.scale / (float)a.n;
  a.grad_scale_d = (double)loss_scale * (double)a.scale / (double)a.n;
  if (use_fused(a, dx_mode)) {
    const hipError_t e = lmr::launch_kl_fused(a, st);
    return e == hipSuccess ? LARARD_OK : hip_fail(e, "kl_bwd fused sweep launch");
  }
  hipError_t e = lmr::launch_kl_row(a, st);
  if (e != hipSuccess) return hip_fail(e, "kl_bwd row sweep launch");
  if ((a.cross ? a.dy : a.dx) != nullptr) {
    e = lmr::launch_kl_col(a, st);
    if (e != hipSuccess) return hip_fail(e, "kl_bwd column sweep launch");
  }
  return LARARD_OK;
}

// Whole-path calls (loss with gradient) run phase 1 and phase 2 head group by
// head group (larard.h, larard_loss_head_group): a group's projections are
// then still in the last-level cache when its phase-2 sweeps re-read them.
// Measured on MI355X, ms per step, all heads at once -> grouped: n = 32K
// 105.3 -> 101.7 (split), 107.3 -> 101.8 (fused); at n = 16K one group of
// 32 heads (split 25.7) and two of 16 (25.9) are equal within noise, and
// two groups would cost phase 1 its 12-wave shape, so 16K stays one group.
// Every head's arithmetic is its own, so the results are the same bits
// either way.
#ifndef LMR_GROUP_MIB
#define LMR_GROUP_MIB 256
#endif
constexpr int64_t kGroupBytes = int64_t(LMR_GROUP_MIB) << 20;
// Phase 2 of a group runs in sub-groups of at most this many bytes of
// projections (still at least kGroupGrid workgroups per sweep): the split
// sweeps read them twice, the fused sweep twice within one launch.
// Measured on MI355X, ms per step, phase 2 per group -> per sub-group of
// 128 MiB: n = 16K split 25.70-25.79 -> 25.37-25.49, fused 26.23 -> 25.36-25.54;
// n = 32K fused 102.5-103.1 -> 100.5; GQA 8K fused 6.92-6.94 -> 6.66-6.69;
// 4K unchanged (one sub-group).
#ifndef LMR_GROUP2_MIB
#define LMR_GROUP2_MIB 128
#endif
constexpr int64_t kSweepGroupBytes = int64_t(LMR_GROUP2_MIB) << 20;
#ifndef LMR_GROUP2_GRID
#define LMR_GROUP2_GRID 1024
#endif
constexpr int64_t kGroupGrid = 1024;

int64_t group_of(bool fp32, bool cross, int64_t bh, int64_t n, int64_t d, int64_t budget = kGroupBytes,
                 int64_t grid = kGroupGrid) {
  if (fp32) return bh;
  const int64_t per_head = (cross ? 4 : 2) * n * d * 2;
  const int64_t rows_blk = (n + 255) / 256;
  int64_t g = per_head > 0 ? budget / per_head : bh;
  if (rows_blk > 0) g = std::max(g, (grid + rows_blk - 1) / rows_blk);
  return std::max<int64_t>(1, std::min(g, bh));
}

int64_t head_group(const lmr::SweepArgs& a) { return group_of(a.fp32 != 0, a.cross != 0, a.bh, a.n, a.d); }

// The argument set of heads h0 .. h0+cnt-1 of a (bf16 inputs, fp64 statistics).
lmr::SweepArgs head_slice(const lmr::SweepArgs& a, int64_t h0, int64_t cnt) {
  lmr::SweepArgs g = a;
  const int64_t xo = h0 * a.n * a.d * (a.fp32 ? 4 : 2), ro = h0 * a.n, go = h0 * a.n * a.d;
  g.xt = static_cast<const char*>(a.xt) + xo;
  g.xs = static_cast<const char*>(a.xs) + xo;
  g.yt = static_cast<const char*>(a.yt) + xo;
  g.ys = static_cast<const char*>(a.ys) + xo;
  g.lse_t = static_cast<double*>(a.lse_t) + ro;
  g.lse_s = static_cast<double*>(a.lse_s) + ro;
  g.row_kl = a.row_kl + ro;
  g.dx = a.dx != nullptr ? a.dx + go : nullptr;
  g.dy = a.dy != nullptr ? a.dy + go : nullptr;
  g.bh = cnt;
  return g;
}

// Phase 1 and phase 2 of a whole-path call with a gradient, group by group;
// within a group, phase 2 runs in sub-groups (larard_loss_sweep_group).
larard_status run_grouped(const lmr::SweepArgs& a, float loss_scale, int dx_mode, hipStream_t st) {
  const int64_t g = head_group(a);
  const int64_t g2 = group_of(a.fp32 != 0, a.cross != 0, a.bh, a.n, a.d, kSweepGroupBytes, LMR_GROUP2_GRID);
  for (int64_t h0 = 0; h0 < a.bh; h0 += g) {
    const lmr::SweepArgs part = head_slice(a, h0, std::min(g, a.bh - h0));
    const hipError_t e = lmr::launch_lse_fwd(part, st);
    if (e != hipSuccess) return hip_fail(e, "lse_fwd launch");
    for (int64_t k0 = 0; k0 < part.bh; k0 += g2) {
      const larard_status s = run_kl_bwd(head_slice(part, k0, std::min(g2, part.bh - k0)), loss_scale, dx_mode, st);
      if (s != LARARD_OK) return s;
    }
  }
  return LARARD_OK;
}

// Validation shared by the phase-2 entry points; fills *out on success.
larard_status check_phase2(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H, int64_t n,
                           int64_t d, float scale, int causal, const void* lse_t, const void* lse_s,
                           float loss_scale, lmr::SweepArgs* out) {
  larard_status s = check_common(x_t, x_s, dtype, B, H, n, d, scale);
  if (s != LARARD_OK) return s;
  if (!std::isfinite(loss_scale)) return fail(LARARD_E_INVALID, "loss_scale must be finite");
  if (n == 0) return LARARD_OK;
  if (lse_t == nullptr || lse_s == nullptr) return fail(LARARD_E_INVALID, "lse_t / lse_s must not be NULL");
  if (!aligned(lse_t, stat_bytes(dtype)) || !aligned(lse_s, stat_bytes(dtype)))
    return fail(LARARD_E_INVALID, "lse buffers must be aligned to their element size");
  *out = make_args(x_t, x_s, dtype, B, H, n, d, scale, causal);
  out->lse_t = const_cast<void*>(lse_t);
  out->lse_s = const_cast<void*>(lse_s);
  out->grad_scale = loss_scale * scale / (float)n;
  out->grad_scale_d = (double)loss_scale * (double)scale / (double)n;
  return LARARD_OK;
}

// Validation of larard_loss and its allocation-free variant (no HIP state touched).
larard_status check_loss(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H, int64_t n,
                         int64_t d, float scale, float loss_scale, const float* loss, const float* dx_s,
                         int dx_mode) {
  larard_status s = check_common(x_t, x_s, dtype, B, H, n, d, scale);
  if (s != LARARD_OK) return s;
  if ((s = check_dx_mode(dx_mode)) != LARARD_OK) return s;
  if (!std::isfinite(loss_scale)) return fail(LARARD_E_INVALID, "loss_scale must be finite");
  if (loss == nullptr || !aligned(loss, 4)) return fail(LARARD_E_INVALID, "loss must be a 4-byte aligned device pointer");
  if (dx_s != nullptr && !aligned(dx_s, 16)) return fail(LARARD_E_INVALID, "dx_s must be 16-byte aligned");
  return LARARD_OK;
}

larard_status zero_loss(float* loss, hipStream_t st) {
  const hipError_t e = lmr::launch_zero_scalar(loss, st);
  return e == hipSuccess ? LARARD_OK : hip_fail(e, "zero loss launch");
}

// Whole path of one map on a validated call, with scratch ws (256-byte aligned,
// >= larard_workspace_bytes): phase 1, phase 2 (or the forward-only sweep) and
// the fp64 reduction.  Every scratch byte read is written earlier in the same
// call (LSE and row KL of every row, one partial per head), so ws needs no
// clearing.
larard_status run_loss(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H, int64_t n,
                       int64_t d, float scale, int causal, float loss_scale, char* ws, float* loss, float* dx_s,
                       int dx_mode, hipStream_t st) {
  size_t off[4];
  larard_status s = larard_workspace_layout(dtype, B, H, n, off);
  if (s != LARARD_OK) return s;
  lmr::SweepArgs a = make_args(x_t, x_s, dtype, B, H, n, d, scale, causal);
  a.lse_t = ws + off[0];
  a.lse_s = ws + off[1];
  a.row_kl = reinterpret_cast<float*>(ws + off[2]);
  double* partials = reinterpret_cast<double*>(ws + off[3]);
  hipError_t e;
  if (dx_s == nullptr) {
    // Loss only: LSE and row KL in one phase-1 sweep.
    e = lmr::launch_kl_fwd(a, st);
    if (e != hipSuccess) return hip_fail(e, "kl_fwd launch");
  } else {
    a.dx = dx_s;
    if ((s = run_grouped(a, loss_scale, dx_mode, st)) != LARARD_OK) return s;
  }
  e = lmr::launch_reduce(a.row_kl, a.bh, a.n, loss_scale, partials, loss, st);
  if (e != hipSuccess) return hip_fail(e, "loss reduction launch");
  return LARARD_OK;
}

// ---------------------------------------------------------------------------
// Scratch of larard_loss_noalloc: one array per GPU, loaded with the library's
// device code and held until the process ends.  In host code `scratch` only
// names the symbol; its device address (one per GPU) comes from
// hipGetSymbolAddress, looked up once per device and cached.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[LARARD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

larard_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LARARD_E_INVALID, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || !aligned(p, 256)) return fail(LARARD_E_HIP, "scratch symbol has no 256-byte aligned address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LARARD_OK;
}

}  // namespace

extern "C" {

size_t larard_workspace_bytes(larard_dtype dtype, int64_t B, int64_t H, int64_t n) {
  size_t off[4];
  if (larard_workspace_layout(dtype, B, H, n, off) != LARARD_OK) return 0;
  return off[3] + align256((size_t)(B * H) * sizeof(double));
}

int64_t larard_loss_head_group(larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d, int cross) {
  if (B < 1 || H < 1 || n < 0 || n > kMaxN || B > kMaxGrid / H || (d != 64 && d != 128)) return 0;
  if (dtype != LARARD_BF16 && dtype != LARARD_FP32) return 0;
  return group_of(dtype == LARARD_FP32, cross != 0, B * H, n, d);
}

int64_t larard_loss_sweep_group(larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d, int cross) {
  if (B < 1 || H < 1 || n < 0 || n > kMaxN || B > kMaxGrid / H || (d != 64 && d != 128)) return 0;
  if (dtype != LARARD_BF16 && dtype != LARARD_FP32) return 0;
  return group_of(dtype == LARARD_FP32, cross != 0, B * H, n, d, kSweepGroupBytes, LMR_GROUP2_GRID);
}

larard_status larard_workspace_layout(larard_dtype dtype, int64_t B, int64_t H, int64_t n, size_t off[4]) {
  if (off == nullptr || B < 1 || H < 1 || n < 0 || n > kMaxN || B > kMaxGrid / H)
    return fail(LARARD_E_INVALID, "invalid sizes for workspace layout");
  if (dtype != LARARD_BF16 && dtype != LARARD_FP32) return fail(LARARD_E_UNSUPPORTED, "dtype %d not supported", (int)dtype);
  const size_t rows = (size_t)(B * H) * (size_t)n;
  const size_t stat = align256(rows * stat_bytes(dtype));
  off[0] = 0;
  off[1] = stat;
  off[2] = 2 * stat;
  off[3] = 2 * stat + align256(rows * sizeof(float));
  return LARARD_OK;
}

larard_status larard_lse_fwd(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H,
                             int64_t n, int64_t d, float scale, int causal, void* lse_t, void* lse_s,
                             void* stream) {
  larard_status s = check_common(x_t, x_s, dtype, B, H, n, d, scale);
  if (s != LARARD_OK) return s;
  if (n == 0) return LARARD_OK;
  if (lse_t == nullptr || lse_s == nullptr) return fail(LARARD_E_INVALID, "lse_t / lse_s must not be NULL");
  if (!aligned(lse_t, stat_bytes(dtype)) || !aligned(lse_s, stat_bytes(dtype)))
    return fail(LARARD_E_INVALID, "lse buffers must be aligned to their element size");
  lmr::SweepArgs a = make_args(x_t, x_s, dtype, B, H, n, d, scale, causal);
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  const hipError_t e = lmr::launch_lse_fwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "lse_fwd launch");
  return LARARD_OK;
}

larard_status larard_kl_fwd(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H,
                            int64_t n, int64_t d, float scale, int causal, void* lse_t, void* lse_s,
                            float* row_kl, void* stream) {
  larard_status s = check_common(x_t, x_s, dtype, B, H, n, d, scale);
  if (s != LARARD_OK) return s;
  if (n == 0) return LARARD_OK;
  if (lse_t == nullptr || lse_s == nullptr) return fail(LARARD_E_INVALID, "lse_t / lse_s must not be NULL");
  if (!aligned(lse_t, stat_bytes(dtype)) || !aligned(lse_s, stat_bytes(dtype)))
    return fail(LARARD_E_INVALID, "lse buffers must be aligned to their element size");
  if (row_kl == nullptr || !aligned(row_kl, 4)) return fail(LARARD_E_INVALID, "row_kl must be a 4-byte aligned pointer");
  lmr::SweepArgs a = make_args(x_t, x_s, dtype, B, H, n, d, scale, causal);
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  a.row_kl = row_kl;
  const hipError_t e = lmr::launch_kl_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LARARD_OK : hip_fail(e, "kl_fwd launch");
}

larard_status larard_kl_bwd(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H,
                            int64_t n, int64_t d, float scale, int causal, const void* lse_t,
                            const void* lse_s, float loss_scale, float* row_kl, float* dx_s, int dx_mode,
                            void* stream) {
  lmr::SweepArgs a;
  larard_status s = check_phase2(x_t, x_s, dtype, B, H, n, d, scale, causal, lse_t, lse_s, loss_scale, &a);
  if (s != LARARD_OK) return s;
  if ((s = check_dx_mode(dx_mode)) != LARARD_OK) return s;
  if (n == 0) return LARARD_OK;
  if (row_kl == nullptr || !aligned(row_kl, 4)) return fail(LARARD_E_INVALID, "row_kl must be a 4-byte aligned pointer");
  if (dx_s != nullptr && !aligned(dx_s, 16)) return fail(LARARD_E_INVALID, "dx_s must be 16-byte aligned");
  a.row_kl = row_kl;
  a.dx = dx_s;
  return run_kl_bwd(a, loss_scale, dx_mode, static_cast<hipStream_t>(stream));
}

larard_status larard_loss(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H,
                          int64_t n, int64_t d, float scale, int causal, float loss_scale, void* workspace,
                          size_t workspace_bytes, float* loss, float* dx_s, int dx_mode, void* stream) {
  larard_status s = check_loss(x_t, x_s, dtype, B, H, n, d, scale, loss_scale, loss, dx_s, dx_mode);
  if (s != LARARD_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (n == 0) return zero_loss(loss, st);
  const size_t need = larard_workspace_bytes(dtype, B, H, n);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(LARARD_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(LARARD_E_WORKSPACE, "workspace must be 256-byte aligned");
  return run_loss(x_t, x_s, dtype, B, H, n, d, scale, causal, loss_scale, static_cast<char*>(workspace), loss, dx_s,
                  dx_mode, st);
}

larard_status larard_loss_noalloc(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H,
                                  int64_t n, int64_t d, float scale, int causal, float loss_scale, float* loss,
                                  float* dx_s, int dx_mode, void* stream) {
  larard_status s = check_loss(x_t, x_s, dtype, B, H, n, d, scale, loss_scale, loss, dx_s, dx_mode);
  if (s != LARARD_OK) return s;
  const size_t need = larard_workspace_bytes(dtype, B, H, n);
  if (need > (size_t)LARARD_NOALLOC_SCRATCH_BYTES)
    return fail(LARARD_E_WORKSPACE, "larard_loss_noalloc: B*H*n = %lld rows need %zu bytes of scratch, above the "
                "library's static %zu bytes; use larard_loss with a caller workspace",
                (long long)(B * H * n), need, (size_t)LARARD_NOALLOC_SCRATCH_BYTES);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (n == 0) return zero_loss(loss, st);
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != LARARD_OK) return s;
  return run_loss(x_t, x_s, dtype, B, H, n, d, scale, causal, loss_scale, static_cast<char*>(ws), loss, dx_s, dx_mode,
                  st);
}

larard_status larard_kl_bwd_rows(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H,
                                 int64_t n, int64_t d, float scale, int causal, const void* lse_t,
                                 const void* lse_s, float loss_scale, float* row_kl, float* dx_s, void* stream) {
  lmr::SweepArgs a;
  larard_status s = check_phase2(x_t, x_s, dtype, B, H, n, d, scale, causal, lse_t, lse_s, loss_scale, &a);
  if (s != LARARD_OK || n == 0) return s;
  if (row_kl == nullptr || !aligned(row_kl, 4)) return fail(LARARD_E_INVALID, "row_kl must be a 4-byte aligned pointer");
  if (dx_s != nullptr && !aligned(dx_s, 16)) return fail(LARARD_E_INVALID, "dx_s must be 16-byte aligned");
  a.row_kl = row_kl;
  a.dx = dx_s;
  const hipError_t e = lmr::launch_kl_row(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LARARD_OK : hip_fail(e, "kl_bwd row sweep launch");
}

larard_status larard_kl_bwd_cols(const void* x_t, const void* x_s, larard_dtype dtype, int64_t B, int64_t H,
                                 int64_t n, int64_t d, float scale, int causal, const void* lse_t,
                                 const void* lse_s, float loss_scale, float* dx_s, void* stream) {
  lmr::SweepArgs a;
  larard_status s = check_phase2(x_t, x_s, dtype, B, H, n, d, scale, causal, lse_t, lse_s, loss_scale, &a);
  if (s != LARARD_OK || n == 0) return s;
  if (dx_s == nullptr || !aligned(dx_s, 16)) return fail(LARARD_E_INVALID, "dx_s must be a 16-byte aligned pointer");
  a.dx = dx_s;
  const hipError_t e = lmr::launch_kl_col(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LARARD_OK : hip_fail(e, "kl_bwd column sweep launch");
}

larard_status larard_reduce_loss(const float* row_kl, int64_t B, int64_t H, int64_t n, float loss_scale,
                                 double* partials, float* loss, void* stream) {
  if (B < 1 || H < 1 || n < 0 || n > kMaxN || B > kMaxGrid / H) return fail(LARARD_E_INVALID, "invalid sizes");
  if (!std::isfinite(loss_scale)) return fail(LARARD_E_INVALID, "loss_scale must be finite");
  if (loss == nullptr || !aligned(loss, 4)) return fail(LARARD_E_INVALID, "loss must be a 4-byte aligned pointer");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (n == 0) {
    const hipError_t e = lmr::launch_zero_scalar(loss, st);
    return e == hipSuccess ? LARARD_OK : hip_fail(e, "zero loss launch");
  }
  if (row_kl == nullptr || !aligned(row_kl, 4)) return fail(LARARD_E_INVALID, "row_kl must be a 4-byte aligned pointer");
  if (partials == nullptr || !aligned(partials, 8)) return fail(LARARD_E_INVALID, "partials must be an 8-byte aligned pointer");
  const hipError_t e = lmr::launch_reduce(row_kl, B * H, (int)n, loss_scale, partials, loss, st);
  return e == hipSuccess ? LARARD_OK : hip_fail(e, "loss reduction launch");
}

// ---------------------------------------------------------------------------
// General relation X != Y (larard.h, "cross relation" entry points).
// ---------------------------------------------------------------------------
larard_status larard_xy_lse_fwd(const void* x_t, const void* x_s, const void* y_t, const void* y_s,
                                larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d, float scale,
                                int causal, void* lse_t, void* lse_s, void* stream) {
  larard_status s = check_common(x_t, x_s, dtype, B, H, n, d, scale);
  if (s != LARARD_OK) return s;
  lmr::SweepArgs a = make_args(x_t, x_s, dtype, B, H, n, d, scale, causal);
  if ((s = set_cross(&a, y_t, y_s, n)) != LARARD_OK || n == 0) return s;
  if (lse_t == nullptr || lse_s == nullptr) return fail(LARARD_E_INVALID, "lse_t / lse_s must not be NULL");
  if (!aligned(lse_t, stat_bytes(dtype)) || !aligned(lse_s, stat_bytes(dtype)))
    return fail(LARARD_E_INVALID, "lse buffers must be aligned to their element size");
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  const hipError_t e = lmr::launch_lse_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LARARD_OK : hip_fail(e, "xy_lse_fwd launch");
}

larard_status larard_xy_kl_fwd(const void* x_t, const void* x_s, const void* y_t, const void* y_s,
                               larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d, float scale,
                               int causal, void* lse_t, void* lse_s, float* row_kl, void* stream) {
  larard_status s = check_common(x_t, x_s, dtype, B, H, n, d, scale);
  if (s != LARARD_OK) return s;
  lmr::SweepArgs a = make_args(x_t, x_s, dtype, B, H, n, d, scale, causal);
  if ((s = set_cross(&a, y_t, y_s, n)) != LARARD_OK || n == 0) return s;
  if (lse_t == nullptr || lse_s == nullptr) return fail(LARARD_E_INVALID, "lse_t / lse_s must not be NULL");
  if (!aligned(lse_t, stat_bytes(dtype)) || !aligned(lse_s, stat_bytes(dtype)))
    return fail(LARARD_E_INVALID, "lse buffers must be aligned to their element size");
  if (row_kl == nullptr || !aligned(row_kl, 4)) return fail(LARARD_E_INVALID, "row_kl must be a 4-byte aligned pointer");
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  a.row_kl = row_kl;
  const hipError_t e = lmr::launch_kl_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LARARD_OK : hip_fail(e, "xy_kl_fwd launch");
}

larard_status larard_xy_kl_bwd(const void* x_t, const void* x_s, const void* y_t, const void* y_s,
                               larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d, float scale,
                               int causal, const void* lse_t, const void* lse_s, float loss_scale,
                               float* row_kl, float* dx_s, float* dy_s, void* stream) {
  lmr::SweepArgs a;
  larard_status s = check_phase2(x_t, x_s, dtype, B, H, n, d, scale, causal, lse_t, lse_s, loss_scale, &a);
  if (s != LARARD_OK) return s;
  if (n == 0) return set_cross(&a, y_t, y_s, n);
  if ((s = set_cross(&a, y_t, y_s, n)) != LARARD_OK) return s;
  if (row_kl == nullptr || !aligned(row_kl, 4)) return fail(LARARD_E_INVALID, "row_kl must be a 4-byte aligned pointer");
  if ((dx_s != nullptr && !aligned(dx_s, 16)) || (dy_s != nullptr && !aligned(dy_s, 16)))
    return fail(LARARD_E_INVALID, "dx_s / dy_s must be 16-byte aligned");
  a.row_kl = row_kl;
  a.dx = dx_s;
  a.dy = dy_s;
  return run_kl_bwd(a, loss_scale, LARARD_DX_SPLIT, static_cast<hipStream_t>(stream));
}

larard_status larard_xy_loss(const void* x_t, const void* x_s, const void* y_t, const void* y_s,
                             larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d, float scale,
                             int causal, float loss_scale, void* workspace, size_t workspace_bytes, float* loss,
                             float* dx_s, float* dy_s, void* stream) {
  larard_status s = check_common(x_t, x_s, dtype, B, H, n, d, scale);
  if (s != LARARD_OK) return s;
  lmr::SweepArgs a = make_args(x_t, x_s, dtype, B, H, n, d, scale, causal);
  if ((s = set_cross(&a, y_t, y_s, n)) != LARARD_OK) return s;
  if (!std::isfinite(loss_scale)) return fail(LARARD_E_INVALID, "loss_scale must be finite");
  if (loss == nullptr || !aligned(loss, 4)) return fail(LARARD_E_INVALID, "loss must be a 4-byte aligned device pointer");
  if ((dx_s != nullptr && !aligned(dx_s, 16)) || (dy_s != nullptr && !aligned(dy_s, 16)))
    return fail(LARARD_E_INVALID, "dx_s / dy_s must be 16-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (n == 0) {
    const hipError_t e = lmr::launch_zero_scalar(loss, st);
    return e == hipSuccess ? LARARD_OK : hip_fail(e, "zero loss launch");
  }
  size_t off[4];
  if ((s = larard_workspace_layout(dtype, B, H, n, off)) != LARARD_OK) return s;
  const size_t need = larard_workspace_bytes(dtype, B, H, n);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(LARARD_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(LARARD_E_WORKSPACE, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  a.lse_t = ws + off[0];
  a.lse_s = ws + off[1];
  a.row_kl = reinterpret_cast<float*>(ws + off[2]);
  double* partials = reinterpret_cast<double*>(ws + off[3]);
  hipError_t e;
  if (dx_s == nullptr && dy_s == nullptr) {
    e = lmr::launch_kl_fwd(a, st);
    if (e != hipSuccess) return hip_fail(e, "xy_kl_fwd launch");
  } else {
    a.dx = dx_s;
    a.dy = dy_s;
    if ((s = run_grouped(a, loss_scale, LARARD_DX_SPLIT, st)) != LARARD_OK) return s;
  }
  e = lmr::launch_reduce(a.row_kl, a.bh, a.n, loss_scale, partials, loss, st);
  if (e != hipSuccess) return hip_fail(e, "loss reduction launch");
  return LARARD_OK;
}

// ---------------------------------------------------------------------------
// Several maps in one launch per phase (larard.h, larard_multi_loss).
namespace {
// The maps run one after another, each as larard_loss runs it (head groups
// and phase-2 sub-groups), when the projections of all maps together exceed
// one head group's budget: a single launch per phase over all maps would
// then re-read them from HBM in phase 2.  Measured on MI355X: at n = 16K
// (three maps of 32 heads, 768 MiB) the single-launch row and column sweeps
// took 5% longer than the maps' own launches in sequence; GQA 8K (Q over 64
// heads, K and V over 16 each, 384 MiB) 7.29 ms per step in one launch per
// phase against 6.84 for the maps apart.  Small sets (4K: 192 MiB) keep the
// single launch, which saves the launch gaps and tails of short kernels
// (1.77 against 1.87 ms).
bool maps_run_apart(const larard_map* maps, int n_maps, int64_t B, int64_t n, int64_t d) {
  int64_t bytes = 0;
  for (int m = 0; m < n_maps; ++m) bytes += B * maps[m].H * n * d * 2 * 2;
  return bytes > kGroupBytes;
}
}  // namespace
// ---------------------------------------------------------------------------
static_assert(LARARD_MAX_MAPS == lmr::kMaxMaps, "map-set capacity");

size_t larard_multi_workspace_bytes(larard_dtype dtype, int64_t B, int64_t n, const larard_map* maps, int n_maps) {
  if (maps == nullptr || n_maps < 1 || n_maps > LARARD_MAX_MAPS || B < 1) return 0;
  int64_t heads = 0;
  for (int m = 0; m < n_maps; ++m) {
    if (maps[m].H < 1 || maps[m].H > kMaxGrid) return 0;
    heads += maps[m].H;
  }
  if (heads > kMaxGrid / B) return 0;
  return larard_workspace_bytes(dtype, 1, B * heads, n);
}

larard_status larard_multi_loss(const larard_map* maps, int n_maps, larard_dtype dtype, int64_t B, int64_t n,
                                int64_t d, float scale, int causal, float loss_scale, void* workspace,
                                size_t workspace_bytes, float* loss, void* stream) {
  if (maps == nullptr || n_maps < 1 || n_maps > LARARD_MAX_MAPS)
    return fail(LARARD_E_INVALID, "n_maps must be in [1, %d] with a non-NULL map array", LARARD_MAX_MAPS);
  int64_t heads = 0;
  int with_dx = 0;
  larard_status s;
  for (int m = 0; m < n_maps; ++m) {
    const larard_map& mp = maps[m];
    if ((s = check_common(mp.x_t, mp.x_s, dtype, B, mp.H, n, d, scale)) != LARARD_OK) return s;
    if (!std::isfinite(mp.weight)) return fail(LARARD_E_INVALID, "map %d: weight must be finite", m);
    if (mp.dx_s != nullptr && !aligned(mp.dx_s, 16)) return fail(LARARD_E_INVALID, "map %d: dx_s must be 16-byte aligned", m);
    with_dx += mp.dx_s != nullptr;
    heads += mp.H;
  }
  if (with_dx != 0 && with_dx != n_maps) return fail(LARARD_E_INVALID, "either every map has dx_s or none has");
  if (heads > kMaxGrid / B) return fail(LARARD_E_INVALID, "B * sum of heads too large");
  const int64_t bh_all = B * heads;
  const int64_t nblk = (n + kOwnRows - 1) / kOwnRows;
  if (nblk > 0 && bh_all > kMaxGrid / nblk) return fail(LARARD_E_INVALID, "B*sum(H)*ceil(n/32) exceeds the launch grid");
  if (!std::isfinite(loss_scale)) return fail(LARARD_E_INVALID, "loss_scale must be finite");
  if (loss == nullptr || !aligned(loss, 4)) return fail(LARARD_E_INVALID, "loss must be a 4-byte aligned device pointer");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (n == 0) {
    const hipError_t e = lmr::launch_zero_scalar(loss, st);
    return e == hipSuccess ? LARARD_OK : hip_fail(e, "zero loss launch");
  }
  size_t off[4];
  if ((s = larard_workspace_layout(dtype, 1, bh_all, n, off)) != LARARD_OK) return s;
  const size_t need = larard_workspace_bytes(dtype, 1, bh_all, n);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(LARARD_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(LARARD_E_WORKSPACE, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  double* lse_t = reinterpret_cast<double*>(ws + off[0]);
  double* lse_s = reinterpret_cast<double*>(ws + off[1]);
  float* row_kl = reinterpret_cast<float*>(ws + off[2]);
  double* partials = reinterpret_cast<double*>(ws + off[3]);

  lmr::MapSet set{};
  int64_t head0[LARARD_MAX_MAPS + 1];
  float weight[LARARD_MAX_MAPS];
  head0[0] = 0;
  for (int m = 0; m < n_maps; ++m) {
    const larard_map& mp = maps[m];
    lmr::SweepArgs a = make_args(mp.x_t, mp.x_s, dtype, B, mp.H, n, d, scale, causal);
    const int64_t rows0 = head0[m] * n;
    a.lse_t = lse_t + rows0;
    a.lse_s = lse_s + rows0;
    a.row_kl = row_kl + rows0;
    a.dx = mp.dx_s;
    const double gsd = (double)loss_scale * (double)mp.weight * (double)scale / (double)n;
    a.grad_scale = (float)gsd;
    a.grad_scale_d = gsd;
    set.map[m] = a;
    head0[m + 1] = head0[m] + B * mp.H;
    set.head0[m] = head0[m];
    weight[m] = mp.weight;
  }
  set.head0[n_maps] = head0[n_maps];
  set.nmaps = n_maps;
  hipError_t e = hipSuccess;
  if (dtype == LARARD_FP32) {
    // Precision mode: the fp64 kernels, map by map.
    for (int m = 0; m < n_maps && e == hipSuccess; ++m) {
      const lmr::SweepArgs& a = set.map[m];
      if (with_dx == 0) {
        e = lmr::launch_kl_fwd(a, st);
      } else {
        e = lmr::launch_lse_fwd(a, st);
        if (e == hipSuccess) e = lmr::launch_kl_row(a, st);
        if (e == hipSuccess) e = lmr::launch_kl_col(a, st);
      }
    }
    if (e != hipSuccess) return hip_fail(e, "multi-map launch");
  } else if (with_dx == 0) {
    if ((e = lmr::launch_kl_fwd_multi(set, st)) != hipSuccess) return hip_fail(e, "multi-map kl_fwd launch");
  } else if (maps_run_apart(maps, n_maps, B, n, d)) {
    for (int m = 0; m < n_maps; ++m) {
      // grad_scale already carries the map's weight; run_kl_bwd sets it
      // from loss_scale, so pass the weighted scale.
      if ((s = run_grouped(set.map[m], loss_scale * maps[m].weight, LARARD_DX_AUTO, st)) != LARARD_OK) return s;
    }
  } else {
    if ((e = lmr::launch_lse_fwd_multi(set, st)) != hipSuccess) return hip_fail(e, "multi-map lse_fwd launch");
    if (use_fused(set.map[0], LARARD_DX_AUTO)) {
      if ((e = lmr::launch_kl_fused_multi(set, st)) != hipSuccess) return hip_fail(e, "multi-map fused sweep launch");
    } else {
      if ((e = lmr::launch_kl_row_multi(set, st)) != hipSuccess) return hip_fail(e, "multi-map row sweep launch");
      if ((e = lmr::launch_kl_col_multi(set, st)) != hipSuccess) return hip_fail(e, "multi-map column sweep launch");
    }
  }
  e = lmr::launch_reduce_weighted(row_kl, head0, weight, n_maps, (int)n, loss_scale, partials, loss, st);
  return e == hipSuccess ? LARARD_OK : hip_fail(e, "loss reduction launch");
}

// ---------------------------------------------------------------------------
// Projection backward (larard.h, larard_proj_bwd).
// ---------------------------------------------------------------------------
namespace {
bool proj_sizes_ok(int64_t B, int64_t n, int64_t dm, int64_t H, int64_t d) {
  return B >= 1 && H >= 1 && n >= 0 && n <= kMaxN && (d == 64 || d == 128) && dm >= 128 && dm % 128 == 0 &&
         (H * d) % 128 == 0 && dm / 64 <= 65535 && H <= 65535 && B <= kMaxGrid / (n > 0 ? n : 1);
}
int64_t proj_kp(int64_t B, int64_t n) { return (B * n + 63) / 64 * 64; }
}  // namespace

size_t larard_proj_bwd_workspace_bytes(int64_t B, int64_t n, int64_t dm, int64_t H, int64_t d) {
  if (!proj_sizes_ok(B, n, dm, H, d)) return 0;
  const size_t kp = (size_t)proj_kp(B, n);
  const size_t g = align256((size_t)(H * d) * kp * 2);
  return lmr::proj_uses_256_tiles(dm, H * d) ? g + align256((size_t)dm * kp * 2) : g;
}

larard_status larard_proj_bwd(const void* h, const float* dx_s, int64_t B, int64_t n, int64_t dm, int64_t H,
                              int64_t d, const float* rope_cos, const float* rope_sin, void* workspace,
                              size_t workspace_bytes, float* dw, void* stream) {
  if (!proj_sizes_ok(B, n, dm, H, d)) {
    if (d != 64 && d != 128) return fail(LARARD_E_UNSUPPORTED, "head dim d=%lld not supported (64 or 128)", (long long)d);
    if (dm < 128 || dm % 128 != 0 || (H * d) % 128 != 0)
      return fail(LARARD_E_UNSUPPORTED, "model dim and H*d must be multiples of 128 (got %lld, %lld)",
                  (long long)dm, (long long)(H * d));
    return fail(LARARD_E_INVALID, "invalid sizes B=%lld n=%lld dm=%lld H=%lld", (long long)B, (long long)n,
                (long long)dm, (long long)H);
  }
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(LARARD_E_INVALID, "rope_cos and rope_sin must both be given or both be NULL");
  if (rope_cos != nullptr && (!aligned(rope_cos, 4) || !aligned(rope_sin, 4)))
    return fail(LARARD_E_INVALID, "rope tables must be 4-byte aligned");
  if (n > 0 && (h == nullptr || dx_s == nullptr || !aligned(h, 16) || !aligned(dx_s, 16)))
    return fail(LARARD_E_INVALID, "h and dx_s must be 16-byte aligned device pointers");
  if (dw == nullptr || !aligned(dw, 16)) return fail(LARARD_E_INVALID, "dw must be a 16-byte aligned device pointer");
  const size_t need = larard_proj_bwd_workspace_bytes(B, n, dm, H, d);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(LARARD_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (need > 0 && !aligned(workspace, 256)) return fail(LARARD_E_WORKSPACE, "workspace must be 256-byte aligned");
  lmr::ProjArgs p{};
  p.h = static_cast<const uint16_t*>(h);
  p.dx = dx_s;
  p.cos = rope_cos;
  p.sin = rope_sin;
  p.B = B;
  p.n = n;
  p.dm = dm;
  p.H = H;
  p.d = d;
  p.kp = proj_kp(B, n);
  p.g = static_cast<uint16_t*>(workspace);
  p.ht = lmr::proj_uses_256_tiles(dm, H * d)
             ? reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + align256((size_t)(H * d) * (size_t)p.kp * 2))
             : nullptr;
  p.dw = dw;
  const hipError_t e = lmr::launch_proj_bwd(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LARARD_OK : hip_fail(e, "proj_bwd launch");
}

const char* larard_status_str(larard_status status) {
  switch (status) {
    case LARARD_OK: return "LARARD_OK";
    case LARARD_E_INVALID: return "LARARD_E_INVALID: invalid argument";
    case LARARD_E_UNSUPPORTED: return "LARARD_E_UNSUPPORTED: unsupported head dim, dtype or mode";
    case LARARD_E_WORKSPACE: return "LARARD_E_WORKSPACE: workspace too small or misaligned";
    case LARARD_E_HIP: return "LARARD_E_HIP: HIP runtime error";
    default: break;
  }
  return "unknown larard_status";
}

const char* larard_last_error(void) { return g_last_error.c_str(); }

#ifndef LARARD_SOURCE_ID
#define LARARD_SOURCE_ID "unstamped"
#endif
const char* larard_version(void) { return "larard 0.1.0 gfx950 (src " LARARD_SOURCE_ID ")"; }

}  // extern "C"
