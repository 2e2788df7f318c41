/*
 * larard.h -- C ABI of the linear-memory relation-KL library (liblarard.so).
 *
 * The operation ("LinearARD: Linear-Memory Attention Distillation for RoPE
 * Restoration", paper-notes page, section "Key designs", items 1 and 3):
 * for every head, teacher (t) and student (s) projections X_t, X_s in
 * R^{n x d} define logits Z_m = scale * X_m X_m^T, a causal mask keeps
 * j <= i, and R_m = row-softmax(Z_m).  The per-head loss is the row mean of
 * the forward divergence KL(R_t(i,:) || R_s(i,:)); the student gradient is
 *     dX_s = scale * (dZ X_s + dZ^T X_s),   dZ = (R_s - R_t) / n,
 * where both terms land in dX_s because the relation is a self-relation
 * (X = Y).  Phase 1 stores only the per-row log-sum-exp LSE_m(i); phase 2
 * recomputes logit tiles on chip and never stores an n x n map, so extra
 * memory is O(B*H*n).  The teacher is frozen: no teacher gradient exists.
 *
 * Conventions shared by every entry point
 *   - Tensors X_t, X_s are [B, H, n, d] contiguous, row-major (d fastest),
 *     in bf16 (LARARD_BF16) or fp32 (LARARD_FP32), 16-byte aligned.
 *     d must be 64 or 128.  B, H >= 1; 0 <= n <= 2^24.
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the
 *     library allocates no device memory and keeps no pointer after return.
 *   - LSE buffers are fp64 [B, H, n] in natural log, 8-byte aligned;
 *     row_kl is fp32 [B, H, n].  The statistics are fp64 because phase 2
 *     rebuilds every probability from them: an fp32 LSE near 45 (peaky
 *     rows) is off by ~4e-6, which shifts a whole probability row by that
 *     factor and can exceed a nearly vanishing dZ.
 *   - bf16 inputs run on bf16 MFMA with fp32 accumulation.  fp32 inputs run
 *     a precision mode that keeps logits, probabilities and statistics in
 *     fp64 (each dZ row sums to zero, so dZ X_s is a small difference of
 *     weighted means and fp32 logits alone would cost ~1e-4 of it); it is
 *     meant for checking and small inputs, not for throughput.
 *   - dx_s is fp32 [B, H, n, d], 16-byte aligned, and is OVERWRITTEN.
 *   - scale must be finite and > 0 (the workloads use 1/sqrt(d)).
 *   - causal != 0 keeps j <= i (diagonal included); causal == 0 keeps all
 *     n columns (the bidirectional variant).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous; arguments are validated before any
 *     launch, and on a validation error nothing is launched or written.
 *     A failing HIP call returns LARARD_E_HIP; its text is available from
 *     larard_last_error() on the calling thread.
 *   - The library is thread-safe.  Its only mutable global state belongs to
 *     larard_loss_noalloc: a static device scratch array per GPU and a
 *     mutex-guarded cache of its address per device.
 */
#ifndef LARARD_H
#define LARARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The _RANGE_MIN_ / _RANGE_MAX_ sentinels make every 32-bit value a valid
 * object of the enum type, so a caller may pass any int (e.g. from another
 * language) without undefined behaviour; the library rejects all values but
 * the named ones. */
typedef enum {
  LARARD_OK = 0,
  LARARD_E_INVALID = 1,     /* null pointer, bad size, bad scale, misalignment */
  LARARD_E_UNSUPPORTED = 2, /* head dim, dtype or mode not built */
  LARARD_E_WORKSPACE = 3,   /* workspace too small or misaligned */
  LARARD_E_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  LARARD_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
  LARARD_STATUS_RANGE_MAX_ = 0x7fffffff
} larard_status;

typedef enum {
  LARARD_BF16 = 0,
  LARARD_FP32 = 1,
  LARARD_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  LARARD_DTYPE_RANGE_MAX_ = 0x7fffffff
} larard_dtype;

/* How phase 2 produces the column term dZ^T X_s of the gradient.
 *   FUSED : one launch in which each workgroup owns a block of rows k and
 *           sweeps both the key tiles j <= k (row term) and the row tiles
 *           i >= k (column term, the rows' role as keys), adding both into one
 *           register accumulator and storing dX_s once; deterministic, no
 *           atomics, every workgroup does the same work.  bf16 self-relations
 *           only; the fp32 precision kernels and the X != Y relation run SPLIT.
 *   SPLIT : a row-owned sweep stores the row term, then a column-owned sweep
 *           recomputes the logit tiles and adds the column term;
 *           deterministic, no atomics.
 *   ATOMIC: not built; every call that passes it returns
 *           LARARD_E_UNSUPPORTED.  (A row sweep that adds its column partials
 *           with fp32 atomics must add B*H*n^2 bytes per map with 256-row
 *           workgroups -- 8.6 GB at n = 16K, H = 32.  On MI355X the row sweep
 *           with only that atomic flush added, before any of the column
 *           term's own arithmetic, took 6.6 ms per 16K map against 3.2 ms
 *           for the row sweep and 6.4 ms for the split's two sweeps.)
 *   AUTO  : FUSED for n <= 8192, SPLIT above, by measurement on MI355X:
 *           FUSED is 3% faster per step at n = 4K and 2% at 8K, where the
 *           split sweeps' causal tails show, and 1.4% slower at 16K, although
 *           it moves a third less HBM traffic.  (larard_multi_loss follows
 *           the same rule.)
 * FUSED and SPLIT execute the same contractions (phase 2 computes every
 * logit tile twice) and give the same results to fp32 rounding; each is
 * bitwise reproducible. */
typedef enum { LARARD_DX_AUTO = 0, LARARD_DX_SPLIT = 1, LARARD_DX_ATOMIC = 2, LARARD_DX_FUSED = 3 } larard_dx_mode;

/* Bytes of workspace larard_loss needs: LSE_t and LSE_s (B*H*n fp64 each),
 * row_kl (B*H*n fp32) and B*H fp64 partial sums, each region 256-byte
 * aligned: 20*B*H*n + 8*B*H (+ alignment).  O(B*H*n):
 * the notes page ("Key designs", item 3) stores only per-row statistics.
 * Returns 0 for invalid sizes. */
size_t larard_workspace_bytes(larard_dtype dtype, int64_t B, int64_t H, int64_t n);

/* Heads per group of the whole-path calls with a gradient (larard_loss,
 * larard_loss_noalloc, larard_xy_loss, and larard_multi_loss when its maps
 * run apart): they run phase 1 and phase 2 for heads [h0, h0+g) of the
 * flattened B*H heads before the next group, so that the group's
 * projections are still in the GPU's 256 MB last-level cache when phase 2
 * re-reads them.  g is the largest head count whose bf16 projections
 * (X_t, X_s, and Y_t, Y_s when cross != 0) fit 256 MiB, raised if needed to
 * ceil(1024 / ceil(n/256)) heads so that each sweep still has 1024
 * workgroups, and capped at B*H.  fp32 inputs run as one group.  A caller
 * of larard_lse_fwd / larard_kl_bwd can slice its heads the same way.
 * Measured on MI355X (ms per step, one group -> groups of 8 or 16 heads):
 * n = 32K 105.3 -> 101.7; at n = 16K (32 heads, one group) grouping gained
 * nothing.  Results are the same bits either way.  Returns 0 for invalid
 * sizes. */
int64_t larard_loss_head_group(larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d, int cross);

/* Heads per phase-2 sub-group of the same calls: within each head group,
 * phase 2 (the row and column sweeps, or the fused sweep, which read a
 * head's projections twice) runs for sub-groups of at most this many heads,
 * the same rule with a 128 MiB budget (still at least 1024 workgroups per
 * sweep).  Measured on MI355X (ms per step, phase 2 per group -> per
 * sub-group): n = 16K 25.7 -> 25.4 (split), GQA 8K 6.93 -> 6.68 (fused).
 * Returns 0 for invalid sizes. */
int64_t larard_loss_sweep_group(larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d, int cross);

/* Phase 1 (notes page, "Key designs" item 3; summary page, "Method"):
 * streams key tiles and writes
 *   lse_t[b,h,i] = log sum_{j kept} exp(scale * <x_t,i , x_t,j>)
 * and likewise lse_s, fp64 [B, H, n].  No other output.  Each row's sum is
 * taken against a fixed shift, the row's own diagonal logit (always a kept
 * entry), instead of a running maximum; if any row of a 256-row block
 * overflows or underflows that shift, the block redoes its rows with an
 * online maximum.  The result is the same exact LSE either way. */
larard_status larard_lse_fwd(const void* x_t, const void* x_s, larard_dtype dtype,
                             int64_t B, int64_t H, int64_t n, int64_t d,
                             float scale, int causal,
                             void* lse_t, void* lse_s, void* stream);

/* Forward-only loss in one sweep (notes page, "Key designs" items 1 and 3;
 * the KL needs only the logits and both row statistics): phase 1 extended
 * with a teacher-weighted log-ratio accumulator.  Writes lse_t and lse_s as
 * larard_lse_fwd does (fp64 [B,H,n], natural log) and
 *   row_kl[b,h,i] = KL(R_t(i,:) || R_s(i,:))          (fp32, not scaled)
 * at the cost of phase 1 alone (2 of the 6 contractions of the full path).
 * All three outputs are required.  The row KL agrees with larard_kl_bwd's to
 * fp32 rounding, not bit for bit. */
larard_status larard_kl_fwd(const void* x_t, const void* x_s, larard_dtype dtype,
                            int64_t B, int64_t H, int64_t n, int64_t d,
                            float scale, int causal,
                            void* lse_t, void* lse_s, float* row_kl, void* stream);

/* Phase 2 (notes page, "Key designs" item 3): recomputes the logit tiles,
 * rebuilds R_t and R_s from lse_t / lse_s (which must come from
 * larard_lse_fwd with the same inputs and arguments), and writes
 *   row_kl[b,h,i] = KL(R_t(i,:) || R_s(i,:))          (fp32, not scaled)
 *   dx_s[b,h,i,:] = loss_scale * scale * (dZ X_s + dZ^T X_s)[i,:]
 * with dZ = (R_s - R_t)/n.  loss_scale = 1 is the pages' convention (heads
 * summed); 1/(B*H) gives a head mean.  dx_s == NULL computes row_kl only.
 * dx_mode is a larard_dx_mode. */
larard_status larard_kl_bwd(const void* x_t, const void* x_s, larard_dtype dtype,
                            int64_t B, int64_t H, int64_t n, int64_t d,
                            float scale, int causal,
                            const void* lse_t, const void* lse_s,
                            float loss_scale, float* row_kl, float* dx_s,
                            int dx_mode, void* stream);

/* The two halves of larard_kl_bwd in split mode, for callers that schedule
 * them separately (e.g. to overlap maps on several streams).
 * larard_kl_bwd_rows: row-owned sweep; writes row_kl and STORES the row term
 *   loss_scale * scale * (dZ X_s)[i,:] into dx_s (dx_s == NULL: row_kl only).
 * larard_kl_bwd_cols: column-owned sweep; ADDS the column term
 *   loss_scale * scale * (dZ^T X_s)[j,:] into dx_s, which must already hold
 *   the row term of the same call sequence.  Running rows then cols on one
 *   stream equals larard_kl_bwd with LARARD_DX_SPLIT, bit for bit. */
larard_status larard_kl_bwd_rows(const void* x_t, const void* x_s, larard_dtype dtype,
                                 int64_t B, int64_t H, int64_t n, int64_t d,
                                 float scale, int causal,
                                 const void* lse_t, const void* lse_s,
                                 float loss_scale, float* row_kl, float* dx_s, void* stream);
larard_status larard_kl_bwd_cols(const void* x_t, const void* x_s, larard_dtype dtype,
                                 int64_t B, int64_t H, int64_t n, int64_t d,
                                 float scale, int causal,
                                 const void* lse_t, const void* lse_s,
                                 float loss_scale, float* dx_s, void* stream);

/* Loss reduction (notes page, "Key designs" item 1: row mean, summed over
 * heads): *loss = loss_scale * sum_{b,h} (1/n) sum_i row_kl[b,h,i], summed in
 * fp64 in a fixed order (bitwise reproducible).  partials: device scratch of
 * B*H doubles, 8-byte aligned.  n == 0 writes *loss = 0. */
larard_status larard_reduce_loss(const float* row_kl, int64_t B, int64_t H, int64_t n,
                                 float loss_scale, double* partials, float* loss, void* stream);

/* Whole path for one relation map: phase 1, phase 2 and a deterministic
 * fp64 reduction.  Writes
 *   *loss = loss_scale * sum_{b,h} (1/n) sum_i KL_i        (device fp32 scalar)
 * and dx_s as in larard_kl_bwd (same bits).  Phase 1 and phase 2 run head
 * group by head group (larard_loss_head_group, larard_loss_sweep_group).  dx_s == NULL computes the
 * loss only, with larard_kl_fwd's single sweep instead of phase 1 + phase 2.  The workspace (device,
 * 256-byte aligned, >= larard_workspace_bytes(dtype,B,H,n)) holds LSE_t, LSE_s,
 * row_kl and partial sums; after return-and-sync it contains them in that
 * order (see larard_workspace_layout).  n == 0 writes *loss = 0. */
larard_status larard_loss(const void* x_t, const void* x_s, larard_dtype dtype,
                          int64_t B, int64_t H, int64_t n, int64_t d,
                          float scale, int causal, float loss_scale,
                          void* workspace, size_t workspace_bytes,
                          float* loss, float* dx_s, int dx_mode, void* stream);

/* Allocation-free larard_loss, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and kernels as larard_loss
 * without the workspace pair: LSE_t, LSE_s, row_kl and the partial sums live
 * in a static device array of LARARD_NOALLOC_SCRATCH_BYTES bytes that the
 * library's device code carries (one copy per GPU, held until the process
 * ends).  Its device address is looked up once per device, with that device
 * current, on the first call there; nothing is allocated, by this call or by
 * any routine it calls.
 *   - Shapes whose larard_workspace_bytes(dtype, B, H, n) exceeds
 *     LARARD_NOALLOC_SCRATCH_BYTES are rejected with LARARD_E_WORKSPACE
 *     (64 MiB: B*H*n up to ~3.3 million rows, e.g. 32 heads at n = 64K).
 *   - Every call on one GPU shares that GPU's array and leaves its own
 *     statistics there.  Calls that overlap in time on one GPU (other
 *     streams, other threads) race on it and must be ordered by the caller.
 *   - No clearing is needed between calls: every scratch byte a call reads is
 *     written earlier by the same call. */
#define LARARD_NOALLOC_SCRATCH_BYTES (64u << 20)
larard_status larard_loss_noalloc(const void* x_t, const void* x_s, larard_dtype dtype,
                                  int64_t B, int64_t H, int64_t n, int64_t d,
                                  float scale, int causal, float loss_scale,
                                  float* loss, float* dx_s, int dx_mode, void* stream);

/* ---------------------------------------------------------------------------
 * General relation X != Y (notes page, "Key designs" item 1 defines the map
 * for projected sequences X_m, Y_m; item 3 contracts dZ into both dX_s and
 * dY_s).  For each head:
 *     Z_m = scale * X_m Y_m^T   (rows i from X, columns j from Y; causal keeps j <= i)
 *     R_m = row-softmax(Z_m),   loss = (1/n) sum_i KL(R_t(i,:) || R_s(i,:))
 *     dX_s = loss_scale * scale * dZ Y_s,   dY_s = loss_scale * scale * dZ^T X_s,
 *     dZ = (R_s - R_t)/n,
 * e.g. the query/key attention map (X = Q, Y = K).  y_t, y_s are [B,H,n,d]
 * device tensors of the same dtype and layout as x_t, x_s (16-byte aligned);
 * every other convention is that of the self-relation calls above.  Passing
 * y = x gives dX_s + dY_s = the self-relation gradient.
 * ------------------------------------------------------------------------- */

/* Phase 1 of the X/Y relation: lse_t, lse_s over the rows of Z (fp64 [B,H,n]). */
larard_status larard_xy_lse_fwd(const void* x_t, const void* x_s, const void* y_t, const void* y_s,
                                larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d,
                                float scale, int causal, void* lse_t, void* lse_s, void* stream);

/* Forward-only X/Y relation: lse_t, lse_s and row_kl in one sweep (as
 * larard_kl_fwd).  All outputs required. */
larard_status larard_xy_kl_fwd(const void* x_t, const void* x_s, const void* y_t, const void* y_s,
                               larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d,
                               float scale, int causal, void* lse_t, void* lse_s, float* row_kl,
                               void* stream);

/* Phase 2 of the X/Y relation (split mode): row_kl (required) and the
 * gradients dx_s and dy_s (fp32 [B,H,n,d], OVERWRITTEN; either may be NULL
 * to skip it).  lse_t / lse_s must come from larard_xy_lse_fwd (or
 * larard_xy_kl_fwd) with the same inputs. */
larard_status larard_xy_kl_bwd(const void* x_t, const void* x_s, const void* y_t, const void* y_s,
                               larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d,
                               float scale, int causal, const void* lse_t, const void* lse_s,
                               float loss_scale, float* row_kl, float* dx_s, float* dy_s,
                               void* stream);

/* Whole X/Y path for one relation map with the workspace of larard_loss
 * (same size and layout).  dx_s == dy_s == NULL computes the loss only,
 * in one sweep. */
larard_status larard_xy_loss(const void* x_t, const void* x_s, const void* y_t, const void* y_s,
                             larard_dtype dtype, int64_t B, int64_t H, int64_t n, int64_t d,
                             float scale, int causal, float loss_scale,
                             void* workspace, size_t workspace_bytes,
                             float* loss, float* dx_s, float* dy_s, void* stream);

/* ---------------------------------------------------------------------------
 * Several self-relation maps in one launch per phase (notes page, "Key
 * designs" item 1 and "Loss function / training strategy": the loss is the
 * weighted sum of the Q/Q, K/K and V/V map losses, weights lambda = 1 in the
 * pages).  Maps share B, n, d, dtype, scale and causal; each has its own head
 * count (GQA: 32 query heads, 8 key/value heads) and weight.  Every kernel
 * runs once over the heads of all maps, saving the launch gaps and the
 * drained tail between per-map launches.  Work is ordered map by map (map 0
 * first), and within a map by row-block length (longest first) and then by
 * head.  Exception: when the bf16 projections of all maps together exceed
 * 256 MiB, the maps run one after another, each as larard_loss runs it
 * (head groups, AUTO phase 2), which keeps a map's projections in the
 * last-level cache between its sweeps (on MI355X: 5% faster phase 2 at
 * n = 16K with three maps of 32 heads; 6.84 against 7.29 ms per step for
 * the GQA 8K maps).  Results are the same bits either way.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* x_t;   /* [B, H, n, d] teacher projections of this map (device) */
  const void* x_s;   /* [B, H, n, d] student projections */
  int64_t H;         /* heads of this map */
  float weight;      /* lambda_m: multiplies this map's loss and gradient */
  float* dx_s;       /* [B, H, n, d] fp32 gradient (OVERWRITTEN) or NULL */
} larard_map;

#define LARARD_MAX_MAPS 8

/* Workspace of larard_multi_loss: larard_workspace_bytes(dtype, 1, B * sum_m H_m, n),
 * laid out as larard_workspace_layout of that shape with map m's heads
 * following those of maps 0..m-1.  Returns 0 for invalid arguments. */
size_t larard_multi_workspace_bytes(larard_dtype dtype, int64_t B, int64_t n, const larard_map* maps,
                                    int n_maps);

/* *loss = loss_scale * sum_m weight_m * sum_{b,h} (1/n) sum_i KL_i(map m), and
 * for each map dx_s = loss_scale * weight_m * scale * (dZ X_s + dZ^T X_s).
 * Either every map has dx_s or none has (loss only: one sweep per map set).
 * 1 <= n_maps <= LARARD_MAX_MAPS.  fp32 inputs run the precision kernels map
 * by map. */
larard_status larard_multi_loss(const larard_map* maps, int n_maps, larard_dtype dtype,
                                int64_t B, int64_t n, int64_t d, float scale, int causal,
                                float loss_scale, void* workspace, size_t workspace_bytes,
                                float* loss, void* stream);

/* ---------------------------------------------------------------------------
 * Projection backward: the gradient of the student projection weights
 * (notes page, "Method details -> Overall framework" and "Loss function /
 * training strategy": stage 1 updates only W_q, W_k, W_v).  With hidden
 * states h [B, n, dm] and per-head student projections
 *     X_s[b,hd,i,:] = R(i) (h[b,i,:] W[:, hd*d:(hd+1)*d]),
 * R(i) the student's rotate-half rotation at token i (pairs k, k + d/2,
 * angle table entries cos/sin[i, k]) or the identity (V, tables NULL):
 *     dw[c, hd*d + k] = sum_{b,i} h[b,i,c] (R(i)^T dX_s[b,hd,i,:])_k.
 * h: bf16 [B, n, dm] device, 16-byte aligned; dx_s: fp32 [B, H, n, d] (e.g.
 * the dx_s of larard_loss); rope_cos / rope_sin: fp32 [n, d/2] device or both
 * NULL; dw: fp32 [dm, H*d], OVERWRITTEN.  R^T dX_s is rounded to bf16 and
 * contracted on bf16 MFMA with fp32 accumulation.  dm and H*d must be
 * multiples of 128 (LARARD_E_UNSUPPORTED otherwise), d 64 or 128.  The
 * workspace (device, 256-byte aligned) holds (R^T dX_s)^T in bf16,
 * [H*d, B*n rounded up to 64], and for large outputs (dm and H*d multiples
 * of 256 with (dm/256)*(H*d/256) >= 256) h^T [dm, B*n rounded up to 64] as
 * well; smaller outputs read h in place.
 * ------------------------------------------------------------------------- */
size_t larard_proj_bwd_workspace_bytes(int64_t B, int64_t n, int64_t dm, int64_t H, int64_t d);

larard_status larard_proj_bwd(const void* h, const float* dx_s, int64_t B, int64_t n, int64_t dm,
                              int64_t H, int64_t d, const float* rope_cos, const float* rope_sin,
                              void* workspace, size_t workspace_bytes, float* dw, void* stream);

/* Byte offsets of the regions larard_loss carves from its workspace:
 * off[0] = lse_t, off[1] = lse_s, off[2] = row_kl, off[3] = fp64 partials.
 * Returns LARARD_E_INVALID for invalid sizes. */
larard_status larard_workspace_layout(larard_dtype dtype, int64_t B, int64_t H, int64_t n,
                                      size_t off[4]);

/* Static description of a status code. */
const char* larard_status_str(larard_status status);

/* Text of the last LARARD_E_HIP / validation failure on this thread ("" if none). */
const char* larard_last_error(void);

/* Library version string, e.g. "larard 0.1.0 gfx950 (src 0123456789abcdef)";
 * the src field is a hash of the sources the library was built from. */
const char* larard_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LARARD_H */
