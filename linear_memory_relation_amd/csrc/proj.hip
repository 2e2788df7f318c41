// Projection backward: the gradient of the student projection weights from
// the relation-KL gradient dX_s ("LinearARD: Linear-Memory Attention
// Distillation for RoPE Restoration", paper-notes page, "Method details ->
// Overall framework" and "Loss function / training strategy": stage 1
// updates only the attention projections W_q, W_k, W_v).
//
// Per head the student map is X_s[b,h,i,:] = R(i) (h[b,i,:] W[:, h*d:(h+1)*d])
// with R(i) the student's rotate-half rotation at token i (identity for V),
// so with G[b,h,i,:] = R(i)^T dX_s[b,h,i,:]
//     dW[c, h*d + k] = sum_{b,i} h[b,i,c] G[b,h,i,k].
// Kernels:
//   * rope_t_kernel: G = R^T dX_s in fp32, rounded once to bf16, written
//     K-major as G^T [H*d, Kp] (token index b*n + i along K, columns past
//     B*n zero, Kp a multiple of 64), the tokens of every 16-token group
//     stored in the order in which the LDS transpose read hands them out
//     (gt_pos below);
//   * large outputs (256 x 256 tiles): transpose_h_kernel writes h^T
//     [dm, Kp] in the same token order, and gemm_nt_kernel forms
//     dW[c, hd*d + k] = sum over tokens of h^T[c, tok] G^T[hd*d + k, tok]
//     from two K-major operands;
//   * small outputs (128 x 128 tiles): gemm_kt_kernel forms dW^T tile by
//     tile from G^T and h read token-major in place, through the LDS
//     transpose read (ds_read_b64_tr_b16), and stores it transposed; h then
//     makes no transposed round trip through HBM.  (With 256 x 256 tiles
//     the transpose-read form measured 19% slower than the K-major GEMM at
//     the 16K query shape; with 128 x 128 tiles 25% faster.)
//   All products are bf16 MFMA with fp32 accumulation.
#include <stdint.h>

#include "launch.h"

namespace lmr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTok = 64;          // tokens per GEMM K step

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint16_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);   // round to nearest even (finite inputs)
  return (uint16_t)(r >> 16);
}

// Position of token t of a 64-token block in a G^T row: bits 2 and 3 of t
// swapped.  A 16-byte fragment read of positions 8h .. 8h+7 then yields
// tokens 4h+0..3 and 8+4h+0..3, the order in which the transpose read hands
// a lane the tokens of h (TokTile::frag), so both MFMA operands agree on
// which token each k slot holds.
__device__ inline int gt_pos(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

constexpr int kPitch = kTok + 8;   // LDS row pitch of the G^T staging tile (16-byte aligned rows)

// One block: 64 tokens x all d components of one head.  Reads dX_s rows with
// 16-byte loads, rotates every pair (k, k + d/2) back, stages bf16 values in
// LDS at their permuted positions and writes d rows of 64 tokens of G^T with
// 16-byte stores.
template <int D>
__global__ __launch_bounds__(256) void rope_t_kernel(const float* dx, const float* cosv, const float* sinv,
                                                     int64_t B, int n, int H, int64_t kp, uint16_t* gt) {
  constexpr int HALF = D / 2, TPT = HALF / 4;
  __shared__ __attribute__((aligned(16))) uint16_t tile[D][kPitch];
  const int hd = blockIdx.y;
  const int64_t tok0 = (int64_t)blockIdx.x * kTok;
  const int64_t ntok = B * (int64_t)n;
  for (int e = threadIdx.x; e < kTok * TPT; e += blockDim.x) {
    const int t = e / TPT, q = e % TPT;
    const int64_t tok = tok0 + t;
    float g1[4] = {0.f, 0.f, 0.f, 0.f}, g2[4] = {0.f, 0.f, 0.f, 0.f};
    if (tok < ntok) {
      const int64_t b = tok / n, i = tok % n;
      const float* row = dx + ((b * H + hd) * (int64_t)n + i) * D;
      const f32x4 y1 = *reinterpret_cast<const f32x4*>(row + 4 * q);
      const f32x4 y2 = *reinterpret_cast<const f32x4*>(row + HALF + 4 * q);
      if (cosv != nullptr) {
        const float* cr = cosv + i * HALF + 4 * q;   // the tables need only 4-byte alignment
        const float* sr = sinv + i * HALF + 4 * q;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // forward: y1 = x1 c - x2 s, y2 = x2 c + x1 s; the transpose applied to (y1, y2)
          const float c = cr[k], s = sr[k];
          g1[k] = fmaf(y1[k], c, y2[k] * s);
          g2[k] = fmaf(y2[k], c, -y1[k] * s);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          g1[k] = y1[k];
          g2[k] = y2[k];
        }
      }
    }
    const int pos = gt_pos(t);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      tile[4 * q + k][pos] = bf16_rne(g1[k]);
      tile[HALF + 4 * q + k][pos] = bf16_rne(g2[k]);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < D * (kTok / 8); e += blockDim.x) {
    const int k = e / (kTok / 8), t = 8 * (e % (kTok / 8));
    *reinterpret_cast<uint4*>(gt + ((int64_t)hd * D + k) * kp + tok0 + t) = *reinterpret_cast<const uint4*>(&tile[k][t]);
  }
}

// K-major operand tile of W rows x 64 bf16 (128-byte rows) in LDS, 16-byte
// chunks XOR-swizzled per row: chunk c of row r sits at slot c ^ sw(r).  Two
// rows share a 256-byte bank line; sw takes 8 distinct values over 8
// consecutive row pairs, so the 16 rows read by one fragment instruction
// land in 16 distinct 16-byte bank groups.
__device__ inline int sw(int r) {
  const int m = r >> 1;
  return ((m & 1) << 2) | ((m >> 1) & 3);
}
__device__ inline int slot_off(int r, int c) { return r * 128 + ((c ^ sw(r)) << 4); }

// Copy rows row0 .. row0+32*NW-1, K columns k0 .. k0+63 of a [rows, kp]
// matrix into the tile; NW waves x 4 instructions of 1 KB (16 B per lane).
__device__ inline void load_kmajor(char* lds, const uint16_t* g, int64_t row0, int64_t kp, int64_t k0, int wave,
                                   int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int blk = (wave * 4 + u) * 1024;
    const int P = blk + 16 * lane;
    const int r = P >> 7, pos = (P & 127) >> 4;
    const int c = pos ^ sw(r);
    const uint16_t* src = g + (row0 + r) * kp + k0 + 8 * c;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(lds + blk), 16, 0, 0);
  }
}

// MFMA operand of row r, 16-step ks, lane half h: K positions 16ks+8h .. +7.
__device__ inline bf16x8 frag_kmajor(const char* tile, int r, int ks, int h) {
  return *reinterpret_cast<const bf16x8*>(tile + slot_off(r, 2 * ks + h));
}

// h [ntok, dm] bf16 -> h^T [dm, kp] bf16 in tiles of 64 tokens x 128
// columns, tokens at gt_pos positions, zero padded along K; 16-byte loads
// (8 columns of a token) and stores (8 positions of a column).
__global__ __launch_bounds__(256) void transpose_h_kernel(const uint16_t* h, int64_t ntok, int64_t dm, int64_t kp,
                                                          uint16_t* ht) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[128][kPitch];
  const int64_t tok0 = (int64_t)blockIdx.x * kTok, c0 = (int64_t)blockIdx.y * 128;
  for (int e = threadIdx.x; e < kTok * 16; e += blockDim.x) {
    const int t = e / 16, c = 8 * (e % 16);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tok0 + t < ntok) v = *reinterpret_cast<const uint4*>(h + (tok0 + t) * dm + c0 + c);
    const int pos = gt_pos(t);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[c + 2 * q][pos] = (uint16_t)(w[q] & 0xffffu);
      tile[c + 2 * q + 1][pos] = (uint16_t)(w[q] >> 16);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 128 * (kTok / 8); e += blockDim.x) {
    const int c = e / (kTok / 8), t = 8 * (e % (kTok / 8));
    *reinterpret_cast<uint4*>(ht + (c0 + c) * kp + tok0 + t) = *reinterpret_cast<const uint4*>(&tile[c][t]);
  }
}

// C[M, N] = A[M, K] B[N, K]^T with A, B bf16 K-major (row stride kp, the
// same token order), C fp32 row-major.  Workgroup tile 256 x 256: 8 waves of
// 128 x 64 (two along M, four along N), 4 x 2 blocks of 32 x 32 each; K step
// 64, double-buffered direct global -> LDS copies (128 KiB: one workgroup,
// 2 waves per SIMD, per CU).  The fragments of 16-step ks+1 are read while
// the MFMAs of step ks run.
__global__ __launch_bounds__(512, 1) void gemm_nt_kernel(const uint16_t* A, const uint16_t* Bm, int64_t kp, int64_t N,
                                                         float* C) {
  constexpr int MI = 4;
  __shared__ __attribute__((aligned(1024))) char lds[2][2][256 * 128];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.y * 256, n0 = (int64_t)blockIdx.x * 256;
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 64;
  f32x16 acc[MI][2] = {};
  const int64_t nk = kp / kTok;
  if (nk > 0) {
    load_kmajor(lds[0][0], A, m0, kp, 0, wave, lane);
    load_kmajor(lds[0][1], Bm, n0, kp, 0, wave, lane);
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) {
      load_kmajor(lds[buf ^ 1][0], A, m0, kp, (kt + 1) * kTok, wave, lane);
      load_kmajor(lds[buf ^ 1][1], Bm, n0, kp, (kt + 1) * kTok, wave, lane);
    }
    const char* ta = lds[buf][0];
    const char* tb = lds[buf][1];
    bf16x8 fa[2][MI], fb[2][2];
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[0][i] = frag_kmajor(ta, wm + 32 * i + l32, 0, h);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[0][j] = frag_kmajor(tb, wn + 32 * j + l32, 0, h);
#pragma unroll
    for (int ks = 0; ks < kTok / 16; ++ks) {
      const int cur = ks & 1;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][0], fb[cur][j], acc[0][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < kTok / 16) {
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[cur ^ 1][i] = frag_kmajor(ta, wm + 32 * i + l32, ks + 1, h);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[cur ^ 1][j] = frag_kmajor(tb, wn + 32 * j + l32, ks + 1, h);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 1; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    }
  }
  // C register r of block (i, j): row wm + 32i + 8(r/4) + 4h + r%4, column wn + 32j + l32.
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        C[row * N + n0 + wn + 32 * j + l32] = acc[i][j][r];
      }
}

// Token-major operand tile in LDS: kTok token rows of W bf16 columns
// (2W bytes per row), 16-byte chunks XOR-swizzled per row: chunk c of row r
// sits at slot c ^ 4(r & 3).  A transpose read covers 8 rows x 32 columns
// (rows 16q + 4h + 0..3 for the two lane halves h); its four rows r & 3 =
// 0..3 of one half land in the four 64-byte quarters of a 256-byte bank
// line, so each instruction takes the minimum two passes.
template <int W>
struct TokTile {
  static constexpr int RB = 2 * W;
  static constexpr int BYTES = kTok * RB;
  __device__ static inline int off(int r, int c) { return r * RB + ((c ^ (4 * (r & 3))) << 4); }
  // Copy token rows k0 .. k0+63 (rows >= rows_valid are read from the last
  // valid row and zeroed later), columns col0 .. col0+W-1 of a token-major
  // [rows, ld] matrix; NW waves, 1 KB per wave-instruction.
  template <int NW>
  __device__ static inline void load(char* lds, const uint16_t* g, int64_t ld, int64_t col0, int64_t k0,
                                     int64_t rows_valid, int wave, int lane) {
    constexpr int U = BYTES / 1024 / NW;
    static_assert(U * 1024 * NW == BYTES, "tile copy split");
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = (wave * U + u) * 1024;
      const int P = blk + 16 * lane;
      const int r = P / RB, pos = (P % RB) >> 4;
      const int c = pos ^ (4 * (r & 3));
      const int64_t gr = min(k0 + r, rows_valid - 1);
      const uint16_t* src = g + gr * ld + col0 + 8 * c;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(lds + blk), 16, 0, 0);
    }
  }
  // After this wave's copies have landed: zero the 16-byte slots it copied
  // from rows past rows_valid (the token tail of the last K step).
  template <int NW>
  __device__ static inline void zero_tail(char* lds, int64_t k0, int64_t rows_valid, int wave, int lane) {
    constexpr int U = BYTES / 1024 / NW;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int P = (wave * U + u) * 1024 + 16 * lane;
      if (k0 + P / RB >= rows_valid) *reinterpret_cast<uint4*>(lds + P) = make_uint4(0, 0, 0, 0);
    }
  }
  // MFMA operand of 32 columns col .. col+31 and 16-token step ks: lane
  // (column col + lane%32, half h) gets tokens 16ks+4h+0..3 and
  // 16ks+8+4h+0..3 (the same token order for both operands of a product).
  __device__ static inline bf16x8 frag(const char* base, int col, int ks, int lane) {
    const int G = lane >> 4, L = lane & 15, h = G >> 1;
    const int row = 16 * ks + 4 * h + (L >> 2);
    const int cc = col + 16 * (G & 1) + 4 * (L & 3);
    const int c = cc >> 3, sub = (cc & 7) * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off(row, c) + sub));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off(row + 8, c) + sub));
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
    return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// C^T tile product: Ct[m, n] = sum over tokens of A[m, tok] B[tok, n] with
// A K-major [M rows, kp] (G^T, tokens permuted by gt_pos), B token-major
// [ntok, ldb] (h), and Ct stored transposed into C [N, ldc] fp32 (dW).  W x W
// output tile per workgroup, 2*W/64 waves (8 for W = 256, 4 for W = 128),
// wave tile (W/2) x 64 (W/64 x 2 blocks of 32 x 32), double-buffered direct
// global -> LDS copies, one barrier per 64-token step.
template <int W>
__global__ __launch_bounds__(W * 2, 1) void gemm_kt_kernel(const uint16_t* A, int64_t kp, const uint16_t* Bm,
                                                           int64_t ldb, int64_t ntok, int64_t ldc, float* C) {
  constexpr int NW = 2 * W / 64, MI = W / 64, TB = W * 128;
  static_assert(TokTile<W>::BYTES == TB, "both operand tiles take W x 128 bytes");
  __shared__ __attribute__((aligned(1024))) char lds[2][2][TB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.y * W, n0 = (int64_t)blockIdx.x * W;
  const int wm = (wave & 1) * (W / 2), wn = (wave >> 1) * 64;
  f32x16 acc[MI][2] = {};
  const int64_t nk = kp / kTok;
  if (nk > 0) {
    load_kmajor(lds[0][0], A, m0, kp, 0, wave, lane);
    TokTile<W>::template load<NW>(lds[0][1], Bm, ldb, n0, 0, ntok, wave, lane);
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if ((kt + 1) * kTok > ntok) TokTile<W>::template zero_tail<NW>(lds[buf][1], kt * kTok, ntok, wave, lane);
    __syncthreads();
    if (kt + 1 < nk) {
      load_kmajor(lds[buf ^ 1][0], A, m0, kp, (kt + 1) * kTok, wave, lane);
      TokTile<W>::template load<NW>(lds[buf ^ 1][1], Bm, ldb, n0, (kt + 1) * kTok, ntok, wave, lane);
    }
    const char* ta = lds[buf][0];
    const char* tb = lds[buf][1];
    // Fragments of 16-step ks+1 are read while the MFMAs of step ks run:
    // after the first two MFMAs of step ks (whose operands arrived during
    // step ks-1), so the waits before them cover older reads only.
    bf16x8 fa[2][MI], fb[2][2];
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[0][i] = frag_kmajor(ta, wm + 32 * i + l32, 0, h);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[0][j] = TokTile<W>::frag(tb, wn + 32 * j, 0, lane);
#pragma unroll
    for (int ks = 0; ks < kTok / 16; ++ks) {
      const int cur = ks & 1;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][0], fb[cur][j], acc[0][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < kTok / 16) {
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[cur ^ 1][i] = frag_kmajor(ta, wm + 32 * i + l32, ks + 1, h);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[cur ^ 1][j] = TokTile<W>::frag(tb, wn + 32 * j, ks + 1, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 1; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    }
  }
  // Ct register r of block (i, j): row m = wm + 32i + 8(r/4) + 4h + r%4,
  // column n = wn + 32j + l32; four consecutive m per lane go out as one
  // 16-byte store into row n of C.
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int64_t col = n0 + wn + 32 * j + l32;
        const int64_t row = m0 + wm + 32 * i + 8 * g4 + 4 * h;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g4 + e];
        *reinterpret_cast<f32x4*>(C + col * ldc + row) = v;
      }
}

}  // namespace

// The 256 x 256 tile only when its grid still covers every CU (256).
bool proj_uses_256_tiles(int64_t dm, int64_t hd) {
  return dm % 256 == 0 && hd % 256 == 0 && (dm / 256) * (hd / 256) >= 256;
}

namespace {

hipError_t launch_gemm(const ProjArgs& p, int64_t ntok, int64_t HD, hipStream_t st) {
  if (proj_uses_256_tiles(p.dm, HD)) {
    if (p.kp > 0) {
      hipLaunchKernelGGL(transpose_h_kernel, dim3((unsigned)(p.kp / kTok), (unsigned)(p.dm / 128)), dim3(256), 0, st,
                         p.h, ntok, p.dm, p.kp, p.ht);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(gemm_nt_kernel, dim3((unsigned)(HD / 256), (unsigned)(p.dm / 256)), dim3(512), 0, st, p.ht,
                       p.g, p.kp, HD, p.dw);
  } else {
    hipLaunchKernelGGL(gemm_kt_kernel<128>, dim3((unsigned)(p.dm / 128), (unsigned)(HD / 128)), dim3(256), 0, st, p.g,
                       p.kp, p.h, p.dm, ntok, HD, p.dw);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_bwd(const ProjArgs& p, hipStream_t st) {
  const int64_t ntok = p.B * p.n;
  const int64_t HD = p.H * p.d;
  if (p.kp == 0)   // no tokens: the GEMM runs no K step and writes dW = 0
    return launch_gemm(p, ntok, HD, st);
  const dim3 grid((unsigned)(p.kp / kTok), (unsigned)p.H);
  if (p.d == 64)
    hipLaunchKernelGGL(rope_t_kernel<64>, grid, dim3(256), 0, st, p.dx, p.cos, p.sin, p.B, (int)p.n, (int)p.H, p.kp, p.g);
  else
    hipLaunchKernelGGL(rope_t_kernel<128>, grid, dim3(256), 0, st, p.dx, p.cos, p.sin, p.B, (int)p.n, (int)p.H, p.kp, p.g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gemm(p, ntok, HD, st);
}

}  // namespace lmr
