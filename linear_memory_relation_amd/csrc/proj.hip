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
// Three kernels:
//   * rope_t_kernel: G = R^T dX_s in fp32, rounded once to bf16, written
//     transposed as G^T [H*d, Kp] (token index b*n + i along K, zero padded
//     to Kp, a multiple of 64);
//   * transpose_h_kernel: h^T [D, Kp] bf16 (D a multiple of 128);
//   * gemm_nt_kernel / gemm_nt_256_kernel: dW[M=D, N=H*d] = h^T G (both
//     operands K-contiguous), bf16 MFMA with fp32 accumulation, a 128x128 or
//     256x256 output tile per workgroup.
#include <stdint.h>

#include "launch.h"

namespace lmr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTok = 64;          // tokens per transpose tile (= GEMM K step)

__device__ inline uint16_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);   // round to nearest even (finite inputs)
  return (uint16_t)(r >> 16);
}

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
constexpr int kPitch = kTok + 8;   // LDS row pitch of the transpose tiles (16-byte aligned rows)

// One block: 64 tokens x all d components of one head.  Reads dX_s rows
// (d fp32 each), rotates every pair (k, k + d/2) back, stages bf16 values in
// LDS and writes d rows of 64 tokens of G^T.
template <int D>
__global__ __launch_bounds__(256) void rope_t_kernel(const float* dx, const float* cosv, const float* sinv,
                                                     int64_t B, int n, int H, int64_t kp, uint16_t* gt) {
  __shared__ uint16_t tile[D][kTok + 2];
  const int hd = blockIdx.y;
  const int64_t tok0 = (int64_t)blockIdx.x * kTok;
  const int64_t ntok = B * (int64_t)n;
  constexpr int HALF = D / 2;
  for (int e = threadIdx.x; e < kTok * HALF; e += blockDim.x) {
    const int t = e / HALF, k = e % HALF;
    const int64_t tok = tok0 + t;
    float g1 = 0.f, g2 = 0.f;
    if (tok < ntok) {
      const int64_t b = tok / n, i = tok % n;
      const float* row = dx + ((b * H + hd) * (int64_t)n + i) * D;
      const float y1 = row[k], y2 = row[k + HALF];
      if (cosv != nullptr) {
        const float c = cosv[i * HALF + k], s = sinv[i * HALF + k];
        // forward: y1 = x1 c - x2 s, y2 = x2 c + x1 s; transpose applied to (y1, y2)
        g1 = fmaf(y1, c, y2 * s);
        g2 = fmaf(y2, c, -y1 * s);
      } else {
        g1 = y1;
        g2 = y2;
      }
    }
    tile[k][t] = bf16_rne(g1);
    tile[k + HALF][t] = bf16_rne(g2);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < D * kTok; e += blockDim.x) {
    const int k = e / kTok, t = e % kTok;
    gt[((int64_t)hd * D + k) * kp + tok0 + t] = tile[k][t];
  }
}

// h [ntok, Dm] bf16 -> h^T [Dm, kp] bf16 in tiles of 64 tokens x 128 columns,
// zero padded along K; 16-byte loads (8 columns of a token) and stores (8
// tokens of a column).
__global__ __launch_bounds__(256) void transpose_h_kernel(const uint16_t* h, int64_t ntok, int64_t dm, int64_t kp,
                                                          uint16_t* ht) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[128][kPitch];
  const int64_t tok0 = (int64_t)blockIdx.x * kTok, c0 = (int64_t)blockIdx.y * 128;
  for (int e = threadIdx.x; e < kTok * 16; e += blockDim.x) {
    const int t = e / 16, c = 8 * (e % 16);
    u16x8 v = {};
    if (tok0 + t < ntok) v = *reinterpret_cast<const u16x8*>(h + (tok0 + t) * dm + c0 + c);
#pragma unroll
    for (int q = 0; q < 8; ++q) tile[c + q][t] = v[q];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 128 * (kTok / 8); e += blockDim.x) {
    const int c = e / (kTok / 8), t = 8 * (e % (kTok / 8));
    *reinterpret_cast<u16x8*>(ht + (c0 + c) * kp + tok0 + t) = *reinterpret_cast<const u16x8*>(&tile[c][t]);
  }
}

// K-contiguous operand tile of 128 rows x 64 bf16 (128-byte rows) in LDS,
// 16-byte chunks XOR-swizzled per row: chunk c of row r sits at slot
// c ^ sw(r).  Two rows share a 256-byte bank line; sw takes 8 distinct
// values over 8 consecutive row pairs, so the 16 rows read by one fragment
// instruction land in 16 distinct 16-byte bank groups.
__device__ inline int sw(int r) {
  const int m = r >> 1;
  return ((m & 1) << 2) | ((m >> 1) & 3);
}
__device__ inline int slot_off(int r, int c) { return r * 128 + ((c ^ sw(r)) << 4); }

// Copy rows row0..row0+32*NW-1, K columns k0..k0+63 of a [rows, kp] matrix
// into the tile; NW waves x 4 instructions of 1 KB (16 B per lane), so 4 waves
// copy 128 rows and 8 waves 256.
__device__ inline void load_tile(char* lds, const uint16_t* g, int64_t row0, int64_t kp, int64_t k0, int wave,
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

__device__ inline bf16x8 frag(const char* tile, int r, int ks, int h) {
  return *reinterpret_cast<const bf16x8*>(tile + slot_off(r, 2 * ks + h));
}

// C[M, N] = A[M, K] B[N, K]^T with A, B bf16 K-contiguous (row stride kp),
// C fp32 row-major.  Workgroup tile 128 x 128, wave tile 64 x 64 (2 x 2
// blocks of 32 x 32), K step 64, double-buffered direct global -> LDS copies.
__global__ __launch_bounds__(256, 2) void gemm_nt_kernel(const uint16_t* A, const uint16_t* Bm, int64_t kp,
                                                         int64_t N, float* C) {
  __shared__ __attribute__((aligned(1024))) char lds[2][2][128 * 128];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.y * 128, n0 = (int64_t)blockIdx.x * 128;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x16 acc[2][2] = {};
  const int64_t nk = kp / 64;
  if (nk > 0) {
    load_tile(lds[0][0], A, m0, kp, 0, wave, lane);
    load_tile(lds[0][1], Bm, n0, kp, 0, wave, lane);
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) {
      load_tile(lds[buf ^ 1][0], A, m0, kp, (kt + 1) * 64, wave, lane);
      load_tile(lds[buf ^ 1][1], Bm, n0, kp, (kt + 1) * 64, wave, lane);
    }
    const char* ta = lds[buf][0];
    const char* tb = lds[buf][1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = frag(ta, wm + 32 * i + l32, ks, h);
        fb[i] = frag(tb, wn + 32 * i + l32, ks, h);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
  // C register r of block (i, j): row wm + 32i + 8(r/4) + 4h + r%4, column wn + 32j + l32.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        C[row * N + n0 + wn + 32 * j + l32] = acc[i][j][r];
      }
}

// The same product with a 256 x 256 workgroup tile: 8 waves of 128 x 64 (two
// along M, four along N), 4 x 2 blocks of 32 x 32 each.  Per 16-step a wave
// reads 6 fragments for 8 MFMAs (the 128 x 128 kernel: 4 for 4), and every
// copied operand row serves twice as many outputs.  128 KiB of LDS: one
// workgroup (2 waves per SIMD) per CU.
__global__ __launch_bounds__(512) void gemm_nt_256_kernel(const uint16_t* A, const uint16_t* Bm, int64_t kp,
                                                          int64_t N, float* C) {
  __shared__ __attribute__((aligned(1024))) char lds[2][2][256 * 128];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.y * 256, n0 = (int64_t)blockIdx.x * 256;
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 64;
  f32x16 acc[4][2] = {};
  const int64_t nk = kp / 64;
  if (nk > 0) {
    load_tile(lds[0][0], A, m0, kp, 0, wave, lane);
    load_tile(lds[0][1], Bm, n0, kp, 0, wave, lane);
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) {
      load_tile(lds[buf ^ 1][0], A, m0, kp, (kt + 1) * 64, wave, lane);
      load_tile(lds[buf ^ 1][1], Bm, n0, kp, (kt + 1) * 64, wave, lane);
    }
    const char* ta = lds[buf][0];
    const char* tb = lds[buf][1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = frag(ta, wm + 32 * i + l32, ks, h);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = frag(tb, wn + 32 * j + l32, ks, h);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        C[row * N + n0 + wn + 32 * j + l32] = acc[i][j][r];
      }
}

// The 256 x 256 tile only when its grid still covers every CU (256).
bool use_256_tiles(int64_t M, int64_t N) { return M % 256 == 0 && N % 256 == 0 && (M / 256) * (N / 256) >= 256; }

hipError_t launch_gemm(const uint16_t* A, const uint16_t* Bm, int64_t kp, int64_t M, int64_t N, float* C,
                       hipStream_t st) {
  if (use_256_tiles(M, N))
    hipLaunchKernelGGL(gemm_nt_256_kernel, dim3((unsigned)(N / 256), (unsigned)(M / 256)), dim3(512), 0, st, A, Bm,
                       kp, N, C);
  else
    hipLaunchKernelGGL(gemm_nt_kernel, dim3((unsigned)(N / 128), (unsigned)(M / 128)), dim3(256), 0, st, A, Bm, kp,
                       N, C);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_bwd(const ProjArgs& p, hipStream_t st) {
  const int64_t ntok = p.B * p.n;
  const int64_t N = p.H * p.d;
  hipError_t e;
  if (p.kp == 0)   // no tokens: the GEMM runs no K step and writes dW = 0
    return launch_gemm(p.ht, p.gt, p.kp, p.dm, N, p.dw, st);
  const dim3 tgrid((unsigned)(p.kp / kTok), (unsigned)p.H);
  if (p.d == 64)
    hipLaunchKernelGGL(rope_t_kernel<64>, tgrid, dim3(256), 0, st, p.dx, p.cos, p.sin, p.B, (int)p.n, (int)p.H, p.kp, p.gt);
  else
    hipLaunchKernelGGL(rope_t_kernel<128>, tgrid, dim3(256), 0, st, p.dx, p.cos, p.sin, p.B, (int)p.n, (int)p.H, p.kp, p.gt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(transpose_h_kernel, dim3((unsigned)(p.kp / kTok), (unsigned)(p.dm / 128)), dim3(256), 0, st,
                     p.h, ntok, p.dm, p.kp, p.ht);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_gemm(p.ht, p.gt, p.kp, p.dm, N, p.dw, st);
}

}  // namespace lmr
