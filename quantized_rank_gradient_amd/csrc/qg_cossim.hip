// Subspace similarity of the layer-adaptive refresh schedule (AIMech curated page on
// Q-GaLore, mechanism claim "layer-adaptive subspace cosine schedule", paper Section 3.1,
// Equation (5)): CosSim(P_new, P_old) = (1/r) * sum_i sigma_i(P_new^T P_old).
//
// For a batch of projection pairs (same rank r, any row counts):
//   1. C = P~_new^T P~_old (r x r) on bf16 MFMA, INT4 dequant in LDS, split over the rows.
//   2. The nuclear norm of C as trace(X^T C), where X is the orthogonal polar factor of C,
//      obtained by Newton-Schulz iterations on X, which map every singular value of X
//      through an odd polynomial while keeping its singular vectors:
//        * X0 = C / ||C||_F, then rescaled by ||X0^T X0||_F^(-1/2) = (sum_i s_i^4)^(-1/4),
//          which keeps every singular value at most 1 and brings the large ones near 1;
//        * quintic steps X <- a X + X (b A + c A^2), A = X^T X, with the coefficients of
//          the Muon optimizer's orthogonalization (Jordan et al., 2024: a = 3.4445,
//          b = -4.7750, c = 2.0315): small singular values grow 3.4x per step, and values
//          already lifted stay in [0.68, 1.2];
//        * cubic steps X <- 1.5 X - 0.5 X A, which converge all of them to 1.
//      All but the last steps run with bf16 operands; the last ones use hi/lo split operands
//      (about 16 significant bits) so that X ends orthogonal to fp32-level accuracy.
//      trace(X^T C) is maximal at the exact polar factor, so what error the bf16 steps leave
//      in X enters the trace only to second order.
#include "qg_gemm.hpp"
#include "qg_kernels.hpp"

namespace qg {

using CosTile = Tile<128, 128, 32, 2, 2, true, true>;     // C = P~n^T P~o, X^T X
using NsTileNN = Tile<128, 128, 32, 2, 2, false, true>;   // X A

// --------------------------------------------------------------- fp32 -> LDS stagers ---
// fp32 sources are rounded to bf16 on the way into LDS; with PARTS == 2 the bf16 remainder
// x - bf16(x) goes to a second copy LO_OFF elements further on.

// fp32 source [k][c] (row pitch ld, ld % 8 == 0) -> K-major LDS tile [k][c].
template <int W, int BK, int PARTS, int LO_OFF>
struct StageF32K {
  static constexpr int CPR = W / 8;
  static constexpr int NC = BK * CPR / kThreads;
  const float* src;
  int64_t ld, k_end, c_end;
  int c0;
  float f[NC][8];

  __device__ StageF32K(const float* s, int64_t ld_, int64_t k_end_, int64_t c_end_, int c0_)
      : src(s), ld(ld_), k_end(k_end_), c_end(c_end_), c0(c0_) {}

  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      const int64_t k = k0 + q / CPR;
      const int64_t c = c0 + 8 * (q % CPR);
      if (k < k_end && c < c_end) {
        const float4 x = gload(reinterpret_cast<const float4*>(src + k * ld + c));
        const float4 y = gload(reinterpret_cast<const float4*>(src + k * ld + c + 4));
        f[u][0] = x.x; f[u][1] = x.y; f[u][2] = x.z; f[u][3] = x.w;
        f[u][4] = y.x; f[u][5] = y.y; f[u][6] = y.z; f[u][7] = y.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[u][e] = 0.0f;
      }
    }
  }

  template <int PITCH>
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      const int off = (q / CPR) * PITCH + 8 * (q % CPR);
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = pack_bf16x2(f[u][2 * e], f[u][2 * e + 1]);
        if constexpr (PARTS == 2)
          l[e] = pack_bf16x2(f[u][2 * e] - bf16_to_f32(h[e] & 0xFFFFu),
                             f[u][2 * e + 1] - bf16_to_f32(h[e] >> 16));
      }
      *reinterpret_cast<uint4*>(lds + off) = make_uint4(h[0], h[1], h[2], h[3]);
      if constexpr (PARTS == 2)
        *reinterpret_cast<uint4*>(lds + LO_OFF + off) = make_uint4(l[0], l[1], l[2], l[3]);
    }
  }
};

// fp32 source [c][k] (row pitch ld = the K extent, ld % 8 == 0) -> K-contiguous LDS [c][k].
template <int W, int BK, int PARTS, int LO_OFF>
struct StageF32C {
  static constexpr int CPR = BK / 8;
  static constexpr int NC = W * CPR / kThreads;
  const float* src;
  int64_t ld, c_end;
  int c0;
  float f[NC][8];

  __device__ StageF32C(const float* s, int64_t ld_, int64_t c_end_, int c0_)
      : src(s), ld(ld_), c_end(c_end_), c0(c0_) {}

  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      const int64_t row = c0 + q / CPR;
      const int64_t k = k0 + 8 * (q % CPR);
      if (row < c_end && k < ld) {
        const float4 x = gload(reinterpret_cast<const float4*>(src + row * ld + k));
        const float4 y = gload(reinterpret_cast<const float4*>(src + row * ld + k + 4));
        f[u][0] = x.x; f[u][1] = x.y; f[u][2] = x.z; f[u][3] = x.w;
        f[u][4] = y.x; f[u][5] = y.y; f[u][6] = y.z; f[u][7] = y.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[u][e] = 0.0f;
      }
    }
  }

  template <int PITCH>
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      static_assert(PITCH == 32 && CPR == 4, "K-contiguous tiles take 32-element rows");
      const int off = kc_off(q / CPR, q % CPR);
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = pack_bf16x2(f[u][2 * e], f[u][2 * e + 1]);
        if constexpr (PARTS == 2)
          l[e] = pack_bf16x2(f[u][2 * e] - bf16_to_f32(h[e] & 0xFFFFu),
                             f[u][2 * e + 1] - bf16_to_f32(h[e] >> 16));
      }
      *reinterpret_cast<uint4*>(lds + off) = make_uint4(h[0], h[1], h[2], h[3]);
      if constexpr (PARTS == 2)
        *reinterpret_cast<uint4*>(lds + LO_OFF + off) = make_uint4(l[0], l[1], l[2], l[3]);
    }
  }
};

// ------------------------------------------------------------------ batch lookups ---

__device__ __forceinline__ int pair_of_block(const CosBatch& b, int blk, int& local) {
  int p = 0;
  while (p + 1 < b.count && blk >= b.pair[p + 1].gemm_base) ++p;
  local = blk - b.pair[p].gemm_base;
  return p;
}

__device__ __forceinline__ float* pair_mat(const CosBatch& b, int p, int64_t off) {
  return reinterpret_cast<float*>(b.ws + (int64_t)p * b.pair_stride + off);
}

// ------------------------------------------------------------- 1: C = P~n^T P~o ---

__global__ __launch_bounds__(kThreads) void qg_cossim_gemm(CosBatch b) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * CosTile::STAGE];
  int local;
  const int p = pair_of_block(b, blockIdx.x, local);
  const CosPair& q = b.pair[p];
  const int per_split = b.tiles * b.tiles;
  const int s = local / per_split;
  const int rem = local - s * per_split;
  const int ti = rem / b.tiles, tj = rem - ti * b.tiles;
  const int i0 = ti * CosTile::BM, j0 = tj * CosTile::BN;
  const int64_t k_begin = (int64_t)s * q.kslab;
  const int64_t k_end = min<int64_t>(q.m, k_begin + q.kslab);
  StageInt4K<128, CosTile::BK> sa(q.qa, q.sa, b.r, q.m, k_end, b.r, i0);
  StageInt4K<128, CosTile::BK> sb(q.qb, q.sb, b.r, q.m, k_end, b.r, j0);
  f32x16 acc[2][2];
  gemm_kloop<CosTile, 1>(
      sa, sb, [](auto& st, uint16_t* p) { st.template store<CosTile::A_PITCH>(p); },
      [](auto& st, uint16_t* p) { st.template store<CosTile::B_PITCH>(p + CosTile::A_ELEMS); },
      k_begin, k_end, lds, acc);
  float* out = pair_mat(b, p, b.off_part) + (int64_t)s * b.r * b.r;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int64_t j = j0 + acc_col<CosTile>(y);
      if (j >= b.r) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + acc_row<CosTile>(x, v);
        if (i < b.r) gstore(out + i * b.r + j, (float)acc[x][y][v]);
      }
    }
}

// ------------------------------------- 2a: sum split partials, per-block squares ---

// grid = count * nblk; each thread handles 4 consecutive elements of its pair's C.
__global__ __launch_bounds__(kThreads) void qg_cossim_reduce(CosBatch b) {
  __shared__ float red[kThreads];
  const int p = blockIdx.x / b.nblk;
  const int blk = blockIdx.x - p * b.nblk;
  const int64_t n2 = (int64_t)b.r * b.r;
  const int64_t e0 = ((int64_t)blk * kThreads + threadIdx.x) * 4;
  const float* part = pair_mat(b, p, b.off_part);
  float* C = pair_mat(b, p, b.off_c);
  float sq = 0.0f;
  if (e0 < n2) {   // n2 is a multiple of 64 since r % 8 == 0
    float4 v = gload(reinterpret_cast<const float4*>(part + e0));
    for (int s = 1; s < b.pair[p].split; ++s) {
      const float4 w = gload(reinterpret_cast<const float4*>(part + (int64_t)s * n2 + e0));
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    gstore(reinterpret_cast<float4*>(C + e0), v);
    sq = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  red[threadIdx.x] = sq;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) pair_mat(b, p, b.off_blk)[blk] = red[0];
}

// 2b: one workgroup per pair folds the block sums (fixed order) into the pair's scalar slot.
__global__ __launch_bounds__(kThreads) void qg_cossim_fold(CosBatch b, int64_t off_dst,
                                                          float inv_r, float* out) {
  __shared__ double red[kThreads];
  const int p = blockIdx.x;
  const float* blk = pair_mat(b, p, b.off_blk);
  double acc = 0.0;
  for (int k = threadIdx.x; k < b.nblk; k += kThreads) acc += blk[k];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (out)
      out[p] = (float)(red[0] * inv_r);
    else
      pair_mat(b, p, off_dst)[0] = (float)red[0];
  }
}

// 2c: X0 = C / ||C||_F.
__global__ __launch_bounds__(kThreads) void qg_cossim_init(CosBatch b) {
  const int p = blockIdx.x / b.nblk;
  const int blk = blockIdx.x - p * b.nblk;
  const int64_t n2 = (int64_t)b.r * b.r;
  const int64_t e0 = ((int64_t)blk * kThreads + threadIdx.x) * 4;
  if (e0 >= n2) return;
  const float sq = pair_mat(b, p, b.off_norm)[0];
  const float inv = sq > 0.0f ? 1.0f / sqrtf(sq) : 0.0f;
  const float4 c = gload(reinterpret_cast<const float4*>(pair_mat(b, p, b.off_c) + e0));
  gstore(reinterpret_cast<float4*>(pair_mat(b, p, b.off_x) + e0),
         make_float4(c.x * inv, c.y * inv, c.z * inv, c.w * inv));
}

// ---------------------------------------------------- 3: Newton-Schulz products ---

// TA: Y = beta * (M^T M) + alpha * E      (M at off_m; E at off_e, skipped when alpha == 0)
// !TA: Y = alpha * E + beta * (M Bop)     (Bop at off_bop)
template <bool TA, int PARTS>
__global__ __launch_bounds__(kThreads) void qg_ns_gemm(CosBatch b, int64_t off_m,
                                                      int64_t off_bop, int64_t off_e,
                                                      int64_t off_y, float alpha, float beta) {
  constexpr int STAGE = CosTile::STAGE > NsTileNN::STAGE ? CosTile::STAGE : NsTileNN::STAGE;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * PARTS * STAGE];
  const int per_pair = b.tiles * b.tiles;
  const int p = blockIdx.x / per_pair;
  const int rem = blockIdx.x - p * per_pair;
  const int ti = rem / b.tiles, tj = rem - ti * b.tiles;
  const int i0 = ti * CosTile::BM, j0 = tj * CosTile::BN;
  const int r = b.r;
  const float* M = pair_mat(b, p, off_m);
  const float* E = pair_mat(b, p, off_e);
  float* Y = pair_mat(b, p, off_y);
  f32x16 acc[2][2];
  if constexpr (TA) {
    using T = CosTile;
    StageF32K<128, T::BK, PARTS, T::STAGE> sa(M, r, r, r, i0);
    StageF32K<128, T::BK, PARTS, T::STAGE> sb(M, r, r, r, j0);
    gemm_kloop<T, PARTS>(
        sa, sb, [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); },
        [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); }, 0, r, lds,
        acc);
  } else {
    using T = NsTileNN;
    StageF32C<128, T::BK, PARTS, T::STAGE> sa(M, r, r, i0);
    StageF32K<128, T::BK, PARTS, T::STAGE> sb(pair_mat(b, p, off_bop), r, r, r, j0);
    gemm_kloop<T, PARTS>(
        sa, sb, [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); },
        [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); }, 0, r, lds,
        acc);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int64_t j = j0 + acc_col<CosTile>(y);
      if (j >= r) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + acc_row<CosTile>(x, v);
        if (i >= r) continue;
        float out = beta * acc[x][y][v];
        if (alpha != 0.0f) out += alpha * gload(E + i * r + j);
        gstore(Y + i * r + j, out);
      }
    }
}

// ------------------------------------------- 4: sum of X .* Y per pair, rescaling ---

// Per-block partial sums of the elementwise product of two r x r matrices of each pair
// (trace(X^T Y)); sum of squares when X == Y.
__global__ __launch_bounds__(kThreads) void qg_cossim_dot(CosBatch b, int64_t off_x,
                                                         int64_t off_y) {
  __shared__ float red[kThreads];
  const int p = blockIdx.x / b.nblk;
  const int blk = blockIdx.x - p * b.nblk;
  const int64_t n2 = (int64_t)b.r * b.r;
  const int64_t e0 = ((int64_t)blk * kThreads + threadIdx.x) * 4;
  float acc = 0.0f;
  if (e0 < n2) {
    const float4 x = gload(reinterpret_cast<const float4*>(pair_mat(b, p, off_x) + e0));
    const float4 c = gload(reinterpret_cast<const float4*>(pair_mat(b, p, off_y) + e0));
    acc = x.x * c.x + x.y * c.y + x.z * c.z + x.w * c.w;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) pair_mat(b, p, b.off_blk)[blk] = red[0];
}

// X *= s and A *= s^2 with s = ||A||_F^(-1/2) (A = X^T X): afterwards the singular values of
// X are s_i / (sum_j s_j^4)^(1/4) <= 1.
__global__ __launch_bounds__(kThreads) void qg_ns_rescale(CosBatch b) {
  const int p = blockIdx.x / b.nblk;
  const int blk = blockIdx.x - p * b.nblk;
  const int64_t n2 = (int64_t)b.r * b.r;
  const int64_t e0 = ((int64_t)blk * kThreads + threadIdx.x) * 4;
  if (e0 >= n2) return;
  const float sq = pair_mat(b, p, b.off_norm)[1];   // ||A||_F^2
  const float s = sq > 0.0f ? 1.0f / sqrtf(sqrtf(sq)) : 0.0f;
  const float s2 = s * s;
  float4* X = reinterpret_cast<float4*>(pair_mat(b, p, b.off_x) + e0);
  float4* A = reinterpret_cast<float4*>(pair_mat(b, p, b.off_a) + e0);
  const float4 x = gload(X), a = gload(A);
  gstore(X, make_float4(x.x * s, x.y * s, x.z * s, x.w * s));
  gstore(A, make_float4(a.x * s2, a.y * s2, a.z * s2, a.w * s2));
}

// ------------------------------------------------------------------------ driver ---

hipError_t launch_cossim_batch(const CosBatch& b, float* out, hipStream_t s) {
  constexpr float kQa = 3.4445f, kQb = -4.7750f, kQc = 2.0315f;
  int gemm_blocks = 0;
  for (int p = 0; p < b.count; ++p) gemm_blocks += b.pair[p].split * b.tiles * b.tiles;
  hipLaunchKernelGGL(qg_cossim_gemm, dim3(gemm_blocks), dim3(kThreads), 0, s, b);
  const int eblocks = b.count * b.nblk;
  hipLaunchKernelGGL(qg_cossim_reduce, dim3(eblocks), dim3(kThreads), 0, s, b);
  hipLaunchKernelGGL(qg_cossim_fold, dim3(b.count), dim3(kThreads), 0, s, b, b.off_norm, 0.0f,
                     (float*)nullptr);
  hipLaunchKernelGGL(qg_cossim_init, dim3(eblocks), dim3(kThreads), 0, s, b);
  const int nsb = b.count * b.tiles * b.tiles;
  // A = X0^T X0 and the rescaling by ||A||_F^(-1/2)
  hipLaunchKernelGGL((qg_ns_gemm<true, 1>), dim3(nsb), dim3(kThreads), 0, s, b, b.off_x,
                     int64_t(0), b.off_a, b.off_a, 0.0f, 1.0f);
  hipLaunchKernelGGL(qg_cossim_dot, dim3(eblocks), dim3(kThreads), 0, s, b, b.off_a, b.off_a);
  hipLaunchKernelGGL(qg_cossim_fold, dim3(b.count), dim3(kThreads), 0, s, b,
                     b.off_norm + (int64_t)sizeof(float), 0.0f, (float*)nullptr);
  hipLaunchKernelGGL(qg_ns_rescale, dim3(eblocks), dim3(kThreads), 0, s, b);
  int64_t x = b.off_x, xn = b.off_xn;
  for (int it = 0; it < b.iters_quintic; ++it) {
    if (it > 0)
      hipLaunchKernelGGL((qg_ns_gemm<true, 1>), dim3(nsb), dim3(kThreads), 0, s, b, x,
                         int64_t(0), b.off_a, b.off_a, 0.0f, 1.0f);
    // B = b A + c A^2 (A is symmetric: A^2 = A^T A), then X <- a X + X B
    hipLaunchKernelGGL((qg_ns_gemm<true, 1>), dim3(nsb), dim3(kThreads), 0, s, b, b.off_a,
                       int64_t(0), b.off_a, b.off_b, kQb, kQc);
    hipLaunchKernelGGL((qg_ns_gemm<false, 1>), dim3(nsb), dim3(kThreads), 0, s, b, x, b.off_b,
                       x, xn, kQa, 1.0f);
    const int64_t t = x;
    x = xn;
    xn = t;
  }
  for (int it = 0; it < b.iters_cubic_bf16 + b.iters_cubic_split; ++it) {
    if (it < b.iters_cubic_bf16) {
      hipLaunchKernelGGL((qg_ns_gemm<true, 1>), dim3(nsb), dim3(kThreads), 0, s, b, x,
                         int64_t(0), b.off_a, b.off_a, 0.0f, 1.0f);
      hipLaunchKernelGGL((qg_ns_gemm<false, 1>), dim3(nsb), dim3(kThreads), 0, s, b, x,
                         b.off_a, x, xn, 1.5f, -0.5f);
    } else {
      hipLaunchKernelGGL((qg_ns_gemm<true, 2>), dim3(nsb), dim3(kThreads), 0, s, b, x,
                         int64_t(0), b.off_a, b.off_a, 0.0f, 1.0f);
      hipLaunchKernelGGL((qg_ns_gemm<false, 2>), dim3(nsb), dim3(kThreads), 0, s, b, x,
                         b.off_a, x, xn, 1.5f, -0.5f);
    }
    const int64_t t = x;
    x = xn;
    xn = t;
  }
  hipLaunchKernelGGL(qg_cossim_dot, dim3(eblocks), dim3(kThreads), 0, s, b, x, b.off_c);
  hipLaunchKernelGGL(qg_cossim_fold, dim3(b.count), dim3(kThreads), 0, s, b, (int64_t)0,
                     1.0f / (float)b.r, out);
  return hipGetLastError();
}

}  // namespace qg
