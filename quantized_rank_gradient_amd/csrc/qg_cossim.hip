// Subspace similarity of the layer-adaptive refresh schedule (AIMech curated page on
// Q-GaLore, mechanism claim "layer-adaptive subspace cosine schedule", paper Section 3.1,
// Equation (5)): CosSim(P_new, P_old) = (1/r) * sum_i sigma_i(P_new^T P_old).
//
// For a batch of projection pairs (same rank r, any row counts):
//   1. C = P~_new^T P~_old (r x r) on bf16 MFMA, INT4 dequant in LDS, split over the rows.
//   2. The nuclear norm of C as trace(X^T C), where X is the orthogonal polar factor of C,
//      obtained by the Newton-Schulz iteration X <- 1.5 X - 0.5 X (X^T X) from X0 = C/||C||_F
//      (singular values in [0, 1], where the iteration converges to 1 for every nonzero one).
//      The first iterations only have to lift small singular values towards 1 and run with
//      bf16 operands; the last ones run with hi/lo split operands (about 16 significant bits)
//      so that X ends orthogonal to fp32-level accuracy. trace(X^T C) is maximal at the exact
//      polar factor, so the error that the bf16 phase leaves in X enters the trace only to
//      second order.
#include "qg_gemm.hpp"
#include "qg_kernels.hpp"

namespace qg {

// --------------------------------------------------------------- fp32 -> LDS stagers ---

// fp32 source stored [k][c] (row pitch ld, ld % 8 == 0), tile columns [c0, c0+128), written
// to LDS [c][k] as bf16 (and, when PARTS == 2, the bf16 remainder x - bf16(x) into the low
// copy). Thread t stages rows k+2p, k+2p+1 (p = t / 16), columns c0 + 8*(t % 16) .. +7.
template <int PARTS>
struct StageF32T {
  const float* src;
  int64_t ld, k_end, c_end;
  int c, kp;
  float f[2][8];

  __device__ StageF32T(const float* s, int64_t ld_, int64_t k_end_, int64_t c_end_, int c0)
      : src(s), ld(ld_), k_end(k_end_), c_end(c_end_) {
    const int t = threadIdx.x;
    kp = t >> 4;
    c = c0 + 8 * (t & 15);
  }

  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t k = k0 + 2 * kp + rr;
      if (k < k_end && c < c_end) {
        const float4 x = gload(reinterpret_cast<const float4*>(src + k * ld + c));
        const float4 y = gload(reinterpret_cast<const float4*>(src + k * ld + c + 4));
        f[rr][0] = x.x; f[rr][1] = x.y; f[rr][2] = x.z; f[rr][3] = x.w;
        f[rr][4] = y.x; f[rr][5] = y.y; f[rr][6] = y.z; f[rr][7] = y.w;
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) f[rr][u] = 0.0f;
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* hi, uint16_t* lo, int c0) const {
    uint32_t* dh = reinterpret_cast<uint32_t*>(hi);
    uint32_t* dl = reinterpret_cast<uint32_t*>(lo);
    const int cl = c - c0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const uint32_t h = pack_bf16x2(f[0][cc], f[1][cc]);
      dh[(cl + cc) * (LDK / 2) + kp] = h;
      if constexpr (PARTS == 2) {
        const float r0 = f[0][cc] - bf16_to_f32(h & 0xFFFFu);
        const float r1 = f[1][cc] - bf16_to_f32(h >> 16);
        dl[(cl + cc) * (LDK / 2) + kp] = pack_bf16x2(r0, r1);
      }
    }
  }
};

// fp32 source stored [c][k] (row pitch ld, K contiguous, ld % 8 == 0), tile rows
// [c0, c0+128), written to LDS [c][k] as bf16 (+ remainder). Thread t stages two runs: row
// (t / 4) + 64*h, columns k0 + 8*(t % 4) .. +7.
template <int PARTS>
struct StageF32N {
  const float* src;
  int64_t ld, c_end;
  int c0;
  float f[2][8];

  __device__ StageF32N(const float* s, int64_t ld_, int64_t c_end_, int c0_)
      : src(s), ld(ld_), c_end(c_end_), c0(c0_) {}

  __device__ __forceinline__ void load(int64_t k0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t row = c0 + (t >> 2) + 64 * h;
      const int64_t k = k0 + 8 * (t & 3);
      if (row < c_end && k < ld) {
        const float4 x = gload(reinterpret_cast<const float4*>(src + row * ld + k));
        const float4 y = gload(reinterpret_cast<const float4*>(src + row * ld + k + 4));
        f[h][0] = x.x; f[h][1] = x.y; f[h][2] = x.z; f[h][3] = x.w;
        f[h][4] = y.x; f[h][5] = y.y; f[h][6] = y.z; f[h][7] = y.w;
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) f[h][u] = 0.0f;
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* hi, uint16_t* lo) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rl = (t >> 2) + 64 * h;
      uint32_t w[4], wl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w[u] = pack_bf16x2(f[h][2 * u], f[h][2 * u + 1]);
        if constexpr (PARTS == 2)
          wl[u] = pack_bf16x2(f[h][2 * u] - bf16_to_f32(w[u] & 0xFFFFu),
                              f[h][2 * u + 1] - bf16_to_f32(w[u] >> 16));
      }
      *reinterpret_cast<uint4*>(hi + rl * LDK + 8 * (t & 3)) = make_uint4(w[0], w[1], w[2], w[3]);
      if constexpr (PARTS == 2)
        *reinterpret_cast<uint4*>(lo + rl * LDK + 8 * (t & 3)) =
            make_uint4(wl[0], wl[1], wl[2], wl[3]);
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
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE_ELEMS];
  int local;
  const int p = pair_of_block(b, blockIdx.x, local);
  const CosPair& q = b.pair[p];
  const int per_split = b.tiles * b.tiles;
  const int s = local / per_split;
  const int rem = local - s * per_split;
  const int ti = rem / b.tiles, tj = rem - ti * b.tiles;
  const int i0 = ti * TM, j0 = tj * TN;
  const int64_t k_begin = (int64_t)s * q.kslab;
  const int64_t k_end = min<int64_t>(q.m, k_begin + q.kslab);
  StageInt4T sa(q.qa, q.sa, b.r, k_end, b.r, i0);
  StageInt4T sb(q.qb, q.sb, b.r, k_end, b.r, j0);
  f32x16 acc[2][2];
  gemm_kloop<1>(sa, sb, [i0](StageInt4T& st, uint16_t* st0) { st.store(st0, i0); },
                [j0](StageInt4T& st, uint16_t* st0) { st.store(st0 + TM * LDK, j0); },
                k_begin, k_end, lds, acc);
  float* out = pair_mat(b, p, b.off_part) + (int64_t)s * b.r * b.r;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int64_t j = j0 + acc_col(y);
      if (j >= b.r) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + acc_row(x, v);
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

// TA: Y = X^T X  (Y at off_y, X at off_x).   !TA: Y = 1.5 X - 0.5 X A  (A at off_a).
template <bool TA, int PARTS>
__global__ __launch_bounds__(kThreads) void qg_ns_gemm(CosBatch b, int64_t off_x, int64_t off_a,
                                                      int64_t off_y) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * PARTS * STAGE_ELEMS];
  const int per_pair = b.tiles * b.tiles;
  const int p = blockIdx.x / per_pair;
  const int rem = blockIdx.x - p * per_pair;
  const int ti = rem / b.tiles, tj = rem - ti * b.tiles;
  const int i0 = ti * TM, j0 = tj * TN;
  const int r = b.r;
  const float* X = pair_mat(b, p, off_x);
  const float* A = pair_mat(b, p, off_a);
  float* Y = pair_mat(b, p, off_y);
  f32x16 acc[2][2];
  if constexpr (TA) {
    StageF32T<PARTS> sa(X, r, r, r, i0);
    StageF32T<PARTS> sb(X, r, r, r, j0);
    gemm_kloop<PARTS>(
        sa, sb,
        [i0](StageF32T<PARTS>& st, uint16_t* s0) { st.store(s0, s0 + STAGE_ELEMS, i0); },
        [j0](StageF32T<PARTS>& st, uint16_t* s0) {
          st.store(s0 + TM * LDK, s0 + STAGE_ELEMS + TM * LDK, j0);
        },
        0, r, lds, acc);
  } else {
    StageF32N<PARTS> sa(X, r, r, i0);
    StageF32T<PARTS> sb(A, r, r, r, j0);
    gemm_kloop<PARTS>(
        sa, sb, [](StageF32N<PARTS>& st, uint16_t* s0) { st.store(s0, s0 + STAGE_ELEMS); },
        [j0](StageF32T<PARTS>& st, uint16_t* s0) {
          st.store(s0 + TM * LDK, s0 + STAGE_ELEMS + TM * LDK, j0);
        },
        0, r, lds, acc);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int64_t j = j0 + acc_col(y);
      if (j >= r) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + acc_row(x, v);
        if (i >= r) continue;
        float out = acc[x][y][v];
        if constexpr (!TA) out = 1.5f * gload(X + i * r + j) - 0.5f * out;
        gstore(Y + i * r + j, out);
      }
    }
}

// ------------------------------------------------------- 4: trace(X^T C) per pair ---

__global__ __launch_bounds__(kThreads) void qg_cossim_trace(CosBatch b, int64_t off_x) {
  __shared__ float red[kThreads];
  const int p = blockIdx.x / b.nblk;
  const int blk = blockIdx.x - p * b.nblk;
  const int64_t n2 = (int64_t)b.r * b.r;
  const int64_t e0 = ((int64_t)blk * kThreads + threadIdx.x) * 4;
  float acc = 0.0f;
  if (e0 < n2) {
    const float4 x = gload(reinterpret_cast<const float4*>(pair_mat(b, p, off_x) + e0));
    const float4 c = gload(reinterpret_cast<const float4*>(pair_mat(b, p, b.off_c) + e0));
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

// ------------------------------------------------------------------------ driver ---

hipError_t launch_cossim_batch(const CosBatch& b, float* out, hipStream_t s) {
  int gemm_blocks = 0;
  for (int p = 0; p < b.count; ++p) gemm_blocks += b.pair[p].split * b.tiles * b.tiles;
  hipLaunchKernelGGL(qg_cossim_gemm, dim3(gemm_blocks), dim3(kThreads), 0, s, b);
  const int eblocks = b.count * b.nblk;
  hipLaunchKernelGGL(qg_cossim_reduce, dim3(eblocks), dim3(kThreads), 0, s, b);
  hipLaunchKernelGGL(qg_cossim_fold, dim3(b.count), dim3(kThreads), 0, s, b, b.off_norm, 0.0f,
                     (float*)nullptr);
  hipLaunchKernelGGL(qg_cossim_init, dim3(eblocks), dim3(kThreads), 0, s, b);
  const int nsb = b.count * b.tiles * b.tiles;
  int64_t x = b.off_x, xn = b.off_xn;
  for (int it = 0; it < b.iters_bf16 + b.iters_split; ++it) {
    if (it < b.iters_bf16) {
      hipLaunchKernelGGL((qg_ns_gemm<true, 1>), dim3(nsb), dim3(kThreads), 0, s, b, x, x, b.off_a);
      hipLaunchKernelGGL((qg_ns_gemm<false, 1>), dim3(nsb), dim3(kThreads), 0, s, b, x, b.off_a, xn);
    } else {
      hipLaunchKernelGGL((qg_ns_gemm<true, 2>), dim3(nsb), dim3(kThreads), 0, s, b, x, x, b.off_a);
      hipLaunchKernelGGL((qg_ns_gemm<false, 2>), dim3(nsb), dim3(kThreads), 0, s, b, x, b.off_a, xn);
    }
    const int64_t t = x;
    x = xn;
    xn = t;
  }
  hipLaunchKernelGGL(qg_cossim_trace, dim3(eblocks), dim3(kThreads), 0, s, b, x);
  hipLaunchKernelGGL(qg_cossim_fold, dim3(b.count), dim3(kThreads), 0, s, b, (int64_t)0,
                     1.0f / (float)b.r, out);
  return hipGetLastError();
}

}  // namespace qg
