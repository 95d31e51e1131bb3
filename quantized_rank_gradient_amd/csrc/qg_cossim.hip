// Subspace similarity of the layer-adaptive refresh schedule (AIMech curated page on
// Q-GaLore, mechanism claim "layer-adaptive subspace cosine schedule", paper Section 3.1,
// Equation (5)): CosSim(P_new, P_old) = (1/r) * sum_i sigma_i(P_new^T P_old).
//
// For a batch of projection pairs (same rank r, any row counts):
//   1. C = P~_new^T P~_old (r x r) on bf16 MFMA, the INT4 (or INT8) dequant on the way into
//      LDS, split over the rows.
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
//      All but the last steps run with bf16 operands and keep X, A and B in bf16; the last
//      ones keep X in fp32 and use hi/lo split operands (about 16 significant bits) so that
//      X ends orthogonal to fp32-level accuracy.
//      trace(X^T C) is maximal at the exact polar factor, so what error the bf16 steps leave
//      in X enters the trace only to second order.
#include "qg_gemm.hpp"
#include "qg_kernels.hpp"

namespace qg {

using CosTile = Tile<kCosTile, kCosTile, 32, 2, 2, true, true>;     // C = P~n^T P~o, X^T X
using NsTileNN = Tile<kCosTile, kCosTile, 32, 2, 2, false, true>;   // X A
using CosTileC = Tile<kCosCTile, kCosCTile, 32, 2, 2, true, true>;  // C at rank >= 256
static_assert(CosTile::XM == NsTileNN::XM && CosTile::XN == NsTileNN::XN, "same wave tiling");

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
__device__ __forceinline__ uint16_t* pair_bf(const CosBatch& b, int p, int64_t off) {
  return reinterpret_cast<uint16_t*>(b.ws + (int64_t)p * b.pair_stride + off);
}

// ------------------------------------------------------------- 1: C = P~n^T P~o ---

// The projections' dequant (INT4 or INT8 codes times the group scale, rounded to bf16) or
// the bf16 values themselves, staged straight into LDS.
template <class T, class SA>
__device__ __forceinline__ void cos_c_product(SA& sa, SA& sb, int64_t k_begin, int64_t k_end,
                                              uint16_t* lds, f32x16 (&acc)[T::XM][T::XN]) {
  gemm_kloop<T, 1>(
      sa, sb, [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); },
      [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); },
      k_begin, k_end, lds, acc);
}

// T: CosTile (edge kCosTile) or CosTileC (edge kCosCTile), as cos_ctile(r) selects.
template <class T>
__global__ __launch_bounds__(kThreads) void qg_cossim_gemm(CosBatch b) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::STAGE];
  int local;
  // consecutive blocks (one pair's tiles) share an XCD and its L2
  const int p = pair_of_block(b, xcd_remap(blockIdx.x, gridDim.x), local);
  const CosPair& q = b.pair[p];
  const int per_split = b.ctiles * b.ctiles;
  const int s = local / per_split;
  const int rem = local - s * per_split;
  const int ti = rem / b.ctiles, tj = rem - ti * b.ctiles;
  const int i0 = ti * T::BM, j0 = tj * T::BN;
  const int64_t k_begin = (int64_t)s * q.kslab;
  const int64_t k_end = min<int64_t>(q.m, k_begin + q.kslab);
  f32x16 acc[T::XM][T::XN];
  if (q.format == kPInt8) {
    StageInt8K<T::BM, T::BK> sa(q.qa, q.sa, b.r, q.m, k_end, b.r, i0);
    StageInt8K<T::BM, T::BK> sb(q.qb, q.sb, b.r, q.m, k_end, b.r, j0);
    cos_c_product<T>(sa, sb, k_begin, k_end, lds, acc);
  } else if (q.format == kPBf16) {
    const uint16_t* pa = reinterpret_cast<const uint16_t*>(q.qa);
    const uint16_t* pb = reinterpret_cast<const uint16_t*>(q.qb);
    StageBf16K<T::BM, T::BK, true> sa(pa, b.r, q.m, k_end, b.r, i0);
    StageBf16K<T::BM, T::BK, true> sb(pb, b.r, q.m, k_end, b.r, j0);
    cos_c_product<T>(sa, sb, k_begin, k_end, lds, acc);
  } else {
    StageInt4K<T::BM, T::BK> sa(q.qa, q.sa, b.r, q.m, k_end, b.r, i0);
    StageInt4K<T::BM, T::BK> sb(q.qb, q.sb, b.r, q.m, k_end, b.r, j0);
    cos_c_product<T>(sa, sb, k_begin, k_end, lds, acc);
  }
  float* out = pair_mat(b, p, b.off_part) + (int64_t)s * b.r * b.r;
#pragma unroll
  for (int x = 0; x < T::XM; ++x)
#pragma unroll
    for (int y = 0; y < T::XN; ++y) {
      const int64_t j = j0 + acc_col<T>(y);
      if (j >= b.r) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + acc_row<T>(x, v);
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

// 2c: X0 = C / ||C||_F, stored in bf16 (the first iterations use bf16 operands).
__global__ __launch_bounds__(kThreads) void qg_cossim_init(CosBatch b) {
  const int p = blockIdx.x / b.nblk;
  const int blk = blockIdx.x - p * b.nblk;
  const int64_t n2 = (int64_t)b.r * b.r;
  const int64_t e0 = ((int64_t)blk * kThreads + threadIdx.x) * 4;
  if (e0 >= n2) return;
  const float sq = pair_mat(b, p, b.off_norm)[0];
  const float inv = sq > 0.0f ? 1.0f / sqrtf(sq) : 0.0f;
  const float4 c = gload(reinterpret_cast<const float4*>(pair_mat(b, p, b.off_c) + e0));
  gstore(reinterpret_cast<uint2*>(pair_bf(b, p, b.off_xb0) + e0),
         make_uint2(pack_bf16x2(c.x * inv, c.y * inv), pack_bf16x2(c.z * inv, c.w * inv)));
}

// ---------------------------------------------------- 3: Newton-Schulz products ---

// TA: Y = beta * (M^T M) + alpha * E      (M at off_m; E at off_e, skipped when alpha == 0)
// !TA: Y = alpha * E + beta * (M Bop)     (Bop at off_bop)
// IN_BF16: M, Bop and E are stored in bf16 (then PARTS == 1); otherwise in fp32, split into
// hi/lo bf16 parts on the way into LDS when PARTS == 2. OUT_BF16: Y is rounded to bf16.
template <bool TA, int PARTS, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void qg_ns_gemm(CosBatch b, int64_t off_m,
                                                      int64_t off_bop, int64_t off_e,
                                                      int64_t off_y, float alpha, float beta) {
  static_assert(!IN_BF16 || PARTS == 1, "bf16 operands have no low part");
  constexpr int STAGE = CosTile::STAGE > NsTileNN::STAGE ? CosTile::STAGE : NsTileNN::STAGE;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * PARTS * STAGE];
  // TA products are symmetric: only tiles with ti <= tj are computed, each written to both
  // of its mirror positions.
  const int per_pair = TA ? b.tiles * (b.tiles + 1) / 2 : b.tiles * b.tiles;
  // consecutive blocks (one pair's tiles) share an XCD and its L2
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int p = blk / per_pair;
  int rem = blk - p * per_pair;
  int ti, tj;
  if constexpr (TA) {
    ti = 0;
    while (rem >= b.tiles - ti) {
      rem -= b.tiles - ti;
      ++ti;
    }
    tj = ti + rem;
  } else {
    ti = rem / b.tiles;
    tj = rem - ti * b.tiles;
  }
  const int i0 = ti * CosTile::BM, j0 = tj * CosTile::BN;
  const int r = b.r;
  f32x16 acc[CosTile::XM][CosTile::XN];
  if constexpr (IN_BF16) {
    // short K loop over L2-resident operands: four stages in flight
    constexpr int D = 4;
    const uint16_t* M = pair_bf(b, p, off_m);
    if constexpr (TA) {
      StageBf16K<CosTile::BM, CosTile::BK, true, D> sa(M, r, r, r, r, i0);
      StageBf16K<CosTile::BM, CosTile::BK, true, D> sb(M, r, r, r, r, j0);
      gemm_kloop_ring<CosTile, D>(sa, sb, 0, r, lds, acc);
    } else {
      StageBf16C<NsTileNN::BM, NsTileNN::BK, D> sa(M, r, r, i0);
      StageBf16K<NsTileNN::BN, NsTileNN::BK, true, D> sb(pair_bf(b, p, off_bop), r, r, r, r, j0);
      gemm_kloop_ring<NsTileNN, D>(sa, sb, 0, r, lds, acc);
    }
  } else {
    const float* M = pair_mat(b, p, off_m);
    if constexpr (TA) {
      using T = CosTile;
      StageF32K<T::BM, T::BK, PARTS, T::STAGE> sa(M, r, r, r, i0);
      StageF32K<T::BN, T::BK, PARTS, T::STAGE> sb(M, r, r, r, j0);
      gemm_kloop<T, PARTS>(
          sa, sb, [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); },
          [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); }, 0, r,
          lds, acc);
    } else {
      using T = NsTileNN;
      StageF32C<T::BM, T::BK, PARTS, T::STAGE> sa(M, r, r, i0);
      StageF32K<T::BN, T::BK, PARTS, T::STAGE> sb(pair_mat(b, p, off_bop), r, r, r, j0);
      gemm_kloop<T, PARTS>(
          sa, sb, [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); },
          [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); }, 0, r,
          lds, acc);
    }
  }
#pragma unroll
  for (int x = 0; x < CosTile::XM; ++x)
#pragma unroll
    for (int y = 0; y < CosTile::XN; ++y) {
      const int64_t j = j0 + acc_col<CosTile>(y);
      if (j >= r) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + acc_row<CosTile>(x, v);
        if (i >= r) continue;
        float out = beta * acc[x][y][v];
        if (alpha != 0.0f) {
          const float e = IN_BF16 ? bf16_to_f32(gload(pair_bf(b, p, off_e) + i * r + j))
                                  : gload(pair_mat(b, p, off_e) + i * r + j);
          out += alpha * e;
        }
        if constexpr (OUT_BF16) {
          gstore(pair_bf(b, p, off_y) + i * r + j, to_bf16(out));
          if (TA && ti != tj) gstore(pair_bf(b, p, off_y) + j * r + i, to_bf16(out));
        } else {
          gstore(pair_mat(b, p, off_y) + i * r + j, out);
          if (TA && ti != tj) gstore(pair_mat(b, p, off_y) + j * r + i, out);
        }
      }
    }
}

// ------------------------------------------- 4: sum of X .* Y per pair, rescaling ---

// Per-block partial sums of the elementwise product of two r x r matrices of each pair
// (trace(X^T Y)); sum of squares when X == Y.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void qg_cossim_dot(CosBatch b, int64_t off_x,
                                                         int64_t off_y) {
  __shared__ float red[kThreads];
  const int p = blockIdx.x / b.nblk;
  const int blk = blockIdx.x - p * b.nblk;
  const int64_t n2 = (int64_t)b.r * b.r;
  const int64_t e0 = ((int64_t)blk * kThreads + threadIdx.x) * 4;
  float acc = 0.0f;
  if (e0 < n2) {
    float4 x, c;
    if constexpr (BF16) {
      const uint2 xb = gload(reinterpret_cast<const uint2*>(pair_bf(b, p, off_x) + e0));
      const uint2 cb = gload(reinterpret_cast<const uint2*>(pair_bf(b, p, off_y) + e0));
      x = make_float4(bf16_to_f32(xb.x & 0xFFFFu), bf16_to_f32(xb.x >> 16),
                      bf16_to_f32(xb.y & 0xFFFFu), bf16_to_f32(xb.y >> 16));
      c = make_float4(bf16_to_f32(cb.x & 0xFFFFu), bf16_to_f32(cb.x >> 16),
                      bf16_to_f32(cb.y & 0xFFFFu), bf16_to_f32(cb.y >> 16));
    } else {
      x = gload(reinterpret_cast<const float4*>(pair_mat(b, p, off_x) + e0));
      c = gload(reinterpret_cast<const float4*>(pair_mat(b, p, off_y) + e0));
    }
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

// X *= s and A *= s^2 with s = ||A||_F^(-1/2) (A = X^T X; both in bf16): afterwards the
// singular values of X are s_i / (sum_j s_j^4)^(1/4) <= 1.
__global__ __launch_bounds__(kThreads) void qg_ns_rescale(CosBatch b) {
  const int p = blockIdx.x / b.nblk;
  const int blk = blockIdx.x - p * b.nblk;
  const int64_t n2 = (int64_t)b.r * b.r;
  const int64_t e0 = ((int64_t)blk * kThreads + threadIdx.x) * 4;
  if (e0 >= n2) return;
  const float sq = pair_mat(b, p, b.off_norm)[1];   // ||A||_F^2
  const float s = sq > 0.0f ? 1.0f / sqrtf(sqrtf(sq)) : 0.0f;
  const float s2 = s * s;
  uint2* X = reinterpret_cast<uint2*>(pair_bf(b, p, b.off_xb0) + e0);
  uint2* A = reinterpret_cast<uint2*>(pair_bf(b, p, b.off_ab) + e0);
  const uint2 x = gload(X), a = gload(A);
  gstore(X, make_uint2(pack_bf16x2(bf16_to_f32(x.x & 0xFFFFu) * s, bf16_to_f32(x.x >> 16) * s),
                       pack_bf16x2(bf16_to_f32(x.y & 0xFFFFu) * s, bf16_to_f32(x.y >> 16) * s)));
  gstore(A,
         make_uint2(pack_bf16x2(bf16_to_f32(a.x & 0xFFFFu) * s2, bf16_to_f32(a.x >> 16) * s2),
                    pack_bf16x2(bf16_to_f32(a.y & 0xFFFFu) * s2, bf16_to_f32(a.y >> 16) * s2)));
}

// ------------------------------- 5: the whole chain in one workgroup (r <= 128) ---
// For ranks up to kNsSmallMax the r x r matrices fit in LDS and the chain above costs far
// more in launches than in products. One workgroup per pair then runs it from the block sums
// of ||C||^2 to the result, on LDS-resident matrices, with the same products (same operand
// ports, K order and hi/lo splitting), the same epilogue arithmetic and roundings, and the
// same block and fold reductions, so that its result equals the multi-launch chain's.

constexpr int kNsP = kNsSmallMax + 16;        // LDS row pitch (bf16): rows 8 banks apart
constexpr int kNsMat = kNsSmallMax * kNsP;    // elements of one LDS matrix
constexpr int kNsWM = 4, kNsWN = 4;           // waves along rows and columns
constexpr int kNsXM = kNsSmallMax / 32 / kNsWM;  // 32-row blocks per wave
constexpr int kNsThreads = 64 * kNsWM * kNsWN;
constexpr int kNsRed = 256;                   // block width of the reductions (as qg_cossim_dot)

__device__ __forceinline__ int ns_wm() { return (threadIdx.x >> 6) / kNsWN; }
__device__ __forceinline__ int ns_wn() { return (threadIdx.x >> 6) % kNsWN; }
// output row of accumulator entry v of 32-block x, and output column, for this lane
__device__ __forceinline__ int ns_row(int x, int v) {
  return ns_wm() * 32 * kNsXM + 32 * x + 8 * (v >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (v & 3);
}
__device__ __forceinline__ int ns_col() { return ns_wn() * 32 + (threadIdx.x & 31); }

// Symmetric products (M^T M) are formed as the multi-launch chain forms them: 64 x 64 tiles
// on and above the diagonal, each also written to its mirror position.
__device__ __forceinline__ int ns_ti() { return ns_wm() * 32 * kNsXM / 64; }
__device__ __forceinline__ int ns_tj() { return ns_wn() / 2; }
__device__ __forceinline__ bool ns_upper() { return ns_ti() <= ns_tj(); }
__device__ __forceinline__ bool ns_mirrors() { return ns_ti() < ns_tj(); }

// A-port fragment of a row-major LDS matrix read K-contiguous (8 K values of row c + lane%32).
__device__ __forceinline__ bf16x8 ns_frag_rows(const uint16_t* M, int c, int ks) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const bf16x8*>(M + (c + (lane & 31)) * kNsP + ks + 8 * (lane >> 5));
}

// acc = products over K < kext (a multiple of 32) for this wave's blocks: TA: M^T M
// (both ports read M K-major); otherwise M Bop. PARTS == 2: Ml / Bl hold the bf16 low parts,
// and each 16-K step adds hi*hi for all blocks, then hi*lo and lo*hi per block, in that
// order (the multi-launch chain's order).
template <bool TA, int PARTS>
__device__ __forceinline__ void ns_mul(const uint16_t* M, const uint16_t* Ml, const uint16_t* Bo,
                                       const uint16_t* Bl, int kext, f32x16 (&acc)[kNsXM]) {
  const int am = ns_wm() * 32 * kNsXM, bn = ns_wn() * 32;
#pragma unroll 2
  for (int ks = 0; ks < kNsSmallMax; ks += 16) {
    if (ks >= kext) break;
    bf16x8 a[kNsXM];
#pragma unroll
    for (int x = 0; x < kNsXM; ++x)
      a[x] = TA ? frag<true, kNsP>(M, am + 32 * x, ks) : ns_frag_rows(M, am + 32 * x, ks);
    const bf16x8 b = frag<true, kNsP>(TA ? M : Bo, bn, ks);
#pragma unroll
    for (int x = 0; x < kNsXM; ++x)
      acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], b, ks == 0 ? f32x16{} : acc[x], 0, 0, 0);
    if constexpr (PARTS == 2) {
      bf16x8 al[kNsXM];
#pragma unroll
      for (int x = 0; x < kNsXM; ++x)
        al[x] = TA ? frag<true, kNsP>(Ml, am + 32 * x, ks) : ns_frag_rows(Ml, am + 32 * x, ks);
      const bf16x8 bl = frag<true, kNsP>(TA ? Ml : Bl, bn, ks);
#pragma unroll
      for (int x = 0; x < kNsXM; ++x) {
        acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], bl, acc[x], 0, 0, 0);
        acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[x], b, acc[x], 0, 0, 0);
      }
    }
  }
}

// Y = beta * acc + alpha * E (E in bf16 from the LDS matrix E, skipped when alpha == 0),
// rounded to bf16 into the LDS matrix Y; Y may be E (each lane reads and writes only its own
// entries). Entries past r are left alone (they stay zero). SYM: a symmetric product's
// blocks (see ns_upper).
template <bool SYM>
__device__ __forceinline__ void ns_put_bf16(const f32x16 (&acc)[kNsXM], int r, float alpha,
                                            float beta, const uint16_t* E, uint16_t* Y) {
  if (SYM && !ns_upper()) return;
  const bool mirror = SYM && ns_mirrors();
  const int j = ns_col();
#pragma unroll
  for (int x = 0; x < kNsXM; ++x)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = ns_row(x, v);
      if (i >= r || j >= r) continue;
      float out = beta * acc[x][v];
      if (alpha != 0.0f) out += alpha * bf16_to_f32(E[i * kNsP + j]);
      Y[i * kNsP + j] = to_bf16(out);
      if (mirror) Y[j * kNsP + i] = to_bf16(out);
    }
}

// Sum over the block sums of 4-element dot products over the flat r x r order, as
// qg_cossim_dot and qg_cossim_fold form it: thread t of block k takes elements
// 4 (256 k + t) .. + 3, each block is reduced by the 256-way halving tree (all blocks at
// once here), and the block sums are folded in double (strided, then the same tree).
// V: LDS scratch of nblk * 256 floats; D: 256 doubles. Returns the fold on every thread.
template <class Dot4>
__device__ __forceinline__ double ns_blocked_dot(int n2, int nblk, Dot4 dot4, float* V, double* D) {
  const int t = threadIdx.x;
  for (int q = t; q < nblk * kNsRed; q += kNsThreads) {
    const int e0 = q * 4;
    V[q] = e0 < n2 ? dot4(e0) : 0.0f;
  }
  __syncthreads();
  for (int w = kNsRed / 2; w > 0; w >>= 1) {
    for (int q = t; q < nblk * w; q += kNsThreads) {
      const int k = q / w, u = q - k * w;
      V[k * kNsRed + u] += V[k * kNsRed + u + w];
    }
    __syncthreads();
  }
  if (t < kNsRed) {
    double acc = 0.0;
    for (int k = t; k < nblk; k += kNsRed) acc += V[k * kNsRed];
    D[t] = acc;
  }
  __syncthreads();
  for (int w = kNsRed / 2; w > 0; w >>= 1) {
    if (t < w) D[t] += D[t + w];
    __syncthreads();
  }
  const double res = D[0];
  __syncthreads();
  return res;
}

// grid = count (one workgroup per pair); runs after qg_cossim_gemm and qg_cossim_reduce.
__global__ __launch_bounds__(kNsThreads, 1) void qg_ns_small(CosBatch b, float* out) {
  __shared__ __attribute__((aligned(16))) uint16_t L[4 * kNsMat];
  __shared__ double D[kNsRed];
  constexpr float kQa = 3.4445f, kQb = -4.7750f, kQc = 2.0315f;
  const int p = blockIdx.x, t = threadIdx.x;
  const int r = b.r, n2 = r * r, nblk = b.nblk;
  const int kext = (r + 31) / 32 * 32;
  uint16_t* X = L;                 // X (bf16), then the high parts of the fp32 X
  uint16_t* XL = L + kNsMat;       // low parts of the fp32 X
  uint16_t* A = L + 2 * kNsMat;    // A = X^T X (bf16), then its high parts
  uint16_t* Bm = L + 3 * kNsMat;   // B = b A + c A^2, then the low parts of A
  f32x16 acc[kNsXM];

  // zero padding: entries past r read as zero in every product
  for (int q = t; q < 4 * kNsMat / 8; q += kNsThreads)
    reinterpret_cast<uint4*>(L)[q] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  // ||C||_F^2 from the reduce kernel's block sums (qg_cossim_fold's order), X0 = bf16(C / ||C||)
  {
    const float* blk = pair_mat(b, p, b.off_blk);
    if (t < kNsRed) {
      double a0 = 0.0;
      for (int k = t; k < nblk; k += kNsRed) a0 += blk[k];
      D[t] = a0;
    }
    __syncthreads();
    for (int w = kNsRed / 2; w > 0; w >>= 1) {
      if (t < w) D[t] += D[t + w];
      __syncthreads();
    }
    const float sq = (float)D[0];
    __syncthreads();
    const float inv = sq > 0.0f ? 1.0f / sqrtf(sq) : 0.0f;
    const float* C = pair_mat(b, p, b.off_c);
    for (int e0 = 4 * t; e0 < n2; e0 += 4 * kNsThreads) {
      const float4 c = gload(reinterpret_cast<const float4*>(C + e0));
      const int i = e0 / r, j = e0 - i * r;
      *reinterpret_cast<uint2*>(X + i * kNsP + j) =
          make_uint2(pack_bf16x2(c.x * inv, c.y * inv), pack_bf16x2(c.z * inv, c.w * inv));
    }
    __syncthreads();
  }

  // A = X0^T X0, then X *= s and A *= s^2 with s = ||A||_F^(-1/2)
  if (ns_upper()) ns_mul<true, 1>(X, nullptr, nullptr, nullptr, kext, acc);
  ns_put_bf16<true>(acc, r, 0.0f, 1.0f, nullptr, A);
  __syncthreads();
  {
    float* V = reinterpret_cast<float*>(Bm);
    const double sq = ns_blocked_dot(n2, nblk, [&](int e0) {
      const int i = e0 / r, j = e0 - i * r;
      const uint2 xb = *reinterpret_cast<const uint2*>(A + i * kNsP + j);
      const float x0 = bf16_to_f32(xb.x & 0xFFFFu), x1 = bf16_to_f32(xb.x >> 16);
      const float x2 = bf16_to_f32(xb.y & 0xFFFFu), x3 = bf16_to_f32(xb.y >> 16);
      return x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
    }, V, D);
    const float sqf = (float)sq;
    const float sc = sqf > 0.0f ? 1.0f / sqrtf(sqrtf(sqf)) : 0.0f;
    const float s2 = sc * sc;
    for (int e0 = 4 * t; e0 < n2; e0 += 4 * kNsThreads) {
      const int i = e0 / r, j = e0 - i * r;
      uint2* xp = reinterpret_cast<uint2*>(X + i * kNsP + j);
      uint2* ap = reinterpret_cast<uint2*>(A + i * kNsP + j);
      const uint2 x = *xp, a = *ap;
      *xp = make_uint2(pack_bf16x2(bf16_to_f32(x.x & 0xFFFFu) * sc, bf16_to_f32(x.x >> 16) * sc),
                       pack_bf16x2(bf16_to_f32(x.y & 0xFFFFu) * sc, bf16_to_f32(x.y >> 16) * sc));
      *ap = make_uint2(pack_bf16x2(bf16_to_f32(a.x & 0xFFFFu) * s2, bf16_to_f32(a.x >> 16) * s2),
                       pack_bf16x2(bf16_to_f32(a.y & 0xFFFFu) * s2, bf16_to_f32(a.y >> 16) * s2));
    }
    // the block-sum scratch in Bm must read as zero again before B is formed there
    for (int q = t; q < kNsMat / 8; q += kNsThreads)
      reinterpret_cast<uint4*>(Bm)[q] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }

  // quintic steps: B = c A^2 + b A, X <- a X + X B
  for (int it = 0; it < b.iters_quintic; ++it) {
    if (it > 0) {
      if (ns_upper()) ns_mul<true, 1>(X, nullptr, nullptr, nullptr, kext, acc);
      ns_put_bf16<true>(acc, r, 0.0f, 1.0f, nullptr, A);
      __syncthreads();
    }
    if (ns_upper()) ns_mul<true, 1>(A, nullptr, nullptr, nullptr, kext, acc);
    ns_put_bf16<true>(acc, r, kQb, kQc, A, Bm);
    __syncthreads();
    ns_mul<false, 1>(X, nullptr, Bm, nullptr, kext, acc);
    __syncthreads();                                  // every wave done reading X
    ns_put_bf16<false>(acc, r, kQa, 1.0f, X, X);
    __syncthreads();
  }
  // cubic steps with bf16 operands: X <- 1.5 X - 0.5 X A; the last one keeps X in fp32
  float* Xg = pair_mat(b, p, b.off_x);   // this lane's fp32 X entries, read back only by it
  for (int it = 0; it < b.iters_cubic_bf16; ++it) {
    if (ns_upper()) ns_mul<true, 1>(X, nullptr, nullptr, nullptr, kext, acc);
    ns_put_bf16<true>(acc, r, 0.0f, 1.0f, nullptr, A);
    __syncthreads();
    ns_mul<false, 1>(X, nullptr, A, nullptr, kext, acc);
    __syncthreads();
    if (it + 1 < b.iters_cubic_bf16) {
      ns_put_bf16<false>(acc, r, 1.5f, -0.5f, X, X);
    } else {
      const int j = ns_col();
#pragma unroll
      for (int x = 0; x < kNsXM; ++x)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = ns_row(x, v);
          if (i >= r || j >= r) continue;
          float o = -0.5f * acc[x][v];
          o += 1.5f * bf16_to_f32(X[i * kNsP + j]);
          gstore(Xg + i * r + j, o);
          const uint16_t h = to_bf16(o);
          X[i * kNsP + j] = h;
          XL[i * kNsP + j] = to_bf16(o - bf16_to_f32(h));
        }
    }
    __syncthreads();
  }
  // split steps: fp32 X and A as hi/lo bf16 pairs; the last X goes to LDS as flat fp32
  float* Xf = reinterpret_cast<float*>(A);   // r * r floats over the A and Bm areas
  for (int it = 0; it < b.iters_cubic_split; ++it) {
    if (ns_upper()) ns_mul<true, 2>(X, XL, nullptr, nullptr, kext, acc);
    __syncthreads();                                  // A and Bm are free
    if (ns_upper()) {
      const bool mirror = ns_mirrors();
      const int j = ns_col();
#pragma unroll
      for (int x = 0; x < kNsXM; ++x)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = ns_row(x, v);
          if (i >= r || j >= r) continue;
          const float o = 1.0f * acc[x][v];
          const uint16_t h = to_bf16(o), l = to_bf16(o - bf16_to_f32(h));
          A[i * kNsP + j] = h;
          Bm[i * kNsP + j] = l;
          if (mirror) {
            A[j * kNsP + i] = h;
            Bm[j * kNsP + i] = l;
          }
        }
    }
    __syncthreads();
    ns_mul<false, 2>(X, XL, A, Bm, kext, acc);
    __syncthreads();
    const bool last = it + 1 == b.iters_cubic_split;
    const int j = ns_col();
#pragma unroll
    for (int x = 0; x < kNsXM; ++x)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = ns_row(x, v);
        if (i >= r || j >= r) continue;
        float o = -0.5f * acc[x][v];
        o += 1.5f * gload(Xg + i * r + j);
        if (last) {
          Xf[i * r + j] = o;
        } else {
          gstore(Xg + i * r + j, o);
          const uint16_t h = to_bf16(o);
          X[i * kNsP + j] = h;
          XL[i * kNsP + j] = to_bf16(o - bf16_to_f32(h));
        }
      }
    __syncthreads();
  }
  // trace(X^T C) / r by the blocked dot and fold of qg_cossim_dot / qg_cossim_fold
  const float* C = pair_mat(b, p, b.off_c);
  const double tr = ns_blocked_dot(n2, nblk, [&](int e0) {
    const float4 c = gload(reinterpret_cast<const float4*>(C + e0));
    return Xf[e0] * c.x + Xf[e0 + 1] * c.y + Xf[e0 + 2] * c.z + Xf[e0 + 3] * c.w;
  }, reinterpret_cast<float*>(X), D);
  if (t == 0) out[p] = (float)(tr * (1.0f / (float)r));
}

// ------------------------------------------------------------------------ driver ---

hipError_t launch_cossim_batch(const CosBatch& b, float* out, hipStream_t s) {
  constexpr float kQa = 3.4445f, kQb = -4.7750f, kQc = 2.0315f;
  int gemm_blocks = 0;
  for (int p = 0; p < b.count; ++p) gemm_blocks += b.pair[p].split * b.ctiles * b.ctiles;
  if (cos_ctile(b.r) == kCosCTile)
    hipLaunchKernelGGL(qg_cossim_gemm<CosTileC>, dim3(gemm_blocks), dim3(kThreads), 0, s, b);
  else
    hipLaunchKernelGGL(qg_cossim_gemm<CosTile>, dim3(gemm_blocks), dim3(kThreads), 0, s, b);
  const int eblocks = b.count * b.nblk;
  hipLaunchKernelGGL(qg_cossim_reduce, dim3(eblocks), dim3(kThreads), 0, s, b);
  if (b.r <= kNsSmallMax) {
    hipLaunchKernelGGL(qg_ns_small, dim3(b.count), dim3(kNsThreads), 0, s, b, out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(qg_cossim_fold, dim3(b.count), dim3(kThreads), 0, s, b, b.off_norm, 0.0f,
                     (float*)nullptr);
  hipLaunchKernelGGL(qg_cossim_init, dim3(eblocks), dim3(kThreads), 0, s, b);
  const dim3 nsb(b.count * b.tiles * b.tiles), thr(kThreads);
  const dim3 nsy(b.count * b.tiles * (b.tiles + 1) / 2);   // symmetric products
  const int64_t z = 0;
  // bf16 phase: X in xb0 / xb1, A and B in bf16. A = X0^T X0, then the rescaling.
  hipLaunchKernelGGL((qg_ns_gemm<true, 1, true, true>), nsy, thr, 0, s, b, b.off_xb0, z,
                     b.off_ab, b.off_ab, 0.0f, 1.0f);
  hipLaunchKernelGGL(qg_cossim_dot<true>, dim3(eblocks), thr, 0, s, b, b.off_ab, b.off_ab);
  hipLaunchKernelGGL(qg_cossim_fold, dim3(b.count), thr, 0, s, b,
                     b.off_norm + (int64_t)sizeof(float), 0.0f, (float*)nullptr);
  hipLaunchKernelGGL(qg_ns_rescale, dim3(eblocks), thr, 0, s, b);
  int64_t x = b.off_xb0, xn = b.off_xb1;
  for (int it = 0; it < b.iters_quintic; ++it) {
    if (it > 0)
      hipLaunchKernelGGL((qg_ns_gemm<true, 1, true, true>), nsy, thr, 0, s, b, x, z, b.off_ab,
                         b.off_ab, 0.0f, 1.0f);
    // B = b A + c A^2 (A is symmetric: A^2 = A^T A), then X <- a X + X B
    hipLaunchKernelGGL((qg_ns_gemm<true, 1, true, true>), nsy, thr, 0, s, b, b.off_ab, z,
                       b.off_ab, b.off_bb, kQb, kQc);
    hipLaunchKernelGGL((qg_ns_gemm<false, 1, true, true>), nsb, thr, 0, s, b, x, b.off_bb, x,
                       xn, kQa, 1.0f);
    const int64_t t = x;
    x = xn;
    xn = t;
  }
  // cubic steps with bf16 operands; the last one writes X in fp32 for the split phase
  for (int it = 0; it < b.iters_cubic_bf16; ++it) {
    hipLaunchKernelGGL((qg_ns_gemm<true, 1, true, true>), nsy, thr, 0, s, b, x, z, b.off_ab,
                       b.off_ab, 0.0f, 1.0f);
    if (it + 1 < b.iters_cubic_bf16) {
      hipLaunchKernelGGL((qg_ns_gemm<false, 1, true, true>), nsb, thr, 0, s, b, x, b.off_ab, x,
                         xn, 1.5f, -0.5f);
      const int64_t t = x;
      x = xn;
      xn = t;
    } else {
      hipLaunchKernelGGL((qg_ns_gemm<false, 1, true, false>), nsb, thr, 0, s, b, x, b.off_ab,
                         x, b.off_x, 1.5f, -0.5f);
    }
  }
  // split phase in fp32
  x = b.off_x;
  xn = b.off_xn;
  for (int it = 0; it < b.iters_cubic_split; ++it) {
    hipLaunchKernelGGL((qg_ns_gemm<true, 2, false, false>), nsy, thr, 0, s, b, x, z, b.off_a,
                       b.off_a, 0.0f, 1.0f);
    hipLaunchKernelGGL((qg_ns_gemm<false, 2, false, false>), nsb, thr, 0, s, b, x, b.off_a, x,
                       xn, 1.5f, -0.5f);
    const int64_t t = x;
    x = xn;
    xn = t;
  }
  hipLaunchKernelGGL(qg_cossim_dot<false>, dim3(eblocks), thr, 0, s, b, x, b.off_c);
  hipLaunchKernelGGL(qg_cossim_fold, dim3(b.count), thr, 0, s, b, z, 1.0f / (float)b.r, out);
  return hipGetLastError();
}

}  // namespace qg
