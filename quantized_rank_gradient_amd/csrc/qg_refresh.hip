// Subspace refresh on the GPU: the new projection of a layer is the span of the r leading
// left singular vectors of its gradient G (AIMech curated page on Q-GaLore: the projections
// are rank-r singular-vector matrices recomputed from an SVD of the gradient at each
// refresh). It is computed here by a randomized range finder with power iterations (Halko,
// Martinsson and Tropp, "Finding structure with randomness", SIAM Review 2011, Algorithms
// 4.3/4.4 and 5.1):
//
//   Y = G Omega (m x k, k = r + oversample, Omega supplied by the caller), Q = orth(Y)
//   q times:  Z = orth(G^T Q),  Q = orth(G Z)
//   B^T = G^T Q (n x k);  C = B B^T (k x k);  C = V diag(lambda) V^T (block Jacobi)
//   P = Q V[:, leading r], each column's sign fixed so that its largest |entry| is positive,
//   then INT4 group quantization (qg_quantize_int4).
//
// orth() is CholeskyQR in fp32: the Gram matrix Y^T Y, its Cholesky factor L (with a small
// diagonal shift), then Q = Y L^-T; the final basis takes a second, unshifted pass
// (CholeskyQR2), the intermediate bases of the power iterations one. The
// products with G run on bf16 MFMA with fp32 accumulation: G is bf16 already and each fp32
// basis enters as two bf16 parts, hi = bf16(x) and lo = bf16(x - hi), side by side as 2k
// columns whose products are added back together (about 16 significant bits per basis
// entry, so that directions far below the leading singular value stay resolved). Up to
// k = kRfMaxK the orthonormalization's k x k work runs in fp32 in one workgroup per step and
// P = Q V in fp32 here; wider sketches, and the eigenproblem at every width, are in
// qg_refresh_wide.hip.
#include "qg_gemm.hpp"
#include "qg_kernels.hpp"

namespace qg {

// ================================================================ products with G ===
// part[s] (M x N fp32) = A (M x K, rows of K slab s) * B (K x N, K-major). A is either
// K-contiguous ([i][k]: G itself, or a basis Q) or K-major ([k][i]: G read transposed).
using RfTileC = Tile<128, 64, 32, 2, 2, false, true>;
using RfTileK = Tile<128, 64, 32, 2, 2, true, true>;
static_assert(RfTileC::BM == kRfTileM && RfTileC::BN == kRfTileN, "host and device tiles agree");

template <class T>
__device__ __forceinline__ void rf_gemm_tile(const RfGemm& g, int local, uint16_t* lds) {
  const int ti = local % g.tiles_m;
  const int rest = local / g.tiles_m;
  const int tj = rest % g.tiles_n;
  const int s = rest / g.tiles_n;
  const int i0 = ti * T::BM, j0 = tj * T::BN;
  const int64_t k_begin = (int64_t)s * g.kslab;
  const int64_t k_end = min<int64_t>(g.K, k_begin + g.kslab);
  f32x16 acc[T::XM][T::XN];
  StageBf16K<T::BN, T::BK, true> sb(g.B, g.ldb, g.K, k_end, g.N, j0);
  if constexpr (T::A_KMAJOR) {
    StageBf16K<T::BM, T::BK, true> sa(g.A, g.lda, g.K, k_end, g.M, i0);
    gemm_kloop<T, 1>(
        sa, sb, [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); },
        [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); }, k_begin,
        k_end, lds, acc);
  } else {
    // rows of A are K-contiguous with pitch lda == K; every K slab but the last is a whole
    // number of K stages, so a stage never reaches into the next slab
    StageBf16C<T::BM, T::BK> sa(g.A, g.lda, g.M, i0);
    gemm_kloop<T, 1>(
        sa, sb, [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); },
        [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); }, k_begin,
        k_end, lds, acc);
  }
  const uint32_t M = (uint32_t)g.M, N = (uint32_t)g.N;
  const rsrc_t ro = make_rsrc(g.part + (int64_t)s * g.M * g.N, M * N * 4);
#pragma unroll
  for (int x = 0; x < T::XM; ++x)
#pragma unroll
    for (int y = 0; y < T::XN; ++y) {
      const uint32_t j = j0 + acc_col<T>(y);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t i = i0 + acc_row<T>(x, v);
        bstoref(ro, (i < M && j < N) ? (i * N + j) * 4 : kOOB, acc[x][y][v]);
      }
    }
}

template <class T>
__global__ __launch_bounds__(kThreads, 2) void qg_rf_gemm(RfGemm g) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::STAGE];
  rf_gemm_tile<T>(g, xcd_remap(blockIdx.x, gridDim.x), lds);
}

// out (M x k) = sum over the `split` partial products (M x N each, in order); with N = 2k the
// columns j and j + k (products with the hi and lo parts of a basis) are added as well.
__global__ __launch_bounds__(kThreads) void qg_rf_reduce(const float* part, int split,
                                                         int64_t M, int N, int k, float* out) {
  const int64_t numel = M * k;
  const int64_t pstride = M * N;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < numel; e += stride) {
    const int64_t i = e / k;
    const int j = (int)(e % k);
    const float* p0 = part + i * N + j;
    float s = 0.0f;
    for (int p = 0; p < split; ++p) {
      s = add_rn(s, gload(p0 + p * pstride));
      if (N != k) s = add_rn(s, gload(p0 + p * pstride + k));
    }
    gstore(out + e, s);
  }
}

// ====================================================================== Gram matrix ===
// part[c] = Y[rows of chunk c]^T Y[rows of chunk c] (k x k fp32), Y row-major M x k. A
// 16 x 16 thread grid; thread (tx, ty) accumulates the entries (tx + 16a, ty + 16b).
constexpr int kRfKp = (kRfMaxK + 15) / 16 * 16;   // k padded to the thread grid
constexpr int kRfGramRows = 32;                   // rows staged in LDS at a time

__global__ __launch_bounds__(kThreads) void qg_rf_gram(const float* Y, int64_t M, int k,
                                                       int64_t rows_per_chunk, float* part) {
  __shared__ float tile[kRfGramRows][kRfKp];
  constexpr int NB = kRfKp / 16;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[NB][NB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = 0.0f;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_chunk;
  const int64_t r1 = min<int64_t>(M, r0 + rows_per_chunk);
  for (int64_t t0 = r0; t0 < r1; t0 += kRfGramRows) {
    for (int rr = threadIdx.x >> 4; rr < kRfGramRows; rr += kThreads / 16)
      for (int c = threadIdx.x & 15; c < kRfKp; c += 16)
        tile[rr][c] = (t0 + rr < r1 && c < k) ? gload(Y + (t0 + rr) * k + c) : 0.0f;
    __syncthreads();
    for (int rr = 0; rr < kRfGramRows; ++rr) {
      float va[NB], vb[NB];
#pragma unroll
      for (int a = 0; a < NB; ++a) va[a] = tile[rr][tx + 16 * a];
#pragma unroll
      for (int b = 0; b < NB; ++b) vb[b] = tile[rr][ty + 16 * b];
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = __builtin_fmaf(va[a], vb[b], acc[a][b]);
    }
    __syncthreads();
  }
  float* out = part + (int64_t)blockIdx.x * k * k;
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = tx + 16 * a, j = ty + 16 * b;
      if (i < k && j < k) gstore(out + i * k + j, acc[a][b]);
    }
}

// out[e] = sum over c of part[c * n + e] (in order of c), e < n.
__global__ __launch_bounds__(kThreads) void qg_rf_sum(const float* part, int chunks, int n,
                                                      float* out) {
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= n) return;
  float s = 0.0f;
  int c = 0;
  for (; c + 8 <= chunks; c += 8) {   // eight loads in flight, added in order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = gload(part + (int64_t)(c + u) * n + e);
#pragma unroll
    for (int u = 0; u < 8; ++u) s = add_rn(s, v[u]);
  }
  for (; c < chunks; ++c) s = add_rn(s, gload(part + (int64_t)c * n + e));
  gstore(out + e, s);
}

// ============================================================ Cholesky and inverse ===
// One workgroup: W (k x k Gram matrix) + shift_rel * trace(W) / k on the diagonal = L L^T,
// then Wt = L^-T (upper triangular, k x k row-major), so that an orthonormal basis is
// Q = Y Wt. Blocked in 16 x 16 blocks (the matrix padded with the identity to a multiple of
// 16, in LDS), right-looking (Golub and Van Loan, Section 4.2, block Cholesky):
//   for each block column jb: 16 lanes of one wave, a column each in registers, factor the
//   diagonal block (elimination without square roots inside the loop: step j subtracts
//   a_ij a_lj / a_jj from the trailing entries, a pivot below a tiny floor, a rank-deficient
//   basis, raised to it so that the direction is left out), scale it to L_jj and invert it
//   (D_jb = L_jj^-1, forward substitution by columns); all threads then form the panel
//   L_ib,jb = A_ib,jb D_jb^T and subtract L_ib,jb L_kb,jb^T from the trailing blocks.
// The inverse X = L^-1 follows by block rows: X_ib,jb = -D_ib sum_{jb <= kb < ib} L_ib,kb
// X_kb,jb, with X stored transposed in the upper triangle of A (the diagonal blocks D_jb^T
// written there by the factorization), where Wt = X^T reads it in place.
constexpr int kRfNb = (kRfMaxK + 15) / 16;   // 16 x 16 blocks per edge
constexpr int kRfCholP = kRfNb * 16 + 1;     // LDS row pitch (odd: column reads hit distinct banks)
// The sums T_jb of one block row of the inverse (one 16 x 17 block per column block).
constexpr int kRfYBuf = (kRfNb - 1) * 16 * 17;

// Value of v in lane `l` (uniform) of the wave.
__device__ __forceinline__ float lane_read(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__global__ __launch_bounds__(kThreads) void qg_rf_chol_inv(const float* W, int k,
                                                           float shift_rel, float* Wt) {
  constexpr int NB = kRfNb, PA = kRfCholP, KP = NB * 16;
  __shared__ float A[KP * PA];
  __shared__ float D[NB][16 * 17];          // D_jb = L_jj^-1, pitch 17
  __shared__ float P[KP * 17];              // panel of the current block column
  __shared__ float Ybuf[kRfYBuf];           // block-row sums of the inverse
  __shared__ float red[kThreads];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // block products: 16 blocks at a time, 16 threads each with a 4 x 4 patch (rows pr ..
  // pr + 3, columns pc .. pc + 3)
  const int blk = t >> 4, pr = ((t >> 2) & 3) * 4, pc = (t & 3) * 4;
  const int nb = (k + 15) / 16;
  const int kp = nb * 16;
  float tr_part = 0.0f;
  for (int e = t; e < kp * kp; e += kThreads) {
    const int i = e / kp, l = e % kp;
    const float v = (i < k && l < k) ? gload(W + i * k + l) : (i == l ? 1.0f : 0.0f);
    A[i * PA + l] = v;
    if (i == l && i < k) tr_part += v;
  }
  red[t] = tr_part;
  __syncthreads();
  if (t == 0) {
    float tr = 0.0f;
    for (int q = 0; q < kThreads; ++q) tr += red[q];
    red[0] = shift_rel * tr / (float)k;
  }
  __syncthreads();
  const float shift = red[0];
  const float floor_piv = fmaxf(shift, 1e-30f);
  for (int i = t; i < k; i += kThreads) A[i * PA + i] += shift;
  __syncthreads();

  for (int jb = 0; jb < nb; ++jb) {
    const int b0 = jb * 16;
    if (wave == 0 && lane < 16) {
      // the diagonal block in registers, lane c holding its column c (both triangles: the
      // trailing updates keep the block symmetric); pivots and columns reach the other
      // lanes by lane reads
      const int c = lane;
      float a[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) a[x] = A[(b0 + x) * PA + b0 + c];
      float dc = 1.0f;   // this lane's (floored) pivot
      // unscaled elimination: step j subtracts a_xj a_jc / d_j from the trailing entries
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float d = lane_read(a[j], j);
        d = d > floor_piv ? d : floor_piv;
        if (c == j) dc = d;
        const float inv = 1.0f / d;
        const float ajc = a[j];
#pragma unroll
        for (int x = j + 1; x < 16; ++x) {
          const float axj = lane_read(a[x], j) * inv;
          if (c > j) a[x] = __builtin_fmaf(-axj, ajc, a[x]);
        }
      }
      // column c of L_jj: the unscaled column over sqrt(pivot), sqrt(pivot) on the diagonal
      const float dl = sqrtf(dc);
#pragma unroll
      for (int x = 0; x < 16; ++x) a[x] = x < c ? 0.0f : (x == c ? dl : a[x] / dl);
      // D_jb = L_jj^-1, column c: forward substitution with the rows of L_jj read from
      // their lanes; also stored transposed in the diagonal block of A (row c of D_jb^T),
      // where the inverse below reads X^T
      float xv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = i == c ? 1.0f : 0.0f;
#pragma unroll
        for (int q = 0; q < i; ++q) acc = __builtin_fmaf(-lane_read(a[i], q), xv[q], acc);
        xv[i] = i < c ? 0.0f : acc / lane_read(a[i], i);
        D[jb][i * 17 + c] = xv[i];
        A[(b0 + c) * PA + b0 + i] = xv[i];
      }
    }
    __syncthreads();
    // panel: P[ib rows][c] = sum_s A[ib row][b0 + s] D_jb[c][s]  (D_jb lower: s <= c); each
    // block by 16 threads, a 4 x 4 patch each
    for (int ib = jb + 1 + blk; ib < nb; ib += 16) {
      float acc[4][4] = {};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = A[(ib * 16 + pr + i) * PA + b0 + q];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = D[jb][(pc + j) * 17 + q];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) P[(ib * 16 + pr + i) * 17 + pc + j] = acc[i][j];
    }
    __syncthreads();
    // the panel into A; trailing blocks (ib, kb), jb < kb <= ib: A -= L_ib,jb L_kb,jb^T
    for (int e = t; e < (nb - jb - 1) * 256; e += kThreads) {
      const int row = (jb + 1) * 16 + e / 16;
      A[row * PA + b0 + (e & 15)] = P[row * 17 + (e & 15)];
    }
    {
      const int nt = nb - jb - 1;   // trailing block rows
      for (int bi = blk; bi < nt * (nt + 1) / 2; bi += 16) {
        int ib = 0, rest = bi;   // bi -> (ib, kb), kb <= ib, row-major over the triangle
        while (rest > ib) {
          rest -= ib + 1;
          ++ib;
        }
        const int row0 = (jb + 1 + ib) * 16 + pr, col0 = (jb + 1 + rest) * 16 + pc;
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = A[(row0 + i) * PA + col0 + j];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          float a[4], b[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = P[(row0 + i) * 17 + q];
#pragma unroll
          for (int j = 0; j < 4; ++j) b[j] = P[(col0 + j) * 17 + q];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(-a[i], b[j], acc[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) A[(row0 + i) * PA + col0 + j] = acc[i][j];
      }
    }
    __syncthreads();
  }

  // X = L^-1 by block rows; X_ib,jb (ib > jb) stored transposed at A[jb block][ib block]
  for (int ib = 1; ib < nb; ++ib) {
    for (int jb = blk; jb < ib; jb += 16) {
      // T_jb = sum_{jb <= kb < ib} L_ib,kb X_kb,jb  (X_jb,jb = D_jb)
      float acc[4][4] = {};
      for (int kb = jb; kb < ib; ++kb) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          float av[4], bv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) av[i] = A[(ib * 16 + pr + i) * PA + kb * 16 + q];
#pragma unroll
          for (int j = 0; j < 4; ++j) bv[j] = A[(jb * 16 + pc + j) * PA + kb * 16 + q];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Ybuf[jb * 16 * 17 + (pr + i) * 17 + pc + j] = acc[i][j];
    }
    __syncthreads();
    for (int jb = blk; jb < ib; jb += 16) {
      // X_ib,jb = -D_ib T_jb  (D_ib lower), written transposed
      float acc[4][4] = {};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        float av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = D[ib][(pr + i) * 17 + q];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = Ybuf[jb * 16 * 17 + q * 17 + pc + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(-av[i], bv[j], acc[i][j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) A[(jb * 16 + pc + j) * PA + ib * 16 + pr + i] = acc[i][j];
    }
    __syncthreads();
  }
  // Wt = X^T: Wt[l][c] = X[c][l] = A[l][c] for c >= l, zero below
  for (int e = t; e < k * k; e += kThreads) {
    const int l = e / k, c = e % k;
    gstore(Wt + e, c >= l ? A[l * PA + c] : 0.0f);
  }
}

// ============================================================ small fp32 products ===
// out (M x N) = Y (M x k) Wm (k x N), fp32, K = k short. A 64 x 64 output tile per
// workgroup; thread (tx, ty) of a 16 x 16 grid computes rows tx + 16a, columns ty + 16b
// (a, b < 4). Optional outputs: outb (M x 2N bf16): the hi parts bf16(x) in columns
// 0 .. N-1 and the lo parts bf16(x - hi) in N .. 2N-1; amax_v (per 64-row tile and column):
// the entry of largest magnitude of the tile's column (signed; the first such row on ties).
__global__ __launch_bounds__(kThreads) void qg_rf_smallmul(const float* Y, const float* Wm,
                                                           int64_t M, int k, int N, float* out,
                                                           uint16_t* outb, float* amax_v) {
  __shared__ float qs[64][kRfMaxK + 1];
  __shared__ float ws[kRfMaxK][64];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int j0 = blockIdx.y * 64;
  for (int rr = ty; rr < 64; rr += 16)
    for (int c = tx; c < k; c += 16)
      qs[rr][c] = i0 + rr < M ? gload(Y + (i0 + rr) * k + c) : 0.0f;
  for (int l = ty; l < k; l += 16)
    for (int c = tx; c < 64; c += 16) ws[l][c] = j0 + c < N ? gload(Wm + l * N + j0 + c) : 0.0f;
  __syncthreads();
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  for (int l = 0; l < k; ++l) {
    float qa[4], wb[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) qa[a] = qs[tx + 16 * a][l];
#pragma unroll
    for (int b = 0; b < 4; ++b) wb[b] = ws[l][ty + 16 * b];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(qa[a], wb[b], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t i = i0 + tx + 16 * a;
      const int j = j0 + ty + 16 * b;
      if (i < M && j < N) {
        const float v = acc[a][b];
        gstore(out + i * N + j, v);
        if (outb) {
          const uint16_t hi = to_bf16(v);
          gstore(outb + i * 2 * N + j, hi);
          gstore(outb + i * 2 * N + N + j, to_bf16(v - bf16_to_f32(hi)));
        }
      }
    }
  if (!amax_v) return;
  // per-column scan of the tile: the operand tiles are no longer needed, so qs holds the
  // values (transposed: qs[column][row])
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) qs[ty + 16 * b][tx + 16 * a] = acc[a][b];
  __syncthreads();
  if (threadIdx.x < 64 && j0 + (int)threadIdx.x < N) {
    const int c = threadIdx.x;
    const int rows = (int)min<int64_t>(64, M - i0);
    float bv = qs[c][0];
    for (int rr = 1; rr < rows; ++rr)
      if (fabsf(qs[c][rr]) > fabsf(bv)) bv = qs[c][rr];
    gstore(amax_v + (int64_t)blockIdx.x * N + j0 + c, bv);
  }
}

// Column signs of P from the per-tile maxima (tiles in row order: the first tile holding
// the column's largest |entry| wins ties, so the first such row decides), then P's columns
// with a negative deciding entry are negated.
__global__ __launch_bounds__(kThreads) void qg_rf_sign(const float* amax_v, int tiles, int r,
                                                       float* sgn) {
  for (int c = threadIdx.x; c < r; c += kThreads) {
    float bv = gload(amax_v + c);
    for (int t = 1; t < tiles; ++t) {
      const float v = gload(amax_v + (int64_t)t * r + c);
      if (fabsf(v) > fabsf(bv)) bv = v;
    }
    gstore(sgn + c, bv < 0.0f ? -1.0f : 1.0f);
  }
}

__global__ __launch_bounds__(kThreads) void qg_rf_flip(float* P, int64_t numel, int r,
                                                       const float* sgn) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < numel; e += stride) {
    const float g = gload(sgn + (int)(e % r));
    if (g < 0.0f) gstore(P + e, -gload(P + e));
  }
}

// ======================================================================= launchers ===
hipError_t launch_rf_gemm(const RfGemm& g, hipStream_t s) {
  const int grid = g.tiles_m * g.tiles_n * g.split;
  if (g.a_kmajor)
    hipLaunchKernelGGL(qg_rf_gemm<RfTileK>, dim3(grid), dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL(qg_rf_gemm<RfTileC>, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_rf_reduce(const float* part, int split, int64_t M, int N, int k, float* out,
                            hipStream_t s) {
  const int64_t want = (M * k + kThreads - 1) / kThreads;
  const int64_t blocks = want < 4096 ? want : 4096;
  hipLaunchKernelGGL(qg_rf_reduce, dim3((unsigned)blocks), dim3(kThreads), 0, s, part, split, M,
                     N, k, out);
  return hipGetLastError();
}

hipError_t launch_rf_gram(const float* Y, int64_t M, int k, int64_t rows_per_chunk,
                          int chunks, float* part, float* out, hipStream_t s) {
  hipLaunchKernelGGL(qg_rf_gram, dim3(chunks), dim3(kThreads), 0, s, Y, M, k, rows_per_chunk,
                     part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = k * k;
  hipLaunchKernelGGL(qg_rf_sum, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s, part,
                     chunks, n, out);
  return hipGetLastError();
}

hipError_t launch_rf_sum(const float* part, int chunks, int64_t n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(qg_rf_sum, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     s, part, chunks, (int)n, out);
  return hipGetLastError();
}

hipError_t launch_rf_chol_inv(const float* W, int k, float shift_rel, float* Wt, hipStream_t s) {
  hipLaunchKernelGGL(qg_rf_chol_inv, dim3(1), dim3(kThreads), 0, s, W, k, shift_rel, Wt);
  return hipGetLastError();
}

hipError_t launch_rf_smallmul(const float* Y, const float* Wm, int64_t M, int k, int N,
                              float* out, uint16_t* outb, float* amax_v, hipStream_t s) {
  const dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64));
  hipLaunchKernelGGL(qg_rf_smallmul, grid, dim3(kThreads), 0, s, Y, Wm, M, k, N, out, outb,
                     amax_v);
  return hipGetLastError();
}

hipError_t launch_rf_signs(float* P, int64_t m, int r, const float* amax_v, float* sgn,
                           hipStream_t s) {
  const int tiles = (int)((m + 63) / 64);
  hipLaunchKernelGGL(qg_rf_sign, dim3(1), dim3(kThreads), 0, s, amax_v, tiles, r, sgn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t want = (m * r + kThreads - 1) / kThreads;
  const int64_t blocks = want < 4096 ? want : 4096;
  hipLaunchKernelGGL(qg_rf_flip, dim3((unsigned)blocks), dim3(kThreads), 0, s, P, m * r, r, sgn);
  return hipGetLastError();
}

}  // namespace qg
