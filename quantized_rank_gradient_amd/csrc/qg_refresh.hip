// Subspace refresh on the GPU: the new projection of a layer is the span of the r leading
// left singular vectors of its gradient G (AIMech curated page on Q-GaLore: the projections
// are rank-r singular-vector matrices recomputed from an SVD of the gradient at each
// refresh). It is computed here by a randomized range finder with power iterations (Halko,
// Martinsson and Tropp, "Finding structure with randomness", SIAM Review 2011, Algorithms
// 4.3/4.4 and 5.1):
//
//   Y = G Omega (m x k, k = r + oversample, Omega supplied by the caller), Q = orth(Y)
//   q times:  Z = orth(G^T Q),  Q = orth(G Z)
//   B^T = G^T Q (n x k);  C = B B^T (k x k);  C = V diag(lambda) V^T (Jacobi)
//   P = Q V[:, leading r], each column's sign fixed so that its largest |entry| is positive,
//   then INT4 group quantization (qg_quantize_int4).
//
// orth() is CholeskyQR in fp32: the Gram matrix Y^T Y, its Cholesky factor L (with a small
// diagonal shift), then Q = Y L^-T; the final basis takes a second, unshifted pass
// (CholeskyQR2), the intermediate bases of the power iterations one. The
// products with G run on bf16 MFMA with fp32 accumulation: G is bf16 already and each fp32
// basis enters as two bf16 parts, hi = bf16(x) and lo = bf16(x - hi), side by side as 2k
// columns whose products are added back together (about 16 significant bits per basis
// entry, so that directions far below the leading singular value stay resolved). The k x k
// work runs in fp32 in one workgroup, and P = Q V in fp32. Sizes: k <= kRfMaxK.
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
  for (int c = 0; c < chunks; ++c) s = add_rn(s, gload(part + (int64_t)c * n + e));
  gstore(out + e, s);
}

// ============================================================ Cholesky and inverse ===
// One workgroup: W (k x k Gram matrix) + shift_rel * trace(W) / k on the diagonal = L L^T,
// then Wt = L^-T (upper triangular, k x k row-major), so that an orthonormal basis is
// Q = Y Wt. The matrix lives in registers: thread (ty, tx) of a 16 x 16 grid holds the
// entries (ty + 16a, tx + 16b). Elimination step j (right-looking, no square roots inside
// the loop): the holders of column j publish it through LDS, then every thread subtracts
// a_ij a_lj / a_jj from its trailing entries. A pivot below a tiny floor (a rank-deficient
// basis) is raised to it, which leaves that direction out. The inverse X = L^-1 is formed
// the same way from the identity: step j divides row j by l_jj and subtracts l_ij times it
// from the rows below.
constexpr int kRfNb = (kRfMaxK + 15) / 16;   // register rows / columns per thread

__global__ __launch_bounds__(kThreads) void qg_rf_chol_inv(const float* W, int k,
                                                           float shift_rel, float* Wt) {
  constexpr int NB = kRfNb;
  __shared__ float colv[kRfMaxK];
  __shared__ float rowv[kRfMaxK];
  __shared__ float piv[kRfMaxK];
  __shared__ float red[kThreads];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float R[NB][NB];
  float tr_part = 0.0f;
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = ty + 16 * a, l = tx + 16 * b;
      R[a][b] = (i < k && l < k) ? gload(W + i * k + l) : 0.0f;
      if (i == l && i < k) tr_part += R[a][b];
    }
  red[threadIdx.x] = tr_part;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tr = 0.0f;
    for (int t = 0; t < kThreads; ++t) tr += red[t];
    red[0] = shift_rel * tr / (float)k;
  }
  __syncthreads();
  const float shift = red[0];
  const float floor_piv = fmaxf(shift, 1e-30f);
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (ty + 16 * a == tx + 16 * b) R[a][b] += shift;
  // ---- Cholesky (unscaled): after step j, column j holds l_ij * l_jj. Steps run as
  // j = 16 jb + jj with the register block jb a compile-time index.
  static_for<NB>([&](auto jbc) {
    constexpr int jb = decltype(jbc)::value;
    for (int jj = 0; jj < 16; ++jj) {
      const int j = 16 * jb + jj;
      if (j >= k) break;   // uniform across the workgroup
      if (tx == jj) {
#pragma unroll
        for (int a = 0; a < NB; ++a) {
          const int i = ty + 16 * a;
          if (i >= j && i < k) colv[i] = R[a][jb];
        }
      }
      __syncthreads();
      float d2 = colv[j];
      d2 = d2 > floor_piv ? d2 : floor_piv;
      if (threadIdx.x == 0) piv[j] = d2;
      const float inv = 1.0f / d2;
      float cl[NB];
#pragma unroll
      for (int b = jb; b < NB; ++b) {
        const int l = tx + 16 * b;
        cl[b] = (l > j && l < k) ? colv[l] : 0.0f;
      }
#pragma unroll
      for (int a = jb; a < NB; ++a) {
        const int i = ty + 16 * a;
        const float aij = (i > j && i < k) ? colv[i] * inv : 0.0f;
#pragma unroll
        for (int b = jb; b <= a; ++b)
          if (tx + 16 * b <= i) R[a][b] = __builtin_fmaf(-aij, cl[b], R[a][b]);
      }
      __syncthreads();
    }
  });
  // L = (unscaled column j) / sqrt(piv_j); held in R (lower triangle), then X = L^-1 with
  // the identity as starting point in B
  float B[NB][NB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = ty + 16 * a, l = tx + 16 * b;
      float v = 0.0f;
      if (l <= i && i < k) {
        const float dl = sqrtf(piv[l]);
        v = i == l ? dl : R[a][b] / dl;
      }
      R[a][b] = v;
      B[a][b] = (i == l && i < k) ? 1.0f : 0.0f;
    }
  // ---- forward elimination on [L | I]: step j scales row j of B by 1 / l_jj and subtracts
  // l_ij times it from the rows i > j (row j of X is zero right of the diagonal)
  static_for<NB>([&](auto jbc) {
    constexpr int jb = decltype(jbc)::value;
    for (int jj = 0; jj < 16; ++jj) {
      const int j = 16 * jb + jj;
      if (j >= k) break;
      if (tx == jj) {   // column j of L
#pragma unroll
        for (int a = jb; a < NB; ++a) {
          const int i = ty + 16 * a;
          if (i >= j && i < k) colv[i] = R[a][jb];
        }
      }
      __syncthreads();
      if (ty == jj) {   // row j of B, scaled: row j of X
        const float rl = 1.0f / colv[j];
#pragma unroll
        for (int b = 0; b <= jb; ++b) {
          const int c = tx + 16 * b;
          const float v = B[jb][b] * rl;
          B[jb][b] = v;
          if (c <= j) rowv[c] = v;
        }
      }
      __syncthreads();
      float xr[NB];
#pragma unroll
      for (int b = 0; b <= jb; ++b) {
        const int c = tx + 16 * b;
        xr[b] = c <= j ? rowv[c] : 0.0f;
      }
#pragma unroll
      for (int a = jb; a < NB; ++a) {
        const int i = ty + 16 * a;
        const float lij = (i > j && i < k) ? colv[i] : 0.0f;
#pragma unroll
        for (int b = 0; b <= jb; ++b) B[a][b] = __builtin_fmaf(-lij, xr[b], B[a][b]);
      }
      __syncthreads();
    }
  });
  // Wt = X^T: Wt[l][c] = X[c][l]
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = ty + 16 * a, l = tx + 16 * b;   // X[i][l]
      if (i < k && l < k) gstore(Wt + l * k + i, l <= i ? B[a][b] : 0.0f);
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

// =================================================================== Jacobi eigen ===
// One workgroup: C (k x k symmetric, k even) diagonalized by cyclic Jacobi rotations
// (Golub and Van Loan, Matrix Computations, Section 8.5: the 2 x 2 symmetric Schur
// decomposition and the parallel ordering). In each of the k - 1 rounds of a sweep the k/2
// disjoint index pairs of a round-robin tournament are rotated together: C <- J^T C J and
// V <- V J, with J the product of the round's plane rotations. C' = J^T C J is formed 2 x 2
// block by 2 x 2 block (rows of one pair, columns of another), each block from its own old
// entries, so a round needs one pass; C stays symmetric, so only its upper triangle is kept
// and only blocks on or above the block diagonal are computed. A pair is rotated while
// |c_pq| exceeds both tol * sqrt(|c_pp c_qq|) and 1e-7 * trace(C) (the level of fp32
// rounding noise in the entries); a sweep without rotations ends the iteration. The
// eigenvalues are ranked in descending order (ties by index); the eigenvectors of the r
// largest go to the columns of Vr (k x r), the eigenvalues to evals (k, descending) and,
// when sigma is given, the square roots of the r largest to sigma.
constexpr int kRfJacobiThreads = 1024;
constexpr int kRfJacobiPitch = kRfMaxK + 1;

__global__ __launch_bounds__(kRfJacobiThreads) void qg_rf_jacobi(
    const float* Cm, int k, int r, int max_sweeps, float tol, float* evals, float* Vr,
    float* sigma, int* sweeps_out) {
  constexpr int PT = kRfJacobiPitch;
  constexpr int NW = kRfJacobiThreads / 64;
  __shared__ float A[kRfMaxK * PT];
  __shared__ float V[kRfMaxK * PT];
  __shared__ float cs_c[kRfMaxK / 2], cs_s[kRfMaxK / 2];
  __shared__ int pp[kRfMaxK / 2], pq[kRfMaxK / 2], rot[kRfMaxK / 2];
  __shared__ int rotated;
  __shared__ int rank_of[kRfMaxK];
  __shared__ float abs_tol_sh;
  // the 2 x 2 blocks (w1, w2), w1 <= w2, of a round as one list (w1 in the high byte)
  constexpr int kMaxBlocks = (kRfMaxK / 2) * (kRfMaxK / 2 + 1) / 2;
  __shared__ uint16_t blk[kMaxBlocks];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = wave; i < k; i += NW)
    for (int j = lane; j < k; j += 64) {
      A[i * PT + j] = gload(Cm + i * k + j);
      V[i * PT + j] = i == j ? 1.0f : 0.0f;
    }
  const int half = k / 2;
  const int nblocks = half * (half + 1) / 2;
  if ((int)threadIdx.x < half) {
    const int w1 = threadIdx.x;
    const int first = w1 * half - w1 * (w1 - 1) / 2;   // blocks of rows before w1
    for (int w2 = w1; w2 < half; ++w2) blk[first + w2 - w1] = (uint16_t)((w1 << 8) | w2);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float tr = 0.0f;
    for (int i = 0; i < k; ++i) tr += fabsf(A[i * PT + i]);
    abs_tol_sh = 1e-7f * tr;
  }
  __syncthreads();
  const float abs_tol = abs_tol_sh;
  int sweeps = 0;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    if (threadIdx.x == 0) rotated = 0;
    __syncthreads();
    for (int round = 0; round < k - 1; ++round) {
      // round-robin pairing: position 0 holds index 0, positions 1 .. k-1 the others
      // rotated by `round`; position w meets position k - 1 - w
      if (threadIdx.x < half) {
        const int w = threadIdx.x;
        const int a = w == 0 ? 0 : 1 + (w - 1 + round) % (k - 1);
        const int b = 1 + (k - 2 - w + round) % (k - 1);
        const int p = min(a, b), qq = max(a, b);
        const float app = A[p * PT + p], aqq = A[qq * PT + qq], apq = A[p * PT + qq];
        float c = 1.0f, s = 0.0f;
        const bool go = fabsf(apq) > tol * sqrtf(fabsf(app * aqq)) && fabsf(apq) > abs_tol;
        if (go) {
          // the rotation's own rounding only needs c^2 + s^2 = 1 to fp32 accuracy
          const float tau = (aqq - app) * __builtin_amdgcn_rcpf(2.0f * apq);
          const float t = (tau >= 0.0f ? 1.0f : -1.0f) *
                          __builtin_amdgcn_rcpf(fabsf(tau) + sqrtf(1.0f + tau * tau));
          c = __builtin_amdgcn_rsqf(1.0f + t * t);
          s = t * c;
          rotated = 1;
        }
        pp[w] = p;
        pq[w] = qq;
        cs_c[w] = c;
        cs_s[w] = s;
        rot[w] = go ? 1 : 0;
      }
      __syncthreads();
      // blocks (w1, w2), w1 <= w2: rows p1, q1 rotated by pair w1, columns p2, q2 by w2.
      // Only the upper triangle of C is stored (entry (i, j) at (min, max)); every stored
      // entry belongs to exactly one block with w1 <= w2. Blocks of two unrotated pairs and
      // V columns of an unrotated pair do not change. Each thread takes every 1024th block
      // of the list and every 1024th (pair, row) update of V, and reads all of its entries
      // before it writes any, so the LDS latencies overlap.
      constexpr int BPT = (kMaxBlocks + kRfJacobiThreads - 1) / kRfJacobiThreads;
      constexpr int VPT = (kRfMaxK / 2 * kRfMaxK + kRfJacobiThreads - 1) / kRfJacobiThreads;
      {
        int o[BPT][4], wb[BPT];   // entry offsets; block code (w1 << 8 | w2), -1 when idle
        float x[BPT][4];
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
          const int b = threadIdx.x + u * kRfJacobiThreads;
          wb[u] = -1;
          if (b < nblocks) {
            const int w1 = blk[b] >> 8, w2 = blk[b] & 0xFF;
            if (rot[w1] | rot[w2]) {
              wb[u] = blk[b];
              const int p1 = pp[w1], q1 = pq[w1], p2 = pp[w2], q2 = pq[w2];
              o[u][0] = min(p1, p2) * PT + max(p1, p2);
              o[u][1] = min(p1, q2) * PT + max(p1, q2);
              o[u][2] = min(q1, p2) * PT + max(q1, p2);
              o[u][3] = min(q1, q2) * PT + max(q1, q2);
#pragma unroll
              for (int e = 0; e < 4; ++e) x[u][e] = A[o[u][e]];
            }
          }
        }
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
          if (wb[u] < 0) continue;
          const int w1 = wb[u] >> 8, w2 = wb[u] & 0xFF;
          const float c1 = cs_c[w1], s1 = cs_s[w1], c2 = cs_c[w2], s2 = cs_s[w2];
          const float a = x[u][0], bb = x[u][1], c = x[u][2], d = x[u][3];
          const float ra = c1 * a - s1 * c, rb = c1 * bb - s1 * d;   // J1^T rows
          const float rc = s1 * a + c1 * c, rd = s1 * bb + c1 * d;
          A[o[u][0]] = c2 * ra - s2 * rb;   // * J2 columns
          A[o[u][1]] = s2 * ra + c2 * rb;
          if (w1 != w2) A[o[u][2]] = c2 * rc - s2 * rd;   // on the diagonal o2 == o1
          A[o[u][3]] = s2 * rc + c2 * rd;
        }
        // V: the (pair, row) updates idx = threadIdx.x + 1024 u, in two batches of reads
        // then writes; (pair, row) = (idx / k, idx % k) advanced incrementally
        int w = threadIdx.x / k, i = threadIdx.x - w * k;
        const int dq = kRfJacobiThreads / k, dr = kRfJacobiThreads - dq * k;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          constexpr int NB = (VPT + 1) / 2;
          int vo[NB];   // row offset << 8 | pair, -1 when idle
          float vx[NB], vy[NB];
#pragma unroll
          for (int u = 0; u < NB; ++u) {
            vo[u] = -1;
            if (w < half && rot[w]) {
              vo[u] = ((i * PT) << 8) | w;
              vx[u] = V[i * PT + pp[w]];
              vy[u] = V[i * PT + pq[w]];
            }
            w += dq;
            i += dr;
            if (i >= k) {
              i -= k;
              ++w;
            }
          }
#pragma unroll
          for (int u = 0; u < NB; ++u) {
            if (vo[u] < 0) continue;
            const int wu = vo[u] & 0xFF, row = vo[u] >> 8;
            const float c = cs_c[wu], sn = cs_s[wu];
            V[row + pp[wu]] = c * vx[u] - sn * vy[u];
            V[row + pq[wu]] = sn * vx[u] + c * vy[u];
          }
        }
      }
      __syncthreads();
    }
    ++sweeps;
    if (!rotated) break;
    __syncthreads();
  }
  for (int i = threadIdx.x; i < k; i += kRfJacobiThreads) {
    const float li = A[i * PT + i];
    int rk = 0;
    for (int j = 0; j < k; ++j) {
      const float lj = A[j * PT + j];
      rk += (lj > li || (lj == li && j < i)) ? 1 : 0;
    }
    rank_of[i] = rk;
    gstore(evals + rk, li);
    if (sigma && rk < r) gstore(sigma + rk, sqrtf(fmaxf(li, 0.0f)));
  }
  __syncthreads();
  for (int i = wave; i < k; i += NW)
    for (int col = lane; col < k; col += 64) {   // V[i][col]: entry i of eigenvector col
      const int rk = rank_of[col];
      if (rk < r) gstore(Vr + i * r + rk, V[i * PT + col]);
    }
  if (threadIdx.x == 0 && sweeps_out) gstore(sweeps_out, sweeps);
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

hipError_t launch_rf_jacobi(const float* C, int k, int r, int max_sweeps, float tol,
                            float* evals, float* Vr, float* sigma, int* sweeps, hipStream_t s) {
  hipLaunchKernelGGL(qg_rf_jacobi, dim3(1), dim3(kRfJacobiThreads), 0, s, C, k, r, max_sweeps,
                     tol, evals, Vr, sigma, sweeps);
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
