// Host-visible launch interface of the gfx950 kernels.
#pragma once

#include "qg_device.hpp"

namespace qg {

// A batch of projection pairs for the similarity test (same rank r, any row count m).
constexpr int kCosMaxPairs = 32;
// Output tile edge of the similarity kernels: small tiles, so that the short K loops of the
// r x r products run with several workgroups per CU.
constexpr int kCosTile = 64;
// Output tile edge of the cross product C = P~_new^T P~_old (K = the projections' rows) for
// rank 256 and above, where the long K loop pays for a larger tile and split-K fills the
// chip; smaller ranks use kCosTile.
constexpr int kCosCTile = 128;
constexpr int cos_ctile(int r) { return r >= 256 ? kCosCTile : kCosTile; }

struct CosPair {
  int format;          // projection storage format of both (kPInt4, kPInt8, kPBf16)
  const uint8_t* qa;   // P_new codes (or bf16 values)
  const float* sa;
  const uint8_t* qb;   // P_old codes (or bf16 values)
  const float* sb;
  int64_t m;
  int kslab;           // rows per split of C = P~_new^T P~_old
  int split;
  int gemm_base;       // first workgroup of this pair in the C launch
};

struct CosBatch {
  CosPair pair[kCosMaxPairs];
  char* ws;              // workspace base; pair p owns [p * pair_stride, (p+1) * pair_stride)
  int64_t pair_stride;
  int64_t off_part;      // split x r x r partial sums of C
  int64_t off_c, off_x, off_xn, off_a;        // r x r fp32 matrices
  int64_t off_xb0, off_xb1, off_ab, off_bb;   // r x r bf16 matrices
  int64_t off_blk;       // per-block partial sums
  int64_t off_norm;      // [0]: squared Frobenius norm of C, [1]: of X0^T X0
  int count, r, tiles, nblk;
  int ctiles;             // tiles per edge of the C product (edge cos_ctile(r))
  int iters_quintic;     // Newton-Schulz iterations lifting small singular values (bf16)
  int iters_cubic_bf16;  // then cubic iterations with bf16 operands (at least one)
  int iters_cubic_split; // and with hi/lo split operands
};

constexpr int kDeqCodes = 32;   // projection codes each dequant thread converts

// Tile edges of the MFMA kernels (back-projection: "big" for rank above 128).
constexpr int kProjTileM = 128;
constexpr int kProjTileN = 256;
constexpr int kBackTileM(bool big) { return big ? 128 : 128; }
constexpr int kBackTileN(bool big) { return big ? 256 : 128; }

hipError_t launch_project(const StepArgs& a, int grid, hipStream_t s);
hipError_t launch_dequant(const StepArgs& a, int grid, hipStream_t s);
hipError_t launch_adam(const StepArgs& a, int grid, hipStream_t s);
hipError_t launch_backproject(const StepArgs& a, int grid, bool big, hipStream_t s);
hipError_t launch_quantize_int4(const float* P, int64_t numel, uint8_t* Pq, float* Ps,
                                hipStream_t s);
hipError_t launch_quantize_int8(const float* P, int64_t numel, int8_t* Pq, float* Ps,
                                hipStream_t s);
// Calibration kernel (qg_probe.hip): `grid` workgroups of 4 waves, each wave 16 bf16 MFMA
// 32x32x16 per round for `iters` rounds on fragments read from `operands`.
hipError_t launch_mfma_probe(const uint16_t* operands, int64_t n_elems, float* out, int grid,
                             int iters, hipStream_t s);
hipError_t launch_cossim_batch(const CosBatch& b, float* out, hipStream_t s);

// ---- subspace refresh (randomized range finder of G's leading left singular vectors) ----
constexpr int kRfMaxK = 136;   // widest sketch (rank + oversampling) the k x k kernels hold
constexpr int kRfTileM = 128;  // output tile of the products with G
constexpr int kRfTileN = 64;

// part[s] (M x N fp32) = A (M x K, K slab s) * B (K x N), bf16 operands. A is K-contiguous
// (a_kmajor = 0: A[i][k] at A + i*lda + k, lda == K) or K-major (A[i][k] at A + k*lda + i);
// B is K-major (B[k][j] at B + k*ldb + j). lda and ldb are multiples of 8.
struct RfGemm {
  const uint16_t* A;
  const uint16_t* B;
  float* part;
  int64_t M, N, K, lda, ldb, kslab;
  int tiles_m, tiles_n, split, a_kmajor;
};

hipError_t launch_rf_gemm(const RfGemm& g, hipStream_t s);
hipError_t launch_rf_reduce(const float* part, int split, int64_t M, int N, int k, float* out,
                            hipStream_t s);
// Gram matrix of Y (M x k): partials over row chunks into part, their sum into out (k x k).
hipError_t launch_rf_gram(const float* Y, int64_t M, int k, int64_t rows_per_chunk,
                          int chunks, float* part, float* out, hipStream_t s);
hipError_t launch_rf_chol_inv(const float* W, int k, float shift_rel, float* Wt, hipStream_t s);
hipError_t launch_rf_smallmul(const float* Y, const float* Wm, int64_t M, int k, int N,
                              float* out, uint16_t* outb, float* amax_v, hipStream_t s);
hipError_t launch_rf_jacobi(const float* C, int k, int r, int max_sweeps, float tol,
                            float* evals, float* Vr, float* sigma, int* sweeps, hipStream_t s);
hipError_t launch_rf_signs(float* P, int64_t m, int r, const float* amax_v, float* sgn,
                           hipStream_t s);

// ---- products of a linear layer with an INT8-stored weight (dequantized in the stager) ----
constexpr int kLinTileM = 128;
constexpr int kLinTileN = 256;
enum { kLinFwd = 0, kLinBwdData = 1, kLinBwdWeight = 2 };
// forward:      act = X (T x n),  out = Y  (T x m)
// data grad:    act = dY (T x m), out = dX (T x n)
// weight grad:  act = dY (T x m), act2 = X (T x n), out = G (m x n)
struct LinArgs {
  const uint16_t* act;
  const uint16_t* act2;
  const int8_t* Wq;
  const float* Ws;
  uint16_t* out;
  int64_t T, m, n;
};
hipError_t launch_linear(const LinArgs& a, int which, hipStream_t s);

}  // namespace qg
