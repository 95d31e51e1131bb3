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
// Ranks up to this run the Newton-Schulz chain in one workgroup per pair, on LDS-resident
// matrices (one launch instead of a launch per product).
constexpr int kNsSmallMax = 128;

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

// pmode: kPStaged, kPInline or kPMixed (the layers of the launch).
hipError_t launch_project(const StepArgs& a, int grid, int pmode, hipStream_t s);
hipError_t launch_dequant(const StepArgs& a, int grid, hipStream_t s);
hipError_t launch_adam(const StepArgs& a, int grid, hipStream_t s);
// fold: every layer of the launch has fold_alpha set.
hipError_t launch_backproject(const StepArgs& a, int grid, bool big, int pmode, bool fold,
                              hipStream_t s);
// A rank whose INT4 projection the MFMA kernels can dequantize in their stagers: each row's
// run of a projection tile (128 rank indices) and of a back-projection stage (32) lies inside
// one 256-element scale group.
constexpr bool inline_rank(int64_t r) { return r % 32 == 0 && (r % 128 == 0 || 256 % r == 0); }
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
// out[e] = sum over c < chunks of part[c * n + e], in order of c.
hipError_t launch_rf_sum(const float* part, int chunks, int64_t n, float* out, hipStream_t s);
hipError_t launch_rf_chol_inv(const float* W, int k, float shift_rel, float* Wt, hipStream_t s);
hipError_t launch_rf_smallmul(const float* Y, const float* Wm, int64_t M, int k, int N,
                              float* out, uint16_t* outb, float* amax_v, hipStream_t s);
hipError_t launch_rf_signs(float* P, int64_t m, int r, const float* amax_v, float* sgn,
                           hipStream_t s);

// ---- wide sketches (k above kRfMaxK): fp32 products on the matrix cores, block Jacobi ----
constexpr int kRfMaxKWide = 2048;
constexpr int kSgTile = 128;   // output tile of the fp32 products
enum { kSgPartial = 0, kSgSubtract = 1, kSgStore = 2 };
// out (M x N) op= A (M x K) B (K x N) in fp32. A is K-major (a_kmajor = 1: A[i][t] at
// A + t*lda + i) or K-contiguous (A + i*lda + t); B is K-major (B + t*ldb + j). kSgPartial
// writes the product over K slab s densely at out + s*M*N; kSgSubtract: out[i*ldo + j] -=
// product; kSgStore: out[i*ldo + j] = product. The contiguous extent of each operand (K of a
// K-contiguous A, M of a K-major A, N of B) and every leading dimension are multiples of 4,
// kslab a multiple of 16, and the pointers 16-byte aligned. tile: output tile edge, kSgTile
// or 64 (tiles_m, tiles_n counted in it).
struct SGemm {
  const float* A;
  const float* B;
  float* out;
  int64_t M, N, K, lda, ldb, ldo, kslab;
  int tiles_m, tiles_n, split, a_kmajor, mode, tile;
};
hipError_t launch_rf_sgemm(const SGemm& g, hipStream_t s);
// Qb (M x 2k bf16): hi parts of Qf (M x k fp32) in columns 0 .. k-1, lo parts in k .. 2k-1.
hipError_t launch_rf_split(const float* Qf, int64_t M, int k, uint16_t* Qb, hipStream_t s);
// Gp (m x n8 bf16) = G (m x n) padded with zero columns.
hipError_t launch_rf_pad(const uint16_t* G, int64_t m, int64_t n, int64_t n8, uint16_t* Gp,
                         hipStream_t s);
// Per 64-row tile and column of P (m x r): the signed entry of largest magnitude.
hipError_t launch_rf_colmax(const float* P, int64_t m, int r, float* amax_v, hipStream_t s);

// Indices per block of the block Jacobi solver (subproblems of twice that order): 16 or 32.
// Blocks of 32 halve the rounds of a sweep, whose fixed cost (two dependent launches) dominates
// the per-round time of either size at the sketch widths measured (136 to 1032).
constexpr int kRfJacobiBlockSwitch = 0;   // sketch width from which blocks of 32 are used
constexpr int rf_bj_block(int k) { return k >= kRfJacobiBlockSwitch ? 32 : 16; }
// Blocks of the padded problem: ceil(k / B) rounded up to an even count.
constexpr int rf_bj_blocks(int k, int B) { return (k + 2 * B - 1) / (2 * B) * 2; }
// Device buffers of the block Jacobi solver for K = B * rf_bj_blocks(k, B), B = rf_bj_block(k):
// C and V (fp64 K x K), J (fp64, K / 2B pieces of 2B x 2B, each the transpose of the round's
// rotation product of one pair of blocks), jrot (K / 2B), abs_tol (1), rot
// (max_sweeps), rank_of (k).
struct RfBj {
  double* C;
  double* V;
  double* J;
  int* jrot;
  float* abs_tol;
  int* rot;
  int* rank_of;
};
// Eigen-decomposition of the symmetric C (k x k, k <= kRfMaxKWide): the eigenvalues in
// descending order (ties by index) to evals (k), the eigenvectors of the r largest to the
// columns of Vr (k x r, fp32), the square roots of the r largest to sigma (when given), the
// number of sweeps run to sweeps.
hipError_t launch_rf_block_jacobi(const float* C, int k, int r, int max_sweeps, float tol,
                                  const RfBj& w, float* evals, float* Vr, float* sigma,
                                  int* sweeps, hipStream_t s);

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
// Shapes whose forward / data-gradient product stages the INT8 weight by LDS DMA: a row's
// 32 codes of a K stage (forward) or a column tile's 128 codes of a row (data gradient) lie
// in one 256-element scale group.
constexpr bool lin_fwd_dma(int64_t n) { return n % 32 == 0; }
// Forward shapes staged in 64-K stages (whole lines of the activation rows, halves of the
// weight rows).
constexpr bool lin_fwd_rows(int64_t n) { return n % 128 == 0; }
constexpr bool lin_bwd_data_dma(int64_t n) { return n % 128 == 0; }

}  // namespace qg
