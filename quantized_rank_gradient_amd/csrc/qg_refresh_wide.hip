// Subspace refresh for wide sketches (k = r + oversample above what one workgroup holds):
// the k x k work of the range finder spread over the whole chip.
//
//  * fp32 products (qg_rf_sgemm) on the matrix cores: v_mfma_f32_32x32x2_f32 multiplies fp32
//    operands exactly and accumulates in fp32. They form the Gram matrices, the projections
//    of block Gram-Schmidt and P = Q V.
//  * orth() of a wide basis is block classical Gram-Schmidt with reorthogonalization (BCGS2:
//    each block of columns has its projection on the finished blocks removed twice, which
//    leaves it orthogonal to them to working accuracy as long as it is not numerically inside
//    their span), then the block is orthonormalized by the one-workgroup CholeskyQR kernels.
//  * The eigenproblem C = V diag(lambda) V^T is solved by parallel block Jacobi (Golub and Van
//    Loan, Matrix Computations, Section 8.5 on the parallel ordering and block Jacobi): the
//    indices are cut into blocks of 32 and padded to an even number of blocks; in each round
//    of a round-robin tournament on the blocks, every pair of blocks forms a 64 x 64
//    subproblem that one workgroup treats with one cyclic sweep of 2 x 2 rotations
//    (qg_rf_bj_solve), and the product J of the round's rotations is applied to all of C and
//    V at once (qg_rf_bj_apply: C <- J^T C J and V <- V J, 64 x 64 pieces on the matrix cores).
//    A sweep is nb - 1 rounds; the kernels of later sweeps return at once after a sweep in
//    which no subproblem rotated, so the whole solve is issued without reading anything back.
#include "qg_gemm.hpp"
#include "qg_kernels.hpp"

namespace qg {

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ==================================================================== fp32 products ===
// A BM x BM output tile per workgroup of four waves (2 x 2, each BM/2 x BM/2: blocks of
// 32 x 32), BM = 128, or 64 for products too narrow to fill the chip with the larger tile.
// K advances in stages of 16, both operands staged in LDS K-major ([k][i], pitch BM + 32:
// the two half-waves of a fragment read land in opposite halves of the banks); the next
// stage's global loads are in flight while the current stage's products run. Every output
// accumulates its K terms in the same order at either tile size.
constexpr int kSgBK = 16;
template <int BM>
struct SgCfg {
  static constexpr int PITCH = BM + 32;
  static constexpr int STAGE = 2 * kSgBK * PITCH;   // floats per stage (A then B)
  static constexpr int V = BM * kSgBK / 4 / kThreads;   // float4 per thread and operand
  static constexpr int X = BM / 64;                  // 32 x 32 blocks per wave and edge
};
static_assert(kSgTile == 128, "host and device tiles agree");

__device__ __forceinline__ float4 ld4(const float* p, bool ok) {
  return ok ? gload(reinterpret_cast<const float4*>(p)) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// One stage of a K-major operand (rows k of length `cols`, contiguous): 16 rows x BM
// columns.
template <int BM>
struct SgKmaj {
  static constexpr int CPR = BM / 4;   // float4 per row
  const float* base;
  int64_t ld, cols;
  int c0;
  float4 v[SgCfg<BM>::V];
  __device__ void load(int64_t k0, int64_t k_end) {
#pragma unroll
    for (int u = 0; u < SgCfg<BM>::V; ++u) {
      const int q = threadIdx.x + kThreads * u;
      const int64_t kr = k0 + q / CPR;
      const int64_t c = c0 + 4 * (q % CPR);
      v[u] = ld4(base + kr * ld + c, kr < k_end && c < cols);
    }
  }
  __device__ void store(float* lds) const {
#pragma unroll
    for (int u = 0; u < SgCfg<BM>::V; ++u) {
      const int q = threadIdx.x + kThreads * u;
      *reinterpret_cast<float4*>(lds + (q / CPR) * SgCfg<BM>::PITCH + 4 * (q % CPR)) = v[u];
    }
  }
};

// One stage of a K-contiguous operand (row i holds its K values contiguously): BM rows x 16
// K values, transposed into the K-major LDS layout.
template <int BM>
struct SgKcon {
  const float* base;
  int64_t ld, rows;
  int r0;
  float4 v[SgCfg<BM>::V];
  __device__ void load(int64_t k0, int64_t k_end) {
#pragma unroll
    for (int u = 0; u < SgCfg<BM>::V; ++u) {
      const int q = threadIdx.x + kThreads * u;
      const int64_t row = r0 + (q >> 2);
      const int64_t kc = k0 + 4 * (q & 3);
      v[u] = ld4(base + row * ld + kc, row < rows && kc < k_end);
    }
  }
  __device__ void store(float* lds) const {
    constexpr int P = SgCfg<BM>::PITCH;
#pragma unroll
    for (int u = 0; u < SgCfg<BM>::V; ++u) {
      const int q = threadIdx.x + kThreads * u;
      const int row = q >> 2, kc = 4 * (q & 3);
      lds[(kc + 0) * P + row] = v[u].x;
      lds[(kc + 1) * P + row] = v[u].y;
      lds[(kc + 2) * P + row] = v[u].z;
      lds[(kc + 3) * P + row] = v[u].w;
    }
  }
};

template <int BM, class SA>
__device__ __forceinline__ void sgemm_tile(const SGemm& g, SA& sa, int i0, int j0, int s,
                                           float* lds) {
  using C = SgCfg<BM>;
  constexpr int XB = C::X, H = BM / 2;
  const int64_t k_begin = (int64_t)s * g.kslab;
  const int64_t k_end = min<int64_t>(g.K, k_begin + g.kslab);
  SgKmaj<BM> sb{g.B, g.ldb, g.N, j0};
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int am = (wave >> 1) * H, bn = (wave & 1) * H;
  const int kh = lane >> 5, li = lane & 31;
  f32x16 acc[XB][XB];
#pragma unroll
  for (int x = 0; x < XB; ++x)
#pragma unroll
    for (int y = 0; y < XB; ++y) acc[x][y] = f32x16{};
  if (k_begin < k_end) {
    sa.load(k_begin, k_end);
    sb.load(k_begin, k_end);
    sa.store(lds);
    sb.store(lds + kSgBK * C::PITCH);
    __syncthreads();
    int it = 0;
    for (int64_t k0 = k_begin; k0 < k_end; k0 += kSgBK, ++it) {
      const float* As = lds + (it & 1) * C::STAGE;
      const float* Bs = As + kSgBK * C::PITCH;
      const bool more = k0 + kSgBK < k_end;
      if (more) {
        sa.load(k0 + kSgBK, k_end);
        sb.load(k0 + kSgBK, k_end);
      }
#pragma unroll
      for (int kp = 0; kp < kSgBK / 2; ++kp) {
        const int kr = (2 * kp + kh) * C::PITCH;
        float a[XB], b[XB];
#pragma unroll
        for (int x = 0; x < XB; ++x) a[x] = As[kr + am + 32 * x + li];
#pragma unroll
        for (int y = 0; y < XB; ++y) b[y] = Bs[kr + bn + 32 * y + li];
#pragma unroll
        for (int x = 0; x < XB; ++x)
#pragma unroll
          for (int y = 0; y < XB; ++y) acc[x][y] = mfma_f32(a[x], b[y], acc[x][y]);
      }
      if (more) {
        float* nxt = lds + ((it + 1) & 1) * C::STAGE;
        sa.store(nxt);
        sb.store(nxt + kSgBK * C::PITCH);
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int x = 0; x < XB; ++x)
#pragma unroll
    for (int y = 0; y < XB; ++y) {
      const int64_t j = j0 + bn + 32 * y + li;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + am + 32 * x + 8 * (v >> 2) + 4 * kh + (v & 3);
        if (i >= g.M || j >= g.N) continue;
        const float val = acc[x][y][v];
        if (g.mode == kSgPartial) {
          gstore(g.out + (int64_t)s * g.M * g.N + i * g.N + j, val);
        } else if (g.mode == kSgSubtract) {
          float* o = g.out + i * g.ldo + j;
          gstore(o, gload(o) - val);
        } else {
          gstore(g.out + i * g.ldo + j, val);
        }
      }
    }
}

template <int BM>
__device__ __forceinline__ void sgemm_run(const SGemm& g, float* lds) {
  const int local = xcd_remap(blockIdx.x, gridDim.x);
  const int ti = local % g.tiles_m;
  const int rest = local / g.tiles_m;
  const int tj = rest % g.tiles_n;
  const int s = rest / g.tiles_n;
  const int i0 = ti * BM, j0 = tj * BM;
  if (g.a_kmajor) {
    SgKmaj<BM> sa{g.A, g.lda, g.M, i0};
    sgemm_tile<BM>(g, sa, i0, j0, s, lds);
  } else {
    SgKcon<BM> sa{g.A, g.lda, g.M, i0};
    sgemm_tile<BM>(g, sa, i0, j0, s, lds);
  }
}

__global__ __launch_bounds__(kThreads, 2) void qg_rf_sgemm(SGemm g) {
  __shared__ __attribute__((aligned(16))) float lds[2 * SgCfg<128>::STAGE];
  if (g.tile == 64)
    sgemm_run<64>(g, lds);
  else
    sgemm_run<128>(g, lds);
}

// ============================================================ basis format helpers ===
// Qb (M x 2k bf16) = the hi parts bf16(x) of Qf (M x k) in columns 0 .. k-1 and the lo parts
// bf16(x - hi) in k .. 2k-1.
__global__ __launch_bounds__(kThreads) void qg_rf_split(const float* Qf, int64_t M, int k,
                                                        uint16_t* Qb) {
  const int64_t numel = M * k;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < numel; e += stride) {
    const int64_t i = e / k;
    const int j = (int)(e - i * k);
    const float v = gload(Qf + e);
    const uint16_t hi = to_bf16(v);
    gstore(Qb + i * 2 * k + j, hi);
    gstore(Qb + i * 2 * k + k + j, to_bf16(v - bf16_to_f32(hi)));
  }
}

// Gp (m x n8) = G (m x n) with zero columns n .. n8-1, so that rows start on 16-byte bounds.
__global__ __launch_bounds__(kThreads) void qg_rf_pad(const uint16_t* G, int64_t m, int64_t n,
                                                      int64_t n8, uint16_t* Gp) {
  const int64_t numel = m * n8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < numel; e += stride) {
    const int64_t i = e / n8, j = e - i * n8;
    gstore(Gp + e, j < n ? gload(G + i * n + j) : (uint16_t)0);
  }
}

// Per 64-row tile and column of P (m x r): the entry of largest magnitude (signed; the first
// such row on ties), the input of the column sign rule.
__global__ __launch_bounds__(kThreads) void qg_rf_colmax(const float* P, int64_t m, int r,
                                                         float* amax_v) {
  const int c = blockIdx.y * kThreads + threadIdx.x;
  if (c >= r) return;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int64_t i1 = min<int64_t>(m, i0 + 64);
  float bv = gload(P + i0 * r + c);
  for (int64_t i = i0 + 1; i < i1; ++i) {
    const float v = gload(P + i * r + c);
    if (fabsf(v) > fabsf(bv)) bv = v;
  }
  gstore(amax_v + (int64_t)blockIdx.x * r + c, bv);
}

// ================================================================ block Jacobi eigen ===
// C, V and the block rotations J are held in fp64, so that the thousands of rotations a solve
// applies leave V orthogonal and the eigenvalues unmoved to far below fp32 resolution. Inside
// a subproblem the rotations are chosen on an fp32 copy (enough to decide them; any
// orthogonal J serves Jacobi), while J itself is accumulated in fp64 from each rotation's
// (c, s) renormalized in fp64.
typedef double f64x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// The two blocks of pair w in round `round` of the round-robin tournament on nb blocks
// (position 0 holds block 0, positions 1 .. nb-1 the others rotated by `round`; position w
// meets position nb - 1 - w), smaller first.
__device__ __forceinline__ void bj_pair(int nb, int round, int w, int& lo, int& hi) {
  const int a = w == 0 ? 0 : 1 + (w - 1 + round) % (nb - 1);
  const int b = 1 + (nb - 2 - w + round) % (nb - 1);
  lo = min(a, b);
  hi = max(a, b);
}
// Index of a subproblem's local index l (0 .. 2B-1): the first block, then the second.
template <int B>
__device__ __forceinline__ int bj_index(int lo, int hi, int l) {
  return (l < B ? lo : hi) * B + (l & (B - 1));
}
// A sweep is skipped when the previous one rotated nothing.
__device__ __forceinline__ bool bj_converged(const int* rot, int sweep) {
  return sweep > 0 && gload(rot + sweep - 1) == 0;
}

// Cj (K x K) = C (k x k) symmetrized from its upper triangle, zero outside k x k; Vj = I.
__global__ __launch_bounds__(kThreads) void qg_rf_bj_init(const float* C, int k, int K,
                                                          double* Cj, double* Vj) {
  const int64_t numel = (int64_t)K * K;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < numel; e += stride) {
    const int i = (int)(e / K), j = (int)(e - (int64_t)i * K);
    const int lo = min(i, j), hi = max(i, j);
    gstore(Cj + e, hi < k ? (double)gload(C + (int64_t)lo * k + hi) : 0.0);
    gstore(Vj + e, i == j ? 1.0 : 0.0);
  }
}

// abs_tol = 1e-7 * (largest diagonal entry of C), the level of fp32 rounding noise in the
// entries of a positive semidefinite matrix; the rotation flags of all sweeps cleared.
__global__ __launch_bounds__(kThreads) void qg_rf_bj_prep(const float* C, int k, float* abs_tol,
                                                          int* rot, int max_sweeps) {
  __shared__ float red[kThreads];
  float mx = 0.0f;
  for (int i = threadIdx.x; i < k; i += kThreads)
    mx = fmaxf(mx, fabsf(gload(C + (int64_t)i * k + i)));
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + h]);
    __syncthreads();
  }
  if (threadIdx.x == 0) gstore(abs_tol, 1e-7f * red[0]);
  for (int s = threadIdx.x; s < max_sweeps; s += kThreads) gstore(rot + s, 0);
}

// A rotation of the pair (p, q) is taken while |a_pq| exceeds both tol * sqrt(|a_pp a_qq|)
// and abs_tol.
__device__ __forceinline__ bool bj_needs(float app, float aqq, float apq, float tol,
                                         float abs_tol) {
  return fabsf(apq) > tol * __builtin_amdgcn_sqrtf(fabsf(app * aqq)) && fabsf(apq) > abs_tol;
}

// Threads of the subproblem kernel for blocks of B indices: two 2 x 2 blocks of the
// subproblem and four rows of a pair slot of Q per thread.
template <int B>
constexpr int bj_solve_threads() { return B * 2 * B / 4; }

// The symmetric 2 x 2 Schur rotation (Golub and Van Loan, Algorithm 8.5.1) of the pair whose
// smaller index holds app, the larger aqq and the pair apq, in fp32 with the hardware
// reciprocal and square roots (the angle need not be correctly rounded: any rotation close
// to the exact one lowers the off-diagonal norm, and (c, s) are orthonormalized below), with
// (c, s) also in fp64
// scaled to unit length: h = c^2 + s^2 is 1 to fp32 accuracy, and 1.5 - h / 2 is 1 / sqrt(h)
// up to (h - 1)^2. The identity when the pair is below the rotation level.
__device__ __forceinline__ bool bj_rotation(float app, float aqq, float apq, float tol,
                                            float abs_tol, float& c, float& s, double& cd,
                                            double& sd) {
  c = 1.0f;
  s = 0.0f;
  cd = 1.0;
  sd = 0.0;
  if (!bj_needs(app, aqq, apq, tol, abs_tol)) return false;
  const float tau = (aqq - app) * __builtin_amdgcn_rcpf(2.0f * apq);
  const float t = (tau >= 0.0f ? 1.0f : -1.0f) *
                  __builtin_amdgcn_rcpf(fabsf(tau) + __builtin_amdgcn_sqrtf(1.0f + tau * tau));
  c = __builtin_amdgcn_rsqf(1.0f + t * t);
  s = t * c;
  const double h = (double)c * c + (double)s * s;
  const double g = 1.5 - 0.5 * h;
  cd = c * g;
  sd = s * g;
  return true;
}

// Where the indices of a 2B x 2B subproblem sit during its sweep. The B pair slots of an inner
// round are fixed positions (2u, 2u + 1) of the stored matrices; between inner rounds the
// entries move to the positions their indices take in the next round, so that every access
// of the sweep is at an address fixed for the thread.
//   FULL (all index pairs, 2B - 1 inner rounds): the round-robin ("circle") schedule with index
//   0 fixed; slot u pairs a_u = (u == 0 ? 0 : 1 + (u - 1 + rd) mod (2B - 1)) with
//   b_u = 1 + (2B - 2 - u + rd) mod (2B - 1).
//   Cross (the B^2 pairs across the two blocks, B inner rounds): slot u pairs index u with
//   B + (u + rd) mod B.
// Either schedule returns every index to its first position after its last round.
template <int B, bool FULL>
struct BjSched {
  static constexpr int S = 2 * B;
  static constexpr int ROUNDS = FULL ? S - 1 : B;
  // index held at position pos in the first inner round
  __device__ static int index0(int pos) {
    const int u = pos >> 1;
    return (pos & 1) ? (FULL ? S - 1 - u : B + u) : u;
  }
  // position of index j in the first inner round
  __device__ static int pos0(int j) {
    return j < B ? 2 * j : (FULL ? 2 * (S - 1 - j) + 1 : 2 * (j - B) + 1);
  }
  // position that the entry at pos moves to for the next inner round
  __device__ static int next(int pos) {
    const int u = pos >> 1;
    if (!FULL) return (pos & 1) ? 2 * ((u + B - 1) & (B - 1)) + 1 : pos;
    if (pos & 1) return u == B - 1 ? 2 * (B - 1) : 2 * (u + 1) + 1;
    return u <= 1 ? u : 2 * (u - 1);   // p(0) stays, p(1) -> q(0), p(u) -> p(u - 1)
  }
  // whether slot u's first position (2u) holds the larger index of its pair in round rd
  __device__ static bool flipped(int u, int rd) {
    if (!FULL) return false;
    const int a = u == 0 ? 0 : 1 + (u - 1 + rd) % (S - 1);
    const int b = 1 + (S - 2 - u + rd) % (S - 1);
    return a > b;
  }
};

// One sweep of 2 x 2 rotations on the 2B x 2B subproblem of a pair of blocks (the workgroup's
// pair in this round of the tournament on blocks): S <- R^T S R and Q <- Q R from Q = I, S
// held as fp32 and Q as fp64. Q^T goes to Jm[w] (row j of Jm[w] is column j of Q), whether Q
// differs from I to jrot[w], and a rotation taken to rot[sweep].
//
// In the first round of an outer sweep every block is in exactly one subproblem, and the
// sweep covers all index pairs of the subproblem; in the other rounds only the pairs across
// its two blocks, since the pairs inside a block were treated in the first round: every index
// pair of C is thus rotated once per outer sweep, as in cyclic Jacobi.
//
// The subproblem is stored whole (both triangles) in position order (BjSched) in one of two
// buffers, and so is Q^T (row = position, column = row of Q). An inner round reads only the
// current buffers and writes only the other: each thread computes the rotations of the slots
// it needs from the diagonal 2 x 2 blocks, rotates its two 2 x 2 blocks and its four rows of a
// slot of Q, and writes them where their indices sit in the next round; one barrier ends the
// round. A block is computed with the rows of its lower slot rotated first, so both copies of
// an entry agree exactly. A subproblem with no pair over the rotation level is left as it is.
template <int B, bool FULL>
__device__ __forceinline__ void bj_solve_sweep(const double* Cj, int K, int lo, int hi,
                                               float tol, float abs_tol, float* As, double* Qs,
                                               int* need, double* out, bool& active) {
  using Sch = BjSched<B, FULL>;
  constexpr int S = 2 * B, NT = bj_solve_threads<B>(), PA = S + 16, H = B / 2;
  const int t = threadIdx.x;
  // entries (i, j), (i, j + 1) of the subproblem by one 16-byte load (j even: both in one
  // block) to their positions
  for (int e2 = t; e2 < S * S / 2; e2 += NT) {
    const int i = e2 / (S / 2), j = 2 * (e2 % (S / 2));
    const double2 v = gload(reinterpret_cast<const double2*>(
        Cj + (int64_t)bj_index<B>(lo, hi, i) * K + bj_index<B>(lo, hi, j)));
    const int pi = Sch::pos0(i) * PA;
    As[pi + Sch::pos0(j)] = (float)v.x;
    As[pi + Sch::pos0(j + 1)] = (float)v.y;
  }
  for (int e = t; e < S * S; e += NT) {
    const int P = e / S, P2 = e % S;
    Qs[P * S + P2] = Sch::index0(P) == P2 ? 1.0 : 0.0;
  }
  if (t == 0) *need = 0;
  __syncthreads();
  {
    int mine = 0;
    for (int e = t; e < S * S; e += NT) {
      const int i = e / S, j = e % S;
      const bool considered = FULL ? i < j : (i < B && j >= B);
      if (considered) {
        const int pi = Sch::pos0(i), pj = Sch::pos0(j);
        if (bj_needs(As[pi * PA + pi], As[pj * PA + pj], As[pi * PA + pj], tol, abs_tol))
          mine = 1;
      }
    }
    if (mine) *need = 1;
  }
  __syncthreads();
  active = *need != 0;
  // this thread: row slot u1, column slots u2 in {l, l + H}; rows 2l, 2l + 1, B + 2l,
  // B + 2l + 1 of Q in slot u1
  const int u1 = t / H, l = t % H;
  int buf = 0;
  for (int rd = 0; active && rd < Sch::ROUNDS; ++rd) {
    const float* Ac = As + buf * S * PA;
    float* An = As + (buf ^ 1) * S * PA;
    const double* Qc = Qs + buf * S * S;
    double* Qn = Qs + (buf ^ 1) * S * S;
    // slot rotations: lane u of every wave computes slot u's (every lane slot u mod B), and
    // the threads take the ones they need by cross-lane reads. Flip: the slot's first
    // position holds the larger index of its pair; pp, pq: positions of the smaller and the
    // larger index.
    float c_l, s_l;
    double cd_l, sd_l;
    int f_l;
    {
      const int u = (t & 63) & (B - 1);
      const bool f = Sch::flipped(u, rd);
      const float2 d0 = *reinterpret_cast<const float2*>(Ac + 2 * u * PA + 2 * u);
      const float a11 = Ac[(2 * u + 1) * PA + 2 * u + 1];
      bj_rotation(f ? a11 : d0.x, f ? d0.x : a11, d0.y, tol, abs_tol, c_l, s_l, cd_l, sd_l);
      f_l = f ? 1 : 0;
    }
    bool fl[3];
    int pp[3], pq[3];
    float c[3], s[3];
    const int us[3] = {u1, l, l + H};
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      fl[k] = __shfl(f_l, us[k]) != 0;
      c[k] = __shfl(c_l, us[k]);
      s[k] = __shfl(s_l, us[k]);
      pp[k] = 2 * us[k] + (fl[k] ? 1 : 0);
      pq[k] = 2 * us[k] + (fl[k] ? 0 : 1);
    }
    const double cd = __shfl(cd_l, u1), sd = __shfl(sd_l, u1);
    // the two blocks (u1, u2)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int u2 = us[1 + b];
      const float2 r0 = *reinterpret_cast<const float2*>(Ac + 2 * u1 * PA + 2 * u2);
      const float2 r1 = *reinterpret_cast<const float2*>(Ac + (2 * u1 + 1) * PA + 2 * u2);
      // in index order: rows (smaller, larger index of u1), columns (same for u2)
      const bool f1 = fl[0], f2 = fl[1 + b];
      const float2 R0 = f1 ? r1 : r0, R1 = f1 ? r0 : r1;
      const float y00 = f2 ? R0.y : R0.x, y01 = f2 ? R0.x : R0.y;
      const float y10 = f2 ? R1.y : R1.x, y11 = f2 ? R1.x : R1.y;
      // the lower slot's rows are rotated first (the block transposed when u2 < u1)
      const bool rows_low = u1 <= u2;
      const float a = y00, bb = rows_low ? y01 : y10, cc = rows_low ? y10 : y01, d = y11;
      const float c1 = rows_low ? c[0] : c[1 + b], s1 = rows_low ? s[0] : s[1 + b];
      const float c2 = rows_low ? c[1 + b] : c[0], s2 = rows_low ? s[1 + b] : s[0];
      const float ra = c1 * a - s1 * cc, rb = c1 * bb - s1 * d;
      const float rc = s1 * a + c1 * cc, rd2 = s1 * bb + c1 * d;
      const float n_pp = c2 * ra - s2 * rb, n_pq = s2 * ra + c2 * rb;
      const float n_qp = u1 == u2 ? n_pq : c2 * rc - s2 * rd2, n_qq = s2 * rc + c2 * rd2;
      // back in this block's orientation (rows u1): entries (p1, p2), (p1, q2), (q1, p2),
      // (q1, q2)
      const float w_pq = rows_low ? n_pq : n_qp, w_qp = rows_low ? n_qp : n_pq;
      const int np1 = Sch::next(pp[0]) * PA, nq1 = Sch::next(pq[0]) * PA;
      const int np2 = Sch::next(pp[1 + b]), nq2 = Sch::next(pq[1 + b]);
      An[np1 + np2] = n_pp;
      An[np1 + nq2] = w_pq;
      An[nq1 + np2] = w_qp;
      An[nq1 + nq2] = n_qq;
    }
    // rows of Q in slot u1: column p <- cd x - sd y, column q <- sd x + cd y
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = h * B + 2 * l;
      const double2 x = *reinterpret_cast<const double2*>(Qc + pp[0] * S + row);
      const double2 y = *reinterpret_cast<const double2*>(Qc + pq[0] * S + row);
      *reinterpret_cast<double2*>(Qn + Sch::next(pp[0]) * S + row) =
          make_double2(cd * x.x - sd * y.x, cd * x.y - sd * y.y);
      *reinterpret_cast<double2*>(Qn + Sch::next(pq[0]) * S + row) =
          make_double2(sd * x.x + cd * y.x, sd * x.y + cd * y.y);
    }
    __syncthreads();
    buf ^= 1;
  }
  // every index is back at its first position: row j of Q^T is at position pos0(j)
  const double* Qf = Qs + buf * S * S;
  for (int e2 = t; e2 < S * S / 2; e2 += NT) {
    const int e = 2 * e2;
    gstore(reinterpret_cast<double2*>(out + e),
           *reinterpret_cast<const double2*>(Qf + Sch::pos0(e / S) * S + e % S));
  }
}

template <int B>
__global__ __launch_bounds__(bj_solve_threads<B>()) void qg_rf_bj_solve(
    const double* Cj, int K, int nb, int round, int sweep, float tol, const float* abs_tol_p,
    int* rot, double* Jm, int* jrot) {
  if (bj_converged(rot, sweep)) return;
  constexpr int S = 2 * B, PA = S + 16;
  __shared__ __attribute__((aligned(16))) float As[2 * S * PA];
  __shared__ __attribute__((aligned(16))) double Qs[2 * S * S];
  __shared__ int need;
  int lo, hi;
  bj_pair(nb, round, blockIdx.x, lo, hi);
  const float abs_tol = gload(abs_tol_p);
  double* out = Jm + (int64_t)blockIdx.x * S * S;
  bool active;
  if (round == 0)
    bj_solve_sweep<B, true>(Cj, K, lo, hi, tol, abs_tol, As, Qs, &need, out, active);
  else
    bj_solve_sweep<B, false>(Cj, K, lo, hi, tol, abs_tol, As, Qs, &need, out, active);
  if (threadIdx.x == 0) {
    gstore(jrot + blockIdx.x, active ? 1 : 0);
    if (active) gstore(rot + sweep, 1);
  }
}

// A 2B x 2B fp64 product on four waves: wave (wm, wn) holds the B x B quarter at rows wm*B,
// columns wn*B, as (B/16)^2 tiles of 16 x 16 (v_mfma_f64_16x16x4_f64, which gives lane l the
// entries (l / 16 + 4 v, l % 16) of a tile). acc = sum over t < 2B of A(i, t) B(t, j), A and
// B in LDS with pitch 2B + 1, A read as stored ([i][t]) or transposed (stored [t][i]).
template <int B>
struct BjMul {
  static constexpr int S = 2 * B, PT = S + 1, T = B / 16;
  f64x4 acc[T][T];
  __device__ static int row(int x, int v) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave >> 1) * B + 16 * x + (lane >> 4) + 4 * v;
  }
  __device__ static int col(int y) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave & 1) * B + 16 * y + (lane & 15);
  }
  template <bool A_TRANSPOSED>
  __device__ void mul(const double* Am, const double* Bm) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i0 = (wave >> 1) * B, j0 = (wave & 1) * B;
    const int l16 = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int x = 0; x < T; ++x)
#pragma unroll
      for (int y = 0; y < T; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int t = 0; t < S; t += 4) {
      double a[T], b[T];
#pragma unroll
      for (int x = 0; x < T; ++x) {
        const int i = i0 + 16 * x + l16;
        a[x] = A_TRANSPOSED ? Am[(t + kq) * PT + i] : Am[i * PT + t + kq];
      }
#pragma unroll
      for (int y = 0; y < T; ++y) b[y] = Bm[(t + kq) * PT + j0 + 16 * y + l16];
#pragma unroll
      for (int x = 0; x < T; ++x)
#pragma unroll
        for (int y = 0; y < T; ++y) acc[x][y] = mfma_f64(a[x], b[y], acc[x][y]);
    }
  }
  __device__ void put(double* X) const {
#pragma unroll
    for (int x = 0; x < T; ++x)
#pragma unroll
      for (int y = 0; y < T; ++y)
#pragma unroll
        for (int v = 0; v < 4; ++v) X[row(x, v) * PT + col(y)] = acc[x][y][v];
  }
};

// The round's rotations applied to C and V. Workgroups 0 .. nC-1 take the 2B x 2B pieces
// (pairs w1 <= w2) of C: X = C[rows of w1][columns of w2], X' = J1^T X J2, written at
// (w1, w2) and transposed at (w2, w1); a diagonal piece is symmetrized from its upper
// triangle. The others take 2B-row strips of V restricted to one pair's columns: V' = V J.
// Pieces whose rotations are all the identity are left as they are.
template <int B>
__global__ __launch_bounds__(kThreads) void qg_rf_bj_apply(double* Cj, double* Vj, int K, int nb,
                                                           int round, int sweep, const int* rot,
                                                           const double* Jm, const int* jrot) {
  if (bj_converged(rot, sweep)) return;
  constexpr int S = 2 * B, PT = S + 1;
  // two buffers (two workgroups fit on a CU): X, and J1 then J2
  __shared__ double X[S * PT];
  __shared__ double J1[S * PT];
  double* J2 = J1;
  const int P = nb / 2;
  const int nC = P * (P + 1) / 2;
  int bid = blockIdx.x;
  // Jm[w] holds J^T (row j = column j of J); 16-byte loads, two consecutive entries of a row
  // of J^T each
  constexpr int NJ = S * S / 2 / kThreads;   // double2 per thread for a 2B x 2B matrix
  auto fetch_j = [&](double2 (&r)[NJ], int w) {
    const double2* src = reinterpret_cast<const double2*>(Jm + (int64_t)w * S * S);
#pragma unroll
    for (int q = 0; q < NJ; ++q) r[q] = gload(src + threadIdx.x + q * kThreads);
  };
  auto put_j = [&](double* dst, const double2 (&r)[NJ]) {
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
      const int e = 2 * (threadIdx.x + q * kThreads);   // entries e, e + 1 of J^T
      dst[(e % S) * PT + e / S] = r[q].x;
      dst[((e + 1) % S) * PT + e / S] = r[q].y;
    }
  };
  // X[i][j] = M[row(i)][col(j)], 16-byte loads (columns j, j + 1 of one block)
  auto load_x = [&](const double* M, auto row, auto col) {
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
      const int e2 = threadIdx.x + q * kThreads;
      const int i = e2 / (S / 2), j = 2 * (e2 % (S / 2));
      const double2 v = gload(reinterpret_cast<const double2*>(M + row(i) + col(j)));
      X[i * PT + j] = v.x;
      X[i * PT + j + 1] = v.y;
    }
  };
  BjMul<B> m;
  if (bid < nC) {
    int w1 = 0;
    while (bid >= P - w1) {
      bid -= P - w1;
      ++w1;
    }
    const int w2 = w1 + bid;
    if (gload(jrot + w1) == 0 && gload(jrot + w2) == 0) return;
    int lo1, hi1, lo2, hi2;
    bj_pair(nb, round, w1, lo1, hi1);
    bj_pair(nb, round, w2, lo2, hi2);
    double2 jr[NJ];
    fetch_j(jr, w1);
    load_x(Cj, [&](int i) { return (int64_t)bj_index<B>(lo1, hi1, i) * K; },
           [&](int j) { return (int64_t)bj_index<B>(lo2, hi2, j); });
    put_j(J1, jr);
    fetch_j(jr, w2);   // J2 in flight during the first product
    __syncthreads();
    m.template mul<true>(J1, X);   // J1^T X
    __syncthreads();
    m.put(X);
    put_j(J2, jr);
    __syncthreads();
    m.template mul<false>(X, J2);   // (J1^T X) J2
    __syncthreads();
    m.put(X);
    __syncthreads();
    const bool diag = w1 == w2;
    // 16-byte stores of entry pairs (j, j + 1), and of the transposed piece (element
    // (ti, tj) of X to (tj, ti), pairs ti, ti + 1)
    for (int e2 = threadIdx.x; e2 < S * S / 2; e2 += kThreads) {
      const int i = e2 / (S / 2), j = 2 * (e2 % (S / 2));
      const double v0 = diag ? X[min(i, j) * PT + max(i, j)] : X[i * PT + j];
      const double v1 = diag ? X[min(i, j + 1) * PT + max(i, j + 1)] : X[i * PT + j + 1];
      gstore(reinterpret_cast<double2*>(Cj + (int64_t)bj_index<B>(lo1, hi1, i) * K +
                                        bj_index<B>(lo2, hi2, j)),
             make_double2(v0, v1));
      if (!diag) {
        const int tj = i, ti = j;
        gstore(reinterpret_cast<double2*>(Cj + (int64_t)bj_index<B>(lo2, hi2, tj) * K +
                                          bj_index<B>(lo1, hi1, ti)),
               make_double2(X[ti * PT + tj], X[(ti + 1) * PT + tj]));
      }
    }
  } else {
    bid -= nC;
    const int w = bid % P, strip = bid / P;
    if (gload(jrot + w) == 0) return;
    int lo, hi;
    bj_pair(nb, round, w, lo, hi);
    const int64_t r0 = (int64_t)strip * S;
    double2 jr[NJ];
    fetch_j(jr, w);
    load_x(Vj, [&](int i) { return (r0 + i) * K; },
           [&](int j) { return (int64_t)bj_index<B>(lo, hi, j); });
    put_j(J1, jr);
    __syncthreads();
    m.template mul<false>(X, J1);
#pragma unroll
    for (int x = 0; x < BjMul<B>::T; ++x)
#pragma unroll
      for (int y = 0; y < BjMul<B>::T; ++y) {
        const int j = bj_index<B>(lo, hi, BjMul<B>::col(y));
#pragma unroll
        for (int v = 0; v < 4; ++v)
          gstore(Vj + (r0 + BjMul<B>::row(x, v)) * K + j, m.acc[x][y][v]);
      }
  }
}

// Eigenvalues (the diagonal of the converged C) ranked in descending order (ties by index),
// over the k real indices; evals (k), sigma (the square roots of the r largest), the rank of
// each index, and the number of sweeps run (those that rotated, plus the one that found
// nothing left to rotate, at most max_sweeps).
__global__ __launch_bounds__(1024) void qg_rf_bj_rank(const double* Cj, int K, int k, int r,
                                                      const int* rot, int max_sweeps,
                                                      float* evals, float* sigma, int* rank_of,
                                                      int* sweeps_out) {
  __shared__ double d[kRfMaxKWide];
  for (int i = threadIdx.x; i < k; i += 1024) d[i] = gload(Cj + (int64_t)i * K + i);
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += 1024) {
    const double li = d[i];
    int rk = 0;
    for (int j = 0; j < k; ++j) rk += (d[j] > li || (d[j] == li && j < i)) ? 1 : 0;
    gstore(rank_of + i, rk);
    gstore(evals + rk, (float)li);
    if (sigma && rk < r) gstore(sigma + rk, (float)sqrt(fmax(li, 0.0)));
  }
  if (threadIdx.x == 0 && sweeps_out) {
    int s = 0;
    while (s < max_sweeps && gload(rot + s) != 0) ++s;
    gstore(sweeps_out, min(s + 1, max_sweeps));
  }
}

// Vr (k x r, fp32): the eigenvectors of the r largest eigenvalues, in rank order.
__global__ __launch_bounds__(kThreads) void qg_rf_bj_gather(const double* Vj, int K, int k, int r,
                                                            const int* rank_of, float* Vr) {
  const int64_t numel = (int64_t)k * k;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < numel; e += stride) {
    const int i = (int)(e / k), col = (int)(e - (int64_t)i * k);
    const int rk = gload(rank_of + col);
    if (rk < r) gstore(Vr + (int64_t)i * r + rk, (float)gload(Vj + (int64_t)i * K + col));
  }
}

// ======================================================================= launchers ===
namespace {
unsigned grid_for(int64_t numel) {
  const int64_t want = (numel + kThreads - 1) / kThreads;
  return (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
}
}  // namespace

hipError_t launch_rf_sgemm(const SGemm& g, hipStream_t s) {
  const int grid = g.tiles_m * g.tiles_n * g.split;
  hipLaunchKernelGGL(qg_rf_sgemm, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_rf_split(const float* Qf, int64_t M, int k, uint16_t* Qb, hipStream_t s) {
  hipLaunchKernelGGL(qg_rf_split, dim3(grid_for(M * k)), dim3(kThreads), 0, s, Qf, M, k, Qb);
  return hipGetLastError();
}

hipError_t launch_rf_pad(const uint16_t* G, int64_t m, int64_t n, int64_t n8, uint16_t* Gp,
                         hipStream_t s) {
  hipLaunchKernelGGL(qg_rf_pad, dim3(grid_for(m * n8)), dim3(kThreads), 0, s, G, m, n, n8, Gp);
  return hipGetLastError();
}

hipError_t launch_rf_colmax(const float* P, int64_t m, int r, float* amax_v, hipStream_t s) {
  const dim3 grid((unsigned)((m + 63) / 64), (unsigned)((r + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(qg_rf_colmax, grid, dim3(kThreads), 0, s, P, m, r, amax_v);
  return hipGetLastError();
}

template <int B>
static hipError_t block_jacobi_sweeps(int k, int max_sweeps, float tol, const RfBj& w,
                                      hipStream_t s) {
  const int nb = rf_bj_blocks(k, B);
  const int K = nb * B;
  const int P = nb / 2;
  const int apply_grid = P * (P + 1) / 2 + (K / (2 * B)) * P;
  hipError_t e = hipSuccess;
  for (int sweep = 0; sweep < max_sweeps && e == hipSuccess; ++sweep)
    for (int round = 0; round < nb - 1 && e == hipSuccess; ++round) {
      hipLaunchKernelGGL(qg_rf_bj_solve<B>, dim3(P), dim3(bj_solve_threads<B>()), 0, s, w.C, K,
                         nb, round, sweep, tol, w.abs_tol, w.rot, w.J, w.jrot);
      hipLaunchKernelGGL(qg_rf_bj_apply<B>, dim3(apply_grid), dim3(kThreads), 0, s, w.C, w.V, K,
                         nb, round, sweep, w.rot, w.J, w.jrot);
      e = hipGetLastError();
    }
  return e;
}

hipError_t launch_rf_block_jacobi(const float* C, int k, int r, int max_sweeps, float tol,
                                  const RfBj& w, float* evals, float* Vr, float* sigma,
                                  int* sweeps, hipStream_t s) {
  const int B = rf_bj_block(k);
  const int K = rf_bj_blocks(k, B) * B;
  hipLaunchKernelGGL(qg_rf_bj_init, dim3(grid_for((int64_t)K * K)), dim3(kThreads), 0, s, C, k,
                     K, w.C, w.V);
  hipLaunchKernelGGL(qg_rf_bj_prep, dim3(1), dim3(kThreads), 0, s, C, k, w.abs_tol, w.rot,
                     max_sweeps);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess)
    e = B == 16 ? block_jacobi_sweeps<16>(k, max_sweeps, tol, w, s)
                : block_jacobi_sweeps<32>(k, max_sweeps, tol, w, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qg_rf_bj_rank, dim3(1), dim3(1024), 0, s, w.C, K, k, r, w.rot, max_sweeps,
                     evals, sigma, w.rank_of, sweeps);
  hipLaunchKernelGGL(qg_rf_bj_gather, dim3(grid_for((int64_t)k * k)), dim3(kThreads), 0, s, w.V,
                     K, k, r, w.rank_of, Vr);
  return hipGetLastError();
}

}  // namespace qg
