// Products of a linear layer whose weight is stored as INT8 codes with group scales (AIMech
// curated page on Q-GaLore, limitation claim "simulated weight quantization throughput":
// activations stay 16-bit and the INT8 weights are dequantized inside the forward and
// backward passes, so throughput rests on fusing that dequantization). The dequantized
// weight W~ = bf16(q * s) is formed by the stager on its way into LDS and never exists in
// memory. Shapes: X is T x n, W is m x n (outputs x inputs), Y and dY are T x m.
//
//   forward      Y  (T x m) = X W~^T   A = X  [t][i] K-contiguous, B = W [o][i] K-contiguous
//   data grad    dX (T x n) = dY W~    A = dY [t][o] K-contiguous, B = W [o][i] K-major
//   weight grad  G  (m x n) = dY^T X   A = dY [t][o] K-major,      B = X [t][i] K-major
//
// All three accumulate in fp32 on bf16 MFMA and round the result to bf16. The weight
// gradient has only bf16 operands and stages them by LDS DMA.
#include "qg_gemm.hpp"
#include "qg_kernels.hpp"

namespace qg {

// INT8 source [c][k] (row pitch ld codes = the K extent, ld % 8 == 0, c_end rows) with
// group scales over the flat index -> K-contiguous bf16 LDS tile [c][k] (kc_off layout).
// A chunk of 8 codes starting at a multiple of 8 lies inside one 256-element group.
template <int W, int BK>
struct StageInt8C {
  static constexpr int CPR = BK / 8;
  static constexpr int NC = W * CPR / kThreads;
  static constexpr int RPU = kThreads / CPR;
  static_assert(NC * kThreads == W * CPR && RPU * CPR == kThreads && BK == 32,
                "tile splits evenly over the threads");
  rsrc_t rq, rsc;
  uint32_t ld, c_end;
  int c0;
  uint2 w[NC];
  float s[NC];

  __device__ StageInt8C(const int8_t* q, const float* sc, int64_t ld_, int64_t c_end_, int c0_)
      : ld((uint32_t)ld_), c_end((uint32_t)c_end_), c0(c0_) {
    const uint32_t numel = (uint32_t)(c_end_ * ld_);
    rq = make_rsrc(q, numel);
    rsc = make_rsrc(sc, ((numel + kGroup - 1) / kGroup) * 4);
  }

  __device__ __forceinline__ void load(int64_t k0_) {
    const uint32_t k = (uint32_t)k0_ + 8 * (threadIdx.x % CPR);
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const uint32_t row = c0 + threadIdx.x / CPR + u * RPU;
      const bool in = row < c_end && k < ld;
      const uint32_t e = row * ld + k;
      w[u] = bload64(rq, in ? e : kOOB);
      s[u] = bloadf(rsc, in ? (e >> 8) * 4 : kOOB);
    }
  }

  template <int PITCH>
  __device__ __forceinline__ void store(uint16_t* lds) const {
    static_assert(PITCH == 32, "K-contiguous tiles take 32-element rows");
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        f[e] = mul_rn((float)(int8_t)((e < 4 ? w[u].x : w[u].y) >> (8 * (e & 3))), s[u]);
      *reinterpret_cast<uint4*>(lds + kc_off(q / CPR, q % CPR)) =
          make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7]));
    }
  }
};

using LinFwdTile = Tile<128, 256, 32, 2, 2, false, false>;
using LinBwdDataTile = Tile<128, 256, 32, 2, 2, false, true>;
using LinBwdWeightTile = Tile<128, 256, 32, 2, 2, true, true, true>;
static_assert(LinFwdTile::BM == kLinTileM && LinFwdTile::BN == kLinTileN &&
                  LinBwdDataTile::BM == kLinTileM && LinBwdDataTile::BN == kLinTileN &&
                  LinBwdWeightTile::BM == kLinTileM && LinBwdWeightTile::BN == kLinTileN,
              "host and device tiles agree");

constexpr int cmax_i(int a, int b) { return a > b ? a : b; }
constexpr int lin_lds_elems() {
  return cmax_i(cmax_i(2 * LinFwdTile::STAGE, 2 * LinBwdDataTile::STAGE),
                3 * LinBwdWeightTile::STAGE);
}

// Rounds the accumulators to bf16 and stores the tile of out (M x N row-major); positions
// outside the matrix are dropped by the buffer range.
template <class T>
__device__ __forceinline__ void store_bf16_tile(uint16_t* out, int64_t M, int64_t N, int i0,
                                                int j0, const f32x16 (&acc)[T::XM][T::XN]) {
  const uint32_t Mu = (uint32_t)M, Nu = (uint32_t)N;
  const rsrc_t ro = make_rsrc(out, Mu * Nu * 2);
#pragma unroll
  for (int x = 0; x < T::XM; ++x)
#pragma unroll
    for (int y = 0; y < T::XN; ++y) {
      const uint32_t j = j0 + acc_col<T>(y);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t i = i0 + acc_row<T>(x, v);
        bstore16(ro, (i < Mu && j < Nu) ? (i * Nu + j) * 2 : kOOB, to_bf16(acc[x][y][v]));
      }
    }
}

__global__ __launch_bounds__(kThreads, 2) void qg_lin_fwd(LinArgs a) {
  using T = LinFwdTile;
  __shared__ __attribute__((aligned(16))) uint16_t lds[lin_lds_elems()];
  const int local = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles_m = (int)((a.T + T::BM - 1) / T::BM);
  const int i0 = (local % tiles_m) * T::BM, j0 = (local / tiles_m) * T::BN;
  StageBf16C<T::BM, T::BK> sa(a.act, a.n, a.T, i0);
  StageInt8C<T::BN, T::BK> sb(a.Wq, a.Ws, a.n, a.m, j0);
  f32x16 acc[T::XM][T::XN];
  gemm_kloop<T, 1>(
      sa, sb, [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); },
      [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); }, 0, a.n,
      lds, acc);
  store_bf16_tile<T>(a.out, a.T, a.m, i0, j0, acc);
}

__global__ __launch_bounds__(kThreads, 2) void qg_lin_bwd_data(LinArgs a) {
  using T = LinBwdDataTile;
  __shared__ __attribute__((aligned(16))) uint16_t lds[lin_lds_elems()];
  const int local = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles_m = (int)((a.T + T::BM - 1) / T::BM);
  const int i0 = (local % tiles_m) * T::BM, j0 = (local / tiles_m) * T::BN;
  StageBf16C<T::BM, T::BK> sa(a.act, a.m, a.T, i0);
  StageInt8K<T::BN, T::BK> sb(reinterpret_cast<const uint8_t*>(a.Wq), a.Ws, a.n, a.m, a.m, a.n,
                              j0);
  f32x16 acc[T::XM][T::XN];
  gemm_kloop<T, 1>(
      sa, sb, [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); },
      [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); }, 0, a.m,
      lds, acc);
  store_bf16_tile<T>(a.out, a.T, a.n, i0, j0, acc);
}

__global__ __launch_bounds__(kThreads, 2) void qg_lin_bwd_weight(LinArgs a) {
  using T = LinBwdWeightTile;
  __shared__ __attribute__((aligned(16))) uint16_t lds[lin_lds_elems()];
  const int local = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles_m = (int)((a.m + T::BM - 1) / T::BM);
  const int i0 = (local % tiles_m) * T::BM, j0 = (local / tiles_m) * T::BN;
  const DmaBf16K<T::BM, T::BK> sa(a.act, a.m, a.T, a.m, i0);    // dY as [t][o]
  const DmaBf16K<T::BN, T::BK> sb(a.act2, a.n, a.T, a.n, j0);   // X as [t][i]
  f32x16 acc[T::XM][T::XN];
  gemm_kloop_dma<T>(sa, sb, 0, a.T, lds, acc);
  store_bf16_tile<T>(a.out, a.m, a.n, i0, j0, acc);
}

hipError_t launch_linear(const LinArgs& a, int which, hipStream_t s) {
  const int64_t tm = (which == kLinBwdWeight ? a.m : a.T);
  const int64_t tn = (which == kLinFwd ? a.m : a.n);
  const int grid = (int)(((tm + kLinTileM - 1) / kLinTileM) * ((tn + kLinTileN - 1) / kLinTileN));
  if (which == kLinFwd)
    hipLaunchKernelGGL(qg_lin_fwd, dim3(grid), dim3(kThreads), 0, s, a);
  else if (which == kLinBwdData)
    hipLaunchKernelGGL(qg_lin_bwd_data, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(qg_lin_bwd_weight, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qg
