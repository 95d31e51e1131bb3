// gfx950 kernels of the Q-GaLore optimizer step.
//
// Method: AIMech curated page "Q-GaLore (Quantized GaLore with INT4 Projection and
// Layer-Adaptive Low-Rank Gradients)", mechanism claim "INT4 projection and INT8 stochastic
// rounding" (paper Section 3.2): W^Q <- W^Q + xi(alpha * P^Q * G~) with INT4 P, INT8 W and
// INT8 low-rank moments M, V; and mechanism claim "layer-adaptive subspace cosine schedule"
// (paper Section 3.1, Equation (5)) for the similarity test.
//
// One step of one layer is three launches:
//   qg_project      R (split-K partials) = P~^T G          bf16 MFMA, fp32 accumulation
//   qg_adam         R -> Adam with INT8 M, V -> N~ (bf16)  one wave per 256-element group
//   qg_backproject  U = alpha * P~ N~ and the stochastic rounding of W, fused
// A grouped launch runs each kernel once over a whole table of layers.
#include "qg_gemm.hpp"
#include "qg_kernels.hpp"

namespace qg {

// ========================================================================== dequant ===
// P~ = bf16(q * s) for the whole m x r projection, once per step, into the workspace: the
// projection and the back-projection both stage P~ from it (the INT4 (or INT8) store is
// what persists; this copy lives only for the step). Each thread converts four chunks of 8
// codes (each in one 256-element scale group); a chunk past the end of P is skipped. A bf16
// projection needs no pass (its layers have no workgroups here).
// Dequantize 8 INT8 codes (two little-endian words) with their group scale.
__device__ __forceinline__ uint4 dequant8_i8(uint2 w, float s) {
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    f[e] = mul_rn((float)(int8_t)((e < 4 ? w.x : w.y) >> (8 * (e & 3))), s);
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

__global__ __launch_bounds__(kThreads) void qg_dequant(StepArgs a) {
  int local;
  const LayerDev L = fetch_layer(a, KDEQ, blockIdx.x, local);
  const uint32_t numel = (uint32_t)(L.m * L.r);
  // the workgroup's kThreads * kDeqCodes codes as kDeqCodes / 8 passes of one 8-code chunk
  // per thread, consecutive threads on consecutive chunks: each store instruction of a wave
  // writes 1 KiB of bf16 contiguously
  const uint32_t base = (uint32_t)local * kThreads * kDeqCodes;
  const rsrc_t rs = make_rsrc(L.Ps, ((numel + kGroup - 1) / kGroup) * 4);
  const rsrc_t ro = make_rsrc(a.ws + L.off_p, numel * 2);
  const bool i8 = L.p_format == kPInt8;
  const rsrc_t rq = make_rsrc(L.Pq, i8 ? numel : (numel + 1) / 2);
  constexpr int NP = kDeqCodes / 8;
  uint32_t e[NP];
  uint2 w[NP];
  float sc[NP];
#pragma unroll
  for (int c = 0; c < NP; ++c) {   // all loads first
    e[c] = base + ((uint32_t)c * kThreads + threadIdx.x) * 8;
    const bool in = e[c] < numel;   // numel is a multiple of 8
    w[c] = i8 ? bload64(rq, in ? e[c] : kOOB) : make_uint2(bload32(rq, in ? e[c] >> 1 : kOOB), 0u);
    sc[c] = bloadf(rs, in ? (e[c] >> 8) * 4 : kOOB);
  }
#pragma unroll
  for (int c = 0; c < NP; ++c)
    if (e[c] < numel)
      bstore128(ro, e[c] * 2, i8 ? dequant8_i8(w[c], sc[c]) : dequant8(w[c].x, sc[c]));
}

// ============================================================================== Adam ===
// One wave per group of 256 flat elements of the r x n moments; lane l owns elements
// 4l .. 4l+3 of the group. adam_group takes the lane's four entries of R (its fp32 sums)
// and does the rest: moments from their INT8 codes, the update, N~, absmax requantization.

// The lane's four M and V codes of group g (packed little-endian; zero past the end).
__device__ __forceinline__ void adam_codes(const LayerDev& L, int64_t g, int lane,
                                           uint32_t& wm, uint32_t& wv) {
  const int64_t numel = L.r * L.n;
  const int64_t e0 = g * kGroup + 4 * lane;
  if (e0 + 4 <= numel) {
    wm = gload(reinterpret_cast<const uint32_t*>(L.Mq + e0));
    wv = gload(reinterpret_cast<const uint32_t*>(L.Vq + e0));
  } else {
    wm = wv = 0;
    for (int t = 0; t < 4; ++t)
      if (e0 + t < numel) {
        wm |= (uint32_t)(uint8_t)gload(L.Mq + e0 + t) << (8 * t);
        wv |= (uint32_t)(uint8_t)gload(L.Vq + e0 + t) << (8 * t);
      }
  }
}

// wm, wv: the lane's codes (adam_codes); ms, vs: the group's scales.
__device__ __forceinline__ void adam_group(const StepArgs& a, const LayerDev& L, int64_t g,
                                           int lane, const float (&R)[4], uint32_t wm,
                                           uint32_t wv, float ms, float vs) {
  const int64_t numel = L.r * L.n;
  const int64_t e0 = g * kGroup + 4 * lane;
  const bool full = e0 + 4 <= numel;
  uint16_t* Nb = reinterpret_cast<uint16_t*>(a.ws + L.off_n);
  int8_t mq[4], vq[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    mq[t] = (int8_t)(wm >> (8 * t));
    vq[t] = (int8_t)(wv >> (8 * t));
  }

  float m1[4], v1[4], N[4];
  float am = 0.f, av = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float m0 = mul_rn((float)mq[t], ms);
    const float v0 = mul_rn((float)vq[t], vs);
    m1[t] = add_rn(mul_rn(a.beta1, m0), mul_rn(a.c1, R[t]));
    v1[t] = add_rn(mul_rn(a.beta2, v0), mul_rn(a.c2, mul_rn(R[t], R[t])));
    const float mh = div_by_recip64(m1[t], a.ibc1);   // RN(m1 / bc1)
    const float vh = div_by_recip64(v1[t], a.ibc2);   // RN(v1 / bc2)
    N[t] = -div_rn(mul_rn(L.lr, mh), add_rn(sqrt_rn(vh), L.eps));
    if (e0 + t >= numel) {
      m1[t] = 0.f;
      v1[t] = 0.f;
    }
    am = fmaxf(am, fabsf(m1[t]));
    av = fmaxf(av, fabsf(v1[t]));
  }
  am = wave_max(am);
  av = wave_max(av);
  const float sm = div_rn(am, 127.0f), sv = div_rn(av, 127.0f);
  const float im = recip_or_zero(sm), iv = recip_or_zero(sv);
  uint32_t om = 0, ov = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int qm = (int)fminf(fmaxf(rintf(mul_rn(m1[t], im)), -127.f), 127.f);
    const int qv = (int)fminf(fmaxf(rintf(mul_rn(v1[t], iv)), -127.f), 127.f);
    om |= (uint32_t)(qm & 0xFF) << (8 * t);
    ov |= (uint32_t)(qv & 0xFF) << (8 * t);
  }
  if (full) {
    gstore(reinterpret_cast<uint32_t*>(L.Mq + e0), om);
    gstore(reinterpret_cast<uint32_t*>(L.Vq + e0), ov);
    if (L.R_out)
      gstore(reinterpret_cast<float4*>(L.R_out + e0), make_float4(R[0], R[1], R[2], R[3]));
  } else {
    for (int t = 0; t < 4; ++t)
      if (e0 + t < numel) {
        gstore(L.Mq + e0 + t, (int8_t)(om >> (8 * t)));
        gstore(L.Vq + e0 + t, (int8_t)(ov >> (8 * t)));
        if (L.R_out) gstore(L.R_out + e0 + t, R[t]);
      }
  }
  // N~ rows are ldn elements apart (n rounded up to a multiple of 8): element e of the flat
  // r x n order sits at (e / n) * ldn + e % n
  if (full && L.ldn == L.n) {
    gstore(reinterpret_cast<uint2*>(Nb + e0),
           make_uint2(pack_bf16x2(N[0], N[1]), pack_bf16x2(N[2], N[3])));
  } else {
    int64_t k = e0 / L.n, j = e0 - k * L.n;
    for (int t = 0; t < 4; ++t) {
      if (e0 + t < numel) gstore(Nb + k * L.ldn + j, to_bf16(N[t]));
      if (++j == L.n) {
        j = 0;
        ++k;
      }
    }
  }
  if (lane == 0) {
    gstore(L.Ms + g, sm);
    gstore(L.Vs + g, sv);
  }
}

__global__ __launch_bounds__(kThreads) void qg_adam(StepArgs a) {
  int local;
  const LayerDev L = fetch_layer(a, KADAM, blockIdx.x, local);
  const int lane = threadIdx.x & 63;
  const int64_t numel = L.r * L.n;
  const int64_t ngroups = (numel + kGroup - 1) / kGroup;
  const int64_t g = (int64_t)local * (kThreads / 64) + (threadIdx.x >> 6);
  if (g >= ngroups) return;
  const int64_t e0 = g * kGroup + 4 * lane;
  const bool full = e0 + 4 <= numel;
  // R = the split-K partial sums, added in order
  float R[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < L.split; ++s) {
    const float* src = reinterpret_cast<const float*>(a.ws + L.off_r) + (int64_t)s * L.rpitch + e0;
    float p[4] = {0.f, 0.f, 0.f, 0.f};
    if (full) {
      const float4 q = gload(reinterpret_cast<const float4*>(src));
      p[0] = q.x; p[1] = q.y; p[2] = q.z; p[3] = q.w;
    } else {
      for (int t = 0; t < 4; ++t)
        if (e0 + t < numel) p[t] = gload(src + t);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) R[t] = (s == 0) ? p[t] : add_rn(R[t], p[t]);
  }
  uint32_t wm, wv;
  adam_codes(L, g, lane, wm, wv);
  adam_group(a, L, g, lane, R, wm, wv, gload(L.Ms + g), gload(L.Vs + g));
}

// Adam on one whole 256-element group by 16 lanes (the fused projection epilogue): lane l
// of the group owns columns 64k + 4l .. 64k + 4l + 3 (k = 0..3) of the row. Same arithmetic
// per element as adam_group; the group absmax is a max, so the lane layout does not change
// the result. R holds the lane's 16 values (R[4k + t] for column 64k + 4l + t); cm / cv its
// 4 words of M / V codes.
__device__ __forceinline__ void adam_group16(const StepArgs& a, const LayerDev& L, int64_t g,
                                             int l, const float (&R)[16],
                                             const uint32_t (&cm)[4], const uint32_t (&cv)[4]) {
  const int64_t e0 = g * kGroup + 4 * l;
  uint16_t* Nb = reinterpret_cast<uint16_t*>(a.ws + L.off_n);
  const float ms = gload(L.Ms + g), vs = gload(L.Vs + g);
  // fresh moments and their group absmax first; the update is formed per 4-element run
  // afterwards, so that only m1 and v1 stay live across the reduction
  float m1[16], v1[16];
  float am = 0.f, av = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float m0 = mul_rn((float)(int8_t)(cm[e >> 2] >> (8 * (e & 3))), ms);
    const float v0 = mul_rn((float)(int8_t)(cv[e >> 2] >> (8 * (e & 3))), vs);
    m1[e] = add_rn(mul_rn(a.beta1, m0), mul_rn(a.c1, R[e]));
    v1[e] = add_rn(mul_rn(a.beta2, v0), mul_rn(a.c2, mul_rn(R[e], R[e])));
    am = fmaxf(am, fabsf(m1[e]));
    av = fmaxf(av, fabsf(v1[e]));
  }
  if (L.R_out) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      gstore(reinterpret_cast<float4*>(L.R_out + e0 + 64 * k),
             make_float4(R[4 * k], R[4 * k + 1], R[4 * k + 2], R[4 * k + 3]));
  }
  am = max16(am);
  av = max16(av);
  const float sm = div_rn(am, 127.0f), sv = div_rn(av, 127.0f);
  const float im = recip_or_zero(sm), iv = recip_or_zero(sv);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t om = 0, ov = 0;
    float N[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float mh = div_by_recip64(m1[4 * k + t], a.ibc1);   // RN(m1 / bc1)
      const float vh = div_by_recip64(v1[4 * k + t], a.ibc2);   // RN(v1 / bc2)
      N[t] = -div_rn(mul_rn(L.lr, mh), add_rn(sqrt_rn(vh), L.eps));
      const int qm = (int)fminf(fmaxf(rintf(mul_rn(m1[4 * k + t], im)), -127.f), 127.f);
      const int qv = (int)fminf(fmaxf(rintf(mul_rn(v1[4 * k + t], iv)), -127.f), 127.f);
      om |= (uint32_t)(qm & 0xFF) << (8 * t);
      ov |= (uint32_t)(qv & 0xFF) << (8 * t);
    }
    const int64_t e = e0 + 64 * k;
    gstore(reinterpret_cast<uint32_t*>(L.Mq + e), om);
    gstore(reinterpret_cast<uint32_t*>(L.Vq + e), ov);
    gstore(reinterpret_cast<uint2*>(Nb + e),
           make_uint2(pack_bf16x2(N[0], N[1]), pack_bf16x2(N[2], N[3])));
  }
  if (l == 0) {
    gstore(L.Ms + g, sm);
    gstore(L.Vs + g, sv);
  }
}

// ======================================================================== projection ===

// Tile: 128 rows of R (rank index) x 256 columns, K stages of 32, four waves of 64 x 128
// (eight MFMA accumulator blocks each), two workgroups per CU. Both operands are K-major in
// memory (P is [k][i], G is [k][j]).
using ProjTile = Tile<128, 256, 32, 2, 2, true, true>;
using ProjTileD = Tile<128, 256, 32, 2, 2, true, true, true>;   // direct-to-LDS staging
static_assert(ProjTile::BM == kProjTileM && ProjTile::BN == kProjTileN,
              "host and device projection tiles agree");
static_assert(ProjTile::BN == kGroup, "a tile row spans one Adam group when n % 256 == 0");

// The fused Adam epilogue stages one 32-row chunk of both wave rows (64 rows x 256 columns,
// fp32) in LDS; the row pitch is 8 (mod 16) words so that the two row halves a staging store
// writes (rows R and R + 4) fall on disjoint banks.
constexpr int kAdamPitch = ProjTile::BN + 8;
constexpr int kAdamLdsElems = 2 * ProjTile::WM * 32 * kAdamPitch;   // fp32 = two bf16 slots
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kProjLdsElems =
    cmax(cmax(2 * ProjTile::STAGE, 3 * ProjTileD::STAGE), kAdamLdsElems);

// LDS code areas of the projection kernel's INT4 stager (three stages). They sit after the
// DMA ring in the kernel's LDS array, which the register-staged path and the Adam epilogue
// share as well (neither of them uses code areas).
using ProjCodes = DmaInt4K<ProjTile::BM, ProjTile::BK>;
constexpr int kProjRingBytes = 3 * ProjTileD::STAGE * 2;
constexpr int kProjLdsBytes(int pm) {
  return pm == kPStaged ? kProjLdsElems * 2
                        : cmax(kProjLdsElems * 2, kProjRingBytes + 3 * ProjCodes::AREA);
}

// VEC: rows of G are a multiple of 8 elements: 16-byte chunks staged straight into LDS
// (T in the DMA layout). Otherwise G goes through registers (each 8-element chunk from
// aligned dwords, funnel-shifted to its start).
// PM: which projection paths to compile (kPStaged, kPInline, kPMixed); a layer takes the
// INT4 stager path when L.p_inline.
template <class T, bool VEC, int PM>
__device__ __forceinline__ void project_tile(const StepArgs& a, const LayerDev& L, int local,
                                             uint16_t* lds, uint8_t* codes) {
  static_assert(T::DMA == VEC, "DMA layout exactly on the vector path");
  // local = ((s * tiles_j) + tj) * tiles_i + ti: the row tiles that share a block of G
  // columns are neighbours (and, after the renumbering, on the same XCD).
  const int ti = local % L.p_tiles_i;
  const int rest = local / L.p_tiles_i;
  const int tj = rest % L.p_tiles_j;
  const int s = rest / L.p_tiles_j;
  const int i0 = ti * T::BM, j0 = tj * T::BN;
  const int64_t k_begin = (int64_t)s * L.kslab;
  const int64_t k_end = min<int64_t>(L.m, k_begin + L.kslab);

  // A = P~^T: the INT4 codes of P (m x r, [k][i]) dequantized on their way into LDS, or the
  // bf16 P~ the dequant kernel wrote for this step (or the caller's bf16 P).
  const bool inl = PM == kPInline || (PM == kPMixed && L.p_inline);
  f32x16 acc[T::XM][T::XN];
  auto store_a = [](auto& st, uint16_t* p) { st.template store<T::A_PITCH>(p); };
  auto store_b = [](auto& st, uint16_t* p) { st.template store<T::B_PITCH>(p + T::A_ELEMS); };
  if constexpr (VEC) {
    const DmaBf16K<T::BN, T::BK> sb(L.G, L.n, k_end, L.n, j0);
    if (PM != kPStaged && inl) {
      const ProjCodes sa(L.Pq, L.Ps, L.r, L.m, k_end, i0);
      gemm_kloop_dma_cvt<T, 3>(sa, sb, k_begin, k_end, lds, codes, acc);
    } else if (PM != kPInline) {
      const DmaBf16K<T::BM, T::BK> sa(p_tilde(a, L), L.r, k_end, L.r, i0);
      gemm_kloop_dma<T>(sa, sb, k_begin, k_end, lds, acc);
    }
  } else {
    StageBf16K<T::BN, T::BK, false> sb(L.G, L.n, L.m, k_end, L.n, j0);
    if (PM != kPStaged && inl) {
      StageInt4K<T::BM, T::BK> sa(L.Pq, L.Ps, L.r, L.m, k_end, L.r, i0);
      gemm_kloop<T, 1>(sa, sb, store_a, store_b, k_begin, k_end, lds, acc);
    } else if (PM != kPInline) {
      StageBf16K<T::BM, T::BK, true> sa(p_tilde(a, L), L.r, L.m, k_end, L.r, i0);
      gemm_kloop<T, 1>(sa, sb, store_a, store_b, k_begin, k_end, lds, acc);
    }
  }

  if (L.fuse_adam) {
    // One K split and rows made of whole 256-element groups: each tile row is one Adam group,
    // complete in this workgroup, so Adam runs here instead of a separate pass over R.
    // Chunk x holds rows 32x .. 32x+31 of both wave rows (64 rows: tile rows wm*WTM + 32x +
    // rr). Wave w takes chunk rows 16w .. 16w+15 in four passes of four rows, 16 lanes per
    // row (adam_group16).
    float* E = reinterpret_cast<float*>(lds);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave_m<T>(), wn = wave_n<T>();
    const int l16 = lane & 15;
    const int64_t gpr = L.n / kGroup;   // groups per row of R
    static_for<T::XM>([&](auto xc) {
      constexpr int x = decltype(xc)::value;
#pragma unroll
      for (int y = 0; y < T::XN; ++y)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          E[(wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * kAdamPitch + wn * T::WTN +
            32 * y + (lane & 31)] = acc[x][y][v];
      __syncthreads();
#pragma unroll 1
      for (int p = 0; p < 4; ++p) {
        const int rc = 16 * wave + 4 * p + (lane >> 4);   // chunk row 0 .. 63
        const uint32_t i = i0 + (rc >> 5) * T::WTM + 32 * x + (rc & 31);
        if (i < (uint32_t)L.r) {
          const int64_t g = (int64_t)i * gpr + j0 / kGroup;
          const int64_t e0 = g * kGroup + 4 * l16;
          uint32_t cm[4], cv[4];
          float R[16];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            cm[k] = gload(reinterpret_cast<const uint32_t*>(L.Mq + e0 + 64 * k));
            cv[k] = gload(reinterpret_cast<const uint32_t*>(L.Vq + e0 + 64 * k));
            const float4 q =
                *reinterpret_cast<const float4*>(E + rc * kAdamPitch + 64 * k + 4 * l16);
            R[4 * k] = q.x;
            R[4 * k + 1] = q.y;
            R[4 * k + 2] = q.z;
            R[4 * k + 3] = q.w;
          }
          adam_group16(a, L, g, l16, R, cm, cv);
        }
      }
      __syncthreads();
    });
    return;
  }

  // Partial sums of this K-split; out-of-range rows and columns are dropped by the buffer.
  const rsrc_t ro = make_rsrc(a.ws + L.off_r + (int64_t)s * L.rpitch * 4,
                              (uint32_t)(L.r * L.n * 4));
  const uint32_t n = (uint32_t)L.n, r = (uint32_t)L.r;
#pragma unroll
  for (int x = 0; x < T::XM; ++x)
#pragma unroll
    for (int y = 0; y < T::XN; ++y) {
      const uint32_t j = j0 + acc_col<T>(y);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t i = i0 + acc_row<T>(x, v);
        bstoref(ro, (i < r && j < n) ? (i * n + j) * 4 : kOOB, acc[x][y][v]);
      }
    }
}

// Held to 256 registers per lane so that two waves share each SIMD.
template <int PM>
__global__ __launch_bounds__(kThreads, 2) void qg_project(StepArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kProjLdsBytes(PM) / 2];
  uint8_t* codes = reinterpret_cast<uint8_t*>(lds) + kProjRingBytes;
  int local;
  const LayerDev L = fetch_layer(a, KPROJ, xcd_remap(blockIdx.x, gridDim.x), local);
  if (L.n % 8 == 0)
    project_tile<ProjTileD, true, PM>(a, L, local, lds, codes);
  else
    project_tile<ProjTile, false, PM>(a, L, local, lds, codes);
}

// ===================================================== back-projection + rounding ===

// Stochastic rounding of 8 consecutive weights (i, j8 .. j8+7), j8 a multiple of 8: one
// Philox call yields the 8 16-bit uniforms of the column block.
struct SrCtx {
  rsrc_t rw, rws, ru;
  uint32_t n, m;
  bool write_u;
};

// New INT8 code of one weight: d = (w + U * inv) + u with one rounding per operation. u is a
// multiple of 2^-16 below 1, so fma(bits, 2^-16, t) is exactly the rounded sum t + u.
__device__ __forceinline__ float sr_pre(int w, float U, float inv, uint32_t bits) {
  const float tp = add_rn((float)w, mul_rn(U, inv));
  return __builtin_fmaf((float)bits, 1.0f / 65536.0f, tp);
}
__device__ __forceinline__ int sr_code(float d) {
  return (int)fminf(fmaxf(floorf(d), -127.f), 127.f);
}

// Vector path (rows a multiple of 16): 16 consecutive weights (i, j16 .. j16+15), j16 a
// multiple of 16, arrive prefetched in `wv`; they lie in one scale group (reciprocal `inv`)
// and take two Philox blocks. FOLD (the layer's fold_alpha): U is not written and `inv`
// holds fl(alpha * (1/s)), so that U * (1/s) is taken as S * inv, one multiply per weight.
template <bool FOLD>
__device__ __forceinline__ void sr_block16(const SrCtx& c, const LayerDev& L,
                                           const StepArgs& a, uint32_t i, uint32_t j16,
                                           const float* S, float inv, uint4 wv) {
  uint32_t words[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 ph =
        philox4x32_10(make_uint4((j16 >> 3) + h, i, a.step, L.layer_id), a.seed_lo, a.seed_hi);
    words[4 * h + 0] = ph.x;
    words[4 * h + 1] = ph.y;
    words[4 * h + 2] = ph.z;
    words[4 * h + 3] = ph.w;
  }
  const uint32_t e0 = i * c.n + j16;
  const uint32_t win[4] = {wv.x, wv.y, wv.z, wv.w};
  float U[16], d[16], wf[16];
  // d = W + a + u (|W| <= 127, 0 <= u < 1) is finite exactly when a = U * inv is, so the run
  // is tested once: the largest |a|, by the NaN-propagating maximum (v_maximum3_f32)
  float amax = 0.0f;
  static_for<16>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    U[t] = FOLD ? S[t] : mul_rn(L.alpha, S[t]);
    wf[t] = sbyte_to_f32<t & 3>(win[t >> 2]);
    const uint32_t bits = (t & 1) ? (words[t >> 1] >> 16) : (words[t >> 1] & 0xFFFFu);
    const float a = mul_rn(U[t], inv);
    amax = t == 0 ? __builtin_fabsf(a) : __builtin_elementwise_maximum(amax, __builtin_fabsf(a));
    d[t] = __builtin_fmaf((float)bits, 1.0f / 65536.0f, add_rn(wf[t], a));
  });
  uint32_t wout[4] = {0, 0, 0, 0};
  if (__builtin_isfinite(amax)) {
    // clamp(floor(d), -127, 127) as floor(clamp(d, -127, 127)) (floor is monotone and the
    // bounds are integers): a float clamp, then the floor conversion writes the code
    // straight into its byte of the packed word
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = __builtin_amdgcn_fmed3f(d[4 * k + u], -127.f, 127.f);
      uint32_t w = floor_into_byte<0>(0u, q[0]);
      w = floor_into_byte<1>(w, q[1]);
      w = floor_into_byte<2>(w, q[2]);
      wout[k] = floor_into_byte<3>(w, q[3]);
    }
  } else {
    int w[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) w[t] = (int)wf[t];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int nw = __builtin_isfinite(d[t]) ? sr_code(d[t]) : w[t];
      wout[t >> 2] |= (uint32_t)(nw & 0xFF) << (8 * (t & 3));
    }
  }
  bstore128(c.rw, e0, make_uint4(wout[0], wout[1], wout[2], wout[3]));
  if (!FOLD && c.write_u) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      bstore128(c.ru, (e0 + 4 * k) * 4,
                make_uint4(__float_as_uint(U[4 * k]), __float_as_uint(U[4 * k + 1]),
                           __float_as_uint(U[4 * k + 2]), __float_as_uint(U[4 * k + 3])));
  }
}

// Element path for rows whose length is not a multiple of 16 (possibly straddling scale
// groups): byte accesses and a scale lookup per element. FOLD as for sr_block16.
template <bool FOLD>
__device__ __forceinline__ void sr_block8_elem(const SrCtx& c, const LayerDev& L,
                                               const StepArgs& a, uint32_t i, uint32_t j8,
                                               const float* S) {
  if (j8 >= c.n) return;
  const uint4 ph = philox4x32_10(make_uint4(j8 >> 3, i, a.step, L.layer_id), a.seed_lo, a.seed_hi);
  const uint32_t words[4] = {ph.x, ph.y, ph.z, ph.w};
  const uint32_t e0 = i * c.n + j8;
  // the run's (at most 8) weights lie in at most two scale groups
  const uint32_t g0 = e0 >> 8, g1 = (e0 + min(8u, c.n - j8) - 1) >> 8;
  float inv0 = recip_or_zero(bloadf(c.rws, g0 * 4));
  float inv1 = inv0;
  if (g1 != g0) inv1 = recip_or_zero(bloadf(c.rws, g1 * 4));
  if (FOLD) {
    inv0 = mul_rn(L.alpha, inv0);
    inv1 = mul_rn(L.alpha, inv1);
  }
  // the run's 8 code bytes from the three dwords at the aligned offset at or below e0 (bytes
  // past the row belong to the next one and are not used); the layer's last run, whose dwords
  // may reach past W's end, reads byte by byte
  uint32_t wb[2];
  const uint32_t base = e0 & ~3u;
  if (base + 12 <= c.m * c.n) {
    const uint32_t w0 = bload32(c.rw, base), w1 = bload32(c.rw, base + 4);
    const uint32_t w2 = bload32(c.rw, base + 8);
    wb[0] = __builtin_amdgcn_alignbyte(w1, w0, e0 & 3u);
    wb[1] = __builtin_amdgcn_alignbyte(w2, w1, e0 & 3u);
  } else {
    wb[0] = wb[1] = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      wb[t >> 2] |= (bload8(c.rw, j8 + t < c.n ? e0 + t : kOOB) & 0xFFu) << (8 * (t & 3));
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const bool in = j8 + t < c.n;
    const uint32_t e = e0 + t;
    const float U = FOLD ? S[t] : mul_rn(L.alpha, S[t]);
    const float iv = (e >> 8) == g0 ? inv0 : inv1;
    const int w = (int)(int8_t)(wb[t >> 2] >> (8 * (t & 3)));
    const uint32_t bits = (t & 1) ? (words[t >> 1] >> 16) : (words[t >> 1] & 0xFFFFu);
    const float d = sr_pre(w, U, iv, bits);
    const int nw = __builtin_isfinite(d) ? sr_code(d) : w;
    bstore8(c.rw, in ? e : kOOB, (uint32_t)nw);
    if (!FOLD && c.write_u) bstoref(c.ru, in ? e * 4 : kOOB, U);
  }
}

// Write one 32-row chunk of a wave's accumulators (MFMA layout) to its LDS staging block.
template <class T, int EP>
__device__ __forceinline__ void stage_rows(float* E, const f32x16 (&accx)[T::XN]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int y = 0; y < T::XN; ++y)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      E[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * EP + 32 * y + (lane & 31)] = accx[y][v];
  __syncthreads();
}

__device__ __forceinline__ void read_run16(const float* E, int off, float (&S)[16]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 f = *reinterpret_cast<const float4*>(E + off + 4 * k);
    S[4 * k] = f.x;
    S[4 * k + 1] = f.y;
    S[4 * k + 2] = f.z;
    S[4 * k + 3] = f.w;
  }
}

__device__ __forceinline__ void read_run(const float* E, int off, float (&S)[8]) {
  const float4 f0 = *reinterpret_cast<const float4*>(E + off);
  const float4 f1 = *reinterpret_cast<const float4*>(E + off + 4);
  S[0] = f0.x; S[1] = f0.y; S[2] = f0.z; S[3] = f0.w;
  S[4] = f1.x; S[5] = f1.y; S[6] = f1.z; S[7] = f1.w;
}

// P~ rows are K-contiguous ([i][k]); N~ is K-major ([k][j]).
using BackBig = Tile<128, 256, 32, 2, 2, false, true>;
using BackSmall = Tile<128, 128, 32, 2, 2, false, true>;
static_assert(BackBig::BM == kBackTileM(true) && BackBig::BN == kBackTileN(true) &&
                  BackSmall::BM == kBackTileM(false) && BackSmall::BN == kBackTileN(false),
              "host and device back-projection tiles agree");

// The same tile in the direct-to-LDS layout (vector path).
template <class T>
using DmaOf = Tile<T::BM, T::BN, T::BK, T::WM, T::WN, T::A_KMAJOR, T::B_KMAJOR, true>;

// LDS and occupancy of a back-projection tile. The small tile (rank up to 128: a K loop of a
// few stages, time dominated by streaming W) keeps two DMA buffers, so that four workgroups
// fit on a CU and more weight traffic is in flight; the large one three.
template <class T>
struct BackLds {
  // fp32 row pitch of the redistribution block: 4 (mod 16) words, so that the 16 lanes of a
  // 16-byte read group (4 rows x 4 runs of 16 columns) hit distinct banks
  static constexpr int EP = T::WTN + 4;
  static constexpr bool SMALL = T::BN == 128;
  static constexpr int NST = SMALL ? 2 : 3;   // DMA ring buffers
  static constexpr int MINB = SMALL ? 4 : 2;  // workgroups per CU
  static constexpr int RING = NST * DmaOf<T>::STAGE * 2;   // bytes of the DMA ring
  static constexpr int BYTES = cmax(RING, kThreads / 64 * 32 * EP * 4);
  // with the INT4 stager's code areas after the ring (they share the array with the
  // epilogue, which does not use them)
  static constexpr int bytes(int pm) {
    return pm == kPStaged ? BYTES : cmax(BYTES, RING + NST * DmaInt4C<128, 32>::AREA);
  }
};

using BackCodes = DmaInt4C<128, 32>;

// Both operands are staged straight into LDS (T in the DMA layout; N~'s rows are padded to a
// multiple of 8 elements in the workspace). VEC: rows of W are a multiple of 16 elements, so
// the rounding takes 16-byte weight accesses (prefetched before the product); otherwise it
// takes byte accesses along the rows. BASE is the tile whose LDS area the kernel declares. PM
// as for the projection. FOLD: every layer of the launch has fold_alpha (alpha folded into
// the reciprocals of the rounding, U not written).
template <class T, bool VEC, class BASE, int PM, bool FOLD>
__device__ __forceinline__ void back_tile(const StepArgs& a, const LayerDev& L, int local,
                                          uint16_t* lds, uint8_t* codes) {
  static_assert(T::DMA, "operands staged by DMA");
  constexpr int EP = BackLds<BASE>::EP;
  constexpr int LPR = T::WTN / 16; // vector path: lanes per row, 16 columns each
  constexpr int RPP = 64 / LPR;    //   rows per pass of a 32-row chunk
  constexpr int NP = 32 / RPP;     //   passes per chunk
  constexpr int LPR8 = T::WTN / 8; // element path: lanes per row, 8 columns each
  constexpr int RPP8 = 64 / LPR8;  //   rows per pass
  constexpr int NP8 = 32 / RPP8;   //   passes per chunk
  // Tiles are numbered in bands of 4 row tiles, column-major inside a band: the tiles that
  // run together on one XCD (consecutive after the renumbering) cover about 4 row tiles x 8
  // column tiles, whose P~ rows and N~ columns fit in that XCD's L2 together.
  constexpr int GM = 4;
  const int band = local / (GM * L.b_tiles_j);
  const int first = band * GM;
  const int gm = min(L.b_tiles_i - first, GM);
  const int in_band = local - band * GM * L.b_tiles_j;
  const int ti = first + in_band % gm;
  const int tj = in_band / gm;
  const int i0 = ti * T::BM, j0 = tj * T::BN;

  // After the product, each wave's block goes through LDS 32 rows at a time so that lanes
  // own runs of consecutive columns of one row: whole Philox blocks and wide W accesses. On
  // the vector path a lane takes 16 columns (one 16-byte weight access, two Philox blocks)
  // and LPR lanes cover a row of the wave's block. The weights and scales a lane will need
  // do not depend on the product, so their loads are issued first and arrive while the
  // MFMAs run.
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave_m<T>(), wn = wave_n<T>();
  SrCtx c;
  c.n = (uint32_t)L.n;
  c.m = (uint32_t)L.m;
  c.write_u = (L.U_out != nullptr);
  const uint32_t numel = (uint32_t)(L.m * L.n);
  c.rw = make_rsrc(L.Wq, numel);
  c.rws = make_rsrc(L.Ws, ((numel + kGroup - 1) / kGroup) * 4);
  c.ru = make_rsrc(L.U_out, c.write_u ? numel * 4 : 0);
  const int vr = lane / LPR, vc = (lane % LPR) * 16;
  const uint32_t jw = (uint32_t)j0 + wn * T::WTN;   // the wave's first column
  const uint32_t j16 = jw + vc;
  // When rows are whole scale groups apart (n % 256 == 0), the wave's WTN columns of a row
  // lie in one group: lane l then loads the scale of the wave's row l (WTM == 64 rows) and
  // computes its reciprocal once, and each lane takes the reciprocals of its rows from the
  // lanes that hold them. Otherwise every lane loads and inverts the scale of each run.
  static_assert(!VEC || T::WTM == 64, "one wave row per lane");
  const bool row_groups = c.n % kGroup == 0 && T::WTN <= kGroup;
  uint4 wv[T::XM][NP];
  float sv[T::XM][NP];
  float s_row = 0.0f;
  if constexpr (VEC) {
    if (row_groups) {
      const uint32_t i = (uint32_t)i0 + wm * T::WTM + lane;
      s_row = bloadf(c.rws, i < c.m && jw < c.n ? ((i * c.n + jw) >> 8) * 4 : kOOB);
    }
#pragma unroll
    for (int x = 0; x < T::XM; ++x)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t i = (uint32_t)i0 + wm * T::WTM + 32 * x + RPP * p + vr;
        const uint32_t e = i * c.n + j16;
        const bool in = i < c.m && j16 < c.n;
        wv[x][p] = bload128(c.rw, in ? e : kOOB);
        sv[x][p] = row_groups ? 0.0f : bloadf(c.rws, in ? (e >> 8) * 4 : kOOB);
      }
  }

  // A = P~ (rows i, K = rank index contiguous): the INT4 codes of P dequantized on their way
  // into LDS, or the bf16 P~ (the dequant kernel's copy or the caller's bf16 P).
  // B = N~ stored [k][j] (r x n, rows ldn apart: 16-byte chunks for any n; a chunk that runs
  // past column n reads row padding, which only feeds output columns that are dropped).
  const bool inl = PM == kPInline || (PM == kPMixed && L.p_inline);
  const uint16_t* Nb = reinterpret_cast<const uint16_t*>(a.ws + L.off_n);
  f32x16 acc[T::XM][T::XN];
  const DmaBf16K<T::BN, T::BK> sb(Nb, L.ldn, L.r, L.n, j0);
  if (PM != kPStaged && inl) {
    const BackCodes sa(L.Pq, L.Ps, L.r, L.m, i0);
    gemm_kloop_dma_cvt<T, BackLds<BASE>::NST, true>(sa, sb, 0, L.r, lds, codes, acc);
  } else if (PM != kPInline) {
    const DmaBf16C<T::BM, T::BK> sa(p_tilde(a, L), L.r, L.m, i0);
    gemm_kloop_dma<T, BackLds<BASE>::NST, true>(sa, sb, 0, L.r, lds, acc);
  }

  float* E = reinterpret_cast<float*>(lds) + wave * 32 * EP;
  if constexpr (VEC) {
    const float inv_row0 = row_groups ? recip_or_zero(s_row) : 0.0f;
    const float inv_row = FOLD ? mul_rn(L.alpha, inv_row0) : inv_row0;
    const int vr4 = 4 * vr;   // ds_bpermute byte address of lane vr
#pragma clang loop unroll(full)
    for (int x = 0; x < T::XM; ++x) {
      stage_rows<T, EP>(E, acc[x]);
#pragma clang loop unroll(full)
      for (int p = 0; p < NP; ++p) {
        const int row = RPP * p + vr;
        const uint32_t i = (uint32_t)i0 + wm * T::WTM + 32 * x + row;
        // the shuffle runs on every lane (a lane whose run is off the layer only serves); its
        // byte address is the lane's own part plus a constant the instruction's offset holds
        float inv;
        if (row_groups) {
          inv = __int_as_float(__builtin_amdgcn_ds_bpermute(
              vr4 + 4 * (32 * x + RPP * p), __float_as_int(inv_row)));
        } else {
          inv = recip_or_zero(sv[x][p]);
          if (FOLD) inv = mul_rn(L.alpha, inv);
        }
        if (i < c.m && j16 < c.n) {
          float S[16];
          read_run16(E, row * EP + vc, S);
          sr_block16<FOLD>(c, L, a, i, j16, S, inv, wv[x][p]);
        }
      }
      __syncthreads();
    }
  } else {
    // lanes along a row, 8 columns each, so that each byte access of the wave covers a few
    // rows' contiguous runs
    const int vr8 = lane / LPR8, vc8 = (lane % LPR8) * 8;
    const uint32_t j8 = jw + vc8;
#pragma clang loop unroll(full)
    for (int x = 0; x < T::XM; ++x) {
      stage_rows<T, EP>(E, acc[x]);
#pragma clang loop unroll(full)
      for (int p = 0; p < NP8; ++p) {
        const int row = RPP8 * p + vr8;
        const uint32_t i = (uint32_t)i0 + wm * T::WTM + 32 * x + row;
        if (i < c.m && j8 < c.n) {
          float S[8];
          read_run(E, row * EP + vc8, S);
          sr_block8_elem<FOLD>(c, L, a, i, j8, S);
        }
      }
      __syncthreads();
    }
  }
}

// The large tile is held to 256 registers per lane: two workgroups per CU (two waves per
// SIMD) hide the load latency better than more registers in one. The small one to 128.
template <class T, int PM, bool FOLD>
__global__ __launch_bounds__(kThreads, BackLds<T>::MINB) void qg_backproject(StepArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[BackLds<T>::bytes(PM) / 2];
  uint8_t* codes = reinterpret_cast<uint8_t*>(lds) + BackLds<T>::RING;
  int local;
  const LayerDev L = fetch_layer(a, KBACK, xcd_remap(blockIdx.x, gridDim.x), local);
  if (L.n % 16 == 0)
    back_tile<DmaOf<T>, true, T, PM, FOLD>(a, L, local, lds, codes);
  else
    back_tile<DmaOf<T>, false, T, PM, FOLD>(a, L, local, lds, codes);
}

// ================================================================ quantization of P ===
// Symmetric absmax over groups of 256 flat elements: one wave per group, 4 elements a lane.

__global__ __launch_bounds__(kThreads) void qg_quantize_int4(const float* P, int64_t numel,
                                                            uint8_t* Pq, float* Ps) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t ngroups = (numel + kGroup - 1) / kGroup;
  if (g >= ngroups) return;
  const int64_t e0 = g * kGroup + 4 * lane;
  float x[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) x[t] = (e0 + t < numel) ? P[e0 + t] : 0.0f;
  float am = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  am = wave_max(am);
  const float s = div_rn(am, 7.0f);
  const float inv = recip_or_zero(s);
  uint32_t nib = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int q = (int)fminf(fmaxf(rintf(mul_rn(x[t], inv)), -7.f), 7.f);
    nib |= (uint32_t)(q & 0xF) << (4 * t);
  }
  if (e0 + 4 <= numel) {
    *reinterpret_cast<uint16_t*>(Pq + (e0 >> 1)) = (uint16_t)nib;
  } else if (e0 < numel) {
    Pq[e0 >> 1] = (uint8_t)(nib & 0xFF);
    if (e0 + 2 < numel) Pq[(e0 >> 1) + 1] = (uint8_t)(nib >> 8);
  }
  if (lane == 0) Ps[g] = s;
}

__global__ __launch_bounds__(kThreads) void qg_quantize_int8(const float* P, int64_t numel,
                                                            int8_t* Pq, float* Ps) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t ngroups = (numel + kGroup - 1) / kGroup;
  if (g >= ngroups) return;
  const int64_t e0 = g * kGroup + 4 * lane;
  float x[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) x[t] = (e0 + t < numel) ? P[e0 + t] : 0.0f;
  float am = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  am = wave_max(am);
  const float s = div_rn(am, 127.0f);
  const float inv = recip_or_zero(s);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (e0 + t < numel) Pq[e0 + t] = (int8_t)fminf(fmaxf(rintf(mul_rn(x[t], inv)), -127.f), 127.f);
  if (lane == 0) Ps[g] = s;
}

// ==================================================================== launchers ===

hipError_t launch_project(const StepArgs& a, int grid, int pmode, hipStream_t s) {
  if (pmode == kPInline)
    hipLaunchKernelGGL(qg_project<kPInline>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (pmode == kPMixed)
    hipLaunchKernelGGL(qg_project<kPMixed>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(qg_project<kPStaged>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_dequant(const StepArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(qg_dequant, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_adam(const StepArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(qg_adam, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
template <class T, bool FOLD>
static void launch_back_t(const StepArgs& a, int grid, int pmode, hipStream_t s) {
  if (pmode == kPInline)
    hipLaunchKernelGGL((qg_backproject<T, kPInline, FOLD>), dim3(grid), dim3(kThreads), 0, s, a);
  else if (pmode == kPMixed)
    hipLaunchKernelGGL((qg_backproject<T, kPMixed, FOLD>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((qg_backproject<T, kPStaged, FOLD>), dim3(grid), dim3(kThreads), 0, s, a);
}
hipError_t launch_backproject(const StepArgs& a, int grid, bool big, int pmode, bool fold,
                              hipStream_t s) {
  if (big)
    fold ? launch_back_t<BackBig, true>(a, grid, pmode, s)
         : launch_back_t<BackBig, false>(a, grid, pmode, s);
  else
    fold ? launch_back_t<BackSmall, true>(a, grid, pmode, s)
         : launch_back_t<BackSmall, false>(a, grid, pmode, s);
  return hipGetLastError();
}
hipError_t launch_quantize_int4(const float* P, int64_t numel, uint8_t* Pq, float* Ps,
                                hipStream_t s) {
  const int64_t groups = (numel + kGroup - 1) / kGroup;
  const int grid = (int)((groups + 3) / 4);
  hipLaunchKernelGGL(qg_quantize_int4, dim3(grid), dim3(kThreads), 0, s, P, numel, Pq, Ps);
  return hipGetLastError();
}
hipError_t launch_quantize_int8(const float* P, int64_t numel, int8_t* Pq, float* Ps,
                                hipStream_t s) {
  const int64_t groups = (numel + kGroup - 1) / kGroup;
  const int grid = (int)((groups + 3) / 4);
  hipLaunchKernelGGL(qg_quantize_int8, dim3(grid), dim3(kThreads), 0, s, P, numel, Pq, Ps);
  return hipGetLastError();
}

}  // namespace qg
