// MFMA tile machinery shared by the projection (R = P~^T G), back-projection (U = P~ N~)
// and subspace-similarity (C = P~_new^T P~_old) kernels.
//
// Workgroup tile 128 x 128 over the output, K consumed 32 at a time, 4 waves in a 2 x 2
// arrangement, each wave owning a 64 x 64 sub-tile as 2 x 2 v_mfma_f32_32x32x16_bf16 blocks.
// Both operands live in LDS "k-contiguous": row c of the tile holds its 32 K values, so an
// MFMA lane reads its 8 consecutive K values with one 16-byte LDS read. Sources whose K index
// is the slow (row) index in memory -- the gradient G, the update N~ and the projection when
// it is used transposed -- are transposed while being written to LDS; the INT4 dequant
// (code * group scale, then bf16 rounding) happens in the same step, so P~ never exists in HBM.
#pragma once

#include "qg_device.hpp"

namespace qg {

constexpr int TM = 128;             // output tile rows (MFMA "A" side)
constexpr int TN = 128;             // output tile cols (MFMA "B" side)
constexpr int TK = 32;              // K per stage
constexpr int LDK = TK + 8;         // LDS row pitch in bf16 (80 bytes: keeps 16-byte reads aligned)
constexpr int STAGE_ELEMS = (TM + TN) * LDK;
constexpr int LDS_ELEMS = 2 * STAGE_ELEMS;   // double-buffered: 40 KiB

// ---------------------------------------------------------------------------------------
// bf16 source stored [k][c] (row pitch ld), tile columns [c0, c0+128), written to LDS [c][k].
// Thread t stages rows k+2p, k+2p+1 (p = t / 16) and columns c0 + 8*(t % 16) .. +7.
// ---------------------------------------------------------------------------------------
struct StageBf16T {
  const uint16_t* src;
  int64_t ld, k_end, c_end;
  int c;            // first column this thread stages
  int kp;           // row pair
  bool vec_ok;      // 16-byte loads possible for in-bounds rows
  uint4 v[2];

  __device__ StageBf16T(const uint16_t* s, int64_t ld_, int64_t k_end_, int64_t c_end_, int c0)
      : src(s), ld(ld_), k_end(k_end_), c_end(c_end_) {
    const int t = threadIdx.x;
    kp = t >> 4;
    c = c0 + 8 * (t & 15);
    vec_ok = (ld % 8 == 0) && (c + 8 <= c_end);
  }

  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t k = k0 + 2 * kp + rr;
      if (k < k_end && vec_ok) {
        v[rr] = gload(reinterpret_cast<const uint4*>(src + k * ld + c));
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
        if (k < k_end) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c + e < c_end) w[e >> 1] |= (uint32_t)gload(src + k * ld + c + e) << (16 * (e & 1));
        }
        v[rr] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  // Transpose the 2 x 8 block into 8 dwords (k, k+1) and write them to LDS [c][k].
  __device__ __forceinline__ void store(uint16_t* lds, int c0) const {
    uint32_t* d = reinterpret_cast<uint32_t*>(lds);
    const int cl = c - c0;
    const uint32_t a[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
    const uint32_t b[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
      d[(cl + cc) * (LDK / 2) + kp] = __builtin_amdgcn_perm(b[cc >> 1], a[cc >> 1], sel);
    }
  }
};

// ---------------------------------------------------------------------------------------
// INT4 source stored [k][c] (row pitch ld codes, ld % 8 == 0), dequantized and written to LDS
// [c][k]. Same thread mapping as StageBf16T. A run of 8 codes starting at a multiple of 8 in
// the flat index lies inside one 256-element scale group, and since ld % 8 == 0 it is either
// wholly inside the tile or wholly outside (then it stages zeros).
// ---------------------------------------------------------------------------------------
struct StageInt4T {
  const uint8_t* q;
  const float* sc;
  int64_t ld, k_end, c_end;
  int c, kp;
  uint32_t w[2];
  float s[2];

  __device__ StageInt4T(const uint8_t* q_, const float* sc_, int64_t ld_, int64_t k_end_,
                        int64_t c_end_, int c0)
      : q(q_), sc(sc_), ld(ld_), k_end(k_end_), c_end(c_end_) {
    const int t = threadIdx.x;
    kp = t >> 4;
    c = c0 + 8 * (t & 15);
  }

  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t k = k0 + 2 * kp + rr;
      w[rr] = 0u;
      s[rr] = 0.0f;
      if (k < k_end && c < c_end) {
        const int64_t e = k * ld + c;
        w[rr] = gload(reinterpret_cast<const uint32_t*>(q + (e >> 1)));
        s[rr] = gload(sc + (e >> 8));
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int c0) const {
    uint32_t* d = reinterpret_cast<uint32_t*>(lds);
    const int cl = c - c0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const float f0 = mul_rn((float)nibble(w[0], cc), s[0]);
      const float f1 = mul_rn((float)nibble(w[1], cc), s[1]);
      d[(cl + cc) * (LDK / 2) + kp] = pack_bf16x2(f0, f1);
    }
  }
};

// ---------------------------------------------------------------------------------------
// INT4 source stored [c][k] (row pitch ld codes, K contiguous, ld % 8 == 0), tile rows
// [c0, c0+128), dequantized and written to LDS [c][k] without transposition. Thread t stages
// two runs: row (t / 4) + 64*h, codes k0 + 8*(t % 4) .. +7, h = 0, 1.
// ---------------------------------------------------------------------------------------
struct StageInt4N {
  const uint8_t* q;
  const float* sc;
  int64_t ld, c_end;   // ld = K extent (codes per row)
  int c0;
  uint32_t w[2];
  float s[2];

  __device__ StageInt4N(const uint8_t* q_, const float* sc_, int64_t ld_, int64_t c_end_, int c0_)
      : q(q_), sc(sc_), ld(ld_), c_end(c_end_), c0(c0_) {}

  __device__ __forceinline__ void load(int64_t k0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t row = c0 + (t >> 2) + 64 * h;
      const int64_t k = k0 + 8 * (t & 3);
      w[h] = 0u;
      s[h] = 0.0f;
      if (row < c_end && k < ld) {
        const int64_t e = row * ld + k;
        w[h] = gload(reinterpret_cast<const uint32_t*>(q + (e >> 1)));
        s[h] = gload(sc + (e >> 8));
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float f[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) f[u] = mul_rn((float)nibble(w[h], u), s[h]);
      const int rl = (t >> 2) + 64 * h;
      const uint4 pk = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                  pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
      *reinterpret_cast<uint4*>(lds + rl * LDK + 8 * (t & 3)) = pk;
    }
  }
};

// ---------------------------------------------------------------------------------------
// The K loop: acc[x][y] (wave sub-tile rows 32*x, cols 32*y) += A_tile * B_tile over K in
// [k_begin, k_end). A stage holds PARTS copies of the [A | B] tile pair: PARTS = 1 is the
// plain bf16 product; PARTS = 2 holds the bf16 "high" parts followed by the bf16 "low"
// remainders of fp32 operands, and the product keeps hi*hi + hi*lo + lo*hi (about 16
// significant bits per operand). store_a(sa, stage) / store_b(sb, stage) fill one stage.
// ---------------------------------------------------------------------------------------
template <int PARTS>
__device__ __forceinline__ void mfma_stage(const uint16_t* stage, f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hk = (lane >> 5) * 8;
  const uint16_t* As = stage;
  const uint16_t* Bs = stage + TM * LDK;
#pragma unroll
  for (int ks = 0; ks < TK; ks += 16) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      a[x] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + 32 * x + l32) * LDK + ks + hk);
      b[x] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + 32 * x + l32) * LDK + ks + hk);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], b[y], acc[x][y], 0, 0, 0);
    if constexpr (PARTS == 2) {
      const uint16_t* Al = stage + STAGE_ELEMS;
      const uint16_t* Bl = Al + TM * LDK;
      bf16x8 al[2], bl[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        al[x] = *reinterpret_cast<const bf16x8*>(Al + (wm * 64 + 32 * x + l32) * LDK + ks + hk);
        bl[x] = *reinterpret_cast<const bf16x8*>(Bl + (wn * 64 + 32 * x + l32) * LDK + ks + hk);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], bl[y], acc[x][y], 0, 0, 0);
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[x], b[y], acc[x][y], 0, 0, 0);
        }
    }
  }
}

template <int PARTS, class SA, class SB, class StoreA, class StoreB>
__device__ __forceinline__ void gemm_kloop(SA& sa, SB& sb, StoreA store_a, StoreB store_b,
                                           int64_t k_begin, int64_t k_end, uint16_t* lds,
                                           f32x16 (&acc)[2][2]) {
  constexpr int STAGE = PARTS * STAGE_ELEMS;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
  if (k_end <= k_begin) return;
  const int nk = (int)((k_end - k_begin + TK - 1) / TK);
  sa.load(k_begin);
  sb.load(k_begin);
  store_a(sa, lds);
  store_b(sb, lds);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      sa.load(k_begin + (int64_t)(kt + 1) * TK);
      sb.load(k_begin + (int64_t)(kt + 1) * TK);
    }
    uint16_t* now = lds + cur * STAGE;
    uint16_t* nxt = lds + (cur ^ 1) * STAGE;
    mfma_stage<PARTS>(now, acc);
    if (more) {
      store_a(sa, nxt);
      store_b(sb, nxt);
    }
    __syncthreads();
  }
}

// Output coordinates of accumulator element v of block (x, y) for this lane, relative to the
// workgroup tile: row = wm*64 + 32x + 8*(v/4) + 4*(lane/32) + v%4, col = wn*64 + 32y + lane%32.
__device__ __forceinline__ int acc_row(int x, int v) {
  const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) >> 1;
  return wm * 64 + 32 * x + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int acc_col(int y) {
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
  return wn * 64 + 32 * y + (lane & 31);
}

}  // namespace qg
