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

constexpr int cmax_i_(int a, int b) { return a > b ? a : b; }

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

// Dequantize 8 INT8 codes (two little-endian words) with their group scale: bf16(fl(q * s)).
__device__ __forceinline__ uint4 dequant8_int8(uint2 w, float s) {
  float f[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = mul_rn((float)(int8_t)(w.x >> (8 * e)), s);
    f[4 + e] = mul_rn((float)(int8_t)(w.y >> (8 * e)), s);
  }
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// ---------------------------------------------------------------------------------------
// The INT8 weight as the first MFMA operand, staged by LDS DMA and converted in LDS (the
// machinery of the INT4 projection stagers): per K stage the codes of the tile's 128 weight
// rows or columns and one group scale per tile row reach a code area by DMA; convert() then
// writes the bf16 tile. The weight is the 128-edge of the tile and the tokens the 256-edge,
// so each weight element is converted once per 256 tokens.
// ---------------------------------------------------------------------------------------

// W [o][i] read by rows (forward: tile rows o, K = i = n codes per row, n % 32 == 0 so that
// a row's 32 codes of a stage lie in one group). K-contiguous tile [128][32] (kc_off).
struct DmaInt8C {
  static constexpr int W = 128, BK = 32;
  static constexpr int ROWB = BK;                  // code bytes per tile row and stage
  static constexpr int CODE_BYTES = W * ROWB;      // 4 KiB
  static constexpr int AREA = CODE_BYTES + 4 * W;  // + the row scales
  static constexpr int RPI = 1024 / ROWB;          // tile rows per 16-byte wave-level load
  static constexpr int NI = W / (4 * RPI);         // code loads per wave and stage (one)
  static constexpr int NV = NI + 1;
  static_assert(NI * 4 * RPI == W, "a stage splits evenly over the four waves");
  const int8_t* q;
  v4i32 rsc;
  uint32_t ld, c_end, c0;
  uint32_t vo[NI];

  __device__ DmaInt8C(const int8_t* q_, const float* sc_, int64_t ld_, int64_t c_end_, int c0_)
      : q(q_), ld((uint32_t)ld_), c_end((uint32_t)c_end_), c0((uint32_t)c0_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    rsc = rsrc_words(sc_, (uint32_t)(((c_end_ * ld_ + kGroup - 1) / kGroup) * 4));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t rg = c0 + (wave * NI + i) * RPI + lane / (ROWB / 16);
      vo[i] = rg < c_end ? rg * ld + 16 * (lane % (ROWB / 16)) : kOOB;
    }
  }

  __device__ __forceinline__ void issue(int64_t k0_, uint32_t area) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t k0 = (uint32_t)k0_ < ld ? (uint32_t)k0_ : ld;
    const v4i32 st = rsrc_words(q + k0, c_end * ld - k0);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(st, vo[i], area + (wave * NI + i) * 1024);
    if ((lane >> 5) == (wave & 1)) {   // tile rows 64 (w / 2) + lane
      const uint32_t rg = c0 + 64 * (wave >> 1) + lane;
      const uint32_t off = rg < c_end ? ((rg * ld + k0) >> 8) * 4 : kOOB;
      dma4(rsc, off, area + CODE_BYTES + 256 * (wave >> 1));
    }
  }

  // thread t: chunk t % 4 of tile rows t / 4 and t / 4 + 64
  __device__ __forceinline__ void convert(const uint8_t* area, uint16_t* tile) const {
    const int c = threadIdx.x % 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = threadIdx.x / 4 + 64 * h;
      const uint2 w = *reinterpret_cast<const uint2*>(area + row * ROWB + 8 * c);
      const float sc = *reinterpret_cast<const float*>(area + CODE_BYTES + 4 * row);
      *reinterpret_cast<uint4*>(tile + kc_off(row, c)) = dequant8_int8(w, sc);
    }
  }
};

// The forward product for n % 128 == 0 (every LLaMA shape), in stages of 64 K values: both
// operands are K-contiguous, and a stage of 32 reads only 64 bytes of each activation row and
// 32 of each weight row, so that a wave-level load touches 16 or 32 cache lines and waits
// long for them (counters: the same instruction mix as the data gradient's, 50% more wait
// cycles). Here the activation rows come as full 128-byte lines (tile [256][64] bf16,
// 16-byte chunk c of row r at slot c ^ ((r / 2) % 8)) and the weight codes as 64-byte halves
// (area [128][64], chunk c of row r at slot c ^ ((r / 4) % 4)); the swizzles keep the
// fragment reads of 16 (bf16) or 32 (codes) consecutive rows on distinct banks. Each wave
// dequantizes its own A fragments from the codes straight into registers, bf16(fl(q s)) with
// the row's group scale held in a register (a 64-code run starting at a multiple of 64 of
// the flat index lies in one 256-element group). Two buffers of each operand (80 KiB, two
// workgroups per CU); every stage issues the next stage's codes, scales and activations after
// its barrier, so waiting for the current stage needs nothing else in flight.
struct Fwd64 {
  static constexpr int BK = 64;
  static constexpr int BROWS = 256, WROWS = 128;
  static constexpr int B_BYTES = BROWS * BK * 2;    // 32 KiB
  static constexpr int C_BYTES = WROWS * BK;        // 8 KiB
  static constexpr int NIB = B_BYTES / 1024 / 4;    // activation loads per wave (eight)
  static constexpr int NIC = C_BYTES / 1024 / 4;    // code loads per wave (two)
  const uint16_t* act;
  const int8_t* q;
  rsrc_t rsc;
  uint32_t ld, t_end, m_end, w0;
  uint32_t vb[NIB], vc[NIC];

  __device__ Fwd64(const uint16_t* act_, const int8_t* q_, const float* sc_, int64_t ld_,
                   int64_t t_end_, int64_t m_end_, int t0, int w0_)
      : act(act_), q(q_), ld((uint32_t)ld_), t_end((uint32_t)t_end_), m_end((uint32_t)m_end_),
        w0((uint32_t)w0_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    rsc = make_rsrc(sc_, (uint32_t)(((m_end_ * ld_ + kGroup - 1) / kGroup) * 4));
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
      const int row = 8 * (NIB * wave + i) + lane / 8;
      const int chunk = (lane % 8) ^ ((row >> 1) & 7);
      const uint32_t rg = t0 + row;
      vb[i] = rg < t_end ? (rg * ld + 8 * chunk) * 2 : kOOB;
    }
#pragma unroll
    for (int i = 0; i < NIC; ++i) {
      const int row = 16 * (NIC * wave + i) + lane / 4;
      const int chunk = (lane % 4) ^ ((row >> 2) & 3);
      const uint32_t rg = w0 + row;
      vc[i] = rg < m_end ? rg * ld + 16 * chunk : kOOB;
    }
  }

  __device__ __forceinline__ void issue(int64_t k0_, uint32_t btile, uint32_t carea) const {
    const int wave = threadIdx.x >> 6;
    const uint32_t k0 = (uint32_t)k0_;
    const v4i32 sq = rsrc_words(q + k0, m_end * ld - k0);
#pragma unroll
    for (int i = 0; i < NIC; ++i) dma16(sq, vc[i], carea + (NIC * wave + i) * 1024);
    const v4i32 sa = rsrc_words(act + k0, (t_end * ld - k0) * 2);
#pragma unroll
    for (int i = 0; i < NIB; ++i) dma16(sa, vb[i], btile + (NIB * wave + i) * 1024);
  }
  __device__ __forceinline__ float scale(int row, int64_t k0) const {
    const uint32_t rg = w0 + row;
    return bloadf(rsc, rg < m_end ? ((rg * ld + (uint32_t)k0) >> 8) * 4 : kOOB);
  }
  // bf16 of K values kk .. kk + 7 of weight row `row` (kk a multiple of 8)
  __device__ __forceinline__ bf16x8 afrag(const uint8_t* area, int row, int kk, float s) const {
    const int off = row * BK + 16 * ((kk >> 4) ^ ((row >> 2) & 3)) + 8 * ((kk >> 3) & 1);
    return __builtin_bit_cast(bf16x8, dequant8_int8(*reinterpret_cast<const uint2*>(area + off), s));
  }
  // K values kk .. kk + 7 of activation row `row`
  __device__ __forceinline__ bf16x8 bfrag(const uint16_t* tile, int row, int kk) const {
    return *reinterpret_cast<const bf16x8*>(tile + row * BK + 8 * ((kk >> 3) ^ ((row >> 1) & 7)));
  }
};

template <class T>
__device__ __forceinline__ void gemm_kloop_fwd64(const Fwd64& st, int64_t K, uint16_t* lds,
                                                 f32x16 (&acc)[T::XM][T::XN]) {
  static_assert(T::BM == Fwd64::WROWS && T::BN == Fwd64::BROWS, "tile edges");
  constexpr int BK = Fwd64::BK;
  const int lane = threadIdx.x & 63;
  const int am = wave_m<T>() * T::WTM, bn = wave_n<T>() * T::WTN;
#pragma unroll
  for (int x = 0; x < T::XM; ++x)
#pragma unroll
    for (int y = 0; y < T::XN; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
  const int nk = (int)(K / BK);
  if (nk <= 0) return;
  uint8_t* codes = reinterpret_cast<uint8_t*>(lds) + 2 * Fwd64::B_BYTES;
  const uint32_t base = lds_addr(lds);
  const uint32_t cbase = lds_addr(reinterpret_cast<const uint16_t*>(codes));
  float sc_next[T::XM], sc[T::XM];
#pragma unroll
  for (int x = 0; x < T::XM; ++x) sc_next[x] = st.scale(am + 32 * x + (lane & 31), 0);
  st.issue(0, base, cbase);
  for (int k0 = 0; k0 < nk; k0 += 2) {
    static_for<2>([&](auto dc) {
      constexpr int buf = decltype(dc)::value;
      const int j = k0 + buf;
      if (j < nk) {
        wait_vm_lds<0>();
        barrier_nofence();
#pragma unroll
        for (int x = 0; x < T::XM; ++x) sc[x] = sc_next[x];
        if (j + 1 < nk) {
          const int64_t kn = (int64_t)(j + 1) * BK;
#pragma unroll
          for (int x = 0; x < T::XM; ++x) sc_next[x] = st.scale(am + 32 * x + (lane & 31), kn);
          st.issue(kn, base + (buf ^ 1) * Fwd64::B_BYTES, cbase + (buf ^ 1) * Fwd64::C_BYTES);
        }
        const uint16_t* Bs = lds + buf * (Fwd64::B_BYTES / 2);
        const uint8_t* area = codes + buf * Fwd64::C_BYTES;
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
          bf16x8 a[T::XM], b[T::XN];
#pragma unroll
          for (int x = 0; x < T::XM; ++x)
            a[x] = st.afrag(area, am + 32 * x + (lane & 31), ks + 8 * (lane >> 5), sc[x]);
#pragma unroll
          for (int y = 0; y < T::XN; ++y)
            b[y] = st.bfrag(Bs, bn + 32 * y + (lane & 31), ks + 8 * (lane >> 5));
#pragma unroll
          for (int x = 0; x < T::XM; ++x)
#pragma unroll
            for (int y = 0; y < T::XN; ++y)
              acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], b[y], acc[x][y], 0, 0, 0);
        }
      }
    });
  }
  __syncthreads();
}

// W [o][i] read by columns (data gradient: tile rows are K = o, tile columns i0 .. i0 + 127;
// n % 128 == 0, so that a row's 128 codes lie in one group). K-major tile [32][128]
// (kmaj_slot layout).
struct DmaInt8K {
  static constexpr int W = 128, BK = 32;
  static constexpr int ROWB = W;                   // code bytes per tile row
  static constexpr int CODE_BYTES = BK * ROWB;     // 4 KiB
  static constexpr int AREA = CODE_BYTES + 256;    // + the BK row scales
  static constexpr int RPI = 1024 / ROWB;          // tile rows per 16-byte wave-level load
  static constexpr int NI = BK / (4 * RPI);        // code loads per wave and stage (one)
  static constexpr int NV = NI + 1;
  static_assert(NI * 4 * RPI == BK, "a stage splits evenly over the four waves");
  const int8_t* q;
  v4i32 rsc;
  uint32_t ld, k_end, c0;
  uint32_t vo[NI];

  __device__ DmaInt8K(const int8_t* q_, const float* sc_, int64_t ld_, int64_t rows,
                      int64_t k_end_, int c0_)
      : q(q_), ld((uint32_t)ld_), k_end((uint32_t)k_end_), c0((uint32_t)c0_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    rsc = rsrc_words(sc_, (uint32_t)(((rows * ld_ + kGroup - 1) / kGroup) * 4));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t row = (wave * NI + i) * RPI + lane / (ROWB / 16);
      const uint32_t col = c0 + 16 * (lane % (ROWB / 16));
      vo[i] = col < ld ? row * ld + col : kOOB;
    }
  }

  __device__ __forceinline__ void issue(int64_t k0_, uint32_t area) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t k0 = (uint32_t)k0_ < k_end ? (uint32_t)k0_ : k_end;
    const v4i32 st = rsrc_words(q + (size_t)k0 * ld, (k_end - k0) * ld);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(st, vo[i], area + (wave * NI + i) * 1024);
    if (lane >= 8 * wave && lane < 8 * wave + 8) {   // tile rows 8 w .. 8 w + 7
      const uint32_t k = k0 + lane;
      const uint32_t off = k < k_end ? ((k * ld + c0) >> 8) * 4 : kOOB;
      dma4(rsc, off, area + CODE_BYTES);
    }
  }

  // thread t: chunk t % 16 of tile rows t / 16 and t / 16 + 16
  __device__ __forceinline__ void convert(const uint8_t* area, uint16_t* tile) const {
    const int c = threadIdx.x % 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = threadIdx.x / 16 + 16 * h;
      const uint2 w = *reinterpret_cast<const uint2*>(area + row * ROWB + 8 * c);
      const float sc = *reinterpret_cast<const float*>(area + CODE_BYTES + 4 * row);
      *reinterpret_cast<uint4*>(tile + row * W + 8 * kmaj_slot<W>(row, c)) =
          dequant8_int8(w, sc);
    }
  }
};

// Tiles of the DMA products: weight side 128 (M), tokens 256 (N, K-contiguous rows of the
// activation). Forward: A = W rows (K-contiguous); data gradient: A = W^T (K-major).
using LinFwdTileD = Tile<128, 256, 32, 2, 2, false, false, true>;
using LinBwdDataTileD = Tile<128, 256, 32, 2, 2, true, false, true>;
constexpr int kLinNst = 2;   // LDS ring depth of the DMA products (two workgroups per CU)

// Writes the accumulator tile (rows: weight side, columns: tokens) transposed into out
// (tokens x ld, row-major bf16): each wave rounds its 64 x 128 block to bf16 in LDS 32 rows
// at a time, then stores 16-byte runs of one token's outputs. Positions past the matrix are
// dropped by the buffer range.
template <class T>
__device__ __forceinline__ void store_bf16_transposed(uint16_t* out, int64_t tokens, int64_t ld,
                                                      int64_t wcols, int i0, int j0,
                                                      const f32x16 (&acc)[T::XM][T::XN],
                                                      uint16_t* lds) {
  constexpr int PI = 40;   // bf16 pitch of a token row of the staging block (32 + 8)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave_m<T>(), wn = wave_n<T>();
  uint16_t* E = lds + wave * (T::WTN * PI);
  const rsrc_t ro = make_rsrc(out, (uint32_t)(tokens * ld * 2));
#pragma unroll
  for (int x = 0; x < T::XM; ++x) {
#pragma unroll
    for (int y = 0; y < T::XN; ++y)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int jl = 32 * y + (lane & 31);
        const int il = 8 * qd + 4 * (lane >> 5);
        *reinterpret_cast<uint2*>(E + jl * PI + il) =
            make_uint2(pack_bf16x2(acc[x][y][4 * qd], acc[x][y][4 * qd + 1]),
                       pack_bf16x2(acc[x][y][4 * qd + 2], acc[x][y][4 * qd + 3]));
      }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < T::WTN * 4 / 64; ++c) {
      const int q = c * 64 + lane;
      const int jl = q / 4, ic = q % 4;
      const uint32_t j = (uint32_t)(j0 + wn * T::WTN + jl);
      const uint32_t i = (uint32_t)(i0 + wm * T::WTM + 32 * x + 8 * ic);
      const uint4 v = *reinterpret_cast<const uint4*>(E + jl * PI + 8 * ic);
      bstore128(ro, (j < (uint32_t)tokens && i < (uint32_t)wcols) ? (j * (uint32_t)ld + i) * 2
                                                                   : kOOB, v);
    }
    __syncthreads();
  }
}

constexpr int lin_dma_lds_bytes() {
  return cmax_i_(cmax_i_(kLinNst * LinFwdTileD::STAGE * 2 + kLinNst * DmaInt8C::AREA,
                         kLinNst * LinBwdDataTileD::STAGE * 2 + kLinNst * DmaInt8K::AREA),
                 4 * LinFwdTileD::WTN * 40 * 2);
}

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

// Forward by DMA (n % 32 == 0): the tile is Y^T (weight rows o x tokens t) = W~ X^T.
__global__ __launch_bounds__(kThreads, 2) void qg_lin_fwd_dma(LinArgs a) {
  using T = LinFwdTileD;
  __shared__ __attribute__((aligned(16))) uint16_t lds[lin_dma_lds_bytes() / 2];
  uint8_t* codes = reinterpret_cast<uint8_t*>(lds) + kLinNst * T::STAGE * 2;
  const int local = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles_m = (int)((a.m + T::BM - 1) / T::BM);
  const int i0 = (local % tiles_m) * T::BM, j0 = (local / tiles_m) * T::BN;
  const DmaInt8C sa(a.Wq, a.Ws, a.n, a.m, i0);
  const DmaBf16C<T::BN, T::BK> sb(a.act, a.n, a.T, j0);
  f32x16 acc[T::XM][T::XN];
  gemm_kloop_dma_cvt<T, kLinNst>(sa, sb, 0, a.n, lds, codes, acc);
  store_bf16_transposed<T>(a.out, a.T, a.m, a.m, i0, j0, acc, lds);
}

// Forward by 64-K stages (n % 128 == 0): the tile is Y^T (weight rows o x tokens t) = W~ X^T.
constexpr int lin_fwd64_lds_bytes() {
  return cmax_i_(2 * Fwd64::B_BYTES + 2 * Fwd64::C_BYTES, 4 * LinFwdTileD::WTN * 40 * 2);
}
static_assert(lin_fwd64_lds_bytes() <= 80 * 1024, "two workgroups per CU");

__global__ __launch_bounds__(kThreads, 2) void qg_lin_fwd64(LinArgs a) {
  using T = LinFwdTileD;
  __shared__ __attribute__((aligned(16))) uint16_t lds[lin_fwd64_lds_bytes() / 2];
  const int local = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles_m = (int)((a.m + T::BM - 1) / T::BM);
  const int i0 = (local % tiles_m) * T::BM, j0 = (local / tiles_m) * T::BN;
  const Fwd64 st(a.act, a.Wq, a.Ws, a.n, a.T, a.m, j0, i0);
  f32x16 acc[T::XM][T::XN];
  gemm_kloop_fwd64<T>(st, a.n, lds, acc);
  store_bf16_transposed<T>(a.out, a.T, a.m, a.m, i0, j0, acc, lds);
}

// Data gradient by DMA (n % 128 == 0): the tile is dX^T (inputs i x tokens t) = W~^T dY^T.
__global__ __launch_bounds__(kThreads, 2) void qg_lin_bwd_data_dma(LinArgs a) {
  using T = LinBwdDataTileD;
  __shared__ __attribute__((aligned(16))) uint16_t lds[lin_dma_lds_bytes() / 2];
  uint8_t* codes = reinterpret_cast<uint8_t*>(lds) + kLinNst * T::STAGE * 2;
  const int local = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles_m = (int)((a.n + T::BM - 1) / T::BM);
  const int i0 = (local % tiles_m) * T::BM, j0 = (local / tiles_m) * T::BN;
  const DmaInt8K sa(a.Wq, a.Ws, a.n, a.m, a.m, i0);
  const DmaBf16C<T::BN, T::BK> sb(a.act, a.m, a.T, j0);
  f32x16 acc[T::XM][T::XN];
  gemm_kloop_dma_cvt<T, kLinNst>(sa, sb, 0, a.m, lds, codes, acc);
  store_bf16_transposed<T>(a.out, a.T, a.n, a.n, i0, j0, acc, lds);
}

hipError_t launch_linear(const LinArgs& a, int which, hipStream_t s) {
  const int64_t tm = (which == kLinBwdWeight ? a.m : a.T);
  const int64_t tn = (which == kLinFwd ? a.m : a.n);
  const int grid = (int)(((tm + kLinTileM - 1) / kLinTileM) * ((tn + kLinTileN - 1) / kLinTileN));
  // weight side 128 x tokens 256 tiles for the DMA forward and data-gradient kernels
  const int64_t wside = which == kLinFwd ? a.m : a.n;
  const int grid_dma =
      (int)(((wside + kLinTileM - 1) / kLinTileM) * ((a.T + kLinTileN - 1) / kLinTileN));
  if (which == kLinFwd && lin_fwd_rows(a.n))
    hipLaunchKernelGGL(qg_lin_fwd64, dim3(grid_dma), dim3(kThreads), 0, s, a);
  else if (which == kLinFwd && lin_fwd_dma(a.n))
    hipLaunchKernelGGL(qg_lin_fwd_dma, dim3(grid_dma), dim3(kThreads), 0, s, a);
  else if (which == kLinFwd)
    hipLaunchKernelGGL(qg_lin_fwd, dim3(grid), dim3(kThreads), 0, s, a);
  else if (which == kLinBwdData && lin_bwd_data_dma(a.n))
    hipLaunchKernelGGL(qg_lin_bwd_data_dma, dim3(grid_dma), dim3(kThreads), 0, s, a);
  else if (which == kLinBwdData)
    hipLaunchKernelGGL(qg_lin_bwd_data, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(qg_lin_bwd_weight, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qg
