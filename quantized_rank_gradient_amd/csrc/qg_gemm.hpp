// MFMA tile machinery shared by the projection (R = P~^T G), back-projection (U = P~ N~)
// and subspace-similarity kernels.
//
// A workgroup of 4 wave64 computes a BM x BN output tile; the waves sit in a WM x WN grid and
// each owns a (BM/WM) x (BN/WN) sub-tile made of 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation). K is consumed BK at a time through LDS
// stages: either a double buffer filled from registers (gemm_kloop), or a ring of two or
// three stages filled by LDS DMA with one or two stages in flight (gemm_kloop_dma).
//
// An MFMA lane needs 8 consecutive K values of one row of A (or one column of B). Operands
// are kept in LDS in the layout their source has, so staging is a straight copy, or for an
// INT4 projection a dequantization on the way into LDS (code * group scale, then bf16
// rounding: the DmaInt4 stagers below, whose codes arrive by LDS DMA and are converted in
// LDS, so that the bf16 P~ exists only in LDS):
//   * "K-contiguous" tiles (source [c][k]: the projection in the back-projection) are read
//     with one 16-byte ds_read_b128 per fragment;
//   * "K-major" tiles (source [k][c]: the gradient G, the update N~, the projection used
//     transposed) are read with two ds_read_b64_tr_b16, the gfx950 LDS transpose read: in a
//     group of 16 lanes, lane i receives element i % 4 of the 8-byte chunks addressed by
//     lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12. Addressing the chunk of row k0 + (i/4) + 4h,
//     columns c0 + 16 ((l/16) % 2) + 4 (l % 4), gives lane l the K values k0 .. k0+3 (h = 0)
//     and k0+4 .. k0+7 (h = 1) of column c0 + l % 32.
#pragma once

#include <utility>

#include "qg_device.hpp"

namespace qg {

typedef short v4i16 __attribute__((ext_vector_type(4)));

// DMA_ selects the layout the direct-to-LDS stagers write (kmaj_swz below): K-major tiles
// unpadded with permuted chunks instead of padded rows.
template <int BM_, int BN_, int BK_, int WM_, int WN_, bool A_KMAJOR_, bool B_KMAJOR_,
          bool DMA_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr bool A_KMAJOR = A_KMAJOR_, B_KMAJOR = B_KMAJOR_, DMA = DMA_;
  static_assert(WM * WN == 4, "four waves per workgroup");
  static_assert(BK % 16 == 0, "K stage is a multiple of the MFMA K");
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave sub-tile
  static constexpr int XM = WTM / 32, XN = WTN / 32;   // MFMA blocks per wave
  static_assert(XM * 32 == WTM && XN * 32 == WTN, "wave tile is a multiple of 32");
  // LDS pitches (bf16 elements): K-major tiles are BK rows of (edge + 32), so consecutive rows
  // start 16 banks apart and the 4-row x 32-byte footprint of a 16-lane transpose read covers
  // all 64 banks once; K-contiguous tiles are edge rows of BK, unpadded, with the chunks of a
  // row permuted (kc_off below).
  static_assert(A_KMAJOR || BK == 32, "K-contiguous tiles take 32-element rows");
  static_assert(B_KMAJOR || BK == 32, "K-contiguous tiles take 32-element rows");
  static constexpr int A_PITCH = A_KMAJOR ? BM + (DMA ? 0 : 32) : BK;
  static constexpr int B_PITCH = B_KMAJOR ? BN + (DMA ? 0 : 32) : BK;
  static constexpr int A_ELEMS = A_KMAJOR ? BK * A_PITCH : BM * A_PITCH;
  static constexpr int B_ELEMS = B_KMAJOR ? BK * B_PITCH : BN * B_PITCH;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;      // one [A | B] stage, bf16 elements
};

// Element offset of 8-element chunk `chunk` (0..3) of row `row` in a K-contiguous tile: rows
// of 32 elements, chunk c of row i stored at position c ^ ((i / 4) % 4). A 16-lane group then
// covers the 64 LDS banks exactly once both when it writes four whole rows (staging) and when
// it reads one chunk of 16 consecutive rows (an MFMA fragment).
__device__ __forceinline__ int kc_off(int row, int chunk) {
  return row * 32 + 8 * (chunk ^ ((row >> 2) & 3));
}

// Position of 16-byte chunk j of row k in an unpadded K-major tile of W >= 128 columns (rows
// of 256 or 512 bytes, so every row starts on the same bank): chunk j sits at j ^ 4 (k % 4).
// The 32 lanes of a transpose read address four consecutive rows and the four chunks of one
// aligned 64-byte column block; the permutation puts the four rows' blocks in the four
// distinct 64-byte bank groups.
template <int W>
__device__ __forceinline__ int kmaj_slot(int k, int j) {
  static_assert(W >= 128 && W % 64 == 0, "rows span whole bank rows");
  return j ^ (4 * (k & 3));
}

// ---------------------------------------------------------------------------------------
// Stagers: each fills one operand tile (W = its edge along the output, BK along K) with 256
// threads, in 8-element chunks. load() issues the global loads into registers, store()
// converts and writes LDS. Consecutive lanes take consecutive chunks along the contiguous
// dimension of the source, so global loads are coalesced.
// ---------------------------------------------------------------------------------------

// bf16 source [k][c] (row pitch ld, `rows` rows in all) -> K-major LDS tile [k][c].
// VEC (requires ld % 8 == 0): each stage reads 16-byte chunks through a buffer resource that
// starts at the stage's first row and ends at k_end, so rows past the K range read as zero
// without a per-lane test and the per-lane offsets stay fixed for the whole loop. Otherwise
// (rows of any pitch) a chunk's 8 elements come from the five dwords at the dword-aligned
// offset at or below it, shifted by half a dword when the chunk starts on an odd element.
// Elements past c_end (a chunk running over its row's end) then hold the next row's values;
// they only feed output columns that are dropped. Rows past k_end read as zero, and a chunk
// whose five dwords would run past the source's end is read element by element.
template <int W, int BK, bool VEC, int SETS = 1>
struct StageBf16K {
  static constexpr int CPR = W / 8;                    // chunks per row
  static constexpr int NC = BK * CPR / kThreads;       // chunks per thread
  static constexpr int RPU = kThreads / CPR;           // rows between a thread's chunks
  static_assert(NC * kThreads == BK * CPR && RPU * CPR == kThreads,
                "tile splits evenly over the threads");
  const uint16_t* src;
  rsrc_t rs;
  uint32_t ld, k_end, c_end, nbytes;
  int c0;
  uint32_t vo[NC];   // byte offset of chunk u from the stage's first row; kOOB off the tile
  uint4 v[SETS][NC];   // SETS stages in flight (see gemm_kloop_ring)

  __device__ StageBf16K(const uint16_t* s, int64_t ld_, int64_t rows, int64_t k_end_,
                        int64_t c_end_, int c0_)
      : src(s), ld((uint32_t)ld_), k_end((uint32_t)k_end_), c_end((uint32_t)c_end_),
        nbytes((uint32_t)(rows * ld_ * 2)), c0(c0_) {
    rs = make_rsrc(s, nbytes);
    const uint32_t c = c0 + 8 * (threadIdx.x % CPR);
#pragma unroll
    for (int u = 0; u < NC; ++u)
      vo[u] = c < c_end ? ((threadIdx.x / CPR + u * RPU) * ld + c) * 2 : kOOB;
  }

  template <int S = 0>
  __device__ __forceinline__ void load(int64_t k0_) {
    const uint32_t k0 = (uint32_t)k0_;
    if constexpr (VEC) {
      const uint32_t kb = k0 < k_end ? k0 : k_end;
      const rsrc_t st = make_rsrc(src + (size_t)kb * ld, (k_end - kb) * ld * 2);
#pragma unroll
      for (int u = 0; u < NC; ++u) v[S][u] = bload128(st, vo[u]);
    } else {
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        const int q = threadIdx.x + kThreads * u;
        const uint32_t k = k0 + q / CPR;
        const uint32_t c = c0 + 8 * (q % CPR);
        const uint32_t o = k * ld + c;            // the chunk's first element
        const uint32_t b = (o & ~1u) * 2;         // dword-aligned byte offset at or below it
        const bool in = k < k_end && c < c_end;
        if (in && b + 20 > nbytes) {              // the source's last chunk: element-wise
          uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t off = c + e < c_end ? (o + e) * 2 : kOOB;
            w[e >> 1] |= bload16(rs, off) << (16 * (e & 1));
          }
          v[S][u] = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          const uint4 x = bload128(rs, in ? b : kOOB);
          const uint32_t y = bload32(rs, in ? b + 16 : kOOB);
          const uint32_t sh = (o & 1u) * 16;
          v[S][u] = make_uint4(__builtin_amdgcn_alignbit(x.y, x.x, sh),
                               __builtin_amdgcn_alignbit(x.z, x.y, sh),
                               __builtin_amdgcn_alignbit(x.w, x.z, sh),
                               __builtin_amdgcn_alignbit(y, x.w, sh));
        }
      }
    }
  }

  template <int PITCH, int S = 0>
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      *reinterpret_cast<uint4*>(lds + (q / CPR) * PITCH + 8 * (q % CPR)) = v[S][u];
    }
  }
};

// Dequantize one word of 8 INT4 codes with its group scale: bf16(fl(q * s)) for each code,
// packed. With u = q + 8 (the nibble with its top bit flipped, 0..15, converted exactly by a
// byte-to-float conversion) a single fma gives RN(u * s - 8 s) = RN(q * s): the exact value of
// u * s - 8 s is q * s, and -8 s is exact (a power-of-two multiple of s). That holds for every
// scale of magnitude below 2^125, where 8 s stays finite; larger projection scales (entries
// near the fp32 maximum) are outside the contract. (A code 0 with a negative scale gives +0
// where the product gives -0; the quantizers never produce negative scales.) Every kernel
// that reads INT4 projections converts them here, so all paths agree bit for bit.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float s) {
  const uint32_t x = w ^ 0x88888888u;
  const uint32_t lo = x & 0x0F0F0F0Fu;          // u of elements 0, 2, 4, 6 (bytes 0..3)
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;   // u of elements 1, 3, 5, 7
  const float c = -8.0f * s;
  float f[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = __builtin_fmaf((float)((lo >> (8 * k)) & 0xFFu), s, c);
    f[2 * k + 1] = __builtin_fmaf((float)((hi >> (8 * k)) & 0xFFu), s, c);
  }
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// INT4 source [k][c] (row pitch ld codes, ld % 8 == 0, `rows` rows) -> K-major LDS tile [k][c]
// in bf16. A chunk of 8 codes starting at a multiple of 8 in the flat index lies inside one
// 256-element scale group, and since ld % 8 == 0 it is either wholly inside the tile or
// wholly outside (then it stages zeros).
template <int W, int BK>
struct StageInt4K {
  static constexpr int CPR = W / 8;
  static constexpr int NC = BK * CPR / kThreads;
  static_assert(NC * kThreads == BK * CPR, "tile splits evenly over the threads");
  rsrc_t rq, rsc;
  uint32_t ld, k_end, c_end;
  int c0;
  uint32_t w[NC];
  float s[NC];

  __device__ StageInt4K(const uint8_t* q_, const float* sc_, int64_t ld_, int64_t rows,
                        int64_t k_end_, int64_t c_end_, int c0_)
      : ld((uint32_t)ld_), k_end((uint32_t)k_end_), c_end((uint32_t)c_end_), c0(c0_) {
    const int64_t numel = rows * ld_;
    rq = make_rsrc(q_, (uint32_t)((numel + 1) / 2));
    rsc = make_rsrc(sc_, (uint32_t)(((numel + kGroup - 1) / kGroup) * 4));
  }

  __device__ __forceinline__ void load(int64_t k0_) {
    const uint32_t k0 = (uint32_t)k0_;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      const uint32_t k = k0 + q / CPR;
      const uint32_t c = c0 + 8 * (q % CPR);
      const bool in = k < k_end && c < c_end;
      const uint32_t e = k * ld + c;
      w[u] = bload32(rq, in ? (e >> 1) : kOOB);
      s[u] = bloadf(rsc, in ? (e >> 8) * 4 : kOOB);
    }
  }

  template <int PITCH>
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      *reinterpret_cast<uint4*>(lds + (q / CPR) * PITCH + 8 * (q % CPR)) = dequant8(w[u], s[u]);
    }
  }
};

// INT8 source [k][c] (row pitch ld codes, ld % 8 == 0, `rows` rows) -> K-major LDS tile [k][c]
// in bf16; like StageInt4K with one byte per code.
template <int W, int BK>
struct StageInt8K {
  static constexpr int CPR = W / 8;
  static constexpr int NC = BK * CPR / kThreads;
  static_assert(NC * kThreads == BK * CPR, "tile splits evenly over the threads");
  rsrc_t rq, rsc;
  uint32_t ld, k_end, c_end;
  int c0;
  uint2 w[NC];
  float s[NC];

  __device__ StageInt8K(const uint8_t* q_, const float* sc_, int64_t ld_, int64_t rows,
                        int64_t k_end_, int64_t c_end_, int c0_)
      : ld((uint32_t)ld_), k_end((uint32_t)k_end_), c_end((uint32_t)c_end_), c0(c0_) {
    const int64_t numel = rows * ld_;
    rq = make_rsrc(q_, (uint32_t)numel);
    rsc = make_rsrc(sc_, (uint32_t)(((numel + kGroup - 1) / kGroup) * 4));
  }

  __device__ __forceinline__ void load(int64_t k0_) {
    const uint32_t k0 = (uint32_t)k0_;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      const uint32_t k = k0 + q / CPR;
      const uint32_t c = c0 + 8 * (q % CPR);
      const bool in = k < k_end && c < c_end;
      const uint32_t e = k * ld + c;
      w[u] = bload64(rq, in ? e : kOOB);
      s[u] = bloadf(rsc, in ? (e >> 8) * 4 : kOOB);
    }
  }

  template <int PITCH>
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        f[e] = mul_rn((float)(int8_t)((e < 4 ? w[u].x : w[u].y) >> (8 * (e & 3))), s[u]);
      *reinterpret_cast<uint4*>(lds + (q / CPR) * PITCH + 8 * (q % CPR)) =
          make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7]));
    }
  }
};

// bf16 source [c][k] (row pitch ld = the K extent, ld % 8 == 0, c_end rows) -> K-contiguous
// LDS tile [c][k]. Each stage reads through a buffer resource starting at column k0; rows past
// c_end fall outside it. Only a last, partial stage (ld % BK != 0) tests columns per lane.
template <int W, int BK, int SETS = 1>
struct StageBf16C {
  static constexpr int CPR = BK / 8;
  static constexpr int NC = W * CPR / kThreads;
  static constexpr int RPU = kThreads / CPR;
  static_assert(NC * kThreads == W * CPR && RPU * CPR == kThreads,
                "tile splits evenly over the threads");
  const uint16_t* src;
  uint32_t ld, c_end, kk;
  int c0;
  uint32_t vo[NC];
  uint4 v[SETS][NC];   // SETS stages in flight (see gemm_kloop_ring)

  __device__ StageBf16C(const uint16_t* s, int64_t ld_, int64_t c_end_, int c0_)
      : src(s), ld((uint32_t)ld_), c_end((uint32_t)c_end_), c0(c0_) {
    kk = 8 * (threadIdx.x % CPR);
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const uint32_t row = c0 + threadIdx.x / CPR + u * RPU;
      vo[u] = row < c_end ? (row * ld + kk) * 2 : kOOB;
    }
  }

  template <int S = 0>
  __device__ __forceinline__ void load(int64_t k0_) {
    const uint32_t k0 = (uint32_t)k0_ < ld ? (uint32_t)k0_ : ld;
    const rsrc_t st = make_rsrc(src + k0, (c_end * ld - k0) * 2);
    if (k0 + BK <= ld) {
#pragma unroll
      for (int u = 0; u < NC; ++u) v[S][u] = bload128(st, vo[u]);
    } else {
#pragma unroll
      for (int u = 0; u < NC; ++u) v[S][u] = bload128(st, k0 + kk < ld ? vo[u] : kOOB);
    }
  }

  template <int PITCH, int S = 0>
  __device__ __forceinline__ void store(uint16_t* lds) const {
    static_assert(PITCH == 32 && CPR == 4, "K-contiguous tiles take 32-element rows");
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = threadIdx.x + kThreads * u;
      *reinterpret_cast<uint4*>(lds + kc_off(q / CPR, q % CPR)) = v[S][u];
    }
  }
};

// ---------------------------------------------------------------------------------------
// Direct-to-LDS staging (gfx950 LDS DMA). buffer_load_dwordx4 with the lds flag writes lane
// i's 16 bytes to LDS at M0 + 16 i, whatever address the lane read: data goes from memory to
// LDS without registers or LDS store instructions, so several stages can be in flight at no
// register cost. One wave-level load fills one contiguous KiB; the tile layout inside it is
// chosen through the chunk each lane fetches. Lanes whose offset is out of the resource's
// range write zeros.
//
// The load is issued from inline assembly: the compiler's own wait insertion does not tell
// these loads apart from the stage being read, and would wait for every load in flight
// before each LDS transpose read. Completion is tracked by hand instead (wait_vm_lds in
// gemm_kloop_dma); loads the compiler does not know of can only make its own vmcnt waits
// stricter, never looser, since vector loads complete in issue order. M0 (which the hardware
// reads when the load issues) is set in the same assembly block and declared clobbered.
// Destinations are LDS byte addresses held in scalar registers: the area's base is converted
// once per loop, and each load adds constant offsets to it.
// ---------------------------------------------------------------------------------------
typedef int v4i32 __attribute__((ext_vector_type(4)));

// Raw buffer resource words (as make_rsrc builds them) for use as an assembly operand. The
// values are uniform across the wave; readfirstlane makes that explicit, so that they are
// held in scalar registers as the instruction requires.
__device__ __forceinline__ v4i32 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return v4i32{__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
               __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFF)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// LDS byte address of a pointer into a __shared__ array (uniform across the wave).
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)(p));
}

// One wave-level load of 64 x 16 bytes into the KiB at LDS byte address m0 (uniform across
// the wave; readfirstlane states it).
__device__ __forceinline__ void dma16(v4i32 rs, uint32_t off, uint32_t m0) {
  const uint32_t m0s = __builtin_amdgcn_readfirstlane(m0);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(off), "s"(rs), "s"(m0s)
      : "memory", "m0");
}

// bf16 source [k][c] (row pitch ld, ld % 8 == 0 and c_end % 8 == 0) -> unpadded K-major
// tile [k][c] in the kmaj_slot layout. Each stage reads through a resource that starts at
// the stage's first row and ends at k_end, so rows past the K range are zeros.
template <int W, int BK>
struct DmaBf16K {
  static constexpr int CPR = W / 8;                 // chunks per row
  static constexpr int RPI = 64 / CPR;              // rows per wave-level load (one KiB)
  static constexpr int NI = BK / (4 * RPI);         // loads per wave and stage
  static_assert(NI * 4 * RPI == BK, "a stage splits evenly over the four waves");
  const uint16_t* src;
  uint32_t ld, k_end;
  uint32_t wofs;     // byte offset of this wave's rows in the tile
  uint32_t vo[NI];   // byte offset of this lane's chunk from the stage's first row

  __device__ DmaBf16K(const uint16_t* s, int64_t ld_, int64_t k_end_, int64_t c_end, int c0)
      : src(s), ld((uint32_t)ld_), k_end((uint32_t)k_end_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    wofs = __builtin_amdgcn_readfirstlane(wave * NI * RPI * W * 2);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int row = (wave * NI + q) * RPI + lane / CPR;
      const uint32_t c = c0 + 8 * kmaj_slot<W>(row, lane % CPR);   // the permutation is an
      vo[q] = c < (uint32_t)c_end ? (row * ld + c) * 2 : kOOB;      // involution
    }
  }

  // tile: LDS byte address of the stage's tile
  __device__ __forceinline__ void issue(int64_t k0_, uint32_t tile) const {
    const uint32_t k0 = (uint32_t)k0_ < k_end ? (uint32_t)k0_ : k_end;
    const v4i32 st = rsrc_words(src + (size_t)k0 * ld, (k_end - k0) * ld * 2);
#pragma unroll
    for (int q = 0; q < NI; ++q) dma16(st, vo[q], tile + wofs + q * RPI * W * 2);
  }
};

// bf16 source [c][k] (row pitch ld = the K extent, ld % 8 == 0, c_end rows) -> K-contiguous
// tile [c][k] in the kc_off layout (rows of BK = 32, 16 rows per wave-level load). Chunks
// past the K extent (a last, partial stage) and rows past c_end are zeros.
template <int W, int BK>
struct DmaBf16C {
  static_assert(BK == 32, "K-contiguous tiles take 32-element rows");
  static constexpr int NI = W / (4 * 16);
  static_assert(NI * 64 == W, "a stage splits evenly over the four waves");
  const uint16_t* src;
  uint32_t ld, c_end;
  uint32_t wofs;             // byte offset of this wave's rows in the tile
  uint32_t vo[NI], kc[NI];   // byte offset of this lane's chunk from column 0; its K offset

  __device__ DmaBf16C(const uint16_t* s, int64_t ld_, int64_t c_end_, int c0)
      : src(s), ld((uint32_t)ld_), c_end((uint32_t)c_end_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    wofs = __builtin_amdgcn_readfirstlane(wave * NI * 16 * 32 * 2);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int row = (wave * NI + q) * 16 + lane / 4;
      const uint32_t rg = c0 + row;
      kc[q] = 8 * ((lane & 3) ^ ((row >> 2) & 3));   // kc_off is an involution on chunks
      vo[q] = rg < c_end ? (rg * ld + kc[q]) * 2 : kOOB;
    }
  }

  // tile: LDS byte address of the stage's tile
  __device__ __forceinline__ void issue(int64_t k0_, uint32_t tile) const {
    const uint32_t k0 = (uint32_t)k0_ < ld ? (uint32_t)k0_ : ld;
    const v4i32 st = rsrc_words(src + k0, (c_end * ld - k0) * 2);
    const uint32_t lim = ld - k0;   // K values left in the rows
    if (lim >= (uint32_t)BK) {
#pragma unroll
      for (int q = 0; q < NI; ++q) dma16(st, vo[q], tile + wofs + q * 16 * 32 * 2);
    } else {
#pragma unroll
      for (int q = 0; q < NI; ++q)
        dma16(st, kc[q] < lim ? vo[q] : kOOB, tile + wofs + q * 16 * 32 * 2);
    }
  }
};

// One wave-level load of 64 x 4 bytes: active lane i's word lands at LDS byte address
// m0 + 4 i (inactive lanes write nothing). m0 is uniform across the wave (readfirstlane
// states it, so that it is held in a scalar register).
__device__ __forceinline__ void dma4(v4i32 rs, uint32_t off, uint32_t m0) {
  const uint32_t m0s = __builtin_amdgcn_readfirstlane(m0);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(off), "s"(rs), "s"(m0s)
      : "memory", "m0");
}

// ---------------------------------------------------------------------------------------
// INT4 projection operands staged by LDS DMA and converted in LDS. Per K stage the packed
// codes and one group scale per tile row go by DMA into a small code area; convert() then
// writes the bf16 tile the MFMA fragments read (bf16(fl(q * s)), dequant8). The codes are a
// quarter of the bf16 tile's bytes, so the projection is fetched from L2 at a quarter of the
// traffic, and no bf16 copy of it exists outside LDS. One scale per row needs each row's run
// of the stage inside one 256-element group; the host checks the rank for that.
// ---------------------------------------------------------------------------------------

// The projection P (m x r, INT4 row-major: row pitch ld = r codes) read as P~^T by the
// projection kernel: tile rows are rows k of P (the K dimension), tile columns c0 .. c0 + W - 1
// are rank indices. Each row's W codes lie in one group when r % 128 == 0 (c0 a multiple of
// 128) or r divides 256 (then c0 = 0). Produces the K-major tile [BK][W] in the kmaj_slot
// layout.
template <int W, int BK>
struct DmaInt4K {
  static_assert(W == 128 && BK == 32, "the projection kernel's tile");
  static constexpr int ROWB = W / 2;               // code bytes per tile row
  static constexpr int CODE_BYTES = BK * ROWB;     // 2 KiB
  static constexpr int AREA = CODE_BYTES + 256;    // + the BK row scales (a wave-load's span)
  static constexpr int RPI = 256 / ROWB;           // tile rows per wave-level load
  static constexpr int NI = BK / (4 * RPI);        // code loads per wave and stage
  static constexpr int NV = NI + 1;                // vector memory operations per wave, stage
  static_assert(NI * 4 * RPI == BK, "a stage splits evenly over the four waves");
  const uint8_t* q;
  v4i32 rsc;
  uint32_t ld, k_end, c0;
  uint32_t vo[NI];   // byte offset of this lane's code word from the stage's first row

  __device__ DmaInt4K(const uint8_t* q_, const float* sc_, int64_t ld_, int64_t rows,
                      int64_t k_end_, int c0_)
      : q(q_), ld((uint32_t)ld_), k_end((uint32_t)k_end_), c0((uint32_t)c0_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    rsc = rsrc_words(sc_, (uint32_t)(((rows * ld_ + kGroup - 1) / kGroup) * 4));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t row = (wave * NI + i) * RPI + lane / (ROWB / 4);
      const uint32_t word = lane % (ROWB / 4);
      const uint32_t col = c0 + 8 * word;
      vo[i] = col < ld ? row * (ld / 2) + c0 / 2 + 4 * word : kOOB;
    }
  }

  // area: LDS byte address of the stage's code area
  __device__ __forceinline__ void issue(int64_t k0_, uint32_t area) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t k0 = (uint32_t)k0_ < k_end ? (uint32_t)k0_ : k_end;
    const v4i32 st = rsrc_words(q + (size_t)k0 * (ld / 2), (k_end - k0) * (ld / 2));
#pragma unroll
    for (int i = 0; i < NI; ++i) dma4(st, vo[i], area + (wave * NI + i) * 256);
    // the scales of tile rows 8 w .. 8 w + 7 (lane = tile row)
    if (lane >= 8 * wave && lane < 8 * wave + 8) {
      const uint32_t k = k0 + lane;
      const uint32_t off = k < k_end ? ((k * ld + c0) >> 8) * 4 : kOOB;
      dma4(rsc, off, area + CODE_BYTES);
    }
  }
  // Thread t converts chunk t % 16 of tile rows t / 16 and t / 16 + 16 (16 lanes write one
  // whole 256-byte row: every bank once).
  __device__ __forceinline__ void convert(const uint8_t* area, uint16_t* tile) const {
    const int c = threadIdx.x % 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = threadIdx.x / 16 + 16 * h;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(area + row * ROWB + 4 * c);
      const float sc = *reinterpret_cast<const float*>(area + CODE_BYTES + 4 * row);
      *reinterpret_cast<uint4*>(tile + row * W + 8 * kmaj_slot<W>(row, c)) = dequant8(w, sc);
    }
  }
};

// The projection P (m x r) read by rows in the back-projection: tile rows c0 .. c0 + W - 1 are
// rows of P, K is the rank (ld = r codes per row, r % 32 == 0, so that a row's 32 codes of a
// stage lie in one group). Produces the K-contiguous tile [W][BK] in the kc_off layout.
template <int W, int BK>
struct DmaInt4C {
  static_assert(W == 128 && BK == 32, "the back-projection kernel's tile");
  static constexpr int ROWB = BK / 2;              // code bytes per tile row and stage
  static constexpr int CODE_BYTES = W * ROWB;      // 2 KiB
  static constexpr int AREA = CODE_BYTES + 4 * W;  // + the W row scales
  static constexpr int RPI = 256 / ROWB;           // tile rows per wave-level load
  static constexpr int NI = W / (4 * RPI);         // code loads per wave and stage
  static constexpr int NV = NI + 1;
  static_assert(NI * 4 * RPI == W, "a stage splits evenly over the four waves");
  const uint8_t* q;
  v4i32 rsc;
  uint32_t ld, c_end, c0;
  uint32_t vo[NI];   // byte offset of this lane's code word from column 0 of the stage

  __device__ DmaInt4C(const uint8_t* q_, const float* sc_, int64_t ld_, int64_t c_end_, int c0_)
      : q(q_), ld((uint32_t)ld_), c_end((uint32_t)c_end_), c0((uint32_t)c0_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    rsc = rsrc_words(sc_, (uint32_t)(((c_end_ * ld_ + kGroup - 1) / kGroup) * 4));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t rg = c0 + (wave * NI + i) * RPI + lane / (ROWB / 4);
      vo[i] = rg < c_end ? rg * (ld / 2) + 4 * (lane % (ROWB / 4)) : kOOB;
    }
  }

  __device__ __forceinline__ void issue(int64_t k0_, uint32_t area) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t k0 = (uint32_t)k0_ < ld ? (uint32_t)k0_ : ld;
    const v4i32 st = rsrc_words(q + k0 / 2, (c_end * ld - k0) / 2);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma4(st, vo[i], area + (wave * NI + i) * 256);
    // the scales: wave w loads tile rows 64 (w / 2) + lane for the lanes of half w % 2
    if ((lane >> 5) == (wave & 1)) {
      const uint32_t rg = c0 + 64 * (wave >> 1) + lane;
      const uint32_t off = rg < c_end ? ((rg * ld + k0) >> 8) * 4 : kOOB;
      dma4(rsc, off, area + CODE_BYTES + 256 * (wave >> 1));
    }
  }

  // Thread t converts chunk t % 4 of tile rows t / 4 and t / 4 + 64 (16 lanes write four whole
  // 64-byte rows: every bank once).
  __device__ __forceinline__ void convert(const uint8_t* area, uint16_t* tile) const {
    const int c = threadIdx.x % 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = threadIdx.x / 4 + 64 * h;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(area + row * ROWB + 4 * c);
      const float sc = *reinterpret_cast<const float*>(area + CODE_BYTES + 4 * row);
      *reinterpret_cast<uint4*>(tile + kc_off(row, c)) = dequant8(w, sc);
    }
  }
};

// ---------------------------------------------------------------------------------------
// Fragment reads and the K loop.
// ---------------------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ int wave_m() { return (threadIdx.x >> 6) / T::WN; }
template <class T>
__device__ __forceinline__ int wave_n() { return (threadIdx.x >> 6) % T::WN; }

// 8 K values (ks .. ks+7 of this lane's half) of row/column `c` (c = tile-relative index of
// lane 0's row for this 32-block) from a tile with the given layout.
template <bool KMAJOR, int PITCH, bool DMA = false>
__device__ __forceinline__ bf16x8 frag(const uint16_t* tile, int c, int ks) {
  const int lane = threadIdx.x & 63;
  if constexpr (!KMAJOR) {
    return *reinterpret_cast<const bf16x8*>(tile +
                                            kc_off(c + (lane & 31), (ks >> 3) + (lane >> 5)));
  } else {
    typedef __attribute__((address_space(3))) v4i16* lptr;
    const int row = ks + 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int col = c + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // the hi half reads row + 4, which has the same chunk permutation as row
    const uint16_t* p0;
    if constexpr (DMA)
      p0 = tile + row * PITCH + 8 * kmaj_slot<PITCH>(row, col >> 3) + (col & 7);
    else
      p0 = tile + row * PITCH + col;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lptr)(__attribute__((address_space(3))) void*)(p0));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lptr)(__attribute__((address_space(3))) void*)(p0 + 4 * PITCH));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 all = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, all);
  }
}

// PARTS = 1: plain bf16 product. PARTS = 2: the stage holds the bf16 "high" parts followed by
// the bf16 "low" remainders of fp32 operands; the product keeps hi*hi + hi*lo + lo*hi (about
// 16 significant bits per operand). FIRST: the stage is the first of the product, so the
// accumulators start from zero as the first MFMAs' inline-constant C operand (no register
// clearing).
template <class T, int PARTS, bool FIRST = false>
__device__ __forceinline__ void mfma_stage(const uint16_t* stage,
                                           f32x16 (&acc)[T::XM][T::XN]) {
  const int am = wave_m<T>() * T::WTM, bn = wave_n<T>() * T::WTN;
  const uint16_t* As = stage;
  const uint16_t* Bs = stage + T::A_ELEMS;
#pragma unroll
  for (int ks = 0; ks < T::BK; ks += 16) {
    bf16x8 a[T::XM], b[T::XN];
#pragma unroll
    for (int x = 0; x < T::XM; ++x) a[x] = frag<T::A_KMAJOR, T::A_PITCH, T::DMA>(As, am + 32 * x, ks);
#pragma unroll
    for (int y = 0; y < T::XN; ++y) b[y] = frag<T::B_KMAJOR, T::B_PITCH, T::DMA>(Bs, bn + 32 * y, ks);
#pragma unroll
    for (int x = 0; x < T::XM; ++x)
#pragma unroll
      for (int y = 0; y < T::XN; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a[x], b[y], (FIRST && ks == 0) ? f32x16{} : acc[x][y], 0, 0, 0);
    if constexpr (PARTS == 2) {
      bf16x8 al[T::XM], bl[T::XN];
#pragma unroll
      for (int x = 0; x < T::XM; ++x)
        al[x] = frag<T::A_KMAJOR, T::A_PITCH, T::DMA>(As + T::STAGE, am + 32 * x, ks);
#pragma unroll
      for (int y = 0; y < T::XN; ++y)
        bl[y] = frag<T::B_KMAJOR, T::B_PITCH, T::DMA>(Bs + T::STAGE, bn + 32 * y, ks);
#pragma unroll
      for (int x = 0; x < T::XM; ++x)
#pragma unroll
        for (int y = 0; y < T::XN; ++y) {
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], bl[y], acc[x][y], 0, 0, 0);
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[x], b[y], acc[x][y], 0, 0, 0);
        }
    }
  }
}

// acc[x][y] += A_tile * B_tile over K in [k_begin, k_end). store_a(sa, stage) /
// store_b(sb, stage) fill one stage from the loaded registers. The loop body has no branch,
// so the scheduler can interleave the next stage's conversion and LDS writes with the MFMAs.
template <class T, int PARTS, class SA, class SB, class StoreA, class StoreB>
__device__ __forceinline__ void gemm_kloop(SA& sa, SB& sb, StoreA store_a, StoreB store_b,
                                           int64_t k_begin, int64_t k_end, uint16_t* lds,
                                           f32x16 (&acc)[T::XM][T::XN]) {
  constexpr int STAGE = PARTS * T::STAGE;
#pragma unroll
  for (int x = 0; x < T::XM; ++x)
#pragma unroll
    for (int y = 0; y < T::XN; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
  if (k_end <= k_begin) return;
  const int nk = (int)((k_end - k_begin + T::BK - 1) / T::BK);
  sa.load(k_begin);
  sb.load(k_begin);
  store_a(sa, lds);
  store_b(sb, lds);
  __syncthreads();
  for (int kt = 0; kt + 1 < nk; ++kt) {
    sa.load(k_begin + (int64_t)(kt + 1) * T::BK);
    sb.load(k_begin + (int64_t)(kt + 1) * T::BK);
    // keep the next stage's global loads ahead of this stage's MFMAs
    __builtin_amdgcn_sched_barrier(0);
    mfma_stage<T, PARTS>(lds + (kt & 1) * STAGE, acc);
    store_a(sa, lds + ((kt + 1) & 1) * STAGE);
    store_b(sb, lds + ((kt + 1) & 1) * STAGE);
    __syncthreads();
  }
  mfma_stage<T, PARTS>(lds + ((nk - 1) & 1) * STAGE, acc);
  __syncthreads();
}

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1 (compile-time unrolled).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The same product for latency-bound cases (short K loops over operands in L2): the stagers
// hold D register sets (D even), and the loads of stage s + D are issued while stage s is
// multiplied, so D stages are in flight. Stages past k_end read as zero; the loop runs a
// whole number of D-stage rounds.
template <class T, int D, class SA, class SB>
__device__ __forceinline__ void gemm_kloop_ring(SA& sa, SB& sb, int64_t k_begin, int64_t k_end,
                                                uint16_t* lds, f32x16 (&acc)[T::XM][T::XN]) {
  static_assert(D % 2 == 0, "stage s sits in LDS buffer s % 2");
#pragma unroll
  for (int x = 0; x < T::XM; ++x)
#pragma unroll
    for (int y = 0; y < T::XN; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
  if (k_end <= k_begin) return;
  const int nk = (int)((k_end - k_begin + T::BK - 1) / T::BK);
  static_for<D>([&](auto dc) {
    constexpr int d = decltype(dc)::value;
    sa.template load<d>(k_begin + (int64_t)d * T::BK);
    sb.template load<d>(k_begin + (int64_t)d * T::BK);
  });
  sa.template store<T::A_PITCH, 0>(lds);
  sb.template store<T::B_PITCH, 0>(lds + T::A_ELEMS);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += D) {
    static_for<D>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      const int64_t kn = k_begin + (int64_t)(kt + d + D) * T::BK;
      sa.template load<d>(kn);
      sb.template load<d>(kn);
      __builtin_amdgcn_sched_barrier(0);
      mfma_stage<T, 1>(lds + (d & 1) * T::STAGE, acc);
      uint16_t* nxt = lds + ((d + 1) & 1) * T::STAGE;
      sa.template store<T::A_PITCH, (d + 1) % D>(nxt);
      sb.template store<T::B_PITCH, (d + 1) % D>(nxt + T::A_ELEMS);
      __syncthreads();
    });
  }
}

// Waits until at most N of this wave's vector-memory operations are outstanding (vmcnt;
// vector loads complete in issue order) and all of its LDS operations are done (lgkmcnt 0).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// Workgroup barrier without the memory fence of __syncthreads (which would also wait for the
// LDS loads still in flight); the asm memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// The product with direct-to-LDS stages in a ring of NST LDS buffers (NST = 3: stage kt + 2
// is loaded while stage kt is multiplied; NST = 2: stage kt + 1). Per iteration: wait for this
// wave's share of stage kt and for its own LDS reads of the previous iteration, barrier
// (every share of stage kt is in LDS, and no wave still reads buffer (kt - 1) % NST), issue
// stage kt + NST - 1 into that buffer, multiply stage kt. The lds area holds NST * T::STAGE
// elements.
// ZFIRST: the first stage's MFMAs start from an inline zero instead of cleared accumulator
// registers (worth it for short K loops; a long loop keeps the simpler code).
template <class T, int NST = 3, bool ZFIRST = false, class SA, class SB>
__device__ __forceinline__ void gemm_kloop_dma(const SA& sa, const SB& sb, int64_t k_begin,
                                               int64_t k_end, uint16_t* lds,
                                               f32x16 (&acc)[T::XM][T::XN]) {
  static_assert(T::DMA, "tile in the DMA layout");
  static_assert(NST == 2 || NST == 3, "two or three LDS buffers");
  constexpr int NI = SA::NI + SB::NI;   // loads per wave and stage
  if (k_end <= k_begin) {
#pragma unroll
    for (int x = 0; x < T::XM; ++x)
#pragma unroll
      for (int y = 0; y < T::XN; ++y)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
    return;
  }
  if constexpr (!ZFIRST) {
#pragma unroll
    for (int x = 0; x < T::XM; ++x)
#pragma unroll
      for (int y = 0; y < T::XN; ++y)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
  }
  const int nk = (int)((k_end - k_begin + T::BK - 1) / T::BK);
  const uint32_t base = lds_addr(lds);   // byte addresses: stage s at base + 2 s STAGE
  sa.issue(k_begin, base);
  sb.issue(k_begin, base + 2 * T::A_ELEMS);
  if (NST == 3 && nk > 1) {
    sa.issue(k_begin + T::BK, base + 2 * T::STAGE);
    sb.issue(k_begin + T::BK, base + 2 * (T::STAGE + T::A_ELEMS));
  }
  // The loop is unrolled over the ring, so that each copy reads a buffer known at compile
  // time: the fragment addresses are then loop-invariant registers plus immediate offsets.
  for (int k0 = 0; k0 < nk; k0 += NST) {
    static_for<NST>([&](auto dc) {
      constexpr int buf = decltype(dc)::value;   // kt % NST
      const int kt = k0 + buf;
      if (kt < nk) {
        if (NST == 3 && kt + 1 < nk)
          wait_vm_lds<NI>();
        else
          wait_vm_lds<0>();
        barrier_nofence();
        if (kt + NST - 1 < nk) {
          const uint32_t nxt = base + 2 * ((buf + NST - 1) % NST) * T::STAGE;
          sa.issue(k_begin + (int64_t)(kt + NST - 1) * T::BK, nxt);
          sb.issue(k_begin + (int64_t)(kt + NST - 1) * T::BK, nxt + 2 * T::A_ELEMS);
        }
        if (ZFIRST && buf == 0 && kt == 0)
          mfma_stage<T, 1, true>(lds, acc);
        else
          mfma_stage<T, 1>(lds + buf * T::STAGE, acc);
      }
    });
  }
  // the caller may reuse the LDS area: every wave is done with the last stage
  __syncthreads();
}

// The product with an INT4 first operand converted in LDS (SA: DmaInt4K or DmaInt4C) and a
// bf16 second operand by LDS DMA (SB), in a ring of NST LDS buffers (stage s in buffer
// s % NST) and NST code areas (codes of stage s in area s % NST; `codes` holds NST * SA::AREA
// bytes). Stage s's codes are issued one iteration before its B operand and converted one
// iteration before it is multiplied. Per iteration j:
//   wait until the B operand of stage j and the codes of stage j + 1 are in LDS (NST = 3:
//   the loads issued in iteration j - 1 stay in flight; NST = 2: nothing does), and for this
//   wave's LDS writes; barrier;
//   issue the B operand of stage j + NST - 1 (into the buffer stage j - 1 left) and the codes
//   of stage j + NST (into the area stage j's codes left);
//   multiply stage j;
//   convert the codes of stage j + 1 into the A tile of its buffer (free since stage j + 1 - NST
//   was multiplied, before the previous barrier).
template <class T, int NST, bool ZFIRST = false, class SA, class SB>
__device__ __forceinline__ void gemm_kloop_dma_cvt(const SA& sa, const SB& sb, int64_t k_begin,
                                                   int64_t k_end, uint16_t* lds, uint8_t* codes,
                                                   f32x16 (&acc)[T::XM][T::XN]) {
  static_assert(T::DMA, "tile in the DMA layout");
  static_assert(NST == 2 || NST == 3, "two or three LDS buffers");
  constexpr int NB = SB::NI;   // B loads per wave and stage
  constexpr int NC = SA::NV;   // code and scale loads per wave and stage
  if (k_end <= k_begin) {
#pragma unroll
    for (int x = 0; x < T::XM; ++x)
#pragma unroll
      for (int y = 0; y < T::XN; ++y)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
    return;
  }
  if constexpr (!ZFIRST) {
#pragma unroll
    for (int x = 0; x < T::XM; ++x)
#pragma unroll
      for (int y = 0; y < T::XN; ++y)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
  }
  const int nk = (int)((k_end - k_begin + T::BK - 1) / T::BK);
  const uint32_t base = lds_addr(lds);   // byte addresses: stage s at base + 2 s STAGE
  const uint32_t cbase = lds_addr(reinterpret_cast<const uint16_t*>(codes));
  auto issue_b = [&](int s) {
    sb.issue(k_begin + (int64_t)s * T::BK, base + 2 * ((s % NST) * T::STAGE + T::A_ELEMS));
  };
  auto issue_c = [&](int s) { sa.issue(k_begin + (int64_t)s * T::BK, cbase + (s % NST) * SA::AREA); };
  // codes(0); then what iterations -(NST-1) .. -1 would have issued: B(s), codes(s + 1)
  issue_c(0);
  issue_b(0);
  if (nk > 1) {
    issue_c(1);
    wait_vm_lds<NC>();
  } else {
    wait_vm_lds<0>();
  }
  barrier_nofence();
  sa.convert(codes, lds);
  if constexpr (NST == 3) {
    if (nk > 1) issue_b(1);
    if (nk > 2) issue_c(2);
  }
  for (int k0 = 0; k0 < nk; k0 += NST) {
    static_for<NST>([&](auto dc) {
      constexpr int buf = decltype(dc)::value;   // j % NST
      const int j = k0 + buf;
      if (j < nk) {
        if constexpr (NST == 3) {
          if (j + 2 < nk)
            wait_vm_lds<NB + NC>();
          else if (j + 1 < nk)
            wait_vm_lds<NB>();
          else
            wait_vm_lds<0>();
        } else {
          wait_vm_lds<0>();
        }
        barrier_nofence();
        if (j + NST - 1 < nk) issue_b(j + NST - 1);
        if (j + NST < nk) issue_c(j + NST);
        if (ZFIRST && buf == 0 && j == 0)
          mfma_stage<T, 1, true>(lds, acc);
        else
          mfma_stage<T, 1>(lds + buf * T::STAGE, acc);
        if (j + 1 < nk) {
          constexpr int nb = (buf + 1) % NST;
          sa.convert(codes + nb * SA::AREA, lds + nb * T::STAGE);
        }
      }
    });
  }
  // the caller may reuse the LDS area: every wave is done with the last stage
  __syncthreads();
}

// Output coordinates of accumulator element v of block (x, y) for this lane, relative to the
// workgroup tile: row = wm*WTM + 32x + 8(v/4) + 4(lane/32) + v%4, col = wn*WTN + 32y + lane%32.
template <class T>
__device__ __forceinline__ int acc_row(int x, int v) {
  const int lane = threadIdx.x & 63;
  return wave_m<T>() * T::WTM + 32 * x + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
template <class T>
__device__ __forceinline__ int acc_col(int y) {
  const int lane = threadIdx.x & 63;
  return wave_n<T>() * T::WTN + 32 * y + (lane & 31);
}

// Workgroups are dispatched to the 8 XCDs round-robin; renumber them so that consecutive
// logical tiles (which share input rows or columns) run on the same XCD and hit its L2.
__device__ __forceinline__ int xcd_remap(int b, int grid) {
  const int n8 = (grid / 8) * 8;
  if (b >= n8) return b;
  return (b & 7) * (n8 >> 3) + (b >> 3);
}

}  // namespace qg
