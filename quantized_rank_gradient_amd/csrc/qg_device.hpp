// Device-side types and helpers shared by the Q-GaLore gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

constexpr int kGroup = 256;     // flat elements per quantization group
constexpr int kThreads = 256;   // threads per workgroup in every step kernel (4 wave64)

// Everything one layer's kernels need. In a grouped launch the host uploads one of these per
// layer; a single-layer launch passes it by value in the kernel arguments.
struct LayerDev {
  const uint16_t* G;   // bf16 m x n
  int8_t* Wq;          // int8 m x n
  const float* Ws;     // W group scales
  const uint8_t* Pq;   // INT4 m x r
  const float* Ps;     // P group scales
  int8_t* Mq;          // int8 r x n
  float* Ms;
  int8_t* Vq;          // int8 r x n
  float* Vs;
  int64_t off_r;       // workspace byte offset: split x rpitch fp32 partial sums of R
  int64_t off_n;       // workspace byte offset: bf16 r x n update N~ (rows ldn apart)
  int64_t off_p;       // workspace byte offset: bf16 m x r dequantized projection P~
                       // (written at the start of every step, read by both MFMA kernels;
                       // absent when p_inline)
  float* R_out;        // optional
  float* U_out;        // optional
  int64_t m, n, r;
  int64_t ldn;         // row pitch (elements) of N~ in the workspace: n rounded up to a
                       // multiple of 8, so that its rows can be staged in 16-byte chunks
  int64_t rpitch;      // elements between split slabs of Rpart
  uint32_t layer_id;
  int32_t p_format;    // 0: INT4 codes, 1: INT8 codes, 2: bf16 values (Pq then holds them)
  int32_t p_inline;    // 1: INT4 codes dequantized inside the MFMA kernels' stagers (no P~
                       // region in the workspace, no dequant workgroups); 0: the kernels
                       // stage the bf16 P~ (the dequant kernel's copy or the caller's bf16 P)
  int32_t split;       // K-splits of the projection
  int32_t fuse_adam;   // 1: one split and n % 256 == 0, so the projection kernel runs Adam
                       // on its tile rows (no R partials, no Adam launch for this layer)
  int32_t kslab;       // rows of G per split (multiple of the K tile)
  int32_t p_tiles_i;   // projection tiles along r
  int32_t p_tiles_j;   // projection tiles along n
  int32_t b_tiles_i;   // back-projection tiles along m
  int32_t b_tiles_j;   // back-projection tiles along n
  int32_t wg_base[4];  // first workgroup of this layer in the projection / Adam /
                       // back-projection / dequant launch of a grouped step
  int32_t fold_alpha;  // 1: U is not written and alpha = 2^k (-126 < k <= 0), so the rounding
                       // takes S * fl(alpha / s) in place of fl(alpha S) * (1 / s): the same
                       // value wherever alpha S is a normal number or zero
  float lr, eps, alpha;
};

struct StepArgs {
  LayerDev one;              // the layer of a single-layer launch (table == nullptr)
  char* ws;                  // workspace base
  const LayerDev* table;     // grouped launch: per-layer descriptors
  const int32_t* wg_layer;   // grouped launch: workgroup -> layer index for this kernel
  float beta1, beta2, c1, c2, bc1, bc2;
  double ibc1, ibc2;         // RN64(1 / bc1), RN64(1 / bc2)
  uint32_t step, seed_lo, seed_hi;
};

enum { KPROJ = 0, KADAM = 1, KBACK = 2, KDEQ = 3 };

// Which projection paths a launch of the MFMA kernels compiles in: every layer stages a bf16
// P~, every layer dequantizes its INT4 P in the stagers, or a mix of both.
enum { kPStaged = 0, kPInline = 1, kPMixed = 2 };

// `logical` is the workgroup's position in the launch after any renumbering.
// Projection storage formats (the values of qg_p_format).
constexpr int kPInt4 = 0, kPInt8 = 1, kPBf16 = 2;

// The bf16 projection P~ both MFMA kernels stage: the caller's own bf16 P, or the copy the
// dequant kernel writes into the workspace.
__device__ __forceinline__ const uint16_t* p_tilde(const StepArgs& a, const LayerDev& L) {
  return L.p_format == kPBf16 ? reinterpret_cast<const uint16_t*>(L.Pq)
                              : reinterpret_cast<const uint16_t*>(a.ws + L.off_p);
}

__device__ __forceinline__ LayerDev fetch_layer(const StepArgs& a, int kernel, int logical,
                                               int& local) {
  if (a.table == nullptr) {
    local = logical;
    return a.one;
  }
  const int li = a.wg_layer[logical];
  LayerDev L = a.table[li];
  local = logical - L.wg_base[kernel];
  return L;
}

// --------------------------------------------------------------- global accesses ---
// Loads and stores through an explicit global-address-space pointer, so that pointers that
// come out of a layer descriptor still compile to global_* (not flat_*) instructions.
// (The host compilation pass of this file never executes device code; it only needs the
// functions to parse, so it takes the plain pointer.)
template <class T>
__device__ __forceinline__ T gload(const T* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return *(const __attribute__((address_space(1))) T*)(p);
#else
  return *p;
#endif
}
template <class T>
__device__ __forceinline__ void gstore(T* p, T v) {
#if defined(__HIP_DEVICE_COMPILE__)
  *(__attribute__((address_space(1))) T*)(p) = v;
#else
  *p = v;
#endif
}

// --------------------------------------------------------------- buffer accesses ---
// Raw buffer loads and stores through a resource descriptor that bounds the tensor: an offset
// at or past the end reads zeros and drops stores, so tile edges need no branches, and the
// per-lane address is a 32-bit byte offset. Every tensor addressed this way is below 2 GiB.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;   // an offset past the end of any such tensor

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3: raw (untyped) access with a 32-bit data format, as gfx9 buffer loads require
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload128(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 bload64(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t bload32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload16(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload8(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ float bloadf(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void bstore32(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ __forceinline__ void bstoref(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore64(rsrc_t r, uint32_t off, uint2 v) {
  typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
  const v2u32 x = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(x, r, off, 0, 0);
}
__device__ __forceinline__ void bstore128(rsrc_t r, uint32_t off, uint4 v) {
  typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
  const v4u32 x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, 0);
}
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, r, off, 0, 0);
}

// ---------------------------------------------------------------- numeric helpers ---

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Correctly rounded fp32 square root. The compiler's sqrtf lowering (HIP's default
// correctly rounded fp32 divide and sqrt) already refines the hardware estimate with the
// exact residuals of its two neighbours, scaling tiny inputs first.
__device__ __forceinline__ float sqrt_rn(float x) { return __builtin_sqrtf(x); }

// a / b correctly rounded to fp32, for a divisor known on the host as yd = RN64(1 / b):
// the fp64 product a * yd is within 2^-52 (relative) of a / b, while the quotient of two
// fp32 values is either a float or at least ~2^-48 (relative) away from every midpoint
// between floats (its distance to a 25-bit midpoint is a non-zero multiple of 2^-47 of
// its size), so rounding the product to fp32 gives RN(a / b). Zeros, infinities, NaN,
// subnormal quotients and overflow all round as the quotient does.
__device__ __forceinline__ float div_by_recip64(float a, double yd) {
  return (float)((double)a * yd);
}

__device__ __forceinline__ float div_rn(float a, float b) { return __fdiv_rn(a, b); }
__device__ __forceinline__ float mul_rn(float a, float b) { return __fmul_rn(a, b); }
__device__ __forceinline__ float add_rn(float a, float b) { return __fadd_rn(a, b); }

__device__ __forceinline__ float recip_or_zero(float s) {
  return s == 0.0f ? 0.0f : div_rn(1.0f, s);
}

// floor(x) converted to int32, its low byte written into byte K of w in the same instruction
// (v_cvt_flr_i32_f32 with an SDWA byte destination): the other bytes of w are kept, or for
// K == 0 cleared, so four calls K = 0..3 build a packed word. Only called on finite x in
// [-128, 127], where the low byte is the two's-complement code.
template <int K>
__device__ __forceinline__ uint32_t floor_into_byte(uint32_t w, float x) {
  if constexpr (K == 0)
    asm("v_cvt_flr_i32_f32_sdwa %0, %1 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD"
        : "=v"(w) : "v"(x));
  else if constexpr (K == 1)
    asm("v_cvt_flr_i32_f32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
        : "+v"(w) : "v"(x));
  else if constexpr (K == 2)
    asm("v_cvt_flr_i32_f32_sdwa %0, %1 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
        : "+v"(w) : "v"(x));
  else
    asm("v_cvt_flr_i32_f32_sdwa %0, %1 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
        : "+v"(w) : "v"(x));
  return w;
}

// Signed byte K (0..3) of w converted to float in one instruction (SDWA operand select with
// sign extension).
template <int K>
__device__ __forceinline__ float sbyte_to_f32(uint32_t w) {
  float r;
  if constexpr (K == 0)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0"
        : "=v"(r) : "v"(w));
  else if constexpr (K == 1)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1"
        : "=v"(r) : "v"(w));
  else if constexpr (K == 2)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2"
        : "=v"(r) : "v"(w));
  else
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3"
        : "=v"(r) : "v"(w));
  return r;
}

// ---------------------------------------------------------------- Philox4x32-10 ---
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11),
// Section 3: each round multiplies words 0 and 2 by the round multipliers and mixes the
// 64-bit products' halves with words 1, 3 and the key; the key advances by the Weyl
// constants between rounds. Ten rounds.
// Three-way XOR in one gfx950 bitop3 instruction (truth table 0x96 = a ^ b ^ c).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)c.x * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c.z * 0xCD9E8D57u;
    if (round == 0) {
      // plain XORs let the compiler fold the parts that are uniform across the wave
      c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1,
                     (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
    } else {
      c = make_uint4(xor3((uint32_t)(p1 >> 32), c.y, k0), (uint32_t)p1,
                     xor3((uint32_t)(p0 >> 32), c.w, k1), (uint32_t)p0);
    }
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// ---------------------------------------------------------------- wave reductions ---
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
// Maximum over each aligned group of 16 lanes.
__device__ __forceinline__ float max16(float v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 16));
  return v;
}

}  // namespace qg
