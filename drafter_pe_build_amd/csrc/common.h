// Device-side building blocks shared by the gfx950 kernels: storage types,
// 16-byte loads, bf16 conversion and the matrix-core (MFMA) step.
//
// Matrix-core convention used everywhere (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32, wave64): lane l = 16*g + r (r = l % 16,
// g = l / 16).  The A operand of lane l belongs to row r of the 16-row A
// tile, the B operand of lane l to column r of the 16-column B tile; the
// 16 bytes a lane supplies are its share of the contraction index.  Since
// the hardware pairs the A and B contributions of the same lane slot, any
// assignment of contraction indices to (g, element) works as long as A and
// B use the same one; each kernel documents its assignment.  The 16x16 f32
// result is spread as D[4*g + j][r] in element j (0..3) of lane l.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage types: float, or bf16 carried as uint16_t bits.
template <typename S> struct Storage;
template <> struct Storage<float> {
  static constexpr int CH = 4;  // elements per 16 bytes
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct Storage<uint16_t> {
  static constexpr int CH = 8;
  __device__ static float to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
  __device__ static uint16_t from_f32(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);  // v_cvt_pk_bf16_f32, round to nearest even
  }
};

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ uint16_t f2bf(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two floats to a bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32, RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// One 16-byte copy per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l writes bytes [16 l, 16 l + 16) after the
// wave-uniform LDS address dst.  Counted by vmcnt like any global load.
__device__ __forceinline__ void copy16_to_lds(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// One 16-byte-per-lane contraction step into a 16x16 f32 tile.
__device__ __forceinline__ void mma16(f32x4& acc, u32x4 a, u32x4 b, uint16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, u32x4 a, u32x4 b, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// Argmax order: larger value wins, equal values go to the lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// SplitMix64 output for state x (Steele, Lea and Flood, OOPSLA 2014).
__device__ __forceinline__ uint64_t mix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace pe
