// Device-side helpers shared by the mHC kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Storage traits: one 16-byte vector holds V elements of the storage type.
struct BF16 {
  static constexpr int V = 8;
  typedef uint16_t elem;
};
struct F32 {
  static constexpr int V = 4;
  typedef float elem;
};

// 16-byte vector load / store through the vector memory path.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming (non-temporal) load for data read once: 1.3 us faster per mhc_post
// call at T = 2048, n = 4, D = 7168 than plain loads. (Not for the
// single-pass pre kernel, where neighbouring slices share 128-byte lines
// through L2: streaming loads made it 5.6 us slower there.)
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// Streaming (non-temporal) store for outputs that no part of the same kernel
// reads back: the lines do not stay dirty in L2 and the memory-side cache,
// so neither the end-of-kernel L2 writeback nor the next kernel's reads pay
// for writing them back later.
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Unpack one 16-byte vector of the storage type into fp32 values.
template <class S> struct Vec;
template <> struct Vec<BF16> {
  static __device__ __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { f[2 * k] = bf16_lo(v[k]); f[2 * k + 1] = bf16_hi(v[k]); }
  }
  static __device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = pack_bf16x2(f[2 * k], f[2 * k + 1]);
    return v;
  }
  // value after storage rounding, back in fp32
  static __device__ __forceinline__ float round_trip(float f) {
    return __uint_as_float((uint32_t)to_bf16_bits(f) << 16);
  }
};
template <> struct Vec<F32> {
  static __device__ __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(v[k]);
  }
  static __device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __float_as_uint(f[k]);
    return v;
  }
  static __device__ __forceinline__ float round_trip(float f) { return f; }
};

// acc + lo^2 + hi^2 of a packed bf16 pair (v_dot2: products exact, fp32 sum).
__device__ __forceinline__ float dot2_self(uint32_t w, float acc) {
  const bf16x2 p = __builtin_bit_cast(bf16x2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
}

// Logistic function with IEEE division and the library expf.
__device__ __forceinline__ float sigmoidf_ieee(float u) { return 1.0f / (1.0f + expf(-u)); }

}  // namespace mhc
